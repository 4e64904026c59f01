// Device-wide exchange of the tensor amax between the G workgroups of one
// single-pass quantize launch.  The protocol is written against an abstract
// set of atomic operations so that the same code runs in the HIP kernel and
// in a CPU emulation with one thread per workgroup.
//
// Contention: device-scope atomics on one address are serialized (about 7 ns
// each on MI355X, so 512 workgroups x 3 atomics on one line cost ~11 us).
// Workgroup w therefore works on group line w % kGroups (<= 32 workgroups per
// line) and only the last workgroup of each group touches the top line.
//
// One launch (epoch e, a nonzero number the host makes unique per slot):
//   arrive  : w maxes its amax into its group's `amax`, then adds 1 to the
//             group's `arrive` (after its max is performed).  The group's
//             last arriver reads the group max, resets the group's fields,
//             maxes it into the top `amax` and adds 1 to the top `arrive`;
//             the last group arriver -- the publisher -- reads the tensor
//             amax, resets the top and publishes the amax through the gate.
//   gate    : one 64-bit word, [amax 63:32 | epoch bits 31:14 | closed bit 13
//             | count 12:0]; a word of another epoch reads as this epoch's
//             open gate with count 0.  The publisher swaps in (amax, e,
//             closed, 0) with one atomic exchange; the word it takes out
//             holds the number of workgroups of this epoch that gave up.
//   wait    : every other workgroup polls the gate until it is closed for e
//             (the amax comes with it), at most spin_limit polls, then tries
//             to give up: a compare-and-swap that adds 1 to the count of the
//             still-open gate.  The count before its swap is its index in
//             `gave_up_list`, where it then stores w + 1, and it leaves
//             without encoding.  No swap can add to a closed gate, so the
//             count the publisher takes out is exactly the set that gave up;
//             a workgroup whose swap fails on a closed gate takes the amax
//             from it and goes on normally.
//   second  : a launch may exchange a second maximum (the fused row + RHT
//             cast needs the amax of the input and of its transform).  It
//             travels through the lines' `amax2` fields, and the publisher
//             stores [max2 | epoch] into `result2` before it swaps the gate
//             (the swap is ordered after that store); a workgroup that sees
//             the gate closed reads it from there.
//   recover : after its own blocks, the publisher encodes the blocks of the
//             workgroups in gave_up_list[0 .. count) (from memory; it waits
//             for each entry to be stored) and clears those entries.
// So a launch whose grid is not all resident at once never hangs and never
// leaves outputs unwritten: workgroups that wait too long leave their blocks
// to the publisher, which runs after all have arrived.  No workgroup has to
// wait for the others to finish.  When the launch ends, the lines and the
// list are back at zero; the gate carries the epoch, so it needs no reset.
#pragma once

#include <stdint.h>

namespace nvfp4 {

constexpr uint32_t kSyncGroups = 16;
constexpr uint32_t kSyncMaxGrid = 4096;  // workgroups per launch

struct alignas(128) SyncLine {
  uint32_t arrive;
  uint32_t amax;  // FP32 bits of a non-negative maximum (integer order = float order)
  uint32_t amax2;  // a second maximum (grid_max_arrive)
  uint32_t pad[29];
};

struct GridSyncSlot {
  SyncLine group[kSyncGroups];
  SyncLine top;
  alignas(128) uint64_t gate;  // [amax 63:32 | epoch 31:14 | closed 13 | count 12:0]
  uint64_t result2;            // [second maximum 63:32 | epoch 31:0]
  uint32_t gave_ups;           // running total over all launches
  alignas(128) uint32_t gave_up_list[kSyncMaxGrid];  // w + 1, 0 = empty
};

constexpr uint64_t kGateClosed = 1u << 13;
constexpr uint64_t kGateCount = kGateClosed - 1u;
constexpr uint64_t kGateTagMask = 0xFFFFC000ull;

__host__ __device__ inline uint64_t gate_tag(uint32_t epoch) { return (uint64_t)(epoch << 14); }

// This epoch's view of a gate word: another epoch's word is an open gate
// with count 0.
__host__ __device__ inline uint64_t gate_view(uint64_t g, uint32_t epoch) {
  return (g & kGateTagMask) == gate_tag(epoch) ? g : gate_tag(epoch);
}

// Ops (all device-scope):
//   static void max_relaxed(uint32_t* p, uint32_t v);
//   static uint32_t add_release(uint32_t* p, uint32_t v);  // after this thread's earlier
//                                                          // atomics; returns the old value
//   static bool cas64(uint64_t* p, uint64_t& expected, uint64_t desired);
//   static uint64_t exchange64(uint64_t* p, uint64_t v);
//   static uint64_t exchange64_release(uint64_t* p, uint64_t v);  // after earlier stores
//   static void store64_relaxed(uint64_t* p, uint64_t v);
//   static uint64_t load64(uint64_t* p);
//   static uint32_t load_relaxed(uint32_t* p);
//   static void store_release(uint32_t* p, uint32_t v);   // after earlier atomics
//   static void store_relaxed(uint32_t* p, uint32_t v);
//   static void fence_acquire();                          // later loads after earlier ones
//   static void pause();

__host__ __device__ inline uint32_t sync_group_size(uint32_t G, uint32_t g) {
  return g < G ? (G - g + kSyncGroups - 1) / kSyncGroups : 0u;
}

__host__ __device__ inline uint32_t sync_groups_used(uint32_t G) {
  return G < kSyncGroups ? G : kSyncGroups;
}

enum GridRole : uint32_t { kGridWaited = 0, kGridGaveUp = 1, kGridPublisher = 2 };

// The second maximum of this epoch from result2 (stored before the gate was
// closed, so the first read normally has it; at most spin_limit more polls).
template <typename Ops>
__host__ __device__ inline uint32_t grid_second(GridSyncSlot* s, uint32_t epoch, uint64_t spin_limit) {
  uint64_t r = Ops::load64(&s->result2);
  for (uint64_t n = 0; (uint32_t)r != epoch && n < spin_limit; n++) {
    Ops::pause();
    r = Ops::load64(&s->result2);
  }
  return (uint32_t)(r >> 32);
}

// Arrive with this workgroup's maximum (and, with amax2_bits not null, a
// second one) and obtain the tensor maxima.  Called by one thread per
// workgroup.  kGridWaited / kGridPublisher: *amax_bits (and *amax2_bits)
// hold the tensor maxima and the workgroup encodes its blocks; the publisher
// then also covers the *recover workgroups in gave_up_list (grid_recovered)
// and writes the tensor-level outputs.  kGridGaveUp: recorded; the
// workgroup must not write its outputs.
template <typename Ops>
__host__ __device__ inline GridRole grid_arrive_wait(GridSyncSlot* s, uint32_t G, uint32_t w,
                                                     uint32_t my_max, uint32_t epoch,
                                                     uint64_t spin_limit, uint32_t* amax_bits,
                                                     uint32_t* recover, uint32_t my_max2 = 0u,
                                                     uint32_t* amax2_bits = nullptr) {
  const bool two = amax2_bits != nullptr;
  const uint32_t g = w % kSyncGroups;
  SyncLine* gl = &s->group[g];
  Ops::max_relaxed(&gl->amax, my_max);
  if (two) Ops::max_relaxed(&gl->amax2, my_max2);
  if (Ops::add_release(&gl->arrive, 1u) == sync_group_size(G, g) - 1u) {
    // last of the group: every member's max is performed before its arrival
    Ops::fence_acquire();
    const uint32_t gm = Ops::load_relaxed(&gl->amax);
    const uint32_t gm2 = two ? Ops::load_relaxed(&gl->amax2) : 0u;
    Ops::store_relaxed(&gl->amax, 0u);
    if (two) Ops::store_relaxed(&gl->amax2, 0u);
    Ops::store_relaxed(&gl->arrive, 0u);
    Ops::max_relaxed(&s->top.amax, gm);
    if (two) Ops::max_relaxed(&s->top.amax2, gm2);
    if (Ops::add_release(&s->top.arrive, 1u) == sync_groups_used(G) - 1u) {
      Ops::fence_acquire();
      const uint32_t tm = Ops::load_relaxed(&s->top.amax);
      Ops::store_relaxed(&s->top.amax, 0u);
      if (two) {
        const uint32_t tm2 = Ops::load_relaxed(&s->top.amax2);
        Ops::store_relaxed(&s->top.amax2, 0u);
        Ops::store64_relaxed(&s->result2, ((uint64_t)tm2 << 32) | epoch);
        *amax2_bits = tm2;
      }
      Ops::store_relaxed(&s->top.arrive, 0u);
      const uint64_t gate = ((uint64_t)tm << 32) | gate_tag(epoch) | kGateClosed;
      const uint64_t old = two ? Ops::exchange64_release(&s->gate, gate) : Ops::exchange64(&s->gate, gate);
      *recover = (uint32_t)(gate_view(old, epoch) & kGateCount);
      *amax_bits = tm;
      return kGridPublisher;
    }
  }
  *recover = 0u;
  uint64_t cur = 0;
  for (uint64_t n = 0;; n++) {
    cur = gate_view(Ops::load64(&s->gate), epoch);
    if (cur & kGateClosed) break;
    if (n >= spin_limit) {
      for (;;) {
        uint64_t expected = Ops::load64(&s->gate);
        const uint64_t v = gate_view(expected, epoch);
        if (v & kGateClosed) {  // published meanwhile
          cur = v;
          break;
        }
        if (Ops::cas64(&s->gate, expected, v + 1u)) {
          Ops::store_release(&s->gave_up_list[v & kGateCount], w + 1u);
          Ops::add_release(&s->gave_ups, 1u);
          return kGridGaveUp;
        }
      }
      break;
    }
    Ops::pause();
  }
  *amax_bits = (uint32_t)(cur >> 32);
  if (two) {
    Ops::fence_acquire();
    *amax2_bits = grid_second<Ops>(s, epoch, spin_limit);
  }
  return kGridWaited;
}

// The publisher's recovery: the workgroup that took entry i of the give-up
// list (waiting for its store, at most spin_limit polls; UINT32_MAX if it
// never came), the entry cleared for the next launch.
template <typename Ops>
__host__ __device__ inline uint32_t grid_recovered(GridSyncSlot* s, uint32_t i, uint64_t spin_limit) {
  for (uint64_t n = 0;; n++) {
    const uint32_t e = Ops::load_relaxed(&s->gave_up_list[i]);
    if (e != 0u) {
      Ops::store_relaxed(&s->gave_up_list[i], 0u);
      return e - 1u;
    }
    if (n >= spin_limit) return 0xFFFFFFFFu;
    Ops::pause();
  }
}

// A grid-wide maximum without waiting (the amax passes of the two-pass
// path): every workgroup contributes two maxima through the same two-level
// lines; the one that arrives last overall gets both results (returns true)
// and writes them wherever they are needed, and the lines it used are back
// at zero.  No workgroup waits, so any grid size and any residency works.
template <typename Ops>
__host__ __device__ inline bool grid_max_arrive(GridSyncSlot* s, uint32_t G, uint32_t w, uint32_t m0,
                                                uint32_t m1, uint32_t* r0, uint32_t* r1) {
  const uint32_t g = w % kSyncGroups;
  SyncLine* gl = &s->group[g];
  Ops::max_relaxed(&gl->amax, m0);
  Ops::max_relaxed(&gl->amax2, m1);
  if (Ops::add_release(&gl->arrive, 1u) != sync_group_size(G, g) - 1u) return false;
  Ops::fence_acquire();
  const uint32_t g0 = Ops::load_relaxed(&gl->amax), g1 = Ops::load_relaxed(&gl->amax2);
  Ops::store_relaxed(&gl->amax, 0u);
  Ops::store_relaxed(&gl->amax2, 0u);
  Ops::store_relaxed(&gl->arrive, 0u);
  Ops::max_relaxed(&s->top.amax, g0);
  Ops::max_relaxed(&s->top.amax2, g1);
  if (Ops::add_release(&s->top.arrive, 1u) != sync_groups_used(G) - 1u) return false;
  Ops::fence_acquire();
  *r0 = Ops::load_relaxed(&s->top.amax);
  *r1 = Ops::load_relaxed(&s->top.amax2);
  Ops::store_relaxed(&s->top.amax, 0u);
  Ops::store_relaxed(&s->top.amax2, 0u);
  Ops::store_relaxed(&s->top.arrive, 0u);
  return true;
}

}  // namespace nvfp4
