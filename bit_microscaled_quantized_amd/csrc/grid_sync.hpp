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
//   arrive : w maxes its amax into its group's `amax`, then adds 1 to the
//            group's `arrive` (after its max is performed).  The group's last
//            arriver reads the group max, resets the group's fields, maxes it
//            into the top `amax` and adds 1 to the top `arrive`; the last
//            group arriver reads the tensor amax, resets the top, publishes
//            it in `result` and sets `done` = e.
//   wait   : every workgroup polls `done` == e, at most spin_limit polls.  One
//            that gives up records its index in `gave_up_list` and counts in
//            `gave_ups` (a running total the host can read).
//   depart : after encoding its own blocks (or giving up), w adds 1 to its
//            group's `depart`; the group's last departer adds 1 to the top
//            `depart`; the last one overall has seen every workgroup arrive
//            and leave, so `result` is final and the give-up list complete:
//            it encodes the blocks of the workgroups that gave up (from
//            memory), writes the tensor-level outputs, and clears the list.
// So a launch whose grid is not all resident at once never hangs and never
// leaves outputs unwritten: workgroups that wait too long leave their blocks
// to the last one, which runs after all have arrived.  Every field the next
// launch on the slot relies on is back at zero when the launch ends (`done`
// is compared with the epoch, so it needs no reset).
#pragma once

#include <stdint.h>

namespace nvfp4 {

constexpr uint32_t kSyncGroups = 16;
constexpr uint32_t kSyncMaxGrid = 4096;  // workgroups per launch

struct alignas(128) SyncLine {
  uint32_t arrive;
  uint32_t amax;  // FP32 bits of a non-negative maximum (integer order = float order)
  uint32_t depart;
  uint32_t amax2;  // a second maximum (grid_max_arrive)
  uint32_t pad[28];
};

struct GridSyncSlot {
  SyncLine group[kSyncGroups];
  SyncLine top;
  alignas(128) uint32_t done;  // epoch of the last published result
  uint32_t result;             // tensor amax bits of that epoch
  alignas(128) uint32_t gave_up_n;   // workgroups of this launch in gave_up_list
  uint32_t gave_ups;                 // running total over all launches
  alignas(128) uint32_t gave_up_list[kSyncMaxGrid];
};

// Ops (all device-scope):
//   static void max_relaxed(uint32_t* p, uint32_t v);
//   static uint32_t add_release(uint32_t* p, uint32_t v);  // after this thread's earlier
//                                                          // atomics; returns the old value
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

// Arrive with this workgroup's maximum and wait for the tensor amax.  Called
// by one thread per workgroup.  True: *amax_bits holds the tensor amax.
// False: the workgroup gave up (recorded); it must not write its outputs.
template <typename Ops>
__host__ __device__ inline bool grid_arrive_wait(GridSyncSlot* s, uint32_t G, uint32_t w,
                                                 uint32_t my_max, uint32_t epoch,
                                                 uint64_t spin_limit, uint32_t* amax_bits) {
  const uint32_t g = w % kSyncGroups;
  SyncLine* gl = &s->group[g];
  Ops::max_relaxed(&gl->amax, my_max);
  if (Ops::add_release(&gl->arrive, 1u) == sync_group_size(G, g) - 1u) {
    // last of the group: every member's max is performed before its arrival
    Ops::fence_acquire();
    const uint32_t gm = Ops::load_relaxed(&gl->amax);
    Ops::store_relaxed(&gl->amax, 0u);
    Ops::store_relaxed(&gl->arrive, 0u);
    Ops::max_relaxed(&s->top.amax, gm);
    if (Ops::add_release(&s->top.arrive, 1u) == sync_groups_used(G) - 1u) {
      Ops::fence_acquire();
      const uint32_t tm = Ops::load_relaxed(&s->top.amax);
      Ops::store_relaxed(&s->top.amax, 0u);
      Ops::store_relaxed(&s->top.arrive, 0u);
      Ops::store_relaxed(&s->result, tm);
      Ops::store_release(&s->done, epoch);
    }
  }
  for (uint64_t n = 0;; n++) {
    if (Ops::load_relaxed(&s->done) == epoch) {
      Ops::fence_acquire();
      *amax_bits = Ops::load_relaxed(&s->result);
      return true;
    }
    if (n >= spin_limit) break;
    Ops::pause();
  }
  const uint32_t i = Ops::add_release(&s->gave_up_n, 1u);
  Ops::store_relaxed(&s->gave_up_list[i], w);
  Ops::add_release(&s->gave_ups, 1u);
  return false;
}

// Leave the launch (after this workgroup's own encoding, or after giving up).
// True for the last workgroup to leave: it must then call grid_recover_list
// to learn which workgroups gave up, encode their blocks, write the tensor
// outputs, and call grid_finish.
template <typename Ops>
__host__ __device__ inline bool grid_depart(GridSyncSlot* s, uint32_t G, uint32_t w) {
  const uint32_t g = w % kSyncGroups;
  SyncLine* gl = &s->group[g];
  if (Ops::add_release(&gl->depart, 1u) != sync_group_size(G, g) - 1u) return false;
  Ops::store_relaxed(&gl->depart, 0u);
  if (Ops::add_release(&s->top.depart, 1u) != sync_groups_used(G) - 1u) return false;
  Ops::store_relaxed(&s->top.depart, 0u);
  Ops::fence_acquire();
  return true;
}

// For the last departer: the tensor amax and the number of workgroups that
// gave up (their indices are gave_up_list[0 .. n)).
template <typename Ops>
__host__ __device__ inline uint32_t grid_recover_list(GridSyncSlot* s, uint32_t* amax_bits) {
  *amax_bits = Ops::load_relaxed(&s->result);
  return Ops::load_relaxed(&s->gave_up_n);
}

template <typename Ops>
__host__ __device__ inline void grid_finish(GridSyncSlot* s) {
  Ops::store_relaxed(&s->gave_up_n, 0u);
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
