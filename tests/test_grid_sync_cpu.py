"""CPU emulation of the single-pass quantizer's device-wide amax exchange
(bit_microscaled_quantized_amd/csrc/grid_sync.hpp), run before and beside the
GPU: the header's protocol is compiled with g++ against std::atomic and each
workgroup of a launch is a thread.  Per launch it checks that exactly one
workgroup publishes, that every workgroup either learns the exact tensor
maximum and writes its own blocks, or gives up and has its blocks written by
the publisher (each block written exactly once), that nothing hangs, and
that the slot is back at its idle state for the next launch on it.

* full residency: launches of G = 1 .. 200 workgroups (random start delays)
  on one slot, nobody gives up; every other launch also exchanges a second
  maximum (the fused row + RHT cast's), which every workgroup that stays
  must learn exactly, and which the slot's result word then holds with the
  launch's epoch;
* limited residency (at most R < G workgroups run at once, the rest start
  only when one ends, as on a GPU whose grid is partly displaced): workgroups
  that wait past the spin limit give up and are counted, the publisher
  covers their blocks, and the next launch on the slot runs clean;
* a spin limit of zero: only workgroups that arrive after the result is
  published pass; the rest are covered;
* the no-wait grid maximum of the two-pass amax kernels (two maxima per
  workgroup, any residency): exactly one workgroup, the last to arrive, gets
  both exact maxima, and the slot is idle after it, interleaved on the same
  slot with single-pass launches as on one stream.

The same program is also built with ThreadSanitizer to check that the
protocol has no data race."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "bit_microscaled_quantized_amd", "csrc")

SRC = r"""
#define __host__
#define __device__
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <mutex>
#include <random>
#include <thread>
#include <vector>
#include "grid_sync.hpp"
using nvfp4::GridSyncSlot;

struct CpuOps {
  static std::atomic_ref<uint32_t> at(uint32_t* p) { return std::atomic_ref<uint32_t>(*p); }
  static void max_relaxed(uint32_t* p, uint32_t v) {
    auto a = at(p);
    uint32_t cur = a.load(std::memory_order_relaxed);
    while (cur < v && !a.compare_exchange_weak(cur, v, std::memory_order_relaxed)) {
    }
  }
  static uint32_t add_release(uint32_t* p, uint32_t v) { return at(p).fetch_add(v, std::memory_order_acq_rel); }
  static std::atomic_ref<uint64_t> at64(uint64_t* p) { return std::atomic_ref<uint64_t>(*p); }
  static bool cas64(uint64_t* p, uint64_t& expected, uint64_t desired) {
    return at64(p).compare_exchange_strong(expected, desired, std::memory_order_acq_rel);
  }
  static uint64_t exchange64(uint64_t* p, uint64_t v) { return at64(p).exchange(v, std::memory_order_acq_rel); }
  static uint64_t exchange64_release(uint64_t* p, uint64_t v) { return at64(p).exchange(v, std::memory_order_acq_rel); }
  static void store64_relaxed(uint64_t* p, uint64_t v) { at64(p).store(v, std::memory_order_relaxed); }
  static uint64_t load64(uint64_t* p) { return at64(p).load(std::memory_order_acquire); }
  static uint32_t load_relaxed(uint32_t* p) { return at(p).load(std::memory_order_relaxed); }
  static void store_relaxed(uint32_t* p, uint32_t v) { at(p).store(v, std::memory_order_relaxed); }
  static void store_release(uint32_t* p, uint32_t v) { at(p).store(v, std::memory_order_release); }
  static void fence_acquire() { std::atomic_thread_fence(std::memory_order_acquire); }
  static void pause() { std::this_thread::yield(); }
};

// counting semaphore: at most `cap` workgroups resident at once
struct Residency {
  std::mutex mu;
  std::condition_variable cv;
  int free;
  explicit Residency(int cap) : free(cap) {}
  void enter() { std::unique_lock<std::mutex> l(mu); cv.wait(l, [&] { return free > 0; }); free--; }
  void leave() { { std::lock_guard<std::mutex> l(mu); free++; } cv.notify_one(); }
};

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL line %d: %s\n", __LINE__, #c); fails++; } } while (0)

static bool idle(const GridSyncSlot* s) {
  for (uint32_t g = 0; g < nvfp4::kSyncGroups; g++)
    if (s->group[g].arrive || s->group[g].amax || s->group[g].amax2) return false;
  for (uint32_t i = 0; i < nvfp4::kSyncMaxGrid; i++)
    if (s->gave_up_list[i]) return false;
  return !s->top.arrive && !s->top.amax && !s->top.amax2;
}

// one launch of G workgroups (with `two`, exchanging a second maximum too);
// returns how many gave up
static int launch(GridSyncSlot* s, uint32_t epoch, int G, int resident, uint64_t spin,
                  std::mt19937& rng, bool two = false) {
  std::vector<uint32_t> vals(G), got(G, 0xFFFFFFFFu), vals2(G), got2(G, 0xFFFFFFFFu);
  std::vector<int> writes(G, 0);  // how many times workgroup i's blocks were written
  std::vector<int> ok(G, 0);
  uint32_t want = 0;
  uint32_t want2 = 0;
  for (int i = 0; i < G; i++) { vals[i] = rng() >> 1; want = vals[i] > want ? vals[i] : want; }
  for (int i = 0; i < G; i++) { vals2[i] = rng() >> 1; want2 = vals2[i] > want2 ? vals2[i] : want2; }
  std::vector<int> delay(G);
  for (int i = 0; i < G; i++) delay[i] = (int)(rng() % 200);
  std::mutex wmu;
  int lasts = 0;
  uint32_t last_amax = 0xFFFFFFFFu, last_amax2 = 0xFFFFFFFFu;
  Residency res(resident);
  std::vector<std::thread> th;
  for (int i = 0; i < G; i++)
    th.emplace_back([&, i] {
      res.enter();
      std::this_thread::sleep_for(std::chrono::microseconds(delay[i]));
      uint32_t bits = 0, n = 0, bits2 = 0;
      const nvfp4::GridRole role =
          nvfp4::grid_arrive_wait<CpuOps>(s, (uint32_t)G, (uint32_t)i, vals[i], epoch, spin, &bits, &n,
                                          vals2[i], two ? &bits2 : nullptr);
      ok[i] = role != nvfp4::kGridGaveUp;
      got[i] = bits;
      got2[i] = bits2;
      if (ok[i]) { std::lock_guard<std::mutex> l(wmu); writes[i]++; }
      if (role == nvfp4::kGridPublisher) {
        std::vector<uint32_t> ws;
        for (uint32_t k = 0; k < n; k++) ws.push_back(nvfp4::grid_recovered<CpuOps>(s, k, uint64_t(1) << 22));
        std::lock_guard<std::mutex> l(wmu);
        lasts++;
        last_amax = bits;
        last_amax2 = bits2;
        for (uint32_t w : ws) {
          CHECK(w < (uint32_t)G);
          if (w < (uint32_t)G) writes[w]++;
        }
      }
      res.leave();
    });
  for (auto& t : th) t.join();
  int gave_up = 0;
  for (int i = 0; i < G; i++) {
    if (ok[i]) {
      CHECK(got[i] == want);
      if (two) CHECK(got2[i] == want2);
    } else {
      gave_up++;
    }
    CHECK(writes[i] == 1);
  }
  CHECK(lasts == 1);
  CHECK(last_amax == want);
  if (two) {
    CHECK(last_amax2 == want2);
    CHECK(s->result2 == (((uint64_t)want2 << 32) | epoch));
  }
  // the gate is closed for this epoch and carries the tensor amax
  CHECK((s->gate & nvfp4::kGateTagMask) == nvfp4::gate_tag(epoch));
  CHECK((s->gate & nvfp4::kGateClosed) != 0);
  CHECK((uint32_t)(s->gate >> 32) == want);
  CHECK(idle(s));
  return gave_up;
}

// one two-pass amax launch of G workgroups, at most `resident` at once
static void max_launch(GridSyncSlot* s, int G, int resident, std::mt19937& rng) {
  std::vector<uint32_t> v0(G), v1(G);
  uint32_t w0 = 0, w1 = 0;
  for (int i = 0; i < G; i++) {
    v0[i] = rng() >> 1;
    v1[i] = (rng() >> 1) & (rng() % 2 ? 0x7FFFFFFFu : 0xFFFFu);
    w0 = v0[i] > w0 ? v0[i] : w0;
    w1 = v1[i] > w1 ? v1[i] : w1;
  }
  std::vector<int> delay(G);
  for (int i = 0; i < G; i++) delay[i] = (int)(rng() % 100);
  std::mutex mu;
  int lasts = 0;
  uint32_t r0 = 0, r1 = 0;
  Residency res(resident);
  std::vector<std::thread> th;
  for (int i = 0; i < G; i++)
    th.emplace_back([&, i] {
      res.enter();
      std::this_thread::sleep_for(std::chrono::microseconds(delay[i]));
      uint32_t a = 0, b = 0;
      if (nvfp4::grid_max_arrive<CpuOps>(s, (uint32_t)G, (uint32_t)i, v0[i], v1[i], &a, &b)) {
        std::lock_guard<std::mutex> l(mu);
        lasts++;
        r0 = a;
        r1 = b;
      }
      res.leave();
    });
  for (auto& t : th) t.join();
  CHECK(lasts == 1);
  CHECK(r0 == w0);
  CHECK(r1 == w1);
  CHECK(idle(s));
}

int main() {
  std::mt19937 rng(1234);
  static GridSyncSlot slot;  // zero-initialized, as the device array
  uint32_t epoch = 0;
  // full residency, generous spin limit
  const int Gs[] = {1, 2, 3, 15, 16, 17, 33, 64, 200};
  for (int rep = 0; rep < 20 && !fails; rep++)
    for (int G : Gs) {
      CHECK(launch(&slot, ++epoch, G, G, uint64_t(1) << 22, rng, rep % 2 == 1) == 0);
      if (fails) break;
    }
  CHECK(slot.gave_ups == 0);
  if (fails) { std::printf("FAILED\n"); return 1; }
  // limited residency: must end, some give up, all blocks covered, the slot recovers
  for (int rep = 0; rep < 10; rep++) {
    const uint32_t before = slot.gave_ups;
    const int g = launch(&slot, ++epoch, 40, 6, 2000, rng, rep % 2 == 0);
    CHECK(g >= 1 && g <= 39);
    CHECK(slot.gave_ups == before + (uint32_t)g);
    CHECK(launch(&slot, ++epoch, 40, 40, uint64_t(1) << 22, rng) == 0);
    if (fails) break;
  }
  // spin limit zero, full residency
  for (int rep = 0; rep < 20 && !fails; rep++) launch(&slot, ++epoch, 24, 24, 0, rng, rep % 2 == 0);
  // no-wait grid maxima, alternating with single-pass launches on the slot
  const int Ms[] = {1, 2, 15, 16, 17, 31, 100, 300};
  for (int rep = 0; rep < 8 && !fails; rep++)
    for (int G : Ms) {
      max_launch(&slot, G, rep % 2 ? 4 : G, rng);
      CHECK(launch(&slot, ++epoch, 20, 20, uint64_t(1) << 22, rng, rep % 2 == 0) == 0);
      if (fails) break;
    }
  std::printf("%s\n", fails ? "FAILED" : "OK");
  return fails ? 1 : 0;
}
"""


def _build_and_run(tmp_path, extra):
    src = tmp_path / "grid_sync_emu.cpp"
    src.write_text(SRC)
    exe = tmp_path / ("emu" + ("_tsan" if extra else ""))
    cmd = ["g++", "-std=c++20", "-O1", "-g", "-pthread", "-I", HDR, *extra, "-o", str(exe), str(src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr


def test_grid_exchange_protocol(tmp_path):
    _build_and_run(tmp_path, [])


def test_grid_exchange_protocol_threadsanitizer(tmp_path):
    probe = subprocess.run(["g++", "-fsanitize=thread", "-x", "c++", "-", "-o", os.devnull],
                           input="int main(){return 0;}", capture_output=True, text=True)
    if probe.returncode != 0:
        pytest.skip("g++ has no ThreadSanitizer here")
    _build_and_run(tmp_path, ["-fsanitize=thread"])
