// Concurrent callers of libopt8's host code, linked with the host-only HIP
// stand-in and built with ThreadSanitizer by tests/test_host_sanitizers.py.
// Several threads step at once: a list they all share, on one stream they all
// use; on a stream of its own, each thread's lists that fit the caches under
// all three rules, and fresh lists every few steps (cache misses, slot
// rewrites, growth and releases under a 1 MiB byte budget); one thread also
// calls the entry point without allocation.  Every call must succeed, every
// launch must carry a well-formed descriptor list, and no staging buffer may
// be rewritten under a pending copy.  Prints "all thread checks passed".
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "fake_hip.h"
#include "opt8_host_limits.h"
#include "opt8.h"

using fake::g;

namespace {

std::atomic<int> failures{0};

// fake device addresses: tensor i owns a 2 GiB window, its six buffers 256 MiB apart
uintptr_t base_of(int i, int k) { return (uintptr_t(1) << 40) + (uintptr_t(i) << 31) + (uintptr_t(k) << 28); }

opt8_tensor tensor(int i, int64_t numel, int mode, uint32_t id) {
  opt8_tensor t;
  std::memset(&t, 0, sizeof t);
  t.param = reinterpret_cast<uint16_t*>(base_of(i, 0));
  t.grad = reinterpret_cast<const uint16_t*>(base_of(i, 1));
  t.m = reinterpret_cast<void*>(base_of(i, 2));
  t.v = reinterpret_cast<void*>(base_of(i, 3));
  t.absmax_m = mode == OPT8_STATE_8BIT ? reinterpret_cast<float*>(base_of(i, 4)) : nullptr;
  t.absmax_v = mode == OPT8_STATE_8BIT ? reinterpret_cast<float*>(base_of(i, 5)) : nullptr;
  t.numel = numel;
  t.tensor_id = id;
  t.mode = mode;
  return t;
}

opt8_hparams hparams(int64_t step) {
  opt8_hparams h;
  std::memset(&h, 0, sizeof h);
  h.lr = 1e-3;
  h.beta1 = 0.9;
  h.beta2 = 0.999;
  h.eps = 1e-8;
  h.weight_decay = 0.01;
  h.step = step;
  h.seed = 7;
  return h;
}

// a list of `count` tensors from window `first` on, sizes cycling through the
// kinds of work (8-bit full blocks, short and long last blocks, fp32 and bf16 state)
std::vector<opt8_tensor> make_list(int first, int count) {
  static const int64_t kSizes[] = {3 * 2048, 2048 + 7, 2048 + 300, 1000, 4096 + 5};
  static const int kModes[] = {OPT8_STATE_8BIT, OPT8_STATE_8BIT, OPT8_STATE_8BIT, OPT8_STATE_FP32,
                               OPT8_STATE_BF16_SR};
  std::vector<opt8_tensor> l;
  for (int k = 0; k < count; ++k)
    l.push_back(tensor(first + k, kSizes[(first + k) % 5], kModes[(first + k) % 5], static_cast<uint32_t>(k)));
  return l;
}

void expect_ok(int rc, const char* what, int thread, int step) {
  if (rc != OPT8_OK) {
    std::printf("FAILED thread %d step %d: %s returned %d (%s)\n", thread, step, what, rc, opt8_last_error());
    ++failures;
  }
}

constexpr int kThreads = 4;
constexpr int kSteps = 200;

void worker(int t, const std::vector<opt8_tensor>* shared) {
  void* stream = reinterpret_cast<void*>(uintptr_t(0x1000) + uintptr_t(t) * 0x100);
  void* shared_stream = reinterpret_cast<void*>(uintptr_t(0x900));
  std::vector<std::vector<opt8_tensor>> own;
  for (int k = 0; k < 6; ++k) own.push_back(make_list(1000 * (t + 1) + 10 * k, 3 + k));
  for (int s = 0; s < kSteps; ++s) {
    const opt8_hparams h = hparams(s + 1);
    const int32_t ns = static_cast<int32_t>(shared->size());
    // the shared buffers on one stream that all threads use (different streams need disjoint buffers)
    expect_ok(opt8_adamw_step(shared->data(), ns, &h, shared_stream), "shared list", t, s);
    const auto& mine = own[s % own.size()];
    const int32_t nm = static_cast<int32_t>(mine.size());
    if (s % 3 == 1) expect_ok(opt8_lion_step(mine.data(), nm, &h, stream), "lion", t, s);
    else if (s % 3 == 2) expect_ok(opt8_momentum_step(mine.data(), nm, &h, stream), "momentum", t, s);
    else expect_ok(opt8_adamw_step(mine.data(), nm, &h, stream), "own list", t, s);
    if (s % 5 == 0) {
      // a list never seen before: a miss that takes, rewrites or evicts a slot
      auto fresh = make_list(100000 + 1000 * (kSteps * t + s), 40);
      // with one tensor of 2^27 or 2^28 elements (a 256 or 512 KiB block map) the
      // budget makes misses rewrite other lists' slots, growing them, and release
      // least recently used ones
      const uintptr_t w = base_of(100000 + 1000 * (kSteps * t + s), 0);   // its 2 GiB window
      fresh[0].numel = int64_t{1} << (s % 10 == 5 ? 28 : 27);
      fresh[0].mode = OPT8_STATE_8BIT;
      fresh[0].param = reinterpret_cast<uint16_t*>(w);
      fresh[0].grad = reinterpret_cast<const uint16_t*>(w + (uintptr_t(1) << 29));
      fresh[0].m = reinterpret_cast<void*>(w + (uintptr_t(1) << 30));
      fresh[0].v = reinterpret_cast<void*>(w + (uintptr_t(5) << 28));
      fresh[0].absmax_m = reinterpret_cast<float*>(w + (uintptr_t(6) << 28));
      fresh[0].absmax_v = reinterpret_cast<float*>(w + (uintptr_t(7) << 28));
      expect_ok(opt8_adamw_step(fresh.data(), static_cast<int32_t>(fresh.size()), &h, stream), "fresh list", t, s);
    }
    // one thread only: concurrent calls of this entry point share the device's one array
    if (t == 0 && s % 7 == 0)
      expect_ok(opt8_adamw_step_noalloc(mine.data(), nm, &h, stream), "no-allocation entry", t, s);
  }
}

}  // namespace

int main() {
  setenv("OPT8_CACHE_MB", "1", 1);
  if (opt8_init_codebooks(nullptr, nullptr) != OPT8_OK) {
    std::printf("FAILED: init (%s)\n", opt8_last_error());
    return 1;
  }
  const std::vector<opt8_tensor> shared = make_list(10, 12);
  std::vector<std::thread> threads;
  for (int t = 0; t < kThreads; ++t) threads.emplace_back(worker, t, &shared);
  for (auto& th : threads) th.join();

  long bad = 0;
  for (const auto& L : g.launches) bad += L.ok ? 0 : 1;
  if (bad) {
    std::printf("FAILED: %ld of %zu launches had a malformed descriptor list\n", bad, g.launches.size());
    ++failures;
  }
  if (g.reuse_violations) {
    std::printf("FAILED: %ld staging buffers rewritten under a pending copy\n", g.reuse_violations);
    ++failures;
  }
  if (g.uploads <= g.mallocs || g.frees == 0) {
    std::printf("FAILED: the byte budget never made a miss rewrite or release a slot\n");
    ++failures;
  }
  if (static_cast<int>(g.device_live.size()) > opt8::kSlotCache) {
    std::printf("FAILED: %zu device buffers live, more than the slot cache holds\n", g.device_live.size());
    ++failures;
  }
  std::printf("%zu launches, %ld uploads, %ld device allocations, %ld frees from %d threads\n", g.launches.size(),
              g.uploads, g.mallocs, g.frees, kThreads);
  if (failures) return 1;
  std::printf("all thread checks passed\n");
  return 0;
}
