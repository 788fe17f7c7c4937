// Drives libopt8's host code (linked with the host-only HIP stand-in) through
// its tables, every validation error, capture refusal, launch planning, the
// scalar prologue and the descriptor cache.  Built with AddressSanitizer and
// UBSan by tests/test_host_sanitizers.py; prints "all host checks passed".
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "fake_hip.h"
#include "opt8_host_limits.h"
#include "opt8_launch.h"
#include "opt8.h"

using fake::g;

// Global allocation functions that fail on request, to check that an
// allocation failure inside the library comes back as a status, not an exception.
static bool g_fail_new = false;
void* operator new(std::size_t n) {
  if (g_fail_new) throw std::bad_alloc();
  void* p = std::malloc(n ? n : 1);
  if (!p) throw std::bad_alloc();
  return p;
}
void operator delete(void* p) noexcept { std::free(p); }
void operator delete(void* p, std::size_t) noexcept { std::free(p); }

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, opt8_last_error()); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

// Fake device addresses: tensor i owns a 2 GiB window, its six buffers 256 MiB apart
static uintptr_t base_of(int i, int k) { return (uintptr_t(1) << 40) + (uintptr_t(i) << 31) + (uintptr_t(k) << 28); }

static opt8_tensor tensor(int i, int64_t numel, int mode, uint32_t id) {
  opt8_tensor t;
  std::memset(&t, 0, sizeof t);
  t.param = reinterpret_cast<uint16_t*>(base_of(i, 0));
  t.grad = reinterpret_cast<const uint16_t*>(base_of(i, 1));
  t.m = reinterpret_cast<void*>(base_of(i, 2));
  t.v = reinterpret_cast<void*>(base_of(i, 3));
  t.absmax_m = mode == OPT8_STATE_8BIT ? reinterpret_cast<float*>(base_of(i, 4)) : nullptr;
  t.absmax_v = mode == OPT8_STATE_8BIT ? reinterpret_cast<float*>(base_of(i, 5)) : nullptr;
  t.numel = numel;
  t.index_base = 0;
  t.tensor_id = id;
  t.mode = mode;
  return t;
}

static opt8_hparams hparams(int64_t step) {
  opt8_hparams h;
  std::memset(&h, 0, sizeof h);
  h.lr = 1e-3;
  h.beta1 = 0.9;
  h.beta2 = 0.999;
  h.eps = 1e-8;
  h.weight_decay = 0.01;
  h.step = step;
  h.seed = 0x0123456789ABCDEFull;
  return h;
}

// The scalar prologue as defined: beta^t by t - 1 repeated double
// multiplications, each derived scalar rounded once to fp32.
static void expect_scalars(const opt8::StepScalars& s, const opt8_hparams& h, bool adamw) {
  double p1 = 1.0, p2 = 1.0;
  if (adamw) {
    p1 = h.beta1;
    p2 = h.beta2;
    // once 1 - p is exactly 1.0 for both, every later (smaller) power leaves it there
    for (int64_t k = 1; k < h.step && !(1.0 - p1 == 1.0 && 1.0 - p2 == 1.0); ++k) {
      p1 *= h.beta1;
      p2 *= h.beta2;
    }
  } else {
    p1 = p2 = 0.0;
  }
  CHECK(s.beta1 == static_cast<float>(h.beta1));
  CHECK(s.beta2 == static_cast<float>(h.beta2));
  CHECK(s.w1 == static_cast<float>(1.0 - h.beta1));
  CHECK(s.w2 == static_cast<float>(1.0 - h.beta2));
  CHECK(s.eps == static_cast<float>(h.eps));
  CHECK(s.step_size == static_cast<float>(h.lr / (1.0 - p1)));
  CHECK(s.rbc2 == static_cast<float>(1.0 / std::sqrt(1.0 - p2)));
  CHECK(s.lrwd == static_cast<float>(h.lr * h.weight_decay));
  CHECK(s.seed_lo == static_cast<uint32_t>(h.seed) && s.seed_hi == static_cast<uint32_t>(h.seed >> 32));
  CHECK(s.step_lo == static_cast<uint32_t>(h.step));
  CHECK(s.param_round == h.param_round && s.state_round == h.state_round);
}

static int step(const std::vector<opt8_tensor>& ts, const opt8_hparams& h, void* stream = nullptr) {
  return opt8_adamw_step(ts.data(), static_cast<int32_t>(ts.size()), &h, stream);
}

int main() {
  // the caches' byte budget for this run (read at the first step): 16 MiB, which the
  // lists below reach only in the budget check (the count checks stay within it)
  setenv("OPT8_CACHE_MB", "16", 1);
  // ---------------------------------------------------------------- tables
  g.have_device = false;
  float cs[256], cu[256];
  CHECK(opt8_init_codebooks(cs, cu) == OPT8_E_HIP);   // tables still copied out
  CHECK(cs[0] == -1.0f && cs[127] == 0.0f && cs[255] == 1.0f);
  CHECK(cu[0] == 0.0f && cu[255] == 1.0f);
  for (int k = 1; k < 256; ++k) CHECK(cs[k - 1] < cs[k] && cu[k - 1] < cu[k]);
  const opt8_hparams h1 = hparams(1);
  std::vector<opt8_tensor> one = {tensor(0, 5000, OPT8_STATE_8BIT, 0)};
  CHECK(step(one, h1) == OPT8_E_HIP);                  // no device
  g.have_device = true;
  CHECK(step(one, h1) == OPT8_E_NOT_INIT);
  CHECK(opt8_init_codebooks(nullptr, nullptr) == OPT8_OK);
  CHECK(opt8_init_codebooks(cs, cu) == OPT8_OK);       // idempotent: uploaded once
  CHECK(g.table_uploads == 1);
  g.device = 1;
  CHECK(step(one, h1) == OPT8_E_NOT_INIT);             // another device needs its own init
  g.device = 0;

  // ---------------------------------------------------------------- validation
  CHECK(opt8_adamw_step(one.data(), 1, nullptr, nullptr) == OPT8_E_NULL);
  CHECK(opt8_adamw_step(nullptr, 1, &h1, nullptr) == OPT8_E_NULL);
  CHECK(opt8_adamw_step(one.data(), -1, &h1, nullptr) == OPT8_E_SIZE);
  CHECK(opt8_adamw_step(nullptr, 0, &h1, nullptr) == OPT8_OK);
  auto bad = [&](void (*edit)(opt8_tensor&), int want) {
    std::vector<opt8_tensor> ts = {tensor(0, 5000, OPT8_STATE_8BIT, 0), tensor(1, 3000, OPT8_STATE_BF16_SR, 1)};
    edit(ts[1]);
    const size_t before = g.launches.size();
    CHECK(step(ts, h1) == want);
    CHECK(g.launches.size() == before);                // nothing queued on an error
  };
  bad([](opt8_tensor& t) { t.param = nullptr; }, OPT8_E_NULL);
  bad([](opt8_tensor& t) { t.v = nullptr; }, OPT8_E_NULL);
  bad([](opt8_tensor& t) { t.mode = OPT8_STATE_8BIT; }, OPT8_E_NULL);          // no absmax arrays
  bad([](opt8_tensor& t) { t.grad = reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(t.grad) + 8); }, OPT8_E_ALIGN);
  bad([](opt8_tensor& t) { t.numel = 0; }, OPT8_E_SIZE);
  bad([](opt8_tensor& t) { t.numel = (int64_t(1) << 42) + 1; }, OPT8_E_SIZE);
  bad([](opt8_tensor& t) { t.index_base = 1024; }, OPT8_E_SIZE);
  bad([](opt8_tensor& t) { t.index_base = (int64_t(1) << 60) + 2048; }, OPT8_E_SIZE);
  bad([](opt8_tensor& t) { t.mode = 7; }, OPT8_E_MODE);
  bad([](opt8_tensor& t) { t.tensor_id = 0; }, OPT8_E_DUPID);
  bad([](opt8_tensor& t) { t.m = reinterpret_cast<void*>(base_of(0, 0) + 4096); }, OPT8_E_ALIAS);
  {
    std::vector<opt8_tensor> ts = {tensor(0, 5000, OPT8_STATE_8BIT, 0)};
    opt8_hparams h = h1;
    const double nan = std::nan("");
    struct { double opt8_hparams::*f; double v; } cases[] = {
        {&opt8_hparams::lr, -1.0}, {&opt8_hparams::lr, nan}, {&opt8_hparams::beta1, 1.0},
        {&opt8_hparams::beta2, -0.1}, {&opt8_hparams::eps, 0.0}, {&opt8_hparams::weight_decay, -1.0},
        {&opt8_hparams::weight_decay, INFINITY}};
    for (auto& c : cases) {
      h = h1;
      h.*(c.f) = c.v;
      CHECK(step(ts, h) == OPT8_E_HPARAM);
    }
    h = h1;
    h.step = 0;
    CHECK(step(ts, h) == OPT8_E_HPARAM);
    h = h1;
    h.param_round = 5;
    CHECK(step(ts, h) == OPT8_E_MODE);
    h = h1;
    h.state_round = 3;
    CHECK(step(ts, h) == OPT8_E_MODE);
  }

  // ---------------------------------------------------------------- capture refusal
  g.capturing = true;
  {
    const size_t before = g.launches.size();
    const long up = g.uploads;
    CHECK(step(one, h1) == OPT8_E_CAPTURE);
    CHECK(g.launches.size() == before && g.uploads == up);
  }
  g.capturing = false;

  // ---------------------------------------------------------------- launch planning
  std::vector<opt8_tensor> mixed = {
      tensor(0, 100, OPT8_STATE_FP32, 10),  tensor(1, 4096, OPT8_STATE_8BIT, 11),
      tensor(2, 5000, OPT8_STATE_8BIT, 12), tensor(3, 3 * 2048, OPT8_STATE_8BIT, 13),
      tensor(4, 7, OPT8_STATE_BF16_SR, 14), tensor(5, 3000, OPT8_STATE_BF16_SR, 15),
      tensor(6, 2047, OPT8_STATE_8BIT, 16)};
  g.launches.clear();
  CHECK(step(mixed, h1) == OPT8_OK);
  CHECK(g.launches.size() == 4);
  if (g.launches.size() == 4) {
    const fake::Launch& a = g.launches[0];   // full 8-bit blocks: 2 + 2 + 3
    CHECK(a.kind == 0 && a.n == 3 && a.total_blocks == 7 && a.ok);
    CHECK(a.has_map);                        // the block map comes with the full 8-bit blocks only
    const fake::Launch& b = g.launches[1];   // bf16 state: 1 + 2 blocks
    CHECK(b.kind == 1 && b.n == 2 && b.total_blocks == 3 && b.ok);
    const fake::Launch& c = g.launches[2];   // fp32 state
    CHECK(c.kind == 2 && c.n == 1 && c.total_blocks == 1 && c.ok);
    const fake::Launch& d = g.launches[3];   // partial last blocks of 5000 and 2047
    CHECK(d.kind == 3 && d.n == 2 && d.total_blocks == 2 && d.ok);
    CHECK(!b.has_map && !c.has_map && !d.has_map);
    for (const auto& L : g.launches) CHECK(L.num_cu == 256 && L.resident == 256 * 3 && L.algo == 0);
    expect_scalars(a.sc, h1, true);
  }
  // partial last blocks of at most 64 elements go to the short-block kernel, under every rule
  {
    const std::vector<opt8_tensor> tails = {tensor(7, 4097, OPT8_STATE_8BIT, 20), tensor(8, 2048 + 64, OPT8_STATE_8BIT, 21),
                                            tensor(9, 2048 + 65, OPT8_STATE_8BIT, 22), tensor(10, 30, OPT8_STATE_8BIT, 23)};
    g.launches.clear();
    CHECK(step(tails, h1) == OPT8_OK);
    CHECK(g.launches.size() == 3);
    if (g.launches.size() == 3) {
      CHECK(g.launches[0].kind == 0 && g.launches[0].n == 3 && g.launches[0].total_blocks == 4 && g.launches[0].ok);
      CHECK(g.launches[1].kind == 3 && g.launches[1].n == 1 && g.launches[1].ok);           // 65 elements
      CHECK((g.launches[1].ids == std::vector<uint32_t>{22}));
      CHECK(g.launches[2].kind == 4 && g.launches[2].n == 3 && g.launches[2].total_blocks == 3 && g.launches[2].ok);
      CHECK((g.launches[2].ids == std::vector<uint32_t>{20, 21, 23}));                      // 1, 64 and 30 elements
    }
    g.launches.clear();
    CHECK(opt8_lion_step(tails.data(), static_cast<int32_t>(tails.size()), &h1, nullptr) == OPT8_OK);
    CHECK(g.launches.size() == 3);
    if (g.launches.size() == 3) {
      CHECK(g.launches[1].kind == 3 && g.launches[1].n == 1 && g.launches[1].algo == 1 && g.launches[1].ok);
      CHECK(g.launches[2].kind == 4 && g.launches[2].n == 3 && g.launches[2].algo == 1 && g.launches[2].ok);
    }
  }

  // a list that passed is not checked again while it stays byte-identical; edited in
  // place it is checked afresh
  {
    const opt8_tensor keep = mixed[3];
    mixed[3].grad = mixed[2].grad;                     // now overlaps tensor 2's gradient
    CHECK(step(mixed, h1) == OPT8_E_ALIAS);
    mixed[3] = keep;
    CHECK(step(mixed, h1) == OPT8_OK);
    mixed[6].tensor_id = 10;                           // duplicates tensor 0's id
    CHECK(step(mixed, h1) == OPT8_E_DUPID);
    mixed[6].tensor_id = 16;
    CHECK(step(mixed, h1) == OPT8_OK);
    // two lists alternating (two parameter groups) both stay cached
    for (int k = 0; k < 3; ++k) {
      CHECK(step(mixed, h1) == OPT8_OK);
      CHECK(step(one, h1) == OPT8_OK);
    }
    // a list that passed under a one-state rule (v unused, may be NULL) is still checked
    // under AdamW's
    std::vector<opt8_tensor> nov = one;
    nov[0].v = nullptr;
    nov[0].absmax_v = nullptr;
    CHECK(step(nov, h1) == OPT8_E_NULL);
    CHECK(opt8_lion_step(nov.data(), 1, &h1, nullptr) == OPT8_OK);
    CHECK(step(nov, h1) == OPT8_E_NULL);
  }

  // ---------------------------------------------------------------- scalar prologue
  {
    const int64_t steps[] = {1, 2, 3, 10, 1000, 5, 200000, 1, (int64_t(1) << 32) + 7};
    for (int64_t t : steps) {
      g.launches.clear();
      const opt8_hparams h = hparams(t);
      CHECK(step(one, h) == OPT8_OK);
      if (!g.launches.empty()) expect_scalars(g.launches[0].sc, h, true);
    }
    opt8_hparams h = hparams(3);
    h.beta1 = 0.5;
    h.beta2 = 0.25;
    h.param_round = OPT8_ROUND_NEAREST;
    h.state_round = OPT8_STATE_ROUND_STOCHASTIC;
    g.launches.clear();
    CHECK(step(one, h) == OPT8_OK);
    if (!g.launches.empty()) expect_scalars(g.launches[0].sc, h, true);
    g.launches.clear();
    CHECK(opt8_lion_step(one.data(), 1, &h, nullptr) == OPT8_OK);
    if (!g.launches.empty()) {
      expect_scalars(g.launches[0].sc, h, false);
      CHECK(g.launches[0].algo == 1);
    }
  }

  // ---------------------------------------------------------------- descriptor cache
  {
    std::vector<std::vector<opt8_tensor>> lists;
    for (int l = 0; l < opt8::kSlotCache + 2; ++l)
      lists.push_back({tensor(20 + 2 * l, 4096 + 64 * l, OPT8_STATE_8BIT, 0),
                       tensor(21 + 2 * l, 9000, OPT8_STATE_BF16_SR, 1)});
    for (int round = 0; round < 3; ++round)
      for (auto& L : lists) {
        const long up = g.uploads;
        CHECK(step(L, h1) == OPT8_OK);
        CHECK(g.uploads == up + 1);           // more lists than slots, round-robin: always a miss
        const long up2 = g.uploads;
        CHECK(step(L, h1) == OPT8_OK);
        CHECK(g.uploads == up2);              // the same list again: reused, no upload
      }
    CHECK(g.event_syncs > 0);                 // evictions waited for the last reader
    const long waits = g.stream_waits;
    void* other = reinterpret_cast<void*>(uintptr_t(0x1000));
    CHECK(step(lists.back(), h1, other) == OPT8_OK);
    CHECK(g.stream_waits == waits + 1);       // moved to another stream: ordered after the last launch
    CHECK(step(lists.back(), h1, other) == OPT8_OK);
    CHECK(g.stream_waits == waits + 1);

    // a list this thread has validated and planned, while another thread
    // rewrites every slot: uploaded again, and its launch reads its own descriptors
    {
      const std::vector<opt8_tensor> A = {tensor(60, 4096, OPT8_STATE_8BIT, 7),
                                          tensor(61, 4096, OPT8_STATE_8BIT, 8)};
      CHECK(step(A, h1) == OPT8_OK);
      long up = g.uploads;
      CHECK(step(A, h1) == OPT8_OK);
      CHECK(g.uploads == up);
      std::vector<int> rcs(opt8::kSlotCache, -1);
      std::thread writer([&] {
        for (int l = 0; l < opt8::kSlotCache; ++l)
          rcs[l] = step({tensor(6000 + l, 8192, OPT8_STATE_8BIT, 0)}, h1);
      });
      writer.join();
      for (int rc : rcs) CHECK(rc == OPT8_OK);
      up = g.uploads;
      g.launches.clear();
      CHECK(step(A, h1) == OPT8_OK);
      CHECK(g.uploads == up + 1);
      CHECK(g.launches.size() == 1 && g.launches[0].ok);
      if (g.launches.size() == 1) CHECK((g.launches[0].ids == std::vector<uint32_t>{7, 8}));
      CHECK(step(A, h1) == OPT8_OK);
      CHECK(g.uploads == up + 1);            // linked to its new slot
      // the other thread steps the same list: its own cache misses, the slot is found by content
      int rc_same = -1;
      std::thread reader([&] { rc_same = step(A, h1); });
      reader.join();
      CHECK(rc_same == OPT8_OK && g.uploads == up + 1);
    }

    // a list longer than any slot holds: the slot grows
    std::vector<opt8_tensor> big;
    for (int i = 0; i < 1000; ++i) big.push_back(tensor(100 + i, 2048 + i, OPT8_STATE_8BIT, static_cast<uint32_t>(i)));
    const long mallocs = g.mallocs;
    g.launches.clear();
    CHECK(step(big, h1) == OPT8_OK);
    CHECK(g.mallocs > mallocs);
    CHECK(g.launches.size() == 3 && g.launches[0].n == 1000 && g.launches[0].ok);
    if (g.launches.size() == 3) {   // last blocks of 65..999 elements, and of 1..64
      CHECK(g.launches[1].kind == 3 && g.launches[1].n == 935 && g.launches[1].ok);
      CHECK(g.launches[2].kind == 4 && g.launches[2].n == 64 && g.launches[2].ok);
    }
    // an overlap far down a long list is found
    big[999].grad = reinterpret_cast<const uint16_t*>(base_of(100 + 500, 1) + 1024);
    CHECK(step(big, h1) == OPT8_E_ALIAS);
    big[999] = tensor(100 + 999, 2048 + 999, OPT8_STATE_8BIT, 999);

    // an allocation failure is reported and leaves the cache usable
    std::vector<opt8_tensor> huge;
    for (int i = 0; i < 3000; ++i) huge.push_back(tensor(2000 + i, 4096, OPT8_STATE_8BIT, static_cast<uint32_t>(i)));
    g.fail_malloc = true;
    CHECK(step(huge, h1) == OPT8_E_HIP);
    g.fail_malloc = false;
    for (auto& L : lists) CHECK(step(L, h1) == OPT8_OK);
    CHECK(step(huge, h1) == OPT8_OK);
  }

  // ---------------------------------------------------------------- entry point without allocation
  {
    CHECK(g.scratch_queries == 1);            // the scratch address was taken once, at init
    auto noalloc = [](const std::vector<opt8_tensor>& ts, const opt8_hparams& h, void* stream = nullptr) {
      return opt8_adamw_step_noalloc(ts.data(), static_cast<int32_t>(ts.size()), &h, stream);
    };
    std::vector<opt8_tensor> mixed = {tensor(300, 5000, OPT8_STATE_8BIT, 0), tensor(301, 9000, OPT8_STATE_BF16_SR, 1),
                                      tensor(302, 100, OPT8_STATE_FP32, 2), tensor(303, 4096, OPT8_STATE_8BIT, 3)};
    std::vector<opt8_tensor> big;
    for (int i = 0; i < 4096; ++i) big.push_back(tensor(400 + i, 2048 + 7, OPT8_STATE_8BIT, static_cast<uint32_t>(i)));
    const long mallocs = g.mallocs, host_mallocs = g.host_mallocs, frees = g.frees, syncs = g.event_syncs;
    for (int round = 0; round < 3; ++round) {
      for (const auto* L : {&mixed, &big}) {
        g.launches.clear();
        const long up = g.uploads;
        CHECK(noalloc(*L, h1) == OPT8_OK);
        CHECK(g.uploads == up + 1);           // one copy into the scratch per call, never cached
        bool in_scratch = !g.launches.empty();
        for (const auto& x : g.launches)
          in_scratch = in_scratch && x.ok && x.list >= g.scratch_lo && x.list < g.scratch_hi && !x.has_map;
        CHECK(in_scratch);                    // every launch reads the scratch array, and searches (no map)
      }
    }
    CHECK(g.launches.size() == 2 && g.launches[0].n == 4096 && g.launches[1].n == 4096);   // 4096 + 4096 tails
    CHECK(g.mallocs == mallocs && g.host_mallocs == host_mallocs && g.frees == frees);   // nothing allocated
    CHECK(g.event_syncs == syncs);            // and no waiting on the host
    big.push_back(tensor(400 + 4096, 4096, OPT8_STATE_8BIT, 4096));
    g.launches.clear();
    const long up = g.uploads;
    CHECK(noalloc(big, h1) == OPT8_E_SIZE);   // over the limit: refused, nothing queued
    CHECK(g.launches.empty() && g.uploads == up);
    CHECK(std::strstr(opt8_last_error(), "at most 4096") != nullptr);
    g.capturing = true;
    CHECK(noalloc(mixed, h1) == OPT8_E_CAPTURE);
    g.capturing = false;
    std::vector<opt8_tensor> dup = mixed;
    dup[2].tensor_id = 0;
    CHECK(noalloc(dup, h1) == OPT8_E_DUPID);  // the same validation as opt8_adamw_step
    CHECK(g.launches.empty() && g.uploads == up);
    // the cached entry point still works alongside
    CHECK(step(mixed, h1) == OPT8_OK);
  }

  // host allocation failure: a status and a message, nothing queued, and the
  // same list steps normally once memory is back
  {
    const std::vector<opt8_tensor> L = {tensor(90, 8192, OPT8_STATE_8BIT, 0)};
    g.launches.clear();
    const long up = g.uploads;
    g_fail_new = true;
    const int rc = step(L, h1);
    g_fail_new = false;
    CHECK(rc == OPT8_E_NOMEM);
    CHECK(g.launches.empty() && g.uploads == up);
    CHECK(std::strstr(opt8_last_error(), "host memory") != nullptr);
    CHECK(step(L, h1) == OPT8_OK);
    CHECK(g.launches.size() == 1);
  }

  // a launch that fails right after its list was uploaded: the slot's event
  // follows the upload, so a later rewrite of that slot's staging buffer waits
  // for the copy; and the list steps normally afterwards
  {
    const std::vector<opt8_tensor> F = {tensor(1300, 8192, OPT8_STATE_8BIT, 0)};
    g.fail_launch_kind = 0;
    const long up = g.uploads;
    CHECK(step(F, h1) == OPT8_E_HIP);
    g.fail_launch_kind = -1;
    CHECK(g.uploads == up + 1);
    CHECK(std::strstr(opt8_last_error(), "already queued: nothing") != nullptr);
    for (int l = 0; l <= opt8::kSlotCache; ++l)   // more new lists than slots: every slot rewritten
      CHECK(step({tensor(6100 + l, 8192, OPT8_STATE_8BIT, 0)}, h1) == OPT8_OK);
    g.launches.clear();
    CHECK(step(F, h1) == OPT8_OK);
    CHECK(g.launches.size() == 1 && g.launches[0].ok);
  }

  // one list per parameter group, more groups than a cache of four would keep: once each has
  // been seen, every list stays validated and uploaded and no call waits for an earlier step
  {
    std::vector<std::vector<opt8_tensor>> groups;
    for (int l = 0; l < 40; ++l) groups.push_back({tensor(6200 + l, 4096, OPT8_STATE_8BIT, 0)});
    const long fills = g.map_fills;
    for (auto& L : groups) CHECK(step(L, h1) == OPT8_OK);
    CHECK(g.map_fills == fills + 40);         // each upload fills its block map on the device
    const long up = g.uploads, syncs = g.event_syncs;
    for (int round = 0; round < 2; ++round)
      for (auto& L : groups) CHECK(step(L, h1) == OPT8_OK);
    CHECK(g.uploads == up && g.event_syncs == syncs && g.map_fills == fills + 40);
  }

  // the byte budget (16 MiB in this run) bounds both caches whatever their counts: lists with
  // 4 MiB block maps stay a few at a time, the oldest is dropped (its slot rewritten only after
  // the launches that read it: the check on reuse_violations below) and uploaded again, and the
  // slots' device memory stays within the budget plus one list
  {
    auto huge_tensor = [](int j) {   // 2^31 elements (2^20 blocks), its buffers 8 GiB apart
      opt8_tensor t;
      std::memset(&t, 0, sizeof t);
      const uintptr_t b = (uintptr_t(1) << 44) + (uintptr_t(j) << 36);
      t.param = reinterpret_cast<uint16_t*>(b);
      t.grad = reinterpret_cast<const uint16_t*>(b + (uintptr_t(1) << 33));
      t.m = reinterpret_cast<void*>(b + (uintptr_t(2) << 33));
      t.v = reinterpret_cast<void*>(b + (uintptr_t(3) << 33));
      t.absmax_m = reinterpret_cast<float*>(b + (uintptr_t(4) << 33));
      t.absmax_v = reinterpret_cast<float*>(b + (uintptr_t(5) << 33));
      t.numel = int64_t(1) << 31;
      t.mode = OPT8_STATE_8BIT;
      return t;
    };
    std::vector<std::vector<opt8_tensor>> big;
    for (int l = 0; l < 6; ++l) big.push_back({huge_tensor(l)});
    for (auto& L : big) CHECK(step(L, h1) == OPT8_OK);
    const size_t list_bytes = (size_t(1) << 20) * 4 + 1024;   // one list: its map and descriptor
    CHECK(g.device_bytes <= (size_t(16) << 20) + 2 * list_bytes);
    const long up = g.uploads;
    CHECK(step(big[5], h1) == OPT8_OK);       // the newest stays
    CHECK(g.uploads == up);
    CHECK(step(big[0], h1) == OPT8_OK);       // the oldest was dropped: uploaded again
    CHECK(g.uploads == up + 1);
    g.launches.clear();
    CHECK(step(big[0], h1) == OPT8_OK);
    CHECK(g.uploads == up + 1 && g.launches.size() == 1 && g.launches[0].ok);
  }

  // lists whose buffers move every step (every call a miss): once the budget is full, slots are
  // rewritten, not freed and allocated again (freeing device memory waits for the device)
  {
    auto moved = [](int k) {   // the same 2^31-element tensor, its gradient 16 bytes further each time
      opt8_tensor t;
      std::memset(&t, 0, sizeof t);
      const uintptr_t b = (uintptr_t(1) << 45);
      t.param = reinterpret_cast<uint16_t*>(b);
      t.grad = reinterpret_cast<const uint16_t*>(b + (uintptr_t(1) << 33) + 16 * uintptr_t(k));
      t.m = reinterpret_cast<void*>(b + (uintptr_t(2) << 33));
      t.v = reinterpret_cast<void*>(b + (uintptr_t(3) << 33));
      t.absmax_m = reinterpret_cast<float*>(b + (uintptr_t(4) << 33));
      t.absmax_v = reinterpret_cast<float*>(b + (uintptr_t(5) << 33));
      t.numel = int64_t(1) << 31;
      t.mode = OPT8_STATE_8BIT;
      return std::vector<opt8_tensor>{t};
    };
    for (int k = 0; k < 8; ++k) CHECK(step(moved(k), h1) == OPT8_OK);
    const long mallocs = g.mallocs, frees = g.frees, up = g.uploads;
    for (int k = 8; k < 24; ++k) CHECK(step(moved(k), h1) == OPT8_OK);
    CHECK(g.uploads == up + 16);                        // every call a miss, uploaded
    CHECK(g.mallocs == mallocs && g.frees == frees);    // into slots that are rewritten
    CHECK(g.device_bytes <= (size_t(16) << 20) + 2 * ((size_t(1) << 22) + 1024));
  }
  CHECK(g.reuse_violations == 0);   // no staging buffer was rewritten or freed under its copy

  // launch sizes: the measured counts per CU on the big lists, two blocks per wave on a list of
  // small tensors, and for every list size a grid of at least one workgroup, no more workgroups
  // than blocks / 4, a multiple of 32 from 64 on, and
  // at least the resident count while there are blocks for it
  {
    using opt8::Kind;
    CHECK((opt8::launch_groups<Kind::k8bit, opt8::kAdamW>(3251174, 256, 768) == 192 * 256));
    CHECK((opt8::launch_groups<Kind::k8bit, opt8::kLion>(3251174, 256, 512) == 96 * 256));
    CHECK((opt8::launch_groups<Kind::k8bit, opt8::kMomentum>(3251174, 256, 512) == 384 * 256));
    CHECK((opt8::launch_groups<Kind::k8bit, opt8::kMomentum, true>(3251174, 256, 512) == 96 * 256));
    CHECK((opt8::launch_groups<Kind::k8bit, opt8::kAdamW, true>(3251174, 256, 768) == 192 * 256));
    CHECK((opt8::launch_groups<Kind::kBf16, opt8::kAdamW>(1294710, 256, 1280) == 384 * 256));
    CHECK((opt8::launch_groups<Kind::k8bit, opt8::kAdamW>(60000, 256, 768) == 60000 / 8 / 32 * 32));
    CHECK((opt8::launch_groups<Kind::kFp32, opt8::kAdamW>(30000, 256, 1280) == 7500 / 32 * 32));
    CHECK((opt8::launch_groups<Kind::k8bitTail, opt8::kAdamW>(30000, 256, 768) == 768));
    bool ok = true;
    for (int64_t blocks = 1; blocks < 4000000; blocks = blocks * 3 / 2 + 1) {
      const int64_t grids[5] = {opt8::launch_groups<Kind::k8bit, opt8::kAdamW>(blocks, 256, 768),
                                opt8::launch_groups<Kind::k8bit, opt8::kLion>(blocks, 256, 512),
                                opt8::launch_groups<Kind::kBf16, opt8::kAdamW>(blocks, 256, 1280),
                                opt8::launch_groups<Kind::kFp32, opt8::kMomentum>(blocks, 256, 1280),
                                opt8::launch_groups<Kind::k8bitTail, opt8::kAdamW>(blocks, 256, 768)};
      const int64_t resident[5] = {768, 512, 1280, 1280, 768};
      for (int k = 0; k < 5; ++k) {
        const int64_t gsz = grids[k];
        ok = ok && gsz >= 1 && gsz <= (blocks + 3) / 4 && (gsz < 64 || gsz % 32 == 0);
        ok = ok && gsz >= std::min<int64_t>(resident[k], (blocks + 3) / 4) / 32 * 32;
      }
    }
    CHECK(ok);
  }

  if (failures) {
    std::printf("%d host checks failed\n", failures);
    return 1;
  }
  std::printf("all host checks passed\n");
  return 0;
}
