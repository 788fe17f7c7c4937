// Host side of libopt8: codebook construction, step scalars, argument
// validation, the per-device descriptor cache and the C entry points.
#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/opt8.h"
#include "opt8_host_limits.h"
#include "opt8_internal.h"
#include "opt8_map.h"

namespace opt8 {
namespace {

// the calling thread's last error message (a fixed buffer: reporting an
// allocation failure must not allocate)
thread_local char t_error[512];

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(t_error, sizeof t_error, fmt, ap);
  va_end(ap);
  return code;
}

// No exception crosses the C ABI: host allocation failures become OPT8_E_NOMEM.
template <class F>
int guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(OPT8_E_NOMEM, "out of host memory");
  } catch (...) {
    return fail(OPT8_E_HIP, "internal error: unexpected exception");
  }
}

// ----------------------------------------------------------------------------- codebooks
struct Tables {
  alignas(16) uint8_t bytes[kTableBytesSR];
  const float* cb_s() const { return reinterpret_cast<const float*>(bytes + kOffCbS); }
  const float* cb_u() const { return reinterpret_cast<const float*>(bytes + kOffCbU); }
  bool ok = false;
};

Tables make_tables() {
  Tables t;
  t.ok = build_table_image(t.bytes);
  return t;
}

const Tables& tables() {
  static const Tables t = make_tables();
  return t;
}

// ----------------------------------------------------------------------------- scalars
// beta^t by repeated double multiplication (no pow), cached per beta pair so a
// training run advances it incrementally; once both powers are below 2^-60,
// 1 - beta^t is exactly 1.0 in double and further products cannot change it.
struct PowCache {
  double b1 = -1, b2 = -1, p1 = 1, p2 = 1;
  int64_t t = 0;
};

void beta_powers(double b1, double b2, int64_t t, PowCache& c, double& p1, double& p2) {
  if (c.b1 != b1 || c.b2 != b2 || c.t > t) c = PowCache{b1, b2, 1.0, 1.0, 0};
  const double tiny = std::ldexp(1.0, -60);
  while (c.t < t) {
    if (c.p1 < tiny && c.p2 < tiny) { c.t = t; break; }
    c.p1 *= b1;
    c.p2 *= b2;
    ++c.t;
  }
  p1 = c.p1;
  p2 = c.p2;
}

StepScalars make_scalars(const opt8_hparams& hp, int algo, PowCache& cache) {
  // Lion and momentum have no bias correction
  double b1t = 0.0, b2t = 0.0;
  if (algo == kAdamW) beta_powers(hp.beta1, hp.beta2, hp.step, cache, b1t, b2t);
  const double bc1 = 1.0 - b1t;
  const double bc2 = 1.0 - b2t;
  StepScalars s;
  s.beta1 = static_cast<float>(hp.beta1);
  s.beta2 = static_cast<float>(hp.beta2);
  s.w1 = static_cast<float>(1.0 - hp.beta1);
  s.w2 = static_cast<float>(1.0 - hp.beta2);
  s.eps = static_cast<float>(hp.eps);
  s.step_size = static_cast<float>(hp.lr / bc1);
  s.rbc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  s.lrwd = static_cast<float>(hp.lr * hp.weight_decay);
  s.lr = static_cast<float>(hp.lr);
  s.seed_lo = static_cast<uint32_t>(hp.seed);
  s.seed_hi = static_cast<uint32_t>(hp.seed >> 32);
  s.step_lo = static_cast<uint32_t>(hp.step);
  s.param_round = hp.param_round;
  s.state_round = hp.state_round;
  return s;
}

// ----------------------------------------------------------------------------- validation
size_t state_bytes(int mode) { return mode == OPT8_STATE_8BIT ? 1 : mode == OPT8_STATE_BF16_SR ? 2 : 4; }
int64_t nblocks_of(int64_t numel) { return (numel + kBlock - 1) / kBlock; }

int validate_hparams(const opt8_hparams& hp, int algo) {
  if (!(std::isfinite(hp.lr) && hp.lr >= 0)) return fail(OPT8_E_HPARAM, "lr must be finite and >= 0 (got %g)", hp.lr);
  if (!(hp.beta1 >= 0 && hp.beta1 < 1)) return fail(OPT8_E_HPARAM, "beta1 must be in [0, 1) (got %g)", hp.beta1);
  if (!(hp.beta2 >= 0 && hp.beta2 < 1)) return fail(OPT8_E_HPARAM, "beta2 must be in [0, 1) (got %g)", hp.beta2);
  if (algo == kAdamW && !(std::isfinite(hp.eps) && hp.eps > 0))
    return fail(OPT8_E_HPARAM, "eps must be finite and > 0 (got %g)", hp.eps);
  if (!(std::isfinite(hp.weight_decay) && hp.weight_decay >= 0))
    return fail(OPT8_E_HPARAM, "weight_decay must be finite and >= 0 (got %g)", hp.weight_decay);
  if (hp.step < 1) return fail(OPT8_E_HPARAM, "step is 1-based (got %lld)", static_cast<long long>(hp.step));
  if (hp.state_round != OPT8_STATE_ROUND_NEAREST && hp.state_round != OPT8_STATE_ROUND_STOCHASTIC)
    return fail(OPT8_E_MODE, "unknown state_round %d", hp.state_round);
  if (hp.param_round != OPT8_ROUND_STOCHASTIC && hp.param_round != OPT8_ROUND_NEAREST)
    return fail(OPT8_E_MODE, "unknown param_round %d", hp.param_round);
  return OPT8_OK;
}

struct Range {
  uintptr_t lo, hi;
  int tensor;
  const char* what;
};

// Two-state rules (AdamW) use v and absmax_v; one-state rules ignore them.
int validate_tensors(const opt8_tensor* t, int32_t n, bool two_state) {
  std::vector<Range> ranges;
  std::vector<uint32_t> ids;
  ranges.reserve(static_cast<size_t>(n) * 6);
  ids.reserve(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    const opt8_tensor& x = t[i];
    if (x.mode != OPT8_STATE_8BIT && x.mode != OPT8_STATE_BF16_SR && x.mode != OPT8_STATE_FP32)
      return fail(OPT8_E_MODE, "tensor %d: unknown state mode %d", i, x.mode);
    if (!x.param || !x.grad || !x.m || (two_state && !x.v))
      return fail(OPT8_E_NULL, two_state ? "tensor %d: NULL param/grad/m/v" : "tensor %d: NULL param/grad/m", i);
    const bool q8 = x.mode == OPT8_STATE_8BIT;
    if (q8 && (!x.absmax_m || (two_state && !x.absmax_v)))
      return fail(OPT8_E_NULL, two_state ? "tensor %d: 8-bit mode needs absmax_m/absmax_v"
                                         : "tensor %d: 8-bit mode needs absmax_m", i);
    if (x.numel <= 0) return fail(OPT8_E_SIZE, "tensor %d: numel must be > 0", i);
    // the kernels hold a tensor's block count in 32 bits: at most 2^42 elements (2^31 blocks)
    if (x.numel > (int64_t(1) << 42))
      return fail(OPT8_E_SIZE, "tensor %d: numel %lld exceeds 2^42", i, static_cast<long long>(x.numel));
    if (x.index_base < 0 || x.index_base % kBlock != 0 || x.index_base > (int64_t(1) << 60))
      return fail(OPT8_E_SIZE, "tensor %d: index_base must be >= 0 and a multiple of 2048", i);
    auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
    if (!al(x.param, 16) || !al(x.grad, 16) || !al(x.m, 16) || (two_state && !al(x.v, 16)))
      return fail(OPT8_E_ALIGN, "tensor %d: param/grad/state buffers must be 16-byte aligned", i);
    if (q8 && (!al(x.absmax_m, 4) || (two_state && !al(x.absmax_v, 4))))
      return fail(OPT8_E_ALIGN, "tensor %d: absmax arrays must be 4-byte aligned", i);
    const uintptr_t ne = static_cast<uintptr_t>(x.numel);
    const uintptr_t sb = state_bytes(x.mode);
    auto add = [&](const void* p, uintptr_t bytes, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      ranges.push_back(Range{lo, lo + bytes, i, what});
    };
    add(x.param, 2 * ne, "param");
    add(x.grad, 2 * ne, "grad");
    add(x.m, sb * ne, "m");
    if (two_state) add(x.v, sb * ne, "v");
    if (q8) {
      const uintptr_t ab = 4 * static_cast<uintptr_t>(nblocks_of(x.numel));
      add(x.absmax_m, ab, "absmax_m");
      if (two_state) add(x.absmax_v, ab, "absmax_v");
    }
    ids.push_back(x.tensor_id);
  }
  std::sort(ids.begin(), ids.end());
  for (size_t k = 1; k < ids.size(); ++k)
    if (ids[k] == ids[k - 1]) return fail(OPT8_E_DUPID, "tensor_id %u appears twice", ids[k]);
  std::sort(ranges.begin(), ranges.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t k = 1; k < ranges.size(); ++k)
    if (ranges[k].lo < ranges[k - 1].hi)
      return fail(OPT8_E_ALIAS, "buffers overlap: tensor %d %s and tensor %d %s", ranges[k - 1].tensor,
                  ranges[k - 1].what, ranges[k].tensor, ranges[k].what);
  return OPT8_OK;
}

// ----------------------------------------------------------------------------- launch plans
constexpr int kKinds = 5;

// The device-side form of a tensor list: one sub-list per kernel, each with its
// own block numbering (full blocks of 8-bit tensors, bf16-state tensors,
// fp32-state tensors, the partial last block of 8-bit tensors longer than
// kShortTail elements, and those of at most kShortTail elements, which the
// short-block kernel packs eight to a wave), in that order.
struct Plan {
  std::vector<DevTensor> list;
  int count[kKinds] = {};
  int first[kKinds] = {};
  int64_t blocks[kKinds] = {};
};

// Descriptor-sized device units after the descriptors that hold the block map:
// for every full 8-bit block, the entry of its sub-list that holds it (the
// kernels read it instead of searching the descriptors; filled on the device
// after each upload, launch_block_map).
size_t map_units(const Plan& p) {
  const size_t blocks = static_cast<size_t>(p.blocks[static_cast<int>(Kind::k8bit)]);
  return (blocks * sizeof(uint32_t) + sizeof(DevTensor) - 1) / sizeof(DevTensor);
}

// Blocks tensor `x` contributes to the sub-list of `kind` (0: not in it).
int64_t blocks_in_kind(const opt8_tensor& x, int kind) {
  const bool tail = kind == static_cast<int>(Kind::k8bitTail) || kind == static_cast<int>(Kind::k8bitShort);
  const int mode = tail ? OPT8_STATE_8BIT : kind;
  if (x.mode != mode) return 0;
  if (tail) {
    const int64_t rest = x.numel % kBlock;
    const bool short_tail = rest > 0 && rest <= kShortTail;
    if (kind == static_cast<int>(Kind::k8bitShort)) return short_tail ? 1 : 0;
    return (rest > 0 && !short_tail) ? 1 : 0;
  }
  if (kind == static_cast<int>(Kind::k8bit)) return x.numel / kBlock;
  return nblocks_of(x.numel);
}

// Two passes over the caller's array: count each sub-list, then place every
// descriptor at its final position.
void build_plan(const opt8_tensor* t, int32_t n, bool two_state, Plan& p) {
  // reset in place: the vector keeps its capacity for the next list
  p.list.clear();
  for (int kind = 0; kind < kKinds; ++kind) {
    p.count[kind] = 0;
    p.first[kind] = 0;
    p.blocks[kind] = 0;
  }
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i)
    for (int kind = 0; kind < kKinds; ++kind)
      if (blocks_in_kind(t[i], kind)) ++p.count[kind];
  for (int kind = 0; kind < kKinds; ++kind) {
    p.first[kind] = static_cast<int>(total);
    total += p.count[kind];
  }
  p.list.resize(static_cast<size_t>(total));
  int pos[kKinds];
  for (int kind = 0; kind < kKinds; ++kind) pos[kind] = p.first[kind];
  for (int32_t i = 0; i < n; ++i) {
    const opt8_tensor& x = t[i];
    const bool q8 = x.mode == OPT8_STATE_8BIT;
    for (int kind = 0; kind < kKinds; ++kind) {
      const int64_t nb = blocks_in_kind(x, kind);
      if (!nb) continue;
      DevTensor& d = p.list[pos[kind]++];
      d.param = x.param;
      d.grad = x.grad;
      d.m = x.m;
      d.v = two_state ? x.v : nullptr;
      d.amax_m = q8 ? x.absmax_m : nullptr;
      d.amax_v = (two_state && q8) ? x.absmax_v : nullptr;
      d.numel = x.numel;
      d.index_base = x.index_base;
      d.block_begin = p.blocks[kind];
      d.tensor_id = x.tensor_id;
      d.nblocks = static_cast<uint32_t>(nb);
      p.blocks[kind] += nb;
    }
  }
}

// Validation and the launch plan are pure functions of the descriptor values,
// and a training loop passes the same lists every step (two for parameters
// with and without weight decay, one per group where every layer has its own
// learning rate): each thread keeps copies of the lists that passed, with
// their plans, and a list identical to one of them (byte for byte, same rule)
// is neither checked nor planned again.  A hit costs one memcmp instead of
// sorting 6n ranges and building 2n descriptors and the block map.
struct ValidatedList {
  std::vector<opt8_tensor> list;
  uint64_t hash = 0;   // list_hash of the list, compared before its bytes
  bool two_state = false;
  bool valid = false;
  uint64_t stamp = 0;
  Plan plan;
  // the device descriptor slot that held plan.list when it was last uploaded;
  // the link holds while that slot's generation is unchanged
  int slot_dev = -1;
  int slot_index = -1;
  uint64_t slot_gen = 0;
};
struct ValidatedCache {
  std::vector<ValidatedList> entry;   // grows to kListCache entries (capacity reserved: addresses stay)
  uint64_t clock = 0;
};
thread_local ValidatedCache t_validated;

// A filter before the byte compare, in constant time: FNV-1a over the count and
// the 8-byte words of the first and last four descriptors (lists that differ
// only in between share it and are told apart by the compare).
uint64_t list_hash(const opt8_tensor* t, int32_t n) {
  static_assert(sizeof(opt8_tensor) % sizeof(uint64_t) == 0, "descriptor size");
  constexpr size_t kWords = sizeof(opt8_tensor) / sizeof(uint64_t);
  uint64_t h = (0xCBF29CE484222325ull ^ static_cast<uint64_t>(n)) * 0x100000001B3ull;
  auto mix = [&](int32_t i) {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(t + i);
    for (size_t k = 0; k < kWords; ++k) {
      uint64_t w;
      std::memcpy(&w, p + k * sizeof w, sizeof w);
      h = (h ^ w) * 0x100000001B3ull;
    }
  };
  for (int32_t i = 0; i < std::min<int32_t>(n, 4); ++i) mix(i);
  for (int32_t i = std::max<int32_t>(4, n - 4); i < n; ++i) mix(i);
  return h;
}

// The byte budget of each cache (kCacheBytesDefault, or OPT8_CACHE_MB).
size_t cache_budget() {
  static const size_t bytes = [] {
    const char* e = std::getenv("OPT8_CACHE_MB");
    const long long mb = e ? std::atoll(e) : 0;
    return mb > 0 ? static_cast<size_t>(mb) << 20 : kCacheBytesDefault;
  }();
  return bytes;
}

size_t entry_bytes(const ValidatedList& e) {
  return e.list.capacity() * sizeof(opt8_tensor) + e.plan.list.capacity() * sizeof(DevTensor);
}

// Invalidates an entry; with release its memory is freed (budget eviction),
// else kept for the list that replaces it (the vectors' capacity is reused).
void drop_entry(ValidatedList& e, bool release) {
  e.valid = false;
  if (release) {
    std::vector<opt8_tensor>().swap(e.list);
    e.plan = Plan{};
  }
  e.slot_dev = -1;
  e.slot_index = -1;
}

int validate_tensors_cached(const opt8_tensor* t, int32_t n, bool two_state, ValidatedList*& out) {
  ValidatedCache& c = t_validated;
  if (c.entry.capacity() < static_cast<size_t>(kListCache)) c.entry.reserve(kListCache);
  ++c.clock;
  const size_t bytes = sizeof(opt8_tensor) * static_cast<size_t>(n);
  const uint64_t hash = list_hash(t, n);
  ValidatedList* victim = nullptr;
  for (ValidatedList& e : c.entry) {
    if (e.valid && e.hash == hash && e.two_state == two_state && e.list.size() == static_cast<size_t>(n) &&
        std::memcmp(e.list.data(), t, bytes) == 0) {
      e.stamp = c.clock;
      out = &e;
      return OPT8_OK;
    }
    if (!victim || (victim->valid && (!e.valid || e.stamp < victim->stamp))) victim = &e;
  }
  const int rc = validate_tensors(t, n, two_state);
  if (rc != OPT8_OK) return rc;
  // a new entry while there is room, else an empty or the least recently used one
  if (c.entry.size() < static_cast<size_t>(kListCache) && (!victim || victim->valid)) {
    c.entry.emplace_back();
    victim = &c.entry.back();
  }
  drop_entry(*victim, false);
  victim->hash = hash;
  victim->list.assign(t, t + n);
  build_plan(t, n, two_state, victim->plan);
  victim->two_state = two_state;
  victim->slot_gen = 0;
  victim->valid = true;
  victim->stamp = c.clock;
  // over the byte budget: drop the least recently used other lists
  size_t total = 0;
  for (const ValidatedList& e : c.entry)
    if (e.valid) total += entry_bytes(e);
  while (total > cache_budget()) {
    ValidatedList* lru = nullptr;
    for (ValidatedList& e : c.entry)
      if (e.valid && &e != victim && (!lru || e.stamp < lru->stamp)) lru = &e;
    if (!lru) break;
    total -= entry_bytes(*lru);
    drop_entry(*lru, true);
  }
  out = victim;
  return OPT8_OK;
}

// ----------------------------------------------------------------------------- device state
// Descriptor lists live in device memory, one slot per distinct list; a list
// passed again (the usual training loop) is launched without a new upload.
constexpr int kMaxDevices = 64;
constexpr int kAlgos = 3;

struct Slot {
  DevTensor* dev = nullptr;
  DevTensor* host = nullptr;   // pinned staging buffer
  size_t cap = 0;              // descriptors
  std::vector<DevTensor> key;  // contents now on the device
  hipEvent_t done = nullptr;   // recorded after the last launch that read it
  hipStream_t last_stream = nullptr;
  bool used = false;
  uint64_t stamp = 0;
  uint64_t gen = 0;            // changes whenever the contents are rewritten
};

struct DeviceState {
  bool init = false;
  int num_cu = 0;
  DevTensor* scratch = nullptr;      // device address of the no-allocation descriptor array
  int occ[2][kAlgos][kKinds] = {};   // [state_round][algo][kind]
  // grows to kSlotCache slots (capacity reserved at init, so addresses stay);
  // never destroyed, like the device buffers it points to, which live until
  // the process ends (freeing them from a static destructor could run after
  // the HIP runtime has shut down)
  std::vector<Slot>& slots = *new std::vector<Slot>();
  uint64_t clock = 0;
  PowCache pow;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];
uint64_t g_slot_gen = 0;   // source of slot generations, unique across devices

int hip_fail(hipError_t e, const char* what) {
  return fail(OPT8_E_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

int current_device(int& dev) {
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(OPT8_E_HIP, "device index %d out of range", dev);
  return OPT8_OK;
}

int ensure_capacity(Slot& s, size_t count) {
  if (s.cap >= count) return OPT8_OK;
  size_t cap = std::max<size_t>(count, 64);
  cap = std::max(cap, s.cap * 2);
  if (s.dev) (void)hipFree(s.dev);
  if (s.host) (void)hipHostFree(s.host);
  s.dev = nullptr;
  s.host = nullptr;
  s.cap = 0;
  hipError_t e = hipMalloc(&s.dev, cap * sizeof(DevTensor));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(descriptors)");
  e = hipHostMalloc(&s.host, cap * sizeof(DevTensor), hipHostMallocDefault);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(descriptors)");
  s.cap = cap;
  return OPT8_OK;
}

// Frees a slot's buffers once the launches that read it and its last upload
// have finished.
int release_slot(Slot& s) {
  const hipError_t e = hipEventSynchronize(s.done);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  if (s.dev) (void)hipFree(s.dev);
  if (s.host) (void)hipHostFree(s.host);
  s.dev = nullptr;
  s.host = nullptr;
  s.cap = 0;
  s.used = false;
  std::vector<DevTensor>().swap(s.key);
  return OPT8_OK;
}

bool same_list(const std::vector<DevTensor>& a, const std::vector<DevTensor>& b) {
  return a.size() == b.size() && std::memcmp(a.data(), b.data(), a.size() * sizeof(DevTensor)) == 0;
}

// Marks slot `s`, which already holds the list, as used by work queued next on
// `stream`: that work is ordered after the launches that last read it.
int reuse_slot(DeviceState& ds, Slot& s, hipStream_t stream) {
  if (s.last_stream != stream) {
    const hipError_t e = hipStreamWaitEvent(stream, s.done, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  s.stamp = ++ds.clock;
  return OPT8_OK;
}

// Returns the slot holding `list` on the device, ordered before work queued
// next on `stream`.
int acquire_slot(DeviceState& ds, const Plan& plan, hipStream_t stream, Slot*& out) {
  const std::vector<DevTensor>& list = plan.list;
  for (Slot& s : ds.slots) {
    if (s.used && same_list(s.key, list)) {
      out = &s;
      return reuse_slot(ds, s, stream);
    }
  }
  ++ds.clock;
  // the descriptors, then the block map (a function of them, so the key stays the list)
  const size_t units = list.size() + map_units(plan);
  size_t total = 0;
  for (const Slot& o : ds.slots) total += o.cap * sizeof(DevTensor);
  // the slot to write: the smallest unused one that holds the list; else a new one while the
  // count and the byte budget allow; else the least recently used of those that hold it, its
  // buffers reused, or failing that the least recently used of all (so a loop whose lists
  // change every step rewrites slots instead of freeing and allocating device and pinned
  // memory, which waits for the device, on every call)
  Slot* victim = nullptr;
  for (Slot& o : ds.slots)
    if (!o.used && o.cap >= units && (!victim || o.cap < victim->cap)) victim = &o;
  if (!victim && ds.slots.size() < static_cast<size_t>(kSlotCache) &&
      total + units * sizeof(DevTensor) <= cache_budget()) {
    hipEvent_t ev = nullptr;
    const hipError_t ce = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (ce != hipSuccess) return hip_fail(ce, "hipEventCreateWithFlags");
    ds.slots.emplace_back();
    victim = &ds.slots.back();
    victim->done = ev;
  }
  if (!victim) {
    for (Slot& o : ds.slots)
      if (o.cap >= units && (!victim || o.stamp < victim->stamp)) victim = &o;
  }
  if (!victim) {
    for (Slot& o : ds.slots)
      if (!victim || o.stamp < victim->stamp) victim = &o;
  }
  if (!victim) {   // no slot yet and the list alone exceeds the budget
    hipEvent_t ev = nullptr;
    const hipError_t ce = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (ce != hipSuccess) return hip_fail(ce, "hipEventCreateWithFlags");
    ds.slots.emplace_back();
    victim = &ds.slots.back();
    victim->done = ev;
  }
  Slot& s = *victim;
  // the last upload from the staging buffer and every launch that read the
  // slot have finished before either is rewritten (an event never recorded
  // counts as complete)
  hipError_t e = hipEventSynchronize(s.done);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  s.used = false;
  int rc = ensure_capacity(s, units);
  if (rc != OPT8_OK) return rc;
  // over the byte budget (a slot grew): free the least recently used other slots
  total = 0;
  for (const Slot& o : ds.slots) total += o.cap * sizeof(DevTensor);
  while (total > cache_budget()) {
    Slot* lru = nullptr;
    for (Slot& o : ds.slots)
      if (&o != &s && o.cap && (!lru || o.stamp < lru->stamp)) lru = &o;
    if (!lru) break;
    total -= lru->cap * sizeof(DevTensor);
    rc = release_slot(*lru);
    if (rc != OPT8_OK) return rc;
  }
  s.key = list;   // may throw: nothing is queued yet
  std::memcpy(s.host, list.data(), list.size() * sizeof(DevTensor));
  e = hipMemcpyAsync(s.dev, s.host, list.size() * sizeof(DevTensor), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(descriptors)");
  const int k8 = static_cast<int>(Kind::k8bit);
  e = launch_block_map(s.dev + plan.first[k8], plan.count[k8], reinterpret_cast<uint32_t*>(s.dev + list.size()),
                       stream);
  if (e != hipSuccess) {
    (void)hipEventRecord(s.done, stream);   // the copy above is queued: a rewrite waits for it
    return hip_fail(e, "block map launch");
  }
  // until the step's launches record it again, the event follows the upload
  e = hipEventRecord(s.done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  s.last_stream = stream;
  s.used = true;
  s.stamp = ds.clock;
  s.gen = ++g_slot_gen;
  out = &s;
  return OPT8_OK;
}

}  // namespace
}  // namespace opt8

using namespace opt8;

extern "C" int opt8_init_codebooks(float* signed_out, float* unsigned_out) {
  return guarded([&]() -> int {
    std::lock_guard<std::mutex> lock(g_mu);
    const Tables& t = tables();
    if (signed_out) std::memcpy(signed_out, t.cb_s(), sizeof(float) * kCodes);
    if (unsigned_out) std::memcpy(unsigned_out, t.cb_u(), sizeof(float) * kCodes);
    if (!t.ok) return fail(OPT8_E_HIP, "internal error: code lookup tables failed their construction check");
    int dev = 0;
    int rc = current_device(dev);
    if (rc != OPT8_OK) return rc;
    DeviceState& ds = g_dev[dev];
    if (ds.init) return OPT8_OK;
    hipError_t e = upload_tables(t.bytes);
    if (e != hipSuccess) return hip_fail(e, "upload of codebooks");
    // this device's copy of the descriptor scratch (each device has its own address)
    e = scratch_address(&ds.scratch);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    e = hipDeviceGetAttribute(&ds.num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
    for (int sr = 0; sr < 2; ++sr)
      for (int a = 0; a < kAlgos; ++a)
        for (int k = 0; k < kKinds; ++k) ds.occ[sr][a][k] = occupancy_per_cu(static_cast<Kind>(k), a, sr != 0);
    ds.slots.reserve(kSlotCache);
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    ds.init = true;
    return OPT8_OK;
  });
}

extern "C" int32_t opt8_default_mode(int64_t numel) {
  return numel < OPT8_FP32_STATE_THRESHOLD ? OPT8_STATE_FP32 : OPT8_STATE_8BIT;
}

extern "C" const char* opt8_last_error(void) { return t_error; }

namespace opt8 {
namespace {

// One step of update rule `algo` over a tensor list (every entry point).
// noalloc: the descriptor lists go to the device's fixed scratch array with
// one copy per call instead of the cached, allocated slots.
int run_step(int algo, const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp, void* hip_stream,
             bool noalloc = false) {
  t_error[0] = '\0';
  if (!hp) return fail(OPT8_E_NULL, "hparams is NULL");
  if (n < 0) return fail(OPT8_E_SIZE, "n must be >= 0 (got %d)", n);
  if (n > 0 && !tensors) return fail(OPT8_E_NULL, "tensor list is NULL");
  if (noalloc && n > kNoAllocMaxTensors)
    return fail(OPT8_E_SIZE, "the no-allocation entry point takes at most %d tensors (got %d)",
                kNoAllocMaxTensors, n);
  const bool two_state = algo == kAdamW;
  int rc = validate_hparams(*hp, algo);
  if (rc != OPT8_OK) return rc;
  if (n == 0) return OPT8_OK;
  ValidatedList* vl = nullptr;
  rc = validate_tensors_cached(tensors, n, two_state, vl);
  if (rc != OPT8_OK) return rc;

  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0;
  rc = current_device(dev);
  if (rc != OPT8_OK) return rc;
  DeviceState& ds = g_dev[dev];
  if (!ds.init) return fail(OPT8_E_NOT_INIT, "opt8_init_codebooks has not run on device %d", dev);
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // a graph replay would repeat the launches but not the descriptor upload or the cache
  // bookkeeping, and a later call may rewrite the slot the graph's kernels read
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  const hipError_t ce = hipStreamIsCapturing(stream, &capture);
  if (ce != hipSuccess) return hip_fail(ce, "hipStreamIsCapturing");
  if (capture != hipStreamCaptureStatusNone)
    return fail(OPT8_E_CAPTURE, "hip_stream is being captured into a graph; the step cannot be captured");

  const Plan& plan = vl->plan;
  Slot* slot = nullptr;
  DevTensor* dev_list = nullptr;
  if (noalloc) {
    // ordered on the stream after the work queued before it; calls on other
    // streams that are not ordered with this one race on the array
    const hipError_t e = hipMemcpyAsync(ds.scratch, plan.list.data(), plan.list.size() * sizeof(DevTensor),
                                        hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(descriptors to scratch)");
    dev_list = ds.scratch;
  } else {
    // the slot this list was uploaded to, if nothing has rewritten it since
    if (vl->slot_dev == dev && vl->slot_index >= 0 && vl->slot_index < static_cast<int>(ds.slots.size())) {
      Slot& s = ds.slots[vl->slot_index];
      if (s.used && s.gen == vl->slot_gen) slot = &s;
    }
    if (slot) {
      rc = reuse_slot(ds, *slot, stream);
    } else {
      rc = acquire_slot(ds, plan, stream, slot);
      if (rc == OPT8_OK) {
        vl->slot_dev = dev;
        vl->slot_index = static_cast<int>(slot - ds.slots.data());
        vl->slot_gen = slot->gen;
      }
    }
    if (rc != OPT8_OK) return rc;
    dev_list = slot->dev;
  }
  const StepScalars sc = make_scalars(*hp, algo, ds.pow);
  static const char* const kKindName[kKinds] = {"8-bit full blocks", "bf16 state", "fp32 state",
                                                "8-bit last partial blocks", "8-bit short last blocks"};
  std::string queued;
  for (int kind = 0; kind < kKinds; ++kind) {
    if (!plan.count[kind]) continue;
    const int resident = ds.num_cu * ds.occ[sc.state_round != 0][algo][kind];
    // the block map follows the descriptors in a cached slot; the fixed array of the
    // entry point without allocation holds descriptors only, and its kernels search
    const uint32_t* map = nullptr;
    if (slot && kind == static_cast<int>(Kind::k8bit))
      map = reinterpret_cast<const uint32_t*>(dev_list + plan.list.size());
    const hipError_t e = launch_step(static_cast<Kind>(kind), algo, dev_list + plan.first[kind],
                                     plan.count[kind], plan.blocks[kind], sc, stream, ds.num_cu, resident, map);
    if (e != hipSuccess) {
      // launches queued before this one still read the slot: keep its event
      // and stream current so a later call that reuses or rewrites it waits
      if (slot) {
        (void)hipEventRecord(slot->done, stream);
        slot->last_stream = stream;
      }
      return fail(OPT8_E_HIP, "kernel launch (%s) failed: %s; already queued: %s", kKindName[kind],
                  hipGetErrorString(e), queued.empty() ? "nothing" : queued.c_str());
    }
    if (!queued.empty()) queued += ", ";
    queued += kKindName[kind];
  }
  if (!slot) return OPT8_OK;
  const hipError_t e = hipEventRecord(slot->done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  slot->last_stream = stream;
  return OPT8_OK;
}

}  // namespace
}  // namespace opt8

extern "C" int opt8_adamw_step(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                               void* hip_stream) {
  return guarded([&]() -> int { return run_step(kAdamW, tensors, n, hp, hip_stream); });
}

extern "C" int opt8_adamw_step_noalloc(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                                       void* hip_stream) {
  return guarded([&]() -> int { return run_step(kAdamW, tensors, n, hp, hip_stream, true); });
}

extern "C" int opt8_lion_step(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                              void* hip_stream) {
  return guarded([&]() -> int { return run_step(kLion, tensors, n, hp, hip_stream); });
}

extern "C" int opt8_momentum_step(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                                  void* hip_stream) {
  return guarded([&]() -> int { return run_step(kMomentum, tensors, n, hp, hip_stream); });
}
