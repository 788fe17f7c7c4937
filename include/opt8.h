/*
 * opt8.h -- C ABI of the fused block-wise 8-bit AdamW step with a
 * stochastically rounded bf16 parameter write, for AMD Instinct MI355X
 * (gfx950).  Library: libopt8.so (precision_optimizer_step_amd/).
 *
 * What the step computes, per element i of a tensor (all arithmetic fp32,
 * one rounding per operation, no fused multiply-add, IEEE sqrt and divide):
 *
 *   g = bf16 grad, p = bf16 param (both widened exactly)
 *   m1, v1 = moments read from the state (8-bit: codebook[code] * block absmax)
 *   m2 = beta1*m1 + (1-beta1)*g
 *   v2 = beta2*v1 + (1-beta2)*(g*g)
 *   den = sqrt(v2) * rbc2 + eps          rbc2 = 1/sqrt(1 - beta2^t)
 *   p'  = (p - lrwd*p) - step_size*(m2/den)
 *                                        step_size = lr/(1 - beta1^t), lrwd = lr*wd
 *   param <- bf16(p') by stochastic rounding (or nearest-even on request)
 *   state <- m2, v2 (8-bit: block absmax + nearest codebook entry; bf16:
 *            stochastic rounding; fp32: stored as is)
 *
 * Passages defining it (page title, part of the page):
 *  - "8-bit Optimizers via Block-wise Quantization", method bullets: 2048-
 *    element blocks each normalised by its own absolute maximum; non-linear
 *    8-bit codes found by binary search and decoded by a lookup table times the
 *    block maximum; dequantise, update in 32-bit and requantise in registers;
 *    the innovations list: dynamic tree quantisation extended to unipolar data.
 *  - "Stochastic rounding support for 8-bit optimizers", feature request: the
 *    update is computed in full precision and the bf16 parameter is rounded up
 *    or down with a probability set by the rounding error; the scoping
 *    comment: opt-in, non-paged AdamW with 8-bit state, no fp32 master copy, an
 *    fp32-state fallback for small tensors, a weight-decay baseline to pick,
 *    and work on the caller's stream.  The "Your contribution" paragraph: the
 *    gradient transform and parameter update form one step outside Python.
 *  - "[Feat]: Stochastic rounding of AdamW momentums": Adam arithmetic in
 *    float32, the p + value*exp_avg/denom update with value = -step_size
 *    done in fp32 before rounding, a state-precision flag, bf16 momenta cast
 *    back with stochastic rounding each step.
 *  - "Stochastic Rounding for LLM Training: Theory and Practice", TL;DR:
 *    BF16-AdamW-SR and randomness shared across data-parallel replicas.
 *
 * Random bits: Philox4x32-10 (Salmon et al., SC'11) with
 *   key = (lo32(seed), hi32(seed)),
 *   counter = (lo32(j/8), hi32(j/8) | stream<<30, lo32(step), tensor_id),
 *   j = index_base + i, element j taking 16-bit half (j%8)&1 (low first) of
 *   output word (j%8)>>1; stream 0 = param, 1 = m, 2 = v.  The bits never
 *   depend on a rank, a launch shape or a device, so replicas agree.
 *
 * Codebooks: the dynamic tree code read as a decimal exponent by leading
 * zeros plus a linear fraction taking the upper end of its step; signed
 * table (first moment) and unsigned table (second moment), 256 fp32 entries
 * each, ascending, code == index; zero code 127 (signed) and 0 (unsigned).
 * A value is rounded to the entry whose midpoint interval holds it, ties to
 * the lower code.  A block whose new absmax is below 2^-126 stores the zero
 * code everywhere (the absmax itself is stored as computed).
 *
 * Stochastic state rounding (state_round = 1, 8-bit state; the pages suggest
 * stochastic rounding of the momenta, "[Feat]: Stochastic rounding of AdamW
 * momentums", comment thread, and this carries it to the 8-bit codes): with
 * n the normalised value, k = (number of entries <= n) - 1 clamped to
 * [0, 254], W[k] = fp32(65536 / (C[k+1] - C[k])) (double arithmetic) and
 * f = fp32(fp32(n - C[k]) * W[k]), the code is k + 1 if f > r and k
 * otherwise, r being the element's 16 random bits on stream 1 (first moment)
 * or 2 (second moment); a NaN n stores 255.
 */
#ifndef OPT8_H_
#define OPT8_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OPT8_BLOCK 2048                /* elements per quantisation block        */
#define OPT8_FP32_STATE_THRESHOLD 4096 /* default policy: fp32 state below this  */
#define OPT8_NUM_CODES 256

typedef enum {
  OPT8_OK = 0,
  OPT8_E_NULL = -1,      /* a required pointer is NULL                               */
  OPT8_E_ALIGN = -2,     /* param/grad/m/v not 16-byte aligned, absmax not 4-byte    */
  OPT8_E_SIZE = -3,      /* n < 0 (> 4096 without allocation), numel <= 0 or > 2^42, */
                         /*   bad index_base                                         */
  OPT8_E_MODE = -4,      /* unknown state mode, rounding mode or state rounding      */
  OPT8_E_HPARAM = -5,    /* lr/betas/eps/weight_decay/step outside their ranges      */
  OPT8_E_ALIAS = -6,     /* two buffers of the list overlap                          */
  OPT8_E_DUPID = -7,     /* tensor_id repeated in one list                           */
  OPT8_E_NOT_INIT = -8,  /* opt8_init_codebooks not called on the current device     */
  OPT8_E_HIP = -9,       /* a HIP runtime call or a kernel launch failed             */
  OPT8_E_CAPTURE = -10,  /* hip_stream is being captured into a graph (see below)    */
  OPT8_E_NOMEM = -11     /* host memory for the library's copies of a list ran out   */
} opt8_status;

typedef enum {
  OPT8_STATE_8BIT = 0,    /* u8 codes + fp32 absmax per 2048-element block           */
  OPT8_STATE_BF16_SR = 1, /* bf16 moments written with stochastic rounding           */
  OPT8_STATE_FP32 = 2     /* fp32 moments                                            */
} opt8_state_mode;

typedef enum {
  OPT8_ROUND_STOCHASTIC = 0, /* parameter written with stochastic rounding          */
  OPT8_ROUND_NEAREST = 1     /* parameter written round-to-nearest-even             */
} opt8_round_mode;

typedef enum {
  OPT8_STATE_ROUND_NEAREST = 0,    /* 8-bit state: nearest codebook entry (default) */
  OPT8_STATE_ROUND_STOCHASTIC = 1  /* 8-bit state: one of the two entries around    */
                                   /*   the value, the upper one with probability   */
                                   /*   (n - C[k]) / (C[k+1] - C[k])                */
} opt8_state_round;

/* One tensor of the list.  All pointers are DEVICE pointers on the current
 * HIP device, owned by the caller, and must stay valid until the work queued
 * on the stream has finished.  Tensors are flat (row-major) arrays.          */
typedef struct opt8_tensor {
  uint16_t* param;        /* bf16[numel], in/out, 16-byte aligned                      */
  const uint16_t* grad;   /* bf16[numel], read only, 16-byte aligned                   */
  void* m;                /* first moment [numel]: u8 (8-bit), bf16 or f32 by mode,    */
  void* v;                /*   second moment likewise; in/out, 16-byte aligned         */
  float* absmax_m;        /* f32[ceil(numel/2048)], in/out, 8-bit mode only (else     */
  float* absmax_v;        /*   ignored and may be NULL); 4-byte aligned               */
  int64_t numel;          /* > 0 and <= 2^42                                           */
  int64_t index_base;     /* global index of element 0 in the unsharded tensor (RNG   */
                          /*   counter); >= 0, <= 2^60 and a multiple of 2048 (so     */
                          /*   hi32(j/8) < 2^30 stays clear of the stream bits); 0 if */
                          /*   unsharded                                              */
  uint32_t tensor_id;     /* RNG stream id; unique in the list, stable over steps     */
  int32_t mode;           /* opt8_state_mode                                           */
} opt8_tensor;

typedef struct opt8_hparams {
  double lr;              /* >= 0, finite                                              */
  double beta1;           /* [0, 1)                                                    */
  double beta2;           /* [0, 1)                                                    */
  double eps;             /* > 0, finite                                               */
  double weight_decay;    /* >= 0, finite; decoupled (AdamW)                           */
  int64_t step;           /* 1-based step count t of this update, >= 1                 */
  uint64_t seed;          /* Philox key                                                */
  int32_t param_round;    /* opt8_round_mode                                           */
  int32_t state_round;    /* opt8_state_round (8-bit state only; 0 keeps the nearest   */
                          /*   entry)                                                  */
} opt8_hparams;

/* Build the two 256-entry codebooks (and their 255 midpoints) on the host and
 * upload them to the CURRENT device; idempotent, once per device.  If
 * signed_out / unsigned_out are non-NULL the fp32 tables are also copied to
 * those host arrays, before the upload, so a host without a GPU still gets
 * them (the call then returns OPT8_E_HIP).  Returns OPT8_OK or OPT8_E_HIP.
 * Defined by: "8-bit Optimizers via Block-wise Quantization", method bullets
 * (non-linear 8-bit codes searched by binary search, decoded by lookup table)
 * and innovations list (dynamic tree quantisation, extended to unipolar data
 * for the unsigned table).  Outputs: signed_out[k], unsigned_out[k] = entry
 * of code k, ascending; host arrays owned by the caller, written in full.   */
int opt8_init_codebooks(float* signed_out, float* unsigned_out);

/* Default state mode for a tensor of numel elements: OPT8_STATE_FP32 below
 * 4096 elements, OPT8_STATE_8BIT otherwise (the small-tensor fallback).
 * Defined by: "Stochastic rounding support for 8-bit optimizers", scoping
 * comment (small tensors keep 32-bit state); the 4096 threshold is this
 * library's choice.  Pure function; never fails.                            */
int32_t opt8_default_mode(int64_t numel);

/* Defined by: "8-bit Optimizers via Block-wise Quantization", method bullets
 * (block-wise absmax, dequantise -> 32-bit update -> requantise in registers);
 * "Stochastic rounding support for 8-bit optimizers", feature request
 * (stochastic rounding of the bf16 parameter) and scoping comment (opt-in,
 * non-paged, no fp32 master copy, fp32 state for small tensors, the caller's
 * stream); "[Feat]: Stochastic rounding of AdamW momentums", comment thread
 * (fp32 Adam arithmetic, the p + value*exp_avg/denom update, bf16 momenta
 * written with stochastic rounding).
 *
 * One AdamW step over a list of n tensors, queued on hip_stream (a
 * hipStream_t; NULL = the null stream) and asynchronous to the host.
 * Every descriptor and hyperparameter is validated first; on a validation
 * error (every status but OPT8_E_HIP and OPT8_E_NOMEM) nothing is queued and
 * nothing is modified; OPT8_E_NOMEM (the host could not allocate the
 * library's copy of the list) is returned before any launch, with at most a
 * descriptor upload into an unused cache slot queued.  A step is up to five kernel launches, one per kind of tensor in
 * the list (8-bit full blocks, bf16 state, fp32 state, 8-bit last partial
 * blocks longer than 64 elements, and those of at most 64, eight to a
 * wave); if a launch fails (OPT8_E_HIP) the kinds launched before it have
 * been queued and will step their tensors, and the message names them.
 * n == 0 is a no-op.  Tensors of
 * different modes may be mixed.  Concurrent calls on different streams must
 * use disjoint buffers.  Device faults surface at the caller's next
 * synchronisation.  A stream that is being captured into a HIP graph is
 * refused with OPT8_E_CAPTURE before anything is queued: a step may upload
 * its descriptor list into a cache slot that later calls reuse, which a
 * graph replay would not follow.
 * Caching: the library keeps, per calling thread, the last 1024 lists that
 * passed validation (with their launch plans), and on each device up to 1024
 * descriptor slots (device copies of a list's descriptors and block map).  A
 * list passed again byte for byte -- a training loop passes one per parameter
 * group, every step -- is neither validated nor uploaded again.  Beyond 1024
 * lists, or beyond a byte budget per cache (256 MiB; the environment variable
 * OPT8_CACHE_MB, read at the first step, replaces it), the least recently used
 * lists are dropped; a call that rewrites or frees a slot first waits on the
 * host for the launches that last read it.  Lion and momentum share the same
 * caches.  Returns OPT8_OK or a negative opt8_status. */
int opt8_adamw_step(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                    void* hip_stream);

/* The step of opt8_adamw_step for callers that cannot allocate memory
 * (code paths that must not call hipMalloc, tight serving or training loops,
 * harnesses that forbid allocation).  Same arguments, validation, kernels,
 * results and status codes as opt8_adamw_step.  The difference is where the
 * per-kernel descriptor lists live: opt8_adamw_step keeps them in device
 * buffers it allocates (and grows) on first use; this entry point writes
 * them into a fixed array in the library's device image ("scratch", 8192
 * descriptors of 80 bytes = 640 KiB on each device the library runs on,
 * held until the process ends) with one host-to-device copy on hip_stream,
 * and calls no hipMalloc, hipFree or other allocating routine.
 * Limit: n <= 4096 tensors; a longer list returns OPT8_E_SIZE with nothing
 * queued.  Every call on a device shares that device's array, which keeps
 * the last call's descriptors: calls on one stream are ordered by it, but
 * calls that overlap on one device (different streams with no ordering
 * between them) race on the array and must be ordered by the caller.  A
 * stream under graph capture is refused with OPT8_E_CAPTURE, as for
 * opt8_adamw_step.                                                          */
int opt8_adamw_step_noalloc(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                            void* hip_stream);

/* One-state update rules on the same state machinery (codebook, block absmax,
 * state modes, rounding, Random bits; the SIGNED codebook holds the state in
 * 8-bit mode).  The pages name both without defining them ("8-bit Optimizers
 * via Block-wise Quantization", introduction: the state of Adam and of
 * Momentum; "Stochastic rounding support for 8-bit optimizers", motivation:
 * more memory saved with 8-bit Lion); the readings below follow the papers
 * that introduced them, with weight decay decoupled as in the AdamW step.
 * v and absmax_v are ignored (may be NULL) and eps is neither validated nor
 * used; step is still validated (>= 1) and keys the random bits; there is
 * no bias correction.
 * Validation, error behaviour, streams and ownership as for opt8_adamw_step.
 *
 * Lion (Chen et al., "Symbolic Discovery of Optimization Algorithms"):
 *   c  = beta1*m1 + (1-beta1)*g          (the direction uses the old moment)
 *   m2 = beta2*m1 + (1-beta2)*g
 *   p' = (p - lrwd*p) - lr*sign(c)       sign(+-0) = 0, sign(NaN) = NaN     */
int opt8_lion_step(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                   void* hip_stream);

/* SGD with momentum (heavy ball, dampening 0; beta1 is the momentum, beta2
 * is validated but unused):
 *   m2 = beta1*m1 + g
 *   p' = (p - lrwd*p) - lr*m2                                                */
int opt8_momentum_step(const opt8_tensor* tensors, int32_t n, const opt8_hparams* hp,
                       void* hip_stream);

/* Message of the last failure on the calling thread ("" if none).  The
 * string is owned by the library and valid until the thread's next call.
 * (Not from the pages: the error channel of this C ABI.)                    */
const char* opt8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OPT8_H_ */
