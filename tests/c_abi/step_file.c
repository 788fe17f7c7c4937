/* One optimizer step through the C ABI alone (include/opt8.h, libopt8.so and the
 * HIP runtime; no Python, no torch): test infrastructure for the boundary.
 *
 *   step_file <dir> <n> <mode> <tensor_id> <step> <seed> <lr> <wd> <noalloc>
 *
 * Reads <dir>/in_{param,grad,m,v,absmax_m,absmax_v}.bin (bf16 patterns, state
 * in the mode's type; absmax files only in 8-bit mode), copies them to device
 * memory from hipMalloc, runs opt8_adamw_step (or opt8_adamw_step_noalloc when
 * <noalloc> is 1) on the null stream with betas (0.9, 0.999) and eps 1e-8,
 * and writes <dir>/out_*.bin.  Exit status 0 on success; the failing call and
 * opt8_last_error() on stderr otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "opt8.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/in_%s.bin", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes);
  const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/out_%s.bin", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  const size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

#define HIP_OK(call)                                                                 \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));              \
      return 3;                                                                      \
    }                                                                                \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s dir n mode tensor_id step seed lr wd noalloc\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int64_t n = strtoll(argv[2], NULL, 10);
  const int mode = atoi(argv[3]);
  const uint32_t tid = (uint32_t)strtoul(argv[4], NULL, 10);
  opt8_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.step = strtoll(argv[5], NULL, 10);
  hp.seed = strtoull(argv[6], NULL, 10);
  hp.lr = strtod(argv[7], NULL);
  hp.weight_decay = strtod(argv[8], NULL);
  hp.beta1 = 0.9;
  hp.beta2 = 0.999;
  hp.eps = 1e-8;
  hp.param_round = OPT8_ROUND_STOCHASTIC;
  hp.state_round = OPT8_STATE_ROUND_NEAREST;
  const int noalloc = atoi(argv[9]);
  if (n <= 0 || (mode != OPT8_STATE_8BIT && mode != OPT8_STATE_BF16_SR && mode != OPT8_STATE_FP32)) return 2;

  const size_t sb = mode == OPT8_STATE_8BIT ? 1 : mode == OPT8_STATE_BF16_SR ? 2 : 4;
  const size_t nb = (size_t)((n + OPT8_BLOCK - 1) / OPT8_BLOCK);
  const char* names[6] = {"param", "grad", "m", "v", "absmax_m", "absmax_v"};
  const size_t bytes[6] = {2 * (size_t)n, 2 * (size_t)n, sb * (size_t)n, sb * (size_t)n, 4 * nb, 4 * nb};
  const int count = mode == OPT8_STATE_8BIT ? 6 : 4;
  void* host[6] = {0};
  void* dev[6] = {0};
  for (int i = 0; i < count; ++i) {
    host[i] = read_file(dir, names[i], bytes[i]);
    if (!host[i]) {
      fprintf(stderr, "cannot read %s/in_%s.bin (%zu bytes)\n", dir, names[i], bytes[i]);
      return 2;
    }
    HIP_OK(hipMalloc(&dev[i], bytes[i]));
    HIP_OK(hipMemcpy(dev[i], host[i], bytes[i], hipMemcpyHostToDevice));
  }

  int rc = opt8_init_codebooks(NULL, NULL);
  if (rc != OPT8_OK) {
    fprintf(stderr, "opt8_init_codebooks: %d %s\n", rc, opt8_last_error());
    return 4;
  }
  opt8_tensor t;
  memset(&t, 0, sizeof t);
  t.param = (uint16_t*)dev[0];
  t.grad = (const uint16_t*)dev[1];
  t.m = dev[2];
  t.v = dev[3];
  t.absmax_m = (float*)dev[4];
  t.absmax_v = (float*)dev[5];
  t.numel = n;
  t.index_base = 0;
  t.tensor_id = tid;
  t.mode = mode;
  rc = noalloc ? opt8_adamw_step_noalloc(&t, 1, &hp, NULL) : opt8_adamw_step(&t, 1, &hp, NULL);
  if (rc != OPT8_OK) {
    fprintf(stderr, "step: %d %s\n", rc, opt8_last_error());
    return 4;
  }
  HIP_OK(hipDeviceSynchronize());
  for (int i = 0; i < count; ++i) {
    if (i == 1) continue;   /* the gradient is read only */
    HIP_OK(hipMemcpy(host[i], dev[i], bytes[i], hipMemcpyDeviceToHost));
    if (write_file(dir, names[i], host[i], bytes[i]) != 0) return 2;
  }
  for (int i = 0; i < count; ++i) {
    HIP_OK(hipFree(dev[i]));
    free(host[i]);
  }
  printf("step_file: %lld elements, mode %d, %s, ok\n", (long long)n, mode,
         noalloc ? "opt8_adamw_step_noalloc" : "opt8_adamw_step");
  return 0;
}
