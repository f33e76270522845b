/* A C caller that takes one DAMP decode step on the GPU through the C ABI alone: the HIP runtime
 * for device memory, libdamp.so for everything else, no Python in the process. It reads its
 * inputs from a file, packs the states into a pool (damp_state_quantize), takes one step
 * (damp_decode_step, fp32 inputs, default stream) and writes the readouts and the pool blocks of
 * the batch's slots to a file; tests/test_gpu_c_caller.py compares them with the oracle.
 *
 * Input file (little-endian): int32 {num_slots, num_heads, d, r, B, per_key}; int32 fp16_rows
 * [num_heads][r]; int32 slot_idx [B]; fp32 S [B][num_heads][d][d]; fp32 q, k, v
 * [B][num_heads][d]; fp32 alpha [B][num_heads] or [B][num_heads][d] (per_key); fp32 beta
 * [B][num_heads].
 * Output file: fp32 out [B][num_heads][d]; uint8 blocks [B][num_heads][damp_block_bytes].
 * Exit status 0 on success; otherwise a message on stderr and status 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "damp.h"

static int fail_hip(hipError_t e, const char* what) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int fail_damp(damp_status s, const char* what) {
  fprintf(stderr, "%s: status %d: %s\n", what, (int)s, damp_last_error());
  return 1;
}

static void* read_all(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static void* to_device(const void* host, size_t bytes, hipError_t* e) {
  void* d = NULL;
  *e = hipMalloc(&d, bytes);
  if (*e == hipSuccess) *e = hipMemcpy(d, host, bytes, hipMemcpyHostToDevice);
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hdr[6];
  if (fread(hdr, sizeof hdr, 1, in) != 1) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int32_t num_slots = hdr[0], H = hdr[1], d = hdr[2], r = hdr[3], B = hdr[4], per_key = hdr[5];
  if (num_slots <= 0 || H <= 0 || d <= 0 || r < 0 || B < 0 || B > num_slots) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const size_t nv = (size_t)B * H * d, ns = nv * d, na = per_key ? nv : (size_t)B * H;
  int32_t* rows = read_all(in, sizeof(int32_t) * H * r);
  int32_t* slots = read_all(in, sizeof(int32_t) * B);
  float* S = read_all(in, sizeof(float) * ns);
  float* q = read_all(in, sizeof(float) * nv);
  float* k = read_all(in, sizeof(float) * nv);
  float* v = read_all(in, sizeof(float) * nv);
  float* alpha = read_all(in, sizeof(float) * na);
  float* beta = read_all(in, sizeof(float) * B * H);
  fclose(in);
  if (!rows || !slots || !S || !q || !k || !v || !alpha || !beta) {
    fprintf(stderr, "short input\n");
    return 1;
  }

  damp_layout L = {num_slots, H, d, d, r};
  const size_t pool_bytes = damp_state_bytes(&L), bb = damp_block_bytes(&L);
  if (pool_bytes == 0) return fail_damp(DAMP_ERR_INVALID_ARGUMENT, "damp_state_bytes");
  hipError_t e;
  void* pool = NULL;
  if ((e = hipMalloc(&pool, pool_bytes)) != hipSuccess) return fail_hip(e, "hipMalloc pool");
  damp_state* st = NULL;
  damp_status s = damp_state_alloc(&L, rows, pool, pool_bytes, &st);
  if (s != DAMP_OK) return fail_damp(s, "damp_state_alloc");

  void *d_slots = to_device(slots, sizeof(int32_t) * B, &e);
  if (e != hipSuccess) return fail_hip(e, "slots");
  void *d_S = to_device(S, sizeof(float) * ns, &e);
  if (e != hipSuccess) return fail_hip(e, "S");
  void *d_q = to_device(q, sizeof(float) * nv, &e);
  if (e != hipSuccess) return fail_hip(e, "q");
  void *d_k = to_device(k, sizeof(float) * nv, &e);
  if (e != hipSuccess) return fail_hip(e, "k");
  void *d_v = to_device(v, sizeof(float) * nv, &e);
  if (e != hipSuccess) return fail_hip(e, "v");
  void *d_a = to_device(alpha, sizeof(float) * na, &e);
  if (e != hipSuccess) return fail_hip(e, "alpha");
  void *d_b = to_device(beta, sizeof(float) * B * H, &e);
  if (e != hipSuccess) return fail_hip(e, "beta");
  void* d_out = NULL;
  if ((e = hipMalloc(&d_out, sizeof(float) * nv)) != hipSuccess) return fail_hip(e, "hipMalloc out");

  if ((s = damp_state_quantize(st, d_S, d_slots, B, NULL)) != DAMP_OK) return fail_damp(s, "damp_state_quantize");
  s = damp_decode_step(st, d_slots, B, d_q, d_k, d_v, DAMP_F32, d_a,
                       per_key ? DAMP_DECAY_PER_KEY : DAMP_DECAY_SCALAR, d_b, d_out, NULL);
  if (s != DAMP_OK) return fail_damp(s, "damp_decode_step");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");

  float* out = malloc(sizeof(float) * nv);
  uint8_t* blocks = malloc(bb * H * (size_t)B);
  if (!out || !blocks) return 1;
  if ((e = hipMemcpy(out, d_out, sizeof(float) * nv, hipMemcpyDeviceToHost)) != hipSuccess)
    return fail_hip(e, "readouts");
  for (int32_t b = 0; b < B; ++b) {
    const uint8_t* src = (const uint8_t*)pool + (size_t)slots[b] * H * bb;
    if ((e = hipMemcpy(blocks + (size_t)b * H * bb, src, H * bb, hipMemcpyDeviceToHost)) != hipSuccess)
      return fail_hip(e, "blocks");
  }
  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(out, sizeof(float), nv, o) != nv || fwrite(blocks, 1, bb * H * (size_t)B, o) != bb * H * (size_t)B) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(o);
  damp_state_free(st);
  hipFree(pool);
  hipFree(d_slots);
  hipFree(d_S);
  hipFree(d_q);
  hipFree(d_k);
  hipFree(d_v);
  hipFree(d_a);
  hipFree(d_b);
  hipFree(d_out);
  return 0;
}
