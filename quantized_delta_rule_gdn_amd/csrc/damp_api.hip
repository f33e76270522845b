// damp_api.hip -- host side of libdamp.so: argument validation, the DAMP pool layout, the
// frozen row map, error reporting and kernel dispatch for the entry points declared in
// include/damp.h. Every check that can be done on the host runs before any HIP call, so the
// validation paths work (and are tested) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "damp.h"
#include "launch.h"

struct damp_state {
  damp_layout layout;
  uint8_t* pool;
  size_t block_bytes;
  uint8_t* rowmap_dev;  // [num_heads][d]: storage row -> key row
};

namespace {

thread_local std::string g_last_error;

damp_status fail(damp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

damp_status ok() {
  g_last_error.clear();
  return DAMP_OK;
}

bool debug_mode() {
  static const bool on = [] {
    const char* e = std::getenv("DAMP_DEBUG");
    return e && e[0] && std::strcmp(e, "0") != 0;
  }();
  return on;
}

bool supported_d(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kBlockAlign = 256;

// Validates a layout; returns DAMP_OK or the status to report (message already set).
damp_status check_layout(const damp_layout* L) {
  if (!L) return fail(DAMP_ERR_INVALID_ARGUMENT, "layout is NULL");
  if (L->num_slots <= 0 || L->num_heads <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "num_slots (%d) and num_heads (%d) must be positive",
                L->num_slots, L->num_heads);
  if (L->d_k <= 0 || L->d_v <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "d_k (%d) and d_v (%d) must be positive", L->d_k, L->d_v);
  if (L->num_fp16_rows < 0 || L->num_fp16_rows > L->d_k)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "num_fp16_rows (%d) must be in [0, d_k = %d]",
                L->num_fp16_rows, L->d_k);
  if (L->d_k != L->d_v || !supported_d(L->d_k))
    return fail(DAMP_ERR_UNSUPPORTED, "d_k = %d, d_v = %d: supported sizes are d_k == d_v in "
                "{16, 32, 64, 128}", L->d_k, L->d_v);
  return DAMP_OK;
}

size_t data_bytes(const damp_layout* L) {
  const size_t d = static_cast<size_t>(L->d_k), r = static_cast<size_t>(L->num_fp16_rows);
  return 2 * r * d + (d - r) * d + 4 * (d - r);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Common checks of a step call's vector arguments.
damp_status check_step_args(int32_t B, int32_t H, int32_t d, const int32_t* slot_idx,
                            const void* q, const void* k, const void* v, damp_dtype dt,
                            const float* alpha, damp_decay decay, const float* beta,
                            const float* out) {
  if (B < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "B (%d) must be >= 0", B);
  if (dt != DAMP_F32 && dt != DAMP_BF16)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "qkv_dtype %d is not DAMP_F32 or DAMP_BF16", int(dt));
  if (decay != DAMP_DECAY_SCALAR && decay != DAMP_DECAY_PER_KEY)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "decay %d is not DAMP_DECAY_SCALAR or DAMP_DECAY_PER_KEY",
                int(decay));
  if (B == 0) return DAMP_OK;
  if (!slot_idx || !q || !k || !v || !alpha || !beta || !out)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL device pointer among slot_idx/q/k/v/alpha/beta/out");
  const size_t es = dt == DAMP_BF16 ? 2 : 4;
  if (!aligned(slot_idx, 4) || !aligned(q, es) || !aligned(k, es) || !aligned(v, es) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "misaligned input pointer (need natural alignment)");
  if (!aligned(out, 16)) return fail(DAMP_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  if (static_cast<int64_t>(B) * H > 0x7fffffffLL)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "B * num_heads = %lld exceeds the grid limit",
                static_cast<long long>(B) * H);
  (void)d;
  return DAMP_OK;
}

// DAMP_DEBUG=1: synchronously validate slot indices (range and uniqueness).
damp_status debug_check_slots(const int32_t* slot_idx, int32_t n, int32_t num_slots,
                              hipStream_t stream) {
  if (!debug_mode() || n == 0) return DAMP_OK;
  std::vector<int32_t> h(static_cast<size_t>(n));
  hipError_t e = hipMemcpyAsync(h.data(), slot_idx, sizeof(int32_t) * h.size(),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(DAMP_ERR_HIP, "reading slot_idx for DAMP_DEBUG: %s", hipGetErrorString(e));
  std::vector<unsigned char> seen(static_cast<size_t>(num_slots), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = h[static_cast<size_t>(i)];
    if (s < 0 || s >= num_slots)
      return fail(DAMP_ERR_SLOT_INDEX, "slot_idx[%d] = %d outside [0, %d)", i, s, num_slots);
    if (seen[static_cast<size_t>(s)])
      return fail(DAMP_ERR_SLOT_INDEX, "slot_idx[%d] = %d repeats an earlier index", i, s);
    seen[static_cast<size_t>(s)] = 1;
  }
  return DAMP_OK;
}

damp_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DAMP_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

damp::StateRef damp_ref(const damp_state* s) {
  const damp_layout& L = s->layout;
  const int64_t d = L.d_k, r = L.num_fp16_rows;
  damp::StateRef ref{};
  ref.hbase = s->pool;
  ref.cbase = s->pool + 2 * r * d;
  ref.sbase = s->pool + 2 * r * d + (d - r) * d;
  ref.hstride = ref.cstride = ref.sstride = static_cast<int64_t>(s->block_bytes);
  ref.r = L.num_fp16_rows;
  ref.rowmap = s->rowmap_dev;
  ref.contiguous = 1;
  return ref;
}

damp::StateRef int8_ref(int8_t* codes, float* scales, int32_t d) {
  damp::StateRef ref{};
  ref.hbase = nullptr;
  ref.cbase = reinterpret_cast<uint8_t*>(codes);
  ref.sbase = reinterpret_cast<uint8_t*>(scales);
  ref.hstride = 0;
  ref.cstride = static_cast<int64_t>(d) * d;
  ref.sstride = static_cast<int64_t>(d) * 4;
  ref.r = 0;
  ref.rowmap = nullptr;
  ref.contiguous = 0;
  return ref;
}

damp_status run_step(int fmt, const damp::StateRef& ref, int32_t d, int32_t H, int32_t num_slots,
                     const int32_t* slot_idx, int32_t B, const void* q, const void* k,
                     const void* v, damp_dtype dt, const float* alpha, damp_decay decay,
                     const float* beta, float* out, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  damp_status st = debug_check_slots(slot_idx, B, num_slots, s);
  if (st != DAMP_OK) return st;
  damp::StepArgs a{};
  a.st = ref;
  a.slot_idx = slot_idx;
  a.B = B;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  return launched(damp::launch_step(fmt, d, decay == DAMP_DECAY_PER_KEY, dt == DAMP_BF16, a, s),
                  "decode step");
}

}  // namespace

extern "C" {

int32_t damp_abi_version(void) { return (1 << 16) | 0; }

const char* damp_last_error(void) { return g_last_error.c_str(); }

size_t damp_block_data_bytes(const damp_layout* L) {
  if (check_layout(L) != DAMP_OK) return 0;
  return data_bytes(L);
}

size_t damp_block_bytes(const damp_layout* L) {
  if (check_layout(L) != DAMP_OK) return 0;
  return round_up(data_bytes(L), kBlockAlign);
}

size_t damp_state_bytes(const damp_layout* L) {
  if (check_layout(L) != DAMP_OK) return 0;
  const size_t blk = round_up(data_bytes(L), kBlockAlign);
  const size_t units = static_cast<size_t>(L->num_slots) * static_cast<size_t>(L->num_heads);
  if (units != 0 && blk > SIZE_MAX / units) return 0;
  return units * blk;
}

damp_status damp_state_alloc(const damp_layout* L, const int32_t* fp16_rows, void* pool,
                             size_t pool_bytes, damp_state** out) {
  if (!out) return fail(DAMP_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  damp_status st = check_layout(L);
  if (st != DAMP_OK) return st;
  const int32_t H = L->num_heads, d = L->d_k, r = L->num_fp16_rows;
  if (r > 0 && !fp16_rows) return fail(DAMP_ERR_INVALID_ARGUMENT, "fp16_rows is NULL with r = %d", r);
  if (!pool) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (!aligned(pool, kBlockAlign)) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool must be 256-byte aligned");
  const size_t need = damp_state_bytes(L);
  if (need == 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool size overflows size_t");
  if (pool_bytes < need)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "pool_bytes %zu < %zu needed", pool_bytes, need);
  // storage order per head: the r FP16 rows ascending, then the remaining rows ascending
  std::vector<uint8_t> map(static_cast<size_t>(H) * d);
  std::vector<unsigned char> isfp16(static_cast<size_t>(d));
  for (int32_t h = 0; h < H; ++h) {
    std::fill(isfp16.begin(), isfp16.end(), 0);
    for (int32_t j = 0; j < r; ++j) {
      const int32_t row = fp16_rows[static_cast<size_t>(h) * r + j];
      if (row < 0 || row >= d)
        return fail(DAMP_ERR_INVALID_ARGUMENT, "fp16_rows[%d][%d] = %d outside [0, %d)", h, j, row, d);
      if (j > 0 && row <= fp16_rows[static_cast<size_t>(h) * r + j - 1])
        return fail(DAMP_ERR_INVALID_ARGUMENT, "fp16_rows[%d] must be strictly ascending", h);
      isfp16[static_cast<size_t>(row)] = 1;
      map[static_cast<size_t>(h) * d + j] = static_cast<uint8_t>(row);
    }
    int32_t p = r;
    for (int32_t i = 0; i < d; ++i)
      if (!isfp16[static_cast<size_t>(i)]) map[static_cast<size_t>(h) * d + p++] = static_cast<uint8_t>(i);
  }
  damp_state* s = new (std::nothrow) damp_state{};
  if (!s) return fail(DAMP_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
  s->layout = *L;
  s->pool = static_cast<uint8_t*>(pool);
  s->block_bytes = round_up(data_bytes(L), kBlockAlign);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&s->rowmap_dev), map.size());
  if (e != hipSuccess) {
    delete s;
    (void)hipGetLastError();
    return fail(e == hipErrorOutOfMemory ? DAMP_ERR_OUT_OF_MEMORY : DAMP_ERR_HIP,
                "hipMalloc of the row map: %s", hipGetErrorString(e));
  }
  e = hipMemcpy(s->rowmap_dev, map.data(), map.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(s->rowmap_dev);
    delete s;
    return fail(DAMP_ERR_HIP, "copying the row map: %s", hipGetErrorString(e));
  }
  *out = s;
  return ok();
}

damp_status damp_state_free(damp_state* s) {
  if (!s) return ok();
  const hipError_t e = s->rowmap_dev ? hipFree(s->rowmap_dev) : hipSuccess;
  delete s;
  if (e != hipSuccess) return fail(DAMP_ERR_HIP, "hipFree of the row map: %s", hipGetErrorString(e));
  return ok();
}

damp_status damp_state_layout(const damp_state* s, damp_layout* L) {
  if (!s || !L) return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL state or layout");
  *L = s->layout;
  return ok();
}

damp_status damp_state_quantize(damp_state* s, const float* S, const int32_t* slot_idx, int32_t n,
                                void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  if (n < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "n (%d) must be >= 0", n);
  if (n == 0) return ok();
  if (!S || !slot_idx) return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL S or slot_idx");
  if (!aligned(S, 16) || !aligned(slot_idx, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "S must be 16-byte and slot_idx 4-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  damp_status r = debug_check_slots(slot_idx, n, s->layout.num_slots, st);
  if (r != DAMP_OK) return r;
  damp::PackArgs a{};
  a.st = damp_ref(s);
  a.slot_idx = slot_idx;
  a.n = n;
  a.H = s->layout.num_heads;
  a.S = const_cast<float*>(S);
  return launched(damp::launch_quantize(s->layout.d_k, a, st), "quantize");
}

damp_status damp_state_dequantize(const damp_state* s, float* S, const int32_t* slot_idx, int32_t n,
                                  void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  if (n < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "n (%d) must be >= 0", n);
  if (n == 0) return ok();
  if (!S || !slot_idx) return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL S or slot_idx");
  if (!aligned(S, 16) || !aligned(slot_idx, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "S must be 16-byte and slot_idx 4-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  damp_status r = debug_check_slots(slot_idx, n, s->layout.num_slots, st);
  if (r != DAMP_OK) return r;
  damp::PackArgs a{};
  a.st = damp_ref(s);
  a.slot_idx = slot_idx;
  a.n = n;
  a.H = s->layout.num_heads;
  a.S = S;
  return launched(damp::launch_dequantize(s->layout.d_k, a, st), "dequantize");
}

damp_status damp_decode_step(damp_state* s, const int32_t* slot_idx, int32_t B, const void* q,
                             const void* k, const void* v, damp_dtype dt, const float* alpha,
                             damp_decay decay, const float* beta, float* out, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, alpha, decay, beta, out, stream);
}

damp_status fp32_decode_step(float* pool, int32_t num_slots, int32_t H, int32_t d_k, int32_t d_v,
                             const int32_t* slot_idx, int32_t B, const void* q, const void* k,
                             const void* v, damp_dtype dt, const float* alpha, damp_decay decay,
                             const float* beta, float* out, void* stream) {
  if (num_slots <= 0 || H <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "num_slots (%d) and num_heads (%d) must be positive",
                num_slots, H);
  if (d_k != d_v || !supported_d(d_k))
    return fail(DAMP_ERR_UNSUPPORTED, "d_k = %d, d_v = %d: supported sizes are d_k == d_v in "
                "{16, 32, 64, 128}", d_k, d_v);
  damp_status st = check_step_args(B, H, d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  if (!pool) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (!aligned(pool, 16)) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool must be 16-byte aligned");
  damp::StateRef ref{};
  ref.hbase = reinterpret_cast<uint8_t*>(pool);
  ref.hstride = static_cast<int64_t>(d_k) * d_k * 4;
  return run_step(damp::FMT_F32, ref, d_k, H, num_slots, slot_idx, B, q, k, v, dt, alpha, decay,
                  beta, out, stream);
}

damp_status uniform_int8_decode_step(int8_t* codes, float* scales, int32_t num_slots, int32_t H,
                                     int32_t d_k, int32_t d_v, const int32_t* slot_idx, int32_t B,
                                     const void* q, const void* k, const void* v, damp_dtype dt,
                                     const float* alpha, damp_decay decay, const float* beta,
                                     float* out, void* stream) {
  if (num_slots <= 0 || H <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "num_slots (%d) and num_heads (%d) must be positive",
                num_slots, H);
  if (d_k != d_v || !supported_d(d_k))
    return fail(DAMP_ERR_UNSUPPORTED, "d_k = %d, d_v = %d: supported sizes are d_k == d_v in "
                "{16, 32, 64, 128}", d_k, d_v);
  damp_status st = check_step_args(B, H, d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  if (!codes || !scales) return fail(DAMP_ERR_INVALID_ARGUMENT, "codes or scales is NULL");
  if (!aligned(codes, 16) || !aligned(scales, 16))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "codes and scales must be 16-byte aligned");
  return run_step(damp::FMT_Q, int8_ref(codes, scales, d_k), d_k, H, num_slots, slot_idx, B, q, k,
                  v, dt, alpha, decay, beta, out, stream);
}

damp_status uniform_int8_quantize(int8_t* codes, float* scales, int32_t num_slots, int32_t H,
                                  int32_t d_k, int32_t d_v, const float* S, const int32_t* slot_idx,
                                  int32_t n, void* stream) {
  if (num_slots <= 0 || H <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "num_slots (%d) and num_heads (%d) must be positive",
                num_slots, H);
  if (d_k != d_v || !supported_d(d_k))
    return fail(DAMP_ERR_UNSUPPORTED, "d_k = %d, d_v = %d: supported sizes are d_k == d_v in "
                "{16, 32, 64, 128}", d_k, d_v);
  if (n < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "n (%d) must be >= 0", n);
  if (n == 0) return ok();
  if (!codes || !scales || !S || !slot_idx)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL codes, scales, S or slot_idx");
  if (!aligned(codes, 16) || !aligned(scales, 16) || !aligned(S, 16) || !aligned(slot_idx, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  damp_status r = debug_check_slots(slot_idx, n, num_slots, st);
  if (r != DAMP_OK) return r;
  damp::PackArgs a{};
  a.st = int8_ref(codes, scales, d_k);
  a.slot_idx = slot_idx;
  a.n = n;
  a.H = H;
  a.S = const_cast<float*>(S);
  return launched(damp::launch_quantize(d_k, a, st), "quantize");
}

}  // extern "C"
