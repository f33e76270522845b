// damp_api.hip -- host side of libdamp.so: argument validation, the DAMP pool layout, the
// frozen row map, error reporting and kernel dispatch for the entry points declared in
// include/damp.h. Every check that can be done on the host runs before any HIP call, so the
// validation paths work (and are tested) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "damp.h"
#include "launch.h"

struct damp_state {
  damp_layout layout;    // num_fp16_rows = -1 for a per-head layout
  uint8_t* pool;
  size_t block_bytes;    // uniform layout: the block stride
  uint8_t* rowmap_dev;   // [num_heads][d]: storage row -> key row; per-head layout: followed by
                         // the int2 table {block offset in the slot, r} per head
  bool per_head;
  std::vector<int32_t> head_r;    // per head: r
  std::vector<int64_t> head_off;  // per head: byte offset of its block inside a slot
  size_t slot_bytes;
  int32_t r_or, r_max;            // bitwise OR and maximum of head_r
};

struct stq_state {
  int32_t num_slots, num_heads, d;
  uint8_t* pool;
  size_t slot_bytes;
  std::vector<int64_t> head_off;
  uint8_t* table_dev;   // rowmap [H][d] (uint8) | w2 [H][d] (fp32) | heads [H] (int4)
  int32_t max_pivots;   // the largest number of pivot rows in one head
};

// The library-held order buffer of damp_decode_step_sorted: one copy of this file-scope device
// array on every GPU the library runs on, held until the process ends. In host code its name
// stands for a host-side symbol, not a device address: the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that address is ever handed
// to a kernel.
static __device__ __align__(256) int32_t scratch[DAMP_SORTED_MAX_B];

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

// Data bytes of one DAMP block: r FP16 rows, d - r INT8 rows, d - r fp32 scales.
size_t data_bytes_r(int32_t d_, int32_t r_) {
  const size_t d = static_cast<size_t>(d_), r = static_cast<size_t>(r_);
  return 2 * r * d + (d - r) * d + 4 * (d - r);
}

size_t data_bytes(const damp_layout* L) { return data_bytes_r(L->d_k, L->num_fp16_rows); }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout checks of the per-head calls (num_fp16_rows not used); *L2 = the layout with
// num_fp16_rows = -1.
damp_status check_layout_per_head(const damp_layout* L, const int32_t* r_per_head, damp_layout* L2) {
  if (!L) return fail(DAMP_ERR_INVALID_ARGUMENT, "layout is NULL");
  damp_layout T = *L;
  T.num_fp16_rows = 0;
  damp_status st = check_layout(&T);
  if (st != DAMP_OK) return st;
  if (!r_per_head) return fail(DAMP_ERR_INVALID_ARGUMENT, "r_per_head is NULL");
  for (int32_t h = 0; h < L->num_heads; ++h)
    if (r_per_head[h] < 0 || r_per_head[h] > L->d_k)
      return fail(DAMP_ERR_INVALID_ARGUMENT, "r_per_head[%d] = %d outside [0, d_k = %d]", h,
                  r_per_head[h], L->d_k);
  T.num_fp16_rows = -1;
  if (L2) *L2 = T;
  return DAMP_OK;
}

// Device copy of the row map ([H][d] bytes), followed for a per-head layout by the int2 table
// {block offset in the slot, r} per head (8-byte aligned).
damp_status upload_table(damp_state* s, const std::vector<uint8_t>& map) {
  std::vector<uint8_t> blob(map);
  if (s->per_head) {
    const size_t H = s->head_r.size();
    blob.resize(round_up(blob.size(), 8) + 8 * H);
    int32_t* tab = reinterpret_cast<int32_t*>(blob.data() + round_up(map.size(), 8));
    for (size_t h = 0; h < H; ++h) {
      tab[2 * h] = static_cast<int32_t>(s->head_off[h]);
      tab[2 * h + 1] = s->head_r[h];
    }
  }
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&s->rowmap_dev), blob.size());
  if (e != hipSuccess) {
    (void)hipGetLastError();
    s->rowmap_dev = nullptr;
    return fail(e == hipErrorOutOfMemory ? DAMP_ERR_OUT_OF_MEMORY : DAMP_ERR_HIP,
                "hipMalloc of the row map: %s", hipGetErrorString(e));
  }
  e = hipMemcpy(s->rowmap_dev, blob.data(), blob.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(s->rowmap_dev);
    s->rowmap_dev = nullptr;
    return fail(DAMP_ERR_HIP, "copying the row map: %s", hipGetErrorString(e));
  }
  return DAMP_OK;
}

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

// DAMP_DEBUG=1: synchronously check that order is a permutation of [0, B).
damp_status debug_check_order(const int32_t* order, int32_t B, hipStream_t stream) {
  if (!debug_mode() || !order || B == 0) return DAMP_OK;
  std::vector<int32_t> h(static_cast<size_t>(B));
  hipError_t e = hipMemcpyAsync(h.data(), order, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(DAMP_ERR_HIP, "reading order for DAMP_DEBUG: %s", hipGetErrorString(e));
  std::vector<unsigned char> seen(static_cast<size_t>(B), 0);
  for (int32_t i = 0; i < B; ++i) {
    const int32_t p = h[static_cast<size_t>(i)];
    if (p < 0 || p >= B || seen[static_cast<size_t>(p)])
      return fail(DAMP_ERR_SLOT_INDEX, "order is not a permutation of [0, %d): order[%d] = %d", B, i, p);
    seen[static_cast<size_t>(p)] = 1;
  }
  return DAMP_OK;
}

damp_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DAMP_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- STEPQuant-style layout (stq_*) ----------------------------------------------------------
bool stq_supported_d(int32_t d) { return d == 64 || d == 128; }

// The block's regions (pivots, 8-, 6-, 4-bit rows, row factors, column scales) each start on a
// 128-byte line; the result is the end of the column scales (before the 256-byte rounding).
size_t stq_block_bytes(int32_t d_, int n16, int n8, int n6, int n4) {
  const size_t d = static_cast<size_t>(d_);
  auto up = [](size_t x) { return (x + 127) / 128 * 128; };
  // the 6- and 4-bit regions begin at the 4-row group of their first storage row
  const size_t r6 = n6 > 0 ? n6 + (n16 + n8) % 4 : 0, r4 = n4 > 0 ? n4 + (n16 + n8 + n6) % 4 : 0;
  const size_t o8 = up(2 * d * n16), o6 = up(o8 + d * n8), o4 = up(o6 + (3 * d / 4) * r6);
  const size_t orf = up(o4 + (d / 2) * r4), ocs = up(orf + 2 * (d - n16));
  return ocs + 2 * d;
}

// Per-head counts of each code width; row_bits must hold 16, 8, 6 or 4.
damp_status stq_counts(int32_t H, int32_t d, const uint8_t* row_bits, std::vector<int>* counts) {
  if (!row_bits) return fail(DAMP_ERR_INVALID_ARGUMENT, "row_bits is NULL");
  counts->assign(static_cast<size_t>(H) * 4, 0);
  for (int32_t h = 0; h < H; ++h)
    for (int32_t i = 0; i < d; ++i) {
      const int b = row_bits[static_cast<size_t>(h) * d + i];
      const int k = b == 16 ? 0 : b == 8 ? 1 : b == 6 ? 2 : b == 4 ? 3 : -1;
      if (k < 0)
        return fail(DAMP_ERR_INVALID_ARGUMENT, "row_bits[%d][%d] = %d is not 16, 8, 6 or 4", h, i, b);
      (*counts)[static_cast<size_t>(h) * 4 + k] += 1;
    }
  return DAMP_OK;
}

damp_status stq_check_dims(int32_t num_slots, int32_t H, int32_t d) {
  if (num_slots <= 0 || H <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "num_slots (%d) and num_heads (%d) must be positive", num_slots, H);
  if (!stq_supported_d(d))
    return fail(DAMP_ERR_UNSUPPORTED, "d = %d: the STEPQuant-style state supports d in {64, 128}", d);
  return DAMP_OK;
}

damp::StqArgs stq_args(const stq_state* s) {
  damp::StqArgs a{};
  const size_t H = static_cast<size_t>(s->num_heads), d = static_cast<size_t>(s->d);
  a.pool = s->pool;
  a.num_slots = s->num_slots;
  a.slot_stride = static_cast<int64_t>(s->slot_bytes);
  a.rowmap = s->table_dev;
  a.w1 = reinterpret_cast<const float*>(s->table_dev + H * d);
  a.heads = reinterpret_cast<const int4*>(s->table_dev + H * d + 4 * H * d);
  a.H = s->num_heads;
  a.step.st.rowmap = s->table_dev;
  a.step.H = s->num_heads;
  a.max_pivots = s->max_pivots;
  return a;
}

damp::StateRef damp_ref(const damp_state* s) {
  const damp_layout& L = s->layout;
  damp::StateRef ref{};
  if (s->per_head) {
    ref.hbase = s->pool;
    ref.rowmap = s->rowmap_dev;
    ref.contiguous = 1;
    ref.heads = reinterpret_cast<const int2*>(s->rowmap_dev + static_cast<size_t>(L.num_heads) * L.d_k);
    ref.slot_stride = static_cast<int64_t>(s->slot_bytes);
    ref.heads_r_or = s->r_or;
    ref.heads_r_max = s->r_max;
    return ref;
  }
  const int64_t d = L.d_k, r = L.num_fp16_rows;
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

size_t window_unit_bytes(int32_t d, int32_t window) {
  return round_up(4 * (4 + static_cast<size_t>(d) + 2 * static_cast<size_t>(window) * d), kBlockAlign);
}

damp_status check_window(const void* win, int32_t window) {
  if (window < 1 || window > damp::window_max())
    return fail(DAMP_ERR_INVALID_ARGUMENT, "window %d outside [1, %d]", window, damp::window_max());
  if (!win) return fail(DAMP_ERR_INVALID_ARGUMENT, "window_buf is NULL");
  if (!aligned(win, kBlockAlign)) return fail(DAMP_ERR_INVALID_ARGUMENT, "window_buf must be 256-byte aligned");
  return DAMP_OK;
}

damp_status run_step(int fmt, const damp::StateRef& ref, int32_t d, int32_t H, int32_t num_slots,
                     const int32_t* slot_idx, int32_t B, const void* q, const void* k,
                     const void* v, damp_dtype dt, const float* alpha, damp_decay decay,
                     const float* beta, float* out, void* stream, int prestep = 0,
                     void* win = nullptr, int32_t window = 0, bool flush_only = false,
                     const int32_t* order = nullptr) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  damp_status st = debug_check_slots(slot_idx, B, num_slots, s);
  if (st != DAMP_OK) return st;
  st = debug_check_order(order, B, s);
  if (st != DAMP_OK) return st;
  damp::StepArgs a{};
  a.order = order;
  a.st = ref;
  a.st.num_slots = num_slots;
  a.slot_idx = slot_idx;
  a.B = B;
  a.H = H;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.prestep = prestep;
  if (win) {
    a.win = static_cast<uint8_t*>(win);
    a.win_stride = static_cast<int64_t>(window_unit_bytes(d, window));
    a.window = window;
    return launched(damp::launch_window(d, decay == DAMP_DECAY_PER_KEY, dt == DAMP_BF16, flush_only, a, s),
                    flush_only ? "window flush" : "window step");
  }
  return launched(damp::launch_step(fmt, d, decay == DAMP_DECAY_PER_KEY, dt == DAMP_BF16, a, s),
                  "decode step");
}

// ---- the library-held order buffer of damp_decode_step_sorted (`scratch`, below) ----------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that runs `stream`, in *out.
damp_status scratch_for(hipStream_t stream, int32_t** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DAMP_ERR_HIP, "finding the stream's device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DAMP_ERR_UNSUPPORTED, "device %d is beyond the %d devices this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return fail(DAMP_ERR_HIP, "looking up the order buffer on device %d: %s", dev,
                                     hipGetErrorString(e));
    if (!ptr) return fail(DAMP_ERR_HIP, "the order buffer has no address on device %d", dev);
    g_scratch_ptr[dev] = static_cast<int32_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return DAMP_OK;
}

}  // namespace

extern "C" {

int32_t damp_abi_version(void) { return (1 << 16) | 3; }

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

size_t damp_state_bytes_per_head(const damp_layout* L, const int32_t* r_per_head) {
  if (check_layout_per_head(L, r_per_head, nullptr) != DAMP_OK) return 0;
  size_t slot = 0;
  for (int32_t h = 0; h < L->num_heads; ++h) slot += round_up(data_bytes_r(L->d_k, r_per_head[h]), kBlockAlign);
  const size_t n = static_cast<size_t>(L->num_slots);
  if (slot != 0 && n > SIZE_MAX / slot) return 0;
  return n * slot;
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
  s->per_head = false;
  s->head_r.assign(static_cast<size_t>(H), r);
  s->head_off.resize(static_cast<size_t>(H));
  for (int32_t h = 0; h < H; ++h) s->head_off[static_cast<size_t>(h)] = static_cast<int64_t>(h) * s->block_bytes;
  s->slot_bytes = static_cast<size_t>(H) * s->block_bytes;
  s->r_or = s->r_max = r;
  st = upload_table(s, map);
  if (st != DAMP_OK) {
    delete s;
    return st;
  }
  *out = s;
  return ok();
}

damp_status damp_state_alloc_per_head(const damp_layout* L, const int32_t* r_per_head,
                                      const int32_t* row_map, void* pool, size_t pool_bytes,
                                      damp_state** out) {
  if (!out) return fail(DAMP_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  damp_layout L2{};
  damp_status st = check_layout_per_head(L, r_per_head, &L2);
  if (st != DAMP_OK) return st;
  const int32_t H = L->num_heads, d = L->d_k;
  if (!row_map) return fail(DAMP_ERR_INVALID_ARGUMENT, "row_map is NULL");
  if (!pool) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (!aligned(pool, kBlockAlign)) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool must be 256-byte aligned");
  const size_t need = damp_state_bytes_per_head(L, r_per_head);
  if (need == 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool size overflows size_t");
  if (pool_bytes < need)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "pool_bytes %zu < %zu needed", pool_bytes, need);
  std::vector<uint8_t> map(static_cast<size_t>(H) * d);
  std::vector<unsigned char> seen(static_cast<size_t>(d));
  for (int32_t h = 0; h < H; ++h) {
    const int32_t r = r_per_head[h];
    const int32_t* row = row_map + static_cast<size_t>(h) * d;
    std::fill(seen.begin(), seen.end(), 0);
    for (int32_t p = 0; p < d; ++p) {
      if (row[p] < 0 || row[p] >= d)
        return fail(DAMP_ERR_INVALID_ARGUMENT, "row_map[%d][%d] = %d outside [0, %d)", h, p, row[p], d);
      if (seen[static_cast<size_t>(row[p])])
        return fail(DAMP_ERR_INVALID_ARGUMENT, "row_map[%d] repeats row %d", h, row[p]);
      seen[static_cast<size_t>(row[p])] = 1;
      if (p > 0 && p != r && row[p] <= row[p - 1])
        return fail(DAMP_ERR_INVALID_ARGUMENT, "row_map[%d]: the FP16 rows and the other rows must each "
                    "be strictly ascending", h);
      map[static_cast<size_t>(h) * d + p] = static_cast<uint8_t>(row[p]);
    }
  }
  damp_state* s = new (std::nothrow) damp_state{};
  if (!s) return fail(DAMP_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
  s->layout = L2;
  s->pool = static_cast<uint8_t*>(pool);
  s->block_bytes = 0;
  s->per_head = true;
  s->head_r.assign(r_per_head, r_per_head + H);
  s->head_off.resize(static_cast<size_t>(H));
  size_t off = 0;
  s->r_or = 0;
  s->r_max = 0;
  for (int32_t h = 0; h < H; ++h) {
    s->head_off[static_cast<size_t>(h)] = static_cast<int64_t>(off);
    off += round_up(data_bytes_r(d, r_per_head[h]), kBlockAlign);
    s->r_or |= r_per_head[h];
    s->r_max = std::max(s->r_max, r_per_head[h]);
  }
  s->slot_bytes = off;
  st = upload_table(s, map);
  if (st != DAMP_OK) {
    delete s;
    return st;
  }
  *out = s;
  return ok();
}

damp_status damp_state_head_info(const damp_state* s, int32_t* r_out, int64_t* offset_out,
                                 int64_t* slot_bytes) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  for (size_t h = 0; h < s->head_r.size(); ++h) {
    if (r_out) r_out[h] = s->head_r[h];
    if (offset_out) offset_out[h] = s->head_off[h];
  }
  if (slot_bytes) *slot_bytes = static_cast<int64_t>(s->slot_bytes);
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
  a.st.num_slots = s->layout.num_slots;
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
  a.st.num_slots = s->layout.num_slots;
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

damp_status damp_batch_order(const int32_t* slot_idx, int32_t B, int32_t num_slots, int32_t* order,
                             void* stream) {
  if (B < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "B (%d) must be >= 0", B);
  if (num_slots <= 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "num_slots (%d) must be positive", num_slots);
  if (B == 0) return ok();
  if (!slot_idx || !order) return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL slot_idx or order");
  if (!aligned(slot_idx, 4) || !aligned(order, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "slot_idx and order must be 4-byte aligned");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(slot_idx), a1 = reinterpret_cast<uintptr_t>(order);
  const uintptr_t n = sizeof(int32_t) * static_cast<uintptr_t>(B);
  if (a0 < a1 + n && a1 < a0 + n) return fail(DAMP_ERR_INVALID_ARGUMENT, "order overlaps slot_idx");
  return launched(damp::launch_batch_order(slot_idx, B, num_slots, order, static_cast<hipStream_t>(stream)),
                  "batch order");
}

damp_status damp_decode_step_ordered(damp_state* s, const int32_t* slot_idx, const int32_t* order,
                                     int32_t B, const void* q, const void* k, const void* v,
                                     damp_dtype dt, const float* alpha, damp_decay decay,
                                     const float* beta, float* out, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  if (!order || !aligned(order, 4)) return fail(DAMP_ERR_INVALID_ARGUMENT, "order is NULL or misaligned");
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, alpha, decay, beta, out, stream, 0, nullptr, 0, false, order);
}

damp_status damp_decode_step_sorted(damp_state* s, const int32_t* slot_idx, int32_t B, const void* q,
                                    const void* k, const void* v, damp_dtype dt, const float* alpha,
                                    damp_decay decay, const float* beta, float* out, void* stream) {
  if (B > DAMP_SORTED_MAX_B)
    return fail(DAMP_ERR_UNSUPPORTED, "B = %d exceeds the library-held order buffer (%d entries); "
                "use damp_batch_order and damp_decode_step_ordered with a caller buffer", B,
                DAMP_SORTED_MAX_B);
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* order = nullptr;
  st = scratch_for(hs, &order);
  if (st != DAMP_OK) return st;
  // every entry of order[0, B) is written by the ordering kernel before the step reads it
  st = launched(damp::launch_batch_order(slot_idx, B, L.num_slots, order, hs), "batch order");
  if (st != DAMP_OK) return st;
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, alpha, decay, beta, out, stream, 0, nullptr, 0, false, order);
}

damp_status damp_decode_step_fused(damp_state* s, const int32_t* slot_idx, int32_t B, const void* q,
                                   const void* k, const void* v, damp_dtype dt,
                                   const float* gate_logit, damp_decay decay,
                                   const float* beta_logit, float* out, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, gate_logit, decay,
                                   beta_logit, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, gate_logit, decay, beta_logit, out, stream, 1);
}

damp_status damp_decode_step_fused_ordered(damp_state* s, const int32_t* slot_idx, const int32_t* order,
                                           int32_t B, const void* q, const void* k, const void* v,
                                           damp_dtype dt, const float* gate_logit, damp_decay decay,
                                           const float* beta_logit, float* out, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, gate_logit, decay,
                                   beta_logit, out);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  if (!order || !aligned(order, 4)) return fail(DAMP_ERR_INVALID_ARGUMENT, "order is NULL or misaligned");
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, gate_logit, decay, beta_logit, out, stream, 1, nullptr, 0, false, order);
}

size_t damp_window_bytes(const damp_layout* L, int32_t window) {
  if (!L || window < 1 || window > damp::window_max()) return 0;
  damp_layout T = *L;
  T.num_fp16_rows = 0;
  if (check_layout(&T) != DAMP_OK) return 0;
  const size_t units = static_cast<size_t>(L->num_slots) * static_cast<size_t>(L->num_heads);
  const size_t per = window_unit_bytes(L->d_k, window);
  if (units != 0 && per > SIZE_MAX / units) return 0;
  return units * per;
}

damp_status damp_window_step(damp_state* s, void* window_buf, int32_t window, const int32_t* slot_idx,
                             int32_t B, const void* q, const void* k, const void* v, damp_dtype dt,
                             const float* alpha, damp_decay decay, const float* beta, float* out,
                             void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  st = check_window(window_buf, window);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, alpha, decay, beta, out, stream, 0, window_buf, window, false);
}

damp_status damp_window_step_ordered(damp_state* s, void* window_buf, int32_t window,
                                    const int32_t* slot_idx, const int32_t* order, int32_t B,
                                    const void* q, const void* k, const void* v, damp_dtype dt,
                                    const float* alpha, damp_decay decay, const float* beta,
                                    float* out, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  const damp_layout& L = s->layout;
  damp_status st = check_step_args(B, L.num_heads, L.d_k, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  st = check_window(window_buf, window);
  if (st != DAMP_OK) return st;
  if (B == 0) return ok();
  if (!order || !aligned(order, 4)) return fail(DAMP_ERR_INVALID_ARGUMENT, "order is NULL or misaligned");
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, B, q, k, v,
                  dt, alpha, decay, beta, out, stream, 0, window_buf, window, false, order);
}

damp_status damp_window_flush(damp_state* s, void* window_buf, int32_t window, const int32_t* slot_idx,
                              int32_t n, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  if (n < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "n (%d) must be >= 0", n);
  damp_status st = check_window(window_buf, window);
  if (st != DAMP_OK) return st;
  if (n == 0) return ok();
  if (!slot_idx || !aligned(slot_idx, 4)) return fail(DAMP_ERR_INVALID_ARGUMENT, "slot_idx NULL or misaligned");
  const damp_layout& L = s->layout;
  if (static_cast<int64_t>(n) * L.num_heads > 0x7fffffffLL)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "n * num_heads exceeds the grid limit");
  return run_step(damp::FMT_Q, damp_ref(s), L.d_k, L.num_heads, L.num_slots, slot_idx, n, nullptr,
                  nullptr, nullptr, DAMP_F32, nullptr, DAMP_DECAY_SCALAR, nullptr, nullptr, stream, 0,
                  window_buf, window, true);
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
  a.st.num_slots = num_slots;
  a.slot_idx = slot_idx;
  a.n = n;
  a.H = H;
  a.S = const_cast<float*>(S);
  return launched(damp::launch_quantize(d_k, a, st), "quantize");
}

damp_status damp_risk_scores(const float* S, int32_t n, int32_t H, int32_t d, const float* abar,
                             double* row_error, double* score, void* stream) {
  if (n <= 0 || H <= 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "n (%d) and num_heads (%d) must be positive", n, H);
  if (!supported_d(d))
    return fail(DAMP_ERR_UNSUPPORTED, "d = %d: supported sizes are {16, 32, 64, 128}", d);
  if (!S || !abar || !row_error || !score)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL S, abar, row_error or score");
  if (!aligned(S, 16) || !aligned(abar, 4) || !aligned(row_error, 8) || !aligned(score, 8))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "misaligned pointer (S 16 bytes, abar 4, outputs 8)");
  if (static_cast<int64_t>(n) * H * d > (static_cast<int64_t>(1) << 40))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "n * num_heads * d is too large");
  return launched(damp::launch_risk_scores(d, S, n, H, abar, row_error, score,
                                           static_cast<hipStream_t>(stream)),
                  "risk scores");
}

int64_t damp_budget_rows(int32_t d, int32_t H, double bits_per_value, int32_t g, int32_t r_max) {
  if (d <= 4 || H <= 0 || g < 1 || r_max < 0 || r_max > d) return -1;
  const double budget = bits_per_value * H * static_cast<double>(d) * d / 8.0;
  const double base = static_cast<double>(H) * (static_cast<double>(d) * d + 4.0 * d);
  int64_t R = -1;
  for (int64_t t = 0; t <= static_cast<int64_t>(H) * r_max; t += g)
    if (base + static_cast<double>(d - 4) * t <= budget) R = t;
  return R;
}

damp_status damp_allocate_rows(const double* score, int32_t H, int32_t d, int64_t R, int32_t g,
                               int32_t r_max, int32_t* r_out, int32_t* map_out, void* stream) {
  if (H <= 0 || d <= 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "num_heads (%d) and d (%d) must be positive", H, d);
  if (d > 128) return fail(DAMP_ERR_UNSUPPORTED, "d = %d: at most 128 key rows per head", d);
  if (g < 1 || r_max < 0 || r_max > d)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "g (%d) must be >= 1 and r_max (%d) in [0, d]", g, r_max);
  if (R < 0 || R % g != 0)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "R (%lld) must be >= 0 and a multiple of g (%d)",
                static_cast<long long>(R), g);
  if (static_cast<int64_t>(H) * d > damp::alloc_max_rows())
    return fail(DAMP_ERR_UNSUPPORTED, "num_heads * d = %lld exceeds %d",
                static_cast<long long>(H) * d, damp::alloc_max_rows());
  if (static_cast<int64_t>(H) * (r_max / g) > damp::alloc_max_groups())
    return fail(DAMP_ERR_UNSUPPORTED, "num_heads * (r_max / g) = %lld groups exceeds %d",
                static_cast<long long>(H) * (r_max / g), damp::alloc_max_groups());
  if (!score || !r_out || !map_out) return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL score, r_out or map_out");
  if (!aligned(score, 8) || !aligned(r_out, 4) || !aligned(map_out, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "misaligned pointer");
  return launched(damp::launch_allocate_rows(score, H, d, R, g, r_max, r_out, map_out,
                                             static_cast<hipStream_t>(stream)),
                  "allocate rows");
}

size_t stq_state_bytes(int32_t num_slots, int32_t H, int32_t d, const uint8_t* row_bits) {
  if (stq_check_dims(num_slots, H, d) != DAMP_OK) return 0;
  std::vector<int> cnt;
  if (stq_counts(H, d, row_bits, &cnt) != DAMP_OK) return 0;
  size_t slot = 0;
  for (int32_t h = 0; h < H; ++h)
    slot += round_up(stq_block_bytes(d, cnt[4 * h], cnt[4 * h + 1], cnt[4 * h + 2], cnt[4 * h + 3]), kBlockAlign);
  if (slot != 0 && static_cast<size_t>(num_slots) > SIZE_MAX / slot) return 0;
  return static_cast<size_t>(num_slots) * slot;
}

damp_status stq_state_alloc(int32_t num_slots, int32_t H, int32_t d, const uint8_t* row_bits,
                            const float* impact, void* pool, size_t pool_bytes, stq_state** out) {
  if (!out) return fail(DAMP_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  damp_status st = stq_check_dims(num_slots, H, d);
  if (st != DAMP_OK) return st;
  std::vector<int> cnt;
  st = stq_counts(H, d, row_bits, &cnt);
  if (st != DAMP_OK) return st;
  if (!impact) return fail(DAMP_ERR_INVALID_ARGUMENT, "impact is NULL");
  for (size_t e = 0; e < static_cast<size_t>(H) * d; ++e)
    if (!(impact[e] >= 0.0f) || impact[e] > 1e18f)
      return fail(DAMP_ERR_INVALID_ARGUMENT, "impact[%zu] must be finite and >= 0", e);
  if (!pool) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (!aligned(pool, kBlockAlign)) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool must be 256-byte aligned");
  const size_t need = stq_state_bytes(num_slots, H, d, row_bits);
  if (need == 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool size overflows size_t");
  if (pool_bytes < need) return fail(DAMP_ERR_INVALID_ARGUMENT, "pool_bytes %zu < %zu needed", pool_bytes, need);
  const size_t Hs = static_cast<size_t>(H), ds = static_cast<size_t>(d);
  // device table: rowmap (storage order: pivots, 8-bit, 6-bit, 4-bit, each ascending) | w1 | heads
  std::vector<uint8_t> blob(Hs * ds + 4 * Hs * ds + 16 * Hs, 0);
  float* w1 = reinterpret_cast<float*>(blob.data() + Hs * ds);
  int32_t* heads = reinterpret_cast<int32_t*>(blob.data() + Hs * ds + 4 * Hs * ds);
  stq_state* s = new (std::nothrow) stq_state{};
  if (!s) return fail(DAMP_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
  s->num_slots = num_slots;
  s->num_heads = H;
  s->d = d;
  s->pool = static_cast<uint8_t*>(pool);
  s->head_off.resize(Hs);
  size_t off = 0;
  static const int kWidths[4] = {16, 8, 6, 4};
  for (int32_t h = 0; h < H; ++h) {
    const uint8_t* bits = row_bits + static_cast<size_t>(h) * d;
    const float* w = impact + static_cast<size_t>(h) * d;
    double sw = 0.0;
    for (int32_t i = 0; i < d; ++i)
      if (bits[i] != 16) sw += static_cast<double>(w[i]) * w[i];
    const bool unweighted = !(sw > 0.0);
    if (unweighted) sw = static_cast<double>(d - cnt[4 * h]);   // every integer row weighs 1
    int p = 0;
    for (int k = 0; k < 4; ++k)
      for (int32_t i = 0; i < d; ++i) {
        if (bits[i] != kWidths[k]) continue;
        blob[static_cast<size_t>(h) * d + p] = static_cast<uint8_t>(i);
        w1[static_cast<size_t>(h) * d + p] = k == 0 ? 0.0f : (unweighted ? 1.0f : w[i]);
        ++p;
      }
    s->head_off[static_cast<size_t>(h)] = static_cast<int64_t>(off);
    s->max_pivots = std::max(s->max_pivots, cnt[4 * h]);
    heads[4 * h] = static_cast<int32_t>(off);
    heads[4 * h + 1] = cnt[4 * h] | (cnt[4 * h + 1] << 8) | (cnt[4 * h + 2] << 16) | (cnt[4 * h + 3] << 24);
    std::memcpy(&heads[4 * h + 2], &sw, 8);   // the binary64 sum of w_i^2 over the integer rows
    off += round_up(stq_block_bytes(d, cnt[4 * h], cnt[4 * h + 1], cnt[4 * h + 2], cnt[4 * h + 3]), kBlockAlign);
  }
  s->slot_bytes = off;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&s->table_dev), blob.size());
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete s;
    return fail(e == hipErrorOutOfMemory ? DAMP_ERR_OUT_OF_MEMORY : DAMP_ERR_HIP, "hipMalloc of the table: %s",
                hipGetErrorString(e));
  }
  e = hipMemcpy(s->table_dev, blob.data(), blob.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(s->table_dev);
    delete s;
    return fail(DAMP_ERR_HIP, "copying the table: %s", hipGetErrorString(e));
  }
  *out = s;
  return ok();
}

damp_status stq_state_free(stq_state* s) {
  if (!s) return ok();
  const hipError_t e = s->table_dev ? hipFree(s->table_dev) : hipSuccess;
  delete s;
  if (e != hipSuccess) return fail(DAMP_ERR_HIP, "hipFree of the table: %s", hipGetErrorString(e));
  return ok();
}

damp_status stq_state_head_info(const stq_state* s, int64_t* offset_out, int64_t* slot_bytes) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  for (size_t h = 0; h < s->head_off.size(); ++h)
    if (offset_out) offset_out[h] = s->head_off[h];
  if (slot_bytes) *slot_bytes = static_cast<int64_t>(s->slot_bytes);
  return ok();
}

namespace {
damp_status stq_pack(const stq_state* s, float* S, const int32_t* slot_idx, int32_t n, void* stream, int mode) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  if (n < 0) return fail(DAMP_ERR_INVALID_ARGUMENT, "n (%d) must be >= 0", n);
  if (n == 0) return ok();
  if (!S || !slot_idx) return fail(DAMP_ERR_INVALID_ARGUMENT, "NULL S or slot_idx");
  if (!aligned(S, 16) || !aligned(slot_idx, 4))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "S must be 16-byte and slot_idx 4-byte aligned");
  if (static_cast<int64_t>(n) * s->num_heads > 0x7fffffffLL)
    return fail(DAMP_ERR_INVALID_ARGUMENT, "n * num_heads exceeds the grid limit");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  damp_status r = debug_check_slots(slot_idx, n, s->num_slots, st);
  if (r != DAMP_OK) return r;
  damp::StqArgs a = stq_args(s);
  a.slot_idx = slot_idx;
  a.B = n;
  a.S = S;
  return launched(damp::launch_stq(mode, s->d, 0, 0, a, st), mode == 1 ? "stq quantize" : "stq dequantize");
}
}  // namespace

damp_status stq_state_quantize(stq_state* s, const float* S, const int32_t* slot_idx, int32_t n, void* stream) {
  return stq_pack(s, const_cast<float*>(S), slot_idx, n, stream, 1);
}

damp_status stq_state_dequantize(const stq_state* s, float* S, const int32_t* slot_idx, int32_t n, void* stream) {
  return stq_pack(s, S, slot_idx, n, stream, 2);
}

damp_status stq_decode_step(stq_state* s, void* dst_pool, const int32_t* slot_idx, int32_t B, const void* q,
                            const void* k, const void* v, damp_dtype dt, const float* alpha, damp_decay decay,
                            const float* beta, float* out, void* stream) {
  if (!s) return fail(DAMP_ERR_INVALID_ARGUMENT, "state is NULL");
  damp_status st = check_step_args(B, s->num_heads, s->d, slot_idx, q, k, v, dt, alpha, decay, beta, out);
  if (st != DAMP_OK) return st;
  if (dst_pool && !aligned(dst_pool, kBlockAlign))
    return fail(DAMP_ERR_INVALID_ARGUMENT, "dst_pool must be 256-byte aligned");
  if (B == 0) return ok();
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  st = debug_check_slots(slot_idx, B, s->num_slots, hs);
  if (st != DAMP_OK) return st;
  damp::StqArgs a = stq_args(s);
  a.dst = static_cast<uint8_t*>(dst_pool);
  a.slot_idx = slot_idx;
  a.B = B;
  a.step.slot_idx = slot_idx;
  a.step.B = B;
  a.step.q = q;
  a.step.k = k;
  a.step.v = v;
  a.step.alpha = alpha;
  a.step.beta = beta;
  a.step.out = out;
  return launched(damp::launch_stq(0, s->d, decay == DAMP_DECAY_PER_KEY, dt == DAMP_BF16, a, hs), "stq step");
}

}  // extern "C"
