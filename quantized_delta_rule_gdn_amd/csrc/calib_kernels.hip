// calib_kernels.hip -- gfx950 kernels of the offline calibration: per-row INT8 error energy of
// calibration states, decay-weighted risk scores, and the grouped allocation of a storage
// budget's FP16 rows over the heads (the DAMP abstracts: high-risk key channels are chosen
// offline from quantization-error energy and decay-based error retention and kept in FP16
// under a fixed storage budget).
//
// These kernels run once per model, not per token. Their results are integers (which rows are
// FP16) decided by comparing floating-point scores, so the scores are computed in binary64 in
// one fixed order (row errors with j ascending, then slots ascending, then the two divisions),
// which makes them identical on every run and to any other evaluation in that order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace damp {
namespace {

// Squared INT8 error of one row, binary64 with j ascending. The row's scale and codes follow
// the INT8 rule exactly: scale = fl32(m / 127) and code = rint(fl32(x / scale)) clamped to
// [-127, 127], both with IEEE division. d = x - scale * code is exact in binary64 (the product
// has at most 31 significant bits and, when the code is non-zero, both terms lie within a factor
// 256 of the scale), so only the square and the running sum round.
template <int D>
__device__ double row_error(const float* row) {
  float m = 0.0f;
  for (int j = 0; j < D; j += 4) {
    const float4 x = *reinterpret_cast<const float4*>(row + j);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
  }
  if (m == 0.0f) return 0.0;
  const float sc = __fdiv_rn(m, 127.0f);
  double e = 0.0;
  for (int j = 0; j < D; j += 4) {
    const float4 x4 = *reinterpret_cast<const float4*>(row + j);
    const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float c = fminf(fmaxf(rintf(__fdiv_rn(xs[u], sc)), -127.0f), 127.0f);
      const double d = static_cast<double>(xs[u]) - static_cast<double>(sc) * static_cast<double>(c);
      e += d * d;
    }
  }
  return e;
}

// One thread per (slot, head, key row): row_error[s][h][i].
template <int D>
__global__ __launch_bounds__(256) void row_error_kernel(const float* S, int64_t rows, double* out) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= rows) return;
  out[t] = row_error<D>(S + t * D);
}

// One thread per (head, key row): the slots' errors added in ascending slot order, divided by
// n and by (1 - abar).
__global__ __launch_bounds__(256) void score_kernel(const double* row_err, int32_t n, int32_t hd,
                                                   const float* abar, double* score) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= hd) return;
  double e = 0.0;
  for (int32_t s = 0; s < n; ++s) e += row_err[int64_t(s) * hd + t];
  e /= static_cast<double>(n);
  score[t] = e / (1.0 - static_cast<double>(abar[t]));
}

// ---- allocation ------------------------------------------------------------------------------
constexpr int kAllocThreads = 1024;
constexpr int kMaxRows = 8192;    // num_heads * d
constexpr int kMaxGroups = 4096;  // num_heads * (r_max / g)

// One workgroup: (1) each head's ranking by (score desc, row asc), as a rank per row and the row
// at each rank; (2) each group's gain, summed in rank order; (3) each group's global rank by
// (gain desc, group index asc) and whether it is among the K taken; (4) r_h; (5) the row map.
// Every rank is a count of the entries that precede it, so ties resolve exactly as the order
// states and the result does not depend on thread scheduling.
__global__ __launch_bounds__(kAllocThreads) void allocate_kernel(const double* score, int32_t H,
                                                                 int32_t D, int64_t K, int32_t g,
                                                                 int32_t G, int32_t* r_out,
                                                                 int32_t* map_out) {
  __shared__ uint8_t rank_of[kMaxRows];   // [h][i] -> rank of row i in head h
  __shared__ uint8_t row_at[kMaxRows];    // [h][t] -> row at rank t
  __shared__ double gain[kMaxGroups];     // [h][j]
  __shared__ uint8_t taken[kMaxGroups];
  __shared__ int32_t rh[kMaxRows / 16];   // r_h (num_heads <= 8192 / 16)
  const int tid = threadIdx.x;
  const int HD = H * D, C = H * G;

  for (int t = tid; t < HD; t += kAllocThreads) {
    const int h = t / D, i = t - h * D;
    const double* sc = score + int64_t(h) * D;
    const double s = sc[i];
    int rank = 0;
    for (int i2 = 0; i2 < D; ++i2) {
      const double s2 = sc[i2];
      rank += (s2 > s || (s2 == s && i2 < i)) ? 1 : 0;
    }
    rank_of[t] = static_cast<uint8_t>(rank);
    row_at[h * D + rank] = static_cast<uint8_t>(i);
  }
  __syncthreads();
  for (int x = tid; x < C; x += kAllocThreads) {
    const int h = x / G, j = x - h * G;
    double sum = 0.0;
    for (int t = j * g; t < j * g + g; ++t) sum += score[int64_t(h) * D + row_at[h * D + t]];
    gain[x] = sum;
  }
  __syncthreads();
  for (int x = tid; x < C; x += kAllocThreads) {
    const double gx = gain[x];
    int64_t rank = 0;
    for (int x2 = 0; x2 < C; ++x2) {
      const double g2 = gain[x2];
      rank += (g2 > gx || (g2 == gx && x2 < x)) ? 1 : 0;
    }
    taken[x] = rank < K ? 1 : 0;
  }
  __syncthreads();
  for (int h = tid; h < H; h += kAllocThreads) {
    int r = 0;
    for (int j = 0; j < G; ++j) r += taken[h * G + j] ? g : 0;
    rh[h] = r;
    r_out[h] = r;
  }
  __syncthreads();
  for (int t = tid; t < HD; t += kAllocThreads) {
    const int h = t / D, i = t - h * D;
    const int r = rh[h];
    const bool fp16 = rank_of[t] < r;
    int pos = fp16 ? 0 : r;
    for (int i2 = 0; i2 < i; ++i2) pos += ((rank_of[h * D + i2] < r) == fp16) ? 1 : 0;
    map_out[int64_t(h) * D + pos] = i;
  }
}

template <int D>
hipError_t risk_d(const float* S, int32_t n, int32_t H, const float* abar, double* row_err,
                  double* score, hipStream_t s) {
  const int64_t rows = int64_t(n) * H * D;
  hipLaunchKernelGGL(row_error_kernel<D>, dim3(static_cast<unsigned>((rows + 255) / 256)), dim3(256),
                     0, s, S, rows, row_err);
  const int hd = H * D;
  hipLaunchKernelGGL(score_kernel, dim3(static_cast<unsigned>((hd + 255) / 256)), dim3(256), 0, s,
                     row_err, n, hd, abar, score);
  return hipGetLastError();
}

}  // namespace

int alloc_max_rows() { return kMaxRows; }
int alloc_max_groups() { return kMaxGroups; }

hipError_t launch_risk_scores(int d, const float* S, int32_t n, int32_t H, const float* abar,
                              double* row_err, double* score, hipStream_t s) {
  switch (d) {
    case 16: return risk_d<16>(S, n, H, abar, row_err, score, s);
    case 32: return risk_d<32>(S, n, H, abar, row_err, score, s);
    case 64: return risk_d<64>(S, n, H, abar, row_err, score, s);
    case 128: return risk_d<128>(S, n, H, abar, row_err, score, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_allocate_rows(const double* score, int32_t H, int32_t d, int64_t R, int32_t g,
                                int32_t r_max, int32_t* r_out, int32_t* map_out, hipStream_t s) {
  const int32_t G = r_max / g;
  int64_t K = R / g;
  if (K > int64_t(H) * G) K = int64_t(H) * G;
  hipLaunchKernelGGL(allocate_kernel, dim3(1), dim3(kAllocThreads), 0, s, score, H, d, K, g, G,
                     r_out, map_out);
  return hipGetLastError();
}

}  // namespace damp
