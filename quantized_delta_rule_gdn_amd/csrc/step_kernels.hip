// step_kernels.hip -- gfx950 kernels for the GDN / KDA recurrent-state decode step in three
// state formats (FP32; DAMP FP16 + INT8 rows; uniform INT8 = DAMP with no FP16 rows), and the
// pack / unpack kernels between fp32 states and the quantized formats.
//
// The step (STEPQuant page, appendix Table C2, steps 1-3 and 6; DAMP abstract for the FP16 /
// INT8 split and the per-key-channel KDA gate), per unit = one (slot, head) state:
//   S_hat = reconstruct(state)          codes * scale, or binary16, or fp32
//   S'    = diag(a) S_hat               a_i = alpha (GDN) or alpha_i (KDA)
//   u     = S'^T k,  p = S'^T q         column reductions over the key rows
//   delta = beta (v - u)
//   X     = S' + k delta^T
//   y     = X^T q = p + (q.k) delta     readout from X, before requantization
//   state = requantize(X)               FP16 rows RNE; INT8 rows absmax/127 scale, RNE codes
//
// Mapping on CDNA4 (wave64). One workgroup per unit; the whole state stays in VGPRs, so every
// state byte crosses HBM once in and once out. Lanes: 16 consecutive lanes own one key row
// (CPL = d/16 value columns each), the 4 row slots of a wave cover 4 consecutive storage rows,
// and a row step of the workgroup covers 4 * NW rows, so each load/store instruction of a wave
// touches 4 whole consecutive rows (512 B INT8 / 1 KiB FP16 / 2 KiB fp32 at d = 128):
// fully coalesced. Column sums over key rows use the gfx950 cross-row lane swaps
// (v_permlane16_swap / v_permlane32_swap) inside a wave and LDS across waves; the row absmax for
// requantization is a DPP butterfly inside the 16 lanes of a row. No MFMA: each unit is a
// matrix-vector update at ~4 flop/byte, far below the fp32 ridge; the kernel is HBM-bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace damp {
namespace {

template <int D>
struct Geo {
  static constexpr int NW = D >= 128 ? 4 : (D >= 64 ? 2 : 1);  // waves per workgroup
  static constexpr int NT = NW * 64;                           // threads per workgroup
  static constexpr int CPL = D / 16;                           // value columns per lane
  static constexpr int RPS = NW * 4;                           // storage rows per row step
  static constexpr int RPL = D / RPS;                          // row steps (rows) per lane
  static_assert(D % 16 == 0 && RPL * RPS == D, "unsupported d");
};

// ---- raw byte movement: N bytes per lane as 32-bit words ----------------------------------
template <int N>
struct Words {
  static constexpr int W = N >= 4 ? N / 4 : 1;
};

template <int N>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* w) {
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i + 0] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  } else if constexpr (N == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else if constexpr (N == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (N == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    static_assert(N == 1, "bad width");
    w[0] = *p;
  }
}

template <int N>
__device__ __forceinline__ void store_bytes(uint8_t* p, const uint32_t* w) {
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i)
      reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (N == 8) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint32_t*>(p) = w[0];
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w[0]);
  } else {
    *p = static_cast<uint8_t>(w[0]);
  }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  const uint16_t b = static_cast<uint16_t>(bits16);
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);  // exact widening
}

__device__ __forceinline__ uint32_t float_to_half_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);  // v_cvt_f16_f32: round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

template <int BF16>
__device__ __forceinline__ float load_in(const void* base, int64_t i) {
  if constexpr (BF16) {
    const uint32_t b = reinterpret_cast<const uint16_t*>(base)[i];
    return __uint_as_float(b << 16);  // exact widening
  } else {
    return reinterpret_cast<const float*>(base)[i];
  }
}

// ---- cross-lane reductions ------------------------------------------------------------------
// Sum over the 4 row slots of a wave (lanes l, l^16, l^32, l^48). permlane16_swap(x, x) returns
// {x of the even row of each row pair, x of the odd row}, so their sum is the pair sum in
// every lane of the pair; permlane32_swap does the same for the two halves of the wave.
// Every lane ends with the same value, added in the same order.
__device__ __forceinline__ float sum_row_slots(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t u2 = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Max over the 16 lanes of a row: DPP quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror. Exact (max is order-free); every lane of the row ends with the row max.
__device__ __forceinline__ float max_row16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)));
  return x;
}

// INT8 code of x for a row scale s (s > 0) with inv = fl(1/s): round-half-to-even of the
// binary32 quotient fl(x / s), as the row rule defines it. The fast estimate y = fl(x * inv)
// is within 2^-23 relative (|y| <= 127.5, so within 1.6e-5 absolute) of x/s, and fl(x/s) is
// within 3.9e-6 of x/s; when y is farther than 2^-15 from a half-integer, fl(x/s) rounds to
// the same integer as y, otherwise the exact division is taken (a few cases per million).
__device__ __forceinline__ int32_t int8_code(float x, float s, float inv) {
  const float y = x * inv;
  float n = rintf(y);
  if (fabsf(y - n) > 0.5f - 0x1p-15f) n = rintf(__fdiv_rn(x, s));
  n = fminf(fmaxf(n, -127.0f), 127.0f);
  return static_cast<int32_t>(n);
}

// ---- requantize-and-store of the lane's RPL x CPL values (shared by step and pack) -------
template <int D, int FMT>
__device__ __forceinline__ void store_state(const StateRef& st, int64_t unit, int w, int rs,
                                            int cg, float (&X)[Geo<D>::RPL][Geo<D>::CPL]) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL;
  const int r = FMT == FMT_Q ? st.r : 0;
#pragma unroll
  for (int t = 0; t < G::RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    if constexpr (FMT == FMT_F32) {
      uint32_t wd[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) wd[c] = __float_as_uint(X[t][c]);
      store_bytes<CPL * 4>(st.hbase + unit * st.hstride + (int64_t(p) * D + cg * CPL) * 4, wd);
    } else {
      if (p < r) {
        uint32_t wd[Words<CPL * 2>::W];
#pragma unroll
        for (int i = 0; i < Words<CPL * 2>::W; ++i) wd[i] = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) wd[c >> 1] |= float_to_half_bits(X[t][c]) << (16 * (c & 1));
        store_bytes<CPL * 2>(st.hbase + unit * st.hstride + (int64_t(p) * D + cg * CPL) * 2, wd);
      } else {
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) m = fmaxf(m, fabsf(X[t][c]));
        m = max_row16(m);
        const float s = m > 0.0f ? __fdiv_rn(m, 127.0f) : 0.0f;
        const float inv = m > 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
        uint32_t wd[Words<CPL>::W];
#pragma unroll
        for (int i = 0; i < Words<CPL>::W; ++i) wd[i] = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int32_t code = m > 0.0f ? int8_code(X[t][c], s, inv) : 0;
          wd[c >> 2] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (c & 3));
        }
        store_bytes<CPL>(st.cbase + unit * st.cstride + int64_t(p - r) * D + cg * CPL, wd);
        if (cg == 0)
          reinterpret_cast<float*>(st.sbase + unit * st.sstride)[p - r] = s;
      }
    }
  }
}

// Raw words a lane holds for one storage row before decoding.
template <int D, int FMT>
struct RawRow {
  static constexpr int W = FMT == FMT_F32 ? Geo<D>::CPL : Words<Geo<D>::CPL * 2>::W;
};

template <int D, int FMT>
__device__ __forceinline__ void load_state(const StateRef& st, int64_t unit, int w, int rs, int cg,
                                           uint32_t (&raw)[Geo<D>::RPL][RawRow<D, FMT>::W]) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL;
  const int r = FMT == FMT_Q ? st.r : 0;
#pragma unroll
  for (int t = 0; t < G::RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    if constexpr (FMT == FMT_F32) {
      load_bytes<CPL * 4>(st.hbase + unit * st.hstride + (int64_t(p) * D + cg * CPL) * 4, raw[t]);
    } else {
      if (p < r)
        load_bytes<CPL * 2>(st.hbase + unit * st.hstride + (int64_t(p) * D + cg * CPL) * 2, raw[t]);
      else
        load_bytes<CPL>(st.cbase + unit * st.cstride + int64_t(p - r) * D + cg * CPL, raw[t]);
    }
  }
}

// Element c of a raw row: fp32 bits, binary16 bits, or an int8 code.
template <int FMT>
__device__ __forceinline__ float raw_fp(const uint32_t* w, int c, bool fp16) {
  if constexpr (FMT == FMT_F32) {
    return __uint_as_float(w[c]);
  } else {
    if (fp16) return half_bits_to_float(w[c >> 1] >> (16 * (c & 1)));
    return static_cast<float>(static_cast<int8_t>(w[c >> 2] >> (8 * (c & 3))));
  }
}

// ---- the decode step -----------------------------------------------------------------------
template <int D, int FMT, int PER_KEY, int BF16>
__global__ __launch_bounds__(Geo<D>::NT) void step_kernel(const StepArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL, RPL = G::RPL, NW = G::NW;
  __shared__ float sk[D], sq[D], sv[D], sa[D], ssc[D];
  __shared__ float red[NW][2 * D + 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int bh = blockIdx.x;  // b * H + head
  const int b = bh / a.H;
  const int head = bh - b * a.H;
  const int64_t unit = int64_t(a.slot_idx[b]) * a.H + head;
  const int r = FMT == FMT_Q ? a.st.r : 0;

  // (1) issue every state load of this lane first, so the whole block is in flight
  uint32_t raw[RPL][RawRow<D, FMT>::W];
  load_state<D, FMT>(a.st, unit, w, rs, cg, raw);

  // (2) stage k, q, v, the gate and the (gate-folded) row scales in LDS, in storage-row order
  const int64_t vec = int64_t(bh) * D;
  for (int i = tid; i < D; i += G::NT) {
    const int src = a.st.rowmap ? a.st.rowmap[head * D + i] : i;
    sk[i] = load_in<BF16>(a.k, vec + src);
    sq[i] = load_in<BF16>(a.q, vec + src);
    sv[i] = load_in<BF16>(a.v, vec + i);
    const float g = PER_KEY ? a.alpha[vec + src] : a.alpha[bh];
    sa[i] = g;
    if constexpr (FMT == FMT_Q)
      ssc[i] = i >= r ? reinterpret_cast<const float*>(a.st.sbase + unit * a.st.sstride)[i - r] * g
                      : 0.0f;
  }
  __syncthreads();

  // (3) reconstruct + decay, partial u = S'^T k, p = S'^T q over this lane's rows
  float S[RPL][CPL];
  float kr[RPL];
  float pu[CPL], pp[CPL], pqk = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) pu[c] = pp[c] = 0.0f;
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    const float kp = sk[p], qp = sq[p];
    kr[t] = kp;
    const bool fp16 = p < r;
    const float mul = (FMT == FMT_Q && !fp16) ? ssc[p] : sa[p];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      S[t][c] = raw_fp<FMT>(raw[t], c, fp16) * mul;
      pu[c] = fmaf(kp, S[t][c], pu[c]);
      pp[c] = fmaf(qp, S[t][c], pp[c]);
    }
    pqk = fmaf(qp, kp, pqk);
  }

  // (4) finish the column reductions: row slots in the wave, then waves through LDS
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    pu[c] = sum_row_slots(pu[c]);
    pp[c] = sum_row_slots(pp[c]);
  }
  pqk = sum_row_slots(pqk);
  if constexpr (NW > 1) {
    if (rs == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        red[w][cg * CPL + c] = pu[c];
        red[w][D + cg * CPL + c] = pp[c];
      }
      if (cg == 0) red[w][2 * D] = pqk;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float uu = red[0][cg * CPL + c], vv = red[0][D + cg * CPL + c];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) {
        uu += red[w2][cg * CPL + c];
        vv += red[w2][D + cg * CPL + c];
      }
      pu[c] = uu;
      pp[c] = vv;
    }
    float qk = red[0][2 * D];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) qk += red[w2][2 * D];
    pqk = qk;
  }

  // (5) delta, readout y = p + (q.k) delta, rank-1 write X = S' + k delta^T
  const float beta = a.beta[bh];
  float dl[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) dl[c] = beta * (sv[cg * CPL + c] - pu[c]);
  if (w == 0 && rs == 0) {
    uint32_t o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = __float_as_uint(fmaf(pqk, dl[c], pp[c]));
    store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(a.out + vec + cg * CPL), o);
  }
#pragma unroll
  for (int t = 0; t < RPL; ++t)
#pragma unroll
    for (int c = 0; c < CPL; ++c) S[t][c] = fmaf(kr[t], dl[c], S[t][c]);

  // (6) requantize in place
  store_state<D, FMT>(a.st, unit, w, rs, cg, S);
}

// ---- pack: fp32 states (original key order) -> state format ---------------------------------
template <int D, int FMT>
__global__ __launch_bounds__(Geo<D>::NT) void quantize_kernel(const PackArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int ih = blockIdx.x;  // i * H + head
  const int i = ih / a.H;
  const int head = ih - i * a.H;
  const int64_t unit = int64_t(a.slot_idx[i]) * a.H + head;
  float X[G::RPL][CPL];
#pragma unroll
  for (int t = 0; t < G::RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    const int src = a.st.rowmap ? a.st.rowmap[head * D + p] : p;
    uint32_t wd[CPL];
    load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(a.S + (int64_t(ih) * D + src) * D + cg * CPL), wd);
#pragma unroll
    for (int c = 0; c < CPL; ++c) X[t][c] = __uint_as_float(wd[c]);
  }
  store_state<D, FMT>(a.st, unit, w, rs, cg, X);
}

// ---- unpack: state format -> fp32 states (original key order) ------------------------------
template <int D, int FMT>
__global__ __launch_bounds__(Geo<D>::NT) void dequantize_kernel(const PackArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int ih = blockIdx.x;
  const int i = ih / a.H;
  const int head = ih - i * a.H;
  const int64_t unit = int64_t(a.slot_idx[i]) * a.H + head;
  const int r = FMT == FMT_Q ? a.st.r : 0;
  uint32_t raw[G::RPL][RawRow<D, FMT>::W];
  load_state<D, FMT>(a.st, unit, w, rs, cg, raw);
#pragma unroll
  for (int t = 0; t < G::RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    const int src = a.st.rowmap ? a.st.rowmap[head * D + p] : p;
    const bool fp16 = p < r;
    const float sc = (FMT == FMT_Q && !fp16)
                         ? reinterpret_cast<const float*>(a.st.sbase + unit * a.st.sstride)[p - r]
                         : 1.0f;
    uint32_t wd[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) wd[c] = __float_as_uint(raw_fp<FMT>(raw[t], c, fp16) * sc);
    store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(a.S + (int64_t(ih) * D + src) * D + cg * CPL), wd);
  }
}

template <int D>
hipError_t step_d(int fmt, int per_key, int bf16, const StepArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H));
  const dim3 block(Geo<D>::NT);
#define DAMP_LAUNCH(F, K, T) \
  hipLaunchKernelGGL((step_kernel<D, F, K, T>), grid, block, 0, s, a)
  if (fmt == FMT_F32) {
    if (per_key) { if (bf16) DAMP_LAUNCH(FMT_F32, 1, 1); else DAMP_LAUNCH(FMT_F32, 1, 0); }
    else         { if (bf16) DAMP_LAUNCH(FMT_F32, 0, 1); else DAMP_LAUNCH(FMT_F32, 0, 0); }
  } else {
    if (per_key) { if (bf16) DAMP_LAUNCH(FMT_Q, 1, 1); else DAMP_LAUNCH(FMT_Q, 1, 0); }
    else         { if (bf16) DAMP_LAUNCH(FMT_Q, 0, 1); else DAMP_LAUNCH(FMT_Q, 0, 0); }
  }
#undef DAMP_LAUNCH
  return hipGetLastError();
}

template <int D>
hipError_t quant_d(const PackArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((quantize_kernel<D, FMT_Q>), dim3(unsigned(a.n) * unsigned(a.H)),
                     dim3(Geo<D>::NT), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t dequant_d(const PackArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((dequantize_kernel<D, FMT_Q>), dim3(unsigned(a.n) * unsigned(a.H)),
                     dim3(Geo<D>::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(int fmt, int d, int per_key, int bf16, const StepArgs& a, hipStream_t s) {
  switch (d) {
    case 16: return step_d<16>(fmt, per_key, bf16, a, s);
    case 32: return step_d<32>(fmt, per_key, bf16, a, s);
    case 64: return step_d<64>(fmt, per_key, bf16, a, s);
    case 128: return step_d<128>(fmt, per_key, bf16, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize(int d, const PackArgs& a, hipStream_t s) {
  switch (d) {
    case 16: return quant_d<16>(a, s);
    case 32: return quant_d<32>(a, s);
    case 64: return quant_d<64>(a, s);
    case 128: return quant_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequantize(int d, const PackArgs& a, hipStream_t s) {
  switch (d) {
    case 16: return dequant_d<16>(a, s);
    case 32: return dequant_d<32>(a, s);
    case 64: return dequant_d<64>(a, s);
    case 128: return dequant_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace damp
