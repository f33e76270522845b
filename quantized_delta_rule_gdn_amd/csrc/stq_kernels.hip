// stq_kernels.hip -- gfx950 kernels for the STEPQuant-style state (the STEPQuant page, appendix
// Table C2 steps 1-6, Table C1 for KDA's per-key-row allocation): the decode step, pack and
// unpack. Each key row of a head is a pivot kept in FP16 or an integer row of 8, 6 or 4 bits (a
// frozen precision map); the integer rows carry one FP16 row factor each and share one FP16
// column-scale vector per unit; entry (i, j) of an integer row is code * rf_i * cs_j. After the
// update the step refits the scales to X (the fit, for the non-pivot rows N of the unit, with
// row-impact weights w_i):
//   cs_j = fp16( sqrt( sum_{i in N} w_i^2 X_ij^2 / sum_{i in N} w_i^2 ) )
//   rf_i = fp16( max_{j: cs_j > 0} (|X_ij| / cs_j) / qmax_i ),   qmax = 2^(b-1) - 1
//   code = clamp(rint(X_ij / (rf_i cs_j)), -qmax, qmax)   (0 where rf_i cs_j = 0)
// with IEEE binary32 divisions for every decision (rf_i cs_j is exact in binary32). The page
// gives the structure (shared column scales fitted with squared row-impact factors, row factors,
// FP16 scales and pivots) but not these formulas; they are the library's reading.
//
// Block of one (slot, head), storage rows ordered pivots, 8-bit, 6-bit, 4-bit (each ascending
// key index): FP16 pivot rows (2 d bytes each) | 8-bit rows (d) | 6-bit rows (3 d / 4: a plane of
// the low nibbles, d / 2 bytes, then a plane of the top two bits, d / 4 bytes) | 4-bit rows
// (d / 2) | FP16 row factors of the integer rows | FP16 column scales (d) | zero padding to 256 B.
// Codes are two's complement in their width. A lane owns CPL = d / 16 columns of a row, so its
// codes of a row are CPL bytes (8-bit), CPL / 2 + CPL / 4 bytes (6-bit) or CPL / 2 bytes (4-bit):
// d is 64 or 128.
//
// The state is held as fp32 X in VGPRs (64 per lane at d = 128), which the fit needs three times
// (column sums, row maxima, codes). The step may write its new state to another pool than it
// read (Table C2 step 6: the old representation stays valid until its readers finish).
#include "step_common.h"

namespace damp {
namespace {

enum StqKind : int { SK_F16 = 0, SK_I8 = 1, SK_I6 = 2, SK_I4 = 3 };
enum StqMode : int { SM_STEP = 0, SM_PACK = 1, SM_UNPACK = 2 };

struct StqBlock {
  uint32_t o8, o6, o4, orf, ocs;
  int n16, n8, n6, n4;
  float sw;
};

template <int D>
__device__ __forceinline__ StqBlock stq_block(const StqArgs& a, int head) {
  const int4 hi = a.heads[head];   // {offset, counts n16 | n8 << 8 | n6 << 16 | n4 << 24, sw, 0}
  StqBlock b;
  b.n16 = hi.y & 0xff;
  b.n8 = (hi.y >> 8) & 0xff;
  b.n6 = (hi.y >> 16) & 0xff;
  b.n4 = (hi.y >> 24) & 0xff;
  b.o8 = 2u * D * b.n16;
  b.o6 = b.o8 + D * b.n8;
  b.o4 = b.o6 + (3 * D / 4) * b.n6;
  b.orf = b.o4 + (D / 2) * b.n4;
  b.ocs = b.orf + 2 * (D - b.n16);
  b.sw = __int_as_float(hi.z);
  return b;
}

__device__ __forceinline__ int stq_kind(const StqBlock& b, int p) {
  return p < b.n16 ? SK_F16 : (p < b.n16 + b.n8 ? SK_I8 : (p < b.n16 + b.n8 + b.n6 ? SK_I6 : SK_I4));
}

__device__ __forceinline__ int stq_qmax(int kind) {
  return kind == SK_I8 ? 127 : (kind == SK_I6 ? 31 : 7);
}

// The lane's codes of row p, as raw words: F16 CPL halves, I8 CPL bytes, I6 / I4 the nibbles in
// w[0..] and (I6) the top bits in hw.
template <int D>
__device__ __forceinline__ void stq_load(const uint8_t* blk, const StqBlock& b, int kind, int p,
                                         int cg, uint32_t* w, uint32_t& hw) {
  constexpr int CPL = D / 16;
  if (kind == SK_F16) {
    load_bytes<CPL * 2>(blk + (p * D + cg * CPL) * 2, w);
  } else if (kind == SK_I8) {
    load_bytes<CPL>(blk + b.o8 + (p - b.n16) * D + cg * CPL, w);
  } else if (kind == SK_I6) {
    const uint8_t* row = blk + b.o6 + (p - b.n16 - b.n8) * (3 * D / 4);
    load_bytes<CPL / 2>(row + cg * (CPL / 2), w);
    uint32_t t[1];
    load_bytes<CPL / 4>(row + D / 2 + cg * (CPL / 4), t);
    hw = t[0];
  } else {
    load_bytes<CPL / 2>(blk + b.o4 + (p - b.n16 - b.n8 - b.n6) * (D / 2) + cg * (CPL / 2), w);
  }
}

// Code (or FP16 value) c of a loaded row.
__device__ __forceinline__ float stq_decode(int kind, const uint32_t* w, uint32_t hw, int c) {
  if (kind == SK_F16) return half_bits_to_float(w[c >> 1] >> (16 * (c & 1)));
  if (kind == SK_I8) return static_cast<float>(static_cast<int8_t>(w[c >> 2] >> (8 * (c & 3))));
  const uint32_t nib = (w[c >> 3] >> (4 * (c & 7))) & 0xFu;
  if (kind == SK_I4) return static_cast<float>(static_cast<int32_t>(nib << 28) >> 28);
  const uint32_t top = (hw >> (2 * c)) & 0x3u;
  return static_cast<float>(static_cast<int32_t>((nib | (top << 4)) << 26) >> 26);
}

// Store the lane's part of row p: FP16 values, or codes of the row's width.
template <int D>
__device__ __forceinline__ void stq_store(uint8_t* blk, const StqBlock& b, int kind, int p, int cg,
                                          const float* x, const int32_t* code) {
  constexpr int CPL = D / 16;
  if (kind == SK_F16) {
    uint32_t wd[CPL / 2];
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) wd[i] = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) wd[c >> 1] |= float_to_half_bits(x[c]) << (16 * (c & 1));
    store_bytes<CPL * 2>(blk + (p * D + cg * CPL) * 2, wd);
  } else if (kind == SK_I8) {
    uint32_t wd[CPL / 4];
#pragma unroll
    for (int i = 0; i < CPL / 4; ++i) wd[i] = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) wd[c >> 2] |= (static_cast<uint32_t>(code[c]) & 0xFFu) << (8 * (c & 3));
    store_bytes<CPL>(blk + b.o8 + (p - b.n16) * D + cg * CPL, wd);
  } else {
    uint32_t lo[(CPL + 7) / 8], hi = 0;
#pragma unroll
    for (int i = 0; i < (CPL + 7) / 8; ++i) lo[i] = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint32_t u = static_cast<uint32_t>(code[c]);
      lo[c >> 3] |= (u & 0xFu) << (4 * (c & 7));
      hi |= ((u >> 4) & 0x3u) << (2 * c);
    }
    if (kind == SK_I6) {
      uint8_t* row = blk + b.o6 + (p - b.n16 - b.n8) * (3 * D / 4);
      store_bytes<CPL / 2>(row + cg * (CPL / 2), lo);
      store_bytes<CPL / 4>(row + D / 2 + cg * (CPL / 4), &hi);
    } else {
      store_bytes<CPL / 2>(blk + b.o4 + (p - b.n16 - b.n8 - b.n6) * (D / 2) + cg * (CPL / 2), lo);
    }
  }
}

template <int D, int NW>
struct StqSmem {
  float4 srow[D];        // {gate_p, k_p, q_p, w_p^2}, storage order
  float sv[D];           // v, then delta
  float redu[4 * NW][D];
  float redp[4 * NW][D];
  float redqk[NW];
  float scs[D];          // column scales (binary16 values as fp32)
};

// MODE = SM_STEP: one decode step (reads src, writes dst). SM_PACK: fp32 states (key order) ->
// format. SM_UNPACK: format -> fp32 states (key order).
template <int D, int PER_KEY, int BF16, int MODE>
__global__ __launch_bounds__(Geo<D>::NT) void stq_kernel(const StqArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL, RPL = G::RPL, NW = G::NW;
  __shared__ StqSmem<D, NW> sm;
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int bh = __builtin_amdgcn_workgroup_id_x();
  const int b = bh / a.H;
  const int head = bh - b * a.H;
  const int64_t slot = a.slot_idx[b];
  const StqBlock blk = stq_block<D>(a, head);
  const int64_t boff = slot * a.slot_stride + a.heads[head].x;
  const uint8_t* src = a.pool + boff;
  uint8_t* dst = (a.dst ? a.dst : a.pool) + boff;
  const uint8_t* rowmap = a.rowmap + head * D;

  float X[RPL][CPL];
  if constexpr (MODE == SM_PACK) {
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int p = t * G::RPS + w * 4 + rs;
      load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(a.S + (int64_t(bh) * D + rowmap[p]) * D + cg * CPL),
                          reinterpret_cast<uint32_t*>(X[t]));
    }
  } else {
    // (1) the stored state: codes, row factors, column scales; reconstructed into X
    float csv[CPL];
    {
      uint32_t cw[CPL / 2];
      load_bytes<CPL * 2>(src + blk.ocs + cg * CPL * 2, cw);
#pragma unroll
      for (int c = 0; c < CPL; ++c) csv[c] = half_bits_to_float(cw[c >> 1] >> (16 * (c & 1)));
    }
    uint32_t raw[RPL][CPL / 2];
    uint32_t hw[RPL];
    float rfv[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int p = t * G::RPS + w * 4 + rs;
      const int kind = stq_kind(blk, p);
      hw[t] = 0;
      stq_load<D>(src, blk, kind, p, cg, raw[t], hw[t]);
      rfv[t] = 1.0f;
      if (kind != SK_F16) rfv[t] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(src + blk.orf + 2 * (p - blk.n16)));
    }
    if constexpr (MODE == SM_UNPACK) {
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const int p = t * G::RPS + w * 4 + rs;
        const int kind = stq_kind(blk, p);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float v = stq_decode(kind, raw[t], hw[t], c);
          X[t][c] = kind == SK_F16 ? v : v * (rfv[t] * csv[c]);
        }
        store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(a.S + (int64_t(bh) * D + rowmap[p]) * D + cg * CPL),
                             reinterpret_cast<const uint32_t*>(X[t]));
      }
      return;
    } else {
      // (2) per-row scalars: gate, k, q (storage order) and v
      const float beta = stage_rows<D, G::NT, PER_KEY, BF16, false>(a.step, nullptr, bh, head, 0, tid,
                                                                     sm.srow, sm.sv, &sm.redu[0][0]);
      // (3) S' = gate * S_hat in X, and the column sums u, p
      float pu[CPL], pp[CPL], pqk = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) pu[c] = pp[c] = 0.0f;
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const int p = t * G::RPS + w * 4 + rs;
        const int kind = stq_kind(blk, p);
        const float4 rw = sm.srow[p];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float v = stq_decode(kind, raw[t], hw[t], c);
          X[t][c] = rw.x * (kind == SK_F16 ? v : v * (rfv[t] * csv[c]));
          pu[c] = fmaf(rw.y, X[t][c], pu[c]);
          pp[c] = fmaf(rw.z, X[t][c], pp[c]);
        }
        pqk = fmaf(rw.z, rw.y, pqk);
      }
      finish_columns<D, G>(sm.redu, sm.redp, sm.redqk, sm.sv, pu, pp, pqk, beta,
                           a.step.out + int64_t(bh) * D, tid, w, rs, lane, cg);
      float dl[CPL];
      load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.sv + cg * CPL), reinterpret_cast<uint32_t*>(dl));
      // (4) X = S' + k delta^T
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const float kp = sm.srow[t * G::RPS + w * 4 + rs].y;
#pragma unroll
        for (int c = 0; c < CPL; ++c) X[t][c] = fmaf(kp, dl[c], X[t][c]);
      }
    }
  }

  // (5) the fit. Row weights w_p^2 of the integer rows (0 for pivots), in storage order.
  float cs_part[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) cs_part[c] = 0.0f;
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    const float w2 = a.w2[head * D + p];
#pragma unroll
    for (int c = 0; c < CPL; ++c) cs_part[c] = fmaf(w2 * X[t][c], X[t][c], cs_part[c]);
  }
  store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(&sm.redu[w * 4 + rs][cg * CPL]),
                       reinterpret_cast<const uint32_t*>(cs_part));
  __syncthreads();
  for (int j = tid; j < D; j += G::NT) {
    float s = sm.redu[0][j];
#pragma unroll
    for (int k = 1; k < 4 * NW; ++k) s += sm.redu[k][j];
    const uint32_t hb = blk.sw > 0.0f ? float_to_half_bits(sqrtf(__fdiv_rn(s, blk.sw))) : 0u;
    sm.scs[j] = half_bits_to_float(hb);
    reinterpret_cast<uint16_t*>(dst + blk.ocs)[j] = static_cast<uint16_t>(hb);
  }
  __syncthreads();
  float csv2[CPL];
  load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.scs + cg * CPL), reinterpret_cast<uint32_t*>(csv2));
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p = t * G::RPS + w * 4 + rs;
    const int kind = stq_kind(blk, p);
    int32_t code[CPL];
    if (kind != SK_F16) {
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (csv2[c] > 0.0f) m = fmaxf(m, __fdiv_rn(fabsf(X[t][c]), csv2[c]));
      m = max_row16(m);
      const int qm = stq_qmax(kind);
      const uint32_t rb = float_to_half_bits(__fdiv_rn(m, static_cast<float>(qm)));
      const float rf = half_bits_to_float(rb);
      if (cg == 0) reinterpret_cast<uint16_t*>(dst + blk.orf)[p - blk.n16] = static_cast<uint16_t>(rb);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float sc = rf * csv2[c];   // exact: two binary16 significands
        float q = sc > 0.0f ? rintf(__fdiv_rn(X[t][c], sc)) : 0.0f;
        q = fminf(fmaxf(q, static_cast<float>(-qm)), static_cast<float>(qm));
        code[c] = static_cast<int32_t>(q);
      }
    }
    stq_store<D>(dst, blk, kind, p, cg, X[t], code);
  }
}

template <int D, int MODE>
hipError_t stq_launch_mode(int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H)), block(Geo<D>::NT);
  if constexpr (MODE != SM_STEP) {
    hipLaunchKernelGGL((stq_kernel<D, 0, 0, MODE>), grid, block, 0, s, a);
  } else if (per_key) {
    if (bf16) hipLaunchKernelGGL((stq_kernel<D, 1, 1, MODE>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stq_kernel<D, 1, 0, MODE>), grid, block, 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((stq_kernel<D, 0, 1, MODE>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stq_kernel<D, 0, 0, MODE>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t stq_d(int mode, int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  if (mode == SM_STEP) return stq_launch_mode<D, SM_STEP>(per_key, bf16, a, s);
  if (mode == SM_PACK) return stq_launch_mode<D, SM_PACK>(per_key, bf16, a, s);
  return stq_launch_mode<D, SM_UNPACK>(per_key, bf16, a, s);
}

}  // namespace

hipError_t launch_stq(int mode, int d, int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  switch (d) {
    case 64: return stq_d<64>(mode, per_key, bf16, a, s);
    case 128: return stq_d<128>(mode, per_key, bf16, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace damp
