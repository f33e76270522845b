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
// The page gives the structure (per-head column scales whose fit weighs each row by the square of
// its impact score, row factors, FP16 scales and pivots) but not these formulas; they are the
// library's reading.
//
// Block of one (slot, head), storage rows ordered pivots, 8-bit, 6-bit, 4-bit (each ascending
// key index): FP16 pivot rows (2 d bytes each) | 8-bit rows (d) | 6-bit rows (3 d / 4: a plane of
// the low nibbles, d / 2 bytes, then a plane of the top two bits, d / 4 bytes) | 4-bit rows
// (d / 2) | FP16 row factors of the integer rows | FP16 column scales (d) | zero padding to 256 B.
// Codes are two's complement in their width. A lane owns CPL = d / 16 columns of a row, so its
// codes of a row are CPL bytes (8-bit), CPL / 2 + CPL / 4 bytes (6-bit) or CPL / 2 bytes (4-bit):
// d is 64 or 128.
//
// Mapping. One workgroup per unit; 16 lanes own a row, a wave's 4 row slots take 4 consecutive
// storage rows. The precision map is a runtime table, but the rows are stored by kind, so a
// wave's 4 rows almost always share one kind: every per-kind step (load, decode, pack + store)
// is chosen by a wave-uniform test of the kinds of the wave's first and last row, and only the
// few row groups that straddle two kinds run two kinds under an exec mask. The state is held as
// fp32 X in VGPRs (the fit needs it three times: column sums, row maxima, codes); state bytes go
// through raw buffer instructions with the non-temporal policy, like the DAMP step.
//
// Decoding. 6-bit codes are rebuilt as signed bytes holding 4 * code and 4-bit codes as 16 * code
// (the sign bit moved to bit 7), so every integer row converts with one signed-byte instruction
// per value; the staged row multiplier carries the exact power-of-two inverse.
//
// Arithmetic of the fit. Column scales: each lane sums (w_i X_ij)^2 over its rows in order
// (pack: in binary64, w_i X_ij exact, so only the order of the sums differs from the oracle's
// and pack's scales agree unless a square root lies within ~1e-15 of a binary16 tie; the step:
// in binary32, within 5 binary32 ulps of the binary64 fit at d = 128, see the fit below); the
// column thread adds the lanes' partials in binary64 in a fixed order, divides by the binary64
// sum of w_i^2 and takes the square root (IEEE binary64 division and square root), rounded once
// to binary16 (through a round-to-odd binary32 value).
// The column thread also forms rcs_j = RN(1 / cs_j). Row factor: the row maximum m of |X_ij| rcs_j (pack: the quotient
// corrected to the IEEE one by one residual step, exact because cs_j has an 11-bit significand),
// divided by qmax with one multiply and one residual correction (correctly rounded for 7, 31 and
// 127 at every binary32 significand). Codes: pack takes the IEEE quotient X / (rf cs) for each
// (rf cs is exact in binary32); the step rounds a_j rcp(rf), with a_j = X_ij rcs_j the same
// product its row maximum used, by one fma against 1.5 * 2^23, like the DAMP step's codes. Since
// |a_j| <= m and rf >= (m / qmax)(1 - 2^-11) for a normal binary16 rf, no such code rounds past
// qmax; only a row group holding a subnormal or zero row factor clamps.
// The step may write its new state to another pool than it read (Table C2 step 6: the previous
// copy stays intact while readers still use it).
#include <type_traits>

#include "step_common.h"

namespace damp {
namespace {

enum StqKind : int { SK_F16 = 0, SK_I8 = 1, SK_I6 = 2, SK_I4 = 3 };
enum StqMode : int { SM_STEP = 0, SM_PACK = 1, SM_UNPACK = 2 };

struct StqBlock {
  uint32_t o8, o6, o4, orf, ocs, bytes;
  int n16, n8, n6, n4;
  double sw;   // the binary64 sum of w_i^2 over the integer rows
};

template <int D>
__device__ __forceinline__ StqBlock stq_block(const StqArgs& a, int head) {
  const int4 hi = a.heads[head];   // {offset, counts n16 | n8 << 8 | n6 << 16 | n4 << 24, sw (2 words)}
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
  b.bytes = b.ocs + 2 * D;
  b.sw = __hiloint2double(hi.w, hi.z);
  return b;
}

__device__ __forceinline__ int stq_kind(const StqBlock& b, int p) {
  return p < b.n16 ? SK_F16 : (p < b.n16 + b.n8 ? SK_I8 : (p < b.n16 + b.n8 + b.n6 ? SK_I6 : SK_I4));
}

// The lane's row slot, made opaque to the compiler once per row group and phase: without it the
// compiler computes the per-kind addresses and lane masks of every row group once, early, and
// holds them (some 40 VGPRs and many scalar pairs) from the loads to the stores.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The same for a wave-uniform value (the group's first row, from which the kind tests follow).
__device__ __forceinline__ int fresh_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Run f(kind) for the lanes whose row has that kind; k0 / k3 (wave-uniform) are the kinds of the
// wave's first and last row of the group, so kinds outside [k0, k3] cost one scalar compare.
template <int K, typename F>
__device__ __forceinline__ void on_kind(int k0, int k3, int mine, F& f) {
  if (K >= k0 && K <= k3) {
    if (mine == K) f(std::integral_constant<int, K>{});
  }
}

// The row group of storage rows p0 .. p0 + 3 (p0 wave-uniform, p = the lane's row): f(kind) runs
// for each kind in the group, on the lanes whose row has it. A group almost always holds one
// kind; then every lane takes it from the scalar kind of the group, and only a group that
// straddles two kinds forms each lane's own kind (a branch the compiler may not flatten, so the
// per-lane compares are not paid by every group).
template <typename F>
__device__ __forceinline__ void by_kind(const StqBlock& blk, int p0, int p, F&& f) {
  const int k0 = stq_kind(blk, p0), k3 = stq_kind(blk, p0 + 3);
  int mine = k0;
  if (k0 != k3) {
    mine = stq_kind(blk, p);
    asm volatile("" : "+v"(mine));
  }
  on_kind<SK_F16>(k0, k3, mine, f);
  on_kind<SK_I8>(k0, k3, mine, f);
  on_kind<SK_I6>(k0, k3, mine, f);
  on_kind<SK_I4>(k0, k3, mine, f);
}

// Byte offset of the lane's part of storage row p (kind K) in the block; I6: of its nibbles (its
// top bits: stq_top_off).
template <int D, int K>
__device__ __forceinline__ uint32_t stq_off(const StqBlock& b, int p, int cg) {
  constexpr int CPL = D / 16;
  if constexpr (K == SK_F16) return static_cast<uint32_t>(p * 2 * D + cg * 2 * CPL);
  if constexpr (K == SK_I8) return b.o8 + static_cast<uint32_t>((p - b.n16) * D + cg * CPL);
  if constexpr (K == SK_I6)
    return b.o6 + static_cast<uint32_t>((p - b.n16 - b.n8) * (3 * D / 4) + cg * (CPL / 2));
  return b.o4 + static_cast<uint32_t>((p - b.n16 - b.n8 - b.n6) * (D / 2) + cg * (CPL / 2));
}

template <int D>
__device__ __forceinline__ uint32_t stq_top_off(const StqBlock& b, int p, int cg) {
  constexpr int CPL = D / 16;
  return b.o6 + static_cast<uint32_t>((p - b.n16 - b.n8) * (3 * D / 4) + D / 2 + cg * (CPL / 4));
}

// The lane's stored words of row p (kind K): F16 CPL halves, I8 CPL bytes, I6 / I4 CPL nibbles
// in w, and (I6) the CPL top-bit pairs in top.
template <int D, int K>
__device__ __forceinline__ void stq_load(rsrc_t rs, const StqBlock& b, int p, int cg, uint32_t* w,
                                         uint32_t& top) {
  constexpr int CPL = D / 16;
  constexpr int N = K == SK_F16 ? 2 * CPL : (K == SK_I8 ? CPL : CPL / 2);
  buf_load<N>(rs, stq_off<D, K>(b, p, cg), 0u, w);
  if constexpr (K == SK_I6) {
    uint32_t t[1];
    buf_load<CPL / 4>(rs, stq_top_off<D>(b, p, cg), 0u, t);
    top = t[0];
  }
}

// Power of two each row kind's decoded values carry (the row multiplier divides it out
// exactly): 6-bit codes decode as 4 * code and 4-bit codes as 16 * code, the code's sign bit
// moved to bit 7 of a byte so that one signed-byte conversion reads it.
template <int K>
constexpr float kDecodeScale = K == SK_I6 ? 4.0f : (K == SK_I4 ? 16.0f : 1.0f);

// The lane's CPL values of a loaded row, times kDecodeScale<K>: FP16 values widened, codes
// converted from signed bytes.
template <int D, int K>
__device__ __forceinline__ void stq_decode_row(const uint32_t* w, uint32_t top, float* out) {
  constexpr int CPL = D / 16;
  auto sbyte = [](uint32_t x, int k) { return static_cast<float>(static_cast<int8_t>(x >> (8 * k))); };
  if constexpr (K == SK_F16) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = half_bits_to_float(w[c >> 1] >> (16 * (c & 1)));
  } else if constexpr (K == SK_I8) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = sbyte(w[c >> 2], c & 3);
  } else {
    // codes 2k in the bytes of e, codes 2k + 1 in the bytes of o, each at bits 4..7 (I4) or 2..7
    // (I6, the top bits from t: byte k of t = the top-bit pairs of codes 2k and 2k + 1)
    uint32_t e, o;
    if constexpr (K == SK_I4) {
      e = (w[0] << 4) & 0xF0F0F0F0u;
      o = w[0] & 0xF0F0F0F0u;
    } else {
      const uint32_t y = __builtin_amdgcn_perm(0u, top, 0x01010000u);   // bytes t0 t0 t1 t1
      const uint32_t t = (y & 0x000F000Fu) | ((y >> 4) & 0x0F000F00u);
      e = ((w[0] << 2) & 0x3C3C3C3Cu) | ((t << 6) & 0xC0C0C0C0u);
      o = ((w[0] >> 2) & 0x3C3C3C3Cu) | ((t << 4) & 0xC0C0C0C0u);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) out[c] = sbyte((c & 1) ? o : e, c >> 1);
  }
}

// Store the lane's part of row p: F16 from x, else the codes in the low bits of tb (two's
// complement: tb holds 1.5 * 2^23 + code as binary32 bits).
template <int D, int K>
__device__ __forceinline__ void stq_store(rsrc_t rs, const StqBlock& b, int p, int cg, const float* x,
                                          const uint32_t* tb) {
  constexpr int CPL = D / 16;
  const uint32_t off = stq_off<D, K>(b, p, cg);
  if constexpr (K == SK_F16) {
    uint32_t wd[CPL / 2];
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i)
      wd[i] = float_to_half_bits(x[2 * i]) | (float_to_half_bits(x[2 * i + 1]) << 16);
    buf_store<2 * CPL>(rs, off, 0u, wd);
  } else if constexpr (K == SK_I8) {
    uint32_t wd[CPL / 4];
#pragma unroll
    for (int i = 0; i < CPL / 4; ++i) wd[i] = pack4_low_bytes(tb[4 * i], tb[4 * i + 1], tb[4 * i + 2], tb[4 * i + 3]);
    buf_store<CPL>(rs, off, 0u, wd);
  } else {
    uint32_t lo, hi = 0;
    if constexpr (CPL == 8) {
      // even codes in the bytes of e, odd codes in the bytes of o
      const uint32_t e = pack4_low_bytes(tb[0], tb[2], tb[4], tb[6]);
      const uint32_t o = pack4_low_bytes(tb[1], tb[3], tb[5], tb[7]);
      lo = (e & 0x0F0F0F0Fu) | ((o & 0x0F0F0F0Fu) << 4);
      if constexpr (K == SK_I6) {
        // byte k of n: top bits of codes 2k (bits 0-1) and 2k+1 (bits 2-3); then two nibbles a byte
        const uint32_t n = ((e >> 4) & 0x03030303u) | (((o >> 4) & 0x03030303u) << 2);
        hi = __builtin_amdgcn_perm(0u, n | (n >> 4), 0x0c0c0200u);
      }
    } else {
      lo = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        lo |= (tb[c] & 0xFu) << (4 * c);
        hi |= ((tb[c] >> 4) & 0x3u) << (2 * c);
      }
    }
    buf_store<CPL / 2>(rs, off, 0u, &lo);
    if constexpr (K == SK_I6) buf_store<CPL / 4>(rs, stq_top_off<D>(b, p, cg), 0u, &hi);
  }
}

// binary64 -> binary16, one rounding (to nearest, ties to even): round to odd into binary32
// first (keep the truncation, set the last bit when inexact), then v_cvt_f16_f32. Binary32 has
// more than two bits beyond binary16's significand over binary16's whole range, so the odd
// intermediate never creates or hides a tie.
__device__ __forceinline__ uint32_t f16_from_f64(double d) {
  float f = static_cast<float>(d);   // to nearest
  const double back = static_cast<double>(f);
  if (back != d) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(d)) u -= 1u;   // rounded away from zero: one step back toward zero
    f = __uint_as_float(u | 1u);
  }
  return float_to_half_bits(f);
}

// m / qmax correctly rounded: one multiply by RN(1 / qmax) and one residual correction (checked
// against IEEE division for every binary32 significand at exponents 2^-120 .. 2^127 for qmax in
// {7, 31, 127}).
__device__ __forceinline__ float div_qmax(float m, float qm, float inv) {
  const float q = m * inv;
  const float r = fmaf(-q, qm, m);
  return fmaf(r, inv, q);
}

template <int D, int NW>
struct StqSmem {
  float4 srow[D];            // {gate_p, k_p, q_p, rf_p (1 for pivots)}, storage order
  float sw1[D];              // w_p (0 for pivots), storage order
  float sv[D];               // v, then delta
  union {
    float red[2][4 * NW][D];   // partial sums: u and p
    double red64[4 * NW][D];   // then the column-scale sums (binary64)
  };
  float redqk[NW];
  float scs[D];              // column scales (binary16 values as fp32)
  float srcs[D];             // RN(1 / cs_j), 0 where cs_j = 0
  uint16_t srf[D];           // the new row factors (binary16 bits), integer-row order
};

// The step's per-row scalars in two halves, so that their loads overlap the state loads while
// the state is decoded in between: stq_stage_load issues the loads (k, q, the gate, v, the row
// map, the fit's row weights and the stored row factors, one element per thread),
// stq_stage_store writes them to LDS in storage order (srow = {gate_p, k_p, q_p, rf_p / scale_p}
// with rf = 1 for pivots and scale_p the row kind's decode scale, sv = v, sw1) and returns beta.
template <int D, int NT>
struct StqStage {
  static constexpr int PER = (D + NT - 1) / NT;
  int src[PER];
  float kv[PER], qv[PER], gv[PER], vv[PER], w1[PER];
  uint32_t rf[PER];
  float g0, beta;
};

template <int D, int NT, int PER_KEY, int BF16>
__device__ __forceinline__ StqStage<D, NT> stq_stage_load(const StqArgs& a, rsrc_t blk_rs, const StqBlock& blk,
                                                          int bh, int head, int tid) {
  StqStage<D, NT> st;
  const int64_t vec = int64_t(bh) * D;
#pragma unroll
  for (int n = 0; n < StqStage<D, NT>::PER; ++n) {
    const int i = tid + n * NT;
    if (i < D) {
      st.src[n] = a.rowmap[head * D + i];
      st.kv[n] = load_in<BF16>(a.step.k, vec + i);
      st.qv[n] = load_in<BF16>(a.step.q, vec + i);
      st.gv[n] = PER_KEY ? a.step.alpha[vec + i] : 0.0f;
      st.vv[n] = load_in<BF16>(a.step.v, vec + i);
      st.w1[n] = a.w1[head * D + i];
      const int ri = i - blk.n16;
      st.rf[n] = 0x3C00u;   // 1.0 for pivots
      if (ri >= 0) buf_load<2>(blk_rs, blk.orf + 2u * static_cast<uint32_t>(ri), 0u, &st.rf[n]);
    }
  }
  st.g0 = PER_KEY ? 0.0f : a.step.alpha[bh];
  st.beta = a.step.beta[bh];
  return st;
}

template <int D, int NT, int PER_KEY>
__device__ __forceinline__ float stq_stage_store(const StqStage<D, NT>& st, const StqBlock& blk, int tid,
                                                 float4* srow, float* sv,
                                                 float* sw1, float* tmp) {
#pragma unroll
  for (int n = 0; n < StqStage<D, NT>::PER; ++n) {
    const int i = tid + n * NT;
    if (i < D) {
      tmp[i] = st.kv[n];
      tmp[D + i] = st.qv[n];
      if constexpr (PER_KEY) tmp[2 * D + i] = st.gv[n];
      sv[i] = st.vv[n];
      sw1[i] = st.w1[n];
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < StqStage<D, NT>::PER; ++n) {
    const int i = tid + n * NT;
    if (i < D) {
      const int j = st.src[n];
      const int kind = stq_kind(blk, i);   // exact: a power-of-two division of a binary16 value
      const float rfs = half_bits_to_float(st.rf[n]) *
                        (kind == SK_I6 ? 1.0f / kDecodeScale<SK_I6> : (kind == SK_I4 ? 1.0f / kDecodeScale<SK_I4> : 1.0f));
      srow[i] = make_float4(PER_KEY ? tmp[2 * D + j] : st.g0, tmp[j], tmp[D + j], rfs);
    }
  }
  __syncthreads();
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st.beta)));
}

// MODE = SM_STEP: one decode step (reads src, writes dst). SM_PACK: fp32 states (key order) ->
// format. SM_UNPACK: format -> fp32 states (key order).
// At least four waves per SIMD (<= 128 VGPRs): the step holds X (64 VGPRs at d = 128) and
// is bound by how many units are in flight per CU; the allocator meets this without spilling.
template <int D, int NW, int PER_KEY, int BF16, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) void stq_kernel(const StqArgs a) {
  using G = Geo<D, NW>;
  constexpr int CPL = G::CPL, RPL = G::RPL, RPS = G::RPS, NT = G::NT;
  constexpr bool EXACT = MODE == SM_PACK;
  constexpr float kMagic = 0x1.8p23f;
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
  const rsrc_t src = make_rsrc(a.pool + boff, blk.bytes);
  const rsrc_t dst = make_rsrc((a.dst ? a.dst : a.pool) + boff, blk.bytes);
  if (!slot_in_pool(slot, a.num_slots)) return;   // before any access through src or dst
  const uint8_t* rowmap = a.rowmap + head * D;

  float X[RPL][CPL];
  if constexpr (MODE == SM_PACK) {
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int p = t * RPS + w * 4 + rs;
      load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(a.S + (int64_t(bh) * D + rowmap[p]) * D + cg * CPL),
                          reinterpret_cast<uint32_t*>(X[t]));
    }
    for (int i = tid; i < D; i += NT) sm.sw1[i] = a.w1[head * D + i];
    __syncthreads();
  } else {
    // (1) the stored state: the lane's words of each row, its row factor, its column scales
    uint32_t raw[RPL][CPL / 2];
    uint32_t top[RPL];
    float rfv[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
      const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
      top[t] = 0;
      by_kind(blk, p0, p, [&](auto KC) { stq_load<D, decltype(KC)::value>(src, blk, p, cg, raw[t], top[t]); });
      if constexpr (MODE == SM_UNPACK) {
        const int ri = p - blk.n16;
        uint32_t rb[1];
        buf_load<2>(src, blk.orf + 2u * static_cast<uint32_t>(ri < 0 ? 0 : ri), 0u, rb);
        rfv[t] = ri < 0 ? 1.0f : half_bits_to_float(rb[0]);
      }
    }
    float csv[CPL];
    {
      uint32_t cw[CPL / 2];
      buf_load<2 * CPL>(src, blk.ocs + 2u * cg * CPL, 0u, cw);
#pragma unroll
      for (int c = 0; c < CPL; ++c) csv[c] = half_bits_to_float(cw[c >> 1] >> (16 * (c & 1)));
    }
    if constexpr (MODE == SM_UNPACK) {
      // code * (rf * cs): rf * cs is exact in binary32, so one rounding, as the definition
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
        by_kind(blk, p0, p, [&](auto KC) {
          constexpr int K = decltype(KC)::value;
          stq_decode_row<D, K>(raw[t], top[t], X[t]);
          if constexpr (K != SK_F16) {
            const float rs_ = rfv[t] * (1.0f / kDecodeScale<K>);   // exact
#pragma unroll
            for (int c = 0; c < CPL; ++c) X[t][c] *= rs_ * csv[c];
          }
        });
        store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(a.S + (int64_t(bh) * D + rowmap[p]) * D + cg * CPL),
                             reinterpret_cast<const uint32_t*>(X[t]));
      }
      return;
    } else {
      // (2) the per-row scalars' loads go out; meanwhile the state is decoded as it arrives:
      // X = code * cs_j (integer rows) or the FP16 value, and the stored words are dropped
      const StqStage<D, NT> stage = stq_stage_load<D, NT, PER_KEY, BF16>(a, src, blk, bh, head, tid);
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
        by_kind(blk, p0, p, [&](auto KC) {
          constexpr int K = decltype(KC)::value;
          stq_decode_row<D, K>(raw[t], top[t], X[t]);
          if constexpr (K != SK_F16) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) X[t][c] *= csv[c];
          }
        });
      }
      const float beta = stq_stage_store<D, NT, PER_KEY>(stage, blk, tid, sm.srow, sm.sv, sm.sw1, &sm.red[0][0][0]);
      // (3) S' = diag(gate) S_hat (row multiplier gate_p * rf_p), and the partial column sums of
      // u = S'^T k and p = S'^T q
      float pu[CPL], pp[CPL], pqk = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) pu[c] = pp[c] = 0.0f;
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const float4 rw = sm.srow[t * RPS + w * 4 + rs];
        const float m = rw.x * rw.w;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          X[t][c] *= m;
          pu[c] = fmaf(rw.y, X[t][c], pu[c]);
          pp[c] = fmaf(rw.z, X[t][c], pp[c]);
        }
        pqk = fmaf(rw.z, rw.y, pqk);
      }
      finish_columns<D, G>(sm.red[0], sm.red[1], sm.redqk, sm.sv, pu, pp, pqk, beta,
                           a.step.out + int64_t(bh) * D, tid, w, rs, lane, cg);
      // (4) X = S' + k delta^T
      float dl[CPL];
      load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.sv + cg * CPL), reinterpret_cast<uint32_t*>(dl));
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const float kp = sm.srow[t * RPS + w * 4 + rs].y;
#pragma unroll
        for (int c = 0; c < CPL; ++c) X[t][c] = fmaf(kp, dl[c], X[t][c]);
      }
    }
  }

  // (5) the fit: column scales from the weighted column sums of squares. Each lane sums its rows'
  // (w_i X_ij)^2 in order; the column thread adds the lanes' partials in binary64. Pack forms
  // the lane sums in binary64 too (each w_i X_ij exact, each square-and-add rounded once). The
  // step forms them in binary32 (w_i X_ij rounded, then one fma per row): for RPL positive
  // terms that is within (RPL + 2) u of the exact sum (u = 2^-24), so the column scale before
  // its binary16 rounding is within (RPL + 2) u / 2 = 5u (d = 128) of the binary64 fit of the
  // same X, and the two can differ only where that value lies so close to a binary16 tie.
  {
    double acc[CPL];
    if constexpr (EXACT) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = 0.0;
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const double w1 = sm.sw1[t * RPS + w * 4 + rs];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const double y = w1 * static_cast<double>(X[t][c]);   // exact: two 24-bit significands
          acc[c] = fma(y, y, acc[c]);
        }
      }
    } else {
      float accf[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) accf[c] = 0.0f;
#pragma unroll
      for (int t = 0; t < RPL; ++t) {
        const float w1 = sm.sw1[t * RPS + w * 4 + rs];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float y = w1 * X[t][c];
          accf[c] = fmaf(y, y, accf[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = static_cast<double>(accf[c]);
    }
    store_bytes<CPL * 8>(reinterpret_cast<uint8_t*>(&sm.red64[w * 4 + rs][cg * CPL]),
                         reinterpret_cast<const uint32_t*>(acc));
  }
  __syncthreads();
  for (int j = tid; j < D; j += NT) {
    double s = sm.red64[0][j];
#pragma unroll
    for (int k = 1; k < 4 * NW; ++k) s += sm.red64[k][j];
    const uint32_t hb = blk.sw > 0.0 ? f16_from_f64(sqrt(s / blk.sw)) : 0u;
    const float cs = half_bits_to_float(hb);
    sm.scs[j] = cs;
    sm.srcs[j] = cs > 0.0f ? __fdiv_rn(1.0f, cs) : 0.0f;
    buf_store<2>(dst, blk.ocs + 2u * j, 0u, &hb);
  }
  __syncthreads();
  float rcs[CPL], csx[CPL];
  load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.srcs + cg * CPL), reinterpret_cast<uint32_t*>(rcs));
  if constexpr (EXACT)
    load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.scs + cg * CPL), reinterpret_cast<uint32_t*>(csx));

  // (6) per row: row factor, codes, store, with the row kind (and so qmax) known at compile time
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
    by_kind(blk, p0, p, [&](auto KC) {
      constexpr int K = decltype(KC)::value;
      uint32_t tb[CPL];
      if constexpr (K != SK_F16) {
        constexpr float qm = K == SK_I8 ? 127.0f : (K == SK_I6 ? 31.0f : 7.0f);
        constexpr float inv = 1.0f / qm;
        float av[CPL];
        float mq = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if constexpr (EXACT) {
            const float ax = fabsf(X[t][c]);
            const float q = ax * rcs[c];
            mq = fmaxf(mq, fmaf(fmaf(-q, csx[c], ax), rcs[c], q));   // = fl(|x| / cs) (0 if cs = 0)
          } else {
            av[c] = X[t][c] * rcs[c];
            mq = fmaxf(mq, fabsf(av[c]));
          }
        }
        const float m = max_row16(mq);
        const uint32_t rb = float_to_half_bits(div_qmax(m, qm, inv));
        const float rf = half_bits_to_float(rb);
        if (cg == 0) sm.srf[p - blk.n16] = static_cast<uint16_t>(rb);
        if constexpr (EXACT) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float sc = rf * csx[c];   // exact: two binary16 significands
            float n = sc > 0.0f ? rintf(__fdiv_rn(X[t][c], sc)) : 0.0f;
            n = fminf(fmaxf(n, -qm), qm);
            tb[c] = __float_as_uint(n + kMagic);
          }
        } else {
          const float rrf = rf > 0.0f ? __builtin_amdgcn_rcpf(rf) : 0.0f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) tb[c] = __float_as_uint(fmaf(av[c], rrf, kMagic));
          if (__any(rf < 0x1p-14f)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
              tb[c] = __float_as_uint(__builtin_amdgcn_fmed3f(__uint_as_float(tb[c]), kMagic - qm, kMagic + qm));
          }
        }
      }
      stq_store<D, K>(dst, blk, p, cg, X[t], tb);
    });
  }
  // the row factors, gathered in LDS, go out as one contiguous run (scattered 2-byte stores by
  // one lane per row reached HBM as partial lines)
  __syncthreads();
  const int nint = D - blk.n16;
  for (int i = 2 * tid; i < nint; i += 2 * NT) {
    const uint32_t two = sm.srf[i] | (i + 1 < nint ? static_cast<uint32_t>(sm.srf[i + 1]) << 16 : 0u);
    if (i + 1 < nint)
      buf_store<4>(dst, blk.orf + 2u * static_cast<uint32_t>(i), 0u, &two);
    else
      buf_store<2>(dst, blk.orf + 2u * static_cast<uint32_t>(i), 0u, &two);
  }
}

template <int D, int NW, int MODE>
hipError_t stq_launch_mode(int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H)), block(NW * 64);
  if constexpr (MODE != SM_STEP) {
    hipLaunchKernelGGL((stq_kernel<D, NW, 0, 0, MODE>), grid, block, 0, s, a);
  } else if (per_key) {
    if (bf16) hipLaunchKernelGGL((stq_kernel<D, NW, 1, 1, MODE>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stq_kernel<D, NW, 1, 0, MODE>), grid, block, 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((stq_kernel<D, NW, 0, 1, MODE>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stq_kernel<D, NW, 0, 0, MODE>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// Waves per unit: four at d = 128 (each lane holds 8 rows x 8 columns of X), two at d = 64.
template <int D>
constexpr int kStqWaves = D >= 128 ? 4 : 2;

template <int D>
hipError_t stq_d(int mode, int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  constexpr int NW = kStqWaves<D>;
  if (mode == SM_STEP) return stq_launch_mode<D, NW, SM_STEP>(per_key, bf16, a, s);
  if (mode == SM_PACK) return stq_launch_mode<D, NW, SM_PACK>(per_key, bf16, a, s);
  return stq_launch_mode<D, NW, SM_UNPACK>(per_key, bf16, a, s);
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
