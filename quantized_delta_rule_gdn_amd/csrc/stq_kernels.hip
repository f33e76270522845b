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
// Each region after the pivots starts at the next multiple of 128 bytes, and the 6- and 4-bit
// regions at the 4-row group of their first storage row (never-touched padding): the 4 rows a
// wave stores together then cover whole 128-byte lines.
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
#include <cstdlib>
#include <type_traits>

#include "step_common.h"

namespace damp {
namespace {

enum StqKind : int { SK_F16 = 0, SK_I8 = 1, SK_I6 = 2, SK_I4 = 3 };
enum StqMode : int { SM_STEP = 0, SM_PACK = 1, SM_UNPACK = 2 };

struct StqBlock {
  uint32_t o8, o6, o4, orf, ocs, bytes;
  int n16, n8, n6, n4;
  int f6, f4;  // the storage row at the start of the 6- / 4-bit region (first row rounded down to 4)
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
  // every region starts on a 128-byte line, so no line holds two regions (a store never writes
  // part of a line another store completes)
  // and the 6- and 4-bit regions begin at the row group (4 storage rows) of their first row, so
  // that the 4 rows a wave stores together cover whole lines (4 x 3d/4 and 4 x d/2 bytes)
  auto up = [](uint32_t x) { return (x + 127u) & ~127u; };
  const int b2 = b.n16 + b.n8, b3 = b2 + b.n6;
  b.f6 = b2 & ~3;
  b.f4 = b3 & ~3;
  b.o8 = up(2u * D * b.n16);
  b.o6 = up(b.o8 + D * b.n8);
  b.o4 = up(b.o6 + (3 * D / 4) * (b.n6 > 0 ? b.n6 + (b2 & 3) : 0));
  b.orf = up(b.o4 + (D / 2) * (b.n4 > 0 ? b.n4 + (b3 & 3) : 0));
  b.ocs = up(b.orf + 2 * (D - b.n16));
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

// r 6-bit rows of 3 d / 4 bytes, as two shifts and an add (no quarter-rate integer multiply).
template <int D>
__device__ __forceinline__ int i6_row_bytes(int r) {
  return r * (D / 2) + r * (D / 4);
}

// Byte offset of the lane's part of storage row p (kind K) in the block; I6: of its nibbles (its
// top bits: stq_top_off).
template <int D, int K>
__device__ __forceinline__ uint32_t stq_off(const StqBlock& b, int p, int cg) {
  constexpr int CPL = D / 16;
  if constexpr (K == SK_F16) return static_cast<uint32_t>(p * 2 * D + cg * 2 * CPL);
  if constexpr (K == SK_I8) return b.o8 + static_cast<uint32_t>((p - b.n16) * D + cg * CPL);
  if constexpr (K == SK_I6)
    return b.o6 + static_cast<uint32_t>(i6_row_bytes<D>(p - b.f6) + cg * (CPL / 2));
  return b.o4 + static_cast<uint32_t>((p - b.f4) * (D / 2) + cg * (CPL / 2));
}

template <int D>
__device__ __forceinline__ uint32_t stq_top_off(const StqBlock& b, int p, int cg) {
  constexpr int CPL = D / 16;
  return b.o6 + static_cast<uint32_t>(i6_row_bytes<D>(p - b.f6) + D / 2 + cg * (CPL / 4));
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

// ---- the decode step at d = 128 with the codes held ------------------------------------------
// The kernel above holds the whole fp32 X of a unit (64 VGPRs per lane at d = 128), so a CU fits
// four units, and issues ~21 VALU instructions per state element. This one keeps each row's
// codes as they were stored (2 words per lane and row, FP16 pivot rows 4) until the update is
// known, and takes the two column sums of Table C2 step 2 on the matrix cores:
//  - Projections. For an integer row, S'_ij = gate_i rf_i cs_j c_ij, so
//    u_j = cs_j sum_i z_i c_ij + (pivot rows) with z_i = gate_i rf_i k_i (q_i for p). The codes
//    are exact int8 (6- and 4-bit codes as 4 c and 16 c, their factor in rf); each wave splits
//    its 32 rows' z into four int8 pieces of 7 bits below a per-wave power of two (z = 2^-S
//    (P0 + P1 2^-7 + P2 2^-14 + P3 2^-21) + e, |e| <= 2^-27 max|z|), so one v_mfma_i32_16x16x64_i8
//    per pair of columns gives exact integer sums of pieces times codes for both k and q; the
//    lanes then recombine the pieces (three roundings) and scale by 2^-S cs_j. Pivot rows are
//    summed on the VALU.
//  - The update in the old column scale's units: Y_ij = X_ij / g_j = gate_i rf_i c_ij +
//    k_i delta_j / g_j, with g_j = cs_j (1 where cs_j = 0; the codes of such a column are
//    masked to zero, which is what they reconstruct to). Pivot rows hold X_ij itself.
//  - The fit reads Y: sum_i (w_i Y_ij)^2 in binary32 per lane, the column thread adds the
//    partials in binary64 and multiplies by g_j^2 (exact); a row's maximum and codes use
//    a_ij = Y_ij * RN(g_j / cs'_j), the quotient X_ij / cs'_j up to a few binary32 ulps.
// Y is recomputed from the held codes for the codes (3 VALU instructions per element) rather than
// kept: holding it takes 64 more VGPRs, four units per CU instead of six, and measured slower
// (392 against 352 us on the pool of 1,024 active slots x 32 heads).
// NP: row steps that may hold pivot rows (the host picks NP >= ceil(max pivots per head / 16)).
typedef int stq_v4i __attribute__((ext_vector_type(4)));

template <int NW>
struct Stq2Smem {
  static constexpr int HZ = 128 / (4 * NW) / 8;   // halves of 8 row steps per lane
  float4 srow[128];   // {gate_p, k_p, q_p, rf_p / scale_p}, storage order
  float sw1[128];     // w_p (0 for pivots)
  float sv[128];      // v, then delta
  float sd[128];      // delta / g_j
  union {
    float red[2][NW][128];      // u and p: one partial per wave
    float red2[4 * NW][128];    // the fit's lane partials (binary32), one per wave and row slot
    float tmp[3 * 128];         // the staging's permutation to storage order
  };
  uint8_t apc[NW][2][4][HZ][32];   // pieces of z: [wave][k | q][piece][half][g * 8 + t]
  float redqk[NW];
  float sratio[128];  // g_j / cs'_j, 0 where cs'_j = 0
  uint16_t srf[128];  // the new row factors (binary16 bits), integer-row order
};

// Row-kind dispatch for the codes-held step: a row group of one kind (nearly all of them) takes
// a scalar branch on that kind, with no per-lane compare or exec-mask change; only a group that
// straddles two kinds forms each lane's kind and runs the kinds under exec masks. F16OK = false
// for row steps that cannot hold pivot rows.
template <bool F16OK, typename F>
__device__ __forceinline__ void by_kind2(const StqBlock& blk, int p0, int p, F&& f) {
  const int k0 = stq_kind(blk, p0), k3 = stq_kind(blk, p0 + 3);
  if (k0 == k3) {
    if (F16OK && k0 == SK_F16) {
      if constexpr (F16OK) f(std::integral_constant<int, SK_F16>{});
    } else if (k0 == SK_I8) {
      f(std::integral_constant<int, SK_I8>{});
    } else if (k0 == SK_I6) {
      f(std::integral_constant<int, SK_I6>{});
    } else {
      f(std::integral_constant<int, SK_I4>{});
    }
  } else {
    int mine = stq_kind(blk, p);
    asm volatile("" : "+v"(mine));
    if constexpr (F16OK) on_kind<SK_F16>(k0, k3, mine, f);
    on_kind<SK_I8>(k0, k3, mine, f);
    on_kind<SK_I6>(k0, k3, mine, f);
    on_kind<SK_I4>(k0, k3, mine, f);
  }
}

// Where the lane's words of storage row p lie in the block, for a row of kind k: off = the
// codes (pivot rows: the halves; 6-bit rows: the nibbles), offt = the 6-bit top bits.
template <int D>
__device__ __forceinline__ void stq_row_at(const StqBlock& b, int k, int p, int cg, uint32_t& off, uint32_t& offt) {
  constexpr int CPL = D / 16;
  const int b1 = b.n16, b2 = b1 + b.n8, b3 = b2 + b.n6;
  const uint32_t base = k == SK_F16 ? 0u : (k == SK_I8 ? b.o8 : (k == SK_I6 ? b.o6 : b.o4));
  const int first = k == SK_F16 ? 0 : (k == SK_I8 ? b1 : (k == SK_I6 ? b.f6 : b.f4));
  const int stride = k == SK_F16 ? 2 * D : (k == SK_I8 ? D : (k == SK_I6 ? 3 * D / 4 : D / 2));
  const int lw = k == SK_F16 ? 2 * CPL : (k == SK_I8 ? CPL : CPL / 2);
  // 24-bit products: full-rate v_mad_u32_u24 (the row index and the stride are small and
  // non-negative for the lane's own kind; offt is used only by 6-bit rows)
  off = base + __umul24(static_cast<uint32_t>(p - first), static_cast<uint32_t>(stride)) + static_cast<uint32_t>(cg * lw);
  offt = b.o6 + static_cast<uint32_t>(i6_row_bytes<D>(p - b.f6) + D / 2 + cg * (CPL / 4));
}

// The step's per-row scalars for the codes-held kernel (d = 128, 256 threads): every thread
// issues the same loads (thread i and i + 128 the same row), none of them under a branch, before
// the state loads; the raw words stay opaque until store(), so no wait for them lands between
// the state loads. store() writes srow / sv / sw1 in storage order (two barriers) and returns
// beta in a scalar register.
template <int PER_KEY, int BF16>
struct Stq2Stage {
  static constexpr int D = 128;
  uint32_t src, kv, qv, gv, vv, w1, rf, csj;
  float g0, beta;

  __device__ __forceinline__ void load(const StqArgs& a, rsrc_t rs, const StqBlock& blk, int bh, int head,
                                       int tid) {
    const int i = tid & (D - 1);
    const int64_t vec = int64_t(bh) * D;
    auto raw = [](const void* base, int64_t j) -> uint32_t {
      if constexpr (BF16) return reinterpret_cast<const uint16_t*>(base)[j];
      else return reinterpret_cast<const uint32_t*>(base)[j];
    };
    src = a.rowmap[head * D + i];
    kv = raw(a.step.k, vec + i);
    qv = raw(a.step.q, vec + i);
    gv = PER_KEY ? reinterpret_cast<const uint32_t*>(a.step.alpha)[vec + i] : 0u;
    vv = raw(a.step.v, vec + i);
    w1 = __float_as_uint(a.w1[head * D + i]);
    const int ri = i - blk.n16;
    buf_load<2>(rs, blk.orf + 2u * static_cast<uint32_t>(ri < 0 ? 0 : ri), 0u, &rf);
    buf_load<2>(rs, blk.ocs + 2u * static_cast<uint32_t>(i), 0u, &csj);
    g0 = PER_KEY ? 0.0f : a.step.alpha[bh];
    beta = a.step.beta[bh];
  }

  __device__ __forceinline__ void fence() {
    asm volatile("" : "+v"(src), "+v"(kv), "+v"(qv), "+v"(gv), "+v"(vv), "+v"(w1), "+v"(rf), "+v"(csj));
  }

  __device__ __forceinline__ float store(const StqBlock& blk, int tid, float4* srow, float* sv, float* sw1,
                                         float* tmp) {
    fence();
    auto widen = [](uint32_t w) { return BF16 ? __uint_as_float(w << 16) : __uint_as_float(w); };
    if (tid < D) {
      tmp[tid] = widen(kv);
      tmp[D + tid] = widen(qv);
      if constexpr (PER_KEY) tmp[2 * D + tid] = __uint_as_float(gv);
      sv[tid] = widen(vv);
      sw1[tid] = __uint_as_float(w1);
    }
    __syncthreads();
    if (tid < D) {
      const int j = static_cast<int>(src);
      const int kind = stq_kind(blk, tid);   // exact: a power-of-two division of a binary16 value
      const float rfs = tid < blk.n16 ? 1.0f
                                      : half_bits_to_float(rf) *
                                            (kind == SK_I6 ? 1.0f / kDecodeScale<SK_I6>
                                                           : (kind == SK_I4 ? 1.0f / kDecodeScale<SK_I4> : 1.0f));
      srow[tid] = make_float4(PER_KEY ? tmp[2 * D + j] : g0, tmp[j], tmp[D + j], rfs);
    }
    __syncthreads();
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(beta)));
  }
};

// Signed byte k of x as a float (v_cvt_f32_i32 with a sign-extended byte select).
__device__ __forceinline__ float sbyte_f(uint32_t x, int k) {
  return static_cast<float>(static_cast<int8_t>(x >> (8 * k)));
}

// Canonical code words of a row: E holds the codes of the lane's even columns 0, 2, 4, 6 in
// bytes 0..3, O those of the odd columns (6- and 4-bit codes as 4 c and 16 c).
template <int K>
__device__ __forceinline__ void stq_canon(uint32_t* w, uint32_t top) {
  if constexpr (K == SK_I8) {
    const uint32_t e = __builtin_amdgcn_perm(w[1], w[0], 0x06040200u);
    const uint32_t o = __builtin_amdgcn_perm(w[1], w[0], 0x07050301u);
    w[0] = e;
    w[1] = o;
  } else if constexpr (K == SK_I4) {
    const uint32_t x = w[0];
    w[0] = (x << 4) & 0xF0F0F0F0u;
    w[1] = x & 0xF0F0F0F0u;
  } else if constexpr (K == SK_I6) {
    const uint32_t x = w[0];
    const uint32_t y = __builtin_amdgcn_perm(0u, top, 0x01010000u);   // bytes t0 t0 t1 t1
    const uint32_t t = (y & 0x000F000Fu) | ((y >> 4) & 0x0F000F00u);
    w[0] = ((x << 2) & 0x3C3C3C3Cu) | ((t << 6) & 0xC0C0C0C0u);
    w[1] = ((x >> 2) & 0x3C3C3C3Cu) | ((t << 4) & 0xC0C0C0C0u);
  }
}

// The first of the two lane columns MFMA i reads (the second is 2 further): E bytes 0, 1 are
// columns 0, 2; E bytes 2, 3 columns 4, 6; O bytes 0, 1 columns 1, 3; O bytes 2, 3 columns 5, 7.
__device__ constexpr int kColOfMfma[4] = {0, 4, 1, 5};

template <int PER_KEY, int BF16, int NP, int NW>
__global__ __launch_bounds__(64 * NW) void stq_step2_kernel(const StqArgs a) {
  constexpr int D = 128, NT = 64 * NW, CPL = 8, RPS = 4 * NW, RPL = D / RPS;
  constexpr int HZ = RPL / 8;   // halves of 8 row steps: one MFMA K-block each
  static_assert(RPL % 8 == 0, "8 or 16 row steps per lane");
  constexpr float kMagic = 0x1.8p23f;
  __shared__ Stq2Smem<NW> sm;
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

  // (1) the per-row scalars' loads, then the stored state: each row step's words (pivot rows:
  // 4 words of halves) and the lane's 8 old column scales
  Stq2Stage<PER_KEY, BF16> stage;
  stage.load(a, src, blk, bh, head, tid);
  uint32_t csw[CPL / 2];   // before the state loads: the in-order counter then lets its wait pass them
  buf_load<2 * CPL>(src, blk.ocs + 2u * cg * CPL, 0u, csw);
  uint32_t cw[RPL][4];
  uint32_t top[RPL];
  // The loads are the same instructions for every kind: no load sits in a branch (the
  // compiler would then wait for each row step's loads at the branches' join). Each reads
  // exactly the bytes of its kind, and a lane whose row does not need it gets an offset past
  // the block (the buffer's range check returns 0 without a memory access), so no line is
  // fetched twice: 4 bytes at the row (every kind), 4 more (8-bit and pivot rows), 8 more
  // (pivot rows, only in row steps that may hold them) and the 2 bytes of a 6-bit row's top
  // bits. For a group of one kind the offsets are a scalar row base plus the lane's part for
  // that kind (precomputed); a group that straddles two kinds forms them per lane.
  constexpr uint32_t kOut = 0x80000000u;   // past any block: no access
  const int b2 = blk.n16 + blk.n8;
  uint32_t lp[4];   // the lane's byte offset within a row group of each kind: rs rows + cg parts
  lp[SK_F16] = __umul24(rs, 2 * D) + cg * (2 * CPL);
  lp[SK_I8] = __umul24(rs, D) + cg * CPL;
  lp[SK_I6] = __umul24(rs, 3 * D / 4) + cg * (CPL / 2);
  lp[SK_I4] = __umul24(rs, D / 2) + cg * (CPL / 2);
  const uint32_t lpt = __umul24(rs, 3 * D / 4) + D / 2 + cg * (CPL / 4);
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
    const int k0 = stq_kind(blk, p0), k3 = stq_kind(blk, p0 + 3);
    const uint32_t sT = blk.o6 + static_cast<uint32_t>((p0 - blk.f6) * (3 * D / 4));
    uint32_t off, off4, off8 = kOut, offt;   // 4 bytes at off (all), 4 at off4, 8 at off8, 2 at offt
    if (k0 == k3) {
      // a scalar branch per kind; the empty volatile statements keep the compiler from turning
      // them into per-lane selects
      if (k0 == SK_F16) {
        asm volatile("");
        off = static_cast<uint32_t>(p0 * 2 * D) + lp[SK_F16];
        off4 = off + 4u;
        off8 = off + 8u;
        offt = kOut;
      } else if (k0 == SK_I8) {
        asm volatile("");
        off = blk.o8 + static_cast<uint32_t>((p0 - blk.n16) * D) + lp[SK_I8];
        off4 = off + 4u;
        offt = kOut;
      } else if (k0 == SK_I6) {
        asm volatile("");
        off = sT + lp[SK_I6];
        off4 = kOut;
        offt = sT + lpt;
      } else {
        asm volatile("");
        off = blk.o4 + static_cast<uint32_t>((p0 - blk.f4) * (D / 2)) + lp[SK_I4];
        off4 = kOut;
        offt = kOut;
      }
    } else {
      int mine = stq_kind(blk, p);
      asm volatile("" : "+v"(mine));
      uint32_t ot;
      stq_row_at<D>(blk, mine, p, cg, off, ot);
      off4 = mine == SK_F16 || mine == SK_I8 ? off + 4u : kOut;
      off8 = mine == SK_F16 ? off + 8u : kOut;
      offt = mine == SK_I6 ? ot : kOut;
    }
    buf_load<4>(src, off, 0u, &cw[t][0]);
    buf_load<4>(src, off4, 0u, &cw[t][1]);
    if (t < NP) {
      buf_load<8>(src, off8, 0u, &cw[t][2]);
    } else {
      cw[t][2] = cw[t][3] = 0u;
    }
    buf_load<2>(src, offt, 0u, &top[t]);
  }

  // (2) the codes put in canonical form as they arrive
  float csf[CPL];
  uint32_t mE = 0u, mO = 0u;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    csf[c] = half_bits_to_float(csw[c >> 1] >> (16 * (c & 1)));
    const uint32_t nz = csf[c] > 0.0f ? 0xFFu : 0u;
    if (c & 1) mO |= nz << (8 * (c >> 1));
    else mE |= nz << (8 * (c >> 1));
  }
  const bool zero_cols = __any((mE & mO) != 0xFFFFFFFFu);   // wave-uniform
  float cso[4];   // the old scales of the columns this lane's MFMA outputs land in
#pragma unroll
  for (int i = 0; i < 4; ++i) cso[i] = (rs & 1) ? csf[kColOfMfma[i] + 2] : csf[kColOfMfma[i]];
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
    auto canon = [&](auto KC) {
      constexpr int K = decltype(KC)::value;
      if constexpr (K != SK_F16) {
        stq_canon<K>(cw[t], top[t]);
        if (zero_cols) {
          cw[t][0] &= mE;
          cw[t][1] &= mO;
        }
      }
    };
    if (t < NP) by_kind2<true>(blk, p0, p, canon);
    else by_kind2<false>(blk, p0, p, canon);
  }
  const uint32_t csj = stage.csj;
  const float beta = stage.store(blk, tid, sm.srow, sm.sv, sm.sw1, sm.tmp);

  // (3) the projection weights of this wave's rows (32 per half of 8 row steps) in int8 pieces:
  // lane (k | q, j) takes row (8 h + j / 4) RPS + 4 w + j % 4 of each half h; S = the wave's power
  // of two for its k or q weights
  const int kq = lane >> 5;
  int S;
  {
    const int j = lane & 31, tz = j >> 2, gz = j & 3;
    float z[HZ], qk = 0.0f, zm = 0.0f;
#pragma unroll
    for (int h = 0; h < HZ; ++h) {
      const int row = (tz + 8 * h) * RPS + w * 4 + gz;
      const float4 r4 = sm.srow[row];
      z[h] = row < blk.n16 ? 0.0f : r4.x * r4.w * (kq ? r4.z : r4.y);
      qk = fmaf(r4.y, r4.z, qk);
      zm = fmaxf(zm, fabsf(z[h]));
    }
    // q.k over the wave's rows (each 32-lane half holds all of them)
    qk = sum_row16(qk);
    {
      const uint32_t u = __float_as_uint(qk);
      const auto sw2 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      qk = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
    }
    if (lane == 0) sm.redqk[w] = qk;
    zm = max_row16(zm);
    {
      const uint32_t u = __float_as_uint(zm);
      const auto sw2 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      zm = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1]));
    }
    S = zm > 0.0f ? 6 - __builtin_amdgcn_frexp_expf(zm) : 0;   // |z| 2^S < 64
#pragma unroll
    for (int h = 0; h < HZ; ++h) {
      float r = ldexpf(z[h], S);
      uint32_t pc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float pk = rintf(r);
        pc[k] = static_cast<uint32_t>(static_cast<int32_t>(pk)) & 0xFFu;
        r = (r - pk) * 128.0f;   // exact
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) sm.apc[w][kq][k][h][gz * 8 + tz] = static_cast<uint8_t>(pc[k]);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // A operands (one per half): lane (m = cg, g = rs), m = (k | q) * 8 + cc * 4 + piece; byte
  // 2 t + cc' holds the piece of row (8 h + t) RPS + 4 w + g when cc' = cc, else 0
  stq_v4i Av[HZ];
  {
    const int kqa = cg >> 3, cca = (cg >> 2) & 1, pa = cg & 3;
    const uint32_t s_even = cca ? 0x010c000cu : 0x0c010c00u;
    const uint32_t s_odd = cca ? 0x030c020cu : 0x0c030c02u;
#pragma unroll
    for (int h = 0; h < HZ; ++h) {
      uint32_t xw[2];
      load_bytes<8>(&sm.apc[w][kqa][pa][h][rs * 8], xw);
      const stq_v4i a4 = {static_cast<int>(__builtin_amdgcn_perm(0u, xw[0], s_even)),
                          static_cast<int>(__builtin_amdgcn_perm(0u, xw[0], s_odd)),
                          static_cast<int>(__builtin_amdgcn_perm(0u, xw[1], s_even)),
                          static_cast<int>(__builtin_amdgcn_perm(0u, xw[1], s_odd))};
      Av[h] = a4;
    }
  }
  // B operands: MFMA i takes two columns of the lane's 8 (i = 0: E bytes 0, 1 = columns 0, 2;
  // 1: E bytes 2, 3 = 4, 6; 2: O bytes 0, 1 = 1, 3; 3: O bytes 2, 3 = 5, 7) for the row steps
  // of a half; the halves accumulate in one integer sum
  stq_v4i acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int wd = i >> 1;
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    stq_v4i c4 = {0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < HZ; ++h) {
      int bw[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        bw[d] = static_cast<int>(__builtin_amdgcn_perm(cw[8 * h + 2 * d + 1][wd], cw[8 * h + 2 * d][wd], sel));
      const stq_v4i Bv = {bw[0], bw[1], bw[2], bw[3]};
      c4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(Av[h], Bv, c4, 0, 0, 0);
    }
    acc[i] = c4;
  }
  // recombine: lane (g = rs, cg) holds, for MFMA i, the four pieces of (k | q = g / 2) at
  // column 8 cg + col(i, cc = g % 2)
  const int kqo = rs >> 1, cco = rs & 1;
  float vo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = fmaf(static_cast<float>(acc[i][3]), 0x1p-7f, static_cast<float>(acc[i][2]));
    v = fmaf(v, 0x1p-7f, static_cast<float>(acc[i][1]));
    v = fmaf(v, 0x1p-7f, static_cast<float>(acc[i][0]));
    vo[i] = ldexpf(v, -S) * cso[i];
  }
  // pivot rows on the VALU, summed over the wave's row slots
  bool wpiv = false;
#pragma unroll
  for (int t = 0; t < NP; ++t) wpiv |= t * RPS + w * 4 < blk.n16;
  if (wpiv) {
    float pvu[CPL], pvp[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) pvu[c] = pvp[c] = 0.0f;
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const int p = t * RPS + w * 4 + rs;
      if (p < blk.n16) {
        const float4 r4 = sm.srow[p];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float x = r4.x * half_bits_to_float(cw[t][c >> 1] >> (16 * (c & 1)));
          pvu[c] = fmaf(r4.y, x, pvu[c]);
          pvp[c] = fmaf(r4.z, x, pvp[c]);
        }
      }
    }
    // every column's sum over the row slots first: the lanes of different row slots select
    // different columns afterwards
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      pvu[c] = sum_row_slots(pvu[c]);
      pvp[c] = sum_row_slots(pvp[c]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c0 = kColOfMfma[i];
      const float pu = cco ? pvu[c0 + 2] : pvu[c0];
      const float pq = cco ? pvp[c0 + 2] : pvp[c0];
      vo[i] += kqo ? pq : pu;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.red[kqo][w][cg * CPL + kColOfMfma[i] + 2 * cco] = vo[i];
  __syncthreads();
  // (4) columns: u, p, delta, the readout; delta / g_j for the integer rows
  float gj = 1.0f;
  if (tid < D) {
    const int j = tid;
    float uu = sm.red[0][0][j], pv = sm.red[1][0][j], qk = sm.redqk[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) {
      uu += sm.red[0][w2][j];
      pv += sm.red[1][w2][j];
      qk += sm.redqk[w2];
    }
    const float dj = beta * (sm.sv[j] - uu);
    a.step.out[int64_t(bh) * D + j] = fmaf(qk, dj, pv);
    const float cs = half_bits_to_float(csj);
    gj = cs > 0.0f ? cs : 1.0f;
    sm.sv[j] = dj;
    sm.sd[j] = __fdiv_rn(dj, gj);
  }
  __syncthreads();

  // (5) the update and the fit's lane sums of (w_i Y_ij)^2. The held words are made opaque
  // before each use, so the compiler cannot keep their decoded values (64 floats) from this
  // pass to the next.
#pragma unroll
  for (int t = 0; t < RPL; ++t) asm volatile("" : "+v"(cw[t][0]), "+v"(cw[t][1]), "+v"(cw[t][2]), "+v"(cw[t][3]));
  float dl[CPL];
  load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.sd + cg * CPL), reinterpret_cast<uint32_t*>(dl));
  float accf[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) accf[c] = 0.0f;
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p = t * RPS + w * 4 + rs;
    const float4 r4 = sm.srow[p];
    const float wt = sm.sw1[p];
    const bool piv_grp = t < NP && fresh_s(t * RPS + w * 4) < blk.n16;   // wave-uniform
    // pivot rows (w = 0) take no part in the fit
    if (!(piv_grp && p < blk.n16)) {
      // w_i Y_ij = (w_i k_i) delta'_j + (w_i gate_i rf_i) c_ij: the weight folded into the row's
      // two factors
      const float wm = wt * (r4.x * r4.w), wk = wt * r4.y;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float yw = fmaf(wk, dl[c], wm * sbyte_f(cw[t][c & 1], c >> 1));
        accf[c] = fmaf(yw, yw, accf[c]);
      }
    }
  }
  store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(&sm.red2[w * 4 + rs][cg * CPL]),
                       reinterpret_cast<const uint32_t*>(accf));
  __syncthreads();
  if (tid < D) {
    const int j = tid;
    double s = static_cast<double>(sm.red2[0][j]);
#pragma unroll
    for (int k = 1; k < 4 * NW; ++k) s += static_cast<double>(sm.red2[k][j]);
    const double g = static_cast<double>(gj);
    const uint32_t hb = blk.sw > 0.0 ? f16_from_f64(sqrt(s * (g * g) / blk.sw)) : 0u;
    const float cs = half_bits_to_float(hb);
    sm.sratio[j] = cs > 0.0f ? __fdiv_rn(gj, cs) : 0.0f;
    buf_store<2>(dst, blk.ocs + 2u * j, 0u, &hb);
  }
  __syncthreads();

  // (6) per row: row factor, codes, store, with the row kind (and so qmax) known at compile time
#pragma unroll
  for (int t = 0; t < RPL; ++t) asm volatile("" : "+v"(cw[t][0]), "+v"(cw[t][1]), "+v"(cw[t][2]), "+v"(cw[t][3]));
  float ratio[CPL];
  load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.sratio + cg * CPL), reinterpret_cast<uint32_t*>(ratio));
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = fresh_s(t * RPS + w * 4), p = p0 + fresh(rs);
    float yr[CPL];
    {
      const float4 r4 = sm.srow[p];
      const bool piv_grp = t < NP && p0 < blk.n16;
      if (piv_grp && p < blk.n16) {
        float dv[CPL];
        load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sm.sv + cg * CPL), reinterpret_cast<uint32_t*>(dv));
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          yr[c] = fmaf(r4.y, dv[c], r4.x * half_bits_to_float(cw[t][c >> 1] >> (16 * (c & 1))));
      } else {
        const float m = r4.x * r4.w;
#pragma unroll
        for (int c = 0; c < CPL; ++c) yr[c] = fmaf(r4.y, dl[c], m * sbyte_f(cw[t][c & 1], c >> 1));
      }
    }
    auto rowf = [&](auto KC) {
      constexpr int K = decltype(KC)::value;
      uint32_t tb[CPL];
      if constexpr (K != SK_F16) {
        constexpr float qm = K == SK_I8 ? 127.0f : (K == SK_I6 ? 31.0f : 7.0f);
        constexpr float inv = 1.0f / qm;
        float av[CPL];
        float mq = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          av[c] = yr[c] * ratio[c];
          mq = fmaxf(mq, fabsf(av[c]));
        }
        const float m = max_row16(mq);
        const uint32_t rb = float_to_half_bits(div_qmax(m, qm, inv));
        const float rf = half_bits_to_float(rb);
        if (cg == 0) sm.srf[p - blk.n16] = static_cast<uint16_t>(rb);
        // rf = 0 only where every a_j is 0, which then codes 0 with any finite factor
        const float rrf = __builtin_amdgcn_rcpf(fmaxf(rf, 0x1p-126f));
#pragma unroll
        for (int c = 0; c < CPL; ++c) tb[c] = __float_as_uint(fmaf(av[c], rrf, kMagic));
        if (__any(rf < 0x1p-14f)) {
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            tb[c] = __float_as_uint(__builtin_amdgcn_fmed3f(__uint_as_float(tb[c]), kMagic - qm, kMagic + qm));
        }
      }
      stq_store<D, K>(dst, blk, p, cg, yr, tb);
    };
    if (t < NP) by_kind2<true>(blk, p0, p, rowf);
    else by_kind2<false>(blk, p0, p, rowf);
  }
  // the row factors, gathered in LDS, go out as one contiguous run
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

template <int NP, int NW>
hipError_t stq_step2_launch(int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H)), block(64 * NW);
  if (per_key) {
    if (bf16) hipLaunchKernelGGL((stq_step2_kernel<1, 1, NP, NW>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stq_step2_kernel<1, 0, NP, NW>), grid, block, 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((stq_step2_kernel<0, 1, NP, NW>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((stq_step2_kernel<0, 0, NP, NW>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// The d = 128 step runs the codes-held kernel; DAMP_STQ_STEP=x (read once) selects the X-held
// kernel instead, for comparisons.
bool stq_step_x_held() {
  static const bool x = [] {
    const char* e = getenv("DAMP_STQ_STEP");
    return e && e[0] == 'x';
  }();
  return x;
}

template <int D>
hipError_t stq_d(int mode, int per_key, int bf16, const StqArgs& a, hipStream_t s) {
  constexpr int NW = kStqWaves<D>;
  if constexpr (D == 128) {
    // four waves per unit (16-row steps; NP = row steps that may hold pivot rows): with two
    // (the kernel's NW = 2, 103 VGPRs, four waves per SIMD) the step measured 342-344 us
    // against 330 us on the 1,024-slot pool, 102 against 95.5 us on 256 KDA slots
    if (mode == SM_STEP && !stq_step_x_held())
      return a.max_pivots <= 16 ? stq_step2_launch<1, 4>(per_key, bf16, a, s) : stq_step2_launch<8, 4>(per_key, bf16, a, s);
  }
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
