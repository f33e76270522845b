// step_common.h -- device building blocks shared by the gfx950 kernels of libdamp.so: geometry,
// byte movement, binary16 conversions, cross-lane reductions, the INT8 row rule, raw buffer
// instructions, the per-row load / decode / requantize-store of the state formats, row plans,
// the staging of the per-row scalars and the column pass of the decode step.
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
// fully coalesced. Column sums over key rows go through LDS: every lane writes its partial sums
// once and one thread per column adds them in a fixed order (only q.k, one value per lane, uses
// the gfx950 cross-row lane swaps v_permlane16_swap / v_permlane32_swap); the row absmax for
// requantization is a DPP butterfly inside the 16 lanes of a row. No MFMA: each unit is a
// matrix-vector update at ~4 flop/byte, far below the fp32 ridge; the kernel is HBM-bound, and
// its VALU work per state element is kept to about ten instructions so that it stays so
// (CDNA4 issues one wave64 VALU instruction per SIMD every 4 cycles).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace damp {
namespace {

template <int D, int NW_ = (D >= 128 ? 4 : (D >= 64 ? 2 : 1))>
struct Geo {
  static constexpr int NW = NW_;                               // waves per workgroup
  static constexpr int NT = NW * 64;                           // threads per workgroup
  static constexpr int CPL = D / 16;                           // value columns per lane
  static constexpr int RPS = NW * 4;                           // storage rows per row step
  static constexpr int RPL = D / RPS;                          // row steps (rows) per lane
  // row steps that may hold FP16 rows in PLAN_SMALL (at least the first two; D / 4 rows)
  static constexpr int T16 = (D / 4) / RPS > 2 ? (D / 4) / RPS : 2;
  static_assert(D % 16 == 0 && RPL * RPS == D, "unsupported d");
};

// Kind of one stored row.
// K_MIX: a wave's row step holding both kinds (the FP16 / INT8 boundary when r % 4 != 0).
enum Kind : int { K_F32 = 0, K_F16 = 1, K_I8 = 2, K_MIX = 3 };

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
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true)));
  return x;
}

// Sum over the 16 lanes of a row, by the same DPP pattern as max_row16 (every lane of the row
// ends with the same sum; the addition order is fixed).
__device__ __forceinline__ float sum_row16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
  return x;
}

// ---- the INT8 row rule --------------------------------------------------------------------
// scale = fl(m / 127). q = fl(m * fl(1/127)) followed by one residual correction gives the
// correctly rounded quotient: checked against IEEE division for every binary32 significand at
// exponents from 2^-120 to 2^127, which covers every finite non-negative m the rule meets.
constexpr float kInv127 = 1.0f / 127.0f;

__device__ __forceinline__ float div127(float m) {
  const float q = m * kInv127;
  const float r = fmaf(-q, 127.0f, m);
  return fmaf(r, kInv127, q);
}

// Exact code: round-half-to-even of the binary32 quotient fl(x / s) (s > 0, inv = fl(1/s)).
// The estimate y = fl(x * inv) is within 2^-23 relative (|y| <= 127.5: 1.6e-5 absolute) of
// x/s, and fl(x/s) within 3.9e-6 of it, so unless y is within 2^-15 of a half-integer both
// round to the same integer; otherwise the IEEE division decides. Used where the input is
// the caller's fp32 state (pack), so that packing is bit-identical to the rule.
__device__ __forceinline__ int32_t int8_code_exact(float x, float s, float inv) {
  const float y = x * inv;
  float n = rintf(y);
  if (fabsf(y - n) > 0.5f - 0x1p-15f) n = rintf(__fdiv_rn(x, s));
  n = fminf(fmaxf(n, -127.0f), 127.0f);
  return static_cast<int32_t>(n);
}

// Fast code inside the step: round-half-to-even of x * rcp(s), with v_rcp_f32 (1 ulp) and the
// rounding done by one fma against 1.5 * 2^23 (the integer lands in the low mantissa bits, so
// the low byte is the two's-complement code). |x * rcp(s)| <= 127 (1 + 2^-22) < 127.5, so no
// clamp is needed. It can differ from the exact rule only where x/s lies within ~2e-5 of a
// half-integer (a few codes per 100,000, by one); the step's X itself differs from the
// oracle's by a few fp32 ulps, which moves codes at the same places.
__device__ __forceinline__ uint32_t int8_code_fast_bits(float x, float inv) {
  return __float_as_uint(fmaf(x, inv, 0x1.8p23f));
}

// Pack the low bytes of four words: v_perm_b32 picks byte 0 of each source.
__device__ __forceinline__ uint32_t pack4_low_bytes(uint32_t f0, uint32_t f1, uint32_t f2,
                                                    uint32_t f3) {
  const uint32_t lo = __builtin_amdgcn_perm(f1, f0, 0x0c0c0400u);  // f0.b0, f1.b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(f3, f2, 0x04000c0cu);  // 0, 0, f2.b0, f3.b0
  return lo | hi;
}

// ---- one lane's part of one stored row: load, decode, requantize + store ----------------
// State traffic goes through raw buffer instructions: one scalar resource per region of the
// unit (base, byte size), a 32-bit per-lane offset, and hardware range checking (an offset
// past the region reads 0 and drops the write).
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor word 3 for raw byte access
// Cache policy of the state traffic: non-temporal ("nt"). Every state byte is read once and
// written once per step, so keeping it out of the caches' normal replacement matters: on MI355X
// a streaming copy runs ~6 TB/s with nt and ~3.7-5.3 TB/s without.
constexpr int kNT = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRsrcWord3);
}

template <int N>
__device__ __forceinline__ void buf_load(rsrc_t rs, uint32_t off, uint32_t soff, uint32_t* w) {
  if constexpr (N == 32) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, kNT);
    const auto b = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, soff, kNT);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else if constexpr (N == 16) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, kNT);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else if constexpr (N == 8) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(rs, off, soff, kNT);
    w[0] = a[0]; w[1] = a[1];
  } else if constexpr (N == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, soff, kNT);
  } else if constexpr (N == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, soff, kNT);
  } else {
    static_assert(N == 1, "bad width");
    w[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, off, soff, kNT);
  }
}

// A store of more than 64 bits of data reads its data registers after it issues, so a VALU
// instruction right behind it must not overwrite them. The compiler inserts that wait only when
// the instruction's soffset is a constant; with an SGPR soffset it does not, and on gfx950 the
// overwrite then reaches memory (seen as corrupted first dwords of 16-byte row chunks when a
// conversion was scheduled directly after the store). guard_store keeps the data registers
// live across an s_nop of two wait states issued after the store.
using v4u = __attribute__((ext_vector_type(4))) unsigned int;
using v2u = __attribute__((ext_vector_type(2))) unsigned int;

__device__ __forceinline__ void guard_store(v4u data) { asm volatile("s_nop 1" ::"v"(data)); }
__device__ __forceinline__ void guard_store2(v4u a, v4u b) { asm volatile("s_nop 1" ::"v"(a), "v"(b)); }

template <int N>
__device__ __forceinline__ void buf_store(rsrc_t rs, uint32_t off, uint32_t soff, const uint32_t* w) {
  if constexpr (N == 32) {
    const v4u a{w[0], w[1], w[2], w[3]}, b{w[4], w[5], w[6], w[7]};
    // back to back, then one guard: the two halves of the lane's 32 bytes stay one clause
    __builtin_amdgcn_raw_buffer_store_b128(a, rs, off, soff, kNT);
    __builtin_amdgcn_raw_buffer_store_b128(b, rs, off + 16, soff, kNT);
    guard_store2(a, b);
  } else if constexpr (N == 16) {
    const v4u a{w[0], w[1], w[2], w[3]};
    __builtin_amdgcn_raw_buffer_store_b128(a, rs, off, soff, kNT);
    guard_store(a);
  } else if constexpr (N == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(v2u{w[0], w[1]}, rs, off, soff, kNT);
  } else if constexpr (N == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, off, soff, kNT);
  } else if constexpr (N == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w[0]), rs, off, soff, kNT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(w[0]), rs, off, soff, kNT);
  }
}

// The unit's three regions (FP16 rows or the fp32 state; INT8 rows; INT8 row scales), each
// a resource plus the region's byte offset inside it. With ONE (a contiguous DAMP block and no
// mixed row step, so no access relies on region range checks) a single resource spans the
// block and the regions are offsets into it: fewer scalar registers.
struct UnitPtr {
  rsrc_t h;
  rsrc_t c;
  rsrc_t s;
  uint32_t coff;
  uint32_t soff;
  int r;
};

// Where the unit of (slot, head) lives: its FP16 (or fp32) region, INT8 region, scale region
// and FP16 row count. Per-head DAMP layouts read the head's block offset and r from a table.
struct UnitAddr {
  uint8_t* h;
  uint8_t* c;
  uint8_t* s;
  int r;
};

template <int D, int FMT>
__device__ __forceinline__ UnitAddr unit_addr(const StateRef& st, int64_t slot, int head, int H) {
  if (FMT == FMT_Q && st.heads) {
    const int2 hi = st.heads[head];
    uint8_t* blk = st.hbase + slot * st.slot_stride + hi.x;
    return UnitAddr{blk, blk + 2 * hi.y * D, blk + 2 * hi.y * D + (D - hi.y) * D, hi.y};
  }
  const int64_t unit = slot * H + head;
  return UnitAddr{st.hbase + unit * st.hstride, st.cbase + unit * st.cstride,
                  st.sbase + unit * st.sstride, FMT == FMT_Q ? st.r : 0};
}

template <int D, int FMT, bool ONE = false>
__device__ __forceinline__ UnitPtr unit_ptr(const UnitAddr& ua, int r_rows) {
  const uint32_t r = FMT == FMT_Q ? static_cast<uint32_t>(r_rows) : 0u;
  if constexpr (ONE) {
    const rsrc_t blk = make_rsrc(ua.h, 2 * r * D + (D - r) * D + 4 * (D - r));
    return UnitPtr{blk, blk, blk, 2 * r * D, 2 * r * D + (D - r) * D, static_cast<int>(r)};
  }
  const uint32_t hbytes = FMT == FMT_F32 ? D * D * 4 : 2 * r * D;
  return UnitPtr{make_rsrc(ua.h, hbytes), make_rsrc(ua.c, (D - r) * D),
                 make_rsrc(ua.s, (D - r) * 4), 0u, 0u, static_cast<int>(r)};
}

// Byte offset of one lane's part of a storage row inside its region, split into a per-lane part
// (voff) and a wave-uniform part (soff, an unsigned scalar register of the instruction).
struct Loc {
  uint32_t voff;
  uint32_t soff;
};

// Storage row p = p0 + rs (p0: the wave's first row of this row step), value columns
// cg*CPL .. cg*CPL + CPL - 1. MIX: the wave's 4 rows mix FP16 and INT8 rows (r % 4 != 0), so
// the INT8 row index p - r is formed per lane.
template <int D, int KIND>
struct Row {
  static constexpr int CPL = Geo<D>::CPL;
  static constexpr int BYTES = KIND == K_F32 ? CPL * 4 : (KIND == K_F16 ? CPL * 2 : CPL);
  static constexpr int W = Words<BYTES>::W;
  static constexpr int E = KIND == K_F32 ? 4 : (KIND == K_F16 ? 2 : 1);  // bytes per value

  // MIX: the whole offset goes in voff, which the buffer range check covers, so an access to
  // a row of the other kind falls outside this region (the INT8 index p - r wraps to a huge
  // unsigned value; an FP16 offset of an INT8 row is past the FP16 region) and is discarded.
  template <bool MIX>
  __device__ static __forceinline__ Loc loc(const UnitPtr& u, int p0, int rs, int cg) {
    if constexpr (KIND == K_I8) {
      if constexpr (MIX)
        return Loc{static_cast<uint32_t>((p0 + rs - u.r) * D + cg * CPL), 0u};
      return Loc{static_cast<uint32_t>(rs * D + cg * CPL), u.coff + static_cast<uint32_t>((p0 - u.r) * D)};
    }
    if constexpr (MIX) return Loc{static_cast<uint32_t>(((p0 + rs) * D + cg * CPL) * E), 0u};
    return Loc{static_cast<uint32_t>((rs * D + cg * CPL) * E), static_cast<uint32_t>(p0 * D * E)};
  }

  // scale of the INT8 row (4 bytes per row)
  template <bool MIX>
  __device__ static __forceinline__ Loc scale_loc(const UnitPtr& u, int p0, int rs) {
    if constexpr (MIX) return Loc{static_cast<uint32_t>((p0 + rs - u.r) * 4), 0u};
    return Loc{static_cast<uint32_t>(rs * 4), u.soff + static_cast<uint32_t>((p0 - u.r) * 4)};
  }

  __device__ static __forceinline__ rsrc_t region(const UnitPtr& u) {
    return KIND == K_I8 ? u.c : u.h;
  }

  __device__ static __forceinline__ void load(const UnitPtr& u, Loc l, uint32_t* raw) {
    buf_load<BYTES>(region(u), l.voff, l.soff, raw);
  }

  __device__ static __forceinline__ float decode(const uint32_t* w, int c) {
    if constexpr (KIND == K_F32) return __uint_as_float(w[c]);
    if constexpr (KIND == K_F16) return half_bits_to_float(w[c >> 1] >> (16 * (c & 1)));
    return static_cast<float>(static_cast<int8_t>(w[c >> 2] >> (8 * (c & 3))));
  }

  // EXACT selects int8_code_exact (pack kernel) instead of the fast code (step kernel).
  // SC_LDS: the INT8 row scale goes to sc_lds[p] (the caller writes the unit's scales to memory
  // later with one coalesced store) instead of a 4-byte store per row.
  template <bool EXACT, bool MIX, bool SC_LDS = false>
  __device__ static __forceinline__ void store(const UnitPtr& u, int p0, int rs, int cg,
                                               const float* x, float* sc_lds = nullptr) {
    uint32_t wd[W];
    if constexpr (KIND == K_F32) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) wd[c] = __float_as_uint(x[c]);
    } else if constexpr (KIND == K_F16) {
#pragma unroll
      for (int i = 0; i < W; ++i) wd[i] = 0;
#pragma unroll
      for (int c = 0; c < CPL; ++c) wd[c >> 1] |= float_to_half_bits(x[c]) << (16 * (c & 1));
    } else {
      float m = fabsf(x[0]);
#pragma unroll
      for (int c = 1; c < CPL; ++c) m = fmaxf(m, fabsf(x[c]));
      m = max_row16(m);
      const float s = div127(m);
      // The codes of values xx with scale ss: ss normal, or 0 (an all-zero row, or one whose
      // absmax is below 127 * 2^-150, where m / 127 rounds to zero): then every code is 0.
      auto codes = [&](const float* xx, float ss) __attribute__((always_inline)) {
        if constexpr (EXACT) {
          const float inv = ss > 0.0f ? __fdiv_rn(1.0f, ss) : 0.0f;
#pragma unroll
          for (int i = 0; i < W; ++i) wd[i] = 0;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const int32_t code = ss > 0.0f ? int8_code_exact(xx[c], ss, inv) : 0;
            wd[c >> 2] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (c & 3));
          }
        } else {
          const float inv = ss > 0.0f ? __builtin_amdgcn_rcpf(ss) : 0.0f;
          uint32_t f[CPL];
#pragma unroll
          for (int c = 0; c < CPL; ++c) f[c] = int8_code_fast_bits(xx[c], inv);
          if constexpr (CPL >= 4) {
#pragma unroll
            for (int i = 0; i < CPL / 4; ++i)
              wd[i] = pack4_low_bytes(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
          } else if constexpr (CPL == 2) {
            wd[0] = __builtin_amdgcn_perm(f[1], f[0], 0x0c0c0400u);
          } else {
            wd[0] = f[0] & 0xFFu;
          }
        }
      };
      // A row whose absmax is below 127 * 2^-126 (~1.5e-36) has a subnormal scale, whose
      // reciprocal overflows. Its codes are taken on the row and the scale both multiplied by
      // 2^64, which is exact and leaves every quotient x / s as it is. The branch is
      // wave-uniform and only waves holding such a row take it; the stored scale is s itself.
      const bool tiny = s > 0.0f && s < 0x1p-126f;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(tiny) != 0, 0)) {
        const float k2 = tiny ? 0x1p64f : 1.0f;
        float xs[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) xs[c] = x[c] * k2;
        codes(xs, s * k2);
      } else {
        codes(x, s);
      }
      if (cg == 0) {
        if constexpr (SC_LDS) {
          sc_lds[p0 + rs] = s;
        } else {
          const uint32_t sb = __float_as_uint(s);
          const Loc sl = scale_loc<MIX>(u, p0, rs);
          buf_store<4>(u.s, sl.voff, sl.soff, &sb);
        }
      }
    }
    const Loc l = loc<MIX>(u, p0, rs, cg);
    buf_store<BYTES>(region(u), l.voff, l.soff, wd);
  }
};

// Dispatch one row step on the row kind. p0 = first storage row of the wave's 4 rows
// (wave-uniform, so the FP16 / INT8 choice is a scalar branch unless r is not a multiple of
// 4, where one row step of one wave mixes both kinds and branches per lane).
// ---- row plans ------------------------------------------------------------------------------
// Which kind each row step of a wave holds. A wave's row step covers storage rows p0..p0+3, so
// with r % 4 == 0 every row step is all-FP16 or all-INT8 (a scalar branch); otherwise the one
// row step that straddles r mixes both (K_MIX). The plans are separate kernel instances so the
// common cases carry no code (and no registers) for the mixed one.
//   PLAN_F32:   fp32 state
//   PLAN_SMALL: r % 4 == 0 and r <= T16 * RPS: only the first T16 row steps can hold FP16
//               rows, every later row step is INT8 at compile time (its raw words are half as
//               many)
//   PLAN_R4:    r % 4 == 0
//   PLAN_ANY:   any r
//   PLAN_FIXED: r = T * RPS fixed at compile time: row steps 0 .. T-1 are FP16, the rest INT8,
//               so after unrolling no row step branches on its kind
enum Plan : int { PLAN_F32 = 0, PLAN_SMALL = 1, PLAN_R4 = 2, PLAN_ANY = 3, PLAN_FIXED = 4 };

// T: PLAN_SMALL's T16, or PLAN_FIXED's FP16 row step count.
template <int PLAN, int T = 2, typename F>
__device__ __forceinline__ void by_plan(int t, int p0, int r, F&& f) {
  constexpr int T16 = T;
  if constexpr (PLAN == PLAN_F32) {
    f.template operator()<K_F32>();
  } else if constexpr (PLAN == PLAN_FIXED) {
    if (t < T)
      f.template operator()<K_F16>();
    else
      f.template operator()<K_I8>();
  } else {
    if (PLAN == PLAN_SMALL && t >= T16) {
      f.template operator()<K_I8>();
    } else if (p0 + 4 <= r) {
      f.template operator()<K_F16>();
    } else if (PLAN != PLAN_ANY || p0 >= r) {
      f.template operator()<K_I8>();
    } else {
      f.template operator()<K_MIX>();
    }
  }
}

// A per-kind operation for one of the kinds above: K_MIX runs both the FP16 and the INT8 form
// with MIX offsets (each lane's access of the other kind falls outside its region and is
// discarded by the buffer range check).
template <int K, typename F>
__device__ __forceinline__ void each_kind(F&& f) {
  if constexpr (K == K_MIX) {
    f.template operator()<K_F16, true>();
    f.template operator()<K_I8, true>();
  } else {
    f.template operator()<K, false>();
  }
}

// Load the lane's part of row step t into raw (K_MIX: both loads; the one outside its region
// reads zeros, so OR-ing merges them).
template <int D, int K>
__device__ __forceinline__ void load_row_step(const UnitPtr& up, int p0, int rs, int cg, uint32_t* raw) {
  if constexpr (K == K_MIX) {
    uint32_t w8[Row<D, K_I8>::W];
    Row<D, K_F16>::load(up, Row<D, K_F16>::template loc<true>(up, p0, rs, cg), raw);
    Row<D, K_I8>::load(up, Row<D, K_I8>::template loc<true>(up, p0, rs, cg), w8);
#pragma unroll
    for (int i = 0; i < Row<D, K_I8>::W; ++i) raw[i] |= w8[i];
  } else {
    Row<D, K>::load(up, Row<D, K>::template loc<false>(up, p0, rs, cg), raw);
  }
}

// Decoded value c of a lane's raw row (storage row p; K_MIX decides per lane).
template <int D, int K>
__device__ __forceinline__ float decode_row(const uint32_t* raw, int c, int p, int r) {
  if constexpr (K == K_MIX)
    return p < r ? Row<D, K_F16>::decode(raw, c) : Row<D, K_I8>::decode(raw, c);
  else
    return Row<D, K>::decode(raw, c);
}

// Per-row scalars of the unit in storage order: srow[i] = {m_i, k_i, q_i, -} with the row
// multiplier m_i = a_i * scale_i for INT8 rows and a_i otherwise (the gate folded into the
// scale: S'_ij = code_ij * m_i), and v in sv. Every global load here is independent of the
// others (k, q and the gate are read in key order, the row map in parallel) and the
// permutation to storage order goes through LDS (tmp: 3 * D floats), so the staging costs one
// memory round trip rather than a row-map load followed by dependent k / q loads.
//
// Fused pre-step (a.prestep != 0): q and k arrive as the layer's projections and alpha / beta as
// logits; the step uses q / ||q||, k / ||k|| (a zero vector stays zero), alpha = exp(-softplus(g))
// = 1 / (1 + e^g) and beta = 1 / (1 + e^-b). The squared norms are summed in fp32 (each thread's
// elements, then a wave butterfly, then the waves in order, in tmp[3 D ..]) and applied as
// rsqrt(||x||^2) while permuting into storage order. Returns beta (after the activation).
__device__ __forceinline__ float gate_from_logit(float g) { return 1.0f / (1.0f + expf(g)); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Whether a slot index addresses the pool. Distinct indices in [0, num_slots) are the caller's
// contract (DAMP_DEBUG checks it on the host); a workgroup whose slot lies outside returns before
// it touches the pool, its window buffer or its readout, so a bad index cannot send an access
// outside them.
__device__ __forceinline__ bool slot_in_pool(int64_t slot, int32_t num_slots) {
  return static_cast<uint64_t>(slot) < static_cast<uint64_t>(static_cast<uint32_t>(num_slots));
}

// The unit of this workgroup: head = w mod H of batch position order[w / H] (w / H without an
// order). False for an order entry outside [0, B): the workgroup then does nothing.
__device__ __forceinline__ bool unit_of(const StepArgs& a, int& b, int& head) {
  const int w = __builtin_amdgcn_workgroup_id_x();
  const int p = w / a.H;
  head = w - p * a.H;
  b = a.order ? a.order[p] : p;
  return static_cast<unsigned>(b) < static_cast<unsigned>(a.B);
}

// The staging in two phases. load() issues every global load the staging needs (row map, old
// INT8 scales, k, q, the gate, v, beta) into registers and touches no LDS; store() writes them to
// LDS, applies the fused pre-step and permutes to storage order. A step kernel calls load()
// BEFORE it issues the state loads: the memory counter is in order, so store()'s wait then
// covers only these few older loads and the staging and its barriers run while the unit's state
// is still arriving, instead of after the last state byte (the state loads are the bulk of the
// unit's bytes; the first row steps can be reduced as soon as they land).
template <int D, int NT, int PER_KEY, int BF16, bool Q>
struct Stage {
  static constexpr int PER = (D + NT - 1) / NT;
  static constexpr int NWS = NT / 64;
  // Loaded values as raw words: bf16 inputs are widened only in store(), so no instruction that
  // uses a loaded value (and waits for it) sits before the caller's state loads.
  uint32_t src[PER], sc[PER], kv[PER], qv[PER], gv[PER], vv[PER];
  float g0, beta;

  template <int B16>
  __device__ static __forceinline__ uint32_t raw_in(const void* base, int64_t i) {
    if constexpr (B16)
      return reinterpret_cast<const uint16_t*>(base)[i];
    else
      return reinterpret_cast<const uint32_t*>(base)[i];
  }
  __device__ static __forceinline__ float widen(uint32_t w) {
    return BF16 ? __uint_as_float(w << 16) : __uint_as_float(w);  // bf16 -> fp32 is exact
  }

  __device__ __forceinline__ void load(const StepArgs& a, const float* sc_old, int bh, int head, int r,
                                       int tid) {
    const int64_t vec = int64_t(bh) * D;
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int i = tid + n * NT;
      src[n] = static_cast<uint32_t>(i);
      sc[n] = __float_as_uint(1.0f);
      kv[n] = qv[n] = gv[n] = vv[n] = 0u;
      if (PER * NT == D || i < D) {
        if (a.st.rowmap) src[n] = a.st.rowmap[head * D + i];
        if constexpr (Q)
          if (i >= r) sc[n] = reinterpret_cast<const uint32_t*>(sc_old)[i - r];
        kv[n] = raw_in<BF16>(a.k, vec + i);
        qv[n] = raw_in<BF16>(a.q, vec + i);
        if constexpr (PER_KEY) gv[n] = reinterpret_cast<const uint32_t*>(a.alpha)[vec + i];
        vv[n] = raw_in<BF16>(a.v, vec + i);
      }
    }
    g0 = PER_KEY ? 0.0f : a.alpha[bh];
    beta = a.beta[bh];
  }

  // An empty asm statement that takes the staged values: the compiler keeps memory accesses on
  // their side of it, so a caller that issues its state loads between load() and store() gets
  // them issued before the first use of the staged values (and before the wait for them).
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int n = 0; n < PER; ++n)
      asm volatile("" : "+v"(src[n]), "+v"(sc[n]), "+v"(kv[n]), "+v"(qv[n]), "+v"(gv[n]), "+v"(vv[n]));
  }

  // Returns beta (after the activation with the fused pre-step) in a scalar register.
  __device__ __forceinline__ float store(const StepArgs& a, int tid, float4* srow, float* sv, float* tmp) {
    fence();
    const bool pre = a.prestep != 0;
    float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int i = tid + n * NT;
      if (PER * NT == D || i < D) {
        const float kf = widen(kv[n]), qf = widen(qv[n]), gf = __uint_as_float(gv[n]);
        tmp[i] = kf;
        tmp[D + i] = qf;
        ssk = fmaf(kf, kf, ssk);
        ssq = fmaf(qf, qf, ssq);
        if constexpr (PER_KEY) tmp[2 * D + i] = pre ? gate_from_logit(gf) : gf;
        sv[i] = widen(vv[n]);
      }
    }
    float g = g0, bt = beta;
    if (pre) {
      if constexpr (!PER_KEY) g = gate_from_logit(g);
      bt = 1.0f / (1.0f + expf(-bt));
      ssq = wave_sum(ssq);
      ssk = wave_sum(ssk);
      if ((tid & 63) == 0) {
        tmp[3 * D + 2 * (tid >> 6)] = ssq;
        tmp[3 * D + 2 * (tid >> 6) + 1] = ssk;
      }
    }
    __syncthreads();
    float invq = 1.0f, invk = 1.0f;
    if (pre) {
      float nq = tmp[3 * D], nk = tmp[3 * D + 1];
#pragma unroll
      for (int w2 = 1; w2 < NWS; ++w2) {
        nq += tmp[3 * D + 2 * w2];
        nk += tmp[3 * D + 2 * w2 + 1];
      }
      invq = nq > 0.0f ? rsqrtf(nq) : 0.0f;
      invk = nk > 0.0f ? rsqrtf(nk) : 0.0f;
    }
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int i = tid + n * NT;
      if (PER * NT == D || i < D) {
        const float gi = PER_KEY ? tmp[2 * D + src[n]] : g;
        srow[i] = make_float4(__uint_as_float(sc[n]) * gi, tmp[src[n]] * invk, tmp[D + src[n]] * invq, 0.0f);
      }
    }
    __syncthreads();
    // beta (uniform over the workgroup) for the column pass, in a scalar register
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bt)));
  }
};

// Column sums over the key rows, shared by the step kernels. Every lane writes its CPL partial
// sums of u = S'^T k and p = S'^T q (over its RPL rows) to LDS; thread j then adds the 4*NW
// partials of column j in a fixed order, forms delta_j = beta (v_j - u_j) (left in sv[j]) and
// the readout y_j = p_j + (q.k) delta_j. (q.k is summed over row slots with lane swaps.)
template <int D, typename G>
__device__ __forceinline__ void finish_columns(float (*redu)[D], float (*redp)[D], float* redqk,
                                               float* sv, float* pu, float* pp, float pqk,
                                               float beta, float* out_row, int tid, int w, int rs,
                                               int lane, int cg) {
  constexpr int CPL = G::CPL, NW = G::NW;
  store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(&redu[w * 4 + rs][cg * CPL]),
                       reinterpret_cast<const uint32_t*>(pu));
  store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(&redp[w * 4 + rs][cg * CPL]),
                       reinterpret_cast<const uint32_t*>(pp));
  pqk = sum_row_slots(pqk);
  if (lane == 0) redqk[w] = pqk;
  __syncthreads();
  for (int j = tid; j < D; j += G::NT) {
    float uu = redu[0][j], pv = redp[0][j];
#pragma unroll
    for (int k = 1; k < 4 * NW; ++k) {
      uu += redu[k][j];
      pv += redp[k][j];
      // with many waves, keep the LDS reads to eight in flight: read all at once, the 2 * 4 * NW
      // partials would take as many VGPRs while the caller's state is live
      if constexpr (4 * NW > 8)
        if ((k & 7) == 7) asm volatile("" ::: "memory");
    }
    float qk = redqk[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) qk += redqk[w2];
    const float dj = beta * (sv[j] - uu);
    sv[j] = dj;
    out_row[j] = fmaf(qk, dj, pv);
  }
  __syncthreads();
}

// Write the INT8 row scales gathered in sc_lds[r .. D) with consecutive lanes (coalesced).
template <int D, int NT>
__device__ __forceinline__ void flush_scales(const UnitPtr& u, const float* sc_lds, int r, int tid) {
  __syncthreads();
  for (int i = r + tid; i < D; i += NT) {
    const uint32_t sb = __float_as_uint(sc_lds[i]);
    buf_store<4>(u.s, static_cast<uint32_t>(i - r) * 4u, u.soff, &sb);
  }
}

// Waves per workgroup of the quantized step with the row kinds fixed at compile time: two at
// d = 128 (78 VGPRs with 24 FP16 rows), which measured a few percent faster than four waves per
// unit on the short batches and equal on the long one; one wave per unit (115 VGPRs) measured
// slower everywhere. A CU was measured to hold at most 8 workgroups of the step at once
// whatever their register count, so a unit's two waves may use up to 128 VGPRs at no cost.
constexpr int kStepWaves = 2;
template <int D>
constexpr int kWaves = kStepWaves < Geo<D>::NW ? kStepWaves : Geo<D>::NW;

}  // namespace
}  // namespace damp
