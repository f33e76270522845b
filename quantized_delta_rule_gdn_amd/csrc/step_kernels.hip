// step_kernels.hip -- gfx950 kernels for the GDN / KDA recurrent-state decode step in three
// state formats (FP32; DAMP FP16 + INT8 rows; uniform INT8 = DAMP with no FP16 rows), and the
// pack / unpack kernels between fp32 states and the quantized formats. The building blocks (and
// the description of the step and of its mapping on CDNA4) are in step_common.h.
#include "step_common.h"

namespace damp {
namespace {

// ---- the decode step, fp32 state ---------------------------------------------------------
// The state is read once into VGPRs (64 fp32 per lane at d = 128), decayed, reduced, updated
// and written back.
template <int D, int PER_KEY, int BF16>
__global__ __launch_bounds__(Geo<D>::NT) void step_kernel_f32(const StepArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL, RPL = G::RPL, NW = G::NW;
  __shared__ float4 srow[D];
  __shared__ float sv[D];  // v, then delta
  __shared__ float redu[4 * NW][D], redp[4 * NW][D], redqk[NW];

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int bh = __builtin_amdgcn_workgroup_id_x();  // b * H + head
  const int b = bh / a.H;
  const int head = bh - b * a.H;
  const int64_t slot = a.slot_idx[b];
  const UnitAddr ua = unit_addr<D, FMT_F32>(a.st, slot, head, a.H);   // arithmetic only
  if (!slot_in_pool(slot, a.st.num_slots)) return;
  const UnitPtr up = unit_ptr<D, FMT_F32>(ua, 0);

  // (1) the staging loads (per-row scalars, v), then every state load of this lane, so the
  // whole block is in flight while the staging completes
  Stage<D, G::NT, PER_KEY, BF16, false> sg;
  sg.load(a, nullptr, bh, head, 0, tid);
  float S[RPL][CPL];
#pragma unroll
  for (int t = 0; t < RPL; ++t)
    Row<D, K_F32>::load(up, Row<D, K_F32>::template loc<false>(up, t * G::RPS + w * 4, rs, cg),
                        reinterpret_cast<uint32_t*>(S[t]));

  // (2) per-row scalars and v into LDS
  const float beta = sg.store(a, tid, srow, sv, &redu[0][0]);

  // (3) decay, partial u = S'^T k, p = S'^T q over this lane's rows
  float pu[CPL], pp[CPL], pqk = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) pu[c] = pp[c] = 0.0f;
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const float4 rw = srow[t * G::RPS + w * 4 + rs];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      S[t][c] *= rw.x;
      pu[c] = fmaf(rw.y, S[t][c], pu[c]);
      pp[c] = fmaf(rw.z, S[t][c], pp[c]);
    }
    pqk = fmaf(rw.z, rw.y, pqk);
    __builtin_amdgcn_sched_barrier(0);  // row steps in load order, as in the quantized step
  }

  // (4) column reductions, delta and the readout y = p + (q.k) delta (one thread per column)
  finish_columns<D, G>(redu, redp, redqk, sv, pu, pp, pqk, beta, a.out + int64_t(bh) * D,
                       tid, w, rs, lane, cg);
  float dl[CPL];
  load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sv + cg * CPL), reinterpret_cast<uint32_t*>(dl));

  // (5) X = S' + k delta^T, stored in place
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = t * G::RPS + w * 4;
    const float kp = srow[p0 + rs].y;
#pragma unroll
    for (int c = 0; c < CPL; ++c) S[t][c] = fmaf(kp, dl[c], S[t][c]);
    Row<D, K_F32>::template store<false, false>(up, p0, rs, cg, S[t]);
  }
}

// ---- the decode step, quantized state (DAMP, uniform INT8): two passes over the codes ------
// The state stays in VGPRs in its stored, compressed form (~40 registers per lane at d = 128
// with two waves per unit) rather than as fp32 values: pass 1 decodes it into the column sums
// u = S'^T k and p = S'^T q (the row multiplier folded into k and q per row), pass 2 decodes it
// again row step by row step to form X = S' + k delta^T, requantize and store. The second
// decode costs about one VALU instruction per element; the registers it frees let twice as
// many units share a CU, which is what keeps enough bytes in flight to HBM.
// LDS of the quantized step.
template <int D, int NW>
struct StepSmem {
  float4 srow[D];
  float sv[D];               // v, then delta
  float redu[4 * NW][D];
  float redp[4 * NW][D];
  float redqk[NW];
  float ssc[D];              // new INT8 row scales, storage order
};

// The step for one unit (ua) of workgroup bh = b * H + head. PLAN_FIXED: r = NF * RPS.
template <int D, int PER_KEY, int BF16, int PLAN, int WAVES, int NF>
__device__ __forceinline__ void step_q_unit(const StepArgs& a, const UnitAddr& ua, int bh, int head,
                                            StepSmem<D, Geo<D, WAVES>::NW>& sm) {
  using G = Geo<D, WAVES>;
  constexpr int T16 = PLAN == PLAN_FIXED ? NF : G::T16;
  constexpr int CPL = G::CPL, RPL = G::RPL, RW = Words<CPL * 2>::W;
  float4* srow = sm.srow;
  float* sv = sm.sv;
  float* ssc = sm.ssc;

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int r = PLAN == PLAN_FIXED ? NF * G::RPS : ua.r;
  // one buffer resource over a contiguous block unless a row step mixes kinds
  const UnitPtr up = (PLAN != PLAN_ANY && a.st.contiguous) ? unit_ptr<D, FMT_Q, true>(ua, r)
                                                           : unit_ptr<D, FMT_Q>(ua, r);

  // (1) the staging loads (per-row scalars, v), then every state load of this lane, so the
  // whole block is in flight while the staging completes
  Stage<D, G::NT, PER_KEY, BF16, true> sg;
  sg.load(a, reinterpret_cast<const float*>(ua.s), bh, head, r, tid);
  uint32_t raw[RPL][RW];
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = t * G::RPS + w * 4;
    by_plan<PLAN, T16>(t, p0, r, [&]<int K>() __attribute__((always_inline)) {
      load_row_step<D, K>(up, p0, rs, cg, raw[t]);
    });
  }

  // (2) per-row scalars and v into LDS
  const float beta = sg.store(a, tid, srow, sv, &sm.redu[0][0]);

  // (3) pass 1: u_j += (k_i m_i) c_ij, p_j += (q_i m_i) c_ij over the lane's rows. The lane's
  // rows are my_rows[t * RPS]: one LDS base address with immediate offsets per row step. Each
  // row step's raw words pass through an empty asm statement first: those keep their order, so
  // the compiler cannot hoist a later row step's decode (and the wait for its load) ahead of
  // the earlier ones, and the reduction follows the loads as they land.
  const float4* my_rows = srow + (w * 4 + rs);
  float pu[CPL], pp[CPL], pqk = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) pu[c] = pp[c] = 0.0f;
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = t * G::RPS + w * 4, p = p0 + rs;
    const float4 rw = my_rows[t * G::RPS];
    const float kk = rw.y * rw.x, qq = rw.z * rw.x;
    by_plan<PLAN, T16>(t, p0, r, [&]<int K>() __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float x = decode_row<D, K>(raw[t], c, p, r);
        pu[c] = fmaf(kk, x, pu[c]);
        pp[c] = fmaf(qq, x, pp[c]);
      }
    });
    pqk = fmaf(rw.z, rw.y, pqk);
    __builtin_amdgcn_sched_barrier(0);
  }

  // (4) column reductions, delta and the readout y = p + (q.k) delta (one thread per column)
  finish_columns<D, G>(sm.redu, sm.redp, sm.redqk, sv, pu, pp, pqk, beta,
                       a.out + int64_t(bh) * D, tid, w, rs, lane, cg);
  float dl[CPL];
  load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(sv + cg * CPL), reinterpret_cast<uint32_t*>(dl));

  // The raw words pass through an empty asm statement, so the compiler cannot keep pass 1's
  // decoded values (64 fp32 registers) alive across the reduction instead of decoding again.
#pragma unroll
  for (int t = 0; t < RPL; ++t)
#pragma unroll
    for (int i = 0; i < RW; ++i) asm volatile("" : "+v"(raw[t][i]));

  // (5) pass 2: X = m_i c_ij + k_i delta_j, requantize and store, one row step at a time
#pragma unroll
  for (int t = 0; t < RPL; ++t) {
    const int p0 = t * G::RPS + w * 4, p = p0 + rs;
    const float4 rw = my_rows[t * G::RPS];
    by_plan<PLAN, T16>(t, p0, r, [&]<int K>() __attribute__((always_inline)) {
      float X[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) X[c] = fmaf(rw.y, dl[c], decode_row<D, K>(raw[t], c, p, r) * rw.x);
      each_kind<K>([&]<int K2, bool MIX>() __attribute__((always_inline)) {
        Row<D, K2>::template store<false, MIX, true>(up, p0, rs, cg, X, ssc);
      });
    });
  }
  flush_scales<D, G::NT>(up, ssc, r, tid);
}

template <int D, int PER_KEY, int BF16, int PLAN, int WAVES, int NF = 0>
__global__ __launch_bounds__(64 * WAVES) void step_kernel_q(const StepArgs a) {
  __shared__ StepSmem<D, Geo<D, WAVES>::NW> sm;
  int b, head;
  if (!unit_of(a, b, head)) return;
  const int bh = b * a.H + head;
  const int64_t slot = a.slot_idx[b];
  const UnitAddr ua = unit_addr<D, FMT_Q>(a.st, slot, head, a.H);   // arithmetic only
  if (!slot_in_pool(slot, a.st.num_slots)) return;
  step_q_unit<D, PER_KEY, BF16, PLAN, WAVES, NF>(a, ua, bh, head, sm);
}

// Per-head DAMP layout whose every r is a multiple of the row step and at most T16 row steps:
// the row kinds are fixed at compile time per r, chosen by a wave-uniform branch on the head's r.
template <int D, int PER_KEY, int BF16, int WAVES, int NF>
__device__ __forceinline__ void step_q_heads_case(const StepArgs& a, const UnitAddr& ua, int bh,
                                                  int head, StepSmem<D, Geo<D, WAVES>::NW>& sm) {
  if constexpr (NF >= 0) {
    if (ua.r == NF * Geo<D, WAVES>::RPS)
      step_q_unit<D, PER_KEY, BF16, PLAN_FIXED, WAVES, NF>(a, ua, bh, head, sm);
    else
      step_q_heads_case<D, PER_KEY, BF16, WAVES, NF - 1>(a, ua, bh, head, sm);
  }
}

template <int D, int PER_KEY, int BF16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void step_kernel_q_heads(const StepArgs a) {
  __shared__ StepSmem<D, Geo<D, WAVES>::NW> sm;
  int b, head;
  if (!unit_of(a, b, head)) return;
  const int bh = b * a.H + head;
  const int64_t slot = a.slot_idx[b];
  const UnitAddr ua = unit_addr<D, FMT_Q>(a.st, slot, head, a.H);   // arithmetic only
  if (!slot_in_pool(slot, a.st.num_slots)) return;
  step_q_heads_case<D, PER_KEY, BF16, WAVES, Geo<D, WAVES>::T16>(a, ua, bh, head, sm);
}

// ---- pack: fp32 states (original key order) -> quantized format (exact rule) -------------
template <int D, int PLAN>
__global__ __launch_bounds__(Geo<D>::NT) void quantize_kernel(const PackArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL;
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int ih = __builtin_amdgcn_workgroup_id_x();  // i * H + head
  const int i = ih / a.H;
  const int head = ih - i * a.H;
  const int64_t slot = a.slot_idx[i];
  const UnitAddr ua = unit_addr<D, FMT_Q>(a.st, slot, head, a.H);   // arithmetic only
  if (!slot_in_pool(slot, a.st.num_slots)) return;
  const int r = ua.r;
  const UnitPtr up = unit_ptr<D, FMT_Q>(ua, r);
#pragma unroll
  for (int t = 0; t < G::RPL; ++t) {
    const int p0 = t * G::RPS + w * 4, p = p0 + rs;
    const int src = a.st.rowmap ? a.st.rowmap[head * D + p] : p;
    float x[CPL];
    load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(a.S + (int64_t(ih) * D + src) * D + cg * CPL),
                        reinterpret_cast<uint32_t*>(x));
    by_plan<PLAN>(t, p0, r, [&]<int K>() __attribute__((always_inline)) {
      each_kind<K>([&]<int K2, bool MIX>() __attribute__((always_inline)) {
        Row<D, K2>::template store<true, MIX>(up, p0, rs, cg, x);
      });
    });
  }
}

// ---- unpack: quantized format -> fp32 states (original key order) -----------------------
template <int D, int PLAN>
__global__ __launch_bounds__(Geo<D>::NT) void dequantize_kernel(const PackArgs a) {
  using G = Geo<D>;
  constexpr int CPL = G::CPL;
  const int tid = __builtin_amdgcn_workitem_id_x();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int ih = __builtin_amdgcn_workgroup_id_x();
  const int i = ih / a.H;
  const int head = ih - i * a.H;
  const int64_t slot = a.slot_idx[i];
  const UnitAddr ua = unit_addr<D, FMT_Q>(a.st, slot, head, a.H);   // arithmetic only
  if (!slot_in_pool(slot, a.st.num_slots)) return;
  const int r = ua.r;
  const UnitPtr up = unit_ptr<D, FMT_Q>(ua, r);
#pragma unroll
  for (int t = 0; t < G::RPL; ++t) {
    const int p0 = t * G::RPS + w * 4, p = p0 + rs;
    const int src = a.st.rowmap ? a.st.rowmap[head * D + p] : p;
    const float sc = p < r ? 1.0f : reinterpret_cast<const float*>(ua.s)[p - r];
    float x[CPL];
    by_plan<PLAN>(t, p0, r, [&]<int K>() __attribute__((always_inline)) {
      uint32_t raw[Words<CPL * 2>::W];
      load_row_step<D, K>(up, p0, rs, cg, raw);
#pragma unroll
      for (int c = 0; c < CPL; ++c) x[c] = decode_row<D, K>(raw, c, p, r) * sc;
    });
    store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(a.S + (int64_t(ih) * D + src) * D + cg * CPL),
                         reinterpret_cast<const uint32_t*>(x));
  }
}

// ---- launchers -------------------------------------------------------------------------------
// r = NF * RPS FP16 rows, NF <= T16: the instance for that NF.
template <int D, int PER_KEY, int BF16, int NF>
bool launch_step_fixed(int nf, const StepArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (NF < 0) {
    return false;
  } else {
    if (nf == NF) {
      hipLaunchKernelGGL((step_kernel_q<D, PER_KEY, BF16, PLAN_FIXED, kWaves<D>, NF>), grid,
                         dim3(64 * kWaves<D>), 0, s, a);
      return true;
    }
    return launch_step_fixed<D, PER_KEY, BF16, NF - 1>(nf, a, grid, s);
  }
}

// Instance choice by r: the row kinds fixed at compile time when r is a multiple of the row
// step (the usual layouts: r in {0, 8, 16, 24, 32} at d = 128); else PLAN_SMALL (r % 4 == 0,
// r <= 32 at d = 128) with the default workgroup shape; else the general instance.
template <int D, int PER_KEY, int BF16>
void launch_step_q(const StepArgs& a, dim3 grid, hipStream_t s) {
  using GS = Geo<D, kWaves<D>>;
  using G = Geo<D>;
  if (a.st.heads) {
    // per-head r: every r a multiple of the row step and <= T16 row steps -> compile-time row
    // kinds with a branch on the head's r; otherwise the general instance
    if (a.st.heads_r_or % GS::RPS == 0 && a.st.heads_r_max <= GS::T16 * GS::RPS)
      hipLaunchKernelGGL((step_kernel_q_heads<D, PER_KEY, BF16, kWaves<D>>), grid, dim3(GS::NT), 0, s, a);
    else
      hipLaunchKernelGGL((step_kernel_q<D, PER_KEY, BF16, PLAN_ANY, G::NW>), grid, dim3(G::NT), 0, s, a);
    return;
  }
  const int r = a.st.r;
  if (r % GS::RPS == 0 && r <= GS::T16 * GS::RPS &&
      launch_step_fixed<D, PER_KEY, BF16, GS::T16>(r / GS::RPS, a, grid, s))
    return;
  if (r % 4 == 0 && r <= G::T16 * G::RPS)
    hipLaunchKernelGGL((step_kernel_q<D, PER_KEY, BF16, PLAN_SMALL, G::NW>), grid, dim3(G::NT), 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel_q<D, PER_KEY, BF16, PLAN_ANY, G::NW>), grid, dim3(G::NT), 0, s, a);
}

template <int D, int PER_KEY, int BF16>
void launch_step_dt(int fmt, const StepArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H));
  if (fmt == FMT_F32)
    hipLaunchKernelGGL((step_kernel_f32<D, PER_KEY, BF16>), grid, dim3(Geo<D>::NT), 0, s, a);
  else
    launch_step_q<D, PER_KEY, BF16>(a, grid, s);
}

template <int D>
hipError_t step_d(int fmt, int per_key, int bf16, const StepArgs& a, hipStream_t s) {
  if (per_key) {
    if (bf16) launch_step_dt<D, 1, 1>(fmt, a, s); else launch_step_dt<D, 1, 0>(fmt, a, s);
  } else {
    if (bf16) launch_step_dt<D, 0, 1>(fmt, a, s); else launch_step_dt<D, 0, 0>(fmt, a, s);
  }
  return hipGetLastError();
}

template <int D>
hipError_t quant_d(const PackArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.n) * unsigned(a.H)), block(Geo<D>::NT);
  if ((a.st.heads ? a.st.heads_r_or : a.st.r) % 4 == 0)
    hipLaunchKernelGGL((quantize_kernel<D, PLAN_R4>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<D, PLAN_ANY>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t dequant_d(const PackArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.n) * unsigned(a.H)), block(Geo<D>::NT);
  if ((a.st.heads ? a.st.heads_r_or : a.st.r) % 4 == 0)
    hipLaunchKernelGGL((dequantize_kernel<D, PLAN_R4>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((dequantize_kernel<D, PLAN_ANY>), grid, block, 0, s, a);
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
