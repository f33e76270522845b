// window_kernels.hip -- gfx950 kernels of per-window requantization (window step and flush) on
// the DAMP layouts; building blocks in step_common.h.
#include "step_common.h"

namespace damp {
namespace {

// ---- per-window requantization ------------------------------------------------------------
// The LeapQuant page: the low-bit state stays fixed for a window of tokens, the window's updates
// are held in high precision, outputs come from both, and the state is quantized once at the
// window's end. Within a window the state of a unit is
//   S = diag(a) S_hat + sum_{tau < t} K_tau E_tau^T
// with S_hat the stored (DAMP) state, a its cumulative row decay and (K_tau, E_tau) one fp32 key
// vector (decayed as the window goes on) and one delta per token. A token's step decays a and
// every K_tau by the gate, reads S_hat once (pass 1 with row multiplier scale * a'), adds the
// buffered terms to u and p, and appends (k, delta); the state block is not written. The
// window's last token also materialises X = diag(a') S_hat + sum K'_tau E_tau^T + k delta^T,
// requantizes it in place and empties the buffer.
// With one gate per unit (GDN) every row decays alike, so a is one number and the decay of K_tau
// is one number c_tau: the keys are stored as appended and only the scalars change per token
// (with a gate per key row, KDA, a and every K_tau are rewritten decayed).
//
// Window buffer of one unit, fp32 words at a.win + (slot * H + head) * a.win_stride bytes:
//   [0]            t, the tokens applied in the current window (int32; 0 = empty, a = 1)
//   [1]            scalar gate: a, the product of the window's gates so far
//   [2]            1 for a window with a scalar gate (written by its tokens), 0 for per-row gates
//   [4, 4 + D)     per-row gates: a, storage row order
//                  scalar gate: [4, 4 + W) c[tau], the product of the gates after token tau
//   [4 + D, ..)    K[tau][p], tau < W, storage row order (per-row gates: decayed; scalar gate:
//                  as appended)
//   then           E[tau][j], tau < W
constexpr int kMaxWindow = 8;

template <int D, int NW>
struct WinSmem {
  static constexpr int RR = 4 * NW > kMaxWindow ? 4 * NW : kMaxWindow;
  float4 srow[D];            // {m_p = scale * a'_p, k_p, q_p, gate_p}
  float sv[D];               // v, then delta
  float redu[RR][D];         // column partials; at the window's end E[tau][j]
  float redp[RR][D];         // column partials; at the window's end K'[tau][p]
  float redqk[NW];
  float ssc[D];
  float sdot[NW][kMaxWindow][2];   // per wave: K'_tau . k and K'_tau . q
};

struct WinPtr {
  int32_t* hdr;
  float* A;   // per-row gates: a; scalar gate: c[tau] (the same words)
  float* K;
  float* E;
};

template <int D>
__device__ __forceinline__ WinPtr win_ptr(const StepArgs& a, int64_t slot, int head) {
  float* wb = reinterpret_cast<float*>(a.win + (slot * a.H + head) * a.win_stride);
  return WinPtr{reinterpret_cast<int32_t*>(wb), wb + 4, wb + 4 + D, wb + 4 + D + a.window * D};
}

// Whether the unit's window holds the scalar-gate form: a step knows it from its gate; a flush
// (no token, no gate) reads the flag its tokens left.
template <int PER_KEY, bool FLUSH_ONLY>
__device__ __forceinline__ bool win_scalar(const WinPtr& wp, int t) {
  if constexpr (!FLUSH_ONLY) return !PER_KEY;
  return t > 0 && __builtin_amdgcn_readfirstlane(wp.hdr[2]) == 1;
}

// Staging of a window step (FLUSH_ONLY = false) or of a flush with no token (true). As
// stage_rows, plus: a'_p = gate_p * a_p (a = 1 when the window is empty), srow.x = scale * a'_p,
// srow.w = gate_p; every buffered key decayed, K'_tau,p = gate_p K_tau,p, and its dot products
// with k and q summed per wave into sdot. Unless the window ends here, a' and K' go back to the
// buffer. Scalar gate (scal): a' = gate a and K'_tau = c'_tau K_tau with c'_tau = gate c_tau,
// so the dot products are c'_tau (K_tau . k); a', c' and c[t] = 1 go back to the header words.
// Returns beta.
template <int D, int NT, int PER_KEY, int BF16, bool FLUSH_ONLY>
__device__ __forceinline__ float stage_rows_win(const StepArgs& a, const WinPtr& wp, int t,
                                                bool ends, const float* sc_old, int bh, int head,
                                                int r, int tid, float4* srow, float* sv,
                                                float* tmp, float (*sdot)[kMaxWindow][2],
                                                bool scal) {
  const int64_t vec = int64_t(bh) * D;
  constexpr int PER = (D + NT - 1) / NT;
  constexpr int NWS = NT / 64;
  const bool pre = !FLUSH_ONLY && a.prestep != 0;
  int src[PER];
  float sc[PER];
  float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
  for (int n = 0; n < PER; ++n) {
    const int i = tid + n * NT;
    if (i < D) {
      src[n] = a.st.rowmap ? a.st.rowmap[head * D + i] : i;
      sc[n] = i >= r ? sc_old[i - r] : 1.0f;
      if constexpr (!FLUSH_ONLY) {
        const float kv = load_in<BF16>(a.k, vec + i), qv = load_in<BF16>(a.q, vec + i);
        tmp[i] = kv;
        tmp[D + i] = qv;
        ssk = fmaf(kv, kv, ssk);
        ssq = fmaf(qv, qv, ssq);
        if constexpr (PER_KEY) tmp[2 * D + i] = pre ? gate_from_logit(a.alpha[vec + i]) : a.alpha[vec + i];
        sv[i] = load_in<BF16>(a.v, vec + i);
      }
    }
  }
  float g0 = 1.0f, beta = 0.0f;
  if constexpr (!FLUSH_ONLY) {
    g0 = PER_KEY ? 0.0f : a.alpha[bh];
    beta = a.beta[bh];
    if (pre) {
      if constexpr (!PER_KEY) g0 = gate_from_logit(g0);
      beta = 1.0f / (1.0f + expf(-beta));
      ssq = wave_sum(ssq);
      ssk = wave_sum(ssk);
      if ((tid & 63) == 0) {
        tmp[3 * D + 2 * (tid >> 6)] = ssq;
        tmp[3 * D + 2 * (tid >> 6) + 1] = ssk;
      }
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
  // scalar gate: the gate of this token (1 for a flush) and the window's product before it
  const float gs = FLUSH_ONLY ? 1.0f : g0;
  const float as = scal && t > 0 ? __int_as_float(__builtin_amdgcn_readfirstlane(wp.hdr[1])) : 1.0f;
  float kh[PER], qh[PER], gt[PER];
#pragma unroll
  for (int n = 0; n < PER; ++n) {
    const int i = tid + n * NT;
    kh[n] = qh[n] = 0.0f;
    gt[n] = 1.0f;
    if (i < D) {
      if constexpr (!FLUSH_ONLY) {
        gt[n] = PER_KEY ? tmp[2 * D + src[n]] : g0;
        kh[n] = tmp[src[n]] * invk;
        qh[n] = tmp[D + src[n]] * invq;
      }
      const float ap = scal ? gs * as : gt[n] * (t > 0 ? wp.A[i] : 1.0f);
      srow[i] = make_float4(sc[n] * ap, kh[n], qh[n], gt[n]);
      if (!FLUSH_ONLY && !ends && !scal) wp.A[i] = ap;
    }
  }
  if constexpr (!FLUSH_ONLY) {
    for (int tau = 0; tau < t; ++tau) {
      float ck = 0.0f, cq = 0.0f;
#pragma unroll
      for (int n = 0; n < PER; ++n) {
        const int i = tid + n * NT;
        if (i < D) {
          const float kb = wp.K[tau * D + i];
          const float kd = scal ? kb : gt[n] * kb;
          if (!scal && !ends) wp.K[tau * D + i] = kd;
          ck = fmaf(kd, kh[n], ck);
          cq = fmaf(kd, qh[n], cq);
        }
      }
      ck = wave_sum(ck);
      cq = wave_sum(cq);
      if (scal) {
        const float cf = gs * __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wp.A[tau])));
        ck *= cf;
        cq *= cf;
      }
      if ((tid & 63) == 0) {
        sdot[tid >> 6][tau][0] = ck;
        sdot[tid >> 6][tau][1] = cq;
      }
    }
  }
  __syncthreads();
  // scalar gate: every wave has read the old words above; the next token's words go back now
  if (!FLUSH_ONLY && scal && !ends && tid == 0) {
    for (int tau = 0; tau < t; ++tau) wp.A[tau] = gs * wp.A[tau];
    wp.A[t] = 1.0f;
    wp.hdr[1] = __float_as_int(gs * as);
    wp.hdr[2] = 1;
  }
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(beta)));
}

// finish_columns plus the buffered terms: u_j += sum_tau E_tau,j (K'_tau . k),
// p_j += sum_tau E_tau,j (K'_tau . q). Unless the window ends here, delta goes to E[t].
template <int D, typename G>
__device__ __forceinline__ void finish_columns_win(float (*redu)[D], float (*redp)[D], float* redqk,
                                                   float (*sdot)[kMaxWindow][2], const WinPtr& wp,
                                                   int t, bool ends, float* sv, float* pu, float* pp,
                                                   float pqk, float beta, float* out_row, int tid,
                                                   int w, int rs, int lane, int cg) {
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
    }
    for (int tau = 0; tau < t; ++tau) {
      float ck = sdot[0][tau][0], cq = sdot[0][tau][1];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) {
        ck += sdot[w2][tau][0];
        cq += sdot[w2][tau][1];
      }
      const float e = wp.E[tau * D + j];
      uu = fmaf(e, ck, uu);
      pv = fmaf(e, cq, pv);
    }
    float qk = redqk[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) qk += redqk[w2];
    const float dj = beta * (sv[j] - uu);
    sv[j] = dj;
    out_row[j] = fmaf(qk, dj, pv);
    if (!ends) wp.E[t * D + j] = dj;
  }
  __syncthreads();
}

// One window step (FLUSH_ONLY = false) or one flush (true) of a unit.
template <int D, int PER_KEY, int BF16, int PLAN, int WAVES, int NF, bool FLUSH_ONLY>
__device__ __forceinline__ void window_q_unit(const StepArgs& a, const UnitAddr& ua, int64_t slot,
                                              int bh, int head, WinSmem<D, Geo<D, WAVES>::NW>& sm) {
  using G = Geo<D, WAVES>;
  constexpr int T16 = PLAN == PLAN_FIXED ? NF : G::T16;
  constexpr int CPL = G::CPL, RPL = G::RPL, RW = Words<CPL * 2>::W;
  const WinPtr wp = win_ptr<D>(a, slot, head);
  const int t = __builtin_amdgcn_readfirstlane(*wp.hdr);
  if (FLUSH_ONLY && t == 0) return;   // nothing pending (uniform over the workgroup)
  const bool ends = FLUSH_ONLY || t + 1 >= a.window;
  const bool scal = win_scalar<PER_KEY, FLUSH_ONLY>(wp, t);
  float4* srow = sm.srow;
  float* sv = sm.sv;
  float* ssc = sm.ssc;

  const int tid = __builtin_amdgcn_workitem_id_x();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, rs = lane >> 4, cg = lane & 15;
  const int r = PLAN == PLAN_FIXED ? NF * G::RPS : ua.r;
  const UnitPtr up = (PLAN != PLAN_ANY && a.st.contiguous) ? unit_ptr<D, FMT_Q, true>(ua, r)
                                                           : unit_ptr<D, FMT_Q>(ua, r);
  uint32_t raw[RPL][RW];
#pragma unroll
  for (int tt = 0; tt < RPL; ++tt) {
    const int p0 = tt * G::RPS + w * 4;
    by_plan<PLAN, T16>(tt, p0, r, [&]<int K>() __attribute__((always_inline)) {
      load_row_step<D, K>(up, p0, rs, cg, raw[tt]);
    });
  }
  const float beta = stage_rows_win<D, G::NT, PER_KEY, BF16, FLUSH_ONLY>(
      a, wp, t, ends, reinterpret_cast<const float*>(ua.s), bh, head, r, tid, srow, sv,
      &sm.redu[0][0], sm.sdot, scal);
  const float4* my_rows = srow + (w * 4 + rs);

  int terms = t;   // buffered terms in X at the window's end (the token's own one included)
  if constexpr (!FLUSH_ONLY) {
    // pass 1 on the stored state with row multiplier scale * a'
    float pu[CPL], pp[CPL], pqk = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) pu[c] = pp[c] = 0.0f;
#pragma unroll
    for (int tt = 0; tt < RPL; ++tt) {
      const int p0 = tt * G::RPS + w * 4, p = p0 + rs;
      const float4 rw = my_rows[tt * G::RPS];
      const float kk = rw.y * rw.x, qq = rw.z * rw.x;
      by_plan<PLAN, T16>(tt, p0, r, [&]<int K>() __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float x = decode_row<D, K>(raw[tt], c, p, r);
          pu[c] = fmaf(kk, x, pu[c]);
          pp[c] = fmaf(qq, x, pp[c]);
        }
      });
      pqk = fmaf(rw.z, rw.y, pqk);
    }
    finish_columns_win<D, G>(sm.redu, sm.redp, sm.redqk, sm.sdot, wp, t, ends, sv, pu, pp, pqk,
                             beta, a.out + int64_t(bh) * D, tid, w, rs, lane, cg);
    if (!ends) {
      // append the token's key (storage order) and count it; the stored state stays as it is
      for (int i = tid; i < D; i += G::NT) wp.K[t * D + i] = srow[i].y;
      if (tid == 0) *wp.hdr = t + 1;
      return;
    }
    terms = t + 1;
  }
  // the window ends: E[tau][j] and K'[tau][p] of every buffered term into LDS (the token's own
  // term last: its key and delta)
  for (int x = tid; x < terms * D; x += G::NT) {
    const int tau = x / D, i = x - tau * D;
    if (!FLUSH_ONLY && tau == t) {
      sm.redu[tau][i] = sv[i];
      sm.redp[tau][i] = srow[i].y;
    } else {
      sm.redu[tau][i] = wp.E[tau * D + i];
      // K'_tau,p: per-row gates gate_p K_tau,p (K decayed up to the previous token); scalar
      // gate (gate c_tau) K_tau,p with the key as appended
      const float g = scal ? srow[i].w * wp.A[tau] : srow[i].w;
      sm.redp[tau][i] = g * wp.K[tau * D + i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < RPL; ++tt)
#pragma unroll
    for (int i = 0; i < RW; ++i) asm volatile("" : "+v"(raw[tt][i]));
  // X = m_p c_pj + sum_tau K'_tau,p E_tau,j, requantized and stored in place
#pragma unroll
  for (int tt = 0; tt < RPL; ++tt) {
    const int p0 = tt * G::RPS + w * 4, p = p0 + rs;
    const float m = my_rows[tt * G::RPS].x;
    by_plan<PLAN, T16>(tt, p0, r, [&]<int K>() __attribute__((always_inline)) {
      float X[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) X[c] = decode_row<D, K>(raw[tt], c, p, r) * m;
      for (int tau = 0; tau < terms; ++tau) {
        const float kp = sm.redp[tau][p];
        float e[CPL];
        load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(&sm.redu[tau][cg * CPL]),
                            reinterpret_cast<uint32_t*>(e));
#pragma unroll
        for (int c = 0; c < CPL; ++c) X[c] = fmaf(kp, e[c], X[c]);
      }
      each_kind<K>([&]<int K2, bool MIX>() __attribute__((always_inline)) {
        Row<D, K2>::template store<false, MIX, true>(up, p0, rs, cg, X, ssc);
      });
    });
  }
  flush_scales<D, G::NT>(up, ssc, r, tid);
  if (tid == 0) *wp.hdr = 0;
}

template <int D, int PER_KEY, int BF16, int WAVES, int NF, bool FLUSH_ONLY>
__device__ __forceinline__ void window_heads_case(const StepArgs& a, const UnitAddr& ua, int64_t slot,
                                                  int bh, int head, WinSmem<D, Geo<D, WAVES>::NW>& sm) {
  if constexpr (NF >= 0) {
    if (ua.r == NF * Geo<D, WAVES>::RPS)
      window_q_unit<D, PER_KEY, BF16, PLAN_FIXED, WAVES, NF, FLUSH_ONLY>(a, ua, slot, bh, head, sm);
    else
      window_heads_case<D, PER_KEY, BF16, WAVES, NF - 1, FLUSH_ONLY>(a, ua, slot, bh, head, sm);
  }
}

// HEADS: per-head layout whose r are all multiples of the row step (kinds fixed per head's r).
template <int D, int PER_KEY, int BF16, int PLAN, int WAVES, int NF, bool FLUSH_ONLY, bool HEADS>
__global__ __launch_bounds__(64 * WAVES) void window_kernel(const StepArgs a) {
  __shared__ WinSmem<D, Geo<D, WAVES>::NW> sm;
  int b, head;
  if (!unit_of(a, b, head)) return;
  const int bh = b * a.H + head;
  const int64_t slot = a.slot_idx[b];
  const UnitAddr ua = unit_addr<D, FMT_Q>(a.st, slot, head, a.H);
  if constexpr (HEADS)
    window_heads_case<D, PER_KEY, BF16, WAVES, Geo<D, WAVES>::T16, FLUSH_ONLY>(a, ua, slot, bh, head, sm);
  else
    window_q_unit<D, PER_KEY, BF16, PLAN, WAVES, NF, FLUSH_ONLY>(a, ua, slot, bh, head, sm);
}

// Window kernels: at d = 128 the compile-time row-kind instances (uniform r a multiple of the row
// step, or a per-head layout whose r all are), else the general instance; smaller d always use
// the general instance. A flush has no token, so one gate / input-type instance serves it.
template <int D, int PER_KEY, int BF16, bool FLUSH_ONLY, int NF>
bool launch_window_fixed(int nf, const StepArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (NF < 0) {
    return false;
  } else {
    if (nf == NF) {
      hipLaunchKernelGGL((window_kernel<D, PER_KEY, BF16, PLAN_FIXED, kWaves<D>, NF, FLUSH_ONLY, false>),
                         grid, dim3(64 * kWaves<D>), 0, s, a);
      return true;
    }
    return launch_window_fixed<D, PER_KEY, BF16, FLUSH_ONLY, NF - 1>(nf, a, grid, s);
  }
}

template <int D, int PER_KEY, int BF16, bool FLUSH_ONLY>
void launch_window_q(const StepArgs& a, dim3 grid, hipStream_t s) {
  using G = Geo<D>;
  if constexpr (D == 128) {
    using GS = Geo<D, kWaves<D>>;
    if (a.st.heads) {
      if (a.st.heads_r_or % GS::RPS == 0 && a.st.heads_r_max <= GS::T16 * GS::RPS) {
        hipLaunchKernelGGL((window_kernel<D, PER_KEY, BF16, PLAN_FIXED, kWaves<D>, 0, FLUSH_ONLY, true>),
                           grid, dim3(GS::NT), 0, s, a);
        return;
      }
    } else if (a.st.r % GS::RPS == 0 && a.st.r <= GS::T16 * GS::RPS &&
               launch_window_fixed<D, PER_KEY, BF16, FLUSH_ONLY, GS::T16>(a.st.r / GS::RPS, a, grid, s)) {
      return;
    }
  }
  hipLaunchKernelGGL((window_kernel<D, PER_KEY, BF16, PLAN_ANY, G::NW, 0, FLUSH_ONLY, false>), grid,
                     dim3(G::NT), 0, s, a);
}

template <int D>
hipError_t window_d(int per_key, int bf16, bool flush_only, const StepArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H));
  if (flush_only) {
    launch_window_q<D, 0, 0, true>(a, grid, s);
  } else if (per_key) {
    if (bf16) launch_window_q<D, 1, 1, false>(a, grid, s); else launch_window_q<D, 1, 0, false>(a, grid, s);
  } else {
    if (bf16) launch_window_q<D, 0, 1, false>(a, grid, s); else launch_window_q<D, 0, 0, false>(a, grid, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_window(int d, int per_key, int bf16, bool flush_only, const StepArgs& a,
                         hipStream_t s) {
  switch (d) {
    case 16: return window_d<16>(per_key, bf16, flush_only, a, s);
    case 32: return window_d<32>(per_key, bf16, flush_only, a, s);
    case 64: return window_d<64>(per_key, bf16, flush_only, a, s);
    case 128: return window_d<128>(per_key, bf16, flush_only, a, s);
    default: return hipErrorInvalidValue;
  }
}

int window_max() { return kMaxWindow; }

}  // namespace damp
