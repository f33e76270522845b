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
//   [2]            1 for a window with a scalar gate, 0 for per-row gates (written by every
//                  token that leaves the window open; cleared when the window ends)
//   [3]            scalar gate: bit tau set when K[tau] is stored as bf16 (the first 2 D bytes
//                  of its row): the key of a call with bf16 inputs and no fused pre-step is a
//                  bf16 value, so it is stored exactly in half the bytes; 0 otherwise
//   [4, 4 + D)     per-row gates: a, storage row order
//                  scalar gate: [4, 4 + W) c[tau], the product of the gates after token tau
//   [4 + D, ..)    K[tau][p], tau < W, storage row order (per-row gates: decayed; scalar gate:
//                  as appended, fp32 or bf16 by word [3])
//   then           E[tau][j], tau < W
constexpr int kMaxWindow = 8;

template <int D, int NW>
struct WinSmem {
  float4 srow[D];            // {m_p = scale * a'_p, k_p, q_p, gate_p}
  float sv[D];               // v, then delta
  union {
    struct {
      float redu[4 * NW][D];   // column partials
      float redp[4 * NW][D];
    };
    float skT[D][kMaxWindow];  // at the window's end: every term's key, transposed
  };
  float se[kMaxWindow][D];   // the window's deltas E[tau][j] (the token's own last)
  float sk[kMaxWindow][D];   // the window's keys decayed to this token, K'[tau][p]
  float redqk[NW];
  float ssc[D];
  float sdot[kMaxWindow][2];  // K'_tau . k and K'_tau . q
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

// Staging of a window step (FLUSH_ONLY = false) or of a flush with no token (true), in two
// phases as the step's Stage. load() issues every small global load of the unit into registers,
// before the caller issues the state loads: the row map and old INT8 scales, k, q, the gate and v
// of the token, and of the t tokens already in the window their keys K[tau][i], their deltas
// E[tau][i] (column i) and the decay words (per-row gains a_i, or the scalars c[tau] and a).
// store() then stages as Stage::store does, plus: a'_p = gate_p * a_p (a = 1 when the window is
// empty), srow.x = scale * a'_p, srow.w = gate_p; every buffered key decayed, K'_tau,p =
// gate_p K_tau,p, and its dot products with k and q, all tokens' products first and then their
// wave sums side by side, summed per wave into sdot. Unless the window ends here, a' and K' go
// back to the buffer. Scalar gate (scal): a' = gate a and K'_tau = c'_tau K_tau with c'_tau =
// gate c_tau, so the dot products are c'_tau (K_tau . k); a', c' and c[t] = 1 go back to the
// header words. The buffered keys and deltas stay in registers for the column pass and for the
// window's end.
template <int D, int NT, int PER_KEY, int BF16, bool FLUSH_ONLY>
struct WinStage {
  static constexpr int PER = (D + NT - 1) / NT;
  static constexpr int NWS = NT / 64;
  static constexpr int WM = kMaxWindow;
  uint32_t src[PER], sc[PER], kv[PER], qv[PER], gv[PER], vv[PER];
  float A[PER], Eb[WM][PER], cA[WM];
  uint32_t Kb[WM][PER];   // the buffered keys' words as loaded (decoded in store())
  float g0, beta, as;
  uint32_t kbf;   // header word [3] of the window so far (scalar gate), else 0

  // hdr3: header word [3], read with the token count (so that its wait is the count's).
  __device__ __forceinline__ void load(const StepArgs& a, const WinPtr& wp, int t, bool scal,
                                       uint32_t hdr3, const float* sc_old, int bh, int head, int r,
                                       int tid) {
    const int64_t vec = int64_t(bh) * D;
    kbf = scal && t > 0 ? hdr3 : 0u;
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int i = tid + n * NT;
      src[n] = static_cast<uint32_t>(i);
      sc[n] = __float_as_uint(1.0f);
      kv[n] = qv[n] = gv[n] = vv[n] = 0u;
      A[n] = 1.0f;
#pragma unroll
      for (int tau = 0; tau < WM; ++tau) {
        Kb[tau][n] = 0u;
        Eb[tau][n] = 0.0f;
      }
      if (PER * NT == D || i < D) {
        if (a.st.rowmap) src[n] = a.st.rowmap[head * D + i];
        if (i >= r) sc[n] = reinterpret_cast<const uint32_t*>(sc_old)[i - r];
        if constexpr (!FLUSH_ONLY) {
          kv[n] = Stage<D, NT, PER_KEY, BF16, true>::template raw_in<BF16>(a.k, vec + i);
          qv[n] = Stage<D, NT, PER_KEY, BF16, true>::template raw_in<BF16>(a.q, vec + i);
          if constexpr (PER_KEY) gv[n] = reinterpret_cast<const uint32_t*>(a.alpha)[vec + i];
          vv[n] = Stage<D, NT, PER_KEY, BF16, true>::template raw_in<BF16>(a.v, vec + i);
        }
        if (!scal && t > 0) A[n] = wp.A[i];
#pragma unroll
        for (int tau = 0; tau < WM; ++tau)
          if (tau < t) {
            // one 4-byte load either way, kept as loaded: a bf16 row's element i is half i & 1
            // of its word i / 2 (no use of a loaded value here, so no wait before the state loads)
            const bool hb = (kbf >> tau) & 1u;
            Kb[tau][n] = reinterpret_cast<const uint32_t*>(wp.K + tau * D)[hb ? (i >> 1) : i];
            Eb[tau][n] = wp.E[tau * D + i];
          }
      }
    }
    g0 = FLUSH_ONLY ? 1.0f : (PER_KEY ? 0.0f : a.alpha[bh]);
    beta = FLUSH_ONLY ? 0.0f : a.beta[bh];
    as = scal && t > 0 ? __int_as_float(wp.hdr[1]) : 1.0f;
#pragma unroll
    for (int tau = 0; tau < WM; ++tau) cA[tau] = scal && tau < t ? wp.A[tau] : 1.0f;
  }

  __device__ __forceinline__ float store(const StepArgs& a, const WinPtr& wp, int t, bool ends,
                                         bool scal, int tid, float4* srow, float* sv, float* tmp,
                                         float (*sdot)[2], float (*se)[D], float (*sk)[D]) {
    // the loaded registers are used from here on: the caller's state loads are issued above
#pragma unroll
    for (int n = 0; n < PER; ++n)
      asm volatile("" : "+v"(src[n]), "+v"(sc[n]), "+v"(kv[n]), "+v"(qv[n]), "+v"(gv[n]), "+v"(vv[n]), "+v"(A[n]));
    const bool pre = !FLUSH_ONLY && a.prestep != 0;
    using S = Stage<D, NT, PER_KEY, BF16, true>;
    // the buffered terms to LDS first, so their registers are free from here on: E as stored,
    // K as fp32 from its stored form (decayed below, each thread its own entries)
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int i = tid + n * NT;
      if (PER * NT == D || i < D) {
#pragma unroll
        for (int tau = 0; tau < WM; ++tau)
          if (tau < t) {
            se[tau][i] = Eb[tau][n];
            sk[tau][i] = (kbf >> tau) & 1u ? __uint_as_float((i & 1) ? (Kb[tau][n] & 0xFFFF0000u) : (Kb[tau][n] << 16))
                                           : __uint_as_float(Kb[tau][n]);
          }
      }
    }
    float ssq = 0.0f, ssk = 0.0f;
    if constexpr (!FLUSH_ONLY) {
#pragma unroll
      for (int n = 0; n < PER; ++n) {
        const int i = tid + n * NT;
        if (PER * NT == D || i < D) {
          const float kf = S::widen(kv[n]), qf = S::widen(qv[n]), gf = __uint_as_float(gv[n]);
          tmp[i] = kf;
          tmp[D + i] = qf;
          ssk = fmaf(kf, kf, ssk);
          ssq = fmaf(qf, qf, ssq);
          if constexpr (PER_KEY) tmp[2 * D + i] = pre ? gate_from_logit(gf) : gf;
          sv[i] = S::widen(vv[n]);
        }
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
    // scalar gate: the gate of this token (1 for a flush) and the window's product before it
    const float gs = g;
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int i = tid + n * NT;
      if (PER * NT == D || i < D) {
        float gt = 1.0f, kh = 0.0f, qh = 0.0f;
        if constexpr (!FLUSH_ONLY) {
          gt = PER_KEY ? tmp[2 * D + src[n]] : g;
          kh = tmp[src[n]] * invk;
          qh = tmp[D + src[n]] * invq;
        }
        const float ap = scal ? gs * as : gt * A[n];
        srow[i] = make_float4(__uint_as_float(sc[n]) * ap, kh, qh, gt);
        if (!FLUSH_ONLY && !ends && !scal) wp.A[i] = ap;
        // the thread's own entries of the buffered keys, decayed to this token: per-row gates
        // gate_p K_tau,p (also written back unless the window ends); scalar gate c'_tau K_tau,p
#pragma unroll
        for (int tau = 0; tau < WM; ++tau)
          if (tau < t) {
            const float kd = (scal ? gs * cA[tau] : gt) * sk[tau][i];
            sk[tau][i] = kd;
            if (!FLUSH_ONLY && !ends && !scal) wp.K[tau * D + i] = kd;
          }
      }
    }
    __syncthreads();
    if constexpr (!FLUSH_ONLY) {
      // the dot products K'_tau . k and K'_tau . q: 16 lanes per token, each over every 16th
      // row, then a sum over the 16 lanes of a row of the wave
      constexpr int TPP = NT / 16;   // tokens per pass
      const int part = tid & 15;
#pragma unroll
      for (int t0 = 0; t0 < WM; t0 += TPP) {
        const int tau = t0 + (tid >> 4);
        float ck = 0.0f, cq = 0.0f;
        if (tau < t) {
#pragma unroll
          for (int i = part; i < D; i += 16) {
            const float4 rw = srow[i];
            ck = fmaf(sk[tau][i], rw.y, ck);
            cq = fmaf(sk[tau][i], rw.z, cq);
          }
        }
        ck = sum_row16(ck);
        cq = sum_row16(cq);
        if (part == 0 && tau < t) {
          sdot[tau][0] = ck;
          sdot[tau][1] = cq;
        }
      }
    }
    // scalar gate: every wave has read the old words (at its start); the next token's go back
    if (!FLUSH_ONLY && scal && !ends && tid == 0) {
#pragma unroll
      for (int tau = 0; tau < WM; ++tau)
        if (tau < t) wp.A[tau] = gs * cA[tau];
      wp.A[t] = 1.0f;
      wp.hdr[1] = __float_as_int(gs * as);
      wp.hdr[2] = 1;
    }
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bt)));
  }
};

// finish_columns plus the buffered terms: u_j += sum_tau E_tau,j (K'_tau . k),
// p_j += sum_tau E_tau,j (K'_tau . q), with E from the LDS copy the staging made. Unless the
// window ends here, delta goes to E[t].
template <int D, typename G>
__device__ __forceinline__ void finish_columns_win(float (*redu)[D], float (*redp)[D], float* redqk,
                                                   float (*sdot)[2], float (*se)[D],
                                                   const WinPtr& wp, int t, bool ends, float* sv,
                                                   float* pu, float* pp, float pqk, float beta,
                                                   float* out_row, int tid, int w, int rs, int lane,
                                                   int cg) {
  constexpr int CPL = G::CPL, NW = G::NW;
  store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(&redu[w * 4 + rs][cg * CPL]),
                       reinterpret_cast<const uint32_t*>(pu));
  store_bytes<CPL * 4>(reinterpret_cast<uint8_t*>(&redp[w * 4 + rs][cg * CPL]),
                       reinterpret_cast<const uint32_t*>(pp));
  pqk = sum_row_slots(pqk);
  if (lane == 0) redqk[w] = pqk;
  __syncthreads();
  for (int j = tid; j < D; j += G::NT) {
    {
      float uu = redu[0][j], pv = redp[0][j];
#pragma unroll
      for (int k = 1; k < 4 * NW; ++k) {
        uu += redu[k][j];
        pv += redp[k][j];
      }
#pragma unroll
      for (int tau = 0; tau < kMaxWindow; ++tau)
        if (tau < t) {
          uu = fmaf(se[tau][j], sdot[tau][0], uu);
          pv = fmaf(se[tau][j], sdot[tau][1], pv);
        }
      float qk = redqk[0];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) qk += redqk[w2];
      const float dj = beta * (sv[j] - uu);
      sv[j] = dj;
      out_row[j] = fmaf(qk, dj, pv);
      if (!ends) wp.E[t * D + j] = dj;
    }
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
  // A count outside [0, window) (a buffer that was never zero-filled, or one last used with
  // another window length) reads as an empty window: every term index then stays inside the
  // unit's buffer, and t = 0 reads nothing else from it.
  int t = __builtin_amdgcn_readfirstlane(wp.hdr[0]);
  if (t < 0 || t >= a.window) t = 0;
  const uint32_t hdr3 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wp.hdr[3]));
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
  // the staging loads (and the window's buffered terms), then every state load of this lane
  WinStage<D, G::NT, PER_KEY, BF16, FLUSH_ONLY> ws;
  ws.load(a, wp, t, scal, hdr3, reinterpret_cast<const float*>(ua.s), bh, head, r, tid);
  uint32_t raw[RPL][RW];
#pragma unroll
  for (int tt = 0; tt < RPL; ++tt) {
    const int p0 = tt * G::RPS + w * 4;
    by_plan<PLAN, T16>(tt, p0, r, [&]<int K>() __attribute__((always_inline)) {
      load_row_step<D, K>(up, p0, rs, cg, raw[tt]);
    });
  }
  const float beta = ws.store(a, wp, t, ends, scal, tid, srow, sv, &sm.redu[0][0], sm.sdot, sm.se, sm.sk);
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
    finish_columns_win<D, G>(sm.redu, sm.redp, sm.redqk, sm.sdot, sm.se, wp, t, ends, sv, pu, pp, pqk,
                             beta, a.out + int64_t(bh) * D, tid, w, rs, lane, cg);
    if (!ends) {
      // append the token's key (storage order) and count it; the stored state stays as it is.
      // With a scalar gate the key is kept as given: from bf16 inputs without the fused pre-step
      // it is a bf16 value, stored exactly in 2 bytes.
      const bool kb = BF16 && scal && a.prestep == 0;
      for (int i = tid; i < D; i += G::NT) {
        if (kb)
          reinterpret_cast<uint16_t*>(wp.K + t * D)[i] = static_cast<uint16_t>(__float_as_uint(srow[i].y) >> 16);
        else
          wp.K[t * D + i] = srow[i].y;
      }
      if (tid == 0) {
        wp.hdr[0] = t + 1;
        if (!scal) wp.hdr[2] = 0;   // per-row gates (the scalar form set its flag in staging)
        wp.hdr[3] = (ws.kbf & ~(1u << t)) | (kb ? 1u << t : 0u);
      }
      return;
    }
    terms = t + 1;
  }
  // The window ends. Every term's key goes to LDS transposed, skT[p][tau] (zero past the last
  // term), over the column partials, which nothing reads any more; the token's own delta joins
  // the buffered ones.
  float (*skT)[kMaxWindow] = sm.skT;
  for (int i = tid; i < D; i += G::NT) {
    float kt[kMaxWindow];
#pragma unroll
    for (int tau = 0; tau < kMaxWindow; ++tau)
      kt[tau] = tau < t ? sm.sk[tau][i] : (!FLUSH_ONLY && tau == t ? srow[i].y : 0.0f);
    store_bytes<4 * kMaxWindow>(reinterpret_cast<uint8_t*>(skT[i]), reinterpret_cast<const uint32_t*>(kt));
    if (!FLUSH_ONLY) sm.se[t][i] = sv[i];
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < RPL; ++tt)
#pragma unroll
    for (int i = 0; i < RW; ++i) asm volatile("" : "+v"(raw[tt][i]));
  // X = m_p c_pj + sum_tau K'_tau,p E_tau,j, requantized and stored in place, over TM terms
  // (zero past the last one). The lane's columns of the first TR terms' deltas stay in registers
  // over all row steps; a row step reads from LDS its row's keys and the lane's columns of the
  // other TM - TR deltas. (TR < TM keeps the register count within four waves per SIMD.)
  auto materialise = [&]<int TM, int TR>() __attribute__((always_inline)) {
    float e[TR][CPL];
#pragma unroll
    for (int tau = 0; tau < TR; ++tau) {
      if (tau < terms) {
        load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(&sm.se[tau][cg * CPL]),
                            reinterpret_cast<uint32_t*>(e[tau]));
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) e[tau][c] = 0.0f;
      }
    }
#pragma unroll
    for (int tt = 0; tt < RPL; ++tt) {
      const int p0 = tt * G::RPS + w * 4, p = p0 + rs;
      const float m = my_rows[tt * G::RPS].x;
      by_plan<PLAN, T16>(tt, p0, r, [&]<int K>() __attribute__((always_inline)) {
        float X[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) X[c] = decode_row<D, K>(raw[tt], c, p, r) * m;
#pragma unroll
        for (int tau = 0; tau < TM; ++tau) {
          const float kp = skT[p][tau];
          if (tau < TR) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) X[c] = fmaf(kp, e[tau < TR ? tau : 0][c], X[c]);
          } else if (tau < terms) {
            float el[CPL];
            load_bytes<CPL * 4>(reinterpret_cast<const uint8_t*>(&sm.se[tau][cg * CPL]),
                                reinterpret_cast<uint32_t*>(el));
#pragma unroll
            for (int c = 0; c < CPL; ++c) X[c] = fmaf(kp, el[c], X[c]);
          }
        }
        each_kind<K>([&]<int K2, bool MIX>() __attribute__((always_inline)) {
          Row<D, K2>::template store<false, MIX, true>(up, p0, rs, cg, X, ssc);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  constexpr int TR8 = PLAN == PLAN_FIXED ? kMaxWindow - 1 : kMaxWindow / 2;
  if (terms <= kMaxWindow / 2)
    materialise.template operator()<kMaxWindow / 2, kMaxWindow / 2>();
  else
    materialise.template operator()<kMaxWindow, TR8>();
  flush_scales<D, G::NT>(up, ssc, r, tid);
  if (tid == 0) {   // an empty window, with no gate form yet
    wp.hdr[0] = 0;
    wp.hdr[2] = 0;
    wp.hdr[3] = 0;
  }
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
// At least four waves per SIMD (at most 128 VGPRs): at d = 128 that is every workgroup a CU
// holds; the window's end keeps its deltas in registers within that bound.
template <int D, int PER_KEY, int BF16, int PLAN, int WAVES, int NF, bool FLUSH_ONLY, bool HEADS>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4))) void window_kernel(const StepArgs a) {
  __shared__ WinSmem<D, Geo<D, WAVES>::NW> sm;
  int b, head;
  if (!unit_of(a, b, head)) return;
  const int bh = b * a.H + head;
  const int64_t slot = a.slot_idx[b];
  const UnitAddr ua = unit_addr<D, FMT_Q>(a.st, slot, head, a.H);   // arithmetic only
  if (!slot_in_pool(slot, a.st.num_slots)) return;
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
