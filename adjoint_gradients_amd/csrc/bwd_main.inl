// bwd_main.inl -- the fused reverse adjoint + local-VJP kernel (included by scan_bwd.hip).
//
// One workgroup = 4 wavefronts = 4 channel blocks of the same chunk k.
// Per wavefront (CH channels x NN states, NL states per lane):
//   phase 1  forward walk from the chunk checkpoint h_{t0-1}; the state at
//            the start of every S-token sub-chunk goes to a per-wavefront
//            scratch area in global memory (written and read back by the same
//            lanes).  Where k_bwd_hsub can stage the chunk's rows, it does this
//            walk beforehand at higher occupancy and this phase is skipped;
//   phase 2  sub-chunks right to left: recompute the S states into registers,
//            then walk them in reverse with the adjoint recurrence and the
//            local VJPs (equations in scan_bwd.hip).
// Latency hiding: the per-token rows b_t, c_t and c_{t+W} (shared by all
// channels) of the next sub-chunk are loaded into registers at the start of a
// sub-chunk and written to a double-buffered LDS area at its end; the
// per-lane scalars (s, x, g and the partner token's s, g) come through small
// register rings filled two tokens ahead.

namespace {

struct Tok {
  float s, x, g, sm, gm;
};

// Row-pointer addressing: `row` is uniform across the wavefront (a scalar
// register pair), `off` the lane's channel offset -- one VGPR shared by all
// tokens instead of a 64-bit address per token.
template <typename T>
__device__ __forceinline__ T* row_ptr(T* base, int64_t t, int64_t ld) {
  return base + t * ld;
}

template <typename IO, bool WIN>
__device__ __forceinline__ Tok load_tok(const BwdArgs& a, const IO* __restrict__ xp, int64_t i, uint32_t off) {
  Tok o;
  const int64_t P = a.P;
  o.s = row_ptr(a.s, i, P)[off];
  o.x = load_io(row_ptr(xp, i, P) + off);
  o.g = row_ptr(a.g, i, P)[off];
  if constexpr (WIN) {
    const int64_t m = i + a.W;
    const bool in = m < a.T;        // uniform
    const int64_t mm = in ? m : i;  // any valid row; the value is replaced by 0
    const float sm = row_ptr(a.s, mm, P)[off];
    const float gm = row_ptr(a.g, mm, P)[off];
    o.sm = in ? sm : 0.0f;
    o.gm = in ? gm : 0.0f;
  } else {
    o.sm = 0.0f;
    o.gm = 0.0f;
  }
  return o;
}

// Waits for this wavefront's outstanding LDS operations only (vmcnt untouched).
__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
}

// Keeps the instruction scheduler from hoisting one token's loads into the
// previous token's code (which would multiply the live registers).
__device__ __forceinline__ void token_fence() { __builtin_amdgcn_sched_barrier(0); }

// NL consecutive floats of a staged row; 16-byte reads when NL % 4 == 0 (the
// row offsets are then multiples of 4 floats).
template <int NL>
__device__ __forceinline__ void lds_row(const float* src, float (&dst)[NL]) {
  if constexpr (NL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < NL / 4; q++) {
      const float4 v = reinterpret_cast<const float4*>(src)[q];
      dst[4 * q] = v.x;
      dst[4 * q + 1] = v.y;
      dst[4 * q + 2] = v.z;
      dst[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NL; j++) dst[j] = src[j];
  }
}

// Per-wavefront running state of the reverse walk.
template <int NL>
struct RevState {
  float al2[NL];   // alpha * log2(e)
  float inc[NL];   // a_{i+1} mu_{i+1}
  float dal[NL];   // sum_i da_i s_i a_i  (dalpha = -dal)
  float dbias;
  double H, sigma, suffix;  // window sums of s (fp64)
};

// One token of the reverse walk: adjoint recurrence + local VJPs + channel
// sums of db / dc into xw_tau.
template <typename IO, int NL, int G, bool WIN>
__device__ __forceinline__ void rev_token(RevState<NL>& st, const BwdArgs& a, const Tok& tk, const float (&bt)[NL],
                                          const float (&ct)[NL], const float (&cm)[NL], const float (&hp)[NL],
                                          const float (&hc)[NL], int64_t i, uint32_t off, bool valid, int grp,
                                          int pl, int lane, float* red, float* xw_tau) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int OUT = 2 * NN;
  float av[NL], mu[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    av[j] = fast_exp2(-tk.s * st.al2[j]);
    mu[j] = fmaf(tk.g, ct[j], st.inc[j]);
  }
  if constexpr (WIN) {
    // drop the token leaving the window: - g_{i+W} c_{i+W} prod_{j=i+1}^{i+W} a_j
    const float E = static_cast<float>(st.sigma + st.H - st.suffix);
#pragma unroll
    for (int j = 0; j < NL; j++) {
      const float D = fast_exp2(-E * st.al2[j]);
      mu[j] = fmaf(-tk.gm * cm[j], D, mu[j]);
    }
    st.suffix += static_cast<double>(tk.sm);
    st.sigma += static_cast<double>(tk.s);
  }
  float ds = 0.0f, dxd = 0.0f;
#pragma unroll
  for (int j = 0; j < NL; j++) {
    const float tt = mu[j] * hp[j] * av[j];
    st.inc[j] = av[j] * mu[j];
    ds = fmaf(tt, st.al2[j], ds);
    st.dal[j] = fmaf(tt, tk.s, st.dal[j]);
    dxd = fmaf(mu[j], bt[j], dxd);
  }
  if constexpr (G > 1) {
    ds = group_sum<G, CH>(ds);
    dxd = group_sum<G, CH>(dxd);
  }
  const float dD = -(ds * (1.0f / kLog2e)) * one_minus_exp_neg(tk.s);
  if (valid && grp == 0) {
    store_io(row_ptr(static_cast<IO*>(a.dY), i, a.ldy) + off, dD);
    if (a.dxdir) row_ptr(a.dxdir, i, a.P)[off] = dxd;
  }
  st.dbias += dD;
  // channel sums of db = mu x and dc = g h through an LDS transpose (placement
  // in red_layout.hpp).  Lanes past the last channel contribute zeros; their x
  // and g are zeroed once per token rather than per product.
  using RL = redl::Layout<NL, G>;
  const float xz = valid ? tk.x : 0.0f;
  const float gz = valid ? tk.g : 0.0f;
  const int n0 = grp * NL;
#pragma unroll
  for (int j = 0; j < NL; j++) {
    red[RL::at(n0 + j, pl)] = mu[j] * xz;
    red[RL::at(NN + n0 + j, pl)] = gz * hc[j];
  }
  if constexpr (RL::kSwz) {
    // A wavefront's LDS operations execute in issue order, so its reads see
    // its own writes without a wait; the wave barrier only keeps the compiler
    // from moving accesses across this point.
    __builtin_amdgcn_wave_barrier();
    const int o = lane >> 1, r = lane & 1;
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 v = *reinterpret_cast<const float4*>(red + RL::chunk(o, 4 * r + q));
      sum += (v.x + v.y) + (v.z + v.w);
    }
    sum = xor_sum<1>(sum);
    if (r == 0) xw_tau[o] = sum;
    __builtin_amdgcn_wave_barrier();
  } else {
    constexpr int RS = RL::kRS;
    lds_wait();
    if constexpr (OUT <= 64) {
      constexpr int LPO = 64 / OUT;  // lanes per output
      constexpr int V = CH / LPO;    // values summed per lane
      const int o = lane / LPO, r = lane % LPO;
      const float* src = red + o * RS + r * V;
      float sum = 0.0f;
#pragma unroll
      for (int v = 0; v < V; v++) sum += src[v];
      if constexpr (LPO >= 2) sum = xor_sum<1>(sum);
      if constexpr (LPO >= 4) sum = xor_sum<2>(sum);
      if constexpr (LPO >= 8) sum = xor_sum<4>(sum);
      if constexpr (LPO >= 16) sum = xor_sum<8>(sum);
      if constexpr (LPO >= 32) sum = xor_sum<16>(sum);
      if (r == 0) xw_tau[o] = sum;
    } else {
#pragma unroll
      for (int q = 0; q < OUT / 64; q++) {
        const int o = lane + 64 * q;
        const float* src = red + o * RS;
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < CH; v++) sum += src[v];
        xw_tau[o] = sum;
      }
    }
    lds_wait();
  }
}

}  // namespace

template <typename IO, int NL, int G, bool WIN>
__global__ __launch_bounds__(256, 2) void k_bwd_main(BwdArgs a, int64_t NB, int64_t NBW) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int S = kSub;
  constexpr int OUT = 2 * NN;
  constexpr int NQ = WIN ? 3 : 2;                    // staged rows per token: b, c (, c_{t+W})
  constexpr int STG = NQ * S * NN;                   // floats per staging buffer
  constexpr int RPT = (STG + 64 * kWpb - 1) / (64 * kWpb);  // staged floats per thread
  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t T = a.T, P = a.P;
  const int C = a.C;
  const int64_t k = blockIdx.x;
  const int64_t cb = static_cast<int64_t>(blockIdx.y) * kWpb + w;
  const bool wave_live = cb < NB;
  const int64_t p = cb * CH + pl;
  const bool valid = p < P;
  const int64_t pc = valid ? p : P - 1;
  const uint32_t off = static_cast<uint32_t>(pc);  // lane offset within a token row
  const int n0 = grp * NL;
  const int nsub_max = (C + S - 1) / S;
  constexpr int RED = redl::Layout<NL, G>::kFloats;  // transpose area per wavefront
  float* red = lds + 2 * STG + w * RED;
  float* xw = lds + 2 * STG + kWpb * RED;  // [kWpb][S][OUT]
  float* hsg = a.hsub + ((k * NB + (wave_live ? cb : 0)) * nsub_max) * (NL * 64);
  const IO* xp = static_cast<const IO*>(a.x);
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  const int nsub = static_cast<int>((t1 - t0 + S - 1) / S);

  // rows of sub-chunk u (b, c, c_{t+W}) -> registers -> LDS buffer
  float rows[RPT];
  auto fetch_rows = [&](int u) {
    const int64_t ta = t0 + static_cast<int64_t>(u) * S;
#pragma unroll
    for (int r = 0; r < RPT; r++) {
      const int e = tid + r * 64 * kWpb;
      if (e < STG) {
        const int q = e / (S * NN), tau = (e / NN) % S, n = e % NN;
        int64_t t = ta + tau + (q == 2 ? a.W : 0);
        if (t >= T) t = T - 1;  // such rows only meet zero weights
        rows[r] = (q == 0 ? a.b : a.c)[t * NN + n];
      }
    }
  };
  auto put_rows = [&](int buf) {
#pragma unroll
    for (int r = 0; r < RPT; r++) {
      const int e = tid + r * 64 * kWpb;
      if (e < STG) lds[buf * STG + e] = rows[r];
    }
  };
  fetch_rows(nsub - 1);

  RevState<NL> st;
#pragma unroll
  for (int j = 0; j < NL; j++) {
    st.al2[j] = a.alpha[pc * NN + n0 + j] * kLog2e;
    st.inc[j] = a.carry[(k * P + pc) * NN + n0 + j];
    st.dal[j] = 0.0f;
  }
  st.dbias = 0.0f;
  st.sigma = 0.0;
  st.suffix = 0.0;
  st.H = 0.0;
  if constexpr (WIN) st.H = a.hwin[k * P + pc];

  // ---------------- phase 1: forward walk, sub-chunk start states to scratch
  // (skipped when the separate sub-chunk pass already wrote them)
  if (!a.hsub_ready) {
    float h[NL];
#pragma unroll
    for (int j = 0; j < NL; j++) h[j] = a.h_ckpt[(k * P + pc) * NN + n0 + j];
    const int64_t nwalk = static_cast<int64_t>(nsub - 1) * S;  // multiple of S (and of 4)
    float rs[4], rx[4], rb[4][NL];
    auto ld = [&](int slot, int64_t t) {
      rs[slot] = row_ptr(a.s, t, P)[off];
      rx[slot] = load_io(row_ptr(xp, t, P) + off);
      load_row<NL>(row_ptr(a.b, t, NN) + n0, rb[slot]);
    };
    if (nwalk > 0) {
      ld(0, t0);
      ld(1, t0 + 1);
      ld(2, t0 + 2);
    }
    for (int64_t q4 = 0; q4 < nwalk; q4 += 4) {
      if (wave_live && (q4 % S) == 0) {
        const int u = static_cast<int>(q4 / S);
#pragma unroll
        for (int j = 0; j < NL; j++) hsg[(u * NL + j) * 64 + lane] = h[j];
      }
#pragma unroll
      for (int r = 0; r < 4; r++) {
        if (q4 + r + 3 < nwalk) ld((r + 3) & 3, t0 + q4 + r + 3);
        const float ns = -rs[r];
#pragma unroll
        for (int j = 0; j < NL; j++) h[j] = fmaf(fast_exp2(ns * st.al2[j]), h[j], rb[r][j] * rx[r]);
      }
    }
    if (wave_live) {
#pragma unroll
      for (int j = 0; j < NL; j++) hsg[((nsub - 1) * NL + j) * 64 + lane] = h[j];
    }
  }
  put_rows((nsub - 1) & 1);
  __syncthreads();

  // ---------------- phase 2: sub-chunks right to left
  float fs[4], fx[4];  // recompute ring (s, x)
  Tok ring[4];         // reverse-walk ring
  float hs[NL];
  bool pre = false;    // fs/fx slots 0,1 and hs already hold the next sub-chunk's values
  for (int u = nsub - 1; u >= 0; u--) {
    const int buf = u & 1;
    const float* sb = lds + buf * STG;  // b rows [S][NN], then c rows, then partner c rows
    const int64_t ta = t0 + static_cast<int64_t>(u) * S;
    const int len = static_cast<int>((t1 - ta < S) ? t1 - ta : S);
    if (u > 0) fetch_rows(u - 1);
    if (!pre) {
#pragma unroll
      for (int j = 0; j < NL; j++) hs[j] = hsg[(u * NL + j) * 64 + lane];
    }
    float hr[S][NL];
    if (len == S) {
      // recompute the sub-chunk's states
      if (!pre) {
        fs[0] = row_ptr(a.s, ta, P)[off];
        fx[0] = load_io(row_ptr(xp, ta, P) + off);
        fs[1] = row_ptr(a.s, ta + 1, P)[off];
        fx[1] = load_io(row_ptr(xp, ta + 1, P) + off);
      }
      {
        float hh[NL];
#pragma unroll
        for (int j = 0; j < NL; j++) hh[j] = hs[j];
#pragma unroll
        for (int tau = 0; tau < S; tau++) {
          token_fence();
          if (tau + 2 < S) {
            fs[(tau + 2) & 3] = row_ptr(a.s, ta + tau + 2, P)[off];
            fx[(tau + 2) & 3] = load_io(row_ptr(xp, ta + tau + 2, P) + off);
          }
          if (tau == S - 2) ring[(S - 1) & 3] = load_tok<IO, WIN>(a, xp, ta + S - 1, off);
          if (tau == S - 1) ring[(S - 2) & 3] = load_tok<IO, WIN>(a, xp, ta + S - 2, off);
          float bt[NL];
          lds_row<NL>(sb + tau * NN + n0, bt);
          const float ns = -fs[tau & 3];
          const float xv = fx[tau & 3];
#pragma unroll
          for (int j = 0; j < NL; j++) {
            hh[j] = fmaf(fast_exp2(ns * st.al2[j]), hh[j], bt[j] * xv);
            hr[tau][j] = hh[j];
          }
        }
      }
      // reverse walk
      pre = false;
#pragma unroll
      for (int tau = S - 1; tau >= 0; tau--) {
        token_fence();
        if (tau >= 2) ring[(tau - 2) & 3] = load_tok<IO, WIN>(a, xp, ta + tau - 2, off);
        if (tau == 1 && u > 0) {
          // prefetch the next (left) sub-chunk's first recompute tokens
          const int64_t tn = ta - S;
          fs[0] = row_ptr(a.s, tn, P)[off];
          fx[0] = load_io(row_ptr(xp, tn, P) + off);
          fs[1] = row_ptr(a.s, tn + 1, P)[off];
          fx[1] = load_io(row_ptr(xp, tn + 1, P) + off);
        }
        float bt[NL], ct[NL], cm[NL];
        lds_row<NL>(sb + tau * NN + n0, bt);
        lds_row<NL>(sb + S * NN + tau * NN + n0, ct);
        if constexpr (WIN) lds_row<NL>(sb + 2 * S * NN + tau * NN + n0, cm);
        else {
#pragma unroll
          for (int j = 0; j < NL; j++) cm[j] = 0.0f;
        }
        float hp[NL];
#pragma unroll
        for (int j = 0; j < NL; j++) hp[j] = (tau > 0) ? hr[tau > 0 ? tau - 1 : 0][j] : hs[j];
        rev_token<IO, NL, G, WIN>(st, a, ring[tau & 3], bt, ct, cm, hp, hr[tau], ta + tau, off, valid, grp, pl, lane,
                                  red, xw + (w * S + tau) * OUT);
        if (tau == 0 && u > 0) {
          // start state of the next sub-chunk (hs is no longer needed here)
#pragma unroll
          for (int j = 0; j < NL; j++) hs[j] = hsg[((u - 1) * NL + j) * 64 + lane];
          pre = true;
        }
      }
    } else {
      // partial sub-chunk (end of a ragged chunk): no register rings
      {
        float hh[NL];
#pragma unroll
        for (int j = 0; j < NL; j++) hh[j] = hs[j];
#pragma unroll
        for (int tau = 0; tau < S; tau++) {
          if (tau < len) {
            const int64_t t = ta + tau;
            const float ns = -row_ptr(a.s, t, P)[off];
            const float xv = load_io(row_ptr(xp, t, P) + off);
            float bt[NL];
            lds_row<NL>(sb + tau * NN + n0, bt);
#pragma unroll
            for (int j = 0; j < NL; j++) {
              hh[j] = fmaf(fast_exp2(ns * st.al2[j]), hh[j], bt[j] * xv);
              hr[tau][j] = hh[j];
            }
          }
        }
      }
      pre = false;
#pragma unroll
      for (int tau = S - 1; tau >= 0; tau--) {
        if (tau < len) {
          const Tok tk = load_tok<IO, WIN>(a, xp, ta + tau, off);
          float bt[NL], ct[NL], cm[NL];
          lds_row<NL>(sb + tau * NN + n0, bt);
          lds_row<NL>(sb + S * NN + tau * NN + n0, ct);
          if constexpr (WIN) lds_row<NL>(sb + 2 * S * NN + tau * NN + n0, cm);
          else {
#pragma unroll
            for (int j = 0; j < NL; j++) cm[j] = 0.0f;
          }
          float hp[NL];
#pragma unroll
          for (int j = 0; j < NL; j++) hp[j] = (tau > 0) ? hr[tau > 0 ? tau - 1 : 0][j] : hs[j];
          rev_token<IO, NL, G, WIN>(st, a, tk, bt, ct, cm, hp, hr[tau], ta + tau, off, valid, grp, pl, lane, red,
                                    xw + (w * S + tau) * OUT);
        }
      }
    }
    __syncthreads();
    // sum over the workgroup's wavefronts -> one partial per (token, workgroup)
    const int tot = len * OUT;
    for (int idx = tid; idx < tot; idx += 64 * kWpb) {
      const int tau = idx / OUT, o = idx % OUT;
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWpb; ww++) v += xw[(ww * S + tau) * OUT + o];
      a.part[((ta + tau) * NBW + blockIdx.y) * OUT + o] = v;
    }
    if (u > 0) put_rows((u - 1) & 1);
    __syncthreads();  // staged rows of u-1 visible; xw free again
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NL; j++) a.dal_part[(k * P + p) * NN + n0 + j] = -st.dal[j];
    if (grp == 0) a.dbias_part[k * P + p] = st.dbias;
  }
}
