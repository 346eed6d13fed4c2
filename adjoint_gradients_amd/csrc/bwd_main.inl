// bwd_main.inl -- the fused reverse adjoint + local-VJP kernel (included by scan_bwd.hip).
//
// One workgroup = 4 wavefronts = 4 channel blocks of the same chunk k.
// Per wavefront (CH channels x NN states, NL states per lane):
//   phase 1  forward walk from the chunk checkpoint h_{t0-1}; the state at
//            the start of every S-token sub-chunk goes to a per-wavefront
//            scratch area in global memory (written and read back by the same
//            lanes).  Where the states are already there -- kept by the
//            forward, or written by the slab's rebuild walk beforehand
//            (k_bwd_local_hsub, or k_bwd_hsub where it can stage the chunk's
//            rows), at higher occupancy -- this phase is skipped;
//   phase 2  sub-chunks right to left: recompute the S states into registers,
//            then walk them in reverse with the adjoint recurrence and the
//            local VJPs (equations in scan_bwd.hip).  A sub-chunk compiles to
//            one basic block: a partial one runs the same code on tokens
//            staged as zeros, stores go through buffer resources whose
//            out-of-range lanes are dropped, and window partners past the
//            sequence end (and lanes past the last channel) read zeros.
// Latency hiding: everything a sub-chunk reads from memory is brought by LDS
// DMA during the previous sub-chunk (issued at its start, waited for at its
// end, where the wait lets the walk's own stores stay in flight) -- the
// per-token rows b_t, c_t and c_{t+W} (shared by all channels) into a
// double-buffered area, the per-lane quantities (s, x, g and the partner
// token's s, g) into a double-buffered area of each wavefront's own -- so no
// register holds prefetched data; only the next sub-chunk's start state is
// loaded into registers ahead of time, on a single code path (a load on one
// path only would make the compiler wait for every load in flight where the
// paths meet).

namespace {

struct Tok {
  float s, x, g, sm, gm;
};

// Tokens at the end of a sub-chunk whose decay factors the recompute keeps
// for the reverse walk, which starts with them (their exps are not repeated).
// Seven fit in the 256 VGPRs of two waves per SIMD without spilling (eight
// spill), with each token's LDS values (b and c rows, per-lane values) read
// at the token rather than one token ahead, which held 29 more registers.
// Measured at the 1M-token layer: none kept 30.4 ms, four (values read ahead)
// 29.3, six 28.9, seven 28.8.
constexpr int kKeepA = 7;

// Vector-memory operations the reverse walk issues per token (rev_token's
// dDelta and dx_dir stores).
constexpr int kWalkStoresPerToken = 2;


typedef __attribute__((address_space(3))) char lds_byte;

// LDS byte address of a pointer into the kernel's dynamic LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_byte*)(p)));
}

// LDS DMA (global_load_lds_*): lane l's element goes from global memory
// straight to LDS byte address lds + 4 l, without a register round trip; a
// 2-byte element is zero-extended to 4 bytes there.  dma_s takes a
// wave-uniform base (scalar registers) plus the lane's 32-bit byte offset,
// dma_v the lane's own 64-bit address (the LDS address is wave-uniform in
// both).  M0 carries the LDS address; it is saved and restored.  The loads count in vmcnt like any other; their data
// may be read once this wavefront has waited for them (and, for data read by
// other wavefronts, after a barrier).
// A wave-uniform value moved to scalar registers (free when it is there).
template <typename T>
__device__ __forceinline__ const T* sgpr_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <typename T>
__device__ __forceinline__ void dma_s(const T* base_any, uint32_t voff, uint32_t lds_any) {
  const T* base = sgpr_ptr(base_any);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_any);
  uint32_t saved;
  if constexpr (sizeof(T) == 2)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}
template <typename T>
__device__ __forceinline__ void dma_v(const T* addr, uint32_t lds_any) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_any);
  uint32_t saved;
  if constexpr (sizeof(T) == 2)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(addr) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(addr) : "memory");
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row-pointer addressing: `row` is uniform across the wavefront (a scalar
// register pair), `off` the lane's channel offset -- one VGPR shared by all
// tokens instead of a 64-bit address per token.
template <typename T>
__device__ __forceinline__ T* row_ptr(T* base, int64_t t, int64_t ld) {
  return base + t * ld;
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
  double E64;  // sum of s over tokens i+1 .. i+W for the next token i (fp64)
};

// One token of the reverse walk: adjoint recurrence + local VJPs + channel
// sums of db / dc into xw_tau.  a_in: the token's decay factors when the
// caller still holds them (else they are computed here).
template <typename IO, int NL, int G, bool WIN>
__device__ __forceinline__ void rev_token(RevState<NL>& st, const BwdArgs& a, const Tok& tk, const float (&bt)[NL],
                                          const float (&ct)[NL], const float (&cm)[NL], const float (&hp)[NL],
                                          const float (&hc)[NL], float sg, char* yrow, char* xrow, bool live,
                                          int grp, int pl, int lane, float* red, int rd_off,
                                          int voff_dy, int voff_dx, float* xw_tau, const float* a_in) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int OUT = 2 * NN;
  float av[NL], mu[NL];
#pragma unroll
  for (int j = 0; j < NL; j++) {
    av[j] = a_in ? a_in[j] : fast_exp2(-tk.s * st.al2[j]);
    mu[j] = fmaf(tk.g, ct[j], st.inc[j]);
  }
  if constexpr (WIN) {
    // drop the token leaving the window: - g_{i+W} c_{i+W} prod_{j=i+1}^{i+W} a_j.
    // Where the partner token i + W lies past the sequence end there is no
    // such term: its g and s arrive as zeros.
    const float gm = tk.gm;
    const float sm = tk.sm;
    const float E = static_cast<float>(st.E64);
#pragma unroll
    for (int j = 0; j < NL; j++) {
      const float D = fast_exp2(-E * st.al2[j]);
      mu[j] = fmaf(-gm * cm[j], D, mu[j]);
    }
    // token i + W leaves the window of token i - 1, token i enters it (the
    // difference rounded to fp32 adds at most 2^-24 of it per token, far
    // below the fp32 rounding of E itself)
    st.E64 += static_cast<double>(tk.s - sm);
  }
  float ds = 0.0f, dxd = 0.0f;
#pragma unroll
  for (int j = 0; j < NL; j++) {
    st.inc[j] = av[j] * mu[j];
    const float tt = st.inc[j] * hp[j];  // mu_i a_i h_{i-1}
    ds = fmaf(tt, st.al2[j], ds);
    st.dal[j] = fmaf(tt, tk.s, st.dal[j]);
    dxd = fmaf(mu[j], bt[j], dxd);
  }
  // Sums over the lane groups of a channel.  With two groups one exchange
  // serves both: group 0 then holds the sum of ds, group 1 that of dxd, and
  // each group stores its own (dD and dbias are only kept from group 0).
  if constexpr (G == 2) {
    ds = half_sums_pair(ds, dxd);
    dxd = ds;
  } else if constexpr (G > 1) {
    ds = group_sum<G, CH>(ds);
    dxd = group_sum<G, CH>(dxd);
  }
  const float dD = -(ds * (1.0f / kLog2e)) * sg;  // sg = sigma(Delta_i) = 1 - e^{-s_i}
  // Exactly kWalkStoresPerToken vector-memory operations per token (the two
  // stores below): the end-of-sub-chunk wait in k_bwd_main counts on it.
  // Stores through buffer resources over token i's rows: lanes that store
  // nothing carry an offset past the row, and the hardware drops such a
  // store, so no lane mask (and no branch) splits the token's code.
  // A token past the chunk end (live false) gets empty resources: its row
  // may lie past the arrays, and nothing of it is stored.
  {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(yrow, 0, live ? static_cast<int>(a.P * sizeof(IO)) : 0, kBufWord3);
    if constexpr (sizeof(IO) == 2)
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, f32_to_bf16(dD)), ry, voff_dy, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dD), ry, voff_dy, 0, 0);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(xrow, 0, (live && a.dxdir) ? static_cast<int>(a.P * 4) : 0, kBufWord3);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dxd), rx, voff_dx, 0, 0);
  }
  st.dbias += dD;
  // channel sums of db = mu x and dc = g h through an LDS transpose (placement
  // in red_layout.hpp).  Lanes past the last channel contribute zeros: their
  // x and g arrive as zeros.
  using RL = redl::Layout<NL, G>;
  const float xz = tk.x;
  const float gz = tk.g;
  float* wr = red + RL::lane_base(grp, pl);
#pragma unroll
  for (int j = 0; j < NL; j++) {
    wr[RL::row_off(0, j)] = mu[j] * xz;
    wr[RL::row_off(1, j)] = gz * hc[j];
  }
  if constexpr (RL::kSwz) {
    // A wavefront's LDS operations execute in issue order, so its reads see
    // its own writes without a wait; the wave barrier only keeps the compiler
    // from moving accesses across this point.
    __builtin_amdgcn_wave_barrier();
    const int o = lane >> 1, r = lane & 1;
    const float4* rd = reinterpret_cast<const float4*>(red + rd_off);
    float sum;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 v = rd[q];
      const float pq = (v.x + v.y) + (v.z + v.w);
      sum = q == 0 ? pq : sum + pq;
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

// ST: every state was kept by the forward (a.hall; the store-everything
// baseline): each sub-chunk's states are loaded instead of recomputed.
template <typename IO, int NL, int G, bool WIN, bool ST>
__global__ __launch_bounds__(256, 2) void k_bwd_main(BwdArgs a, int64_t NB, int64_t NBW) {
  constexpr int CH = 64 / G;
  constexpr int NN = NL * G;
  constexpr int S = kSub;
  constexpr int OUT = 2 * NN;
  constexpr int NQ = WIN ? 3 : 2;                    // staged rows per token: b, c (, c_{t+W})
  constexpr int STG = NQ * S * NN;                   // floats per staging buffer
  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int grp = lane / CH, pl = lane % CH;
  const int64_t T = a.T, P = a.P;
  const int C = a.C;
  const int64_t k = a.k_lo + blockIdx.x;  // chunk (the launch covers one slab)
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
  // this lane's read position in the transpose buffer (swizzled layout),
  // fixed for the whole kernel
  const int rd_off = redl::Layout<NL, G>::kSwz ? redl::Layout<NL, G>::chunk(lane >> 1, 4 * (lane & 1)) : 0;
  // byte offsets of this lane's dDelta and dx_dir stores within a token row;
  // lanes that store nothing get an offset past every row (dropped store).
  // dDelta comes from lane group 0; dx_dir from group 1 with two groups (the
  // paired group sum leaves it there), else from group 0.
  const int voff_dy = (valid && grp == 0) ? static_cast<int>(off * sizeof(IO)) : kBufOutside;
  const int voff_dx = (valid && grp == (G == 2 ? 1 : 0)) ? static_cast<int>(off * 4) : kBufOutside;
  // base of the dx_dir rows (any valid pointer when there is no dx_dir: its
  // resources are then empty)
  float* const dxb = a.dxdir ? a.dxdir : static_cast<float*>(a.dY);
  const int64_t ldy_b = a.ldy * static_cast<int64_t>(sizeof(IO)), ldx_b = P * 4;
  float* xw = lds + 2 * STG + kWpb * RED;  // [kWpb][S][OUT]
  float* hsg = ST ? nullptr : a.hsub + hsub_offset(k - a.hsub_k0, wave_live ? cb : 0, 0, NB, nsub_max, NL);
  const IO* xp = static_cast<const IO*>(a.x);
  const int64_t t0 = k * C;
  const int64_t t1 = (t0 + C < T) ? t0 + C : T;
  const int nsub = static_cast<int>((t1 - t0 + S - 1) / S);

  // Rows of sub-chunk u (b, c, c_{t+W}, shared by all channels) -> LDS
  // buffer u & 1, by DMA spread over the workgroup's wavefronts: instruction r
  // moves elements 64 r .. 64 r + 63 of the buffer [3][S][NN].
  auto dma_rows = [&](int u) {
    const int64_t ta = t0 + static_cast<int64_t>(u) * S;
    const uint32_t dst = lds_addr(lds + (u & 1) * STG);
    for (int r = w; r * 64 < STG; r += kWpb) {
      const int e = r * 64 + lane;
      if (e < STG) {
        const int q = e / (S * NN), tau = (e / NN) % S, n = e % NN;
        int64_t t = ta + tau + (q == 2 ? a.W : 0);
        if (t >= T) t = T - 1;  // such rows only meet zero weights
        dma_v((q == 0 ? a.b : a.c) + t * NN + n, dst + 256u * r);
      }
    }
  };

  // Per-lane quantities of sub-chunk u (s, x, g and, with a window, s and g
  // of the partner token t + W) -> this wavefront's own double-buffered LDS
  // area [2][NQS][S][CH], by DMA; each quantity's block is padded by 32
  // floats so that reads or writes of two quantities merged into one
  // instruction (32 lanes per pass) hit disjoint banks.  Lane (grp, pl) brings
  // tokens grp, grp + G, ... of channel pc, so each instruction covers G token
  // rows.  x arrives raw (bf16 zero-extended to 4 bytes, or the float).  Only
  // this wavefront reads the area.  Lanes past the last channel keep zeros
  // there (see below).  Partner values of tokens whose partner
  // lies past the sequence end are zeros (written here), so the walk drops no
  // window term for them.
  constexpr int NQS = WIN ? 5 : 3;
  constexpr int SPL = S / G;       // tokens fetched per lane
  constexpr int SQ = S * CH + 32;  // floats per quantity block
  float* sc0 = xw + kWpb * S * OUT + w * (2 * NQS * SQ);
  static_assert(2 * STG + kWpb * (RED + S * OUT + 2 * NQS * SQ) <= bwd_main_lds_floats(NL, G),
                "LDS layout exceeds the planned size");
  const uint32_t lrow = static_cast<uint32_t>(grp) * static_cast<uint32_t>(P) + off;  // P <= 2^20
  const uint32_t voff4 = lrow * 4u, voffx = lrow * static_cast<uint32_t>(sizeof(IO));
  auto dma_scal = [&](int u) {
    const int64_t ta = t0 + static_cast<int64_t>(u) * S;
    const uint32_t dst = lds_addr(sc0 + (u & 1) * (NQS * SQ));
    if (ta + S <= t1 && (!WIN || ta + S - 1 + a.W < T)) {
      // every token inside the chunk and every partner inside the sequence
      if (valid) {
#pragma unroll
        for (int i = 0; i < SPL; i++) {
          const int64_t tb = ta + G * i;  // the lane's token is tb + grp
          const uint32_t d = dst + 4u * (G * i * CH);
          dma_s(a.s + tb * P, voff4, d);
          dma_s(xp + tb * P, voffx, d + 4u * SQ);
          dma_s(a.g + tb * P, voff4, d + 8u * SQ);
          if constexpr (WIN) {
            dma_s(a.s + (tb + a.W) * P, voff4, d + 12u * SQ);
            dma_s(a.g + (tb + a.W) * P, voff4, d + 16u * SQ);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPL; i++) {
        const int64_t t = ta + G * i + grp;
        const uint32_t d = dst + 4u * (G * i * CH);
        if (t < t1) {
          if (!valid) continue;  // the lane's slots hold zeros
          dma_v(a.s + t * P + pc, d);
          dma_v(xp + t * P + pc, d + 4u * SQ);
          dma_v(a.g + t * P + pc, d + 8u * SQ);
          if constexpr (WIN) {
            const int64_t m = t + a.W;
            if (m < T) {
              dma_v(a.s + m * P + pc, d + 12u * SQ);
              dma_v(a.g + m * P + pc, d + 16u * SQ);
            } else {
              // partner past the sequence end: no window term (zeros)
              float* z = sc0 + (u & 1) * (NQS * SQ) + G * i * CH + lane;
              z[3 * SQ] = 0.0f;
              z[4 * SQ] = 0.0f;
            }
          }
        } else {
          // past the chunk end: zeros (the walk then passes the token by)
          float* z = sc0 + (u & 1) * (NQS * SQ) + G * i * CH + lane;
#pragma unroll
          for (int q = 0; q < NQS; q++) z[q * SQ] = 0.0f;
        }
      }
    }
  };
  // Lanes past the last channel take no part in the channel sums: their
  // slots of the area hold zeros, written here and never refilled (their DMA
  // is masked off).
  if (!valid) {
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int q = 0; q < NQS; q++)
#pragma unroll
        for (int i = 0; i < SPL; i++) sc0[b * (NQS * SQ) + q * SQ + G * i * CH + lane] = 0.0f;
  }
  const float* sc = sc0;  // area of the current sub-chunk
  auto scal = [&](int q, int tau) { return sc[q * SQ + tau * CH + pl]; };
  auto scal_x = [&](int tau) {
    return raw_to_f32(__builtin_bit_cast(typename IoRaw<IO>::type, scal(1, tau)));
  };
  auto read_tok = [&](int tau) {
    Tok o;
    o.s = scal(0, tau);
    o.x = scal_x(tau);
    o.g = scal(2, tau);
    o.sm = WIN ? scal(3, tau) : 0.0f;
    o.gm = WIN ? scal(4, tau) : 0.0f;
    return o;
  };
  dma_rows(nsub - 1);
  dma_scal(nsub - 1);

  RevState<NL> st;
#pragma unroll
  for (int j = 0; j < NL; j++) {
    st.al2[j] = a.alpha[pc * NN + n0 + j] * kLog2e;
    st.inc[j] = a.carry[(k * P + pc) * NN + n0 + j];
    st.dal[j] = 0.0f;
  }
  st.dbias = 0.0f;
  st.E64 = 0.0;
  if constexpr (WIN) st.E64 = a.hwin[k * P + pc];  // sum of s over the W tokens after the chunk

  // ---------------- phase 1: forward walk, sub-chunk start states to scratch
  // (skipped when the separate sub-chunk pass already wrote them)
  if (!ST && !a.hsub_ready) {
    float h[NL];
#pragma unroll
    for (int j = 0; j < NL; j++) h[j] = a.h_ckpt[(k * P + pc) * NN + n0 + j];
    const int64_t nwalk = static_cast<int64_t>(nsub - 1) * S;  // multiple of S (and of 4)
    float rs[4], rb[4][NL];
    typename IoRaw<IO>::type rx[4];
    auto ld = [&](int slot, int64_t t) {
      rs[slot] = row_ptr(a.s, t, P)[off];
      rx[slot] = load_raw(row_ptr(xp, t, P) + off);
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
        for (int j = 0; j < NL; j++) h[j] = fmaf(fast_exp2(ns * st.al2[j]), h[j], rb[r][j] * raw_to_f32(rx[r]));
      }
    }
    if (wave_live) {
#pragma unroll
      for (int j = 0; j < NL; j++) hsg[((nsub - 1) * NL + j) * 64 + lane] = h[j];
    }
  }
  wait_vm_all();
  __syncthreads();  // staged data of the first sub-chunk visible

  // ---------------- phase 2: sub-chunks right to left
  float hs[NL], hn[NL];  // start states of the current and of the next sub-chunk
  // the last sub-chunk's start state, loaded as the walk's prefetches load
  // the others (one code path at the loop head: a load on one path only
  // would make the compiler drain every load in flight where the paths meet)
  if constexpr (!ST) {
#pragma unroll
    for (int j = 0; j < NL; j++) hn[j] = hsg[((nsub - 1) * NL + j) * 64 + lane];
  }
  // stored states of this wavefront's channels (any wavefront may read them)
  const float* hag = ST ? a.hall + hsub_offset(k, wave_live ? cb : NB - 1, 0, NB, C, NL) + lane : nullptr;
  const int clen = static_cast<int>(t1 - t0);
  for (int u = nsub - 1; u >= 0; u--) {
    const int buf = u & 1;
    const float* sb = lds + buf * STG;  // b rows [S][NN], then c rows, then partner c rows
    const int64_t ta = t0 + static_cast<int64_t>(u) * S;
    const int len = static_cast<int>((t1 - ta < S) ? t1 - ta : S);
    sc = sc0 + buf * (NQS * SQ);
    // A wavefront past the last channel block has no states of its own; it
    // starts from zero (it must not read another wavefront's, which a
    // different workgroup may still be writing) and contributes zeros.
    if constexpr (!ST) {
#pragma unroll
      for (int j = 0; j < NL; j++) hs[j] = wave_live ? hn[j] : 0.0f;
    }
    auto prefetch = [&]() {
      if (u > 0) {
        dma_rows(u - 1);
        dma_scal(u - 1);
        if constexpr (!ST) {
#pragma unroll
          for (int j = 0; j < NL; j++) {
            // loaded by every wavefront (hsg is a valid address for all) and
            // kept only by live ones, where the next sub-chunk starts: an
            // unconditional load issued here, ahead of the walk, with nothing
            // waiting for it until then
            hn[j] = hsg[((u - 1) * NL + j) * 64 + lane];
          }
        }
      }
    };
    // A partial sub-chunk (the end of a ragged chunk) runs the same code:
    // its tokens past the chunk end were staged as zeros (s = x = g = 0 and
    // no partner), so they leave the states and the adjoint unchanged, add
    // nothing to any sum, and their stores are dropped.
    float hr[S][NL];
    // decay factors of the sub-chunk's last kKeepA tokens, kept from the
    // recompute for the first tokens of the reverse walk
    float alast[kKeepA][NL];
    if constexpr (ST) {
      // the stored states: the chunk's checkpoint or the state after the
      // previous token, then the state after each token of the sub-chunk
      // (tokens past the chunk end repeat its last one; they add nothing)
      const float* src = u == 0 ? a.h_ckpt + (k * P + pc) * NN + n0 : hag + (u * S - 1) * NL * 64;
      const int stride = u == 0 ? 1 : 64;
#pragma unroll
      for (int j = 0; j < NL; j++) hs[j] = src[j * stride];
#pragma unroll
      for (int tau = 0; tau < S; tau++) {
        const int tc = (u * S + tau < clen) ? u * S + tau : clen - 1;
#pragma unroll
        for (int j = 0; j < NL; j++) hr[tau][j] = hag[(tc * NL + j) * 64];
      }
    }
    // bring sub-chunk u - 1's data and start state now: the buffers it
    // fills were last read before the previous sub-chunk's end barrier, and
    // the loads get the whole sub-chunk to land
    prefetch();
    // recompute the sub-chunk's states
    if constexpr (!ST) {
      float hh[NL];
#pragma unroll
      for (int j = 0; j < NL; j++) hh[j] = hs[j];
      // each token's LDS reads (s, x and the b row) are issued one token
      // ahead, so their latency hides behind the previous token's arithmetic
      float cs = scal(0, 0), cx = scal_x(0);
      float bn[NL];
      lds_row<NL>(sb + n0, bn);
#pragma unroll
      for (int tau = 0; tau < S; tau++) {
        token_fence();
        const float ns = -cs;
        const float xv = cx;
        float bt[NL];
#pragma unroll
        for (int j = 0; j < NL; j++) bt[j] = bn[j];
        if (tau + 1 < S) {
          cs = scal(0, tau + 1);
          cx = scal_x(tau + 1);
          lds_row<NL>(sb + (tau + 1) * NN + n0, bn);
        }
#pragma unroll
        for (int j = 0; j < NL; j++) {
          const float av = fast_exp2(ns * st.al2[j]);
          if (tau >= S - kKeepA) alast[tau >= S - kKeepA ? tau - (S - kKeepA) : 0][j] = av;
          hh[j] = fmaf(av, hh[j], bt[j] * xv);
          hr[tau][j] = hh[j];
        }
      }
    }
    // sigma(Delta) = 1 - e^{-s} of the sub-chunk's tokens.  With two lane
    // groups only group 0 needs it (it stores dDelta and keeps dbias): group 0
    // evaluates tokens 0 .. S/2-1 and group 1 tokens S/2 .. S-1 of the same
    // channel, and one lane exchange per pair hands group 1's values over.
    float sig[S];
    if constexpr (G == 2) {
#pragma unroll
      for (int q = 0; q < S / 2; q++) {
        const float v = one_minus_exp_neg(scal(0, grp * (S / 2) + q));
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        sig[q] = __uint_as_float(r[0]);          // lanes 0..31: own value (token q)
        sig[S / 2 + q] = __uint_as_float(r[1]);  // lanes 0..31: group 1's (token S/2 + q)
      }
    }
    // reverse walk; a token's per-lane values and its b, c (and partner c)
    // rows are read from LDS at the token
    struct Rows {
      float b[NL], c[NL], m[NL];
    };
    auto read_rows = [&](int tau, Rows& r) {
      lds_row<NL>(sb + tau * NN + n0, r.b);
      lds_row<NL>(sb + S * NN + tau * NN + n0, r.c);
      if constexpr (WIN) lds_row<NL>(sb + 2 * S * NN + tau * NN + n0, r.m);
      else {
#pragma unroll
        for (int j = 0; j < NL; j++) r.m[j] = 0.0f;
      }
    };
    // rows of the token being walked (dDelta in dY, dx_dir), stepped down by
    // one row per token
    char* yrow = reinterpret_cast<char*>(static_cast<IO*>(a.dY) + (ta + S - 1) * a.ldy);
    char* xrow = reinterpret_cast<char*>(dxb + (ta + S - 1) * P);
#pragma unroll
    for (int tau = S - 1; tau >= 0; tau--) {
      token_fence();
      const Tok cur = read_tok(tau);
      Rows rcur;
      read_rows(tau, rcur);
      float bt[NL], ct[NL], cm[NL];
#pragma unroll
      for (int j = 0; j < NL; j++) {
        bt[j] = rcur.b[j];
        ct[j] = rcur.c[j];
        cm[j] = rcur.m[j];
      }
      float hp[NL];
#pragma unroll
      for (int j = 0; j < NL; j++) hp[j] = (tau > 0) ? hr[tau > 0 ? tau - 1 : 0][j] : hs[j];
      const float sg = (G == 2) ? sig[tau] : one_minus_exp_neg(cur.s);
      rev_token<IO, NL, G, WIN>(st, a, cur, bt, ct, cm, hp, hr[tau], sg, yrow, xrow, tau < len, grp,
                                pl, lane, red, rd_off, voff_dy, voff_dx, xw + (w * S + tau) * OUT,
                                (!ST && tau >= S - kKeepA) ? alast[tau >= S - kKeepA ? tau - (S - kKeepA) : 0]
                                                           : nullptr);
      yrow -= ldy_b;
      xrow -= ldx_b;
    }
    // Wait for the prefetch of sub-chunk u - 1 (and the start states): the
    // vector memory counter retires in issue order, and the only operations
    // issued after the prefetch are the walk's stores (kWalkStoresPerToken
    // per token), which may stay in flight.  Were the walk to issue fewer,
    // this wait would end before the prefetch has landed.
    static_assert(kWalkStoresPerToken * S <= 63, "vmcnt field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWalkStoresPerToken * S) : "memory");
    __syncthreads();  // staged data of u - 1 visible; token sums complete
    // sum over the workgroup's wavefronts -> one partial per (token, workgroup)
    const int tot = len * OUT;
    for (int idx = tid; idx < tot; idx += 64 * kWpb) {
      const int tau = idx / OUT, o = idx % OUT;
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWpb; ww++) v += xw[(ww * S + tau) * OUT + o];
      a.part[((ta + tau) * NBW + blockIdx.y) * OUT + o] = v;
    }
    __syncthreads();  // xw free again
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < NL; j++) a.dal_part[(k * P + p) * NN + n0 + j] = -st.dal[j];
    if (grp == 0) a.dbias_part[k * P + p] = st.dbias;
  }
}
