// gemm_bf16.inl -- large-tile bf16 MFMA GEMM for gfx950 (included by gemm.hip).
//
// Macro tile 256 x 256 x 64 per 512-thread workgroup; each of the 8
// wavefronts owns a 128 x 64 sub-tile = 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane), so two
// wavefronts share each SIMD and hide each other's memory waits.  One barrier per K step: the next K step's operand
// tiles are loaded from global memory into registers while the current one
// is multiplied out of LDS, then written to the other LDS buffer.
// Operands whose reduction index is the slow (outer) index in memory are
// transposed in registers on their way to LDS: every thread loads an 8 x 8
// block of bf16 (8 rows of 16 bytes) and rebuilds it column-wise with
// v_perm_b32, so both LDS tiles are always [row][k] and every MFMA operand
// fetch is one 16-byte LDS read.
// The 1-D grid is remapped so consecutive tiles of one output row band land
// on the same XCD (the hardware deals workgroups round-robin over the 8 XCDs),
// which keeps the shared operand band in that XCD's L2.

#include <type_traits>

namespace gbf {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements): 144 bytes
constexpr int NT = 512;      // 8 wavefronts: 2 (rows) x 4 (columns) of 128 x 64
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// K-contiguous operand X[r][k]: 256 rows x 64 k = 2048 chunks of 16 bytes,
// 4 per thread; 8 consecutive threads read one 128-byte row segment.
__device__ __forceinline__ void load_kc(uint4 (&v)[4], const bf16_t* __restrict__ X, int64_t ld, int64_t R,
                                        int64_t kend, int64_t r0, int64_t k0, int tid, bool vec_ok) {
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int c = tid + NT * r;
    const int row = c >> 3, kc = (c & 7) * 8;
    const int64_t gr = r0 + row, gk = k0 + kc;
    if (vec_ok && gr < R && gk + 8 <= kend) {
      v[r] = *reinterpret_cast<const uint4*>(X + gr * ld + gk);
    } else {
      alignas(16) bf16_t e[8];
#pragma unroll
      for (int q = 0; q < 8; q++) e[q] = (gr < R && gk + q < kend) ? X[gr * ld + gk + q] : bf16_t(0);
      v[r] = *reinterpret_cast<const uint4*>(e);
    }
  }
}

__device__ __forceinline__ void store_kc(bf16_t* lds, const uint4 (&v)[4], int tid) {
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int c = tid + NT * r;
    const int row = c >> 3, kc = (c & 7) * 8;
    *reinterpret_cast<uint4*>(lds + row * LDK + kc) = v[r];
  }
}

// K-outer operand X[k][r]: 64 k x 256 rows = 256 blocks of 8 x 8, one per
// thread of a 256-thread half (t = tid & 255): kb = t & 7 picks the 8 k-rows,
// rb = t >> 3 the 8 columns.  After the transpose, the 8 threads sharing rb
// write the 8 k-chunks of the same LDS rows (one 128-byte segment each), so
// the stores are free of bank conflicts.
__device__ __forceinline__ void load_ko(uint4 (&v)[8], const bf16_t* __restrict__ X, int64_t ld, int64_t R,
                                        int64_t kend, int64_t r0, int64_t k0, int t, bool vec_ok) {
  const int kb = t & 7, rb = t >> 3;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int64_t gk = k0 + kb * 8 + i, gr = r0 + rb * 8;
    if (vec_ok && gk < kend && gr + 8 <= R) {
      v[i] = *reinterpret_cast<const uint4*>(X + gk * ld + gr);
    } else {
      alignas(16) bf16_t e[8];
#pragma unroll
      for (int q = 0; q < 8; q++) e[q] = (gk < kend && gr + q < R) ? X[gk * ld + gr + q] : bf16_t(0);
      v[i] = *reinterpret_cast<const uint4*>(e);
    }
  }
}

__device__ __forceinline__ void store_ko(bf16_t* lds, const uint4 (&v)[8], int t) {
  const int kb = t & 7, rb = t >> 3;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    uint32_t o[4];
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const uint32_t lo = dword_of(v[2 * d], j >> 1), hi = dword_of(v[2 * d + 1], j >> 1);
      o[d] = __builtin_amdgcn_perm(hi, lo, (j & 1) ? 0x07060302u : 0x05040100u);
    }
    *reinterpret_cast<uint4*>(lds + (rb * 8 + j) * LDK + kb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// One operand's global -> register -> LDS staging.  K-outer operands are
// handled by one half of the workgroup (A: threads 0..255, B: 256..511).
struct Operand {
  const bf16_t* X;
  int64_t ld, R;
  bool kc, vec;
  int half;  // 0 for A, 1 for B
};

template <class Epi, bool a_kc, bool b_kc>
__global__ __launch_bounds__(512) void k_gemm_bf16(int64_t M, int64_t Nc, int64_t K, const bf16_t* __restrict__ A,
                                                   int64_t lda, const bf16_t* __restrict__ B, int64_t ldb,
                                                   int64_t k_per_split, int64_t tilesM, int64_t tilesN, Epi epi) {
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* As = smem;                  // [2][BM][LDK]
  bf16_t* Bs = smem + 2 * BM * LDK;   // [2][BN][LDK]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int half = __builtin_amdgcn_readfirstlane(tid >> 8), t256 = tid & 255;

  // XCD-aware bijection of the workgroup id onto (split, tile row, tile column)
  const int64_t nwg = gridDim.x;
  const int64_t pid = blockIdx.x;
  const int64_t xcd = pid % kXcds, loc = pid / kXcds;
  const int64_t full = nwg / kXcds, rem = nwg % kXcds;
  const int64_t vid = xcd < rem ? xcd * (full + 1) + loc : rem * (full + 1) + (xcd - rem) * full + loc;
  const int64_t tn = vid % tilesN;
  const int64_t tm = (vid / tilesN) % tilesM;
  const int z = static_cast<int>(vid / (tilesN * tilesM));
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t kbeg = static_cast<int64_t>(z) * k_per_split;
  const int64_t kend = (kbeg + k_per_split < K) ? kbeg + k_per_split : K;
  const bool a_vec = (lda % 8) == 0, b_vec = (ldb % 8) == 0;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  // staging registers: 4 chunks per K-contiguous operand, 8 for the K-outer
  // operand(s) (one 8 x 8 block per thread of the owning half)
  uint4 ka[a_kc ? 4 : 1], kb4[b_kc ? 4 : 1], ko[(a_kc && b_kc) ? 1 : 8];
  auto load = [&](int64_t k0) {
    if constexpr (a_kc) load_kc(ka, A, lda, M, kend, m0, k0, tid, a_vec);
    else if (half == 0) load_ko(ko, A, lda, M, kend, m0, k0, t256, a_vec);
    if constexpr (b_kc) load_kc(kb4, B, ldb, Nc, kend, n0, k0, tid, b_vec);
    else if (half == 1) load_ko(ko, B, ldb, Nc, kend, n0, k0, t256, b_vec);
  };
  auto store = [&](int buf) {
    if constexpr (a_kc) store_kc(As + buf * BM * LDK, ka, tid);
    else if (half == 0) store_ko(As + buf * BM * LDK, ko, t256);
    if constexpr (b_kc) store_kc(Bs + buf * BN * LDK, kb4, tid);
    else if (half == 1) store_ko(Bs + buf * BN * LDK, ko, t256);
  };

  if (kbeg < kend) {
    load(kbeg);
    store(0);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) load(k0 + BK);
    const bf16_t* as = As + buf * BM * LDK + (wm * 128 + (l & 31)) * LDK + (l >> 5) * 8;
    const bf16_t* bs = Bs + buf * BN * LDK + (wn * 64 + (l & 31)) * LDK + (l >> 5) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; i++)
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(as + i * 32 * LDK + kk));
#pragma unroll
      for (int j = 0; j < 2; j++)
        bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(bs + j * 32 * LDK + kk));
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int64_t col = n0 + wn * 64 + j * 32 + (l & 31);
    if (col < Nc) {
      const auto q = epi.prep(col, z);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int64_t row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3);
          if (row < M) epi.apply(q, row, acc[i][j][r]);
        }
    }
  }
}

constexpr size_t kLdsBytes = static_cast<size_t>(2) * (BM + BN) * LDK * sizeof(bf16_t);

template <class Epi, bool AKC, bool BKC>
hipError_t run_t(const GemmOperands& op, int splits, int64_t kps, Epi epi, hipStream_t st) {
  const int64_t tilesM = (op.M + BM - 1) / BM, tilesN = (op.Nc + BN - 1) / BN;
  const int64_t nwg = tilesM * tilesN * splits;
  auto kern = k_gemm_bf16<Epi, AKC, BKC>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (e != hipSuccess) return e;
  kern<<<static_cast<unsigned>(nwg), NT, kLdsBytes, st>>>(op.M, op.Nc, op.K, static_cast<const bf16_t*>(op.A),
                                                         op.lda, static_cast<const bf16_t*>(op.B), op.ldb, kps,
                                                         tilesM, tilesN, epi);
  return hipGetLastError();
}

// The three layouts this library uses: projections (A, B both K-contiguous),
// weight gradient (both K-outer), input cotangent (A K-contiguous, B K-outer).
// Each epilogue is instantiated for its own GEMM's layout only.
template <class Epi>
hipError_t run(const GemmOperands& op, int splits, int64_t kps, Epi epi, hipStream_t st) {
  if constexpr (std::is_same_v<Epi, EpiProj>) {
    if (op.a_kc && op.b_kc) return run_t<Epi, true, true>(op, splits, kps, epi, st);
  } else if constexpr (std::is_same_v<Epi, EpiPart>) {
    if (!op.a_kc && !op.b_kc) return run_t<Epi, false, false>(op, splits, kps, epi, st);
  } else {
    if (op.a_kc && !op.b_kc) return run_t<Epi, true, false>(op, splits, kps, epi, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gbf
