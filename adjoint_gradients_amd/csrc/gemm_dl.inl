// gemm_dl.inl -- bf16 MFMA GEMM with direct-to-LDS operand loads for gfx950
// (included by gemm.hip after gemm_bf16.inl).
//
// C[m][n] = sum_k A[m][k] B[n][k], fp32 accumulation, each element handed to
// an epilogue.  Operands may be K-contiguous (X[r][k]) or K-outer (X[k][r]).
//
// Macro tile 256 x 256 per workgroup of four or eight wavefronts, each owning
// 128 x 128 (4 x 4) or 128 x 64 (4 x 2) tiles of v_mfma_f32_32x32x16_bf16
// (256 or 128 fp32 accumulators per lane).  K advances in stages of 32: every
// operand tile of a stage (256 x 32 bf16, 16 KB) is fetched by 16 wave-wide
// global_load_lds_dwordx4 instructions straight into LDS, so no register
// holds operands in flight and no VALU work moves them.  Four LDS stages
// (128 KB) let the loads run three stages ahead of the MFMAs; each stage is
// consumed after a vmcnt wait on the wave's own loads and one barrier.
// Tile layouts, swizzles and the operand fetches (ds_read_b128 for
// K-contiguous tiles, the transposing ds_read_b64_tr_b16 for K-outer ones)
// are defined in gemm_dl_index.hpp, where a host test checks them
// exhaustively.
//
// Edges: rows of a K-contiguous operand beyond the matrix are clamped to its
// last row, and 8-column chunks of a K-outer operand beyond it to its last
// chunk: the loads stay inside the matrix and the values they bring only
// reach output rows / columns that the epilogue discards.  The K range of
// every split must be a multiple of 32, the leading dimensions multiples of
// 8, and K-outer operands must have a multiple of 8 columns; other shapes use
// the register-staged kernel.

#include <type_traits>

#include "gemm_dl_index.hpp"

namespace gdl {

// Wavefronts of a workgroup: 2 along M (128 rows each, kBI = 4 blocks of 32)
// by WN along N (256 / WN columns, kBJ = 8 / WN blocks of 32).  WN = 2 gives
// four waves, one per SIMD with 256 accumulators per lane; WN = 4 gives
// eight, two per SIMD with 128 each, whose second wave can issue while the
// first waits on LDS.  An epilogue picks WN with kWaveCols (default 2).
template <int WN>
struct Waves {
  static constexpr int kWM = 2;
  static constexpr int kWN = WN;
  static constexpr int kBI = 4;
  static constexpr int kBJ = 8 / WN;
  static constexpr int kWaves = kWM * kWN;
  static constexpr int NT = 64 * kWaves;
  static constexpr int kLPW = kInstrPerTile / kWaves;  // load instructions per operand, wave and stage
  static constexpr int kLoadsPerWave = 2 * kLPW;       // both operands, per stage
  // Per sub-step of 16 k a wave runs kBI kBJ MFMAs; a stage's refill loads are
  // spread over the second sub-step's, one every kEvery MFMAs, A and B alternating.
  static constexpr int kEvery = kBI * kBJ / (2 * kLPW);
  static_assert(kWM * kBI * 32 == kRows && kWN * kBJ * 32 == kRows, "wave layout covers the tile");
  static_assert(kLPW * kWaves == kInstrPerTile, "loads divide over the waves");
  static_assert(kEvery >= 1 && kEvery * 2 * kLPW == kBI * kBJ, "refill spacing");
};
constexpr int NS = 4;                          // LDS stages (wait_stages covers NS <= 5)
static_assert(NS >= 3 && NS <= 5, "stage count");
constexpr int kStageBytes = 2 * kTileBytes;    // A tile, then B tile
constexpr size_t kLdsBytes = static_cast<size_t>(NS) * kStageBytes;
constexpr int kXcds = 8;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// The operand loads, the waits on them and the barrier are written as inline
// assembly.  The compiler's wait insertion does not follow LDS written by
// DMA through one dynamically indexed LDS array: given the builtin it waits
// for every outstanding load before each LDS read, and a workgroup fence
// adds a full wait before each barrier, which would serialise the pipeline.
// Here the waits are placed by hand (vmcnt counts this wave's loads in issue
// order).  The waits and the barrier carry "memory" clobbers, so no LDS
// access moves across them; the loads themselves do not, so the compiler may
// interleave them with the operand reads and MFMAs of the current stage (they
// write a stage nobody reads until the loads have been waited for), while
// volatile asm statements keep their order among themselves.

// 16 bytes from global address g (per lane) to LDS address lds + 16 * lane
// (lds wave-uniform).  M0 carries the LDS base; it is saved and restored.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g));
}

// s_waitcnt vmcnt(n): at most n of this wave's loads still outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most `n` stages' loads of this wave (n = 0 .. 3) are still
// outstanding.
template <int L>
__device__ __forceinline__ void wait_stages(int64_t n) {
  if (n >= 3) wait_vm<3 * L>();
  else if (n == 2) wait_vm<2 * L>();
  else if (n == 1) wait_vm<L>();
  else wait_vm<0>();
}

template <bool KC, int NBLK, int kLPW>
struct Operand {
  const bf16_t* base;  // wave-uniform: the tile corner at k = 0
  int64_t ld;
  uint32_t off[kLPW];  // per-lane element offsets of this wave's load instructions
  int rd[KC ? 2 : NBLK];  // per-lane byte offsets of the operand fetches (see read())

  __device__ __forceinline__ void init(const bf16_t* X, int64_t ldx, int64_t R, int64_t r0, int wave, int lane,
                                       int rb) {
    ld = ldx;
    base = X + (KC ? r0 * ldx : r0);
#pragma unroll
    for (int j = 0; j < kLPW; j++) {
      const int gi = wave * kLPW + j;
      if constexpr (KC) {
        const int64_t row = r0 + kc_load_row(gi, lane);
        const int64_t rr = (row < R ? row : R - 1) - r0;
        off[j] = static_cast<uint32_t>(rr * ldx + 8 * kc_load_chunk(gi, lane));
      } else {
        const int64_t col = 8 * static_cast<int64_t>(ko_load_chunk(gi, lane));
        const int64_t cc = (r0 + col + 8 <= R) ? col : R - 8 - r0;
        off[j] = static_cast<uint32_t>(ko_load_krow(gi, lane) * ldx + cc);
      }
    }
    if constexpr (KC) {
      rd[0] = kc_read_off(lane, rb, 0);  // + 2048 per further 32-row block, + 32 for q = 1
      rd[1] = kc_read_off(lane, rb, 1);
    } else {
#pragma unroll
      for (int i = 0; i < NBLK; i++) rd[i] = ko_read_off(lane, rb + 32 * i, 0, 0);  // + 8192 q, + 2048 h
    }
  }

  // Stage loads for K offset k0 into the tile at LDS address `tile`: this
  // wave's kLPW load instructions (issue) or its j-th one (issue_one).
  __device__ __forceinline__ void issue_one(uint32_t tile, int64_t k0, int wave, int j) const {
    const bf16_t* src = base + (KC ? k0 : k0 * ld);
    dma16(src + off[j], tile + static_cast<uint32_t>((wave * kLPW + j) * 1024));
  }
  __device__ __forceinline__ void issue(uint32_t tile, int64_t k0, int wave) const {
#pragma unroll
    for (int j = 0; j < kLPW; j++) issue_one(tile, k0, wave, j);
  }

  // MFMA operand (8 bf16) of 32-row block i of this wave, k sub-step q.
  __device__ __forceinline__ bf16x8_t read(const lds_char* tile, int i, int q) const {
    if constexpr (KC) {
      const int o = rd[q] + i * 2048;
      return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(tile + o));
    } else {
      const int o = rd[i] + q * 8192;
      typedef __attribute__((address_space(3))) v4s lv4s;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s*)(tile + o));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s*)(tile + o + 2048));
      struct Pair { v4s a, b; } pr{lo, hi};
      return __builtin_bit_cast(bf16x8_t, pr);
    }
  }
};

// Epilogues whose outputs read memory provide at_batch (loads before stores).
template <class E, class = void>
constexpr bool kHasBatchImpl = false;
template <class E>
constexpr bool kHasBatchImpl<E, decltype(&E::template at_batch<16>, void())> = true;
template <class E>
constexpr bool kHasBatch = kHasBatchImpl<E>;

// Epilogues that opt into per-wave tail variants of the K loop (kSkipTail).
template <class E, class = void>
constexpr bool kSkipTailImpl = false;
template <class E>
constexpr bool kSkipTailImpl<E, std::void_t<decltype(E::kSkipTail)>> = E::kSkipTail;

// Wave count of an epilogue's GEMM (kWaveCols wavefronts along N).
template <class E, class = void>
constexpr int kWaveColsImpl = 2;
template <class E>
constexpr int kWaveColsImpl<E, std::void_t<decltype(E::kWaveCols)>> = E::kWaveCols;
template <class Epi>
using WavesOf = Waves<kWaveColsImpl<Epi>>;

template <class Epi, bool a_kc, bool b_kc>
__global__ __launch_bounds__(WavesOf<Epi>::NT, 1) void k_gemm_dl(int64_t M, int64_t Nc, int64_t K,
                                                                const bf16_t* __restrict__ A, int64_t lda,
                                                                const bf16_t* __restrict__ B, int64_t ldb,
                                                                int64_t k_per_split, int64_t tilesM, int64_t tilesN,
                                                                Epi epi) {
  extern __shared__ __attribute__((aligned(1024))) char smem_dl[];
  lds_char* const lds = (lds_char*)(smem_dl);  // generic -> LDS address space
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  using W = WavesOf<Epi>;
  constexpr int kWN = W::kWN, kBI = W::kBI, kBJ = W::kBJ, kLPW = W::kLPW;
  constexpr int kLoadsPerWave = W::kLoadsPerWave, kEvery = W::kEvery;
  const int wm = wave / kWN, wn = wave % kWN;

  // XCD-aware bijection of the workgroup id onto (split, tile row, tile column)
  const int64_t nwg = gridDim.x;
  const int64_t pid = blockIdx.x;
  const int64_t xcd = pid % kXcds, loc = pid / kXcds;
  const int64_t full = nwg / kXcds, rem = nwg % kXcds;
  const int64_t vid = xcd < rem ? xcd * (full + 1) + loc : rem * (full + 1) + (xcd - rem) * full + loc;
  const int64_t tn = vid % tilesN;
  const int64_t tm = (vid / tilesN) % tilesM;
  const int z = static_cast<int>(vid / (tilesN * tilesM));
  const int64_t m0 = tm * kRows, n0 = tn * kRows;
  const int64_t kbeg = static_cast<int64_t>(z) * k_per_split;
  const int64_t kend = (kbeg + k_per_split < K) ? kbeg + k_per_split : K;
  const int64_t nsteps = kbeg < kend ? (kend - kbeg) / kBK : 0;

  Operand<a_kc, kBI, kLPW> oa;
  Operand<b_kc, kBJ, kLPW> ob;
  oa.init(A, lda, M, m0, wave, l, wm * (32 * kBI));
  ob.init(B, ldb, Nc, n0, wave, l, wn * (32 * kBJ));

  f32x16_t acc[kBI][kBJ];
#pragma unroll
  for (int i = 0; i < kBI; i++)
#pragma unroll
    for (int j = 0; j < kBJ; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  auto issue = [&](int64_t step) {
    const uint32_t st = lds_base + static_cast<uint32_t>((step % NS) * kStageBytes);
    oa.issue(st, kbeg + step * kBK, wave);
    ob.issue(st + kTileBytes, kbeg + step * kBK, wave);
  };

#pragma unroll
  for (int p = 0; p < NS - 1; p++)
    if (p < nsteps) issue(p);

  if constexpr (!kSkipTailImpl<Epi>) {
    // every wave runs the whole loop (the tail variants below cost the
    // weight-gradient split-K kernel more in its schedule than they save)
    // Operand fragments of one k sub-step: A blocks 0..kBI-1, B blocks 0..kBJ-1.
    struct Frags {
      bf16x8_t a[kBI], b[kBJ];
    };
    auto read_frags = [&](Frags& f, int64_t s, int q) {
      const lds_char* st = lds + (s % NS) * kStageBytes;
#pragma unroll
      for (int i = 0; i < kBI; i++) f.a[i] = oa.read(st, i, q);
#pragma unroll
      for (int j = 0; j < kBJ; j++) f.b[j] = ob.read(st + kTileBytes, j, q);
    };

    // Stage s: multiply sub-step 0 (read one sub-step earlier) with the reads
    // of sub-step 1's fragments spread between the MFMAs; then -- mid-stage --
    // wait for stage s + 1's loads and
    // pass the barrier: every wave's loads of stage s + 1 are then in LDS and
    // every wave has finished reading stage s - 1, whose LDS the loads of stage
    // s + NS - 1 refill.  Sub-step 1's MFMAs follow, with those loads (REFILL)
    // and the reads of stage s + 1's sub-step 0 fragments spread between them,
    // where the wave has issue slots to spare.  Every MFMA's operands were read
    // 16 MFMAs earlier.  At the mid-stage wait the loads issued after stage
    // s + 1's are those of stages s + 2 .. s + NS - 2 that exist.
    // Scheduling barriers keep this issue order (left alone, the scheduler
    // sinks the fragment reads next to their MFMAs and waits on each).
    Frags f0, f1;
    auto stage = [&](int64_t s, auto refill_tag, auto next_tag) {
      constexpr bool REFILL = decltype(refill_tag)::value;  // load stage s + NS - 1
      constexpr bool NEXT = decltype(next_tag)::value;      // stage s + 1 exists
      const lds_char* st0 = lds + (s % NS) * kStageBytes;
#pragma unroll
      for (int i = 0; i < kBI; i++) {
#pragma unroll
        for (int j = 0; j < kBJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.a[i], f0.b[j], acc[i][j], 0, 0, 0);
        f1.a[i] = oa.read(st0, i, 1);
        if (i < kBJ) f1.b[i < kBJ ? i : 0] = ob.read(st0 + kTileBytes, i, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NEXT) {
        // stages issued after s + 1: up to s + NS - 2 (this stage's refill comes later)
        const int64_t last = (s + NS - 2 < nsteps - 1) ? s + NS - 2 : nsteps - 1;
        wait_stages<kLoadsPerWave>(last - (s + 1));
        barrier();
      }
      const int64_t kn = kbeg + (s + NS - 1) * kBK;
      const uint32_t stn = lds_base + static_cast<uint32_t>(((s + NS - 1) % NS) * kStageBytes);
      const lds_char* st1 = lds + ((s + 1) % NS) * kStageBytes;
#pragma unroll
      for (int i = 0; i < kBI; i++) {
#pragma unroll
        for (int j = 0; j < kBJ; j++) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.a[i], f1.b[j], acc[i][j], 0, 0, 0);
          if constexpr (REFILL) {
            const int m = i * kBJ + j;
            if (m % kEvery == 0) {
              const int q = m / kEvery;
              if (q % 2 == 0) oa.issue_one(stn, kn, wave, q / 2);
              else ob.issue_one(stn + kTileBytes, kn, wave, q / 2);
            }
          }
        }
        if constexpr (NEXT) {
          f0.a[i] = oa.read(st1, i, 0);
          if (i < kBJ) f0.b[i < kBJ ? i : 0] = ob.read(st1 + kTileBytes, i, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (nsteps > 0) {
      // stages 0 .. min(NS - 1, nsteps) - 1 were issued; stage 0 must be in
      const int64_t issued = (nsteps < NS - 1) ? nsteps : NS - 1;
      wait_stages<kLoadsPerWave>(issued - 1);
      barrier();
      read_frags(f0, 0, 0);
      // Nothing pending in LGKM at the loop entry (scalar argument loads
      // included), so the loop's waits count only its own in-order LDS reads.
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    int64_t s = 0;
    for (; s + NS - 1 < nsteps; s++) stage(s, std::true_type{}, std::true_type{});
    for (; s + 1 < nsteps; s++) stage(s, std::false_type{}, std::true_type{});
    if (s < nsteps) stage(s, std::false_type{}, std::false_type{});
  } else {
    // The K loop, for a wave that multiplies its A blocks 0 .. NI-1 with its B
    // blocks 0 .. NJ-1.  Blocks that lie wholly past the matrix edge (a tail
    // tile: 2080 = 8 x 256 + 32 output columns leave one 32-wide block in the
    // last tile column) are neither fetched from LDS nor multiplied; the wave
    // still issues its share of the tile loads and meets every barrier.
    auto kloop = [&](auto ni_tag, auto nj_tag) {
      constexpr int NI = decltype(ni_tag)::value;
      constexpr int NJ = decltype(nj_tag)::value;
      // Operand fragments of one k sub-step: A blocks 0..kBI-1, B blocks 0..kBJ-1.
      struct Frags {
        bf16x8_t a[kBI], b[kBJ];
      };
      auto read_frags = [&](Frags& f, int64_t s, int q) {
        const lds_char* st = lds + (s % NS) * kStageBytes;
#pragma unroll
        for (int i = 0; i < NI; i++) f.a[i] = oa.read(st, i, q);
#pragma unroll
        for (int j = 0; j < NJ; j++) f.b[j] = ob.read(st + kTileBytes, j, q);
      };
      // Stage s: multiply sub-step 0 (read one sub-step earlier), issuing the
      // reads of sub-step 1's fragments together after the first row of MFMAs;
      // then -- mid-stage -- wait for stage s + 1's loads and pass the barrier:
      // every wave's loads of stage s + 1 are then in LDS and every wave has
      // finished reading stage s - 1, whose LDS the loads of stage s + NS - 1
      // refill.  Sub-step 1's MFMAs follow, with those loads (REFILL) spread
      // between them and the reads of stage s + 1's sub-step 0 fragments issued
      // together after its first row.  The compiler waits for all of a wave's
      // outstanding LDS reads before each sub-step's first MFMA here (the DMA
      // asm keeps it from counting them one by one), so the reads go early and
      // have landed by then: measured at 1M x 2080 x 2048, 10.1 -> 9.6 ms
      // against reads spread one row apart.  (The four-wave weight-gradient
      // GEMM measured slower with early reads and keeps them spread.)  At the
      // mid-stage wait the loads issued after stage s + 1's are those of stages
      // s + 2 .. s + NS - 2 that exist, all of them in a stage with a refill.
      // Scheduling barriers keep this issue order (left alone, the scheduler
      // moves the fragment reads next to their MFMAs and waits on each).
      Frags f0, f1;
      auto stage = [&](int64_t s, auto refill_tag, auto next_tag) {
        constexpr bool REFILL = decltype(refill_tag)::value;  // load stage s + NS - 1
        constexpr bool NEXT = decltype(next_tag)::value;      // stage s + 1 exists
        const lds_char* st0 = lds + (s % NS) * kStageBytes;
#pragma unroll
        for (int i = 0; i < kBI; i++) {
#pragma unroll
          for (int j = 0; j < kBJ; j++)
            if (i < NI && j < NJ)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.a[i], f0.b[j], acc[i][j], 0, 0, 0);
          if (i == 0) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(f1, s, 1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NEXT) {
          // stages issued after s + 1: up to s + NS - 2 (this stage's refill comes later)
          const int64_t last = (s + NS - 2 < nsteps - 1) ? s + NS - 2 : nsteps - 1;
          // a stage with a refill to come: stages s + 2 .. s + NS - 2 all in
          // flight (a constant wait keeps the loop body one basic block)
          if constexpr (REFILL) wait_vm<(NS - 3) * kLoadsPerWave>();
          else wait_stages<kLoadsPerWave>(last - (s + 1));
          barrier();
        }
        const int64_t kn = kbeg + (s + NS - 1) * kBK;
        const uint32_t stn = lds_base + static_cast<uint32_t>(((s + NS - 1) % NS) * kStageBytes);
        const lds_char* st1 = lds + ((s + 1) % NS) * kStageBytes;
#pragma unroll
        for (int i = 0; i < kBI; i++) {
#pragma unroll
          for (int j = 0; j < kBJ; j++) {
            if (i < NI && j < NJ)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.a[i], f1.b[j], acc[i][j], 0, 0, 0);
            if constexpr (REFILL) {
              const int m = i * kBJ + j;
              if (m % kEvery == 0) {
                const int q = m / kEvery;
                if (q % 2 == 0) oa.issue_one(stn, kn, wave, q / 2);
                else ob.issue_one(stn + kTileBytes, kn, wave, q / 2);
              }
            }
          }
          if constexpr (NEXT) {
            if (i == 0) {
              __builtin_amdgcn_sched_barrier(0);
              read_frags(f0, s + 1, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      if (nsteps > 0) {
        // stages 0 .. min(NS - 1, nsteps) - 1 were issued; stage 0 must be in
        const int64_t issued = (nsteps < NS - 1) ? nsteps : NS - 1;
        wait_stages<kLoadsPerWave>(issued - 1);
        barrier();
        read_frags(f0, 0, 0);
        // Nothing pending in LGKM at the loop entry (scalar argument loads
        // included), so the loop's waits count only its own in-order LDS reads.
        __builtin_amdgcn_s_waitcnt(0xC07F);
      }
      int64_t s = 0;
      for (; s + NS - 1 < nsteps; s++) stage(s, std::true_type{}, std::true_type{});
      for (; s + 1 < nsteps; s++) stage(s, std::false_type{}, std::true_type{});
      if (s < nsteps) stage(s, std::false_type{}, std::false_type{});
    };
    // Blocks of 32 rows (A) and columns (B) of this wave that hold output:
    // all inside the matrix, 0 .. all - 1 at a tail; 1 and 0 take their own
    // loop variants, the others run the full loop.
    auto nblk = [](int64_t left, int all) -> int {
      return left >= 32 * all ? all : left <= 0 ? 0 : left <= 32 ? 1 : all;
    };
    const int bi = nblk(M - (m0 + wm * (32 * kBI)), kBI), bj = nblk(Nc - (n0 + wn * (32 * kBJ)), kBJ);
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using IA = std::integral_constant<int, kBI>;
    using IB = std::integral_constant<int, kBJ>;
    if (bi == kBI) {
      if (bj == kBJ) kloop(IA{}, IB{});
      else if (bj == 1) kloop(IA{}, I1{});
      else kloop(IA{}, I0{});
    } else if (bi == 1) {
      kloop(I1{}, IB{});
    } else {
      kloop(I0{}, IB{});
    }
  }

  // Epilogue.  Lane l holds, in acc[i][j][r], row m0 + 32 kBI wm + 32 i +
  // 8 (r / 4) + 4 (l / 32) + r % 4 of column n0 + 32 kBJ wn + 32 j + l % 32.
  // The element offsets (row * ld) are stepped by additions; interior tiles
  // skip the row bound.
  const bool full_rows = m0 + kRows <= M;
  const int64_t row0 = m0 + wm * (32 * kBI) + (l >> 5) * 4;
#pragma unroll
  for (int j = 0; j < kBJ; j++) {
    const int64_t col = n0 + wn * (32 * kBJ) + j * 32 + (l & 31);
    if (col >= Nc) continue;
    const auto q = epi.prep(col, z);
    const int64_t ld = q.ld;
    int64_t oi = row0 * ld;
    if (full_rows) {
#pragma unroll
      for (int i = 0; i < kBI; i++, oi += 32 * ld) {
        if constexpr (kHasBatch<Epi>) {
          int64_t offs[16];
          float vals[16];
          int64_t orr = oi;
#pragma unroll
          for (int rr = 0; rr < 4; rr++, orr += 8 * ld) {
            int64_t o = orr;
#pragma unroll
            for (int r3 = 0; r3 < 4; r3++, o += ld) {
              offs[rr * 4 + r3] = o;
              vals[rr * 4 + r3] = acc[i][j][rr * 4 + r3];
            }
          }
          epi.at_batch(q, offs, vals);
        } else {
          int64_t orr = oi;
#pragma unroll
          for (int rr = 0; rr < 4; rr++, orr += 8 * ld) {
            int64_t o = orr;
#pragma unroll
            for (int r3 = 0; r3 < 4; r3++, o += ld) epi.at(q, o, acc[i][j][rr * 4 + r3]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBI; i++, oi += 32 * ld) {
        int64_t orr = oi;
#pragma unroll
        for (int rr = 0; rr < 4; rr++, orr += 8 * ld) {
          int64_t o = orr;
#pragma unroll
          for (int r3 = 0; r3 < 4; r3++, o += ld)
            if (row0 + i * 32 + rr * 8 + r3 < M) epi.at(q, o, acc[i][j][rr * 4 + r3]);
        }
      }
    }
  }
}

// Whether the direct-to-LDS kernel takes this GEMM (see the header comment).
inline bool supports(const GemmOperands& op, int64_t kps) {
  if (op.M < 1 || op.Nc < 1 || op.K < 1) return false;
  if (op.lda % 8 != 0 || op.ldb % 8 != 0) return false;
  if (kps % kBK != 0 || op.K % kBK != 0) return false;
  if (!op.a_kc && op.M % 8 != 0) return false;
  if (!op.b_kc && op.Nc % 8 != 0) return false;
  // per-lane 32-bit element offsets
  const int64_t span_a = op.a_kc ? kRows * op.lda : kBK * op.lda;
  const int64_t span_b = op.b_kc ? kRows * op.ldb : kBK * op.ldb;
  return span_a < (int64_t(1) << 31) && span_b < (int64_t(1) << 31);
}

template <class Epi, bool AKC, bool BKC>
hipError_t run_t(const GemmOperands& op, int splits, int64_t kps, Epi epi, hipStream_t st) {
  const int64_t tilesM = (op.M + kRows - 1) / kRows, tilesN = (op.Nc + kRows - 1) / kRows;
  const int64_t nwg = tilesM * tilesN * splits;
  constexpr int NT = WavesOf<Epi>::NT;
  auto kern = k_gemm_dl<Epi, AKC, BKC>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
  if (e != hipSuccess) return e;
  kern<<<static_cast<unsigned>(nwg), NT, kLdsBytes, st>>>(op.M, op.Nc, op.K, static_cast<const bf16_t*>(op.A),
                                                         op.lda, static_cast<const bf16_t*>(op.B), op.ldb, kps,
                                                         tilesM, tilesN, epi);
  return hipGetLastError();
}

// Each epilogue is instantiated for the operand layouts its GEMM has: the
// projection X W_cat^T (both K-contiguous), the weight gradient dY^T X (both
// K-outer) and the input cotangent dY W_cat (A K-contiguous, B K-outer).
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

}  // namespace gdl
