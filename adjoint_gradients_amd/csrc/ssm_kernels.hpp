// ssm_kernels.hpp -- internal launch interface between the C ABI (api.hip)
// and the kernel files.  Host-side declarations only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Optional timing marks: caller-owned hipEvent_t handles recorded on the
// stream at the boundaries of the internal phases (NULL entries skipped).
// Optional per-launch marks bracket each launch of the fused reverse kernel
// (entries 2 s and 2 s + 1 around the launch over chunk slab s).
struct Marks {
  void* const* ev = nullptr;
  int n = 0;
  void* const* slab_ev = nullptr;
  int slab_n = 0;
  void rec(int i, hipStream_t st) const {
    if (ev && i < n && ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), st);
  }
  void rec_slab(int i, hipStream_t st) const {
    if (slab_ev && i < slab_n && slab_ev[i]) (void)hipEventRecord(static_cast<hipEvent_t>(slab_ev[i]), st);
  }
};

// Sub-chunk start states of the gradient kernel: the state entering token
// kC + kSub u of chunk k, for channel block cb (CH = 64 / G channels) and lane
// l = grp CH + pl of the scan layout, state n = grp NL + j, stored at float
// offset hsub_offset(k - k0, cb, u, NB, nsub_max, NL) + j 64 + l, nsub_max =
// ceil(C / kSub), where k0 is the first chunk the region holds.  Written
// either by the final forward scan for every chunk (k0 = 0, when the caller
// keeps them) or by a pass of the gradient, one slab of chunks at a time
// into a region of the workspace that holds one slab.
constexpr int kSub = 8;  // tokens per recomputed sub-chunk
__host__ __device__ constexpr int64_t hsub_offset(int64_t k, int64_t cb, int64_t u, int64_t NB, int64_t nsub_max,
                                                  int NL) {
  return ((k * NB + cb) * nsub_max + u) * (static_cast<int64_t>(NL) * 64);
}

struct FwdArgs {
  int64_t T, P, N;
  int C;
  const float* s;       // [T][P] softplus(Delta)
  const void* x;        // [T][P] io
  const float* b;       // [T][N]
  const float* c;       // [T][N]
  const float* alpha;   // [P][N]
  float* hloc;          // [K][P][N] workspace
  double* ssum;         // [K][P]   per-chunk sum of s (saved)
  float* h_ckpt;        // [K][P][N] saved
  float* y;             // [T][P]
  float* hsub = nullptr;  // optional: sub-chunk start states (bwd_hsub_floats floats)
  float* hall = nullptr;  // optional: every state, h_t after token t (hsub_offset layout with
                          // one-token sub-chunks: hsub_offset(k, cb, t - kC, NB, C, NL))
  Marks marks{};        // phases 2..4: after local scan, carry, final scan
};

struct BwdArgs {
  int64_t T, P, N, W;   // W: window (>= T means exact)
  int C;
  const float* s;       // [T][P]
  const void* x;        // [T][P] io
  const float* b;       // [T][N]
  const float* c;       // [T][N]
  const float* alpha;   // [P][N]
  const float* h_ckpt;  // [K][P][N]
  const double* ssum;   // [K][P]
  const float* g;       // [T][P]
  // workspace
  double* ps64;         // [K+1][P] prefix sums of ssum over chunks (windowed)
  double* hwin;         // [K][P]   sum of s over the W tokens after each chunk (windowed)
  float* umu;           // [K][P][N] local adjoint aggregates
  float* carry;         // [K][P][N] adjoint carry entering each chunk from the right
  float* edge;          // [P][N] carry handed from one slab of chunks to the next one left
  float* part;          // [T][NBW][2N] per-workgroup partial sums of db | dc
  float* dal_part;      // [K][P][N]
  float* dbias_part;    // [K][P]
  float* hsub;          // per-wavefront sub-chunk start states (hsub_offset layout)
  int hsub_ready;       // 1: a separate pass already wrote hsub (the main kernel skips its walk)
  int hsub_given;       // 1: hsub was written by the forward for every chunk (no pass needed)
  int64_t hsub_chunks;  // chunks the hsub region holds (the slab; all chunks when given)
  int64_t k_lo;         // first chunk of a launch over a slab (set by the launcher)
  int64_t hsub_k0;      // chunk held by the region's first slot (set by the launcher)
  const float* hall;    // every state kept by the forward (store-everything baseline), or nullptr
  // outputs of the scan
  void* dY;             // [T][ldy] io: columns [0,P) = dDelta, [P,P+N) = db, [P+N,P+2N) = dc
  int64_t ldy;
  float* dxdir;         // [T][P] or nullptr
  float* dalpha;        // [P][N] or nullptr
  float* dbias;         // [P] or nullptr
  Marks marks{};        // phases 1..4: after local aggregates, carry, main, reductions
};

// Layout queries of the backward scan (shared by the workspace planner).
struct BwdPlan {
  int NL, G, CH, S;
  int wpb;              // waves per workgroup of the main kernel
  int64_t NB;           // channel blocks (of CH channels)
  int64_t NBW;          // workgroups along channels = ceil(NB / wpb)
  size_t lds_bytes;     // dynamic LDS of the main kernel
};
bool bwd_plan(int64_t P, int64_t N, int C, BwdPlan* plan);
// Floats of sub-chunk states for `chunks` chunks.
size_t bwd_hsub_floats_chunks(int64_t chunks, int64_t P, int64_t N, int C);
// Floats of sub-chunk states for every chunk of T tokens (the forward's h_sub).
size_t bwd_hsub_floats(int64_t T, int64_t P, int64_t N, int C);
// Floats of every state of T tokens in the one-token-sub-chunk layout (the
// store-everything baseline's buffer).
size_t bwd_hall_floats(int64_t T, int64_t P, int64_t N, int C);
// Chunks per segment of the gradient's carry scan: kSegLen, or kSegLenShort
// when the default slab holds few chunks (the length follows from the shapes
// alone).  Slabs that start at multiples of kSegLen give the same carries,
// bit for bit, whatever their size.
constexpr int kSegLen = 16;
constexpr int kSegLenShort = 4;
static_assert(kSegLen % kSegLenShort == 0, "both segment lengths divide kSegLen");
// Chunks per slab of the gradient's own sub-chunk-state region: at most
// kHsubSlabBytes of states, a multiple of 32 chunks when that many fit (else
// of kSegLen when that many fit), never more than the chunk count.
constexpr size_t kHsubSlabBytes = size_t(1) << 30;
int64_t bwd_hsub_slab_chunks(int64_t T, int64_t P, int64_t N, int C);

hipError_t launch_forward_scan(const FwdArgs& a, bool bf16, hipStream_t st);

// RMS normalisation of the residual stream (norm.hip).  Forward: xio =
// io(gamma r rinv), rinv per row, rcopy = r.  VJP for the cotangent d of xio:
// delta += dr, dgamma (may be null) = sum over rows; m [T] and part
// [norm_row_blocks(T)][P] are scratch.
constexpr float kNormEps = 1e-5f;
int64_t norm_row_blocks(int64_t T);
hipError_t rmsnorm_forward(int64_t T, int64_t P, const float* r, const float* gamma, float eps, void* xio,
                           bool bf16, float* rinv, float* rcopy, hipStream_t st);
hipError_t rmsnorm_vjp(int64_t T, int64_t P, const float* r, const float* rinv, const float* gamma, const float* d,
                       float* m, float* delta, float* part, float* dgamma, hipStream_t st);
hipError_t launch_backward_scan(const BwdArgs& a, bool bf16, hipStream_t st);

// ---------------------------------------------------------------- GEMMs
// C[M][Nc] = sum_k A(m,k) B(k,n) on MFMA, with one of three epilogues.
//   A(m,k) = a_kc ? A[m*lda + k] : A[k*lda + m]
//   B(k,n) = b_kc ? B[n*ldb + k] : B[k*ldb + n]
struct GemmOperands {
  int64_t M, Nc, K;
  const void* A; int64_t lda; bool a_kc;
  const void* B; int64_t ldb; bool b_kc;
};

// Projection epilogue: columns [0,P) -> s = softplus(v + bias), [P,P+N) -> b, [P+N,P+2N) -> c.
struct EpiProjArgs { int64_t P, N; const float* bias; float* s; float* b; float* c; };
hipError_t gemm_projection(const GemmOperands& op, bool bf16, const EpiProjArgs& e, hipStream_t st);

// Split-K partial sums: part[z][M][Nc] for z < splits.
hipError_t gemm_splitk(const GemmOperands& op, bool bf16, int splits, float* part, hipStream_t st);

// Input-cotangent epilogue: out[m][n] = v + add0[m][n] (+ add1[m][n]); ld = Nc.
struct EpiAddArgs { const float* add0; const float* add1; float* out; };
hipError_t gemm_add(const GemmOperands& op, bool bf16, const EpiAddArgs& e, hipStream_t st);

// Sum of the split-K partials into the three weight-gradient outputs
// (rows [0,P) -> dW_delta, [P,P+N) -> dW_B, [P+N,P+2N) -> dW_C).
hipError_t reduce_weight_grads(const float* part, int splits, int64_t P, int64_t N, float* dWd, float* dWb,
                               float* dWc, hipStream_t st);

// ---------------------------------------------------------------- stack helpers
// r += y (if y; the sum goes to rout instead of r when rout is set) ; xio = io(r + y)
hipError_t residual_update(int64_t n, float* r, const float* y, void* xio, bool bf16, hipStream_t st,
                           float* rout = nullptr);
// r = io value of x0 (float32 residual stream initialised from the io input)
hipError_t residual_init(int64_t n, const void* x0, bool bf16, float* r, hipStream_t st);

}  // namespace ssm
