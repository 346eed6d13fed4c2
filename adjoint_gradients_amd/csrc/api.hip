// api.hip -- the C ABI declared in include/ssm_adjoint.h.
//
// Every entry point validates its arguments completely before the first
// enqueue, carves its scratch buffers out of the caller's workspace (no
// allocation, no synchronisation) and launches the kernels on the caller's
// stream.  The launch order is the method's data flow:
//   forward:  pack W_cat -> projection GEMM (s, b, c) -> chunk-local scan ->
//             chunk carry (checkpoints) -> final scan (y)
//   gradient: reverse local aggregates -> reverse carry -> fused reverse
//             adjoint + local VJPs -> db/dc channel sums -> split-K weight
//             gradient GEMM -> reduction (+ input-cotangent GEMM)
//   stack:    K forwards with the residual update, then the layers in reverse
//             with the total cotangent (Proposition 3 of the review of
//             "Adjoint sharding for very long context training of state space
//             models", Core claim).
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/ssm_adjoint.h"
#include "ssm_kernels.hpp"

namespace {

using ssm::BwdArgs;
using ssm::BwdPlan;
using ssm::FwdArgs;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sequential carve-out of a workspace; in "plan" mode only sizes are summed.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T> T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

bool supported_N(int64_t N) {
  return N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64;
}

ssm_status check_dims(const ssm_dims* d) {
  if (!d) return SSM_ERR_ARG;
  if (d->T < 1 || d->P < 1 || d->N < 1 || d->chunk < 1) return SSM_ERR_ARG;
  if (d->io != SSM_F32 && d->io != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (!supported_N(d->N) || d->chunk > 512) return SSM_ERR_UNSUPPORTED;
  if (d->T > (int64_t(1) << 31) || d->P > (int64_t(1) << 20)) return SSM_ERR_UNSUPPORTED;
  BwdPlan pl;
  if (!ssm::bwd_plan(d->P, d->N, d->chunk, &pl)) return SSM_ERR_UNSUPPORTED;
  return SSM_OK;
}

int64_t nchunks(const ssm_dims* d) { return (d->T + d->chunk - 1) / d->chunk; }
size_t io_size(const ssm_dims* d) { return d->io == SSM_BF16 ? 2 : 4; }

ssm_status check_layer(const ssm_layer* L) {
  if (!L || !L->W_delta || !L->W_B || !L->W_C || !L->alpha) return SSM_ERR_ARG;
  if (!aligned16(L->W_delta) || !aligned16(L->W_B) || !aligned16(L->W_C) || !aligned16(L->alpha))
    return SSM_ERR_ARG;
  if (L->delta_bias && !aligned16(L->delta_bias)) return SSM_ERR_ARG;
  if (L->norm_scale && !aligned16(L->norm_scale)) return SSM_ERR_ARG;
  return SSM_OK;
}

ssm_status check_saved(const ssm_saved* s) {
  if (!s || !s->s || !s->b || !s->c || !s->h_ckpt || !s->s_sum) return SSM_ERR_ARG;
  if (!aligned16(s->s) || !aligned16(s->b) || !aligned16(s->c) || !aligned16(s->h_ckpt) || !aligned16(s->s_sum))
    return SSM_ERR_ARG;
  if (s->h_sub && !aligned16(s->h_sub)) return SSM_ERR_ARG;
  if (s->h_all && !aligned16(s->h_all)) return SSM_ERR_ARG;
  if (s->h_sub && s->h_all) return SSM_ERR_ARG;  // one kind of kept states at most
  return SSM_OK;
}

ssm_status check_grads(const ssm_grads* g) {
  if (!g || !g->dW_delta || !g->dW_B || !g->dW_C) return SSM_ERR_ARG;
  const void* ps[] = {g->dW_delta, g->dW_B, g->dW_C, g->dalpha, g->dbias, g->dx, g->dnorm_scale};
  for (const void* p : ps)
    if (p && !aligned16(p)) return SSM_ERR_ARG;
  return SSM_OK;
}

ssm_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return SSM_OK;
  if (!ws) return SSM_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return SSM_ERR_WORKSPACE;
  if (have < need) return SSM_ERR_WORKSPACE;
  return SSM_OK;
}

// ---------------------------------------------------------------- workspace plans

struct FwdWs {
  void* wcat;
  float* hloc;
};

FwdWs carve_fwd(Carver& cv, const ssm_dims* d) {
  FwdWs w;
  const int64_t M = d->P + 2 * d->N;
  w.wcat = cv.take<char>(static_cast<size_t>(M * d->P) * io_size(d));
  w.hloc = cv.take<float>(static_cast<size_t>(nchunks(d) * d->P * d->N));
  return w;
}

int splitk_for(const ssm_dims* d) {
  const int64_t M = d->P + 2 * d->N;
  if (d->io == SSM_BF16) {
    // 256 x 256 tiles, one workgroup per CU at a time on 256 CUs: pick the
    // split count (8..64, at least 512 tokens each) whose workgroup count
    // fills the last round best; ties go to fewer splits
    const int64_t tiles = ((M + 255) / 256) * ((d->P + 255) / 256);
    int best = 1;
    double best_eff = -1.0;
    for (int s = 8; s <= 64; s++) {
      if (d->T / s < 512) break;
      const int64_t wg = tiles * s;
      const double eff = static_cast<double>(wg) / (256.0 * static_cast<double>((wg + 255) / 256));
      if (eff > best_eff + 1e-9) {
        best_eff = eff;
        best = s;
      }
    }
    return best;
  }
  const int64_t tiles = ((M + 127) / 128) * ((d->P + 127) / 128);
  int64_t s = 2048 / (tiles > 0 ? tiles : 1);
  const int64_t cap = d->T / 512;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

struct BwdWs {
  void* wcat;      // only when dx is needed
  void* dY;
  float* dxdir;    // only in the stack (a single layer writes dx_dir into its dx output)
  float* part;
  float* umu;
  float* carry;
  float* edge;
  double* ps64;
  double* hwin;
  float* dal_part;
  float* dbias_part;
  float* hsub;
  int64_t hsub_chunks;  // chunks the hsub region holds (one slab)
  float* wpart;
  int splits;
};

// own_hsub: the workspace holds a slab of sub-chunk states (the caller did
// not keep them); own_dxdir: the direct input cotangent needs a buffer of its
// own (the stack, whose cotangent stream is read while it is written);
// slab_chunks > 0: chunks per slab instead of the default
BwdWs carve_bwd(Carver& cv, const ssm_dims* d, int64_t W, bool need_dx, bool own_hsub = true,
                bool own_dxdir = false, int64_t slab_chunks = 0) {
  BwdWs w;
  BwdPlan pl;
  ssm::bwd_plan(d->P, d->N, d->chunk, &pl);
  const int64_t T = d->T, P = d->P, N = d->N, K = nchunks(d);
  const int64_t M = P + 2 * N;
  const bool win = W < T;
  w.wcat = need_dx ? cv.take<char>(static_cast<size_t>(M * P) * io_size(d)) : nullptr;
  w.dY = cv.take<char>(static_cast<size_t>(T * M) * io_size(d));
  w.dxdir = (need_dx && own_dxdir) ? cv.take<float>(static_cast<size_t>(T * P)) : nullptr;
  w.part = cv.take<float>(static_cast<size_t>(T * pl.NBW * 2 * N));
  w.umu = cv.take<float>(static_cast<size_t>(K * P * N + P));  // + P: also the chunk-reduction scratch
  w.carry = cv.take<float>(static_cast<size_t>(K * P * N));
  w.edge = cv.take<float>(static_cast<size_t>(P * N));
  w.ps64 = win ? cv.take<double>(static_cast<size_t>((K + 1) * P)) : nullptr;
  w.hwin = win ? cv.take<double>(static_cast<size_t>(K * P)) : nullptr;
  w.dal_part = cv.take<float>(static_cast<size_t>(K * P * N));
  w.dbias_part = cv.take<float>(static_cast<size_t>(K * P));
  w.hsub_chunks = !own_hsub ? K
                  : slab_chunks > 0 ? (slab_chunks < K ? slab_chunks : K)
                                    : ssm::bwd_hsub_slab_chunks(T, P, N, d->chunk);
  w.hsub = own_hsub ? cv.take<float>(ssm::bwd_hsub_floats_chunks(w.hsub_chunks, P, N, d->chunk)) : nullptr;
  w.splits = splitk_for(d);
  w.wpart = cv.take<float>(static_cast<size_t>(w.splits) * M * P);
  return w;
}

ssm_saved carve_saved(Carver& cv, const ssm_dims* d) {
  ssm_saved s;
  const int64_t T = d->T, P = d->P, N = d->N, K = nchunks(d);
  s.s = cv.take<float>(static_cast<size_t>(T * P));
  s.b = cv.take<float>(static_cast<size_t>(T * N));
  s.c = cv.take<float>(static_cast<size_t>(T * N));
  s.h_ckpt = cv.take<float>(static_cast<size_t>(K * P * N));
  s.s_sum = cv.take<double>(static_cast<size_t>(K * P));
  s.h_sub = nullptr;  // the stack keeps only the chunk checkpoints
  s.h_all = nullptr;
  return s;
}

size_t fwd_ws_bytes(const ssm_dims* d) {
  Carver cv(nullptr);
  carve_fwd(cv, d);
  return cv.off;
}

size_t bwd_ws_bytes(const ssm_dims* d, int64_t W, bool need_dx, bool own_hsub = true, bool own_dxdir = false,
                    int64_t slab_chunks = 0) {
  Carver cv(nullptr);
  carve_bwd(cv, d, W, need_dx, own_hsub, own_dxdir, slab_chunks);
  return cv.off;
}

// Normalisation buffers of the stack, present only when KN >= 1 of its layers
// normalise: per such layer the residual r^k and 1/rms per token (kept for
// the VJP, slot = the layer's rank among the normalising ones), the layer's
// dx, and the VJP's row scratch.
struct NormWs {
  float* rk;      // [KN][T][P]
  float* rinv;    // [KN][T]
  float* dx;      // [T][P]
  float* m;       // [T]
  float* part;    // [row blocks][P]
};

NormWs carve_norm(Carver& cv, const ssm_dims* d, int32_t KN) {
  NormWs n{};
  if (KN < 1) return n;
  const int64_t T = d->T, P = d->P;
  n.rk = cv.take<float>(static_cast<size_t>(KN) * T * P);
  n.rinv = cv.take<float>(static_cast<size_t>(KN) * T);
  n.dx = cv.take<float>(static_cast<size_t>(T * P));
  n.m = cv.take<float>(static_cast<size_t>(T));
  n.part = cv.take<float>(static_cast<size_t>(ssm::norm_row_blocks(T) * P));
  return n;
}

// Workspace of a stack of K layers of which KN normalise their input.
size_t stack_ws_bytes(const ssm_dims* d, int64_t W, int32_t K, int32_t KN) {
  Carver cv(nullptr);
  for (int32_t k = 0; k < K; k++) carve_saved(cv, d);
  cv.take<char>(static_cast<size_t>(K) * d->T * d->P * io_size(d));
  cv.take<float>(static_cast<size_t>(d->T * d->P));
  cv.take<float>(static_cast<size_t>(d->T * d->P));
  cv.take<float>(static_cast<size_t>(d->T * d->P));
  carve_norm(cv, d, KN);
  const size_t f = fwd_ws_bytes(d), b = bwd_ws_bytes(d, W, true, true, true);
  return cv.off + (f > b ? f : b);
}

int32_t count_norm(int32_t K, const ssm_layer* layers) {
  int32_t n = 0;
  for (int32_t k = 0; k < K; k++) n += layers[k].norm_scale ? 1 : 0;
  return n;
}

// ---------------------------------------------------------------- internal passes

hipError_t pack_wcat(const ssm_dims* d, const ssm_layer* L, void* wcat, hipStream_t st) {
  const size_t es = io_size(d);
  const size_t rowb = static_cast<size_t>(d->P) * es;
  char* dst = static_cast<char*>(wcat);
  hipError_t e = hipMemcpyAsync(dst, L->W_delta, rowb * d->P, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(dst + rowb * d->P, L->W_B, rowb * d->N, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return e;
  return hipMemcpyAsync(dst + rowb * (d->P + d->N), L->W_C, rowb * d->N, hipMemcpyDeviceToDevice, st);
}

hipError_t run_forward(const ssm_dims* d, const ssm_layer* L, const void* x, float* y, const ssm_saved* sv,
                       const FwdWs& w, hipStream_t st, ssm::Marks mk = {}) {
  const bool bf = d->io == SSM_BF16;
  mk.rec(0, st);
  hipError_t e = pack_wcat(d, L, w.wcat, st);
  if (e != hipSuccess) return e;
  ssm::GemmOperands op{d->T, d->P + 2 * d->N, d->P, x, d->P, true, w.wcat, d->P, true};
  ssm::EpiProjArgs ep{d->P, d->N, L->delta_bias, sv->s, sv->b, sv->c};
  e = ssm::gemm_projection(op, bf, ep, st);
  if (e != hipSuccess) return e;
  mk.rec(1, st);
  FwdArgs fa{d->T, d->P, d->N, d->chunk, sv->s, x, sv->b, sv->c, L->alpha, w.hloc, sv->s_sum, sv->h_ckpt, y};
  fa.hsub = sv->h_sub;
  fa.hall = sv->h_all;
  fa.marks = mk;
  return ssm::launch_forward_scan(fa, bf, st);
}

// Gradient of one layer.  If delta_out is set (stack), dx is folded into the
// cotangent stream: delta_out <- delta_in + dx (delta_out may be delta_in);
// otherwise dx goes to grads->dx when requested.
hipError_t run_backward(const ssm_dims* d, const ssm_layer* L, const void* x, const ssm_saved* sv,
                        const float* g, int64_t W, const ssm_grads* gr, const float* delta_in, float* delta_out,
                        const BwdWs& w, hipStream_t st, ssm::Marks mk = {}) {
  mk.rec(0, st);
  const bool bf = d->io == SSM_BF16;
  const int64_t T = d->T, P = d->P, N = d->N;
  const int64_t M = P + 2 * N;
  const bool need_dx = (delta_out != nullptr) || (gr->dx != nullptr);
  BwdArgs a{};
  a.T = T; a.P = P; a.N = N; a.W = W; a.C = d->chunk;
  a.s = sv->s; a.x = x; a.b = sv->b; a.c = sv->c; a.alpha = L->alpha; a.h_ckpt = sv->h_ckpt;
  a.ssum = sv->s_sum; a.g = g;
  a.ps64 = w.ps64; a.hwin = w.hwin; a.umu = w.umu; a.carry = w.carry; a.edge = w.edge; a.part = w.part;
  a.dal_part = w.dal_part; a.dbias_part = w.dbias_part;
  a.hsub = sv->h_sub ? sv->h_sub : w.hsub;
  a.hsub_given = sv->h_sub ? 1 : 0;
  a.hall = sv->h_all;
  a.hsub_chunks = w.hsub_chunks;
  a.dY = w.dY; a.ldy = M;
  // the direct input cotangent: the stack's own buffer (its cotangent stream
  // is g here, read while dx_dir is written), else the dx output itself,
  // which the input-cotangent GEMM then completes in place
  float* dxdir = delta_out ? w.dxdir : gr->dx;
  a.dxdir = need_dx ? dxdir : nullptr;
  a.dalpha = gr->dalpha; a.dbias = gr->dbias;
  a.marks = mk;
  hipError_t e = ssm::launch_backward_scan(a, bf, st);
  if (e != hipSuccess) return e;
  // dW_cat = dY^T X  (K = T, both operands token-major)
  ssm::GemmOperands op{M, P, T, w.dY, M, false, x, P, false};
  e = ssm::gemm_splitk(op, bf, w.splits, w.wpart, st);
  if (e != hipSuccess) return e;
  e = ssm::reduce_weight_grads(w.wpart, w.splits, P, N, gr->dW_delta, gr->dW_B, gr->dW_C, st);
  if (e != hipSuccess) return e;
  mk.rec(5, st);
  if (need_dx) {
    e = pack_wcat(d, L, w.wcat, st);
    if (e != hipSuccess) return e;
    // dx = dY W_cat + dxdir  (+ delta for the stack, in place)
    ssm::GemmOperands opx{T, P, M, w.dY, M, true, w.wcat, P, false};
    ssm::EpiAddArgs ea{dxdir, delta_out ? delta_in : nullptr, delta_out ? delta_out : gr->dx};
    e = ssm::gemm_add(opx, bf, ea, st);
  }
  mk.rec(6, st);
  return e;
}

}  // namespace

// ---------------------------------------------------------------- no-allocation gradient
// ssm_adjoint_grad_noalloc takes its workspace from this array instead of the
// caller.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is obtained once per device with
// hipGetSymbolAddress (each device holds its own copy) and only that address
// is used.  Calls on one device share the array, so calls that overlap on a
// device race; nothing in it needs to start at zero (every element the
// gradient reads was written earlier in the same call).
constexpr size_t kNoAllocScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

struct ScratchTable {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
static ScratchTable g_scratch;

// Device address of the current device's scratch array (looked up on its
// first use on that device, with that device current).
static ssm_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SSM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSM_ERR_HIP;
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return SSM_OK;
}

extern "C" {

int32_t ssm_version(void) { return 301; }

const char* ssm_status_str(int32_t s) {
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_ARG: return "SSM_ERR_ARG: invalid argument";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: kernel launch failed";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: shape or dtype not supported";
    default: return "SSM_ERR_UNKNOWN";
  }
}

size_t ssm_saved_bytes(const ssm_dims* d) {
  if (check_dims(d) != SSM_OK) return 0;
  Carver cv(nullptr);
  carve_saved(cv, d);
  return cv.off;
}

size_t ssm_sub_state_bytes(const ssm_dims* d) {
  if (check_dims(d) != SSM_OK) return 0;
  return ssm::bwd_hsub_floats(d->T, d->P, d->N, d->chunk) * sizeof(float);
}

size_t ssm_stack_workspace_bytes(int32_t K, const ssm_dims* d, const ssm_layer* layers, int64_t window) {
  if (check_dims(d) != SSM_OK || K < 1 || K > 64 || !layers || window < 1) return 0;
  return stack_ws_bytes(d, window < d->T ? window : d->T, K, count_norm(K, layers));
}

int32_t ssm_grad_slab_count(const ssm_dims* d, int64_t window, int32_t sub_states_given) {
  if (check_dims(d) != SSM_OK || window < 1) return 0;
  if (sub_states_given) return 1;
  const int64_t K = nchunks(d);
  const int64_t slab = ssm::bwd_hsub_slab_chunks(d->T, d->P, d->N, d->chunk);
  return static_cast<int32_t>((K + slab - 1) / slab);
}

size_t ssm_all_state_bytes(const ssm_dims* d) {
  if (check_dims(d) != SSM_OK) return 0;
  return ssm::bwd_hall_floats(d->T, d->P, d->N, d->chunk) * sizeof(float);
}

size_t ssm_grad_workspace_bytes_sub(const ssm_dims* d, int64_t window) {
  if (check_dims(d) != SSM_OK || window < 1) return 0;
  return bwd_ws_bytes(d, window < d->T ? window : d->T, true, false);
}

size_t ssm_workspace_bytes(const ssm_dims* d, int64_t window, int32_t K) {
  if (check_dims(d) != SSM_OK) return 0;
  if (K < 0 || window < 0) return 0;
  if (K >= 1) {
    if (window < 1) return 0;
    return stack_ws_bytes(d, window, K, 0);
  }
  if (window == 0) return fwd_ws_bytes(d);
  return bwd_ws_bytes(d, window, true);
}

static ssm_status forward_impl(const ssm_dims* d, const ssm_layer* L, const void* x, float* y,
                               const ssm_saved* sv, void* ws, size_t ws_bytes, void* stream, ssm::Marks mk) {
  ssm_status s = check_dims(d);
  if (s != SSM_OK) return s;
  if ((s = check_layer(L)) != SSM_OK) return s;
  if (L->norm_scale) return SSM_ERR_ARG;  // normalisation belongs to the stack
  if ((s = check_saved(sv)) != SSM_OK) return s;
  if (!x || !y || !aligned16(x) || !aligned16(y)) return SSM_ERR_ARG;
  if (mk.n < 0 || (mk.n > 0 && !mk.ev)) return SSM_ERR_ARG;
  if ((s = check_ws(ws, ws_bytes, fwd_ws_bytes(d))) != SSM_OK) return s;
  Carver cv(ws);
  FwdWs w = carve_fwd(cv, d);
  hipError_t e = run_forward(d, L, x, y, sv, w, static_cast<hipStream_t>(stream), mk);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

// Argument checks of the single-layer gradient (everything but the workspace).
static ssm_status check_adjoint(const ssm_dims* d, const ssm_layer* L, const void* x, const ssm_saved* sv,
                                const float* g, int64_t window, const ssm_grads* gr) {
  ssm_status s = check_dims(d);
  if (s != SSM_OK) return s;
  if ((s = check_layer(L)) != SSM_OK) return s;
  if (L->norm_scale) return SSM_ERR_ARG;  // normalisation belongs to the stack
  if ((s = check_saved(sv)) != SSM_OK) return s;
  if ((s = check_grads(gr)) != SSM_OK) return s;
  if (!x || !g || !aligned16(x) || !aligned16(g)) return SSM_ERR_ARG;
  if (window < 1) return SSM_ERR_ARG;
  return SSM_OK;
}

static ssm_status adjoint_impl(const ssm_dims* d, const ssm_layer* L, const void* x, const ssm_saved* sv,
                               const float* g, int64_t window, const ssm_grads* gr, void* ws, size_t ws_bytes,
                               void* stream, ssm::Marks mk, int64_t slab_chunks = 0) {
  ssm_status s = check_adjoint(d, L, x, sv, g, window, gr);
  if (s != SSM_OK) return s;
  if (mk.n < 0 || (mk.n > 0 && !mk.ev)) return SSM_ERR_ARG;
  const int64_t W = window < d->T ? window : d->T;
  const bool need_dx = gr->dx != nullptr;
  const bool own_hsub = sv->h_sub == nullptr && sv->h_all == nullptr;
  if ((s = check_ws(ws, ws_bytes, bwd_ws_bytes(d, W, need_dx, own_hsub, false, slab_chunks))) != SSM_OK) return s;
  Carver cv(ws);
  BwdWs w = carve_bwd(cv, d, W, need_dx, own_hsub, false, slab_chunks);
  hipError_t e = run_backward(d, L, x, sv, g, W, gr, nullptr, nullptr, w, static_cast<hipStream_t>(stream), mk);
  return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}


ssm_status ssm_adjoint_grad_noalloc(const ssm_dims* d, const ssm_layer* L, const void* x, const ssm_saved* sv,
                                    const float* g, int64_t window, const ssm_grads* gr, void* stream) {
  ssm_status s = check_adjoint(d, L, x, sv, g, window, gr);
  if (s != SSM_OK) return s;
  const int64_t W = window < d->T ? window : d->T;
  const bool need_dx = gr->dx != nullptr;
  const bool own_hsub = sv->h_sub == nullptr && sv->h_all == nullptr;
  // everything but the sub-chunk-state slab must fit; the rest of the array
  // holds as large a slab as fits (at most the default one)
  const size_t fixed = bwd_ws_bytes(d, W, need_dx, false);
  if (fixed > kNoAllocScratchBytes) return SSM_ERR_WORKSPACE;
  int64_t slab = 0;
  if (own_hsub) {
    const size_t per = ssm::bwd_hsub_floats_chunks(1, d->P, d->N, d->chunk) * sizeof(float);
    const size_t room = kNoAllocScratchBytes - fixed;
    slab = per ? static_cast<int64_t>(room / per) : 0;
    while (slab > 0 && bwd_ws_bytes(d, W, need_dx, true, false, slab) > kNoAllocScratchBytes) slab--;
    if (slab < 1) return SSM_ERR_WORKSPACE;
    const int64_t dflt = ssm::bwd_hsub_slab_chunks(d->T, d->P, d->N, d->chunk);
    if (slab > dflt) slab = dflt;
    // slabs at multiples of the carry's segments give the default path's values bit for bit
    if (slab < dflt && slab >= ssm::kSegLen) slab -= slab % ssm::kSegLen;
  }
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != SSM_OK) return s;
  return adjoint_impl(d, L, x, sv, g, window, gr, ws, kNoAllocScratchBytes, stream, ssm::Marks{}, slab);
}

ssm_status ssm_forward(const ssm_dims* d, const ssm_layer* L, const void* x, float* y, const ssm_saved* sv,
                       void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(d, L, x, y, sv, ws, ws_bytes, stream, ssm::Marks{});
}

ssm_status ssm_adjoint_grad(const ssm_dims* d, const ssm_layer* L, const void* x, const ssm_saved* sv,
                            const float* g, int64_t window, const ssm_grads* gr, void* ws, size_t ws_bytes,
                            void* stream) {
  return adjoint_impl(d, L, x, sv, g, window, gr, ws, ws_bytes, stream, ssm::Marks{});
}

ssm_status ssm_forward_timed(const ssm_dims* d, const ssm_layer* L, const void* x, float* y, const ssm_saved* sv,
                             void* ws, size_t ws_bytes, void* stream, void* const* events, int32_t n_events) {
  ssm::Marks mk;
  mk.ev = events;
  mk.n = n_events;
  return forward_impl(d, L, x, y, sv, ws, ws_bytes, stream, mk);
}

ssm_status ssm_adjoint_grad_timed(const ssm_dims* d, const ssm_layer* L, const void* x, const ssm_saved* sv,
                                  const float* g, int64_t window, const ssm_grads* gr, void* ws, size_t ws_bytes,
                                  void* stream, void* const* events, int32_t n_events) {
  ssm::Marks mk;
  mk.ev = events;
  mk.n = n_events < 7 ? n_events : 7;
  if (events && n_events > 7) {
    mk.slab_ev = events + 7;
    mk.slab_n = n_events - 7;
  }
  return adjoint_impl(d, L, x, sv, g, window, gr, ws, ws_bytes, stream, mk);
}

ssm_status ssm_stack_grad(int32_t K, const ssm_dims* d, const ssm_layer* layers, const void* x0, const float* g,
                          int64_t window, const ssm_grads* grads, float* dx0, float* xK, void* ws,
                          size_t ws_bytes, void* stream) {
  ssm_status s = check_dims(d);
  if (s != SSM_OK) return s;
  if (K < 1 || !layers || !grads) return SSM_ERR_ARG;
  if (K > 64) return SSM_ERR_UNSUPPORTED;
  for (int32_t k = 0; k < K; k++) {
    if ((s = check_layer(&layers[k])) != SSM_OK) return s;
    if ((s = check_grads(&grads[k])) != SSM_OK) return s;
    if (grads[k].dx) return SSM_ERR_ARG;  // per-layer dx is internal to the stack; use dx0
  }
  if (!x0 || !g || !aligned16(x0) || !aligned16(g)) return SSM_ERR_ARG;
  if ((dx0 && !aligned16(dx0)) || (xK && !aligned16(xK))) return SSM_ERR_ARG;
  if (window < 1) return SSM_ERR_ARG;
  const int64_t W = window < d->T ? window : d->T;
  const int32_t KN = count_norm(K, layers);
  if ((s = check_ws(ws, ws_bytes, stack_ws_bytes(d, W, K, KN))) != SSM_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = d->io == SSM_BF16;
  const int64_t TP = d->T * d->P;
  const size_t xbytes = static_cast<size_t>(TP) * io_size(d);

  Carver cv(ws);
  ssm_saved saved[64];
  ssm_saved* sv = saved;
  for (int32_t k = 0; k < K; k++) sv[k] = carve_saved(cv, d);
  char* xs = cv.take<char>(static_cast<size_t>(K) * xbytes);
  float* r = cv.take<float>(static_cast<size_t>(TP));
  float* y = cv.take<float>(static_cast<size_t>(TP));
  float* delta = cv.take<float>(static_cast<size_t>(TP));
  NormWs nw = carve_norm(cv, d, KN);
  int32_t nslot[64];  // rank of each normalising layer among them (its r^k, 1/rms slot)
  for (int32_t k = 0, q = 0; k < K; k++) nslot[k] = layers[k].norm_scale ? q++ : -1;
  const size_t shared_off = cv.off;
  const int64_t T = d->T, P = d->P;
  // x^k = io(r^k), or the normalised stream for a layer with norm_scale
  // (which also keeps r^k and 1/rms for its VJP)
  auto make_input = [&](int32_t k) -> hipError_t {
    void* xk = xs + static_cast<size_t>(k) * xbytes;
    if (layers[k].norm_scale)
      return ssm::rmsnorm_forward(T, P, r, layers[k].norm_scale, ssm::kNormEps, xk, bf, nw.rinv + nslot[k] * T,
                                  nw.rk + static_cast<size_t>(nslot[k]) * TP, st);
    return ssm::residual_update(TP, r, nullptr, xk, bf, st);
  };

  hipError_t e = ssm::residual_init(TP, x0, bf, r, st);
  if (e != hipSuccess) return SSM_ERR_HIP;
  if ((e = make_input(0)) != hipSuccess) return SSM_ERR_HIP;
  for (int32_t k = 0; k < K; k++) {
    void* xk = xs + static_cast<size_t>(k) * xbytes;
    Carver fc(static_cast<char*>(ws) + shared_off);
    FwdWs fw = carve_fwd(fc, d);
    if ((e = run_forward(d, &layers[k], xk, y, &sv[k], fw, st)) != hipSuccess) return SSM_ERR_HIP;
    // r^{k+1} = r^k + y^k, then x^{k+1} (fused into the update when it is a plain cast)
    const bool plain_next = k + 1 < K && !layers[k + 1].norm_scale;
    void* xnext = plain_next ? xs + static_cast<size_t>(k + 1) * xbytes : nullptr;
    // the last layer's sum is the output x_K itself (r is not read afterwards)
    float* rout = (k + 1 == K && xK) ? xK : nullptr;
    if ((e = ssm::residual_update(TP, r, y, xnext, bf, st, rout)) != hipSuccess) return SSM_ERR_HIP;
    if (k + 1 < K && !plain_next && (e = make_input(k + 1)) != hipSuccess) return SSM_ERR_HIP;
  }
  // The cotangent stream delta starts as g.  A plain top layer reads g itself
  // and writes g + dx^{K-1} into delta; a normalised one updates delta in
  // place, so delta is first a copy of g.
  const bool top_plain = !layers[K - 1].norm_scale;
  if (!top_plain &&
      (e = hipMemcpyAsync(delta, g, static_cast<size_t>(TP) * 4, hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return SSM_ERR_HIP;
  for (int32_t k = K - 1; k >= 0; k--) {
    void* xk = xs + static_cast<size_t>(k) * xbytes;
    Carver bc(static_cast<char*>(ws) + shared_off);
    BwdWs bw = carve_bwd(bc, d, W, true, true, true);
    // layer k is driven by delta^{k+1}; then delta^k = delta^{k+1} + dx^k, or
    // + the normalisation's VJP of dx^k
    if (layers[k].norm_scale) {
      ssm_grads gl = grads[k];
      gl.dx = nw.dx;
      if ((e = run_backward(d, &layers[k], xk, &sv[k], delta, W, &gl, nullptr, nullptr, bw, st)) != hipSuccess)
        return SSM_ERR_HIP;
      if ((e = ssm::rmsnorm_vjp(T, P, nw.rk + static_cast<size_t>(nslot[k]) * TP, nw.rinv + nslot[k] * T,
                                layers[k].norm_scale,
                                nw.dx, nw.m, delta, nw.part, grads[k].dnorm_scale, st)) != hipSuccess)
        return SSM_ERR_HIP;
    } else {
      // cotangent of this layer: g for a plain top layer, else delta; the
      // bottom layer's sum goes straight to dx0
      const float* cot = (k == K - 1) ? g : delta;
      float* out = (k == 0 && dx0) ? dx0 : delta;
      if ((e = run_backward(d, &layers[k], xk, &sv[k], cot, W, &grads[k], cot, out, bw, st)) != hipSuccess)
        return SSM_ERR_HIP;
    }
  }
  if (dx0 && layers[0].norm_scale) {
    if ((e = hipMemcpyAsync(dx0, delta, static_cast<size_t>(TP) * 4, hipMemcpyDeviceToDevice, st)) != hipSuccess)
      return SSM_ERR_HIP;
  }
  return SSM_OK;
}

}  // extern "C"
