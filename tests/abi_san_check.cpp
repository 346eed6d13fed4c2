// Drives the C ABI's host-side paths -- size queries, workspace planning and
// argument validation -- on tiny and on full-size shapes, for a host-only
// build with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py).  No call here reaches a device: every
// gradient, forward and stack call is given an argument the validation
// rejects (no device code is built into this binary), so any out-of-bounds
// access or undefined arithmetic in the planning and checks stops the run.
#include <stdint.h>
#include <stdio.h>

#include "../include/ssm_adjoint.h"

#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main() {
  const ssm_dims shapes[] = {
      {1, 1, 1, 1, SSM_F32},           {300, 40, 8, 3, SSM_F32},          {1000, 96, 16, 64, SSM_BF16},
      {512, 48, 64, 256, SSM_F32},     {76800, 1024, 32, 256, SSM_F32},   {1 << 20, 2048, 16, 256, SSM_BF16},
      {262144, 1536, 64, 256, SSM_BF16}, {int64_t(1) << 31, 8, 1, 512, SSM_F32},
  };
  void* fake = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned, never dereferenced
  ssm_layer L{fake, fake, fake, static_cast<const float*>(fake), nullptr, nullptr};
  ssm_saved S{static_cast<float*>(fake), static_cast<float*>(fake), static_cast<float*>(fake),
              static_cast<float*>(fake), static_cast<double*>(fake), nullptr};
  ssm_grads G{static_cast<float*>(fake), static_cast<float*>(fake), static_cast<float*>(fake),
              nullptr, nullptr, nullptr, nullptr};
  for (const ssm_dims& d : shapes) {
    const size_t sv = ssm_saved_bytes(&d), sub = ssm_sub_state_bytes(&d);
    const size_t fw = ssm_workspace_bytes(&d, 0, 0);
    const size_t bw = ssm_workspace_bytes(&d, 100, 0), bwx = ssm_workspace_bytes(&d, d.T, 0);
    const size_t bs = ssm_grad_workspace_bytes_sub(&d, 100);
    const size_t st = ssm_workspace_bytes(&d, 100, 3);
    ssm_layer ls[3] = {L, L, L};
    ls[1].norm_scale = static_cast<const float*>(fake);
    const size_t stn = ssm_stack_workspace_bytes(3, &d, ls, 100);
    const int32_t slabs = ssm_grad_slab_count(&d, 100, 0);
    EXPECT(sv > 0 && sub > 0 && fw > 0 && bw > 0 && bwx > 0 && bs > 0 && st > 0 && stn > st && slabs >= 1);
    EXPECT(bs < bw);
    // validation failures: nothing is launched
    EXPECT(ssm_forward(&d, &L, fake, static_cast<float*>(fake), &S, fake, fw - 1, nullptr) == SSM_ERR_WORKSPACE);
    EXPECT(ssm_forward(&d, nullptr, fake, static_cast<float*>(fake), &S, fake, fw, nullptr) == SSM_ERR_ARG);
    EXPECT(ssm_adjoint_grad(&d, &L, fake, &S, static_cast<float*>(fake), 0, &G, fake, bw, nullptr) ==
           SSM_ERR_ARG);
    // (a workspace far below any requirement: this call must not get past validation)
    EXPECT(ssm_adjoint_grad(&d, &L, fake, &S, static_cast<float*>(fake), 100, &G, fake, 256, nullptr) ==
           SSM_ERR_WORKSPACE);
    ssm_grads G0 = G;
    G0.dW_B = nullptr;
    EXPECT(ssm_adjoint_grad(&d, &L, fake, &S, static_cast<float*>(fake), 100, &G0, fake, bw, nullptr) ==
           SSM_ERR_ARG);
    EXPECT(ssm_adjoint_grad_noalloc(&d, &L, fake, &S, static_cast<float*>(fake), -1, &G, nullptr) == SSM_ERR_ARG);
    ssm_grads gs[3] = {G, G, G};
    EXPECT(ssm_stack_grad(3, &d, ls, fake, static_cast<float*>(fake), 100, gs, nullptr, nullptr, fake, st,
                          nullptr) == SSM_ERR_WORKSPACE);
    EXPECT(ssm_stack_grad(0, &d, ls, fake, static_cast<float*>(fake), 100, gs, nullptr, nullptr, fake, stn,
                          nullptr) == SSM_ERR_ARG);
    EXPECT(ssm_stack_grad(65, &d, ls, fake, static_cast<float*>(fake), 100, gs, nullptr, nullptr, fake, stn,
                          nullptr) == SSM_ERR_UNSUPPORTED);
  }
  // the full-size gradient's fixed buffers exceed the no-allocation array
  EXPECT(ssm_adjoint_grad_noalloc(&shapes[5], &L, fake, &S, static_cast<float*>(fake), 4096, &G, nullptr) ==
         SSM_ERR_WORKSPACE);
  // unsupported and invalid dims
  const ssm_dims bad[] = {{0, 8, 4, 16, SSM_F32}, {8, 8, 3, 16, SSM_F32}, {8, 8, 4, 513, SSM_F32},
                          {8, 8, 4, 16, 7}, {(int64_t(1) << 31) + 1, 8, 4, 16, SSM_F32}};
  for (const ssm_dims& d : bad) {
    EXPECT(ssm_saved_bytes(&d) == 0 && ssm_workspace_bytes(&d, 0, 0) == 0 && ssm_grad_slab_count(&d, 1, 0) == 0);
    EXPECT(ssm_forward(&d, &L, fake, static_cast<float*>(fake), &S, fake, 1 << 20, nullptr) != SSM_OK);
  }
  EXPECT(ssm_saved_bytes(nullptr) == 0);
  for (int32_t c = -1; c < 6; c++) EXPECT(ssm_status_str(c) != nullptr);
  EXPECT(ssm_status_str(INT32_MIN) != nullptr && ssm_status_str(INT32_MAX) != nullptr);
  printf("ABI sanitizer run OK (version %d)\n", ssm_version());
  return 0;
}
