"""ssm_adjoint_grad_noalloc (the gradient with the library's own device
array as workspace) against ssm_adjoint_grad on the same inputs: two calls in
a row, the second smaller, each bitwise equal to the workspace entry point
(same kernels; the slab grouping of chunks does not change any value)."""
import numpy as np
import pytest

from gpu_util import layer_tensors, say, to_dev
from ssm_inputs import make_layer, small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import adjoint_gradients_amd  # noqa: F401  (fails loudly if the library is missing)


def _both(T, P, N, io, window, chunk, sub_states, seed):
    import torch

    import adjoint_gradients_amd as agm

    inp = make_layer(small_case(T, P, N, seed, io=io))
    dims = agm.make_dims(T, P, N, chunk, io)
    lay = layer_tensors(inp, io)
    x, g = to_dev(inp["x"], io), to_dev(inp["g"])
    y, saved = agm.forward(dims, lay, x, sub_states=sub_states)
    ref = agm.adjoint_grad(dims, lay, x, saved, g, window, want_dx=True)
    got = agm.alloc_grads(dims, want_dx=True, device=x.device)
    for v in got.values():
        v.fill_(float("nan"))
    agm.ssm_adjoint_grad_noalloc(dims, lay.struct(dims), x, agm.saved_struct(saved, dims), g, window,
                                 agm.grads_struct(got, dims))
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in ref.items()}, {k: v.cpu().numpy() for k, v in got.items()})


def test_noalloc_matches_workspace_entry_point():
    import adjoint_gradients_amd as agm

    cases = [
        # (T, P, N, io, window, chunk, sub-chunk states kept, seed): the first
        # needs several slabs of rebuilt states in the array, the second is
        # smaller and reuses the array the first left behind.  The fourth (a
        # window of whole chunks, so the chunk aggregates and the carries are
        # formed slab by slab) runs 2 slabs of 80 and 48 chunks in the array
        # against 1 slab of 128 in the workspace entry point: the segmented
        # carry must give the same bits either way.
        (32768, 512, 16, "f32", 1000, 256, False, 71),
        (4096, 256, 16, "bf16", 4096, 256, False, 72),
        (3000, 96, 32, "f32", 512, 128, True, 73),
        (32768, 512, 16, "f32", 4096, 256, False, 74),
    ]
    for T, P, N, io, W, C, sub, seed in cases:
        d = agm.make_dims(T, P, N, C, io)
        say(f"case noalloc T={T} P={P} N={N} io={io} W={W} C={C} sub_states={sub} "
            f"(workspace entry point needs {agm.ssm_workspace_bytes(d, W, 0) / 2**20:.0f} MiB)")
        ref, got = _both(T, P, N, io, W, C, sub, seed)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), k
        say("  bitwise equal: " + ", ".join(sorted(ref)))
