"""GPU test of gdn2_chunk_bwd_noalloc, the backward entry point that
allocates nothing (its workspace is the library's own device array): its
outputs must equal those of gdn2_chunk_bwd with a caller workspace, bit for
bit, on two calls in a row, the second on a smaller input (the array keeps
the first call's contents, which the second must not depend on)."""
import numpy as np
import pytest

import gpu_util as G
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "db", "dw", "d_initial_state")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def _case(seed, dtype, **shape):
    rng = np.random.default_rng(seed + 1)
    x = W.make("batched_bf16", seed=seed, dtype=dtype, **shape)
    B, T, H, _ = x["q"].shape
    dv = x["v"].shape[-1]
    dk = x["q"].shape[-1]
    N = B if x.get("cu_seqlens") is None else len(x["cu_seqlens"]) - 1
    g = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    if dtype == "bf16":
        g = W.round_bf16(g)
    gs = rng.standard_normal((N, H, dk, dv)).astype(np.float32)
    return x, g, gs


def _both(x, g, gs, dtype):
    import torch

    d = G.to_dev(x, dtype)
    dg = W.to_torch(g, dtype, "cuda")
    dgs = torch.from_numpy(gs).cuda()
    ref = binding.gdn2_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], dg, d["initial_state"], dgs,
                                 cu_seqlens=d["cu_seqlens"])
    out = {n: torch.full_like(ref[n], float("nan")) for n in GRADS}
    got = binding.gdn2_chunk_bwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], dg, d["initial_state"],
                                         dgs, out=out, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_entry_twice():
    import torch

    cap = binding.gdn2_chunk_bwd_noalloc_max_workspace_bytes()
    calls = [("bf16", dict(B=2, T=300, H=4, dk=128, dv=128), 501),   # the larger call first
             ("f32", dict(B=1, T=70, H=2, dk=64, dv=32), 502)]       # then a smaller one
    for dtype, shape, seed in calls:
        x, g, gs = _case(seed, dtype, **shape)
        ws = binding.gdn2_chunk_bwd_workspace_bytes(shape["B"], shape["T"], shape["H"], shape["dk"], shape["dv"], 0,
                                                    binding.DTYPE_BF16 if dtype == "bf16" else binding.DTYPE_F32)
        assert 0 < ws <= cap
        G.log(f"noalloc backward {dtype} {shape}: workspace {ws} bytes of {cap}")
        ref, got = _both(x, g, gs, dtype)
        for n in GRADS:
            assert torch.equal(got[n], ref[n]), f"{dtype} {shape}: {n} differs from gdn2_chunk_bwd"
            G.assert_rel(G.f64(got[n]), G.f64(ref[n]), G.TOL[dtype], f"noalloc {dtype} {n}")
