"""GPU parity of gdn2_recurrent_fwd, the fused recurrent form over T tokens
per sequence in one call (needs an MI355X).

Checks: the FP64 oracle on the same tokens; bitwise equality with T calls of
the single-token step (the state round-trips through HBM in FP32 between
steps, which is exact, so the two must agree bit for bit); the handoff from a
chunkwise prefill to a multi-token continuation against the oracle on the
whole sequence; compact gate layouts against the full layout."""
import numpy as np
import pytest

import gpu_util as G
import oracle
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def _inputs(seed, N, T, H, dk, dv, dtype, gate_mode="gdn2"):
    """[N, T, H, .] token tensors and an N(0, 0.1^2) state [N, H, dk, dv]."""
    x = W.make("batched_bf16", gate_mode=gate_mode, seed=seed, B=N, T=T, H=H, dk=dk, dv=dv, dtype=dtype)
    x["initial_state"] = 0.1 * np.random.default_rng(seed + 1).standard_normal((N, H, dk, dv)).astype(np.float32)
    return x


def _run(d, state, gates=binding.GATES_FULL):
    import torch

    o = binding.gdn2_recurrent_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], state, gates=gates)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 32, 32), ("f32", 64, 128), ("f32", 128, 64),
                                         ("bf16", 128, 128), ("bf16", 64, 32)])
@pytest.mark.parametrize("T", [1, 2, 7, 23, 24, 64, 130])
def test_recurrent_fwd_parity(dtype, dk, dv, T):
    """N=6 sequences x 3 heads, T tokens each, random initial state.  For
    bf16 with dk = 128, T = 23 is the longest call the recurrent kernel
    takes and T = 24 the shortest the chunkwise kernel takes."""
    import torch

    x = _inputs(120 + T, 6, T, 3, dk, dv, dtype)
    d = G.to_dev(x, dtype)
    state = torch.from_numpy(x["initial_state"]).cuda()
    o = _run(d, state)
    ro, rs = G.oracle_full(x)
    what = f"recurrent_fwd {dtype} dk={dk} dv={dv} T={T}"
    G.assert_rel(G.f64(o), ro, G.TOL[dtype], f"{what} o")
    G.assert_rel(G.f64(state), rs, G.TOL[dtype], f"{what} state")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_recurrent_fwd_equals_steps(dtype, d):
    """T = 9 tokens in one call == nine single-token steps, bit for bit."""
    import torch

    T, N, H = 9, 10, 4
    x = _inputs(131, N, T, H, d, d, dtype)
    dd = G.to_dev(x, dtype)
    s_multi = torch.from_numpy(x["initial_state"]).cuda()
    s_step = s_multi.clone()
    o = _run(dd, s_multi)
    for t in range(T):
        sl = {n: dd[n][:, t].contiguous() for n in G.NAMES}
        ot = binding.gdn2_recurrent_step(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["b"], sl["w"], s_step)
        torch.cuda.synchronize()
        assert torch.equal(ot, o[:, t]), f"token {t}: multi-token and stepped outputs differ"
    assert torch.equal(s_multi, s_step), "multi-token and stepped final states differ"


@pytest.mark.parametrize("P,T", [(256, 16), (300, 64), (64, 1), (1, 40)])
def test_prefill_then_multi_token(P, T):
    """Chunkwise prefill of P tokens (bf16, d=128: the matrix-core kernel), then
    T tokens in one recurrent call continuing from its final state; compared
    with the oracle on the whole P + T token sequence."""
    import torch

    N, H, d = 4, 8, 128
    x = _inputs(140 + P + T, N, P + T, H, d, d, "bf16")
    d_all = G.to_dev(x, "bf16")
    pre = {n: d_all[n][:, :P].contiguous() for n in G.NAMES}
    post = {n: d_all[n][:, P:].contiguous() for n in G.NAMES}
    s0 = torch.from_numpy(x["initial_state"]).cuda()
    o_pre, state = binding.gdn2_chunk_fwd(pre["q"], pre["k"], pre["v"], pre["alpha"], pre["b"], pre["w"], s0)
    o_post = _run(post, state)
    ro, rs = G.oracle_full(x)
    what = f"prefill {P} + {T}"
    G.assert_rel(G.f64(o_pre), ro[:, :P], G.TOL["bf16"], f"{what}: prefill o")
    G.assert_rel(G.f64(o_post), ro[:, P:], G.TOL["bf16"], f"{what}: continuation o")
    G.assert_rel(G.f64(state), rs, G.TOL["bf16"], f"{what}: final state")


@pytest.mark.parametrize("gates", [binding.GATES_KDA, binding.GATES_GDN, binding.GATES_SCALAR_WRITE])
def test_recurrent_fwd_gate_layouts(gates):
    """Compact gates over 12 tokens == the full layout on broadcast gates, bit
    for bit; the oracle on the broadcast gates."""
    import torch

    import test_gpu_gates as TG

    T, N, H, d = 12, 8, 4, 128
    x = _inputs(150, N, T, H, d, d, "bf16")
    arrs, xb = TG.averaged(x, gates, "bf16")
    dd = G.to_dev(xb, "bf16")
    cb, cw, ca = TG._dev_compact(arrs, "bf16")
    s_c = torch.from_numpy(x["initial_state"]).cuda()
    s_f = s_c.clone()
    oc = binding.gdn2_recurrent_fwd(dd["q"], dd["k"], dd["v"], ca, cb, cw, s_c, gates=gates)
    of = _run(dd, s_f)
    assert torch.equal(oc, of) and torch.equal(s_c, s_f), f"layout {gates}: compact and full differ"
    ro, rs = G.oracle_full(xb)
    G.assert_rel(G.f64(oc), ro, G.TOL["bf16"], f"recurrent_fwd layout {gates} o")
    G.assert_rel(G.f64(s_c), rs, G.TOL["bf16"], f"recurrent_fwd layout {gates} state")


def test_recurrent_fwd_verification_shape():
    """256 sequences x 16 heads, d=128, bf16, 16 tokens per call (a verification
    step): every chain against the oracle."""
    import torch

    x = _inputs(160, 256, 16, 16, 128, 128, "bf16")
    d = G.to_dev(x, "bf16")
    state = torch.from_numpy(x["initial_state"]).cuda()
    o = _run(d, state)
    ro, rs = G.oracle_full(x)
    G.assert_rel(G.f64(o), ro, G.TOL["bf16"], "verification shape o")
    G.assert_rel(G.f64(state), rs, G.TOL["bf16"], "verification shape state")


def test_recurrent_fwd_zero_tokens():
    import torch

    x = _inputs(170, 3, 0, 2, 64, 64, "bf16")
    d = G.to_dev(x, "bf16")
    state = torch.from_numpy(x["initial_state"]).cuda()
    before = state.clone()
    o = _run(d, state)
    assert o.shape == (3, 0, 2, 64)
    assert torch.equal(state, before)
