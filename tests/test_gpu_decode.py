"""GPU parity of gdn2_recurrent_step (fused decode) against the FP64 oracle,
and the cross-mode identity chunkwise == stepped (needs an MI355X)."""
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


def _step_all(x, dtype, state):
    """Run the decode step over every pre-generated slice; x[name]: [steps, N, H, d]."""
    import torch

    outs = []
    for t in range(x["q"].shape[0]):
        sl = {n: x[n][t] for n in G.NAMES}
        d = G.to_dev(dict(sl, initial_state=None), dtype)
        outs.append(binding.gdn2_recurrent_step(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"],
                                                state))
    torch.cuda.synchronize()
    return torch.stack(outs)  # [steps, N, H, dv]


def _as_sequences(x):
    """[steps, N, H, d] decode slices -> [N, steps, H, d] sequences for the oracle."""
    return {n: np.ascontiguousarray(np.swapaxes(x[n], 0, 1)) for n in G.NAMES}


def test_tiny_f32_stepped():
    """The tiny FP32 case (H=2, dk=dv=32, 256 tokens) stepped token by token."""
    import torch

    x = W.make("tiny_f32")
    steps = {n: np.ascontiguousarray(np.swapaxes(x[n], 0, 1)) for n in G.NAMES}  # [T, 1, H, d]
    state = torch.zeros((1, 2, 32, 32), dtype=torch.float32, device="cuda")
    o = _step_all(steps, "f32", state)
    ro, rs = G.oracle_full(x)
    G.assert_rel(G.f64(o).swapaxes(0, 1), ro, G.TOL["f32"], "tiny stepped o")
    G.assert_rel(G.f64(state), rs, G.TOL["f32"], "tiny stepped state")


def test_decode_b256():
    """256 sequences x 16 heads, d=128, bf16, 64 consecutive in-place steps:
    all 4,096 chains, every step's output and the state after the last."""
    import torch

    x = W.make("decode_b256")
    state = torch.from_numpy(x["initial_state"]).cuda()
    o = G.f64(_step_all(x, "bf16", state)).swapaxes(0, 1)  # [N, steps, H, dv]
    sg = G.f64(state)
    assert np.isfinite(o).all() and np.isfinite(sg).all()
    seqs = _as_sequences(x)
    ro, rs = oracle.recurrent(seqs["q"], seqs["k"], seqs["v"], seqs["alpha"], seqs["b"], seqs["w"],
                              x["initial_state"])
    G.assert_chains(o, sg, ro, rs, G.TOL["bf16"], "decode_b256")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (128, 128), (32, 128), (128, 32), (64, 128)])
def test_decode_shapes(dtype, dk, dv):
    import torch

    x = W.make("decode_b256", seed=40, B=5, H=3, dk=dk, dv=dv, steps=10, dtype=dtype)
    state = torch.from_numpy(x["initial_state"]).cuda()
    o = G.f64(_step_all(x, dtype, state))
    seqs = _as_sequences(x)
    ro, rs = oracle.recurrent(seqs["q"], seqs["k"], seqs["v"], seqs["alpha"], seqs["b"], seqs["w"],
                              x["initial_state"])
    G.assert_rel(o.swapaxes(0, 1), ro, G.TOL[dtype], f"decode {dtype} {dk}x{dv} o")
    G.assert_rel(G.f64(state), rs, G.TOL[dtype], f"decode {dtype} {dk}x{dv} state")


def test_decode_bitwise_deterministic():
    import torch

    x = W.make("decode_b256", seed=41, B=7, H=4, steps=3)
    s1 = torch.from_numpy(x["initial_state"]).cuda()
    s2 = s1.clone()
    o1 = _step_all(x, "bf16", s1)
    o2 = _step_all(x, "bf16", s2)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_equals_stepped(dtype):
    """The two execution modes compute the same mathematics ("DeltaNet" entity
    trail, mindpattern.ai): the chunk kernel and T decode steps agree with
    each other and with the oracle."""
    import torch

    x = W.make("batched_bf16", seed=42, B=2, T=150, H=2, dtype=dtype)
    d = G.to_dev(x, dtype)
    oc, sc = G.gpu_chunk(d)
    steps = {n: np.ascontiguousarray(np.swapaxes(x[n], 0, 1)) for n in G.NAMES}
    state = torch.from_numpy(x["initial_state"]).cuda()
    os_ = _step_all(steps, dtype, state).transpose(0, 1)
    ro, rs = G.oracle_full(x)
    G.assert_rel(G.f64(os_), ro, G.TOL[dtype], f"stepped {dtype} o")
    G.assert_rel(G.f64(oc), G.f64(os_), G.TOL[dtype], f"chunk vs stepped {dtype} o")
    G.assert_rel(G.f64(sc), G.f64(state), G.TOL[dtype], f"chunk vs stepped {dtype} state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ["no_decay", "zero_alpha", "steep_3", "erase_0_2"])
def test_decode_gate_edges(dtype, d, case):
    """The decode step over 48 consecutive steps with the gate edge cases of
    the chunkwise tests: alpha = 1 (nothing decays, so the state keeps every
    write), alpha = 0 in some channels (acts as 2^-15), one channel decaying
    by 2^-3 per step, and the erase gate widened to [0, 2]; a random initial
    state.  Every step's output and the final state against the oracle."""
    import torch

    x = W.make("decode_b256", seed=50, B=6, H=3, dk=d, dv=d, steps=48, dtype=dtype)
    rng = np.random.default_rng(51)
    if case == "no_decay":
        x["alpha"][:] = 1.0
    elif case == "zero_alpha":
        x["alpha"][..., ::7] = 0.0
    elif case == "steep_3":
        x["alpha"][..., 5] = 2.0 ** -3
    else:
        b = 2.0 / (1.0 + np.exp(-rng.standard_normal(x["b"].shape)))
        x["b"] = W.round_bf16(b.astype(np.float32)) if dtype == "bf16" else b.astype(np.float32)
    state = torch.from_numpy(x["initial_state"]).cuda()
    o = G.f64(_step_all(x, dtype, state))
    seqs = _as_sequences(x)
    ro, rs = oracle.recurrent(seqs["q"], seqs["k"], seqs["v"], seqs["alpha"], seqs["b"], seqs["w"],
                              x["initial_state"])
    what = f"decode gate edge {case} {dtype} d={d}"
    G.assert_rel(o.swapaxes(0, 1), ro, G.TOL[dtype], f"{what} o")
    G.assert_rel(G.f64(state), rs, G.TOL[dtype], f"{what} state")
