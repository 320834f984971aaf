"""GPU parity of gdn2_chunk_fwd against the FP64 oracle (needs an MI355X).

Bar: relative L2 error, over the whole compared tensor, of at most 1e-4 for
FP32 inputs and 1e-2 for bf16 q/k/v/b/w with FP32 alpha and state; checked
separately for the outputs and for the final states.  Every workload is
compared over its whole tensors, every (sequence, head) chain included; the
worst chain is logged."""
import numpy as np
import pytest

import gpu_util as G
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    torch.cuda.init()
    yield


def _full_parity(x, dtype, what, tol=None):
    tol = tol or G.TOL[dtype]
    d = G.to_dev(x, dtype)
    o, sf = G.gpu_chunk(d)
    og, sg = G.f64(o), G.f64(sf)
    assert np.isfinite(og).all() and np.isfinite(sg).all(), f"{what}: non-finite output"
    ro, rs = G.oracle_full(x)
    G.assert_chains(og, sg, ro, rs, tol, what, x.get("cu_seqlens"))
    return o, sf


def test_tiny_f32():
    """B=1, H=2, T=256, dk=dv=32, FP32, zero initial state."""
    _full_parity(W.make("tiny_f32"), "f32", "tiny_f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (128, 128), (32, 128), (128, 64), (64, 32)])
def test_reduced_shapes(dtype, dk, dv):
    """Several chunks, a ragged tail (300 = 4 x 64 + 44), random initial state."""
    x = W.make("batched_bf16", seed=77, B=2, T=300, H=3, dk=dk, dv=dv, dtype=dtype)
    _full_parity(x, dtype, f"reduced {dtype} dk={dk} dv={dv}")


def test_layer_bf16():
    """B=1, H=16, T=4096, d=128, bf16, zero initial state: every chain checked."""
    _full_parity(W.make("layer_bf16"), "bf16", "layer_bf16")


def test_batched_bf16():
    """B=8, H=16, T=4096, d=128, bf16, N(0, 0.1^2) initial state (headline
    shape): all 128 chains."""
    _full_parity(W.make("batched_bf16"), "bf16", "batched_bf16")


@pytest.mark.parametrize("mode", ["gdn2", "kda", "gdn"])
def test_varlen(mode):
    """32 packed sequences, lengths U{256..8192}, H=16, d=128, bf16, three gate
    modes: all 512 chains."""
    x = W.make("varlen32_bf16", gate_mode=mode)
    _full_parity(x, "bf16", f"varlen {mode}")


@pytest.mark.parametrize("case", ["no_decay", "slow_decay"])
def test_long_horizon(case):
    """The headline shape (B=8, H=16, T=4096, d=128, bf16) with the state kept
    across all 64 chunks: alpha = 1, or alpha = sigmoid(N(6, 0.5)) per key
    channel.  The carried FP32 state reaches the matrix-core products as a
    rounded operand in every chunk, so this is where a lossy carry would
    accumulate."""
    x = W.make("batched_bf16")
    rng = np.random.default_rng(13)
    if case == "no_decay":
        x["alpha"] = np.ones_like(x["alpha"])
    else:
        x["alpha"] = (1.0 / (1.0 + np.exp(-rng.normal(6.0, 0.5, x["alpha"].shape)))).astype(np.float32)
    _full_parity(x, "bf16", f"long horizon {case}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cut_to_32(dtype):
    """One key channel per head decaying by 2^-1.5 per token from token 700 on:
    a 64-token chunk there would span 2^-96, so the matrix-core kernel cuts
    its chunks to 32 tokens (2^-48), back to 64 where the channel recovers
    (from token 2500), across a ragged tail (T = 3001)."""
    x = W.make("batched_bf16", seed=14, B=2, T=3001, H=4, dtype=dtype)
    for h in range(4):
        x["alpha"][:, 700:2500, h, 3 + 17 * h] = np.float32(2.0 ** -1.5)
    _full_parity(x, "bf16" if dtype == "bf16" else "f32", f"cut to 32 {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_edges(dtype, d):
    """Zero-length, one-token, chunk-boundary and ragged sequences packed together."""
    lens = [0, 1, 63, 64, 65, 130, 0, 7, 200]
    cu = W.cu_from_lengths(lens)
    x = W.make("batched_bf16", seed=92, B=1, T=int(cu[-1]), H=2, dk=d, dv=d, dtype=dtype)
    x["cu_seqlens"] = cu
    x["initial_state"] = 0.1 * np.random.default_rng(93).standard_normal((len(lens), 2, d, d)).astype(np.float32)
    o, sf = _full_parity(x, dtype, f"varlen edges {dtype} d={d}")
    # zero-length sequences pass their state through unchanged
    np.testing.assert_array_equal(G.f64(sf)[0], x["initial_state"][0])
    np.testing.assert_array_equal(G.f64(sf)[6], x["initial_state"][6])


def test_empty_sequence_copies_state():
    import torch

    x = W.make("batched_bf16", seed=5, B=2, T=0, H=2, dk=32, dv=64)
    d = G.to_dev(x, "bf16")
    o, sf = G.gpu_chunk(d)
    assert o.numel() == 0
    assert torch.equal(sf, d["initial_state"])


def test_no_initial_state_and_no_final_state():
    x = W.make("tiny_f32", seed=8, T=130)
    d = G.to_dev(x, "f32")
    o, sf = G.gpu_chunk(d, output_final_state=False)
    assert sf is None
    ro, _ = G.oracle_full(x)
    G.assert_rel(G.f64(o), ro, G.TOL["f32"], "no-final-state o")


def test_in_place_state_update():
    import torch

    x = W.make("batched_bf16", seed=9, B=2, T=200, H=2)
    d = G.to_dev(x, "bf16")
    ref_o, ref_s = G.gpu_chunk(d)
    state = d["initial_state"].clone()
    o, sf = G.gpu_chunk(dict(d, initial_state=state), final_state=state)
    assert sf.data_ptr() == state.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(state, ref_s)


def test_bitwise_deterministic():
    import torch

    x = W.make("batched_bf16", seed=10, B=2, T=520, H=4)
    d = G.to_dev(x, "bf16")
    o1, s1 = G.gpu_chunk(d)
    o2, s2 = G.gpu_chunk(d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ["no_decay", "slow_decay", "zero_alpha", "steep_3", "steep_4", "erase_0_2"])
def test_gate_edges(dtype, d, case):
    """alpha = 1 (state carried across every chunk), slow decay sigmoid(N(6, 0.5)),
    alpha = 0 in some channels (acts as 2^-15), one channel decaying by 2^-3 or
    2^-4 per token (a 64-token chunk would span more than 2^-120 there), erase
    gate widened to [0, 2].  d = 128 with bf16 runs the matrix-core kernel, the
    rest the generic one."""
    x = W.make("batched_bf16", seed=11, B=1, T=257, H=2, dk=d, dv=d, dtype=dtype)
    rng = np.random.default_rng(12)
    if case == "no_decay":
        x["alpha"][:] = 1.0
    elif case == "slow_decay":
        x["alpha"][:] = (1.0 / (1.0 + np.exp(-rng.normal(6.0, 0.5, x["alpha"].shape)))).astype(np.float32)
    elif case == "zero_alpha":
        x["alpha"][..., ::7] = 0.0
    elif case in ("steep_3", "steep_4"):
        x["alpha"][..., 5] = 2.0 ** -int(case[-1])
    elif case == "erase_0_2":
        b = 2.0 / (1.0 + np.exp(-rng.standard_normal(x["b"].shape)))
        x["b"] = W.round_bf16(b.astype(np.float32)) if dtype == "bf16" else b.astype(np.float32)
    _full_parity(x, dtype, f"gate edge {case} {dtype} d={d}")
