"""GPU parity of the segmented path of gdn2_chunk_fwd (few (sequence, head)
chains, each batch row cut into segments whose affine state maps are
combined) against the FP64 oracle, over whole tensors (needs an MI355X).

The path runs when the caller passes the workspace gdn2_chunk_fwd_workspace_bytes
asks for; the binding does so by default and ``segmented=False`` forces the
single pass.  Bar: as for the single pass, relative L2 <= 1e-2 (bf16)."""
import numpy as np
import pytest

import gpu_util as G
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def _ws(x):
    B, T, H, dk = x["q"].shape
    return binding.gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, x["v"].shape[-1], 0, binding.DTYPE_BF16)


def _both(x, what, tol=1e-2):
    """Segmented and single-pass results, each against the oracle."""
    assert _ws(x) > 0, f"{what}: the segmented path does not apply to this shape"
    d = G.to_dev(x, "bf16")
    o1, s1 = G.gpu_chunk(d)
    o0, s0 = G.gpu_chunk(d, segmented=False)
    ro, rs = G.oracle_full(x)
    G.assert_chains(G.f64(o1), G.f64(s1), ro, rs, tol, f"{what} segmented")
    G.assert_chains(G.f64(o0), G.f64(s0), ro, rs, tol, f"{what} single pass")
    return o1, s1


def test_layer_bf16_segmented():
    """B=1, H=16, T=4096, d=128 (the single-layer training shape): five segments."""
    _both(W.make("layer_bf16"), "layer_bf16")


def test_16k_by_1():
    """B=1, H=16, T=16384, d=128: the 16K x 1 setting of the pages' training sweep."""
    x = W.make("layer_bf16", seed=1301, T=16384)
    x["initial_state"] = 0.1 * np.random.default_rng(1302).standard_normal((1, 16, 128, 128)).astype(np.float32)
    _both(x, "B=1 T=16384")


@pytest.mark.parametrize("case", ["no_decay", "slow_decay"])
def test_segmented_long_horizon(case):
    """alpha = 1 or sigmoid(N(6, 0.5)): the state maps M_p are then far from
    zero, so errors in them reach the later segments."""
    x = W.make("layer_bf16", seed=1303)
    rng = np.random.default_rng(1304)
    if case == "no_decay":
        x["alpha"] = np.ones_like(x["alpha"])
    else:
        x["alpha"] = (1.0 / (1.0 + np.exp(-rng.normal(6.0, 0.5, x["alpha"].shape)))).astype(np.float32)
    x["initial_state"] = 0.1 * rng.standard_normal((1, 16, 128, 128)).astype(np.float32)
    _both(x, f"segmented {case}")


def test_segmented_in_place_ragged():
    """B=2, H=4, T=3001 (the last segment ragged), random initial state
    updated in place; one key channel decays by 2^-1.5 per token over part of
    the sequence, so chunks are cut to 32 tokens inside segments."""
    import torch

    x = W.make("batched_bf16", seed=1305, B=2, T=3001, H=4)
    for h in range(4):
        x["alpha"][:, 900:2100, h, 5 + 11 * h] = np.float32(2.0 ** -1.5)
    assert _ws(x) > 0
    d = G.to_dev(x, "bf16")
    state = d["initial_state"].clone()
    o, sf = G.gpu_chunk(dict(d, initial_state=state), final_state=state)
    assert sf.data_ptr() == state.data_ptr()
    ro, rs = G.oracle_full(x)
    G.assert_chains(G.f64(o), G.f64(state), ro, rs, 1e-2, "segmented in place, ragged")


@pytest.mark.parametrize("dv", [64])
def test_segmented_value_widths(dv):
    """dv = 64 with dk = 128: the map columns take tiles 1 and 2 of pass 1."""
    x = W.make("batched_bf16", seed=1306 + dv, B=1, T=2048, H=8, dk=128, dv=dv)
    _both(x, f"segmented dv={dv}")


@pytest.mark.parametrize("mode", ["kda", "gdn"])
def test_segmented_gate_layouts(mode):
    """The compact KDA and GDN layouts through the segmented path: bitwise
    equal to the full layout on the broadcast gates, and the oracle's bar."""
    import torch

    flags = {"kda": binding.GATES_KDA, "gdn": binding.GATES_GDN}[mode]
    x = W.make("batched_bf16", gate_mode=mode, seed=1310, B=1, T=2048, H=8)
    assert _ws(x) > 0
    d = G.to_dev(x, "bf16")
    beta = d["b"][..., 0].contiguous()
    alpha = d["alpha"][..., 0].contiguous() if mode == "gdn" else d["alpha"]
    o, sf = binding.gdn2_chunk_fwd_gates(d["q"], d["k"], d["v"], alpha, beta, None, flags, d["initial_state"])
    torch.cuda.synchronize()
    fo, fs = G.gpu_chunk(d)
    assert torch.equal(o, fo) and torch.equal(sf, fs), f"{mode}: compact and full layouts differ"
    ro, rs = G.oracle_full(x)
    G.assert_chains(G.f64(o), G.f64(sf), ro, rs, 1e-2, f"segmented {mode} layout")


def test_segmented_deterministic():
    import torch

    x = W.make("layer_bf16", seed=1320, T=2048)
    d = G.to_dev(x, "bf16")
    o1, s1 = G.gpu_chunk(d)
    o2, s2 = G.gpu_chunk(d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("T", [1024, 1025, 1089])
def test_segmented_threshold(T):
    """B=1, H=16 at the shortest rows the segmented path takes: T = 1024 gives
    four segments of 256 tokens, T = 1025 five (the last a single token),
    T = 1089 five (the last one chunk and one token); random initial state."""
    x = W.make("layer_bf16", seed=1330 + T, T=T)
    x["initial_state"] = 0.1 * np.random.default_rng(1331 + T).standard_normal((1, 16, 128, 128)).astype(np.float32)
    _both(x, f"segmented T={T}")
