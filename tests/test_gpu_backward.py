"""GPU parity of gdn2_chunk_bwd (the gate-aware backward pass) against the
FP64 oracle's reverse-mode gradients O5 (needs an MI355X).

Bar: relative L2 error of each gradient tensor (dq, dk, dv, dalpha, db, dw,
dS0), at most 1e-4 for FP32 inputs and 1e-2 for bf16 inputs, the same bar as
the forward pass.  bf16 inputs with dk = dv = 128 take the matrix-core path
(bf16 products); the tests read which path ran from the workspace's first
int32 (0: matrix-core path, 1: the FP32 path after the range check).  The seeds d_o and d_final_state are N(0, 1), rounded to the
input dtype, and the oracle sees exactly the values the kernels see."""
import numpy as np
import pytest

import gpu_util as G
import oracle
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "db", "dw")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def _seeds(x, dtype, seed, with_dsf=True):
    rng = np.random.default_rng(seed)
    B, T, H, _ = x["q"].shape
    dv = x["v"].shape[-1]
    dk = x["q"].shape[-1]
    N = B if x.get("cu_seqlens") is None else len(x["cu_seqlens"]) - 1
    g = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    if dtype == "bf16":
        g = W.round_bf16(g)
    gs = rng.standard_normal((N, H, dk, dv)).astype(np.float32) if with_dsf else None
    return g, gs


def gpu_bwd(x, dtype, g, gs, **kw):
    import torch

    d = G.to_dev(x, dtype)
    if kw.pop("want_path", False):
        B, T, H, dk = x["q"].shape
        N = 0 if x.get("cu_seqlens") is None else len(x["cu_seqlens"]) - 1
        n = binding.gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, x["v"].shape[-1], N, 1 if dtype == "bf16" else 0)
        kw["workspace"] = torch.empty(n, dtype=torch.uint8, device="cuda")
    dg = W.to_torch(g, dtype, "cuda")
    dgs = None if gs is None else torch.from_numpy(gs).cuda()
    out = binding.gdn2_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], dg, d["initial_state"], dgs,
                                 cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    if "workspace" in kw:
        out["path_flag"] = int(kw["workspace"][:4].view(torch.int32).item())
    return out


def oracle_bwd(x, g, gs, chains=None, threads=0):
    return oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g, x.get("initial_state"), gs,
                           x.get("cu_seqlens"), chains=chains, threads=threads)


def _compare(out, ref, dtype, what, d_init=True):
    for name in GRADS:
        G.assert_rel(G.f64(out[name]), ref[name], G.TOL[dtype], f"{what} {name}")
    if d_init:
        G.assert_rel(G.f64(out["d_initial_state"]), ref["d_initial_state"], G.TOL[dtype], f"{what} dS0")


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 32, 32), ("f32", 64, 128), ("f32", 128, 64), ("f32", 128, 128),
                                         ("bf16", 128, 128), ("bf16", 64, 32)])
def test_backward_shapes(dtype, dk, dv):
    """B=2, T=100 (three 32-token chunks and a ragged 4), H=3, random initial state and seeds."""
    x = W.make("batched_bf16", seed=201, B=2, T=100, H=3, dk=dk, dv=dv, dtype=dtype)
    g, gs = _seeds(x, dtype, 202)
    out = gpu_bwd(x, dtype, g, gs, want_path=True)
    _compare(out, oracle_bwd(x, g, gs), dtype, f"bwd {dtype} dk={dk} dv={dv}")
    if dtype == "bf16" and dk == dv == 128:
        assert out["path_flag"] == 0, "the matrix-core path must produce these results"


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 128)])
def test_backward_strong_decay(dtype, d):
    """Half of the key channels decay strongly (alpha in [0.05, 0.2]: over a
    32-token chunk far below 2^-64), half as in the workload recipe; both
    ways of forming the pairwise sums run in one call (the split products for
    mild channels, the pairwise loops for strong ones).  alpha stays above the
    clamp so that the oracle, which uses alpha as given, sees the same values."""
    x = W.make("batched_bf16", seed=206, B=2, T=100, H=2, dk=d, dv=d, dtype=dtype)
    rng = np.random.default_rng(207)
    strong = rng.uniform(0.05, 0.2, x["alpha"][..., : d // 2].shape).astype(np.float32)
    x["alpha"] = np.ascontiguousarray(np.concatenate([strong, x["alpha"][..., d // 2:]], axis=-1))
    g, gs = _seeds(x, dtype, 208)
    out = gpu_bwd(x, dtype, g, gs, want_path=True)
    _compare(out, oracle_bwd(x, g, gs), dtype, f"bwd strong decay {dtype} d={d}")
    if dtype == "bf16" and d == 128:
        assert out["path_flag"] == 1, "strong decay must fall back to the FP32 path"


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_backward_varlen_edges(dtype, d):
    """Zero-length, one-token, chunk-boundary and ragged sequences packed together."""
    lens = [0, 1, 31, 32, 33, 70, 0, 7, 100]
    cu = W.cu_from_lengths(lens)
    x = W.make("batched_bf16", seed=203, B=1, T=int(cu[-1]), H=2, dk=d, dv=d, dtype=dtype)
    x["cu_seqlens"] = cu
    x["initial_state"] = 0.1 * np.random.default_rng(204).standard_normal((len(lens), 2, d, d)).astype(np.float32)
    g, gs = _seeds(x, dtype, 205)
    out = gpu_bwd(x, dtype, g, gs)
    ref = oracle_bwd(x, g, gs)
    _compare(out, ref, dtype, f"bwd varlen {dtype} d={d}")
    # zero-length sequences pass the final-state seed through unchanged
    np.testing.assert_array_equal(G.f64(out["d_initial_state"])[0], gs[0])
    np.testing.assert_array_equal(G.f64(out["d_initial_state"])[6], gs[6])


def test_backward_without_state_seed_or_initial_state():
    """No initial state, no final-state seed, no initial-state gradient wanted."""
    x = W.make("tiny_f32", seed=206, T=90)
    g, _ = _seeds(x, "f32", 207, with_dsf=False)
    out = gpu_bwd(x, "f32", g, None, output_d_initial_state=False)
    assert out["d_initial_state"] is None
    _compare(out, oracle_bwd(x, g, None), "f32", "bwd no state", d_init=False)


def test_backward_in_place_state_gradient():
    """d_initial_state may replace d_final_state in place."""
    import torch

    x = W.make("batched_bf16", seed=208, B=2, T=70, H=2, dk=64, dv=64, dtype="f32")
    g, gs = _seeds(x, "f32", 209)
    ref = gpu_bwd(x, "f32", g, gs)
    d = G.to_dev(x, "f32")
    buf = torch.from_numpy(gs).cuda()
    out = binding.gdn2_chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"], W.to_torch(g, "f32", "cuda"),
                                 d["initial_state"], buf, d_initial_state=buf)
    torch.cuda.synchronize()
    assert out["d_initial_state"].data_ptr() == buf.data_ptr()
    assert torch.equal(buf, ref["d_initial_state"])
    for name in GRADS:
        assert torch.equal(out[name], ref[name]), name


def test_backward_bitwise_deterministic():
    import torch

    x = W.make("batched_bf16", seed=210, B=2, T=150, H=4)
    g, gs = _seeds(x, "bf16", 211)
    o1 = gpu_bwd(x, "bf16", g, gs)
    o2 = gpu_bwd(x, "bf16", g, gs)
    for name in GRADS + ("d_initial_state",):
        assert torch.equal(o1[name], o2[name]), name


@pytest.mark.parametrize("mode", ["kda", "gdn"])
def test_backward_reduced_gate_inputs(mode):
    """Inputs with tied scalar gates (broadcast): the same bar."""
    x = W.make("batched_bf16", gate_mode=mode, seed=212, B=2, T=96, H=2, dk=128, dv=128)
    g, gs = _seeds(x, "bf16", 213)
    _compare(gpu_bwd(x, "bf16", g, gs), oracle_bwd(x, g, gs), "bf16", f"bwd {mode} inputs")


def test_backward_batched_bf16():
    """B=8, H=16, T=4096, d=128, bf16 (the headline forward shape): every
    gradient over all 128 chains."""
    x = W.make("batched_bf16")
    g, gs = _seeds(x, "bf16", 214)
    out = gpu_bwd(x, "bf16", g, gs, want_path=True)
    assert out["path_flag"] == 0, "the matrix-core path must produce these results"
    ref = oracle_bwd(x, g, gs)
    _compare(out, ref, "bf16", "batched bwd")


@pytest.mark.parametrize("case", ["ragged", "no_decay", "slow_decay", "erase_0_2", "one_steep_chunk"])
def test_backward_matrix_core_cases(case):
    """The matrix-core path (bf16, d = 128) over several 64-token chunks and a
    ragged tail (B=2, T=300, H=2): the workload's gates; alpha = 1 (state
    carried unchanged); slow decay sigmoid(N(6, 0.5)); erase gate widened to
    [0, 2]; and one channel of one head decaying by 2^-2 per token over tokens
    130..200 only: that chunk spans 2^-128, so the whole call falls back to the
    FP32 path, which must give the same bar."""
    x = W.make("batched_bf16", seed=215, B=2, T=300, H=2)
    rng = np.random.default_rng(216)
    if case == "no_decay":
        x["alpha"][:] = 1.0
    elif case == "slow_decay":
        x["alpha"][:] = (1.0 / (1.0 + np.exp(-rng.normal(6.0, 0.5, x["alpha"].shape)))).astype(np.float32)
    elif case == "erase_0_2":
        x["b"] = W.round_bf16(2.0 * x["b"])
    elif case == "one_steep_chunk":
        x["alpha"][1, 130:200, 1, 17] = 0.25
    g, gs = _seeds(x, "bf16", 217)
    out = gpu_bwd(x, "bf16", g, gs, want_path=True)
    assert out["path_flag"] == (1 if case == "one_steep_chunk" else 0), out["path_flag"]
    _compare(out, oracle_bwd(x, g, gs), "bf16", f"bwd matrix-core {case}")


def test_backward_matrix_core_long_horizon():
    """B=1, H=4, T=4096 with alpha = 1: the state gradient carried over 64
    chunks, every chain compared whole."""
    x = W.make("batched_bf16", seed=218, B=1, T=4096, H=4)
    x["alpha"][:] = 1.0
    g, gs = _seeds(x, "bf16", 219)
    out = gpu_bwd(x, "bf16", g, gs, want_path=True)
    assert out["path_flag"] == 0
    _compare(out, oracle_bwd(x, g, gs), "bf16", "bwd matrix-core long horizon")
