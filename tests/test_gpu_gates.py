"""GPU parity of the compact gate layouts (gdn2_chunk_fwd_gates and
gdn2_recurrent_step_gates, needs an MI355X).

Two checks per case:
  * against the FP64 oracle: its own reduced-gate forms for the two
    reductions (Kimi Delta Attention: tied erase/write scalar beta per token
    and head; Gated DeltaNet: beta and one decay per token and head), and its
    recurrence on the broadcast gates for every other layout (the ablations'
    channel-averaged gates), at the same rel-L2 bar as the full layout;
  * bitwise equality with the full layout called on the same gates broadcast
    to [.., dk] / [.., dv]: the compact layout changes what is read, not the
    arithmetic.
"""
import numpy as np
import pytest

import gpu_util as G
import oracle
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu

MODES = {"kda": binding.GATES_KDA, "gdn": binding.GATES_GDN}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def compact(x: dict, mode: str):
    """beta [..] and alpha ([.., dk] or [..]) of broadcast reduced-gate inputs."""
    beta = np.ascontiguousarray(x["b"][..., 0])
    assert np.array_equal(np.broadcast_to(beta[..., None], x["b"].shape), x["b"])
    assert np.array_equal(np.broadcast_to(beta[..., None], x["w"].shape), x["w"])
    alpha = x["alpha"]
    if mode == "gdn":
        alpha = np.ascontiguousarray(alpha[..., 0])
        assert np.array_equal(np.broadcast_to(alpha[..., None], x["alpha"].shape), x["alpha"])
    return beta, np.ascontiguousarray(alpha)


def oracle_compact(mode, q, k, v, alpha, beta, s0, cu):
    fn = oracle.kda if mode == "kda" else oracle.gdn
    return fn(q, k, v, alpha, beta, s0, cu)


def gpu_gates(x, mode, dtype, final_state=True):
    import torch

    d = G.to_dev(x, dtype)
    beta, alpha = compact(x, mode)
    db = W.to_torch(beta, dtype, "cuda")
    da = W.to_torch(alpha, "f32", "cuda")
    o, sf = binding.gdn2_chunk_fwd_gates(d["q"], d["k"], d["v"], da, db, None, MODES[mode], d["initial_state"],
                                         cu_seqlens=d["cu_seqlens"], output_final_state=final_state)
    torch.cuda.synchronize()
    return d, o, sf


def _check(x, mode, dtype, what):
    import torch

    d, o, sf = gpu_gates(x, mode, dtype)
    fo, fs = G.gpu_chunk(d)  # full layout, broadcast gates
    assert torch.equal(o, fo), f"{what}: compact and full layouts differ in o"
    assert torch.equal(sf, fs), f"{what}: compact and full layouts differ in the final state"
    beta, alpha = compact(x, mode)
    ro, rs = oracle_compact(mode, x["q"], x["k"], x["v"], alpha, beta, x.get("initial_state"), x.get("cu_seqlens"))
    G.assert_rel(G.f64(o), ro, G.TOL[dtype], f"{what} o")
    G.assert_rel(G.f64(sf), rs, G.TOL[dtype], f"{what} final state")


@pytest.mark.parametrize("mode", ["kda", "gdn"])
@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("f32", 32, 128), ("bf16", 128, 128),
                                         ("bf16", 128, 64), ("bf16", 64, 32)])
def test_chunk_gates(mode, dtype, dk, dv):
    """Several chunks, a ragged tail (300 = 4 x 64 + 44), random initial state."""
    x = W.make("batched_bf16", gate_mode=mode, seed=71, B=2, T=300, H=3, dk=dk, dv=dv, dtype=dtype)
    _check(x, mode, dtype, f"{mode} {dtype} dk={dk} dv={dv}")


@pytest.mark.parametrize("mode", ["kda", "gdn"])
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_chunk_gates_varlen_edges(mode, dtype, d):
    """Zero-length, one-token, chunk-boundary and ragged sequences packed together."""
    lens = [0, 1, 63, 64, 65, 130, 0, 7, 200]
    cu = W.cu_from_lengths(lens)
    x = W.make("batched_bf16", gate_mode=mode, seed=94, B=1, T=int(cu[-1]), H=2, dk=d, dv=d, dtype=dtype)
    x["cu_seqlens"] = cu
    x["initial_state"] = 0.1 * np.random.default_rng(95).standard_normal((len(lens), 2, d, d)).astype(np.float32)
    _check(x, mode, dtype, f"{mode} varlen edges {dtype} d={d}")


@pytest.mark.parametrize("mode", ["kda", "gdn"])
def test_chunk_gates_varlen32(mode):
    """32 packed sequences, lengths U{256..8192}, H=16, d=128, bf16, compact
    layout: bitwise equal to the full layout everywhere; the oracle's
    recurrence on the broadcast gates over all 512 chains; and its separately
    written reduced form (a dk x dk matrix per token, too slow for every
    chain) on one head of every fourth sequence and of the longest."""
    import torch

    x = W.make("varlen32_bf16", gate_mode=mode)
    d, o, sf = gpu_gates(x, mode, "bf16")
    fo, fs = G.gpu_chunk(d)
    assert torch.equal(o, fo) and torch.equal(sf, fs), f"varlen32 {mode}: compact and full layouts differ"
    og, sg = G.f64(o), G.f64(sf)
    G.log(f"varlen32 {mode}: oracle recurrence on all chains")
    ro, rs = G.oracle_full(x)
    G.assert_chains(og, sg, ro, rs, G.TOL["bf16"], f"varlen32 {mode} compact", x["cu_seqlens"])
    beta, alpha = compact(x, mode)
    H = x["q"].shape[2]
    N = len(x["cu_seqlens"]) - 1
    lens = np.diff(x["cu_seqlens"])
    seqs = sorted(set(range(0, N, 4)) | {int(np.argmax(lens))})
    chains = [n * H + (n % H) for n in seqs]
    G.log(f"varlen32 {mode}: oracle {mode} form on {len(chains)} chains")
    fn = oracle.kda if mode == "kda" else oracle.gdn
    ro, rs = fn(x["q"], x["k"], x["v"], alpha, beta, x["initial_state"], x["cu_seqlens"], chains=chains)
    cu = x["cu_seqlens"]
    go = np.concatenate([og[0, cu[n]:cu[n + 1], n % H].ravel() for n in seqs])
    eo = np.concatenate([ro[0, cu[n]:cu[n + 1], n % H].ravel() for n in seqs])
    G.assert_rel(go, eo, G.TOL["bf16"], f"varlen32 {mode} o vs the {mode} form ({len(seqs)} chains)")
    G.assert_rel(np.stack([sg[n, n % H] for n in seqs]), np.stack([rs[n, n % H] for n in seqs]),
                 G.TOL["bf16"], f"varlen32 {mode} state vs the {mode} form ({len(seqs)} chains)")


@pytest.mark.parametrize("mode", ["kda", "gdn"])
@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 128)])
def test_recurrent_step_gates(mode, dtype, d):
    """Eight in-place decode steps of 24 sequences x 4 heads."""
    import torch

    steps, N, H = 8, 24, 4
    x = W.make("batched_bf16", gate_mode=mode, seed=96, B=steps, T=N, H=H, dk=d, dv=d, dtype=dtype)
    # rows of x are steps, columns sequences: [steps, N, H, d]
    s0 = 0.1 * np.random.default_rng(97).standard_normal((N, H, d, d)).astype(np.float32)
    beta, alpha = compact(x, mode)
    state_c = torch.from_numpy(s0).cuda()
    state_f = state_c.clone()
    outs = []
    for t in range(steps):
        dt = G.to_dev({n: x[n][t] for n in G.NAMES}, dtype)
        oc = binding.gdn2_recurrent_step_gates(dt["q"], dt["k"], dt["v"], W.to_torch(alpha[t], "f32", "cuda"),
                                               W.to_torch(beta[t], dtype, "cuda"), None, MODES[mode], state_c)
        of = binding.gdn2_recurrent_step(dt["q"], dt["k"], dt["v"], dt["alpha"], dt["b"], dt["w"], state_f)
        torch.cuda.synchronize()
        assert torch.equal(oc, of), f"decode {mode} step {t}: compact and full layouts differ"
        outs.append(oc)
    assert torch.equal(state_c, state_f), f"decode {mode}: states differ"
    seq = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))  # noqa: E731  [N, steps, H, ..]
    ro, rs = oracle_compact(mode, seq(x["q"]), seq(x["k"]), seq(x["v"]), seq(alpha), seq(beta), s0, None)
    G.assert_rel(G.f64(torch.stack(outs)).swapaxes(0, 1), ro, G.TOL[dtype], f"decode {mode} {dtype} o")
    G.assert_rel(G.f64(state_c), rs, G.TOL[dtype], f"decode {mode} {dtype} state")


ABLATION_LAYOUTS = [g for g in binding.VALID_GATES if g != binding.GATES_FULL]


def averaged(x: dict, gates: int, dtype: str):
    """Gated DeltaNet-2 inputs with the gates that `gates` makes scalar
    replaced by their channel mean (rounded to the input dtype): returns the
    compact (b, w, alpha) for the layout and x with those gates broadcast."""
    lead = x["b"].shape[:-1]
    rnd = W.round_bf16 if dtype == "bf16" else (lambda a: a)
    mean = lambda a: rnd(a.mean(axis=-1, dtype=np.float64).astype(np.float32))  # noqa: E731
    xb = dict(x)
    b, w, alpha = x["b"], x["w"], x["alpha"]
    if gates & binding.GATES_SCALAR_ERASE:
        b = np.ascontiguousarray(mean(x["b"]))
        xb["b"] = np.ascontiguousarray(np.broadcast_to(b[..., None], x["b"].shape))
    if gates & binding.GATES_TIED:
        xb["w"] = np.ascontiguousarray(np.broadcast_to(b[..., None], lead + x["w"].shape[-1:]))
        w = None
    elif gates & binding.GATES_SCALAR_WRITE:
        w = np.ascontiguousarray(mean(x["w"]))
        xb["w"] = np.ascontiguousarray(np.broadcast_to(w[..., None], x["w"].shape))
    if gates & binding.GATES_SCALAR_DECAY:
        alpha = np.ascontiguousarray(x["alpha"].mean(axis=-1, dtype=np.float64).astype(np.float32))
        xb["alpha"] = np.ascontiguousarray(np.broadcast_to(alpha[..., None], x["alpha"].shape))
    return (b, w, alpha), xb


def _dev_compact(arrs, dtype):
    b, w, alpha = arrs
    return (W.to_torch(b, dtype, "cuda"), None if w is None else W.to_torch(w, dtype, "cuda"),
            W.to_torch(alpha, "f32", "cuda"))


@pytest.mark.parametrize("gates", ABLATION_LAYOUTS)
@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("bf16", 128, 128), ("bf16", 128, 64)])
def test_chunk_layouts(gates, dtype, dk, dv):
    """Every layout on channel-averaged Gated DeltaNet-2 gates: several chunks,
    a ragged tail, random initial state."""
    import torch

    x = W.make("batched_bf16", seed=72, B=2, T=300, H=3, dk=dk, dv=dv, dtype=dtype)
    arrs, xb = averaged(x, gates, dtype)
    d = G.to_dev(xb, dtype)
    cb, cw, ca = _dev_compact(arrs, dtype)
    o, sf = binding.gdn2_chunk_fwd_gates(d["q"], d["k"], d["v"], ca, cb, cw, gates, d["initial_state"])
    torch.cuda.synchronize()
    fo, fs = G.gpu_chunk(d)
    what = f"layout {gates} {dtype} dk={dk} dv={dv}"
    assert torch.equal(o, fo) and torch.equal(sf, fs), f"{what}: compact and full layouts differ"
    ro, rs = G.oracle_full(xb)
    G.assert_rel(G.f64(o), ro, G.TOL[dtype], f"{what} o")
    G.assert_rel(G.f64(sf), rs, G.TOL[dtype], f"{what} final state")


@pytest.mark.parametrize("gates", ABLATION_LAYOUTS)
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_recurrent_step_layouts(gates, dtype, d):
    """Every layout, four in-place decode steps of 16 sequences x 4 heads."""
    import torch

    steps, N, H = 4, 16, 4
    x = W.make("batched_bf16", seed=98, B=steps, T=N, H=H, dk=d, dv=d, dtype=dtype)
    arrs, xb = averaged(x, gates, dtype)
    s0 = 0.1 * np.random.default_rng(99).standard_normal((N, H, d, d)).astype(np.float32)
    state_c = torch.from_numpy(s0).cuda()
    state_f = state_c.clone()
    outs = []
    for t in range(steps):
        dt = G.to_dev({n: xb[n][t] for n in G.NAMES}, dtype)
        cb, cw, ca = _dev_compact(tuple(None if a is None else np.ascontiguousarray(a[t]) for a in arrs), dtype)
        oc = binding.gdn2_recurrent_step_gates(dt["q"], dt["k"], dt["v"], ca, cb, cw, gates, state_c)
        of = binding.gdn2_recurrent_step(dt["q"], dt["k"], dt["v"], dt["alpha"], dt["b"], dt["w"], state_f)
        torch.cuda.synchronize()
        assert torch.equal(oc, of), f"decode layout {gates} step {t}: compact and full layouts differ"
        outs.append(oc)
    assert torch.equal(state_c, state_f), f"decode layout {gates}: states differ"
    seq = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1))  # noqa: E731
    ro, rs = oracle.recurrent(*(seq(xb[n]) for n in G.NAMES), s0)
    G.assert_rel(G.f64(torch.stack(outs)).swapaxes(0, 1), ro, G.TOL[dtype], f"decode layout {gates} {dtype} o")
    G.assert_rel(G.f64(state_c), rs, G.TOL[dtype], f"decode layout {gates} {dtype} state")
