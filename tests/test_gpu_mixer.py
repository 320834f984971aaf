"""GPU parity of the token mixer (gdn2_mixer_prologue, gdn2_mixer_epilogue)
against the FP64 oracle in oracle/mixer.py (needs an MI355X).

Bar: relative L2 error per output tensor, at most 1e-4 for FP32 and 1e-2 for
bf16 inputs; the oracle sees exactly the values the kernels see."""
import numpy as np
import pytest

import gpu_util as G
import oracle
from oracle import mixer
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def _rnd(rng, shape, dtype, scale=1.0):
    x = (scale * rng.standard_normal(shape)).astype(np.float32)
    return W.round_bf16(x) if dtype == "bf16" else x


def _inputs(seed, B, T, H, dk, dv, K, dtype, N=None):
    rng = np.random.default_rng(seed)
    N = B if N is None else N
    x = dict(xq=_rnd(rng, (B, T, H, dk), dtype), xk=_rnd(rng, (B, T, H, dk), dtype),
             xv=_rnd(rng, (B, T, H, dv), dtype), b_logit=_rnd(rng, (B, T, H, dk), dtype),
             w_logit=_rnd(rng, (B, T, H, dv), dtype),
             conv_q=(0.5 * rng.standard_normal((H * dk, K))).astype(np.float32),
             conv_k=(0.5 * rng.standard_normal((H * dk, K))).astype(np.float32),
             conv_v=(0.5 * rng.standard_normal((H * dv, K))).astype(np.float32),
             conv_state=rng.standard_normal((N, H * (2 * dk + dv), K - 1)).astype(np.float32))
    if dtype == "bf16":
        x["conv_state"] = W.round_bf16(x["conv_state"])  # a state carried from bf16 inputs holds bf16 values
    return x


def _dev(x, dtype):
    import torch

    d = {}
    for n in ("xq", "xk", "xv", "b_logit", "w_logit"):
        d[n] = W.to_torch(x[n], dtype, "cuda")
    for n in ("conv_q", "conv_k", "conv_v", "conv_state"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).cuda()
    return d


def _gpu_prologue(x, dtype, cu=None, q_scale=1.0):
    import torch

    d = _dev(x, dtype)
    cu_d = None if cu is None else torch.from_numpy(cu).cuda()
    out = binding.gdn2_mixer_prologue(d["xq"], d["xk"], d["xv"], d["conv_q"], d["conv_k"], d["conv_v"],
                                      d["b_logit"], d["w_logit"], conv_state=d["conv_state"], cu_seqlens=cu_d,
                                      q_scale=q_scale)
    torch.cuda.synchronize()
    return out


def _oracle_prologue(x, cu=None, q_scale=1.0):
    return mixer.prologue(x["xq"], x["xk"], x["xv"], x["conv_q"], x["conv_k"], x["conv_v"], x["b_logit"],
                          x["w_logit"], cu, x["conv_state"], q_scale=q_scale)


def _compare(out, ref, dtype, what):
    for name in ("q", "k", "v", "b", "w"):
        G.assert_rel(G.f64(out[name]), ref[name], G.TOL[dtype], f"{what} {name}")
    # the carried state is a copy of inputs: exact
    np.testing.assert_array_equal(G.f64(out["conv_state"]), ref["conv_state"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,K", [(32, 32, 4), (64, 128, 4), (128, 64, 2), (128, 128, 4), (64, 64, 1), (64, 32, 3),
                                     (32, 64, 7), (128, 32, 16)])
def test_prologue(dtype, dk, dv, K):
    x = _inputs(300 + dk + dv + K, B=2, T=37, H=3, dk=dk, dv=dv, K=K, dtype=dtype)
    _compare(_gpu_prologue(x, dtype, q_scale=0.125), _oracle_prologue(x, q_scale=0.125), dtype,
             f"prologue {dtype} dk={dk} dv={dv} K={K}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [2, 4, 8])
def test_prologue_packed(dtype, K):
    """Packed sequences: empty ones (state passed through), ones shorter than the
    filter, and longer ones, some crossing the token runs of a wavefront; the
    convolution restarts at each."""
    lens = [0, 1, 2, 9, 0, 40, 3, 33, 1, 70]
    cu = W.cu_from_lengths(lens)
    x = _inputs(320 + K, B=1, T=int(cu[-1]), H=2, dk=64, dv=64, K=K, dtype=dtype, N=len(lens))
    _compare(_gpu_prologue(x, dtype, cu=cu), _oracle_prologue(x, cu=cu), dtype, f"prologue packed {dtype}")


def test_prologue_decode_steps_in_place():
    """T = 1 calls with the state updated in place == one call over the tokens, bit for bit."""
    import torch

    x = _inputs(330, B=6, T=5, H=2, dk=128, dv=128, K=4, dtype="bf16")
    full = _gpu_prologue(x, "bf16")
    d = _dev(x, "bf16")
    state = d["conv_state"].clone()
    for t in range(5):
        sl = {n: d[n][:, t:t + 1].contiguous() for n in ("xq", "xk", "xv", "b_logit", "w_logit")}
        out = binding.gdn2_mixer_prologue(sl["xq"], sl["xk"], sl["xv"], d["conv_q"], d["conv_k"], d["conv_v"],
                                          sl["b_logit"], sl["w_logit"], conv_state=state, conv_state_out=state)
        torch.cuda.synchronize()
        for name in ("q", "k", "v", "b", "w"):
            assert torch.equal(out[name][:, 0], full[name][:, t]), f"step {t}: {name}"
    assert torch.equal(state, full["conv_state"])


def test_prologue_headline_shape_sampled():
    """B=8, T=4096, H=16, d=128, K=4, bf16: two (row, head) chains, first 384 tokens
    against the oracle (the convolution is causal)."""
    import torch

    x = _inputs(340, B=8, T=4096, H=16, dk=128, dv=128, K=4, dtype="bf16")
    out = _gpu_prologue(x, "bf16")
    for n, h in ((0, 0), (5, 11)):
        sub = {k: np.ascontiguousarray(x[k][n:n + 1, :384, h:h + 1]) for k in ("xq", "xk", "xv", "b_logit", "w_logit")}
        for k, d in (("conv_q", 128), ("conv_k", 128), ("conv_v", 128)):
            sub[k] = x[k][h * d:(h + 1) * d]
        H = 16
        cs = x["conv_state"][n:n + 1]
        sub["conv_state"] = np.concatenate([cs[:, h * 128:(h + 1) * 128], cs[:, H * 128 + h * 128:H * 128 + (h + 1) * 128],
                                            cs[:, 2 * H * 128 + h * 128:2 * H * 128 + (h + 1) * 128]], axis=1)
        ref = _oracle_prologue(sub)
        for name in ("q", "k", "v", "b", "w"):
            G.assert_rel(G.f64(out[name][n:n + 1, :384, h:h + 1]), ref[name], G.TOL["bf16"],
                         f"headline prologue ({n}, {h}) {name}")
    del out
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dv", [32, 64, 128])
@pytest.mark.parametrize("act", ["sigmoid", "silu"])
def test_epilogue(dtype, dv, act):
    import torch

    rng = np.random.default_rng(350 + dv)
    o, gate = _rnd(rng, (3, 41, 4, dv), dtype), _rnd(rng, (3, 41, 4, dv), dtype)
    wgt = rng.standard_normal(dv).astype(np.float32)
    y = binding.gdn2_mixer_epilogue(W.to_torch(o, dtype, "cuda"), W.to_torch(gate, dtype, "cuda"),
                                    torch.from_numpy(wgt).cuda(), eps=1e-5, act=act)
    torch.cuda.synchronize()
    G.assert_rel(G.f64(y), mixer.epilogue(o, gate, wgt, 1e-5, act), G.TOL[dtype], f"epilogue {dtype} dv={dv} {act}")


def test_layer_pipeline():
    """Prologue -> chunkwise recurrence -> epilogue on the GPU against the oracle's
    prologue -> recurrence -> epilogue (bf16, d=128, alpha from the workload recipe)."""
    import torch

    B, T, H, d, K = 2, 100, 2, 128, 4
    x = _inputs(360, B=B, T=T, H=H, dk=d, dv=d, K=K, dtype="bf16")
    rng = np.random.default_rng(361)
    alpha = (1.0 / (1.0 + np.exp(-rng.normal(3.0, 1.0, (B, T, H, d))))).astype(np.float32)
    gate = _rnd(rng, (B, T, H, d), "bf16")
    wgt = rng.standard_normal(d).astype(np.float32)
    pro = _gpu_prologue(x, "bf16", q_scale=d ** -0.5)
    o, _ = binding.gdn2_chunk_fwd(pro["q"], pro["k"], pro["v"], torch.from_numpy(alpha).cuda(), pro["b"], pro["w"])
    y = binding.gdn2_mixer_epilogue(o, W.to_torch(gate, "bf16", "cuda"), torch.from_numpy(wgt).cuda())
    torch.cuda.synchronize()
    rp = _oracle_prologue(x, q_scale=d ** -0.5)
    ro, _ = oracle.recurrent(rp["q"], rp["k"], rp["v"], alpha, rp["b"], rp["w"])
    G.assert_rel(G.f64(y), mixer.epilogue(ro, gate, wgt), G.TOL["bf16"], "layer pipeline output")
