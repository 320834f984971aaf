"""GPU parity at the largest sizes: tensors whose element offsets pass 2^31
and 2^32 (needs an MI355X with about 90 GB of free HBM).

Every kernel forms its offsets in 64-bit arithmetic; these tests check that
on the GPU.  The tensors are filled on the device with torch's seeded
generator (workloads.device_token_tensors).  The sampled chains, placed on
both sides of each power-of-two boundary and at the very end, are then
overwritten with host inputs from the numpy recipe, so they differ from every
other row: a wrapped offset would read other data and fail the comparison.
The oracle sees exactly the sampled chains' values.  Bar: as everywhere,
relative L2 at most 1e-2 for bf16 inputs."""
import numpy as np
import pytest

import gpu_util as G
import oracle
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W
from oracle import mixer

pytestmark = pytest.mark.gpu

D = 128
H = 16


@pytest.fixture(autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _host_chain(seed, T, with_state=True):
    """Inputs of one (sequence, head) chain from the host recipe: [1, T, 1, d] tensors."""
    ss_tok, ss_state = np.random.SeedSequence(seed).spawn(2)
    x = W.token_tensors(ss_tok, (1, T), 1, D, D, "bf16")
    x["initial_state"] = W.initial_state(np.random.default_rng(ss_state), 1, 1, D, D) if with_state else None
    return x


def _put(dev, name, index, arr):
    """Host values (exact in bf16; alpha FP32) into dev[name][index]."""
    dev[name][index] = W.to_torch(np.ascontiguousarray(arr), "f32" if name == "alpha" else "bf16", "cuda")


def _oracle(x):
    o, s = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], x["initial_state"])
    return o[0, :, 0], s[0, 0]


def test_chunk_fwd_batched_past_4g_elements():
    """B=520, T=4096, H=16, d=128, bf16: 4.4e9 elements per bf16 input (8.7 GB),
    byte offsets past 2^34 for alpha.  Chains beside the 2^30, 2^31 and 2^32
    element boundaries (rows 128, 256, 512) and the last."""
    import torch

    B, T = 520, 4096
    dev = W.device_token_tensors((B, T), H, D, D, "bf16", seed=901)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(902)
    s0 = 0.1 * torch.randn((B, H, D, D), generator=gen, device="cuda")
    chains = [(127, 3), (128, 0), (255, 15), (256, 0), (511, 15), (512, 0), (519, 15)]
    host = {}
    for i, (n, h) in enumerate(chains):
        x = _host_chain(910 + i, T)
        for name in G.NAMES:
            _put(dev, name, (n, slice(None), h), x[name][0, :, 0])
        s0[n, h] = torch.from_numpy(x["initial_state"][0, 0]).cuda()
        host[(n, h)] = x
    G.log(f"batched B={B}: inputs on the device, {len(chains)} host chains placed")
    o, sf = binding.gdn2_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["b"], dev["w"], s0)
    torch.cuda.synchronize()
    for (n, h), x in host.items():
        ro, rs = _oracle(x)
        G.assert_rel(G.f64(o[n, :, h]), ro, G.TOL["bf16"], f"large batched o ({n}, {h})")
        G.assert_rel(G.f64(sf[n, h]), rs, G.TOL["bf16"], f"large batched state ({n}, {h})")


def test_chunk_fwd_packed_past_4g_elements():
    """One packed row of 2.2M tokens (600-odd sequences of 1..8192 tokens), H=16,
    d=128, bf16: the sequences that hold packed tokens 2^20 and 2^21 (element
    offsets 2^31 and 2^32) and the last one."""
    import torch

    rng = np.random.default_rng(920)
    lengths = []
    while sum(lengths) < 2_150_000:
        lengths.append(int(rng.integers(1, 8193)))
    lengths.append(3000)
    cu = W.cu_from_lengths(lengths)
    total, N = int(cu[-1]), len(lengths)
    dev = W.device_token_tensors((1, total), H, D, D, "bf16", seed=921)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(922)
    s0 = 0.1 * torch.randn((N, H, D, D), generator=gen, device="cuda")
    seqs = sorted({int(np.searchsorted(cu, 1 << 20, side="right")) - 1,
                   int(np.searchsorted(cu, 1 << 21, side="right")) - 1, N - 1})
    host = {}
    for i, n in enumerate(seqs):
        h = 15 if i % 2 == 0 else 0
        lo, hi = int(cu[n]), int(cu[n + 1])
        x = _host_chain(930 + i, hi - lo)
        for name in G.NAMES:
            _put(dev, name, (0, slice(lo, hi), h), x[name][0, :, 0])
        s0[n, h] = torch.from_numpy(x["initial_state"][0, 0]).cuda()
        host[(n, h)] = x
    G.log(f"packed: {total} tokens in {N} sequences; checking sequences {seqs}")
    o, sf = binding.gdn2_chunk_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["b"], dev["w"], s0,
                                   cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    for (n, h), x in host.items():
        lo, hi = int(cu[n]), int(cu[n + 1])
        ro, rs = _oracle(x)
        G.assert_rel(G.f64(o[0, lo:hi, h]), ro, G.TOL["bf16"], f"large packed o (sequence {n}, head {h})")
        G.assert_rel(G.f64(sf[n, h]), rs, G.TOL["bf16"], f"large packed state (sequence {n}, head {h})")


@pytest.mark.parametrize("T", [1, 16, 32])
def test_recurrent_past_4g_state_elements(T):
    """N=16640 sequences x 16 heads of 128 x 128 FP32 state (4.4e9 elements, 17 GB),
    updated in place: T = 1 (gdn2_recurrent_step), 16 (the recurrent kernel) and
    32 (dispatched to the chunkwise kernel).  Chains beside the 2^31 and 2^32
    element boundaries of the state (sequences 8192, 16384) and the last."""
    import torch

    N = 16640
    dev = W.device_token_tensors((N, T), H, D, D, "bf16", seed=940 + T)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(941)
    state = 0.1 * torch.randn((N, H, D, D), generator=gen, device="cuda")
    chains = [(8191, 15), (8192, 0), (16383, 15), (16384, 0), (16639, 15)]
    host = {}
    for i, (n, h) in enumerate(chains):
        x = _host_chain(950 + 10 * T + i, T)
        for name in G.NAMES:
            _put(dev, name, (n, slice(None), h), x[name][0, :, 0])
        state[n, h] = torch.from_numpy(x["initial_state"][0, 0]).cuda()
        host[(n, h)] = x
    if T == 1:
        step = {name: dev[name][:, 0] for name in G.NAMES}
        o = binding.gdn2_recurrent_step(step["q"], step["k"], step["v"], step["alpha"], step["b"], step["w"], state)
        o = o[:, None]
    else:
        o = binding.gdn2_recurrent_fwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["b"], dev["w"], state)
    torch.cuda.synchronize()
    for (n, h), x in host.items():
        ro, rs = _oracle(x)
        G.assert_rel(G.f64(o[n, :, h]), ro, G.TOL["bf16"], f"large recurrent T={T} o ({n}, {h})")
        G.assert_rel(G.f64(state[n, h]), rs, G.TOL["bf16"], f"large recurrent T={T} state ({n}, {h})")


def test_mixer_past_4g_elements():
    """Prologue at B=520, T=4096, H=16, d=128, K=4, bf16 (4.4e9 elements per
    tensor): the last 48 tokens of chains beside the 2^31 and 2^32 element
    boundaries and at the end, with the three inputs before them as the
    convolution state on the oracle side; then the epilogue over the same
    4.4e9 elements with host rows at the same places."""
    import torch

    B, T, K, tail = 520, 4096, 4, 48
    gen = torch.Generator(device="cuda")
    gen.manual_seed(960)
    names = ("xq", "xk", "xv", "b_logit", "w_logit")
    dev = {n: torch.randn((B, T, H, D), generator=gen, device="cuda").to(torch.bfloat16) for n in names}
    rng = np.random.default_rng(961)
    conv = {n: (0.5 * rng.standard_normal((H * D, K))).astype(np.float32) for n in ("conv_q", "conv_k", "conv_v")}
    chains = [(255, 15), (256, 0), (511, 15), (512, 0), (519, 15)]
    host = {}
    for n, h in chains:
        x = {nm: W.round_bf16(rng.standard_normal((1, tail + K - 1, 1, D)).astype(np.float32)) for nm in names}
        for nm in names:
            dev[nm][n, T - tail - (K - 1):, h] = W.to_torch(x[nm][0, :, 0], "bf16", "cuda")
        host[(n, h)] = x
    cd = {nm: torch.from_numpy(a).cuda() for nm, a in conv.items()}
    out = binding.gdn2_mixer_prologue(dev["xq"], dev["xk"], dev["xv"], cd["conv_q"], cd["conv_k"], cd["conv_v"],
                                      dev["b_logit"], dev["w_logit"], q_scale=D ** -0.5)
    torch.cuda.synchronize()
    del dev
    for (n, h), x in host.items():
        # the window before the tail, oldest first, as the convolution state [1, H*(2dk+dv), K-1] of one head
        st = np.concatenate([x[nm][0, :K - 1, 0].T for nm in ("xq", "xk", "xv")], axis=0)[None]
        sub = {nm: np.ascontiguousarray(x[nm][:, K - 1:]) for nm in names}
        cw = {nm: conv[nm][h * D:(h + 1) * D] for nm in conv}
        ref = mixer.prologue(sub["xq"], sub["xk"], sub["xv"], cw["conv_q"], cw["conv_k"], cw["conv_v"],
                             sub["b_logit"], sub["w_logit"], conv_state=st, q_scale=D ** -0.5)
        for nm in ("q", "k", "v", "b", "w"):
            G.assert_rel(G.f64(out[nm][n, T - tail:, h]), ref[nm][0, :, 0], G.TOL["bf16"],
                         f"large prologue {nm} ({n}, {h})")
        # the carried state: the last K - 1 inputs, exactly
        cs = G.f64(out["conv_state"][n])
        for j, nm in enumerate(("xq", "xk", "xv")):
            np.testing.assert_array_equal(cs[(j * H + h) * D:(j * H + h + 1) * D], x[nm][0, tail:, 0].T)
    o_dev, g_dev = out["v"], out["b"]
    del out
    for n, h in chains:  # host rows: the last 256 tokens of each chain
        ho = W.round_bf16(rng.standard_normal((256, D)).astype(np.float32))
        hg = W.round_bf16(rng.standard_normal((256, D)).astype(np.float32))
        o_dev[n, T - 256:, h] = W.to_torch(ho, "bf16", "cuda")
        g_dev[n, T - 256:, h] = W.to_torch(hg, "bf16", "cuda")
        host[(n, h)] = (ho, hg)
    wgt = rng.standard_normal(D).astype(np.float32)
    y = binding.gdn2_mixer_epilogue(o_dev, g_dev, torch.from_numpy(wgt).cuda())
    torch.cuda.synchronize()
    for (n, h), (ho, hg) in host.items():
        G.assert_rel(G.f64(y[n, T - 256:, h]), mixer.epilogue(ho, hg, wgt), G.TOL["bf16"],
                     f"large epilogue ({n}, {h})")


def test_backward_past_4g_workspace_elements():
    """B=136, T=4096, H=16, d=128, bf16: the workspace's per-chunk state blocks
    hold 4.6e9 floats each (offsets past 2^32).  Chains beside the 2^31 and
    2^32 boundaries of that region (rows 64, 128) and the last."""
    import torch

    B, T = 136, 4096
    dev = W.device_token_tensors((B, T), H, D, D, "bf16", seed=970)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(971)
    s0 = 0.1 * torch.randn((B, H, D, D), generator=gen, device="cuda")
    d_o = torch.randn((B, T, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    dsf = torch.randn((B, H, D, D), generator=gen, device="cuda")
    chains = [(63, 15), (64, 0), (127, 15), (128, 0), (135, 15)]
    rng = np.random.default_rng(972)
    host = {}
    for i, (n, h) in enumerate(chains):
        x = _host_chain(980 + i, T)
        for name in G.NAMES:
            _put(dev, name, (n, slice(None), h), x[name][0, :, 0])
        s0[n, h] = torch.from_numpy(x["initial_state"][0, 0]).cuda()
        g = W.round_bf16(rng.standard_normal((1, T, 1, D)).astype(np.float32))
        gs = rng.standard_normal((1, 1, D, D)).astype(np.float32)
        d_o[n, :, h] = W.to_torch(g[0, :, 0], "bf16", "cuda")
        dsf[n, h] = torch.from_numpy(gs[0, 0]).cuda()
        host[(n, h)] = (x, g, gs)
    ws = binding.gdn2_chunk_bwd_workspace_bytes(B, T, H, D, D, B, binding.DTYPE_BF16)
    G.log(f"backward B={B}: workspace {ws / 2**30:.1f} GiB")
    out = binding.gdn2_chunk_bwd(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["b"], dev["w"], d_o, s0, dsf)
    torch.cuda.synchronize()
    for (n, h), (x, g, gs) in host.items():
        ref = oracle.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g, x["initial_state"], gs)
        for name in ("dq", "dk", "dv", "dalpha", "db", "dw"):
            G.assert_rel(G.f64(out[name][n, :, h]), ref[name][0, :, 0], G.TOL["bf16"], f"large bwd {name} ({n}, {h})")
        G.assert_rel(G.f64(out["d_initial_state"][n, h]), ref["d_initial_state"][0, 0], G.TOL["bf16"],
                     f"large bwd dS0 ({n}, {h})")
