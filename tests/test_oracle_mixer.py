"""Pins of the token-mixer oracle (oracle/mixer.py), CPU only.

Closed forms of the convolution, torch's CPU library routines for each
stage, and invariants (packed sequences equal separate runs; carrying the
convolution state equals one run)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mixer


def _x(seed, B=2, T=9, H=2, d=3):
    return np.random.default_rng(seed).standard_normal((B, T, H, d))


def test_conv_impulse_is_identity():
    x = _x(1)
    w = np.zeros((6, 4))
    w[:, 3] = 1.0
    y, _ = mixer.causal_conv(x, w)
    np.testing.assert_allclose(y, x, rtol=0, atol=0)


def test_conv_first_tap_is_a_delay():
    x = _x(2)
    rng = np.random.default_rng(20)
    K = 4
    state = rng.standard_normal((2, 6, K - 1))
    w = np.zeros((6, K))
    w[:, 0] = 1.0
    y, s_out = mixer.causal_conv(x, w, state=state)
    for n in range(2):
        for h in range(2):
            for c in range(3):
                ch = h * 3 + c
                for t in range(9):
                    exp = x[n, t - 3, h, c] if t >= 3 else state[n, ch, t]
                    assert y[n, t, h, c] == exp
                # final state: the last three inputs, oldest first
                np.testing.assert_array_equal(s_out[n, ch], x[n, 6:9, h, c])


def test_conv_matches_torch_conv1d():
    x = _x(3, B=2, T=11, H=3, d=4)
    w = np.random.default_rng(30).standard_normal((12, 4))
    y, _ = mixer.causal_conv(x, w)
    xt = torch.from_numpy(x).reshape(2, 11, 12).transpose(1, 2)          # [B, channels, T]
    yt = F.conv1d(F.pad(xt, (3, 0)), torch.from_numpy(w).unsqueeze(1), groups=12)
    np.testing.assert_allclose(y, yt.transpose(1, 2).reshape(2, 11, 3, 4).numpy(), rtol=1e-12, atol=1e-12)


def test_conv_packed_equals_separate_and_state_passing():
    rng = np.random.default_rng(4)
    lens = [5, 0, 2, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = rng.standard_normal((1, int(cu[-1]), 2, 3))
    w = rng.standard_normal((6, 4))
    st = rng.standard_normal((4, 6, 3))
    y, s = mixer.causal_conv(x, w, cu, st)
    for n, L in enumerate(lens):
        yn, sn = mixer.causal_conv(x[:, cu[n]:cu[n + 1]], w, None, st[n:n + 1])
        np.testing.assert_allclose(y[:, cu[n]:cu[n + 1]], yn, rtol=0, atol=1e-15)
        np.testing.assert_allclose(s[n:n + 1], sn, rtol=0, atol=1e-15)
    # one token at a time through the state == one run
    y1, s1 = mixer.causal_conv(x[:, :7], w, None, st[:1])
    sc = st[:1]
    for t in range(7):
        yt, sc = mixer.causal_conv(x[:, t:t + 1], w, None, sc)
        np.testing.assert_allclose(yt[:, 0], y1[:, t], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sc, s1, rtol=0, atol=1e-15)


def test_activations_match_torch():
    z = np.linspace(-30, 30, 121)
    sig = np.array([mixer.sigmoid(v) for v in z])
    silu = np.array([mixer.silu(v) for v in z])
    np.testing.assert_allclose(sig, torch.sigmoid(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(silu, F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-14)


def test_prologue_stages_match_torch():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv, K = 2, 6, 2, 4, 3, 4
    xq, xk = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))
    xv = rng.standard_normal((B, T, H, dv))
    cq, ck, cv = (rng.standard_normal((H * d, K)) for d in (dk, dk, dv))
    bl, wl = rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dv))
    out = mixer.prologue(xq, xk, xv, cq, ck, cv, bl, wl, q_scale=0.5, eps_l2=0.0)

    def torch_path(x, wgt, d, norm):
        xt = torch.from_numpy(x).reshape(B, T, H * d).transpose(1, 2)
        y = F.conv1d(F.pad(xt, (K - 1, 0)), torch.from_numpy(wgt).unsqueeze(1), groups=H * d)
        y = F.silu(y.transpose(1, 2).reshape(B, T, H, d))
        return F.normalize(y, dim=-1, eps=1e-300) if norm else y

    np.testing.assert_allclose(out["q"], 0.5 * torch_path(xq, cq, dk, True).numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["k"], torch_path(xk, ck, dk, True).numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["v"], torch_path(xv, cv, dv, False).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["b"], torch.sigmoid(torch.from_numpy(bl)).numpy(), rtol=1e-14)
    np.testing.assert_allclose(out["w"], torch.sigmoid(torch.from_numpy(wl)).numpy(), rtol=1e-14)
    # the combined state holds the three paths' final states in order q, k, v
    _, sk = mixer.causal_conv(xk, ck)
    np.testing.assert_array_equal(out["conv_state"][:, H * dk:2 * H * dk], sk)


@pytest.mark.parametrize("act", ["sigmoid", "silu"])
def test_epilogue_matches_torch(act):
    rng = np.random.default_rng(6)
    o, gate = rng.standard_normal((3, 5, 2, 8)), rng.standard_normal((3, 5, 2, 8))
    wgt = rng.standard_normal(8)
    y = mixer.epilogue(o, gate, wgt, eps_rms=1e-5, act=act)
    ot = torch.from_numpy(o)
    ref = F.rms_norm(ot, (8,), torch.from_numpy(wgt), eps=1e-5)
    ref = ref * (torch.sigmoid(torch.from_numpy(gate)) if act == "sigmoid" else F.silu(torch.from_numpy(gate)))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_l2_normalize_eps_closed_form():
    # sqrt(3^2 + 4^2 + 11) = 6; a zero row stays zero
    np.testing.assert_allclose(mixer.l2_normalize(np.array([[3.0, 4.0], [0.0, 0.0]]), 11.0),
                               [[0.5, 4.0 / 6.0], [0.0, 0.0]], rtol=1e-15)
