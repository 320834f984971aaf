"""FP64 oracle of the token mixer around the recurrence (TEST INFRASTRUCTURE ONLY).

The "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
analysis (iplexlaw.co.kr), section "Token processing and parallel training",
lists the layer around the recurrence.  Queries and keys go through a linear
projection, a causal convolution of a few taps, SiLU and an L2 norm; values
through a projection, a convolution and SiLU.  The erase and
write gates come from their own projections through a sigmoid (section
"Independent decisions on two axes").  After the recurrence, an RMS
normalisation and a separate output gate precede the output projection.  The
projections are dense layers over trained weights and are not part of this
oracle.  Everything else is written out here in plain loops, one
(sequence, head, channel) at a time.

Readings where the page is silent:
  * The convolution is depthwise (one filter per channel) and causal.  Its
    kernel has K taps, and tap K - 1 multiplies the current token.  A
    sequence starts from a convolution state: the K - 1 inputs before it,
    oldest first, or zeros.  The state after a sequence is its last K - 1
    inputs, in the same layout.
  * L2 normalisation is x / sqrt(sum x^2 + eps_l2).  The query is then
    multiplied by q_scale, since the recurrence itself has no query scale.
  * RMS normalisation is o / sqrt(mean o^2 + eps_rms) times a per-channel
    weight.
  * The output-gate activation is a parameter: "sigmoid" or "silu".

Layouts: x tensors [B, T, H, d] (packed sequences: B = 1 with cu_seqlens
[N + 1]); filters [H * d, K]; convolution state [N, H * d, K - 1].
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _bounds(B, T, cu, n):
    if cu is None:
        return n, 0, T
    return 0, int(cu[n]), int(cu[n + 1])


def sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x)) if x >= 0 else math.exp(x) / (1.0 + math.exp(x))


def silu(x):
    return x * sigmoid(x)


def causal_conv(x, weight, cu_seqlens=None, state=None):
    """Depthwise causal convolution.  x [B, T, H, d], weight [H * d, K],
    state [N, H * d, K - 1] or None (zeros).  Returns (y, final_state)."""
    x = _f64(x)
    weight = _f64(weight)
    B, T, H, d = x.shape
    K = weight.shape[1]
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    st = np.zeros((N, H * d, K - 1)) if state is None else _f64(state)
    y = np.zeros_like(x)
    out_state = np.zeros((N, H * d, K - 1))
    for n in range(N):
        row, bos, eos = _bounds(B, T, cu_seqlens, n)
        for h in range(H):
            for c in range(d):
                ch = h * d + c

                def inp(s):  # input at packed position s of sequence n
                    if s >= bos:
                        return x[row, s, h, c]
                    j = (K - 1) - (bos - s)  # position in the state, oldest first
                    return st[n, ch, j] if j >= 0 else 0.0

                for t in range(bos, eos):
                    acc = 0.0
                    for i in range(K):
                        acc += weight[ch, i] * inp(t - (K - 1) + i)
                    y[row, t, h, c] = acc
                for j in range(K - 1):
                    out_state[n, ch, j] = inp(eos - (K - 1) + j)
    return y, out_state


def l2_normalize(x, eps):
    """x / sqrt(sum over the last axis of x^2 + eps), row by row."""
    x = _f64(x)
    out = np.zeros_like(x)
    for idx in np.ndindex(x.shape[:-1]):
        ss = 0.0
        for val in x[idx]:
            ss += val * val
        out[idx] = x[idx] / math.sqrt(ss + eps)
    return out


def prologue(xq, xk, xv, conv_q, conv_k, conv_v, b_logit, w_logit, cu_seqlens=None, conv_state=None,
             q_scale=1.0, eps_l2=1e-6):
    """q, k, v, b, w of the recurrence from the projection outputs.

    conv_state: [N, H * (2 dk + dv), K - 1] or None; channels are q (H * dk),
    then k (H * dk), then v (H * dv).  Returns dict(q, k, v, b, w,
    conv_state)."""
    xq, xk, xv = _f64(xq), _f64(xk), _f64(xv)
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    sq = sk = sv = None
    if conv_state is not None:
        cs = _f64(conv_state)
        sq, sk, sv = cs[:, :H * dk], cs[:, H * dk:2 * H * dk], cs[:, 2 * H * dk:]
    yq, oq = causal_conv(xq, conv_q, cu_seqlens, sq)
    yk, ok = causal_conv(xk, conv_k, cu_seqlens, sk)
    yv, ov = causal_conv(xv, conv_v, cu_seqlens, sv)
    act = np.vectorize(silu)
    q = l2_normalize(act(yq), eps_l2) * q_scale
    k = l2_normalize(act(yk), eps_l2)
    v = act(yv)
    sig = np.vectorize(sigmoid)
    b = sig(_f64(b_logit))
    w = sig(_f64(w_logit))
    return dict(q=q, k=k, v=v, b=b, w=w, conv_state=np.concatenate([oq, ok, ov], axis=1))


def epilogue(o, gate, weight, eps_rms=1e-5, act="sigmoid"):
    """RMS-normalised o (last axis) times weight, times act(gate)."""
    o, gate, weight = _f64(o), _f64(gate), _f64(weight)
    f = sigmoid if act == "sigmoid" else silu
    y = np.zeros_like(o)
    d = o.shape[-1]
    for idx in np.ndindex(o.shape[:-1]):
        ms = 0.0
        for val in o[idx]:
            ms += val * val
        r = 1.0 / math.sqrt(ms / d + eps_rms)
        for c in range(d):
            y[idx + (c,)] = o[idx + (c,)] * r * weight[c] * f(gate[idx + (c,)])
    return y
