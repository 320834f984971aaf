"""Pins for the FP64 oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
if the oracle's recurrence disagrees with the fact.  They are used twice: on
the real oracle (tests/test_oracle_pins.py) and on deliberately broken copies
of it (tests/test_oracle_mutants.py), which checks that every plausible
mistake in the recurrence is caught by at least one pin.

Sources, cited by page title and section:
  IPX = "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
        analysis (iplexlaw.co.kr)
  MP  = "DeltaNet" entity trail (mindpattern.ai), finding "You Could Have Come
        Up With Kimi Delta Attention"
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _close(x, ref, tol=TOL, what=""):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    err = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    assert err <= tol * scale, f"{what}: max |diff| {err:.3e} > {tol * scale:.3e}"


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def rand_inputs(seed, B=2, T=37, H=2, dk=8, dv=6, state=True, unit_k=True, alpha_mu=3.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = _sig(rng.normal(alpha_mu, 1.0, (B, T, H, dk)))
    b = _sig(rng.standard_normal((B, T, H, dk)))
    w = _sig(rng.standard_normal((B, T, H, dv)))
    s0 = 0.1 * rng.standard_normal((B, H, dk, dv)) if state else None
    return dict(q=q, k=k, v=v, alpha=alpha, b=b, w=w), s0


def _run(orc, x, s0=None, cu=None):
    return orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], s0, cu)


# --------------------------------------------------------------------------
# P1: worked example (exact rationals), tests/golden/worked_example_2x2.txt


def load_worked_example(path=os.path.join(GOLDEN, "worked_example_2x2.txt")):
    tokens, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "token":
            cur = {}
            tokens.append(cur)
        elif key in ("dk", "dv"):
            continue
        else:
            cur[key] = [Fraction(v) for v in vals]
    return tokens


def pin_worked_example(orc):
    """P1: hand-derived two-token example [IPX, "Independent decisions on two axes"]."""
    toks = load_worked_example()
    f = lambda key: np.array([[float(x) for x in t[key]] for t in toks]).reshape(1, len(toks), 1, 2)
    x = {name: f(name) for name in ("q", "k", "v", "alpha", "b", "w")}
    # after token 1 alone
    o1, s1 = _run(orc, {n: a[:, :1] for n, a in x.items()})
    _close(s1.reshape(4), [float(v) for v in toks[0]["S"]], 1e-15, "S after token 1")
    _close(o1.reshape(2), [float(v) for v in toks[0]["o"]], 1e-15, "o_1")
    o, s = _run(orc, x)
    _close(o.reshape(2, 2), [[float(v) for v in t["o"]] for t in toks], 1e-15, "o_1, o_2")
    _close(s.reshape(4), [float(v) for v in toks[1]["S"]], 1e-15, "S after token 2")


# --------------------------------------------------------------------------
# P2: with b = 0, w = 1, alpha = 1 the update is plain causal linear attention
# [MP: the outer-product identity; IPX "From a growing cache to a fixed state"].


def pin_linear_attention(orc):
    x, s0 = rand_inputs(11, unit_k=False)
    x["b"] = np.zeros_like(x["b"])
    x["w"] = np.ones_like(x["w"])
    x["alpha"] = np.ones_like(x["alpha"])
    o, s = _run(orc, x, s0)
    B, T, H, _ = x["q"].shape
    for n in range(B):
        for h in range(H):
            Q, K, V = x["q"][n, :, h], x["k"][n, :, h], x["v"][n, :, h]
            ref_o = np.tril(Q @ K.T) @ V + Q @ s0[n, h]
            ref_s = s0[n, h] + K.T @ V
            _close(o[n, :, h], ref_o, what=f"linear-attention o (n={n},h={h})")
            _close(s[n, h], ref_s, what=f"linear-attention state (n={n},h={h})")


# --------------------------------------------------------------------------
# P3: with b = w = 0 only the channel-wise decay acts, on key rows, before the
# read [IPX, "Independent decisions on two axes"]:  S_T = Diag(prod alpha) S0,
# o_t = S0^T (gamma_t * q_t) with gamma_t the running product of alpha.


def pin_pure_decay(orc):
    x, s0 = rand_inputs(12, dk=7, dv=5)
    x["b"] = np.zeros_like(x["b"])
    x["w"] = np.zeros_like(x["w"])
    o, s = _run(orc, x, s0)
    gamma = np.cumprod(x["alpha"], axis=1)                     # [B, T, H, dk]
    ref_o = np.einsum("bthc,bhcj->bthj", gamma * x["q"], s0)
    ref_s = gamma[:, -1][..., None] * s0
    _close(o, ref_o, what="pure-decay o")
    _close(s, ref_s, what="pure-decay state")


# --------------------------------------------------------------------------
# P4: the delta rule stores the prediction error, not the raw value [MP; IPX
# "From a growing cache to a fixed state"]: with b = w = 1 and a unit key the update makes the state
# return exactly v_t for key k_t, whatever the decay and the prior state.
# Reading with q_t = k_t, the output must be v_t at every token.


def pin_retrieval_any_alpha(orc):
    x, s0 = rand_inputs(13, alpha_mu=0.0)
    x["b"] = np.ones_like(x["b"])
    x["w"] = np.ones_like(x["w"])
    x["q"] = x["k"].copy()
    o, _ = _run(orc, x, s0)
    _close(o, x["v"], what="S_t^T k_t = v_t")


def pin_retrieval_orthonormal(orc):
    """With alpha = 1, S0 = 0 and orthonormal keys every stored pair is retrieved."""
    rng = np.random.default_rng(14)
    dk, dv, T = 8, 5, 6
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[:, :T].T.reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    x = dict(q=rng.standard_normal((1, T, 1, dk)), k=k, v=v, alpha=np.ones((1, T, 1, dk)),
             b=np.ones((1, T, 1, dk)), w=np.ones((1, T, 1, dv)))
    _, s = _run(orc, x)
    _close(k[0, :, 0] @ s[0, 0], v[0, :, 0], what="S_T^T k_j = v_j")


# --------------------------------------------------------------------------
# P5: reductions to the published relatives [IPX, "Independent decisions on
# two axes"]: b = w = beta gives KDA; a scalar decay as well gives Gated DeltaNet.


def pin_kda_reduction(orc):
    x, s0 = rand_inputs(15)
    rng = np.random.default_rng(150)
    beta = _sig(rng.standard_normal(x["q"].shape[:3]))
    x["b"] = np.broadcast_to(beta[..., None], x["b"].shape).copy()
    x["w"] = np.broadcast_to(beta[..., None], x["w"].shape).copy()
    o, s = _run(orc, x, s0)
    ok, sk = orc.kda(x["q"], x["k"], x["v"], x["alpha"], beta, s0)
    _close(o, ok, what="KDA o")
    _close(s, sk, what="KDA state")


def pin_gdn_reduction(orc):
    x, s0 = rand_inputs(16)
    rng = np.random.default_rng(160)
    beta = _sig(rng.standard_normal(x["q"].shape[:3]))
    a1 = _sig(rng.normal(3.0, 1.0, x["q"].shape[:3]))
    x["alpha"] = np.broadcast_to(a1[..., None], x["alpha"].shape).copy()
    x["b"] = np.broadcast_to(beta[..., None], x["b"].shape).copy()
    x["w"] = np.broadcast_to(beta[..., None], x["w"].shape).copy()
    o, s = _run(orc, x, s0)
    og, sg = orc.gdn(x["q"], x["k"], x["v"], a1, beta, s0)
    _close(o, og, what="GDN o")
    _close(s, sg, what="GDN state")


# --------------------------------------------------------------------------
# P6: the chunkwise WY form computes the same mathematics as the token loop
# [MP: the recurrent and chunkwise modes compute the same result; IPX "Token
# processing and parallel training"],
# for any chunk size, with a short last chunk, with and without packing.


def pin_chunked_equals_recurrent(orc):
    x, s0 = rand_inputs(17, T=37)
    o, s = _run(orc, x, s0)
    for C in (1, 2, 3, 5, 16, 64):
        oc, sc = orc.chunked(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], C, s0)
        _close(oc, o, what=f"chunked C={C} o")
        _close(sc, s, what=f"chunked C={C} state")
    cu = np.array([0, 5, 5, 29, 40], dtype=np.int32)
    xv, s0v = rand_inputs(18, B=1, T=40, state=True)
    s0v = 0.1 * np.random.default_rng(180).standard_normal((4,) + s0v.shape[1:])
    o, s = _run(orc, xv, s0v, cu)
    for C in (3, 16):
        oc, sc = orc.chunked(xv["q"], xv["k"], xv["v"], xv["alpha"], xv["b"], xv["w"], C, s0v, cu)
        _close(oc, o, what=f"varlen chunked C={C} o")
        _close(sc, s, what=f"varlen chunked C={C} state")


# --------------------------------------------------------------------------
# P7: products of per-token transitions (diagonal decay with a rank-one correction) [MP].


def pin_transition_products(orc):
    x, s0 = rand_inputs(19, T=23, dk=6, dv=4)
    o, s = _run(orc, x, s0)
    ot, st = orc.transition(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], s0)
    _close(ot, o, what="transition o")
    _close(st, s, what="transition state")


# --------------------------------------------------------------------------
# P8: value columns evolve independently: every shared quantity (k, e, alpha,
# q) is the same for all columns, and column j of the state only meets column
# j of z and r in the update [IPX, "Independent decisions on two axes"].


def pin_column_split(orc):
    x, s0 = rand_inputs(20, dv=7)
    o, s = _run(orc, x, s0)
    for lo, hi in ((0, 3), (3, 7), (2, 5)):
        xs = dict(x, v=x["v"][..., lo:hi], w=x["w"][..., lo:hi])
        op, sp = _run(orc, xs, s0[..., lo:hi])
        _close(op, o[..., lo:hi], what=f"columns [{lo},{hi}) o")
        _close(sp, s[..., lo:hi], what=f"columns [{lo},{hi}) state")


# --------------------------------------------------------------------------
# P9: the state is the whole memory of the past [IPX, "From a growing cache to
# a fixed state"]: splitting a sequence and passing the state on gives the same
# result; a packed batch equals its sequences run one by one.


def pin_state_passing(orc):
    x, s0 = rand_inputs(21, T=41)
    o, s = _run(orc, x, s0)
    for t1 in (1, 17, 40):
        oa, sa = _run(orc, {n: a[:, :t1] for n, a in x.items()}, s0)
        ob, sb = _run(orc, {n: a[:, t1:] for n, a in x.items()}, sa)
        _close(np.concatenate([oa, ob], axis=1), o, what=f"split at {t1} o")
        _close(sb, s, what=f"split at {t1} state")


def pin_packed_equals_separate(orc):
    lens = [7, 0, 19, 1, 13]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x, _ = rand_inputs(22, B=1, T=int(cu[-1]), state=False)
    s0 = 0.1 * np.random.default_rng(220).standard_normal((len(lens), 2, 8, 6))
    o, s = _run(orc, x, s0, cu)
    for n, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        on, sn = _run(orc, {k: v[:, a:e] for k, v in x.items()}, s0[n:n + 1])
        _close(o[:, a:e], on, what=f"packed seq {n} o")
        _close(s[n:n + 1], sn, what=f"packed seq {n} state")


# --------------------------------------------------------------------------
# P10: with k, b, alpha, q fixed the map (S0, v) -> (o, S_T) is linear: the
# update is affine in the state with a write term linear in v.


def pin_linearity(orc):
    x, s0 = rand_inputs(23)
    _, s1 = rand_inputs(24)
    v1 = np.random.default_rng(240).standard_normal(x["v"].shape)
    a, c = 0.7, -1.3
    oa, sa = _run(orc, x, s0)
    ob, sb = _run(orc, dict(x, v=v1), s1)
    oc, sc = _run(orc, dict(x, v=a * x["v"] + c * v1), a * s0 + c * s1)
    _close(oc, a * oa + c * ob, what="linearity o")
    _close(sc, a * sa + c * sb, what="linearity state")


PINS = [
    pin_worked_example,
    pin_linear_attention,
    pin_pure_decay,
    pin_retrieval_any_alpha,
    pin_retrieval_orthonormal,
    pin_kda_reduction,
    pin_gdn_reduction,
    pin_chunked_equals_recurrent,
    pin_transition_products,
    pin_column_split,
    pin_state_passing,
    pin_packed_equals_separate,
    pin_linearity,
]


# ==========================================================================
# Pins of the backward oracle O5 (gradients of O1).  The loss is
#   L = <dO, o> + <dS_final, S_final>;
# O5 must return its gradients.  The reference values come from central
# finite differences of the forward oracles, which are pinned above.

BWD_NAMES = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("alpha", "dalpha"), ("b", "db"), ("w", "dw"))


def _loss(orc, x, s0, g, gs, cu=None):
    o, s = orc.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], s0, cu)
    return float((o * g).sum() + (s * gs).sum())


def _fd(f, arr, idx, h=1e-6):
    """Central difference of f() with respect to arr[idx] (arr modified in place, restored)."""
    old = arr[idx]
    arr[idx] = old + h
    fp = f()
    arr[idx] = old - h
    fm = f()
    arr[idx] = old
    return (fp - fm) / (2 * h)


def _bwd_inputs(seed, B, T, H, dk, dv, N=None):
    x, _ = rand_inputs(seed, B=B, T=T, H=H, dk=dk, dv=dv, state=False)
    rng = np.random.default_rng(seed + 1000)
    N = B if N is None else N
    s0 = 0.3 * rng.standard_normal((N, H, dk, dv))
    g = rng.standard_normal((B, T, H, dv))
    gs = rng.standard_normal((N, H, dk, dv))
    return x, s0, g, gs


def _check_fd(orc, x, s0, g, gs, cu=None, sample=None, seed=0, tol=1e-6):
    gr = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g, s0, gs, cu)
    rng = np.random.default_rng(seed)
    targets = [(name, x[name], gr[key]) for name, key in BWD_NAMES] + [("s0", s0, gr["d_initial_state"])]
    for name, arr, an in targets:
        idxs = list(np.ndindex(arr.shape))
        if sample is not None and len(idxs) > sample:
            idxs = [idxs[i] for i in rng.choice(len(idxs), sample, replace=False)]
        fd = np.array([_fd(lambda: _loss(orc, x, s0, g, gs, cu), arr, i) for i in idxs])
        got = np.array([an[i] for i in idxs])
        scale = max(1e-3, float(np.abs(fd).max()))
        err = float(np.abs(got - fd).max())
        assert err <= tol * scale, f"d{name}: max |analytic - finite difference| {err:.3e} > {tol * scale:.3e}"


def pin_bwd_finite_differences(orc):
    """Every gradient entry of a small batched problem with an initial state
    and a final-state seed against central differences of O1."""
    x, s0, g, gs = _bwd_inputs(40, B=2, T=9, H=2, dk=3, dv=2)
    _check_fd(orc, x, s0, g, gs)


def pin_bwd_packed_long(orc):
    """Packed sequences (one empty, one crossing the 64-token recomputation
    segment of O5, one short) against central differences on sampled entries."""
    cu = np.array([0, 0, 70, 75], dtype=np.int32)
    x, s0, g, gs = _bwd_inputs(41, B=1, T=75, H=1, dk=2, dv=2, N=3)
    _check_fd(orc, x, s0, g, gs, cu=cu, sample=40, seed=41)


def pin_bwd_kda_chain_rule(orc):
    """With b = w = beta broadcast, dL/dbeta = sum_c db_c + sum_j dw_j and
    dL/dalpha = dalpha; the references are central differences of the KDA
    oracle O4a, an independent forward implementation."""
    x, s0, g, gs = _bwd_inputs(42, B=1, T=11, H=2, dk=3, dv=2)
    rng = np.random.default_rng(420)
    beta = _sig(rng.standard_normal(x["q"].shape[:3]))
    xb = dict(x, b=np.broadcast_to(beta[..., None], x["b"].shape).copy(),
              w=np.broadcast_to(beta[..., None], x["w"].shape).copy())
    gr = orc.backward(xb["q"], xb["k"], xb["v"], xb["alpha"], xb["b"], xb["w"], g, s0, gs)
    alpha = xb["alpha"].copy()

    def lk():
        o, s = orc.kda(xb["q"], xb["k"], xb["v"], alpha, beta, s0)
        return float((o * g).sum() + (s * gs).sum())

    fd_beta = np.array([_fd(lk, beta, i) for i in np.ndindex(beta.shape)]).reshape(beta.shape)
    fd_alpha = np.array([_fd(lk, alpha, i) for i in np.ndindex(alpha.shape)]).reshape(alpha.shape)
    _close(gr["db"].sum(-1) + gr["dw"].sum(-1), fd_beta, tol=1e-6, what="KDA dbeta")
    _close(gr["dalpha"], fd_alpha, tol=1e-6, what="KDA dalpha")


def pin_bwd_gdn_chain_rule(orc):
    """With a scalar decay broadcast over the key channels, dL/dalpha_scalar =
    sum_c dalpha_c; the reference is central differences of the Gated DeltaNet
    oracle O4b."""
    x, s0, g, gs = _bwd_inputs(43, B=1, T=11, H=2, dk=3, dv=2)
    rng = np.random.default_rng(430)
    beta = _sig(rng.standard_normal(x["q"].shape[:3]))
    a1 = _sig(rng.normal(2.0, 1.0, x["q"].shape[:3]))
    xb = dict(x, b=np.broadcast_to(beta[..., None], x["b"].shape).copy(),
              w=np.broadcast_to(beta[..., None], x["w"].shape).copy(),
              alpha=np.broadcast_to(a1[..., None], x["alpha"].shape).copy())
    gr = orc.backward(xb["q"], xb["k"], xb["v"], xb["alpha"], xb["b"], xb["w"], g, s0, gs)

    def lg():
        o, s = orc.gdn(xb["q"], xb["k"], xb["v"], a1, beta, s0)
        return float((o * g).sum() + (s * gs).sum())

    fd_a = np.array([_fd(lg, a1, i) for i in np.ndindex(a1.shape)]).reshape(a1.shape)
    _close(gr["dalpha"].sum(-1), fd_a, tol=1e-6, what="GDN dalpha")


def pin_bwd_causal(orc):
    """A seed on the output of token t0 alone (no final-state seed) leaves the
    gradients of every later token zero, and of token t0 itself dq nonzero."""
    x, s0, g, gs = _bwd_inputs(44, B=1, T=12, H=1, dk=4, dv=3)
    t0 = 6
    g1 = np.zeros_like(g)
    g1[:, t0] = g[:, t0]
    gr = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g1, s0, None)
    for _, key in BWD_NAMES:
        assert not gr[key][:, t0 + 1:].any(), f"{key}: nonzero after the seeded token"
    assert np.abs(gr["dq"][:, t0]).max() > 0


def pin_bwd_linear_in_seeds(orc):
    """The gradients are linear in the seeds (dO, dS_final)."""
    x, s0, g, gs = _bwd_inputs(45, B=1, T=10, H=2, dk=3, dv=3)
    rng = np.random.default_rng(450)
    g2, gs2 = rng.standard_normal(g.shape), rng.standard_normal(gs.shape)
    a, c = 0.7, -1.3
    r1 = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g, s0, gs)
    r2 = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], g2, s0, gs2)
    r3 = orc.backward(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"], a * g + c * g2, s0, a * gs + c * gs2)
    for key in r1:
        _close(r3[key], a * r1[key] + c * r2[key], tol=1e-11, what=f"linearity {key}")


BACKWARD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_packed_long,
    pin_bwd_kda_chain_rule,
    pin_bwd_gdn_chain_rule,
    pin_bwd_causal,
    pin_bwd_linear_in_seeds,
]
