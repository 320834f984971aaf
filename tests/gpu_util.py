"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
HIP path through the C ABI (via the ctypes binding), and evaluate the FP64
oracle on whole tensors or on sampled (sequence, head) chains."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from delta_rule_linear_gdn2_amd import binding
from delta_rule_linear_gdn2_amd import workloads as W

TOL = {"f32": 1e-4, "bf16": 1e-2}
NAMES = ("q", "k", "v", "alpha", "b", "w")


def log(msg):
    print(f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: dict, dtype: str):
    import torch

    d = {}
    for n in NAMES:
        d[n] = W.to_torch(x[n], "f32" if n == "alpha" else dtype, "cuda")
    s0 = x.get("initial_state")
    d["initial_state"] = None if s0 is None else torch.from_numpy(np.ascontiguousarray(s0)).cuda()
    cu = x.get("cu_seqlens")
    d["cu_seqlens"] = None if cu is None else torch.from_numpy(np.ascontiguousarray(cu)).cuda()
    return d


def gpu_chunk(d: dict, **kw):
    import torch

    o, sf = binding.gdn2_chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["b"], d["w"],
                                   d["initial_state"], cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, sf


def f64(t):
    import torch

    return t.detach().to(torch.float64).cpu().numpy()


def oracle_full(x: dict, threads=0):
    return oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["b"], x["w"],
                            x.get("initial_state"), x.get("cu_seqlens"), threads=threads)


def chain_slice(x: dict, n: int, h: int):
    """Inputs of one (sequence, head) chain as a B=1, H=1 problem."""
    cu = x.get("cu_seqlens")
    if cu is not None:
        lo, hi = int(cu[n]), int(cu[n + 1])
        sl = {k: x[k][0:1, lo:hi, h:h + 1] for k in NAMES}
    else:
        lo = hi = None
        sl = {k: x[k][n:n + 1, :, h:h + 1] for k in NAMES}
    s0 = x.get("initial_state")
    sl["initial_state"] = None if s0 is None else s0[n:n + 1, h:h + 1]
    return sl, (lo, hi)


def oracle_chain(x: dict, n: int, h: int):
    sl, _ = chain_slice(x, n, h)
    o, s = oracle.recurrent(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["b"], sl["w"],
                            sl["initial_state"])
    return o[0, :, 0], s[0, 0]


def gpu_chain_view(o_gpu: np.ndarray, s_gpu: np.ndarray, x: dict, n: int, h: int):
    cu = x.get("cu_seqlens")
    if cu is not None:
        lo, hi = int(cu[n]), int(cu[n + 1])
        return o_gpu[0, lo:hi, h], s_gpu[n, h]
    return o_gpu[n, :, h], s_gpu[n, h]


def chain_sq_sums(x: np.ndarray, cu=None):
    """Sum of squares per (sequence, head) chain of an output [B, T, H, d]
    (batched) or [1, T_total, H, d] (packed by ``cu``): returns [N, H]."""
    per_tok = np.einsum("bthd,bthd->bth", x, x)
    if cu is None:
        return per_tok.sum(axis=1)
    c = np.concatenate([np.zeros((1, per_tok.shape[2])), np.cumsum(per_tok[0], axis=0)])
    cu = np.asarray(cu, dtype=np.int64)
    return c[cu[1:]] - c[cu[:-1]]


def assert_chains(o, s, ro, rs, tol, what, cu=None):
    """Whole-tensor relative L2 of the outputs and of the final states against
    the oracle, plus the worst (sequence, head) chain of each as a log line."""
    eo = assert_rel(o, ro, tol, f"{what} o")
    es = assert_rel(s, rs, tol, f"{what} final state")
    num_o = chain_sq_sums(o - ro, cu)
    den_o = chain_sq_sums(ro, cu)
    with np.errstate(divide="ignore", invalid="ignore"):
        per_o = np.sqrt(np.where(den_o > 0, num_o / den_o, num_o))
        per_s = np.sqrt(((s - rs) ** 2).sum(axis=(2, 3)) / np.maximum((rs ** 2).sum(axis=(2, 3)), 1e-300))
    wo = np.unravel_index(int(np.argmax(per_o)), per_o.shape)
    ws = np.unravel_index(int(np.argmax(per_s)), per_s.shape)
    log(f"{what}: {per_o.size} chains; worst o chain (n={wo[0]}, h={wo[1]}) rel L2 {per_o[wo]:.3e}; "
        f"worst state chain (n={ws[0]}, h={ws[1]}) rel L2 {per_s[ws]:.3e}")
    return eo, es


def assert_rel(x, ref, tol, what):
    err = oracle.rel_l2(x, ref)
    log(f"{what}: rel L2 = {err:.3e} (tol {tol:.0e})")
    assert np.isfinite(err) and err <= tol, f"{what}: rel L2 {err:.3e} > {tol:.0e}"
    return err
