"""FP64 CPU oracle for the Gated DeltaNet-2 forward recurrence.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
``cpu_baseline`` leg are the only users.  The product (the HIP library and its
binding) never imports this package, and this package imports nothing from
the product.

The arithmetic lives in ``gdn2_oracle.c`` (plain loops, FP64); this module
only marshals numpy arrays.  Sources, cited by page title and section:

* "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention" analysis
  (iplexlaw.co.kr), "Independent decisions on two axes": the update
  e = b*k, z = w*v, Sbar = Diag(alpha) S, r = Sbar^T e, S = Sbar + k (z - r)^T,
  and the output is read from the state after the update.  -> ``recurrent``
  (THE oracle).
* Same page, "Token processing and parallel training": 64-token chunkwise WY
  form, the running per-channel decay folded into unequal row and column
  factors.
  -> ``chunked`` (any chunk size; a self-consistency pin).
* "DeltaNet" entity trail (mindpattern.ai), "You Could Have Come Up With Kimi
  Delta Attention": each token's transition is a diagonal decay composed with
  a rank-one correction of the identity, and the chunkwise and fused
  recurrent forms compute the same result.  -> ``transition``.
* IPX "Independent decisions on two axes": tying b = w = beta gives KDA, and a
  scalar decay as well gives Gated DeltaNet.  -> ``kda``, ``gdn``.

All functions take float arrays of shape q, k, b, alpha: [B, T, H, dk];
v, w: [B, T, H, dv]; state: [N, H, dk, dv] and return FP64 ``(o, final_state)``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def load(path: str | None = None):
    """Load (building first if stale) the oracle shared library.  The
    environment variable GDN2_ORACLE_LIB names another build of the same
    source to load instead (the sanitizer check uses it)."""
    global _LIB
    if path is None and os.environ.get("GDN2_ORACLE_LIB"):
        path = os.environ["GDN2_ORACLE_LIB"]
        if _LIB is None:
            _LIB = ctypes.CDLL(path)
            _declare(_LIB)
        return _LIB
    if path is not None:
        lib = ctypes.CDLL(path)
        _declare(lib)
        return lib
    if _LIB is None:
        if _build.needs_build():
            _build.compile_oracle()
        _LIB = ctypes.CDLL(_build.LIB)
        _declare(_LIB)
    return _LIB


_P = ctypes.c_void_p
_I = ctypes.c_int32


def _declare(lib) -> None:
    six = [_P] * 6
    common = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I]
    tail = [_P, _I, _I]
    lib.gdn2_oracle_recurrent.argtypes = six + common + tail
    lib.gdn2_oracle_transition.argtypes = six + common + tail
    lib.gdn2_oracle_chunked.argtypes = six + common + [_I] + tail
    lib.gdn2_oracle_kda.argtypes = [_P] * 5 + common + tail
    lib.gdn2_oracle_gdn.argtypes = [_P] * 5 + common + tail
    lib.gdn2_oracle_backward.argtypes = six + [_P, _P, _P] + [_P] * 7 + [_P, _I, _I, _I, _I, _I, _I] + tail
    for name in ("recurrent", "transition", "chunked", "kda", "gdn", "backward"):
        getattr(lib, "gdn2_oracle_" + name).restype = ctypes.c_int
    lib.gdn2_oracle_max_threads.argtypes = []
    lib.gdn2_oracle_max_threads.restype = ctypes.c_int


def max_threads() -> int:
    return int(load().gdn2_oracle_max_threads())


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _prepare(q, k, v, initial_state, cu_seqlens, chains):
    q = _f64(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = int(cu.shape[0] - 1)
    else:
        cu = None
        N = B
    s0 = _f64(initial_state)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError(f"initial_state shape {s0.shape} != {(N, H, dk, dv)}")
    ch = None if chains is None else np.ascontiguousarray(chains, dtype=np.int32)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    if s0 is not None and ch is not None:
        sf[...] = s0  # untouched chains keep their initial state
    return q, (B, T, H, dk, dv, N), cu, s0, ch, o, sf


def _call(fn, arrays, dims, cu, s0, sf, o, ch, threads, extra=()):
    B, T, H, dk, dv, N = dims
    rc = fn(*[_ptr(a) for a in arrays], _ptr(s0), _ptr(sf), _ptr(o), _ptr(cu),
            B, T, H, dk, dv, N, *extra, _ptr(ch), 0 if ch is None else int(ch.shape[0]),
            int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")


class Oracle:
    """The oracle functions bound to one build of the library."""

    def __init__(self, lib):
        self.lib = lib

    def recurrent(self, q, k, v, alpha, b, w, initial_state=None, cu_seqlens=None, chains=None,
                  threads=0):
        """O1: the token-by-token recurrence in FP64 (the oracle)."""
        q, dims, cu, s0, ch, o, sf = _prepare(q, k, v, initial_state, cu_seqlens, chains)
        arrays = [q] + [_f64(x) for x in (k, v, alpha, b, w)]
        _call(self.lib.gdn2_oracle_recurrent, arrays, dims, cu, s0, sf, o, ch, threads)
        return o, sf

    def chunked(self, q, k, v, alpha, b, w, chunk, initial_state=None, cu_seqlens=None,
                chains=None, threads=0):
        """O2: chunkwise WY form with chunk size ``chunk`` in FP64."""
        q, dims, cu, s0, ch, o, sf = _prepare(q, k, v, initial_state, cu_seqlens, chains)
        arrays = [q] + [_f64(x) for x in (k, v, alpha, b, w)]
        _call(self.lib.gdn2_oracle_chunked, arrays, dims, cu, s0, sf, o, ch, threads,
              extra=(int(chunk),))
        return o, sf

    def transition(self, q, k, v, alpha, b, w, initial_state=None, cu_seqlens=None, chains=None,
                   threads=0):
        """O3: explicit transition-matrix products in FP64."""
        q, dims, cu, s0, ch, o, sf = _prepare(q, k, v, initial_state, cu_seqlens, chains)
        arrays = [q] + [_f64(x) for x in (k, v, alpha, b, w)]
        _call(self.lib.gdn2_oracle_transition, arrays, dims, cu, s0, sf, o, ch, threads)
        return o, sf

    def kda(self, q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, chains=None,
            threads=0):
        """O4a: Kimi Delta Attention form; alpha [B,T,H,dk], beta [B,T,H]."""
        q, dims, cu, s0, ch, o, sf = _prepare(q, k, v, initial_state, cu_seqlens, chains)
        arrays = [q] + [_f64(x) for x in (k, v, alpha, beta)]
        _call(self.lib.gdn2_oracle_kda, arrays, dims, cu, s0, sf, o, ch, threads)
        return o, sf

    def gdn(self, q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, chains=None,
            threads=0):
        """O4b: Gated DeltaNet form; alpha [B,T,H] (scalar decay), beta [B,T,H]."""
        q, dims, cu, s0, ch, o, sf = _prepare(q, k, v, initial_state, cu_seqlens, chains)
        arrays = [q] + [_f64(x) for x in (k, v, alpha, beta)]
        _call(self.lib.gdn2_oracle_gdn, arrays, dims, cu, s0, sf, o, ch, threads)
        return o, sf


    def backward(self, q, k, v, alpha, b, w, d_o, initial_state=None, d_final_state=None, cu_seqlens=None,
                 chains=None, threads=0):
        """O5: gradients of O1 for the loss <d_o, o> + <d_final_state, S_final>.

        Returns dict(dq, dk, dv, dalpha, db, dw, d_initial_state) in FP64 (chains
        not selected by ``chains`` are left zero)."""
        q, dims, cu, s0, ch, o, sf = _prepare(q, k, v, initial_state, cu_seqlens, chains)
        B, T, H, dk, dv, N = dims
        g = _f64(d_o)
        if g.shape != (B, T, H, dv):
            raise ValueError(f"d_o shape {g.shape} != {(B, T, H, dv)}")
        dsf = _f64(d_final_state)
        if dsf is not None and dsf.shape != (N, H, dk, dv):
            raise ValueError(f"d_final_state shape {dsf.shape} != {(N, H, dk, dv)}")
        out = {name: np.zeros((B, T, H, width), dtype=np.float64)
               for name, width in (("dq", dk), ("dk", dk), ("dv", dv), ("dalpha", dk), ("db", dk), ("dw", dv))}
        out["d_initial_state"] = np.zeros((N, H, dk, dv), dtype=np.float64)
        arrays = [q] + [_f64(x) for x in (k, v, alpha, b, w)]
        rc = self.lib.gdn2_oracle_backward(
            *[_ptr(a) for a in arrays], _ptr(s0), _ptr(g), _ptr(dsf),
            *[_ptr(out[n]) for n in ("dq", "dk", "dv", "dalpha", "db", "dw", "d_initial_state")],
            _ptr(cu), B, T, H, dk, dv, N, _ptr(ch), 0 if ch is None else int(ch.shape[0]), int(threads))
        if rc != 0:
            raise ValueError(f"oracle rejected its arguments (rc={rc})")
        return out


_DEFAULT = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(load())
    return _DEFAULT


def recurrent(*args, **kw):
    return default().recurrent(*args, **kw)


def chunked(*args, **kw):
    return default().chunked(*args, **kw)


def transition(*args, **kw):
    return default().transition(*args, **kw)


def kda(*args, **kw):
    return default().kda(*args, **kw)


def gdn(*args, **kw):
    return default().gdn(*args, **kw)


def backward(*args, **kw):
    return default().backward(*args, **kw)


def rel_l2(x, ref) -> float:
    """Relative L2 error ||x - ref|| / ||ref|| in FP64 over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    return num / den if den > 0 else num


__all__ = ["Oracle", "default", "recurrent", "chunked", "transition", "kda", "gdn", "rel_l2",
           "max_threads", "load"]
