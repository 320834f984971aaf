"""ctypes binding of ``libgdn2.so`` (the C ABI declared in include/gdn2.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing or cannot bind to the
HIP runtime torch uses, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# GDN2_LIBRARY names another build of the library to load (the sanitizer
# check loads a build whose host code carries AddressSanitizer).
LIB_PATH = os.environ.get("GDN2_LIBRARY") or os.path.join(PKG, "libgdn2.so")

GDN2_OK = 0
STATUS_NAMES = {
    0: "GDN2_OK", 1: "GDN2_ERR_NULL_POINTER", 2: "GDN2_ERR_BAD_SHAPE", 3: "GDN2_ERR_UNSUPPORTED",
    4: "GDN2_ERR_BAD_DTYPE", 5: "GDN2_ERR_MISALIGNED", 6: "GDN2_ERR_ALIAS", 7: "GDN2_ERR_WORKSPACE",
    8: "GDN2_ERR_HIP",
}
DTYPE_F32 = 0
DTYPE_BF16 = 1

EXPORTS = ("gdn2_chunk_bwd", "gdn2_chunk_bwd_noalloc", "gdn2_chunk_bwd_noalloc_max_workspace_bytes",
           "gdn2_chunk_bwd_workspace_bytes", "gdn2_chunk_fwd", "gdn2_chunk_fwd_gates",
           "gdn2_chunk_fwd_workspace_bytes",
           "gdn2_mixer_epilogue", "gdn2_mixer_prologue", "gdn2_recurrent_fwd", "gdn2_recurrent_step",
           "gdn2_recurrent_step_gates", "gdn2_status_string", "gdn2_version")

# gdn2_gate_flags: layout of the gates (b, w, alpha), OR-ed together
GATES_FULL, GATES_SCALAR_ERASE, GATES_SCALAR_WRITE, GATES_TIED, GATES_SCALAR_DECAY = 0, 1, 2, 4, 8
GATES_KDA = GATES_SCALAR_ERASE | GATES_TIED
GATES_GDN = GATES_KDA | GATES_SCALAR_DECAY
VALID_GATES = (0, 1, 2, 3, 5, 8, 9, 10, 11, 13)


class Gdn2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)}")


_LIB = None


def _hip_runtimes_loaded() -> set[str]:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load(path: str = LIB_PATH):
    """Load ``libgdn2.so`` (after torch, so it binds to torch's HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  -- loads torch's libamdhip64 first (same SONAME)

    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with `python -m delta_rule_linear_gdn2_amd.build` "
            "(the GDN-2 ops have no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.gdn2_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.gdn2_chunk_fwd.restype = ctypes.c_int
    lib.gdn2_chunk_fwd_gates.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, Z, P]
    lib.gdn2_chunk_fwd_gates.restype = ctypes.c_int
    lib.gdn2_chunk_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.gdn2_chunk_fwd_workspace_bytes.restype = Z
    lib.gdn2_recurrent_step.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.gdn2_recurrent_step.restype = ctypes.c_int
    lib.gdn2_recurrent_step_gates.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.gdn2_recurrent_step_gates.restype = ctypes.c_int
    lib.gdn2_recurrent_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.gdn2_recurrent_fwd.restype = ctypes.c_int
    lib.gdn2_chunk_bwd.argtypes = [P] * 17 + [I, I, I, I, I, I, I, P, Z, P]
    lib.gdn2_chunk_bwd.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_noalloc.argtypes = [P] * 17 + [I, I, I, I, I, I, I, P]
    lib.gdn2_chunk_bwd_noalloc.restype = ctypes.c_int
    lib.gdn2_chunk_bwd_noalloc_max_workspace_bytes.argtypes = []
    lib.gdn2_chunk_bwd_noalloc_max_workspace_bytes.restype = Z
    lib.gdn2_chunk_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.gdn2_chunk_bwd_workspace_bytes.restype = Z
    F = ctypes.c_float
    lib.gdn2_mixer_prologue.argtypes = [P] * 16 + [I] * 7 + [F, F, I, P]
    lib.gdn2_mixer_prologue.restype = ctypes.c_int
    lib.gdn2_mixer_epilogue.argtypes = [P, P, P, P, ctypes.c_int64, I, F, I, I, P]
    lib.gdn2_mixer_epilogue.restype = ctypes.c_int
    lib.gdn2_status_string.argtypes = [ctypes.c_int]
    lib.gdn2_status_string.restype = ctypes.c_char_p
    lib.gdn2_version.argtypes = []
    lib.gdn2_version.restype = ctypes.c_int32
    runtimes = _hip_runtimes_loaded()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped in this process: {sorted(runtimes)}")
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().gdn2_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt) -> int:
    import torch

    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _check(name, t, shape, dtype, device):
    if t.shape != shape:
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {shape}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, num_seqs, dtype_code) -> int:
    return int(load().gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, num_seqs, dtype_code))


def _gate_widths(gates, dk, dv):
    """Trailing sizes of (b, w, alpha) for a gate layout (w None: not used)."""
    if gates not in VALID_GATES:
        raise ValueError(f"gates must be one of {VALID_GATES} (got {gates})")
    bw = () if gates & GATES_SCALAR_ERASE else (dk,)
    ww = None if gates & GATES_TIED else () if gates & GATES_SCALAR_WRITE else (dv,)
    aw = () if gates & GATES_SCALAR_DECAY else (dk,)
    return bw, ww, aw


def _chunk_fwd(q, k, v, alpha, b, w, gates, initial_state, output_final_state, final_state, out,
               cu_seqlens, stream, segmented=True):
    import torch

    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    N = B if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    bw, ww, aw = _gate_widths(gates, dk, dv)
    for name, t, width in (("q", q, dk), ("k", k, dk), ("v", v, dv)):
        _check(name, t, (B, T, H, width), dt, dev)
    _check("b", b, (B, T, H) + bw, dt, dev)
    if ww is not None:
        _check("w", w, (B, T, H) + ww, dt, dev)
    else:
        w = None
    _check("alpha", alpha, (B, T, H) + aw, torch.float32, dev)
    if initial_state is not None:
        _check("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if cu_seqlens is not None:
        _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _check("out", out, (B, T, H, dv), dt, dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    ws_bytes = gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N if cu_seqlens is not None else 0, code)
    if not segmented:
        ws_bytes = 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(initial_state), _ptr(final_state),
            _ptr(out), _ptr(cu_seqlens), B, T, H, dk, dv, N, code)
    tail = (_ptr(ws), ws_bytes, _stream(stream))
    if gates == GATES_FULL:
        rc, name = lib.gdn2_chunk_fwd(*args, *tail), "gdn2_chunk_fwd"
    else:
        rc, name = lib.gdn2_chunk_fwd_gates(*args, gates, *tail), "gdn2_chunk_fwd_gates"
    if rc != GDN2_OK:
        raise Gdn2Error(rc, name)
    return out, final_state


def gdn2_chunk_fwd(q, k, v, alpha, b, w, initial_state=None, *, output_final_state=True,
                   final_state=None, out=None, cu_seqlens=None, stream=None, segmented=True):
    """Chunkwise GDN-2 forward.  Returns ``(o, final_state)`` (final_state may be None).

    q, k, b: [B, T, H, dk]; v, w: [B, T, H, dv] (float32 or bfloat16, all the
    same); alpha: [B, T, H, dk] float32; initial_state: [N, H, dk, dv] float32
    or None; cu_seqlens: int32 [N + 1] on the device or None (then B must be 1).
    ``final_state`` may be passed (e.g. the initial_state tensor itself for an
    in-place update); otherwise it is allocated when ``output_final_state``.
    The workspace gdn2_chunk_fwd_workspace_bytes asks for is allocated, which
    selects the segmented path for few-chain shapes; ``segmented=False``
    passes none (the single pass).
    """
    return _chunk_fwd(q, k, v, alpha, b, w, GATES_FULL, initial_state, output_final_state, final_state, out,
                      cu_seqlens, stream, segmented)


def gdn2_chunk_fwd_gates(q, k, v, alpha, b, w, gates, initial_state=None, *, output_final_state=True,
                         final_state=None, out=None, cu_seqlens=None, stream=None, segmented=True):
    """gdn2_chunk_fwd with a gate layout, an OR of the GATES_* flags:
    SCALAR_ERASE takes b as [B, T, H]; SCALAR_WRITE takes w as [B, T, H];
    TIED (with SCALAR_ERASE) uses b as the write gate too (w ignored, may be
    None); SCALAR_DECAY takes alpha as [B, T, H] float32.  GATES_FULL is
    gdn2_chunk_fwd; GATES_KDA and GATES_GDN are the two reductions."""
    return _chunk_fwd(q, k, v, alpha, b, w, gates, initial_state, output_final_state, final_state, out,
                      cu_seqlens, stream, segmented)


def _recurrent_step(q, k, v, alpha, b, w, gates, state, out, stream):
    import torch

    lib = load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    bw, ww, aw = _gate_widths(gates, dk, dv)
    for name, t, width in (("q", q, dk), ("k", k, dk), ("v", v, dv)):
        _check(name, t, (N, H, width), dt, dev)
    _check("b", b, (N, H) + bw, dt, dev)
    if ww is not None:
        _check("w", w, (N, H) + ww, dt, dev)
    else:
        w = None
    _check("alpha", alpha, (N, H) + aw, torch.float32, dev)
    _check("state", state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _check("out", out, (N, H, dv), dt, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(state), _ptr(out), N, H, dk, dv, code)
    if gates == GATES_FULL:
        rc, name = lib.gdn2_recurrent_step(*args, _stream(stream)), "gdn2_recurrent_step"
    else:
        rc, name = lib.gdn2_recurrent_step_gates(*args, gates, _stream(stream)), "gdn2_recurrent_step_gates"
    if rc != GDN2_OK:
        raise Gdn2Error(rc, name)
    return out


def gdn2_recurrent_step(q, k, v, alpha, b, w, state, *, out=None, stream=None):
    """One fused recurrent (decode) step; updates ``state`` in place, returns o.

    q, k, b: [N, H, dk]; v, w: [N, H, dv]; alpha: [N, H, dk] float32;
    state: [N, H, dk, dv] float32.
    """
    return _recurrent_step(q, k, v, alpha, b, w, GATES_FULL, state, out, stream)


def gdn2_recurrent_step_gates(q, k, v, alpha, b, w, gates, state, *, out=None, stream=None):
    """gdn2_recurrent_step with a gate layout (see gdn2_chunk_fwd_gates); a
    scalar gate is [N, H]."""
    return _recurrent_step(q, k, v, alpha, b, w, gates, state, out, stream)


def gdn2_recurrent_fwd(q, k, v, alpha, b, w, state, *, gates=GATES_FULL, out=None, stream=None):
    """The fused recurrent form over T tokens per sequence in one call; updates
    ``state`` in place and returns o.

    q, k, b: [N, T, H, dk]; v, w: [N, T, H, dv]; alpha: [N, T, H, dk] float32
    (scalar gates [N, T, H] as the ``gates`` layout says); state:
    [N, H, dk, dv] float32.
    """
    import torch

    lib = load()
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    bw, ww, aw = _gate_widths(gates, dk, dv)
    for name, t, width in (("q", q, dk), ("k", k, dk), ("v", v, dv)):
        _check(name, t, (N, T, H, width), dt, dev)
    _check("b", b, (N, T, H) + bw, dt, dev)
    if ww is not None:
        _check("w", w, (N, T, H) + ww, dt, dev)
    else:
        w = None
    _check("alpha", alpha, (N, T, H) + aw, torch.float32, dev)
    _check("state", state, (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, T, H, dv), dtype=dt, device=dev)
    else:
        _check("out", out, (N, T, H, dv), dt, dev)
    rc = lib.gdn2_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(state), _ptr(out),
                                N, T, H, dk, dv, code, gates, _stream(stream))
    if rc != GDN2_OK:
        raise Gdn2Error(rc, "gdn2_recurrent_fwd")
    return out


def gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs, dtype_code) -> int:
    return int(load().gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs, dtype_code))


def gdn2_chunk_bwd(q, k, v, alpha, b, w, d_o, initial_state=None, d_final_state=None, *, cu_seqlens=None,
                   output_d_initial_state=True, d_initial_state=None, workspace=None, stream=None):
    """Gradients of gdn2_chunk_fwd for the loss <d_o, o> + <d_final_state, S_final>.

    Inputs as for gdn2_chunk_fwd, plus d_o [B, T, H, dv] (input dtype) and
    d_final_state [N, H, dk, dv] float32 or None.  Returns a dict with dq, dk,
    db [B, T, H, dk] and dv, dw [B, T, H, dv] (input dtype), dalpha [B, T, H, dk]
    float32 and d_initial_state [N, H, dk, dv] float32 (None if not wanted).
    ``workspace`` (uint8 device tensor) is allocated when not given.
    """
    import torch

    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    N = B if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    for name, t, width in (("q", q, dk), ("k", k, dk), ("b", b, dk), ("v", v, dv), ("w", w, dv),
                           ("d_o", d_o, dv)):
        _check(name, t, (B, T, H, width), dt, dev)
    _check("alpha", alpha, (B, T, H, dk), torch.float32, dev)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check(name, t, (N, H, dk, dv), torch.float32, dev)
    if cu_seqlens is not None:
        _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    out = {name: torch.empty((B, T, H, width), dtype=dt, device=dev)
           for name, width in (("dq", dk), ("dk", dk), ("db", dk), ("dv", dv), ("dw", dv))}
    out["dalpha"] = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    if d_initial_state is not None:
        _check("d_initial_state", d_initial_state, (N, H, dk, dv), torch.float32, dev)
    elif output_d_initial_state:
        d_initial_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    out["d_initial_state"] = d_initial_state
    ws_bytes = gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N if cu_seqlens is not None else 0, code)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    elif workspace.numel() < ws_bytes:
        raise ValueError(f"workspace of {workspace.numel()} bytes < {ws_bytes}")
    rc = lib.gdn2_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(initial_state),
                            _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dalpha"]), _ptr(out["db"]), _ptr(out["dw"]), _ptr(d_initial_state),
                            _ptr(cu_seqlens), B, T, H, dk, dv, N, code, _ptr(workspace),
                            0 if workspace is None else workspace.numel(), _stream(stream))
    if rc != GDN2_OK:
        raise Gdn2Error(rc, "gdn2_chunk_bwd")
    return out


def gdn2_chunk_bwd_noalloc_max_workspace_bytes() -> int:
    return int(load().gdn2_chunk_bwd_noalloc_max_workspace_bytes())


def gdn2_chunk_bwd_noalloc(q, k, v, alpha, b, w, d_o, initial_state=None, d_final_state=None, *, out,
                           cu_seqlens=None, stream=None):
    """gdn2_chunk_bwd on the library's own workspace (the call allocates nothing).

    ``out``: dict of preallocated outputs dq, dk, db [B, T, H, dk] and dv, dw
    [B, T, H, dv] (input dtype), dalpha [B, T, H, dk] float32 and
    d_initial_state [N, H, dk, dv] float32 or None; filled in place and
    returned."""
    import torch

    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    N = B if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    for name, t, width in (("q", q, dk), ("k", k, dk), ("b", b, dk), ("v", v, dv), ("w", w, dv),
                           ("d_o", d_o, dv), ("dq", out["dq"], dk), ("dk", out["dk"], dk), ("db", out["db"], dk),
                           ("dv", out["dv"], dv), ("dw", out["dw"], dv)):
        _check(name, t, (B, T, H, width), dt, dev)
    _check("alpha", alpha, (B, T, H, dk), torch.float32, dev)
    _check("dalpha", out["dalpha"], (B, T, H, dk), torch.float32, dev)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state),
                    ("d_initial_state", out.get("d_initial_state"))):
        if t is not None:
            _check(name, t, (N, H, dk, dv), torch.float32, dev)
    if cu_seqlens is not None:
        _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    rc = lib.gdn2_chunk_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(initial_state),
                                    _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
                                    _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["db"]), _ptr(out["dw"]),
                                    _ptr(out.get("d_initial_state")), _ptr(cu_seqlens), B, T, H, dk, dv, N, code,
                                    _stream(stream))
    if rc != GDN2_OK:
        raise Gdn2Error(rc, "gdn2_chunk_bwd_noalloc")
    return out


GATE_ACTS = {"sigmoid": 0, "silu": 1}


def gdn2_mixer_prologue(xq, xk, xv, conv_q, conv_k, conv_v, b_logit, w_logit, *, conv_state=None,
                        output_conv_state=True, conv_state_out=None, cu_seqlens=None, q_scale=1.0, eps_l2=1e-6,
                        stream=None):
    """q, k, v, b, w of the recurrence from the projection outputs (one pass).

    xq, xk, b_logit: [B, T, H, dk]; xv, w_logit: [B, T, H, dv] (float32 or
    bfloat16); conv_q, conv_k: [H * dk, K], conv_v: [H * dv, K] float32;
    conv_state: [N, H * (2 dk + dv), K - 1] float32 or None (zeros).  Returns
    dict(q, k, v, b, w, conv_state) with the final convolution state (None if
    not wanted; pass conv_state_out=conv_state for an in-place decode step).
    """
    import torch

    lib = load()
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    K = conv_q.shape[-1]
    dev, dt = xq.device, xq.dtype
    code = _dtype_code(dt)
    N = B if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    for name, t, width in (("xq", xq, dk), ("xk", xk, dk), ("b_logit", b_logit, dk), ("xv", xv, dv),
                           ("w_logit", w_logit, dv)):
        _check(name, t, (B, T, H, width), dt, dev)
    for name, t, width in (("conv_q", conv_q, dk), ("conv_k", conv_k, dk), ("conv_v", conv_v, dv)):
        _check(name, t, (H * width, K), torch.float32, dev)
    st_shape = (N, H * (2 * dk + dv), K - 1)
    if conv_state is not None:
        _check("conv_state", conv_state, st_shape, torch.float32, dev)
    if conv_state_out is not None:
        _check("conv_state_out", conv_state_out, st_shape, torch.float32, dev)
    elif output_conv_state:
        conv_state_out = torch.empty(st_shape, dtype=torch.float32, device=dev)
    if cu_seqlens is not None:
        _check("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    out = {name: torch.empty((B, T, H, width), dtype=dt, device=dev)
           for name, width in (("q", dk), ("k", dk), ("b", dk), ("v", dv), ("w", dv))}
    rc = lib.gdn2_mixer_prologue(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_q), _ptr(conv_k), _ptr(conv_v),
                                 _ptr(b_logit), _ptr(w_logit), _ptr(conv_state), _ptr(conv_state_out),
                                 _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["b"]), _ptr(out["w"]),
                                 _ptr(cu_seqlens), B, T, H, dk, dv, K, N, float(q_scale), float(eps_l2), code,
                                 _stream(stream))
    if rc != GDN2_OK:
        raise Gdn2Error(rc, "gdn2_mixer_prologue")
    out["conv_state"] = conv_state_out
    return out


def gdn2_mixer_epilogue(o, gate, weight, *, eps=1e-5, act="sigmoid", out=None, stream=None):
    """RMS-normalised o times weight times act(gate), over the last axis (dv).

    o, gate: [..., dv] (float32 or bfloat16, same shape); weight: [dv] float32;
    act: "sigmoid" or "silu"."""
    import torch

    lib = load()
    dv = o.shape[-1]
    dev, dt = o.device, o.dtype
    code = _dtype_code(dt)
    _check("gate", gate, tuple(o.shape), dt, dev)
    _check("weight", weight, (dv,), torch.float32, dev)
    if not o.is_contiguous():
        raise ValueError("o: must be contiguous")
    if out is None:
        out = torch.empty_like(o)
    else:
        _check("out", out, tuple(o.shape), dt, dev)
    if act not in GATE_ACTS:
        raise ValueError(f"act must be one of {tuple(GATE_ACTS)}")
    rows = o.numel() // dv
    rc = lib.gdn2_mixer_epilogue(_ptr(o), _ptr(gate), _ptr(weight), _ptr(out), rows, dv, float(eps),
                                 GATE_ACTS[act], code, _stream(stream))
    if rc != GDN2_OK:
        raise Gdn2Error(rc, "gdn2_mixer_epilogue")
    return out
