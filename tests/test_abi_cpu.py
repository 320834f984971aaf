"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/gdn2.h declares, and rejects bad arguments synchronously,
before any HIP call (so no device is needed)."""
import ctypes
import os
import re

import pytest

from delta_rule_linear_gdn2_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")

OK, NULLP, SHAPE, UNSUP, DTYPE, MISAL, ALIAS, WS, HIP = range(9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail(f"{binding.LIB_PATH} is not built (run __graft_entry__.build())")
    return binding.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(9):
        s = binding.status_string(code)
        assert s.startswith(binding.STATUS_NAMES[code])
    assert "unknown" in binding.status_string(99)
    assert lib.gdn2_version() == 10000


def test_workspace_query(lib):
    # the segmented path: bf16, dk = 128, no packed input, few chains (plans for 256 compute units here)
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    seg = lambda B, P, H, dk, dv: al(B * P * H * dk * (dv + dk) * 4) + al(B * P * H * dk * dv * 4)  # noqa: E731
    # B=1 H=16: 64 pass-1 workgroups per segment, 4 fit, P = 5 segments of 832 tokens
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, 0, 1) == seg(1, 5, 16, 128, 128)
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 16384, 16, 128, 128, 0, 1) == seg(1, 5, 16, 128, 128)
    assert binding.gdn2_chunk_fwd_workspace_bytes(2, 4096, 16, 128, 128, 0, 1) == seg(2, 3, 16, 128, 128)
    assert binding.gdn2_chunk_fwd_workspace_bytes(8, 4096, 16, 128, 128, 0, 1) == 0    # enough chains already
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, 3, 1) == 0    # packed input
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, 0, 0) == 0    # FP32
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 4096, 16, 64, 64, 0, 1) == 0      # dk = 64
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 1000, 16, 128, 128, 0, 1) == 0    # rows under 1024 tokens
    assert binding.gdn2_chunk_fwd_workspace_bytes(1, 1024, 16, 128, 128, 0, 1) == seg(1, 4, 16, 128, 128)


# Fake, well-separated, 256-byte aligned device addresses: validation must
# reject every case below before touching them.
BASE = 1 << 40
GAP = 1 << 32


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * GAP + off)


def chunk_call(lib, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=fake(5),
                s0=fake(6), sf=fake(7), o=fake(8), cu=None,
                B=2, T=64, H=4, dk=64, dv=64, num_seqs=0, dtype=1, ws=None, ws_bytes=0)
    args.update(kw)
    a = args
    return lib.gdn2_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["s0"], a["sf"],
                              a["o"], a["cu"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                              a["num_seqs"], a["dtype"], a["ws"], a["ws_bytes"], None)


def step_call(lib, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=fake(5),
                state=fake(6), o=fake(8), N=4, H=2, dk=128, dv=128, dtype=1)
    args.update(kw)
    a = args
    return lib.gdn2_recurrent_step(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["state"],
                                   a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)


@pytest.mark.parametrize("kw,expected", [
    (dict(dtype=2), DTYPE),
    (dict(dtype=-1), DTYPE),
    (dict(B=0), SHAPE),
    (dict(T=-1), SHAPE),
    (dict(H=0), SHAPE),
    (dict(dk=0), SHAPE),
    (dict(cu=fake(9), B=2, num_seqs=3), SHAPE),
    (dict(cu=fake(9), B=1, num_seqs=0), SHAPE),
    (dict(dk=48), UNSUP),
    (dict(dv=256), UNSUP),
    (dict(dk=16), UNSUP),
    (dict(q=None), NULLP),
    (dict(alpha=None), NULLP),
    (dict(o=None), NULLP),
    (dict(q=fake(0, 8)), MISAL),
    (dict(alpha=fake(3, 4)), MISAL),
    (dict(sf=fake(7, 2)), MISAL),
    (dict(cu=fake(9, 2), B=1, num_seqs=2), MISAL),
    (dict(o=fake(0, 256)), ALIAS),                    # o inside q
    (dict(o=fake(6, 16)), ALIAS),                     # o inside the initial state
    (dict(sf=fake(3, 64)), ALIAS),                    # final state inside alpha
    (dict(sf=fake(8)), ALIAS),                        # final state == o
    (dict(sf=fake(6, 1024)), ALIAS),                  # partial overlap with initial state
    (dict(ws=fake(10, 8)), MISAL),                    # workspace not 16-byte aligned
])
def test_chunk_fwd_rejects(lib, kw, expected):
    assert chunk_call(lib, **kw) == expected


@pytest.mark.parametrize("kw,expected", [
    (dict(dtype=5), DTYPE),
    (dict(N=0), SHAPE),
    (dict(H=-2), SHAPE),
    (dict(dv=96), UNSUP),
    (dict(state=None), NULLP),
    (dict(w=None), NULLP),
    (dict(v=fake(2, 4)), MISAL),
    (dict(o=fake(6, 512)), ALIAS),                    # o inside the state
    (dict(state=fake(1, 64)), ALIAS),                 # state overlaps k
])
def test_recurrent_step_rejects(lib, kw, expected):
    assert step_call(lib, **kw) == expected


def chunk_gates_call(lib, gates, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=None,
                s0=fake(6), sf=fake(7), o=fake(8), cu=None,
                B=2, T=64, H=4, dk=64, dv=64, num_seqs=0, dtype=1, ws=None, ws_bytes=0)
    args.update(kw)
    a = args
    return lib.gdn2_chunk_fwd_gates(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["s0"], a["sf"],
                                    a["o"], a["cu"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                    a["num_seqs"], a["dtype"], gates, a["ws"], a["ws_bytes"], None)


def step_gates_call(lib, gates, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=None,
                state=fake(6), o=fake(8), N=8, H=4, dk=128, dv=128, dtype=1)
    args.update(kw)
    a = args
    return lib.gdn2_recurrent_step_gates(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["state"],
                                         a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], gates, None)


# 2 x 64 x 4 = 512 (token, head) rows: a scalar gate takes 1024 bytes in
# bf16, a scalar alpha 2048 bytes.  Every case must be rejected before launch.
@pytest.mark.parametrize("gates,kw,expected", [
    (16, {}, SHAPE),                                  # an unknown flag
    (-1, {}, SHAPE),
    (4, {}, SHAPE),                                   # tied without a scalar erase gate
    (7, {}, SHAPE),                                   # tied and a scalar write gate
    (0, {}, NULLP),                                   # the full layout needs w
    (1, {}, NULLP),                                   # an untied layout needs w
    (5, dict(b=None), NULLP),
    (13, dict(alpha=None), NULLP),
    (5, dict(b=fake(4, 2)), MISAL),
    (2, dict(w=fake(5, 8)), MISAL),
    (5, dict(o=fake(4, 512)), ALIAS),                 # o inside the compact beta
    (13, dict(o=fake(3, 1024)), ALIAS),               # o inside the compact alpha
    (13, dict(sf=fake(4, 992)), ALIAS),               # final state over the end of beta
    (3, dict(w=fake(5), o=fake(5, 512)), ALIAS),      # o inside the compact write gate
    (5, dict(dk=96), UNSUP),
    (5, dict(dtype=3), DTYPE),
])
def test_chunk_fwd_gates_rejects(lib, gates, kw, expected):
    assert chunk_gates_call(lib, gates, **kw) == expected


# 8 x 4 = 32 (sequence, head) rows: a scalar gate takes 64 bytes in bf16, a
# scalar alpha 128 bytes.
@pytest.mark.parametrize("gates,kw,expected", [
    (16, {}, SHAPE),
    (6, {}, SHAPE),                                   # tied and a scalar write gate, no scalar erase
    (0, {}, NULLP),
    (13, dict(b=None), NULLP),
    (13, dict(alpha=fake(3, 8)), MISAL),
    (5, dict(o=fake(4, 32)), ALIAS),                  # o inside beta
    (13, dict(state=fake(3, 96)), ALIAS),             # state over the compact alpha
    (10, dict(w=fake(5), o=fake(5, 32)), ALIAS),      # o inside the compact write gate
])
def test_recurrent_step_gates_rejects(lib, gates, kw, expected):
    assert step_gates_call(lib, gates, **kw) == expected


def recurrent_fwd_call(lib, gates=0, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=fake(5),
                state=fake(6), o=fake(8), N=4, T=8, H=2, dk=128, dv=128, dtype=1)
    args.update(kw)
    a = args
    return lib.gdn2_recurrent_fwd(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["state"], a["o"],
                                  a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dtype"], gates, None)


# 4 x 8 x 2 = 64 (token, head) rows.  Every case must be rejected before launch;
# T = 0 succeeds without launching.
@pytest.mark.parametrize("gates,kw,expected", [
    (0, dict(T=0), OK),
    (0, dict(T=-1), SHAPE),
    (0, dict(N=0), SHAPE),
    (12, {}, SHAPE),
    (0, dict(dtype=2), DTYPE),
    (0, dict(dk=256), UNSUP),
    (0, dict(w=None), NULLP),
    (0, dict(state=None, T=0), NULLP),
    (0, dict(o=fake(1, 16)), ALIAS),                  # o inside k
    (0, dict(state=fake(8, 4096)), ALIAS),            # state over o ([4, 8, 2, 128] bf16 = 16 KiB)
    (0, dict(o=fake(0, 12288)), ALIAS),               # o over the end of q (16 KiB; o starts in its last quarter)
    (5, dict(w=None, o=fake(4, 96)), ALIAS),          # o inside the compact beta (128 bytes)
    (0, dict(alpha=fake(3, 4)), MISAL),
])
def test_recurrent_fwd_rejects(lib, gates, kw, expected):
    assert recurrent_fwd_call(lib, gates, **kw) == expected


def bwd_call(lib, **kw):
    # B=2, T=64, H=4, dk=dv=64 bf16: token tensors 64 KiB, states 128 KiB
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=fake(5), s0=fake(6),
                d_o=fake(7), dsf=fake(8), dq=fake(9), dk=fake(10), dv=fake(11), dalpha=fake(12),
                db=fake(13), dw=fake(14), ds0=fake(15), cu=None, B=2, T=64, H=4, dk_=64, dv_=64,
                num_seqs=0, dtype=1, ws=fake(16), ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return lib.gdn2_chunk_bwd(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["s0"], a["d_o"], a["dsf"],
                              a["dq"], a["dk"], a["dv"], a["dalpha"], a["db"], a["dw"], a["ds0"], a["cu"],
                              a["B"], a["T"], a["H"], a["dk_"], a["dv_"], a["num_seqs"], a["dtype"],
                              a["ws"], a["ws_bytes"], None)


def _bwd_ws(B, T, H, dk, dv, slots):
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    prep = 2 * 32 * 32 + 3 * 32 * dk + dk  # Tm, Pm, Et, Qt, Kb, 2^G_L per chunk
    return (2 * al(B * slots * H * dk * dv * 4) + 2 * al(B * T * H * dv * 4) + al(B * slots * H * prep * 4))


def _bwd_ws_mfma(B, T, H, slots, slots64):
    # the range flag, then the larger of the FP32 path's regions and the
    # matrix-core path's bf16 states, state gradients, U and dX rows per 64-token slot
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    own = 2 * al(B * slots64 * H * 128 * 128 * 2) + 2 * al(B * slots64 * H * 64 * 128 * 2)
    return 256 + max(_bwd_ws(B, T, H, 128, 128, slots), own)


def test_bwd_workspace_query(lib):
    # states and state gradients per chunk slot, U and dX rows, prepared chunk algebra
    assert binding.gdn2_chunk_bwd_workspace_bytes(8, 4096, 16, 128, 128, 0, 0) == _bwd_ws(8, 4096, 16, 128, 128, 128)
    assert binding.gdn2_chunk_bwd_workspace_bytes(8, 4096, 16, 128, 128, 0, 1) == _bwd_ws_mfma(8, 4096, 16, 128, 64)
    assert binding.gdn2_chunk_bwd_workspace_bytes(1, 300, 2, 128, 128, 3, 1) == _bwd_ws_mfma(1, 300, 2, 10 + 3, 5 + 3)
    assert binding.gdn2_chunk_bwd_workspace_bytes(1, 300, 2, 128, 64, 3, 1) == _bwd_ws(1, 300, 2, 128, 64, 10 + 3)
    assert binding.gdn2_chunk_bwd_workspace_bytes(1, 0, 4, 64, 64, 3, 1) == 0
    assert binding.gdn2_chunk_bwd_workspace_bytes(1, 100, 2, 32, 32, 3, 0) == _bwd_ws(1, 100, 2, 32, 32, 4 + 3)
    assert binding.gdn2_chunk_bwd_workspace_bytes(0, 100, 2, 32, 32, 0, 0) == 0


# Every case must be rejected before launch.
@pytest.mark.parametrize("kw,expected", [
    (dict(dtype=2), DTYPE),
    (dict(B=0), SHAPE),
    (dict(T=-3), SHAPE),
    (dict(cu=fake(17), B=2, num_seqs=2), SHAPE),
    (dict(dk_=48), UNSUP),
    (dict(d_o=None), NULLP),
    (dict(dalpha=None), NULLP),
    (dict(w=None), NULLP),
    (dict(dalpha=fake(12, 4)), MISAL),
    (dict(ws=fake(16, 8)), MISAL),
    (dict(ws=None), WS),
    (dict(ws_bytes=4096), WS),
    (dict(dq=fake(0, 1024)), ALIAS),                  # dq inside q
    (dict(dk=fake(9, 512)), ALIAS),                   # dk inside dq
    (dict(ws=fake(1)), ALIAS),                        # workspace over k
    (dict(ds0=fake(6)), ALIAS),                       # d_initial_state == initial_state
    (dict(dalpha=fake(7, 2048)), ALIAS),              # dalpha inside d_o
    (dict(ds0=fake(8, 1024)), ALIAS),                 # partial overlap with d_final_state
])
def test_chunk_bwd_rejects(lib, kw, expected):
    assert bwd_call(lib, **kw) == expected


def bwd_noalloc_call(lib, **kw):
    # as bwd_call, without the workspace arguments
    args = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), b=fake(4), w=fake(5), s0=fake(6),
                d_o=fake(7), dsf=fake(8), dq=fake(9), dk=fake(10), dv=fake(11), dalpha=fake(12),
                db=fake(13), dw=fake(14), ds0=fake(15), cu=None, B=2, T=64, H=4, dk_=64, dv_=64,
                num_seqs=0, dtype=1)
    args.update(kw)
    a = args
    return lib.gdn2_chunk_bwd_noalloc(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], a["s0"], a["d_o"],
                                      a["dsf"], a["dq"], a["dk"], a["dv"], a["dalpha"], a["db"], a["dw"], a["ds0"],
                                      a["cu"], a["B"], a["T"], a["H"], a["dk_"], a["dv_"], a["num_seqs"],
                                      a["dtype"], None)


def test_bwd_noalloc_capacity(lib):
    assert binding.gdn2_chunk_bwd_noalloc_max_workspace_bytes() == 256 << 20
    # the documented examples: B=1 T=2048 H=16 d=128 fits, the B=8 T=4096 training shape does not
    assert binding.gdn2_chunk_bwd_workspace_bytes(1, 2048, 16, 128, 128, 0, 1) <= 256 << 20
    assert binding.gdn2_chunk_bwd_workspace_bytes(8, 4096, 16, 128, 128, 0, 1) > 256 << 20


# Every case must be rejected on the host, before the library's array is looked up.
@pytest.mark.parametrize("kw,expected", [
    (dict(dtype=2), DTYPE),
    (dict(B=0), SHAPE),
    (dict(dk_=48), UNSUP),
    (dict(d_o=None), NULLP),
    (dict(dalpha=fake(12, 4)), MISAL),
    (dict(dq=fake(0, 1024)), ALIAS),                  # dq inside q
    (dict(ds0=fake(6)), ALIAS),                       # d_initial_state == initial_state
    (dict(B=8, T=4096, H=16, dk_=128, dv_=128), WS),  # workspace of 3.4 GB > 256 MiB
    (dict(B=1, T=4096, H=16, dk_=128, dv_=128), WS),  # 335 MB > 256 MiB
])
def test_chunk_bwd_noalloc_rejects(lib, kw, expected):
    assert bwd_noalloc_call(lib, **kw) == expected


def pro_call(lib, **kw):
    # B=2, T=64, H=4, dk=dv=64, K=4 bf16: token tensors 64 KiB; filters 4 KiB; state 2 x 768 x 3 x 4 B
    args = dict(xq=fake(0), xk=fake(1), xv=fake(2), cq=fake(3), ck=fake(4), cv=fake(5), bl=fake(6), wl=fake(7),
                si=fake(8), so=fake(9), q=fake(10), k=fake(11), v=fake(12), b=fake(13), w=fake(14), cu=None,
                B=2, T=64, H=4, dk_=64, dv_=64, K=4, num_seqs=0, scale=1.0, eps=1e-6, dtype=1)
    args.update(kw)
    a = args
    return lib.gdn2_mixer_prologue(a["xq"], a["xk"], a["xv"], a["cq"], a["ck"], a["cv"], a["bl"], a["wl"],
                                   a["si"], a["so"], a["q"], a["k"], a["v"], a["b"], a["w"], a["cu"], a["B"],
                                   a["T"], a["H"], a["dk_"], a["dv_"], a["K"], a["num_seqs"], a["scale"], a["eps"],
                                   a["dtype"], None)


# Every case must be rejected before launch.
@pytest.mark.parametrize("kw,expected", [
    (dict(dtype=7), DTYPE),
    (dict(K=0), SHAPE),
    (dict(K=17), SHAPE),
    (dict(eps=-1.0), SHAPE),
    (dict(T=-1), SHAPE),
    (dict(dk_=96), UNSUP),
    (dict(cq=None), NULLP),
    (dict(w=None), NULLP),
    (dict(xv=fake(2, 8)), MISAL),
    (dict(q=fake(0, 512)), ALIAS),                    # q inside xq
    (dict(k=fake(10, 4096)), ALIAS),                  # k inside q
    (dict(so=fake(8)), ALIAS),                        # in-place state with T > 1
    (dict(so=fake(8), T=1, cu=fake(15), B=1, num_seqs=2), ALIAS),  # in place with packed sequences
    (dict(v=fake(3, 1024)), ALIAS),                   # v over the q filters
])
def test_mixer_prologue_rejects(lib, kw, expected):
    assert pro_call(lib, **kw) == expected


@pytest.mark.parametrize("kw,expected", [
    (dict(dtype=3), DTYPE),
    (dict(act=2), SHAPE),
    (dict(eps=0.0), SHAPE),
    (dict(rows=-1), SHAPE),
    (dict(dv_=80), UNSUP),
    (dict(gate=None), NULLP),
    (dict(weight=fake(2, 4)), MISAL),
    (dict(y=fake(0, 256)), ALIAS),                    # y inside o
    (dict(y=fake(2)), ALIAS),                         # y over the weight
])
def test_mixer_epilogue_rejects(lib, kw, expected):
    args = dict(o=fake(0), gate=fake(1), weight=fake(2), y=fake(3), rows=100, dv_=64, eps=1e-5, act=0, dtype=1)
    args.update(kw)
    a = args
    assert lib.gdn2_mixer_epilogue(a["o"], a["gate"], a["weight"], a["y"], a["rows"], a["dv_"], a["eps"], a["act"],
                                   a["dtype"], None) == expected
