"""Bit-exact pin of the bf16 output rounding (round to nearest, ties to even)
of the decode step and of the chunkwise kernel (needs an MI355X).

With k = 0, v = 0, alpha = 1 and q = e_0 (the first unit vector), the
recurrence leaves the state unchanged and reads its first row:
o_t = S[0, :].  Every product that enters o is then an exact product by 1 or
0, so o is the state's first row rounded once to bf16: the test writes chosen
FP32 bit patterns there (random values of every exponent, ties, values that
round up into the next binade or to infinity) and compares the output bits
with torch's CPU bf16 conversion of the same values."""
import numpy as np
import pytest

import gpu_util as G
from delta_rule_linear_gdn2_amd import binding

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


def _patterns(seed, n, decode):
    """n FP32 bit patterns: finite, nonzero magnitudes of every exponent; a
    quarter exact ties (low half 0x8000); a few values at the top of the range.
    decode: subnormals and values that round to infinity included; chunk
    (the state passes through bf16 matrix-core operands): normal values that
    stay finite in bf16."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    e = (u >> np.uint32(23)) & np.uint32(0xFF)
    lo, hi = (0, 254) if decode else (1, 253)
    e = np.clip(e, lo, hi).astype(np.uint32)
    u = (u & np.uint32(0x807FFFFF)) | (e << np.uint32(23))
    tie = rng.random(n) < 0.25
    u[tie] = (u[tie] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    top = [0x7F7F8000, 0x7F7FFFFF, 0xFF7F8000, 0x7F7F7FFF] if decode else [0x7F7F7FFF, 0xFF7F7FFF, 0x3F808000]
    u[:len(top)] = np.array(top, dtype=np.uint32)
    u[len(top):len(top) + 2] = np.array([0x3F818000, 0x3F808000], dtype=np.uint32)  # ties to the odd / even side
    u[(u & np.uint32(0x7FFFFFFF)) == 0] = 0x3F800000  # no zeros: -0 comes back as +0 (added to a +0 partial sum)
    return u


def _expected_bits(u):
    import torch

    x = torch.from_numpy(u.view(np.float32).copy())
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _inputs(shape_tok, dv):
    """q = e_0, k = v = b = w = 0, alpha = 1 (bf16 inputs, FP32 alpha)."""
    import torch

    q = torch.zeros(shape_tok + (D,), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = 1.0
    z = torch.zeros(shape_tok + (D,), dtype=torch.bfloat16, device="cuda")
    zv = torch.zeros(shape_tok + (dv,), dtype=torch.bfloat16, device="cuda")
    alpha = torch.ones(shape_tok + (D,), dtype=torch.float32, device="cuda")
    return q, z, zv, alpha


@pytest.mark.parametrize("seed", [1, 2])
def test_decode_output_rounding_bit_exact(seed):
    import torch

    N, H = 64, 16
    u = _patterns(500 + seed, N * H * D, decode=True)
    state = torch.zeros((N, H, D, D), dtype=torch.float32, device="cuda")
    state[:, :, 0, :] = torch.from_numpy(u.view(np.float32).reshape(N, H, D).copy()).cuda()
    before = state.clone()
    q, z, zv, alpha = _inputs((N, H), D)
    o = binding.gdn2_recurrent_step(q, z, zv, alpha, z, zv, state)
    torch.cuda.synchronize()
    got = o.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    exp = _expected_bits(u)
    bad = np.flatnonzero(got != exp)
    G.log(f"decode rounding: {bad.size} of {u.size} patterns differ")
    assert bad.size == 0, f"first: input 0x{u[bad[0]]:08x} -> 0x{got[bad[0]]:04x}, expected 0x{exp[bad[0]]:04x}"
    assert torch.equal(state, before), "the state must be unchanged (k = 0, alpha = 1)"


def test_chunk_output_rounding_bit_exact():
    import torch

    B, T, H = 4, 70, 16  # one full chunk and a partial one
    u = _patterns(510, B * H * D, decode=False)
    s0 = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    s0[:, :, 0, :] = torch.from_numpy(u.view(np.float32).reshape(B, H, D).copy()).cuda()
    q, z, zv, alpha = _inputs((B, T, H), D)
    o, sf = binding.gdn2_chunk_fwd(q, z, zv, alpha, z, zv, s0)
    torch.cuda.synchronize()
    got = o.cpu().view(torch.int16).numpy().view(np.uint16)  # [B, T, H, D]
    exp = _expected_bits(u).reshape(B, 1, H, D)
    bad = np.argwhere(got != exp)
    G.log(f"chunk rounding: {len(bad)} of {got.size} outputs differ")
    assert len(bad) == 0, f"first mismatch at {tuple(bad[0])}"
    assert torch.equal(sf, s0), "the state must be unchanged (k = 0, alpha = 1)"
