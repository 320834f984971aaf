"""Seeded synthetic inputs for the Gated DeltaNet-2 forward pass.

This module only draws random numbers and rounds them to the device dtype; it
holds none of the method's arithmetic, and both the HIP path and the FP64
oracle consume its output.  Everything is generated on the CPU with numpy's
PCG64 (``numpy.random.default_rng(seed)``), so inputs do not depend on the
device.

Value distributions follow the setting of the pages: 16 heads with a 128 x 128
state per head, 4K training length and 64-token chunks ("Gated DeltaNet-2"
analysis at iplexlaw.co.kr, "What was compared" and "Token processing and
parallel training"); gates are sigmoid outputs, q and k are L2-normalised per
head and token (same page, "Token processing and parallel training"), and the
decay sits close to one.  The pages train on FineWeb-Edu; no dataset is used
here: Gaussian / sigmoid tensors of the same shapes stand in for the
activations.

Recipes (seed = 1000 + workload index; see ``make`` for how it is split):
  q, k  ~ N(0, 1), then L2-normalised over dk per (token, head)
  v     ~ N(0, 1)
  alpha = sigmoid(N(3, 1)) per key channel           (FP32 always)
  b, w  = sigmoid(N(0, 1)) per key / value channel
  initial state ~ N(0, 0.1^2) where the workload has one, else zeros
  bf16 workloads round q, k, v, b, w to bfloat16 (round-to-nearest-even)
  once, at generation: the oracle receives the same rounded values in FP32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GEN_NAME = "numpy.random.PCG64"


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    kind: str          # "chunk" | "decode" | "varlen"
    dtype: str         # "f32" | "bf16"  (q, k, v, b, w, o); alpha and state are FP32
    B: int = 1
    T: int = 0
    H: int = 16
    dk: int = 128
    dv: int = 128
    init_state: bool = False
    steps: int = 0               # decode: consecutive in-place steps
    num_seqs: int = 0            # varlen
    min_len: int = 0
    max_len: int = 0
    gate_modes: tuple = field(default_factory=tuple)

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 0, "chunk", "f32", B=1, T=256, H=2, dk=32, dv=32),
    "layer_bf16": Workload("layer_bf16", 1, "chunk", "bf16", B=1, T=4096, H=16),
    "batched_bf16": Workload("batched_bf16", 2, "chunk", "bf16", B=8, T=4096, H=16, init_state=True),
    "decode_b256": Workload("decode_b256", 3, "decode", "bf16", B=256, H=16, init_state=True, steps=64),
    "varlen32_bf16": Workload("varlen32_bf16", 4, "varlen", "bf16", B=1, H=16, init_state=True,
                              num_seqs=32, min_len=256, max_len=8192,
                              gate_modes=("gdn2", "kda", "gdn")),
    # one long row: the 16K x 1 end of the pages' training sweep (16 heads,
    # 128 x 128 state); chunkwise, N(0, 0.1^2) initial state
    "long16k_bf16": Workload("long16k_bf16", 5, "chunk", "bf16", B=1, T=16384, H=16, init_state=True),
}


# ---------------------------------------------------------------------------
# dtype helpers


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32 (exact)."""
    return bf16_to_f32(bf16_bits(x))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    """float32 sigmoid, in place on ``x``."""
    np.negative(x, out=x)
    np.exp(x, out=x)
    x += np.float32(1.0)
    np.reciprocal(x, out=x)
    return x


def _l2norm(x: np.ndarray) -> np.ndarray:
    """float32 L2 normalisation over the last axis, in place on ``x``."""
    n = np.sqrt(np.einsum("...c,...c->...", x, x))[..., None]
    np.maximum(n, np.float32(1e-12), out=n)
    x /= n
    return x


def _normal(rng, shape, mean=0.0, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


# ---------------------------------------------------------------------------
# generators


TOKEN_BLOCK = 2048  # tokens per independently seeded generation block


def _token_block(seed_seq, ntok: int, H: int, dk: int, dv: int, dtype: str, gate_mode: str,
                 alpha_mean: float, alpha_std: float) -> dict:
    rng = np.random.default_rng(seed_seq)
    lead = (ntok,)
    q = _l2norm(_normal(rng, lead + (H, dk)))
    k = _l2norm(_normal(rng, lead + (H, dk)))
    v = _normal(rng, lead + (H, dv))
    if gate_mode == "gdn2":
        alpha = _sigmoid(_normal(rng, lead + (H, dk), alpha_mean, alpha_std))
        b = _sigmoid(_normal(rng, lead + (H, dk)))
        w = _sigmoid(_normal(rng, lead + (H, dv)))
    elif gate_mode in ("kda", "gdn"):
        if gate_mode == "kda":
            alpha = _sigmoid(_normal(rng, lead + (H, dk), alpha_mean, alpha_std))
        else:
            alpha = np.broadcast_to(_sigmoid(_normal(rng, lead + (H, 1), alpha_mean, alpha_std)),
                                    lead + (H, dk))
        beta = _sigmoid(_normal(rng, lead + (H, 1)))
        if dtype == "bf16":
            beta = round_bf16(beta)
        b = np.broadcast_to(beta, lead + (H, dk))
        w = np.broadcast_to(beta, lead + (H, dv))
    else:
        raise ValueError(gate_mode)
    out = dict(q=q, k=k, v=v, alpha=alpha, b=b, w=w)
    if dtype == "bf16":
        for name in ("q", "k", "v", "b", "w"):
            out[name] = round_bf16(out[name])
    return out


def token_tensors(seed_seq, lead: tuple, H: int, dk: int, dv: int, dtype: str,
                  gate_mode: str = "gdn2", alpha_mean: float = 3.0, alpha_std: float = 1.0,
                  workers: int | None = None) -> dict:
    """q, k, v, alpha, b, w with leading shape ``lead`` (e.g. (B, T)).

    Returned arrays are float32 holding values exactly representable in
    ``dtype``.  The flattened token axis is cut into blocks of TOKEN_BLOCK
    tokens, each drawn from its own child of ``seed_seq`` (so the values do not
    depend on the number of worker threads).  ``gate_mode``:
      "gdn2" - channel-wise alpha, b, w (full method)
      "kda"  - b = w = beta broadcast, beta = sigmoid(N(0,1)) per (token, head)
      "gdn"  - as "kda" and a scalar alpha per (token, head) broadcast over dk
    """
    ntok = int(np.prod(lead)) if lead else 1
    widths = dict(q=dk, k=dk, v=dv, alpha=dk, b=dk, w=dv)
    out = {n: np.empty((ntok, H, d), dtype=np.float32) for n, d in widths.items()}
    nblocks = max(1, -(-ntok // TOKEN_BLOCK))
    children = seed_seq.spawn(nblocks)

    def fill(i):
        lo = i * TOKEN_BLOCK
        hi = min(ntok, lo + TOKEN_BLOCK)
        blk = _token_block(children[i], hi - lo, H, dk, dv, dtype, gate_mode, alpha_mean, alpha_std)
        for n in widths:
            out[n][lo:hi] = blk[n]

    workers = workers or min(16, os.cpu_count() or 1)
    if nblocks == 1 or workers == 1:
        for i in range(nblocks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(nblocks)))
    return {n: a.reshape(tuple(lead) + (H, widths[n])) for n, a in out.items()}


def initial_state(rng, N: int, H: int, dk: int, dv: int, std: float = 0.1) -> np.ndarray:
    return _normal(rng, (N, H, dk, dv), 0.0, std)


def varlen_lengths(rng, num_seqs: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=num_seqs).astype(np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def make(name: str, gate_mode: str = "gdn2", seed: int | None = None, **overrides) -> dict:
    """Generate the inputs of a named workload.

    Returns a dict with the workload, the tensors (float32, values exact in the
    workload dtype), ``initial_state`` (or None) and, for varlen, ``cu_seqlens``.
    ``overrides`` replace shape fields (e.g. T=300 for a reduced-size case).
    Seeding: SeedSequence(seed) spawns three children, for the varlen lengths,
    the token tensors and the initial state, in that order.
    """
    wl = WORKLOADS[name]
    if overrides:
        wl = Workload(**{**wl.__dict__, **overrides})
    ss_len, ss_tok, ss_state = np.random.SeedSequence(wl.seed if seed is None else seed).spawn(3)
    out: dict = {"workload": wl, "gate_mode": gate_mode, "generator": GEN_NAME,
                 "numpy": np.__version__}
    state_rng = np.random.default_rng(ss_state)
    if wl.kind == "chunk":
        out.update(token_tensors(ss_tok, (wl.B, wl.T), wl.H, wl.dk, wl.dv, wl.dtype, gate_mode))
        out["initial_state"] = (initial_state(state_rng, wl.B, wl.H, wl.dk, wl.dv)
                                if wl.init_state else None)
        out["cu_seqlens"] = None
    elif wl.kind == "varlen":
        lengths = varlen_lengths(np.random.default_rng(ss_len), wl.num_seqs, wl.min_len, wl.max_len)
        cu = cu_from_lengths(lengths)
        total = int(cu[-1])
        out.update(token_tensors(ss_tok, (1, total), wl.H, wl.dk, wl.dv, wl.dtype, gate_mode))
        out["initial_state"] = (initial_state(state_rng, wl.num_seqs, wl.H, wl.dk, wl.dv)
                                if wl.init_state else None)
        out["cu_seqlens"] = cu
    elif wl.kind == "decode":
        # `steps` pre-generated token slices [steps, N, H, d]; state [N, H, dk, dv]
        out.update(token_tensors(ss_tok, (wl.steps, wl.B), wl.H, wl.dk, wl.dv, wl.dtype, gate_mode))
        out["initial_state"] = initial_state(state_rng, wl.B, wl.H, wl.dk, wl.dv)
        out["cu_seqlens"] = None
    else:
        raise ValueError(wl.kind)
    return out


def device_token_tensors(lead: tuple, H: int, dk: int, dv: int, dtype: str, seed: int, device="cuda",
                         tokens_per_draw: int = 65536) -> dict:
    """q, k, v, alpha, b, w of leading shape ``lead`` drawn on ``device``.

    For sizes too large to draw on the host (tens of GB): torch's seeded
    generator on the device, with the distributions of ``token_tensors`` (the
    values differ from it).  Tests that use it overwrite the chains they check
    with host inputs from ``token_tensors``, so every value the oracle sees
    comes from the host recipe.  q, k, v, b, w are rounded to ``dtype``; alpha
    is FP32.  Drawn ``tokens_per_draw`` tokens at a time (bounded scratch).
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    widths = dict(q=dk, k=dk, v=dv, alpha=dk, b=dk, w=dv)
    ntok = int(np.prod(lead)) if lead else 1
    out = {n: torch.empty((ntok, H, d), dtype=torch.float32 if n == "alpha" else tdt, device=device)
           for n, d in widths.items()}
    for t0 in range(0, ntok, tokens_per_draw):
        t1 = min(ntok, t0 + tokens_per_draw)
        for n, d in widths.items():
            x = torch.randn((t1 - t0, H, d), generator=g, device=device)
            if n in ("q", "k"):
                x /= x.norm(dim=-1, keepdim=True).clamp_min(1e-12)
            elif n == "alpha":
                x = torch.sigmoid(x + 3.0)
            elif n in ("b", "w"):
                x = torch.sigmoid(x)
            out[n][t0:t1] = x
            del x
    return {n: t.view(tuple(lead) + (H, widths[n])) for n, t in out.items()}


def to_torch(arr: np.ndarray, dtype: str, device="cpu"):
    """float32 numpy array (values exact in ``dtype``) -> torch tensor on ``device``."""
    import torch

    if dtype == "bf16":
        bits = bf16_bits(arr).view(np.int16)
        t = torch.from_numpy(bits).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to(device)
