"""Seeded synthetic inputs for the calibration-Hessian workloads.

This module only draws inputs: activations, batch sizes, dead columns,
expert routing.  It holds none of the Hessian arithmetic and is shared by the
tests, the bench and the smoke check, which hand the same arrays to the
library and to the float64 oracle.

Recipe (the pages measure on real-model activations from calibration text;
these synthetic inputs stand in for them):
* column scales ``s_j = exp(0.5 g_j)``, g ~ N(0, 1) (lognormal(0, 0.5));
* activations ``X[t, j] = z * s_j``, z ~ N(0, 1), drawn in float32;
* bf16 inputs are the float32 values rounded to nearest-even bf16;
* ragged batch sizes are uniform integers in [1, 2000];
* a chosen set of columns is zeroed to exercise dead-column neutralization;
* routed-expert inputs: each token picks 8 distinct experts of 64 with
  popularity proportional to (e + 1)^-1.1 (Gumbel top-k).

Two backends draw the same recipe: ``numpy`` (PCG64, used by tests, exact
values reproducible on any host) and ``torch`` (the device's own seeded
generator, used for the multi-gigabyte bench buffers).  Their values differ;
each side of a comparison always receives the same arrays.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"
F16 = "f16"


# ----------------------------------------------------------------------------
# numpy backend
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bf16; return the uint16 bit patterns.

    NaN inputs map to a quiet NaN pattern.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        b = flat_in[s:s + step]
        r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        r = np.where(nan, np.uint32(0x7FC0), r)
        flat_out[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def column_scales(rng: np.random.Generator, d: int) -> np.ndarray:
    """Per-column scales, lognormal(0, 0.5), float32."""
    return np.exp(0.5 * rng.standard_normal(d)).astype(np.float32)


def normal_rows(rng: np.random.Generator, n: int, d: int, scales=None) -> np.ndarray:
    """(n, d) float32 N(0, 1) activations, optionally times per-column scales."""
    x = rng.standard_normal((n, d), dtype=np.float32)
    if scales is not None:
        x *= scales[None, :]
    return x


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 activations in the requested storage format (bf16 -> uint16 bits, f16 -> numpy float16)."""
    if dtype == BF16:
        return to_bf16_bits(x)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    raise ValueError(dtype)


@dataclass
class Workload:
    """A Hessian's worth of calibration batches (host arrays)."""
    d: int
    dtype: str
    batches: list
    dead_cols: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))
    scales: np.ndarray | None = None

    @property
    def total_tokens(self) -> int:
        return int(sum(b.shape[0] for b in self.batches))


def tiny_case() -> Workload:
    """d=256, three batches of 100, 37 and 0 tokens, N(0,1) float32, seed 0."""
    rng = np.random.default_rng(0)
    batches = [normal_rows(rng, n, 256) for n in (100, 37, 0)]
    return Workload(d=256, dtype=F32, batches=batches)


def ragged_sizes(rng: np.random.Generator, count: int, lo: int = 1, hi: int = 2000) -> np.ndarray:
    """``count`` batch sizes uniform in [lo, hi]."""
    return rng.integers(lo, hi + 1, size=count)


def dead_columns(rng: np.random.Generator, d: int, frac: float) -> np.ndarray:
    """round(frac * d) distinct column indices, sorted."""
    k = int(round(frac * d))
    return np.sort(rng.choice(d, size=k, replace=False)) if k > 0 else np.zeros(0, dtype=np.int64)


def ragged_case(d: int, sizes, seed: int, dtype: str = BF16, dead_frac: float = 0.0) -> Workload:
    """Batches of the given sizes with lognormal column scales (numpy backend)."""
    rng = np.random.default_rng(seed)
    scales = column_scales(rng, d)
    dead = dead_columns(rng, d, dead_frac)
    if dead.size:
        scales = scales.copy()
        scales[dead] = 0.0
    batches = []
    for n in sizes:
        x = normal_rows(rng, int(n), d, scales)
        batches.append(encode(x, dtype))
    return Workload(d=d, dtype=dtype, batches=batches, dead_cols=dead, scales=scales)


def moe_routing(rng: np.random.Generator, tokens: int, experts: int = 64, topk: int = 8,
                zipf: float = 1.1):
    """Route each token to ``topk`` distinct experts (Gumbel top-k on log popularity).

    Returns ``(row_idx, offsets)``: row_idx (int32) lists token ids grouped by
    expert, ascending within each expert; offsets (int64, experts + 1) bounds
    each expert's slice.
    """
    logp = -zipf * np.log(np.arange(1, experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(tokens, experts))
    choice = np.argpartition(-(logp[None, :] + g), topk - 1, axis=1)[:, :topk]
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))
    row_idx = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return row_idx, offsets


# ----------------------------------------------------------------------------
# torch backend (device-side generation of large bench buffers)
# ----------------------------------------------------------------------------

def torch_generator(seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def torch_column_scales(gen, d: int, device):
    import torch
    return torch.exp(0.5 * torch.randn(d, generator=gen, device=device, dtype=torch.float32))


def torch_rows(gen, n: int, d: int, scales, dtype: str, device, out=None):
    """(n, d) activations N(0,1)*scales drawn on ``device``; bf16, fp16 or float32."""
    import torch
    x = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
    x.mul_(scales[None, :])
    if dtype == BF16:
        x = x.to(torch.bfloat16)
    elif dtype == F16:
        x = x.to(torch.float16)
    if out is not None:
        out.copy_(x)
        return out
    return x


def torch_ragged(d: int, seed: int, dtype: str = BF16, count: int = 360, dead_frac: float = 0.0,
                 device="cuda"):
    """A ragged calibration Hessian's batches, resident on ``device``.

    Batch sizes are uniform integers in [1, 2000] and the dead columns are
    chosen with numpy PCG64 (seed ``seed``, in that order); column scales and
    activations come from the device generator seeded the same.  The batches
    are views into one buffer, back to back.  For one seed, the float32
    values are the same whatever ``dtype`` is; bf16 and fp16 round them.
    Returns ``(buf, views, sizes, dead)``.
    """
    import torch
    rng = np.random.default_rng(seed)
    sizes = ragged_sizes(rng, count)
    dead = dead_columns(rng, d, dead_frac)
    gen = torch_generator(seed, device)
    scales = torch_column_scales(gen, d, device)
    if dead.size:
        scales[torch.from_numpy(dead).to(device)] = 0.0
    buf = torch_rows(gen, int(sizes.sum()), d, scales, dtype, device)
    views, off = [], 0
    for n in sizes:
        views.append(buf[off:off + int(n)])
        off += int(n)
    return buf, views, sizes, dead


def torch_single(d: int, n: int, seed: int, dtype: str = BF16, dead_frac: float = 0.0, device="cuda"):
    """One batch of ``n`` tokens on ``device``, same recipe as ``torch_ragged``.

    Returns ``(x, dead)``.
    """
    import torch
    rng = np.random.default_rng(seed)
    dead = dead_columns(rng, d, dead_frac)
    gen = torch_generator(seed, device)
    scales = torch_column_scales(gen, d, device)
    if dead.size:
        scales[torch.from_numpy(dead).to(device)] = 0.0
    return torch_rows(gen, n, d, scales, dtype, device), dead


def host_copy(x, dtype: str) -> np.ndarray:
    """Host array of a device batch in the storage format the oracle reads
    (bf16 as uint16 bit patterns, fp16 as numpy float16, float32 as is)."""
    import torch
    if dtype == BF16:
        return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return x.contiguous().cpu().numpy()
