"""Seeded generators for the five top-k workloads and for the edge-case rows.

Every array returned here holds raw element bits in row-major
``[batch, row_stride]`` layout: ``np.uint16`` for bfloat16 (the upper half of
an IEEE binary32) and ``np.float32`` for fp32.  Columns ``[n, row_stride)``
are padding and may hold anything, including NaN.

Shapes and options follow the workloads the pages name:

* the usage example on the CSDN page "DeepSeek 一次开源三个仓库" (section
  三, 算子层): bf16, 4 x 204800, topk 1024, int32 indices;
* the two official performance groups on the same page and section: bf16 with
  topk 512, and fp32 sampling with vocab 129280 and topk 512;
* the scenario split on the aiutil project card "deepseek-ai/DeepSelect"
  (关键技术亮点, item 1): the Lightning Indexer path is bf16 with any batch and
  vocab, the sampler path is fp32 with a vocab of about 128K, both topk <= 4096.

Score distributions are synthetic stand-ins: the pages print no data, and
the real indexer scores and model logits come from trained models.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One generated batch of rows plus the call options that go with it."""

    name: str
    dtype: str  # "bf16" or "f32"
    batch: int
    n: int
    row_stride: int
    k: int
    sorted_index: bool
    return_value: bool
    seed: int
    raw: np.ndarray  # [batch, row_stride], uint16 (bf16 bits) or float32
    meta: dict

    @property
    def elem_size(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def algorithmic_bytes(self) -> int:
        """Bytes a top-k call must move at minimum: every valid input element
        read once, k int32 indices written per row, and k values per row when
        values are returned."""
        s = self.elem_size
        per_row = self.n * s + self.k * 4 + (self.k * s if self.return_value else 0)
        return self.batch * per_row


# name -> (dtype, batch, n, k, sorted_index, return_value, seed, description)
CONFIGS: Dict[str, dict] = {
    "C1": dict(name="indexer_smoke", dtype=BF16, batch=4, n=8192, k=64,
               sorted_index=True, return_value=True, seed=1,
               desc="bf16 N(0,1), 4 x 8192, k=64, sorted, values"),
    "C2": dict(name="lightning_indexer", dtype=BF16, batch=4, n=204800, k=1024,
               sorted_index=False, return_value=False, seed=2,
               desc="bf16 N(0,1), 4 x 204800, k=1024, unsorted, indices only"),
    "C3": dict(name="sampler", dtype=F32, batch=64, n=129280, k=512,
               sorted_index=True, return_value=True, seed=3,
               desc="fp32 N(0,sigma=2) + 32 boosts U(5,15) per row, 64 x 129280, k=512, sorted, values"),
    "C4": dict(name="indexer_ragged_decode", dtype=BF16, batch=128, n=65536, k=512,
               sorted_index=False, return_value=True, seed=4,
               desc="bf16 N(0,1) valid prefix L~U[1024,65536], -inf tail, 128 x 65536, k=512, unsorted, values"),
    "C5": dict(name="adversarial_maxk", dtype=BF16, batch=256, n=32768, k=4096,
               sorted_index=True, return_value=True, seed=5,
               desc="bf16 16 levels ascending per row, 256 x 32768, k=4096, sorted, values"),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Quantise float32 values to bfloat16 bit patterns, round to nearest even.

    Input preparation only (the workloads are bf16 scores); NaN inputs are
    not expected here -- NaNs are planted directly as bit patterns.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _stride_for(n: int, dtype: str) -> int:
    """Smallest row pitch >= n that is a multiple of 16 bytes."""
    per16 = 8 if dtype == BF16 else 4
    return (n + per16 - 1) // per16 * per16


def pad_rows(valid: np.ndarray, row_stride: int, pad_value=None) -> np.ndarray:
    """Copy ``[batch, n]`` into a fresh ``[batch, row_stride]`` array.

    The padding columns get ``pad_value`` (raw bits for uint16 arrays), or a
    NaN pattern when it is None, so that a kernel reading them for results
    would be caught.
    """
    batch, n = valid.shape
    out = np.empty((batch, row_stride), dtype=valid.dtype)
    out[:, :n] = valid
    if row_stride > n:
        if pad_value is None:
            pad_value = 0x7FC1 if valid.dtype == np.uint16 else np.float32(np.nan)
        out[:, n:] = pad_value
    return out


def _normal_bf16(rng: np.random.Generator, batch: int, n: int, scale: float = 1.0) -> np.ndarray:
    return bf16_bits_from_f32(rng.standard_normal((batch, n), dtype=np.float32) * np.float32(scale))


def _gen_c1_c2(rng, batch, n):
    return _normal_bf16(rng, batch, n), {}


def _gen_c3(rng, batch, n):
    # logits ~ N(0, sigma = 2); 32 distinct positions per row get +U(5, 15),
    # added in fp32 with round-to-nearest-even.
    x = (rng.standard_normal((batch, n), dtype=np.float32) * np.float32(2.0)).astype(np.float32)
    boosts = []
    for r in range(batch):
        pos = rng.choice(n, 32, replace=False)
        add = rng.uniform(5.0, 15.0, size=32).astype(np.float32)
        x[r, pos] = (x[r, pos] + add).astype(np.float32)
        boosts.append(np.sort(pos).tolist())
    return x, {"sigma": 2.0, "boost_positions": boosts}


NEG_INF_BF16 = 0xFF80
POS_INF_BF16 = 0x7F80


def _gen_c4(rng, batch, n):
    x = _normal_bf16(rng, batch, n)
    lengths = rng.integers(1024, 65536, size=batch, endpoint=True)
    lengths = np.minimum(lengths, n)
    for r in range(batch):
        x[r, lengths[r]:] = NEG_INF_BF16
    return x, {"lengths": lengths.tolist()}


C5_LEVELS = np.arange(-7.5, 8.0, 1.0, dtype=np.float32)  # 16 levels, exact in bf16


def _gen_c5(rng, batch, n):
    ids = np.sort(rng.integers(0, 16, size=(batch, n)), axis=1)
    x = bf16_bits_from_f32(C5_LEVELS[ids])
    counts = np.stack([np.bincount(ids[r], minlength=16) for r in range(batch)])
    return x, {"levels": C5_LEVELS.tolist(), "level_counts": counts.tolist()}


_GENERATORS = {"C1": _gen_c1_c2, "C2": _gen_c1_c2, "C3": _gen_c3, "C4": _gen_c4, "C5": _gen_c5}


def make_workload(cfg: str, batch: Optional[int] = None, n: Optional[int] = None,
                  seed: Optional[int] = None, row_stride: Optional[int] = None,
                  k: Optional[int] = None) -> Workload:
    """Generate one of the five workloads (optionally at another size/seed).

    Draws are row-major from ``numpy.random.default_rng(seed)``.
    """
    c = dict(CONFIGS[cfg])
    batch = c["batch"] if batch is None else batch
    n = c["n"] if n is None else n
    k = c["k"] if k is None else k
    seed = c["seed"] if seed is None else seed
    rs = _stride_for(n, c["dtype"]) if row_stride is None else row_stride
    rng = np.random.default_rng(seed)
    valid, meta = _GENERATORS[cfg](rng, batch, n)
    raw = pad_rows(valid, rs)
    return Workload(name=c["name"], dtype=c["dtype"], batch=batch, n=n, row_stride=rs, k=k,
                    sorted_index=c["sorted_index"], return_value=c["return_value"], seed=seed,
                    raw=raw, meta=meta)


# Bit patterns used by the edge-case rows.
_BF16_SPECIALS = np.array([0x0000, 0x8000, POS_INF_BF16, NEG_INF_BF16, 0x0001, 0x8001,
                           0x3F80, 0xBF80, 0x7F7F, 0xFF7F], dtype=np.uint16)
_F32_SPECIALS = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001,
                          0x80000001, 0x3F800000, 0xBF800000, 0x7F7FFFFF, 0xFF7FFFFF],
                         dtype=np.uint32).view(np.float32)


def make_edge_rows(dtype: str, batch: int, n: int, seed: int, levels: int = 0,
                   specials: float = 0.0, row_stride: Optional[int] = None,
                   pad_value=None) -> np.ndarray:
    """Rows built to force ties and special values.

    ``levels`` > 0 draws every value from that many distinct magnitudes (so
    ties are everywhere); ``specials`` is the fraction of positions replaced by
    +-0, +-inf, denormals and extreme finite values.
    """
    rng = np.random.default_rng(seed)
    if levels > 0:
        base = (rng.integers(-levels // 2, levels - levels // 2, size=(batch, n)).astype(np.float32)
                * np.float32(0.25))
    else:
        base = rng.standard_normal((batch, n), dtype=np.float32)
    if dtype == BF16:
        x = bf16_bits_from_f32(base)
        sp = _BF16_SPECIALS
    else:
        x = base.astype(np.float32)
        sp = _F32_SPECIALS
    if specials > 0:
        mask = rng.random((batch, n)) < specials
        x[mask] = rng.choice(sp, size=int(mask.sum()))
    rs = _stride_for(n, dtype) if row_stride is None else row_stride
    return pad_rows(x, rs, pad_value)
