"""Seeded synthetic inputs for the MoE layout / dispatch / combine path.

This module only draws inputs: routing ids, routing weights, opaque payload
bytes and expert outputs. It holds none of the arithmetic the path computes
(no histogram, scan, copy or reduction), so both the CPU oracle and the GPU
library can be fed from it without sharing any of the method.

Workloads follow the shapes the DeepEP README (deepseek-ai/DeepEP, section
"Performance") and the vLLM Lamport all-gather benchmark (karylab vLLM branch
compare ds-exp-2...ds-exp-ag, bench_moe_allgather.py) run on:

* ``tiny``     N=8, E=64, top-8 uniform distinct ids, |N(0,1)| weights,
               payload 3584 B hidden + 448 B scales (the all-gather benchmark's
               NVFP4 record), bf16 expert outputs of width 7168.
* ``decode``   N=128, E=256, top-8 uniform distinct ids, weights = softmax of
               8 N(0,1) logits; fp8 e4m3 hidden 7168 (random codes, NaN codes
               0x7F/0xFF excluded) + 56 fp32 scales U(0.01, 1); bf16 7168.
* ``prefill``  N=4096, E=256 in 8 groups of 32, group-limited routing from
               N(0,1) scores (top-4 groups by group max, then top-8 experts
               inside them, descending score, ties to the lower id); weights =
               softmax over the 8 chosen scores; fp8 hidden 7168 + 56 fp32
               scales; bf16 7168.
* ``skewed``   N=4096, E=128, 8 seeded experts with zero mass and Zipf(1.2)
               popularity over the other 120 (rank -> id by a seeded
               permutation), 8 distinct ids per token drawn without
               replacement; |N(0,1)| weights; bf16 hidden 8192 as the payload
               (no scales); bf16 8192 expert outputs.
* ``large``    N=32768, E=256, top-8 uniform distinct; one 4096-byte record
               per token: ids at byte 0, weights at 32, 3584 hidden bytes at
               64, 448 scale bytes at 3648; bf16 7168 expert outputs.

bf16 values are returned as ``uint16`` bit patterns (numpy has no bf16).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "CONFIGS",
    "SEEDS",
    "Workload",
    "make",
    "make_random",
    "make_y",
    "make_x",
    "bf16_bits_from_f32",
    "uniform_distinct_ids",
]

# name -> (N, K, E, combine hidden Hc)
CONFIGS = {
    "tiny": (8, 8, 64, 7168),
    "decode": (128, 8, 256, 7168),
    "prefill": (4096, 8, 256, 7168),
    "skewed": (4096, 8, 128, 8192),
    "large": (32768, 8, 256, 7168),
}
SEEDS = {"tiny": 0, "decode": 1, "prefill": 2, "skewed": 3, "large": 4}

# Packed per-token record of the large workload: ids, weights, hidden, scales,
# each at a 16-byte aligned offset.
LARGE_RECORD = (("ids", 0, 32), ("weights", 32, 32), ("hidden", 64, 3584), ("scales", 3648, 448))
LARGE_RECORD_BYTES = 4096


@dataclass
class Workload:
    name: str
    N: int
    K: int
    E: int
    Hc: int
    seed: int
    ids: np.ndarray                    # int32 [N, K] (possibly a strided view)
    ids_row_stride: int                # in int32 elements
    weights: np.ndarray                # float32 [N, K] (possibly a strided view)
    w_row_stride: int                  # in float32 elements
    fields: List[Tuple[str, np.ndarray]] = field(default_factory=list)  # uint8 [N, row_bytes]
    records: Optional[np.ndarray] = None   # uint8 [N, record_bytes] (record mode)
    _y: Optional[np.ndarray] = None

    @property
    def rows(self) -> int:
        """Receive rows with no masked entries: one per (token, k)."""
        return self.N * self.K

    def y(self) -> np.ndarray:
        """bf16 expert outputs [N*K, Hc] as uint16 bits (drawn on first use)."""
        if self._y is None:
            self._y = make_y(self.rows, self.Hc, self.seed + 7919)
        return self._y

    def payload_bytes(self) -> int:
        if self.records is not None:
            return self.records.shape[1]
        return sum(a.shape[1] for _, a in self.fields)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Draw-side conversion of float32 samples to bf16 bit patterns.

    Uses torch's CPU conversion (a library routine), so the generator carries
    no rounding code of its own.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_y(rows: int, hc: int, seed: int, chunk_rows: int = 8192) -> np.ndarray:
    """bf16 N(0,1) matrix [rows, hc] as uint16 bits, drawn in row chunks."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, hc), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0, hc), dtype=np.float32))
    return out


def make_x(rows: int, h: int, seed: int) -> np.ndarray:
    """bf16 token activations [rows, h] as uint16 bits: N(0,1) entries times
    a per-token magnitude exp(N(0,1)), so per-block scales vary by token."""
    rng = np.random.default_rng(seed)
    mag = np.exp(rng.standard_normal((rows, 1))).astype(np.float32)
    return bf16_bits_from_f32(rng.standard_normal((rows, h), dtype=np.float32) * mag)


def uniform_distinct_ids(rng: np.random.Generator, n: int, k: int, e: int) -> np.ndarray:
    """k distinct expert ids per token, uniform, in random order."""
    keys = rng.random((n, e))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)


def _fp8_bytes(rng: np.random.Generator, n: int, h: int) -> np.ndarray:
    """Random e4m3 codes with the two NaN codes (0x7F, 0xFF) left out."""
    v = rng.integers(0, 254, size=(n, h), dtype=np.uint16)
    v = v + (v >= 0x7F)
    return v.astype(np.uint8)


def _softmax_rows(x: np.ndarray) -> np.ndarray:
    z = x.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def _group_limited_topk(scores: np.ndarray, n_groups: int, top_groups: int, k: int):
    """Group-limited routing: keep the top groups by their max score, then
    the top-k experts inside them (descending score, ties to the lower id)."""
    n, e = scores.shape
    gsz = e // n_groups
    gmax = scores.reshape(n, n_groups, gsz).max(axis=2)
    gorder = np.argsort(-gmax, axis=1, kind="stable")[:, :top_groups]
    keep = np.zeros((n, n_groups), dtype=bool)
    np.put_along_axis(keep, gorder, True, axis=1)
    masked = np.where(np.repeat(keep, gsz, axis=1), scores, -np.inf)
    ids = np.argsort(-masked, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(scores, ids, axis=1)
    return ids.astype(np.int32), chosen


def _zipf_ids(rng: np.random.Generator, n: int, k: int, e: int, s: float, n_empty: int) -> np.ndarray:
    perm = rng.permutation(e)
    empty = perm[:n_empty]
    live = perm[n_empty:]                        # rank r -> expert live[r]
    p = np.zeros(e)
    p[live] = 1.0 / np.arange(1, len(live) + 1, dtype=np.float64) ** s
    p /= p.sum()
    # Sampling k distinct ids without replacement proportional to p, via
    # Gumbel top-k keys; zero-mass experts get -inf and are never drawn.
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    keys = logp[None, :] + rng.gumbel(size=(n, e))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    assert not np.isin(ids, empty).any()
    return ids


def _u8(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint8).reshape(a.shape[0], -1)


def make(name: str, seed: Optional[int] = None) -> Workload:
    """Build one of the named workloads (``CONFIGS``) from its seed."""
    n, k, e, hc = CONFIGS[name]
    seed = SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)

    if name == "tiny":
        ids = uniform_distinct_ids(rng, n, k, e)
        w = np.abs(rng.standard_normal((n, k))).astype(np.float32)
        hidden = rng.integers(0, 256, size=(n, 3584), dtype=np.uint8)
        scales = rng.integers(0, 256, size=(n, 448), dtype=np.uint8)
        fields = [("hidden", hidden), ("scales", scales), ("ids", _u8(ids)), ("weights", _u8(w))]
        return Workload(name, n, k, e, hc, seed, ids, k, w, k, fields)

    if name in ("decode", "prefill"):
        if name == "decode":
            ids = uniform_distinct_ids(rng, n, k, e)
            w = _softmax_rows(rng.standard_normal((n, k)))
        else:
            scores = rng.standard_normal((n, e)).astype(np.float32)
            ids, chosen = _group_limited_topk(scores, 8, 4, k)
            w = _softmax_rows(chosen)
        hidden = _fp8_bytes(rng, n, 7168)
        scales = rng.uniform(0.01, 1.0, size=(n, 56)).astype(np.float32)
        fields = [("hidden", hidden), ("scales", _u8(scales)), ("ids", _u8(ids)), ("weights", _u8(w))]
        return Workload(name, n, k, e, hc, seed, ids, k, w, k, fields)

    if name == "skewed":
        ids = _zipf_ids(rng, n, k, e, 1.2, 8)
        w = np.abs(rng.standard_normal((n, k))).astype(np.float32)
        hidden = bf16_bits_from_f32(rng.standard_normal((n, 8192), dtype=np.float32))
        fields = [("hidden", _u8(hidden)), ("ids", _u8(ids)), ("weights", _u8(w))]
        return Workload(name, n, k, e, hc, seed, ids, k, w, k, fields)

    if name == "large":
        rec = np.zeros((n, LARGE_RECORD_BYTES), dtype=np.uint8)
        ids = uniform_distinct_ids(rng, n, k, e)
        w = np.abs(rng.standard_normal((n, k))).astype(np.float32)
        rec[:, 0:32] = _u8(ids)
        rec[:, 32:64] = _u8(w)
        rec[:, 64:3648] = rng.integers(0, 256, size=(n, 3584), dtype=np.uint8)
        rec[:, 3648:4096] = rng.integers(0, 256, size=(n, 448), dtype=np.uint8)
        stride = LARGE_RECORD_BYTES // 4
        ids_view = rec.view(np.int32)[:, 0:k]
        w_view = rec.view(np.float32)[:, 8:8 + k]
        return Workload(name, n, k, e, hc, seed, ids_view, stride, w_view, stride, [], rec)

    raise KeyError(name)


def make_random(seed: int, n: int, k: int, e: int, *, hc: int = 64,
                row_bytes: Tuple[int, ...] = (64, 16), mask_frac: float = 0.0,
                bad_frac: float = 0.0, distinct: bool = True) -> Workload:
    """Random stress workload.

    Ids are uniform (distinct per token when ``distinct`` and k <= e); a
    ``mask_frac`` share of entries is set to -1 (masked) and a ``bad_frac``
    share to an out-of-range id in [e, 2e+7]. Payload fields are random bytes
    of the given row sizes; weights are N(0,1) fp32 (signed).
    """
    rng = np.random.default_rng(seed)
    if distinct and k <= e:
        ids = uniform_distinct_ids(rng, n, k, e)
    else:
        ids = rng.integers(0, e, size=(n, k), dtype=np.int32)
    u = rng.random((n, k))
    ids = np.where(u < mask_frac, -1, ids)
    ids = np.where((u >= mask_frac) & (u < mask_frac + bad_frac),
                   rng.integers(e, 2 * e + 8, size=(n, k)), ids).astype(np.int32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    fields = [(f"f{i}", rng.integers(0, 256, size=(n, rb), dtype=np.uint8))
              for i, rb in enumerate(row_bytes)]
    return Workload(f"random{seed}", n, k, e, hc, seed, ids, k, w, k, fields)
