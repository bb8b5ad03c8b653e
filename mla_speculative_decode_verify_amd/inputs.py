"""Seeded synthetic inputs for MLA verify / sparse-decode attention.

This module is the only code shared by the HIP path's callers and the CPU
oracle's tests. It draws random numbers and stores them in the cache's
storage formats (bf16 by round-to-nearest-even, fp8 E4M3FN by torch's
round-to-nearest-even conversion after clamping to +-448); it performs none
of the attention arithmetic.

Workload shapes follow the pages' verify setting: q_len 9 draft queries, H=64
heads (single-GPU microbenchmark) or H=8 (one tensor-parallel rank's share),
prefixes 256..65536, a page_size=1 slot table, and for sparse decode a
top-k=2048 index list over an fp8 latent cache.

Draw order for one workload (all from ``numpy.random.default_rng(seed)``):
ragged prefixes (if any) -> Q -> referenced pool rows -> slot permutation
-> tree parents -> top-k positions -> per-token scales.
Pool rows that no slot references are filled with a NaN pattern so that a
kernel reading outside the referenced set shows up as NaN in its output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

DK = 576
DV = 512
DROPE = 64
SM_SCALE = 1.0 / math.sqrt(192.0)

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3FN bit patterns (clamped to +-448, then RNE via torch)."""
    import torch

    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


@dataclass
class VerifyInputs:
    """Host arrays for one verify (bf16 cache) or sparse-decode (fp8 cache) call."""

    name: str
    kind: str                     # "verify" or "sparse"
    batch: int
    q_len: int
    heads: int
    mask: str                     # "causal", "tree", "none", "topk"
    q_bits: np.ndarray            # uint16 [B, Q, H, 576]
    slot_table: np.ndarray        # int32 [B, slot_stride]
    seq_lens: np.ndarray          # int32 [B]
    pool_rows: int
    sm_scale: float = SM_SCALE
    pool_bits: Optional[np.ndarray] = None   # verify: uint16 [pool, 576]
    lat_bits: Optional[np.ndarray] = None    # sparse: uint8 [pool, 512]
    rope_bits: Optional[np.ndarray] = None   # sparse: uint16 [pool, 64]
    scale: Optional[np.ndarray] = None       # sparse: float32 [pool]
    parents: Optional[np.ndarray] = None     # tree: int32 [B, Q]
    topk_idx: Optional[np.ndarray] = None    # sparse: int32 [B, Q, topk]
    meta: Dict = field(default_factory=dict)

    @property
    def slot_stride(self) -> int:
        return int(self.slot_table.shape[1])

    @property
    def prefixes(self) -> List[int]:
        if self.kind == "verify" and self.mask != "none":
            return [int(n) - self.q_len for n in self.seq_lens]
        return [int(n) for n in self.seq_lens]


def _normal_bf16(rng, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def make_verify(name: str, *, batch: int, q_len: int, heads: int, prefixes=None, seed: int,
                layout: str = "contiguous", pool_factor: int = 2, mask: str = "causal",
                parents: Optional[np.ndarray] = None, prefix_range=None) -> VerifyInputs:
    """Dense verify workload over a bf16 latent cache.

    layout "contiguous": sequence b occupies pool rows [off_b, off_b + N_b) in
    order (identity slots for batch 1). layout "random": one seeded random
    permutation of a pool of ``pool_factor`` x total tokens; sequence b takes
    the next N_b entries of it. layout "sorted": the same random choice of
    rows, sorted ascending before it is handed out. mask "tree" draws parent(i) uniformly from
    {-1, .., i-1} unless ``parents`` is given. ``prefix_range=(lo, hi)``
    draws each sequence's prefix uniformly from [lo, hi] instead.
    """
    rng = np.random.default_rng(seed)
    if prefix_range is not None:
        lo, hi = prefix_range
        pre = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    else:
        pre = np.broadcast_to(np.asarray(prefixes, dtype=np.int64), (batch,)).copy()
    extra = q_len if mask != "none" else 0
    lens = pre + extra
    total = int(lens.sum())
    q_bits = _normal_bf16(rng, (batch, q_len, heads, DK))
    if layout == "contiguous":
        pool_rows = total
        perm = np.arange(total, dtype=np.int64)
    elif layout == "random":
        pool_rows = pool_factor * total
        ref_rows = _normal_bf16(rng, (total, DK))
        perm = rng.permutation(pool_rows)[:total]
    elif layout == "sorted":
        # a sorted free list over a fragmented pool: the same random choice of
        # free rows, handed out in ascending order (runs with gaps)
        pool_rows = pool_factor * total
        ref_rows = _normal_bf16(rng, (total, DK))
        perm = np.sort(rng.permutation(pool_rows)[:total])
    else:
        raise ValueError(layout)
    pool_bits = np.full((pool_rows, DK), BF16_NAN, dtype=np.uint16)
    if layout == "contiguous":
        pool_bits[:] = _normal_bf16(rng, (total, DK))
    else:
        pool_bits[perm] = ref_rows
    stride = int(lens.max())
    slot_table = np.zeros((batch, stride), dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(lens[b])
        slot_table[b, :n] = perm[off:off + n]
        off += n
    par = None
    if mask == "tree":
        if parents is None:
            par = np.zeros((batch, q_len), dtype=np.int32)
            for b in range(batch):
                for i in range(q_len):
                    par[b, i] = rng.integers(-1, i) if i > 0 else -1
        else:
            par = np.asarray(parents, dtype=np.int32).reshape(batch, q_len)
    return VerifyInputs(name=name, kind="verify", batch=batch, q_len=q_len, heads=heads, mask=mask,
                        q_bits=q_bits, slot_table=slot_table, seq_lens=lens.astype(np.int32),
                        pool_rows=pool_rows, pool_bits=pool_bits, parents=par,
                        meta=dict(seed=seed, layout=layout, prefixes=pre.tolist()))


def make_sparse(name: str, *, batch: int, heads: int, prefix: int, topk: int, seed: int,
                q_len: int = 1, scale_lo: float = 0.5, scale_hi: float = 2.0) -> VerifyInputs:
    """Top-k sparse decode over an fp8 E4M3FN latent cache with per-token scales.

    Each sequence has ``prefix`` cached tokens mapped by one seeded random
    permutation of a pool of batch x prefix rows. Each (sequence, query)
    attends to ``topk`` positions drawn without replacement from the prefix
    (kept in drawn order). Only referenced rows carry data; the rest hold NaN
    patterns.
    """
    rng = np.random.default_rng(seed)
    q_bits = _normal_bf16(rng, (batch, q_len, heads, DK))
    pool_rows = batch * prefix
    n_ref_max = batch * q_len * topk
    lat_vals = rng.standard_normal(size=(n_ref_max, DV), dtype=np.float32)
    rope_vals = _normal_bf16(rng, (n_ref_max, DROPE))
    perm = rng.permutation(pool_rows).astype(np.int64)
    slot_table = perm.reshape(batch, prefix).astype(np.int32)
    topk_idx = np.zeros((batch, q_len, topk), dtype=np.int32)
    for b in range(batch):
        for i in range(q_len):
            topk_idx[b, i] = rng.choice(prefix, size=topk, replace=False)
    scale_vals = rng.uniform(scale_lo, scale_hi, size=n_ref_max).astype(np.float32)
    lat_bits = np.full((pool_rows, DV), E4M3_NAN, dtype=np.uint8)
    rope_bits = np.full((pool_rows, DROPE), BF16_NAN, dtype=np.uint16)
    scale = np.full(pool_rows, np.nan, dtype=np.float32)
    ref = np.unique(slot_table[np.arange(batch)[:, None, None], topk_idx].reshape(-1).astype(np.int64))
    nref = ref.size
    lat_bits[ref] = f32_to_e4m3fn_bits(lat_vals[:nref])
    rope_bits[ref] = rope_vals[:nref]
    scale[ref] = scale_vals[:nref]
    return VerifyInputs(name=name, kind="sparse", batch=batch, q_len=q_len, heads=heads, mask="topk",
                        q_bits=q_bits, slot_table=slot_table, seq_lens=np.full(batch, prefix, dtype=np.int32),
                        pool_rows=pool_rows, lat_bits=lat_bits, rope_bits=rope_bits, scale=scale,
                        topk_idx=topk_idx, meta=dict(seed=seed, prefix=prefix, topk=topk))


# --------------------------------------------------------------------------
# Named workloads. The pages' verify microbenchmark used 1 stream, q_len 9,
# H=64 and prefixes 256..65536; the deployed tensor-parallel rank holds H=8.
# --------------------------------------------------------------------------

def workload(name: str, seed: Optional[int] = None) -> VerifyInputs:
    """Build a named workload.

    c1          batch 1, q_len 9, H 8, prefix 256, contiguous, causal (seed 1)
    c2          batch 1, q_len 9, H 64, prefix 4096, contiguous, causal (seed 2)
    c3_16k      batch 1, q_len 9, H 8, prefix 16384, random slots in a 2x pool, causal (seed 3)
    c3_64k      same at prefix 65536 (seed 4)
    c3_<P>_contig, c3_<P>_sorted (P in 16k, 64k)
                the same call with contiguous slots, or with the random rows
                handed out in ascending order (seeds 3, 4)
    c4          8 sequences, prefixes U{1024..32768}, H 64, 9-node random tree,
                random slots in a 2x pool (seed 5)
    c5          batch 32, q_len 1, H 64, prefix 65536, fp8 latent, top-k 2048 (seed 6)
    sweep_<P>   batch 1, q_len 9, H 64, prefix P, contiguous, causal (seeds 10..14)
    h8_<P>      batch 1, q_len 9, H 8, prefix P, random slots in a 2x pool, causal
                (seed 20): the H=8 shape at other prefix lengths
    """
    if name == "c1":
        return make_verify(name, batch=1, q_len=9, heads=8, prefixes=256, seed=seed or 1)
    if name == "c2":
        return make_verify(name, batch=1, q_len=9, heads=64, prefixes=4096, seed=seed or 2)
    if name == "c3_16k":
        return make_verify(name, batch=1, q_len=9, heads=8, prefixes=16384, seed=seed or 3, layout="random")
    if name == "c3_64k":
        return make_verify(name, batch=1, q_len=9, heads=8, prefixes=65536, seed=seed or 4, layout="random")
    for p, sd in (("16k", 3), ("64k", 4)):
        for lay, tag in (("contiguous", "contig"), ("sorted", "sorted")):
            if name == f"c3_{p}_{tag}":
                return make_verify(name, batch=1, q_len=9, heads=8, prefixes=16384 if p == "16k" else 65536,
                                   seed=seed or sd, layout=lay)
    if name == "c4":
        return make_verify(name, batch=8, q_len=9, heads=64, prefix_range=(1024, 32768), seed=seed or 5,
                           layout="random", mask="tree")
    if name == "c5":
        return make_sparse(name, batch=32, heads=64, prefix=65536, topk=2048, seed=seed or 6)
    if name.startswith("sweep_"):
        p = int(name.split("_")[1])
        sweep_seeds = {256: 10, 1024: 11, 4096: 12, 16384: 13, 65536: 14}
        return make_verify(name, batch=1, q_len=9, heads=64, prefixes=p, seed=seed or sweep_seeds.get(p, 15))
    if name.startswith("h8_"):
        return make_verify(name, batch=1, q_len=9, heads=8, prefixes=int(name.split("_")[1]), seed=seed or 20,
                           layout="random")
    raise KeyError(name)


WORKLOADS = ["c1", "c2", "c3_16k", "c3_64k", "c4", "c5"]
