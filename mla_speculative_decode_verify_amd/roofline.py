"""Algorithmic work and traffic of one verify / sparse-decode call, and MI355X peaks.

Counting convention (pinned against the work estimate of "How a CUDA Kernel
Designer Discovered That GPU Utilization Trumps Memory Bandwidth", section
"The Back-of-the-Envelope Calculation"): every (query row, visible key) pair
costs 576 multiply-adds for the score and 512 for the value accumulation, 2
FLOP per multiply-add. Masked pairs are not counted.

Algorithmic bytes are what the method itself must move once: each visible
cache row is read exactly once for all query rows of its sequence (the
absorbed form shares the latent row across heads), plus its slot index, the
queries, the fp32 outputs and the fp32 LSE. Split-partial traffic is
overhead of the implementation and is deliberately not counted.
"""

from __future__ import annotations

from typing import Iterable, Optional

DK = 576
DV = 512
DROPE = 64

# MI355X datasheet peaks used for roofline fractions.
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP32_VALU_TFLOPS = 157.3
RIDGE_BF16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)


def _draft_visible(q_len: int, parents: Optional[Iterable[int]]) -> int:
    """Number of (draft query, draft key) visible pairs of one sequence."""
    if parents is None:
        return q_len * (q_len + 1) // 2
    par = list(parents)
    total = 0
    for i in range(q_len):
        depth = 1
        node = par[i]
        while node != -1:
            depth += 1
            node = par[node]
        total += depth
    return total


def verify_counts(q_len: int, heads: int, seq_lens, mask: str = "causal", parents=None) -> dict:
    """FLOPs and bytes of one bf16-cache verify call.

    seq_lens lists N_b per sequence (prefix + q_len when masked, all visible for
    mask "none"). parents is [B][Q] for mask "tree".
    """
    pairs = 0
    kv_rows = 0
    nseq = 0
    for b, n in enumerate(seq_lens):
        n = int(n)
        nseq += 1
        kv_rows += n
        if mask == "none":
            pairs += q_len * heads * n
        else:
            prefix = n - q_len
            dv = _draft_visible(q_len, None if mask == "causal" else parents[b])
            pairs += heads * (q_len * prefix + dv)
    rows = nseq * q_len * heads
    flops = 2.0 * (DK + DV) * pairs
    bytes_ = kv_rows * (DK * 2 + 4) + rows * (DK * 2 + DV * 4 + 4) + nseq * 4
    if mask == "tree":
        bytes_ += nseq * q_len * 8
    return dict(flops=flops, bytes=float(bytes_), pairs=pairs, kv_rows=kv_rows, rows=rows)


def sparse_counts(batch: int, q_len: int, heads: int, topk: int) -> dict:
    """FLOPs and bytes of one fp8 top-k sparse decode call.

    Per selected index: 512 fp8 latent + 64 bf16 rope + 4 B scale + 4 B index
    + 4 B slot = 652 B, read once for all heads.
    """
    idx = batch * q_len * topk
    rows = batch * q_len * heads
    pairs = rows * topk
    flops = 2.0 * (DK + DV) * pairs
    bytes_ = idx * (DV + DROPE * 2 + 4 + 4 + 4) + rows * (DK * 2 + DV * 4 + 4) + batch * 4
    return dict(flops=flops, bytes=float(bytes_), pairs=pairs, kv_rows=idx, rows=rows)


def split_partial_bytes(batch: int, rows_per_seq: int, nsplit: int) -> float:
    """Overhead traffic of the split partials: written once and read once (fp16 O,
    two fp32 power-of-two scales and the fp32 LSE per split and row)."""
    if nsplit <= 1:
        return 0.0
    return 2.0 * batch * nsplit * rows_per_seq * (DV * 2 + 12)


def roofline_us(flops: float, bytes_: float, peak_tflops: float = PEAK_BF16_TFLOPS,
                peak_gbps: float = PEAK_HBM_GBPS) -> dict:
    """Roofline time (us) and which resource bounds it."""
    t_mem = bytes_ / (peak_gbps * 1e9) * 1e6
    t_mfma = flops / (peak_tflops * 1e12) * 1e6
    return dict(us=max(t_mem, t_mfma), bound="hbm" if t_mem >= t_mfma else "mfma",
                t_hbm_us=t_mem, t_mfma_us=t_mfma)
