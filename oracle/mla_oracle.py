"""CPU fp64 oracle for absorbed-MLA speculative-decoding verify attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it. It shares no code with the HIP library (no common
helpers, tables or constants); the two meet only in the seeded input
generator, which holds none of the arithmetic below.

What it computes (all in float64, from the stored input bytes):

* The pages ("How a CUDA Kernel Designer Discovered That GPU Utilization
  Trumps Memory Bandwidth", sections *Context* and *The Warp-Per-Key Dot
  Product*) describe verify attention: every draft-token query attends over
  the whole latent KV cache, each score being a 576-element dot product
  against a head-shared latent row whose first 512 elements are the value
  (the 512-wide latent accumulator of "The Occupancy Probe", section *The
  Scene*). The softmax is the ordinary numerically stable one (page 1,
  *Knowledge Required*: online softmax).
* The oracle evaluates the plain definition directly, with no KV splitting:
  split-KV with a log-sum-exp merge reaches the same value in exact
  arithmetic, so ``split_emulated_verify`` exists only to check that claim.

Readings of points the pages leave open:

1. The softmax scale multiplies the whole 576-dim dot product (rope part
   included); the configurations fix it at 1/sqrt(192).
2. LSE is the natural log of the sum of exp(scaled score).
3. Row layout: elements [0, 512) are the latent (= V), [512, 576) the rope.
4. Draft rows are already in the cache at positions P .. P+q_len-1, so
   ``seq_lens`` counts prefix + drafts for verify.
5. Causal: draft i sees the prefix and drafts 0..i (itself included).
6. Tree: parent(i) in [-1, i-1], -1 meaning a child of the prefix tail;
   node i sees the prefix plus its ancestors and itself.
7. Sparse decode: each (sequence, query) attends to exactly the listed
   prefix positions; the list is shared by all heads.
8. fp8 is OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN); the
   per-token fp32 scale multiplies the 512 latent elements only.
9. Split s of S covers [s*c, min(N, (s+1)*c)) with c = ceil(N / S); an empty
   split contributes (lse=-inf, O=0).
10. An empty visible set gives out = 0 and lse = -inf.
11. Draft-KV append (the step before a verify call): the q_len new rows of
    sequence b land at the pool rows of positions N_b - q_len .. N_b - 1 of
    its slot table, consistent with reading 4 ("How One Environment
    Variable Unlocked 3x Throughput", section *The Central Dilemma*: each
    request's KV sits in allocator-assigned slots). Every other pool row is
    untouched.
12. Top-k selection feeding the sparse decode (a sparse indexer kernel, "The
    Occupancy Probe", sections *The Thinking Process* and *Assumptions and
    Potential Pitfalls*; the pages give no scoring formula): the topk
    eligible positions with the largest scores, ties to the lower position,
    listed in ascending position order. Scores compare as real numbers with
    -0.0 below +0.0 and NaN below every number. A row with fewer eligible
    positions than topk lists them all, then -1.
13. Weight absorption around the attention (the 576 = 512 + 64 query and
    512-wide latent output of readings 1-3): q = [q_nope . W_UK[h] | q_rope]
    and o = o_latent . W_UV[h]. The pages fix only the 576 / 512 widths; the
    per-head widths 128 (q_nope) and 128 (value) are an assumption. Weights
    are given transposed, W_UK^T [H, 512, 128] and W_UV^T [H, 128, 512].
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

DK = 576  # absorbed query / key width: 512 latent + 64 rope
DV = 512  # value width: the latent part of the same row
DROPE = 64


# --------------------------------------------------------------------------
# Storage decoding (exact).
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN bit patterns -> float64 from the bit fields.

    Sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0. Exponent 0
    is subnormal (m/8 * 2^-6). Exponent 15 with mantissa 7 is NaN; there is
    no infinity, so exponent 15 with mantissa < 7 is a normal number (max 448).
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & ((b & 7) == 7), np.nan, val)
    return sign * val


# --------------------------------------------------------------------------
# Masks.
# --------------------------------------------------------------------------

def ancestor_masks(parents: np.ndarray) -> np.ndarray:
    """Draft tree parent arrays [B, Q] -> ancestor-or-self bitmasks uint64 [B, Q].

    Bit j of mask[b, i] is set when draft j is node i itself or one of its
    ancestors (reading 6). Raises ValueError unless every parent lies in
    [-1, i-1], i.e. the nodes are topologically ordered.
    """
    par = np.asarray(parents, dtype=np.int64)
    if par.ndim != 2:
        raise ValueError("parents must be [batch, q_len]")
    bsz, q_len = par.shape
    if q_len > 64:
        raise ValueError("q_len > 64 does not fit a 64-bit mask")
    out = np.zeros((bsz, q_len), dtype=np.uint64)
    for b in range(bsz):
        for i in range(q_len):
            p = int(par[b, i])
            if p < -1 or p >= i:
                raise ValueError(f"parent[{b},{i}] = {p} is outside [-1, {i - 1}]")
            bits = 1 << i
            node = p
            while node != -1:
                bits |= 1 << node
                node = int(par[b, node])
            out[b, i] = np.uint64(bits)
    return out


def causal_masks(batch: int, q_len: int) -> np.ndarray:
    """Causal draft masks: draft i sees drafts 0..i (reading 5)."""
    row = np.array([(1 << (i + 1)) - 1 for i in range(q_len)], dtype=np.uint64)
    return np.tile(row, (batch, 1))


def visible_positions(prefix: int, q_len: int, anc_bits: Optional[int]) -> np.ndarray:
    """Boolean visibility over the N = prefix + q_len cache positions of one query.

    ``anc_bits`` None means no mask (every position visible).
    """
    n = prefix + q_len
    vis = np.zeros(n, dtype=bool)
    if anc_bits is None:
        vis[:] = True
        return vis
    vis[:prefix] = True
    a = int(anc_bits)
    for j in range(q_len):
        if (a >> j) & 1:
            vis[prefix + j] = True
    return vis


# --------------------------------------------------------------------------
# Attention.
# --------------------------------------------------------------------------

def _softmax_rows(scores: np.ndarray, values: np.ndarray):
    """scores [H, n] (fp64, n may be 0), values [n, DV] -> (out [H, DV], lse [H])."""
    h = scores.shape[0]
    if scores.shape[1] == 0:
        return np.zeros((h, values.shape[1])), np.full(h, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    ssum = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(ssum))[:, 0]
    w = e / ssum
    return w @ values, lse


def verify_attention(q_bits, pool_bits, slot_table, seq_lens, anc, sm_scale):
    """Dense verify attention over a bf16 latent cache addressed through slots.

    q_bits     uint16 [B, Q, H, 576]   bf16 absorbed queries
    pool_bits  uint16 [pool, 576]      bf16 latent cache rows (page_size 1)
    slot_table int32  [B, >= N_b]      cache position -> pool row
    seq_lens   int32  [B]              N_b = prefix + q_len (reading 4)
    anc        uint64 [B, Q] or None   ancestor-or-self masks; None = no mask
    Returns (out float64 [B, Q, H, 512], lse float64 [B, Q, H]).
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, q_len, heads, dk = q.shape
    assert dk == DK
    out = np.zeros((bsz, q_len, heads, DV))
    lse = np.zeros((bsz, q_len, heads))
    for b in range(bsz):
        n = int(seq_lens[b])
        prefix = n - q_len if anc is not None else n
        if anc is not None and prefix < 0:
            raise ValueError("seq_len shorter than q_len")
        slots = np.asarray(slot_table[b, :n], dtype=np.int64)
        k = bf16_bits_to_f64(pool_bits[slots])          # [n, 576]
        v = k[:, :DV]
        s_all = (q[b].reshape(q_len * heads, DK) @ k.T).reshape(q_len, heads, n) * sm_scale
        for i in range(q_len):
            if anc is None:
                vis = np.ones(n, dtype=bool)
            else:
                vis = visible_positions(prefix, q_len, int(anc[b, i]))
            o, l = _softmax_rows(s_all[i][:, vis], v[vis])
            out[b, i] = o
            lse[b, i] = l
    return out, lse


def sparse_rows(lat_bits, rope_bits, scale, slots):
    """Decode sparse-cache rows: [scale * e4m3(latent) || bf16(rope)] -> [n, 576] (reading 8)."""
    lat = e4m3fn_bits_to_f64(lat_bits[slots]) * np.asarray(scale, dtype=np.float64)[slots][:, None]
    rope = bf16_bits_to_f64(rope_bits[slots])
    return np.concatenate([lat, rope], axis=1)


def sparse_decode_attention(q_bits, lat_bits, rope_bits, scale, slot_table, topk_idx, sm_scale):
    """Top-k sparse decode over an fp8 E4M3FN latent cache with per-token scale.

    q_bits    uint16 [B, Q, H, 576]; lat_bits uint8 [pool, 512];
    rope_bits uint16 [pool, 64]; scale float32 [pool];
    slot_table int32 [B, stride]; topk_idx int32 [B, Q, topk] (prefix positions).
    Each (b, i) attends to exactly its listed positions (reading 7).
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, q_len, heads, _ = q.shape
    out = np.zeros((bsz, q_len, heads, DV))
    lse = np.zeros((bsz, q_len, heads))
    for b in range(bsz):
        for i in range(q_len):
            pos = np.asarray(topk_idx[b, i], dtype=np.int64)
            slots = np.asarray(slot_table[b], dtype=np.int64)[pos]
            k = sparse_rows(lat_bits, rope_bits, scale, slots)
            s = (q[b, i] @ k.T) * sm_scale   # [H, topk]
            o, l = _softmax_rows(s, k[:, :DV])
            out[b, i] = o
            lse[b, i] = l
    return out, lse


def split_bounds(n: int, nsplit: int):
    """Split partition of reading 9: contiguous chunks of ceil(n / nsplit)."""
    c = -(-n // nsplit) if n > 0 else 0
    return [(min(n, s * c), min(n, (s + 1) * c)) for s in range(nsplit)]


def combine_partials(lse_parts: np.ndarray, o_parts: np.ndarray):
    """Log-sum-exp merge of per-split normalised partials.

    lse_parts [S, H], o_parts [S, H, DV]. Splits with lse = -inf carry no
    weight (and never produce NaN).
    """
    finite = np.isfinite(lse_parts)
    out = np.zeros(o_parts.shape[1:])
    lse = np.full(lse_parts.shape[1], -np.inf)
    for h in range(lse_parts.shape[1]):
        idx = np.nonzero(finite[:, h])[0]
        if idx.size == 0:
            continue
        m = lse_parts[idx, h].max()
        w = np.exp(lse_parts[idx, h] - m)
        tot = w.sum()
        lse[h] = m + math.log(tot)
        out[h] = (w[:, None] * o_parts[idx, h]).sum(axis=0) / tot
    return out, lse


def split_emulated_verify(q_bits, pool_bits, slot_table, seq_lens, anc, sm_scale, nsplit):
    """Same result as verify_attention, computed as nsplit KV partials plus a merge."""
    q = bf16_bits_to_f64(q_bits)
    bsz, q_len, heads, _ = q.shape
    out = np.zeros((bsz, q_len, heads, DV))
    lse = np.zeros((bsz, q_len, heads))
    for b in range(bsz):
        n = int(seq_lens[b])
        prefix = n - q_len if anc is not None else n
        k = bf16_bits_to_f64(pool_bits[np.asarray(slot_table[b, :n], dtype=np.int64)])
        for i in range(q_len):
            if anc is None:
                vis = np.ones(n, dtype=bool)
            else:
                vis = visible_positions(prefix, q_len, int(anc[b, i]))
            lse_p = np.full((nsplit, heads), -np.inf)
            o_p = np.zeros((nsplit, heads, DV))
            for s, (lo, hi) in enumerate(split_bounds(n, nsplit)):
                sel = np.arange(lo, hi)[vis[lo:hi]]
                sc = (q[b, i] @ k[sel].T) * sm_scale
                o_p[s], lse_p[s] = _softmax_rows(sc, k[sel, :DV])
            out[b, i], lse[b, i] = combine_partials(lse_p, o_p)
    return out, lse


# --------------------------------------------------------------------------
# Tiny-case brute force: scalar loops, math.fsum, ancestry walked directly.
# --------------------------------------------------------------------------

def brute_force_verify(q_bits, pool_bits, slot_table, seq_lens, parents, mask_kind, sm_scale):
    """Scalar reference for tiny cases. ``mask_kind`` is 'causal', 'tree' or 'none'.

    Visibility is decided by walking the parent array (tree), comparing
    indices (causal) or not at all (none): no bitmasks are involved.
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, q_len, heads, _ = q.shape
    out = np.zeros((bsz, q_len, heads, DV))
    lse = np.zeros((bsz, q_len, heads))
    for b in range(bsz):
        n = int(seq_lens[b])
        prefix = n - q_len if mask_kind != "none" else n
        rows = [bf16_bits_to_f64(pool_bits[int(slot_table[b, j])]) for j in range(n)]
        for i in range(q_len):
            visible = []
            for j in range(n):
                if j < prefix or mask_kind == "none":
                    visible.append(j)
                    continue
                d = j - prefix
                if mask_kind == "causal":
                    ok = d <= i
                else:
                    ok = False
                    node = i
                    while node != -1:
                        if node == d:
                            ok = True
                            break
                        node = int(parents[b, node])
                if ok:
                    visible.append(j)
            for h in range(heads):
                if not visible:
                    lse[b, i, h] = -math.inf
                    continue
                sc = [math.fsum(float(q[b, i, h, d]) * float(rows[j][d]) for d in range(DK)) * sm_scale
                      for j in visible]
                m = max(sc)
                ws = [math.exp(x - m) for x in sc]
                tot = math.fsum(ws)
                lse[b, i, h] = m + math.log(tot)
                for c in range(DV):
                    out[b, i, h, c] = math.fsum(w * float(rows[j][c]) for w, j in zip(ws, visible)) / tot
    return out, lse


def brute_force_sparse(q_bits, lat_bits, rope_bits, scale, slot_table, topk_idx, sm_scale):
    """Scalar reference for the sparse fp8 decode on tiny cases."""
    q = bf16_bits_to_f64(q_bits)
    bsz, q_len, heads, _ = q.shape
    out = np.zeros((bsz, q_len, heads, DV))
    lse = np.zeros((bsz, q_len, heads))
    for b in range(bsz):
        for i in range(q_len):
            keys = []
            for pos in topk_idx[b, i]:
                s = int(slot_table[b, int(pos)])
                lat = e4m3fn_bits_to_f64(lat_bits[s]) * float(scale[s])
                rope = bf16_bits_to_f64(rope_bits[s])
                keys.append(list(lat) + list(rope))
            for h in range(heads):
                sc = [math.fsum(float(q[b, i, h, d]) * kk[d] for d in range(DK)) * sm_scale for kk in keys]
                m = max(sc)
                ws = [math.exp(x - m) for x in sc]
                tot = math.fsum(ws)
                lse[b, i, h] = m + math.log(tot)
                for c in range(DV):
                    out[b, i, h, c] = math.fsum(w * kk[c] for w, kk in zip(ws, keys)) / tot
    return out, lse


def append_kv(pool_bits: np.ndarray, new_bits: np.ndarray, slot_table: np.ndarray, seq_lens: np.ndarray):
    """Pool after the draft-KV append of reading 11 (a new array; the input is not modified).

    new_bits: bf16 bits [batch, q_len, 576]; the row of draft i of sequence b
    is stored at pool row slot_table[b, seq_lens[b] - q_len + i].
    """
    out = np.array(pool_bits, copy=True)
    bsz, q_len = new_bits.shape[:2]
    for b in range(bsz):
        n = int(seq_lens[b])
        for i in range(q_len):
            out[int(slot_table[b, n - q_len + i])] = new_bits[b, i]
    return out


def topk_select(scores: np.ndarray, seq_lens: np.ndarray, topk: int) -> np.ndarray:
    """Reading 12, straight from its statement: rank every eligible position by
    (score, then lower position first) and keep the best topk, listed ascending."""
    bsz, q_len, _ = scores.shape
    out = np.full((bsz, q_len, topk), -1, dtype=np.int32)
    for b in range(bsz):
        n = max(0, min(int(seq_lens[b]), scores.shape[2]))
        for i in range(q_len):
            def rank(p):
                x = float(scores[b, i, p])
                if math.isnan(x):
                    return (0, 0.0, 0, -p)
                return (1, x, 0 if (x == 0.0 and math.copysign(1.0, x) < 0) else 1, -p)
            best = sorted(range(n), key=rank, reverse=True)[:topk]
            best.sort()
            out[b, i, :len(best)] = best
    return out


def absorb_q(q_nope_bits, q_rope_bits, w_uk_t_bits):
    """Reading 13, before the attention: fp64 [T, H, 576] = [q_nope . W_UK[h] | q_rope].

    q_nope bf16 bits [T, H, 128]; q_rope bf16 bits [T, H, 64]; w_uk_t bf16 bits
    [H, 512, 128] (W_UK[h] transposed: element [h, c, k] multiplies q_nope[.., k]
    into latent column c).
    """
    qn = bf16_bits_to_f64(q_nope_bits)
    w = bf16_bits_to_f64(w_uk_t_bits)
    T, H, _ = qn.shape
    out = np.zeros((T, H, DK))
    for h in range(H):
        out[:, h, :DV] = qn[:, h, :] @ w[h].T
    out[:, :, DV:] = bf16_bits_to_f64(q_rope_bits)
    return out


def project_o(o_latent, w_uv_t_bits):
    """Reading 13, after the attention: fp64 [T, H, 128] = o_latent . W_UV[h].

    o_latent fp64 [T, H, 512]; w_uv_t bf16 bits [H, 128, 512] (element [h, c, k]
    multiplies o_latent[.., k] into value column c).
    """
    w = bf16_bits_to_f64(w_uv_t_bits)
    T, H, _ = o_latent.shape
    out = np.zeros((T, H, w.shape[1]))
    for h in range(H):
        out[:, h, :] = o_latent[:, h, :] @ w[h].T
    return out
