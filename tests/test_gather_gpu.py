"""Slot gathering is bit-exact: each query row's output is exactly one cache row.

The inputs make exactly one key carry weight for every query row, through
the page_size=1 slot table of a 2x pool addressed by a random permutation
("How a CUDA Kernel Designer Discovered That GPU Utilization Trumps Memory
Bandwidth", section "Context: The Problem and the Stakes": the gather of
scattered single-token pages is the path's central cost):

* queries are zero in the 512 latent elements and +A at one rope element,
  d = (query * heads + head) mod 64, so every score comes from the rope part;
* per sequence, 64 target positions are drawn; target k's rope is +A at
  element k and zero elsewhere, every other row's rope is -A everywhere.

So query row d scores A*A*sm_scale (about 296) against its own target, 0
against the other targets and about -296 against everything else: every
other weight, relative to the target's, is below exp(-290) and rounds to
exactly 0 in fp32. The output row must then equal the target row's latent
(bf16, or E4M3FN with scale 1.0) decoded exactly: a wrong slot, row, column
or byte shows as a mismatch. Values are compared exactly as floats, so the
only freedom is the sign of zero: the output is a sum that starts from +0,
so a -0 cache element (E4M3FN rounds tiny values to it) comes out +0.
Unreferenced pool rows are NaN.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")  # (also needed on the CPU: the fp8 generator rounds through torch)

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402
from oracle import mla_oracle as O  # noqa: E402

A = 64.0


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _layout(rng, lens, extra_rows=0):
    """Random page_size=1 slot table of a 2x pool: (slot_table, pool_rows, row_of[b] = pool rows of b)."""
    total = int(sum(lens))
    pool_rows = 2 * total + extra_rows
    perm = rng.permutation(pool_rows)[:total].astype(np.int32)
    stride = max(lens)
    table = np.zeros((len(lens), stride), dtype=np.int32)
    rows, off = [], 0
    for b, n in enumerate(lens):
        table[b, :n] = perm[off:off + n]
        table[b, n:] = perm[off]
        rows.append(perm[off:off + n])
        off += n
    return table, pool_rows, rows


def _rope_block(rng, lens):
    """Rope bits per sequence: -A everywhere except 64 target rows (one-hot +A); and the targets."""
    neg, pos, zero = I.f32_to_bf16_bits(np.array([-A, A, 0.0], dtype=np.float32))
    ropes, targets = [], []
    for n in lens:
        r = np.full((n, 64), neg, dtype=np.uint16)
        t = rng.choice(n, size=64, replace=False)
        for k in range(64):
            r[t[k]] = zero
            r[t[k], k] = pos
        ropes.append(r)
        targets.append(t)
    return ropes, targets


def _assert_exact(got, want, what):
    """Exact float equality (-0 == +0), no NaN."""
    assert not np.isnan(got).any(), what
    bad = got != want
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first at {np.argwhere(bad)[0].tolist()}"


def _queries(batch, q_len, heads):
    q = np.zeros((batch, q_len, heads, 576), dtype=np.float32)
    for i in range(q_len):
        for h in range(heads):
            q[:, i, h, 512 + (i * heads + h) % 64] = A
    return I.f32_to_bf16_bits(q)


def _bf16_case(lens=(65536, 5000, 300), q_len=8, heads=8, seed=91):
    """Pool, slots and queries of the bf16 gather check, and the expected output rows."""
    rng = np.random.default_rng(seed)
    lens = list(lens)
    table, pool_rows, rows = _layout(rng, lens)
    ropes, targets = _rope_block(rng, lens)
    pool = np.full((pool_rows, 576), I.BF16_NAN, dtype=np.uint16)
    lats = []
    for b, n in enumerate(lens):
        lat = I.f32_to_bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
        pool[rows[b], :512] = lat
        pool[rows[b], 512:] = ropes[b]
        lats.append(lat)
    q = _queries(len(lens), q_len, heads)
    want = np.zeros((len(lens), q_len, heads, 512), dtype=np.float32)
    for b in range(len(lens)):
        for i in range(q_len):
            for h in range(heads):
                want[b, i, h] = O.bf16_bits_to_f64(lats[b][targets[b][(i * heads + h) % 64]])
    return dict(q=q, pool=pool, table=table, lens=np.array(lens, dtype=np.int32), want=want)


@pytest.mark.cpu
def test_bf16_gather_case_against_oracle():
    # the construction itself: the fp64 oracle returns the target rows (every
    # other weight is below exp(-290)) and lse = A*A*sm_scale
    c = _bf16_case(lens=(3000, 300), q_len=8, heads=8, seed=93)
    out, lse = O.verify_attention(c["q"], c["pool"], c["table"], c["lens"], None, I.SM_SCALE)
    _assert_exact(out.astype(np.float32), c["want"], "oracle bf16")
    np.testing.assert_allclose(lse, A * A * I.SM_SCALE, rtol=1e-15)


@pytest.mark.gpu
@pytest.mark.parametrize("nsplit", [1, 0, 37])
def test_bf16_gather_bit_exact(nsplit):
    c = _bf16_case()
    print(f"[gather] bf16 nsplit={nsplit}", flush=True)
    out, lse = B.verify_attn(_dev_bf16(c["q"]), _dev_bf16(c["pool"]), torch.from_numpy(c["table"]).cuda(),
                             torch.from_numpy(c["lens"]).cuda(), sm_scale=I.SM_SCALE, mask="none", nsplit=nsplit)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    _assert_exact(got, c["want"], f"bf16 nsplit={nsplit}")
    np.testing.assert_allclose(lse.cpu().numpy(), A * A * I.SM_SCALE, rtol=0, atol=1e-3)
    assert B.device_error() == 0


def _fp8_case(lens=(65536, 65536, 9000, 2048), heads=64, topk=2048, seed=92):
    """fp8 cache, slots, top-k lists and queries of the fp8 gather check, and the expected output rows."""
    rng = np.random.default_rng(seed)
    lens = list(lens)
    table, pool_rows, rows = _layout(rng, lens)
    ropes, targets = _rope_block(rng, lens)
    lat8 = np.full((pool_rows, 512), I.E4M3_NAN, dtype=np.uint8)
    rope = np.full((pool_rows, 64), I.BF16_NAN, dtype=np.uint16)
    scale = np.ones(pool_rows, dtype=np.float32)
    lats = []
    idx = np.zeros((len(lens), 1, topk), dtype=np.int32)
    for b, n in enumerate(lens):
        lat = I.f32_to_e4m3fn_bits(rng.standard_normal((n, 512)).astype(np.float32))
        lat8[rows[b]] = lat
        rope[rows[b]] = ropes[b]
        lats.append(lat)
        others = np.setdiff1d(np.arange(n), targets[b])
        pick = np.concatenate([targets[b], rng.choice(others, size=topk - 64, replace=False)])
        idx[b, 0] = rng.permutation(pick)
    q = _queries(len(lens), 1, heads)
    want = np.zeros((len(lens), 1, heads, 512), dtype=np.float32)
    for b in range(len(lens)):
        for h in range(heads):
            want[b, 0, h] = O.e4m3fn_bits_to_f64(lats[b][targets[b][h]])
    return dict(q=q, lat8=lat8, rope=rope, scale=scale, table=table, idx=idx,
                lens=np.array(lens, dtype=np.int32), want=want)


@pytest.mark.cpu
def test_fp8_gather_case_against_oracle():
    c = _fp8_case(lens=(3000, 700), heads=64, topk=256, seed=94)
    out, lse = O.sparse_decode_attention(c["q"], c["lat8"], c["rope"], c["scale"], c["table"], c["idx"],
                                         I.SM_SCALE)
    _assert_exact(out.astype(np.float32), c["want"], "oracle fp8")
    np.testing.assert_allclose(lse, A * A * I.SM_SCALE, rtol=1e-15)


@pytest.mark.gpu
@pytest.mark.parametrize("nsplit", [1, 0])
def test_fp8_gather_bit_exact(nsplit):
    c = _fp8_case()
    print(f"[gather] fp8 nsplit={nsplit}", flush=True)
    out, lse = B.sparse_decode(_dev_bf16(c["q"]), torch.from_numpy(c["lat8"]).cuda(), _dev_bf16(c["rope"]),
                               torch.from_numpy(c["scale"]).cuda(), torch.from_numpy(c["table"]).cuda(),
                               torch.from_numpy(c["lens"]).cuda(), torch.from_numpy(c["idx"]).cuda(),
                               sm_scale=I.SM_SCALE, nsplit=nsplit)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    _assert_exact(got, c["want"], f"fp8 nsplit={nsplit}")
    np.testing.assert_allclose(lse.cpu().numpy(), A * A * I.SM_SCALE, rtol=0, atol=1e-3)
    assert B.device_error() == 0
