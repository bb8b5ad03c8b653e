"""GPU parity of the top-k sparse decode over an fp8 E4M3FN cache (HIP path
through the C ABI) against the fp64 oracle, plus its exact-decode,
out-of-range and split-count cases.

Tolerances as for verify: output max-abs <= 1e-2, relative L2 <= 5e-3, LSE
max-abs <= 1e-3.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402
from oracle import mla_oracle as O  # noqa: E402

from gpu_util import DeviceInputs, compare, oracle  # noqa: E402

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check(w, nsplits):
    d = DeviceInputs(w)
    ref_out, ref_lse = oracle(w)
    for ns in nsplits:
        _log(f"[sparse] {w.name} nsplit={ns}")
        out, lse = d.run(nsplit=ns)
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, f"{w.name} nsplit={ns}")
    assert B.device_error() == 0


def test_c5_full_size():
    # 32 sequences, H=64, 65536-token prefix, top-k 2048 per query
    _check(I.workload("c5"), [0, 1, 4, 16])


@pytest.mark.parametrize("batch,q_len,heads,prefix,topk", [
    (2, 1, 8, 100, 37),        # half a row block, ragged last tile
    (3, 3, 16, 1000, 300),     # several queries, each with its own list
    (1, 1, 80, 5000, 4500),    # two row groups; more entries than one staged chunk
    (1, 2, 64, 64, 64),        # every prefix position listed
    (2, 1, 128, 700, 33),      # maximum heads
])
def test_sparse_shapes(batch, q_len, heads, prefix, topk):
    w = I.make_sparse(f"sparse_b{batch}_q{q_len}_h{heads}_k{topk}", batch=batch, q_len=q_len, heads=heads,
                      prefix=prefix, topk=topk, seed=60 + heads + topk)
    _check(w, [1, 2, 7, min(topk + 3, 1024), 0])


def _single_key_case(scale):
    w = I.make_sparse("single", batch=1, q_len=1, heads=16, prefix=10, topk=1, seed=70)
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0      # the two NaN codes
    row = w.slot_table[0, w.topk_idx[0, 0, 0]]
    lat = w.lat_bits.copy()
    lat[row] = np.concatenate([codes, codes[::-1]])
    sc = w.scale.copy()
    sc[row] = scale
    return I.VerifyInputs(**{**w.__dict__, "lat_bits": lat, "scale": sc}), row


@pytest.mark.parametrize("scale", [1.0, 1.7, 0.0])
def test_single_key_reproduces_scaled_latent(scale):
    # With one key every weight is 1: the output is scale * decode(latent),
    # which checks the E4M3FN decode of all 254 finite codes (subnormals
    # included) and the fp32 handling of the scale.
    w, row = _single_key_case(scale)
    out, lse = DeviceInputs(w).run(nsplit=1)
    torch.cuda.synchronize()
    want = O.e4m3fn_bits_to_f64(w.lat_bits[row]) * np.float64(np.float32(scale))
    got = out.cpu().numpy().astype(np.float64)
    for h in range(w.heads):
        np.testing.assert_allclose(got[0, 0, h], want, rtol=2e-6, atol=0)
    ref_out, ref_lse = oracle(w)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-3)
    assert B.device_error() == 0


def test_zero_scale_keys():
    w = I.make_sparse("zero_scale", batch=2, q_len=1, heads=32, prefix=400, topk=200, seed=71)
    sc = w.scale.copy()
    rows = w.slot_table[np.arange(2)[:, None], w.topk_idx[:, 0, ::5]].reshape(-1)
    sc[rows] = 0.0
    _check(I.VerifyInputs(**{**w.__dict__, "scale": sc}), [1, 3, 0])


def test_out_of_range_entries_are_masked_and_flagged():
    w = I.make_sparse("oob", batch=1, q_len=1, heads=16, prefix=600, topk=100, seed=72)
    B.device_error()  # start clean
    topk = w.topk_idx.copy()
    topk[0, 0, [3, 50]] = [-1, 600]           # positions outside [0, prefix)
    slots = w.slot_table.copy()
    slots[0, topk[0, 0, 70]] = w.pool_rows + 3  # a listed position whose slot is outside the pool
    bad = [3, 50, 70]
    keep = np.setdiff1d(np.arange(100), bad)
    ref_w = I.VerifyInputs(**{**w.__dict__, "topk_idx": w.topk_idx[:, :, keep]})
    ref_out, ref_lse = oracle(ref_w)
    d = DeviceInputs(I.VerifyInputs(**{**w.__dict__, "topk_idx": topk, "slot_table": slots}))
    for ns in (1, 4):
        out, lse = d.run(nsplit=ns)
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, f"oob nsplit={ns}")
        err = B.device_error()
        assert err == (B.MLA_DEVERR_TOPK_RANGE | B.MLA_DEVERR_SLOT_RANGE), err


def test_sparse_repeat_bitwise():
    w = I.make_sparse("repeat", batch=4, q_len=2, heads=64, prefix=3000, topk=777, seed=73)
    d = DeviceInputs(w)
    o1, l1 = d.run(nsplit=5)
    o2, l2 = d.run(nsplit=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_verify_bad_slot_is_masked_and_flagged():
    # bf16 verify path: a cache position whose slot is outside the pool is
    # dropped like a masked key and raises the slot-range flag.
    w = I.make_verify("badslot", batch=1, q_len=9, heads=8, prefixes=[300], seed=74, layout="random")
    B.device_error()
    slots = w.slot_table.copy()
    slots[0, 123] = w.pool_rows + 10
    slots[0, 7] = -5
    # oracle: the same sequence without positions 7 and 123
    keep = np.setdiff1d(np.arange(int(w.seq_lens[0])), [7, 123])
    ref_slots = np.zeros_like(w.slot_table)
    ref_slots[0, :keep.size] = w.slot_table[0, keep]
    ref_w = I.VerifyInputs(**{**w.__dict__, "slot_table": ref_slots,
                              "seq_lens": np.array([keep.size], dtype=np.int32)})
    ref_out, ref_lse = oracle(ref_w)
    d = DeviceInputs(I.VerifyInputs(**{**w.__dict__, "slot_table": slots}))
    for ns in (1, 3):
        out, lse = d.run(nsplit=ns)
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, f"badslot nsplit={ns}")
        assert B.device_error() == B.MLA_DEVERR_SLOT_RANGE


def test_verify_bad_slots_in_long_prefetching_splits():
    # Long splits (about 79 tiles of 32 positions, so two staged chunks each)
    # take the L2 prefetch, which reads the staged row addresses four tiles
    # ahead: invalid slots are staged as the zero row there too, so they are
    # dropped like masked keys wherever they fall (first tile, chunk edge,
    # prefetch distance) and raise the slot-range flag.
    w = I.make_verify("badslot_long", batch=1, q_len=9, heads=8, prefixes=[20000], seed=76, layout="random")
    assert B.plan(w.batch, w.q_len, w.heads, w.slot_stride, nsplit=8)["l2_prefetch"] == 1
    B.device_error()
    bad = [0, 31, 32, 2047, 2048, 2600, 2629, 5101, 19990]
    slots = w.slot_table.copy()
    for k, pos in enumerate(bad):
        slots[0, pos] = w.pool_rows + 7 + k if k % 2 == 0 else -1 - k
    keep = np.setdiff1d(np.arange(int(w.seq_lens[0])), bad)
    ref_slots = np.zeros_like(w.slot_table)
    ref_slots[0, :keep.size] = w.slot_table[0, keep]
    ref_w = I.VerifyInputs(**{**w.__dict__, "slot_table": ref_slots,
                              "seq_lens": np.array([keep.size], dtype=np.int32)})
    ref_out, ref_lse = oracle(ref_w)
    d = DeviceInputs(I.VerifyInputs(**{**w.__dict__, "slot_table": slots}))
    for ns in (8, 3):
        out, lse = d.run(nsplit=ns)
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, f"badslot_long nsplit={ns}")
        assert B.device_error() == B.MLA_DEVERR_SLOT_RANGE


@pytest.mark.parametrize("nsplit", [3, 8, 40, 0])
def test_sparse_stages_equal_full_call(nsplit):
    # Split and merge entry points called in turn equal the full call bit
    # for bit (4 key sets of 64 heads), and a repeated call reproduces it.
    w = I.make_sparse("stages", batch=2, q_len=2, heads=64, prefix=3000, topk=2048, seed=75)
    d = DeviceInputs(w)
    print(f"[sparse stages] nsplit={nsplit}", flush=True)
    o1, l1 = d.run(nsplit=nsplit)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    d.run(nsplit=nsplit, stage="split", out=o2, lse=l2)
    d.run(nsplit=nsplit, stage="combine", out=o2, lse=l2)
    o3, l3 = d.run(nsplit=nsplit)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert B.device_error() == 0
