"""GPU parity of the draft-KV append (mla_append_kv) against the oracle.

A byte copy, so the bar is bit-exact: the whole pool after the append must
equal the oracle's pool, rows the append must not touch included.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402
from oracle import mla_oracle as O  # noqa: E402

from gpu_util import DeviceInputs, bf16_tensor  # noqa: E402

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("batch,q_len,prefixes,layout", [
    (1, 9, [300], "random"),
    (3, 1, [5, 1000, 77], "random"),
    (2, 64, [0, 130], "sorted"),
    (4, 9, [64, 65, 2000, 31], "contiguous"),
])
def test_append_matches_oracle(batch, q_len, prefixes, layout):
    w = I.make_verify(f"app_{batch}_{q_len}", batch=batch, q_len=q_len, heads=1, prefixes=prefixes,
                      seed=50 + batch + q_len, layout=layout)
    rng = np.random.default_rng(7 + q_len)
    new = (rng.integers(0, 0x7F00, size=(batch, q_len, 576))).astype(np.uint16)  # finite bf16 patterns
    print(f"[append] batch={batch} q_len={q_len} layout={layout}", flush=True)
    kv = bf16_tensor(w.pool_bits)
    B.append_kv(kv, bf16_tensor(new), torch.from_numpy(w.slot_table).cuda(), torch.from_numpy(w.seq_lens).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(kv), O.append_kv(w.pool_bits, new, w.slot_table, w.seq_lens))
    assert B.device_error() == 0


def test_append_then_verify_equals_prebuilt_pool():
    # Wipe the drafts' pool rows, append them back on the GPU: the pool and a
    # following verify call equal those of the generator's own pool exactly.
    w = I.workload("c3_16k")
    d = DeviceInputs(w)
    ref_o, ref_l = d.run(nsplit=0)
    n = int(w.seq_lens[0])
    rows = [int(w.slot_table[0, n - w.q_len + i]) for i in range(w.q_len)]
    new = w.pool_bits[rows][None].copy()
    wiped = w.pool_bits.copy()
    wiped[rows] = 0x7FC0
    kv = bf16_tensor(wiped)
    B.append_kv(kv, bf16_tensor(new), d.slots, d.seq_lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(kv), w.pool_bits)
    o, l = B.verify_attn(d.q, kv, d.slots, d.seq_lens, sm_scale=w.sm_scale, mask=w.mask)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    assert B.device_error() == 0


def test_append_bad_inputs_are_skipped_and_flagged():
    w = I.make_verify("app_bad", batch=3, q_len=4, heads=1, prefixes=[10, 20, 30], seed=58, layout="random")
    new = np.full((3, 4, 576), 0x3F80, dtype=np.uint16)  # 1.0
    slots = w.slot_table.copy()
    lens = w.seq_lens.copy()
    slots[0, int(lens[0]) - 2] = w.pool_rows + 5   # draft 2 of sequence 0: slot past the pool
    lens[2] = 2                                    # sequence 2 shorter than q_len: nothing written
    B.device_error()
    kv = bf16_tensor(w.pool_bits)
    B.append_kv(kv, bf16_tensor(new), torch.from_numpy(slots).cuda(), torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    got = _bits(kv)
    expected = w.pool_bits.copy()
    for b in (0, 1):
        n = int(lens[b])
        for i in range(4):
            s = int(slots[b, n - 4 + i])
            if 0 <= s < w.pool_rows:
                expected[s] = new[b, i]
    np.testing.assert_array_equal(got, expected)
    assert B.device_error() == (B.MLA_DEVERR_SLOT_RANGE | B.MLA_DEVERR_SEQ_LEN)
