"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: output max-abs <= 1e-2 and relative L2 <= 5e-3 over the whole
tensor, LSE max-abs <= 1e-3; tree masks bit-exact; repeated and
pool-permuted runs bitwise equal.
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


def _check(w, nsplits, heads=None):
    d = DeviceInputs(w)
    ref_out, ref_lse = oracle(w, heads)
    for ns in nsplits:
        _log(f"[parity] {w.name} nsplit={ns}")
        out, lse = d.run(nsplit=ns)
        torch.cuda.synchronize()
        if heads is not None:
            out, lse = out[:, :, heads], lse[:, :, heads]
        compare(out, lse, ref_out, ref_lse, f"{w.name} nsplit={ns}")
    assert B.device_error() == 0


def test_c1_small_verify():
    _check(I.workload("c1"), [1, 4, 0])


def test_c2_full_heads():
    # 8 splits and the library's 13 run 18 row groups of 2 blocks, 16 run 12
    # groups of 3, 32 and 64 run 8 groups of 5 (the last with one live block)
    _check(I.workload("c2"), [8, 16, 32, 64, 0])


def test_c3_16k_random_slots():
    _check(I.workload("c3_16k"), [16, 64, 128, 0])


def test_c3_64k_random_slots():
    _check(I.workload("c3_64k"), [16, 64, 128, 0])


def test_h64_prefix_64k_all_heads():
    # the pages' largest sweep point: q_len 9, H=64, prefix 65536, compared
    # over the whole output tensor (all 64 heads)
    # the library's plan: 6 row groups of 6 blocks, 42 splits of 49 tiles
    # with the L2 prefetch; 16 splits: 9 groups of 4, 129 tiles over three
    # 2048-position chunks, prefetching across them
    w = I.workload("sweep_65536")
    _check(w, [0, 16])


@pytest.mark.parametrize("name,nsplits", [
    ("sweep_256", [1, 4, 0]),      # one tile per split at the library's count
    ("sweep_1024", [8, 0]),
    ("sweep_16384", [0, 64]),      # library: 9 row groups of 4 blocks, 27 splits; 64: 5-block groups, two passes
])
def test_h64_prefix_sweep_all_heads(name, nsplits):
    # the other points of the pages' H=64 prefix sweep, over all 64 heads
    _check(I.workload(name), nsplits)


def test_five_block_groups_with_prefetch():
    # H=64 at 32k with 32 splits: 8 row groups of 5 blocks, each with the two
    # gather-only wavefronts, and splits of 33 tiles, long enough for the L2
    # prefetch (the only layout that runs both)
    w = I.make_verify("h64_32k_random", batch=1, q_len=9, heads=64, prefixes=[32768], seed=65, layout="random")
    p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, nsplit=32)
    assert (p["row_blocks"], p["row_groups"], p["l2_prefetch"]) == (5, 8, 1)
    _check(w, [32])


@pytest.mark.parametrize("name,batch,q_len,heads,prefixes,nsplits,blocks,balanced,prefetch", [
    ("gw_nb1_prefetch", 1, 1, 8, [20000], [8], 1, 0, 1),     # one block, long splits: L2 prefetch
    ("gw_nb1_ragged", 3, 1, 8, [9000, 300, 5000], [0], 1, 1, 0),
    ("gw_nb3_ragged", 3, 9, 4, [9000, 300, 5000], [0], 3, 1, 0),
    ("gw_nb3_prefetch", 3, 9, 4, [9000, 300, 5000], [4], 3, 0, 1),
    ("gw_nb2_ragged", 3, 9, 3, [9000, 300, 5000], [0], 2, 1, 0),
    ("gw_nb2_prefetch", 1, 9, 3, [20000], [8], 2, 0, 1),
    ("gw_nb4_ragged", 2, 8, 8, [9000, 5000], [0], 4, 1, 0),
    ("gw_nb4_prefetch", 2, 8, 8, [9000, 5000], [4], 4, 0, 1),
])
def test_gather_wave_layouts(name, batch, q_len, heads, prefixes, nsplits, blocks, balanced, prefetch):
    # block counts that run gather-only wavefronts (two for 1, 3 and 5 blocks,
    # four for 2 and 4) besides the headline shapes, with uniform and
    # length-following split counts and with the L2 prefetch
    w = I.make_verify(name, batch=batch, q_len=q_len, heads=heads, prefixes=prefixes, seed=66 + batch + heads,
                      layout="random", mask="tree" if q_len > 1 else "causal")
    p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, nsplit=nsplits[0],
               mask="tree" if q_len > 1 else "causal")
    assert (p["row_blocks"], p["balanced"], p["l2_prefetch"], p["waves_per_group"]) == \
        (blocks, balanced, prefetch, 2 * blocks + (2 if blocks % 2 else 4))
    _check(w, nsplits)


def test_c4_tree_ragged_all_heads():
    w = I.workload("c4")
    _check(w, [0, 8])


@pytest.mark.parametrize("q_len,heads,prefixes,mask", [
    (1, 8, [100], "causal"),          # plain decode, one query
    (9, 3, [0, 5, 40], "causal"),     # 27 rows: padded row block; prefix 0
    (4, 5, [31, 32, 33], "tree"),     # tile-boundary prefixes
    (64, 2, [70], "causal"),          # maximum q_len
    (9, 16, [1000, 37], "none"),      # no mask, ragged
    (7, 20, [300], "tree"),           # 140 rows -> several row groups
    (2, 128, [513, 64], "causal"),    # the largest head count: 256 rows in several row groups
    (9, 8, [int(x) for x in np.random.default_rng(3).integers(0, 700, size=40)], "tree"),  # 40 ragged sequences
])
def test_edge_shapes(q_len, heads, prefixes, mask):
    w = I.make_verify(f"edge_q{q_len}_h{heads}_{mask}", batch=len(prefixes), q_len=q_len, heads=heads,
                      prefixes=prefixes, seed=21 + q_len + heads, layout="random", mask=mask)
    _check(w, [1, 2, 5, 300, 1024, 0])


@pytest.mark.parametrize("heads,prefixes,mask", [
    (8, [0, 40000], "causal"),        # one sequence takes nearly all splits, the other one
    (8, [int(x) for x in np.random.default_rng(7).integers(0, 3000, size=64)], "tree"),  # 64: one per lane
    (64, [5000, 300, 12000], "tree"),  # 6 row groups of 6 blocks: 42 splits shared by 3 sequences
])
def test_length_following_splits(heads, prefixes, mask):
    # library-chosen splits on a ragged batch: the split counts follow the
    # lengths (derived on the device by the split and the merge kernels)
    w = I.make_verify(f"balanced_h{heads}_b{len(prefixes)}", batch=len(prefixes), q_len=9, heads=heads,
                      prefixes=prefixes, seed=50 + len(prefixes), layout="random", mask=mask)
    assert B.plan(w.batch, w.q_len, w.heads, w.slot_stride, mask=mask)["balanced"] == 1
    _check(w, [0])


def test_repeat_bitwise_and_pool_permutation():
    w = I.make_verify("perm", batch=2, q_len=9, heads=8, prefixes=[700, 1500], seed=31, layout="random",
                      mask="tree")
    d = DeviceInputs(w)
    o1, l1 = d.run(nsplit=7)
    o2, l2 = d.run(nsplit=7)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.pool_rows)
    pool2 = np.empty_like(w.pool_bits)
    pool2[perm] = w.pool_bits
    w2 = I.VerifyInputs(**{**w.__dict__, "pool_bits": pool2, "slot_table": perm[w.slot_table].astype(np.int32)})
    d2 = DeviceInputs(w2)
    o3, l3 = d2.run(nsplit=7)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_masked_rows_do_not_leak():
    w = I.make_verify("leak", batch=1, q_len=9, heads=8, prefixes=[500], seed=32, layout="random")
    d = DeviceInputs(w)
    o1, l1 = d.run(nsplit=3)
    last = w.slot_table[0, int(w.seq_lens[0]) - 1]      # draft 8: visible only to query 8
    pool = w.pool_bits.copy()
    pool[last] = I.f32_to_bf16_bits(np.full(576, 3.0e4, dtype=np.float32))
    w2 = I.VerifyInputs(**{**w.__dict__, "pool_bits": pool})
    o2, l2 = DeviceInputs(w2).run(nsplit=3)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :8], o2[:, :8]) and torch.equal(l1[:, :8], l2[:, :8])


def test_tree_mask_device_bit_exact():
    rng = np.random.default_rng(40)
    for q_len in (1, 9, 33, 64):
        par = np.array([[rng.integers(-1, i) if i else -1 for i in range(q_len)] for _ in range(5)], dtype=np.int32)
        anc = B.build_tree_mask(torch.from_numpy(par).cuda())
        got = anc.cpu().numpy().view(np.uint64)
        np.testing.assert_array_equal(got, O.ancestor_masks(par))
        np.testing.assert_array_equal(B.build_tree_mask_host(par), O.ancestor_masks(par))
    assert B.device_error() == 0


@pytest.mark.parametrize("name,nsplit", [
    ("c1", 4),        # few splits: whole-row merge units
    ("c3_16k", 0),    # library's choice: many splits, 64-column merge units
    ("c3_64k", 0),
    ("c3_64k", 40),
    ("c2", 0),
    ("c4", 0),        # ragged batch: split counts that follow the lengths
])
def test_split_and_combine_stages_equal_full_call(name, nsplit):
    # The two entry points of the split and the merge, called in turn, give
    # the full call's result bit for bit, for whole-row and 64-column merge
    # units alike; a repeated full call reproduces it.
    w = I.workload(name)
    d = DeviceInputs(w)
    _log(f"[stages] {name} nsplit={nsplit}")
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


@pytest.mark.parametrize("factor", [1.0e5, 1.0e-4])
def test_partials_keep_value_range(factor):
    # Cache values far above the fp16 range (or far below 1): the split
    # partials carry a per-half power-of-two scale, so the merged result
    # matches the oracle to the usual tolerances once rescaled. The softmax
    # scale is divided by the same factor so the scores keep their spread.
    w = I.make_verify("range", batch=2, q_len=9, heads=8, prefixes=[900, 2000], seed=33, layout="random")
    vals = O.bf16_bits_to_f64(w.pool_bits) * factor
    pool = I.f32_to_bf16_bits(vals.astype(np.float32))
    w2 = I.VerifyInputs(**{**w.__dict__, "pool_bits": pool, "sm_scale": w.sm_scale / factor})
    ref_out, ref_lse = oracle(w2)
    d = DeviceInputs(w2)
    for ns in (1, 7, 64):
        _log(f"[parity] range factor={factor} nsplit={ns}")
        out, lse = d.run(nsplit=ns)
        torch.cuda.synchronize()
        compare(out / factor, lse, ref_out / factor, ref_lse, f"range {factor} nsplit={ns}")
    assert B.device_error() == 0


def test_mixed_plans_share_the_workspace():
    # Calls with different plans run back to back on one stream and share the
    # library's workspace: uniform splits with two groups of 3 blocks (H=8 at
    # 9k) and with one 5-block group (H=8 at 60k), length-following splits
    # with 6-block groups and the L2 prefetch (ragged tree batch, H=64), 9
    # groups of 4 blocks with four gather-only wavefronts each (H=64), and the
    # fp8 sparse path.
    # Each result must equal, bit for bit, the same call made first on its
    # own, whatever ran between (stale split counts or partials would show).
    import numpy as np

    shapes = [
        I.make_verify("mix_h8", batch=1, q_len=9, heads=8, prefixes=[9000], seed=61, layout="random"),
        I.make_verify("mix_ragged", batch=3, q_len=9, heads=64, prefixes=[30000, 700, 12000], seed=62,
                      layout="random", mask="tree"),
        I.make_verify("mix_h64", batch=1, q_len=9, heads=64, prefixes=[16000], seed=63, layout="contiguous"),
        I.workload("c5"),
        I.make_verify("mix_h8_long", batch=1, q_len=9, heads=8, prefixes=[60000], seed=64, layout="random"),
    ]
    devs = [DeviceInputs(w) for w in shapes]
    first = []
    for d in devs:
        o, l = d.run()
        torch.cuda.synchronize()
        first.append((o.clone(), l.clone()))
    plans = [B.plan(w.batch, w.q_len, w.heads, w.slot_stride, mask=w.mask) for w in shapes[:3] + shapes[4:]]
    assert plans[0]["row_blocks"] == 3 and plans[0]["row_groups"] == 2 and plans[0]["balanced"] == 0
    assert plans[1]["balanced"] == 1 and plans[1]["row_blocks"] == 6 and plans[1]["l2_prefetch"] == 1
    assert plans[2]["row_blocks"] == 4 and plans[2]["row_groups"] == 9 and plans[2]["waves_per_group"] == 12
    assert plans[3]["row_blocks"] == 5 and plans[3]["row_groups"] == 1
    order = [1, 0, 4, 3, 2, 1, 3, 0, 4, 2, 1]
    for k in order:
        _log(f"[mixed] {shapes[k].name}")
        o, l = devs[k].run()
        torch.cuda.synchronize()
        assert torch.equal(o, first[k][0]) and torch.equal(l, first[k][1]), shapes[k].name
    # and the first of them still matches the oracle
    ref_out, ref_lse = oracle(shapes[0])
    compare(first[0][0], first[0][1], ref_out, ref_lse, shapes[0].name)
    assert B.device_error() == 0
    assert np.isfinite(first[1][1].cpu().numpy()).all()
