"""C-ABI boundary checks that need no GPU: the library loads, exports every
declared entry point, rejects bad arguments before any HIP call, and its
host-side helpers (tree masks, split choice, workspace size) are exact."""

import ctypes
import os
import re

import numpy as np
import pytest

from mla_speculative_decode_verify_amd import binding as B
from oracle import mla_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.cpu


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmla_verify.so is not built (run __graft_entry__.build())")
    return B.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mla_verify.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mla_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/mla_verify.h but not exported"
    assert B.abi_version() == 4


def test_header_compiles_as_c_and_links(L, tmp_path):
    # a plain C99 consumer of the boundary: the header parses as C, the
    # library links, and mla_plan answers as it does through ctypes
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "c_consumer")
    # linked by path, so a library selected with MLA_VERIFY_LIB is the one tested
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_consumer.c"), "-o", exe, os.path.abspath(B.LIB_PATH)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    first, second = r.stdout.strip().splitlines()[:2]
    st, abi, nsplit, blocks, groups, waves, ws = (int(x) for x in first.split())
    p = B.plan(1, 9, 8, 65545, nsplit=0)
    assert (st, abi) == (0, 4)
    assert (nsplit, blocks, groups, waves, ws) == (p["nsplit"], p["row_blocks"], p["row_groups"],
                                                   p["waves_per_group"], p["workspace_bytes"])
    assert second == B.lib().mla_status_string(-2).decode()


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert B.status_string(code) and B.status_string(code) != "unknown status"
    assert B.status_string(-99) == "unknown status"


# A fake but 16-byte aligned, non-null "device pointer": validation must fail
# before the library ever dereferences or launches with it.
FAKE = 0x10000


def call(q_over=None, kv_over=None, mask_over=None, nsplit=0, out=FAKE, lse=None, slots=FAKE, seq=FAKE,
         entry="mla_verify_attn"):
    q = dict(data=FAKE, batch=1, q_len=9, heads=8, sm_scale=0.07)
    kv = dict(dtype=B.MLA_KV_BF16, latent=FAKE, rope=None, scale=None, pool_rows=100, slot_stride=50, max_seq_len=0)
    m = dict(kind=1, tree_anc=None, topk_idx=None, topk=0)
    q.update(q_over or {})
    kv.update(kv_over or {})
    m.update(mask_over or {})
    qd, kd, md = B.MlaQ(**q), B.MlaKV(**kv), B.MlaMask(**m)
    return getattr(B.lib(), entry)(ctypes.byref(qd), ctypes.byref(kd), slots, seq, ctypes.byref(md), out, lse,
                                   nsplit, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_over=dict(data=None)), B.MLA_ERR_INVALID_ARG),
    (dict(out=None), B.MLA_ERR_INVALID_ARG),
    (dict(slots=None), B.MLA_ERR_INVALID_ARG),
    (dict(q_over=dict(batch=0)), B.MLA_ERR_INVALID_ARG),
    (dict(q_over=dict(q_len=0)), B.MLA_ERR_INVALID_ARG),
    (dict(q_over=dict(q_len=65)), B.MLA_ERR_UNSUPPORTED),
    (dict(q_over=dict(heads=129)), B.MLA_ERR_UNSUPPORTED),
    (dict(q_over=dict(sm_scale=0.0)), B.MLA_ERR_INVALID_ARG),
    (dict(q_over=dict(sm_scale=float("inf"))), B.MLA_ERR_INVALID_ARG),
    (dict(q_over=dict(data=FAKE + 8)), B.MLA_ERR_ALIGN),
    (dict(out=FAKE + 4), B.MLA_ERR_ALIGN),
    (dict(lse=FAKE + 2), B.MLA_ERR_ALIGN),
    (dict(slots=FAKE + 2), B.MLA_ERR_ALIGN),
    (dict(kv_over=dict(latent=FAKE + 8)), B.MLA_ERR_ALIGN),
    (dict(kv_over=dict(pool_rows=0)), B.MLA_ERR_INVALID_ARG),
    (dict(kv_over=dict(max_seq_len=51)), B.MLA_ERR_INVALID_ARG),
    (dict(kv_over=dict(dtype=7)), B.MLA_ERR_INVALID_ARG),
    (dict(mask_over=dict(kind=9)), B.MLA_ERR_INVALID_ARG),
    (dict(mask_over=dict(kind=2)), B.MLA_ERR_INVALID_ARG),             # tree without masks
    (dict(mask_over=dict(kind=2, tree_anc=FAKE + 4)), B.MLA_ERR_ALIGN),
    (dict(mask_over=dict(kind=3)), B.MLA_ERR_UNSUPPORTED),             # top-k on a bf16 cache
    (dict(nsplit=1025), B.MLA_ERR_INVALID_ARG),
    (dict(kv_over=dict(dtype=1, rope=FAKE, scale=FAKE)), B.MLA_ERR_UNSUPPORTED),  # fp8 needs top-k
    (dict(kv_over=dict(dtype=1, rope=FAKE, scale=FAKE), mask_over=dict(kind=3, topk_idx=FAKE, topk=0)),
     B.MLA_ERR_INVALID_ARG),
    (dict(kv_over=dict(dtype=1, rope=None, scale=FAKE), mask_over=dict(kind=3, topk_idx=FAKE, topk=8)),
     B.MLA_ERR_INVALID_ARG),
    (dict(kv_over=dict(dtype=1, rope=FAKE + 8, scale=FAKE), mask_over=dict(kind=3, topk_idx=FAKE, topk=8)),
     B.MLA_ERR_ALIGN),
])
def test_bad_arguments_rejected_before_launch(L, kw, code):
    assert call(**kw) == code
    # the no-allocation variant validates the same way, before any HIP call
    assert call(entry="mla_verify_attn_noalloc", **kw) == code


def test_null_descriptors(L):
    assert L.mla_verify_attn(None, None, None, None, None, None, None, 0, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_verify_attn_noalloc(None, None, None, None, None, None, None, 0, None) == B.MLA_ERR_INVALID_ARG
    assert L.mla_plan(None, None, None, 0, None) == B.MLA_ERR_INVALID_ARG


def five_block_cost(nb, tiles, s, rows=72):
    """The planner's fitted split + merge time of a batch-1 call whose rows fill five 16-row blocks."""
    f, t, p, q = {5: (14.025, 1.379, 0.516, 0.0), 3: (12.831, 1.222, 0.282, 0.183),
                  2: (11.968, 1.454, 0.097, 0.771)}[nb]
    groups = -(-5 // nb)
    tl = -(-tiles // s)
    return f + t * tl + p * rows * s / 1000 + q * groups * s * tl / 1000 - (4.5 if s == 1 else 0.0)


def test_choose_nsplit_rules(L):
    # one tensor-parallel rank's share: H=8, q_len 9 -> 72 rows = 5 blocks of
    # 16. At 64k (2049 tiles of 32) one group of 5 blocks over at most 256
    # splits: 9 tiles for the slowest, which 228 splits already achieve
    assert B.choose_nsplit(1, 9, 8, 65545, num_cus=256) == 228
    p = B.plan(1, 9, 8, 65545)
    assert (p["row_blocks"], p["row_groups"], p["grid"]) == (5, 1, 228)
    assert B.choose_nsplit(1, 9, 8, 65536, num_cus=256) == 256      # 2048 tiles: 8 each
    # at 16k (513 tiles) two groups (3 + 2 blocks) of 103 splits, 5 tiles
    # each, beat one group of 171 splits with 3 tiles each (measured 22.0
    # against 25.7 us of split + merge kernel time)
    assert B.choose_nsplit(1, 9, 8, 16393, num_cus=256) == 103
    p = B.plan(1, 9, 8, 16393)
    assert (p["row_blocks"], p["row_groups"], p["grid"]) == (3, 2, 206)
    assert five_block_cost(3, 513, 103) < five_block_cost(5, 513, 171)
    # up to 4k three groups of 2 blocks: prefix 256 (9 tiles) one tile each
    p = B.plan(1, 9, 8, 265)
    assert (p["nsplit"], p["row_blocks"], p["row_groups"], p["grid"]) == (9, 2, 3, 27)
    p = B.plan(1, 9, 8, 4105)
    assert (p["nsplit"], p["row_blocks"], p["row_groups"], p["grid"]) == (65, 2, 3, 195)
    # every layout and split count the planner could take costs at least as
    # much under the fits as the one it took
    for n in (265, 1033, 4105, 8201, 16393, 32777, 65545):
        tiles = -(-n // 32)
        p = B.plan(1, 9, 8, n)
        chosen = five_block_cost(p["row_blocks"], tiles, p["nsplit"])
        for nb in (5, 3, 2):
            for s in range(1, min(256 // -(-5 // nb), tiles) + 1):
                assert chosen <= five_block_cost(nb, tiles, s) + 1e-9, (n, nb, s)
    # an explicit split count keeps one pass of the grid for the smaller groups
    assert B.plan(1, 9, 8, 16393, nsplit=129)["row_groups"] == 1
    assert B.plan(1, 9, 8, 16393, nsplit=128)["row_groups"] == 2
    # H=64 short: 18 row groups of 2 blocks, at most 14 splits (252
    # workgroups, one wave); 129 tiles need 10 per split, which 13 splits
    # give. Fewer splits than 9 groups of 4 (26) means fewer partials: split +
    # merge measured 24.6 against 27.5 us
    assert B.choose_nsplit(1, 9, 64, 4105, num_cus=256) == 13
    p = B.plan(1, 9, 64, 4105)
    assert (p["row_blocks"], p["row_groups"], p["grid"], p["waves_per_group"]) == (2, 18, 234, 8)
    # from 8k positions the larger groups win again (fewer key reads per row)
    assert B.plan(1, 9, 64, 8201)["row_blocks"] == 4
    # H=64 at 16k: 9 row groups of 4 blocks (each with four gather-only
    # wavefronts) and 27 splits, 19 tiles each; 8 groups of 5 would give 17
    # tiles but a dearer tile (measured 43.7 against 46.2 us of kernel time)
    p = B.plan(1, 9, 64, 16393)
    assert (p["nsplit"], p["row_blocks"], p["row_groups"], p["grid"]) == (27, 4, 9, 243)
    assert p["waves_per_group"] == 12
    # H=64 at 64k: 6 row groups of 6 blocks read each key 6 times instead of
    # 9; at most 42 splits, 49 tiles each against 74 (2.21 us per tile
    # instead of 1.86, 3.3 us more fixed cost)
    p = B.plan(1, 9, 64, 65545)
    assert (p["nsplit"], p["row_blocks"], p["row_groups"], p["grid"]) == (42, 6, 6, 252)
    # L2 prefetch ahead of the gathers from 24 tiles per split: 49 here, 17
    # at 16k, 9 for one H=8 rank at 64k
    assert p["l2_prefetch"] == 1
    assert B.plan(1, 9, 64, 16393)["l2_prefetch"] == 0
    assert B.plan(1, 9, 8, 65545)["l2_prefetch"] == 0
    assert B.plan(1, 9, 8, 65545, nsplit=64)["l2_prefetch"] == 1   # 33 tiles each
    assert B.plan(1, 9, 8, 65545, nsplit=86)["l2_prefetch"] == 1   # 2049 tiles: 24 in the longest
    assert B.plan(1, 9, 8, 65545, nsplit=90)["l2_prefetch"] == 0   # 23
    assert B.choose_nsplit(1, 9, 8, 32, num_cus=256) == 1           # one tile: no merge
    assert B.choose_nsplit(32, 1, 64, 2048, kv_dtype=B.MLA_KV_FP8_E4M3, num_cus=256) == 8
    for args in [(0, 9, 8, 10, 0, 256), (1, 9, 8, -1, 0, 256), (1, 9, 8, 10, 5, 256), (1, 9, 8, 10, 0, 0)]:
        assert L.mla_choose_nsplit(*args) == B.MLA_ERR_INVALID_ARG


def test_plan_shapes(L):
    # 72 rows: 5 blocks of 16, two wavefronts each (plus two gather-only
    # wavefronts for an odd block count); with 64 splits two groups of 3
    # blocks (the last one with 2) fit one pass of the grid
    p = B.plan(1, 9, 8, 16393, nsplit=64)
    assert (p["nsplit"], p["waves_per_group"], p["row_groups"], p["grid"], p["row_blocks"]) == (64, 8, 2, 128, 3)
    assert p["workspace_bytes"] == 64 * 72 * 1036 + 4
    p = B.plan(1, 9, 8, 16393, nsplit=200)
    assert (p["nsplit"], p["waves_per_group"], p["row_groups"], p["grid"], p["row_blocks"]) == (200, 12, 1, 200, 5)
    # 16 splits: 18 groups of 2 would need 288 workgroups (two passes), so
    # 12 groups of 3 (192, one pass)
    p = B.plan(1, 9, 64, 4105, nsplit=16)
    assert (p["waves_per_group"], p["row_groups"], p["grid"], p["row_blocks"]) == (8, 12, 192, 3)
    # 144 rows = 9 blocks: one pass of the grid with any group size, so 5
    # groups of 2 (the cheapest tile)
    p = B.plan(1, 9, 16, 4105, nsplit=16)
    assert (p["waves_per_group"], p["row_groups"], p["row_blocks"]) == (8, 5, 2)
    p = B.plan(2, 1, 1, 10, nsplit=1)
    assert p["workspace_bytes"] == 0 and p["waves_per_group"] == 4


def test_plan_balanced_splits(L):
    # ragged batch, library-chosen splits: counts follow the lengths. 6 row
    # groups of 6 blocks -> 42 splits in one pass of 256 CUs (252 workgroups);
    # the partial stride is what one sequence can take: 42 - 7 = 35
    p = B.plan(8, 9, 64, 26681)
    assert (p["balanced"], p["nsplit"], p["row_groups"], p["row_blocks"], p["grid"]) == (1, 35, 6, 6, 252)
    assert p["workspace_bytes"] == 8 * 35 * 576 * 1036 + 8 * 4
    assert p["l2_prefetch"] == 1                # 834 tiles over a stride of 35
    # the stride never exceeds ceil(tiles / 4) of the longest allowed sequence
    p = B.plan(2, 9, 8, 300)                   # 10 tiles -> at most 3 splits each, 6 in all
    assert (p["balanced"], p["nsplit"], p["grid"]) == (1, 3, 6)
    # uniform counts: an explicit nsplit, one sequence, more than 64, or too
    # many sequences for the grid
    assert B.plan(8, 9, 64, 26681, nsplit=3)["balanced"] == 0
    assert B.plan(1, 9, 8, 65545)["balanced"] == 0
    assert B.plan(65, 1, 8, 4096)["balanced"] == 0
    assert B.plan(60, 9, 64, 4096)["balanced"] == 0   # 42 units < 60 sequences
    # 30 sequences: 8 groups of 5 blocks fit one pass (240 workgroups), and
    # the 32 units they leave cover the batch
    p = B.plan(30, 9, 64, 4096)
    assert (p["balanced"], p["row_blocks"], p["row_groups"], p["nsplit"]) == (1, 5, 8, 3)
    assert B.plan(2, 9, 8, 100)["balanced"] == 0      # 4 tiles: one split each anyway


def test_plan_shapes_fp8_topk(L):
    fp8 = dict(kv_dtype=B.MLA_KV_FP8_E4M3, mask="topk", topk=2048)
    p = B.plan(32, 1, 64, 65536, nsplit=8, **fp8)     # one query per sequence, 64 heads = 4 blocks
    assert (p["kernel"], p["row_blocks"], p["row_groups"], p["grid"]) == (1, 4, 1, 8 * 32)
    assert p["workspace_bytes"] == 32 * 8 * 64 * 1036 + 32 * 4
    p = B.plan(2, 3, 80, 5000, nsplit=2, **fp8)       # 5 blocks -> groups of at most 4; grid over (seq, query)
    assert (p["row_blocks"], p["row_groups"], p["grid"]) == (4, 2, 2 * 2 * 2 * 3)
    p = B.plan(1, 1, 8, 100, nsplit=1, **fp8)        # one block: a pair and four load-only wavefronts
    assert (p["row_blocks"], p["waves_per_group"], p["workspace_bytes"]) == (1, 6, 0)
    # auto split count: key sets are (sequence, query) pairs; >= 128 list entries per split
    assert B.choose_nsplit(4, 3, 16, 512, kv_dtype=B.MLA_KV_FP8_E4M3) == 4
    assert B.choose_nsplit(1, 1, 64, 65536, kv_dtype=B.MLA_KV_FP8_E4M3) == 256
    assert B.plan(32, 1, 64, 65536, **fp8)["nsplit"] == 8


def test_workspace_bytes(L):
    assert B.workspace_bytes(1, 9, 8, 1) == 0
    assert B.workspace_bytes(3, 9, 8, 16) == 3 * 16 * 72 * 1036 + 3 * 4


def test_host_tree_mask_bit_exact_vs_oracle(L):
    rng = np.random.default_rng(0)
    for q_len in (1, 2, 9, 31, 64):
        par = np.array([[rng.integers(-1, i) if i else -1 for i in range(q_len)] for _ in range(7)], dtype=np.int32)
        np.testing.assert_array_equal(B.build_tree_mask_host(par), O.ancestor_masks(par))
    chain = np.array([[i - 1 for i in range(64)]], dtype=np.int32)
    np.testing.assert_array_equal(B.build_tree_mask_host(chain), O.causal_masks(1, 64))


def test_host_tree_mask_rejects_bad_parents(L):
    for bad in ([[0]], [[-1, 1]], [[-1, -2]], [[-1, 0, 5]]):
        with pytest.raises(B.MlaError) as e:
            B.build_tree_mask_host(np.array(bad, dtype=np.int32))
        assert e.value.status == B.MLA_ERR_INVALID_ARG
    with pytest.raises(B.MlaError):
        B.build_tree_mask_host(np.zeros((1, 65), dtype=np.int32) - 1)


@pytest.mark.parametrize("args,code", [
    # (scores, batch, q_len, score_stride, seq_lens, topk, out)
    ((0, 1, 1, 64, FAKE, 8, FAKE), B.MLA_ERR_INVALID_ARG),             # null scores
    ((FAKE, 0, 1, 64, FAKE, 8, FAKE), B.MLA_ERR_INVALID_ARG),          # no rows
    ((FAKE, 1, 1, 64, FAKE, 0, FAKE), B.MLA_ERR_INVALID_ARG),          # topk 0
    ((FAKE, 1, 1, 66, FAKE, 8, FAKE), B.MLA_ERR_ALIGN),                # stride not a multiple of 4
    ((FAKE + 4, 1, 1, 64, FAKE, 8, FAKE), B.MLA_ERR_ALIGN),            # scores not 16-byte aligned
    ((FAKE, 1, 1, (1 << 20) + 4, FAKE, 8, FAKE), B.MLA_ERR_UNSUPPORTED),  # rows longer than 2^20
    ((FAKE, 300, 256, 64, FAKE, 8, FAKE), B.MLA_ERR_UNSUPPORTED),      # more than 65535 rows
])
def test_topk_select_bad_arguments_rejected_before_launch(L, args, code):
    assert L.mla_topk_select(*args, None) == code


@pytest.mark.parametrize("args,code", [
    # (latent, pool_rows, slot_stride, new_rows, batch, q_len, slot_table, seq_lens)
    ((0, 10, 16, FAKE, 1, 4, FAKE, FAKE), B.MLA_ERR_INVALID_ARG),      # null pool
    ((FAKE, 10, 3, FAKE, 1, 4, FAKE, FAKE), B.MLA_ERR_INVALID_ARG),    # slot_stride < q_len
    ((FAKE, 10, 128, FAKE, 1, 65, FAKE, FAKE), B.MLA_ERR_UNSUPPORTED),  # q_len above 64
    ((FAKE + 8, 10, 16, FAKE, 1, 4, FAKE, FAKE), B.MLA_ERR_ALIGN),      # pool not 16-byte aligned
])
def test_append_kv_bad_arguments_rejected_before_launch(L, args, code):
    assert L.mla_append_kv(*args, None) == code


def test_topk_workspace_bytes(L):
    # per row: 8 parts of 8192 positions -> histograms, candidate pairs, row and part counters
    assert B.topk_workspace_bytes(32, 1, 65536) == 32 * (8 * 2048 * 4 + 8 * 8192 * 8 + 16 + 8 * 12)
    assert B.topk_workspace_bytes(0, 1, 64) == 0


def test_plan_invariants_over_shapes(L):
    # Library-chosen plans over a grid of bf16 shapes: at most six blocks per
    # workgroup and enough groups for every row, a one-pass grid whenever a
    # split count of 1 already fits the CUs, no more splits than tiles, a
    # workspace that matches the split count, and L2 prefetch exactly when
    # the longest split holds 24 tiles or more.
    for batch in (1, 3, 8):
        for q_len, heads in ((1, 8), (9, 8), (9, 16), (9, 64), (4, 128), (64, 2)):
            for n in (9, 300, 4105, 16393, 65545):
                if n < q_len:
                    continue
                p = B.plan(batch, q_len, heads, n)
                rows = q_len * heads
                blocks = (rows + 15) // 16
                assert 1 <= p["row_blocks"] <= 6
                assert p["row_groups"] * p["row_blocks"] >= blocks
                assert (p["row_groups"] - 1) * p["row_blocks"] < blocks
                nb = p["row_blocks"]
                assert p["waves_per_group"] == 2 * nb + (2 if nb % 2 else 4 if nb in (2, 4) else 0)
                tiles = -(-n // 32)
                if p["balanced"]:
                    assert p["grid"] <= 256
                    # the stride bounds every sequence's count, so the longest
                    # sequence's splits hold at least ceil(tiles / stride) tiles
                    assert p["l2_prefetch"] == int(-(-tiles // p["nsplit"]) >= 24)
                else:
                    assert 1 <= p["nsplit"] <= tiles
                    if batch * p["row_groups"] <= 256:
                        assert p["grid"] <= 256
                    assert (p["workspace_bytes"] == 0) == (p["nsplit"] == 1)
                    assert p["l2_prefetch"] == int(-(-tiles // p["nsplit"]) >= 24)
                    # the exported split-count rule is the plan's
                    assert B.choose_nsplit(batch, q_len, heads, n, num_cus=256) == p["nsplit"]
