"""The no-allocation entry point (mla_verify_attn_noalloc) against mla_verify_attn.

Both run the same plan and kernels; the no-allocation call keeps its split
partials in the library's static per-device scratch instead of a workspace.
Its outputs must equal the ordinary call's bit for bit (the parity bar of
the path is tolerance against the oracle; bitwise equality with the checked
entry point is stricter), on two calls in a row with the second smaller, so
that stale partials of the first would show. A call whose partials would not
fit the scratch is refused before anything is launched.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402

from gpu_util import DeviceInputs, compare, oracle  # noqa: E402

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _both(d, nsplit=0):
    """(ordinary, no-allocation) results of the same call, both through the C ABI."""
    o1, l1 = d.run(nsplit=nsplit)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    d.run(nsplit=nsplit, stage="noalloc", out=o2, lse=l2)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def test_noalloc_equals_ordinary_call_large_then_small():
    big = I.workload("c3_64k")          # 228 splits: 17 MB of partials in the scratch
    small = I.make_verify("noalloc_small", batch=2, q_len=9, heads=8, prefixes=[3000, 640], seed=71,
                          layout="random", mask="tree")
    for w in (big, small):
        p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, mask=w.mask)
        assert 0 < p["workspace_bytes"] <= B.MLA_NOALLOC_SCRATCH_BYTES, p
        _log(f"[noalloc] {w.name} plan {p}")
        d = DeviceInputs(w)
        (o1, l1), (o2, l2) = _both(d)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), w.name
        if w is small:
            ref_out, ref_lse = oracle(w)
            compare(o2, l2, ref_out, ref_lse, f"noalloc {w.name}")
    assert B.device_error() == 0


def test_noalloc_sparse_and_explicit_splits():
    # the fp8 sparse path and an explicit split count share the same scratch
    for name, ns in (("c5", 0), ("c1", 4), ("c3_16k", 64)):
        _log(f"[noalloc] {name} nsplit={ns}")
        d = DeviceInputs(I.workload(name))
        (o1, l1), (o2, l2) = _both(d, nsplit=ns)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), name
    assert B.device_error() == 0


def test_noalloc_allocates_nothing_as_calls_grow():
    # A larger call after a smaller one leaves the device's free memory as it
    # was; the ordinary entry point grows its workspace in the same situation,
    # which the same measurement sees (the control). The first call on a new
    # stream warms the runtime's own per-stream state.
    small = DeviceInputs(I.make_verify("noalloc_s", batch=1, q_len=9, heads=8, prefixes=[2000], seed=72,
                                       layout="random"))
    large = DeviceInputs(I.make_verify("noalloc_l", batch=1, q_len=9, heads=8, prefixes=[20000], seed=73,
                                       layout="random"))
    ref_o, ref_l = large.run()
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    torch.cuda.synchronize()
    for stage, grows in (("noalloc", False), ("both", True)):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            small.run(stage=stage)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        with torch.cuda.stream(s):
            large.run(stage=stage, out=out, lse=lse)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        _log(f"[noalloc] {stage}: free memory {free0} -> {free1}")
        assert (free1 < free0) if grows else (free1 == free0), (stage, free0, free1)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        if grows:
            B.release_workspace(stream=s)


def test_noalloc_refuses_partials_beyond_the_scratch():
    w = I.workload("c4")                # 8 x 576 rows x 35 splits: 167 MB of partials
    p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, mask=w.mask)
    assert p["workspace_bytes"] > B.MLA_NOALLOC_SCRATCH_BYTES
    d = DeviceInputs(w)
    out = torch.full((w.batch, w.q_len, w.heads, 512), 7.0, device="cuda")
    lse = torch.full((w.batch, w.q_len, w.heads), 7.0, device="cuda")
    with pytest.raises(B.MlaError) as e:
        d.run(stage="noalloc", out=out, lse=lse)
    assert e.value.status == B.MLA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())   # nothing was launched
    # with one split per sequence there are no partials: the call runs
    o1, l1 = d.run(nsplit=1)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    d.run(nsplit=1, stage="noalloc", out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.isfinite(l2.cpu().numpy()).all()
    assert B.device_error() == 0
