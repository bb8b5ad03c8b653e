"""Graph capture: a verify call recorded into a HIP graph (through
torch.cuda.graph) and replayed matches the eager call bit for bit.

The workspace is reserved on the capturing stream first, so the captured
call allocates nothing; between replays the outputs are cleared eagerly and
the device is synchronised, and every replay is checked.
"""

import pytest

torch = pytest.importorskip("torch")

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402

from gpu_util import DeviceInputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,nsplit", [("c1", 4), ("c3_16k", 0), ("c4", 0), ("c5", 0)])
def test_graph_replay_matches_eager(name, nsplit):
    w = I.workload(name)
    d = DeviceInputs(w)
    print(f"[graph] {name} nsplit={nsplit}", flush=True)
    ref_o, ref_l = d.run(nsplit=nsplit)
    torch.cuda.synchronize()
    sparse = w.kind == "sparse"
    p = B.plan(w.batch, w.q_len, w.heads, w.slot_stride, nsplit=nsplit, mask=w.mask,
               kv_dtype=B.MLA_KV_FP8_E4M3 if sparse else B.MLA_KV_BF16,
               topk=w.meta["topk"] if sparse else 0)
    s = torch.cuda.Stream()
    B.reserve_workspace(p["workspace_bytes"], stream=s)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    if sparse:
        call = B.PreparedCall(d.q, latent=d.lat, rope=d.rope, scale=d.scale, slot_table=d.slots,
                              seq_lens=d.seq_lens, topk_idx=d.topk, sm_scale=w.sm_scale, out=out, lse=lse,
                              nsplit=nsplit)
    else:
        call = B.PreparedCall(d.q, kv=d.kv, slot_table=d.slots, seq_lens=d.seq_lens, sm_scale=w.sm_scale,
                              mask=w.mask, tree_anc=d.anc, out=out, lse=lse, nsplit=nsplit)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    assert B.device_error() == 0


def test_graph_replay_topk_matches_eager():
    # the top-k selection uses the workspace too: reserved first, then captured
    import numpy as np

    rng = np.random.default_rng(3)
    scores = torch.from_numpy(rng.standard_normal((4, 2, 20000)).astype(np.float32)).cuda()
    lens = torch.tensor([20000, 9000, 300, 19999], dtype=torch.int32).cuda()
    B.device_error()
    ref = B.topk_select(scores, lens, 512)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    B.reserve_workspace(B.topk_workspace_bytes(4, 2, 20000), stream=s)
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        B.topk_select(scores, lens, 512, out=out)
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    # the 300-position row is shorter than topk: flagged (and the flag cleared here)
    assert B.device_error() == B.MLA_DEVERR_SEQ_LEN


def test_graph_keeps_its_workspace_when_an_eager_call_grows_it():
    # A graph captured after reserving the workspace keeps replaying with that
    # buffer: a later, larger eager call on the same stream gets a new buffer
    # and the captured one stays alive (parked) until it is released.
    small = I.make_verify("ws_small", batch=1, q_len=9, heads=8, prefixes=[4000], seed=81, layout="random")
    large = I.workload("c3_64k")
    ds, dl = DeviceInputs(small), DeviceInputs(large)
    ref_o, ref_l = ds.run()
    big_o, big_l = dl.run()
    torch.cuda.synchronize()
    p = B.plan(small.batch, small.q_len, small.heads, small.slot_stride, mask=small.mask)
    s = torch.cuda.Stream()
    B.reserve_workspace(p["workspace_bytes"], stream=s)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    call = B.PreparedCall(ds.q, kv=ds.kv, slot_table=ds.slots, seq_lens=ds.seq_lens, sm_scale=small.sm_scale,
                          mask=small.mask, out=out, lse=lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for rnd in range(2):
        print(f"[graph] workspace growth round {rnd}", flush=True)
        # eager call on the capture stream needing a larger workspace
        with torch.cuda.stream(s):
            o2, l2 = dl.run()
        torch.cuda.synchronize()
        assert torch.equal(o2, big_o) and torch.equal(l2, big_l)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    del g
    torch.cuda.synchronize()
    B.release_workspace(stream=s)
    with torch.cuda.stream(s):
        o3, l3 = ds.run()              # allocates afresh after the release
    torch.cuda.synchronize()
    assert torch.equal(o3, ref_o) and torch.equal(l3, ref_l)
    assert B.device_error() == 0
