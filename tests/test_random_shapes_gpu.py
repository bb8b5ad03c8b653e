"""GPU parity on seeded random shapes: batch, q_len, head count, ragged prefixes,
mask kind and split count drawn together, so that layouts the named cases do
not reach (odd head counts, several row groups with ragged batches, forced and
library split counts) meet the oracle too; likewise for the fp8 top-k sparse
decode (batch, q_len, heads, prefix, top-k count, split count). Same bar as
the other parity tests: output max-abs <= 1e-2 and relative L2 <= 5e-3 over
the whole tensor, LSE max-abs <= 1e-3.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402

from gpu_util import DeviceInputs, compare, oracle  # noqa: E402

pytestmark = pytest.mark.gpu

_Q_LENS = [1, 2, 3, 5, 9, 16, 33, 64]
_HEADS = [1, 3, 5, 8, 12, 16, 20, 33, 64, 100, 128]
_MASKS = ["causal", "tree", "none"]
_CASES = 32
# oracle work per case: query rows x visible positions, kept to a few seconds of fp64 BLAS
_MAX_ROW_KEYS = 2.5e7


def _case(i):
    rng = np.random.default_rng(9000 + i)
    q_len = int(rng.choice(_Q_LENS))
    heads = int(rng.choice(_HEADS))
    batch = int(rng.integers(1, 7))
    mask = str(rng.choice(_MASKS))
    rows = q_len * heads
    p_max = int(min(20000, max(40, _MAX_ROW_KEYS / (rows * batch))))
    prefixes = [int(x) for x in rng.integers(0, p_max + 1, size=batch)]
    nsplit = 0 if rng.random() < 0.5 else int(rng.integers(1, 65))
    return dict(batch=batch, q_len=q_len, heads=heads, mask=mask, prefixes=prefixes, nsplit=nsplit, seed=9000 + i)


@pytest.mark.parametrize("i", range(_CASES))
def test_random_shape(i):
    c = _case(i)
    print(f"[random] case {i}: {c}", flush=True)
    w = I.make_verify(f"random{i}", batch=c["batch"], q_len=c["q_len"], heads=c["heads"], prefixes=c["prefixes"],
                      seed=c["seed"], layout="random", mask=c["mask"])
    d = DeviceInputs(w)
    ref_out, ref_lse = oracle(w)
    out, lse = d.run(nsplit=c["nsplit"])
    torch.cuda.synchronize()
    compare(out, lse, ref_out, ref_lse, f"random case {i} {c}")
    assert B.device_error() == 0


_SPARSE_CASES = 16


def _sparse_case(i):
    rng = np.random.default_rng(9500 + i)
    heads = int(rng.choice([1, 8, 16, 33, 64, 128]))
    q_len = int(rng.integers(1, 5))
    batch = int(rng.integers(1, 7))
    prefix = int(rng.integers(100, 20001))
    topk = int(rng.choice([1, 7, 64, 500, 2048]))
    topk = min(topk, prefix)
    nsplit = 0 if rng.random() < 0.5 else int(rng.integers(1, 17))
    return dict(batch=batch, q_len=q_len, heads=heads, prefix=prefix, topk=topk, nsplit=nsplit, seed=9500 + i)


@pytest.mark.parametrize("i", range(_SPARSE_CASES))
def test_random_sparse_shape(i):
    c = _sparse_case(i)
    print(f"[random sparse] case {i}: {c}", flush=True)
    w = I.make_sparse(f"rsparse{i}", batch=c["batch"], heads=c["heads"], prefix=c["prefix"], topk=c["topk"],
                      seed=c["seed"], q_len=c["q_len"])
    d = DeviceInputs(w)
    ref_out, ref_lse = oracle(w)
    out, lse = d.run(nsplit=c["nsplit"])
    torch.cuda.synchronize()
    compare(out, lse, ref_out, ref_lse, f"random sparse case {i} {c}")
    assert B.device_error() == 0
