"""GPU parity of the weight absorptions (mla_absorb_q, mla_project_o) against the oracle.

Bounds derived from the arithmetic (bf16 operands, fp32 accumulation):
  absorb_q: the latent part is the fp32 sum rounded to bf16, so
    |got - ref| <= 2^-8 |ref| + 2^-16 sum_k |q_k w_k|; the rope part is copied bit-exactly.
  project_o: o_latent is rounded to bf16 (relative 2^-9 per term) before an
    fp32 sum of 512 terms, so |got - ref| <= 2^-8 sum_k |o_k w_k|.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mla_speculative_decode_verify_amd import binding as B  # noqa: E402
from mla_speculative_decode_verify_amd import inputs as I  # noqa: E402
from oracle import mla_oracle as O  # noqa: E402

from gpu_util import bf16_tensor, compare  # noqa: E402

pytestmark = pytest.mark.gpu


def _rand_bits(rng, shape, scale=1.0):
    return I.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _absorb_bound(qn_bits, w_bits):
    qn, w = O.bf16_bits_to_f64(qn_bits), O.bf16_bits_to_f64(w_bits)
    return np.einsum("thk,hck->thc", np.abs(qn), np.abs(w))


@pytest.mark.parametrize("T,H", [(9, 8), (9, 64), (1, 3), (40, 5)])
def test_absorb_q_matches_oracle(T, H):
    rng = np.random.default_rng(90 + T + H)
    qn, qr = _rand_bits(rng, (T, H, 128)), _rand_bits(rng, (T, H, 64))
    w = _rand_bits(rng, (H, 512, 128), scale=128 ** -0.5)
    print(f"[absorb_q] T={T} H={H}", flush=True)
    got = B.absorb_q(bf16_tensor(qn), bf16_tensor(qr), bf16_tensor(w))
    torch.cuda.synchronize()
    got_bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = O.absorb_q(qn, qr, w)
    np.testing.assert_array_equal(got_bits[:, :, 512:], qr)
    g = O.bf16_bits_to_f64(got_bits[:, :, :512])
    bound = 2.0 ** -8 * np.abs(ref[:, :, :512]) + 2.0 ** -16 * _absorb_bound(qn, w)
    assert (np.abs(g - ref[:, :, :512]) <= bound).all()


@pytest.mark.parametrize("T,H", [(9, 8), (9, 64), (1, 3), (33, 5)])
def test_project_o_matches_oracle(T, H):
    rng = np.random.default_rng(95 + T + H)
    o_lat = rng.standard_normal((T, H, 512)).astype(np.float32)
    w = _rand_bits(rng, (H, 128, 512), scale=512 ** -0.5)
    print(f"[project_o] T={T} H={H}", flush=True)
    got = B.project_o(torch.from_numpy(o_lat).cuda(), bf16_tensor(w))
    torch.cuda.synchronize()
    ref = O.project_o(o_lat.astype(np.float64), w)
    bound = 2.0 ** -8 * np.einsum("thk,hck->thc", np.abs(o_lat.astype(np.float64)), np.abs(O.bf16_bits_to_f64(w)))
    assert (np.abs(got.cpu().numpy() - ref) <= bound).all()


def test_absorb_verify_project_chain():
    # q_nope, q_rope -> absorbed query -> verify over the cache -> value
    # projection; each GPU stage checked against the oracle on the GPU's own
    # input for that stage.
    w = I.workload("c1")
    rng = np.random.default_rng(99)
    T, H = w.batch * w.q_len, w.heads
    qn, qr = _rand_bits(rng, (T, H, 128)), _rand_bits(rng, (T, H, 64))
    w_uk = _rand_bits(rng, (H, 512, 128), scale=128 ** -0.5)
    w_uv = _rand_bits(rng, (H, 128, 512), scale=512 ** -0.5)
    q = B.absorb_q(bf16_tensor(qn), bf16_tensor(qr), bf16_tensor(w_uk))
    q_bits = q.view(torch.int16).cpu().numpy().view(np.uint16).reshape(w.batch, w.q_len, H, 576)
    kv = bf16_tensor(w.pool_bits)
    slots, lens = torch.from_numpy(w.slot_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    out, lse = B.verify_attn(q.view(w.batch, w.q_len, H, 576), kv, slots, lens, sm_scale=w.sm_scale,
                             mask="causal", nsplit=4)
    o = B.project_o(out.view(T, H, 512), bf16_tensor(w_uv))
    torch.cuda.synchronize()
    ref_out, ref_lse = O.verify_attention(q_bits, w.pool_bits, w.slot_table, w.seq_lens,
                                          O.causal_masks(w.batch, w.q_len), w.sm_scale)
    compare(out, lse, ref_out, ref_lse, "chain verify")
    o_in = out.cpu().numpy().astype(np.float64).reshape(T, H, 512)
    ref_o = O.project_o(o_in, w_uv)
    bound = 2.0 ** -8 * np.einsum("thk,hck->thc", np.abs(o_in), np.abs(O.bf16_bits_to_f64(w_uv)))
    assert (np.abs(o.cpu().numpy() - ref_o) <= bound).all()
    assert B.device_error() == 0
