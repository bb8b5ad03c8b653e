"""Helpers shared by the GPU tests: upload seeded inputs, run the C ABI, compare to the oracle."""

from __future__ import annotations

import numpy as np
import torch

from mla_speculative_decode_verify_amd import binding as B
from mla_speculative_decode_verify_amd.inputs import VerifyInputs
from oracle import mla_oracle as O

# Tolerances of the verify path (fp32 accumulation over bf16 operands, bf16 probabilities).
OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


class DeviceInputs:
    """Device copies of a VerifyInputs workload."""

    def __init__(self, w: VerifyInputs, device="cuda"):
        self.w = w
        self.q = bf16_tensor(w.q_bits, device)
        self.slots = torch.from_numpy(w.slot_table).to(device)
        self.seq_lens = torch.from_numpy(w.seq_lens).to(device)
        self.anc = None
        if w.kind == "verify":
            self.kv = bf16_tensor(w.pool_bits, device)
            if w.mask == "tree":
                par = torch.from_numpy(w.parents.astype(np.int32)).to(device)
                self.anc = B.build_tree_mask(par)
        else:
            self.lat = torch.from_numpy(w.lat_bits).to(device)
            self.rope = bf16_tensor(w.rope_bits, device)
            self.scale = torch.from_numpy(w.scale).to(device)
            self.topk = torch.from_numpy(w.topk_idx).to(device)

    def run(self, nsplit=0, stage="both", out=None, lse=None, max_seq_len=0):
        w = self.w
        if w.kind == "verify":
            return B.verify_attn(self.q, self.kv, self.slots, self.seq_lens, sm_scale=w.sm_scale, mask=w.mask,
                                 tree_anc=self.anc, nsplit=nsplit, stage=stage, out=out, lse=lse,
                                 max_seq_len=max_seq_len)
        return B.sparse_decode(self.q, self.lat, self.rope, self.scale, self.slots, self.seq_lens, self.topk,
                               sm_scale=w.sm_scale, nsplit=nsplit, stage=stage, out=out, lse=lse,
                               max_seq_len=max_seq_len)


def oracle(w: VerifyInputs, heads=None):
    """Oracle result; `heads` restricts to a subset of heads (rows are independent)."""
    q_bits = w.q_bits if heads is None else w.q_bits[:, :, heads]
    if w.kind == "sparse":
        return O.sparse_decode_attention(q_bits, w.lat_bits, w.rope_bits, w.scale, w.slot_table, w.topk_idx,
                                         w.sm_scale)
    if w.mask == "causal":
        anc = O.causal_masks(w.batch, w.q_len)
    elif w.mask == "tree":
        anc = O.ancestor_masks(w.parents)
    else:
        anc = None
    return O.verify_attention(q_bits, w.pool_bits, w.slot_table, w.seq_lens, anc, w.sm_scale)


def compare(out, lse, ref_out, ref_lse, what=""):
    """Assert the parity tolerances (output max-abs 1e-2 and relative L2 5e-3, LSE max-abs 1e-3); returns the metrics."""
    o = out.detach().float().cpu().numpy().astype(np.float64)
    l = lse.detach().float().cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    max_abs = float(np.abs(o - ref_out).max())
    rel_l2 = float(np.linalg.norm(o - ref_out) / max(np.linalg.norm(ref_out), 1e-300))
    fin = np.isfinite(ref_lse)
    assert (np.isfinite(l) == fin).all(), f"{what}: lse finiteness differs"
    lse_abs = float(np.abs(l[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    msg = f"{what}: max_abs {max_abs:.3e} rel_l2 {rel_l2:.3e} lse_abs {lse_abs:.3e}"
    assert max_abs <= OUT_MAX_ABS, msg
    assert rel_l2 <= OUT_REL_L2, msg
    assert lse_abs <= LSE_MAX_ABS, msg
    return dict(max_abs=max_abs, rel_l2=rel_l2, lse_abs=lse_abs)
