"""ctypes binding of libmla_verify.so (include/mla_verify.h) over torch tensors.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. torch supplies device memory and the current
stream. If the library is missing the first call raises; there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

# The in-tree build; MLA_VERIFY_LIB may name another build of the same library.
LIB_PATH = os.environ.get("MLA_VERIFY_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "libmla_verify.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_ALIGN = -2
MLA_ERR_UNSUPPORTED = -3
MLA_ERR_WORKSPACE = -4
MLA_ERR_LAUNCH = -5
MLA_ERR_SCRATCH = -6
MLA_NOALLOC_SCRATCH_BYTES = 32 << 20

MLA_DEVERR_SLOT_RANGE = 0x1
MLA_DEVERR_SEQ_LEN = 0x2
MLA_DEVERR_TREE_PARENT = 0x4
MLA_DEVERR_TOPK_RANGE = 0x8
MLA_DEVERR_SYNC = 0x10

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1

MASK_KINDS = {"none": 0, "causal": 1, "tree": 2, "topk": 3}

DK = 576
DV = 512


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class MlaQ(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("batch", ctypes.c_int), ("q_len", ctypes.c_int),
                ("heads", ctypes.c_int), ("sm_scale", ctypes.c_float)]


class MlaKV(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("latent", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("pool_rows", ctypes.c_int64), ("slot_stride", ctypes.c_int),
                ("max_seq_len", ctypes.c_int)]


class MlaMask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("tree_anc", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("topk", ctypes.c_int)]


class MlaPlan(ctypes.Structure):
    _fields_ = [("nsplit", ctypes.c_int), ("waves_per_group", ctypes.c_int), ("row_groups", ctypes.c_int),
                ("grid", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t), ("kernel", ctypes.c_int),
                ("row_blocks", ctypes.c_int), ("balanced", ctypes.c_int), ("l2_prefetch", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_speculative_decode_verify_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    attn_args = [P(MlaQ), P(MlaKV), ctypes.c_void_p, ctypes.c_void_p, P(MlaMask), ctypes.c_void_p,
                 ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    for name in ("mla_verify_attn", "mla_verify_split", "mla_verify_combine", "mla_verify_attn_noalloc"):
        fn = getattr(L, name)
        fn.argtypes = attn_args
        fn.restype = ctypes.c_int
    L.mla_plan.argtypes = [P(MlaQ), P(MlaKV), P(MlaMask), ctypes.c_int, P(MlaPlan)]
    L.mla_plan.restype = ctypes.c_int
    L.mla_choose_nsplit.argtypes = [ctypes.c_int] * 6
    L.mla_choose_nsplit.restype = ctypes.c_int
    L.mla_workspace_bytes.argtypes = [ctypes.c_int] * 4
    L.mla_workspace_bytes.restype = ctypes.c_size_t
    L.mla_reserve_workspace.argtypes = [ctypes.c_size_t, ctypes.c_void_p]
    L.mla_reserve_workspace.restype = ctypes.c_int
    L.mla_release_workspace.argtypes = [ctypes.c_void_p]
    L.mla_release_workspace.restype = ctypes.c_int
    L.mla_build_tree_mask.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_build_tree_mask.restype = ctypes.c_int
    L.mla_build_tree_mask_host.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.mla_build_tree_mask_host.restype = ctypes.c_int
    L.mla_append_kv.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_append_kv.restype = ctypes.c_int
    L.mla_topk_select.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_topk_select.restype = ctypes.c_int
    L.mla_topk_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.mla_topk_workspace_bytes.restype = ctypes.c_size_t
    L.mla_absorb_q.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.mla_absorb_q.restype = ctypes.c_int
    L.mla_project_o.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p]
    L.mla_project_o.restype = ctypes.c_int
    L.mla_get_device_error.argtypes = [ctypes.c_int]
    L.mla_get_device_error.restype = ctypes.c_int
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_abi_version.argtypes = []
    L.mla_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != MLA_OK:
        raise MlaError(status, what)


def _stream_handle(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _req(t, dtype, name: str, shape=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _descs(q, kv_dtype, latent, rope, scale, slot_table, mask, tree_anc, topk_idx, sm_scale, max_seq_len):
    import torch

    _req(q, torch.bfloat16, "q")
    if q.dim() != 4 or q.shape[-1] != DK:
        raise ValueError("q must be [batch, q_len, heads, 576]")
    B, Q, H, _ = q.shape
    _req(slot_table, torch.int32, "slot_table")
    if slot_table.dim() != 2 or slot_table.shape[0] != B:
        raise ValueError("slot_table must be [batch, slot_stride]")
    qd = MlaQ(q.data_ptr(), B, Q, H, float(sm_scale))
    kind = MASK_KINDS[mask]
    md = MlaMask(kind, None, None, 0)
    if kv_dtype == MLA_KV_BF16:
        _req(latent, torch.bfloat16, "kv")
        if latent.dim() != 2 or latent.shape[1] != DK:
            raise ValueError("kv must be [pool_rows, 576]")
        kd = MlaKV(MLA_KV_BF16, latent.data_ptr(), None, None, latent.shape[0], slot_table.shape[1], int(max_seq_len))
        if kind == MASK_KINDS["tree"]:
            if tree_anc is None:
                raise ValueError("mask='tree' needs tree_anc")
            _req(tree_anc, torch.int64, "tree_anc", (B, Q))
            md.tree_anc = tree_anc.data_ptr()
    else:
        _req(latent, torch.uint8, "latent")
        _req(rope, torch.bfloat16, "rope")
        _req(scale, torch.float32, "scale")
        if latent.dim() != 2 or latent.shape[1] != DV or rope.shape != (latent.shape[0], 64) or \
                scale.shape != (latent.shape[0],):
            raise ValueError("fp8 cache must be latent [pool,512] u8, rope [pool,64] bf16, scale [pool] f32")
        kd = MlaKV(MLA_KV_FP8_E4M3, latent.data_ptr(), rope.data_ptr(), scale.data_ptr(), latent.shape[0],
                   slot_table.shape[1], int(max_seq_len))
        _req(topk_idx, torch.int32, "topk_idx")
        if topk_idx.dim() != 3 or topk_idx.shape[:2] != (B, Q):
            raise ValueError("topk_idx must be [batch, q_len, topk]")
        md.topk_idx = topk_idx.data_ptr()
        md.topk = topk_idx.shape[2]
    return qd, kd, md, (B, Q, H)


_STAGES = {"both": "mla_verify_attn", "split": "mla_verify_split", "combine": "mla_verify_combine",
           "noalloc": "mla_verify_attn_noalloc"}


def _run(stage, qd, kd, md, slot_table, seq_lens, out, lse, nsplit, stream):
    fn = getattr(lib(), _STAGES[stage])
    st = fn(ctypes.byref(qd), ctypes.byref(kd), slot_table.data_ptr(), seq_lens.data_ptr(), ctypes.byref(md),
            out.data_ptr(), None if lse is None else lse.data_ptr(), int(nsplit), _stream_handle(stream))
    _check(st, _STAGES[stage])


def _outputs(shape, out, lse, want_lse, device):
    import torch

    B, Q, H = shape
    if out is None:
        out = torch.empty((B, Q, H, DV), dtype=torch.float32, device=device)
    else:
        _req(out, torch.float32, "out", (B, Q, H, DV))
    if lse is None and want_lse:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=device)
    elif lse is not None:
        _req(lse, torch.float32, "lse", (B, Q, H))
    return out, lse


def verify_attn(q, kv, slot_table, seq_lens, *, sm_scale: float, mask: str = "causal", tree_anc=None,
                out=None, lse=None, want_lse: bool = True, nsplit: int = 0, max_seq_len: int = 0,
                stream=None, stage: str = "both"):
    """Verify attention over a bf16 latent cache. Returns (out, lse)."""
    import torch

    qd, kd, md, shape = _descs(q, MLA_KV_BF16, kv, None, None, slot_table, mask, tree_anc, None, sm_scale,
                               max_seq_len)
    _req(seq_lens, torch.int32, "seq_lens", (shape[0],))
    out, lse = _outputs(shape, out, lse, want_lse, q.device)
    _run(stage, qd, kd, md, slot_table, seq_lens, out, lse, nsplit, stream)
    return out, lse


def sparse_decode(q, latent, rope, scale, slot_table, seq_lens, topk_idx, *, sm_scale: float, out=None,
                  lse=None, want_lse: bool = True, nsplit: int = 0, max_seq_len: int = 0, stream=None,
                  stage: str = "both"):
    """Top-k sparse decode over an fp8 E4M3FN latent cache with per-token scale. Returns (out, lse)."""
    import torch

    qd, kd, md, shape = _descs(q, MLA_KV_FP8_E4M3, latent, rope, scale, slot_table, "topk", None, topk_idx,
                               sm_scale, max_seq_len)
    _req(seq_lens, torch.int32, "seq_lens", (shape[0],))
    out, lse = _outputs(shape, out, lse, want_lse, q.device)
    _run(stage, qd, kd, md, slot_table, seq_lens, out, lse, nsplit, stream)
    return out, lse


def plan(batch: int, q_len: int, heads: int, slot_stride: int, *, kv_dtype: int = MLA_KV_BF16,
         mask: str = "causal", topk: int = 0, nsplit: int = 0, max_seq_len: int = 0, pool_rows: int = 1) -> dict:
    """The library's plan for a call of this shape (no device memory needed)."""
    qd = MlaQ(None, batch, q_len, heads, 1.0)
    kd = MlaKV(kv_dtype, None, None, None, pool_rows, slot_stride, max_seq_len)
    md = MlaMask(MASK_KINDS[mask], None, None, topk)
    p = MlaPlan()
    _check(lib().mla_plan(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(md), int(nsplit), ctypes.byref(p)),
           "mla_plan")
    return {f: getattr(p, f) for f, _ in MlaPlan._fields_}


def choose_nsplit(batch, q_len, heads, max_seq_len, kv_dtype=MLA_KV_BF16, num_cus=256) -> int:
    r = lib().mla_choose_nsplit(batch, q_len, heads, max_seq_len, kv_dtype, num_cus)
    if r < 0:
        raise MlaError(r, "mla_choose_nsplit")
    return r


def workspace_bytes(batch, q_len, heads, nsplit) -> int:
    return int(lib().mla_workspace_bytes(batch, q_len, heads, nsplit))


def reserve_workspace(nbytes: int, stream=None) -> None:
    _check(lib().mla_reserve_workspace(int(nbytes), _stream_handle(stream)), "mla_reserve_workspace")


def release_workspace(stream=None) -> None:
    _check(lib().mla_release_workspace(_stream_handle(stream)), "mla_release_workspace")


def build_tree_mask(parents, stream=None):
    """Device ancestor-or-self masks (int64 tensor holding the uint64 bits) from int32 parents [B, Q]."""
    import torch

    _req(parents, torch.int32, "parents")
    B, Q = parents.shape
    anc = torch.empty((B, Q), dtype=torch.int64, device=parents.device)
    _check(lib().mla_build_tree_mask(parents.data_ptr(), B, Q, anc.data_ptr(), _stream_handle(stream)),
           "mla_build_tree_mask")
    return anc


def append_kv(kv, new_rows, slot_table, seq_lens, stream=None):
    """Write the drafts' latent rows (bf16 [B, Q, 576]) into the bf16 pool ``kv`` [pool_rows, 576] in place,
    at the pool rows of positions seq_lens[b] - Q .. seq_lens[b] - 1 of each slot table row."""
    import torch

    _req(kv, torch.bfloat16, "kv")
    _req(new_rows, torch.bfloat16, "new_rows")
    _req(slot_table, torch.int32, "slot_table")
    if kv.dim() != 2 or kv.shape[1] != 576 or new_rows.dim() != 3 or new_rows.shape[2] != 576:
        raise ValueError("kv must be [pool_rows, 576] and new_rows [B, Q, 576]")
    bsz, q_len = int(new_rows.shape[0]), int(new_rows.shape[1])
    if slot_table.dim() != 2 or slot_table.shape[0] != bsz:
        raise ValueError("slot_table must be [B, slot_stride]")
    _req(seq_lens, torch.int32, "seq_lens", (bsz,))
    _check(lib().mla_append_kv(kv.data_ptr(), int(kv.shape[0]), int(slot_table.shape[1]), new_rows.data_ptr(), bsz,
                               q_len, slot_table.data_ptr(), seq_lens.data_ptr(), _stream_handle(stream)),
           "mla_append_kv")


def topk_select(scores, seq_lens, topk: int, out=None, stream=None):
    """Top-k positions (int32 [B, Q, topk], ascending) of fp32 scores [B, Q, S] below seq_lens[b]."""
    import torch

    _req(scores, torch.float32, "scores")
    if scores.dim() != 3:
        raise ValueError("scores must be [B, Q, S]")
    bsz, q_len, stride = (int(x) for x in scores.shape)
    _req(seq_lens, torch.int32, "seq_lens", (bsz,))
    if out is None:
        out = torch.empty((bsz, q_len, topk), dtype=torch.int32, device=scores.device)
    _req(out, torch.int32, "out", (bsz, q_len, topk))
    _check(lib().mla_topk_select(scores.data_ptr(), bsz, q_len, stride, seq_lens.data_ptr(), int(topk),
                                 out.data_ptr(), _stream_handle(stream)), "mla_topk_select")
    return out


def absorb_q(q_nope, q_rope, w_uk, out=None, stream=None):
    """Absorbed query bf16 [T, H, 576] = [q_nope . W_UK[h] | q_rope]; w_uk is bf16 [H, 512, 128] (transposed)."""
    import torch

    T, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    _req(q_nope, torch.bfloat16, "q_nope", (T, H, 128))
    _req(q_rope, torch.bfloat16, "q_rope", (T, H, 64))
    _req(w_uk, torch.bfloat16, "w_uk", (H, 512, 128))
    if out is None:
        out = torch.empty((T, H, 576), dtype=torch.bfloat16, device=q_nope.device)
    _req(out, torch.bfloat16, "out", (T, H, 576))
    _check(lib().mla_absorb_q(q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(), T, H, out.data_ptr(),
                              _stream_handle(stream)), "mla_absorb_q")
    return out


def project_o(o_latent, w_uv, out=None, stream=None):
    """Per-head output fp32 [T, H, 128] = o_latent . W_UV[h]; w_uv is bf16 [H, 128, 512] (transposed)."""
    import torch

    T, H = int(o_latent.shape[0]), int(o_latent.shape[1])
    _req(o_latent, torch.float32, "o_latent", (T, H, 512))
    _req(w_uv, torch.bfloat16, "w_uv", (H, 128, 512))
    if out is None:
        out = torch.empty((T, H, 128), dtype=torch.float32, device=o_latent.device)
    _req(out, torch.float32, "out", (T, H, 128))
    _check(lib().mla_project_o(o_latent.data_ptr(), w_uv.data_ptr(), T, H, out.data_ptr(), _stream_handle(stream)),
           "mla_project_o")
    return out


def topk_workspace_bytes(batch: int, q_len: int, score_stride: int) -> int:
    return int(lib().mla_topk_workspace_bytes(batch, q_len, score_stride))


def build_tree_mask_host(parents: np.ndarray) -> np.ndarray:
    """Host ancestor-or-self masks (uint64 [B, Q]) from parents [B, Q]."""
    par = np.ascontiguousarray(parents, dtype=np.int32)
    B, Q = par.shape
    out = np.zeros((B, Q), dtype=np.uint64)
    _check(lib().mla_build_tree_mask_host(par.ctypes.data, B, Q, out.ctypes.data), "mla_build_tree_mask_host")
    return out


def device_error(clear: bool = True) -> int:
    r = lib().mla_get_device_error(1 if clear else 0)
    if r < 0:
        raise MlaError(r, "mla_get_device_error")
    return r


def abi_version() -> int:
    return lib().mla_abi_version()


class PreparedCall:
    """A verify / sparse-decode call with its descriptors marshalled once.

    ``__call__`` re-issues exactly the same C call (same tensors, same stream
    handle unless one is given) with no per-call Python validation, for
    tight timing loops and graph capture. The tensors must stay alive.
    """

    def __init__(self, q, *, kv=None, latent=None, rope=None, scale=None, slot_table, seq_lens, sm_scale,
                 mask="causal", tree_anc=None, topk_idx=None, out=None, lse=None, nsplit=0, max_seq_len=0,
                 stage="both"):
        import torch

        if kv is not None:
            self.qd, self.kd, self.md, shape = _descs(q, MLA_KV_BF16, kv, None, None, slot_table, mask, tree_anc,
                                                      None, sm_scale, max_seq_len)
        else:
            self.qd, self.kd, self.md, shape = _descs(q, MLA_KV_FP8_E4M3, latent, rope, scale, slot_table, "topk",
                                                      None, topk_idx, sm_scale, max_seq_len)
        _req(seq_lens, torch.int32, "seq_lens", (shape[0],))
        self.out, self.lse = _outputs(shape, out, lse, True, q.device)
        self._keep = (q, kv, latent, rope, scale, slot_table, seq_lens, tree_anc, topk_idx)
        self.fn = getattr(lib(), _STAGES[stage])
        self.args = (ctypes.byref(self.qd), ctypes.byref(self.kd), ctypes.c_void_p(slot_table.data_ptr()),
                     ctypes.c_void_p(seq_lens.data_ptr()), ctypes.byref(self.md),
                     ctypes.c_void_p(self.out.data_ptr()), ctypes.c_void_p(self.lse.data_ptr()), int(nsplit))
        self.what = _STAGES[stage]

    def __call__(self, stream_handle: Optional[int] = None):
        st = self.fn(*self.args, _stream_handle(None) if stream_handle is None else stream_handle)
        if st != MLA_OK:
            raise MlaError(st, self.what)
