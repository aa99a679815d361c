"""Dynamic block-sparse causal prefill attention for AMD MI355X (gfx950).

Python binding of ``libbsp.so`` (include/bsp.h).  This module only marshals
arguments: torch provides device memory and the current stream, and every
step of the computation runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: if the library is missing, loading fails loudly.

Three stages, as on the FlashPrefill summary page (paperlayer.ai, Appendix B):
``score`` (pool + block scores), ``mask`` (max-based dynamic threshold +
index compaction) and ``attn_fwd`` (block-sparse online-softmax attention);
``prefill`` chains them.
"""
from __future__ import annotations

import ctypes
import itertools
import os
from typing import Optional

import torch

__all__ = [
    "BspError", "BspDesc", "lib", "library_path", "desc", "score", "mask", "attn_fwd", "prefill",
    "calibrate_gamma", "score_arith", "score_rescue", "mask_dual", "score_mask", "bsp_score",
    "bsp_score_arith", "bsp_score_mask",
    "bsp_score_rescue", "bsp_mask", "bsp_mask_dual", "bsp_attn_fwd", "bsp_calibrate_gamma",
    "BspVarlen", "bsp_attn_fwd_varlen", "attn_fwd_varlen", "bsp_score_varlen", "bsp_mask_varlen",
    "score_varlen", "mask_varlen", "prefill_varlen",
    "bsp_status_string", "bsp_abi_version", "bsp_widen_e4m3", "widen_e4m3",
    "DTYPE_F32", "DTYPE_BF16", "DTYPE_FP8_E4M3", "DTYPE_FP8_E4M3_V_BF16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libbsp.so")

DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3, DTYPE_FP8_E4M3_V_BF16 = 0, 1, 2, 3
_STATUS = {0: "BSP_OK", 1: "BSP_ERR_NULL_POINTER", 2: "BSP_ERR_BAD_SHAPE", 3: "BSP_ERR_BAD_DTYPE",
           4: "BSP_ERR_BAD_VALUE", 5: "BSP_ERR_UNSUPPORTED", 6: "BSP_ERR_HIP"}


class BspDesc(ctypes.Structure):
    """Mirror of ``bsp_desc`` in include/bsp.h."""
    _fields_ = [
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("seq", ctypes.c_int32),
        ("d", ctypes.c_int32), ("block", ctypes.c_int32), ("gamma", ctypes.c_float),
        ("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("sink_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class BspVarlen(ctypes.Structure):
    """Mirror of ``bsp_varlen`` in include/bsp.h."""
    _fields_ = [
        ("cu_seqlens", ctypes.c_void_p), ("cu_blocks", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("nseq", ctypes.c_int32),
        ("total_blocks", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("idx_stride", ctypes.c_int32), ("block_order", ctypes.c_void_p),
    ]


class BspError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """Load libbsp.so (built in-tree by block_sparse_attention_bsp_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run "
                               "`python -m block_sparse_attention_bsp_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, P = ctypes.c_void_p, ctypes.POINTER(BspDesc)
        L.bsp_score.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.bsp_mask.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.bsp_score_mask.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.bsp_score_arith.argtypes = [P, vp, vp, vp, vp, vp]
        L.bsp_score_rescue.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.bsp_mask_dual.argtypes = [P, vp, vp, ctypes.c_float, vp, vp, vp, vp]
        L.bsp_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.bsp_attn_fwd_varlen.argtypes = [P, ctypes.POINTER(BspVarlen), vp, vp, vp, vp, vp, vp,
                                          vp, vp]
        L.bsp_score_varlen.argtypes = [P, ctypes.POINTER(BspVarlen), vp, vp, vp, vp, vp, vp]
        L.bsp_mask_varlen.argtypes = [P, ctypes.POINTER(BspVarlen), vp, vp, vp, vp, vp, vp]
        L.bsp_widen_e4m3.argtypes = [vp, vp, ctypes.c_int64, vp]
        f32 = ctypes.c_float
        L.bsp_calibrate_gamma.argtypes = [P, vp, f32, f32, vp, vp, vp, vp,
                                          ctypes.POINTER(f32), ctypes.POINTER(f32), vp]
        for f in (L.bsp_score, L.bsp_score_mask, L.bsp_score_arith, L.bsp_score_rescue, L.bsp_mask,
                  L.bsp_mask_dual, L.bsp_attn_fwd, L.bsp_attn_fwd_varlen,
                  L.bsp_calibrate_gamma, L.bsp_score_varlen, L.bsp_mask_varlen,
                  L.bsp_widen_e4m3):
            f.restype = ctypes.c_int32
        L.bsp_status_string.argtypes = [ctypes.c_int32]
        L.bsp_status_string.restype = ctypes.c_char_p
        L.bsp_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


# ---------------------------------------------------------------- raw C ABI
def bsp_status_string(status: int) -> str:
    return lib().bsp_status_string(status).decode()


def bsp_abi_version() -> int:
    return int(lib().bsp_abi_version())


def _check(status: int):
    if status != 0:
        raise BspError(status, bsp_status_string(status))


def bsp_score(d: BspDesc, q, k, q_pool, k_pool, score_out, stream) -> int:
    return lib().bsp_score(ctypes.byref(d), q, k, q_pool, k_pool, score_out, stream)


def bsp_score_mask(d: BspDesc, q, k, q_pool, k_pool, score_out, mask_out, kv_idx, kv_cnt,
                   stream) -> int:
    return lib().bsp_score_mask(ctypes.byref(d), q, k, q_pool, k_pool, score_out, mask_out, kv_idx,
                                kv_cnt, stream)


def bsp_score_arith(d: BspDesc, q, k, k_pool, score_out, stream) -> int:
    return lib().bsp_score_arith(ctypes.byref(d), q, k, k_pool, score_out, stream)


def bsp_score_rescue(d: BspDesc, k, q_pool, k_pool, k_radius, rescue_out, stream) -> int:
    return lib().bsp_score_rescue(ctypes.byref(d), k, q_pool, k_pool, k_radius, rescue_out, stream)


def bsp_mask_dual(d: BspDesc, score_in, rescue_in, gamma_rescue: float, mask_out, kv_idx, kv_cnt,
                  stream) -> int:
    return lib().bsp_mask_dual(ctypes.byref(d), score_in, rescue_in, gamma_rescue, mask_out,
                               kv_idx, kv_cnt, stream)


def bsp_mask(d: BspDesc, score_in, user_mask, mask_out, kv_idx, kv_cnt, stream) -> int:
    return lib().bsp_mask(ctypes.byref(d), score_in, user_mask, mask_out, kv_idx, kv_cnt, stream)


def bsp_attn_fwd(d: BspDesc, q, k, v, kv_idx, kv_cnt, o, lse, stream) -> int:
    return lib().bsp_attn_fwd(ctypes.byref(d), q, k, v, kv_idx, kv_cnt, o, lse, stream)


def bsp_calibrate_gamma(d: BspDesc, score_in, target: float, tol: float, mask_out, kv_idx,
                        kv_cnt, cnt_host, gamma_out, density_out, stream) -> int:
    return lib().bsp_calibrate_gamma(ctypes.byref(d), score_in, target, tol, mask_out, kv_idx,
                                     kv_cnt, cnt_host, ctypes.byref(gamma_out),
                                     ctypes.byref(density_out), stream)


def bsp_attn_fwd_varlen(d: BspDesc, vl: BspVarlen, q, k_cache, v_cache, kv_idx, kv_cnt, o, lse,
                        stream) -> int:
    return lib().bsp_attn_fwd_varlen(ctypes.byref(d), ctypes.byref(vl), q, k_cache, v_cache,
                                     kv_idx, kv_cnt, o, lse, stream)


def bsp_score_varlen(d: BspDesc, vl: BspVarlen, q, k_cache, q_pool, k_pool, score_out,
                     stream) -> int:
    return lib().bsp_score_varlen(ctypes.byref(d), ctypes.byref(vl), q, k_cache, q_pool, k_pool,
                                  score_out, stream)


def bsp_mask_varlen(d: BspDesc, vl: BspVarlen, score_in, user_mask, mask_out, kv_idx, kv_cnt,
                    stream) -> int:
    return lib().bsp_mask_varlen(ctypes.byref(d), ctypes.byref(vl), score_in, user_mask, mask_out,
                                 kv_idx, kv_cnt, stream)


def bsp_widen_e4m3(src, dst, n: int, stream) -> int:
    return lib().bsp_widen_e4m3(src, dst, n, stream)


# ---------------------------------------------------------------- torch level
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DTYPE_FP8_E4M3
    raise BspError(3, f"unsupported tensor dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.numel() == 0:
        return None
    if not t.is_cuda:
        raise BspError(1, "tensors must be device tensors")
    if not t.is_contiguous():
        raise BspError(2, "tensors must be contiguous")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def desc(hq: int, hkv: int, seq: int, d: int, block: int, dtype: int, gamma: float = 0.0,
         sm_scale: float = 0.0, sink_blocks: int = 1, local_blocks: int = 1, causal: int = 1,
         q_scale=None, k_scale=None, v_scale=None) -> BspDesc:
    return BspDesc(hq, hkv, seq, d, block, gamma, sm_scale, causal, sink_blocks, local_blocks,
                   dtype, _ptr(q_scale), _ptr(k_scale), _ptr(v_scale))


def _shape(t: Optional[torch.Tensor], want, name: str):
    """Shape checks before the C call: the C ABI sees only pointers, so a
    tensor smaller than the descriptor says would be read out of bounds."""
    if t is not None and tuple(t.shape) != tuple(want):
        raise BspError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _is_e4m3(t: torch.Tensor) -> bool:
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def _desc_qkv(q, k, block, v=None, **kw):
    if q.dim() != 3 or k.dim() != 3:
        raise BspError(2, "q and k must be [heads, seq, d]")
    hq, seq, d = q.shape
    _shape(k, (k.shape[0], seq, d), "k")
    _shape(v, k.shape, "v")
    # e4m3 Q and K may come with V already widened to bf16 (widen_e4m3)
    v_wide = v is not None and _is_e4m3(q) and v.dtype == torch.bfloat16
    for t in (k, None if v_wide else v):
        if t is not None and t.dtype != q.dtype:
            raise BspError(3, "q, k and v must share one dtype (or v bf16 with e4m3 q and k)")
    for name, want in (("q_scale", hq), ("k_scale", k.shape[0]), ("v_scale", k.shape[0])):
        t = kw.get(name)
        _shape(t, (want,), name)
        if t is not None and t.dtype != torch.float32:
            raise BspError(3, f"{name} must be float32")
    code = DTYPE_FP8_E4M3_V_BF16 if v_wide else _dtype_code(q)
    return desc(hq, k.shape[0], seq, d, block, code, **kw)


def widen_e4m3(x: torch.Tensor, out=None) -> torch.Tensor:
    """bsp_widen_e4m3: the exact bf16 values of e4m3 codes (scales not applied)."""
    if not _is_e4m3(x):
        raise BspError(3, "widen_e4m3 takes e4m3 codes (uint8 or float8_e4m3fn)")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    elif tuple(out.shape) != tuple(x.shape) or out.dtype != torch.bfloat16:
        raise BspError(2, "out must be bf16 of the input's shape")
    _check(bsp_widen_e4m3(_ptr(x), _ptr(out), x.numel(), _stream()))
    return out


def score(q: torch.Tensor, k: torch.Tensor, block: int, sm_scale: float = 0.0,
          q_scale=None, k_scale=None):
    """Stage 1.  Returns (q_pool [hq,nb,d], k_pool [hkv,nb,d], score [hq,nb,nb]) fp32."""
    dsc = _desc_qkv(q, k, block, sm_scale=sm_scale, q_scale=q_scale, k_scale=k_scale)
    hq, seq, d = q.shape
    nb = -(-seq // block)
    qp = torch.empty((hq, nb, d), dtype=torch.float32, device=q.device)
    kp = torch.empty((k.shape[0], nb, d), dtype=torch.float32, device=q.device)
    sc = torch.empty((hq, nb, nb), dtype=torch.float32, device=q.device)
    _check(bsp_score(dsc, _ptr(q), _ptr(k), _ptr(qp), _ptr(kp), _ptr(sc), _stream()))
    return qp, kp, sc


def score_mask(q: torch.Tensor, k: torch.Tensor, block: int, gamma: float, sm_scale: float = 0.0,
               sink_blocks: int = 1, local_blocks: int = 1, q_scale=None, k_scale=None,
               want_mask: bool = True):
    """Stages 1 and 2 in one pass (bsp_score_mask): the outputs of score()
    followed by mask() without a caller mask.  Returns (q_pool, k_pool, score,
    mask or None, kv_idx, kv_cnt)."""
    dsc = _desc_qkv(q, k, block, gamma=gamma, sm_scale=sm_scale, sink_blocks=sink_blocks,
                    local_blocks=local_blocks, q_scale=q_scale, k_scale=k_scale)
    hq, seq, d = q.shape
    nb = -(-seq // block)
    dev = q.device
    qp = torch.empty((hq, nb, d), dtype=torch.float32, device=dev)
    kp = torch.empty((k.shape[0], nb, d), dtype=torch.float32, device=dev)
    sc = torch.empty((hq, nb, nb), dtype=torch.float32, device=dev)
    m = torch.empty((hq, nb, nb), dtype=torch.uint8, device=dev) if want_mask else None
    idx = torch.empty((hq, nb, nb), dtype=torch.int32, device=dev)
    cnt = torch.empty((hq, nb), dtype=torch.int32, device=dev)
    _check(bsp_score_mask(dsc, _ptr(q), _ptr(k), _ptr(qp), _ptr(kp), _ptr(sc), _ptr(m), _ptr(idx),
                          _ptr(cnt), _stream()))
    return qp, kp, sc, m, idx, cnt


def score_arith(q: torch.Tensor, k: torch.Tensor, block: int, sm_scale: float = 0.0,
                q_scale=None, k_scale=None):
    """Stage 1 with the per-query block approximation.  Returns
    (k_pool [hkv,nb,d], score [hq,nb,nb]) fp32."""
    dsc = _desc_qkv(q, k, block, sm_scale=sm_scale, q_scale=q_scale, k_scale=k_scale)
    hq, seq, d = q.shape
    nb = -(-seq // block)
    kp = torch.empty((k.shape[0], nb, d), dtype=torch.float32, device=q.device)
    sc = torch.empty((hq, nb, nb), dtype=torch.float32, device=q.device)
    _check(bsp_score_arith(dsc, _ptr(q), _ptr(k), _ptr(kp), _ptr(sc), _stream()))
    return kp, sc


def score_rescue(k: torch.Tensor, q_pool: torch.Tensor, k_pool: torch.Tensor, seq: int, block: int,
                 sm_scale: float = 0.0, k_scale=None):
    """Rescue branch.  Returns (k_radius [hkv,nb], rescue [hq,nb,nb]) fp32."""
    hq, nb, d = q_pool.shape
    hkv = k.shape[0]
    _shape(k, (hkv, seq, d), "k")
    _shape(k_pool, (hkv, nb, d), "k_pool")
    _shape(k_scale, (hkv,), "k_scale")
    if nb != -(-seq // block):
        raise BspError(2, "q_pool does not match seq and block")
    for t in (q_pool, k_pool):
        if t.dtype != torch.float32:
            raise BspError(3, "q_pool / k_pool must be float32")
    dsc = desc(hq, hkv, seq, d, block, _dtype_code(k), sm_scale=sm_scale, k_scale=k_scale)
    kr = torch.empty((hkv, nb), dtype=torch.float32, device=k.device)
    rs = torch.empty((hq, nb, nb), dtype=torch.float32, device=k.device)
    _check(bsp_score_rescue(dsc, _ptr(k), _ptr(q_pool), _ptr(k_pool), _ptr(kr), _ptr(rs),
                            _stream()))
    return kr, rs


def mask_dual(score_t: torch.Tensor, rescue_t: torch.Tensor, gamma: float, gamma_rescue: float,
              seq: int, block: int, sink_blocks: int = 1, local_blocks: int = 1,
              want_mask: bool = True):
    """Both branches thresholded and combined.  Returns (mask or None, kv_idx, kv_cnt)."""
    hq, nb, _ = score_t.shape
    if nb != -(-seq // block):
        raise BspError(2, "score does not match seq and block")
    for name, t in (("score", score_t), ("rescue", rescue_t)):
        _shape(t, (hq, nb, nb), name)
        if t.dtype != torch.float32:
            raise BspError(3, f"{name} must be float32")
    dsc = desc(hq, 1, seq, 64, block, DTYPE_F32, gamma=gamma, sink_blocks=sink_blocks,
               local_blocks=local_blocks)
    m = (torch.empty((hq, nb, nb), dtype=torch.uint8, device=score_t.device) if want_mask
         else None)
    idx = torch.empty((hq, nb, nb), dtype=torch.int32, device=score_t.device)
    cnt = torch.empty((hq, nb), dtype=torch.int32, device=score_t.device)
    _check(bsp_mask_dual(dsc, _ptr(score_t), _ptr(rescue_t), gamma_rescue, _ptr(m), _ptr(idx),
                         _ptr(cnt), _stream()))
    return m, idx, cnt


def mask(score_t: Optional[torch.Tensor], gamma: float, seq: int, block: int,
         sink_blocks: int = 1, local_blocks: int = 1, user_mask: Optional[torch.Tensor] = None,
         want_mask: bool = True):
    """Stage 2.  Returns (mask uint8 or None, kv_idx int32 [hq,nb,nb], kv_cnt int32 [hq,nb])."""
    ref = score_t if score_t is not None else user_mask
    hq, nb, _ = ref.shape
    if nb != -(-seq // block):
        raise BspError(2, "score / user_mask do not match seq and block")
    _shape(score_t, (hq, nb, nb), "score")
    _shape(user_mask, (hq, nb, nb), "user_mask")
    if score_t is not None and score_t.dtype != torch.float32:
        raise BspError(3, "score must be float32")
    if user_mask is not None and user_mask.dtype not in (torch.uint8, torch.bool):
        raise BspError(3, "user_mask must be uint8")
    dsc = desc(hq, 1, seq, 64, block, DTYPE_F32, gamma=gamma, sink_blocks=sink_blocks,
               local_blocks=local_blocks)
    m = torch.empty((hq, nb, nb), dtype=torch.uint8, device=ref.device) if want_mask else None
    idx = torch.empty((hq, nb, nb), dtype=torch.int32, device=ref.device)
    cnt = torch.empty((hq, nb), dtype=torch.int32, device=ref.device)
    _check(bsp_mask(dsc, _ptr(score_t), _ptr(user_mask), _ptr(m), _ptr(idx), _ptr(cnt), _stream()))
    return m, idx, cnt


def calibrate_gamma(score_t: torch.Tensor, seq: int, block: int, target: float,
                    tol: float = 1e-4, sink_blocks: int = 1, local_blocks: int = 1,
                    want_mask: bool = True):
    """Threshold factor for a target density (bsp_calibrate_gamma; blocks the
    host).  Returns (gamma, density, mask or None, kv_idx, kv_cnt) at that gamma."""
    hq, nb, _ = score_t.shape
    if nb != -(-seq // block):
        raise BspError(2, "score does not match seq and block")
    _shape(score_t, (hq, nb, nb), "score")
    if score_t.dtype != torch.float32:
        raise BspError(3, "score must be float32")
    dsc = desc(hq, 1, seq, 64, block, DTYPE_F32, sink_blocks=sink_blocks,
               local_blocks=local_blocks)
    m = (torch.empty((hq, nb, nb), dtype=torch.uint8, device=score_t.device) if want_mask
         else None)
    idx = torch.empty((hq, nb, nb), dtype=torch.int32, device=score_t.device)
    cnt = torch.empty((hq, nb), dtype=torch.int32, device=score_t.device)
    host = torch.empty((hq * nb,), dtype=torch.int32)
    g, dens = ctypes.c_float(), ctypes.c_float()
    _check(bsp_calibrate_gamma(dsc, _ptr(score_t), target, tol, _ptr(m), _ptr(idx), _ptr(cnt),
                               ctypes.c_void_p(host.data_ptr()), g, dens, _stream()))
    return g.value, dens.value, m, idx, cnt


def attn_fwd(q, k, v, block: int, kv_idx=None, kv_cnt=None, sm_scale: float = 0.0,
             q_scale=None, k_scale=None, v_scale=None, want_lse: bool = True, out=None, lse=None):
    """Stage 3.  Returns (o [hq,seq,d] fp32 for fp32 input else bf16, lse [hq,seq] fp32)."""
    dsc = _desc_qkv(q, k, block, v=v, sm_scale=sm_scale, q_scale=q_scale, k_scale=k_scale,
                    v_scale=v_scale)
    hq, seq, d = q.shape
    nb = -(-seq // block)
    _shape(kv_idx, (hq, nb, nb), "kv_idx")
    _shape(kv_cnt, (hq, nb), "kv_cnt")
    for t in (kv_idx, kv_cnt):
        if t is not None and t.dtype != torch.int32:
            raise BspError(3, "kv_idx / kv_cnt must be int32")
    odt = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    if out is not None and (tuple(out.shape) != (hq, seq, d) or out.dtype != odt):
        raise BspError(2, "out has the wrong shape or dtype")
    o = out if out is not None else torch.empty((hq, seq, d), dtype=odt, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((hq, seq), dtype=torch.float32, device=q.device)
    _shape(lse, (hq, seq), "lse")
    _check(bsp_attn_fwd(dsc, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), _ptr(o),
                        _ptr(lse), _stream()))
    return o, lse


def _varlen_meta(seqlens, block: int, ntok: int, device):
    """Lengths, per-sequence block counts, total blocks and the device offset
    arrays (cu_seqlens, cu_blocks) of a packed batch."""
    lens = [int(x) for x in seqlens]
    if not lens or min(lens) < 0:
        raise BspError(2, "seqlens must be a non-empty list of lengths >= 0")
    if ntok != sum(lens):
        raise BspError(2, "the token axis must equal sum(seqlens)")
    nbs = [-(-n // block) for n in lens]
    cu_s = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device=device)
    cu_b = torch.tensor([0] + list(itertools.accumulate(nbs)), dtype=torch.int32, device=device)
    return lens, nbs, sum(nbs), cu_s, cu_b


def _varlen_cache(q, k_cache, page_table, nbs, block: int):
    d = q.shape[2]
    if k_cache.dim() != 4 or k_cache.shape[2] != block or k_cache.shape[3] != d:
        raise BspError(2, "k_cache must be [pages, hkv, block, d]")
    if k_cache.dtype != q.dtype:
        raise BspError(3, "q and the caches must share one dtype")
    if (page_table.dim() != 2 or page_table.shape[0] != len(nbs)
            or page_table.dtype != torch.int32):
        raise BspError(2, "page_table must be int32 [nseq, max_pages]")
    if page_table.shape[1] < max(nbs + [1]):
        raise BspError(2, "page_table rows are shorter than a sequence's block count")


def score_varlen(q, k_cache, page_table, seqlens, block: int, sm_scale: float = 0.0,
                 q_scale=None, k_scale=None, idx_stride: Optional[int] = None):
    """Stage 1 for a packed batch over a paged K cache (bsp_score_varlen).
    Returns (q_pool [hq, total_blocks, d], k_pool [hkv, total_blocks, d],
    score [hq, total_blocks, idx_stride]); idx_stride defaults to the largest
    block count of a sequence.  Row entries past a sequence's block count are
    left as allocated."""
    hq, ntok, d = q.shape
    lens, nbs, tb, cu_s, cu_b = _varlen_meta(seqlens, block, ntok, q.device)
    _varlen_cache(q, k_cache, page_table, nbs, block)
    hkv = k_cache.shape[1]
    stride = max(nbs + [1]) if idx_stride is None else int(idx_stride)
    if stride < max(nbs + [1]):
        raise BspError(2, "idx_stride is smaller than a sequence's block count")
    _shape(q_scale, (hq,), "q_scale")
    _shape(k_scale, (hkv,), "k_scale")
    dsc = desc(hq, hkv, ntok, d, block, _dtype_code(q), sm_scale=sm_scale, q_scale=q_scale,
               k_scale=k_scale)
    vl = BspVarlen(_ptr(cu_s), _ptr(cu_b), _ptr(page_table), len(lens), tb, page_table.shape[1],
                   stride, None)
    qp = torch.empty((hq, tb, d), dtype=torch.float32, device=q.device)
    kp = torch.empty((hkv, tb, d), dtype=torch.float32, device=q.device)
    sc = torch.empty((hq, tb, stride), dtype=torch.float32, device=q.device)
    _check(bsp_score_varlen(dsc, vl, _ptr(q), _ptr(k_cache), _ptr(qp), _ptr(kp), _ptr(sc),
                            _stream()))
    return qp, kp, sc


def mask_varlen(score_t: Optional[torch.Tensor], gamma: float, seqlens, block: int,
                sink_blocks: int = 1, local_blocks: int = 1,
                user_mask: Optional[torch.Tensor] = None, want_mask: bool = True):
    """Stage 2 for a packed batch (bsp_mask_varlen).  score_t / user_mask:
    [hq, total_blocks, idx_stride].  Returns (mask uint8 or None, kv_idx int32
    [hq, total_blocks, idx_stride], kv_cnt int32 [hq, total_blocks]): the lists
    bsp_attn_fwd_varlen reads."""
    ref = score_t if score_t is not None else user_mask
    hq, tb_in, stride = ref.shape
    lens, nbs, tb, cu_s, cu_b = _varlen_meta(seqlens, block, sum(int(x) for x in seqlens),
                                             ref.device)
    if tb_in != tb or stride < max(nbs + [1]):
        raise BspError(2, "score / user_mask do not match seqlens and block")
    _shape(score_t, (hq, tb, stride), "score")
    _shape(user_mask, (hq, tb, stride), "user_mask")
    if score_t is not None and score_t.dtype != torch.float32:
        raise BspError(3, "score must be float32")
    if user_mask is not None and user_mask.dtype not in (torch.uint8, torch.bool):
        raise BspError(3, "user_mask must be uint8")
    dsc = desc(hq, 1, sum(lens), 64, block, DTYPE_F32, gamma=gamma, sink_blocks=sink_blocks,
               local_blocks=local_blocks)
    vl = BspVarlen(_ptr(cu_s), _ptr(cu_b), None, len(lens), tb, 1, stride, None)
    m = torch.zeros((hq, tb, stride), dtype=torch.uint8, device=ref.device) if want_mask else None
    idx = torch.empty((hq, tb, stride), dtype=torch.int32, device=ref.device)
    cnt = torch.empty((hq, tb), dtype=torch.int32, device=ref.device)
    _check(bsp_mask_varlen(dsc, vl, _ptr(score_t), _ptr(user_mask), _ptr(m), _ptr(idx),
                           _ptr(cnt), _stream()))
    return m, idx, cnt


def attn_fwd_varlen(q, k_cache, v_cache, page_table, seqlens, block: int, kv_idx=None,
                    kv_cnt=None, sm_scale: float = 0.0, q_scale=None, k_scale=None,
                    v_scale=None, want_lse: bool = True, block_order=None):
    """Packed variable-length batch over a paged cache (bsp_attn_fwd_varlen).
    q: [hq, sum(seqlens), d]; k_cache, v_cache: [pages, hkv, block, d];
    page_table: int32 [nseq, max_pages]; seqlens: host list of lengths;
    kv_idx: int32 [hq, total_blocks, stride] with kv_cnt [hq, total_blocks];
    block_order: optional int32 [total_blocks] launch order of the blocks.
    Returns (o, lse) over the packed tokens."""
    hq, ntok, d = q.shape
    lens, nbs, tb, cu_s, cu_b = _varlen_meta(seqlens, block, ntok, q.device)
    nseq = len(lens)
    _varlen_cache(q, k_cache, page_table, nbs, block)
    _shape(v_cache, k_cache.shape, "v_cache")
    hkv = k_cache.shape[1]
    v_wide = _is_e4m3(q) and v_cache.dtype == torch.bfloat16
    if k_cache.dtype != q.dtype or (v_cache.dtype != q.dtype and not v_wide):
        raise BspError(3, "q and the caches must share one dtype (or a bf16 v_cache with e4m3)")
    stride = 1
    if kv_idx is not None:
        if kv_idx.dim() != 3 or kv_idx.shape[:2] != (hq, tb) or kv_idx.dtype != torch.int32:
            raise BspError(2, "kv_idx must be int32 [hq, total_blocks, stride]")
        stride = kv_idx.shape[2]
        _shape(kv_cnt, (hq, tb), "kv_cnt")
        if kv_cnt.dtype != torch.int32:
            raise BspError(3, "kv_cnt must be int32")
    for name, t, want in (("q_scale", q_scale, hq), ("k_scale", k_scale, hkv),
                          ("v_scale", v_scale, hkv)):
        _shape(t, (want,), name)
    dsc = desc(hq, hkv, ntok, d, block, DTYPE_FP8_E4M3_V_BF16 if v_wide else _dtype_code(q),
               sm_scale=sm_scale, q_scale=q_scale, k_scale=k_scale, v_scale=v_scale)
    if block_order is not None:
        _shape(block_order, (tb,), "block_order")
        if block_order.dtype != torch.int32:
            raise BspError(3, "block_order must be int32")
    vl = BspVarlen(_ptr(cu_s), _ptr(cu_b), _ptr(page_table), nseq, tb, page_table.shape[1], stride,
                   _ptr(block_order))
    o = torch.empty((hq, ntok, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((hq, ntok), dtype=torch.float32, device=q.device) if want_lse else None
    _check(bsp_attn_fwd_varlen(dsc, vl, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_idx),
                               _ptr(kv_cnt), _ptr(o), _ptr(lse), _stream()))
    return o, lse


def prefill_varlen(q, k_cache, v_cache, page_table, seqlens, block: int, gamma: float,
                   sm_scale: float = 0.0, sink_blocks: int = 1, local_blocks: int = 1,
                   q_scale=None, k_scale=None, v_scale=None, widen_v: bool = False):
    """All three stages for a packed batch over a paged cache, on the current
    stream.  Returns a dict of every output.  widen_v: for an e4m3 cache,
    widen the V cache to bf16 first (every page, used or not; same outputs)."""
    out = {}
    if widen_v and _is_e4m3(v_cache):
        v_cache = widen_e4m3(v_cache)
    out["q_pool"], out["k_pool"], out["score"] = score_varlen(
        q, k_cache, page_table, seqlens, block, sm_scale, q_scale, k_scale)
    m, idx, cnt = mask_varlen(out["score"], gamma, seqlens, block, sink_blocks, local_blocks)
    o, lse = attn_fwd_varlen(q, k_cache, v_cache, page_table, seqlens, block, idx, cnt, sm_scale,
                             q_scale, k_scale, v_scale)
    out.update(mask=m, kv_idx=idx, kv_cnt=cnt, o=o, lse=lse)
    return out


def prefill(q, k, v, block: int, gamma: float, sm_scale: float = 0.0, sink_blocks: int = 1,
            local_blocks: int = 1, user_mask=None, q_scale=None, k_scale=None, v_scale=None,
            fused: bool = False, widen_v: bool = True):
    """All three stages on the current stream.  Returns a dict of every output.
    fused: stages 1 and 2 as one bsp_score_mask call (same outputs).
    widen_v: for e4m3 codes, widen V to bf16 first (bsp_widen_e4m3; the
    outputs are bit-identical, the attention launch faster)."""
    out = {}
    if widen_v and _is_e4m3(v):
        v = widen_e4m3(v)
    if fused and user_mask is None:
        (out["q_pool"], out["k_pool"], out["score"], m, idx, cnt) = score_mask(
            q, k, block, gamma, sm_scale, sink_blocks, local_blocks, q_scale, k_scale)
        o, lse = attn_fwd(q, k, v, block, idx, cnt, sm_scale, q_scale, k_scale, v_scale)
        out.update(mask=m, kv_idx=idx, kv_cnt=cnt, o=o, lse=lse)
        return out
    if user_mask is None:
        out["q_pool"], out["k_pool"], out["score"] = score(q, k, block, sm_scale, q_scale, k_scale)
    m, idx, cnt = mask(out.get("score"), gamma, q.shape[1], block, sink_blocks, local_blocks,
                       user_mask=user_mask)
    o, lse = attn_fwd(q, k, v, block, idx, cnt, sm_scale, q_scale, k_scale, v_scale)
    out.update(mask=m, kv_idx=idx, kv_cnt=cnt, o=o, lse=lse)
    return out
