"""Brute-force numpy references used to pin the oracle.

These are textbook definitions written independently of ``oracle/``: dense
L x L logits, token-level masks and a plain softmax.  They are only usable on
tiny inputs.  Decoding uses torch's own float8/bfloat16 conversions, so the
decoders are pinned against a library too.
"""
import math

import numpy as np
import torch


def decode(x: np.ndarray, dtype: str, scales=None) -> np.ndarray:
    """Storage bits -> float64 values (times per-head scales for fp8)."""
    if dtype == "f32":
        out = x.astype(np.float64)
    elif dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        out = t.to(torch.float64).numpy()
    elif dtype == "fp8":
        t = torch.from_numpy(np.ascontiguousarray(x)).view(torch.float8_e4m3fn)
        out = t.to(torch.float64).numpy()
    else:
        raise ValueError(dtype)
    if scales is not None:
        out = out * np.asarray(scales, np.float64)[:, None, None]
    return out


def values(case):
    return (decode(case.q, case.dtype, case.q_scale), decode(case.k, case.dtype, case.k_scale),
            decode(case.v, case.dtype, case.v_scale))


def dense_logits(q, k, hq, hkv, c):
    """[hq, L, L] = c * q_i . k_j with GQA head mapping."""
    grp = hq // hkv
    return np.stack([c * (q[h] @ k[h // grp].T) for h in range(hq)])


def token_mask(block_mask, seq, block):
    """Token-level visibility: kept block AND causal (j <= i)."""
    blk = np.arange(seq) // block
    m = block_mask[:, blk][:, :, blk].astype(bool)
    causal = np.tril(np.ones((seq, seq), bool))
    return m & causal[None]


def attention(q, k, v, hq, hkv, c, tmask):
    """Masked softmax attention; empty rows give 0 output and -inf LSE."""
    grp = hq // hkv
    L = dense_logits(q, k, hq, hkv, c)
    L = np.where(tmask, L, -np.inf)
    mx = L.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(mx)
    mx = np.where(empty, 0.0, mx)
    e = np.exp(L - mx)
    z = e.sum(-1, keepdims=True)
    p = np.where(empty, 0.0, e / np.where(z == 0, 1.0, z))
    out = np.stack([p[h] @ v[h // grp] for h in range(hq)])
    lse = np.where(empty[..., 0], -np.inf, (mx + np.log(np.where(z == 0, 1.0, z)))[..., 0])
    return out, lse


def block_tile_mean_logits(q, k, hq, hkv, c, block):
    """Mean of the dense logit tile over i in I and j in J (ragged-aware)."""
    seq = q.shape[1]
    nb = -(-seq // block)
    L = dense_logits(q, k, hq, hkv, c)
    out = np.zeros((hq, nb, nb))
    for I in range(nb):
        for J in range(nb):
            out[:, I, J] = L[:, I * block:(I + 1) * block, J * block:(J + 1) * block].mean(axis=(1, 2))
    return out


def causal_softmax_rows(S):
    """Row softmax over J <= I; 0 above the diagonal."""
    hq, nb, _ = S.shape
    P = np.zeros_like(S)
    for I in range(nb):
        s = S[:, I, :I + 1]
        e = np.exp(s - s.max(-1, keepdims=True))
        P[:, I, :I + 1] = e / e.sum(-1, keepdims=True)
    return P


def sm(d):
    return 1.0 / math.sqrt(d)
