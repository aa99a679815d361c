"""CPU oracle for dynamic block-sparse causal prefill attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or runs anything here, and this package imports nothing from it.

Thin ctypes marshalling over ``bsp_oracle.c`` (plain C, double precision,
OpenMP over rows).  Every function returns numpy arrays; see the C file for
the passages of the FlashPrefill summary page that each stage follows.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libbsp_oracle.so")
_DT = {"f32": 0, "bf16": 1, "fp8": 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into oracle/libbsp_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_pool.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp]
        L.oracle_score.argtypes = [i32, i32, i32, i32, vp, vp, dbl, vp, vp]
        L.oracle_mask.argtypes = [i32, i32, vp, vp, dbl, i32, i32, vp, vp, vp]
        L.oracle_key_radius.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_score_rescue.argtypes = [i32, i32, i32, i32, vp, vp, vp, dbl, vp, vp]
        L.oracle_mask_dual.argtypes = [i32, i32, vp, vp, dbl, dbl, i32, i32, vp, vp, vp]
        L.oracle_score_arith.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, dbl,
                                         ctypes.c_long, vp, vp]
        L.oracle_attn.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, dbl,
                                  vp, i64, vp, vp, vp]
        L.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        L.oracle_decode_e4m3fn.restype = dbl
        L.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_bf16.restype = dbl
        L.oracle_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    """OpenMP threads the last parallel call used."""
    return int(lib().oracle_threads())


def decode_e4m3fn(code: int) -> float:
    return float(lib().oracle_decode_e4m3fn(code))


def decode_bf16(bits: int) -> float:
    return float(lib().oracle_decode_bf16(bits))


def pool(x: np.ndarray, dtype: str, block: int, scales: Optional[np.ndarray] = None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    heads, seq, d = x.shape
    nb = -(-seq // block)
    out = np.empty((heads, nb, d), np.float64)
    sc = _c(scales, np.float32)
    lib().oracle_pool(heads, seq, d, block, _DT[dtype], _p(x), _p(sc), _p(out))
    return out


def score(qbar: np.ndarray, kbar: np.ndarray, c: float):
    """Returns (S, P), both [hq, nb, nb] float64, zero above the diagonal."""
    qbar = _c(qbar, np.float64)
    kbar = _c(kbar, np.float64)
    hq, nb, d = qbar.shape
    hkv = kbar.shape[0]
    S = np.empty((hq, nb, nb), np.float64)
    P = np.empty((hq, nb, nb), np.float64)
    lib().oracle_score(hq, hkv, nb, d, _p(qbar), _p(kbar), float(c), _p(S), _p(P))
    return S, P


def score_arith(q: np.ndarray, k: np.ndarray, dtype: str, block: int, c: float, hkv: int,
                q_scale=None, k_scale=None, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-query block approximation (see oracle_score_arith): P[h, I, J] is
    the mean over the tokens of block I of their softmax over the pooled key
    blocks J <= I.  rows: optional flat ids h*nb + I; then the result is
    [len(rows), nb], else [hq, nb, nb]."""
    q = np.ascontiguousarray(q)
    hq, seq, d = q.shape
    nb = -(-seq // block)
    kbar = pool(k, dtype, block, k_scale)
    assert kbar.shape[0] == hkv
    r = _c(rows, np.int64)
    n = hq * nb if r is None else r.shape[0]
    out = np.empty((n, nb), np.float64)
    lib().oracle_score_arith(hq, hkv, seq, d, block, _DT[dtype], _p(q),
                             _p(_c(q_scale, np.float32)), _p(kbar), float(c), n, _p(r), _p(out))
    return out.reshape(hq, nb, nb) if r is None else out


def key_radius(k: np.ndarray, dtype: str, block: int, k_scale=None) -> np.ndarray:
    """[hkv, nb]: max distance of a block's keys from their mean (the
    rescue-branch radius; see oracle_key_radius)."""
    k = np.ascontiguousarray(k)
    hkv, seq, d = k.shape
    kbar = pool(k, dtype, block, k_scale)
    r = np.empty((hkv, kbar.shape[1]), np.float64)
    lib().oracle_key_radius(hkv, seq, d, block, _DT[dtype], _p(k), _p(_c(k_scale, np.float32)),
                            _p(kbar), _p(r))
    return r


def score_rescue(qbar: np.ndarray, kbar: np.ndarray, radius: np.ndarray, c: float):
    """Rescue scores R = c (Qbar.Kbar + |Qbar| r) and their row softmax Pr,
    both [hq, nb, nb], zero above the diagonal."""
    qbar = _c(qbar, np.float64)
    kbar = _c(kbar, np.float64)
    hq, nb, d = qbar.shape
    R = np.empty((hq, nb, nb), np.float64)
    Pr = np.empty((hq, nb, nb), np.float64)
    lib().oracle_score_rescue(hq, kbar.shape[0], nb, d, _p(qbar), _p(kbar),
                              _p(_c(radius, np.float64)), float(c), _p(R), _p(Pr))
    return R, Pr


def mask_dual(P: np.ndarray, Pr: np.ndarray, gamma: float, gamma_r: float, sink_blocks: int = 1,
              local_blocks: int = 1):
    """Base and rescue branches thresholded independently and combined.
    Returns (mask, idx (-1 past cnt), cnt)."""
    P = _c(P, np.float64)
    Pr = _c(Pr, np.float64)
    hq, nb, _ = P.shape
    m = np.empty((hq, nb, nb), np.uint8)
    idx = np.empty((hq, nb, nb), np.int32)
    cnt = np.empty((hq, nb), np.int32)
    lib().oracle_mask_dual(hq, nb, _p(P), _p(Pr), float(gamma), float(gamma_r), sink_blocks,
                           local_blocks, _p(m), _p(idx), _p(cnt))
    return m, idx, cnt


def mask(P: Optional[np.ndarray], gamma: float, sink_blocks: int = 1, local_blocks: int = 1,
         user_mask: Optional[np.ndarray] = None, shape=None):
    """Returns (mask uint8, idx int32 (-1 past cnt), cnt int32)."""
    P = _c(P, np.float64)
    um = _c(user_mask, np.uint8)
    hq, nb, _ = (P if P is not None else um).shape
    m = np.empty((hq, nb, nb), np.uint8)
    idx = np.empty((hq, nb, nb), np.int32)
    cnt = np.empty((hq, nb), np.int32)
    lib().oracle_mask(hq, nb, _p(P), _p(um), float(gamma), sink_blocks, local_blocks,
                      _p(m), _p(idx), _p(cnt))
    return m, idx, cnt


def calibrate_gamma(P: np.ndarray, target: float, sink_blocks: int = 1, local_blocks: int = 1):
    """The threshold factor that keeps a target share of the causal blocks
    (FlashPrefill summary page, Appendix A "Hyperparameter Configurations":
    the single threshold hyperparameter is calibrated on computational
    density, with block size and structural retention fixed).

    Definition: density(gamma) = kept causal blocks / causal blocks under the
    mask rule (P >= gamma * row max, or forced), and the answer is the
    largest gamma in [0, 1] with density(gamma) >= target.  Written out: a
    causal block that is not forced is kept exactly when its ratio
    r = P / row max is at least gamma, so kept(gamma) = forced + #{r >= gamma}.
    If gamma = 1 already keeps the target, the answer is 1.  Otherwise it is
    the n-th largest ratio, n = (fewest kept blocks that reach the target) -
    forced: at that ratio n blocks are kept, and above it fewer than n.
    Returns (gamma, density) in float64."""
    P = np.asarray(P, np.float64)
    hq, nb, _ = P.shape
    I = np.arange(nb)[:, None]
    J = np.arange(nb)[None, :]
    causal = np.broadcast_to(J <= I, P.shape)
    forced = causal & np.broadcast_to((J < sink_blocks) | (I - J < local_blocks), P.shape)
    total = hq * nb * (nb + 1) // 2
    pmax = np.where(causal, P, -np.inf).max(-1, keepdims=True)
    ratio = P / pmax
    free = causal & ~forced
    n_forced = int(forced.sum())
    # fewest kept blocks k with k / total >= target, as the density compares
    k = max(0, int(math.ceil(target * total)) - 1)
    while k / total < target:
        k += 1
    at_one = n_forced + int((free & (ratio >= 1.0)).sum())
    if at_one >= k:
        return 1.0, at_one / total
    r = np.sort(ratio[free])[::-1]
    g = float(r[k - n_forced - 1])
    return g, (n_forced + int((r >= g).sum())) / total


def attn(q, k, v, dtype: str, block: int, block_mask: np.ndarray, sm_scale: Optional[float] = None,
         q_scale=None, k_scale=None, v_scale=None, rows: Optional[np.ndarray] = None):
    """Exact attention per query token over its kept, causally visible keys.
    rows: optional flat query ids h*seq + i.  Returns (out [n, d], lse [n]);
    with rows=None, out is [hq, seq, d] and lse [hq, seq]."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    hq, seq, d = q.shape
    hkv = k.shape[0]
    if sm_scale is None or sm_scale <= 0:
        sm_scale = 1.0 / math.sqrt(d)
    bm = _c(block_mask, np.uint8)
    r = _c(rows, np.int64)
    n = hq * seq if r is None else r.shape[0]
    out = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    lib().oracle_attn(hq, hkv, seq, d, block, _DT[dtype], _p(q), _p(k), _p(v),
                      _p(_c(q_scale, np.float32)), _p(_c(k_scale, np.float32)),
                      _p(_c(v_scale, np.float32)), float(sm_scale), _p(bm), n, _p(r),
                      _p(out), _p(lse))
    if r is None:
        return out.reshape(hq, seq, d), lse.reshape(hq, seq)
    return out, lse


def prefill(case, gamma: Optional[float] = None, sink_blocks: int = 1, local_blocks: int = 1,
            sm_scale: Optional[float] = None, rows=None, user_mask=None, with_attn=True):
    """All stages on a generated case (any object with the fields hq, hkv,
    seq, d, block, gamma, dtype, q, k, v, q_scale, k_scale, v_scale)."""
    g = case.gamma if gamma is None else gamma
    c = 1.0 / math.sqrt(case.d) if (sm_scale is None or sm_scale <= 0) else sm_scale
    qbar = pool(case.q, case.dtype, case.block, case.q_scale)
    kbar = pool(case.k, case.dtype, case.block, case.k_scale)
    S, P = score(qbar, kbar, c)
    m, idx, cnt = mask(None if user_mask is not None else P, g, sink_blocks, local_blocks,
                       user_mask=user_mask)
    res = dict(qbar=qbar, kbar=kbar, S=S, P=P, mask=m, idx=idx, cnt=cnt)
    if with_attn:
        res["out"], res["lse"] = attn(case.q, case.k, case.v, case.dtype, case.block, m, c,
                                      case.q_scale, case.k_scale, case.v_scale, rows=rows)
    return res
