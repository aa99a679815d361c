"""Seeded synthetic inputs for dynamic block-sparse causal prefill attention.

This module builds inputs only.  It holds none of the method's arithmetic
(no pooling, scoring, thresholding or attention): the CPU oracle and the HIP
library both consume what it returns, and neither is imported here.

Workloads follow the shapes of the FlashPrefill summary page (paperlayer.ai,
"FlashPrefill: Instantaneous Pattern Discovery and Thresholding for
Ultra-Fast Long-Context Prefilling", Appendix A: block size 128) and the five
layer shapes this library is measured on: a tiny fp32 case, a Llama-3-8B
shaped layer (32 q / 8 kv heads, d=128) at 4K, 32K and 128K in bf16, and a
Qwen-style layer (28 q / 4 kv heads) at 256K in fp8 e4m3 with per-head fp32
scales.  The planted "vertical" (column-invariant) and "slash" (constant
i-j) structure mirrors the pattern kinds named in section 3 of that page.

Recipe (every step seeded, numpy PCG64):
  * config i uses seed 1234 + i unless a seed is given;
  * draw order: for each kv head g: u_g (unit vector), the planted key
    positions (without replacement), then (slash only) an orthonormal pair
    e1_g, e2_g; then Q heads, K heads, V heads, each head one
    ``standard_normal((seq, d), float32)`` call, in that order;
  * RoPE (rotate-half convention, base 500000, positions 0..seq-1) is applied
    to Q and K before planting;
  * vertical planting: K[g, p] += s_v * u_g at the planted positions and
    Q[h, i] += s_q * u_{g(h)} for every i (s_v = 4, s_q = 1);
  * slash planting: r_g(i) = cos(w i) e1_g + sin(w i) e2_g with w = 2 pi / 2048;
    Q[h, i] += 3 r_{g(h)}(i) and K[g, j] += 3 r_g(j);
  * V is never planted;
  * cast: fp32 stays fp32; bf16 is fp32 -> bf16 round-to-nearest-even;
    fp8 is per-head scale = amax / 448, then round-to-nearest-even to OCP
    e4m3fn with saturation at +-448.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "CONFIGS", "Case", "make_config", "make_case", "make_s1", "make_s2",
    "random_block_mask", "bf16_bits", "e4m3fn_bits", "gqa_group",
]

ROPE_BASE = 500000.0
SLASH_PERIOD = 2048
E4M3_MAX = 448.0

# The five measured layer shapes.  ``n_vert`` planted key columns; ``slash``
# adds the rotating shared vector.  gamma is the threshold factor.
CONFIGS = [
    dict(name="tiny", hq=2, hkv=1, seq=1024, d=64, block=64, gamma=0.1,
         dtype="f32", rope=False, n_vert=4, slash=False),
    dict(name="llama_4k", hq=32, hkv=8, seq=4096, d=128, block=128, gamma=0.1,
         dtype="bf16", rope=True, n_vert=16, slash=False),
    dict(name="llama_32k", hq=32, hkv=8, seq=32768, d=128, block=128, gamma=0.05,
         dtype="bf16", rope=True, n_vert=32, slash=True),
    dict(name="llama_128k", hq=32, hkv=8, seq=131072, d=128, block=128, gamma=0.05,
         dtype="bf16", rope=True, n_vert=32, slash=True),
    dict(name="qwen_256k", hq=28, hkv=4, seq=262144, d=128, block=128, gamma=0.05,
         dtype="fp8", rope=True, n_vert=32, slash=True),
]


@dataclasses.dataclass
class Case:
    """One generated layer.  q/k/v hold the storage bits:
    float32 arrays (f32), uint16 bf16 bit patterns (bf16) or uint8 e4m3fn
    codes (fp8); shape [heads, seq, d], C order."""
    name: str
    hq: int
    hkv: int
    seq: int
    d: int
    block: int
    gamma: float
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_scale: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    seed: int = 0

    @property
    def nb(self) -> int:
        return -(-self.seq // self.block)


def gqa_group(h: int, hq: int, hkv: int) -> int:
    """kv head read by q head h (contiguous groups of hq/hkv q heads)."""
    return h // (hq // hkv)


# ----------------------------------------------------------------------------
# storage encoders (input construction: the bits both sides read)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.
    Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    return (r >> np.uint32(16)).astype(np.uint16)


def e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """float32 (already divided by the scale) -> OCP e4m3fn codes.
    1 sign, 4 exponent (bias 7), 3 mantissa bits; round to nearest even;
    magnitudes above 448 saturate to 448 (code 0x7E); 0x7F is never made."""
    x = np.asarray(x, dtype=np.float32)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(x), np.float32(E4M3_MAX)).astype(np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(20)) & np.uint32(1)
    r = (u + np.uint32(0x7FFFF) + lsb) & np.uint32(0xFFF00000)
    exp = (r >> np.uint32(23)).astype(np.int32) - 127 + 7
    man = ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32)
    normal = (np.clip(exp, 0, 15) << 3) | man
    # below 2^-6: multiples of 2^-9; rint is ties-to-even; 8 -> code 0x08 = 2^-6
    sub = np.rint(a * np.float32(512.0)).astype(np.int32)
    code = np.where(a < np.float32(2.0 ** -6), sub, normal).astype(np.uint8)
    return code | sign


# ----------------------------------------------------------------------------
# generator pieces
# ----------------------------------------------------------------------------
def _unit(rng, d):
    v = rng.standard_normal(d)
    return (v / np.linalg.norm(v)).astype(np.float32)


def _orthonormal_pair(rng, d):
    a = rng.standard_normal(d)
    b = rng.standard_normal(d)
    a = a / np.linalg.norm(a)
    b = b - np.dot(a, b) * a
    b = b / np.linalg.norm(b)
    return a.astype(np.float32), b.astype(np.float32)


def _rope_tables(seq, d):
    half = d // 2
    inv = ROPE_BASE ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(seq, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _rope(x, cos, sin):
    half = x.shape[-1] // 2
    x1 = x[:, :half].copy()
    x2 = x[:, half:].copy()
    x[:, :half] = x1 * cos - x2 * sin
    x[:, half:] = x2 * cos + x1 * sin
    return x


def _slash(seq, e1, e2):
    w = 2.0 * math.pi / SLASH_PERIOD
    t = np.arange(seq, dtype=np.float64) * w
    return (np.cos(t)[:, None].astype(np.float32) * e1[None, :]
            + np.sin(t)[:, None].astype(np.float32) * e2[None, :])


class _Store:
    """Per-head encoder into the storage dtype."""

    def __init__(self, dtype, heads, seq, d):
        self.dtype = dtype
        if dtype == "f32":
            self.arr = np.empty((heads, seq, d), np.float32)
        elif dtype == "bf16":
            self.arr = np.empty((heads, seq, d), np.uint16)
        elif dtype == "fp8":
            self.arr = np.empty((heads, seq, d), np.uint8)
            self.scale = np.empty(heads, np.float32)
        else:
            raise ValueError(dtype)

    def put(self, h, x):
        if self.dtype == "f32":
            self.arr[h] = x
        elif self.dtype == "bf16":
            self.arr[h] = bf16_bits(x)
        else:
            amax = np.float32(np.max(np.abs(x)))
            s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
            self.scale[h] = s
            self.arr[h] = e4m3fn_bits(x / s)


def make_case(hq, hkv, seq, d, block, dtype, seed, *, gamma=0.1, rope=False,
              n_vert=0, slash=False, strength=1.0, block_offset=0.0,
              name="case") -> Case:
    """General planted generator (see the module docstring for the recipe).

    strength multiplies every planted vector (1 for the measured configs;
    d**0.25 turns the stated strengths into softmax-logit units).
    block_offset > 0 adds, after the recipe above, a per-block offset
    a[h, I] ~ N(0, block_offset^2 I_d) to every query of block I and
    b[g, J] ~ N(0, block_offset^2 I_d) to every key of block J."""
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    rng = np.random.Generator(np.random.PCG64(seed))
    us, pos, es = [], [], []
    for _g in range(hkv):
        us.append(_unit(rng, d))
        nv = min(n_vert, seq)
        pos.append(np.sort(rng.choice(seq, size=nv, replace=False)) if nv else
                   np.zeros(0, np.int64))
        es.append(_orthonormal_pair(rng, d) if slash else None)
    cos = sin = None
    if rope:
        cos, sin = _rope_tables(seq, d)
    slash_cache = {}

    def slash_vec(g):
        if g not in slash_cache:
            slash_cache[g] = _slash(seq, *es[g])
        return slash_cache[g]

    nb = -(-seq // block)
    grp = hq // hkv
    qs = _Store(dtype, hq, seq, d)
    ks = _Store(dtype, hkv, seq, d)
    vs = _Store(dtype, hkv, seq, d)
    # Q, K, V draws happen before the block offsets, in this order.
    raw_q = [rng.standard_normal((seq, d), dtype=np.float32) for _ in range(hq)] \
        if block_offset else None
    for h in range(hq):
        x = raw_q[h] if raw_q is not None else rng.standard_normal((seq, d), dtype=np.float32)
        g = h // grp
        if rope:
            _rope(x, cos, sin)
        if n_vert:
            x += np.float32(strength) * us[g][None, :]
        if slash:
            x += np.float32(3.0 * strength) * slash_vec(g)
        if raw_q is not None:
            raw_q[h] = x
        else:
            qs.put(h, x)
    raw_k = []
    for g in range(hkv):
        x = rng.standard_normal((seq, d), dtype=np.float32)
        if rope:
            _rope(x, cos, sin)
        if n_vert:
            x[pos[g]] += np.float32(4.0 * strength) * us[g][None, :]
        if slash:
            x += np.float32(3.0 * strength) * slash_vec(g)
        if block_offset:
            raw_k.append(x)
        else:
            ks.put(g, x)
    for g in range(hkv):
        vs.put(g, rng.standard_normal((seq, d), dtype=np.float32))
    if block_offset:
        a = rng.standard_normal((hq, nb, d)).astype(np.float32) * np.float32(block_offset)
        b = rng.standard_normal((hkv, nb, d)).astype(np.float32) * np.float32(block_offset)
        blk = np.arange(seq) // block
        for h in range(hq):
            qs.put(h, raw_q[h] + a[h][blk])
        for g in range(hkv):
            ks.put(g, raw_k[g] + b[g][blk])
    return Case(name=name, hq=hq, hkv=hkv, seq=seq, d=d, block=block, gamma=gamma,
                dtype=dtype, q=qs.arr, k=ks.arr, v=vs.arr,
                q_scale=getattr(qs, "scale", None), k_scale=getattr(ks, "scale", None),
                v_scale=getattr(vs, "scale", None), seed=seed)


def make_config(i: int, seed: Optional[int] = None, seq: Optional[int] = None) -> Case:
    """Measured layer config i (0..4).  ``seq`` may shrink the sequence for
    quick tests (same heads, d, B, gamma, dtype and planting recipe)."""
    c = CONFIGS[i]
    s = 1234 + i if seed is None else seed
    return make_case(c["hq"], c["hkv"], c["seq"] if seq is None else seq, c["d"],
                     c["block"], c["dtype"], s, gamma=c["gamma"], rope=c["rope"],
                     n_vert=c["n_vert"], slash=c["slash"], name=c["name"])


def make_s1(seed: int) -> Case:
    """Mask test case on the tiny shape: config 0's recipe plus per-block
    offsets of scale 1.5, so block scores spread and masks are nonuniform."""
    c = CONFIGS[0]
    return make_case(c["hq"], c["hkv"], c["seq"], c["d"], c["block"], c["dtype"], seed,
                     gamma=c["gamma"], rope=False, n_vert=c["n_vert"], slash=False,
                     block_offset=1.5, name=f"s1_seed{seed}")


def make_s2(i: int, seq: Optional[int] = None) -> Case:
    """Configs 2/3 with every planted vector scaled by d**0.25, so the stated
    strengths are bumps in softmax-logit units."""
    c = CONFIGS[i]
    return make_case(c["hq"], c["hkv"], c["seq"] if seq is None else seq, c["d"],
                     c["block"], c["dtype"], 1234 + i, gamma=c["gamma"], rope=c["rope"],
                     n_vert=c["n_vert"], slash=c["slash"], strength=c["d"] ** 0.25,
                     name=c["name"] + "_s2")


def random_block_mask(hq: int, nb: int, density: float, seed: int,
                      sink_blocks: int = 1, local_blocks: int = 1) -> np.ndarray:
    """Caller-supplied block mask [hq, nb, nb] uint8 for kernel-efficiency
    sweeps: each causal off-structure block kept with probability ``density``,
    sink and local (diagonal) blocks always set, upper triangle zero."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = (rng.random((hq, nb, nb)) < density)
    I = np.arange(nb)[:, None]
    J = np.arange(nb)[None, :]
    m |= (J < sink_blocks) | ((I - J) < local_blocks)
    m &= (J <= I)
    return m.astype(np.uint8)
