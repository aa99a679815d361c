"""Shared helpers for the GPU parity tests: move generated cases to the
device, turn oracle masks into index lists, and compare with the bands and
tolerances the method's outputs are held to."""
import numpy as np
import torch

import block_sparse_attention_bsp_amd as bsp

# Max-abs tolerance of the attention output against the oracle, per input dtype.
# bf16 / fp8 are the stated bars for this method; fp32 follows from fp32 FMA
# accumulation over at most a few thousand keys.
O_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
LSE_TOL = {"f32": 1e-4, "bf16": 2e-3, "fp8": 2e-3}
MASK_BAND = 1e-4  # relative band around the threshold where the mask may differ


def dev(case):
    """Device tensors of a generated case (+ fp8 scales)."""
    def t(a):
        if case.dtype == "f32":
            return torch.from_numpy(a).cuda()
        if case.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()
    out = dict(q=t(case.q), k=t(case.k), v=t(case.v), q_scale=None, k_scale=None, v_scale=None)
    if case.dtype == "fp8":
        for n in ("q_scale", "k_scale", "v_scale"):
            out[n] = torch.from_numpy(getattr(case, n)).cuda()
    return out


def idx_from_mask(m: np.ndarray):
    """Ascending kept-block lists (-1 padded) and counts from a 0/1 block mask."""
    keep = m.astype(bool)
    idx = np.argsort(~keep, axis=-1, kind="stable").astype(np.int32)
    cnt = keep.sum(-1).astype(np.int32)
    pos = np.arange(m.shape[-1])[None, None, :]
    idx = np.where(pos < cnt[..., None], idx, -1).astype(np.int32)
    return idx, cnt


def band(P: np.ndarray, gamma: float, sink: int, local: int) -> np.ndarray:
    """Blocks whose keep/drop decision is within MASK_BAND of the threshold
    (and not forced): the only places a correct fp32 mask may differ."""
    hq, nb, _ = P.shape
    I = np.arange(nb)[:, None]
    J = np.arange(nb)[None, :]
    causal = J <= I
    pmax = np.where(causal, P, -np.inf).max(-1, keepdims=True)
    thr = gamma * pmax
    near = np.abs(P - thr) <= MASK_BAND * thr
    forced = (J < sink) | ((I - J) < local)
    return near & causal & ~forced


def check_mask(gm, gidx, gcnt, orc, gamma, sink=1, local=1):
    """Mask equal to the oracle's outside the band; idx/cnt consistent with
    the GPU mask everywhere and equal to the oracle's on rows without band
    blocks.  Returns the number of band blocks."""
    om = orc["mask"]
    b = band(orc["P"], gamma, sink, local)
    diff = gm != om
    assert not np.any(diff & ~b), f"{int((diff & ~b).sum())} mask blocks differ outside the band"
    want_idx, want_cnt = idx_from_mask(gm)
    assert np.array_equal(gcnt, want_cnt)
    keep = np.arange(gm.shape[-1])[None, None, :] < want_cnt[..., None]
    assert np.array_equal(np.where(keep, gidx, -1), want_idx)
    rows_clean = ~b.any(-1)
    assert np.array_equal(gcnt[rows_clean], orc["cnt"][rows_clean])
    return int(b.sum())


def sample_rows(hq, seq, block, n_pos=24, seed=0, heads=None):
    """Flat query ids h*seq + i: first/last tokens of the first and last
    blocks, a block boundary, plus random positions, for every head."""
    rng = np.random.default_rng(seed)
    pos = {0, 1, min(block - 1, seq - 1), min(block, seq - 1), seq - 1, max(seq - block, 0)}
    pos |= set(rng.integers(0, seq, n_pos).tolist())
    pos = np.array(sorted(pos), np.int64)
    hs = np.arange(hq) if heads is None else np.asarray(heads)
    return (hs[:, None] * seq + pos[None, :]).reshape(-1)


def gather_rows(o: torch.Tensor, lse: torch.Tensor, rows: np.ndarray):
    hq, seq, d = o.shape
    r = torch.from_numpy(rows).to(o.device)
    go = o.reshape(hq * seq, d).index_select(0, r).float().cpu().numpy()
    gl = lse.reshape(-1).index_select(0, r).cpu().numpy()
    return go, gl


def check_attn(go, gl, oo, ol, dtype):
    err = np.abs(go - oo).max() if go.size else 0.0
    assert err <= O_TOL[dtype], f"max-abs O error {err} > {O_TOL[dtype]}"
    fin = np.isfinite(ol)
    assert np.array_equal(np.isfinite(gl), fin)
    if fin.any():
        lerr = np.abs(gl[fin] - ol[fin]).max()
        assert lerr <= LSE_TOL[dtype], f"LSE error {lerr}"
    return float(err)


def run_gpu_prefill(case, gamma=None, sink=1, local=1, user_mask=None):
    d = dev(case)
    g = case.gamma if gamma is None else gamma
    um = None if user_mask is None else torch.from_numpy(user_mask).cuda()
    res = bsp.prefill(d["q"], d["k"], d["v"], case.block, g, sink_blocks=sink,
                      local_blocks=local, user_mask=um, q_scale=d["q_scale"],
                      k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    return d, res
