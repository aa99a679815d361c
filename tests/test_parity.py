"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
small and medium seeded inputs: every stage, every dtype, several tiles,
ragged tails, sparse masks and the method's degenerate cases."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_bsp_amd as bsp
import gen
import oracle
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def full_check(case, gamma=None, sink=1, local=1, rows=None):
    """Stages 1-2 on every block; stage 3 given the oracle's mask."""
    g = case.gamma if gamma is None else gamma
    d, res = H.run_gpu_prefill(case, gamma=g, sink=sink, local=local)
    orc = oracle.prefill(case, gamma=g, sink_blocks=sink, local_blocks=local, with_attn=False)
    np.testing.assert_allclose(res["q_pool"].cpu().numpy(), orc["qbar"], rtol=1e-5, atol=2e-6)
    np.testing.assert_allclose(res["k_pool"].cpu().numpy(), orc["kbar"], rtol=1e-5, atol=2e-6)
    np.testing.assert_allclose(res["score"].cpu().numpy(), orc["P"], rtol=1e-4, atol=1e-6)
    nband = H.check_mask(res["mask"].cpu().numpy(), res["kv_idx"].cpu().numpy(),
                         res["kv_cnt"].cpu().numpy(), orc, g, sink, local)
    # attention given the oracle's mask
    idx, cnt = H.idx_from_mask(orc["mask"])
    o, lse = bsp.attn_fwd(d["q"], d["k"], d["v"], case.block, torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), q_scale=d["q_scale"],
                          k_scale=d["k_scale"], v_scale=d["v_scale"])
    torch.cuda.synchronize()
    oo, ol = oracle.attn(case.q, case.k, case.v, case.dtype, case.block, orc["mask"],
                         q_scale=case.q_scale, k_scale=case.k_scale, v_scale=case.v_scale,
                         rows=rows)
    if rows is None:
        go = o.float().cpu().numpy().reshape(-1, case.d)
        gl = lse.cpu().numpy().reshape(-1)
        oo = oo.reshape(-1, case.d)
        ol = ol.reshape(-1)
    else:
        go, gl = H.gather_rows(o, lse, rows)
    err = H.check_attn(go, gl, oo, ol, case.dtype)
    dens = orc["mask"].sum() / (case.hq * case.nb * (case.nb + 1) / 2)
    print(f"  density {dens:.3f} band blocks {nband} max-abs O err {err:.2e}", flush=True)
    return res, orc


def test_config0_tiny_fp32():
    announce("config 0 tiny fp32")
    full_check(gen.make_config(0))


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_s1_sparse_masks_fp32(seed):
    announce(f"S1 seed {seed}")
    full_check(gen.make_s1(seed))


@pytest.mark.parametrize("dtype,d,block,seq", [
    ("bf16", 128, 128, 1000), ("bf16", 64, 64, 777), ("bf16", 128, 64, 640),
    ("bf16", 64, 128, 513), ("fp8", 128, 128, 1000), ("fp8", 64, 64, 700),
    ("f32", 128, 128, 300), ("f32", 64, 128, 250), ("f32", 128, 64, 333),
])
def test_sparse_ragged_shapes(dtype, d, block, seq):
    announce(f"sparse ragged {dtype} d={d} B={block} seq={seq}")
    c = gen.make_case(8, 2, seq, d, block, dtype, 42 + seq, gamma=0.2, rope=True, n_vert=6,
                      slash=True, block_offset=1.0)
    full_check(c)


@pytest.mark.parametrize("dtype,hq,hkv,seq", [
    ("bf16", 6, 3, 900), ("fp8", 6, 3, 900), ("bf16", 7, 7, 640), ("bf16", 12, 6, 1280),
    ("fp8", 10, 5, 1024), ("bf16", 16, 16, 512),
])
def test_head_layouts_outside_the_xcd_grouping(dtype, hq, hkv, seq):
    """Head counts whose kv groups do not divide the 8 XCDs (the plain
    workgroup order) and large MHA: every row against the oracle."""
    announce(f"heads {hq}/{hkv} {dtype} seq={seq}")
    c = gen.make_case(hq, hkv, seq, 128, 128, dtype, 300 + hq + seq, gamma=0.2, rope=True,
                      n_vert=4, slash=True, block_offset=1.0)
    full_check(c)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_config_shape_4k_sampled(dtype):
    """Config 1 (or config 4's heads/dtype) at seq 4096: every head, sampled rows."""
    announce(f"4K {dtype}")
    c = gen.make_config(1) if dtype == "bf16" else gen.make_config(4, seq=4096)
    rows = H.sample_rows(c.hq, c.seq, c.block, n_pos=16)
    full_check(c, rows=rows)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_long_kv_lists(dtype):
    """Rows whose kv lists are long enough to span several 64-entry chunks:
    exact counts around 64 and 128, random rows, and lists padded with
    entries outside [0, I] that must be skipped."""
    announce(f"long kv lists {dtype}")
    c = gen.make_case(2, 1, 260 * 64, 64, 64, dtype, 77, rope=True, n_vert=4)
    nb = c.nb
    rng = np.random.default_rng(3)
    m = (rng.random((2, nb, nb)) < 0.6).astype(np.uint8) & np.tril(np.ones((nb, nb), np.uint8))
    special = {200: 63, 201: 64, 202: 65, 203: 127, 204: 128, 205: 129, 259: 130}
    for I, kk in special.items():
        m[0, I, :] = 0
        m[0, I, :kk] = 1
    idx, cnt = H.idx_from_mask(m)
    # head 1, rows 100..139: two entries the kernel must skip, at random places
    bad = idx.copy()
    bcnt = cnt.copy()
    for I in range(100, 140):
        lst = list(bad[1, I, :bcnt[1, I]])
        for x in (-1, I + 1 + int(rng.integers(0, nb - I - 1))):
            lst.insert(int(rng.integers(0, len(lst) + 1)), x)
        bad[1, I, :len(lst)] = lst
        bcnt[1, I] = len(lst)
    d = H.dev(c)
    kw = dict(q_scale=d["q_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"])
    o, lse = bsp.attn_fwd(d["q"], d["k"], d["v"], c.block, torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), **kw)
    o2, lse2 = bsp.attn_fwd(d["q"], d["k"], d["v"], c.block, torch.from_numpy(bad).cuda(),
                            torch.from_numpy(bcnt).cuda(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    B = c.block
    pos = [I * B + t for I in special for t in (0, 17, B - 1)]
    pos += [I * B + t for I in (100, 120, 139) for t in (0, B - 1)]
    pos += rng.integers(0, c.seq, 24).tolist()
    pos = np.array(sorted(set(pos)), np.int64)
    rows = np.concatenate([pos, c.seq + pos])
    oo, ol = oracle.attn(c.q, c.k, c.v, dtype, B, m, q_scale=c.q_scale, k_scale=c.k_scale,
                         v_scale=c.v_scale, rows=rows)
    go, gl = H.gather_rows(o, lse, rows)
    err = H.check_attn(go, gl, oo, ol, dtype)
    print(f"  max-abs O err {err:.2e}", flush=True)


def _arith_case(which):
    if which.startswith("s1_"):
        return gen.make_s1(int(which[-1]))
    if which == "llama_4k":
        return gen.make_config(1)
    if which == "qwen_4k_fp8":
        return gen.make_config(4, seq=4096)
    dtype, d, block, seq = which.split("_")
    return gen.make_case(8, 2, int(seq), int(d), int(block), dtype, 7 + int(seq), gamma=0.2,
                         rope=True, n_vert=6, slash=True, block_offset=1.0)


@pytest.mark.parametrize("which", ["s1_0", "s1_3", "bf16_128_128_1000", "bf16_64_64_777",
                                   "fp8_128_128_1000", "fp8_64_64_700", "f32_128_64_333",
                                   "f32_64_128_250", "llama_4k", "qwen_4k_fp8"])
def test_score_arith_matches_oracle(which):
    """Per-query block-approximation scores and the mask built on them."""
    announce(f"arithmetic scorer {which}")
    c = _arith_case(which)
    d = H.dev(c)
    kp, sc = bsp.score_arith(d["q"], d["k"], c.block, q_scale=d["q_scale"], k_scale=d["k_scale"])
    g = c.gamma
    m, idx, cnt = bsp.mask(sc, g, c.seq, c.block)
    torch.cuda.synchronize()
    cs = 1.0 / math.sqrt(c.d)
    P = oracle.score_arith(c.q, c.k, c.dtype, c.block, cs, c.hkv, c.q_scale, c.k_scale)
    np.testing.assert_allclose(kp.cpu().numpy(), oracle.pool(c.k, c.dtype, c.block, c.k_scale),
                               rtol=1e-5, atol=2e-6)
    np.testing.assert_allclose(sc.cpu().numpy(), P, rtol=1e-4, atol=1e-6)
    om, oidx, ocnt = oracle.mask(P, g)
    nband = H.check_mask(m.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
                         dict(P=P, mask=om, idx=oidx, cnt=ocnt), g)
    dens = om.sum() / (c.hq * c.nb * (c.nb + 1) / 2)
    print(f"  density {dens:.3f} band blocks {nband}", flush=True)


def _check_dual(gm, gidx, gcnt, P, Pr, g, gr, om, ocnt, sink=1, local=1):
    """Dual mask equal to the oracle's outside either branch's band."""
    b = H.band(P, g, sink, local) | H.band(Pr, gr, sink, local)
    diff = gm != om
    assert not np.any(diff & ~b), f"{int((diff & ~b).sum())} blocks differ outside the bands"
    want_idx, want_cnt = H.idx_from_mask(gm)
    assert np.array_equal(gcnt, want_cnt)
    keep = np.arange(gm.shape[-1])[None, None, :] < want_cnt[..., None]
    assert np.array_equal(np.where(keep, gidx, -1), want_idx)
    clean = ~b.any(-1)
    assert np.array_equal(gcnt[clean], ocnt[clean])
    return int(b.sum())


@pytest.mark.parametrize("which", ["s1_0", "s1_2", "bf16_128_128_1000", "bf16_64_64_777",
                                   "fp8_128_128_1000", "fp8_64_64_700", "f32_128_64_333",
                                   "llama_4k", "qwen_4k_fp8"])
def test_rescue_branch_matches_oracle(which):
    """Key-block radii, rescue scores and the dual-branch mask."""
    announce(f"rescue branch {which}")
    c = _arith_case(which)
    d = H.dev(c)
    qp, kp, sc = bsp.score(d["q"], d["k"], c.block, q_scale=d["q_scale"], k_scale=d["k_scale"])
    kr, rs = bsp.score_rescue(d["k"], qp, kp, c.seq, c.block, k_scale=d["k_scale"])
    g, gr = c.gamma, 0.5
    m, idx, cnt = bsp.mask_dual(sc, rs, g, gr, c.seq, c.block)
    torch.cuda.synchronize()
    cs = 1.0 / math.sqrt(c.d)
    qb = oracle.pool(c.q, c.dtype, c.block, c.q_scale)
    kb = oracle.pool(c.k, c.dtype, c.block, c.k_scale)
    _, P = oracle.score(qb, kb, cs)
    r = oracle.key_radius(c.k, c.dtype, c.block, c.k_scale)
    _, Pr = oracle.score_rescue(qb, kb, r, cs)
    np.testing.assert_allclose(kr.cpu().numpy(), r, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(rs.cpu().numpy(), Pr, rtol=1e-4, atol=1e-6)
    om, oidx, ocnt = oracle.mask_dual(P, Pr, g, gr)
    nband = _check_dual(m.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), P, Pr, g, gr, om,
                        ocnt)
    base = oracle.mask(P, g)[0].sum()
    print(f"  kept {om.sum()} (base alone {base}), band blocks {nband}", flush=True)


def _pooled_accuracy_case(which):
    """Planted block offsets (scores spread over several logits), several
    32-block tiles with a ragged last one."""
    dtype, d, block, nb = which.split("_")
    d, block, nb = int(d), int(block), int(nb)
    return gen.make_case(4, 2, block * nb - block // 3, d, block, dtype, 11 + nb, gamma=0.2,
                         n_vert=4, block_offset=1.5)


@pytest.mark.parametrize("which", ["f32_64_64_100", "bf16_128_128_70", "fp8_128_128_45",
                                   "bf16_64_128_130", "bf16_64_64_1100", "fp8_128_128_1030"])
@pytest.mark.parametrize("rescue", [False, True])
def test_pooled_scores_at_fp32_accuracy(which, rescue):
    """The pooled scores are as accurate as fp32 dot products (rows of 45 to
    1100 blocks, whole and ragged last tiles).

    Where P is at least 1e-6 of its row maximum, log P is within
    2e-6 + 2^-20 * c * sum_i |Qbar_i Kbar_i| of the fp64 oracle: the size of
    an fp32 accumulation error.  Products that drop a bf16 plane term err by
    about 2^-16 of that sum, sixteen times the bound."""
    announce(f"pooled score accuracy {which} rescue={rescue}")
    c = _pooled_accuracy_case(which)
    d = H.dev(c)
    qp, kp, sc = bsp.score(d["q"], d["k"], c.block, q_scale=d["q_scale"], k_scale=d["k_scale"])
    cs = 1.0 / math.sqrt(c.d)
    qb = oracle.pool(c.q, c.dtype, c.block, c.q_scale)
    kb = oracle.pool(c.k, c.dtype, c.block, c.k_scale)
    grp = c.hq // c.hkv
    mag = np.stack([np.abs(qb[h]) @ np.abs(kb[h // grp]).T for h in range(c.hq)]) * cs
    if rescue:
        kr, sc = bsp.score_rescue(d["k"], qp, kp, c.seq, c.block, k_scale=d["k_scale"])
        r = oracle.key_radius(c.k, c.dtype, c.block, c.k_scale)
        _, P = oracle.score_rescue(qb, kb, r, cs)
        qn = np.sqrt((qb.astype(np.float64) ** 2).sum(-1))
        mag = mag + cs * qn[:, :, None] * r[np.arange(c.hq) // grp][:, None, :]
    else:
        _, P = oracle.score(qb, kb, cs)
    torch.cuda.synchronize()
    G = sc.cpu().numpy().astype(np.float64)
    sel = P >= 1e-6 * P.max(-1, keepdims=True)
    sel &= np.tril(np.ones(P.shape[-2:], bool))[None]
    err = np.abs(np.log(G[sel]) - np.log(P[sel]))
    tol = 2e-6 + 2.0 ** -20 * mag[sel]
    worst = float((err / tol).max())
    print(f"  nb {c.nb} max |dlog P| {err.max():.2e}, worst err/tol {worst:.3f}", flush=True)
    assert worst <= 1.0


def test_long_rows_over_2048_blocks():
    """nb = 2188: rows longer than 2048 blocks (the general mask path), base and
    rescue branches, against the oracle."""
    announce("long rows nb=2188")
    c = gen.make_case(2, 1, 2188 * 64, 64, 64, "bf16", 21, gamma=0.2, rope=True, n_vert=8,
                      slash=True, block_offset=1.0)
    d = H.dev(c)
    qp, kp, sc = bsp.score(d["q"], d["k"], c.block)
    m, idx, cnt = bsp.mask(sc, c.gamma, c.seq, c.block)
    kr, rs = bsp.score_rescue(d["k"], qp, kp, c.seq, c.block)
    md, idxd, cntd = bsp.mask_dual(sc, rs, c.gamma, 0.5, c.seq, c.block)
    torch.cuda.synchronize()
    cs = 1.0 / math.sqrt(c.d)
    qb = oracle.pool(c.q, c.dtype, c.block)
    kb = oracle.pool(c.k, c.dtype, c.block)
    _, P = oracle.score(qb, kb, cs)
    np.testing.assert_allclose(sc.cpu().numpy(), P, rtol=1e-4, atol=1e-6)
    om, oidx, ocnt = oracle.mask(P, c.gamma)
    H.check_mask(m.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
                 dict(P=P, mask=om, idx=oidx, cnt=ocnt), c.gamma)
    r = oracle.key_radius(c.k, c.dtype, c.block)
    _, Pr = oracle.score_rescue(qb, kb, r, cs)
    np.testing.assert_allclose(rs.cpu().numpy(), Pr, rtol=1e-4, atol=1e-6)
    omd, _, ocntd = oracle.mask_dual(P, Pr, c.gamma, 0.5)
    _check_dual(md.cpu().numpy(), idxd.cpu().numpy(), cntd.cpu().numpy(), P, Pr, c.gamma, 0.5,
                omd, ocntd)



@pytest.mark.parametrize("nb", [1022, 2047, 2190])
def test_mask_long_rows_not_16_byte_aligned(nb):
    """Rows of nb % 4 != 0 blocks, long enough that a row's kept list leaves
    in several whole 256-entry runs while its rows are not 16-byte aligned:
    the threshold path (register kernel up to 2048 blocks, the general one
    beyond) against the oracle, and the caller-mask path against the causal
    part of the mask itself."""
    announce(f"long unaligned mask rows nb={nb}")
    rng = np.random.default_rng(nb)
    hq, block, gamma = 2, 64, 0.1
    P = np.tril(rng.random((hq, nb, nb)) ** 2).astype(np.float32)
    m, idx, cnt = bsp.mask(torch.from_numpy(P).cuda(), gamma, nb * block, block)
    um = (rng.random((hq, nb, nb)) < 0.9).astype(np.uint8)
    um[:, np.arange(nb), np.arange(nb)] = 1
    m2, idx2, cnt2 = bsp.mask(None, gamma, nb * block, block, user_mask=torch.from_numpy(um).cuda())
    torch.cuda.synchronize()
    om, oidx, ocnt = oracle.mask(P.astype(np.float64), gamma)
    H.check_mask(m.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
                 dict(P=P.astype(np.float64), mask=om, idx=oidx, cnt=ocnt), gamma)
    assert int(cnt.max()) > 512  # rows with at least two whole runs
    want = np.tril(um)
    assert np.array_equal(m2.cpu().numpy(), want)
    widx, wcnt = H.idx_from_mask(want)
    gcnt = cnt2.cpu().numpy()
    assert np.array_equal(gcnt, wcnt)
    keep = np.arange(nb)[None, None, :] < wcnt[..., None]
    assert np.array_equal(np.where(keep, idx2.cpu().numpy(), -1), widx)


def test_mask_varlen_long_rows_unaligned_stride():
    """Packed batch whose sequences have 301 and 270 blocks, idx_stride 302
    (rows not 16-byte aligned): every row's kept list, from a caller mask,
    against the mask itself."""
    announce("varlen mask, long rows, idx_stride 302")
    rng = np.random.default_rng(5)
    hq, block = 2, 64
    lens = [300 * block + 5, 270 * block]
    nbs = [-(-n // block) for n in lens]
    tb, stride = sum(nbs), max(nbs) + 1
    um = (rng.random((hq, tb, stride)) < 0.9).astype(np.uint8)
    m, idx, cnt = bsp.mask_varlen(None, 0.1, lens, block,
                                  user_mask=torch.from_numpy(um).cuda())
    torch.cuda.synchronize()
    gm, gidx, gcnt = m.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    b0 = 0
    for nb in nbs:
        want = np.tril(um[:, b0:b0 + nb, :nb])
        assert np.array_equal(gm[:, b0:b0 + nb, :nb], want)
        widx, wcnt = H.idx_from_mask(want)
        assert np.array_equal(gcnt[:, b0:b0 + nb], wcnt)
        keep = np.arange(nb)[None, None, :] < wcnt[..., None]
        assert np.array_equal(np.where(keep, gidx[:, b0:b0 + nb, :nb], -1), widx)
        b0 += nb
    assert int(gcnt.max()) > 256

_NAN_BITS = {"bf16": 0x7FC0, "fp8": 0x7F}


def _varlen_case(dtype, d, block, lens, seed, density):
    """One generated batch split along tokens into sequences; K/V written into
    a shuffled paged cache whose unused rows hold NaN bits; random masks."""
    c = gen.make_case(4, 2, sum(lens), d, block, dtype, seed, rope=True, n_vert=4)
    rng = np.random.default_rng(seed)
    nbs = [-(-n // block) for n in lens]
    tb = sum(nbs)
    npages = tb + 7
    perm = rng.permutation(npages).astype(np.int32)
    kc = np.full((npages, c.hkv, block, d), _NAN_BITS[dtype], c.k.dtype)
    vc = np.full_like(kc, _NAN_BITS[dtype])
    ptab = np.zeros((len(lens), max(nbs) + 2), np.int32)
    masks, t0, b0 = [], 0, 0
    for s, (n, nb) in enumerate(zip(lens, nbs)):
        for J in range(nb):
            pg = perm[b0 + J]
            ptab[s, J] = pg
            r1 = min(block, n - J * block)
            kc[pg, :, :r1] = c.k[:, t0 + J * block:t0 + J * block + r1]
            vc[pg, :, :r1] = c.v[:, t0 + J * block:t0 + J * block + r1]
        masks.append(gen.random_block_mask(c.hq, nb, density, seed + s))
        t0 += n
        b0 += nb
    return c, kc, vc, ptab, masks, nbs


@pytest.mark.parametrize("dtype,d,block,dense", [("bf16", 128, 128, False), ("bf16", 128, 128, True),
                                                  ("bf16", 64, 64, False), ("fp8", 128, 128, False),
                                                  ("fp8", 64, 64, True)])
def test_varlen_paged_matches_oracle_per_sequence(dtype, d, block, dense):
    lens = [1000, 130, 512, 64, 777, 1]
    announce(f"varlen paged {dtype} d={d} B={block} dense={dense} lens={lens}")
    c, kc, vc, ptab, masks, nbs = _varlen_case(dtype, d, block, lens, 31 + d + block, 0.5)
    dv = H.dev(c)
    t = lambda x: (torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) if dtype == "bf16"
                   else torch.from_numpy(x).cuda())
    kv_idx = kv_cnt = None
    if not dense:
        stride = max(nbs) + 3
        tb = sum(nbs)
        idx = np.full((c.hq, tb, stride), -7, np.int32)
        cnt = np.zeros((c.hq, tb), np.int32)
        b0 = 0
        for m, nb in zip(masks, nbs):
            i_s, c_s = H.idx_from_mask(m)
            idx[:, b0:b0 + nb, :nb] = np.where(i_s >= 0, i_s, -7)
            cnt[:, b0:b0 + nb] = c_s
            b0 += nb
        kv_idx, kv_cnt = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    o, lse = bsp.attn_fwd_varlen(dv["q"], t(kc), t(vc), torch.from_numpy(ptab).cuda(), lens, block,
                                 kv_idx, kv_cnt, q_scale=dv["q_scale"], k_scale=dv["k_scale"],
                                 v_scale=dv["v_scale"])
    torch.cuda.synchronize()
    go, gl = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(go))
    t0, err = 0, 0.0
    for n, nb, m in zip(lens, nbs, masks):
        sl = slice(t0, t0 + n)
        mm = np.tril(np.ones((c.hq, nb, nb), np.uint8)) if dense else m
        oo, ol = oracle.attn(c.q[:, sl], c.k[:, sl], c.v[:, sl], dtype, block, mm,
                             q_scale=c.q_scale, k_scale=c.k_scale, v_scale=c.v_scale)
        err = max(err, H.check_attn(go[:, sl].reshape(-1, d), gl[:, sl].reshape(-1),
                                    oo.reshape(-1, d), ol.reshape(-1), dtype))
        t0 += n
    print(f"  max-abs O err {err:.2e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_block_order(dtype):
    """A caller's launch order (block_order, a permutation of the batch's
    query blocks) changes only which workgroup serves a row: the output is
    bit-identical to the default order and matches the oracle per sequence."""
    lens = [1000, 130, 512, 64, 777, 1, 1200]
    d, block = 128, 128
    announce(f"varlen block_order {dtype} lens={lens}")
    c, kc, vc, ptab, masks, nbs = _varlen_case(dtype, d, block, lens, 91, 0.5)
    dv = H.dev(c)
    t = lambda x: (torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) if dtype == "bf16"
                   else torch.from_numpy(x).cuda())
    stride = max(nbs)
    tb = sum(nbs)
    idx = np.zeros((c.hq, tb, stride), np.int32)
    cnt = np.zeros((c.hq, tb), np.int32)
    b0 = 0
    for m, nb in zip(masks, nbs):
        i_s, c_s = H.idx_from_mask(m)
        idx[:, b0:b0 + nb, :nb] = i_s
        cnt[:, b0:b0 + nb] = c_s
        b0 += nb
    order = np.random.default_rng(5).permutation(tb).astype(np.int32)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], v_scale=dv["v_scale"])
    args = (dv["q"], t(kc), t(vc), torch.from_numpy(ptab).cuda(), lens, block,
            torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda())
    o1, l1 = bsp.attn_fwd_varlen(*args, **kw)
    o2, l2 = bsp.attn_fwd_varlen(*args, block_order=torch.from_numpy(order).cuda(), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    go, gl = o2.float().cpu().numpy(), l2.cpu().numpy()
    t0, err = 0, 0.0
    for n, nb, m in zip(lens, nbs, masks):
        sl = slice(t0, t0 + n)
        oo, ol = oracle.attn(c.q[:, sl], c.k[:, sl], c.v[:, sl], dtype, block, m,
                             q_scale=c.q_scale, k_scale=c.k_scale, v_scale=c.v_scale)
        err = max(err, H.check_attn(go[:, sl].reshape(-1, d), gl[:, sl].reshape(-1),
                                    oo.reshape(-1, d), ol.reshape(-1), dtype))
        t0 += n
    print(f"  max-abs O err {err:.2e}", flush=True)


@pytest.mark.parametrize("dtype,d,block,gamma,sink,local", [
    ("bf16", 128, 128, 0.3, 1, 1), ("fp8", 128, 128, 0.2, 1, 1), ("bf16", 64, 64, 0.4, 1, 1),
    ("fp8", 64, 64, 0.3, 1, 1), ("bf16", 128, 128, 0.3, 2, 4), ("fp8", 64, 64, 0.4, 4, 8)])
def test_varlen_pipeline_matches_oracle_per_sequence(dtype, d, block, gamma, sink, local):
    """Score, mask and attention of a packed batch over a shuffled paged cache
    (unused cache rows NaN bits): every sequence against the oracle run on
    that sequence alone.  Includes the pages' sink and window sizes, counted
    from each sequence's own first block."""
    import dataclasses
    lens = [1000, 130, 512, 64, 777, 1, 900]
    announce(f"varlen pipeline {dtype} d={d} B={block} gamma={gamma} sink={sink} local={local} "
             f"lens={lens}")
    c = gen.make_case(4, 2, sum(lens), d, block, dtype, 47 + d, rope=True, n_vert=4,
                      block_offset=1.5)  # masks keep 45-73% of the causal blocks
    rng = np.random.default_rng(d + block)
    nbs = [-(-n // block) for n in lens]
    tb = sum(nbs)
    npages = tb + 5
    perm = rng.permutation(npages).astype(np.int32)
    kc = np.full((npages, c.hkv, block, d), _NAN_BITS[dtype], c.k.dtype)
    vc = np.full_like(kc, _NAN_BITS[dtype])
    ptab = np.zeros((len(lens), max(nbs) + 1), np.int32)
    t0, b0 = 0, 0
    for s_, (n, nb) in enumerate(zip(lens, nbs)):
        for J in range(nb):
            pg = perm[b0 + J]
            ptab[s_, J] = pg
            r1 = min(block, n - J * block)
            kc[pg, :, :r1] = c.k[:, t0 + J * block:t0 + J * block + r1]
            vc[pg, :, :r1] = c.v[:, t0 + J * block:t0 + J * block + r1]
        t0 += n
        b0 += nb
    dv = H.dev(c)
    t = lambda x: (torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) if dtype == "bf16"
                   else torch.from_numpy(x).cuda())
    res = bsp.prefill_varlen(dv["q"], t(kc), t(vc), torch.from_numpy(ptab).cuda(), lens, block,
                             gamma, sink_blocks=sink, local_blocks=local, q_scale=dv["q_scale"],
                             k_scale=dv["k_scale"], v_scale=dv["v_scale"])
    torch.cuda.synchronize()
    g = {k_: v_.cpu().numpy() for k_, v_ in res.items() if v_ is not None and k_ not in ("o", "lse")}
    go, gl = res["o"].float().cpu().numpy(), res["lse"].cpu().numpy()
    t0, cb, err, nband = 0, 0, 0.0, 0
    for n, nb in zip(lens, nbs):
        sub = dataclasses.replace(c, seq=n, q=c.q[:, t0:t0 + n], k=c.k[:, t0:t0 + n],
                                  v=c.v[:, t0:t0 + n])
        orc = oracle.prefill(sub, gamma, sink_blocks=sink, local_blocks=local, with_attn=False)
        rb = slice(cb, cb + nb)
        np.testing.assert_allclose(g["q_pool"][:, rb], orc["qbar"], rtol=1e-5, atol=2e-6)
        np.testing.assert_allclose(g["k_pool"][:, rb], orc["kbar"], rtol=1e-5, atol=2e-6)
        np.testing.assert_allclose(g["score"][:, rb, :nb], orc["P"], rtol=1e-4, atol=1e-6)
        gm = g["mask"][:, rb, :nb]
        nband += H.check_mask(gm, g["kv_idx"][:, rb, :nb], g["kv_cnt"][:, rb], orc, gamma, sink,
                              local)
        oo, ol = oracle.attn(sub.q, sub.k, sub.v, dtype, block, gm, q_scale=c.q_scale,
                             k_scale=c.k_scale, v_scale=c.v_scale)
        sl = slice(t0, t0 + n)
        err = max(err, H.check_attn(go[:, sl].reshape(-1, d), gl[:, sl].reshape(-1),
                                    oo.reshape(-1, d), ol.reshape(-1), dtype))
        t0 += n
        cb += nb
    dens = g["mask"].sum() / sum(c.hq * nb * (nb + 1) / 2 for nb in nbs)
    print(f"  density {dens:.3f} band {nband} max-abs O err {err:.2e}", flush=True)


@pytest.mark.parametrize("which,target,sink,local", [
    ("s1_0", 0.3, 1, 1), ("s1_1", 0.7, 1, 1), ("llama_4k", 0.7, 1, 1), ("s1_2", 0.5, 4, 8),
    ("llama_4k", 0.7, 2, 4), ("s1_3", 0.9, 0, 0)])
def test_calibrate_gamma_meets_the_definition(which, target, sink, local):
    """bsp_calibrate_gamma against the definition (the largest gamma whose
    density reaches the target, computed exactly by the oracle): the GPU's
    gamma lies at most tol below it, up to the threshold band; its density
    reaches the target and is the density of its own returned counts, which
    match the oracle's mask at that gamma outside the band; the buffers it
    leaves are bsp_mask's result at that gamma.  Includes the pages' sink
    and window sizes."""
    announce(f"calibrate gamma {which} target {target} sink {sink} local {local}")
    c = gen.make_s1(int(which[-1])) if which.startswith("s1") else gen.make_config(1)
    d = H.dev(c)
    _, _, sc = bsp.score(d["q"], d["k"], c.block, q_scale=d["q_scale"], k_scale=d["k_scale"])
    tol = 1e-4
    g, dens, m, idx, cnt = bsp.calibrate_gamma(sc, c.seq, c.block, target, tol, sink, local)
    _, _, idx0, cnt0 = bsp.calibrate_gamma(sc, c.seq, c.block, target, tol, sink, local,
                                           want_mask=False)[1:]
    torch.cuda.synchronize()
    orc = oracle.prefill(c, with_attn=False)
    t32 = float(np.float32(target))
    exact, edens = oracle.calibrate_gamma(orc["P"], t32, sink, local)
    total = c.hq * c.nb * (c.nb + 1) / 2
    gcnt = cnt.cpu().numpy()
    print(f"  gpu gamma {g:.6f} density {dens:.4f}; exact gamma {exact:.6f} density {edens:.4f}",
          flush=True)
    assert dens >= np.float32(target)
    assert abs(dens - gcnt.sum() / total) <= 1e-6
    band = H.MASK_BAND
    if exact == 1.0:
        assert g == 1.0
    else:
        assert exact * (1 - band) - tol <= g <= exact * (1 + band)
    om, oidx, ocnt = oracle.mask(orc["P"], float(g), sink, local)
    nb_ = H.check_mask(m.cpu().numpy(), idx.cpu().numpy(), gcnt,
                       dict(P=orc["P"], mask=om, idx=oidx, cnt=ocnt), float(g), sink, local)
    assert abs(gcnt.sum() - ocnt.sum()) <= nb_
    m2, idx2, cnt2 = bsp.mask(sc, g, c.seq, c.block, sink, local)
    torch.cuda.synchronize()
    assert torch.equal(m, m2) and torch.equal(cnt, cnt2) and torch.equal(cnt0, cnt2)
    keep = torch.arange(c.nb, device=cnt.device)[None, None, :] < cnt2[..., None]
    assert torch.equal(idx[keep], idx2[keep]) and torch.equal(idx0[keep], idx2[keep])


@pytest.mark.parametrize("nb,block,sink,local", [(40, 128, 2, 4), (300, 64, 4, 8),
                                                 (1022, 128, 2, 4), (2047, 64, 4, 8),
                                                 (2190, 64, 4, 8), (2190, 128, 2, 4)])
def test_mask_page_retention(nb, block, sink, local):
    """The pages' structural retention (a 256-token sink and a 512-token
    window: 2 and 4 blocks at B = 128, 4 and 8 at B = 64) on rows of 40 to
    2190 blocks, through the register mask kernel (up to 2048 blocks) and the
    general one (beyond), for the base and the dual-branch masks, with and
    without the block-mask output (NULL mask: the lists alone)."""
    announce(f"page retention nb={nb} B={block} sink={sink} local={local}")
    rng = np.random.default_rng(nb * 10 + sink)
    hq, gamma, gr = 2, 0.3, 0.6
    P = np.tril(rng.random((hq, nb, nb)) ** 4).astype(np.float32)
    Pr = np.tril(rng.random((hq, nb, nb)) ** 4).astype(np.float32)
    seq = nb * block
    Pt, Prt = torch.from_numpy(P).cuda(), torch.from_numpy(Pr).cuda()
    m, idx, cnt = bsp.mask(Pt, gamma, seq, block, sink, local)
    m0, idx0, cnt0 = bsp.mask(Pt, gamma, seq, block, sink, local, want_mask=False)
    md, idxd, cntd = bsp.mask_dual(Pt, Prt, gamma, gr, seq, block, sink, local)
    md0, idxd0, cntd0 = bsp.mask_dual(Pt, Prt, gamma, gr, seq, block, sink, local,
                                      want_mask=False)
    torch.cuda.synchronize()
    assert m0 is None and md0 is None
    P64, Pr64 = P.astype(np.float64), Pr.astype(np.float64)
    om, oidx, ocnt = oracle.mask(P64, gamma, sink, local)
    gm = m.cpu().numpy()
    H.check_mask(gm, idx.cpu().numpy(), cnt.cpu().numpy(),
                 dict(P=P64, mask=om, idx=oidx, cnt=ocnt), gamma, sink, local)
    I = np.arange(nb)[:, None]
    J = np.arange(nb)[None, :]
    forced = (J <= I) & ((J < sink) | (I - J < local))
    assert np.all(gm[:, forced] == 1)
    omd, _, ocntd = oracle.mask_dual(P64, Pr64, gamma, gr, sink, local)
    _check_dual(md.cpu().numpy(), idxd.cpu().numpy(), cntd.cpu().numpy(), P64, Pr64, gamma, gr,
                omd, ocntd, sink, local)
    for c1, i1, c2, i2 in ((cnt, idx, cnt0, idx0), (cntd, idxd, cntd0, idxd0)):
        assert torch.equal(c1, c2)
        keep = torch.arange(nb, device=c1.device)[None, None, :] < c1[..., None]
        assert torch.equal(i1[keep], i2[keep])


@pytest.mark.parametrize("dtype,d,block,seq,sink,local", [
    ("bf16", 128, 128, 5000, 2, 4), ("fp8", 128, 128, 4100, 2, 4), ("bf16", 64, 64, 3000, 4, 8),
    ("f32", 64, 64, 2000, 4, 8)])
def test_page_retention_pipeline(dtype, d, block, seq, sink, local):
    """Score, mask and attention with the pages' sink and window sizes on
    generated inputs: every block of the stage 1-2 outputs, sampled rows of
    the attention output."""
    announce(f"page retention pipeline {dtype} d={d} B={block} seq={seq} sink={sink} "
             f"local={local}")
    c = gen.make_case(8, 2, seq, d, block, dtype, 500 + seq, gamma=0.2, rope=True, n_vert=6,
                      slash=True, block_offset=1.0)
    full_check(c, sink=sink, local=local, rows=H.sample_rows(c.hq, c.seq, c.block, n_pos=16))


def _equal_lists(c1, i1, c2, i2, nb):
    assert torch.equal(c1, c2)
    keep = torch.arange(nb, device=c1.device)[None, None, :] < c1[..., None]
    assert torch.equal(i1[keep], i2[keep])


@pytest.mark.parametrize("dtype,d,block,hq,hkv,seq,gamma,sink,local", [
    ("bf16", 128, 128, 8, 2, 1000, 0.2, 1, 1), ("bf16", 64, 64, 8, 2, 777, 0.2, 4, 8),
    ("fp8", 128, 128, 8, 2, 1000, 0.3, 2, 4), ("fp8", 64, 64, 6, 3, 700, 0.2, 1, 1),
    ("f32", 128, 64, 4, 2, 333, 0.2, 1, 1), ("f32", 64, 128, 4, 1, 250, 0.0, 0, 0),
    ("bf16", 64, 64, 2, 1, 1022 * 64 - 5, 0.2, 1, 1), ("bf16", 64, 64, 2, 1, 2047 * 64, 0.1, 4, 8),
    ("bf16", 64, 64, 2, 1, 2190 * 64, 0.2, 2, 4), ("bf16", 128, 128, 4, 2, 1024 * 128, 1.0, 1, 1),
])
def test_score_mask_equals_score_then_mask(dtype, d, block, hq, hkv, seq, gamma, sink, local):
    """bsp_score_mask writes exactly what bsp_score followed by bsp_mask
    writes (block means, scores, mask, kv lists and counts, bit for bit),
    with and without the block-mask output; rows of 4 to 2190 blocks, rows
    whose length is not a multiple of 4, the pages' sink and window."""
    announce(f"score_mask {dtype} d={d} B={block} heads {hq}/{hkv} seq={seq} gamma={gamma} "
             f"sink={sink} local={local}")
    c = gen.make_case(hq, hkv, seq, d, block, dtype, 900 + seq % 1000, gamma=gamma, rope=True,
                      n_vert=6, slash=True, block_offset=1.0)
    dv = H.dev(c)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"])
    qp, kp, sc = bsp.score(dv["q"], dv["k"], block, **kw)
    m, idx, cnt = bsp.mask(sc, gamma, seq, block, sink, local)
    qp2, kp2, sc2, m2, idx2, cnt2 = bsp.score_mask(dv["q"], dv["k"], block, gamma,
                                                   sink_blocks=sink, local_blocks=local, **kw)
    r3 = bsp.score_mask(dv["q"], dv["k"], block, gamma, sink_blocks=sink, local_blocks=local,
                        want_mask=False, **kw)
    torch.cuda.synchronize()
    assert r3[3] is None
    for a, b in ((qp, qp2), (kp, kp2), (sc, sc2), (m, m2), (sc, r3[2])):
        assert torch.equal(a, b)
    _equal_lists(cnt, idx, cnt2, idx2, c.nb)
    _equal_lists(cnt, idx, r3[5], r3[4], c.nb)
    if c.nb <= 1024:  # the mask against the oracle (larger rows: the long-row tests)
        orc = oracle.prefill(c, gamma, sink_blocks=sink, local_blocks=local, with_attn=False)
        nband = H.check_mask(m2.cpu().numpy(), idx2.cpu().numpy(), cnt2.cpu().numpy(), orc, gamma,
                             sink, local)
        print(f"  band blocks {nband}", flush=True)


def test_gamma0_equals_dense_path_bitwise():
    announce("gamma=0 vs dense")
    c = gen.make_case(4, 2, 1024, 128, 128, "bf16", 5, rope=True, n_vert=4)
    d, res = H.run_gpu_prefill(c, gamma=0.0)
    nb = c.nb
    assert torch.equal(res["kv_cnt"].cpu(), torch.arange(1, nb + 1, dtype=torch.int32).expand(4, nb))
    o, lse = bsp.attn_fwd(d["q"], d["k"], d["v"], c.block)
    torch.cuda.synchronize()
    assert torch.equal(o, res["o"]) and torch.equal(lse, res["lse"])


def test_user_mask_with_empty_rows():
    announce("user mask, empty rows")
    c = gen.make_case(4, 1, 640, 128, 128, "bf16", 8)
    nb = c.nb
    rng = np.random.default_rng(1)
    um = (rng.random((4, nb, nb)) < 0.5).astype(np.uint8)
    um[1, 2, :] = 0
    um[3, :, :] = 0
    d, res = H.run_gpu_prefill(c, user_mask=um)
    m = res["mask"].cpu().numpy()
    assert np.array_equal(m, um & np.tril(np.ones((nb, nb), np.uint8)))
    oo, ol = oracle.attn(c.q, c.k, c.v, "bf16", c.block, m)
    go = res["o"].float().cpu().numpy()
    gl = res["lse"].cpu().numpy()
    H.check_attn(go.reshape(-1, 128), gl.reshape(-1), oo.reshape(-1, 128), ol.reshape(-1), "bf16")
    assert np.all(go[3] == 0) and np.all(np.isneginf(gl[3]))
    assert np.all(go[1, 256:384] == 0)


def test_rows_sum_to_one():
    announce("V == 1")
    c = gen.make_case(4, 2, 512, 128, 128, "bf16", 9, block_offset=1.0)
    c.v[:] = gen.bf16_bits(np.ones(1, np.float32))[0]
    d, res = H.run_gpu_prefill(c, gamma=0.3)
    assert torch.all(res["o"].float() == 1.0)


def test_index_order_does_not_matter():
    announce("permuted kv_idx")
    c = gen.make_case(4, 2, 1024, 128, 128, "bf16", 10)
    d, res = H.run_gpu_prefill(c, gamma=0.0)
    idx = res["kv_idx"].cpu().numpy().copy()
    cnt = res["kv_cnt"].cpu().numpy()
    rng = np.random.default_rng(0)
    for h in range(4):
        for I in range(c.nb):
            idx[h, I, :cnt[h, I]] = rng.permutation(idx[h, I, :cnt[h, I]])
    o, lse = bsp.attn_fwd(d["q"], d["k"], d["v"], c.block, torch.from_numpy(idx).cuda(),
                          res["kv_cnt"])
    torch.cuda.synchronize()
    assert (o.float() - res["o"].float()).abs().max().item() <= 1e-2
    assert (lse - res["lse"]).abs().max().item() <= 1e-4


def test_duplicated_heads_and_mha_expansion():
    announce("duplicated heads / MHA")
    c = gen.make_case(4, 2, 512, 128, 128, "bf16", 11)
    c.q[1] = c.q[0]
    d, res = H.run_gpu_prefill(c, gamma=0.0)
    assert torch.equal(res["o"][0], res["o"][1])
    k4 = d["k"].repeat_interleave(2, dim=0).contiguous()
    v4 = d["v"].repeat_interleave(2, dim=0).contiguous()
    o4, _ = bsp.attn_fwd(d["q"], k4, v4, c.block)
    torch.cuda.synchronize()
    assert torch.equal(o4, res["o"])


def test_deterministic():
    announce("determinism")
    c = gen.make_case(8, 2, 2048, 128, 128, "bf16", 12, rope=True, slash=True, block_offset=1.0)
    _, a = H.run_gpu_prefill(c)
    _, b = H.run_gpu_prefill(c)
    for key in ("score", "mask", "kv_idx", "kv_cnt", "o", "lse"):
        if key == "kv_idx":
            cnt = a["kv_cnt"]
            keep = torch.arange(c.nb, device=cnt.device)[None, None, :] < cnt[..., None]
            assert torch.equal(a[key][keep], b[key][keep])
        else:
            assert torch.equal(a[key], b[key]), key


def test_errors_leave_outputs_untouched():
    announce("error path canaries")
    q = torch.zeros(4, 256, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.full((4, 256, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsp.BspError) as e:
        bsp.attn_fwd(q, q[:3].contiguous(), q[:3].contiguous(), 128, out=o)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)


def test_empty_sequence():
    announce("seq = 0")
    q = torch.zeros(4, 0, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = bsp.attn_fwd(q, q[:2], q[:2], 128)
    qp, kp, sc = bsp.score(q, q[:2], 128)
    assert o.shape == (4, 0, 128) and sc.shape == (4, 0, 0)


def test_sm_scale_override():
    announce("explicit sm_scale")
    c = gen.make_case(2, 1, 256, 64, 64, "bf16", 13)
    d = H.dev(c)
    bm = np.tril(np.ones((2, 4, 4), np.uint8))
    idx, cnt = H.idx_from_mask(bm)
    o, lse = bsp.attn_fwd(d["q"], d["k"], d["v"], 64, torch.from_numpy(idx).cuda(),
                          torch.from_numpy(cnt).cuda(), sm_scale=0.3)
    torch.cuda.synchronize()
    oo, ol = oracle.attn(c.q, c.k, c.v, "bf16", 64, bm, sm_scale=0.3)
    H.check_attn(o.float().cpu().numpy().reshape(-1, 64), lse.cpu().numpy().reshape(-1),
                 oo.reshape(-1, 64), ol.reshape(-1), "bf16")
