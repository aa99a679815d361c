"""GPU parity of the e4m3 -> bf16 widening (bsp_widen_e4m3) and of attention
on e4m3 Q/K with that widened V (BSP_DTYPE_FP8_E4M3_V_BF16): the widening
against the oracle's decoding of every code, and the attention bit for bit
against the same launch on the codes, plus against the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_bsp_amd as bsp
import gen
import oracle
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _decode_table():
    """The value of every e4m3fn code by the oracle's decoding (NaN codes NaN)."""
    return np.array([oracle.decode_e4m3fn(c) for c in range(256)], np.float64)


@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 256, 4099, (1 << 23) + 5])
def test_widen_every_code(n):
    print(f"\n[case] widen n={n}", flush=True)
    rng = np.random.default_rng(n)
    codes = np.arange(256, dtype=np.uint8)
    src = np.concatenate([codes, rng.integers(0, 256, max(0, n - 256), dtype=np.uint8)])[:n]
    x = torch.from_numpy(src).cuda()
    # a NaN-filled output of one extra element shows what was written
    out = torch.full((n + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")
    bsp.widen_e4m3(x, out=out[:n])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want = _decode_table()[src]
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got[:n]), nan)
    assert np.array_equal(got[:n][~nan], want[~nan])
    assert np.isnan(got[n])  # nothing past the end


def _attn_both(c, idx, cnt):
    dv = H.dev(c)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], v_scale=dv["v_scale"])
    o8, l8 = bsp.attn_fwd(dv["q"], dv["k"], dv["v"], c.block, idx, cnt, **kw)
    vw = bsp.widen_e4m3(dv["v"])
    ow, lw = bsp.attn_fwd(dv["q"], dv["k"], vw, c.block, idx, cnt, **kw)
    torch.cuda.synchronize()
    return (o8, l8), (ow, lw)


@pytest.mark.parametrize("d,block,hq,hkv,seq,density", [
    (128, 128, 8, 2, 1000, 0.4), (64, 64, 6, 3, 700, 0.5), (128, 64, 4, 4, 900, None),
    (64, 128, 8, 4, 513, 0.3), (128, 128, 4, 1, 2048, None)])
def test_attn_wide_v_equals_codes(d, block, hq, hkv, seq, density):
    """Same launch on the codes and on the widened V: bit-identical O and
    LSE (the widening is exact and the products are the same), and within
    the fp8 bound of the oracle."""
    print(f"\n[case] wide V d={d} B={block} hq={hq} hkv={hkv} seq={seq} density={density}",
          flush=True)
    c = gen.make_case(hq, hkv, seq, d, block, "fp8", 7 + d + seq, rope=True, n_vert=4)
    if density is None:
        idx = cnt = None
        m = np.tril(np.ones((hq, c.nb, c.nb), np.uint8))
    else:
        m = gen.random_block_mask(hq, c.nb, density, seq)
        i, n = H.idx_from_mask(m)
        idx, cnt = torch.from_numpy(i).cuda(), torch.from_numpy(n).cuda()
    (o8, l8), (ow, lw) = _attn_both(c, idx, cnt)
    assert torch.equal(o8, ow) and torch.equal(l8, lw)
    oo, ol = oracle.attn(c.q, c.k, c.v, "fp8", block, m, q_scale=c.q_scale, k_scale=c.k_scale,
                         v_scale=c.v_scale)
    err = H.check_attn(ow.float().cpu().numpy().reshape(-1, d), lw.cpu().numpy().reshape(-1),
                       oo.reshape(-1, d), ol.reshape(-1), "fp8")
    print(f"  max-abs O err {err:.2e}", flush=True)


def test_varlen_wide_v_cache_equals_codes():
    """A packed batch over a shuffled paged cache whose V pages are widened:
    bit-identical to the codes path (unused rows hold NaN codes and stay
    unread either way)."""
    lens = [1000, 130, 512, 64, 777, 1]
    print(f"\n[case] varlen wide V lens={lens}", flush=True)
    from tests.test_parity import _varlen_case
    c, kc, vc, ptab, masks, nbs = _varlen_case("fp8", 128, 128, lens, 77, 0.5)
    dv = H.dev(c)
    stride = max(nbs) + 1
    tb = sum(nbs)
    idx = np.full((c.hq, tb, stride), -1, np.int32)
    cnt = np.zeros((c.hq, tb), np.int32)
    b0 = 0
    for m, nb in zip(masks, nbs):
        i_s, c_s = H.idx_from_mask(m)
        idx[:, b0:b0 + nb, :nb] = i_s
        cnt[:, b0:b0 + nb] = c_s
        b0 += nb
    kv_idx, kv_cnt = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    kcd, vcd, pt = (torch.from_numpy(x).cuda() for x in (kc, vc, ptab))
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], v_scale=dv["v_scale"])
    o8, l8 = bsp.attn_fwd_varlen(dv["q"], kcd, vcd, pt, lens, 128, kv_idx, kv_cnt, **kw)
    ow, lw = bsp.attn_fwd_varlen(dv["q"], kcd, bsp.widen_e4m3(vcd), pt, lens, 128, kv_idx, kv_cnt,
                                 **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(ow.float()).all().item()
    assert torch.equal(o8, ow) and torch.equal(l8, lw)


def test_prefill_widens_v_by_default():
    """The pipeline helper widens e4m3 V first; its outputs equal those of
    the pipeline on the codes."""
    print("\n[case] prefill widen_v on / off", flush=True)
    c = gen.make_case(8, 2, 1500, 128, 128, "fp8", 5, rope=True, n_vert=4)
    dv = H.dev(c)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], v_scale=dv["v_scale"])
    a = bsp.prefill(dv["q"], dv["k"], dv["v"], 128, 0.2, **kw)
    b = bsp.prefill(dv["q"], dv["k"], dv["v"], 128, 0.2, widen_v=False, **kw)
    torch.cuda.synchronize()
    for key in ("mask", "kv_cnt", "o", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_widen_accepts_torch_float8_codes():
    """The same bytes as torch.float8_e4m3fn widen to the same bf16 values."""
    print("\n[case] widen float8_e4m3fn view", flush=True)
    x = torch.from_numpy(np.random.default_rng(11).integers(0, 256, 4099, dtype=np.uint8)).cuda()
    a = bsp.widen_e4m3(x)
    b = bsp.widen_e4m3(x.view(torch.float8_e4m3fn))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefill_varlen_widen_v_equals_codes():
    """prefill_varlen with widen_v: every output bit for bit that of the
    pipeline on the V codes."""
    lens = [700, 129, 1000, 1]
    print(f"\n[case] prefill_varlen widen_v lens={lens}", flush=True)
    from tests.test_parity import _varlen_case
    c, kc, vc, ptab, _, _ = _varlen_case("fp8", 64, 64, lens, 19, 0.5)
    dv = H.dev(c)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"], v_scale=dv["v_scale"])
    kcd, vcd, pt = (torch.from_numpy(x).cuda() for x in (kc, vc, ptab))
    a = bsp.prefill_varlen(dv["q"], kcd, vcd, pt, lens, 64, 0.3, **kw)
    b = bsp.prefill_varlen(dv["q"], kcd, vcd, pt, lens, 64, 0.3, widen_v=True, **kw)
    torch.cuda.synchronize()
    for key in ("mask", "kv_cnt", "o", "lse"):
        assert torch.equal(a[key], b[key]), key
