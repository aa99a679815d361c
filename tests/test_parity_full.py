"""GPU parity at the measured layer sizes, in the launch configuration the
benchmark times (score -> mask -> attention on the GPU's own mask): every
block of the pooled values, scores and masks, and sampled output rows that
the oracle computes one by one.

Besides the five measured layers (whose masks keep every causal block), the
same checks run where the threshold prunes: the planted strengths in logit
units at 32K and 128K (about 29% of the causal blocks kept; at 32K with the
pages' 256-token sink and 512-token window), and a caller mask keeping 3% of
the causal blocks at 128K, the sparsity the pages' speedups imply.  At 128K
bf16 the attention launch runs its kv groups in phases, so these cases also
cover that order on scattered kept lists."""
import time

import numpy as np
import pytest
import torch

import block_sparse_attention_bsp_amd as bsp
import gen
import oracle
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _full_size_check(c, seed, sink=1, local=1, user_mask=None, t0=None):
    t0 = time.time() if t0 is None else t0
    d, res = H.run_gpu_prefill(c, sink=sink, local=local, user_mask=user_mask)
    print(f"  gpu prefill done {time.time() - t0:.1f}s", flush=True)
    orc = oracle.prefill(c, sink_blocks=sink, local_blocks=local, user_mask=user_mask,
                         with_attn=False)
    print(f"  oracle stages 1-2 done {time.time() - t0:.1f}s", flush=True)
    gm = res["mask"].cpu().numpy()
    if user_mask is None:
        np.testing.assert_allclose(res["q_pool"].cpu().numpy(), orc["qbar"], rtol=1e-5, atol=2e-6)
        np.testing.assert_allclose(res["k_pool"].cpu().numpy(), orc["kbar"], rtol=1e-5, atol=2e-6)
        np.testing.assert_allclose(res["score"].cpu().numpy(), orc["P"], rtol=1e-4, atol=1e-6)
        nband = H.check_mask(gm, res["kv_idx"].cpu().numpy(), res["kv_cnt"].cpu().numpy(), orc,
                             c.gamma, sink, local)
    else:
        # a caller mask is exact: no threshold band
        assert np.array_equal(gm, orc["mask"])
        gcnt = res["kv_cnt"].cpu().numpy()
        assert np.array_equal(gcnt, orc["cnt"])
        keep = np.arange(c.nb)[None, None, :] < gcnt[..., None]
        assert np.array_equal(res["kv_idx"].cpu().numpy()[keep], orc["idx"][keep])
        nband = 0
    rows = H.sample_rows(c.hq, c.seq, c.block, n_pos=12, seed=seed)
    oo, ol = oracle.attn(c.q, c.k, c.v, c.dtype, c.block, gm, q_scale=c.q_scale,
                         k_scale=c.k_scale, v_scale=c.v_scale, rows=rows)
    go, gl = H.gather_rows(res["o"], res["lse"], rows)
    err = H.check_attn(go, gl, oo, ol, c.dtype)
    # every (head, query block) workgroup of the launch ran: a second launch
    # into NaN-filled outputs writes every O and LSE element (each row keeps
    # its diagonal block, so every LSE is finite) and matches the first bit
    # for bit
    o1, l1 = res["o"].clone(), res["lse"].clone()
    res["o"].fill_(float("nan"))
    res["lse"].fill_(float("nan"))
    bsp.attn_fwd(d["q"], d["k"], d["v"], c.block, res["kv_idx"], res["kv_cnt"],
                 q_scale=d["q_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"],
                 out=res["o"], lse=res["lse"])
    torch.cuda.synchronize()
    assert torch.isfinite(res["lse"]).all().item()
    assert torch.equal(res["o"], o1) and torch.equal(res["lse"], l1)
    del o1, l1
    dens = gm.sum() / (c.hq * c.nb * (c.nb + 1) / 2)
    print(f"  density {dens:.4f} band {nband} rows {rows.size} max-abs O err {err:.2e} "
          f"total {time.time() - t0:.1f}s", flush=True)
    return dens


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_full_size(cfg):
    t0 = time.time()
    print(f"\n[case] config {cfg} ({gen.CONFIGS[cfg]['name']}) full size", flush=True)
    c = gen.make_config(cfg)
    print(f"  generated in {time.time() - t0:.1f}s", flush=True)
    _full_size_check(c, cfg, t0=t0)


@pytest.mark.parametrize("cfg,sink,local", [(2, 2, 4), (3, 1, 1)])
def test_pruning_threshold_full_size(cfg, sink, local):
    """Planted strengths in logit units (the threshold prunes about 70% of
    the causal blocks) at 32K with the pages' sink and window, and at 128K."""
    t0 = time.time()
    print(f"\n[case] S2 config {cfg} full size, sink {sink} local {local}", flush=True)
    c = gen.make_s2(cfg)
    print(f"  generated in {time.time() - t0:.1f}s", flush=True)
    dens = _full_size_check(c, 10 + cfg, sink=sink, local=local, t0=t0)
    assert dens < 0.5  # the threshold really prunes


def test_sparse_caller_mask_full_size_128k():
    """A caller mask keeping 3% of the causal blocks (sink and diagonal set)
    at 128K bf16: scattered kept blocks through the phased launch order."""
    t0 = time.time()
    print("\n[case] config 3 full size, caller mask density 0.03", flush=True)
    c = gen.make_config(3)
    um = gen.random_block_mask(c.hq, c.nb, 0.03, 0)
    print(f"  generated in {time.time() - t0:.1f}s", flush=True)
    dens = _full_size_check(c, 33, user_mask=um, t0=t0)
    assert dens < 0.05


@pytest.mark.parametrize("which", ["config3", "config4", "s2_config3"])
def test_score_mask_full_size_equals_two_calls(which):
    """The one-pass score and mask at the measured sizes (128K bf16, 256K
    fp8 with 2048-block rows, and the pruning 128K layer) writes what
    bsp_score followed by bsp_mask writes, bit for bit."""
    t0 = time.time()
    print(f"\n[case] score_mask vs score + mask, {which}", flush=True)
    c = gen.make_s2(3) if which.startswith("s2") else gen.make_config(int(which[-1]))
    dv = H.dev(c)
    kw = dict(q_scale=dv["q_scale"], k_scale=dv["k_scale"])
    qp, kp, sc = bsp.score(dv["q"], dv["k"], c.block, **kw)
    m, idx, cnt = bsp.mask(sc, c.gamma, c.seq, c.block)
    r = bsp.score_mask(dv["q"], dv["k"], c.block, c.gamma, **kw)
    torch.cuda.synchronize()
    for a, b in ((qp, r[0]), (kp, r[1]), (sc, r[2]), (m, r[3]), (cnt, r[5])):
        assert torch.equal(a, b)
    keep = torch.arange(c.nb, device=cnt.device)[None, None, :] < cnt[..., None]
    assert torch.equal(idx[keep], r[4][keep])
    dens = cnt.sum().item() / (c.hq * c.nb * (c.nb + 1) / 2)
    print(f"  density {dens:.4f} total {time.time() - t0:.1f}s", flush=True)
