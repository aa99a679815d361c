"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/bsp.h declares, and rejects bad arguments on the host before
any launch (so these calls never reach the device)."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_bsp_amd as bsp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsp.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(bsp_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(bsp.library_path):
        from block_sparse_attention_bsp_amd import build
        build.build()


def test_header_declares_the_entry_points():
    assert _declared() == ["bsp_abi_version", "bsp_attn_fwd", "bsp_attn_fwd_varlen",
                           "bsp_calibrate_gamma", "bsp_mask", "bsp_mask_dual", "bsp_mask_varlen",
                           "bsp_score", "bsp_score_arith", "bsp_score_mask", "bsp_score_rescue",
                           "bsp_score_varlen", "bsp_status_string", "bsp_widen_e4m3"]


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", bsp.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(bsp_\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name
        assert hasattr(bsp.lib(), name)


def test_abi_version_matches_header():
    want = int(re.search(r"#define BSP_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert bsp.bsp_abi_version() == want


def test_desc_struct_layout_matches_header():
    # int32 x5, float x2, int32 x4, then three pointers (8-byte aligned)
    assert ctypes.sizeof(bsp.BspDesc) == 11 * 4 + 4 + 3 * 8
    assert bsp.BspDesc.q_scale.offset == 48


def test_status_strings():
    for code, name in [(0, "BSP_OK"), (1, "BSP_ERR_NULL_POINTER"), (2, "BSP_ERR_BAD_SHAPE"),
                       (3, "BSP_ERR_BAD_DTYPE"), (4, "BSP_ERR_BAD_VALUE"),
                       (5, "BSP_ERR_UNSUPPORTED"), (6, "BSP_ERR_HIP")]:
        assert bsp.bsp_status_string(code).startswith(name)
    assert "unknown" in bsp.bsp_status_string(99)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation


def _d(**kw):
    base = dict(hq=4, hkv=2, seq=256, d=128, block=128, dtype=bsp.DTYPE_BF16, gamma=0.1)
    base.update(kw)
    return bsp.desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=0), 2), (dict(hkv=3), 2), (dict(hkv=8), 2), (dict(seq=-1), 2),
    (dict(seq=(1 << 21) + 1), 2), (dict(d=96), 2), (dict(block=32), 2), (dict(causal=0), 5),
    (dict(dtype=7), 3), (dict(sm_scale=float("inf")), 4), (dict(sm_scale=float("nan")), 4),
])
def test_score_rejects_bad_desc(kw, status):
    assert bsp.bsp_score(_d(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, None) == status


def test_null_pointers_rejected():
    assert bsp.lib().bsp_score(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert bsp.bsp_score(_d(), None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert bsp.bsp_score(_d(), FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert bsp.bsp_mask(_d(), None, None, None, FAKE, FAKE, None) == 1
    assert bsp.bsp_mask(_d(), FAKE, None, None, None, FAKE, None) == 1
    assert bsp.bsp_attn_fwd(_d(), FAKE, FAKE, None, None, None, FAKE, None, None) == 1
    # kv_idx and kv_cnt go together
    assert bsp.bsp_attn_fwd(_d(), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None) == 1


@pytest.mark.parametrize("gamma", [-0.1, 1.5, float("nan")])
def test_mask_rejects_bad_gamma(gamma):
    assert bsp.bsp_mask(_d(gamma=gamma), FAKE, None, None, FAKE, FAKE, None) == 4


def test_mask_rejects_negative_windows():
    assert bsp.bsp_mask(_d(sink_blocks=-1), FAKE, None, None, FAKE, FAKE, None) == 4
    assert bsp.bsp_mask(_d(local_blocks=-2), FAKE, None, None, FAKE, FAKE, None) == 4


def test_fp8_scale_rules():
    fp8 = _d(dtype=bsp.DTYPE_FP8_E4M3)
    assert bsp.bsp_score(fp8, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert bsp.bsp_attn_fwd(fp8, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 3
    withscale = _d()
    withscale.q_scale = 0x2000
    assert bsp.bsp_score(withscale, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3
    half = _d(dtype=bsp.DTYPE_FP8_E4M3)
    half.q_scale = 0x2000
    half.k_scale = 0x2000
    assert bsp.bsp_attn_fwd(half, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 3  # no v_scale


def test_mixed_dtype_scale_rules():
    # e4m3 Q/K with bf16 V: the fp8 scale rules hold, seq == 0 is accepted
    mix = _d(dtype=bsp.DTYPE_FP8_E4M3_V_BF16)
    assert bsp.bsp_score(mix, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3
    assert bsp.bsp_attn_fwd(mix, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 3
    mix.q_scale = mix.k_scale = 0x2000
    assert bsp.bsp_attn_fwd(mix, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 3  # no v_scale
    assert bsp.bsp_attn_fwd(_d(dtype=bsp.DTYPE_FP8_E4M3_V_BF16, seq=0), FAKE, FAKE, FAKE, None,
                            None, FAKE, None, None) == 0  # a known dtype: empty is a no-op
    assert bsp.bsp_score(_d(dtype=4), FAKE, FAKE, FAKE, FAKE, FAKE, None) == 3


def test_widen_host_checks():
    w = lambda src, dst, n: bsp.bsp_widen_e4m3(src, dst, n, None)
    assert w(FAKE, ctypes.c_void_p(0x4000), -1) == 2
    assert w(None, None, 0) == 0  # n == 0 is a no-op
    assert w(None, ctypes.c_void_p(0x4000), 16) == 1
    assert w(FAKE, None, 16) == 1
    assert w(ctypes.c_void_p(0x1008), ctypes.c_void_p(0x4000), 16) == 4  # misaligned source
    assert w(FAKE, ctypes.c_void_p(0x4008), 16) == 4  # misaligned destination
    # overlap: dst covers 2n bytes from 0x1000 - 16
    assert w(FAKE, ctypes.c_void_p(0x1000 - 16), 16) == 4
    assert w(ctypes.c_void_p(0x1000 + 32), FAKE, 64) == 4


def test_empty_sequence_is_a_no_op():
    # seq == 0 is valid and launches nothing
    assert bsp.bsp_score(_d(seq=0), FAKE, FAKE, FAKE, FAKE, FAKE, None) == 0
    assert bsp.bsp_mask(_d(seq=0), FAKE, None, None, FAKE, FAKE, None) == 0
    assert bsp.bsp_attn_fwd(_d(seq=0), FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 0


def test_score_mask_host_checks():
    sm = lambda d, *p: bsp.bsp_score_mask(d, *p, None)
    full = (FAKE,) * 8
    assert sm(_d(gamma=1.5), *full) == 4
    assert sm(_d(gamma=float("nan")), *full) == 4
    assert sm(_d(sink_blocks=-1), *full) == 4
    assert sm(_d(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE) == 1  # kv_idx
    assert sm(_d(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1  # kv_cnt
    assert sm(_d(), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE) == 1  # score
    assert sm(_d(dtype=bsp.DTYPE_FP8_E4M3), *full) == 3                 # no fp8 scales
    assert sm(_d(d=96), *full) == 2
    assert sm(_d(seq=0), *((None,) * 8)) == 0


def test_python_layer_raises_bsp_error():
    import torch
    x = torch.zeros(2, 64, 64)
    with pytest.raises(bsp.BspError):
        bsp.score(x, x, 64)  # host tensors are rejected before the C call


def test_binding_picks_the_mixed_dtype_for_a_widened_v():
    """Host-side dtype selection of the binding (no C call): e4m3 Q/K with a
    bf16 V is the mixed dtype, with e4m3 V the plain fp8 one; other mixes
    are rejected."""
    import torch
    sc = {}  # the scales are checked in the C call, not in the dtype choice
    q8 = torch.zeros(4, 256, 128, dtype=torch.uint8)
    k8 = torch.zeros(2, 256, 128, dtype=torch.uint8)
    f8 = torch.zeros(2, 256, 128, dtype=torch.float8_e4m3fn)
    vb = torch.zeros(2, 256, 128, dtype=torch.bfloat16)
    assert bsp._desc_qkv(q8, k8, 128, v=vb, **sc).dtype == bsp.DTYPE_FP8_E4M3_V_BF16
    assert bsp._desc_qkv(q8, k8, 128, v=k8, **sc).dtype == bsp.DTYPE_FP8_E4M3
    assert bsp._desc_qkv(torch.zeros(4, 256, 128, dtype=torch.bfloat16), vb, 128, v=vb).dtype == \
        bsp.DTYPE_BF16
    with pytest.raises(bsp.BspError):  # bf16 Q with a bf16 V but e4m3 K
        bsp._desc_qkv(torch.zeros(4, 256, 128, dtype=torch.bfloat16), k8, 128, v=vb)
    with pytest.raises(bsp.BspError):  # e4m3 Q/K with an fp32 V
        bsp._desc_qkv(q8, k8, 128, v=torch.zeros(2, 256, 128), **sc)
    with pytest.raises(bsp.BspError):  # Q and K must be the same torch type of codes
        bsp._desc_qkv(q8, f8, 128, v=vb, **sc)
    with pytest.raises(bsp.BspError):  # widening takes e4m3 codes only
        bsp.widen_e4m3(vb)


def test_calibrate_gamma_host_checks():
    import ctypes as C
    d = bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_F32)
    fake = C.c_void_p(0x1000)  # never dereferenced: every case fails before a launch
    g, dens = C.c_float(), C.c_float()
    for target, tol in [(0.0, 1e-4), (1.5, 1e-4), (float("nan"), 1e-4), (0.5, 0.0), (0.5, 1.0)]:
        assert bsp.bsp_calibrate_gamma(d, fake, target, tol, fake, fake, fake, fake, g, dens,
                                       None) == 4
    assert bsp.lib().bsp_calibrate_gamma(C.byref(d), fake, 0.5, 1e-4, fake, fake, fake, fake,
                                         None, C.byref(dens), None) == 1
    assert bsp.bsp_calibrate_gamma(d, None, 0.5, 1e-4, fake, fake, fake, fake, g, dens,
                                   None) == 1
    d0 = bsp.desc(4, 1, 0, 64, 64, bsp.DTYPE_F32)
    assert bsp.bsp_calibrate_gamma(d0, None, 0.5, 1e-4, None, None, None, None, g, dens,
                                   None) == 0
    assert g.value == 1.0 and dens.value == 1.0


def test_rescue_entry_points_host_checks():
    import ctypes as C
    fake = C.c_void_p(0x1000)  # never dereferenced: every case fails before a launch
    d = bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_BF16)
    assert bsp.bsp_score_rescue(d, fake, fake, fake, fake, None, None) == 1
    d8 = bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_FP8_E4M3)
    assert bsp.bsp_score_rescue(d8, fake, fake, fake, fake, fake, None) == 3  # needs k_scale
    for gr in (-0.1, 1.1, float("nan")):
        assert bsp.bsp_mask_dual(d, fake, fake, gr, fake, fake, fake, None) == 4
    assert bsp.bsp_mask_dual(d, fake, None, 0.5, fake, fake, fake, None) == 1
    d0 = bsp.desc(4, 1, 0, 64, 64, bsp.DTYPE_BF16)
    assert bsp.bsp_score_rescue(d0, None, None, None, None, None, None) == 0


def test_varlen_host_checks():
    fake = 0x1000  # never dereferenced: every case fails before a launch
    d = bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_BF16)
    ok = dict(cu_seqlens=fake, cu_blocks=fake, page_table=fake, nseq=2, total_blocks=16,
              max_pages=16, idx_stride=16)
    call = lambda dd, **kw: bsp.bsp_attn_fwd_varlen(dd, bsp.BspVarlen(**{**ok, **kw}), fake, fake,
                                                    fake, None, None, fake, None, None)
    assert call(d, nseq=0) == 2
    assert call(d, total_blocks=-1) == 2
    assert call(d, max_pages=0) == 2
    assert call(d, page_table=None) == 1
    assert call(bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_F32)) == 5
    assert call(d, total_blocks=0) == 0
    assert bsp.lib().bsp_attn_fwd_varlen(ctypes.byref(d), None, fake, fake, fake, None, None,
                                         fake, None, None) == 1
    assert ctypes.sizeof(bsp.BspVarlen) == 3 * 8 + 4 * 4 + 8


def test_varlen_score_and_mask_host_checks():
    fake = 0x1000  # never dereferenced: every case fails before a launch
    d = bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_BF16, gamma=0.1)
    ok = dict(cu_seqlens=fake, cu_blocks=fake, page_table=fake, nseq=2, total_blocks=16,
              max_pages=16, idx_stride=16)
    vl = lambda **kw: bsp.BspVarlen(**{**ok, **kw})
    score = lambda dd, v, **kw: bsp.bsp_score_varlen(dd, v, kw.get("q", fake), fake, fake, fake,
                                                     kw.get("s", fake), None)
    mask = lambda dd, v, **kw: bsp.bsp_mask_varlen(dd, v, kw.get("s", fake), None, None,
                                                   kw.get("i", fake), fake, None)
    for fn in (score, mask):
        assert fn(d, vl(nseq=0)) == 2
        assert fn(d, vl(total_blocks=-1)) == 2
        assert fn(d, vl(idx_stride=0)) == 2
        assert fn(d, vl(cu_blocks=None)) == 1
        assert fn(d, vl(total_blocks=0)) == 0  # nothing to do
        assert fn(bsp.desc(4, 3, 1024, 64, 64, bsp.DTYPE_BF16), vl()) == 2  # hq % hkv
    assert score(d, vl(page_table=None)) == 1
    assert score(d, vl(), q=None) == 1
    assert score(d, vl(), s=None) == 1
    d8 = bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_FP8_E4M3)
    assert score(d8, vl()) == 3  # fp8 needs q_scale and k_scale
    assert mask(d, vl(), s=None) == 1  # neither scores nor a caller mask
    assert mask(d, vl(), i=None) == 1
    assert mask(bsp.desc(4, 1, 1024, 64, 64, bsp.DTYPE_BF16, gamma=1.5), vl()) == 4
    assert bsp.lib().bsp_score_varlen(ctypes.byref(d), None, fake, fake, fake, fake, fake,
                                      None) == 1
