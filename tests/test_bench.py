"""Host logic of bench.py (no GPU): the one-GPU contract, the FLOP and byte
counts its JSON line reports, and the guard on the counter-derived traffic."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("hq,nb,block,d", [(2, 7, 16, 64), (3, 32, 128, 128)])
def test_kept_flops_all_blocks_is_the_dense_causal_count(bench, hq, nb, block, d):
    """Every causal block kept: sum over rows of I full tiles and one
    triangular tile equals the dense-causal pair count seq (seq + 1) / 2."""
    seq = nb * block
    cnt = np.tile(np.arange(1, nb + 1, dtype=np.int32), (hq, 1))
    assert bench.kept_flops(cnt, d, block, seq) == pytest.approx(bench.dense_flops(hq, seq, d),
                                                                rel=1e-15)


def test_kept_flops_matches_a_brute_force_pair_count(bench):
    """A random mask that keeps each row's diagonal: 4 d times the number of
    (query, key) pairs with key <= query inside the kept tiles, counted one
    by one."""
    rng = np.random.default_rng(3)
    hq, nb, block, d = 2, 9, 8, 32
    seq = nb * block
    keep = rng.random((hq, nb, nb)) < 0.4
    keep &= np.tril(np.ones((nb, nb), bool))[None]
    keep[:, np.arange(nb), np.arange(nb)] = True
    pairs = 0
    for h in range(hq):
        for I in range(nb):
            for J in range(nb):
                if keep[h, I, J]:
                    for qi in range(I * block, (I + 1) * block):
                        for kj in range(J * block, (J + 1) * block):
                            pairs += kj <= qi
    cnt = keep.sum(-1).astype(np.int32)
    assert bench.kept_flops(cnt, d, block, seq) == 4.0 * d * pairs


def test_scoring_bytes_at_128k_equal_the_three_kernels_algorithmic_bytes(bench):
    """The 128K bf16 layer (32/8 heads, d 128, B 128) with every causal block
    kept: the per-kernel algorithmic bytes of the committed counter profile
    (pool 1.363 GB, score 0.155 GB, mask 0.168 GB) add up to the bench's
    scoring bytes."""
    hq, hkv, seq, d, B = 32, 8, 131072, 128, 128
    nb = seq // B
    causal = nb * (nb + 1) // 2
    pool = (hq + hkv) * seq * d * 2 + (hq + hkv) * nb * d * 4   # read Q, K; write the means
    score = (hq + hkv) * nb * d * 4 + hq * nb * nb * 4           # read the means; write P
    mask = hq * causal * 4 + hq * nb * nb + hq * causal * 4 + hq * nb * 4
    got = bench.scoring_bytes(hq, hkv, seq, d, B, 2, hq * causal)
    assert got == pool + score + mask == 1686372352
    assert round(pool / 1e9, 3) == 1.363 and round(score / 1e9, 3) == 0.155
    assert round(mask / 1e9, 3) == 0.168
    # the one-pass form decides the mask as P is written: no read of P's causal half
    fused = bench.scoring_bytes(hq, hkv, seq, d, B, 2, hq * causal, fused=True)
    assert got - fused == hq * causal * 4


def test_traffic_is_reported_only_for_the_counted_sources(bench, tmp_path, monkeypatch):
    """A counter note's traffic figure is returned while the attention
    sources hash to the fingerprint it records, and dropped once they do not
    (a note written here, so the check does not depend on which sources the
    committed note was taken on)."""
    import hashlib
    h = hashlib.sha256()
    for f in bench.ATTN_SRCS:
        h.update(open(f, "rb").read())
    note = tmp_path / "note.md"
    note.write_text(f"source_sha256: {h.hexdigest()}\ntraffic_bytes_per_launch: 2.1e10\n")
    monkeypatch.setattr(bench, "PMC_NOTE", str(note))
    assert bench.traffic_from_note() == 2.1e10
    changed = []
    for f in bench.ATTN_SRCS:
        p = tmp_path / os.path.basename(f)
        p.write_bytes(open(f, "rb").read() + b"\n// edited\n")
        changed.append(str(p))
    monkeypatch.setattr(bench, "ATTN_SRCS", changed)
    assert bench.traffic_from_note() is None
    monkeypatch.setattr(bench, "PMC_NOTE", str(tmp_path / "missing.md"))
    assert bench.traffic_from_note() is None
