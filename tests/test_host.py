"""Host-side logic: workload arithmetic and the seeded input generator."""
import torch

from trainable_dynamic_mask_amd.configs import WORKLOADS, Workload
from trainable_dynamic_mask_amd.inputs import make_inputs, make_small


def _kept_brute(wl):
    return sum(min(p + 1, wl.w) for p in range(wl.q_offset, wl.q_offset + wl.Sq)) * wl.B * wl.Hq


def test_kept_pairs_formula():
    for S, w, q0, Sq in [(256, 64, 0, 256), (100, 200, 0, 100), (50, 7, 30, 20), (10, 1, 0, 10),
                         (4096, 2048, 0, 4096), (32768, 2048, 32767, 1)]:
        wl = Workload("t", "bf16", 2, 4, 2, Sq, S, q0, 128, w, 0.02, 0)
        assert wl.kept_pairs() == _kept_brute(wl)
    assert WORKLOADS["prefill_16k"].kept_pairs() == 1_006_665_728
    # chunked prefill: rows 12288..16383 all keep w = 2048 keys, 32 query heads
    assert WORKLOADS["chunk_16k"].kept_pairs() == 4096 * 2048 * 32
    assert WORKLOADS["prefill_64k"].effective_flops() == 4 * 128 * 8_321_564_672


def test_inputs_seeded_and_shaped():
    wl = WORKLOADS["tiny_f32"]
    a, b = make_inputs(wl), make_inputs(wl)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert a["Q"].shape == (1, 256, 2, 64) and a["Q"].dtype == torch.float32
    assert a["Delta"].shape == (128, 2)
    assert (a["A"] >= 0.5).all() and (a["A"] < 1.5).all()
    wl2, x = make_small(1, 4, 2, 10, 10, 128, 3, dtype="bf16")
    assert x["K"].dtype == torch.bfloat16 and x["K"].shape == (1, 10, 2, 128)


def _bench_module():
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py")
    spec = importlib.util.spec_from_file_location("bench_under_test", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod, path


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    _, path = _bench_module()
    r = subprocess.run([sys.executable, path, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    bench, _ = _bench_module()
    good = tmp_path / "traffic.txt"
    good.write_text(f"kernel_source_sha256: {bench.attn_source_hash()}\n"
                    "hbm_bytes_per_launch: 123456\n# a comment: 1\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic("prefill_16k") == 123456.0
    assert bench.measured_traffic("prefill_64k") is None   # taken on the 16K workload only
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha256: 0000000000000000\nhbm_bytes_per_launch: 1\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic("prefill_16k") is None  # sources changed since
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("prefill_16k") is None


def test_binding_rejects_mismatched_mask_and_delta():
    # the kernels index the mask arrays and delta by the call's sizes, so the
    # binding refuses arrays built for other sizes before anything reaches the
    # C ABI (these checks run on the host, ahead of the device check)
    import pytest
    import trainable_dynamic_mask_amd as dma
    B, S, Hq, Hkv, D, w = 1, 128, 4, 2, 128, 16
    Q = torch.zeros(B, S, Hq, D, dtype=torch.bfloat16)
    K = torch.zeros(B, S, Hkv, D, dtype=torch.bfloat16)
    V = torch.zeros_like(K)
    delta = torch.ones(B, Hkv, S)
    short = dma.alloc_mask(B, Hkv, 64, S, 0, w, "cpu")
    with pytest.raises(ValueError, match="mask was built"):
        dma.attn_fwd(Q, K, V, delta, short)
    other_sk = dma.alloc_mask(B, Hkv, 64, 64, 0, w, "cpu")
    with pytest.raises(ValueError, match="mask was built"):
        dma.attn_fwd(Q[:, :64], K, V, delta, other_sk)
    good = dma.alloc_mask(B, Hkv, S, S, 0, w, "cpu")
    with pytest.raises(ValueError, match="delta must be"):
        dma.attn_fwd(Q, K, V, delta[:, :, :100], good)
    with pytest.raises(ValueError, match="delta must be"):
        dma.attn_fwd(Q, K, V, delta.double(), good)
    good.u_idx = good.u_idx[:10]
    with pytest.raises(ValueError, match="u_idx"):
        dma.attn_fwd(Q, K, V, delta, good)
    good = dma.alloc_mask(B, Hkv, S, S, 0, w, "cpu")
    with pytest.raises(ValueError, match="lse must be"):
        dma.attn_bwd(Q, K, V, delta, good, Q, torch.zeros(B, Hq, S, dtype=torch.float64), Q)
    with pytest.raises(ValueError, match="O and dO"):
        dma.attn_bwd(Q, K, V, delta, good, Q[:, :64], torch.zeros(B, Hq, S), Q)
    with pytest.raises(ValueError, match="share one dtype"):
        dma.attn_fwd(Q.float(), K, V, delta, good)
    with pytest.raises(ValueError, match="GPU"):
        dma.attn_fwd(Q, K, V, delta, good)   # every size matches: only the device is wrong
