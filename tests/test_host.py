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
