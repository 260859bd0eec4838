"""The allocation-free mask entry point (dma_topk_mask_noalloc), through the
C ABI: its lists must equal dma_topk_mask's (which takes a workspace) bit for
bit, on two calls in a row, the second smaller (the static scratch keeps the
first call's contents)."""
import numpy as np
import pytest
import torch

import trainable_dynamic_mask_amd as dma

pytestmark = pytest.mark.gpu


def _delta(B, H, S, seed):
    g = torch.Generator().manual_seed(seed)
    # ties on purpose: few distinct values
    return (torch.randint(0, 50, (B, H, S), generator=g).float() / 7.0 + 1.0).cuda()


def _same(a, b):
    nt = a.dims["n_tiles_total"]
    for f in ("evict", "u_cnt", "u_nfull", "u_dmax", "kt_cnt", "u_dlo"):
        ta, tb = getattr(a, f), getattr(b, f)
        if ta is None:
            assert tb is None, f
            continue
        n = nt if f != "evict" else ta.numel()
        assert torch.equal(ta[:n], tb[:n]), f
    for f, cnt, stride in (("u_idx", a.u_cnt, a.dims["u_stride"]),
                           ("kt_idx", a.kt_cnt, a.dims["kt_stride"])):
        ta = getattr(a, f)[: nt * stride].view(nt, stride).cpu().numpy()
        tb = getattr(b, f)[: nt * stride].view(nt, stride).cpu().numpy()
        c = cnt[:nt].cpu().numpy()
        for g in range(nt):
            np.testing.assert_array_equal(ta[g, : c[g]], tb[g, : c[g]], err_msg=f"{f} tile {g}")


@pytest.mark.parametrize("first,second", [
    ((1, 8, 16384, 16384, 0, 2048), (2, 2, 1000, 1000, 0, 100)),
    ((1, 8, 4096, 16384, 12288, 2048), (1, 3, 700, 900, 200, 64)),
])
def test_noalloc_matches_workspace_call_twice(gpu_lib, first, second):
    for (B, H, Sq, Sk, q0, w), seed in ((first, 1), (second, 2)):
        print(f"noalloc mask B={B} Hkv={H} Sq={Sq} Sk={Sk} q0={q0} w={w}", flush=True)
        d = _delta(B, H, Sk, seed)
        ref = dma.topk_mask(d, Sq, q0, w)
        m = dma.alloc_mask(B, H, Sq, Sk, q0, w, d.device)
        got = dma.topk_mask(d, Sq, q0, w, mask=m, noalloc=True)
        torch.cuda.synchronize()
        _same(got, ref)


def test_noalloc_one_row_and_empty(gpu_lib):
    d = _delta(3, 2, 5000, 3)
    ref = dma.topk_mask(d, 1, 4999, 700)
    got = dma.topk_mask(d, 1, 4999, 700, mask=dma.alloc_mask(3, 2, 1, 5000, 4999, 700, d.device),
                        noalloc=True)
    torch.cuda.synchronize()
    _same(got, ref)
    e = dma.topk_mask(d, 0, 10, 3, noalloc=True)   # no rows: nothing launched
    assert e.dims["n_tiles_total"] == 0
