"""GPU masked attention (Hugging Face blog "Trainable Dynamic Mask Sparse
Attention", section "Efficient Sparse Attention Computation") against the
fp64 oracle, through the C ABI.

Stage-wise: the oracle gets the GPU's delta, so it selects exactly the keys
the mask step selected (the mask itself is pinned bit-exactly elsewhere).
End-to-end: the oracle's own fp64 delta; rows whose keep set differs from the
GPU's (fp32 vs fp64 near-ties) are counted, explained and left out.
"""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd.configs import WORKLOADS
from trainable_dynamic_mask_amd.inputs import make_inputs, make_small
from tests.dma_check import compare_rows, sample_rows, tile_edge_rows, to64

pytestmark = pytest.mark.gpu


def _run(x, wl, scale=None):
    """Both forwards: with the log-sum-exp (logits rounded as the backward
    recomputes them) and without it (the score scale inside the exponent)."""
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, wl.Sq, wl.q_offset, wl.w)
    O, lse = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, scale=scale, return_lse=True)
    Oi = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, scale=scale)
    torch.cuda.synchronize()
    return d, gm, O, lse, Oi


def _oracle_rows(x, d, wl, rows, scale=None):
    return oracle.attn_rows(x["Q"], x["K"], x["V"], to64(d), wl.q_offset, wl.w, rows, scale)


def _all_rows(wl):
    b, h, i = np.meshgrid(np.arange(wl.B), np.arange(wl.Hq), np.arange(wl.Sq), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], 1)


def test_tiny_f32_every_row(gpu_lib):
    wl = WORKLOADS["tiny_f32"]
    x = make_inputs(wl, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    m, r = compare_rows(O, lse, Or, Lr, rows, "f32", "tiny_f32")
    compare_rows(Oi, None, Or, Lr, rows, "f32", "tiny_f32 (no lse)")
    print(f"tiny_f32: max abs {m:.2e} rel L2 {r:.2e}")


@pytest.mark.parametrize("B,Hq,Hkv,S,w,dtype,D", [
    (1, 4, 1, 64, 16, "bf16", 128),      # one tile, MQA group of 4
    (2, 8, 2, 200, 37, "bf16", 128),     # ragged last tile
    (1, 2, 2, 129, 129, "bf16", 128),    # w >= S: plain causal
    (1, 8, 8, 300, 1, "bf16", 128),      # w = 1, G = 1
    (1, 16, 2, 260, 70, "bf16", 128),    # G = 8: two head groups per kv head
    (2, 6, 2, 190, 50, "bf16", 128),     # G = 3
    (1, 4, 2, 333, 100, "f32", 64),
    (1, 4, 4, 150, 20, "f32", 128),
])
def test_small_every_row(gpu_lib, B, Hq, Hkv, S, w, dtype, D):
    wl, x = make_small(B, Hq, Hkv, S, S, D, w, dtype=dtype, delta_std=0.05, seed=S + w,
                       device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    compare_rows(O, lse, Or, Lr, rows, dtype, f"{(B, Hq, Hkv, S, w, dtype, D)}")
    compare_rows(Oi, None, Or, Lr, rows, dtype, f"{(B, Hq, Hkv, S, w, dtype, D)} (no lse)")


def test_window_one_copies_value_rows_exactly(gpu_lib):
    wl, x = make_small(1, 4, 2, 200, 200, 128, 1, dtype="bf16", seed=5, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    d64 = to64(d)
    for hq in range(4):
        h = hq // 2
        best = np.array([int(np.argmax(d64[0, h, : i + 1])) for i in range(200)])
        assert torch.equal(O[0, :, hq], x["V"][0, torch.as_tensor(best, device="cuda"), h])


def test_custom_scale_and_strided_inputs(gpu_lib):
    # Q, K, V as views into packed per-token buffers
    B, S, Hq, Hkv, D, w = 2, 150, 8, 2, 128, 40
    wl, x = make_small(B, Hq, Hkv, S, S, D, w, dtype="bf16", seed=11, device="cuda")
    qkv = torch.zeros(B, S, Hq + 2 * Hkv + 1, D, dtype=torch.bfloat16, device="cuda")
    qkv[:, :, :Hq] = x["Q"]
    qkv[:, :, Hq:Hq + Hkv] = x["K"]
    qkv[:, :, Hq + Hkv:Hq + 2 * Hkv] = x["V"]
    Q, K, V = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:Hq + 2 * Hkv]
    kv = torch.zeros(B, S, 2 * Hkv, D, dtype=torch.bfloat16, device="cuda")
    kv[:, :, :Hkv] = K
    kv[:, :, Hkv:] = V
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, S, 0, w)
    O, lse = dma.attn_fwd(Q, kv[:, :, :Hkv], kv[:, :, Hkv:], d, gm, scale=0.05, return_lse=True)
    Oi = dma.attn_fwd(Q, kv[:, :, :Hkv], kv[:, :, Hkv:], d, gm, scale=0.05)
    rows = _all_rows(wl)
    Or, Lr = oracle.attn_rows(x["Q"], x["K"], x["V"], to64(d), 0, w, rows, scale=0.05)
    compare_rows(O, lse, Or, Lr, rows, "bf16", "strided")
    compare_rows(Oi, None, Or, Lr, rows, "bf16", "strided (no lse)")


@pytest.mark.parametrize("q0,Sq,Sk,w", [(100, 70, 170, 30), (500, 129, 629, 200),
                                        (64, 64, 128, 64)])
def test_chunked_prefill_query_offset(gpu_lib, q0, Sq, Sk, w):
    wl, x = make_small(1, 8, 2, Sq, Sk, 128, w, dtype="bf16", q_offset=q0, seed=q0, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    compare_rows(O, lse, Or, Lr, rows, "bf16", "chunked")
    compare_rows(Oi, None, Or, Lr, rows, "bf16", "chunked (no lse)")


def test_heavy_tailed_delta(gpu_lib):
    # Delta std 0.5: delta spans many orders of magnitude within a tile
    wl, x = make_small(1, 4, 1, 500, 500, 128, 60, dtype="bf16", delta_std=0.5, seed=2,
                       device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    assert float(d.max()) > 1e3
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    compare_rows(O, lse, Or, Lr, rows, "bf16", "heavy tail")
    compare_rows(Oi, None, Or, Lr, rows, "bf16", "heavy tail (no lse)")


@pytest.mark.parametrize("scale,delta_std,q0,seed", [(1.0, 0.02, 0, 31), (3.0, 0.05, 0, 32),
                                                     (3.0, 0.02, 150, 33)])
def test_large_score_terms(gpu_lib, scale, delta_std, q0, seed):
    # Score scales far above 1/sqrt(D): q.k*scale reaches +-100 and beyond, so
    # rows meet keys far above and far below their running reference (the
    # rescale path, and weights that overflow before it) in every tile.
    S = 700
    wl, x = make_small(1, 8, 2, S - q0, S, 128, 300, dtype="bf16", delta_std=delta_std,
                       q_offset=q0, seed=seed, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl, scale=scale)
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows, scale=scale)
    assert float(np.abs(Lr).max()) > 20.0 * scale  # the logits really are large
    compare_rows(O, lse, Or, Lr, rows, "bf16", f"scale {scale}")
    compare_rows(Oi, None, Or, Lr, rows, "bf16", f"scale {scale} (no lse)")


def test_f32_heavy_tail_every_row(gpu_lib):
    # delta std 0.1 (delta up to ~1e8, fp32 spacing ~8 there): rows that do not
    # see their tile's largest delta keep full precision because the fp32 path
    # takes each row's bias relative to the largest delta it keeps
    B, Hq, Hkv, S, w = 2, 3, 3, 1923, 605
    wl, x = make_small(B, Hq, Hkv, S, S, 64, w, dtype="f32", seed=302831582, delta_std=0.1,
                       device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    m, r = compare_rows(O, lse, Or, Lr, rows, "f32", "f32 heavy tail")
    compare_rows(Oi, None, Or, Lr, rows, "f32", "f32 heavy tail (no lse)")
    print(f"f32 heavy tail: max abs {m:.2e} rel L2 {r:.2e}")


@pytest.mark.parametrize("name", ["prefill_4k", "prefill_16k", "chunk_16k"])
def test_workload_every_row(gpu_lib, name):
    # every output row of the workload against the oracle (both forwards)
    wl = WORKLOADS[name]
    print(f"{name}: every row", flush=True)
    x = make_inputs(wl, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    assert torch.isfinite(O.float()).all()
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    m, r = compare_rows(O, lse, Or, Lr, rows, wl.dtype, name)
    mi, ri = compare_rows(Oi, None, Or, Lr, rows, wl.dtype, name + " (no lse)")
    print(f"{name}: {len(rows)} rows (all), max abs {m:.2e} rel L2 {r:.2e}; "
          f"no-lse forward max abs {mi:.2e} rel L2 {ri:.2e}")


def test_workload_64k_tile_edges_and_random_rows(gpu_lib):
    # the 64K workload has the largest delta range (the per-tile offset is least
    # exact there): every query tile's first and last row of every head, plus
    # random rows, at least 4096 rows per head
    wl = WORKLOADS["prefill_64k"]
    print("prefill_64k: tile edges + random rows", flush=True)
    x = make_inputs(wl, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    assert torch.isfinite(O.float()).all()
    rows = tile_edge_rows(wl.B, wl.Hq, wl.Sq, wl.w, per_head=4096, seed=wl.seed)
    per_head = np.bincount(rows[:, 0] * wl.Hq + rows[:, 1], minlength=wl.B * wl.Hq)
    assert per_head.min() >= 4096
    Or, Lr = _oracle_rows(x, d, wl, rows)
    m, r = compare_rows(O, lse, Or, Lr, rows, wl.dtype, "prefill_64k")
    mi, ri = compare_rows(Oi, None, Or, Lr, rows, wl.dtype, "prefill_64k (no lse)")
    print(f"prefill_64k: {len(rows)} rows ({per_head.min()} per head or more), max abs {m:.2e} "
          f"rel L2 {r:.2e}; no-lse forward max abs {mi:.2e} rel L2 {ri:.2e}")


@pytest.mark.parametrize("name", ["prefill_4k", "prefill_16k"])
def test_end_to_end_with_oracle_delta(gpu_lib, name):
    wl = WORKLOADS[name]
    x = make_inputs(wl, device="cuda")
    d, gm, O, lse, Oi = _run(x, wl)
    d64 = oracle.weights(x["V"], x["Delta"], x["A"])       # the oracle's own delta
    e_gpu = gm.evict.cpu().numpy().reshape(wl.B, wl.Hkv, wl.Sk)
    rows = sample_rows(wl.B, wl.Hq, wl.Sq, wl.w, 200, seed=wl.seed + 1)
    keep, differ = [], 0
    for (b, hq, i) in rows:
        h = hq // wl.G
        ref = oracle.keep_row(d64[b, h], i, wl.w)
        j = np.arange(i + 1)
        gpu = j[(j <= i) & (e_gpu[b, h, : i + 1] > i)]
        if np.array_equal(ref, gpu):
            keep.append((b, hq, i))
        else:
            differ += 1
            # a differing keep set must come from a near tie of fp64 delta
            sd = sorted(set(ref) ^ set(gpu))
            vals = d64[b, h, sd]
            assert vals.max() - vals.min() <= 1e-4 * vals.max(), (b, hq, i, sd, vals)
    rows = np.array(keep, np.int64)
    Or, Lr = oracle.attn_rows(x["Q"], x["K"], x["V"], d64, wl.q_offset, wl.w, rows)
    m, r = compare_rows(O, lse, Or, Lr, rows, wl.dtype, name + " end-to-end")
    compare_rows(Oi, None, Or, Lr, rows, wl.dtype, name + " end-to-end (no lse)")
    print(f"{name} end-to-end: {len(rows)} rows compared, {differ} left out (near ties); "
          f"max abs {m:.2e} rel L2 {r:.2e}")


def test_empty_query_rows(gpu_lib):
    wl, x = make_small(1, 4, 2, 10, 10, 128, 3, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, 0, 10, 3)
    O = dma.attn_fwd(x["Q"][:, :0], x["K"], x["V"], d, gm)
    assert O.shape == (1, 0, 4, 128)


@pytest.mark.parametrize("q0", [0, 70])
def test_large_delta_born_inside_a_tile(gpu_lib, q0):
    # delta ~ 1..5 except a few keys of 1e4..3e4 born in the middle of query
    # tiles: the rows of a tile before such a key keep only small deltas, far
    # below the tile's largest.  Their scores must keep full precision (the
    # kernel takes a per-row reference there); every row's O and lse against
    # the oracle on the same delta.
    S = 520
    wl, x = make_small(1, 8, 2, S - q0, S, 128, 48, dtype="bf16", q_offset=q0, seed=77,
                       device="cuda")
    g = torch.Generator().manual_seed(5)
    d = (torch.rand(1, 2, S, generator=g) * 4 + 1)
    for j, v in ((100, 1.0e4), (150, 2.5e4), (333, 3.0e4), (334, 3.0e4 + 1.0), (470, 8.0e3)):
        d[0, j % 2, j] = v
    d = d.cuda()
    gm = dma.topk_mask(d, wl.Sq, q0, wl.w)
    O, lse = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, return_lse=True)
    Oi = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm)
    torch.cuda.synchronize()
    rows = _all_rows(wl)
    Or, Lr = oracle.attn_rows(x["Q"], x["K"], x["V"], to64(d), q0, wl.w, rows)
    m, r = compare_rows(O, lse, Or, Lr, rows, "bf16", "large delta births")
    compare_rows(Oi, None, Or, Lr, rows, "bf16", "large delta births (no lse)")
    # the rows in front of a birth have lse near their own small deltas
    lg = lse[0].cpu().double().numpy()
    lr = Lr.reshape(wl.Hq, wl.Sq)
    small = np.abs(lr) < 100
    err = np.abs(lg - lr)[small]
    print(f"large births q0={q0}: max abs {m:.2e}, lse err over {small.sum()} small-delta rows "
          f"{err.max():.2e}")
    assert small.sum() > 100 and err.max() <= 2e-4


@pytest.mark.parametrize("B,Hq,Hkv,S,w,seed", [
    (1, 8, 2, 1024, 128, 1),   # 16 query tiles, lists much shorter than the prefix
    (2, 4, 1, 640, 300, 2),    # G = 4, a partial last query tile
    (1, 4, 2, 256, 256, 3),    # w >= S: every key kept
])
def test_natural_order_lists(gpu_lib, B, Hq, Hkv, S, w, seed):
    """Natural-order block skipping (every key of each query tile's active
    64-key tiles, per-element keep test) is the comparison schedule of the
    bench's --natural-ab mode; on the same kernel it must give the oracle's
    outputs on every row, as the gathered lists do."""
    from trainable_dynamic_mask_amd.blockskip import chunk_counts, natural_order_mask
    wl, x = make_small(B, Hq, Hkv, S, S, 128, w, dtype="bf16", delta_std=0.05, seed=seed,
                       device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, wl.Sq, wl.q_offset, wl.w, kt_lists=True)
    nat = natural_order_mask(gm)
    On, lse_n = dma.attn_fwd(x["Q"], x["K"], x["V"], d, nat, return_lse=True)
    torch.cuda.synchronize()
    rows = _all_rows(wl)
    Or, Lr = _oracle_rows(x, d, wl, rows)
    compare_rows(On, lse_n, Or, Lr, rows, "bf16", f"natural {(B, Hq, Hkv, S, w)}")
    cg, cn = chunk_counts(gm, nat)
    # every active key tile is visited whole, so the natural schedule does at
    # least the gathered lists' work
    assert cn >= cg
