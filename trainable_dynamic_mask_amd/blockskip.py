"""Natural-order block skipping, as a comparison configuration of the prefill
attention (DMA blog, "Hardware-Optimized Implementation": block-wise
computation that skips the blocks the mask leaves empty).

The mask step writes, for each 64-row query tile, its block-skip list kt_idx:
the 64-key tiles holding at least one key that some row of the tile keeps.
`natural_order_mask` turns a mask into the list form of natural-order block
processing: each query tile lists every key of those key tiles, ascending,
and every chunk takes the per-element keep test (no chunk is marked as kept
whole).  The eviction rows and the tiles' delta references are the mask's
own, so the attention kernel computes the same outputs from it (up to the
order of the floating-point sums) while doing the work of the block-skip
schedule instead of that of the gathered keep lists.  This is benchmark and
test infrastructure: nothing on the product path calls it.
"""
import torch

from . import Mask, mask_dims

_BK = 64  # keys per key tile (the mask step's block size)


def natural_order_mask(mask: Mask) -> Mask:
    """The natural-order block-skip form of a prefill mask (Sq > 1, built with
    its key-tile lists, Sk a multiple of 64)."""
    if mask.Sq <= 1 or mask.kt_idx is None or mask.kt_cnt is None:
        raise ValueError("natural_order_mask needs a prefill mask built with its key-tile lists")
    if mask.Sk % _BK:
        raise ValueError("natural_order_mask needs Sk to be a multiple of 64")
    B, Hkv, Sq, Sk, q0 = mask.B, mask.Hkv, mask.Sq, mask.Sk, mask.q_offset
    d = mask_dims(B, Hkv, Sq, Sk, q0, Sk)  # lists of up to Sk keys per tile
    n = d["n_tiles_total"]
    ks = mask.dims["kt_stride"]
    if d["u_stride"] != ks * _BK:
        raise ValueError("unexpected list stride")
    dev = mask.u_idx.device
    kt = mask.kt_idx[: n * ks].view(n, ks)
    cnt = mask.kt_cnt[:n].to(torch.int32)
    live = torch.arange(ks, device=dev, dtype=torch.int32)[None, :] < cnt[:, None]
    first = torch.where(live, kt, torch.zeros_like(kt)) * _BK
    keys = first[:, :, None] + torch.arange(_BK, device=dev, dtype=torch.int32)[None, None, :]
    u_idx = keys.reshape(n * ks * _BK).contiguous()
    return Mask(B, Hkv, Sq, Sk, q0, Sk, d,
                evict=mask.evict,
                u_idx=u_idx,
                u_cnt=(cnt * _BK).contiguous(),
                u_nfull=torch.zeros(n, dtype=torch.int32, device=dev),
                u_dmax=mask.u_dmax,
                kt_idx=None, kt_cnt=None,
                u_dlo=mask.u_dlo)


def chunk_counts(mask: Mask, natural: Mask):
    """Executed 64-key chunks of the gathered lists and of the natural-order
    lists, over all tiles."""
    n = mask.dims["n_tiles_total"]
    gathered = int(((mask.u_cnt[:n].to(torch.int64) + _BK - 1) // _BK).sum())
    nat = int((natural.u_cnt[:n].to(torch.int64) // _BK).sum())
    return gathered, nat
