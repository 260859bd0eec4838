"""CPU checks of the C ABI library: it loads, exports every function that
include/dma.h declares, and rejects bad arguments on the host before any
launch (no GPU needed for these paths)."""
import ctypes
import math
import os
import re

import pytest

from trainable_dynamic_mask_amd import _lib
from trainable_dynamic_mask_amd._lib import DmaMask, DmaMaskDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10004)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dma.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dma_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_versions(lib):
    assert lib.dma_status_string(0) == b"ok"
    assert lib.dma_status_string(3) == b"workspace too small"
    assert lib.dma_abi_version() == 6
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    lib.dma_tile_sizes(ctypes.byref(bq), ctypes.byref(bk))
    assert (bq.value, bk.value) == (64, 64)


def _dims(lib, *args):
    d = DmaMaskDims()
    return lib.dma_mask_dims_for(*args, ctypes.byref(d)), d


def test_mask_dims(lib):
    rc, d = _dims(lib, 1, 8, 16384, 16384, 0, 2048)
    assert rc == OK
    assert (d.n_tiles, d.n_tiles_total, d.u_stride, d.kt_stride) == (256, 2048, 2111, 256)
    assert d.evict_elems == 8 * 16384 and d.u_elems == 2048 * 2111
    rc, d = _dims(lib, 64, 8, 1, 32768, 32767, 2048)      # one decode row
    assert rc == OK and d.u_stride == 2048 and d.evict_elems == 0
    rc, d = _dims(lib, 1, 1, 10, 10, 0, 50)                # w larger than the sequence
    assert rc == OK and d.u_stride == 10
    assert _dims(lib, 1, 1, 10, 9, 0, 5)[0] == INVALID     # rows past the keys
    assert _dims(lib, 1, 1, 5, 10, 6, 5)[0] == INVALID     # q_offset + Sq > Sk
    assert _dims(lib, 1, 1, 10, 10, 0, 0)[0] == INVALID    # w < 1
    assert _dims(lib, 1, 0, 10, 10, 0, 3)[0] == INVALID    # no heads
    assert _dims(lib, 1, 1, 2, (1 << 20) + 1, 0, 3)[0] == UNSUPPORTED
    assert _dims(lib, 1, 1, 1, 40000, 39999, 3)[0] == OK  # decode rows of any length
    assert _dims(lib, 70000, 1, 2, 2, 0, 1)[0] == UNSUPPORTED


def test_workspace_sizes(lib):
    # sort buffers and ranks, plus 32 groups of 8 tiles with candidate lists (w + 512 keys, 8 bytes)
    assert lib.dma_topk_workspace_bytes(1, 8, 16384, 16384, 2048) >= 8 * 16384 * 20 + 8 * 32 * 2560 * 8
    assert lib.dma_topk_workspace_bytes(1, 8, 1, 16384, 2048) == 0
    assert lib.dma_attn_workspace_bytes(2, 32, 4096, 128, 2048) == 0
    # one-row attention: a (max, sum, o[128]) partial per query head and split; the
    # bf16 kernel splits the 2048-entry list into 32 waves of 64 entries, the generic
    # one into 8 pieces of 256: the workspace covers the larger count
    assert lib.dma_attn_workspace_bytes(64, 32, 1, 128, 2048) == 64 * 32 * 32 * 130 * 4
    assert lib.dma_attn_workspace_bytes(1, 2, 1, 64, 100) == 1 * 2 * 2 * 66 * 4


def _weights(lib, V=FAKE, vt=1, B=1, Sk=16, Hkv=2, D=64, sb=None, ss=None, Dl=FAKE, A=FAKE,
             out=FAKE):
    ss = Hkv * D if ss is None else ss
    sb = ss * Sk if sb is None else sb
    return lib.dma_weights(V, vt, B, Sk, Hkv, D, sb, ss, Dl, A, out, None)


def test_weights_validation(lib):
    assert _weights(lib, D=96) == UNSUPPORTED
    assert _weights(lib, Hkv=32, D=128) == UNSUPPORTED       # value row over 2048
    assert _weights(lib, Hkv=0) == INVALID
    assert _weights(lib, vt=7) == INVALID
    assert _weights(lib, V=None) == INVALID
    assert _weights(lib, out=None) == INVALID
    assert _weights(lib, V=MISALIGNED) == INVALID
    assert _weights(lib, ss=100) == INVALID                  # row stride below Hkv*D
    assert _weights(lib, ss=132) == INVALID                  # 264-byte rows: not 16-aligned
    assert _weights(lib, B=0, V=None) == OK                  # empty: nothing launched
    assert _weights(lib, Sk=0, V=None) == OK


def _vproj(lib, B=1, Sk=16, Cin=128, xsb=None, xss=None, X=FAKE, Wv=FAKE, Hkv=2, D=128, V=FAKE,
           vsb=None, vss=None, Delta=FAKE, A=FAKE, delta=FAKE, ws=FAKE, ws_bytes=1 << 30):
    xss = Cin if xss is None else xss
    xsb = xss * Sk if xsb is None else xsb
    vss = Hkv * D if vss is None else vss
    vsb = vss * Sk if vsb is None else vsb
    return lib.dma_vproj_weights(X, B, Sk, Cin, xsb, xss, Wv, Hkv, D, V, vsb, vss, Delta, A,
                                 delta, ws, ws_bytes, None)


def test_vproj_validation(lib):
    assert _vproj(lib, Cin=96) == UNSUPPORTED                # K steps of 64
    assert _vproj(lib, Hkv=1, D=128) == UNSUPPORTED          # 128 columns: tiles of 256
    assert _vproj(lib, Hkv=32, D=128) == UNSUPPORTED         # over 2048 columns
    assert _vproj(lib, Hkv=16, D=64) == UNSUPPORTED          # delta for more than 8 heads
    assert _vproj(lib, Hkv=16, D=64, delta=None, ws=None, ws_bytes=0, B=0) == OK
    assert _vproj(lib, Cin=0) == INVALID
    assert _vproj(lib, X=None) == INVALID
    assert _vproj(lib, Wv=None) == INVALID
    assert _vproj(lib, A=None) == INVALID                    # delta asked without A
    assert _vproj(lib, X=MISALIGNED) == INVALID
    assert _vproj(lib, xss=100) == INVALID                   # row stride below Cin
    assert _vproj(lib, xss=132) == INVALID                   # 264-byte rows: not 16-aligned
    assert _vproj(lib, vss=200) == INVALID                   # row stride below Hkv*D
    assert _vproj(lib, ws=None) == WORKSPACE
    need = lib.dma_vproj_workspace_bytes(1, 16, 2, 128)
    assert need > 0 and _vproj(lib, ws_bytes=need - 1) == WORKSPACE
    assert _vproj(lib, B=0, X=None) == OK                    # empty: nothing launched
    assert lib.dma_vproj_workspace_bytes(0, 16, 2, 128) == 0


def _topk(lib, B=1, Hkv=2, Sq=16, Sk=16, q0=0, w=4, mask=True, ws=FAKE, ws_bytes=1 << 30):
    m = DmaMask(FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    return lib.dma_topk_mask(FAKE, B, Hkv, Sq, Sk, q0, w, ctypes.byref(m) if mask else None,
                             ws, ws_bytes, None)


def test_topk_validation(lib):
    assert _topk(lib, q0=1) == INVALID
    assert _topk(lib, w=0) == INVALID
    assert _topk(lib, mask=False) == INVALID
    assert _topk(lib, ws=None, ws_bytes=0) == WORKSPACE
    assert _topk(lib, ws_bytes=10) == WORKSPACE
    assert _topk(lib, ws=MISALIGNED) == INVALID
    assert _topk(lib, Sq=0, Sk=16, q0=16) == OK
    assert _topk(lib, B=0) == OK
    m = DmaMask(None, FAKE, FAKE, FAKE, FAKE, None, None)       # evict missing for Sq > 1
    assert lib.dma_topk_mask(FAKE, 1, 2, 16, 16, 0, 4, ctypes.byref(m), FAKE, 1 << 30, None) == INVALID
    m = DmaMask(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)       # kt_idx without kt_cnt
    assert lib.dma_topk_mask(FAKE, 1, 2, 16, 16, 0, 4, ctypes.byref(m), FAKE, 1 << 30, None) == INVALID


def _append(lib, B=2, Hkv=2, Sk=17, w=16, kt=False, mask=True, delta=FAKE):
    m = DmaMask(None, FAKE, FAKE, FAKE, FAKE, FAKE if kt else None, FAKE if kt else None)
    return lib.dma_decode_keep_append(delta, B, Hkv, Sk, w, ctypes.byref(m) if mask else None,
                                      None)


def test_decode_append_validation(lib):
    assert _append(lib, Sk=16) == INVALID                    # keep(Sk-2) would not be full
    assert _append(lib, w=0) == INVALID
    assert _append(lib, kt=True) == INVALID                  # key-tile lists are not kept
    assert _append(lib, mask=False) == INVALID
    assert _append(lib, delta=None) == INVALID
    assert _append(lib, Sk=70000, w=40000) == UNSUPPORTED    # a list larger than LDS holds
    assert _append(lib, B=0) == OK                           # empty: nothing launched


def _attn(lib, t=1, B=1, Sq=16, Sk=16, Hq=4, Hkv=2, D=128, qs=None, ks=None, q0=0, w=4,
          scale=0.0, Q=FAKE, O=FAKE, ws=None, ws_bytes=0, dlo=FAKE):
    qs = qs or (Sq * Hq * D, Hq * D, D)
    ks = ks or (Sk * Hkv * D, Hkv * D, D)
    m = DmaMask(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, dlo)
    return lib.dma_attn_fwd(Q, FAKE, FAKE, t, B, Sq, Sk, Hq, Hkv, D, (ctypes.c_int64 * 3)(*qs),
                            (ctypes.c_int64 * 3)(*ks), q0, w, FAKE, ctypes.byref(m), scale, O,
                            None, ws, ws_bytes, None)


def test_attn_validation(lib):
    assert _attn(lib, Hq=3) == INVALID                       # Hq not a multiple of Hkv
    assert _attn(lib, D=96) == UNSUPPORTED
    assert _attn(lib, D=64) == UNSUPPORTED                   # bf16 prefill is built for D=128
    assert _attn(lib, scale=math.nan) == INVALID
    assert _attn(lib, Q=MISALIGNED) == INVALID
    assert _attn(lib, O=None) == INVALID
    assert _attn(lib, qs=(16 * 4 * 128, 4 * 128, 100)) == INVALID   # head stride below D
    assert _attn(lib, ks=(16 * 2 * 128, 2 * 128 + 3, 128)) == INVALID  # odd row stride
    assert _attn(lib, Sq=1, Sk=16, q0=15) == WORKSPACE       # decode row needs split partials
    assert _attn(lib, dlo=None) == INVALID                   # bf16 prefill reads u_dlo
    # bf16 prefill gathers: 32-bit row offsets, 24-bit index and stride products
    assert _attn(lib, Sk=70000, q0=69984, ks=(70000 << 16, 1 << 16, 128)) == UNSUPPORTED
    assert _attn(lib, ks=(16 << 23, 1 << 23, 128)) == UNSUPPORTED
    assert _attn(lib, Sk=(1 << 24) + 1, q0=(1 << 24) - 15, ks=(0, 0, 128)) == UNSUPPORTED
    assert _attn(lib, Sq=0, q0=16) == OK
    assert _attn(lib, B=0) == OK


def _bwd(lib, t=1, B=1, Sq=16, Sk=16, Hq=4, Hkv=2, D=128, q0=0, w=4, lse=FAKE, Ores=None,
         dQ=FAKE, ws=FAKE, ws_bytes=1 << 30):
    qs = (Sq * Hq * D, Hq * D, D)
    ks = (Sk * Hkv * D, Hkv * D, D)
    m = DmaMask(FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    return lib.dma_attn_bwd(FAKE, FAKE, FAKE, t, B, Sq, Sk, Hq, Hkv, D,
                            (ctypes.c_int64 * 3)(*qs), (ctypes.c_int64 * 3)(*ks), q0, w, FAKE,
                            ctypes.byref(m), 0.0, FAKE, Ores, lse, FAKE, dQ, FAKE, FAKE, FAKE, ws,
                            ws_bytes, None)


def test_attn_bwd_validation(lib):
    assert _bwd(lib, t=0) == UNSUPPORTED                     # fp32 backward is not built
    assert _bwd(lib, D=64) == UNSUPPORTED
    assert _bwd(lib, Sq=1, Sk=16, q0=15) == UNSUPPORTED       # one decode row
    assert _bwd(lib, lse=None) == INVALID                     # the forward's lse is required
    assert _bwd(lib, dQ=MISALIGNED) == INVALID
    assert _bwd(lib, Ores=MISALIGNED) == INVALID
    assert _bwd(lib, ws_bytes=100) == WORKSPACE
    assert _bwd(lib, ws=ctypes.c_void_p(0x10010)) == INVALID  # workspace is 256-byte aligned
    assert _bwd(lib, B=0) == OK
    assert lib.dma_attn_bwd_workspace_bytes(1, 4, 2, 1, 16, 4) == 0
    assert lib.dma_attn_bwd_workspace_bytes(1, 32, 8, 16384, 16384, 2048) > 0


def test_fwd_train_and_weights_bwd_validation(lib):
    qs = (ctypes.c_int64 * 3)(16 * 4 * 128, 4 * 128, 128)
    ks = (ctypes.c_int64 * 3)(16 * 2 * 128, 2 * 128, 128)
    m = DmaMask(FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    fwd = lambda t, Ores: lib.dma_attn_fwd_train(FAKE, FAKE, FAKE, t, 1, 16, 16, 4, 2, 128, qs,
                                                  ks, 0, 4, FAKE, ctypes.byref(m), 0.0, FAKE,
                                                  FAKE, Ores, None)
    assert fwd(0, FAKE) == UNSUPPORTED                        # fp32: no residual output
    assert fwd(1, None) == INVALID                            # the residual buffer is required
    assert fwd(1, MISALIGNED) == INVALID
    wb = lambda vt=1, D=128, Hkv=2, ws_bytes=1 << 20: lib.dma_weights_bwd(
        FAKE, vt, 1, 16, Hkv, D, 16 * Hkv * D, Hkv * D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        ws_bytes, None)
    assert wb(vt=0) == UNSUPPORTED
    assert wb(D=96) == UNSUPPORTED
    assert wb(Hkv=32) == UNSUPPORTED                          # Hkv*D above 2048
    assert wb(ws_bytes=4) == WORKSPACE
    assert lib.dma_weights_bwd_workspace_bytes(2, 10, 3) == 2 * 10 * 3 * 4


def test_safe_sync_build_loads_with_the_same_exports():
    # the cross-check build (every attention barrier waits for all loads) is the
    # same library: it loads and exports every declared function
    safe = _lib.load_safe()
    for n in declared_functions():
        assert hasattr(safe, n), n
    assert safe.dma_abi_version() == _lib.load().dma_abi_version()


def test_noalloc_mask_rejects_more_than_its_scratch(lib):
    # the static scratch holds 64 MiB; a call that needs more is refused on the
    # host before anything is enqueued
    m = DmaMask(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE)
    assert lib.dma_topk_workspace_bytes(1, 16, 65536, 65536, 4096) > (64 << 20)
    assert lib.dma_topk_mask_noalloc(FAKE, 1, 16, 65536, 65536, 0, 4096, ctypes.byref(m),
                                     None) == WORKSPACE
    assert lib.dma_topk_mask_noalloc(FAKE, 1, 8, 16, 16, 0, 0, ctypes.byref(m), None) == INVALID
