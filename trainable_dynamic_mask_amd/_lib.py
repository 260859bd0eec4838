"""ctypes loader of the in-tree HIP library (libdma_hip.so) and its C ABI.

The library must have been built (``python -m trainable_dynamic_mask_amd.build``
or ``__graft_entry__.build()``); nothing here falls back to another
implementation: a missing library raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdma_hip.so")
LIB_SAFE_PATH = os.path.join(HERE, "libdma_hip_safe.so")

DMA_F32 = 0
DMA_BF16 = 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace too small",
          4: "HIP runtime error"}

_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t


class DmaMask(ctypes.Structure):
    _fields_ = [("evict", _P), ("u_idx", _P), ("u_cnt", _P), ("u_nfull", _P), ("u_dmax", _P),
                ("kt_idx", _P), ("kt_cnt", _P), ("u_dlo", _P), ("u_dval", _P)]


class DmaMaskDims(ctypes.Structure):
    _fields_ = [("n_tiles", _I64), ("n_tiles_total", _I64), ("u_stride", _I64),
                ("kt_stride", _I64), ("evict_elems", _I64), ("u_elems", _I64),
                ("kt_elems", _I64)]


EXPORTS = ["dma_status_string", "dma_abi_version", "dma_tile_sizes", "dma_mask_dims_for",
           "dma_topk_workspace_bytes", "dma_attn_workspace_bytes", "dma_weights",
           "dma_topk_mask", "dma_topk_mask_noalloc", "dma_decode_keep_append", "dma_attn_fwd",
           "dma_attn_fwd_train", "dma_attn_bwd_workspace_bytes", "dma_attn_bwd",
           "dma_weights_bwd_workspace_bytes", "dma_weights_bwd", "dma_vproj_workspace_bytes",
           "dma_vproj_weights"]

_lib = None
_lib_safe = None


class DmaError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} (status {code})")
        self.code = code


def load():
    """Load the library (once) and declare the C signatures."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_safe():
    """The cross-check build of the same library (every barrier of the
    hand-synchronised attention waits for all loads in flight); the tests
    compare its results bit for bit with load()'s."""
    global _lib_safe
    if _lib_safe is None:
        _lib_safe = _open(LIB_SAFE_PATH)
    return _lib_safe


def _open(path):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m trainable_dynamic_mask_amd.build`")
    lib = ctypes.CDLL(path)
    lib.dma_status_string.argtypes = [ctypes.c_int]
    lib.dma_status_string.restype = ctypes.c_char_p
    lib.dma_abi_version.restype = ctypes.c_int
    lib.dma_tile_sizes.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.dma_tile_sizes.restype = None
    lib.dma_mask_dims_for.argtypes = [_I64, _I64, _I64, _I64, _I64, _I64,
                                      ctypes.POINTER(DmaMaskDims)]
    lib.dma_mask_dims_for.restype = ctypes.c_int
    lib.dma_topk_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64]
    lib.dma_topk_workspace_bytes.restype = _SZ
    lib.dma_attn_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64]
    lib.dma_attn_workspace_bytes.restype = _SZ
    lib.dma_weights.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                                _P]
    lib.dma_weights.restype = ctypes.c_int
    lib.dma_topk_mask.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _I64,
                                  ctypes.POINTER(DmaMask), _P, _SZ, _P]
    lib.dma_topk_mask.restype = ctypes.c_int
    lib.dma_topk_mask_noalloc.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _I64,
                                          ctypes.POINTER(DmaMask), _P]
    lib.dma_topk_mask_noalloc.restype = ctypes.c_int
    lib.dma_decode_keep_append.argtypes = [_P, _I64, _I64, _I64, _I64, ctypes.POINTER(DmaMask), _P]
    lib.dma_decode_keep_append.restype = ctypes.c_int
    lib.dma_attn_fwd.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _I64,
                                 ctypes.POINTER(_I64), ctypes.POINTER(_I64), _I64, _I64, _P,
                                 ctypes.POINTER(DmaMask), ctypes.c_float, _P, _P, _P, _SZ, _P]
    lib.dma_attn_fwd.restype = ctypes.c_int
    lib.dma_attn_bwd_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64, _I64]
    lib.dma_attn_bwd_workspace_bytes.restype = _SZ
    lib.dma_attn_bwd.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _I64,
                                 ctypes.POINTER(_I64), ctypes.POINTER(_I64), _I64, _I64, _P,
                                 ctypes.POINTER(DmaMask), ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                 _P, _P, _P, _SZ, _P]
    lib.dma_attn_bwd.restype = ctypes.c_int
    lib.dma_attn_fwd_train.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                                       _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64), _I64,
                                       _I64, _P, ctypes.POINTER(DmaMask), ctypes.c_float, _P, _P,
                                       _P, _P]
    lib.dma_attn_fwd_train.restype = ctypes.c_int
    lib.dma_weights_bwd_workspace_bytes.argtypes = [_I64, _I64, _I64]
    lib.dma_weights_bwd_workspace_bytes.restype = _SZ
    lib.dma_weights_bwd.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P,
                                    _P, _P, _P, _P, _P, _SZ, _P]
    lib.dma_weights_bwd.restype = ctypes.c_int
    lib.dma_vproj_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64]
    lib.dma_vproj_workspace_bytes.restype = _SZ
    lib.dma_vproj_weights.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P, _I64,
                                      _I64, _P, _P, _P, _P, _SZ, _P]
    lib.dma_vproj_weights.restype = ctypes.c_int
    return lib


def check(fn, code):
    if code != 0:
        raise DmaError(fn, code)
