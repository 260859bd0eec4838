"""Guards on the gfx950 machine code of the kernels (CPU: compiles to assembly only).

- Direct global-to-LDS loads take their LDS address in m0, which must come
  from a scalar register; an address the compiler keeps in a vector register
  would still assemble as a move from it, and the loads would land at the
  wrong address.
- No 64-bit LDS atomics: an 8-byte LDS atomic at an address that is not
  8-byte aligned faults the GPU, and dynamic LDS placement is not fixed by
  the source alone.
- No packed fp32 arithmetic: the build disables it for all device code.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

import trainable_dynamic_mask_amd.build as B

SOURCES = ["attn_prefill.hip", "attn_bwd.hip", "attn_decode.hip", "topk.hip", "weights.hip",
           "attn_f32.hip"]


def _asm(src, out):
    cmd = ["hipcc", *[f for f in B.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _asm(s, str(d / (s + ".s"))), SOURCES))
    return dict(zip(SOURCES, texts))


def test_m0_is_set_from_scalars(isa):
    for src, text in isa.items():
        bad = re.findall(r"s_mov_b32\s+m0,\s*v\d+", text)
        assert not bad, (src, bad[:3])


def test_direct_loads_present_where_expected(isa):
    # the check above is only meaningful if the direct loads are there
    for src in ("attn_prefill.hip", "attn_bwd.hip", "attn_decode.hip", "topk.hip"):
        assert "global_load_lds_dwordx4" in isa[src], src


def test_no_64bit_lds_atomics(isa):
    pat = re.compile(r"\bds_(?:add|sub|rsub|inc|dec|min|max|and|or|xor|mskor|wrxchg|cmpst|cmpswap)"
                     r"(?:_rtn)?_(?:b64|u64|i64|f64)\b")
    for src, text in isa.items():
        bad = pat.findall(text)
        assert not bad, (src, bad[:3])


def test_no_packed_fp32(isa):
    pat = re.compile(r"\bv_pk_(?:add|mul|fma)_f32\b")
    for src, text in isa.items():
        assert not pat.findall(text), src
