"""Workload shapes of the Dynamic Mask Attention forward.

Six synthetic workloads: a tiny fp32 causal case, two bf16 GQA prefills
(4K and 16K tokens), a 64K-token prefill whose dynamic weights are heavy
tailed, a batched decode step against a 32K-token cache, and a chunked
prefill (the last 4K tokens of a 16K sequence, against the 12K before them
as cache).  The method
(dynamic weights, causal top-w keep mask, masked softmax attention) is the
one stated on the Hugging Face blog "Trainable Dynamic Mask Sparse
Attention" (sections "Dynamic Sparse Mask Generation", "Mask Combination
with Causal Constraints", "Efficient Sparse Attention Computation").
"""
from dataclasses import dataclass, asdict


def sum_range(a: int, b: int) -> int:
    """a + (a+1) + ... + b for a <= b."""
    return (a + b) * (b - a + 1) // 2


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage type of Q, K, V and O
    B: int
    Hq: int
    Hkv: int
    Sq: int             # query rows per sequence
    Sk: int             # key rows per sequence
    q_offset: int       # absolute position of query row 0
    D: int
    w: int              # keys kept per query row
    delta_std: float    # standard deviation of the Delta matrix entries
    seed: int

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kept_pairs(self) -> int:
        """Kept (query head, query row, key) triples: row p keeps min(p+1, w) keys."""
        lo, hi = self.q_offset, self.q_offset + self.Sq      # rows p in [lo, hi)
        m = min(hi, self.w)
        part = sum_range(lo + 1, m) if m > lo else 0         # rows p < w keep p+1 keys
        full = max(0, hi - max(lo, self.w)) * self.w         # rows p >= w keep w keys
        return (part + full) * self.B * self.Hq

    def effective_flops(self) -> int:
        """4*D flops per kept pair: 2*D for the score, 2*D for the weighted value sum."""
        return 4 * self.D * self.kept_pairs()

    def as_dict(self):
        return asdict(self)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", B=1, Hq=2, Hkv=2, Sq=256, Sk=256, q_offset=0,
                         D=64, w=64, delta_std=0.02, seed=1000),
    "prefill_4k": Workload("prefill_4k", "bf16", B=2, Hq=32, Hkv=8, Sq=4096, Sk=4096, q_offset=0,
                           D=128, w=2048, delta_std=0.02, seed=1001),
    "prefill_16k": Workload("prefill_16k", "bf16", B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384,
                            q_offset=0, D=128, w=2048, delta_std=0.02, seed=1002),
    "prefill_64k": Workload("prefill_64k", "bf16", B=1, Hq=32, Hkv=8, Sq=65536, Sk=65536,
                            q_offset=0, D=128, w=4096, delta_std=0.05, seed=1003),
    "decode_32k": Workload("decode_32k", "bf16", B=64, Hq=32, Hkv=8, Sq=1, Sk=32768,
                           q_offset=32767, D=128, w=2048, delta_std=0.02, seed=1004),
    "chunk_16k": Workload("chunk_16k", "bf16", B=1, Hq=32, Hkv=8, Sq=4096, Sk=16384,
                          q_offset=12288, D=128, w=2048, delta_std=0.02, seed=1005),
}

HEADLINE = "prefill_16k"
