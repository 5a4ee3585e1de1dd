"""Workload shapes for the slot-mapped attention engine.

Five synthetic workloads, shaped like the attention of LLaDA-8B (32 layers,
32 MHA heads, head_dim 128) and Dream-7B (28 layers, 28 query / 4 KV heads,
head_dim 128), with the generation length 256 and block length 32 of
"Affix Cache for Diffusion Large Language Models", Section 5 (Default
Settings), and the three affix placements of its Appendix A (prefix
Ex.Qry.Mask, infix Qry_head.Ex.Ans.Mask, suffix Qry.Mask.Ex).

This module holds layout bookkeeping only: where the affix sits, how many
request and generation positions there are.  It computes nothing that the
method computes (no anchor count, no slot maps); each side derives those on
its own.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    dtype: str                      # "f32" or "bf16": storage/compute type of Q, K, V, O
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    # logical layout of one request: ("affix"|"req"|"gen", length) in order
    segments: Tuple[Tuple[str, int], ...]
    batch: int
    rate: float                     # anchor ratio
    page_size: int = 16
    page_order: str = "identity"    # identity | random | fragmented
    shared_slot_order: str = "page"  # page (page-granular) | slot (slot-granular shuffle)
    key_tweak: str = "none"         # none | sinks | heavy
    n_sinks: int = 8
    sink_scale: float = 4.0
    heavy_frac: float = 0.01
    heavy_nu: float = 3.0
    block_len: int = 32             # decode block (queries per request per step)
    steps: int = 1                  # decode steps (one generation block each)
    free_frac: float = 0.0          # fraction of free pages interleaved (fragmented pool)

    # ---- layout bookkeeping -------------------------------------------------
    @property
    def affix_l(self) -> int:
        p = 0
        for kind, n in self.segments:
            if kind == "affix":
                return p
            p += n
        raise ValueError("no affix segment")

    @property
    def L(self) -> int:
        return sum(n for k, n in self.segments if k == "affix")

    @property
    def T(self) -> int:
        return sum(n for _, n in self.segments)

    @property
    def P(self) -> int:
        """Non-affix positions per request (request tokens + generation)."""
        return self.T - self.L

    @property
    def m(self) -> int:
        """Initially masked (generation) positions per request."""
        return sum(n for k, n in self.segments if k == "gen")

    def positions(self, kind):
        """Logical positions of one request that belong to segments of `kind`."""
        out, p = [], 0
        for k, n in self.segments:
            if k == kind:
                out.extend(range(p, p + n))
            p += n
        return out

    def non_affix_positions(self):
        return [p for p in range(self.T) if not (self.affix_l <= p < self.affix_l + self.L)]

    def gen_start(self) -> int:
        return self.positions("gen")[0]

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload(1, "tiny-fp32", "f32", 1, 2, 2, 16,
                (("affix", 64), ("req", 16), ("gen", 32)), 1, 0.2,
                page_order="identity"),
    2: Workload(2, "llada-probe-L1024", "bf16", 32, 32, 32, 128,
                (("affix", 1024), ("req", 128), ("gen", 256)), 1, 0.2,
                key_tweak="sinks"),
    3: Workload(3, "dream-infix-L2048", "bf16", 28, 28, 4, 128,
                (("req", 64), ("affix", 2048), ("req", 64), ("gen", 256)), 16, 0.2,
                page_order="random"),
    4: Workload(4, "llada-prefix-L4096-b16", "bf16", 32, 32, 32, 128,
                (("affix", 4096), ("req", 256), ("gen", 256)), 16, 0.2,
                page_order="random"),
    5: Workload(5, "llada-suffix-L16384-b32", "bf16", 32, 32, 32, 128,
                (("req", 512), ("gen", 256), ("affix", 16384)), 32, 0.3,
                page_order="fragmented", key_tweak="heavy", steps=8, free_frac=0.125),
}

# the workload the headline measurement is taken on (affix L=4096)
BENCH_WORKLOAD = 4
