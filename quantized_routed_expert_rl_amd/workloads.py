"""Named synthetic workloads for the routed-expert MoE layer.

Each workload fixes a layer shape (hidden size H, experts E, top-k, expert
width F), the number of stacked layers, the token schedule and the routing
skew.  The shapes are those of the Qwen3-Next-style decoder that the Red Lite
notes run (48 layers, 512 routed experts, top-10, hidden 2048, expert width
512; "Red Lite dev21 - GPU-routed decode", section "What changed", and
"Red Lite dev38", section "Finding"), plus one tiny shape that a pure-Python
check finishes in seconds.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # stream id used in every seed of this workload
    hidden: int              # H
    n_experts: int           # E
    top_k: int               # k
    width: int               # F (expert intermediate width)
    n_layers: int            # L
    tokens: int              # decode: tokens per run; prefill: prompt length
    chunks: Tuple[int, ...] = field(default=())   # prefill chunk sizes
    plan_cap: int = 512      # distinct experts per prefill plan
    zipf: bool = False       # per-expert Zipf(1.1) router bias
    resident: int = -1       # resident (layer, expert) entries; -1 = all
    qbits: int = 2
    popular: bool = False    # resident entries: each layer's most popular experts

    @property
    def mode(self) -> str:
        return "prefill" if self.chunks else "decode"


WORKLOADS = {
    # Tiny layer: every result checkable by the pure-Python brute force.
    "tiny": Workload("tiny", 0, 256, 16, 2, 64, 1, 4),
    # One layer at real shape, single-token decode, all 512 experts resident.
    "decode_1l": Workload("decode_1l", 1, 2048, 512, 10, 512, 1, 256),
    # 48 stacked decode layers, Zipf-skewed routing, 4608 of 48*512 resident.
    "decode_48l": Workload("decode_48l", 2, 2048, 512, 10, 512, 48, 256,
                           zipf=True, resident=4608),
    # 48 decode layers whose resident set is each layer's 224 most popular
    # experts under the Zipf bias (10752 of 24576, ~86 % of selections hit):
    # the regime of a bounded expert cache, served by loading misses.
    "decode_48l_hot": Workload("decode_48l_hot", 5, 2048, 512, 10, 512, 48, 64,
                               zipf=True, resident=48 * 224, popular=True),
    # One layer, one 512-token prefill chunk (5120 expert-token pairs).
    "prefill_1l": Workload("prefill_1l", 3, 2048, 512, 10, 512, 1, 512,
                           chunks=(512,), plan_cap=512),
    # 48 stacked prefill layers over a 1100-token prompt, Zipf routing.
    "prefill_48l": Workload("prefill_48l", 4, 2048, 512, 10, 512, 48, 1100,
                            chunks=(512, 512, 76), plan_cap=512, zipf=True),
}


def get(name: str, qbits: int = 2) -> Workload:
    w = WORKLOADS[name]
    if qbits != w.qbits:
        w = Workload(**{**w.__dict__, "qbits": qbits})
    return w
