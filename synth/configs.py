"""The five synthetic workloads of the DSA decode step, as named specs.

Shapes follow the decode setting described on the GLM-5.2 shared-Indexer
offload page (lmnt.cn, sections 2.1 and 4.1: top-2048 selection, groups of 4
layers sharing one top-k) and the MLA latent row of the TokenSpeed audit page
(devpress.csdn.net, "MLA (tokenspeed-mla)": 512 latent + 64 rope, one row used as
both K and V).  Sizes, head counts and value distributions are those of the
workload definitions; every tensor is drawn from a seeded generator.

A spec can be shrunk with ``spec(cid).scaled(...)`` for parity cases that the
oracle finishes in seconds while still spanning several tiles and a ragged tail.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadSpec:
    cid: int
    name: str
    B: int                      # requests in the batch
    Sq: int                     # query tokens per request (1 = plain decode)
    L: int                      # cache length per request (fixed-length configs)
    page_size: int = 64
    # indexer
    idx_heads: int = 64
    idx_dim: int = 128
    idx_q_kind: str = "bf16"    # "grid_f32" | "bf16" | "e4m3"
    idx_k_kind: str = "e4m3_scaled"  # "grid_f32" | "e4m3_scaled" | "mxfp4"
    w_kind: str = "u01_div64"   # "quarters" | "u01_div64"
    draft_sigma: float = 0.0    # > 0: query t >= 1 of a request is query 0 + draft_sigma * its own draw
    topk: int = 2048
    # MLA
    mla_heads: int = 128
    kv_dim: int = 576
    v_dim: int = 512
    # mixed-length share (page-sharded cache)
    lens_kind: str = "fixed"    # "fixed" | "loguniform_plus_long"
    n_short: int = 0
    short_lo: int = 0
    short_hi: int = 0
    n_long: int = 0
    long_len: int = 0
    n_ranks: int = 1
    rank: int = 0
    # device pool group (set-associative FIFO)
    steps: int = 0
    layers: int = 0
    n_sets: int = 0
    ways: int = 0
    id_range: int = 0
    keep_frac: float = 0.0
    zipf_a: float = 0.0
    seed: int = 0

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(576) for every workload
        return 1.0 / math.sqrt(self.kv_dim)

    def scaled(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: WorkloadSpec(cid=1, name="tiny", B=1, Sq=1, L=4096, idx_heads=4, idx_dim=64,
                    idx_q_kind="grid_f32", idx_k_kind="grid_f32", w_kind="quarters",
                    topk=256, mla_heads=16),
    2: WorkloadSpec(cid=2, name="decode_b32_64k", B=32, Sq=1, L=65536),
    3: WorkloadSpec(cid=3, name="mtp_verify_b8_200k", B=8, Sq=4, L=200000 + 4,
                    idx_q_kind="e4m3"),
    4: WorkloadSpec(cid=4, name="pool_group_b16_128k", B=16, Sq=1, L=131072,
                    steps=8, layers=4, n_sets=1024, ways=8, id_range=131072,
                    keep_frac=0.6, zipf_a=1.1),
    5: WorkloadSpec(cid=5, name="rank0_share_mixed", B=66, Sq=1, L=0,
                    lens_kind="loguniform_plus_long", n_short=64, short_lo=30000,
                    short_hi=200000, n_long=2, long_len=1_000_000, n_ranks=4, rank=0),
}


def spec(cid: int) -> WorkloadSpec:
    return CONFIGS[cid]
