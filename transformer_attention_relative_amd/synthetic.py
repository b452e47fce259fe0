"""Seeded synthetic workloads for relative-position attention.

This module holds only shapes, distributions and a seeded random generator:
none of the method's arithmetic.  Tests, the benchmark and the smoke check
use it to feed identical inputs to the HIP library and to the float64
oracle.

Recipe (every workload): ``torch.Generator('cpu').manual_seed(seed)``; all
draws are float32 ``randn`` times the stated standard deviation, in the
order Q, K, V, table, table2, then the per-sequence valid key lengths
(``randint(lo, hi + 1)``); Q/K/V (and the Shaw / DeBERTa tables) are then
rounded to the workload dtype on the CPU (round to nearest even).  The T5
bias table stays float32.  ALiBi slopes are not drawn: head h of H gets
-2^(-8(h+1)/H) (a geometric set of distance penalties, float32).  The
oracle consumes these rounded values upcast to float64.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "t5" | "shaw" | "deberta" | "alibi" | "txl"
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str                # "fp32" | "bf16"
    num_buckets: int = 32
    max_distance: int = 128
    bidirectional: bool = True
    clip_k: int = 0
    q_pos_offset: int = 0
    k_pos_offset: int = 0
    causal: bool = False
    valid_len_range: Optional[tuple] = None   # (lo, hi) inclusive, per sequence
    table_sigma: float = 0.5
    description: str = ""

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def table_shapes(self):
        """Shapes of (table, table2) for this kind."""
        if self.kind == "t5":
            return (self.num_buckets, self.H), None
        if self.kind == "alibi":
            return (self.H,), None
        if self.kind == "txl":
            return (self.clip_k, self.H, self.d), (2, self.H, self.d)
        if self.kind == "shaw":
            n = 2 * self.clip_k + 1
            return (n, self.d), (n, self.d)
        n = 2 * self.clip_k
        return (n, self.H, self.d), (n, self.H, self.d)


WORKLOADS = {
    "t5_tiny_fp32": Workload(
        name="t5_tiny_fp32", kind="t5", B=1, H=2, Lq=64, Lk=64, d=32, dtype="fp32",
        num_buckets=32, max_distance=128, bidirectional=True, table_sigma=0.5,
        description="T5 bucket bias, bidirectional 32/128, B1 H2 L64 d32 fp32, no mask"),
    "t5_encoder_padded": Workload(
        name="t5_encoder_padded", kind="t5", B=8, H=12, Lq=512, Lk=512, d=64,
        dtype="bf16", num_buckets=32, max_distance=128, bidirectional=True,
        valid_len_range=(256, 512), table_sigma=0.5,
        description="T5 encoder, bidirectional 32/128, B8 H12 L512 d64 bf16, "
                    "key padding with valid length U{256..512} per sequence"),
    "t5_decoder_kvcache": Workload(
        name="t5_decoder_kvcache", kind="t5", B=4, H=16, Lq=128, Lk=4096, d=64,
        dtype="bf16", num_buckets=32, max_distance=128, bidirectional=False,
        q_pos_offset=3968, causal=True, table_sigma=0.5,
        description="T5 causal decoder with KV cache: 128 queries at positions "
                    "3968..4095 against keys 0..4095, B4 H16 d64 bf16"),
    "alibi_causal_d128": Workload(
        name="alibi_causal_d128", kind="alibi", B=4, H=16, Lq=4096, Lk=4096, d=128,
        dtype="bf16", causal=True,
        description="ALiBi causal with 128-wide heads, slopes -2^(-8(h+1)/16), "
                    "B4 H16 L4096 d128 bf16"),
    "txl_memory": Workload(
        name="txl_memory", kind="txl", B=4, H=16, Lq=2048, Lk=4096, d=64, dtype="bf16",
        clip_k=4096, q_pos_offset=2048, causal=True, table_sigma=0.1,
        description="Transformer-XL: a 2048-token segment at positions 2048..4095 "
                    "attending to itself and a 2048-token memory, encodings "
                    "E [4096,16,64] and u, v [2,16,64] ~N(0,0.1), B4 H16 d64 bf16"),
    "t5_decode_evicted": Workload(
        name="t5_decode_evicted", kind="t5", B=4, H=16, Lq=1, Lk=3072, d=64,
        dtype="bf16", num_buckets=32, max_distance=128, bidirectional=False,
        q_pos_offset=4095, k_pos_offset=1024, causal=True, table_sigma=0.5,
        description="T5 causal decode step: one query at position 4095 against "
                    "a cache whose first 1024 keys were evicted (keys at "
                    "positions 1024..4095), B4 H16 d64 bf16"),
    "alibi_causal": Workload(
        name="alibi_causal", kind="alibi", B=4, H=16, Lq=4096, Lk=4096, d=64,
        dtype="bf16", causal=True,
        description="ALiBi causal, slopes -2^(-8(h+1)/16) per head, B4 H16 "
                    "L4096 d64 bf16"),
    "shaw_causal_k16": Workload(
        name="shaw_causal_k16", kind="shaw", B=4, H=16, Lq=4096, Lk=4096, d=64,
        dtype="bf16", clip_k=16, causal=True, table_sigma=0.1,
        description="Shaw relative keys+values, clip 16 (33 vectors shared "
                    "across heads), B4 H16 L4096 d64 bf16, causal"),
    "deberta_k512": Workload(
        name="deberta_k512", kind="deberta", B=8, H=12, Lq=2048, Lk=2048, d=64,
        dtype="bf16", clip_k=512, causal=False, table_sigma=0.1,
        description="DeBERTa disentangled c2c+c2p+p2c, k=512 (1024 rows), "
                    "B8 H12 L2048 d64 bf16, bidirectional"),
}


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    """Draw the workload's tensors on the CPU (see the module docstring)."""
    g = torch.Generator("cpu").manual_seed(seed)
    qshape = (wl.B, wl.H, wl.Lq, wl.d)
    kshape = (wl.B, wl.H, wl.Lk, wl.d)
    q = torch.randn(qshape, generator=g, dtype=torch.float32)
    k = torch.randn(kshape, generator=g, dtype=torch.float32)
    v = torch.randn(kshape, generator=g, dtype=torch.float32)
    s1, s2 = wl.table_shapes()
    if wl.kind == "alibi":
        table = -torch.exp2(-8.0 * torch.arange(1, wl.H + 1, dtype=torch.float32) / wl.H)
    else:
        table = torch.randn(s1, generator=g, dtype=torch.float32) * wl.table_sigma
    table2 = None
    if s2 is not None:
        table2 = torch.randn(s2, generator=g, dtype=torch.float32) * wl.table_sigma
    kv_valid_len = None
    if wl.valid_len_range is not None:
        lo, hi = wl.valid_len_range
        kv_valid_len = torch.randint(lo, hi + 1, (wl.B,), generator=g, dtype=torch.int32)
    dt = wl.torch_dtype
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if wl.kind in ("shaw", "deberta", "txl"):
        table = table.to(dt)
        table2 = table2.to(dt)
    return {"q": q, "k": k, "v": v, "table": table, "table2": table2,
            "kv_valid_len": kv_valid_len}


def params_of(wl: Workload) -> dict:
    """Keyword arguments shared by the library binding and the oracle."""
    return dict(num_buckets=wl.num_buckets, max_distance=wl.max_distance,
                bidirectional=wl.bidirectional, clip_k=wl.clip_k,
                q_pos_offset=wl.q_pos_offset, k_pos_offset=wl.k_pos_offset,
                causal=wl.causal)
