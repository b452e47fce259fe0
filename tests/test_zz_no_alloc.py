"""relattn_fwd_noalloc, the entry point that allocates nothing (its workspace
is the library's fixed device scratch), against relattn_fwd with a
caller-owned workspace, through the C ABI: same kernels, so the outputs and
row LSEs must be identical.  Two calls in a row per case, the second with a
smaller input, so the second runs on the scratch the first left behind."""

import pytest
import torch

import transformer_attention_relative_amd as ra
from transformer_attention_relative_amd.synthetic import WORKLOADS, make_inputs, params_of

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# every kind of scratch use: split-KV partials (KV-cache step, one-token
# decode), per-key constants (DeBERTa in float32; in bfloat16 the kernel forms
# them itself), per-key and per-distance constants (Transformer-XL)
PAIRS = [
    (WORKLOADS["t5_decoder_kvcache"],
     WORKLOADS["t5_decoder_kvcache"].replace(B=1, H=3, Lk=2000, q_pos_offset=1872)),
    (WORKLOADS["t5_decode_evicted"], WORKLOADS["t5_decode_evicted"].replace(B=2, H=3, Lk=1500)),
    (WORKLOADS["deberta_k512"].replace(B=2, dtype="fp32"),
     WORKLOADS["deberta_k512"].replace(B=1, H=2, Lq=700, Lk=900, dtype="fp32")),
    (WORKLOADS["txl_memory"],
     WORKLOADS["txl_memory"].replace(B=1, H=2, Lq=300, Lk=800, q_pos_offset=500, clip_k=800)),
]


def _run(wl, noalloc, seed):
    inp = make_inputs(wl, seed)
    dev = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:3], dtype=torch.float32, device=DEV)
    kw = dict(kv_valid_len=dev["kv_valid_len"], out=out, lse=lse, **params_of(wl))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    if noalloc:
        ra.relattn_fwd_noalloc(dev["q"], dev["k"], dev["v"], wl.kind, dev["table"],
                               dev["table2"], **kw)
    else:
        ra.relattn_fwd(dev["q"], dev["k"], dev["v"], wl.kind, dev["table"], dev["table2"], **kw)
    torch.cuda.synchronize()
    if noalloc:
        assert torch.cuda.memory_allocated() == before
    return out, lse


@pytest.mark.parametrize("pair", PAIRS, ids=[p[0].name for p in PAIRS])
def test_noalloc_equals_workspace_entry_point(pair):
    for i, wl in enumerate(pair):
        p = ra.make_params(wl.kind, wl.dtype, wl.B, wl.H, wl.Lq, wl.Lk, wl.d,
                           table=torch.empty(16, device=DEV), table2=torch.empty(16, device=DEV),
                           **params_of(wl))
        assert 0 < ra.relattn_workspace_bytes(p) <= ra.binding.NOALLOC_SCRATCH_BYTES
        print(f"[noalloc] call {i}: {wl.name} B{wl.B} H{wl.H} Lq{wl.Lq} Lk{wl.Lk}", flush=True)
        want_o, want_l = _run(wl, False, seed=40 + i)
        got_o, got_l = _run(wl, True, seed=40 + i)
        assert torch.equal(got_o, want_o), f"{wl.name}: outputs differ"
        assert torch.equal(got_l, want_l), f"{wl.name}: row LSEs differ"
