"""The C-ABI library on a machine without a GPU: it loads, exports every
declared symbol, validates arguments before any HIP call, and its host-side
T5 thresholds reproduce the exact-integer bucket criterion."""

import ctypes
import os
import re

import numpy as np
import pytest

import transformer_attention_relative_amd as ra
from transformer_attention_relative_amd.binding import relattn_params
from tests.closed_forms import t5_bucket_exact

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relattn.h")


@pytest.fixture(scope="module")
def lib():
    return ra.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(relattn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_binding_exports():
    assert set(_declared_functions()) == set(ra.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.relattn_abi_version() == ra.binding.ABI_VERSION == 2


def _params(**kw):
    base = dict(kind="t5", dtype="bf16", B=1, H=2, Lq=64, Lk=64, d=64)
    base.update(kw)
    args = [base.pop(k) for k in ("kind", "dtype", "B", "H", "Lq", "Lk", "d")]
    return ra.make_params(*args, **base)


class _FakeTensor:
    """Stands in for a tensor when only the pointer value is marshalled."""
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


FAKE = _FakeTensor(0x10000)


def _fwd_status(lib, p):
    # q/k/v/out are NULL: even if validation of the params passed, the
    # pointer checks would stop the call before any launch.
    return lib.relattn_fwd(ctypes.byref(p), None, None, None, None, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kind="t5"), 1),                                   # table NULL
    (dict(kind="t5", table=FAKE, d=48), 2),                 # unsupported head dim
    (dict(kind="t5", dtype="fp32", table=FAKE, d=128), 2),  # 128 is built for bfloat16 only
    (dict(kind="t5", table=FAKE, d=0), 1),
    (dict(kind="t5", table=FAKE, B=0), 1),
    (dict(kind="t5", table=FAKE, Lk=0), 1),
    (dict(kind="t5", table=FAKE, num_buckets=2), 1),        # no exact slot per half
    (dict(kind="t5", table=FAKE, num_buckets=1, bidirectional=False), 1),
    (dict(kind="t5", table=FAKE, max_distance=8), 1),       # max_distance inside exact range
    (dict(kind="t5", table=FAKE, num_buckets=512), 1),
    (dict(kind="t5", table=FAKE, num_buckets=32, max_distance=100000), 2),  # LUT too large
    (dict(kind="t5", table=FAKE, q_pos_offset=-1), 1),
    (dict(kind="t5", table=FAKE, k_pos_offset=-1), 1),
    (dict(kind="t5", table=FAKE, k_pos_offset=(1 << 28) - 10), 2),   # key positions too large
    (dict(kind="t5", table=FAKE, scale=-1.0), 1),
    (dict(kind="t5", table=FAKE, scale=float("inf")), 1),
    (dict(kind="shaw", table=FAKE, clip_k=4), 1),           # table2 NULL
    (dict(kind="shaw", table=FAKE, table2=FAKE, clip_k=0), 1),
    (dict(kind="shaw", table=FAKE, table2=FAKE, clip_k=33), 2),
    (dict(kind="deberta", table=FAKE, table2=FAKE, clip_k=0), 1),
    (dict(kind="deberta", table=FAKE, table2=_FakeTensor(0x10004), clip_k=4), 1),  # misaligned
    (dict(kind="txl", table=FAKE, table2=FAKE, clip_k=64), 1),                     # not causal
    (dict(kind="txl", table=FAKE, table2=FAKE, clip_k=63, causal=True), 1),        # E too short
    (dict(kind="alibi", table=_FakeTensor(0x10002)), 1),                           # misaligned slopes
    (dict(kind="t5", table=FAKE, lse=_FakeTensor(0x10002)), 1),                    # misaligned lse
    (dict(kind="t5", table=FAKE), 1),                       # valid params, NULL tensors
])
def test_fwd_validation_rejects_before_launch(lib, kw, status):
    p = _params(**kw)
    assert _fwd_status(lib, p) == status
    assert lib.relattn_last_error().decode() != ""


# sizes past what the kernels index with 32-bit integers or build for: the
# status says unsupported and the message names the limit
@pytest.mark.parametrize("kw,reason", [
    (dict(kind="t5", table=FAKE, q_pos_offset=(1 << 28) - 10), "query positions above 2^28"),
    (dict(kind="t5", table=FAKE, k_pos_offset=(1 << 28) - 10), "key positions above 2^28"),
    (dict(kind="t5", table=FAKE, B=1 << 12, H=(1 << 12) + 1), "B*H too large"),
    (dict(kind="t5", table=FAKE, Lq=(1 << 26) + 1), "sequence length above 2^26"),
    (dict(kind="t5", table=FAKE, Lk=(1 << 26) + 1), "sequence length above 2^26"),
    (dict(kind="t5", table=FAKE, B=1 << 12, H=1 << 12, Lq=1 << 26), "grid too large"),
    (dict(kind="deberta", table=FAKE, table2=FAKE, clip_k=65537), "above 65536"),
])
def test_fwd_rejects_sizes_past_the_limits(lib, kw, reason):
    p = _params(**kw)
    assert _fwd_status(lib, p) == 2
    assert reason in lib.relattn_last_error().decode()


def test_fwd_rejects_bad_kind_and_dtype(lib):
    p = _params(table=FAKE)
    p.kind = 7
    assert _fwd_status(lib, p) == 1
    p = _params(table=FAKE)
    p.dtype = 5
    assert _fwd_status(lib, p) == 1
    assert lib.relattn_fwd(None, None, None, None, None, None, 0, None) == 1


def test_fwd_workspace_too_small(lib):
    # decode-like problem: few workgroups -> split-KV partials in the workspace
    p = _params(kind="t5", table=FAKE, B=1, H=2, Lq=128, Lk=8192, q_pos_offset=8064,
                causal=True, bidirectional=False)
    need = ra.relattn_workspace_bytes(p)
    assert need > 0
    st = lib.relattn_fwd(ctypes.byref(p), 0x10000, 0x10000, 0x10000, 0x10000, 0x10000,
                         need - 1, None)
    assert st == 3
    st = lib.relattn_fwd(ctypes.byref(p), 0x10000, 0x10000, 0x10000, 0x10000, None, need, None)
    assert st == 3


def test_workspace_sizes():
    p = _params(kind="t5", table=FAKE, B=8, H=12, Lq=512, Lk=512)
    assert ra.relattn_workspace_bytes(p) == 0          # enough workgroups, no split
    # DeBERTa in bfloat16 forms its per-key constants inside the forward
    # kernel; in float32 they come from the pre-pass, 8 bytes per (head, key)
    p = _params(kind="deberta", table=FAKE, table2=FAKE, clip_k=512, B=8, H=12,
                Lq=2048, Lk=2048)
    assert ra.relattn_workspace_bytes(p) == 0
    p = _params(kind="deberta", table=FAKE, table2=FAKE, clip_k=512, B=8, H=12,
                Lq=2048, Lk=2048, dtype="fp32")
    assert ra.relattn_workspace_bytes(p) == 96 * 2048 * 8   # per-key constants, no split
    # decode-like shape: few query tiles over a long key range -> split-KV partials
    p = _params(kind="t5", table=FAKE, B=4, H=16, Lq=128, Lk=4096, q_pos_offset=3968,
                causal=1, bidirectional=0)
    n = ra.relattn_workspace_bytes(p)
    assert n >= 2 * 64 * 128 * (64 + 2) * 4 and n % 256 == 0
    # a 128-row query tile aims at one workgroup per CU: 64 heads x 4 key
    # parts, each part holding (output, max, sum) per row in float32
    assert n == 4 * 64 * 128 * (64 + 2) * 4
    # ALiBi needs no per-key pass; Transformer-XL holds u.k_j per (head, key)
    # and v.E[r] per (head, encoding row), 8 bytes each, each region rounded
    # up to 256 bytes; a one-token decode step splits its key range
    p = _params(kind="alibi", table=FAKE, B=4, H=16, Lq=4096, Lk=4096, causal=1)
    assert ra.relattn_workspace_bytes(p) == 0
    p = _params(kind="txl", table=FAKE, table2=FAKE, clip_k=4096, B=4, H=16, Lq=2048,
                Lk=4096, q_pos_offset=2048, causal=1)
    assert ra.relattn_workspace_bytes(p) == 64 * 4096 * 8 + 16 * 4096 * 8
    p = _params(kind="txl", table=FAKE, table2=FAKE, clip_k=333, B=1, H=3, Lq=130,
                Lk=330, q_pos_offset=203, causal=1)
    assert ra.relattn_workspace_bytes(p) == (3 * 330 * 8 + 255) // 256 * 256 + (3 * 333 * 8 + 255) // 256 * 256
    p = _params(kind="alibi", table=FAKE, B=4, H=16, Lq=1, Lk=3072, q_pos_offset=4095,
                k_pos_offset=1024, causal=1)
    n = ra.relattn_workspace_bytes(p)
    assert n >= 2 * 64 * 1 * (64 + 2) * 4 and n % 256 == 0
    # a one-token step aims at two workgroups per CU: 8 key parts
    assert n == 8 * 64 * 1 * (64 + 2) * 4
    # 128-wide heads in bfloat16 (enough workgroups: no split)
    p = _params(kind="shaw", table=FAKE, table2=FAKE, clip_k=16, d=128, B=4, H=16, Lq=2048,
                Lk=2048, causal=1)
    assert ra.relattn_workspace_bytes(p) == 0
    p = _params(kind="deberta", table=FAKE, table2=FAKE, clip_k=64, d=128, B=4, H=16, Lq=2048,
                Lk=2048)
    assert ra.relattn_workspace_bytes(p) == 0


def test_rel_index_validation(lib):
    p = _params(kind="shaw", clip_k=0)
    assert lib.relattn_rel_index(ctypes.byref(p), None, None, 4, 0, None, None) == 1
    p = _params(kind="t5")
    assert lib.relattn_rel_index(ctypes.byref(p), None, None, 4, 1, None, None) == 1  # which=1 is DeBERTa only
    assert lib.relattn_rel_index(ctypes.byref(p), None, None, -1, 0, None, None) == 1
    assert lib.relattn_rel_index(ctypes.byref(p), None, None, 0, 0, None, None) == 0  # nothing to do
    assert lib.relattn_rel_index(ctypes.byref(p), None, None, 3, 0, None, None) == 1  # NULL buffers


@pytest.mark.parametrize("nb,md", [(8, 16), (16, 64), (32, 128), (32, 256), (64, 128),
                                   (64, 512), (128, 1024), (32, 4096), (30, 100), (256, 4096)])
@pytest.mark.parametrize("bidir", [True, False])
def test_host_thresholds_match_exact_criterion(nb, md, bidir):
    """Buckets rebuilt from the library's thresholds equal the exact-integer
    closed form for every offset in [-8192, 8192] (bit-exact integer work)."""
    thr = ra.relattn_t5_thresholds(nb, md, bidir)
    slots = nb // 2 if bidir else nb
    exact = slots // 2
    assert len(thr) == slots - exact and thr[0] == exact
    assert all(a <= b for a, b in zip(thr, thr[1:]))
    thr_arr = np.array(thr[1:], dtype=np.int64)
    for off in range(-8192, 8193, 1 if nb <= 64 else 7):
        if bidir:
            base, dist = (slots if off > 0 else 0), abs(off)
        else:
            base, dist = 0, max(-off, 0)
        got = base + (dist if dist < exact else exact + int((dist >= thr_arr).sum()))
        assert got == t5_bucket_exact(off, bidir, nb, md), (off, got)


def test_header_abi_version_matches_binding():
    src = open(HEADER).read()
    m = re.search(r"#define RELATTN_ABI_VERSION (\d+)", src)
    assert m and int(m.group(1)) == ra.binding.ABI_VERSION


# ----------------------------------------------------------------------------
# the Python binding checks every tensor before it calls the library (dtype,
# exact shape per kind as include/relattn.h states it, layout, then device);
# here the tensors live on the CPU, so the call must stop at a check
# ----------------------------------------------------------------------------

def _fwd_args(kind="deberta", dtype=None, B=2, H=3, Lq=5, Lk=7, d=32, k=4):
    import torch
    dt = torch.bfloat16 if dtype is None else dtype
    q = torch.zeros(B, H, Lq, d, dtype=dt)
    kk = torch.zeros(B, H, Lk, d, dtype=dt)
    v = torch.zeros(B, H, Lk, d, dtype=dt)
    tabs = {"t5": (torch.zeros(32, H), None), "alibi": (torch.zeros(H), None),
            "shaw": (torch.zeros(2 * k + 1, d, dtype=dt), torch.zeros(2 * k + 1, d, dtype=dt)),
            "deberta": (torch.zeros(2 * k, H, d, dtype=dt), torch.zeros(2 * k, H, d, dtype=dt)),
            "txl": (torch.zeros(k, H, d, dtype=dt), torch.zeros(2, H, d, dtype=dt))}[kind]
    return q, kk, v, tabs[0], tabs[1], dict(clip_k=k)


@pytest.mark.parametrize("kind", ["t5", "alibi", "shaw", "deberta", "txl"])
def test_binding_wellformed_cpu_tensors_stop_at_the_device_check(kind):
    q, k, v, t1, t2, kw = _fwd_args(kind)
    with pytest.raises(ValueError, match="GPU tensor"):
        ra.relattn_fwd(q, k, v, kind, t1, t2, **kw)


@pytest.mark.parametrize("case", [
    "k_dtype", "v_shape", "table_shape", "table_dtype", "table2_missing", "table2_extra",
    "table2_shape", "lens_dtype", "lens_short", "lse_shape", "lse_dtype", "out_shape",
    "out_dtype", "out_layout", "q_3d", "bad_kind", "t5_buckets"])
def test_binding_rejects_malformed_tensors(case):
    import torch
    kind = "t5" if case == "t5_buckets" else ("shaw" if case == "table2_extra" else "deberta")
    q, k, v, t1, t2, kw = _fwd_args(kind)
    extra = {}
    if case == "k_dtype":
        k = k.float()
    elif case == "v_shape":
        v = v[:, :, :-1].contiguous()
    elif case == "table_shape":
        t1 = t1[:-1].contiguous()            # 2k - 1 rows
    elif case == "table_dtype":
        t1 = t1.float()
    elif case == "table2_missing":
        t2 = None
    elif case == "table2_extra":
        kind = "alibi"
        t1, t2 = torch.zeros(q.shape[1]), t2
    elif case == "table2_shape":
        t2 = torch.zeros(2 * kw["clip_k"], q.shape[1] + 1, q.shape[3], dtype=q.dtype)
    elif case == "lens_dtype":
        extra["kv_valid_len"] = torch.zeros(q.shape[0], dtype=torch.int64)
    elif case == "lens_short":
        extra["kv_valid_len"] = torch.zeros(q.shape[0] - 1, dtype=torch.int32)
    elif case == "lse_shape":
        extra["lse"] = torch.zeros(q.shape[:3][::-1], dtype=torch.float32)
    elif case == "lse_dtype":
        extra["lse"] = torch.zeros(q.shape[:3], dtype=torch.bfloat16)
    elif case == "out_shape":
        extra["out"] = torch.zeros(q.shape[0], q.shape[1], q.shape[2] + 1, q.shape[3], dtype=q.dtype)
    elif case == "out_dtype":
        extra["out"] = torch.zeros(q.shape, dtype=torch.float32)
    elif case == "out_layout":
        extra["out"] = torch.zeros(q.shape[::-1], dtype=q.dtype).permute(3, 2, 1, 0)
    elif case == "q_3d":
        q = q[0]
    elif case == "bad_kind":
        kind = "rope"
    elif case == "t5_buckets":
        kw["num_buckets"] = 64                # table has 32 rows
    with pytest.raises((TypeError, ValueError)) as e:
        ra.relattn_fwd(q, k, v, kind, t1, t2, **kw, **extra)
    assert "GPU tensor" not in str(e.value)


def test_binding_rel_index_checks():
    import torch
    qp = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError, match="shape"):
        ra.relattn_rel_index("t5", qp, torch.zeros(7, dtype=torch.int32))
    with pytest.raises(TypeError):
        ra.relattn_rel_index("t5", qp, torch.zeros(8, dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU tensor"):
        ra.relattn_rel_index("t5", qp, qp.clone())


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    # float32 DeBERTa's per-key constants of 64 x 16 heads x 4096 keys take
    # 32 MiB, twice the fixed scratch: refused before any HIP call, with the
    # reason
    p = _params(kind="deberta", table=FAKE, table2=FAKE, clip_k=512, B=64, H=16, Lq=4096,
                Lk=4096, dtype="fp32")
    need = ra.relattn_workspace_bytes(p)
    assert need > ra.binding.NOALLOC_SCRATCH_BYTES
    st = lib.relattn_fwd_noalloc(ctypes.byref(p), 0x10000, 0x10000, 0x10000, 0x10000, None)
    assert st == 3
    msg = lib.relattn_last_error().decode()
    assert "scratch" in msg and str(need) in msg
    # and the usual argument checks come first
    assert lib.relattn_fwd_noalloc(ctypes.byref(p), None, None, None, None, None) == 1
    assert lib.relattn_fwd_noalloc(None, None, None, None, None, None) == 1


def test_noalloc_scratch_size_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define RELATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ra.binding.NOALLOC_SCRATCH_BYTES


def _supported_configs():
    """Every kind at the extremes of its supported parameters (head widths,
    dtypes, clip windows, T5 bucket geometry) and of the problem shapes that
    pick different kernel variants (decode-like, key-split, two query blocks
    per wave, many heads)."""
    shapes = [dict(B=1, H=2, Lq=1, Lk=4096, q_pos_offset=4095, causal=True),  # decode: split keys
              dict(B=4, H=16, Lq=128, Lk=4096, q_pos_offset=3968, causal=True),  # key-split halves
              dict(B=8, H=16, Lq=2048, Lk=2048),                                 # many workgroups
              dict(B=1, H=1, Lq=33, Lk=65)]                                      # ragged, tiny
    widths = [("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp32", 32), ("fp32", 64)]
    out = []
    for dtype, d in widths:
        for shp in shapes:
            for nb, md, bidir in [(2, 4, False), (32, 128, True), (64, 2048, True), (8, 8, True)]:
                out.append(dict(kind="t5", dtype=dtype, d=d, table=FAKE, num_buckets=nb,
                                max_distance=md, bidirectional=bidir and not shp.get("causal"), **shp))
            for k in (1, 16, 32):
                out.append(dict(kind="shaw", dtype=dtype, d=d, table=FAKE, table2=FAKE, clip_k=k, **shp))
            for k in (1, 63, 64, 512, 65536):
                out.append(dict(kind="deberta", dtype=dtype, d=d, table=FAKE, table2=FAKE, clip_k=k, **shp))
            out.append(dict(kind="alibi", dtype=dtype, d=d, table=FAKE, **shp))
            if shp.get("causal"):
                far = shp.get("q_pos_offset", 0) + shp["Lq"]
                out.append(dict(kind="txl", dtype=dtype, d=d, table=FAKE, table2=FAKE,
                                clip_k=far, **shp))
    return out


def test_every_supported_configuration_plans():
    # the host plan picks a built kernel variant whose LDS fits a CU (160 KiB)
    # for every kind at the extremes of its parameters; a layout change that
    # overflows LDS or a variant missing from the launch table shows up here
    # as RELATTN_ERR_UNSUPPORTED
    for kw in _supported_configs():
        try:
            ra.relattn_workspace_bytes(_params(**kw))
        except Exception as e:  # noqa: BLE001 - report the failing configuration
            raise AssertionError(f"{kw}: {e}") from e
