"""CPU tests of the C ABI: the library loads, exports what include/attn.h
declares, and rejects bad arguments before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import exact_attention_02_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# status codes as declared in the header
STATUS = {}
with open(HEADER) as _f:
    for _m in re.finditer(r"^\s*(ATTN_[A-Z_]+)\s*=\s*(\d+)", _f.read(), re.M):
        STATUS[_m.group(1)] = int(_m.group(2))


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, re.M))


@pytest.fixture(scope="module")
def lib():
    return ea.load_library()


def test_header_declares_expected_functions():
    assert _declared_functions() == set(ea.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.attn_abi_version() == 8


def test_status_strings_distinct(lib):
    msgs = {ea.attn_status_string(v) for v in STATUS.values()}
    assert len(msgs) == len(STATUS)
    assert ea.attn_status_string(9999) == "unknown status"


# fake, never-dereferenced device addresses (16-byte aligned, disjoint)
MiB = 1 << 20
Q, K, V, O, L = (0x100000000 + i * 64 * MiB for i in range(5))


def call(lib, q=Q, k=K, v=V, o=O, l=L, B=1, H_q=4, H_kv=2, N=16, D=64, scale=0.125, causal=0):
    return lib.attn_fwd(q, k, v, o, l, B, H_q, H_kv, N, D, ctypes.c_float(scale), causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(N=-5), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(D=-64), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(H_kv=0), "ATTN_ERR_HEAD_RATIO"),
    (dict(H_q=6, H_kv=4), "ATTN_ERR_HEAD_RATIO"),
    (dict(H_q=2, H_kv=4), "ATTN_ERR_HEAD_RATIO"),
    (dict(D=96), "ATTN_ERR_HEAD_DIM"),
    (dict(D=256), "ATTN_ERR_HEAD_DIM"),
    (dict(causal=2), "ATTN_ERR_CAUSAL_FLAG"),
    (dict(causal=-1), "ATTN_ERR_CAUSAL_FLAG"),
    (dict(scale=float("nan")), "ATTN_ERR_SCALE"),
    (dict(scale=float("inf")), "ATTN_ERR_SCALE"),
    (dict(N=(1 << 24) + 1), "ATTN_ERR_SIZE_OVERFLOW"),
    (dict(N=(1 << 23) + 1, D=128), "ATTN_ERR_SIZE_OVERFLOW"),
    (dict(B=1 << 15, H_q=1 << 12, H_kv=1 << 12, N=1 << 4), "ATTN_ERR_SIZE_OVERFLOW"),
    (dict(q=0), "ATTN_ERR_NULL_POINTER"),
    (dict(l=0), "ATTN_ERR_NULL_POINTER"),
    (dict(k=K + 8), "ATTN_ERR_ALIGNMENT"),
    (dict(o=O + 2), "ATTN_ERR_ALIGNMENT"),
    (dict(l=L + 2), "ATTN_ERR_ALIGNMENT"),
    (dict(o=Q), "ATTN_ERR_ALIAS"),
    (dict(l=K + 64), "ATTN_ERR_ALIAS"),
    (dict(l=O + 16), "ATTN_ERR_ALIAS"),
])
def test_invalid_arguments_rejected(lib, kw, code):
    assert call(lib, **kw) == STATUS[code]


def test_checks_run_in_declared_order(lib):
    # negative size wins over a null pointer and a bad head ratio
    assert call(lib, q=0, B=-1, H_q=3, H_kv=2) == STATUS["ATTN_ERR_NEGATIVE_SIZE"]
    assert call(lib, q=0, D=80) == STATUS["ATTN_ERR_HEAD_DIM"]
    assert call(lib, q=0, k=K + 4) == STATUS["ATTN_ERR_NULL_POINTER"]


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(H_q=0, H_kv=1)])
def test_empty_work_is_success_without_pointers(lib, kw):
    assert call(lib, q=0, k=0, v=0, o=0, l=0, **kw) == STATUS["ATTN_OK"]


# ------------------------------------------------------------ split-KV entry
W = 0x100000000 + 5 * 64 * MiB   # fake workspace address


def call_split(lib, q=Q, k=K, v=V, o=O, l=L, B=1, H_q=4, H_kv=2, N_q=16, N_kv=40, D=64,
               scale=0.125, causal=0, n_splits=4, ws=W, ws_bytes=64 * MiB):
    return lib.attn_fwd_splitkv(q, k, v, o, l, B, H_q, H_kv, N_q, N_kv, D, ctypes.c_float(scale),
                                causal, n_splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N_q=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(N_kv=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(n_splits=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(H_q=6, H_kv=4), "ATTN_ERR_HEAD_RATIO"),
    (dict(D=32), "ATTN_ERR_HEAD_DIM"),
    (dict(causal=3), "ATTN_ERR_CAUSAL_FLAG"),
    (dict(scale=float("-inf")), "ATTN_ERR_SCALE"),
    (dict(n_splits=257), "ATTN_ERR_SPLITS"),
    (dict(causal=1, N_q=41, N_kv=40), "ATTN_ERR_CAUSAL_SHAPE"),
    (dict(N_kv=(1 << 24) + 1), "ATTN_ERR_SIZE_OVERFLOW"),
    (dict(N_q=(1 << 24), H_q=128, H_kv=1), "ATTN_ERR_SIZE_OVERFLOW"),
    # 2^20 one-wave decode workgroups times 256 forced splits: 2^34 work-items
    (dict(B=1 << 14, H_q=64, H_kv=64, N_q=1, N_kv=1, n_splits=256), "ATTN_ERR_SIZE_OVERFLOW"),
    # the same at 16 splits fits one dispatch; its workspace is what is short
    (dict(B=1 << 14, H_q=64, H_kv=64, N_q=1, N_kv=1, n_splits=16), "ATTN_ERR_WORKSPACE"),
    (dict(N_kv=0), "ATTN_ERR_NO_KEYS"),
    (dict(v=0), "ATTN_ERR_NULL_POINTER"),
    (dict(q=Q + 4), "ATTN_ERR_ALIGNMENT"),
    (dict(ws=0), "ATTN_ERR_WORKSPACE"),
    (dict(ws=W + 8), "ATTN_ERR_WORKSPACE"),
    (dict(ws_bytes=100), "ATTN_ERR_WORKSPACE"),
    (dict(ws=Q + 64 * MiB - 256), "ATTN_ERR_ALIAS"),
    (dict(ws=O - 1024, ws_bytes=64 * MiB), "ATTN_ERR_ALIAS"),
    (dict(l=V + 32), "ATTN_ERR_ALIAS"),
])
def test_splitkv_invalid_arguments_rejected(lib, kw, code):
    assert call_split(lib, **kw) == STATUS[code]


def test_splitkv_check_order(lib):
    assert call_split(lib, n_splits=300, D=80) == STATUS["ATTN_ERR_HEAD_DIM"]
    assert call_split(lib, n_splits=300, causal=1, N_q=50) == STATUS["ATTN_ERR_SPLITS"]
    assert call_split(lib, q=0, N_kv=0) == STATUS["ATTN_ERR_NO_KEYS"]
    assert call_split(lib, q=0, ws=0) == STATUS["ATTN_ERR_NULL_POINTER"]
    assert call_split(lib, ws=0, l=Q) == STATUS["ATTN_ERR_WORKSPACE"]


@pytest.mark.parametrize("kw", [dict(B=0), dict(N_q=0), dict(N_q=0, N_kv=0), dict(B=0, N_kv=0)])
def test_splitkv_empty_work_is_success_without_pointers(lib, kw):
    assert call_split(lib, q=0, k=0, v=0, o=0, l=0, ws=0, **kw) == STATUS["ATTN_OK"]


def test_splitkv_single_pass_needs_no_workspace(lib):
    # with one split there is no workspace: its absence is no error, and the
    # call only fails later, at a check of real arguments
    assert call_split(lib, n_splits=1, ws=0, ws_bytes=0, o=Q) == STATUS["ATTN_ERR_ALIAS"]


def test_workspace_size_formula():
    for (B, H_q, N_q, D, ns) in [(1, 32, 1, 128, 16), (2, 8, 100, 64, 3), (1, 1, 1, 64, 256)]:
        assert ea.attn_splitkv_workspace_size(B, H_q, N_q, D, ns) == ns * B * H_q * N_q * (2 * D + 4)
    assert ea.attn_splitkv_workspace_size(1, 32, 1, 128, 1) == 0
    assert ea.attn_splitkv_workspace_size(1, 32, 1, 128, 0) == 0
    assert ea.attn_splitkv_workspace_size(1, 32, 1, 128, 257) == 0
    assert ea.attn_splitkv_workspace_size(-1, 32, 1, 128, 4) == 0


def test_num_splits_choice():
    # the unsplit launch already fills the device: one pass
    assert ea.attn_splitkv_num_splits(1, 32, 8, 32768, 32768, 128, True) == 1
    # decode over a long cache: several splits, each with enough key tiles
    n = ea.attn_splitkv_num_splits(1, 32, 32, 1, 65536, 128, False)
    assert 2 <= n <= 256
    assert 65536 // 32 // n >= 8
    # too few keys to split
    assert ea.attn_splitkv_num_splits(1, 32, 32, 1, 100, 128, False) == 1
    # eight-wave shape (512 rows x 4 heads per kv head): one workgroup per CU, so
    # 64 workgroups take 4 splits on 256 CUs (this CPU run sees no device: 256 assumed)
    assert ea.attn_splitkv_num_splits(1, 32, 8, 512, 8192, 128, True) == 4
    assert ea.attn_splitkv_num_splits(1, 32, 32, 0, 100, 128, False) == 1
    assert ea.attn_splitkv_num_splits(1, 32, 32, 1, 100, 96, False) == -1
    assert ea.attn_splitkv_num_splits(1, 4, 4, 20, 10, 64, True) == -1


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.fwd(q, k, k)


def test_binding_rejects_wrong_dtype():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float32)
    with pytest.raises(TypeError):
        ea.fwd(q, q, q)


def test_product_path_does_not_import_oracle():
    """The binding and build modules never reference the oracle package."""
    pkg = os.path.join(ROOT, "exact_attention_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert "import oracle" not in txt and "from oracle" not in txt, fn


# ------------------------------------------------------------ backward entry
DO, DQ, DK, DV, WB = (0x200000000 + i * 64 * MiB for i in range(5))


def call_bwd(lib, q=Q, k=K, v=V, o=O, do=DO, l=L, dq=DQ, dk=DK, dv=DV, B=1, H_q=4, H_kv=2, N_q=16,
             N_kv=40, D=64, scale=0.125, causal=0, n_splits=1, ws=WB, ws_bytes=64 * MiB):
    return lib.attn_bwd(q, k, v, o, do, l, dq, dk, dv, B, H_q, H_kv, N_q, N_kv, D,
                        ctypes.c_float(scale), causal, n_splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(N_q=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(H_q=5, H_kv=2), "ATTN_ERR_HEAD_RATIO"),
    (dict(D=80), "ATTN_ERR_HEAD_DIM"),
    (dict(causal=5), "ATTN_ERR_CAUSAL_FLAG"),
    (dict(scale=float("nan")), "ATTN_ERR_SCALE"),
    (dict(n_splits=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(n_splits=65), "ATTN_ERR_SPLITS"),
    (dict(causal=1, N_q=41), "ATTN_ERR_CAUSAL_SHAPE"),
    (dict(N_kv=(1 << 23) + 1, D=128), "ATTN_ERR_SIZE_OVERFLOW"),
    (dict(N_q=1 << 20, H_q=16, H_kv=1, D=128, N_kv=1 << 20), "ATTN_ERR_SIZE_OVERFLOW"),
    # 2^29 query rows: the prep kernel's 8 threads per row pass one dispatch
    (dict(N_q=1 << 24, N_kv=1 << 24, H_q=32, H_kv=32, D=64), "ATTN_ERR_SIZE_OVERFLOW"),
    # 2^28 rows fit one dispatch; the workspace is what is short
    (dict(N_q=1 << 24, N_kv=1 << 24, H_q=16, H_kv=16, D=64), "ATTN_ERR_WORKSPACE"),
    (dict(N_kv=0), "ATTN_ERR_NO_KEYS"),
    (dict(do=0), "ATTN_ERR_NULL_POINTER"),
    (dict(dv=0), "ATTN_ERR_NULL_POINTER"),
    (dict(dq=DQ + 8), "ATTN_ERR_ALIGNMENT"),
    (dict(l=L + 1), "ATTN_ERR_ALIGNMENT"),
    (dict(ws=0), "ATTN_ERR_WORKSPACE"),
    (dict(ws_bytes=100), "ATTN_ERR_WORKSPACE"),
    (dict(ws=WB + 4), "ATTN_ERR_WORKSPACE"),
    (dict(n_splits=4, ws_bytes=4 * 2 * 2 * 40 * 64 * 4), "ATTN_ERR_WORKSPACE"),
    (dict(n_splits=4, ws=DO - 1024), "ATTN_ERR_ALIAS"),
    (dict(dq=Q), "ATTN_ERR_ALIAS"),
    (dict(dk=DV), "ATTN_ERR_ALIAS"),
    (dict(ws=DO + 16), "ATTN_ERR_ALIAS"),
    (dict(dv=L), "ATTN_ERR_ALIAS"),
])
def test_bwd_invalid_arguments_rejected(lib, kw, code):
    assert call_bwd(lib, **kw) == STATUS[code]


def test_bwd_check_order(lib):
    assert call_bwd(lib, D=80, q=0, causal=1, N_q=50) == STATUS["ATTN_ERR_HEAD_DIM"]
    assert call_bwd(lib, q=0, N_kv=0) == STATUS["ATTN_ERR_NO_KEYS"]
    assert call_bwd(lib, q=0, ws=0) == STATUS["ATTN_ERR_NULL_POINTER"]
    assert call_bwd(lib, ws=0, dq=Q) == STATUS["ATTN_ERR_WORKSPACE"]
    assert call_bwd(lib, n_splits=65, causal=1, N_q=41) == STATUS["ATTN_ERR_SPLITS"]
    assert call_bwd(lib, n_splits=65, scale=float("inf")) == STATUS["ATTN_ERR_SCALE"]
    # no query rows: nothing is split, so no workspace is needed whatever n_splits
    # says (the call gets past the workspace check to the alias check)
    assert call_bwd(lib, N_q=0, q=0, o=0, do=0, l=0, dq=0, ws=0, n_splits=8, dk=K) == STATUS["ATTN_ERR_ALIAS"]


@pytest.mark.parametrize("kw", [dict(B=0), dict(H_q=0, H_kv=1), dict(N_q=0, N_kv=0)])
def test_bwd_empty_work_is_success_without_pointers(lib, kw):
    assert call_bwd(lib, q=0, k=0, v=0, o=0, do=0, l=0, dq=0, dk=0, dv=0, ws=0, **kw) == STATUS["ATTN_OK"]


def test_bwd_no_query_rows_needs_only_key_buffers(lib):
    # N_q = 0 with keys: dK = dV = 0 are still written, so k, v, dk, dv are required
    assert call_bwd(lib, N_q=0, dk=0) == STATUS["ATTN_ERR_NULL_POINTER"]
    assert call_bwd(lib, N_q=0, q=0, o=0, do=0, l=0, dq=0, ws=0, dk=K) == STATUS["ATTN_ERR_ALIAS"]


def test_bwd_workspace_size():
    # large balanced grids: only the per-row statistics
    assert ea.attn_bwd_workspace_size(2, 32, 8, 1024, 1024, 128) == 2 * 32 * 1024 * 8
    assert ea.attn_bwd_workspace_size(2, 32, 8, 1024, 1024, 128, False, 1) == 2 * 32 * 1024 * 8
    assert ea.attn_bwd_workspace_size(1, 4, 4, 0, 10, 64) == 0
    assert ea.attn_bwd_workspace_size(-1, 4, 4, 4, 4, 64) == 0
    assert ea.attn_bwd_workspace_size(1, 4, 1, 4, 4, 64, False, 65) == 0
    assert ea.attn_bwd_workspace_size(1, 4, 4, 10, 5, 64, True) == 0    # causal with N_q > N_kv
    # statistics rounded up to 256 bytes, then fp32 dK and dV partials per range
    assert ea.attn_bwd_workspace_size(1, 3, 1, 5, 70, 64, False, 3) == 256 + 3 * 2 * 70 * 64 * 4
    # (the cases below assume 256 CUs: this CPU run sees no device)
    # one dQ workgroup over 128 key tiles: 32 dQ splits of fp32 partial dQ
    assert ea.attn_bwd_workspace_size(1, 4, 1, 64, 8192, 128, False, 1) == 2048 + 32 * 4 * 64 * 128 * 4
    # MQA N=512: 32 dK/dV ranges; two dQ ranges would save 4 tiles of the
    # heaviest workgroup, less than their partial sums and launch cost
    assert ea.attn_bwd_workspace_size(1, 16, 1, 512, 512, 128, False, 32) == 65536 + 32 * 2 * 512 * 128 * 4


def test_bwd_num_splits():
    # large grids are not split; one kv head over a short sequence is
    assert ea.attn_bwd_num_splits(1, 32, 8, 32768, 32768, 128, True) == 1
    assert ea.attn_bwd_num_splits(1, 16, 1, 512, 512, 128, True) > 1
    assert 1 <= ea.attn_bwd_num_splits(1, 16, 1, 512, 512, 128, False) <= 64
    assert ea.attn_bwd_num_splits(1, 4, 4, 0, 100, 64, True) == 1
    assert ea.attn_bwd_num_splits(0, 4, 4, 10, 100, 64, True) == 1
    assert ea.attn_bwd_num_splits(1, 5, 2, 10, 100, 64, True) == -1
    assert ea.attn_bwd_num_splits(1, 4, 4, 10, 5, 64, True) == -1
    # at most one range per row tile of the heaviest key block (4 heads x 1 tile)
    assert ea.attn_bwd_num_splits(1, 4, 1, 64, 64, 64, False) <= 4


# ------------------------------------------------------------ MLA entries
QL, KVC, OL, LL, WM = (0x300000000 + i * 64 * MiB for i in range(5))


def call_mla(lib, q=QL, kv=KVC, o=OL, l=LL, B=1, H=16, S=1, T=100, d_c=512, d_r=64, scale=0.07,
             causal=1, n_splits=4, ws=WM, ws_bytes=64 * MiB):
    return lib.attn_mla_decode(q, kv, o, l, B, H, S, T, d_c, d_r, ctypes.c_float(scale), causal,
                               n_splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(d_c=256), "ATTN_ERR_HEAD_DIM"),
    (dict(d_r=32), "ATTN_ERR_HEAD_DIM"),
    (dict(causal=2), "ATTN_ERR_CAUSAL_FLAG"),
    (dict(n_splits=300), "ATTN_ERR_SPLITS"),
    (dict(S=101), "ATTN_ERR_CAUSAL_SHAPE"),
    (dict(T=(1 << 21)), "ATTN_ERR_SIZE_OVERFLOW"),
    # 2^17 pair blocks times 128 splits: 2^24 workgroups of 256 work-items
    (dict(B=1 << 16, H=128, n_splits=128), "ATTN_ERR_SIZE_OVERFLOW"),
    (dict(B=1 << 16, H=128, n_splits=64), "ATTN_ERR_WORKSPACE"),
    (dict(scale=float("inf")), "ATTN_ERR_SCALE"),
    (dict(T=0, causal=0), "ATTN_ERR_NO_KEYS"),
    (dict(kv=0), "ATTN_ERR_NULL_POINTER"),
    (dict(o=OL + 8), "ATTN_ERR_ALIGNMENT"),
    (dict(ws=0), "ATTN_ERR_WORKSPACE"),
    (dict(ws_bytes=1000), "ATTN_ERR_WORKSPACE"),
    (dict(o=KVC + 1024), "ATTN_ERR_ALIAS"),
    (dict(ws=QL), "ATTN_ERR_ALIAS"),
])
def test_mla_invalid_arguments_rejected(lib, kw, code):
    assert call_mla(lib, **kw) == STATUS[code]


def test_mla_empty_and_sizes(lib):
    assert call_mla(lib, q=0, kv=0, o=0, l=0, ws=0, B=0) == STATUS["ATTN_OK"]
    assert call_mla(lib, q=0, kv=0, o=0, l=0, ws=0, S=0) == STATUS["ATTN_OK"]
    assert ea.attn_mla_workspace_size(2, 128, 1, 8) == 8 * 2 * 128 * (2 * 512 + 4)
    assert ea.attn_mla_workspace_size(2, 128, 1, 1) == 0
    assert ea.attn_mla_num_splits(1, 128, 1, 16384, True) >= 2
    assert ea.attn_mla_num_splits(256, 128, 1, 16384, True) == 1
    assert ea.attn_mla_num_splits(1, 128, 2, 1, True) == -1


def test_mla_projection_arguments_rejected(lib):
    ok = dict(B=1, H=4, S=1)
    assert lib.mla_absorb_q(QL, KVC, WM, OL, 1, 4, 1, 128, 256, 64, None) == STATUS["ATTN_ERR_HEAD_DIM"]
    assert lib.mla_absorb_q(QL, KVC, WM, OL, 1, 4, 1, 300, 512, 64, None) == STATUS["ATTN_ERR_HEAD_DIM"]
    assert lib.mla_absorb_q(QL, 0, WM, OL, 1, 4, 1, 128, 512, 64, None) == STATUS["ATTN_ERR_NULL_POINTER"]
    assert lib.mla_absorb_q(QL, KVC, WM, QL, 1, 4, 1, 128, 512, 64, None) == STATUS["ATTN_ERR_ALIAS"]
    assert lib.mla_absorb_q(0, 0, 0, 0, 0, 4, 1, 128, 512, 64, None) == STATUS["ATTN_OK"]
    assert lib.mla_up_project(QL, WM, OL, 1, 4, 1, 512, 100, None) == STATUS["ATTN_ERR_HEAD_DIM"]
    assert lib.mla_up_project(QL + 4, WM, OL, 1, 4, 1, 512, 128, None) == STATUS["ATTN_ERR_ALIGNMENT"]
    assert lib.mla_up_project(QL, WM, WM, 1, 4, 1, 512, 128, None) == STATUS["ATTN_ERR_ALIAS"]
    assert lib.mla_up_project(QL, WM, OL, -1, 4, 1, 512, 128, None) == STATUS["ATTN_ERR_NEGATIVE_SIZE"]
    # 2^26 rows with d_v = 1024: 2^26 one-wave blocks, 2^32 work-items, past a
    # dispatch's 32-bit work-item count
    assert lib.mla_up_project(QL, WM, OL, 1 << 17, 512, 1, 512, 1024, None) == STATUS["ATTN_ERR_SIZE_OVERFLOW"]
    # 2^25 blocks (d_v = 512) fit: the call gets past the size checks to the NULL output
    assert lib.mla_up_project(QL, WM, 0, 1 << 17, 512, 1, 512, 512, None) == STATUS["ATTN_ERR_NULL_POINTER"]
    assert ok


# ------------------------------------------------------------ static-scratch split entry
def call_static(lib, q=Q, k=K, v=V, o=O, l=L, B=1, H_q=4, H_kv=2, N_q=16, N_kv=40, D=64,
                scale=0.125, causal=0, n_splits=4):
    return lib.attn_fwd_splitkv_static(q, k, v, o, l, B, H_q, H_kv, N_q, N_kv, D, ctypes.c_float(scale),
                                       causal, n_splits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_splits=-1), "ATTN_ERR_NEGATIVE_SIZE"),
    (dict(H_q=6, H_kv=4), "ATTN_ERR_HEAD_RATIO"),
    (dict(scale=float("nan")), "ATTN_ERR_SCALE"),
    (dict(n_splits=257), "ATTN_ERR_SPLITS"),
    (dict(causal=1, N_q=41, N_kv=40), "ATTN_ERR_CAUSAL_SHAPE"),
    (dict(N_kv=0), "ATTN_ERR_NO_KEYS"),
    (dict(o=0), "ATTN_ERR_NULL_POINTER"),
    (dict(k=K + 2), "ATTN_ERR_ALIGNMENT"),
    # 256 splits of 320 rows at D=128: 21 MB of partials, above the 16 MiB scratch
    (dict(N_q=80, D=128, n_splits=256), "ATTN_ERR_STATIC_SCRATCH"),
    (dict(l=Q + 64), "ATTN_ERR_ALIAS"),
])
def test_static_invalid_arguments_rejected(lib, kw, code):
    assert call_static(lib, **kw) == STATUS[code]


def test_static_scratch_size_and_limit(lib):
    assert ea.attn_static_scratch_bytes() == 16 << 20
    # the largest request that fits is accepted up to the alias check
    # 320 rows at D=128: the limit falls below the 256-split maximum
    ns = 1
    while ns < 256 and ea.attn_splitkv_workspace_size(1, 4, 80, 128, ns + 1) <= ea.attn_static_scratch_bytes():
        ns += 1
    assert ns < 256
    assert call_static(lib, N_q=80, D=128, n_splits=ns, o=Q) == STATUS["ATTN_ERR_ALIAS"]
    assert call_static(lib, N_q=80, D=128, n_splits=ns + 1, o=Q) == STATUS["ATTN_ERR_STATIC_SCRATCH"]


@pytest.mark.parametrize("kw", [dict(B=0), dict(N_q=0)])
def test_static_empty_work_is_success_without_pointers(lib, kw):
    assert call_static(lib, q=0, k=0, v=0, o=0, l=0, **kw) == STATUS["ATTN_OK"]
