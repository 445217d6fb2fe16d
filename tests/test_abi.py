"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments before any HIP call (nothing launched)."""
import ctypes
import os
import re
import subprocess

import pytest

import attention_fa_fwd_07_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms


def test_library_holds_gfx950_code():
    blob = open(fa.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_abi_version_and_status_strings():
    lib = fa.load_library()
    assert lib.fa_abi_version() == 8
    names = [fa.status_str(c) for c in range(14)]
    assert names[0] == "FA_OK" and names[10] == "FA_ERR_HIP" and names[11] == "FA_ERR_WORKSPACE"
    assert names[12] == "FA_ERR_UNSUPPORTED_MASK" and names[13] == "FA_ERR_SCRATCH"
    assert len(set(names)) == 14
    assert fa.status_str(99) == "FA_ERR_UNKNOWN"


# fake but aligned, non-overlapping "device" addresses: never dereferenced,
# because every case below fails validation before any HIP call.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
DQ, DK, DV = 0x60000000, 0x60000100, 0x60000200


def call(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=64, Sk=64, D=128,
             layout=fa.FA_LAYOUT_BNSD, scale=0.125, causal=0, keep_prob=1.0,
             in_dtype=fa.FA_F16, o_dtype=fa.FA_F16, descale_q=None, descale_k=None,
             descale_v=None, stream=None)
    a.update(over)
    return fa.fa_fwd_raw(**a)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(k=None), fa.FA_ERR_NULL_POINTER),
    (dict(v=None), fa.FA_ERR_NULL_POINTER),
    (dict(o=None), fa.FA_ERR_NULL_POINTER),
    (dict(lse=None), fa.FA_ERR_NULL_POINTER),
    (dict(B=0), fa.FA_ERR_BAD_SHAPE),
    (dict(H=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(Sq=0), fa.FA_ERR_BAD_SHAPE),
    (dict(Sk=0), fa.FA_ERR_BAD_SHAPE),
    (dict(B=1 << 30, H=1 << 30), fa.FA_ERR_BAD_SHAPE),
    (dict(Sq=1 << 41), fa.FA_ERR_BAD_SHAPE),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(D=256), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(o_dtype=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED_DTYPE),
    (dict(in_dtype=fa.FA_BF16, o_dtype=fa.FA_F16), fa.FA_ERR_UNSUPPORTED_DTYPE),
    (dict(in_dtype=fa.FA_F32, o_dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED_DTYPE),
    (dict(in_dtype=fa.FA_FP8_E4M3, o_dtype=fa.FA_F16), fa.FA_ERR_NULL_POINTER),
    (dict(in_dtype=fa.FA_FP8_E4M3, o_dtype=fa.FA_BF16, descale_q=DQ, descale_k=DK,
          descale_v=DV), fa.FA_ERR_UNSUPPORTED_DTYPE),
    (dict(layout=2), fa.FA_ERR_UNSUPPORTED_LAYOUT),
    (dict(keep_prob=0.9), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(scale=float("inf")), fa.FA_ERR_BAD_SCALE),
    (dict(q=Q + 8), fa.FA_ERR_MISALIGNED),
    (dict(o=O + 2), fa.FA_ERR_MISALIGNED),
    (dict(lse=L + 2), fa.FA_ERR_MISALIGNED),
    (dict(o=Q + 64), fa.FA_ERR_ALIASING),
    (dict(o=V), fa.FA_ERR_ALIASING),
    (dict(lse=K + 1024), fa.FA_ERR_ALIASING),
    (dict(lse=O + 256), fa.FA_ERR_ALIASING),
])
def test_rejects_before_launch(over, code):
    assert call(**over) == code


def test_python_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x)


# ---- split-KV entry points ----
W = 0x70000000   # fake, 256-byte aligned workspace address


def call_split(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=64, Sk=1024, D=128,
             layout=fa.FA_LAYOUT_BNSD, scale=0.125, causal=0, keep_prob=1.0,
             in_dtype=fa.FA_F16, o_dtype=fa.FA_F16, descale_q=None, descale_k=None,
             descale_v=None, num_splits=4, workspace=W, workspace_size=1 << 24, stream=None)
    a.update(over)
    return fa.fa_fwd_splitkv_raw(**a)


def test_splitkv_workspace_size():
    # 4 ranges of B*H*Sq rows: O (D fp32) padded to 256 bytes, then lse (fp32)
    rows = 1 * 2 * 64
    o_bytes = 4 * rows * 128 * 4
    assert fa.splitkv_workspace_size(1, 2, 64, 1024, 128, False, 4) == o_bytes + 4 * rows * 4
    assert fa.splitkv_workspace_size(1, 2, 64, 1024, 128, False, 1) == 0
    # automatic count: a shape that fills the GPU needs no workspace
    assert fa.splitkv_workspace_size(4, 32, 4096, 4096, 128, False, 0) == 0
    # the automatic count splits only grids that leave most of the GPU idle,
    # with long key ranges
    assert fa.splitkv_workspace_size(1, 4, 8192, 8192, 128, False, 0) == \
        fa.splitkv_workspace_size(1, 4, 8192, 8192, 128, False, 3)
    assert fa.splitkv_workspace_size(1, 8, 512, 512, 64, False, 0) == 0
    assert fa.splitkv_workspace_size(1, 16, 4096, 4096, 128, True, 0) == 0
    for bad in (dict(D=96), dict(num_splits=-1), dict(num_splits=257), dict(B=0)):
        a = dict(B=1, H=2, Sq=64, Sk=1024, D=128, causal=False, num_splits=4)
        a.update(bad)
        assert fa.splitkv_workspace_size(**a) == -1


@pytest.mark.parametrize("over,code", [
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(num_splits=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(num_splits=257), fa.FA_ERR_BAD_SHAPE),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(workspace_size=1024), fa.FA_ERR_WORKSPACE),
    (dict(workspace=W + 16), fa.FA_ERR_MISALIGNED),
    (dict(workspace=Q), fa.FA_ERR_ALIASING),
    (dict(workspace=O - 256), fa.FA_ERR_ALIASING),
    (dict(keep_prob=0.5), fa.FA_ERR_UNSUPPORTED_DROPOUT),
])
def test_splitkv_rejects_before_launch(over, code):
    assert call_split(**over) == code


# ---- the split-KV entry point that allocates nothing ----
def call_noalloc(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=64, Sk=1024, D=128,
             layout=fa.FA_LAYOUT_BNSD, scale=0.125, causal=0, keep_prob=1.0,
             in_dtype=fa.FA_F16, o_dtype=fa.FA_F16, descale_q=None, descale_k=None,
             descale_v=None, num_splits=4, stream=None)
    a.update(over)
    return fa.fa_fwd_splitkv_noalloc_raw(**a)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(num_splits=-1), fa.FA_ERR_BAD_SHAPE),
    (dict(num_splits=257), fa.FA_ERR_BAD_SHAPE),
    (dict(keep_prob=0.5), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    # 64 ranges of 8 * 32 * 1024 rows of 129 floats: 541 MB, over the 64 MiB array
    (dict(B=8, H=32, Sq=1024, num_splits=64), fa.FA_ERR_SCRATCH),
    # just over: 2 ranges of B*H*Sq rows with (D + 1) floats each
    (dict(B=1, H=64, Sq=1017, D=128, num_splits=2), fa.FA_ERR_SCRATCH),
])
def test_noalloc_rejects_before_launch(over, code):
    assert call_noalloc(**over) == code


def test_noalloc_limit_is_the_workspace_size():
    """The largest accepted problem is the one whose split-KV workspace fits
    64 MiB (checked by size only: the largest that fits needs the array)."""
    assert fa.splitkv_workspace_size(1, 64, 1017, 1024, 128, False, 2) > 64 << 20
    assert fa.splitkv_workspace_size(1, 64, 1016, 1024, 128, False, 2) <= 64 << 20


# ---- the general entry point ----
def call_ex(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=8, H_kv=2, Sq=64, Sk=64, D=128,
             layout=fa.FA_LAYOUT_BNSD, scale=0.125, mask=fa.FA_MASK_CAUSAL_BOTTOM_RIGHT,
             keep_prob=1.0, in_dtype=fa.FA_F16, o_dtype=fa.FA_F16, descale_q=None,
             descale_k=None, descale_v=None, num_splits=1, workspace=None, workspace_size=0,
             stream=None)
    a.update(over)
    return fa.fa_fwd_ex_raw(**a)


@pytest.mark.parametrize("over,code", [
    (dict(H_kv=0), fa.FA_ERR_BAD_SHAPE),
    (dict(H_kv=3), fa.FA_ERR_BAD_SHAPE),
    (dict(H_kv=16), fa.FA_ERR_BAD_SHAPE),
    (dict(mask=3), fa.FA_ERR_UNSUPPORTED_MASK),
    (dict(mask=-1), fa.FA_ERR_UNSUPPORTED_MASK),
    (dict(num_splits=4), fa.FA_ERR_WORKSPACE),
    (dict(v=None), fa.FA_ERR_NULL_POINTER),
    # k of H_kv heads ends before o starts: o right after k is no alias,
    # o inside k's H_kv-head extent is
    (dict(o=K + 2 * 64 * 128 * 2 - 256), fa.FA_ERR_ALIASING),
])
def test_ex_rejects_before_launch(over, code):
    assert call_ex(**over) == code


def test_python_wrapper_rejects_unknown_mask():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa._mask_code("diagonal")


# ---- the variable-length entry point ----
CQ, CK = 0x7100000, 0x7200000   # fake offset arrays


def call_varlen(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, cu_q=CQ, cu_k=CK, B=3, H=4, H_kv=2, total_q=300,
             total_k=400, max_seqlen_q=200, D=128, scale=0.125, mask=fa.FA_MASK_NONE,
             keep_prob=1.0, in_dtype=fa.FA_F16, o_dtype=fa.FA_F16, descale_q=None,
             descale_k=None, descale_v=None, stream=None)
    a.update(over)
    return fa.fa_fwd_varlen_raw(**a)


@pytest.mark.parametrize("over,code", [
    (dict(cu_q=None), fa.FA_ERR_NULL_POINTER),
    (dict(cu_k=None), fa.FA_ERR_NULL_POINTER),
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(cu_q=CQ + 2), fa.FA_ERR_MISALIGNED),
    (dict(cu_k=CK + 1), fa.FA_ERR_MISALIGNED),
    (dict(B=0), fa.FA_ERR_BAD_SHAPE),
    (dict(max_seqlen_q=0), fa.FA_ERR_BAD_SHAPE),
    (dict(max_seqlen_q=301), fa.FA_ERR_BAD_SHAPE),
    (dict(total_q=0, max_seqlen_q=0), fa.FA_ERR_BAD_SHAPE),
    (dict(total_k=0), fa.FA_ERR_BAD_SHAPE),
    (dict(H_kv=3), fa.FA_ERR_BAD_SHAPE),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(mask=7), fa.FA_ERR_UNSUPPORTED_MASK),
    (dict(keep_prob=0.5), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    # o [total_q, H, D] overlapping k [total_k, H_kv, D]
    (dict(o=K + 256), fa.FA_ERR_ALIASING),
    # lse [H, total_q] fp32 right after o is fine, inside it is not
    (dict(lse=O + 1024), fa.FA_ERR_ALIASING),
])
def test_varlen_rejects_before_launch(over, code):
    assert call_varlen(**over) == code


def test_varlen_wrapper_checks_offsets():
    import torch
    x = torch.zeros(8, 2, 64, dtype=torch.float16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(x, x, x, cu, cu, 8)          # CPU tensors


# ---- the backward entry point ----
DO, GQ, GK, GV, WS = 0x80000000, 0x90000000, 0xA0000000, 0xB0000000, 0xC0000000


def call_bwd(**over):
    a = dict(q=Q, k=K, v=V, o=O, dout=DO, lse=L, dq=GQ, dk=GK, dv=GV, B=1, H=4, H_kv=2, Sq=100,
             Sk=300, D=128, scale=0.125, mask=fa.FA_MASK_CAUSAL_BOTTOM_RIGHT,
             in_dtype=fa.FA_F16, grad_dtype=fa.FA_F32, workspace=WS, workspace_size=1 << 20,
             stream=None)
    a.update(over)
    return fa.fa_bwd_raw(**a)


def test_bwd_workspace_size():
    # lse2 and Delta, fp32, per query row; rows rounded up to 32 per head
    assert fa.bwd_workspace_size(1, 4, 100) == 1 * 4 * 128 * 8
    assert fa.bwd_workspace_size(2, 3, 64) == 2 * 3 * 64 * 8
    for bad in ((0, 4, 100), (1, 0, 100), (1, 4, 0), (1 << 20, 1 << 10, 1 << 10)):
        assert fa.bwd_workspace_size(*bad) == -1


@pytest.mark.parametrize("over,code", [
    (dict(dout=None), fa.FA_ERR_NULL_POINTER),
    (dict(lse=None), fa.FA_ERR_NULL_POINTER),
    (dict(dv=None), fa.FA_ERR_NULL_POINTER),
    (dict(H_kv=3), fa.FA_ERR_BAD_SHAPE),
    (dict(Sk=0), fa.FA_ERR_BAD_SHAPE),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_UNSUPPORTED_DTYPE),
    (dict(in_dtype=fa.FA_BF16, grad_dtype=fa.FA_F16), fa.FA_ERR_UNSUPPORTED_DTYPE),
    (dict(mask=5), fa.FA_ERR_UNSUPPORTED_MASK),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(dq=GQ + 8), fa.FA_ERR_MISALIGNED),
    (dict(lse=L + 2), fa.FA_ERR_MISALIGNED),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(workspace_size=100), fa.FA_ERR_WORKSPACE),
    (dict(workspace=WS + 64), fa.FA_ERR_MISALIGNED),
    (dict(dq=Q + 256), fa.FA_ERR_ALIASING),
    (dict(dk=GQ + 1024), fa.FA_ERR_ALIASING),
    (dict(workspace=GV), fa.FA_ERR_ALIASING),
    (dict(dv=DO), fa.FA_ERR_ALIASING),
])
def test_bwd_rejects_before_launch(over, code):
    assert call_bwd(**over) == code


# ---- dropout ----
def call_drop(**over):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=4, H_kv=2, Sq=64, Sk=64, D=128,
             layout=fa.FA_LAYOUT_BNSD, scale=0.125, mask=fa.FA_MASK_NONE, keep_prob=0.9,
             seed=1, offset=0, in_dtype=fa.FA_F16, o_dtype=fa.FA_F16, descale_q=None,
             descale_k=None, descale_v=None, stream=None)
    a.update(over)
    return fa.fa_fwd_dropout_raw(**a)


@pytest.mark.parametrize("over,code", [
    (dict(keep_prob=0.0), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(keep_prob=-0.5), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(keep_prob=1.5), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(keep_prob=float("nan")), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(H_kv=3), fa.FA_ERR_BAD_SHAPE),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(mask=9), fa.FA_ERR_UNSUPPORTED_MASK),
    (dict(o=K), fa.FA_ERR_ALIASING),
])
def test_dropout_rejects_before_launch(over, code):
    assert call_drop(**over) == code


def test_dropout_needs_a_seed():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x, keep_prob=0.9)



def call_bwd_drop(**over):
    a = dict(q=Q, k=K, v=V, o=O, dout=DO, lse=L, dq=GQ, dk=GK, dv=GV, B=1, H=4, H_kv=2, Sq=100,
             Sk=300, D=128, scale=0.125, mask=fa.FA_MASK_NONE, keep_prob=0.8, seed=3, offset=1,
             in_dtype=fa.FA_BF16, grad_dtype=fa.FA_F32, workspace=WS, workspace_size=1 << 20,
             stream=None)
    a.update(over)
    return fa.fa_bwd_dropout_raw(**a)


@pytest.mark.parametrize("over,code", [
    (dict(keep_prob=0.0), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(keep_prob=2.0), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(keep_prob=float("nan")), fa.FA_ERR_UNSUPPORTED_DROPOUT),
    (dict(q=None), fa.FA_ERR_NULL_POINTER),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(dk=GQ), fa.FA_ERR_ALIASING),
])
def test_bwd_dropout_rejects_before_launch(over, code):
    assert call_bwd_drop(**over) == code
