"""CPU checks of the C ABI: the library loads, exports every entry point that
include/msa.h declares, and validates arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from block_sparse_long_bk_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(api.EXPORTS)


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    m = re.search(r"#define MSA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == api.NOALLOC_SCRATCH_BYTES


def test_library_exports_every_declared_symbol():
    L = api.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def good(**kw):
    p = dict(batch=1, n_q=1024, n_k=1024, h_q=8, h_kv=2, d=64, d_idx=32, topk=4, dtype="f32")
    p.update(kw)
    return api.problem(**p)


def test_status_strings():
    L = api.lib()
    for code in (0, -1, -2, -3, -4):
        assert L.msa_status_string(code)


@pytest.mark.parametrize("kw,status", [
    (dict(), api.MSA_OK),
    (dict(dtype="bf16", d=128, d_idx=128, h_q=64, h_kv=8, topk=16), api.MSA_OK),
    (dict(batch=0), api.MSA_ERR_INVALID_ARG),
    (dict(n_q=0), api.MSA_ERR_INVALID_ARG),
    (dict(h_q=6, h_kv=4), api.MSA_ERR_INVALID_ARG),
    (dict(n_q=2000), api.MSA_ERR_INVALID_ARG),            # n_q > n_k
    (dict(q_offset=1), api.MSA_ERR_INVALID_ARG),           # q_offset + n_q > n_k
    (dict(q_offset=-1, n_q=10), api.MSA_ERR_INVALID_ARG),
    (dict(topk=0), api.MSA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), api.MSA_ERR_INVALID_ARG),
    (dict(sched=7), api.MSA_ERR_INVALID_ARG),
    (dict(idx_format=2), api.MSA_ERR_INVALID_ARG),
    (dict(idx_format="mxfp8"), api.MSA_OK),
    (dict(idx_format="mxfp8", dtype="bf16", d=128, d_idx=32, h_q=64, h_kv=8, topk=16), api.MSA_OK),
    (dict(kv_format="mxfp8"), api.MSA_OK),
    (dict(kv_format=3), api.MSA_ERR_INVALID_ARG),
    (dict(block_size=64), api.MSA_OK),
    (dict(block_size=32), api.MSA_OK),
    (dict(block_size=96), api.MSA_ERR_UNSUPPORTED),
    (dict(block_size=256), api.MSA_ERR_UNSUPPORTED),
    (dict(block_size=32, n_k=1 << 20, n_q=1, q_offset=(1 << 20) - 1), api.MSA_ERR_UNSUPPORTED),  # 32768 blocks
    (dict(d=96), api.MSA_ERR_UNSUPPORTED),
    (dict(d_idx=48), api.MSA_ERR_UNSUPPORTED),
    (dict(topk=33), api.MSA_ERR_UNSUPPORTED),
    (dict(h_q=12, h_kv=2), api.MSA_ERR_UNSUPPORTED),      # 6 heads per group
    (dict(h_q=64, h_kv=1), api.MSA_ERR_UNSUPPORTED),      # 64 heads per group
])
def test_validate(kw, status):
    assert api.validate(good(**kw)) == status


def test_invalid_dtype_code():
    p = good()
    p.dtype = 5
    assert api.validate(p) == api.MSA_ERR_INVALID_ARG


def test_entry_points_reject_before_any_hip_call():
    L = api.lib()
    p = good()
    x = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    null = None
    assert L.msa_forward(ctypes.byref(p), null, x, x, x, x, x, x, null, null, 0, null) == api.MSA_ERR_INVALID_ARG
    assert L.msa_sparse_attention(ctypes.byref(p), x, x, x, x, null, null, null, 0, null) == api.MSA_ERR_INVALID_ARG
    mis = ctypes.c_void_p(4100)  # not 16-byte aligned
    assert L.msa_index_topk(ctypes.byref(p), mis, x, x, null, 0, null) == api.MSA_ERR_INVALID_ARG
    assert L.msa_block_scores(None, x, x, x, null) == api.MSA_ERR_INVALID_ARG
    bad = good(d=96)
    assert L.msa_forward(ctypes.byref(bad), x, x, x, x, x, x, x, null, null, 0, null) == api.MSA_ERR_UNSUPPORTED
    # attention with too little workspace
    big = good(dtype="bf16", n_q=32768, n_k=32768, h_q=64, h_kv=8, d=128, d_idx=128, topk=16, sched="kv_outer")
    assert L.msa_sparse_attention(ctypes.byref(big), x, x, x, x, x, null, x, 1024, null) == api.MSA_ERR_WORKSPACE
    assert L.msa_workspace_size(ctypes.byref(p), 9, ctypes.byref(ctypes.c_size_t()), None) == api.MSA_ERR_INVALID_ARG
    # backward: a missing gradient output, then too little workspace
    bw = L.msa_sparse_attention_backward
    assert bw(ctypes.byref(p), x, x, x, x, x, x, x, null, x, x, x, 1 << 30, null) == api.MSA_ERR_INVALID_ARG
    assert bw(ctypes.byref(p), x, x, x, x, x, x, x, x, x, x, x, 1024, null) == api.MSA_ERR_WORKSPACE
    assert bw(ctypes.byref(bad), x, x, x, x, x, x, x, x, x, x, x, 1 << 30, null) == api.MSA_ERR_UNSUPPORTED
    # indexer loss: plain index keys only, finite loss scale, workspace
    kl = L.msa_indexer_kl
    assert kl(ctypes.byref(p), x, x, x, x, x, x, 1.0, x, x, x, x, 1024, null) == api.MSA_ERR_WORKSPACE
    assert kl(ctypes.byref(p), x, x, x, x, x, x, float("inf"), x, x, x, x, 1 << 30, null) == api.MSA_ERR_INVALID_ARG
    assert kl(ctypes.byref(p), x, x, x, x, x, x, 1.0, x, null, x, x, 1 << 30, null) == api.MSA_ERR_INVALID_ARG
    mx = good(idx_format="mxfp8")
    assert kl(ctypes.byref(mx), x, x, x, x, x, x, 1.0, x, x, x, x, 1 << 30, null) == api.MSA_ERR_UNSUPPORTED
    # the training entry points need plain K and V
    kvmx = good(kv_format="mxfp8")
    assert kl(ctypes.byref(kvmx), x, x, x, x, x, x, 1.0, x, x, x, x, 1 << 30, null) == api.MSA_ERR_UNSUPPORTED
    assert bw(ctypes.byref(kvmx), x, x, x, x, x, x, x, x, x, x, x, 1 << 30, null) == api.MSA_ERR_UNSUPPORTED
    # MXFP8 quantiser: sizes, dtype and pointers are checked before any launch
    q = L.msa_mxfp8_quantize
    assert q(x, api.BF16, 4, 48, x, x, null) == api.MSA_ERR_INVALID_ARG   # row length not a multiple of 32
    assert q(x, 7, 4, 64, x, x, null) == api.MSA_ERR_INVALID_ARG         # unknown dtype
    assert q(null, api.F32, 4, 64, x, x, null) == api.MSA_ERR_INVALID_ARG
    assert q(x, api.F32, 4, 64, mis, x, null) == api.MSA_ERR_INVALID_ARG  # codes not 16-byte aligned
    assert q(x, api.F32, -1, 64, x, x, null) == api.MSA_ERR_INVALID_ARG
    assert q(x, api.F32, 0, 64, x, x, null) == api.MSA_OK                 # nothing to do
    # the forward on the library's own scratch: problems whose least workspace
    # exceeds the scratch are refused before the GPU is touched
    na = L.msa_forward_noalloc
    assert na(ctypes.byref(p), null, x, x, x, x, x, x, null, null) == api.MSA_ERR_INVALID_ARG
    assert na(ctypes.byref(bad), x, x, x, x, x, x, x, null, null) == api.MSA_ERR_UNSUPPORTED
    huge = good(dtype="bf16", batch=8, n_q=32768, n_k=32768, h_q=64, h_kv=8, d=128, d_idx=128, topk=32,
                block_size=32)
    _, least = api.workspace_size(huge, api.OP_FORWARD)
    assert least > api.NOALLOC_SCRATCH_BYTES
    assert na(ctypes.byref(huge), x, x, x, x, x, x, x, null, null) == api.MSA_ERR_WORKSPACE


def test_workspace_sizes():
    pre = good(dtype="bf16", n_q=32768, n_k=32768, h_q=64, h_kv=8, d=128, d_idx=128, topk=16)
    full, least = api.workspace_size(pre, api.OP_INDEX_TOPK)
    assert full == least == 0  # fused scoring + selection needs no scratch
    full, least = api.workspace_size(pre, api.OP_ATTENTION)
    # KV-outer partials: bf16 output + fp32 lse per (query, head, slot)
    assert full >= 32768 * 64 * 16 * (128 * 2 + 4)
    assert least < full / 64
    dec = good(dtype="bf16", batch=16, n_q=1, n_k=1 << 20, q_offset=(1 << 20) - 1, h_q=64, h_kv=8, d=128,
               d_idx=128, topk=16)
    full, least = api.workspace_size(dec, api.OP_INDEX_TOPK)
    assert full == 16 * 8 * 1 * 8192 * 4  # block scores of the decode scan
    fwd, _ = api.workspace_size(dec, api.OP_FORWARD)
    att, _ = api.workspace_size(dec, api.OP_ATTENTION)
    assert fwd == max(full, att)
    # the inversion alone is sized for the whole problem, whatever the schedule
    inv, inv_least = api.workspace_size(dec, api.OP_INVERT)
    assert inv == inv_least > 0
    inv_pre, _ = api.workspace_size(pre, api.OP_INVERT)
    assert inv_pre >= 8 * 256 * 4  # at least one count per (group, block)
    # backward: dq partials per (query, head, slot) in the input type dominate
    bwd, bwd_least = api.workspace_size(pre, api.OP_BACKWARD)
    assert bwd == bwd_least >= 32768 * 64 * 16 * 128 * 2
    # indexer loss: fp32 d_iq partials per (query, group, slot)
    klw, klw_least = api.workspace_size(pre, api.OP_INDEXER_KL)
    assert klw == klw_least >= 32768 * 8 * 16 * 128 * 2  # d idx_q partials in bf16
