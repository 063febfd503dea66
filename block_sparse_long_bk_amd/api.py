"""Python binding of libmsa (``include/msa.h``): argument marshalling only.

Every step of the MSA forward pass runs in the HIP kernels of ``libmsa.so``;
this module checks tensor shapes on the host, hands raw device pointers and
torch's current HIP stream to the C entry points, and raises on any non-zero
status.  There is no fallback: without the built library every call raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
SCHED_AUTO, SCHED_KV_OUTER, SCHED_Q_OUTER = 0, 1, 2
OP_INDEX_TOPK, OP_ATTENTION, OP_FORWARD, OP_INVERT, OP_BACKWARD, OP_INDEXER_KL = 0, 1, 2, 3, 4, 5
IDX_PLAIN, IDX_MXFP8 = 0, 1
NOALLOC_SCRATCH_BYTES = 256 << 20  # MSA_NOALLOC_SCRATCH_BYTES of msa.h
_IDXF = {"plain": IDX_PLAIN, "mxfp8": IDX_MXFP8}
_SCHED = {"auto": SCHED_AUTO, "kv_outer": SCHED_KV_OUTER, "q_outer": SCHED_Q_OUTER}


class Problem(ctypes.Structure):
    """Mirror of msa_problem_t."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
        ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("d_idx", ctypes.c_int32), ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("q_offset", ctypes.c_int64), ("softmax_scale", ctypes.c_float),
        ("sched", ctypes.c_int32), ("idx_format", ctypes.c_int32), ("kv_format", ctypes.c_int32),
    ]


class MSAError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = f"{what}: {_lib().msa_status_string(status).decode()} ({status})"
        if status == MSA_ERR_HIP:
            msg += f", hipError {_lib().msa_last_hip_error()}"
        super().__init__(msg)


_L = None

EXPORTS = ["msa_status_string", "msa_last_hip_error", "msa_validate", "msa_workspace_size", "msa_block_scores",
           "msa_topk_from_scores", "msa_index_topk", "msa_invert", "msa_sparse_attention", "msa_forward",
           "msa_forward_noalloc",
           "msa_sparse_attention_backward", "msa_indexer_kl", "msa_mxfp8_quantize", "msa_profile_enable", "msa_profile_reset",
           "msa_profile_count", "msa_profile_read"]


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_bk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, st = ctypes.c_void_p, ctypes.c_int
        L.msa_status_string.argtypes = [st]
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_last_hip_error.restype = ctypes.c_int
        L.msa_validate.argtypes = [P]
        L.msa_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]
        L.msa_block_scores.argtypes = [P, vp, vp, vp, vp]
        L.msa_topk_from_scores.argtypes = [P, vp, vp, vp]
        L.msa_index_topk.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_invert.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_sparse_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.msa_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.msa_sparse_attention_backward.argtypes = [P] + [vp] * 10 + [vp, ctypes.c_size_t, vp]
        L.msa_indexer_kl.argtypes = [P] + [vp] * 6 + [ctypes.c_float] + [vp] * 4 + [ctypes.c_size_t, vp]
        L.msa_mxfp8_quantize.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
        L.msa_profile_enable.argtypes = [ctypes.c_int]
        L.msa_profile_count.restype = ctypes.c_int
        L.msa_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        for name in EXPORTS:
            if name not in ("msa_status_string", "msa_last_hip_error", "msa_profile_count"):
                getattr(L, name).restype = ctypes.c_int
        _L = L
    return _L


def lib():
    """The loaded ctypes handle of libmsa.so."""
    return _lib()


def problem(batch, n_q, n_k, h_q, h_kv, d, d_idx, topk, dtype="bf16", q_offset=0, block_size=128,
            softmax_scale=0.0, sched="auto", idx_format="plain", kv_format="plain"):
    return Problem(batch, n_q, n_k, h_q, h_kv, d, d_idx, block_size, topk,
                   BF16 if dtype in ("bf16", torch.bfloat16) else F32, q_offset, softmax_scale,
                   _SCHED[sched] if isinstance(sched, str) else int(sched),
                   _IDXF[idx_format] if isinstance(idx_format, str) else int(idx_format),
                   _IDXF[kv_format] if isinstance(kv_format, str) else int(kv_format))


def problem_of(wl, sched="auto", **kw):
    """Problem for a workload description from ``inputs``."""
    p = dict(batch=wl.batch, n_q=wl.n_q, n_k=wl.n_k, h_q=wl.h_q, h_kv=wl.h_kv, d=wl.d, d_idx=wl.d_idx,
             topk=wl.topk, dtype=wl.dtype, q_offset=wl.q_offset, block_size=wl.block_size, sched=sched)
    p.update(kw)
    return problem(**p)


def nblk(p):
    return (p.n_k + p.block_size - 1) // p.block_size


def _check(rc, what):
    if rc != MSA_OK:
        raise MSAError(rc, what)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _expect(t, shape, dtype, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got "
                         f"{t.device} {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


def _tdtype(p):
    return torch.bfloat16 if p.dtype == BF16 else torch.float32


def _expect_ik(p, ik):
    """idx_k in the problem's dtype, or an MXFP8 cache (codes then scales, uint8)."""
    if p.idx_format == IDX_MXFP8:
        n = p.batch * p.n_k * p.h_kv * p.d_idx
        _expect(ik, (n + n // 32,), torch.uint8, "idx_k (MXFP8 codes + scales)")
    else:
        _expect(ik, (p.batch, p.n_k, p.h_kv, p.d_idx), _tdtype(p), "idx_k")


def _expect_kv(p, t, name):
    """K or V in the problem's dtype, or an MXFP8 cache (codes then scales, uint8)."""
    if p.kv_format == IDX_MXFP8:
        n = p.batch * p.n_k * p.h_kv * p.d
        _expect(t, (n + n // 32,), torch.uint8, f"{name} (MXFP8 codes + scales)")
    else:
        _expect(t, (p.batch, p.n_k, p.h_kv, p.d), _tdtype(p), name)


def _expect_plain_kv(p, what):
    if p.kv_format != IDX_PLAIN:
        raise ValueError(f"{what} needs plain K and V")


def mxfp8_quantize(x, out=None):
    """MXFP8 cache of x (cuda bf16/fp32, last axis a multiple of 32): one uint8
    tensor holding the E4M3 codes of every element followed by the E8M0 scale
    of every 32-element block -- the idx_k layout of an IDX_MXFP8 problem."""
    if x.dtype not in (torch.bfloat16, torch.float32) or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("mxfp8_quantize: expected a contiguous cuda bf16/fp32 tensor")
    n, row = x.numel(), x.shape[-1]
    if out is None:
        out = torch.empty(n + n // 32, dtype=torch.uint8, device=x.device)
    _expect(out, (n + n // 32,), torch.uint8, "out")
    base = out.data_ptr()
    _check(_lib().msa_mxfp8_quantize(_ptr(x), BF16 if x.dtype == torch.bfloat16 else F32, n // row, row,
                                     ctypes.c_void_p(base), ctypes.c_void_p(base + n), _stream()),
           "msa_mxfp8_quantize")
    return out


def validate(p):
    return _lib().msa_validate(ctypes.byref(p))


def workspace_size(p, op):
    """(bytes for a single pass, least bytes accepted)."""
    full, least = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib().msa_workspace_size(ctypes.byref(p), op, ctypes.byref(full), ctypes.byref(least)),
           "msa_workspace_size")
    return full.value, least.value


def alloc_workspace(p, op, device="cuda", minimal=False):
    full, least = workspace_size(p, op)
    n = least if minimal else full
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ws(ws):
    return (_ptr(ws), ws.numel()) if ws is not None else (None, 0)


def block_scores(p, iq, ik, scores=None):
    dt = _tdtype(p)
    _expect(iq, (p.batch, p.n_q, p.h_kv, p.d_idx), dt, "idx_q")
    _expect_ik(p, ik)
    if scores is None:
        scores = torch.empty((p.batch, p.h_kv, p.n_q, nblk(p)), dtype=torch.float32, device=iq.device)
    _check(_lib().msa_block_scores(ctypes.byref(p), _ptr(iq), _ptr(ik), _ptr(scores), _stream()), "msa_block_scores")
    return scores


def topk_from_scores(p, scores, ids=None):
    _expect(scores, (p.batch, p.h_kv, p.n_q, nblk(p)), torch.float32, "scores")
    if ids is None:
        ids = torch.empty((p.batch, p.n_q, p.h_kv, p.topk), dtype=torch.int32, device=scores.device)
    _check(_lib().msa_topk_from_scores(ctypes.byref(p), _ptr(scores), _ptr(ids), _stream()), "msa_topk_from_scores")
    return ids


def index_topk(p, iq, ik, ids=None, ws=None):
    dt = _tdtype(p)
    _expect(iq, (p.batch, p.n_q, p.h_kv, p.d_idx), dt, "idx_q")
    _expect_ik(p, ik)
    if ids is None:
        ids = torch.empty((p.batch, p.n_q, p.h_kv, p.topk), dtype=torch.int32, device=iq.device)
    if ws is None:
        ws = alloc_workspace(p, OP_INDEX_TOPK, iq.device)
    wp, wn = _ws(ws)
    _check(_lib().msa_index_topk(ctypes.byref(p), _ptr(iq), _ptr(ik), _ptr(ids), wp, wn, _stream()), "msa_index_topk")
    return ids


def invert(p, ids, ws=None):
    """(offsets [B, Hkv, nblk+1], entries [B, Hkv, Nq*topk]) of the block -> query lists."""
    _expect(ids, (p.batch, p.n_q, p.h_kv, p.topk), torch.int32, "block_ids")
    offsets = torch.empty((p.batch, p.h_kv, nblk(p) + 1), dtype=torch.int32, device=ids.device)
    entries = torch.empty((p.batch, p.h_kv, p.n_q * p.topk), dtype=torch.int32, device=ids.device)
    if ws is None:
        ws = alloc_workspace(p, OP_INVERT, ids.device)
    wp, wn = _ws(ws)
    _check(_lib().msa_invert(ctypes.byref(p), _ptr(ids), _ptr(offsets), _ptr(entries), wp, wn, _stream()),
           "msa_invert")
    return offsets, entries


def sparse_attention(p, q, k, v, ids, out=None, lse=None, want_lse=True, ws=None):
    dt = _tdtype(p)
    _expect(q, (p.batch, p.n_q, p.h_q, p.d), dt, "q")
    _expect_kv(p, k, "k")
    _expect_kv(p, v, "v")
    _expect(ids, (p.batch, p.n_q, p.h_kv, p.topk), torch.int32, "block_ids")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.n_q, p.h_q), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = alloc_workspace(p, OP_ATTENTION, q.device)
    wp, wn = _ws(ws)
    _check(_lib().msa_sparse_attention(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(ids), _ptr(out), _ptr(lse),
                                       wp, wn, _stream()), "msa_sparse_attention")
    return out, lse


def sparse_attention_backward(p, q, k, v, out, lse, dout, ids, dq=None, dk=None, dv=None, ws=None):
    """Gradients (dq, dk, dv) of the Main Branch for the fixed selection ids,
    given the forward's out and lse and the upstream gradient dout."""
    dt = _tdtype(p)
    _expect_plain_kv(p, "sparse_attention_backward")
    _expect(q, (p.batch, p.n_q, p.h_q, p.d), dt, "q")
    _expect(k, (p.batch, p.n_k, p.h_kv, p.d), dt, "k")
    _expect(v, (p.batch, p.n_k, p.h_kv, p.d), dt, "v")
    _expect(out, (p.batch, p.n_q, p.h_q, p.d), dt, "out")
    _expect(dout, (p.batch, p.n_q, p.h_q, p.d), dt, "dout")
    _expect(lse, (p.batch, p.n_q, p.h_q), torch.float32, "lse")
    _expect(ids, (p.batch, p.n_q, p.h_kv, p.topk), torch.int32, "block_ids")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _expect(dq, tuple(q.shape), dt, "dq")
    _expect(dk, tuple(k.shape), dt, "dk")
    _expect(dv, tuple(v.shape), dt, "dv")
    if ws is None:
        ws = alloc_workspace(p, OP_BACKWARD, q.device)
    wp, wn = _ws(ws)
    _check(_lib().msa_sparse_attention_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                _ptr(dout), _ptr(ids), _ptr(dq), _ptr(dk), _ptr(dv), wp, wn,
                                                _stream()), "msa_sparse_attention_backward")
    return dq, dk, dv


def indexer_kl(p, q, k, iq, ik, lse, ids, loss_scale=1.0, kl=None, d_iq=None, d_ik=None, ws=None):
    """Index-Branch alignment loss: kl [B, Nq, Hkv] (fp32) and the gradients
    (d_iq, d_ik) of loss_scale * sum(kl) for the index queries and keys, given
    the Main Branch inputs, the forward's lse and the selection."""
    dt = _tdtype(p)
    if p.idx_format != IDX_PLAIN:
        raise ValueError("indexer_kl needs plain index keys")
    _expect_plain_kv(p, "indexer_kl")
    _expect(q, (p.batch, p.n_q, p.h_q, p.d), dt, "q")
    _expect(k, (p.batch, p.n_k, p.h_kv, p.d), dt, "k")
    _expect(iq, (p.batch, p.n_q, p.h_kv, p.d_idx), dt, "idx_q")
    _expect(ik, (p.batch, p.n_k, p.h_kv, p.d_idx), dt, "idx_k")
    _expect(lse, (p.batch, p.n_q, p.h_q), torch.float32, "lse")
    _expect(ids, (p.batch, p.n_q, p.h_kv, p.topk), torch.int32, "block_ids")
    kl = torch.empty((p.batch, p.n_q, p.h_kv), dtype=torch.float32, device=q.device) if kl is None else kl
    d_iq = torch.empty_like(iq) if d_iq is None else d_iq
    d_ik = torch.empty_like(ik) if d_ik is None else d_ik
    _expect(kl, (p.batch, p.n_q, p.h_kv), torch.float32, "kl")
    _expect(d_iq, tuple(iq.shape), dt, "d_iq")
    _expect(d_ik, tuple(ik.shape), dt, "d_ik")
    if ws is None:
        ws = alloc_workspace(p, OP_INDEXER_KL, q.device)
    wp, wn = _ws(ws)
    _check(_lib().msa_indexer_kl(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(iq), _ptr(ik), _ptr(lse), _ptr(ids),
                                 float(loss_scale), _ptr(kl), _ptr(d_iq), _ptr(d_ik), wp, wn, _stream()),
           "msa_indexer_kl")
    return kl, d_iq, d_ik


def forward(p, q, k, v, iq, ik, ids=None, out=None, lse=None, want_lse=True, ws=None):
    dt = _tdtype(p)
    _expect(q, (p.batch, p.n_q, p.h_q, p.d), dt, "q")
    _expect_kv(p, k, "k")
    _expect_kv(p, v, "v")
    _expect(iq, (p.batch, p.n_q, p.h_kv, p.d_idx), dt, "idx_q")
    _expect_ik(p, ik)
    if ids is None:
        ids = torch.empty((p.batch, p.n_q, p.h_kv, p.topk), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.n_q, p.h_q), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = alloc_workspace(p, OP_FORWARD, q.device)
    wp, wn = _ws(ws)
    _check(_lib().msa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(iq), _ptr(ik), _ptr(ids), _ptr(out),
                              _ptr(lse), wp, wn, _stream()), "msa_forward")
    return ids, out, lse


def forward_noalloc(p, q, k, v, iq, ik, ids=None, out=None, lse=None, want_lse=True):
    """msa_forward on the library's own per-GPU scratch (no workspace argument)."""
    dt = _tdtype(p)
    _expect(q, (p.batch, p.n_q, p.h_q, p.d), dt, "q")
    _expect_kv(p, k, "k")
    _expect_kv(p, v, "v")
    _expect(iq, (p.batch, p.n_q, p.h_kv, p.d_idx), dt, "idx_q")
    _expect_ik(p, ik)
    if ids is None:
        ids = torch.empty((p.batch, p.n_q, p.h_kv, p.topk), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.n_q, p.h_q), dtype=torch.float32, device=q.device)
    _check(_lib().msa_forward_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(iq), _ptr(ik), _ptr(ids),
                                      _ptr(out), _ptr(lse), _stream()), "msa_forward_noalloc")
    return ids, out, lse


def profile_enable(on=True):
    _check(_lib().msa_profile_enable(1 if on else 0), "msa_profile_enable")


def profile_reset():
    _check(_lib().msa_profile_reset(), "msa_profile_reset")


def profile_read():
    """{kernel name: (total ms, launches)} since the last reset."""
    L = _lib()
    res = {}
    for i in range(L.msa_profile_count()):
        name, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
        _check(L.msa_profile_read(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)), "msa_profile_read")
        res[name.value.decode()] = (ms.value, n.value)
    return res
