"""ctypes front end of the fp64 CPU oracle (``libmsa_oracle.so``).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py``; never by the product package.

Inputs are numpy arrays (or CPU torch tensors) holding the exact values the
GPU consumed: float64, float32, or bfloat16 carried as uint16 bit patterns.
The arithmetic follows the MiniMax Sparse Attention pages (paper summary page,
"Method"; zhichai.net write-up, sections 2 and 4.1); see ``msa_oracle.c``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F64 = 0, 1, 2


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
        ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("d_idx", ctypes.c_int32), ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("q_offset", ctypes.c_int64), ("softmax_scale", ctypes.c_double),
    ]


class Oracle:
    """One loaded copy of the oracle library (the tests also load mutants)."""

    def __init__(self, path):
        self.path = path
        self.L = load(path)

    def block_scores(self, prob, iq, ik, rows=None):
        """fp64 block scores [n_rows, h_kv, nblk]; -inf for non-candidate blocks."""
        iq, dt1 = _host(iq)
        ik, dt2 = _host(ik)
        assert dt1 == dt2
        r, n = _rows(prob, rows)
        out = np.empty((n, prob.h_kv, nblk(prob)), dtype=np.float64)
        rc = self.L.mo_block_scores(ctypes.byref(prob), _ptr(iq), _ptr(ik), dt1, _ptr(r), n, _ptr(out))
        if rc:
            raise ValueError(f"mo_block_scores: invalid argument ({rc})")
        return out

    def select(self, prob, scores, rows=None):
        """Selected block ids [n_rows, h_kv, topk] (int32, ascending, -1 padded)."""
        scores = np.ascontiguousarray(scores, dtype=np.float64)
        r, n = _rows(prob, rows)
        assert scores.shape == (n, prob.h_kv, nblk(prob))
        ids = np.empty((n, prob.h_kv, prob.topk), dtype=np.int32)
        rc = self.L.mo_select(ctypes.byref(prob), _ptr(scores), _ptr(r), n, _ptr(ids))
        if rc:
            raise ValueError(f"mo_select: invalid argument ({rc})")
        return ids

    def attend(self, prob, q, k, v, ids, rows=None):
        """fp64 attention output [n_rows, h_q, d] and LSE [n_rows, h_q]."""
        q, d1 = _host(q)
        k, d2 = _host(k)
        v, d3 = _host(v)
        assert d1 == d2 == d3
        r, n = _rows(prob, rows)
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        assert ids.shape == (n, prob.h_kv, prob.topk)
        out = np.empty((n, prob.h_q, prob.d), dtype=np.float64)
        lse = np.empty((n, prob.h_q), dtype=np.float64)
        rc = self.L.mo_attend(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), d1, _ptr(ids), _ptr(r), n,
                              _ptr(out), _ptr(lse))
        if rc:
            raise ValueError(f"mo_attend: invalid argument ({rc})")
        return out, lse

    def attend_backward(self, prob, q, k, v, dout, ids, rows=None):
        """fp64 (dq [n_rows, h_q, d], dk [B, Nk, h_kv, d], dv [B, Nk, h_kv, d]) of the
        attention step for upstream gradient dout and the fixed selection ids
        ([n_rows, h_kv, topk]); dk and dv sum the listed rows' contributions."""
        q, d1 = _host(q)
        k, d2 = _host(k)
        v, d3 = _host(v)
        dout, d4 = _host(dout)
        assert d1 == d2 == d3 == d4
        r, n = _rows(prob, rows)
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        assert ids.size == n * prob.h_kv * prob.topk
        dq = np.empty((n, prob.h_q, prob.d), dtype=np.float64)
        dk = np.empty((prob.batch, prob.n_k, prob.h_kv, prob.d), dtype=np.float64)
        dv = np.empty_like(dk)
        rc = self.L.mo_attend_backward(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), d1, _ptr(ids),
                                       _ptr(r), n, _ptr(dq), _ptr(dk), _ptr(dv))
        if rc:
            raise ValueError(f"mo_attend_backward: invalid argument ({rc})")
        if rows is None:
            dq = dq.reshape(prob.batch, prob.n_q, prob.h_q, prob.d)
        return dq, dk, dv

    def indexer_kl(self, prob, q, k, iq, ik, ids, rows=None, loss_scale=1.0):
        """fp64 (kl [n_rows, h_kv], d_iq [n_rows, h_kv, d_idx], d_ik [B, Nk, h_kv, d_idx]):
        the Index-Branch alignment loss per (row, group) and the gradients of
        loss_scale * sum(kl) with respect to the index queries and keys."""
        q, d1 = _host(q)
        k, d2 = _host(k)
        iq, d3 = _host(iq)
        ik, d4 = _host(ik)
        assert d1 == d2 == d3 == d4
        r, n = _rows(prob, rows)
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        assert ids.size == n * prob.h_kv * prob.topk
        kl = np.empty((n, prob.h_kv), dtype=np.float64)
        d_iq = np.empty((n, prob.h_kv, prob.d_idx), dtype=np.float64)
        d_ik = np.empty((prob.batch, prob.n_k, prob.h_kv, prob.d_idx), dtype=np.float64)
        rc = self.L.mo_indexer_kl(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(iq), _ptr(ik), d1, _ptr(ids), _ptr(r), n,
                                  float(loss_scale), _ptr(kl), _ptr(d_iq), _ptr(d_ik))
        if rc:
            raise ValueError(f"mo_indexer_kl: invalid argument ({rc})")
        return kl, d_iq, d_ik

    def forward(self, prob, q, k, v, iq, ik, rows=None):
        """Select then attend; returns (ids, out, lse, scores)."""
        s = self.block_scores(prob, iq, ik, rows)
        ids = self.select(prob, s, rows)
        out, lse = self.attend(prob, q, k, v, ids, rows)
        return ids, out, lse, s

    def num_threads(self):
        return self.L.mo_num_threads()

    def set_num_threads(self, n):
        self.L.mo_set_num_threads(int(n))

    # MXFP8 (OCP Microscaling Formats: 32-element blocks, E8M0 scale, E4M3 codes).
    def e4m3_value(self, code):
        return self.L.mo_e4m3_value(int(code) & 0xFF)

    def e4m3_encode(self, y):
        return self.L.mo_e4m3_encode(float(y))

    def mx_quantize(self, x):
        """(codes uint8 [..., n], scales uint8 [..., n/32]) of x (last axis a multiple of 32)."""
        x, dt = _host(x)
        n = x.shape[-1]
        assert n % 32 == 0
        rows = x.size // n
        codes = np.empty(x.shape, dtype=np.uint8)
        scales = np.empty(x.shape[:-1] + (n // 32,), dtype=np.uint8)
        rc = self.L.mo_mxfp8_quantize(_ptr(x), dt, rows, n, _ptr(codes), _ptr(scales))
        if rc:
            raise ValueError(f"mo_mxfp8_quantize: invalid argument ({rc})")
        return codes, scales

    def mx_dequantize(self, codes, scales):
        """fp64 values of an MXFP8 array (exact)."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        n = codes.shape[-1]
        assert scales.shape == codes.shape[:-1] + (n // 32,)
        out = np.empty(codes.shape, dtype=np.float64)
        rc = self.L.mo_mxfp8_dequantize(_ptr(codes), _ptr(scales), codes.size // n, n, _ptr(out))
        if rc:
            raise ValueError(f"mo_mxfp8_dequantize: invalid argument ({rc})")
        return out


_default = None


def default():
    """The oracle built from msa_oracle.c (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def block_scores(prob, iq, ik, rows=None):
    return default().block_scores(prob, iq, ik, rows)


def select(prob, scores, rows=None):
    return default().select(prob, scores, rows)


def attend(prob, q, k, v, ids, rows=None):
    return default().attend(prob, q, k, v, ids, rows)


def forward(prob, q, k, v, iq, ik, rows=None):
    return default().forward(prob, q, k, v, iq, ik, rows)


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)


def attend_backward(prob, q, k, v, dout, ids, rows=None):
    return default().attend_backward(prob, q, k, v, dout, ids, rows)


def indexer_kl(prob, q, k, iq, ik, ids, rows=None, loss_scale=1.0):
    return default().indexer_kl(prob, q, k, iq, ik, ids, rows, loss_scale)


def mx_quantize(x):
    return default().mx_quantize(x)


def mx_dequantize(codes, scales):
    return default().mx_dequantize(codes, scales)


def load(path):
    L = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp = ctypes.c_void_p
    L.mo_block_scores.argtypes = [P, vp, vp, ctypes.c_int, vp, ctypes.c_int64, vp]
    L.mo_select.argtypes = [P, vp, vp, ctypes.c_int64, vp]
    L.mo_attend.argtypes = [P, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int64, vp, vp]
    L.mo_invert.argtypes = [P, vp, vp, vp]
    L.mo_attend_backward.argtypes = [P, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int64, vp, vp, vp]
    L.mo_indexer_kl.argtypes = [P, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_double, vp, vp, vp]
    for f in (L.mo_block_scores, L.mo_select, L.mo_attend, L.mo_invert, L.mo_attend_backward, L.mo_indexer_kl):
        f.restype = ctypes.c_int
    L.mo_num_threads.restype = ctypes.c_int
    L.mo_set_num_threads.argtypes = [ctypes.c_int]
    L.mo_set_num_threads.restype = None
    L.mo_e4m3_value.argtypes = [ctypes.c_uint8]
    L.mo_e4m3_value.restype = ctypes.c_double
    L.mo_e4m3_encode.argtypes = [ctypes.c_double]
    L.mo_e4m3_encode.restype = ctypes.c_uint8
    L.mo_mxfp8_quantize.argtypes = [vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, vp, vp]
    L.mo_mxfp8_dequantize.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int32, vp]
    L.mo_mxfp8_quantize.restype = ctypes.c_int
    L.mo_mxfp8_dequantize.restype = ctypes.c_int
    return L


def make_problem(batch, n_q, n_k, h_q, h_kv, d, d_idx, block_size, topk, q_offset=0,
                 softmax_scale=0.0):
    return Problem(batch, n_q, n_k, h_q, h_kv, d, d_idx, block_size, topk, q_offset,
                   softmax_scale)


def problem_of(wl, **kw):
    """Problem for a workload description (any object with the usual fields)."""
    p = dict(batch=wl.batch, n_q=wl.n_q, n_k=wl.n_k, h_q=wl.h_q, h_kv=wl.h_kv, d=wl.d,
             d_idx=wl.d_idx, block_size=wl.block_size, topk=wl.topk, q_offset=wl.q_offset)
    p.update(kw)
    return make_problem(**p)


def nblk(prob):
    return (prob.n_k + prob.block_size - 1) // prob.block_size


def _host(x):
    """numpy view of x (CPU torch tensors are accepted; bf16 -> uint16 bits)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            assert x.device.type == "cpu", "oracle inputs must be host tensors"
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            return _host(x.numpy())
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"unsupported oracle input dtype {x.dtype}")


def _rows(prob, rows):
    if rows is None:
        return None, prob.batch * prob.n_q
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    return r, r.shape[0]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def invert(prob, ids, orc=None):
    """Block -> query lists: (offsets [B, h_kv, nblk+1], entries [B, h_kv, n_q*topk])."""
    orc = orc or default()
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32)).reshape(prob.batch, prob.n_q, prob.h_kv, prob.topk)
    offsets = np.empty((prob.batch, prob.h_kv, nblk(prob) + 1), dtype=np.int32)
    entries = np.full((prob.batch, prob.h_kv, prob.n_q * prob.topk), -1, dtype=np.int32)
    rc = orc.L.mo_invert(ctypes.byref(prob), _ptr(ids), _ptr(offsets), _ptr(entries))
    if rc:
        raise ValueError(f"mo_invert: invalid argument ({rc})")
    return offsets, entries
