"""GPU parity of the MXFP8 index-key path (OCP MX: E8M0 block scales, E4M3
codes) against the oracle.

* The quantiser kernel must reproduce the oracle's codes and scales bit for
  bit (bf16 and fp32 sources; zero, saturating, tiny, huge and mixed blocks).
* Index selection over an MXFP8 cache: the cache is built by the *oracle's*
  quantiser from the workload's idx_k, and the oracle selects from the
  exactly dequantised keys in fp64; the GPU must match row by row within the
  tie band (both index kernels: the MFMA tile for prefill, the scan for
  decode), block scores within 1e-5 of the largest, and the forward pass must
  give the same attention as the oracle on that selection.
* Attention over MXFP8 K and V caches (both schedules, Bk 32/64/128): the
  caches are built by the oracle's quantiser and the oracle attends over the
  exactly dequantised keys and values; the GPU decodes them while staging a
  block, so the usual attention tolerance applies.  A forward over an
  all-MXFP8 cache (index keys too) must select as the MX index path does and
  attend exactly as the attention call on that selection.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs
from oracle import oracle as O

from tests.parity import assert_attention, check_selection, host, to_f64

pytestmark = pytest.mark.gpu


def _blocks(rng, n_rows, row_len):
    """Rows whose 32-element blocks span many magnitudes, plus edge blocks."""
    x = rng.standard_normal((n_rows, row_len)) * np.exp2(rng.integers(-20, 20, (n_rows, row_len // 32)))\
        .repeat(32, axis=1)
    x[0, :32] = 0.0                    # all-zero block
    x[0, 32:64] = -0.0
    x[1, :32] = 1.9                    # the block maximum saturates (1.9 * 256 > 448)
    x[1, 32:64] = np.linspace(-448, 448, 32) * 2.0 ** -5
    x[2, :32] = 3e38                   # near the fp32 maximum
    x[2, 32:64] = 2.0 ** -140          # fp32 subnormals
    x[3, :32] = rng.uniform(-1, 1, 32) * 2.0 ** -120
    return x


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_bit_exact(src):
    rng = np.random.default_rng(21)
    x = _blocks(rng, 257, 128).astype(np.float32)
    if src == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        x_host = xt
    else:
        xt = torch.from_numpy(x)
        x_host = x
    cache = api.mxfp8_quantize(xt.cuda())
    torch.cuda.synchronize()
    cache = host(cache).numpy()
    codes_o, scales_o = O.mx_quantize(x_host)
    n = x.size
    assert np.array_equal(cache[:n].reshape(x.shape), codes_o)
    assert np.array_equal(cache[n:].reshape(scales_o.shape), scales_o)


MX_CASES = {
    # prefill shapes: MFMA tile path
    "mx_bf16_prefill": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=6),
    "mx_f32_prefill": dict(n_q=600, n_k=600, h_q=8, h_kv=2, d=64, d_idx=32, topk=4),
    "mx_bf16_di64_offset": dict(dtype="bf16", n_q=300, n_k=2000, q_offset=1700, h_q=8, h_kv=2, d=64, d_idx=64,
                                topk=5),
    # decode shapes: streaming scan
    "mx_bf16_decode": dict(dtype="bf16", batch=3, n_q=1, n_k=5000, q_offset=4999, h_q=16, h_kv=2, d=128,
                           d_idx=128, topk=8),
    "mx_f32_few_queries": dict(n_q=5, n_k=3000, q_offset=2995, d_idx=64, topk=4),
    "mx_bf16_bk64": dict(dtype="bf16", n_q=700, n_k=700, h_q=8, h_kv=2, d=64, d_idx=128, topk=8, block_size=64),
    "mx_bf16_bk32_decode": dict(dtype="bf16", batch=2, n_q=1, n_k=3001, q_offset=3000, h_q=8, h_kv=2, d=64,
                                d_idx=64, topk=8, block_size=32),
    "mx_bf16_long_decode": dict(dtype="bf16", batch=2, n_q=1, n_k=2100 * 128 + 77, q_offset=2100 * 128 + 76,
                                h_q=8, h_kv=2, d=64, d_idx=32, topk=16),
}


def _mx_case(name):
    wl = inputs.small(name, seed=3000 + sorted(MX_CASES).index(name), **MX_CASES[name])
    x = inputs.generate(wl, device="cuda")
    ik_host = host(x["ik"])
    codes, scales = O.mx_quantize(ik_host)                   # the oracle builds the cache
    cache = torch.from_numpy(np.concatenate([codes.reshape(-1), scales.reshape(-1)])).cuda()
    ik64 = O.mx_dequantize(codes, scales)                    # exact key values
    iq64 = to_f64(x["iq"]).reshape(wl.batch, wl.n_q, wl.h_kv, wl.d_idx)
    return wl, x, cache, iq64, ik64


@pytest.mark.parametrize("name", sorted(MX_CASES))
def test_index_over_mxfp8_cache(name):
    wl, x, cache, iq64, ik64 = _mx_case(name)
    p = api.problem_of(wl, idx_format="mxfp8")
    prob = O.problem_of(wl)
    s_o = O.block_scores(prob, np.ascontiguousarray(iq64), np.ascontiguousarray(ik64))
    ids_o = O.select(prob, s_o)
    ids = api.index_topk(p, x["iq"], cache)
    S = api.block_scores(p, x["iq"], cache)
    torch.cuda.synchronize()
    got = host(ids).numpy().reshape(wl.batch * wl.n_q, wl.h_kv, wl.topk)
    res = check_selection(wl, got, ids_o, s_o)
    assert res["fail"] == 0, res
    S = host(S).numpy().astype(np.float64).transpose(0, 2, 1, 3).reshape(wl.batch * wl.n_q, wl.h_kv, -1)
    cand = np.isfinite(s_o)
    assert np.array_equal(np.isfinite(S), cand)
    if cand.any():
        scale = max(np.max(np.abs(s_o[cand])), 1.0)
        assert np.max(np.abs(S[cand] - s_o[cand])) <= 1e-5 * scale
    # the forward pass composes the MX index with the attention of the selection
    ids_f, out, lse = api.forward(p, x["q"], x["k"], x["v"], x["iq"], cache)
    torch.cuda.synchronize()
    assert torch.equal(ids_f, ids)
    ids_fixed = torch.from_numpy(ids_o.reshape(wl.batch, wl.n_q, wl.h_kv, wl.topk)).cuda()
    o2, l2 = api.sparse_attention(api.problem_of(wl), x["q"], x["k"], x["v"], ids_fixed)
    torch.cuda.synchronize()
    o_o, l_o = O.attend(prob, host(x["q"]), host(x["k"]), host(x["v"]), ids_o)
    assert_attention(wl.dtype, to_f64(o2).reshape(o_o.shape), o_o, host(l2).numpy().reshape(l_o.shape), l_o,
                     what=f"{name}/attention")
    print(f"{name}: selection {res}")


def _dequant_f32(codes, scales, chunk=1 << 16):
    """Exact key values (fp32 holds every MXFP8 value of a quantised finite
    cache) without a full fp64 copy of a 1M-token cache."""
    out = np.empty(codes.shape, dtype=np.float32)
    for t0 in range(0, codes.shape[1], chunk):
        out[:, t0:t0 + chunk] = O.mx_dequantize(codes[:, t0:t0 + chunk], scales[:, t0:t0 + chunk])
    return out


def test_decode_16x1m_over_mxfp8_cache():
    """Full-size decode rows (1M-token cache, 8191 candidate blocks) over an
    MXFP8 cache built by the oracle, for the first and last sequence."""
    wl = inputs.WORKLOADS["decode_16x1m"]
    x = inputs.generate(wl, device="cuda", tensors=("iq", "ik"))
    sub = wl.with_(batch=1)
    prob = O.problem_of(sub)
    for b in (0, wl.batch - 1):
        codes, scales = O.mx_quantize(host(x["ik"][b:b + 1]))
        cache = torch.from_numpy(np.concatenate([codes.reshape(-1), scales.reshape(-1)])).cuda()
        iq = x["iq"][b:b + 1].contiguous()
        ids = api.index_topk(api.problem_of(sub, idx_format="mxfp8"), iq, cache)
        torch.cuda.synchronize()
        s_o = O.block_scores(prob, host(iq).float().numpy(), _dequant_f32(codes, scales))
        ids_o = O.select(prob, s_o)
        res = check_selection(sub, host(ids).numpy().reshape(1, wl.h_kv, wl.topk), ids_o, s_o)
        print(f"decode_16x1m/mxfp8 b={b}: {res}", flush=True)
        assert res["fail"] == 0, res
        del cache


# ---- MXFP8 K / V caches: attention over the exactly decoded keys and values.
KV_CASES = {
    "kv_bf16_kvouter": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=6,
                            sched="kv_outer"),
    "kv_f32_kvouter": dict(n_q=600, n_k=600, h_q=8, h_kv=2, d=64, d_idx=32, topk=4, sched="kv_outer"),
    "kv_f32_d128_kvouter": dict(n_q=700, n_k=700, h_q=8, h_kv=2, d=128, d_idx=64, topk=5, sched="kv_outer"),
    "kv_bf16_qouter": dict(dtype="bf16", n_q=300, n_k=2000, q_offset=1700, h_q=8, h_kv=2, d=64, d_idx=64,
                           topk=5, sched="q_outer"),
    "kv_bf16_decode": dict(dtype="bf16", batch=3, n_q=1, n_k=5000, q_offset=4999, h_q=16, h_kv=2, d=128,
                           d_idx=128, topk=8, sched="auto"),
    "kv_bf16_bk64": dict(dtype="bf16", n_q=700, n_k=700, h_q=8, h_kv=2, d=64, d_idx=128, topk=8, block_size=64,
                         sched="kv_outer"),
    "kv_f32_bk32_qouter": dict(n_q=5, n_k=3000, q_offset=2995, topk=4, block_size=32, sched="q_outer"),
}


@pytest.mark.parametrize("name", sorted(KV_CASES))
def test_attention_over_mxfp8_kv_cache(name):
    kw = dict(KV_CASES[name])
    sched = kw.pop("sched")
    wl = inputs.small(name, seed=3500 + sorted(KV_CASES).index(name), **kw)
    x = inputs.generate(wl, device="cuda")
    prob = O.problem_of(wl)
    # the oracle builds both caches and decodes them exactly
    kv = {}
    for t in ("k", "v"):
        codes, scales = O.mx_quantize(host(x[t]))
        kv[t] = (torch.from_numpy(np.concatenate([codes.reshape(-1), scales.reshape(-1)])).cuda(),
                 O.mx_dequantize(codes, scales).reshape(wl.batch, wl.n_k, wl.h_kv, wl.d))
    s_o = O.block_scores(prob, host(x["iq"]), host(x["ik"]))
    ids_o = O.select(prob, s_o)
    ids = torch.from_numpy(ids_o.reshape(wl.batch, wl.n_q, wl.h_kv, wl.topk)).cuda()
    p = api.problem_of(wl, sched=sched, kv_format="mxfp8")
    out, lse = api.sparse_attention(p, x["q"], kv["k"][0], kv["v"][0], ids)
    torch.cuda.synchronize()
    q64 = to_f64(x["q"])
    o_o, l_o = O.attend(prob, q64, np.ascontiguousarray(kv["k"][1]), np.ascontiguousarray(kv["v"][1]), ids_o)
    mx, rl = assert_attention(wl.dtype, to_f64(out).reshape(o_o.shape), o_o, host(lse).numpy().reshape(l_o.shape),
                              l_o, what=f"{name}/attention")
    # the whole forward over an all-MXFP8 cache (index keys too) selects as the
    # MX index path does and attends as above
    pa = api.problem_of(wl, sched=sched, idx_format="mxfp8", kv_format="mxfp8")
    ik_cache = api.mxfp8_quantize(x["ik"])
    ids_a, out_a, _ = api.forward(pa, x["q"], kv["k"][0], kv["v"][0], x["iq"], ik_cache)
    ids_i, _, _ = api.forward(api.problem_of(wl, sched=sched, idx_format="mxfp8"), x["q"], x["k"], x["v"], x["iq"],
                              ik_cache)
    out_b, _ = api.sparse_attention(p, x["q"], kv["k"][0], kv["v"][0], ids_a)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_i)
    assert torch.equal(out_a.view(torch.uint8) if out_a.dtype == torch.bfloat16 else out_a,
                       out_b.view(torch.uint8) if out_b.dtype == torch.bfloat16 else out_b)
    print(f"{name}: attention max-abs {mx:.2e} rel-L2 {rl:.2e}")
