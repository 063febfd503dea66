"""GPU parity of the Main Branch backward (dq, dk, dv for a fixed selection):
HIP path through the C ABI vs the fp64 oracle on the same seeded inputs.

The selection is the oracle's; the forward's out and lse come from the HIP
forward on that selection (as a training step would have them).

Tolerances, from the arithmetic of the kernels (fp32 accumulation throughout):
  * bf16: the MFMA operands P and dS are rounded to bf16 (relative error
    2^-9 each, independent across the k*Bk terms of a sum) and the outputs are
    stored in bf16 (another 2^-9): rel-L2 <= 1e-2 and max-abs <= 3e-2 of the
    tensor's largest magnitude.
  * fp32: products in fp32 MFMA (about 2^-24 per term, sums of up to
    k*Bk = 4096 terms), exponentials from the hardware exp2 (about 1 ulp):
    rel-L2 <= 2e-5, max-abs <= 2e-5 of the tensor's largest magnitude.
Keys that no query attends get exactly zero gradients, and two runs give
bitwise-equal results (every sum has a fixed order).
"""
import numpy as np
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs
from oracle import oracle as O

from tests.parity import host, to_f64

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(rel_l2=1e-2, max_rel=3e-2), "f32": dict(rel_l2=2e-5, max_rel=2e-5)}

# name -> overrides of the tiny fp32 workload (B=1, N=4096, k=4, Hq=8, Hkv=2, d=64, d_idx=32)
CASES = {
    "tiny_f32_4k": dict(),
    "bf16_ragged": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=6),
    "bf16_offset": dict(dtype="bf16", n_q=700, n_k=3000, q_offset=2300, h_q=8, h_kv=1, d=128, d_idx=64, topk=5),
    "f32_g1": dict(n_q=900, n_k=900, h_q=4, h_kv=4, d=64, d_idx=64, topk=3),
    "bf16_k1": dict(dtype="bf16", n_q=600, n_k=600, topk=1),
    "bf16_short": dict(dtype="bf16", n_q=50, n_k=50, topk=4),
    "bf16_decode": dict(dtype="bf16", batch=3, n_q=1, n_k=5000, q_offset=4999, h_q=16, h_kv=2, d=128, d_idx=128,
                        topk=8),
    "bf16_batch2": dict(dtype="bf16", batch=2, n_q=800, n_k=800, topk=4),
    "bf16_g32": dict(dtype="bf16", n_q=500, n_k=500, h_q=32, h_kv=1, d=64, d_idx=32, topk=3),
    # most queries pick the same few blocks: several work items per block
    "bf16_hot": dict(dtype="bf16", n_q=2048, n_k=2048, h_q=16, h_kv=2, d=128, d_idx=128, topk=6, hot_frac=0.1),
    "f32_d128": dict(n_q=1200, n_k=1200, h_q=8, h_kv=2, d=128, d_idx=128, topk=5),
    "f32_d128_hot": dict(n_q=1500, n_k=1500, h_q=16, h_kv=2, d=128, d_idx=64, topk=4, hot_frac=0.2),
    "bf16_bk64": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=8, block_size=64),
    "f32_bk32": dict(n_q=700, n_k=700, h_q=8, h_kv=2, d=64, d_idx=32, topk=6, block_size=32),
    "f32_d128_bk64": dict(n_q=900, n_k=900, h_q=8, h_kv=2, d=128, d_idx=32, topk=6, block_size=64),
    "bf16_bk32_offset": dict(dtype="bf16", n_q=300, n_k=2050, q_offset=1750, h_q=8, h_kv=1, d=128, d_idx=64,
                             topk=12, block_size=32),
    "bf16_g1_d128": dict(dtype="bf16", n_q=700, n_k=700, h_q=4, h_kv=4, d=128, d_idx=128, topk=5),
    "bf16_g16_d128": dict(dtype="bf16", n_q=600, n_k=600, h_q=16, h_kv=1, d=128, d_idx=64, topk=4),
}
NAMES = sorted(CASES)
_cache = {}


def case(name):
    if name not in _cache:
        wl = inputs.small(name, seed=4000 + NAMES.index(name), **CASES[name])
        x = inputs.generate(wl, device="cuda", tensors=("q", "k", "v", "iq", "ik", "dout"))
        h = {k: host(v) for k, v in x.items()}
        prob = O.problem_of(wl)
        s = O.block_scores(prob, h["iq"], h["ik"])
        ids = O.select(prob, s)
        grads = O.attend_backward(prob, h["q"], h["k"], h["v"], h["dout"], ids)
        _cache[name] = (wl, x, ids, grads)
    return _cache[name]


def run_backward(wl, x, ids_np):
    p = api.problem_of(wl)
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).reshape(
        wl.batch, wl.n_q, wl.h_kv, wl.topk).to("cuda")
    out, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    dq, dk, dv = api.sparse_attention_backward(p, x["q"], x["k"], x["v"], out, lse, x["dout"], ids)
    torch.cuda.synchronize()
    return dq, dk, dv


def attended_keys(wl, ids):
    """[B, Nk, Hkv] bool: token t of group g is visible to some query that selects its block."""
    ids = np.asarray(ids).reshape(wl.batch, wl.n_q, wl.h_kv, wl.topk)
    seen = np.zeros((wl.batch, wl.n_k, wl.h_kv), dtype=bool)
    bk = wl.block_size
    for b in range(wl.batch):
        for g in range(wl.h_kv):
            # the largest visible position per block over the queries selecting it
            last = np.full(wl.nblk, -1, dtype=np.int64)
            pos = wl.q_offset + np.arange(wl.n_q)
            for s in range(wl.topk):
                blk = ids[b, :, g, s]
                ok = blk >= 0
                np.maximum.at(last, blk[ok], pos[ok])
            for j in np.nonzero(last >= 0)[0]:
                t0 = j * bk
                t1 = min(wl.n_k, t0 + bk, last[j] + 1)
                seen[b, t0:t1, g] = True
    return seen


def check(dtype, got, ref, what):
    tol = TOL[dtype]
    a = to_f64(got)
    diff = a - ref
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    mx = float(np.max(np.abs(diff))) / scale
    rl = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    assert mx <= tol["max_rel"] and rl <= tol["rel_l2"], f"{what}: max-abs/max {mx:.3e} rel-L2 {rl:.3e} ({dtype})"
    return mx, rl


@pytest.mark.parametrize("name", NAMES)
def test_backward_matches_oracle(name):
    wl, x, ids, (rq, rk, rv) = case(name)
    dq, dk, dv = run_backward(wl, x, ids)
    errs = [check(wl.dtype, dq, rq, "dq"), check(wl.dtype, dk, rk, "dk"), check(wl.dtype, dv, rv, "dv")]
    # keys nobody attends: exactly zero
    seen = attended_keys(wl, ids)
    for t, nm in ((dk, "dk"), (dv, "dv")):
        z = to_f64(t)[~seen]
        assert np.all(z == 0), f"{nm}: {int(np.count_nonzero(z))} nonzero values at unattended keys"
    print(f"{name}: " + ", ".join(f"{n} max {a:.2e} rl2 {b:.2e}" for n, (a, b) in zip(("dq", "dk", "dv"), errs)))


@pytest.mark.parametrize("name", ["bf16_hot", "f32_d128_hot"])
def test_backward_is_deterministic(name):
    wl, x, ids, _ = case(name)
    a = run_backward(wl, x, ids)
    b = run_backward(wl, x, ids)
    for u, w, nm in zip(a, b, ("dq", "dk", "dv")):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           w.view(torch.uint8) if w.dtype == torch.bfloat16 else w), nm


def test_backward_full_size_prefill_32k():
    """The bench's prefill shape (32k tokens, Hq 64, Hkv 8, d 128, k 16, bf16),
    whole problem in one call.  Checked against the oracle on a sample of query
    rows (dq) and on the last key block of every group (dk, dv: only the last
    Bk queries can select it, and all of them are in the sample), with the
    oracle's selection substituted for those rows.  Over all rows, two
    properties of the chain rule through a softmax: sum_t dv_t equals the sum
    of dout over the group's query rows (the P of a row sum to 1), and
    sum_t dk_t vanishes (the dS of a row sum to 0)."""
    wl = inputs.WORKLOADS["prefill_32k"]
    print(f"[{wl.name}] generating", flush=True)
    x = inputs.generate(wl, device="cuda", tensors=("q", "k", "v", "iq", "ik", "dout"))
    p = api.problem_of(wl)
    ids = api.index_topk(p, x["iq"], x["ik"])
    Bk, N = wl.block_size, wl.n_q
    last0 = (wl.nblk - 1) * Bk
    qi = np.unique(np.concatenate([np.linspace(0, last0 - 1, 24).astype(np.int64), np.arange(last0, N)]))
    rows = np.stack([np.zeros_like(qi), qi], axis=1)
    prob = O.problem_of(wl)
    hx = {k: host(v) for k, v in x.items()}
    s = O.block_scores(prob, hx["iq"], hx["ik"], rows)
    ids_o = O.select(prob, s, rows)
    ids[0, qi] = torch.from_numpy(ids_o).cuda()
    print(f"[{wl.name}] oracle selection of {len(qi)} rows done", flush=True)
    out, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    dq, dk, dv = api.sparse_attention_backward(p, x["q"], x["k"], x["v"], out, lse, x["dout"], ids)
    torch.cuda.synchronize()
    print(f"[{wl.name}] GPU backward done", flush=True)
    rq, rk, rv = O.attend_backward(prob, hx["q"], hx["k"], hx["v"], hx["dout"], ids_o, rows=rows)
    print(f"[{wl.name}] oracle backward done", flush=True)
    e_q = check(wl.dtype, dq[0, qi], rq, "dq (sampled rows)")
    e_k = check(wl.dtype, dk[0, last0:], rk[0, last0:], "dk (last block)")
    e_v = check(wl.dtype, dv[0, last0:], rv[0, last0:], "dv (last block)")
    print(f"[{wl.name}] dq {e_q}, dk {e_k}, dv {e_v}", flush=True)
    # properties over every row
    G = wl.h_q // wl.h_kv
    dv_sum = dv.double().sum(dim=1)                                             # [B, Hkv, D]
    do_sum = x["dout"].double().sum(dim=1).reshape(wl.batch, wl.h_kv, G, wl.d).sum(dim=2)
    rel_v = float((dv_sum - do_sum).norm() / do_sum.norm())
    dk_sum = dk.double().sum(dim=1)
    rel_k = float(dk_sum.norm() / dk.double().abs().sum(dim=1).norm())
    print(f"[{wl.name}] sum dv vs sum dout rel {rel_v:.2e}; |sum dk| / sum |dk| {rel_k:.2e}", flush=True)
    assert rel_v <= 1e-2 and rel_k <= 1e-2
