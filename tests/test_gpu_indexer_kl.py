"""GPU parity of the Index-Branch alignment loss (KL from the Main Branch's
group-averaged distribution to the Index Branch's, on the selected tokens) and
its gradients for the index queries and keys: HIP path through the C ABI vs
the fp64 oracle on the same seeded inputs and the oracle's selection.  The
Main Branch lse comes from the HIP forward on that selection.

Tolerances, from the arithmetic of the kernels:
  * kl: every term is formed in fp32 from exactly widened inputs (scores,
    exponentials, logarithms; no bf16 rounding on this path), so
    |kl - kl_oracle| <= 1e-4 * max(kl_oracle) + 1e-6 per row.
  * gradients: the per-element gradient g = loss_scale * (pi - pm) enters the
    MFMA products rounded to the input type.  bf16: rel-L2 <= 1e-2 and
    max-abs <= 3e-2 of the tensor's largest magnitude (2^-9 per operand and
    per output, as for the attention backward).  fp32: rel-L2 <= 2e-5 and
    max-abs <= 2e-5 of the largest magnitude (pi - pm cancels where the two
    distributions agree, so fp32 rounding of pi and pm, about 1e-7 of the
    larger one, shows at a few 1e-6 of the gradient scale).
Keys that no query selects get exactly zero d_ik; two runs are bitwise equal.
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
    "bf16_g32": dict(dtype="bf16", n_q=500, n_k=500, h_q=32, h_kv=1, d=64, d_idx=32, topk=3),
    "bf16_hot": dict(dtype="bf16", n_q=2048, n_k=2048, h_q=16, h_kv=2, d=128, d_idx=128, topk=6, hot_frac=0.1),
    "f32_d128": dict(n_q=1200, n_k=1200, h_q=8, h_kv=2, d=128, d_idx=128, topk=5),
    "bf16_bk64": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=8, block_size=64),
    "f32_bk32": dict(n_q=700, n_k=700, h_q=8, h_kv=2, d=64, d_idx=32, topk=6, block_size=32),
    "bf16_bk32_offset": dict(dtype="bf16", n_q=300, n_k=2050, q_offset=1750, h_q=8, h_kv=1, d=128, d_idx=64,
                             topk=12, block_size=32),
    # group sizes around the head chunks of the 16-bit pass: one head (the odd-head waves idle), two heads, and
    # sixteen heads of d 128 (several chunks per tile)
    "bf16_g1_d128": dict(dtype="bf16", n_q=700, n_k=700, h_q=4, h_kv=4, d=128, d_idx=128, topk=5),
    "bf16_g2_bk64": dict(dtype="bf16", n_q=800, n_k=800, h_q=4, h_kv=2, d=64, d_idx=128, topk=6, block_size=64),
    "bf16_g16_d128": dict(dtype="bf16", n_q=600, n_k=600, h_q=16, h_kv=1, d=128, d_idx=64, topk=4),
}
NAMES = sorted(CASES)
LOSS_SCALE = 0.5
_cache = {}


def case(name):
    if name not in _cache:
        wl = inputs.small(name, seed=5000 + NAMES.index(name), **CASES[name])
        x = inputs.generate(wl, device="cuda")
        h = {k: host(v) for k, v in x.items()}
        prob = O.problem_of(wl)
        s = O.block_scores(prob, h["iq"], h["ik"])
        ids = O.select(prob, s)
        ref = O.indexer_kl(prob, h["q"], h["k"], h["iq"], h["ik"], ids, loss_scale=LOSS_SCALE)
        _cache[name] = (wl, x, ids, ref)
    return _cache[name]


def run_kl(wl, x, ids_np):
    p = api.problem_of(wl)
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).reshape(
        wl.batch, wl.n_q, wl.h_kv, wl.topk).to("cuda")
    _, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    kl, d_iq, d_ik = api.indexer_kl(p, x["q"], x["k"], x["iq"], x["ik"], lse, ids, loss_scale=LOSS_SCALE)
    torch.cuda.synchronize()
    return kl, d_iq, d_ik


def selected_keys(wl, ids):
    """[B, Nk, Hkv] bool: token t of group g is visible to some query that selects its block."""
    ids = np.asarray(ids).reshape(wl.batch, wl.n_q, wl.h_kv, wl.topk)
    seen = np.zeros((wl.batch, wl.n_k, wl.h_kv), dtype=bool)
    pos = wl.q_offset + np.arange(wl.n_q)
    for b in range(wl.batch):
        for g in range(wl.h_kv):
            last = np.full(wl.nblk, -1, dtype=np.int64)
            for s in range(wl.topk):
                blk = ids[b, :, g, s]
                ok = blk >= 0
                np.maximum.at(last, blk[ok], pos[ok])
            for j in np.nonzero(last >= 0)[0]:
                t0 = j * wl.block_size
                seen[b, t0:min(wl.n_k, t0 + wl.block_size, last[j] + 1), g] = True
    return seen


def check(dtype, got, ref, what):
    tol = TOL[dtype]
    diff = to_f64(got) - ref
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    mx = float(np.max(np.abs(diff))) / scale
    rl = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    assert mx <= tol["max_rel"] and rl <= tol["rel_l2"], f"{what}: max-abs/max {mx:.3e} rel-L2 {rl:.3e} ({dtype})"
    return mx, rl


@pytest.mark.parametrize("name", NAMES)
def test_indexer_kl_matches_oracle(name):
    wl, x, ids, (rkl, riq, rik) = case(name)
    kl, d_iq, d_ik = run_kl(wl, x, ids)
    got = host(kl).numpy().astype(np.float64).reshape(-1, wl.h_kv)
    err = float(np.max(np.abs(got - rkl)))
    assert err <= 1e-4 * float(np.max(rkl)) + 1e-6, f"kl: max-abs {err:.3e}, max kl {np.max(rkl):.3e}"
    e_q = check(wl.dtype, d_iq, riq.reshape(d_iq.shape), "d_iq")
    e_k = check(wl.dtype, d_ik, rik, "d_ik")
    z = to_f64(d_ik)[~selected_keys(wl, ids)]
    assert np.all(z == 0), f"d_ik: {int(np.count_nonzero(z))} nonzero values at unselected keys"
    print(f"{name}: kl max-abs {err:.2e} (mean kl {np.mean(rkl):.3e}), d_iq {e_q}, d_ik {e_k}")


def test_indexer_kl_is_deterministic():
    wl, x, ids, _ = case("bf16_hot")
    a = run_kl(wl, x, ids)
    b = run_kl(wl, x, ids)
    for u, w, nm in zip(a, b, ("kl", "d_iq", "d_ik")):
        assert torch.equal(u.view(torch.uint8), w.view(torch.uint8)), nm


def test_indexer_kl_full_size_prefill_32k():
    """The prefill shape (32k tokens, Hq 64, Hkv 8, d = d_idx = 128, k 16,
    bf16), whole problem in one call.  Checked against the oracle on a sample
    of query rows (kl, d_iq) and on the last key block of every group (d_ik:
    only the last Bk queries can select it, all of them sampled), with the
    oracle's selection substituted for those rows.  Over all rows: kl >= 0,
    and sum_t d_ik_t vanishes per group (sum_t (pi - pm) = 0 for every row)."""
    wl = inputs.WORKLOADS["prefill_32k"]
    print(f"[{wl.name}] generating", flush=True)
    x = inputs.generate(wl, device="cuda")
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
    _, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    kl, d_iq, d_ik = api.indexer_kl(p, x["q"], x["k"], x["iq"], x["ik"], lse, ids, loss_scale=LOSS_SCALE)
    torch.cuda.synchronize()
    print(f"[{wl.name}] GPU loss done", flush=True)
    rkl, riq, rik = O.indexer_kl(prob, hx["q"], hx["k"], hx["iq"], hx["ik"], ids_o, rows=rows, loss_scale=LOSS_SCALE)
    print(f"[{wl.name}] oracle done", flush=True)
    got = host(kl[0, qi]).numpy().astype(np.float64)
    err = float(np.max(np.abs(got - rkl)))
    assert err <= 1e-4 * float(np.max(rkl)) + 1e-6, f"kl: max-abs {err:.3e}"
    e_q = check(wl.dtype, d_iq[0, qi], riq, "d_iq (sampled rows)")
    e_k = check(wl.dtype, d_ik[0, last0:], rik[0, last0:], "d_ik (last block)")
    kmin = float(kl.min())
    dsum = d_ik.double().sum(dim=1)
    rel = float(dsum.norm() / d_ik.double().abs().sum(dim=1).norm())
    print(f"[{wl.name}] kl max-abs {err:.2e}, d_iq {e_q}, d_ik {e_k}, min kl {kmin:.2e}, "
          f"|sum d_ik| / sum |d_ik| {rel:.2e}", flush=True)
    assert kmin >= -1e-5 and rel <= 1e-2
