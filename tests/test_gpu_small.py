"""GPU parity on small and edge-case shapes: HIP path (through the C ABI) vs
the fp64 oracle on the same seeded inputs, element by element.

Each case is small enough for the oracle to evaluate every query, yet spans
several key blocks and query tiles, and most end in a ragged partial block.
"""
import numpy as np
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs
from oracle import oracle as O

from tests.parity import assert_attention, check_selection, host, to_f64

pytestmark = pytest.mark.gpu

# name -> overrides of the tiny fp32 workload (B=1, N=4096, k=4, Hq=8, Hkv=2, d=64, d_idx=32)
CASES = {
    "tiny_f32_4k": dict(),
    "bf16_ragged": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=6),
    "bf16_offset": dict(dtype="bf16", n_q=700, n_k=3000, q_offset=2300, h_q=8, h_kv=1, d=128, d_idx=64, topk=5),
    "f32_g1": dict(n_q=900, n_k=900, h_q=4, h_kv=4, d=64, d_idx=64, topk=3),
    "bf16_k1": dict(dtype="bf16", n_q=600, n_k=600, topk=1),
    "bf16_dense": dict(dtype="bf16", n_q=700, n_k=700, topk=8),
    "bf16_short": dict(dtype="bf16", n_q=50, n_k=50, topk=4),
    "bf16_decode": dict(dtype="bf16", batch=3, n_q=1, n_k=5000, q_offset=4999, h_q=16, h_kv=2, d=128, d_idx=128,
                        topk=8),
    "f32_few_queries": dict(n_q=5, n_k=3000, q_offset=2995, topk=4),
    "bf16_batch2": dict(dtype="bf16", batch=2, n_q=800, n_k=800, topk=4),
    "bf16_sharp": dict(dtype="bf16", n_q=1200, n_k=1200, h_q=16, h_kv=2, d=128, d_idx=128, topk=5, sharp=True),
    "bf16_g32": dict(dtype="bf16", n_q=500, n_k=500, h_q=32, h_kv=1, d=64, d_idx=32, topk=3),
    "bf16_hot": dict(dtype="bf16", n_q=2048, n_k=2048, h_q=16, h_kv=2, d=128, d_idx=128, topk=6, hot_frac=0.1),
    "f32_sharp_offset": dict(n_q=333, n_k=1500, q_offset=1111, h_q=8, h_kv=2, d=128, d_idx=128, topk=5, sharp=True),
    # smaller key blocks (the pages' block-size ablation): both index kernels,
    # both schedules, partial last 128-token chunks
    "bf16_bk64": dict(dtype="bf16", n_q=1000, n_k=1000, h_q=16, h_kv=4, d=128, d_idx=128, topk=8, block_size=64),
    "f32_bk32": dict(n_q=700, n_k=700, h_q=8, h_kv=2, d=64, d_idx=32, topk=6, block_size=32),
    "bf16_bk32_offset": dict(dtype="bf16", n_q=300, n_k=2050, q_offset=1750, h_q=8, h_kv=1, d=128, d_idx=64,
                             topk=12, block_size=32),
    "bf16_bk64_decode": dict(dtype="bf16", batch=2, n_q=1, n_k=5001, q_offset=5000, h_q=16, h_kv=2, d=128,
                             d_idx=128, topk=16, block_size=64),
    "f32_bk32_few": dict(n_q=5, n_k=3000, q_offset=2995, topk=4, block_size=32),
    # more than 2048 candidate blocks and few rows: the workgroup-per-row Top-k
    "bf16_long_decode": dict(dtype="bf16", batch=2, n_q=1, n_k=2100 * 128 + 77, q_offset=2100 * 128 + 76, h_q=8,
                             h_kv=2, d=64, d_idx=32, topk=16),
}

_cache = {}


def case(name):
    if name not in _cache:
        wl = inputs.small(name, seed=2000 + sorted(CASES).index(name), **CASES[name])
        x = inputs.generate(wl, device="cuda")
        h = {k: host(v) for k, v in x.items()}
        prob = O.problem_of(wl)
        ids, out, lse, s = O.forward(prob, h["q"], h["k"], h["v"], h["iq"], h["ik"])
        _cache[name] = (wl, x, h, dict(ids=ids, out=out, lse=lse, s=s))
    return _cache[name]


NAMES = sorted(CASES)


@pytest.mark.parametrize("name", NAMES)
def test_selection(name):
    wl, x, h, ora = case(name)
    p = api.problem_of(wl)
    ids = api.index_topk(p, x["iq"], x["ik"])
    torch.cuda.synchronize()
    ids_h = host(ids).numpy().reshape(wl.batch * wl.n_q, wl.h_kv, wl.topk)
    res = check_selection(wl, ids_h, ora["ids"], ora["s"])
    assert res["fail"] == 0, res
    print(f"{name}: exact rows {res['exact']}, tie-band rows {res['tie']}")


@pytest.mark.parametrize("name", NAMES)
def test_block_scores(name):
    wl, x, h, ora = case(name)
    p = api.problem_of(wl)
    S = api.block_scores(p, x["iq"], x["ik"])
    torch.cuda.synchronize()
    S = host(S).numpy().astype(np.float64).transpose(0, 2, 1, 3).reshape(wl.batch * wl.n_q, wl.h_kv, -1)
    cand = np.isfinite(ora["s"])
    assert np.array_equal(np.isfinite(S), cand), "candidate pattern differs"
    assert np.all(np.isneginf(S[~cand]))
    # fp32 accumulation of exact products: error far below the 1e-3 tie band
    scale = np.max(np.abs(ora["s"][cand])) if cand.any() else 1.0
    err = np.max(np.abs(S[cand] - ora["s"][cand])) if cand.any() else 0.0
    assert err <= 1e-5 * max(scale, 1.0), err


@pytest.mark.parametrize("name", NAMES)
def test_topk_of_same_scores_is_exact(name):
    """Given identical block scores, GPU Top-k equals the oracle's exactly."""
    wl, x, h, ora = case(name)
    p = api.problem_of(wl)
    S = api.block_scores(p, x["iq"], x["ik"])
    ids = api.topk_from_scores(p, S)
    torch.cuda.synchronize()
    S64 = host(S).numpy().astype(np.float64).transpose(0, 2, 1, 3).reshape(wl.batch * wl.n_q, wl.h_kv, -1)
    want = O.select(O.problem_of(wl), S64)
    got = host(ids).numpy().reshape(wl.batch * wl.n_q, wl.h_kv, wl.topk)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n_q,n_k,topk", [(40, 40 * 128, 9), (3, 3000 * 128, 16), (2, 2500 * 128 + 5, 32)])
def test_topk_planted_ties(n_q, n_k, topk):
    """Scores drawn from three values, so nearly every row is decided by the
    lowest-id rule; both Top-k kernels (wave per row, workgroup per row for
    long rows) must equal the oracle exactly."""
    wl = inputs.small("ties", n_q=n_q, n_k=n_k, q_offset=n_k - n_q, h_q=4, h_kv=2, topk=topk)
    p = api.problem_of(wl)
    nb = (n_k + 127) // 128
    rng = np.random.default_rng(7 + n_q)
    S = rng.integers(0, 3, size=(1, wl.h_kv, n_q, nb)).astype(np.float32)
    ids = api.topk_from_scores(p, torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    S64 = S.astype(np.float64).transpose(0, 2, 1, 3).reshape(n_q, wl.h_kv, nb)
    L = (np.arange(n_q) + wl.q_offset) // 128
    S64 = np.where(np.arange(nb)[None, None, :] >= L[:, None, None], -np.inf, S64)  # only j < L is read
    want = O.select(O.problem_of(wl), S64)
    got = host(ids).numpy().reshape(n_q, wl.h_kv, wl.topk)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", NAMES)
def test_invert_exact(name):
    wl, x, h, ora = case(name)
    p = api.problem_of(wl)
    ids = torch.from_numpy(ora["ids"].reshape(wl.batch, wl.n_q, wl.h_kv, wl.topk)).cuda()
    off, ent = api.invert(p, ids)
    torch.cuda.synchronize()
    off_o, ent_o = O.invert(O.problem_of(wl), ora["ids"])
    off, ent = host(off).numpy(), host(ent).numpy()
    assert np.array_equal(off, off_o)
    for b in range(wl.batch):
        for g in range(wl.h_kv):
            n = off_o[b, g, -1]
            assert np.array_equal(ent[b, g, :n], ent_o[b, g, :n])


@pytest.mark.parametrize("sched", ["kv_outer", "q_outer"])
@pytest.mark.parametrize("name", NAMES)
def test_attention(name, sched):
    wl, x, h, ora = case(name)
    p = api.problem_of(wl, sched=sched)
    ids = torch.from_numpy(ora["ids"].reshape(wl.batch, wl.n_q, wl.h_kv, wl.topk)).cuda()
    out, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    torch.cuda.synchronize()
    mx, rl = assert_attention(wl.dtype, to_f64(out).reshape(ora["out"].shape), ora["out"],
                              host(lse).numpy().reshape(ora["lse"].shape), ora["lse"], what=f"{name}/{sched}")
    print(f"{name}/{sched}: max-abs {mx:.2e} rel-L2 {rl:.2e}")


@pytest.mark.parametrize("name", NAMES)
def test_forward_composes(name):
    """msa_forward = msa_index_topk then msa_sparse_attention, bitwise."""
    wl, x, h, ora = case(name)
    p = api.problem_of(wl)
    ids, out, lse = api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    ids2 = api.index_topk(p, x["iq"], x["ik"])
    out2, lse2 = api.sparse_attention(p, x["q"], x["k"], x["v"], ids2)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("sched", ["kv_outer", "q_outer"])
@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_hot", "tiny_f32_4k", "bf16_decode"])
def test_deterministic_and_chunk_independent(name, sched):
    wl, x, h, ora = case(name)
    p = api.problem_of(wl, sched=sched)
    ids = api.index_topk(p, x["iq"], x["ik"])
    o1, l1 = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    o2, l2 = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    ws_min = api.alloc_workspace(p, api.OP_ATTENTION, minimal=True)
    o3, l3 = api.sparse_attention(p, x["q"], x["k"], x["v"], ids, ws=ws_min)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
