"""GPU parity on block id tables a caller hands in, not ones the Index Branch
wrote: repeated blocks in a row, -1 and other negative ids, ids at or past the
number of blocks (up to INT32_MAX), blocks past the query's own and rows that
select nothing visible.  The result of every such table is defined by the
fp64 oracle (pinned on the CPU against SDPA and autograd over the gathered
keys, tests/test_tables.py); both attention schedules, the inversion, the
backward and the indexer loss must match it, and no kernel may read or write
outside its buffers (a stray write would show up as a wrong value elsewhere).

Also the exp-free Top-k on score rows holding -inf and NaN, through both Top-k
kernels: bit-exact against the oracle's selection (NaN ranks with -inf, below
every finite score; ties to the lower id).
"""
import numpy as np
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs
from oracle import oracle as O

from tests.parity import assert_attention, host, to_f64

pytestmark = pytest.mark.gpu

INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1

CASES = {
    # several query tiles, a ragged last block, q_offset inside a block
    "bf16_offset": dict(dtype="bf16", n_q=700, n_k=3000, q_offset=2300, h_q=16, h_kv=2, d=128, d_idx=64, topk=8),
    "f32_bk64": dict(n_q=600, n_k=1500, q_offset=900, h_q=8, h_kv=2, d=64, d_idx=32, topk=6, block_size=64),
    # few blocks, many queries: a repeated block becomes several work items
    "bf16_crowded": dict(dtype="bf16", n_q=1500, n_k=1500, h_q=16, h_kv=1, d=128, d_idx=128, topk=16),
    # one query per sequence (query-outer with split partials)
    "bf16_decode": dict(dtype="bf16", batch=3, n_q=1, n_k=5000, q_offset=4999, h_q=16, h_kv=2, d=128, d_idx=128,
                        topk=8),
}
NAMES = sorted(CASES)
_cache = {}


def messy_table(wl, seed):
    """[B, Nq, Hkv, k] int32 built to hold every kind of entry."""
    rng = np.random.default_rng(seed)
    nb = wl.nblk
    B, Nq, H, K = wl.batch, wl.n_q, wl.h_kv, wl.topk
    L = (wl.q_offset + np.arange(Nq)) // wl.block_size
    # start from random blocks at or before the local one
    ids = (rng.random((B, Nq, H, K)) * (L[None, :, None, None] + 1)).astype(np.int64)
    junk = np.array([-1, -1, -7, INT32_MIN, nb, nb + 5, 10 ** 6, INT32_MAX], dtype=np.int64)
    r = rng.random(ids.shape)
    ids[r < 0.15] = rng.choice(junk, size=int((r < 0.15).sum()))
    # repeats: copy another slot of the same row
    rep = (r >= 0.15) & (r < 0.30)
    src = rng.integers(0, K, size=ids.shape)
    ids[rep] = np.take_along_axis(ids, src, axis=3)[rep]
    # blocks past the query (where there are any)
    fut = (r >= 0.30) & (r < 0.36)
    later = L[None, :, None, None] + 1 + (rng.random(ids.shape) * np.maximum(nb - 1 - L, 0)[None, :, None, None])
    ids[fut & (L[None, :, None, None] < nb - 1)] = later.astype(np.int64)[fut & (L[None, :, None, None] < nb - 1)]
    # whole rows of one kind
    ids[0, 0, 0, :] = L[0]                          # the local block, K times
    if B > 1:
        ids[1, 0, H - 1, :] = -1                    # nothing listed (one query per sequence too)
    if Nq > 3:
        ids[0, 1, :, :] = -1                        # nothing listed
        ids[0, 2, 0, :] = INT32_MAX                 # nothing valid
        ids[0, 3, H - 1, :] = np.where(np.arange(K) % 2 == 0, 0, -1)  # block 0 on every other slot
    if Nq > 40:
        hot = int(L[40] // 2)
        ids[:, 40:, 0, 0] = hot                     # a hot block, listed twice by every later query
        ids[:, 40:, 0, K - 1] = hot
    return ids.astype(np.int32)


def case(name):
    if name not in _cache:
        wl = inputs.small(name, seed=7000 + NAMES.index(name), **CASES[name])
        x = inputs.generate(wl, device="cuda", tensors=("q", "k", "v", "iq", "ik", "dout"))
        h = {k: host(v) for k, v in x.items()}
        ids = messy_table(wl, 7100 + NAMES.index(name))
        prob = O.problem_of(wl)
        rows = ids.reshape(-1, wl.h_kv, wl.topk)
        out, lse = O.attend(prob, h["q"], h["k"], h["v"], rows)
        _cache[name] = (wl, x, h, ids, out, lse)
    return _cache[name]


def _ids_dev(ids):
    return torch.from_numpy(np.ascontiguousarray(ids)).cuda()


@pytest.mark.parametrize("name", NAMES)
def test_invert_messy_table(name):
    wl, x, h, ids, _, _ = case(name)
    off, ent = api.invert(api.problem_of(wl), _ids_dev(ids))
    torch.cuda.synchronize()
    off_o, ent_o = O.invert(O.problem_of(wl), ids)
    off, ent = host(off).numpy(), host(ent).numpy()
    assert np.array_equal(off, off_o)
    for b in range(wl.batch):
        for g in range(wl.h_kv):
            n = off_o[b, g, -1]
            assert np.array_equal(ent[b, g, :n], ent_o[b, g, :n])


@pytest.mark.parametrize("sched", ["kv_outer", "q_outer"])
@pytest.mark.parametrize("name", NAMES)
def test_attention_messy_table(name, sched):
    wl, x, h, ids, out_o, lse_o = case(name)
    p = api.problem_of(wl, sched=sched)
    out, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], _ids_dev(ids))
    # a second call with the smallest workspace (query chunks) must agree bitwise
    ws = api.alloc_workspace(p, api.OP_ATTENTION, minimal=True)
    out2, lse2 = api.sparse_attention(p, x["q"], x["k"], x["v"], _ids_dev(ids), ws=ws)
    torch.cuda.synchronize()
    empty = np.isneginf(lse_o)
    assert empty.any()
    mx, rl = assert_attention(wl.dtype, to_f64(out).reshape(out_o.shape), out_o,
                              host(lse).numpy().reshape(lse_o.shape), lse_o, what=f"{name}/{sched}")
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    print(f"{name}/{sched}: max-abs {mx:.2e} rel-L2 {rl:.2e}, {int(empty.sum())} empty rows")


def _check_grad(dtype, got, ref, what):
    tol = dict(bf16=(1e-2, 3e-2), f32=(2e-5, 2e-5))[dtype]
    diff = to_f64(got).reshape(ref.shape) - ref
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    mx = float(np.max(np.abs(diff))) / scale
    rl = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    assert rl <= tol[0] and mx <= tol[1], f"{what}: max-abs/max {mx:.3e} rel-L2 {rl:.3e} ({dtype})"
    return mx, rl


@pytest.mark.parametrize("name", NAMES)
def test_backward_messy_table(name):
    wl, x, h, ids, _, lse_o = case(name)
    p = api.problem_of(wl)
    d = _ids_dev(ids)
    out, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], d)
    dq, dk, dv = api.sparse_attention_backward(p, x["q"], x["k"], x["v"], out, lse, x["dout"], d)
    torch.cuda.synchronize()
    rq, rk, rv = O.attend_backward(O.problem_of(wl), h["q"], h["k"], h["v"], h["dout"],
                                   ids.reshape(-1, wl.h_kv, wl.topk))
    e = [_check_grad(wl.dtype, dq, rq, "dq"), _check_grad(wl.dtype, dk, rk, "dk"), _check_grad(wl.dtype, dv, rv, "dv")]
    # rows with nothing visible: exactly zero dq
    empty = np.isneginf(lse_o).reshape(wl.batch, wl.n_q, wl.h_q)
    assert np.all(to_f64(dq)[empty] == 0)
    print(f"{name}: " + ", ".join(f"{n} {a:.2e}/{b:.2e}" for n, (a, b) in zip(("dq", "dk", "dv"), e)))


@pytest.mark.parametrize("name", NAMES)
def test_indexer_kl_messy_table(name):
    wl, x, h, ids, _, _ = case(name)
    p = api.problem_of(wl)
    d = _ids_dev(ids)
    _, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], d)
    kl, d_iq, d_ik = api.indexer_kl(p, x["q"], x["k"], x["iq"], x["ik"], lse, d, loss_scale=0.25)
    torch.cuda.synchronize()
    rkl, riq, rik = O.indexer_kl(O.problem_of(wl), h["q"], h["k"], h["iq"], h["ik"],
                                 ids.reshape(-1, wl.h_kv, wl.topk), loss_scale=0.25)
    got = host(kl).numpy().astype(np.float64).reshape(rkl.shape)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - rkl)))
    assert err <= 1e-4 * float(np.max(rkl)) + 1e-6, f"kl: max-abs {err:.3e}"
    e_q = _check_grad(wl.dtype, d_iq, riq, "d_iq")
    e_k = _check_grad(wl.dtype, d_ik, rik, "d_ik")
    print(f"{name}: kl {err:.2e}, d_iq {e_q}, d_ik {e_k}")


@pytest.mark.parametrize("n_q,n_k,topk", [(40, 40 * 128, 9), (3, 3000 * 128, 16), (2, 2500 * 128 + 5, 32)])
def test_topk_nonfinite_scores(n_q, n_k, topk):
    """Rows with -inf, NaN and few finite scores: both Top-k kernels (a wave
    per row; a workgroup per row for long rows) equal the oracle exactly."""
    wl = inputs.small("nonfinite", n_q=n_q, n_k=n_k, q_offset=n_k - n_q, h_q=4, h_kv=2, topk=topk)
    p = api.problem_of(wl)
    nb = wl.nblk
    rng = np.random.default_rng(11 + n_q)
    S = rng.integers(-2, 3, size=(1, wl.h_kv, n_q, nb)).astype(np.float32)
    kind = rng.random(S.shape)
    S[kind < 0.3] = -np.inf
    S[(kind >= 0.3) & (kind < 0.5)] = np.nan
    S[0, 0, 0, :] = np.nan                        # nothing finite
    S[0, 1, 0, :] = -np.inf
    S[0, 0, 1, :] = np.nan
    S[0, 0, 1, 5:8] = 1.0                         # three finite scores only
    ids = api.topk_from_scores(p, torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    S64 = S.astype(np.float64).transpose(0, 2, 1, 3).reshape(n_q, wl.h_kv, nb)
    L = (np.arange(n_q) + wl.q_offset) // wl.block_size
    S64 = np.where(np.arange(nb)[None, None, :] >= L[:, None, None], -np.inf, S64)  # only j < L is read
    want = O.select(O.problem_of(wl), S64)
    got = host(ids).numpy().reshape(n_q, wl.h_kv, wl.topk)
    assert np.array_equal(got, want)
