"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

Nothing here re-types the oracle's formulas.  Each pin is one of:
  * a hand-worked example (tests/golden/worked_example_bk2.json);
  * a closed form on planted data (block max pooling, causality);
  * brute-force enumeration (Top-k with ties on tiny inputs);
  * a special case that reduces to a library routine (k >= number of blocks
    gives dense causal GQA attention: torch's scaled_dot_product_attention in
    fp64; any selection gives SDPA with the selection as a boolean mask);
  * an invariant (permutation inside a block, monotone transforms of the
    scores, V == 1, one-hot V).
``test_planted_mistakes_are_caught`` builds mutated copies of the oracle
(one plausible mistake each) and checks that at least one pin fails for each.

Sources: MiniMax Sparse Attention paper summary (hyper.ai), Method;
zhichai.net write-up sections 2 and 4.1; readings for what the pages leave
open (ties to the lowest id, ascending ids with -1 padding, t <= p causality).
"""
import itertools
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import build as obuild
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _inputs(rng, B, Nq, Nk, Hq, Hkv, d, di):
    return dict(q=_rand((B, Nq, Hq, d), rng), k=_rand((B, Nk, Hkv, d), rng), v=_rand((B, Nk, Hkv, d), rng),
                iq=_rand((B, Nq, Hkv, di), rng), ik=_rand((B, Nk, Hkv, di), rng))


def _sdpa_masked(prob, q, k, v, allowed):
    """torch SDPA in fp64 with a boolean mask allowed[b, i, g, t] (True = attend)."""
    G = prob.h_q // prob.h_kv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                                # [B,Hq,Nq,d]
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)     # [B,Hq,Nk,d]
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    m = torch.from_numpy(allowed).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)  # [B,Hq,Nq,Nk]
    scale = prob.softmax_scale if prob.softmax_scale > 0 else 1.0 / math.sqrt(prob.d)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    logits = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~m, -math.inf), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def _causal_allowed(prob):
    B, Nq, Nk = prob.batch, prob.n_q, prob.n_k
    pos = prob.q_offset + np.arange(Nq)
    allowed = np.arange(Nk)[None, :] <= pos[:, None]
    return np.broadcast_to(allowed[None, :, None, :], (B, Nq, prob.h_kv, Nk)).copy()


# ----------------------------------------------------------------------------
# Pins.  Each takes an Oracle instance and raises AssertionError on failure.
# ----------------------------------------------------------------------------

def pin_golden_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_bk2.json")))
    prob = O.make_problem(**g["problem"])
    iq = np.array(g["idx_q"], dtype=np.float64).reshape(1, 8, 1, 2)
    ik = np.array(g["idx_k"], dtype=np.float64).reshape(1, 8, 1, 2)
    q = np.array(g["q"], dtype=np.float64).reshape(1, 8, 2, 2)
    k = np.array(g["k"], dtype=np.float64).reshape(1, 8, 1, 2)
    v = np.array(g["v"], dtype=np.float64).reshape(1, 8, 1, 2)
    s = orc.block_scores(prob, iq, ik)
    exp_s = np.array([[np.nan if x is None else x for x in row] for row in g["expect_scores"]])
    got_s = s[:, 0, :]
    cand = ~np.isnan(exp_s)
    assert np.array_equal(got_s[cand], exp_s[cand]), (got_s, exp_s)
    assert np.all(np.isneginf(got_s[~cand]))
    ids = orc.select(prob, s)
    assert np.array_equal(ids[:, 0, :], np.array(g["expect_ids"])), ids[:, 0, :]
    out, lse = orc.attend(prob, q, k, v, ids)
    np.testing.assert_allclose(out, np.array(g["expect_out"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(g["expect_lse"]), rtol=1e-14, atol=1e-14)


def pin_maxpool_closed_form(orc):
    """idx_q = a_i e0; block j: every token c_j e0 except one spike (c_j + e_j) e0.
    Then S_j = a_i (c_j + e_j) if a_i > 0 and a_i c_j if a_i < 0 (exact in fp64)."""
    rng = np.random.default_rng(7)
    B, Nq, Nk, H, di, Bk = 1, 40, 40, 2, 4, 4
    nb = Nk // Bk
    prob = O.make_problem(B, Nq, Nk, 2, H, 4, di, Bk, 3)
    a = rng.choice([-2.0, -0.5, 0.25, 1.0, 3.0], size=(Nq, H))
    iq = np.zeros((B, Nq, H, di))
    iq[0, :, :, 0] = a
    c = rng.integers(-8, 8, size=(nb, H)).astype(np.float64) / 4
    e = rng.integers(1, 8, size=(nb, H)).astype(np.float64) / 2
    spike = rng.integers(0, Bk, size=(nb, H))
    ik = np.zeros((B, Nk, H, di))
    ik[0, :, :, 1:] = rng.standard_normal((Nk, H, di - 1))  # orthogonal to idx_q: no effect
    for j in range(nb):
        for g in range(H):
            ik[0, j * Bk:(j + 1) * Bk, g, 0] = c[j, g]
            ik[0, j * Bk + spike[j, g], g, 0] = c[j, g] + e[j, g]
    s = orc.block_scores(prob, iq, ik)
    for i in range(Nq):
        L = i // Bk
        for g in range(H):
            exp = np.where(a[i, g] > 0, a[i, g] * (c[:, g] + e[:, g]), a[i, g] * c[:, g])
            assert np.array_equal(s[i, g, :L], exp[:L]), (i, g)
            assert np.all(np.isneginf(s[i, g, L:]))


def pin_scores_ignore_future_and_token_order(orc):
    """Permuting tokens inside a key block leaves block scores unchanged, and so
    does any change to keys at or after the local block."""
    rng = np.random.default_rng(11)
    B, N, H, di, Bk = 2, 48, 2, 8, 4
    prob = O.make_problem(B, N, N, 4, H, 8, di, Bk, 3)
    x = _inputs(rng, B, N, N, 4, H, 8, di)
    s0 = orc.block_scores(prob, x["iq"], x["ik"])
    ik2 = x["ik"].copy()
    for j in range(N // Bk):
        perm = rng.permutation(Bk)
        ik2[:, j * Bk:(j + 1) * Bk] = ik2[:, j * Bk + perm]
    assert np.array_equal(s0, orc.block_scores(prob, x["iq"], ik2))
    # keys of the last four blocks scaled up: only queries whose candidates
    # include those blocks may change.
    ik3 = x["ik"].copy()
    ik3[:, 32:] *= 1e3
    s3 = orc.block_scores(prob, x["iq"], ik3)
    assert np.array_equal(s0[:, :, :8], s3[:, :, :8])
    qs = np.arange(B * N) % N
    early = qs < 36  # L(i) <= 8: candidates are blocks 0..7 only
    assert np.array_equal(s0[early], s3[early])


def _brute_select(S, L, K):
    """Enumerate every (K-1)-subset of the candidates 0..L-1; keep the ones in
    which each member outranks each non-member under (score desc, id asc)."""
    if L <= K - 1:
        return list(range(L + 1))
    cands = range(L)
    found = []
    for T in itertools.combinations(cands, K - 1):
        Ts = set(T)
        ok = all((S[a] > S[b]) or (S[a] == S[b] and a < b) for a in Ts for b in cands if b not in Ts)
        if ok:
            found.append(T)
    assert len(found) == 1, found
    return sorted(list(found[0]) + [L])


def pin_topk_bruteforce(orc):
    rng = np.random.default_rng(3)
    for K in (1, 2, 3, 4):
        B, N, H, Bk = 1, 36, 3, 4  # 9 blocks
        prob = O.make_problem(B, N, N, H, H, 2, 2, Bk, K)
        nb = 9
        # integer scores in a narrow range: many ties
        S = rng.integers(-2, 3, size=(N, H, nb)).astype(np.float64)
        for i in range(N):
            S[i, :, i // Bk:] = -np.inf
        ids = orc.select(prob, S)
        for i in range(N):
            for g in range(H):
                exp = _brute_select(S[i, g], i // Bk, K)
                exp = exp + [-1] * (K - len(exp))
                assert list(ids[i, g]) == exp, (K, i, g, list(ids[i, g]), exp)


def pin_topk_special_cases(orc):
    B, N, H, Bk, K = 1, 64, 1, 4, 5  # 16 blocks
    prob = O.make_problem(B, N, N, H, H, 2, 2, Bk, K)
    S = np.zeros((N, H, 16))
    for i in range(N):
        S[i, :, i // Bk:] = -np.inf
    ids = orc.select(prob, S)
    for i in range(N):
        L = i // Bk
        if L <= K - 1:
            exp = list(range(L + 1)) + [-1] * (K - L - 1)
        else:  # all tied: the lowest ids win
            exp = list(range(K - 1)) + [L]
        assert list(ids[i, 0]) == exp, (i, list(ids[i, 0]), exp)
    # -0.0 and +0.0 are equal scores: the lower id wins
    S2 = S.copy()
    S2[N - 1, 0, 0] = -0.0
    S2[N - 1, 0, 1:15] = 0.0
    assert list(orc.select(prob, S2)[N - 1, 0]) == [0, 1, 2, 3, 15]


def pin_exp_free(orc):
    """Top-k on raw scores equals Top-k on softmax probabilities (the softmax
    is strictly increasing), zhichai.net write-up section 4.1."""
    rng = np.random.default_rng(5)
    B, N, H, Bk, K = 1, 256, 2, 4, 6
    prob = O.make_problem(B, N, N, H, H, 2, 2, Bk, K)
    S = rng.standard_normal((N, H, 64))
    P = np.zeros_like(S)
    for i in range(N):
        L = i // Bk
        S[i, :, L:] = -np.inf
        if L:
            P[i, :, :L] = torch.softmax(torch.from_numpy(S[i, :, :L]), dim=-1).numpy()
        P[i, :, L:] = -np.inf
    assert np.array_equal(orc.select(prob, S), orc.select(prob, P))
    # and invariance to any positive scale and shift
    assert np.array_equal(orc.select(prob, S), orc.select(prob, 3.0 * S - 7.0))


def pin_dense_equals_sdpa(orc):
    """k >= number of blocks: MSA is dense causal GQA attention."""
    rng = np.random.default_rng(13)
    for (B, Nq, Nk, off, Hq, Hkv, d, Bk) in [(2, 24, 24, 0, 4, 2, 8, 4), (1, 10, 27, 17, 6, 3, 16, 4),
                                             (1, 9, 9, 0, 2, 1, 4, 8)]:
        nb = (Nk + Bk - 1) // Bk
        prob = O.make_problem(B, Nq, Nk, Hq, Hkv, d, 4, Bk, nb + 1, off)
        x = _inputs(rng, B, Nq, Nk, Hq, Hkv, d, 4)
        ids, out, lse, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
        ref, ref_lse = _sdpa_masked(prob, x["q"], x["k"], x["v"], _causal_allowed(prob))
        np.testing.assert_allclose(out, ref.reshape(out.shape), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse.reshape(lse.shape), rtol=0, atol=1e-12)


def pin_sparse_equals_masked_sdpa(orc):
    """Any selection: attention over the visible tokens of the chosen blocks is
    SDPA with that token set as a boolean mask (shared by the group's heads)."""
    rng = np.random.default_rng(17)
    B, N, Hq, Hkv, d, di, Bk, K = 2, 40, 6, 2, 8, 4, 4, 3
    prob = O.make_problem(B, N, N, Hq, Hkv, d, di, Bk, K)
    x = _inputs(rng, B, N, N, Hq, Hkv, d, di)
    ids, out, lse, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    allowed = np.zeros((B, N, Hkv, N), dtype=bool)
    idr = ids.reshape(B, N, Hkv, K)
    for b in range(B):
        for i in range(N):
            for g in range(Hkv):
                for j in idr[b, i, g]:
                    if j >= 0:
                        allowed[b, i, g, j * Bk:(j + 1) * Bk] = True
    allowed &= _causal_allowed(prob)
    ref, ref_lse = _sdpa_masked(prob, x["q"], x["k"], x["v"], allowed)
    np.testing.assert_allclose(out, ref.reshape(out.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.reshape(lse.shape), rtol=0, atol=1e-12)


def pin_value_invariants(orc):
    """V == 1 gives O == 1; one-hot V recovers a probability vector that sums to
    one, vanishes off the visible selected tokens and peaks where q.k peaks."""
    rng = np.random.default_rng(19)
    B, N, Hq, Hkv, Bk, K = 1, 32, 2, 1, 4, 3
    d = 32  # one-hot over the 32 tokens
    prob = O.make_problem(B, N, N, Hq, Hkv, d, 2, Bk, K)
    x = _inputs(rng, B, N, N, Hq, Hkv, d, 2)
    ones = np.ones_like(x["v"])
    ids, out, _, _ = orc.forward(prob, x["q"], x["k"], ones, x["iq"], x["ik"])
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)
    eye = np.eye(N).reshape(1, N, 1, N)
    out, _ = orc.attend(prob, x["q"], x["k"], eye, ids)
    for i in range(N):
        vis = np.zeros(N, dtype=bool)
        for j in ids[i, 0]:
            if j >= 0:
                vis[j * Bk:(j + 1) * Bk] = True
        vis[i + 1:] = False
        for h in range(Hq):
            p = out[i, h]
            assert abs(p.sum() - 1) < 1e-13
            assert np.all(p[~vis] == 0)
            logits = x["k"][0, :, 0, :] @ x["q"][0, i, h, :]
            assert np.argmax(p) == np.flatnonzero(vis)[np.argmax(logits[vis])]


def pin_causal_diagonal(orc):
    """The query's own position is visible (t <= p): a key at t = p that matches
    the query takes (almost) all the weight; keys after p never do."""
    B, N, Hq, Hkv, d, Bk, K = 1, 16, 1, 1, 4, 4, 4
    prob = O.make_problem(B, N, N, Hq, Hkv, d, 2, Bk, K, 0, 1.0)
    q = np.zeros((B, N, Hq, d))
    q[..., 0] = 1.0
    k = np.zeros((B, N, Hkv, d))
    v = np.zeros((B, N, Hkv, d))
    v[0, :, 0, 1] = np.arange(N)
    ids = np.tile(np.arange(K, dtype=np.int32), (N, 1)).reshape(N, 1, K)
    for i in range(N):
        kk = k.copy()
        kk[0, i, 0, 0] = 800.0       # the diagonal key
        kk[0, i + 1:, 0, 0] = 1600.0  # future keys: must be invisible
        out, lse = orc.attend(prob, q, kk, v, ids[i:i + 1], rows=[[0, i]])
        assert out[0, 0, 1] == i, (i, out[0, 0])
        assert lse[0, 0] == 800.0


# ---- Backward of the attention step (chain rule through the softmax): checked
# against torch autograd of the masked-SDPA special case and against central
# finite differences of the oracle's own forward.

def _selection_mask(prob, ids):
    B, N, Hkv, K, Bk = prob.batch, prob.n_q, prob.h_kv, prob.topk, prob.block_size
    allowed = np.zeros((B, N, Hkv, prob.n_k), dtype=bool)
    idr = ids.reshape(B, N, Hkv, K)
    for b in range(B):
        for i in range(N):
            for g in range(Hkv):
                for j in idr[b, i, g]:
                    if j >= 0:
                        allowed[b, i, g, j * Bk:(j + 1) * Bk] = True
    return allowed & _causal_allowed(prob)


def pin_backward_equals_autograd(orc):
    """dq, dk, dv of L = sum(O * dout) equal torch autograd through fp64 SDPA
    with the selection as a boolean mask (GQA heads share k, v)."""
    rng = np.random.default_rng(23)
    B, N, Hq, Hkv, d, di, Bk, K = 2, 36, 4, 2, 8, 4, 4, 3
    prob = O.make_problem(B, N, N, Hq, Hkv, d, di, Bk, K, q_offset=0)
    x = _inputs(rng, B, N, N, Hq, Hkv, d, di)
    x["q"] *= 2.0  # sharper softmax
    dout = rng.standard_normal((B, N, Hq, d))
    ids, _, _, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    dq, dk, dv = orc.attend_backward(prob, x["q"], x["k"], x["v"], dout, ids)
    allowed = _selection_mask(prob, ids)
    G = Hq // Hkv
    qt = torch.tensor(x["q"], requires_grad=True)
    kt = torch.tensor(x["k"], requires_grad=True)
    vt = torch.tensor(x["v"], requires_grad=True)
    qh = qt.permute(0, 2, 1, 3)
    kh = kt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vh = vt.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    m = torch.from_numpy(allowed).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=m, scale=1.0 / math.sqrt(d))
    (o.permute(0, 2, 1, 3) * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-12)
    assert np.abs(dk).max() > 1e-3 and np.abs(dq).max() > 1e-3  # not trivially zero


def pin_backward_finite_differences(orc):
    """Central differences of L = sum(O * dout) through the oracle's forward
    (mo_attend) match the analytic gradients, including with q_offset > 0."""
    rng = np.random.default_rng(29)
    B, Nq, Nk, Hq, Hkv, d, di, Bk, K = 1, 6, 14, 2, 1, 4, 4, 4, 2
    prob = O.make_problem(B, Nq, Nk, Hq, Hkv, d, di, Bk, K, q_offset=Nk - Nq)
    x = _inputs(rng, B, Nq, Nk, Hq, Hkv, d, di)
    dout = rng.standard_normal((B, Nq, Hq, d))
    ids, _, _, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    dq, dk, dv = orc.attend_backward(prob, x["q"], x["k"], x["v"], dout, ids)

    def loss(q, k, v):
        o, _ = orc.attend(prob, q, k, v, ids)
        return float((o.reshape(dout.shape) * dout).sum())

    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for idx in [tuple(rng.integers(0, n) for n in grad.shape) for _ in range(12)]:
            xp = {k_: v_.copy() for k_, v_ in x.items()}
            xm = {k_: v_.copy() for k_, v_ in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd = (loss(xp["q"], xp["k"], xp["v"]) - loss(xm["q"], xm["k"], xm["v"])) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7, (name, idx, fd, grad[idx])


# ---- Index-Branch alignment loss (KL from the Main Branch's group-averaged
# distribution to the Index Branch's, on the selected tokens).

def _kl_torch(prob, x, ids, loss_scale):
    """Dense fp64 torch formulation: masked softmaxes, kl_div, autograd for the
    index inputs (the Main Branch distribution is a constant target)."""
    B, N, Hq, Hkv, d = prob.batch, prob.n_q, prob.h_q, prob.h_kv, prob.d
    G = Hq // Hkv
    allowed = torch.from_numpy(_selection_mask(prob, ids))                      # [B, Nq, Hkv, Nk]
    q = torch.from_numpy(x["q"]).reshape(B, N, Hkv, G, d)
    k = torch.from_numpy(x["k"])
    logits = torch.einsum("bigch,btgh->bigct", q, k) / math.sqrt(d)             # [B, Nq, Hkv, G, Nk]
    logits = logits.masked_fill(~allowed[:, :, :, None, :], float("-inf"))
    pm = torch.softmax(logits, dim=-1).mean(dim=3)                              # [B, Nq, Hkv, Nk]
    iq = torch.tensor(x["iq"], requires_grad=True)
    ik = torch.tensor(x["ik"], requires_grad=True)
    si = torch.einsum("bigc,btgc->bigt", iq, ik).masked_fill(~allowed, float("-inf"))
    logpi = torch.log_softmax(si, dim=-1)
    # kl_div(input=log q, target=p) = p (log p - log q) elementwise, 0 where p = 0
    kl = torch.nn.functional.kl_div(logpi.masked_fill(~allowed, 0.0), pm, reduction="none").sum(dim=-1)
    (loss_scale * kl.sum()).backward()
    return kl.detach().numpy(), iq.grad.numpy(), ik.grad.numpy()


def pin_kl_equals_autograd(orc):
    """KL per (row, group) and the gradients for the index queries and keys
    equal torch autograd of the dense masked formulation (G = 2, offset queries)."""
    rng = np.random.default_rng(37)
    B, Nq, Nk, Hq, Hkv, d, di, Bk, K = 2, 20, 30, 4, 2, 8, 6, 4, 3
    prob = O.make_problem(B, Nq, Nk, Hq, Hkv, d, di, Bk, K, q_offset=Nk - Nq)
    x = _inputs(rng, B, Nq, Nk, Hq, Hkv, d, di)
    x["q"] *= 2.0
    ids, _, _, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    kl, d_iq, d_ik = orc.indexer_kl(prob, x["q"], x["k"], x["iq"], x["ik"], ids, loss_scale=0.3)
    kl_t, giq, gik = _kl_torch(prob, x, ids, 0.3)
    np.testing.assert_allclose(kl, kl_t.reshape(B * Nq, Hkv), rtol=0, atol=1e-12)
    np.testing.assert_allclose(d_iq, giq.reshape(B * Nq, Hkv, di), rtol=0, atol=1e-12)
    np.testing.assert_allclose(d_ik, gik, rtol=0, atol=1e-12)
    assert kl.min() >= 0 and kl.max() > 1e-2 and np.abs(d_ik).max() > 1e-3


def pin_kl_vanishes_when_aligned(orc):
    """With the index scores equal to the Main Branch logits (G = 1,
    iq = scale * q, ik = k) the two distributions coincide: KL and its
    gradients vanish.  Perturbing iq makes KL strictly positive."""
    rng = np.random.default_rng(41)
    B, N, H, d, Bk, K = 1, 16, 2, 4, 4, 2
    prob = O.make_problem(B, N, N, H, H, d, d, Bk, K)
    x = _inputs(rng, B, N, N, H, H, d, d)
    x["iq"] = x["q"] / math.sqrt(d)
    x["ik"] = x["k"].copy()
    ids, _, _, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    kl, d_iq, d_ik = orc.indexer_kl(prob, x["q"], x["k"], x["iq"], x["ik"], ids)
    assert np.abs(kl).max() < 1e-13 and np.abs(d_iq).max() < 1e-13 and np.abs(d_ik).max() < 1e-13
    x["iq"] = x["iq"] * 1.5
    kl2, _, _ = orc.indexer_kl(prob, x["q"], x["k"], x["iq"], x["ik"], ids)
    rows_with_choice = [r for r in range(N) if r >= 1]  # more than one visible token
    assert kl2.reshape(N, H)[rows_with_choice].min() > 0


def pin_kl_finite_differences(orc):
    """Central differences of loss_scale * sum(kl) in the index inputs match the
    analytic gradients (G = 4: the group average matters)."""
    rng = np.random.default_rng(43)
    B, Nq, Nk, Hq, Hkv, d, di, Bk, K = 1, 7, 13, 4, 1, 4, 3, 4, 2
    prob = O.make_problem(B, Nq, Nk, Hq, Hkv, d, di, Bk, K, q_offset=Nk - Nq)
    x = _inputs(rng, B, Nq, Nk, Hq, Hkv, d, di)
    ids, _, _, _ = orc.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    _, d_iq, d_ik = orc.indexer_kl(prob, x["q"], x["k"], x["iq"], x["ik"], ids, loss_scale=2.0)

    def loss(iq, ik):
        kl, _, _ = orc.indexer_kl(prob, x["q"], x["k"], iq, ik, ids)
        return 2.0 * float(kl.sum())

    eps = 1e-6
    for name, grad in (("iq", d_iq.reshape(x["iq"].shape)), ("ik", d_ik)):
        for idx in [tuple(rng.integers(0, n) for n in grad.shape) for _ in range(10)]:
            xp = {k_: v_.copy() for k_, v_ in x.items()}
            xm = {k_: v_.copy() for k_, v_ in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd = (loss(xp["iq"], xp["ik"]) - loss(xm["iq"], xm["ik"])) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7, (name, idx, fd, grad[idx])


# ---- MXFP8 index-key caches (OCP Microscaling Formats v1.0; OCP 8-bit floating
# point E4M3).  torch's float8_e4m3fn is an independent implementation of the
# element format; the shared-exponent rule and the saturation are the MX
# spec's and are checked on hand-computed blocks.

def _torch_e4m3_codes(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_decode_table(orc):
    """Every code decodes as torch's float8_e4m3fn does; published anchors."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])
    anchors = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0xC0: -2.0, 0x00: 0.0}
    for c, v in anchors.items():
        assert got[c] == v, (hex(c), got[c])


def pin_e4m3_encode_rne(orc):
    """Nearest code, ties to the even code: equal to torch's conversion on every
    representable value, every midpoint between neighbours (the ties), and
    random values; magnitudes above 448 saturate (the MX conversion)."""
    vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()  # 0 .. 448
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(11)
    rand = rng.uniform(0, 448, 2000)
    tiny = rng.uniform(0, 2.0 ** -6, 500)
    ys = np.concatenate([vals, mids, rand, tiny, [2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -10 * 1.0001]])
    ys = np.concatenate([ys, -ys])
    got = np.array([orc.e4m3_encode(y) for y in ys], dtype=np.uint8)
    assert np.array_equal(got, _torch_e4m3_codes(ys))
    for y in (448.5, 464.0, 480.0, 1e6, 1e300):
        assert orc.e4m3_encode(y) == 0x7E and orc.e4m3_encode(-y) == 0xFE, y
    assert orc.e4m3_encode(-0.0) == 0x80


def pin_mx_shared_exponent(orc):
    """Hand-computed blocks: scale = floor(log2 max|v|) - 8 (+127 bias), clamped;
    elements = E4M3(v / 2^scale), the block maximum saturating when its scaled
    value passes 448."""
    def q(block):
        c, sc = orc.mx_quantize(np.asarray(block, dtype=np.float64).reshape(1, 32))
        return c[0], int(sc[0, 0])
    c, sc = q(np.ones(32))                       # 1 = 2^0 -> X = 2^-8, 1/X = 256 = 2^8
    assert sc == 119 and np.all(c == 0x78)
    blk = np.zeros(32); blk[3] = 56.0; blk[4] = -7.0  # log2 56 = 5.8 -> X = 2^-3: 448 and -56 = -1.75 * 2^5
    c, sc = q(blk)
    assert sc == 124 and c[3] == 0x7E and c[4] == 0xE6 and np.all(np.delete(c, [3, 4]) == 0)
    blk = np.full(32, 1.9)                      # X = 2^-8: 1.9 * 256 = 486.4 saturates to 448
    c, sc = q(blk)
    assert sc == 119 and np.all(c == 0x7E)
    c, sc = q(np.zeros(32))                      # all zero: smallest scale, zero codes
    assert sc == 0 and np.all(c == 0)
    c, sc = q(np.full(32, 2.0 ** -130))          # exponent clamped at -127: 2^-130 * 2^127 = 2^-3
    assert sc == 0 and np.all(c == 0x20)
    c, sc = q(np.full(32, 2.0 ** 200))           # exponent clamped at 127: saturates
    assert sc == 254 and np.all(c == 0x7E)
    # two blocks per row are independent
    row = np.concatenate([np.full(32, 0.5), np.full(32, 8.0)]).reshape(1, 64)
    c, sc = orc.mx_quantize(row)
    assert list(sc[0]) == [127 - 9, 127 - 5] and np.all(c == 0x78)


def pin_mx_roundtrip(orc):
    """Dequantised values are the block scale times a code value, exactly, and
    agree with torch's element conversion of v / X for every element below the
    saturation point."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    c, sc = orc.mx_quantize(x)
    d = orc.mx_dequantize(c, sc)
    X = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=1)
    y = x / X
    ok = np.abs(y) <= 448
    ref = torch.from_numpy(y[ok]).to(torch.float8_e4m3fn).double().numpy() * X[ok]
    assert np.array_equal(d[ok], ref)
    assert np.all(np.abs(d[~ok]) == 448 * X[~ok])
    assert (~ok).sum() > 0  # the saturating case does occur on Gaussian blocks


PINS = [pin_golden_worked_example, pin_maxpool_closed_form, pin_scores_ignore_future_and_token_order,
        pin_topk_bruteforce, pin_topk_special_cases, pin_exp_free, pin_dense_equals_sdpa,
        pin_sparse_equals_masked_sdpa, pin_value_invariants, pin_causal_diagonal,
        pin_e4m3_decode_table, pin_e4m3_encode_rne, pin_mx_shared_exponent, pin_mx_roundtrip,
        pin_backward_equals_autograd, pin_backward_finite_differences, pin_kl_equals_autograd,
        pin_kl_vanishes_when_aligned, pin_kl_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(O.default())


def test_row_subsets_match_full():
    """Evaluating a list of (b, i) rows gives the same values as the full run."""
    rng = np.random.default_rng(23)
    B, N, Hq, Hkv, d, di, Bk, K = 2, 24, 4, 2, 8, 4, 4, 3
    prob = O.make_problem(B, N, N, Hq, Hkv, d, di, Bk, K)
    x = _inputs(rng, B, N, N, Hq, Hkv, d, di)
    ids, out, lse, s = O.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    rows = [[1, 5], [0, 23], [1, 0]]
    ids2, out2, lse2, s2 = O.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"], rows=rows)
    flat = [b * N + i for b, i in rows]
    assert np.array_equal(ids[flat], ids2)
    assert np.array_equal(out[flat], out2) and np.array_equal(lse[flat], lse2)
    assert np.array_equal(s[flat], s2)


def test_backward_row_subsets():
    """The backward over a list of rows: dq equals the full run's rows, and
    dk, dv equal the full gradients of the loss restricted to those rows
    (dout zeroed elsewhere, so every other row contributes exact zeros)."""
    rng = np.random.default_rng(31)
    B, N, Hq, Hkv, d, di, Bk, K = 2, 24, 4, 2, 8, 4, 4, 3
    prob = O.make_problem(B, N, N, Hq, Hkv, d, di, Bk, K)
    x = _inputs(rng, B, N, N, Hq, Hkv, d, di)
    dout = rng.standard_normal((B, N, Hq, d))
    ids, _, _, _ = O.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    dq, dk, dv = O.attend_backward(prob, x["q"], x["k"], x["v"], dout, ids)
    rows = [[0, 3], [0, 17], [1, 0], [1, 22]]  # ascending (b, i): the full run's order
    flat = [b * N + i for b, i in rows]
    dq2, dk2, dv2 = O.attend_backward(prob, x["q"], x["k"], x["v"], dout, ids[flat], rows=rows)
    assert np.array_equal(dq.reshape(B * N, Hq, d)[flat], dq2)
    masked = np.zeros_like(dout)
    for b, i in rows:
        masked[b, i] = dout[b, i]
    _, dk3, dv3 = O.attend_backward(prob, x["q"], x["k"], x["v"], masked, ids)
    assert np.array_equal(dk2, dk3) and np.array_equal(dv2, dv3)
    assert np.abs(dk2).max() > 0 and not np.array_equal(dk2, dk)


def test_bf16_and_f32_inputs_widen_exactly():
    rng = np.random.default_rng(29)
    B, N, Hq, Hkv, d, di, Bk, K = 1, 16, 2, 1, 8, 8, 4, 2
    prob = O.make_problem(B, N, N, Hq, Hkv, d, di, Bk, K)
    x = {n: torch.from_numpy(a).to(torch.bfloat16) for n, a in _inputs(rng, B, N, N, Hq, Hkv, d, di).items()}
    r_bf = O.forward(prob, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    x64 = {n: t.to(torch.float64).numpy() for n, t in x.items()}
    r_64 = O.forward(prob, x64["q"], x64["k"], x64["v"], x64["iq"], x64["ik"])
    x32 = {n: t.to(torch.float32) for n, t in x.items()}
    r_32 = O.forward(prob, x32["q"], x32["k"], x32["v"], x32["iq"], x32["ik"])
    for a, b, c in zip(r_bf, r_64, r_32):
        assert np.array_equal(a, b) and np.array_equal(a, c)


def test_invert_matches_definition():
    """Block -> query lists: for every block, exactly the (query, slot) picks of
    that block, ascending; brute force over every (block, query, slot)."""
    rng = np.random.default_rng(31)
    B, N, Hkv, K, Bk = 2, 40, 3, 4, 4
    prob = O.make_problem(B, N, N, Hkv, Hkv, 2, 2, Bk, K)
    nb = N // Bk
    ids = rng.integers(-1, nb, size=(B, N, Hkv, K)).astype(np.int32)
    for b in range(B):  # a query never picks a block twice
        for i in range(N):
            for g in range(Hkv):
                row = rng.choice(nb, size=K, replace=False)
                row[rng.random(K) < 0.2] = -1
                ids[b, i, g] = row
    off, ent = O.invert(prob, ids)
    for b in range(B):
        for g in range(Hkv):
            assert off[b, g, 0] == 0 and off[b, g, -1] == int((ids[b, :, g] >= 0).sum())
            for j in range(nb):
                want = [i * K + s for i in range(N) for s in range(K) if ids[b, i, g, s] == j]
                assert list(ent[b, g, off[b, g, j]:off[b, g, j + 1]]) == want


def test_invalid_arguments_rejected():
    prob = O.make_problem(1, 8, 4, 2, 1, 2, 2, 2, 2)  # n_q > n_k
    with pytest.raises(ValueError):
        O.block_scores(prob, np.zeros((1, 8, 1, 2)), np.zeros((1, 4, 1, 2)))
    prob = O.make_problem(1, 4, 4, 3, 2, 2, 2, 2, 2)  # h_q not a multiple of h_kv
    with pytest.raises(ValueError):
        O.block_scores(prob, np.zeros((1, 4, 2, 2)), np.zeros((1, 4, 2, 2)))


# Plausible mistakes, planted by text substitution into a copy of the oracle.
MUTANTS = {
    "drops_diagonal_token": ("if (t <= pos && t < p->n_k) tok[n++] = t;", "if (t < pos && t < p->n_k) tok[n++] = t;"),
    "forgets_local_block": ("chosen[n++] = (int32_t)L; /* the local block is always kept */", ""),
    "ties_to_highest_id": ("return (x->j > y->j) - (x->j < y->j);", "return (x->j < y->j) - (x->j > y->j);"),
    "sum_pooling": ("if (s > best) best = s;", "best = (best == -INFINITY ? 0.0 : best) + s;"),
    "min_pooling": ("if (s > best) best = s;", "if (s < best || best == -INFINITY) best = s;"),
    "scale_one_over_d": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "strided_group_map": ("return h / (p->h_q / p->h_kv);", "return h % p->h_kv;"),
    "k_excludes_local": ("for (int64_t m = 0; m < K - 1; ++m) chosen[n++] = cand[m].j;",
                         "for (int64_t m = 0; m < K && m < L; ++m) chosen[n++] = cand[m].j;"),
    "values_from_keys": ("o[c] += x[a] * widen(v, dtype, vbase + c);", "o[c] += x[a] * widen(k, dtype, vbase + c);"),
    # (Dropping the visibility test inside the max pool is not a mistake one can
    # catch: candidate blocks lie wholly before the query, so it never fires.)
    "scores_include_local_block": ("for (int64_t j = 0; j < L; ++j) {\n      double best",
                                   "for (int64_t j = 0; j <= L && j < nblk; ++j) {\n      double best"),
    "bwd_drops_rowsum": ("const double ds = x[a] * (dp - dot_do_o);", "const double ds = x[a] * dp;"),
    "bwd_dk_unscaled": ("dk[kvbase + c] += scale * ds * widen(q, dtype, qbase + c);",
                        "dk[kvbase + c] += ds * widen(q, dtype, qbase + c);"),
    "bwd_dv_from_scores": ("dv[kvbase + c] += x[a] * widen(dout, dtype, qbase + c);",
                           "dv[kvbase + c] += ds * widen(dout, dtype, qbase + c);"),
    "bwd_dq_from_values": ("dqr[c] += scale * ds * widen(k, dtype, kvbase + c);",
                           "dqr[c] += scale * ds * widen(v, dtype, kvbase + c);"),
    "kl_no_group_average": ("pm[a] += x[a] / (double)G;", "pm[a] += x[a];"),
    "kl_reversed_gradient": ("const double gs = loss_scale * (exp(logpi) - pm[a]);",
                             "const double gs = loss_scale * (pm[a] - exp(logpi));"),
    "kl_drops_target_entropy": ("if (pm[a] > 0.0) acc += pm[a] * (log(pm[a]) - logpi);",
                                "if (pm[a] > 0.0) acc += -pm[a] * logpi;"),
    "kl_unnormalised_index": ("const double logpi = si[a] - lse;", "const double logpi = si[a] - m;"),
    "kl_dik_from_keys": ("d_ik[ki + c] += gs * widen(iq, dtype, qi + c);", "d_ik[ki + c] += gs * widen(ik, dtype, ki + c);"),
    "mx_truncates": ("double q = nearbyint(ldexp(a, 3 - e));", "double q = floor(ldexp(a, 3 - e));"),
    "mx_ties_away": ("const double m = nearbyint(ldexp(a, 9));", "const double m = round(ldexp(a, 9));"),
    "mx_emax_7": ("e = (ex - 1) - 8;", "e = (ex - 1) - 7;"),
    "mx_no_saturation": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 480.0) return sign | 0x7F;"),
    "mx_scale_not_clamped": ("if (e < -127) e = -127;", ""),
    "mx_exponent_sign": ("out[i] = ldexp(mo_e4m3_value(codes[i]), (int)scales[i / 32] - 127);",
                         "out[i] = ldexp(mo_e4m3_value(codes[i]), 127 - (int)scales[i / 32]);"),
}


def test_planted_mistakes_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(obuild.__file__), "msa_oracle.c")).read()
    hdr = os.path.join(os.path.dirname(obuild.__file__), "msa_oracle.h")
    survivors = []
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutant {name}: anchor text not found exactly once"
        d = tmp_path / name
        d.mkdir()
        shutil.copy(hdr, d / "msa_oracle.h")
        (d / "msa_oracle.c").write_text(src.replace(old, new))
        so = str(d / "libm.so")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-o", so,
                        str(d / "msa_oracle.c"), "-lm"], check=True, capture_output=True)
        orc = O.Oracle(so)
        failed = []
        for pin in PINS:
            try:
                pin(orc)
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
        if not failed:
            survivors.append(name)
    assert not survivors, f"mutants not caught by any pin: {survivors}"
