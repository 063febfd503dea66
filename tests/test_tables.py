"""Block id tables given by a caller, on the CPU: the oracle's result for every
int32 table, pinned to library routines, and a model of the GPU inversion's
placement rule checked against the oracle's inversion.

Reading (the pages define selections the Index Branch makes, which never
repeat a block; for a caller's table the plainest reading of "attention over
the tokens of the listed blocks", paper summary page "Method", is):
  * ids outside [0, nblk) list nothing;
  * a block listed twice puts its visible tokens into the softmax twice;
  * tokens past the query position stay invisible;
  * a row with no visible listed token has out = 0 and lse = -inf (an empty
    sum), zero gradients and a zero indexer loss.
Block scores handed to the Top-k may be non-finite: -inf and NaN rank below
every finite score (NaN as -inf), ties to the lower id.

Pins: torch's scaled_dot_product_attention (fp64) over keys gathered with the
repeats written out; torch autograd through that gather for the gradients and
the KL loss; Python's sort for the non-finite Top-k.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import build as obuild
from oracle import oracle as O

INT32_MIN, INT32_MAX = -(2 ** 31), 2 ** 31 - 1


def _problem(**kw):
    p = dict(batch=2, n_q=12, n_k=40, h_q=4, h_kv=2, d=8, d_idx=4, block_size=4, topk=5, q_offset=28)
    p.update(kw)
    return O.make_problem(**p)


def _inputs(prob, seed):
    rng = np.random.default_rng(seed)
    B, Nq, Nk, Hq, Hkv, d, di = prob.batch, prob.n_q, prob.n_k, prob.h_q, prob.h_kv, prob.d, prob.d_idx
    return dict(q=rng.standard_normal((B, Nq, Hq, d)), k=rng.standard_normal((B, Nk, Hkv, d)),
                v=rng.standard_normal((B, Nk, Hkv, d)), iq=rng.standard_normal((B, Nq, Hkv, di)),
                ik=rng.standard_normal((B, Nk, Hkv, di)))


def _messy_table(prob, seed):
    """Rows mixing repeats, -1, other negatives, ids >= nblk, blocks past the
    query and rows that select nothing visible."""
    rng = np.random.default_rng(seed)
    nb = O.nblk(prob)
    pool = np.array([-1, -7, INT32_MIN, nb, nb + 3, 10 ** 6, INT32_MAX], dtype=np.int64)
    ids = rng.integers(0, nb, size=(prob.batch, prob.n_q, prob.h_kv, prob.topk)).astype(np.int64)
    bad = rng.random(ids.shape) < 0.3
    ids[bad] = rng.choice(pool, size=int(bad.sum()))
    ids[0, 0, 0, :] = 2                         # one block, five times
    ids[0, 1, 0, :] = [3, -1, 3, 9, 3]          # repeats, and block 9 (past the query: L = 7 here)
    ids[0, 2, 1, :] = -1                        # nothing listed
    ids[1, 3, 0, :] = [nb - 1, nb, -5, nb - 1, INT32_MAX]  # the last block (past every query here) and junk
    ids[1, 4, 1, :] = [0, 1, 0, 1, 0]           # repeats only
    return ids.astype(np.int32)


def _rows(prob, ids):
    """[B, Nq, Hkv, k] -> the oracle's [rows, Hkv, k]."""
    return np.ascontiguousarray(ids.reshape(-1, prob.h_kv, prob.topk))


def _tokens(prob, sel, pos):
    nb, Bk = O.nblk(prob), prob.block_size
    return [t for j in sel if 0 <= j < nb for t in range(j * Bk, (j + 1) * Bk) if t <= pos and t < prob.n_k]


def _scale(prob):
    return prob.softmax_scale if prob.softmax_scale > 0 else 1.0 / math.sqrt(prob.d)


def pin_attend_follows_sdpa_over_repeated_keys(orc):
    """Every row: SDPA over K/V rows gathered with the listing's repeats."""
    prob = _problem()
    x = _inputs(prob, 1)
    ids = _messy_table(prob, 2)
    out, lse = orc.attend(prob, x["q"], x["k"], x["v"], _rows(prob, ids))
    G = prob.h_q // prob.h_kv
    empty = 0
    for b in range(prob.batch):
        for i in range(prob.n_q):
            pos = prob.q_offset + i
            for h in range(prob.h_q):
                g = h // G
                r = b * prob.n_q + i
                T = _tokens(prob, ids[b, i, g], pos)
                if not T:
                    empty += 1
                    assert np.all(out[r, h] == 0.0) and lse[r, h] == -np.inf
                    continue
                q = torch.from_numpy(x["q"][b, i, h]).view(1, 1, 1, -1)
                kk = torch.from_numpy(x["k"][b, T, g]).view(1, 1, len(T), -1)
                vv = torch.from_numpy(x["v"][b, T, g]).view(1, 1, len(T), -1)
                o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=_scale(prob))
                ref_lse = torch.logsumexp((kk[0, 0] @ q[0, 0, 0]) * _scale(prob), dim=0)
                np.testing.assert_allclose(out[r, h], o.view(-1).numpy(), rtol=0, atol=1e-12)
                assert abs(lse[r, h] - float(ref_lse)) < 1e-12
    assert empty > 0  # the table has rows with nothing visible


def pin_repeating_every_listing_keeps_output_and_adds_ln2(orc):
    prob = _problem(topk=8)
    x = _inputs(prob, 3)
    rng = np.random.default_rng(4)
    L = (prob.q_offset + np.arange(prob.n_q)) // prob.block_size
    once = np.full((prob.batch, prob.n_q, prob.h_kv, 8), -1, dtype=np.int32)
    for i in range(prob.n_q):
        for b in range(prob.batch):
            for g in range(prob.h_kv):
                sel = rng.choice(L[i] + 1, size=4, replace=False)
                once[b, i, g, :4] = np.sort(sel)
    twice = once.copy()
    twice[..., 4:] = once[..., :4]
    o1, l1 = orc.attend(prob, x["q"], x["k"], x["v"], _rows(prob, once))
    o2, l2 = orc.attend(prob, x["q"], x["k"], x["v"], _rows(prob, twice))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, math.log(2.0), rtol=0, atol=1e-12)


def pin_backward_and_kl_follow_autograd_over_repeated_keys(orc):
    """Gradients of the attention and the indexer loss for a messy table:
    torch autograd through index gathers (repeated tokens get summed
    gradients), the Main Branch target detached."""
    prob = _problem(batch=1, n_q=9, q_offset=31)
    x = _inputs(prob, 5)
    ids = np.ascontiguousarray(_messy_table(_problem(), 6)[:1, :9])  # same n_k, so the same blocks
    rng = np.random.default_rng(7)
    dout = rng.standard_normal(x["q"].shape)
    dq, dk, dv = orc.attend_backward(prob, x["q"], x["k"], x["v"], dout, _rows(prob, ids))
    kl, diq, dik = orc.indexer_kl(prob, x["q"], x["k"], x["iq"], x["ik"], _rows(prob, ids), loss_scale=0.5)

    q, k, v = (torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v"))
    iq, ik = (torch.tensor(x[n], requires_grad=True) for n in ("iq", "ik"))
    G = prob.h_q // prob.h_kv
    loss_attn = torch.zeros((), dtype=torch.float64)
    loss_kl = torch.zeros((), dtype=torch.float64)
    kl_ref = np.zeros((prob.n_q, prob.h_kv))
    for i in range(prob.n_q):
        pos = prob.q_offset + i
        for g in range(prob.h_kv):
            T = _tokens(prob, ids[0, i, g], pos)
            if not T:
                continue
            Ti = torch.tensor(T)
            pm = 0
            for h in range(g * G, (g + 1) * G):
                logits = (k[0, Ti, g] @ q[0, i, h]) * _scale(prob)
                p = torch.softmax(logits, dim=0)
                loss_attn = loss_attn + (torch.from_numpy(dout[0, i, h]) * (p @ v[0, Ti, g])).sum()
                pm = pm + p.detach() / G
            logpi = torch.log_softmax(ik[0, Ti, g] @ iq[0, i, g], dim=0)
            kl_row = (pm * (torch.log(pm) - logpi)).sum()
            kl_ref[i, g] = float(kl_row.detach())
            loss_kl = loss_kl + 0.5 * kl_row
    loss_attn.backward()
    loss_kl.backward()
    np.testing.assert_allclose(dq.reshape(q.shape), q.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk.reshape(k.shape), k.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv.reshape(v.shape), v.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(kl.reshape(kl_ref.shape), kl_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(diq.reshape(iq.shape), iq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dik.reshape(ik.shape), ik.grad.numpy(), rtol=0, atol=1e-11)


def _select_by_sort(prob, S, i):
    """Selection of one row by Python's sort: key (finite first, score desc, id asc)."""
    L = (prob.q_offset + i) // prob.block_size
    cand = list(range(L))
    key = lambda j: (0, -S[j], j) if np.isfinite(S[j]) or S[j] == np.inf else (1, 0.0, j)
    picked = sorted(cand, key=key)[:prob.topk - 1]
    row = sorted(picked + [L])
    return row + [-1] * (prob.topk - len(row))


def pin_select_with_nonfinite_scores(orc):
    for seed in range(6):
        _select_nonfinite_case(orc, seed)


def _select_nonfinite_case(orc, seed):
    prob = _problem(batch=1, n_q=20, n_k=80, block_size=4, topk=6, q_offset=60, h_kv=2)
    rng = np.random.default_rng(100 + seed)
    nb = O.nblk(prob)
    S = rng.integers(-2, 3, size=(prob.n_q, prob.h_kv, nb)).astype(np.float64)
    kind = rng.random(S.shape)
    S[kind < 0.35] = -np.inf
    S[(kind >= 0.35) & (kind < 0.6)] = np.nan
    S[0, 0, :] = np.nan            # nothing finite
    S[1, 1, :] = -np.inf
    S[2, 0, :3] = 5.0              # fewer finite scores than picks
    S[2, 0, 3:] = np.nan
    ids = orc.select(prob, S)
    for i in range(prob.n_q):
        for g in range(prob.h_kv):
            assert list(ids[i, g]) == _select_by_sort(prob, S[i, g], i), (i, g)


PINS = [pin_attend_follows_sdpa_over_repeated_keys, pin_repeating_every_listing_keeps_output_and_adds_ln2,
        pin_backward_and_kl_follow_autograd_over_repeated_keys, pin_select_with_nonfinite_scores]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_table_pin(pin):
    pin(O.default())


# One plausible mistake each in the oracle's handling of caller tables; every
# one must fail at least one pin above.
MUTANTS = {
    "repeats_collapsed": ("    if (j < 0 || j >= nblk) continue;\n    for (int64_t t = j * Bk;",
                          "    if (j < 0 || j >= nblk) continue;\n    { int seen = 0; for (int64_t u = 0; u < s; ++u)"
                          " seen |= sel[u] == j; if (seen) continue; }\n    for (int64_t t = j * Bk;"),
    "empty_row_divides": ("  if (n == 0) { /* no visible selected token: zero output, empty sum */",
                          "  if (0) { /* no visible selected token: zero output, empty sum */"),
    "nan_ranks_high": ("cand[j].s = isnan(S[j]) ? -INFINITY : S[j];", "cand[j].s = isnan(S[j]) ? INFINITY : S[j];"),
}


def test_planted_table_mistakes_are_caught(tmp_path):
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


# ---- the GPU inversion's placement rule, modelled on the CPU ---------------

TILE = 256  # queries per histogram / scatter tile


def _model_invert(prob, ids):
    """Model of the inversion kernels: per-tile counts, column and block scans,
    then a walk over each tile's queries in which the slots of one query (the
    lanes of one step) rank themselves among the lower slots naming the same
    block, and the last of them advances that block's cursor.  (The kernel
    takes a single-pass step for rows whose valid ids ascend strictly; there
    every rank is 0 and every count 1, so the rule below covers it.)"""
    nb, K, Nq = O.nblk(prob), prob.topk, prob.n_q
    ntile = (Nq + TILE - 1) // TILE
    offsets = np.zeros((prob.batch, prob.h_kv, nb + 1), dtype=np.int64)
    entries = np.full((prob.batch, prob.h_kv, Nq * K), -1, dtype=np.int64)
    for b in range(prob.batch):
        for g in range(prob.h_kv):
            hist = np.zeros((ntile, nb), dtype=np.int64)
            for t in range(ntile):
                for i in range(t * TILE, min(Nq, (t + 1) * TILE)):
                    for j in ids[b, i, g]:
                        if 0 <= j < nb:
                            hist[t, j] += 1
            pre = np.cumsum(hist, axis=0) - hist        # column scan (exclusive, over tiles)
            tot = hist.sum(axis=0)
            off = np.concatenate([[0], np.cumsum(tot)])  # block scan
            offsets[b, g] = off
            for t in range(ntile):
                cur = off[:nb] + pre[t]
                for i in range(t * TILE, min(Nq, (t + 1) * TILE)):
                    row = ids[b, i, g]
                    base = {}
                    writes = []
                    for lane in range(K):
                        j = int(row[lane])
                        if not 0 <= j < nb:
                            continue
                        rank = sum(1 for s in range(lane) if row[s] == j)
                        cnt = sum(1 for s in range(K) if row[s] == j)
                        base.setdefault(j, cur[j])            # every lane reads before any writes
                        writes.append((j, base[j] + rank, i * K + lane, rank == cnt - 1, cnt))
                    for j, pos, e, last, cnt in writes:
                        assert entries[b, g, pos] == -1, "two writers for one entry"
                        entries[b, g, pos] = e
                        if last:
                            cur[j] = base[j] + cnt
    return offsets, entries


@pytest.mark.parametrize("n_q,topk,seed", [(30, 5, 0), (300, 7, 1), (520, 16, 2), (257, 32, 3)])
def test_scatter_placement_matches_oracle_inversion(n_q, topk, seed):
    prob = _problem(batch=2, n_q=n_q, n_k=max(n_q, 200), block_size=8, topk=topk, q_offset=0, h_kv=2)
    nb = O.nblk(prob)
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, min(nb, 6), size=(2, n_q, 2, topk)).astype(np.int64)  # few blocks: many repeats
    bad = rng.random(ids.shape) < 0.2
    ids[bad] = rng.choice([-1, -3, nb, nb + 100, INT32_MAX, INT32_MIN], size=int(bad.sum()))
    ids = ids.astype(np.int32)
    off_m, ent_m = _model_invert(prob, ids)
    off_o, ent_o = O.invert(prob, ids)
    assert np.array_equal(off_m, off_o)
    for b in range(2):
        for g in range(2):
            n = off_o[b, g, -1]
            assert np.array_equal(ent_m[b, g, :n], ent_o[b, g, :n])
            assert np.all(ent_m[b, g, n:] == -1)
