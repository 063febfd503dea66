"""Comparison helpers shared by the GPU parity tests (HIP path vs the oracle).

Criteria (fixed before any kernel existed):
  * selection: bit-exact per (query, group) row, except rows whose difference
    lies inside the tie band -- both sets hold the local block, both have
    min(k, L+1) entries, and every block in one set but not the other scores
    within 1e-3 relative (oracle fp64 scores) of every block in the reverse
    difference.  Such rows are counted; failing rows must be zero.
  * attention (computed from the oracle's selection): bf16 max-abs <= 2e-2
    and rel-L2 <= 5e-3; fp32 max-abs <= 1e-4 and rel-L2 <= 1e-4.
  * attention, row by row (so that a few wrong rows cannot hide in the
    global figures): the rel-L2 of every (query, head) output row must stay
    within 1e-2 for bf16 -- the output is rounded to bf16 (2^-9 relative),
    the KV-outer partials are bf16 (another 2^-9) and P enters the PV product
    in bf16 (2^-9 per weight) -- and within 1e-4 for fp32; a row whose oracle
    output is exactly zero (no visible selected token) must be exactly zero.
"""
import numpy as np
import torch

TIE_REL = 1e-3
TOL = {"bf16": dict(max_abs=2e-2, rel_l2=5e-3, lse_abs=2e-2, row_rel_l2=1e-2),
       "f32": dict(max_abs=1e-4, rel_l2=1e-4, lse_abs=1e-4, row_rel_l2=1e-4)}


def host(t):
    return t.detach().cpu()


def positions(wl):
    return wl.q_offset + np.arange(wl.n_q)


def check_selection(wl, ids_gpu, ids_ora, s_ora, rows=None):
    """ids_*: [n_rows, h_kv, k] int; s_ora: [n_rows, h_kv, nblk] fp64.
    Returns dict(exact, tie, fail, fail_examples)."""
    ids_gpu = np.asarray(ids_gpu)
    ids_ora = np.asarray(ids_ora)
    if rows is None:
        qi = np.tile(np.arange(wl.n_q), wl.batch)
    else:
        qi = np.asarray(rows)[:, 1]
    L = (wl.q_offset + qi) // wl.block_size
    exact = tie = fail = 0
    examples = []
    same = np.all(ids_gpu == ids_ora, axis=2)
    for r, g in zip(*np.nonzero(~same)):
        a = set(int(x) for x in ids_gpu[r, g] if x >= 0)
        b = set(int(x) for x in ids_ora[r, g] if x >= 0)
        need = min(wl.topk, int(L[r]) + 1)
        ok = int(L[r]) in a and int(L[r]) in b and len(a) == need and len(b) == need
        ok = ok and list(ids_gpu[r, g]) == sorted(a) + [-1] * (wl.topk - len(a))
        if ok:
            S = s_ora[r, g]
            for x in a - b:
                for y in b - a:
                    if not abs(S[x] - S[y]) < TIE_REL * max(abs(S[x]), abs(S[y])):
                        ok = False
        if ok:
            tie += 1
        else:
            fail += 1
            if len(examples) < 5:
                examples.append((int(r), int(g), sorted(a), sorted(b)))
    exact = int(same.sum())
    return dict(exact=exact, tie=tie, fail=fail, fail_examples=examples)


def attention_errors(out_gpu, out_ora):
    """(max-abs, rel-L2) in fp64."""
    a = np.asarray(out_gpu, dtype=np.float64)
    b = np.asarray(out_ora, dtype=np.float64)
    diff = a - b
    return float(np.max(np.abs(diff))), float(np.linalg.norm(diff) / max(np.linalg.norm(b), 1e-300))


def worst_row(out_gpu, out_ora):
    """Largest rel-L2 over the output rows (the last axis is d) and its row
    index; rows whose oracle output is zero count as 0 if the GPU's is zero
    too and as inf otherwise."""
    a = np.asarray(out_gpu, dtype=np.float64)
    b = np.asarray(out_ora, dtype=np.float64)
    a = a.reshape(-1, a.shape[-1])
    b = b.reshape(-1, b.shape[-1])
    nb = np.linalg.norm(b, axis=1)
    nd = np.linalg.norm(a - b, axis=1)
    rel = np.where(nb > 0, nd / np.where(nb > 0, nb, 1.0), np.where(nd == 0, 0.0, np.inf))
    r = int(np.argmax(rel)) if rel.size else 0
    return (float(rel[r]) if rel.size else 0.0), r


def assert_lse(dtype, lse_gpu, lse_ora, what=""):
    """lse within the tolerance where the oracle's is finite; -inf exactly
    where it is -inf (rows with no visible selected token)."""
    a = np.asarray(lse_gpu, dtype=np.float64)
    b = np.asarray(lse_ora, dtype=np.float64)
    fin = np.isfinite(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b)) and np.all(np.isfinite(a[fin])), f"{what}: lse -inf pattern"
    d = float(np.max(np.abs(a[fin] - b[fin]))) if fin.any() else 0.0
    assert d <= TOL[dtype]["lse_abs"], f"{what}: lse max-abs {d:.3e}"


def assert_attention(dtype, out_gpu, out_ora, lse_gpu=None, lse_ora=None, what=""):
    tol = TOL[dtype]
    mx, rl = attention_errors(out_gpu, out_ora)
    assert mx <= tol["max_abs"] and rl <= tol["rel_l2"], f"{what}: max-abs {mx:.3e} rel-L2 {rl:.3e} ({dtype})"
    wr, r = worst_row(out_gpu, out_ora)
    assert wr <= tol["row_rel_l2"], f"{what}: worst row {r} rel-L2 {wr:.3e} ({dtype})"
    if lse_gpu is not None:
        assert_lse(dtype, lse_gpu, lse_ora, what)
    print(f"{what}: worst row rel-L2 {wr:.2e}")
    return mx, rl


def to_f64(t):
    return host(t).to(torch.float64).numpy()
