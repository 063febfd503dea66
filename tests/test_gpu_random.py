"""GPU parity on seeded random problems: msa_forward through the C ABI against
the fp64 oracle, every row of every case.

Each case draws, from its own seed, one point of the supported space: key
block size 32/64/128, dtype bf16/fp32, d 64/128, d_idx 32/64/128, 1-4 groups
of 1-32 query heads, k from 1 to 32 (so every Top-k list size the index
kernels are built for), up to 40 key blocks with a ragged end, a query chunk
at a random offset, batch 1 or 2, hot blocks or sharp logits now and then,
and the AUTO, KV-outer or query-outer schedule.  Selection must match row by
row (tie band allowed and counted); attention is then compared, from the
oracle's selection where a row lies in the tie band, under the same
tolerances as every other parity test.  The attention backward and the
Index-Branch loss are checked on the same draws (alternate cases), for the
oracle's selection, under their own tests' tolerances, and alternate cases
run the whole forward over an all-MXFP8 cache that the oracle's quantiser
built (the oracle scores and attends over the exactly decoded values).
"""
import numpy as np
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs
from oracle import oracle as O

from tests.parity import assert_attention, check_selection, host, to_f64

pytestmark = pytest.mark.gpu

N_CASES = 32


def draw(i):
    rng = np.random.default_rng(7000 + i)
    bk = int(rng.choice([32, 64, 128]))
    h_kv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16, 32]))
    n_k = int(rng.integers(1, 40 * bk + 1))
    n_q = int(rng.integers(1, min(n_k, 500) + 1))
    wl = inputs.small(f"random_{i}", seed=7000 + i, batch=int(rng.choice([1, 1, 2])), n_q=n_q, n_k=n_k,
                      q_offset=int(rng.integers(0, n_k - n_q + 1)), block_size=bk, topk=int(rng.integers(1, 33)),
                      h_q=h_kv * g, h_kv=h_kv, d=int(rng.choice([64, 128])), d_idx=int(rng.choice([32, 64, 128])),
                      dtype=str(rng.choice(["bf16", "f32"])), hot_frac=float(rng.choice([0.0, 0.0, 0.1])),
                      sharp=bool(rng.random() < 0.2))
    return wl, str(rng.choice(["auto", "kv_outer", "q_outer"]))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_problem(i):
    wl, sched = draw(i)
    print(f"case {i}: {wl} sched={sched}", flush=True)
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl, sched=sched)
    ids, out, lse = api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    torch.cuda.synchronize()
    h = {k: host(v) for k, v in x.items()}
    ids_o, out_o, lse_o, s_o = O.forward(O.problem_of(wl), h["q"], h["k"], h["v"], h["iq"], h["ik"])
    got = host(ids).numpy().reshape(wl.batch * wl.n_q, wl.h_kv, wl.topk)
    res = check_selection(wl, got, ids_o, s_o)
    assert res["fail"] == 0, res
    if res["tie"]:
        out, lse = api.sparse_attention(p, x["q"], x["k"], x["v"],
                                        torch.from_numpy(ids_o.reshape(tuple(ids.shape))).cuda())
        torch.cuda.synchronize()
    mx, rl = assert_attention(wl.dtype, to_f64(out).reshape(out_o.shape), out_o,
                              host(lse).numpy().reshape(lse_o.shape), lse_o, what=f"random_{i}/{sched}")
    print(f"case {i}: selection {res['exact']} exact, {res['tie']} tie; max-abs {mx:.2e} rel-L2 {rl:.2e}")


@pytest.mark.parametrize("i", range(0, N_CASES, 2))
def test_random_backward(i):
    """The attention backward on the same random problems (every other one),
    for the oracle's selection, under the backward tests' tolerances."""
    from tests.test_gpu_backward import attended_keys, check, run_backward
    wl, _ = draw(i)
    print(f"case {i}: {wl}", flush=True)
    x = inputs.generate(wl, device="cuda", tensors=("q", "k", "v", "iq", "ik", "dout"))
    h = {k: host(v) for k, v in x.items()}
    prob = O.problem_of(wl)
    ids = O.select(prob, O.block_scores(prob, h["iq"], h["ik"]))
    rq, rk, rv = O.attend_backward(prob, h["q"], h["k"], h["v"], h["dout"], ids)
    dq, dk, dv = run_backward(wl, x, ids)
    errs = [check(wl.dtype, dq, rq, "dq"), check(wl.dtype, dk, rk, "dk"), check(wl.dtype, dv, rv, "dv")]
    unseen = ~attended_keys(wl, ids)
    assert np.all(to_f64(dk)[unseen] == 0) and np.all(to_f64(dv)[unseen] == 0), "gradients at unattended keys"
    print(f"case {i}: (max-abs/max, rel-L2) dq {errs[0]}, dk {errs[1]}, dv {errs[2]}")


@pytest.mark.parametrize("i", range(1, N_CASES, 2))
def test_random_indexer_kl(i):
    """The Index-Branch loss and its gradients on the other random problems,
    for the oracle's selection, under the indexer-loss tests' tolerances."""
    from tests.test_gpu_indexer_kl import LOSS_SCALE, check, run_kl, selected_keys
    wl, _ = draw(i)
    print(f"case {i}: {wl}", flush=True)
    x = inputs.generate(wl, device="cuda")
    h = {k: host(v) for k, v in x.items()}
    prob = O.problem_of(wl)
    ids = O.select(prob, O.block_scores(prob, h["iq"], h["ik"]))
    rkl, riq, rik = O.indexer_kl(prob, h["q"], h["k"], h["iq"], h["ik"], ids, loss_scale=LOSS_SCALE)
    kl, d_iq, d_ik = run_kl(wl, x, ids)
    got = host(kl).numpy().astype(np.float64).reshape(-1, wl.h_kv)
    err = float(np.max(np.abs(got - rkl)))
    assert err <= 1e-4 * float(np.max(rkl)) + 1e-6, f"kl: max-abs {err:.3e}, max kl {np.max(rkl):.3e}"
    e_q = check(wl.dtype, d_iq, riq.reshape(d_iq.shape), "d_iq")
    e_k = check(wl.dtype, d_ik, rik, "d_ik")
    assert np.all(to_f64(d_ik)[~selected_keys(wl, ids)] == 0), "d_ik at unselected keys"
    print(f"case {i}: kl max-abs {err:.2e}, d_iq {e_q}, d_ik {e_k}")


def _mx_cache(t):
    """The oracle's MXFP8 cache of a tensor (codes then scales, as the library
    takes it) and its exactly dequantised values."""
    codes, scales = O.mx_quantize(host(t))
    cache = torch.from_numpy(np.concatenate([codes.reshape(-1), scales.reshape(-1)])).cuda()
    return cache, np.ascontiguousarray(O.mx_dequantize(codes, scales).reshape(tuple(t.shape)))


@pytest.mark.parametrize("i", range(0, N_CASES, 2))
def test_random_all_mxfp8_cache(i):
    """msa_forward over an all-MXFP8 cache (index keys, K and V) on the same
    random problems: the oracle selects and attends over the exactly decoded
    caches it built itself."""
    wl, sched = draw(i)
    print(f"case {i}: {wl} sched={sched}", flush=True)
    x = inputs.generate(wl, device="cuda")
    (ikc, ik64), (kc, k64), (vc, v64) = _mx_cache(x["ik"]), _mx_cache(x["k"]), _mx_cache(x["v"])
    p = api.problem_of(wl, sched=sched, idx_format="mxfp8", kv_format="mxfp8")
    ids, out, lse = api.forward(p, x["q"], kc, vc, x["iq"], ikc)
    torch.cuda.synchronize()
    prob = O.problem_of(wl)
    s_o = O.block_scores(prob, np.ascontiguousarray(to_f64(x["iq"])), ik64)
    ids_o = O.select(prob, s_o)
    res = check_selection(wl, host(ids).numpy().reshape(wl.batch * wl.n_q, wl.h_kv, wl.topk), ids_o, s_o)
    assert res["fail"] == 0, res
    if res["tie"]:
        out, lse = api.sparse_attention(p, x["q"], kc, vc, torch.from_numpy(ids_o.reshape(tuple(ids.shape))).cuda())
        torch.cuda.synchronize()
    o_o, l_o = O.attend(prob, np.ascontiguousarray(to_f64(x["q"])), k64, v64, ids_o)
    mx, rl = assert_attention(wl.dtype, to_f64(out).reshape(o_o.shape), o_o, host(lse).numpy().reshape(l_o.shape),
                              l_o, what=f"random_{i}/mxfp8/{sched}")
    print(f"case {i}: selection {res['exact']} exact, {res['tie']} tie; max-abs {mx:.2e} rel-L2 {rl:.2e}")
