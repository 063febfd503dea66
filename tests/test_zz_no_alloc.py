"""msa_forward_noalloc (the forward on the library's own per-GPU scratch)
against msa_forward with a caller workspace, through the C ABI: bitwise equal
selections, outputs and lse, on two calls in a row -- a problem that does not
fit the scratch in one pass (so the queries run in chunks), then a smaller one
(the array keeps the first call's contents, which must not leak into it)."""
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs

pytestmark = pytest.mark.gpu


def _run_pair(wl):
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl)
    ids_a, out_a, lse_a = api.forward_noalloc(p, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    ids_b, out_b, lse_b = api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(out_a.view(torch.int16) if out_a.dtype == torch.bfloat16 else out_a,
                       out_b.view(torch.int16) if out_b.dtype == torch.bfloat16 else out_b)
    assert torch.equal(lse_a, lse_b)


def test_noalloc_matches_forward_twice():
    big = inputs.small("noalloc_big", dtype="bf16", n_q=8192, n_k=8192, h_q=64, h_kv=8, d=128, d_idx=128,
                       topk=16, seed=91)
    p = api.problem_of(big)
    full, least = api.workspace_size(p, api.OP_FORWARD)
    assert least <= api.NOALLOC_SCRATCH_BYTES < full  # runs in query chunks inside the scratch
    print(f"[noalloc] big: full workspace {full >> 20} MiB, minimum {least >> 20} MiB", flush=True)
    _run_pair(big)
    small = inputs.small("noalloc_small", dtype="bf16", n_q=1000, n_k=1500, q_offset=500, h_q=16, h_kv=2,
                         d=128, d_idx=64, topk=6, seed=92)
    print("[noalloc] small", flush=True)
    _run_pair(small)
    # and a decode step (query-outer with split partials in the scratch)
    dec = inputs.small("noalloc_decode", dtype="bf16", batch=2, n_q=1, n_k=9000, q_offset=8999, h_q=16, h_kv=2,
                       d=128, d_idx=128, topk=8, seed=93)
    print("[noalloc] decode", flush=True)
    _run_pair(dec)
