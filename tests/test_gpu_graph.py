"""The entry points under HIP graph capture.

The library allocates nothing, never synchronises and records no memset, so a
caller can capture a whole step in a hipGraph and replay it.  Each test
captures one entry point with every buffer (outputs and workspace) passed in,
replays the graph several times with eager work of the library and
synchronisations in between, and checks every replay bit for bit against the
eager call on the same inputs (the library is deterministic).
"""
import pytest
import torch

from block_sparse_long_bk_amd import api, inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def replay_and_check(capture, outputs, reference, disturb):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture()
    for r in range(REPLAYS):
        for o in outputs:
            o.zero_()
        disturb()  # eager work of the library on other buffers between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("first", "second", "third"), outputs, reference):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {r}: {name} output differs"


def test_forward_prefill_under_graph_capture():
    wl = inputs.small("graph_prefill", seed=7101, dtype="bf16", n_q=2048, n_k=2048, h_q=16, h_kv=2, d=128,
                      d_idx=128, topk=8)
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl)
    ws = api.alloc_workspace(p, api.OP_FORWARD, "cuda")
    ids = torch.empty((wl.batch, wl.n_q, wl.h_kv, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"])
    lse = torch.empty((wl.batch, wl.n_q, wl.h_q), dtype=torch.float32, device="cuda")
    api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ids=ids, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    ref = (ids.clone(), out.clone(), lse.clone())
    # the same problem on other inputs, eagerly, between the replays
    y = inputs.generate(wl.with_(seed=7102), device="cuda")
    ws2 = api.alloc_workspace(p, api.OP_FORWARD, "cuda")
    replay_and_check(
        lambda: api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ids=ids, out=out, lse=lse, ws=ws),
        (ids, out, lse), ref,
        lambda: api.forward(p, y["q"], y["k"], y["v"], y["iq"], y["ik"], ws=ws2))


def test_forward_decode_under_graph_capture():
    wl = inputs.small("graph_decode", seed=7103, dtype="bf16", batch=4, n_q=1, n_k=20000, q_offset=19999, h_q=16,
                      h_kv=2, d=128, d_idx=128, topk=16)
    x = inputs.generate(wl, device="cuda")
    p = api.problem_of(wl)
    ws = api.alloc_workspace(p, api.OP_FORWARD, "cuda")
    ids = torch.empty((wl.batch, wl.n_q, wl.h_kv, wl.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"])
    lse = torch.empty((wl.batch, wl.n_q, wl.h_q), dtype=torch.float32, device="cuda")
    api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ids=ids, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    ref = (ids.clone(), out.clone(), lse.clone())
    ws2 = api.alloc_workspace(p, api.OP_FORWARD, "cuda")
    replay_and_check(
        lambda: api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ids=ids, out=out, lse=lse, ws=ws),
        (ids, out, lse), ref,
        lambda: api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], ws=ws2))


def test_backward_under_graph_capture():
    wl = inputs.small("graph_backward", seed=7104, dtype="bf16", n_q=1024, n_k=1024, h_q=16, h_kv=2, d=128,
                      d_idx=128, topk=6)
    x = inputs.generate(wl, device="cuda", tensors=("q", "k", "v", "iq", "ik", "dout"))
    p = api.problem_of(wl)
    ids = api.index_topk(p, x["iq"], x["ik"])
    o, lse = api.sparse_attention(p, x["q"], x["k"], x["v"], ids)
    ws = api.alloc_workspace(p, api.OP_BACKWARD, "cuda")
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    api.sparse_attention_backward(p, x["q"], x["k"], x["v"], o, lse, x["dout"], ids, dq, dk, dv, ws=ws)
    torch.cuda.synchronize()
    ref = (dq.clone(), dk.clone(), dv.clone())
    ws2 = api.alloc_workspace(p, api.OP_BACKWARD, "cuda")
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    replay_and_check(
        lambda: api.sparse_attention_backward(p, x["q"], x["k"], x["v"], o, lse, x["dout"], ids, dq, dk, dv, ws=ws),
        (dq, dk, dv), ref,
        lambda: api.sparse_attention_backward(p, x["q"], x["k"], x["v"], o, lse, x["dout"], ids, dq2, dk2, dv2,
                                              ws=ws2))
