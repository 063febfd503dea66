"""The C ABI from a plain C program (tests/c_abi/msa_c_client.c).

The client is compiled with gcc against include/msa.h alone (-std=c11,
warnings as errors) and linked to libmsa.so, so the header is checked as C and
the library as a C library.  CPU: its validation and workspace answers must
equal the Python binding's.  GPU: a small fp32 forward issued from C must give
bit for bit the block ids, output and lse that the binding gets for the same
inputs (the client draws them from a 32-bit LCG that this file replays).
"""
import os
import re
import subprocess

import numpy as np
import pytest

from block_sparse_long_bk_amd import api

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.dirname(api.LIB_PATH)


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("c_client") / "msa_c_client")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "c_abi", "msa_c_client.c"), "-L", LIBDIR, "-lmsa", f"-Wl,-rpath,{LIBDIR}",
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, mode):
    r = subprocess.run([exe, mode], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"{mode}: exit {r.returncode}: {r.stderr}"
    return r.stdout


def problem(n_q, n_k, h_q, h_kv, d, d_idx, topk, dtype):
    return api.problem(1, n_q, n_k, h_q, h_kv, d, d_idx, topk, dtype=dtype, q_offset=n_k - n_q)


def test_c_client_validation_and_workspace_match_the_binding(client):
    out = run(client, "cpu")
    lines = dict(re.findall(r"^validate (\w+) (-?\d+)$", out, re.M))
    assert int(lines["ok"]) == 0
    for name, args in {"group3": (4096, 4096, 12, 4, 64, 32, 4, "f32"), "offset": (4096, 2048, 8, 2, 64, 32, 4, "f32"),
                       "d96": (4096, 4096, 8, 2, 96, 32, 4, "f32")}.items():
        p = problem(*args)  # q_offset = n_k - n_q, negative for "offset" as in the client
        assert int(lines[name]) == api.validate(p), name
        assert int(lines[name]) != 0, name
    assert int(lines["null"]) == -1  # MSA_ERR_INVALID_ARG
    ok = problem(32768, 32768, 64, 8, 128, 128, 16, "bf16")
    for op, st, full, least in re.findall(r"^workspace (\d+) (-?\d+) (\d+) (\d+)$", out, re.M):
        assert int(st) == 0, op
        assert (int(full), int(least)) == tuple(api.workspace_size(ok, int(op))), op
    assert "status " in out


def lcg_values(n, state):
    """The client's generator: x <- 1664525 x + 1013904223 (mod 2^32), value
    (x >> 8) / 2^24 - 0.5 in fp32."""
    out = np.empty(n, dtype=np.float32)
    x = state
    for i in range(n):
        x = (x * 1664525 + 1013904223) & 0xFFFFFFFF
        out[i] = np.float32(x >> 8) * np.float32(1.0 / 16777216.0) - np.float32(0.5)
    return out, x


@pytest.mark.gpu
def test_c_client_forward_matches_the_binding(client):
    import torch
    text = run(client, "gpu")
    ids_c = np.array(re.search(r"^ids (.*)$", text, re.M).group(1).split(), dtype=np.int64)
    out_c = np.array([int(w, 16) for w in re.search(r"^out (.*)$", text, re.M).group(1).split()], dtype=np.uint32)
    lse_c = np.array([int(w, 16) for w in re.search(r"^lse (.*)$", text, re.M).group(1).split()], dtype=np.uint32)
    p = problem(512, 1024, 8, 2, 64, 32, 4, "f32")
    state = 12345
    shapes = {"q": (1, 512, 8, 64), "k": (1, 1024, 2, 64), "v": (1, 1024, 2, 64), "iq": (1, 512, 2, 32),
              "ik": (1, 1024, 2, 32)}
    x = {}
    for name, shape in shapes.items():  # the client's upload order
        vals, state = lcg_values(int(np.prod(shape)), state)
        x[name] = torch.from_numpy(vals.reshape(shape)).cuda()
    ids, out, lse = api.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"])
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy().reshape(-1), ids_c)
    assert np.array_equal(out.cpu().numpy().reshape(-1).view(np.uint32), out_c)
    assert np.array_equal(lse.cpu().numpy().reshape(-1).view(np.uint32), lse_c)
