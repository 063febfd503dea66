"""Seeded synthetic inputs for the MSA forward pass.

This module only draws random tensors; it holds none of the method's
arithmetic and is shared by the tests (GPU path and oracle alike) and the
benchmark.  Nothing here imports the HIP binding or the oracle.

Recipe (the pages use MiniMax-M3 activations at up to 1M context, which are
not available; these tensors stand in for them):
  * q, k, v           ~ N(0, 1) / sqrt(d)          (``sharp``: N(0, 1))
  * idx_q, idx_k      ~ N(0, 1) / sqrt(d_idx)
  * every token of key block j of group g in idx_k gets the same offset
    vector o[b, g, j, :] ~ N(0, 0.5^2) per element, so block scores separate;
  * ``hot_frac`` > 0: a seeded set of floor(hot_frac * nblk) blocks and a
    seeded unit vector u_g per group; idx_q[:, :, g] += u_g and the tokens of
    the hot blocks get idx_k[..., g, :] += sqrt(2) * u_g, shifting their
    scores by about two standard deviations of the block-offset term.
Values are drawn in fp32 in chunks of 65536 tokens from a generator whose seed
is a fixed function of (config seed, tensor, batch, chunk), then rounded once
to the requested dtype.  Generation runs on the target device.
"""
import math
from dataclasses import dataclass, replace

import torch

CHUNK = 65536

# Tensor ids mixed into the per-chunk seeds.
_T_Q, _T_K, _T_V, _T_IQ, _T_IK, _T_OFF, _T_HOT, _T_DOUT = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic MSA problem."""
    name: str
    batch: int
    n_q: int
    n_k: int
    q_offset: int
    block_size: int
    topk: int
    h_q: int
    h_kv: int
    d: int
    d_idx: int
    dtype: str = "bf16"          # "bf16" or "f32"
    hot_frac: float = 0.0
    seed: int = 1000
    sharp: bool = False
    offset_std: float = 0.5

    @property
    def nblk(self):
        return (self.n_k + self.block_size - 1) // self.block_size

    @property
    def torch_dtype(self):
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    def with_(self, **kw):
        return replace(self, **kw)


# The five workloads the method is measured on (sizes from the pages:
# Bk = 128, k = 16, a 2048-token budget, contexts up to 1M tokens).
WORKLOADS = {
    "tiny_f32_4k": Workload("tiny_f32_4k", 1, 4096, 4096, 0, 128, 4, 8, 2, 64, 32, "f32", 0.0, 1000),
    "prefill_32k": Workload("prefill_32k", 1, 32768, 32768, 0, 128, 16, 64, 8, 128, 128, "bf16", 0.0, 1001),
    "skewed_prefill_128k": Workload("skewed_prefill_128k", 1, 131072, 131072, 0, 128, 16, 64, 8, 128, 128,
                                    "bf16", 0.05, 1002),
    "decode_16x1m": Workload("decode_16x1m", 16, 1, 1 << 20, (1 << 20) - 1, 128, 16, 64, 8, 128, 128,
                             "bf16", 0.0, 1003),
    "chunk_16k_at_1m": Workload("chunk_16k_at_1m", 1, 16384, 1 << 20, (1 << 20) - 16384, 128, 16, 64, 8, 128,
                                128, "bf16", 0.02, 1004),
    # The block-size ablation at the prefill shape: 64-token blocks keep the
    # 2048-token budget (k = 32); 32-token blocks with k = 32 (the largest k
    # supported) select 1024 tokens.
    "prefill_32k_bk64": Workload("prefill_32k_bk64", 1, 32768, 32768, 0, 64, 32, 64, 8, 128, 128, "bf16", 0.0,
                                 1005),
    "prefill_32k_bk32": Workload("prefill_32k_bk32", 1, 32768, 32768, 0, 32, 32, 64, 8, 128, 128, "bf16", 0.0,
                                 1006),
}


def _seed(base, tensor, b, chunk):
    # A fixed mixing of the four integers into a 63-bit seed.
    x = (base * 1000003 + tensor) * 1000033 + b
    x = x * 1000037 + chunk
    return (x * 0x9E3779B97F4A7C15) & ((1 << 63) - 1)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _fill_gaussian(out, wl, tensor, scale, device, block_offsets=None, hot_add=None):
    """out: [B, N, H, D] in the target dtype; filled chunk by chunk."""
    B, N, H, D = out.shape
    for b in range(B):
        for c0 in range(0, N, CHUNK):
            c1 = min(N, c0 + CHUNK)
            g = _gen(device, _seed(wl.seed, tensor, b, c0 // CHUNK))
            x = torch.randn((c1 - c0, H, D), generator=g, device=device, dtype=torch.float32)
            x.mul_(scale)
            if block_offsets is not None:
                # token t belongs to key block t // Bk
                blk = torch.arange(c0, c1, device=device) // wl.block_size
                x.add_(block_offsets[b].index_select(0, blk))
            if hot_add is not None:
                x.add_(hot_add(b, c0, c1))
            out[b, c0:c1].copy_(x)
            del x


def hot_blocks(wl, device="cpu"):
    """The seeded hot-block ids (sorted) and the per-group unit vectors u_g."""
    n_hot = int(math.floor(wl.hot_frac * wl.nblk))
    g = _gen("cpu", _seed(wl.seed, _T_HOT, 0, 0))
    perm = torch.randperm(wl.nblk, generator=g)
    ids = torch.sort(perm[:n_hot]).values
    u = torch.randn((wl.h_kv, wl.d_idx), generator=g, dtype=torch.float32)
    u = u / u.norm(dim=1, keepdim=True)
    return ids.to(device), u.to(device)


def generate(wl, device="cpu", tensors=("q", "k", "v", "iq", "ik")):
    """Return a dict of the requested tensors for workload ``wl`` on ``device``."""
    dt = wl.torch_dtype
    B, Nq, Nk = wl.batch, wl.n_q, wl.n_k
    out = {}
    qk_scale = 1.0 if wl.sharp else 1.0 / math.sqrt(wl.d)
    if "q" in tensors:
        out["q"] = torch.empty((B, Nq, wl.h_q, wl.d), dtype=dt, device=device)
        _fill_gaussian(out["q"], wl, _T_Q, qk_scale, device)
    if "k" in tensors:
        out["k"] = torch.empty((B, Nk, wl.h_kv, wl.d), dtype=dt, device=device)
        _fill_gaussian(out["k"], wl, _T_K, qk_scale, device)
    if "v" in tensors:
        out["v"] = torch.empty((B, Nk, wl.h_kv, wl.d), dtype=dt, device=device)
        _fill_gaussian(out["v"], wl, _T_V, 1.0 / math.sqrt(wl.d), device)
    if "dout" in tensors:
        # upstream gradient of the attention output (for the backward pass)
        out["dout"] = torch.empty((B, Nq, wl.h_q, wl.d), dtype=dt, device=device)
        _fill_gaussian(out["dout"], wl, _T_DOUT, 1.0, device)
    hot = None
    if wl.hot_frac > 0 and ("iq" in tensors or "ik" in tensors):
        hot = hot_blocks(wl, device)
    if "iq" in tensors:
        out["iq"] = torch.empty((B, Nq, wl.h_kv, wl.d_idx), dtype=dt, device=device)
        add = None
        if hot is not None:
            u = hot[1]
            add = lambda b, c0, c1: u.unsqueeze(0)  # noqa: E731  every query, its group's u_g
        _fill_gaussian(out["iq"], wl, _T_IQ, 1.0 / math.sqrt(wl.d_idx), device, hot_add=add)
    if "ik" in tensors:
        out["ik"] = torch.empty((B, Nk, wl.h_kv, wl.d_idx), dtype=dt, device=device)
        offs = []
        for b in range(B):
            g = _gen(device, _seed(wl.seed, _T_OFF, b, 0))
            o = torch.randn((wl.nblk, wl.h_kv, wl.d_idx), generator=g, device=device, dtype=torch.float32)
            offs.append(o.mul_(wl.offset_std))
        add = None
        if hot is not None:
            is_hot = torch.zeros(wl.nblk, dtype=torch.bool, device=device)
            is_hot[hot[0]] = True
            shift = math.sqrt(2.0) * hot[1]  # [h_kv, d_idx]

            def add(b, c0, c1):
                blk = torch.arange(c0, c1, device=device) // wl.block_size
                m = is_hot.index_select(0, blk).to(torch.float32)
                return m[:, None, None] * shift[None]
        _fill_gaussian(out["ik"], wl, _T_IK, 1.0 / math.sqrt(wl.d_idx), device, block_offsets=offs,
                       hot_add=add)
    return out


def small(name="tiny", **kw):
    """A small workload for tests, derived from the tiny fp32 shape."""
    base = WORKLOADS["tiny_f32_4k"].with_(name=name)
    return base.with_(**kw)
