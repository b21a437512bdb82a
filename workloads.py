"""Seeded synthetic inputs for the bf16 delta-sync hot path.

This module is shared by the tests, the smoke check and the benchmark, and it
feeds the same bits to both the CPU oracle and the HIP library.  It holds
none of the method's arithmetic (no compare, compaction, scatter or XOR): it
only builds parameter shapes and draws pre-step / post-step bf16 snapshots.

Step model.  The optimizer-step picture of the TRL delta-sync article
(section 2, "why bf16 RL weights are almost always sparse"): an Adam update
has magnitude close to the learning rate, dw = -lr * u with u ~ N(0, 1), and
weights are drawn from N(0, 0.02).  Two readings are generated:

* ``fp32_master``:   old = bf16(w),  new = bf16(w - lr*u)   (w kept in fp32)
* ``bf16_resident``: old = bf16(w),  new = bf16(float(old) - lr*u)

Both casts are round-to-nearest-even (torch's float32 -> bfloat16 cast).

Density sweep.  A seeded subset of exactly k = round(f*n) elements (uniform
pattern) or of whole aligned 2048-element (4 KB) runs (clustered pattern) is
forced to a different bf16 value by toggling the lowest significand bit.

Seeds: tensor t of a workload whose seed family is f uses seed
(f << 20) | (t << 1) for w and that value | 1 for u.  Generation runs on whatever device the caller names;
parity never depends on the RNG because both sides receive the same bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

WEIGHT_STD = 0.02
ALIGN_ELEMS = 128          # 256-byte alignment of every parameter in a flat arena
CLUSTER_RUN = 2048         # elements per 4 KB run in the clustered pattern
DENSITIES = (0.00085, 0.01, 0.02, 0.10, 0.50)


@dataclass(frozen=True)
class Config:
    key: str
    seed_family: int         # the f of the seed recipe above
    title: str
    params: tuple            # ((name, shape), ...)
    lrs: tuple
    mode: str                # default step reading

    @property
    def numels(self):
        return [math.prod(s) for _, s in self.params]

    @property
    def total(self):
        return sum(self.numels)


def _qwen3_0p6b():
    h, inter, layers, vocab = 1024, 3072, 28, 151936
    ps = [("model.embed_tokens.weight", (vocab, h))]
    for i in range(layers):
        p = f"model.layers.{i}."
        ps += [
            (p + "self_attn.q_proj.weight", (2048, h)),
            (p + "self_attn.k_proj.weight", (1024, h)),
            (p + "self_attn.v_proj.weight", (1024, h)),
            (p + "self_attn.o_proj.weight", (h, 2048)),
            (p + "self_attn.q_norm.weight", (128,)),
            (p + "self_attn.k_norm.weight", (128,)),
            (p + "mlp.gate_proj.weight", (inter, h)),
            (p + "mlp.up_proj.weight", (inter, h)),
            (p + "mlp.down_proj.weight", (h, inter)),
            (p + "input_layernorm.weight", (h,)),
            (p + "post_attention_layernorm.weight", (h,)),
        ]
    ps.append(("model.norm.weight", (h,)))
    return tuple(ps)


def _llama_7b():
    h, inter, layers, vocab = 4096, 11008, 32, 32000
    ps = [("model.embed_tokens.weight", (vocab, h))]
    for i in range(layers):
        p = f"model.layers.{i}."
        ps += [
            (p + "self_attn.q_proj.weight", (h, h)),
            (p + "self_attn.k_proj.weight", (h, h)),
            (p + "self_attn.v_proj.weight", (h, h)),
            (p + "self_attn.o_proj.weight", (h, h)),
            (p + "mlp.gate_proj.weight", (inter, h)),
            (p + "mlp.up_proj.weight", (inter, h)),
            (p + "mlp.down_proj.weight", (h, inter)),
            (p + "input_layernorm.weight", (h,)),
            (p + "post_attention_layernorm.weight", (h,)),
        ]
    ps.append(("model.norm.weight", (h,)))
    ps.append(("lm_head.weight", (vocab, h)))
    return tuple(ps)


def _llama_405b_share(layers=10):
    h, kv, inter = 16384, 1024, 53248
    ps = []
    for i in range(layers):
        p = f"model.layers.{i}."
        ps += [
            (p + "self_attn.q_proj.weight", (h, h)),
            (p + "self_attn.k_proj.weight", (kv, h)),
            (p + "self_attn.v_proj.weight", (kv, h)),
            (p + "self_attn.o_proj.weight", (h, h)),
            (p + "mlp.gate_proj.weight", (inter, h)),
            (p + "mlp.up_proj.weight", (inter, h)),
            (p + "mlp.down_proj.weight", (h, inter)),
        ]
    return tuple(ps)


CONFIGS = {
    "tensor1m": Config("tensor1m", 1, "single bf16 tensor 1024x1024", (("w", (1024, 1024)),),
                 (3e-6,), "fp32_master"),
    "qwen3_0p6b": Config("qwen3_0p6b", 2, "Qwen3-0.6B-shaped parameter list", _qwen3_0p6b(),
                 (3e-6,), "fp32_master"),
    "llama7b": Config("llama7b", 3, "Llama-7B-shaped parameter list", _llama_7b(),
                 (1e-6, 3e-6, 1e-5), "bf16_resident"),
    "sweep256m": Config("sweep256m", 4, "flat 256M-element tensor, density sweep",
                 (("flat", (1 << 28,)),), (), "forced"),
    "llama405b_share": Config("llama405b_share", 5, "Llama-3.1-405B-shaped 10-layer share", _llama_405b_share(),
                 (3e-6,), "fp32_master"),
}


def seeds(seed_family: int, tensor_index: int):
    s_w = (seed_family << 20) | (tensor_index << 1)
    return s_w, s_w | 1


def flat_layout(numels, align=ALIGN_ELEMS):
    """Element offsets of each parameter in one flat arena (each start aligned)."""
    offs, pos = [], 0
    for n in numels:
        offs.append(pos)
        pos += (n + align - 1) // align * align
    return offs, max(pos, align)


def _gen(device):
    return torch.Generator(device=device)


@torch.no_grad()
def fill_step_pair_(old_out: torch.Tensor, new_out: torch.Tensor, seed_w: int, seed_u: int,
                    lr: float, mode: str, chunk: int = 1 << 28):
    """Fill bf16 views ``old_out``/``new_out`` (same numel) with one synthetic step.

    Large tensors are drawn in chunks of ``chunk`` elements from one generator
    stream per seed, so the bits depend only on (seed, numel, chunk)."""
    if old_out.dtype != torch.bfloat16 or new_out.dtype != torch.bfloat16:
        raise TypeError("outputs must be bfloat16")
    n = old_out.numel()
    if new_out.numel() != n:
        raise ValueError("size mismatch")
    dev = old_out.device
    o, nw = old_out.view(-1), new_out.view(-1)
    gw, gu = _gen(dev), _gen(dev)
    gw.manual_seed(seed_w)
    gu.manual_seed(seed_u)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        w = torch.randn(e - s, generator=gw, device=dev, dtype=torch.float32)
        w.mul_(WEIGHT_STD)
        u = torch.randn(e - s, generator=gu, device=dev, dtype=torch.float32)
        o[s:e] = w.to(torch.bfloat16)
        if mode == "fp32_master":
            w.sub_(u, alpha=lr)
            nw[s:e] = w.to(torch.bfloat16)
        elif mode == "bf16_resident":
            base = o[s:e].float()
            base.sub_(u, alpha=lr)
            nw[s:e] = base.to(torch.bfloat16)
        else:
            raise ValueError(f"unknown step mode {mode!r}")
        del w, u


def make_step_pair(numel: int, seed_w: int, seed_u: int, lr: float, mode: str,
                   device="cpu"):
    old = torch.empty(numel, dtype=torch.bfloat16, device=device)
    new = torch.empty(numel, dtype=torch.bfloat16, device=device)
    fill_step_pair_(old, new, seed_w, seed_u, lr, mode)
    return old, new


def _toggle_lsb_(bits16: torch.Tensor, sel: torch.Tensor):
    """Move the selected bf16 values one unit in the last place (lowest
    significand bit toggled, written without bitwise operators)."""
    v = bits16[sel]
    odd = torch.remainder(v, 2) == 1
    bits16[sel] = torch.where(odd, v - 1, v + 1)


@torch.no_grad()
def density_case(n: int, frac: float, pattern: str, density_index: int, device="cpu",
                 seed_base: int = 4 << 20):
    """Density-sweep input: returns (old, new, expected_changed_count)."""
    old = torch.empty(n, dtype=torch.bfloat16, device=device)
    g = _gen(device)
    g.manual_seed(seed_base)
    old.copy_((torch.randn(n, generator=g, device=device) * WEIGHT_STD).to(torch.bfloat16))
    new = old.clone()
    pat = {"uniform": 0, "clustered": 1}[pattern]
    g.manual_seed(seed_base | (pat << 8) | density_index)
    if pattern == "uniform":
        k = int(round(frac * n))
        sel = torch.randperm(n, generator=g, device=device)[:k]
    else:
        runs = n // CLUSTER_RUN
        r = int(round(frac * n / CLUSTER_RUN))
        pick = torch.randperm(runs, generator=g, device=device)[:r]
        sel = (pick[:, None] * CLUSTER_RUN
               + torch.arange(CLUSTER_RUN, device=device)[None, :]).reshape(-1)
        k = r * CLUSTER_RUN
    _toggle_lsb_(new.view(torch.int16), sel)
    return old, new, k


def bits_numpy(t: torch.Tensor):
    """Host numpy uint16 copy of a bf16 tensor's bit patterns."""
    import numpy as np

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
