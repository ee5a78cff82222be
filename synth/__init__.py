"""Seeded synthetic inputs for the verification step.

This module only draws random tensors and names workload shapes.  It holds
none of the verification method's arithmetic (no softmax, no forward pass, no
acceptance rule), so both the HIP path's tests and the oracle may use it.

Recipe (shared by tests and the benchmark):
  * weights W ~ N(0, std = 1/sqrt(fan_in)), drawn in float32; bfloat16
    weights are the float32 draw rounded to nearest-even.  fan_in is d for
    W_up and the LM head and ffn for W_down.
  * hidden states ~ N(0, 1), float32, [B, gamma+1, d].
  * draft-noise ~ N(0, sigma), float32, [B, gamma, V] (the workload turns it
    into q = softmax(target logits + noise) with the oracle or the target
    pass; that step lives with the caller).
  * RMSNorm gains are all ones unless a test asks for random gains.

CPU draws use numpy's PCG64 seeded by SeedSequence(ROOT_SEED, spawn_key=...);
device draws for the large shapes use torch's generator on the device, seeded
from the same key, so a workload is reproducible on either side.
"""

from dataclasses import dataclass

import numpy as np

ROOT_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    gamma: int
    d: int
    ffn: int
    n_blocks: int
    V: int
    wdtype: str          # "f32" or "bf16"
    temperature: float
    top_p: float
    alpha_target: float  # mean acceptance the draft noise is tuned for (0: n/a)


# The five synthetic verification workloads.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 256, 1024, 1, 512, "f32", 1.0, 1.0, 0.0),
    "mid": Workload("mid", 1, 4, 4096, 14336, 4, 32000, "bf16", 1.0, 1.0, 0.8),
    "large": Workload("large", 1, 5, 8192, 28672, 8, 128256, "bf16", 1.0, 1.0, 0.7),
    "topp": Workload("topp", 8, 8, 4096, 14336, 4, 128256, "bf16", 0.7, 0.9, 0.0),
    "greedy": Workload("greedy", 32, 6, 8192, 28672, 8, 128256, "bf16", 0.0, 1.0, 0.75),
}

# Tensor ids inside a workload's seed tree.
T_W_UP, T_W_DOWN, T_LM, T_HIDDEN, T_NOISE, T_DRAFT, T_GAIN, T_MISC = range(8)


def generator(*key):
    """numpy Generator for a spawn key of small non-negative ints."""
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(int(k) for k in key))))


def torch_seed(*key):
    """A 63-bit torch seed derived from the same key."""
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(int(k) for k in key))
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 (nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def normal(gen, shape, std=1.0):
    return (gen.standard_normal(shape, dtype=np.float32) * np.float32(std))


def weight_np(gen, fan_in, fan_out, wdtype):
    w = normal(gen, (fan_in, fan_out), 1.0 / np.sqrt(fan_in))
    return f32_to_bf16_bits(w) if wdtype == "bf16" else w


def model_np(key, d, ffn, n_blocks, V, wdtype, random_gain=False):
    """Host weights for a small model: dict(blocks=[...], lm_head=...)."""
    blocks = []
    for l in range(n_blocks):
        blk = {"w_up": weight_np(generator(*key, T_W_UP, l), d, ffn, wdtype),
               "w_down": weight_np(generator(*key, T_W_DOWN, l), ffn, d, wdtype),
               "gain": None}
        if random_gain:
            g = 1.0 + 0.25 * normal(generator(*key, T_GAIN, l), (d,))
            blk["gain"] = f32_to_bf16_bits(g) if wdtype == "bf16" else g
        blocks.append(blk)
    lm = weight_np(generator(*key, T_LM, 0), d, V, wdtype)
    return {"blocks": blocks, "lm_head": lm, "eps": 1e-6}


def hidden_np(key, B, gamma, d):
    return normal(generator(*key, T_HIDDEN), (B, gamma + 1, d))


def noise_np(key, B, gamma, V, sigma):
    """N(0, sigma) noise; sigma may be a scalar or a per-row array [B]."""
    z = normal(generator(*key, T_NOISE), (B, gamma, V))
    s = np.asarray(sigma, dtype=np.float32).reshape(-1, 1, 1) if np.ndim(sigma) else np.float32(sigma)
    return z * s


# ---- device-side draws for the large shapes (torch only as a random source)

def weight_torch(key, fan_in, fan_out, wdtype, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(*key))
    w = torch.randn((fan_in, fan_out), generator=g, device=device, dtype=torch.float32)
    w.mul_(1.0 / np.sqrt(fan_in))
    return w.to(torch.bfloat16) if wdtype == "bf16" else w


def model_torch(key, d, ffn, n_blocks, V, wdtype, device):
    blocks = []
    for l in range(n_blocks):
        blocks.append({"w_up": weight_torch((*key, T_W_UP, l), d, ffn, wdtype, device),
                       "w_down": weight_torch((*key, T_W_DOWN, l), ffn, d, wdtype, device),
                       "gain": None})
    lm = weight_torch((*key, T_LM, 0), d, V, wdtype, device)
    return {"blocks": blocks, "lm_head": lm, "eps": 1e-6}


def normal_torch(key, shape, std, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(*key))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * float(std)


def torch_to_host(t):
    """Host numpy copy; bfloat16 tensors come back as uint16 bit patterns."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
