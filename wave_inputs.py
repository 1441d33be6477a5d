"""Seeded synthetic inputs and workload shapes for wave attention.

Shared by the tests, ``bench.py`` and ``__graft_entry__``: it generates the
Q/K/V tensors that both the HIP path and the CPU oracle consume, and holds
none of the method's arithmetic (no masks, no schedules, no attention).

Recipe
------
* Every tensor is keyed by (workload seed, layer, chunk, level | COND, which)
  with which in {q, k, v}; the key is hashed with splitmix64 into a 63-bit
  seed.
* Values are N(0, sigma^2) drawn in float32.
* The toy denoiser chain adds, per layer, a projection matrix W [3D][D]
  (D = heads * head_dim) drawn N(0, 1/D), keyed (workload seed, layer, "w"),
  and per chunk a noise input X [L][D] drawn N(0, 1), keyed (workload seed,
  chunk, "x").
* The tiny workload draws on the host with numpy's PCG64 and hands float32 to
  the kernels (they round to bfloat16).  The large workloads draw on the
  device with a ``torch.Generator`` and round to bfloat16 with torch before
  any kernel sees them.

Workloads (sizes of the Wan2.1-T2V-1.3B video setting in the streaming video
diffusion design-space paper, arXiv 2609.22283 listing, appendix Table 4:
832x480, 21 latent frames in 7 chunks of 3; and of the Wan-Streamer v0.2
640x368 stream with K/V-only language/state conditioning and unsharded audio):
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Policy and schedule codes (same values as the C header's enums).
CLEAN, SAME_LEVEL, PROGRESSIVE = 0, 1, 2
SERIAL, WAVE = 0, 1
COND_LEVEL = -1
POLICY_NAMES = {CLEAN: "clean", SAME_LEVEL: "same-level", PROGRESSIVE: "progressive"}


@dataclass(frozen=True)
class Workload:
    key: int                 # workload seed
    name: str
    B: int
    K: int
    policies: tuple
    chunk_len: int
    heads: int
    head_dim: int
    layers: int = 1
    cond_len: int = 0
    history_cap: int = -1
    sigma: float = 1.0
    host_fp32: bool = False  # draw on host as float32 (tiny case)
    round: int = -1          # single measured round, -1 = whole rollout
    query_len: int = 0       # query rows per node, 0 = chunk_len (fewer: decode-shaped)
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS = {
    1: Workload(1, "tiny-progressive-B4K2", B=4, K=2, policies=(PROGRESSIVE,),
                chunk_len=128, heads=2, head_dim=64, host_fp32=True),
    2: Workload(2, "wan1.3b-832x480-7chunk-K4-progressive-round6", B=7, K=4,
                policies=(PROGRESSIVE,), chunk_len=4680, heads=12, head_dim=128,
                round=6),
    3: Workload(3, "wan1.3b-832x480-7chunk-K5-30layer-rollout", B=7, K=5,
                policies=(CLEAN, SAME_LEVEL, PROGRESSIVE), chunk_len=4680,
                heads=12, head_dim=128, layers=30),
    4: Workload(4, "long-video-B28-K4-progressive-H6", B=28, K=4,
                policies=(PROGRESSIVE,), chunk_len=4680, heads=12, head_dim=128,
                history_cap=6, sigma=0.5),
    5: Workload(5, "wan-streamer-640x368-B8-K2-same-level-cond512-audio64", B=8, K=2,
                policies=(SAME_LEVEL,), chunk_len=2760 + 64, heads=40, head_dim=128,
                cond_len=512, round=7),
    # Decode-shaped: only the 64 audio tokens of each chunk query (the audio
    # latents follow the 2760 video tokens of the chunk).
    6: Workload(6, "wan-streamer-640x368-audio-decode-64rows-round7", B=8, K=2,
                policies=(SAME_LEVEL,), chunk_len=2760 + 64, heads=40, head_dim=128,
                cond_len=512, round=7, query_len=64),
}

_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def tensor_seed(workload_key: int, layer: int, chunk: int, level: int, which: str,
                policy: int = 0) -> int:
    """63-bit seed of one tensor; level COND_LEVEL marks a conditioning slot."""
    w = {"q": 0, "k": 1, "v": 2, "x": 3, "w": 4}[which]
    h = 0
    for part in (workload_key, policy, layer, chunk, level + 1, w):
        h = _splitmix64(h ^ (int(part) & _MASK64))
    return h >> 1


def host_normal(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = (x * np.float32(sigma)).astype(np.float32)
    return x


def device_normal_bf16(seed: int, shape, sigma: float, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def slot_shape(w: Workload, level: int):
    n = w.cond_len if level == COND_LEVEL else w.chunk_len
    return (n, w.heads, w.head_dim)


def q_shape(w: Workload):
    return (w.chunk_len, w.heads, w.head_dim)


def host_tensor(w: Workload, layer, chunk, level, which, policy=0) -> np.ndarray:
    shape = q_shape(w) if which == "q" else slot_shape(w, level)
    return host_normal(tensor_seed(w.key, layer, chunk, level, which, policy), shape, w.sigma)


def device_tensor(w: Workload, layer, chunk, level, which, device, policy=0):
    shape = q_shape(w) if which == "q" else slot_shape(w, level)
    return device_normal_bf16(tensor_seed(w.key, layer, chunk, level, which, policy),
                              shape, w.sigma, device)


# --- toy denoiser chain inputs ------------------------------------------------

def chain_weight_seed(workload_key: int, layer: int) -> int:
    """Seed of layer `layer`'s projection matrix."""
    return tensor_seed(workload_key, layer, -1, -1, "w")


def chain_noise_seed(workload_key: int, chunk: int) -> int:
    """Seed of chunk `chunk`'s noise input (the input of its first update)."""
    return tensor_seed(workload_key, 0, chunk, COND_LEVEL - 1, "x")


def host_chain_weight(workload_key: int, layer: int, model_dim: int) -> np.ndarray:
    """W [3D][D] float32, N(0, 1/D)."""
    return host_normal(chain_weight_seed(workload_key, layer), (3 * model_dim, model_dim),
                       float(1.0 / np.sqrt(model_dim)))


def host_chain_noise(workload_key: int, chunk: int, tokens: int, model_dim: int) -> np.ndarray:
    """X [L][D] float32, N(0, 1)."""
    return host_normal(chain_noise_seed(workload_key, chunk), (tokens, model_dim), 1.0)


def device_chain_weight(workload_key: int, layer: int, model_dim: int, device):
    """W [3D][D] bfloat16 on the device, N(0, 1/D)."""
    return device_normal_bf16(chain_weight_seed(workload_key, layer), (3 * model_dim, model_dim),
                              float(1.0 / np.sqrt(model_dim)), device)


def device_chain_noise(workload_key: int, chunk: int, tokens: int, model_dim: int, device):
    """X [L][D] bfloat16 on the device, N(0, 1)."""
    return device_normal_bf16(chain_noise_seed(workload_key, chunk), (tokens, model_dim), 1.0, device)
