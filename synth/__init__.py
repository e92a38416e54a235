"""Seeded synthetic inputs for decode attention over a vector-quantized KV cache.

This module draws random numbers and shapes them; it holds none of the method's
arithmetic (no smoothing, no Hadamard transform, no nearest-centroid search, no
attention).  Both the CPU oracle (through the tests) and the HIP library (through
the tests and the benchmark) take their inputs from here, so neither side depends
on the other for its inputs.

Value laws follow the workloads the VecInfer pages evaluate (Llama-3.1-8B and
Qwen2.5-14B attention shapes at long context; VecInfer summary card, "Key points"):
keys are standard normal with a few fixed outlier channels per KV head scaled up
(the key-cache outliers the VecInfer abstract names as the cause of poor codebook
use); values and queries are standard normal.

Two generators are provided:

* ``numpy`` (PCG64, seeded) for cases small enough for the CPU;
* ``torch`` on a device (Philox via ``torch.Generator``) for the full-size
  caches, which are tens of GB and are produced directly in HBM.

The two streams differ; every test hands the *same* drawn tensor to both sides,
copying slices to the host where the oracle needs them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

HEAD_DIM = 128
FMT_2BIT = 0      # 2^8 entries x 4 dims  -> 2 bits per element
FMT_1P5BIT = 1    # 2^12 entries x 8 dims -> 1.5 bits per element
FMT_3BIT = 2      # 2^12 entries x 4 dims -> 3 bits per element
FMT_1P25BIT = 3   # 2^10 entries x 8 dims -> 1.25 bits per element
FMT_4BIT = 4      # 2^8 entries x 2 dims  -> 4 bits per element
FORMATS = {FMT_2BIT: dict(entries=256, dsub=4), FMT_1P5BIT: dict(entries=4096, dsub=8),
           FMT_3BIT: dict(entries=4096, dsub=4), FMT_1P25BIT: dict(entries=1024, dsub=8),
           FMT_4BIT: dict(entries=256, dsub=2)}

N_OUTLIER = 4
OUTLIER_SCALE = 15.0
N_CALIB = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq_len: int
    fmt: int
    dtype: str            # "fp32" or "bf16": dtype of q, k, v as handed to the library

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def entries(self) -> int:
        return FORMATS[self.fmt]["entries"]

    @property
    def dsub(self) -> int:
        return FORMATS[self.fmt]["dsub"]

    @property
    def nsub(self) -> int:
        return HEAD_DIM // self.dsub


# The workloads: a tiny CPU-fast case, the Llama-3.1-8B attention shape at
# 32k and 196k context (batch 1 and batch 32), and a Qwen2.5-14B shape at 1.5 bits.
WORKLOADS = {
    "tiny_g4_t2048": Workload("tiny_g4_t2048", 1, 4, 1, 2048, FMT_2BIT, "fp32"),
    "llama8b_b1_t32k": Workload("llama8b_b1_t32k", 1, 32, 8, 32768, FMT_2BIT, "bf16"),
    "llama8b_b1_t196k": Workload("llama8b_b1_t196k", 1, 32, 8, 196608, FMT_2BIT, "bf16"),
    "llama8b_b32_t196k": Workload("llama8b_b32_t196k", 32, 32, 8, 196608, FMT_2BIT, "bf16"),
    "qwen14b_b8_t128k_1p5": Workload("qwen14b_b8_t128k_1p5", 8, 40, 8, 131072, FMT_1P5BIT, "bf16"),
    # The added 3-bit width (2^12 x 4) on the Llama-3.1-8B attention shape.
    "llama8b_b8_t196k_3bit": Workload("llama8b_b8_t196k_3bit", 8, 32, 8, 196608, FMT_3BIT, "bf16"),
    # The 1.25-bit width (2^10 x 8) on the Qwen2.5-14B attention shape of the 1.5-bit workload.
    "qwen14b_b8_t128k_1p25": Workload("qwen14b_b8_t128k_1p25", 8, 40, 8, 131072, FMT_1P25BIT, "bf16"),
    # The 4-bit width (2^8 x 2) on the Llama-3.1-8B attention shape of the 3-bit workload.
    "llama8b_b8_t196k_4bit": Workload("llama8b_b8_t196k_4bit", 8, 32, 8, 196608, FMT_4BIT, "bf16"),
}


def seed_for(name: str) -> int:
    """A fixed seed per workload: 0x5EED0000 plus the workload's position."""
    return 0x5EED0000 + list(WORKLOADS).index(name)


# --------------------------------------------------------------------------- numpy side

def outlier_channels(seed: int, num_kv_heads: int, n: int = N_OUTLIER) -> np.ndarray:
    """[Hkv][n] distinct channel indices per KV head, from a seeded permutation."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0xC0FFEE))
    return np.stack([rng.permutation(HEAD_DIM)[:n] for _ in range(num_kv_heads)]).astype(np.int64)


def _round_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage dtype; returns float32 holding exact values."""
    if dtype == "fp32":
        return x.astype(np.float32)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def keys_numpy(rng: np.random.Generator, shape, channels: np.ndarray, dtype: str) -> np.ndarray:
    """Keys [..., Hkv, T, 128]: N(0,1) with the head's outlier channels scaled by 15."""
    k = rng.standard_normal(shape, dtype=np.float32)
    hkv = shape[-3]
    for h in range(hkv):
        k[..., h, :, channels[h]] *= OUTLIER_SCALE
    return _round_dtype(k, dtype)


def normal_numpy(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _round_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclasses.dataclass
class CpuCase:
    """All inputs of one workload as float32 arrays holding exactly representable values."""
    wl: Workload
    q: np.ndarray          # [B][Hq][128]
    k: np.ndarray          # [B][Hkv][T][128]
    v: np.ndarray          # [B][Hkv][T][128]
    k_cal: np.ndarray      # [Hkv][Ncal][128]
    v_cal: np.ndarray      # [Hkv][Ncal][128]
    channels: np.ndarray   # [Hkv][4]


def make_cpu_case(wl: Workload, seed: int, seq_len: Optional[int] = None, n_cal: int = N_CALIB,
                  batch: Optional[int] = None) -> CpuCase:
    """Draw one workload on the CPU.  ``seq_len``/``batch`` override for reduced cases."""
    T = wl.seq_len if seq_len is None else seq_len
    B = wl.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(seed))
    ch = outlier_channels(seed, wl.num_kv_heads)
    k_cal = keys_numpy(rng, (wl.num_kv_heads, n_cal, HEAD_DIM), ch, wl.dtype)
    v_cal = normal_numpy(rng, (wl.num_kv_heads, n_cal, HEAD_DIM), wl.dtype)
    k = keys_numpy(rng, (B, wl.num_kv_heads, T, HEAD_DIM), ch, wl.dtype)
    v = normal_numpy(rng, (B, wl.num_kv_heads, T, HEAD_DIM), wl.dtype)
    q = normal_numpy(rng, (B, wl.num_q_heads, HEAD_DIM), wl.dtype)
    return CpuCase(wl, q, k, v, k_cal, v_cal, ch)


def kmeans_init_indices(seed: int, n_points: int, entries: int) -> np.ndarray:
    """Forgy initialisation: ``entries`` distinct point indices drawn without replacement."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x1A1A))
    return np.sort(rng.choice(n_points, size=entries, replace=False)).astype(np.int64)


def random_codes(seed: int, shape, entries: int) -> np.ndarray:
    """Uniform code indices in [0, entries) as uint16."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0xC0DE))
    return rng.integers(0, entries, size=shape, dtype=np.uint16)


def random_fp16_book(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """A codebook of N(0, scale^2) entries stored as float16 bit patterns (uint16)."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0xB00C))
    return (rng.standard_normal(shape) * scale).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------- torch (device) side

def _torch_gen(device, seed: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def keys_torch(gen, shape, channels: np.ndarray, dtype, device, chunk_heads: bool = True):
    """Device keys [B][Hkv][T][128] in ``dtype``; drawn per (b, h) slice to bound fp32 scratch."""
    import torch
    B, H, T, D = shape
    out = torch.empty(shape, dtype=dtype, device=device)
    mult = torch.ones(H, D, dtype=torch.float32, device=device)
    for h in range(H):
        mult[h, torch.as_tensor(channels[h], device=device)] = OUTLIER_SCALE
    for b in range(B):
        for h in range(H):
            x = torch.randn((T, D), generator=gen, dtype=torch.float32, device=device)
            x.mul_(mult[h])
            out[b, h].copy_(x)
    return out


def normal_torch(gen, shape, dtype, device):
    import torch
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    rows = flat.shape[0]
    step = max(1, (1 << 26) // flat.shape[1])
    for r in range(0, rows, step):
        n = min(step, rows - r)
        flat[r:r + n].copy_(torch.randn((n, flat.shape[1]), generator=gen, dtype=torch.float32, device=device))
    return out


def make_device_case(wl: Workload, seed: int, device, seq_len: Optional[int] = None,
                     n_cal: int = N_CALIB, batch: Optional[int] = None):
    """Draw one workload directly on ``device``; returns a dict of tensors plus outlier channels."""
    import torch
    T = wl.seq_len if seq_len is None else seq_len
    B = wl.batch if batch is None else batch
    dt = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
    gen = _torch_gen(device, seed)
    ch = outlier_channels(seed, wl.num_kv_heads)
    k_cal = keys_torch(gen, (1, wl.num_kv_heads, n_cal, HEAD_DIM), ch, dt, device)[0]
    v_cal = normal_torch(gen, (wl.num_kv_heads, n_cal, HEAD_DIM), dt, device)
    k = keys_torch(gen, (B, wl.num_kv_heads, T, HEAD_DIM), ch, dt, device)
    v = normal_torch(gen, (B, wl.num_kv_heads, T, HEAD_DIM), dt, device)
    q = normal_torch(gen, (B, wl.num_q_heads, HEAD_DIM), dt, device)
    return dict(q=q, k=k, v=v, k_cal=k_cal, v_cal=v_cal, channels=ch)
