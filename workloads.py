"""Seeded synthetic inputs for the five workloads (generation only).

This module holds no step of the codec.  It only draws the raw BF16 / FP8 bits
that both the oracle and the HIP library then consume byte for byte.  The pages
measure real checkpoints and K/V caches, which are not available here.  These
tensors stand in for them with the same shapes and the value distributions named
for each workload:

  c1  BF16 [1024, 1024]      N(0, 0.02) cast round-to-nearest-even, seed 0
  c2  BF16 [4096, 4096]      N(0, 1/sqrt(4096)) cast RNE
  c3  Llama-3-8B-shaped BF16 weight set: 32 layers x {q, k, v, o, gate, up, down}
      + lm_head, each N(0, 1/sqrt(fan_in)), fan_in = input features
  c4  FP8 E4M3FN [8192, 8192]: x ~ N(0,1) in fp32, scale = amax|x| / 448,
      q = e4m3(clamp(x / scale, -448, 448)) (RNE); the fp32 scale is kept raw
  c5  BF16 K/V cache [2, 32, 8, 32768, 128]: 0.5 * Student-t(5); in every
      (kv, layer, head) slab, 4 of the 128 channels (drawn without replacement)
      are multiplied by 20; cast RNE

  low entropy  BF16 [4096, 4096] or FP8 E4M3FN [8192, 8192] whose exponent is one
      value (120 BF16, 7 FP8) with probability 0.85 and otherwise that value minus
      a geometric(0.45) draw (clipped to 40 BF16, 7 FP8), with uniform sign and
      mantissa bits: the skew the pages report for K/V caches and scale factors,
      a mean code length of about 1.3 bits

  fp4 scales  E8M0 block scale factors of MX-FP4 weights: per 32 consecutive
      input features of a N(0, 1/sqrt(fan_in)) weight, the byte
      floor(log2(amax)) - 2 + 127 (2 = the largest exponent of FP4 E2M1),
      clamped to [0, 254]; for the whole Llama-3-8B-shaped set of c3

CPU generation uses numpy's PCG64 seeded with SeedSequence(0, spawn_key=(cfg, i)).
The two big sets (c3: 15 GB, c5: 4.3 GB) are drawn on the GPU with a seeded torch
generator, one tensor or slab at a time.  The values differ from the CPU draw, but
the oracle always reads back the exact bytes the GPU side used.
"""
from __future__ import annotations

import math

import numpy as np
import torch

BF16 = 0
FP8 = 1
E8M0 = 2
MX_BLOCK = 32

C3_LAYERS = 32
C3_SHAPES = {  # name -> (out_features, in_features)
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}
C3_LM_HEAD = (128256, 4096)
C5_SHAPE = (2, 32, 8, 32768, 128)


def _rng(cfg: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=(cfg, idx))))


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (RNE) -> raw bits as int16 (same device)."""
    return x.to(torch.bfloat16).view(torch.int16)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """Raw BF16 bits of a (CPU) tensor as a numpy uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def normal_bf16(shape, std: float, cfg: int, idx: int = 0) -> torch.Tensor:
    """N(0, std) drawn in fp32 on the CPU, cast RNE to bf16; returns int16 bits."""
    g = _rng(cfg, idx)
    x = g.standard_normal(size=int(np.prod(shape)), dtype=np.float32)
    x *= np.float32(std)
    return _bf16_bits(torch.from_numpy(x)).reshape(shape)


def c1() -> torch.Tensor:
    return normal_bf16((1024, 1024), 0.02, cfg=1)


def c2() -> torch.Tensor:
    return normal_bf16((4096, 4096), 1.0 / math.sqrt(4096), cfg=2)


def c3_names():
    """Tensor names in call order: per layer the 7 projections, then the lm_head."""
    names = []
    for layer in range(C3_LAYERS):
        for nm in C3_SHAPES:
            names.append((f"layers.{layer}.{nm}", C3_SHAPES[nm]))
    names.append(("lm_head", C3_LM_HEAD))
    return names


def c3_tensor(index: int, device="cuda") -> torch.Tensor:
    """The index-th tensor of the c3 set (order of c3_names) as int16 bits."""
    name, shape = c3_names()[index]
    fan_in = shape[1]
    g = torch.Generator(device=device)
    g.manual_seed(3_000_000 + index)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(1.0 / math.sqrt(fan_in))
    return _bf16_bits(x)


def c4(device="cpu"):
    """(uint8 e4m3 bits [8192, 8192], fp32 scale)."""
    g = _rng(4)
    x = torch.from_numpy(g.standard_normal(size=8192 * 8192, dtype=np.float32)).reshape(8192, 8192)
    x = x.to(device)
    scale = (x.abs().max() / 448.0).to(torch.float32)
    q = torch.clamp(x / scale, -448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), float(scale.item())


def low_entropy(dtype: int, p_top: float = 0.85, seed: int = 0) -> torch.Tensor:
    """Low-entropy exponents (see the module docstring): BF16 [4096, 4096] as int16
    bits, or FP8 [8192, 8192] as uint8 bits."""
    g = _rng(6 + dtype, seed)
    n = 4096 * 4096 if dtype == BF16 else 8192 * 8192
    top = 120 if dtype == BF16 else 7
    tail = np.clip(g.geometric(0.45, n), 1, 40 if dtype == BF16 else 7)
    e = np.where(g.random(n) < p_top, top, top - tail).astype(np.uint32)
    if dtype == BF16:
        r = g.integers(0, 1 << 16, n, dtype=np.uint32)   # sign bit 15, mantissa bits 0..6
        bits = ((r & 0x807F) | (e << 7)).astype(np.uint16)
        return torch.from_numpy(bits.view(np.int16)).reshape(4096, 4096)
    r = g.integers(0, 1 << 8, n, dtype=np.uint32)        # sign bit 7, mantissa bits 0..2
    bits = ((r & 0x87) | (e << 3)).astype(np.uint8)
    return torch.from_numpy(bits).reshape(8192, 8192)


def c5_outlier_channels() -> np.ndarray:
    """[2, 32, 8, 4] channel indices multiplied by 20 in each slab."""
    g = _rng(5, 1)
    out = np.empty((2, 32, 8, 4), np.int64)
    for kv in range(2):
        for layer in range(32):
            for head in range(8):
                out[kv, layer, head] = g.choice(128, size=4, replace=False)
    return out


def student_t5(shape, gen: torch.Generator, device) -> torch.Tensor:
    """Student-t with 5 degrees of freedom from its definition Z / sqrt(chi2_5 / 5)."""
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    chi2 = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(5):
        w = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        chi2.addcmul_(w, w)
    return z / torch.sqrt(chi2 / 5.0)


def c5_slab(kv: int, layer: int, device="cuda", tokens: int = 32768) -> torch.Tensor:
    """One [8, tokens, 128] (kv, layer) slab of the K/V cache as int16 bits."""
    g = torch.Generator(device=device)
    g.manual_seed(5_000_000 + kv * 32 + layer)
    x = 0.5 * student_t5((8, tokens, 128), g, device)
    ch = torch.from_numpy(c5_outlier_channels()[kv, layer]).to(device)
    for head in range(8):
        x[head][:, ch[head]] *= 20.0
    return _bf16_bits(x)


def c5(device="cuda") -> torch.Tensor:
    """Full [2, 32, 8, 32768, 128] K/V cache bits (int16) on `device`."""
    out = torch.empty(C5_SHAPE, dtype=torch.int16, device=device)
    for kv in range(2):
        for layer in range(32):
            out[kv, layer] = c5_slab(kv, layer, device)
    return out


def mx_scale_bytes(w: torch.Tensor) -> torch.Tensor:
    """E8M0 scale bytes of MX-FP4 blocks of 32 along the last dimension of `w`
    (float32): floor(log2(amax)) - 2 + 127, clamped to [0, 254]; an all-zero
    block gets 0."""
    a = w.abs().reshape(*w.shape[:-1], w.shape[-1] // MX_BLOCK, MX_BLOCK).amax(-1)
    e = torch.floor(torch.log2(torch.where(a > 0, a, torch.ones_like(a)))) - 2 + 127
    e = torch.where(a > 0, e, torch.zeros_like(e))
    return e.clamp(0, 254).to(torch.uint8)


def fp4_scales(out_f: int, in_f: int, idx: int = 0) -> np.ndarray:
    """CPU draw: the scale bytes [out_f, in_f / 32] of one N(0, 1/sqrt(in_f)) weight."""
    g = _rng(6, idx)
    w = g.standard_normal(size=(out_f, in_f), dtype=np.float32) * np.float32(1.0 / math.sqrt(in_f))
    return mx_scale_bytes(torch.from_numpy(w)).numpy()


def fp4_scales_c3(device="cuda") -> torch.Tensor:
    """Scale bytes of every tensor of the c3 set (call order of c3_names), drawn on
    `device` one tensor at a time and concatenated: one uint8 tensor."""
    parts = []
    for index, (name, shape) in enumerate(c3_names()):
        g = torch.Generator(device=device)
        g.manual_seed(6_000_000 + index)
        w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        w.mul_(1.0 / math.sqrt(shape[1]))
        parts.append(mx_scale_bytes(w).reshape(-1))
        del w
    return torch.cat(parts)
