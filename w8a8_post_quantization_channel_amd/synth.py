"""Seeded synthetic inputs for the W8A8 layer workloads.

This module only draws inputs; it holds none of the method's arithmetic. Both
the GPU path (tests, bench) and the CPU oracle's checks consume what it
returns. Inputs stand in for real LLM activations and weights, which are not
available: Gaussian (or Student-t) activations with a seeded set of outlier
input channels scaled as whole columns (the outliers are systematic per
channel, kwkr.cn blog §1.1), Gaussian weights.

Every array is drawn with numpy's PCG64 generator in float32 and, for bf16
workloads, rounded to bf16 with round-to-nearest-even (returned as uint16 bit
patterns). `to_torch` turns those into torch tensors on a device.

Workloads (the shapes are those of Llama-2 projections):
  C1  one fp32 layer: X[16,1024] ~ N(0,1)*5 with input channel 50 set to
      100.0, W[2048,1024] ~ N(0,1); calibration on the same X.
  C2  13B prefill projections, M = 2048 tokens: qkvo 5120x5120, gate/up
      13824x5120, down 5120x13824; N(0,1) activations with round(0.003 K)
      outlier channels scaled by U(20,100); W ~ N(0, 0.02); calibration over
      512 sequences x 512 tokens in 16 chunks.
  C3  7B decode, M in {1, 8, 16, 64}: 4096x4096, 11008x4096, 4096x11008.
  C4  alpha search, K=4096 -> N=11008: 8 batches x 2048 tokens of Student-t
      (nu = 3) activations with 12 channels x50.
  C5  70B prefill, M = 4096: 8192x8192, 1024x8192, 28672x8192, 8192x28672.
"""
from __future__ import annotations

import numpy as np

OUTLIER_FRACTION = 0.003

# (name, N, K) per projection shape id
SHAPES_13B = [("qkvo", 5120, 5120), ("gate_up", 13824, 5120), ("down", 5120, 13824)]
SHAPES_7B = [("qkvo", 4096, 4096), ("gate_up", 11008, 4096), ("down", 4096, 11008)]
SHAPES_70B = [("q_o", 8192, 8192), ("k_v", 1024, 8192), ("gate_up", 28672, 8192), ("down", 8192, 28672)]
# 13B layer: projection name -> shape id (q/k/v/o share shape 0, gate/up shape 1)
LAYER_13B = [("q", 0), ("k", 0), ("v", 0), ("o", 0), ("gate", 1), ("up", 1), ("down", 2)]
DECODE_M = (1, 8, 16, 64)
ALPHA_GRID = (0.25, 0.5, 0.75, 1.0)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 to bf16, nearest-even; returns uint16 bit patterns."""
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def n_outliers(k: int) -> int:
    return int(round(OUTLIER_FRACTION * k))


def outlier_channels(seed: int, k: int, count: int | None = None, lo: float = 20.0, hi: float = 100.0,
                     fixed: float | None = None):
    """Seeded outlier channel set: (indices, per-channel factors)."""
    g = rng(seed)
    count = n_outliers(k) if count is None else count
    idx = np.sort(g.choice(k, size=count, replace=False))
    fac = np.full(count, fixed, np.float32) if fixed is not None else g.uniform(lo, hi, count).astype(np.float32)
    return idx, fac


def activations(seed: int, rows: int, k: int, outliers=None, dist: str = "normal", scale: float = 1.0,
                bf16: bool = True) -> np.ndarray:
    """[rows, k] activations; outlier columns multiplied by their factors."""
    g = rng(seed)
    if dist == "normal":
        x = g.standard_normal((rows, k), dtype=np.float32)
    elif dist == "t3":
        x = g.standard_t(3, size=(rows, k)).astype(np.float32)
    else:
        raise ValueError(dist)
    if scale != 1.0:
        x *= np.float32(scale)
    if outliers is not None:
        idx, fac = outliers
        x[:, idx] *= fac[None, :]
    return to_bf16_bits(x) if bf16 else x


def weights(seed: int, n: int, k: int, std: float = 0.02, bf16: bool = True) -> np.ndarray:
    g = rng(seed)
    w = g.standard_normal((n, k), dtype=np.float32)
    if std != 1.0:
        w *= np.float32(std)
    return to_bf16_bits(w) if bf16 else w


# ---- named workloads --------------------------------------------------------

def c1():
    """Single fp32 layer (the tbr8.org example's shapes): X, W (fp32)."""
    g = rng(101)
    x = (g.standard_normal((16, 1024), dtype=np.float32) * np.float32(5.0)).astype(np.float32)
    x[:, 50] = 100.0
    w = g.standard_normal((2048, 1024), dtype=np.float32)
    return x, w


# One 13B decoder layer: four distinct projection inputs (q/k/v share the
# attention input, gate/up the MLP input) and seven weights.
# group name -> (K, outlier seed, activation seed)
C2_GROUPS = {"attn_in": (5120, 2000, 2200), "mlp_in": (5120, 2001, 2201), "mlp_mid": (13824, 2002, 2202),
             "attn_out": (5120, 2003, 2203)}
# (projection, input group, N, K, weight seed)
C2_PROJECTIONS = [("q", "attn_in", 5120, 5120, 2310), ("k", "attn_in", 5120, 5120, 2311),
                  ("v", "attn_in", 5120, 5120, 2312), ("o", "attn_out", 5120, 5120, 2313),
                  ("gate", "mlp_in", 13824, 5120, 2314), ("up", "mlp_in", 13824, 5120, 2315),
                  ("down", "mlp_mid", 5120, 13824, 2316)]
C2_TOKENS = 2048


def c2_group_x(group: str, rows: int = C2_TOKENS):
    k, oseed, xseed = C2_GROUPS[group]
    return activations(xseed, rows, k, outlier_channels(oseed, k))


def c2_projection_w(name: str):
    for p, _, n, k, seed in C2_PROJECTIONS:
        if p == name:
            return weights(seed, n, k)
    raise KeyError(name)


def c2_outliers(shape_id: int):
    k = SHAPES_13B[shape_id][2]
    return outlier_channels(2000 + shape_id, k)


def c2_calib_chunk(shape_id: int, chunk: int, rows: int = 16384):
    """One of the 16 calibration chunks (512 x 512 tokens in total)."""
    k = SHAPES_13B[shape_id][2]
    return activations(2100 + 16 * shape_id + chunk, rows, k, c2_outliers(shape_id))


def c2_runtime_x(shape_id: int, rows: int = 2048):
    k = SHAPES_13B[shape_id][2]
    return activations(2200 + shape_id, rows, k, c2_outliers(shape_id))


def c2_weight(shape_id: int):
    _, n, k = SHAPES_13B[shape_id]
    return weights(2300 + shape_id, n, k)


def c3_outliers(shape_id: int):
    return outlier_channels(3000 + shape_id, SHAPES_7B[shape_id][2])


def c4_batches(n_batches: int = 8, rows: int = 2048, k: int = 4096):
    out = outlier_channels(4000, k, count=12, fixed=50.0)
    return [activations(4001 + b, rows, k, out, dist="t3") for b in range(n_batches)]


def c4_weight(n: int = 11008, k: int = 4096):
    return weights(4100, n, k)


def c5_outliers(shape_id: int):
    return outlier_channels(5000 + shape_id, SHAPES_70B[shape_id][2])


# ---- device-side generation (large calibration sets) -------------------------

def device_activations(seed: int, rows: int, k: int, outliers, device, dist: str = "normal"):
    """[rows, k] bf16 activations drawn on the GPU with torch's seeded
    generator (used where host generation of gigabytes would dominate a run).
    The host copy of the result is what any CPU check consumes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((rows, k), generator=g, device=device, dtype=torch.float32)
    if dist == "t3":
        raise NotImplementedError("device draws are Gaussian only")
    if outliers is not None:
        idx, fac = outliers
        x[:, torch.as_tensor(idx, device=device)] *= torch.as_tensor(fac, device=device)
    return x.to(torch.bfloat16)


def to_torch(a: np.ndarray, device):
    """numpy -> torch on `device`; uint16 arrays are bf16 bit patterns."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_torch(t) -> np.ndarray:
    """torch -> numpy on the host; bf16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
