"""Seeded synthetic Q/K/V for the sparse-attention workloads.

The generator is shared by the GPU path, the CPU oracle's tests and the
benchmark so that both sides see the same bytes.  It draws random numbers and
shapes them into the value models below; it computes no part of the method.

Value models
  iid  Q, K, V ~ N(0, 1) independently per element.
  grf  One smooth Gaussian random field F per (batch, head) on the unpadded
       latent grid, Q = F + sqrt(0.5) * e_q, K = F + sqrt(0.5) * e_k with
       e_q, e_k ~ N(0, 1), and V ~ N(0, 1).  F is white noise filtered
       circularly along each grid axis with g(x) ~ exp(-x^2 / l^2),
       |x| <= ceil(3 l), scaled so that sum g^2 = 1: F has unit variance and
       correlation exp(-r^2 / (2 l^2)) at lag r along an axis.
Text tokens (when present) are i.i.d. N(0, 1) for Q, K and V, drawn after all
video tokens.

Draw order, for reproducibility: for each batch b, for each head h:
  iid: Q, K, V (each T*Hs*Ws*d values);
  grf: white noise of F, e_q, e_k, V;
then text Q, K, V of shape [B, H, n_text, d].
The torch generator is seeded with 1000 + config id and lives on the device
the tensors are made on, so the bytes depend on that device type; every
comparison uses one generated set on both sides.
"""
import hashlib
import math

import torch


def _axis_kernel(length: float, device) -> torch.Tensor:
    r = int(math.ceil(3.0 * length))
    x = torch.arange(-r, r + 1, dtype=torch.float64)
    g = torch.exp(-(x * x) / (length * length))
    g = g / torch.sqrt((g * g).sum())
    return g.to(device=device, dtype=torch.float32)


def _smooth(white: torch.Tensor, axis: int, length: float) -> torch.Tensor:
    """Circular convolution of `white` along `axis` with the axis kernel."""
    if length <= 0:
        return white
    g = _axis_kernel(length, white.device)
    r = (g.numel() - 1) // 2
    out = torch.zeros_like(white)
    for i in range(g.numel()):
        out.add_(torch.roll(white, shifts=i - r, dims=axis), alpha=float(g[i]))
    return out


def make_qkv(cfg, device="cpu", dtype=None, B=None, H=None):
    """Return (q, k, v), each [B, H, N + n_text, d], raster token order
    n = (t * Hs + h) * Ws + w, text tokens after the video tokens."""
    dev = torch.device(device)
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    if dtype is None:
        dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + cfg.cid)
    T, Hs, Ws, d = cfg.T, cfg.Hs, cfg.Ws, cfg.d
    N = T * Hs * Ws
    L = N + cfg.n_text
    q = torch.empty(B, H, L, d, dtype=dtype, device=dev)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    shape = (T, Hs, Ws, d)

    def normal():
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)

    for b in range(B):
        for h in range(H):
            if cfg.values == "iid":
                qh, kh, vh = normal(), normal(), normal()
            elif cfg.values == "grf":
                f = normal()
                f = _smooth(f, 0, cfg.lt)
                f = _smooth(f, 1, cfg.ls)
                f = _smooth(f, 2, cfg.ls)
                eq, ek = normal(), normal()
                s = math.sqrt(0.5)
                qh = f + s * eq
                kh = f + s * ek
                vh = normal()
            else:
                raise ValueError(f"unknown value model {cfg.values!r}")
            q[b, h, :N] = qh.reshape(N, d).to(dtype)
            k[b, h, :N] = kh.reshape(N, d).to(dtype)
            v[b, h, :N] = vh.reshape(N, d).to(dtype)
    if cfg.n_text:
        tshape = (B, H, cfg.n_text, d)
        for dst in (q, k, v):
            dst[:, :, N:] = torch.randn(tshape, generator=gen, device=dev,
                                        dtype=torch.float32).to(dtype)
    return q, k, v


def random_tensor(shape, seed, device="cpu", dtype=torch.float32):
    """Plain N(0, 1) tensor from its own seeded generator (small test cases)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=dev,
                       dtype=torch.float32).to(dtype)


def sha256(t: torch.Tensor) -> str:
    """Hex digest of a tensor's bytes (logged beside each measurement)."""
    a = t.detach().contiguous().cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return hashlib.sha256(a.numpy().tobytes()).hexdigest()
