"""Seeded synthetic inputs (counter-based), shared by tests, bench and smoke.

Holds none of the method's arithmetic: it only draws numbers.  Each value is a
function of (seed, tag, element index) alone, so any slice can be generated
on any device without generating the rest.  The generator is splitmix64
(Steele, Lea, Flood, 2014) used as a counter-based stream: draw n of stream
(seed, tag) is the splitmix64 mix of state0 + n * golden_gamma; normals come
from Box-Muller over two draws.

The shapes and value statistics follow the workloads the pages describe
(they measure on real cached activations, which are not available here):
K channel-RMS outliers, planted high-norm sink rows, log-uniform channel
spread, AR(1) channel correlation.
"""

import math

import torch

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB


def _s64(x):
    x &= (1 << 64) - 1
    return x - (1 << 64) if x >= (1 << 63) else x


def _srl(x, k):
    """Logical right shift of int64 tensors."""
    return (x >> k) & ((1 << (64 - k)) - 1)


def _mix(z):
    z = (z ^ _srl(z, 30)) * _s64(M1)
    z = (z ^ _srl(z, 27)) * _s64(M2)
    return z ^ _srl(z, 31)


def _state0(seed, tag):
    return _s64((seed * 0x632BE59BD9B4E019 + tag * 0xD1B54A32D192ED03) & ((1 << 64) - 1))


def uniform(n, seed, tag, device="cpu", offset=0):
    """n draws in (0, 1) as float64."""
    idx = torch.arange(offset, offset + n, dtype=torch.int64, device=device)
    z = _mix(_state0(seed, tag) + (idx + 1) * _s64(GAMMA))
    return (_srl(z, 11).to(torch.float64) + 0.5) * 2.0 ** -53


def normal(shape, seed, tag, device="cpu"):
    n = math.prod(shape)
    u1 = uniform(n, seed, tag * 2 + 1, device)
    u2 = uniform(n, seed, tag * 2 + 2, device)
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)
    return z.reshape(shape)


# ---- workload shapers ------------------------------------------------------------------------

def channel_multipliers(n_kv_heads, head_dim, spread, seed, tag, device="cpu"):
    """Per (KV head, channel) RMS multipliers spread**u, u ~ U(0, 1)."""
    u = uniform(n_kv_heads * head_dim, seed, tag, device).reshape(n_kv_heads, head_dim)
    return spread ** u


def q2k_multipliers(n_kv_heads, head_dim, seed, tag, device="cpu", lo=5.8, hi=74.9):
    """Per KV head spread S ~ log-uniform[lo, hi]; channel multipliers S**u with one channel at 1 and one at S."""
    us = uniform(n_kv_heads, seed, tag, device)
    S = torch.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * us)
    u = uniform(n_kv_heads * head_dim, seed, tag + 1, device).reshape(n_kv_heads, head_dim)
    pick = (uniform(2 * n_kv_heads, seed, tag + 2, device).reshape(n_kv_heads, 2) * head_dim).long()
    pick[:, 1] = torch.where(pick[:, 1] == pick[:, 0], (pick[:, 0] + 1) % head_dim, pick[:, 1])
    ar = torch.arange(n_kv_heads, device=device)
    u[ar, pick[:, 0]] = 0.0
    u[ar, pick[:, 1]] = 1.0
    return S[:, None] ** u


def ar1(shape, rho, seed, tag, device="cpu"):
    """AR(1) over the last axis: x_0 ~ N(0, 1), x_c = rho x_{c-1} + sqrt(1 - rho^2) eps_c."""
    e = normal(shape, seed, tag, device)
    out = torch.empty_like(e)
    out[..., 0] = e[..., 0]
    a = math.sqrt(1.0 - rho * rho)
    for c in range(1, shape[-1]):
        out[..., c] = rho * out[..., c - 1] + a * e[..., c]
    return out


def planted_positions(batch, n_sink, length, seed, tag, device="cpu"):
    """n_sink distinct positions per batch element, uniform in [0, length)."""
    out = []
    for b in range(batch):
        u = uniform(4 * n_sink + 16, seed, tag * 1000 + b, device).cpu()
        pos = []
        for x in u.tolist():
            p = int(x * length)
            if p not in pos:
                pos.append(p)
            if len(pos) == n_sink:
                break
        out.append(sorted(pos))
    return out
