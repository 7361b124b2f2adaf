"""fp64 oracle of the retriever's query encoder: hidden states -> indexer queries q and weights w.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP library.

What it computes follows the FlashMemory-DeepSeek-V4 repository page, section "Retriever
architecture" (the per-layer pipeline) and its "Hyperparameters" table, written out in the
order the page lists the steps, all in fp64 from the exact values of the bf16 inputs:

    a = hidden . wq_a^T                       wq_a    [q_rank, d_model]   (a Linear: out x in)
    r = RMSNorm(a) = a / sqrt(mean(a^2) + eps) * q_norm
    b = r . wq_b^T                            wq_b    [n_heads * head_dim, q_rank]
    x = b reshaped to [n_heads, head_dim]
    x[..., head_dim - rope_dim:] rotated by YaRN RoPE at the row's position
    q = normalised Walsh-Hadamard transform of x over head_dim
    w = (hidden . w_proj^T) * head_dim^-0.5 * n_heads^-0.5      w_proj [n_heads, d_model]

Readings where the page leaves a step open (each also listed in the design notes):
  * weights are Linear weights, [out, in] row-major, applied as x . W^T;
  * RoPE rotates consecutive pairs (2i, 2i + 1) of the rope dimensions by pos * theta_i;
  * YaRN: theta_i = base^(-2i / rope_dim), blended towards theta_i / factor by the linear ramp
    between the correction dimensions of beta_fast and beta_slow, as the YaRN paper defines
    them (Peng et al., "YaRN: Efficient Context Window Extension of Large Language Models",
    the "NTK-by-parts" interpolation); no attention-temperature factor is applied;
  * the Hadamard matrix is Sylvester's (natural order), scaled by 1 / sqrt(head_dim);
  * "x weight_scale" multiplies the projected weights by head_dim^-0.5 * n_heads^-0.5.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """A bf16 value is the float32 whose upper 16 bits are the code (lower bits zero)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rms_norm(a: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: a / sqrt(mean(a^2) + eps), then times the weight g."""
    ms = np.mean(a * a, axis=-1, keepdims=True)
    return a / np.sqrt(ms + eps) * g


def yarn_inv_freq(rope_dim: int, base: float, factor: float, orig_len: int,
                  beta_fast: float, beta_slow: float) -> np.ndarray:
    """Per-pair angular frequency theta_i (i < rope_dim / 2) of YaRN RoPE.

    The correction dimension of a rotation count beta is the pair index whose wavelength fits
    beta times into the original context: d * ln(orig / (2 pi beta)) / (2 ln base).  Pairs below
    the fast one keep theta_i, pairs above the slow one take theta_i / factor, and the ramp
    between them (linear in the pair index) blends the two.
    """
    half = rope_dim // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / rope_dim)
    if factor == 1.0:
        return theta

    def corr_dim(beta):
        return rope_dim * math.log(orig_len / (beta * 2.0 * math.pi)) / (2.0 * math.log(base))

    low = max(math.floor(corr_dim(beta_fast)), 0)
    high = min(math.ceil(corr_dim(beta_slow)), half - 1)
    if high == low:
        high = low + 0.001
    ramp = np.clip((i - low) / (high - low), 0.0, 1.0)
    return theta / factor * ramp + theta * (1.0 - ramp)


def rope(x: np.ndarray, pos: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotate consecutive pairs of the last axis of x [T, ..., 2 P] by pos[t] * inv_freq[p]."""
    out = np.array(x, dtype=np.float64, copy=True)
    ang = np.asarray(pos, np.float64).reshape((-1,) + (1,) * (x.ndim - 1)) * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order n (a power of two): H_2m = [[H, H], [H, -H]]."""
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n, "n must be a power of two"
    return H


def hadamard(x: np.ndarray) -> np.ndarray:
    """Normalised Walsh-Hadamard transform over the last axis: x . H / sqrt(n)."""
    n = x.shape[-1]
    return x @ hadamard_matrix(n) / math.sqrt(n)


def encode(hidden, pos, wq_a, q_norm, wq_b, w_proj, *, n_heads: int, head_dim: int = 128,
           rope_dim: int = 64, eps: float = 1e-6, rope_base: float = 160000.0,
           rope_factor: float = 16.0, rope_orig_len: int = 65536, beta_fast: float = 32.0,
           beta_slow: float = 1.0):
    """Queries q [T, n_heads, head_dim] and weights w [T, n_heads], fp64.

    Every matrix argument is either fp64 values or bf16 codes (uint16), decoded exactly.
    """
    def val(a):
        a = np.asarray(a)
        return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    h, Wa, g, Wb, Wp = val(hidden), val(wq_a), val(q_norm), val(wq_b), val(w_proj)
    T = h.shape[0]
    a = h @ Wa.T
    r = rms_norm(a, g, eps)
    x = (r @ Wb.T).reshape(T, n_heads, head_dim)
    if rope_dim:
        inv = yarn_inv_freq(rope_dim, rope_base, rope_factor, rope_orig_len, beta_fast, beta_slow)
        x[..., head_dim - rope_dim:] = rope(x[..., head_dim - rope_dim:],
                                            np.asarray(pos, np.float64), inv)
    q = hadamard(x)
    w = (h @ Wp.T) * (head_dim ** -0.5) * (n_heads ** -0.5)
    return q, w
