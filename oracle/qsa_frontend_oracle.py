"""Plain CPU oracle for the QSA indexer front end (hidden states -> int8 indexer
query and keys).

TEST INFRASTRUCTURE ONLY, like qsa_oracle: only the tests (and the benchmark's
CPU leg) use it; it shares nothing with the HIP library.  float64 throughout.

Source: [PR53896] "PR #53896 完整报告" (prhub.com.cn report on vLLM PR #53896),
section "关键源码片段" (key source snippets), QSAIndexer: the indexer first
projects Q and K from the hidden states (a replicated projection), normalises
them with a Gemma-style RMSNorm and applies a rotary position embedding, 1-D
or MRoPE (apply_qsa_rmsnorm, apply_qsa_rope; the forward slices its positions
as positions[..., :num_tokens], i.e. a leading component axis for MRoPE),
then writes the token K into the raw-key ring and selects with Q.  The pages
name these steps but print none of their formulas, dimensions or the
quantisation of this library's int8 indexer; the readings taken (and listed
in the design notes):

  F1  projection: q = h W_q^T, k = h W_k^T with one weight w_qk [2D, H] (rows
      0..D-1 project q, rows D..2D-1 project k), bf16 inputs, exact products;
  F2  Gemma RMSNorm, per vector of D: y = x / sqrt(mean(x^2) + 1e-6) * (1 + g),
      with its own g for q and for k;
  F3  rotary embedding after the norm, rotate-half layout: for i < D/2,
      angle a = p * base^(-2i/D) at token position p,
      (y_i, y_{i+D/2}) <- (y_i cos a - y_{i+D/2} sin a, y_{i+D/2} cos a + y_i sin a);
  F4  int8: round half to even of x * scale, clamped to [-127, 127] (q and k
      have their own scale);
  F5  MRoPE: a token's position has three components (temporal, height,
      width), positions int [3, T]; the D/2 rotary frequencies are split into
      three contiguous sections of sizes (s_t, s_h, s_w), s_t + s_h + s_w =
      D/2, and frequency i takes its angle from the component of the section
      it lies in: a = p_c * base^(-2i/D), c = 0 for i < s_t, 1 for
      s_t <= i < s_t + s_h, 2 otherwise; the pairs rotate as in F3.  A token
      whose three components are equal (text) is rotated exactly as by F3.
"""
from __future__ import annotations

import numpy as np

RMS_EPS = 1e-6


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (int16/uint16) -> float64, exactly (F1 inputs)."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def project(hidden: np.ndarray, w_qk: np.ndarray, D: int):
    """F1: q = h W_q^T, k = h W_k^T.  hidden [T, H], w_qk [2D, H] (float64)."""
    out = hidden @ w_qk.T
    return out[:, :D], out[:, D:]


def rmsnorm(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    """F2: x / sqrt(mean(x^2) + eps) * (1 + g), per row."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + RMS_EPS) * (1.0 + g)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """F3: rotate pairs (i, i + D/2) by pos * base^(-2i/D)."""
    D = x.shape[-1]
    h = D // 2
    i = np.arange(h, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / D)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :h], x[:, h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def mrope(x: np.ndarray, pos3: np.ndarray, base: float, sections) -> np.ndarray:
    """F5: rotate pairs (i, i + D/2) by p_c * base^(-2i/D), c the section of i."""
    D = x.shape[-1]
    h = D // 2
    s_t, s_h, s_w = (int(v) for v in sections)
    assert s_t + s_h + s_w == h and min(s_t, s_h, s_w) >= 0
    comp = np.array([0] * s_t + [1] * s_h + [2] * s_w)
    pos3 = np.asarray(pos3, dtype=np.float64)
    i = np.arange(h, dtype=np.float64)
    ang = pos3[comp, :].T * base ** (-2.0 * i / D)[None, :]   # [T, D/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :h], x[:, h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """F4: round half to even, clamp to [-127, 127]."""
    return np.clip(np.rint(x * scale), -127, 127).astype(np.int8)


def indexer_frontend(hidden: np.ndarray, positions: np.ndarray, w_qk: np.ndarray, g_q: np.ndarray,
                     g_k: np.ndarray, base: float, q_scale: float, k_scale: float, D: int, prequant: bool = False,
                     mrope_sections=None):
    """hidden [T, H] and w_qk [2D, H] as float64 (or bf16 bits via bf16_bits_to_f64).
    positions [T] (1-D RoPE, F3) or, with mrope_sections (s_t, s_h, s_w), [3, T] (F5).
    Returns (q_index int8 [T, D], keys int8 [T, D]); with prequant also the float64
    values before rounding (x * scale)."""
    q, k = project(hidden, w_qk, D)
    if mrope_sections is None:
        rot = lambda x: rope(x, positions, base)
    else:
        rot = lambda x: mrope(x, positions, base, mrope_sections)
    q = rot(rmsnorm(q, g_q))
    k = rot(rmsnorm(k, g_k))
    if prequant:
        return quantize(q, q_scale), quantize(k, k_scale), q * q_scale, k * k_scale
    return quantize(q, q_scale), quantize(k, k_scale)
