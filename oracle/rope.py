"""YaRN rotary position encoding and the KV append step, in fp64 (test infrastructure only).

Source page: "GPT-OSS on Day 0", section "GPT-OSS on Hopper": the model encodes positions
with YaRN, as DeepSeek-V3 does; the pages give neither a formula nor parameters. Computed
here is the published YaRN method written out directly:
  * rotary embedding: the pair (x[i], x[i + d/2]) of a head vector at position p is rotated
    by the angle p * f_i, with base frequencies f_i = theta^(-2i/d), i < d/2;
  * YaRN's frequency scaling with factor s > 1 over an original context of L0 positions:
    with r_i = L0 * f_i / (2 pi) (how many turns dimension i makes over L0), a ramp g_i
    keeps fast dimensions (g = 1 where r_i >= beta) and divides slow ones by s (g = 0 where
    r_i <= alpha): f'_i = g_i f_i + (1 - g_i) f_i / s. Two ramp forms share those limits:
      "turns": g_i = clip((r_i - alpha) / (beta - alpha), 0, 1), linear in r_i (the ramp
               function of the YaRN paper);
      "index": g_i linear in the pair index i between the (real) indices where r_i = beta
               and r_i = alpha; since ln r_i is linear in i this is
               g_i = clip(ln(r_i / alpha) / ln(beta / alpha), 0, 1) (the form of released
               YaRN implementations that compute correction dimensions);
  * YaRN's attention temperature: cos and sin are scaled by m = 0.1 ln(s) + 1 for both
    q and k (the logits by m^2); m = 1 when s <= 1.
The pairing (i with i + d/2), the angle sign, the ramp form and every parameter value are
readings stated in the design notes. The ramp's interior is pinned by hand-derived fixtures
(tests/golden/yarn_ramp.json) for both forms.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def yarn_frequencies(head_dim: int, theta: float, factor: float, orig_len: int, alpha: float,
                     beta: float, ramp: str = "turns") -> Tuple[np.ndarray, float]:
    """Per-pair angular frequencies [head_dim // 2] and the temperature m (fp64). ``ramp`` is
    "turns" (linear in r_i) or "index" (linear in the pair index, i.e. in ln r_i)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    f = float(theta) ** (-2.0 * i / head_dim)
    if factor <= 1.0:
        return f, 1.0
    r = orig_len * f / (2.0 * np.pi)
    if ramp == "turns":
        g = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    elif ramp == "index":
        g = np.clip(np.log(r / alpha) / np.log(beta / alpha), 0.0, 1.0)
    else:
        raise ValueError(f"unknown YaRN ramp form {ramp!r}")
    return g * f + (1.0 - g) * f / factor, 0.1 * np.log(factor) + 1.0


def rotate(x: np.ndarray, pos: np.ndarray, freqs: np.ndarray, mscale: float) -> np.ndarray:
    """x [T, H, d], pos [T] -> rotated x (fp64): pair (i, i + d/2) turned by pos * freqs[i], times m."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * freqs[None, :]      # [T, half]
    c = (np.cos(ang) * mscale)[:, None, :]
    s = (np.sin(ang) * mscale)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_append(q, k, v, cu_seqlens_q, kv_lens, page_table, k_cache, v_cache, freqs, mscale):
    """The step before attention for new tokens: sequence b's rows cu[b]:cu[b+1] are its newest
    tokens, at positions kv_lens[b] - Lq_b + t (kv_lens counts them). Returns the rotated q, and
    copies of the caches with the rotated k and the unchanged v of each new token written at
    page page_table[b][p // page_size], slot p % page_size (fp64; untouched slots unchanged)."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    P = k_cache.shape[2]
    pos = np.zeros(int(cu[-1]), dtype=np.int64)
    for b in range(len(kv_lens)):
        n = int(cu[b + 1] - cu[b])
        pos[cu[b]:cu[b + 1]] = int(kv_lens[b]) - n + np.arange(n)
    q_rot = rotate(q, pos, freqs, mscale)
    k_rot = rotate(k, pos, freqs, mscale)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    for b in range(len(kv_lens)):
        for row in range(int(cu[b]), int(cu[b + 1])):
            p = int(pos[row])
            page = int(page_table[b][p // P])
            kc[page, :, p % P, :] = k_rot[row]
            vc[page, :, p % P, :] = v[row]
    return q_rot, kc, vc
