"""YaRN rotary position encoding: plain fp64 CPU reference.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may call it.  It shares no code with the HIP kernels.

"GPT-OSS on day 0" (*model deltas*) says only that the model uses YaRN position
encoding as DeepSeek-V3 does.  The computation below is the published YaRN method
(rotary embedding with "NTK-by-parts" frequency interpolation and an attention
temperature), restated; every choice the pages leave open is a reading:

* rotary frequencies of a head of size D: f_i = theta ** (-2 i / D), i = 0 .. D/2 - 1;
* YaRN interpolation with scale factor s over an original context L: a frequency with
  r_i = L * f_i / (2 pi) full turns over L keeps f_i when r_i >= beta_fast, becomes f_i / s
  when r_i <= beta_slow, and in between mixes the two linearly in
  gamma_i = (r_i - beta_slow) / (beta_fast - beta_slow):  f_i' = (1 - gamma_i) f_i / s +
  gamma_i f_i;
* attention temperature: q and k are each multiplied by m = 0.1 ln(s) + 1 (m = 1 for
  s <= 1);
* rotated vectors are attention inputs and are stored as bfloat16 (as a separate
  rotation pass would write them): ``bf16_round`` rounds to the nearest bfloat16, ties to
  even, so a comparison with attention on rotated inputs can take the same rounding;
* rotation pairs: dimension i with dimension i + D/2 (the "half-split" layout):
  x'_i = m (x_i cos(p f_i') - x_{i+D/2} sin(p f_i')),
  x'_{i+D/2} = m (x_{i+D/2} cos(p f_i') + x_i sin(p f_i')), at integer position p.
"""
from __future__ import annotations

import math

import numpy as np

from .sink_attention import _f64, _i64

__all__ = ["yarn_inv_freq", "yarn_mscale", "apply_rope", "bf16_round"]


def yarn_inv_freq(head_dim: int, theta: float, factor: float, original_max_pos: int,
                  beta_fast: float, beta_slow: float) -> np.ndarray:
    """The D/2 rotary frequencies after YaRN interpolation (float64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    f = theta ** (-2.0 * i / head_dim)
    if factor <= 1.0:
        return f
    r = original_max_pos * f / (2.0 * math.pi)
    gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - gamma) * (f / factor) + gamma * f


def yarn_mscale(factor: float) -> float:
    return 1.0 if factor <= 1.0 else 0.1 * math.log(factor) + 1.0


def apply_rope(x, positions, theta: float, factor: float = 1.0, original_max_pos: int = 4096,
               beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Rotate x [..., D] (any leading shape) at integer positions broadcast over the
    leading axes (positions has the shape of x without its last axis, or broadcasts to
    it).  Returns float64."""
    x = _f64(x)
    d = x.shape[-1]
    pos = _i64(positions).astype(np.float64)
    f = yarn_inv_freq(d, theta, factor, original_max_pos, beta_fast, beta_slow)
    ang = pos[..., None] * f                      # [..., D/2]
    c, s = np.cos(ang), np.sin(ang)
    m = yarn_mscale(factor)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return m * np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties to even;
    returned as float64.  Finite normal inputs only (what the rotation produces)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)   # np.round: half to even
