"""Per-token int8 quantization of Q and K for the int8 QK product (test infrastructure
only).

Source (web page): "H3 SLA Attention", inputs table, use_int8_qk: Q and K are
rounded to int8 row by row, each row with a scale computed from its own values, and
only then multiplied on the attended blocks; the PV product keeps full precision (an
int8 QK product next to a 16-bit PV product).

Reading (the page gives no formula). For each (row, head) vector x of head_dim
float32 values, in float32 arithmetic with correct rounding:
    amax = max_d |x_d|
    s    = fl32(amax / 127)
    x8_d = clamp(rint(fl32(x_d / s)), -127, 127)      (rint: round half to even)
and s = 0, x8 = 0 when amax = 0. The dequantized value is x8_d * s (exact in
float64). Scores then use the dequantized q and k:
    s_ij = scale * s_q,i * s_k,j * sum_d q8_id k8_jd - p_ij,
which is the ordinary score rule on dequantized inputs; v is used as given.
"""
from __future__ import annotations

import numpy as np


def quantize_int8(x32):
    """(x8 int8 [..., d], s float32 [...]) per the reading above; x32 float32 [..., d]."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (x32 / safe[..., None]).astype(np.float32)
    x8 = np.clip(np.rint(r), -127, 127).astype(np.int8)
    x8[s == 0] = 0
    return x8, s


def dequantize_int8(x8, s):
    """float64 x8 * s."""
    return np.asarray(x8, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]


def int8_roundtrip(x):
    """Dequantized per-token int8 image of float32-valued x [..., d], as float64."""
    x8, s = quantize_int8(np.asarray(x, dtype=np.float32))
    return dequantize_int8(x8, s)
