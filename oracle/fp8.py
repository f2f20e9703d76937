"""Float64 reference for attention over FP8 (E4M3) inputs: test infrastructure
only, like the rest of this package.

Sources: the pranaymahendrakar.com lesson "FlashAttention", Researcher tier,
version lineage table (FlashAttention-3 adds an FP8 forward pass). The pages
give no format or scaling convention; the reading taken here is the OCP 8-bit
floating-point format E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 holds subnormals m/8 * 2^-6; the all-ones exponent with
all-ones mantissa is NaN; no infinities; largest finite 448) with one float
scale per tensor: the real input is code value * descale. What is computed is
then plain attention of the real inputs, so the reference decodes the codes
exactly into float64 and applies the definition in ``oracle.attention``.
"""

import numpy as np

from . import attention as _attention


def e4m3_decode(codes):
    """float64 values of uint8 E4M3 codes (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def forward_fp8(q8, k8, v8, scale, q_descale, k_descale, v_descale, causal=False, heads=None, rows=None,
                window=(-1, -1)):
    """Attention of the real inputs q = decode(q8) * q_descale (likewise k, v):
    o [B, H, R, d] and lse [B, H, R] as ``oracle.attention.forward``."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    v = e4m3_decode(v8) * float(v_descale)
    return _attention.forward(q, k, v, scale, causal, None, heads=heads, rows=rows, window=window)
