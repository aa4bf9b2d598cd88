"""The 8-bit copy of Phi behind the second pruning stage: its code rule and
bounds, checked over every bfloat16 pattern of the high plane.

The kernels (csrc/k_select.hip) give a high-plane value h (bits hb) the code
c = floor((hb - Q8_HB_OFF) / 16) clamped to [Q8_CMIN, 254] (with Q8_HB_OFF =
the grid base's high half less 16), decode g(c) = the float32 with bits
Q8_BASE + c 2^20 (the sweep: 2^96 times the float32 with bits c 2^20), and
bound Phi, which lies in [h (1 - 2^-24), next(h)), by
  g(c) >= Phi   and   Phi >= Q8_KAPPA g(c) - [code raised to Q8_CMIN] 2^-30.
This reads the constants from the source and checks both bounds, the decode
identity, and that the code sits one grid step above h (the tightest such
code) wherever it was not raised."""
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(__file__), "..", "attention_matching_least_amd", "csrc", "k_select.hip")


def _constants():
    text = open(SRC).read()
    base = re.search(r"constexpr uint32_t Q8_BASE = (\d+)u << (\d+);", text)
    off = re.search(r"constexpr int Q8_HB_OFF = \((\d+) << (\d+)\) - (\d+);", text)
    kap = re.search(r"constexpr float Q8_KAPPA = ([\d.]+)f / ([\d.]+)f;", text)
    cmin = re.search(r"constexpr int Q8_CMIN = (\d+);", text)
    assert base and off and kap and cmin, "8-bit plane constants not found"
    K = int(base.group(1)) << int(base.group(2))
    hb_off = (int(off.group(1)) << int(off.group(2))) - int(off.group(3))
    kappa = float(kap.group(1)) / float(kap.group(2))
    return K, hb_off, kappa, int(cmin.group(1))


def _f32(bits):
    return np.asarray(bits, dtype=np.int64).astype(np.uint32).view(np.float32).astype(np.float64)


def test_q8_bounds_every_bf16_value():
    K, hb_off, kappa, cmin = _constants()
    assert K == (127 - 31) << 23 and hb_off == (K >> 16) - 16 and cmin >= 1
    hb = np.arange(0, 0x7F80, dtype=np.int64)  # every finite non-negative bfloat16
    natural = (np.maximum(hb, hb_off) - hb_off) >> 4
    code = np.minimum(np.maximum(natural, cmin), 254)
    # the kernels' form: clamp hb below at the offset of code cmin, then shift
    assert np.array_equal(code, np.minimum((np.maximum(hb, hb_off + 16 * cmin) - hb_off) >> 4, 254))
    usable = hb < hb_off + 16 * 255  # larger values mark the plane unusable
    hb, code, natural = hb[usable], code[usable], natural[usable]
    h = _f32(hb << 16)
    phi_hi = _f32((hb + 1) << 16)  # Phi < next(h)
    phi_lo = h * (1.0 - 2.0 ** -24)  # Phi >= h (1 - 2^-24)
    up = _f32(K + (code << 20))
    assert np.all(up >= phi_hi)
    raised = natural < cmin
    lower = np.where(raised, kappa * up - 2.0 ** -30, kappa * up)
    assert np.all(lower <= phi_lo)
    # tight: one grid step below the code is at most h
    below = _f32(K + ((code - 1) << 20))
    assert np.all(raised | (below <= h))
    # the sweep's decode: 2^96 times the float32 with bits c 2^20
    assert np.array_equal(up, _f32(code << 20) * 2.0 ** 96)
    # the usable range reaches past 1 (a shifted Phi is at most about 1)
    assert h.max() >= 1.7


def test_q8_kappa_is_the_grid_ratio():
    """Two neighbouring grid values differ by at most 8/9: the constant sits
    just under it (allowing the one-ulp step below g(c - 1))."""
    K, _, kappa, cmin = _constants()
    c = np.arange(cmin, 255)
    ratio = (_f32(K + ((c - 1) << 20) - 1) / _f32(K + (c << 20))).min()
    assert kappa <= ratio < 8.0 / 9.0 + 1e-12
    assert ratio - kappa < 0.01
