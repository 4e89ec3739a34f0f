"""bf16 weight tensors whose NVFP4 quantisation sits on or next to rounding
ties (inputs only: no quantiser arithmetic here; the expected codes come
from the oracle, which the CPU pins check against exact rationals).

Both tensors are built around one global scale g, from the tensor's largest
magnitude amax (g = amax / 2688, one fp32 division), and put into blocks:

* element ties: a block whose largest magnitude is 6 * e4m3(s) * g (so its
  scale is s) holds, for each midpoint mu between neighbouring e2m1 values,
  bf16 weights at or next to mu * e4m3(s) * g;
* scale ties: blocks whose largest magnitude is at or next to 6 * g * m for
  each midpoint m between neighbouring e4m3 values.

``tie_weights("pow2")``: amax = 21 = 2688 * 2^-7, so g = 2^-7 exactly and
every tie value above is itself a bf16 value (at most 7 significant bits):
exact ties, and one bf16 step either side.

``tie_weights("near")``: amax is chosen among bf16 values in [1/16, 1/4)
so that g (24 significant bits) puts the most element ties within 2^-20
(relative) of a bf16 value; those weights are then within ~2^-24 of a tie
without being on it, where fp32 evaluations of the quotient decide wrongly.
"""
from __future__ import annotations

import numpy as np

# value of the non-negative e4m3 codes 0..0x7E (OCP E4M3: bias 7, subnormal
# step 2^-9) and of the e2m1 magnitudes 0..7 (OCP MX FP4), as grids
E4M3_POS = np.array([(c & 7) * 2.0 ** -9 if (c >> 3) == 0 else
                     (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7) for c in range(0x7F)])
E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MIDS = (E2M1_POS[:-1] + E2M1_POS[1:]) / 2
E4M3_MIDS = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2


def _bf16_bits_near(v: np.ndarray) -> np.ndarray:
    """bit patterns of the bf16 value below-or-at v (v > 0, float64) and of its
    two bf16 neighbours: shape (len(v), 3)."""
    f = v.astype(np.float32)                         # within 2^-24 of v
    b = (f.view(np.uint32) >> 16).astype(np.int64)   # truncation: at most f
    return np.stack([b - 1, b, b + 1], axis=1)


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _global_scale(amax: float) -> float:
    return float(np.float32(amax) / np.float32(2688.0))


def _near_tie_amax() -> float:
    """the bf16 amax in [1/16, 1/4) whose g puts the most element-tie values
    within 2^-20 of a bf16 value without being one (ties broken by the
    smaller amax)"""
    cand = _bf16_value(np.arange(0x3D80, 0x3E80))    # bf16 patterns of [1/16, 1/4)
    best, best_n = None, -1
    prods = (E2M1_MIDS[None, :] * E4M3_POS[1:, None]).ravel()
    for a in cand:
        g = _global_scale(a)
        t = prods * g
        near = _bf16_value(_bf16_bits_near(t)[:, 1])
        rel = np.minimum(np.abs(t - near), np.abs(t - _bf16_value(_bf16_bits_near(t)[:, 2])))
        n = int(np.count_nonzero((rel > 0) & ((rel / t) < 2.0 ** -20)))
        if n > best_n:
            best, best_n = a, n
    return float(best)


def tie_weights(kind: str, K: int = 512):
    """(bf16 bit patterns uint16 [N][K], amax): weights at and next to the
    rounding ties of the quantiser around one global scale."""
    assert K % 16 == 0
    amax = 21.0 if kind == "pow2" else _near_tie_amax()
    g = _global_scale(amax)
    blocks = []
    # element ties: per nonzero scale code, two blocks led by 6 e4m3(s) g
    for s in range(1, 0x7F):
        target = 6 * E4M3_POS[s] * g
        lead = _bf16_bits_near(np.array([target]))[0]
        lead_bits = lead[np.argmin(np.abs(_bf16_value(lead) - target))]      # nearest bf16
        ties = _bf16_bits_near(E2M1_MIDS * E4M3_POS[s] * g).ravel()          # 21 values
        vals = np.concatenate([[lead_bits], ties[:15], [lead_bits], ties[15:],
                               ties[:9] | 0x8000])                             # signed copies
        blocks += [vals[:16], vals[16:32]]
    # scale ties: per e4m3 midpoint, blocks led by the bf16 values next to 6 g m
    lead = _bf16_bits_near(6 * E4M3_MIDS * g).ravel()
    frac = np.arange(16) / 16.0
    for b in lead:
        v = _bf16_value(np.array([b]))[0]
        body = (v * frac).astype(np.float32).view(np.uint32) >> 16
        body[0] = b
        blocks.append(body.astype(np.int64))
    flat = np.concatenate([np.asarray(x, np.int64) for x in blocks])
    per_row = K
    n = -(-flat.size // per_row)
    out = np.zeros(n * per_row, np.int64)
    out[:flat.size] = flat
    bits = out.astype(np.uint16).reshape(n, K)
    mag = _bf16_value(bits.astype(np.int64) & 0x7FFF)
    assert mag.max() == amax, (mag.max(), amax)
    return bits, amax
