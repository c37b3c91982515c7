"""How much the gate projection's FP32 reduction order matters (reading R2).

The kda.wide page (kernel body, gate-projection block) accumulates
raw_g = BF16(sum_j F_B[f][j] f_a[t][j]) on BF16 MMAs with FP32 accumulators
over 8 K chunks of 16 columns: gate_mode 0 as one chain of eight MMAs,
gate_mode 1 as four chains of two that are then added in order
(((c0 + c1) + c2) + c3).  The oracle and the HIP path both take the sum
exactly (R1, R2: the order is free), so neither mode's order is reproduced.
This test measures, on the record-mode verify workload (B=128, H=32, T=8),
how often each chained FP32 order would round raw_g to a different BF16
value than the exact sum, with the MMA modelled as adding its exact
16-product chunk sum to the accumulator in one FP32 rounding.  It is a
measurement of the reading, not a pin: a 1-ulp raw_g difference changes the
state far beyond the parity tolerance, which is why both sides use the
exact sum.
"""

import numpy as np

from linear_attention_decode_03_amd import inputs
from linear_attention_decode_03_amd.inputs import from_bf16, to_bf16

D = 128


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def gate_orders(p):
    """raw_g as BF16 bits [B*T, H*128] for the exact sum and both chained orders."""
    fa = from_bf16(p["f_a"]).astype(np.float64)           # [B*T, 128]
    fb = from_bf16(p["f_b"]).astype(np.float64)           # [H*128, 128]
    # exact 16-column chunk sums: [8, B*T, H*128] (16 products of 16-bit
    # significands fit a float64 sum exactly at these magnitudes)
    chunks = np.stack([fa[:, 16 * k:16 * k + 16] @ fb[:, 16 * k:16 * k + 16].T
                       for k in range(8)])
    exact = to_bf16(_f32(chunks.sum(axis=0)))
    acc = np.zeros(chunks.shape[1:])
    for k in range(8):                                    # gate_mode 0
        acc = _f32(acc + chunks[k])
    mode0 = to_bf16(acc)
    chain = [_f32(_f32(chunks[2 * c]) + chunks[2 * c + 1]) for c in range(4)]
    value = _f32(_f32(_f32(chain[0] + chain[1]) + chain[2]) + chain[3])
    mode1 = to_bf16(value)
    return exact, mode0, mode1


def test_chained_gate_orders_rarely_change_raw_g():
    p = inputs.make_problem("verify_record_t8")
    exact, mode0, mode1 = gate_orders(p)
    n = exact.size
    d0 = int((mode0 != exact).sum())
    d1 = int((mode1 != exact).sum())
    print(f"raw_g elements {n}: gate_mode 0 order differs from the exact sum at {d0} "
          f"({d0 / n:.3%}), gate_mode 1 at {d1} ({d1 / n:.3%})")
    # Rare, and only where the FP32 chain's rounding (a few 2^-24 of the sum
    # of |chunk sums|) reaches a BF16 rounding boundary: a few ulps apart at
    # most for raw_g near zero after cancellation, one ulp elsewhere.
    ex = from_bf16(exact).astype(np.float64)
    fa = from_bf16(p["f_a"]).astype(np.float64)
    fb = from_bf16(p["f_b"]).astype(np.float64)
    scale = np.abs(fa) @ np.abs(fb).T                      # sum_j |products|
    for m in (mode0, mode1):
        got = from_bf16(m).astype(np.float64)
        big = np.maximum(np.abs(got), np.abs(ex))
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(big, 2.0 ** -126))) - 7)
        assert np.all(np.abs(got - ex) <= np.maximum(ulp, 16 * 2.0 ** -24 * scale))
    assert d0 / n < 0.001 and d1 / n < 0.001
