"""CPU checks of the seeded input generator (shared by the oracle and the GPU
path, holding none of the method's arithmetic): the 16-bit roundings are
round-to-nearest-even with the right special values, and the widening back to
float32 is exact."""
import numpy as np

import seeded_inputs as si


def test_bf16_rounding_ties_to_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)                  # bf16 spacing at 1
    x = np.array([one + ulp / 2,                 # tie, even below
                  one + 3 * ulp / 2,             # tie, even above
                  one + ulp / 2 + np.float32(2.0 ** -20),  # above the tie
                  -2.5, 0.0], dtype=np.float32)
    back = si.bf16_bits_to_f32(si.f32_to_bf16_bits(x))
    assert back.tolist() == [1.0, 1.0 + 2 * 2.0 ** -7, 1.0 + 2.0 ** -7, -2.5, 0.0]


def test_fp16_rounding_ties_to_even_and_range():
    ulp = 2.0 ** -10                             # fp16 spacing at 1
    x = np.array([1 + ulp / 2, 1 + 3 * ulp / 2, 65504.0, 65520.0, 2.0 ** -24, 2.0 ** -26,
                  -3.0], dtype=np.float32)
    back = si.f16_bits_to_f32(si.f32_to_f16_bits(x))
    assert back[0] == 1.0 and back[1] == 1 + 2 * ulp
    assert back[2] == 65504.0 and np.isinf(back[3])   # 65520 rounds past the largest half
    assert back[4] == 2.0 ** -24 and back[5] == 0.0   # smallest subnormal; below half of it
    assert back[6] == -3.0


def test_draw_is_exact_in_the_element_type():
    for dt, rt in (("bf16", (si.f32_to_bf16_bits, si.bf16_bits_to_f32)),
                   ("fp16", (si.f32_to_f16_bits, si.f16_bits_to_f32))):
        inp = si.draw_custom(1, 1, 33, 16, dt, seed=5)
        for n in ("Q", "K", "V", "dO"):
            a = getattr(inp, n)
            assert np.array_equal(rt[1](inp.bits[n]), a)      # bits widen to the arrays
            assert np.array_equal(rt[0](a), inp.bits[n])      # and the arrays are representable
    a = si.draw_custom(1, 1, 33, 16, "fp16", seed=5).Q
    b = si.draw_custom(1, 1, 33, 16, "fp16", seed=5).Q
    assert np.array_equal(a, b)                                # seeded
