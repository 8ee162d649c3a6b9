"""The seeded input generator's roundings, pinned to values fixed by the formats' definitions
(bfloat16: the top 16 bits of binary32, ties to even; IEEE binary16 round-to-nearest-even)."""
import numpy as np

from attention_backward_sdpa_amd import synth


def test_bf16_rounding_pins():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e38, 2.0 ** -133],
                 dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: to even (1.0); 1 + 3*2^-8 -> 1 + 2^-6;
    # 2^-133 is the binary32 subnormal 0x00010000, exact in bf16
    want = [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62, 0x0001]
    got = synth.bf16_bits(x)
    assert [int(v) for v in got] == want
    assert synth.bf16_to_f32(np.array([0x3F82], dtype=np.uint16))[0] == np.float32(1.015625)


def test_fp16_rounding_pins():
    x = np.array([1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -2.5, 65504.0, 2.0 ** -24, 2.0 ** -26],
                 dtype=np.float32)
    # 1 + 2^-11 is a tie between 1 and 1 + 2^-10: to even; 2^-24 is the smallest subnormal; 2^-26
    # rounds to zero
    want = [0x3C00, 0x3C00, 0x3C02, 0xC100, 0x7BFF, 0x0001, 0x0000]
    got = synth.fp16_bits(x)
    assert [int(v) for v in got] == want
    assert synth.fp16_to_f32(np.array([0x3C02], dtype=np.uint16))[0] == np.float32(1.001953125)
    assert synth.bits_to_f32(np.array([0x3C00], dtype=np.uint16), "fp16")[0] == 1.0
    assert synth.bits_to_f32(np.array([0x3F80], dtype=np.uint16), "bf16")[0] == 1.0


def test_draw_inputs_types_share_the_draw():
    w = synth.small_variant(synth.WORKLOADS["mha_s128_d64"], Sq=16, Skv=16)
    a = synth.draw_inputs(w)
    b = synth.draw_inputs(w, dtype="fp16")
    # the same float32 draw, rounded two ways: both within their formats' half-ulp of each other
    fa, fb = synth.bf16_to_f32(a.q), synth.fp16_to_f32(b.q)
    assert np.max(np.abs(fa - fb) / np.maximum(np.abs(fb), 1e-3)) < 2.0 ** -7
