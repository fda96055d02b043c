"""Pins of the oracle's NVFP4 codec against facts fixed outside the oracle.

Sources: "MiniMax-M3.1-Flash serving notes", section "The capacity numbers" (4-bit values with
one FP8 scale per 16 values, 4.5 bits per element, 34,560 vs 61,440 bytes of KV per token);
"vLLM day-0 support for MiniMax-M3.1-Flash", sections "MSA primer" (128 B index vs 1,024 B of
FP8 K/V per token per layer, about 12.5% of the traffic) and "NVFP4 MSA kernel" (256 E4M3
scales times 8 E2M1 magnitudes, a 2 KB table). The E2M1 magnitude set {0, .5, 1, 1.5, 2, 3, 4,
6} is the standard FP4 E2M1 element; the E4M3 byte decoding is checked against torch's
float8_e4m3fn type, an independent implementation of the OCP format.
"""
import math

import numpy as np
import pytest
import torch

import oracle

E2M1_SET = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def torch_e4m3(byte: int) -> float:
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def test_e4m3_decode_exhaustive_vs_torch():
    for b in range(256):
        ref = torch_e4m3(b)
        got = oracle.e4m3_value(b)
        if math.isnan(ref):
            assert math.isnan(got), b
        else:
            assert got == ref, (b, got, ref)


def test_e4m3_landmarks():
    assert oracle.e4m3_value(0x7E) == 448.0          # largest finite
    assert oracle.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x00) == 0.0
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0xB8) == -1.0


def test_e2m1_value_set():
    assert [oracle.e2m1_value(n) for n in range(8)] == E2M1_SET
    assert [oracle.e2m1_value(8 + n) for n in range(8)] == [-v for v in E2M1_SET]
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0  # negative zero keeps its sign


def test_dequant_table_is_2kb_and_exact_in_bf16():
    # 256 scale bytes x 8 magnitudes = 2,048 entries: the 2 KB table at one byte per entry.
    finite_scales = [b for b in range(256) if not math.isnan(oracle.e4m3_value(b))]
    table = [oracle.e2m1_value(m) * oracle.e4m3_value(s) for s in range(256) for m in range(8)]
    assert len(table) == 2048
    # every product of an E2M1 magnitude and a finite E4M3 scale is exact in bf16 and in fp16
    vals = torch.tensor([oracle.e2m1_value(m) * oracle.e4m3_value(s)
                         for s in finite_scales for m in range(8)], dtype=torch.float64)
    assert torch.equal(vals.to(torch.bfloat16).double(), vals)
    assert torch.equal(vals.to(torch.float16).double(), vals)


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(7)
    xs = list(np.exp(rng.uniform(math.log(2.0 ** -12), math.log(448.0), 20000)).astype(np.float32))
    # every midpoint between neighbouring codes, and one float ulp either side
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)
        xs += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    xs += [np.float32(0.0), np.float32(2.0 ** -10), np.float32(448.0)]
    for x in xs:
        x = np.float32(x)
        ref = int(torch.tensor([float(x)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])
        assert oracle.e4m3_encode(float(x)) == ref, (float(x), oracle.e4m3_encode(float(x)), ref)


def test_e4m3_encode_saturates():
    for x in [448.0, 449.0, 464.0, 470.0, 1e6, 3.0e38]:
        assert oracle.e4m3_encode(x) == 0x7E


def test_e2m1_midpoints_round_to_even():
    # exact midpoints of the magnitude grid go to the even code
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for r, code in mids.items():
        assert oracle.e2m1_encode_magnitude(r) == code, r
        below = float(np.nextafter(np.float32(r), np.float32(0)))
        above = float(np.nextafter(np.float32(r), np.float32(100)))
        # one ulp off the midpoint goes to the nearer neighbour
        assert E2M1_SET[oracle.e2m1_encode_magnitude(below)] < r
        assert E2M1_SET[oracle.e2m1_encode_magnitude(above)] > r
    for c, v in enumerate(E2M1_SET):
        assert oracle.e2m1_encode_magnitude(v) == c
    assert oracle.e2m1_encode_magnitude(7.0) == 7 and oracle.e2m1_encode_magnitude(1e30) == 7


def test_quantize_storage_is_4p5_bits_per_element():
    x = np.random.default_rng(0).standard_normal((3, 128)).astype(np.float32)
    codes, scales = oracle.quantize(x)
    per_vector_bytes = codes.shape[-1] + scales.shape[-1]
    assert per_vector_bytes == 72
    assert per_vector_bytes * 8 / 128 == 4.5


def test_quantize_scale_is_rne_of_amax_over_6():
    x = np.random.default_rng(1).standard_normal((64, 128)).astype(np.float32) * 3
    _, scales = oracle.quantize(x)
    amax = np.abs(x.reshape(64, 8, 16)).max(-1)
    s32 = torch.from_numpy((amax / np.float32(6.0)).astype(np.float32))
    ref = s32.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)


def test_quantize_error_bound_and_nearest_code():
    x = np.random.default_rng(2).standard_normal((256, 128)).astype(np.float32)
    codes, scales = oracle.quantize(x)
    deq = oracle.dequantize(codes, scales)
    s = np.repeat(np.array([[oracle.e4m3_value(b) for b in row] for row in scales]), 16, axis=1)
    r = np.abs(x.astype(np.float64)) / s
    grid = np.array(E2M1_SET)
    # the chosen magnitude is a nearest grid point of r (within fp32 rounding of the quotient)
    best = np.min(np.abs(r[..., None] - grid), axis=-1)
    assert np.all(np.abs(np.abs(deq) / s - r) <= best + 1e-6)
    # signs follow x
    assert np.all((deq == 0) | (np.sign(deq) == np.sign(x)))


def test_quantize_idempotent_on_representable_vectors():
    rng = np.random.default_rng(3)
    for _ in range(200):
        sc = int(rng.integers(1, 0x7F))              # any finite non-zero scale
        mags = rng.integers(0, 8, 16)
        mags[rng.integers(0, 16)] = 7                # amax = 6 * scale exactly
        signs = rng.integers(0, 2, 16)
        nib = (signs << 3 | mags).astype(np.uint8)
        x = np.array([oracle.e2m1_value(int(n)) * oracle.e4m3_value(sc) for n in nib], np.float32)
        codes, scales = oracle.quantize(np.tile(x, 8)[None, :])
        assert int(scales[0, 0]) == sc
        got = np.array([(codes[0, i // 2] >> (4 * (i % 2))) & 15 for i in range(16)], np.uint8)
        assert np.array_equal(got, nib)


def test_quantize_zero_tiny_and_saturating_groups():
    x = np.zeros((1, 128), np.float32)
    x[0, 16:32] = -0.0
    x[0, 32:48] = np.float32(2.0 ** -12)     # amax/6 rounds to a zero scale
    x[0, 48:64] = np.float32(1e4)            # amax/6 > 448: scale saturates
    x[0, 50] = -np.float32(2e4)
    codes, scales = oracle.quantize(x)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[0, 2] == 0
    assert np.all(codes[0, 0:8] == 0)
    assert np.all(codes[0, 8:16] == 0x88)    # negative zero keeps its sign bit
    assert np.all(codes[0, 16:24] == 0)
    assert scales[0, 3] == 0x7E
    deq = oracle.dequantize(codes, scales)
    assert deq[0, 50] == -6 * 448.0 and deq[0, 48] == 6 * 448.0


def test_quantize_is_elementwise_per_group_and_layout():
    # element 2i is the low nibble of byte i; scale g covers elements 16g..16g+15
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 6.0
    x[0, 1] = -3.0
    x[0, 127] = 0.5
    codes, scales = oracle.quantize(x)
    assert scales[0, 0] == 0x38 and codes[0, 0] == (7 | (13 << 4))
    assert oracle.e4m3_value(int(scales[0, 7])) * 6 == pytest.approx(0.5, rel=0.07)
    assert codes[0, 63] >> 4 == 7 and codes[0, 63] & 15 == 0


def test_byte_model_of_the_pages():
    vec = 72                                   # one 128-element NVFP4 vector
    kv_per_token_layer = 2 * 4 * vec          # K and V, 4 KV heads
    assert kv_per_token_layer == 576
    assert kv_per_token_layer * 60 == 34560   # 60 layers: NVFP4 KV bytes per token
    assert 2 * 4 * 128 * 60 == 61440          # the same in FP8
    assert 1 - 34560 / 61440 == 0.4375        # 43.75% less
    assert 128 / 1024 == 0.125                # FP8 index key vs FP8 K/V per token per layer
    assert vec / kv_per_token_layer == 0.125  # the same ratio holds in NVFP4
