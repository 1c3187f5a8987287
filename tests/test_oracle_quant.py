"""Pins for the fp8 latent-cache encoder: byte layout, the block maximum
landing on +-448, the e4m3 round-trip error bound, zero blocks, and the
encoder agreeing with torch's float8_e4m3fn cast of the same fp32 quotients."""

import numpy as np
import torch

from oracle import quant as Q
from oracle.formats import e4m3_decode


def _bf16_bits(n, seed=0, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(n, 576, generator=g) * scale).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16), x.to(torch.float64).numpy()


def test_layout_and_block_max():
    bits, x = _bf16_bits(33)
    raw = Q.quantize_k_cache(bits)
    assert raw.shape == (33, 656)
    scales = raw[:, 512:528].copy().view("<f4")
    for b in range(4):
        amax = np.abs(x[:, b * 128:(b + 1) * 128]).max(1).astype(np.float32)
        np.testing.assert_array_equal(scales[:, b], amax / np.float32(448))
        codes = raw[:, b * 128:(b + 1) * 128]
        # the element of largest magnitude encodes as +-448
        j = np.abs(x[:, b * 128:(b + 1) * 128]).argmax(1)
        top = codes[np.arange(33), j]
        assert ((top & 0x7F) == 0x7E).all()
    # rope copied bit for bit
    np.testing.assert_array_equal(raw[:, 528:].copy().view("<u2"), bits[:, 512:])


def test_round_trip_error_bound():
    bits, x = _bf16_bits(64, seed=1, scale=3.0)
    raw = Q.quantize_k_cache(bits)
    y = Q.dequantize_rows(raw)
    np.testing.assert_array_equal(y[:, 512:], x[:, 512:])
    scales = np.repeat(raw[:, 512:528].copy().view("<f4").astype(np.float64), 128, 1)
    err = np.abs(y[:, :512] - x[:, :512])
    # half a unit in the last place: 2^-4 relative for normals, and half the
    # subnormal spacing (2^-10 of the scale) below 2^-6 * scale; plus the fp32
    # rounding of the quotient
    bound = np.maximum(np.abs(x[:, :512]) * 2.0 ** -4, scales * 2.0 ** -10) * (1 + 1e-6)
    assert (err <= bound).all()


def test_zero_block_and_matches_torch_cast():
    bits, x = _bf16_bits(8, seed=2)
    bits = bits.copy()
    bits[0, 128:256] = 0
    raw = Q.quantize_k_cache(bits)
    assert (raw[0, 128:256] == 0).all()
    assert raw[0, 512 + 4:512 + 8].copy().view("<f4")[0] == 1.0
    xf = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float32)
    for b in range(4):
        blk = xf[:, b * 128:(b + 1) * 128]
        amax = blk.abs().amax(1)
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
        ref = (blk / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(raw[:, b * 128:(b + 1) * 128], ref)


def test_decode_values():
    raw = np.zeros((1, 656), np.uint8)
    raw[0, 0] = 0x38                      # 1.0
    raw[0, 200] = 0xC0                    # -2.0
    raw[0, 512:528] = np.array([2.0, 0.5, 1.0, 4.0], "<f4").view(np.uint8)
    raw[0, 528:530] = np.array([0x3F80], "<u2").view(np.uint8)   # bf16 1.0
    y = Q.dequantize_rows(raw)[0]
    assert y[0] == 2.0 and y[200] == -1.0 and y[512] == 1.0
    assert np.count_nonzero(y) == 3
    assert e4m3_decode(np.array([0xC0], np.uint8))[0] == -2.0


def test_set_mla_kv_buffer_scatter():
    # quantize-on-write: each new row lands in its slot in the cache's
    # format; other slots and out-of-range destinations leave no trace
    bits, x = _bf16_bits(6, seed=5, scale=2.0)
    nope, rope = bits[:, :512], bits[:, 512:]
    slots = 10
    rng = np.random.default_rng(0)
    cache8 = rng.integers(0, 256, (slots, 656), dtype=np.uint8)
    loc = np.array([7, 2, -1, 9, 10, 0])          # -1 and 10: skipped
    out8 = Q.set_mla_kv_buffer(cache8, nope, rope, loc, fp8=True)
    want = Q.quantize_k_cache(bits)
    for i, s in enumerate(loc):
        if 0 <= s < slots:
            np.testing.assert_array_equal(out8[s], want[i])
    untouched = [s for s in range(slots) if s not in set(loc.tolist())]
    np.testing.assert_array_equal(out8[untouched], cache8[untouched])
    # decoding a written row stays within the e4m3 half-ulp of its values
    y = Q.dequantize_rows(out8[[7]])[0]
    err = np.abs(y[:512] - x[0, :512])
    scale = np.repeat(out8[7, 512:528].copy().view("<f4").astype(np.float64), 128)
    assert (err <= np.maximum(np.abs(x[0, :512]) * 2.0 ** -4, scale * 2.0 ** -10) + 1e-300).all()
    np.testing.assert_array_equal(y[512:], x[0, 512:])
    # bf16 cache: the 576 values copied
    cache16 = rng.integers(0, 1 << 16, (slots, 576), dtype=np.uint16)
    out16 = Q.set_mla_kv_buffer(cache16, nope, rope, loc, fp8=False)
    np.testing.assert_array_equal(out16[7], bits[0])
    np.testing.assert_array_equal(out16[0], bits[5])
    np.testing.assert_array_equal(out16[untouched], cache16[untouched])
