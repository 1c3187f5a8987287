"""Pins for the oracle's number formats: exhaustive over the 256 fp8 codes
against torch's own float8_e4m3fn cast, and the format's closed-form extremes."""

import numpy as np
import torch

from oracle.formats import e4m3_decode, e4m3_encode_rne_sat, bf16_bits_to_f64


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_exhaustive_matches_torch():
    ours = e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert nan_ours.sum() == 2                     # 0x7F and 0xFF only
    np.testing.assert_array_equal(ours[~nan_ours], ref[~nan_ref])


def test_e4m3_closed_form_extremes():
    v = e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x00, 0x80, 0x38], np.uint8))
    assert v[0] == 448.0                  # largest finite
    assert v[1] == 2.0 ** -6              # smallest normal
    assert v[2] == 2.0 ** -9              # smallest subnormal
    assert v[3] == 0.0 and v[4] == 0.0 and np.signbit(v[4])
    assert v[5] == 1.0                    # exponent field 7 = bias


def test_e4m3_encode_matches_torch_rne_on_dense_grid():
    # every midpoint between adjacent codes, the codes themselves, and values
    # one float32 ulp either side of each midpoint
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    pts = np.concatenate([vals, mids, np.nextafter(m32, np.float32(np.inf)),
                          np.nextafter(m32, np.float32(-np.inf))]).astype(np.float32)
    rng = np.random.default_rng(1)
    pts = np.concatenate([pts, rng.uniform(-463.9, 463.9, 200000).astype(np.float32),
                          rng.uniform(-0.02, 0.02, 50000).astype(np.float32)])
    pts = np.concatenate([pts, -pts])
    ours = e4m3_encode_rne_sat(pts)
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of zero the same way
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_saturates():
    x = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e6, -500.0, -448.0])
    codes = e4m3_encode_rne_sat(x)
    assert list(codes) == [0x7E] * 6 + [0xFE, 0xFE]


def test_e4m3_encode_ties_to_even():
    # 1.0 (0x38) and 1.125 (0x39): the midpoint 1.0625 goes to the even code
    assert e4m3_encode_rne_sat(np.array([1.0625]))[0] == 0x38
    # 1.125 (0x39) and 1.25 (0x3A): midpoint 1.1875 goes to 0x3A
    assert e4m3_encode_rne_sat(np.array([1.1875]))[0] == 0x3A
    # subnormal midpoint between 0 and 2^-9 goes to 0
    assert e4m3_encode_rne_sat(np.array([2.0 ** -10]))[0] == 0x00


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
