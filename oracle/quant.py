"""fp8 block-scaled latent-KV cache: ``quantize_k_cache`` -- oracle, test
infrastructure.

The pages call ``quantize_k_cache(kv_cache)`` to turn the bf16 latent cache
into the fp8 format the sparse decode kernel reads ("nsa_backend.py
(EngineX-Hygon sglang fork)", ``_forward_flashmla_decode``; "dsa_backend.py
(sglang main)", ``_forward_flashmla_kv``), viewed as ``[pages, 64, 1,
kv_cache_dim]``. Its body is not shown. Reading adopted, one 656-byte row
per slot:

    bytes   0..511  e4m3fn codes of the 512 no-rope values, in 4 blocks of 128
    bytes 512..527  4 little-endian fp32 block scales
    bytes 528..655  the 64 rope values, bf16, copied unchanged

Block b: ``amax = max |x|`` over its 128 values (exact, fp32);
``scale = amax / 448`` in fp32 (correctly rounded; ``scale = 1`` when
``amax == 0``); ``code = e4m3_rne_sat(x / scale)`` with ``x / scale`` an fp32
correctly rounded division. Decoding: ``value = e4m3(code) * scale``.
"""

import numpy as np

from .formats import e4m3_decode, e4m3_encode_rne_sat, bf16_bits_to_f64

D_NOPE = 512
D_ROPE = 64
D_QK = D_NOPE + D_ROPE
BLOCK = 128
ROW_BYTES = D_NOPE + 4 * (D_NOPE // BLOCK) + 2 * D_ROPE  # 656


def quantize_k_cache(kv_bits):
    """bf16 latent rows ``[n, 576]`` (uint16 bit patterns) -> ``[n, 656]``
    uint8."""
    kv_bits = np.asarray(kv_bits, dtype=np.uint16)
    n = kv_bits.shape[0]
    x = bf16_bits_to_f64(kv_bits[:, :D_NOPE]).astype(np.float32)  # exact
    out = np.zeros((n, ROW_BYTES), dtype=np.uint8)
    scales = np.zeros((n, D_NOPE // BLOCK), dtype=np.float32)
    for b in range(D_NOPE // BLOCK):
        blk = x[:, b * BLOCK:(b + 1) * BLOCK]
        amax = np.max(np.abs(blk), axis=1)
        scale = amax / np.float32(448.0)                    # fp32 division
        scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
        y = (blk / scale[:, None]).astype(np.float32)       # fp32 division
        out[:, b * BLOCK:(b + 1) * BLOCK] = e4m3_encode_rne_sat(y)
        scales[:, b] = scale
    out[:, D_NOPE:D_NOPE + 16] = np.ascontiguousarray(
        scales.astype("<f4")).view(np.uint8).reshape(n, 16)
    out[:, D_NOPE + 16:] = np.ascontiguousarray(
        kv_bits[:, D_NOPE:].astype("<u2")).view(np.uint8).reshape(n, 2 * D_ROPE)
    return out


def dequantize_rows(raw):
    """``[n, 656]`` uint8 rows -> ``[n, 576]`` float64: the latent vector the
    attention sees (codes times their block scale; rope exact)."""
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    n = raw.shape[0]
    codes = e4m3_decode(raw[:, :D_NOPE])
    scales = np.ascontiguousarray(raw[:, D_NOPE:D_NOPE + 16]).view("<f4") \
        .astype(np.float64).reshape(n, 4)
    nope = codes * np.repeat(scales, BLOCK, axis=1)
    rope = bf16_bits_to_f64(np.ascontiguousarray(raw[:, D_NOPE + 16:])
                            .view("<u2").reshape(n, D_ROPE))
    return np.concatenate([nope, rope], axis=1)


class Bf16Cache:
    """Latent cache stored as bf16 rows ``[slots, 576]`` (uint16 bits)."""

    def __init__(self, bits):
        self.bits = np.asarray(bits, dtype=np.uint16)
        self.num_slots = self.bits.shape[0]

    def rows(self, slots):
        return bf16_bits_to_f64(self.bits[np.asarray(slots, np.int64)])


class Fp8Cache:
    """Latent cache stored as 656-byte fp8 rows."""

    def __init__(self, raw):
        self.raw = np.asarray(raw, dtype=np.uint8)
        self.num_slots = self.raw.shape[0]

    def rows(self, slots):
        return dequantize_rows(self.raw[np.asarray(slots, np.int64)])


def set_mla_kv_buffer(cache, k_nope_bits, k_rope_bits, cache_loc, fp8):
    """Quantize-on-write of new latent rows ("dsa_backend.py (sglang main)",
    ``forward_extend`` / ``forward_decode``: ``set_mla_kv_buffer(layer,
    cache_loc, k, k_rope)``): row i (512 no-rope + 64 rope bf16 bit patterns)
    is stored at slot ``cache_loc[i]`` in the cache's own format -- the
    656-byte encoding of ``quantize_k_cache`` for an fp8 cache, the 576 bf16
    values for a bf16 cache. Slots outside the cache are skipped. Returns a
    new cache array (``[slots, 656]`` uint8 or ``[slots, 576]`` uint16)."""
    out = np.array(cache, copy=True)
    rows = np.concatenate([np.asarray(k_nope_bits, np.uint16)[:, :D_NOPE],
                           np.asarray(k_rope_bits, np.uint16)[:, :D_ROPE]], axis=1)
    for i, slot in enumerate(np.asarray(cache_loc, dtype=np.int64)):
        if not 0 <= slot < out.shape[0]:
            continue
        out[slot] = quantize_k_cache(rows[i:i + 1])[0] if fp8 else rows[i]
    return out
