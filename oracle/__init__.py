"""CPU oracle for the sparse-attention decode path (test infrastructure only).

This package is the plain, slow, obviously correct reference that the HIP path
is checked against. It is TEST INFRASTRUCTURE: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The library under ``sparse_attention_decode_indexer_amd`` never
imports it, and the two share no code (no helpers, tables or constants).

Arithmetic is numpy float64 for floating point and int64 for integers, unless
the method fixes a precision (the fp8 cache encoder works in float32, as the
cache format does).

Source pages cited in docstrings, by title:

* "nsa_backend.py (sglang 0.5.3rc2 -> 0.5.4 diff)": the diff page that adds
  speculative target-verify metadata to the native sparse attention backend.
* "nsa_backend.py (EngineX-Hygon sglang fork)": the early native sparse
  attention backend, full file.
* "dsa_backend.py (sglang main)": the current DeepSeek sparse attention
  backend, full file.

Modules, one per step of the path:

* ``formats``   -- OCP fp8 e4m3fn and bfloat16 codecs.
* ``metadata``  -- per-forward sequence-length metadata and page tables.
* ``indexer``   -- paged MQA indexer logits (formula is a reading; see module).
* ``topk``      -- length-masked top-k.
* ``transform`` -- logical position -> physical KV slot.
* ``sparse_mla``-- MLA attention over the selected slots.
* ``quant``     -- fp8 block-scaled latent-KV cache encoder / decoder, and
  quantize-on-write of new rows.
* ``ragged``    -- the RAGGED extend route: per-token key windows, shifted
  top-k positions, the flattened token table, paged dequantization, CSR
  index lists.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
except the indexer's scoring formula itself, which the pages never show; the
oracle's implementation of the adopted reading is pinned by closed forms, but
the reading is not (see ``indexer``).
"""

from . import formats, metadata, indexer, topk, transform, sparse_mla, quant, ragged  # noqa: F401
