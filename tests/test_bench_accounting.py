"""The benchmark's roofline accounting: the indexer's algorithmic bytes count
each request's keys once however many of its rows read them, and its flops
are 2 * heads * dim per (row, position)."""

import bench


def test_decode_rows_each_read_their_own_keys():
    b, fl = bench.indexer_cost([100, 64], [0, 1], hi=64, di=128)
    per_row = lambda L: 64 * 128 + 64 * 4 + L * 4 + L * 132 + ((L + 63) // 64) * 4  # noqa: E731
    assert b == per_row(100) + per_row(64)
    assert fl == 2 * 64 * 128 * 164


def test_rows_of_one_request_share_its_keys():
    # four verify rows of one request (lengths L-3..L) and one other request
    L = 1000
    b, fl = bench.indexer_cost([L - 3, L - 2, L - 1, L, 50], [0, 0, 0, 0, 1])
    rows = 5 * (64 * 128 + 64 * 4) + 4 * (4 * L - 6 + 50)
    keys = L * 132 + 16 * 4 + 50 * 132 + 1 * 4
    assert b == rows + keys
    assert fl == 2 * 64 * 128 * (4 * L - 6 + 50)


def test_pipeline_bytes_drop_the_logits():
    b = bench.pipeline_bytes([3000], [0], topk=2048, heads=16, kv_row_bytes=656)
    idx, _ = bench.indexer_cost([3000], [0])
    assert b == idx - 3000 * 4 + 2048 * 656 + 16 * (576 * 2 + 512 * 2 + 4)
