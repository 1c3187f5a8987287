"""The benchmark's roofline accounting: the indexer's strict algorithmic bytes
count each request's keys once however many of its rows read them and leave
out the logits (an intermediate, reported apart); its flops are 2 * heads *
dim per (row, position)."""

import bench


def test_decode_rows_each_read_their_own_keys():
    b, fl, lg = bench.indexer_cost([100, 64], [0, 1], hi=64, di=128)
    per_row = lambda L: 64 * 128 + 64 * 4 + L * 132 + ((L + 63) // 64) * 4  # noqa: E731
    assert b == per_row(100) + per_row(64)
    assert lg == (100 + 64) * 4
    assert fl == 2 * 64 * 128 * 164


def test_rows_of_one_request_share_its_keys():
    # four verify rows of one request (lengths L-3..L) and one other request
    L = 1000
    b, fl, lg = bench.indexer_cost([L - 3, L - 2, L - 1, L, 50], [0, 0, 0, 0, 1])
    rows = 5 * (64 * 128 + 64 * 4)
    keys = L * 132 + 16 * 4 + 50 * 132 + 1 * 4
    assert b == rows + keys
    assert lg == 4 * (4 * L - 6 + 50)
    assert fl == 2 * 64 * 128 * (4 * L - 6 + 50)


def test_pipeline_bytes_are_strict():
    b = bench.pipeline_bytes([3000], [0], topk=2048, heads=16, kv_row_bytes=656)
    idx, _, _ = bench.indexer_cost([3000], [0])
    assert b == idx + 2048 * 656 + 16 * (576 * 2 + 512 * 2 + 4)


def test_decode_b128_strict_bytes_match_the_hand_count():
    # one decode row of L positions reads 132 L bytes of keys and scales,
    # 8448 B of q and weights, 4 B per page id; 2048 selected 656-byte
    # latent rows; q (128 x 576 bf16) and out (128 x 512 bf16) and lse
    L = 100000
    b = bench.pipeline_bytes([L], [0], topk=2048, heads=128, kv_row_bytes=656)
    assert b == (132 * L + 8448 + 4 * ((L + 63) // 64) + 2048 * 656
                 + 128 * (1152 + 1024 + 4))
