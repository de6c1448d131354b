"""The FLOP / logical-byte model against the pages' printed numbers. CPU only."""
from io_aware_flashattention_amd import cost_model as cm
from tests.conftest import golden

MiB = 2 ** 20


def test_page4_traffic_table():
    g = golden("t5_traffic_model.json")
    N, d, b, Br, Bc = g["N"], g["d"], g["elem_bytes"], g["Br"], g["Bc"]
    r, w = cm.naive_traffic(N, d, b)
    assert (r / MiB, w / MiB, (r + w) / MiB) == (g["naive_unmasked_mib"]["reads"], g["naive_unmasked_mib"]["writes"], g["naive_unmasked_mib"]["total"])
    assert r + w == g["naive_unmasked_mib"]["total_bytes"]
    r, w = cm.naive_traffic(N, d, b, causal=True)
    assert (r / MiB, w / MiB) == (g["naive_causal_ideal_mib"]["reads"], g["naive_causal_ideal_mib"]["writes"])
    r, w = cm.fa2_traffic(N, d, Br, Bc, b)
    assert (r / MiB, w / MiB) == (g["fa2_unmasked_mib"]["reads"], g["fa2_unmasked_mib"]["writes"])
    assert r + w == g["fa2_unmasked_mib"]["total_bytes"]
    r, w = cm.fa2_traffic(N, d, Br, Bc, b, causal=True)
    assert (r / MiB, w / MiB) == (g["fa2_causal_mib"]["reads"], g["fa2_causal_mib"]["writes"])
    assert r + w == g["fa2_causal_mib"]["total_bytes"]
    assert cm.kv_passes(N, Br, Bc, causal=True) == g["causal_kv_passes"]
    r2, w2 = cm.fa2_traffic(N, d, Br, Bc, b, causal=True, lse=True)
    assert w2 - w == g["lse_bytes_per_head"]


def test_page5_one_head_arithmetic():
    g = golden("t5_traffic_model.json")
    f = cm.attention_flops(1, 1, 4096, 4096, 128, causal=False)
    assert abs(f - g["page5_flops"]["value"]) <= g["page5_flops"]["tol"]
    r, w = cm.naive_traffic(4096, 128, 2)
    assert abs((r + w) / 1e6 - g["page5_naive_bytes_mb"]["value"]) <= g["page5_naive_bytes_mb"]["tol"]
    assert 4096 * 4096 * 2 == g["page5_score_matrix_bytes"]


def test_page4_exercise4_tile_ranges():
    g = golden("t4_causal_tiles.json")
    i = g["query_tile"] - 1
    n = cm.causal_kv_tiles(i, g["Br"], g["Bc"], g["N"])
    assert n == g["loaded_tiles"][1]
    diag = cm.causal_diagonal_tiles(i, g["Br"], g["Bc"], g["N"])
    assert [j + 1 for j in diag] == list(range(g["diagonal_tiles"][0], g["diagonal_tiles"][1] + 1))
    assert diag.start == g["unmasked_tiles"][1]


def test_causal_tiles_ragged_and_square():
    # Br == Bc: tile i loads i+1 tiles and only the last is diagonal
    for i in range(5):
        assert cm.causal_kv_tiles(i, 64, 64, 1000) == i + 1
        assert list(cm.causal_diagonal_tiles(i, 64, 64, 1000)) == [i]
    # ragged: 1000 rows, Br=128: last query tile covers rows 896..999 -> 16 tiles of 64
    assert cm.causal_kv_tiles(7, 128, 64, 1000) == 16


def test_decode_bytes_per_token():
    # 2 (K and V) x 8 kv heads x 128 x 2 bytes = 4096 bytes per token per layer
    assert cm.decode_kv_bytes([1], 8, 128) == 4096
    assert cm.decode_kv_bytes([32768], 8, 128) * 80 / 1e9 > 10.7 - 0.05
    assert cm.decode_flops([10], 64, 128) == 4 * 64 * 128 * 10


def test_compulsory_bytes_long_context_gqa():
    # causal GQA prefill B1 Hq64 Hkv8 N8192 d128 bf16: Q + K + V + O + LSE
    b = cm.compulsory_bytes(1, 64, 8, 8192, 128)
    assert b == 134217728 + 2 * 16777216 + 134217728 + 4 * 64 * 8192


def test_window_flops_counts_visible_pairs():
    for n, w in [(1, 0), (5, 0), (5, 2), (10, 3), (10, 20), (64, 63)]:
        pairs = sum(1 for r in range(n) for c in range(n) if c <= r and r - c <= w)
        assert cm.window_flops(3, n, 8, w) == 4.0 * 3 * 8 * pairs
    # the pages' example: 8192 tokens, keys at most 1024 behind
    assert cm.window_flops(1, 8192, 1, 1024) == 4.0 * (7168 * 1025 + 1024 * 1025 // 2)


def test_varlen_flops_sums_sequences():
    assert cm.varlen_flops([3, 0, 5], 2, 4, False) == 4.0 * 2 * 4 * (9 + 25)
    assert cm.varlen_flops([3, 5], 2, 4, True) == 4.0 * 2 * 4 * (9 + 25) / 2


def test_backward_flops_are_five_matmuls():
    fwd = cm.attention_flops(1, 64, 8192, 8192, 128, True)
    assert cm.backward_flops(1, 64, 8192, 8192, 128, True) == fwd * 5 / 2
    # one (row, key) pair, d = 1: five products of 2 FLOPs each
    assert cm.backward_flops(1, 1, 1, 1, 1, False) == 10.0
