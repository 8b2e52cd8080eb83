"""The byte model the bench's roofline figures divide by (bench.algorithmic_bytes), against hand counts
on small caches: packed codes and metadata of every valid bulk token, K metadata once per block that
still holds a compressed row, 2 * 2 * D bytes per fp16 sink or window row, plus q and out (CPU)."""
import bench

KW = dict(batch=1, n_kv_heads=1, n_q_heads=1, head_dim=128)


def _bytes(P, lo, sinks, **kw):
    return bench.algorithmic_bytes(dict(KW, **kw), P, lo, [sinks])[0]


QO = 128 * 2 + 128 * 4  # fp16 query in, fp32 output


def test_kivi2_bulk_only():
    # 64 tokens x (32 B K codes + 32 B V codes + 4 V groups x 4 B metadata) + 2 blocks x 512 B K metadata
    assert _bytes(64, 0, [], fmt="kivi", k_bits=2, v_bits=2) == 64 * 80 + 2 * 512 + QO


def test_kivi2_window_rows_and_a_sink():
    # residual 16: tokens 48..63 read as fp16 rows (512 B each); 48 bulk tokens in 2 blocks
    assert _bytes(64, 0, [], fmt="kivi", k_bits=2, v_bits=2, residual=16) == 48 * 80 + 2 * 512 + 16 * 512 + QO
    # a committed sink at position 3: one fp16 row, one bulk token fewer, block 0 still holds 31 rows
    assert _bytes(64, 0, [3], fmt="kivi", k_bits=2, v_bits=2) == 63 * 80 + 2 * 512 + 512 + QO


def test_block_of_sinks_only_carries_no_k_metadata():
    # positions 32..63 all sinks (n_sink 32): block 1 holds no compressed row
    sinks = list(range(32, 64))
    assert _bytes(64, 0, sinks, fmt="kivi", k_bits=4, v_bits=4) == 32 * (64 + 64 + 16) + 512 + 32 * 512 + QO


def test_turboquant_slots_and_dense_stream():
    # 3-bit codes in 4-bit slots: 64 + 32 B codes + 2 fp32 norms per token, no K block metadata
    assert _bytes(64, 0, [], fmt="tq", k_bits=3, v_bits=2) == 64 * (64 + 32 + 8) + QO
    # the dense 8-in-3 stream: 48 + 32 B codes per token
    assert _bytes(64, 0, [], fmt="tq", k_bits=3, v_bits=2, tq_dense3=True) == 64 * (48 + 32 + 8) + QO
    assert _bytes(64, 0, [], fmt="tq", k_bits=4, v_bits=3) == 64 * (64 + 64 + 8) + QO


def test_q2k_and_eviction():
    # q2k: K 2-bit (32 B) + V 4-bit (64 B) + V scales 4 x 2 B per token, K rms 2 B per channel and block;
    # lo = 40 evicts tokens below 40: blocks 1 (rows 40..63) only
    assert _bytes(64, 40, [], fmt="q2k", k_bits=2, v_bits=4) == 24 * (32 + 64 + 8) + 256 + QO
