"""GPU parity of the top-k key-norm sink selection alone, through the C ABI, against the oracle.

Bar: sink positions, scores (fp32 bits) and counts bit-exact after every call.  Chunk lengths
cover the single-workgroup path (n <= 64) and the split path (n > 64: one workgroup per 64 rows,
up to 64 workgroups per batch element, then a merge), for every row load shape (fp16 and fp32
input, head_dim 32, 64 and 128) and head counts below and above one round of head loads (8).
Ties: rows that repeat one vector score equal, and the rank then falls back to the position, so
the earliest positions must win across workgroup boundaries.
"""
import numpy as np
import pytest
import torch

from harness import Pair

pytestmark = pytest.mark.gpu

SHAPES = [("f16", 32, 5), ("f16", 64, 3), ("f16", 128, 9), ("f32", 32, 2), ("f32", 64, 9), ("f32", 128, 3)]
CHUNKS = [1, 64, 65, 700, 129, 3, 1000]


def _log(*a):
    print(*a, flush=True)


def _check(pair, layer):
    pos, sc, cnt = pair.model.sink_state(layer)
    g = pair.gpu_regions(layer)
    assert np.array_equal(g["sink_count"], cnt), (g["sink_count"], cnt)
    assert np.array_equal(g["sink_pos"], pos), (g["sink_pos"], pos)
    assert np.array_equal(g["sink_score"].view(np.uint32), sc.view(np.uint32))


def _pair(dtype, D, H, n_sink, seed):
    return Pair(data_seed=seed, n_layers=1, batch=2, n_kv_heads=H, n_q_heads=H, head_dim=D, fmt="kivi", k_bits=4,
                v_bits=4, sink_mode="topk", n_sink=n_sink, residual=0, capacity=4096, in_dtype=dtype)


@pytest.mark.parametrize("dtype,D,H", SHAPES)
def test_select_chunks(dtype, D, H):
    pair = _pair(dtype, D, H, 16, 31 + D + H)
    rng = np.random.default_rng(D * 10 + H)
    for step, n in enumerate(CHUNKS):
        # a few strong rows per chunk, so that later chunks still bring new sinks until the set is full
        planted = [(b, [int(x) for x in rng.choice(n, min(n, 3), replace=False)]) for b in range(2)]
        k, v = pair.rows(n, planted=planted if step % 2 else None)
        _log(f"[select {dtype} D={D} H={H}] chunk {step} n={n}")
        pair.select(0, k)
        pair.append(0, k, v)
        _check(pair, 0)


def test_select_ties_across_workgroups():
    """Identical rows in every position: all scores tie, so the first n_sink positions are the sinks."""
    pair = _pair("f16", 128, 3, 16, 5)
    k, v = pair.rows(3000)
    k = k[:, :, :1, :].expand(-1, -1, 3000, -1).contiguous()
    pair.select(0, k)
    pair.append(0, k, v)
    _check(pair, 0)
    pos, _, cnt = pair.model.sink_state(0)
    assert (cnt == 16).all() and (pos == np.arange(16)[None, :]).all()


def test_select_ties_with_committed_sinks():
    """A set that is not full meets a tie with its own committed scores in a later chunk."""
    pair = _pair("f32", 64, 2, 7, 6)
    k1, v1 = pair.rows(3)
    pair.select(0, k1)
    pair.append(0, k1, v1)
    _check(pair, 0)
    k2, v2 = pair.rows(900)
    k2[:, :, 100:900:97, :] = k1[:, :, 1:2, :]  # same score as a committed sink, later position
    k2 = k2.contiguous()
    pair.select(0, k2)
    pair.append(0, k2, v2)
    _check(pair, 0)


def test_select_rejects_misaligned_rows():
    from quantized_kv_cache_kivi_amd import kvq
    pair = _pair("f16", 64, 2, 4, 7)
    buf = torch.zeros(2 * 2 * 10 * 64 + 1, dtype=torch.float16, device="cuda")
    k = buf[1:].view(2, 2, 10, 64)
    with pytest.raises(kvq.KvqError) as e:
        pair.gpu.kvq_select_sinks(0, k)
    assert e.value.status == -1  # KVQ_EINVAL
