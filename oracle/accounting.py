"""Byte accounting of the cache (test infrastructure only).

Follows the kivi_sink page ("How it works", item 4: sink bytes and residual
fp16 bytes are tracked separately with no double counting; "Evidence": the
accounting partitions tokens exactly across the compressed, sink and residual
pools) and the StreamingLLM + KIVI page ("Caveats": the generation counter is
reported next to the stored count).

Counts per (layer, b) are taken by enumerating the valid positions and their
read source, never from a formula, so the partition pin is independent of the
library's arithmetic.

Parity: pinned by hand-counted cases (KIVI and q2k with partially evicted
blocks, top-k sinks inside blocks, a block whose valid rows are all sinks, a
window covering every valid row, TurboQuant after eviction) and by
position-by-position enumeration in tests/test_oracle_accounting.py, and by the
page figures of the q2k page ("Memory math": 448 B per cell at 2 x 256
channels) in tests/test_oracle_q2k.py.
"""

from .layout import record_sections, slot_bits


def bytes_per_token_head(fmt, D, k_bits, v_bits, G=32):
    """Compressed bytes one token of one KV head costs, metadata amortised over its block."""
    _, size, _ = record_sections(fmt, D, k_bits, v_bits)
    return (size["k_codes"] + size["v_codes"] + size["k_meta"] + size["v_meta"]) / G


def account(model, layer, b):
    cfg = model.cfg
    src = model.valid(layer, b)
    n_sink = sum(1 for s in src.values() if s == "sink")
    n_res = sum(1 for s in src.values() if s == "window")
    n_q = sum(1 for s in src.values() if s == "bulk")
    H, D = cfg.n_kv_heads, cfg.store_dim  # stored width (TurboQuant pads a non-power-of-two head_dim)
    _, size, _ = record_sections(cfg.fmt, D, cfg.k_bits, cfg.v_bits, cfg.tq_dense3)
    blocks = {p // 32 for p, s in src.items() if s == "bulk"}
    if cfg.fmt == "tq":
        meta = n_q * 8 * H
    else:
        meta = len(blocks) * size["k_meta"] * H + n_q * (size["v_meta"] // 32) * H
    return {
        "n_valid": len(src), "n_compressed": n_q, "n_sink": n_sink, "n_residual": n_res,
        "current_length": model.P[layer],
        "compressed_bytes": n_q * H * D * (slot_bits(cfg.k_bits, cfg.tq_dense3) +
                                           slot_bits(cfg.v_bits, cfg.tq_dense3)) // 8 + meta,
        "sink_fp16_bytes": n_sink * H * D * 2 * 2,
        "residual_fp16_bytes": n_res * H * D * 2 * 2,
    }
