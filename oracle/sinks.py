"""Attention-sink selection (test infrastructure only).

Follows the kivi_sink page, "How it works": on every update the per-token key
L2 norm, averaged over KV heads, is folded into a running top-k of absolute
positions; tokens in the sink set are kept in fp16 and never quantized;
selection is deterministic.  "Fidelity to the paper" adds the v1 limit: a
token quantized in an earlier call is never restored later.  The static mode
keeps the first N tokens (StreamingLLM + KIVI page, "StreamingLLM — why
softmax needs an anchor").

Readings:

* score_t = (sum over heads h, in order, of sqrt(canonical sumsq of K[b,h,t,:]))
  / n_kv_heads, in fp32.
* Ranking by (score descending, position ascending).
* Commit rule for one call: fold the call's rows into the running top-k
  (TK = top-k of TK and the new rows); every *new* row now in TK joins the
  committed set C, in TK order, while |C| < n_sink.  C is permanent.  While C
  is not full, TK equals C, so C with its scores is the whole state.

Parity: pinned by brute-force ranking on small inputs, the planted-sink
recovery of the kivi_sink page's "Evidence" section, and first-N equivalence
when rows arrive one at a time (tests/test_oracle_sinks.py).
"""

import numpy as np

from .numerics import f32, sumsq_canonical


def token_scores(k_b):
    """k_b: fp32 [Hkv, n, D] keys of one batch element -> fp32 [n] scores."""
    k_b = f32(k_b)
    acc = np.zeros(k_b.shape[1], dtype=np.float32)
    for h in range(k_b.shape[0]):
        acc = acc + np.sqrt(sumsq_canonical(k_b[h]))
    return acc / np.float32(k_b.shape[0])


def topk_commit(committed, new_positions, new_scores, n_sink):
    """One select call.  committed: list of (position, score) in commit order.

    Returns the new committed list (the old one extended).
    """
    C = list(committed)
    if len(C) >= n_sink:
        return C
    new = [(int(p), np.float32(s)) for p, s in zip(new_positions, new_scores)]
    cand = [(p, s, False) for p, s in C] + [(p, s, True) for p, s in new]
    cand.sort(key=lambda e: (-float(e[1]), e[0]))
    for p, s, is_new in cand[:n_sink]:
        if is_new and len(C) < n_sink:
            C.append((p, s))
    return C


def first_n(P, n_sink):
    """FIRST_N mode: committed positions after P rows have been appended."""
    return [(p, np.float32(0.0)) for p in range(min(P, n_sink))]
