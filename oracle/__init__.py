"""CPU oracle for the quantized KV cache hot path — TEST INFRASTRUCTURE ONLY.

Nothing in the product (the HIP library and its Python binding) may import,
call or execute anything in this package.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle exists twice, written independently of the HIP library:

* the numpy modules of this package, the readable reference, which cover
  every row (the decode hot path, prefill attention, the whole-T cache of
  the StreamingLLM + KIVI page, RoPE on read);
* ``c/kvq_oracle.c``, a plain C99 implementation of the decode hot path
  (sink selection, KIVI / q2k / TurboQuant quantization and packing,
  eviction, stored bytes, dequantization, fp64 decode attention, byte
  accounting), built with -O2 -ffp-contract=off -fno-fast-math and OpenMP,
  used through ``c_model.py``.  It reproduces the numpy modules' codes,
  bytes, sinks and tables bit for bit and their attention to fp64 rounding
  (tests/test_oracle_c.py), and it is what the bench times as the CPU
  baseline on the host's cores.

Every step that decides an integer (a code, a sink rank) is computed in IEEE
fp32 exactly as the method states it, one rounded operation at a time (numpy
never contracts a*b+c into an FMA; the C build forbids contraction).  The
attention reference is fp64 over exactly dequantized keys and values.

The four web pages it follows are cited by title and section:

* "StreamingLLM + KIVI — long-context decode without growing the KV cache"
  (the StreamingLLM + KIVI page),
* "TurboQuant KV Cache Compression — Spec" (the TurboQuant spec page),
* "KV cache: FP16 sliding window + attention sinks, and an optional 2-bit K /
  4-bit V cache scheme (--kv q2k)" (the q2k pull-request page),
* "KVSink-Adapted Sink Protection" (the kivi_sink page).

Parity status of each function is stated in its module docstring; every
function here is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``
against something other than itself (a closed form, a textbook value, a value
printed on a page, brute force, or an invariant).
"""

from . import numerics, layout, kivi, q2k, turboquant, sinks, cache, attention, accounting, kivi_whole, rope  # noqa: F401
# c_model (the C oracle's front end) is imported on demand: it loads or builds oracle/c/libkvq_oracle.so
