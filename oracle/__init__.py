"""CPU oracle for the tile-synchronized decoder: test infrastructure only.

Plain, slow, float64 numpy code that states what the decoder computes
(``numerics``), how the instruction queue and its tile barriers are built
(``queue_spec``) and how to check that a queue enforces every producer ->
consumer dependency (``checker``).

Only the test-suite, the package's smoke check and the benchmark's CPU
baseline leg may import this package.  It shares no code with the GPU library
and never imports it; the two meet only through the seeded inputs of the
``workloads`` package.

Sources: the MegaOps abstract (dependencies enforced on tiles of intermediate
tensors), the "Production Megakernels" lecture summary (interpreter popping a
global queue; symbolic shapes; barriers as tensors), and the standard pre-norm
Llama/Qwen decoder block, which the pages name but do not write out.

Parity status: every function here is pinned by a test under ``tests/`` that
does not reuse its formula (brute-force loops, closed forms, invariants,
library routines); see ``tests/test_oracle_*.py``.
"""
