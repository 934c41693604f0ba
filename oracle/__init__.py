"""CPU float64 oracle for paged decode attention and GrowPage's page-boundary budgeting pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package: only the test
suite, the smoke check and the benchmark's CPU-baseline leg call it. It shares no code with
the HIP library and is written from the definitions on the pages:

* GrowPage: On-Demand KV Budgeting for Efficient LLM Reasoning Serving (arXiv 2609.03494):
  Eq. 2 and 7 (p-coverage working set), Eq. 3 and 5 (renormalised subset output and its
  worst-case error), Eq. 6 (dual-timescale EMA), Eq. 8 (demand trend), Eq. 9 and 10
  (importance and block-local + global selection), Eq. 12 (RMS calibration), Sec. 3.3 and
  Sec. 4.2 (Compress & Hold / Grow by One Page), App. E.1 and E.2 (slot pool, prefix sharing).
* PASK: Parser-Aware Structural KV Persistence: Sec. 3.1 (attention definition) and App. B.5
  (packed attention inputs, symmetric per-row INT4 quantisation, split-KV merge).

Parity status per function is listed in each module header; every function here is pinned by
a CPU test against closed forms, invariants, hand-derived fixtures, library special cases or
brute force.
"""
from . import fp8, int4, attention, summaries, boundary  # noqa: F401
