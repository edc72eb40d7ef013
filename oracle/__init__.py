"""fp64 CPU oracle of the MoE-layer forward.  Test infrastructure only: used by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
library itself."""
