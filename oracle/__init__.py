"""fp64 CPU oracle (test infrastructure: used only by the tests, the smoke
check and the benchmark's CPU baseline)."""
