"""CPU oracle for the H3-style DiT forward.  Test infrastructure only: imported
by the tests, the smoke check and the benchmark's CPU-baseline leg, never by
the product path."""
