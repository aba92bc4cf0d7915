"""CPU oracle for the row softmax.  TEST INFRASTRUCTURE ONLY: imported by the
tests, the smoke check and the benchmark's CPU-baseline leg, never by the
GPU package."""
