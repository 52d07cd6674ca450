"""CPU oracle for the skip-masked attention forward.  Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg."""
