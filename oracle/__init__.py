"""CPU oracle (test infrastructure). Imported only by tests, the smoke check and
the benchmark's CPU-baseline leg; the library never imports it."""
