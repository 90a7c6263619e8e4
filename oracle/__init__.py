"""fp64 CPU oracle for grouped-query prefill attention with sinks and a window.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the HIP path.
"""
