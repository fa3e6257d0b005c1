"""Plain CPU oracle for the CSA2 hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the device library.
"""
