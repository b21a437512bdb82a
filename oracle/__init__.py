"""CPU oracle for the bf16 delta-sync hot path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  Every function
that is not pinned against something other than itself would be marked
"parity unpinned" here; at present every function has a pin (see the tests).
"""
