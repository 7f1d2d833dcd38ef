"""CPU oracle for the gated delta rule with FP8-E4M3 state QDQ.

Test infrastructure only: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg.  It shares no code with the HIP library.
"""
