"""fp64 CPU oracle for the gated delta rule backward -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import it.
"""
