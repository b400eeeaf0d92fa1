"""fp64 CPU oracle for the KDA recurrence -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the product path never does.
"""
