"""CPU oracle of the routed-MoE decode step: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
it.  The product package never does.
"""
