"""CPU oracle of the int4 routed-expert MoE layer — test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
it.  See moe_oracle.py for the steps and the pages they follow.
"""
