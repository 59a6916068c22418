"""CPU oracle for MoE dispatch/combine.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in this package.
It shares no code with the HIP library and never imports it.
"""
