"""CPU oracle for absorbed-MLA decode (fp64 reference + FP4 reference codec).

TEST INFRASTRUCTURE: imported only by tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py. The HIP product path
never imports, links or executes anything in this package.
"""
