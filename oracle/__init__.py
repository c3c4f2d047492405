"""CPU oracle for the CSA hot path (test infrastructure only).

``csa_oracle`` is the vectorised float64 NumPy evaluation of eqs 1-11 of the
page "Compressed Sparse Attention (压缩稀疏注意力)"; ``brute`` restates the same
equations as pure-Python scalar loops for tiny inputs.  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may use this package;
the HIP implementation never imports it and it never imports the HIP side.
"""
from . import csa_oracle, brute  # noqa: F401
