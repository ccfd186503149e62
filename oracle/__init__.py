"""fp64 CPU oracle for Out = A . B^T -- test infrastructure only (see oracle.py)."""
