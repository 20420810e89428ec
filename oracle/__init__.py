"""CPU oracle for the K-quant decode GEMV -- test infrastructure only (see oracle.py)."""
