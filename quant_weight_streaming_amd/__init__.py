"""K-quant (Q4_K / Q5_K / Q6_K) decode GEMV for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libkq.so`` built from ``csrc/``;
``quant_weight_streaming_amd.kq`` is its thin Python binding (argument
marshalling only).  ``synth`` holds the seeded synthetic-input generators.
"""
