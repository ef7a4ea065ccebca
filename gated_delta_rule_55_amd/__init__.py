"""MI355X (gfx950) implementation of the Kimi Delta Attention (KDA) operator.

The compute path is the HIP library ``libkda.so`` built from ``csrc/``; the
Python functions here only marshal arguments to its C-ABI.
"""
