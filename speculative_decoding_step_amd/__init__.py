"""MI355X-native EAGLE-3 speculative-decoding step (draft tree, verify, accept, compact).

The compute path lives in the HIP library ``libeagle3.so`` built from ``csrc/``
and reached through :mod:`binding`; this package's Python only marshals
arguments and owns device memory through PyTorch.  Submodules are imported
lazily so that the seeded input generator can be used without a GPU.
"""
