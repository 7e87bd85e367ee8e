"""MI355X-native DSA / MISA / MISA-dagger token indexer.

The compute path is the HIP library ``libmisa_indexer.so`` (C ABI declared in
``include/misa_indexer.h``); :mod:`long_context_sparse_05_amd.abi` is its thin
Python binding and :mod:`long_context_sparse_05_amd.synth` the seeded input
generator.  Importing the package loads nothing.
"""
__all__ = ["abi", "synth"]
