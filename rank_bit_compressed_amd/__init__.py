"""Decode attention over a rank/bit-compressed KV cache on AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(librbc_kvc.so, declared in include/kvc.h); rank_bit_compressed_amd.kvc is
its thin Python binding.  PyTorch supplies device memory and streams only.
"""
