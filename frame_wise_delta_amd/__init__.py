"""Video Delta Attention (VDA) linear branch on AMD MI355X (gfx950).

The compute path is the C-ABI library ``libvda.so`` (hand-written HIP
kernels, built from ``csrc/``); ``frame_wise_delta_amd.vda`` is its thin
Python binding.  Importing this package loads nothing; ``vda.load()`` opens
the library and fails loudly if it has not been built.
"""
