"""MI355X-native theta-bundle reconstructed linear: HIP kernels for gfx950 behind
a C ABI (``include/aq.h``, ``libaq.so``), with a thin ctypes binding.

``from rank_shared_block_amd import binding`` gives the C-ABI functions and the
torch-tensor helpers; ``rank_shared_block_amd.inputs`` holds the seeded synthetic
workloads.  Importing the package loads nothing; the first call into
``binding`` loads ``libaq.so`` and raises if it has not been built.
"""
