"""MI355X-native VoxelBlockManager stencil pipeline (HIP kernels behind a C ABI).

``vbm`` is the binding of libvbm.so; ``inputs`` generates seeded synthetic
grids and sidecars; ``build`` compiles the library for gfx950.
"""
