"""LCSA forward on AMD MI355X (gfx950): pool -> block score + mask + Top-K -> block-sparse attention.

The compute path is the C-ABI library `liblcsa.so` (hand-written HIP kernels); `lcsa` is its thin
Python binding. `workloads` and `inputs` describe problem shapes and seeded synthetic inputs.
"""
