"""Selective decode attention for MI355X (gfx950).

The compute path is the C-ABI library libcsa.so (hand-written HIP kernels);
`csa` is its thin Python binding and `workloads` the seeded input recipes."""
