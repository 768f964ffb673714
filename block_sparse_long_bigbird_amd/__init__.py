"""BigBird block-sparse self-attention forward for MI355X (gfx950).

The compute lives in a C-ABI shared library (libbb_attn.so: hand-written HIP
kernels plus a C++ host adjacency builder).  `binding` marshals arguments to
it; `workloads` draws seeded synthetic inputs.
"""
