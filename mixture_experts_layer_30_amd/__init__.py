"""MoE feed-forward layer forward pass (softmax top-K routing, block-padded
alignment, SwiGLU grouped GEMM, weighted combine) and its FLOP-matched dense
baseline, as hand-written HIP kernels for MI355X (gfx950) behind a C ABI.

Submodules: ``binding`` (ctypes binding of libmoe_layer.so), ``layer`` (the
five-call layer pass), ``configs`` (layer shapes), ``synth`` (seeded inputs),
``build`` (compiles the library).
"""
