"""SmoothQuant W8A8 linear-layer path for AMD Instinct MI355X (gfx950).

The computation lives in libsq.so (HIP kernels behind the C ABI of
include/sq.h); `capi` is the thin Python binding, `synth` draws seeded
synthetic inputs, `build` compiles the library in-tree.
"""
