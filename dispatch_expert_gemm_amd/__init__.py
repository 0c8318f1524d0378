"""MI355X-native expert-parallel MoE layer hot path: route, dispatch layout and permute, grouped
SwiGLU expert GEMM, and weighted combine, as hand-written gfx950 HIP kernels behind a C ABI
(libmoe.so). The Python side only marshals arguments; see ``moe`` for the binding."""
