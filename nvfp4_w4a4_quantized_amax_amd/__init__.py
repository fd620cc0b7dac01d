"""libnvfp4: NVFP4 dynamic W4A4 quantization and GEMM on AMD MI355X (gfx950).

The compute path lives in hand-written HIP kernels behind the C ABI declared in include/nvfp4.h.
`nvfp4_w4a4_quantized_amax_amd.nvfp4` is the thin ctypes binding (argument marshalling only);
importing it loads the shared library and fails loudly if it has not been built.
`nvfp4_w4a4_quantized_amax_amd.workloads` holds the seeded synthetic input generators.
"""
