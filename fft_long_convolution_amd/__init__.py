"""MI355X (gfx950) causal FFT long convolution: HIP kernels behind a C ABI (include/lconv.h).

Python side: ``lconv`` (ctypes binding, torch for memory/streams), ``workloads`` (seeded
synthetic inputs) and ``build`` (hipcc build of liblconv.so).
"""
