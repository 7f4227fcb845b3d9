"""FP8 scaled linear layer for AMD MI355X (gfx950): amax, scales (current,
delayed from an amax history, block-wise), saturating RNE casts to E4M3 /
E5M2 with fused transpose, and FP8 GEMMs with FP32 accumulation.

The compute path is the HIP library libfp8lin.so behind the C ABI in
include/fp8lin.h; `fp8_mixed_precision_linear_amd.lib` is its Python binding
(import it explicitly: it raises if the library is not built).
`fp8_mixed_precision_linear_amd.datagen` holds the seeded synthetic inputs.
"""

__all__ = ["lib", "datagen", "build"]
