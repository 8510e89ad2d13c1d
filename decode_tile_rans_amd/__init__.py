"""decode_tile_rans_amd — MI355X-native EntroPack-style weight compression.

Python layer over libentropack_hip.so (include/entropack.h).  PyTorch is used
for device memory and streams only; every step of compression and decoding runs
in the library (host C++ encoder, gfx950 HIP decode and MFMA GEMM kernels).

    import decode_tile_rans_amd as ep
    c = ep.compress(w_bf16_cuda, target_bpp=3.5)       # EntroPack README 快速开始
    w_hat = ep.decompress(c)                           # same shape and dtype
    layer = ep.CompressedLinear.from_linear(linear, target_bpp=4.0)
    y = layer(x)
"""
from .api import (Compressed, compress, decompress, decompress_batch, CompressedLinear,  # noqa: F401
                  gemm_bf16_nt, gemm_fp8_nt, plan_bitrates, compress_lossless, compress_many, linear_batch,
                  EPError)
from . import _lib  # noqa: F401
