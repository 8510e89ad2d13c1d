"""ctypes binding of libentropack_hip.so: the C ABI of include/entropack.h, same names.

Argument marshalling only.  Every computation happens in the library (host
encoder, HIP kernels); there is no Python or CPU fallback.  Loading fails loudly
when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# EP_LIB_PATH selects another build of the same C ABI (the host-only sanitizer build,
# which exports the host entry points alone)
LIB_PATH = os.environ.get("EP_LIB_PATH") or os.path.join(HERE, "libentropack_hip.so")

EP_BF16, EP_FP16, EP_FP32, EP_FP8_E4M3FN, EP_INT8 = 1, 2, 3, 4, 5
ERRORS = {0: "EP_OK", -1: "EP_E_ARG", -2: "EP_E_RANGE", -3: "EP_E_DTYPE", -4: "EP_E_SHAPE",
          -5: "EP_E_NONFINITE", -6: "EP_E_CORRUPT", -7: "EP_E_NOMEM", -8: "EP_E_DEVICE",
          -9: "EP_E_WORKSPACE", -10: "EP_E_STATE"}

# every symbol include/entropack.h declares, with (restype, argtypes)
_vp, _i64, _int, _dbl, _sz, _flt = C.c_void_p, C.c_int64, C.c_int, C.c_double, C.c_size_t, C.c_float
SIGNATURES = {
    "ep_compress": (_int, [_vp, _int, _i64, _i64, _dbl, C.POINTER(_vp)]),
    "ep_compress_ex": (_int, [_vp, _int, _i64, _i64, _dbl, _int, C.POINTER(_vp)]),
    "ep_blob_upload": (_int, [_vp, _vp]),
    "ep_device_bytes": (_sz, [_vp]),
    "ep_decompress": (_int, [_vp, _vp, _vp]),
    "ep_decompress_tiles": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "ep_decompress_batch": (_int, [C.POINTER(_vp), C.POINTER(_vp), _int, _vp]),
    "ep_test_decode_coords": (_int, [_vp, _vp, _vp]),
    "ep_blob_device_errors": (_i64, [_vp]),
    "ep_linear_workspace_bytes": (_sz, [_vp]),
    "ep_compressed_linear_forward": (_int, [_vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "ep_linear_seq_workspace_bytes": (_sz, [C.POINTER(_vp), _int]),
    "ep_matvec_workspace_bytes": (_sz, [_vp, _i64]),
    "ep_compressed_matvec": (_int, [_vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "ep_compressed_matvec_noalloc": (_int, [_vp, _vp, _i64, _vp, _vp, _vp]),
    "ep_compressed_linear_prefill": (_int, [_vp, _vp, _i64, _vp, _vp, _vp]),
    "ep_test_cast": (_int, [_int, _vp, _vp, _i64, _int, _vp]),
    "ep_matvec_batch_workspace_bytes": (_sz, [C.POINTER(_vp), _int, _i64]),
    "ep_compressed_matvec_batch": (_int, [C.POINTER(_vp), _int, _vp, _i64, C.POINTER(_vp), C.POINTER(_vp), _vp, _sz,
                                          _vp]),
    "ep_compressed_linear_seq_forward": (_int, [C.POINTER(_vp), _int, C.POINTER(_vp), _i64, C.POINTER(_vp),
                                                C.POINTER(_vp), _vp, _sz, _vp, _vp]),
    "ep_gemm_bf16_nt": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "ep_gemm_fp8_nt": (_int, [_vp, _vp, _flt, _vp, _vp, _i64, _i64, _i64, _vp]),
    "ep_plan_bitrates": (_int, [_int, _int, C.POINTER(_dbl), C.POINTER(_dbl), _dbl, C.POINTER(_int)]),
    "ep_blob_distortion": (_int, [_vp, C.POINTER(_dbl), C.POINTER(_dbl)]),
    "ep_actual_bpp": (_dbl, [_vp]),
    "ep_compress_device": (_int, [_vp, _int, _i64, _i64, _dbl, _int, _vp, C.POINTER(_vp)]),
    "ep_compress_device_batch": (_int, [C.POINTER(_vp), C.POINTER(_i64), C.POINTER(_i64), _int, _int, _dbl, _int,
                                        _vp, C.POINTER(_vp)]),
    "ep_compress_lossless": (_int, [_vp, _i64, _int, C.POINTER(_i64), _int, _int, _int, C.POINTER(_vp)]),
    "ep_blob_kind": (_int, [_vp]),
    "ep_blob_dims": (_int, [_vp, C.POINTER(_i64), _int]),
    "ep_blob_elem_bytes": (_int, [_vp]),
    "ep_blob_shape": (None, [_vp, C.POINTER(_i64), C.POINTER(_i64)]),
    "ep_blob_dtype": (_int, [_vp]),
    "ep_blob_params": (None, [_vp, C.POINTER(_int), C.POINTER(_int), C.POINTER(_int)]),
    "ep_serialized_size": (_sz, [_vp]),
    "ep_serialize": (_int, [_vp, _vp, _sz]),
    "ep_deserialize": (_int, [_vp, _sz, C.POINTER(_vp)]),
    "ep_blob_free": (None, [_vp]),
    "ep_last_error": (C.c_char_p, []),
}


class EPError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


_lib = None


def lib():
    """Load the shared library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_tile_rans_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            if os.environ.get("EP_LIB_PATH") and not hasattr(L, name):
                continue
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(rc: int):
    if rc != 0:
        msg = lib().ep_last_error()
        raise EPError(rc, msg.decode() if msg else "")
    return rc


# ------------------------------------------------------------------ same-name wrappers
def ep_compress(host_src_ptr: int, dtype: int, rows: int, cols: int, target_bpp: float,
                chains_per_tile: int = 0) -> int:
    out = C.c_void_p()
    check(lib().ep_compress_ex(host_src_ptr, dtype, rows, cols, target_bpp, chains_per_tile, C.byref(out)))
    return out.value


def ep_blob_upload(blob: int, stream: int = 0):
    check(lib().ep_blob_upload(blob, stream))


def ep_decompress(blob: int, dev_dst: int, stream: int = 0):
    check(lib().ep_decompress(blob, dev_dst, stream))


def ep_decompress_tiles(blob: int, tile_begin: int, tile_end: int, dev_dst: int, stream: int = 0):
    check(lib().ep_decompress_tiles(blob, tile_begin, tile_end, dev_dst, stream))


def ep_decompress_batch(blobs, dsts, stream: int = 0):
    n = len(blobs)
    ba = (C.c_void_p * n)(*blobs)
    da = (C.c_void_p * n)(*dsts)
    check(lib().ep_decompress_batch(ba, da, n, stream))


def ep_test_decode_coords(blob: int, dev_u: int, stream: int = 0):
    check(lib().ep_test_decode_coords(blob, dev_u, stream))


def ep_blob_device_errors(blob: int) -> int:
    return int(lib().ep_blob_device_errors(blob))


def ep_linear_workspace_bytes(blob: int) -> int:
    return int(lib().ep_linear_workspace_bytes(blob))


def ep_compressed_linear_forward(blob, dev_x, T, dev_bias, dev_y, dev_ws, ws_bytes, stream=0):
    check(lib().ep_compressed_linear_forward(blob, dev_x, T, dev_bias, dev_y, dev_ws, ws_bytes, stream))


def ep_test_cast(dtype, dev_in, dev_out, n, hw=0, stream=0):
    check(lib().ep_test_cast(dtype, dev_in, dev_out, n, hw, stream))


def ep_device_bytes(blob: int) -> int:
    return int(lib().ep_device_bytes(blob))


def ep_matvec_workspace_bytes(blob: int, T: int) -> int:
    return int(lib().ep_matvec_workspace_bytes(blob, T))


def ep_compressed_matvec(blob, dev_x, T, dev_bias, dev_y, dev_ws, ws_bytes, stream=0):
    check(lib().ep_compressed_matvec(blob, dev_x, T, dev_bias, dev_y, dev_ws, ws_bytes, stream))


def ep_compressed_matvec_noalloc(blob, dev_x, T, dev_bias, dev_y, stream=0):
    check(lib().ep_compressed_matvec_noalloc(blob, dev_x, T, dev_bias, dev_y, stream))


def ep_compressed_linear_prefill(blob, dev_x, T, dev_bias, dev_y, stream=0):
    check(lib().ep_compressed_linear_prefill(blob, dev_x, T, dev_bias, dev_y, stream))


def _ptrs(seq):
    return (_vp * len(seq))(*[p if p else None for p in seq])


def ep_matvec_batch_workspace_bytes(blobs, T) -> int:
    return int(lib().ep_matvec_batch_workspace_bytes(_ptrs(blobs), len(blobs), T))


def ep_compressed_matvec_batch(blobs, dev_x, T, dev_biases, dev_ys, dev_ws, ws_bytes, stream=0):
    biases = _ptrs(dev_biases) if dev_biases is not None else None
    check(lib().ep_compressed_matvec_batch(_ptrs(blobs), len(blobs), dev_x, T, biases, _ptrs(dev_ys), dev_ws,
                                           ws_bytes, stream))


def ep_linear_seq_workspace_bytes(blobs) -> int:
    return int(lib().ep_linear_seq_workspace_bytes(_ptrs(blobs), len(blobs)))


def ep_compressed_linear_seq_forward(blobs, dev_xs, T, dev_biases, dev_ys, dev_ws, ws_bytes, main_stream, side_stream):
    n = len(blobs)
    bias = _ptrs(dev_biases) if dev_biases is not None else None
    check(lib().ep_compressed_linear_seq_forward(_ptrs(blobs), n, _ptrs(dev_xs), T, bias, _ptrs(dev_ys), dev_ws,
                                                 ws_bytes, main_stream, side_stream))


def ep_gemm_bf16_nt(dev_x, dev_w, dev_bias, dev_y, T, N, K, stream=0):
    check(lib().ep_gemm_bf16_nt(dev_x, dev_w, dev_bias, dev_y, T, N, K, stream))


def ep_gemm_fp8_nt(dev_xq, dev_wq, a_x, dev_aw, dev_y, T, N, K, stream=0):
    check(lib().ep_gemm_fp8_nt(dev_xq, dev_wq, a_x, dev_aw, dev_y, T, N, K, stream))


def ep_plan_bitrates(bits, cost, budget_bits):
    """bits, cost: n x n_cand nested sequences. Returns the chosen candidate per matrix."""
    n, m = len(bits), len(bits[0])
    fb = (_dbl * (n * m))(*[float(v) for row in bits for v in row])
    fc = (_dbl * (n * m))(*[float(v) for row in cost for v in row])
    out = (_int * n)()
    check(lib().ep_plan_bitrates(n, m, fb, fc, float(budget_bits), out))
    return list(out)


def ep_blob_distortion(blob: int):
    e, r = _dbl(), _dbl()
    check(lib().ep_blob_distortion(blob, C.byref(e), C.byref(r)))
    return e.value, r.value


def ep_compress_device(dev_ptr: int, dtype: int, rows: int, cols: int, target_bpp: float,
                       chains_per_tile: int = 0, stream: int = 0) -> int:
    out = _vp()
    check(lib().ep_compress_device(dev_ptr, dtype, rows, cols, float(target_bpp), chains_per_tile, stream,
                                   C.byref(out)))
    return out.value


def ep_compress_device_batch(dev_ptrs, shapes, dtype: int, target_bpp: float, chains_per_tile: int = 0,
                             stream: int = 0):
    n = len(dev_ptrs)
    src = (_vp * n)(*dev_ptrs)
    rows = (_i64 * n)(*[int(r) for r, _ in shapes])
    cols = (_i64 * n)(*[int(c) for _, c in shapes])
    out = (_vp * n)()
    check(lib().ep_compress_device_batch(src, rows, cols, n, dtype, float(target_bpp), chains_per_tile, stream, out))
    return [out[i] for i in range(n)]


def ep_compress_lossless(src_ptr: int, n_bytes: int, elem_bytes: int, dims, dtype_tag: int = 0,
                         chains_per_tile: int = 0) -> int:
    d = (_i64 * len(dims))(*[int(v) for v in dims])
    out = _vp()
    check(lib().ep_compress_lossless(src_ptr, n_bytes, elem_bytes, d, len(dims), dtype_tag, chains_per_tile,
                                     C.byref(out)))
    return out.value


def ep_blob_kind(blob: int) -> int:
    return int(lib().ep_blob_kind(blob))


def ep_blob_dims(blob: int):
    d = (_i64 * 8)()
    n = lib().ep_blob_dims(blob, d, 8)
    return tuple(int(d[i]) for i in range(n))


def ep_blob_elem_bytes(blob: int) -> int:
    return int(lib().ep_blob_elem_bytes(blob))


def ep_actual_bpp(blob: int) -> float:
    return float(lib().ep_actual_bpp(blob))


def ep_blob_shape(blob: int):
    r, c = C.c_int64(), C.c_int64()
    lib().ep_blob_shape(blob, C.byref(r), C.byref(c))
    return r.value, c.value


def ep_blob_dtype(blob: int) -> int:
    return int(lib().ep_blob_dtype(blob))


def ep_blob_params(blob: int):
    s, k, f = C.c_int(), C.c_int(), C.c_int()
    lib().ep_blob_params(blob, C.byref(s), C.byref(k), C.byref(f))
    return s.value, k.value, f.value


def ep_serialized_size(blob: int) -> int:
    return int(lib().ep_serialized_size(blob))


def ep_serialize(blob: int) -> bytes:
    n = ep_serialized_size(blob)
    buf = (C.c_uint8 * n)()
    check(lib().ep_serialize(blob, buf, n))
    return bytes(buf)


def ep_deserialize(data: bytes) -> int:
    out = C.c_void_p()
    buf = (C.c_uint8 * len(data)).from_buffer_copy(data)
    check(lib().ep_deserialize(buf, len(data), C.byref(out)))
    return out.value


def ep_blob_free(blob: int):
    lib().ep_blob_free(blob)


def ep_last_error() -> str:
    m = lib().ep_last_error()
    return m.decode() if m else ""
