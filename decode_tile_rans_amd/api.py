"""High-level Python API over the C ABI ([README] 快速开始: compress / decompress /
CompressedLinear.from_linear; [NEWS]: results stored through state_dict).

Marshalling only: tensors are handed to the library as raw pointers; torch
provides device memory and the current HIP stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L
from ._lib import EPError

_TORCH_TO_EP = {torch.bfloat16: L.EP_BF16, torch.float16: L.EP_FP16, torch.float32: L.EP_FP32,
                torch.float8_e4m3fn: L.EP_FP8_E4M3FN, torch.int8: L.EP_INT8}
_EP_TO_TORCH = {v: k for k, v in _TORCH_TO_EP.items()}
# TileANS blobs carry the tensor's dtype as a tag (an index into this list)
_LOSSLESS_DTYPES = [torch.bfloat16, torch.float16, torch.float32, torch.float64, torch.float8_e4m3fn,
                    torch.float8_e5m2, torch.int8, torch.uint8, torch.int16, torch.int32, torch.int64, torch.bool,
                    torch.uint16, torch.uint32, torch.uint64, torch.complex64]


def _stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Compressed:
    """A compressed 2-D tensor (owns an ep_blob: host bytes + device copy)."""

    def __init__(self, handle: int):
        self._h = handle
        self.lossless = L.ep_blob_kind(handle) == 1
        if self.lossless:
            self.shape = L.ep_blob_dims(handle)
            self.ep_dtype = None
            self.dtype = _LOSSLESS_DTYPES[L.ep_blob_dtype(handle)]
        else:
            self.shape = L.ep_blob_shape(handle)
            self.ep_dtype = L.ep_blob_dtype(handle)
            self.dtype = _EP_TO_TORCH[self.ep_dtype]
        self.chains_per_tile, self.k_log2, self.flags = L.ep_blob_params(handle)

    @property
    def handle(self) -> int:
        return self._h

    @property
    def actual_bpp(self) -> float:
        """Stored bits per parameter including all metadata ([README] 快速开始)."""
        return L.ep_actual_bpp(self._h)

    @property
    def distortion(self):
        """(sum (w - h_r u)^2, sum w^2) of the lattice reconstruction, float64; known
        only for blobs compressed in this process (EPError otherwise)."""
        return L.ep_blob_distortion(self._h)

    @property
    def nbytes(self) -> int:
        return L.ep_serialized_size(self._h)

    @property
    def device_bytes(self) -> int:
        """Bytes of GPU memory the uploaded blob holds (0 before upload)."""
        return L.ep_device_bytes(self._h)

    def to_bytes(self) -> bytes:
        return L.ep_serialize(self._h)

    @classmethod
    def from_bytes(cls, data: bytes) -> "Compressed":
        return cls(L.ep_deserialize(bytes(data)))

    def upload(self, stream=None):
        L.ep_blob_upload(self._h, _stream_ptr(stream))
        return self

    def device_errors(self) -> int:
        return L.ep_blob_device_errors(self._h)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            try:
                L.ep_blob_free(h)
            except Exception:
                pass


def compress(x, target_bpp: float, dtype=None, chains_per_tile: int = 0, stream=None) -> Compressed:
    """Compress a 2-D tensor (torch on any device, or numpy with ``dtype`` = torch dtype).

    A tensor on the GPU is compressed there (ep_compress_device); the blob is the same,
    byte for byte, as the host encoder's."""
    if isinstance(x, torch.Tensor) and x.is_cuda:
        if x.dim() != 2:
            raise EPError(-4, "lossy compression takes 2-D tensors only")
        if x.dtype not in _TORCH_TO_EP:
            raise EPError(-3, f"unsupported dtype {x.dtype}")
        xc = x.detach().contiguous()
        h = L.ep_compress_device(xc.data_ptr(), _TORCH_TO_EP[xc.dtype], xc.shape[0], xc.shape[1], float(target_bpp),
                                 chains_per_tile, _stream_ptr(stream))
        return Compressed(h)
    if isinstance(x, np.ndarray):
        if dtype is None:
            raise ValueError("numpy input needs dtype= (a torch dtype)")
        host = np.ascontiguousarray(x)
        ep_dt = _TORCH_TO_EP[dtype]
        ptr = host.ctypes.data
    else:
        if x.dim() != 2:
            raise EPError(-4, "lossy compression takes 2-D tensors only")
        if x.dtype not in _TORCH_TO_EP:
            raise EPError(-3, f"unsupported dtype {x.dtype}")
        host = x.detach().to("cpu").contiguous()
        ep_dt = _TORCH_TO_EP[x.dtype]
        ptr = host.data_ptr()
    if len(host.shape) != 2:
        raise EPError(-4, "lossy compression takes 2-D tensors only")
    h = L.ep_compress(ptr, ep_dt, host.shape[0], host.shape[1], float(target_bpp), chains_per_tile)
    return Compressed(h)


def compress_many(tensors, target_bpp: float, chains_per_tile: int = 0, stream=None):
    """compress() over several 2-D tensors at one target; CUDA tensors of one dtype go
    through the GPU encoder's batch entry (several matrices in flight at once)."""
    tensors = list(tensors)
    if tensors and all(isinstance(t, torch.Tensor) and t.is_cuda and t.dim() == 2 for t in tensors) and \
            len({t.dtype for t in tensors}) == 1 and tensors[0].dtype in _TORCH_TO_EP:
        xs = [t.detach().contiguous() for t in tensors]
        hs = L.ep_compress_device_batch([x.data_ptr() for x in xs], [tuple(x.shape) for x in xs],
                                        _TORCH_TO_EP[xs[0].dtype], float(target_bpp), chains_per_tile,
                                        _stream_ptr(stream))
        return [Compressed(h) for h in hs]
    return [compress(t, target_bpp, chains_per_tile=chains_per_tile, stream=stream) for t in tensors]


def compress_lossless(x: torch.Tensor, chains_per_tile: int = 0) -> Compressed:
    """TileANS: a bit-exact compressed copy of a tensor of any shape and of the dtypes in
    ``_LOSSLESS_DTYPES`` ([README] Config：压缩配置 TileANSConfig)."""
    if x.dtype not in _LOSSLESS_DTYPES:
        raise EPError(-3, f"unsupported dtype {x.dtype}")
    host = x.detach().to("cpu").contiguous()
    shape = tuple(host.shape) if host.dim() > 0 else (1,)
    raw = host.reshape(-1).view(torch.uint8)
    h = L.ep_compress_lossless(raw.data_ptr(), raw.numel(), host.element_size(), shape,
                               _LOSSLESS_DTYPES.index(host.dtype), chains_per_tile)
    return Compressed(h)


def plan_bitrates(mats, budget_bpp: float, candidates=(2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0), weights=None,
                  dtype=None, chains_per_tile: int = 0):
    """Compress every matrix at one of ``candidates`` so that all of them together take
    at most ``budget_bpp`` x (total parameters) stored bits and the summed cost
    weight_i x squared reconstruction error is small (ep_plan_bitrates).

    The default weights (all 1) minimise the stack's overall relative L2 error
    sqrt(sum err / sum |W|^2).  Each matrix is compressed once per candidate to
    measure (bits, error) and once more at its chosen target (the encoder is
    deterministic, so the bits match).  Returns (list of Compressed, chosen targets).
    """
    mats = list(mats)
    cands = [float(t) for t in candidates]
    if weights is None:
        weights = [1.0] * len(mats)
    bits, cost, numel = [], [], 0
    for x, wgt in zip(mats, weights):
        row_b, row_c = [], []
        for t in cands:
            c = compress(x, t, dtype=dtype, chains_per_tile=chains_per_tile)
            n = c.shape[0] * c.shape[1]
            row_b.append(c.actual_bpp * n)
            row_c.append(float(wgt) * c.distortion[0])
            del c
        bits.append(row_b)
        cost.append(row_c)
        numel += n
    choice = L.ep_plan_bitrates(bits, cost, float(budget_bpp) * numel)
    out = [compress(x, cands[j], dtype=dtype, chains_per_tile=chains_per_tile) for x, j in zip(mats, choice)]
    return out, [cands[j] for j in choice]


def decompress(c: Compressed, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode on the current GPU into a new (or given) tensor of the original shape/dtype
    (both blob kinds)."""
    c.upload(stream)
    if out is None:
        out = torch.empty(c.shape, dtype=c.dtype, device="cuda")
    L.ep_decompress(c.handle, out.data_ptr(), _stream_ptr(stream))
    return out


def decompress_batch(cs, outs=None, stream=None):
    for c in cs:
        c.upload(stream)
    if outs is None:
        outs = [torch.empty(c.shape, dtype=c.dtype, device="cuda") for c in cs]
    L.ep_decompress_batch([c.handle for c in cs], [o.data_ptr() for o in outs], _stream_ptr(stream))
    return outs


def gemm_bf16_nt(x: torch.Tensor, w: torch.Tensor, bias=None, out=None, stream=None) -> torch.Tensor:
    T, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    L.ep_gemm_bf16_nt(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                      out.data_ptr(), T, N, K, _stream_ptr(stream))
    return out


def gemm_fp8_nt(xq: torch.Tensor, wq: torch.Tensor, a_x: float, a_w: torch.Tensor, out=None, stream=None):
    T, K = xq.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=xq.device)
    L.ep_gemm_fp8_nt(xq.data_ptr(), wq.data_ptr(), float(a_x), a_w.data_ptr(), out.data_ptr(), T, N, K,
                     _stream_ptr(stream))
    return out


class CompressedLinear(torch.nn.Module):
    """Drop-in replacement of a BF16 ``torch.nn.Linear`` whose weight is stored compressed.

    forward(x) decodes the weight into a workspace and runs the MFMA GEMM
    (ep_compressed_linear_forward); with at most 8 input rows the decode kernel forms
    the product itself and no weights are written.  The compressed bytes live in the
    ``packed`` buffer so they travel with ``state_dict``.
    """

    def __init__(self, c: Compressed, bias: torch.Tensor | None = None):
        super().__init__()
        self._c = c
        self.out_features, self.in_features = c.shape
        self.register_buffer("packed", torch.frombuffer(bytearray(c.to_bytes()), dtype=torch.uint8))
        self.register_buffer("bias", bias)
        self._ws = None

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, target_bpp: float = 4.0, chains_per_tile: int = 0):
        w = linear.weight.detach()
        if w.dtype != torch.bfloat16:
            w = w.to(torch.bfloat16)
        c = compress(w, target_bpp, chains_per_tile=chains_per_tile)
        b = None
        if linear.bias is not None:
            b = linear.bias.detach().to(torch.bfloat16).to(linear.weight.device)
        return cls(c, b)

    @property
    def compressed_bits(self) -> float:
        return self._c.actual_bpp

    def _load_from_state_dict(self, state_dict, prefix, *args, **kwargs):
        # The stored blob's length depends on the weight and its target rate, so the
        # ``packed`` buffer takes the incoming length before the copy; the blob is parsed
        # (and a corrupt one refused) before anything of the module changes, and the
        # handle is rebuilt from the bytes that actually landed in ``packed``.
        key = prefix + "packed"
        if key in state_dict:
            incoming = state_dict[key]
            Compressed.from_bytes(incoming.detach().cpu().contiguous().numpy().tobytes())
            if incoming.shape != self.packed.shape:
                self.packed = torch.empty(incoming.shape, dtype=torch.uint8, device=self.packed.device)
        super()._load_from_state_dict(state_dict, prefix, *args, **kwargs)
        if key in state_dict:
            self._c = Compressed.from_bytes(self.packed.detach().cpu().numpy().tobytes())
            self.out_features, self.in_features = self._c.shape
            self._ws = None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        self._c.upload()
        need = L.ep_linear_workspace_bytes(self._c.handle)
        if self._ws is None or self._ws.numel() < need or self._ws.device != x2.device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=x2.device)
        y = torch.empty((x2.shape[0], self.out_features), dtype=torch.bfloat16, device=x2.device)
        b = self.bias.data_ptr() if self.bias is not None else None
        L.ep_compressed_linear_forward(self._c.handle, x2.data_ptr(), x2.shape[0], b, y.data_ptr(),
                                       self._ws.data_ptr(), need, _stream_ptr())
        return y.reshape(*lead, self.out_features)


def linear_batch(layers, x: torch.Tensor):
    """Several CompressedLinear layers applied to the same input (e.g. a block's query,
    key and value projections): [layer(x) for layer in layers], bit for bit.  With at most
    8 input rows the layers' decodes share launches (ep_compressed_matvec_batch)."""
    layers = list(layers)
    if not layers:
        return []
    lead = x.shape[:-1]
    x2 = x.reshape(-1, layers[0].in_features).to(torch.bfloat16).contiguous()
    T = x2.shape[0]
    for m in layers:
        m._c.upload()
    hs = [m._c.handle for m in layers]
    need = L.ep_matvec_batch_workspace_bytes(hs, T) if all(m.in_features == layers[0].in_features for m in layers) else 0
    fused = need > 0 and all(L.ep_matvec_workspace_bytes(h, T) <= L.ep_linear_workspace_bytes(h) for h in hs)
    if not fused:
        return [m(x) for m in layers]
    ws = torch.empty(need, dtype=torch.uint8, device=x2.device)
    ys = [torch.empty((T, m.out_features), dtype=torch.bfloat16, device=x2.device) for m in layers]
    biases = [m.bias.data_ptr() if m.bias is not None else None for m in layers]
    L.ep_compressed_matvec_batch(hs, x2.data_ptr(), T, biases, [y.data_ptr() for y in ys], ws.data_ptr(), need,
                                 _stream_ptr())
    return [y.reshape(*lead, m.out_features) for y, m in zip(ys, layers)]
