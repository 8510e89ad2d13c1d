"""Helpers for the GPU parity tests (device buffers through torch, calls through the C ABI)."""
import os
import sys

import numpy as np

import oracle
from oracle import numerics as nx

TORCH_DT = None


def torch_dtype(dt):
    import torch
    return {nx.DT_BF16: torch.bfloat16, nx.DT_FP16: torch.float16, nx.DT_FP32: torch.float32,
            nx.DT_FP8: torch.uint8, nx.DT_INT8: torch.int8}[dt]


def np_view(dt):
    return {nx.DT_BF16: np.uint16, nx.DT_FP16: np.uint16, nx.DT_FP32: np.float32,
            nx.DT_FP8: np.uint8, nx.DT_INT8: np.int8}[dt]


def to_np(t, dt):
    """Device tensor -> numpy array of the container's raw element type."""
    import torch
    shape = tuple(t.shape)
    return t.detach().cpu().contiguous().view(torch.uint8).numpy().view(np_view(dt)).reshape(shape)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def stream_ptr():
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


class DevBlob:
    """An ep_blob made from serialized bytes and uploaded to the current GPU."""

    def __init__(self, data: bytes):
        from decode_tile_rans_amd import _lib as L
        self.L = L
        self.data = data
        self.h = L.ep_deserialize(data)
        L.ep_blob_upload(self.h, stream_ptr())
        self.R, self.C = L.ep_blob_shape(self.h)
        self.dt = L.ep_blob_dtype(self.h)

    def empty_out(self, fill=0):
        import torch
        t = torch.empty((self.R, self.C), dtype=torch_dtype(self.dt), device="cuda")
        t.view(torch.uint8).fill_(fill)
        return t

    def decode(self, fill=0):
        import torch
        out = self.empty_out(fill)
        self.L.ep_decompress(self.h, out.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        return to_np(out, self.dt)

    def decode_tiles(self, t0, t1, fill=0):
        import torch
        out = self.empty_out(fill)
        self.L.ep_decompress_tiles(self.h, t0, t1, out.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        return to_np(out, self.dt)

    def coords(self):
        import torch
        out = torch.zeros((self.R, self.C), dtype=torch.int32, device="cuda")
        self.L.ep_test_decode_coords(self.h, out.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def errors(self):
        return self.L.ep_blob_device_errors(self.h)

    def __del__(self):
        try:
            self.L.ep_blob_free(self.h)
        except Exception:
            pass


def linear_bound(ref, mag, K, scale_roundings=0):
    """Per-element error bound of a BF16-out product with fp32 accumulation.

    ref: exact (float64) outputs; mag: the same product of the absolute values (times
    any scales); K: terms per output.  Products of BF16 (or FP8) inputs are exact in
    fp32, so the fp32 sum of K terms (plus bias) is within (K + 1) 2^-24 mag of the exact
    one in any order (Higham's gamma_n bound), each fp32 scaling adds 2^-24 |ref|, and the
    final rounding to BF16 half an ulp, at most 2^-8 of the value."""
    u = 2.0 ** -24
    acc = (K + 1) * u * mag + scale_roundings * u * np.abs(ref)
    return 2.0 ** -8 * (np.abs(ref) + acc) + acc * 1.000001 + 1e-30


def check_linear(got, ref, mag, K, scale_roundings=0):
    """Every output within linear_bound; names the first offending element.  A NaN in
    the output, the reference or the bound counts as a failure (never a vacuous pass)."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    bound = linear_bound(ref, mag, K, scale_roundings)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, (f"{len(bad)} of {err.size} outputs off, first {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]} bound {bound[tuple(bad[0])]}")
