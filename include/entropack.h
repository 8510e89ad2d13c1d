/*
 * entropack.h — C ABI of libentropack_hip.so, a gfx950 (MI355X) implementation of
 * EntroPack-style lossy weight compression: row-normalised E8 lattice quantisation,
 * a conditional model of the lattice coordinates, rANS in independently decodable
 * tiles, and fused GPU decode (symbol decode, algebraic inverse-lattice
 * reconstruction, per-row rescale, container cast) feeding an MFMA GEMM.
 *
 * Sources (the only specification; cited by page title and section):
 *  [ABS]    "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at Arbitrary
 *           Bitrates", English abstract (arxivdaily.com / modelscope.ai paper pages):
 *           E8 + conditional model, sampled rate selection, independently decodable
 *           tiles, BF16/FP16/FP8/INT8 containers, decode cost grows with weight count.
 *  [SUM]    same paper, modelscope.ai page, section "摘要": rANS tiles; symbol decode,
 *           algebraic inverse-lattice reconstruction and row rescale fused on the GPU
 *           with no intermediate symbol tensor and no reconstruction codebook.
 *  [README] EntroPack README_zh.md, section "快速开始": compress/decompress restore shape
 *           and dtype; 0.001 <= target_bpp <= 11 (finite, non-integer allowed);
 *           actual_bpp includes metadata; CompressedLinear.from_linear / layer(x).
 *           Section "Config：压缩配置": lossy mode for 2-D float and integer tensors.
 *  [NEWS]   techmoon.xyz, "EntroPack 開源模型壓縮…", section "任意位元率的本體…": lossy
 *           mode only for 2-D tensors; results saved with state_dict; FP8@5 packs use
 *           an FP8 GEMM at inference.
 *
 * Conventions
 *  - Every function returning int returns EP_OK (0) or a negative EP_E_* code; the
 *    calling thread's message is available from ep_last_error().
 *  - "host" pointers are CPU memory, "dev" pointers are device memory of the current
 *    HIP device.  The caller owns every pointer it passes; the library owns ep_blob
 *    (host bytes + device copy) and frees both in ep_blob_free().
 *  - GPU work is asynchronous on the given hipStream_t (NULL = default stream);
 *    device-side errors (a corrupt stream failing the final-state check) are counted
 *    in the blob and read back by ep_blob_device_errors() after synchronisation.
 *  - Matrices are row-major.  BF16/FP16/FP8 elements are passed as their bit patterns.
 */
#ifndef ENTROPACK_H
#define ENTROPACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ep_blob ep_blob;
typedef struct ihipStream_t* ep_stream;   /* a hipStream_t */

enum {
  EP_BF16 = 1,          /* bfloat16 */
  EP_FP16 = 2,          /* IEEE binary16 */
  EP_FP32 = 3,          /* IEEE binary32 */
  EP_FP8_E4M3FN = 4,    /* OCP FP8 E4M3FN (bias 7, max 448, no Inf) */
  EP_INT8 = 5           /* two's complement int8 */
};

enum {
  EP_OK = 0,
  EP_E_ARG = -1,        /* null pointer, rows/cols < 1, bad option */
  EP_E_RANGE = -2,      /* target_bpp not finite / outside [0.001, 11] / above the 8-bit
                           container cap of 8; or a nonzero row whose RMS is below the
                           BF16 normal range */
  EP_E_DTYPE = -3,      /* container not one of the five above */
  EP_E_SHAPE = -4,      /* not a 2-D tensor (raised by the Python layer) */
  EP_E_NONFINITE = -5,  /* NaN or Inf in the input */
  EP_E_CORRUPT = -6,    /* blob failed validation */
  EP_E_NOMEM = -7,      /* host or device allocation failed */
  EP_E_DEVICE = -8,     /* a HIP runtime error */
  EP_E_WORKSPACE = -9,  /* workspace smaller than ep_linear_workspace_bytes() */
  EP_E_STATE = -10      /* blob not uploaded to the device */
};

/* ---------------------------------------------------------------- compression
 * ep_compress — [ABS], [README] 快速开始, [NEWS].
 * Compress a rows x cols host matrix of container `dtype` at `target_bpp` bits per
 * parameter (the data part; actual_bpp adds the metadata).  Runs on the host CPU
 * (multi-threaded; EP_NUM_THREADS caps the thread count) and is deterministic: the
 * same input gives the same bytes on any machine.  `chains_per_tile` = 0 picks the
 * default (8 for rows*cols >= 2^22, else 1); otherwise one of 1,2,4,8,16,32,64.
 * On success *out owns a host-only blob (call ep_blob_upload before decoding). */
int ep_compress(const void* host_src, int dtype, int64_t rows, int64_t cols,
                double target_bpp, ep_blob** out);
int ep_compress_ex(const void* host_src, int dtype, int64_t rows, int64_t cols,
                   double target_bpp, int chains_per_tile, ep_blob** out);

/* The same compression on the GPU ([README] 快速开始 / [NEWS]: GPU encode and decode;
 * [README] 性能: 276 layers compressed in seconds): dev_src is a device array of rows x
 * cols container values; row statistics, the E8 quantisation of every resolution probe,
 * the symbol counts, the rANS chains, the fetch schedule and the stream layout run on
 * the device (on `stream`; the call returns when the blob is complete), the search
 * and model construction on the host.  The blob is byte-identical to ep_compress_ex's
 * with the same arguments.  Uses temporary device memory of about 36 bytes per
 * coordinate plus 50 bytes per group of 8 at one chain per tile.  Errors as
 * ep_compress_ex, plus EP_E_NOMEM / EP_E_DEVICE. */
int ep_compress_device(const void* dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                       int chains_per_tile, ep_stream stream, ep_blob** out);

/* The GPU encoder over n matrices of one dtype and target (a whole model's layers,
 * [README] 性能: the 276 layers compressed in seconds): dev_src[i] is rows[i] x cols[i],
 * out[i] (caller-owned array of n) receives blob i, equal byte for byte to
 * ep_compress_device's.  Work already queued on `stream` completes first; the matrices
 * are then encoded by up to four host threads on streams of their own, and the call
 * returns when all are done.  On an error no blob is returned (every out[i] NULL) and
 * the message names the first failing matrix. */
int ep_compress_device_batch(const void* const* dev_src, const int64_t* rows, const int64_t* cols, int n,
                             int dtype, double target_bpp, int chains_per_tile, ep_stream stream,
                             ep_blob** out);

/* TileANS lossless compression ([README] Config：压缩配置: a lossless codec for BF16, FP16,
 * FP32, FP8, INT8 and other dtypes whose ratio depends on the data; [NEWS]: tensors
 * that are not 2-D take the lossless way).  host_src: the tensor's n_bytes raw bytes
 * (C order, little-endian elements of elem_bytes = 1, 2, 4 or 8 bytes), dims[ndim]
 * its shape (ndim 1..8, n_bytes = elem_bytes x prod(dims)), dtype_tag an opaque
 * 0..255 label returned by ep_blob_dtype.  Bytes are coded with per-byte-position
 * tables (byte index mod min(elem_bytes, 4)) or raw, in the lossy blob's tiles,
 * chains and stream layout.  chains_per_tile 0 = default (8 from 4 MiB on, else 1).
 * Decoded with ep_decompress / ep_decompress_tiles (tiles of 4096 bytes) /
 * ep_decompress_batch into n_bytes (16-byte aligned).  Errors: EP_E_ARG, EP_E_SHAPE,
 * EP_E_NOMEM. */
int ep_compress_lossless(const void* host_src, int64_t n_bytes, int elem_bytes, const int64_t* dims, int ndim,
                         int dtype_tag, int chains_per_tile, ep_blob** out);

/* Copy the blob's stream and chain area (block offsets, chunk counts, tail lengths and
 * states, as stored), its row half-scales (float32) and the 7 expanded 2048-slot decode
 * tables to the current device (one allocation, one H2D copy enqueued on `stream`; the
 * host side waits for it).  The decoder derives each chain's stream offsets on the
 * device (one wave prefix sum per 64 chains), so nothing per chain is expanded.
 * Idempotent.  The device copy lives until ep_blob_free().  EP_E_ARG for streams of
 * 2^31 words or more, EP_E_NOMEM when an allocation fails. */
int ep_blob_upload(ep_blob* blob, ep_stream stream);

/* Bytes of device memory the blob holds (0 before ep_blob_upload): the resident cost
 * of a compressed weight, to set against its serialized size (actual_bpp). */
size_t ep_device_bytes(const ep_blob* blob);

/* ---------------------------------------------------------------- decode
 * ep_decompress — [SUM]: fused symbol decode + algebraic inverse lattice + row rescale.
 * Writes rows*cols elements of the blob's container dtype, row-major, to dev_dst.
 * No intermediate symbol or coordinate tensor is written.  Every decode entry point
 * refuses (EP_E_ARG, before any launch) a destination the GPU cannot dereference
 * (pageable host memory); device, managed and pinned host memory are accepted. */
int ep_decompress(const ep_blob* blob, void* dev_dst, ep_stream stream);

/* Decode only tiles [tile_begin, tile_end) (each 4096 coordinates = 512 groups of
 * 8 columns, row-major) into dev_dst; other elements are left untouched.  This is
 * the tile-independence of [ABS]. */
int ep_decompress_tiles(const ep_blob* blob, int64_t tile_begin, int64_t tile_end,
                        void* dev_dst, ep_stream stream);

/* Decode n blobs in one launch (e.g. all matrices of one transformer block);
 * dev_dsts[i] receives blob i.  Same results as n ep_decompress calls. */
int ep_decompress_batch(const ep_blob* const* blobs, void* const* dev_dsts, int n,
                        ep_stream stream);

/* Test hook: write the doubled lattice coordinates u (int32, rows*cols, u = 2p for
 * the E8 point p) instead of weights.  Same kernel, coordinate-emitting variant. */
int ep_test_decode_coords(const ep_blob* blob, int32_t* dev_u, ep_stream stream);

/* Test hook: the decoder's container casts of float32 values ([NEWS]: the stored dtype
 * is restored; BF16 and FP16 round to nearest even and saturate, FP8-E4M3FN rounds to
 * nearest even and saturates at 448, INT8 rounds half to even and clamps to [-128, 127])
 * applied to n device floats, writing n container elements to dev_out.  For FP8, hw = 1
 * uses the conversion instruction (after clamping), hw = 0 the bit manipulation; other
 * dtypes ignore hw.  EP_E_DTYPE for FP32 or unknown dtypes.  Asynchronous. */
int ep_test_cast(int dtype, const float* dev_in, void* dev_out, int64_t n, int hw, ep_stream stream);

/* Device-side error count of the blob (decodes whose rANS chains did not end in the
 * initial state).  Synchronises the device. */
int64_t ep_blob_device_errors(const ep_blob* blob);

/* ---------------------------------------------------------------- compressed linear
 * [README] 快速开始 (CompressedLinear.from_linear, layer(x)): y = x W^T (+ bias).
 * W is the decoded BF16 blob (rows = out features, cols = in features); x is T x cols
 * BF16, y is T x rows BF16, bias is rows BF16 or NULL.  The decode goes to dev_ws
 * (>= ep_linear_workspace_bytes bytes), then an MFMA BF16 GEMM with fp32
 * accumulation runs on the same stream.  With T <= 8, when ep_compressed_matvec takes
 * the blob and its partial sums fit ep_linear_workspace_bytes, that fused product runs
 * instead (for T >= 5 only where ep_compressed_linear_prefill does not take it);
 * otherwise, when ep_compressed_linear_prefill takes the blob and T (4096 or 8192 cols,
 * S = 8, T <= 256), that one (same result up to fp32 summation order; dev_ws unused).
 * x, y, bias and dev_ws must be
 * device, managed or pinned memory (EP_E_ARG otherwise, for every T, before any
 * launch).  Asynchronous. */
size_t ep_linear_workspace_bytes(const ep_blob* blob);
int ep_compressed_linear_forward(const ep_blob* w, const void* dev_x, int64_t T,
                                 const void* dev_bias, void* dev_y,
                                 void* dev_ws, size_t ws_bytes, ep_stream stream);

/* A sequence of compressed linear layers, y_i = x_i W_i^T (+ bias_i), i = 0..n-1
 * ([README] 快速开始 layer(x), applied layer after layer as a model runs them; [ABS]:
 * decoding cost grows with the weight count, so it should hide behind the GEMMs).
 * Each layer is decoded, then multiplied (layers that ep_compressed_linear_forward
 * sends to a fused product run that product on `main` instead).  The decode of layer i+1 runs on `side`, beside
 * the GEMM of layer i on `main`, when that GEMM has fewer output tiles than the GPU has
 * CUs (its workgroups leave CUs idle), on at most as many workgroups as there are idle
 * CUs; otherwise it runs on `main` before its GEMM (a decode workgroup cannot share a CU with a GEMM workgroup: their LDS needs add
 * up to more than a CU holds, so a side-stream decode could only take CUs away from a
 * GEMM that fills them).  Two weight buffers in dev_ws (>= ep_linear_seq_workspace_bytes
 * bytes) alternate.  x[i] is T x cols_i, y[i] is T x rows_i, bias may be NULL or hold
 * NULLs; every pointer must be device, managed or pinned memory (EP_E_ARG otherwise,
 * before any launch).  The side stream first waits for the work already queued on
 * `main`; all GEMMs run on `main`, so work queued on `main` afterwards sees every
 * output.  Asynchronous. */
size_t ep_linear_seq_workspace_bytes(const ep_blob* const* w, int n);
int ep_compressed_linear_seq_forward(const ep_blob* const* w, int n, const void* const* dev_x, int64_t T,
                                     const void* const* dev_bias, void* const* dev_y,
                                     void* dev_ws, size_t ws_bytes, ep_stream main, ep_stream side);

/* Fused decode and product for few activation rows (decode-time inference: [ABS] and
 * [README] 快速开始 decode weights on the spot inside the layer; [ABS]: decoding cost
 * grows with the weight count, which for T <= 8 rows dominates the product):
 * y = x W^T (+ bias) with the BF16 weights of W decoded and multiplied inside the decode
 * kernel, never written to memory.  x is T x cols BF16 (16-byte aligned), y is T x rows
 * BF16, bias rows BF16 or NULL, 1 <= T <= 8.  Takes lossy BF16 blobs with cols % 8 == 0
 * and at least S groups of 8 per row (cols >= 8 S); EP_E_ARG otherwise.  Each chain sums
 * w * x over its groups of one row in fp32 (two-term BF16 dot steps) into a partial sum
 * in dev_ws (>= ep_matvec_workspace_bytes(w, T) bytes, which returns 0 when the blob or
 * T is not taken); a second kernel adds a row's partial sums in a fixed order, adds the
 * bias and rounds to BF16, so repeated calls give identical bits.  For rows of whole
 * tiles (4096 or 8192 cols at S = 8 or 16) a row's chains share one wavefront and the decode
 * kernel adds their sums itself, in the same order (same bits; dev_ws unused).
 * Asynchronous. */
size_t ep_matvec_workspace_bytes(const ep_blob* w, int64_t T);
int ep_compressed_matvec(const ep_blob* w, const void* dev_x, int64_t T, const void* dev_bias,
                         void* dev_y, void* dev_ws, size_t ws_bytes, ep_stream stream);

/* Fused decode and product for prefill-sized activations ([SUM]: symbol decode,
 * inverse lattice and row rescale fused on the GPU with no intermediate tensor; [ABS]:
 * the method targets prefill, where a GEMM follows the decode): y = x W^T (+ bias) with
 * every K slab of W's BF16 weights decoded into an LDS operand tile that MFMAs multiply
 * by the activations, so the weights are decoded once and never written to memory.
 * Takes lossy BF16 blobs of 4096 or 8192 cols at S = 8 (one or two tiles per row) and
 * 1 <= T <= 256; EP_E_ARG otherwise (ep_compressed_linear_forward covers the rest).
 * x is T x 4096 BF16 (16-byte aligned), y is T x rows BF16 (8-byte aligned), bias rows
 * BF16 or NULL; all device, managed or pinned memory (EP_E_ARG otherwise, before any
 * launch).  No workspace.  fp32 accumulation (its order differs from the GEMM's), bias
 * added, rounded to BF16 (nearest even).  Asynchronous. */
int ep_compressed_linear_prefill(const ep_blob* w, const void* dev_x, int64_t T, const void* dev_bias,
                                 void* dev_y, ep_stream stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): ep_compressed_matvec with its partial sums in the
 * library's own scratch array instead of a caller workspace.  Same arguments, rules,
 * errors and bits as ep_compressed_matvec minus dev_ws / ws_bytes.  The array is one
 * file-scope device array of 16 MiB per GPU, held until the process ends; a blob whose
 * partial sums (ep_matvec_workspace_bytes(w, T) - 256 bytes) exceed it is refused with
 * EP_E_WORKSPACE before any launch (14336 x 4096 at S = 8 and T = 8 needs 11 MB).  No
 * hipMalloc, hipFree or other allocation is made.  Every call on one GPU shares that
 * array: calls that overlap on one GPU (other streams, other host threads) race and must
 * be ordered by the caller.  Nothing needs clearing between calls (each call writes
 * every partial sum it reads).  Asynchronous. */
int ep_compressed_matvec_noalloc(const ep_blob* w, const void* dev_x, int64_t T, const void* dev_bias,
                                 void* dev_y, ep_stream stream);

/* The fused product for n blobs that take the same activations (e.g. the query, key
 * and value projections of one layer): y[i] = x W_i^T (+ bias[i]), all W_i with the same
 * cols; bias may be NULL or hold NULLs.  The blobs' blocks share decode launches, which
 * fills the GPU better than n separate calls (one matrix of a few thousand rows leaves
 * most wave slots idle).  dev_ws >= ep_matvec_batch_workspace_bytes(w, n, T) (0 when a
 * blob or T is not taken).  Each y[i] equals ep_compressed_matvec's result for blob i,
 * bit for bit.  Same requirements and errors as ep_compressed_matvec, and EP_E_ARG when
 * the blobs' cols differ.  Asynchronous. */
size_t ep_matvec_batch_workspace_bytes(const ep_blob* const* w, int n, int64_t T);
int ep_compressed_matvec_batch(const ep_blob* const* w, int n, const void* dev_x, int64_t T,
                               const void* const* dev_bias, void* const* dev_y, void* dev_ws,
                               size_t ws_bytes, ep_stream stream);

/* Plain BF16 "NT" GEMM on MFMA: y[T x N] = x[T x K] w[N x K]^T (+ bias[N]), fp32
 * accumulate, BF16 out.  The uncompressed baseline of the linear layer.  x and w
 * 16-byte aligned, K % 8 == 0; every pointer must be device, managed or pinned memory
 * (EP_E_ARG otherwise, checked before any launch).  Asynchronous. */
int ep_gemm_bf16_nt(const void* dev_x, const void* dev_w, const void* dev_bias,
                    void* dev_y, int64_t T, int64_t N, int64_t K, ep_stream stream);

/* FP8 (E4M3FN) "NT" GEMM on MFMA ([NEWS]/[README] FP8@5: FP8 W8A8 codes, FP8 GEMM):
 * y[T x N] (BF16) = (xq[T x K] wq[N x K]^T) * a_x * a_w[N], fp32 accumulate.
 * a_w is a device float array (per output row), a_x a host float.  K % 16 == 0; the
 * same alignment and pointer rules as ep_gemm_bf16_nt. */
int ep_gemm_fp8_nt(const void* dev_xq, const void* dev_wq, float a_x, const float* dev_aw,
                   void* dev_y, int64_t T, int64_t N, int64_t K, ep_stream stream);

/* ---------------------------------------------------------------- budgeted bitrates
 * [ABS] arbitrary target rates from sampled storage estimates; [README] 性能 / [NEWS]:
 * whole-model packs at a fixed average rate.  ep_plan_bitrates spends a total bit
 * budget over n matrices, each with n_cand measured candidates: bits[i*n_cand + j] =
 * stored bits of matrix i at candidate j, cost[...] = the caller's weight x its squared
 * reconstruction error (both finite, >= 0).  Lagrangian pick (per matrix the candidate
 * minimising cost + lambda bits; ties: fewer bits, lower index; lambda = 0 or the
 * smallest pick-changing value that fits, else every matrix at its fewest bits), then
 * greedy upgrades by cost saved per extra bit while the budget allows (ties: lower
 * matrix, lower candidate).  choice[i] (caller-owned, n ints) receives the candidate
 * index of matrix i.  EP_E_ARG for null/empty/negative/non-finite input, EP_E_RANGE if
 * even the smallest candidates exceed the budget.  Host only, deterministic. */
int ep_plan_bitrates(int n, int n_cand, const double* bits, const double* cost, double budget_bits, int* choice);

/* Squared error of the lattice reconstruction fl32(h_r u) (before the container cast)
 * against the compressed input, and the input's squared norm, summed over all entries
 * in double (row by row, left to right).  Known for blobs made by ep_compress in this
 * process (EP_E_STATE otherwise). */
int ep_blob_distortion(const ep_blob* blob, double* sq_err, double* sq_ref);

/* ---------------------------------------------------------------- blob accessors
 * actual_bpp = 8 * serialized bytes / elements  ([README]: includes metadata).
 * ep_blob_shape: rows x cols of a lossy blob; 1 x elements of a TileANS blob.
 * ep_blob_dtype: EP_* container of a lossy blob; the caller's tag of a TileANS blob. */
double ep_actual_bpp(const ep_blob* blob);
void ep_blob_shape(const ep_blob* blob, int64_t* rows, int64_t* cols);
int ep_blob_dtype(const ep_blob* blob);
/* 0 = lossy (E8 lattice), 1 = TileANS (lossless); -1 for NULL */
int ep_blob_kind(const ep_blob* blob);
/* the tensor's shape: writes up to max_dims extents, returns the rank (lossy: 2) */
int ep_blob_dims(const ep_blob* blob, int64_t* dims, int max_dims);
/* bytes per element of the decoded tensor */
int ep_blob_elem_bytes(const ep_blob* blob);
/* chains per tile, K_LOG2, flags (bit0 escapes present, bit1 clamping needed) */
void ep_blob_params(const ep_blob* blob, int* chains_per_tile, int* k_log2, int* flags);

/* Serialise (the blob v2 bytes; what a state_dict stores, [NEWS]) / deserialise
 * with full validation (EP_E_CORRUPT on any inconsistency). */
size_t ep_serialized_size(const ep_blob* blob);
int ep_serialize(const ep_blob* blob, void* host_dst, size_t capacity);
int ep_deserialize(const void* host_src, size_t size, ep_blob** out);
void ep_blob_free(ep_blob* blob);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* ep_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ENTROPACK_H */
