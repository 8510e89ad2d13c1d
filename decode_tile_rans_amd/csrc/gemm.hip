// MFMA GEMMs for the compressed linear layer on gfx950.
//
// [README] 快速开始: CompressedLinear.from_linear(...) returns a layer called as layer(x)
// that behaves like torch.nn.Linear, y = x W^T + b.  [ABS]: decoding cost grows with
// the weight count, so the method suits compute-heavy work (diffusion denoising,
// transformer prefill) where the GEMM dominates.  [NEWS] / [README] "FP8@5": FP8 W8A8
// weight codes compressed by EntroPack and an FP8 GEMM at inference.
//
// Both kernels are "NT": X [T x K] and W [N x K] are K-contiguous, Y = X W^T is
// [T x N] row-major BF16 with fp32 accumulation.  Workgroup tile 128 x 128, 4 waves
// in a 2 x 2 arrangement, each wave 64 x 64 = 2 x 2 MFMA 32x32 tiles; K tiles of 128
// bytes per row staged in LDS (double buffered through registers).
//   BF16: v_mfma_f32_32x32x16_bf16   (A/B: 8 bf16 per lane, lane -> row l%32,
//                                      k = 8 (l/32) .. +8)
//   FP8:  v_mfma_f32_32x32x64_f8f6f4 (A/B: 32 e4m3 per lane, k = 32 (l/32) .. +32)
//   D:    lane l holds column l%32, rows 8 (r/4) + 4 (l/32) + r%4 for r = 0..15.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ep_internal.h"

namespace ep {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 128;            // bytes of K per row per tile
constexpr int LDSROW = ROWB + 16;    // padded LDS row (bytes)
constexpr int TILE_BYTES = BM * LDSROW;
constexpr int GEMM_LDS = 2 * 2 * TILE_BYTES;   // A + B, double buffered

__device__ inline float bf16_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline uint16_t float_to_bf16(float f) {
  __bf16 x = (__bf16)f;
  return __builtin_bit_cast(uint16_t, x);
}

// Load one K tile (128 bytes per row) of a [rows x kbytes] K-contiguous matrix into
// registers: 1024 16-byte chunks per operand, 4 per thread; zero outside the matrix.
__device__ inline void load_tile(const uint8_t* __restrict__ M, int64_t rows, int64_t kbytes, int64_t r0, int64_t kb0,
                                 int tid, uint4 (&reg)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = tid + 256 * i;
    int r = c >> 3, ch = c & 7;
    int64_t gr = r0 + r, gk = kb0 + ch * 16;
    if (gr < rows && gk < kbytes) reg[i] = *(const uint4*)(M + gr * kbytes + gk);
    else reg[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ inline void store_tile(uint8_t* s, int tid, const uint4 (&reg)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = tid + 256 * i;
    int r = c >> 3, ch = c & 7;
    *(uint4*)(s + r * LDSROW + ch * 16) = reg[i];
  }
}

template <bool FP8>
__global__ void __launch_bounds__(256) gemm_nt_kernel(const uint8_t* __restrict__ X, const uint8_t* __restrict__ W,
                                                      const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                                                      int64_t T, int64_t N, int64_t K, float ax,
                                                      const float* __restrict__ aw) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t kbytes = FP8 ? K : 2 * K;
  const int64_t nkt = (kbytes + ROWB - 1) / ROWB;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  uint4 ra[4], rb[4];
  load_tile(X, T, kbytes, m0, 0, tid, ra);
  load_tile(W, N, kbytes, n0, 0, tid, rb);
  store_tile(lds, tid, ra);
  store_tile(lds + TILE_BYTES, tid, rb);
  __syncthreads();

  const int lr = lane & 31, lh = lane >> 5;
  for (int64_t kt = 0; kt < nkt; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nkt) {
      load_tile(X, T, kbytes, m0, (kt + 1) * ROWB, tid, ra);
      load_tile(W, N, kbytes, n0, (kt + 1) * ROWB, tid, rb);
    }
    const uint8_t* sA = lds + buf * 2 * TILE_BYTES;
    const uint8_t* sB = sA + TILE_BYTES;
    if (!FP8) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {       // 4 x K16 per 64-element tile
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          fa[t] = *(const bf16x8*)(sA + (wm * 64 + t * 32 + lr) * LDSROW + ks * 32 + lh * 16);
          fb[t] = *(const bf16x8*)(sB + (wn * 64 + t * 32 + lr) * LDSROW + ks * 32 + lh * 16);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {       // 2 x K64 per 128-byte tile
        i32x8 fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          fa[t] = *(const i32x8*)(sA + (wm * 64 + t * 32 + lr) * LDSROW + ks * 64 + lh * 32);
          fb[t] = *(const i32x8*)(sB + (wn * 64 + t * 32 + lr) * LDSROW + ks * 64 + lh * 32);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[a], fb[b], acc[a][b], 0, 0, 0, 0, 0, 0);
      }
    }
    if (kt + 1 < nkt) {
      uint8_t* dA = lds + (buf ^ 1) * 2 * TILE_BYTES;
      store_tile(dA, tid, ra);
      store_tile(dA + TILE_BYTES, tid, rb);
    }
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + lr;
      if (col >= N) continue;
      float bv = 0.f, sc = 1.f;
      if (FP8) sc = ax * aw[col];
      else if (bias) bv = bf16_to_float(bias[col]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < T) Y[row * N + col] = float_to_bf16(FP8 ? acc[a][b][r] * sc : acc[a][b][r] + bv);
      }
    }
}

template <bool FP8>
int launch_gemm(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t K, float ax,
                const float* aw, hipStream_t st) {
  if (!x || !w || !y || (FP8 && !aw)) return fail(EP_E_ARG, "null pointer");
  if (T < 1 || N < 1 || K < 1) return fail(EP_E_ARG, "GEMM sizes must be >= 1");
  const int64_t kb = FP8 ? K : 2 * K;
  if (kb % 16) return fail(EP_E_ARG, "K must be a multiple of 8 (BF16) or 16 (FP8)");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & 15)
    return fail(EP_E_ARG, "operands must be 16-byte aligned");
  auto kern = gemm_nt_kernel<FP8>;
  static std::once_flag once;
  std::call_once(once, [&] { (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS); });
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((T + BM - 1) / BM));
  hipLaunchKernelGGL(kern, grid, dim3(256), GEMM_LDS, st, (const uint8_t*)x, (const uint8_t*)w,
                     (const uint16_t*)bias, (uint16_t*)y, T, N, K, ax, aw);
  return hip_check(hipGetLastError(), "gemm launch");
}

}  // namespace
}  // namespace ep

using namespace ep;

extern "C" {

int ep_gemm_bf16_nt(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t K,
                    ep_stream stream) {
  set_error("");
  return launch_gemm<false>(x, w, bias, y, T, N, K, 1.f, nullptr, (hipStream_t)stream);
}

int ep_gemm_fp8_nt(const void* xq, const void* wq, float a_x, const float* aw, void* y, int64_t T, int64_t N,
                   int64_t K, ep_stream stream) {
  set_error("");
  return launch_gemm<true>(xq, wq, nullptr, y, T, N, K, a_x, aw, (hipStream_t)stream);
}

int ep_compressed_linear_forward(const ep_blob* w, const void* x, int64_t T, const void* bias, void* y, void* ws,
                                 size_t ws_bytes, ep_stream stream) {
  set_error("");
  if (!w || !x || !y || !ws) return fail(EP_E_ARG, "null pointer");
  const Blob& b = w->b;
  if (b.dtype != EP_BF16) return fail(EP_E_DTYPE, "compressed linear takes a BF16 blob");
  if (ws_bytes < ep_linear_workspace_bytes(w)) return fail(EP_E_WORKSPACE, "workspace too small");
  void* wd = (void*)(((uintptr_t)ws + 255) & ~uintptr_t(255));
  int rc = ep_decompress(w, wd, stream);
  if (rc) return rc;
  return launch_gemm<false>(x, wd, bias, y, T, b.R, b.C, 1.f, nullptr, (hipStream_t)stream);
}

}  // extern "C"
