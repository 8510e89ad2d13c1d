// MFMA GEMMs for the compressed linear layer on gfx950.
//
// [README] 快速开始: CompressedLinear.from_linear(...) returns a layer called as layer(x)
// that behaves like torch.nn.Linear, y = x W^T + b.  [ABS]: decoding cost grows with
// the weight count, so the method suits compute-heavy work (diffusion denoising,
// transformer prefill) where the GEMM dominates.  [NEWS] / [README] "FP8@5": FP8 W8A8
// weight codes compressed by EntroPack and an FP8 GEMM at inference.
//
// Both GEMMs are "NT": X [T x K] and W [N x K] are K-contiguous, Y = X W^T is [T x N]
// row-major BF16 with fp32 accumulation.  One kernel (below, 256 x 256 or 256 x 128
// tiles, LDS filled by direct-to-LDS loads, 128 bytes of K per row and stage) serves
// both element types: BF16 (the compressed linear layer and its uncompressed baseline)
// and FP8 E4M3 codes (y = acc * a_x * a_w[n]).
//   BF16: v_mfma_f32_32x32x16_bf16   (A/B: 8 bf16 per lane, lane -> row l%32,
//                                      k = 8 (l/32) .. +8)
//   FP8:  v_mfma_f32_32x32x64_f8f6f4 (A/B: 32 e4m3 per lane, k = 32 (l/32) .. +32)
//   D:    lane l holds column l%32, rows 8 (r/4) + 4 (l/32) + r%4 for r = 0..15.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "ep_internal.h"

namespace ep {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------- GEMM, 256 x BN tiles
// Workgroup tile 256 x BN, waves 2 along M x W/2 along N (BN = 128: 4 waves of 128 x 64;
// BN = 256: 8 waves of 128 x 64, two per SIMD), each wave 4 x 2 MFMA 32x32x16 blocks.
// K tiles of 128 bytes go from HBM straight into one of NST LDS stages
// (global_load_lds, 16 bytes per lane, lane l landing at base + 16 l), issued NST - 1
// tiles ahead; one barrier per K tile.  LDS rows are 128 bytes; their 16-byte
// chunks are XOR-swizzled by the row so that the eight lanes reading one fragment row
// group touch all 32 banks once.  Chunks outside the matrix load a zero line.  The MFMA
// takes the W fragment as its first operand, so each lane ends with four consecutive
// outputs of one row (one 8-byte store).
//   BN = 128: 3 stages (144 KB);  BN = 256: 2 stages (128 KB).  A stage holds 128 bytes of
//   K per row: 64 BF16 (four MFMA 32x32x16 steps) or 128 FP8 (two 32x32x64 steps, a lane's
//   32-byte operand read as two swizzled 16-byte chunks).
constexpr int GBM = 256;

__device__ inline float bf16_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline uint16_t float_to_bf16(float f) {
  __bf16 x = (__bf16)f;
  return __builtin_bit_cast(uint16_t, x);
}
__device__ __align__(16) uint4 g_zero_line[4];   // zero-initialised; the source of out-of-range chunks

#define EP_LDS3 __attribute__((address_space(3)))

// a per-wave value the compiler may keep in a scalar register
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// waves per workgroup by tile width
constexpr int gemm_waves(int BN) { return BN == 256 ? 8 : 4; }

// chunk position of logical chunk c in row r (CPR chunks per row)
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return CPR == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 1) & 3));
}

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// The epilogue's per-column terms for four consecutive output columns n .. n + 3: the BF16
// bias (added) or the FP8 scale a_x a_w[n] (multiplied; 0 past the matrix), read once for
// all the rows a lane stores, as one 8- or 16-byte load where the four columns lie inside
// the matrix and the vector is aligned.
template <bool FP8>
__device__ __forceinline__ void column_terms(const uint16_t* __restrict__ bias, const float* __restrict__ aw, float ax,
                                             int64_t n, int64_t N, bool vec, float* c) {
  if constexpr (FP8) {
    if (vec && n + 3 < N) {
      const float4 s = *(const float4*)(aw + n);
      c[0] = ax * s.x; c[1] = ax * s.y; c[2] = ax * s.z; c[3] = ax * s.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = n + e < N ? ax * aw[n + e] : 0.f;
    }
  } else {
    if (!bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = 0.f;
    } else if (vec && n + 3 < N) {
      const u32x2 b = *(const u32x2*)(bias + n);
      c[0] = __uint_as_float(b.x << 16); c[1] = __uint_as_float(b.x & 0xffff0000u);
      c[2] = __uint_as_float(b.y << 16); c[3] = __uint_as_float(b.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = n + e < N ? bf16_to_float(bias[n + e]) : 0.f;
    }
  }
}

// Stores a lane's four outputs of row m, columns n .. n + 3 (BF16, round to nearest even)
__device__ __forceinline__ void store4(uint16_t* __restrict__ Y, int64_t m, int64_t ldy, int64_t n, int64_t N, bool vec,
                                       const float* v) {
  uint16_t* yp = Y + m * ldy + n;
  if (vec && n + 3 < N) {
    u32x2 pk;
    pk.x = (uint32_t)float_to_bf16(v[0]) | ((uint32_t)float_to_bf16(v[1]) << 16);
    pk.y = (uint32_t)float_to_bf16(v[2]) | ((uint32_t)float_to_bf16(v[3]) << 16);
    *(u32x2*)yp = pk;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < N) yp[e] = float_to_bf16(v[e]);
  }
}

template <int BN, int NST, int RB, bool FP8>
__global__ void __launch_bounds__(64 * gemm_waves(BN), 1) gemm_tile_kernel(const uint8_t* __restrict__ X, const uint8_t* __restrict__ W,
                                                           const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                                                           int64_t T, int64_t N, int64_t ldy, int64_t K, int ntm, int ntn, int GM, float ax,
                                                           const float* __restrict__ aw) {
  constexpr int NW = gemm_waves(BN);
  constexpr int CPR = RB / 16, RPL = 64 / CPR;                // chunks per row, rows per load
  constexpr int NKS = RB / (FP8 ? 64 : 32);                   // MFMA K steps per stage
  constexpr bool kDoubleFrag = !(FP8 && BN == 256);           // fragments double-buffered
  const int64_t KB = FP8 ? K : 2 * K;                         // bytes of K per matrix row
  constexpr int A_BYTES = GBM * RB, B_BYTES = BN * RB, STAGE = A_BYTES + B_BYTES;
  constexpr int WN = BN / (NW / 2), NJ = WN / 32, MI = 4;     // waves: 2 along M x NW/2 along N
  constexpr int A_LD = GBM / RPL / NW, B_LD = BN / RPL / NW;  // load instructions per wave
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);   // uniform per wave
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  // tile of this workgroup: workgroups are dealt to the 8 XCDs in turn, so each XCD gets
  // a contiguous range of tiles; tiles are ordered in groups of 4 M-tiles x all N-tiles,
  // so the tiles resident on one XCD share X and W panels in its L2
  const int ntiles = ntm * ntn;
  int t = (int)blockIdx.x;
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  const int gsz = GM * ntn, g = t / gsz, rem = t % gsz;
  const int gm = ntm - g * GM < GM ? ntm - g * GM : GM;
  const int64_t m0 = (int64_t)(g * GM + rem % gm) * GBM, n0 = (int64_t)(rem / gm) * BN;
  const int64_t nkt = (KB + RB - 1) / RB;

  // this lane's part of each load instruction: row (within RPL) and the chunk it fetches.
  // Rows past the matrix read its last row (their outputs are never stored); the byte
  // offsets from the panel start are fixed, the panel base advances by one K tile.
  const int lrow = lane / CPR, lpos = lane % CPR;
  uint32_t offA[A_LD], offB[B_LD], kcA[A_LD], kcB[B_LD];   // byte offset, its K part
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = (wave * A_LD + i) * RPL + lrow;
    const int64_t gr = m0 + r < T ? m0 + r : T - 1;
    kcA[i] = (uint32_t)(swz<CPR>(r, lpos) * 16);
    offA[i] = (uint32_t)((gr - m0) * KB) + kcA[i];
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int r = (wave * B_LD + i) * RPL + lrow;
    const int64_t gr = n0 + r < N ? n0 + r : N - 1;
    kcB[i] = (uint32_t)(swz<CPR>(r, lpos) * 16);
    offB[i] = (uint32_t)((gr - n0) * KB) + kcB[i];
  }
  const char* xpan = (const char*)(X + m0 * KB);
  const char* wpan = (const char*)(W + n0 * KB);
  const char* pA[A_LD];
  const char* pB[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) pA[i] = xpan + offA[i];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) pB[i] = wpan + offB[i];
  const bool ktail = (KB % RB) != 0;
  const char* zero = (const char*)g_zero_line;
  auto issue = [&](int64_t kt, int st) {
    EP_LDS3 uint8_t* sbase = (EP_LDS3 uint8_t*)lds + st * STAGE;
    const int64_t kb = kt * RB;
    if (!ktail || kt + 1 < nkt) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(pA[i] + kb), (EP_LDS3 void*)(sbase + (wave * A_LD + i) * 1024), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < B_LD; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(pB[i] + kb), (EP_LDS3 void*)(sbase + A_BYTES + (wave * B_LD + i) * 1024), 16, 0, 0);
    } else {
      // last, partial K tile: chunks at or past K load the zero line
      const int64_t kleft = KB - kb;   // bytes of K left
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const bool in = (int64_t)kcA[i] < kleft;
        __builtin_amdgcn_global_load_lds((const void*)(in ? pA[i] + kb : zero), (EP_LDS3 void*)(sbase + (wave * A_LD + i) * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const bool in = (int64_t)kcB[i] < kleft;
        __builtin_amdgcn_global_load_lds((const void*)(in ? pB[i] + kb : zero), (EP_LDS3 void*)(sbase + A_BYTES + (wave * B_LD + i) * 1024), 16, 0, 0);
      }
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment addresses within a stage (the K16 step adds a swizzled chunk position)
  const int lr = lane & 31, lh = lane >> 5;
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type frag_t;
  // a lane's operand: BF16 chunk 2 ks + lh (8 elements); FP8 chunks 4 ks + 2 lh and the
  // next one (32 codes)
  auto frag_at = [&](const uint8_t* s, int r, int ks) -> frag_t {
    if constexpr (FP8) {
      const int c = 4 * ks + 2 * lh;
      const uint4 lo = *(const uint4*)(s + r * RB + (swz<CPR>(r, c) << 4));
      const uint4 hi = *(const uint4*)(s + r * RB + (swz<CPR>(r, c + 1) << 4));
      const i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      return v;
    } else {
      return *(const bf16x8*)(s + r * RB + (swz<CPR>(r, 2 * ks + lh) << 4));
    }
  };
  auto frag_load = [&](const uint8_t* sA, const uint8_t* sB, int ks, frag_t* fa, frag_t* fb) {
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = frag_at(sA, wm * 128 + 32 * i + lr, ks);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[j] = frag_at(sB, wn * WN + 32 * j + lr, ks);
  };

  // prologue: tiles 0 .. NST-2 in flight
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nkt) issue(s, s);
  constexpr int LD = A_LD + B_LD;
  auto tile = [&](int64_t kt, int st) {
    // this wave's loads of tile kt are done once at most the later tiles' loads remain
    const int64_t later = (nkt - 1 - kt) < (NST - 2) ? (nkt - 1 - kt) : (NST - 2);
    if (NST >= 5 && later >= 3) __builtin_amdgcn_s_waitcnt((3 * LD & 15) | (((3 * LD) >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (NST >= 4 && later >= 2) __builtin_amdgcn_s_waitcnt((2 * LD & 15) | (((2 * LD) >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (later >= 1) __builtin_amdgcn_s_waitcnt((LD & 15) | ((LD >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    // every wave's part of tile kt is in LDS and stage (kt - 1) % NST is free once all
    // waves pass; a plain s_barrier (no fence: the loads of later tiles stay in flight)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const uint8_t* sA = lds + st * STAGE;
    const uint8_t* sB = sA + A_BYTES;
    if constexpr (!kDoubleFrag) {
      // one set of fragments at a time (the wider FP8 operands of the 256-wide tile
      // would not fit twice beside the accumulators).  The next tile's loads go out after
      // this tile's last fragment reads: an LDS read issued while a direct-to-LDS load is
      // in flight makes the compiler wait for that load first, which would expose its
      // whole latency at every tile
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        frag_t fa[MI], fb[NJ];
        frag_load(sA, sB, ks, fa, fb);
        if (ks == NKS - 1 && kt + NST - 1 < nkt) issue(kt + NST - 1, (st + NST - 1) % NST);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, 0, 0, 0);
      }
      return;
    }
    // When the next tile's loads go out: an LDS read issued while a direct-to-LDS load is
    // in flight waits for all earlier LDS reads, so issuing them after the fragment
    // requests of this tile's first K steps keeps those steps' read-ahead, at the cost of
    // less time for the loads to land.  Measured at 4096 x 14336 x 4096 (same process,
    // interleaved): the two-stage BF16 tile after step 2's requests (-2.7 %), FP8 tiles
    // at the end (-4 %); the three-stage 128-wide BF16 tile right after the barrier.
    constexpr int kIssueAt = FP8 ? NKS - 1 : (NST == 2 ? 1 : -1);
    if (kIssueAt < 0 && kt + NST - 1 < nkt) issue(kt + NST - 1, (st + NST - 1) % NST);
    frag_t fa[2][MI], fb[2][NJ];
    frag_load(sA, sB, 0, fa[0], fb[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      // the next step's fragments are requested before this step's MFMAs
      if (ks + 1 < NKS) frag_load(sA, sB, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      if (ks == kIssueAt && kt + NST - 1 < nkt) issue(kt + NST - 1, (st + NST - 1) % NST);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if constexpr (FP8)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0,
                                                                      0, 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int64_t kt = 0; kt < nkt; kt += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s)
      if (kt + s < nkt) tile(kt + s, s);
  }

  // epilogue: lane holds row m = m0 + wm 128 + 32 i + lr and columns
  // n = n0 + wn WN + 32 j + 8 (r / 4) + 4 lh + r % 4
  const bool vec = (N % 4) == 0 && (ldy % 4) == 0;
  const bool cvec = vec && ((reinterpret_cast<uintptr_t>(FP8 ? (const void*)aw : (const void*)bias) & (FP8 ? 15 : 7)) == 0);
  float c[NJ][4][4];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      column_terms<FP8>(bias, aw, ax, n0 + wn * WN + 32 * j + 8 * rq + 4 * lh, N, cvec, c[j][rq]);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t m = m0 + wm * 128 + 32 * i + lr;
    if (m >= T) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = FP8 ? acc[i][j][4 * rq + e] * c[j][rq][e] : acc[i][j][4 * rq + e] + c[j][rq][e];
        store4(Y, m, ldy, n0 + wn * WN + 32 * j + 8 * rq + 4 * lh, N, vec, v);
      }
  }
}

// ------------------------------------------- BF16 GEMM, 256 x 256 tiles of four waves
// Each wave owns 128 x 128 outputs (8 x 8 MFMA 16x16x32 blocks: 256 accumulators per
// lane, held in AGPRs), one wave per SIMD, so a 32-element K step's sixteen fragments
// feed 64 MFMAs (LDS reads per MFMA: two thirds of the 8-wave tile's).  Operands go HBM
// -> registers -> LDS through buffer loads (an SGPR descriptor per panel, 32-bit lane
// offsets): tile kt + 2's loads are issued while tile kt is multiplied, into the
// registers that held tile kt + 1, which that same tile writes to the LDS stage tile
// kt - 1 used.  Each K step's share of those stores and loads sits between its MFMAs,
// and since every LDS access is an ordinary read or write the compiler waits for
// exactly the fragments an MFMA needs (a direct-to-LDS load in flight would make it wait
// for all).  LDS: two stages of (256 + 256) rows x 128 bytes (128 KB), the 16-byte chunks
// of a row swizzled as in gemm_tile_kernel (conflict-free for 16-row fragments too).
// Whole K tiles only (K % 64 == 0).
// Measured against gemm_tile_kernel (same process, bit-identical outputs):
// 4096 x 14336 x 4096 0.395 vs 0.423 ms, 4096^3 0.113 vs 0.124 ms, 4096 x 4096 x 14336
// 0.347 vs 0.388 ms.  Also measured and not kept: 32x32x16 blocks (0.412 ms at the first
// shape), a second register set for a two-tile load lead (1-3 %), direct-to-LDS loads
// into per-stage LDS arrays (no faster than the register path), and the same tile for
// FP8 codes with 16x16x128 blocks (bit-identical to gemm_tile_kernel but 4-15 % slower:
// a K tile is a single MFMA step, so its fragments cannot be requested a step ahead).
__global__ void __launch_bounds__(256, 1) gemm_w4_kernel(const uint8_t* __restrict__ X, const uint8_t* __restrict__ W,
                                                      const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                                                      int64_t T, int64_t N, int64_t ldy, int64_t K, int ntm, int ntn,
                                                      int GM) {
  constexpr int RB = 128, CPR = 8, RPL = 8, NL = 8;   // bytes of K per row and stage, chunks per row,
                                                      // rows per load, loads per wave and operand
  constexpr int OPB = GBM * RB, STAGE = 2 * OPB;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile of this workgroup (the same XCD-aware order as gemm_tile_kernel)
  const int ntiles = ntm * ntn;
  int t = (int)blockIdx.x;
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  const int gsz = GM * ntn, g = t / gsz, rem = t % gsz;
  const int gm = ntm - g * GM < GM ? ntm - g * GM : GM;
  const int64_t m0 = (int64_t)(g * GM + rem % gm) * GBM, n0 = (int64_t)(rem / gm) * GBM;
  const int64_t KB = 2 * K, nkt = KB / RB;

  // load i of this wave: LDS row (wave NL + i) RPL + lane / CPR, position lane % CPR,
  // holding the row's logical chunk swz(row, position); rows past the matrix read its
  // last row (their outputs are never stored)
  const int lrow = lane / CPR, lpos = lane % CPR;
  uint32_t offA[NL], offB[NL], kc[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = (wave * NL + i) * RPL + lrow;
    kc[i] = (uint32_t)(swz<CPR>(r, lpos) * 16);
    const int64_t ga = m0 + r < T ? m0 + r : T - 1, gb = n0 + r < N ? n0 + r : N - 1;
    offA[i] = (uint32_t)((ga - m0) * KB) + kc[i];
    offB[i] = (uint32_t)((gb - n0) * KB) + kc[i];
  }
  // buffer descriptors of the two 256-row panels (32-bit offsets from an SGPR base)
  const int64_t rows_a = T - m0 < GBM ? T - m0 : GBM, rows_b = N - n0 < GBM ? N - n0 : GBM;
  auto rsrc = [](const uint8_t* p, int64_t bytes) {
    // every lane holds the same values: make that visible, so the descriptor sits in SGPRs
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t xr = rsrc(X + m0 * KB, rows_a * KB);
  const __amdgpu_buffer_rsrc_t wr = rsrc(W + n0 * KB, rows_b * KB);
  u32x4 ra[NL], rb[NL];
  // whole K tiles only (the launcher sends K % 64 != 0 to gemm_tile_kernel); half h:
  // loads 4h .. 4h + 3 of each operand
  auto gload = [&](int64_t kt, int h) {
    const int kb = (int)(kt * RB);
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) ra[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)offA[i], kb, 0);
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) rb[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)offB[i], kb, 0);
  };
  auto swrite = [&](int st, int h) {
    uint8_t* s0 = lds + st * STAGE + (wave * NL) * 1024 + lane * 16;
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) *(u32x4*)(s0 + i * 1024) = ra[i];
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) *(u32x4*)(s0 + OPB + i * 1024) = rb[i];
  };
  // every wave's stores to LDS are done, then all waves meet (a plain s_barrier: the
  // register loads of the next tile stay in flight)
  auto lds_barrier = [&] {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  typedef __attribute__((ext_vector_type(4))) float f32x4;
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  // fragment of MFMA block i (rows 16 i + lane % 16 of this wave's 128) at K step ks
  // (32 elements): logical chunk 4 ks + lane / 16 of the row; (row >> 1) & 7 is
  // (lane % 16 >> 1) & 7
  const int lr = lane & 15, lq = lane >> 4, sw = (lr >> 1) & 7;
  const uint32_t rowA = (uint32_t)(wm * 128 + lr) * RB, rowB = OPB + (uint32_t)(wn * 128 + lr) * RB;
  uint32_t cofs[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) cofs[ks] = (uint32_t)(((4 * ks + lq) ^ sw) << 4);
  auto frags = [&](int st, int ks, bf16x8* fa, bf16x8* fb) {
    const uint8_t* s = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i] = *(const bf16x8*)(s + rowA + i * 16 * RB + cofs[ks]);
#pragma unroll
    for (int j = 0; j < 8; ++j) fb[j] = *(const bf16x8*)(s + rowB + j * 16 * RB + cofs[ks]);
  };
  // tile kt sits in stage st and tile kt + 1 in the registers.  K step ks (of two):
  // step 1's fragments requested during step 0, half of tile kt + 1 moved from the
  // registers to the other stage and those registers reloaded with tile kt + 2 (past the
  // end: the last tile again, never used), spread between the step's 64 MFMAs
  auto tile = [&](int64_t kt, int st) {
    bf16x8 fa[2][8], fb[2][8];
    frags(st, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t knext = kt + 2 < nkt ? kt + 2 : nkt - 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 0) frags(st, 1, fa[1], fb[1]);
      swrite(st ^ 1, ks);
      gload(knext, ks);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
      if (ks == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);     // LDS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
      }
      if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, 56, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
  };

  // tile 0 to stage 0, tile 1 in the registers
#pragma unroll
  for (int h = 0; h < 2; ++h) gload(0, h);
#pragma unroll
  for (int h = 0; h < 2; ++h) swrite(0, h);
#pragma unroll
  for (int h = 0; h < 2; ++h) gload(nkt > 1 ? 1 : 0, h);
  lds_barrier();
  int64_t kt = 0;
  for (; kt + 2 <= nkt; kt += 2) {
    tile(kt, 0);
    tile(kt + 1, 1);
  }
  if (kt < nkt) tile(kt, 0);

  // epilogue: lane holds row m = m0 + wm 128 + 16 i + lane % 16 and columns
  // n = n0 + wn 128 + 16 j + 4 (lane / 16) + r
  const bool vec = (N % 4) == 0 && (ldy % 4) == 0;
  const bool cvec = vec && (reinterpret_cast<uintptr_t>(bias) & 7) == 0;
  float c[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) column_terms<false>(bias, nullptr, 1.f, n0 + wn * 128 + 16 * j + 4 * lq, N, cvec, c[j]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + wm * 128 + 16 * i + lr;
    if (m >= T) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e] + c[j][e];
      store4(Y, m, ldy, n0 + wn * 128 + 16 * j + 4 * lq, N, vec, v);
    }
  }
}

int launch_w4(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t ldy, int64_t K,
              hipStream_t st) {
  constexpr int lds = 2 * 2 * GBM * 128;
  static std::once_flag once;
  std::call_once(once, [&] {
    (void)hipFuncSetAttribute((const void*)gemm_w4_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  const int ntm = (int)((T + GBM - 1) / GBM), ntn = (int)((N + GBM - 1) / GBM);
  hipLaunchKernelGGL(gemm_w4_kernel, dim3((unsigned)(ntm * ntn)), dim3(256), lds, st, (const uint8_t*)x,
                     (const uint8_t*)w, (const uint16_t*)bias, (uint16_t*)y, T, N, ldy, K, ntm, ntn, 4);
  return hip_check(hipGetLastError(), "gemm launch");
}

template <int BN, int NST, int RB, bool FP8>
int launch_tile(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t ldy, int64_t K,
                float ax, const float* aw, hipStream_t st) {
  constexpr int lds = NST * (GBM + BN) * RB;
  auto kern = gemm_tile_kernel<BN, NST, RB, FP8>;
  static std::once_flag once;
  std::call_once(once, [&] { (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds); });
  const int ntm = (int)((T + GBM - 1) / GBM), ntn = (int)((N + BN - 1) / BN);
  const int gm = 4;   // tile groups of 4 M-tiles (measured: 2, 8 or all M-tiles are no faster)
  hipLaunchKernelGGL(kern, dim3((unsigned)(ntm * ntn)), dim3(64 * gemm_waves(BN)), lds, st, (const uint8_t*)x,
                     (const uint8_t*)w, (const uint16_t*)bias, (uint16_t*)y, T, N, ldy, K, ntm, ntn, gm, ax, aw);
  return hip_check(hipGetLastError(), "gemm launch");
}

// BN = 256 unless 128-wide tiles fill the CUs' rounds much better (a 256 x 256 tile does
// about 1.25x the work per cycle of a 256 x 128 one).
int gemm_cu_count() {
  static int v = -1;
  if (v < 0) {
    int dev = 0, x = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || x <= 0) x = 256;
    v = x;
  }
  return v;
}

// Whether launch_gemm takes the 128-wide tiles for T x N (they fill the CUs' rounds much
// better than 256-wide ones)
bool gemm_narrow(int64_t T, int64_t N) {
  const int64_t ntm = (T + GBM - 1) / GBM;
  auto eff = [&](int64_t bn) {
    const int64_t tiles = ntm * ((N + bn - 1) / bn);
    const int64_t rounds = (tiles + 255) / 256;
    return (double)(T * N) / (double)(rounds * 256 * GBM * bn);
  };
  bool narrow = eff(128) > 1.25 * eff(256);
  if (const char* e = std::getenv("EP_GEMM_BN")) narrow = std::atoi(e) == 128;
  return narrow;
}

// Workgroups (one per CU) of the BF16 GEMM for T x N when it takes one launch
int64_t gemm_tiles(int64_t T, int64_t N) {
  const int64_t ntm = (T + GBM - 1) / GBM;
  return gemm_narrow(T, N) ? ntm * ((N + 127) / 128) : ntm * ((N + 255) / 256);
}

// The four-wave BF16 kernel takes whole 64-element K tiles and 32-bit panel offsets;
// EP_GEMM_W4=0 selects gemm_tile_kernel instead (for comparisons)
bool use_w4(int64_t K) {
  const char* e = std::getenv("EP_GEMM_W4");
  return K % 64 == 0 && 2 * K * GBM < (int64_t)INT32_MAX && !(e && std::atoi(e) == 0);
}

template <bool FP8>
int launch_gemm(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t K, float ax,
                const float* aw, hipStream_t st) {
  if (!x || !w || !y || (FP8 && !aw)) return fail(EP_E_ARG, "null pointer");
  if (T < 1 || N < 1 || K < 1) return fail(EP_E_ARG, "GEMM sizes must be >= 1");
  if ((FP8 ? K : 2 * K) % 16) return fail(EP_E_ARG, "K must be a multiple of 8 (BF16) or 16 (FP8)");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & 15)
    return fail(EP_E_ARG, "operands must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(y) & 7) && N % 4 == 0) return fail(EP_E_ARG, "output must be 8-byte aligned");
  // pageable host memory would fault the kernel: refuse it before any launch
  int rc;
  if ((rc = check_gpu_pointer(x, "activations")) || (rc = check_gpu_pointer(w, "weights")) ||
      (rc = check_gpu_pointer(y, "output")) || (bias && (rc = check_gpu_pointer(bias, "bias"))) ||
      (aw && (rc = check_gpu_pointer(aw, "weight scales"))))
    return rc;
  const int64_t ntm = (T + GBM - 1) / GBM;
  if (gemm_narrow(T, N)) return launch_tile<128, 3, 128, FP8>(x, w, bias, y, T, N, N, K, ax, aw, st);
  // When the 256-wide tiles leave the last round of the CUs partly idle, the columns of
  // the whole rounds take 256-wide tiles and the rest 128-wide ones (a second launch of
  // about one round at roughly 0.6 of a 256-wide tile's time), e.g. 4096 x 14336: 768 +
  // 256 tiles in 3.6 round-times instead of 896 in 4.
  const int64_t cus = gemm_cu_count();
  const int64_t tiles = ntm * ((N + 255) / 256);
  const int64_t n1 = (tiles / cus) * cus / ntm;   // 256-wide column tiles of the whole rounds
  if (tiles % cus != 0 && n1 >= 1 && n1 * 256 < N) {
    const int64_t rem = N - n1 * 256, tiles2 = ntm * ((rem + 127) / 128);
    const double split = (double)((ntm * n1 + cus - 1) / cus) + 0.625 * (double)((tiles2 + cus - 1) / cus);
    if (split < (double)((tiles + cus - 1) / cus) - 0.2) {
      const int64_t c0 = n1 * 256, kb = FP8 ? K : 2 * K;
      rc = (!FP8 && use_w4(K)) ? launch_w4(x, w, bias, y, T, c0, N, K, st)
                              : launch_tile<256, 2, 128, FP8>(x, w, bias, y, T, c0, N, K, ax, aw, st);
      if (rc) return rc;
      return launch_tile<128, 3, 128, FP8>(x, (const uint8_t*)w + c0 * kb, bias ? (const uint16_t*)bias + c0 : nullptr,
                                           (uint16_t*)y + c0, T, rem, N, K, ax, aw ? aw + c0 : nullptr, st);
    }
  }
  if (!FP8 && use_w4(K)) return launch_w4(x, w, bias, y, T, N, N, K, st);
  return launch_tile<256, 2, 128, FP8>(x, w, bias, y, T, N, N, K, ax, aw, st);
}

int launch_bf16(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t K,
                hipStream_t st) {
  return launch_gemm<false>(x, w, bias, y, T, N, K, 1.f, nullptr, st);
}



}  // namespace
}  // namespace ep

using namespace ep;

extern "C" {

int ep_gemm_bf16_nt(const void* x, const void* w, const void* bias, void* y, int64_t T, int64_t N, int64_t K,
                    ep_stream stream) {
  set_error("");
  return launch_bf16(x, w, bias, y, T, N, K, (hipStream_t)stream);
}

int ep_gemm_fp8_nt(const void* xq, const void* wq, float a_x, const float* aw, void* y, int64_t T, int64_t N,
                   int64_t K, ep_stream stream) {
  set_error("");
  return launch_gemm<true>(xq, wq, nullptr, y, T, N, K, a_x, aw, (hipStream_t)stream);
}

// (5-8 rows take the fused prefill product where it applies: 63 us against 67 us for the
// eight-row product kernel on a 14336 x 4096 layer)
static bool use_matvec(const ep_blob* w, int64_t T) {
  return matvec_supported(w->b, T) && matvec_workspace_bytes(w->b, T) <= ep_linear_workspace_bytes(w) &&
         !(T > 4 && prefill_supported(w->b, T));
}
// up to 256 activation rows (4096 or 8192 columns, S = 8): the fused prefill product, which
// decodes every K slab of W into the MFMA product's LDS operand (1.1-1.6x faster than
// decode then GEMM on a 14336 x 4096 layer)
static bool use_prefill(const ep_blob* w, int64_t T) { return !use_matvec(w, T) && prefill_supported(w->b, T); }

int ep_compressed_linear_forward(const ep_blob* w, const void* x, int64_t T, const void* bias, void* y, void* ws,
                                 size_t ws_bytes, ep_stream stream) {
  set_error("");
  if (!w || !x || !y || !ws) return fail(EP_E_ARG, "null pointer");
  const Blob& b = w->b;
  if (b.kind != kKindLossy || b.dtype != EP_BF16) return fail(EP_E_DTYPE, "compressed linear takes a lossy BF16 blob");
  if (ws_bytes < ep_linear_workspace_bytes(w)) return fail(EP_E_WORKSPACE, "workspace too small");
  int rc;
  if ((rc = check_gpu_pointer(x, "activations")) || (rc = check_gpu_pointer(y, "output")) ||
      (rc = check_gpu_pointer(ws, "workspace")) || (bias && (rc = check_gpu_pointer(bias, "bias"))))
    return rc;
  // a few activation rows: the product runs inside the decode kernel (no BF16 weights
  // written and read back), when its partial sums fit the same workspace
  if (use_matvec(w, T)) return matvec_forward(b, x, T, bias, y, ws, ws_bytes, stream);
  if (use_prefill(w, T)) return prefill_launch(b, x, T, bias, y, stream);
  void* wd = (void*)(((uintptr_t)ws + 255) & ~uintptr_t(255));
  rc = decompress_for_gemm(b, wd, stream);
  if (rc) return rc;
  return launch_bf16(x, wd, bias, y, T, b.R, b.C, (hipStream_t)stream);
}

size_t ep_matvec_workspace_bytes(const ep_blob* w, int64_t T) {
  if (!w || !matvec_supported(w->b, T)) return 0;
  return matvec_workspace_bytes(w->b, T);
}

int ep_compressed_matvec(const ep_blob* w, const void* x, int64_t T, const void* bias, void* y, void* ws,
                         size_t ws_bytes, ep_stream stream) {
  set_error("");
  if (!w || !x || !y || !ws) return fail(EP_E_ARG, "null pointer");
  return matvec_forward(w->b, x, T, bias, y, ws, ws_bytes, stream);
}

size_t ep_matvec_batch_workspace_bytes(const ep_blob* const* w, int n, int64_t T) {
  if (!w || n < 1) return 0;
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (!w[i] || !matvec_supported(w[i]->b, T)) return 0;
    total += (matvec_workspace_bytes(w[i]->b, T) - 256 + 255) & ~size_t(255);
  }
  return total + 256;
}

int ep_compressed_matvec_batch(const ep_blob* const* w, int n, const void* x, int64_t T, const void* const* bias,
                               void* const* y, void* ws, size_t ws_bytes, ep_stream stream) {
  set_error("");
  if (!w || !x || !y || !ws || n < 1) return fail(EP_E_ARG, "null pointer or empty batch");
  for (int i = 0; i < n; ++i)
    if (!w[i] || !y[i]) return fail(EP_E_ARG, "null blob or output");
  const size_t need = ep_matvec_batch_workspace_bytes(w, n, T);
  if (need == 0)
    return fail(EP_E_ARG, "the fused product takes lossy BF16 blobs, 1..8 activation rows, C % 8 == 0 and at least S groups per row");
  if (ws_bytes < need) return fail(EP_E_WORKSPACE, "workspace too small");
  std::vector<const Blob*> bs(n);
  std::vector<float*> part(n);
  uintptr_t p = ((uintptr_t)ws + 255) & ~uintptr_t(255);
  for (int i = 0; i < n; ++i) {
    bs[i] = &w[i]->b;
    part[i] = (float*)p;
    p += (matvec_workspace_bytes(w[i]->b, T) - 256 + 255) & ~size_t(255);
  }
  return matvec_batch_launch(bs.data(), n, x, T, bias, y, part.data(), stream);
}

size_t ep_linear_seq_workspace_bytes(const ep_blob* const* w, int n) {
  if (!w || n < 1) return 0;
  size_t mx = 0;
  for (int i = 0; i < n; ++i) {
    if (!w[i]) return 0;
    mx = std::max(mx, (size_t)w[i]->b.R * (size_t)w[i]->b.C * 2);
  }
  return 2 * ((mx + 255) & ~size_t(255)) + 256;
}

// Layers 0..n-1, each decode then GEMM.  The decode of layer i+1 runs on `side`, beside
// the GEMM of layer i, only when that GEMM's tiles leave CUs idle for its whole run
// (fewer tiles than CUs), and then on at most as many workgroups as there are idle CUs:
// a decode workgroup holds 56 KB of tables plus its chains' rings and a GEMM workgroup
// 128-144 KB of LDS, so the two never share a CU, and when the GEMM fills every CU a
// side-stream decode only takes CUs away from it (measured: eight 4096-token layers 7 %
// slower than in order).  Otherwise the decode runs on `main` right before its GEMM.  Two weight buffers alternate; a side-stream decode
// into a buffer waits for the GEMM that last read it, a GEMM for its side-stream
// decode.  The side stream starts after everything already queued on main.
int ep_compressed_linear_seq_forward(const ep_blob* const* w, int n, const void* const* x, int64_t T,
                                     const void* const* bias, void* const* y, void* ws, size_t ws_bytes,
                                     ep_stream main_s, ep_stream side_s) {
  set_error("");
  if (!w || !x || !y || !ws || n < 1) return fail(EP_E_ARG, "null pointer or empty sequence");
  int rc = EP_OK;
  for (int i = 0; i < n; ++i) {
    if (!w[i] || !x[i] || !y[i]) return fail(EP_E_ARG, "null blob, input or output");
    if (w[i]->b.kind != kKindLossy || w[i]->b.dtype != EP_BF16)
      return fail(EP_E_DTYPE, "compressed linear takes lossy BF16 blobs");
    if ((rc = check_gpu_pointer(x[i], "activations")) || (rc = check_gpu_pointer(y[i], "output")) ||
        (bias && bias[i] && (rc = check_gpu_pointer(bias[i], "bias"))))
      return rc;
  }
  const size_t need = ep_linear_seq_workspace_bytes(w, n);
  if (ws_bytes < need) return fail(EP_E_WORKSPACE, "workspace too small");
  if ((rc = check_gpu_pointer(ws, "workspace"))) return rc;
  const size_t half = (need - 256) / 2;
  uint8_t* base = (uint8_t*)(((uintptr_t)ws + 255) & ~uintptr_t(255));
  void* buf[2] = {base, base + half};
  hipStream_t ms = (hipStream_t)main_s, ss = (hipStream_t)side_s;
  // layers with few activation rows take the fused product (as the one-layer entry does),
  // with their buffer as its partial-sum space, and layers the fused prefill product
  // takes need no buffer: neither needs a decode
  std::vector<char> mv(n), pf(n), on_side(n, 0);
  for (int i = 0; i < n; ++i) {
    mv[i] = use_matvec(w[i], T);
    pf[i] = use_prefill(w[i], T);
  }
  const int64_t cus = gemm_cu_count();
  bool any_side = false;
  std::vector<int64_t> free_cus(n, 0);
  for (int i = 1; i < n; ++i) {
    const int64_t tiles = gemm_tiles(T, w[i - 1]->b.R);
    on_side[i] = !mv[i] && !pf[i] && !mv[i - 1] && !pf[i - 1] && tiles < cus;
    free_cus[i] = cus - tiles;
    any_side = any_side || on_side[i];
  }
  hipEvent_t ev_start = nullptr, ev_dec[2] = {nullptr, nullptr}, ev_used[2] = {nullptr, nullptr};
  auto mk = [&](hipEvent_t* e) {
    if (!rc) rc = hip_check(hipEventCreateWithFlags(e, hipEventDisableTiming), "event create");
  };
  if (any_side) {
    mk(&ev_start);
    for (int k = 0; k < 2; ++k) {
      mk(&ev_dec[k]);
      mk(&ev_used[k]);
    }
    if (!rc) rc = hip_check(hipEventRecord(ev_start, ms), "event record");
    if (!rc) rc = hip_check(hipStreamWaitEvent(ss, ev_start, 0), "stream wait");
  }
  auto decode_side = [&](int i) {
    const int k = i & 1;
    if (i >= 2 && !rc) rc = hip_check(hipStreamWaitEvent(ss, ev_used[k], 0), "stream wait");
    // on the CUs the GEMM leaves free (a decode workgroup queued behind a GEMM workgroup
    // would only start when that GEMM ends)
    if (!rc) rc = decompress_beside(w[i]->b, buf[k], side_s, free_cus[i]);
    if (!rc) rc = hip_check(hipEventRecord(ev_dec[k], ss), "event record");
  };
  for (int i = 0; i < n && !rc; ++i) {
    if (i + 1 < n && on_side[i + 1]) decode_side(i + 1);
    const int k = i & 1;
    if (mv[i]) {
      if (!rc) rc = matvec_launch(w[i]->b, x[i], T, bias ? bias[i] : nullptr, y[i], (float*)buf[k], ms);
    } else if (pf[i]) {
      if (!rc) rc = prefill_launch(w[i]->b, x[i], T, bias ? bias[i] : nullptr, y[i], ms);
    } else {
      if (on_side[i]) {
        if (!rc) rc = hip_check(hipStreamWaitEvent(ms, ev_dec[k], 0), "stream wait");
      } else if (!rc) {
        rc = decompress_for_gemm(w[i]->b, buf[k], main_s);
      }
      if (!rc) rc = launch_bf16(x[i], buf[k], bias ? bias[i] : nullptr, y[i], T, w[i]->b.R, w[i]->b.C, ms);
    }
    if (any_side && !rc) rc = hip_check(hipEventRecord(ev_used[k], ms), "event record");
  }
  // events may be destroyed while still pending; the runtime releases them when done
  if (ev_start) (void)hipEventDestroy(ev_start);
  for (int k = 0; k < 2; ++k) {
    if (ev_dec[k]) (void)hipEventDestroy(ev_dec[k]);
    if (ev_used[k]) (void)hipEventDestroy(ev_used[k]);
  }
  return rc;
}

}  // extern "C"

