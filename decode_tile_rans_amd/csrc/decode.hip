// Fused tile-rANS decode for gfx950 (MI355X).
//
// [SUM]: symbol decode, algebraic inverse-lattice reconstruction and per-row rescale
// run fused on the GPU, with no intermediate symbol tensor and no reconstruction
// codebook.  [ABS]: tiles are independently decodable; containers BF16/FP16/FP8/INT8.
//
// Work mapping (MI355X-first, not the pages' H20 design):
//   * one wavefront = one block of 64 rANS chains, one chain per lane (64/S tiles);
//     the wave's prefix sum over its 32 region lengths gives every lane its stream
//     start, so only one u32 checkpoint per 64 chains is stored;
//   * a workgroup of W waves stages the 7 decode tables (7 x 2048 packed u32 = 56 KB)
//     into LDS once; each wave copies its block's contiguous stream span into LDS
//     with coalesced 16-byte loads; lanes then read their own words from LDS;
//   * per coordinate: one LDS table read, x = f (x >> 11) + bias (24-bit mad), a
//     16-bit renormalisation from a prefetched word, the doubled coordinate taken
//     straight from the table entry (escapes: bypass bits, rare), h_r * u in fp32,
//     container cast, one 16-byte store per 8-coordinate group (BF16);
//   * nothing but the final weights is written to HBM.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ep_internal.h"

namespace ep {

int hip_check(int err, const char* what) {
  if (err != hipSuccess) return fail(EP_E_DEVICE, std::string(what) + ": " + hipGetErrorString((hipError_t)err));
  return EP_OK;
}

namespace {

enum OutKind { OUT_BF16 = 0, OUT_BF16_SAT = 1, OUT_FP16 = 2, OUT_FP32 = 3, OUT_FP8 = 4, OUT_INT8 = 5, OUT_COORDS = 6 };

constexpr int kTabWords = kNumCtx * kM;          // 14336 u32
constexpr int kTabBytes = kTabWords * 4;         // 57344 B
constexpr uint32_t kEscBit = 1u << 22;

struct DecJob {
  const uint16_t* stream;
  const uint32_t* states;
  const uint16_t* rlen;
  const uint32_t* ckpt;
  const float* hr;
  const uint32_t* tab;
  uint32_t* err;
  void* out;
  int64_t n_groups, G, C, n_chains, n_regions, n_blocks;
  int64_t chain_lo, chain_hi;
  int64_t block_lo;          // first block decoded by workgroup 0 of this job
  int64_t wg_begin;          // batch: first workgroup of this job
  uint32_t n_words;
  int log2S, k, c8;
};

// ---------------------------------------------------------------- container stores
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ inline uint32_t pack_f16x2(float a, float b) {
  a = fminf(fmaxf(a, -65504.f), 65504.f);
  b = fminf(fmaxf(b, -65504.f), 65504.f);
  __half x = __float2half_rn(a), y = __float2half_rn(b);
  return (uint32_t)__half_as_ushort(x) | ((uint32_t)__half_as_ushort(y) << 16);
}

// OCP E4M3FN, round to nearest even, saturating at 448.
__device__ inline uint32_t f32_to_e4m3fn(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.f);
  uint32_t code;
  if (a < 0.015625f) {                 // below 2^-6: units of 2^-9, exact scaling
    code = (uint32_t)rintf(a * 512.f);
  } else {
    uint32_t b = __float_as_uint(a);
    int e = (int)(b >> 23) - 127;
    uint32_t man = b & 0x7FFFFFu;
    uint32_t q = man >> 20, rem = man & 0xFFFFFu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    if (q == 8u) {
      q = 0;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | q;
  }
  return code | sign;
}

__device__ inline uint32_t f32_to_i8(float v) {
  float r = fminf(fmaxf(rintf(v), -128.f), 127.f);
  return (uint32_t)((int32_t)r) & 0xFFu;
}

template <int OUT>
__device__ inline void store_group(void* out, int64_t base, const int32_t* u, float h, bool full, int64_t nvalid) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = h * (float)u[i];
  if (OUT == OUT_BF16_SAT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i], -3.38953139e38f), 3.38953139e38f);
  }
  if (OUT == OUT_BF16 || OUT == OUT_BF16_SAT || OUT == OUT_FP16) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = (OUT == OUT_FP16) ? pack_f16x2(v[2 * i], v[2 * i + 1]) : pack_bf16x2(v[2 * i], v[2 * i + 1]);
    uint16_t* o = (uint16_t*)out + base;
    if (full) {
      *(uint4*)o = make_uint4(p[0], p[1], p[2], p[3]);
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = (uint16_t)(p[i >> 1] >> ((i & 1) * 16));
    }
  } else if (OUT == OUT_FP32) {
    float* o = (float*)out + base;
    if (full) {
      *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = v[i];
    }
  } else if (OUT == OUT_FP8 || OUT == OUT_INT8) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t a = (OUT == OUT_FP8) ? f32_to_e4m3fn(v[i]) : f32_to_i8(v[i]);
      uint32_t b = (OUT == OUT_FP8) ? f32_to_e4m3fn(v[i + 4]) : f32_to_i8(v[i + 4]);
      lo |= a << (8 * i);
      hi |= b << (8 * i);
    }
    uint8_t* o = (uint8_t*)out + base;
    if (full) {
      *(uint2*)o = make_uint2(lo, hi);
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
    }
  } else {  // OUT_COORDS
    int32_t* o = (int32_t*)out + base;
    if (full) {
      *(int4*)o = make_int4(u[0], u[1], u[2], u[3]);
      *(int4*)(o + 4) = make_int4(u[4], u[5], u[6], u[7]);
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = u[i];
    }
  }
}

// ---------------------------------------------------------------- the decode kernel
constexpr int kMaxBatch = 12;
constexpr int kRingWords = 32;                  // per-lane LDS ring (16-bit words)
constexpr int kRingDw = kRingWords / 2;
constexpr int kWaveRingBytes = 64 * kRingWords * 2;   // 4 KB per wave
constexpr int kMaxWaves = 16;

// Job descriptors travel by value in the kernel arguments (no per-launch copy).
struct DecBatch {
  DecJob j[kMaxBatch];
  int n;
};

template <int OUT, bool ESC>
__global__ void __launch_bounds__(1024) decode_kernel(const DecBatch B) {
  extern __shared__ __align__(16) uint32_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;

  // which job (uniform per workgroup)
  int ji = 0;
  for (int q = 1; q < B.n; ++q)
    if (B.j[q].wg_begin <= (int64_t)blockIdx.x) ji = q;
  const DecJob& J = B.j[ji];
  const int64_t blk = J.block_lo + ((int64_t)blockIdx.x - J.wg_begin) * nwaves + wave;

  // stage the decode tables (shared by the workgroup's waves)
  {
    const uint4* src = (const uint4*)J.tab;
    uint4* dst = (uint4*)smem;
    for (int i = tid; i < kTabWords / 4; i += blockDim.x) dst[i] = src[i];
  }
  __syncthreads();
  if (blk >= J.n_blocks) return;

  const int S = 1 << J.log2S;
  const int64_t chain = blk * 64 + lane;
  // region start via a wave prefix sum of the block's 32 region lengths
  const int64_t reg = blk * 32 + (lane >> 1);
  const uint32_t rl = (reg < J.n_regions) ? (uint32_t)J.rlen[reg] : 0u;
  uint32_t v = (lane & 1) ? 0u : rl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  const uint32_t rstart = J.ckpt[blk] + v - rl;      // absolute word index of the region start
  const uint32_t rend = rstart + rl;                 // one past the region
  const bool fwd = (lane & 1) == 0;
  const int dir = fwd ? 1 : -1;

  const bool live = chain < J.n_chains && chain >= J.chain_lo && chain < J.chain_hi;
  const int64_t t = chain >> J.log2S;
  const int j = (int)(chain & (S - 1));
  int64_t gt = J.n_groups - (t << 9);
  if (gt > kTileGroups) gt = kTileGroups;
  const int ngr = (live && gt > j) ? (int)((gt - j + S - 1) >> J.log2S) : 0;
  uint32_t x = (chain < J.n_chains) ? J.states[chain] : kL;

  // ---- per-lane ring of stream words: word w lives in ring[w % 32].
  // Invariant: whenever the lane reads word `pos` from the ring, it is resident.  A group
  // consumes at most 8 words for its symbols, so each group starts with >= 9 resident
  // words ahead; an escape consumes at most 2 more, so escapes top up to >= 11 first.
  // 16-byte chunks (8 words, 16-byte aligned) are loaded one group ahead of use.
  uint16_t* ring = (uint16_t*)(smem + kTabWords + (wave * 64 + lane) * kRingDw);
  const uint4* chunks = (const uint4*)J.stream;
  // fwd: fetched words end at `fetch` (multiple of 8); bwd: fetched words begin at `fetch`
  uint32_t pos = fwd ? rstart : rend - 1;            // next word to consume
  uint32_t fetch = fwd ? (rstart & ~7u) : ((rend + 7u) & ~7u);
  const uint32_t lim_hi = (rend + 7u) & ~7u;
  const uint32_t lim_lo = rstart & ~7u;
  uint4 pend = make_uint4(0, 0, 0, 0);
  uint32_t pend_c = 0;
  bool have_pend = false;
  auto resident = [&]() -> int {                     // words from pos on that are in the ring
    int a = fwd ? (int)(fetch - pos) : (int)(pos + 1 - fetch);
    return have_pend ? a - 8 : a;
  };
  auto more = [&]() -> bool { return fwd ? fetch < lim_hi : fetch > lim_lo; };
  auto next_chunk = [&]() -> uint32_t {
    uint32_t c = fwd ? fetch : fetch - 8u;
    fetch = fwd ? fetch + 8u : fetch - 8u;
    return c;
  };
  auto put = [&](uint32_t c, uint4 d) { *(uint4*)(ring + (c & (kRingWords - 1))) = d; };
  auto flush_pend = [&]() {
    if (have_pend) {
      put(pend_c, pend);
      have_pend = false;
    }
  };
  auto top_up = [&](int need) {                      // synchronous; rare after the prime
    flush_pend();
    while (resident() < need && more()) {
      uint32_t c = next_chunk();
      put(c, chunks[c >> 3]);
    }
  };
  if (live && rl) {
    // prime: two chunks loaded together (>= 9 words ahead of any start position)
    uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
    uint32_t c0 = 0, c1 = 0;
    bool h0 = false, h1 = false;
    if (more()) { c0 = next_chunk(); d0 = chunks[c0 >> 3]; h0 = true; }
    if (more()) { c1 = next_chunk(); d1 = chunks[c1 >> 3]; h1 = true; }
    if (h0) put(c0, d0);
    if (h1) put(c1, d1);
    top_up(9);
  }
  uint32_t nw = ring[pos & (kRingWords - 1)];

  int64_t g = (t << 9) + j;
  int64_t row = live ? g / J.G : 0;
  int64_t col = g - row * J.G;
  const int k = J.k;

  auto renorm = [&]() {
    if (x < kL) {
      x = (x << 16) | nw;
      pos += dir;
      nw = ring[pos & (kRingWords - 1)];
    }
  };
  auto step = [&](const uint32_t* tb) -> uint32_t {
    uint32_t e = tb[x & (kM - 1)];
    x = __umul24(e & 2047u, x >> 11) + ((e >> 11) & 2047u);
    renorm();
    return e;
  };
  auto bypass = [&](int nb) -> uint32_t {
    uint32_t r = x & ((1u << nb) - 1u);
    x >>= nb;
    renorm();
    return r;
  };
  auto escape = [&](uint32_t e, int last, int pi) -> int32_t {
    if (resident() < 11) top_up(11);
    uint32_t info = e >> 23;
    int c = (int)(info & 1u), neg = (int)((info >> 1) & 1u), top2 = (int)((info >> 2) & 3u);
    int ex = k + (int)(info >> 4);
    int nb = ex - 2 - last;
    uint32_t raw = bypass(nb < 16 ? nb : 16);
    if (nb > 16) raw |= bypass(nb - 16) << 16;
    if (last) raw = (raw << 1) | (uint32_t)(c == 0 ? pi : (pi ^ neg));
    uint32_t m = (1u << ex) | ((uint32_t)top2 << (ex - 2)) | raw;
    int32_t uu = (int32_t)(2u * m + (uint32_t)c);
    return neg ? -uu : uu;
  };

  float h = ngr > 0 ? J.hr[row] : 0.f;
  for (int kk = 0; kk < ngr; ++kk) {
    // ---- keep the ring fed: land last group's chunk, guarantee 9 resident words,
    // then start loading the next chunk if its ring slots are already consumed
    flush_pend();
    if (resident() < 9) top_up(9);
    if ((fwd ? (int)(fetch - pos) : (int)(pos + 1 - fetch)) <= kRingWords - 8 && more()) {
      pend_c = next_chunk();
      pend = chunks[pend_c >> 3];
      have_pend = true;
    }
    // ---- row scale of the next group, loaded one group ahead
    int64_t nrow = row, ncol = col + S;
    while (ncol >= J.G) {
      ncol -= J.G;
      ++nrow;
    }
    const float h_next = (kk + 1 < ngr) ? J.hr[nrow] : 0.f;

    int32_t u[8];
    uint32_t e = step(smem);
    u[0] = (int32_t)e >> 23;
    if (ESC && (e & kEscBit)) u[0] = escape(e, 0, 0);
    const int c = (int)((e >> 23) & 1u);
    const uint32_t* tf = smem + ((1 + c) << 11);
    int par = u[0] >> 1;
#pragma unroll
    for (int i = 1; i < 7; ++i) {
      e = step(tf);
      u[i] = (int32_t)e >> 23;
      if (ESC && (e & kEscBit)) u[i] = escape(e, 0, 0);
      par ^= u[i] >> 1;
    }
    const int pi = par & 1;
    e = step(smem + ((3 + 2 * c + pi) << 11));
    u[7] = (int32_t)e >> 23;
    if (ESC && (e & kEscBit)) u[7] = escape(e, 1, pi);

    const int64_t c0 = col * 8;
    const bool full = J.c8 || (c0 + 8 <= J.C);
    store_group<OUT>(J.out, row * J.C + c0, u, h, full, J.C - c0);
    row = nrow;
    col = ncol;
    h = h_next;
  }
  if (live && x != kL) atomicAdd(J.err, 1u);
}

// ---------------------------------------------------------------- launch helpers
int lds_max_bytes() {
  static int v = -1;
  if (v < 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    int x = 0;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || x <= 0) x = 65536;
    v = x;
  }
  return v;
}

template <int OUT, bool ESC>
int launch_t(const DecBatch& B, int64_t n_wg, int waves, hipStream_t st) {
  auto kern = decode_kernel<OUT, ESC>;
  size_t lds = (size_t)kTabBytes + (size_t)waves * kWaveRingBytes;
  static std::once_flag once;
  std::call_once(once, [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max_bytes());
  });
  hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(64 * waves), lds, st, B);
  return hip_check(hipGetLastError(), "decode launch");
}

template <bool ESC>
int launch_out(int out, const DecBatch& B, int64_t n_wg, int waves, hipStream_t st) {
  switch (out) {
    case OUT_BF16: return launch_t<OUT_BF16, ESC>(B, n_wg, waves, st);
    case OUT_BF16_SAT: return launch_t<OUT_BF16_SAT, ESC>(B, n_wg, waves, st);
    case OUT_FP16: return launch_t<OUT_FP16, ESC>(B, n_wg, waves, st);
    case OUT_FP32: return launch_t<OUT_FP32, ESC>(B, n_wg, waves, st);
    case OUT_FP8: return launch_t<OUT_FP8, ESC>(B, n_wg, waves, st);
    case OUT_INT8: return launch_t<OUT_INT8, ESC>(B, n_wg, waves, st);
    default: return launch_t<OUT_COORDS, ESC>(B, n_wg, waves, st);
  }
}

int launch_any(int out, bool esc, const DecBatch& B, int64_t n_wg, int waves, hipStream_t st) {
  return esc ? launch_out<true>(out, B, n_wg, waves, st) : launch_out<false>(out, B, n_wg, waves, st);
}

int out_kind(const Blob& b) {
  switch (b.dtype) {
    case EP_BF16: return (b.flags & kFlagSat) ? OUT_BF16_SAT : OUT_BF16;
    case EP_FP16: return OUT_FP16;
    case EP_FP32: return OUT_FP32;
    case EP_FP8_E4M3FN: return OUT_FP8;
    default: return OUT_INT8;
  }
}

DecJob make_job(const Blob& b, void* out) {
  DecJob j{};
  j.stream = b.d_stream;
  j.states = b.d_states;
  j.rlen = b.d_rlen;
  j.ckpt = b.d_ckpt;
  j.hr = b.d_hr;
  j.tab = b.d_tab;
  j.err = b.d_err;
  j.out = out;
  j.n_groups = b.n_groups();
  j.G = (b.C + 7) / 8;
  j.C = b.C;
  j.n_chains = b.n_chains;
  j.n_regions = b.n_regions;
  j.n_blocks = b.n_blocks;
  j.chain_lo = 0;
  j.chain_hi = b.n_chains;
  j.block_lo = 0;
  j.wg_begin = 0;
  j.n_words = (uint32_t)b.n_words;
  j.log2S = __builtin_ctz((unsigned)b.S);
  j.k = b.k;
  j.c8 = (b.C % 8) == 0;
  return j;
}

// Waves per workgroup.  One table copy (56 KB of LDS) serves the workgroup; each wave
// adds a 4 KB ring.  Small launches use small workgroups so the blocks spread over all
// 256 CUs; big launches use up to 16 waves (4 per SIMD) to hide the per-step latency.
int pick_waves(int64_t n_blocks) {
  const int cus = 256;
  int w = (int)std::min<int64_t>(kMaxWaves, std::max<int64_t>(1, (n_blocks + cus - 1) / cus));
  const int by_lds = (lds_max_bytes() - kTabBytes) / kWaveRingBytes;
  w = std::min(w, by_lds);
  if (const char* e = std::getenv("EP_DECODE_WAVES")) {
    int v = std::atoi(e);
    if (v >= 1 && v <= kMaxWaves) w = std::min(v, by_lds);
  }
  return std::max(w, 1);
}

int check_uploaded(const Blob& b) {
  if (!b.d_base) return fail(EP_E_STATE, "blob not uploaded (call ep_blob_upload)");
  int dev = -1;
  (void)hipGetDevice(&dev);
  if (dev != b.device) return fail(EP_E_STATE, "blob uploaded to another device");
  return EP_OK;
}

int decode_one(const Blob& b, void* dst, int64_t chain_lo, int64_t chain_hi, int out, hipStream_t st) {
  int rc = check_uploaded(b);
  if (rc) return rc;
  if (!dst) return fail(EP_E_ARG, "null destination");
  if (out != OUT_COORDS && (reinterpret_cast<uintptr_t>(dst) & 15)) return fail(EP_E_ARG, "destination must be 16-byte aligned");
  if (out == OUT_COORDS && (reinterpret_cast<uintptr_t>(dst) & 15)) return fail(EP_E_ARG, "destination must be 16-byte aligned");
  DecJob j = make_job(b, dst);
  j.chain_lo = chain_lo;
  j.chain_hi = chain_hi;
  const int64_t blo = chain_lo / kBlockChains;
  const int64_t bhi = (chain_hi + kBlockChains - 1) / kBlockChains;
  if (bhi <= blo) return EP_OK;
  j.block_lo = blo;
  const int64_t nblk = bhi - blo;
  const int waves = pick_waves(nblk);
  const int64_t n_wg = (nblk + waves - 1) / waves;
  j.n_blocks = bhi;   // blocks beyond the range are skipped
  DecBatch B{};
  B.j[0] = j;
  B.n = 1;
  return launch_any(out, (b.flags & kFlagEsc) != 0, B, n_wg, waves, st);
}

}  // namespace
}  // namespace ep

using namespace ep;

// Release the device mirror (called from ep_blob_free).
void ep_device_release(ep::Blob* b) {
  if (b->d_base) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (b->device >= 0 && b->device != cur) (void)hipSetDevice(b->device);
    (void)hipFree(b->d_base);
    if (b->device >= 0 && b->device != cur) (void)hipSetDevice(cur);
  }
  b->d_base = nullptr;
}

extern "C" {

int ep_blob_upload(ep_blob* blob, ep_stream stream) {
  set_error("");
  if (!blob) return fail(EP_E_ARG, "null blob");
  Blob& b = blob->b;
  if (b.d_base) return EP_OK;
  auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t o_tab = 0;
  const size_t o_hr = o_tab + al(kTabBytes);
  const size_t o_st = o_hr + al(4 * (size_t)b.R);
  const size_t o_ck = o_st + al(4 * (size_t)b.n_chains);
  const size_t o_rl = o_ck + al(4 * (size_t)(b.n_blocks + 1));
  const size_t o_err = o_rl + al(2 * (size_t)b.n_regions);
  const size_t o_stream = o_err + 256;
  const size_t total = o_stream + al(2 * (size_t)b.n_words + 64);
  std::vector<uint8_t> host;
  try {
    host.assign(total, 0);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  build_slot_tables(b.model, (uint32_t*)&host[o_tab]);
  half_scales(b, (float*)&host[o_hr]);
  std::memcpy(&host[o_st], &b.bytes[b.off_states], 4 * (size_t)b.n_chains);
  std::memcpy(&host[o_ck], &b.bytes[b.off_ckpt], 4 * (size_t)b.n_blocks);
  uint32_t nw = (uint32_t)b.n_words;
  std::memcpy(&host[o_ck + 4 * (size_t)b.n_blocks], &nw, 4);
  std::memcpy(&host[o_rl], &b.bytes[b.off_rlen], 2 * (size_t)b.n_regions);
  std::memcpy(&host[o_stream], &b.bytes[b.off_stream], 2 * (size_t)b.n_words);
  void* d = nullptr;
  if (hipMalloc(&d, total) != hipSuccess) {
    (void)hipGetLastError();
    return fail(EP_E_NOMEM, "device allocation failed");
  }
  int rc = hip_check(hipMemcpyAsync(d, host.data(), total, hipMemcpyHostToDevice, (hipStream_t)stream), "upload");
  if (!rc) rc = hip_check(hipStreamSynchronize((hipStream_t)stream), "upload sync");
  if (rc) {
    (void)hipFree(d);
    return rc;
  }
  (void)hipGetDevice(&b.device);
  b.d_base = d;
  uint8_t* p = (uint8_t*)d;
  b.d_tab = (const uint32_t*)(p + o_tab);
  b.d_hr = (const float*)(p + o_hr);
  b.d_states = (const uint32_t*)(p + o_st);
  b.d_ckpt = (const uint32_t*)(p + o_ck);
  b.d_rlen = (const uint16_t*)(p + o_rl);
  b.d_err = (uint32_t*)(p + o_err);
  b.d_stream = (const uint16_t*)(p + o_stream);
  return EP_OK;
}

int ep_decompress(const ep_blob* blob, void* dev_dst, ep_stream stream) {
  set_error("");
  if (!blob) return fail(EP_E_ARG, "null blob");
  const Blob& b = blob->b;
  return decode_one(b, dev_dst, 0, b.n_chains, out_kind(b), (hipStream_t)stream);
}

int ep_decompress_tiles(const ep_blob* blob, int64_t tile_begin, int64_t tile_end, void* dev_dst, ep_stream stream) {
  set_error("");
  if (!blob) return fail(EP_E_ARG, "null blob");
  const Blob& b = blob->b;
  if (tile_begin < 0 || tile_end > b.n_tiles || tile_begin > tile_end) return fail(EP_E_ARG, "tile range out of bounds");
  return decode_one(b, dev_dst, tile_begin * b.S, tile_end * b.S, out_kind(b), (hipStream_t)stream);
}

int ep_test_decode_coords(const ep_blob* blob, int32_t* dev_u, ep_stream stream) {
  set_error("");
  if (!blob) return fail(EP_E_ARG, "null blob");
  const Blob& b = blob->b;
  return decode_one(b, dev_u, 0, b.n_chains, OUT_COORDS, (hipStream_t)stream);
}

int ep_decompress_batch(const ep_blob* const* blobs, void* const* dsts, int n, ep_stream stream) {
  set_error("");
  if (n < 0 || (n > 0 && (!blobs || !dsts))) return fail(EP_E_ARG, "null pointer");
  if (n == 0) return EP_OK;
  // all blobs of one launch share the container kind and the escape path
  int out = -1;
  bool esc = false;
  int64_t total_blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (!blobs[i] || !dsts[i]) return fail(EP_E_ARG, "null blob or destination");
    const Blob& b = blobs[i]->b;
    int rc = check_uploaded(b);
    if (rc) return rc;
    if (reinterpret_cast<uintptr_t>(dsts[i]) & 15) return fail(EP_E_ARG, "destination must be 16-byte aligned");
    int o = out_kind(b);
    if (o == OUT_BF16_SAT) o = OUT_BF16_SAT;
    if (out < 0) out = o;
    else if ((out == OUT_BF16 || out == OUT_BF16_SAT) && (o == OUT_BF16 || o == OUT_BF16_SAT))
      out = (out == OUT_BF16_SAT || o == OUT_BF16_SAT) ? OUT_BF16_SAT : OUT_BF16;
    else if (o != out) return fail(EP_E_ARG, "batch mixes container dtypes");
    esc |= (b.flags & kFlagEsc) != 0;
    total_blocks += b.n_blocks;
  }
  const int waves = pick_waves(total_blocks);
  // up to kMaxBatch blobs per launch
  for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
    DecBatch B{};
    B.n = std::min(kMaxBatch, n - i0);
    int64_t wg = 0;
    for (int q = 0; q < B.n; ++q) {
      B.j[q] = make_job(blobs[i0 + q]->b, dsts[i0 + q]);
      B.j[q].wg_begin = wg;
      wg += (B.j[q].n_blocks + waves - 1) / waves;
    }
    int rc = launch_any(out, esc, B, wg, waves, (hipStream_t)stream);
    if (rc) return rc;
  }
  return EP_OK;
}

int64_t ep_blob_device_errors(const ep_blob* blob) {
  if (!blob || !blob->b.d_base) return -1;
  uint32_t v = 0;
  if (hipDeviceSynchronize() != hipSuccess) return -1;
  if (hipMemcpy(&v, blob->b.d_err, 4, hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return (int64_t)v;
}

size_t ep_linear_workspace_bytes(const ep_blob* blob) {
  if (!blob) return 0;
  return (size_t)blob->b.R * (size_t)blob->b.C * 2 + 256;
}

}  // extern "C"
