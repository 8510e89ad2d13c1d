// The lossy encoder on the GPU: the same blob, byte for byte, as the host encoder.
//
// [README] 快速开始 / [NEWS]: the library encodes and decodes on the GPU; [README] 性能:
// the 276 linear layers of a diffusion transformer compress in seconds.  [ABS]: row
// normalisation, E8 quantisation at a resolution picked from sampled storage
// estimates, a conditional model, tile-wise rANS.
//
// Steps (device unless noted):
//   row statistics   per row (one lane per row, rows staged through LDS in 32-column
//                    slices): RMS summed left to right in float64, BF16 row scale, the
//                    row's largest |w|, non-finite / too-small rows
//   search (host)    the host encoder's resolution search; each probe quantises the
//                    sample rows on the device (E8 per group of 8, counts of large
//                    magnitudes for k), then counts symbols per context; the host builds
//                    the model and prices the counts with LOG2Q
//   final pass       quantise all rows, count, model (host); per-row distortion and
//                    clamping; one thread per rANS chain encodes its groups backwards;
//                    one thread per tile replays the decoder's fetch schedule to rank
//                    the chain's chunks; one thread per chain scatters them into the
//                    block areas.  Block offsets and the header are assembled on the host.
// Per-group arithmetic comes from codec_math.h, shared with the host encoder.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <string>
#include <thread>
#include <vector>

#include "codec_math.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kHistIds = 1024;
constexpr int kHistBins = kNumCtx * kHistIds;

__device__ inline uint16_t dev_f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((uint64_t(u) + 0x7FFFu + lsb) >> 16);
}

// ---------------------------------------------------------------- row statistics
// flags: bit 0 = some value is not finite, bit 1 = a nonzero row's RMS is below the BF16
// normal range
__global__ void row_stats_kernel(const void* src, int dtype, int64_t R, int64_t C, uint16_t* s_bits, float* s,
                                 double* amax, uint32_t* flags) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  double acc = 0.0, am = 0.0;
  bool live = false, bad = false;
  for (int64_t c = 0; c < C; ++c) {
    const double v = cm::widen_one(src, dtype, r * C + c);
    if (!isfinite(v)) bad = true;
    acc = acc + v * v;
    const double a = fabs(v);
    if (a > am) am = a;
    live |= v != 0.0;
  }
  const double rms = sqrt(acc / (double)C);
  const uint16_t sb = dev_f32_to_bf16_rne((float)rms);
  s_bits[r] = sb;
  s[r] = __uint_as_float((uint32_t)sb << 16);
  amax[r] = am;
  if (bad) atomicOr(flags, 1u);
  if (live && ((sb >> 7) & 0xFF) == 0) atomicOr(flags, 2u);
}

// ---------------------------------------------------------------- quantisation
// Groups of the listed rows (all rows when rows == nullptr): u (8 doubled coordinates
// per group) and ge[k - 3] += #coordinates with magnitude >= 2^k, k = 3..7.
__global__ void quantize_kernel(const void* src, int dtype, int64_t C, int64_t G, const int64_t* rows,
                                int64_t n_rows, const float* s, float delta, int32_t* u,
                                unsigned long long* ge) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  if (gi < n_rows * G) {
    const int64_t ri = gi / G, gc = gi - ri * G;
    const int64_t r = rows ? rows[ri] : ri;
    const float h = s[r] * delta;
    const double den = 2.0 * (double)h;
    double y[8];
    for (int i = 0; i < 8; ++i) {
      const int64_t col = gc * 8 + i;
      const double v = col < C ? cm::widen_one(src, dtype, r * C + col) : 0.0;
      y[i] = (den != 0.0) ? v / den : 0.0;
    }
    int32_t uu[8];
    cm::e8_doubled(y, uu);
    const int c = uu[0] & 1;
    for (int i = 0; i < 8; ++i) {
      u[gi * 8 + i] = uu[i];
      const int a = uu[i] < 0 ? -uu[i] : uu[i];
      const int64_t m = (a - c) >> 1;
      for (int kk = 0; kk < 5; ++kk) cnt[kk] += m >= (1 << (kk + 3));
    }
  }
  for (int kk = 0; kk < 5; ++kk) {
    uint32_t v = cnt[kk];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off);
    if ((threadIdx.x & 63) == 0 && v) atomicAdd(&ge[kk], (unsigned long long)v);
  }
}

// Symbol counts per (context, id) and the raw bits, for a chosen k.
// k < 0: the escape bucket k is picked here from the quantiser's counts ge of
// magnitudes >= 2^k (the smallest k in 3..7 whose count is at most 2^-20 of the
// coordinates, else 7) and written to k_out, so the host needs no round trip for it
__global__ void histogram_kernel(const int32_t* u, int64_t n_groups, int k, const unsigned long long* ge,
                                 unsigned long long* hist, unsigned long long* rawbits, unsigned long long* k_out) {
  __shared__ uint32_t lh[kHistBins];
  if (k < 0) {
    k = 7;
    for (int kk = 3; kk <= 7; ++kk)
      if ((int64_t)ge[kk - 3] * (int64_t(1) << 20) <= n_groups * 8) {
        k = kk;
        break;
      }
    if (blockIdx.x == 0 && threadIdx.x == 0) *k_out = (unsigned long long)k;
  }
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0;
  __syncthreads();
  uint32_t rb = 0;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n_groups; g += (int64_t)gridDim.x * blockDim.x) {
    cm::Sym sy[8];
    int ms[8];
    cm::symbolize(u + g * 8, k, sy, ms);
    for (int i = 0; i < 8; ++i) {
      atomicAdd(&lh[sy[i].ctx * kHistIds + sy[i].id], 1u);
      rb += (uint32_t)sy[i].rawbits;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (lh[i]) atomicAdd(&hist[i], (unsigned long long)lh[i]);
  for (int off = 32; off > 0; off >>= 1) rb += __shfl_down(rb, off);
  if ((threadIdx.x & 63) == 0 && rb) atomicAdd(rawbits, (unsigned long long)rb);
}

// Per row: squared error of fl32(h u) against w and w^2 (left to right), and whether a
// value leaves its container's range.
__global__ void row_error_kernel(const void* src, int dtype, int64_t R, int64_t C, int64_t G, const float* s,
                                 float delta, const int32_t* u, double cmax, double* se, double* sw,
                                 uint32_t* sat) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const float h = s[r] * delta;
  double e = 0.0, q = 0.0;
  bool out = false;
  for (int64_t c = 0; c < C; ++c) {
    const double w = cm::widen_one(src, dtype, r * C + c);
    const float v = h * (float)u[r * G * 8 + c];
    const double d = w - (double)v;
    e += d * d;
    q += w * w;
    const double dv = (double)v;
    if (dtype != EP_FP32) {
      if (dtype == EP_INT8) out |= nearbyint(dv) > 127.0 || nearbyint(dv) < -128.0;
      else out |= fabs(dv) > cmax;
    }
  }
  se[r] = e;
  sw[r] = q;
  if (out) atomicOr(sat, 1u);
}

// ---------------------------------------------------------------- tiled row passes
// The same per-row sums with one wave per 64 rows: the wave stages 32-column slices of
// its rows (and of the lattice coordinates) in LDS with coalesced 16-byte loads, then
// every lane walks its own row's slice left to right, so each row's float64 sums keep
// the one-thread-per-row order exactly.  Needs rows of a multiple of 16 bytes and a
// 16-byte aligned source.
constexpr int kTileRowBytes = 144;   // 128-byte slice + 16 bytes against bank conflicts

// element k of a 32-column slice held in registers (w: 2 esz dwords per 16 bytes)
template <int DT>
__device__ __forceinline__ double slice_value(const uint32_t* w, int k) {
  if constexpr (DT == EP_FP32) {
    return (double)__uint_as_float(w[k]);
  } else if constexpr (DT == EP_BF16 || DT == EP_FP16) {
    const uint16_t b = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
    return DT == EP_BF16 ? cm::bf16_value(b) : cm::fp16_value(b);
  } else {
    const uint8_t b = (uint8_t)(w[k >> 2] >> (8 * (k & 3)));
    return DT == EP_FP8_E4M3FN ? cm::fp8_e4m3fn_value(b) : (double)(int8_t)b;
  }
}

// the lane's row of a staged slice, into registers (nd dwords)
template <int ND>
__device__ __forceinline__ void slice_regs(const uint8_t* ts, int lane, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < ND / 4; ++i) {
    const uint4 v = *(const uint4*)(ts + lane * kTileRowBytes + 16 * i);
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// stage rows r0 .. r0 + 63, columns c0 .. c0 + 31 of a row-major array with `rowb`
// bytes per row (element size esz) into ts (row rr at rr * kTileRowBytes); pieces past
// the rows' end or past R read as zero
__device__ __forceinline__ void stage_slice(const uint8_t* base, int64_t R, int64_t rowb, int esz, int64_t r0,
                                            int64_t c0, uint8_t* ts, int lane) {
  const int spr = 2 * esz;   // 16-byte pieces per row of a 32-column slice
  for (int p = lane; p < 64 * spr; p += 64) {
    const int rr = p / spr, pp = p % spr;
    const int64_t gr = r0 + rr;
    const int64_t cb = c0 * esz + pp * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (gr < R && cb < rowb) v = *(const uint4*)(base + gr * rowb + cb);
    *(uint4*)(ts + rr * kTileRowBytes + pp * 16) = v;
  }
}

template <int DT>
__global__ void __launch_bounds__(64) row_stats_tiled_kernel(const void* src, int64_t R, int64_t C, uint16_t* s_bits,
                                                             float* s, double* amax, uint32_t* flags) {
  __shared__ __align__(16) uint8_t ts[64 * kTileRowBytes];
  constexpr int esz = DT == EP_FP32 ? 4 : (DT == EP_FP8_E4M3FN || DT == EP_INT8 ? 1 : 2);
  const int lane = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 64, r = r0 + lane;
  double acc = 0.0, am = 0.0;
  bool live = false, bad = false;
  for (int64_t c0 = 0; c0 < C; c0 += 32) {
    stage_slice((const uint8_t*)src, R, C * esz, esz, r0, c0, ts, lane);
    __syncthreads();
    const int n = C - c0 < 32 ? (int)(C - c0) : 32;
    uint32_t wr[8 * esz];
    slice_regs<8 * esz>(ts, lane, wr);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k >= n) break;
      const double v = slice_value<DT>(wr, k);
      if (!isfinite(v)) bad = true;
      acc = acc + v * v;
      const double a = fabs(v);
      if (a > am) am = a;
      live |= v != 0.0;
    }
    __syncthreads();
  }
  if (r >= R) return;
  const double rms = sqrt(acc / (double)C);
  const uint16_t sb = dev_f32_to_bf16_rne((float)rms);
  s_bits[r] = sb;
  s[r] = __uint_as_float((uint32_t)sb << 16);
  amax[r] = am;
  if (bad) atomicOr(flags, 1u);
  if (live && ((sb >> 7) & 0xFF) == 0) atomicOr(flags, 2u);
}

template <int DT>
__global__ void __launch_bounds__(64) row_error_tiled_kernel(const void* src, int64_t R, int64_t C, int64_t G,
                                                             const float* s, float delta, const int32_t* u,
                                                             double cmax, double* se, double* sw, uint32_t* sat) {
  __shared__ __align__(16) uint8_t ts[64 * kTileRowBytes];
  __shared__ __align__(16) uint8_t tu[64 * kTileRowBytes];
  constexpr int esz = DT == EP_FP32 ? 4 : (DT == EP_FP8_E4M3FN || DT == EP_INT8 ? 1 : 2);
  const int lane = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 64, r = r0 + lane;
  const float h = r < R ? s[r] * delta : 0.f;
  double e = 0.0, q = 0.0;
  bool out = false;
  for (int64_t c0 = 0; c0 < C; c0 += 32) {
    stage_slice((const uint8_t*)src, R, C * esz, esz, r0, c0, ts, lane);
    stage_slice((const uint8_t*)u, R, G * 8 * 4, 4, r0, c0, tu, lane);
    __syncthreads();
    const int n = C - c0 < 32 ? (int)(C - c0) : 32;
    uint32_t wr[8 * esz], ur[32];
    slice_regs<8 * esz>(ts, lane, wr);
    slice_regs<32>(tu, lane, ur);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k >= n) break;
      const double w = slice_value<DT>(wr, k);
      const float v = h * (float)(int32_t)ur[k];
      const double d = w - (double)v;
      e += d * d;
      q += w * w;
      const double dv = (double)v;
      if (DT != EP_FP32) {
        if (DT == EP_INT8) out |= nearbyint(dv) > 127.0 || nearbyint(dv) < -128.0;
        else out |= fabs(dv) > cmax;
      }
    }
    __syncthreads();
  }
  if (r >= R) return;
  se[r] = e;
  sw[r] = q;
  if (out) atomicOr(sat, 1u);
}


// ---------------------------------------------------------------- rANS chains
// One thread per chain: groups j, j+S, ... of its tile, encoded last to first (the
// decoder reads them first to last).  Words are stored in emission order (the reverse
// of decoding order); cons (words per group) feeds the schedule.
__global__ void encode_chains_kernel(const int32_t* u, int64_t n_groups, int S, int log2S, int64_t n_chains, int k,
                                     const int32_t* F, const int32_t* CUM, int max_words, int steps, uint16_t* words,
                                     uint8_t* cons, uint32_t* len, uint32_t* state) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= n_chains) return;
  const int64_t t = ch >> log2S;
  const int j = (int)(ch & (S - 1));
  const int64_t gt = min((int64_t)kTileGroups, n_groups - (int64_t)kTileGroups * t);
  const int ngr = gt > j ? (int)((gt - j + S - 1) / S) : 0;
  uint16_t* w = words + ch * (int64_t)max_words;
  uint32_t x = kL;
  int n = 0;
  const int P = k >= 6 ? 11 : 10;   // the table precision of escape threshold 2^k (precision())
  for (int kk = ngr - 1; kk >= 0; --kk) {
    const int64_t g = (int64_t)kTileGroups * t + j + (int64_t)kk * S;
    cm::Sym sy[8];
    int ms[8];
    cm::symbolize(u + g * 8, k, sy, ms);
    const int n0 = n;
    for (int i = 7; i >= 0; --i) {
      const int rb = sy[i].rawbits;
      if (rb > 16) {
        const int b = rb - 16;
        if (x >= (1u << (32 - b))) {
          w[n++] = (uint16_t)(x & 0xFFFFu);
          x >>= 16;
        }
        x = (x << b) | (sy[i].rawval >> 16);
      }
      if (rb > 0) {
        const int b = rb < 16 ? rb : 16;
        if (b == 16 ? (x >= 65536u) : (x >= (1u << (32 - b)))) {
          w[n++] = (uint16_t)(x & 0xFFFFu);
          x >>= 16;
        }
        x = (b == 32 ? 0u : (x << b)) | (sy[i].rawval & 0xFFFFu);
      }
      const uint32_t f = (uint32_t)F[sy[i].ctx * kHistIds + sy[i].id];
      const uint32_t cum = (uint32_t)CUM[sy[i].ctx * kHistIds + sy[i].id];
      if ((uint64_t)x >= ((uint64_t)f << (32 - P))) {
        w[n++] = (uint16_t)(x & 0xFFFFu);
        x >>= 16;
      }
      x = (x / f) * (1u << P) + (x % f) + cum;
    }
    cons[ch * steps + kk] = (uint8_t)(n - n0);
  }
  len[ch] = (uint32_t)n;
  state[ch] = x;
}

// One thread per tile: the decoder's fetch schedule, handing out the tile's main-area
// positions in request order.  Blobs without escapes: prime to 17 words ahead, before
// every even group to 17 ahead plus one round for chains at most 24 ahead; blobs with
// escapes: prime to 24 ahead, before every group to 24 ahead plus the same round.
__global__ void schedule_kernel(const uint32_t* len, const uint8_t* cons, int64_t n_groups, int S, int64_t n_tiles,
                                int steps, int max_full, bool esc, uint16_t* rank) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_tiles) return;
  int32_t Fw[64], q[64], n[64], ngr[64], nf[64];
  uint16_t ctr = 0;
  int gmax = 0;
  const int64_t gt = min((int64_t)kTileGroups, n_groups - (int64_t)kTileGroups * t);
  for (int j = 0; j < S; ++j) {
    Fw[j] = 0;
    q[j] = 0;
    nf[j] = 0;
    n[j] = (int32_t)len[t * S + j];
    ngr[j] = gt > j ? (int)((gt - j + S - 1) / S) : 0;
    gmax = max(gmax, ngr[j]);
  }
  auto take = [&](int j) {
    if (n[j] - Fw[j] >= 8) {
      rank[(t * S + j) * (int64_t)max_full + nf[j]++] = ctr++;
      Fw[j] += 8;
    } else {
      Fw[j] = n[j];
    }
  };
  // sync: rounds until no candidate wants more (all chains, or those decoding group g)
  auto sync = [&](bool all, int g, int32_t ahead) {
    for (;;) {
      bool any = false;
      for (int j = 0; j < S; ++j) {
        if ((all || g < ngr[j]) && Fw[j] - q[j] < ahead && Fw[j] < n[j]) {
          take(j);
          any = true;
        }
      }
      if (!any) return;
    }
  };
  const int32_t ahead = esc ? 24 : 17;
  sync(true, 0, ahead);
  for (int g = 0; g < gmax; ++g) {
    if (esc || (g & 1) == 0) {
      sync(false, g, ahead);
      for (int j = 0; j < S; ++j)
        if (g < ngr[j] && Fw[j] - q[j] <= 24 && Fw[j] < n[j]) take(j);
    }
    for (int j = 0; j < S; ++j)
      if (g < ngr[j]) q[j] += cons[(t * S + j) * steps + g];
  }
}

// One thread per chain: full chunks to their request-order slots, the tail to the
// block's tail area (word i of the chain in decoding order is emitted word len-1-i).
__global__ void layout_kernel(const uint16_t* words, int max_words, const uint32_t* len, const uint16_t* rank,
                              int max_full, const int64_t* dst_main, const int64_t* dst_tail, int64_t n_chains,
                              uint16_t* stream, int64_t n_words) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= n_chains) return;
  const uint16_t* w = words + ch * (int64_t)max_words;
  const int L0 = (int)len[ch];
  const int nfull = L0 / 8;
  // (positions are checked against the stream: a bad schedule cannot write outside it)
  for (int nn = 0; nn < nfull; ++nn) {
    const int64_t p = dst_main[ch] + 8 * (int64_t)rank[ch * (int64_t)max_full + nn];
    if (p < 0 || p + 8 > n_words) continue;
    for (int i = 0; i < 8; ++i) stream[p + i] = w[L0 - 1 - (8 * nn + i)];
  }
  for (int i = 8 * nfull; i < L0; ++i) {
    const int64_t p = dst_tail[ch] + (i - 8 * nfull);
    if (p >= 0 && p < n_words) stream[p] = w[L0 - 1 - i];
  }
}

// ---------------------------------------------------------------- host side
// Device buffers of one encode.  A batch worker turns on a per-thread cache, so the
// buffers of one matrix are reused by the next instead of freed (a free waits for the
// whole device and would serialise the workers); a matrix's work on its stream is done
// before its buffers go back (the encode ends with a stream synchronisation).
thread_local bool t_cache_on = false;
thread_local std::vector<std::pair<void*, size_t>> t_cache;   // free blocks and their sizes

struct DevBuf {
  void* p = nullptr;
  size_t cap = 0;
  ~DevBuf() {
    if (!p) return;
    if (t_cache_on) t_cache.emplace_back(p, cap);
    else (void)hipFree(p);
  }
  template <class T>
  T* as() const {
    return (T*)p;
  }
};

int dalloc(DevBuf& b, size_t bytes) {
  bytes = std::max<size_t>(bytes, 16);
  if (t_cache_on) {   // the smallest cached block that fits
    size_t best = t_cache.size();
    for (size_t i = 0; i < t_cache.size(); ++i)
      if (t_cache[i].second >= bytes && (best == t_cache.size() || t_cache[i].second < t_cache[best].second)) best = i;
    if (best < t_cache.size()) {
      b.p = t_cache[best].first;
      b.cap = t_cache[best].second;
      t_cache.erase(t_cache.begin() + (ptrdiff_t)best);
      return EP_OK;
    }
  }
  if (hipMalloc(&b.p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    b.p = nullptr;
    return fail(EP_E_NOMEM, "device allocation failed");
  }
  b.cap = bytes;
  return EP_OK;
}

void cache_release() {
  for (auto& e : t_cache) (void)hipFree(e.first);
  t_cache.clear();
  t_cache_on = false;
}

// pinned host memory (allocated here, never registered after the fact)
struct HostBuf {
  void* p = nullptr;
  ~HostBuf() {
    if (p) (void)hipHostFree(p);
  }
};

int halloc(HostBuf& b, size_t bytes) {
  if (hipHostMalloc(&b.p, std::max<size_t>(bytes, 16), hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    b.p = nullptr;
    return fail(EP_E_NOMEM, "pinned host allocation failed");
  }
  return EP_OK;
}

void put16(std::vector<uint8_t>& b, size_t off, uint16_t v) { std::memcpy(&b[off], &v, 2); }
void put32(std::vector<uint8_t>& b, size_t off, uint32_t v) { std::memcpy(&b[off], &v, 4); }
void put64(std::vector<uint8_t>& b, size_t off, uint64_t v) { std::memcpy(&b[off], &v, 8); }

// coset counts and per-coset magnitude counts from the (context, id) counts
void model_counts(const std::vector<unsigned long long>& h, int k, int64_t cc[2], std::vector<int64_t>& mag0,
                  std::vector<int64_t>& mag1) {
  const int nm = n_msym(k);
  mag0.assign(nm, 0);
  mag1.assign(nm, 0);
  cc[0] = cc[1] = 0;
  for (int c = 0; c < 2; ++c) {
    auto& mg = c ? mag1 : mag0;
    for (int sid = 0; sid < 2 * nm; ++sid) {
      const int64_t first = (int64_t)h[0 * kHistIds + 512 * c + sid];
      cc[c] += first;
      int64_t v = first + (int64_t)h[(1 + c) * kHistIds + sid] + (int64_t)h[(3 + 2 * c) * kHistIds + sid] +
                  (int64_t)h[(4 + 2 * c) * kHistIds + sid];
      mg[sid >> 1] += v;
    }
  }
}

}  // namespace

int compress_device(const void* dsrc, int dtype, int64_t R, int64_t C, double t, int S_req, hipStream_t st,
                    std::vector<uint8_t>* out, Distortion* dist) {
  if (!dsrc || !out) return fail(EP_E_ARG, "null pointer");
  if (dtype < EP_BF16 || dtype > EP_INT8) return fail(EP_E_DTYPE, "unsupported dtype");
  if (R < 1 || C < 1) return fail(EP_E_ARG, "rows and cols must be >= 1");
  if (R > 0xFFFFFFFFll || C > 0xFFFFFFFFll) return fail(EP_E_ARG, "rows/cols exceed 2^32-1");
  if (!std::isfinite(t) || t < 0.001 || t > 11.0)
    return fail(EP_E_RANGE, "target_bpp must be finite and in [0.001, 11]");
  if ((dtype == EP_FP8_E4M3FN || dtype == EP_INT8) && t > 8.0)
    return fail(EP_E_RANGE, "target_bpp above 8 for an 8-bit container");
  if (S_req != 0 && S_req != 1 && S_req != 2 && S_req != 4 && S_req != 8 && S_req != 16 &&
      S_req != 32 && S_req != 64)
    return fail(EP_E_ARG, "chains_per_tile must be 0 or a power of two <= 64");
  const int64_t G = (C + 7) / 8;
  const int64_t N = R * C;
  const int64_t n_groups = R * G;
  int rc;
  if ((rc = check_gpu_pointer(dsrc, "source"))) return rc;
  auto hc = [&](hipError_t e, const char* what) { return hip_check((int)e, what); };

  // ---- row statistics
  DevBuf d_sb, d_s, d_am, d_flags;
  if ((rc = dalloc(d_sb, 2 * R)) || (rc = dalloc(d_s, 4 * R)) || (rc = dalloc(d_am, 8 * R)) ||
      (rc = dalloc(d_flags, 16)))
    return rc;
  if ((rc = hc(hipMemsetAsync(d_flags.p, 0, 4, st), "memset"))) return rc;
  const int esz = dtype == EP_FP32 ? 4 : (dtype == EP_FP8_E4M3FN || dtype == EP_INT8 ? 1 : 2);
  const bool tiled = (C * esz) % 16 == 0 && (reinterpret_cast<uintptr_t>(dsrc) & 15) == 0;
  const dim3 tgrid((unsigned)((R + 63) / 64)), tblock(64);
  if (tiled) {
    auto launch_stats = [&](auto kern) {
      hipLaunchKernelGGL(kern, tgrid, tblock, 0, st, dsrc, R, C, d_sb.as<uint16_t>(), d_s.as<float>(),
                         d_am.as<double>(), d_flags.as<uint32_t>());
    };
    switch (dtype) {
      case EP_BF16: launch_stats(row_stats_tiled_kernel<EP_BF16>); break;
      case EP_FP16: launch_stats(row_stats_tiled_kernel<EP_FP16>); break;
      case EP_FP32: launch_stats(row_stats_tiled_kernel<EP_FP32>); break;
      case EP_FP8_E4M3FN: launch_stats(row_stats_tiled_kernel<EP_FP8_E4M3FN>); break;
      default: launch_stats(row_stats_tiled_kernel<EP_INT8>); break;
    }
  } else {
    hipLaunchKernelGGL(row_stats_kernel, dim3((unsigned)((R + 127) / 128)), dim3(128), 0, st, dsrc, dtype, R, C,
                       d_sb.as<uint16_t>(), d_s.as<float>(), d_am.as<double>(), d_flags.as<uint32_t>());
  }
  std::vector<uint16_t> s_bits((size_t)R);
  std::vector<float> s((size_t)R);
  std::vector<double> amax((size_t)R);
  uint32_t flags = 0;
  if ((rc = hc(hipMemcpyAsync(s_bits.data(), d_sb.p, 2 * R, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipMemcpyAsync(s.data(), d_s.p, 4 * R, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipMemcpyAsync(amax.data(), d_am.p, 8 * R, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipMemcpyAsync(&flags, d_flags.p, 4, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipStreamSynchronize(st), "sync")))
    return rc;
  if (flags & 1u) return fail(EP_E_NONFINITE, "input holds NaN or Inf");
  if (flags & 2u) return fail(EP_E_RANGE, "a nonzero row has an RMS below the BF16 normal range");

  // ---- sample rows and the resolution search
  std::vector<int64_t> rows;
  const int64_t kSample = 1 << 18;
  if (N <= kSample) {
    for (int64_t r = 0; r < R; ++r) rows.push_back(r);
  } else {
    const int64_t ks = N / kSample;
    for (int64_t r = 0; r < R; r += ks) rows.push_back(r);
  }
  const int64_t n_sample = (int64_t)rows.size() * C;
  const int64_t T = (int64_t)std::ceil(t * 65536.0 * (double)n_sample);
  int jmin = 999;
  for (int j = -126; j <= 4; ++j)
    if (resolution_admissible(s.data(), amax.data(), R, std::ldexp(1.0f, j))) {
      jmin = j;
      break;
    }
  if (jmin == 999) return fail(EP_E_RANGE, "no admissible resolution");
  const int64_t sg = (int64_t)rows.size() * G;
  DevBuf d_rows, d_us, d_cnt, d_u, d_se, d_sw;
  if ((rc = dalloc(d_rows, 8 * rows.size())) || (rc = dalloc(d_us, 32 * (size_t)sg)) ||
      (rc = dalloc(d_cnt, 8 * (size_t)(8 + kHistBins + 1))))
    return rc;
  if ((rc = hc(hipMemcpyAsync(d_rows.p, rows.data(), 8 * rows.size(), hipMemcpyHostToDevice, st), "copy"))) return rc;
  unsigned long long* d_ge = d_cnt.as<unsigned long long>();
  unsigned long long* d_hist = d_ge + 8;
  unsigned long long* d_raw = d_hist + kHistBins;
  std::vector<unsigned long long> hist((size_t)kHistBins + 1);
  HostBuf cnt_host;   // pinned: the probes' counts come back by DMA
  if ((rc = halloc(cnt_host, 8 * (size_t)(8 + kHistBins + 1)))) return rc;
  const int32_t* lq = log2q_table();
  int err = EP_OK;

  // k from the magnitude counts, then the (context, id) counts
  auto count = [&](const int64_t* drows, int64_t nrows, int32_t* du, float delta, int* k_out) -> int {
    int e;
    if ((e = hc(hipMemsetAsync(d_cnt.p, 0, 8 * (size_t)(8 + kHistBins + 1), st), "memset"))) return e;
    const int64_t ng = nrows * G;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, st, dsrc, dtype, C, G,
                       drows, nrows, d_s.as<float>(), delta, du, d_ge);
    // the bucket k is picked on the device; one copy back per probe (counts, k, histogram)
    const unsigned nb = (unsigned)std::min<int64_t>(1024, (ng + 255) / 256);
    hipLaunchKernelGGL(histogram_kernel, dim3(nb), dim3(256), 0, st, du, ng, -1, d_ge, d_hist, d_raw, d_ge + 7);
    if ((e = hc(hipMemcpyAsync(cnt_host.p, d_cnt.p, 8 * (size_t)(8 + kHistBins + 1), hipMemcpyDeviceToHost, st),
                "copy")) ||
        (e = hc(hipStreamSynchronize(st), "sync")))
      return e;
    const unsigned long long* ch = (const unsigned long long*)cnt_host.p;
    std::copy(ch + 8, ch + 8 + kHistBins + 1, hist.begin());
    *k_out = (int)ch[7];
    return EP_OK;
  };
  auto estimate_at = [&](uint32_t bits) -> Estimate {
    float delta;
    std::memcpy(&delta, &bits, 4);
    int k = 3;
    const int e = count(d_rows.as<int64_t>(), (int64_t)rows.size(), d_us.as<int32_t>(), delta, &k);
    if (e) {
      err = e;
      return {0, k};
    }
    int64_t cc[2];
    std::vector<int64_t> mag0, mag1;
    model_counts(hist, k, cc, mag0, mag1);
    Model m = build_model(k, cc, mag0.data(), mag1.data());
    int64_t est = 65536 * (int64_t)hist[kHistBins];
    for (int ctx = 0; ctx < kNumCtx; ++ctx)
      for (int id = 0; id < kHistIds; ++id) {
        const int64_t c = (int64_t)hist[(size_t)(ctx * kHistIds + id)];
        if (c) est += c * ((int64_t)m.P * 65536 - lq[m.F[ctx][id]]);
      }
    return {est, k};
  };
  uint32_t dbits;
  int k;
  select_resolution(t, T, jmin, estimate_at, &dbits, &k);
  if (err) return err;
  float delta;
  std::memcpy(&delta, &dbits, 4);

  // ---- all rows
  if ((rc = dalloc(d_u, 32 * (size_t)n_groups))) return rc;
  int k_all = 3;
  if ((rc = count(nullptr, R, d_u.as<int32_t>(), delta, &k_all))) return rc;
  // (k stays the sampled one; the counts are redone with it when the full data picks another)
  if (k_all != k) {
    const unsigned nb = (unsigned)std::min<int64_t>(1024, (n_groups + 255) / 256);
    if ((rc = hc(hipMemsetAsync(d_hist, 0, 8 * (size_t)(kHistBins + 1), st), "memset"))) return rc;
    hipLaunchKernelGGL(histogram_kernel, dim3(nb), dim3(256), 0, st, d_u.as<int32_t>(), n_groups, k, d_ge, d_hist,
                       d_raw, d_ge + 7);
    if ((rc = hc(hipMemcpyAsync(hist.data(), d_hist, 8 * hist.size(), hipMemcpyDeviceToHost, st), "copy")) ||
        (rc = hc(hipStreamSynchronize(st), "sync")))
      return rc;
  }
  const unsigned long long* ge_all = (const unsigned long long*)cnt_host.p;   // the full pass's counts
  const bool any_esc = ge_all[k - 3] > 0;
  int64_t cc[2];
  std::vector<int64_t> mag0, mag1;
  model_counts(hist, k, cc, mag0, mag1);
  Model m = build_model(k, cc, mag0.data(), mag1.data());

  // ---- distortion and clamping
  if ((rc = dalloc(d_se, 8 * R)) || (rc = dalloc(d_sw, 8 * R))) return rc;
  if ((rc = hc(hipMemsetAsync(d_flags.p, 0, 4, st), "memset"))) return rc;
  const double cmax = dtype == EP_BF16 ? (double)__builtin_bit_cast(float, 0x7F7F0000u)
                                       : (dtype == EP_FP16 ? 65504.0 : (dtype == EP_FP8_E4M3FN ? 448.0 : 127.0));
  if (tiled) {
    auto launch_err = [&](auto kern) {
      hipLaunchKernelGGL(kern, tgrid, tblock, 0, st, dsrc, R, C, G, d_s.as<float>(), delta, d_u.as<int32_t>(), cmax,
                         d_se.as<double>(), d_sw.as<double>(), d_flags.as<uint32_t>());
    };
    switch (dtype) {
      case EP_BF16: launch_err(row_error_tiled_kernel<EP_BF16>); break;
      case EP_FP16: launch_err(row_error_tiled_kernel<EP_FP16>); break;
      case EP_FP32: launch_err(row_error_tiled_kernel<EP_FP32>); break;
      case EP_FP8_E4M3FN: launch_err(row_error_tiled_kernel<EP_FP8_E4M3FN>); break;
      default: launch_err(row_error_tiled_kernel<EP_INT8>); break;
    }
  } else {
    hipLaunchKernelGGL(row_error_kernel, dim3((unsigned)((R + 127) / 128)), dim3(128), 0, st, dsrc, dtype, R, C, G,
                       d_s.as<float>(), delta, d_u.as<int32_t>(), cmax, d_se.as<double>(), d_sw.as<double>(),
                       d_flags.as<uint32_t>());
  }
  std::vector<double> se((size_t)R), sw((size_t)R);
  uint32_t sat = 0;
  if ((rc = hc(hipMemcpyAsync(se.data(), d_se.p, 8 * R, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipMemcpyAsync(sw.data(), d_sw.p, 8 * R, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipMemcpyAsync(&sat, d_flags.p, 4, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipStreamSynchronize(st), "sync")))
    return rc;
  if (dist) {
    dist->sq_err = 0.0;
    dist->sq_ref = 0.0;
    for (int64_t r = 0; r < R; ++r) {
      dist->sq_err += se[(size_t)r];
      dist->sq_ref += sw[(size_t)r];
    }
  }

  // ---- chains, schedule, layout
  const int S = S_req ? S_req : (N >= (1ll << 22) ? 8 : 1);
  const int log2S = __builtin_ctz((unsigned)S);
  const int64_t n_tiles = std::max<int64_t>(1, (n_groups + kTileGroups - 1) / kTileGroups);
  const int64_t n_chains = n_tiles * S;
  const int steps = kTileGroups / S;
  const int max_words = 24 * steps + 2;
  const int max_full = max_words / 8 + 1;
  DevBuf d_tab, d_words, d_cons, d_len, d_state, d_rank, d_dst, d_stream;
  if ((rc = dalloc(d_tab, 8 * (size_t)kHistBins)) || (rc = dalloc(d_words, 2 * (size_t)n_chains * max_words)) ||
      (rc = dalloc(d_cons, (size_t)n_chains * steps)) ||
      (rc = dalloc(d_len, 4 * (size_t)n_chains)) || (rc = dalloc(d_state, 4 * (size_t)n_chains)) ||
      (rc = dalloc(d_rank, 2 * (size_t)n_chains * max_full)) || (rc = dalloc(d_dst, 16 * (size_t)n_chains)))
    return rc;
  {
    std::vector<int32_t> tab((size_t)2 * kHistBins, 0);
    for (int ctx = 0; ctx < kNumCtx; ++ctx)
      for (int id = 0; id < kHistIds; ++id) {
        tab[(size_t)(ctx * kHistIds + id)] = m.F[ctx][id];
        tab[(size_t)(kHistBins + ctx * kHistIds + id)] = m.CUM[ctx][id];
      }
    if ((rc = hc(hipMemcpyAsync(d_tab.p, tab.data(), 4 * tab.size(), hipMemcpyHostToDevice, st), "copy"))) return rc;
    if ((rc = hc(hipStreamSynchronize(st), "sync"))) return rc;
  }
  if ((rc = hc(hipMemsetAsync(d_rank.p, 0, 2 * (size_t)n_chains * max_full, st), "memset"))) return rc;
  hipLaunchKernelGGL(encode_chains_kernel, dim3((unsigned)((n_chains + 127) / 128)), dim3(128), 0, st,
                     d_u.as<int32_t>(), n_groups, S, log2S, n_chains, k, d_tab.as<int32_t>(),
                     d_tab.as<int32_t>() + kHistBins, max_words, steps, d_words.as<uint16_t>(), d_cons.as<uint8_t>(),
                     d_len.as<uint32_t>(), d_state.as<uint32_t>());
  hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)((n_tiles + 63) / 64)), dim3(64), 0, st, d_len.as<uint32_t>(),
                     d_cons.as<uint8_t>(), n_groups, S, n_tiles, steps, max_full, any_esc, d_rank.as<uint16_t>());
  std::vector<uint32_t> lens((size_t)n_chains), states((size_t)n_chains);
  if ((rc = hc(hipMemcpyAsync(lens.data(), d_len.p, 4 * (size_t)n_chains, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipMemcpyAsync(states.data(), d_state.p, 4 * (size_t)n_chains, hipMemcpyDeviceToHost, st), "copy")) ||
      (rc = hc(hipStreamSynchronize(st), "sync")))
    return rc;

  // block areas: [tile main areas][tails][pad to 8 words]
  const int64_t n_blocks = (n_chains + kBlockChains - 1) / kBlockChains;
  const int64_t max_full_field = S >= 8 ? 0xFF : 0xFFFF;
  std::vector<uint64_t> block_off((size_t)n_blocks + 1, 0);
  std::vector<int64_t> dst((size_t)2 * n_chains);
  for (int64_t bk = 0; bk < n_blocks; ++bk) {
    const int64_t c0 = bk * kBlockChains, c1 = std::min(n_chains, c0 + kBlockChains);
    uint64_t words = 0, full_words = 0;
    for (int64_t c = c0; c < c1; ++c) {
      if ((int64_t)(lens[c] / 8) > max_full_field) return fail(EP_E_ARG, "chain longer than the chunk count field");
      words += lens[c];
      full_words += 8 * (lens[c] / 8);
    }
    block_off[bk + 1] = block_off[bk] + (words + 7) / 8;
    const int64_t base = 8 * (int64_t)block_off[bk];
    int64_t tile_main = 0, tails = (int64_t)full_words;
    for (int64_t t0 = c0; t0 < c1; t0 += S) {
      int64_t tile_words = 0;
      for (int64_t c = t0; c < t0 + S; ++c) {
        dst[(size_t)c] = base + tile_main;
        tile_words += 8 * (lens[c] / 8);
      }
      tile_main += tile_words;
    }
    for (int64_t c = c0; c < c1; ++c) {
      dst[(size_t)(n_chains + c)] = base + tails;
      tails += lens[c] % 8;
    }
  }
  const uint64_t n_words = 8 * block_off[n_blocks];
  if (block_off[n_blocks] > 0xFFFFFFFFull) return fail(EP_E_ARG, "stream too long for the block offsets");
  if ((rc = dalloc(d_stream, 2 * (size_t)n_words + 16))) return rc;
  if ((rc = hc(hipMemsetAsync(d_stream.p, 0, 2 * (size_t)n_words + 16, st), "memset")) ||
      (rc = hc(hipMemcpyAsync(d_dst.p, dst.data(), 8 * dst.size(), hipMemcpyHostToDevice, st), "copy")))
    return rc;
  hipLaunchKernelGGL(layout_kernel, dim3((unsigned)((n_chains + 127) / 128)), dim3(128), 0, st,
                     d_words.as<uint16_t>(), max_words, d_len.as<uint32_t>(), d_rank.as<uint16_t>(), max_full,
                     d_dst.as<int64_t>(), d_dst.as<int64_t>() + n_chains, n_chains, d_stream.as<uint16_t>(),
                     (int64_t)n_words);

  // ---- the blob: header | row scales | model | chain area
  const std::vector<uint8_t> mbytes = m.to_bytes();
  const size_t fw = S >= 8 ? 1 : 2;
  const size_t n_nib = (size_t)((n_chains + 1) / 2);
  const size_t off_area = kHeaderBytes + 2 * (size_t)R + mbytes.size();
  const size_t off_full = off_area + 4 * (size_t)n_blocks;
  const size_t off_nib = off_full + fw * (size_t)n_chains;
  const size_t off_st = off_nib + n_nib;
  const size_t off_stream = off_st + 4 * (size_t)n_chains;
  std::vector<uint8_t>& b = *out;
  try {
    b.assign(off_stream + 2 * (size_t)n_words, 0);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  if ((rc = hc(hipMemcpyAsync(&b[off_stream], d_stream.p, 2 * (size_t)n_words, hipMemcpyDeviceToHost, st), "copy")))
    return rc;
  std::memcpy(&b[0], "EPK1", 4);
  put16(b, 4, 3);
  b[6] = (uint8_t)dtype;
  b[7] = (uint8_t)precision(k);
  b[8] = (uint8_t)S;
  b[9] = (uint8_t)k;
  b[10] = (uint8_t)((any_esc ? kFlagEsc : 0) | (sat ? kFlagSat : 0));
  b[11] = 12;
  put32(b, 12, (uint32_t)R);
  put32(b, 16, (uint32_t)C);
  put32(b, 20, dbits);
  put32(b, 24, (uint32_t)n_tiles);
  put32(b, 28, (uint32_t)n_blocks);
  put64(b, 32, n_words);
  put32(b, 40, (uint32_t)mbytes.size());
  put32(b, 44, 0);
  size_t off = kHeaderBytes;
  for (int64_t r = 0; r < R; ++r, off += 2) put16(b, off, s_bits[(size_t)r]);
  std::memcpy(&b[off], mbytes.data(), mbytes.size());
  for (int64_t bk = 0; bk < n_blocks; ++bk) put32(b, off_area + 4 * (size_t)bk, (uint32_t)block_off[bk]);
  for (int64_t c = 0; c < n_chains; ++c) {
    const uint32_t len = lens[(size_t)c];
    if (fw == 1) b[off_full + (size_t)c] = (uint8_t)(len / 8);
    else put16(b, off_full + 2 * (size_t)c, (uint16_t)(len / 8));
    b[off_nib + (size_t)(c / 2)] |= (uint8_t)((len % 8) << (4 * (c & 1)));
    put32(b, off_st + 4 * (size_t)c, states[(size_t)c]);
  }
  if ((rc = hc(hipStreamSynchronize(st), "sync"))) return rc;
  return EP_OK;
}

}  // namespace ep

using namespace ep;

extern "C" {

int ep_compress_device(const void* dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                       int chains_per_tile, ep_stream stream, ep_blob** out) {
  set_error("");
  if (!out) return fail(EP_E_ARG, "null output pointer");
  *out = nullptr;
  std::vector<uint8_t> bytes;
  Distortion dist;
  int rc = ep::compress_device(dev_src, dtype, rows, cols, target_bpp, chains_per_tile, (hipStream_t)stream, &bytes,
                               &dist);
  if (rc) return rc;
  ep_blob* blob = new (std::nothrow) ep_blob();
  if (!blob) return fail(EP_E_NOMEM, "out of host memory");
  rc = parse_blob(std::move(bytes), &blob->b);
  if (rc) {
    delete blob;
    return rc;
  }
  blob->b.dist = dist;
  *out = blob;
  return EP_OK;
}

// n matrices on up to four host threads, each with a stream of its own (the encoder's
// host steps and its small per-probe round trips overlap across matrices).  Every blob
// equals ep_compress_device's for that matrix.
int ep_compress_device_batch(const void* const* dev_src, const int64_t* rows, const int64_t* cols, int n, int dtype,
                             double target_bpp, int chains_per_tile, ep_stream stream, ep_blob** out) {
  set_error("");
  if (n < 0 || (n > 0 && (!dev_src || !rows || !cols || !out))) return fail(EP_E_ARG, "null pointer or negative count");
  for (int i = 0; i < n; ++i) out[i] = nullptr;
  if (n == 0) return EP_OK;
  int dev = 0;
  int rc = hip_check((int)hipGetDevice(&dev), "get device");
  if (rc) return rc;
  // the inputs are ready once the work already queued on `stream` is done
  if ((rc = hip_check((int)hipStreamSynchronize((hipStream_t)stream), "stream sync"))) return rc;
  const int nw = std::min(n, 4);
  std::vector<int> codes(n, EP_OK);
  std::vector<std::string> msgs(n);
  std::atomic<int> next{0};
  auto work = [&]() {
    if (hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) {
      (void)hipGetLastError();
      st = nullptr;
    }
    t_cache_on = true;
    for (int i = next++; i < n; i = next++) {
      if (!st) {
        codes[i] = EP_E_DEVICE;
        msgs[i] = "stream creation failed";
        continue;
      }
      codes[i] = ep_compress_device(dev_src[i], dtype, rows[i], cols[i], target_bpp, chains_per_tile, (ep_stream)st,
                                    &out[i]);
      if (codes[i]) msgs[i] = ep_last_error();
    }
    cache_release();
    if (st) (void)hipStreamDestroy(st);
  };
  std::vector<std::thread> pool;
  for (int w = 1; w < nw; ++w) pool.emplace_back(work);
  work();
  for (auto& t : pool) t.join();
  for (int i = 0; i < n; ++i)
    if (codes[i] != EP_OK || !out[i]) {
      const int code = codes[i] != EP_OK ? codes[i] : EP_E_DEVICE;
      const std::string msg = "matrix " + std::to_string(i) + ": " + (msgs[i].empty() ? "not compressed" : msgs[i]);
      for (int k = 0; k < n; ++k) {
        ep_blob_free(out[k]);
        out[k] = nullptr;
      }
      return fail(code, msg);
    }
  return EP_OK;
}

}  // extern "C"
