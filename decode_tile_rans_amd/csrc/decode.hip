// Fused tile-rANS decode for gfx950 (MI355X).
//
// [SUM]: symbol decode, algebraic inverse-lattice reconstruction and per-row rescale
// run fused on the GPU, with no intermediate symbol tensor and no reconstruction
// codebook.  [ABS]: tiles are independently decodable; containers BF16/FP16/FP8/INT8.
//
// Work mapping (MI355X-first, not the pages' H20 design):
//   * one wavefront = one block of 64 rANS chains, one chain per lane (64/S tiles), or two
//     blocks with two chains per lane; a wave-wide prefix sum over the block's stored
//     chunk counts and tail lengths gives every chain its stream positions, so the stored
//     per-chain metadata stays at one byte of chunk count and half a byte of tail length
//     (plus the chain's initial state) and one u32 offset per block;
//   * a workgroup of W waves stages the 7 decode tables into LDS once (56 KB: 1024 slots
//     of two-word entries, or 1024 / 2048 slots of packed words, by table precision and
//     escapes); every chain keeps a 32-word ring of stream words in LDS, fed by 16-byte
//     loads in the order the stream stores them, issued two groups ahead of use;
//   * per coordinate: one LDS table read, x = f (x >> P) + bias (24-bit mad), a
//     16-bit renormalisation from a prefetched ring word, the doubled coordinate taken
//     straight from the table entry (escapes: bypass bits, replayed on a careful path),
//     h_r * u in fp32, container cast, one 16-byte store per 8-coordinate group (BF16);
//   * nothing but the final weights is written to HBM.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "ep_internal.h"

namespace ep {

int hip_check(int err, const char* what) {
  if (err != hipSuccess) return fail(EP_E_DEVICE, std::string(what) + ": " + hipGetErrorString((hipError_t)err));
  return EP_OK;
}

namespace {

enum OutKind { OUT_BF16 = 0, OUT_BF16_SAT = 1, OUT_FP16 = 2, OUT_FP32 = 3, OUT_FP8 = 4, OUT_INT8 = 5, OUT_COORDS = 6,
               OUT_BYTES = 7 /* TileANS: the decoded symbols are the tensor's bytes */,
               // fused matrix-vector product with 1, 2, 4 or 8 activation rows: the BF16
               // weights are multiplied into per-chain partial sums and never stored
               OUT_MV1 = 8, OUT_MV2 = 9, OUT_MV4 = 10, OUT_MV8 = 11,
               // BF16 stored through the caches (a GEMM reads the weights right after)
               OUT_BF16_L2 = 12,
               // fused prefill product: each K slab of BF16 weights goes to an LDS operand
               // tile that MFMAs multiply by up to 128 (MMA1) or 256 (MMA2) activation rows;
               // 4096 columns (one tile a row), or 8192 (two tiles a row: MMA1X2, MMA2X2)
               OUT_MMA1 = 13, OUT_MMA2 = 14, OUT_MMA1X2 = 15, OUT_MMA2X2 = 16 };
template <int OUT>
constexpr int mv_tokens() {
  return (OUT >= OUT_MV1 && OUT <= OUT_MV8) ? 1 << (OUT - OUT_MV1) : 0;
}
// 16-row activation blocks per wave of the fused prefill product (0: another output)
template <int OUT>
constexpr int mma_blocks() {
  return (OUT == OUT_MMA1 || OUT == OUT_MMA1X2) ? 1 : (OUT == OUT_MMA2 || OUT == OUT_MMA2X2) ? 2 : 0;
}
// tiles per row of W in the fused prefill product (4096 columns a tile)
template <int OUT>
constexpr int mma_tiles_per_row() {
  return (OUT == OUT_MMA1X2 || OUT == OUT_MMA2X2) ? 2 : 1;
}
template <int OUT>
constexpr int out_elem_bytes() {
  return (OUT == OUT_FP32 || OUT == OUT_COORDS) ? 4 : ((OUT == OUT_FP8 || OUT == OUT_INT8 || OUT == OUT_BYTES) ? 1 : 2);
}

constexpr int kTabBytes = kNumCtx * kMMax * 4;   // 57344 B: LDS region of any table layout
// packed table entry: f (bits 0..10) | bias (11..21) | value (22..30) | escape (31);
// value = doubled coordinate u (signed 9 bit) or, for escapes, c | neg<<1 | top2<<2 | (e-k)<<4
constexpr int kValShift = 22;

struct DecJob {
  const uint16_t* stream;
  // the blob's chain area as stored: per block the start of its area (in 8-word chunks),
  // per chain its full chunks (u8 at S >= 8, else u16), its tail words (4 bits) and the
  // initial decoder state
  const uint32_t* boff;
  const void* full;
  const uint8_t* nib;
  const uint32_t* states;
  const float* hr;
  const uint32_t* tab;
  uint32_t* err;
  void* out;
  int64_t n_groups, G, C, n_chains, n_blocks;
  int64_t chain_lo, chain_hi;
  int64_t block_lo;          // first block decoded by workgroup 0 of this job
  int64_t wg_begin;          // batch: first workgroup of this job
  uint32_t n_words;
  int log2S, k, c8;
  uint32_t s_div_g, s_mod_g;   // S = s_div_g * G + s_mod_g (group stride in rows / columns)
  uint32_t R;
  uint32_t ctx_mask;           // TileANS: byte contexts - 1 (symbol i of a group uses i & ctx_mask)
  uint32_t tab_words;          // table words to stage
  // fused matrix-vector product (OUT_MV*): activations X (mv_T rows of C BF16), partial
  // sums out[(chain * mv_slots + row - first row of the chain) * tokens + t]
  const uint16_t* mv_x;
  uint32_t mv_T, mv_slots, mv_sat;
  uint32_t mv_direct;          // rows of whole tiles: the product is summed in the wave, out = y
  uint32_t mv_lanes;           // lanes of one row (S per tile) when mv_direct
  const uint16_t* bias;        // fused prefill product: BF16 bias of the R outputs, or null
  uint32_t big_h;              // some |128 h_r| overflows float: reconstruct as h u
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

// Four values to E4M3FN bytes (value i in byte i).  HW: clamp to +-448 (v_med3), then
// the conversion instruction (round to nearest even, OCP E4M3FN on gfx950), two values
// per instruction; otherwise the bit manipulation above, one value at a time.
template <bool HW>
__device__ inline uint32_t pack_fp8x4(float a, float b, float c, float d) {
  if constexpr (HW) {
    a = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
    b = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
    c = __builtin_amdgcn_fmed3f(c, -448.f, 448.f);
    d = __builtin_amdgcn_fmed3f(d, -448.f, 448.f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
  } else {
    return f32_to_e4m3fn(a) | (f32_to_e4m3fn(b) << 8) | (f32_to_e4m3fn(c) << 16) | (f32_to_e4m3fn(d) << 24);
  }
}
constexpr bool kFp8Hw = true;    // the decoder's FP8 cast

__device__ inline uint32_t f32_to_i8(float v) {
  float r = fminf(fmaxf(rintf(v), -128.f), 127.f);
  return (uint32_t)((int32_t)r) & 0xFFu;
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Write one group: v = reconstructed fp32 weights, u = doubled coordinates (COORDS).
template <int OUT>
__device__ inline void store_group(void* out, int64_t base, const float* vin, const int32_t* u, bool full,
                                   int64_t nvalid) {
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (OUT != OUT_BYTES && OUT != OUT_COORDS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = vin[i];
  }
  if (OUT == OUT_BF16_SAT) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(v[i], -3.38953139e38f), 3.38953139e38f);
  }
  if (OUT == OUT_BF16 || OUT == OUT_BF16_L2 || OUT == OUT_BF16_SAT || OUT == OUT_FP16) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (OUT == OUT_FP16) {
        p[i] = pack_f16x2(v[2 * i], v[2 * i + 1]);
      } else {
        f32x2 fv = {v[2 * i], v[2 * i + 1]};
        p[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(fv, bf16x2));
      }
    }
    uint16_t* o = (uint16_t*)out + base;
    if (full) {
      // streaming store: the weights are written once, so they should not evict the
      // compressed stream's lines from L2 (the lanes re-read those lines chunk by chunk);
      // weights a GEMM reads next are stored through the caches, where it finds them
      u32x4 pv = {p[0], p[1], p[2], p[3]};
      if constexpr (OUT == OUT_BF16_L2) *(u32x4*)o = pv;
      else __builtin_nontemporal_store(pv, (u32x4*)o);
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = (uint16_t)(p[i >> 1] >> ((i & 1) * 16));
    }
  } else if (OUT == OUT_FP32) {
    float* o = (float*)out + base;
    if (full) {
      typedef __attribute__((ext_vector_type(4))) float f32x4;
      f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
      __builtin_nontemporal_store(a, (f32x4*)o);
      __builtin_nontemporal_store(b, (f32x4*)(o + 4));
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = v[i];
    }
  } else if (OUT == OUT_FP8 || OUT == OUT_INT8) {
    uint32_t lo = 0, hi = 0;
    if constexpr (OUT == OUT_FP8) {
      lo = pack_fp8x4<kFp8Hw>(v[0], v[1], v[2], v[3]);
      hi = pack_fp8x4<kFp8Hw>(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= f32_to_i8(v[i]) << (8 * i);
        hi |= f32_to_i8(v[i + 4]) << (8 * i);
      }
    }
    uint8_t* o = (uint8_t*)out + base;
    if (full) {
      typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
      u32x2 pv = {lo, hi};
      __builtin_nontemporal_store(pv, (u32x2*)o);
    } else {
      for (int i = 0; i < nvalid; ++i) o[i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
    }
  } else if (OUT == OUT_BYTES) {
    // (u holds the eight bytes, one per entry's top byte)
    const uint32_t lo = ((uint32_t)u[0] >> 24) | (((uint32_t)u[1] >> 24) << 8) | (((uint32_t)u[2] >> 24) << 16) |
                        ((uint32_t)u[3] & 0xFF000000u);
    const uint32_t hi = ((uint32_t)u[4] >> 24) | (((uint32_t)u[5] >> 24) << 8) | (((uint32_t)u[6] >> 24) << 16) |
                        ((uint32_t)u[7] & 0xFF000000u);
    uint8_t* o = (uint8_t*)out + base;
    if (full) {
      typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
      u32x2 pv = {lo, hi};
      __builtin_nontemporal_store(pv, (u32x2*)o);
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
constexpr int kRingWords = 32;                   // per-chain LDS ring (16-bit words)
constexpr int kChunkWords = 8;                   // one 16-byte stream load
constexpr int kMirrorBytes = 32;                 // copy of ring bytes 0..31 after the ring
// LDS bytes per chain: one chain per lane keeps a mirror after its ring (96 B), two chains
// per lane do without (64 B; their reads wrap), so that twice the chains fit a CU
template <int ILP>
constexpr int ring_bytes() {
  return ILP == 1 ? kRingWords * 2 + kMirrorBytes : kRingWords * 2;
}
constexpr int kMaxWaves = 16;
constexpr int kHrPad = 128;                      // zero row scales after the last row (prefetch slack)
static_assert(kRingWords - kChunkWords >= 17, "ring too small for two groups plus a chunk");

// Job descriptors travel by value in the kernel arguments (no per-launch copy).
struct DecBatch {
  DecJob j[kMaxBatch];
  int n;
  int64_t bpw;   // blocks per workgroup
};

// Entry layouts (chosen per blob when its tables are expanded):
//   wide   (K >= 64): f 0..10 | bias 11..21 | u (9 bit) 22..30 | escape 31
//   narrow (K <= 32): f 0..10 | bias 11..21 | c 22 | escape 23 | u + 128 24..31
// An escape (bucket) symbol holds instead the coset c, the sign, n2 = e - 2 (the number of
// magnitude bits below the leading three; e = floor(log2 m)) and the two bits top2 after
// the leading one:  wide  c 22 | neg 23 | n2 24..28 | top2 29..30 | 1 31  (so that bits
//                               29..31 are the leading three bits 1 top2 themselves)
//                   narrow c 22 | 1 23 | n2 24..28 | top2 29..30 | neg 31
// In both, bit 22 is the coset of a FIRST symbol.  The parity of floor(u/2) (bit 1 of u)
// sits at bit 23 (wide) or 25 (narrow).
template <bool NARROW>
struct EntryLayout {
  static constexpr uint32_t kEsc = NARROW ? (1u << 23) : (1u << 31);
  static constexpr int kPar = NARROW ? 25 : 23;
  __device__ static int32_t u_of(uint32_t e) {
    return NARROW ? (int32_t)(e >> 24) - 128 : __builtin_amdgcn_sbfe((int32_t)e, 22, 9);
  }
  // fl32(h * u) for a direct symbol: narrow uses the exact fma(u + 128, h, -128 h)
  __device__ static float w_of(uint32_t e, float h, float nh128) {
    return NARROW ? __builtin_fmaf((float)(e >> 24), h, nh128) : h * (float)u_of(e);
  }
  // escape info: c, the sign as 0 / -1, the leading three magnitude bits 4 + top2, n2
  __device__ static void esc_info(uint32_t e, uint32_t& c, int32_t& sgn, uint32_t& lead3, uint32_t& n2) {
    c = (e >> 22) & 1u;
    n2 = (e >> 24) & 31u;
    if (NARROW) {
      sgn = (int32_t)e >> 31;
      lead3 = ((e >> 29) & 3u) | 4u;
    } else {
      sgn = __builtin_amdgcn_sbfe((int32_t)e, 23, 1);
      lead3 = e >> 29;
    }
  }
};

// ---- table geometry of a kernel variant
// Lossy blobs with escape threshold K <= 32 (narrow entries) use M = 1024 slots per table,
// K >= 64 (wide entries) and TileANS byte tables 2048.  Narrow blobs without escapes get
// split entries, two words per slot (build_split_tables); the others one packed word.
// In LDS the 7 tables sit in the order FREE[0], FIRST, FREE[1], LAST[0][0..1],
// LAST[1][0..1], one table every kTable bytes, so a LAST table is the FREE table of the
// same coset plus 3 kTable plus kTable for parity 1.
typedef __attribute__((ext_vector_type(2))) uint32_t EntPair;   // a split entry: value word, bias

template <int OUT, bool ESC, bool NARROW>
struct Geo {
  static constexpr bool kSplit = NARROW && !ESC && OUT != OUT_BYTES;
  static constexpr int kP = (NARROW && OUT != OUT_BYTES) ? 10 : 11;
  static constexpr uint32_t kMask = (1u << kP) - 1u;
  static constexpr int kTableLog2 = kP + (kSplit ? 3 : 2);          // bytes per table, log2
  static constexpr uint32_t kTable = 1u << kTableLog2;
  static constexpr uint32_t kFirstOff = kTable;
  static constexpr uint32_t kLastOff = 3u * kTable;
  using Ent = typename std::conditional<kSplit, EntPair, uint32_t>::type;
  // the entry word holding the value (coset, parity and u + 128 or the wide value)
  __device__ static uint32_t lo(Ent e) {
    if constexpr (kSplit) return e.x;
    else return e;
  }
  // FREE table of a FIRST entry's coset: 2 kTable c, the coset being bit 24 of a split
  // entry and bit 22 of a packed one
  __device__ static uint32_t free_base(uint32_t e_first) {
    constexpr int cbit = kSplit ? 24 : 22;
    return (e_first >> (cbit - (kTableLog2 + 1))) & (2u * kTable);
  }
};

// ---- one rANS chain: its state and its stream reader
//
// Stream layout: a block of 64 chains holds, per tile, the tile's 8-word chunks in the
// order its chains request them (positions handed out by a ballot in chain order, the
// tile's cursor advancing by 8 words per chunk), then every chain's last short piece
// (tail).  Each chain keeps its words in a 32-word LDS ring: word i at ring byte
// 2 (i mod 32), so chunk n fills ring bytes 16 (n mod 4) .. +15; chunks 0 and 1 of the
// ring are also written to bytes 64..95 (a mirror), so that a reader may run up to 16
// words past the ring's end without wrapping.  Counters are kept in bytes (2 per word):
// fb = fetched (a chunk in flight included), a2 = consumed.  Between services a chain
// reads through a linear pointer ra (set from a2 at the service, a2 brought up to date
// at the next one; blobs with escapes re-derive it within a group); fetches work on a2.
// Fetches happen only at these sites, exactly as the encoder's schedule assumed:
//   blobs without escapes: prime until 17 ahead; every even group: until 17 ahead,
//   then one round for chains at most 24 ahead (a 16-byte load issued now, written to
//   the ring at the next service);
//   blobs with escapes: prime until 24 ahead; every group: until 24 ahead, then the
//   same round.
// Two escape-free groups consume <= 16 words and one group with escapes <= 24, so the
// chain only reads words already in its ring; it never holds more than 32 words ahead.
struct Chain {
  uint32_t x;        // rANS state
  uint32_t a2;       // 2 x words consumed (behind by the pair's reads until its end)
  uint32_t ra;       // LDS byte address of the next word within a group pair (unwrapped)
  uint32_t d;        // a2 - ra at the pair's start
  uint32_t nw;       // the next word, already read from the ring
  uint32_t rb;       // LDS byte address of the ring (16-byte aligned)
  uint32_t fb;       // 2 x words fetched
  int32_t rem;       // words not fetched yet
  uint32_t cur;      // the tile's main-area cursor (word index; equal on the tile's lanes)
  uint32_t tailp;    // word index of the chain's tail
  uint32_t seg_lo;   // lanes of the chain's tile (ballot mask)
  uint32_t seg_hi;
  uint4 pend;        // chunk in flight
  uint32_t pend_at;  // its ring address
  bool have_pend;
  bool pend_mirror;  // it also goes to the mirror
};

struct StreamRef {
  const uint16_t* w;
  uint32_t last_chunk;   // highest word index a 16-byte load may start at: the stream's
                         // length (the allocation has 256 bytes of slack after it)
};

// three-input xor in one instruction (gfx950 v_bitop3, truth table 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// LDS is addressed with plain 32-bit local addresses (ring and table bases include the
// dynamic LDS base), so a ring address is one and-or and a table address one shift-add.
#define EP_LDS __attribute__((address_space(3)))
__device__ __forceinline__ uint32_t lds_u16(uint32_t a) { return *(const EP_LDS uint16_t*)(uintptr_t)a; }
__device__ __forceinline__ void lds_st128(uint32_t a, uint4 d) {
  const u32x4 v = {d.x, d.y, d.z, d.w};
  *(EP_LDS u32x4*)(uintptr_t)a = v;
}

// (MIR: the ring has its mirror, and ra is an LDS address that may run up to 16 words
// past the ring's end; without it ra counts bytes like a2 and every read wraps)
__device__ __forceinline__ uint32_t ch_word(const Chain& r) { return lds_u16((r.a2 & 62u) + r.rb); }
template <bool MIR>
__device__ __forceinline__ uint32_t ch_at(const Chain& r) {
  if constexpr (MIR) return r.ra;
  else return (r.ra & 62u) + r.rb;
}
template <bool MIR>
__device__ __forceinline__ void ch_put(const Chain& r, uint4 d) {
  const uint32_t o = r.fb & 48u;
  lds_st128(r.rb + o, d);
  if (MIR && o < (uint32_t)kMirrorBytes) lds_st128(r.rb + o + 2u * kRingWords, d);
}
// start of a group pair: the linear read pointer from the consumed count
template <bool MIR>
__device__ __forceinline__ void ch_linear(Chain& r) {
  if constexpr (MIR) {
    r.ra = r.rb + (r.a2 & 62u);
    r.d = r.a2 - r.ra;
  } else {
    r.ra = r.a2;
  }
}
// end of a group pair: the consumed count from the linear read pointer
template <bool MIR>
__device__ __forceinline__ void ch_settle(Chain& r) {
  if constexpr (MIR) r.a2 = r.ra + r.d;
  else r.a2 = r.ra;
}
// Positions for one round of requests: full chunks take the tile's next main-area
// slots in lane (= chain) order, a tail sits at its own place.
__device__ __forceinline__ uint32_t ch_claim(Chain& r, bool want, bool& full) {
  full = want && r.rem >= kChunkWords;
  const uint64_t m = __ballot(full);
  const uint32_t mlo = (uint32_t)m & r.seg_lo, mhi = (uint32_t)(m >> 32) & r.seg_hi;
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
  const uint32_t pos = full ? r.cur + kChunkWords * rank : r.tailp;
  r.cur += kChunkWords * (uint32_t)(__builtin_popcount(mlo) + __builtin_popcount(mhi));
  return pos;
}
__device__ __forceinline__ uint4 ld_chunk(const StreamRef& s, uint32_t pos) {
  return *(const uint4*)(s.w + (pos < s.last_chunk ? pos : s.last_chunk));
}
__device__ __forceinline__ uint4 ld_tail(const StreamRef& s, uint32_t pos) {
  const uint16_t* p = s.w + (pos < s.last_chunk ? pos : s.last_chunk);
  uint4 d;
  d.x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
  d.y = (uint32_t)p[2] | ((uint32_t)p[3] << 16);
  d.z = (uint32_t)p[4] | ((uint32_t)p[5] << 16);
  d.w = (uint32_t)p[6] | ((uint32_t)p[7] << 16);
  return d;
}
// Sync site: rounds until no lane of the wave wants more (every active lane calls it);
// ahead2 = the target in bytes.
template <bool MIR>
__device__ __forceinline__ void ch_sync(const StreamRef& s, Chain& r, bool cand, int32_t ahead2) {
  for (;;) {
    const bool want = cand && (int32_t)(r.fb - r.a2) < ahead2 && r.rem > 0;
    if (__ballot(want) == 0) return;
    bool full;
    const uint32_t pos = ch_claim(r, want, full);
    if (want) {
      ch_put<MIR>(r, full ? ld_chunk(s, pos) : ld_tail(s, pos));
      const int32_t n = full ? kChunkWords : r.rem;
      r.fb += 2u * (uint32_t)n;
      r.rem -= n;
    }
  }
}
// Prime: the rounds of a sync site to 17 ahead from an empty ring.  Three rounds always
// suffice (each request adds 8 words, or the tail, after which the chain wants no more),
// and request positions do not depend on the data, so all loads are issued before the
// first is written: one memory latency instead of three.
// (Full chunks load unconditionally, lanes without one reading the stream's first
// chunk, so that no loaded value is merged before its wait; a tail, at most one per
// chain and rare, is fetched after the rounds.)
struct PrimeLoads {
  uint4 dat[3];
  uint32_t at[3];
  bool put[3], mir[3];
  uint32_t t_at, t_pos;
  bool t_has, t_mir;
};
template <bool MIR>
__device__ __forceinline__ void ch_prime_issue(const StreamRef& s, Chain& r, bool cand, int32_t ahead2,
                                               PrimeLoads& P) {
  uint4* dat = P.dat;
  uint32_t* at = P.at;
  bool* put = P.put;
  bool* mir = P.mir;
  uint32_t t_at = 0u, t_pos = 0u;
  bool t_has = false, t_mir = false;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const bool want = cand && (int32_t)(r.fb - r.a2) < ahead2 && r.rem > 0;
    bool full;
    const uint32_t pos = ch_claim(r, want, full);
    const uint32_t o = r.fb & 48u;
    at[k] = r.rb + o;
    put[k] = full;
    mir[k] = MIR && full && o < (uint32_t)kMirrorBytes;
    dat[k] = ld_chunk(s, full ? pos : 0u);
    if (want && !full) {
      t_has = true;
      t_at = r.rb + o;
      t_pos = pos;
      t_mir = MIR && o < (uint32_t)kMirrorBytes;
    }
    if (want) {
      const int32_t n = full ? kChunkWords : r.rem;
      r.fb += 2u * (uint32_t)n;
      r.rem -= n;
    }
  }
  P.t_at = t_at;
  P.t_pos = t_pos;
  P.t_has = t_has;
  P.t_mir = t_mir;
}
__device__ __forceinline__ void ch_prime_finish(const StreamRef& s, const PrimeLoads& P) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (P.put[k]) lds_st128(P.at[k], P.dat[k]);
    if (P.mir[k]) lds_st128(P.at[k] + 2u * kRingWords, P.dat[k]);
  }
  if (P.t_has) {
    const uint4 d = ld_tail(s, P.t_pos);
    lds_st128(P.t_at, d);
    if (P.t_mir) lds_st128(P.t_at + 2u * kRingWords, d);
  }
}
__device__ __forceinline__ void ch_flush(Chain& r) {
  if (r.have_pend) lds_st128(r.pend_at, r.pend);
  if (r.pend_mirror) lds_st128(r.pend_at + 2u * kRingWords, r.pend);
  r.have_pend = false;
  r.pend_mirror = false;
}
// Service (every even group; every group of a blob with escapes): write the chunk in
// flight, top up to ahead2 / 2 words ahead (17, or 24 with escapes), then one round for
// chains at most 24 ahead.  Full chunks load asynchronously with a fixed pattern (one
// 16-byte load per lane; lanes without a chunk read the stream's first one, a line
// every lane shares); tails, rare, are fetched at once.
template <bool MIR>
__device__ __forceinline__ void ch_service(const StreamRef& s, Chain& r, bool act, int32_t ahead2) {
  ch_flush(r);
  ch_sync<MIR>(s, r, act, ahead2);
  const bool want = act && (int32_t)(r.fb - r.a2) <= 2 * (kRingWords - kChunkWords) && r.rem > 0;
  bool full;
  const uint32_t pos = ch_claim(r, want, full);
  const bool tail = want && !full;
  if (__ballot(tail) != 0) {
    if (tail) {
      ch_put<MIR>(r, ld_tail(s, pos));
      r.fb += 2u * (uint32_t)r.rem;
      r.rem = 0;
    }
  }
  r.pend_at = (r.fb & 48u) + r.rb;
  r.pend_mirror = MIR && full && (r.fb & 32u) == 0u;
  r.pend = ld_chunk(s, full ? pos : 0u);
  if (full) {
    r.fb += 2u * kChunkWords;
    r.rem -= kChunkWords;
  }
  r.have_pend = full;
}
// 16-bit renormalisation from the word already read, through the linear pointer (the
// next word is read at once, for the next renormalisation)
template <bool MIR>
__device__ __forceinline__ void ch_renorm_lin_if(Chain& r, bool need) {
  if (need) {
    r.x = (r.x << 16) | r.nw;
    r.ra += 2u;
    r.nw = lds_u16(ch_at<MIR>(r));
  }
}
// the same without a branch: selects, and the next word read every symbol (the same
// word again when the state did not renormalise).  Shorter per-symbol latency (no
// exec-mask switch) for more ring reads: faster for launches of few waves per CU,
// slower when LDS is busy.
template <bool MIR>
__device__ __forceinline__ void ch_renorm_lin_sel(Chain& r, bool need) {
  const uint32_t xs = (r.x << 16) | r.nw;
  r.x = need ? xs : r.x;
  r.ra += need ? 2u : 0u;
  r.nw = lds_u16(ch_at<MIR>(r));
}
// Renormalise ILP chains: all conditions first, so that no chain's state update is
// sunk below another chain's (conditional) ring read.
template <int ILP, bool SEL>
__device__ __forceinline__ void ch_renorm_all(Chain* rd) {
  bool need[ILP];
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    // pin the state update here (an empty asm that reads it), ahead of every ring read
    if (ILP > 1) asm volatile("" ::"v"(rd[c].x));
    need[c] = rd[c].x < kL;
  }
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    if constexpr (SEL) ch_renorm_lin_sel<ILP == 1>(rd[c], need[c]);
    else ch_renorm_lin_if<ILP == 1>(rd[c], need[c]);
  }
}
// table entry of the chain's next symbol; `base` = byte offset of the table in LDS
template <class G>
__device__ __forceinline__ typename G::Ent ch_entry(uint32_t base, const Chain& r) {
  if constexpr (G::kSplit) return ((const EP_LDS EntPair*)(uintptr_t)base)[r.x & G::kMask];
  else return ((const EP_LDS uint32_t*)(uintptr_t)base)[r.x & G::kMask];
}
// x = f (x >> P) + (slot - cum)
// (split entries: f alone in the low 24 bits of the first word, the bias alone in the
// second, so the 24-bit multiply-add takes them as they are)
template <class G>
__device__ __forceinline__ void ch_decode(Chain& r, typename G::Ent e) {
  if constexpr (G::kSplit) r.x = __umul24(e.x, r.x >> G::kP) + e.y;
  else r.x = __umul24(e & 2047u, r.x >> G::kP) + ((e >> 11) & 2047u);
}
// Bypass field of nb <= 16 raw bits (the state's low bits), through the linear pointer
template <bool MIR>
__device__ __forceinline__ uint32_t ch_bypass_lin(Chain& r, uint32_t nb) {
  const uint32_t v = __builtin_amdgcn_ubfe(r.x, 0u, nb);
  r.x >>= nb;
  ch_renorm_lin_if<MIR>(r, r.x < kL);
  return v;
}
// Doubled coordinate of an escape symbol: its raw bits follow the table step (low 16
// first, then the rest), the last coordinate's lowest bit implied by the E8 parity pi.
template <class LY, bool MIR>
__device__ __forceinline__ int32_t ch_escape_lin(Chain& r, uint32_t e, bool last, uint32_t pi) {
  uint32_t c, lead3, n2;
  int32_t sgn;
  LY::esc_info(e, c, sgn, lead3, n2);
  const uint32_t nb = last ? n2 - 1u : n2;
  uint32_t raw;
  if (nb <= 16u) {
    raw = ch_bypass_lin<MIR>(r, nb);
  } else {   // (magnitudes of 2^19 and more)
    raw = ch_bypass_lin<MIR>(r, 16u);
    raw |= ch_bypass_lin<MIR>(r, nb - 16u) << 16;
  }
  if (last) raw = (raw << 1) | (pi ^ ((uint32_t)sgn & c));
  const uint32_t m = (lead3 << n2) | raw;
  const uint32_t a = (m << 1) | c;
  return (int32_t)((a ^ (uint32_t)sgn) - (uint32_t)sgn);   // -a for a negative coordinate
}
// LDS table slot of stored table t (stored order FIRST, FREE[0], FREE[1], LAST...)
__host__ __device__ constexpr int lds_table_slot(int t) { return t == 0 ? 1 : (t == 1 ? 0 : t); }

// Stages a job's decode tables into LDS (stored order FIRST, FREE[0], ...; in LDS the
// first two swap places).  issue() starts four 16-byte loads per thread, commit()
// stores them (and does the rest on small workgroups), then waits at the workgroup
// barrier; the first block's stream loads go out in between, so a starting workgroup
// waits about one memory latency for both.
struct TabStager {
  int q;                              // uint4 per table
  int kN;                             // uint4 to stage (at most kTabBytes / 16)
  const uint4* src;
  uint4* dst;
  int tid, nt;
  bool swap;    // the lossy layout: stored FIRST, FREE[0] change places (TileANS: as stored)
  uint4 v[4];
  // (indices past the end are clamped to the last element, which then is loaded and
  // stored by several threads with the same value: no conditional stores, so the
  // loads stay where they are issued)
  __device__ void issue() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = k * nt + tid;
      v[k] = src[i < kN ? i : kN - 1];
    }
  }
  __device__ void put(int i, uint4 d) { dst[swap && i < 2 * q ? (i ^ q) : i] = d; }
  __device__ void commit() {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = k * nt + tid;
      put(i < kN ? i : kN - 1, v[k]);
    }
    for (int i = 4 * nt + tid; i < kN; i += nt) put(i, src[i]);
    __syncthreads();
  }
};

// Row scale of a chain's groups.  A chain's groups are g0, g0 + S, g0 + 2S, ...  When
// S <= G (the row length in groups) consecutive ones are at most one row apart, so the
// scale changes only at precomputed group counts; otherwise every group is on a later row.
// The scale of the row the chain moves to next is loaded at every group (the same
// address until the row changes), so a group's memory pattern is fixed and a row change
// only moves registers.
struct RowScale {
  float h, nh;          // h_r of the current group's row, and -128 h_r
  float hn;             // the scale at pn (loaded one group ahead)
  const float* pn;      // scale of the row the chain moves to next
  uint32_t row;         // row of the current group
  uint32_t kchg;        // group count at which the row changes next
  uint32_t bnd;         // S <= G: first group of the row after the next one, - g0 + S - 1
  uint32_t rown, coln;  // S > G: row and column group of the chain's next group
};

struct GroupCtx {
  const DecJob* J;
  StreamRef sref;
  uint32_t lds0;   // LDS address of the tables
  uint32_t ctx_mask;
  uint32_t G;
  int S;
  bool rowwise;
  // fused prefill product: LDS address of the operand tiles, of this lane's row in the
  // first one and that row's chunk swizzle; the workgroup's first output column
  uint32_t bt_base, bt_row, bt_swz;
  int64_t mma_n0;
};

// Fused matrix-vector product: a chain's running dot products of its weights in the
// current row with the NT activation rows, written to the chain's partial-sum slot of
// that row when the chain moves on (a chain's groups run through the rows in order).
struct MvAcc {
  float a[8];
  uint32_t row, rlo;   // row being summed, the chain's first row
  int64_t slot0;       // partial-sum slot of (chain, rlo)
};

template <int NT>
__device__ __forceinline__ void mv_flush(const DecJob& J, MvAcc& m) {
  float* o = (float*)J.out + (m.slot0 + (int64_t)(m.row - m.rlo)) * NT;
  typedef __attribute__((ext_vector_type(4))) float f32x4;
  if constexpr (NT >= 4) {
#pragma unroll
    for (int t = 0; t < NT; t += 4) *(f32x4*)(o + t) = f32x4{m.a[t], m.a[t + 1], m.a[t + 2], m.a[t + 3]};
  } else if constexpr (NT == 2) {
    *(f32x2*)o = f32x2{m.a[0], m.a[1]};
  } else {
    o[0] = m.a[0];
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) m.a[t] = 0.f;
}

// ---- fused prefill product (OUT_MMA*): Y[T x R] = X[T x C] W^T (+ bias) with W decoded
// into LDS, C = 4096 TP (TP = 1 or 2 tiles a row).  At S = 8 a tile is 4096 consecutive
// columns of one row, so a wave's block of 64 chains is 8 tiles (8 / TP rows of W) and,
// at a chain's group pair kk, kk + 1, the 8 chains of a tile yield the tile's columns
// 64 kk .. 64 kk + 127 in chunks of 8.  A workgroup of 8 waves (64 tiles: 64 / TP rows of
// W and as many output columns) writes each pair's slab (per row, TP segments of 128
// columns: one at 128 i of each tile) to one of two LDS operand tiles (rows of 256 TP
// bytes, the 16-byte chunks of each segment XOR-swizzled by the row), meets at a
// barrier, and every wave multiplies the slab by its own 16-row blocks of X (wave w: rows
// 16 (w + 8 b) .. + 15, b < MB), read straight from memory into registers at the start
// of the pair: v_mfma_f32_16x16x32_bf16 with the W fragment first, so a lane ends with
// four consecutive output columns of one activation row.  The weights never leave LDS.
constexpr int kMmaWaves = 8;
constexpr uint32_t kBRowBytes = 256;
constexpr uint32_t kBTileBytes = 64 * kBRowBytes;
constexpr int kPrefillMaxT = 16 * kMmaWaves * 2;   // 256 activation rows
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// activation fragments of slab `it` (columns 4096 sg + 128 it .. + 127 of segment sg):
// block b, segment sg, K step ks
template <int MB, int TP>
__device__ __forceinline__ void mma_xload(const DecJob& J, int it, int wave, int lane, u32x4 (&xf)[MB][TP][4]) {
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const uint32_t t = (uint32_t)((wave + kMmaWaves * b) * 16 + lr);
    const uint32_t tt = t < J.mv_T ? t : J.mv_T - 1u;
    const uint16_t* xp = J.mv_x + (int64_t)tt * J.C + it * 128 + 8 * lq;
#pragma unroll
    for (int sg = 0; sg < TP; ++sg)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) xf[b][sg][ks] = *(const u32x4*)(xp + 8 * kTileGroups * sg + 32 * ks);
  }
}
// the slab in operand tile `buf` times this wave's activation blocks
// (a wave whose activation blocks all lie past the T rows skips the slab: no LDS reads,
// no MFMAs; a branch uniform per wave.  Its activation loads stay unconditional, so the
// memory counters the decode's waits rely on do not depend on T: with those loads
// conditional too, the kernel was slower, not faster)
template <int MB, int TP>
__device__ __forceinline__ void mma_slab(const GroupCtx& X, uint32_t buf, int wave, int lane,
                                         const u32x4 (&xf)[MB][TP][4], f32x4 (&acc)[MB][4 / TP]) {
  if ((uint32_t)(wave * 16) >= X.J->mv_T) return;
  const uint32_t lr = (uint32_t)lane & 15u, lq = (uint32_t)lane >> 4;
  const uint32_t base = X.bt_base + buf * kBTileBytes;
#pragma unroll
  for (int sg = 0; sg < TP; ++sg) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int cb = 0; cb < 4 / TP; ++cb) {
        const uint32_t row = 16u * (uint32_t)cb + lr;   // (row & 15 == lr)
        const uint32_t a = base + row * (kBRowBytes * TP) + (uint32_t)sg * kBRowBytes +
                           ((((uint32_t)ks * 4u + lq) ^ lr) << 4);
        const bf16x8 wf = *(const EP_LDS bf16x8*)(uintptr_t)a;
#pragma unroll
        for (int b = 0; b < MB; ++b)
          acc[b][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, __builtin_bit_cast(bf16x8, xf[b][sg][ks]), acc[b][cb],
                                                               0, 0, 0);
      }
    }
  }
}
// outputs: lane l holds activation row 16 (w + 8 b) + l % 16, output columns
// mma_n0 + 16 cb + 4 (l / 16) .. + 3; bias added, rounded to BF16 (nearest even)
template <int MB, int TP>
__device__ __forceinline__ void mma_store(const GroupCtx& X, int wave, int lane, const f32x4 (&acc)[MB][4 / TP]) {
  const DecJob& J = *X.J;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t N = J.R;
  uint16_t* Y = (uint16_t*)J.out;
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int64_t t = (int64_t)(wave + kMmaWaves * b) * 16 + lr;
    if (t >= (int64_t)J.mv_T) continue;
#pragma unroll
    for (int cb = 0; cb < 4 / TP; ++cb) {
      const int64_t n = X.mma_n0 + 16 * cb + 4 * lq;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float bb = (J.bias && n + e < N) ? __uint_as_float((uint32_t)J.bias[n + e] << 16) : 0.f;
        v[e] = acc[b][cb][e] + bb;
      }
      uint16_t* yp = Y + t * N + n;
      if ((N & 3) == 0 && n + 3 < N) {
        *(uint2*)yp = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) yp[e] = (uint16_t)(pack_bf16x2(v[e], 0.f) & 0xFFFFu);
      }
    }
  }
}

// Row scale of group kk: move to the next row at a precomputed group count, then issue
// the (usually repeated) load of the scale the chain moves to next.
template <int ILP>
__device__ __forceinline__ void row_scale(const GroupCtx& X, int kk, RowScale* rs, const int* ngr) {
  const DecJob& J = *X.J;
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    RowScale& q = rs[c];
    if ((uint32_t)kk == q.kchg && ((ILP == 1) || kk < ngr[c])) {
      q.h = q.hn;
      q.nh = -128.f * q.hn;
      if (X.rowwise) {
        ++q.row;
        q.kchg = q.bnd >> J.log2S;
        q.bnd += X.G;
        q.pn += 1;
      } else {
        q.row = q.rown;
        q.kchg = (uint32_t)kk + 1u;
        q.coln += J.s_mod_g;
        q.rown += J.s_div_g;
        if (q.coln >= X.G) {
          q.coln -= X.G;
          ++q.rown;
        }
        q.pn = J.hr + q.rown;
      }
    }
    q.hn = *q.pn;
  }

}

// Decode group kk of ILP chains: eight symbols per chain (escape symbols' raw bits read
// in place), container store or fused product.
template <int OUT, bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
__device__ __forceinline__ void decode_group(const GroupCtx& X, int kk, Chain* rd, RowScale* rs, const int* ngr,
                                             const uint32_t* g0, char** optr, MvAcc* mv) {
  using LY = EntryLayout<NARROW>;
  using G = Geo<OUT, ESC, NARROW>;
  constexpr bool MIR = ILP == 1;
  const DecJob& J = *X.J;
  constexpr int NT = mv_tokens<OUT>();
  // fused product: this group's activation chunks are requested before its symbols are
  // decoded (row and column of the group are known; idle chains read column 0)
  uint4 xv[ILP][NT > 0 ? NT : 1];
  uint32_t mrow[ILP];
  if constexpr (NT > 0) {
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      const bool act = kk < ngr[c];
      mrow[c] = rs[c].row;
      const uint32_t gk = g0[c] + (uint32_t)kk * (uint32_t)X.S;
      const int64_t c0 = act ? (int64_t)(gk - mrow[c] * X.G) * 8 : 0;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int64_t tt = (uint32_t)t < J.mv_T ? t : (int64_t)J.mv_T - 1;
        xv[c][t] = *(const uint4*)(J.mv_x + tt * J.C + c0);
      }
    }
  }
  if constexpr (OUT == OUT_BYTES) {
    // TileANS: eight byte symbols, symbol i from the table of context i & ctx_mask
    uint32_t xs[ILP], ras[ILP], nws[ILP];
    int32_t e[ILP][8];
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      xs[c] = rd[c].x;
      ras[c] = rd[c].ra;
      nws[c] = rd[c].nw;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t tb = X.lds0 + ((i & X.ctx_mask) << G::kTableLog2);
#pragma unroll
      for (int c = 0; c < ILP; ++c) e[c][i] = (int32_t)ch_entry<G>(tb, rd[c]);
#pragma unroll
      for (int c = 0; c < ILP; ++c) ch_decode<G>(rd[c], (uint32_t)e[c][i]);
      ch_renorm_all<ILP, SEL>(rd);
    }
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      const bool act = (ILP == 1) || kk < ngr[c];
      if (act) {
        if (C8) {
          store_group<OUT>(optr[c], 0, nullptr, e[c], true, 8);
        } else {
          const int64_t c0 = (int64_t)(g0[c] + (uint32_t)kk * (uint32_t)X.S) * 8;
          store_group<OUT>(J.out, c0, nullptr, e[c], c0 + 8 <= J.C, J.C - c0);
        }
      }
      if (ILP > 1 && kk >= ngr[c]) {
        rd[c].x = xs[c];
        rd[c].ra = ras[c];
        rd[c].nw = nws[c];
      }
      optr[c] += (int64_t)X.S * 8;
    }
    return;
  }
  uint32_t xs[ILP], ras[ILP], nws[ILP], ds[ILP];
  uint32_t e[ILP][8];
  int32_t uu[ILP][8];
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    xs[c] = rd[c].x;
    ras[c] = rd[c].ra;
    nws[c] = rd[c].nw;
    ds[c] = rd[c].d;
  }
  if constexpr (ESC) {
    // ---- blobs with escapes: one pass, each escape symbol's raw bits read where it
    // stands.  A symbol reads at most three words (a renormalisation and two bypass
    // fields), so four symbols stay within the 16 words the linear pointer may run past
    // the ring's end: it is re-derived from the consumed count after the fourth.
    static_assert(!G::kSplit, "escapes take packed entries");
    uint32_t fbs[ILP], pp[ILP];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i == 4) {
#pragma unroll
        for (int c = 0; c < ILP; ++c) {
          ch_settle<MIR>(rd[c]);
          ch_linear<MIR>(rd[c]);
        }
      }
      uint32_t ee[ILP];
#pragma unroll
      for (int c = 0; c < ILP; ++c) {
        uint32_t tb;
        if (i == 0) tb = X.lds0 + G::kFirstOff;
        else if (i < 7) tb = fbs[c];
        else tb = fbs[c] + G::kLastOff + ((pp[c] & 1u) << G::kTableLog2);
        ee[c] = ch_entry<G>(tb, rd[c]);
      }
#pragma unroll
      for (int c = 0; c < ILP; ++c) ch_decode<G>(rd[c], ee[c]);
      ch_renorm_all<ILP, SEL>(rd);
#pragma unroll
      for (int c = 0; c < ILP; ++c) {
        if (i == 0) fbs[c] = X.lds0 + G::free_base(ee[c]);
        int32_t v = LY::u_of(ee[c]);
        if (ee[c] & LY::kEsc) v = ch_escape_lin<LY, MIR>(rd[c], ee[c], i == 7, pp[c] & 1u);
        uu[c][i] = v;
        // parity of the first seven floor(u / 2): bit 1 of their xor
        if (i == 0) pp[c] = (uint32_t)v >> 1;
        else if (i < 7) pp[c] ^= (uint32_t)v >> 1;
      }
    }
  } else {
  // ---- escape-free blobs: eight symbols per chain, the coordinate straight from the
  // entry (e holds each entry's value word; a split entry's bias word is used by its
  // decode step only)
  uint32_t fbs[ILP];
  typename G::Ent en[ILP];
#pragma unroll
  for (int c = 0; c < ILP; ++c) en[c] = ch_entry<G>(X.lds0 + G::kFirstOff, rd[c]);
  // per step: every chain's table read, then every chain's state update, then the
  // renormalisations (whose ring reads are conditional and so end the step's LDS batch)
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    ch_decode<G>(rd[c], en[c]);
    e[c][0] = G::lo(en[c]);
    fbs[c] = X.lds0 + G::free_base(e[c][0]);
  }
  ch_renorm_all<ILP, SEL>(rd);
#pragma unroll
  for (int i = 1; i < 7; ++i) {
#pragma unroll
    for (int c = 0; c < ILP; ++c) en[c] = ch_entry<G>(fbs[c], rd[c]);
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      ch_decode<G>(rd[c], en[c]);
      e[c][i] = G::lo(en[c]);
    }
    ch_renorm_all<ILP, SEL>(rd);
  }
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    // LAST[c][pi]: pi = parity of the seven floor(u/2), one bit of each entry
    const uint32_t par = xor3(xor3(e[c][1], e[c][2], e[c][3]), xor3(e[c][4], e[c][5], e[c][6]), e[c][0]);
    const uint32_t lb = fbs[c] + G::kLastOff + (((par >> LY::kPar) & 1u) << G::kTableLog2);
    en[c] = ch_entry<G>(lb, rd[c]);
  }
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    ch_decode<G>(rd[c], en[c]);
    e[c][7] = G::lo(en[c]);
  }
  ch_renorm_all<ILP, SEL>(rd);
  }

#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    const bool act = (ILP == 1) || kk < ngr[c];
    float w[8];
    int32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (ESC) {
        if (OUT == OUT_COORDS) u[i] = uu[c][i];
        else w[i] = rs[c].h * (float)uu[c][i];
      } else {
        if (OUT == OUT_COORDS) u[i] = LY::u_of(e[c][i]);
        else w[i] = LY::w_of(e[c][i], rs[c].h, rs[c].nh);
      }
    }
    if constexpr (NARROW && !ESC && OUT != OUT_COORDS) {
      // rows whose -128 h_r overflows: the plain product (a branch uniform per blob)
      if (J.big_h) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = rs[c].h * (float)LY::u_of(e[c][i]);
      }
    }
    if constexpr (mma_blocks<OUT>() > 0) {
      // the weights as the BF16 container holds them, to this row's chunk of the slab
      // (every lane writes, also past the matrix: those rows feed no stored output)
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = w[2 * i], b = w[2 * i + 1];
        if (J.mv_sat) {
          a = fminf(fmaxf(a, -3.38953139e38f), 3.38953139e38f);
          b = fminf(fmaxf(b, -3.38953139e38f), 3.38953139e38f);
        }
        f32x2 fv = {a, b};
        p[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(fv, bf16x2));
      }
      const uint32_t chunk = (((uint32_t)kk & 1u) << 3) | ((uint32_t)threadIdx.x & 7u);
      const uint32_t at = X.bt_row + (((uint32_t)kk >> 1) & 1u) * kBTileBytes + ((chunk ^ X.bt_swz) << 4);
      lds_st128(at, make_uint4(p[0], p[1], p[2], p[3]));
    } else if constexpr (NT > 0) {
      if (act) {
        // the weights as the BF16 container holds them, then two products per dot step
        uint32_t p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = w[2 * i], b = w[2 * i + 1];
          if (J.mv_sat) {
            a = fminf(fmaxf(a, -3.38953139e38f), 3.38953139e38f);
            b = fminf(fmaxf(b, -3.38953139e38f), 3.38953139e38f);
          }
          f32x2 fv = {a, b};
          p[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(fv, bf16x2));
        }
        if (mrow[c] != mv[c].row) {
          mv_flush<NT>(J, mv[c]);
          mv[c].row = mrow[c];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float acc = mv[c].a[t];
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[0]), __builtin_bit_cast(bf16x2, xv[c][t].x), acc, false);
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[1]), __builtin_bit_cast(bf16x2, xv[c][t].y), acc, false);
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[2]), __builtin_bit_cast(bf16x2, xv[c][t].z), acc, false);
          acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[3]), __builtin_bit_cast(bf16x2, xv[c][t].w), acc, false);
          mv[c].a[t] = acc;
        }
      }
    } else if (act) {
      if (C8) {
        store_group<OUT>(optr[c], 0, w, u, true, 8);
      } else {
        const uint32_t gk = g0[c] + (uint32_t)kk * (uint32_t)X.S;
        const int64_t c0 = (int64_t)(gk - rs[c].row * X.G) * 8;
        store_group<OUT>(J.out, (int64_t)rs[c].row * J.C + c0, w, u, c0 + 8 <= J.C, J.C - c0);
      }
    }
  }
  if (ILP > 1) {
    // a chain past its last group keeps its final state
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      if (kk >= ngr[c]) {
        rd[c].x = xs[c];
        rd[c].ra = ras[c];
        rd[c].nw = nws[c];
        if constexpr (ESC) rd[c].d = ds[c];   // (the escape pass re-derives the pointer)
      }
    }
  }
  constexpr int ESZ = out_elem_bytes<OUT>();
#pragma unroll
  for (int c = 0; c < ILP; ++c) optr[c] += (int64_t)X.S * 8 * ESZ;
}

// Where chain `lane` of block blk starts: its initial state, the word index of its tile's
// main area, the word index of its tail and its length in words, from the stored chunk
// counts and tail lengths.  Chains store their full chunks tile after tile and then all
// tails in chain order, so a wave-wide exclusive prefix sum over the block's 64 chains of
// (full chunks | tail words << 22) gives every offset: a tile's main area starts at the
// chunk sum of the chains before its first lane, the tails after the block's chunk total.
// (Full chunks of one block stay below 2^22 and tail words below 2^10.)  Every lane of the
// wave takes part; blk is uniform per wave.
__device__ __forceinline__ uint4 chain_meta(const DecJob& J, int64_t blk, int lane, int s0) {
  if (blk >= J.n_blocks) return make_uint4(kL, 0u, 0u, 0u);
  const int64_t ch = blk * 64 + lane;
  uint32_t nf = 0u, tl = 0u, st = kL;
  if (ch < J.n_chains) {
    nf = J.log2S >= 3 ? (uint32_t)((const uint8_t*)J.full)[ch] : (uint32_t)((const uint16_t*)J.full)[ch];
    tl = (uint32_t)(J.nib[ch >> 1] >> (4 * (ch & 1))) & 15u;
    st = J.states[ch];
  }
  const uint32_t v = nf | (tl << 22);
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)inc, (unsigned)o, 64);
    inc += lane >= o ? t : 0u;
  }
  const uint32_t exc = inc - v;
  const uint32_t tot = (uint32_t)__shfl((int)inc, 63, 64);
  const uint32_t tile = (uint32_t)__shfl((int)exc, s0, 64);
  const uint32_t base = 8u * J.boff[blk];   // the block's first word
  constexpr uint32_t kLo = (1u << 22) - 1u;
  return make_uint4(st, base + 8u * (tile & kLo), base + 8u * (tot & kLo) + (exc >> 22), 8u * nf + tl);
}

// One wave decodes ILP blocks of 64 chains (blocks blk0 .. blk0 + ILP - 1, those below
// blk_end): lane l runs chain l of each, the ILP chains interleaved step by step so
// that one chain's table read is in flight while another computes.
template <int OUT, bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
__device__ __forceinline__ void decode_blocks(const GroupCtx& X, int64_t blk0, int64_t blk_end, int lane, int wave,
                                              TabStager& st, bool stage) {
  const DecJob& J = *X.J;
  const int S = X.S;
  const uint32_t G = X.G;
  // lanes of this lane's tile (S consecutive lanes)
  const int s0 = lane & ~(S - 1);
  const uint64_t seg = (S == 64) ? ~0ull : (((1ull << S) - 1ull) << s0);

  constexpr int ESZ = out_elem_bytes<OUT>();
  constexpr bool MIR = ILP == 1;
  // words kept ahead by a service (in bytes): two escape-free groups, or one group with escapes
  constexpr int32_t kAhead2 = ESC ? 2 * 24 : 2 * 17;
  Chain rd[ILP];
  RowScale rs[ILP];
  int ngr[ILP];
  bool live[ILP];
  uint32_t g0[ILP];
  char* optr[ILP];
  MvAcc mv[ILP];
  constexpr int NT = mv_tokens<OUT>();
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    const int64_t ch = (blk0 + c) * 64 + lane;
    live[c] = blk0 + c < blk_end && ch < J.n_chains && ch >= J.chain_lo && ch < J.chain_hi;
    const int64_t t = ch >> J.log2S;
    const int j = (int)(ch & (S - 1));
    int64_t gt = J.n_groups - (t << 9);
    if (gt > kTileGroups) gt = kTileGroups;
    ngr[c] = (live[c] && gt > j) ? (int)((gt - j + S - 1) >> J.log2S) : 0;
    Chain& r = rd[c];
    uint4 meta = chain_meta(J, blk0 + c, lane, s0);
    if (!live[c]) meta = make_uint4(kL, 0u, 0u, 0u);
    r.x = meta.x;
    r.cur = meta.y;
    r.tailp = meta.z;
    r.rem = (int32_t)meta.w;
    // rotate each ring by a lane-dependent number of chunks (counters start there), so
    // lanes whose rings share LDS banks touch different banks
    r.fb = 16u * (uint32_t)(((lane >> 1) + (lane >> 3)) & 3);
    r.a2 = r.fb;
    uint32_t rb = X.lds0 + (uint32_t)kTabBytes + (uint32_t)(((wave * 64 + lane) * ILP + c) * ring_bytes<ILP>());
    asm volatile("" : "+v"(rb));   // keep the ring base opaque: ring addresses are one and-or
    r.rb = rb;
    r.seg_lo = (uint32_t)seg;
    r.seg_hi = (uint32_t)(seg >> 32);
    r.pend = make_uint4(0u, 0u, 0u, 0u);
    r.pend_at = rb;
    r.have_pend = false;
    r.pend_mirror = false;
    r.ra = MIR ? rb : r.a2;
    r.d = 0u;
    const bool any = ngr[c] > 0;
    const int64_t gg = (t << 9) + j;
    g0[c] = any ? (uint32_t)gg : 0u;
    const uint32_t row0 = any ? (uint32_t)(gg / J.G) : 0u;
    const uint32_t col0 = g0[c] - row0 * G;
    RowScale& q = rs[c];
    q.row = row0;
    if constexpr (NT > 0) {
      mv[c].row = mv[c].rlo = row0;
      mv[c].slot0 = ch * (int64_t)J.mv_slots;
#pragma unroll
      for (int t = 0; t < 8; ++t) mv[c].a[t] = 0.f;
    }
    if constexpr (OUT == OUT_BYTES) {   // no row scales
      q.h = q.nh = q.hn = 0.f;
      q.pn = nullptr;
      q.kchg = 0xFFFFFFFFu;
      q.bnd = q.rown = q.coln = 0;
      optr[c] = (char*)J.out + (live[c] ? gg * 8 : 0);
      continue;
    }
    q.h = any ? J.hr[row0] : 0.f;
    q.nh = -128.f * q.h;
    if (X.rowwise) {
      q.pn = J.hr + row0 + 1;                 // row scales are padded past the last row
      q.kchg = any ? (((row0 + 1) * G - g0[c] + (uint32_t)S - 1u) >> J.log2S) : 0xFFFFFFFFu;
      q.bnd = (row0 + 2) * G - g0[c] + (uint32_t)S - 1u;
      q.rown = q.coln = 0;
    } else {
      q.coln = col0 + J.s_mod_g;
      q.rown = row0 + J.s_div_g;
      if (q.coln >= G) {
        q.coln -= G;
        ++q.rown;
      }
      q.pn = J.hr + (any ? q.rown : 0u);
      q.kchg = any ? 1u : 0xFFFFFFFFu;
      q.bnd = 0;
    }
    q.hn = *q.pn;
    optr[c] = (char*)J.out + (live[c] ? gg * 8 * ESZ : 0);   // C % 8 == 0: groups are contiguous
  }
  // (the workgroup's first blocks: table loads, then stream loads, then table stores
  // and the barrier, then ring stores)
  // (both branches leave the same loads in flight, the stream loads, so that the wait
  // counts after them need not assume the table loads outstanding)
  PrimeLoads pl[ILP];
  if (stage) {
    st.issue();
#pragma unroll
    for (int c = 0; c < ILP; ++c) ch_prime_issue<MIR>(X.sref, rd[c], live[c], kAhead2, pl[c]);
    st.commit();
  } else {
#pragma unroll
    for (int c = 0; c < ILP; ++c) ch_prime_issue<MIR>(X.sref, rd[c], live[c], kAhead2, pl[c]);
  }
#pragma unroll
  for (int c = 0; c < ILP; ++c) {
    ch_prime_finish(X.sref, pl[c]);
    rd[c].nw = ch_word(rd[c]);
  }
  int nmax = ngr[0];
#pragma unroll
  for (int c = 1; c < ILP; ++c) nmax = ngr[c] > nmax ? ngr[c] : nmax;
  // fused prefill product: every lane of the workgroup runs all 64 groups (the slab
  // barriers are workgroup-wide); chains past the matrix decode rows no output reads
  constexpr int MB = mma_blocks<OUT>(), TP = mma_tiles_per_row<OUT>();
  f32x4 macc[MB > 0 ? MB : 1][4 / TP];
  u32x4 xf[MB > 0 ? MB : 1][TP][4];
  if constexpr (MB > 0) {
    nmax = kTileGroups / 8;   // (S = 8)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int cb = 0; cb < 4 / TP; ++cb) macc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // two groups per iteration: the stream service runs before every even group, and
  // (blobs with escapes) before every odd one too
  // (the row scale of a group is settled before its service, so that its load is
  // followed by a fixed sequence of memory operations)
  for (int kk = 0; kk < nmax; kk += 2) {
    if constexpr (MB > 0) mma_xload<MB, TP>(J, kk >> 1, wave, lane, xf);
    if constexpr (OUT != OUT_BYTES) row_scale<ILP>(X, kk, rs, ngr);
#pragma unroll
    for (int c = 0; c < ILP; ++c) {
      ch_service<MIR>(X.sref, rd[c], (ILP == 1) || kk < ngr[c], kAhead2);
      ch_linear<MIR>(rd[c]);
    }
    decode_group<OUT, ESC, C8, NARROW, ILP, SEL>(X, kk, rd, rs, ngr, g0, optr, mv);
    if (kk + 1 < nmax) {
      if constexpr (OUT != OUT_BYTES) row_scale<ILP>(X, kk + 1, rs, ngr);
      if constexpr (ESC) {
#pragma unroll
        for (int c = 0; c < ILP; ++c) {
          ch_settle<MIR>(rd[c]);
          ch_service<MIR>(X.sref, rd[c], (ILP == 1) || kk + 1 < ngr[c], kAhead2);
          ch_linear<MIR>(rd[c]);
        }
      }
      decode_group<OUT, ESC, C8, NARROW, ILP, SEL>(X, kk + 1, rd, rs, ngr, g0, optr, mv);
    }
#pragma unroll
    for (int c = 0; c < ILP; ++c) ch_settle<MIR>(rd[c]);
    if constexpr (MB > 0) {
      __syncthreads();   // the pair's slab is in LDS (and the tile written next is free)
      mma_slab<MB, TP>(X, ((uint32_t)kk >> 1) & 1u, wave, lane, xf, macc);
    }
  }
  if constexpr (NT > 0) {
    if (J.mv_direct) {
      // rows of whole tiles (S = 8 or 16, one or two tiles a row): a row's running sums sit in
      // mv_lanes consecutive lanes of this wave (its tiles' chains in order), each chain
      // having stayed on the row; the row's first lane adds them in the finishing
      // kernel's order (tiles, then chains, from 0), adds the bias and rounds to BF16
      static_assert(ILP == 1, "the fused product runs one chain per lane");
      const int l0 = lane & ~(int)(J.mv_lanes - 1u);
      const int64_t row = (blk0 * 64 + l0) / (int64_t)J.mv_lanes;
      // (lanes outer, activation rows inner: the NT sums advance side by side)
      float sum[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sum[t] = 0.f;
      for (int q = 0; q < (int)J.mv_lanes; ++q) {
#pragma unroll
        for (int t = 0; t < NT; ++t) sum[t] += __shfl(mv[0].a[t], l0 + q, 64);
      }
      if (lane == l0 && row < (int64_t)J.R) {
        const float bb = J.bias ? __uint_as_float((uint32_t)J.bias[row] << 16) : 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if ((uint32_t)t >= J.mv_T) break;
          const __bf16 o = (__bf16)(J.bias ? sum[t] + bb : sum[t]);
          ((uint16_t*)J.out)[(int64_t)t * J.R + row] = __builtin_bit_cast(uint16_t, o);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < ILP; ++c)
        if (live[c] && ngr[c] > 0) mv_flush<NT>(J, mv[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < ILP; ++c)
    if (live[c] && ngr[c] > 0 && rd[c].x != kL) atomicAdd(J.err, 1u);
  if constexpr (MB > 0) mma_store<MB, TP>(X, wave, lane, macc);
}

// A workgroup stages the decode tables of its job into LDS once, then its waves take
// the workgroup's blocks in turn (wave w: blocks w ILP, (w + W) ILP, ...).  Each job
// gives every workgroup `bpw` consecutive blocks (the last one fewer).
template <int OUT, bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
__device__ __forceinline__ void decode_kernel_body(const DecBatch& B) {
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
  const int64_t wg_blk0 = J.block_lo + ((int64_t)blockIdx.x - J.wg_begin) * B.bpw;
  const int64_t wg_blk1 = wg_blk0 + B.bpw < J.n_blocks ? wg_blk0 + B.bpw : J.n_blocks;

  // the decode tables, shared by the workgroup's waves: staged during each wave's
  // first block (every wave passes the stager's barrier exactly once)
  static_assert(lds_table_slot(0) == 1 && lds_table_slot(1) == 0 && lds_table_slot(2) == 2, "");
  TabStager st;
  st.src = (const uint4*)J.tab;
  st.dst = (uint4*)smem;
  st.tid = tid;
  st.nt = (int)blockDim.x;
  st.swap = OUT != OUT_BYTES;
  st.q = (int)(Geo<OUT, ESC, NARROW>::kTable / 16);
  st.kN = (int)(J.tab_words / 4);

  GroupCtx X;
  X.J = &J;
  X.lds0 = (uint32_t)(uintptr_t)(EP_LDS uint8_t*)smem;
  X.sref = StreamRef{J.stream, J.n_words};
  X.S = 1 << J.log2S;
  X.G = (uint32_t)J.G;
  X.rowwise = (uint32_t)X.S <= X.G;
  X.ctx_mask = J.ctx_mask;
  int64_t b = wg_blk0 + (int64_t)wave * ILP;
  if constexpr (mma_blocks<OUT>() > 0) {
    // fused prefill product: 8 waves of one block each (8 rows of W: S = 8, one tile a
    // row), the operand tiles after the rings; waves past the matrix run too (barriers)
    constexpr uint32_t TP = (uint32_t)mma_tiles_per_row<OUT>();
    X.bt_base = X.lds0 + (uint32_t)kTabBytes + (uint32_t)(nwaves * 64 * ring_bytes<1>());
    const uint32_t tile = (uint32_t)(wave * 8 + (lane >> 3)), rho = tile / TP;   // (tile, row) in the workgroup
    X.bt_row = X.bt_base + rho * kBRowBytes * TP + (tile % TP) * kBRowBytes;
    X.bt_swz = rho & 15u;
    X.mma_n0 = wg_blk0 * 8 / (int64_t)TP;
    decode_blocks<OUT, ESC, C8, NARROW, ILP, SEL>(X, b, wg_blk1, lane, wave, st, true);
    return;
  }
  if (b >= wg_blk1) {   // a wave without blocks still stages its share
    st.issue();
    st.commit();
    return;
  }
  for (bool first = true; b < wg_blk1; b += (int64_t)nwaves * ILP, first = false)
    decode_blocks<OUT, ESC, C8, NARROW, ILP, SEL>(X, b, wg_blk1, lane, wave, st, first);
}
template <int OUT, bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
__global__ void __launch_bounds__(1024) decode_kernel(const DecBatch B) {
  decode_kernel_body<OUT, ESC, C8, NARROW, ILP, SEL>(B);
}
// the fused prefill product: 8 waves a workgroup, so a lane may hold 256 registers
template <int OUT, bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
__global__ void __launch_bounds__(64 * kMmaWaves) mma_kernel(const DecBatch B) {
  decode_kernel_body<OUT, ESC, C8, NARROW, ILP, SEL>(B);
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

// Launch shape: ILP chains per lane, `waves` waves per workgroup, `bpw` blocks of 64
// chains per workgroup (its waves loop over them).
struct Shape {
  int ilp;
  int waves;
  int64_t bpw;
  bool partial;   // less than one full round at <= 8 waves per CU: latency-bound
};

template <int OUT, bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
int launch_t(const DecBatch& B, int64_t n_wg, int waves, hipStream_t st) {
  void (*kern)(const DecBatch);
  if constexpr (mma_blocks<OUT>() > 0) kern = mma_kernel<OUT, ESC, C8, NARROW, ILP, SEL>;
  else kern = decode_kernel<OUT, ESC, C8, NARROW, ILP, SEL>;
  size_t lds = (size_t)kTabBytes + (size_t)waves * 64 * ILP * ring_bytes<ILP>() +
               (mma_blocks<OUT>() > 0 ? 2 * (size_t)kBTileBytes : 0);
  static std::once_flag once;
  std::call_once(once, [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max_bytes());
  });
  hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(64 * waves), lds, st, B);
  return hip_check(hipGetLastError(), "decode launch");
}

template <bool ESC, bool C8, bool NARROW, int ILP, bool SEL>
int launch_out(int out, const DecBatch& B, int64_t n_wg, int waves, hipStream_t st) {
  switch (out) {
    case OUT_BF16: return launch_t<OUT_BF16, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_BF16_L2: return launch_t<OUT_BF16_L2, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_BF16_SAT: return launch_t<OUT_BF16_SAT, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_FP16: return launch_t<OUT_FP16, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_FP32: return launch_t<OUT_FP32, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_FP8: return launch_t<OUT_FP8, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_INT8: return launch_t<OUT_INT8, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
    case OUT_BYTES:
      if constexpr (!ESC && NARROW) return launch_t<OUT_BYTES, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
      return fail(EP_E_ARG, "byte output takes the escape-free narrow kernel");
    case OUT_MV1:
    case OUT_MV2:
    case OUT_MV4:
    case OUT_MV8:
      if constexpr (C8 && ILP == 1) {
        if (out == OUT_MV1) return launch_t<OUT_MV1, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
        if (out == OUT_MV2) return launch_t<OUT_MV2, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
        if (out == OUT_MV4) return launch_t<OUT_MV4, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
        return launch_t<OUT_MV8, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
      }
      return fail(EP_E_ARG, "the fused product takes whole groups per row and one chain per lane");
    default: return launch_t<OUT_COORDS, ESC, C8, NARROW, ILP, SEL>(B, n_wg, waves, st);
  }
}

template <bool NARROW, int ILP, bool SEL>
int launch_n(int out, bool esc, bool c8, const DecBatch& B, int64_t n_wg, int waves, hipStream_t st) {
  if (c8) return esc ? launch_out<true, true, NARROW, ILP, SEL>(out, B, n_wg, waves, st)
                     : launch_out<false, true, NARROW, ILP, SEL>(out, B, n_wg, waves, st);
  return esc ? launch_out<true, false, NARROW, ILP, SEL>(out, B, n_wg, waves, st)
             : launch_out<false, false, NARROW, ILP, SEL>(out, B, n_wg, waves, st);
}

int launch_any(int out, bool esc, bool c8, bool narrow, Shape sh, const DecBatch& B, int64_t n_wg, hipStream_t st) {
  if (sh.ilp == 2)
    return narrow ? launch_n<true, 2, false>(out, esc, c8, B, n_wg, sh.waves, st)
                  : launch_n<false, 2, false>(out, esc, c8, B, n_wg, sh.waves, st);
  // few waves per CU: the branch-free renormalisation (latency-bound)
  if (sh.partial)
    return narrow ? launch_n<true, 1, true>(out, esc, c8, B, n_wg, sh.waves, st)
                  : launch_n<false, 1, true>(out, esc, c8, B, n_wg, sh.waves, st);
  return narrow ? launch_n<true, 1, false>(out, esc, c8, B, n_wg, sh.waves, st)
                : launch_n<false, 1, false>(out, esc, c8, B, n_wg, sh.waves, st);
}

int out_kind(const Blob& b) {
  if (b.kind == kKindTileAns) return OUT_BYTES;
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
  j.boff = b.d_boff;
  j.full = b.d_full;
  j.nib = b.d_nib;
  j.states = b.d_states;
  j.hr = b.d_hr;
  j.tab = b.d_tab;
  j.err = b.d_err;
  j.out = out;
  j.n_groups = b.n_groups();
  j.G = (b.C + 7) / 8;
  j.C = b.C;
  j.n_chains = b.n_chains;
  j.n_blocks = b.n_blocks;
  j.chain_lo = 0;
  j.chain_hi = b.n_chains;
  j.block_lo = 0;
  j.wg_begin = 0;
  j.n_words = (uint32_t)b.n_words;
  j.log2S = __builtin_ctz((unsigned)b.S);
  j.k = b.k;
  j.c8 = (b.C % 8) == 0;
  j.s_div_g = (uint32_t)(b.S / j.G);
  j.s_mod_g = (uint32_t)(b.S % j.G);
  j.R = (uint32_t)b.R;
  j.ctx_mask = b.kind == kKindTileAns ? (uint32_t)(b.n_ctx - 1) : 0u;
  // TileANS stages only its contexts' tables
  j.tab_words = b.d_tab_words;
  j.big_h = b.d_big_h ? 1u : 0u;
  return j;
}

int cu_count() {
  static int v = -1;
  if (v < 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    int x = 0;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || x <= 0) x = 256;
    v = x;
  }
  return v;
}

// Launch shape.  One table copy (56 KB of LDS) serves the workgroup and each chain adds
// a 96-byte ring with its mirror (one chain per lane) or a 64-byte ring (two chains per
// lane), so a workgroup holds at most 16 waves of one chain per lane or 13 of two.  A launch of at least one full round (every CU a workgroup of 16 waves) gives each
// wave one block: all waves of a workgroup finish together, the 4 SIMDs carry equal
// work, and a launch queued on another stream fills the CUs the last round leaves idle.
// A smaller launch gives each workgroup at least 8 blocks (more when one workgroup per
// CU would not hold them all): every block is resident at once either way, so a lone
// launch takes one block's time, while the tables (56 KB of LDS per workgroup) serve
// more waves, so launches running side by side on other streams fit more waves on the
// chip (per-layer decode of the 276-matrix stack on four streams: 8.3 -> 6.0 ms).  Two chains per lane
// (EP_DECODE_ILP=2) is an option; EP_DECODE_WAVES / EP_DECODE_BPW override the shape.
// Launch shape for launches of at least one full round.  By default every wave takes one
// block, so a workgroup's LDS frees as its 16 waves end and launches queued on other
// streams overlap the last round (the fastest way through a model's worth of matrices).
// EP_DECODE_SPREAD=1 (read at every launch) spreads the blocks evenly instead, one
// workgroup per CU whose waves loop over their share: a launch that runs alone ends with
// every CU busy to its last round rather than a last round on part of the CUs.
bool spread_mode() {
  const char* e = std::getenv("EP_DECODE_SPREAD");
  return e && std::atoi(e) == 1;
}

int max_waves(int ilp) {
  const int ring = ilp == 1 ? ring_bytes<1>() : ring_bytes<2>();
  return std::max(1, std::min(kMaxWaves, (lds_max_bytes() - kTabBytes) / (ilp * 64 * ring)));
}

Shape pick_shape(const int64_t* n_blocks, int n, int64_t max_wg = 0) {
  // (max_wg > 0: a launch meant to run beside other work, on at most max_wg CUs)
  const int64_t cus = max_wg > 0 ? std::min<int64_t>(max_wg, cu_count()) : cu_count();
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += n_blocks[i];
  int ilp = 1;
  if (const char* e = std::getenv("EP_DECODE_ILP"))
    if (std::atoi(e) == 2) ilp = 2;
  // a spread launch beyond one round of one chain per lane that fits one round of two:
  // two chains per lane, every block resident at once (a 9-matrix DiT block, 6300
  // blocks: 155.9 -> 151.4 us)
  if (spread_mode() && max_wg <= 0 && total > cus * max_waves(1) && total <= cus * max_waves(2) * 2) ilp = 2;
  const int wmax = max_waves(ilp);
  int64_t bpw;
  if (total >= cus * wmax * ilp && spread_mode()) {
    // one workgroup per CU, its waves looping over an even share of the blocks: a lone
    // launch ends with every CU busy to its last round instead of a last round that
    // holds only part of the CUs (it leaves no room for a launch on another stream)
    bpw = (total + cus - 1) / cus;
    for (;;) {
      int64_t wg = 0;
      for (int i = 0; i < n; ++i) wg += (n_blocks[i] + bpw - 1) / bpw;
      if (wg <= cus) break;
      ++bpw;
    }
  } else if (total >= cus * wmax * ilp) {
    bpw = (int64_t)wmax * ilp;
  } else {
    bpw = std::max<int64_t>(std::min<int64_t>(8, (int64_t)wmax * ilp), (total + cus - 1) / cus);
    for (;;) {
      int64_t wg = 0;
      for (int i = 0; i < n; ++i) wg += (n_blocks[i] + bpw - 1) / bpw;
      if (wg <= cus) break;
      ++bpw;
    }
  }
  if (const char* e = std::getenv("EP_DECODE_BPW"))
    if (std::atoll(e) >= 1) bpw = std::atoll(e);
  int waves = (int)std::min<int64_t>(wmax, (bpw + ilp - 1) / ilp);
  if (const char* e = std::getenv("EP_DECODE_WAVES")) {
    const int v = std::atoi(e);
    if (v >= 1 && v <= kMaxWaves) waves = std::min(v, wmax);
  }
  // (the branch-free variant only where a CU holds at most 8 of these waves: with more,
  // its extra ring reads cost more than the branch, e.g. 2700 blocks at 11 waves per CU
  // took 83 us against 77)
  return Shape{ilp, waves, bpw, total < cus * wmax * ilp && waves <= 8};
}

}  // namespace

// A pointer the GPU may dereference: device or managed memory, or pinned host memory.
// (A pageable host pointer would fault the kernel; HIP does not know it.)
int check_gpu_pointer(const void* p, const char* what) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type == hipMemoryTypeUnregistered) {
    (void)hipGetLastError();
    return fail(EP_E_ARG, std::string(what) + " is not memory the GPU can access");
  }
  return EP_OK;
}

namespace {

int check_uploaded(const Blob& b) {
  if (!b.d_base) return fail(EP_E_STATE, "blob not uploaded (call ep_blob_upload)");
  int dev = -1;
  (void)hipGetDevice(&dev);
  if (dev != b.device) return fail(EP_E_STATE, "blob uploaded to another device");
  return EP_OK;
}

int decode_one(const Blob& b, void* dst, int64_t chain_lo, int64_t chain_hi, int out, hipStream_t st,
               int64_t max_wg = 0) {
  int rc = check_uploaded(b);
  if (rc) return rc;
  if (!dst) return fail(EP_E_ARG, "null destination");
  if ((rc = check_gpu_pointer(dst, "destination"))) return rc;
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
  const Shape sh = pick_shape(&nblk, 1, max_wg);
  const int64_t n_wg = (nblk + sh.bpw - 1) / sh.bpw;
  j.n_blocks = bhi;   // blocks beyond the range are skipped
  DecBatch B{};
  B.j[0] = j;
  B.n = 1;
  B.bpw = sh.bpw;
  return launch_any(out, (b.flags & kFlagEsc) != 0, (b.C % 8) == 0, b.k <= 5, sh, B, n_wg, st);
}

// Sum of the fused product's partial sums of row r for activation row t, in a fixed
// order (tiles, then chains of a tile, ascending), plus the bias; rounded to BF16 as the
// GEMM's epilogue rounds.
__global__ void matvec_finish_kernel(const float* __restrict__ part, const uint16_t* __restrict__ bias,
                                     uint16_t* __restrict__ y, int64_t T, int64_t R, int64_t G, int log2S,
                                     int64_t n_groups, int slots, int NT) {
  // thread (x, y): row r, activation row t (no division for either)
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, t = blockIdx.y;
  if (r >= R) return;
  const int64_t S = 1 << log2S;
  const int64_t g_lo = r * G, g_hi = (r + 1) * G;   // the row's groups
  float sum = 0.f;
  for (int64_t tile = g_lo >> 9; tile <= (g_hi - 1) >> 9; ++tile) {
    int64_t gt = n_groups - (tile << 9);
    if (gt > kTileGroups) gt = kTileGroups;
    // the row of the tile's first group; chain j starts S > j groups later, at most
    // one row further (G >= S)
    const int64_t rt = (tile << 9) / G, rem = (tile << 9) - rt * G;
    for (int64_t j = 0; j < S; ++j) {
      const int64_t g0 = (tile << 9) + j;
      const int64_t ngr = gt > j ? (gt - j + S - 1) >> log2S : 0;
      const int64_t k = g_lo > g0 ? (g_lo - g0 + S - 1) >> log2S : 0;   // first group at or past the row
      if (k >= ngr || g0 + (k << log2S) >= g_hi) continue;
      const int64_t ch = (tile << log2S) + j;
      const int64_t r0 = rt + (rem + j >= G ? 1 : 0);   // = g0 / G
      sum += part[(ch * slots + (r - r0)) * NT + t];
    }
  }
  if (bias) sum += __uint_as_float((uint32_t)bias[r] << 16);
  const __bf16 o = (__bf16)sum;
  y[t * R + r] = __builtin_bit_cast(uint16_t, o);
}

// Test hook: the container casts of the decoder applied to plain float inputs, one
// group of eight per thread (FP8 through the instruction or the bit manipulation).
template <int OUT, bool HW>
__global__ void cast_test_kernel(const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t base = g * 8;
  if (base >= n) return;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = base + i < n ? in[base + i] : 0.f;
  if constexpr (OUT == OUT_FP8) {
    const uint32_t lo = pack_fp8x4<HW>(v[0], v[1], v[2], v[3]), hi = pack_fp8x4<HW>(v[4], v[5], v[6], v[7]);
    for (int i = 0; i < 8 && base + i < n; ++i) out[base + i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
  } else {
    store_group<OUT>(out, base, v, nullptr, base + 8 <= n, n - base);
  }
}

}  // namespace

int test_cast(int dtype, const float* in, void* out, int64_t n, int hw, ep_stream stream) {
  hipStream_t st = (hipStream_t)stream;
  if (n < 0 || (n > 0 && (!in || !out))) return fail(EP_E_ARG, "null pointer or negative size");
  if (n == 0) return EP_OK;
  int rc;
  if ((rc = check_gpu_pointer(in, "input")) || (rc = check_gpu_pointer(out, "output"))) return rc;
  const dim3 grid((unsigned)((n + 8 * 256 - 1) / (8 * 256))), block(256);
  uint8_t* o = (uint8_t*)out;
  switch (dtype) {
    case EP_BF16: hipLaunchKernelGGL((cast_test_kernel<OUT_BF16_SAT, false>), grid, block, 0, st, in, o, n); break;
    case EP_FP16: hipLaunchKernelGGL((cast_test_kernel<OUT_FP16, false>), grid, block, 0, st, in, o, n); break;
    case EP_INT8: hipLaunchKernelGGL((cast_test_kernel<OUT_INT8, false>), grid, block, 0, st, in, o, n); break;
    case EP_FP8_E4M3FN:
      if (hw) hipLaunchKernelGGL((cast_test_kernel<OUT_FP8, true>), grid, block, 0, st, in, o, n);
      else hipLaunchKernelGGL((cast_test_kernel<OUT_FP8, false>), grid, block, 0, st, in, o, n);
      break;
    default: return fail(EP_E_DTYPE, "cast test takes BF16, FP16, FP8 or INT8");
  }
  return hip_check(hipGetLastError(), "cast test launch");
}

// Rows a chain's groups can touch: the chain's groups lie within its tile's 512
// consecutive groups, so at most 511 / G + 2 rows.
int matvec_slots(const Blob& b) { return (int)(511 / ((b.C + 7) / 8)) + 2; }

size_t matvec_workspace_bytes(const Blob& b, int64_t T) {
  const int nt = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
  return (size_t)b.n_chains * (size_t)matvec_slots(b) * (size_t)nt * 4 + 256;
}

// Rows of whole tiles (4096 or 8192 columns at S = 8): a row's chains sit in one wave, so
// the decode kernel sums them itself (same order and bits as matvec_finish_kernel) and no
// finishing launch follows.  EP_MATVEC_DIRECT=0 keeps the finishing kernel (comparisons).
bool matvec_direct(const Blob& b) {
  if (const char* e = std::getenv("EP_MATVEC_DIRECT"))
    if (std::atoi(e) == 0) return false;
  // (a row's chains, S per tile, one or two tiles a row, fill 8 to 32 consecutive lanes)
  return (b.S == 8 || b.S == 16) && (b.C == 8 * kTileGroups || b.C == 16 * kTileGroups);
}

bool matvec_supported(const Blob& b, int64_t T) {
  return b.kind == kKindLossy && b.dtype == EP_BF16 && T >= 1 && T <= kMatvecMaxT && b.C % 8 == 0 &&
         b.S <= (b.C + 7) / 8;
}

// Y_i[T x R_i] = X[T x C] W_i^T (+ bias_i) for blobs i < n sharing the activations, with
// each W_i decoded inside the product (never stored); part[i] (256-byte aligned,
// matvec_workspace_bytes - 256 bytes) holds blob i's partial sums.  The blobs' blocks
// share launches (by table layout and escape variant, up to kMaxBatch blobs each).
int matvec_batch_launch(const Blob* const* bs, int n, const void* x, int64_t T, const void* const* bias,
                        void* const* y, float* const* part, ep_stream stream, bool check_part) {
  hipStream_t st = (hipStream_t)stream;
  if (n < 1) return fail(EP_E_ARG, "empty batch");
  if (!x || (reinterpret_cast<uintptr_t>(x) & 15)) return fail(EP_E_ARG, "activations must be 16-byte aligned");
  int rc = check_gpu_pointer(x, "activations");
  if (rc) return rc;
  for (int i = 0; i < n; ++i) {
    const Blob& b = *bs[i];
    if ((rc = check_uploaded(b))) return rc;
    if (!matvec_supported(b, T))
      return fail(EP_E_ARG, "the fused product takes lossy BF16 blobs, 1..8 activation rows, C % 8 == 0 and at least S groups per row");
    if (b.C != bs[0]->C) return fail(EP_E_ARG, "blobs sharing activations need the same number of columns");
    if (!y[i] || !part[i]) return fail(EP_E_ARG, "null output or workspace");
    if ((rc = check_gpu_pointer(y[i], "output")) || (check_part && (rc = check_gpu_pointer(part[i], "workspace"))))
      return rc;
    if (bias && bias[i] && (rc = check_gpu_pointer(bias[i], "bias"))) return rc;
  }
  const int nt = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
  const int out = nt == 1 ? OUT_MV1 : nt == 2 ? OUT_MV2 : nt == 4 ? OUT_MV4 : OUT_MV8;
  // (no host allocation here: the launches' blob lists are fixed-size arrays, filled
  // in blob order per table layout and escape variant)
  for (int pass = 0; pass < 4; ++pass) {
    const bool narrow = pass < 2, pesc = (pass & 1) != 0;
    int idx[kMaxBatch];
    int m = 0;
    for (int i = 0; i <= n; ++i) {
      if (i < n && (bs[i]->k <= 5) == narrow && ((bs[i]->flags & kFlagEsc) != 0) == pesc) idx[m++] = i;
      if (m == 0 || (m < kMaxBatch && i < n)) continue;
      DecBatch B{};
      B.n = m;
      m = 0;
      int64_t nblk[kMaxBatch];
      for (int q = 0; q < B.n; ++q) nblk[q] = bs[idx[q]]->n_blocks;
      Shape sh = pick_shape(nblk, B.n);
      sh.ilp = 1;
      B.bpw = sh.bpw;
      int64_t wg = 0;
      for (int q = 0; q < B.n; ++q) {
        const int i = idx[q];
        const Blob& b = *bs[i];
        const bool direct = matvec_direct(b);
        DecJob j = make_job(b, direct ? y[i] : (void*)part[i]);
        j.mv_x = (const uint16_t*)x;
        j.mv_T = (uint32_t)T;
        j.mv_slots = (uint32_t)matvec_slots(b);
        j.mv_sat = (b.flags & kFlagSat) ? 1u : 0u;
        j.mv_direct = direct ? 1u : 0u;
        j.mv_lanes = (uint32_t)(b.C / (8 * kTileGroups)) * (uint32_t)b.S;
        j.bias = (const uint16_t*)(bias ? bias[i] : nullptr);
        j.wg_begin = wg;
        wg += (j.n_blocks + sh.bpw - 1) / sh.bpw;
        B.j[q] = j;
      }
      if ((rc = launch_any(out, pesc, true, narrow, sh, B, wg, st))) return rc;
    }
  }
  for (int i = 0; i < n; ++i) {
    const Blob& b = *bs[i];
    if (matvec_direct(b)) continue;   // summed inside the decode kernel
    hipLaunchKernelGGL(matvec_finish_kernel, dim3((unsigned)((b.R + 255) / 256), (unsigned)T), dim3(256), 0, st, part[i],
                       (const uint16_t*)(bias ? bias[i] : nullptr), (uint16_t*)y[i], T, b.R, (int64_t)((b.C + 7) / 8),
                       (int)__builtin_ctz((unsigned)b.S), b.n_groups(), matvec_slots(b), nt);
    if ((rc = hip_check(hipGetLastError(), "fused product finish launch"))) return rc;
  }
  return EP_OK;
}

int matvec_launch(const Blob& b, const void* x, int64_t T, const void* bias, void* y, float* part, ep_stream stream) {
  const Blob* bs[1] = {&b};
  const void* bi[1] = {bias};
  void* ys[1] = {y};
  float* ps[1] = {part};
  return matvec_batch_launch(bs, 1, x, T, bi, ys, ps, stream);
}

int matvec_forward(const Blob& b, const void* x, int64_t T, const void* bias, void* y, void* ws, size_t ws_bytes,
                   ep_stream stream) {
  if (!ws) return fail(EP_E_ARG, "null workspace");
  if (ws_bytes < matvec_workspace_bytes(b, T)) return fail(EP_E_WORKSPACE, "workspace too small");
  return matvec_launch(b, x, T, bias, y, (float*)(((uintptr_t)ws + 255) & ~uintptr_t(255)), stream);
}

// Decode for a GEMM that reads the weights next: BF16 stored through the caches
int gemm_out_kind(const Blob& b) {
  const int o = out_kind(b);
  return o == OUT_BF16 ? OUT_BF16_L2 : o;
}
int decompress_for_gemm(const Blob& b, void* dst, ep_stream st) {
  return decode_one(b, dst, 0, b.n_chains, gemm_out_kind(b), (hipStream_t)st);
}
int decompress_beside(const Blob& b, void* dst, ep_stream st, int64_t max_wg) {
  return decode_one(b, dst, 0, b.n_chains, gemm_out_kind(b), (hipStream_t)st, max_wg);
}

// ---------------------------------------------------------------- fused prefill product
bool prefill_supported(const Blob& b, int64_t T) {
  return b.kind == kKindLossy && b.dtype == EP_BF16 && b.S == 8 && (b.C == 8 * kTileGroups || b.C == 16 * kTileGroups) &&
         T >= 1 && T <= kPrefillMaxT;
}

template <int OUT>
int launch_mma(bool esc, bool narrow, const DecBatch& B, int64_t n_wg, hipStream_t st) {
  if (narrow)
    return esc ? launch_t<OUT, true, true, true, 1, false>(B, n_wg, kMmaWaves, st)
               : launch_t<OUT, false, true, true, 1, false>(B, n_wg, kMmaWaves, st);
  return esc ? launch_t<OUT, true, true, false, 1, false>(B, n_wg, kMmaWaves, st)
             : launch_t<OUT, false, true, false, 1, false>(B, n_wg, kMmaWaves, st);
}

int prefill_launch(const Blob& b, const void* x, int64_t T, const void* bias, void* y, ep_stream stream) {
  int rc = check_uploaded(b);
  if (rc) return rc;
  if (!prefill_supported(b, T))
    return fail(EP_E_ARG, "the fused prefill product takes lossy BF16 blobs of 4096 or 8192 columns at 8 chains "
                "per tile and 1.." + std::to_string(kPrefillMaxT) + " activation rows");
  if (!x || !y) return fail(EP_E_ARG, "null activations or output");
  if (reinterpret_cast<uintptr_t>(x) & 15) return fail(EP_E_ARG, "activations must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(y) & 7) || (reinterpret_cast<uintptr_t>(bias) & 1))
    return fail(EP_E_ARG, "output must be 8-byte aligned and bias 2-byte aligned");
  if ((rc = check_gpu_pointer(x, "activations")) || (rc = check_gpu_pointer(y, "output")) ||
      (bias && (rc = check_gpu_pointer(bias, "bias"))))
    return rc;
  DecJob j = make_job(b, y);
  j.mv_x = (const uint16_t*)x;
  j.mv_T = (uint32_t)T;
  j.mv_sat = (b.flags & kFlagSat) ? 1u : 0u;
  j.bias = (const uint16_t*)bias;
  DecBatch B{};
  B.j[0] = j;
  B.n = 1;
  B.bpw = kMmaWaves;   // one block (8 rows of W) per wave
  const int64_t n_wg = (b.n_blocks + kMmaWaves - 1) / kMmaWaves;
  const bool esc = (b.flags & kFlagEsc) != 0, narrow = b.k <= 5;
  const hipStream_t st = (hipStream_t)stream;
  if (b.C == 8 * kTileGroups)
    return T <= kPrefillMaxT / 2 ? launch_mma<OUT_MMA1>(esc, narrow, B, n_wg, st)
                                 : launch_mma<OUT_MMA2>(esc, narrow, B, n_wg, st);
  return T <= kPrefillMaxT / 2 ? launch_mma<OUT_MMA1X2>(esc, narrow, B, n_wg, st)
                               : launch_mma<OUT_MMA2X2>(esc, narrow, B, n_wg, st);
}

// ---------------------------------------------------------------- the fused product without a workspace
// Partial sums of ep_compressed_matvec_noalloc: one file-scope device array (every GPU the
// library runs on holds its own copy until the process ends).  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxScratchDevices] = {};

static int scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return fail(EP_E_DEVICE, "no current device for the scratch array");
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(EP_E_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = (float*)g_scratch_ptr[dev];
  return EP_OK;
}

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
  // the decoder addresses stream words with 32-bit indices
  if (b.n_words >= ((uint64_t)1 << 31)) return fail(EP_E_ARG, "stream too long for the device decoder (2^31 words)");
  auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
  // decode tables: TileANS byte tables; split entries (two words a slot) for lossy blobs
  // with escape threshold <= 64 and no escape; packed entries otherwise (M slots a table)
  const bool split = b.kind != kKindTileAns && b.k <= 5 && !(b.flags & kFlagEsc);
  const int M = 1 << precision(b.k);
  const size_t tab_words = b.kind == kKindTileAns ? (size_t)b.n_ctx * kMBytes
                                                  : (size_t)kNumCtx * M * (split ? 2 : 1);
  const size_t o_tab = 0;
  const size_t o_hr = o_tab + al(4 * tab_words);
  // the chain area as stored (block offsets, chunk counts, tail nibbles, states), each
  // section 256-byte aligned; the kernel derives every chain's offsets from it
  const size_t fw = b.S >= 8 ? 1 : 2, n_nib = ((size_t)b.n_chains + 1) / 2;
  const size_t o_boff = o_hr + al(4 * ((size_t)b.R + kHrPad));
  const size_t o_full = o_boff + al(4 * (size_t)b.n_blocks);
  const size_t o_nib = o_full + al(fw * (size_t)b.n_chains);
  const size_t o_states = o_nib + al(n_nib);
  const size_t o_err = o_states + al(4 * (size_t)b.n_chains);
  const size_t o_stream = o_err + 256;
  const size_t total = o_stream + al(2 * (size_t)b.n_words + 256);
  std::vector<uint8_t> host;
  try {
    host.assign(total, 0);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  if (b.kind == kKindTileAns) {
    build_byte_tables(b.LF, b.n_ctx, (uint32_t*)&host[o_tab]);   // (no row scales: zeros)
  } else {
    if (split) build_split_tables(b.model, (uint32_t*)&host[o_tab]);
    else build_slot_tables(b.model, (uint32_t*)&host[o_tab], b.k <= 5);
    half_scales(b, (float*)&host[o_hr]);
    // (the escape-free narrow kernel reconstructs fma(u + 128, h, -128 h), which needs
    // -128 h finite; rows beyond that take the plain product h u)
    const float* hr = (const float*)&host[o_hr];
    for (int64_t r = 0; r < b.R; ++r)
      if (!(std::fabs(hr[r]) < 3.4028234663852886e38f / 128.f)) b.d_big_h = true;
  }
  std::memcpy(&host[o_boff], &b.bytes[b.off_boff], 4 * (size_t)b.n_blocks);
  std::memcpy(&host[o_full], &b.bytes[b.off_full], fw * (size_t)b.n_chains);
  std::memcpy(&host[o_nib], &b.bytes[b.off_tail], n_nib);
  std::memcpy(&host[o_states], &b.bytes[b.off_states], 4 * (size_t)b.n_chains);
  std::memcpy(&host[o_stream], &b.bytes[b.off_stream], 2 * (size_t)b.n_words);
  void* d = nullptr;
  if (hipMalloc(&d, total) != hipSuccess) {
    (void)hipGetLastError();
    return fail(EP_E_NOMEM, "device allocation failed");
  }
  uint8_t* p = (uint8_t*)d;
  b.d_tab = (const uint32_t*)(p + o_tab);
  b.d_hr = (const float*)(p + o_hr);
  b.d_boff = (const uint32_t*)(p + o_boff);
  b.d_full = (const void*)(p + o_full);
  b.d_nib = (const uint8_t*)(p + o_nib);
  b.d_states = (const uint32_t*)(p + o_states);
  b.d_err = (uint32_t*)(p + o_err);
  b.d_stream = (const uint16_t*)(p + o_stream);
  int rc = hip_check(hipMemcpyAsync(d, host.data(), total, hipMemcpyHostToDevice, (hipStream_t)stream), "upload");
  if (!rc) rc = hip_check(hipStreamSynchronize((hipStream_t)stream), "upload sync");
  if (rc) {
    (void)hipFree(d);
    b.d_tab = nullptr;
    b.d_hr = nullptr;
    b.d_boff = nullptr;
    b.d_full = nullptr;
    b.d_nib = nullptr;
    b.d_states = nullptr;
    b.d_err = nullptr;
    b.d_stream = nullptr;
    return rc;
  }
  (void)hipGetDevice(&b.device);
  b.d_base = d;
  b.d_bytes = total;
  b.d_tab_words = (uint32_t)tab_words;
  return EP_OK;
}

size_t ep_device_bytes(const ep_blob* blob) { return blob ? blob->b.d_bytes : 0; }

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

int ep_test_cast(int dtype, const float* dev_in, void* dev_out, int64_t n, int hw, ep_stream stream) {
  set_error("");
  return test_cast(dtype, dev_in, dev_out, n, hw, stream);
}

int ep_test_decode_coords(const ep_blob* blob, int32_t* dev_u, ep_stream stream) {
  set_error("");
  if (!blob) return fail(EP_E_ARG, "null blob");
  const Blob& b = blob->b;
  if (b.kind != kKindLossy) return fail(EP_E_ARG, "lattice coordinates exist for lossy blobs only");
  return decode_one(b, dev_u, 0, b.n_chains, OUT_COORDS, (hipStream_t)stream);
}

int ep_decompress_batch(const ep_blob* const* blobs, void* const* dsts, int n, ep_stream stream) {
  set_error("");
  if (n < 0 || (n > 0 && (!blobs || !dsts))) return fail(EP_E_ARG, "null pointer");
  if (n == 0) return EP_OK;
  // all blobs of one call share the container kind
  int out = -1;
  for (int i = 0; i < n; ++i) {
    if (!blobs[i] || !dsts[i]) return fail(EP_E_ARG, "null blob or destination");
    const Blob& b = blobs[i]->b;
    int rc = check_uploaded(b);
    if (rc) return rc;
    if (reinterpret_cast<uintptr_t>(dsts[i]) & 15) return fail(EP_E_ARG, "destination must be 16-byte aligned");
    if ((rc = check_gpu_pointer(dsts[i], "destination"))) return rc;
    const int o = out_kind(b);
    if (out < 0) out = o;
    else if ((out == OUT_BF16 || out == OUT_BF16_SAT) && (o == OUT_BF16 || o == OUT_BF16_SAT))
      out = (out == OUT_BF16_SAT || o == OUT_BF16_SAT) ? OUT_BF16_SAT : OUT_BF16;
    else if (o != out) return fail(EP_E_ARG, "batch mixes container dtypes");
  }
  // Blobs go to separate launches by table layout (narrow / wide entries) and by
  // whether they hold escapes (the kernel without the escape path is faster), each of
  // up to kMaxBatch blobs with its own launch shape.
  for (int pass = 0; pass < 4; ++pass) {
    const bool narrow = pass < 2;
    const bool pesc = (pass & 1) != 0;
    std::vector<int> idx;
    bool pc8 = true;
    for (int i = 0; i < n; ++i) {
      const Blob& b = blobs[i]->b;
      if ((b.k <= 5) == narrow && ((b.flags & kFlagEsc) != 0) == pesc) {
        idx.push_back(i);
        pc8 &= (b.C % 8) == 0;
      }
    }
    for (size_t i0 = 0; i0 < idx.size(); i0 += kMaxBatch) {
      DecBatch B{};
      B.n = (int)std::min<size_t>(kMaxBatch, idx.size() - i0);
      int64_t nblk[kMaxBatch];
      for (int q = 0; q < B.n; ++q) nblk[q] = blobs[idx[i0 + q]]->b.n_blocks;
      const Shape sh = pick_shape(nblk, B.n);
      B.bpw = sh.bpw;
      int64_t wg = 0;
      for (int q = 0; q < B.n; ++q) {
        B.j[q] = make_job(blobs[idx[i0 + q]]->b, dsts[idx[i0 + q]]);
        B.j[q].wg_begin = wg;
        wg += (B.j[q].n_blocks + sh.bpw - 1) / sh.bpw;
      }
      int rc = launch_any(out, pesc, pc8, narrow, sh, B, wg, (hipStream_t)stream);
      if (rc) return rc;
    }
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

int ep_compressed_linear_prefill(const ep_blob* w, const void* x, int64_t T, const void* bias, void* y,
                                 ep_stream stream) {
  set_error("");
  if (!w) return fail(EP_E_ARG, "null blob");
  return prefill_launch(w->b, x, T, bias, y, stream);
}

// The fused product with its partial sums in the library's scratch array (no allocation,
// no workspace argument).  Every slot the finishing kernel reads is written by the
// decode kernel of the same call, so nothing needs clearing between calls.
int ep_compressed_matvec_noalloc(const ep_blob* w, const void* x, int64_t T, const void* bias, void* y,
                                 ep_stream stream) {
  set_error("");
  if (!w || !x || !y) return fail(EP_E_ARG, "null pointer");
  const Blob& b = w->b;
  if (!matvec_supported(b, T))
    return fail(EP_E_ARG, "the fused product takes lossy BF16 blobs, 1..8 activation rows, C % 8 == 0 and at least S groups per row");
  const size_t need = matvec_workspace_bytes(b, T) - 256;
  if (need > kScratchBytes)
    return fail(EP_E_WORKSPACE, "partial sums of " + std::to_string(need) + " bytes exceed the 16 MiB scratch array "
                "(use ep_compressed_matvec with a workspace)");
  float* part = nullptr;
  int rc = scratch_address(&part);
  if (rc) return rc;
  const Blob* bs[1] = {&b};
  const void* bi[1] = {bias};
  void* ys[1] = {y};
  float* ps[1] = {part};
  return matvec_batch_launch(bs, 1, x, T, bi, ys, ps, stream, false);
}

}  // extern "C"
