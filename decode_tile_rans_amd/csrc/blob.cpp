// Blob v2 parsing / validation and the host-only C ABI entry points.
//
// Layout (little-endian, packed; this project's format — the pages only say the
// stream is tile-wise rANS and that actual_bpp counts metadata, [README] 快速开始):
//   header 48 B | bf16 row scales[R] | model | u32 block offsets[n_blocks] (chunks) |
//   full chunks per chain (u8 if S >= 8, else u16)[n_chains] |
//   tail lengths (4 bits per chain, chain 2i in the low nibble)[ceil(n_chains/2)] |
//   u32 states[n_chains] | u16 stream[n_words]
// A block area is [tile main areas (chunks in request order)][tails][pad to 8 words].
#include <cmath>

#include "ep_internal.h"

namespace ep {

const char* last_error_cstr();

namespace {
template <class T>
T rd(const std::vector<uint8_t>& b, size_t off) {
  T v;
  std::memcpy(&v, &b[off], sizeof(T));
  return v;
}
}  // namespace

namespace {
// The chain area (block offsets, chunk counts, tails, states, stream) from `off` to the
// end of the blob; shared by both kinds.
int parse_area(Blob& b, size_t off) {
  const auto& by = b.bytes;
  const int64_t ng = b.n_groups();
  if (b.n_tiles != std::max<int64_t>(1, (ng + kTileGroups - 1) / kTileGroups)) return fail(EP_E_CORRUPT, "bad tile count");
  b.n_chains = b.n_tiles * b.S;
  if (b.n_blocks != (b.n_chains + kBlockChains - 1) / kBlockChains) return fail(EP_E_CORRUPT, "bad block count");
  const size_t fw = b.S >= 8 ? 1 : 2;
  const size_t n_nib = (size_t)((b.n_chains + 1) / 2);
  b.off_boff = off;
  b.off_full = b.off_boff + 4 * (size_t)b.n_blocks;
  b.off_tail = b.off_full + fw * (size_t)b.n_chains;
  b.off_states = b.off_tail + n_nib;
  b.off_stream = b.off_states + 4 * (size_t)b.n_chains;
  if (b.n_words > (uint64_t)1 << 40 || by.size() != b.off_stream + 2 * (size_t)b.n_words)
    return fail(EP_E_CORRUPT, "blob size mismatch");
  b.chain_len.assign((size_t)b.n_chains, 0);
  for (int64_t c = 0; c < b.n_chains; ++c) {
    const uint32_t full = fw == 1 ? by[b.off_full + (size_t)c] : rd<uint16_t>(by, b.off_full + 2 * (size_t)c);
    const uint32_t tail = (by[b.off_tail + (size_t)(c / 2)] >> (4 * (c & 1))) & 15u;
    if (tail >= 8) return fail(EP_E_CORRUPT, "bad tail length");
    b.chain_len[c] = 8 * full + tail;
  }
  if ((b.n_chains & 1) && (by[b.off_tail + n_nib - 1] >> 4)) return fail(EP_E_CORRUPT, "bad tail length");
  uint64_t chunks = 0;
  for (int64_t bk = 0; bk < b.n_blocks; ++bk) {
    if (rd<uint32_t>(by, b.off_boff + 4 * (size_t)bk) != chunks) return fail(EP_E_CORRUPT, "block offset mismatch");
    const int64_t c1 = std::min<int64_t>(b.n_chains, (bk + 1) * kBlockChains);
    uint64_t words = 0;
    for (int64_t c = bk * kBlockChains; c < c1; ++c) words += b.chain_len[c];
    chunks += (words + 7) / 8;
    if (chunks > 0xFFFFFFFFull) return fail(EP_E_CORRUPT, "stream too long");
  }
  if (8 * chunks != b.n_words) return fail(EP_E_CORRUPT, "chain lengths do not cover the stream");
  for (int64_t c = 0; c < b.n_chains; ++c)
    if (rd<uint32_t>(by, b.off_states + 4 * (size_t)c) < kL) return fail(EP_E_CORRUPT, "state below L");
  return EP_OK;
}

// TileANS header: 'EPT1' u16 ver=1 | u8 tag | u8 E | u8 P | u8 S | u8 ndim | u8 uniform
// mask | u8 tile_log2=12 | 3 x 0 | u64 n_bytes | u32 n_tiles | u32 n_blocks | u64 n_words
// | u64 0, then u64 dims[ndim], u16[256] per non-uniform context, the chain area.
int parse_tileans(Blob& b) {
  const auto& by = b.bytes;
  if (rd<uint16_t>(by, 4) != 1) return fail(EP_E_CORRUPT, "unsupported version");
  b.kind = kKindTileAns;
  b.dtype = by[6];
  b.E = by[7];
  const int P = by[8];
  b.S = by[9];
  const int ndim = by[10];
  b.umask = by[11];
  if (P != kPBytes || by[12] != 12 || by[13] || by[14] || by[15] || rd<uint64_t>(by, 40) != 0)
    return fail(EP_E_CORRUPT, "bad header constants");
  if (b.E != 1 && b.E != 2 && b.E != 4 && b.E != 8) return fail(EP_E_CORRUPT, "bad element size");
  b.n_ctx = b.E < 4 ? b.E : 4;
  if (b.S < 1 || b.S > 64 || (b.S & (b.S - 1))) return fail(EP_E_CORRUPT, "bad chains per tile");
  if (ndim < 1 || ndim > 8 || (b.umask >> b.n_ctx)) return fail(EP_E_CORRUPT, "bad header fields");
  const uint64_t n_bytes = rd<uint64_t>(by, 16);
  b.n_tiles = rd<uint32_t>(by, 24);
  b.n_blocks = rd<uint32_t>(by, 28);
  b.n_words = rd<uint64_t>(by, 32);
  size_t off = kHeaderBytes;
  if (by.size() < off + 8 * (size_t)ndim) return fail(EP_E_CORRUPT, "blob truncated");
  __int128 prod = b.E;
  b.dims.clear();
  for (int d = 0; d < ndim; ++d, off += 8) {
    const uint64_t v = rd<uint64_t>(by, off);
    if (v < 1 || v > ((uint64_t)1 << 40)) return fail(EP_E_CORRUPT, "bad shape");
    prod *= (__int128)v;
    if (prod > ((__int128)1 << 40)) return fail(EP_E_CORRUPT, "bad shape");
    b.dims.push_back((int64_t)v);
  }
  if ((uint64_t)prod != n_bytes) return fail(EP_E_CORRUPT, "bad shape");
  b.R = 1;
  b.C = (int64_t)n_bytes;
  for (int c = 0; c < b.n_ctx; ++c) {
    int32_t sum = 0;
    if ((b.umask >> c) & 1) {
      for (int v = 0; v < 256; ++v) b.LF[c][v] = kMBytes / 256;
      continue;
    }
    if (by.size() < off + 512) return fail(EP_E_CORRUPT, "blob truncated");
    for (int v = 0; v < 256; ++v, off += 2) {
      b.LF[c][v] = rd<uint16_t>(by, off);
      sum += b.LF[c][v];
    }
    if (sum != kMBytes) return fail(EP_E_CORRUPT, "table does not sum to 2048");
  }
  return parse_area(b, off);
}
}  // namespace

int parse_blob(std::vector<uint8_t>&& bytes, Blob* out) {
  Blob& b = *out;
  b.bytes = std::move(bytes);
  const auto& by = b.bytes;
  if (by.size() < (size_t)kHeaderBytes) return fail(EP_E_CORRUPT, "blob truncated");
  if (std::memcmp(&by[0], "EPT1", 4) == 0) return parse_tileans(b);
  if (std::memcmp(&by[0], "EPK1", 4) != 0) return fail(EP_E_CORRUPT, "bad magic");
  if (rd<uint16_t>(by, 4) != 3) return fail(EP_E_CORRUPT, "unsupported version");
  b.dtype = by[6];
  int P = by[7];
  b.S = by[8];
  b.k = by[9];
  b.flags = by[10];
  int tl = by[11];
  b.R = rd<uint32_t>(by, 12);
  b.C = rd<uint32_t>(by, 16);
  b.delta = rd<float>(by, 20);
  b.n_tiles = rd<uint32_t>(by, 24);
  b.n_blocks = rd<uint32_t>(by, 28);
  b.n_words = rd<uint64_t>(by, 32);
  b.model_bytes = rd<uint32_t>(by, 40);
  if (tl != 12 || rd<uint32_t>(by, 44) != 0) return fail(EP_E_CORRUPT, "bad header constants");
  if (b.dtype < EP_BF16 || b.dtype > EP_INT8) return fail(EP_E_CORRUPT, "bad dtype");
  if (b.S < 1 || b.S > 64 || (b.S & (b.S - 1))) return fail(EP_E_CORRUPT, "bad chains per tile");
  if (b.k < 3 || b.k > 7 || b.flags > 3) return fail(EP_E_CORRUPT, "bad header fields");
  if (P != precision(b.k)) return fail(EP_E_CORRUPT, "table precision does not match the escape threshold");
  if (b.R < 1 || b.C < 1) return fail(EP_E_CORRUPT, "bad shape");
  if (!(std::isfinite(b.delta) && b.delta > 0.f)) return fail(EP_E_CORRUPT, "bad resolution");
  b.off_scales = kHeaderBytes;
  b.off_model = b.off_scales + 2 * (size_t)b.R;
  if (by.size() < b.off_model + b.model_bytes) return fail(EP_E_CORRUPT, "blob size mismatch");
  int rc = parse_area(b, b.off_model + b.model_bytes);
  if (rc) return rc;
  for (int64_t r = 0; r < b.R; ++r) {
    uint16_t s = rd<uint16_t>(by, b.off_scales + 2 * (size_t)r);
    if ((s & 0x8000) || ((s >> 7) & 0xFF) == 0xFF) return fail(EP_E_CORRUPT, "bad row scale");
  }
  std::string err;
  if (!Model::from_bytes(&by[b.off_model], b.model_bytes, b.k, &b.model, &err)) return fail(EP_E_CORRUPT, err);
  return EP_OK;
}

void half_scales(const Blob& b, float* hr) {
  for (int64_t r = 0; r < b.R; ++r) {
    uint16_t s;
    std::memcpy(&s, &b.bytes[b.off_scales + 2 * (size_t)r], 2);
    hr[r] = bf16_to_f32(s) * b.delta;
  }
}

}  // namespace ep

using namespace ep;

void ep_device_release(ep::Blob* b);   // decode.hip

extern "C" {

int ep_compress_ex(const void* src, int dtype, int64_t rows, int64_t cols, double target_bpp, int S,
                   ep_blob** out) {
  set_error("");
  if (!out) return fail(EP_E_ARG, "null output pointer");
  *out = nullptr;
  std::vector<uint8_t> bytes;
  Distortion dist;
  int rc = ep::compress(src, dtype, rows, cols, target_bpp, S, &bytes, &dist);
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

int ep_compress(const void* src, int dtype, int64_t rows, int64_t cols, double target_bpp, ep_blob** out) {
  return ep_compress_ex(src, dtype, rows, cols, target_bpp, 0, out);
}

int ep_compress_lossless(const void* src, int64_t n_bytes, int elem_bytes, const int64_t* dims, int ndim,
                         int dtype_tag, int chains_per_tile, ep_blob** out) {
  set_error("");
  if (!out) return fail(EP_E_ARG, "null output pointer");
  *out = nullptr;
  std::vector<uint8_t> bytes;
  int rc = ep::compress_lossless(src, n_bytes, elem_bytes, dims, ndim, dtype_tag, chains_per_tile, &bytes);
  if (rc) return rc;
  ep_blob* blob = new (std::nothrow) ep_blob();
  if (!blob) return fail(EP_E_NOMEM, "out of host memory");
  rc = parse_blob(std::move(bytes), &blob->b);
  if (rc) {
    delete blob;
    return rc;
  }
  *out = blob;
  return EP_OK;
}

int ep_blob_kind(const ep_blob* blob) { return blob ? blob->b.kind : -1; }

int ep_blob_dims(const ep_blob* blob, int64_t* dims, int max_dims) {
  if (!blob) return 0;
  const Blob& b = blob->b;
  if (b.kind == kKindTileAns) {
    for (int d = 0; d < (int)b.dims.size() && d < max_dims; ++d) dims[d] = b.dims[d];
    return (int)b.dims.size();
  }
  if (max_dims > 0) dims[0] = b.R;
  if (max_dims > 1) dims[1] = b.C;
  return 2;
}

int ep_blob_elem_bytes(const ep_blob* blob) {
  if (!blob) return 0;
  const Blob& b = blob->b;
  if (b.kind == kKindTileAns) return b.E;
  return b.dtype == EP_FP32 ? 4 : ((b.dtype == EP_FP8_E4M3FN || b.dtype == EP_INT8) ? 1 : 2);
}

int ep_deserialize(const void* src, size_t size, ep_blob** out) {
  set_error("");
  if (!out || (!src && size)) return fail(EP_E_ARG, "null pointer");
  *out = nullptr;
  ep_blob* blob = new (std::nothrow) ep_blob();
  if (!blob) return fail(EP_E_NOMEM, "out of host memory");
  std::vector<uint8_t> bytes((const uint8_t*)src, (const uint8_t*)src + size);
  int rc = parse_blob(std::move(bytes), &blob->b);
  if (rc) {
    delete blob;
    return rc;
  }
  *out = blob;
  return EP_OK;
}

size_t ep_serialized_size(const ep_blob* blob) { return blob ? blob->b.bytes.size() : 0; }

int ep_serialize(const ep_blob* blob, void* dst, size_t cap) {
  if (!blob || !dst) return fail(EP_E_ARG, "null pointer");
  if (cap < blob->b.bytes.size()) return fail(EP_E_ARG, "destination too small");
  std::memcpy(dst, blob->b.bytes.data(), blob->b.bytes.size());
  return EP_OK;
}

double ep_actual_bpp(const ep_blob* blob) {
  if (!blob) return 0.0;
  const Blob& b = blob->b;
  const double n = b.kind == kKindTileAns ? (double)(b.C / b.E) : (double)b.R * (double)b.C;
  return 8.0 * (double)b.bytes.size() / n;
}

void ep_blob_shape(const ep_blob* blob, int64_t* rows, int64_t* cols) {
  const bool ta = blob && blob->b.kind == kKindTileAns;
  if (rows) *rows = blob ? (ta ? 1 : blob->b.R) : 0;
  if (cols) *cols = blob ? (ta ? blob->b.C / blob->b.E : blob->b.C) : 0;
}

int ep_blob_dtype(const ep_blob* blob) { return blob ? blob->b.dtype : 0; }

void ep_blob_params(const ep_blob* blob, int* S, int* k, int* flags) {
  if (S) *S = blob ? blob->b.S : 0;
  if (k) *k = blob ? blob->b.k : 0;
  if (flags) *flags = blob ? blob->b.flags : 0;
}

void ep_blob_free(ep_blob* blob) {
  if (!blob) return;
  ep_device_release(&blob->b);
  delete blob;
}

const char* ep_last_error(void) { return ep::last_error_cstr(); }

}  // extern "C"
