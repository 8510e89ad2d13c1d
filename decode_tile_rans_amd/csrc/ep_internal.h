// Internal declarations shared by the host encoder, the blob code and the HIP
// decode/GEMM units of libentropack_hip.so.
//
// Format constants (this project's reading of the pages; see include/entropack.h
// for the page keys):
//   M = 2^P slots per table, P = 10 when the escape threshold K = 2^k is at most 32 and
//   P = 11 when K >= 64; 32-bit rANS state in [2^16, 2^32), 16-bit words;
//   tiles of 512 groups x 8 columns (4096 coordinates), S chains per tile, chain j
//   decodes the tile's groups j, j+S, ...; a block of 64 chains stores its tiles'
//   8-word chunks in the order the decoder requests them, then the chains' short
//   tails; one u32 offset per block, one full-chunk count and one tail length per
//   chain.
#pragma once
#include <cstdint>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

#include "../../include/entropack.h"

namespace ep {

constexpr int kPMax = 11;
constexpr int kMMax = 1 << kPMax;    // the largest tables: 2048 slots
// table precision of a lossy blob with escape threshold 2^k
inline int precision(int k) { return k >= 6 ? 11 : 10; }
// TileANS byte tables: P = 11
constexpr int kPBytes = 11;
constexpr int kMBytes = 1 << kPBytes;
constexpr int kNumCtx = 7;
constexpr int kIdSpace = 1024;
constexpr int kMaxE = 28;
constexpr uint32_t kL = 1u << 16;
constexpr int kTileGroups = 512;
constexpr int kBlockChains = 64;
constexpr int kHeaderBytes = 48;
constexpr uint8_t kFlagEsc = 1;
constexpr uint8_t kFlagSat = 2;

inline int n_msym(int k) { return (1 << k) + 4 * (kMaxE + 1 - k); }

// thread-local error message
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);

// Frequency quantiser Q (see model.cpp).
void quantize_freqs(const int64_t* w, int n, int total, int32_t* f_out);

// Stored model + derived decode frequencies for the 7 contexts.
struct Model {
  int k = 3;
  int nm = 0;
  int P = 10, M = 1024;                // table precision and slots (precision(k))
  int w[2] = {0, 0};
  std::vector<int32_t> g[2];           // magnitude frequencies (sum M / 2)
  int32_t F[kNumCtx][kIdSpace];        // frequency per symbol id
  int32_t CUM[kNumCtx][kIdSpace];      // first slot per symbol id
  bool last_ok(int c, int pi, int sid) const;
  void derive();                       // fill F, CUM from w, g
  std::vector<uint8_t> to_bytes() const;
  static bool from_bytes(const uint8_t* p, size_t n, int k, Model* out, std::string* err);
};

Model build_model(int k, const int64_t coset_counts[2], const int64_t* mag0, const int64_t* mag1);

extern const int32_t* log2q_table();   // floor(2^16 log2 f + 1/2), f in [0, 2048] (any precision)

// Packed decode-table entry (device tables, one u32 per slot, M slots per table):
//   bits  0..10  f      (1..M-1)
//   bits 11..21  bias   (slot - cum)
//   wide layout (K >= 64):
//     bits 22..30  direct symbol: doubled coordinate u (signed 9 bit; bit 22 = coset,
//                  bit 23 = parity of floor(u/2)); escape: c | neg<<1 | (e-2)<<2 | top2<<7
//     bit  31      escape (bucket symbol: raw bits follow)
//   narrow layout (K <= 32, |u| <= 127):
//     bit 22 coset, bit 23 escape, bits 24..31 u + 128 (direct) or
//     (e-2) | top2<<5 | neg<<7 (escape)
void build_slot_tables(const Model& m, uint32_t* out /* 7*M */, bool narrow);
// Split entries for narrow blobs without escapes (two u32 per slot, 7*M pairs): the
// first holds f in bits 0..9 (bits 10..23 zero, so a 24-bit multiply takes it as is)
// and u + 128 in bits 24..31 (bit 24 = coset, bit 25 = parity of floor(u/2)), the
// second the bias alone, so that x' = f (x >> P) + bias needs no field extraction.
void build_split_tables(const Model& m, uint32_t* out /* 2*7*M */);
// TileANS entries: f | bias << 11 | byte << 24, one 2048-slot table per context
void build_byte_tables(const int32_t (*F)[256], int n_ctx, uint32_t* out /* n_ctx*kMBytes */);

// Squared error of the lattice reconstruction fl32(h_r u) against the input, and the
// input's squared norm (both over all rows x cols entries).
struct Distortion {
  double sq_err = -1.0, sq_ref = -1.0;
};
int compress(const void* src, int dtype, int64_t R, int64_t C, double t, int S_req, std::vector<uint8_t>* out,
             Distortion* dist);
// Sampled storage estimate (2^-16 bits) at one resolution, and the k it chose.
struct Estimate {
  int64_t est;
  int k;
};
bool resolution_admissible(const float* s, const double* amax, int64_t R, float delta);
void select_resolution(double t, int64_t T, int jmin, const std::function<Estimate(uint32_t)>& estimate_at,
                       uint32_t* dbits, int* k);
// TileANS (lossless) blob of a tensor's raw bytes.
int compress_lossless(const void* src, int64_t n_bytes, int E, const int64_t* dims, int ndim, int tag, int S_req,
                      std::vector<uint8_t>* out);
constexpr int kKindLossy = 0;
constexpr int kKindTileAns = 1;

// Parsed blob (host side) + device mirror.  A TileANS blob is held as one row of
// n_bytes "columns" (R = 1, C = n_bytes: the same groups, tiles and chains as a
// lossy blob of that shape); `dtype` is then the caller's opaque tag.
struct Blob {
  std::vector<uint8_t> bytes;          // serialized form
  int kind = kKindLossy;
  int dtype = 0, S = 0, k = 0, flags = 0;
  int64_t R = 0, C = 0;
  // TileANS only
  int E = 0, n_ctx = 0, umask = 0;
  std::vector<int64_t> dims;
  int32_t LF[4][256];                  // per-context byte frequencies (sum kMBytes)
  float delta = 0.f;
  int64_t n_tiles = 0, n_blocks = 0, n_chains = 0;
  uint64_t n_words = 0;
  size_t off_scales = 0, off_model = 0, off_boff = 0, off_full = 0, off_tail = 0, off_states = 0,
         off_stream = 0;
  uint32_t model_bytes = 0;
  Model model;
  std::vector<uint32_t> chain_len;     // words per chain
  Distortion dist;                     // known for blobs made by ep_compress in this process
  // device mirror
  int device = -1;
  void* d_base = nullptr;              // one allocation
  const uint16_t* d_stream = nullptr;
  size_t d_bytes = 0;                  // size of the device allocation
  uint32_t d_tab_words = 0;            // u32 words of its decode tables
  bool d_big_h = false;                // some row half-scale h_r has |128 h_r| beyond float range
  const uint32_t* d_boff = nullptr;    // the stored chain area: block offsets (u32),
  const void* d_full = nullptr;        //   full chunks per chain (u8 at S >= 8, else u16),
  const uint8_t* d_nib = nullptr;      //   tail nibbles,
  const uint32_t* d_states = nullptr;  //   initial states
  const float* d_hr = nullptr;         // per-row half scales h_r
  const uint32_t* d_tab = nullptr;     // decode tables (build_slot_tables / build_split_tables)
  uint32_t* d_err = nullptr;
  int64_t n_groups() const { return R * ((C + 7) / 8); }
};

// Parse + validate serialized bytes (takes ownership of `bytes`).
int parse_blob(std::vector<uint8_t>&& bytes, Blob* out);

// Host reference pieces reused by upload: h_r = fl32(s_r * delta).
void half_scales(const Blob& b, float* hr_out);

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  return uint16_t((uint64_t(u) + 0x7FFFu + lsb) >> 16);
}

int hip_check(int err, const char* what);
// EP_E_ARG unless the GPU can dereference p (device, managed or pinned host memory)
int check_gpu_pointer(const void* p, const char* what);

int test_cast(int dtype, const float* in, void* out, int64_t n, int hw, ep_stream stream);

// Fused matrix-vector product of a lossy BF16 blob (decode.hip): up to kMatvecMaxT
// activation rows; the weights are decoded and multiplied in one kernel.
constexpr int64_t kMatvecMaxT = 8;
bool matvec_supported(const Blob& b, int64_t T);
size_t matvec_workspace_bytes(const Blob& b, int64_t T);
// (check_part = false only for the library's own scratch array, which the runtime's
// pointer query does not describe as an allocation)
int matvec_batch_launch(const Blob* const* bs, int n, const void* x, int64_t T, const void* const* bias,
                        void* const* y, float* const* part, ep_stream st, bool check_part = true);
int matvec_launch(const Blob& b, const void* x, int64_t T, const void* bias, void* y, float* part, ep_stream st);
int matvec_forward(const Blob& b, const void* x, int64_t T, const void* bias, void* y, void* ws, size_t ws_bytes,
                   ep_stream st);
// Decode the whole blob with at most max_wg workgroups (one per CU): a launch that runs
// beside another kernel which holds the other CUs.
int decompress_beside(const Blob& b, void* dst, ep_stream st, int64_t max_wg);
// the whole blob for a GEMM that reads the weights next (stores kept in the caches)
int decompress_for_gemm(const Blob& b, void* dst, ep_stream st);
// Fused prefill product (decode.hip): Y = X W^T (+ bias) for 1..256 activation rows with
// W decoded into LDS operand tiles of an MFMA product (4096 or 8192 columns, S = 8); no workspace.
bool prefill_supported(const Blob& b, int64_t T);
int prefill_launch(const Blob& b, const void* x, int64_t T, const void* bias, void* y, ep_stream st);

}  // namespace ep

struct ep_blob {
  ep::Blob b;
};
