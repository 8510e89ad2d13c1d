// Host encoder: ep_compress.
//
// Steps ([ABS]: row-normalised E8 quantisation, conditional model, sampled rate
// selection, tile entropy coding; [README] 快速开始: target_bpp in [0.001, 11],
// actual_bpp includes metadata; [NEWS]: 2-D tensors only):
//   1. validate; widen the container values to double
//   2. row scale s_r = BF16(fl32(sqrt(sum_c w^2 / C))), sum left to right
//   3. resolution: half-step delta (float32) found by bracketing over powers of two and
//      bisecting the float32 bit pattern, each probe estimating the sample's code
//      length with the sample's own tables (no full encode per probe)
//   4. quantise every 8-wide group: y = w / (2 h_r), h_r = fl32(s_r delta); nearest E8
//      point (Conway & Sloane 1982 decoder), doubled coordinates u = 2p
//   5. model from the full-data symbol counts; 6. rANS-encode every chain; 7. pack.
// Determinism: float64 arithmetic without contraction (this file is built with
// -ffp-contract=off), fixed summation orders, integer rate estimates, per-thread
// partial results merged in a fixed order.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <functional>
#include <thread>

#include "codec_math.h"
#include "ep_internal.h"

namespace ep {
namespace {

int num_threads() {
  int n = (int)std::thread::hardware_concurrency();
  if (n < 1) n = 1;
  if (const char* e = std::getenv("EP_NUM_THREADS")) {
    int v = std::atoi(e);
    if (v >= 1) n = std::min(n, v);
  }
  return std::min(n, 64);
}

template <class Fn>
void parallel_for(int64_t n, Fn fn, int64_t min_chunk = 1) {
  int nt = num_threads();
  if (n <= 0) return;
  int64_t chunks = std::min<int64_t>(nt, (n + min_chunk - 1) / min_chunk);
  if (chunks <= 1) {
    fn(0, n, 0);
    return;
  }
  std::vector<std::thread> th;
  for (int64_t t = 0; t < chunks; ++t) {
    int64_t b = n * t / chunks, e = n * (t + 1) / chunks;
    th.emplace_back([=, &fn] { fn(b, e, (int)t); });
  }
  for (auto& x : th) x.join();
}

// ------------------------------------------------------------------ containers
void widen(const void* src, int dtype, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = cm::widen_one(src, dtype, i);
}

double container_max(int dtype) {
  switch (dtype) {
    case EP_BF16: return (double)bf16_to_f32(0x7F7F);
    case EP_FP16: return 65504.0;
    case EP_FP8_E4M3FN: return 448.0;
    case EP_INT8: return 127.0;
    default: return 3.4028234663852886e38;
  }
}

using cm::Sym;
using cm::e8_doubled;
using cm::symbolize;

// ------------------------------------------------------------------ row geometry
struct Matrix {
  int64_t R, C, G;             // G = groups per row
  std::vector<double> w;       // R x C
  std::vector<uint16_t> s_bits;
  std::vector<float> s;
  std::vector<double> amax;
};

inline float f32_from_bits(uint32_t b) {
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}
inline uint32_t f32_bits(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  return b;
}

// Quantise row r into groups (G x 8 doubled coordinates).
void quantize_row(const Matrix& mx, int64_t r, float delta, int32_t* u_out) {
  float h = mx.s[r] * delta;
  double den = 2.0 * (double)h;
  const double* wr = &mx.w[r * mx.C];
  double y[8];
  for (int64_t g = 0; g < mx.G; ++g) {
    for (int i = 0; i < 8; ++i) {
      int64_t col = g * 8 + i;
      double v = col < mx.C ? wr[col] : 0.0;
      y[i] = (den != 0.0) ? v / den : 0.0;
    }
    e8_doubled(y, u_out + g * 8);
  }
}

bool admissible(const Matrix& mx, float delta) { return resolution_admissible(mx.s.data(), mx.amax.data(), mx.R, delta); }

// est(delta) over the sample rows.
Estimate estimate(const Matrix& mx, const std::vector<int64_t>& rows, float delta) {
  const int64_t G = mx.G;
  const int64_t ng = (int64_t)rows.size() * G;
  std::vector<int32_t> u((size_t)ng * 8);
  parallel_for((int64_t)rows.size(), [&](int64_t b, int64_t e, int) {
    for (int64_t i = b; i < e; ++i) quantize_row(mx, rows[i], delta, &u[(size_t)(i * G * 8)]);
  }, 8);
  // choose k: smallest k with #(m >= 2^k) * 2^20 <= #coords (escapes at most one in 2^20)
  int64_t ge[8] = {0};
  for (int64_t gi = 0; gi < ng; ++gi) {
    const int32_t* ug = &u[gi * 8];
    int c = ug[0] & 1;
    for (int i = 0; i < 8; ++i) {
      int a = ug[i] < 0 ? -ug[i] : ug[i];
      int64_t m = (a - c) >> 1;
      for (int kk = 3; kk <= 7; ++kk) ge[kk] += m >= (1 << kk);
    }
  }
  int k = 7;
  for (int kk = 3; kk <= 7; ++kk)
    if (ge[kk] * (int64_t(1) << 20) <= ng * 8) {
      k = kk;
      break;
    }
  const int nm = n_msym(k);
  int64_t cc[2] = {0, 0};
  std::vector<int64_t> mag0(nm, 0), mag1(nm, 0);
  Sym s[8];
  int ms[8];
  for (int64_t gi = 0; gi < ng; ++gi) {
    int c = symbolize(&u[gi * 8], k, s, ms);
    cc[c]++;
    auto& mg = c ? mag1 : mag0;
    for (int i = 0; i < 8; ++i) mg[ms[i]]++;
  }
  Model m = build_model(k, cc, mag0.data(), mag1.data());
  const int32_t* lq = log2q_table();
  int64_t est = 0;
  for (int64_t gi = 0; gi < ng; ++gi) {
    symbolize(&u[gi * 8], k, s, ms);
    for (int i = 0; i < 8; ++i) {
      int32_t f = m.F[s[i].ctx][s[i].id];
      est += (int64_t)m.P * 65536 - lq[f];
      est += (int64_t)65536 * s[i].rawbits;
    }
  }
  return {est, k};
}

// ------------------------------------------------------------------ rANS encoder
struct ChainOut {
  std::vector<uint16_t> words;   // decoding order
  uint32_t state;
  std::vector<uint8_t> cons;     // words the decoder reads in each of the chain's groups
  std::vector<uint16_t> rank;    // main-area position of each full chunk in its tile
};

void encode_chain(const int32_t* u_all, const Model& m, int64_t t, int j, int S, int64_t n_groups,
                  ChainOut* out) {
  int64_t gt = std::min<int64_t>(kTileGroups, n_groups - (int64_t)kTileGroups * t);
  int ngr = gt > j ? (int)((gt - j + S - 1) / S) : 0;
  uint64_t x = kL;
  std::vector<uint16_t>& w = out->words;
  w.clear();
  auto emit = [&]() {
    w.push_back((uint16_t)(x & 0xFFFFu));
    x >>= 16;
  };
  auto bypass = [&](uint32_t v, int b) {
    if (x >= (1ull << (32 - b))) emit();
    x = (x << b) | v;
  };
  Sym s[8];
  int ms[8];
  out->cons.assign((size_t)ngr, 0);
  for (int kk = ngr - 1; kk >= 0; --kk) {
    int64_t g = (int64_t)kTileGroups * t + j + (int64_t)kk * S;
    symbolize(u_all + g * 8, m.k, s, ms);
    const size_t w0 = w.size();
    for (int i = 7; i >= 0; --i) {
      int rb = s[i].rawbits;
      if (rb > 16) bypass(s[i].rawval >> 16, rb - 16);
      if (rb > 0) bypass(s[i].rawval & 0xFFFFu, std::min(rb, 16));
      uint64_t f = (uint64_t)m.F[s[i].ctx][s[i].id];
      uint64_t cum = (uint64_t)m.CUM[s[i].ctx][s[i].id];
      // before a step x stays below f (L / M) 2^16 = f << (32 - P)
      if (x >= (f << (32 - m.P))) emit();
      x = (x / f) * (uint64_t)m.M + (x % f) + cum;
    }
    out->cons[kk] = (uint8_t)(w.size() - w0);
  }
  std::reverse(w.begin(), w.end());
  out->state = (uint32_t)x;
}

// ------------------------------------------------------------------ stream layout
// Request order of one tile's full chunks.  The decoder keeps a window of at most 32
// fetched words per chain and fetches 8-word chunks only at these sites, chains taking
// turns in chain order; a sync site repeats rounds until no chain wants more:
//   no escapes in the blob: prime until 17 words ahead; every even group: until 17
//   ahead, then one round for chains at most 24 ahead;
//   escapes in the blob: prime until 24 ahead; every group: until 24 ahead, then one
//   round for chains at most 24 ahead.
// Only chains that decode the group take part; a chain's last short chunk (its tail)
// counts as a request but lives in the block's tail area.
void schedule_tile(ChainOut* ch, int S, bool esc) {
  int32_t F[64], q[64], n[64], ngr[64];
  uint16_t ctr = 0;
  int gmax = 0;
  for (int j = 0; j < S; ++j) {
    F[j] = 0;
    q[j] = 0;
    n[j] = (int32_t)ch[j].words.size();
    ngr[j] = (int32_t)ch[j].cons.size();
    gmax = std::max(gmax, ngr[j]);
    ch[j].rank.clear();
  }
  auto take = [&](int j) {
    if (n[j] - F[j] >= 8) {
      ch[j].rank.push_back(ctr++);
      F[j] += 8;
    } else {
      F[j] = n[j];
    }
  };
  auto sync = [&](auto cand, int32_t ahead) {
    for (;;) {
      bool any = false;
      for (int j = 0; j < S; ++j)
        if (cand(j) && F[j] - q[j] < ahead && F[j] < n[j]) {
          take(j);
          any = true;
        }
      if (!any) return;
    }
  };
  const int32_t ahead = esc ? 24 : 17;
  sync([](int) { return true; }, ahead);
  for (int g = 0; g < gmax; ++g) {
    auto act = [&](int j) { return g < ngr[j]; };
    if (esc || (g & 1) == 0) {
      sync(act, ahead);
      for (int j = 0; j < S; ++j)
        if (act(j) && F[j] - q[j] <= 24 && F[j] < n[j]) take(j);
    }
    for (int j = 0; j < S; ++j)
      if (act(j)) q[j] += ch[j].cons[g];
  }
}

void put_u16(std::vector<uint8_t>& b, size_t off, uint16_t v) { std::memcpy(&b[off], &v, 2); }
void put_u32(std::vector<uint8_t>& b, size_t off, uint32_t v) { std::memcpy(&b[off], &v, 4); }
void put_u64(std::vector<uint8_t>& b, size_t off, uint64_t v) { std::memcpy(&b[off], &v, 8); }

// The chain area shared by both blob kinds: u32 block offsets | full chunks per chain
// (u8 if S >= 8, else u16) | tail nibbles | u32 states | u16 stream; a block of 64
// chains holds [tile main areas (chunks in request order)][tails][pad to 8 words].
struct Area {
  std::vector<uint64_t> block_off;   // in chunks, n_blocks + 1 entries
  int64_t n_blocks = 0;
  uint64_t n_words = 0;
  size_t bytes = 0;                  // size of the whole area
};

int plan_area(const std::vector<ChainOut>& chains, int S, Area* a) {
  const int64_t n_chains = (int64_t)chains.size();
  a->n_blocks = (n_chains + kBlockChains - 1) / kBlockChains;
  const int64_t max_full = S >= 8 ? 0xFF : 0xFFFF;
  a->block_off.assign((size_t)a->n_blocks + 1, 0);
  for (int64_t bk = 0; bk < a->n_blocks; ++bk) {
    const int64_t c0 = bk * kBlockChains, c1 = std::min(n_chains, c0 + kBlockChains);
    uint64_t words = 0;
    for (int64_t c = c0; c < c1; ++c) {
      const uint64_t len = chains[c].words.size();
      if ((int64_t)(len / 8) > max_full) return fail(EP_E_ARG, "chain longer than the chunk count field");
      words += len;
    }
    a->block_off[bk + 1] = a->block_off[bk] + (words + 7) / 8;
  }
  a->n_words = 8 * a->block_off[a->n_blocks];
  if (a->block_off[a->n_blocks] > 0xFFFFFFFFull) return fail(EP_E_ARG, "stream too long for the block offsets");
  const size_t fw = S >= 8 ? 1 : 2;
  a->bytes = 4 * (size_t)a->n_blocks + fw * (size_t)n_chains + (size_t)((n_chains + 1) / 2) +
             4 * (size_t)n_chains + 2 * (size_t)a->n_words;
  return EP_OK;
}

// b[off ..) must be zeroed
void write_area(const std::vector<ChainOut>& chains, int S, const Area& a, std::vector<uint8_t>& b, size_t off) {
  const int64_t n_chains = (int64_t)chains.size();
  const size_t fw = S >= 8 ? 1 : 2;
  const size_t off_bo = off;
  const size_t off_full = off_bo + 4 * (size_t)a.n_blocks;
  const size_t off_nib = off_full + fw * (size_t)n_chains;
  const size_t off_st = off_nib + (size_t)((n_chains + 1) / 2);
  const size_t off_stream = off_st + 4 * (size_t)n_chains;
  for (int64_t bk = 0; bk < a.n_blocks; ++bk) put_u32(b, off_bo + 4 * (size_t)bk, (uint32_t)a.block_off[bk]);
  for (int64_t c = 0; c < n_chains; ++c) {
    const size_t len = chains[c].words.size();
    if (fw == 1) b[off_full + (size_t)c] = (uint8_t)(len / 8);
    else put_u16(b, off_full + 2 * (size_t)c, (uint16_t)(len / 8));
    b[off_nib + (size_t)(c / 2)] |= (uint8_t)((len % 8) << (4 * (c & 1)));
  }
  parallel_for(a.n_blocks, [&](int64_t bb, int64_t be, int) {
    for (int64_t bk = bb; bk < be; ++bk) {
      const int64_t c0 = bk * kBlockChains, c1 = std::min(n_chains, c0 + kBlockChains);
      const size_t base = off_stream + 16 * (size_t)a.block_off[bk];
      size_t tile_main = 0;   // words from the block start
      size_t tails = 0;
      for (int64_t c = c0; c < c1; ++c) tails += 8 * (chains[c].words.size() / 8);
      for (int64_t t0 = c0; t0 < c1; t0 += S) {
        size_t tile_words = 0;
        for (int64_t c = t0; c < t0 + S; ++c) {
          const auto& w = chains[c].words;
          const size_t nf = w.size() / 8;
          for (size_t nn = 0; nn < nf; ++nn)
            std::memcpy(&b[base + 2 * (tile_main + 8 * (size_t)chains[c].rank[nn])], &w[8 * nn], 16);
          tile_words += 8 * nf;
        }
        tile_main += tile_words;
      }
      for (int64_t c = c0; c < c1; ++c) {
        const auto& w = chains[c].words;
        const size_t nf = w.size() / 8, r = w.size() % 8;
        if (r) std::memcpy(&b[base + 2 * tails], &w[8 * nf], 2 * r);
        tails += r;
      }
    }
  }, 1);
  for (int64_t ch = 0; ch < n_chains; ++ch) put_u32(b, off_st + 4 * (size_t)ch, chains[ch].state);
}

// TileANS: chain j of tile t codes the bytes of its groups, context = byte position
// within the group modulo the context count
void encode_chain_bytes(const uint8_t* by, const int32_t (*F)[256], const int32_t (*CUM)[256], int n_ctx,
                        int64_t t, int j, int S, int64_t n_groups, ChainOut* out) {
  int64_t gt = std::min<int64_t>(kTileGroups, n_groups - (int64_t)kTileGroups * t);
  int ngr = gt > j ? (int)((gt - j + S - 1) / S) : 0;
  uint64_t x = kL;
  std::vector<uint16_t>& w = out->words;
  w.clear();
  out->cons.assign((size_t)ngr, 0);
  for (int kk = ngr - 1; kk >= 0; --kk) {
    const int64_t g = (int64_t)kTileGroups * t + j + (int64_t)kk * S;
    const size_t w0 = w.size();
    for (int i = 7; i >= 0; --i) {
      const int ctx = i % n_ctx;
      const uint8_t v = by[g * 8 + i];
      const uint64_t f = (uint64_t)F[ctx][v], cum = (uint64_t)CUM[ctx][v];
      if (x >= (f << (32 - kPBytes))) {
        w.push_back((uint16_t)(x & 0xFFFFu));
        x >>= 16;
      }
      x = (x / f) * (uint64_t)kMBytes + (x % f) + cum;
    }
    out->cons[kk] = (uint8_t)(w.size() - w0);
  }
  std::reverse(w.begin(), w.end());
  out->state = (uint32_t)x;
}

}  // namespace

bool resolution_admissible(const float* s, const double* amax, int64_t R, float delta) {
  for (int64_t r = 0; r < R; ++r) {
    if (!(s[r] > 0.f)) continue;
    float h = s[r] * delta;
    if (!(h > 0.f) || !std::isfinite(h)) return false;
    if (!(amax[r] / (2.0 * (double)h) < 536870912.0)) return false;
  }
  return true;
}

// The resolution search over float32 bit patterns: bracket between powers of two from
// 2^floor(1 - t) (within [2^jmin, 2^4]), then bisect to adjacent patterns, keeping the
// largest delta whose sampled estimate reaches T; the finest admissible delta if the
// target is out of reach.  Estimates are computed once per pattern.
void select_resolution(double t, int64_t T, int jmin, const std::function<Estimate(uint32_t)>& estimate_at,
                       uint32_t* dbits_out, int* k_out) {
  struct Probe {
    uint32_t bits;
    Estimate e;
  };
  std::vector<Probe> cache;
  auto est_at = [&](uint32_t bits) -> Estimate {
    for (auto& p : cache)
      if (p.bits == bits) return p.e;
    Estimate e = estimate_at(bits);
    cache.push_back({bits, e});
    return e;
  };
  auto ok = [&](uint32_t bits) { return est_at(bits).est >= T; };
  auto pow2bits = [](int j) {
    float f = std::ldexp(1.0f, j);
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return b;
  };
  const int jmax = 4;
  int j0 = (int)std::floor(1.0 - t);
  j0 = std::min(std::max(j0, jmin), jmax);
  uint32_t dbits = 0;
  bool done = false;
  uint32_t lo = 0, hi = 0;
  if (ok(pow2bits(j0))) {
    int j = j0;
    while (j < jmax && ok(pow2bits(j + 1))) ++j;
    if (j == jmax) {
      dbits = pow2bits(j);
      done = true;
    } else {
      lo = pow2bits(j);
      hi = pow2bits(j + 1);
    }
  } else {
    int j = j0 - 1;
    while (j >= jmin && !ok(pow2bits(j))) --j;
    if (j < jmin) {
      dbits = pow2bits(jmin);
      done = true;
    } else {
      lo = pow2bits(j);
      hi = pow2bits(j + 1);
    }
  }
  if (!done) {
    while (hi - lo > 1) {
      uint32_t mid = lo + ((hi - lo) >> 1);
      if (ok(mid)) lo = mid;
      else hi = mid;
    }
    dbits = lo;
  }
  *dbits_out = dbits;
  *k_out = est_at(dbits).k;
}

int compress(const void* src, int dtype, int64_t R, int64_t C, double t, int S_req,
             std::vector<uint8_t>* out, Distortion* dist) {
  if (!src || !out) return fail(EP_E_ARG, "null pointer");
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

  Matrix mx;
  mx.R = R;
  mx.C = C;
  mx.G = (C + 7) / 8;
  const int64_t N = R * C;
  try {
    mx.w.resize((size_t)N);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  parallel_for(R, [&](int64_t b, int64_t e, int) {
    size_t esz = dtype == EP_FP32 ? 4 : (dtype == EP_BF16 || dtype == EP_FP16 ? 2 : 1);
    widen((const uint8_t*)src + (size_t)(b * C) * esz, dtype, (e - b) * C, &mx.w[(size_t)(b * C)]);
  }, 64);
  std::atomic<bool> nonfinite{false};
  mx.s_bits.resize(R);
  mx.s.resize(R);
  mx.amax.resize(R);
  std::atomic<bool> tiny{false};
  parallel_for(R, [&](int64_t b, int64_t e, int) {
    for (int64_t r = b; r < e; ++r) {
      const double* wr = &mx.w[(size_t)(r * C)];
      double acc = 0.0, am = 0.0;
      bool live = false;
      for (int64_t c = 0; c < C; ++c) {
        double v = wr[c];
        if (!std::isfinite(v)) nonfinite = true;
        acc = acc + v * v;
        double a = std::fabs(v);
        if (a > am) am = a;
        live |= v != 0.0;
      }
      double rms = std::sqrt(acc / (double)C);
      uint16_t sb = f32_to_bf16_rne((float)rms);
      mx.s_bits[r] = sb;
      mx.s[r] = bf16_to_f32(sb);
      mx.amax[r] = am;
      if (live && ((sb >> 7) & 0xFF) == 0) tiny = true;
    }
  }, 16);
  if (nonfinite) return fail(EP_E_NONFINITE, "input holds NaN or Inf");
  if (tiny) return fail(EP_E_RANGE, "a nonzero row has an RMS below the BF16 normal range");

  // ---- sample rows
  std::vector<int64_t> rows;
  const int64_t kSample = 1 << 18;
  if (N <= kSample) {
    for (int64_t r = 0; r < R; ++r) rows.push_back(r);
  } else {
    int64_t ks = N / kSample;
    for (int64_t r = 0; r < R; r += ks) rows.push_back(r);
  }
  const int64_t n_sample = (int64_t)rows.size() * C;
  const int64_t T = (int64_t)std::ceil(t * 65536.0 * (double)n_sample);

  // ---- resolution search
  int jmin = 999;
  for (int j = -126; j <= 4; ++j)
    if (admissible(mx, std::ldexp(1.0f, j))) {
      jmin = j;
      break;
    }
  if (jmin == 999) return fail(EP_E_RANGE, "no admissible resolution");
  uint32_t dbits;
  int k;
  select_resolution(t, T, jmin, [&](uint32_t bits) { return estimate(mx, rows, f32_from_bits(bits)); }, &dbits, &k);
  const float delta = f32_from_bits(dbits);

  // ---- full quantisation
  const int64_t n_groups = R * mx.G;
  std::vector<int32_t> u;
  try {
    u.resize((size_t)n_groups * 8);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  parallel_for(R, [&](int64_t b, int64_t e, int) {
    for (int64_t r = b; r < e; ++r) quantize_row(mx, r, delta, &u[(size_t)(r * mx.G * 8)]);
  }, 4);
  // ---- counts (per-thread partials merged in order)
  const int nm = n_msym(k);
  const int nt = num_threads();
  std::vector<std::vector<int64_t>> part(nt, std::vector<int64_t>(2 * nm + 3, 0));
  parallel_for(n_groups, [&](int64_t b, int64_t e, int tid) {
    auto& p = part[tid];
    Sym s[8];
    int ms[8];
    for (int64_t g = b; g < e; ++g) {
      int c = symbolize(&u[(size_t)(g * 8)], k, s, ms);
      p[c]++;
      for (int i = 0; i < 8; ++i) {
        p[2 + c * nm + ms[i]]++;
        if (ms[i] >= (1 << k)) p[2 + 2 * nm] = 1;
      }
    }
  }, 4096);
  int64_t cc[2] = {0, 0};
  std::vector<int64_t> mag0(nm, 0), mag1(nm, 0);
  bool any_esc = false;
  for (auto& p : part) {
    cc[0] += p[0];
    cc[1] += p[1];
    for (int i = 0; i < nm; ++i) {
      mag0[i] += p[2 + i];
      mag1[i] += p[2 + nm + i];
    }
    any_esc |= p[2 + 2 * nm] != 0;
  }
  Model m = build_model(k, cc, mag0.data(), mag1.data());

  // ---- chains
  const int S = S_req ? S_req : (N >= (1ll << 22) ? 8 : 1);
  const int64_t n_tiles = std::max<int64_t>(1, (n_groups + kTileGroups - 1) / kTileGroups);
  const int64_t n_chains = n_tiles * S;
  std::vector<ChainOut> chains((size_t)n_chains);
  parallel_for(n_chains, [&](int64_t b, int64_t e, int) {
    for (int64_t ch = b; ch < e; ++ch) encode_chain(u.data(), m, ch / S, (int)(ch % S), S, n_groups, &chains[ch]);
  }, 64);
  parallel_for(n_tiles, [&](int64_t b, int64_t e, int) {
    for (int64_t tt = b; tt < e; ++tt) schedule_tile(&chains[(size_t)(tt * S)], S, any_esc);
  }, 16);

  // ---- distortion of the lattice reconstruction fl32(h_r u) (before the container
  // cast): per-row sums left to right, rows added in order
  if (dist) {
    std::vector<double> re((size_t)R, 0.0), rw((size_t)R, 0.0);
    parallel_for(R, [&](int64_t b, int64_t e, int) {
      for (int64_t r = b; r < e; ++r) {
        const float h = mx.s[r] * delta;
        double se = 0.0, sw = 0.0;
        for (int64_t c = 0; c < C; ++c) {
          const double w = mx.w[(size_t)(r * C + c)];
          const double d = w - (double)(h * (float)u[(size_t)(r * mx.G * 8 + c)]);
          se += d * d;
          sw += w * w;
        }
        re[(size_t)r] = se;
        rw[(size_t)r] = sw;
      }
    }, 16);
    dist->sq_err = 0.0;
    dist->sq_ref = 0.0;
    for (int64_t r = 0; r < R; ++r) {
      dist->sq_err += re[(size_t)r];
      dist->sq_ref += rw[(size_t)r];
    }
  }

  // ---- saturation flag
  std::atomic<bool> sat{false};
  if (dtype != EP_FP32) {
    const double cmax = container_max(dtype);
    parallel_for(R, [&](int64_t b, int64_t e, int) {
      for (int64_t r = b; r < e && !sat; ++r) {
        float h = mx.s[r] * delta;
        for (int64_t c = 0; c < C; ++c) {
          float v = h * (float)u[(size_t)(r * mx.G * 8 + c)];
          double dv = (double)v;
          bool out_of_range = dtype == EP_INT8 ? (std::nearbyint(dv) > 127.0 || std::nearbyint(dv) < -128.0)
                                               : std::fabs(dv) > cmax;
          if (out_of_range) {
            sat = true;
            break;
          }
        }
      }
    }, 16);
  }

  // ---- blob: header | row scales | model | chain area
  Area area;
  int rc = plan_area(chains, S, &area);
  if (rc) return rc;
  const std::vector<uint8_t> mbytes = m.to_bytes();
  const size_t total = kHeaderBytes + 2 * (size_t)R + mbytes.size() + area.bytes;
  std::vector<uint8_t>& b = *out;
  try {
    b.assign(total, 0);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  std::memcpy(&b[0], "EPK1", 4);
  put_u16(b, 4, 3);
  b[6] = (uint8_t)dtype;
  b[7] = (uint8_t)precision(k);
  b[8] = (uint8_t)S;
  b[9] = (uint8_t)k;
  b[10] = (uint8_t)((any_esc ? kFlagEsc : 0) | (sat ? kFlagSat : 0));
  b[11] = 12;
  put_u32(b, 12, (uint32_t)R);
  put_u32(b, 16, (uint32_t)C);
  put_u32(b, 20, dbits);
  put_u32(b, 24, (uint32_t)n_tiles);
  put_u32(b, 28, (uint32_t)area.n_blocks);
  put_u64(b, 32, area.n_words);
  put_u32(b, 40, (uint32_t)mbytes.size());
  put_u32(b, 44, 0);
  size_t off = kHeaderBytes;
  for (int64_t r = 0; r < R; ++r, off += 2) put_u16(b, off, mx.s_bits[r]);
  std::memcpy(&b[off], mbytes.data(), mbytes.size());
  off += mbytes.size();
  write_area(chains, S, area, b, off);
  return EP_OK;
}

// TileANS (lossless): the tensor's raw bytes, per-byte-position tables (or uniform),
// the lossy blob's chains and chain area.
int compress_lossless(const void* src, int64_t n_bytes, int E, const int64_t* dims, int ndim, int tag, int S_req,
                      std::vector<uint8_t>* out) {
  if (!src || !out || (ndim > 0 && !dims)) return fail(EP_E_ARG, "null pointer");
  if (E != 1 && E != 2 && E != 4 && E != 8) return fail(EP_E_ARG, "element size must be 1, 2, 4 or 8 bytes");
  if (ndim < 1 || ndim > 8) return fail(EP_E_SHAPE, "rank must be 1..8");
  if (tag < 0 || tag > 255) return fail(EP_E_ARG, "dtype tag must be 0..255");
  __int128 prod = E;
  for (int d = 0; d < ndim; ++d) {
    if (dims[d] < 1) return fail(EP_E_SHAPE, "every extent must be >= 1");
    prod *= dims[d];
    if (prod > ((__int128)1 << 40)) return fail(EP_E_SHAPE, "tensor too large");
  }
  if (n_bytes != (int64_t)prod) return fail(EP_E_SHAPE, "byte count does not match the shape");
  if (S_req != 0 && S_req != 1 && S_req != 2 && S_req != 4 && S_req != 8 && S_req != 16 &&
      S_req != 32 && S_req != 64)
    return fail(EP_E_ARG, "chains_per_tile must be 0 or a power of two <= 64");
  const int n_ctx = E < 4 ? E : 4;
  const int64_t n_groups = (n_bytes + 7) / 8;
  std::vector<uint8_t> by;
  try {
    by.assign((size_t)(8 * n_groups), 0);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  std::memcpy(by.data(), src, (size_t)n_bytes);

  // ---- per-context tables
  const int nt = num_threads();
  std::vector<std::vector<int64_t>> part((size_t)nt, std::vector<int64_t>(4 * 256, 0));
  parallel_for(8 * n_groups, [&](int64_t b0, int64_t e0, int tid) {
    auto& p = part[tid];
    for (int64_t q = b0; q < e0; ++q) p[(size_t)((q % n_ctx) * 256 + by[q])]++;
  }, 1 << 16);
  int32_t F[4][256], CUM[4][256];
  int umask = 0;
  const int32_t* lq = log2q_table();
  for (int c = 0; c < n_ctx; ++c) {
    int64_t cnt[256];
    for (int v = 0; v < 256; ++v) {
      cnt[v] = 0;
      for (auto& p : part) cnt[v] += p[(size_t)(c * 256 + v)];
    }
    int32_t f[256];
    quantize_freqs(cnt, 256, kMBytes, f);
    // coded estimate (plus the stored table's 4096 bits) against 8 raw bits a byte
    __int128 coded = (__int128)256 * 16 * 65536, raw = 0;
    for (int v = 0; v < 256; ++v) {
      if (cnt[v] > 0) coded += (__int128)cnt[v] * (kPBytes * 65536 - lq[f[v]]);
      raw += (__int128)cnt[v] * 8 * 65536;
    }
    if (coded >= raw) {
      umask |= 1 << c;
      for (int v = 0; v < 256; ++v) F[c][v] = kMBytes / 256;
    } else {
      for (int v = 0; v < 256; ++v) F[c][v] = f[v];
    }
    int32_t acc = 0;
    for (int v = 0; v < 256; ++v) {
      CUM[c][v] = acc;
      acc += F[c][v];
    }
  }

  // ---- chains
  const int S = S_req ? S_req : (n_bytes >= (1ll << 22) ? 8 : 1);
  const int64_t n_tiles = std::max<int64_t>(1, (n_groups + kTileGroups - 1) / kTileGroups);
  const int64_t n_chains = n_tiles * S;
  std::vector<ChainOut> chains((size_t)n_chains);
  parallel_for(n_chains, [&](int64_t b0, int64_t e0, int) {
    for (int64_t ch = b0; ch < e0; ++ch)
      encode_chain_bytes(by.data(), F, CUM, n_ctx, ch / S, (int)(ch % S), S, n_groups, &chains[ch]);
  }, 64);
  parallel_for(n_tiles, [&](int64_t b0, int64_t e0, int) {
    for (int64_t tt = b0; tt < e0; ++tt) schedule_tile(&chains[(size_t)(tt * S)], S, false);
  }, 16);

  // ---- blob: header | dims | tables | chain area
  Area area;
  int rc = plan_area(chains, S, &area);
  if (rc) return rc;
  int n_coded = 0;
  for (int c = 0; c < n_ctx; ++c) n_coded += !((umask >> c) & 1);
  const size_t total = kHeaderBytes + 8 * (size_t)ndim + 512 * (size_t)n_coded + area.bytes;
  std::vector<uint8_t>& b = *out;
  try {
    b.assign(total, 0);
  } catch (...) {
    return fail(EP_E_NOMEM, "out of host memory");
  }
  std::memcpy(&b[0], "EPT1", 4);
  put_u16(b, 4, 1);
  b[6] = (uint8_t)tag;
  b[7] = (uint8_t)E;
  b[8] = (uint8_t)kPBytes;
  b[9] = (uint8_t)S;
  b[10] = (uint8_t)ndim;
  b[11] = (uint8_t)umask;
  b[12] = 12;
  put_u64(b, 16, (uint64_t)n_bytes);
  put_u32(b, 24, (uint32_t)n_tiles);
  put_u32(b, 28, (uint32_t)area.n_blocks);
  put_u64(b, 32, area.n_words);
  put_u64(b, 40, 0);
  size_t off = kHeaderBytes;
  for (int d = 0; d < ndim; ++d, off += 8) put_u64(b, off, (uint64_t)dims[d]);
  for (int c = 0; c < n_ctx; ++c) {
    if ((umask >> c) & 1) continue;
    for (int v = 0; v < 256; ++v, off += 2) put_u16(b, off, (uint16_t)F[c][v]);
  }
  write_area(chains, S, area, b, off);
  return EP_OK;
}

}  // namespace ep
