// Conditional model of the lattice coordinates ([ABS]: "conditional probability model
// of lattice coordinates"; the pages give no detail — this is the project's reading).
//
// A group is one E8 point in doubled coordinates u (8 integers of one parity, sum
// divisible by 4); its coset is c = u0 mod 2.  Each coordinate is a magnitude
// m = (|u| - c)/2 and a sign.  Magnitudes below K = 2^k are direct symbols; larger ones
// are log-buckets (4 per octave) with e-2 raw bits.  Signed symbol sid = 2 msym + neg.
//
// Seven tables of M = 2^P slots (P = precision(k)):
//   FIRST        coordinate 0, joint (c, sid), id = 512 c + sid
//   FREE[c]      coordinates 1..6 (signs share a magnitude's probability evenly)
//   LAST[c][pi]  coordinate 7, pi = parity of sum_{i<7} floor(u_i / 2); E8 fixes the
//                parity of floor(u_7 / 2), so only agreeing direct symbols remain and
//                buckets send one raw bit fewer.
// Stored: coset weights (sum M) and per-coset magnitude frequencies (sum M / 2);
// FIRST and LAST are derived with the quantiser Q below.
#include <algorithm>
#include <cmath>
#include <numeric>

#include "ep_internal.h"

namespace ep {

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }
int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
const char* last_error_cstr() { return g_err.c_str(); }

// Q(w, T): present entries (w > 0) get max(1, floor(w T / W)); with fewer than two
// present, the first absent entries join with weight 0; a shortfall goes +1 by
// largest remainder (ties: earlier entry), an excess comes back -1 from the largest
// frequency above 1 (ties: earlier entry).  Zero total weight: the two joined
// entries split T.
void quantize_freqs(const int64_t* w, int n, int total, int32_t* f) {
  std::vector<char> present(n);
  int np = 0;
  for (int i = 0; i < n; ++i) {
    present[i] = w[i] > 0;
    np += present[i];
  }
  for (int i = 0; i < n && np < 2; ++i)
    if (!present[i]) {
      present[i] = 1;
      ++np;
    }
  int64_t W = 0;
  for (int i = 0; i < n; ++i) W += w[i];
  for (int i = 0; i < n; ++i) f[i] = 0;
  if (W == 0) {
    int a = -1, b = -1;
    for (int i = 0; i < n; ++i)
      if (present[i]) {
        if (a < 0) a = i;
        else if (b < 0) b = i;
      }
    f[a] = total / 2;
    f[b] = total - total / 2;
    return;
  }
  std::vector<int64_t> rem(n, 0);
  int64_t sum = 0;
  for (int i = 0; i < n; ++i) {
    if (!present[i]) continue;
    __int128 p = (__int128)w[i] * total;
    int64_t fl = (int64_t)(p / W);
    rem[i] = (int64_t)(p % W);
    f[i] = (int32_t)std::max<int64_t>(1, fl);
    sum += f[i];
  }
  int64_t d = total - sum;
  if (d > 0) {
    std::vector<int> order;
    for (int i = 0; i < n; ++i)
      if (present[i]) order.push_back(i);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      if (rem[a] != rem[b]) return rem[a] > rem[b];
      return a < b;
    });
    for (int64_t q = 0; q < d; ++q) f[order[q]] += 1;
  }
  while (d < 0) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (present[i] && f[i] > 1 && (best < 0 || f[i] > f[best])) best = i;
    f[best] -= 1;
    ++d;
  }
}

bool Model::last_ok(int c, int pi, int sid) const {
  int msym = sid >> 1, neg = sid & 1;
  if (msym >= (1 << k)) return !(c == 0 && sid == 1);
  if (c == 0) return ((msym & 1) == pi) && sid != 1;
  return ((msym + neg) & 1) == pi;
}

void Model::derive() {
  std::memset(F, 0, sizeof(F));
  int64_t freeF[2][kIdSpace];
  std::memset(freeF, 0, sizeof(freeF));
  for (int c = 0; c < 2; ++c) {
    for (int m = 0; m < nm; ++m) {
      freeF[c][2 * m] = g[c][m];
      freeF[c][2 * m + 1] = g[c][m];
    }
    if (c == 0) {
      freeF[0][0] = 2 * int64_t(g[0][0]);
      freeF[0][1] = 0;
    }
    for (int s = 0; s < 2 * nm; ++s) F[1 + c][s] = (int32_t)freeF[c][s];
  }
  // FIRST: ids 512 c + sid (sid 1 of coset 0 does not exist)
  {
    std::vector<int> ids;
    std::vector<int64_t> wts;
    for (int c = 0; c < 2; ++c)
      for (int s = 0; s < 2 * nm; ++s) {
        if (c == 0 && s == 1) continue;
        ids.push_back(512 * c + s);
        wts.push_back(int64_t(w[c]) * freeF[c][s]);
      }
    std::vector<int32_t> f(ids.size());
    quantize_freqs(wts.data(), (int)ids.size(), M, f.data());
    for (size_t i = 0; i < ids.size(); ++i) F[0][ids[i]] = f[i];
  }
  for (int c = 0; c < 2; ++c)
    for (int pi = 0; pi < 2; ++pi) {
      std::vector<int> ids;
      std::vector<int64_t> wts;
      for (int s = 0; s < 2 * nm; ++s)
        if (last_ok(c, pi, s)) {
          ids.push_back(s);
          wts.push_back(freeF[c][s]);
        }
      std::vector<int32_t> f(ids.size());
      quantize_freqs(wts.data(), (int)ids.size(), M, f.data());
      for (size_t i = 0; i < ids.size(); ++i) F[3 + 2 * c + pi][ids[i]] = f[i];
    }
  for (int t = 0; t < kNumCtx; ++t) {
    int32_t acc = 0;
    for (int i = 0; i < kIdSpace; ++i) {
      CUM[t][i] = acc;
      acc += F[t][i];
    }
  }
}

namespace {
struct BitWriter {
  std::vector<uint8_t> out;
  int nbits = 0;
  void put(uint32_t v, int n) {
    for (int i = 0; i < n; ++i) {
      if ((nbits >> 3) >= (int)out.size()) out.push_back(0);
      out[nbits >> 3] |= uint8_t(((v >> i) & 1u) << (nbits & 7));
      ++nbits;
    }
  }
};
struct BitReader {
  const uint8_t* p;
  size_t n;
  size_t pos = 0;
  bool ok = true;
  uint32_t get(int nb) {
    uint32_t v = 0;
    for (int i = 0; i < nb; ++i) {
      size_t q = pos + i;
      if ((q >> 3) >= n) {
        ok = false;
        return 0;
      }
      v |= uint32_t((p[q >> 3] >> (q & 7)) & 1u) << i;
    }
    pos += nb;
    return v;
  }
};
}  // namespace

std::vector<uint8_t> Model::to_bytes() const {
  BitWriter bw;
  bw.put(uint32_t(w[1]), 11);
  for (int c = 0; c < 2; ++c) {
    int n_mag = 0;
    for (int m = 0; m < nm; ++m)
      if (g[c][m] > 0) n_mag = m + 1;
    bw.put(uint32_t(n_mag), 8);
    for (int m = 0; m < n_mag; ++m) bw.put(uint32_t(g[c][m]), 10);
  }
  return bw.out;
}

bool Model::from_bytes(const uint8_t* p, size_t n, int k, Model* out, std::string* err) {
  BitReader br{p, n};
  Model m;
  m.k = k;
  m.nm = n_msym(k);
  m.P = precision(k);
  m.M = 1 << m.P;
  uint32_t w1 = br.get(11);
  for (int c = 0; c < 2; ++c) {
    uint32_t n_mag = br.get(8);
    if (!br.ok || n_mag < 1 || (int)n_mag > m.nm) {
      *err = "bad magnitude alphabet size";
      return false;
    }
    m.g[c].assign(m.nm, 0);
    int64_t s = 0;
    int npres = 0;
    for (uint32_t i = 0; i < n_mag; ++i) {
      m.g[c][i] = (int32_t)br.get(10);
      s += m.g[c][i];
      npres += m.g[c][i] > 0;
    }
    if (!br.ok || s != m.M / 2 || npres < 2) {
      *err = "bad magnitude frequencies";
      return false;
    }
  }
  if (w1 < 1 || w1 > uint32_t(m.M - 1)) {
    *err = "bad coset weight";
    return false;
  }
  if (n * 8 - br.pos >= 8) {
    *err = "model has trailing bytes";
    return false;
  }
  m.w[0] = m.M - (int)w1;
  m.w[1] = (int)w1;
  m.derive();
  *out = m;
  return true;
}

Model build_model(int k, const int64_t cc[2], const int64_t* mag0, const int64_t* mag1) {
  Model m;
  m.k = k;
  m.nm = n_msym(k);
  m.P = precision(k);
  m.M = 1 << m.P;
  int32_t wq[2];
  quantize_freqs(cc, 2, m.M, wq);
  m.w[0] = wq[0];
  m.w[1] = wq[1];
  for (int c = 0; c < 2; ++c) {
    m.g[c].assign(m.nm, 0);
    quantize_freqs(c == 0 ? mag0 : mag1, m.nm, m.M / 2, m.g[c].data());
  }
  m.derive();
  return m;
}

const int32_t* log2q_table() {
  static int32_t t[kMMax + 1] = {0};
  static bool init = false;
  if (!init) {
    for (int f = 1; f <= kMMax; ++f) t[f] = (int32_t)std::floor(65536.0 * std::log2((double)f) + 0.5);
    init = true;
  }
  return t;
}

void build_slot_tables(const Model& m, uint32_t* out, bool narrow) {
  const int K = 1 << m.k;
  for (int t = 0; t < kNumCtx; ++t) {
    for (int id = 0; id < kIdSpace; ++id) {
      int32_t f = m.F[t][id];
      if (f <= 0) continue;
      int c, sid;
      if (t == 0) {
        c = id >> 9;
        sid = id & 511;
      } else {
        c = (t == 1 || t == 3 || t == 4) ? 0 : 1;
        sid = id;
      }
      int msym = sid >> 1, neg = sid & 1;
      uint32_t hi;   // bits 22..31
      if (msym < K) {
        int u = 2 * msym + c;
        if (neg) u = -u;
        hi = narrow ? (uint32_t(c) | (uint32_t(u + 128) << 2)) : (uint32_t(u) & 0x1FFu);
      } else {
        // bucket: n2 = e - 2 magnitude bits below the leading three (1, top2)
        int n2 = ((msym - K) >> 2) + m.k - 2, top2 = (msym - K) & 3;
        hi = narrow ? (uint32_t(c) | (1u << 1) | (uint32_t(n2) << 2) | (uint32_t(top2) << 7) | (uint32_t(neg) << 9))
                    : (uint32_t(c) | (uint32_t(neg) << 1) | (uint32_t(n2) << 2) | (uint32_t(top2) << 7) | (1u << 9));
      }
      int32_t cum = m.CUM[t][id];
      for (int s = cum; s < cum + f; ++s) {
        uint32_t bias = uint32_t(s - cum);
        out[t * m.M + s] = uint32_t(f) | (bias << 11) | (hi << 22);
      }
    }
  }
}

void build_split_tables(const Model& m, uint32_t* out) {
  const int K = 1 << m.k;
  for (int t = 0; t < kNumCtx; ++t) {
    for (int id = 0; id < kIdSpace; ++id) {
      const int32_t f = m.F[t][id];
      if (f <= 0) continue;
      const int c = t == 0 ? id >> 9 : ((t == 1 || t == 3 || t == 4) ? 0 : 1);
      const int sid = t == 0 ? id & 511 : id;
      const int msym = sid >> 1, neg = sid & 1;
      // (blobs without escapes: every symbol is direct, msym < K)
      int u = msym < K ? 2 * msym + c : 0;
      if (neg) u = -u;
      const int32_t cum = m.CUM[t][id];
      for (int s = cum; s < cum + f; ++s) {
        out[2 * (t * m.M + s)] = uint32_t(f) | (uint32_t(u + 128) << 24);
        out[2 * (t * m.M + s) + 1] = uint32_t(s - cum);
      }
    }
  }
}

void build_byte_tables(const int32_t (*F)[256], int n_ctx, uint32_t* out) {
  for (int c = 0; c < n_ctx; ++c) {
    int32_t cum = 0;
    for (int v = 0; v < 256; ++v) {
      for (int32_t q = 0; q < F[c][v]; ++q)
        out[c * kMBytes + cum + q] = uint32_t(F[c][v]) | (uint32_t(q) << 11) | (uint32_t(v) << 24);
      cum += F[c][v];
    }
  }
}

}  // namespace ep
