// Host-side encoder and blob parser of libnwc (C++17, no device code).
//
// Method (pages): a BF16 weight is split into a raw byte (sign + 7 fraction
// bits, stored as is) and its 8-bit exponent, which is Huffman coded --
// "NWC -- Neural Weight Compression", How it works, "Byte planes";
// "Unweight: how we compressed an LLM 22% ...", Compressing BF16 Weights.
// The code is per tensor, length-limited (package-merge, Larmore & Hirschberg
// 1990) and canonical (RFC 1951 section 3.2.2); codes are sent most
// significant bit first into little-endian 32-bit words (RFC 1951 3.1.1).
//
// Blob layout (all little-endian, sections 256-byte aligned):
//   header 256 B | code_len u8[256] | decode table u32[4096] |
//   tile_words u32[n_tiles+1] | chunk_bits u16[n_chunks] |
//   raw u8[rows][raw_ld] | stream u32[stream_words] + 16 zero bytes
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "nwc_internal.hpp"

namespace nwc {

namespace {

constexpr uint32_t kMagic = 0x4243574Eu;  // "NWCB"
constexpr uint16_t kVersion = 1;
constexpr uint32_t kHeader = 256;
constexpr uint32_t kTableBits = 12;
constexpr uint32_t kTableSize = 1u << kTableBits;

inline uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

template <typename T>
inline void store_le(uint8_t* p, T v) {
  for (size_t i = 0; i < sizeof(T); i++) p[i] = static_cast<uint8_t>(static_cast<uint64_t>(v) >> (8 * i));
}
template <typename T>
inline T load_le(const uint8_t* p) {
  uint64_t v = 0;
  for (size_t i = 0; i < sizeof(T); i++) v |= static_cast<uint64_t>(p[i]) << (8 * i);
  return static_cast<T>(v);
}

inline uint8_t exponent_of(uint16_t b) { return static_cast<uint8_t>((b >> 7) & 0xFF); }
inline uint8_t raw_of(uint16_t b) { return static_cast<uint8_t>(((b >> 8) & 0x80) | (b & 0x7F)); }

unsigned worker_count(uint64_t work_items, uint64_t min_per_worker) {
  unsigned hw = std::thread::hardware_concurrency();
  if (hw == 0) hw = 1;
  hw = std::min(hw, 32u);
  uint64_t by_work = std::max<uint64_t>(1, work_items / std::max<uint64_t>(1, min_per_worker));
  return static_cast<unsigned>(std::min<uint64_t>(hw, by_work));
}

// Run fn(begin, end) over [0, n) split in contiguous blocks across threads.
template <typename F>
void parallel_blocks(uint64_t n, uint64_t min_per_worker, F fn) {
  unsigned nt = worker_count(n, min_per_worker);
  if (nt <= 1) {
    fn(uint64_t{0}, n);
    return;
  }
  std::vector<std::thread> ts;
  ts.reserve(nt);
  for (unsigned i = 0; i < nt; i++) {
    uint64_t b = n * i / nt, e = n * (i + 1) / nt;
    ts.emplace_back([=, &fn] { fn(b, e); });
  }
  for (auto& t : ts) t.join();
}

}  // namespace

// ---------------------------------------------------------------- code build

// Package-merge, expressed through prefix counts.  Leaves are sorted by
// (count, symbol).  List 0 is the leaves; list j merges the leaves with the
// packages formed by pairing consecutive items of list j-1 (a leaf wins a
// tie).  Selecting the first 2n-2 items of the last list and expanding
// packages downwards selects, at every list, a prefix; the leaves inside the
// prefix of each list are the first `a_j` sorted leaves, and each such
// selection adds one bit to those symbols' lengths.
// Ranked unary code with an escape ("NWC -- Neural Weight Compression", How
// it works, bullet "Prefix code instead of rANS"): exponents ranked by count
// (ties: smaller value first); rank r < R takes r + 1 bits (r ones, a zero);
// the others an escape of R ones and a ceil(log2(#escaped))-bit index, so
// every code stays within lmax bits and the canonical code built from these
// lengths is exactly "unary rank, or escape prefix + index in symbol order".
// R minimises the total bits (smallest R on a tie).
bool build_unary_lengths(const uint64_t hist[256], int lmax, uint8_t len[256]) {
  std::memset(len, 0, 256);
  std::vector<int> sym;
  for (int v = 0; v < 256; v++)
    if (hist[v]) sym.push_back(v);
  const int n = static_cast<int>(sym.size());
  if (n == 0 || lmax < 1) return false;
  if (n == 1) {
    len[sym[0]] = 1;
    return true;
  }
  std::stable_sort(sym.begin(), sym.end(), [&](int a, int b) { return hist[a] > hist[b]; });
  // bits(R) = sum over ranks < R of count * (rank + 1) + (count of the rest) * (R + index bits)
  std::vector<uint64_t> suffix(n + 1, 0);
  for (int r = n - 1; r >= 0; r--) suffix[r] = suffix[r + 1] + hist[sym[r]];
  int best = -1;
  unsigned __int128 best_bits = 0, head = 0;
  for (int R = 0; R < n; R++) {
    if (R > 0) head += static_cast<unsigned __int128>(hist[sym[R - 1]]) * static_cast<unsigned>(R);
    int b = 0;
    while ((1 << b) < n - R) b++;
    if (R + b <= lmax && R + b > 0) {
      const unsigned __int128 bits = head + static_cast<unsigned __int128>(suffix[R]) * static_cast<unsigned>(R + b);
      if (best < 0 || bits < best_bits) {
        best = R;
        best_bits = bits;
      }
    }
  }
  if (best < 0) return false;
  int b = 0;
  while ((1 << b) < n - best) b++;
  for (int r = 0; r < n; r++) len[sym[r]] = static_cast<uint8_t>(r < best ? r + 1 : best + b);
  return true;
}

bool build_lengths(const uint64_t hist[256], int lmax, uint8_t len[256], uint32_t pair_fit) {
  std::memset(len, 0, 256);
  std::vector<int> sym;
  for (int s = 0; s < 256; s++)
    if (hist[s]) sym.push_back(s);
  const int n = static_cast<int>(sym.size());
  if (n == 0 || lmax < 1 || lmax > 30) return false;
  if (n == 1) {
    len[sym[0]] = 1;
    return true;
  }
  if (static_cast<uint64_t>(n) > (uint64_t{1} << lmax)) return false;
  std::stable_sort(sym.begin(), sym.end(), [&](int a, int b) { return hist[a] < hist[b]; });
  std::vector<uint64_t> leafw(n);
  for (int i = 0; i < n; i++) leafw[i] = hist[sym[i]];
  // Per-symbol caps (pair_fit): symbols with count * pair_fit >= total may
  // use at most 6 bits, the others lmax.  The capped ones are the heaviest,
  // so the leaves whose cap reaches a level deeper than 6 are the first
  // n_deep sorted leaves: list j (level lmax - j) merges leaves
  // [0, leaves_at(j)) only, and the expansion below stays a prefix count.
  int n_deep = n;
  if (pair_fit && lmax > 6) {
    uint64_t total = 0;
    for (int s = 0; s < 256; s++) total += hist[s];
    n_deep = 0;
    while (n_deep < n && static_cast<double>(leafw[n_deep]) * pair_fit < static_cast<double>(total)) n_deep++;
  }
  auto leaves_at = [&](int j) { return lmax - j > 6 ? n_deep : n; };

  // lists[j] holds weights and a leaf flag per item, in merged order
  std::vector<std::vector<uint64_t>> w(lmax);
  std::vector<std::vector<uint8_t>> is_leaf(lmax);
  w[0].assign(leafw.begin(), leafw.begin() + leaves_at(0));
  is_leaf[0].assign(leaves_at(0), 1);
  for (int j = 1; j < lmax; j++) {
    const auto& prev = w[j - 1];
    const size_t npk = prev.size() / 2;
    const size_t nl = static_cast<size_t>(leaves_at(j));
    w[j].reserve(nl + npk);
    is_leaf[j].reserve(nl + npk);
    size_t a = 0, b = 0;
    while (a < nl || b < npk) {
      const bool take_pkg = b < npk && (a >= nl || prev[2 * b] + prev[2 * b + 1] < leafw[a]);
      if (take_pkg) {
        w[j].push_back(prev[2 * b] + prev[2 * b + 1]);
        is_leaf[j].push_back(0);
        b++;
      } else {
        w[j].push_back(leafw[a]);
        is_leaf[j].push_back(1);
        a++;
      }
    }
  }
  std::vector<int> bits(n, 0);
  size_t take = static_cast<size_t>(2 * n - 2);
  // the caps leave no complete code (over 64 common symbols): the plain limit
  if (take > w[lmax - 1].size()) return pair_fit ? build_lengths(hist, lmax, len, 0) : false;
  for (int j = lmax - 1; j >= 0; j--) {
    size_t leaves = 0;
    for (size_t i = 0; i < take; i++) leaves += is_leaf[j][i];
    for (size_t i = 0; i < leaves; i++) bits[i]++;
    take = 2 * (take - leaves);
  }
  for (int i = 0; i < n; i++) len[sym[i]] = static_cast<uint8_t>(bits[i]);
  return true;
}

// Canonical code values (RFC 1951 3.2.2); false if the lengths over-subscribe.
bool canonical(const uint8_t len[256], uint16_t code[256]) {
  uint32_t per_len[16] = {0};
  for (int s = 0; s < 256; s++) {
    if (len[s] > 15) return false;
    per_len[len[s]]++;
  }
  per_len[0] = 0;
  uint64_t space = 0;
  for (int l = 1; l <= 15; l++) space += static_cast<uint64_t>(per_len[l]) << (15 - l);
  if (space > (1u << 15)) return false;
  uint32_t first[16] = {0};
  uint32_t c = 0;
  for (int l = 1; l <= 15; l++) {
    c = (c + per_len[l - 1]) << 1;
    first[l] = c;
  }
  for (int s = 0; s < 256; s++) code[s] = len[s] ? static_cast<uint16_t>(first[len[s]]++) : 0;
  return true;
}

// Decode table for 12-bit windows (window bit 0 = next stream bit).  A
// one-code table is filled from every code's bit-reversed pattern, then each
// entry looks up a second code in the bits left over.
void build_table(const uint8_t len[256], uint32_t table[4096]) {
  uint16_t code[256];
  canonical(len, code);
  std::vector<uint16_t> one(kTableSize, 0);  // (len << 8) | sym, len 0 = no code
  for (int s = 0; s < 256; s++) {
    const uint32_t l = len[s];
    if (!l || l > kTableBits) continue;
    uint32_t rev = 0;
    for (uint32_t i = 0; i < l; i++) rev |= ((code[s] >> (l - 1 - i)) & 1u) << i;
    for (uint32_t hi = 0; hi < (kTableSize >> l); hi++) one[rev | (hi << l)] = static_cast<uint16_t>((l << 8) | s);
  }
  for (uint32_t win = 0; win < kTableSize; win++) {
    const uint32_t l0 = one[win] >> 8, s0 = one[win] & 0xFF;
    if (!l0) {
      table[win] = 0;
      continue;
    }
    const uint32_t rest = win >> l0;  // 12 - l0 valid bits, zeros above
    const uint32_t l1 = one[rest] >> 8, s1 = one[rest] & 0xFF;
    if (l1 && l0 + l1 <= kTableBits)
      table[win] = (l0 + l1) | (l0 << 16) | (s0 << 7) | (s1 << 23);
    else
      table[win] = l0 | (l0 << 16) | (s0 << 7) | (1u << 31);
  }
}

// ------------------------------------------------------------------ geometry

bool params_resolve(const nwc_params* p, Geometry* g) {
  g->tr = (p && p->tile_rows) ? p->tile_rows : 8;
  g->tc = (p && p->tile_cols) ? p->tile_cols : 512;
  g->s = (p && p->chunks_per_tile) ? p->chunks_per_tile : 64;
  g->lmax = (p && p->max_code_len) ? p->max_code_len : 8;
  g->pair_fit = (p && p->pair_fit) ? p->pair_fit : 1024;
  g->family = p ? p->code_family : 0;
  if (g->family > 1) return false;
  if (g->tc % g->s) return false;
  if (g->lmax < 6 || g->lmax > 12) return false;
  g->v = g->tc / g->s;
  if (static_cast<uint64_t>(g->tr) * g->v * g->lmax > 65535u) return false;
  return true;
}

void layout(Geometry* g, uint64_t rows, uint64_t cols, uint64_t stream_words) {
  g->rows = rows;
  g->cols = cols;
  g->n_tr = (rows + g->tr - 1) / g->tr;
  g->n_tc = (cols + g->tc - 1) / g->tc;
  g->n_tiles = g->n_tr * g->n_tc;
  g->n_chunks = g->n_tiles * g->s;
  g->raw_ld = round_up(cols, 16);
  g->stream_words = stream_words;
  g->off_code_len = kHeader;
  g->off_table = g->off_code_len + 256;
  g->off_tile_words = g->off_table + 4 * kTableSize;
  g->off_chunk_bits = round_up(g->off_tile_words + 4 * (g->n_tiles + 1), 256);
  g->off_raw = round_up(g->off_chunk_bits + 2 * g->n_chunks, 256);
  g->off_stream = round_up(g->off_raw + g->raw_ld * rows, 256);
  g->total = round_up(g->off_stream + 4 * stream_words + 16, 256);
}

// ------------------------------------------------------------------- encoder

nwc_status encode_bound(uint64_t rows, uint64_t cols, const nwc_params* p, size_t* max_bytes) {
  if (!max_bytes || rows < 1 || cols < 1 || rows > (1ull << 32) || cols > (1ull << 32))
    return NWC_ERR_INVALID_ARG;
  Geometry g;
  if (!params_resolve(p, &g)) return NWC_ERR_INVALID_ARG;
  layout(&g, rows, cols, 0);
  const uint64_t words = (rows * cols * g.lmax + 31) / 32 + g.n_tiles;
  if (words > 0xFFFFFFFFull) return NWC_ERR_UNSUPPORTED;
  layout(&g, rows, cols, words);
  *max_bytes = g.total;
  return NWC_OK;
}

nwc_status encode(const uint16_t* w, uint64_t rows, uint64_t cols, uint64_t ld, const nwc_params* p,
                  void* blob_v, size_t cap, size_t* used) {
  if (!w || !blob_v || !used || rows < 1 || cols < 1 || ld < cols || rows > (1ull << 32) ||
      cols > (1ull << 32))
    return NWC_ERR_INVALID_ARG;
  Geometry g;
  if (!params_resolve(p, &g)) return NWC_ERR_INVALID_ARG;
  layout(&g, rows, cols, 0);
  uint8_t* blob = static_cast<uint8_t*>(blob_v);

  // exponent histogram (per-thread partial counts, summed in thread order)
  std::vector<std::array<uint64_t, 256>> parts(worker_count(rows, 64));
  std::atomic<unsigned> slot{0};
  parallel_blocks(rows, 64, [&](uint64_t r0, uint64_t r1) {
    auto& h = parts[slot++];
    h.fill(0);
    for (uint64_t r = r0; r < r1; r++) {
      const uint16_t* row = w + r * ld;
      for (uint64_t c = 0; c < cols; c++) h[exponent_of(row[c])]++;
    }
  });
  uint64_t hist[256] = {0};
  for (unsigned i = 0; i < slot.load(); i++)
    for (int s = 0; s < 256; s++) hist[s] += parts[i][s];

  uint8_t len[256];
  uint16_t code[256];
  const bool lengths_ok = g.family == 1 ? build_unary_lengths(hist, static_cast<int>(g.lmax), len)
                                        : build_lengths(hist, static_cast<int>(g.lmax), len, g.pair_fit);
  if (!lengths_ok || !canonical(len, code))
    return NWC_ERR_INVALID_ARG;
  // codes bit-reversed so that emitting low bits first sends the MSB first
  uint32_t rev[256];
  for (int s = 0; s < 256; s++) {
    uint32_t r = 0;
    for (uint32_t i = 0; i < len[s]; i++) r |= ((code[s] >> (len[s] - 1 - i)) & 1u) << i;
    rev[s] = r;
  }

  // pass 1: bit length of every chunk
  std::vector<uint16_t> chunk_bits(g.n_chunks);
  parallel_blocks(g.n_tiles, 16, [&](uint64_t t0, uint64_t t1) {
    for (uint64_t t = t0; t < t1; t++) {
      const uint64_t ti = t / g.n_tc, tj = t % g.n_tc;
      const uint64_t r0 = ti * g.tr, r1 = std::min(rows, r0 + g.tr);
      const uint64_t tile_c1 = std::min(cols, tj * g.tc + g.tc);
      for (uint32_t c = 0; c < g.s; c++) {
        const uint64_t c0 = tj * g.tc + static_cast<uint64_t>(c) * g.v;
        uint32_t bits = 0;
        if (c0 < tile_c1) {
          const uint64_t c1 = std::min(tile_c1, c0 + g.v);
          for (uint64_t r = r0; r < r1; r++)
            for (uint64_t k = c0; k < c1; k++) bits += len[exponent_of(w[r * ld + k])];
        }
        chunk_bits[t * g.s + c] = static_cast<uint16_t>(bits);
      }
    }
  });
  std::vector<uint32_t> tile_words(g.n_tiles + 1);
  uint64_t words = 0;
  for (uint64_t t = 0; t < g.n_tiles; t++) {
    tile_words[t] = static_cast<uint32_t>(words);
    uint64_t bits = 0;
    for (uint32_t c = 0; c < g.s; c++) bits += chunk_bits[t * g.s + c];
    words += (bits + 31) / 32;
    if (words > 0xFFFFFFFFull) return NWC_ERR_UNSUPPORTED;
  }
  tile_words[g.n_tiles] = static_cast<uint32_t>(words);
  layout(&g, rows, cols, words);
  *used = g.total;
  if (g.total > cap) return NWC_ERR_BUFFER_TOO_SMALL;

  // header and small sections
  std::memset(blob, 0, g.off_raw);
  store_le<uint32_t>(blob + 0, kMagic);
  store_le<uint16_t>(blob + 4, kVersion);
  store_le<uint16_t>(blob + 6, static_cast<uint16_t>(kHeader));
  store_le<uint64_t>(blob + 8, rows);
  store_le<uint64_t>(blob + 16, cols);
  store_le<uint32_t>(blob + 24, g.tr);
  store_le<uint32_t>(blob + 28, g.tc);
  store_le<uint32_t>(blob + 32, g.s);
  store_le<uint32_t>(blob + 36, g.lmax);
  store_le<uint32_t>(blob + 40, 1);  // table kind: 12-bit pair table
  store_le<uint32_t>(blob + 44, 0);  // flags
  store_le<uint64_t>(blob + 48, g.raw_ld);
  store_le<uint64_t>(blob + 56, g.n_tiles);
  store_le<uint64_t>(blob + 64, g.n_chunks);
  store_le<uint64_t>(blob + 72, g.stream_words);
  store_le<uint64_t>(blob + 80, g.off_code_len);
  store_le<uint64_t>(blob + 88, g.off_table);
  store_le<uint64_t>(blob + 96, g.off_tile_words);
  store_le<uint64_t>(blob + 104, g.off_chunk_bits);
  store_le<uint64_t>(blob + 112, g.off_raw);
  store_le<uint64_t>(blob + 120, g.off_stream);
  store_le<uint64_t>(blob + 128, g.total);
  std::memcpy(blob + g.off_code_len, len, 256);
  uint32_t table[kTableSize];
  build_table(len, table);
  for (uint32_t i = 0; i < kTableSize; i++) store_le<uint32_t>(blob + g.off_table + 4 * i, table[i]);
  for (uint64_t t = 0; t <= g.n_tiles; t++) store_le<uint32_t>(blob + g.off_tile_words + 4 * t, tile_words[t]);
  for (uint64_t c = 0; c < g.n_chunks; c++) store_le<uint16_t>(blob + g.off_chunk_bits + 2 * c, chunk_bits[c]);

  // raw plane (row padding and the gap before the stream are zero)
  uint8_t* raw = blob + g.off_raw;
  parallel_blocks(rows, 64, [&](uint64_t r0, uint64_t r1) {
    for (uint64_t r = r0; r < r1; r++) {
      uint8_t* dst = raw + r * g.raw_ld;
      const uint16_t* src = w + r * ld;
      for (uint64_t c = 0; c < cols; c++) dst[c] = raw_of(src[c]);
      std::memset(dst + cols, 0, g.raw_ld - cols);
    }
  });
  std::memset(blob + g.off_raw + g.raw_ld * rows, 0, g.off_stream - (g.off_raw + g.raw_ld * rows));

  // pass 2: stream, one tile per task (tiles own disjoint word ranges)
  uint8_t* stream = blob + g.off_stream;
  parallel_blocks(g.n_tiles, 16, [&](uint64_t t0, uint64_t t1) {
    for (uint64_t t = t0; t < t1; t++) {
      const uint64_t ti = t / g.n_tc, tj = t % g.n_tc;
      const uint64_t r0 = ti * g.tr, r1 = std::min(rows, r0 + g.tr);
      const uint64_t tile_c1 = std::min(cols, tj * g.tc + g.tc);
      uint8_t* out = stream + 4ull * tile_words[t];
      uint64_t acc = 0;
      unsigned nacc = 0;
      auto flush = [&]() {
        store_le<uint32_t>(out, static_cast<uint32_t>(acc));
        out += 4;
        acc >>= 32;
        nacc -= 32;
      };
      for (uint32_t c = 0; c < g.s; c++) {
        const uint64_t c0 = tj * g.tc + static_cast<uint64_t>(c) * g.v;
        if (c0 >= tile_c1) continue;
        const uint64_t c1 = std::min(tile_c1, c0 + g.v);
        for (uint64_t r = r0; r < r1; r++)
          for (uint64_t k = c0; k < c1; k++) {
            const uint8_t e = exponent_of(w[r * ld + k]);
            acc |= static_cast<uint64_t>(rev[e]) << nacc;
            nacc += len[e];
            if (nacc >= 32) flush();
          }
      }
      if (nacc > 0) {
        store_le<uint32_t>(out, static_cast<uint32_t>(acc));
        out += 4;
      }
    }
  });
  std::memset(stream + 4 * g.stream_words, 0, g.total - (g.off_stream + 4 * g.stream_words));
  return NWC_OK;
}

// -------------------------------------------------------------------- parser

nwc_status inspect(const void* blob_v, size_t bytes, nwc_info* info) {
  if (!blob_v || !info) return NWC_ERR_INVALID_ARG;
  const uint8_t* b = static_cast<const uint8_t*>(blob_v);
  if (bytes < kHeader + 256) return NWC_ERR_BAD_FORMAT;
  if (load_le<uint32_t>(b) != kMagic || load_le<uint16_t>(b + 4) != kVersion ||
      load_le<uint16_t>(b + 6) != kHeader)
    return NWC_ERR_BAD_FORMAT;
  const uint64_t rows = load_le<uint64_t>(b + 8), cols = load_le<uint64_t>(b + 16);
  if (rows < 1 || cols < 1 || rows > (1ull << 32) || cols > (1ull << 32)) return NWC_ERR_BAD_FORMAT;
  nwc_params p{};  // fields the header does not hold (encoder-only choices) stay zero
  p.tile_rows = load_le<uint32_t>(b + 24);
  p.tile_cols = load_le<uint32_t>(b + 28);
  p.chunks_per_tile = load_le<uint32_t>(b + 32);
  p.max_code_len = load_le<uint32_t>(b + 36);
  if (!p.tile_rows || !p.tile_cols || !p.chunks_per_tile || !p.max_code_len) return NWC_ERR_BAD_FORMAT;
  Geometry g;
  if (!params_resolve(&p, &g)) return NWC_ERR_BAD_FORMAT;
  if (load_le<uint32_t>(b + 40) != 1 || load_le<uint32_t>(b + 44) != 0) return NWC_ERR_BAD_FORMAT;
  const uint64_t sw = load_le<uint64_t>(b + 72);
  if (sw > 0xFFFFFFFFull) return NWC_ERR_BAD_FORMAT;
  layout(&g, rows, cols, sw);
  const uint64_t want[] = {g.raw_ld, g.n_tiles, g.n_chunks, sw, g.off_code_len, g.off_table,
                           g.off_tile_words, g.off_chunk_bits, g.off_raw, g.off_stream, g.total};
  for (int i = 0; i < 11; i++)
    if (load_le<uint64_t>(b + 48 + 8 * i) != want[i]) return NWC_ERR_BAD_FORMAT;
  if (g.total > bytes) return NWC_ERR_BAD_FORMAT;

  const uint8_t* len = b + g.off_code_len;
  uint16_t code[256];
  unsigned nsym = 0;
  for (int s = 0; s < 256; s++) {
    if (len[s] > g.lmax) return NWC_ERR_BAD_FORMAT;
    nsym += len[s] != 0;
  }
  if (!nsym || !canonical(len, code)) return NWC_ERR_BAD_FORMAT;
  uint32_t table[kTableSize];
  build_table(len, table);
  for (uint32_t i = 0; i < kTableSize; i++)
    if (load_le<uint32_t>(b + g.off_table + 4 * i) != table[i]) return NWC_ERR_BAD_FORMAT;

  uint64_t payload = 0;
  uint32_t max_tw = 0;
  uint64_t max_cb = 0;
  if (load_le<uint32_t>(b + g.off_tile_words) != 0) return NWC_ERR_BAD_FORMAT;
  for (uint64_t t = 0; t < g.n_tiles; t++) {
    uint64_t bits = 0;
    for (uint32_t c = 0; c < g.s; c++) {
      const uint32_t cb = load_le<uint16_t>(b + g.off_chunk_bits + 2 * (t * g.s + c));
      // a chunk's bits lie between 1 and lmax per symbol it holds
      const uint64_t ti = t / g.n_tc, tj = t % g.n_tc;
      const uint64_t nr = std::min<uint64_t>(rows, ti * g.tr + g.tr) - ti * g.tr;
      const uint64_t tile_c1 = std::min<uint64_t>(cols, tj * g.tc + g.tc);
      const uint64_t c0 = tj * g.tc + static_cast<uint64_t>(c) * g.v;
      const uint64_t nc = c0 < tile_c1 ? std::min<uint64_t>(tile_c1, c0 + g.v) - c0 : 0;
      if (cb < nr * nc || cb > nr * nc * g.lmax) return NWC_ERR_BAD_FORMAT;
      bits += cb;
      max_cb = std::max<uint64_t>(max_cb, cb);
    }
    const uint32_t a = load_le<uint32_t>(b + g.off_tile_words + 4 * t);
    const uint32_t e = load_le<uint32_t>(b + g.off_tile_words + 4 * (t + 1));
    if (e < a || e - a != (bits + 31) / 32) return NWC_ERR_BAD_FORMAT;
    max_tw = std::max(max_tw, e - a);
    payload += bits;
  }
  if (load_le<uint32_t>(b + g.off_tile_words + 4 * g.n_tiles) != sw) return NWC_ERR_BAD_FORMAT;

  std::memset(info, 0, sizeof(*info));
  info->rows = rows;
  info->cols = cols;
  info->blob_bytes = g.total;
  info->tile_rows = g.tr;
  info->tile_cols = g.tc;
  info->chunks_per_tile = g.s;
  info->max_code_len = g.lmax;
  info->n_tiles = g.n_tiles;
  info->n_chunks = g.n_chunks;
  info->raw_ld = g.raw_ld;
  info->stream_words = sw;
  info->off_code_len = g.off_code_len;
  info->off_table = g.off_table;
  info->off_tile_words = g.off_tile_words;
  info->off_chunk_bits = g.off_chunk_bits;
  info->off_raw = g.off_raw;
  info->off_stream = g.off_stream;
  info->max_tile_words = max_tw;
  info->n_symbols = nsym;
  info->max_chunk_bits = static_cast<uint32_t>(max_cb);
  info->payload_bits = payload;
  std::memcpy(info->code_len, len, 256);
  return NWC_OK;
}

// Re-derive the geometry of an nwc_info (for the device entry points).
bool info_geometry(const nwc_info* info, Geometry* g) {
  if (!info) return false;
  nwc_params p{info->tile_rows, info->tile_cols, info->chunks_per_tile, info->max_code_len, 0, 0};
  if (!p.tile_rows || !p.tile_cols || !p.chunks_per_tile || !p.max_code_len) return false;
  if (!params_resolve(&p, g)) return false;
  if (info->rows < 1 || info->cols < 1) return false;
  layout(g, info->rows, info->cols, info->stream_words);
  return g->n_tiles == info->n_tiles && g->total == info->blob_bytes && g->off_raw == info->off_raw &&
         g->off_stream == info->off_stream && g->off_table == info->off_table &&
         g->off_tile_words == info->off_tile_words && g->off_chunk_bits == info->off_chunk_bits &&
         g->raw_ld == info->raw_ld;
}

}  // namespace nwc
