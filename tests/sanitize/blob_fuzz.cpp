// Sanitizer fuzz driver (test infrastructure, built only by
// tests/test_sanitize.py): the library's host encoder and blob parser
// (host_codec.cpp) and the CPU oracle (nwc_oracle.c), compiled with
// -fsanitize=address,undefined so that any out-of-bounds access, use after
// free or undefined behaviour aborts the run.
//
// For `iters` random cases: draw a BF16 matrix (a random shape and one of
// several value distributions) and encoding parameters (either code family); encode it with
// nwc_encode and with the oracle; the two must agree on success and write
// the same bytes; the oracle must decode the blob to the input bits.  (The
// C-ABI entry points nwc_encode / nwc_inspect forward to these functions.)  Then
// mutate the blob (flipped bits, overwritten bytes and header fields,
// truncation) and give every mutant to both parsers: neither may crash, and
// every mutant the oracle accepts (it also decodes every chunk) the library
// must accept too.  A mutant the library accepts is decoded by the oracle
// (an error is fine, a crash is not).  Exits non-zero at the first failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "nwc_internal.hpp"  // the library's host codec (nwc::encode, nwc::inspect behind the C ABI)

extern "C" {
int orc_encode_bound(uint64_t rows, uint64_t cols, uint32_t tr, uint32_t tc, uint32_t s, uint32_t lmax,
                     uint64_t* bytes);
int orc_encode_family(const uint16_t* w, uint64_t rows, uint64_t cols, uint64_t ld, uint32_t tr, uint32_t tc,
                      uint32_t s, uint32_t lmax, uint32_t pair_fit, uint32_t family, uint8_t* blob, uint64_t cap,
                      uint64_t* used);
int orc_decode(const uint8_t* blob, uint64_t bytes, uint16_t* w, uint64_t ld);
int orc_validate(const uint8_t* blob, uint64_t bytes);
}

namespace {

struct Rng {  // splitmix64
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  uint32_t below(uint32_t n) { return static_cast<uint32_t>(next() % n); }
};

int fail(const char* what, uint64_t it) {
  std::fprintf(stderr, "blob_fuzz: %s (case %llu)\n", what, static_cast<unsigned long long>(it));
  return 1;
}

// A BF16 pattern from one of several distributions: a narrow band of
// exponents around a scale (Gaussian-like weights), uniformly random bits,
// a couple of symbols only, or mostly zeros.
uint16_t draw(Rng& r, int mode) {
  switch (mode) {
    case 0: {
      const uint32_t e = 118 + r.below(6) + (r.below(64) == 0 ? r.below(20) : 0) - (r.below(8) == 0 ? r.below(30) : 0);
      return static_cast<uint16_t>((r.below(2) << 15) | ((e & 0xFF) << 7) | r.below(128));
    }
    case 1: return static_cast<uint16_t>(r.next());
    case 2: return static_cast<uint16_t>((r.below(2) << 15) | ((120 + r.below(2)) << 7) | r.below(128));
    default: return r.below(16) == 0 ? static_cast<uint16_t>(r.next()) : 0;
  }
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t iters = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 200;
  Rng r{argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1};
  uint64_t accepted_mutants = 0, mutants = 0;
  for (uint64_t it = 0; it < iters; it++) {
    const uint64_t rows = 1 + r.below(r.below(4) == 0 ? 300 : 40);
    const uint64_t cols = 1 + r.below(r.below(4) == 0 ? 1200 : 100);
    const int mode = static_cast<int>(r.below(4));
    std::vector<uint16_t> w(rows * cols);
    for (auto& v : w) v = draw(r, mode);
    const uint32_t trs[] = {1, 3, 4, 5, 8, 16, 32};
    const uint32_t tcs[][2] = {{512, 64}, {24, 3}, {7, 7}, {1024, 64}, {64, 8}, {512, 32}};
    const uint32_t lms[] = {6, 7, 8, 9, 11, 12};
    const uint32_t pfs[] = {0, 1, 1024};
    const auto& tc = tcs[r.below(6)];
    nwc_params p{trs[r.below(7)], tc[0], tc[1], lms[r.below(6)], pfs[r.below(3)], r.below(2)};
    size_t bound = 0;
    const nwc_status bs = nwc::encode_bound(rows, cols, &p, &bound);
    uint64_t obound = 0;
    const int obs = orc_encode_bound(rows, cols, p.tile_rows, p.tile_cols, p.chunks_per_tile, p.max_code_len, &obound);
    if ((bs == NWC_OK) != (obs == 0)) return fail("encode_bound disagrees", it);
    if (bs != NWC_OK) continue;
    std::vector<uint8_t> a(bound), b(obound);
    size_t used = 0;
    uint64_t oused = 0;
    const nwc_status es = nwc::encode(w.data(), rows, cols, cols, &p, a.data(), a.size(), &used);
    const int oes = orc_encode_family(w.data(), rows, cols, cols, p.tile_rows, p.tile_cols, p.chunks_per_tile,
                                      p.max_code_len, p.pair_fit ? p.pair_fit : 1024, p.code_family, b.data(),
                                      b.size(), &oused);
    if ((es == NWC_OK) != (oes == 0)) return fail("encode success disagrees", it);
    if (es != NWC_OK) continue;  // e.g. more distinct exponents than a short limit codes
    if (used != oused || std::memcmp(a.data(), b.data(), used) != 0) return fail("blobs differ", it);
    a.resize(used);
    std::vector<uint16_t> back(rows * cols, 0x5A5A);
    if (orc_decode(a.data(), a.size(), back.data(), cols) != 0 || back != w) return fail("round trip", it);
    nwc_info info;
    if (nwc::inspect(a.data(), a.size(), &info) != NWC_OK) return fail("valid blob rejected", it);
    for (int m = 0; m < 24; m++) {
      std::vector<uint8_t> mut(a);
      size_t len = mut.size();
      switch (r.below(5)) {
        case 0:  // flipped bits anywhere
          for (uint32_t k = 1 + r.below(4); k > 0; k--) mut[r.below(static_cast<uint32_t>(len))] ^= 1u << r.below(8);
          break;
        case 1:  // a header field overwritten with a random or extreme value
          for (int k = 0; k < 8; k++) mut[8 * r.below(17) + k] = r.below(3) == 0 ? 0xFF : static_cast<uint8_t>(r.next());
          break;
        case 2:  // truncated
          len = r.below(static_cast<uint32_t>(len));
          break;
        case 3:  // a run of bytes in the offsets / chunk lengths / stream overwritten
        {
          const size_t at = info.off_tile_words + r.below(static_cast<uint32_t>(len - info.off_tile_words));
          for (size_t k = at; k < len && k < at + 1 + r.below(16); k++) mut[k] = static_cast<uint8_t>(r.next());
          break;
        }
        default:  // a code length changed
          mut[info.off_code_len + r.below(256)] = static_cast<uint8_t>(r.below(14));
      }
      mutants++;
      nwc_info mi;
      const bool lib_ok = nwc::inspect(mut.data(), len, &mi) == NWC_OK;
      const bool orc_ok = orc_validate(mut.data(), len) == 0;
      if (orc_ok && !lib_ok) return fail("library rejects a blob the oracle accepts", it);
      if (lib_ok) {
        accepted_mutants++;
        if (mi.rows * mi.cols > (uint64_t{1} << 26)) return fail("accepted a blob larger than its bytes allow", it);
        std::vector<uint16_t> out(mi.rows * mi.cols + 1);
        orc_decode(mut.data(), len, out.data(), mi.cols);  // any status; it must not crash
      }
    }
  }
  std::printf("blob_fuzz: %llu cases, %llu mutants (%llu accepted by the library), no failure\n",
              static_cast<unsigned long long>(iters), static_cast<unsigned long long>(mutants),
              static_cast<unsigned long long>(accepted_mutants));
  return 0;
}
