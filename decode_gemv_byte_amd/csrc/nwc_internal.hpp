// Internal declarations shared by the host codec and the device entry points.
#pragma once

#include <array>
#include <cstddef>
#include <cstdint>

#include "nwc.h"

namespace nwc {

// Tile geometry and section layout of one blob.
struct Geometry {
  uint32_t tr = 0, tc = 0, s = 0, lmax = 0, v = 0;  // tile rows/cols, chunks, max code length, chunk cols
  uint32_t pair_fit = 0;                             // encoder only: 6-bit cap for common exponents
  uint32_t family = 0;                               // encoder only: 0 Huffman, 1 ranked unary + escape
  uint64_t rows = 0, cols = 0;
  uint64_t n_tr = 0, n_tc = 0, n_tiles = 0, n_chunks = 0;
  uint64_t raw_ld = 0, stream_words = 0;
  uint64_t off_code_len = 0, off_table = 0, off_tile_words = 0, off_chunk_bits = 0, off_raw = 0,
           off_stream = 0, total = 0;
};

bool build_lengths(const uint64_t hist[256], int lmax, uint8_t len[256], uint32_t pair_fit = 0);
bool canonical(const uint8_t len[256], uint16_t code[256]);
void build_table(const uint8_t len[256], uint32_t table[4096]);
bool params_resolve(const nwc_params* p, Geometry* g);
void layout(Geometry* g, uint64_t rows, uint64_t cols, uint64_t stream_words);
bool info_geometry(const nwc_info* info, Geometry* g);

nwc_status encode_bound(uint64_t rows, uint64_t cols, const nwc_params* p, size_t* max_bytes);
nwc_status encode(const uint16_t* w, uint64_t rows, uint64_t cols, uint64_t ld, const nwc_params* p,
                  void* blob, size_t cap, size_t* used);
nwc_status inspect(const void* blob, size_t bytes, nwc_info* info);

}  // namespace nwc
