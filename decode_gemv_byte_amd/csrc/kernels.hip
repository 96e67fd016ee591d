// HIP kernels of libnwc for gfx950 (CDNA4) and the C-ABI entry points that
// launch them.
//
// Method (pages): weights stay compressed in HBM -- raw sign+fraction byte plus
// Huffman-coded exponent -- and are decoded on chip right before the product,
// so no decompressed weight is written to memory ("NWC -- Neural Weight
// Compression", How it works, "Fused kernel"; "Unweight ...", Direct GPU
// Decompression).  Token generation is bandwidth bound, so fewer bytes read
// means a faster matrix-vector product (NWC, opening section; GINIGEN AI feed,
// "A bandwidth ceiling, not a promise").
//
// Kernel structure (MI355X-specific; not the pages' NVIDIA design):
//  * A wavefront (64 lanes) owns one tile of TR rows x 512 columns at a time.
//    Lane l owns chunk l: all TR rows of columns [8l, 8l+8), decoded row by
//    row.  Raw-plane loads are 8 bytes per lane per row, 512 contiguous bytes
//    per wavefront per row.
//  * The tile's exponent stream (word aligned, about 2.7 KB) is staged in LDS
//    with coalesced loads; each lane finds its chunk's start bit by a
//    wavefront prefix sum over the chunk lengths.
//  * The 4096-entry decode table lives in LDS (16 KB per workgroup).  One
//    lookup of the 12-bit window yields two exponents already placed at BF16
//    bit positions 7..14 and 23..30; a byte permute spreads two raw bytes and
//    one bit-field insert builds two BF16 weights in one dword.
//  * B = 1: v_dot2c_f32_bf16 accumulates into one FP32 register per row
//    (subnormal inputs are kept); a transposed butterfly reduces the TR row
//    sums across lanes; per-(column tile, row) partials go to the workspace
//    and a second kernel adds them in column-tile order.
//  * B = 2..16: decoded BF16 rows go to LDS and feed
//    v_mfma_f32_16x16x32_bf16 (A = 16 weight rows x 32 columns, B = the
//    batch rows of X padded to 16).
//  * Every read from the blob is clamped to its sections.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "nwc_internal.hpp"

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kTable = 4096;
constexpr int kGuardWords = 4;
constexpr uint32_t kExpMask = 0x7F807F80u;  // exponent bits of two packed BF16

struct BlobDev {
  const uint32_t* table;
  const uint32_t* tile_words;
  const uint16_t* chunk_bits;
  const uint8_t* raw;
  const uint32_t* stream;
  uint64_t rows, cols, raw_ld;
  uint64_t n_tiles;
  uint32_t n_tc, tr, tc, s, v;
  uint32_t stream_words;
  uint32_t buf_words;  // LDS stream buffer per wavefront (>= max tile words + guard)
};

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Exclusive prefix sum of v across the 64 lanes.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v) {
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t y = __shfl_up(incl, off, kWave);
    if (lane_id() >= static_cast<uint32_t>(off)) incl += y;
  }
  return incl - v;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copy the decode table into LDS (whole workgroup).
__device__ __forceinline__ void load_table(uint32_t* lds_table, const uint32_t* table) {
  const uint4* src = reinterpret_cast<const uint4*>(table);
  uint4* dst = reinterpret_cast<uint4*>(lds_table);
  for (int i = threadIdx.x; i < kTable / 4; i += blockDim.x) dst[i] = src[i];
}

// Stage tile t's stream words into this wavefront's LDS buffer; returns the
// number of words (clamped to the buffer and to the stream).
__device__ __forceinline__ void stage_tile(const BlobDev& b, uint64_t t, uint32_t* buf) {
  const uint32_t w0 = b.tile_words[t];
  uint32_t w1 = b.tile_words[t + 1];
  w1 = w1 < w0 ? w0 : w1;
  uint32_t n = w1 - w0;
  const uint32_t cap = b.buf_words - kGuardWords;
  n = n > cap ? cap : n;
  for (uint32_t i = lane_id(); i < n + kGuardWords; i += kWave) {
    const uint32_t g = w0 + i;
    buf[i] = (i < n && g < b.stream_words) ? b.stream[g] : 0u;
  }
  wave_sync_lds();
}

// 64-bit window at bit q of the LDS buffer, shifted so bit q is bit 0.
__device__ __forceinline__ uint32_t window_at(const uint32_t* buf, uint32_t q, uint32_t limit) {
  uint32_t wi = q >> 5;
  wi = wi > limit ? limit : wi;
  const uint32_t lo = buf[wi], hi = buf[wi + 1];
  return __builtin_amdgcn_alignbit(hi, lo, q);
}

// Decode the next two exponents at bit q: returns a dword with exponent 0 at
// bits 7..14, exponent 1 at bits 23..30, and advances q.
__device__ __forceinline__ uint32_t decode_pair(const uint32_t* tab, const uint32_t* buf, uint32_t& q,
                                                uint32_t limit) {
  const uint32_t win = window_at(buf, q, limit);
  uint32_t ent = tab[win & 0xFFFu];
  if (ent >> 31) {  // second code did not fit in the 12-bit window
    const uint32_t l0 = ent & 0xFu;
    const uint32_t ent2 = tab[(win >> l0) & 0xFFFu];
    // the merged advance l0 + l1 can reach 24: it uses bits 0..4 (bits
    // 4..6 are zero in table entries)
    ent = (ent & 0x7F80u) | ((ent2 & 0x7F80u) << 16) | (l0 + ((ent2 >> 16) & 0xFu));
  }
  q += ent & 0x1Fu;
  return ent;
}

// Two BF16 weights from the pair entry and 4 raw bytes; `hi` selects raw
// bytes 2,3 instead of 0,1.
__device__ __forceinline__ uint32_t assemble(uint32_t ent, uint32_t raw4, bool hi) {
  const uint32_t spread = __builtin_amdgcn_perm(raw4, raw4, hi ? 0x03030202u : 0x01010000u);
  return (ent & kExpMask) | (spread & ~kExpMask);
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x),
                                         acc, false);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Transposed butterfly: on entry every lane holds R partial sums (rows
// 0..R-1); on exit lane l with (l & (64/R - 1)) == 0 holds the full sum of
// row l / (64/R), summed in a fixed order.
template <int R>
__device__ __forceinline__ float reduce_rows(float (&v)[R]) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int half = R / 2, m = 32; half >= 1; half >>= 1, m >>= 1) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < half; i++) {
      const float keep = up ? v[half + i] : v[i];
      const float send = up ? v[i] : v[half + i];
      v[i] = keep + __shfl_xor(send, m, kWave);
    }
  }
  float s = v[0];
#pragma unroll
  for (int m = 32 / R; m >= 1; m >>= 1) s += __shfl_xor(s, m, kWave);
  return s;
}

// ------------------------------------------------------------------ decode

// Fast path: S = 64 chunks of 8 columns, K a multiple of 8.
template <int TR>
__global__ __launch_bounds__(kThreads) void k_decode_fast(BlobDev b, uint16_t* __restrict__ out, uint64_t ld) {
  extern __shared__ uint32_t lds[];
  uint32_t* tab = lds;
  const uint32_t wave = threadIdx.x / kWave;
  uint32_t* buf = lds + kTable + wave * b.buf_words;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint32_t limit = b.buf_words - 2;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + wave; t < b.n_tiles;
       t += static_cast<uint64_t>(gridDim.x) * kWavesPerBlock) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * TR;
    const uint32_t nrows = static_cast<uint32_t>(umin64(TR, b.rows - row0));
    const uint64_t c0 = tj * 512 + lane * 8;
    const bool active = c0 < b.cols;
    const uint32_t cb = b.chunk_bits[t * 64 + lane];
    uint32_t q = wave_excl_scan(cb);
    stage_tile(b, t, buf);
    if (active) {
      for (uint32_t r = 0; r < nrows; r++) {
        const uint2 rw = *reinterpret_cast<const uint2*>(b.raw + (row0 + r) * b.raw_ld + c0);
        uint4 o;
        o.x = assemble(decode_pair(tab, buf, q, limit), rw.x, false);
        o.y = assemble(decode_pair(tab, buf, q, limit), rw.x, true);
        o.z = assemble(decode_pair(tab, buf, q, limit), rw.y, false);
        o.w = assemble(decode_pair(tab, buf, q, limit), rw.y, true);
        *reinterpret_cast<uint4*>(out + (row0 + r) * ld + c0) = o;
      }
    }
  }
}

// Generic path: any geometry, one symbol at a time.
__global__ __launch_bounds__(kThreads) void k_decode_generic(BlobDev b, uint16_t* __restrict__ out, uint64_t ld) {
  extern __shared__ uint32_t lds[];
  uint32_t* tab = lds;
  const uint32_t wave = threadIdx.x / kWave;
  uint32_t* buf = lds + kTable + wave * b.buf_words;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint32_t limit = b.buf_words - 2;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + wave; t < b.n_tiles;
       t += static_cast<uint64_t>(gridDim.x) * kWavesPerBlock) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * b.tr;
    const uint64_t r1 = umin64(b.rows, row0 + b.tr);
    const uint64_t tile_c1 = umin64(b.cols, tj * b.tc + b.tc);
    stage_tile(b, t, buf);
    uint32_t base = 0;  // start bit of the first chunk handled in this round
    for (uint32_t c0i = 0; c0i < b.s; c0i += kWave) {
      const uint32_t c = c0i + lane;
      const uint32_t cb = c < b.s ? b.chunk_bits[t * b.s + c] : 0u;
      const uint32_t excl = wave_excl_scan(cb);
      uint32_t q = base + excl;
      base += __shfl(excl + cb, kWave - 1, kWave);
      if (c >= b.s) continue;
      const uint64_t cc0 = tj * b.tc + static_cast<uint64_t>(c) * b.v;
      if (cc0 >= tile_c1) continue;
      const uint64_t cc1 = umin64(tile_c1, cc0 + b.v);
      for (uint64_t r = row0; r < r1; r++)
        for (uint64_t k = cc0; k < cc1; k++) {
          const uint32_t ent = tab[window_at(buf, q, limit) & 0xFFFu];
          q += (ent >> 16) & 0xFu;
          const uint32_t e = (ent >> 7) & 0xFFu;
          const uint32_t rb = b.raw[r * b.raw_ld + k];
          out[r * ld + k] = static_cast<uint16_t>(((rb & 0x80u) << 8) | (e << 7) | (rb & 0x7Fu));
        }
    }
  }
}

// -------------------------------------------------------------------- GEMV

// Fast path, batch 1: partial[tj * rows + n] = sum over the tile's columns.
template <int TR>
__global__ __launch_bounds__(kThreads) void k_gemv_fast(BlobDev b, const uint16_t* __restrict__ x,
                                                        float* __restrict__ partial) {
  extern __shared__ uint32_t lds[];
  uint32_t* tab = lds;
  const uint32_t wave = threadIdx.x / kWave;
  uint32_t* buf = lds + kTable + wave * b.buf_words;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint32_t limit = b.buf_words - 2;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + wave; t < b.n_tiles;
       t += static_cast<uint64_t>(gridDim.x) * kWavesPerBlock) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * TR;
    const uint32_t nrows = static_cast<uint32_t>(umin64(TR, b.rows - row0));
    const uint64_t c0 = tj * 512 + lane * 8;
    const bool active = c0 < b.cols;
    const uint32_t cb = b.chunk_bits[t * 64 + lane];
    uint32_t q = wave_excl_scan(cb);
    stage_tile(b, t, buf);
    float acc[TR];
#pragma unroll
    for (int r = 0; r < TR; r++) acc[r] = 0.0f;
    if (active) {
      const uint4 xv = *reinterpret_cast<const uint4*>(x + c0);
      uint2 rw[TR];
#pragma unroll
      for (int r = 0; r < TR; r++)
        rw[r] = r < static_cast<int>(nrows)
                    ? *reinterpret_cast<const uint2*>(b.raw + (row0 + r) * b.raw_ld + c0)
                    : make_uint2(0, 0);
#pragma unroll
      for (int r = 0; r < TR; r++) {
        if (r < static_cast<int>(nrows)) {
          float a = 0.0f;
          a = dot2(assemble(decode_pair(tab, buf, q, limit), rw[r].x, false), xv.x, a);
          a = dot2(assemble(decode_pair(tab, buf, q, limit), rw[r].x, true), xv.y, a);
          a = dot2(assemble(decode_pair(tab, buf, q, limit), rw[r].y, false), xv.z, a);
          a = dot2(assemble(decode_pair(tab, buf, q, limit), rw[r].y, true), xv.w, a);
          acc[r] = a;
        }
      }
    }
    const float s = reduce_rows<TR>(acc);
    constexpr uint32_t lanes_per_row = kWave / TR;
    if ((lane & (lanes_per_row - 1)) == 0) {
      const uint32_t r = lane / lanes_per_row;
      if (r < nrows) partial[tj * b.rows + row0 + r] = s;
    }
  }
}

// Generic path for any geometry; batch rows handled one after another.
// partial[(tj * batch + beta) * rows + n].
__global__ __launch_bounds__(kThreads) void k_gemv_generic(BlobDev b, const uint16_t* __restrict__ X, uint64_t ldx,
                                                           int batch, float* __restrict__ partial) {
  extern __shared__ uint32_t lds[];
  uint32_t* tab = lds;
  const uint32_t wave = threadIdx.x / kWave;
  uint32_t* buf = lds + kTable + wave * b.buf_words;
  float* rowsum = reinterpret_cast<float*>(lds + kTable + kWavesPerBlock * b.buf_words) +
                  wave * static_cast<size_t>(b.tr) * b.s;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint32_t limit = b.buf_words - 2;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + wave; t < b.n_tiles;
       t += static_cast<uint64_t>(gridDim.x) * kWavesPerBlock) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * b.tr;
    const uint32_t nrows = static_cast<uint32_t>(umin64(b.tr, b.rows - row0));
    const uint64_t tile_c1 = umin64(b.cols, tj * b.tc + b.tc);
    stage_tile(b, t, buf);
    for (int beta = 0; beta < batch; beta++) {
      const uint16_t* x = X + beta * ldx;
      uint32_t base = 0;
      for (uint32_t c0i = 0; c0i < b.s; c0i += kWave) {
        const uint32_t c = c0i + lane;
        const uint32_t cb = c < b.s ? b.chunk_bits[t * b.s + c] : 0u;
        const uint32_t excl = wave_excl_scan(cb);
        uint32_t q = base + excl;
        base += __shfl(excl + cb, kWave - 1, kWave);
        if (c >= b.s) continue;
        const uint64_t cc0 = tj * b.tc + static_cast<uint64_t>(c) * b.v;
        const uint64_t cc1 = cc0 < tile_c1 ? umin64(tile_c1, cc0 + b.v) : cc0;
        for (uint32_t r = 0; r < nrows; r++) {
          float a = 0.0f;
          for (uint64_t k = cc0; k < cc1; k++) {
            const uint32_t ent = tab[window_at(buf, q, limit) & 0xFFFu];
            q += (ent >> 16) & 0xFu;
            const uint32_t e = (ent >> 7) & 0xFFu;
            const uint32_t rb = b.raw[(row0 + r) * b.raw_ld + k];
            const uint32_t wbits = (((rb & 0x80u) << 8) | (e << 7) | (rb & 0x7Fu)) << 16;
            const float xf = __builtin_bit_cast(float, static_cast<uint32_t>(x[k]) << 16);
            a = __builtin_fmaf(__builtin_bit_cast(float, wbits), xf, a);
          }
          rowsum[r * b.s + c] = a;
        }
      }
      wave_sync_lds();
      for (uint32_t r = lane; r < nrows; r += kWave) {
        float s = 0.0f;
        for (uint32_t c = 0; c < b.s; c++) s += rowsum[r * b.s + c];
        partial[(tj * batch + beta) * b.rows + row0 + r] = s;
      }
      wave_sync_lds();
    }
  }
}

// Skinny GEMM with MFMA, batch 2..16, TR = 16:
// partial[(tj * batch + beta) * rows + n].
__global__ __launch_bounds__(kThreads) void k_gemm_mfma(BlobDev b, const uint16_t* __restrict__ X, uint64_t ldx,
                                                        int batch, float* __restrict__ partial) {
  constexpr int TR = 16;
  constexpr int kRowPad = 512 + 8;  // bf16 per LDS row (pad against bank conflicts)
  extern __shared__ uint32_t lds[];
  uint32_t* tab = lds;
  const uint32_t wave = threadIdx.x / kWave;
  uint32_t* buf = lds + kTable + wave * b.buf_words;
  uint16_t* wt = reinterpret_cast<uint16_t*>(lds + kTable + kWavesPerBlock * b.buf_words) +
                 wave * static_cast<size_t>(TR) * kRowPad;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint32_t limit = b.buf_words - 2;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + wave; t < b.n_tiles;
       t += static_cast<uint64_t>(gridDim.x) * kWavesPerBlock) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * TR;
    const uint32_t nrows = static_cast<uint32_t>(umin64(TR, b.rows - row0));
    const uint64_t c0 = tj * 512 + lane * 8;
    const bool active = c0 < b.cols;
    const uint32_t cb = b.chunk_bits[t * 64 + lane];
    uint32_t q = wave_excl_scan(cb);
    stage_tile(b, t, buf);
    // decode the tile into LDS, rows past the matrix (or columns past the
    // edge) as zeros
    for (int r = 0; r < TR; r++) {
      uint4 o = make_uint4(0, 0, 0, 0);
      if (active && r < static_cast<int>(nrows)) {
        const uint2 rw = *reinterpret_cast<const uint2*>(b.raw + (row0 + r) * b.raw_ld + c0);
        o.x = assemble(decode_pair(tab, buf, q, limit), rw.x, false);
        o.y = assemble(decode_pair(tab, buf, q, limit), rw.x, true);
        o.z = assemble(decode_pair(tab, buf, q, limit), rw.y, false);
        o.w = assemble(decode_pair(tab, buf, q, limit), rw.y, true);
      }
      *reinterpret_cast<uint4*>(wt + r * kRowPad + lane * 8) = o;
    }
    wave_sync_lds();
    // D[16 rows x 16 batch] += W[16 x 32] * X^T[32 x 16] over 16 column blocks
    f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t mrow = lane % 16, kq = lane / 16;  // A: row, 8-column group
    const uint32_t nb = lane % 16;                    // B: batch column
#pragma unroll 4
    for (int kb = 0; kb < 16; kb++) {
      const uint32_t kcol = kb * 32 + kq * 8;
      const uint4 av = *reinterpret_cast<const uint4*>(wt + mrow * kRowPad + kcol);
      uint4 bv = make_uint4(0, 0, 0, 0);
      const uint64_t gk = tj * 512 + kcol;
      if (static_cast<int>(nb) < batch && gk < b.cols)
        bv = *reinterpret_cast<const uint4*>(X + nb * ldx + gk);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), d, 0, 0, 0);
    }
    wave_sync_lds();
    // lane holds D[4 * (lane / 16) + i][lane % 16]
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t r = 4 * (lane / 16) + i;
      if (static_cast<int>(nb) < batch && r < nrows) partial[(tj * batch + nb) * b.rows + row0 + r] = d[i];
    }
  }
}

// y[beta, n] = sum over column tiles of partial, in tile order.
__global__ void k_reduce(const float* __restrict__ partial, uint64_t rows, uint32_t n_tc, int batch,
                         void* __restrict__ y, uint64_t ldy, int y_f32) {
  const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * static_cast<uint64_t>(batch)) return;
  const uint64_t beta = i / rows, n = i % rows;
  float s = 0.0f;
  for (uint32_t tj = 0; tj < n_tc; tj++) s += partial[(tj * static_cast<uint64_t>(batch) + beta) * rows + n];
  if (y_f32)
    static_cast<float*>(y)[beta * ldy + n] = s;
  else
    static_cast<uint16_t*>(y)[beta * ldy + n] = f32_to_bf16_rne(s);
}

// ------------------------------------------------- uncompressed comparator

// Same tiling and reduction as k_gemv_fast, reading BF16 weights directly.
template <int TR>
__global__ __launch_bounds__(kThreads) void k_gemv_bf16(const uint16_t* __restrict__ w, uint64_t rows,
                                                        uint64_t cols, uint64_t ld, uint32_t n_tc,
                                                        const uint16_t* __restrict__ x,
                                                        float* __restrict__ partial) {
  const uint32_t wave = threadIdx.x / kWave;
  const uint32_t lane = lane_id();
  const uint64_t n_tiles = ((rows + TR - 1) / TR) * n_tc;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + wave; t < n_tiles;
       t += static_cast<uint64_t>(gridDim.x) * kWavesPerBlock) {
    const uint64_t ti = t / n_tc, tj = t % n_tc;
    const uint64_t row0 = ti * TR;
    const uint32_t nrows = static_cast<uint32_t>(umin64(TR, rows - row0));
    const uint64_t c0 = tj * 512 + lane * 8;
    float acc[TR];
#pragma unroll
    for (int r = 0; r < TR; r++) acc[r] = 0.0f;
    if (c0 < cols) {
      const uint4 xv = *reinterpret_cast<const uint4*>(x + c0);
#pragma unroll
      for (int r = 0; r < TR; r++) {
        if (r < static_cast<int>(nrows)) {
          const uint4 wv = *reinterpret_cast<const uint4*>(w + (row0 + r) * ld + c0);
          float a = 0.0f;
          a = dot2(wv.x, xv.x, a);
          a = dot2(wv.y, xv.y, a);
          a = dot2(wv.z, xv.z, a);
          a = dot2(wv.w, xv.w, a);
          acc[r] = a;
        }
      }
    }
    const float s = reduce_rows<TR>(acc);
    constexpr uint32_t lanes_per_row = kWave / TR;
    if ((lane & (lanes_per_row - 1)) == 0) {
      const uint32_t r = lane / lanes_per_row;
      if (r < nrows) partial[tj * rows + row0 + r] = s;
    }
  }
}

// ------------------------------------------------------------- host glue

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Launch {
  BlobDev b;
  bool fast;       // S = 64, V = 8, TR in {8, 16, 32}, K % 8 == 0
  size_t lds;      // dynamic LDS bytes (table + stream buffers)
  unsigned grid;
};

nwc_status prepare(const nwc_info* info, const void* blob_dev, Launch* L) {
  nwc::Geometry g;
  if (!info || !blob_dev || !nwc::info_geometry(info, &g)) return NWC_ERR_INVALID_ARG;
  if (!aligned(blob_dev, 256)) return NWC_ERR_ALIGNMENT;
  if (info->max_tile_words > 3u * 65536u) return NWC_ERR_BAD_FORMAT;
  const uint8_t* base = static_cast<const uint8_t*>(blob_dev);
  BlobDev& b = L->b;
  b.table = reinterpret_cast<const uint32_t*>(base + g.off_table);
  b.tile_words = reinterpret_cast<const uint32_t*>(base + g.off_tile_words);
  b.chunk_bits = reinterpret_cast<const uint16_t*>(base + g.off_chunk_bits);
  b.raw = base + g.off_raw;
  b.stream = reinterpret_cast<const uint32_t*>(base + g.off_stream);
  b.rows = g.rows;
  b.cols = g.cols;
  b.raw_ld = g.raw_ld;
  b.n_tiles = g.n_tiles;
  b.n_tc = static_cast<uint32_t>(g.n_tc);
  b.tr = g.tr;
  b.tc = g.tc;
  b.s = g.s;
  b.v = g.v;
  b.stream_words = static_cast<uint32_t>(g.stream_words);
  b.buf_words = (info->max_tile_words + kGuardWords + 3) & ~3u;
  L->fast = g.s == 64 && g.v == 8 && (g.tr == 8 || g.tr == 16 || g.tr == 32) && g.cols % 8 == 0;
  L->lds = (kTable + static_cast<size_t>(kWavesPerBlock) * b.buf_words) * 4;
  const uint64_t blocks = (g.n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  L->grid = static_cast<unsigned>(std::min<uint64_t>(blocks, 256ull * 8));
  return NWC_OK;
}

template <typename K>
hipError_t set_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds));
}

constexpr size_t kMaxLds = 160 * 1024;

nwc_status launched() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? NWC_OK : NWC_ERR_HIP;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

const char* nwc_status_str(nwc_status s) {
  switch (s) {
    case NWC_OK: return "NWC_OK";
    case NWC_ERR_INVALID_ARG: return "NWC_ERR_INVALID_ARG";
    case NWC_ERR_BUFFER_TOO_SMALL: return "NWC_ERR_BUFFER_TOO_SMALL";
    case NWC_ERR_BAD_FORMAT: return "NWC_ERR_BAD_FORMAT";
    case NWC_ERR_UNSUPPORTED: return "NWC_ERR_UNSUPPORTED";
    case NWC_ERR_ALIGNMENT: return "NWC_ERR_ALIGNMENT";
    case NWC_ERR_HIP: return "NWC_ERR_HIP";
  }
  return "NWC_ERR_UNKNOWN";
}

nwc_status nwc_encode_bound(uint64_t rows, uint64_t cols, const nwc_params* p, size_t* max_bytes) {
  return nwc::encode_bound(rows, cols, p, max_bytes);
}

nwc_status nwc_encode(const uint16_t* w, uint64_t rows, uint64_t cols, uint64_t ld, const nwc_params* p,
                      void* blob, size_t cap, size_t* used) {
  return nwc::encode(w, rows, cols, ld, p, blob, cap, used);
}

nwc_status nwc_inspect(const void* blob, size_t bytes, nwc_info* info) { return nwc::inspect(blob, bytes, info); }

nwc_status nwc_workspace_size(const nwc_info* info, int batch, size_t* bytes) {
  nwc::Geometry g;
  if (!info || !bytes || batch < 1 || batch > 16 || !nwc::info_geometry(info, &g)) return NWC_ERR_INVALID_ARG;
  *bytes = static_cast<size_t>(g.n_tc) * batch * g.rows * sizeof(float);
  return NWC_OK;
}

nwc_status nwc_decode(const nwc_info* info, const void* blob_dev, uint16_t* w_dev, uint64_t ld, void* stream) {
  if (!w_dev) return NWC_ERR_INVALID_ARG;
  Launch L;
  nwc_status st = prepare(info, blob_dev, &L);
  if (st) return st;
  if (ld < L.b.cols) return NWC_ERR_INVALID_ARG;
  const bool vec = aligned(w_dev, 16) && ld % 8 == 0;
  if (L.lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.fast && vec) {
    switch (L.b.tr) {
      case 8:
        if (set_lds(k_decode_fast<8>, L.lds) != hipSuccess) return NWC_ERR_HIP;
        k_decode_fast<8><<<L.grid, kThreads, L.lds, s>>>(L.b, w_dev, ld);
        break;
      case 16:
        if (set_lds(k_decode_fast<16>, L.lds) != hipSuccess) return NWC_ERR_HIP;
        k_decode_fast<16><<<L.grid, kThreads, L.lds, s>>>(L.b, w_dev, ld);
        break;
      default:
        if (set_lds(k_decode_fast<32>, L.lds) != hipSuccess) return NWC_ERR_HIP;
        k_decode_fast<32><<<L.grid, kThreads, L.lds, s>>>(L.b, w_dev, ld);
        break;
    }
  } else {
    if (!aligned(w_dev, 2)) return NWC_ERR_ALIGNMENT;
    if (set_lds(k_decode_generic, L.lds) != hipSuccess) return NWC_ERR_HIP;
    k_decode_generic<<<L.grid, kThreads, L.lds, s>>>(L.b, w_dev, ld);
  }
  return launched();
}

static nwc_status launch_reduce(const float* ws, uint64_t rows, uint32_t n_tc, int batch, void* y, uint64_t ldy,
                                nwc_out_type yt, hipStream_t s) {
  const uint64_t n = rows * static_cast<uint64_t>(batch);
  const unsigned threads = 256;
  const unsigned blocks = static_cast<unsigned>((n + threads - 1) / threads);
  k_reduce<<<blocks, threads, 0, s>>>(ws, rows, n_tc, batch, y, ldy, yt == NWC_OUT_F32 ? 1 : 0);
  return launched();
}

static nwc_status gemm_common(const nwc_info* info, const void* blob_dev, const uint16_t* X, uint64_t ldx, int batch,
                              void* Y, uint64_t ldy, nwc_out_type yt, void* ws, size_t ws_bytes, void* stream) {
  if (!X || !Y || !ws) return NWC_ERR_INVALID_ARG;
  if (yt != NWC_OUT_BF16 && yt != NWC_OUT_F32) return NWC_ERR_INVALID_ARG;
  Launch L;
  nwc_status st = prepare(info, blob_dev, &L);
  if (st) return st;
  size_t need = 0;
  nwc_workspace_size(info, batch, &need);
  if (ws_bytes < need) return NWC_ERR_BUFFER_TOO_SMALL;
  if (batch > 1 && (ldx < L.b.cols || ldy < L.b.rows)) return NWC_ERR_INVALID_ARG;
  if (!aligned(ws, 16) || !aligned(Y, yt == NWC_OUT_F32 ? 4 : 2) || !aligned(X, 2)) return NWC_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(ws);
  const bool xvec = aligned(X, 16) && (batch == 1 || ldx % 8 == 0);
  if (batch == 1 && L.fast && xvec) {
    if (L.lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
    switch (L.b.tr) {
      case 8:
        if (set_lds(k_gemv_fast<8>, L.lds) != hipSuccess) return NWC_ERR_HIP;
        k_gemv_fast<8><<<L.grid, kThreads, L.lds, s>>>(L.b, X, part);
        break;
      case 16:
        if (set_lds(k_gemv_fast<16>, L.lds) != hipSuccess) return NWC_ERR_HIP;
        k_gemv_fast<16><<<L.grid, kThreads, L.lds, s>>>(L.b, X, part);
        break;
      default:
        if (set_lds(k_gemv_fast<32>, L.lds) != hipSuccess) return NWC_ERR_HIP;
        k_gemv_fast<32><<<L.grid, kThreads, L.lds, s>>>(L.b, X, part);
        break;
    }
  } else if (batch > 1 && L.fast && L.b.tr == 16 && xvec) {
    const size_t lds = L.lds + static_cast<size_t>(kWavesPerBlock) * 16 * (512 + 8) * 2;
    if (lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
    if (set_lds(k_gemm_mfma, lds) != hipSuccess) return NWC_ERR_HIP;
    k_gemm_mfma<<<L.grid, kThreads, lds, s>>>(L.b, X, ldx, batch, part);
  } else {
    const size_t lds = L.lds + static_cast<size_t>(kWavesPerBlock) * L.b.tr * L.b.s * 4;
    if (lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
    if (set_lds(k_gemv_generic, lds) != hipSuccess) return NWC_ERR_HIP;
    k_gemv_generic<<<L.grid, kThreads, lds, s>>>(L.b, X, batch == 1 ? 0 : ldx, batch, part);
  }
  st = launched();
  if (st) return st;
  return launch_reduce(part, L.b.rows, L.b.n_tc, batch, Y, batch == 1 ? 0 : ldy, yt, s);
}

nwc_status nwc_gemv(const nwc_info* info, const void* blob_dev, const uint16_t* x_dev, void* y_dev,
                    nwc_out_type y_type, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(info, blob_dev, x_dev, 0, 1, y_dev, 0, y_type, ws, ws_bytes, stream);
}

nwc_status nwc_gemm_skinny(const nwc_info* info, const void* blob_dev, const uint16_t* X_dev, uint64_t ldx, int batch,
                           void* Y_dev, uint64_t ldy, nwc_out_type y_type, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 2 || batch > 16) return NWC_ERR_INVALID_ARG;
  return gemm_common(info, blob_dev, X_dev, ldx, batch, Y_dev, ldy, y_type, ws, ws_bytes, stream);
}

nwc_status nwc_bf16_workspace_size(uint64_t rows, uint64_t cols, size_t* bytes) {
  if (!bytes || rows < 1 || cols < 1) return NWC_ERR_INVALID_ARG;
  *bytes = ((cols + 511) / 512) * rows * sizeof(float);
  return NWC_OK;
}

nwc_status nwc_gemv_bf16(const uint16_t* w_dev, uint64_t rows, uint64_t cols, uint64_t ld, const uint16_t* x_dev,
                         void* y_dev, nwc_out_type y_type, void* ws, size_t ws_bytes, void* stream) {
  if (!w_dev || !x_dev || !y_dev || !ws || rows < 1 || cols < 1 || ld < cols) return NWC_ERR_INVALID_ARG;
  if (y_type != NWC_OUT_BF16 && y_type != NWC_OUT_F32) return NWC_ERR_INVALID_ARG;
  size_t need = 0;
  nwc_bf16_workspace_size(rows, cols, &need);
  if (ws_bytes < need) return NWC_ERR_BUFFER_TOO_SMALL;
  if (cols % 8 || ld % 8 || !aligned(w_dev, 16) || !aligned(x_dev, 16) || !aligned(ws, 16)) return NWC_ERR_ALIGNMENT;
  if (!aligned(y_dev, y_type == NWC_OUT_F32 ? 4 : 2)) return NWC_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t n_tc = static_cast<uint32_t>((cols + 511) / 512);
  const uint64_t tiles = ((rows + 15) / 16) * n_tc;
  const unsigned grid = static_cast<unsigned>(std::min<uint64_t>((tiles + kWavesPerBlock - 1) / kWavesPerBlock, 256ull * 8));
  float* part = static_cast<float*>(ws);
  k_gemv_bf16<16><<<grid, kThreads, 0, s>>>(w_dev, rows, cols, ld, n_tc, x_dev, part);
  nwc_status st = launched();
  if (st) return st;
  return launch_reduce(part, rows, n_tc, 1, y_dev, 0, y_type, s);
}

}  // extern "C"
