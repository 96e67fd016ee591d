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
//  * A wavefront (64 lanes) decodes one tile of TR rows x 512 columns at a
//    time.  Lane l owns chunk l: all TR rows of columns [8l, 8l+8), decoded
//    row by row.  Raw-plane loads are 8 bytes per lane per row, 512
//    contiguous bytes per wavefront per row.
//  * All global loads of a tile are issued before the first use (rows past
//    the matrix edge are clamped, not branched around), so a tile costs one
//    memory latency.  The tile's exponent stream (word aligned, about 2.7 KB)
//    goes straight to LDS with global_load_lds_dwordx4; each lane finds its
//    chunk's start bit by a wavefront prefix sum over the chunk lengths.
//  * Each lane keeps a 64-bit bit buffer in two registers plus the next word,
//    so one decode step costs one LDS lookup: the 4096-entry decode table
//    (16 KB per workgroup) maps the next 12 bits to two exponents already at
//    BF16 bit positions 7..14 and 23..30.  A byte permute spreads two raw
//    bytes and one bit-field insert builds two BF16 weights in one dword.
//  * B = 1: v_dot2c_f32_bf16 accumulates one FP32 register per row (subnormal
//    inputs are kept).  A workgroup owns whole row blocks and splits their
//    column tiles across its wavefronts; a transposed butterfly reduces each
//    wavefront's row sums across lanes and the workgroup adds the wavefronts'
//    sums through LDS in a fixed order, so y is written once, by one kernel.
//  * B = 2..16: decoded BF16 rows go to LDS and feed
//    v_mfma_f32_16x16x32_bf16 (A = 16 weight rows x 32 columns, B = the batch
//    rows of X padded to 16); the same workgroup split and LDS reduction.
//  * Shapes or geometries outside the fast path use one-symbol-at-a-time
//    kernels with an FP32 partial-sum workspace and a separate reduction.
//  * Every global read from the blob is clamped to its sections.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <tuple>

#include "nwc_internal.hpp"

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;      // wavefronts per workgroup, fused kernels
constexpr int kGenericWaves = 4;   // wavefronts per workgroup, generic kernels
constexpr int kTable = 4096;
constexpr uint32_t kExpMask = 0x7F807F80u;  // exponent bits of two packed BF16

struct BlobDev {
  const uint32_t* table;
  const uint32_t* tile_words;
  const uint16_t* chunk_bits;
  const uint8_t* raw;
  const uint32_t* stream;
  uint64_t rows, cols, raw_ld;
  uint64_t n_tiles, n_tr;
  uint32_t n_tc, tr, tc, s, v;
  uint32_t stream_words;  // words of codes; 4 zero guard words follow in the blob
  uint32_t buf_words;     // LDS stream buffer per wavefront
};

// How a fused launch splits the matrix: a work item is `rb` row blocks; its
// workgroup has rb * nw wavefronts and wavefront (i, j) takes column tiles
// j, j + nw, ... of row block i.
struct Split {
  uint32_t nw, rb, waves;
  uint64_t items;
};

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }
// Wave-uniform read through the constant address space (a scalar load).
__device__ __forceinline__ uint32_t sload(const uint32_t* p, uint64_t i) {
  typedef const __attribute__((address_space(4))) uint32_t cu32;
  return ((cu32*)(reinterpret_cast<uintptr_t>(p)))[i];
}
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// DPP move of v from a lane chosen by CTRL (0 where the source lane is
// outside the row or the row is masked off).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, true));
}
constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143, kRowMirror = 0x140,
              kRowHalfMirror = 0x141;

// Exclusive prefix sum of v across the 64 lanes (DPP: shifts within rows of
// 16 lanes, then row broadcasts).
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v) {
  uint32_t s = v;
  s += dpp<kRowShr + 1>(s);
  s += dpp<kRowShr + 2>(s);
  s += dpp<kRowShr + 4>(s);
  s += dpp<kRowShr + 8>(s);
  s += dpp<kRowBcast15, 0xA>(s);
  s += dpp<kRowBcast31, 0xC>(s);
  return s - v;
}

// Value of v in a partner lane whose lane index differs in bit M (M = 1..32),
// for the butterflies below: quad permutes, half-row and row mirrors, a
// 32-lane swizzle and, for bit 5, a lane permute through the LDS crossbar.
template <int M>
__device__ __forceinline__ float partner(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint32_t r;
  if constexpr (M == 1) r = dpp<0xB1>(u);                 // quad_perm [1,0,3,2]
  else if constexpr (M == 2) r = dpp<0x4E>(u);            // quad_perm [2,3,0,1]
  else if constexpr (M == 4) r = dpp<kRowHalfMirror>(u);  // lane i <-> 7 - i within 8
  else if constexpr (M == 8) r = dpp<kRowMirror>(u);      // lane i <-> 15 - i within 16
  else if constexpr (M == 16) r = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(u), 0x401F));
  else r = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(static_cast<int>((lane_id() ^ 32u) << 2),
                                                             static_cast<int>(u)));
  return __builtin_bit_cast(float, r);
}

// Wait for every outstanding vector-memory load (including loads into LDS).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// all but the last N vector-memory operations of this wavefront are complete
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copy the decode table into LDS with 16-byte loads straight to LDS; the
// caller synchronizes the workgroup.
__device__ __forceinline__ void load_table(uint32_t* lds_table, const uint32_t* table) {
  const uint32_t nthreads = blockDim.x;
  const uint32_t wave = uniform(threadIdx.x / kWave);
  for (uint32_t base = wave * kWave * 4; base < kTable; base += nthreads * 4) {
    __builtin_amdgcn_global_load_lds(table + base + lane_id() * 4, lds_table + base, 16, 0, 0);
  }
  wait_vmem();
}

// Issue the loads that bring stream words [a0, a0 + n) of a tile into this
// wavefront's LDS buffer (a0 = the tile's first word rounded down to 4 words,
// n a multiple of 4), 16 bytes per lane.  Sources past the stream's guard
// words are redirected to its start; those LDS words are never read for a
// well-formed blob.
__device__ __forceinline__ void stage_stream(const BlobDev& b, uint32_t a0, uint32_t n, uint32_t* buf) {
  const uint32_t lane = lane_id();
  if (lane < 4) buf[lane] = 0u;  // guard words before the stream
  buf += 4;
  for (uint32_t j = 0; j < n; j += 4 * kWave) {
    const uint32_t o = j + 4 * lane;
    uint32_t g = a0 + o;
    g = g + 4 <= b.stream_words + 4 ? g : 0u;
    if (o < n) __builtin_amdgcn_global_load_lds(b.stream + g, buf + j, 16, 0, 0);
  }
}

// Words to stage for a tile [w0, w1): through the bit reader's two words of
// look-ahead, in whole 16-byte pieces, capped by the buffer.
__device__ __forceinline__ uint32_t stage_blocks(const BlobDev& b, uint32_t a0, uint32_t w1) {
  const uint32_t need = (w1 - a0 + 2 + 3) & ~3u;
  const uint32_t cap = b.buf_words - 8;
  return need > cap ? cap : need;
}

// LDS access by byte address (a 32-bit offset into the workgroup's LDS).
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u32*)p));
}
__device__ __forceinline__ uint32_t lds_word(uint32_t byte_addr) {
  return *(lds_u32*)(static_cast<uintptr_t>(byte_addr));
}
typedef __attribute__((address_space(3))) uint32_t lds_u32w;
__device__ __forceinline__ void lds_put(uint32_t byte_addr, uint32_t v) {
  *(lds_u32w*)(static_cast<uintptr_t>(byte_addr)) = v;
}
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u128;
__device__ __forceinline__ void lds_put4(uint32_t byte_addr, uint4 v) {
  *(lds_u128*)(static_cast<uintptr_t>(byte_addr)) = __builtin_bit_cast(u32x4_t, v);
}
__device__ __forceinline__ uint4 lds_get4(uint32_t byte_addr) {
  return __builtin_bit_cast(uint4, *(const lds_u128*)(static_cast<uintptr_t>(byte_addr)));
}

// Raw buffer resource over [base, base + bytes) (bytes capped at 4 GiB - 1):
// loads past the end return zero instead of faulting.  Built from
// wave-uniform values, so it lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(n),
                                           0x00020000);
}

// Bit reader over a wavefront's LDS stream buffer.  The buffer keeps 4 zero
// guard words before the staged stream, so every start bit b >= 128.  The
// whole state is p = (LDS bit address of the next code) - 2: a step reads the
// word holding bit p and the next one (one ds_read2), and a funnel shift by
// p (mod 32) leaves the next 12 stream bits at bits 2..13, already a byte
// address into the 4-byte-entry decode table.  Six VALU operations per step
// besides the table lookup; the stream words are re-read from LDS instead of
// being shifted through registers.
struct Bits {
  uint32_t p;
  __device__ __forceinline__ void init(const uint32_t* buf, uint32_t bit) { p = lds_addr(buf) * 8u + bit - 2u; }
  __device__ __forceinline__ uint32_t window() const {
    const uint32_t a = (p >> 3) & ~3u;
    return __builtin_amdgcn_alignbit(lds_word(a + 4), lds_word(a), p);
  }
  __device__ __forceinline__ void advance(uint32_t n) { p += n; }
  __device__ __forceinline__ uint32_t pair(const uint32_t* tab);
  // One exponent (generic paths): returns it and advances.
  __device__ __forceinline__ uint32_t one(const uint32_t* tab) {
    const uint32_t ent = tab[(window() & 0x3FFCu) >> 2];
    p += (ent >> 16) & 0xFu;
    return (ent >> 7) & 0xFFu;
  }
};

// Bit reader over a lane-interleaved LDS stream buffer: word j of this lane's
// staged words is LDS word 64 j + lane of the slot, so at every step the 64
// lanes read 64 different banks.  q = (bit position in the staged words) - 2.
// The slot starts on a 256-byte boundary, so q carries the slot's base (as
// 32 * base / 256 added to the bit position): the word address is then
// ((q >> 5) << 8) | (4 * lane), one shift and one and-or.
struct LaneBits {
  uint32_t lane4, q;
  __device__ __forceinline__ void init(const uint32_t* slot, uint32_t q0) {
    lane4 = lane_id() * 4u;
    q = q0 + (lds_addr(slot) >> 3);
  }
  __device__ __forceinline__ uint32_t window() const {
    const uint32_t a = ((q << 3) & ~0xFFu) | lane4;
    return __builtin_amdgcn_alignbit(lds_word(a + 256), lds_word(a), q);
  }
  __device__ __forceinline__ void advance(uint32_t n) { q += n; }
};

// Decode the next two exponents with either reader: returns a dword with
// exponent 0 at bits 7..14 and exponent 1 at bits 23..30.  FIT2: the code is
// limited to 6 bits, so two codes always fit the 12-bit window and the
// second lookup never happens.
template <bool FIT2 = false, class R>
__device__ __forceinline__ uint32_t decode_pair(R& rd, const uint32_t* tab) {
  const uint32_t win = rd.window();
  uint32_t ent = tab[(win & 0x3FFCu) >> 2];
  if constexpr (FIT2) {
    rd.advance(ent & 0x1Fu);
    return ent;
  }
  // Rarely the second code does not fit in the 12-bit window.  The test is
  // made for the whole wavefront, and inside the branch every lane does the
  // second lookup and keeps it only if it needs it, so the common path has no
  // exec-mask changes.  The window holds 30 bits past the first code's start,
  // so the second code (<= 12 bits after <= 12) is inside it.
  const bool single = static_cast<int32_t>(ent) < 0;
  if (__builtin_amdgcn_ballot_w64(single)) {
    const uint32_t l0 = ent & 0xFu;
    const uint32_t ent2 = tab[((win >> l0) & 0x3FFCu) >> 2];
    // merged advance l0 + l1 may reach 24: it occupies bits 0..4
    const uint32_t merged = (ent & 0x7F80u) | ((ent2 & 0x7F80u) << 16) | (l0 + ((ent2 >> 16) & 0xFu));
    ent = single ? merged : ent;
  }
  rd.advance(ent & 0x1Fu);
  return ent;
}
__device__ __forceinline__ uint32_t Bits::pair(const uint32_t* tab) { return decode_pair(*this, tab); }

// Two BF16 weights from a pair entry and 4 raw bytes; `hi` selects raw bytes
// 2,3 instead of 0,1.
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

__device__ __forceinline__ void store_y(void* y, uint64_t i, float v, int y_f32) {
  if (y_f32)
    static_cast<float*>(y)[i] = v;
  else
    static_cast<uint16_t*>(y)[i] = f32_to_bf16_rne(v);
}

// One level of the transposed butterfly: lanes with bit M set keep the upper
// half of their sums and receive the partner's upper half; the others keep
// the lower half.  Indices are compile-time, so no dynamic register indexing.
// Partners differ in bit M and hold sums over disjoint lane sets, so after
// all levels every row's sum covers all 64 lanes exactly once.
// For M = 32 and M = 16 one lane-swap instruction moves exactly the two
// halves that change hands (v[i] from the upper lanes down, v[HALF + i] from
// the lower lanes up), so a level costs a swap and an add; the sums are the
// same two operands as the select form (addition commutes).
template <int R, int HALF, int M>
__device__ __forceinline__ void butterfly(float (&v)[R], uint32_t lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < HALF; i++) {
    if constexpr (M == 32 || M == 16) {
      const uint32_t lo = __builtin_bit_cast(uint32_t, v[i]), hi = __builtin_bit_cast(uint32_t, v[HALF + i]);
      const auto p = M == 32 ? __builtin_amdgcn_permlane32_swap(lo, hi, false, false)
                             : __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
      v[i] = __builtin_bit_cast(float, static_cast<uint32_t>(p[0])) +
             __builtin_bit_cast(float, static_cast<uint32_t>(p[1]));
    } else {
      const float keep = up ? v[HALF + i] : v[i];
      const float send = up ? v[i] : v[HALF + i];
      v[i] = keep + partner<M>(send);
    }
  }
  if constexpr (HALF > 1) butterfly<R, HALF / 2, M / 2>(v, lane);
}

template <int M>
__device__ __forceinline__ float allsum_low(float s) {
  if constexpr (M >= 1) {
    s += partner<M>(s);
    return allsum_low<M / 2>(s);
  }
  return s;
}

// Transposed butterfly: on entry every lane holds R partial sums (rows
// 0..R-1); on exit lane l holds the full sum of row (l / (64/R)) % R (every
// lane of a row's group holds it), added in a fixed order.
template <int R>
__device__ __forceinline__ float reduce_rows(float (&v)[R]) {
  butterfly<R, R / 2, 32>(v, lane_id());
  return allsum_low<32 / R>(v[0]);
}

// Everything one lane needs from global memory for one tile, loaded up front.
template <int TR>
struct TileIn {
  uint2 raw[TR];
  uint32_t cb, a0, w0;
  uint64_t c0;
  uint32_t nrows;
  bool active;

  __device__ __forceinline__ void load(const BlobDev& b, uint64_t ti, uint32_t tj, uint32_t* buf) {
    const uint32_t lane = lane_id();
    const uint64_t t = ti * b.n_tc + tj;
    const uint64_t row0 = ti * TR;
    nrows = static_cast<uint32_t>(umin64(TR, b.rows - row0));
    c0 = static_cast<uint64_t>(tj) * 512 + lane * 8;
    active = c0 < b.cols;
    const uint64_t cc = active ? c0 : 0;
    w0 = sload(b.tile_words, t);
    const uint32_t w1 = sload(b.tile_words, t + 1);
    a0 = w0 & ~3u;
    stage_stream(b, a0, stage_blocks(b, a0, w1 < w0 ? w0 : w1), buf);
    cb = b.chunk_bits[t * 64 + lane];
#pragma unroll
    for (int r = 0; r < TR; r++) {
      const uint64_t row = row0 + (static_cast<uint32_t>(r) < nrows ? r : nrows - 1);
      raw[r] = *reinterpret_cast<const uint2*>(b.raw + row * b.raw_ld + cc);
    }
  }
  // start bit of this lane's chunk inside the LDS buffer (after the 4 guard words)
  __device__ __forceinline__ uint32_t start_bit() const { return 128 + (w0 - a0) * 32 + wave_excl_scan(cb); }
};

// ------------------------------------------------------------------ decode

// Generic path: any geometry, two codes per table lookup, scalar stores.
__global__ __launch_bounds__(kGenericWaves * kWave) void k_decode_generic(BlobDev b, uint16_t* __restrict__ out,
                                                                          uint64_t ld) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ __attribute__((aligned(16))) uint32_t tab[kTable];  // static: LDS address 0
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds + wave * b.buf_words;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint64_t nwaves = static_cast<uint64_t>(gridDim.x) * (blockDim.x / kWave);
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * (blockDim.x / kWave) + wave; t < b.n_tiles; t += nwaves) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * b.tr;
    const uint64_t r1 = umin64(b.rows, row0 + b.tr);
    const uint64_t tile_c1 = umin64(b.cols, tj * b.tc + b.tc);
    const uint32_t w0 = sload(b.tile_words, t);
    const uint32_t w1 = sload(b.tile_words, t + 1);
    const uint32_t a0 = w0 & ~3u;
    stage_stream(b, a0, stage_blocks(b, a0, w1 < w0 ? w0 : w1), buf);
    wait_vmem();
    wave_sync_lds();
    uint32_t base = 128 + (w0 - a0) * 32;  // start bit of the first chunk of this round
    for (uint32_t c0i = 0; c0i < b.s; c0i += kWave) {
      const uint32_t c = c0i + lane;
      const uint32_t cb = c < b.s ? b.chunk_bits[t * b.s + c] : 0u;
      const uint32_t excl = wave_excl_scan(cb);
      const uint32_t bit = base + excl;
      base += __builtin_amdgcn_readlane(excl + cb, kWave - 1);
      if (c < b.s) {
        const uint64_t cc0 = tj * b.tc + static_cast<uint64_t>(c) * b.v;
        if (cc0 < tile_c1) {
          const uint64_t cc1 = umin64(tile_c1, cc0 + b.v);
          Bits br;
          br.init(buf, bit);
          // the chunk's symbols in row order, two codes per table lookup
          const uint32_t wdt = static_cast<uint32_t>(cc1 - cc0);
          const uint32_t nsym = static_cast<uint32_t>(r1 - row0) * wdt;
          auto put = [&](uint32_t idx, uint32_t e) __attribute__((always_inline)) {
            const uint64_t r = row0 + idx / wdt, k = cc0 + idx % wdt;
            const uint32_t rb = b.raw[r * b.raw_ld + k];
            out[r * ld + k] = static_cast<uint16_t>(((rb & 0x80u) << 8) | (e << 7) | (rb & 0x7Fu));
          };
          uint32_t idx = 0;
          for (; idx + 1 < nsym; idx += 2) {
            const uint32_t ent = br.pair(tab);
            put(idx, (ent >> 7) & 0xFFu);
            put(idx + 1, (ent >> 23) & 0xFFu);
          }
          if (idx < nsym) put(idx, br.one(tab));
        }
      }
    }
    wave_sync_lds();
  }
}

// Rows of W by index (an embedding lookup from the compressed table of a tied
// LM head): work item (i, tj) decodes column tile tj of the row block that
// holds row ids[i], each chunk up to that row (the rows of a chunk follow
// one another in its code stream), two codes per table lookup, and writes that
// row's columns of the tile to out row i.  Any geometry.  An id past the
// matrix gives a row of zeros.
__global__ __launch_bounds__(kGenericWaves * kWave) void k_gather(BlobDev b, const uint32_t* __restrict__ ids,
                                                                  uint32_t n_ids, uint16_t* __restrict__ out,
                                                                  uint64_t ld) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ __attribute__((aligned(16))) uint32_t tab[kTable];  // static: LDS address 0
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds + wave * b.buf_words;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint64_t nwaves = static_cast<uint64_t>(gridDim.x) * (blockDim.x / kWave);
  const uint64_t items = static_cast<uint64_t>(n_ids) * b.n_tc;
  for (uint64_t it = static_cast<uint64_t>(blockIdx.x) * (blockDim.x / kWave) + wave; it < items; it += nwaves) {
    const uint64_t i = it / b.n_tc, tj = it % b.n_tc;
    const uint64_t id = uniform(ids[i]);
    const uint64_t tile_c0 = tj * b.tc, tile_c1 = umin64(b.cols, tile_c0 + b.tc);
    uint16_t* orow = out + i * ld;
    if (id >= b.rows) {
      for (uint64_t k = tile_c0 + lane; k < tile_c1; k += kWave) orow[k] = 0;
      continue;
    }
    const uint64_t ti = id / b.tr;
    const uint64_t t = ti * b.n_tc + tj;
    const uint64_t row0 = ti * b.tr;
    const uint32_t w0 = sload(b.tile_words, t);
    const uint32_t w1 = sload(b.tile_words, t + 1);
    const uint32_t a0 = w0 & ~3u;
    stage_stream(b, a0, stage_blocks(b, a0, w1 < w0 ? w0 : w1), buf);
    wait_vmem();
    wave_sync_lds();
    uint32_t base = 128 + (w0 - a0) * 32;  // start bit of the first chunk of this round
    for (uint32_t c0i = 0; c0i < b.s; c0i += kWave) {
      const uint32_t c = c0i + lane;
      const uint32_t cb = c < b.s ? b.chunk_bits[t * b.s + c] : 0u;
      const uint32_t excl = wave_excl_scan(cb);
      const uint32_t bit = base + excl;
      base += __builtin_amdgcn_readlane(excl + cb, kWave - 1);
      if (c < b.s) {
        const uint64_t cc0 = tile_c0 + static_cast<uint64_t>(c) * b.v;
        if (cc0 < tile_c1) {
          const uint64_t cc1 = umin64(tile_c1, cc0 + b.v);
          Bits br;
          br.init(buf, bit);
          // the rows before it, two codes per table lookup
          uint64_t skip = (id - row0) * (cc1 - cc0);
          for (; skip >= 2; skip -= 2) br.pair(tab);
          if (skip) br.one(tab);
          const uint8_t* rr = b.raw + id * b.raw_ld;
          auto put = [&](uint64_t k, uint32_t e) __attribute__((always_inline)) {
            const uint32_t rb = rr[k];
            orow[k] = static_cast<uint16_t>(((rb & 0x80u) << 8) | (e << 7) | (rb & 0x7Fu));
          };
          uint64_t k = cc0;
          for (; k + 1 < cc1; k += 2) {
            const uint32_t ent = br.pair(tab);
            put(k, (ent >> 7) & 0xFFu);
            put(k + 1, (ent >> 23) & 0xFFu);
          }
          if (k < cc1) put(k, br.one(tab));
        }
      }
    }
    wave_sync_lds();
  }
}

// -------------------------------------------------------------------- GEMV

// One matrix of a fused batch-1 launch.  Its tiles, numbered row block by row
// block (t = i * n_tc + j), are cut into `groups` contiguous ranges, one per
// workgroup: whole row blocks (whole_rows), or equal ranges (sizes differ by
// at most one) that may cut a row block.  A row block inside a range is
// summed in LDS; a cut one is finished through `slots` (one 64-bit slot per
// tile and row, all zero between launches) by the chain described at the end
// of the kernel.
struct GemvJob {
  BlobDev b;
  const uint16_t* x;
  void* y;
  uint64_t* slots;      // [n_tiles][TR]: link i of row block rb's chain at tile rb * n_tc + i
  uint32_t g0;          // first workgroup of this matrix
  uint32_t groups;      // workgroups of this matrix
  uint32_t whole_rows;  // 1: each range is whole row blocks; 0: equal ranges
  uint64_t ld;          // decode mode: row stride of W' in elements
};
// a chain slot holds a partial sum's FP32 bits with this flag set
constexpr uint64_t kSlotFull = 1ull << 32;
constexpr int kMaxJobs = 8;
constexpr uint32_t kGroupLds = 8192;       // least per-workgroup LDS for control words, offsets, tile sums
constexpr uint32_t kSkinnyLds = 24576;     // per-workgroup LDS for the skinny mode's tile sums
struct GemvGroup {
  GemvJob job[kMaxJobs];
  uint32_t count;
  int y_f32;
  uint32_t lane_words;  // stream words per lane in the interleaved slot (J, even)
  uint32_t buf_words;   // linear staging buffer per wavefront
  uint32_t tw_words;    // LDS words for a range's tile offsets (>= tiles + 1)
  // skinny mode (one matrix): X rows of ldx elements, Y rows of ldy entries
  uint64_t ldx, ldy;
  uint32_t batch;
};

// Registers of one tile for the batch-1 kernel: raw bytes of this lane's
// 8 columns in every row, x for those columns, this lane's chunk length, and
// where the tile's stream starts.  Every load goes through a buffer resource
// built from wave-uniform addresses (row offsets in scalar registers, one
// constant lane offset), so issuing a tile costs almost no vector ALU work.
// The tile's word offsets (tw0, tw1) come in from a vector load issued one
// tile earlier: a scalar load would share its wait counter with the LDS
// reads of the decode loop and stall it for a full memory round trip.
template <int TR, int NX>
struct TileRegs {
  uint2 raw[TR];
  uint4 x[NX > 0 ? NX : 1];  // X rows 0 .. NX - 1 at this lane's 8 columns
  // cbw: the dword holding this lane's chunk length (lanes 2k and 2k + 1
  // share one); the half is picked where it is used, so no instruction
  // touches the loaded value before the tile is waited for
  uint32_t cbw, w0, a0, nrows;
  uint32_t col;     // column tile
  uint32_t rowblk;  // row block
  bool active;
  __device__ __forceinline__ uint32_t cb() const { return __builtin_amdgcn_ubfe(cbw, (lane_id() & 1) * 16, 16); }
  // A tile's loads come in two groups: what the first half of its rows needs
  // (load_stream, load_planes) and the raw bytes of the second half
  // (load_rest), issued last so that decoding can start before they land.
  // The stream goes first: its number of pieces varies, and with a fixed
  // number of loads behind it every wait on this tile has a known count.
  __device__ __forceinline__ void load(const BlobDev& b, const uint16_t* xp, uint64_t ldx, uint32_t nxr, uint64_t ti,
                                       uint32_t tj, uint32_t tw0, uint32_t tw1, uint32_t* buf) {
    load_stream(b, tw0, tw1, buf);
    load_planes(b, xp, ldx, nxr, ti, tj);
  }
  // chunk lengths, x (X rows below nxr; the others zero) and the raw bytes
  // of rows [0, TR / 2): no dependence on the tile's word offsets
  __device__ __forceinline__ void load_planes(const BlobDev& b, const uint16_t* xp, uint64_t ldx, uint32_t nxr,
                                              uint64_t ti, uint32_t tj) {
    const uint32_t lane = lane_id();
    const uint64_t t = ti * b.n_tc + tj;
    const uint64_t row0 = ti * TR;
    nrows = static_cast<uint32_t>(umin64(TR, b.rows - row0));
    active = static_cast<uint64_t>(tj) * 512 + lane * 8 < b.cols;
    col = tj;
    rowblk = static_cast<uint32_t>(ti);
    const uint64_t col0 = static_cast<uint64_t>(tj) * 512;
    cbw = __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(b.chunk_bits + t * 64, 128), (lane & ~1u) * 2, 0, 0);
#pragma unroll
    for (int k = 0; k < NX; k++) {
      x[k] = make_uint4(0, 0, 0, 0);
      if (k == 0 || static_cast<uint32_t>(k) < nxr)
        x[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             buf_rsrc(xp + k * ldx + col0, (b.cols - col0) * 2), lane * 16, 0, 0));
    }
    load_raw<0, TR / 2>(b, ti, tj);
  }
  __device__ __forceinline__ void load_rest(const BlobDev& b, uint64_t ti, uint32_t tj) {
    load_raw<TR / 2, TR>(b, ti, tj);
  }
  // raw plane rows [R0, R1) of the tile: rows past the matrix edge re-read
  // the last valid row
  template <int R0, int R1>
  __device__ __forceinline__ void load_raw(const BlobDev& b, uint64_t ti, uint32_t tj) {
    const uint32_t lane = lane_id();
    const uint64_t row0 = ti * TR;
    const uint64_t col0 = static_cast<uint64_t>(tj) * 512;
    const __amdgpu_buffer_rsrc_t rr =
        buf_rsrc(b.raw + row0 * b.raw_ld + col0, (b.rows - row0) * b.raw_ld - col0);
#pragma unroll
    for (int r = R0; r < R1; r++) {
      const uint32_t rr_off = static_cast<uint32_t>((static_cast<uint32_t>(r) < nrows ? r : nrows - 1) * b.raw_ld);
      raw[r] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rr, lane * 8, rr_off, 0));
    }
  }
  // the tile's stream words [w0 & ~3, w1 + 2) in 16-byte pieces, behind 4 zero
  // guard words
  __device__ __forceinline__ void load_stream(const BlobDev& b, uint32_t tw0, uint32_t tw1, uint32_t* buf) {
    const uint32_t lane = lane_id();
    w0 = tw0;
    const uint32_t w1 = tw1;
    a0 = w0 & ~3u;
    const uint32_t n = stage_blocks(b, a0, w1 < w0 ? w0 : w1);
    if (lane < 4) buf[lane] = 0u;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(b.stream + a0, (static_cast<uint64_t>(b.stream_words) + 4 - a0) * 4);
    for (uint32_t j = 0; j < n; j += 4 * kWave)
      if (j + 4 * lane < n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(buf + 4 + j), 16,
                                                 lane * 16, j * 4, 0, 0);
  }
};

// Copy this lane's words of the linearly staged stream into the lane-
// interleaved slot (word j of lane l at slot word 64 j + l, so the decode
// steps of the 64 lanes always hit 64 different banks).  A lane takes J
// words starting with the one that holds bit (chunk start - 2); returns the
// reader's start position within them.
__device__ __forceinline__ uint32_t interleave(const uint32_t* buf, uint32_t w0, uint32_t a0, uint32_t cb,
                                               uint32_t J, uint32_t* slot) {
  const uint32_t sb = 128u + (w0 - a0) * 32u + wave_excl_scan(cb) - 2u;
  const uint32_t src = lds_addr(buf) + (sb >> 5) * 4u;
  const uint32_t dst = lds_addr(slot) + lane_id() * 4u;
  // four words read before any is written (the compiler cannot reorder LDS
  // reads and writes through computed addresses itself); J is even
  for (uint32_t j = 0; j < J; j += 4) {
    const bool two = j + 2 < J;
    const uint32_t w0 = lds_word(src + 4 * j), w1 = lds_word(src + 4 * j + 4);
    uint32_t w2 = 0, w3 = 0;
    if (two) {
      w2 = lds_word(src + 4 * j + 8);
      w3 = lds_word(src + 4 * j + 12);
    }
    lds_put(dst + 256 * j, w0);
    lds_put(dst + 256 * j + 256, w1);
    if (two) {
      lds_put(dst + 256 * j + 512, w2);
      lds_put(dst + 256 * j + 768, w3);
    }
  }
  return sb & 31u;
}

// Decode rows [R0, R1) of a staged tile (stream in the lane-interleaved
// slot, raw bytes and x in registers) into this lane's row sums over its 8
// columns.  Rows past the matrix edge (last row block only; a wave-uniform
// test) are not decoded and keep their zero sums.
template <int TR, int NX, int R0, int R1, bool FIT2 = false>
__device__ __forceinline__ void gemv_rows(const TileRegs<TR, NX>& in, LaneBits& br, const uint32_t* tab,
                                          float (&acc)[TR * NX]) {
#pragma unroll
  for (int r = R0; r < R1; r++) {
    if (static_cast<uint32_t>(r) < in.nrows) {
      float a[NX];
#pragma unroll
      for (int k = 0; k < NX; k++) a[k] = 0.0f;
      // each product is pinned next to its decode step: left alone, the
      // compiler defers all of them to the end of the tile and keeps every
      // decoded pair live, which costs occupancy
      const uint32_t p0 = assemble(decode_pair<FIT2>(br, tab), in.raw[r].x, false);
#pragma unroll
      for (int k = 0; k < NX; k++) {
        a[k] = dot2(p0, in.x[k].x, a[k]);
        asm volatile("" : "+v"(a[k]));
      }
      const uint32_t p1 = assemble(decode_pair<FIT2>(br, tab), in.raw[r].x, true);
#pragma unroll
      for (int k = 0; k < NX; k++) {
        a[k] = dot2(p1, in.x[k].y, a[k]);
        asm volatile("" : "+v"(a[k]));
      }
      const uint32_t p2 = assemble(decode_pair<FIT2>(br, tab), in.raw[r].y, false);
#pragma unroll
      for (int k = 0; k < NX; k++) {
        a[k] = dot2(p2, in.x[k].z, a[k]);
        asm volatile("" : "+v"(a[k]));
      }
      const uint32_t p3 = assemble(decode_pair<FIT2>(br, tab), in.raw[r].y, true);
#pragma unroll
      for (int k = 0; k < NX; k++) {
        a[k] = dot2(p3, in.x[k].w, a[k]);
        asm volatile("" : "+v"(a[k]));
      }
#pragma unroll
      for (int k = 0; k < NX; k++) acc[r * NX + k] = a[k];
    }
  }
}

// Skinny mode: rows [R0, R1) of the tile decoded into registers, four BF16
// pairs per row (rows past the matrix edge stay zero).
template <int TR, int NX, int R0, int R1, bool FIT2 = false>
__device__ __forceinline__ void decode_rows(const TileRegs<TR, NX>& in, LaneBits& br, const uint32_t* tab,
                                            uint32_t (&wv)[TR][4]) {
#pragma unroll
  for (int r = R0; r < R1; r++) {
    if (static_cast<uint32_t>(r) < in.nrows) {
      wv[r][0] = assemble(decode_pair<FIT2>(br, tab), in.raw[r].x, false);
      wv[r][1] = assemble(decode_pair<FIT2>(br, tab), in.raw[r].x, true);
      wv[r][2] = assemble(decode_pair<FIT2>(br, tab), in.raw[r].y, false);
      wv[r][3] = assemble(decode_pair<FIT2>(br, tab), in.raw[r].y, true);
    }
  }
}

// Skinny mode: this lane's 8 columns of X rows [g GB, g GB + GB) for column
// tile tj (zero past the matrix edge and past the batch).
template <int GB>
__device__ __forceinline__ void load_xg(const BlobDev& b, const uint16_t* X, uint64_t ldx, uint32_t batch, uint32_t g,
                                        uint32_t tj, uint4 (&xg)[GB]) {
  const uint64_t col0 = static_cast<uint64_t>(tj) * 512;
#pragma unroll
  for (int k = 0; k < GB; k++) {
    const uint32_t beta = g * GB + k;
    xg[k] = make_uint4(0, 0, 0, 0);
    if (beta < batch)
      xg[k] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(X + beta * ldx + col0, (b.cols - col0) * 2),
                                                       lane_id() * 16, 0, 0));
  }
}

// Partial sums handed between workgroups travel inside agent-scope atomic
// exchanges.  On this chip each XCD has its own L2, and an agent-scope fence
// writes back or invalidates a whole L2, far too slow to do per workgroup;
// an agent-scope atomic is performed at the level all XCDs share, and a
// value carried by the atomic itself needs no fence at all.

// the range that holds tile t, for ranges [w T / W, (w + 1) T / W)
__device__ __forceinline__ uint64_t range_of(uint64_t t, uint64_t T, uint64_t W) { return ((t + 1) * W - 1) / T; }

// Fused decode-GEMV, batch 1, for up to kMaxJobs matrices: y_j = W_j x_j.
// LDS: static decode table | per wavefront: linear staging buffer
// (buf_words) | lane-interleaved slot (64 J words) | per workgroup: control
// words | word offsets of the range's tiles | the range's tile sums
// [tiles][TR].
// Each workgroup owns a contiguous range of a matrix's tiles (whole row
// blocks when that keeps the ranges even).  Its wavefronts start on the
// range's first tiles, then claim the rest one at a time from an LDS
// counter 7/8 of the way through their current tile, so a tile goes to
// whichever wavefront is furthest along.  While tile t decodes from the slot, the next
// tile's stream lands in the linear buffer.  Every tile sum goes to LDS;
// after one barrier the workgroup adds each row's sums in column order.  A
// row block cut by a range edge has its tile sums added through the
// workspace by whichever workgroup finishes it last.
// NB: 1 for y = W x; 2 or 4 for Y = X W^T with up to NB X rows (TR NB <= 32),
// their products formed as each pair is decoded; 0 for any batch 2..16, the tile
// decoded into registers first and then multiplied by the X rows 32 / TR at
// a time (NB 0, 2, 4: the skinny mode, one matrix, ranges of whole row
// blocks); -1 for the standalone decode, which writes each decoded tile to
// W' (job.y, rows of g.ldy elements) once the next tile's data is in; 16
// for Y = X W^T with up to 16 X rows on the matrix cores (8-row tiles: the
// decoded tile goes through LDS into MFMA operand layout).
template <int TR, int MAXW, int NB, bool FIT2 = false>
__global__ __launch_bounds__(MAXW * kWave) void k_gemv(const GemvGroup g) {
  constexpr bool DECODE = NB < 0;
  constexpr bool MF = NB == 16;
  constexpr bool SKINNY = NB == 0 || NB > 1;
  constexpr int NX = NB > 0 && !MF ? NB : 0;  // X rows that come with each tile
  constexpr int NA = NB > 0 && !MF ? NB : 1;  // sums per row of a tile formed while decoding
  static_assert(!MF || TR == 8, "the matrix-core mode takes 8-row tiles");
  __shared__ __attribute__((aligned(16))) uint32_t tab[kTable];  // static: LDS address 0
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const uint32_t nw = blockDim.x / kWave;
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t lane = lane_id();
  int j = 0;
  while (j + 1 < static_cast<int>(g.count) && blockIdx.x >= g.job[j + 1].g0) j++;
  // select the job with compile-time indices (no dynamic indexing of the
  // kernel-argument struct, which would copy it to scratch)
  GemvJob job = g.job[0];
#pragma unroll
  for (int jj = 1; jj < kMaxJobs; jj++)
    if (jj == j) job = g.job[jj];
  const BlobDev& b = job.b;
  const uint32_t J = g.lane_words;
  uint32_t* buf = lds + wave * (g.buf_words + kWave * J);
  uint32_t* slot = buf + g.buf_words;
  // [0] next tile of the range, [1] cut row blocks this workgroup completes
  // (bit 0 the first, bit 1 the last)
  uint32_t* ctl = lds + nw * (g.buf_words + kWave * J);
  uint32_t* tw = ctl + 4;  // tile_words[r0 .. r1]
  float* gsum = reinterpret_cast<float*>(tw + g.tw_words);
  const uint32_t n_tc = b.n_tc;
  const uint64_t T = b.n_tiles;
  // this workgroup's tiles [r0, r1)
  const uint64_t G = job.groups, gi = blockIdx.x - job.g0;
  uint64_t r0, r1;
  if (job.whole_rows) {
    r0 = gi * b.n_tr / G * n_tc;
    r1 = (gi + 1) * b.n_tr / G * n_tc;
  } else {
    r0 = gi * T / G;
    r1 = (gi + 1) * T / G;
  }
  const uint32_t n_r = static_cast<uint32_t>(r1 - r0);

  // the next tile of the range (claimed by lane 0, given to the wavefront)
  auto claim = [&]() __attribute__((always_inline)) {
    uint32_t v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return r0 + __builtin_amdgcn_readfirstlane(v);
  };
  // Wavefronts 1.. take the range's first tiles in order and ask for them at
  // once.  Wavefront 0 sets the counter past those, loads the decode table
  // and the range's word offsets, and waits for them alone; the barrier then
  // publishes all three, and wavefront 0 claims its first tile after it.
  // (when the first tiles cover the whole range, nothing is claimed)
  const bool claims = n_r > nw - 1;
  TileRegs<TR, NX> in;
  uint64_t t = r1;
  if (wave == 0) {
    if (lane == 0) {
      ctl[0] = nw - 1;
      ctl[1] = 0u;
    }
    for (uint32_t base = 0; base < kTable; base += kWave * 4)
      __builtin_amdgcn_global_load_lds(b.table + base + lane * 4, tab + base, 16, 0, 0);
    if (claims)
      for (uint32_t i = lane; i <= n_r; i += kWave) tw[i] = b.tile_words[r0 + i];
    wait_vmem();
  } else if (wave - 1 < n_r) {
    // the first tile's word offsets come by scalar loads (no LDS reads are
    // in flight yet)
    t = r0 + wave - 1;
    const uint64_t ti = t / n_tc;
    const uint32_t tj = static_cast<uint32_t>(t - ti * n_tc);
    const uint32_t w0 = sload(b.tile_words, t), w1 = sload(b.tile_words, t + 1);
    in.load(b, job.x, g.ldx, g.batch, ti, tj, w0, w1, buf);
    asm volatile("" ::: "memory");
    in.load_rest(b, ti, tj);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's LDS writes are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (wave == 0 && claims) {
    t = claim();
    if (t < r1) {
      const uint64_t ti = t / n_tc;
      const uint32_t tj = static_cast<uint32_t>(t - ti * n_tc);
      const uint32_t w0 = __builtin_amdgcn_readfirstlane(tw[t - r0]);
      const uint32_t w1 = __builtin_amdgcn_readfirstlane(tw[t - r0 + 1]);
      in.load(b, job.x, g.ldx, g.batch, ti, tj, w0, w1, buf);
      asm volatile("" ::: "memory");
      in.load_rest(b, ti, tj);
    }
  }

  // decode mode: the tile decoded last, stored right after the next tile's
  // data is in, as exactly TR stores (rows past the matrix edge write row 0
  // again, the same bytes), so that the wait partway through the tile can
  // leave just those stores outstanding: memory operations of a wavefront
  // complete in the order they were issued
  uint32_t pv[TR][4];
  uint32_t p_row = 0, p_col = 0, p_nrows = 0;
  bool p_active = false;
  auto store_prev = [&]() __attribute__((always_inline)) {
    if (p_nrows == 0) return;
    uint16_t* out = static_cast<uint16_t*>(job.y);
#pragma unroll
    for (int rr = 0; rr < TR; rr++) {
      const bool in_matrix = static_cast<uint32_t>(rr) < p_nrows;
      const uint32_t row = in_matrix ? rr : 0;
      const uint4 v = in_matrix ? make_uint4(pv[rr][0], pv[rr][1], pv[rr][2], pv[rr][3])
                                : make_uint4(pv[0][0], pv[0][1], pv[0][2], pv[0][3]);
      if (p_active)
        *reinterpret_cast<uint4*>(out + (static_cast<uint64_t>(p_row) * TR + row) * job.ld +
                                  static_cast<uint64_t>(p_col) * 512 + lane * 8) = v;
    }
  };
  while (t < r1) {
    if constexpr (MF) {
      // Matrix-core mode.  The whole tile is in (the next tile's loads go out
      // at the end of this one, so that the X loads below never wait behind
      // them: vector memory operations retire in order).
      wait_vmem();
      wave_sync_lds();
      const uint32_t q0 = interleave(buf, in.w0, in.a0, in.cb(), J, slot);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wave_sync_lds();
      uint32_t wv[TR][4];
#pragma unroll
      for (int k = 0; k < TR; k++) wv[k][0] = wv[k][1] = wv[k][2] = wv[k][3] = 0u;
      LaneBits br;
      br.init(slot, q0);
      if (in.active) decode_rows<TR, NX, 0, TR, FIT2>(in, br, tab, wv);
      // Y block (16 weight rows x 16 X rows) += W block (16 x 32) x X^T block
      // (32 x 16), 16 times over the tile's 512 columns.  MFMA operands: lane
      // l holds row l % 16 of W (rows 8..15 zero) and row l % 16 of X (zero
      // past the batch), columns 8 (l / 16) .. + 7 of the 32; the result holds
      // W rows 4 (l / 16) .. + 3 for X row l % 16.  The tile goes through the
      // slot, whose stream is no longer needed, 128 columns (16 lanes) at a
      // time: T[r][c] at byte r * 272 + 2 c (rows padded against bank
      // conflicts).
      const uint32_t m = lane & 15u, gq = lane >> 4;
      const uint32_t T = lds_addr(slot);
      const uint32_t zero = lds_addr(buf);  // the staging buffer's 4 zero guard words
      const uint32_t a_at = m < TR ? T + m * 272u + gq * 16u : zero;
      const uint32_t a_step = m < TR ? 64u : 0u;
      const uint64_t col0 = static_cast<uint64_t>(in.col) * 512;
      const bool x_row = m < g.batch;
      const uint16_t* xr = job.x + (x_row ? static_cast<uint64_t>(m) * g.ldx : 0) + col0;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < 4; h++) {
        // this phase's X (issued here, not hoisted: four phases at once would
        // not fit the registers)
        asm volatile("" ::: "memory");
        uint4 xb[4];
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
          const uint32_t kc = static_cast<uint32_t>(128 * h + 32 * qq) + gq * 8u;
          const bool ok = x_row && col0 + kc < b.cols;
          xb[qq] = *reinterpret_cast<const uint4*>(xr + (ok ? kc : 0u));
          if (!ok) xb[qq] = make_uint4(0, 0, 0, 0);
        }
        if (gq == static_cast<uint32_t>(h)) {
#pragma unroll
          for (int r = 0; r < TR; r++)
            lds_put4(T + static_cast<uint32_t>(r) * 272u + m * 16u,
                     make_uint4(wv[r][0], wv[r][1], wv[r][2], wv[r][3]));
        }
        wave_sync_lds();
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
          const uint4 av = lds_get4(a_at + static_cast<uint32_t>(qq) * a_step);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, xb[qq]), acc, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // this phase's reads are done before T is written again
        wave_sync_lds();
      }
      if (gq < TR / 4 && x_row) {
#pragma unroll
        for (int e = 0; e < 4; e++) gsum[((t - r0) * TR + gq * 4 + e) * g.batch + m] = acc[e];
      }
      TileRegs<TR, NX> nx;
      const uint64_t tn = claims ? claim() : r1;
      if (tn < r1) {
        const uint64_t ni = tn / n_tc;
        const uint32_t nj = static_cast<uint32_t>(tn - ni * n_tc);
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(tw[tn - r0]);
        const uint32_t w1 = __builtin_amdgcn_readfirstlane(tw[tn - r0 + 1]);
        nx.load(b, job.x, g.ldx, g.batch, ni, nj, w0, w1, buf);
        asm volatile("" ::: "memory");
        nx.load_rest(b, ni, nj);
      }
      in = nx;
      t = tn;
      continue;
    }
    // rows [0, PRE) decode before the next tile's loads go out: 7/8 of the
    // tile (issuing loads stalls a wavefront while HBM is saturated, and with
    // the loads later the first tiles of a launch decode sooner; measured
    // against half the tile: batch 1 on 9728 x 2560 pairs 5% faster, the
    // skinny modes 1-5% and the standalone decode 2%, nothing slower)
    constexpr int PRE = TR * 7 / 8;
    // every raw row below PRE is in: all but the last TR - PRE of the second
    // half's TR / 2 row loads (issued last, in row order)
    wait_vmem_but<(TR - PRE < TR / 2 ? TR - PRE : TR / 2)>();
    if constexpr (DECODE) store_prev();
    wave_sync_lds();
    // this tile's stream into the slot; the linear buffer is then free for
    // the next tile
    const uint32_t q0 = interleave(buf, in.w0, in.a0, in.cb(), J, slot);
    // skinny mode: the first batch rows' X, on its way while this tile decodes
    constexpr int GB = 32 / TR;  // batch rows per group: TR GB sums reduce at once
    uint4 xg[GB];
    if constexpr (NB == 0) load_xg<GB>(b, job.x, g.ldx, g.batch, 0, in.col, xg);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the copy's reads are done
    wave_sync_lds();
    float acc[TR * NA];
    uint32_t wv[TR][4];
#pragma unroll
    for (int k = 0; k < TR * NA; k++) acc[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < TR; k++) wv[k][0] = wv[k][1] = wv[k][2] = wv[k][3] = 0u;
    LaneBits br;
    br.init(slot, q0);
    if constexpr (NB <= 0) {
      if (in.active) decode_rows<TR, NX, 0, PRE, FIT2>(in, br, tab, wv);
    } else if constexpr (!MF) {
      if (in.active) gemv_rows<TR, NX, 0, PRE, FIT2>(in, br, tab, acc);
    }
    // the rest of the raw bytes, then the next tile's loads: they go out
    // PRE rows into this tile and nothing touches them before the next
    // iteration (decode mode: the previous tile's TR stores may stay in flight)
    if (DECODE && p_nrows > 0)
      wait_vmem_but<TR>();
    else
      wait_vmem();
    asm volatile("" ::: "memory");
    TileRegs<TR, NX> nx;
    const uint64_t tn = claims ? claim() : r1;
    if (tn < r1) {
      const uint64_t ni = tn / n_tc;
      const uint32_t nj = static_cast<uint32_t>(tn - ni * n_tc);
      const uint32_t w0 = __builtin_amdgcn_readfirstlane(tw[tn - r0]);
      const uint32_t w1 = __builtin_amdgcn_readfirstlane(tw[tn - r0 + 1]);
      nx.load(b, job.x, g.ldx, g.batch, ni, nj, w0, w1, buf);
      asm volatile("" ::: "memory");
      nx.load_rest(b, ni, nj);
    }
    if constexpr (DECODE) {
      if (in.active) decode_rows<TR, NX, PRE, TR, FIT2>(in, br, tab, wv);
#pragma unroll
      for (int rr = 0; rr < TR; rr++)
#pragma unroll
        for (int k = 0; k < 4; k++) pv[rr][k] = wv[rr][k];
      p_row = in.rowblk;
      p_col = in.col;
      p_nrows = in.nrows;
      p_active = in.active;
    } else if constexpr (NB == 0) {
      if (in.active) decode_rows<TR, NX, PRE, TR, FIT2>(in, br, tab, wv);
      // X rows in groups of GB: TR GB sums per lane, reduced over the
      // wavefront at once; lanes 2v and 2v + 1 end with sum v (row v / GB,
      // batch row g GB + v % GB)
      const uint32_t v = lane / 2, vr = v / GB;
      for (uint32_t gi2 = 0; gi2 * GB < g.batch; gi2++) {
        if (gi2 > 0) load_xg<GB>(b, job.x, g.ldx, g.batch, gi2, in.col, xg);
        float sums[TR * GB];
#pragma unroll
        for (int rr = 0; rr < TR; rr++)
#pragma unroll
          for (int k = 0; k < GB; k++) {
            float a = dot2(wv[rr][0], xg[k].x, 0.0f);
            a = dot2(wv[rr][1], xg[k].y, a);
            a = dot2(wv[rr][2], xg[k].z, a);
            sums[rr * GB + k] = dot2(wv[rr][3], xg[k].w, a);
          }
        const float sv = reduce_rows<TR * GB>(sums);
        const uint32_t beta = gi2 * GB + v % GB;
        if ((lane & 1u) == 0 && beta < g.batch) gsum[((t - r0) * TR + vr) * g.batch + beta] = sv;
      }
    } else if constexpr (!MF) {
      if (in.active) gemv_rows<TR, NX, PRE, TR, FIT2>(in, br, tab, acc);
      // lanes (64 / (TR NB)) v .. hold sum v: row v / NB, X row v % NB
      const float s = reduce_rows<TR * NA>(acc);
      constexpr uint32_t lanes_per_sum = kWave / (TR * NA);
      const uint32_t v = lane / lanes_per_sum;
      if ((lane & (lanes_per_sum - 1)) == 0) gsum[(t - r0) * TR * NA + v] = s;
    }
    in = nx;
    t = tn;
  }
  if constexpr (DECODE) {
    store_prev();  // nothing if this wavefront decoded no tile
    return;
  }
  __syncthreads();

  if constexpr (SKINNY) {
    // whole row blocks only: every output adds its tile sums in column order
    if (n_r == 0) return;
    const uint64_t rb_a = r0 / n_tc;
    const uint32_t nbs = NB > 0 && !MF ? NB : g.batch;  // sums per row of a tile in LDS
    const uint32_t per_rb = TR * g.batch;
    for (uint32_t k = threadIdx.x; k < n_r / n_tc * per_rb; k += blockDim.x) {
      const uint64_t rb = rb_a + k / per_rb;
      const uint32_t rr = (k % per_rb) / g.batch, beta = k % g.batch;
      const uint64_t row = rb * TR + rr;
      if (row >= b.rows) continue;
      float sum = 0.0f;
      for (uint64_t c = rb * n_tc; c < rb * n_tc + n_tc; c++) sum += gsum[((c - r0) * TR + rr) * nbs + beta];
      store_y(job.y, beta * g.ldy + row, sum, g.y_f32);
    }
    return;
  }

  // Row blocks [rb_a, rb_b] meet the range.  A row block inside it: each
  // row adds its tile sums in column order and is stored.  A row block that
  // range edges cut has contributors c = 0 .. k - 1, the workgroups whose
  // ranges meet it in column order, each with p_c, its own tile sums of the
  // row added in column order; y = ((p_0 + p_1) + p_2) + ... is formed along
  // a chain of k - 1 links, one workspace slot each (per row).  Link i meets
  // the running sum of p_0 .. p_(i-1) and p_i (p_0 goes to link 1): each
  // side swaps its value into the slot with the flag set, and the one that
  // finds the other's value there adds the two (one rounding of the same two
  // operands in either order), clears the slot, and carries the sum on to
  // link i + 1, or stores y at the last link.  One atomic per link and no
  // waiting on another workgroup; the order of the additions is fixed by the
  // ranges, so repeated calls give the same bits.
  if (n_r == 0) return;
  const uint64_t rb_a = r0 / n_tc, rb_b = (r1 - 1) / n_tc;
  for (uint32_t k = threadIdx.x; k < (rb_b - rb_a + 1) * TR; k += blockDim.x) {
    const uint64_t rb = rb_a + k / TR;
    const uint32_t rr = k % TR;
    const uint64_t row = rb * TR + rr;
    if (row >= b.rows) continue;
    const uint64_t first = rb * n_tc, last = first + n_tc;
    const uint64_t c0 = first > r0 ? first : r0;
    const uint64_t c1 = last < r1 ? last : r1;
    float sum = 0.0f;
    for (uint64_t c = c0; c < c1; c++) sum += gsum[(c - r0) * TR + rr];
    if (c0 == first && c1 == last) {
      store_y(job.y, row, sum, g.y_f32);
      continue;
    }
    // a cut row block (equal ranges only): links 1 .. g_last - g_first
    const uint64_t g_first = range_of(first, T, G), links = range_of(last - 1, T, G) - g_first;
    uint64_t link = gi == g_first ? 1 : gi - g_first;
    for (;;) {
      uint64_t* slot = job.slots + (first + link) * TR + rr;
      const uint64_t old = __hip_atomic_exchange(slot, kSlotFull | __builtin_bit_cast(uint32_t, sum), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
      if (!(old & kSlotFull)) break;  // first at this link: the other side carries on
      sum += __builtin_bit_cast(float, static_cast<uint32_t>(old));
      __hip_atomic_store(slot, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (link == links) {
        store_y(job.y, row, sum, g.y_f32);
        break;
      }
      link++;
    }
  }
}

// Generic path for any geometry, batch rows one after another:
// partial[(tj * batch + beta) * rows + n].
__global__ __launch_bounds__(kGenericWaves * kWave) void k_gemv_generic(BlobDev b, const uint16_t* __restrict__ X,
                                                                        uint64_t ldx, int batch,
                                                                        float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ __attribute__((aligned(16))) uint32_t tab[kTable];  // static: LDS address 0
  const uint32_t nw = blockDim.x / kWave;
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds + wave * b.buf_words;
  float* rowsum = reinterpret_cast<float*>(lds + nw * b.buf_words) + wave * static_cast<size_t>(b.tr) * b.s;
  load_table(tab, b.table);
  __syncthreads();
  const uint32_t lane = lane_id();
  const uint64_t nwaves = static_cast<uint64_t>(gridDim.x) * nw;
  for (uint64_t t = static_cast<uint64_t>(blockIdx.x) * nw + wave; t < b.n_tiles; t += nwaves) {
    const uint64_t ti = t / b.n_tc, tj = t % b.n_tc;
    const uint64_t row0 = ti * b.tr;
    const uint32_t nrows = static_cast<uint32_t>(umin64(b.tr, b.rows - row0));
    const uint64_t tile_c1 = umin64(b.cols, tj * b.tc + b.tc);
    const uint32_t w0 = sload(b.tile_words, t);
    const uint32_t w1 = sload(b.tile_words, t + 1);
    const uint32_t a0 = w0 & ~3u;
    stage_stream(b, a0, stage_blocks(b, a0, w1 < w0 ? w0 : w1), buf);
    wait_vmem();
    wave_sync_lds();
    for (int beta = 0; beta < batch; beta++) {
      const uint16_t* x = X + beta * ldx;
      uint32_t base = 128 + (w0 - a0) * 32;
      for (uint32_t c0i = 0; c0i < b.s; c0i += kWave) {
        const uint32_t c = c0i + lane;
        const uint32_t cb = c < b.s ? b.chunk_bits[t * b.s + c] : 0u;
        const uint32_t excl = wave_excl_scan(cb);
        const uint32_t bit = base + excl;
        base += __builtin_amdgcn_readlane(excl + cb, kWave - 1);
        if (c < b.s) {
          const uint64_t cc0 = tj * b.tc + static_cast<uint64_t>(c) * b.v;
          const uint64_t cc1 = cc0 < tile_c1 ? umin64(tile_c1, cc0 + b.v) : cc0;
          Bits br;
          br.init(buf, bit);
          // the chunk's symbols in row order, two codes per table lookup; each
          // row's products added in column order
          const uint32_t wdt = static_cast<uint32_t>(cc1 - cc0);
          if (wdt == 0) {
            for (uint32_t r = 0; r < nrows; r++) rowsum[r * b.s + c] = 0.0f;
          } else {
            const uint32_t nsym = nrows * wdt;
            uint32_t r = 0, kk = 0;  // row and column of the next symbol
            float a = 0.0f;
            auto add = [&](uint32_t e) __attribute__((always_inline)) {
              const uint64_t k = cc0 + kk;
              const uint32_t rb = b.raw[(row0 + r) * b.raw_ld + k];
              const uint32_t wbits = (((rb & 0x80u) << 8) | (e << 7) | (rb & 0x7Fu)) << 16;
              const float xf = __builtin_bit_cast(float, static_cast<uint32_t>(x[k]) << 16);
              a = __builtin_fmaf(__builtin_bit_cast(float, wbits), xf, a);
              if (++kk == wdt) {
                rowsum[r * b.s + c] = a;
                a = 0.0f;
                kk = 0;
                r++;
              }
            };
            uint32_t idx = 0;
            for (; idx + 1 < nsym; idx += 2) {
              const uint32_t ent = br.pair(tab);
              add((ent >> 7) & 0xFFu);
              add((ent >> 23) & 0xFFu);
            }
            if (idx < nsym) add(br.one(tab));
          }
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

// y[beta, n] = sum over column tiles of partial, in tile order.
__global__ void k_reduce(const float* __restrict__ partial, uint64_t rows, uint32_t n_tc, int batch,
                         void* __restrict__ y, uint64_t ldy, int y_f32) {
  const uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * static_cast<uint64_t>(batch)) return;
  const uint64_t beta = i / rows, n = i % rows;
  float s = 0.0f;
  for (uint32_t tj = 0; tj < n_tc; tj++) s += partial[(tj * static_cast<uint64_t>(batch) + beta) * rows + n];
  store_y(y, beta * ldy + n, s, y_f32);
}

// ------------------------------------------------- uncompressed comparator

// Same tiling, split, loads-up-front and reductions as k_gemv, reading BF16
// weights (16 bytes per lane per row) instead of decoding them.
template <int TR>
__global__ __launch_bounds__(kMaxWaves * kWave) void k_gemv_bf16(const uint16_t* __restrict__ w, uint64_t rows,
                                                                 uint64_t cols, uint64_t ld, uint32_t n_tc,
                                                                 uint64_t n_tr, Split sp,
                                                                 const uint16_t* __restrict__ x,
                                                                 void* __restrict__ y, int y_f32) {
  __shared__ float red[kMaxWaves * TR];
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t lane = lane_id();
  const uint32_t rbl = wave / sp.nw, wt = wave % sp.nw;
  for (uint64_t item = blockIdx.x; item < sp.items; item += gridDim.x) {
    const uint64_t ti = item * sp.rb + rbl;
    float acc[TR];
#pragma unroll
    for (int r = 0; r < TR; r++) acc[r] = 0.0f;
    if (ti < n_tr) {
      const uint64_t row0 = ti * TR;
      const uint32_t nrows = static_cast<uint32_t>(umin64(TR, rows - row0));
      for (uint32_t tj = wt; tj < n_tc; tj += sp.nw) {
        const uint64_t c0 = static_cast<uint64_t>(tj) * 512 + lane * 8;
        const bool active = c0 < cols;
        const uint64_t cc = active ? c0 : 0;
        const uint4 xv = *reinterpret_cast<const uint4*>(x + cc);
        uint4 wv[TR];
#pragma unroll
        for (int r = 0; r < TR; r++) {
          const uint64_t row = row0 + (static_cast<uint32_t>(r) < nrows ? r : nrows - 1);
          wv[r] = *reinterpret_cast<const uint4*>(w + row * ld + cc);
        }
        if (active) {
#pragma unroll
          for (int r = 0; r < TR; r++) {
            if (static_cast<uint32_t>(r) < nrows) {
              float a = acc[r];
              a = dot2(wv[r].x, xv.x, a);
              a = dot2(wv[r].y, xv.y, a);
              a = dot2(wv[r].z, xv.z, a);
              a = dot2(wv[r].w, xv.w, a);
              acc[r] = a;
            }
          }
        }
      }
    }
    const float s = reduce_rows<TR>(acc);
    constexpr uint32_t lanes_per_row = kWave / TR;
    if ((lane & (lanes_per_row - 1)) == 0) red[wave * TR + lane / lanes_per_row] = s;
    __syncthreads();
    if (threadIdx.x < sp.rb * TR) {
      const uint32_t rl = threadIdx.x / TR, r = threadIdx.x % TR;
      const uint64_t row = (item * sp.rb + rl) * TR + r;
      if (row < rows) {
        float sum = 0.0f;
        for (uint32_t wv2 = 0; wv2 < sp.nw; wv2++) sum += red[(rl * sp.nw + wv2) * TR + r];
        store_y(y, row, sum, y_f32);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- host glue

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr size_t kMaxLds = 160 * 1024 - kTable * 4;  // dynamic LDS beside the static table
constexpr int kCUs = 256;

struct Launch {
  BlobDev b;
  bool fast;  // S = 64, V = 8, TR in {4, 8, 16, 32}, K % 8 == 0
  uint32_t max_chunk_bits;
  uint32_t max_code_len;
};

nwc_status prepare(const nwc_info* info, const void* blob_dev, Launch* L) {
  nwc::Geometry g;
  if (!info || !blob_dev || !nwc::info_geometry(info, &g)) return NWC_ERR_INVALID_ARG;
  if (!aligned(blob_dev, 256)) return NWC_ERR_ALIGNMENT;
  if (info->max_tile_words > 65536u) return NWC_ERR_UNSUPPORTED;
  if (info->max_chunk_bits > static_cast<uint64_t>(g.tr) * g.v * g.lmax) return NWC_ERR_INVALID_ARG;
  L->max_chunk_bits = info->max_chunk_bits;
  L->max_code_len = info->max_code_len;
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
  b.n_tr = g.n_tr;
  b.n_tc = static_cast<uint32_t>(g.n_tc);
  b.tr = g.tr;
  b.tc = g.tc;
  b.s = g.s;
  b.v = g.v;
  b.stream_words = static_cast<uint32_t>(g.stream_words);
  // 4 zero guard words, room for the largest tile starting 3 words into a
  // 4-word block plus the bit reader's two words of look-ahead (in 16-byte
  // pieces), and 4 spare words that the reader may fetch past the end
  b.buf_words = 4 + ((info->max_tile_words + 3 + 2 + 3) / 4) * 4 + 4;
  L->fast = g.s == 64 && g.v == 8 && (g.tr == 4 || g.tr == 8 || g.tr == 16 || g.tr == 32) && g.cols % 8 == 0;
  return NWC_OK;
}

// Split for the fused kernels: up to 16 wavefronts per workgroup; several row
// blocks per work item when the matrix has few column tiles and many rows.
Split make_split(uint64_t n_tr, uint32_t n_tc, uint32_t max_waves) {
  Split sp;
  sp.nw = std::min<uint32_t>(n_tc, max_waves);
  const uint32_t fit = std::max<uint32_t>(1, max_waves / sp.nw);
  const uint64_t want = (n_tr + 2 * kCUs - 1) / (2 * kCUs);  // keep >= 2 items per CU when possible
  sp.rb = static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(fit, want)));
  sp.waves = sp.nw * sp.rb;
  sp.items = (n_tr + sp.rb - 1) / sp.rb;
  return sp;
}

template <typename K>
hipError_t set_lds(K kernel, size_t lds) {
  if (lds + kTable * 4 <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(lds));
}

// Launch a kernel and report that launch's own status (hipLaunchKernel
// returns it; the triple-chevron form would leave it in the process-wide
// last-error slot, where another library's error could be read as ours).
// The arguments are converted to the kernel's parameter types first.
template <typename... P, typename... A>
nwc_status launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  std::tuple<P...> args{static_cast<P>(a)...};
  void* argv[sizeof...(P)];
  std::apply([&](auto&... e) {
    int i = 0;
    ((argv[i++] = static_cast<void*>(&e)), ...);
  }, args);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, s) == hipSuccess
             ? NWC_OK
             : NWC_ERR_HIP;
}

// grid for a persistent loop over `items` work items of `waves` wavefronts
unsigned grid_for(uint64_t items, uint32_t waves, size_t lds) {
  const uint64_t by_waves = std::max<uint64_t>(1, 32 / waves);
  const uint64_t by_lds = std::max<uint64_t>(1, (160 * 1024) / (lds + kTable * 4));
  const uint64_t per_cu = std::min(by_waves, by_lds);
  return static_cast<unsigned>(std::min<uint64_t>(items, kCUs * per_cu));
}

// Workspace of the fused batch-1 path: one 64-bit chain slot per tile and row.
size_t fused_ws_bytes(const nwc::Geometry& g) {
  return (g.n_tiles * static_cast<uint64_t>(g.tr) * 8 + 255) / 256 * 256;
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return kCUs;
  return n;
}

// Batch-1 fused launch over `count` matrices with the same tile height.
// Split of a launch's tiles into workgroup ranges: the ranges' sizes and the
// LDS they need besides the wavefronts' buffers.
struct GemvPlan {
  uint32_t groups[kMaxJobs];
  uint32_t whole_rows[kMaxJobs];
  uint32_t total_groups;
  uint64_t range;  // tiles in the largest range
  uint32_t tw_words() const { return static_cast<uint32_t>((range + 1 + 3) & ~3ull); }
  // sums per tile: TR (batch 1) or TR x batch (skinny mode)
  size_t group_lds(uint32_t sums_per_tile) const { return (4 + tw_words() + range * sums_per_tile) * 4; }
};

// Workgroups: as many as the chip holds at once (`cap`), or one per tile
// when there are fewer tiles, shared out in proportion to each matrix's tiles
// (largest remainders); each matrix's tiles are cut into equal ranges.
// Workgroups land one per CU, then a second per CU, so equal ranges give
// every CU the same number of tiles and every wavefront the same number give
// or take one, which whole row blocks per range rarely can.  A matrix's
// ranges are whole row blocks instead when that changes neither its
// workgroups nor its tiles per wavefront.
template <int TR>
GemvPlan plan_gemv(const Launch* L, int count, uint64_t cap, uint32_t nw, size_t group_lds) {
  GemvPlan p;
  std::memset(&p, 0, sizeof(p));
  uint64_t total = 0;
  for (int j = 0; j < count; j++) total += L[j].b.n_tiles;
  // the largest range whose offsets and tile sums fit the group's LDS
  const uint64_t max_range = std::max<uint64_t>(1, (group_lds / 4 - 4 - 4) / (TR + 1));
  const uint64_t want = std::max<uint64_t>(count, std::min<uint64_t>(cap, total));
  uint64_t G[kMaxJobs], given = 0;
  for (int j = 0; j < count; j++) {
    G[j] = want * L[j].b.n_tiles / total;
    given += G[j];
  }
  bool bumped[kMaxJobs] = {};
  while (given < want) {  // fewer than count times
    int best = -1;
    uint64_t rem = 0;
    for (int j = 0; j < count; j++) {
      const uint64_t r = want * L[j].b.n_tiles % total;
      if (!bumped[j] && (best < 0 || r > rem)) {
        rem = r;
        best = j;
      }
    }
    bumped[best] = true;
    G[best]++;
    given++;
  }
  p.range = 1;
  for (int j = 0; j < count; j++) {
    const uint64_t T = L[j].b.n_tiles, n_tr = L[j].b.n_tr, n_tc = L[j].b.n_tc;
    uint64_t Gj = std::min<uint64_t>(T, std::max<uint64_t>(1, G[j]));
    Gj = std::max<uint64_t>(Gj, (T + max_range - 1) / max_range);
    const uint64_t range = (T + Gj - 1) / Gj;
    const uint64_t k = (n_tr + Gj - 1) / Gj;  // row blocks per whole-row range
    const bool whole = (n_tr + k - 1) / k == Gj && k * n_tc <= max_range &&
                       (k * n_tc + nw - 1) / nw <= (range + nw - 1) / nw;
    p.whole_rows[j] = whole ? 1u : 0u;
    p.groups[j] = static_cast<uint32_t>(Gj);
    p.range = std::max<uint64_t>(p.range, whole ? k * n_tc : range);
    p.total_groups += p.groups[j];
  }
  return p;
}

// Sums the skinny mode keeps per row of a tile: the batch, except that with
// 8-row tiles a batch of 3 runs as 4 (the cross-lane sum needs a power of two).
uint32_t skinny_sums_per_row(int tr, int batch) { return tr == 8 && batch == 3 ? 4u : static_cast<uint32_t>(batch); }

// Row blocks of one matrix per skinny-mode range: as many as keep one range
// per resident workgroup (so that every range runs in one pass), no more
// than the workgroup's LDS for tile sums holds (at least kSkinnyLds, which
// always holds one row block's).
uint64_t skinny_rows_per_range(uint64_t n_tr, uint64_t n_tc, int tr, int batch, uint64_t cap, size_t group_lds) {
  const uint64_t fit = std::max<size_t>(kSkinnyLds, group_lds) / (n_tc * tr * skinny_sums_per_row(tr, batch) * 4 + 4 * n_tc);
  return std::max<uint64_t>(1, std::min<uint64_t>(fit, (n_tr + cap - 1) / cap));
}

template <int TR>
GemvPlan plan_skinny(const Launch& L, int batch, uint64_t cap, size_t group_lds) {
  GemvPlan p;
  std::memset(&p, 0, sizeof(p));
  const uint64_t k = skinny_rows_per_range(L.b.n_tr, L.b.n_tc, TR, batch, cap, group_lds);
  p.whole_rows[0] = 1;
  p.groups[0] = static_cast<uint32_t>((L.b.n_tr + k - 1) / k);
  p.total_groups = p.groups[0];
  p.range = k * L.b.n_tc;
  return p;
}

// The batch-1 launch (count matrices), the skinny one (one matrix, batch
// 2..16) or the standalone decode (one matrix, W' rows of ldy elements):
// wavefronts per workgroup are the size with the most resident wavefronts
// per CU (registers and LDS both count, the ranges' LDS included), the
// larger size on a tie.
template <int TR, int MAXW, int NB, bool FIT2 = false>
nwc_status launch_gemv(const Launch* L, const uint16_t* const* x, void* const* y, uint8_t* const* ws, int count,
                       int y_f32, hipStream_t s, int batch = 1, uint64_t ldx = 0, uint64_t ldy = 0,
                       const uint64_t* ld_out = nullptr) {
  GemvGroup g;
  std::memset(&g, 0, sizeof(g));
  uint32_t lane_words = 0, buf_words = 0;
  for (int j = 0; j < count; j++) {
    // a lane's words start with the one holding bit (chunk start - 2), so
    // the reader starts at bit <= 31 and its last window (at most chunk
    // bits - 1 further) reads one word of look-ahead; rounded up to even
    lane_words = std::max(lane_words, (((30 + L[j].max_chunk_bits) >> 5) + 2 + 1) & ~1u);
    buf_words = std::max(buf_words, L[j].b.buf_words);
  }
  // the matrix-core mode passes each decoded tile through the slot (8 rows
  // of 272 bytes)
  if (NB == 16) lane_words = std::max(lane_words, 10u);
  // the interleaving copy reads up to lane_words past the last chunk start;
  // whole 256-byte units keep every slot 256-byte aligned
  buf_words = (buf_words + lane_words + 63) & ~63u;
  const size_t per_wave = (static_cast<size_t>(kWave) * lane_words + buf_words) * 4;
  constexpr bool SKINNY = NB == 0 || NB > 1;
  const uint32_t sums = NB < 0 ? 0 : NB == 0 || NB == 16 ? TR * batch : TR * NB;
  const uint32_t cus = static_cast<uint32_t>(cu_count());
  auto occupancy = [&](uint32_t n, size_t lds, int* k) {
    if (lds > kMaxLds) {
      *k = 0;
      return hipSuccess;
    }
    hipError_t e = set_lds(k_gemv<TR, MAXW, NB>, lds);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(k, k_gemv<TR, MAXW, NB>, n * kWave, lds);
    return e;
  };
  // the LDS a workgroup has for its ranges' sums when k workgroups of n
  // wavefronts share a CU (the decode table is static LDS)
  auto group_budget = [&](uint32_t n, int k) -> size_t {
    const size_t per_group = (kMaxLds + kTable * 4) / static_cast<size_t>(k);  // all of a CU's LDS, shared
    const size_t used = kTable * 4 + n * per_wave + 1024;  // table, wavefront buffers, allocation slack
    return per_group > used + 1024 ? per_group - used : 1024;
  };
  auto plan = [&](uint64_t cap, uint32_t n, int k) {
    if constexpr (SKINNY)
      return plan_skinny<TR>(L[0], batch, cap, group_budget(n, k));
    else
      return plan_gemv<TR>(L, count, cap, n, std::max<size_t>(kGroupLds, group_budget(n, k)));
  };
  uint32_t nw = 0;
  int per_cu = 0;
  GemvPlan best;
  std::memset(&best, 0, sizeof(best));
  const uint32_t sizes[] = {16, 12, 8, 4, 2, 1};
  for (uint32_t n : sizes) {
    if (n > MAXW) continue;
    int k = 0;
    if (occupancy(n, n * per_wave, &k) != hipSuccess) return NWC_ERR_HIP;
    if (k < 1) continue;
    // the ranges' LDS may cost residency: plan again with what is left
    GemvPlan p = plan(static_cast<uint64_t>(cus) * k, n, k);
    int k2 = 0;
    if (occupancy(n, n * per_wave + p.group_lds(sums), &k2) != hipSuccess) return NWC_ERR_HIP;
    if (k2 < k) {
      if (k2 < 1) continue;
      k = k2;
      p = plan(static_cast<uint64_t>(cus) * k, n, k);
      if (occupancy(n, n * per_wave + p.group_lds(sums), &k2) != hipSuccess) return NWC_ERR_HIP;
      if (k2 < k) continue;
    }
    if (static_cast<uint64_t>(k) * n > static_cast<uint64_t>(per_cu) * nw) {
      nw = n;
      per_cu = k;
      best = p;
    }
  }
  if (nw == 0 || per_cu < 1) return NWC_ERR_UNSUPPORTED;
  uint32_t groups = 0;
  for (int j = 0; j < count; j++) {
    GemvJob& job = g.job[j];
    job.b = L[j].b;
    job.x = x[j];
    job.y = y[j];
    if (NB == 1) {
      job.slots = reinterpret_cast<uint64_t*>(ws[j]);
    }
    job.whole_rows = best.whole_rows[j];
    job.groups = best.groups[j];
    job.ld = ld_out ? ld_out[j] : 0;
    job.g0 = groups;
    groups += job.groups;
  }
  g.count = static_cast<uint32_t>(count);
  g.y_f32 = y_f32;
  g.lane_words = lane_words;
  g.buf_words = buf_words;
  g.tw_words = best.tw_words();
  g.ldx = ldx;
  g.ldy = ldy;
  g.batch = static_cast<uint32_t>(batch);
  const size_t lds = nw * per_wave + best.group_lds(sums);
  if (set_lds(k_gemv<TR, MAXW, NB, FIT2>, lds) != hipSuccess) return NWC_ERR_HIP;
  return launch(k_gemv<TR, MAXW, NB, FIT2>, dim3(groups), dim3(nw * kWave), lds, s, g);
}

// The batch-1 (NB = 1) or decode (NB = -1) launch for the matrices' tile
// height, with the second-lookup-free decode when every code is <= 6 bits.
template <int NB, typename... A>
nwc_status launch_fused(const Launch* L, int count, A... a) {
  bool fit2 = true;
  for (int j = 0; j < count; j++) fit2 = fit2 && L[j].max_code_len <= 6;
  switch (L[0].b.tr) {
    case 4: return fit2 ? launch_gemv<4, 16, NB, true>(L, a...) : launch_gemv<4, 16, NB>(L, a...);
    case 8: return fit2 ? launch_gemv<8, 16, NB, true>(L, a...) : launch_gemv<8, 16, NB>(L, a...);
    case 16: return fit2 ? launch_gemv<16, 8, NB, true>(L, a...) : launch_gemv<16, 8, NB>(L, a...);
    default: return fit2 ? launch_gemv<32, 4, NB, true>(L, a...) : launch_gemv<32, 4, NB>(L, a...);
  }
}

// Whether a blob and batch take the skinny mode of the fused kernel (no
// workspace): default chunk geometry, 8- or 16-row tiles, and one row
// block's tile sums within kSkinnyLds.
bool skinny_fits(const nwc::Geometry& g, int batch) {
  const bool fast = g.s == 64 && g.v == 8 && (g.tr == 8 || g.tr == 16) && g.cols % 8 == 0;
  return fast && batch >= 2 && batch <= 16 &&
         static_cast<uint64_t>(g.n_tc) * g.tr * skinny_sums_per_row(static_cast<int>(g.tr), batch) * 4 <= kSkinnyLds;
}

size_t generic_ws_bytes(const nwc::Geometry& g, int batch) {
  return static_cast<size_t>(g.n_tc) * batch * g.rows * sizeof(float);
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
  const bool fast = g.s == 64 && g.v == 8 && (g.tr == 4 || g.tr == 8 || g.tr == 16 || g.tr == 32) && g.cols % 8 == 0;
  if (fast && batch == 1)
    *bytes = fused_ws_bytes(g);
  else if (skinny_fits(g, batch))
    *bytes = 0;
  else
    *bytes = generic_ws_bytes(g, batch);
  return NWC_OK;
}

nwc_status nwc_decode(const nwc_info* info, const void* blob_dev, uint16_t* w_dev, uint64_t ld, void* stream) {
  if (!w_dev) return NWC_ERR_INVALID_ARG;
  Launch L;
  nwc_status st = prepare(info, blob_dev, &L);
  if (st) return st;
  if (ld < L.b.cols) return NWC_ERR_INVALID_ARG;
  if (!aligned(w_dev, 2)) return NWC_ERR_ALIGNMENT;
  const bool vec = aligned(w_dev, 16) && ld % 8 == 0;
  const size_t lds = (static_cast<size_t>(kGenericWaves) * L.b.buf_words) * 4;
  if (lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint64_t blocks = (L.b.n_tiles + kGenericWaves - 1) / kGenericWaves;
  const unsigned grid = static_cast<unsigned>(std::min<uint64_t>(blocks, kCUs * 8));
  const unsigned threads = kGenericWaves * kWave;
  if (L.fast && vec) {
    const uint16_t* none = nullptr;
    void* out = w_dev;
    return launch_fused<-1>(&L, 1, &none, &out, static_cast<uint8_t* const*>(nullptr), 1, 0, s, 1, uint64_t{0},
                            uint64_t{0}, static_cast<const uint64_t*>(&ld));
  } else {
    if (set_lds(k_decode_generic, lds) != hipSuccess) return NWC_ERR_HIP;
    return launch(k_decode_generic, dim3(grid), dim3(threads), lds, s, L.b, w_dev, ld);
  }
}

nwc_status nwc_gather_rows(const nwc_info* info, const void* blob_dev, const uint32_t* ids_dev, uint32_t n_ids,
                           uint16_t* out_dev, uint64_t ld, void* stream) {
  if (!ids_dev || !out_dev || n_ids == 0) return NWC_ERR_INVALID_ARG;
  Launch L;
  nwc_status st = prepare(info, blob_dev, &L);
  if (st) return st;
  if (ld < L.b.cols) return NWC_ERR_INVALID_ARG;
  if (!aligned(out_dev, 2) || !aligned(ids_dev, 4)) return NWC_ERR_ALIGNMENT;
  const size_t lds = (static_cast<size_t>(kGenericWaves) * L.b.buf_words) * 4;
  if (lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
  const uint64_t items = static_cast<uint64_t>(n_ids) * L.b.n_tc;
  const unsigned grid = static_cast<unsigned>(std::min<uint64_t>((items + kGenericWaves - 1) / kGenericWaves, kCUs * 8));
  if (set_lds(k_gather, lds) != hipSuccess) return NWC_ERR_HIP;
  return launch(k_gather, dim3(grid), dim3(kGenericWaves * kWave), lds, static_cast<hipStream_t>(stream), L.b, ids_dev,
                n_ids, out_dev, ld);
}

static nwc_status gemm_common(const nwc_info* info, const void* blob_dev, const uint16_t* X, uint64_t ldx, int batch,
                              void* Y, uint64_t ldy, nwc_out_type yt, void* ws, size_t ws_bytes, void* stream) {
  if (!X || !Y) return NWC_ERR_INVALID_ARG;
  if (yt != NWC_OUT_BF16 && yt != NWC_OUT_F32) return NWC_ERR_INVALID_ARG;
  Launch L;
  nwc_status st = prepare(info, blob_dev, &L);
  if (st) return st;
  size_t need = 0;
  nwc_workspace_size(info, batch, &need);
  if (need && !ws) return NWC_ERR_INVALID_ARG;
  if (ws_bytes < need) return NWC_ERR_BUFFER_TOO_SMALL;
  if (batch > 1 && (ldx < L.b.cols || ldy < L.b.rows)) return NWC_ERR_INVALID_ARG;
  if (!aligned(Y, yt == NWC_OUT_F32 ? 4 : 2) || !aligned(X, 2)) return NWC_ERR_ALIGNMENT;
  if (need && !aligned(ws, L.fast && batch == 1 ? 256 : 16)) return NWC_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int y_f32 = yt == NWC_OUT_F32 ? 1 : 0;
  const bool xvec = aligned(X, 16) && (batch == 1 || ldx % 8 == 0);
  if (need == 0 && !xvec) return NWC_ERR_ALIGNMENT;
  if (L.fast && batch == 1) {
    if (!xvec) return NWC_ERR_ALIGNMENT;
    void* yy = Y;
    uint8_t* w8 = static_cast<uint8_t*>(ws);
    return launch_fused<1>(&L, 1, &X, &yy, &w8, 1, y_f32, s);
  }
  if (need == 0) {
    // skinny mode of the fused kernel (nwc_workspace_size said so)
    const uint16_t* XX = X;
    void* yy = Y;
    // up to 32 / TR X rows are multiplied as each pair is decoded; more go
    // through the tile decoded into registers, and from 10 X rows on (8-row
    // tiles) through the matrix cores, which then cost less than the
    // vector products they replace
    // (with codes of at most 6 bits, the second-lookup-free decode)
    const bool fit2 = L.max_code_len <= 6;
#define NWC_SKINNY(TR_, MAXW_, NB_)                                                                      \
  return fit2 ? launch_gemv<TR_, MAXW_, NB_, true>(&L, &XX, &yy, nullptr, 1, y_f32, s, batch, ldx, ldy) \
              : launch_gemv<TR_, MAXW_, NB_>(&L, &XX, &yy, nullptr, 1, y_f32, s, batch, ldx, ldy)
    if (L.b.tr == 8) {
      switch (batch) {
        case 2: NWC_SKINNY(8, 16, 2);
        case 3:  // a power-of-two count of sums per lane: X row 3 is zero
        case 4: NWC_SKINNY(8, 16, 4);
        default:
          if (batch < 10) NWC_SKINNY(8, 16, 0);
          NWC_SKINNY(8, 16, 16);
      }
    }
    if (batch == 2) NWC_SKINNY(16, 8, 2);
    NWC_SKINNY(16, 8, 0);
#undef NWC_SKINNY
  }
  // generic path: partial sums per column tile, then a reduction
  const size_t lds = (static_cast<size_t>(kGenericWaves) * L.b.buf_words) * 4 +
                     static_cast<size_t>(kGenericWaves) * L.b.tr * L.b.s * 4;
  if (lds > kMaxLds) return NWC_ERR_UNSUPPORTED;
  if (set_lds(k_gemv_generic, lds) != hipSuccess) return NWC_ERR_HIP;
  float* part = static_cast<float*>(ws);
  const uint64_t blocks = (L.b.n_tiles + kGenericWaves - 1) / kGenericWaves;
  const unsigned grid = static_cast<unsigned>(std::min<uint64_t>(blocks, kCUs * 8));
  st = launch(k_gemv_generic, dim3(grid), dim3(kGenericWaves * kWave), lds, s, L.b, X, batch == 1 ? 0 : ldx, batch,
              part);
  if (st) return st;
  const uint64_t n = L.b.rows * static_cast<uint64_t>(batch);
  return launch(k_reduce, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, part, L.b.rows, L.b.n_tc,
                batch, Y, batch == 1 ? 0 : ldy, y_f32);
}

nwc_status nwc_gemv(const nwc_info* info, const void* blob_dev, const uint16_t* x_dev, void* y_dev,
                    nwc_out_type y_type, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(info, blob_dev, x_dev, 0, 1, y_dev, 0, y_type, ws, ws_bytes, stream);
}

nwc_status nwc_gemv_batched(int count, const nwc_info* infos, const void* const* blobs_dev,
                            const uint16_t* const* x_dev, void* const* y_dev, nwc_out_type y_type, void* ws,
                            size_t ws_bytes, void* stream) {
  if (count < 1 || count > kMaxJobs || !infos || !blobs_dev || !x_dev || !y_dev || !ws) return NWC_ERR_INVALID_ARG;
  if (y_type != NWC_OUT_BF16 && y_type != NWC_OUT_F32) return NWC_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return NWC_ERR_ALIGNMENT;
  Launch L[kMaxJobs];
  uint8_t* w8[kMaxJobs];
  size_t used = 0;
  for (int j = 0; j < count; j++) {
    if (!x_dev[j] || !y_dev[j]) return NWC_ERR_INVALID_ARG;
    nwc_status st = prepare(&infos[j], blobs_dev[j], &L[j]);
    if (st) return st;
    if (!L[j].fast || L[j].b.tr != L[0].b.tr) return NWC_ERR_UNSUPPORTED;
    if (!aligned(x_dev[j], 16) || !aligned(y_dev[j], y_type == NWC_OUT_F32 ? 4 : 2)) return NWC_ERR_ALIGNMENT;
    nwc::Geometry g;
    nwc::info_geometry(&infos[j], &g);
    w8[j] = static_cast<uint8_t*>(ws) + used;
    used += fused_ws_bytes(g);
  }
  if (ws_bytes < used) return NWC_ERR_BUFFER_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int y_f32 = y_type == NWC_OUT_F32 ? 1 : 0;
  return launch_fused<1>(L, count, x_dev, y_dev, static_cast<uint8_t* const*>(w8), count, y_f32, s);
}

nwc_status nwc_decode_batched(int count, const nwc_info* infos, const void* const* blobs_dev, uint16_t* const* w_dev,
                              const uint64_t* ld, void* stream) {
  if (count < 1 || count > kMaxJobs || !infos || !blobs_dev || !w_dev || !ld) return NWC_ERR_INVALID_ARG;
  Launch L[kMaxJobs];
  const uint16_t* none[kMaxJobs] = {};
  void* out[kMaxJobs];
  for (int j = 0; j < count; j++) {
    if (!w_dev[j]) return NWC_ERR_INVALID_ARG;
    nwc_status st = prepare(&infos[j], blobs_dev[j], &L[j]);
    if (st) return st;
    if (ld[j] < L[j].b.cols) return NWC_ERR_INVALID_ARG;
    if (!L[j].fast || L[j].b.tr != L[0].b.tr) return NWC_ERR_UNSUPPORTED;
    if (!aligned(w_dev[j], 16) || ld[j] % 8) return NWC_ERR_ALIGNMENT;
    out[j] = w_dev[j];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_fused<-1>(L, count, none, out, static_cast<uint8_t* const*>(nullptr), count, 0, s, 1, uint64_t{0},
                          uint64_t{0}, static_cast<const uint64_t*>(ld));
}

nwc_status nwc_gemm_skinny(const nwc_info* info, const void* blob_dev, const uint16_t* X_dev, uint64_t ldx, int batch,
                           void* Y_dev, uint64_t ldy, nwc_out_type y_type, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 2 || batch > 16) return NWC_ERR_INVALID_ARG;
  return gemm_common(info, blob_dev, X_dev, ldx, batch, Y_dev, ldy, y_type, ws, ws_bytes, stream);
}

nwc_status nwc_bf16_workspace_size(uint64_t rows, uint64_t cols, size_t* bytes) {
  if (!bytes || rows < 1 || cols < 1) return NWC_ERR_INVALID_ARG;
  *bytes = 0;
  return NWC_OK;
}

nwc_status nwc_gemv_bf16(const uint16_t* w_dev, uint64_t rows, uint64_t cols, uint64_t ld, const uint16_t* x_dev,
                         void* y_dev, nwc_out_type y_type, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!w_dev || !x_dev || !y_dev || rows < 1 || cols < 1 || ld < cols) return NWC_ERR_INVALID_ARG;
  if (y_type != NWC_OUT_BF16 && y_type != NWC_OUT_F32) return NWC_ERR_INVALID_ARG;
  if (cols % 8 || ld % 8 || !aligned(w_dev, 16) || !aligned(x_dev, 16)) return NWC_ERR_ALIGNMENT;
  if (!aligned(y_dev, y_type == NWC_OUT_F32 ? 4 : 2)) return NWC_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t n_tc = static_cast<uint32_t>((cols + 511) / 512);
  const uint64_t n_tr = (rows + 15) / 16;
  const Split sp = make_split(n_tr, n_tc, kMaxWaves);
  return launch(k_gemv_bf16<16>, dim3(grid_for(sp.items, sp.waves, 4096)), dim3(sp.waves * kWave), 0, s, w_dev, rows,
                cols, ld, n_tc, n_tr, sp, x_dev, y_dev, y_type == NWC_OUT_F32 ? 1 : 0);
}

}  // extern "C"
