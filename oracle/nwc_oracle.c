/*
 * nwc_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, deliberately unoptimised CPU model of lossless BF16 weight
 * compression (raw sign+mantissa byte plane, Huffman-coded exponent plane) and
 * of the FP64 matrix-vector product it feeds.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this file; the
 * product library shares no code, header, table or constant with it.
 *
 * Sources followed (pages as published; statements restated, not quoted):
 *  [BF16]  "Efficient ML #1 -- Deep Learning Data Types" (blog.caveduck.io),
 *          section 4 "Half the size: FP16 and BF16" (1 sign, 8 exponent,
 *          7 fraction bits, bias 127; worked example 2.5) and section 3
 *          "Special values" (exponent 0 = zero/subnormal, 255 = inf/NaN).
 *  [NWC]   "NWC -- Neural Weight Compression" (PyPI project description of
 *          neural-weight-compression 0.9.0), section "How it works", bullets
 *          "Byte planes" (one byte plane stored raw, the exponent plane
 *          entropy coded) and "Fused kernel" (each lane decodes its own bit
 *          stream for a block of rows x columns).
 *  [UNW]   "Unweight: how we compressed an LLM 22% without sacrificing
 *          quality" (Techlist.io summary), section "Compressing BF16 Weights"
 *          (Huffman code on the exponent byte, sign and mantissa kept as is).
 *  [PM]    Larmore & Hirschberg, "A fast algorithm for optimal length-limited
 *          Huffman codes", JACM 1990 (package-merge).  Not on the pages.
 *  [RFC]   RFC 1951 (DEFLATE) section 3.1.1 (bit packing) and 3.2.2
 *          (canonical codes from code lengths).  Not on the pages.
 *
 * Blob layout (format version 1), all integers little-endian:
 *   header (256 B) | code_len[256] u8 | decode table u32[4096] |
 *   tile_words u32[n_tiles+1] | chunk_bits u16[n_chunks] |
 *   raw plane u8[rows][raw_ld] | stream u32[stream_words] + 16 zero bytes
 * Each section starts at a multiple of 256 bytes; gaps are zero.
 *
 * Parity status: every function here is pinned by the CPU tests (see the
 * test files that exercise it); none is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ESMALL (-2)
#define ORC_EFORMAT (-3)

#define ORC_MAGIC 0x4243574Eu /* "NWCB" */
#define ORC_VERSION 1u
#define ORC_HEADER_BYTES 256u
#define ORC_TABLE_BITS 12u
#define ORC_TABLE_ENTRIES 4096u

/* ------------------------------------------------------------------ */
/* BF16 value and byte planes  [BF16], [NWC] "Byte planes", [UNW]       */
/* ------------------------------------------------------------------ */

/* Value of one BF16 bit pattern from the definition: sign bit 15, exponent
 * bits 14..7 with bias 127, fraction bits 6..0.  Exponent 0 gives zero or a
 * subnormal (no implicit 1, scale 2^(1-127)); exponent 255 gives an infinity
 * (fraction 0) or a NaN.  [BF16] sections 3 and 4. */
double orc_bf16_value(uint16_t b) {
  int s = (b >> 15) & 1;
  int e = (b >> 7) & 0xFF;
  int f = b & 0x7F;
  double sign = s ? -1.0 : 1.0;
  if (e == 255) return f == 0 ? sign * INFINITY : NAN;
  if (e == 0) return sign * ldexp((double)f / 128.0, 1 - 127);
  return sign * ldexp(1.0 + (double)f / 128.0, e - 127);
}

/* Split into the exponent byte e (bits 14..7) and the raw byte r, which holds
 * the sign in its bit 7 and the seven fraction bits in bits 6..0. */
void orc_split(const uint16_t *w, uint64_t n, uint8_t *e, uint8_t *r) {
  for (uint64_t i = 0; i < n; i++) {
    uint16_t b = w[i];
    e[i] = (uint8_t)((b >> 7) & 0xFF);
    r[i] = (uint8_t)(((b >> 8) & 0x80) | (b & 0x7F));
  }
}

/* Inverse of orc_split. */
void orc_join(const uint8_t *e, const uint8_t *r, uint64_t n, uint16_t *w) {
  for (uint64_t i = 0; i < n; i++) {
    uint16_t sign = (uint16_t)((r[i] >> 7) & 1);
    uint16_t frac = (uint16_t)(r[i] & 0x7F);
    w[i] = (uint16_t)((sign << 15) | ((uint16_t)e[i] << 7) | frac);
  }
}

void orc_histogram(const uint8_t *e, uint64_t n, uint64_t *h) {
  for (int s = 0; s < 256; s++) h[s] = 0;
  for (uint64_t i = 0; i < n; i++) h[e[i]]++;
}

/* ------------------------------------------------------------------ */
/* Length-limited code lengths by package-merge  [PM]                  */
/* ------------------------------------------------------------------ */

typedef struct {
  uint64_t weight;
  int leaf;   /* 1: a single symbol, 0: a package of two items */
  int sym;    /* symbol, for a leaf */
  int child;  /* for a package: index of its first item in the previous list */
} pm_item;

/* Count the leaves inside item idx of list level `lv`, recursively. */
static void pm_count(pm_item **lists, int lv, int idx, int *len) {
  pm_item *it = &lists[lv][idx];
  if (it->leaf) {
    len[it->sym]++;
    return;
  }
  pm_count(lists, lv - 1, it->child, len);
  pm_count(lists, lv - 1, it->child + 1, len);
}

/* Optimal prefix-code lengths for the symbol counts h, symbol s at most
 * cap[s] bits (every cap[s] <= lmax).  Symbols with h = 0 get length 0.  One
 * present symbol gets length 1.  For n >= 2 present symbols (package-merge,
 * the coin-collector form: a symbol has one coin of width 2^-d for every
 * d = 1 .. cap[s]):
 *   leaves are sorted by (count, symbol) ascending;
 *   list 0 holds the leaves whose cap reaches lmax; then lmax-1 times: pair
 *   consecutive items of the current list into packages (an odd last item is
 *   dropped) and merge the packages with the leaves whose cap reaches the
 *   list's level (lmax - list index) by weight, a leaf going first on equal
 *   weight;
 *   the first 2n-2 items of the final list are selected and a symbol's length
 *   is the number of selected items that contain it.
 * Returns ORC_EINVAL if no symbol is present or the caps leave no prefix code
 * (the sum of 2^-cap over the present symbols exceeds 1; the final list then
 * holds fewer than 2n-2 items). */
static int code_lengths_capped(const uint64_t *h, int lmax, const int *cap, uint8_t *len_out) {
  int n = 0;
  int syms[256];
  for (int s = 0; s < 256; s++) {
    len_out[s] = 0;
    if (h[s] > 0) syms[n++] = s;
  }
  if (n == 0 || lmax < 1 || lmax > 30) return ORC_EINVAL;
  if (n == 1) {
    len_out[syms[0]] = 1;
    return ORC_OK;
  }
  if ((double)n > ldexp(1.0, lmax)) return ORC_EINVAL;

  /* leaves sorted by (count, symbol): simple insertion sort */
  pm_item leaves[256];
  for (int i = 0; i < n; i++) {
    leaves[i].weight = h[syms[i]];
    leaves[i].leaf = 1;
    leaves[i].sym = syms[i];
    leaves[i].child = -1;
  }
  for (int i = 1; i < n; i++) {
    pm_item t = leaves[i];
    int j = i - 1;
    while (j >= 0 && (leaves[j].weight > t.weight ||
                      (leaves[j].weight == t.weight && leaves[j].sym > t.sym))) {
      leaves[j + 1] = leaves[j];
      j--;
    }
    leaves[j + 1] = t;
  }

  pm_item **lists = (pm_item **)calloc((size_t)lmax, sizeof(pm_item *));
  int *sizes = (int *)calloc((size_t)lmax, sizeof(int));
  if (!lists || !sizes) {
    free(lists);
    free(sizes);
    return ORC_EINVAL;
  }
  /* leaves of list lv: those whose cap reaches level lmax - lv */
  pm_item lv_leaves[256];
  lists[0] = (pm_item *)malloc(sizeof(pm_item) * (size_t)n);
  sizes[0] = 0;
  for (int i = 0; i < n; i++)
    if (cap[leaves[i].sym] >= lmax) lists[0][sizes[0]++] = leaves[i];
  for (int lv = 1; lv < lmax; lv++) {
    int nl = 0;
    for (int i = 0; i < n; i++)
      if (cap[leaves[i].sym] >= lmax - lv) lv_leaves[nl++] = leaves[i];
    int prev = sizes[lv - 1];
    int npk = prev / 2;
    pm_item *out = (pm_item *)malloc(sizeof(pm_item) * (size_t)(nl + npk));
    int i = 0, j = 0, k = 0;
    while (i < nl || j < npk) {
      int take_leaf;
      uint64_t pw = 0;
      if (j < npk) pw = lists[lv - 1][2 * j].weight + lists[lv - 1][2 * j + 1].weight;
      if (i >= nl) take_leaf = 0;
      else if (j >= npk) take_leaf = 1;
      else take_leaf = lv_leaves[i].weight <= pw;
      if (take_leaf) {
        out[k++] = lv_leaves[i++];
      } else {
        out[k].weight = pw;
        out[k].leaf = 0;
        out[k].sym = -1;
        out[k].child = 2 * j;
        k++;
        j++;
      }
    }
    lists[lv] = out;
    sizes[lv] = k;
  }
  int len[256];
  memset(len, 0, sizeof(len));
  int take = 2 * n - 2;
  if (take > sizes[lmax - 1]) {  /* the caps leave no complete code */
    for (int lv = 0; lv < lmax; lv++) free(lists[lv]);
    free(lists);
    free(sizes);
    return ORC_EINVAL;
  }
  for (int idx = 0; idx < take; idx++) pm_count(lists, lmax - 1, idx, len);
  for (int s = 0; s < 256; s++) len_out[s] = (uint8_t)len[s];
  for (int lv = 0; lv < lmax; lv++) free(lists[lv]);
  free(lists);
  free(sizes);
  return ORC_OK;
}

/* Optimal prefix-code lengths of at most lmax bits for the counts h. */
int orc_code_lengths(const uint64_t *h, int lmax, uint8_t *len_out) {
  int cap[256];
  for (int s = 0; s < 256; s++) cap[s] = lmax;
  return code_lengths_capped(h, lmax, cap, len_out);
}

/* As orc_code_lengths, with pair_fit > 0: every symbol whose count is at
 * least 1/pair_fit of all counts (count * pair_fit >= total) is capped at 6
 * bits, so that two such codes always fit a 12-bit window; the rest keep the
 * lmax limit.  If those caps leave no prefix code (more than 64 symbols that
 * common), the plain limit applies.  pair_fit = 0 is orc_code_lengths. */
int orc_code_lengths_pair_fit(const uint64_t *h, int lmax, uint32_t pair_fit, uint8_t *len_out) {
  if (pair_fit == 0) return orc_code_lengths(h, lmax, len_out);
  uint64_t total = 0;
  for (int s = 0; s < 256; s++) total += h[s];
  int cap[256];
  for (int s = 0; s < 256; s++) {
    cap[s] = lmax;
    if (lmax > 6 && h[s] > 0 && (double)h[s] * (double)pair_fit >= (double)total) cap[s] = 6;
  }
  if (code_lengths_capped(h, lmax, cap, len_out) == ORC_OK) return ORC_OK;
  return orc_code_lengths(h, lmax, len_out);
}

/* Lengths of the ranked unary code with an escape ("NWC -- Neural Weight
 * Compression", How it works, bullet "Prefix code instead of rANS"): the
 * present symbols are ranked by count (most frequent first, ties by
 * increasing symbol); rank r < R is written as r one bits and a zero (r + 1
 * bits); every other symbol is an escape: R one bits, then the symbol's index
 * among the escaped symbols in b = ceil(log2(number escaped)) bits, R + b
 * bits in all.  Our reading of the escape: an index rather than the raw
 * exponent byte, so that every code fits lmax bits (the decode table of the
 * format reads lmax <= 12 bits at a time) -- with the canonical code built
 * from these lengths, the escaped symbols of equal length take consecutive
 * code values in symbol order, i.e. exactly "prefix, then index".  R is the
 * value in 0 .. n - 1 with R + b <= lmax that minimises the total bits (the
 * smallest such R on a tie).  One present symbol gets length 1. */
int orc_code_lengths_unary(const uint64_t *h, int lmax, uint8_t *len_out) {
  int sym[256], n = 0;
  for (int v = 0; v < 256; v++) {
    len_out[v] = 0;
    if (h[v] > 0) sym[n++] = v;
  }
  if (n == 0 || lmax < 1) return ORC_EINVAL;
  if (n == 1) {
    len_out[sym[0]] = 1;
    return ORC_OK;
  }
  /* rank order: count descending, then symbol ascending (insertion sort) */
  for (int i = 1; i < n; i++) {
    int t = sym[i], j = i - 1;
    while (j >= 0 && (h[sym[j]] < h[t] || (h[sym[j]] == h[t] && sym[j] > t))) {
      sym[j + 1] = sym[j];
      j--;
    }
    sym[j + 1] = t;
  }
  int best_r = -1;
  double best_bits = 0.0;
  for (int R = 0; R < n; R++) {
    int rest = n - R, b = 0;
    while ((1 << b) < rest) b++;
    if (R + b > lmax || R + b == 0) continue;
    double bits = 0.0;
    for (int r = 0; r < n; r++) bits += (double)h[sym[r]] * (double)(r < R ? r + 1 : R + b);
    if (best_r < 0 || bits < best_bits) {
      best_r = R;
      best_bits = bits;
    }
  }
  if (best_r < 0) return ORC_EINVAL;
  int rest = n - best_r, b = 0;
  while ((1 << b) < rest) b++;
  for (int r = 0; r < n; r++) len_out[sym[r]] = (uint8_t)(r < best_r ? r + 1 : best_r + b);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Canonical codes  [RFC] 3.2.2                                        */
/* ------------------------------------------------------------------ */

/* Codes from lengths: count the codes of each length, give each length the
 * first code value after all shorter codes (doubled per extra bit), and hand
 * out consecutive values within a length in increasing symbol order.
 * Returns ORC_EINVAL if the lengths over-subscribe the code space or exceed
 * 15 bits. */
int orc_canonical_codes(const uint8_t *len, uint16_t *code) {
  int bl_count[16];
  int next_code[16];
  memset(bl_count, 0, sizeof(bl_count));
  for (int s = 0; s < 256; s++) {
    if (len[s] > 15) return ORC_EINVAL;
    if (len[s]) bl_count[len[s]]++;
  }
  /* Kraft check: sum 2^-len <= 1 */
  uint64_t kraft = 0;
  for (int l = 1; l <= 15; l++) kraft += (uint64_t)bl_count[l] << (15 - l);
  if (kraft > (1u << 15)) return ORC_EINVAL;
  int c = 0;
  bl_count[0] = 0;
  for (int bits = 1; bits <= 15; bits++) {
    c = (c + bl_count[bits - 1]) << 1;
    next_code[bits] = c;
  }
  for (int s = 0; s < 256; s++) {
    code[s] = 0;
    if (len[s]) code[s] = (uint16_t)(next_code[len[s]]++);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Bit I/O: LSB-first 32-bit words, codes sent most significant bit    */
/* first  [RFC] 3.1.1                                                  */
/* ------------------------------------------------------------------ */

static void put_bit(uint32_t *words, uint64_t pos, int bit) {
  if (bit) words[pos >> 5] |= (uint32_t)1u << (pos & 31);
}

static int get_bit(const uint32_t *words, uint64_t pos) {
  return (int)((words[pos >> 5] >> (pos & 31)) & 1u);
}

static void put_code(uint32_t *words, uint64_t *pos, uint16_t code, int len) {
  for (int i = len - 1; i >= 0; i--) {
    put_bit(words, *pos, (code >> i) & 1);
    (*pos)++;
  }
}

/* Canonical decoding tables (bit-serial, textbook): per length the number of
 * codes, and the symbols listed in (length, symbol) order. */
typedef struct {
  int count[16];
  int sorted[256];
  int maxlen;
} orc_dec;

static int dec_init(orc_dec *d, const uint8_t *len) {
  memset(d, 0, sizeof(*d));
  int k = 0;
  for (int l = 1; l <= 15; l++)
    for (int s = 0; s < 256; s++)
      if (len[s] == l) {
        d->sorted[k++] = s;
        d->count[l]++;
        if (l > d->maxlen) d->maxlen = l;
      }
  return k;
}

/* Decode one symbol reading bits through `bit(i)` for i = 0.. < avail.
 * Returns the symbol and sets *used, or -1 if no code completes within avail
 * bits or maxlen bits. */
static int dec_symbol(const orc_dec *d, const uint32_t *words, uint64_t pos,
                      uint64_t avail, int *used) {
  int code = 0, first = 0, index = 0;
  for (int l = 1; l <= d->maxlen; l++) {
    if ((uint64_t)l > avail) return -1;
    code |= get_bit(words, pos + (uint64_t)(l - 1));
    int cnt = d->count[l];
    if (code - first < cnt) {
      *used = l;
      return d->sorted[index + code - first];
    }
    index += cnt;
    first += cnt;
    first <<= 1;
    code <<= 1;
  }
  return -1;
}

/* ------------------------------------------------------------------ */
/* Decode table (table kind 1): one 32-bit entry per 12-bit window      */
/* ------------------------------------------------------------------ */

/* Window w holds stream bits p..p+11 with bit p in bit 0.  The entry decodes
 * the first code in the window and, when a second complete code fits in the
 * remaining bits, the second one too:
 *   two codes : (l0+l1) | l0<<16 | s0<<7 | s1<<23
 *   one code  :  l0     | l0<<16 | s0<<7 | 1<<31
 *   no code   :  0
 * (l = code length in bits, s = exponent symbol). */
int orc_decode_table(const uint8_t *len, uint32_t *table) {
  orc_dec d;
  dec_init(&d, len);
  for (uint32_t w = 0; w < ORC_TABLE_ENTRIES; w++) {
    uint32_t win = w;
    int l0 = 0, l1 = 0;
    int s0 = dec_symbol(&d, &win, 0, ORC_TABLE_BITS, &l0);
    if (s0 < 0) {
      table[w] = 0;
      continue;
    }
    int s1 = dec_symbol(&d, &win, (uint64_t)l0, ORC_TABLE_BITS - (uint64_t)l0, &l1);
    if (s1 >= 0) {
      table[w] = (uint32_t)(l0 + l1) | ((uint32_t)l0 << 16) | ((uint32_t)s0 << 7) |
                 ((uint32_t)s1 << 23);
    } else {
      table[w] = (uint32_t)l0 | ((uint32_t)l0 << 16) | ((uint32_t)s0 << 7) |
                 (1u << 31);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Blob geometry                                                        */
/* ------------------------------------------------------------------ */

typedef struct {
  uint64_t rows, cols;
  uint32_t tr, tc, s, lmax;
  uint32_t table_kind, flags;
  uint64_t raw_ld, n_tiles, n_chunks, stream_words;
  uint64_t off_code_len, off_table, off_tile_words, off_chunk_bits, off_raw, off_stream;
  uint64_t total_bytes;
  uint64_t n_tr, n_tc;
  uint32_t v;
} orc_geom;

static uint64_t up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

static int geom_check(uint64_t rows, uint64_t cols, uint32_t tr, uint32_t tc,
                      uint32_t s, uint32_t lmax) {
  if (rows < 1 || cols < 1) return ORC_EINVAL;
  if (tr < 1 || tc < 1 || s < 1 || tc % s != 0) return ORC_EINVAL;
  if (lmax < 6 || lmax > 12) return ORC_EINVAL;
  uint64_t v = tc / s;
  if ((uint64_t)tr * v * lmax > 65535u) return ORC_EINVAL;
  return ORC_OK;
}

/* Section offsets for a stream of `stream_words` words. */
static void geom_layout(orc_geom *g, uint64_t stream_words) {
  g->v = g->tc / g->s;
  g->n_tr = (g->rows + g->tr - 1) / g->tr;
  g->n_tc = (g->cols + g->tc - 1) / g->tc;
  g->n_tiles = g->n_tr * g->n_tc;
  g->n_chunks = g->n_tiles * g->s;
  g->raw_ld = up(g->cols, 16);
  g->stream_words = stream_words;
  g->off_code_len = ORC_HEADER_BYTES;
  g->off_table = g->off_code_len + 256;
  g->off_tile_words = g->off_table + 4 * ORC_TABLE_ENTRIES;
  g->off_chunk_bits = up(g->off_tile_words + 4 * (g->n_tiles + 1), 256);
  g->off_raw = up(g->off_chunk_bits + 2 * g->n_chunks, 256);
  g->off_stream = up(g->off_raw + g->raw_ld * g->rows, 256);
  g->total_bytes = up(g->off_stream + 4 * stream_words + 16, 256);
}

static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) {
  for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t *p, uint64_t v) {
  for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
static uint64_t get_u64(const uint8_t *p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

/* Chunk c of tile (ti, tj) covers rows [r0, r1) and columns [c0, c1). */
static void chunk_box(const orc_geom *g, uint64_t ti, uint64_t tj, uint32_t c,
                      uint64_t *r0, uint64_t *r1, uint64_t *c0, uint64_t *c1) {
  *r0 = ti * g->tr;
  *r1 = *r0 + g->tr < g->rows ? *r0 + g->tr : g->rows;
  uint64_t tile_c1 = tj * g->tc + g->tc < g->cols ? tj * g->tc + g->tc : g->cols;
  *c0 = tj * g->tc + (uint64_t)c * g->v;
  *c1 = *c0 + g->v < tile_c1 ? *c0 + g->v : tile_c1;
  if (*c0 >= tile_c1) *c0 = *c1 = tile_c1; /* chunk lies beyond the matrix edge: empty */
}

/* Upper bound of the blob size for any data of this shape. */
int orc_encode_bound(uint64_t rows, uint64_t cols, uint32_t tr, uint32_t tc, uint32_t s,
                     uint32_t lmax, uint64_t *bound) {
  int rc = geom_check(rows, cols, tr, tc, s, lmax);
  if (rc) return rc;
  orc_geom g;
  memset(&g, 0, sizeof(g));
  g.rows = rows; g.cols = cols; g.tr = tr; g.tc = tc; g.s = s; g.lmax = lmax;
  geom_layout(&g, 0);
  /* every code <= lmax bits, plus one word of padding per tile */
  uint64_t words = (rows * cols * lmax + 31) / 32 + g.n_tiles;
  geom_layout(&g, words);
  *bound = g.total_bytes;
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Encoder                                                              */
/* ------------------------------------------------------------------ */

/* w: rows x cols BF16 patterns with row stride ld (elements).
 * Steps: split the planes, count exponents over the whole tensor, build the
 * length-limited code and its canonical codes, then for each tile in row-major
 * tile order and each chunk in order write the codes of the chunk's exponents
 * in row-major order; record each chunk's bit length, start every tile on a
 * 32-bit word boundary, and store the raw bytes row-major. */
int orc_encode_family(const uint16_t *w, uint64_t rows, uint64_t cols, uint64_t ld, uint32_t tr,
                      uint32_t tc, uint32_t s, uint32_t lmax, uint32_t pair_fit, uint32_t family,
                      uint8_t *blob, uint64_t cap, uint64_t *used);

/* Encode with the length-limited Huffman code (family 0). */
int orc_encode(const uint16_t *w, uint64_t rows, uint64_t cols, uint64_t ld, uint32_t tr,
               uint32_t tc, uint32_t s, uint32_t lmax, uint32_t pair_fit, uint8_t *blob,
               uint64_t cap, uint64_t *used) {
  return orc_encode_family(w, rows, cols, ld, tr, tc, s, lmax, pair_fit, 0, blob, cap, used);
}

/* Encode with the code family `family`: 0 = length-limited Huffman (with the
 * pair_fit caps), 1 = ranked unary code with an escape (pair_fit unused). */
int orc_encode_family(const uint16_t *w, uint64_t rows, uint64_t cols, uint64_t ld, uint32_t tr,
                      uint32_t tc, uint32_t s, uint32_t lmax, uint32_t pair_fit, uint32_t family,
                      uint8_t *blob, uint64_t cap, uint64_t *used) {
  if (family > 1) return ORC_EINVAL;
  int rc = geom_check(rows, cols, tr, tc, s, lmax);
  if (rc) return rc;
  if (ld < cols || !w || !blob || !used) return ORC_EINVAL;

  uint64_t n = rows * cols;
  uint8_t *e = (uint8_t *)malloc(n);
  uint8_t *r = (uint8_t *)malloc(n);
  if (!e || !r) { free(e); free(r); return ORC_EINVAL; }
  for (uint64_t i = 0; i < rows; i++) orc_split(w + i * ld, cols, e + i * cols, r + i * cols);

  uint64_t h[256];
  orc_histogram(e, n, h);
  uint8_t len[256];
  uint16_t code[256];
  rc = family == 1 ? orc_code_lengths_unary(h, (int)lmax, len) : orc_code_lengths_pair_fit(h, (int)lmax, pair_fit, len);
  if (!rc) rc = orc_canonical_codes(len, code);
  if (rc) { free(e); free(r); return rc; }

  orc_geom g;
  memset(&g, 0, sizeof(g));
  g.rows = rows; g.cols = cols; g.tr = tr; g.tc = tc; g.s = s; g.lmax = lmax;
  g.table_kind = 1;
  geom_layout(&g, 0);

  /* first pass into a scratch word array sized for the worst case */
  uint64_t max_words = (n * lmax + 31) / 32 + g.n_tiles + 1;
  uint32_t *words = (uint32_t *)calloc(max_words, 4);
  uint32_t *tile_words = (uint32_t *)calloc(g.n_tiles + 1, 4);
  uint16_t *chunk_bits = (uint16_t *)calloc(g.n_chunks ? g.n_chunks : 1, 2);
  if (!words || !tile_words || !chunk_bits) {
    free(e); free(r); free(words); free(tile_words); free(chunk_bits);
    return ORC_EINVAL;
  }
  uint64_t pos = 0;
  for (uint64_t ti = 0; ti < g.n_tr; ti++) {
    for (uint64_t tj = 0; tj < g.n_tc; tj++) {
      uint64_t t = ti * g.n_tc + tj;
      tile_words[t] = (uint32_t)(pos / 32);
      for (uint32_t c = 0; c < s; c++) {
        uint64_t r0, r1, c0, c1;
        chunk_box(&g, ti, tj, c, &r0, &r1, &c0, &c1);
        uint64_t start = pos;
        for (uint64_t i = r0; i < r1; i++)
          for (uint64_t j = c0; j < c1; j++) {
            uint8_t sym = e[i * cols + j];
            put_code(words, &pos, code[sym], len[sym]);
          }
        chunk_bits[t * s + c] = (uint16_t)(pos - start);
      }
      pos = up(pos, 32);
    }
  }
  tile_words[g.n_tiles] = (uint32_t)(pos / 32);
  geom_layout(&g, pos / 32);

  if (g.total_bytes > cap) {
    *used = g.total_bytes;
    free(e); free(r); free(words); free(tile_words); free(chunk_bits);
    return ORC_ESMALL;
  }
  memset(blob, 0, g.total_bytes);
  put_u32(blob + 0, ORC_MAGIC);
  put_u16(blob + 4, ORC_VERSION);
  put_u16(blob + 6, ORC_HEADER_BYTES);
  put_u64(blob + 8, rows);
  put_u64(blob + 16, cols);
  put_u32(blob + 24, tr);
  put_u32(blob + 28, tc);
  put_u32(blob + 32, s);
  put_u32(blob + 36, lmax);
  put_u32(blob + 40, g.table_kind);
  put_u32(blob + 44, 0);
  put_u64(blob + 48, g.raw_ld);
  put_u64(blob + 56, g.n_tiles);
  put_u64(blob + 64, g.n_chunks);
  put_u64(blob + 72, g.stream_words);
  put_u64(blob + 80, g.off_code_len);
  put_u64(blob + 88, g.off_table);
  put_u64(blob + 96, g.off_tile_words);
  put_u64(blob + 104, g.off_chunk_bits);
  put_u64(blob + 112, g.off_raw);
  put_u64(blob + 120, g.off_stream);
  put_u64(blob + 128, g.total_bytes);
  memcpy(blob + g.off_code_len, len, 256);
  uint32_t table[ORC_TABLE_ENTRIES];
  orc_decode_table(len, table);
  for (uint32_t i = 0; i < ORC_TABLE_ENTRIES; i++) put_u32(blob + g.off_table + 4 * i, table[i]);
  for (uint64_t t = 0; t <= g.n_tiles; t++) put_u32(blob + g.off_tile_words + 4 * t, tile_words[t]);
  for (uint64_t c = 0; c < g.n_chunks; c++) put_u16(blob + g.off_chunk_bits + 2 * c, chunk_bits[c]);
  for (uint64_t i = 0; i < rows; i++)
    for (uint64_t j = 0; j < cols; j++) blob[g.off_raw + i * g.raw_ld + j] = r[i * cols + j];
  for (uint64_t k = 0; k < g.stream_words; k++) put_u32(blob + g.off_stream + 4 * k, words[k]);
  *used = g.total_bytes;
  free(e); free(r); free(words); free(tile_words); free(chunk_bits);
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Parser and decoder                                                   */
/* ------------------------------------------------------------------ */

typedef struct {
  orc_geom g;
  const uint8_t *len;
  const uint8_t *tile_words;
  const uint8_t *chunk_bits;
  const uint8_t *raw;
  uint32_t *stream; /* private aligned copy */
  orc_dec dec;
} orc_view;

static int parse(const uint8_t *blob, uint64_t bytes, orc_view *v) {
  memset(v, 0, sizeof(*v));
  if (!blob || bytes < ORC_HEADER_BYTES + 256) return ORC_EFORMAT;
  if (get_u32(blob) != ORC_MAGIC || get_u16(blob + 4) != ORC_VERSION ||
      get_u16(blob + 6) != ORC_HEADER_BYTES)
    return ORC_EFORMAT;
  orc_geom *g = &v->g;
  g->rows = get_u64(blob + 8);
  g->cols = get_u64(blob + 16);
  g->tr = get_u32(blob + 24);
  g->tc = get_u32(blob + 28);
  g->s = get_u32(blob + 32);
  g->lmax = get_u32(blob + 36);
  g->table_kind = get_u32(blob + 40);
  g->flags = get_u32(blob + 44);
  if (geom_check(g->rows, g->cols, g->tr, g->tc, g->s, g->lmax)) return ORC_EFORMAT;
  if (g->table_kind != 1 || g->flags != 0) return ORC_EFORMAT;
  if (g->rows > (1ull << 32) || g->cols > (1ull << 32)) return ORC_EFORMAT;
  uint64_t sw = get_u64(blob + 72);
  if (sw > 0xFFFFFFFFull) return ORC_EFORMAT;
  orc_geom want = *g;
  geom_layout(&want, sw);
  if (get_u64(blob + 48) != want.raw_ld || get_u64(blob + 56) != want.n_tiles ||
      get_u64(blob + 64) != want.n_chunks || get_u64(blob + 80) != want.off_code_len ||
      get_u64(blob + 88) != want.off_table || get_u64(blob + 96) != want.off_tile_words ||
      get_u64(blob + 104) != want.off_chunk_bits || get_u64(blob + 112) != want.off_raw ||
      get_u64(blob + 120) != want.off_stream || get_u64(blob + 128) != want.total_bytes)
    return ORC_EFORMAT;
  if (want.total_bytes > bytes) return ORC_EFORMAT;
  *g = want;
  v->len = blob + g->off_code_len;
  v->tile_words = blob + g->off_tile_words;
  v->chunk_bits = blob + g->off_chunk_bits;
  v->raw = blob + g->off_raw;
  /* the lengths must form a prefix code with every length <= lmax */
  uint16_t code[256];
  for (int s = 0; s < 256; s++)
    if (v->len[s] > g->lmax) return ORC_EFORMAT;
  if (orc_canonical_codes(v->len, code)) return ORC_EFORMAT;
  if (dec_init(&v->dec, v->len) == 0) return ORC_EFORMAT;
  /* the stored decode table must be the one the lengths define */
  uint32_t table[ORC_TABLE_ENTRIES];
  orc_decode_table(v->len, table);
  for (uint32_t i = 0; i < ORC_TABLE_ENTRIES; i++)
    if (get_u32(blob + g->off_table + 4 * i) != table[i]) return ORC_EFORMAT;
  /* tile starts: each tile begins at the word after the previous tile's bits */
  if (get_u32(v->tile_words) != 0) return ORC_EFORMAT;
  for (uint64_t t = 0; t < g->n_tiles; t++) {
    uint64_t bits = 0;
    for (uint32_t c = 0; c < g->s; c++) bits += get_u16(v->chunk_bits + 2 * (t * g->s + c));
    uint64_t a = get_u32(v->tile_words + 4 * t), b = get_u32(v->tile_words + 4 * (t + 1));
    if (b != a + (bits + 31) / 32) return ORC_EFORMAT;
  }
  if (get_u32(v->tile_words + 4 * g->n_tiles) != sw) return ORC_EFORMAT;
  v->stream = (uint32_t *)calloc(sw + 4, 4);
  if (!v->stream) return ORC_EINVAL;
  for (uint64_t k = 0; k < sw; k++) v->stream[k] = get_u32(blob + g->off_stream + 4 * k);
  return ORC_OK;
}

/* Decode chunk c of tile t into out (row-major symbols of the chunk), checking
 * that exactly the recorded number of bits is consumed.  Returns the number
 * of symbols or a negative error. */
static int64_t decode_chunk(const orc_view *v, uint64_t t, uint32_t c, uint8_t *out) {
  const orc_geom *g = &v->g;
  uint64_t ti = t / g->n_tc, tj = t % g->n_tc;
  uint64_t r0, r1, c0, c1;
  chunk_box(g, ti, tj, c, &r0, &r1, &c0, &c1);
  uint64_t start = (uint64_t)get_u32(v->tile_words + 4 * t) * 32;
  for (uint32_t k = 0; k < c; k++) start += get_u16(v->chunk_bits + 2 * (t * g->s + k));
  uint64_t nbits = get_u16(v->chunk_bits + 2 * (t * g->s + c));
  uint64_t end = start + nbits;
  uint64_t limit = g->stream_words * 32;
  if (end > limit) return ORC_EFORMAT;
  uint64_t pos = start;
  int64_t k = 0;
  for (uint64_t i = r0; i < r1; i++)
    for (uint64_t j = c0; j < c1; j++) {
      int used = 0;
      int sym = dec_symbol(&v->dec, v->stream, pos, end - pos, &used);
      if (sym < 0) return ORC_EFORMAT;
      pos += (uint64_t)used;
      out[k++] = (uint8_t)sym;
    }
  if (pos != end) return ORC_EFORMAT;
  return k;
}

/* Reconstruct the BF16 matrix into w (row stride ld elements). */
int orc_decode(const uint8_t *blob, uint64_t bytes, uint16_t *w, uint64_t ld) {
  orc_view v;
  int rc = parse(blob, bytes, &v);
  if (rc) { free(v.stream); return rc; }
  const orc_geom *g = &v.g;
  if (!w || ld < g->cols) { free(v.stream); return ORC_EINVAL; }
  uint8_t *syms = (uint8_t *)malloc((size_t)g->tr * g->v + 1);
  for (uint64_t t = 0; t < g->n_tiles; t++) {
    uint64_t ti = t / g->n_tc, tj = t % g->n_tc;
    for (uint32_t c = 0; c < g->s; c++) {
      int64_t k = decode_chunk(&v, t, c, syms);
      if (k < 0) { free(syms); free(v.stream); return (int)k; }
      uint64_t r0, r1, c0, c1;
      chunk_box(g, ti, tj, c, &r0, &r1, &c0, &c1);
      int64_t q = 0;
      for (uint64_t i = r0; i < r1; i++)
        for (uint64_t j = c0; j < c1; j++) {
          uint8_t rb = v.raw[i * g->raw_ld + j];
          orc_join(&syms[q++], &rb, 1, &w[i * ld + j]);
        }
    }
  }
  free(syms);
  free(v.stream);
  return ORC_OK;
}

/* Decode one chunk alone (symbols in row-major chunk order). */
int64_t orc_decode_chunk(const uint8_t *blob, uint64_t bytes, uint64_t tile, uint32_t c,
                         uint8_t *out, uint64_t cap) {
  orc_view v;
  int rc = parse(blob, bytes, &v);
  if (rc) { free(v.stream); return rc; }
  if (tile >= v.g.n_tiles || c >= v.g.s || cap < (uint64_t)v.g.tr * v.g.v) {
    free(v.stream);
    return ORC_EINVAL;
  }
  int64_t k = decode_chunk(&v, tile, c, out);
  free(v.stream);
  return k;
}

/* Validate a blob: parse every section and decode every chunk, checking
 * that each one consumes exactly its recorded number of bits.  Returns ORC_OK
 * or a negative error. */
int orc_validate(const uint8_t *blob, uint64_t bytes) {
  orc_view v;
  int rc = parse(blob, bytes, &v);
  if (rc) { free(v.stream); return rc; }
  uint8_t *syms = (uint8_t *)malloc((size_t)v.g.tr * v.g.v + 1);
  for (uint64_t t = 0; t < v.g.n_tiles && !rc; t++)
    for (uint32_t c = 0; c < v.g.s && !rc; c++) {
      int64_t k = decode_chunk(&v, t, c, syms);
      if (k < 0) rc = (int)k;
    }
  free(syms);
  free(v.stream);
  return rc;
}

/* ------------------------------------------------------------------ */
/* FP64 products                                                        */
/* ------------------------------------------------------------------ */

/* y[n] = sum_k W[n,k] x[k] and a[n] = sum_k |W[n,k] x[k]|, in FP64, adding in
 * increasing k.  W is rows x cols (nn.Linear [out, in]) with row stride ld. */
void orc_gemv(const uint16_t *w, uint64_t rows, uint64_t cols, uint64_t ld,
              const uint16_t *x, double *y, double *a) {
  for (uint64_t n = 0; n < rows; n++) {
    double acc = 0.0, mag = 0.0;
    for (uint64_t k = 0; k < cols; k++) {
      double p = orc_bf16_value(w[n * ld + k]) * orc_bf16_value(x[k]);
      acc += p;
      mag += fabs(p);
    }
    y[n] = acc;
    if (a) a[n] = mag;
  }
}

/* Y[b,n] = sum_k X[b,k] W[n,k] for b < batch (X row stride ldx), same order. */
void orc_gemm(const uint16_t *w, uint64_t rows, uint64_t cols, uint64_t ld,
              const uint16_t *X, uint64_t batch, uint64_t ldx, double *Y, double *A) {
  for (uint64_t b = 0; b < batch; b++)
    orc_gemv(w, rows, cols, ld, X + b * ldx, Y + b * rows, A ? A + b * rows : NULL);
}
