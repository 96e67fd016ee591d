/*
 * nwc.h -- C ABI of libnwc: lossless BF16 weight compression decoded inside
 * the matrix-vector kernel, for AMD Instinct MI355X (gfx950).
 *
 * The method (pages, cited by title and section):
 *  - "NWC -- Neural Weight Compression" (PyPI description of
 *    neural-weight-compression 0.9.0), "How it works": a BF16 weight splits
 *    into a near-random byte stored raw and an exponent byte that is entropy
 *    coded (bullet "Byte planes"); the matrix-vector kernel decodes in
 *    registers so no decompressed weight reaches memory (bullet "Fused
 *    kernel"); dequantization runs on the same decoder (bullet
 *    "Dequantization and embedding lookup"); the encoder needs only the
 *    weights ("Status and limitations").
 *  - "Unweight: how we compressed an LLM 22% without sacrificing quality"
 *    (Techlist.io summary), "Compressing BF16 Weights": Huffman code on the
 *    exponent, sign and mantissa unchanged; "Direct GPU Decompression":
 *    weights stay compressed in HBM and are decompressed on chip right
 *    before the product.
 *
 * Data format: one self-describing, position-independent blob per matrix W
 * [rows, cols] (nn.Linear [out, in], row-major BF16).  The raw byte of a
 * weight holds its sign (bit 7) and 7 fraction bits; the 8-bit exponent is
 * coded with one canonical Huffman code per tensor, length-limited to
 * max_code_len bits, in tiles of tile_rows x tile_cols split into
 * chunks_per_tile column-strip chunks; per-tile word offsets and per-chunk bit
 * lengths let every tile (and chunk) decode on its own.
 *
 * Conventions for every function:
 *  - Every call returns an nwc_status; nothing throws across the ABI and there
 *    is no global error state.  Host-side validation (null pointers, sizes,
 *    alignment, header consistency) happens before any device work: on an
 *    error nothing is enqueued.
 *  - The caller owns all memory (host blob, device blob, inputs, outputs,
 *    workspace).  The library never allocates device memory, never frees and
 *    never synchronizes a stream; device calls only enqueue work on `stream`
 *    (a hipStream_t, 0 = the null stream) and every buffer must stay valid
 *    until that work completes.
 *  - BF16 data is passed as uint16_t bit patterns.
 *  - Device pointers: blob 256-byte aligned; x, y, X, Y, W 16-byte aligned;
 *    leading dimensions in elements, multiples of 8 for 16-byte rows.
 *  - The device blob must hold the same bytes that were passed to
 *    nwc_inspect.  Corrupted device data is not detected: kernels clamp every
 *    read to the blob, so it yields wrong numbers, never a memory fault.
 *  - Results are deterministic: a fixed summation order, no floating-point
 *    atomics, so repeated calls give bitwise-identical outputs.
 *  - Functions are reentrant; the library holds no mutable global state,
 *    except nwc_gemv_noalloc's per-device static scratch and the wait bound
 *    of the matrix-core skinny GEMM that the test hook nwc_set_wait_limit
 *    sets (see there).
 */
#ifndef NWC_H
#define NWC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NWC_OK = 0,
  NWC_ERR_INVALID_ARG = -1,      /* null pointer, bad size, bad parameter */
  NWC_ERR_BUFFER_TOO_SMALL = -2, /* output or workspace capacity too small */
  NWC_ERR_BAD_FORMAT = -3,       /* blob fails validation */
  NWC_ERR_UNSUPPORTED = -4,      /* valid request the library cannot run */
  NWC_ERR_ALIGNMENT = -5,        /* pointer or leading dimension misaligned */
  NWC_ERR_HIP = -6,              /* a HIP runtime call or launch failed */
  NWC_ERR_SCRATCH_LIMIT = -7     /* needs more than the static scratch holds */
} nwc_status;

typedef enum {
  NWC_OUT_BF16 = 0, /* round-to-nearest-even from the FP32 accumulator */
  NWC_OUT_F32 = 1
} nwc_out_type;

/* Encoding parameters; a zero field takes the default in brackets.
 * Constraints: tile_cols % chunks_per_tile == 0, 6 <= max_code_len <= 12,
 * tile_rows * (tile_cols / chunks_per_tile) * max_code_len <= 65535.
 * A limit of 8 codes any tensor (all 256 exponent values fit); below 8 the
 * tensor may hold at most 2^max_code_len distinct exponent values.  At 6, two
 * codes always fit one 12-bit table lookup, and the fused kernels decode
 * every pair with one lookup, for about 0.4 bit per weight more than at 8.
 * pair_fit trades a little size for fewer decode steps that need a second
 * lookup (two codes longer than 12 bits together): with the common exponents
 * capped at 6 bits, only pairs involving a rare exponent can overflow.  At
 * the default (1024) it costs 0.3-0.6% of the blob on the synthetic workloads.
 * The blob stores only the code lengths, so decoders need no such flag. */
typedef struct {
  uint32_t tile_rows;       /* TR rows per tile [8] */
  uint32_t tile_cols;       /* TC columns per tile [512] */
  uint32_t chunks_per_tile; /* S column-strip chunks per tile [64] */
  uint32_t max_code_len;    /* L, longest code in bits [8] */
  uint32_t pair_fit;        /* K: every exponent value held by at least 1/K of
                               the weights gets a code of at most 6 bits, the
                               rest keep the limit L; 1 turns it off (unless
                               more than 64 values are that common, then the
                               plain limit applies) [1024] */
  uint32_t code_family;     /* 0: the length-limited Huffman code above [0];
                               1: the ranked unary code with an escape ("NWC
                               -- Neural Weight Compression", How it works,
                               bullet "Prefix code instead of rANS"):
                               exponents ranked by count, rank r < R coded
                               as r one bits and a zero, the rest as R one
                               bits and an index among them, R chosen for the
                               fewest bits within L (pair_fit unused).  Both
                               are canonical prefix codes of at most L bits:
                               the blob stores only the lengths and every
                               decoder reads both alike. */
} nwc_params;

/* Everything a device call needs, read from a validated blob. */
typedef struct {
  uint64_t rows, cols;             /* N, K */
  uint64_t blob_bytes;             /* total blob size */
  uint32_t tile_rows, tile_cols, chunks_per_tile, max_code_len;
  uint64_t n_tiles, n_chunks;
  uint64_t raw_ld;                 /* raw-plane row stride in bytes */
  uint64_t stream_words;           /* 32-bit words of exponent codes */
  uint64_t off_code_len, off_table, off_tile_words, off_chunk_bits, off_raw, off_stream;
  uint32_t max_tile_words;         /* largest single-tile stream, in words */
  uint32_t n_symbols;              /* distinct exponent values present */
  uint32_t max_chunk_bits;         /* longest single chunk, in bits */
  uint32_t reserved;               /* 0 */
  uint64_t payload_bits;           /* sum of all chunk lengths */
  uint8_t code_len[256];           /* code length per exponent value */
} nwc_info;

/* Human-readable name of a status code (static string, never NULL). */
const char *nwc_status_str(nwc_status s);

/* Upper bound on the blob size of any rows x cols matrix with parameters p
 * (NULL = defaults).  Host only, synchronous. */
nwc_status nwc_encode_bound(uint64_t rows, uint64_t cols, const nwc_params *p,
                            size_t *max_bytes);

/* Encode W (host, rows x cols BF16 patterns, row stride ld >= cols elements)
 * into blob (host, capacity cap bytes); *used receives the blob size.
 * Steps (pages above): split each weight into raw byte and exponent, count
 * exponents over the tensor, build optimal code lengths <= max_code_len by
 * package-merge and canonical codes from them, write each tile's chunks in
 * order, record offsets, and write the decode table.  A pure function of
 * (W, shape, p): identical inputs give identical bytes.  Multithreaded on the
 * host; no device work.  Errors: INVALID_ARG (bad shape/params/NULL, or
 * more distinct exponent values than max_code_len can code), BUFFER_TOO_SMALL
 * (then *used holds the needed size). */
nwc_status nwc_encode(const uint16_t *w, uint64_t rows, uint64_t cols, uint64_t ld,
                      const nwc_params *p, void *blob, size_t cap, size_t *used);

/* Parse and validate a host blob and fill *info.  Checks the header, section
 * layout, that the code lengths form a prefix code <= max_code_len, that the
 * decode table matches the lengths, and that tile offsets agree with the
 * chunk lengths.  Does not decode the stream.  Host only.
 * Errors: INVALID_ARG (NULL), BAD_FORMAT. */
nwc_status nwc_inspect(const void *blob, size_t bytes, nwc_info *info);

/* Standalone decode (pages: "Dequantization and embedding lookup"): write
 * the exact original BF16 bits of W into w_dev (device, rows x cols, row
 * stride ld >= cols elements).  Reads the compressed bytes once and writes
 * 2 bytes per weight.  Async on `stream`.
 * Errors: INVALID_ARG, ALIGNMENT (w_dev not 16-byte aligned or ld % 8), HIP. */
nwc_status nwc_decode(const nwc_info *info, const void *blob_dev, uint16_t *w_dev,
                      uint64_t ld, void *stream);

/* Workspace bytes needed by nwc_gemv (batch = 1) or nwc_gemm_skinny
 * (batch 2..32) for this blob.
 *  - Fused batch-1 path (default geometry, cols % 8 == 0): one 64-bit slot
 *    per (tile, row), rounded up to 256 bytes.  The kernel splits the tiles
 *    evenly over the GPU, so a row block can be shared by several
 *    workgroups; their partial sums meet in these slots.  The workspace
 *    must be zero-filled before its first use; every call leaves it
 *    zero-filled.
 *  - Fused skinny path (tile_rows 8 or 16 and batch 2..16, or tile_rows 8
 *    and batch 5..32): 0 (ws may be NULL).
 *  - Otherwise FP32 partial sums, one per (column tile, batch row, output
 *    row), for the generic path (any geometry), which runs a second reduction
 *    kernel; contents need not be initialised. */
nwc_status nwc_workspace_size(const nwc_info *info, int batch, size_t *bytes);

/* Fused decode-GEMV (pages: "Fused kernel"; Unweight "Direct GPU
 * Decompression"): y = W x with x (device, cols BF16, 16-byte aligned) and y
 * (device, rows entries of y_type).  Weights are decoded in registers and
 * LDS and never written to memory; FP32 accumulation, each output row's
 * partial sums added in an order fixed by the blob's shape, the launch's
 * other matrices and the GPU, so repeated calls give bitwise-identical y.
 * Each y entry is written once.  ws is a device workspace of at
 * least nwc_workspace_size(info, 1) bytes, 256-byte aligned, used as that
 * function describes (zero-filled before first use on the fused path).
 * Calls that share a workspace must not run concurrently (same stream, or
 * ordered by events).  x and y must not alias.  Async.
 * Errors: INVALID_ARG, BUFFER_TOO_SMALL (ws), ALIGNMENT, HIP; UNSUPPORTED
 * also for a fused-path blob of 2^32 tiles or more or of 65536 column tiles
 * or more (cols >= 2^25), whose tile arithmetic the kernel does not cover. */
nwc_status nwc_gemv(const nwc_info *info, const void *blob_dev, const uint16_t *x_dev,
                    void *y_dev, nwc_out_type y_type, void *ws, size_t ws_bytes,
                    void *stream);

/* nwc_gemv without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same fused kernel and launch as nwc_gemv, with its
 * exchange slots in a static device array of the library, `scratch`
 * (nwc_noalloc_scratch_bytes: 16 MiB), that each GPU the library runs on
 * holds until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); it clears the slots it needs with a small
 * kernel on `stream`, then runs the product, so y has the same bits as
 * nwc_gemv's.  The first call on a device looks the array's address up.
 * Only the fused path: default chunk geometry (64 chunks of 8 columns),
 * tile_rows 4, 8, 16 or 32, cols % 8 == 0.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (different streams, or
 * different host threads) race and give wrong results; order them on one
 * stream or with events.  Async.
 * Errors: as nwc_gemv, plus UNSUPPORTED (another geometry) and SCRATCH_LIMIT
 * (nwc_workspace_size(info, 1) above the scratch size; the LM head of
 * 128256 x 4096 at 8-row tiles needs 7.8 MiB). */
nwc_status nwc_noalloc_scratch_bytes(size_t *bytes);
nwc_status nwc_gemv_noalloc(const nwc_info *info, const void *blob_dev, const uint16_t *x_dev,
                            void *y_dev, nwc_out_type y_type, void *stream);

/* Several independent fused decode-GEMVs in one launch (count <= 8)
 * ("Unweight: how we compressed an LLM 22% without sacrificing quality",
 * Direct GPU Decompression: weights decompressed on chip right before the
 * product, with the execution strategy chosen per weight matrix and batch;
 * The GPU Memory Bottleneck: decompression must overlap the product or token
 * generation slows down):
 * y_i = W_i x_i with blob i described by infos[i] and stored at blobs_dev[i],
 * x_dev[i] / y_dev[i] as for nwc_gemv, all outputs of y_type.  For the GEMVs
 * of one decode step that need no result of each other (q/k/v from the same
 * activations, gate/up), one launch keeps the whole GPU busy where separate
 * small launches each pay a start-up and a tail.  Every blob must be on the
 * fused batch-1 path and all must share tile_rows.  ws (256-byte aligned,
 * zero-filled before first use, left zero-filled) holds the workspaces of
 * all blobs back to back: at least the sum over i of
 * nwc_workspace_size(&infos[i], 1).  Each y_i meets nwc_gemv's accuracy;
 * its bits may differ from a single call's (the tiles are shared out over
 * the whole launch), and repeating the same batched call repeats them.
 * Same concurrency rule as nwc_gemv.  Async.
 * Errors: INVALID_ARG, BUFFER_TOO_SMALL (ws), UNSUPPORTED, ALIGNMENT, HIP. */
nwc_status nwc_gemv_batched(int count, const nwc_info *infos, const void *const *blobs_dev,
                            const uint16_t *const *x_dev, void *const *y_dev,
                            nwc_out_type y_type, void *ws, size_t ws_bytes, void *stream);

/* Several independent standalone decodes in one launch (count <= 8)
 * ("NWC -- Neural Weight Compression", How it works, bullet
 * "Dequantization and embedding lookup": dequantization runs on the same
 * decoder as the fused product; "Unweight ...", Direct GPU Decompression:
 * the conventional alternative decompresses whole matrices back to HBM):
 * blob i
 * (infos[i], blobs_dev[i]) written to w_dev[i] with row stride ld[i] >= its
 * cols, exactly as nwc_decode would.  Every blob must have the default chunk
 * geometry (64 chunks of 8 columns, cols % 8 == 0) and all must share
 * tile_rows; each w_dev[i] 16-byte aligned and ld[i] % 8 == 0.  As with the
 * batched GEMV, one grid keeps the whole GPU busy where small separate
 * launches each pay a start-up and a tail.  Async.
 * Errors: INVALID_ARG, UNSUPPORTED (geometry), ALIGNMENT, HIP. */
nwc_status nwc_decode_batched(int count, const nwc_info *infos, const void *const *blobs_dev,
                              uint16_t *const *w_dev, const uint64_t *ld, void *stream);

/* Rows of W by index ("NWC -- Neural Weight Compression", How it works,
 * bullet "Dequantization and embedding lookup": the same decoder serves the
 * embedding lookup, so a tied LM head's compressed matrix is also the
 * embedding table): out row i (device, row stride ld >= cols elements) gets
 * the exact BF16 bits of W row ids_dev[i] (device, n_ids uint32 ids).  An id
 * >= rows gives a row of zeros (ids live on the device, so they are not
 * checked on the host).  Each row costs the decode of its row block's
 * chunks up to it (chunks are coded row after row).  Any geometry.  Async.
 * Errors: INVALID_ARG, ALIGNMENT (out_dev not 2-byte or ids_dev not 4-byte
 * aligned), UNSUPPORTED, HIP. */
nwc_status nwc_gather_rows(const nwc_info *info, const void *blob_dev, const uint32_t *ids_dev,
                           uint32_t n_ids, uint16_t *out_dev, uint64_t ld, void *stream);

/* Skinny decode-GEMM for batch 2..32 ("Unweight ...", Direct GPU
 * Decompression: weights decompressed in on-chip memory feed the matrix
 * units directly, with a strategy per batch size; "NWC -- Neural Weight
 * Compression", Status and limitations: batch 1 is the fast path there and a
 * matrix-core accumulation path is the planned next step):
 * Y[b, n] = sum_k X[b, k] W[n, k] with X (device, batch x cols, row stride
 * ldx) and Y (device, batch x rows, row stride ldy, y_type).  Same decode as
 * nwc_gemv; FP32 accumulation.  From 5 batch rows on (8-row tiles) the
 * products run on the matrix cores, fed by wavefronts that only decode
 * (decoded tiles pass through LDS, never through HBM), 16 X rows per matrix
 * core pass, up to two passes; other tile heights take more than 16 rows on
 * the generic path (workspace).  Repeated calls give the same bits.  Async.
 * Errors: INVALID_ARG (batch outside 2..32), BUFFER_TOO_SMALL, ALIGNMENT, HIP. */
nwc_status nwc_gemm_skinny(const nwc_info *info, const void *blob_dev, const uint16_t *X_dev,
                           uint64_t ldx, int batch, void *Y_dev, uint64_t ldy,
                           nwc_out_type y_type, void *ws, size_t ws_bytes, void *stream);

/* Prefill-sized batches ("NWC -- Neural Weight Compression", How it works,
 * bullet "Dequantization and embedding lookup": the batched path
 * dequantizes and then calls the vendor GEMM): W is decoded into the
 * workspace (nwc_decode's kernel), then one hipBLASLt GEMM forms
 * Y[b, n] = sum_k X[b, k] W[n, k] for any batch >= 1, FP32 accumulation,
 * X (device, batch x cols, row stride ldx % 8 == 0, 16-byte aligned) and Y
 * (device, batch x rows, row stride ldy, y_type, 16-byte aligned, ldy a
 * multiple of 16 bytes).  Meant for more X rows than nwc_gemm_skinny takes:
 * it reads the compressed weights once, writes and reads them back as BF16,
 * so it saves memory, not time.
 *  - nwc_blas: an opaque context the caller creates and destroys, holding a
 *    hipBLASLt handle (whose creation may allocate) and the algorithm picked
 *    for each problem shape; it may be shared by calls on any stream.
 *  - ws (256-byte aligned): at least nwc_prefill_workspace_size bytes: the
 *    decoded W (rows x cols rounded up to 8, BF16), then 32 MiB for
 *    hipBLASLt.  Calls sharing a workspace must not run concurrently.
 *  - The result is deterministic for a given context state, library and
 *    GPU (the vendor GEMM's own summation order).  Async.
 * Errors: INVALID_ARG, BUFFER_TOO_SMALL, ALIGNMENT, UNSUPPORTED (no GEMM
 * algorithm for the shape), HIP. */
typedef struct nwc_blas nwc_blas;
nwc_status nwc_blas_create(nwc_blas **out);
nwc_status nwc_blas_destroy(nwc_blas *h);
nwc_status nwc_prefill_workspace_size(const nwc_info *info, size_t *bytes);
nwc_status nwc_gemm_prefill(nwc_blas *h, const nwc_info *info, const void *blob_dev,
                            const uint16_t *X_dev, uint64_t ldx, int batch, void *Y_dev,
                            uint64_t ldy, nwc_out_type y_type, void *ws, size_t ws_bytes,
                            void *stream);

/* Uncompressed comparator ("NWC -- Neural Weight Compression", opening
 * section: the fused kernel is measured against the uncompressed matvec):
 * y = W x on a plain BF16 matrix (device, rows x cols, row stride ld; cols
 * and ld multiples of 8, W and x 16-byte aligned).  It runs the fused batch-1
 * kernel itself in a mode that loads each tile's 16 bytes per lane per row of
 * BF16 weights in place of the raw bytes and exponent codes: the same 8 x 512
 * tiles, the same equal workgroup ranges, tile claims, next-tile loads 7/8 of
 * the way through a tile, reductions and exchange chain, so the two differ
 * only in the bytes they read and the decode.  ws (device, 256-byte aligned,
 * at least nwc_bf16_workspace_size bytes: one 64-bit slot per tile row) must
 * be zero-filled before its first use; every call leaves it zero-filled.
 * Same concurrency rule as nwc_gemv.  Async.
 * Errors: INVALID_ARG, BUFFER_TOO_SMALL, ALIGNMENT, UNSUPPORTED, HIP. */
nwc_status nwc_bf16_workspace_size(uint64_t rows, uint64_t cols, size_t *bytes);
nwc_status nwc_gemv_bf16(const uint16_t *w_dev, uint64_t rows, uint64_t cols, uint64_t ld,
                         const uint16_t *x_dev, void *y_dev, nwc_out_type y_type, void *ws,
                         size_t ws_bytes, void *stream);

/* HBM read probe ("Unweight ...", The GPU Memory Bottleneck: every generated
 * token reads the weights from HBM, so the achievable read rate bounds
 * decoding): a plain streaming read of `bytes` (rounded down to 16) from
 * buf_dev (device, 16-byte aligned), 8 loads of 16 bytes in flight per lane,
 * in `groups` workgroups of 256 lanes (0 = 8 per compute unit).  layout 0:
 * grid-stride over the whole buffer; layout 1: one contiguous range per
 * workgroup.  sink_dev (device, 4 bytes, 4-byte aligned) is written only for
 * a value no realistic input produces, so the loads cannot be optimised away.
 * The caller times it (bytes / duration) to know what a kernel can reach on
 * this GPU.  Async.
 * Errors: INVALID_ARG (also for a layout other than 0 or 1), ALIGNMENT, HIP. */
nwc_status nwc_read_probe(const void *buf_dev, size_t bytes, uint32_t *sink_dev, uint32_t groups,
                          int layout, void *stream);

/* Test hook for the bounded waits of nwc_gemm_skinny's matrix-core kernel
 * (batch >= 5, 8-row tiles), whose decoding and matrix-core wavefronts wait
 * for each other through flags in LDS.  Every such wait gives up after
 * `polls` polls (each with a short sleep); the workgroup then marks itself
 * failed, stops, and writes NaN for its outputs, so a broken hand-over shows
 * as NaN rather than as a hung GPU.  polls = 0 restores the default bound,
 * 2^22 polls, far beyond any legitimate wait; a tiny bound lets a test drive
 * the give-up path from the host.  Process-wide, read at each launch; not
 * meant to be changed while calls are being made from other threads.
 * Errors: none. */
nwc_status nwc_set_wait_limit(uint32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* NWC_H */
