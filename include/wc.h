/*
 * wc.h -- C ABI of the MI355X (gfx950) lossless weight codec.
 *
 * What it computes
 * ----------------
 * Lossless compression of BF16 / FP32 weight tensors by byte-plane split and
 * rANS coding of the skewed plane:
 *   - BF16 (weight-compression / Split12 README, the idea paragraph: split
 *     each value into two bytes, code the upper one, keep the lower one as
 *     it is): the high byte (sign + exponent bits 7..1) is rANS coded; the
 *     low byte (exponent bit 0 + 7 mantissa bits) is stored raw.
 *   - FP32 (SMEF README, pass 3: sign / exponent / mantissa byte streams):
 *     the exponent byte is rANS coded; raw = sign bits packed LSB-first
 *     (ceil(n/8) bytes), then mantissa bytes m0 = bits 0-7, m1 = bits 8-15,
 *     m2 = bits 16-22, one byte per element each.
 *   - The coded plane is cut into chunks of 65536 symbols that decode on their
 *     own (PTWM README, "Configuration": independently decodable chunks).
 *     Each chunk has a 256-entry 12-bit frequency table (sum 4096, largest-
 *     remainder rounding, zero counts stay zero) and 32 interleaved 32-bit
 *     rANS states (symbol j -> lane j mod 32), L = 2^16, 16-bit
 *     renormalisation words stored in decode order.
 *   - Chunk payload = 32 final states (u32 LE) + words (u16 LE) + one zero
 *     word if the word count is odd.  seek[0] = 0, seek[k+1] = seek[k] +
 *     payload size of chunk k (u64).  tables = 256 u16 per chunk.
 * Format variants, selected by a format word (plane layout | option bits):
 *   - WC_BF16_REORDER ("PTWM" README, "How it works" step 1, bit reorder:
 *     the exponent moves to the top, the sign right below it): the coded
 *     byte is the 8-bit exponent, the raw byte the sign and 7 mantissa bits.
 *   - WC_FP16 ("PTWM" README, dtype table: float16 takes a 2-plane byte
 *     split): the IEEE half's high byte (sign, 5 exponent bits, 2 mantissa
 *     bits) is coded, its low byte raw.  WC_FP16_REORDER applies the bit
 *     reorder first: the coded byte is the 5 exponent bits, the sign and 2
 *     mantissa bits; the raw byte the other 8 mantissa bits.
 *   - WC_FP8_E4M3, WC_FP8_E5M2 ("PTWM" README, "How it works" steps 1-2:
 *     for the 8-bit floats the reorder brings the exponent bits to the top
 *     four bits of the byte, and the planes are split by nibble):
 *     byte s e4 m3 -> e4 s m3, byte s e5 m2 -> e5 s m2; the high
 *     nibble is coded (16 symbols, same tables and coder), the low nibbles
 *     are raw, two per byte (element 2j in the low nibble of byte j), so the
 *     raw plane is ceil(n/2) bytes.
 *   - WC_OPT_TENSOR_TABLE: one frequency table per tensor, normalised from
 *     the histogram of its whole coded plane, codes all of its chunks
 *     (tables = 256 u16 per tensor; a tensor without elements gets an
 *     all-zero table).
 *   - WC_OPT_RAW_FALLBACK ("PTWM" README, "Configuration": store raw bytes
 *     when compression does not pay; here per chunk): a chunk whose coded
 *     payload would be at least its symbol count rounded up to 4 bytes is
 *     stored as its symbols plus zero padding to that size; a payload of
 *     exactly that size marks such a chunk.
 *   - WC_OPT_CRC32 ("SeedPack" README: every chunk carries a CRC32): crc[k]
 *     = CRC-32 of chunk k's payload bytes (the ISO-HDLC / zlib CRC), written
 *     by encode, checked by decode before it decodes (WC_EF_BAD_CRC).  No
 *     other byte changes.
 *   Format word 0 (WC_BF16) and 1 (WC_FP32) without options is format v1.
 * The result is bit-exact: decode(encode(x)) reproduces every bit pattern,
 * NaN payloads, infinities, subnormals and -0 included (Split12 README: the
 * bar is an exact round trip).
 *
 * Conventions
 * -----------
 * - Pointers named d_* are device pointers (HBM of the current device);
 *   everything else is host memory.  The library allocates nothing, frees
 *   nothing, and never synchronises: every call only validates its arguments
 *   on the host and enqueues kernels on `stream`.  Calls on different streams
 *   may run concurrently if their buffers do not overlap.
 * - Alignment: tensors, raw planes, tables and payload 16 bytes; seek 8
 *   bytes; scratch 256 bytes.  (torch allocations are 256-byte aligned.)
 * - Sizes are in elements unless the name says bytes.  n <= 2^40.
 * - Return codes report argument and launch errors only.  Data errors found
 *   on the device (a corrupt stream, a payload buffer that is too small) are
 *   OR-ed as WC_EF_* bits into *d_err, which the caller zeroes beforehand and
 *   reads after the stream has synchronised.  d_err may be NULL, in which
 *   case such errors are not reported.
 * - For any input bytes, decode reads only inside the buffers it is given
 *   (payload[seek[k], seek[k+1]) within payload_bytes, the tables and raw
 *   planes of its own chunks) and writes only the output elements of its own
 *   chunks.
 */
#ifndef WC_H
#define WC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Plane layouts: the low byte of a format word. */
typedef enum {
    WC_BF16 = 0,
    WC_FP32 = 1,
    WC_BF16_REORDER = 2,
    WC_FP16 = 3,
    WC_FP16_REORDER = 4,
    WC_FP8_E4M3 = 5,
    WC_FP8_E5M2 = 6
} wc_dtype;
/* Option bits of a format word. */
#define WC_LAYOUT_MASK 0xFFu
#define WC_OPT_TENSOR_TABLE 0x100u
#define WC_OPT_RAW_FALLBACK 0x200u
#define WC_OPT_CRC32 0x400u
/* A plane layout OR-ed with option bits.  Encoder and decoder must be given
 * the same format word; any other bit set is WC_ERR_ARG. */
typedef uint32_t wc_format;

typedef enum {
    WC_OK = 0,
    WC_ERR_ARG = 1,      /* null / misaligned pointer, bad format word, size out of range */
    WC_ERR_CAPACITY = 2, /* a buffer is smaller than the layout requires */
    WC_ERR_CORRUPT = 3,  /* (reserved for host-side checks) */
    WC_ERR_HIP = 4       /* a kernel launch failed */
} wc_status;

/* Device error bits (OR-ed into *d_err). */
#define WC_EF_BAD_TABLE 1u       /* a chunk's table does not sum to 4096 */
#define WC_EF_WORD_OVERRUN 2u    /* decoding wanted more words than the chunk holds */
#define WC_EF_BAD_FINAL_STATE 4u /* a lane did not return to the initial state, or a stored state is below 2^16 */
#define WC_EF_BAD_TAIL 8u        /* words left over, or a non-zero pad word */
#define WC_EF_BAD_SEEK 16u       /* seek entries out of order, misaligned or past payload_bytes */
#define WC_EF_CAPACITY 32u       /* encode: the payload did not fit payload_bytes */
#define WC_EF_BAD_CRC 64u        /* decode with WC_OPT_CRC32: a chunk's payload does not match crc[k] */

#define WC_CHUNK 65536u

/* Sizes of every buffer for one tensor (or, from wc_plan_batch, a batch). */
typedef struct {
    uint64_t n;                /* elements */
    uint64_t num_chunks;       /* ceil(n / 65536) (summed over a batch) */
    uint64_t raw_bytes;        /* raw planes */
    uint64_t table_bytes;      /* 512 * num_chunks; with WC_OPT_TENSOR_TABLE 512 per tensor */
    uint64_t seek_bytes;       /* 8 * (num_chunks + 1) */
    uint64_t payload_capacity; /* worst-case payload: 128 + 2 * (len + len % 2) per chunk;
                                  with WC_OPT_RAW_FALLBACK len rounded up to 4 per chunk */
    uint64_t scratch_bytes;    /* encoder scratch */
    uint64_t crc_bytes;        /* 4 * num_chunks with WC_OPT_CRC32, else 0 */
} wc_layout;

/* Device buffers of one encoding.  For encode, payload_bytes is the payload
 * buffer's capacity; for decode, the number of valid payload bytes
 * (seek[num_chunks]). */
typedef struct {
    uint8_t *raw;
    uint16_t *tables;
    uint64_t *seek;
    uint8_t *payload;
    uint64_t payload_bytes;
    uint32_t *crc;             /* WC_OPT_CRC32 only (else ignored): num_chunks u32 */
} wc_buffers;

/* One tensor of a batch.  `ptr` is the device address of the tensor (input
 * of encode, output of decode).  chunk_base / raw_base are filled by
 * wc_plan_batch: tensor i's chunks follow tensor i-1's in the tables, seek
 * table and payload; its raw planes start at raw_base (the previous tensor's
 * raw end rounded up to 256 bytes; encode writes zeros into the gap). */
typedef struct {
    uint64_t ptr;
    uint64_t n;
    uint64_t chunk_base;
    uint64_t raw_base;
} wc_segment;

/* One weight matrix of a fused decode + GEMM batch (wc_decode_gemm_batch).
 * Its segment holds W (rows x cols BF16) encoded in tile order (see
 * wc_tile_order); the call adds X W^T into Y. */
typedef struct {
    uint64_t x;     /* device address of X: m x cols BF16, row-major, 8-byte aligned */
    uint64_t y;     /* device address of Y: m x rows fp32, row-major, 4-byte aligned */
    uint32_t rows;  /* N: rows of W (output features), a multiple of 16 */
    uint32_t cols;  /* K: columns of W (input features), a multiple of 16 */
} wc_gemm;

/* Library version (major * 10000 + minor * 100 + patch). */
int wc_version(void);

/* Human-readable name of a status code. */
const char *wc_status_string(wc_status s);

/* Layout of one tensor of n elements: the size of every buffer the codec
 * reads or writes for it (PTWM README, "Configuration": the stream is cut
 * into independently decodable chunks; SMEF README, file table: the
 * container keeps a seek table).  Pure host function; returns WC_ERR_ARG for
 * a null out, a bad format word or n > 2^40.  The caller allocates every
 * buffer from these sizes and owns it. */
wc_status wc_query_layout(wc_format format, uint64_t n, wc_layout *out);

/* Fills chunk_base and raw_base of segs[0..nseg) (host array; ptr and n are
 * read) and the batch's total layout (SMEF README, "Try it yourself": a
 * whole state dict of named tensors is encoded into one file; here the
 * tensors of a batch are laid end to end, each chunked on its own).  Pure
 * host function; WC_ERR_ARG for a bad format word, segs == NULL with
 * nseg > 0, or an n above 2^40. */
wc_status wc_plan_batch(wc_format format, wc_segment *segs, uint32_t nseg, wc_layout *total);

/* Encode one tensor of n elements at d_in (FP32 as u32 patterns, the 16-bit
 * layouts as u16 patterns, FP8 as bytes): plane split, per-chunk histogram
 * and 12-bit table, chunked rANS, seek-table scan and compaction
 * (weight-compression / Split12 README, the idea paragraph; SMEF README,
 * passes 3 and 4 of the file table).  All pointers are device pointers owned
 * by the caller; the call only enqueues on `stream`.  Argument errors
 * (null or misaligned pointers, a bad format word) return WC_ERR_ARG, a
 * scratch_bytes below the layout WC_ERR_CAPACITY; a payload that does not
 * fit payload_bytes sets WC_EF_CAPACITY in *d_err.  Writes out->raw (layout.raw_bytes), out->tables,
 * out->seek and out->payload (at most out->payload_bytes; layout's
 * payload_capacity always suffices).  d_scratch must hold
 * layout.scratch_bytes.  stage_events may be NULL or point to 5 events that
 * are recorded on `stream` before the split, after the split, after the rANS
 * kernel, after the scan and after the compaction. */
wc_status wc_encode(wc_format format, const void *d_in, uint64_t n, const wc_buffers *out,
                    void *d_scratch, uint64_t scratch_bytes, uint32_t *d_err,
                    hipStream_t stream, hipEvent_t *stage_events);

/* Decode one tensor of n elements into d_out (u32 / u16 / u8 bit patterns):
 * every chunk's rANS stream decoded and joined with the raw planes in one
 * pass (SMEF README, file table: the decoder's full decode;
 * weight-compression / Split12 README: the round trip is bit for bit;
 * SeedPack README: the GPU decodes one tensor at a time).  Device pointers
 * owned by the caller; enqueues on `stream`.  Argument errors return
 * WC_ERR_ARG; stream errors set WC_EF_* bits in *d_err (see above).
 * With WC_OPT_RAW_FALLBACK a chunk stored raw is copied; its padding must be
 * zero (else WC_EF_BAD_TAIL). */
wc_status wc_decode(wc_format format, const wc_buffers *in, uint64_t n, void *d_out,
                    uint32_t *d_err, hipStream_t stream);

/* Batched forms of wc_encode and wc_decode: one launch sequence over all
 * chunks of all tensors (SMEF README, "Try it yourself": a state dict is
 * encoded and decoded as a whole; SeedPack README: a repository is packed
 * file by file into one archive).  h_segs is the host copy of the planned
 * segment array (for validation: a plan that does not match wc_plan_batch's
 * rule is WC_ERR_ARG); d_segs holds the same bytes in device memory (read by
 * the kernels).  The scratch size is the batch layout's scratch_bytes.
 * Errors as for wc_encode / wc_decode. */
wc_status wc_encode_batch(wc_format format, const wc_segment *h_segs, const wc_segment *d_segs,
                          uint32_t nseg, const wc_buffers *out, void *d_scratch,
                          uint64_t scratch_bytes, uint32_t *d_err, hipStream_t stream,
                          hipEvent_t *stage_events);
wc_status wc_decode_batch(wc_format format, const wc_segment *h_segs, const wc_segment *d_segs,
                          uint32_t nseg, const wc_buffers *in, uint32_t *d_err,
                          hipStream_t stream);

/* Tile order of a BF16 (or any 16-bit) matrix W of rows x cols elements,
 * both multiples of 16 (rows * cols < 2^32): 16 x 16 tiles, panel-major
 * (panel p = rows 16p..16p+15; tile t = p * cols/16 + b covers its columns
 * 16b..16b+15), 256 elements per tile, position e of tile (p, b) holding
 * W[16p + (e/8) % 16][16b + 4 ((e/8) / 16) + 8 ((e%8) / 4) + (e%8) % 4].
 * The order is this library's own (a layout transform in the sense of the
 * PTWM docs' Reshape transform): it makes one decoded group of 256 symbols
 * one tile in the matrix cores' operand order.  inverse = 0: d_in is W
 * row-major, d_out the tile stream; inverse = 1: the reverse.  Both buffers
 * 16-byte aligned, rows * cols u16 each, not overlapping.  Enqueued on
 * `stream`; argument errors return WC_ERR_ARG. */
wc_status wc_tile_order(const void *d_in, void *d_out, uint32_t rows, uint32_t cols, int inverse,
                        hipStream_t stream);

/* Decode fused with its consumer (the Split12 README's serving kernels: the
 * compressed weights are the only copy in HBM).  For every segment i (BF16
 * or BF16_REORDER layout, encoded from wc_tile_order's stream of a
 * gemm[i].rows x gemm[i].cols matrix W_i, so segs[i].n = rows * cols):
 * Y_i += X_i W_i^T, X_i with m rows (1 <= m <= 64), products of BF16 values
 * summed in fp32 (matrix-core MFMA per 16 x 16 x 16 block, then fp32 adds in
 * an unspecified order: results are not bitwise reproducible).  No decoded W
 * is written.  h_gemm / d_gemm: host and device copies of the nseg
 * descriptors.  Y must be initialised by the caller (zeros for Y = X W^T).
 * WC_OPT_TENSOR_TABLE and WC_OPT_CRC32 are honoured (the CRC is checked
 * first); WC_OPT_RAW_FALLBACK is rejected (WC_ERR_ARG), as are a chunk that
 * touches more panels of 16 rows than the kernel holds accumulators for
 * (8 / ceil(m/16) rounded down to 2, 4 or 8; cols = 2048 or cols >= 4096
 * never needs more than 2).  Data errors
 * set WC_EF_* bits as in wc_decode_batch; Y is then undefined. */
wc_status wc_decode_gemm_batch(wc_format format, const wc_segment *h_segs, const wc_segment *d_segs, uint32_t nseg,
                               const wc_gemm *h_gemm, const wc_gemm *d_gemm, uint32_t m, const wc_buffers *in,
                               uint32_t *d_err, hipStream_t stream);

/* Host-side self check of the exact division by reciprocal and of the
 * encoder's state update built on it (same inline code, compiled for the
 * CPU): every divisor 1..4096 against boundary and sampled dividends below
 * 2^32, and the update x' = 4096 floor(xr / f) + (xr mod f) + b for every
 * f against boundary and sampled xr in [1, f 2^20).  Returns the number of
 * wrong results (0 expected). */
uint64_t wc_check_division(uint32_t samples_per_divisor);

/* Which decoder wc_decode / wc_decode_batch would launch for num_chunks
 * chunks of n elements in total with payload_bytes of payload, on the
 * device that `stream` belongs to (the current device for the null
 * stream): *one_chunk_per_wave = 1 for the wide-table decoder (one chunk per
 * wavefront, taken while every chunk fits on that device's compute units at
 * once), 0 for two chunks per wavefront; *refill_dwords = 1 or 2 (the ring
 * refill block per lane, 2 above 3.25 bits per coded symbol).  Host
 * function; WC_ERR_HIP if the stream's device cannot be queried. */
wc_status wc_decode_variant(wc_format format, uint64_t num_chunks, uint64_t n, uint64_t payload_bytes,
                            hipStream_t stream, int *one_chunk_per_wave, int *refill_dwords);

/* How the encoder writes the coded words of a chunk; both forms write the
 * same bytes and differ in speed only.  WC_ENC_WORDS_DIRECT: each step's
 * words go straight to the chunk's scratch slot as 2-byte stores (fewest
 * instructions per step: fastest where the grid does not fill the GPU).
 * WC_ENC_WORDS_STAGED: they go to a 256-word LDS ring per chunk and reach
 * the slot as whole 128-byte lines, with 16-byte stores, once per 256
 * symbols (fewer memory operations: fastest where the grid fills every
 * SIMD).  WC_ENC_WORDS_AUTO (the
 * default): for the 16-bit layouts (BF16, FP16 and their reorders) staged
 * when the encoder's grid has at least 16 wavefronts (two chunks each) per
 * compute unit of the stream's device, else direct; FP32 and FP8 direct. */
#define WC_ENC_WORDS_AUTO 0
#define WC_ENC_WORDS_DIRECT 1
#define WC_ENC_WORDS_STAGED 2

/* Sets the encoder word-store form for every later encode call of the
 * process (any thread, any device) and returns the previous setting, or -1
 * (nothing changed) for a value that is not one of WC_ENC_WORDS_*.  Meant
 * for tuning and tests; calls already enqueued are not affected. */
int wc_set_encoder_words(int mode);

/* Which form an encode of num_chunks chunks under `format` would take on
 * the device that `stream` belongs to (the current device for the null
 * stream), given the current setting: *staged = 1 for WC_ENC_WORDS_STAGED,
 * 0 for direct.  Host function; WC_ERR_ARG for a bad format or null
 * pointer, WC_ERR_HIP if the stream's device cannot be queried. */
wc_status wc_encode_variant(wc_format format, uint64_t num_chunks, hipStream_t stream, int *staged);

/* Size of the fixed device array wc_encode_noalloc takes its scratch from
 * (one per device the library runs on, held until the process ends). */
#define WC_NOALLOC_SCRATCH_BYTES (128ull << 20)

/* For callers that cannot allocate device memory -- code under HIP stream
 * capture, tight serving loops, harnesses that forbid hipMalloc: wc_encode
 * with the encoder's scratch taken from the library's fixed array of
 * WC_NOALLOC_SCRATCH_BYTES on the stream's device instead of a caller
 * buffer.  Inputs, outputs, results and errors are those of wc_encode; a
 * tensor whose layout needs more scratch (more chunks than
 * wc_noalloc_max_chunks(format): 1,021 for BF16, about 66.9 million
 * elements) returns WC_ERR_CAPACITY before anything is enqueued.  Calls no
 * allocator.  Every call on a device shares that device's array and leaves
 * its contents behind (nothing in it needs clearing): calls that overlap on
 * one device, from other streams or threads, race and must be serialised by
 * the caller. */
wc_status wc_encode_noalloc(wc_format format, const void *d_in, uint64_t n, const wc_buffers *out, uint32_t *d_err,
                            hipStream_t stream);

/* The most chunks wc_encode_noalloc takes under `format` (0 for a bad
 * format word).  Pure host function. */
uint64_t wc_noalloc_max_chunks(wc_format format);

#ifdef __cplusplus
}
#endif
#endif
