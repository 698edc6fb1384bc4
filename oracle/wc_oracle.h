/*
 * wc_oracle.h -- plain CPU oracle of the chunked byte-plane + rANS weight codec.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header, table or constant with
 * the HIP library: every constant below is restated here on purpose.
 *
 * Sources (titles of the pages the method comes from):
 *   - "SMEF -- blog companion code" README, file table: pass 3 splits each
 *     tensor into sign / exponent / mantissa byte streams; pass 4 codes a
 *     stream with a vectorised rANS coder.
 *   - "weight-compression" README (Split12), the idea paragraph: each BF16
 *     value is cut into its two bytes, the upper one coded against a table
 *     and the lower one stored unchanged; its bar is an exact round trip.
 *   - "PTWM" README, "How it works": exponent-plane separation by byte split;
 *     "Configuration": large tensors coded as independently decodable chunks.
 * The pages name rANS but fix none of its parameters.  This format fixes them
 * (one reading of the pages, stated in full in wc_oracle.c).
 *
 * All functions are synchronous, single-purpose and take host pointers.
 */
#ifndef WC_ORACLE_H
#define WC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format word = plane layout (low byte) | option bits.
 * Layouts: */
#define WCO_BF16 0         /* hi = sign + exponent bits 7..1 coded, lo raw */
#define WCO_FP32 1         /* exponent byte coded; sign bits, m0, m1, m2 raw */
#define WCO_BF16_REORDER 2 /* "PTWM" README, "How it works" 1: exponent byte coded, sign + 7 mantissa bits raw */
#define WCO_FP16 3         /* 2-plane byte split of the IEEE half: hi = sign, exponent, 2 mantissa bits */
#define WCO_FP16_REORDER 4 /* same page: hi = 5 exponent bits, sign, 2 mantissa bits; lo = 8 mantissa bits */
/* FP8 ("PTWM" README: bit reorder puts the exponent in the high nibble, then a
 * 2-plane nibble split): the high nibble of the reordered byte is coded (16
 * symbols), the low nibble stored raw, two per byte (element 2j in the low
 * nibble of byte j). */
#define WCO_FP8_E4M3 5     /* s e4 m3 -> e4 | s m3 */
#define WCO_FP8_E5M2 6     /* s e5 m2 -> e5[4:1] | e5[0] s m2 */
#define WCO_LAYOUT_MASK 0xFF
/* Options: */
#define WCO_OPT_TENSOR_TABLE 0x100 /* one frequency table per tensor (its whole coded plane), not per chunk */
#define WCO_OPT_RAW_FALLBACK 0x200 /* a chunk whose code is not shorter than its symbols stores them raw */
#define WCO_OPT_CRC32 0x400        /* a CRC-32 of every chunk's payload accompanies the encoding */

/* status codes */
#define WCO_OK 0
#define WCO_ERR_ARG 1
#define WCO_ERR_CAPACITY 2
#define WCO_ERR_CORRUPT 3

/* corruption detail bits (OR-ed) */
#define WCO_EF_BAD_TABLE 1u       /* frequency table does not sum to 4096 */
#define WCO_EF_WORD_OVERRUN 2u    /* decoder wanted a word past the chunk payload */
#define WCO_EF_BAD_FINAL_STATE 4u /* a lane did not end at the initial state */
#define WCO_EF_BAD_TAIL 8u        /* unconsumed words or a non-zero pad word */
#define WCO_EF_BAD_SEEK 16u       /* seek entries out of order, out of range or misaligned */
#define WCO_EF_BAD_CRC 64u        /* a chunk's payload does not match its CRC-32 */

typedef struct {
    uint64_t n;                /* elements */
    uint64_t num_chunks;       /* ceil(n / 65536) */
    uint64_t raw_bytes;        /* bytes of the raw (uncoded) planes */
    uint64_t table_bytes;      /* 512 per chunk, or 512 with WCO_OPT_TENSOR_TABLE */
    uint64_t seek_bytes;       /* 8 * (chunks + 1) */
    uint64_t payload_capacity; /* worst-case payload bytes */
} wco_layout;

/* `dtype` arguments below take a whole format word. */
int wco_query_layout(int dtype, uint64_t n, wco_layout *out);

/* Plane split / merge (byte-plane transform). */
void wco_split_bf16(const uint16_t *v, uint64_t n, uint8_t *hi, uint8_t *lo);
void wco_merge_bf16(const uint8_t *hi, const uint8_t *lo, uint64_t n, uint16_t *v);
/* Any of the 16-bit layouts (BF16, BF16_REORDER, FP16, FP16_REORDER). */
void wco_split_u16(int layout, const uint16_t *v, uint64_t n, uint8_t *hi, uint8_t *lo);
void wco_merge_u16(int layout, const uint8_t *hi, const uint8_t *lo, uint64_t n, uint16_t *v);
/* FP32: exp coded; raw = sign bits (LSB-first, ceil(n/8) B) | m0 | m1 | m2. */
void wco_split_fp32(const uint32_t *u, uint64_t n, uint8_t *exp, uint8_t *raw);
/* FP8 layouts: coded nibbles (one per byte, 0..15) and ceil(n/2) raw bytes. */
void wco_split_fp8(int layout, const uint8_t *v, uint64_t n, uint8_t *coded, uint8_t *raw);
void wco_merge_fp8(int layout, const uint8_t *coded, const uint8_t *raw, uint64_t n, uint8_t *v);
void wco_merge_fp32(const uint8_t *exp, const uint8_t *raw, uint64_t n, uint32_t *u);

/* One chunk. */
void wco_histogram(const uint8_t *sym, uint32_t n, uint32_t counts[256]);
void wco_normalize(const uint32_t counts[256], uint32_t total, uint16_t freq[256]);
/* The same normalisation for counts of a whole tensor (total < 2^52). */
void wco_normalize64(const uint64_t counts[256], uint64_t total, uint16_t freq[256]);
/* Encodes n (1..65536) symbols with table freq into out (capacity >= 128 +
 * 2*n + 2).  Returns the chunk payload size in bytes. */
uint32_t wco_encode_chunk(const uint8_t *sym, uint32_t n, const uint16_t freq[256], uint8_t *out);
/* Decodes; returns 0 or WCO_EF_* bits.  Never reads outside p[0, size). */
uint32_t wco_decode_chunk(const uint8_t *p, uint64_t size, const uint16_t freq[256], uint32_t n,
                          uint8_t *sym);

/* CRC-32 (the ISO-HDLC / zlib CRC: reflected polynomial 0xEDB88320, register
 * preset to all ones, result complemented) of n bytes, bit by bit. */
uint32_t wco_crc32(const uint8_t *p, uint64_t n);
/* crc[k] = wco_crc32 of chunk k's payload bytes [seek[k], seek[k+1]). */
void wco_chunk_crc(const uint64_t *seek, const uint8_t *payload, uint64_t chunks, uint32_t *crc);

/* Tile order of a rows x cols matrix of 16-bit values and its inverse (see
 * wc_oracle.c); WCO_ERR_ARG unless both are multiples of 16. */
int wco_tile_order(const uint16_t *in, uint16_t *out, uint32_t rows, uint32_t cols, int inverse);

/* x W^T in double from BF16 patterns (x: m x k, w: n x k); mag (optional)
 * receives the sums of |products|. */
void wco_gemm_bf16(const uint16_t *x, const uint16_t *w, uint32_t m, uint32_t n, uint32_t k, double *y,
                   double *mag);

/* Whole tensor.  threads <= 1 runs on the calling thread; otherwise chunks
 * are split into contiguous ranges over that many POSIX threads. */
int wco_encode(int dtype, const void *in, uint64_t n, uint8_t *raw, uint16_t *tables,
               uint64_t *seek, uint8_t *payload, uint64_t payload_capacity, int threads);
int wco_decode(int dtype, const uint8_t *raw, const uint16_t *tables, const uint64_t *seek,
               const uint8_t *payload, uint64_t payload_bytes, uint64_t n, void *out, int threads,
               uint32_t *err_bits);

/* Batches: tensor i is coded on its own; its chunks follow the previous
 * tensor's in the tables, seek table and payload, and its raw planes start at
 * raw_base[i] = previous raw_base + previous raw bytes, rounded up to 256. */
int wco_plan_batch(int dtype, const uint64_t *n, uint32_t count, uint64_t *chunk_base,
                   uint64_t *raw_base, wco_layout *total);
int wco_encode_batch(int dtype, const void *const *in, const uint64_t *n, uint32_t count,
                     uint8_t *raw, uint16_t *tables, uint64_t *seek, uint8_t *payload,
                     uint64_t payload_capacity, int threads);
int wco_decode_batch(int dtype, void *const *out, const uint64_t *n, uint32_t count,
                     const uint8_t *raw, const uint16_t *tables, const uint64_t *seek,
                     const uint8_t *payload, uint64_t payload_bytes, int threads,
                     uint32_t *err_bits);

#ifdef __cplusplus
}
#endif
#endif
