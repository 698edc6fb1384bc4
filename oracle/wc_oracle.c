/*
 * wc_oracle.c -- plain CPU oracle of the chunked byte-plane + rANS weight codec.
 *
 * TEST INFRASTRUCTURE ONLY (see wc_oracle.h): the definition the GPU path is
 * checked against.  Written for reading, not for speed: every step follows
 * the format description below in the order it is stated, in scalar C.
 *
 * What the pages fix, and what this format reads into them
 * --------------------------------------------------------
 * Split ("SMEF" README, pass 3; "weight-compression"/Split12 README; "PTWM"
 * README, "How it works" step 2): a BF16 value v is split into the high byte
 * hi = v >> 8 (sign and the top seven exponent bits), which is entropy coded,
 * and the low byte lo = v & 0xFF (last exponent bit and seven mantissa bits),
 * which is stored raw.  FP32 u is split into the exponent byte (u >> 23) &
 * 0xFF, which is coded, and raw streams: the sign bits packed eight to a byte
 * (element 8j+k is bit k of byte j), then m0 = u & 0xFF, m1 = (u >> 8) & 0xFF,
 * m2 = (u >> 16) & 0x7F, each one byte per element.
 *
 * Chunks ("PTWM" README, "Configuration": independently decodable chunks):
 * the coded plane is cut into chunks of 65536 symbols, the last one shorter.
 *
 * rANS (named, not specified, by the "SMEF" README's pass 4 and the PTWM
 * codec list).  Per chunk:
 *   - a 256-entry count histogram, normalised by integer arithmetic to
 *     frequencies f that sum to M = 4096 (12-bit), f > 0 exactly where the
 *     count is > 0 (largest-remainder rounding; see wco_normalize);
 *   - b[s] = sum of f[t] for t < s; symbol s owns slots [b[s], b[s] + f[s]);
 *   - 32 interleaved 32-bit states: symbol j goes to lane j mod 32 at step
 *     j div 32; every state starts at L = 65536 and stays in [L, 2^32);
 *   - 16-bit renormalisation words; the encoder runs from the last step to
 *     the first and, within a step, from lane 31 down to lane 0, and every
 *     word it emits is put in front of the words emitted so far, so the
 *     stream is in decode order (steps ascending, lanes ascending);
 *   - chunk payload = 32 final states (u32 little-endian, lane order), then
 *     the words (u16 little-endian), then one zero word if the word count is
 *     odd, so every payload is a multiple of 4 bytes.
 * Tables are stored as 256 u16 per chunk, the seek table as u64 offsets
 * (seek[0] = 0, seek[k+1] = seek[k] + size of chunk k).
 *
 * Format variants (the pages' other layouts and options; a format word is a
 * layout code OR-ed with option bits):
 *   - BF16_REORDER ("PTWM" README, "How it works" step 1, bit reorder): the
 *     exponent moves to the most significant position and the sign right
 *     below it, so for BF16 the coded byte is the 8-bit exponent and the raw
 *     byte is the sign followed by the 7 mantissa bits.
 *   - FP16 ("PTWM" README, dtype table: float16 takes a 2-plane byte split):
 *     the high byte (sign, 5 exponent bits, 2 mantissa bits) is coded, the
 *     low byte raw.  FP16_REORDER applies the same page's bit reorder first:
 *     the coded byte holds the 5 exponent bits, then the sign, then the top
 *     2 mantissa bits; the raw byte the other 8 mantissa bits.
 *   - FP8_E4M3, FP8_E5M2 (the same page: for 8-bit floats the reorder moves
 *     the exponent into the high nibble; then a 2-plane nibble split): the
 *     byte s e4 m3 becomes e4 s m3, the byte s e5 m2 becomes e5 s m2; the
 *     high nibble is coded (symbols 0..15, through the same tables and
 *     coder), the low nibble stored raw, two per byte, element 2j in the low
 *     nibble of byte j (a last odd element leaves the high nibble zero).
 *   - CRC32 (the "SeedPack" README: every chunk of its archive carries a
 *     CRC32; here every chunk of the coded plane): crc[k] is the CRC-32 of
 *     chunk k's payload bytes, the common ISO-HDLC / zlib CRC (polynomial
 *     0x04C11DB7 processed least significant bit first, i.e. 0xEDB88320
 *     reflected, register preset to all ones, result complemented).  It
 *     does not change any other byte of the encoding.
 *   - TENSOR_TABLE (reading: the per-tensor codec records of the "PTWM"
 *     README's container, one table for a tensor's chunks): a single table,
 *     normalised from the histogram of the tensor's whole coded plane, codes
 *     every chunk of the tensor.
 *   - RAW_FALLBACK ("PTWM" README, "Configuration": raw bytes are stored when
 *     compression does not pay; here applied per chunk): a chunk whose coded
 *     payload would be at least its symbol count rounded up to 4 bytes is
 *     stored as its symbols, zero-padded to that size.  A payload of exactly
 *     that size therefore marks a raw chunk.
 */
#include "wc_oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORC_CHUNK 65536u
#define ORC_LANES 32u
#define ORC_SCALE_BITS 12u
#define ORC_M 4096u
#define ORC_L 65536u
#define ORC_MAX_WORDS 65536u

/* ------------------------------------------------------------------ layout */

/* The layout code of a format word, or -1 if the word is not a format. */
static int layout_of(int format)
{
    int layout = format & WCO_LAYOUT_MASK;
    if (layout > WCO_FP8_E5M2) return -1;
    if (format & ~(WCO_LAYOUT_MASK | WCO_OPT_TENSOR_TABLE | WCO_OPT_RAW_FALLBACK | WCO_OPT_CRC32)) return -1;
    return layout;
}

static int is_fp8(int layout) { return layout == WCO_FP8_E4M3 || layout == WCO_FP8_E5M2; }

static uint64_t raw_bytes_of(int layout, uint64_t n)
{
    if (layout == WCO_FP32) return (n + 7) / 8 + 3 * n;
    if (is_fp8(layout)) return (n + 1) / 2;
    return n;
}

/* Payload size of a chunk of len symbols stored raw. */
static uint64_t raw_chunk_size(uint64_t len)
{
    return (len + 3) / 4 * 4;
}

/* Largest payload a chunk of len symbols can take: 32 states, at most one
 * word per symbol, one pad word. */
static uint64_t chunk_capacity(uint64_t len)
{
    uint64_t words = len + (len & 1);
    return 128 + 2 * words;
}

int wco_query_layout(int dtype, uint64_t n, wco_layout *out)
{
    int layout = layout_of(dtype);
    if (!out || layout < 0) return WCO_ERR_ARG;
    uint64_t c = (n + ORC_CHUNK - 1) / ORC_CHUNK;
    out->n = n;
    out->num_chunks = c;
    out->raw_bytes = raw_bytes_of(layout, n);
    out->table_bytes = (dtype & WCO_OPT_TENSOR_TABLE) ? 512 : 512 * c;
    out->seek_bytes = 8 * (c + 1);
    out->payload_capacity = 0;
    for (uint64_t k = 0; k < c; k++) {
        uint64_t len = (k + 1 < c) ? ORC_CHUNK : n - k * ORC_CHUNK;
        out->payload_capacity += (dtype & WCO_OPT_RAW_FALLBACK) ? raw_chunk_size(len) : chunk_capacity(len);
    }
    return WCO_OK;
}

/* ------------------------------------------------------------- plane split */

void wco_split_bf16(const uint16_t *v, uint64_t n, uint8_t *hi, uint8_t *lo)
{
    for (uint64_t i = 0; i < n; i++) {
        hi[i] = (uint8_t)(v[i] >> 8);
        lo[i] = (uint8_t)(v[i] & 0xFF);
    }
}

void wco_merge_bf16(const uint8_t *hi, const uint8_t *lo, uint64_t n, uint16_t *v)
{
    for (uint64_t i = 0; i < n; i++) v[i] = (uint16_t)(((uint16_t)hi[i] << 8) | lo[i]);
}

/* The 16-bit layouts, one element at a time: take the value apart into
 * sign, exponent and mantissa fields, put the fields in the layout's order,
 * and cut the 16 bits into the coded high byte and the raw low byte. */
void wco_split_u16(int layout, const uint16_t *v, uint64_t n, uint8_t *hi, uint8_t *lo)
{
    for (uint64_t i = 0; i < n; i++) {
        uint32_t x = v[i], r;
        uint32_t sign = x >> 15;
        if (layout == WCO_BF16_REORDER) {
            uint32_t e = (x >> 7) & 0xFF, m = x & 0x7F; /* 8 exponent, 7 mantissa bits */
            r = (e << 8) | (sign << 7) | m;
        } else if (layout == WCO_FP16_REORDER) {
            uint32_t e = (x >> 10) & 0x1F, m = x & 0x3FF; /* 5 exponent, 10 mantissa bits */
            r = (e << 11) | (sign << 10) | m;
        } else { /* BF16, FP16: the bits as they are */
            r = x;
        }
        hi[i] = (uint8_t)(r >> 8);
        lo[i] = (uint8_t)(r & 0xFF);
    }
}

void wco_merge_u16(int layout, const uint8_t *hi, const uint8_t *lo, uint64_t n, uint16_t *v)
{
    for (uint64_t i = 0; i < n; i++) {
        uint32_t r = ((uint32_t)hi[i] << 8) | lo[i], x;
        if (layout == WCO_BF16_REORDER) {
            uint32_t e = r >> 8, sign = (r >> 7) & 1, m = r & 0x7F;
            x = (sign << 15) | (e << 7) | m;
        } else if (layout == WCO_FP16_REORDER) {
            uint32_t e = r >> 11, sign = (r >> 10) & 1, m = r & 0x3FF;
            x = (sign << 15) | (e << 10) | m;
        } else {
            x = r;
        }
        v[i] = (uint16_t)x;
    }
}

/* FP8, one element at a time: take the byte apart into sign, exponent and
 * mantissa, put the exponent first and the sign right after it, and cut the
 * byte into its coded high nibble and its raw low nibble. */
void wco_split_fp8(int layout, const uint8_t *v, uint64_t n, uint8_t *coded, uint8_t *raw)
{
    memset(raw, 0, (n + 1) / 2);
    for (uint64_t i = 0; i < n; i++) {
        uint32_t b = v[i], r;
        uint32_t sign = b >> 7;
        if (layout == WCO_FP8_E4M3) {
            uint32_t e = (b >> 3) & 0xF, m = b & 0x7; /* 4 exponent, 3 mantissa bits */
            r = (e << 4) | (sign << 3) | m;
        } else {
            uint32_t e = (b >> 2) & 0x1F, m = b & 0x3; /* 5 exponent, 2 mantissa bits */
            r = (e << 3) | (sign << 2) | m;
        }
        coded[i] = (uint8_t)(r >> 4);
        raw[i / 2] |= (uint8_t)((r & 0xF) << (4 * (i % 2)));
    }
}

void wco_merge_fp8(int layout, const uint8_t *coded, const uint8_t *raw, uint64_t n, uint8_t *v)
{
    for (uint64_t i = 0; i < n; i++) {
        uint32_t r = ((uint32_t)coded[i] << 4) | ((raw[i / 2] >> (4 * (i % 2))) & 0xF), x;
        if (layout == WCO_FP8_E4M3) {
            uint32_t e = r >> 4, sign = (r >> 3) & 1, m = r & 0x7;
            x = (sign << 7) | (e << 3) | m;
        } else {
            uint32_t e = r >> 3, sign = (r >> 2) & 1, m = r & 0x3;
            x = (sign << 7) | (e << 2) | m;
        }
        v[i] = (uint8_t)x;
    }
}

void wco_split_fp32(const uint32_t *u, uint64_t n, uint8_t *exp, uint8_t *raw)
{
    uint64_t sign_bytes = (n + 7) / 8;
    uint8_t *sign = raw;
    uint8_t *m0 = raw + sign_bytes;
    uint8_t *m1 = m0 + n;
    uint8_t *m2 = m1 + n;
    memset(sign, 0, sign_bytes);
    for (uint64_t i = 0; i < n; i++) {
        exp[i] = (uint8_t)((u[i] >> 23) & 0xFF);
        sign[i / 8] |= (uint8_t)((u[i] >> 31) << (i % 8));
        m0[i] = (uint8_t)(u[i] & 0xFF);
        m1[i] = (uint8_t)((u[i] >> 8) & 0xFF);
        m2[i] = (uint8_t)((u[i] >> 16) & 0x7F);
    }
}

void wco_merge_fp32(const uint8_t *exp, const uint8_t *raw, uint64_t n, uint32_t *u)
{
    uint64_t sign_bytes = (n + 7) / 8;
    const uint8_t *sign = raw;
    const uint8_t *m0 = raw + sign_bytes;
    const uint8_t *m1 = m0 + n;
    const uint8_t *m2 = m1 + n;
    for (uint64_t i = 0; i < n; i++) {
        uint32_t s = (sign[i / 8] >> (i % 8)) & 1u;
        u[i] = (s << 31) | ((uint32_t)exp[i] << 23) | ((uint32_t)m2[i] << 16) |
               ((uint32_t)m1[i] << 8) | (uint32_t)m0[i];
    }
}

/* --------------------------------------------------- histogram + normalise */

void wco_histogram(const uint8_t *sym, uint32_t n, uint32_t counts[256])
{
    memset(counts, 0, 256 * sizeof(uint32_t));
    for (uint32_t i = 0; i < n; i++) counts[sym[i]]++;
}

/*
 * Integer normalisation of a chunk's counts to a 12-bit table.
 *  1. For every symbol with count c > 0: q = floor(c*4096/T), r = c*4096 mod T.
 *  2. q >= 1: the symbol is "regular" and f = q.  q = 0: it is "forced" to f = 1.
 *  3. D = 4096 - sum f.
 *  4. D > 0: the D regular symbols with the largest r (ties: smaller symbol
 *     first) get f += 1.  (D < number of regular symbols always holds.)
 *  5. D < 0: -D times, the symbol with the largest f (ties: smaller symbol)
 *     gets f -= 1.  (That f is always >= 2.)
 * The arithmetic is done in 64 bits, so counts of a whole tensor (total below
 * 2^52) are exact too; for a chunk c*4096 <= 2^28.
 */
void wco_normalize64(const uint64_t counts[256], uint64_t total, uint16_t freq[256])
{
    uint64_t f[256], r[256];
    int regular[256];
    int64_t sum = 0;
    for (int s = 0; s < 256; s++) {
        f[s] = 0;
        r[s] = 0;
        regular[s] = 0;
        if (counts[s] == 0) continue;
        uint64_t scaled = counts[s] * ORC_M;
        uint64_t q = scaled / total;
        r[s] = scaled % total;
        if (q >= 1) {
            f[s] = q;
            regular[s] = 1;
        } else {
            f[s] = 1;
        }
        sum += (int64_t)f[s];
    }
    int64_t d = (int64_t)ORC_M - sum;

    if (d > 0) {
        /* order the regular symbols by remainder descending, symbol ascending
         * (insertion sort: at most 256 entries) */
        int order[256];
        int m = 0;
        for (int s = 0; s < 256; s++) {
            if (!regular[s]) continue;
            int j = m++;
            while (j > 0) {
                int t = order[j - 1];
                int t_before_s = (r[t] > r[s]) || (r[t] == r[s] && t < s);
                if (t_before_s) break;
                order[j] = t;
                j--;
            }
            order[j] = s;
        }
        for (int i = 0; i < d; i++) f[order[i]] += 1;
    } else if (d < 0) {
        for (int i = 0; i < -d; i++) {
            int best = -1;
            for (int s = 0; s < 256; s++)
                if (best < 0 || f[s] > f[best]) best = s;
            f[best] -= 1;
        }
    }
    for (int s = 0; s < 256; s++) freq[s] = (uint16_t)f[s];
}

void wco_normalize(const uint32_t counts[256], uint32_t total, uint16_t freq[256])
{
    uint64_t c[256];
    for (int s = 0; s < 256; s++) c[s] = counts[s];
    wco_normalize64(c, total, freq);
}

/* ------------------------------------------------------------ chunk codec */

static void cumulative(const uint16_t freq[256], uint32_t b[256])
{
    uint32_t acc = 0;
    for (int s = 0; s < 256; s++) {
        b[s] = acc;
        acc += freq[s];
    }
}

static void put_u32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

uint32_t wco_encode_chunk(const uint8_t *sym, uint32_t n, const uint16_t freq[256], uint8_t *out)
{
    uint32_t b[256];
    cumulative(freq, b);

    uint32_t x[ORC_LANES];
    for (uint32_t l = 0; l < ORC_LANES; l++) x[l] = ORC_L;

    /* words are prepended: fill a buffer from its end towards its start */
    uint16_t *words = (uint16_t *)malloc(ORC_MAX_WORDS * sizeof(uint16_t));
    uint32_t first = ORC_MAX_WORDS; /* index of the first word in decode order */

    uint32_t steps = (n + ORC_LANES - 1) / ORC_LANES;
    for (uint32_t t = steps; t-- > 0;) {
        for (uint32_t l = ORC_LANES; l-- > 0;) {
            uint32_t j = t * ORC_LANES + l;
            if (j >= n) continue;
            uint32_t s = sym[j];
            uint32_t f = freq[s];
            /* renormalise: x >= f * 2^20, written without overflowing at f = 4096 */
            if ((x[l] >> 20) >= f) {
                words[--first] = (uint16_t)(x[l] & 0xFFFF);
                x[l] >>= 16;
            }
            x[l] = ((x[l] / f) << ORC_SCALE_BITS) + (x[l] % f) + b[s];
        }
    }

    uint32_t w = ORC_MAX_WORDS - first;
    for (uint32_t l = 0; l < ORC_LANES; l++) put_u32(out + 4 * l, x[l]);
    uint8_t *p = out + 128;
    for (uint32_t i = 0; i < w; i++) {
        uint16_t v = words[first + i];
        p[2 * i] = (uint8_t)v;
        p[2 * i + 1] = (uint8_t)(v >> 8);
    }
    uint32_t size = 128 + 2 * w;
    if (w & 1) {
        out[size] = 0;
        out[size + 1] = 0;
        size += 2;
    }
    free(words);
    return size;
}

uint32_t wco_decode_chunk(const uint8_t *p, uint64_t size, const uint16_t freq[256], uint32_t n,
                          uint8_t *sym)
{
    uint32_t err = 0;
    uint64_t fsum = 0;
    for (int s = 0; s < 256; s++) fsum += freq[s];
    if (fsum != ORC_M) return WCO_EF_BAD_TABLE;
    if (size < 128 || size % 4 != 0) return WCO_EF_BAD_SEEK;

    uint32_t b[256];
    cumulative(freq, b);
    uint8_t slot_sym[ORC_M];
    for (int s = 0; s < 256; s++)
        for (uint32_t k = 0; k < freq[s]; k++) slot_sym[b[s] + k] = (uint8_t)s;

    uint32_t x[ORC_LANES];
    for (uint32_t l = 0; l < ORC_LANES; l++) x[l] = get_u32(p + 4 * l);
    /* Every state stays in [L, 2^32) (the interval rANS keeps its state in),
       so the encoder's final states, stored first, are never below L: a
       chunk that stores one is no encoding and is rejected before a step. */
    for (uint32_t l = 0; l < ORC_LANES; l++)
        if (x[l] < ORC_L) return WCO_EF_BAD_FINAL_STATE;

    uint64_t ptr = 128;
    uint32_t steps = (n + ORC_LANES - 1) / ORC_LANES;
    for (uint32_t t = 0; t < steps; t++) {
        for (uint32_t l = 0; l < ORC_LANES; l++) {
            uint32_t j = t * ORC_LANES + l;
            if (j >= n) continue;
            uint32_t slot = x[l] & (ORC_M - 1);
            uint32_t s = slot_sym[slot];
            x[l] = freq[s] * (x[l] >> ORC_SCALE_BITS) + slot - b[s];
            sym[j] = (uint8_t)s;
            if (x[l] < ORC_L) {
                if (ptr + 2 > size) {
                    err |= WCO_EF_WORD_OVERRUN;
                    return err;
                }
                uint32_t w = (uint32_t)p[ptr] | ((uint32_t)p[ptr + 1] << 8);
                x[l] = (x[l] << 16) | w;
                ptr += 2;
            }
        }
    }
    for (uint32_t l = 0; l < ORC_LANES; l++)
        if (x[l] != ORC_L) err |= WCO_EF_BAD_FINAL_STATE;
    uint64_t left = size - ptr;
    if (left == 2) {
        if (p[ptr] != 0 || p[ptr + 1] != 0) err |= WCO_EF_BAD_TAIL;
    } else if (left != 0) {
        err |= WCO_EF_BAD_TAIL;
    }
    return err;
}

/* ------------------------------------------------------------------ CRC-32 */

/* One bit at a time: the register's low bit is the coefficient that leaves
 * next; a 1 leaving means subtracting (xor) the polynomial. */
uint32_t wco_crc32(const uint8_t *p, uint64_t n)
{
    uint32_t r = 0xFFFFFFFFu;
    for (uint64_t i = 0; i < n; i++) {
        r ^= p[i];
        for (int b = 0; b < 8; b++) r = (r & 1u) ? (r >> 1) ^ 0xEDB88320u : r >> 1;
    }
    return r ^ 0xFFFFFFFFu;
}

void wco_chunk_crc(const uint64_t *seek, const uint8_t *payload, uint64_t chunks, uint32_t *crc)
{
    for (uint64_t k = 0; k < chunks; k++) crc[k] = wco_crc32(payload + seek[k], seek[k + 1] - seek[k]);
}

/* ------------------------------------------------- tile order and GEMM */

/* Tile order of a rows x cols matrix (row-major, both multiples of 16): the
 * matrix is cut into 16 x 16 tiles, panel by panel (panel p = rows 16p ..
 * 16p+15; within it tile b = columns 16b .. 16b+15), each tile written as
 * 256 values; value e of a tile (l = e / 8, i = e % 8) is the element at row
 * l % 16 and column 4 (l / 16) + 8 (i / 4) + i % 4 of the tile.  This is not
 * from the pages: it is the GPU library's own order for decoding straight
 * into matrix-core operands, defined here element by element so that the
 * tests can check the GPU's permutation and the bytes encoded after it. */
int wco_tile_order(const uint16_t *in, uint16_t *out, uint32_t rows, uint32_t cols, int inverse)
{
    if (rows % 16 || cols % 16) return WCO_ERR_ARG;
    uint64_t s = 0;
    for (uint32_t p = 0; p < rows / 16; p++)
        for (uint32_t b = 0; b < cols / 16; b++)
            for (uint32_t e = 0; e < 256; e++, s++) {
                const uint32_t l = e / 8, i = e % 8;
                const uint64_t r = 16ull * p + l % 16;
                const uint64_t c = 16ull * b + 4 * (l / 16) + 8 * (i / 4) + i % 4;
                if (inverse) out[r * cols + c] = in[s];
                else out[s] = in[r * cols + c];
            }
    return WCO_OK;
}

/* A BF16 bit pattern is the high half of an IEEE single. */
static double bf16_value(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* y[i][j] = sum over t of x[i][t] w[j][t] (x: m x k, w: n x k, BF16 bit
 * patterns, row-major) in double; each product of two BF16 values is exact
 * in double.  If mag is not NULL, mag[i][j] = sum of |x[i][t] w[j][t]|. */
void wco_gemm_bf16(const uint16_t *x, const uint16_t *w, uint32_t m, uint32_t n, uint32_t k, double *y,
                   double *mag)
{
    for (uint32_t i = 0; i < m; i++)
        for (uint32_t j = 0; j < n; j++) {
            double acc = 0.0, a = 0.0;
            for (uint32_t t = 0; t < k; t++) {
                const double p = bf16_value(x[(uint64_t)i * k + t]) * bf16_value(w[(uint64_t)j * k + t]);
                acc += p;
                a += p < 0 ? -p : p;
            }
            y[(uint64_t)i * n + j] = acc;
            if (mag) mag[(uint64_t)i * n + j] = a;
        }
}

/* ------------------------------------------------------------ whole tensor */

typedef struct {
    int format;
    const void *in;
    uint64_t n;
    const uint8_t *coded; /* the coded plane (hi bytes or exponent bytes) */
    uint16_t *tables;
    uint8_t *scratch;     /* per-chunk slots of chunk_capacity(65536) bytes */
    uint32_t *sizes;
    uint64_t k0, k1;
} enc_job;

static void *encode_range(void *arg)
{
    enc_job *j = (enc_job *)arg;
    uint64_t slot = chunk_capacity(ORC_CHUNK);
    for (uint64_t k = j->k0; k < j->k1; k++) {
        uint64_t start = k * ORC_CHUNK;
        uint32_t len = (uint32_t)((j->n - start < ORC_CHUNK) ? j->n - start : ORC_CHUNK);
        uint16_t *table = j->tables;
        if (!(j->format & WCO_OPT_TENSOR_TABLE)) {
            uint32_t counts[256];
            table = j->tables + 256 * k;
            wco_histogram(j->coded + start, len, counts);
            wco_normalize(counts, len, table);
        }
        uint8_t *out = j->scratch + slot * k;
        uint32_t size = wco_encode_chunk(j->coded + start, len, table, out);
        if ((j->format & WCO_OPT_RAW_FALLBACK) && size >= raw_chunk_size(len)) {
            size = (uint32_t)raw_chunk_size(len);
            memcpy(out, j->coded + start, len);
            memset(out + len, 0, size - len);
        }
        j->sizes[k] = size;
    }
    return NULL;
}

static int run_ranges(void *(*fn)(void *), void *jobs, size_t job_size, uint64_t chunks, int threads,
                      void (*set_range)(void *, uint64_t, uint64_t))
{
    if (threads < 1) threads = 1;
    if ((uint64_t)threads > chunks) threads = chunks ? (int)chunks : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * threads);
    for (int i = 0; i < threads; i++) {
        uint64_t k0 = chunks * i / threads, k1 = chunks * (i + 1) / threads;
        void *job = (char *)jobs + job_size * i;
        set_range(job, k0, k1);
    }
    if (threads == 1) {
        fn(jobs);
    } else {
        for (int i = 0; i < threads; i++) pthread_create(&tid[i], NULL, fn, (char *)jobs + job_size * i);
        for (int i = 0; i < threads; i++) pthread_join(tid[i], NULL);
    }
    free(tid);
    return 0;
}

static void enc_set_range(void *job, uint64_t k0, uint64_t k1)
{
    ((enc_job *)job)->k0 = k0;
    ((enc_job *)job)->k1 = k1;
}

int wco_encode(int dtype, const void *in, uint64_t n, uint8_t *raw, uint16_t *tables,
               uint64_t *seek, uint8_t *payload, uint64_t payload_capacity, int threads)
{
    int layout = layout_of(dtype);
    if (layout < 0) return WCO_ERR_ARG;
    if (!seek) return WCO_ERR_ARG;
    seek[0] = 0;
    if (n == 0) {
        /* a tensor without elements still owns its (empty) table */
        if ((dtype & WCO_OPT_TENSOR_TABLE) && tables) memset(tables, 0, 512);
        return WCO_OK;
    }
    if (!in || !raw || !tables || !payload) return WCO_ERR_ARG;

    uint64_t chunks = (n + ORC_CHUNK - 1) / ORC_CHUNK;
    uint8_t *coded = (uint8_t *)malloc(n);
    if (layout == WCO_FP32)
        wco_split_fp32((const uint32_t *)in, n, coded, raw);
    else if (is_fp8(layout))
        wco_split_fp8(layout, (const uint8_t *)in, n, coded, raw);
    else
        wco_split_u16(layout, (const uint16_t *)in, n, coded, raw);
    if (dtype & WCO_OPT_TENSOR_TABLE) {
        uint64_t counts[256] = {0};
        for (uint64_t i = 0; i < n; i++) counts[coded[i]]++;
        wco_normalize64(counts, n, tables);
    }

    /* each chunk is coded into its own worst-case slot, then the payloads are
     * laid end to end */
    int nthreads = threads < 1 ? 1 : threads;
    uint64_t workers = (uint64_t)nthreads < chunks ? (uint64_t)nthreads : chunks;
    uint64_t slot = chunk_capacity(ORC_CHUNK);
    uint8_t *scratch = (uint8_t *)malloc(slot * chunks);
    uint32_t *sizes = (uint32_t *)malloc(sizeof(uint32_t) * chunks);
    enc_job *jobs = (enc_job *)calloc(workers, sizeof(enc_job));
    for (uint64_t i = 0; i < workers; i++) {
        jobs[i].format = dtype;
        jobs[i].in = in;
        jobs[i].n = n;
        jobs[i].coded = coded;
        jobs[i].tables = tables;
        jobs[i].scratch = scratch;
        jobs[i].sizes = sizes;
    }
    run_ranges(encode_range, jobs, sizeof(enc_job), chunks, (int)workers, enc_set_range);

    int status = WCO_OK;
    for (uint64_t k = 0; k < chunks; k++) seek[k + 1] = seek[k] + sizes[k];
    if (seek[chunks] > payload_capacity) {
        status = WCO_ERR_CAPACITY;
    } else {
        for (uint64_t k = 0; k < chunks; k++) memcpy(payload + seek[k], scratch + slot * k, sizes[k]);
    }
    free(jobs);
    free(sizes);
    free(scratch);
    free(coded);
    return status;
}

typedef struct {
    int format;
    const uint16_t *tables;
    const uint64_t *seek;
    const uint8_t *payload;
    uint64_t payload_bytes;
    uint64_t n;
    uint8_t *coded;
    uint32_t err;
    uint64_t k0, k1;
} dec_job;

static void *decode_range(void *arg)
{
    dec_job *j = (dec_job *)arg;
    for (uint64_t k = j->k0; k < j->k1; k++) {
        uint64_t start = k * ORC_CHUNK;
        uint32_t len = (uint32_t)((j->n - start < ORC_CHUNK) ? j->n - start : ORC_CHUNK);
        uint64_t a = j->seek[k], b = j->seek[k + 1];
        if (a > b || b > j->payload_bytes || a % 4 != 0) {
            j->err |= WCO_EF_BAD_SEEK;
            memset(j->coded + start, 0, len);
            continue;
        }
        if ((j->format & WCO_OPT_RAW_FALLBACK) && b - a == raw_chunk_size(len)) {
            /* stored raw: the symbols, then zero padding */
            memcpy(j->coded + start, j->payload + a, len);
            for (uint64_t i = a + len; i < b; i++)
                if (j->payload[i] != 0) j->err |= WCO_EF_BAD_TAIL;
            continue;
        }
        const uint16_t *table = (j->format & WCO_OPT_TENSOR_TABLE) ? j->tables : j->tables + 256 * k;
        uint32_t e = wco_decode_chunk(j->payload + a, b - a, table, len, j->coded + start);
        if (e & (WCO_EF_BAD_TABLE | WCO_EF_BAD_SEEK)) memset(j->coded + start, 0, len);
        j->err |= e;
    }
    return NULL;
}

static void dec_set_range(void *job, uint64_t k0, uint64_t k1)
{
    ((dec_job *)job)->k0 = k0;
    ((dec_job *)job)->k1 = k1;
}

int wco_decode(int dtype, const uint8_t *raw, const uint16_t *tables, const uint64_t *seek,
               const uint8_t *payload, uint64_t payload_bytes, uint64_t n, void *out, int threads,
               uint32_t *err_bits)
{
    if (err_bits) *err_bits = 0;
    int layout = layout_of(dtype);
    if (layout < 0) return WCO_ERR_ARG;
    if (n == 0) return WCO_OK;
    if (!raw || !tables || !seek || !payload || !out) return WCO_ERR_ARG;

    uint64_t chunks = (n + ORC_CHUNK - 1) / ORC_CHUNK;
    uint8_t *coded = (uint8_t *)malloc(n);
    int nthreads = threads < 1 ? 1 : threads;
    uint64_t workers = (uint64_t)nthreads < chunks ? (uint64_t)nthreads : chunks;
    dec_job *jobs = (dec_job *)calloc(workers, sizeof(dec_job));
    for (uint64_t i = 0; i < workers; i++) {
        jobs[i].format = dtype;
        jobs[i].tables = tables;
        jobs[i].seek = seek;
        jobs[i].payload = payload;
        jobs[i].payload_bytes = payload_bytes;
        jobs[i].n = n;
        jobs[i].coded = coded;
    }
    run_ranges(decode_range, jobs, sizeof(dec_job), chunks, (int)workers, dec_set_range);
    uint32_t err = 0;
    for (uint64_t i = 0; i < workers; i++) err |= jobs[i].err;

    if (layout == WCO_FP32)
        wco_merge_fp32(coded, raw, n, (uint32_t *)out);
    else if (is_fp8(layout))
        wco_merge_fp8(layout, coded, raw, n, (uint8_t *)out);
    else
        wco_merge_u16(layout, coded, raw, n, (uint16_t *)out);
    free(jobs);
    free(coded);
    if (err_bits) *err_bits = err;
    return err ? WCO_ERR_CORRUPT : WCO_OK;
}

/* ------------------------------------------------------------------ batches */

int wco_plan_batch(int dtype, const uint64_t *n, uint32_t count, uint64_t *chunk_base,
                   uint64_t *raw_base, wco_layout *total)
{
    if (layout_of(dtype) < 0) return WCO_ERR_ARG;
    uint64_t chunks = 0, raw = 0, cap = 0, elems = 0;
    for (uint32_t i = 0; i < count; i++) {
        wco_layout one;
        wco_query_layout(dtype, n[i], &one);
        if (chunk_base) chunk_base[i] = chunks;
        if (raw_base) raw_base[i] = raw;
        chunks += one.num_chunks;
        raw += one.raw_bytes;
        if (i + 1 < count) raw = (raw + 255) / 256 * 256;
        cap += one.payload_capacity;
        elems += n[i];
    }
    if (total) {
        total->n = elems;
        total->num_chunks = chunks;
        total->raw_bytes = raw;
        total->table_bytes = (dtype & WCO_OPT_TENSOR_TABLE) ? 512 * (uint64_t)count : 512 * chunks;
        total->seek_bytes = 8 * (chunks + 1);
        total->payload_capacity = cap;
    }
    return WCO_OK;
}

int wco_encode_batch(int dtype, const void *const *in, const uint64_t *n, uint32_t count,
                     uint8_t *raw, uint16_t *tables, uint64_t *seek, uint8_t *payload,
                     uint64_t payload_capacity, int threads)
{
    if (layout_of(dtype) < 0) return WCO_ERR_ARG;
    uint64_t *cb = (uint64_t *)malloc(sizeof(uint64_t) * (count + 1));
    uint64_t *rb = (uint64_t *)malloc(sizeof(uint64_t) * (count + 1));
    wco_layout total;
    wco_plan_batch(dtype, n, count, cb, rb, &total);
    if (raw && total.raw_bytes) memset(raw, 0, total.raw_bytes);
    seek[0] = 0;
    int status = WCO_OK;
    for (uint32_t i = 0; i < count && status == WCO_OK; i++) {
        uint64_t base = seek[cb[i]];
        uint64_t c = (n[i] + ORC_CHUNK - 1) / ORC_CHUNK;
        /* tables: tensor i's own table (one per tensor), or its chunks' */
        uint16_t *tab = tables + 256 * ((dtype & WCO_OPT_TENSOR_TABLE) ? i : cb[i]);
        if (c == 0) {
            if (dtype & WCO_OPT_TENSOR_TABLE) memset(tab, 0, 512);
            continue;
        }
        /* the tensor's own seek table starts at 0; shift it by the payload
         * written so far */
        uint64_t *local = (uint64_t *)malloc(sizeof(uint64_t) * (c + 1));
        status = wco_encode(dtype, in[i], n[i], raw + rb[i], tab, local,
                            payload + base, payload_capacity - base, threads);
        for (uint64_t k = 1; k <= c; k++) seek[cb[i] + k] = base + local[k];
        free(local);
    }
    free(cb);
    free(rb);
    return status;
}

int wco_decode_batch(int dtype, void *const *out, const uint64_t *n, uint32_t count,
                     const uint8_t *raw, const uint16_t *tables, const uint64_t *seek,
                     const uint8_t *payload, uint64_t payload_bytes, int threads,
                     uint32_t *err_bits)
{
    if (err_bits) *err_bits = 0;
    if (layout_of(dtype) < 0) return WCO_ERR_ARG;
    uint64_t *cb = (uint64_t *)malloc(sizeof(uint64_t) * (count + 1));
    uint64_t *rb = (uint64_t *)malloc(sizeof(uint64_t) * (count + 1));
    wco_plan_batch(dtype, n, count, cb, rb, NULL);
    uint32_t err = 0;
    for (uint32_t i = 0; i < count; i++) {
        uint64_t c = (n[i] + ORC_CHUNK - 1) / ORC_CHUNK;
        if (c == 0) continue;
        /* re-base this tensor's slice of the seek table at its first chunk */
        uint64_t base = seek[cb[i]];
        uint64_t *local = (uint64_t *)malloc(sizeof(uint64_t) * (c + 1));
        for (uint64_t k = 0; k <= c; k++)
            local[k] = seek[cb[i] + k] >= base ? seek[cb[i] + k] - base : UINT64_MAX;
        uint32_t e = 0;
        uint64_t avail = payload_bytes >= base ? payload_bytes - base : 0;
        if (payload_bytes < base || base % 4 != 0) {
            e = WCO_EF_BAD_SEEK;
        } else {
            wco_decode(dtype, raw + rb[i], tables + 256 * ((dtype & WCO_OPT_TENSOR_TABLE) ? i : cb[i]),
                       local, payload + base, avail, n[i],
                       out[i], threads, &e);
        }
        err |= e;
        free(local);
    }
    free(cb);
    free(rb);
    if (err_bits) *err_bits = err;
    return err ? WCO_ERR_CORRUPT : WCO_OK;
}
