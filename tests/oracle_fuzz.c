/*
 * oracle_fuzz.c -- corrupted streams through the oracle's decoder, built by
 * tests/test_oracle_pyref.py with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only).
 *
 * TEST INFRASTRUCTURE ONLY: it links the oracle (oracle/wc_oracle.c) and
 * nothing else.  Usage: oracle_fuzz TRIALS.  Encodes a BF16 and an FP32
 * tensor of weight-like bit patterns (two full chunks and a ragged one),
 * then decodes TRIALS corrupted copies (a flipped bit in the payload, a
 * truncated payload, an inflated table entry, a moved seek entry, a table
 * of one symbol at 4096, in turn) and counts those that come back as an
 * error or as a tensor different from the input.  A decoder that ever reads
 * or writes out of bounds, or overflows, is stopped by the sanitizers.
 * Prints "detected trials".
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wc_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) */
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint32_t below(uint32_t n) { return (uint32_t)(next_u64() % n); }

/* A weight-like exponent: mostly a few values a step apart, sometimes far. */
static uint32_t exponent(void)
{
    uint32_t e = 120;
    while (below(2) && e > 100) e--;
    if (below(1000) == 0) e = below(256);
    return e;
}

typedef struct {
    int dtype;
    uint64_t n;
    wco_layout lay;
    uint8_t *raw;
    uint16_t *tables;
    uint64_t *seek;
    uint8_t *payload;
    uint64_t payload_bytes;
} enc_t;

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void release(enc_t *e)
{
    free(e->raw);
    free(e->tables);
    free(e->seek);
    free(e->payload);
}

static int encode(int dtype, const void *x, uint64_t n, enc_t *e)
{
    e->dtype = dtype;
    e->n = n;
    if (wco_query_layout(dtype, n, &e->lay) != WCO_OK) return 1;
    e->raw = xmalloc(e->lay.raw_bytes);
    e->tables = xmalloc(e->lay.table_bytes);
    e->seek = xmalloc(e->lay.seek_bytes);
    e->payload = xmalloc(e->lay.payload_capacity);
    if (wco_encode(dtype, x, n, e->raw, e->tables, e->seek, e->payload, e->lay.payload_capacity, 1) != WCO_OK)
        return 1;
    e->payload_bytes = e->seek[e->lay.num_chunks];
    return 0;
}

/* One corrupted decode; returns 1 if the corruption was detected (an error,
 * or an output that differs from x). */
static int trial(const enc_t *e, const void *x, size_t elem, int kind)
{
    const uint64_t chunks = e->lay.num_chunks;
    uint8_t *payload = xmalloc(e->payload_bytes);
    uint16_t *tables = xmalloc(e->lay.table_bytes);
    uint64_t *seek = xmalloc(e->lay.seek_bytes);
    memcpy(payload, e->payload, e->payload_bytes);
    memcpy(tables, e->tables, e->lay.table_bytes);
    memcpy(seek, e->seek, e->lay.seek_bytes);
    uint64_t payload_bytes = e->payload_bytes;
    switch (kind) {
    case 0: {
        const uint64_t i = next_u64() % payload_bytes;
        payload[i] ^= (uint8_t)(1u << below(8));
        break;
    }
    case 1:
        payload_bytes = next_u64() % payload_bytes;
        break;
    case 2: {
        const uint64_t k = next_u64() % chunks;
        const uint32_t s = below(256);
        tables[256 * k + s] = (uint16_t)(tables[256 * k + s] + 1 + below(4));
        break;
    }
    case 3: {
        const uint64_t k = 1 + next_u64() % chunks;
        seek[k] += 4 * (1 + below(1000));
        break;
    }
    default: {
        const uint64_t k = next_u64() % chunks;
        memset(&tables[256 * k], 0, 512);
        tables[256 * k + below(256)] = 4096;
        break;
    }
    }
    void *out = xmalloc(e->n * elem);
    uint32_t bits = 0;
    const int rc = wco_decode(e->dtype, e->raw, tables, seek, payload, payload_bytes, e->n, out, 1, &bits);
    int detected = 1;
    if (rc == WCO_OK) detected = memcmp(out, x, e->n * elem) != 0;
    else if (rc != WCO_ERR_CORRUPT) {
        fprintf(stderr, "unexpected status %d\n", rc);
        exit(3);
    }
    free(out);
    free(payload);
    free(tables);
    free(seek);
    return detected;
}

int main(int argc, char **argv)
{
    const int trials = argc > 1 ? atoi(argv[1]) : 100;
    const uint64_t n = 2 * 65536 + 3333;
    uint16_t *xb = xmalloc(n * 2);
    uint32_t *xf = xmalloc(n * 4);
    for (uint64_t i = 0; i < n; i++) {
        const uint32_t s = below(2), e = exponent();
        xb[i] = (uint16_t)((s << 15) | (e << 7) | below(128));
        xf[i] = (s << 31) | (e << 23) | (uint32_t)(next_u64() & 0x7FFFFF);
    }
    enc_t eb, ef;
    if (encode(WCO_BF16, xb, n, &eb) || encode(WCO_FP32, xf, n, &ef)) {
        fprintf(stderr, "encode failed\n");
        return 1;
    }
    /* the clean streams decode exactly */
    uint32_t bits = 0;
    uint16_t *yb = xmalloc(n * 2);
    if (wco_decode(WCO_BF16, eb.raw, eb.tables, eb.seek, eb.payload, eb.payload_bytes, n, yb, 1, &bits) != WCO_OK ||
        memcmp(yb, xb, n * 2) != 0) {
        fprintf(stderr, "clean round trip failed\n");
        return 1;
    }
    free(yb);
    int detected = 0;
    for (int t = 0; t < trials; t++) {
        const enc_t *e = (t & 1) ? &ef : &eb;
        detected += trial(e, (t & 1) ? (const void *)xf : (const void *)xb, (t & 1) ? 4 : 2, (t / 2) % 5);
    }
    printf("%d %d\n", detected, trials);
    release(&eb);
    release(&ef);
    free(xb);
    free(xf);
    return 0;
}
