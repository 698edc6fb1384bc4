// wc_crc.hpp -- per-chunk CRC-32 of the payload (format option WC_OPT_CRC32).
//
// The CRC is the common ISO-HDLC / zlib one: polynomial 0x04C11DB7 processed
// least significant bit first (0xEDB88320 reflected), register preset to all
// ones, result complemented.  gfx950 has no carry-less multiply, and a
// byte-serial CRC of a 22 KB chunk would take ~22k dependent table lookups,
// so a chunk is split into 64-byte segments counted from its end, one per
// thread of a 256-thread block:
//   - each thread runs its segments from a zero register with slice-by-4
//     tables in LDS (Kounavis & Berry, "A Systematic Approach to Building
//     High Performance Software-based CRC Generators", 2005): four
//     independent lookups per 4 bytes;
//   - CRC is linear over GF(2): with R(m) the register after m from zero,
//     R(A B) = R(A) x^(8|B|) + R(B) (mod P), so segment s contributes
//     R(segment) x^(512 s), and the block xor-reduces the contributions;
//   - the preset adds ~0 x^(8 size): CRC = R ^ (~0 x^(8 size)) ^ ~0.
// Polynomials are held reflected (bit 31 is the coefficient of x^0); the
// shift constants x^(512 s) and x^(8 2^i) are computed at compile time.
#pragma once

#include "wc_common.hpp"

namespace wc {

constexpr uint32_t kCrcPoly = 0xEDB88320u;

// a b mod P, reflected representation
inline __host__ __device__ constexpr uint32_t gf2_mulmod(uint32_t a, uint32_t b)
{
    uint32_t p = 0;
    for (int i = 0; i < 32; i++) {
        if (a & (0x80000000u >> i)) p ^= b;  // a has x^i: add b x^i
        b = (b & 1u) ? (b >> 1) ^ kCrcPoly : b >> 1;  // b x^i -> b x^(i+1)
    }
    return p;
}

struct CrcConst {
    uint32_t tab[4][256];     // slice-by-4: tab[j][v] = register after byte v then j zero bytes
    uint32_t seg[256];        // x^(8 * 64 * s) mod P
    uint32_t pow2[18];        // x^(8 * 2^i) mod P (payloads are below 2^18 bytes)
};

constexpr CrcConst make_crc_const()
{
    CrcConst c{};
    for (uint32_t v = 0; v < 256; v++) {
        uint32_t r = v;
        for (int b = 0; b < 8; b++) r = (r & 1u) ? (r >> 1) ^ kCrcPoly : r >> 1;
        c.tab[0][v] = r;
    }
    for (uint32_t j = 1; j < 4; j++)
        for (uint32_t v = 0; v < 256; v++) c.tab[j][v] = (c.tab[j - 1][v] >> 8) ^ c.tab[0][c.tab[j - 1][v] & 0xFF];
    c.pow2[0] = 0x80000000u >> 8;  // x^8
    for (int i = 1; i < 18; i++) c.pow2[i] = gf2_mulmod(c.pow2[i - 1], c.pow2[i - 1]);
    c.seg[0] = 0x80000000u;  // x^0
    for (int s = 1; s < 256; s++) c.seg[s] = gf2_mulmod(c.seg[s - 1], c.pow2[6]);  // x^512 per segment
    return c;
}

__device__ const CrcConst kCrc = make_crc_const();

// One block per chunk.  CHECK = false: crc[k] = CRC of chunk k's payload;
// CHECK = true: a mismatch with crc[k] sets WC_EF_BAD_CRC.  A chunk whose
// seek entries are not a valid payload range is left to the decoder, which
// reports it.
template <bool CHECK>
__global__ __launch_bounds__(256) void k_crc32(const uint64_t *__restrict__ seek, const uint8_t *__restrict__ payload,
                                               uint64_t payload_bytes, uint32_t *__restrict__ crc,
                                               uint32_t *__restrict__ err)
{
    __shared__ uint32_t tab[4][256];
    __shared__ uint32_t red[4];
    const uint64_t k = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < 1024; i += 256) (&tab[0][0])[i] = (&kCrc.tab[0][0])[i];
    const uint64_t a = seek[k], b = seek[k + 1];
    __syncthreads();
    if (a > b || b > payload_bytes || (a & 3) || ((b - a) & 3) || b - a > kSlotBytes) return;
    const uint32_t size = (uint32_t)(b - a);
    const WC_GLOBAL uint32_t *w = reinterpret_cast<const WC_GLOBAL uint32_t *>(gptr(payload) + a);
    const uint32_t ns = (size + 63) / 64;
    uint32_t acc = 0;
    uint32_t f = kCrc.seg[tid];
    for (uint32_t s = tid; s < ns; s += 256) {
        // segment s: the 64 bytes (fewer for the first) ending 64 s bytes before the end
        const uint32_t hi = size - 64 * s, lo = hi > 64 ? hi - 64 : 0u;
        uint32_t r = 0;
        for (uint32_t o = lo; o < hi; o += 4) {
            const uint32_t v = r ^ w[o / 4];  // 4 bytes, first in the low byte
            r = tab[3][v & 0xFF] ^ tab[2][(v >> 8) & 0xFF] ^ tab[1][(v >> 16) & 0xFF] ^ tab[0][v >> 24];
        }
        acc ^= gf2_mulmod(r, f);
        f = gf2_mulmod(f, kCrc.pow2[14]);  // the next segment of this thread is 256 segments further
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        uint32_t sh = 0x80000000u;  // x^(8 size)
        for (int i = 0; i < 18; i++)
            if ((size >> i) & 1u) sh = gf2_mulmod(sh, kCrc.pow2[i]);
        const uint32_t c = red[0] ^ red[1] ^ red[2] ^ red[3] ^ gf2_mulmod(0xFFFFFFFFu, sh) ^ 0xFFFFFFFFu;
        if constexpr (CHECK) {
            if (c != crc[k] && err) atomicOr(err, WC_EF_BAD_CRC);
        } else {
            crc[k] = c;
        }
    }
}

}  // namespace wc
