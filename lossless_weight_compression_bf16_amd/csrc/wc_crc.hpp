// wc_crc.hpp -- per-chunk CRC-32 of the payload (format option WC_OPT_CRC32).
//
// The CRC is the common ISO-HDLC / zlib one: polynomial 0x04C11DB7 processed
// least significant bit first (0xEDB88320 reflected), register preset to all
// ones, result complemented.  gfx950 has no carry-less multiply, and a
// byte-serial CRC of a 22 KB chunk would take ~22k dependent table lookups,
// so a chunk is split into 128-byte segments counted from its end (the one
// holding byte 0 may be shorter), spread over the threads of a 256-thread
// block, 256 segments per round:
//   - the block stages a round's 32 KB through LDS with coalesced loads
//     (padded rows: a thread's segment is read without bank conflicts);
//   - each thread runs its segment with slice-by-4 tables in LDS (Kounavis
//     & Berry, "A Systematic Approach to Building High Performance
//     Software-based CRC Generators", 2005): four independent lookups per
//     4 bytes;
//   - CRC is linear over GF(2): with R_I(m) the register after m from
//     register I, R_I(A B) = R_I(A) x^(8|B|) + R_0(B) (mod P), so segment s
//     (every one after the first is 128 bytes long) contributes its register
//     times x^(1024 s), and the block xor-reduces the contributions; only the
//     first segment (the one holding byte 0) starts from the preset ~0, so
//     the sum is the preset register of the whole payload: CRC = sum ^ ~0.
// A chunk payload is at most kSlotBytes (~128 KB), so a segment is at most
// 1024 segments from the end and its shift takes at most four multiplications
// by the stride (one per 256 segments) after the table lookup.
// Polynomials are held reflected (bit 31 is the coefficient of x^0); the
// shift constants are computed at compile time.
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

constexpr uint32_t kCrcSeg = 128;  // bytes per segment
constexpr uint32_t kCrcDw = kCrcSeg / 4;

struct CrcConst {
    uint32_t tab[4][256];  // slice-by-4: tab[j][v] = register after byte v then j zero bytes
    uint32_t seg[256];     // x^(8 kCrcSeg s) mod P
    uint32_t stride;       // x^(8 kCrcSeg 256) mod P: from a thread's segment to its next
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
    uint32_t pow2[17] = {0x80000000u >> 8};  // x^(8 2^i)
    for (int i = 1; i < 17; i++) pow2[i] = gf2_mulmod(pow2[i - 1], pow2[i - 1]);
    c.seg[0] = 0x80000000u;  // x^0
    for (int s = 1; s < 256; s++) c.seg[s] = gf2_mulmod(c.seg[s - 1], pow2[7]);  // x^(8 128) per segment
    c.stride = pow2[15];                                                        // x^(8 128 256)
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
    constexpr uint32_t kRow = kCrcDw + 1;  // padded LDS row of one segment
    __shared__ uint32_t tab[4][256];
    __shared__ uint32_t stage[256 * kRow];
    __shared__ uint32_t red[4];
    const uint64_t k = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < 1024; i += 256) (&tab[0][0])[i] = (&kCrc.tab[0][0])[i];
    const uint64_t a = seek[k], b = seek[k + 1];
    if (a > b || b > payload_bytes || (a & 3) || ((b - a) & 3) || b - a > kSlotBytes) return;
    const uint32_t size = (uint32_t)(b - a);
    const WC_GLOBAL uint32_t *w = reinterpret_cast<const WC_GLOBAL uint32_t *>(gptr(payload) + a);
    const uint32_t ns = (size + kCrcSeg - 1) / kCrcSeg;
    // Segments are numbered q = 0 .. ns-1 from the start; segment q holds the
    // dwords v - pad for v in [kCrcDw q, kCrcDw (q+1)), where the pad dwords
    // before byte 0 (v < pad) do not exist.  Segment q ends kCrcSeg (ns-1-q)
    // bytes before the end of the payload.
    const uint32_t nd = size / 4, pad = kCrcDw * ns - nd;
    uint32_t acc = 0;
    for (uint32_t q0 = 0; q0 < ns; q0 += 256) {
        __syncthreads();  // tables written / previous round's stage read
#pragma unroll
        for (uint32_t j = 0; j < kCrcDw; j++) {
            const uint32_t t = tid + 256 * j;        // dword of this round
            const uint32_t v = kCrcDw * q0 + t;      // dword counted from the first segment's start
            const bool ok = v >= pad && v - pad < nd;
            const uint32_t x = w[ok ? v - pad : 0u];  // nd > 0 here: index 0 is in bounds
            stage[(t / kCrcDw) * kRow + t % kCrcDw] = ok ? x : 0u;
        }
        __syncthreads();
        const uint32_t q = q0 + tid;
        if (q < ns) {
            const uint32_t *row = stage + tid * kRow;
            const uint32_t skip = q == 0 ? pad : 0u;  // the first segment starts at byte 0 ...
            uint32_t r = q == 0 ? 0xFFFFFFFFu : 0u;   // ... from the preset register
#pragma unroll
            for (uint32_t i = 0; i < kCrcDw; i++) {
                const uint32_t v = r ^ row[i];  // 4 bytes, first in the low byte
                const uint32_t n = tab[3][v & 0xFF] ^ tab[2][(v >> 8) & 0xFF] ^ tab[1][(v >> 16) & 0xFF] ^ tab[0][v >> 24];
                r = i < skip ? r : n;
            }
            const uint32_t s = ns - 1 - q;  // kCrcSeg-byte segments after this one
            uint32_t f = kCrc.seg[s & 255];
            for (uint32_t h = s >> 8; h; h--) f = gf2_mulmod(f, kCrc.stride);
            acc ^= gf2_mulmod(r, f);
        }
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        // an empty payload (never written by the encoder) has the CRC 0
        const uint32_t c = size ? red[0] ^ red[1] ^ red[2] ^ red[3] ^ 0xFFFFFFFFu : 0u;
        if constexpr (CHECK) {
            if (c != crc[k] && err) atomicOr(err, WC_EF_BAD_CRC);
        } else {
            crc[k] = c;
        }
    }
}

}  // namespace wc
