// wc_gemm.hpp -- decode fused with its consumer: Y += X W^T computed straight
// from the compressed stream of a BF16 weight matrix W (decompression at
// inference time, the serving side of the Split12 README), on gfx950's
// matrix cores, with no decoded copy of W in HBM.
//
// Tile order.  W (rows x cols, row-major, both multiples of 16) is encoded
// after a permutation into 16 x 16 tiles: panel p holds rows 16p .. 16p+15,
// tile (p, b) its columns 16b .. 16b+15, tiles in the order t = p (cols/16)
// + b, 256 elements each.  Inside a tile, position e (l = e / 8, i = e % 8)
// holds W[16p + l % 16][16b + 4 (l / 16) + 8 (i / 4) + i % 4].  A chunk is
// 256 tiles and one 8-step group of a 32-lane half decodes exactly one tile;
// lane l of the half ends the group with the 8 elements 8l .. 8l+7 joined
// into BF16 (as the plain decoder joins them), which are, with this order,
// the B-operand values of v_mfma_f32_16x16x16_bf16 for wave lanes l
// (i < 4) and l + 32 (i >= 4).  So at the end of a group the two halves of a
// wave swap half their values (two v_permlane32_swap), each
// lane then holds its B operand for both chunks of the wave, and the group
// ends with two MFMAs per 16 rows of X instead of a 16-byte store.
//
// MFMA 16x16x16 bf16 operand layout (wave lane L = 16 j + i, i = L % 16):
// A (16 x 16): lane L holds A[i][4j .. 4j+3]; B (16 x 16): B[4j .. 4j+3][i];
// C / D: D[4j .. 4j+3][i].  Here A = 16 rows of X, B = W_tile^T, D = a
// 16 x 16 block of Y: D[m][n] += sum_k X[m][k] W[n][k].
//
// The X values of a group (8 bytes per lane and tile) are loaded with the
// raw bytes, two groups ahead, from addresses clamped into X so that every
// load of a full group stays unconditional (the decoder's loads are counted
// exactly by the compiler).  Accumulators are kept in registers per (chunk,
// panel); a chunk touches at most P panels.  They are added into Y (fp32
// atomics: a panel can span two chunks) after the chunk's last group, so a
// chunk that the decoder decodes a second time (failed speculation) just
// starts again from zero.
#pragma once

#include "wc_decode.hpp"

namespace wc {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Element s of the tile stream (tile order) <-> element (r, c) of W.
// One thread per 8 elements (lane l of tile t): two 8-byte runs of a row of
// W, one 16-byte run of the stream.
__global__ __launch_bounds__(256) void k_tile_order(const uint16_t *__restrict__ in, uint16_t *__restrict__ out,
                                                    uint32_t rows, uint32_t cols, uint32_t inverse)
{
    const uint64_t id = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint32_t tpp = cols / 16;
    const uint64_t tiles = (uint64_t)(rows / 16) * tpp;
    if (id >= 32 * tiles) return;
    const uint64_t t = id >> 5;
    const uint32_t l = (uint32_t)id & 31;
    const uint64_t p = t / tpp;
    const uint32_t b = (uint32_t)(t - p * tpp);
    const uint64_t m0 = (16 * p + (l & 15)) * cols + 16 * b + 4 * (l >> 4);  // elements m0 .. +3 and m0+8 .. +11
    const uint64_t s0 = 256 * t + 8 * l;
    const WC_GLOBAL uint16_t *src = gptr(in);
    WC_GLOBAL uint16_t *dst = gptr(out);
    if (!inverse) {
        const u32x2 a = *reinterpret_cast<const WC_GLOBAL u32x2 *>(src + m0);
        const u32x2 c = *reinterpret_cast<const WC_GLOBAL u32x2 *>(src + m0 + 8);
        *reinterpret_cast<WC_GLOBAL u32x4 *>(dst + s0) = u32x4{a.x, a.y, c.x, c.y};
    } else {
        const u32x4 v = *reinterpret_cast<const WC_GLOBAL u32x4 *>(src + s0);
        *reinterpret_cast<WC_GLOBAL u32x2 *>(dst + m0) = u32x2{v.x, v.y};
        *reinterpret_cast<WC_GLOBAL u32x2 *>(dst + m0 + 8) = u32x2{v.z, v.w};
    }
}

// One chunk of the wave as every lane of the wave sees it.
struct GemmSide {
    const WC_GLOBAL uint16_t *x;  // X: M x cols BF16
    WC_GLOBAL float *y;           // Y: M x rows fp32
    uint32_t rows, cols;
    uint32_t tpp;                 // tiles per panel, cols / 16
    uint32_t t0;                  // the chunk's first tile
    uint32_t p0;                  // its panel
    uint32_t npan;                // panels the chunk touches
    uint32_t magic, shift;        // t / tpp = mulhi(t << 8, magic) >> shift for t < 2^24
    uint32_t put;                 // its half owns the chunk and decodes it validly
};

// Division of a tile index t < 2^24 by d (1 <= d < 2^28) as a multiply:
// with 2^l >= d and M = ceil(2^(24+l) / d), t M / 2^(24+l) exceeds t / d by
// less than t / 2^(24+l) < 2^-l <= 1/d, too little to reach the next
// integer, so floor(t / d) = (t M) >> (24 + l) = mulhi(t << 8, M) >> l; M
// is below 2^25 + 1.
__device__ __forceinline__ void tile_divisor(uint32_t d, uint32_t &magic, uint32_t &shift)
{
    uint32_t l = 0;
    while ((1u << l) < d) l++;
    magic = (uint32_t)((((uint64_t)1 << (24 + l)) + d - 1) / d);
    shift = l;
}

__device__ __forceinline__ uint32_t xchg32(uint32_t v) { return (uint32_t)__shfl_xor((int)v, 32, 64); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v)
{
    return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v);
}

// The wave-uniform view of one side: every field equal in all 64 lanes
// (held in scalar registers).
__device__ __forceinline__ GemmSide uniform(const GemmSide &a)
{
    GemmSide u;
    u.x = reinterpret_cast<const WC_GLOBAL uint16_t *>(uni64((uint64_t)a.x));
    u.y = reinterpret_cast<WC_GLOBAL float *>(uni64((uint64_t)a.y));
    u.rows = uni(a.rows);
    u.cols = uni(a.cols);
    u.tpp = uni(a.tpp);
    u.t0 = uni(a.t0);
    u.p0 = uni(a.p0);
    u.npan = uni(a.npan);
    u.magic = uni(a.magic);
    u.shift = uni(a.shift);
    u.put = uni(a.put);
    return u;
}

template <int MT, int P, int DT>
struct GemmView {
    static constexpr bool kWave = true;
    using B16 = Bits16<DT>;
    struct Pre {
        u32x2 lo;           // the lane's 8 raw bytes of its own chunk
        u32x2 a[2][MT];     // X operand per chunk of the wave and 16-row block
        uint32_t pi[2];     // panel of the group's tile, relative to the chunk's first
    };
    const WC_GLOBAL uint8_t *lo;
    GemmSide side[2];
    uint32_t my_len, M, L;
    uint32_t xoff[2][MT];
    f32x4_t acc[2][P][MT];

    __device__ void reset()
    {
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int q = 0; q < P; q++)
#pragma unroll
                for (int mt = 0; mt < MT; mt++) acc[h][q][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    __device__ void init(const uint8_t *raw, const wc_segment &sg, uint32_t sidx, uint64_t start, uint32_t len,
                         bool put, const wc_gemm *gm, uint32_t m)
    {
        L = threadIdx.x & 63;
        M = m;
        my_len = len;
        lo = gptr(raw) + sg.raw_base + start;
        const wc_gemm g = gm[sidx];
        const uint32_t tpp = g.cols / 16;
        const uint32_t full = (uint32_t)min((uint64_t)kChunk, sg.n - start);  // the chunk's length
        const uint32_t t0 = (uint32_t)(start / 256);
        const uint32_t t1 = t0 + (full ? (full - 1) / 256 : 0u);
        uint32_t magic, shift;
        tile_divisor(tpp, magic, shift);
        GemmSide me{reinterpret_cast<const WC_GLOBAL uint16_t *>(g.x), reinterpret_cast<WC_GLOBAL float *>(g.y),
                    g.rows, g.cols, tpp, t0, t0 / tpp, t1 / tpp - t0 / tpp + 1, magic, shift, put ? 1u : 0u};
        GemmSide ot;
        ot.x = reinterpret_cast<const WC_GLOBAL uint16_t *>(
            ((uint64_t)xchg32((uint32_t)((uint64_t)me.x >> 32)) << 32) | xchg32((uint32_t)(uint64_t)me.x));
        ot.y = reinterpret_cast<WC_GLOBAL float *>(
            ((uint64_t)xchg32((uint32_t)((uint64_t)me.y >> 32)) << 32) | xchg32((uint32_t)(uint64_t)me.y));
        ot.rows = xchg32(me.rows);
        ot.cols = xchg32(me.cols);
        ot.tpp = xchg32(me.tpp);
        ot.t0 = xchg32(me.t0);
        ot.p0 = xchg32(me.p0);
        ot.npan = xchg32(me.npan);
        ot.magic = xchg32(me.magic);
        ot.shift = xchg32(me.shift);
        ot.put = xchg32(me.put);
        // lane 0 is in half 0: its own side is chunk 0, the exchanged one chunk 1
        side[0] = uniform(me);
        side[1] = uniform(ot);
        // the lane's byte offset into X per side and row block: row 16 mt + i
        // (clamped to the last row: rows past m only feed rows of D that are
        // never added to Y), columns 4j .. 4j+3 of the tile
        const uint32_t i = L & 15, j = L >> 4;
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const uint32_t r = 16 * mt + i < M ? 16 * mt + i : M - 1;
                xoff[h][mt] = 2 * (r * side[h].cols + 4 * j);
            }
        reset();
    }

    // X operands of group g (uniform): the tile's panel (relative to the
    // chunk's first) and column block by scalar arithmetic, then one 8-byte
    // load per side and row block
    __device__ void fetch_x(Pre &p, uint32_t e) const
    {
        const uint32_t g = uni(e >> 8);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const GemmSide &s = side[h];
            const uint32_t t = s.t0 + g;
            const uint32_t q = __umulhi(t << 8, s.magic) >> s.shift;
            const uint32_t kb = t - q * s.tpp;
            p.pi[h] = q - s.p0;
            const WC_GLOBAL uint8_t *base = reinterpret_cast<const WC_GLOBAL uint8_t *>(s.x) + 32 * kb;
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
                p.a[h][mt] = *reinterpret_cast<const WC_GLOBAL u32x2 *>(base + xoff[h][mt]);
        }
    }

    // elements [e, e + 8) of the own chunk's group, e a multiple of 8
    __device__ Pre fetch(uint32_t e) const
    {
        Pre p;
        p.lo = *reinterpret_cast<const WC_GLOBAL u32x2 *>(lo + e);
        fetch_x(p, e);
        return p;
    }
    // the lane's elements of full group g
    __device__ Pre fetch_group(uint32_t g) const { return fetch(kGroupWords * g + 8 * (L & 31)); }
    __device__ Pre fetch_checked(uint32_t e, uint32_t) const
    {
        Pre p;
        p.lo = u32x2{0u, 0u};
        if (e < my_len) p.lo = *reinterpret_cast<const WC_GLOBAL u32x2 *>(lo + e);
        fetch_x(p, e);
        return p;
    }

    __device__ void mma(uint32_t pi_v, int h, const u32x2 (&a)[MT], u32x2 b)
    {
        const uint32_t pi = __builtin_amdgcn_readfirstlane(pi_v);
        bf16x4_t bv;
        __builtin_memcpy(&bv, &b, 8);
#pragma unroll
        for (int q = 0; q < P; q++) {
            if (pi == (uint32_t)q) {
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    bf16x4_t av;
                    __builtin_memcpy(&av, &a[mt], 8);
                    acc[h][q][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc[h][q][mt], 0, 0, 0);
                }
            }
        }
    }

    // join the group's 8 decoded bytes with the raw bytes (zero when the
    // group is not the own chunk's), swap halves, two MFMAs per row block
    __device__ void flush_impl(uint2 sym, const Pre &p, bool have)
    {
        uint32_t d0 = B16::from_coded(__builtin_amdgcn_perm(sym.x, p.lo.x, 0x05010400u));
        uint32_t d1 = B16::from_coded(__builtin_amdgcn_perm(sym.x, p.lo.x, 0x07030602u));
        uint32_t d2 = B16::from_coded(__builtin_amdgcn_perm(sym.y, p.lo.y, 0x05010400u));
        uint32_t d3 = B16::from_coded(__builtin_amdgcn_perm(sym.y, p.lo.y, 0x07030602u));
        if (!have) d0 = d1 = d2 = d3 = 0u;
        // v_permlane32_swap trades lanes 32-63 of its first operand with
        // lanes 0-31 of its second: swapping (d0, d2) and (d1, d3) leaves in
        // the first operand elements 0-3 of half 0's lane l in lane l and its
        // elements 4-7 in lane l + 32 (the B operand of half 0's chunk), and
        // in the second the same for half 1's chunk
        const auto p0 = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
        const auto p1 = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
        const u32x2 b0 = u32x2{p0[0], p1[0]};  // chunk of half 0
        const u32x2 b1 = u32x2{p0[1], p1[1]};  // chunk of half 1
        mma(p.pi[0], 0, p.a[0], b0);
        mma(p.pi[1], 1, p.a[1], b1);
    }
    __device__ void flush(uint32_t, uint2 sym, const Pre &p) { flush_impl(sym, p, true); }
    __device__ void flush_checked(uint32_t e, uint2 sym, const Pre &p, uint32_t)
    {
        flush_impl(sym, p, e < my_len);
    }

    // adds the chunks' blocks of Y (only halves that own a valid chunk)
    __device__ void finish()
    {
        const uint32_t i = L & 15, j = L >> 4;
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const GemmSide &s = side[h];
            if (!s.put) continue;
#pragma unroll
            for (int q = 0; q < P; q++) {
                if ((uint32_t)q >= s.npan) break;
                const uint32_t n = 16 * (s.p0 + q) + i;
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const uint32_t m = 16 * mt + 4 * j + r;
                        if (m < M)
                            unsafeAtomicAdd(reinterpret_cast<float *>((uint64_t)(s.y + (uint64_t)m * s.rows + n)),
                                            acc[h][q][mt][r]);
                    }
                }
            }
        }
    }
};

// Two chunks per wavefront (the narrow-table, one-dword-refill decoder).
template <int DT, int MT, int P>
__global__ __launch_bounds__(64) void k_decode_gemm(SegTable st, const uint8_t *__restrict__ raw,
                                                    const uint16_t *__restrict__ tables,
                                                    const uint64_t *__restrict__ seek,
                                                    const uint8_t *__restrict__ payload, uint64_t payload_bytes,
                                                    uint64_t total_chunks, uint32_t *err, Opts opts,
                                                    const wc_gemm *__restrict__ gm, uint32_t m)
{
    using V = GemmView<MT, P, DT>;
    decode_wave<DT, false, 2, 1, V>(st, tables, seek, payload, payload_bytes, total_chunks, err, opts,
                                    [&](const wc_segment &sg, uint32_t sidx, uint64_t, uint64_t start, uint32_t len,
                                        bool put) {
                                        V v;
                                        v.init(raw, sg, sidx, start, len, put, gm, m);
                                        return v;
                                    });
}

}  // namespace wc
