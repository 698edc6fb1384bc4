// wc_common.hpp -- constants and small device helpers of the gfx950 codec.
//
// Format constants (the pages name rANS but fix none of its parameters; these
// are the format's own choices, restated in the public header wc.h):
//   chunk = 65536 symbols, 32 interleaved u32 states per chunk, 12-bit
//   frequency tables (M = 4096), state lower bound L = 2^16, 16-bit
//   renormalisation words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wc.h"

namespace wc {

constexpr uint32_t kChunk = 65536;
constexpr uint32_t kLanes = 32;
constexpr uint32_t kScaleBits = 12;
constexpr uint32_t kM = 1u << kScaleBits;
constexpr uint32_t kL = 1u << 16;
constexpr uint32_t kMaxWords = kChunk;                  // at most one word per symbol
constexpr uint64_t kSlotBytes = 128 + 2ull * kMaxWords;   // encoder scratch per chunk
// Most words one group of 8 steps of one half consumes (decoder) or writes
// (encoder).  The decoder checks that every stored state is at least
// L = 2^16; then every state stays in [L, 2^32): a step gives
// x' = f q + slot - b >= f q >= 16 f (q = x >> 12 >= 16), and a renormalised
// state x' 2^16 + w is at least 16 f 2^16.  So a lane that renormalises at
// steps t, t+1, ... has x'_t >= 16 f_t, q_(t+1) >= 256 f_t,
// x'_(t+1) >= 256 f_t f_(t+1), ..., x'_(t+3) >= 2^16 f_t f_(t+1) f_(t+2)
// f_(t+3) >= 2^16: four renormalisations in a row are impossible, and a
// lane takes at most 6 words in 8 steps.  The encoder's states, read
// backwards, are the decoder's states for the stream it writes (its final
// states are in [L, 2^32)), so it writes a word exactly where the decoder
// takes one and is held to the same bound.
constexpr uint32_t kGroupMaxWords = 6 * kLanes;
constexpr uint64_t kMaxElems = 1ull << 40;

inline __host__ __device__ uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

inline __host__ __device__ constexpr bool is_fp8(int layout) { return layout == WC_FP8_E4M3 || layout == WC_FP8_E5M2; }

// Raw plane bytes of n elements: one raw byte per element for the 16-bit
// layouts; sign bits plus three mantissa bytes for FP32; a nibble per
// element for FP8.
inline __host__ __device__ uint64_t raw_bytes_of(int layout, uint64_t n)
{
    if (layout == WC_FP32) return (n + 7) / 8 + 3 * n;
    if (is_fp8(layout)) return (n + 1) / 2;
    return n;
}

// Payload of a chunk of len symbols stored raw (WC_OPT_RAW_FALLBACK).
inline __host__ __device__ uint32_t raw_chunk_bytes(uint32_t len) { return (len + 3u) & ~3u; }

// The 16-bit layouts.  Their coded byte is the high byte and their raw byte
// the low byte of a rearrangement of the value's 16 bits: none for BF16 and
// FP16; for the _REORDER layouts the bit reorder of the "PTWM" README ("How
// it works", step 1), which moves the exponent field to the top and the sign
// right below it, i.e. rotates the sign + exponent field left by one bit.
// Both directions work on two values packed in a u32 (a shift pair and two
// bit selects); a lone value zero-extended to 32 bits stays below 2^16.
inline __host__ __device__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

template <int DT>
struct Bits16 {
    __host__ __device__ static uint32_t to_coded(uint32_t v) { return v; }
    __host__ __device__ static uint32_t from_coded(uint32_t t) { return t; }
};

// s e8 m7 <-> e8 s m7
template <>
struct Bits16<WC_BF16_REORDER> {
    __host__ __device__ static uint32_t to_coded(uint32_t v)
    {
        return bitsel(0x007F007Fu, v, bitsel(0x00800080u, v >> 8, v << 1));
    }
    __host__ __device__ static uint32_t from_coded(uint32_t t)
    {
        return bitsel(0x007F007Fu, t, bitsel(0x80008000u, t << 8, t >> 1));
    }
};

// s e5 m10 <-> e5 s m10
template <>
struct Bits16<WC_FP16_REORDER> {
    __host__ __device__ static uint32_t to_coded(uint32_t v)
    {
        return bitsel(0x03FF03FFu, v, bitsel(0x04000400u, v >> 5, v << 1));
    }
    __host__ __device__ static uint32_t from_coded(uint32_t t)
    {
        return bitsel(0x03FF03FFu, t, bitsel(0x80008000u, t << 5, t >> 1));
    }
};

// FP8 layouts: the same reorder within each byte (the "PTWM" README: the
// exponent moves into the high nibble, the sign right below it), on four
// bytes packed in a u32.
template <int DT>
struct Bits8;

// s e4 m3 <-> e4 s m3
template <>
struct Bits8<WC_FP8_E4M3> {
    __host__ __device__ static uint32_t to_coded(uint32_t v)
    {
        return bitsel(0x07070707u, v, bitsel(0x08080808u, v >> 4, v << 1));
    }
    __host__ __device__ static uint32_t from_coded(uint32_t t)
    {
        return bitsel(0x07070707u, t, bitsel(0x80808080u, t << 4, t >> 1));
    }
};

// s e5 m2 <-> e5 s m2
template <>
struct Bits8<WC_FP8_E5M2> {
    __host__ __device__ static uint32_t to_coded(uint32_t v)
    {
        return bitsel(0x03030303u, v, bitsel(0x04040404u, v >> 5, v << 1));
    }
    __host__ __device__ static uint32_t from_coded(uint32_t t)
    {
        return bitsel(0x03030303u, t, bitsel(0x80808080u, t << 5, t >> 1));
    }
};

// Kernel options (the option bits of the format word, passed as a uniform
// kernel argument).
struct Opts {
    uint32_t bits;
    __host__ __device__ bool tensor_table() const { return bits & WC_OPT_TENSOR_TABLE; }
    __host__ __device__ bool raw_fallback() const { return bits & WC_OPT_RAW_FALLBACK; }
    __host__ __device__ bool crc() const { return bits & WC_OPT_CRC32; }
};

// Device addresses held as integers (segment tables) are always global
// memory; saying so lets the compiler emit global_* instead of flat_*
// accesses, whose completion would otherwise also count against LDS waits.
#define WC_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ inline WC_GLOBAL T *gptr(uint64_t a)
{
    return reinterpret_cast<WC_GLOBAL T *>(a);
}
template <typename T>
__device__ inline WC_GLOBAL T *gptr(T *p)
{
    return reinterpret_cast<WC_GLOBAL T *>(reinterpret_cast<uint64_t>(p));
}

// Native 16-byte vector (loads as one global_load_dwordx4).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Segment view handed to every kernel: either one inline tensor (nseg == 0)
// or a device array of planned segments.
struct SegTable {
    const wc_segment *segs;
    uint32_t nseg;
    wc_segment single;
};

// The segment that owns global chunk k: the last one whose chunk_base <= k
// (empty segments share their chunk_base with the next one and are skipped).
// idx receives its index (0 for a single tensor): its table with
// WC_OPT_TENSOR_TABLE.
__device__ inline wc_segment find_segment(const SegTable &st, uint64_t k, uint32_t *idx = nullptr)
{
    if (st.nseg == 0) {
        if (idx) *idx = 0;
        return st.single;
    }
    uint32_t lo = 0, hi = st.nseg;
    while (hi - lo > 1) {
        uint32_t mid = (lo + hi) >> 1;
        if (st.segs[mid].chunk_base <= k) lo = mid; else hi = mid;
    }
    if (idx) *idx = lo;
    return st.segs[lo];
}

// ---------------------------------------------------------------------------
// Exact unsigned division by an invariant divisor d in [1, 4096] for any
// 32-bit dividend: Granlund & Montgomery, "Division by Invariant Integers
// using Multiplication" (PLDI 1994), the round-up method with an N+1-bit
// multiplier (their Figure 4.1): l = ceil(log2 d),
// m' = floor(2^32 (2^l - d) / d) + 1, sh1 = min(l, 1), sh2 = max(l - 1, 0),
// q = (t1 + ((x - t1) >> sh1)) >> sh2 with t1 = mulhi(m', x).
// gfx950 has no integer divide instruction; this is one mul_hi, a subtract,
// an add and two shifts.
// ---------------------------------------------------------------------------
struct DivConst {
    uint32_t mp;
    uint32_t sh1;
    uint32_t sh2;
};

inline __host__ __device__ DivConst div_const(uint32_t d)
{
    uint32_t l = 0;
    while ((1u << l) < d) l++;
    DivConst c;
    c.mp = (uint32_t)((((uint64_t)((1u << l) - d)) << 32) / d) + 1u;
    c.sh1 = l < 1 ? l : 1;
    c.sh2 = l > 1 ? l - 1 : 0;
    return c;
}

// The constants for every divisor 1..4096, built at compile time (the encoder
// looks them up per symbol instead of dividing 64-bit numbers on the GPU).
struct DivTable {
    uint32_t mp[kM + 1];
    uint8_t l[kM + 1];  // ceil(log2 d); sh1 = min(l, 1), sh2 = max(l - 1, 0)
};

constexpr DivTable make_div_table()
{
    DivTable t{};
    for (uint32_t d = 1; d <= kM; d++) {
        uint32_t l = 0;
        while ((1u << l) < d) l++;
        t.mp[d] = (uint32_t)((((uint64_t)((1u << l) - d)) << 32) / d) + 1u;
        t.l[d] = (uint8_t)l;
    }
    return t;
}

__device__ const DivTable kDivTable = make_div_table();

inline __host__ __device__ uint32_t mulhi32(uint32_t a, uint32_t b)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __umulhi(a, b);
#else
    return (uint32_t)(((uint64_t)a * b) >> 32);
#endif
}

inline __host__ __device__ uint32_t div_exact(uint32_t x, uint32_t mp, uint32_t sh1, uint32_t sh2)
{
    uint32_t t1 = mulhi32(mp, x);
    return (t1 + ((x - t1) >> sh1)) >> sh2;
}

// The encoder's state update for a symbol of frequency f and start b:
// x' = 4096 floor(xr / f) + (xr mod f) + b = xr + q (4096 - f) + b, for
// 1 <= xr < f 2^20 (a state is at least 2^16, so even a renormalised xr is
// at least 1).  q comes from one multiply-high and two right shifts, the
// first by the constant 1: for f >= 2 the round-up reciprocal's sh1 is 1 and
// q is the exact quotient; for f = 1 the reciprocal 2^32 - 1 gives
// q = xr - 1 (exact for xr >= 1), and a start raised by 4095 puts the
// missing 4095 back.  Packed per symbol as {mp, fm = sh2 | (4096 - f) << 16,
// bb}: the second shift takes fm's low 5 bits as they stand and the
// multiply its high half.
struct EncConst {
    uint32_t mp, fm, bb;
};

inline __host__ __device__ EncConst enc_const(uint32_t mp, uint32_t l, uint32_t f, uint32_t b)
{
    EncConst c;
    c.mp = f == 1 ? 0xFFFFFFFFu : mp;
    c.fm = (l > 1 ? l - 1 : 0u) | (kM - f) << 16;
    c.bb = f == 1 ? b + (kM - 1) : b;
    return c;
}

inline __host__ __device__ uint32_t enc_update(uint32_t xr, uint32_t mp, uint32_t fm, uint32_t bb)
{
    const uint32_t t1 = mulhi32(mp, xr);
    const uint32_t q = (t1 + ((xr - t1) >> 1)) >> (fm & 31u);  // below 2^20
#if defined(__HIP_DEVICE_COMPILE__)
    return xr + __umul24(q, fm >> 16) + bb;
#else
    return xr + q * (fm >> 16) + bb;
#endif
}

// ---------------------------------------------------------------------------
// Wavefront helpers (wave64).
// ---------------------------------------------------------------------------
// The GPU hands consecutive workgroups to its 8 XCDs in turn; this maps
// block b to slot start(b mod 8) + b / 8, where the grid's slots are cut
// into 8 consecutive ranges (the first gridDim.x mod 8 one longer), so each
// XCD works through one contiguous range.  A bijection on [0, gridDim.x) for
// any grid size: results never depend on the dispatch order.
__device__ inline uint32_t xcd_block()
{
    const uint32_t b = blockIdx.x, G = gridDim.x, per = G >> 3, rem = G & 7, xc = b & 7, i = b >> 3;
    return (xc < rem ? xc * (per + 1) : rem * (per + 1) + (xc - rem) * per) + i;
}

__device__ inline uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ inline uint32_t wave_sum(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// LDS requests of one wavefront are served in issue order, so data that one
// lane writes to LDS is visible to a later read by another lane of the same
// wavefront; only the compiler has to be kept from moving LDS accesses
// across these points.
__device__ inline void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

}  // namespace wc
