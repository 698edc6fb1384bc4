// wc_decode.hpp -- fused decoder for gfx950.
//
// One wavefront decodes two chunks, one per 32-lane half, so every VALU
// instruction of the serial rANS loop carries 64 useful lanes.  Per half the
// LDS holds the chunk's slot -> symbol table (4096 bytes), its per-symbol
// (f, b) pairs (256 u32) and a 1024-word ring of the compressed stream that
// is refilled 256 words at a time, one group of 8 steps ahead, so the word
// fetch of a step is an LDS read instead of a dependent HBM load.  Each step
// of a half decodes 32 consecutive elements; the decoded byte is joined with
// the raw plane (BF16: the low byte) and written straight to the output
// tensor, 64 contiguous bytes per half per step.
#pragma once

#include "wc_common.hpp"

namespace wc {

constexpr uint32_t kRingWords = 1024;     // per half
constexpr uint32_t kRefillWords = 256;    // one refill: 32 lanes x 16 bytes
constexpr uint32_t kGroup = 8;            // steps between refill decisions

struct DecShared {
    uint32_t sym[2][kM / 4];              // slot -> symbol, 4 slots per word (LDS offset 0)
    uint32_t ring[2][kRingWords / 2];     // compressed words, 2 per u32
    uint32_t fb[2][256];                  // b | (f - 4096) << 16
};

// Raw-plane bytes one lane needs for one element, and the output write.
template <int DT>
struct RawView;

template <>
struct RawView<WC_BF16> {
    const WC_GLOBAL uint8_t *lo;
    WC_GLOBAL uint16_t *out;
    __device__ void init(const uint8_t *raw, const wc_segment &sg, uint64_t start)
    {
        lo = gptr(raw) + sg.raw_base + start;
        out = gptr<uint16_t>(sg.ptr) + start;
    }
    struct Pre {
        uint32_t v;
    };
    __device__ Pre fetch(uint32_t j) const { return Pre{lo[j]}; }
    __device__ void put(uint32_t j, uint32_t s, const Pre &p) const { out[j] = (uint16_t)((s << 8) | p.v); }
};

template <>
struct RawView<WC_FP32> {
    const WC_GLOBAL uint8_t *sign, *m0, *m1, *m2;
    WC_GLOBAL uint32_t *out;
    __device__ void init(const uint8_t *raw, const wc_segment &sg, uint64_t start)
    {
        const uint64_t sb = (sg.n + 7) / 8;
        sign = gptr(raw) + sg.raw_base + start / 8;
        m0 = gptr(raw) + sg.raw_base + sb + start;
        m1 = m0 + sg.n;
        m2 = m1 + sg.n;
        out = gptr<uint32_t>(sg.ptr) + start;
    }
    struct Pre {
        uint32_t v;
    };
    __device__ Pre fetch(uint32_t j) const
    {
        const uint32_t sbit = (sign[j >> 3] >> (j & 7)) & 1u;
        return Pre{(sbit << 31) | ((uint32_t)m2[j] << 16) | ((uint32_t)m1[j] << 8) | m0[j]};
    }
    __device__ void put(uint32_t j, uint32_t s, const Pre &p) const { out[j] = p.v | (s << 23); }
};

// The ring is written and read by lanes of the same wavefront.  LDS requests
// of one wavefront are served in issue order, so only the compiler has to be
// kept from moving the reads of the next group above the refill's writes.
__device__ inline void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Per-half stream cursor.  All values are uniform within a half.
struct Stream {
    const uint32_t *words;  // payload + seek[k] + 128, as dwords
    uint32_t nw;            // words in the chunk (pad included, even)
    uint32_t ptr;           // next word to consume
    uint32_t fill;          // words written to the ring so far
};

// Starts a refill of 256 words if the ring runs low; returns whether it did.
__device__ inline bool refill_issue(const Stream &st, uint32_t lane, bool on, uint4 &v)
{
    const bool go = on && st.fill - st.ptr < 2 * kRefillWords && st.fill < st.nw;
    if (go) {
        const uint32_t d0 = st.fill / 2 + 4 * lane, ndw = st.nw / 2;
        const WC_GLOBAL uint32_t *w = gptr(st.words) + d0;
        if (d0 + 4 <= ndw) {
            v.x = w[0];
            v.y = w[1];
            v.z = w[2];
            v.w = w[3];
        } else {
            v.x = d0 + 0 < ndw ? w[0] : 0u;
            v.y = d0 + 1 < ndw ? w[1] : 0u;
            v.z = d0 + 2 < ndw ? w[2] : 0u;
            v.w = 0u;  // ndw - d0 < 4 here
        }
    }
    return go;
}

__device__ inline void refill_commit(Stream &st, uint32_t lane, bool go, const uint4 &v, uint32_t *ring)
{
    if (go) {
        const uint32_t d0 = (st.fill / 2 + 4 * lane) & (kRingWords / 2 - 1);
        *reinterpret_cast<uint4 *>(ring + d0) = v;
        st.fill += kRefillWords;
    }
}

// One decode step for one lane.  With x = 4096 (x >> 12) + slot,
// f (x >> 12) + slot - b  ==  x - b + (f - 4096) (x >> 12)  (mod 2^32),
// one signed 24-bit multiply-add with the table's (f - 4096).
template <int DT, bool CHECK>
__device__ inline void dec_step(uint32_t &x, uint32_t &ptr, const DecShared &sh, uint32_t h, bool active,
                                const RawView<DT> &rv, uint32_t j, const typename RawView<DT>::Pre &pre)
{
    const uint8_t *sym = reinterpret_cast<const uint8_t *>(&sh.sym[0][0]);
    const uint32_t s = sym[(x & (kM - 1)) | (h << 12)];
    const uint32_t fb = sh.fb[h][s];
    const uint32_t xd = (uint32_t)__mul24((int32_t)fb >> 16, (int32_t)(x >> kScaleBits)) + (x - (fb & 0xFFFF));
    const bool need = (!CHECK || active) && xd < kL;
    const uint64_t m = __ballot(need);
    const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
    // rank among the half's renormalising lanes, added to the half's cursor
    const uint32_t widx = __builtin_amdgcn_mbcnt_hi(mh, __builtin_amdgcn_mbcnt_lo(h ? 0u : ml, ptr));
    const uint16_t *ring = reinterpret_cast<const uint16_t *>(&sh.ring[0][0]);
    const uint32_t w = ring[(widx & (kRingWords - 1)) | (h << 10)];
    ptr += __popc(h ? mh : ml);
    if (!CHECK || active) {
        x = need ? (xd << 16) | w : xd;
        rv.put(j, s, pre);
    }
}

template <int DT>
__global__ __launch_bounds__(64) void k_decode(SegTable st, const uint8_t *__restrict__ raw,
                                               const uint16_t *__restrict__ tables,
                                               const uint64_t *__restrict__ seek,
                                               const uint8_t *__restrict__ payload,
                                               uint64_t payload_bytes, uint64_t total_chunks,
                                               uint32_t *err)
{
    __shared__ DecShared sh;
    const uint32_t lane = threadIdx.x & 31, h = threadIdx.x >> 5;
    const uint64_t k = 2ull * blockIdx.x + h;
    bool ok = k < total_chunks;
    uint32_t bits = 0;

    wc_segment sg{0, 0, 0, 0};
    uint64_t start = 0;
    uint32_t len = 0;
    Stream cs{nullptr, 0, 0, 0};
    uint32_t x = kL;
    if (ok) {
        sg = find_segment(st, k);
        start = (k - sg.chunk_base) * kChunk;
        len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
        const uint64_t a = seek[k], b = seek[k + 1];
        if (a > b || b > payload_bytes || b - a < 128 || ((b - a) & 3) || (a & 3)) {
            bits |= WC_EF_BAD_SEEK;
            ok = false;
        } else {
            cs.words = reinterpret_cast<const uint32_t *>(payload + a + 128);
            cs.nw = (uint32_t)min<uint64_t>((b - a - 128) / 2, 2ull * kMaxWords + 2);
            x = reinterpret_cast<const uint32_t *>(payload + a)[lane];
        }
    }
    // table: 8 symbols per lane, validated (sum 4096) before it is used
    uint32_t f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) {
        const uint4 fv = reinterpret_cast<const uint4 *>(tables + k * 256)[lane];
        f[0] = fv.x & 0xFFFF; f[1] = fv.x >> 16; f[2] = fv.y & 0xFFFF; f[3] = fv.y >> 16;
        f[4] = fv.z & 0xFFFF; f[5] = fv.z >> 16; f[6] = fv.w & 0xFFFF; f[7] = fv.w >> 16;
    }
    uint32_t local = 0;
    for (int i = 0; i < 8; i++) local += f[i];
    uint32_t incl = local;
    for (int o = 1; o < 32; o <<= 1) {
        uint32_t v = __shfl_up(incl, o, 32);
        if (lane >= (uint32_t)o) incl += v;
    }
    const uint32_t fsum = __shfl(incl, 31, 32);
    if (ok && fsum != kM) {
        bits |= WC_EF_BAD_TABLE;
        ok = false;
    }
    if (ok) {
        uint32_t b = incl - local;
        for (int i = 0; i < 8; i++) {
            sh.fb[h][8 * lane + i] = (b & 0xFFFF) | ((f[i] - kM) << 16);
            b += f[i];
        }
    }
    __syncthreads();
    if (ok) {
        // slots [128 lane, 128 lane + 128): owner of a slot = the last symbol
        // whose start b is <= slot; walk forward from a binary search.
        const uint32_t s0 = 128 * lane;
        uint32_t lo = 0, hi = 256;
        // b of symbol t from the packed table (b <= 4096 fits 16 bits)
        auto bstart = [&](uint32_t t) -> uint32_t { return sh.fb[h][t] & 0xFFFF; };
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (bstart(mid) <= s0) lo = mid; else hi = mid;
        }
        uint32_t s = lo;
        uint32_t nb = s < 255 ? bstart(s + 1) : kM;
        for (uint32_t q = 0; q < 32; q++) {
            uint32_t word = 0;
            for (uint32_t i = 0; i < 4; i++) {
                const uint32_t slot = s0 + 4 * q + i;
                while (slot >= nb) {
                    s++;
                    nb = s < 255 ? bstart(s + 1) : kM;
                }
                word |= s << (8 * i);
            }
            sh.sym[h][32 * lane + q] = word;
        }
    }
    // initial ring fill: two refills
    for (int r = 0; r < 2; r++) {
        uint4 v;
        const bool go = refill_issue(cs, lane, ok, v);
        refill_commit(cs, lane, go, v, sh.ring[h]);
    }
    __syncthreads();

    RawView<DT> rv;
    if (ok) rv.init(raw, sg, start);

    const uint32_t other_len = __shfl_xor(ok ? len : 0u, 32, 64);
    const bool full = ok && len == kChunk && other_len == kChunk;
    using Pre = typename RawView<DT>::Pre;
    if (full) {
        constexpr uint32_t kSteps = kChunk / kLanes;
        Pre cur[kGroup], nxt[kGroup];
#pragma unroll
        for (uint32_t i = 0; i < kGroup; i++) cur[i] = rv.fetch(32 * i + lane);
        for (uint32_t t0 = 0; t0 < kSteps; t0 += kGroup) {
            uint4 v;
            const bool go = refill_issue(cs, lane, true, v);
            // next group's raw bytes (the last group re-reads its own: no branch)
            const uint32_t tn = t0 + kGroup < kSteps ? t0 + kGroup : t0;
#pragma unroll
            for (uint32_t i = 0; i < kGroup; i++) nxt[i] = rv.fetch(32 * (tn + i) + lane);
#pragma unroll
            for (uint32_t i = 0; i < kGroup; i++)
                dec_step<DT, false>(x, cs.ptr, sh, h, true, rv, 32 * (t0 + i) + lane, cur[i]);
            refill_commit(cs, lane, go, v, sh.ring[h]);
            wave_lds_order();
#pragma unroll
            for (uint32_t i = 0; i < kGroup; i++) cur[i] = nxt[i];
        }
    } else {
        const uint32_t steps = ok ? (len + kLanes - 1) / kLanes : 0;
        const uint32_t other = __shfl_xor(steps, 32, 64);
        const uint32_t smax = steps > other ? steps : other;
        for (uint32_t t0 = 0; t0 < smax; t0 += kGroup) {
            uint4 v;
            const bool go = refill_issue(cs, lane, ok, v);
            for (uint32_t i = 0; i < kGroup; i++) {
                const uint32_t j = 32 * (t0 + i) + lane;
                const bool active = ok && j < len;
                Pre pre{0};
                if (active) pre = rv.fetch(j);
                dec_step<DT, true>(x, cs.ptr, sh, h, active, rv, j, pre);
            }
            refill_commit(cs, lane, go, v, sh.ring[h]);
            wave_lds_order();
        }
    }

    if (ok) {
        if (cs.ptr > cs.nw) {
            bits |= WC_EF_WORD_OVERRUN;
        } else if (cs.nw - cs.ptr > 1) {
            bits |= WC_EF_BAD_TAIL;
        } else if (cs.nw - cs.ptr == 1) {
            const uint32_t last = cs.words[cs.ptr >> 1];
            if ((cs.ptr & 1 ? last >> 16 : last & 0xFFFF) != 0) bits |= WC_EF_BAD_TAIL;
        }
        if (x != kL) bits |= WC_EF_BAD_FINAL_STATE;
    }
    // OR the half's bits into lane 0 of the half
    for (int o = 16; o > 0; o >>= 1) bits |= __shfl_xor(bits, o, 32);
    if (lane == 0 && bits && err) atomicOr(err, bits);
}

}  // namespace wc
