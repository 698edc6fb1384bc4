// wc_encode.hpp -- encoder kernels for gfx950.
//
//   k_split_hist  one 256-thread block per chunk: coalesced 16-byte loads of
//                 the tensor, raw planes written back with vector stores, the
//                 coded plane counted into LDS sub-histograms, then the
//                 chunk's 12-bit table built with integer arithmetic only.
//   k_encode      one wavefront per two chunks (one chunk per 32-lane half):
//                 32 interleaved rANS states, reverse order, words written
//                 downwards into the chunk's scratch slot.
//   k_scan        exclusive scan of the chunk sizes into the seek table.
//   k_compact     moves every chunk's payload from its slot to its offset.
#pragma once

#include <type_traits>

#include "wc_common.hpp"

namespace wc {

// ------------------------------------------------------------ block helpers
// (256 threads = 4 wavefronts)

__device__ inline uint32_t block_sum256(uint32_t v, uint32_t *red)
{
    const uint32_t w = threadIdx.x >> 6;
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    uint32_t r = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return r;
}

// Exclusive prefix count of a predicate over the block, in thread order.
__device__ inline uint32_t block_rank256(bool p, uint32_t *red, uint32_t *total)
{
    const uint32_t w = threadIdx.x >> 6;
    uint64_t m = __ballot(p);
    uint32_t in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if ((threadIdx.x & 63) == 0) red[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (uint32_t i = 0; i < 4; i++) {
        uint32_t c = red[i];
        off += i < w ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return off + in_wave;
}

// Normalises the chunk's counts to a 12-bit table.  Thread s holds count c
// of symbol s; T is the chunk length.  Integer largest-remainder rounding:
// f = floor(4096 c / T), at least 1 when c > 0; a positive shortfall D goes
// +1 to the D regular symbols with the largest remainders (smaller symbol
// first on ties); an excess E = -D is removed the way "take 1 from the
// largest f, smaller symbol on ties" repeated E times would remove it,
// computed in closed form: every f is cut to a level v+1 and the smallest
// symbols at that level drop to v, where v is the largest level whose cut
// removes at least E.
__device__ inline uint32_t normalize256(uint32_t c, uint32_t T, uint32_t *red, uint32_t *keys)
{
    const uint32_t s = threadIdx.x;
    const uint32_t scaled = c * kM;  // <= 2^28
    const uint32_t q = scaled / T;
    const uint32_t r = scaled - q * T;
    const bool regular = q >= 1;
    uint32_t f = c ? (regular ? q : 1u) : 0u;
    const int32_t d = (int32_t)kM - (int32_t)block_sum256(f, red);

    if (d > 0) {
        uint32_t m;
        uint32_t pos = block_rank256(regular, red, &m);
        const uint32_t key = r * 256u + (255u - s);  // r < 65536: unique, fits 24 bits
        if (regular) keys[pos] = key;
        __syncthreads();
        if (regular) {
            uint32_t rank = 0;
            for (uint32_t i = 0; i < m; i++) rank += keys[i] > key ? 1u : 0u;
            if (rank < (uint32_t)d) f += 1;
        }
        __syncthreads();
    } else if (d < 0) {
        const uint32_t e = (uint32_t)(-d);
        // cost(v) = sum max(f - v, 0) is non-increasing; cost(1) >= e and
        // cost(4096) = 0 < e, so the largest v with cost(v) >= e is in [1, 4096).
        uint32_t lo = 1, hi = kM;
        while (hi - lo > 1) {
            uint32_t mid = (lo + hi) >> 1;
            uint32_t cost = block_sum256(f > mid ? f - mid : 0u, red);
            if (cost >= e) lo = mid; else hi = mid;
        }
        const uint32_t v = lo;
        const uint32_t cut = block_sum256(f > v + 1 ? f - (v + 1) : 0u, red);
        const uint32_t left = e - cut;
        const bool at = f >= v + 1;
        uint32_t m;
        uint32_t pos = block_rank256(at, red, &m);
        if (at) f = pos < left ? v : v + 1;
    }
    return f;
}

// ------------------------------------------------------------ split + table

template <int DT>
__global__ __launch_bounds__(256) void k_split_hist(SegTable st, uint8_t *__restrict__ raw,
                                                    uint16_t *__restrict__ tables, uint64_t raw_total)
{
    constexpr int kCopies = 8;             // one sub-histogram per 32 threads
    constexpr int kStride = 257;           // pad: copies land on different banks
    __shared__ uint32_t hist[kCopies * kStride];
    __shared__ uint32_t red[4];
    __shared__ uint32_t keys[256];

    const uint64_t k = blockIdx.x;
    const wc_segment sg = find_segment(st, k);
    const uint64_t start = (k - sg.chunk_base) * kChunk;
    const uint32_t len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
    const uint32_t tid = threadIdx.x;

    for (uint32_t i = tid; i < kCopies * kStride; i += 256) hist[i] = 0;
    // the segment's last chunk zeroes the alignment gap after its raw planes
    if (start + len == sg.n) {
        const uint64_t end = sg.raw_base + raw_bytes_of(DT, sg.n);
        const uint64_t pad_end = min(align_up(end, 256), raw_total);
        if (end + tid < pad_end) raw[end + tid] = 0;
    }
    __syncthreads();
    uint32_t *my = hist + (tid >> 5) * kStride;

    if constexpr (DT == WC_BF16) {
        const WC_GLOBAL uint16_t *in = gptr<uint16_t>(sg.ptr) + start;
        uint8_t *lo = raw + sg.raw_base + start;
        const uint32_t ng = len / 8;
        for (uint32_t g = tid; g < ng; g += 256) {
            const u32x4 v = reinterpret_cast<const WC_GLOBAL u32x4 *>(in)[g];
            uint2 l;
            l.x = __builtin_amdgcn_perm(v.y, v.x, 0x06040200u);
            l.y = __builtin_amdgcn_perm(v.w, v.z, 0x06040200u);
            reinterpret_cast<uint2 *>(lo)[g] = l;
            const uint32_t h0 = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
            const uint32_t h1 = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
            atomicAdd(&my[h0 & 0xFF], 1u);
            atomicAdd(&my[(h0 >> 8) & 0xFF], 1u);
            atomicAdd(&my[(h0 >> 16) & 0xFF], 1u);
            atomicAdd(&my[h0 >> 24], 1u);
            atomicAdd(&my[h1 & 0xFF], 1u);
            atomicAdd(&my[(h1 >> 8) & 0xFF], 1u);
            atomicAdd(&my[(h1 >> 16) & 0xFF], 1u);
            atomicAdd(&my[h1 >> 24], 1u);
        }
        for (uint32_t i = ng * 8 + tid; i < len; i += 256) {
            const uint16_t e = in[i];
            lo[i] = (uint8_t)(e & 0xFF);
            atomicAdd(&my[e >> 8], 1u);
        }
    } else {
        // FP32: exponent counted; raw = sign bits | m0 | m1 | m2 (plane bases
        // follow the segment's element count).
        const WC_GLOBAL uint32_t *in = gptr<uint32_t>(sg.ptr) + start;
        const uint64_t sb = (sg.n + 7) / 8;
        uint8_t *sign = raw + sg.raw_base + start / 8;
        uint8_t *m0 = raw + sg.raw_base + sb + start;
        uint8_t *m1 = m0 + sg.n;
        uint8_t *m2 = m1 + sg.n;
        const uint32_t ng = (len + 7) / 8;  // groups of 8 elements = one sign byte
        for (uint32_t g = tid; g < ng; g += 256) {
            uint32_t sbyte = 0;
            for (uint32_t i = 0; i < 8; i++) {
                const uint32_t j = 8 * g + i;
                if (j >= len) break;
                const uint32_t u = in[j];
                atomicAdd(&my[(u >> 23) & 0xFF], 1u);
                sbyte |= (u >> 31) << i;
                m0[j] = (uint8_t)(u & 0xFF);
                m1[j] = (uint8_t)((u >> 8) & 0xFF);
                m2[j] = (uint8_t)((u >> 16) & 0x7F);
            }
            sign[g] = (uint8_t)sbyte;
        }
    }
    __syncthreads();

    uint32_t c = 0;
    for (int i = 0; i < kCopies; i++) c += hist[i * kStride + tid];
    const uint32_t f = normalize256(c, len, red, keys);
    tables[k * 256 + tid] = (uint16_t)f;
}

// ------------------------------------------------------------------ encoder

// Per-symbol encoder constants: reciprocal, renormalisation threshold,
// (4096 - f) and the two shifts, cumulative start b.
struct EncSym {
    uint32_t mp;
    uint32_t th;     // x > th  <=>  x >= f * 2^20 (renormalise first)
    uint32_t fm_sh;  // (4096 - f) | sh1 << 16 | sh2 << 24
    uint32_t b;
};

constexpr uint32_t kEncGroup = 8;                  // steps per group: 256 symbols per half

struct EncShared {
    EncSym enc[2][256];
    uint32_t stage[2][kLanes * kEncGroup / 4];    // the group's symbols, element order
};

// Coded-plane bytes of 8 consecutive elements [e, e + 8), loaded with wide
// loads two groups ahead and unpacked into the group's stage.
template <int DT>
struct SymView;

template <>
struct SymView<WC_BF16> {
    const WC_GLOBAL uint16_t *in;
    struct Pre {
        u32x4 v;
    };
    __device__ Pre fetch(uint32_t e) const { return Pre{*reinterpret_cast<const WC_GLOBAL u32x4 *>(in + e)}; }
    __device__ uint2 bytes(const Pre &p) const
    {
        return make_uint2(__builtin_amdgcn_perm(p.v.y, p.v.x, 0x07050301u),
                          __builtin_amdgcn_perm(p.v.w, p.v.z, 0x07050301u));
    }
    __device__ Pre fetch_checked(uint32_t e, uint32_t len) const
    {
        if (e + 8 <= len) return fetch(e);
        uint32_t v[4] = {0, 0, 0, 0};
        for (uint32_t i = 0; i < 8; i++)
            if (e + i < len) v[i >> 1] |= (uint32_t)in[e + i] << (16 * (i & 1));
        return Pre{u32x4{v[0], v[1], v[2], v[3]}};
    }
};

template <>
struct SymView<WC_FP32> {
    const WC_GLOBAL uint32_t *in;
    struct Pre {
        u32x4 a, b;
    };
    __device__ Pre fetch(uint32_t e) const
    {
        const WC_GLOBAL u32x4 *p = reinterpret_cast<const WC_GLOBAL u32x4 *>(in + e);
        return Pre{p[0], p[1]};
    }
    // exponent byte of u: bits 23..30
    __device__ static uint32_t ex(uint32_t u) { return (u >> 23) & 0xFF; }
    __device__ uint2 bytes(const Pre &p) const
    {
        return make_uint2(ex(p.a.x) | ex(p.a.y) << 8 | ex(p.a.z) << 16 | ex(p.a.w) << 24,
                          ex(p.b.x) | ex(p.b.y) << 8 | ex(p.b.z) << 16 | ex(p.b.w) << 24);
    }
    __device__ Pre fetch_checked(uint32_t e, uint32_t len) const
    {
        if (e + 8 <= len) return fetch(e);
        uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (uint32_t i = 0; i < 8; i++)
            if (e + i < len) v[i] = in[e + i];
        return Pre{u32x4{v[0], v[1], v[2], v[3]}, u32x4{v[4], v[5], v[6], v[7]}};
    }
};

// One encode step for one lane: renormalise (the low 16 bits go to the word
// list, which grows downwards from index p; the lane's rank among the half's
// emitting lanes orders words within a step) and push the symbol.
template <bool CHECK>
__device__ inline void enc_step(uint32_t &x, uint32_t &p, bool active, const EncSym &e,
                                WC_GLOBAL uint16_t *words, uint32_t h)
{
    const bool emit = (!CHECK || active) && x > e.th;
    const uint64_t m = __ballot(emit);
    const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
    p -= __popc(h ? mh : ml);
    const uint32_t slot = __builtin_amdgcn_mbcnt_hi(mh, __builtin_amdgcn_mbcnt_lo(h ? 0u : ml, p));
    if (emit) words[slot] = (uint16_t)(x & 0xFFFF);
    const uint32_t xr = emit ? x >> 16 : x;
    const uint32_t q = div_exact(xr, e.mp, (e.fm_sh >> 16) & 0xFF, e.fm_sh >> 24);
    const uint32_t xn = xr + __umul24(q, e.fm_sh & 0xFFFF) + e.b;
    if (!CHECK || active) x = xn;
}

template <int DT>
__global__ __launch_bounds__(64) void k_encode(SegTable st, const uint16_t *__restrict__ tables,
                                               uint8_t *__restrict__ slots, uint2 *__restrict__ meta,
                                               uint64_t total_chunks)
{
    __shared__ EncShared sh;
    const uint32_t lane = threadIdx.x & 31, h = threadIdx.x >> 5;
    const uint64_t k = 2ull * blockIdx.x + h;
    const bool valid = k < total_chunks;

    wc_segment sg{0, 0, 0, 0};
    uint64_t start = 0;
    uint32_t len = 0;
    if (valid) {
        sg = find_segment(st, k);
        start = (k - sg.chunk_base) * kChunk;
        len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
        // table: 8 symbols per lane, cumulative start by a scan over the half
        const u32x4 fv = gptr(reinterpret_cast<const u32x4 *>(tables + k * 256))[lane];
        uint32_t f[8] = {fv.x & 0xFFFF, fv.x >> 16, fv.y & 0xFFFF, fv.y >> 16,
                         fv.z & 0xFFFF, fv.z >> 16, fv.w & 0xFFFF, fv.w >> 16};
        uint32_t local = 0;
        for (int i = 0; i < 8; i++) local += f[i];
        uint32_t incl = local;
        for (int o = 1; o < 32; o <<= 1) {
            uint32_t v = __shfl_up(incl, o, 32);
            if (lane >= (uint32_t)o) incl += v;
        }
        uint32_t b = incl - local;
        for (int i = 0; i < 8; i++) {
            EncSym e;
            // absent symbols are never encoded; f > 4096 only in a corrupt
            // table, which the normaliser never produces
            const uint32_t fi = f[i] ? (f[i] <= kM ? f[i] : kM) : 1u;
            const uint32_t l = kDivTable.l[fi];
            e.mp = kDivTable.mp[fi];
            e.th = (fi << 20) - 1u;  // wraps to 0xFFFFFFFF at f = 4096: never renormalise
            e.fm_sh = (kM - fi) | ((l < 1 ? l : 1u) << 16) | ((l > 1 ? l - 1 : 0u) << 24);
            e.b = b;
            sh.enc[h][8 * lane + i] = e;
            b += f[i];
        }
    }
    __syncthreads();

    WC_GLOBAL uint8_t *slot = gptr(slots) + (valid ? k : 0) * kSlotBytes;
    WC_GLOBAL uint16_t *words = reinterpret_cast<WC_GLOBAL uint16_t *>(slot + 128);
    SymView<DT> sv;
    using Elem = typename std::conditional<DT == WC_BF16, uint16_t, uint32_t>::type;
    sv.in = gptr<const Elem>(sg.ptr) + start;
    uint32_t x = kL;
    uint32_t p_w = kMaxWords;  // words are written downwards from here
    const uint8_t *stage = reinterpret_cast<const uint8_t *>(&sh.stage[h][0]);

    // Groups of 8 steps, from the last to the first; both halves run the same
    // number of groups (the shorter or missing chunk idles).  Full chunks take
    // the unchecked path.
    constexpr uint32_t kBlkE = kLanes * kEncGroup;  // 256 symbols per group
    const uint32_t steps = valid ? (len + kLanes - 1) / kLanes : 0;
    const uint32_t steps_other = __shfl_xor(steps, 32, 64);
    const uint32_t ngroups = ((steps > steps_other ? steps : steps_other) + kEncGroup - 1) / kEncGroup;
    const uint32_t mine_full = (valid && len == kChunk) ? 1u : 0u;
    const uint32_t other_full = __shfl_xor(mine_full, 32, 64);
    const bool full = mine_full && other_full;
    using Pre = typename SymView<DT>::Pre;
    auto run = [&](auto check_tag, uint32_t ng) {
        constexpr bool CHECK = decltype(check_tag)::value;
        auto fetch = [&](uint32_t g) -> Pre {
            const uint32_t e = kBlkE * g + 8 * lane;
            if constexpr (CHECK) return valid ? sv.fetch_checked(e, len) : Pre{};
            else return sv.fetch(e);
        };
        // a group's input is loaded two groups ahead into one of three
        // register sets (fixed by unrolling the loop by three)
        Pre pa = fetch(ng - 1);
        Pre pb = fetch(ng > 1 ? ng - 2 : ng - 1);
        Pre pc;
        auto group = [&](uint32_t gj, const Pre &cur, Pre &ahead) {
            const uint32_t g = ng - 1 - gj;
            ahead = fetch(g >= 2 ? g - 2 : g);  // the last groups re-load themselves
            reinterpret_cast<uint2 *>(&sh.stage[h][0])[lane] = sv.bytes(cur);
            wave_lds_order();
#pragma unroll
            for (int i = kEncGroup - 1; i >= 0; i--) {
                const bool active = !CHECK || (valid && kLanes * (kEncGroup * g + i) + lane < len);
                const EncSym e = sh.enc[h][stage[kLanes * i + lane]];
                enc_step<CHECK>(x, p_w, active, e, words, h);
            }
            wave_lds_order();
        };
#pragma unroll 1
        for (uint32_t gj = 0; gj < ng; gj += 3) {
            group(gj, pa, pc);
            if (gj + 1 < ng) group(gj + 1, pb, pa);
            if (gj + 2 < ng) group(gj + 2, pc, pb);
        }
    };
    if (ngroups) {
        if (full) run(std::false_type{}, kChunk / kBlkE);
        else run(std::true_type{}, ngroups);
    }

    if (valid) {
        reinterpret_cast<WC_GLOBAL uint32_t *>(slot)[lane] = x;
        if (lane == 0) {
            const uint32_t nw = kMaxWords - p_w;
            meta[k] = make_uint2(128u + 2u * nw + 2u * (nw & 1u), p_w);
        }
    }
}

// --------------------------------------------------------------------- scan

__global__ __launch_bounds__(1024) void k_scan(const uint2 *__restrict__ meta, uint64_t total_chunks,
                                               uint64_t *__restrict__ seek, uint64_t capacity,
                                               uint32_t *err)
{
    __shared__ uint64_t wsum[16];
    const uint32_t tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t per = (total_chunks + 1023) / 1024;
    const uint64_t b = min(total_chunks, per * tid), e = min(total_chunks, b + per);
    uint64_t local = 0;
    for (uint64_t i = b; i < e; i++) local += meta[i].x;
    // inclusive scan in the wavefront, then across the 16 wavefronts
    uint64_t incl = local;
    for (int o = 1; o < 64; o <<= 1) {
        uint64_t v = __shfl_up(incl, o, 64);
        if (lane >= (uint32_t)o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint64_t off = 0;
    for (uint32_t i = 0; i < w; i++) off += wsum[i];
    uint64_t run = off + incl - local;
    if (tid == 0) seek[0] = 0;
    for (uint64_t i = b; i < e; i++) {
        run += meta[i].x;
        seek[i + 1] = run;
    }
    if (tid == 1023) {
        uint64_t total = 0;
        for (int i = 0; i < 16; i++) total += wsum[i];
        if (total > capacity && err) atomicOr(err, WC_EF_CAPACITY);
    }
}

// ------------------------------------------------------------------ compact

__global__ __launch_bounds__(256) void k_compact(const uint8_t *__restrict__ slots,
                                                 const uint2 *__restrict__ meta,
                                                 const uint64_t *__restrict__ seek,
                                                 uint8_t *__restrict__ payload, uint64_t capacity)
{
    const uint64_t k = blockIdx.x;
    const uint2 mk = meta[k];
    const uint64_t dst_off = seek[k];
    if (dst_off + mk.x > capacity) return;  // reported by the scan
    const uint32_t p = mk.y, nw = kMaxWords - p, ndw = (nw + 1) / 2;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(slots + k * kSlotBytes);
    uint32_t *dst = reinterpret_cast<uint32_t *>(payload + dst_off);
    const uint32_t tid = threadIdx.x;
    if (tid < 32) dst[tid] = src[tid];
    const uint32_t *ws = src + 32;  // word area as dwords: word j is half (j & 1) of dword j / 2
    for (uint32_t i = tid; i < ndw; i += 256) {
        const uint32_t j = p + 2 * i;  // word that lands in the low half
        uint32_t v;
        if ((p & 1) == 0) {
            v = ws[j >> 1];
        } else {
            v = ws[j >> 1] >> 16;
            if (j + 1 < kMaxWords) v |= ws[(j + 1) >> 1] << 16;
        }
        if (2 * i + 1 >= nw) v &= 0xFFFFu;  // odd count: zero pad word
        dst[32 + i] = v;
    }
}

}  // namespace wc
