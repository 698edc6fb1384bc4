// wc_encode.hpp -- encoder kernels for gfx950.
//
//   k_split_hist  one 256-thread block per chunk: coalesced 16-byte loads of
//                 the tensor (four in flight per thread), the coded plane
//                 counted into per-lane LDS sub-histograms, then the chunk's
//                 12-bit table built with integer arithmetic only; FP32 and
//                 FP8 raw planes written back with vector stores.
//   k_encode      one wavefront per two chunks (one chunk per 32-lane half):
//                 32 interleaved rANS states, reverse order, words written
//                 downwards into the chunk's scratch slot; the 16-bit
//                 layouts' raw plane (low bytes) written from the same loads,
//                 so the split pass only reads.
//   k_scan_*      exclusive scan of the chunk sizes into the seek table
//                 (tile sums, then per-tile scans).
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
// removes at least E.  C is the count type: 32 bits for a chunk (c 4096 <=
// 2^28), 64 bits for a whole tensor's histogram (T < 2^52).
template <typename C>
__device__ inline uint32_t normalize256(C c, C T, uint32_t *red, C *keys)
{
    const uint32_t s = threadIdx.x;
    const C scaled = c * (C)kM;
    const C q = scaled / T;  // <= 4096
    const C r = scaled - q * T;
    const bool regular = q >= 1;
    uint32_t f = c ? (regular ? (uint32_t)q : 1u) : 0u;
    const int32_t d = (int32_t)kM - (int32_t)block_sum256(f, red);

    if (d > 0) {
        uint32_t m;
        uint32_t pos = block_rank256(regular, red, &m);
        const C key = r * 256u + (255u - s);  // unique per symbol
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

// Sub-histograms: lanes c and c + 32 of every wavefront count into copy c,
// two 16-bit counters per word (a copy sees at most 2048 symbols of a
// chunk, so counters never carry into their neighbour).  At most two lanes
// of one LDS atomic hit the same word; the odd stride spreads the copies
// over the banks.  32 copies (16.5 KiB) leave room for six blocks per CU.
// 16-bit layouts: the encoder, which loads every element anyway, writes the
// raw plane; the split pass only counts.
template <int DT>
constexpr bool raw_in_encoder() { return DT != WC_FP32 && !is_fp8(DT); }

constexpr uint32_t kHistCopies = 32;
constexpr uint32_t kHistStride = 129;

__device__ inline void hist_add(uint32_t *my, uint32_t b)
{
    atomicAdd(&my[b >> 1], 1u << ((b & 1u) << 4));
}

// With a tensor-wide table (WC_OPT_TENSOR_TABLE) the chunk's counts are
// added to its tensor's 64-bit histogram in acc instead, and k_tensor_table
// normalises those.
template <int DT>
__global__ __launch_bounds__(256) void k_split_hist(SegTable st, uint8_t *__restrict__ raw,
                                                    uint16_t *__restrict__ tables, uint64_t raw_total, Opts opts,
                                                    unsigned long long *__restrict__ acc)
{
    __shared__ uint32_t hist[kHistCopies * kHistStride];
    __shared__ uint32_t red[4];
    __shared__ uint32_t keys[256];
    using B = Bits16<DT>;

    const uint64_t k = xcd_block();  // each XCD one contiguous range of chunks
    uint32_t sidx;
    const wc_segment sg = find_segment(st, k, &sidx);
    const uint64_t start = (k - sg.chunk_base) * kChunk;
    const uint32_t len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
    const uint32_t tid = threadIdx.x;

    for (uint32_t i = tid; i < kHistCopies * kHistStride; i += 256) hist[i] = 0;
    // the segment's last chunk zeroes the alignment gap after its raw planes
    if (start + len == sg.n) {
        const uint64_t end = sg.raw_base + raw_bytes_of(DT, sg.n);
        const uint64_t pad_end = min(align_up(end, 256), raw_total);
        if (end + tid < pad_end) raw[end + tid] = 0;
    }
    __syncthreads();
    uint32_t *my = hist + (tid & (kHistCopies - 1)) * kHistStride;

    if constexpr (is_fp8(DT)) {
        // FP8: the reordered byte's high nibble is counted; the low nibbles
        // are packed two per raw byte (element 2j in the low nibble of byte j)
        using B8 = Bits8<DT>;
        const WC_GLOBAL uint8_t *in = gptr<uint8_t>(sg.ptr) + start;
        WC_GLOBAL uint8_t *lo = gptr(raw) + sg.raw_base + start / 2;
        const uint32_t ng = len / 16;  // groups of 16 elements: 16 bytes in, 8 raw bytes out
        auto group16 = [&](u32x4 v, uint32_t g) {
            const u32x4 t = u32x4{B8::to_coded(v.x), B8::to_coded(v.y), B8::to_coded(v.z), B8::to_coded(v.w)};
            // bytes 0 and 2 of pk(a) hold the packed pairs of a's four elements
            auto pk = [](uint32_t a) {
                const uint32_t l = a & 0x0F0F0F0Fu;
                return l | (l >> 4);
            };
            reinterpret_cast<WC_GLOBAL u32x2 *>(lo)[g] = u32x2{__builtin_amdgcn_perm(pk(t.y), pk(t.x), 0x06040200u),
                                                               __builtin_amdgcn_perm(pk(t.w), pk(t.z), 0x06040200u)};
            const uint32_t h[4] = {(t.x >> 4) & 0x0F0F0F0Fu, (t.y >> 4) & 0x0F0F0F0Fu, (t.z >> 4) & 0x0F0F0F0Fu,
                                   (t.w >> 4) & 0x0F0F0F0Fu};
#pragma unroll
            for (uint32_t q = 0; q < 4; q++)
#pragma unroll
                for (uint32_t i = 0; i < 4; i++) hist_add(my, (h[q] >> (8 * i)) & 0xFF);
        };
        constexpr uint32_t U = 4;
        uint32_t g = tid;
        for (; g + 256 * (U - 1) < ng; g += 256 * U) {
            u32x4 v[U];
#pragma unroll
            for (uint32_t u = 0; u < U; u++) v[u] = reinterpret_cast<const WC_GLOBAL u32x4 *>(in)[g + 256 * u];
#pragma unroll
            for (uint32_t u = 0; u < U; u++) group16(v[u], g + 256 * u);
        }
        for (; g < ng; g += 256) group16(reinterpret_cast<const WC_GLOBAL u32x4 *>(in)[g], g);
        // the tail by pairs of elements, so one thread owns each raw byte
        for (uint32_t j = ng * 8 + tid; 2 * j < len; j += 256) {
            const uint32_t t0 = B8::to_coded(in[2 * j]);
            hist_add(my, t0 >> 4);
            uint32_t rb = t0 & 0xF;
            if (2 * j + 1 < len) {
                const uint32_t t1 = B8::to_coded(in[2 * j + 1]);
                hist_add(my, t1 >> 4);
                rb |= (t1 & 0xF) << 4;
            }
            lo[j] = (uint8_t)rb;
        }
    } else if constexpr (DT != WC_FP32) {
        // 16-bit layouts: the coded / raw bytes are the high / low bytes of
        // the layout's rearrangement of each value
        const WC_GLOBAL uint16_t *in = gptr<uint16_t>(sg.ptr) + start;
        WC_GLOBAL uint8_t *lo = gptr(raw) + sg.raw_base + start;
        const uint32_t ng = len / 8;  // groups of 8 elements = 16 bytes
        // four 16-byte loads in flight per thread
        constexpr uint32_t U = 4;
        uint32_t g = tid;
        for (; g + 256 * (U - 1) < ng; g += 256 * U) {
            u32x4 v[U];
#pragma unroll
            for (uint32_t u = 0; u < U; u++) v[u] = reinterpret_cast<const WC_GLOBAL u32x4 *>(in)[g + 256 * u];
#pragma unroll
            for (uint32_t u = 0; u < U; u++) {
                v[u] = u32x4{B::to_coded(v[u].x), B::to_coded(v[u].y), B::to_coded(v[u].z), B::to_coded(v[u].w)};
                const uint32_t h0 = __builtin_amdgcn_perm(v[u].y, v[u].x, 0x07050301u);
                const uint32_t h1 = __builtin_amdgcn_perm(v[u].w, v[u].z, 0x07050301u);
#pragma unroll
                for (uint32_t i = 0; i < 4; i++) hist_add(my, (h0 >> (8 * i)) & 0xFF);
#pragma unroll
                for (uint32_t i = 0; i < 4; i++) hist_add(my, (h1 >> (8 * i)) & 0xFF);
            }
        }
        for (; g < ng; g += 256) {
            u32x4 v = reinterpret_cast<const WC_GLOBAL u32x4 *>(in)[g];
            v = u32x4{B::to_coded(v.x), B::to_coded(v.y), B::to_coded(v.z), B::to_coded(v.w)};
            const uint32_t h0 = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
            const uint32_t h1 = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
            for (uint32_t i = 0; i < 4; i++) hist_add(my, (h0 >> (8 * i)) & 0xFF);
            for (uint32_t i = 0; i < 4; i++) hist_add(my, (h1 >> (8 * i)) & 0xFF);
        }
        for (uint32_t i = ng * 8 + tid; i < len; i += 256) hist_add(my, B::to_coded(in[i]) >> 8);
        (void)lo;
    } else {
        // FP32: exponent counted; raw = sign bits | m0 | m1 | m2 (plane bases
        // follow the segment's element count, so the mantissa planes have no
        // alignment guarantee: byte stores)
        const WC_GLOBAL uint32_t *in = gptr<uint32_t>(sg.ptr) + start;
        const uint64_t sb = (sg.n + 7) / 8;
        WC_GLOBAL uint8_t *sign = gptr(raw) + sg.raw_base + start / 8;
        WC_GLOBAL uint8_t *m0 = gptr(raw) + sg.raw_base + sb + start;
        WC_GLOBAL uint8_t *m1 = m0 + sg.n;
        WC_GLOBAL uint8_t *m2 = m1 + sg.n;
        const uint32_t ng = (len + 7) / 8;  // groups of 8 elements = one sign byte
        for (uint32_t g = tid; g < ng; g += 256) {
            uint32_t sbyte = 0;
            for (uint32_t i = 0; i < 8; i++) {
                const uint32_t j = 8 * g + i;
                if (j >= len) break;
                const uint32_t u = in[j];
                hist_add(my, (u >> 23) & 0xFF);
                sbyte |= (u >> 31) << i;
                m0[j] = (uint8_t)(u & 0xFF);
                m1[j] = (uint8_t)((u >> 8) & 0xFF);
                m2[j] = (uint8_t)((u >> 16) & 0x7F);
            }
            sign[g] = (uint8_t)sbyte;
        }
    }
    __syncthreads();

    // thread s sums symbol s over the 64 copies
    uint32_t c = 0;
    const uint32_t word = tid >> 1, shift = (tid & 1) << 4;
#pragma unroll 8
    for (uint32_t i = 0; i < kHistCopies; i++) c += (hist[i * kHistStride + word] >> shift) & 0xFFFF;
    if (opts.tensor_table()) {
        if (c) atomicAdd(&acc[256ull * sidx + tid], (unsigned long long)c);
        return;
    }
    const uint32_t f = normalize256<uint32_t>(c, len, red, keys);
    tables[k * 256 + tid] = (uint16_t)f;
}

// Tensor-wide tables: zero the 64-bit histograms, then (after k_split_hist)
// one block per tensor normalises its histogram with T = its element count;
// a tensor without elements gets an all-zero table.
__global__ __launch_bounds__(256) void k_zero_u64(unsigned long long *__restrict__ p, uint64_t n)
{
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256) p[i] = 0;
}

__global__ __launch_bounds__(256) void k_tensor_table(SegTable st, const unsigned long long *__restrict__ acc,
                                                      uint16_t *__restrict__ tables)
{
    __shared__ uint32_t red[4];
    __shared__ uint64_t keys[256];
    const uint32_t i = blockIdx.x, tid = threadIdx.x;
    const uint64_t n = st.nseg ? st.segs[i].n : st.single.n;
    uint32_t f = 0;
    if (n) f = normalize256<uint64_t>(acc[256ull * i + tid], n, red, keys);
    tables[256ull * i + tid] = (uint16_t)f;
}

// ------------------------------------------------------------------ encoder

// Per-symbol encoder constants (enc_const): reciprocal, renormalisation
// threshold, the second shift and (4096 - f), cumulative start.
struct EncSym {
    uint32_t mp;
    uint32_t th;  // x > th  <=>  x >= f * 2^20 (renormalise first)
    uint32_t fm;  // sh2 | (4096 - f) << 16
    uint32_t b;   // b, plus 4095 for f = 1
};

constexpr uint32_t kEncGroup = 8;                  // steps per group: 256 symbols per half
constexpr uint32_t kEncBlk = kLanes * kEncGroup;

// The elements a lane encodes in one group: element 32 i + lane of the group
// for step i, loaded (strided, 64 contiguous bytes per half per load) two
// groups ahead of use.
template <int DT>
struct SymView {
    using Elem = typename std::conditional<
        DT == WC_FP32, uint32_t, typename std::conditional<is_fp8(DT), uint8_t, uint16_t>::type>::type;
    const WC_GLOBAL Elem *in;
    struct Pre {
        uint32_t e[kEncGroup];
    };
    template <bool CHECK>
    __device__ Pre fetch(uint32_t g, uint32_t lane, uint32_t len) const
    {
        Pre p;
        const WC_GLOBAL Elem *q = in + kEncBlk * g + lane;
#pragma unroll
        for (uint32_t i = 0; i < kEncGroup; i++) {
            if (CHECK) p.e[i] = kEncBlk * g + kLanes * i + lane < len ? q[kLanes * i] : 0u;
            else p.e[i] = q[kLanes * i];
        }
        return p;
    }
    __device__ static uint32_t symbol(uint32_t e)
    {
        if constexpr (DT == WC_FP32) return (e >> 23) & 0xFF;
        else if constexpr (is_fp8(DT)) return Bits8<DT>::to_coded(e) >> 4;
        else return Bits16<DT>::to_coded(e) >> 8;
    }
};

// Full groups: each lane loads its 8 consecutive elements of a group with
// wide loads; their coded bytes pass through an LDS stage to the lanes that
// encode them (step i of lane l encodes element 32 i + l of the group).
template <int DT>
struct WideView16 {  // the 16-bit layouts
    const WC_GLOBAL u32x4 *in;  // the chunk; 16 bytes = 8 elements per lane per group
    struct Pre {
        u32x4 v;
    };
    __device__ Pre fetch(uint32_t g, uint32_t lane) const { return Pre{in[kLanes * g + lane]}; }
    // the coded (high) bytes of the 8 elements, in element order
    __device__ static uint2 bytes(const Pre &p)
    {
        using B = Bits16<DT>;
        const uint32_t x = B::to_coded(p.v.x), y = B::to_coded(p.v.y);
        const uint32_t z = B::to_coded(p.v.z), w = B::to_coded(p.v.w);
        return make_uint2(__builtin_amdgcn_perm(y, x, 0x07050301u), __builtin_amdgcn_perm(w, z, 0x07050301u));
    }
};

template <int DT>
struct WideView8 {  // FP8
    const WC_GLOBAL u32x2 *in;  // the chunk; 8 bytes = 8 elements per lane per group
    struct Pre {
        u32x2 v;
    };
    __device__ Pre fetch(uint32_t g, uint32_t lane) const { return Pre{in[kLanes * g + lane]}; }
    // the coded nibbles of the 8 elements, one per byte, in element order
    __device__ static uint2 bytes(const Pre &p)
    {
        return make_uint2((Bits8<DT>::to_coded(p.v.x) >> 4) & 0x0F0F0F0Fu,
                          (Bits8<DT>::to_coded(p.v.y) >> 4) & 0x0F0F0F0Fu);
    }
};

struct WideView32 {  // FP32
    const WC_GLOBAL u32x4 *in;  // 32 bytes = 8 elements per lane per group
    struct Pre {
        u32x4 a, b;
    };
    __device__ Pre fetch(uint32_t g, uint32_t lane) const
    {
        return Pre{in[2 * (kLanes * g + lane)], in[2 * (kLanes * g + lane) + 1]};
    }
    // the exponent bytes of the 8 elements, in element order
    __device__ static uint2 bytes(const Pre &p)
    {
        auto e = [](uint32_t u) { return (u >> 23) & 0xFFu; };
        return make_uint2(e(p.a.x) | e(p.a.y) << 8 | e(p.a.z) << 16 | e(p.a.w) << 24,
                          e(p.b.x) | e(p.b.y) << 8 | e(p.b.z) << 16 | e(p.b.w) << 24);
    }
};

template <int DT>
using WideView = typename std::conditional<
    DT == WC_FP32, WideView32, typename std::conditional<is_fp8(DT), WideView8<DT>, WideView16<DT>>::type>::type;

// One encode step for one lane: renormalise (the low 16 bits go to the word
// list, which grows downwards from index p; the lane's rank among the half's
// emitting lanes orders words within a step) and push the symbol.  Only
// emitting lanes write their word (exec-masked).  Words go either straight
// to the slot (STAGE false: a wave-uniform base plus a 32-bit lane offset,
// woff being the half's word area relative to that base) or to the half's
// LDS ring (STAGE true: 256 words per half, word w at w mod 256,
// hsel = 256 h), from which the completed 128-byte lines of the slot are
// written once a group is done.
struct WordDst {
    WC_GLOBAL uint8_t *base;
    uint32_t woff;
    uint16_t *ring;
    uint32_t hsel;
};

template <bool CHECK, bool STAGE>
__device__ __forceinline__ void enc_step(uint32_t &x, uint32_t &p, bool active, const EncSym &e, const WordDst &d,
                                         uint32_t h, uint32_t hs)
{
    const bool emit = (!CHECK || active) && x > e.th;
    const uint64_t m = __ballot(emit);
    const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
    p -= __popc((uint32_t)(m >> hs));
    // rank within the own half: lanes 0-31 count the low mask, lanes 32-63
    // the high one (mbcnt_hi adds nothing below lane 32)
    const uint32_t lo = __builtin_amdgcn_mbcnt_lo(ml, p);
    const uint32_t hi = __builtin_amdgcn_mbcnt_hi(mh, p);
    const uint32_t slot = h ? hi : lo;
    if constexpr (STAGE) {
        if (emit) d.ring[(slot & 255u) | d.hsel] = (uint16_t)(x & 0xFFFF);
    } else {
        uint32_t off = d.woff + 2 * slot;
        asm("" : "+v"(off));  // a 32-bit offset from the uniform base, not a per-lane pointer
        if (emit) *reinterpret_cast<WC_GLOBAL uint16_t *>(d.base + off) = (uint16_t)(x & 0xFFFF);
    }
    const uint32_t xr = emit ? x >> 16 : x;
    const uint32_t xn = enc_update(xr, e.mp, e.fm, e.b);
    if (!CHECK || active) x = xn;
}

// meta[k].y of a chunk stored raw (WC_OPT_RAW_FALLBACK): its slot holds the
// symbols from offset 0 and meta[k].x their padded size.
constexpr uint32_t kRawMark = 0xFFFFFFFFu;

template <int DT, bool STAGE>
__global__ __launch_bounds__(64) void k_encode(SegTable st, const uint16_t *__restrict__ tables,
                                               uint8_t *__restrict__ slots, uint2 *__restrict__ meta,
                                               uint64_t total_chunks, Opts opts, uint8_t *__restrict__ raw)
{
    __shared__ EncSym enc[2][256];
    __shared__ uint32_t estage[2][kEncBlk / 4];  // one full group's coded bytes per half
    // per half: a ring of 256 words (word staging, below)
    __shared__ alignas(16) uint32_t ewring[STAGE ? 2 * 128 : 4];
    const uint32_t lane = threadIdx.x & 31, h = threadIdx.x >> 5;
    // with an odd chunk count the last wavefront's second half shadows the
    // first half's chunk: it runs the same unchecked code but stores nothing
    const uint32_t bid = xcd_block();  // each XCD one contiguous range of chunk pairs
    const uint64_t k_own = 2ull * bid + h;
    const bool real = k_own < total_chunks;
    const uint64_t k = real ? k_own : k_own - 1;

    uint32_t sidx;
    const wc_segment sg = find_segment(st, k, &sidx);
    const uint64_t start = (k - sg.chunk_base) * kChunk;
    const uint32_t len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
    const uint64_t tix = opts.tensor_table() ? sidx : k;
    {
        // table: 8 symbols per lane, cumulative start by a scan over the half
        const u32x4 fv = gptr(reinterpret_cast<const u32x4 *>(tables + tix * 256))[lane];
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
            const EncConst c = enc_const(kDivTable.mp[fi], kDivTable.l[fi], fi, b);
            e.mp = c.mp;
            e.th = (fi << 20) - 1u;  // wraps to 0xFFFFFFFF at f = 4096: never renormalise
            e.fm = c.fm;
            e.b = c.bb;
            enc[h][8 * lane + i] = e;
            b += f[i];
        }
    }
    __syncthreads();

    // Half h writes slot 2 bid + h, so a shadow half (only ever the
    // second half of the last wavefront) writes the spare slot after the
    // last chunk's.  Word stores address a wave-uniform base plus a lane
    // offset: the half's words start 128 bytes into its slot.
    WC_GLOBAL uint8_t *const wbase = gptr(slots) + 2ull * bid * kSlotBytes;
    WC_GLOBAL uint8_t *slot = wbase + h * kSlotBytes;
    uint32_t woff = h * kSlotBytes + 128, hs = 32 * h;
    asm volatile("" : "+v"(woff), "+v"(hs));
    SymView<DT> sv;
    sv.in = gptr<const typename SymView<DT>::Elem>(sg.ptr) + start;
    // 16-bit layouts: this chunk's part of the raw plane (low bytes of the
    // rearranged values); a shadow half writes its sibling's bytes again
    WC_GLOBAL uint8_t *const lo = gptr(raw) + sg.raw_base + start;
    uint32_t x = kL;
    uint32_t p_w = kMaxWords;  // words are written downwards from here

    // Word staging (STAGE).  Steps write their words to the half's LDS
    // ring; words [p_w, wf) are in the ring only.  At the end of a group,
    // wt = p_w rounded up to a multiple of 64 marks the whole 128-byte lines
    // of the slot that are complete (word w is at byte 128 + 2 w of the
    // half's slot, and slots are multiples of 128 bytes); the next group
    // reads them from the ring before its steps (wflush_ld) and writes them
    // to the slot after them (wflush_st), so LDS latency hides behind the
    // steps and every store covers whole lines.  A group writes at most
    // kGroupMaxWords = 192 words per half and fewer than 64 wait below a
    // line, so the ring holds at most 255 words, a flush moves at most 192
    // (one 16-byte read per lane of the first 24 covers the 96 dwords), and
    // the reads come before (in LDS order) the writes that reuse their places.  Where the grid is too
    // small to fill the machine, each wavefront's instruction count sets the
    // time and the words go straight to the slot instead.
    WordDst wd{wbase, woff, reinterpret_cast<uint16_t *>(&ewring[0]), h << 8};
    asm volatile("" : "+v"(wd.hsel));
    const uint32_t *const hring = &ewring[STAGE ? 128 * h : 0];
    uint32_t wf = kMaxWords, wt = kMaxWords;
    // a flush moves at most kGroupMaxWords / 2 = 96 dwords: four per lane
    // of the first 24 lanes, one 16-byte LDS read and one 16-byte store each
    u32x4 fv = {0u, 0u, 0u, 0u};
    auto wflush_ld = [&]() {
        if constexpr (STAGE) {
            // dwords wt / 2 + 4 lane .. + 3 of the half; wt is a multiple of
            // 64, so no 16-byte read straddles the ring's end
            wave_lds_order();
            fv = reinterpret_cast<const u32x4 *>(hring)[((wt >> 3) + lane) & 31u];
        }
    };
    auto wflush_st = [&]() {
        if constexpr (STAGE) {
            // the complete lines, to the half's word area at a 32-bit offset
            // from the uniform base
            const uint32_t n = (wf - wt) >> 1;
            const uint32_t off = woff + 2 * wt + 16 * lane;
            if (4 * lane < n) *reinterpret_cast<WC_GLOBAL u32x4 *>(wbase + off) = fv;
            wf = wt;
            wt = (p_w + 63) & ~63u;
        }
    };

    // Groups of 8 steps run from the last to the first.  Groups where every
    // lane of both halves is active run unchecked; the partial last group of
    // a shorter chunk runs checked, first.
    const uint32_t other_len = __shfl_xor(len, 32, 64);
    // equal in every lane; read as scalars so the group loops are uniform
    const uint32_t ng = __builtin_amdgcn_readfirstlane(((len > other_len ? len : other_len) + kEncBlk - 1) / kEncBlk);
    const uint32_t nfull = __builtin_amdgcn_readfirstlane((len < other_len ? len : other_len) / kEncBlk);
    using Pre = typename SymView<DT>::Pre;
    auto group = [&](auto check_tag, uint32_t g, uint32_t g_next, const Pre &cur, Pre &ahead) {
        constexpr bool CHECK = decltype(check_tag)::value;
        ahead = sv.template fetch<CHECK>(g_next, lane, len);
        if constexpr (raw_in_encoder<DT>()) {
#pragma unroll
            for (uint32_t i = 0; i < kEncGroup; i++) {
                const uint32_t j = kEncBlk * g + kLanes * i + lane;
                if (j < len) lo[j] = (uint8_t)(Bits16<DT>::to_coded(cur.e[i]) & 0xFF);
            }
        }
        EncSym es[kEncGroup];
#pragma unroll
        for (uint32_t i = 0; i < kEncGroup; i++) es[i] = enc[h][SymView<DT>::symbol(cur.e[i])];
        wflush_ld();
#pragma unroll
        for (int i = kEncGroup - 1; i >= 0; i--) {
            const bool active = !CHECK || kEncBlk * g + kLanes * i + lane < len;
            enc_step<CHECK, STAGE>(x, p_w, active, es[i], wd, h, hs);
        }
        wflush_st();
    };
    // Groups run from the last to the first.  The groups above the largest
    // multiple of D below the shorter chunk's full-group count run checked
    // first; then rounds of D full groups run unchecked, each group's input
    // loaded D groups ahead into one of D register sets in fixed registers
    // (D = 8 hides a miss to HBM where a set fits the Infinity Cache only
    // partly; 3 and 4 did not, 16 costs occupancy on large sets).
    constexpr uint32_t D = 8;  // groups per loop round = register sets = prefetch distance
    const uint32_t n3 = nfull / D * D;
    for (uint32_t g = ng; g-- > n3;) {
        const Pre cur = sv.template fetch<true>(g, lane, len);
        Pre dummy;
        group(std::true_type{}, g, g, cur, dummy);
    }
    if (n3) {
        // Full groups, descending: group g's wide load is issued D groups
        // before g is encoded, its bytes go through the stage one group
        // before, and each group reads its per-symbol constants from the
        // symbols so staged.  Loads and stage traffic overlap the steps.
        using WPre = typename WideView<DT>::Pre;
        WideView<DT> wv;
        wv.in = reinterpret_cast<decltype(wv.in)>(sv.in);
        const uint8_t *stg = reinterpret_cast<const uint8_t *>(&estage[h][0]);
        // stages group gs's coded bytes for its steps (and, 16-bit layouts,
        // writes its raw bytes: 8 per lane, contiguous)
        auto transpose = [&](const WPre &d, uint32_t (&sy)[kEncGroup], uint32_t gs) {
            if constexpr (raw_in_encoder<DT>()) {
                using B = Bits16<DT>;
                const uint32_t a0 = B::to_coded(d.v.x), a1 = B::to_coded(d.v.y);
                const uint32_t a2 = B::to_coded(d.v.z), a3 = B::to_coded(d.v.w);
                // a streaming store (nt): the raw plane is not read again by
                // the encode (the coded words' partial lines keep the default
                // policy: written through as nt they cost far more)
                __builtin_nontemporal_store(
                    u32x2{__builtin_amdgcn_perm(a1, a0, 0x06040200u), __builtin_amdgcn_perm(a3, a2, 0x06040200u)},
                    reinterpret_cast<WC_GLOBAL u32x2 *>(lo + kEncBlk * gs) + lane);
            }
            const uint2 b = WideView<DT>::bytes(d);
            wave_lds_order();
            reinterpret_cast<uint2 *>(&estage[h][0])[lane] = b;
            wave_lds_order();
            // each byte is pinned as a 32-bit value at once, so the load
            // zero-extends and no mask is needed where it indexes the table
#pragma unroll
            for (uint32_t i = 0; i < kEncGroup; i++) {
                uint32_t v = stg[kLanes * i + lane];
                asm("" : "+v"(v));
                sy[i] = v;
            }
        };
        uint32_t sy[kEncGroup];
        // g: the group encoded; gl: the group whose load is issued; nx: the
        // next group's data, staged now
        auto fgroup = [&](uint32_t gl, WPre &load_into, const WPre &nx, uint32_t gs) {
            load_into = wv.fetch(gl, lane);
            EncSym es[kEncGroup];
#pragma unroll
            for (uint32_t i = 0; i < kEncGroup; i++) es[i] = enc[h][sy[i]];
            uint32_t sn[kEncGroup];
            transpose(nx, sn, gs);
            wflush_ld();
#pragma unroll
            for (int i = kEncGroup - 1; i >= 0; i--) enc_step<false, STAGE>(x, p_w, true, es[i], wd, h, hs);
            wflush_st();
#pragma unroll
            for (uint32_t i = 0; i < kEncGroup; i++) sy[i] = sn[i];
        };
        // set i holds group k = i (mod D); n3 = 0 (mod D)
        WPre s[D];
#pragma unroll
        for (uint32_t i = 0; i < D; i++) s[i] = wv.fetch(n3 - D + i, lane);
        transpose(s[D - 1], sy, n3 - 1);
#pragma unroll 1
        for (uint32_t g = n3; g > 0; g -= D) {
#pragma unroll
            for (uint32_t j = 1; j <= D; j++) {
                // encode group g - j (its set is free: load group g - j - D into
                // it, group 0 when below) and stage group g - j - 1
                fgroup(g >= j + D ? g - j - D : 0, s[(D - j) % D], s[(2 * D - j - 1) % D], g >= j + 1 ? g - j - 1 : 0);
            }
        }
    }

    // the words still in the ring (at most 255), from the dword holding
    // word p_w (with an odd p_w its other half is not part of the stream)
    if constexpr (STAGE) {
        wt = p_w & ~1u;
        const uint32_t n = (wf - wt) >> 1;
        wave_lds_order();
        for (uint32_t j = lane; j < n; j += kLanes)
            *reinterpret_cast<WC_GLOBAL uint32_t *>(wbase + (woff + 2 * wt + 4 * j)) = hring[((wt >> 1) + j) & 127u];
    }

    if (real) {
        const uint32_t nw = kMaxWords - p_w;  // equal in the half's lanes
        const uint32_t size = 128u + 2u * nw + 2u * (nw & 1u);
        const uint32_t rsize = raw_chunk_bytes(len);
        if (opts.raw_fallback() && size >= rsize) {
            // not worth coding: the slot takes the symbols, zero-padded
            for (uint32_t g = 0; g * kEncBlk < len; g++) {
                const Pre cur = sv.template fetch<true>(g, lane, len);
#pragma unroll
                for (uint32_t i = 0; i < kEncGroup; i++) {
                    const uint32_t j = kEncBlk * g + kLanes * i + lane;
                    if (j < len) slot[j] = (uint8_t)SymView<DT>::symbol(cur.e[i]);
                }
            }
            if (len + lane < rsize) slot[len + lane] = 0;
            if (lane == 0) meta[k] = make_uint2(rsize, kRawMark);
        } else {
            reinterpret_cast<WC_GLOBAL uint32_t *>(slot)[lane] = x;
            if (lane == 0) meta[k] = make_uint2(size, p_w);
        }
    }
}

// --------------------------------------------------------------------- scan
// Two launches over tiles of 4096 chunks: tile sums, then each tile adds the
// sums of the tiles before it and scans its own chunk sizes.  The tile sums
// live in the spare slot after the last chunk's (free once the encoder is
// done: only a shadow half writes there).

constexpr uint32_t kScanTile = 4096;  // chunks per tile: 4 per thread of 1024

__device__ inline uint64_t block_sum1024(uint64_t v, uint64_t *wsum)
{
    const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 5 >> 1;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) wsum[w] = v;
    __syncthreads();
    uint64_t t = 0;
    for (uint32_t i = 0; i < 16; i++) t += wsum[i];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(1024) void k_scan_tiles(const uint2 *__restrict__ meta, uint64_t total_chunks,
                                                     uint64_t *__restrict__ tile_sum)
{
    __shared__ uint64_t wsum[16];
    const uint64_t base = (uint64_t)blockIdx.x * kScanTile;
    uint64_t v = 0;
#pragma unroll
    for (uint32_t u = 0; u < 4; u++) {
        const uint64_t i = base + threadIdx.x + 1024 * u;
        if (i < total_chunks) v += meta[i].x;
    }
    v = block_sum1024(v, wsum);
    if (threadIdx.x == 0) tile_sum[blockIdx.x] = v;
}

__global__ __launch_bounds__(1024) void k_scan_apply(const uint2 *__restrict__ meta, uint64_t total_chunks,
                                                     const uint64_t *__restrict__ tile_sum,
                                                     uint64_t *__restrict__ seek, uint64_t capacity,
                                                     uint32_t *err)
{
    __shared__ uint64_t wsum[16];
    const uint32_t tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // the sizes of every chunk before this tile
    uint64_t before = 0;
    for (uint32_t t = tid; t < blockIdx.x; t += 1024) before += tile_sum[t];
    before = block_sum1024(before, wsum);
    // this thread's four consecutive chunks
    const uint64_t c0 = (uint64_t)blockIdx.x * kScanTile + 4 * tid;
    uint64_t sz[4];
#pragma unroll
    for (uint32_t j = 0; j < 4; j++) sz[j] = c0 + j < total_chunks ? meta[c0 + j].x : 0u;
    const uint64_t local = sz[0] + sz[1] + sz[2] + sz[3];
    uint64_t incl = local;
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t v = __shfl_up(incl, o, 64);
        if (lane >= (uint32_t)o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint64_t run = before + incl - local;
    for (uint32_t i = 0; i < w; i++) run += wsum[i];
#pragma unroll
    for (uint32_t j = 0; j < 4; j++) {
        run += sz[j];
        if (c0 + j < total_chunks) seek[c0 + j + 1] = run;
    }
    if (blockIdx.x == 0 && tid == 0) seek[0] = 0;
    if (c0 < total_chunks && total_chunks <= c0 + 4 && run > capacity && err) atomicOr(err, WC_EF_CAPACITY);
}

// ------------------------------------------------------------------ compact

// Moves chunk k's payload (meta mk) from its slot to dst_off (a chunk that
// would not fit the capacity is skipped: the scan reports it).  Each thread
// moves runs of 4 consecutive output dwords with one 16-byte load and one
// 16-byte store (both only 4-byte aligned: the payload offsets are multiples
// of 4 and the stream starts at any word of the slot), 24 dwords per thread
// per round, so a weight chunk's payload (about 22 KB) moves in one round
// with all its loads in flight.
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ inline void compact_chunk(const uint8_t *__restrict__ slots, uint64_t k, uint2 mk, uint64_t dst_off,
                                     uint8_t *__restrict__ payload, uint64_t capacity)
{
    if (dst_off + mk.x > capacity) return;
    const WC_GLOBAL uint32_t *src = reinterpret_cast<const WC_GLOBAL uint32_t *>(gptr(slots) + k * kSlotBytes);
    WC_GLOBAL uint32_t *dst = reinterpret_cast<WC_GLOBAL uint32_t *>(gptr(payload) + dst_off);
    const uint32_t tid = threadIdx.x;
    if (mk.y == kRawMark) {  // a chunk stored raw: its padded symbols, as dwords
        for (uint32_t i = tid; i < mk.x / 4; i += 256) dst[i] = src[i];
        return;
    }
    const uint32_t p = mk.y, nw = kMaxWords - p, ndw = (nw + 1) / 2;
    if (tid < 32) dst[tid] = src[tid];
    // word area as dwords: word j is half (j & 1) of dword j / 2; output
    // dword i holds words p + 2 i and p + 2 i + 1.  With an odd p each output
    // dword joins two input dwords, and the run's last one needs the dword
    // after it.  Reads reach at most 4 dwords past the slot's end, into the
    // next slot (or the spare slot after the last chunk's); what they bring
    // in only feeds the zero pad word or is not stored.
    const WC_GLOBAL uint32_t *ws = src + 32 + (p >> 1);
    WC_GLOBAL uint32_t *wd = dst + 32;
    const bool odd = p & 1;
    constexpr uint32_t U = 6;  // runs of 4 dwords per thread per round
    for (uint32_t r0 = 0; r0 < ndw; r0 += 256 * 4 * U) {
        u32x4a4 v[U];
        uint32_t nx[U];
#pragma unroll
        for (uint32_t u = 0; u < U; u++) {
            const uint32_t i = r0 + 4 * (tid + 256 * u);
            const bool in = i < ndw;
            v[u] = in ? *reinterpret_cast<const WC_GLOBAL u32x4a4 *>(ws + i) : u32x4a4{0u, 0u, 0u, 0u};
            nx[u] = odd && in ? ws[i + 4] : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < U; u++) {
            const uint32_t i = r0 + 4 * (tid + 256 * u);
            if (i >= ndw) continue;
            u32x4a4 o = v[u];
            if (odd) {
                o.x = __builtin_amdgcn_alignbit(v[u].y, v[u].x, 16);
                o.y = __builtin_amdgcn_alignbit(v[u].z, v[u].y, 16);
                o.z = __builtin_amdgcn_alignbit(v[u].w, v[u].z, 16);
                o.w = __builtin_amdgcn_alignbit(nx[u], v[u].w, 16);
            }
            if (i + 4 <= ndw) {
                if (2 * (i + 3) + 1 >= nw) o.w &= 0xFFFFu;  // odd word count: zero pad word
                *reinterpret_cast<WC_GLOBAL u32x4a4 *>(wd + i) = o;
            } else {
                const uint32_t t[4] = {o.x, o.y, o.z, o.w};
                for (uint32_t q = 0; q < 4 && i + q < ndw; q++)
                    wd[i + q] = 2 * (i + q) + 1 >= nw ? t[q] & 0xFFFFu : t[q];
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_compact(const uint8_t *__restrict__ slots,
                                                 const uint2 *__restrict__ meta,
                                                 const uint64_t *__restrict__ seek,
                                                 uint8_t *__restrict__ payload, uint64_t capacity)
{
    const uint64_t k = xcd_block();  // each XCD one contiguous range of chunks
    compact_chunk(slots, k, meta[k], seek[k], payload, capacity);
}

// Scan and compaction in one launch for at most one scan tile of chunks:
// block k sums the sizes of the chunks before it (at most 4095 8-byte meta
// records, read from L2), writes seek[k] (the last block also the total, and
// the capacity error), then moves its payload.
__global__ __launch_bounds__(256) void k_scan_compact(const uint8_t *__restrict__ slots,
                                                      const uint2 *__restrict__ meta, uint64_t total_chunks,
                                                      uint64_t *__restrict__ seek, uint8_t *__restrict__ payload,
                                                      uint64_t capacity, uint32_t *err)
{
    __shared__ uint64_t wsum[4];
    __shared__ uint64_t off;
    const uint64_t k = blockIdx.x;
    const uint32_t tid = threadIdx.x;
    uint64_t v = 0;
    for (uint64_t i = tid; i < k; i += 256) v += meta[i].x;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((tid & 63) == 0) wsum[tid >> 6] = v;
    __syncthreads();
    const uint2 mk = meta[k];
    if (tid == 0) {
        const uint64_t before = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        off = before;
        seek[k] = before;
        if (k + 1 == total_chunks) {
            seek[total_chunks] = before + mk.x;
            if (before + mk.x > capacity && err) atomicOr(err, WC_EF_CAPACITY);
        }
    }
    __syncthreads();
    compact_chunk(slots, k, mk, off, payload, capacity);
}

}  // namespace wc
