// wc_decode.hpp -- fused decoder for gfx950.
//
// Two forms, chosen by how many chunks there are:
//   - narrow table (kL1 = false, kH = 2): one wavefront decodes two chunks,
//     one per 32-lane half, so every VALU instruction of the serial rANS
//     loop carries 64 useful lanes.  Per half the LDS holds slot -> symbol
//     bytes (4 KiB) plus per-symbol b | (f-4096) << 16 (1 KiB).  With
//     one-dword refills (kSym) the ring also carries the symbol of each
//     word's slot, so a step waits for two dependent LDS reads ((b, f) of
//     its symbol, then its word and next symbol); with two-dword refills it
//     makes two dependent table reads and then its ring read.  12 (11)
//     wavefronts per CU: used when there are enough chunks to fill the
//     machine;
//   - wide table (kL1 = true, kH = 1): one chunk per wavefront, one u32 per
//     slot = symbol | (f-1) << 8 | (slot-b) << 20 (16 KiB), and a ring that
//     keeps each stream word next to the entry of the slot it brings in.  A
//     step starts from the entry of its own slot (known from the step
//     before) and issues in one batch the read of the entry for the state it
//     keeps and the ring read of its next word with that word's entry, so it
//     waits for one LDS latency.  Used while every chunk fits on the machine
//     at once (8 wavefronts per CU), when the run is bound by the serial
//     latency of each chunk.
// Per chunk the LDS also holds
//   - a ring of the compressed stream (256 words, 512 with two-dword
//     refills; its first 64 or 128 words repeated after the end, so a step's
//     32 reads never wrap), refilled 64 or 128 words at a time: a refill is
//     loaded at the start of a group of 8 steps and written to the ring at
//     the start of the group after next, so the load has two groups to land
//     and the word fetch of a step is an LDS read.  The ring is sized for one
//     group's worst case (kGroupMaxWords = 192 words) plus a block, not for
//     the refill latency: a group runs speculatively on the words landed so
//     far; a chunk in which a group consumed a word that had not landed is
//     decoded again from the start with a synchronous fill before every group
//     (rare: it needs more than about 56 words per group for several groups
//     in a row, over 3.5 bits/symbol; weights carry about 2.7);
//   - the 256 decoded bytes of the current group.
// At the end of a group each lane joins 8 consecutive decoded bytes with 8
// raw bytes (loaded with one 8-byte load issued two groups earlier) and
// writes 8 BF16 values with one 16-byte store: the output is written once,
// coalesced, straight to HBM.  The reordered 16-bit layouts undo their bit
// rearrangement on the joined pairs before that store.  Chunks stored raw
// (WC_OPT_RAW_FALLBACK) are skipped here and copied by k_decode_raw.
#pragma once

#include <cstddef>
#include <type_traits>

#include "wc_common.hpp"

namespace wc {

constexpr uint32_t kGroup = 8;                       // steps per group
constexpr uint32_t kGroupWords = kLanes * kGroup;    // lane-steps of a group per half
constexpr uint32_t kStageBytes = kLanes * kGroup;    // decoded bytes per group per half
// Ring geometry for refills of kB dwords per lane.  A refill moves a block
// of 64 kB words, at most one per group, issued while fewer than kAhead
// words are issued and unconsumed, and lands two groups later; so about
// kAhead - 2 r words have landed ahead of a group that consumes r words per
// group, and that must exceed r.  kB = 1 (256-word ring, kAhead 192) covers
// weights (r about 45, up to about 56); kB = 2 (512-word ring, kAhead 384,
// 128-word blocks) covers coded bytes of up to 8 bits, e.g. the FP16 high
// byte (r about 88), which would otherwise outrun the refills and take the
// second pass.  Both rings take a group's worst case (kGroupMaxWords).
// A block never covers an unconsumed word: at issue fewer than kAhead words
// are unconsumed, so with the block fewer than kWords.
// The ring's first kApron words (128; 64 for the narrow table's symbol-
// carrying ring) are repeated after its end, and the cursor is reduced
// modulo the ring size every kWrap = kApron / 32 steps, so the 32 reads of
// a step never wrap.
template <int B, bool kWide = false, bool kSym = false>
struct Ring {
    static constexpr int kB = B;
    static constexpr uint32_t kBlk = 2 * kLanes * kB;
    static constexpr uint32_t kWords = 256u * kB;
    static constexpr uint32_t kApron = (kSym ? 2 : 4) * kLanes;
    static constexpr uint32_t kWrap = kApron / kLanes;
    static constexpr uint32_t kAlloc = kWords + kApron;
    static constexpr uint32_t kAhead = kWords - kBlk;
    static constexpr bool kPow2 = (kWords & (kWords - 1)) == 0;
    // register sets of the pipelined group loop: a refill loaded in group g
    // is written to the ring in group g + kDepth - 1, and a group's raw bytes
    // are loaded kDepth groups before its store
    static constexpr uint32_t kDepth = 3;
    static_assert(kWords % kBlk == 0, "blocks must not wrap the ring");
    static_assert(kAhead >= kGroupMaxWords, "a synchronous fill must land a whole group's worst case");
    static_assert(!kSym || kB == 1, "the symbol-carrying ring takes one-dword refills");
};

// H = chunks per wavefront (one per 32-lane half).  The wide table's ring
// holds each stream word next to the table entry of the slot the word
// brings into a renormalising state (its low 12 bits), both written when
// the word lands; the (b, f) scratch of the table build shares its space.
template <int H, int kB>
struct DecSharedL1 {
    using R = Ring<kB, true>;
    static constexpr uint32_t kRingWords = R::kWords;
    uint32_t tab[H][kM];                    // per slot: sym | (f-1) << 8 | (slot-b) << 20
    union alignas(16) {
        uint32_t fbtmp[H][256];             // (b, f) while the table is built
        u32x2 ring2[H][R::kAlloc];          // per ring word: (tab[word & 4095], word)
    };
    uint32_t stage[H][kStageBytes / 4];
};

template <int H, int kB>
struct alignas(16) DecSharedL2 {
    using R = Ring<kB>;
    static constexpr uint32_t kRingWords = R::kWords;
    uint32_t sym[H][kM / 4];                // slot -> symbol, 4 slots per word
    uint32_t fb[H][256];                    // b | (f - 4096) << 16
    uint32_t ring[H][R::kAlloc / 2];
    uint32_t stage[H][kStageBytes / 4];
};

// The narrow table with a symbol-carrying ring (one-dword refills): next to
// each stream word the symbol of the slot the word brings into a
// renormalising state, looked up when the word lands.  A renormalising lane
// takes its next symbol from the ring read that brings its word, a lane that
// keeps x' reads the symbol of x' meanwhile, so a step waits for two
// dependent LDS reads ((b, f) of the current symbol, then word and symbol)
// instead of three.  Each half's ring symbols start a multiple of 256 bytes
// from sym[0], so the ring cursor can carry that offset (kept by an and-or
// when it is reduced) and serve as the symbol byte's address unchanged.
// 12,800 B per wavefront: ten 1,280-byte LDS granules, 12 wavefronts per CU
// like DecSharedL2<2, 1>.
template <int H>
struct alignas(256) DecSharedS {
    using R = Ring<1, false, true>;
    static constexpr uint32_t kRingWords = R::kWords;
    struct alignas(256) Half {
        uint32_t rsym[R::kAlloc / 4];       // per ring word: sym[word & 4095]
        uint32_t ring[R::kAlloc / 2];       // stream words, two per dword
    };
    uint32_t sym[H][kM / 4];                // slot -> symbol, 4 slots per word
    uint32_t fb[H][256];                    // b | (f - 4096) << 16
    Half hr[H];                             // 1,024 B each (the table build's list scratch)
    uint32_t stage[H][kStageBytes / 4];
};

// Ring block positions: a refill fills block j of the ring (j < kWords /
// kBlk <= 7), and the next one block (j + 1) mod n.  j is kept as the
// selector 0x07070700 | j of a byte permute whose operands hold the
// successor table (bytes 0-6: next(0) .. next(6), byte 7: 7), so one
// v_perm_b32 steps it and the upper selector bytes reproduce themselves.
template <uint32_t n>
struct BlockCycle {
    static_assert(n >= 2 && n <= 7, "ring blocks");
    static constexpr uint32_t next(uint32_t j) { return j + 1 < n ? j + 1 : 0u; }
    static constexpr uint32_t lo = next(0) | next(1) << 8 | next(2) << 16 | next(3) << 24;
    static constexpr uint32_t hi = (n > 4 ? next(4) : 0u) | (n > 5 ? next(5) : 0u) << 8 |
                                   (n > 6 ? next(6) : 0u) << 16 | 7u << 24;
    static constexpr uint32_t start = 0x07070700u;
    __device__ static uint32_t step(uint32_t enc) { return __builtin_amdgcn_perm(hi, lo, enc); }
    __device__ static uint32_t index(uint32_t enc) { return enc & 7u; }
};

// Per-half stream cursor (values uniform within a half).  A lane's refill
// dwords for the words from fill on start at byte lane_off + 2 fill of the
// chunk's payload, clamped to lim, the start of the half's last dword (pair),
// so a refill past the stream end (or one that is not due) still reads in
// bounds; a valid stream never consumes a word past its end.  A half without
// a valid chunk has lane_off = lim = 0 and base at its chunk's table.
struct Stream {
    const WC_GLOBAL uint8_t *base;    // the chunk's payload: 128 bytes of states, then words
    uint32_t lane_off;                // offset of the lane's first refill dword(s)
    uint32_t lim;                     // largest offset a refill load starts at
    uint32_t nw;                      // words in the chunk (pad included, even)
    uint32_t ptr;                     // next word to consume (advanced once per group)
    uint32_t fill;                    // words issued to the ring (landed or in flight)
    uint32_t land;                    // words landed in the ring
    uint32_t fenc;                    // ring block of the next refill (BlockCycle selector), or
                                      // with a power-of-two ring the lane's ring dword
    __device__ uint32_t word_pair(uint32_t d) const  // stream dword d
    {
        return *reinterpret_cast<const WC_GLOBAL uint32_t *>(base + 128 + 4 * d);
    }
};

// A refill moves the next block into the ring, kB dwords per lane.  Its
// loads are issued unconditionally, so the compiler can count outstanding
// memory operations exactly: when no refill is due they read in bounds
// data that is never used.
struct Refill {
    uint32_t v, v1;  // the lane's dwords (v1 with kB = 2)
    uint32_t pos;    // first ring dword the lane writes
    bool go;
    bool first;      // kB = 2: v holds the lane's first dword (else v1 does)
};

__device__ __forceinline__ Refill refill_none()
{
    return Refill{0u, 0u, 0u, false, true};
}

template <typename R>
__device__ __forceinline__ Refill refill_issue(Stream &st, uint32_t lane, bool on)
{
    constexpr int kB = R::kB;
    using C = BlockCycle<R::kWords / R::kBlk>;
    Refill r;
    r.go = on && st.fill - st.ptr < R::kAhead && st.fill < st.nw;
    const uint32_t uoff = st.lane_off + 2 * st.fill;
    const uint32_t off = min(uoff, st.lim);
    const WC_GLOBAL uint32_t *p = reinterpret_cast<const WC_GLOBAL uint32_t *>(st.base + off);
    if constexpr (kB == 1) {
        r.v = p[0];
        r.v1 = 0;
        r.first = true;
    } else {
        // clamped: the pair starts before the lane's first dword, which is
        // then the pair's second (or past the end, like the dword after it)
        r.v = p[0];
        r.v1 = p[1];
        r.first = off == uoff;
    }
    if constexpr (R::kPow2) {
        // fenc is the lane's ring dword itself, stepped a block modulo the ring
        r.pos = st.fenc;
        if (r.go) {
            st.fill += R::kBlk;
            st.fenc = (st.fenc + R::kBlk / 2) & (R::kWords / 2 - 1);
        }
    } else {
        r.pos = (R::kBlk / 2) * C::index(st.fenc) + kB * lane;
        if (r.go) {
            st.fill += R::kBlk;
            st.fenc = C::step(st.fenc);
        }
    }
    return r;
}

// The ring position the first refill of a chunk fills (see Stream::fenc).
template <typename R>
__device__ __forceinline__ uint32_t fenc_start(uint32_t lane)
{
    if constexpr (R::kPow2) return R::kB * lane;
    else return BlockCycle<R::kWords / R::kBlk>::start;
}

template <typename R>
__device__ __forceinline__ void refill_commit(Stream &st, Refill &r, uint32_t *ring)
{
    constexpr int kB = R::kB;
    if (r.go) {
        if constexpr (kB == 1) {
            ring[r.pos] = r.v;
            if (r.pos < R::kApron / 2) ring[R::kWords / 2 + r.pos] = r.v;
        } else {
            // d0 < d: dword d is the pair's second (or past the end), d + 1 is past the end
            const uint2 w = make_uint2(r.first ? r.v : r.v1, r.v1);
            *reinterpret_cast<uint2 *>(&ring[r.pos]) = w;
            if (r.pos < R::kApron / 2) *reinterpret_cast<uint2 *>(&ring[R::kWords / 2 + r.pos]) = w;
        }
        st.land += R::kBlk;
        r.go = false;
    }
}

// The symbol-carrying ring: each landed word is written with the symbol of
// its slot, read from the half's slot -> symbol bytes (sym0: the tables'
// start, sb = 4096 h opaque, so each lookup address is one and-or).
template <typename R>
__device__ __forceinline__ void refill_commit(Stream &st, Refill &r, uint32_t *ring, uint32_t *rsym,
                                              const uint8_t *sym0, uint32_t sb)
{
    static_assert(R::kB == 1, "one dword (two words) per lane");
    if (r.go) {
        const uint32_t s0 = sym0[(r.v & (kM - 1)) | sb];
        const uint32_t s1 = sym0[((r.v >> 16) & (kM - 1)) | sb];
        const uint16_t ss = (uint16_t)__builtin_amdgcn_perm(s1, s0, 0x0c0c0400u);  // s0 | s1 << 8
        ring[r.pos] = r.v;
        reinterpret_cast<uint16_t *>(rsym)[r.pos] = ss;
        if (r.pos < R::kApron / 2) {
            ring[R::kWords / 2 + r.pos] = r.v;
            reinterpret_cast<uint16_t *>(rsym)[R::kWords / 2 + r.pos] = ss;
        }
        st.land += R::kBlk;
        r.go = false;
    }
}

// The wide table's ring: each landed word is written with its slot's entry.
// The lane's words start at ring word 2 r.pos (even), so each pair of words
// is one aligned 16-byte store.
template <typename R>
__device__ __forceinline__ void refill_commit(Stream &st, Refill &r, u32x2 *ring2, const uint32_t *tab)
{
    constexpr int kB = R::kB;
    if (r.go) {
        auto put = [&](uint32_t at, uint32_t v) {
            const uint32_t w0 = v & 0xFFFF, w1 = v >> 16;
            const u32x4 e = {tab[w0 & (kM - 1)], w0, tab[w1 & (kM - 1)], w1};
            *reinterpret_cast<u32x4 *>(&ring2[at]) = e;
            if (at < R::kApron) *reinterpret_cast<u32x4 *>(&ring2[R::kWords + at]) = e;
        };
        if constexpr (kB == 1) {
            put(2 * r.pos, r.v);
        } else {
            put(2 * r.pos, r.first ? r.v : r.v1);
            put(2 * r.pos + 2, r.v1);
        }
        st.land += R::kBlk;
        r.go = false;
    }
}

// Lands what the next group may need (kGroupMaxWords words, or the rest of
// the stream) in blocks loaded together and then written.  Only called with
// nothing in flight, so issued equals landed.
template <typename R, typename... Sink>
__device__ __forceinline__ void refill_sync(Stream &st, uint32_t lane, bool ok, Sink... sink)
{
    constexpr uint32_t n = (kGroupMaxWords + R::kBlk - 1) / R::kBlk;
    Refill r[n];
#pragma unroll
    for (uint32_t j = 0; j < n; j++) r[j] = refill_issue<R>(st, lane, ok && st.fill - st.ptr < kGroupMaxWords);
#pragma unroll
    for (uint32_t j = 0; j < n; j++) refill_commit<R>(st, r[j], sink...);
}

// ----------------------------------------------------------- raw plane views
// fetch(): the raw bytes a lane needs for its 8 elements of a group (issued
// early); flush(): joins them with the 8 decoded bytes and stores.

template <int DT>
struct RawView16 {  // the 16-bit layouts
    using B = Bits16<DT>;
    const WC_GLOBAL uint8_t *lo;
    WC_GLOBAL uint16_t *out;
    struct Pre {
        uint2 v;
    };
    const WC_GLOBAL uint8_t *lol;  // lo + the lane's 8 elements of a group
    __device__ void init(const uint8_t *raw, const wc_segment &sg, uint64_t start)
    {
        lo = gptr(raw) + sg.raw_base + start;
        lol = lo + 8 * (threadIdx.x & 31);
        out = gptr<uint16_t>(sg.ptr) + start;
    }
    // elements [e, e + 8), all inside the chunk, e a multiple of 8
    __device__ Pre fetch(uint32_t e) const
    {
        const WC_GLOBAL uint32_t *p = reinterpret_cast<const WC_GLOBAL uint32_t *>(lo + e);
        return Pre{make_uint2(p[0], p[1])};
    }
    // the lane's elements of full group g (g uniform: one 64-bit add)
    __device__ Pre fetch_group(uint32_t g) const
    {
        const WC_GLOBAL uint32_t *p = reinterpret_cast<const WC_GLOBAL uint32_t *>(lol + (uint64_t)(kGroupWords * g));
        return Pre{make_uint2(p[0], p[1])};
    }
    __device__ void flush(uint32_t e, uint2 sym, const Pre &p) const
    {
        // out[i] = sym[i] << 8 | lo[i]: interleave the bytes pairwise, then
        // undo the layout's bit rearrangement (nothing for BF16 / FP16)
        u32x4 o;
        o.x = B::from_coded(__builtin_amdgcn_perm(sym.x, p.v.x, 0x05010400u));
        o.y = B::from_coded(__builtin_amdgcn_perm(sym.x, p.v.x, 0x07030602u));
        o.z = B::from_coded(__builtin_amdgcn_perm(sym.y, p.v.y, 0x05010400u));
        o.w = B::from_coded(__builtin_amdgcn_perm(sym.y, p.v.y, 0x07030602u));
        // a streaming store (nt): the output is written once and not read
        // back here, so it need not displace the payload and raw lines in
        // the caches (measured about 1% faster on multi-GB weight sets)
        __builtin_nontemporal_store(o, reinterpret_cast<WC_GLOBAL u32x4 *>(out + e));
    }
    // tail chunks: only elements below len exist
    __device__ Pre fetch_checked(uint32_t e, uint32_t len) const
    {
        if (e + 8 <= len) return fetch(e);
        uint32_t v[2] = {0, 0};
        for (uint32_t i = 0; i < 8; i++)
            if (e + i < len) v[i >> 2] |= (uint32_t)lo[e + i] << (8 * (i & 3));
        return Pre{make_uint2(v[0], v[1])};
    }
    __device__ void flush_checked(uint32_t e, uint2 sym, const Pre &p, uint32_t len) const
    {
        if (e + 8 <= len) {
            flush(e, sym, p);
            return;
        }
        for (uint32_t i = 0; i < 8; i++) {
            if (e + i >= len) break;
            const uint32_t sh = 8 * (i & 3);
            const uint32_t sb = ((i < 4 ? sym.x : sym.y) >> sh) & 0xFF;
            const uint32_t lb = ((i < 4 ? p.v.x : p.v.y) >> sh) & 0xFF;
            out[e + i] = (uint16_t)B::from_coded((sb << 8) | lb);
        }
    }
};

// FP8: 8 elements take 4 raw bytes (8 nibbles, element 2j in the low nibble
// of byte j); each output byte is the decoded nibble over the raw nibble
// with the layout's reorder undone, 8 bytes stored at once.
template <int DT>
struct RawView8 {
    using B = Bits8<DT>;
    const WC_GLOBAL uint8_t *lo;
    WC_GLOBAL uint8_t *out;
    struct Pre {
        uint32_t v;
    };
    const WC_GLOBAL uint8_t *lol;  // lo + the raw bytes of the lane's 8 elements of a group
    __device__ void init(const uint8_t *raw, const wc_segment &sg, uint64_t start)
    {
        lo = gptr(raw) + sg.raw_base + start / 2;
        lol = lo + 4 * (threadIdx.x & 31);
        out = gptr<uint8_t>(sg.ptr) + start;
    }
    // elements [e, e + 8), all inside the chunk, e a multiple of 8
    __device__ Pre fetch(uint32_t e) const { return Pre{*reinterpret_cast<const WC_GLOBAL uint32_t *>(lo + e / 2)}; }
    // the lane's elements of full group g (g uniform)
    __device__ Pre fetch_group(uint32_t g) const
    {
        return Pre{*reinterpret_cast<const WC_GLOBAL uint32_t *>(lol + (uint64_t)(kGroupWords / 2 * g))};
    }
    __device__ static u32x2 join(uint2 sym, uint32_t r)
    {
        const uint32_t a = r & 0x0F0F0F0Fu, b = (r >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
        const uint32_t w0 = __builtin_amdgcn_perm(b, a, 0x05010400u), w1 = __builtin_amdgcn_perm(b, a, 0x07030602u);
        return u32x2{B::from_coded((sym.x << 4) | w0), B::from_coded((sym.y << 4) | w1)};
    }
    __device__ void flush(uint32_t e, uint2 sym, const Pre &p) const
    {
        // a streaming store (nt), like the 16-bit layouts' output
        __builtin_nontemporal_store(join(sym, p.v), reinterpret_cast<WC_GLOBAL u32x2 *>(out + e));
    }
    // tail chunks: only elements below len exist
    __device__ Pre fetch_checked(uint32_t e, uint32_t len) const
    {
        if (e + 8 <= len) return fetch(e);
        uint32_t v = 0;
        for (uint32_t i = 0; e + 2 * i < len; i++) v |= (uint32_t)lo[e / 2 + i] << (8 * i);
        return Pre{v};
    }
    __device__ void flush_checked(uint32_t e, uint2 sym, const Pre &p, uint32_t len) const
    {
        if (e + 8 <= len) {
            flush(e, sym, p);
            return;
        }
        const u32x2 o = join(sym, p.v);
        for (uint32_t i = 0; e + i < len; i++) out[e + i] = (uint8_t)(((i < 4 ? o.x : o.y) >> (8 * (i & 3))) & 0xFF);
    }
};

struct RawView32 {
    const WC_GLOBAL uint8_t *sign, *m0, *m1, *m2;
    WC_GLOBAL uint32_t *out;
    struct Pre {
        uint32_t unused;
    };
    __device__ void init(const uint8_t *raw, const wc_segment &sg, uint64_t start)
    {
        const uint64_t sb = (sg.n + 7) / 8;
        sign = gptr(raw) + sg.raw_base + start / 8;
        m0 = gptr(raw) + sg.raw_base + sb + start;
        m1 = m0 + sg.n;
        m2 = m1 + sg.n;
        out = gptr<uint32_t>(sg.ptr) + start;
    }
    // the mantissa planes have no alignment guarantee: they are read with
    // byte loads when the group is written out
    __device__ Pre fetch(uint32_t) const { return Pre{0}; }
    __device__ Pre fetch_group(uint32_t) const { return Pre{0}; }
    __device__ Pre fetch_checked(uint32_t, uint32_t) const { return Pre{0}; }
    __device__ void flush_checked(uint32_t e, uint2 sym, const Pre &, uint32_t len) const
    {
        const uint32_t sbits = sign[e >> 3];
        for (uint32_t i = 0; i < 8; i++) {
            const uint32_t j = e + i;
            if (j >= len) break;
            const uint32_t s = ((i < 4 ? sym.x : sym.y) >> (8 * (i & 3))) & 0xFF;
            out[j] = (((sbits >> i) & 1u) << 31) | (s << 23) | ((uint32_t)m2[j] << 16) |
                     ((uint32_t)m1[j] << 8) | m0[j];
        }
    }
    __device__ void flush(uint32_t e, uint2 sym, const Pre &p) const { flush_checked(e, sym, p, e + 8); }
};

template <int DT>
using RawView = typename std::conditional<
    DT == WC_FP32, RawView32, typename std::conditional<is_fp8(DT), RawView8<DT>, RawView16<DT>>::type>::type;

// -------------------------------------------------------------- table lookup

// The narrow table's lookup, two LDS reads: with x = 4096 q + slot,
// f q + slot - b == x - b + (f - 4096) q  (mod 2^32), one signed 24-bit mad.
struct LookupNarrow {
    // sb = 4096 h and fbb = 1024 h: byte offsets of the half's tables
    template <typename Sh>
    __device__ static inline uint32_t step(const Sh &sh, uint32_t sb, uint32_t fbb, uint32_t x, uint32_t &s)
    {
        const uint8_t *sym = reinterpret_cast<const uint8_t *>(&sh.sym[0][0]);
        s = sym[(x & (kM - 1)) | sb];
        const uint8_t *fbt = reinterpret_cast<const uint8_t *>(&sh.fb[0][0]);
        const uint32_t fb = *reinterpret_cast<const uint32_t *>(fbt + ((s << 2) | fbb));
        return (uint32_t)__mul24((int32_t)fb >> 16, (int32_t)(x >> kScaleBits)) + (x - (fb & 0xFFFF));
    }
};

// One narrow-table decode step of one lane: table lookup, renormalisation
// from the ring (rank among the half's renormalising lanes via ballot +
// mbcnt, added to the stream position of the half's next word), decoded
// byte into the group's stage.  b0, b1 are the half's table bases and hs =
// 32 h, all held opaque so every address is one instruction.
template <bool CHECK, int kH, typename Sh>
__device__ __forceinline__ void dec_step(uint32_t &x, uint32_t &rpos, Sh &sh, uint32_t b0, uint32_t b1, uint32_t hs,
                                uint32_t h, uint32_t lane, bool active, uint32_t i)
{
    uint32_t s;
    const uint32_t xd = LookupNarrow::step(sh, b0, b1, x, s);
    // the decoded byte goes to the stage now: its store can fill the wait
    // the ballot's consumers need after the compare.  The store must not
    // see the table byte itself: then the symbol load would be an
    // any-extending one and need a mask.
    asm("" : "+v"(s));
    reinterpret_cast<uint8_t *>(&sh.stage[h][0])[kLanes * i + lane] = (uint8_t)s;
    const bool need = (!CHECK || active) && xd < kL;
    const uint64_t m = __ballot(need);
    const uint32_t ml = (uint32_t)m, mh = (uint32_t)(m >> 32);
    uint32_t widx, half;
    if constexpr (kH == 1) {
        widx = __builtin_amdgcn_mbcnt_lo(ml, rpos);
        half = ml;
    } else {
        // rank within the own half: lanes 0-31 count the low mask, lanes
        // 32-63 the high one (mbcnt_hi adds nothing below lane 32)
        const uint32_t lo = __builtin_amdgcn_mbcnt_lo(ml, rpos);
        const uint32_t hi = __builtin_amdgcn_mbcnt_hi(mh, rpos);
        widx = h ? hi : lo;
        half = (uint32_t)(m >> hs);
    }
    const uint16_t *ring = reinterpret_cast<const uint16_t *>(&sh.ring[h][0]);
    const uint32_t w = ring[widx];  // widx < Sh::kRingWords + 64
    // x = need ? xd << 16 | w : xd, as one byte permute of (xd, w)
    const uint32_t sel = need ? 0x05040100u : 0x07060504u;
    const uint32_t xn = __builtin_amdgcn_perm(xd, w, sel);
    // the cursor is reduced modulo the ring size every fourth step (after
    // three unreduced steps it is below kRingWords + 96, so a step's reads
    // stay inside the 128-word apron)
    rpos += __popc(half);
    if (i % Sh::R::kWrap == Sh::R::kWrap - 1)
        rpos = Sh::R::kPow2 ? rpos & (Sh::kRingWords - 1) : rpos < Sh::kRingWords ? rpos : rpos - Sh::kRingWords;
    asm volatile("" : "+v"(rpos));
    if (!CHECK || active) x = xn;
}

// One narrow-table step with the symbol-carrying ring.  s, the symbol of
// the slot x holds, is known when the step starts: it is stored to the
// stage and gives (b, f - 4096), hence x' (one signed 24-bit mad).  Then
// the lane reads, in one batch, its ring word at its renormalisation rank
// and one symbol byte: the ring's symbol of that word if it renormalises,
// else the slot table's symbol of x' (an address select, so the byte is a
// single zero-extending load).  The cursor rpos carries rb, the byte offset
// of the half's ring symbols from sym[0] (a multiple of 256): it is the
// symbol byte's address as it stands, and the ring word's address is
// 2 rpos + radj (radj = the ring words' offset - 2 rb, modulo 2^32).  It is
// reduced modulo the ring every second step, (rpos & 255) | rb (a step's
// reads end below kRingWords + 64).  sb = 4096 h and fbb = 1024 h are the
// half's table offsets, hs = 32 h, all opaque.
template <bool CHECK, typename Sh>
__device__ __forceinline__ void dec_step_sym(uint32_t &x, uint32_t &s, uint32_t &rpos, Sh &sh, uint32_t sb,
                                             uint32_t fbb, uint32_t hs, uint32_t rb, uint32_t radj, uint32_t h,
                                             uint32_t lane, uint32_t below, bool active, uint32_t i)
{
    reinterpret_cast<uint8_t *>(&sh.stage[h][0])[kLanes * i + lane] = (uint8_t)s;
    const uint8_t *fbt = reinterpret_cast<const uint8_t *>(&sh.fb[0][0]);
    const uint32_t fb = *reinterpret_cast<const uint32_t *>(fbt + ((s << 2) | fbb));
    const uint32_t xd = (uint32_t)__mul24((int32_t)fb >> 16, (int32_t)(x >> kScaleBits)) + (x - (fb & 0xFFFF));
    const bool need = (!CHECK || active) && xd < kL;
    const uint64_t m = __ballot(need);
    // the own half's mask (one 64-bit shift by 32 h); the lane's rank among
    // the half's renormalising lanes is the count of its bits below the lane
    // (below = 2^lane - 1, one AND and one bit count instead of two mbcnt
    // and a per-half select), and the same mask's count advances the cursor
    const uint32_t half = (uint32_t)(m >> hs);
    const uint32_t widx = __popc(half & below) + rpos;  // rb + (a ring index below Sh::kRingWords + 64)
    // byte offsets from the start of the slot tables (sym[0])
    const uint8_t *base = reinterpret_cast<const uint8_t *>(&sh.sym[0][0]);
    const uint32_t w = *reinterpret_cast<const uint16_t *>(base + (2 * widx + radj));
    const uint32_t at_slot = (xd & (kM - 1)) | sb;
    uint32_t sn = base[need ? widx : at_slot];
    // the next step's stage store must not see the byte itself: the load
    // would then be any-extending and the (b, f) address would need a mask
    asm("" : "+v"(sn));
    const uint32_t sel = need ? 0x05040100u : 0x07060504u;
    const uint32_t xn = __builtin_amdgcn_perm(xd, w, sel);
    rpos += __popc(half);
    if (i % Sh::R::kWrap == Sh::R::kWrap - 1) rpos = (rpos & (Sh::kRingWords - 1)) | rb;
    asm volatile("" : "+v"(rpos));
    if (!CHECK || active) {
        x = xn;
        s = sn;
    }
}

// One decode step with the wide table (one chunk per wavefront).  The entry
// e of the slot x holds is known when the step starts: xd = f (x >> 12) +
// slot - b = (f-1) q + q + (slot-b) needs no read, and the step waits for
// one LDS latency only: it issues together the read of xd's slot entry
// (used if the lane keeps xd) and the ring read of its next word with that
// word's slot entry (used if it renormalises).  The decoded byte is e's low
// byte, stored to the stage at once.
template <bool CHECK, typename Sh>
__device__ __forceinline__ void dec_step_wide(uint32_t &x, uint32_t &e, uint32_t &rpos, Sh &sh, uint32_t b0,
                                              uint32_t lane, bool active, uint32_t i)
{
    const uint32_t q = x >> kScaleBits;
    const uint32_t xd = __umul24((e >> 8) & 0xFFF, q) + (q + (e >> 20));
    reinterpret_cast<uint8_t *>(&sh.stage[0][0])[kLanes * i + lane] = (uint8_t)e;
    const uint32_t et = sh.tab[b0][xd & (kM - 1)];
    const bool need = (!CHECK || active) && xd < kL;
    const uint32_t ml = (uint32_t)__ballot(need);
    const uint32_t widx = __builtin_amdgcn_mbcnt_lo(ml, rpos);  // < Sh::kRingWords + kApron
    const u32x2 rw = sh.ring2[0][widx];                          // (entry, word)
    // x = need ? xd << 16 | w : xd, as one byte permute of (xd, w)
    const uint32_t sel = need ? 0x05040100u : 0x07060504u;
    const uint32_t xn = __builtin_amdgcn_perm(xd, rw.y, sel);
    const uint32_t en = need ? rw.x : et;
    rpos += __popc(ml);
    if (i % Sh::R::kWrap == Sh::R::kWrap - 1)
        rpos = Sh::R::kPow2 ? rpos & (Sh::kRingWords - 1) : rpos < Sh::kRingWords ? rpos : rpos - Sh::kRingWords;
    // keeps the cursor in a VGPR; not volatile, so the scheduler may move
    // the group epilogue into the steps' LDS waits
    asm("" : "+v"(rpos));
    if (!CHECK || active) {
        x = xn;
        e = en;
    }
}

// Builds the slot table of half h from the lane's 8 frequencies f[] (symbols
// 8 lane .. 8 lane + 7) and their cumulative start b0.  The owner of a slot
// is the last present symbol whose start b is <= slot.  The present symbols
// are first listed in symbol order (b | s << 16, at list[], 256 scratch
// dwords of the half), so that the search for a lane's first slot and the
// forward walk over its 128 slots never step through absent symbols (BF16
// weights leave about 120 of them between the positive and the negative
// exponents, which a walk over all symbols crosses one LDS read at a time).
template <bool kL1, typename Sh>
__device__ inline void build_table(Sh &sh, uint32_t h, uint32_t lane, const uint32_t f[8], uint32_t b0,
                                   uint32_t *fbtmp, uint32_t *list)
{
    uint32_t c = 0;
    {
        uint32_t b = b0;
        for (int i = 0; i < 8; i++) {
            fbtmp[8 * lane + i] = (b & 0xFFFF) | ((f[i] - kM) << 16);
            b += f[i];
            c += f[i] != 0;
        }
    }
    // the lane's first list position: exclusive prefix of the counts
    uint32_t incl = c;
    for (int o = 1; o < 32; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 32);
        if (lane >= (uint32_t)o) incl += v;
    }
    const uint32_t npres = __shfl(incl, 31, 32);  // >= 1: the table sums to 4096
    {
        uint32_t b = b0, pos = incl - c;
        for (int i = 0; i < 8; i++) {
            if (f[i]) list[pos++] = b | ((8 * lane + (uint32_t)i) << 16);
            b += f[i];
        }
    }
    wave_lds_order();
    const uint32_t s0 = 128 * lane;
    uint32_t lo = 0, hi = npres;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if ((list[mid] & 0xFFFF) <= s0) lo = mid; else hi = mid;
    }
    uint32_t idx = lo;
    uint32_t s = list[idx] >> 16;
    if constexpr (!kL1) {
        // slot -> symbol bytes without a walk: zero the lane's 128 slots, mark
        // each present symbol at its first slot, then take the running
        // maximum over the slots from the owner of the lane's first slot
        // (present symbols start in increasing order, so the largest mark so
        // far is the owner).  Every lane zeroes its slots before any marks,
        // and marks before any lane reads its slots back (one wavefront, LDS
        // served in issue order).
        u32x4 *row = reinterpret_cast<u32x4 *>(&sh.sym[h][32 * lane]);
#pragma unroll
        for (int j = 0; j < 8; j++) row[j] = u32x4{0u, 0u, 0u, 0u};
        wave_lds_order();
        {
            uint8_t *bytes = reinterpret_cast<uint8_t *>(&sh.sym[h][0]);
            uint32_t b = b0;
            for (int i = 0; i < 8; i++) {
                if (f[i]) bytes[b] = (uint8_t)(8 * lane + (uint32_t)i);
                b += f[i];
            }
        }
        wave_lds_order();
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = row[j];
        uint32_t m = s;
        auto scan = [&](uint32_t w) {
            const uint32_t m0 = max(m, w & 0xFFu), m1 = max(m0, (w >> 8) & 0xFFu);
            const uint32_t m2 = max(m1, (w >> 16) & 0xFFu), m3 = max(m2, w >> 24);
            m = m3;
            return m0 | (m1 << 8) | (m2 << 16) | (m3 << 24);
        };
#pragma unroll
        for (int j = 0; j < 8; j++) {
            u32x4 o;
            o.x = scan(v[j].x);
            o.y = scan(v[j].y);
            o.z = scan(v[j].z);
            o.w = scan(v[j].w);
            row[j] = o;
        }
        return;
    } else {
        // the wide entries the same way: mark each present symbol's first slot
        // b with s | (f-1) << 8 | b << 20 (increasing in b), take the running
        // maximum m from the mark of the owner of the lane's first slot, and
        // turn it into the entry s | (f-1) << 8 | (slot-b) << 20 = m + (slot -
        // 2b) << 20 (mod 2^32)
        const uint32_t bs = list[idx] & 0xFFFF;
        const uint32_t nb = idx + 1 < npres ? list[idx + 1] & 0xFFFF : kM;
        u32x4 *row = reinterpret_cast<u32x4 *>(&sh.tab[h][s0]);
#pragma unroll
        for (int j = 0; j < 32; j++) row[j] = u32x4{0u, 0u, 0u, 0u};
        wave_lds_order();
        {
            uint32_t b = b0;
            for (int i = 0; i < 8; i++) {
                if (f[i]) sh.tab[h][b] = (8 * lane + (uint32_t)i) | ((f[i] - 1) << 8) | (b << 20);
                b += f[i];
            }
        }
        wave_lds_order();
        uint32_t m = s | ((nb - bs - 1) << 8) | (bs << 20);
        auto entry = [&](uint32_t mark, uint32_t slot) {
            m = max(m, mark);
            return m + ((slot - 2 * (m >> 20)) << 20);
        };
#pragma unroll
        for (int j0 = 0; j0 < 32; j0 += 8) {
            u32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = row[j0 + j];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t slot = s0 + 4 * (uint32_t)(j0 + j);
                u32x4 o;
                o.x = entry(v[j].x, slot);
                o.y = entry(v[j].y, slot + 1);
                o.z = entry(v[j].z, slot + 2);
                o.w = entry(v[j].w, slot + 3);
                v[j] = o;
            }
            // rows j0 .. j0+7 are read before they are written (and later
            // rows hold no marks of these slots)
#pragma unroll
            for (int j = 0; j < 8; j++) row[j0 + j] = v[j];
        }
    }
}

// Views of a decoded group.  A view has fetch / flush (full groups) and
// fetch_checked / flush_checked (groups a half may only partly own), and a
// constexpr kWave: false for the store views above, whose calls are made by
// the halves that write output only; true for a view whose flush is a
// wave-wide operation (it exchanges data between the halves), which is then
// called by both halves always and judges ownership itself; such a view
// also has reset() (before a chunk is decoded again) and finish() (after
// the last group).
template <typename V, typename = void>
struct is_wave_view : std::false_type {};
template <typename V>
struct is_wave_view<V, std::void_t<decltype(V::kWave)>> : std::integral_constant<bool, V::kWave> {};

// The decoder for one wavefront (see k_decode).  make_view(sg, sidx, k,
// start, len, put) builds the view of the half's chunk once its segment and
// validity are known.
template <int DT, bool kL1, int kH, int kB, typename View, typename MakeView>
__device__ __forceinline__ void decode_wave(SegTable st, const uint16_t *__restrict__ tables,
                                            const uint64_t *__restrict__ seek,
                                            const uint8_t *__restrict__ payload, uint64_t payload_bytes,
                                            uint64_t total_chunks, uint32_t *err, Opts opts, MakeView make_view)
{
    constexpr bool kWave = is_wave_view<View>::value;
    static_assert(!kL1 || kH == 1, "the wide table decodes one chunk per wavefront");
    // the narrow table with one-dword refills carries symbols in its ring
    constexpr bool kSym = !kL1 && kB == 1;
    using Sh = typename std::conditional<
        kL1, DecSharedL1<kH, kB>,
        typename std::conditional<kSym, DecSharedS<kH>, DecSharedL2<kH, kB>>::type>::type;
    using R = typename Sh::R;
    constexpr uint32_t kRingWords = Sh::kRingWords;
    constexpr uint32_t D = R::kDepth;
    __shared__ Sh sh;
    const uint32_t lane = threadIdx.x & 31, h = kH == 1 ? 0u : threadIdx.x >> 5;
    // each XCD decodes one contiguous range of chunk pairs (xcd_block)
    const uint32_t bid = xcd_block();
    const uint64_t k_own = (uint64_t)kH * bid + h;
    const bool real = k_own < total_chunks;
    const uint64_t k = real ? k_own : k_own - 1;
    bool ok = true;
    uint32_t bits = 0;

    uint32_t sidx;
    const wc_segment sg = find_segment(st, k, &sidx);
    const uint64_t start = (k - sg.chunk_base) * kChunk;
    const uint32_t len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
    const uint64_t tix = opts.tensor_table() ? sidx : k;
    // A half with a bad seek entry still issues its refill loads (never
    // used): they read the first dword(s) at base, here the chunk's own table.
    Stream cs{gptr(reinterpret_cast<const uint8_t *>(tables + tix * 256)), 0, 0, 0, 0, 0, 0,
              fenc_start<R>(lane)};
    uint32_t x = kL;
    // a chunk stored raw (WC_OPT_RAW_FALLBACK) takes no part in the rANS
    // loop (like a bad one, but reports nothing): k_decode_raw copies it
    {
        const uint64_t a = seek[k], b = seek[k + 1];
        if (a > b || b > payload_bytes || (a & 3)) {
            bits |= WC_EF_BAD_SEEK;
            ok = false;
        } else if (opts.raw_fallback() && b - a == raw_chunk_bytes(len)) {
            ok = false;
        } else if (b - a < 128 || ((b - a) & 3)) {
            bits |= WC_EF_BAD_SEEK;
            ok = false;
        } else {
            cs.base = gptr(payload + a);
            cs.nw = (uint32_t)min<uint64_t>((b - a - 128) / 2, 2ull * kMaxWords + 2);
            // dword d of the stream is at 128 + 4 d; the lane's first refill
            // starts at dword kB lane, the last load at dword nw/2 - kB (for
            // nw < 2 kB that is one of the states: still in bounds)
            cs.lane_off = 128 + 4 * kB * lane;
            cs.lim = 128 - 4 * kB + 2 * cs.nw;
            x = reinterpret_cast<const WC_GLOBAL uint32_t *>(cs.base)[lane];
        }
    }
    // table: 8 symbols per lane, validated (sum 4096) before it is used
    uint32_t f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) {
        const u32x4 fv = gptr(reinterpret_cast<const u32x4 *>(tables + tix * 256))[lane];
        f[0] = fv.x & 0xFFFF; f[1] = fv.x >> 16; f[2] = fv.y & 0xFFFF; f[3] = fv.y >> 16;
        f[4] = fv.z & 0xFFFF; f[5] = fv.z >> 16; f[6] = fv.w & 0xFFFF; f[7] = fv.w >> 16;
    }
    uint32_t local = 0;
    for (int i = 0; i < 8; i++) local += f[i];
    uint32_t incl = local;
    for (int o = 1; o < 32; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 32);
        if (lane >= (uint32_t)o) incl += v;
    }
    const uint32_t fsum = __shfl(incl, 31, 32);
    if (ok && fsum != kM) {
        bits |= WC_EF_BAD_TABLE;
        ok = false;
    }
    // every stored state is at least L (no encoder run ends below it); this
    // keeps every state in [L, 2^32) and a group within kGroupMaxWords words
    {
        const uint64_t low = __ballot(ok && x < kL);
        if (ok && (uint32_t)(low >> (32 * h)) != 0) {
            bits |= WC_EF_BAD_FINAL_STATE;
            ok = false;
        }
    }
    if (ok) {
        // scratch for the list of present symbols (256 dwords per half): the
        // ring's space, filled only after the table is built
        uint32_t *fbtmp, *list;
        if constexpr (kL1) {
            static_assert(sizeof(sh.ring2) >= 512 * 4, "list scratch");
            fbtmp = &sh.fbtmp[h][0];
            list = reinterpret_cast<uint32_t *>(&sh.ring2[0][0]) + 256;
        } else if constexpr (kSym) {
            static_assert(sizeof(typename Sh::Half) >= 256 * 4, "list scratch");
            fbtmp = &sh.fb[h][0];
            list = reinterpret_cast<uint32_t *>(&sh.hr[h]);
        } else {
            static_assert(sizeof(Sh) - offsetof(Sh, ring) >= 256 * 4 * kH, "list scratch");
            fbtmp = &sh.fb[h][0];
            list = &sh.ring[0][0] + 256 * h;
        }
        build_table<kL1>(sh, h, lane, f, incl - local, fbtmp, list);
    }
    // the halves' table offsets (4096 h, 1024 h) and 32 h, held opaque;
    // symbol-carrying ring: the cursor's offset rb (the half's ring symbols
    // from sym[0]) and the ring words' address adjustment
    uint32_t b0 = h, b1 = 0, hs = 32 * h, rb = 0, radj = 0;
    if constexpr (!kL1) {
        b0 = h << 12;
        b1 = h << 10;
    }
    if constexpr (kSym) {
        constexpr uint32_t rs0 = (uint32_t)(offsetof(Sh, hr) + offsetof(typename Sh::Half, rsym));
        constexpr uint32_t rw0 = (uint32_t)(offsetof(Sh, hr) + offsetof(typename Sh::Half, ring));
        constexpr uint32_t hstep = (uint32_t)sizeof(typename Sh::Half);
        static_assert(offsetof(Sh, sym) == 0 && rs0 % 256 == 0 && hstep % 256 == 0, "ring symbol offsets");
        rb = rs0 + hstep * h;
        radj = rw0 + hstep * h - 2 * rb;  // modulo 2^32
    }
    asm volatile("" : "+v"(b0), "+v"(b1), "+v"(hs), "+v"(rb), "+v"(radj));
    uint32_t below = (1u << lane) - 1;  // lanes of the own half below this one
    if constexpr (kSym) asm volatile("" : "+v"(below));
    // the wide table's refills also write the slot entries of the words they land
    // (and the symbol-carrying ring the symbols of theirs)
    auto commit = [&](Refill &r) {
        if constexpr (kL1) refill_commit<R>(cs, r, sh.ring2[0], sh.tab[0]);
        else if constexpr (kSym)
            refill_commit<R>(cs, r, sh.hr[h].ring, sh.hr[h].rsym, reinterpret_cast<const uint8_t *>(&sh.sym[0][0]),
                             b0);
        else refill_commit<R>(cs, r, sh.ring[h]);
    };
    auto sync_fill = [&]() {
        if constexpr (kL1) refill_sync<R>(cs, lane, ok, sh.ring2[0], (const uint32_t *)sh.tab[0]);
        else if constexpr (kSym)
            refill_sync<R>(cs, lane, ok, sh.hr[h].ring, sh.hr[h].rsym,
                           reinterpret_cast<const uint8_t *>(&sh.sym[0][0]), b0);
        else refill_sync<R>(cs, lane, ok, sh.ring[h]);
    };
    __syncthreads();
    sync_fill();
    __syncthreads();
    // wide table: the entry of the slot x holds; symbol-carrying ring: its
    // symbol (a half without a valid table reads a value it never uses)
    uint32_t e = 0;
    if constexpr (kL1) e = sh.tab[0][x & (kM - 1)];
    // symbol-carrying ring: the symbol of the slot x holds
    auto sym_of = [&](auto &shr, uint32_t v) -> uint32_t {
        return reinterpret_cast<const uint8_t *>(&shr.sym[h][0])[v & (kM - 1)];
    };
    if constexpr (kSym) e = sym_of(sh, x);

    const uint2 *stage = reinterpret_cast<const uint2 *>(&sh.stage[h][0]);
    const bool put = ok && real;  // this half writes output
    View rv = make_view(sg, sidx, k, start, ok ? len : 0u, put);

    // Groups of 8 steps, first to last.  Groups where every lane of every
    // half is active (and every table valid) run unchecked; the partial last
    // group of a shorter chunk runs checked, last.
    const uint32_t my_len = ok ? len : 0u;
    const uint32_t other_len = kH == 2 ? __shfl_xor(my_len, 32, 64) : my_len;
    const uint32_t hi_len = my_len > other_len ? my_len : other_len;
    const uint32_t lo_len = my_len < other_len ? my_len : other_len;
    // equal in every lane; read as scalars so the group loops are uniform
    const uint32_t ng = __builtin_amdgcn_readfirstlane((hi_len + kGroupWords - 1) / kGroupWords);
    const uint32_t nfull = __builtin_amdgcn_readfirstlane(lo_len / kGroupWords);
    using Pre = typename View::Pre;
    uint32_t rpos = rb;  // cs.ptr modulo the ring size (plus rb), advanced every step
    auto step = [&](auto check_tag, bool active, uint32_t i) {
        constexpr bool CHECK = decltype(check_tag)::value;
        if constexpr (kL1) dec_step_wide<CHECK>(x, e, rpos, sh, b0, lane, active, i);
        else if constexpr (kSym) dec_step_sym<CHECK>(x, e, rpos, sh, b0, b1, hs, rb, radj, h, lane, below, active, i);
        else dec_step<CHECK, kH>(x, rpos, sh, b0, b1, hs, h, lane, active, i);
    };
    // Speculation: set when a group consumed a word that had not landed.
    bool overrun = false;
    // One group: due is the refill to write into the ring now, next where
    // this group's refill goes (the same object in the one-deep remainder).
    // (refills off: the group only reads what a synchronous fill landed)
    auto group = [&](auto check_tag, uint32_t gg, uint32_t g_last, const Pre &cur, Pre &ahead, Refill &due,
                     Refill &next, bool refills = true) {
        constexpr bool CHECK = decltype(check_tag)::value;
        commit(due);
        next = refill_issue<R>(cs, lane, ok && refills);
        // the value loaded for a group past the last is never used
        const uint32_t gn = gg + 2 <= g_last ? gg + 2 : g_last;
        if constexpr (CHECK) ahead = put || kWave ? rv.fetch_checked(kGroupWords * gn + 8 * lane, len) : Pre{};
        else ahead = rv.fetch_group(gn);
        const uint32_t landed = cs.land, r0 = rpos;
        wave_lds_order();
#pragma unroll
        for (uint32_t i = 0; i < kGroup; i++) {
            const bool active = !CHECK || (ok && kLanes * (kGroup * gg + i) + lane < len);
            step(check_tag, active, i);
        }
        wave_lds_order();
        // unconditional in full groups, so the compiler counts memory
        // operations exactly: a shadow half writes what its sibling does
        if constexpr (CHECK) {
            if (put || kWave) rv.flush_checked(kGroupWords * gg + 8 * lane, stage[lane], cur, len);
        } else {
            rv.flush(kGroupWords * gg + 8 * lane, stage[lane], cur);
        }
        wave_lds_order();
        // words this group consumed (at most kGroupMaxWords, less than the
        // ring): the cursor difference, plus the ring size if it wrapped
        const uint32_t dr = rpos - r0;
        const uint32_t used = R::kPow2 ? dr & (kRingWords - 1) : min(dr, dr + kRingWords);
        overrun |= cs.ptr + used > landed;
        cs.ptr += used;
    };
    // Full groups run pipelined: group gg carries group gg-1's epilogue.
    // Its stage bytes are read before step 0 overwrites them; after step 0
    // they are joined with its raw bytes and stored, its consumption is
    // settled (so refills see a cursor one group behind, which only delays
    // them), and this group's refill and the raw bytes of group gg+2 are
    // loaded.  The epilogue's instructions thus fill the step's LDS waits.
    struct Pend {
        uint32_t landed, r0;  // words landed at the group's start, its starting cursor
    };
    auto settle = [&](const Pend &pd, uint32_t r_end) {
        const uint32_t dr = r_end - pd.r0;
        const uint32_t used = R::kPow2 ? dr & (kRingWords - 1) : min(dr, dr + kRingWords);
        overrun |= cs.ptr + used > pd.landed;
        cs.ptr += used;
    };
    auto fast = [&](auto prev_tag, uint32_t gg, uint32_t g_last, Pre &pv, Refill &due, Refill &next, Pend &pd) {
        constexpr bool PREV = decltype(prev_tag)::value;
        commit(due);
        const Pend mine{cs.land, rpos};
        uint2 sprev = make_uint2(0u, 0u);
        wave_lds_order();
        if constexpr (PREV) sprev = stage[lane];
#pragma unroll
        for (uint32_t i = 0; i < kGroup; i++) {
            step(std::false_type{}, true, i);
            if (i == 0) {
                // unconditional, so the compiler counts memory operations
                // exactly: a shadow half writes what its sibling does
                if constexpr (PREV) {
                    rv.flush(kGroupWords * (gg - 1) + 8 * lane, sprev, pv);
                    settle(pd, mine.r0);
                }
                next = refill_issue<R>(cs, lane, ok);
                // the value loaded for a group past the last is never used
                pv = rv.fetch_group(gg + D - 1 <= g_last ? gg + D - 1 : g_last);
            }
        }
        wave_lds_order();
        pd = mine;
    };
    // Raw bytes of group g are loaded D groups before its store into one of
    // D register sets, and the refill issued in group g is written to the
    // ring in group g + D - 1, also from one of D sets: the hot loop runs
    // whole rounds of D full groups so every set stays in fixed registers.
    // Group g + j of a round flushes with set j - 1 (mod D) and reloads it
    // for group g + j + D - 1, writes refill set j + 1 (mod D) and issues
    // into set j.
    Refill q[D];
#pragma unroll
    for (uint32_t j = 0; j < D; j++) q[j] = refill_none();
    const uint32_t nD = nfull / D * D;
    if (nD) {
        const std::false_type no{};
        const std::true_type yes{};
        Pre p[D];
#pragma unroll
        for (uint32_t j = 0; j + 1 < D; j++) p[j] = rv.fetch_group(j);
        Pend pd{0u, 0u};
        const uint32_t last = nD - 1;
        // the first round is peeled, so the loop is entered with the
        // memory operations in flight that every iteration leaves behind
        fast(no, 0, last, p[D - 1], q[1], q[0], pd);
#pragma unroll
        for (uint32_t j = 1; j < D; j++) fast(yes, j, last, p[j - 1], q[(j + 1) % D], q[j], pd);
#pragma unroll 1
        for (uint32_t g = D; g < nD; g += D) {
#pragma unroll
            for (uint32_t j = 0; j < D; j++) fast(yes, g + j, last, p[(j + D - 1) % D], q[(j + 1) % D], q[j], pd);
        }
        // the last full group's epilogue
        wave_lds_order();
        rv.flush(kGroupWords * last + 8 * lane, stage[lane], p[D - 1]);
        wave_lds_order();
        settle(pd, rpos);
    }
    // What is left (fewer than D full groups and a partial one) runs checked,
    // with refills committed one group after they are issued: first the ones
    // still in flight land, oldest first.
#pragma unroll
    for (uint32_t j = 1; j < D; j++) commit(q[j]);
    for (uint32_t g = nD; g < ng; g++) {
        Pre cur = put || kWave ? rv.fetch_checked(kGroupWords * g + 8 * lane, len) : Pre{};
        Pre dummy;
        group(std::true_type{}, g, g, cur, dummy, q[0], q[0]);
    }
    // A chunk whose speculation failed is decoded again from its start,
    // every group checked and preceded by a synchronous fill, and its
    // output written again.
    if (__ballot(overrun)) {
        if constexpr (kWave) rv.reset();
        commit(q[0]);
        cs.ptr = cs.fill = cs.land = 0;
        cs.fenc = fenc_start<R>(lane);
        rpos = rb;
        if (ok) x = reinterpret_cast<const WC_GLOBAL uint32_t *>(cs.base)[lane];
        if constexpr (kL1) e = sh.tab[0][x & (kM - 1)];
        if constexpr (kSym) e = sym_of(sh, x);
        for (uint32_t g = 0; g < ng; g++) {
            sync_fill();
            Pre cur = put || kWave ? rv.fetch_checked(kGroupWords * g + 8 * lane, len) : Pre{};
            Pre dummy;
            Refill none = refill_none();
            group(std::true_type{}, g, g, cur, dummy, none, none, false);
        }
    }

    if (ok) {
        if (cs.ptr > cs.nw) {
            bits |= WC_EF_WORD_OVERRUN;
        } else if (cs.nw - cs.ptr > 1) {
            bits |= WC_EF_BAD_TAIL;
        } else if (cs.nw - cs.ptr == 1) {
            const uint32_t last = cs.word_pair(cs.ptr >> 1);
            if ((cs.ptr & 1 ? last >> 16 : last & 0xFFFF) != 0) bits |= WC_EF_BAD_TAIL;
        }
        if (x != kL) bits |= WC_EF_BAD_FINAL_STATE;
    }
    if constexpr (kWave) rv.finish();
    // OR the half's bits into lane 0 of the half; a shadow half reports nothing
    for (int o = 16; o > 0; o >>= 1) bits |= __shfl_xor(bits, o, 32);
    if (lane == 0 && bits && real && err) atomicOr(err, bits);
}

// kH = 1: one chunk per wavefront (32 lanes; the wide table's variant, so
// a lone wavefront's serial chain has no per-half selects).  kH = 2: two
// chunks per wavefront; with an odd chunk count the last wavefront's second
// half shadows the first half's chunk (same unchecked code, nothing stored).
template <int DT, bool kL1, int kH, int kB>
__global__ __launch_bounds__(32 * kH) void k_decode(SegTable st, const uint8_t *__restrict__ raw,
                                                    const uint16_t *__restrict__ tables,
                                                    const uint64_t *__restrict__ seek,
                                                    const uint8_t *__restrict__ payload,
                                                    uint64_t payload_bytes, uint64_t total_chunks,
                                                    uint32_t *err, Opts opts)
{
    decode_wave<DT, kL1, kH, kB, RawView<DT>>(
        st, tables, seek, payload, payload_bytes, total_chunks, err, opts,
        [&](const wc_segment &sg, uint32_t, uint64_t, uint64_t start, uint32_t, bool) {
            RawView<DT> rv;
            rv.init(raw, sg, start);
            return rv;
        });
}

// Chunks stored raw (WC_OPT_RAW_FALLBACK), after k_decode (which skips
// them): one 256-thread block per chunk; a block whose chunk is coded, or
// whose seek entries are bad (k_decode reports those), exits at once.  The
// payload holds the chunk's symbols, zero-padded to a multiple of 4 bytes;
// they are joined with the raw plane exactly like decoded ones.
template <int DT>
__global__ __launch_bounds__(256) void k_decode_raw(SegTable st, const uint8_t *__restrict__ raw,
                                                    const uint64_t *__restrict__ seek,
                                                    const uint8_t *__restrict__ payload, uint64_t payload_bytes,
                                                    uint32_t *err)
{
    const uint64_t k = blockIdx.x;
    const wc_segment sg = find_segment(st, k);
    const uint64_t start = (k - sg.chunk_base) * kChunk;
    const uint32_t len = (uint32_t)min((uint64_t)kChunk, sg.n - start);
    const uint64_t a = seek[k], b = seek[k + 1];
    if (a > b || b > payload_bytes || (a & 3) || b - a != raw_chunk_bytes(len)) return;
    RawView<DT> rv;
    rv.init(raw, sg, start);
    const WC_GLOBAL uint8_t *pl = gptr(payload) + a;
    const WC_GLOBAL uint32_t *pw = reinterpret_cast<const WC_GLOBAL uint32_t *>(pl);
    for (uint32_t e = 8 * threadIdx.x; e < len; e += 8 * 256) {
        uint2 sy;
        if (e + 8 <= len) {
            sy = make_uint2(pw[e / 4], pw[e / 4 + 1]);
        } else {
            uint32_t v[2] = {0, 0};
            for (uint32_t i = 0; e + i < len; i++) v[i >> 2] |= (uint32_t)pl[e + i] << (8 * (i & 3));
            sy = make_uint2(v[0], v[1]);
        }
        rv.flush_checked(e, sy, rv.fetch_checked(e, len), len);
    }
    if (len + threadIdx.x < raw_chunk_bytes(len) && pl[len + threadIdx.x] != 0 && err) atomicOr(err, WC_EF_BAD_TAIL);
}

}  // namespace wc
