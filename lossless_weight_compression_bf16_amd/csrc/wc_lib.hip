// wc_lib.hip -- C ABI of the gfx950 lossless weight codec (see include/wc.h).
//
// Host side: argument validation, buffer layout, and the launch sequence
//   encode: k_split_hist -> k_encode -> k_scan_tiles, k_scan_apply -> k_compact
//           (at most 4096 chunks: k_scan_compact does scan and compaction)
//           (16-bit layouts: the raw plane is written by k_encode)
//           (tensor-wide tables: k_zero_u64 before the split, k_tensor_table after;
//           CRC-32 option: k_crc32 after the compaction)
//   decode: k_decode (then k_decode_raw for chunks stored raw; CRC-32 option:
//           k_crc32 check before)
//   decode + GEMM: k_decode_gemm (CRC-32 option: k_crc32 check before);
//           tile order: k_tile_order
// on the caller's stream.  No allocation, no synchronisation, no global state.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <string.h>

#include "wc.h"
#include "wc_common.hpp"
#include "wc_crc.hpp"
#include "wc_decode.hpp"
#include "wc_encode.hpp"
#include "wc_gemm.hpp"

using namespace wc;

namespace {

constexpr int kVersion = 10200;  // 1.2.0: format variants, CRC-32, fused decode + GEMM

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

uint64_t chunk_capacity(uint64_t len) { return 128 + 2 * (len + (len & 1)); }

bool valid_format(uint32_t f)
{
    return (f & WC_LAYOUT_MASK) <= WC_FP8_E5M2 &&
           (f & ~(WC_LAYOUT_MASK | WC_OPT_TENSOR_TABLE | WC_OPT_RAW_FALLBACK | WC_OPT_CRC32)) == 0;
}
bool has_crc(uint32_t f) { return (f & WC_OPT_CRC32) != 0; }
int layout_code(uint32_t f) { return (int)(f & WC_LAYOUT_MASK); }
Opts opts_of(uint32_t f) { return Opts{f & (WC_OPT_TENSOR_TABLE | WC_OPT_RAW_FALLBACK | WC_OPT_CRC32)}; }

void layout_of(uint32_t format, uint64_t n, wc_layout *out)
{
    const uint64_t c = (n + kChunk - 1) / kChunk;
    const bool rawfb = opts_of(format).raw_fallback();
    auto cap = [&](uint64_t len) { return rawfb ? (uint64_t)raw_chunk_bytes((uint32_t)len) : chunk_capacity(len); };
    out->n = n;
    out->num_chunks = c;
    out->raw_bytes = raw_bytes_of(layout_code(format), n);
    out->table_bytes = opts_of(format).tensor_table() ? 512 : 512 * c;
    out->seek_bytes = 8 * (c + 1);
    out->payload_capacity = 0;
    if (c) out->payload_capacity = (c - 1) * cap(kChunk) + cap(n - (c - 1) * kChunk);
    out->scratch_bytes = 0;
    out->crc_bytes = has_crc(format) ? 4 * c : 0;
}

// Encoder scratch: 8 bytes of meta per chunk, one slot per chunk plus a
// spare one (written by the idle half of the last wavefront when the chunk
// count is odd; the scan's tile sums go there afterwards), and with
// tensor-wide tables a 256 x u64 histogram per tensor.
uint64_t hist_offset(uint64_t chunks) { return align_up(8 * chunks, 256) + (chunks + 1) * kSlotBytes; }
uint64_t scratch_bytes_for(uint64_t chunks, uint64_t tensor_tables)
{
    return chunks ? hist_offset(chunks) + 2048 * tensor_tables : 0;
}

// Checks a batch's host segment array against the planning rule.
wc_status check_plan(uint32_t format, const wc_segment *segs, uint32_t nseg, wc_layout *total,
                     bool need_ptrs = true)
{
    uint64_t chunks = 0, raw = 0, cap = 0, elems = 0;
    for (uint32_t i = 0; i < nseg; i++) {
        const wc_segment &s = segs[i];
        if (s.n > kMaxElems) return WC_ERR_ARG;
        if (s.chunk_base != chunks || s.raw_base != raw) return WC_ERR_ARG;
        if (need_ptrs && s.n && (s.ptr == 0 || (s.ptr % 16) != 0)) return WC_ERR_ARG;
        wc_layout one;
        layout_of(format, s.n, &one);
        chunks += one.num_chunks;
        raw += one.raw_bytes;
        if (i + 1 < nseg) raw = align_up(raw, 256);
        cap += one.payload_capacity;
        elems += s.n;
    }
    total->n = elems;
    total->num_chunks = chunks;
    total->raw_bytes = raw;
    const bool tt = opts_of(format).tensor_table();
    total->table_bytes = tt ? 512ull * nseg : 512 * chunks;
    total->seek_bytes = 8 * (chunks + 1);
    total->payload_capacity = cap;
    total->scratch_bytes = scratch_bytes_for(chunks, tt ? nseg : 0);
    total->crc_bytes = has_crc(format) ? 4 * chunks : 0;
    return WC_OK;
}

wc_status check_buffers(const wc_buffers *b, uint64_t chunks, uint64_t raw_bytes, uint64_t table_bytes,
                        uint64_t crc_bytes)
{
    if (!b || !b->seek || !aligned(b->seek, 8)) return WC_ERR_ARG;
    if (table_bytes && (!b->tables || !aligned(b->tables, 16))) return WC_ERR_ARG;
    if (chunks == 0) return WC_OK;
    if (crc_bytes && (!b->crc || !aligned(b->crc, 4))) return WC_ERR_ARG;
    if (!b->payload || !aligned(b->payload, 16)) return WC_ERR_ARG;
    if (raw_bytes && (!b->raw || !aligned(b->raw, 16))) return WC_ERR_ARG;
    return WC_OK;
}

// The device whose queue `stream` feeds (the current device for the null
// stream): the encoder and decoder variants depend on that device's CU count, not on
// whichever device happens to be current on the calling thread.
bool stream_device(hipStream_t stream, int *dev)
{
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return false;
        *dev = d;
        return true;
    }
    return hipGetDevice(dev) == hipSuccess;
}

// Encoder word stores.  For the 16-bit layouts a grid that fills every
// SIMD's wavefront slots at least once (k_encode holds 4 wavefronts per
// SIMD, 16 per CU) is bound by the memory pipeline, and staging the words
// in LDS to write them once per group is faster (MoE experts set, dword
// flushes: BF16 8.66 -> 7.99 ms, FP16 9.49 -> 8.87 ms; now whole 128-byte
// lines with 16-byte stores); a smaller grid is bound by
// each wavefront's serial instruction stream, and the direct 2-byte stores,
// with fewer instructions per step, are faster there (up to 24%).  FP8
// (half the input bytes per symbol) is faster direct at any size (6.0
// against 6.3 ms on the same set), FP32 within 3% either way: both store
// directly.
std::atomic<int> g_enc_words{WC_ENC_WORDS_AUTO};

bool use_staged_words(int layout, uint64_t chunks, int dev, bool *staged)
{
    const int mode = g_enc_words.load(std::memory_order_relaxed);
    if (mode != WC_ENC_WORDS_AUTO) {
        *staged = mode == WC_ENC_WORDS_STAGED;
        return true;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    const bool sixteen = layout != WC_FP32 && layout != WC_FP8_E4M3 && layout != WC_FP8_E5M2;
    *staged = sixteen && (chunks + 1) / 2 >= 16 * (uint64_t)cus;
    return true;
}

template <int DT>
wc_status encode_impl(const SegTable &st, uint64_t chunks, uint64_t raw_total, const wc_buffers *out,
                      void *d_scratch, uint32_t *d_err, hipStream_t stream, hipEvent_t *ev, Opts opts)
{
    uint2 *meta = reinterpret_cast<uint2 *>(d_scratch);
    uint8_t *slots = reinterpret_cast<uint8_t *>(d_scratch) + align_up(8 * chunks, 256);
    const uint32_t ntab = st.nseg ? st.nseg : 1;  // tensors (tensor-wide tables)
    unsigned long long *hist =
        chunks ? reinterpret_cast<unsigned long long *>(reinterpret_cast<uint8_t *>(d_scratch) + hist_offset(chunks))
               : nullptr;
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return WC_ERR_HIP;
    if (chunks && opts.tensor_table()) {
        const uint64_t words = 256ull * ntab;
        const uint64_t blocks = (words + 255) / 256;
        hipLaunchKernelGGL(k_zero_u64, dim3((uint32_t)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, hist,
                           words);
    }
    if (chunks) {
        hipLaunchKernelGGL(k_split_hist<DT>, dim3((uint32_t)chunks), dim3(256), 0, stream, st, out->raw,
                           out->tables, raw_total, opts, hist);
    }
    if (opts.tensor_table()) {
        // every tensor's table, also those of tensors without elements
        hipLaunchKernelGGL(k_tensor_table, dim3(ntab), dim3(256), 0, stream, st, hist, out->tables);
    }
    if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return WC_ERR_HIP;
    if (chunks) {
        int dev = 0;
        bool staged = false;
        if (!stream_device(stream, &dev) || !use_staged_words(DT, chunks, dev, &staged)) return WC_ERR_HIP;
        if (staged)
            hipLaunchKernelGGL((k_encode<DT, true>), dim3((uint32_t)((chunks + 1) / 2)), dim3(64), 0, stream, st,
                               out->tables, slots, meta, chunks, opts, out->raw);
        else
            hipLaunchKernelGGL((k_encode<DT, false>), dim3((uint32_t)((chunks + 1) / 2)), dim3(64), 0, stream, st,
                               out->tables, slots, meta, chunks, opts, out->raw);
    }
    if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return WC_ERR_HIP;
    const bool one_tile = chunks > 0 && chunks <= kScanTile;  // scan + compaction in one launch
    if (!one_tile) {
        // tile sums go to the spare slot after the last chunk's
        const uint32_t tiles = (uint32_t)((chunks + kScanTile - 1) / kScanTile);
        uint64_t *tile_sum = reinterpret_cast<uint64_t *>(slots + chunks * kSlotBytes);
        if (chunks)
            hipLaunchKernelGGL(k_scan_tiles, dim3(tiles), dim3(1024), 0, stream, meta, chunks, tile_sum);
        hipLaunchKernelGGL(k_scan_apply, dim3(tiles ? tiles : 1), dim3(1024), 0, stream, meta, chunks, tile_sum,
                           out->seek, out->payload_bytes, d_err);
    }
    if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return WC_ERR_HIP;
    if (one_tile) {
        hipLaunchKernelGGL(k_scan_compact, dim3((uint32_t)chunks), dim3(256), 0, stream, slots, meta, chunks,
                           out->seek, out->payload, out->payload_bytes, d_err);
    } else if (chunks) {
        hipLaunchKernelGGL(k_compact, dim3((uint32_t)chunks), dim3(256), 0, stream, slots, meta, out->seek,
                           out->payload, out->payload_bytes);
    }
    if (chunks && opts.crc()) {
        hipLaunchKernelGGL(k_crc32<false>, dim3((uint32_t)chunks), dim3(256), 0, stream, out->seek, out->payload,
                           out->payload_bytes, out->crc, d_err);
    }
    if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return WC_ERR_HIP;
    return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_HIP;
}

// Decoder variant.  While every chunk fits on the machine at once with one
// chunk per wavefront and the wide table (LDS-bound: 8 wavefronts per CU
// with one-dword refills, 7 with two-dword ones), the run is bound by the
// serial latency of one chunk, and the wide table's single LDS wait per step
// with no per-half selects is fastest.  With more chunks the narrow table's
// two chunks per wavefront and 12 wavefronts per CU win.  gfx950 allocates
// LDS to a workgroup in granules of 1,280 bytes (160 KiB / 128; measured:
// peak resident one-wavefront blocks per CU follow 163,840 div (bytes
// rounded up to 1,280), while the runtime's occupancy query assumes finer
// granules).
constexpr uint32_t kLdsPerCu = 160 * 1024;  // gfx950
constexpr uint32_t kLdsGranule = 1280;
constexpr uint32_t lds_blocks_per_cu(uint32_t bytes)
{
    return kLdsPerCu / ((bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule);
}
template <int kB>
constexpr uint32_t wide_waves_per_cu()
{
    return lds_blocks_per_cu((uint32_t)sizeof(DecSharedL1<1, kB>));
}
static_assert(wide_waves_per_cu<1>() == 8 && wide_waves_per_cu<2>() == 7, "wide decoder LDS footprint");
static_assert(lds_blocks_per_cu((uint32_t)sizeof(DecSharedS<2>)) == 12, "narrow decoder LDS footprint");

template <int kB>
bool use_wide_table(uint64_t chunks, int dev)
{
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    return chunks <= (uint64_t)wide_waves_per_cu<kB>() * (uint64_t)cus;
}

// Refill block (dwords per lane): the stream's words per 8-step group are
// about (bits per coded symbol) * 16; one-dword blocks supply 64 per group.
// Above 3.25 bits per symbol on average (52 words per group) the two-dword
// blocks keep speculative groups from outrunning the refills.
bool use_wide_refills(uint64_t payload_bytes, uint64_t n)
{
    return n && payload_bytes * 8 > n * 13 / 4;
}

template <int DT, int kB>
void launch_decode(const SegTable &st, uint64_t chunks, const wc_buffers *in, uint32_t *d_err,
                   hipStream_t stream, Opts opts, int dev)
{
    if (use_wide_table<kB>(chunks, dev)) {
        hipLaunchKernelGGL((k_decode<DT, true, 1, kB>), dim3((uint32_t)chunks), dim3(32), 0, stream, st, in->raw,
                           in->tables, in->seek, in->payload, in->payload_bytes, chunks, d_err, opts);
    } else {
        hipLaunchKernelGGL((k_decode<DT, false, 2, kB>), dim3((uint32_t)((chunks + 1) / 2)), dim3(64), 0, stream,
                           st, in->raw, in->tables, in->seek, in->payload, in->payload_bytes, chunks, d_err, opts);
    }
}

template <int DT>
wc_status decode_impl(const SegTable &st, uint64_t chunks, uint64_t n, const wc_buffers *in, uint32_t *d_err,
                      hipStream_t stream, Opts opts)
{
    if (chunks == 0) return WC_OK;
    int dev = 0;
    if (!stream_device(stream, &dev)) return WC_ERR_HIP;
    if (opts.crc()) {
        hipLaunchKernelGGL(k_crc32<true>, dim3((uint32_t)chunks), dim3(256), 0, stream, in->seek, in->payload,
                           in->payload_bytes, in->crc, d_err);
    }
    if (use_wide_refills(in->payload_bytes, n))
        launch_decode<DT, 2>(st, chunks, in, d_err, stream, opts, dev);
    else
        launch_decode<DT, 1>(st, chunks, in, d_err, stream, opts, dev);
    if (opts.raw_fallback()) {
        hipLaunchKernelGGL(k_decode_raw<DT>, dim3((uint32_t)chunks), dim3(256), 0, stream, st, in->raw, in->seek,
                           in->payload, in->payload_bytes, d_err);
    }
    return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_HIP;
}

// The kernels of a layout: BF16 and FP16 share the plain byte split.
wc_status encode_any(uint32_t format, const SegTable &st, uint64_t chunks, uint64_t raw_total,
                     const wc_buffers *out, void *d_scratch, uint32_t *d_err, hipStream_t stream, hipEvent_t *ev)
{
    const Opts o = opts_of(format);
    switch (layout_code(format)) {
    case WC_FP32: return encode_impl<WC_FP32>(st, chunks, raw_total, out, d_scratch, d_err, stream, ev, o);
    case WC_BF16_REORDER:
        return encode_impl<WC_BF16_REORDER>(st, chunks, raw_total, out, d_scratch, d_err, stream, ev, o);
    case WC_FP16_REORDER:
        return encode_impl<WC_FP16_REORDER>(st, chunks, raw_total, out, d_scratch, d_err, stream, ev, o);
    case WC_FP8_E4M3: return encode_impl<WC_FP8_E4M3>(st, chunks, raw_total, out, d_scratch, d_err, stream, ev, o);
    case WC_FP8_E5M2: return encode_impl<WC_FP8_E5M2>(st, chunks, raw_total, out, d_scratch, d_err, stream, ev, o);
    default: return encode_impl<WC_BF16>(st, chunks, raw_total, out, d_scratch, d_err, stream, ev, o);
    }
}

wc_status decode_any(uint32_t format, const SegTable &st, uint64_t chunks, uint64_t n, const wc_buffers *in,
                     uint32_t *d_err, hipStream_t stream)
{
    const Opts o = opts_of(format);
    switch (layout_code(format)) {
    case WC_FP32: return decode_impl<WC_FP32>(st, chunks, n, in, d_err, stream, o);
    case WC_BF16_REORDER: return decode_impl<WC_BF16_REORDER>(st, chunks, n, in, d_err, stream, o);
    case WC_FP16_REORDER: return decode_impl<WC_FP16_REORDER>(st, chunks, n, in, d_err, stream, o);
    case WC_FP8_E4M3: return decode_impl<WC_FP8_E4M3>(st, chunks, n, in, d_err, stream, o);
    case WC_FP8_E5M2: return decode_impl<WC_FP8_E5M2>(st, chunks, n, in, d_err, stream, o);
    default: return decode_impl<WC_BF16>(st, chunks, n, in, d_err, stream, o);
    }
}

// Most panels (16-row blocks of W) one chunk of a tile-ordered rows x cols
// matrix touches.
uint32_t panels_per_chunk(uint64_t n, uint32_t cols)
{
    const uint64_t tpp = cols / 16, tiles = n / 256;
    uint32_t most = 0;
    for (uint64_t t0 = 0; t0 < tiles; t0 += 256) {
        const uint64_t t1 = (t0 + 256 < tiles ? t0 + 256 : tiles) - 1;
        const uint32_t p = (uint32_t)(t1 / tpp - t0 / tpp + 1);
        most = p > most ? p : most;
    }
    return most;
}

template <int DT, int MT, int P>
void launch_gemm(const SegTable &st, uint64_t chunks, const wc_buffers *in, uint32_t *d_err, hipStream_t stream,
                 Opts opts, const wc_gemm *d_gemm, uint32_t m)
{
    hipLaunchKernelGGL((k_decode_gemm<DT, MT, P>), dim3((uint32_t)((chunks + 1) / 2)), dim3(64), 0, stream, st,
                       in->raw, in->tables, in->seek, in->payload, in->payload_bytes, chunks, d_err, opts, d_gemm, m);
}

// Accumulator sets per chunk for mt row blocks when a chunk touches at most
// p panels (P * mt <= 8 registers' worth), or 0 if none fits.
uint32_t gemm_panels(uint32_t mt, uint32_t p)
{
    if (mt == 1) return p <= 2 ? 2 : p <= 8 ? 8 : 0;
    if (mt == 2) return p <= 2 ? 2 : p <= 4 ? 4 : 0;
    return p <= 2 ? 2 : 0;
}

template <int DT>
void launch_gemm_any(uint32_t mt, uint32_t pp, const SegTable &st, uint64_t chunks, const wc_buffers *in,
                     uint32_t *d_err, hipStream_t stream, Opts opts, const wc_gemm *d_gemm, uint32_t m)
{
    if (mt == 1 && pp == 2) launch_gemm<DT, 1, 2>(st, chunks, in, d_err, stream, opts, d_gemm, m);
    else if (mt == 1) launch_gemm<DT, 1, 8>(st, chunks, in, d_err, stream, opts, d_gemm, m);
    else if (mt == 2 && pp == 2) launch_gemm<DT, 2, 2>(st, chunks, in, d_err, stream, opts, d_gemm, m);
    else if (mt == 2) launch_gemm<DT, 2, 4>(st, chunks, in, d_err, stream, opts, d_gemm, m);
    else launch_gemm<DT, 4, 2>(st, chunks, in, d_err, stream, opts, d_gemm, m);
}

}  // namespace

extern "C" {

int wc_version(void) { return kVersion; }

const char *wc_status_string(wc_status s)
{
    switch (s) {
    case WC_OK: return "ok";
    case WC_ERR_ARG: return "invalid argument";
    case WC_ERR_CAPACITY: return "buffer too small";
    case WC_ERR_CORRUPT: return "corrupt stream";
    case WC_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

wc_status wc_query_layout(wc_format format, uint64_t n, wc_layout *out)
{
    if (!out || !valid_format(format) || n > kMaxElems) return WC_ERR_ARG;
    layout_of(format, n, out);
    out->scratch_bytes = scratch_bytes_for(out->num_chunks, opts_of(format).tensor_table() ? 1 : 0);
    return WC_OK;
}

wc_status wc_plan_batch(wc_format format, wc_segment *segs, uint32_t nseg, wc_layout *total)
{
    if (!valid_format(format) || (nseg && !segs) || !total) return WC_ERR_ARG;
    uint64_t chunks = 0, raw = 0;
    for (uint32_t i = 0; i < nseg; i++) {
        if (segs[i].n > kMaxElems) return WC_ERR_ARG;
        segs[i].chunk_base = chunks;
        segs[i].raw_base = raw;
        chunks += (segs[i].n + kChunk - 1) / kChunk;
        raw += raw_bytes_of(layout_code(format), segs[i].n);
        if (i + 1 < nseg) raw = align_up(raw, 256);
    }
    return check_plan(format, segs, nseg, total, false);
}

wc_status wc_encode(wc_format format, const void *d_in, uint64_t n, const wc_buffers *out, void *d_scratch,
                    uint64_t scratch_bytes, uint32_t *d_err, hipStream_t stream, hipEvent_t *stage_events)
{
    if (!valid_format(format) || n > kMaxElems) return WC_ERR_ARG;
    wc_layout lay;
    wc_query_layout(format, n, &lay);
    wc_status s = check_buffers(out, lay.num_chunks, lay.raw_bytes, lay.table_bytes, lay.crc_bytes);
    if (s != WC_OK) return s;
    if (n && (!d_in || !aligned(d_in, 16))) return WC_ERR_ARG;
    if (lay.num_chunks && (!d_scratch || !aligned(d_scratch, 256))) return WC_ERR_ARG;
    if (scratch_bytes < lay.scratch_bytes) return WC_ERR_CAPACITY;
    if (d_err && !aligned(d_err, 4)) return WC_ERR_ARG;
    SegTable st{nullptr, 0, {reinterpret_cast<uint64_t>(d_in), n, 0, 0}};
    return encode_any(format, st, lay.num_chunks, lay.raw_bytes, out, d_scratch, d_err, stream, stage_events);
}

int wc_set_encoder_words(int mode)
{
    if (mode != WC_ENC_WORDS_AUTO && mode != WC_ENC_WORDS_DIRECT && mode != WC_ENC_WORDS_STAGED) return -1;
    return g_enc_words.exchange(mode);
}

wc_status wc_encode_variant(wc_format format, uint64_t num_chunks, hipStream_t stream, int *staged)
{
    if (!valid_format(format) || !staged) return WC_ERR_ARG;
    int dev = 0;
    bool st = false;
    if (!stream_device(stream, &dev) || !use_staged_words(layout_code(format), num_chunks, dev, &st))
        return WC_ERR_HIP;
    *staged = st ? 1 : 0;
    return WC_OK;
}

wc_status wc_decode_variant(wc_format format, uint64_t num_chunks, uint64_t n, uint64_t payload_bytes,
                            hipStream_t stream, int *one_chunk_per_wave, int *refill_dwords)
{
    if (!valid_format(format) || !one_chunk_per_wave || !refill_dwords) return WC_ERR_ARG;
    int dev = 0;
    if (!stream_device(stream, &dev)) return WC_ERR_HIP;
    const bool wide_refill = use_wide_refills(payload_bytes, n);
    *refill_dwords = wide_refill ? 2 : 1;
    *one_chunk_per_wave = wide_refill ? use_wide_table<2>(num_chunks, dev) : use_wide_table<1>(num_chunks, dev);
    return WC_OK;
}

wc_status wc_decode(wc_format format, const wc_buffers *in, uint64_t n, void *d_out, uint32_t *d_err,
                    hipStream_t stream)
{
    if (!valid_format(format) || n > kMaxElems) return WC_ERR_ARG;
    wc_layout lay;
    wc_query_layout(format, n, &lay);
    wc_status s = check_buffers(in, lay.num_chunks, lay.raw_bytes, lay.num_chunks ? lay.table_bytes : 0,
                                lay.crc_bytes);
    if (s != WC_OK) return s;
    if (n && (!d_out || !aligned(d_out, 16))) return WC_ERR_ARG;
    if (d_err && !aligned(d_err, 4)) return WC_ERR_ARG;
    SegTable st{nullptr, 0, {reinterpret_cast<uint64_t>(d_out), n, 0, 0}};
    return decode_any(format, st, lay.num_chunks, n, in, d_err, stream);
}

wc_status wc_encode_batch(wc_format format, const wc_segment *h_segs, const wc_segment *d_segs, uint32_t nseg,
                          const wc_buffers *out, void *d_scratch, uint64_t scratch_bytes, uint32_t *d_err,
                          hipStream_t stream, hipEvent_t *stage_events)
{
    if (!valid_format(format) || nseg == 0 || !h_segs || !d_segs || !aligned(d_segs, 8)) return WC_ERR_ARG;
    wc_layout tot;
    wc_status s = check_plan(format, h_segs, nseg, &tot);
    if (s != WC_OK) return s;
    s = check_buffers(out, tot.num_chunks, tot.raw_bytes, tot.table_bytes, tot.crc_bytes);
    if (s != WC_OK) return s;
    if (tot.num_chunks && (!d_scratch || !aligned(d_scratch, 256))) return WC_ERR_ARG;
    if (scratch_bytes < tot.scratch_bytes) return WC_ERR_CAPACITY;
    if (d_err && !aligned(d_err, 4)) return WC_ERR_ARG;
    SegTable st{d_segs, nseg, {0, 0, 0, 0}};
    return encode_any(format, st, tot.num_chunks, tot.raw_bytes, out, d_scratch, d_err, stream, stage_events);
}

wc_status wc_decode_batch(wc_format format, const wc_segment *h_segs, const wc_segment *d_segs, uint32_t nseg,
                          const wc_buffers *in, uint32_t *d_err, hipStream_t stream)
{
    if (!valid_format(format) || nseg == 0 || !h_segs || !d_segs || !aligned(d_segs, 8)) return WC_ERR_ARG;
    wc_layout tot;
    wc_status s = check_plan(format, h_segs, nseg, &tot);
    if (s != WC_OK) return s;
    s = check_buffers(in, tot.num_chunks, tot.raw_bytes, tot.num_chunks ? tot.table_bytes : 0, tot.crc_bytes);
    if (s != WC_OK) return s;
    if (d_err && !aligned(d_err, 4)) return WC_ERR_ARG;
    SegTable st{d_segs, nseg, {0, 0, 0, 0}};
    return decode_any(format, st, tot.num_chunks, tot.n, in, d_err, stream);
}

wc_status wc_tile_order(const void *d_in, void *d_out, uint32_t rows, uint32_t cols, int inverse, hipStream_t stream)
{
    const uint64_t n = (uint64_t)rows * cols;
    if ((rows % 16) || (cols % 16) || n >= (1ull << 32)) return WC_ERR_ARG;
    if (n == 0) return WC_OK;
    if (!d_in || !d_out || !aligned(d_in, 16) || !aligned(d_out, 16)) return WC_ERR_ARG;
    const char *a = static_cast<const char *>(d_in), *b = static_cast<const char *>(d_out);
    if (a < b + 2 * n && b < a + 2 * n) return WC_ERR_ARG;  // overlapping
    const uint64_t threads = n / 8;
    hipLaunchKernelGGL(k_tile_order, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(d_in), static_cast<uint16_t *>(d_out), rows, cols,
                       inverse ? 1u : 0u);
    return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_HIP;
}

wc_status wc_decode_gemm_batch(wc_format format, const wc_segment *h_segs, const wc_segment *d_segs, uint32_t nseg,
                               const wc_gemm *h_gemm, const wc_gemm *d_gemm, uint32_t m, const wc_buffers *in,
                               uint32_t *d_err, hipStream_t stream)
{
    if (!valid_format(format) || nseg == 0 || !h_segs || !d_segs || !aligned(d_segs, 8)) return WC_ERR_ARG;
    const int lay = layout_code(format);
    if ((lay != WC_BF16 && lay != WC_BF16_REORDER) || opts_of(format).raw_fallback()) return WC_ERR_ARG;
    if (!h_gemm || !d_gemm || !aligned(d_gemm, 8) || m < 1 || m > 64) return WC_ERR_ARG;
    wc_layout tot;
    wc_status s = check_plan(format, h_segs, nseg, &tot, false);  // segment ptr unused
    if (s != WC_OK) return s;
    s = check_buffers(in, tot.num_chunks, tot.raw_bytes, tot.num_chunks ? tot.table_bytes : 0, tot.crc_bytes);
    if (s != WC_OK) return s;
    if (d_err && !aligned(d_err, 4)) return WC_ERR_ARG;
    const uint32_t mt = m <= 16 ? 1 : m <= 32 ? 2 : 4;
    uint32_t most = 0;
    for (uint32_t i = 0; i < nseg; i++) {
        const wc_gemm &g = h_gemm[i];
        const uint64_t n = (uint64_t)g.rows * g.cols;
        if ((g.rows % 16) || (g.cols % 16) || n != h_segs[i].n || n >= (1ull << 32)) return WC_ERR_ARG;
        if (n && (!g.x || !g.y || (g.x % 8) || (g.y % 4))) return WC_ERR_ARG;
        if (n) {
            const uint32_t p = panels_per_chunk(n, g.cols);
            most = p > most ? p : most;
        }
    }
    const uint32_t pp = gemm_panels(mt, most);
    if (pp == 0) return WC_ERR_ARG;  // before anything is launched
    if (tot.num_chunks == 0) return WC_OK;
    SegTable st{d_segs, nseg, {0, 0, 0, 0}};
    const Opts o = opts_of(format);
    if (o.crc()) {
        hipLaunchKernelGGL(k_crc32<true>, dim3((uint32_t)tot.num_chunks), dim3(256), 0, stream, in->seek,
                           in->payload, in->payload_bytes, in->crc, d_err);
    }
    if (lay == WC_BF16)
        launch_gemm_any<WC_BF16>(mt, pp, st, tot.num_chunks, in, d_err, stream, o, d_gemm, m);
    else
        launch_gemm_any<WC_BF16_REORDER>(mt, pp, st, tot.num_chunks, in, d_err, stream, o, d_gemm, m);
    return hipGetLastError() == hipSuccess ? WC_OK : WC_ERR_HIP;
}

uint64_t wc_check_division(uint32_t samples_per_divisor)
{
    uint64_t bad = 0;
    uint64_t rng = 0x9E3779B97F4A7C15ull;
    static constexpr DivTable table = make_div_table();
    for (uint32_t d = 1; d <= kM; d++) {
        const DivConst c = div_const(d);
        // the compile-time table the encoder kernel reads must agree
        const uint32_t l = table.l[d];
        if (table.mp[d] != c.mp || (l < 1 ? l : 1u) != c.sh1 || (l > 1 ? l - 1 : 0u) != c.sh2) bad++;
        auto check = [&](uint32_t x) {
            if (div_exact(x, c.mp, c.sh1, c.sh2) != x / d) bad++;
        };
        const uint32_t qmax = 0xFFFFFFFFu / d;
        const uint32_t fixed[] = {0u, 1u, d - 1, d, d + 1, 0xFFFFFFFFu, 0xFFFFFFFFu - d, 0x7FFFFFFFu,
                                  0x80000000u, (d << 20) - 1, qmax * d, qmax * d - 1, qmax * d + (d - 1)};
        for (uint32_t x : fixed) check(x);
        for (uint32_t i = 0; i < samples_per_divisor; i++) {
            rng = rng * 6364136223846793005ull + 1442695040888963407ull;
            const uint32_t q = (uint32_t)((rng >> 32) % ((uint64_t)qmax + 1));
            const uint32_t r = (uint32_t)(rng >> 8) % d;
            const uint64_t x = (uint64_t)q * d + r;
            if (x <= 0xFFFFFFFFu) check((uint32_t)x);
            check(q * d);
            if (q) check(q * d - 1);
        }
        // the state update the kernel runs: every xr in [1, d 2^20) it can
        // see, at the range's ends and sampled, with the start at both ends
        const EncConst e0 = enc_const(table.mp[d], l, d, 0), e1 = enc_const(table.mp[d], l, d, kM - d);
        auto check_update = [&](uint32_t xr) {
            const uint32_t exact = kM * (xr / d) + xr % d;
            if (enc_update(xr, e0.mp, e0.fm, e0.bb) != exact) bad++;
            if (enc_update(xr, e1.mp, e1.fm, e1.bb) != exact + (kM - d)) bad++;
        };
        const uint32_t xmax = (uint32_t)(((uint64_t)d << 20) - 1);
        const uint32_t ends[] = {1u, 2u, d - 1 ? d - 1 : 1u, d, d + 1, 65535u, 65536u, xmax, xmax - 1, xmax - d};
        for (uint32_t x : ends)
            if (x >= 1 && x <= xmax) check_update(x);
        for (uint32_t i = 0; i < samples_per_divisor; i++) {
            rng = rng * 6364136223846793005ull + 1442695040888963407ull;
            check_update(1u + (uint32_t)((rng >> 24) % xmax));
        }
    }
    return bad;
}

}  // extern "C"
