// Chunked KV transfer over a bandwidth-limited link, with or without SplitZip
// compression ("SplitZip: Ultra Fast Lossless KV Compression for
// Disaggregated LLM Serving", gist.science summary page: Problem section, the
// prefill-to-decode KV transfer over 50-100 GB/s links; Results, transfer
// latency: a smaller payload shortens the transfer, and the codec's own time
// is a small share of it for long sequences).
//
// One GPU stands in for both ends.  The link is the PCIe path through pinned
// host memory: the sender's bytes go device -> host (D2H), the receiver's
// come host -> device (H2D), the host buffer playing the wire.  A tensor is
// sent in chunks (for a KV cache, one layer each); with compression every
// chunk is encoded into its own SplitZip stream, exactly the stream's bytes
// cross the link, and the receiver decodes the chunk into place.  Three
// streams (codec, D2H, H2D) and `depth` buffer slots let the stages of
// consecutive chunks overlap; events order the reuse of every slot.  Encode
// and decode share one stream: with the caller's stream that makes four,
// the number of hardware queues a process gets by default, so no two
// streams share a queue (a wait queued on a shared queue would also hold
// back the other stream's copies and serialise the two link directions).
// Host code only: the kernels are the codec's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdint>
#include <cstring>
#include <vector>

#include "splitzip.h"

namespace {

constexpr int kMaxDepth = 8;
constexpr uint64_t kHeaderBytes = 64;

uint64_t up256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

// The pipeline's streams, created by each sz_transfer call and destroyed
// before it returns (the library keeps no streams between calls): default
// priority, non-blocking with respect to the null stream; `dec` is `enc`.
struct PipelineStreams {
    hipStream_t enc = nullptr, d2h = nullptr, h2d = nullptr, dec = nullptr;
    int create()
    {
        hipStream_t *all[3] = {&enc, &d2h, &h2d};
        for (hipStream_t *s : all)
            if (hipStreamCreateWithFlags(s, hipStreamNonBlocking) != hipSuccess) return SZ_E_HIP;
        dec = enc;
        return SZ_OK;
    }
    ~PipelineStreams()
    {
        // every use has been synchronised by then; destroying waits for the
        // stream's work anyway
        hipStream_t all[3] = {enc, d2h, h2d};
        for (hipStream_t s : all)
            if (s) (void)hipStreamDestroy(s);
    }
};

struct Events {
    std::vector<hipEvent_t> all;
    ~Events()
    {
        for (hipEvent_t e : all) (void)hipEventDestroy(e);
    }
    hipEvent_t make()
    {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
        all.push_back(e);
        return e;
    }
};

uint64_t elem_bytes(int dtype) { return dtype == SZ_BF16 ? 2 : 1; }

// Per-slot capacity of one chunk's stream (its worst case), 256-aligned.
uint64_t slot_bytes(int dtype, uint64_t chunk_elems) { return up256(sz_encoded_size(dtype, chunk_elems, chunk_elems)); }

uint64_t chunk_count(uint64_t n, uint64_t chunk) { return chunk ? (n + chunk - 1) / chunk : 0; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Copies a few words (a stream header, a status word) into pinned host
// memory from a kernel on the given stream.  A DMA copy of the same bytes
// would queue behind the chunk-sized copies on the DMA engine of that
// direction and hold back the stream it was issued on.
__global__ void sz_copy_words(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst, uint32_t words)
{
    if (threadIdx.x < words) dst[threadIdx.x] = src[threadIdx.x];
}

#define SZ_HIP_TRY(call)                          \
    do {                                          \
        if ((call) != hipSuccess) return SZ_E_HIP; \
    } while (0)

}  // namespace

extern "C" uint64_t sz_transfer_workspace_size(int dtype, uint64_t chunk_elems, int depth)
{
    if ((dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) || depth < 1 || depth > kMaxDepth) return 0;
    // send and receive slot buffers, then the encode and the decode workspace
    return 2 * (uint64_t)depth * slot_bytes(dtype, chunk_elems) + up256(sz_workspace_size(dtype, chunk_elems)) +
           up256(sz_decode_workspace_size(dtype, chunk_elems));
}

extern "C" uint64_t sz_transfer_host_bytes(int dtype, uint64_t n_elems, uint64_t chunk_elems, int depth)
{
    if ((dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) || depth < 1 || depth > kMaxDepth || chunk_elems == 0) return 0;
    // wire slots, one stream header per slot, one decode status per chunk
    return (uint64_t)depth * slot_bytes(dtype, chunk_elems) + (uint64_t)depth * kHeaderBytes +
           up256(4 * chunk_count(n_elems, chunk_elems));
}

extern "C" int sz_transfer(int dtype, const void *d_src, uint64_t n_elems, uint64_t chunk_elems,
                           const sz_codebook *cb, int compress, int depth, void *h_staging, uint64_t h_bytes,
                           void *d_dst, void *d_ws, uint64_t ws_bytes, void *stream, sz_transfer_stats *stats)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    if (depth < 1 || depth > kMaxDepth || chunk_elems == 0 || (chunk_elems * elem_bytes(dtype)) % 16) return SZ_E_ARG;
    if (!stats || !h_staging || !d_ws || (n_elems && (!d_src || !d_dst)) || (compress && !cb)) return SZ_E_ARG;
    if (!aligned16(d_src) || !aligned16(d_dst) || !aligned16(d_ws) || !aligned16(h_staging)) return SZ_E_ALIGN;
    if (h_bytes < sz_transfer_host_bytes(dtype, n_elems, chunk_elems, depth)) return SZ_E_WORKSPACE;
    if (ws_bytes < sz_transfer_workspace_size(dtype, chunk_elems, depth)) return SZ_E_WORKSPACE;

    PipelineStreams st;
    int rc = st.create();
    if (rc) return rc;
    const uint64_t esz = elem_bytes(dtype);
    const uint64_t chunks = chunk_count(n_elems, chunk_elems);
    const uint64_t slot = slot_bytes(dtype, chunk_elems);
    uint8_t *dws = static_cast<uint8_t *>(d_ws);
    uint8_t *send = dws;                                         // depth slots
    uint8_t *recv = dws + (uint64_t)depth * slot;                // depth slots
    uint8_t *enc_ws = dws + 2 * (uint64_t)depth * slot;
    const uint64_t codec_ws = up256(sz_workspace_size(dtype, chunk_elems));
    const uint64_t dec_ws_bytes = up256(sz_decode_workspace_size(dtype, chunk_elems));
    uint8_t *dec_ws = enc_ws + codec_ws;
    uint8_t *wire = static_cast<uint8_t *>(h_staging);
    uint8_t *headers = wire + (uint64_t)depth * slot;
    int32_t *statuses = reinterpret_cast<int32_t *>(headers + (uint64_t)depth * kHeaderBytes);
    // the device's view of the pinned staging, for the word copies
    void *h_dev = nullptr;
    if (hipHostGetDevicePointer(&h_dev, h_staging, 0) != hipSuccess || !h_dev) return SZ_E_ARG;
    uint8_t *headers_dev = static_cast<uint8_t *>(h_dev) + (uint64_t)depth * slot;
    int32_t *statuses_dev = reinterpret_cast<int32_t *>(headers_dev + (uint64_t)depth * kHeaderBytes);
    const uint8_t *src = static_cast<const uint8_t *>(d_src);
    uint8_t *dst = static_cast<uint8_t *>(d_dst);

    Events ev;
    hipEvent_t done = ev.make();
    hipEvent_t encoded[kMaxDepth], sent[kMaxDepth], received[kMaxDepth], decoded[kMaxDepth];
    for (int k = 0; k < depth; ++k) {
        encoded[k] = ev.make();
        sent[k] = ev.make();
        received[k] = ev.make();
        decoded[k] = ev.make();
        if (!encoded[k] || !sent[k] || !received[k] || !decoded[k]) return SZ_E_HIP;
    }
    if (!done) return SZ_E_HIP;
    hipStream_t caller = static_cast<hipStream_t>(stream);

    // the input is complete once the caller's stream has reached this point
    SZ_HIP_TRY(hipStreamSynchronize(caller));
    std::memset(stats, 0, sizeof(*stats));
    const auto t0 = std::chrono::steady_clock::now();
    uint64_t wire_bytes = 0, escapes = 0;
    auto chunk_len = [&](uint64_t i) { return std::min<uint64_t>(chunk_elems, n_elems - i * chunk_elems); };

    // the pipeline; on an error the streams are drained below before returning
    auto body = [&]() -> int {
        if (!compress) {
            for (uint64_t i = 0; i < chunks; ++i) {
                const int k = (int)(i % depth);
                const uint64_t bytes = chunk_len(i) * esz;
                if (i >= (uint64_t)depth) SZ_HIP_TRY(hipStreamWaitEvent(st.d2h, received[k], 0));
                SZ_HIP_TRY(hipMemcpyAsync(wire + k * slot, src + i * chunk_elems * esz, bytes, hipMemcpyDeviceToHost,
                                          st.d2h));
                SZ_HIP_TRY(hipEventRecord(sent[k], st.d2h));
                SZ_HIP_TRY(hipStreamWaitEvent(st.h2d, sent[k], 0));
                SZ_HIP_TRY(hipMemcpyAsync(dst + i * chunk_elems * esz, wire + k * slot, bytes, hipMemcpyHostToDevice,
                                          st.h2d));
                SZ_HIP_TRY(hipEventRecord(received[k], st.h2d));
                wire_bytes += bytes;
            }
            SZ_HIP_TRY(hipEventRecord(done, st.h2d));
        } else {
            // encode chunk i into send slot i % depth, then copy its header out
            auto issue_encode = [&](uint64_t i) -> int {
                const int k = (int)(i % depth);
                if (i >= (uint64_t)depth) SZ_HIP_TRY(hipStreamWaitEvent(st.enc, sent[k], 0));
                const int r = sz_encode(dtype, src + i * chunk_elems * esz, chunk_len(i), cb, send + k * slot, slot,
                                        enc_ws, codec_ws, st.enc);
                if (r) return r;
                hipLaunchKernelGGL(sz_copy_words, dim3(1), dim3(64), 0, st.enc,
                                   reinterpret_cast<const uint32_t *>(send + k * slot),
                                   reinterpret_cast<uint32_t *>(headers_dev + k * kHeaderBytes),
                                   (uint32_t)(kHeaderBytes / 4));
                SZ_HIP_TRY(hipGetLastError());
                SZ_HIP_TRY(hipEventRecord(encoded[k], st.enc));
                return SZ_OK;
            };
            for (uint64_t i = 0; i < chunks && i < (uint64_t)depth; ++i)
                if ((rc = issue_encode(i))) return rc;
            for (uint64_t i = 0; i < chunks; ++i) {
                const int k = (int)(i % depth);
                // the stream's size is known once its header has arrived
                SZ_HIP_TRY(hipEventSynchronize(encoded[k]));
                uint64_t e = 0;
                std::memcpy(&e, headers + k * kHeaderBytes + 16, 8);
                const uint64_t m = chunk_len(i);
                if (e > m) return SZ_E_FORMAT;
                const uint64_t bytes = sz_encoded_size(dtype, m, e);
                // D2H into wire slot k once the receiver has taken chunk i - depth out of it
                if (i >= (uint64_t)depth) SZ_HIP_TRY(hipStreamWaitEvent(st.d2h, received[k], 0));
                SZ_HIP_TRY(hipMemcpyAsync(wire + k * slot, send + k * slot, bytes, hipMemcpyDeviceToHost, st.d2h));
                SZ_HIP_TRY(hipEventRecord(sent[k], st.d2h));
                // H2D into receive slot k once chunk i - depth has been decoded out of it
                SZ_HIP_TRY(hipStreamWaitEvent(st.h2d, sent[k], 0));
                if (i >= (uint64_t)depth) SZ_HIP_TRY(hipStreamWaitEvent(st.h2d, decoded[k], 0));
                SZ_HIP_TRY(hipMemcpyAsync(recv + k * slot, wire + k * slot, bytes, hipMemcpyHostToDevice, st.h2d));
                SZ_HIP_TRY(hipEventRecord(received[k], st.h2d));
                SZ_HIP_TRY(hipStreamWaitEvent(st.dec, received[k], 0));
                rc = sz_decode(recv + k * slot, bytes, dtype, dst + i * chunk_elems * esz, m, dec_ws, dec_ws_bytes, st.dec);
                if (rc) return rc;
                hipLaunchKernelGGL(sz_copy_words, dim3(1), dim3(64), 0, st.dec, reinterpret_cast<const uint32_t *>(dec_ws),
                                   reinterpret_cast<uint32_t *>(statuses_dev + i), 1u);
                SZ_HIP_TRY(hipGetLastError());
                SZ_HIP_TRY(hipEventRecord(decoded[k], st.dec));
                wire_bytes += bytes;
                escapes += e;
                if (i + depth < chunks && (rc = issue_encode(i + depth))) return rc;
            }
            SZ_HIP_TRY(hipEventRecord(done, st.dec));
        }
        return SZ_OK;
    };
    rc = body();
    hipStream_t all[3] = {st.enc, st.d2h, st.h2d};
    for (hipStream_t s : all)
        if (hipStreamSynchronize(s) != hipSuccess && rc == SZ_OK) rc = SZ_E_HIP;
    if (rc) return rc;
    // the call returns with the received tensor complete
    SZ_HIP_TRY(hipEventSynchronize(done));
    const auto t1 = std::chrono::steady_clock::now();
    stats->total_ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
    stats->chunks = chunks;
    stats->raw_bytes = n_elems * esz;
    stats->wire_bytes = wire_bytes;
    stats->escapes = escapes;
    stats->decode_status = 0;
    if (compress)
        for (uint64_t i = 0; i < chunks; ++i)
            if (statuses[i] != 0) {
                stats->decode_status = statuses[i];
                break;
            }
    return SZ_OK;
}
