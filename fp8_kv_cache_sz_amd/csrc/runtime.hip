// Runtime pieces of the SplitZip library that are not the codec: the launch
// instrumentation (per-kernel HIP events) and the reference streaming copy
// that measurement compares the codec kernels against.
#include "common.hpp"

namespace sz {

std::mutex g_prof_mutex;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event()
{
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void release_records()
{
    for (auto &r : g_prof_records) {
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_prof_records.clear();
}

}  // namespace sz

using namespace sz;

// ---------------------------------------------------------------------------
// Kernel: reference streaming copy (not part of the codec).  Each 256-lane
// workgroup moves one 4 KB tile, one 16-byte word per lane, with a
// non-temporal load and store.  Streaming probes on MI355X found this the
// fastest plain copy shape: more words per lane (larger tiles) copy more
// slowly, so this is the practical ceiling of a two-stream byte mix.
// ---------------------------------------------------------------------------
constexpr uint32_t kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void sz_ref_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                            uint64_t words)
{
    const uint64_t i = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (i < words) store_nt(dst + i, load_nt(src + i));
}

extern "C" int sz_reference_copy(const void *d_src, void *d_dst, uint64_t bytes, void *stream)
{
    if (bytes % 16 != 0) return SZ_E_ARG;
    if (bytes == 0) return SZ_OK;
    if (!d_src || !d_dst) return SZ_E_ARG;
    if (!aligned16(d_src) || !aligned16(d_dst)) return SZ_E_ALIGN;
    const uint8_t *s8 = static_cast<const uint8_t *>(d_src);
    const uint8_t *d8 = static_cast<const uint8_t *>(d_dst);
    if (s8 < d8 + bytes && d8 < s8 + bytes) return SZ_E_ARG;      // overlapping ranges
    const uint64_t words = bytes / 16;
    const uint64_t groups = (words + kCopyThreads - 1) / kCopyThreads;
    if (groups > 0xFFFFFFFFull) return SZ_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    LaunchScope scope("sz_ref_copy", s);
    hipLaunchKernelGGL(sz_ref_copy, dim3((uint32_t)groups), dim3(kCopyThreads), 0, s,
                       static_cast<const uint4 *>(d_src), static_cast<uint4 *>(d_dst), words);
    return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
}

// ---------------------------------------------------------------------------
// Kernel: reference of the dense encoders' memory pattern (not part of the
// codec).  The same grid, tile, lane mapping and memory instructions as
// sz_enc_dense_bf16 / sz_enc_dense_e5m2 on whole 16K tiles, with trivial
// arithmetic in place of the encoding and no escape staging:
//   BF16, per 8-element chunk (one non-temporal dwordx4 load): sym = the
//     low bytes of the 8 elements (dwordx2 store), codes = high bytes of
//     elements 0..3 XOR those of elements 4..7 (dword store);
//   E5M2, per 32-element chunk (two dwordx4 loads, halves a and b):
//     codes = a XOR b (dwordx4 store), sym = bytes 0..11 of b (dwordx3).
// Its rate is the practical ceiling of the encoders' one-read, two-write
// stream mix, against which the encoders' own rate is read.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kEncThreads) void sz_ref_split(const uint8_t *__restrict__ in, uint8_t *__restrict__ codes,
                                                            uint8_t *__restrict__ sym)
{
    const uint32_t lane = lane_id();
    const uint64_t base = (uint64_t)blockIdx.x * kEncTile + (uint64_t)(threadIdx.x / 64) * kRow;
    if (DT == SZ_BF16) {
        uint4 q[kBf16Chunks];
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j)
            q[j] = load_nt(reinterpret_cast<const uint4 *>(in + 2 * (base + (uint64_t)(j * 64 + lane) * 8)));
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 8;
            const uint32_t lo_a = perm(q[j].y, q[j].x, 0x06040200u), lo_b = perm(q[j].w, q[j].z, 0x06040200u);
            const uint32_t hi_a = perm(q[j].y, q[j].x, 0x07050301u), hi_b = perm(q[j].w, q[j].z, 0x07050301u);
            store_nt(reinterpret_cast<uint32_t *>(codes + c0 / 2), hi_a ^ hi_b);
            store_nt(reinterpret_cast<uint2 *>(sym + c0), make_uint2(lo_a, lo_b));
        }
    } else {
        uint4 a[kE5Chunks], b[kE5Chunks];
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
            a[j] = load_nt(reinterpret_cast<const uint4 *>(in + c0));
            b[j] = load_nt(reinterpret_cast<const uint4 *>(in + c0 + 16));
        }
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
            store_nt(reinterpret_cast<uint4 *>(codes + c0 / 2),
                     make_uint4(a[j].x ^ b[j].x, a[j].y ^ b[j].y, a[j].z ^ b[j].z, a[j].w ^ b[j].w));
            const uint32_t w[3] = {b[j].x, b[j].y, b[j].z};
            store3_nt(reinterpret_cast<uint32_t *>(sym + (c0 / 32) * 12), w);
        }
    }
}

extern "C" int sz_reference_split(int dtype, const void *d_in, uint64_t n_elems, void *d_codes, void *d_sym,
                                  void *stream)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    if (n_elems % kEncTile != 0) return SZ_E_ARG;
    if (n_elems == 0) return SZ_OK;
    if (!d_in || !d_codes || !d_sym) return SZ_E_ARG;
    if (!aligned16(d_in) || !aligned16(d_codes) || !aligned16(d_sym)) return SZ_E_ALIGN;
    const uint64_t tiles = n_elems / kEncTile;
    if (tiles > 0xFFFFFFFFull) return SZ_E_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    LaunchScope scope("sz_ref_split", s);
    if (dtype == SZ_BF16)
        hipLaunchKernelGGL(sz_ref_split<SZ_BF16>, dim3((uint32_t)tiles), dim3(kEncThreads), 0, s,
                           static_cast<const uint8_t *>(d_in), static_cast<uint8_t *>(d_codes),
                           static_cast<uint8_t *>(d_sym));
    else
        hipLaunchKernelGGL(sz_ref_split<SZ_FP8_E5M2>, dim3((uint32_t)tiles), dim3(kEncThreads), 0, s,
                           static_cast<const uint8_t *>(d_in), static_cast<uint8_t *>(d_codes),
                           static_cast<uint8_t *>(d_sym));
    return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
}

extern "C" int sz_profile_enable(int on)
{
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    for (auto &r : g_prof_records) {
        (void)hipEventSynchronize(r.stop);
    }
    release_records();
    g_prof_on.store(on != 0, std::memory_order_release);
    return SZ_OK;
}

extern "C" int sz_profile_collect(sz_kernel_stat *stats, int max_stats)
{
    if (max_stats < 0 || (max_stats > 0 && !stats)) return SZ_E_ARG;
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    std::vector<sz_kernel_stat> acc;
    int rc = SZ_OK;
    for (auto &r : g_prof_records) {
        if (hipEventSynchronize(r.stop) != hipSuccess) {
            rc = SZ_E_HIP;
            continue;
        }
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
            rc = SZ_E_HIP;
            continue;
        }
        auto it = std::find_if(acc.begin(), acc.end(),
                               [&](const sz_kernel_stat &k) { return std::strcmp(k.name, r.name) == 0; });
        if (it == acc.end()) {
            sz_kernel_stat k{};
            std::strncpy(k.name, r.name, sizeof(k.name) - 1);
            acc.push_back(k);
            it = acc.end() - 1;
        }
        it->launches += 1;
        it->total_ms += ms;
    }
    release_records();
    if (rc != SZ_OK) return rc;
    const int count = std::min<int>(max_stats, (int)acc.size());
    for (int i = 0; i < count; ++i) stats[i] = acc[i];
    return count;
}
