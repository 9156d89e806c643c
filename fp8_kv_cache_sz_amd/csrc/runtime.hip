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
