// SplitZip calibration: the offline Top-16 codebook on the host, and the
// on-device exponent histogram and Top-16 selection ("SplitZip: Ultra Fast
// Lossless KV Compression for Disaggregated LLM Serving", gist.science
// summary page, Method, fixed-length coding bullet; Results, calibration
// ablation).
#include "common.hpp"

namespace sz {
namespace {

// ---------------------------------------------------------------------------
// On-device calibration: the exponent histogram and the Top-16 selection run
// on the GPU, so a codebook can be fitted to each tensor, or to a sample of
// its 64K blocks, with no host round trip.  (The page's calibration ablation
// weighs such per-tensor books against one offline book.)
//
// sz_cal_hist: every 512-lane workgroup walks 4096-element rows of the
// sampled blocks (grid-stride over rows) and counts exponents in LDS with one
// counter per (symbol, lane), so the 64 lanes of a ds_add never share a word
// and the waves of the workgroup meet only through the atomic add.  It then
// writes its per-symbol totals to column g of partial[symbol][groups].
// sz_cal_select: one workgroup sums each symbol's row of partial counts with
// dwordx4 loads, ranks the symbols by (count descending, symbol ascending),
// and writes the first 16 as the codebook (and the histogram, if asked).
// ---------------------------------------------------------------------------
constexpr uint32_t kCalThreads = 512;
constexpr uint32_t kCalMaxGroups = 512;          // two workgroups per CU
constexpr uint32_t kCalRowsPerBlock = kBlock / kRow;
constexpr uint32_t kSelectThreads = 1024;

template <int DT>
__global__ __launch_bounds__(kCalThreads) void sz_cal_hist(const void *__restrict__ in, uint64_t n, uint64_t every,
                                                           uint64_t rows, uint32_t *__restrict__ partial,
                                                           uint32_t groups)
{
    constexpr uint32_t S = DT == SZ_BF16 ? 256 : 32;
    __shared__ uint32_t cnt[S * 64];
    for (uint32_t i = threadIdx.x; i < S * 64; i += kCalThreads) cnt[i] = 0;
    __syncthreads();
    const uint32_t lane = lane_id();
    const uint64_t waves = (uint64_t)gridDim.x * (kCalThreads / 64);
    for (uint64_t r = (uint64_t)blockIdx.x * (kCalThreads / 64) + threadIdx.x / 64; r < rows; r += waves) {
        const uint64_t base = (r / kCalRowsPerBlock) * every * kBlock + (r % kCalRowsPerBlock) * kRow;
        if (base >= n) continue;
        const bool full_row = base + kRow <= n;
        if (DT == SZ_BF16) {
            const uint16_t *src = static_cast<const uint16_t *>(in) + base;
            if (full_row) {
                uint4 q[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = load_nt(reinterpret_cast<const uint4 *>(src) + j * 64 + lane);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        atomicAdd(&cnt[((w[k] >> 7) & 0xFFu) * 64 + lane], 1u);
                        atomicAdd(&cnt[((w[k] >> 23) & 0xFFu) * 64 + lane], 1u);
                    }
                }
            } else {
                for (uint64_t k = lane; base + k < n; k += 64) atomicAdd(&cnt[((src[k] >> 7) & 0xFFu) * 64 + lane], 1u);
            }
        } else {
            const uint8_t *src = static_cast<const uint8_t *>(in) + base;
            if (full_row) {
                uint4 q[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) q[j] = load_nt(reinterpret_cast<const uint4 *>(src) + j * 64 + lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
#pragma unroll
                        for (int b = 0; b < 4; ++b) atomicAdd(&cnt[((w[k] >> (8 * b + 2)) & 0x1Fu) * 64 + lane], 1u);
                }
            } else {
                for (uint64_t k = lane; base + k < n; k += 64) atomicAdd(&cnt[((src[k] >> 2) & 0x1Fu) * 64 + lane], 1u);
            }
        }
    }
    __syncthreads();
    for (uint32_t v = threadIdx.x; v < S; v += kCalThreads) {
        uint32_t sum = 0;
        for (uint32_t c = 0; c < 64; ++c) sum += cnt[v * 64 + ((c + v) & 63u)];   // rotated: no bank conflicts
        partial[(uint64_t)v * groups + blockIdx.x] = sum;
    }
}

template <int DT>
__global__ __launch_bounds__(kSelectThreads) void sz_cal_select(const uint32_t *__restrict__ partial, uint32_t groups,
                                                                uint32_t *__restrict__ cb_out,
                                                                uint64_t *__restrict__ hist_out)
{
    constexpr uint32_t S = DT == SZ_BF16 ? 256 : 32;
    constexpr uint32_t P = kSelectThreads / S;        // threads per symbol, consecutive lanes
    __shared__ uint64_t hist[S];
    const uint32_t t = threadIdx.x;
    const uint32_t v = t / P, part = t % P;
    const uint4 *row = reinterpret_cast<const uint4 *>(partial + (uint64_t)v * groups);
    uint64_t sum = 0;
    // unrolled so that eight loads are in flight at once
#pragma unroll 8
    for (uint32_t i = part; i < groups / 4; i += P) {
        const uint4 q = row[i];
        sum += (uint64_t)q.x + q.y + q.z + q.w;
    }
    for (uint32_t o = 1; o < P; o <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)sum, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(sum >> 32), o, 64);
        sum += ((uint64_t)hi << 32) | lo;
    }
    if (part == 0) hist[v] = sum;
    __syncthreads();
    if (t < S) {
        const uint64_t h = hist[t];
        uint32_t rank = 0;
        for (uint32_t u = 0; u < S; ++u) {
            const uint64_t hu = hist[u];
            rank += (hu > h || (hu == h && u < t)) ? 1u : 0u;
        }
        if (rank < 16) reinterpret_cast<uint8_t *>(cb_out)[4 + rank] = (uint8_t)t;
        if (hist_out) hist_out[t] = h;
    }
    if (t == 0) cb_out[0] = (uint32_t)DT;
}

}  // namespace
}  // namespace sz

using namespace sz;

extern "C" int sz_calibrate(int dtype, const void *host_data, uint64_t n_elems, sz_codebook *out)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    if (!out || (n_elems && !host_data)) return SZ_E_ARG;
    const uint32_t symbols = symbols_of(dtype);
    std::vector<uint64_t> hist(symbols, 0);
    if (dtype == SZ_BF16) {
        const uint16_t *h = static_cast<const uint16_t *>(host_data);
        for (uint64_t i = 0; i < n_elems; ++i) ++hist[(h[i] >> 7) & 0xFFu];
    } else {
        const uint8_t *h = static_cast<const uint8_t *>(host_data);
        for (uint64_t i = 0; i < n_elems; ++i) ++hist[(h[i] >> 2) & 0x1Fu];
    }
    std::vector<uint32_t> order(symbols);
    for (uint32_t v = 0; v < symbols; ++v) order[v] = v;
    std::stable_sort(order.begin(), order.end(),
                     [&](uint32_t x, uint32_t y) { return hist[x] > hist[y]; });
    out->dtype = (uint32_t)dtype;
    for (int c = 0; c < 16; ++c) out->exp[c] = (uint8_t)order[c];
    return SZ_OK;
}

extern "C" uint64_t sz_calibrate_workspace_size(int dtype)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return 0;
    return (uint64_t)symbols_of(dtype) * kCalMaxGroups * 4;
}

extern "C" int sz_calibrate_device(int dtype, const void *d_in, uint64_t n_elems, uint64_t sample_every,
                                   sz_codebook *d_cb, uint64_t *d_hist, void *d_ws, uint64_t ws_bytes,
                                   void *stream)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    if (n_elems > kMaxElems || sample_every == 0) return SZ_E_ARG;
    if (!d_cb || !d_ws || (n_elems && !d_in)) return SZ_E_ARG;
    if (!aligned16(d_cb) || !aligned16(d_ws) || (n_elems && !aligned16(d_in)) || (d_hist && !aligned16(d_hist)))
        return SZ_E_ALIGN;
    if (ws_bytes < sz_calibrate_workspace_size(dtype)) return SZ_E_WORKSPACE;
    const uint64_t nb = (n_elems + kBlock - 1) / kBlock;
    const uint64_t sampled = (nb + sample_every - 1) / sample_every;
    const uint64_t rows = sampled * kCalRowsPerBlock;
    const uint64_t waves = kCalThreads / 64;
    // one row per wave at least, and a multiple of 4 columns for the dwordx4 sums
    uint64_t groups = std::min<uint64_t>(kCalMaxGroups, (rows + waves - 1) / waves);
    groups = std::max<uint64_t>(4, (groups + 3) & ~uint64_t(3));
    uint32_t *partial = static_cast<uint32_t *>(d_ws);
    uint32_t *cb_out = reinterpret_cast<uint32_t *>(d_cb);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == SZ_BF16) {
        {
            LaunchScope scope("sz_cal_hist_bf16", s);
            hipLaunchKernelGGL(sz_cal_hist<SZ_BF16>, dim3((uint32_t)groups), dim3(kCalThreads), 0, s, d_in, n_elems,
                               sample_every, rows, partial, (uint32_t)groups);
        }
        LaunchScope scope("sz_cal_select", s);
        hipLaunchKernelGGL(sz_cal_select<SZ_BF16>, dim3(1), dim3(kSelectThreads), 0, s, partial, (uint32_t)groups,
                           cb_out, d_hist);
    } else {
        {
            LaunchScope scope("sz_cal_hist_e5m2", s);
            hipLaunchKernelGGL(sz_cal_hist<SZ_FP8_E5M2>, dim3((uint32_t)groups), dim3(kCalThreads), 0, s, d_in,
                               n_elems, sample_every, rows, partial, (uint32_t)groups);
        }
        LaunchScope scope("sz_cal_select", s);
        hipLaunchKernelGGL(sz_cal_select<SZ_FP8_E5M2>, dim3(1), dim3(kSelectThreads), 0, s, partial,
                           (uint32_t)groups, cb_out, d_hist);
    }
    return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
}

