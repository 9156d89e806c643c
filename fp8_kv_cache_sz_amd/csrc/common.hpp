// Shared parts of the SplitZip codec for MI355X (gfx950, CDNA4): constants,
// stream geometry, workspace layout, device helpers used by more than one
// kernel family, and the launch instrumentation.  Everything here is inline
// or constexpr, in namespace sz; kernels live in the .hip files that launch
// them (encode.hip, decode.hip, calibrate.hip, runtime.hip).
//
// Method: "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
// Serving" (gist.science summary page), Method section.  Encode splits every
// value into a raw sign+mantissa symbol and an exponent mapped through a
// Top-16 codebook to a 4-bit code; exponents outside the codebook become
// (16-bit position, 8-bit exponent) escape records.  Decode is a dense
// lookup-table pass followed by an overwrite of the escaped exponents.
//
// The work is integer bit manipulation streamed through HBM: there is no
// contraction, so no MFMA.  Design points for CDNA4:
//   * each wave streams one 4096-element row; every global access of the
//     dense passes is a full-wave coalesced 4/8/16-byte access, issued with
//     the non-temporal hint (the data is touched once);
//   * code tables live in LDS (256-entry exponent->code bytes for encode,
//     256-entry code-pair->shifted-exponent words for decode);
//   * byte shuffles use v_perm_b32 / v_alignbyte_b32;
//   * escape ranks come from a packed 64-lane prefix sum of per-chunk counts
//     plus a per-workgroup prefix over the waves.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "splitzip.h"

namespace sz {


constexpr uint64_t kBlock = 65536;          // elements per escape-position block
constexpr uint32_t kMagic = 0x50495A53u;    // "SZIP"
constexpr uint32_t kLog2Block = 16;

// Every dense kernel gives each lane 64 elements of one 4096-element row per
// wave (BF16: eight 8-element chunks, E5M2: two 32-element chunks).
constexpr uint32_t kRow = 4096;
constexpr uint32_t kEncThreads = 256;                     // 4 waves = one 16K tile
constexpr uint32_t kEncTile = kRow * (kEncThreads / 64);  // 16384
constexpr uint32_t kTilesPerBlock = kBlock / kEncTile;    // 4
constexpr uint32_t kDecThreads = 1024;                    // 16 waves = one 64K block
constexpr uint32_t kScanThreads = 1024;
constexpr int kScanBatch = 8;                             // passes of kScanThreads items per scan batch

constexpr uint64_t up256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

struct Geometry {
    uint64_t n, nb, nt;
    uint64_t off_nib, nib_bytes, off_sm, sm_bytes, off_esc;
};

// Section offsets of a stream; version 2 (Top-8) has 3-bit codes, the
// others 4-bit codes.
inline Geometry geometry(int dtype, uint64_t n, uint32_t version = 1)
{
    Geometry g;
    g.n = n;
    g.nb = (n + kBlock - 1) / kBlock;
    g.nt = (n + kEncTile - 1) / kEncTile;
    g.off_nib = up256(64 + 4 * g.nb);
    g.nib_bytes = version == 2 ? 3 * ((n + 7) / 8) : (n + 1) / 2;
    g.off_sm = g.off_nib + up256(g.nib_bytes);
    g.sm_bytes = dtype == SZ_BF16 ? n : 3 * ((n + 7) / 8);
    g.off_esc = g.off_sm + up256(g.sm_bytes);
    return g;
}

// Escape staging.  Tiles with more escapes than kRederiveRecords are not
// staged in streams of more than kFusedPrefixTiles tiles: the compaction
// kernel derives their records again from the input, which moves 2 bytes per
// element instead of writing and re-reading 3 bytes per escape.  Streams of
// up to kFusedPrefixTiles tiles, whose compaction kernels have few waves, and
// the ablation formats stage every tile.  A tile's staging slot holds the
// most records it can stage.
constexpr uint32_t kRederiveRecords = kEncTile / 4;
constexpr uint64_t kFusedPrefixTiles = 2048;

inline uint64_t stage_slot_bytes(uint32_t version, uint64_t nt)
{
    if (version == 3) return kEncTile;                         // one exponent byte per escape
    if (version == 2 || nt <= kFusedPrefixTiles) return 3ull * kEncTile;
    return 3ull * kRederiveRecords;
}

// Blocks whose escape offsets one scan workgroup computes (kScanBatch passes
// of kScanThreads blocks); larger streams take one workgroup per this many
// blocks, after a reduction of their escape totals.
constexpr uint64_t kScanSuper = (uint64_t)kScanBatch * kScanThreads;

// Encode workspace layout (byte offsets): the status word (first 256 bytes),
// tile counts, block offsets, the scan workgroups' escape totals, their
// flagged-tile words and the escape staging (stage_slot_bytes per tile).
struct WsLayout {
    uint64_t counts, offsets, totals, flags, stage, slot, total;
};

inline WsLayout ws_layout(uint32_t version, int dtype, uint64_t n)
{
    Geometry g = geometry(dtype, n, version);
    WsLayout w;
    w.counts = 256;
    w.offsets = w.counts + up256(4 * g.nt + 16);
    w.totals = w.offsets + up256(8 * g.nb + 16);
    const uint64_t scan_groups = (g.nb + kScanSuper - 1) / kScanSuper;
    w.flags = w.totals + up256(8 * scan_groups);
    w.stage = w.flags + up256(4 * (kScanThreads / 64) * scan_groups);   // one word per scan wave
    w.slot = stage_slot_bytes(version, g.nt);
    // 16 bytes past the last slot: the record copies read whole words
    w.total = w.stage + up256(w.slot * g.nt + 16);
    return w;
}

// Decode workspace layout: status words, then the block offsets.
constexpr uint64_t kDecOffsets = 256;
inline uint64_t decode_ws_bytes(int dtype, uint64_t n)
{
    return kDecOffsets + up256(8 * geometry(dtype, n).nb + 16);
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt(const uint4 *p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt(const uint2 *p)
{
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_nt(const uint32_t *p) { return __builtin_nontemporal_load(p); }
// three consecutive words (4-byte aligned): one dwordx3 access per lane, so a
// wave's 12-byte groups make one contiguous 768-byte access
typedef uint32_t v3u_a4 __attribute__((ext_vector_type(3), aligned(4)));
__device__ __forceinline__ void load3_nt(const uint32_t *p, uint32_t w[3])
{
    const v3u_a4 v = __builtin_nontemporal_load(reinterpret_cast<const v3u_a4 *>(p));
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
}
__device__ __forceinline__ void store3_nt(uint32_t *p, const uint32_t w[3])
{
    const v3u_a4 v = {w[0], w[1], w[2]};
    __builtin_nontemporal_store(v, reinterpret_cast<v3u_a4 *>(p));
}
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v)
{
    v4u w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4u *>(p));
}
__device__ __forceinline__ void store_nt(uint2 *p, uint2 v)
{
    v2u w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<v2u *>(p));
}
__device__ __forceinline__ void store_nt(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    // v_perm_b32: byte i of the result = byte sel[i] of {hi, lo} (lo = bytes 0..3)
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: four row_shr
// steps scan each 16-lane row, then row_bcast:15 and row_bcast:31 carry the
// row totals forward (lanes of disabled rows add the 0 `old` operand).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x)
{
    uint32_t v = x;
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
        v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

__device__ __forceinline__ uint32_t read_lane63(uint32_t x) { return __builtin_amdgcn_readlane(x, 63); }


// Codebook packed as 4 little-endian words: byte c = exponent of code c.
struct Codebook4 {
    uint32_t w[4];
};

__device__ __forceinline__ uint32_t cb_entry(const Codebook4 &cb, uint32_t c)
{
    return (cb.w[c >> 2] >> (8 * (c & 3))) & 0xFFu;
}

// Entry c (0..15) where c differs between lanes: two byte selects of the
// codebook words, so that the compiler does not index the struct (which
// would place a copy of it in per-thread memory).
__device__ __forceinline__ uint32_t cb_entry_lane(const Codebook4 &cb, uint32_t c)
{
    const uint32_t sel = (c & 7u) | 0x0C0C0C00u;          // byte c & 7, three zero bytes
    const uint32_t lo = perm(cb.w[1], cb.w[0], sel);
    const uint32_t hi = perm(cb.w[3], cb.w[2], sel);
    return c < 8 ? lo : hi;
}

// A codebook that lives in device memory as an sz_codebook (word 0 = dtype,
// words 1..4 = the 16 exponent bytes), as sz_calibrate_device writes it.
__device__ __forceinline__ Codebook4 load_codebook(const uint32_t *cb_dev)
{
    Codebook4 cb;
#pragma unroll
    for (int w = 0; w < 4; ++w) cb.w[w] = cb_dev[1 + w];
    return cb;
}

// Per-chunk rank data of a wave row (J chunks per lane): row_base[j] = escapes
// of the wave before chunk row j, row_total[j] = escapes in chunk row j (both
// wave-uniform), lane_before[j] = escapes of lanes below this one in row j.
// Returns the wave's escape total.
template <int J>
__device__ __forceinline__ uint32_t wave_chunk_ranks(const uint32_t (&cnt)[J], uint32_t (&row_base)[J],
                                                     uint32_t (&row_total)[J], uint32_t (&lane_before)[J])
{
    static_assert(J % 2 == 0, "chunk counts are scanned in pairs");
    uint32_t running = 0;
#pragma unroll
    for (int p = 0; p < J / 2; ++p) {
        const uint32_t packed = cnt[2 * p] | (cnt[2 * p + 1] << 16);
        const uint32_t incl = wave_inclusive_sum(packed);
        const uint32_t excl = incl - packed;
        const uint32_t tot = read_lane63(incl);
        row_base[2 * p] = running;
        row_total[2 * p] = tot & 0xFFFFu;
        lane_before[2 * p] = excl & 0xFFFFu;
        running += tot & 0xFFFFu;
        row_base[2 * p + 1] = running;
        row_total[2 * p + 1] = tot >> 16;
        lane_before[2 * p + 1] = excl >> 16;
        running += tot >> 16;
    }
    return running;
}

// Sums the per-wave escape totals of a workgroup through LDS.  Returns the
// escapes of the waves before this one; `total` gets the workgroup's.
template <int WAVES>
__device__ __forceinline__ uint32_t workgroup_wave_prefix(uint32_t wave_total, uint32_t *lds,
                                                          uint32_t &total)
{
    const uint32_t wave = threadIdx.x / 64;
    if (lane_id() == 0) lds[wave] = wave_total;
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const uint32_t v = lds[w];
        if ((uint32_t)w < wave) before += v;
        sum += v;
    }
    total = sum;
    return before;
}

// Chunks of 8 (BF16) or 32 (E5M2) elements per lane in a 4096-element wave row.
constexpr int kBf16Chunks = 8;
constexpr int kE5Chunks = 2;

// Format versions: 1 = Top-16 (the page's design), 2 = Top-8 (3-bit codes,
// position records), 3 = Top-15 with code 15 as escape sentinel (one
// exponent byte per escape, no positions).  2 and 3 are the ablation
// alternatives of the page (Method, decoding design-choice bullet; Results,
// ablations) and exist for BF16 only.
constexpr uint32_t kTop16 = 1, kTop8 = 2, kTop15S = 3;
__host__ __device__ constexpr uint32_t book_entries(uint32_t v) { return v == kTop8 ? 8 : v == kTop15S ? 15 : 16; }
__host__ __device__ constexpr uint32_t escape_item_bytes(uint32_t v) { return v == kTop15S ? 1 : 3; }

// ---------------------------------------------------------------------------
// One-workgroup scans.  Both scan kernels read their counts with coalesced
// dwordx4 loads: in pass i, thread t holds item i * 1024 + t, where an item
// is four consecutive counts (four tiles = one block for encode, four blocks
// for decode).  Up to kScanBatch passes are loaded at once; each pass gets
// its own 64-lane prefix sums, the 16 waves' totals meet in LDS, and one
// thread per pass turns them into exclusive offsets.  A running 64-bit carry
// joins successive batches.
// ---------------------------------------------------------------------------
constexpr uint32_t kScanWaves = kScanThreads / 64;

struct ScanLds {
    uint32_t wave_incl[kScanBatch][kScanWaves];   // per pass: inclusive wave totals -> exclusive prefixes
    uint32_t pass_total[kScanBatch];
    uint64_t pass_base[kScanBatch];                // per pass: offset of its first item
    uint64_t carry;
};

// x[i] = item value of pass i for this thread (0 for missing items); on
// return base[i] = exclusive prefix of this thread's item in pass i.
// lds.carry holds the running total before the batch and is advanced.
__device__ __forceinline__ void scan_batch(const uint32_t (&x)[kScanBatch], uint64_t (&base)[kScanBatch],
                                           ScanLds &lds)
{
    static_assert(kScanBatch * kScanWaves <= kScanThreads && kScanWaves == 16, "one lane per (pass, wave)");
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = tid / 64;
    uint32_t incl[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) {
        incl[i] = wave_inclusive_sum(x[i]);
        if (lane == 63) lds.wave_incl[i][wave] = incl[i];
    }
    __syncthreads();
    // lane (pass i, wave w) for tid < 128: exclusive scan of the 16 wave
    // totals of pass i inside a 16-lane segment
    if (tid < kScanBatch * kScanWaves) {
        const uint32_t i = tid / kScanWaves, w = tid % kScanWaves;
        const uint32_t v0 = lds.wave_incl[i][w];
        uint32_t v = v0;
#pragma unroll
        for (int d = 1; d < (int)kScanWaves; d <<= 1) {
            const uint32_t y = __shfl_up(v, d, kScanWaves);
            if (w >= (uint32_t)d) v += y;
        }
        lds.wave_incl[i][w] = v - v0;
        if (w == kScanWaves - 1) lds.pass_total[i] = v;
    }
    __syncthreads();
    if (tid < kScanBatch) {
        uint64_t b = lds.carry;
        for (uint32_t i = 0; i < tid; ++i) b += lds.pass_total[i];
        lds.pass_base[tid] = b;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) base[i] = lds.pass_base[i] + lds.wave_incl[i][wave] + (incl[i] - x[i]);
    if (tid == 0) lds.carry = lds.pass_base[kScanBatch - 1] + lds.pass_total[kScanBatch - 1];
    __syncthreads();    // the next batch reuses the LDS
}

// ---------------------------------------------------------------------------
// Host side: launch bookkeeping and instrumentation
// ---------------------------------------------------------------------------
struct ProfRecord {
    const char *name;
    hipEvent_t start, stop;
};

// Instrumentation state (defined with sz_profile_enable / sz_profile_collect).
// g_prof_on is read without the lock on every launch, so launches never
// serialise on the mutex while instrumentation is off (its default); the
// mutex guards the event pool and the records, which exist only while it is
// on.
extern std::mutex g_prof_mutex;
extern std::atomic<bool> g_prof_on;
extern std::vector<ProfRecord> g_prof_records;
extern std::vector<hipEvent_t> g_event_pool;
hipEvent_t take_event();
void release_records();

struct LaunchScope {
    const char *name;
    hipStream_t stream;
    hipEvent_t start = nullptr, stop = nullptr;
    LaunchScope(const char *n, hipStream_t s) : name(n), stream(s)
    {
        if (!g_prof_on.load(std::memory_order_acquire)) return;
        std::lock_guard<std::mutex> lock(g_prof_mutex);
        if (!g_prof_on.load(std::memory_order_relaxed)) return;
        start = take_event();
        stop = take_event();
        if (start && stop) (void)hipEventRecord(start, stream);
    }
    ~LaunchScope()
    {
        if (!start || !stop) return;
        (void)hipEventRecord(stop, stream);
        std::lock_guard<std::mutex> lock(g_prof_mutex);
        g_prof_records.push_back({name, start, stop});
    }
};

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline Codebook4 pack_codebook(const uint8_t *e)
{
    Codebook4 cb;
    for (int w = 0; w < 4; ++w)
        cb.w[w] = (uint32_t)e[4 * w] | ((uint32_t)e[4 * w + 1] << 8) | ((uint32_t)e[4 * w + 2] << 16) |
                  ((uint32_t)e[4 * w + 3] << 24);
    return cb;
}

inline uint32_t symbols_of(int dtype) { return dtype == SZ_BF16 ? 256u : 32u; }

constexpr uint64_t kMaxElems = 1ull << 40;

inline uint64_t encoded_size_v(uint32_t version, int dtype, uint64_t n, uint64_t e)
{
    return geometry(dtype, n, version).off_esc + escape_item_bytes(version) * e;
}

}  // namespace sz
