// SplitZip codec for MI355X (gfx950, CDNA4): HIP kernels and the C ABI.
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
//     plus a per-workgroup prefix over the waves;
//   * encode = dense+stage (one 256-lane workgroup per 16K-element tile), a
//     one-workgroup scan of the tile counts, then a compaction of the staged
//     escape records into their final order (escape-heavy tiles are encoded
//     again from the input there instead of being staged);
//   * decode = a one-workgroup validating scan of the block counts, then one
//     1024-lane workgroup per 64K block: dense decode in registers, patched
//     from an LDS map of the block's escapes before a single store (blocks
//     with very many escapes go through an LDS exponent plane);
//   * also here: on-device calibration (exponent histogram + Top-16
//     selection) and the two ablation formats the page weighs against its
//     Top-16 design (Top-8 and Top-15 with a sentinel code, BF16 only).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "splitzip.h"

namespace {

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
constexpr uint32_t kCompactThreads = 256;                 // one wave per block

constexpr uint64_t up256(uint64_t x) { return (x + 255u) & ~uint64_t(255); }

struct Geometry {
    uint64_t n, nb, nt;
    uint64_t off_nib, nib_bytes, off_sm, sm_bytes, off_esc;
};

// Section offsets of a stream; version 2 (Top-8) has 3-bit codes, the
// others 4-bit codes.
Geometry geometry(int dtype, uint64_t n, uint32_t version = 1)
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

// Workspace layout (byte offsets): status word, tile counts, tile offsets
// (encode) / block offsets (decode), escape staging (encode).
struct WsLayout {
    uint64_t counts, offsets, stage, total;
};

WsLayout ws_layout(int dtype, uint64_t n)
{
    Geometry g = geometry(dtype, n);
    WsLayout w;
    w.counts = 256;
    w.offsets = w.counts + up256(4 * g.nt + 16);
    const uint64_t offsets_bytes = std::max<uint64_t>(8 * g.nt, 8 * g.nb);
    w.stage = w.offsets + up256(offsets_bytes + 16);
    w.total = w.stage + up256(3 * g.nt * kEncTile + 16);
    return w;
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

// A codebook that lives in device memory as an sz_codebook (word 0 = dtype,
// words 1..4 = the 16 exponent bytes), as sz_calibrate_device writes it.
__device__ __forceinline__ Codebook4 load_codebook(const uint32_t *cb_dev)
{
    Codebook4 cb;
#pragma unroll
    for (int w = 0; w < 4; ++w) cb.w[w] = cb_dev[1 + w];
    return cb;
}

// Exponent -> code table for encode.  Byte v = code of exponent v, or
// `escape` (the escape flag 0x80 plus the code an escaped element carries)
// when v is not among the first `entries` codebook entries.  Threads 0..63
// fill 4 entries each.
__device__ __forceinline__ void build_encode_table(uint32_t *table32, const Codebook4 &cb,
                                                   uint32_t symbols, uint32_t entries = 16,
                                                   uint32_t escape = 0x80u)
{
    const uint32_t t = threadIdx.x;
    if (t < 64 && t * 4 < symbols) {
        uint32_t word = 0;
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            const uint32_t v = t * 4 + k;
            uint32_t code = escape;
#pragma unroll
            for (uint32_t c = 0; c < 16; ++c)
                if (c < entries && cb_entry(cb, c) == v) code = c;
            word |= code << (8 * k);
        }
        table32[t] = word;
    }
}

// Looks up four exponent bytes in the encode table.
__device__ __forceinline__ uint32_t lookup4(const uint8_t *table, uint32_t e4)
{
    return (uint32_t)table[e4 & 0xFFu] | ((uint32_t)table[(e4 >> 8) & 0xFFu] << 8) |
           ((uint32_t)table[(e4 >> 16) & 0xFFu] << 16) | ((uint32_t)table[e4 >> 24] << 24);
}

// Code bytes of 8 elements (two words of table output) -> one word of nibbles
// (element 2k in the low nibble).  Byte 0 of (k | k >> 4) = code0 | code1 << 4.
__device__ __forceinline__ uint32_t pack_codes8(uint32_t c_a, uint32_t c_b)
{
    const uint32_t k_a = c_a & 0x0F0F0F0Fu;
    const uint32_t k_b = c_b & 0x0F0F0F0Fu;
    return perm(k_b | (k_b >> 4), k_a | (k_a >> 4), 0x06040200u);
}

// Escape flags of 8 elements (bit 7 of each table byte) -> bit k = element k.
// (x >> 7) holds the four flags at bits 0, 8, 16, 24; the multiply moves flag
// k to bit 28 + k without carries.
__device__ __forceinline__ uint32_t escape_mask8(uint32_t c_a, uint32_t c_b)
{
    const uint32_t lo = (((c_a & 0x80808080u) >> 7) * 0x10204080u) >> 28;
    const uint32_t hi = (((c_b & 0x80808080u) >> 7) * 0x10204080u) >> 28;
    return lo | (hi << 4);
}

// ---------------------------------------------------------------------------
// BF16 encode of one 8-element chunk (16 bytes in).
//   nib: 4 bytes of codes;  sm: 8 sign/mantissa bytes (sign << 7 | mantissa7)
//   esc: escape mask (bit k = element k);  ex: exponent of element k in byte k
// ---------------------------------------------------------------------------
// Version 2 (Top-8) packing: 3-bit codes of 8 elements (table bytes c_a =
// elements 0..3, c_b = 4..7) -> 24 bits, element k at bit 3k.
__device__ __forceinline__ uint32_t pack_codes8_top8(uint32_t c_a, uint32_t c_b)
{
    const uint32_t t_a = c_a & 0x07070707u, t_b = c_b & 0x07070707u;
    const uint32_t u_a = (t_a & 7u) | ((t_a >> 5) & 0x38u) | ((t_a >> 10) & 0x1C0u) | ((t_a >> 15) & 0xE00u);
    const uint32_t u_b = (t_b & 7u) | ((t_b >> 5) & 0x38u) | ((t_b >> 10) & 0x1C0u) | ((t_b >> 15) & 0xE00u);
    return u_a | (u_b << 12);
}

template <int V = 1>
__device__ __forceinline__ void encode_chunk_bf16(const uint4 q, const uint8_t *table, uint32_t &nib,
                                                  uint2 &sm, uint32_t &esc, uint64_t &ex)
{
    const uint32_t lo_a = perm(q.y, q.x, 0x06040200u);   // low bytes of elements 0..3
    const uint32_t hi_a = perm(q.y, q.x, 0x07050301u);   // high bytes of elements 0..3
    const uint32_t lo_b = perm(q.w, q.z, 0x06040200u);
    const uint32_t hi_b = perm(q.w, q.z, 0x07050301u);
    sm.x = (hi_a & 0x80808080u) | (lo_a & 0x7F7F7F7Fu);
    sm.y = (hi_b & 0x80808080u) | (lo_b & 0x7F7F7F7Fu);
    const uint32_t e_a = ((hi_a << 1) & 0xFEFEFEFEu) | ((lo_a >> 7) & 0x01010101u);
    const uint32_t e_b = ((hi_b << 1) & 0xFEFEFEFEu) | ((lo_b >> 7) & 0x01010101u);
    const uint32_t c_a = lookup4(table, e_a);
    const uint32_t c_b = lookup4(table, e_b);
    nib = V == 2 ? pack_codes8_top8(c_a, c_b) : pack_codes8(c_a, c_b);
    esc = escape_mask8(c_a, c_b);
    ex = (uint64_t)e_a | ((uint64_t)e_b << 32);
}

// ---------------------------------------------------------------------------
// FP8 E5M2 encode of one 32-element chunk (32 bytes in): 16 code bytes and
// 12 sign/mantissa bytes (four 24-bit groups of eight 3-bit symbols).
//   esc: escape mask (bit k = element k of the 32);  ex[s]: exponents of
//   elements 8s..8s+7.
// ---------------------------------------------------------------------------
// Four 3-bit symbols held in bytes (bits 0-2 of each byte, the rest zero) ->
// 12 contiguous bits.
__device__ __forceinline__ uint32_t pack_sym3x4(uint32_t sym)
{
    const uint32_t u = sym | (sym >> 5);              // f0 | f1 << 3 at bit 0, f2 | f3 << 3 at bit 16
    return (u & 0x3Fu) | ((u >> 10) & 0xFC0u);
}

__device__ __forceinline__ void encode_chunk_e5m2(const uint4 q0, const uint4 q1, const uint8_t *table,
                                                  uint4 &nib, uint32_t sm3[3], uint32_t &esc, uint64_t ex[4])
{
    const uint32_t d[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    uint32_t nibw[4], grp[4];
    esc = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t a = d[2 * s], b = d[2 * s + 1];
        const uint32_t e_a = (a >> 2) & 0x1F1F1F1Fu;
        const uint32_t e_b = (b >> 2) & 0x1F1F1F1Fu;
        const uint32_t s_a = ((a >> 5) & 0x04040404u) | (a & 0x03030303u);
        const uint32_t s_b = ((b >> 5) & 0x04040404u) | (b & 0x03030303u);
        const uint32_t c_a = lookup4(table, e_a);
        const uint32_t c_b = lookup4(table, e_b);
        nibw[s] = pack_codes8(c_a, c_b);
        esc |= escape_mask8(c_a, c_b) << (8 * s);
        ex[s] = (uint64_t)e_a | ((uint64_t)e_b << 32);
        grp[s] = pack_sym3x4(s_a) | (pack_sym3x4(s_b) << 12);
    }
    nib = make_uint4(nibw[0], nibw[1], nibw[2], nibw[3]);
    sm3[0] = grp[0] | (grp[1] << 24);
    sm3[1] = (grp[1] >> 8) | (grp[2] << 16);
    sm3[2] = (grp[2] >> 16) | (grp[3] << 8);
}

// E5M2 encode through a code-pair table: table16[e0 | e1 << 5] holds, for
// two neighbouring elements with exponents e0 and e1, their two codes as one
// code byte (low byte: code0 | code1 << 4, escapes coded 0) and their escape
// flags (high byte: bit 0 = element 0, bit 1 = element 1).  One LDS read per
// two elements replaces two reads, the nibble packing and the escape-mask
// arithmetic of the byte table.
__device__ __forceinline__ void build_pair_table(uint32_t *table16x2, const uint8_t *tab8)
{
    // thread t fills entries 4t .. 4t+3 (two words); e1 is the same for all four
    const uint32_t t = threadIdx.x;
    if (t < 256) {
        const uint32_t c1 = tab8[t >> 3];
        const uint32_t hi = ((c1 & 0xFu) << 4) | ((c1 >> 7) << 9);
        uint32_t e[4];
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            const uint32_t c0 = tab8[(4 * t + k) & 31u];
            e[k] = (c0 & 0xFu) | ((c0 >> 7) << 8) | hi;
        }
        table16x2[2 * t] = e[0] | (e[1] << 16);
        table16x2[2 * t + 1] = e[2] | (e[3] << 16);
    }
}

// One 32-element chunk: 16 code bytes, 12 sign/mantissa bytes, and per group
// of 8 elements a flag word fl[s] whose byte k holds the escape flags of
// elements 2k (bit 0) and 2k + 1 (bit 1) of the group.
__device__ __forceinline__ void encode_chunk_e5m2_pairs(const uint4 q0, const uint4 q1, const uint16_t *table16,
                                                        uint4 &nib, uint32_t sm3[3], uint32_t fl[4])
{
    const uint32_t d[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    uint32_t nibw[4], grp[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t a = d[2 * s], b = d[2 * s + 1];
        // pair index e0 | e1 << 5 of elements (0,1) and (2,3) of a word
        const uint32_t p0 = table16[((a >> 2) & 0x1Fu) | ((a >> 5) & 0x3E0u)];
        const uint32_t p1 = table16[((a >> 18) & 0x1Fu) | ((a >> 21) & 0x3E0u)];
        const uint32_t p2 = table16[((b >> 2) & 0x1Fu) | ((b >> 5) & 0x3E0u)];
        const uint32_t p3 = table16[((b >> 18) & 0x1Fu) | ((b >> 21) & 0x3E0u)];
        const uint32_t lo = perm(p1, p0, 0x0C0C0400u), hi = perm(p3, p2, 0x04000C0Cu);
        nibw[s] = lo | hi;
        fl[s] = perm(p1, p0, 0x0C0C0501u) | perm(p3, p2, 0x05010C0Cu);
        const uint32_t s_a = ((a >> 5) & 0x04040404u) | (a & 0x03030303u);
        const uint32_t s_b = ((b >> 5) & 0x04040404u) | (b & 0x03030303u);
        grp[s] = pack_sym3x4(s_a) | (pack_sym3x4(s_b) << 12);
    }
    nib = make_uint4(nibw[0], nibw[1], nibw[2], nibw[3]);
    sm3[0] = grp[0] | (grp[1] << 24);
    sm3[1] = (grp[1] >> 8) | (grp[2] << 16);
    sm3[2] = (grp[2] >> 16) | (grp[3] << 8);
}

// Flag word of a group (byte k = flags of elements 2k, 2k+1) -> 8-bit mask.
__device__ __forceinline__ uint32_t flags_to_mask8(uint32_t f)
{
    return (f & 3u) | ((f >> 6) & 0xCu) | ((f >> 12) & 0x30u) | ((f >> 18) & 0xC0u);
}

// Flag bits of the first v elements of a group (v in 0..8).
__device__ __forceinline__ uint32_t group_flag_keep(int v)
{
    uint32_t m = 0;
    for (int i = 0; i < 8; ++i)
        if (i < v) m |= 1u << ((i / 2) * 8 + (i & 1));
    return m;
}

// ---------------------------------------------------------------------------
// Escape staging.  Inside a wave the records of a tile come in element order:
// (chunk j, lane, element).  A "segment" is 512 consecutive elements of a
// row (BF16: chunk j of all 64 lanes; E5M2: chunk j of 16 lanes), so it holds
// at most 512 records.  Each lane writes its records of the segment into the
// wave's LDS buffer, shifted by the byte misalignment of the segment's
// destination, and the wave then copies the buffer to the tile's staging
// slot with aligned dword stores; the dwords at both ends, which neighbouring
// segments (possibly of another wave) share, are written byte by byte.
// ---------------------------------------------------------------------------
constexpr uint32_t kSegElems = 512;
constexpr uint32_t kSegBytes = 3 * kSegElems + 8;          // + alignment shift, rounded to dwords

// Appends the records of 8 elements (escape mask esc, exponents ex,
// block-local position of the first element pos0) to an LDS buffer at byte
// `off`; returns the byte after them.
__device__ __forceinline__ uint32_t lds_put_records(uint8_t *buf, uint32_t off, uint32_t esc, uint64_t ex,
                                                    uint32_t pos0)
{
    while (esc) {
        const uint32_t k = (uint32_t)__builtin_ctz(esc);
        esc &= esc - 1;
        const uint32_t pos = (pos0 + k) & 0xFFFFu;
        buf[off] = (uint8_t)pos;
        buf[off + 1] = (uint8_t)(pos >> 8);
        buf[off + 2] = (uint8_t)(ex >> (8 * k));
        off += 3;
    }
    return off;
}

__device__ __forceinline__ void wave_lds_fence()
{
    // LDS operations of one wave complete in order; this only keeps the
    // compiler from moving LDS accesses across the hand-over point
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copies `len` bytes, held in buf[g0 & 3, (g0 & 3) + len), to dst[g0, g0 + len).
__device__ __forceinline__ void flush_segment(const uint8_t *buf, uint8_t *dst, uint32_t g0, uint32_t len)
{
    const uint32_t lane = lane_id();
    const uint32_t first_dw = g0 >> 2;
    const uint32_t end = g0 + len;
    const uint32_t last_dw = (end - 1) >> 2;
    const uint32_t head = g0 & 3;
    const uint32_t tail = ((end - 1) & 3) + 1;
    for (uint32_t i = lane; i <= last_dw - first_dw; i += 64) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(buf)[i];
        const uint32_t lo = (i == 0) ? head : 0;
        const uint32_t hi = (first_dw + i == last_dw) ? tail : 4;
        uint8_t *d = dst + 4ull * (first_dw + i);
        if (lo == 0 && hi == 4) {
            *reinterpret_cast<uint32_t *>(d) = w;
        } else {
            for (uint32_t b = lo; b < hi; ++b) d[b] = (uint8_t)(w >> (8 * b));
        }
    }
}

// Writes the escape records of 8 elements (escape mask esc, exponents ex,
// first block-local position pos0) straight into the staging area,
// ascending, from rank `rank` on.  Used for rows with few escapes.
__device__ __forceinline__ void put_records(uint8_t *tstage, uint32_t rank, uint32_t esc, uint64_t ex,
                                            uint32_t pos0)
{
    while (esc) {
        const uint32_t k = (uint32_t)__builtin_ctz(esc);
        esc &= esc - 1;
        const uint32_t pos = (pos0 + k) & 0xFFFFu;
        uint8_t *r = tstage + 3ull * rank;
        r[0] = (uint8_t)pos;
        r[1] = (uint8_t)(pos >> 8);
        r[2] = (uint8_t)(ex >> (8 * k));
        ++rank;
    }
}

// Rows with more escapes than this go through the LDS segment buffer.
constexpr uint32_t kDirectRecords = 32;
// Tiles with more escapes than this are not staged: the compaction kernel
// derives their records again from the input, which moves 2 bytes per
// element instead of writing and re-reading 3 bytes per escape.  Their tile
// count carries kRederiveFlag.
constexpr uint32_t kRederiveRecords = kEncTile / 4;
constexpr uint32_t kRederiveFlag = 0x80000000u;

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

// ---------------------------------------------------------------------------
// Kernel: BF16 dense encode + escape staging.  One 256-lane workgroup per
// 16K-element tile; wave w streams elements [4096w, 4096w + 4096) of it.  The
// tile's records are staged in element order in the tile's slot (3 bytes per
// element); tile_counts[tile] gets their number.  A tile with more than
// kRederiveRecords escapes stages nothing and is flagged with kRederiveFlag:
// the compaction kernel derives its records again from the input, which
// costs less traffic than writing and re-reading them.
// ---------------------------------------------------------------------------
constexpr int kBf16Chunks = 8;

// Format versions: 1 = Top-16 (the page's design), 2 = Top-8 (3-bit codes,
// position records), 3 = Top-15 with code 15 as escape sentinel (one
// exponent byte per escape, no positions).  2 and 3 are the ablation
// alternatives of the page (Method, decoding design-choice bullet; Results,
// ablations) and exist for BF16 only.
constexpr uint32_t kTop16 = 1, kTop8 = 2, kTop15S = 3;
__host__ __device__ constexpr uint32_t book_entries(uint32_t v) { return v == kTop8 ? 8 : v == kTop15S ? 15 : 16; }
__host__ __device__ constexpr uint32_t escape_item_bytes(uint32_t v) { return v == kTop15S ? 1 : 3; }

// Version 3 staging: the exponent bytes of the escaped elements of 8
// elements, into an LDS buffer at `off` (returns the byte after them) or
// straight into the staging slot at item `rank`.
__device__ __forceinline__ uint32_t lds_put_exponents(uint8_t *buf, uint32_t off, uint32_t esc, uint64_t ex)
{
    while (esc) {
        const uint32_t k = (uint32_t)__builtin_ctz(esc);
        esc &= esc - 1;
        buf[off++] = (uint8_t)(ex >> (8 * k));
    }
    return off;
}

__device__ __forceinline__ void put_exponents(uint8_t *tstage, uint32_t rank, uint32_t esc, uint64_t ex)
{
    while (esc) {
        const uint32_t k = (uint32_t)__builtin_ctz(esc);
        esc &= esc - 1;
        tstage[rank++] = (uint8_t)(ex >> (8 * k));
    }
}

template <int V>
__global__ __launch_bounds__(kEncThreads) void sz_enc_dense_bf16(const uint16_t *__restrict__ in, uint64_t n,
                                                              uint8_t *__restrict__ out, uint64_t off_nib,
                                                              uint64_t off_sm, Codebook4 cb,
                                                              const uint32_t *__restrict__ cb_dev,
                                                              uint32_t *__restrict__ tile_counts,
                                                              uint8_t *__restrict__ stage)
{
    __shared__ uint32_t table32[64];
    __shared__ uint32_t wave_totals[kEncThreads / 64];
    __shared__ __align__(16) uint8_t seg_buf[kEncThreads / 64][kSegBytes];
    // exponents of chunks that hold escapes, parked until the ranks are known
    __shared__ uint64_t ex_park[kEncThreads / 64][kBf16Chunks][64];
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / 64;
    const uint64_t tile = blockIdx.x;
    const uint64_t base = tile * kEncTile + (uint64_t)wave * kRow;
    const bool full_row = base + kRow <= n;

    // the row's loads are issued first and stay in flight while the table is built
    uint4 q[kBf16Chunks];
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 8;
        if (full_row || c0 + 8 <= n) {
            q[j] = load_nt(reinterpret_cast<const uint4 *>(in + c0));
        } else {
            uint16_t v[8];
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) v[k] = (c0 + k < n) ? in[c0 + k] : 0;
            q[j] = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                              v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
        }
    }
    if (cb_dev) cb = load_codebook(cb_dev);
    build_encode_table(table32, cb, 256, book_entries(V), V == kTop15S ? 0x8Fu : 0x80u);
    __syncthreads();
    const uint8_t *table = reinterpret_cast<const uint8_t *>(table32);
    uint8_t *buf = seg_buf[wave];
    uint32_t esc[kBf16Chunks];
    uint32_t cnt[kBf16Chunks];
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 8;
        uint32_t nib;
        uint2 sm;
        uint64_t ex;
        encode_chunk_bf16<V>(q[j], table, nib, sm, esc[j], ex);
        if (esc[j]) ex_park[wave][j][lane] = ex;
        if (full_row || c0 + 8 <= n) {
            if (V != kTop8) store_nt(reinterpret_cast<uint32_t *>(out + off_nib + c0 / 2), nib);
            store_nt(reinterpret_cast<uint2 *>(out + off_sm + c0), sm);
        } else if (c0 < n) {
            // last, partial chunk: missing elements get code 0, sign/mantissa 0
            // and no escape; the bytes past the data are section padding
            const uint32_t valid = (uint32_t)(n - c0);
            const uint64_t keep = (1ull << (8 * valid)) - 1;
            esc[j] &= (1u << valid) - 1;
            nib &= (uint32_t)((1ull << ((V == kTop8 ? 3 : 4) * valid)) - 1);
            const uint64_t smv = ((uint64_t)sm.y << 32 | sm.x) & keep;
            if (V != kTop8) *reinterpret_cast<uint32_t *>(out + off_nib + c0 / 2) = nib;
            *reinterpret_cast<uint2 *>(out + off_sm + c0) = make_uint2((uint32_t)smv, (uint32_t)(smv >> 32));
        } else {
            esc[j] = 0;
            nib = 0;
        }
        if (V == kTop8) {
            // 3 code bytes per chunk: the wave's row of codes (1536 bytes) is
            // assembled in LDS and stored as whole dwords below
            const uint32_t o = j * 192 + 3 * lane;
            buf[o] = (uint8_t)nib;
            buf[o + 1] = (uint8_t)(nib >> 8);
            buf[o + 2] = (uint8_t)(nib >> 16);
        }
        cnt[j] = __popc(esc[j]);
    }
    if (V == kTop8) {
        // the row's code bytes start at 3 * base / 8, a multiple of 1536;
        // dwords past the section's last byte hold only padding and are skipped
        wave_lds_fence();
        const uint64_t row0 = 3 * (base / 8);
        const uint64_t code_bytes = 3 * ((n + 7) / 8);
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const uint32_t d = i * 64 + lane;
            if (row0 + 4 * d < code_bytes)
                *reinterpret_cast<uint32_t *>(out + off_nib + row0 + 4 * d) = reinterpret_cast<const uint32_t *>(buf)[d];
        }
        wave_lds_fence();
    }
    uint32_t row_base[kBf16Chunks], row_total[kBf16Chunks], lane_before[kBf16Chunks];
    const uint32_t wave_total = wave_chunk_ranks<kBf16Chunks>(cnt, row_base, row_total, lane_before);
    uint32_t tile_total;
    const uint32_t wave_before = workgroup_wave_prefix<kEncThreads / 64>(wave_total, wave_totals, tile_total);
    // only the Top-16 format re-derives escape-heavy tiles in the compaction
    const bool rederive = V == kTop16 && tile_total > kRederiveRecords;
    if (wave_total && !rederive) {
        uint8_t *tstage = stage + tile * (3ull * kEncTile);
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t pos0 = (uint32_t)((base + (uint64_t)(j * 64 + lane) * 8) & 0xFFFFu);
            const uint32_t rank = wave_before + row_base[j];
            constexpr uint32_t item = escape_item_bytes(V);
            if (row_total[j] <= kDirectRecords) {                      // wave-uniform
                if (esc[j]) {
                    if (V == kTop15S) put_exponents(tstage, rank + lane_before[j], esc[j], ex_park[wave][j][lane]);
                    else put_records(tstage, rank + lane_before[j], esc[j], ex_park[wave][j][lane], pos0);
                }
            } else {
                const uint32_t g0 = item * rank;
                if (esc[j]) {
                    if (V == kTop15S)
                        lds_put_exponents(buf, (g0 & 3) + lane_before[j], esc[j], ex_park[wave][j][lane]);
                    else
                        lds_put_records(buf, (g0 & 3) + 3 * lane_before[j], esc[j], ex_park[wave][j][lane], pos0);
                }
                wave_lds_fence();
                flush_segment(buf, tstage, g0, item * row_total[j]);
                wave_lds_fence();
            }
        }
    }
    if (threadIdx.x == 0) tile_counts[tile] = tile_total | (rederive ? kRederiveFlag : 0u);
}

// ---------------------------------------------------------------------------
// Kernel: FP8 E5M2 dense encode + escape staging (the page's FP8 extension,
// Contributions item 4).  Same tiling as BF16; a lane holds two 32-element
// chunks of its wave's row.  A chunk row with many escapes is staged through
// LDS as four segments of 16 lanes.
// ---------------------------------------------------------------------------
constexpr int kE5Chunks = 2;

__global__ __launch_bounds__(kEncThreads) void sz_enc_dense_e5m2(const uint8_t *__restrict__ in, uint64_t n,
                                                              uint8_t *__restrict__ out, uint64_t off_nib,
                                                              uint64_t off_sm, uint64_t sm_bytes,
                                                              Codebook4 cb,
                                                              const uint32_t *__restrict__ cb_dev,
                                                              uint32_t *__restrict__ tile_counts,
                                                              uint8_t *__restrict__ stage)
{
    __shared__ uint32_t table32[64];
    __shared__ uint32_t table16x2[512];
    __shared__ uint32_t wave_totals[kEncThreads / 64];
    __shared__ __align__(16) uint8_t seg_buf[kEncThreads / 64][kSegBytes];
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / 64;
    const uint64_t tile = blockIdx.x;
    const uint64_t base = tile * kEncTile + (uint64_t)wave * kRow;
    const bool full_row = base + kRow <= n;

    uint4 q[kE5Chunks][2];
#pragma unroll
    for (int j = 0; j < kE5Chunks; ++j) {
        const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
        if (full_row || c0 + 32 <= n) {
            q[j][0] = load_nt(reinterpret_cast<const uint4 *>(in + c0));
            q[j][1] = load_nt(reinterpret_cast<const uint4 *>(in + c0 + 16));
        } else {
            uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (uint32_t k = 0; k < 32 && c0 + k < n; ++k) w[k / 4] |= (uint32_t)in[c0 + k] << (8 * (k & 3));
            q[j][0] = make_uint4(w[0], w[1], w[2], w[3]);
            q[j][1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
    if (cb_dev) cb = load_codebook(cb_dev);
    build_encode_table(table32, cb, 32);
    __syncthreads();
    build_pair_table(table16x2, reinterpret_cast<const uint8_t *>(table32));
    __syncthreads();
    const uint16_t *table16 = reinterpret_cast<const uint16_t *>(table16x2);
    uint32_t fl[kE5Chunks][4];
    uint32_t cnt[kE5Chunks];
#pragma unroll
    for (int j = 0; j < kE5Chunks; ++j) {
        const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
        uint4 nib;
        uint32_t sm3[3];
        encode_chunk_e5m2_pairs(q[j][0], q[j][1], table16, nib, sm3, fl[j]);
        uint32_t *sm_dst = reinterpret_cast<uint32_t *>(out + off_sm + (c0 / 32) * 12);
        if (full_row || c0 + 32 <= n) {
            store_nt(reinterpret_cast<uint4 *>(out + off_nib + c0 / 2), nib);
            store3_nt(sm_dst, sm3);
        } else if (c0 < n) {
            // last, partial chunk: missing elements get code 0, symbol 0 and
            // no escape; only the sign/mantissa bytes that hold data are stored
            const uint32_t valid = (uint32_t)(n - c0);
            uint32_t nw[4] = {nib.x, nib.y, nib.z, nib.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int v = (int)valid - 8 * s;
                nw[s] &= v >= 8 ? 0xFFFFFFFFu : (v <= 0 ? 0u : (uint32_t)((1ull << (4 * v)) - 1));
                fl[j][s] &= group_flag_keep(v);
            }
            *reinterpret_cast<uint4 *>(out + off_nib + c0 / 2) = make_uint4(nw[0], nw[1], nw[2], nw[3]);
            uint32_t sw[3] = {sm3[0], sm3[1], sm3[2]};
            const uint32_t bits = 3 * valid;
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                const int b = (int)bits - 32 * w;
                sw[w] &= b >= 32 ? 0xFFFFFFFFu : (b <= 0 ? 0u : ((1u << b) - 1));
            }
            const uint64_t sm_start = off_sm + (c0 / 32) * 12;
            const uint64_t sm_end = off_sm + sm_bytes;
            for (uint32_t i = 0; i < 12 && sm_start + i < sm_end; ++i)
                out[sm_start + i] = (uint8_t)(sw[i / 4] >> (8 * (i & 3)));
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) fl[j][s] = 0;
        }
        cnt[j] = __popc(fl[j][0]) + __popc(fl[j][1]) + __popc(fl[j][2]) + __popc(fl[j][3]);
    }
    uint32_t row_base[kE5Chunks], row_total[kE5Chunks], lane_before[kE5Chunks];
    const uint32_t wave_total = wave_chunk_ranks<kE5Chunks>(cnt, row_base, row_total, lane_before);
    uint32_t tile_total;
    const uint32_t wave_before = workgroup_wave_prefix<kEncThreads / 64>(wave_total, wave_totals, tile_total);
    if (wave_total && tile_total <= kRederiveRecords) {
        uint8_t *tstage = stage + tile * (3ull * kEncTile);
        uint8_t *buf = seg_buf[wave];
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
            const uint32_t rank = wave_before + row_base[j];
            // escape masks and exponents of the chunk, from its flag words and input words
            const uint32_t dw[8] = {q[j][0].x, q[j][0].y, q[j][0].z, q[j][0].w,
                                    q[j][1].x, q[j][1].y, q[j][1].z, q[j][1].w};
            uint32_t esc8[4];
            uint64_t ex[4];
#pragma unroll
            for (int s8 = 0; s8 < 4; ++s8) {
                esc8[s8] = flags_to_mask8(fl[j][s8]);
                ex[s8] = (uint64_t)((dw[2 * s8] >> 2) & 0x1F1F1F1Fu) |
                         ((uint64_t)((dw[2 * s8 + 1] >> 2) & 0x1F1F1F1Fu) << 32);
            }
            if (row_total[j] <= kDirectRecords) {                      // wave-uniform
                if (cnt[j]) {
                    uint32_t r = rank + lane_before[j];
#pragma unroll
                    for (int s8 = 0; s8 < 4; ++s8) {
                        put_records(tstage, r, esc8[s8], ex[s8], (uint32_t)((c0 + 8 * s8) & 0xFFFFu));
                        r += __popc(esc8[s8]);
                    }
                }
                continue;
            }
            // four segments of 16 lanes x 32 elements
#pragma unroll
            for (uint32_t q4 = 0; q4 < 4; ++q4) {
                const uint32_t seg_first = __builtin_amdgcn_readlane(lane_before[j], 16 * q4);
                const uint32_t seg_end =
                    q4 < 3 ? (uint32_t)__builtin_amdgcn_readlane(lane_before[j], 16 * (q4 + 1)) : row_total[j];
                if (seg_end == seg_first) continue;                    // wave-uniform
                const uint32_t g0 = 3 * (rank + seg_first);
                if (lane / 16 == q4 && cnt[j]) {
                    uint32_t off = (g0 & 3) + 3 * (lane_before[j] - seg_first);
#pragma unroll
                    for (int s8 = 0; s8 < 4; ++s8)
                        off = lds_put_records(buf, off, esc8[s8], ex[s8], (uint32_t)((c0 + 8 * s8) & 0xFFFFu));
                }
                wave_lds_fence();
                flush_segment(buf, tstage, g0, 3 * (seg_end - seg_first));
                wave_lds_fence();
            }
        }
    }
    if (threadIdx.x == 0) tile_counts[tile] = tile_total | (tile_total > kRederiveRecords ? kRederiveFlag : 0u);
}

// ---------------------------------------------------------------------------
// One-workgroup scans.  Both scan kernels read their counts with coalesced
// dwordx4 loads: in pass i, thread t holds item i * 1024 + t, where an item
// is four consecutive counts (four tiles = one block for encode, four blocks
// for decode).  Up to kScanBatch passes are loaded at once; each pass gets
// its own 64-lane prefix sums, the 16 waves' totals meet in LDS, and one
// thread per pass turns them into exclusive offsets.  A running 64-bit carry
// joins successive batches.
// ---------------------------------------------------------------------------
constexpr int kScanBatch = 8;
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

struct HeaderArgs {
    uint64_t n, nb;
    uint32_t dtype, version;
    Codebook4 cb;
    uint64_t pad_start[3], pad_end[3];
};

// A device codebook (sz_codebook in device memory) replaces `cb` and is
// checked: its dtype word, entries below the symbol count, no repeats.
// Returns 0 or the error code; called by every thread of the workgroup.
__device__ __forceinline__ int32_t device_codebook_verdict(const uint32_t *__restrict__ cb_dev, uint32_t dtype,
                                                           Codebook4 &cb)
{
    if (!cb_dev) return 0;
    cb = load_codebook(cb_dev);
    const uint32_t symbols = dtype == SZ_BF16 ? 256u : 32u;
    bool bad = false;
    if (threadIdx.x < 16) {
        const uint32_t e = cb_entry(cb, threadIdx.x);
        bad = e >= symbols;
        for (uint32_t d = 0; d < threadIdx.x; ++d) bad = bad || cb_entry(cb, d) == e;
    }
    int32_t verdict = __syncthreads_or(bad) ? SZ_E_ARG : 0;
    if (cb_dev[0] != dtype) verdict = SZ_E_DTYPE;
    return verdict;
}

// Writes the stream header (16 little-endian words; E, words 4 and 5, only
// when write_e, as 0), the zero padding between sections and the status
// word.  A bad device codebook (verdict != 0) zeroes the magic, so the
// stream cannot be decoded.  Threads 0..255 of the workgroup take part.
__device__ __forceinline__ void write_header(uint8_t *__restrict__ out, const HeaderArgs &h, const Codebook4 &cb,
                                             int32_t verdict, bool write_e, int32_t *__restrict__ status)
{
    const uint32_t tid = threadIdx.x;
    if (tid < 16 && (write_e || (tid != 4 && tid != 5))) {
        uint32_t w = 0;
        switch (tid) {
        case 0: w = verdict ? 0u : kMagic; break;
        case 1: w = h.version | (h.dtype << 16) | (kLog2Block << 24); break;
        case 2: w = (uint32_t)h.n; break;
        case 3: w = (uint32_t)(h.n >> 32); break;
        case 6: w = (uint32_t)h.nb; break;
        case 8: w = cb.w[0]; break;
        case 9: w = cb.w[1]; break;
        case 10: w = cb.w[2]; break;
        case 11: w = cb.w[3]; break;
        default: w = 0; break;
        }
        reinterpret_cast<uint32_t *>(out)[tid] = w;
    }
    if (tid == 0) status[0] = verdict;
    // zero padding between sections (each range is shorter than 256 bytes)
    if (tid < 256) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const uint64_t a = h.pad_start[r] + tid;
            if (a < h.pad_end[r]) out[a] = 0;
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel: encode scan.  One workgroup turns the tile escape counts into the
// per-block escape counts of the stream and the exclusive escape offset of
// every block, then writes the header (with E) and the zero padding between
// sections.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void sz_enc_scan(const uint32_t *__restrict__ tile_counts,
                                                            uint32_t nt,
                                                            uint64_t *__restrict__ block_offsets,
                                                            uint8_t *__restrict__ out, HeaderArgs h,
                                                            const uint32_t *__restrict__ cb_dev,
                                                            int32_t *__restrict__ status)
{
    __shared__ ScanLds lds;
    const uint32_t tid = threadIdx.x;
    // a bad device codebook zeroes the magic and sets the status word
    Codebook4 cb = h.cb;
    const int32_t verdict = device_codebook_verdict(cb_dev, h.dtype, cb);
    const uint32_t nb = (uint32_t)h.nb;
    if (tid == 0) lds.carry = 0;
    uint32_t *block_counts = reinterpret_cast<uint32_t *>(out + 64);
    for (uint32_t b0 = 0; b0 < nb; b0 += kScanBatch * kScanThreads) {
        uint32_t x[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const uint32_t b = b0 + i * kScanThreads + tid;
            x[i] = 0;
            if (b < nb) {
                const uint4 v = *reinterpret_cast<const uint4 *>(tile_counts + kTilesPerBlock * b);
                const uint32_t t = kTilesPerBlock * b;
                const uint32_t m = ~kRederiveFlag;
                x[i] = (v.x & m) + ((t + 1 < nt) ? v.y & m : 0) + ((t + 2 < nt) ? v.z & m : 0) +
                       ((t + 3 < nt) ? v.w & m : 0);
            }
        }
        uint64_t base[kScanBatch];
        scan_batch(x, base, lds);
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const uint32_t b = b0 + i * kScanThreads + tid;
            if (b < nb) {
                block_counts[b] = x[i];
                block_offsets[b] = base[i];
            }
        }
    }
    const uint64_t total = lds.carry;
    write_header(out, h, cb, verdict, false, status);
    if (tid == 0) {
        reinterpret_cast<uint32_t *>(out)[4] = (uint32_t)total;
        reinterpret_cast<uint32_t *>(out)[5] = (uint32_t)(total >> 32);
    }
}

// ---------------------------------------------------------------------------
// Kernel: escape compaction.  One wave per block (four blocks per workgroup)
// copies the staged records of the block's four tiles (3 bytes each) to
// out[off_esc + 3 * offset ...), tile after tile; when no tile of the block
// holds more than kGroupCopyRecords records, four 16-lane groups copy the four
// tiles at once.  The body of each copy is written with 16-byte aligned
// dwordx4 stores assembled by v_alignbyte_b32 from five staged words; the
// unaligned bytes at both ends, whose dwords the neighbouring tiles share, are
// written byte by byte.  Flagged (escape-heavy) tiles are re-encoded from the
// input instead and their records written straight to their final place.
// ---------------------------------------------------------------------------
// Copies len bytes of staged records to out[dst0, dst0 + len) with the lanes
// [0, width) of a lane group (lane = index inside the group).
__device__ __forceinline__ void copy_records(const uint8_t *__restrict__ src, uint8_t *__restrict__ out,
                                             uint64_t dst0, uint32_t len, uint32_t lane, uint32_t width)
{
    const uint64_t end = dst0 + len;
    const uint64_t body_begin = std::min<uint64_t>((dst0 + 15) & ~uint64_t(15), end);
    const uint64_t body_end = std::max<uint64_t>(end & ~uint64_t(15), body_begin);
    const uint32_t head = (uint32_t)(body_begin - dst0);
    for (uint32_t i = lane; i < head; i += width) out[dst0 + i] = src[i];
    const uint32_t *src32 = reinterpret_cast<const uint32_t *>(src);
    const uint32_t chunks = (uint32_t)((body_end - body_begin) / 16);
    const uint32_t sh = head & 3;
#pragma unroll 4
    for (uint32_t c = lane; c < chunks; c += width) {
        const uint32_t w0 = (head >> 2) + 4 * c;                 // first source word
        const uint32_t a0 = src32[w0], a1 = src32[w0 + 1], a2 = src32[w0 + 2], a3 = src32[w0 + 3],
                       a4 = src32[w0 + 4];
        const uint4 v = make_uint4(__builtin_amdgcn_alignbyte(a1, a0, sh), __builtin_amdgcn_alignbyte(a2, a1, sh),
                                   __builtin_amdgcn_alignbyte(a3, a2, sh), __builtin_amdgcn_alignbyte(a4, a3, sh));
        *reinterpret_cast<uint4 *>(out + body_begin + 16ull * c) = v;
    }
    const uint32_t tail_src = (uint32_t)(body_end - dst0);
    for (uint32_t i = lane; body_end + i < end; i += width) out[body_end + i] = src[tail_src + i];
}

// Derives the records of an escape-heavy tile again from the input, with one
// wave walking the tile's four rows, and writes them at their final place
// (dst = aligned base, shift = byte misalignment of the tile's first record).
// Half rows keep the re-derivation's register footprint close to the copy
// path's, so both share one occupancy.
constexpr int kRedChunks = 4;
constexpr uint32_t kRedRow = kRedChunks * 64 * 8;

__device__ __forceinline__ void rederive_tile_bf16(const uint16_t *__restrict__ in, uint64_t n, uint64_t tile,
                                                   const uint8_t *table, uint8_t *buf, uint8_t *dst, uint32_t shift)
{
    const uint32_t lane = lane_id();
    uint32_t rank = 0;                                          // wave-uniform
    for (uint32_t row = 0; row < kEncTile / kRedRow; ++row) {
        const uint64_t base = tile * kEncTile + (uint64_t)row * kRedRow;
        if (base >= n) break;
        const bool full_row = base + kRedRow <= n;
        uint4 q[kRedChunks];
#pragma unroll
        for (int j = 0; j < kRedChunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 8;
            if (full_row || c0 + 8 <= n) {
                q[j] = load_nt(reinterpret_cast<const uint4 *>(in + c0));
            } else {
                uint16_t v[8];
#pragma unroll
                for (uint32_t k = 0; k < 8; ++k) v[k] = (c0 + k < n) ? in[c0 + k] : 0;
                q[j] = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                                  v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
            }
        }
        uint32_t esc[kRedChunks], cnt[kRedChunks];
        uint64_t ex[kRedChunks];
#pragma unroll
        for (int j = 0; j < kRedChunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 8;
            uint32_t nib;
            uint2 sm;
            encode_chunk_bf16(q[j], table, nib, sm, esc[j], ex[j]);
            if (c0 >= n) esc[j] = 0;
            else if (c0 + 8 > n) esc[j] &= (1u << (uint32_t)(n - c0)) - 1;
            cnt[j] = __popc(esc[j]);
        }
        uint32_t row_base[kRedChunks], row_total[kRedChunks], lane_before[kRedChunks];
        const uint32_t total = wave_chunk_ranks<kRedChunks>(cnt, row_base, row_total, lane_before);
#pragma unroll
        for (int j = 0; j < kRedChunks; ++j) {
            if (row_total[j] == 0) continue;                    // wave-uniform
            const uint32_t g0 = shift + 3 * (rank + row_base[j]);
            const uint32_t pos0 = (uint32_t)((base + (uint64_t)(j * 64 + lane) * 8) & 0xFFFFu);
            if (esc[j]) lds_put_records(buf, (g0 & 3) + 3 * lane_before[j], esc[j], ex[j], pos0);
            wave_lds_fence();
            flush_segment(buf, dst, g0, 3 * row_total[j]);
            wave_lds_fence();
        }
        rank += total;
    }
}

__device__ __forceinline__ void rederive_tile_e5m2(const uint8_t *__restrict__ in, uint64_t n, uint64_t tile,
                                                   const uint8_t *table, uint8_t *buf, uint8_t *dst, uint32_t shift)
{
    const uint32_t lane = lane_id();
    uint32_t rank = 0;                                          // wave-uniform
    for (uint32_t row = 0; row < kEncTile / kRow; ++row) {
        const uint64_t base = tile * kEncTile + (uint64_t)row * kRow;
        if (base >= n) break;
        const bool full_row = base + kRow <= n;
        uint4 q[kE5Chunks][2];
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
            if (full_row || c0 + 32 <= n) {
                q[j][0] = load_nt(reinterpret_cast<const uint4 *>(in + c0));
                q[j][1] = load_nt(reinterpret_cast<const uint4 *>(in + c0 + 16));
            } else {
                uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                for (uint32_t k = 0; k < 32 && c0 + k < n; ++k) w[k / 4] |= (uint32_t)in[c0 + k] << (8 * (k & 3));
                q[j][0] = make_uint4(w[0], w[1], w[2], w[3]);
                q[j][1] = make_uint4(w[4], w[5], w[6], w[7]);
            }
        }
        uint32_t esc[kE5Chunks], cnt[kE5Chunks];
        uint64_t ex[kE5Chunks][4];
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
            uint4 nib;
            uint32_t sm3[3];
            encode_chunk_e5m2(q[j][0], q[j][1], table, nib, sm3, esc[j], ex[j]);
            if (c0 >= n) esc[j] = 0;
            else if (c0 + 32 > n) esc[j] &= (uint32_t)((1ull << (n - c0)) - 1);
            cnt[j] = __popc(esc[j]);
        }
        uint32_t row_base[kE5Chunks], row_total[kE5Chunks], lane_before[kE5Chunks];
        const uint32_t total = wave_chunk_ranks<kE5Chunks>(cnt, row_base, row_total, lane_before);
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            if (row_total[j] == 0) continue;                    // wave-uniform
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
#pragma unroll
            for (uint32_t q4 = 0; q4 < 4; ++q4) {
                const uint32_t seg_first = __builtin_amdgcn_readlane(lane_before[j], 16 * q4);
                const uint32_t seg_end =
                    q4 < 3 ? (uint32_t)__builtin_amdgcn_readlane(lane_before[j], 16 * (q4 + 1)) : row_total[j];
                if (seg_end == seg_first) continue;             // wave-uniform
                const uint32_t g0 = shift + 3 * (rank + row_base[j] + seg_first);
                if (lane / 16 == q4 && cnt[j]) {
                    uint32_t off = (g0 & 3) + 3 * (lane_before[j] - seg_first);
#pragma unroll
                    for (int s8 = 0; s8 < 4; ++s8)
                        off = lds_put_records(buf, off, (esc[j] >> (8 * s8)) & 0xFFu, ex[j][s8],
                                              (uint32_t)((c0 + 8 * s8) & 0xFFFFu));
                }
                wave_lds_fence();
                flush_segment(buf, dst, g0, 3 * (seg_end - seg_first));
                wave_lds_fence();
            }
        }
        rank += total;
    }
}

// Tiles with at most this many records are copied by 16-lane groups, the
// block's four tiles at once; heavier blocks copy tile after tile with the
// whole wave.
constexpr uint32_t kGroupCopyRecords = 1024;

// Moves the records of block b to their place in the stream with one wave.
// Lanes 0..3 of `meta` hold the block's four tile counts (flag bit
// included; 0 past the last tile); `off` is the escape offset of the block's
// first record.
template <int DT>
__device__ __forceinline__ void compact_block(const uint8_t *__restrict__ stage, uint32_t meta, uint64_t b,
                                              uint64_t off, uint8_t *__restrict__ out, uint64_t off_esc,
                                              const void *__restrict__ in, uint64_t n, const uint8_t *table,
                                              uint8_t *buf, uint32_t item)
{
    const uint32_t lane = lane_id();
    const uint64_t t0 = kTilesPerBlock * b;
    uint32_t cnt[kTilesPerBlock], before[kTilesPerBlock], most = 0, run = 0, rederive = 0;
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t) {
        const uint32_t v = __builtin_amdgcn_readlane(meta, t);
        cnt[t] = v & ~kRederiveFlag;
        rederive |= (v >> 31) << t;
        before[t] = run;
        run += cnt[t];
        most = std::max(most, cnt[t]);
    }
    if (most <= kGroupCopyRecords && !rederive) {               // wave-uniform
        const uint32_t g = lane >> 4;
        uint32_t k = 0, bef = 0;
#pragma unroll
        for (uint32_t t = 0; t < kTilesPerBlock; ++t)
            if (g == t) {
                k = cnt[t];
                bef = before[t];
            }
        if (k) copy_records(stage + (t0 + g) * (3ull * kEncTile), out, off_esc + item * (off + bef), item * k, lane & 15, 16);
        return;
    }
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t) {
        if (cnt[t] == 0) continue;
        const uint64_t dst0 = off_esc + item * (off + before[t]);
        if ((rederive >> t) & 1) {
            if (DT == SZ_BF16)
                rederive_tile_bf16(static_cast<const uint16_t *>(in), n, t0 + t, table, buf, out + (dst0 & ~uint64_t(3)),
                                   (uint32_t)(dst0 & 3));
            else
                rederive_tile_e5m2(static_cast<const uint8_t *>(in), n, t0 + t, table, buf, out + (dst0 & ~uint64_t(3)),
                                   (uint32_t)(dst0 & 3));
        } else {
            copy_records(stage + (t0 + t) * (3ull * kEncTile), out, dst0, item * cnt[t], lane, 64);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(kCompactThreads) __attribute__((amdgpu_waves_per_eu(8))) void sz_enc_compact(
    const uint8_t *__restrict__ stage, const uint32_t *__restrict__ tile_counts,
    const uint64_t *__restrict__ block_offsets, uint8_t *__restrict__ out, uint64_t off_esc, uint64_t nt,
    uint64_t nb, const void *__restrict__ in, uint64_t n, Codebook4 cb, const uint32_t *__restrict__ cb_dev,
    uint32_t item)
{
    __shared__ uint32_t table32[64];
    __shared__ __align__(16) uint8_t seg_buf[kCompactThreads / 64][kSegBytes];
    if (cb_dev) cb = load_codebook(cb_dev);
    build_encode_table(table32, cb, DT == SZ_BF16 ? 256 : 32);
    __syncthreads();
    const uint64_t b = (uint64_t)blockIdx.x * (kCompactThreads / 64) + threadIdx.x / 64;
    if (b >= nb) return;
    const uint32_t lane = lane_id();
    // lanes 0..3 fetch the tile counts, lane 4 the block's escape offset
    const uint64_t t0 = kTilesPerBlock * b;
    uint64_t meta = 0;
    if (lane < kTilesPerBlock && t0 + lane < nt) meta = tile_counts[t0 + lane];
    else if (lane == kTilesPerBlock) meta = block_offsets[b];
    const uint64_t off = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(meta >> 32), kTilesPerBlock) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((uint32_t)meta, kTilesPerBlock);
    compact_block<DT>(stage, (uint32_t)meta, b, off, out, off_esc, in, n, reinterpret_cast<const uint8_t *>(table32),
                      seg_buf[threadIdx.x / 64], item);
}

// ---------------------------------------------------------------------------
// Kernel: compaction with its own prefix, in place of sz_enc_scan plus
// sz_enc_compact for streams of up to kFusedPrefixTiles tiles.  A 1024-lane
// workgroup owns 16 consecutive blocks: all its lanes sum the counts of the
// tiles before its first block (aligned dwordx4 loads, from L2 after the
// first workgroups), the 16 block totals meet in LDS, and each wave then
// moves its block's records as sz_enc_compact does.  The wave of a block
// also writes the block's count into the stream, the wave of the last block
// writes E, and workgroup 0 writes the rest of the header, the section
// padding and the status word (device codebook check) as sz_enc_scan does.
// The tile counts before a workgroup are re-read by every later workgroup, a
// cost that grows with the square of the tile count: on MI355X this path
// saves 2-3 us per encode up to 16M elements, breaks even at 32M and loses
// beyond, so larger streams take the scan.
// ---------------------------------------------------------------------------
constexpr uint32_t kFusedThreads = 1024;
constexpr uint32_t kFusedBlocks = kFusedThreads / 64;
constexpr uint64_t kFusedPrefixTiles = 2048;

template <int DT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(8))) void sz_enc_compact_fused(
    const uint8_t *__restrict__ stage, const uint32_t *__restrict__ tile_counts, uint8_t *__restrict__ out,
    uint64_t off_esc, uint64_t nt, const void *__restrict__ in, HeaderArgs h, const uint32_t *__restrict__ cb_dev,
    int32_t *__restrict__ status, uint32_t item)
{
    __shared__ uint32_t table32[64];
    __shared__ __align__(16) uint8_t seg_buf[kFusedBlocks][kSegBytes];
    __shared__ uint64_t wave_part[kFusedBlocks];
    __shared__ uint32_t block_total[kFusedBlocks];
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
    const uint64_t nb = h.nb;
    Codebook4 cb = h.cb;
    const int32_t verdict = device_codebook_verdict(cb_dev, h.dtype, cb);
    build_encode_table(table32, cb, DT == SZ_BF16 ? 256 : 32);
    // escapes of the tiles before this workgroup's first block (a multiple of
    // 64 tiles, all of them below nt)
    const uint64_t b0 = (uint64_t)blockIdx.x * kFusedBlocks;
    const uint64_t tiles_before = kTilesPerBlock * b0;
    uint64_t part = 0;
#pragma unroll 4
    for (uint64_t t = 4 * tid; t < tiles_before; t += 4 * kFusedThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(tile_counts + t);
        part += (uint64_t)(v.x & ~kRederiveFlag) + (v.y & ~kRederiveFlag) + (v.z & ~kRederiveFlag) +
                (v.w & ~kRederiveFlag);
    }
    part = wave_sum_u64(part);
    // this wave's block: lanes 0..3 fetch its tile counts
    const uint64_t b = b0 + wave;
    const uint64_t t0 = kTilesPerBlock * b;
    uint32_t meta = 0;
    if (lane < kTilesPerBlock && t0 + lane < nt) meta = tile_counts[t0 + lane];
    uint32_t total = 0;
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t) total += __builtin_amdgcn_readlane(meta, t) & ~kRederiveFlag;
    if (lane == 0) {
        wave_part[wave] = part;
        block_total[wave] = total;
    }
    __syncthreads();
    uint64_t acc = 0;
#pragma unroll
    for (uint32_t w = 0; w < kFusedBlocks; ++w) {
        acc += wave_part[w];
        if (w < wave) acc += block_total[w];
    }
    // wave-uniform: kept in scalar registers for the copy and re-derivation
    const uint64_t off = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(acc >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)acc);
    uint32_t *header32 = reinterpret_cast<uint32_t *>(out);
    if (b < nb && lane == 0) {
        reinterpret_cast<uint32_t *>(out + 64)[b] = total;
        if (b == nb - 1) {
            const uint64_t e = off + total;
            header32[4] = (uint32_t)e;
            header32[5] = (uint32_t)(e >> 32);
        }
    }
    if (blockIdx.x == 0) write_header(out, h, cb, verdict, nb == 0, status);
    if (b >= nb) return;
    compact_block<DT>(stage, meta, b, off, out, off_esc, in, h.n, reinterpret_cast<const uint8_t *>(table32),
                      seg_buf[wave], item);
}

// ---------------------------------------------------------------------------
// Kernel: decode scan.  One workgroup validates the header and the block
// counts (each at most its block length, summing to E) and writes the
// exclusive escape offset of every block.  It writes its verdict (0 or a
// negative error code) to status[0], the caller-visible status word, and to
// status[1], which the block decoders read: they only ever write status[0],
// so every wave of a decode workgroup sees the same verdict.
// ---------------------------------------------------------------------------
struct DecodeArgs {
    uint64_t n, nb, in_bytes, off_nib, off_sm, off_esc;
    uint32_t dtype, symbols;
    uint32_t version, item, entries;      // format version, escape item bytes, codebook entries used
};

// The stream header's verdict: 0, or the error of the first failed check
// (magic, version, block size, dtype, N, nb, reserved word, E against N and
// in_bytes, codebook entries).
__device__ __forceinline__ int32_t header_verdict(const uint8_t *__restrict__ in, const DecodeArgs &a)
{
    const uint32_t *h32 = reinterpret_cast<const uint32_t *>(in);
    const uint32_t w1 = h32[1];
    const uint64_t n_hdr = (uint64_t)h32[2] | ((uint64_t)h32[3] << 32);
    const uint64_t e_hdr = (uint64_t)h32[4] | ((uint64_t)h32[5] << 32);
    if (h32[0] != kMagic || (w1 & 0xFFFFu) != a.version || (w1 >> 24) != kLog2Block) return SZ_E_FORMAT;
    if (((w1 >> 16) & 0xFFu) != a.dtype) return SZ_E_DTYPE;
    if (n_hdr != a.n || h32[6] != (uint32_t)a.nb || h32[7] != 0) return SZ_E_FORMAT;
    if (e_hdr > a.n || a.off_esc + a.item * e_hdr > a.in_bytes) return SZ_E_FORMAT;
    // used entries must be exponent values, unused ones zero
    int32_t err = 0;
    for (uint32_t c = 0; c < 16; ++c)
        if (c < a.entries ? in[32 + c] >= a.symbols : in[32 + c] != 0) err = SZ_E_FORMAT;
    return err;
}

// ---------------------------------------------------------------------------
// Kernel: decode header check, in place of sz_dec_scan for streams of up to
// kFusedPrefixBlocks blocks, whose decoders find their escape offsets
// themselves (on MI355X 1.5-4.6 us faster per decode up to 64M elements; far
// beyond, every decoder re-reading the counts before it costs more than the
// scan).  One wave checks the header and writes the verdict to both
// status words, as sz_dec_scan does; the block counts are checked by the
// decoders.
// ---------------------------------------------------------------------------
constexpr uint64_t kFusedPrefixBlocks = 1024;

__global__ __launch_bounds__(64) void sz_dec_head(const uint8_t *__restrict__ in, DecodeArgs a,
                                                  int32_t *__restrict__ status)
{
    if (threadIdx.x == 0) {
        const int32_t err = header_verdict(in, a);
        status[0] = err;
        status[1] = err;
    }
}

__global__ __launch_bounds__(kScanThreads) void sz_dec_scan(const uint8_t *__restrict__ in, DecodeArgs a,
                                                            uint64_t *__restrict__ block_offsets,
                                                            int32_t *__restrict__ status)
{
    __shared__ ScanLds lds;
    __shared__ int32_t bad;
    const uint32_t tid = threadIdx.x;
    const uint64_t e_hdr = *reinterpret_cast<const uint64_t *>(in + 16);
    const int32_t err = header_verdict(in, a);
    if (err) {
        if (tid == 0) {
            status[0] = err;
            status[1] = err;
        }
        return;
    }
    if (tid == 0) {
        bad = 0;
        lds.carry = 0;
    }
    // items are groups of four block counts: one aligned dwordx4 each (the
    // count array starts at byte 64 and is followed by padding up to off_nib)
    const uint32_t *counts = reinterpret_cast<const uint32_t *>(in + 64);
    const uint32_t nb = (uint32_t)a.nb;
    // the last block may be shorter than B: its count is bounded by its length
    bool too_many = nb && tid == 0 && counts[nb - 1] > a.n - (uint64_t)(nb - 1) * kBlock;
    for (uint32_t g0 = 0; g0 < nb; g0 += 4 * kScanBatch * kScanThreads) {
        uint4 v[kScanBatch];
        uint32_t x[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const uint32_t g = g0 + 4 * (i * kScanThreads + tid);
            v[i] = make_uint4(0, 0, 0, 0);
            if (g < nb) {
                v[i] = *reinterpret_cast<const uint4 *>(counts + g);
                if (g + 1 >= nb) v[i].y = 0;
                if (g + 2 >= nb) v[i].z = 0;
                if (g + 3 >= nb) v[i].w = 0;
                too_many |= std::max(std::max(v[i].x, v[i].y), std::max(v[i].z, v[i].w)) > (uint32_t)kBlock;
            }
            x[i] = v[i].x + v[i].y + v[i].z + v[i].w;
        }
        uint64_t base[kScanBatch];
        scan_batch(x, base, lds);
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const uint32_t g = g0 + 4 * (i * kScanThreads + tid);
            if (g < nb) {
                const uint64_t o1 = base[i] + v[i].x, o2 = o1 + v[i].y, o3 = o2 + v[i].z;
                if (g + 3 < nb) {
                    // 32 aligned bytes: two dwordx4 stores of offset pairs
                    uint4 *dst = reinterpret_cast<uint4 *>(block_offsets + g);
                    dst[0] = make_uint4((uint32_t)base[i], (uint32_t)(base[i] >> 32), (uint32_t)o1, (uint32_t)(o1 >> 32));
                    dst[1] = make_uint4((uint32_t)o2, (uint32_t)(o2 >> 32), (uint32_t)o3, (uint32_t)(o3 >> 32));
                } else {
                    block_offsets[g] = base[i];
                    if (g + 1 < nb) block_offsets[g + 1] = o1;
                    if (g + 2 < nb) block_offsets[g + 2] = o2;
                }
            }
        }
    }
    if (too_many) bad = 1;
    __syncthreads();
    if (tid == 0) {
        const int32_t verdict = (bad || lds.carry != e_hdr) ? SZ_E_FORMAT : 0;
        status[0] = verdict;
        status[1] = verdict;
    }
}

// ---------------------------------------------------------------------------
// Decode kernels: one 1024-lane workgroup per 64K block.  First an LDS map
// from each chunk to the first escape record inside it is built from the
// block's records (validating their order and range), then every wave
// decodes one 4096-element row in registers, patches the escaped exponents
// and stores once.
// ---------------------------------------------------------------------------
constexpr uint32_t kNoEscape = 0xFFFFu;

// Escape offset of block b and its count check.  With block_offsets (from
// sz_dec_scan, which has checked every count) the offset is read.  Without
// them (at most kFusedPrefixBlocks blocks) the whole workgroup sums the
// counts of blocks 0..b-1 from the stream with aligned dwordx4 loads (the
// count array starts at byte 64 and its section is padded to 256 bytes, so a
// load of four counts never leaves it), each count capped at the block
// length so that 32-bit sums cannot wrap, and checks the block's own count:
// at most the block length, the records inside the E of the header, and for
// the last block offset + count = E.  A failed check sets the status word
// and zeroes k, so the block decodes without touching records; a count
// above its block length fails its own block's check.  Called by every
// thread; the result is workgroup-uniform.
__device__ uint64_t block_escape_offset(const uint8_t *__restrict__ in, const DecodeArgs &a, uint64_t b,
                                        uint32_t blen, uint64_t e_total, const uint64_t *__restrict__ block_offsets,
                                        uint32_t &k, int32_t *__restrict__ status, uint32_t *part)
{
    if (block_offsets) return block_offsets[b];
    if (k == 0 && b + 1 != a.nb) return 0;                      // no records and not the last block
    const uint32_t *counts = reinterpret_cast<const uint32_t *>(in + 64);
    const uint32_t bb = (uint32_t)b;                            // b < kFusedPrefixBlocks
    uint32_t sum = 0;
#pragma unroll 1
    for (uint32_t g = 4 * threadIdx.x; g < bb; g += 4 * kDecThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(counts + g);
        sum += std::min<uint32_t>(v.x, kBlock) + (g + 1 < bb ? std::min<uint32_t>(v.y, kBlock) : 0u) +
               (g + 2 < bb ? std::min<uint32_t>(v.z, kBlock) : 0u) +
               (g + 3 < bb ? std::min<uint32_t>(v.w, kBlock) : 0u);
    }
    sum = read_lane63(wave_inclusive_sum(sum));
    if (lane_id() == 0) part[threadIdx.x / 64] = sum;
    __syncthreads();
    uint32_t r0 = 0;
#pragma unroll
    for (uint32_t w = 0; w < kDecThreads / 64; ++w) r0 += part[w];
    r0 = __builtin_amdgcn_readfirstlane(r0);
    if (k > blen || r0 + (uint64_t)k > e_total || (b + 1 == a.nb && r0 + (uint64_t)k != e_total)) {
        if (threadIdx.x == 0) atomicExch(status, SZ_E_FORMAT);
        k = 0;
    }
    return r0;
}
// Blocks with up to this many escapes decode through an LDS map of their
// records; blocks with more go through the exponent plane.
constexpr uint32_t kMappedEscapes = 8192;

// Escape record r of the stream: position and exponent.
__device__ __forceinline__ void read_record(const uint8_t *esc, uint64_t r, uint32_t &pos, uint32_t &e)
{
    const uint8_t *p = esc + 3 * r;
    pos = (uint32_t)p[0] | ((uint32_t)p[1] << 8);
    e = p[2];
}

// Four consecutive records from one 16-byte window of aligned words.  The
// window never leaves the record section: it starts at most 3 bytes before
// record R and ends at most 3 bytes after record R+3, and callers use it only
// while a whole record group past R+3 remains in the stream (otherwise they
// read the records byte by byte).
__device__ __forceinline__ void read_records4(const uint8_t *esc, uint64_t r, uint32_t pos[4], uint32_t e[4])
{
    const uint64_t byte0 = 3 * r;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(esc + (byte0 & ~uint64_t(3)));
    const uint32_t sh = (uint32_t)(byte0 & 3);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    const uint32_t d0 = __builtin_amdgcn_alignbyte(w1, w0, sh);   // bytes 0..3 of the 12
    const uint32_t d1 = __builtin_amdgcn_alignbyte(w2, w1, sh);   // bytes 4..7
    const uint32_t d2 = __builtin_amdgcn_alignbyte(w3, w2, sh);   // bytes 8..11
    pos[0] = d0 & 0xFFFFu;
    e[0] = (d0 >> 16) & 0xFFu;
    pos[1] = (d0 >> 24) | ((d1 & 0xFFu) << 8);
    e[1] = (d1 >> 8) & 0xFFu;
    pos[2] = d1 >> 16;
    e[2] = d2 & 0xFFu;
    pos[3] = (d2 >> 8) & 0xFFFFu;
    e[3] = d2 >> 24;
}

// Loads the k (<= kMappedEscapes) records of a block into LDS as
// pos | exponent << 16, four records per aligned three-word window where the
// window stays inside the record section, one by one at its end.
__device__ __forceinline__ void load_block_records(const uint8_t *esc, uint64_t r0, uint32_t k, uint64_t e_total,
                                                   uint32_t *rec)
{
    for (uint32_t r = 4 * threadIdx.x; r < k; r += 4 * blockDim.x) {
        uint32_t pos[4], e[4];
        if (r0 + r + 5 < e_total) {
            read_records4(esc, r0 + r, pos, e);
        } else {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                pos[q] = e[q] = 0;
                if (r + q < k) read_record(esc, r0 + r + q, pos[q], e[q]);
            }
        }
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q)
            if (r + q < k) rec[r + q] = pos[q] | (e[q] << 16);
    }
}

// Builds first[chunk] for the k records of a block held in LDS (chunk =
// pos >> log2_chunk) and reports malformed records through the status word.
template <int LOG2_CHUNK>
__device__ __forceinline__ void map_block_escapes(const uint32_t *rec, uint32_t k, uint32_t blen, uint32_t symbols,
                                                  uint16_t *first, int32_t *status)
{
    bool bad = false;
    for (uint32_t r = threadIdx.x; r < k; r += blockDim.x) {
        const uint32_t v = rec[r];
        const uint32_t pos = v & 0xFFFFu;
        const int32_t prev = r > 0 ? (int32_t)(rec[r - 1] & 0xFFFFu) : -1;
        if (pos >= blen || (int32_t)pos <= prev || (v >> 16) >= symbols) {
            bad = true;
            continue;
        }
        if (r == 0 || (uint32_t)(prev >> LOG2_CHUNK) != (pos >> LOG2_CHUNK)) first[pos >> LOG2_CHUNK] = (uint16_t)r;
    }
    if (bad) atomicExch(status, SZ_E_FORMAT);
}

__device__ __forceinline__ uint4 decode_chunk_bf16(uint32_t nib, uint2 sm, const uint32_t *table)
{
    // table[b] = cb[b & 15] << 7 | cb[b >> 4] << 23: both exponents of a
    // code byte, already in place for two packed BF16 values
    uint4 o;
    o.x = (perm(sm.x, sm.x, 0x01010000u) & 0x807F807Fu) | table[nib & 0xFFu];
    o.y = (perm(sm.x, sm.x, 0x03030202u) & 0x807F807Fu) | table[(nib >> 8) & 0xFFu];
    o.z = (perm(sm.y, sm.y, 0x01010000u) & 0x807F807Fu) | table[(nib >> 16) & 0xFFu];
    o.w = (perm(sm.y, sm.y, 0x03030202u) & 0x807F807Fu) | table[nib >> 24];
    return o;
}

__device__ __forceinline__ void patch_bf16(uint4 &o, uint32_t k, uint32_t e)
{
    const uint32_t sh = 7 + 16 * (k & 1);
    const uint32_t clear = ~(0xFFu << sh);
    const uint32_t set = e << sh;
    switch (k >> 1) {
    case 0: o.x = (o.x & clear) | set; break;
    case 1: o.y = (o.y & clear) | set; break;
    case 2: o.z = (o.z & clear) | set; break;
    default: o.w = (o.w & clear) | set; break;
    }
}

// Blocks with more than kMappedEscapes escapes decode through an exponent
// plane: every element's dense exponent goes to a 64 KB LDS byte array, the
// block's records overwrite their entries (validated on the way), and the
// values are rebuilt from the plane and stored once.

// Register code -> exponent lookup for the eight codes of a code word d
// (element 2k in the low nibble of byte k); cb0..cb3 = codebook bytes.
// v_perm_b32 indexes eight bytes, so each half of the book is one v_perm and
// bit 3 of every code picks the half through a byte mask that v_perm's
// sign-replication selectors build (8: bit 15 of the low word, 9: bit 31 of
// the low word, 10/11: the same bits of the high word).  Returns the eight
// exponents in element order (bytes 0..3 then 4..7).
struct CodebookRegs {
    uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ uint2 lookup_codes8(uint32_t d, const CodebookRegs &cb)
{
    const uint32_t sel_e = d & 0x07070707u;
    const uint32_t sel_o = (d >> 4) & 0x07070707u;
    const uint32_t m_e = perm(d << 4, d << 12, 0x0B090A08u);      // bit 3 of the even codes
    const uint32_t m_o = perm(d, d << 8, 0x0B090A08u);            // bit 3 of the odd codes
    const uint32_t e_even = (perm(cb.w3, cb.w2, sel_e) & m_e) | (perm(cb.w1, cb.w0, sel_e) & ~m_e);
    const uint32_t e_odd = (perm(cb.w3, cb.w2, sel_o) & m_o) | (perm(cb.w1, cb.w0, sel_o) & ~m_o);
    return make_uint2(perm(e_odd, e_even, 0x05010400u), perm(e_odd, e_even, 0x07030602u));
}

// Overwrites plane[pos] with the exponent of each of the block's k records,
// four records per aligned three-word window; invalid records (position out
// of the block or not ascending, exponent out of range) are skipped and
// reported through the status word.
__device__ __forceinline__ void overwrite_exponents(const uint8_t *__restrict__ esc, uint64_t r0, uint32_t k,
                                                    uint32_t blen, uint32_t symbols, uint64_t e_total,
                                                    uint8_t *plane, int32_t *__restrict__ status)
{
    const uint32_t lane = lane_id();
    bool bad = false;
    for (uint32_t r = 4 * threadIdx.x; r < k; r += 4 * blockDim.x) {
        uint32_t pos[4], e[4];
        const uint32_t cnt = std::min<uint32_t>(4, k - r);
        if (r0 + r + 5 < e_total) {
            read_records4(esc, r0 + r, pos, e);
        } else {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                pos[q] = 0xFFFFFFFFu;
                e[q] = 0;
                if (q < cnt) read_record(esc, r0 + r + q, pos[q], e[q]);
            }
        }
        uint32_t prev = __shfl_up(pos[3], 1, 64);        // lane l-1 holds records r-4..r-1
        if (lane == 0 && r > 0) {
            uint32_t pe;
            read_record(esc, r0 + r - 1, prev, pe);
        }
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
            if (q >= cnt) continue;
            const uint32_t before = q == 0 ? prev : pos[q - 1];
            if (pos[q] < blen && e[q] < symbols && (r + q == 0 || pos[q] > before)) plane[pos[q]] = (uint8_t)e[q];
            else bad = true;
        }
    }
    if (bad) atomicExch(status, SZ_E_FORMAT);
}

__global__ __launch_bounds__(kDecThreads) void sz_dec_bf16(const uint8_t *__restrict__ in, DecodeArgs a,
                                                           const uint64_t *__restrict__ block_offsets,
                                                           int32_t *__restrict__ status,
                                                           uint16_t *__restrict__ out)
{
    __shared__ uint32_t table[256];
    __shared__ uint32_t prefix_part[kDecThreads / 64];
    // mapped blocks: first[] (first record of each 8-element chunk, 16 KB) and
    // rec[] (the records, 32 KB); heavy blocks: the exponent plane (64 KB)
    __shared__ __align__(16) uint8_t pool[kBlock];
    uint16_t *first = reinterpret_cast<uint16_t *>(pool);
    uint32_t *rec = reinterpret_cast<uint32_t *>(pool + kBlock / 4);
    uint8_t *plane = pool;
    if (status[1] != 0) return;
    const uint32_t tid = threadIdx.x;
    const uint64_t b = blockIdx.x;
    const uint64_t e0 = b * kBlock;
    const uint32_t blen = (uint32_t)std::min<uint64_t>(kBlock, a.n - e0);
    uint32_t k = reinterpret_cast<const uint32_t *>(in + 64)[b];
    const uint64_t e_total = *reinterpret_cast<const uint64_t *>(in + 16);
    const uint8_t *esc = in + a.off_esc;
    if (tid < 256) {
        const uint32_t lo = in[32 + (tid & 15)];
        const uint32_t hi = in[32 + (tid >> 4)];
        table[tid] = (lo << 7) | (hi << 23);
    }
    // the row's loads are issued first and stay in flight while the escape
    // map is built (the barriers only wait for LDS traffic)
    const uint32_t lane = lane_id();
    const uint32_t rbase = (tid / 64) * kRow;                  // block-local first element of the row
    const bool full_row = rbase + kRow <= blen;
    const uint8_t *nib_base = in + a.off_nib;
    const uint8_t *sm_base = in + a.off_sm;
    uint32_t nib[kBf16Chunks];
    uint2 sm[kBf16Chunks];
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const uint32_t c = rbase + (j * 64 + lane) * 8;
        const uint64_t g = e0 + c;
        if (full_row || c < blen) {
            nib[j] = load_nt(reinterpret_cast<const uint32_t *>(nib_base + g / 2));
            sm[j] = load_nt(reinterpret_cast<const uint2 *>(sm_base + g));
        } else {
            nib[j] = 0;
            sm[j] = make_uint2(0, 0);
        }
    }
    const uint64_t r0 = block_escape_offset(in, a, b, blen, e_total, block_offsets, k, status, prefix_part);
    const bool heavy = k > kMappedEscapes;                        // workgroup-uniform
    if (heavy) {
        const uint32_t *cbw = reinterpret_cast<const uint32_t *>(in + 32);
        const CodebookRegs cb = {cbw[0], cbw[1], cbw[2], cbw[3]};
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + lane) * 8;
            if (c < blen) *reinterpret_cast<uint2 *>(plane + c) = lookup_codes8(nib[j], cb);
        }
        __syncthreads();
        overwrite_exponents(esc, r0, k, blen, 256, e_total, plane, status);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + lane) * 8;
            if (c >= blen) continue;
            const uint2 ex = *reinterpret_cast<const uint2 *>(plane + c);   // exponents, element order
            uint4 o;
            o.x = (perm(sm[j].x, sm[j].x, 0x01010000u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C010C00u) << 7);
            o.y = (perm(sm[j].x, sm[j].x, 0x03030202u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C030C02u) << 7);
            o.z = (perm(sm[j].y, sm[j].y, 0x01010000u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C050C04u) << 7);
            o.w = (perm(sm[j].y, sm[j].y, 0x03030202u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C070C06u) << 7);
            const uint64_t g = e0 + c;
            if (full_row || c + 8 <= blen) {
                store_nt(reinterpret_cast<uint4 *>(out + g), o);
            } else {
                const uint32_t w[4] = {o.x, o.y, o.z, o.w};
                for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
            }
        }
        return;
    }
    if (k) {
        reinterpret_cast<uint4 *>(first)[tid] = make_uint4(~0u, ~0u, ~0u, ~0u);
        load_block_records(esc, r0, k, e_total, rec);
    }
    __syncthreads();
    if (k) map_block_escapes<3>(rec, k, blen, 256, first, status);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const uint32_t c = rbase + (j * 64 + lane) * 8;
        if (c >= blen) continue;
        uint4 o = decode_chunk_bf16(nib[j], sm[j], table);
        if (k) {
            uint32_t r = first[c >> 3];
            if (r != kNoEscape) {
                for (; r < k; ++r) {
                    const uint32_t v = rec[r];
                    if (((v & 0xFFFFu) >> 3) != (c >> 3)) break;
                    patch_bf16(o, v & 7, v >> 16);
                }
            }
        }
        const uint64_t g = e0 + c;
        if (full_row || c + 8 <= blen) {
            store_nt(reinterpret_cast<uint4 *>(out + g), o);
        } else {
            const uint32_t w[4] = {o.x, o.y, o.z, o.w};
            for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
        }
    }
}

// ---------------------------------------------------------------------------
// Decode of the ablation formats (BF16), in the shape of sz_dec_bf16: one
// 1024-lane workgroup per 64K block, one 4096-element row per wave, eight
// 8-element chunks per lane, one store per chunk.
//   Version 2 (Top-8): a chunk's codes are the 3 bytes at 3 * chunk, taken
//   from two aligned words; a 64-entry LDS table turns each pair of 3-bit
//   codes into both exponents.  Escapes are position records, patched as in
//   sz_dec_bf16 (an LDS map for blocks with up to kMappedEscapes records,
//   the exponent plane above that).
//   Version 3 (Top-15 + sentinel): nibble codes as in version 1, code 15
//   marks an escape whose exponent is the next byte of the block's escape
//   bytes.  Each sentinel's rank inside its block comes from per-chunk
//   counts, a wave prefix sum and a prefix over the waves; the block's
//   sentinels must number exactly its count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 decode_chunk_top8(uint32_t code24, uint2 sm, const uint32_t *table64)
{
    // table64[p] = cb[p & 7] << 7 | cb[p >> 3] << 23 for a pair p of 3-bit codes
    uint4 o;
    o.x = (perm(sm.x, sm.x, 0x01010000u) & 0x807F807Fu) | table64[code24 & 63u];
    o.y = (perm(sm.x, sm.x, 0x03030202u) & 0x807F807Fu) | table64[(code24 >> 6) & 63u];
    o.z = (perm(sm.y, sm.y, 0x01010000u) & 0x807F807Fu) | table64[(code24 >> 12) & 63u];
    o.w = (perm(sm.y, sm.y, 0x03030202u) & 0x807F807Fu) | table64[(code24 >> 18) & 63u];
    return o;
}

// Four 3-bit codes (12 bits) -> one code per byte, as v_perm selectors.
__device__ __forceinline__ uint32_t spread_codes3x4(uint32_t x)
{
    return (x & 7u) | ((x << 5) & 0x700u) | ((x << 10) & 0x70000u) | ((x << 15) & 0x7000000u);
}

// Nibbles equal to 15 (the version 3 sentinel): bit 4k set for element k.
__device__ __forceinline__ uint32_t sentinel_bits(uint32_t nib)
{
    return nib & (nib >> 1) & (nib >> 2) & (nib >> 3) & 0x11111111u;
}

template <int V>
__global__ __launch_bounds__(kDecThreads) void sz_dec_variant(const uint8_t *__restrict__ in, DecodeArgs a,
                                                              const uint64_t *__restrict__ block_offsets,
                                                              int32_t *__restrict__ status,
                                                              uint16_t *__restrict__ out)
{
    __shared__ uint32_t table[256];
    __shared__ uint32_t wave_totals[kDecThreads / 64];
    __shared__ uint32_t prefix_part[kDecThreads / 64];
    __shared__ __align__(16) uint8_t pool[V == kTop8 ? kBlock : 16];
    uint16_t *first = reinterpret_cast<uint16_t *>(pool);
    uint32_t *rec = reinterpret_cast<uint32_t *>(pool + kBlock / 4);
    uint8_t *plane = pool;
    if (status[1] != 0) return;
    const uint32_t tid = threadIdx.x;
    const uint64_t b = blockIdx.x;
    const uint64_t e0 = b * kBlock;
    const uint32_t blen = (uint32_t)std::min<uint64_t>(kBlock, a.n - e0);
    uint32_t k = reinterpret_cast<const uint32_t *>(in + 64)[b];
    const uint64_t e_total = *reinterpret_cast<const uint64_t *>(in + 16);
    const uint8_t *esc = in + a.off_esc;
    if (V == kTop8) {
        if (tid < 64) table[tid] = ((uint32_t)in[32 + (tid & 7)] << 7) | ((uint32_t)in[32 + (tid >> 3)] << 23);
    } else if (tid < 256) {
        table[tid] = ((uint32_t)in[32 + (tid & 15)] << 7) | ((uint32_t)in[32 + (tid >> 4)] << 23);
    }
    const uint32_t lane = lane_id();
    const uint32_t rbase = (tid / 64) * kRow;
    const bool full_row = rbase + kRow <= blen;
    uint32_t code[kBf16Chunks];
    uint2 sm[kBf16Chunks];
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const uint32_t c = rbase + (j * 64 + lane) * 8;
        const uint64_t g = e0 + c;
        code[j] = 0;
        sm[j] = make_uint2(0, 0);
        if (full_row || c < blen) {
            if (V == kTop8) {
                const uint64_t byte0 = 3 * (g / 8);
                const uint32_t *w = reinterpret_cast<const uint32_t *>(in + a.off_nib + (byte0 & ~uint64_t(3)));
                code[j] = __builtin_amdgcn_alignbit(w[1], w[0], 8 * (uint32_t)(byte0 & 3)) & 0xFFFFFFu;
            } else {
                code[j] = load_nt(reinterpret_cast<const uint32_t *>(in + a.off_nib + g / 2));
            }
            sm[j] = load_nt(reinterpret_cast<const uint2 *>(in + a.off_sm + g));
        }
    }
    const uint64_t r0 = block_escape_offset(in, a, b, blen, e_total, block_offsets, k, status, prefix_part);
    const bool heavy = V == kTop8 && k > kMappedEscapes;          // workgroup-uniform
    if (V == kTop15S) {
        // ranks of the sentinels inside the block
        uint32_t sbits[kBf16Chunks], cnt[kBf16Chunks];
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + lane) * 8;
            sbits[j] = sentinel_bits(code[j]);
            if (c >= blen) sbits[j] = 0;
            else if (c + 8 > blen) sbits[j] &= (1u << (4 * (blen - c))) - 1;   // padding nibbles do not count
            cnt[j] = __popc(sbits[j]);
        }
        uint32_t row_base[kBf16Chunks], row_total[kBf16Chunks], lane_before[kBf16Chunks];
        const uint32_t wave_total = wave_chunk_ranks<kBf16Chunks>(cnt, row_base, row_total, lane_before);
        uint32_t block_total;
        const uint32_t wave_before = workgroup_wave_prefix<kDecThreads / 64>(wave_total, wave_totals, block_total);
        bool bad = block_total != k;
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + lane) * 8;
            if (c >= blen) continue;
            uint4 o = decode_chunk_bf16(code[j], sm[j], table);
            uint32_t rank = wave_before + row_base[j] + lane_before[j];
            for (uint32_t m = sbits[j]; m; m &= m - 1, ++rank) {
                uint32_t e = 0;
                if (rank < k) e = esc[r0 + rank];
                else bad = true;
                patch_bf16(o, (uint32_t)__builtin_ctz(m) / 4, e);
            }
            const uint64_t g = e0 + c;
            if (full_row || c + 8 <= blen) {
                store_nt(reinterpret_cast<uint4 *>(out + g), o);
            } else {
                const uint32_t w[4] = {o.x, o.y, o.z, o.w};
                for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
            }
        }
        if (bad) atomicExch(status, SZ_E_FORMAT);
        return;
    }
    // version 2: position records
    if (heavy) {
        const uint32_t *cbw = reinterpret_cast<const uint32_t *>(in + 32);
        const uint32_t cb0 = cbw[0], cb1 = cbw[1];
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + lane) * 8;
            if (c < blen)
                *reinterpret_cast<uint2 *>(plane + c) = make_uint2(perm(cb1, cb0, spread_codes3x4(code[j] & 0xFFFu)),
                                                                   perm(cb1, cb0, spread_codes3x4(code[j] >> 12)));
        }
        __syncthreads();
        overwrite_exponents(esc, r0, k, blen, 256, e_total, plane, status);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kBf16Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + lane) * 8;
            if (c >= blen) continue;
            const uint2 ex = *reinterpret_cast<const uint2 *>(plane + c);
            uint4 o;
            o.x = (perm(sm[j].x, sm[j].x, 0x01010000u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C010C00u) << 7);
            o.y = (perm(sm[j].x, sm[j].x, 0x03030202u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C030C02u) << 7);
            o.z = (perm(sm[j].y, sm[j].y, 0x01010000u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C050C04u) << 7);
            o.w = (perm(sm[j].y, sm[j].y, 0x03030202u) & 0x807F807Fu) | (perm(ex.y, ex.x, 0x0C070C06u) << 7);
            const uint64_t g = e0 + c;
            if (full_row || c + 8 <= blen) {
                store_nt(reinterpret_cast<uint4 *>(out + g), o);
            } else {
                const uint32_t w[4] = {o.x, o.y, o.z, o.w};
                for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
            }
        }
        return;
    }
    if (k) {
        reinterpret_cast<uint4 *>(first)[tid] = make_uint4(~0u, ~0u, ~0u, ~0u);
        load_block_records(esc, r0, k, e_total, rec);
    }
    __syncthreads();
    if (k) map_block_escapes<3>(rec, k, blen, 256, first, status);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kBf16Chunks; ++j) {
        const uint32_t c = rbase + (j * 64 + lane) * 8;
        if (c >= blen) continue;
        uint4 o = decode_chunk_top8(code[j], sm[j], table);
        if (k) {
            uint32_t r = first[c >> 3];
            if (r != kNoEscape) {
                for (; r < k; ++r) {
                    const uint32_t v = rec[r];
                    if (((v & 0xFFFFu) >> 3) != (c >> 3)) break;
                    patch_bf16(o, v & 7, v >> 16);
                }
            }
        }
        const uint64_t g = e0 + c;
        if (full_row || c + 8 <= blen) {
            store_nt(reinterpret_cast<uint4 *>(out + g), o);
        } else {
            const uint32_t w[4] = {o.x, o.y, o.z, o.w};
            for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
        }
    }
}

// FP8 E5M2 decode: a lane decodes two 32-element chunks (16 code bytes + 12
// sign/mantissa bytes -> 32 bytes each).
__device__ __forceinline__ uint32_t unpack_sm3_x4(uint32_t v12)
{
    // 12 bits = four 3-bit symbols -> one symbol per byte
    return (v12 & 0x7u) | ((v12 << 5) & 0x700u) | ((v12 << 10) & 0x70000u) | ((v12 << 15) & 0x7000000u);
}

__device__ __forceinline__ void decode_chunk_e5m2(const uint4 nib, const uint32_t sm3[3],
                                                  const uint16_t *table, uint32_t o[8])
{
    // table[b] = (cb[b & 15] << 2) | (cb[b >> 4] << 10): the exponent fields of
    // the two elements of code byte b, in place inside two E5M2 bytes
    const uint32_t nw[4] = {nib.x, nib.y, nib.z, nib.w};
    const uint32_t grp[4] = {sm3[0] & 0xFFFFFFu, (sm3[0] >> 24) | ((sm3[1] & 0xFFFFu) << 8),
                             (sm3[1] >> 16) | ((sm3[2] & 0xFFu) << 16), sm3[2] >> 8};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t w = nw[s];
        const uint32_t e_lo = (uint32_t)table[w & 0xFFu] | ((uint32_t)table[(w >> 8) & 0xFFu] << 16);
        const uint32_t e_hi = (uint32_t)table[(w >> 16) & 0xFFu] | ((uint32_t)table[w >> 24] << 16);
        const uint32_t t_lo = unpack_sm3_x4(grp[s] & 0xFFFu);
        const uint32_t t_hi = unpack_sm3_x4(grp[s] >> 12);
        o[2 * s] = ((t_lo & 0x04040404u) << 5) | (t_lo & 0x03030303u) | e_lo;
        o[2 * s + 1] = ((t_hi & 0x04040404u) << 5) | (t_hi & 0x03030303u) | e_hi;
    }
}

// E5M2 rows are decoded with lane 2m on chunk m and lane 2m+1 on chunk
// 32 + m of each 64-chunk row, so that after the two lanes swap the half
// (16 bytes) each one does not keep, each of the two stores of a row writes
// 1 KB of contiguous output.
__device__ __forceinline__ uint32_t e5m2_chunk_of_lane(uint32_t lane)
{
    return (lane & 1) ? 32 + (lane >> 1) : (lane >> 1);
}

__device__ __forceinline__ void store_chunk_pairs(uint8_t *row_out, const uint32_t o[8], uint32_t lane)
{
    const bool odd = lane & 1;
    uint32_t keep[4], give[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        keep[i] = odd ? o[4 + i] : o[i];
        give[i] = odd ? o[i] : o[4 + i];
        give[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)give[i], 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    }
    // even lanes: bytes [16l, 16l+16) of the first KB = their own low half;
    // odd lanes: the same range = the partner's high half
    const uint4 first_kb = odd ? make_uint4(give[0], give[1], give[2], give[3])
                               : make_uint4(keep[0], keep[1], keep[2], keep[3]);
    const uint4 second_kb = odd ? make_uint4(keep[0], keep[1], keep[2], keep[3])
                                : make_uint4(give[0], give[1], give[2], give[3]);
    store_nt(reinterpret_cast<uint4 *>(row_out + 16 * lane), first_kb);
    store_nt(reinterpret_cast<uint4 *>(row_out + 1024 + 16 * lane), second_kb);
}

__global__ __launch_bounds__(kDecThreads) void sz_dec_e5m2(const uint8_t *__restrict__ in, DecodeArgs a,
                                                           const uint64_t *__restrict__ block_offsets,
                                                           int32_t *__restrict__ status,
                                                           uint8_t *__restrict__ out)
{
    __shared__ uint16_t table[256];
    __shared__ uint32_t prefix_part[kDecThreads / 64];
    // mapped blocks: first[] (first record of each 32-element chunk, 4 KB) and
    // rec[] (the records, 32 KB); heavy blocks: the exponent plane (64 KB)
    __shared__ __align__(16) uint8_t pool[kBlock];
    uint16_t *first = reinterpret_cast<uint16_t *>(pool);
    uint32_t *rec = reinterpret_cast<uint32_t *>(pool + kBlock / 16);
    uint8_t *plane = pool;
    if (status[1] != 0) return;
    const uint32_t tid = threadIdx.x;
    const uint64_t b = blockIdx.x;
    const uint64_t e0 = b * kBlock;
    const uint32_t blen = (uint32_t)std::min<uint64_t>(kBlock, a.n - e0);
    uint32_t k = reinterpret_cast<const uint32_t *>(in + 64)[b];
    const uint64_t e_total = *reinterpret_cast<const uint64_t *>(in + 16);
    const uint8_t *esc = in + a.off_esc;
    if (tid < 256) {
        const uint32_t lo = in[32 + (tid & 15)];
        const uint32_t hi = in[32 + (tid >> 4)];
        table[tid] = (uint16_t)((lo << 2) | (hi << 10));
    }
    const uint32_t lane = lane_id();
    const uint32_t rbase = (tid / 64) * kRow;
    const bool full_row = rbase + kRow <= blen;
    const uint8_t *nib_base = in + a.off_nib;
    const uint8_t *sm_base = in + a.off_sm;
    const uint64_t sm_end = a.off_sm + 3 * ((a.n + 7) / 8);
    uint4 nib[kE5Chunks];
    uint32_t sm3[kE5Chunks][3];
#pragma unroll
    for (int j = 0; j < kE5Chunks; ++j) {
        const uint32_t c = rbase + (j * 64 + e5m2_chunk_of_lane(lane)) * 32;
        const uint64_t g = e0 + c;
        if (full_row || c + 32 <= blen) {
            nib[j] = load_nt(reinterpret_cast<const uint4 *>(nib_base + g / 2));
            load3_nt(reinterpret_cast<const uint32_t *>(sm_base + (g / 32) * 12), sm3[j]);
        } else if (c < blen) {
            nib[j] = *reinterpret_cast<const uint4 *>(nib_base + g / 2);
            sm3[j][0] = sm3[j][1] = sm3[j][2] = 0;
            const uint64_t start = a.off_sm + (g / 32) * 12;
            for (uint32_t i = 0; i < 12 && start + i < sm_end; ++i)
                sm3[j][i / 4] |= (uint32_t)in[start + i] << (8 * (i & 3));
        } else {
            nib[j] = make_uint4(0, 0, 0, 0);
            sm3[j][0] = sm3[j][1] = sm3[j][2] = 0;
        }
    }
    const uint64_t r0 = block_escape_offset(in, a, b, blen, e_total, block_offsets, k, status, prefix_part);
    const bool heavy = k > kMappedEscapes;                        // workgroup-uniform
    if (heavy) {
        const uint32_t *cbw = reinterpret_cast<const uint32_t *>(in + 32);
        const CodebookRegs cb = {cbw[0], cbw[1], cbw[2], cbw[3]};
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + e5m2_chunk_of_lane(lane)) * 32;
            if (c >= blen) continue;
            const uint32_t nw[4] = {nib[j].x, nib[j].y, nib[j].z, nib[j].w};
#pragma unroll
            for (int s8 = 0; s8 < 4; ++s8) *reinterpret_cast<uint2 *>(plane + c + 8 * s8) = lookup_codes8(nw[s8], cb);
        }
        __syncthreads();
        overwrite_exponents(esc, r0, k, blen, 32, e_total, plane, status);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint32_t c = rbase + (j * 64 + e5m2_chunk_of_lane(lane)) * 32;
            if (c >= blen) continue;
            const uint32_t grp[4] = {sm3[j][0] & 0xFFFFFFu, (sm3[j][0] >> 24) | ((sm3[j][1] & 0xFFFFu) << 8),
                                     (sm3[j][1] >> 16) | ((sm3[j][2] & 0xFFu) << 16), sm3[j][2] >> 8};
            uint32_t o[8];
#pragma unroll
            for (int s8 = 0; s8 < 4; ++s8) {
                const uint2 ex = *reinterpret_cast<const uint2 *>(plane + c + 8 * s8);
                const uint32_t t_lo = unpack_sm3_x4(grp[s8] & 0xFFFu);
                const uint32_t t_hi = unpack_sm3_x4(grp[s8] >> 12);
                o[2 * s8] = ((t_lo & 0x04040404u) << 5) | (t_lo & 0x03030303u) | (ex.x << 2);
                o[2 * s8 + 1] = ((t_hi & 0x04040404u) << 5) | (t_hi & 0x03030303u) | (ex.y << 2);
            }
            const uint64_t g = e0 + c;
            if (full_row) {
                store_chunk_pairs(out + e0 + rbase + j * 2048, o, lane);
            } else if (c + 32 <= blen) {
                store_nt(reinterpret_cast<uint4 *>(out + g), make_uint4(o[0], o[1], o[2], o[3]));
                store_nt(reinterpret_cast<uint4 *>(out + g + 16), make_uint4(o[4], o[5], o[6], o[7]));
            } else {
                for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint8_t)(o[i / 4] >> (8 * (i & 3)));
            }
        }
        return;
    }
    if (k) {
        if (tid < kBlock / 32 / 8) reinterpret_cast<uint4 *>(first)[tid] = make_uint4(~0u, ~0u, ~0u, ~0u);
        load_block_records(esc, r0, k, e_total, rec);
    }
    __syncthreads();
    if (k) map_block_escapes<5>(rec, k, blen, 32, first, status);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kE5Chunks; ++j) {
        const uint32_t c = rbase + (j * 64 + e5m2_chunk_of_lane(lane)) * 32;
        if (c >= blen) continue;
        uint32_t o[8];
        decode_chunk_e5m2(nib[j], sm3[j], table, o);
        if (k) {
            uint32_t r = first[c >> 5];
            if (r != kNoEscape) {
                for (; r < k; ++r) {
                    const uint32_t v = rec[r];
                    const uint32_t pos = v & 0xFFFFu, e = v >> 16;
                    if ((pos >> 5) != (c >> 5)) break;
                    const uint32_t p = pos & 31;
                    const uint32_t sh = 8 * (p & 3) + 2;
                    const uint32_t clear = ~(0x1Fu << sh);
#pragma unroll
                    for (int w = 0; w < 8; ++w)
                        if ((uint32_t)w == (p >> 2)) o[w] = (o[w] & clear) | (e << sh);
                }
            }
        }
        const uint64_t g = e0 + c;
        if (full_row) {
            store_chunk_pairs(out + e0 + rbase + j * 2048, o, lane);
        } else if (c + 32 <= blen) {
            store_nt(reinterpret_cast<uint4 *>(out + g), make_uint4(o[0], o[1], o[2], o[3]));
            store_nt(reinterpret_cast<uint4 *>(out + g + 16), make_uint4(o[4], o[5], o[6], o[7]));
        } else {
            for (uint32_t i = 0; i < blen - c; ++i) out[g + i] = (uint8_t)(o[i / 4] >> (8 * (i & 3)));
        }
    }
}

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

// ---------------------------------------------------------------------------
// Host side: launch bookkeeping and instrumentation
// ---------------------------------------------------------------------------
struct ProfRecord {
    const char *name;
    hipEvent_t start, stop;
};

std::mutex g_prof_mutex;
bool g_prof_on = false;
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

struct LaunchScope {
    const char *name;
    hipStream_t stream;
    hipEvent_t start = nullptr, stop = nullptr;
    LaunchScope(const char *n, hipStream_t s) : name(n), stream(s)
    {
        std::lock_guard<std::mutex> lock(g_prof_mutex);
        if (!g_prof_on) return;
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

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Codebook4 pack_codebook(const uint8_t *e)
{
    Codebook4 cb;
    for (int w = 0; w < 4; ++w)
        cb.w[w] = (uint32_t)e[4 * w] | ((uint32_t)e[4 * w + 1] << 8) | ((uint32_t)e[4 * w + 2] << 16) |
                  ((uint32_t)e[4 * w + 3] << 24);
    return cb;
}

uint32_t symbols_of(int dtype) { return dtype == SZ_BF16 ? 256u : 32u; }

constexpr uint64_t kMaxElems = 1ull << 40;

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
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

extern "C" uint64_t sz_encoded_size(int dtype, uint64_t n_elems, uint64_t n_escapes)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return 0;
    return geometry(dtype, n_elems).off_esc + 3 * n_escapes;
}

extern "C" uint64_t sz_workspace_size(int dtype, uint64_t n_elems)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return 0;
    return ws_layout(dtype, n_elems).total;
}

namespace {

uint64_t encoded_size_v(uint32_t version, int dtype, uint64_t n, uint64_t e)
{
    return geometry(dtype, n, version).off_esc + escape_item_bytes(version) * e;
}

// Encode behind sz_encode (host codebook cb4), sz_encode_devcb (cb_dev) and
// sz_encode_format (version 2, 3).
int encode_impl(uint32_t version, int dtype, const void *d_in, uint64_t n_elems, const Codebook4 &cb4,
                const uint32_t *cb_dev, void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes,
                void *stream)
{
    if (n_elems > kMaxElems) return SZ_E_ARG;
    if (!d_out || !d_ws || (n_elems && !d_in)) return SZ_E_ARG;
    if (!aligned16(d_out) || !aligned16(d_ws) || (n_elems && !aligned16(d_in))) return SZ_E_ALIGN;
    if (out_capacity < encoded_size_v(version, dtype, n_elems, n_elems)) return SZ_E_CAPACITY;
    if (ws_bytes < sz_workspace_size(dtype, n_elems)) return SZ_E_WORKSPACE;
    const Geometry g = geometry(dtype, n_elems, version);
    const WsLayout w = ws_layout(dtype, n_elems);
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    uint8_t *out = static_cast<uint8_t *>(d_out);
    int32_t *status = reinterpret_cast<int32_t *>(ws);
    uint32_t *tile_counts = reinterpret_cast<uint32_t *>(ws + w.counts);
    uint64_t *block_offsets = reinterpret_cast<uint64_t *>(ws + w.offsets);
    uint8_t *stage = ws + w.stage;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (g.nt && dtype == SZ_BF16) {
        const uint16_t *in16 = static_cast<const uint16_t *>(d_in);
        if (version == kTop8) {
            LaunchScope scope("sz_enc_dense_top8", s);
            hipLaunchKernelGGL(sz_enc_dense_bf16<kTop8>, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s, in16, g.n,
                               out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage);
        } else if (version == kTop15S) {
            LaunchScope scope("sz_enc_dense_top15s", s);
            hipLaunchKernelGGL(sz_enc_dense_bf16<kTop15S>, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s, in16,
                               g.n, out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage);
        } else {
            LaunchScope scope("sz_enc_dense_bf16", s);
            hipLaunchKernelGGL(sz_enc_dense_bf16<kTop16>, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s, in16,
                               g.n, out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage);
        }
    } else if (g.nt) {
        LaunchScope scope("sz_enc_dense_e5m2", s);
        hipLaunchKernelGGL(sz_enc_dense_e5m2, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s,
                           static_cast<const uint8_t *>(d_in), g.n, out, g.off_nib, g.off_sm, g.sm_bytes,
                           cb4, cb_dev, tile_counts, stage);
    }
    {
        HeaderArgs h;
        h.n = g.n;
        h.nb = g.nb;
        h.dtype = (uint32_t)dtype;
        h.version = version;
        h.cb = cb4;
        h.pad_start[0] = 64 + 4 * g.nb;
        h.pad_end[0] = g.off_nib;
        h.pad_start[1] = g.off_nib + g.nib_bytes;
        h.pad_end[1] = g.off_sm;
        h.pad_start[2] = g.off_sm + g.sm_bytes;
        h.pad_end[2] = g.off_esc;
        if (g.nt <= kFusedPrefixTiles) {
            // one launch orders the records and writes the header
            const uint32_t groups = (uint32_t)std::max<uint64_t>(1, (g.nb + kFusedBlocks - 1) / kFusedBlocks);
            LaunchScope scope("sz_enc_compact_fused", s);
            if (dtype == SZ_BF16)
                hipLaunchKernelGGL(sz_enc_compact_fused<SZ_BF16>, dim3(groups), dim3(kFusedThreads), 0, s, stage,
                                   tile_counts, out, g.off_esc, g.nt, d_in, h, cb_dev, status,
                                   escape_item_bytes(version));
            else
                hipLaunchKernelGGL(sz_enc_compact_fused<SZ_FP8_E5M2>, dim3(groups), dim3(kFusedThreads), 0, s, stage,
                                   tile_counts, out, g.off_esc, g.nt, d_in, h, cb_dev, status, 3u);
            return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
        }
        LaunchScope scope("sz_enc_scan", s);
        hipLaunchKernelGGL(sz_enc_scan, dim3(1), dim3(kScanThreads), 0, s, tile_counts, (uint32_t)g.nt,
                           block_offsets, out, h, cb_dev, status);
    }
    if (g.nt) {
        LaunchScope scope("sz_enc_compact", s);
        const uint32_t groups = (uint32_t)((g.nb + kCompactThreads / 64 - 1) / (kCompactThreads / 64));
        if (dtype == SZ_BF16)
            hipLaunchKernelGGL(sz_enc_compact<SZ_BF16>, dim3(groups), dim3(kCompactThreads), 0, s, stage, tile_counts,
                               block_offsets, out, g.off_esc, g.nt, g.nb, d_in, g.n, cb4, cb_dev,
                               escape_item_bytes(version));
        else
            hipLaunchKernelGGL(sz_enc_compact<SZ_FP8_E5M2>, dim3(groups), dim3(kCompactThreads), 0, s, stage,
                               tile_counts, block_offsets, out, g.off_esc, g.nt, g.nb, d_in, g.n, cb4, cb_dev, 3u);
    }
    return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
}

}  // namespace

extern "C" int sz_encode(int dtype, const void *d_in, uint64_t n_elems, const sz_codebook *cb, void *d_out,
                         uint64_t out_capacity, void *d_ws, uint64_t ws_bytes, void *stream)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    if (!cb) return SZ_E_ARG;
    if (cb->dtype != (uint32_t)dtype) return SZ_E_DTYPE;
    const uint32_t symbols = symbols_of(dtype);
    for (int c = 0; c < 16; ++c) {
        if (cb->exp[c] >= symbols) return SZ_E_ARG;
        for (int d = 0; d < c; ++d)
            if (cb->exp[d] == cb->exp[c]) return SZ_E_ARG;
    }
    return encode_impl(kTop16, dtype, d_in, n_elems, pack_codebook(cb->exp), nullptr, d_out, out_capacity, d_ws,
                       ws_bytes, stream);
}

extern "C" uint64_t sz_encoded_size_format(int format, int dtype, uint64_t n_elems, uint64_t n_escapes)
{
    if (format == SZ_FORMAT_TOP16) return sz_encoded_size(dtype, n_elems, n_escapes);
    if ((format != SZ_FORMAT_TOP8 && format != SZ_FORMAT_TOP15_SENTINEL) || dtype != SZ_BF16) return 0;
    return encoded_size_v((uint32_t)format, dtype, n_elems, n_escapes);
}

extern "C" int sz_encode_format(int format, int dtype, const void *d_in, uint64_t n_elems, const sz_codebook *cb,
                                void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes, void *stream)
{
    if (format == SZ_FORMAT_TOP16)
        return sz_encode(dtype, d_in, n_elems, cb, d_out, out_capacity, d_ws, ws_bytes, stream);
    if (format != SZ_FORMAT_TOP8 && format != SZ_FORMAT_TOP15_SENTINEL) return SZ_E_ARG;
    if (dtype != SZ_BF16) return SZ_E_DTYPE;
    if (!cb) return SZ_E_ARG;
    if (cb->dtype != (uint32_t)dtype) return SZ_E_DTYPE;
    // only the first 8 (15) entries are used; they must be distinct, and the
    // stream's header carries zeros in the others
    const uint32_t entries = book_entries((uint32_t)format);
    uint8_t used[16] = {0};
    for (uint32_t c = 0; c < entries; ++c) {
        used[c] = cb->exp[c];
        for (uint32_t d = 0; d < c; ++d)
            if (cb->exp[d] == cb->exp[c]) return SZ_E_ARG;
    }
    return encode_impl((uint32_t)format, dtype, d_in, n_elems, pack_codebook(used), nullptr, d_out, out_capacity,
                       d_ws, ws_bytes, stream);
}

extern "C" int sz_encode_devcb(int dtype, const void *d_in, uint64_t n_elems, const sz_codebook *d_cb,
                               void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes, void *stream)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    if (!d_cb) return SZ_E_ARG;
    if (!aligned16(d_cb)) return SZ_E_ALIGN;
    const uint8_t zero[16] = {0};
    return encode_impl(kTop16, dtype, d_in, n_elems, pack_codebook(zero), reinterpret_cast<const uint32_t *>(d_cb),
                       d_out, out_capacity, d_ws, ws_bytes, stream);
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

namespace {

int decode_impl(uint32_t version, const void *d_in, uint64_t in_bytes, int dtype, void *d_out, uint64_t n_elems,
                void *d_ws, uint64_t ws_bytes, void *stream)
{
    if (n_elems > kMaxElems) return SZ_E_ARG;
    if (!d_in || !d_ws || (n_elems && !d_out)) return SZ_E_ARG;
    if (!aligned16(d_in) || !aligned16(d_ws) || (n_elems && !aligned16(d_out))) return SZ_E_ALIGN;
    if (in_bytes < encoded_size_v(version, dtype, n_elems, 0)) return SZ_E_FORMAT;
    if (ws_bytes < sz_workspace_size(dtype, n_elems)) return SZ_E_WORKSPACE;
    const Geometry g = geometry(dtype, n_elems, version);
    const WsLayout w = ws_layout(dtype, n_elems);
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    int32_t *status = reinterpret_cast<int32_t *>(ws);
    uint64_t *block_offsets = reinterpret_cast<uint64_t *>(ws + w.offsets);
    hipStream_t s = static_cast<hipStream_t>(stream);
    DecodeArgs a;
    a.n = g.n;
    a.nb = g.nb;
    a.in_bytes = in_bytes;
    a.off_nib = g.off_nib;
    a.off_sm = g.off_sm;
    a.off_esc = g.off_esc;
    a.dtype = (uint32_t)dtype;
    a.symbols = symbols_of(dtype);
    a.version = version;
    a.item = escape_item_bytes(version);
    a.entries = book_entries(version);
    const uint8_t *in = static_cast<const uint8_t *>(d_in);
    if (g.nb <= kFusedPrefixBlocks) {
        // the decoders sum the counts before their block themselves
        block_offsets = nullptr;
        LaunchScope scope("sz_dec_head", s);
        hipLaunchKernelGGL(sz_dec_head, dim3(1), dim3(64), 0, s, in, a, status);
    } else {
        LaunchScope scope("sz_dec_scan", s);
        hipLaunchKernelGGL(sz_dec_scan, dim3(1), dim3(kScanThreads), 0, s, in, a, block_offsets, status);
    }
    if (g.nb && version == kTop8) {
        LaunchScope scope("sz_dec_top8", s);
        hipLaunchKernelGGL(sz_dec_variant<kTop8>, dim3((uint32_t)g.nb), dim3(kDecThreads), 0, s, in, a,
                           block_offsets, status, static_cast<uint16_t *>(d_out));
    } else if (g.nb && version == kTop15S) {
        LaunchScope scope("sz_dec_top15s", s);
        hipLaunchKernelGGL(sz_dec_variant<kTop15S>, dim3((uint32_t)g.nb), dim3(kDecThreads), 0, s, in, a,
                           block_offsets, status, static_cast<uint16_t *>(d_out));
    } else if (g.nb && dtype == SZ_BF16) {
        LaunchScope scope("sz_dec_bf16", s);
        hipLaunchKernelGGL(sz_dec_bf16, dim3((uint32_t)g.nb), dim3(kDecThreads), 0, s, in, a, block_offsets,
                           status, static_cast<uint16_t *>(d_out));
    } else if (g.nb) {
        LaunchScope scope("sz_dec_e5m2", s);
        hipLaunchKernelGGL(sz_dec_e5m2, dim3((uint32_t)g.nb), dim3(kDecThreads), 0, s, in, a, block_offsets,
                           status, static_cast<uint8_t *>(d_out));
    }
    return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
}

}  // namespace

extern "C" int sz_decode(const void *d_in, uint64_t in_bytes, int dtype, void *d_out, uint64_t n_elems,
                         void *d_ws, uint64_t ws_bytes, void *stream)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return SZ_E_DTYPE;
    return decode_impl(kTop16, d_in, in_bytes, dtype, d_out, n_elems, d_ws, ws_bytes, stream);
}

extern "C" int sz_decode_format(int format, const void *d_in, uint64_t in_bytes, int dtype, void *d_out,
                                uint64_t n_elems, void *d_ws, uint64_t ws_bytes, void *stream)
{
    if (format == SZ_FORMAT_TOP16) return sz_decode(d_in, in_bytes, dtype, d_out, n_elems, d_ws, ws_bytes, stream);
    if (format != SZ_FORMAT_TOP8 && format != SZ_FORMAT_TOP15_SENTINEL) return SZ_E_ARG;
    if (dtype != SZ_BF16) return SZ_E_DTYPE;
    return decode_impl((uint32_t)format, d_in, in_bytes, dtype, d_out, n_elems, d_ws, ws_bytes, stream);
}

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
    g_prof_on = on != 0;
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
