// SplitZip encode for MI355X: the dense kernels (codes, sign/mantissa
// bytes, escape staging), the ordering of the escape records (a scan, one
// workgroup per 8,192 blocks, + compaction, or for small streams one
// compaction launch that finds its own offsets), the stream header, and the
// encode entry points of the
// C ABI ("SplitZip: Ultra Fast Lossless KV Compression for Disaggregated LLM
// Serving", gist.science summary page, Method, encoding bullets).
#include "common.hpp"

namespace sz {
namespace {

// LDS operations of one wave complete in order; this only keeps the compiler
// from moving LDS accesses of the wave across the hand-over point.
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exponent -> code table for encode.  Byte v = code of exponent v, or
// `escape` (the escape flag 0x80 plus the code an escaped element carries)
// when v is not among the first `entries` codebook entries.  Wave 0 builds
// it: its lanes fill the table with `escape`, then lane c < entries stores
// code c at byte cb[c].  Entries at or above `symbols` (possible only in a
// device codebook, whose stream the header check then invalidates) store
// nothing.  The caller synchronises the workgroup before the table is read.
__device__ __forceinline__ void build_encode_table(uint32_t *table32, const Codebook4 &cb,
                                                   uint32_t symbols, uint32_t entries = 16,
                                                   uint32_t escape = 0x80u)
{
    const uint32_t t = threadIdx.x;
    if (t < 64) {
        if (t * 4 < symbols) table32[t] = escape * 0x01010101u;
        wave_lds_fence();
        const uint32_t v = cb_entry_lane(cb, t & 15u);
        if (t < entries && v < symbols) reinterpret_cast<uint8_t *>(table32)[v] = (uint8_t)t;
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

// E5M2 encode through a code-pair table.  Two neighbouring input bytes
// w = b0 | b1 << 8 (elements 0 and 1 of a pair) are looked up at the LDS byte
// address (w >> 1) & kPairMask: exponent e0 in address bits 1-5, the sign of
// element 0 in bit 6, e1 in bits 9-13.  The sign does not change the entry;
// it is kept in the address because it falls in the bank bits, where it
// spreads a wave's reads over twice as many banks as e0 alone.  Entry (16
// bits): low byte = code0 | code1 << 4 (escapes coded 0), high byte = escape
// flags (bit 0 = element 0, bit 1 = element 1).  One LDS read per two
// elements, and the address takes two VALU operations per input word (a
// shift shared by the word's two pairs, one mask each).
constexpr uint32_t kPairMask = 0x3E7Eu;
constexpr uint32_t kPairTableBytes = kPairMask + 2;

// Address of the pair in bits 16..31 of x (already shifted right by one):
// one SDWA AND that reads the upper half-word of x.
__device__ __forceinline__ uint32_t pair_addr_hi(uint32_t x, uint32_t mask)
{
    uint32_t r;
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
        : "=v"(r)
        : "v"(x), "v"(mask));
    return r;
}

// Builds the pair table from the byte table tab8 (build_encode_table, 32
// symbols).  Row (s0, e1) holds the 32 entries of e0 = 0..31 at byte
// s0 << 6 | e1 << 9; thread t < 256 writes entries 8q .. 8q+7 (q = t & 3) of
// row t >> 2 as one 16-byte store.
__device__ __forceinline__ void build_pair_table(uint32_t *pair32, const uint32_t *table32)
{
    const uint32_t t = threadIdx.x;
    if (t < 256) {
        const uint32_t row = t >> 2, q = t & 3u;
        const uint32_t e1 = row >> 1;
        const uint32_t c1 = (table32[e1 >> 2] >> (8 * (e1 & 3u))) & 0xFFu;
        const uint32_t hi = (((c1 & 0xFu) << 4) | ((c1 >> 7) << 9)) * 0x00010001u;
        uint32_t e[4];
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t w = table32[2 * q + h];                  // codes of e0 = 8q + 4h .. 8q + 4h + 3
            const uint32_t nib = w & 0x0F0F0F0Fu, flg = (w >> 7) & 0x01010101u;
            e[2 * h] = perm(flg, nib, 0x05010400u) | hi;            // entries of e0 = 8q + 4h, +1
            e[2 * h + 1] = perm(flg, nib, 0x07030602u) | hi;        // entries of +2, +3
        }
        const uint32_t addr = ((row & 1u) << 6) | (e1 << 9) | (q << 4);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(pair32) + addr) = make_uint4(e[0], e[1], e[2], e[3]);
    }
}

// One 32-element chunk: 16 code bytes, 12 sign/mantissa bytes, and the
// chunk's escape flags in one word F: bit 8k + 2s + h is element 8s + 2k + h
// (s = group of 8 elements, k = pair in the group, h = element of the pair).
__device__ __forceinline__ void encode_chunk_e5m2_pairs(const uint4 q0, const uint4 q1, const uint8_t *pairs,
                                                        uint32_t mask, uint4 &nib, uint32_t sm3[3], uint32_t &F)
{
    const uint32_t d[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    uint32_t nibw[4], grp[4];
    F = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t a = d[2 * s], b = d[2 * s + 1];
        const uint32_t a1 = a >> 1, b1 = b >> 1;
        const uint32_t p0 = *reinterpret_cast<const uint16_t *>(pairs + (a1 & kPairMask));
        const uint32_t p1 = *reinterpret_cast<const uint16_t *>(pairs + pair_addr_hi(a1, mask));
        const uint32_t p2 = *reinterpret_cast<const uint16_t *>(pairs + (b1 & kPairMask));
        const uint32_t p3 = *reinterpret_cast<const uint16_t *>(pairs + pair_addr_hi(b1, mask));
        const uint32_t lo = perm(p1, p0, 0x05040100u), hi = perm(p3, p2, 0x05040100u);   // p0 | p1 << 16, p2 | p3 << 16
        nibw[s] = perm(hi, lo, 0x06040200u);
        F |= perm(hi, lo, 0x07050301u) << (2 * s);
        const uint32_t s_a = ((a >> 5) & 0x04040404u) | (a & 0x03030303u);
        const uint32_t s_b = ((b >> 5) & 0x04040404u) | (b & 0x03030303u);
        grp[s] = pack_sym3x4(s_a) | (pack_sym3x4(s_b) << 12);
    }
    nib = make_uint4(nibw[0], nibw[1], nibw[2], nibw[3]);
    sm3[0] = grp[0] | (grp[1] << 24);
    sm3[1] = (grp[1] >> 8) | (grp[2] << 16);
    sm3[2] = (grp[2] >> 16) | (grp[3] << 8);
}

// Element index (0..31) of flag bit p of a chunk's flag word F.
__device__ __forceinline__ uint32_t flag_element(uint32_t p)
{
    return ((p << 2) & 0x18u) | ((p >> 2) & 0x6u) | (p & 1u);
}

// Flag word -> escape mask in element order (bit i = element i).  F holds
// 2-bit cells: cell (k, s) at bit 8k + 2s; the mask wants cell (s, k) at
// 8s + 2k.  A 4 x 4 transpose of the cells in two delta swaps: the off-
// diagonal 2 x 2 blocks (distance 12), then the off-diagonal cells inside
// each block (distance 6).
__device__ __forceinline__ uint32_t flags_to_elements(uint32_t F)
{
    uint32_t t = ((F >> 12) ^ F) & 0x0000F0F0u;
    F ^= t ^ (t << 12);
    t = ((F >> 6) ^ F) & 0x00CC00CCu;
    return F ^ t ^ (t << 6);
}

// Flag-word bits of the first v elements of a chunk (v in 0..32).
__device__ __forceinline__ uint32_t chunk_flag_keep(uint32_t v)
{
    uint32_t m = 0;
    for (uint32_t p = 0; p < 32; ++p)
        if (flag_element(p) < v) m |= 1u << p;
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
// segments (possibly of another wave) share, are written byte by byte.  A
// BF16 row with at most 512 records goes through the buffer as one segment
// (one copy: fewer stream lines written in parts by two copies, 2.4 % off
// the dense encode of 1.9 %-escape BF16); a row with at most kDirectRecords
// records skips the buffer.
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
// Tiles above the re-derive limit (kRederiveRecords, or none: kStageAll)
// stage nothing; their tile count carries kRederiveFlag.
constexpr uint32_t kStageAll = 0xFFFFFFFFu;
constexpr uint32_t kRederiveFlag = 0x80000000u;

// ---------------------------------------------------------------------------
// Kernel: BF16 dense encode + escape staging.  One workgroup per 16K-element
// tile; a lane holds C 8-element chunks of its wave's row of 512 C elements
// (C = 8: 256 lanes, wave w streams elements [4096w, 4096w + 4096); small
// streams use C = 2, 1024 lanes, so that each lane's serial work is a
// quarter and a tile's loads go out from four times the lanes).  The
// tile's records are staged in element order in the tile's slot (3 bytes per
// element); tile_counts[tile] gets their number.  A tile with more than
// `rederive_above` escapes stages nothing and is flagged with kRederiveFlag:
// the compaction kernel derives its records again from the input, which
// costs less traffic than writing and re-reading them.
// ---------------------------------------------------------------------------

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

template <int V, int C = kBf16Chunks>
__global__ __launch_bounds__(kEncTile / (8 * C)) void sz_enc_dense_bf16(const uint16_t *__restrict__ in, uint64_t n,
                                                              uint8_t *__restrict__ out, uint64_t off_nib,
                                                              uint64_t off_sm, Codebook4 cb,
                                                              const uint32_t *__restrict__ cb_dev,
                                                              uint32_t *__restrict__ tile_counts,
                                                              uint8_t *__restrict__ stage, uint32_t slot,
                                                              uint32_t rederive_above)
{
    // C chunks of 8 elements per lane: a wave row is 512 C elements, a tile
    // 16384 / (512 C) waves
    constexpr uint32_t kWaves = kEncTile / (512 * C);
    constexpr uint32_t kRowLen = 512 * C;
    static_assert(V != kTop8 || C == kBf16Chunks, "the Top-8 code rows are laid out for eight chunks");
    __shared__ uint32_t table32[64];
    __shared__ uint32_t wave_totals[kWaves];
    __shared__ __align__(16) uint8_t seg_buf[kWaves][kSegBytes];
    // exponents of chunks that hold escapes, parked until the ranks are known
    __shared__ uint64_t ex_park[kWaves][C][64];
    const uint32_t lane = lane_id();
    const uint32_t wave = threadIdx.x / 64;
    const uint64_t tile = blockIdx.x;
    const uint64_t base = tile * kEncTile + (uint64_t)wave * kRowLen;
    const bool full_row = base + kRowLen <= n;

    // the row's loads are issued first and stay in flight while the table is built
    uint4 q[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
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
    uint32_t esc[C];
    uint32_t cnt[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
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
    uint32_t row_base[C], row_total[C], lane_before[C];
    const uint32_t wave_total = wave_chunk_ranks<C>(cnt, row_base, row_total, lane_before);
    uint32_t tile_total;
    const uint32_t wave_before = workgroup_wave_prefix<kWaves>(wave_total, wave_totals, tile_total);
    // only the Top-16 format re-derives escape-heavy tiles in the compaction
    const bool rederive = V == kTop16 && tile_total > rederive_above;
    constexpr uint32_t kItem = escape_item_bytes(V);
    if (wave_total > kDirectRecords && kItem * wave_total + 3 <= kSegBytes && !rederive) {
        // the row's records gathered in the wave's LDS buffer (at most 512:
        // the alignment shift of up to 3 bytes fits), one flush
        uint8_t *tstage = stage + tile * slot;
        const uint32_t g0 = kItem * wave_before;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            if (esc[j]) {
                const uint32_t pos0 = (uint32_t)((base + (uint64_t)(j * 64 + lane) * 8) & 0xFFFFu);
                const uint32_t at = (g0 & 3) + kItem * (row_base[j] + lane_before[j]);
                if (V == kTop15S) lds_put_exponents(buf, at, esc[j], ex_park[wave][j][lane]);
                else lds_put_records(buf, at, esc[j], ex_park[wave][j][lane], pos0);
            }
        }
        wave_lds_fence();
        flush_segment(buf, tstage, g0, kItem * wave_total);
        wave_lds_fence();
    } else if (wave_total && !rederive) {
        uint8_t *tstage = stage + tile * slot;
#pragma unroll
        for (int j = 0; j < C; ++j) {
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

// Writes the records of one E5M2 chunk (escape mask m in element order, the
// chunk's 32 input bytes in dw, block-local position pos0 of element 0) to
// rec, ascending.  Each exponent is picked from the group of 8 input bytes
// that holds it.  rec is LDS or global memory (the caller's pointer decides).
__device__ __forceinline__ void put_chunk_records_e5m2(uint8_t *rec, uint32_t m, const uint32_t (&dw)[8],
                                                       uint32_t pos0)
{
    while (m) {
        const uint32_t k = (uint32_t)__builtin_ctz(m);
        m &= m - 1;
        const uint32_t g = k >> 3;
        const uint32_t lo = g == 0 ? dw[0] : g == 1 ? dw[2] : g == 2 ? dw[4] : dw[6];
        const uint32_t hi = g == 0 ? dw[1] : g == 1 ? dw[3] : g == 2 ? dw[5] : dw[7];
        const uint32_t pos = pos0 + k;
        rec[0] = (uint8_t)pos;
        rec[1] = (uint8_t)(pos >> 8);
        rec[2] = (uint8_t)((perm(hi, lo, k & 7u) >> 2) & 0x1Fu);
        rec += 3;
    }
}

// Stores the first `bytes` bytes of an LDS tile buffer to a tile's staging
// slot as whole dwords (the slot starts on a dword boundary; up to three
// bytes past the records are written, inside the slot).  All threads of the
// workgroup take part.
template <uint32_t THREADS>
__device__ __forceinline__ void store_tile_buffer(const uint8_t *tile_buf, uint8_t *tstage, uint32_t bytes)
{
    const uint32_t words = (bytes + 3) / 4;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(tile_buf);
    uint32_t *dst = reinterpret_cast<uint32_t *>(tstage);
    for (uint32_t i = threadIdx.x; i < words; i += THREADS) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// Kernel: FP8 E5M2 dense encode + escape staging (the page's FP8 extension,
// Contributions item 4).  Same tiling as BF16; a lane holds two 32-element
// chunks of its wave's row.  In a chunk row with few escapes each lane walks
// its chunk's escape mask and writes the records itself, taking each
// exponent from its 8-byte input group with one v_perm; a row with many is
// staged through LDS as four segments of 16 lanes.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kEncThreads) void sz_enc_dense_e5m2(const uint8_t *__restrict__ in, uint64_t n,
                                                              uint8_t *__restrict__ out, uint64_t off_nib,
                                                              uint64_t off_sm, uint64_t sm_bytes,
                                                              Codebook4 cb,
                                                              const uint32_t *__restrict__ cb_dev,
                                                              uint32_t *__restrict__ tile_counts,
                                                              uint8_t *__restrict__ stage, uint32_t slot,
                                                              uint32_t rederive_above)
{
    __shared__ uint32_t table32[8];
    __shared__ __align__(16) uint32_t pair32[kPairTableBytes / 4];
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
    build_pair_table(pair32, table32);
    __syncthreads();
    const uint8_t *pairs = reinterpret_cast<const uint8_t *>(pair32);
    const uint32_t pair_mask = kPairMask;
    uint32_t F[kE5Chunks];
    uint32_t cnt[kE5Chunks];
#pragma unroll
    for (int j = 0; j < kE5Chunks; ++j) {
        const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
        uint4 nib;
        uint32_t sm3[3];
        encode_chunk_e5m2_pairs(q[j][0], q[j][1], pairs, pair_mask, nib, sm3, F[j]);
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
            }
            F[j] &= chunk_flag_keep(valid);
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
            F[j] = 0;
        }
        cnt[j] = __popc(F[j]);
    }
    uint32_t row_base[kE5Chunks], row_total[kE5Chunks], lane_before[kE5Chunks];
    const uint32_t wave_total = wave_chunk_ranks<kE5Chunks>(cnt, row_base, row_total, lane_before);
    uint32_t tile_total;
    const uint32_t wave_before = workgroup_wave_prefix<kEncThreads / 64>(wave_total, wave_totals, tile_total);
    // The records of a tile that fit the LDS tile buffer (all of seg_buf) are
    // gathered there at their rank in the tile and leave as whole dwords
    // after one more barrier (fewer, wider stores than a record at a time);
    // otherwise rows with few records write them straight to the staging slot
    // and rows with many go through the wave's LDS segment buffer.
    constexpr uint32_t kTileBufRecords = (kEncThreads / 64) * kSegBytes / 3;
    const bool to_tile_buf = tile_total <= kTileBufRecords;           // workgroup-uniform
    uint8_t *tile_buf = &seg_buf[0][0];
    if (wave_total && tile_total <= rederive_above) {
        uint8_t *tstage = stage + tile * slot;
        uint8_t *buf = seg_buf[wave];
#pragma unroll
        for (int j = 0; j < kE5Chunks; ++j) {
            const uint64_t c0 = base + (uint64_t)(j * 64 + lane) * 32;
            const uint32_t rank = wave_before + row_base[j];
            const uint32_t dw[8] = {q[j][0].x, q[j][0].y, q[j][0].z, q[j][0].w,
                                    q[j][1].x, q[j][1].y, q[j][1].z, q[j][1].w};
            const uint32_t pos0 = (uint32_t)(c0 & 0xFFFFu);
            if (to_tile_buf) {
                if (cnt[j])
                    put_chunk_records_e5m2(tile_buf + 3 * (rank + lane_before[j]), flags_to_elements(F[j]), dw, pos0);
                continue;
            }
            if (row_total[j] <= kDirectRecords) {                      // wave-uniform
                if (cnt[j])
                    put_chunk_records_e5m2(tstage + 3ull * (rank + lane_before[j]), flags_to_elements(F[j]), dw, pos0);
                continue;
            }
            uint32_t esc8[4];
            uint64_t ex[4];
            const uint32_t m32 = flags_to_elements(F[j]);
#pragma unroll
            for (int s8 = 0; s8 < 4; ++s8) {
                esc8[s8] = (m32 >> (8 * s8)) & 0xFFu;
                ex[s8] = (uint64_t)((dw[2 * s8] >> 2) & 0x1F1F1F1Fu) |
                         ((uint64_t)((dw[2 * s8 + 1] >> 2) & 0x1F1F1F1Fu) << 32);
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
    if (tile_total && tile_total <= rederive_above && to_tile_buf) {   // workgroup-uniform
        __syncthreads();
        store_tile_buffer<kEncThreads>(tile_buf, stage + tile * slot, 3 * tile_total);
    }
    if (threadIdx.x == 0) tile_counts[tile] = tile_total | (tile_total > rederive_above ? kRederiveFlag : 0u);
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

// The escape count of block b: its four tile counts, without the re-derive
// flags and without tiles past nt.
__device__ __forceinline__ uint32_t block_escapes(uint4 v, uint32_t b, uint32_t nt)
{
    const uint32_t t = kTilesPerBlock * b;
    const uint32_t m = ~kRederiveFlag;
    return (v.x & m) + ((t + 1 < nt) ? v.y & m : 0) + ((t + 2 < nt) ? v.z & m : 0) + ((t + 3 < nt) ? v.w & m : 0);
}

// Nonzero when a tile of block b (below nt) carries kRederiveFlag.
__device__ __forceinline__ uint32_t block_flags(uint4 v, uint32_t b, uint32_t nt)
{
    const uint32_t t = kTilesPerBlock * b;
    const uint32_t f = v.x | ((t + 1 < nt) ? v.y : 0) | ((t + 2 < nt) ? v.z : 0) | ((t + 3 < nt) ? v.w : 0);
    return f & kRederiveFlag;
}

// Sum of a 64-bit value over the workgroup (kScanThreads lanes); every
// thread gets it.
__device__ __forceinline__ uint64_t workgroup_sum_u64(uint64_t v, uint64_t *lds)
{
    const uint32_t lane = lane_id(), wave = threadIdx.x / 64;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, d), hi = __shfl_xor((uint32_t)(v >> 32), d);
        v += ((uint64_t)hi << 32) | lo;
    }
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    uint64_t sum = 0;
    for (uint32_t w = 0; w < kScanWaves; ++w) sum += lds[w];
    __syncthreads();
    return sum;
}

// ---------------------------------------------------------------------------
// Kernel: escape totals of the scan's workgroups, for streams of more than
// kScanSuper blocks.  Workgroup g sums the tile counts of blocks
// [g kScanSuper, (g + 1) kScanSuper) into totals[g].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void sz_enc_scan_reduce(const uint32_t *__restrict__ tile_counts,
                                                                   uint32_t nt, uint32_t nb,
                                                                   uint64_t *__restrict__ totals)
{
    __shared__ uint64_t lds[kScanWaves];
    const uint32_t b0 = blockIdx.x * (uint32_t)kScanSuper;
    uint4 v[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) {
        const uint32_t b = b0 + i * kScanThreads + threadIdx.x;
        v[i] = b < nb ? *reinterpret_cast<const uint4 *>(tile_counts + kTilesPerBlock * b) : make_uint4(0, 0, 0, 0);
    }
    uint64_t sum = 0;
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) sum += block_escapes(v[i], b0 + i * kScanThreads + threadIdx.x, nt);
    sum = workgroup_sum_u64(sum, lds);
    if (threadIdx.x == 0) totals[blockIdx.x] = sum;
}

// ---------------------------------------------------------------------------
// Kernel: encode scan.  Workgroup g turns the tile escape counts of blocks
// [g kScanSuper, (g + 1) kScanSuper) into the per-block escape counts of the
// stream and the exclusive escape offset of every block, starting from the
// escapes of the blocks before it (the sum of totals[0 .. g), from
// sz_enc_scan_reduce; one workgroup when the stream has at most kScanSuper
// blocks), and whether one of those tiles is flagged (one word per wave,
// flagged[g kScanWaves + w]).  Workgroup 0 writes the header and the zero padding between sections, the
// last workgroup E.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void sz_enc_scan(const uint32_t *__restrict__ tile_counts,
                                                            uint32_t nt,
                                                            uint64_t *__restrict__ block_offsets,
                                                            uint8_t *__restrict__ out, HeaderArgs h,
                                                            const uint32_t *__restrict__ cb_dev,
                                                            int32_t *__restrict__ status,
                                                            const uint64_t *__restrict__ totals,
                                                            uint32_t *__restrict__ flagged)
{
    __shared__ ScanLds lds;
    __shared__ uint64_t sum_lds[kScanWaves];
    const uint32_t tid = threadIdx.x;
    // a bad device codebook zeroes the magic and sets the status word
    Codebook4 cb = h.cb;
    const int32_t verdict = device_codebook_verdict(cb_dev, h.dtype, cb);
    const uint32_t nb = (uint32_t)h.nb;
    // this workgroup's blocks, and the escapes of the blocks before them
    const uint32_t first = blockIdx.x * (uint32_t)kScanSuper;
    const uint32_t last = (uint32_t)std::min<uint64_t>(nb, (uint64_t)first + kScanSuper);
    uint64_t before = 0;
    for (uint32_t w = tid; w < blockIdx.x; w += kScanThreads) before += totals[w];
    if (gridDim.x > 1) before = workgroup_sum_u64(before, sum_lds);
    if (tid == 0) lds.carry = before;
    uint32_t *block_counts = reinterpret_cast<uint32_t *>(out + 64);
    // the tile counts of block b (four per block, the last block's past nt
    // read as 0); the next batch's loads are issued before this batch's scan
    auto load_batch = [&](uint32_t b0, uint4 (&v)[kScanBatch]) {
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const uint32_t b = b0 + i * kScanThreads + tid;
            v[i] = b < last ? *reinterpret_cast<const uint4 *>(tile_counts + kTilesPerBlock * b) : make_uint4(0, 0, 0, 0);
        }
    };
    uint4 v_next[kScanBatch];
    uint32_t any_flagged = 0;
    load_batch(first, v_next);
    for (uint32_t b0 = first; b0 < last; b0 += kScanBatch * kScanThreads) {
        uint4 v[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) v[i] = v_next[i];
        if (b0 + kScanBatch * kScanThreads < last) load_batch(b0 + kScanBatch * kScanThreads, v_next);
        uint32_t x[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            x[i] = block_escapes(v[i], b0 + i * kScanThreads + tid, nt);
            any_flagged |= block_flags(v[i], b0 + i * kScanThreads + tid, nt);
        }
        uint64_t base[kScanBatch];
        scan_batch(x, base, lds);
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const uint32_t b = b0 + i * kScanThreads + tid;
            if (b < last) {
                block_counts[b] = x[i];
                block_offsets[b] = base[i];
            }
        }
    }
    const uint64_t total = lds.carry;
    // whether a tile of this wave's blocks is flagged, one word per wave (the
    // compaction skips the re-derivation when none of the words is set)
    any_flagged = __any(any_flagged);
    if (lane_id() == 0) flagged[blockIdx.x * kScanWaves + tid / 64] = any_flagged ? 1u : 0u;
    if (blockIdx.x == 0) write_header(out, h, cb, verdict, false, status);
    if (tid == 0 && blockIdx.x == gridDim.x - 1) {
        reinterpret_cast<uint32_t *>(out)[4] = (uint32_t)total;
        reinterpret_cast<uint32_t *>(out)[5] = (uint32_t)(total >> 32);
    }
}

// ---------------------------------------------------------------------------
// Escape compaction: staged records (3 bytes each) are copied to
// out[off_esc + 3 * offset ...), one wave per block, tile after tile; when no
// tile of the block holds more than kGroupCopyRecords records, four 16-lane
// groups copy the four tiles at once.  The body of each copy is written with
// 16-byte aligned dwordx4 stores assembled by v_alignbyte_b32 from five staged
// words; the unaligned bytes at both ends, whose dwords the neighbouring tiles
// share, are written byte by byte.  Flagged (escape-heavy) tiles are derived
// again from the input instead and their records written straight to their
// final place.
// ---------------------------------------------------------------------------
// Copies len bytes of staged records to out[dst0, dst0 + len) with the lanes
// [0, width) of a lane group (lane = index inside the group; width >= 8).
__device__ __forceinline__ void copy_records(const uint8_t *__restrict__ src, uint8_t *__restrict__ out,
                                             uint64_t dst0, uint32_t len, uint32_t lane, uint32_t width)
{
    const uint64_t end = dst0 + len;
    const uint64_t body_begin = std::min<uint64_t>((dst0 + 15) & ~uint64_t(15), end);
    const uint64_t body_end = std::max<uint64_t>(end & ~uint64_t(15), body_begin);
    const uint32_t head = (uint32_t)(body_begin - dst0);                  // < 16 <= 2 width
    const uint32_t tail_src = (uint32_t)(body_end - dst0);
    const uint32_t tail = (uint32_t)(end - body_end);                     // < 16
    const uint32_t *src32 = reinterpret_cast<const uint32_t *>(src);
    const uint32_t chunks = (uint32_t)((body_end - body_begin) / 16);
    const uint32_t sh = head & 3;
    auto chunk = [&](uint32_t c) {
        const uint32_t w0 = (head >> 2) + 4 * c;                 // first source word
        const uint32_t a0 = src32[w0], a1 = src32[w0 + 1], a2 = src32[w0 + 2], a3 = src32[w0 + 3],
                       a4 = src32[w0 + 4];
        return make_uint4(__builtin_amdgcn_alignbyte(a1, a0, sh), __builtin_amdgcn_alignbyte(a2, a1, sh),
                          __builtin_amdgcn_alignbyte(a3, a2, sh), __builtin_amdgcn_alignbyte(a4, a3, sh));
    };
    // the loads of the head bytes, the tail bytes (two of each per lane when
    // the group is 8 lanes wide) and the first body chunk of each lane go out
    // before any store: one memory latency for a short tile
    const uint32_t lane2 = lane + width;
    const uint8_t hb = lane < head ? src[lane] : 0;
    const uint8_t hb2 = lane2 < head ? src[lane2] : 0;
    const uint8_t tb = lane < tail ? src[tail_src + lane] : 0;
    const uint8_t tb2 = lane2 < tail ? src[tail_src + lane2] : 0;
    const uint4 v0 = lane < chunks ? chunk(lane) : make_uint4(0, 0, 0, 0);
    if (lane < head) out[dst0 + lane] = hb;
    if (lane2 < head) out[dst0 + lane2] = hb2;
    if (lane < tail) out[body_end + lane] = tb;
    if (lane2 < tail) out[body_end + lane2] = tb2;
    if (lane < chunks) *reinterpret_cast<uint4 *>(out + body_begin + 16ull * lane) = v0;
#pragma unroll 4
    for (uint32_t c = lane + width; c < chunks; c += width)
        *reinterpret_cast<uint4 *>(out + body_begin + 16ull * c) = chunk(c);
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

// ---------------------------------------------------------------------------
// Escape-heavy tiles of large streams (sz_enc_compact below): the records of
// a tile are derived again from the input and written to their final place
// two chunk rows (1024 elements) at a time, in three steps:
//   * each lane turns an 8-element chunk into the compacted byte string of
//     its records in registers: a 256-entry table gives, for the chunk's
//     escape mask, the element index of each record slot, and v_perm picks
//     the position and exponent bytes by those indices;
//   * the lane ORs the string, shifted to its byte offset (one v_perm per
//     dword), into the wave's LDS segment as whole dwords (the segment's
//     words are zero: the writer clears what it has read; two lanes can
//     share a dword at their edge, and OR keeps both);
//   * the wave stores the segment's whole kLineBytes lines with dwordx4 stores
//     (whole, aligned lines of the stream: no line is written in parts by
//     two stores) and carries the last, partial line over to the next two
//     rows, so only the first and last words of the wave's records take
//     byte stores.
// ---------------------------------------------------------------------------
// The stream lines that the record writer stores whole (bytes, 16-byte words).
constexpr uint32_t kLineBytes = 128;
constexpr uint32_t kLineWords = kLineBytes / 16;
// records of two chunk rows, the lead (up to a line) and the overhang of the
// last lane's dword writes, in 16-byte words
constexpr uint32_t kRdSegWords = (3 * 2 * 512 + kLineBytes + 64) / 16;

struct RederiveLds {
    uint32_t table32[64];      // exponent -> code byte, bit 7 = escape
    uint32_t esc32[64];        // exponent -> 1 if it escapes, else 0 (one byte each)
    uint32_t slots[256];       // escape mask -> element index of record slot j in nibble j (12: unused slot)
    uint4 seg[kRdSegWords];
};

// The encode table and the slot table of one wave, and its zeroed record
// segment (its lanes only, no workgroup barrier).
__device__ __forceinline__ void build_wave_tables(RederiveLds &L, const Codebook4 &cb, uint32_t symbols)
{
    const uint32_t lane = lane_id();
    uint32_t word = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        const uint32_t v = lane * 4 + k;
        uint32_t code = 0x80u;
#pragma unroll
        for (uint32_t c = 0; c < 16; ++c)
            if (cb_entry(cb, c) == v) code = c;
        word |= (v < symbols ? code : 0x80u) << (8 * k);
    }
    L.table32[lane] = word;
    L.esc32[lane] = (word >> 7) & 0x01010101u;
#pragma unroll
    for (uint32_t r = 0; r < 4; ++r) {
        const uint32_t m = lane * 4 + r;
        uint32_t e = 0xCCCCCCCCu, j = 0;
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            if ((m >> k) & 1u) {
                e = (e & ~(0xFu << (4 * j))) | (k << (4 * j));
                ++j;
            }
        }
        L.slots[m] = e;
    }
    // the record segment starts zeroed (the BF16 record writer keeps it so)
    for (uint32_t i = lane; i < kRdSegWords; i += 64) L.seg[i] = make_uint4(0, 0, 0, 0);
    wave_lds_fence();
}

// ORs the records of one 8-element chunk (escape mask m, exponents of
// elements 0..3 in ea and 4..7 in eb, block-local position pos0 of element
// 0, a multiple of 8) into seg32 from byte S on.  Record slot j holds
// (pos lo, pos hi, exponent) of the chunk's j-th escaped element.
__device__ __forceinline__ void or_records8(uint32_t *seg32, uint32_t S, uint32_t m, uint32_t ea, uint32_t eb,
                                            uint32_t pos0, const uint32_t *slots)
{
    const uint32_t sl = slots[m];
    const uint32_t ev = sl & 0x0F0F0F0Fu, od = (sl >> 4) & 0x0F0F0F0Fu;
    const uint32_t k_lo = perm(od, ev, 0x05010400u);              // slot indices 0..3, one per byte
    const uint32_t k_hi = perm(od, ev, 0x07030602u);              // slot indices 4..7
    const uint32_t pl = perm(pos0, pos0, 0x00000000u);            // low position byte in every byte
    const uint32_t posb_lo = pl | 0x03020100u, posb_hi = pl | 0x07060504u;
    const uint32_t hw = perm(pos0, pos0, 0x01010101u);            // high position byte in every byte
    // index 12 selects a zero byte: unused slots come out as zero bytes
    const uint32_t p_lo = perm(posb_hi, posb_lo, k_lo), p_hi = perm(posb_hi, posb_lo, k_hi);
    const uint32_t e_lo = perm(eb, ea, k_lo), e_hi = perm(eb, ea, k_hi);
    const uint32_t h_lo = perm(hw, hw, k_lo), h_hi = perm(hw, hw, k_hi);
    uint32_t d[8];
    {
        const uint32_t ph01 = perm(h_lo, p_lo, 0x05010400u);      // P0 H0 P1 H1
        const uint32_t ph23 = perm(h_lo, p_lo, 0x07030602u);      // P2 H2 P3 H3
        d[1] = perm(e_lo, ph01, 0x02040100u);                       // P0 H0 E0 P1
        const uint32_t x = perm(e_lo, ph01, 0x0C0C0503u);          // H1 E1
        d[2] = perm(ph23, x, 0x05040100u);                          // H1 E1 P2 H2
        d[3] = perm(e_lo, ph23, 0x07030206u);                       // E2 P3 H3 E3
    }
    {
        const uint32_t ph01 = perm(h_hi, p_hi, 0x05010400u);
        const uint32_t ph23 = perm(h_hi, p_hi, 0x07030602u);
        d[4] = perm(e_hi, ph01, 0x02040100u);
        const uint32_t x = perm(e_hi, ph01, 0x0C0C0503u);
        d[5] = perm(ph23, x, 0x05040100u);
        d[6] = perm(e_hi, ph23, 0x07030206u);
    }
    d[0] = 0;
    d[7] = 0;
    const uint32_t dw = S >> 2;
    // LDS word dw + i takes bytes 4 - (S & 3) .. 7 - (S & 3) of {d[i + 1], d[i]}
    const uint32_t sel = 0x03020100u + (4u - (S & 3u)) * 0x01010101u;
    // the string's bytes past its records are zero, so all seven words are
    // ORed: the ones past the records change nothing
#pragma unroll
    for (uint32_t i = 0; i < 7; ++i)
        __hip_atomic_fetch_or(seg32 + dw + i, perm(d[i + 1], d[i], sel), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// Buffer-resource word 3 for untyped (raw) buffer access on this part: the
// hardware drops every store whose offset lies at or past the resource's byte
// count, so a store instruction that all lanes execute can still write only
// some of them, with no branch.
constexpr int32_t kRawBufferWord3 = 0x00020000;
constexpr uint32_t kDroppedOffset = 0x80000000u;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Where byte lane `lane` of store_span stores for the range [from, to) of a
// segment: lanes 0..15 the bytes of the word that holds `from` (when `from`
// is not word-aligned), lanes 16..31 those of the word that holds `to` (when
// `to` is not word-aligned and that word is another one); 0 (and `keep`
// false) for the other lanes.
__device__ __forceinline__ uint32_t span_byte(uint32_t from, uint32_t to, bool &keep)
{
    const uint32_t lane = lane_id();
    const uint32_t hw = from / 16, tw = to / 16;
    uint32_t x = 0;
    keep = false;
    if (lane < 16) {
        x = 16 * hw + lane;
        keep = (from & 15u) && x >= from && x < to;
    } else if (lane < 32) {
        x = 16 * tw + lane - 16;
        keep = (to & 15u) && (tw > hw || (from & 15u) == 0) && x >= from && x < to;
    }
    return keep ? x : 0u;
}

// Stores bytes [from, to) of a segment to dst (a line-aligned stream
// address): its whole words by dwordx4 lanes (word lane + 64 k in v[k]), the
// partial words at either end by the byte lanes of span_byte (byte b, read
// at the position that span_byte gave).  Always the same K + 1 store
// instructions: the buffer's range drops what lies outside.
template <int K>
__device__ __forceinline__ void store_span(const uint4 (&v)[K], uint8_t b, bool keep_b, uint32_t x_b, uint8_t *dst,
                                           uint32_t from, uint32_t to)
{
    const uint32_t lane = lane_id();
    const uint32_t wlo = (from + 15) / 16, whi = to / 16;
    const auto words = __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int32_t)__builtin_amdgcn_readfirstlane(16 * whi),
                                                         kRawBufferWord3);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t i = lane + 64 * k;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{v[k].x, v[k].y, v[k].z, v[k].w}, words,
                                               i >= wlo && i < whi ? 16 * i : kDroppedOffset, 0, 2 /* nt */);
    }
    const auto bytes =
        __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int32_t)__builtin_amdgcn_readfirstlane(to), kRawBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b8(b, bytes, keep_b ? x_b : kDroppedOffset, 0, 0);
}

// Writes a tile's records to the stream from its LDS segment.  LDS word 0
// stands for the line-aligned stream address a0: the segment's first
// `lead` bytes are already in place (records carried over from the previous
// half pass, or, before the first store, bytes that belong to the records
// before this tile, which this wave never writes: `own0` of them).  After
// each half pass the whole lines are stored and the last, partial one (up
// to eight words) is carried to the front, so every store writes whole
// aligned lines except at the tile's first and last line.  Every half pass
// issues the same store instructions (three dwordx4 and one byte store; the
// buffer's range drops what lies outside), so the wait for the next tile's
// loads, issued before these stores, needs no wait for the stores
// themselves.
struct RecordWriter {
    uint64_t a0;
    uint32_t lead, own0;

    __device__ __forceinline__ void begin(RederiveLds &L, uint64_t dst0)
    {
        a0 = dst0 & ~uint64_t(kLineBytes - 1);
        lead = own0 = (uint32_t)(dst0 & (kLineBytes - 1));
        if (lane_id() < kLineWords) L.seg[lane_id()] = make_uint4(0, 0, 0, 0);
    }

    // The byte of the segment where the half pass's records start (the words
    // past the first line are zero: set up by build_wave_tables, kept by
    // flush).
    __device__ __forceinline__ uint32_t open() const { return lead; }

    // Stores the half pass's whole lines (below a line of lead plus 3 * 1024
    // record bytes: at most 3072 bytes, three words per lane), zeroes the
    // words past the first line that its records (and the overhang of the
    // lanes' dword writes) touched, and carries the last, partial line to
    // the front; count may be 0.
    __device__ __forceinline__ void flush(RederiveLds &L, uint8_t *__restrict__ out, uint32_t count)
    {
        wave_lds_fence();
        const uint32_t lane = lane_id();
        const uint32_t end = lead + 3 * count;
        const uint32_t F = __builtin_amdgcn_readfirstlane((end / kLineBytes) * kLineWords);   // whole lines
        const uint32_t to = 16 * F;
        uint4 v[3];
#pragma unroll
        for (uint32_t k = 0; k < 3; ++k) v[k] = L.seg[lane + 64 * k];
        bool keep_b;
        const uint32_t x_b = span_byte(own0, to, keep_b);
        const uint8_t b = reinterpret_cast<const uint8_t *>(L.seg)[x_b];
        const uint4 carry = L.seg[F + lane % kLineWords];
        // the words the half pass touched: (end + 28 + 3) / 16 < kRdSegWords
        const uint32_t touched = (end + 32 + 15) / 16;
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
            const uint32_t i = kLineWords + lane + 64 * k;
            if (i < touched) L.seg[i] = make_uint4(0, 0, 0, 0);
        }
        store_span<3>(v, b, keep_b, x_b, out + a0, own0, to);
        if (F) {
            if (lane < kLineWords) L.seg[lane] = carry;
            a0 += to;
            own0 = 0;
        }
        lead = end - to;
    }

    // The tile's last, partial line.
    __device__ __forceinline__ void finish(RederiveLds &L, uint8_t *__restrict__ out) const
    {
        wave_lds_fence();
        const uint4 v[1] = {L.seg[lane_id() % kLineWords]};
        bool keep_b;
        const uint32_t x_b = span_byte(own0, lead, keep_b);
        store_span<1>(v, reinterpret_cast<const uint8_t *>(L.seg)[x_b], keep_b, x_b, out + a0, own0, lead);
    }
};

// Escape mask of 8 BF16 values (bit k = element k) and their exponent bytes
// (elements 0..3 in ea, 4..7 in eb), from the escape-flag table.
__device__ __forceinline__ uint32_t escapes8_bf16(const uint4 q, const uint8_t *esc8, uint32_t &ea, uint32_t &eb)
{
    const uint32_t lo_a = perm(q.y, q.x, 0x06040200u), hi_a = perm(q.y, q.x, 0x07050301u);
    const uint32_t lo_b = perm(q.w, q.z, 0x06040200u), hi_b = perm(q.w, q.z, 0x07050301u);
    ea = ((hi_a << 1) & 0xFEFEFEFEu) | ((lo_a >> 7) & 0x01010101u);
    eb = ((hi_b << 1) & 0xFEFEFEFEu) | ((lo_b >> 7) & 0x01010101u);
    uint32_t m = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) {
        m |= (uint32_t)esc8[(ea >> (8 * k)) & 0xFFu] << k;
        m |= (uint32_t)esc8[(eb >> (8 * k)) & 0xFFu] << (k + 4);
    }
    return m;
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
                                              uint8_t *buf, uint32_t item, uint32_t slot)
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
        if (k) copy_records(stage + (t0 + g) * (uint64_t)slot, out, off_esc + item * (off + bef), item * k, lane & 15, 16);
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
            copy_records(stage + (t0 + t) * (uint64_t)slot, out, dst0, item * cnt[t], lane, 64);
        }
    }
}

// The metadata of block b, one value per lane: lanes 0..3 the tile counts,
// lane 4 the block's escape offset.
__device__ __forceinline__ uint64_t block_meta(const uint32_t *__restrict__ tile_counts,
                                               const uint64_t *__restrict__ block_offsets, uint64_t nt, uint64_t b)
{
    const uint32_t lane = lane_id();
    const uint64_t t0 = kTilesPerBlock * b;
    uint64_t meta = 0;
    if (lane < kTilesPerBlock && t0 + lane < nt) meta = tile_counts[t0 + lane];
    else if (lane == kTilesPerBlock) meta = block_offsets[b];
    return meta;
}

// Copies the staged records of block b's unflagged tiles (metadata from
// block_meta) to their place in the stream with one wave: 16-lane groups copy
// the four tiles at once when none is flagged and none holds more than
// kGroupCopyRecords records, else the wave copies them tile after tile.
__device__ __forceinline__ void copy_block_records(uint64_t meta, const uint8_t *__restrict__ stage,
                                                   uint8_t *__restrict__ out, uint64_t off_esc, uint64_t b,
                                                   uint32_t item, uint32_t slot)
{
    const uint32_t lane = lane_id();
    const uint64_t t0 = kTilesPerBlock * b;
    const uint64_t off = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(meta >> 32), kTilesPerBlock) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((uint32_t)meta, kTilesPerBlock);
    uint32_t cnt[kTilesPerBlock], before[kTilesPerBlock], most = 0, run = 0, flagged = 0;
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t) {
        const uint32_t v = __builtin_amdgcn_readlane((uint32_t)meta, t);
        cnt[t] = v & ~kRederiveFlag;
        flagged |= (v >> 31) << t;
        before[t] = run;
        run += cnt[t];
        most = std::max(most, cnt[t]);
    }
    if (!flagged && most <= kGroupCopyRecords) {               // wave-uniform
        const uint32_t g = lane >> 4;
        uint32_t k = 0, bef = 0;
#pragma unroll
        for (uint32_t t = 0; t < kTilesPerBlock; ++t)
            if (g == t) {
                k = cnt[t];
                bef = before[t];
            }
        if (k) copy_records(stage + (t0 + g) * (uint64_t)slot, out, off_esc + item * (off + bef), item * k, lane & 15,
                            16);
        return;
    }
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t)
        if (cnt[t] && !((flagged >> t) & 1u))
            copy_records(stage + (t0 + t) * (uint64_t)slot, out, off_esc + item * (off + before[t]), item * cnt[t],
                         lane, 64);
}

// Tiles with at most this many records are copied by 8-lane groups when a
// wave copies two blocks at once.
constexpr uint32_t kPairCopyRecords = 256;

// The metadata of blocks b0 (lanes 0..4, as block_meta) and b1 (lanes
// 32..36; zero when b1 >= nb).
__device__ __forceinline__ uint64_t pair_meta(const uint32_t *__restrict__ tile_counts,
                                              const uint64_t *__restrict__ block_offsets, uint64_t nt, uint64_t nb,
                                              uint64_t b0, uint64_t b1)
{
    const uint32_t lane = lane_id();
    const uint32_t l = lane & 31u;
    const uint64_t b = lane < 32 ? b0 : b1;
    uint64_t meta = 0;
    if (b < nb) {
        const uint64_t t0 = kTilesPerBlock * b;
        if (l < kTilesPerBlock && t0 + l < nt) meta = tile_counts[t0 + l];
        else if (l == kTilesPerBlock) meta = block_offsets[b];
    }
    return meta;
}

// Copies the staged records of blocks b0 and b1 (metadata from pair_meta)
// with one wave: when no tile of either is flagged and none holds more than
// kPairCopyRecords records, eight 8-lane groups copy the eight tiles at once
// (one memory latency for both blocks); else block after block as
// copy_block_records does.
__device__ __forceinline__ void copy_pair_records(uint64_t meta, const uint32_t *__restrict__ tile_counts,
                                                  const uint64_t *__restrict__ block_offsets,
                                                  const uint8_t *__restrict__ stage, uint8_t *__restrict__ out,
                                                  uint64_t off_esc, uint64_t nt, uint64_t nb, uint64_t b0, uint64_t b1,
                                                  uint32_t item, uint32_t slot)
{
    const uint32_t lane = lane_id();
    uint32_t cnt[2][kTilesPerBlock], before[2][kTilesPerBlock], most = 0, flagged = 0;
    uint64_t off[2];
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
        off[h] = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(meta >> 32), 32 * h + kTilesPerBlock) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((uint32_t)meta, 32 * h + kTilesPerBlock);
        uint32_t run = 0;
#pragma unroll
        for (uint32_t t = 0; t < kTilesPerBlock; ++t) {
            const uint32_t v = __builtin_amdgcn_readlane((uint32_t)meta, 32 * h + t);
            cnt[h][t] = v & ~kRederiveFlag;
            flagged |= v & kRederiveFlag;
            before[h][t] = run;
            run += cnt[h][t];
            most = std::max(most, cnt[h][t]);
        }
    }
    if (!flagged && most <= kPairCopyRecords) {                 // wave-uniform
        const uint32_t g = lane >> 3, h = g >> 2, t = g & 3u;
        uint32_t k = 0, bef = 0;
#pragma unroll
        for (uint32_t hh = 0; hh < 2; ++hh)
#pragma unroll
            for (uint32_t tt = 0; tt < kTilesPerBlock; ++tt)
                if (h == hh && t == tt) {
                    k = cnt[hh][tt];
                    bef = before[hh][tt];
                }
        const uint64_t b = h ? b1 : b0;
        if (k)
            copy_records(stage + (kTilesPerBlock * b + t) * (uint64_t)slot, out, off_esc + item * (off[h] + bef),
                         item * k, lane & 7u, 8);
        return;
    }
    copy_block_records(block_meta(tile_counts, block_offsets, nt, b0), stage, out, off_esc, b0, item, slot);
    if (b1 < nb)
        copy_block_records(block_meta(tile_counts, block_offsets, nt, b1), stage, out, off_esc, b1, item, slot);
}

// ---------------------------------------------------------------------------
// Kernel: escape compaction of streams above kFusedPrefixTiles tiles, after
// sz_enc_scan.  512-lane workgroups; wave w of workgroup g copies the staged
// records of blocks 8 g + w, 8 (g + G) + w, ... (G workgroups).  Then, when
// one of the scan's flagged-tile words is set, the flagged (escape-heavy)
// tiles, which the dense encoders did not stage, are derived again from the
// input: workgroup g takes the tiles g, g + G, g + 2G, ... (G workgroups, at
// least kRederiveGroups when the stream has that many tiles, so that the GPU
// is full), reads their tile counts (one per tile and thread), lists the
// flagged ones in LDS in order, and re-derives them.  A tile's first record
// follows its block's offset and the counts of the block's tiles before it.
//   BF16: the eight waves share a tile, wave w its 2048 elements
//   [2048 w, 2048 w + 2048), all loaded at once; the wave totals meet in LDS
//   and each wave writes its records after those of the waves before it, two
//   chunk rows at a time.  The loads of the tile after next are issued
//   before the current tile's records are written.
//   E5M2: each wave re-derives whole tiles of the list on its own.
// ---------------------------------------------------------------------------
constexpr uint32_t kRederiveThreads = 512;
// 2 workgroups of 8 waves (128 registers: two tiles of loads in flight per
// wave) on each compute unit.  Against 3 workgroups of 80 registers and one
// tile ahead, random-bit BF16 (every tile re-derived, 512 MiB) takes 255 us
// instead of 262; the staged copies of the long-context payload 0.5 us more.
constexpr uint32_t kRederiveGroups = 512;
// Blocks whose staged records one wave copies (at most), two at a time: with
// eight, every large Top-16 stream gets the kRederiveGroups workgroups, one
// resident round (a second round of workgroups costs more than the longer
// chain of copies per wave).
constexpr uint64_t kCopyBlocksPerWave = 8;
constexpr int kRdRowChunks = kEncTile / (kRederiveThreads / 64) / 512;   // 4 chunks per lane

// The first record of tile t: its block's offset plus the block's tiles before it.
__device__ __forceinline__ uint64_t tile_first_record(const uint32_t *__restrict__ tile_counts,
                                                      const uint64_t *__restrict__ block_offsets, uint32_t t)
{
    const uint32_t b = t / kTilesPerBlock;
    uint64_t first = block_offsets[b];
    for (uint32_t u = kTilesPerBlock * b; u < t; ++u) first += tile_counts[u] & ~kRederiveFlag;
    return first;
}

// This wave's 512 C elements of tile t: plain dwordx4 loads, or guarded ones
// for the part that holds the end of the input.
template <int C>
__device__ __forceinline__ void load_tile_part_bf16(const uint16_t *__restrict__ in, uint64_t n, uint32_t t,
                                                    uint4 (&q)[C])
{
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint64_t base = (uint64_t)t * kEncTile + (uint64_t)wave * (512 * C);
    if (base + 512 * C <= n) {                                    // wave-uniform
        const uint4 *mine = reinterpret_cast<const uint4 *>(in + base) + lane;
#pragma unroll
        for (int j = 0; j < C; ++j) q[j] = load_nt(mine + 64 * j);
    } else {
        const uint32_t valid = n > base ? (uint32_t)(n - base) : 0u;   // below 512 C here
        const uint16_t *part = in + base;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const uint32_t e0 = (j * 64 + lane) * 8;
            uint16_t v[8];
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) v[k] = (e0 + k < valid) ? part[e0 + k] : 0;
            q[j] = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                              v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
        }
    }
}

// Escape masks and exponent bytes of this wave's part of tile t from its
// loaded words (elements past the end of the input do not escape); returns
// the lane's escape count.
template <int C>
__device__ __forceinline__ uint32_t tile_part_escapes_bf16(const uint4 (&q)[C], const uint8_t *esc8, uint64_t n,
                                                           uint32_t t, uint32_t (&m)[C], uint32_t (&ea)[C],
                                                           uint32_t (&eb)[C])
{
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint64_t base = (uint64_t)t * kEncTile + (uint64_t)wave * (512 * C);
    // elements of this part before the end of the input (wave-uniform)
    const uint32_t valid = n > base ? (uint32_t)std::min<uint64_t>(n - base, 512 * C) : 0u;
    uint32_t lane_total = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        m[j] = escapes8_bf16(q[j], esc8, ea[j], eb[j]);
        const uint32_t e0 = (j * 64 + lane) * 8;
        if (e0 >= valid) m[j] = 0;
        else if (e0 + 8 > valid) m[j] &= (1u << (valid - e0)) - 1;
        lane_total += __popc(m[j]);
    }
    return lane_total;
}

// The BF16 tiles list[0 .. count) (in LDS) of this workgroup, in order.
// Per tile: the wave totals' prefix through LDS, then each wave's records
// after those of the waves before it.  The loads run two tiles ahead in two
// register sets used in turn (the loop body is written out for each): the
// loads of tile i + 2 are issued before tile i's records are written, and
// tile i + 1's words, loaded one tile earlier, are turned into escape masks
// after them.  The stores are a fixed number of instructions, so the wait
// for those loads counts the stores issued after them and does not wait for
// the stores (the vector memory counter completes in issue order).
__device__ __forceinline__ void rederive_tiles_bf16(const uint16_t *__restrict__ in, uint64_t n, const uint32_t *list,
                                                    uint32_t count, const uint32_t *__restrict__ tile_counts,
                                                    const uint64_t *__restrict__ block_offsets, uint64_t off_esc,
                                                    RederiveLds &L, uint32_t *wave_totals, uint8_t *__restrict__ out)
{
    constexpr int C = kRdRowChunks;
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint8_t *esc8 = reinterpret_cast<const uint8_t *>(L.esc32);
    uint32_t *seg32 = reinterpret_cast<uint32_t *>(L.seg);
    uint32_t t = list[0];
    uint32_t tn = 1 < count ? list[1] : t;
    uint4 qa[C], qb[C];
    uint32_t m[C], ea[C], eb[C];
    load_tile_part_bf16<C>(in, n, t, qa);
    load_tile_part_bf16<C>(in, n, tn, qb);
    uint32_t lane_total = tile_part_escapes_bf16<C>(qa, esc8, n, t, m, ea, eb);
    // tile t = list[i] (its masks in m, ea, eb); cur held its words and now
    // takes tile i + 2's, nxt holds tile i + 1's
    auto body = [&](uint4 (&cur)[C], uint4 (&nxt)[C], uint32_t i) {
        // the tile after next (the last again past the end: no branch around the loads)
        const uint32_t tn2 = i + 2 < count ? list[i + 2] : tn;
        load_tile_part_bf16<C>(in, n, tn2, cur);
        const uint32_t base = t * kEncTile + wave * (512 * C);     // low bits: the block positions
        const uint64_t first = tile_first_record(tile_counts, block_offsets, t);
        const uint32_t wave_total = read_lane63(wave_inclusive_sum(lane_total));
        if (lane == 0) wave_totals[wave] = wave_total;
        __syncthreads();
        uint32_t before = 0;
        for (uint32_t w = 0; w < wave; ++w) before += wave_totals[w];
        before = __builtin_amdgcn_readfirstlane(before);            // wave-uniform: the store base
        RecordWriter wr;
        wr.begin(L, off_esc + 3 * (first + before));
#pragma unroll
        for (int h = 0; h < C / 2; ++h) {
            const uint32_t cnt2[2] = {(uint32_t)__popc(m[2 * h]), (uint32_t)__popc(m[2 * h + 1])};
            uint32_t row_base[2], row_total[2], lane_before[2];
            const uint32_t cnt = wave_chunk_ranks<2>(cnt2, row_base, row_total, lane_before);
            const uint32_t lead = wr.open();
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int j = 2 * h + k;
                const uint32_t pos0 = (base + (j * 64 + lane) * 8) & 0xFFFFu;
                if (m[j]) or_records8(seg32, lead + 3 * (row_base[k] + lane_before[k]), m[j], ea[j], eb[j], pos0,
                                      L.slots);
            }
            wr.flush(L, out, cnt);
        }
        wr.finish(L, out);
        __syncthreads();                                          // wave_totals is reused by the next tile
        lane_total = tile_part_escapes_bf16<C>(nxt, esc8, n, tn, m, ea, eb);
        t = tn;
        tn = tn2;
    };
#pragma unroll 1
    for (uint32_t i = 0; i < count; i += 2) {
        body(qa, qb, i);
        if (i + 1 < count) body(qb, qa, i + 1);
    }
}

// Flagged tiles among first + stride (i0 + k), k = 0 .. threads - 1, below
// nt, into list (in order); returns their number.  One tile count per tile
// and thread.
__device__ __forceinline__ uint32_t list_flagged_tiles(const uint32_t *__restrict__ tile_counts, uint32_t nt,
                                                       uint32_t first, uint32_t stride, uint32_t i0, uint32_t *list,
                                                       uint32_t *wave_sums)
{
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
    const uint64_t t64 = first + (uint64_t)stride * (i0 + tid);
    const bool flagged = t64 < nt && (tile_counts[t64 < nt ? t64 : 0] & kRederiveFlag);
    const uint32_t nf = flagged ? 1u : 0u;
    const uint32_t incl = wave_inclusive_sum(nf);
    if (lane == 63) wave_sums[wave] = incl;
    __syncthreads();
    uint32_t at = incl - nf, total = 0;
    for (uint32_t w = 0; w < kRederiveThreads / 64; ++w) {
        const uint32_t v = wave_sums[w];
        if (w < wave) at += v;
        total += v;
    }
    if (flagged) list[at] = (uint32_t)t64;
    __syncthreads();
    return total;
}

template <int DT>
__global__ __launch_bounds__(kRederiveThreads) __attribute__((amdgpu_waves_per_eu(4))) void sz_enc_compact(
    const uint8_t *__restrict__ stage, const uint32_t *__restrict__ tile_counts,
    const uint64_t *__restrict__ block_offsets, uint8_t *__restrict__ out, uint64_t off_esc, uint64_t nt,
    uint64_t nb, uint32_t item, uint32_t slot, const void *__restrict__ in, uint64_t n, Codebook4 cb,
    const uint32_t *__restrict__ cb_dev, const uint32_t *__restrict__ flagged, uint32_t flag_words)
{
    constexpr uint32_t kWaves = kRederiveThreads / 64;
    __shared__ RederiveLds lds[kWaves];
    __shared__ uint32_t list[kRederiveThreads];
    __shared__ uint32_t wave_sums[kWaves];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    // whether the scan saw a flagged tile: the workgroup's lanes share the
    // scan's words (loaded first, so that their latency hides behind the
    // copies) and meet after the copies
    uint32_t any_flagged = 0;
    for (uint32_t i = threadIdx.x; i < flag_words; i += kRederiveThreads) any_flagged |= flagged[i];
    // staged records: wave w of workgroup g copies the blocks b = 8 g + w +
    // 8 G i, two at a time (b and b + 8 G); the next pair's metadata is
    // fetched before the current pair's records are copied
    {
        const uint64_t stride = (uint64_t)gridDim.x * kWaves;
        uint64_t b = (uint64_t)blockIdx.x * kWaves + wave;
        uint64_t meta = b < nb ? pair_meta(tile_counts, block_offsets, nt, nb, b, b + stride) : 0;
        while (b < nb) {                                           // wave-uniform
            const uint64_t b_next = b + 2 * stride;
            const uint64_t meta_next =
                b_next < nb ? pair_meta(tile_counts, block_offsets, nt, nb, b_next, b_next + stride) : 0;
            copy_pair_records(meta, tile_counts, block_offsets, stage, out, off_esc, nt, nb, b, b + stride, item,
                              slot);
            meta = meta_next;
            b = b_next;
        }
    }
    if (!__syncthreads_or(any_flagged)) return;                   // workgroup-uniform
    RederiveLds &L = lds[wave];
    // flagged tiles: workgroup g takes the tiles g, g + G, g + 2G, ...: the
    // tiles that the workgroups work on at one time lie next to each other in
    // memory (which measured markedly faster than giving each workgroup a
    // contiguous range).  Tile indices fit 32 bits (n <= 2^40 gives at most
    // 2^26 tiles).
    const uint32_t tiles = blockIdx.x < nt ? (uint32_t)((nt - blockIdx.x + gridDim.x - 1) / gridDim.x) : 0;
    bool built = false;
#pragma unroll 1
    for (uint32_t i0 = 0; i0 < tiles; i0 += kRederiveThreads) {
        const uint32_t count =
            list_flagged_tiles(tile_counts, (uint32_t)nt, blockIdx.x, gridDim.x, i0, list, wave_sums);
        if (count == 0) continue;                                  // workgroup-uniform
        if (!built) {
            if (cb_dev) cb = load_codebook(cb_dev);
            build_wave_tables(L, cb, DT == SZ_BF16 ? 256 : 32);
            built = true;
        }
        if (DT == SZ_BF16) {
            rederive_tiles_bf16(static_cast<const uint16_t *>(in), n, list, count, tile_counts, block_offsets, off_esc,
                                L, wave_sums, out);
        } else {
#pragma unroll 1
            for (uint32_t i = wave; i < count; i += kWaves) {
                const uint32_t t = list[i];
                const uint64_t dst0 = off_esc + 3 * tile_first_record(tile_counts, block_offsets, t);
                rederive_tile_e5m2(static_cast<const uint8_t *>(in), n, t, reinterpret_cast<const uint8_t *>(L.table32),
                                   reinterpret_cast<uint8_t *>(L.seg), out + (dst0 & ~uint64_t(3)), (uint32_t)(dst0 & 3));
            }
            __syncthreads();                                      // the list is rebuilt for the next range
        }
    }
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
// beyond, so larger streams take the scan.  The dense encoders stage every
// tile of these streams, escape-heavy ones included: a wave copies a heavy
// block's staged records faster than it re-derives them (random bits, 2M to
// 32M elements: 234-278 us per encode against 300-322 us).
// ---------------------------------------------------------------------------
constexpr uint32_t kFusedThreads = 1024;
constexpr uint32_t kFusedBlocks = kFusedThreads / 64;

template <int DT>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(8))) void sz_enc_compact_fused(
    const uint8_t *__restrict__ stage, const uint32_t *__restrict__ tile_counts, uint8_t *__restrict__ out,
    uint64_t off_esc, uint64_t nt, const void *__restrict__ in, HeaderArgs h, const uint32_t *__restrict__ cb_dev,
    int32_t *__restrict__ status, uint32_t item, uint32_t slot)
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
                      seg_buf[wave], item, slot);
}

// ---------------------------------------------------------------------------
// Kernel: compaction with its own prefix for the smallest streams (up to
// kSmallCompactBlocks blocks, one layer of a KV cache), in place of
// sz_enc_compact_fused.  One 1024-lane workgroup per block: its lanes sum the
// counts of the tiles before the block, and each 256-lane quarter then copies
// one of the block's four tiles from its staging slot to its place in the
// stream; the counts, E, the header, the padding and the status word are
// written as sz_enc_compact_fused writes them.  The dense encoders stage
// every tile of these streams, escape-heavy ones included, so that copying
// them takes 1024 lanes per block: a 1M-element stream of random bits encodes
// in 28 us on MI355X, against 297 us when one wave per block re-derived its
// tiles.  A flagged tile, which the dense encoders do not produce for these
// streams, would be re-derived by the first wave of its quarter.  Beyond 16
// blocks this shape costs more than it saves on ordinary streams (3 us at 4M
// elements, 11 us at 16M), so larger streams keep sz_enc_compact_fused.
// ---------------------------------------------------------------------------
constexpr uint32_t kSmallThreads = 1024;
constexpr uint32_t kSmallGroup = kSmallThreads / kTilesPerBlock;   // lanes per tile
constexpr uint64_t kSmallCompactBlocks = 16;

template <int DT>
__global__ __launch_bounds__(kSmallThreads) __attribute__((amdgpu_waves_per_eu(8))) void sz_enc_compact_small(
    const uint8_t *__restrict__ stage, const uint32_t *__restrict__ tile_counts, uint8_t *__restrict__ out,
    uint64_t off_esc, uint64_t nt, const void *__restrict__ in, HeaderArgs h, const uint32_t *__restrict__ cb_dev,
    int32_t *__restrict__ status, uint32_t item, uint32_t slot)
{
    __shared__ uint32_t table32[64];
    __shared__ __align__(16) uint8_t seg_buf[kTilesPerBlock][kSegBytes];
    __shared__ uint64_t wave_part[kSmallThreads / 64];
    const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
    const uint64_t nb = h.nb;
    const uint64_t b = blockIdx.x;                              // the grid has max(1, nb) workgroups
    Codebook4 cb = h.cb;
    const int32_t verdict = device_codebook_verdict(cb_dev, h.dtype, cb);
    build_encode_table(table32, cb, DT == SZ_BF16 ? 256 : 32);
    // escapes of the tiles before this block (a multiple of 4 tiles, all of
    // them below nt)
    const uint64_t t0 = kTilesPerBlock * b;
    uint64_t part = 0;
#pragma unroll 2
    for (uint64_t t = 4 * tid; t < t0; t += 4 * kSmallThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(tile_counts + t);
        part += (uint64_t)(v.x & ~kRederiveFlag) + (v.y & ~kRederiveFlag) + (v.z & ~kRederiveFlag) +
                (v.w & ~kRederiveFlag);
    }
    part = wave_sum_u64(part);
    if (lane == 0) wave_part[wave] = part;
    // the block's four tile counts (flag bit included; 0 past the last tile)
    uint32_t meta[kTilesPerBlock];
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t) meta[t] = b < nb && t0 + t < nt ? tile_counts[t0 + t] : 0u;
    __syncthreads();
    uint64_t acc = 0;
#pragma unroll
    for (uint32_t w = 0; w < kSmallThreads / 64; ++w) acc += wave_part[w];
    const uint64_t off = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(acc >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)acc);
    const uint32_t g = tid / kSmallGroup;                     // this quarter's tile
    uint32_t total = 0, before = 0, k = 0;
    bool flagged = false;
#pragma unroll
    for (uint32_t t = 0; t < kTilesPerBlock; ++t) {
        const uint32_t c = meta[t] & ~kRederiveFlag;
        if (t < g) before += c;
        if (t == g) {
            k = c;
            flagged = meta[t] >> 31;
        }
        total += c;
    }
    uint32_t *header32 = reinterpret_cast<uint32_t *>(out);
    if (b < nb && tid == 0) {
        reinterpret_cast<uint32_t *>(out + 64)[b] = total;
        if (b == nb - 1) {
            const uint64_t e = off + total;
            header32[4] = (uint32_t)e;
            header32[5] = (uint32_t)(e >> 32);
        }
    }
    if (blockIdx.x == 0) write_header(out, h, cb, verdict, nb == 0, status);
    if (b >= nb || k == 0) return;
    const uint64_t dst0 = off_esc + item * (off + before);
    if (flagged) {
        if (tid % kSmallGroup < 64) {
            const uint8_t *table = reinterpret_cast<const uint8_t *>(table32);
            if (DT == SZ_BF16)
                rederive_tile_bf16(static_cast<const uint16_t *>(in), h.n, t0 + g, table, seg_buf[g],
                                   out + (dst0 & ~uint64_t(3)), (uint32_t)(dst0 & 3));
            else
                rederive_tile_e5m2(static_cast<const uint8_t *>(in), h.n, t0 + g, table, seg_buf[g],
                                   out + (dst0 & ~uint64_t(3)), (uint32_t)(dst0 & 3));
        }
    } else {
        copy_records(stage + (t0 + g) * (uint64_t)slot, out, dst0, item * k, tid % kSmallGroup, kSmallGroup);
    }
}

// Streams of up to this many tiles (8M elements) use the BF16 dense encoder
// with two chunks per lane (1024-lane workgroups): on MI355X 1.5 us faster
// per encode at 1M-4M elements, slower from 16M on.
constexpr uint64_t kSmallEncodeTiles = 512;
// Up to this many tiles (64M elements) the Top-16 BF16 encoder runs 512-lane
// workgroups, four chunks per lane: 3 % faster than 256 lanes with eight from
// 32M to 64M elements on MI355X (31.0 -> 29.9 us at 32M, 50.5 -> 48.8 us at
// 64M), the same from 12M to 24M; larger streams keep 256 lanes.
constexpr uint64_t kMidEncodeTiles = 4096;

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
    const WsLayout w = ws_layout(version, dtype, n_elems);
    if (ws_bytes < w.total) return SZ_E_WORKSPACE;
    const Geometry g = geometry(dtype, n_elems, version);
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    uint8_t *out = static_cast<uint8_t *>(d_out);
    int32_t *status = reinterpret_cast<int32_t *>(ws);
    uint32_t *tile_counts = reinterpret_cast<uint32_t *>(ws + w.counts);
    uint64_t *block_offsets = reinterpret_cast<uint64_t *>(ws + w.offsets);
    uint64_t *scan_totals = reinterpret_cast<uint64_t *>(ws + w.totals);
    uint32_t *scan_flagged = reinterpret_cast<uint32_t *>(ws + w.flags);
    uint8_t *stage = ws + w.stage;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // streams that take a compaction with its own prefix stage every tile
    const uint32_t rederive_above = g.nt <= kFusedPrefixTiles ? kStageAll : kRederiveRecords;
    if (g.nt && dtype == SZ_BF16) {
        const uint16_t *in16 = static_cast<const uint16_t *>(d_in);
        if (version == kTop8) {
            LaunchScope scope("sz_enc_dense_top8", s);
            hipLaunchKernelGGL(sz_enc_dense_bf16<kTop8>, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s, in16, g.n,
                               out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage, (uint32_t)w.slot, rederive_above);
        } else if (version == kTop15S) {
            LaunchScope scope("sz_enc_dense_top15s", s);
            hipLaunchKernelGGL(sz_enc_dense_bf16<kTop15S>, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s, in16,
                               g.n, out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage, (uint32_t)w.slot, rederive_above);
        } else if (g.nt <= kSmallEncodeTiles) {
            LaunchScope scope("sz_enc_dense_bf16", s);
            hipLaunchKernelGGL((sz_enc_dense_bf16<kTop16, 2>), dim3((uint32_t)g.nt), dim3(kEncTile / 16), 0, s,
                               in16, g.n, out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage, (uint32_t)w.slot, rederive_above);
        } else if (g.nt <= kMidEncodeTiles) {
            LaunchScope scope("sz_enc_dense_bf16", s);
            hipLaunchKernelGGL((sz_enc_dense_bf16<kTop16, 4>), dim3((uint32_t)g.nt), dim3(kEncTile / 32), 0, s,
                               in16, g.n, out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage, (uint32_t)w.slot, rederive_above);
        } else {
            LaunchScope scope("sz_enc_dense_bf16", s);
            hipLaunchKernelGGL(sz_enc_dense_bf16<kTop16>, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s, in16,
                               g.n, out, g.off_nib, g.off_sm, cb4, cb_dev, tile_counts, stage, (uint32_t)w.slot, rederive_above);
        }
    } else if (g.nt) {
        LaunchScope scope("sz_enc_dense_e5m2", s);
        hipLaunchKernelGGL(sz_enc_dense_e5m2, dim3((uint32_t)g.nt), dim3(kEncThreads), 0, s,
                           static_cast<const uint8_t *>(d_in), g.n, out, g.off_nib, g.off_sm, g.sm_bytes,
                           cb4, cb_dev, tile_counts, stage, (uint32_t)w.slot, rederive_above);
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
            if (g.nb <= kSmallCompactBlocks) {
                const uint32_t blocks = (uint32_t)std::max<uint64_t>(1, g.nb);
                LaunchScope scope("sz_enc_compact_small", s);
                if (dtype == SZ_BF16)
                    hipLaunchKernelGGL(sz_enc_compact_small<SZ_BF16>, dim3(blocks), dim3(kSmallThreads), 0, s, stage,
                                       tile_counts, out, g.off_esc, g.nt, d_in, h, cb_dev, status,
                                       escape_item_bytes(version), (uint32_t)w.slot);
                else
                    hipLaunchKernelGGL(sz_enc_compact_small<SZ_FP8_E5M2>, dim3(blocks), dim3(kSmallThreads), 0, s,
                                       stage, tile_counts, out, g.off_esc, g.nt, d_in, h, cb_dev, status, 3u, (uint32_t)w.slot);
                return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
            }
            const uint32_t groups = (uint32_t)std::max<uint64_t>(1, (g.nb + kFusedBlocks - 1) / kFusedBlocks);
            LaunchScope scope("sz_enc_compact_fused", s);
            if (dtype == SZ_BF16)
                hipLaunchKernelGGL(sz_enc_compact_fused<SZ_BF16>, dim3(groups), dim3(kFusedThreads), 0, s, stage,
                                   tile_counts, out, g.off_esc, g.nt, d_in, h, cb_dev, status,
                                   escape_item_bytes(version), (uint32_t)w.slot);
            else
                hipLaunchKernelGGL(sz_enc_compact_fused<SZ_FP8_E5M2>, dim3(groups), dim3(kFusedThreads), 0, s, stage,
                                   tile_counts, out, g.off_esc, g.nt, d_in, h, cb_dev, status, 3u, (uint32_t)w.slot);
            return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
        }
        // one scan workgroup per kScanSuper blocks, after the reduction of
        // their escape totals when there are several
        const uint32_t scan_groups = (uint32_t)((g.nb + kScanSuper - 1) / kScanSuper);
        if (scan_groups > 1) {
            LaunchScope scope("sz_enc_scan_reduce", s);
            hipLaunchKernelGGL(sz_enc_scan_reduce, dim3(scan_groups), dim3(kScanThreads), 0, s, tile_counts,
                               (uint32_t)g.nt, (uint32_t)g.nb, scan_totals);
        }
        LaunchScope scope("sz_enc_scan", s);
        hipLaunchKernelGGL(sz_enc_scan, dim3(scan_groups), dim3(kScanThreads), 0, s, tile_counts, (uint32_t)g.nt,
                           block_offsets, out, h, cb_dev, status, scan_totals, scan_flagged);
    }
    if (g.nt) {
        // up to kCopyBlocksPerWave blocks per wave for the staged records;
        // for Top-16 at least kRederiveGroups workgroups (the formats other
        // than Top-16 stage every tile: no tile is flagged)
        LaunchScope scope("sz_enc_compact", s);
        const bool rederive = version == kTop16;
        const uint32_t flag_words = rederive ? (uint32_t)((g.nb + kScanSuper - 1) / kScanSuper) * kScanWaves : 0u;
        const uint64_t per_group = kCopyBlocksPerWave * (kRederiveThreads / 64);
        uint64_t groups = (g.nb + per_group - 1) / per_group;
        if (rederive) groups = std::max<uint64_t>(groups, std::min<uint64_t>(kRederiveGroups, g.nt));
        if (dtype == SZ_BF16)
            hipLaunchKernelGGL(sz_enc_compact<SZ_BF16>, dim3((uint32_t)groups), dim3(kRederiveThreads), 0, s, stage,
                               tile_counts, block_offsets, out, g.off_esc, g.nt, g.nb, escape_item_bytes(version),
                               (uint32_t)w.slot, d_in, g.n, cb4, cb_dev, scan_flagged, flag_words);
        else
            hipLaunchKernelGGL(sz_enc_compact<SZ_FP8_E5M2>, dim3((uint32_t)groups), dim3(kRederiveThreads), 0, s,
                               stage, tile_counts, block_offsets, out, g.off_esc, g.nt, g.nb, 3u, (uint32_t)w.slot, d_in,
                               g.n, cb4, cb_dev, scan_flagged, flag_words);
    }
    return hipGetLastError() == hipSuccess ? SZ_OK : SZ_E_HIP;
}

}  // namespace
}  // namespace sz

using namespace sz;

extern "C" uint64_t sz_encoded_size(int dtype, uint64_t n_elems, uint64_t n_escapes)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return 0;
    return geometry(dtype, n_elems).off_esc + 3 * n_escapes;
}

extern "C" uint64_t sz_workspace_size(int dtype, uint64_t n_elems)
{
    if (dtype != SZ_BF16 && dtype != SZ_FP8_E5M2) return 0;
    return ws_layout(kTop16, dtype, n_elems).total;
}

extern "C" uint64_t sz_workspace_size_format(int format, int dtype, uint64_t n_elems)
{
    if (format == SZ_FORMAT_TOP16) return sz_workspace_size(dtype, n_elems);
    if ((format != SZ_FORMAT_TOP8 && format != SZ_FORMAT_TOP15_SENTINEL) || dtype != SZ_BF16) return 0;
    return ws_layout((uint32_t)format, dtype, n_elems).total;
}

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

