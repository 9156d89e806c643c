/*
 * SplitZip CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded definition of what the SplitZip codec
 * computes, written from "SplitZip: Ultra Fast Lossless KV Compression for
 * Disaggregated LLM Serving" (gist.science summary page, Method section:
 * "Encoding strategy" and "Decoding strategy" bullets).  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header, table or helper with the HIP path
 * under fp8_kv_cache_sz_amd/.
 *
 * Every loop walks the elements one at a time in ascending order; there is
 * no blocking, vectorisation or reordering beyond what the stream format
 * itself defines.
 *
 * Stream format v1 (all integers little-endian, A(x) = x rounded up to a
 * multiple of 256, B = 65536 elements per block, nb = ceil(N / B)):
 *   0   u32 magic 0x50495A53        4  u16 version = 1
 *   6   u8  dtype (0 BF16, 1 E5M2)  7  u8  log2(B) = 16
 *   8   u64 N                       16 u64 E (number of escapes)
 *   24  u32 nb                      28 u32 0
 *   32  u8  codebook[16]            48 16 zero bytes
 *   64  u32 counts[nb]              (escapes per block)
 *   off_nib = A(64 + 4 nb): ceil(N/2) bytes of 4-bit codes, element 2k in
 *             the low nibble of byte k, element 2k+1 in the high nibble
 *   off_sm  = off_nib + A(ceil(N/2)): sign/mantissa stream
 *             BF16: N bytes, byte i = sign << 7 | mantissa7
 *             E5M2: 3 * ceil(N/8) bytes; group g holds the 24-bit value
 *                   sum_j sm3[8g+j] << 3j (j = 0..7), sm3 = sign << 2 | mant2
 *   off_esc = off_sm + A(sm bytes): E records of 3 bytes
 *             (pos low byte, pos high byte, original exponent), pos being
 *             the element's index inside its block; records ascend by
 *             element index over the whole stream
 *   size    = off_esc + 3 E
 * Every byte not named above (alignment padding, reserved fields, the
 * unused high nibble of an odd N, the missing elements of the last E5M2
 * group) is zero.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SZO_BF16 0
#define SZO_E5M2 1

#define SZO_OK 0
#define SZO_E_ARG (-1)
#define SZO_E_DTYPE (-2)
#define SZO_E_CAPACITY (-3)
#define SZO_E_FORMAT (-5)

#define SZO_MAGIC 0x50495A53u
#define SZO_VERSION 1u
#define SZO_LOG2_BLOCK 16u
#define SZO_BLOCK 65536ull

/* ------------------------------------------------------------------------- */
/* Field split and join.                                                      */
/* The page's key observation (Method, "core insight"): the redundancy of    */
/* BF16 and FP8 values lives in the exponent field; sign and mantissa are     */
/* high-entropy and are kept raw ("sign/mantissa preservation" bullet).       */
/* The exponent is the raw bit field: zero, subnormals, Inf and NaN are       */
/* ordinary symbols, which keeps every bit pattern lossless.                  */
/* ------------------------------------------------------------------------- */

/* BF16 bit layout: bit 15 sign, bits 14..7 exponent, bits 6..0 mantissa. */
static unsigned bf16_exponent(uint16_t h) { return (h >> 7) & 0xFFu; }
static unsigned bf16_sign(uint16_t h) { return (h >> 15) & 1u; }
static unsigned bf16_mantissa(uint16_t h) { return h & 0x7Fu; }
static uint16_t bf16_join(unsigned sign, unsigned exponent, unsigned mantissa)
{
    return (uint16_t)((sign << 15) | (exponent << 7) | mantissa);
}

/* E5M2 bit layout: bit 7 sign, bits 6..2 exponent, bits 1..0 mantissa. */
static unsigned e5m2_exponent(uint8_t b) { return (b >> 2) & 0x1Fu; }
static unsigned e5m2_sign(uint8_t b) { return (b >> 7) & 1u; }
static unsigned e5m2_mantissa(uint8_t b) { return b & 0x3u; }
static uint8_t e5m2_join(unsigned sign, unsigned exponent, unsigned mantissa)
{
    return (uint8_t)((sign << 7) | (exponent << 2) | mantissa);
}

static unsigned exponent_symbols(int dtype) { return dtype == SZO_BF16 ? 256u : 32u; }

static unsigned element_exponent(int dtype, const void *data, uint64_t i)
{
    if (dtype == SZO_BF16)
        return bf16_exponent(((const uint16_t *)data)[i]);
    return e5m2_exponent(((const uint8_t *)data)[i]);
}

/* The raw sign+mantissa symbol: 8 bits for BF16 (sign << 7 | mantissa),
 * 3 bits for E5M2 (sign << 2 | mantissa). */
static unsigned element_signmant(int dtype, const void *data, uint64_t i)
{
    if (dtype == SZO_BF16) {
        uint16_t h = ((const uint16_t *)data)[i];
        return (bf16_sign(h) << 7) | bf16_mantissa(h);
    }
    uint8_t b = ((const uint8_t *)data)[i];
    return (e5m2_sign(b) << 2) | e5m2_mantissa(b);
}

static void store_element(int dtype, void *out, uint64_t i, unsigned signmant, unsigned exponent)
{
    if (dtype == SZO_BF16)
        ((uint16_t *)out)[i] = bf16_join(signmant >> 7, exponent, signmant & 0x7Fu);
    else
        ((uint8_t *)out)[i] = e5m2_join(signmant >> 2, exponent, signmant & 0x3u);
}

/* ------------------------------------------------------------------------- */
/* Little-endian byte helpers.                                                */
/* ------------------------------------------------------------------------- */
static void put_u16(uint8_t *p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v)
{
    for (int k = 0; k < 4; k++) p[k] = (uint8_t)(v >> (8 * k));
}
static void put_u64(uint8_t *p, uint64_t v)
{
    for (int k = 0; k < 8; k++) p[k] = (uint8_t)(v >> (8 * k));
}
static uint32_t get_u16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get_u32(const uint8_t *p)
{
    uint32_t v = 0;
    for (int k = 3; k >= 0; k--) v = (v << 8) | p[k];
    return v;
}
static uint64_t get_u64(const uint8_t *p)
{
    uint64_t v = 0;
    for (int k = 7; k >= 0; k--) v = (v << 8) | p[k];
    return v;
}

/* ------------------------------------------------------------------------- */
/* Section geometry.                                                          */
/* ------------------------------------------------------------------------- */
static uint64_t round_up_256(uint64_t x) { return (x + 255u) / 256u * 256u; }

static uint64_t block_count(uint64_t n) { return (n + SZO_BLOCK - 1) / SZO_BLOCK; }

static uint64_t nibble_bytes(uint64_t n) { return (n + 1) / 2; }

static uint64_t signmant_bytes(int dtype, uint64_t n)
{
    if (dtype == SZO_BF16) return n;
    return 3u * ((n + 7) / 8);
}

typedef struct {
    uint64_t nb, off_counts, off_nib, off_sm, off_esc;
} layout_t;

static layout_t stream_layout(int dtype, uint64_t n)
{
    layout_t L;
    L.nb = block_count(n);
    L.off_counts = 64;
    L.off_nib = round_up_256(64 + 4 * L.nb);
    L.off_sm = L.off_nib + round_up_256(nibble_bytes(n));
    L.off_esc = L.off_sm + round_up_256(signmant_bytes(dtype, n));
    return L;
}

/* Compressed size: the fixed sections depend on N only; each escape adds one
 * (16-bit position, 8-bit exponent) record ("escape stream" bullet). */
uint64_t szo_encoded_size(int dtype, uint64_t n, uint64_t n_escapes)
{
    if (dtype != SZO_BF16 && dtype != SZO_E5M2) return 0;
    return stream_layout(dtype, n).off_esc + 3u * n_escapes;
}

/* ------------------------------------------------------------------------- */
/* Offline calibration ("fixed-length coding" bullet: an offline-calibrated   */
/* Top-16 codebook of the most frequent exponents).                           */
/* Count every exponent value, then pick the 16 values with the highest       */
/* counts one by one; among equal counts the smaller exponent comes first.    */
/* All 256 (or 32) values take part, so 16 entries exist even when fewer      */
/* than 16 exponents occur.                                                    */
/* ------------------------------------------------------------------------- */
int szo_histogram(int dtype, const void *data, uint64_t n, uint64_t *hist)
{
    if (dtype != SZO_BF16 && dtype != SZO_E5M2) return SZO_E_DTYPE;
    if (!hist || (n && !data)) return SZO_E_ARG;
    unsigned symbols = exponent_symbols(dtype);
    for (unsigned v = 0; v < symbols; v++) hist[v] = 0;
    for (uint64_t i = 0; i < n; i++) hist[element_exponent(dtype, data, i)]++;
    return SZO_OK;
}

int szo_calibrate(int dtype, const void *data, uint64_t n, uint8_t *codebook)
{
    uint64_t hist[256];
    int taken[256];
    int rc = szo_histogram(dtype, data, n, hist);
    if (rc) return rc;
    if (!codebook) return SZO_E_ARG;
    unsigned symbols = exponent_symbols(dtype);
    for (unsigned v = 0; v < symbols; v++) taken[v] = 0;
    for (unsigned c = 0; c < 16; c++) {
        int best = -1;
        for (unsigned v = 0; v < symbols; v++) {
            if (taken[v]) continue;
            if (best < 0 || hist[v] > hist[best]) best = (int)v;
        }
        taken[best] = 1;
        codebook[c] = (uint8_t)best;
    }
    return SZO_OK;
}

/* A codebook is usable when its 16 entries are distinct exponent values. */
static int codebook_valid(int dtype, const uint8_t *codebook)
{
    unsigned symbols = exponent_symbols(dtype);
    for (unsigned c = 0; c < 16; c++) {
        if (codebook[c] >= symbols) return 0;
        for (unsigned d = 0; d < c; d++)
            if (codebook[d] == codebook[c]) return 0;
    }
    return 1;
}

/* Code of exponent v: its index in the codebook, or -1 (an escape). */
static int code_of(const uint8_t *codebook, unsigned v)
{
    for (int c = 0; c < 16; c++)
        if (codebook[c] == v) return c;
    return -1;
}

uint64_t szo_count_escapes(int dtype, const void *data, uint64_t n, const uint8_t *codebook)
{
    uint64_t e = 0;
    for (uint64_t i = 0; i < n; i++)
        if (code_of(codebook, element_exponent(dtype, data, i)) < 0) e++;
    return e;
}

/* ------------------------------------------------------------------------- */
/* Encode ("encoding strategy" bullets): per element, the 4-bit code of the   */
/* exponent goes to the nibble stream (two codes per byte), the raw sign and  */
/* mantissa to the sign/mantissa stream, and an exponent outside the          */
/* codebook becomes an escape record of its position and original exponent   */
/* while its nibble is 0.  Returns the stream size, or a negative error.      */
/* ------------------------------------------------------------------------- */
int64_t szo_encode(int dtype, const void *data, uint64_t n, const uint8_t *codebook,
                   uint8_t *out, uint64_t capacity)
{
    if (dtype != SZO_BF16 && dtype != SZO_E5M2) return SZO_E_DTYPE;
    if (!codebook || !out || (n && !data)) return SZO_E_ARG;
    if (!codebook_valid(dtype, codebook)) return SZO_E_ARG;

    uint64_t total_escapes = szo_count_escapes(dtype, data, n, codebook);
    uint64_t size = szo_encoded_size(dtype, n, total_escapes);
    if (capacity < size) return SZO_E_CAPACITY;

    layout_t L = stream_layout(dtype, n);
    memset(out, 0, size);

    put_u32(out + 0, SZO_MAGIC);
    put_u16(out + 4, SZO_VERSION);
    out[6] = (uint8_t)dtype;
    out[7] = (uint8_t)SZO_LOG2_BLOCK;
    put_u64(out + 8, n);
    put_u64(out + 16, total_escapes);
    put_u32(out + 24, (uint32_t)L.nb);
    put_u32(out + 28, 0);
    for (int c = 0; c < 16; c++) out[32 + c] = codebook[c];

    uint64_t escapes_written = 0;
    for (uint64_t b = 0; b < L.nb; b++) {
        uint64_t first = b * SZO_BLOCK;
        uint64_t last = first + SZO_BLOCK < n ? first + SZO_BLOCK : n;
        uint32_t block_escapes = 0;
        for (uint64_t i = first; i < last; i++) {
            unsigned exponent = element_exponent(dtype, data, i);
            unsigned signmant = element_signmant(dtype, data, i);
            int code = code_of(codebook, exponent);
            if (code < 0) {
                uint8_t *rec = out + L.off_esc + 3 * escapes_written;
                put_u16(rec, (uint32_t)(i - first));
                rec[2] = (uint8_t)exponent;
                escapes_written++;
                block_escapes++;
                code = 0;
            }
            out[L.off_nib + i / 2] |= (uint8_t)(code << (4 * (i % 2)));
            if (dtype == SZO_BF16) {
                out[L.off_sm + i] = (uint8_t)signmant;
            } else {
                /* bit position of element i inside the packed 3-bit stream */
                uint64_t bit = 3 * i;
                for (int k = 0; k < 3; k++, bit++)
                    if ((signmant >> k) & 1u)
                        out[L.off_sm + bit / 8] |= (uint8_t)(1u << (bit % 8));
            }
        }
        put_u32(out + L.off_counts + 4 * b, block_escapes);
    }
    return (int64_t)size;
}

/* ------------------------------------------------------------------------- */
/* Decode ("decoding strategy" bullets): the dense path rebuilds every value  */
/* from its nibble through the code-to-exponent table; the escape stream then */
/* overwrites the exponents of the escaped elements with the stored ones.     */
/* The stream is validated first; returns 0 or a negative error.             */
/* ------------------------------------------------------------------------- */
int szo_validate(const uint8_t *in, uint64_t in_bytes, int dtype, uint64_t n)
{
    if (dtype != SZO_BF16 && dtype != SZO_E5M2) return SZO_E_DTYPE;
    if (!in) return SZO_E_ARG;
    if (in_bytes < 64) return SZO_E_FORMAT;
    if (get_u32(in) != SZO_MAGIC || get_u16(in + 4) != SZO_VERSION) return SZO_E_FORMAT;
    if (in[6] != (uint8_t)dtype) return SZO_E_DTYPE;
    if (in[7] != SZO_LOG2_BLOCK) return SZO_E_FORMAT;
    if (get_u64(in + 8) != n) return SZO_E_FORMAT;
    layout_t L = stream_layout(dtype, n);
    if (get_u32(in + 24) != L.nb || get_u32(in + 28) != 0) return SZO_E_FORMAT;
    uint64_t total_escapes = get_u64(in + 16);
    if (total_escapes > n) return SZO_E_FORMAT;
    if (in_bytes < szo_encoded_size(dtype, n, total_escapes)) return SZO_E_FORMAT;
    unsigned symbols = exponent_symbols(dtype);
    for (int c = 0; c < 16; c++)
        if (in[32 + c] >= symbols) return SZO_E_FORMAT;

    uint64_t sum = 0, r = 0;
    for (uint64_t b = 0; b < L.nb; b++) {
        uint64_t first = b * SZO_BLOCK;
        uint64_t len = (first + SZO_BLOCK < n ? SZO_BLOCK : n - first);
        uint64_t count = get_u32(in + L.off_counts + 4 * b);
        if (count > len) return SZO_E_FORMAT;
        sum += count;
        if (sum > total_escapes) return SZO_E_FORMAT;
        int64_t previous = -1;
        for (uint64_t k = 0; k < count; k++, r++) {
            const uint8_t *rec = in + L.off_esc + 3 * r;
            int64_t pos = (int64_t)get_u16(rec);
            if ((uint64_t)pos >= len || pos <= previous) return SZO_E_FORMAT;
            if (rec[2] >= symbols) return SZO_E_FORMAT;
            previous = pos;
        }
    }
    if (sum != total_escapes) return SZO_E_FORMAT;
    return SZO_OK;
}

int szo_decode(const uint8_t *in, uint64_t in_bytes, int dtype, void *out, uint64_t n)
{
    int rc = szo_validate(in, in_bytes, dtype, n);
    if (rc) return rc;
    if (n && !out) return SZO_E_ARG;
    layout_t L = stream_layout(dtype, n);
    const uint8_t *codebook = in + 32;

    /* dense path: every element from its nibble and its sign/mantissa */
    for (uint64_t i = 0; i < n; i++) {
        unsigned code = (in[L.off_nib + i / 2] >> (4 * (i % 2))) & 0xFu;
        unsigned signmant;
        if (dtype == SZO_BF16) {
            signmant = in[L.off_sm + i];
        } else {
            signmant = 0;
            uint64_t bit = 3 * i;
            for (int k = 0; k < 3; k++, bit++)
                signmant |= (unsigned)((in[L.off_sm + bit / 8] >> (bit % 8)) & 1u) << k;
        }
        store_element(dtype, out, i, signmant, codebook[code]);
    }

    /* sparse path: overwrite the exponent of every escaped element */
    uint64_t r = 0;
    for (uint64_t b = 0; b < L.nb; b++) {
        uint64_t count = get_u32(in + L.off_counts + 4 * b);
        for (uint64_t k = 0; k < count; k++, r++) {
            const uint8_t *rec = in + L.off_esc + 3 * r;
            uint64_t i = b * SZO_BLOCK + get_u16(rec);
            unsigned exponent = rec[2];
            if (dtype == SZO_BF16) {
                uint16_t h = ((uint16_t *)out)[i];
                ((uint16_t *)out)[i] = bf16_join(bf16_sign(h), exponent, bf16_mantissa(h));
            } else {
                uint8_t v = ((uint8_t *)out)[i];
                ((uint8_t *)out)[i] = e5m2_join(e5m2_sign(v), exponent, e5m2_mantissa(v));
            }
        }
    }
    return SZO_OK;
}

/* ------------------------------------------------------------------------- */
/* Canonical check: a stream is canonical when re-encoding its decoded values */
/* with its own codebook reproduces it byte for byte.  Returns 0 when          */
/* canonical, 1 when it decodes but is not canonical, or a negative error.    */
/* ------------------------------------------------------------------------- */
int szo_check_canonical(const uint8_t *in, uint64_t in_bytes, int dtype, uint64_t n)
{
    int rc = szo_validate(in, in_bytes, dtype, n);
    if (rc) return rc;
    uint64_t elem_bytes = dtype == SZO_BF16 ? 2 : 1;
    void *values = malloc(n ? n * elem_bytes : 1);
    if (!values) return SZO_E_ARG;
    rc = szo_decode(in, in_bytes, dtype, values, n);
    if (rc) { free(values); return rc; }
    uint8_t codebook[16];
    memcpy(codebook, in + 32, 16);
    if (!codebook_valid(dtype, codebook)) { free(values); return 1; }
    uint64_t size = szo_encoded_size(dtype, n, get_u64(in + 16));
    uint8_t *again = malloc(size);
    if (!again) { free(values); return SZO_E_ARG; }
    int64_t got = szo_encode(dtype, values, n, codebook, again, size);
    int result = (got == (int64_t)size && memcmp(again, in, size) == 0) ? 0 : 1;
    free(again);
    free(values);
    return result;
}

/* ========================================================================= */
/* Ablation variants (BF16 only).  The page chose a Top-16 book with explicit */
/* escape positions over two alternatives (Method, decoding "design choice"   */
/* bullet; Results, ablations "Top-16 vs Top-8" and "metadata trade-off"):    */
/*                                                                           */
/* Version 2, Top-8: the 8 most frequent exponents get 3-bit codes; every    */
/*   other exponent is an escape with a (position, exponent) record as in    */
/*   version 1, and its code is 0.  Sections:                                 */
/*     off_code = A(64 + 4 nb): 3 * ceil(N/8) bytes; bit 3i + k of the        */
/*                section is bit k of element i's code (LSB first)            */
/*     off_sm   = off_code + A(3 * ceil(N/8)): N bytes sign << 7 | mantissa7  */
/*     off_esc  = off_sm + A(N): E records of 3 bytes as in version 1         */
/*   Header codebook bytes 8..15 are 0.                                       */
/* Version 3, Top-15 + sentinel: the 15 most frequent exponents get codes    */
/*   0..14; code 15 marks an escape whose exponent is the next byte of the    */
/*   escape section (no position is stored).  Sections:                       */
/*     off_nib, off_sm as version 1 (BF16)                                    */
/*     off_esc  = off_sm + A(N): E bytes, the escaped exponents in ascending  */
/*                element order                                                */
/*   counts[b] = escapes of block b as in version 1; header codebook byte 15  */
/*   is 0.                                                                    */
/* The header is the version 1 header with the version field set to 2 or 3. */
/* ========================================================================= */
#define SZO_TOP8 2u
#define SZO_TOP15S 3u

/* Number of codebook entries a version uses. */
static unsigned book_entries(unsigned version)
{
    if (version == SZO_TOP8) return 8;
    if (version == SZO_TOP15S) return 15;
    return 16;
}

static uint64_t code_bytes_v(unsigned version, uint64_t n)
{
    return version == SZO_TOP8 ? 3u * ((n + 7) / 8) : nibble_bytes(n);
}

static layout_t variant_layout(unsigned version, uint64_t n)
{
    layout_t L;
    L.nb = block_count(n);
    L.off_counts = 64;
    L.off_nib = round_up_256(64 + 4 * L.nb);
    L.off_sm = L.off_nib + round_up_256(code_bytes_v(version, n));
    L.off_esc = L.off_sm + round_up_256(n);
    return L;
}

static uint64_t escape_bytes_v(unsigned version) { return version == SZO_TOP15S ? 1u : 3u; }

uint64_t szo_encoded_size_variant(unsigned version, uint64_t n, uint64_t n_escapes)
{
    if (version == 1) return szo_encoded_size(SZO_BF16, n, n_escapes);
    if (version != SZO_TOP8 && version != SZO_TOP15S) return 0;
    return variant_layout(version, n).off_esc + escape_bytes_v(version) * n_escapes;
}

/* Code of exponent v among the first `entries` codebook bytes, or -1. */
static int code_of_first(const uint8_t *codebook, unsigned entries, unsigned v)
{
    for (unsigned c = 0; c < entries; c++)
        if (codebook[c] == v) return (int)c;
    return -1;
}

uint64_t szo_count_escapes_variant(unsigned version, const uint16_t *data, uint64_t n, const uint8_t *codebook)
{
    uint64_t e = 0;
    unsigned entries = book_entries(version);
    for (uint64_t i = 0; i < n; i++)
        if (code_of_first(codebook, entries, bf16_exponent(data[i])) < 0) e++;
    return e;
}

/* Encode a BF16 tensor in version 2 or 3 (version 1 is szo_encode).  Only
 * the first 8 (15) codebook bytes are used and must be distinct.  Returns
 * the stream size or a negative error. */
int64_t szo_encode_variant(unsigned version, const uint16_t *data, uint64_t n, const uint8_t *codebook,
                           uint8_t *out, uint64_t capacity)
{
    if (version == 1) return szo_encode(SZO_BF16, data, n, codebook, out, capacity);
    if (version != SZO_TOP8 && version != SZO_TOP15S) return SZO_E_ARG;
    if (!codebook || !out || (n && !data)) return SZO_E_ARG;
    unsigned entries = book_entries(version);
    for (unsigned c = 0; c < entries; c++)
        for (unsigned d = 0; d < c; d++)
            if (codebook[d] == codebook[c]) return SZO_E_ARG;

    uint64_t total_escapes = szo_count_escapes_variant(version, data, n, codebook);
    uint64_t size = szo_encoded_size_variant(version, n, total_escapes);
    if (capacity < size) return SZO_E_CAPACITY;
    layout_t L = variant_layout(version, n);
    memset(out, 0, size);

    put_u32(out + 0, SZO_MAGIC);
    put_u16(out + 4, version);
    out[6] = (uint8_t)SZO_BF16;
    out[7] = (uint8_t)SZO_LOG2_BLOCK;
    put_u64(out + 8, n);
    put_u64(out + 16, total_escapes);
    put_u32(out + 24, (uint32_t)L.nb);
    put_u32(out + 28, 0);
    for (unsigned c = 0; c < entries; c++) out[32 + c] = codebook[c];

    uint64_t escapes_written = 0;
    for (uint64_t b = 0; b < L.nb; b++) {
        uint64_t first = b * SZO_BLOCK;
        uint64_t last = first + SZO_BLOCK < n ? first + SZO_BLOCK : n;
        uint32_t block_escapes = 0;
        for (uint64_t i = first; i < last; i++) {
            uint16_t h = data[i];
            unsigned exponent = bf16_exponent(h);
            int code = code_of_first(codebook, entries, exponent);
            if (code < 0) {
                if (version == SZO_TOP8) {
                    uint8_t *rec = out + L.off_esc + 3 * escapes_written;
                    put_u16(rec, (uint32_t)(i - first));
                    rec[2] = (uint8_t)exponent;
                    code = 0;
                } else {
                    out[L.off_esc + escapes_written] = (uint8_t)exponent;
                    code = 15;
                }
                escapes_written++;
                block_escapes++;
            }
            if (version == SZO_TOP8) {
                uint64_t bit = 3 * i;
                for (int k = 0; k < 3; k++, bit++)
                    if (((unsigned)code >> k) & 1u)
                        out[L.off_nib + bit / 8] |= (uint8_t)(1u << (bit % 8));
            } else {
                out[L.off_nib + i / 2] |= (uint8_t)(code << (4 * (i % 2)));
            }
            out[L.off_sm + i] = (uint8_t)((bf16_sign(h) << 7) | bf16_mantissa(h));
        }
        put_u32(out + L.off_counts + 4 * b, block_escapes);
    }
    return (int64_t)size;
}

static unsigned variant_code(unsigned version, const uint8_t *in, const layout_t *L, uint64_t i)
{
    if (version == SZO_TOP8) {
        unsigned code = 0;
        uint64_t bit = 3 * i;
        for (int k = 0; k < 3; k++, bit++)
            code |= (unsigned)((in[L->off_nib + bit / 8] >> (bit % 8)) & 1u) << k;
        return code;
    }
    return (in[L->off_nib + i / 2] >> (4 * (i % 2))) & 0xFu;
}

/* Validation of a version 2 or 3 stream: the version 1 header rules, unused
 * codebook bytes zero, per-block counts at most the block length and summing
 * to E, and, per block, version 2 records strictly ascending inside the
 * block, version 3 sentinel codes exactly as many as the block's count. */
int szo_validate_variant(unsigned version, const uint8_t *in, uint64_t in_bytes, uint64_t n)
{
    if (version == 1) return szo_validate(in, in_bytes, SZO_BF16, n);
    if (version != SZO_TOP8 && version != SZO_TOP15S) return SZO_E_ARG;
    if (!in) return SZO_E_ARG;
    if (in_bytes < 64) return SZO_E_FORMAT;
    if (get_u32(in) != SZO_MAGIC || get_u16(in + 4) != version) return SZO_E_FORMAT;
    if (in[6] != (uint8_t)SZO_BF16) return SZO_E_DTYPE;
    if (in[7] != SZO_LOG2_BLOCK) return SZO_E_FORMAT;
    if (get_u64(in + 8) != n) return SZO_E_FORMAT;
    layout_t L = variant_layout(version, n);
    if (get_u32(in + 24) != L.nb || get_u32(in + 28) != 0) return SZO_E_FORMAT;
    for (unsigned c = book_entries(version); c < 16; c++)
        if (in[32 + c] != 0) return SZO_E_FORMAT;
    uint64_t total_escapes = get_u64(in + 16);
    if (total_escapes > n) return SZO_E_FORMAT;
    if (in_bytes < szo_encoded_size_variant(version, n, total_escapes)) return SZO_E_FORMAT;

    uint64_t sum = 0, r = 0;
    for (uint64_t b = 0; b < L.nb; b++) {
        uint64_t first = b * SZO_BLOCK;
        uint64_t len = (first + SZO_BLOCK < n ? SZO_BLOCK : n - first);
        uint64_t count = get_u32(in + L.off_counts + 4 * b);
        if (count > len) return SZO_E_FORMAT;
        sum += count;
        if (sum > total_escapes) return SZO_E_FORMAT;
        if (version == SZO_TOP8) {
            int64_t previous = -1;
            for (uint64_t k = 0; k < count; k++, r++) {
                int64_t pos = (int64_t)get_u16(in + L.off_esc + 3 * r);
                if ((uint64_t)pos >= len || pos <= previous) return SZO_E_FORMAT;
                previous = pos;
            }
        } else {
            uint64_t sentinels = 0;
            for (uint64_t i = first; i < first + len; i++)
                if (variant_code(version, in, &L, i) == 15) sentinels++;
            if (sentinels != count) return SZO_E_FORMAT;
        }
    }
    if (sum != total_escapes) return SZO_E_FORMAT;
    return SZO_OK;
}

/* Decode a version 2 or 3 stream.  Version 2: the dense path rebuilds every
 * value from its 3-bit code, then the records overwrite the escaped
 * exponents (as version 1).  Version 3: one pass in element order; a code
 * of 15 takes the next exponent byte of the escape section. */
int szo_decode_variant(unsigned version, const uint8_t *in, uint64_t in_bytes, uint16_t *out, uint64_t n)
{
    if (version == 1) return szo_decode(in, in_bytes, SZO_BF16, out, n);
    int rc = szo_validate_variant(version, in, in_bytes, n);
    if (rc) return rc;
    if (n && !out) return SZO_E_ARG;
    layout_t L = variant_layout(version, n);
    const uint8_t *codebook = in + 32;
    uint64_t next_escape = 0;
    for (uint64_t i = 0; i < n; i++) {
        unsigned code = variant_code(version, in, &L, i);
        unsigned signmant = in[L.off_sm + i];
        unsigned exponent;
        if (version == SZO_TOP15S && code == 15)
            exponent = in[L.off_esc + next_escape++];
        else
            exponent = codebook[code];
        out[i] = bf16_join(signmant >> 7, exponent, signmant & 0x7Fu);
    }
    if (version == SZO_TOP8) {
        uint64_t r = 0;
        for (uint64_t b = 0; b < L.nb; b++) {
            uint64_t count = get_u32(in + L.off_counts + 4 * b);
            for (uint64_t k = 0; k < count; k++, r++) {
                const uint8_t *rec = in + L.off_esc + 3 * r;
                uint64_t i = b * SZO_BLOCK + get_u16(rec);
                out[i] = bf16_join(bf16_sign(out[i]), rec[2], bf16_mantissa(out[i]));
            }
        }
    }
    return SZO_OK;
}
