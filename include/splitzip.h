/*
 * splitzip.h -- C ABI of the MI355X (gfx950) SplitZip codec.
 *
 * SplitZip ("SplitZip: Ultra Fast Lossless KV Compression for Disaggregated
 * LLM Serving", gist.science summary page) compresses BF16 and FP8-E5M2 KV
 * tensors losslessly: each value splits into its exponent, mapped through an
 * offline-calibrated Top-16 codebook to a 4-bit code (two per byte), and its
 * sign+mantissa bits, stored raw; exponents outside the codebook become
 * escape records (16-bit position, 8-bit exponent).  Decode rebuilds every
 * value from its code through a lookup table and then overwrites the escaped
 * exponents.
 *
 * Conventions for every call:
 *   - Integers in streams are little-endian.  A stream is self-describing:
 *     its 64-byte header carries N, the dtype, the escape count E and the
 *     codebook.  Stream layout (A(x) = x rounded up to 256, B = 65536
 *     elements per block, nb = ceil(N/B)):
 *       [0,64)   header: u32 magic 0x50495A53, u16 version 1, u8 dtype,
 *                u8 log2(B)=16, u64 N, u64 E, u32 nb, u32 0, u8 codebook[16],
 *                16 zero bytes
 *       [64, 64+4nb)  u32 escape count of each block
 *       off_nib = A(64+4nb): ceil(N/2) code bytes, element 2k in the low nibble
 *       off_sm  = off_nib + A(ceil(N/2)): BF16: N bytes sign<<7|mantissa7;
 *                 E5M2: 3*ceil(N/8) bytes, 8 symbols (sign<<2|mantissa2) per
 *                 3 bytes, symbol j of a group at bit 3j
 *       off_esc = off_sm + A(sign/mantissa bytes): E records of 3 bytes
 *                 (pos lo, pos hi, exponent), pos = index inside the block,
 *                 records in ascending element order
 *       size    = off_esc + 3E
 *     Escaped elements carry code 0.  All padding and reserved bytes are 0.
 *   - Device pointers must be 16-byte aligned (torch allocations are).
 *     The caller allocates and owns every buffer.  The library keeps no
 *     state between calls (no buffers, streams or caches) and takes no lock
 *     on the codec path, so calls on different streams with their own
 *     workspaces run concurrently.  The one process-wide state is the
 *     optional instrumentation record (sz_profile_enable): while it is off,
 *     its default, a launch only reads an atomic flag.
 *   - Device calls only enqueue work on `stream` (a hipStream_t; NULL is the
 *     null stream) and return once it is launched.  Calls that share a
 *     workspace must not overlap.  sz_encode, sz_encode_devcb,
 *     sz_encode_format, sz_decode, sz_decode_format and sz_calibrate_device
 *     allocate nothing, issue no memset and never synchronise, so they can
 *     be captured into a HIP graph (with instrumentation off).  sz_transfer
 *     synchronises and cannot.
 *   - Errors are negative return codes; nothing throws or aborts across the
 *     ABI.  Checks made on the device (the stream checks of sz_decode, the
 *     codebook check of sz_encode_devcb) land in the workspace status word,
 *     an int32 at workspace offset 0: 0 or a negative SZ_E_* code, valid once
 *     the stream has synchronised.  sz_encode sets it to 0.
 */
#ifndef SPLITZIP_H
#define SPLITZIP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types: BF16 (exponent 8 bits, sign+mantissa 8 bits) and FP8 E5M2
 * (exponent 5 bits, sign+mantissa 3 bits; the page's FP8 extension,
 * Contributions item 4). */
enum { SZ_BF16 = 0, SZ_FP8_E5M2 = 1 };

enum {
    SZ_OK = 0,
    SZ_E_ARG = -1,       /* null pointer, bad codebook, size out of range */
    SZ_E_DTYPE = -2,     /* unknown dtype, or codebook/stream of another dtype */
    SZ_E_CAPACITY = -3,  /* output smaller than the worst-case stream */
    SZ_E_ALIGN = -4,     /* device pointer not 16-byte aligned */
    SZ_E_FORMAT = -5,    /* malformed or truncated stream */
    SZ_E_HIP = -6,       /* a HIP launch or runtime call failed */
    SZ_E_WORKSPACE = -7, /* workspace smaller than the call's *_workspace_size() */
    SZ_E_SCRATCH = -8    /* request larger than sz_decode_noalloc's fixed scratch */
};

/* Top-16 exponent codebook: exp[c] is the exponent that code c stands for.
 * Entries are distinct and below 256 (BF16) or 32 (E5M2). */
typedef struct sz_codebook {
    uint32_t dtype;
    uint8_t exp[16];
} sz_codebook;

/* Offline calibration (page: Method, "fixed-length coding" bullet, and
 * Results, calibration ablation: one offline codebook, no online histogram).
 * Host call.  host_data holds n_elems raw BF16 (uint16) or E5M2 (uint8)
 * values.  Counts every exponent value and orders all 256 (32) values by
 * count descending, then exponent ascending; the first 16 form the codebook,
 * so 16 entries exist even when fewer exponents occur.  Returns SZ_OK,
 * SZ_E_DTYPE or SZ_E_ARG (null pointer with n_elems > 0, null out). */
int sz_calibrate(int dtype, const void *host_data, uint64_t n_elems, sz_codebook *out);

/* Exact stream size for n_elems values with n_escapes escapes: the fixed
 * sections plus 3 bytes per escape record (page: Method, "escape stream"
 * bullet).  n_escapes = n_elems gives the worst case, which sz_encode needs
 * as output capacity.  Returns 0 for an unknown dtype. */
uint64_t sz_encoded_size(int dtype, uint64_t n_elems, uint64_t n_escapes);

/* Device workspace that sz_encode (and sz_encode_devcb) needs for n_elems
 * values: the status word, tile escape counts, block offsets, one escape
 * total and 16 flagged-tile words per 8,192 blocks (the scan's workgroups)
 * and the escape staging area.  Staging takes one slot per 16384-element tile: 49,152
 * bytes (3 per element) for streams of up to 2,048 tiles (32M elements),
 * whose tiles are all staged, and 12,288 bytes above that, where a tile
 * with more than 4,096 escapes stages nothing (the compaction derives its
 * records again from the input).  About 3 bytes per element up to 32M
 * elements, 0.75 above.  Also enough for sz_decode.  Returns 0 for an
 * unknown dtype. */
uint64_t sz_workspace_size(int dtype, uint64_t n_elems);

/* Device workspace that sz_decode (and sz_decode_format) needs for n_elems
 * values: the status words (256 bytes) and one u64 escape offset per 64K
 * block, 8 bytes per 65,536 elements.  Returns 0 for an unknown dtype. */
uint64_t sz_decode_workspace_size(int dtype, uint64_t n_elems);

/* Encode (page: Method, encoding bullets).  d_in: n_elems raw values on the
 * device.  d_out: stream buffer of out_capacity >= sz_encoded_size(dtype,
 * n_elems, n_elems) bytes.  d_ws: ws_bytes >= sz_workspace_size(dtype,
 * n_elems).  The stream is byte-identical to the format above for the given
 * codebook; its size is sz_encoded_size(dtype, n_elems, E) with E the u64 at
 * stream offset 16, readable after the stream synchronises.  Bytes of d_out
 * past that size are unspecified.  n_elems <= 2^40.  Returns SZ_OK or a
 * negative code (host checks: dtype, codebook, pointers, alignment, capacity,
 * workspace; SZ_E_HIP on launch failure). */
int sz_encode(int dtype, const void *d_in, uint64_t n_elems, const sz_codebook *cb,
              void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes,
              void *stream);

/* sz_encode with the codebook read from device memory: d_cb is an
 * sz_codebook in device memory (16-byte aligned), for instance one written
 * by sz_calibrate_device earlier on the same stream, so a per-tensor book
 * needs no host round trip.  The stream equals sz_encode's for the same
 * codebook.  The codebook is checked on the device: a dtype word other than
 * dtype sets the status word to SZ_E_DTYPE, an entry >= 256 (BF16) / 32
 * (E5M2) or a repeated entry sets SZ_E_ARG; either way the stream's magic is
 * written as 0, so sz_decode rejects it.  Other arguments and return codes
 * as sz_encode. */
int sz_encode_devcb(int dtype, const void *d_in, uint64_t n_elems, const sz_codebook *d_cb,
                    void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes,
                    void *stream);

/* On-device calibration (page: Results, calibration ablation, which sets
 * per-tensor books fitted at run time against one offline book; the Top-16
 * rule of Method, fixed-length coding bullet).  The rule of sz_calibrate,
 * computed on the GPU over the 64K blocks 0, s, 2s, ... of d_in
 * (s = sample_every >= 1; s = 1 takes the whole tensor): the exponents of
 * those blocks' elements are counted, all 256 (32) values are ordered by
 * count descending, then value ascending, and the first 16 are written to
 * d_cb (an sz_codebook in device memory, dtype word included).  d_hist, if
 * not NULL, receives the 256 (BF16) or 32 (E5M2) uint64 exponent counts.
 * d_ws: ws_bytes >= sz_calibrate_workspace_size(dtype) (partial counts).
 * Enqueue only; the results are valid once the stream has run past them.
 * Returns SZ_OK, SZ_E_DTYPE, SZ_E_ARG (null pointer, sample_every = 0,
 * n_elems > 2^40), SZ_E_ALIGN (d_in, d_cb, d_hist, d_ws not 16-byte
 * aligned), SZ_E_WORKSPACE or SZ_E_HIP. */
uint64_t sz_calibrate_workspace_size(int dtype);
int sz_calibrate_device(int dtype, const void *d_in, uint64_t n_elems, uint64_t sample_every,
                        sz_codebook *d_cb, uint64_t *d_hist, void *d_ws, uint64_t ws_bytes,
                        void *stream);

/* Ablation formats (page: Method, decoding "design choice" bullet, which
 * prefers Top-16 with explicit positions to a Top-15 book with a sentinel
 * code; Results, ablations "Top-16 vs Top-8" and "metadata trade-off").
 * BF16 only.  A format is the stream's version field:
 *   SZ_FORMAT_TOP16 (1): the format above (sz_encode / sz_decode).
 *   SZ_FORMAT_TOP8 (2): the 8 most frequent exponents get 3-bit codes; the
 *     code section holds 3*ceil(N/8) bytes, bit 3i+k = bit k of element i's
 *     code; escapes carry code 0 and a 3-byte record as in format 1; header
 *     codebook bytes 8..15 are 0; size = sections + 3 E.
 *   SZ_FORMAT_TOP15_SENTINEL (3): codes 0..14 for the 15 most frequent
 *     exponents, code 15 marks an escape; the escape section holds one byte
 *     per escape, the original exponent, in ascending element order (no
 *     positions); header codebook byte 15 is 0; size = sections + E.
 * Sections are 256-byte aligned as in format 1 (header, u32 counts[nb],
 * codes, N sign/mantissa bytes, escapes).  sz_encode_format uses the first
 * 8 (15) entries of cb, which must be distinct; sz_decode_format checks, on
 * the device, the header (version included), the unused codebook bytes,
 * the counts, the records (format 2) or that each block's sentinel codes
 * number exactly its count (format 3).  sz_encoded_size_format returns 0
 * for an unknown format or a dtype other than BF16 with formats 2 and 3;
 * the calls return SZ_E_ARG for an unknown format and SZ_E_DTYPE for E5M2
 * with formats 2 and 3.  Capacity, alignment and status rules as for
 * sz_encode / sz_decode; the output capacity is
 * sz_encoded_size_format(format, dtype, n_elems, n_elems).  These formats
 * stage every tile, so sz_encode_format needs
 * sz_workspace_size_format(format, dtype, n_elems) bytes of workspace (3
 * bytes per element for Top-8, 1 for Top-15 + sentinel; 0 for an unknown
 * format or dtype); sz_decode_format needs sz_decode_workspace_size. */
enum { SZ_FORMAT_TOP16 = 1, SZ_FORMAT_TOP8 = 2, SZ_FORMAT_TOP15_SENTINEL = 3 };

uint64_t sz_encoded_size_format(int format, int dtype, uint64_t n_elems, uint64_t n_escapes);
uint64_t sz_workspace_size_format(int format, int dtype, uint64_t n_elems);
int sz_encode_format(int format, int dtype, const void *d_in, uint64_t n_elems, const sz_codebook *cb,
                     void *d_out, uint64_t out_capacity, void *d_ws, uint64_t ws_bytes, void *stream);
int sz_decode_format(int format, const void *d_in, uint64_t in_bytes, int dtype, void *d_out,
                     uint64_t n_elems, void *d_ws, uint64_t ws_bytes, void *stream);

/* Chunked transfer over a bandwidth-limited link (page: Problem section,
 * the prefill-to-decode KV transfer over 50-100 GB/s links; Results,
 * transfer latency, where the smaller payload shortens the transfer and
 * the codec's time is a small share of it).  One GPU stands in for both
 * ends: the link is PCIe through pinned host memory (device -> host, then
 * host -> device), the host buffer playing the wire.  d_src (n_elems
 * values on the device) is sent in chunks of chunk_elems values (the last
 * may be shorter; chunk_elems * element size must be a multiple of 16) and
 * arrives in d_dst.  With compress != 0, each chunk is encoded with cb into
 * its own stream, exactly the stream's bytes cross the link both ways, and
 * the chunk is decoded into place; with compress = 0 the raw bytes cross.
 * `depth` (1..8) buffer slots let the encode, D2H, H2D and decode of
 * consecutive chunks overlap on three library-owned streams (codec, D2H,
 * H2D).
 *   h_staging: pinned host memory mapped into the device's address space
 *     (hipHostMalloc; torch's pin_memory) of h_bytes >=
 *     sz_transfer_host_bytes(dtype, n_elems, chunk_elems, depth); the
 *     library writes stream headers and decode statuses into it from
 *     kernels (SZ_E_ARG if the device cannot address it).
 *   d_ws: ws_bytes >= sz_transfer_workspace_size(dtype, chunk_elems, depth).
 *   stream: the caller's stream; the transfer starts once the work already
 *     queued on it is done.
 * Synchronous: returns once d_dst holds the whole tensor.  stats gets the
 * host wall time from the first enqueue to the last completion, the chunk
 * count, the raw bytes, the bytes that crossed the link (each direction),
 * the escape total and the first non-zero decode status (0 when every chunk
 * decoded cleanly).  Returns SZ_OK, SZ_E_DTYPE, SZ_E_ARG (depth, chunk size,
 * null pointers), SZ_E_ALIGN (16 bytes for every pointer), SZ_E_WORKSPACE
 * (either buffer too small), SZ_E_HIP, or an error of sz_encode /
 * sz_decode. */
typedef struct sz_transfer_stats {
    double total_ms;
    uint64_t chunks;
    uint64_t raw_bytes;
    uint64_t wire_bytes;
    uint64_t escapes;
    int32_t decode_status;
} sz_transfer_stats;

uint64_t sz_transfer_workspace_size(int dtype, uint64_t chunk_elems, int depth);
uint64_t sz_transfer_host_bytes(int dtype, uint64_t n_elems, uint64_t chunk_elems, int depth);
int sz_transfer(int dtype, const void *d_src, uint64_t n_elems, uint64_t chunk_elems,
                const sz_codebook *cb, int compress, int depth, void *h_staging, uint64_t h_bytes,
                void *d_dst, void *d_ws, uint64_t ws_bytes, void *stream, sz_transfer_stats *stats);

/* Decode (page: Method, decoding bullets: dense unpack + lookup table, then
 * the sparse escape stream overwrites the escaped exponents).  d_in: a
 * stream of in_bytes bytes on the device.  d_out: n_elems values.  d_ws:
 * ws_bytes >= sz_decode_workspace_size(dtype, n_elems).  The host checks the
 * arguments and in_bytes >= sz_encoded_size(dtype, n_elems, 0); the device
 * checks the header (magic, version, dtype, N, nb), the escape counts (each
 * at most its block length, summing to E), that the E records fit in
 * in_bytes, and that positions ascend strictly inside each block and stay
 * below the block length.  A failed device check sets the workspace status
 * word; d_out is then unspecified, and no byte outside d_out[0, n_elems) is
 * ever written.  Escape records whose exponent is in the codebook are
 * applied like any other. */
int sz_decode(const void *d_in, uint64_t in_bytes, int dtype, void *d_out, uint64_t n_elems,
              void *d_ws, uint64_t ws_bytes, void *stream);

/* sz_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same decode as sz_decode (same kernels, checks and output), with its
 * scratch (the verdict word and the per-block escape offsets) in a fixed
 * 1 MiB array in device memory that the library holds on each device it
 * runs on until the process ends, instead of a caller workspace.  The call
 * itself allocates nothing and issues no memset.
 *   d_status: a caller-owned device int32 (4-byte aligned) that receives the
 *     status: 0, or the negative SZ_E_* code of a failed device check;
 *     valid once the stream has run past the call.
 *   n_elems <= sz_decode_noalloc_max_elems() (8,587,706,368 values:
 *     131,038 blocks of 65,536); larger requests return SZ_E_SCRATCH
 *     before any launch.
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress, with the device current); a failed lookup returns
 * SZ_E_HIP.  Every call on one device shares its array and the array keeps
 * the last call's contents (each call rewrites what it reads before reading
 * it): calls that overlap on one device, on any streams, race and must be
 * serialised by the caller.  Other arguments and return codes as
 * sz_decode. */
uint64_t sz_decode_noalloc_max_elems(void);
int sz_decode_noalloc(const void *d_in, uint64_t in_bytes, int dtype, void *d_out, uint64_t n_elems,
                      int32_t *d_status, void *stream);

/* Instrumentation (not part of the codec).  While enabled, every kernel the
 * library launches is bracketed by a pair of HIP events recorded on the
 * launch stream.  sz_profile_collect waits for the recorded events, writes
 * up to max_stats per-kernel totals (kernel name, launches, summed
 * milliseconds) and clears the record; it returns the number of kernels
 * written, or a negative code.  Enabling or disabling clears the record. */
typedef struct sz_kernel_stat {
    char name[48];
    uint64_t launches;
    double total_ms;
} sz_kernel_stat;

int sz_profile_enable(int on);
int sz_profile_collect(sz_kernel_stat *stats, int max_stats);

/* Reference streaming copy (not part of the codec).  Copies `bytes` bytes
 * (a multiple of 16) from d_src to d_dst on the device, one non-temporal
 * 16-byte load and store per lane, 4 KB per 256-lane workgroup (the fastest
 * plain copy shape measured on MI355X), so its rate is the practical
 * streaming ceiling the codec kernels are measured against.  Both pointers
 * 16-byte aligned, the ranges must not overlap.  Enqueue only.  Returns
 * SZ_OK (also for bytes = 0), SZ_E_ARG (null pointer, bytes not a multiple
 * of 16, overlapping ranges), SZ_E_ALIGN or SZ_E_HIP. */
int sz_reference_copy(const void *d_src, void *d_dst, uint64_t bytes, void *stream);

/* Reference of the dense encoders' memory pattern (not part of the codec).
 * Reads n_elems elements of dtype (SZ_BF16: 2 bytes each, SZ_FP8_E5M2: 1
 * byte) at d_in and writes n_elems / 2 bytes to d_codes and, per element,
 * the sign/mantissa section's share to d_sym (BF16: n_elems bytes, E5M2:
 * 3 n_elems / 8 bytes), with the grid, tile and lane mapping and the memory
 * instructions of the dense encoder of that dtype (BF16: its shape for
 * streams above 4096 tiles, eight 8-element chunks per lane) and trivial
 * arithmetic:
 *   BF16, per 8 elements: d_sym gets the 8 low bytes, d_codes 4 bytes, the
 *     high bytes of elements 0..3 XOR those of elements 4..7;
 *   E5M2, per 32 bytes a (bytes 0..15) and b (16..31): d_codes gets a XOR b,
 *     d_sym bytes 0..11 of b.
 * Its rate is the practical ceiling of the encoders' one-read, two-write
 * stream mix.  n_elems must be a multiple of 16384 (whole encoder tiles);
 * all pointers 16-byte aligned, caller-owned, not overlapping.  Enqueue
 * only.  Returns SZ_OK (also for n_elems = 0), SZ_E_DTYPE, SZ_E_ARG (null
 * pointer, n_elems not a multiple of 16384), SZ_E_ALIGN or SZ_E_HIP. */
int sz_reference_split(int dtype, const void *d_in, uint64_t n_elems, void *d_codes, void *d_sym, void *stream);

/* Reference of the span decoders' memory pattern on large streams (not part
 * of the codec): the inverse stream mix of sz_reference_split.  Reads
 * n_elems / 2 code bytes at d_codes and the sign/mantissa share at d_sym
 * (BF16: n_elems bytes, E5M2: 3 n_elems / 8) and writes n_elems elements
 * (BF16: 2 n_elems bytes, E5M2: n_elems) to d_out, with the wide-span grid,
 * lane mapping and memory instructions of the decoder of that dtype and
 * trivial arithmetic:
 *   BF16, per 8 elements: 16 bytes = the 8 sym bytes, the 4 code bytes,
 *     then those code bytes XOR sym bytes 0..3;
 *   E5M2, per 32 elements: 32 bytes = the 16 code bytes, the 12 sym bytes,
 *     then code bytes 0..3 XOR sym bytes 0..3.
 * n_elems must be a multiple of 16384; all pointers 16-byte aligned,
 * caller-owned, not overlapping.  Enqueue only.  Returns SZ_OK (also for
 * n_elems = 0), SZ_E_DTYPE, SZ_E_ARG (null pointer, n_elems not a multiple
 * of 16384), SZ_E_ALIGN or SZ_E_HIP. */
int sz_reference_join(int dtype, const void *d_codes, const void *d_sym, uint64_t n_elems, void *d_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_H */
