/*
 * aqlm.h - C ABI of libaqlm.so: the AQLM 2-bit quantized linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * Representation ("The AQLM Quantization Algorithm, Explained", section
 * "What is Multi-Codebook Quantization (MCQ)?" and Figure 2): a weight matrix
 * W of shape [out][in] (W.X convention, rows are output channels) is cut
 * row-wise into groups of g consecutive inputs.  Group j of row i is the sum
 * of M codewords, one from each of M codebooks of 2^B fp16 codewords of
 * length g, then multiplied by the row's fp16 scale:
 *
 *     W[i][j*g + t] = s[i] * sum_{m=0}^{M-1} C_m[ code[i][j][m] ][t]
 *
 * Schemes ("Key AQLM quantization parameters" on the same page: (M, B, g)
 * are free hyperparameters, and e.g. (1, 4), (2, 8), ..., (8, 32) at B = 8
 * all cost 2 bits per weight): 1 <= M <= AQLM_MAX_CODEBOOKS, 1 <= B <= 16,
 * g in {1, 2, 4, 8, 16, 32}.  The two named there as XBit-MxB at g = 8,
 * (1, 16, 8) "1x16" and (2, 8, 8) "2x8", run tuned kernels; every other
 * triple runs general kernels with the same semantics, except that the GEMV
 * of the other 2-bit triples with B = 8 ((1, 8, 4), (4, 8, 16), and
 * (8, 8, 32) above batch 8) runs the tuned 2x8 kernel when in % 8 == 0, and
 * the prefill GEMM of (1, 8, 4) the tuned 2x8 pipeline when in % 64 == 0.
 *
 * Memory layouts (all arrays contiguous, row-major, DEVICE pointers):
 *   codes      [out][in/g][M]  uint8 for B <= 8; 16-bit (int16) for
 *                              9 <= B <= 16.  The codeword index is the low
 *                              B bits of the stored pattern read as unsigned
 *                              (the page notes that a B that is not a
 *                              multiple of 8 leaves bits of its bytes unused)
 *   codebooks  [M][2^B][g]     fp16 (IEEE binary16, passed as opaque 16-bit
 *                              storage)
 *   scales     [out]           fp16
 *   x          [batch][in]     fp16 activations
 *   y          [batch][out]    fp16 outputs (decode: W16 [out][in])
 *
 * Ownership: the caller owns every buffer.  No entry point keeps a pointer
 * after it returns, and none allocates device memory.
 *
 * Asynchrony: every call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t; NULL means the null stream) and
 * returns.  Execution errors surface at the caller's next synchronisation.
 * Calls are reentrant and thread-safe.  A call with out == 0 (or, for GEMV
 * and GEMM, batch == 0) enqueues nothing and returns AQLM_OK once the scheme
 * and shape are valid; its pointers may then be NULL.
 *
 * Numerics: GEMV and GEMM accumulate in fp32 and round y to fp16 once
 * (nearest-even).  Decode is bit-exact: per weight, the fp32 sum of the M
 * codewords (codebook 0 first, then m ascending, the sum starting from
 * codebook 0's codeword), times the fp32 scale, rounded to fp16 nearest-even
 * with subnormals kept.
 */
#ifndef AQLM_H
#define AQLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AQLM_OK = 0,
    AQLM_ERR_NULL = 1,   /* a required pointer is NULL (or decode got x != NULL) */
    AQLM_ERR_SHAPE = 2,  /* out/in/batch negative or out of range, in % g != 0 */
    AQLM_ERR_SCHEME = 3, /* (M, B, g) outside 1..AQLM_MAX_CODEBOOKS x 1..16 x {1,2,4,8,16,32} */
    AQLM_ERR_ALIGN = 4,  /* codes, codebooks, x or y not 16-byte aligned, scales not 2-byte aligned */
    AQLM_ERR_HIP = 5,    /* the HIP runtime reported an error at launch */
    AQLM_ERR_SCRATCH = 6 /* more scratch needed than an allocation-free entry point holds */
} aqlm_status;

/* Largest `in` accepted (inputs per row). */
#define AQLM_MAX_IN (1 << 20)
/* Most codebooks (M) a scheme may have. */
#define AQLM_MAX_CODEBOOKS 8
/* Largest batch of aqlm_linear_gemv. */
#define AQLM_GEMV_MAX_BATCH 16

/*
 * y[b][i] = sum_k W[i][k] * x[b][k] for b < batch, with W decoded on the fly
 * (Figure 2 of the MCQ section: weights are dequantized after being fetched,
 * then multiplied).  Decode-phase matrix-vector product: 1 <= batch <= 16.
 * Requires 1 <= in <= AQLM_MAX_IN, in % g == 0, out <= 2^31 - 16.
 */
int aqlm_linear_gemv(const void* codes, const void* codebooks, const void* scales,
                     const void* x, void* y, int M, int B, int g,
                     int64_t out, int64_t in, int64_t batch, void* stream);

/* Most layers one aqlm_linear_gemv_fused call takes. */
#define AQLM_FUSED_MAX_LAYERS 8

/*
 * n_layers decode-phase products that share the activations x, in one launch:
 *
 *     y_l[b][i] = sum_k W_l[i][k] * x[b][k]   for l < n_layers, b < batch,
 *
 * e.g. the q, k and v projections of an attention block, or the gate and up
 * projections of its MLP, which all multiply the same hidden state.  Layer l
 * has its own codes[l], codebooks[l], scales[l], outs[l] rows and output
 * ys[l] ([batch][outs[l]]); all layers share (M, B, g), in, batch and x.
 * codes, codebooks, scales, outs and ys are HOST arrays of n_layers entries;
 * the pointers they hold are device pointers with the layouts above.  The
 * library reads the arrays during the call and keeps nothing.
 *
 * Each layer is validated exactly as by aqlm_linear_gemv and the first
 * failing layer's status is returned (nothing is enqueued then); a layer
 * with outs[l] == 0 is skipped.  1 <= n_layers <= AQLM_FUSED_MAX_LAYERS
 * (else AQLM_ERR_SHAPE); a NULL array gives AQLM_ERR_NULL.  The results are
 * bit-identical to n_layers separate aqlm_linear_gemv calls; fusing pays the
 * launch and the per-workgroup start-up latencies once for the group.  (The
 * triples whose GEMV runs a general kernel are served by one launch per
 * layer.)
 */
int aqlm_linear_gemv_fused(int n_layers, const void* const* codes, const void* const* codebooks,
                           const void* const* scales, const int64_t* outs, const void* x,
                           void* const* ys, int M, int B, int g, int64_t in, int64_t batch,
                           void* stream);

/*
 * Same product for a prefill batch of `batch` >= 1 tokens (batch <= 2^31 - 1):
 * W tiles are decoded into LDS and fed to fp16 matrix cores with fp32
 * accumulation.
 */
int aqlm_linear_gemm(const void* codes, const void* codebooks, const void* scales,
                     const void* x, void* y, int M, int B, int g,
                     int64_t out, int64_t in, int64_t batch, void* stream);

/*
 * The same prefill product in two passes, following the page's statement that
 * the product with the activations runs on the dequantized half-precision
 * weights ("The AQLM Quantization Algorithm, Explained", MCQ section, Figure
 * 2): the weights are decoded once into `workspace` (W16[out][in] fp16,
 * bit-exact as aqlm_linear_decode writes them, the scale applied), then a
 * dense fp16 matrix-core product y = x W16^T runs with fp32 accumulation and
 * one rounding to fp16.  Each weight is decoded once instead of once per
 * 256-token tile.  workspace is caller-owned device memory, 16-byte aligned,
 * of at least aqlm_gemm_dequant_workspace_bytes bytes; its contents are
 * overwritten, and calls that share it must not run concurrently.  Every
 * argument is validated as by aqlm_linear_gemm, and out * (in / g) <
 * 2^32 (else AQLM_ERR_SHAPE).  A NULL or undersized workspace gives
 * AQLM_ERR_NULL / AQLM_ERR_SHAPE, a misaligned one AQLM_ERR_ALIGN.  When
 * in % 64 != 0 the call runs aqlm_linear_gemm instead and does not touch the
 * workspace.
 */
int aqlm_linear_gemm_dequant(const void* codes, const void* codebooks, const void* scales,
                             const void* x, void* y, void* workspace, int64_t workspace_bytes,
                             int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream);

/* Bytes of workspace aqlm_linear_gemm_dequant needs (out * in * 2; 0 when in % 64 != 0). */
int aqlm_gemm_dequant_workspace_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes);

/*
 * Writes the dequantized fp16 weights W16[out][in] to y (bit-exact as stated
 * above).  x must be NULL; batch is ignored.
 */
int aqlm_linear_decode(const void* codes, const void* codebooks, const void* scales,
                       const void* x, void* y, int M, int B, int g,
                       int64_t out, int64_t in, int64_t batch, void* stream);

/* ---------------------------------------------------------------------------
 * Bit-packed codes ("Key AQLM quantization parameters" on the same page: a B
 * that is not a multiple of 8 leaves unused bits in the bytes that hold each
 * code; packing drops them, so e.g. (1, 12, 4) stores 3 bits per weight in its
 * codes instead of 4).  Packed layout: the codes in their stored order
 * ([out][in/g][M] flattened, code n = (i * in/g + j) * M + m) form one bit
 * stream, code n in bits [n B, n B + B), least significant bit first; bit b is
 * bit b % 32 of 32-bit word b / 32 (little-endian words); the stream is padded
 * with zero bits to a whole word.  Rows are not padded (a row may start inside
 * a word).  The buffer holds aqlm_packed_codes_bytes bytes and is 4-byte
 * aligned.
 *
 * aqlm_linear_{gemv,gemm,decode}_packed take such a stream as `codes` and
 * otherwise the arguments, validation and results of aqlm_linear_{gemv,gemm,
 * decode} (decode bit-exact; every scheme of AQLM_ERR_SCHEME's range runs the
 * general kernels); a misaligned stream gives AQLM_ERR_ALIGN.  aqlm_pack_codes
 * writes the stream of whole-byte codes [out][in/g][M] (the low B bits of each
 * stored code; every word of the stream, padding bits zero).
 */
int aqlm_packed_codes_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes);
int aqlm_pack_codes(const void* codes, void* packed, int M, int B, int g, int64_t out, int64_t in, void* stream);
int aqlm_linear_gemv_packed(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                            int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream);
int aqlm_linear_gemm_packed(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                            int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream);
int aqlm_linear_decode_packed(const void* codes, const void* codebooks, const void* scales, const void* x, void* y,
                              int M, int B, int g, int64_t out, int64_t in, int64_t batch, void* stream);

/* ---------------------------------------------------------------------------
 * Building the representation ("The AQLM quantization procedure" on the same
 * page: per layer, the codes are learned first with fixed codebooks that a
 * residual k-means initialises).  The page's learning loss is lost and needs
 * calibration data; these are its data-free counterparts on plain weights:
 *
 *   target of a group    W[i][j*g .. j*g+g) / s_i, one fp32 division each;
 *   code of codebook m   the nearest codeword (squared Euclidean distance,
 *                        sum_t (r_t - c_t)^2 in fp32, t ascending, no fused
 *                        multiply-add, lowest index on a tie) to the target
 *                        minus the codewords chosen for codebooks 0 .. m-1.
 *
 * w is [out][in] fp16 (16-byte aligned), scales [out] fp16 (the page does not
 * say how scales are initialised; the caller gives them), codes and
 * codebooks as above.  Both calls accept every scheme the products accept.
 * out == 0 enqueues nothing.  Results are deterministic and bit-identical to
 * the plain CPU definition.
 */

/* Greedy residual codes for w with the given codebooks; writes codes. */
int aqlm_encode_greedy(const void* w, const void* scales, const void* codebooks, void* codes,
                       int M, int B, int g, int64_t out, int64_t in, void* stream);

/* Largest iteration count aqlm_kmeans_init accepts. */
#define AQLM_KMEANS_MAX_ITERS 10000

/* Bytes of device workspace aqlm_kmeans_init needs for the scheme (into *bytes). */
int aqlm_kmeans_workspace_bytes(int M, int B, int g, int64_t* bytes);

/*
 * Residual k-means: for m = 0 .. M-1, Lloyd's algorithm (`iters` rounds of
 * assign + update) on what codebooks 0 .. m-1 leave of every group's target,
 * seeded with the leftovers of groups seeds[m][0 .. 2^B-1] (device int64
 * [M][2^B], group index = row * in/g + j, clamped into range); writes the fp16
 * codebooks [M][2^B][g] and the codes of the greedy encoding against them.
 * A centroid is the mean of its members, summed exactly as integers in units
 * of 2^-24 and divided in float64, then rounded to fp32; an empty cluster
 * keeps its centroid; codebook m is the fp16 rounding of the centroids.  The
 * sums are exact while every target satisfies |W/s| < 2^29 / n_groups
 * (n_groups = out * in / g; e.g. |W/s| < 256 with 2^21 groups).  A target at
 * or above that bound, or not finite, cannot be summed exactly: the call then
 * does not produce wrapped sums but NaN codebooks (from the first k-means round
 * that meets such a target on; every later codebook too), and the codes
 * assigned against them are 0.  `workspace` is caller-owned device memory of
 * at least aqlm_kmeans_workspace_bytes bytes (16-byte aligned); its contents
 * on entry do not matter.
 */
int aqlm_kmeans_init(const void* w, const void* scales, const int64_t* seeds, void* codebooks, void* codes,
                     void* workspace, int64_t workspace_bytes, int M, int B, int g,
                     int64_t out, int64_t in, int iters, void* stream);

/* ---------------------------------------------------------------------------
 * 1x16 at batch 1 over slice lists ("Key AQLM quantization parameters" on the
 * same page: 1x16 is the scheme with 2^16 codewords, and its decoding is the
 * slower one because of them).  The product above gathers a 16-byte codeword
 * per code from the 1 MiB codebook; these calls instead regroup the codes of
 * a layer once, at load time, so that a workgroup can keep one eighth of the
 * codebook (8192 codewords, 128 KB) in LDS and read only the codes that fall
 * in it.  Only (M, B, g) = (1, 16, 8) (else AQLM_ERR_SCHEME); 8 <= in <=
 * AQLM_MAX_IN, in % 8 == 0, out <= AQLM_LISTS_MAX_OUT and out * in/8 <=
 * 2^32 - 1 (else AQLM_ERR_SHAPE).
 *
 * Layout (all device memory, 16-byte aligned, owned by the caller):
 *   rows form tiles of 64; the groups j of a row form J = ceil(G / 1024)
 *   blocks of Gb = ceil(G / J) groups (G = in / 8); for every unit
 *   u = (s * J + k) * ceil(out / 64) + rt (slice s < 8, block k, row tile
 *   rt), row 64 rt + l lists its codes c with c >> 13 == s and j in block k,
 *   ascending in j, as uint32 entries ((j - k Gb) << 13) | (c & 8191); the
 *   64 lists are padded to the longest, L, with Z << 13 (Z = Gb rounded up
 *   to a multiple of 64) and stored as entries[(off + t) * 64 + l].
 *   table: uint32 pairs (off, L) per unit, then the total number of steps
 *   (sum of L) as a uint64; entries take 256 bytes per step.
 *
 * Building: aqlm_lists_plan(codes, table) writes the table (asynchronous);
 * the caller reads the total (the uint64 at byte aqlm_lists_table_bytes - 8)
 * after synchronising, allocates total * 256 bytes of entries and calls
 * aqlm_lists_fill.  A fill or product whose entries_bytes is smaller than a
 * unit's off + L needs leaves that unit out (no access beyond entries_bytes);
 * a table that does not belong to the codes gives wrong results, never an
 * access outside the buffers.  The product needs a caller workspace of
 * aqlm_lists_workspace_bytes (fp32 partial sums, overwritten by every call;
 * calls that share a workspace must not run concurrently).
 *
 * Result: y = W x for batch 1 (batch 0 enqueues nothing), accumulated in
 * fp32, rounded to fp16 once; deterministic (the summation order is fixed by
 * out and in), but not bit-identical to aqlm_linear_gemv, which adds in
 * another order.
 */
#define AQLM_LISTS_MAX_OUT (1 << 30)

/* Bytes of the table of a layer (into *bytes). */
int aqlm_lists_table_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes);
/* Bytes of workspace aqlm_linear_gemv_lists needs for the shape (into *bytes). */
int aqlm_lists_workspace_bytes(int M, int B, int g, int64_t out, int64_t in, int64_t* bytes);
/* Writes the table of codes [out][in/8] (int16) into table.  codes may be NULL when out == 0. */
int aqlm_lists_plan(const void* codes, void* table, int M, int B, int g, int64_t out, int64_t in, void* stream);
/* Writes the entries of codes, placed by table, into entries (entries_bytes long). */
int aqlm_lists_fill(const void* codes, const void* table, void* entries, int64_t entries_bytes, int M, int B, int g,
                    int64_t out, int64_t in, void* stream);
/* y[0][i] = sum_k W[i][k] x[0][k] over the slice lists (codebooks, scales, x, y as for aqlm_linear_gemv). */
int aqlm_linear_gemv_lists(const void* table, const void* entries, int64_t entries_bytes, const void* codebooks,
                           const void* scales, const void* x, void* y, void* workspace, int64_t workspace_bytes, int M,
                           int B, int g, int64_t out, int64_t in, int64_t batch, void* stream);

/*
 * n_layers slice-list products that share x (q/k/v, gate/up) in one launch of
 * the product and one of the reduction: y_l = W_l x for l < n_layers, batch 1.
 * tables, entries, entries_bytes, codebooks, scales, outs and ys are HOST
 * arrays of n_layers entries (pointers in them are device pointers, laid out
 * as for aqlm_linear_gemv_lists); the library reads them during the call.
 * Each layer is validated as by aqlm_linear_gemv_lists; a layer with
 * outs[l] == 0 is skipped.  workspace (16-byte aligned) holds the layers'
 * partial sums one after another, each rounded up to 256 bytes:
 * aqlm_lists_fused_workspace_bytes gives its size.  Results are bit-identical to separate aqlm_linear_gemv_lists calls.
 * 1 <= n_layers <= AQLM_FUSED_MAX_LAYERS (else AQLM_ERR_SHAPE); a NULL array
 * gives AQLM_ERR_NULL.
 */
int aqlm_linear_gemv_lists_fused(int n_layers, const void* const* tables, const void* const* entries,
                                 const int64_t* entries_bytes, const void* const* codebooks, const void* const* scales,
                                 const int64_t* outs, const void* x, void* const* ys, void* workspace,
                                 int64_t workspace_bytes, int M, int B, int g, int64_t in, int64_t batch,
                                 void* stream);
/* Bytes of workspace aqlm_linear_gemv_lists_fused needs for the layers' outs (host array). */
int aqlm_lists_fused_workspace_bytes(int n_layers, const int64_t* outs, int M, int B, int g, int64_t in,
                                     int64_t* bytes);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): aqlm_linear_gemv_lists
 * without the workspace argument.  The fp32 partial sums go to a static device
 * array of the library, AQLM_LISTS_NOALLOC_SCRATCH_BYTES long, that every GPU the
 * library runs on holds until the process ends; the call allocates and frees
 * nothing (its first call on a device looks the array's address up once).  A
 * layer whose partial sums (aqlm_lists_workspace_bytes) exceed the array gives
 * AQLM_ERR_SCRATCH and enqueues nothing; 4 MiB covers e.g. every Llama-2-7B and
 * 70B projection.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  Each call writes every partial it reads, so the
 * array needs no clearing between calls.  Other arguments, validation and
 * results are those of aqlm_linear_gemv_lists (bit-identical to it).
 */
#define AQLM_LISTS_NOALLOC_SCRATCH_BYTES (4 << 20)
int aqlm_linear_gemv_lists_noalloc(const void* table, const void* entries, int64_t entries_bytes,
                                   const void* codebooks, const void* scales, const void* x, void* y, int M, int B,
                                   int g, int64_t out, int64_t in, int64_t batch, void* stream);

/* Static, human-readable name of a status code. */
const char* aqlm_status_str(int status);

/* hipError_t of the calling thread's last AQLM_ERR_HIP (0 if none). */
int aqlm_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* aqlm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AQLM_H */
