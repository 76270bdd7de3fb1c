/*
 * tb.h - C ABI of libtb, inference with Hadamard-rotated ternary weights on
 * AMD Instinct MI355X (gfx950).
 *
 * Method (cited by page address and the page's own section numbers):
 *   - Activations get a blockwise 128-point Walsh-Hadamard transform along K,
 *     normalised by 1/sqrt(128) (xxqk.cn/news/652513 §2; dpshk.com/news/5289456
 *     §2.1 and §2.3; mhpq.cn/news/1159370 §2.2).
 *   - Weights are stored as {-1, 0, +1} codes with one fp16 scale per 128
 *     consecutive K-elements (mhpq.cn/news/1159370 §1.1, §1.3, §3.1); an
 *     optional 2:4 variant keeps two of every four (same page, §1.2).
 *   - The offline quantiser applies H.W.H^T / 128 to every 128x128 block, takes
 *     the group's mean absolute value as its scale and ternarises by dividing,
 *     rounding and clipping (mhpq.cn §1.1; dpshk.com §3.2 steps 3-5).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers, owned by the caller, contiguous
 *     and row-major, with base addresses aligned to 16 bytes.  Nothing is
 *     retained after return.
 *   - `stream` is a hipStream_t passed as a plain pointer (NULL = the default
 *     stream).  Work is enqueued on it asynchronously; the library never
 *     synchronises, never allocates device memory and never prints.  Outputs
 *     are valid once the stream has completed the call.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is enqueued and the status says why.  Validation touches no
 *     GPU state, so it can be exercised on a machine without a GPU.
 *   - Weight matrices are W[N][K] (out x in, y = W x); N and K must be positive
 *     multiples of 128.  A batch dimension of 0 (rows, B, M) is a valid no-op.
 *   - Calls are re-entrant and thread-safe; concurrent calls on different
 *     streams are independent.
 *
 * Storage formats (bit exact, shared by the quantiser and the products):
 *   Dense codes  uint32 codes[N/16][K/128][128], one 128-word tile per 16 rows
 *                x 128 columns.  In tile (nb, g), word 2l + h (l = 16q + i,
 *                q = 0..3, h = 0..1) holds row 16nb + i, columns
 *                128g + 32q + 16h + r for r = 0..15, the 2-bit field of r at
 *                bit 4*(r%8) + 2 - 2*(r/8).  Field: 0b00 = 0, 0b01 = +1,
 *                0b11 = -1 (bit 0 nonzero, bit 1 negative); 0b10 never
 *                appears.  (Two bits per weight: mhpq.cn/news/1159370 §3.1;
 *                the arrangement is this library's, chosen so that two AND
 *                masks turn a word into the fp4 operand of the gfx950
 *                block-scaled matrix instruction.)
 *   Scales       uint16 fp16 bits, one per row and 128-group: the group's
 *                absmean, rounded to nearest even.  Dense formats store them
 *                tile-major like the codes, scales[N/16][K/128][16]: the scale
 *                of row n, group g at ((n/16)*(K/128) + g)*16 + n%16 (a 16-row
 *                tile's scales for one group are 32 contiguous bytes).
 *   2:4 format   Lane-major in blocks of four 128-groups: a 16-row tile nb
 *                and block b (groups 4b .. 4b+3; G4 = ceil(K/512) blocks, the
 *                groups of the last block past K/128 stored as zeros) hold,
 *                for lane l = 16w + i (row i of the tile, w = 0..3), what
 *                lane l of a wave needs for the quads 32g + 8w .. 32g + 8w + 7
 *                (q = k/4) of each group g of the block:
 *   2:4 meta     uint32 meta[N/16][G4][64][4]: [nb][b][l][j] is the meta word
 *                of row 16nb + i for those quads of group g = 4b + j: the
 *                nibble at bits 4*(q%8) holds idx0 (bits 0-1) and idx1 (bits
 *                2-3), idx0 < idx1, the kept positions inside the quad.
 *   2:4 signs    uint32 signs[N/16][G4][64][2]: the 16-bit sign field of lane
 *                l and group g = 4b + 2p + h in half h (bits 16h .. 16h+15) of
 *                [nb][b][l][p]: bit q%8 set when the element kept at idx0 of
 *                quad q is negative, bit 8 + q%8 for idx1.
 *   2:4 scales   uint16 fp16 bits scales[N/16][G4][4][4][4]: [nb][b][w][j][r]
 *                is the scale of row 16nb + 4w + r in group 4b + j.
 *                A lane reads its four meta words with one 16-byte load, its
 *                eight sign bytes with one 8-byte load, and the scales of its
 *                output rows from a 128-byte block record.
 */
#ifndef TB_H
#define TB_H

#include <stddef.h>
#include <stdint.h>

/* Symbols of the C ABI; everything else in the library is hidden. */
#define TB_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TB_OK = 0,
  TB_ERR_NULL = 1,        /* a required pointer is NULL                         */
  TB_ERR_SHAPE = 2,       /* N or K not a positive multiple of 128, bad batch   */
  TB_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                   */
  TB_ERR_DTYPE = 4,       /* unknown dtype enum value                           */
  TB_ERR_FORMAT = 5,      /* unknown format, or a plane given/missing for it    */
  TB_ERR_LAUNCH = 6,      /* the HIP runtime refused the launch                 */
  TB_ERR_UNSUPPORTED = 7, /* valid request this build does not implement        */
  TB_ERR_ALIAS = 8,       /* input and output overlap where that is not allowed */
  TB_ERR_WORKSPACE = 9    /* workspace missing or smaller than the call needs   */
} tb_status;

typedef enum { TB_F32 = 0, TB_BF16 = 1, TB_ACT8 = 2 } tb_dtype;
/* Quantiser rules and storage formats.  TB_FMT_DENSE_MINERR stores the dense
 * format; only the threshold and scale rule differ (tb_quantize_pack).
 * TB_FMT_DENSE_RESID stores two dense planes with their 128-groups
 * interleaved along K (the two-plane format, see tb_quantize_pack). */
typedef enum { TB_FMT_DENSE = 0, TB_FMT_24 = 1, TB_FMT_DENSE_MINERR = 2, TB_FMT_DENSE_RESID = 3 } tb_format;

/* Bits OR-ed into the optional device error flag of tb_quantize_pack. */
/* TB_EFLAG_NONFINITE: a non-finite weight was seen (or a block's transform
 * overflowed fp32); that block's codes are unspecified. */
#define TB_EFLAG_NONFINITE 1u
#define TB_EFLAG_SCALE_OVF 2u /* a group scale rounded to fp16 infinity (absmean >= 65520)      */

/*
 * TB_ACT8 is the activation operand of the dense GEMV's matrix instruction,
 * for B rows of K activations, in one buffer of tb_act8_bytes(B, K) =
 * 4*B*K + B*K/8 bytes.  tb_ternary_gemv encodes bf16 activations into it
 * itself (in a caller workspace), or takes it already encoded.  An activation
 * is written as the sum of up to four e4m3 values on four sub-rows (two
 * magnitude levels x high and low significand halves) with one E8M0 scale per
 * 32 K-elements and sub-row; the sum is exact for every element the two levels
 * cover (see below), the rest are read as zero:
 *   values  uint8 [B][K/128][2 halves h][4 sub-rows][4 q][16]: the 16 bytes
 *           of (h, q) are K 128g + 64h + 16q + (0..15);
 *   scales  uint8 at byte offset 4*B*K: [B][K/128][4 sub-rows][4 blocks],
 *           block q = K 128g + 32q .. +31; 0xFF marks a block holding a
 *           non-finite activation (the product rows then come out NaN).
 * Sub-rows 0/1 take the elements within 10 binades of their block's largest,
 * sub-rows 2/3 those within 10 binades of the largest of the rest.  Elements
 * below both, and bf16 subnormals, are read as zero: each such element is
 * below 2^-20 of its block's largest magnitude.
 */

/* Largest activation batch of the GEMV entry points. */
#define TB_GEMV_MAX_BATCH 16

/* Most segments one grouped call (tb_fwht128_multi, tb_ternary_gemv_multi) takes. */
#define TB_MAX_SEGMENTS 8

/* Longest K the GEMM entry points take (tb_ternary_gemm and its variants;
 * longer K returns TB_ERR_SHAPE): their kernels address a workgroup's
 * activation rows with 32-bit offsets. */
#define TB_GEMM_MAX_K ((int64_t)1 << 24)

/* Most K parts of one GEMV segment (tb_gemv_segment.parts) and most partial
 * inputs of one rotation segment (tb_fwht_segment.x_parts). */
#define TB_MAX_PARTS 8

/* One array of a grouped tb_fwht128_multi call: arguments as in tb_fwht128,
 * each segment with its own input and output dtypes.
 * x_parts (0 or 1: x is [rows][K]) greater than 1 makes x the x_parts
 * partial results [x_parts][rows][K] of a split product (tb_gemv_segment
 * with parts = x_parts): they are added in part order, in fp32, and the sum
 * is transformed, so the reduction of the split GEMV costs no launch of its
 * own.  Only with x_dtype TB_F32, at most TB_MAX_PARTS, and y must not overlap
 * any part (else TB_ERR_DTYPE, TB_ERR_SHAPE, TB_ERR_ALIAS). */
typedef struct {
  const void* x;
  void* y;
  int64_t rows;
  int64_t K;
  int x_dtype;
  int y_dtype;
  int x_parts;
  int reserved;  /* must be 0 */
} tb_fwht_segment;

/* One product of a grouped tb_ternary_gemv_multi call: arguments as in
 * tb_ternary_gemv.  `planes` is 1 for the one-plane dense formats (0 is read
 * as 1) and 2 for two-plane codes and scales (TB_FMT_DENSE_RESID, as
 * tb_ternary_gemv_resid takes them); anything else returns TB_ERR_FORMAT.
 * `parts` (0 or 1: y is [B][N]) of 2, 4 or 8 splits the product's K over
 * that many workgroups per 16-row tile, for a long-K product with too few
 * tiles to fill the GPU (a 27B layer's down projection: 320 tiles): y is
 * then [parts][B][N], part p holding the sum over the scale groups
 * [floor(G p / parts), floor(G (p + 1) / parts)) (G = K/128 per plane times
 * planes), so the product is the sum of the parts in part order.
 * tb_fwht128_multi adds them on the way into the output rotation
 * (tb_fwht_segment.x_parts).  G >= parts (else TB_ERR_SHAPE). */
typedef struct {
  const uint8_t* act;
  int64_t B;
  const uint32_t* codes;
  const uint16_t* scales;
  int64_t N;
  int64_t K;
  float* y;
  int64_t planes;
  int64_t parts;
} tb_gemv_segment;

/* One product of a grouped tb_ternary24_gemv_multi call: arguments as in
 * tb_ternary24_gemv. */
typedef struct {
  const uint16_t* x;
  const uint32_t* meta;
  const uint32_t* signs;
  const uint16_t* scales;
  float* y;
  int64_t B;
  int64_t N;
  int64_t K;
} tb_gemv24_segment;

/* One product of a grouped tb_ternary_gemm_multi call: arguments as in
 * tb_ternary_gemm. */
typedef struct {
  const uint16_t* x;
  const uint32_t* codes;
  const uint16_t* scales;
  void* y;
  int64_t M;
  int64_t N;
  int64_t K;
  int y_dtype;
  int reserved; /* must be 0 */
} tb_gemm_segment;

/* Human-readable name of a status code (static storage, never NULL). */
TB_API const char* tb_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
TB_API int tb_version(void);

/*
 * Sizes in bytes of the packed planes of an [N][K] matrix in format `fmt`
 * (tb_format).  Dense (both rules): code_bytes = N*K/4, meta_bytes = 0,
 * scale_bytes = N*K/64.  2:4, with K' = K rounded up to a multiple of 512
 * (whole blocks of four groups): code_bytes (the sign plane) = N*K'/16,
 * meta_bytes = N*K'/8, scale_bytes = N*K'/64.  Two-plane
 * (TB_FMT_DENSE_RESID): code_bytes = N*K/2, meta_bytes = 0, scale_bytes =
 * N*K/32.  Any output pointer may be NULL.  Host-only.
 * Cites the 2-bit storage of mhpq.cn/news/1159370 §3.1 and the bit ledger of §1.3.
 */
TB_API tb_status tb_packed_bytes(int fmt, int64_t N, int64_t K, size_t* code_bytes, size_t* meta_bytes,
                          size_t* scale_bytes);

/*
 * Blockwise 128-point orthonormal Walsh-Hadamard transform along K:
 *   y[r][128b + i] = (1/sqrt(128)) * sum_j (-1)^popcount(i & j) * x[r][128b + j]
 * (xxqk.cn/news/652513 §2: log2(n) rounds of (a+b, a-b) butterflies;
 * dpshk.com/news/5289456 §2.1: H[i][j] = (-1)^popcount(i&j), 128-blocks;
 * §2.3: scale 1/sqrt(block size)).  Used on activations before the products
 * and, along N, to rotate an output back (the transform is its own inverse).
 *   x      [rows][K] in x_dtype (TB_BF16 or TB_F32)
 *   y      [rows][K] in y_dtype; bf16 output is rounded to nearest even.
 *          TB_ACT8 writes the rounded bf16 result as the activation operand of
 *          tb_ternary_gemv (tb_act8_bytes(rows, K) bytes), which fuses the
 *          rotation of the activations with their encoding.
 *          y == x is allowed (in place) when the dtypes match; any other
 *          overlap returns TB_ERR_ALIAS.
 *   rows >= 0, K a positive multiple of 128.  Arithmetic is fp32.
 */
TB_API tb_status tb_fwht128(const void* x, int x_dtype, void* y, int y_dtype, int64_t rows, int64_t K,
                     void* stream);

/*
 * tb_fwht128 over up to TB_MAX_SEGMENTS independent arrays in one launch (the
 * activations of several projections, their outputs, or one layer's outputs
 * together with the next layer's inputs); same transform and rules per
 * segment, each with its own x_dtype / y_dtype (a segment's result does not
 * depend on what it is grouped with).  `segs` is a host array read during
 * the call.  Segments must not overlap one another except a segment rotating
 * in place.  count == 0 is a no-op; count outside [0, TB_MAX_SEGMENTS]
 * returns TB_ERR_SHAPE.
 */
TB_API tb_status tb_fwht128_multi(const tb_fwht_segment* segs, int count, void* stream);

/*
 * Offline quantise and pack (mhpq.cn/news/1159370 §1.1-§1.3, §3.1;
 * dpshk.com/news/5289456 §3.2 steps 3-5):
 *   W'  = H B H^T / 128 for every 128x128 block B of W,
 *   s   = mean |W'| over each 128-group (one row of one block),
 *   t   = +1 if W' > s/2, -1 if W' < -s/2, else 0 (dense), written as codes,
 *   scale = fp16(s).
 * TB_FMT_24 first keeps, in every quad of 4 along K, the two largest |W'|
 * (ties to the lower position), takes s over the 64 kept elements of each
 * group and stores their signs (mhpq.cn §1.2).
 * TB_FMT_DENSE_MINERR (dense storage) chooses each group's threshold and
 * scale to minimise ||W' - s t||^2 (the threshold as the accuracy-critical
 * knob, xxqk.cn/news/652513 §3, its per-block threshold search): over the
 * group's magnitudes theta, the kept set {|W'| >= theta} with the largest
 * S^2 / j (S the sum of its magnitudes, j its size), t = sign(W') on it,
 * s = S / j; ties go to the larger theta.
 * The 0.38-quantile threshold of dpshk.com §3.2 step 4 is one of the
 * candidates (it keeps the largest 79 of 128).
 * TB_FMT_DENSE_RESID adds a second ternary plane for what the first misses
 * (the residual calibration of xxqk.cn/news/652513 §3): plane 1 is the
 * absmean rule above; the residual d = W' - fp16(s1) t1 (against the stored
 * scale, in the rotated basis) is ternarised by the same rule, giving
 * W' ~ fp16(s1) t1 + fp16(s2) t2.  Storage: the dense format of both planes
 * with their groups interleaved, codes [N/16][2K/128][128] and scales
 * [N/16][2K/128][16], where group 2g + p is plane p's group g.
 *   W       fp32 [N][K]
 *   codes   dense: [N/16][K/128][128] code words (the tile layout above);
 *           two-plane: [N/16][2K/128][128]; 2:4: the sign plane [N/16][G4][64][2]
 *   meta    2:4: [N/16][G4][64][4] (G4 = ceil(K/512)); must be NULL for the
 *           dense formats (else TB_ERR_FORMAT)
 *   scales  fp16 bits; dense: [N/16][K/128][16] (tile-major, above);
 *           two-plane: [N/16][2K/128][16]; 2:4: [N/16][G4][4][4][4]
 *           (2:4 groups past K/128 in the last block are written as zeros)
 *   err_flag  NULL, or a device int32 the kernels OR TB_EFLAG_* bits into
 *             (the caller zeroes it first).
 * Arithmetic is fp32; the absmean threshold uses the unrounded scale.
 */
TB_API tb_status tb_quantize_pack(const float* W, int64_t N, int64_t K, int fmt, uint32_t* codes,
                           uint32_t* meta, uint16_t* scales, int32_t* err_flag, void* stream);

/*
 * Decode GEMV with dense ternary weights (mhpq.cn/news/1159370 §4.2: read the
 * weight bits, expand the signs, apply the scale, multiply):
 *   y[b][n] = sum_g fp16(scales[n][g]) * sum_{k in g} t[n][k] * x[b][k]
 *   x, x_dtype  the already rotated activations x' [B][K], either
 *           TB_BF16: bf16 bits [B][K].  The call first encodes them as the
 *             TB_ACT8 operand into `workspace` (one launch), then runs the
 *             product (a second launch on the same stream);
 *           TB_ACT8: the operand already encoded, tb_act8_bytes(B, K) bytes
 *             for exactly these B rows (its scales start at byte 4*B*K, so
 *             the operand of more rows cannot be passed with a smaller B);
 *             made by tb_act8_prep or by tb_fwht128 with y_dtype TB_ACT8.
 *             One launch; `workspace` is not used and may be NULL.
 *           Other dtypes return TB_ERR_DTYPE.
 *   B       0 <= B <= TB_GEMV_MAX_BATCH (else TB_ERR_SHAPE)
 *   codes, scales  dense format, [N/16][K/128][128] and [N/16][K/128][16]
 *   y       fp32 [B][N]; must not overlap the inputs (TB_ERR_ALIAS)
 *   workspace, workspace_bytes  for TB_BF16: caller-owned device memory of at
 *           least tb_act8_bytes(B, K) bytes (else TB_ERR_WORKSPACE), 16-byte
 *           aligned, overlapping no other argument (TB_ERR_ALIAS); it holds
 *           the encoded operand when the call completes.  Calls sharing a
 *           workspace must be ordered on one stream.
 * The products are exact; each 32-element block's products are summed
 * exactly inside the matrix instruction, blocks, sub-rows and groups are
 * accumulated in fp32.  Activations more than 20 binades below their
 * 32-block's largest, and bf16 subnormals, are read as zero (TB_ACT8 above).
 */
TB_API tb_status tb_ternary_gemv(const void* x, int x_dtype, int64_t B, const uint32_t* codes, const uint16_t* scales,
                          int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device array tb_ternary_gemv_noalloc encodes its activations
 * into: it takes B and K with tb_act8_bytes(B, K) <= this (B = 16 with
 * K <= 63488, B = 1 with K <= 1016704). */
#define TB_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * tb_ternary_gemv with bf16 activations for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation): the same product and the same kernels,
 * but the act8 encoding of x goes to an array the library holds on each GPU
 * (TB_NOALLOC_SCRATCH_BYTES, held until the process ends) instead of a
 * caller workspace.  The call allocates and frees nothing.
 *   x       bf16 bits [B][K], the already rotated activations
 *   B, codes, scales, N, K, y and the error rules as tb_ternary_gemv;
 *   tb_act8_bytes(B, K) > TB_NOALLOC_SCRATCH_BYTES returns TB_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (different streams, or different host threads without
 * ordering) race and must be serialised by the caller.  The result is that of
 * tb_ternary_gemv with TB_BF16 bit for bit.  Two launches on the stream.
 */
TB_API tb_status tb_ternary_gemv_noalloc(const uint16_t* x, int64_t B, const uint32_t* codes, const uint16_t* scales,
                                  int64_t N, int64_t K, float* y, void* stream);

/*
 * tb_ternary_gemv over up to TB_MAX_SEGMENTS independent products in one
 * launch (e.g. the projections of a layer, so that small matrices do not leave
 * the GPU idle), each given its TB_ACT8 operand (`act`, as tb_ternary_gemv
 * with x_dtype TB_ACT8); each segment is validated and computed as tb_ternary_gemv,
 * and its result is bit for bit that of the single call (how a segment's sum is
 * split and ordered depends only on its own shape, batch and parts).  The
 * launch schedules the longest-K segments first; the order of `segs` does not
 * change any result.
 * A segment with parts > 1 writes its parts instead of the product (see
 * tb_gemv_segment; y then spans parts * B * N floats).
 * `segs` is a host array read during the call; no segment's y may overlap any
 * segment's inputs or another y.  count == 0 is a no-op; count outside
 * [0, TB_MAX_SEGMENTS] returns TB_ERR_SHAPE.
 */
TB_API tb_status tb_ternary_gemv_multi(const tb_gemv_segment* segs, int count, void* stream);

/*
 * Decode GEMV with two-plane dense ternary weights (TB_FMT_DENSE_RESID, the
 * residual calibration of xxqk.cn/news/652513 §3):
 *   y[b][n] = sum_g sum_p fp16(s_p[n][g]) * sum_{k in g} t_p[n][k] * x[b][k]
 *   codes   [N/16][2K/128][128], scales [N/16][2K/128][16]: group 2g + p is plane
 *           p's group g (as tb_quantize_pack writes them)
 *   x, x_dtype, B, y, workspace and the error rules as tb_ternary_gemv; K is
 *   the activation length.  Both planes' products are exact and accumulated
 *   in fp32.
 */
TB_API tb_status tb_ternary_gemv_resid(const void* x, int x_dtype, int64_t B, const uint32_t* codes,
                                const uint16_t* scales, int64_t N, int64_t K, float* y, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Bytes of the TB_ACT8 activation operand for B rows of K activations:
 * 4*B*K + B*K/8.  Host-only; 0 when K is not a positive multiple of 128 or
 * B < 0.
 */
TB_API size_t tb_act8_bytes(int64_t B, int64_t K);

/*
 * Encode bf16 activations x[B][K] (already rotated) as the TB_ACT8 operand of
 * tb_ternary_gemv, without transforming them.  B >= 0 (0 is a no-op), K a
 * positive multiple of 128; act must not overlap x.
 */
TB_API tb_status tb_act8_prep(const uint16_t* x, int64_t B, int64_t K, uint8_t* act, void* stream);

/*
 * Decode GEMV with 2:4 ternary weights (mhpq.cn/news/1159370 §1.2):
 *   y[b][n] = sum_g fp16(scales[n][g]) * sum_q (+-x[b][4q + idx0] +- x[b][4q + idx1])
 *   x       bf16 bits [B][K], the already rotated activations
 *   meta [N/16][G4][64][4], signs [N/16][G4][64][2], scales
 *   [N/16][G4][4][4][4] in the (lane-major) 2:4 format, G4 = ceil(K/512);
 *   the padded groups of the last block are never read;
 *   B and y as tb_ternary_gemv.  Products are exact, accumulation is fp32.
 */
TB_API tb_status tb_ternary24_gemv(const uint16_t* x, int64_t B, const uint32_t* meta, const uint32_t* signs,
                            const uint16_t* scales, int64_t N, int64_t K, float* y, void* stream);

/*
 * tb_ternary24_gemv over up to TB_MAX_SEGMENTS independent products in one
 * launch (a decoder layer's projections: the launch is long enough to keep
 * HBM streaming, where a single product leaves it idle while the launch
 * fills and drains).  Same contraction, rules and accuracy per segment; how
 * a product's K is split over waves (and so the fp32 summation order)
 * depends on the segments it is grouped with; a single segment is the
 * single call.  Segments with B > 4 make the call launch each product on its
 * own.  `segs` is a host array read during
 * the call; no segment's y may overlap any segment's inputs or another y.
 * count == 0 is a no-op; count outside [0, TB_MAX_SEGMENTS] returns
 * TB_ERR_SHAPE.
 */
TB_API tb_status tb_ternary24_gemv_multi(const tb_gemv24_segment* segs, int count, void* stream);

/*
 * Prefill GEMM with dense ternary weights, the same contraction as
 * tb_ternary_gemv for M rows of activations:
 *   y[m][n] = sum_g fp16(scales[n][g]) * sum_{k in g} t[n][k] * x[m][k]
 *   x       bf16 bits [M][K], M >= 0 (any M; ragged tails are handled)
 *   codes, scales  dense format, [N/16][K/128][128] and [N/16][K/128][16]
 *   y       [M][N] in y_dtype: TB_BF16 (rounded to nearest even) or TB_F32;
 *           must not overlap the inputs.
 * The matrix cores take the activations as the bf16 values they are and each
 * weight as the exact bf16 value 2t; every product is exact and sums are
 * fp32.  Per output column the running sum is kept in units of the last
 * nonzero group scale: a group with scale s rescales it by (previous unit) /
 * s, rounded to fp32 (exact when the scales are powers of two), and then
 * adds its products; a zero-scale group adds nothing.  The result is
 * multiplied by the last unit and halved on the way out.
 * M <= 16 runs a kernel of its own (one pass over K for at most 16 rows,
 * weights decoded in registers); a row's result depends on its activations,
 * N and K only, not on M.  K at most TB_GEMM_MAX_K (else TB_ERR_SHAPE).
 */
TB_API tb_status tb_ternary_gemm(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                          int64_t N, int64_t K, void* y, int y_dtype, void* stream);

/*
 * tb_ternary_gemm over up to TB_MAX_SEGMENTS independent products.  When
 * every segment has M <= 16 they run as one launch of the mid-batch kernel
 * (a decoder layer's products at a small batch: the launch is long enough to
 * keep HBM streaming); otherwise each product is launched on its own.  Same
 * contraction and accuracy per segment; in the one launch a product's K
 * slices (and so its fp32 summation order) follow from the whole group's
 * size, and a single segment is the single call.  `segs` is a host array read during the call; no segment's y may
 * overlap any segment's inputs or another y; `reserved` must be 0 (else
 * TB_ERR_SHAPE).  count == 0 is a no-op; count outside [0, TB_MAX_SEGMENTS]
 * returns TB_ERR_SHAPE.
 */
TB_API tb_status tb_ternary_gemm_multi(const tb_gemm_segment* segs, int count, void* stream);

/*
 * Bytes of workspace tb_ternary_gemm_splitk and tb_ternary_gemm_rotated use
 * for an [M][N] result with K-long rows: S * M * N * 4 for the S splits of K
 * they choose (from a time model of the kernel: at most 16 splits, at least
 * one 128-group each), or 0 when one pass suffices (S = 1) or the sizes are
 * invalid.  For M <= 16 only the rotated GEMM splits K.
 * Host-only.
 */
TB_API size_t tb_ternary_gemm_splitk_workspace(int64_t M, int64_t N, int64_t K);

/*
 * tb_ternary_gemm for few rows of activations (M = 16-256, between decode and
 * prefill).  M <= 16 runs tb_ternary_gemm's kernel for such M (one pass, the
 * workspace unused, the same result bit for bit).  Above that one pass over K
 * leaves too few output tiles to fill the GPU: K is cut into S splits at
 * 128-group boundaries, each split's fp32
 * partial product goes to `workspace` ([S][M][N] fp32), and a second kernel
 * adds the partials in split order and writes y (bf16 rounded to nearest
 * even, or fp32).  The same contraction and error rules as tb_ternary_gemm;
 * the sums are grouped by split, so the fp32 result may differ from
 * tb_ternary_gemm's in the last bits.
 *   workspace  device memory of workspace_bytes bytes, caller-owned; S is
 *              reduced to what fits (S <= workspace_bytes / (M*N*4)); with
 *              room for fewer than two partials (or NULL) the call runs as
 *              tb_ternary_gemm.  Must not overlap any other argument
 *              (TB_ERR_ALIAS).  Calls sharing a workspace must be ordered on
 *              one stream.
 */
TB_API tb_status tb_ternary_gemm_splitk(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                 int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * The GEMM with the output rotated back to the unrotated basis in the same
 * launch (the second transform of dpshk.com/news/5289456 §4.2, fused with the
 * product instead of a separate tb_fwht128 along N):
 *   y[m][128b + i] = (1/sqrt(128)) * sum_j H[i][j] * y'[m][128b + j],
 *   y' = the product of tb_ternary_gemm.
 * y' stays in fp32 and y is rounded once (bf16 nearest even, or fp32), so the
 * result equals tb_ternary_gemm with fp32 output followed by tb_fwht128
 * (fp32 in, y_dtype out).  Arguments and errors as tb_ternary_gemm_splitk:
 * with a workspace of tb_ternary_gemm_splitk_workspace bytes K is split and
 * the rotation runs in the reduction; with NULL the product is one pass and
 * the rotation runs in its epilogue.
 */
TB_API tb_status tb_ternary_gemm_rotated(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                  int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
