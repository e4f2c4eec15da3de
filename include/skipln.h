/*
 * libskipln -- SkipLayerNormalization row kernels for AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The operator (com.microsoft SkipLayerNormalization WebGPU manifest):
 *   - `description`, `inputs[input]`: skip addition fused with a layer
 *     normalization over the last (hidden) axis;
 *   - `inputs[skip]`: skip has the input's shape, or for rank-3 input
 *     (N, S, H) the shapes (1, S, H) and (S, H), broadcast over the batch;
 *   - `inputs[bias]`: an optional length-H bias joins input + skip before the
 *     normalization;
 *   - `inputs[gamma]`, `inputs[beta]`: length-H scale (required) and shift
 *     (optional, absent = 0);
 *   - `outputs[output]`: normalized tensor, shape of input;
 *     `outputs[input_skip_bias_sum]`: optional pre-normalization sum;
 *   - `attributes.epsilon` / `attributeDescriptions.epsilon`: non-negative
 *     epsilon added to the variance under the square root, carried as a
 *     binary32 value by the manifest's `Params` structs;
 *   - `typeConstraints.T`: every tensor is float32 or float16.
 *
 * For row r (0 <= r < rows) and column c (0 <= c < hidden), with j = r for an
 * exact skip and j = r mod skip_rows for a broadcast skip:
 *   s[r,c]    = fl32(fl32(input[r,c] + skip[j,c]) + bias[c])   (IEEE binary32)
 *   residual  = s rounded once to T (round to nearest even)
 *   mean      = sum_c s[r,c] / hidden
 *   var       = sum_c (s[r,c] - mean)^2 / hidden               (population)
 *   out[r,c]  = (s[r,c] - mean) / sqrt(var + eps) * gamma[c] + beta[c], to T
 * Arithmetic is binary32 for both I/O types; float16 is converted exactly on
 * load and rounded to nearest even on store.
 *
 * Memory and ownership (every entry point):
 *   - Every tensor pointer is device memory owned by the caller; tensors are
 *     dense and row-major: input/out/residual_out are rows x hidden, skip is
 *     rows x hidden (exact) or skip_rows x hidden (broadcast), gamma/beta/bias
 *     have hidden elements.  All tensors share one element type `dtype`.
 *   - The library allocates nothing, frees nothing and never synchronizes:
 *     work is enqueued on `stream` (NULL = the null stream) and the call
 *     returns at once.  It keeps no mutable state besides a cache of device
 *     attributes, and is safe to call from several host threads.
 *   - Outputs may alias inputs only exactly: out or residual_out may equal
 *     input, or skip when the skip is exact; every other overlap is an error.
 *   - On an error nothing is enqueued (except SKIPLN_ERR_LAUNCH, which reports
 *     a launch the runtime refused).
 */
#ifndef SKIPLN_H
#define SKIPLN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type (hipStream_t), declared without the HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t* skipln_stream_t;

/* Element types (`typeConstraints.T`). */
enum { SKIPLN_F32 = 0, SKIPLN_F16 = 1 };

/* Skip forms (`inputs[skip]`): exact shape, or S rows broadcast over the
 * batch, where row r of the input reads skip row r mod S.  The grouped form
 * (BiasSoftmax's inner broadcast only) has row r read skip row
 * r / (rows / S): consecutive groups of rows / S rows share one skip row. */
enum { SKIPLN_SKIP_EXACT = 0, SKIPLN_SKIP_BROADCAST = 1, SKIPLN_SKIP_BROADCAST_INNER = 2 };

/* Status codes. */
enum {
    SKIPLN_OK = 0,
    SKIPLN_ERR_NULL = 1,        /* a required pointer is NULL while rows > 0 */
    SKIPLN_ERR_SHAPE = 2,       /* rows < 0, hidden <= 0 or > 2^31-1, size
                                   overflow, bad skip_rows for a broadcast */
    SKIPLN_ERR_DTYPE = 3,       /* dtype is neither SKIPLN_F32 nor SKIPLN_F16 */
    SKIPLN_ERR_MODE = 4,        /* unknown skip_mode, or one the operation
                                   does not take */
    SKIPLN_ERR_EPS = 5,         /* eps < 0 or NaN */
    SKIPLN_ERR_ALIAS = 6,       /* outputs overlap inputs or each other */
    SKIPLN_ERR_UNSUPPORTED = 7, /* a forced variant cannot run this shape */
    SKIPLN_ERR_LAUNCH = 8,      /* the HIP runtime refused the launch */
    SKIPLN_ERR_DEVICE = 9,      /* querying the current device failed */
    SKIPLN_ERR_VARIANT = 10,    /* unknown variant, geometry or tiling */
    SKIPLN_ERR_OP = 11,         /* unknown operation */
    SKIPLN_ERR_WORKSPACE = 12   /* the chosen kernels need a workspace: missing,
                                   not 16-byte aligned, or smaller than
                                   skipln_workspace_bytes() */
};

/* Operations sharing the row kernels (for the _variant / _config / validate /
 * select calls).  SKIPLN_OP_SIMPLIFIED is the root-mean-square form selected
 * by the `simplified` template input of every SkipLayerNormalization variant
 * (the manifest sets it false and does not spell it out; reading used here:
 * no mean subtraction, the mean square in place of the variance).
 * SKIPLN_OP_BIAS_ADD is the BiasAdd operator (com.microsoft BiasAdd manifest).
 * SKIPLN_OP_BIAS_SOFTMAX is the BiasSoftmax operator (com.microsoft
 * BiasSoftmax manifest), with the data as `input` and the bias as `skip`. */
enum { SKIPLN_OP_LAYER_NORM = 0, SKIPLN_OP_SIMPLIFIED = 1, SKIPLN_OP_BIAS_ADD = 2, SKIPLN_OP_BIAS_SOFTMAX = 3 };

/* Kernel families, for skipln_forward_variant / skipln_select.  The automatic
 * choice: row tiles up to 2048 chunks of 16 bytes per row, the LDS-staged
 * kernel for longer rows of the reducing operations, the register-resident
 * kernel for BiasSoftmax rows beyond it, then -- for calls that bring a
 * workspace (skipln_forward_ws) -- the split-row kernels, except for 256 or
 * more rows of RMS, or of float32 layer norm up to 65536 values, which the
 * generic kernel runs faster without a workspace; rows that are not
 * whole chunks, or tensors not 16-byte aligned, take element-wise row tiles
 * up to 16384 values, and the generic kernel anything else. */
enum {
    SKIPLN_VARIANT_AUTO = 0,      /* what skipln_forward picks */
    SKIPLN_VARIANT_GENERIC = 1,   /* one workgroup per row, any hidden size and
                                     alignment: aligned rows of whole 16-byte
                                     chunks read twice with 16-byte accesses,
                                     others in three element-wise passes */
    SKIPLN_VARIANT_ROWTILE = 2,   /* row held in registers, 16-byte accesses:
                                     needs hidden*sizeof(T) % 16 == 0, 16-byte
                                     aligned pointers, hidden <= 4096*16/sizeof(T) */
    SKIPLN_VARIANT_MULTIWAVE = 3, /* ROWTILE with at least two wavefronts per
                                     row (exercises the cross-wave combine) */
    SKIPLN_VARIANT_LDSROW = 4,    /* long rows: one 1024-lane block per row, the
                                     row's binary32 values staged in LDS; layer
                                     norm, simplified and BiasSoftmax, 16-byte
                                     chunks, aligned pointers,
                                     hidden * 4 <= 163584 bytes */
    SKIPLN_VARIANT_SPLITROW = 5,  /* rows cut into slices of 16 KiB per tensor,
                                     one workgroup per slice, two kernels
                                     (partial results, then merge and
                                     normalize) through a workspace: layer norm,
                                     simplified and BiasSoftmax, 16-byte chunks,
                                     aligned pointers, at most 64 slices
                                     (262144 float32 / 524288 float16 values);
                                     skipln_forward_ws only; the residual may
                                     not alias input or skip (the automatic
                                     choice then takes the generic kernel) */
    SKIPLN_VARIANT_ELEMENT = 6,   /* row held in registers, one element per
                                     access: any hidden size up to 16384,
                                     tensors aligned to their element size
                                     (what the automatic choice takes for rows
                                     that are not whole 16-byte chunks) */
    SKIPLN_VARIANT_REGROW = 7,    /* long rows of BiasSoftmax: one 1024-lane
                                     block per row, the row's raw data in
                                     registers (up to 20 chunks per lane:
                                     163840 float16 / 81920 float32 values),
                                     z = data + bias formed again in each of
                                     two passes from the bias rows re-read
                                     through the caches; 16-byte chunks,
                                     aligned pointers; no workspace */
    SKIPLN_VARIANT_GEOMETRY = 64, /* + g: ROWTILE with row-tile geometry g,
                                     0 <= g < skipln_rowtile_geometries(), for
                                     tests and tuning */
    SKIPLN_VARIANT_ELEMENT_GEOMETRY = 128 /* + g: ELEMENT with geometry g,
                                     0 <= g < skipln_element_geometries() */
};

/*
 * Fused skip addition + layer normalization (SkipLayerNormalization manifest,
 * `description`, `inputs`, `outputs`, `attributes.epsilon`).
 *
 * input         rows x hidden, T
 * skip          rows x hidden (SKIPLN_SKIP_EXACT; skip_rows ignored) or
 *               skip_rows x hidden (SKIPLN_SKIP_BROADCAST; rows must be a
 *               multiple of skip_rows, the manifest's `Params.skipRows`)
 * gamma         hidden, T, required
 * beta, bias    hidden, T, or NULL (absent)
 * out           rows x hidden, T
 * residual_out  rows x hidden, T, or NULL (input_skip_bias_sum not written)
 * rows          >= 0 (0 is a valid no-op); rank-3 (N, S, H) input is passed
 *               as rows = N*S
 * hidden        1 .. 2^31-1
 * eps           >= 0
 * dtype         SKIPLN_F32 or SKIPLN_F16
 * Returns SKIPLN_OK or an error code above.
 */
int skipln_forward(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                   const void* gamma, const void* beta, const void* bias,
                   void* out, void* residual_out, int64_t rows, int64_t hidden,
                   float eps, int dtype, skipln_stream_t stream);

/*
 * Root-mean-square ("simplified") form of skipln_forward, same arguments:
 * s as above, ms = sum_c s[r,c]^2 / hidden,
 * out[r,c] = s[r,c] / sqrt(ms + eps) * gamma[c] + beta[c] (beta optional).
 * Source: the `simplified` template input of the SkipLayerNormalization
 * manifest's variants (always false there; semantics inferred).
 */
int skipln_forward_simplified(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                              const void* gamma, const void* beta, const void* bias,
                              void* out, void* residual_out, int64_t rows, int64_t hidden,
                              float eps, int dtype, skipln_stream_t stream);

/*
 * BiasAdd (com.microsoft BiasAdd manifest, `description`, `inputs`,
 * `outputs[Y]`): Y = (X + bias) + skip elementwise, the channel bias added to
 * X first and the skip second, each add in IEEE binary32, Y rounded once to T.
 * x, skip, y: rows x channels (an (N, S, C) tensor with rows = N*S), bias:
 * channels.  y may equal x or skip exactly; other overlaps are an error.
 */
int skipln_bias_add(const void* x, const void* bias, const void* skip, void* y, int64_t rows, int64_t channels,
                    int dtype, skipln_stream_t stream);

/*
 * BiasSoftmax (com.microsoft BiasSoftmax manifest, `description`,
 * `attributes.is_inner_broadcast`, `derive.batchCount`, `derive.blockSize`,
 * `derive.biasBlockCount`, `derive.biasContract`, `innerRepeat`): a softmax
 * over each of batch_count rows of block_size values of data + bias.
 *
 * data, out     batch_count x block_size, T (the flattened data tensor: rows
 *               are the dimensions before `axis`, a row the suffix from it)
 * bias          bias_batch_count x block_size, T
 * For row r, bias row j = r / (batch_count / bias_batch_count) when
 * is_inner_broadcast != 0 (consecutive groups share a bias row), else
 * j = r mod bias_batch_count (cyclic reuse), and
 *   z[r,c] = fl32(data[r,c] + bias[j,c]),  M = max_c z[r,c],
 *   out[r,c] = exp(z[r,c] - M) / sum_c' exp(z[r,c'] - M), rounded to T.
 * The exponentials are evaluated in binary32 (2^x on the exponent scaled by
 * log2 e) and summed in binary32; the result follows the definition within
 * a few binary32 rounding steps per term.  A row containing NaN or +inf, or
 * made of -inf only, comes out NaN; -inf terms of other rows give 0.
 *
 * Shapes (`biasContract`): all counts >= 0; empty data with an empty bias
 * (batch_count or block_size 0, and bias_batch_count or block_size 0) is a
 * valid no-op; otherwise block_size >= 1 and 1 <= bias_batch_count <=
 * batch_count with batch_count a multiple of bias_batch_count, else
 * SKIPLN_ERR_SHAPE.  out may equal data exactly, or bias when
 * bias_batch_count == batch_count; other overlaps are SKIPLN_ERR_ALIAS.
 * workspace / workspace_bytes: NULL / 0, or a workspace as for
 * skipln_forward_ws (size from skipln_workspace_bytes with
 * SKIPLN_OP_BIAS_SOFTMAX, rows = batch_count, hidden = block_size and the
 * skip form above).  Rows of 16-byte chunks up to 40896 values stay in one
 * workgroup's LDS and up to 163840 float16 / 81920 float32 values in one
 * workgroup's registers (the manifest's long-row variants split them across
 * workgroups); longer ones split across workgroups through the workspace, or
 * without one take the generic kernel.  Ownership, streams and errors as for
 * skipln_forward.
 */
int skipln_bias_softmax(const void* data, const void* bias, void* out, int64_t batch_count, int64_t block_size,
                        int64_t bias_batch_count, int is_inner_broadcast, int dtype, void* workspace,
                        int64_t workspace_bytes, skipln_stream_t stream);

/*
 * Operation `op` with a caller-provided workspace, which lets the kernel
 * choice (`variant`, SKIPLN_VARIANT_AUTO included) take the split-row kernels
 * for rows too long for one workgroup.  workspace: device memory, 16-byte
 * aligned, overlapping no tensor, of at least skipln_workspace_bytes() bytes
 * for the same arguments; its contents on entry do not matter and are
 * undefined afterwards; it must stay untouched until the enqueued work ends,
 * and two calls in flight at once need two workspaces.  When the chosen
 * kernel needs no workspace, workspace may be NULL.  Otherwise as
 * skipln_forward_variant; SKIPLN_ERR_WORKSPACE when the workspace does not
 * serve.
 */
int skipln_forward_ws(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                      const void* gamma, const void* beta, const void* bias,
                      void* out, void* residual_out, int64_t rows, int64_t hidden,
                      float eps, int dtype, int variant, void* workspace, int64_t workspace_bytes,
                      skipln_stream_t stream);

/* Workspace bytes skipln_forward_ws needs for these arguments (0: none), or a
 * negative status code.  The kernel choice depends on the row count (see
 * skipln_select_ws).  Host code only. */
int64_t skipln_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode, int64_t skip_rows,
                               int variant);

/* Operation `op` (SKIPLN_OP_*) with the kernel family forced
 * (SKIPLN_VARIANT_*); the result is the same operator.  For
 * SKIPLN_OP_BIAS_ADD, gamma, beta, residual_out and eps are ignored, bias is
 * required and the skip must be exact.  For SKIPLN_OP_BIAS_SOFTMAX, input is
 * the data, skip the bias (skip_rows bias rows; SKIPLN_SKIP_BROADCAST is the
 * cyclic and SKIPLN_SKIP_BROADCAST_INNER the grouped reuse), and gamma, beta,
 * bias, residual_out and eps are ignored.  Returns SKIPLN_ERR_UNSUPPORTED
 * when the family cannot run the shape or alignment. */
int skipln_forward_variant(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                           const void* gamma, const void* beta, const void* bias,
                           void* out, void* residual_out, int64_t rows, int64_t hidden,
                           float eps, int dtype, int variant, skipln_stream_t stream);

/* How the row-tile kernel distributes row tiles over workgroups (see
 * skipln_forward_config). */
enum {
    SKIPLN_TILE_CONTIGUOUS = 0,     /* block b: tiles b*T .. b*T + T - 1 */
    SKIPLN_TILE_STRIDED = 1,        /* block b: tiles b, b + grid, b + 2*grid, ... */
    SKIPLN_TILE_SKIP_STATIONARY = 2 /* broadcast skip: block b keeps its skip rows
                                       in registers and walks T batches;
                                       otherwise as SKIPLN_TILE_STRIDED */
};

/* Operation `op` with an explicit launch configuration, for tuning; the
 * result is the same operator.  geometry: row-tile geometry
 * (0 <= geometry < skipln_rowtile_geometries()), -1 for the automatic
 * choice, or SKIPLN_VARIANT_ELEMENT_GEOMETRY + g for element-wise geometry g.  tiles_per_block (T) > 0: row tiles (batches, for
 * SKIPLN_TILE_SKIP_STATIONARY) per block; 0: sized so the grid matches the
 * blocks the device holds at once (SKIPLN_TILE_CONTIGUOUS then behaves as
 * SKIPLN_TILE_STRIDED).  tiling: SKIPLN_TILE_*.  Returns
 * SKIPLN_ERR_UNSUPPORTED when the geometry cannot hold the row or the tensors
 * are not 16-byte aligned, SKIPLN_ERR_SHAPE for tiles_per_block < 0,
 * SKIPLN_ERR_VARIANT for an unknown geometry or tiling. */
int skipln_forward_config(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                          const void* gamma, const void* beta, const void* bias,
                          void* out, void* residual_out, int64_t rows, int64_t hidden,
                          float eps, int dtype, int geometry, int64_t tiles_per_block, int tiling,
                          skipln_stream_t stream);

/* The argument checks of operation `op` alone: host code only, no HIP call,
 * no pointer is dereferenced. */
int skipln_validate(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                    const void* gamma, const void* beta, const void* bias,
                    const void* out, const void* residual_out, int64_t rows, int64_t hidden,
                    float eps, int dtype);

/* Kernel that skipln_forward_variant would launch for this operation, hidden
 * size and skip form: returns a kernel id >= 0 (name via skipln_kernel_name)
 * or a negative status code.  `aligned16` says whether every tensor pointer
 * is 16-byte aligned. */
int skipln_select(int op, int64_t hidden, int dtype, int skip_mode, int aligned16, int variant);

/* The same for skipln_forward_ws given a sufficient workspace, for a call of
 * fewer than 256 rows.  With 256 rows or more, RMS rows and float32 layer
 * norm rows of up to 65536 values that would split across workgroups take
 * the generic kernel instead, which needs no workspace (measured faster
 * there); skipln_workspace_bytes, which knows the row count, then returns 0. */
int skipln_select_ws(int op, int64_t hidden, int dtype, int skip_mode, int aligned16, int variant);

/* Streaming copy of `bytes` bytes from src to dst (device memory, 16-byte
 * aligned, bytes % 16 == 0, no overlap), with the access pattern of the
 * row-tile kernel's streamed input and outputs (16-byte non-temporal loads
 * and stores, persistent grid).
 * It is the reference for the bandwidth one kernel can reach on the device
 * and for calibrating hardware byte counters against a known byte count.
 * Returns SKIPLN_OK, SKIPLN_ERR_NULL, SKIPLN_ERR_SHAPE (bytes < 0 or not a
 * multiple of 16, misaligned pointers), SKIPLN_ERR_ALIAS or SKIPLN_ERR_LAUNCH. */
int skipln_copy(void* dst, const void* src, int64_t bytes, skipln_stream_t stream);

/* Streaming probe with the access pattern of the row kernels (16-byte
 * non-temporal accesses, one tile of `block` lanes x `chunks_per_lane`
 * chunks per stream and workgroup; block 64, 256 or 1024, chunks_per_lane 1
 * or 4): reads 0-2 input streams (src0, then src1; NULL = not read) and
 * writes 0-2 output streams (dst0, then dst1) of `bytes` bytes each.  It
 * measures the HBM rate a kernel of that pattern attains for each mix of
 * reads and writes, the ceiling the row kernels are compared with.
 * xcd_granule (1 .. 65536): tiles in address order (1), or each XCD handed
 * xcd_granule consecutive tiles per round of 8 x xcd_granule (the dispatcher
 * deals workgroup b to XCD b mod 8): the address granularity at which the
 * eight XCDs share the streams, which for a row kernel is one row.
 * store_through: 0 = non-temporal stores; 1 = non-temporal stores with
 * system-scope coherence (the policy the row-tile kernels use for launches
 * that write 512 MiB or more, and the register-resident softmax for such
 * launches whose rows are whole 16 KiB slabs).
 * Outputs: dst0 = src0 XOR src1 (a chunk's index when nothing is read),
 * dst1 = dst0 + 1 per 32-bit word, whatever the tile order.  Device memory,
 * 16-byte aligned, bytes % 16 == 0, outputs overlapping nothing.  Returns
 * SKIPLN_OK, SKIPLN_ERR_NULL (no stream, or src1/dst1 without src0/dst0),
 * SKIPLN_ERR_SHAPE, SKIPLN_ERR_ALIAS, SKIPLN_ERR_VARIANT (tile shape or
 * granule) or SKIPLN_ERR_LAUNCH. */
int skipln_stream(const void* src0, const void* src1, void* dst0, void* dst1, int64_t bytes, int block,
                  int chunks_per_lane, int64_t xcd_granule, int store_through, skipln_stream_t stream);

/* Number of row-tile geometries (for SKIPLN_VARIANT_GEOMETRY + g). */
int skipln_rowtile_geometries(void);

/* Number of element-wise row-tile geometries (SKIPLN_VARIANT_ELEMENT_GEOMETRY + g). */
int skipln_element_geometries(void);

/* Stable name of a kernel id ("generic_f32", "rowtile_f16_g256_c4",
 * "rms_rowtile_f32_g192_c1_b192", "biasadd_generic_f16",
 * "softmax_rowtile_f16_g8_c1", ...); "unknown" for an invalid id. */
const char* skipln_kernel_name(int kernel_id);

/* Static description of a status code. */
const char* skipln_status_string(int status);

/* ABI version of this header: 1. */
int skipln_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKIPLN_H */
