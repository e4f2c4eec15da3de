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
 *
 * This header is the operator library's whole surface: the library exports
 * these functions and nothing else.  Kernel-family forcing, launch tuning,
 * kernel introspection and the bandwidth probes live in a separate library
 * (skipln_tune.h, libskipln_tune.so) built from the same kernels.
 */
#ifndef SKIPLN_H
#define SKIPLN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of this header are the library's only exports. */
#define SKIPLN_API __attribute__((visibility("default")))

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

/* Operations sharing the row kernels (skipln_forward_ws,
 * skipln_workspace_bytes).  SKIPLN_OP_SIMPLIFIED is the root-mean-square form
 * selected by the `simplified` template input of every SkipLayerNormalization
 * variant (the manifest sets it false and does not spell it out; reading used
 * here: no mean subtraction, the mean square in place of the variance).
 * SKIPLN_OP_BIAS_ADD is the BiasAdd operator (com.microsoft BiasAdd manifest).
 * SKIPLN_OP_BIAS_SOFTMAX is the BiasSoftmax operator (com.microsoft
 * BiasSoftmax manifest), with the data as `input` and the bias as `skip`. */
enum { SKIPLN_OP_LAYER_NORM = 0, SKIPLN_OP_SIMPLIFIED = 1, SKIPLN_OP_BIAS_ADD = 2, SKIPLN_OP_BIAS_SOFTMAX = 3 };

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
SKIPLN_API int skipln_forward(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
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
SKIPLN_API int skipln_forward_simplified(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
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
SKIPLN_API int skipln_bias_add(const void* x, const void* bias, const void* skip, void* y, int64_t rows, int64_t channels,
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
SKIPLN_API int skipln_bias_softmax(const void* data, const void* bias, void* out, int64_t batch_count, int64_t block_size,
                        int64_t bias_batch_count, int is_inner_broadcast, int dtype, void* workspace,
                        int64_t workspace_bytes, skipln_stream_t stream);

/*
 * Operation `op` (SKIPLN_OP_*) with a caller-provided workspace, which lets
 * the automatic kernel choice split rows too long for one workgroup's LDS
 * across workgroups: the layer norm and simplified forms up to 262144 float32
 * / 524288 float16 values per row, BiasSoftmax rows beyond what one
 * workgroup's registers hold.  The arguments are those of skipln_forward, with
 * the operation's own rules: for SKIPLN_OP_BIAS_ADD gamma, beta, residual_out
 * and eps are ignored, bias is required and the skip must be exact; for
 * SKIPLN_OP_BIAS_SOFTMAX input is the data, skip the bias (skip_rows bias
 * rows; SKIPLN_SKIP_BROADCAST cyclic, SKIPLN_SKIP_BROADCAST_INNER grouped
 * reuse), and gamma, beta, bias, residual_out and eps are ignored.
 * workspace: device memory, 16-byte aligned, overlapping no tensor, of at
 * least skipln_workspace_bytes() bytes for the same arguments (NULL / 0 when
 * that is 0); its contents on entry do not matter and are undefined
 * afterwards; it must stay untouched until the enqueued work ends, and two
 * calls in flight at once need two workspaces.  With as many rows as the
 * device has compute units or more, RMS rows and float32 layer norm rows of
 * up to 65536 values take the generic kernel instead (one workgroup per row,
 * no workspace; measured faster there).  Returns SKIPLN_ERR_WORKSPACE when the
 * chosen kernels need a workspace and it does not serve; otherwise as
 * skipln_forward.
 */
SKIPLN_API int skipln_forward_ws(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                 const void* gamma, const void* beta, const void* bias,
                                 void* out, void* residual_out, int64_t rows, int64_t hidden,
                                 float eps, int dtype, void* workspace, int64_t workspace_bytes,
                                 skipln_stream_t stream);

/* Workspace bytes skipln_forward_ws may need for these arguments on any
 * device (0: none), or a negative status code.  Host code only, no HIP call. */
SKIPLN_API int64_t skipln_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode,
                                          int64_t skip_rows);

/*
 * skipln_forward_ws without the workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the split-row kernels use the library's own
 * scratch, a device array of 256 KiB per GPU held until the process ends.  It
 * allocates nothing.  Calls whose kernels would need more scratch than that
 * return SKIPLN_ERR_WORKSPACE (the automatic choice needs less than 154 KiB).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams or host threads) race and must be
 * serialized by the caller.  Otherwise as skipln_forward_ws.
 */
SKIPLN_API int skipln_forward_ws_static(int op, const void* input, const void* skip, int skip_mode,
                                        int64_t skip_rows, const void* gamma, const void* beta, const void* bias,
                                        void* out, void* residual_out, int64_t rows, int64_t hidden,
                                        float eps, int dtype, skipln_stream_t stream);

/*
 * The argument checks of skipln_forward alone, with the same arguments (the
 * stream aside): host code only, no HIP call, no pointer dereferenced.
 * Returns the status skipln_forward would return before enqueueing anything.
 * The checks follow the SkipLayerNormalization manifest's `derive` contracts:
 * `epsilonOk` (eps >= 0; NaN is rejected too), `rank2CoreContract` (hidden >
 * 0, gamma of length hidden), `betaContract`, `broadcastSkipShapeOk` and the
 * broadcast binding set's `Params.skipRows` (skip_rows > 0 dividing rows),
 * `f32MainDtypes` / `f16MainDtypes` (one element type); plus this library's
 * size and aliasing rules (above).
 */
SKIPLN_API int skipln_validate(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                               const void* gamma, const void* beta, const void* bias,
                               const void* out, const void* residual_out, int64_t rows, int64_t hidden,
                               float eps, int dtype);

/* Static description of a status code. */
SKIPLN_API const char* skipln_status_string(int status);

/* ABI version of this header: 2. */
SKIPLN_API int skipln_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKIPLN_H */
