// C ABI of libskipln: argument checks, kernel choice and launch.
//
// The checks follow the contracts of the com.microsoft SkipLayerNormalization
// WebGPU manifest (`derive`): epsilon must be non-negative (`epsilonOk`), the
// hidden size positive and gamma/beta/bias of length H (`rank2CoreContract`,
// `betaContract`), all tensors of one element type (`f32MainDtypes`,
// `f16MainDtypes`), a broadcast skip (S, H) read cyclically by the (N*S) rows
// (`broadcastSkipShapeOk`, `Params.skipRows`).  BiasAdd (com.microsoft BiasAdd
// manifest, `inputs`) takes X, a length-C bias and a skip of X's shape.
// BiasSoftmax (com.microsoft BiasSoftmax manifest, `derive.biasContract`)
// takes batchCount rows of blockSize values and biasBlockCount bias rows that
// divide the row count, reused cyclically (outer broadcast) or by consecutive
// groups of batchCount / biasBlockCount rows (inner broadcast); its bias
// travels in the skip slot of the shared kernels.
// Aliasing rules are this library's own: an output may only coincide exactly
// with a tensor that is read row by row by the lane group that later writes
// the same row.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/skipln.h"
#include "skipln_internal.h"

static_assert(SKIPLN_TILE_CONTIGUOUS == skipln::kTileContiguous && SKIPLN_TILE_STRIDED == skipln::kTileStrided &&
                  SKIPLN_TILE_SKIP_STATIONARY == skipln::kTileSkipStationary,
              "tiling modes of the ABI and the kernels agree");
static_assert(SKIPLN_OP_LAYER_NORM == skipln::kOpLayerNorm && SKIPLN_OP_SIMPLIFIED == skipln::kOpSimplified &&
                  SKIPLN_OP_BIAS_ADD == skipln::kOpBiasAdd && SKIPLN_OP_BIAS_SOFTMAX == skipln::kOpBiasSoftmax,
              "operations of the ABI and the kernels agree");

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range span(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& a, const Range& b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

bool same(const Range& a, const Range& b) { return a.lo == b.lo && a.hi == b.hi; }

bool known_op(int op) {
    return op == SKIPLN_OP_LAYER_NORM || op == SKIPLN_OP_SIMPLIFIED || op == SKIPLN_OP_BIAS_ADD ||
           op == SKIPLN_OP_BIAS_SOFTMAX;
}

bool normalizing(int op) { return op == SKIPLN_OP_LAYER_NORM || op == SKIPLN_OP_SIMPLIFIED; }

// Skip forms an operation accepts: grouped (inner) reuse is BiasSoftmax's.
bool mode_ok(int op, int skip_mode) {
    if (skip_mode == SKIPLN_SKIP_EXACT) return true;
    if (skip_mode == SKIPLN_SKIP_BROADCAST) return op != SKIPLN_OP_BIAS_ADD;
    if (skip_mode == SKIPLN_SKIP_BROADCAST_INNER) return op == SKIPLN_OP_BIAS_SOFTMAX;
    return false;
}

// One call's arguments after the operation's own rules: BiasAdd has no
// gamma, beta, residual output or epsilon; BiasSoftmax has none of these and
// no separate bias either (its bias is the skip).
struct Call {
    int op;
    const void *input, *skip, *gamma, *beta, *bias;
    void *out, *residual;
    int skip_mode;
    int64_t skip_rows, rows, hidden;
    float eps;
    int dtype;
};

Call make_call(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
               const void* beta, const void* bias, const void* out, const void* residual_out, int64_t rows,
               int64_t hidden, float eps, int dtype) {
    const bool norm = normalizing(op);
    Call c;
    c.op = op;
    c.input = input;
    c.skip = skip;
    c.gamma = norm ? gamma : nullptr;
    c.beta = norm ? beta : nullptr;
    c.bias = op == SKIPLN_OP_BIAS_SOFTMAX ? nullptr : bias;
    c.out = const_cast<void*>(out);
    c.residual = norm ? const_cast<void*>(residual_out) : nullptr;
    c.skip_mode = skip_mode;
    c.skip_rows = skip_rows;
    c.rows = rows;
    c.hidden = hidden;
    c.eps = norm ? eps : 0.0f;
    c.dtype = dtype;
    return c;
}

int validate(const Call& c) {
    if (!known_op(c.op)) return SKIPLN_ERR_OP;
    if (c.dtype != SKIPLN_F32 && c.dtype != SKIPLN_F16) return SKIPLN_ERR_DTYPE;
    if (!mode_ok(c.op, c.skip_mode)) return SKIPLN_ERR_MODE;
    if (!(c.eps >= 0.0f)) return SKIPLN_ERR_EPS;  // also rejects NaN
    if (c.rows < 0 || c.hidden <= 0 || c.hidden > INT32_MAX) return SKIPLN_ERR_SHAPE;
    const int64_t sz = c.dtype == SKIPLN_F32 ? 4 : 2;
    if (c.rows > INT64_MAX / c.hidden / sz) return SKIPLN_ERR_SHAPE;
    const bool bcast = c.skip_mode != SKIPLN_SKIP_EXACT;
    if (bcast && (c.skip_rows <= 0 || c.rows % c.skip_rows != 0)) return SKIPLN_ERR_SHAPE;
    if (c.rows == 0) return SKIPLN_OK;
    if (!c.input || !c.skip || !c.out) return SKIPLN_ERR_NULL;
    if (normalizing(c.op) && !c.gamma) return SKIPLN_ERR_NULL;
    if (c.op == SKIPLN_OP_BIAS_ADD && !c.bias) return SKIPLN_ERR_NULL;

    const int64_t row_bytes = c.hidden * sz;
    const Range r_in = span(c.input, c.rows * row_bytes);
    const Range r_skip = span(c.skip, (bcast ? c.skip_rows : c.rows) * row_bytes);
    const Range r_gamma = span(c.gamma, c.gamma ? row_bytes : 0);
    const Range r_beta = span(c.beta, c.beta ? row_bytes : 0);
    const Range r_bias = span(c.bias, c.bias ? row_bytes : 0);
    const Range r_out = span(c.out, c.rows * row_bytes);
    const Range r_res = span(c.residual, c.residual ? c.rows * row_bytes : 0);

    for (const Range& o : {r_out, r_res}) {
        if (o.empty()) continue;
        if (overlap(o, r_in) && !same(o, r_in)) return SKIPLN_ERR_ALIAS;
        if (overlap(o, r_skip) && (bcast || !same(o, r_skip))) return SKIPLN_ERR_ALIAS;
        if (overlap(o, r_gamma) || overlap(o, r_beta) || overlap(o, r_bias)) return SKIPLN_ERR_ALIAS;
    }
    if (overlap(r_out, r_res)) return SKIPLN_ERR_ALIAS;
    return SKIPLN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool all_aligned16(const Call& c) {
    return aligned16(c.input) && aligned16(c.skip) && aligned16(c.gamma) && aligned16(c.beta) && aligned16(c.bias) &&
           aligned16(c.out) && aligned16(c.residual);
}

// Every tensor aligned to its element size (what element-wise accesses need).
bool all_element_aligned(const Call& c) {
    const uintptr_t m = c.dtype == SKIPLN_F32 ? 3u : 1u;
    for (const void* p : {c.input, c.skip, c.gamma, c.beta, c.bias, static_cast<const void*>(c.out),
                          static_cast<const void*>(c.residual)})
        if (reinterpret_cast<uintptr_t>(p) & m) return false;
    return true;
}

// Many long rows of a normalization: the generic kernel's chunk form (one
// 1024-lane workgroup per row, the row's first 40,832 sums parked in LDS, no
// workspace) outruns the split-row kernels once there is a row for every CU
// (MI355X: 256).  Measured, generic / split-row time: RMS 0.80-0.93 for 256
// to 2048 rows of 65,536 to 262,144 values (either type; 0.99 at 128 rows);
// float32 layer norm 0.85-0.91 for 256-2048 rows of 65,536 values, 1.29 at
// 128 rows, 0.92-1.00 at 131,072 values; float16 layer norm 0.97-1.08.
constexpr int64_t kGenericManyRows = 256;
bool generic_outruns_split(int op, int64_t hidden, int dtype, int64_t rows) {
    if (rows < kGenericManyRows) return false;
    return op == SKIPLN_OP_SIMPLIFIED || (op == SKIPLN_OP_LAYER_NORM && dtype == SKIPLN_F32 && hidden <= 65536);
}

// Kernel id (>= 0) for this variant, or -status.  vec_ok: tensors 16-byte
// aligned; elem_ok: aligned to their element size.  with_workspace: the call
// brings a workspace, so the automatic choice may take the split-row kernels
// (unless it has `rows` rows that the generic kernel runs faster; rows < 0:
// not known).
int select(int op, int64_t hidden, int dtype, bool broadcast, bool vec_ok, bool elem_ok, int variant,
           bool with_workspace, int64_t rows) {
    const int base = (op * 2 + dtype) * skipln::kIdsPerType;
    const int v = dtype == SKIPLN_F32 ? 4 : 8;  // elements per 16-byte chunk
    const bool chunked = vec_ok && hidden % v == 0;
    if (variant == SKIPLN_VARIANT_GENERIC) return base + skipln::kGenericIndex;
    if (variant == SKIPLN_VARIANT_ELEMENT) {
        const int g = elem_ok ? skipln::elem_pick(op, hidden) : -1;
        return g >= 0 ? base + skipln::kElemFirst + g : -SKIPLN_ERR_UNSUPPORTED;
    }
    if (variant >= SKIPLN_VARIANT_ELEMENT_GEOMETRY && variant < SKIPLN_VARIANT_ELEMENT_GEOMETRY + skipln::elem_count()) {
        const int g = variant - SKIPLN_VARIANT_ELEMENT_GEOMETRY;
        if (!elem_ok || !skipln::elem_holds(g, hidden)) return -SKIPLN_ERR_UNSUPPORTED;
        return base + skipln::kElemFirst + g;
    }
    const bool lds_ok = vec_ok && skipln::ldsrow_holds(op, hidden, dtype);
    const bool split_ok = vec_ok && skipln::split_holds(op, hidden, dtype);
    const bool reg_ok = vec_ok && skipln::regrow_holds(op, hidden, dtype);
    if (variant == SKIPLN_VARIANT_LDSROW) return lds_ok ? base + skipln::kLdsRowIndex : -SKIPLN_ERR_UNSUPPORTED;
    if (variant == SKIPLN_VARIANT_SPLITROW) return split_ok ? base + skipln::kSplitRowIndex : -SKIPLN_ERR_UNSUPPORTED;
    if (variant == SKIPLN_VARIANT_REGROW) return reg_ok ? base + skipln::kRegRowIndex : -SKIPLN_ERR_UNSUPPORTED;
    // Long rows of the reducing operations: staged in LDS; beyond its
    // capacity held in registers (softmax), or split across workgroups when
    // a workspace is at hand.
    if (variant == SKIPLN_VARIANT_AUTO && hidden / v > skipln::kRowtileMaxAutoChunks) {
        if (lds_ok) return base + skipln::kLdsRowIndex;
        if (reg_ok) return base + skipln::kRegRowIndex;
        if (split_ok && with_workspace && !generic_outruns_split(op, hidden, dtype, rows))
            return base + skipln::kSplitRowIndex;
    }
    if (variant == SKIPLN_VARIANT_AUTO || variant == SKIPLN_VARIANT_ROWTILE ||
        variant == SKIPLN_VARIANT_MULTIWAVE) {
        const int g =
            chunked ? skipln::rowtile_pick(op, hidden, dtype, broadcast, variant == SKIPLN_VARIANT_MULTIWAVE) : -1;
        if (g >= 0) return base + skipln::kRowtileFirst + g;
        if (variant != SKIPLN_VARIANT_AUTO) return -SKIPLN_ERR_UNSUPPORTED;
        // Rows that are not whole chunks (or tensors not 16-byte aligned):
        // element-wise row tiles, then the generic kernel.
        const int e = elem_ok && !chunked ? skipln::elem_pick(op, hidden) : -1;
        if (e >= 0) return base + skipln::kElemFirst + e;
        return base + skipln::kGenericIndex;
    }
    if (variant >= SKIPLN_VARIANT_GEOMETRY && variant < SKIPLN_VARIANT_GEOMETRY + skipln::rowtile_count()) {
        const int g = variant - SKIPLN_VARIANT_GEOMETRY;
        // The geometry must hold the whole row.
        if (!chunked || !skipln::rowtile_holds(g, hidden, dtype)) return -SKIPLN_ERR_UNSUPPORTED;
        return base + skipln::kRowtileFirst + g;
    }
    return -SKIPLN_ERR_VARIANT;
}

// Tiling of the automatic launch.  Streaming rows (exact skip): one tile per
// block, so blocks are dispatched in address order and the set of rows in
// flight stays compact; this reached the 2-read/2-write streaming rate on
// MI355X.  A cyclic broadcast skip is shared by every batch: each block of a
// normalization keeps its skip rows (and gamma/beta) in registers and walks
// the batches.  BiasSoftmax has no parameters to keep and measured faster
// streaming its rows in address order, its bias rows served by the caches,
// as is grouped (inner) reuse, whose consecutive rows share a bias row.
skipln::Tiling auto_tiling(int op, int skip_mode) {
    const bool cyclic = skip_mode == SKIPLN_SKIP_BROADCAST && op != SKIPLN_OP_BIAS_SOFTMAX;
    skipln::Tiling t;
    t.tiles_per_block = cyclic ? 0 : 1;
    t.mode = cyclic ? skipln::kTileSkipStationary : skipln::kTileStrided;
    return t;
}

skipln::Args make_args(const Call& c) {
    skipln::Args a;
    a.input = c.input;
    a.skip = c.skip;
    a.gamma = c.gamma;
    a.beta = c.beta;
    a.bias = c.bias;
    a.out = c.out;
    a.residual = c.residual;
    a.rows = c.rows;
    a.skip_rows = c.skip_mode == SKIPLN_SKIP_BROADCAST ? c.skip_rows : 0;
    a.skip_group = c.skip_mode == SKIPLN_SKIP_BROADCAST_INNER ? c.rows / c.skip_rows : 0;
    a.hidden = static_cast<int32_t>(c.hidden);
    a.eps = c.eps;
    a.tiles_per_block = 1;
    a.tiling = skipln::kTileStrided;
    // Bytes the launch writes: the output, and the residual when emitted.
    const int64_t written = c.rows * c.hidden * (c.dtype == SKIPLN_F32 ? 4 : 2) * (c.residual ? 2 : 1);
    a.store_through = written >= skipln::kStoreThroughBytes ? 1 : 0;
    return a;
}

int status_of(hipError_t e) {
    if (e == hipSuccess) return SKIPLN_OK;
    if (e == hipErrorInvalidDevice || e == hipErrorNoDevice) return SKIPLN_ERR_DEVICE;
    return SKIPLN_ERR_LAUNCH;
}

// A caller's workspace: device memory for partial results.
struct Workspace {
    void* ptr;
    int64_t bytes;
};

// The workspace a split-row launch of this call needs.
int64_t workspace_needed(const Call& c) { return skipln::split_workspace_bytes(make_args(c), c.dtype); }

// Validate, choose and launch; `tiling` == nullptr: automatic tiling;
// `ws` == nullptr: the call brings no workspace.
int run(const Call& c, int variant, const skipln::Tiling* tiling, skipln_stream_t stream,
        const Workspace* ws = nullptr) {
    const int st = validate(c);
    if (st != SKIPLN_OK) return st;
    const int id = select(c.op, c.hidden, c.dtype, c.skip_mode != SKIPLN_SKIP_EXACT, all_aligned16(c),
                          all_element_aligned(c), variant, ws != nullptr, c.rows);
    if (id < 0) return -id;
    if (c.rows == 0) return SKIPLN_OK;
    const skipln::Args a = make_args(c);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int index = id % skipln::kIdsPerType;
    if (index == skipln::kSplitRowIndex && c.residual && (c.residual == c.input || c.residual == c.skip)) {
        // The split-row kernels read x and skip twice, so a residual written
        // over either cannot take them: the generic kernel can.
        if (variant != SKIPLN_VARIANT_AUTO) return SKIPLN_ERR_UNSUPPORTED;
        return status_of(skipln::launch_generic(make_args(c), c.op, c.dtype, reinterpret_cast<hipStream_t>(stream)));
    }
    if (index == skipln::kSplitRowIndex) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;  // the split-row kernels have no tiling
        if (!ws || !ws->ptr || !aligned16(ws->ptr) || ws->bytes < workspace_needed(c)) return SKIPLN_ERR_WORKSPACE;
        const int64_t row_bytes = c.hidden * (c.dtype == SKIPLN_F32 ? 4 : 2);
        const Range w = span(ws->ptr, ws->bytes);
        const Range tensors[] = {
            span(c.input, c.rows * row_bytes),
            span(c.skip, (c.skip_mode != SKIPLN_SKIP_EXACT ? c.skip_rows : c.rows) * row_bytes),
            span(c.gamma, c.gamma ? row_bytes : 0), span(c.beta, c.beta ? row_bytes : 0),
            span(c.bias, c.bias ? row_bytes : 0), span(c.out, c.rows * row_bytes),
            span(c.residual, c.residual ? c.rows * row_bytes : 0)};
        for (const Range& t : tensors)
            if (overlap(w, t)) return SKIPLN_ERR_ALIAS;
        return status_of(skipln::launch_split(a, c.op, c.dtype, ws->ptr, s));
    }
    if (index == skipln::kGenericIndex) return status_of(skipln::launch_generic(a, c.op, c.dtype, s));
    if (index == skipln::kRegRowIndex) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;
        return status_of(skipln::launch_regrow(a, c.op, c.dtype, s));
    }
    if (index == skipln::kLdsRowIndex) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;  // the long-row kernel has no tiling
        return status_of(skipln::launch_ldsrow(a, c.op, c.dtype, s));
    }
    if (index >= skipln::kElemFirst) {
        const int g = index - skipln::kElemFirst;
        return status_of(skipln::launch_elem(a, c.op, c.dtype, g, tiling ? *tiling : skipln::elem_tiling(g), s));
    }
    const skipln::Tiling t = tiling ? *tiling : auto_tiling(c.op, c.skip_mode);
    return status_of(skipln::launch_rowtile(a, c.op, c.dtype, index - skipln::kRowtileFirst, t, s));
}

}  // namespace

extern "C" {

int skipln_validate(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
                    const void* beta, const void* bias, const void* out, const void* residual_out, int64_t rows,
                    int64_t hidden, float eps, int dtype) {
    return validate(
        make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps, dtype));
}

int skipln_select(int op, int64_t hidden, int dtype, int skip_mode, int aligned, int variant) {
    if (!known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (!mode_ok(op, skip_mode)) return -SKIPLN_ERR_MODE;
    if (hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    return select(op, hidden, dtype, skip_mode != SKIPLN_SKIP_EXACT, aligned != 0, true, variant, false, -1);
}

int skipln_select_ws(int op, int64_t hidden, int dtype, int skip_mode, int aligned, int variant) {
    if (!known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (!mode_ok(op, skip_mode)) return -SKIPLN_ERR_MODE;
    if (hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    return select(op, hidden, dtype, skip_mode != SKIPLN_SKIP_EXACT, aligned != 0, true, variant, true, -1);
}

int64_t skipln_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode, int64_t skip_rows,
                               int variant) {
    if (!known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (!mode_ok(op, skip_mode)) return -SKIPLN_ERR_MODE;
    if (rows < 0 || hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    if (skip_mode != SKIPLN_SKIP_EXACT && (skip_rows <= 0 || rows % skip_rows != 0)) return -SKIPLN_ERR_SHAPE;
    const int id = select(op, hidden, dtype, skip_mode != SKIPLN_SKIP_EXACT, true, true, variant, true, rows);
    if (id < 0) return id;
    if (id % skipln::kIdsPerType != skipln::kSplitRowIndex || rows == 0) return 0;
    Call c = make_call(op, nullptr, nullptr, skip_mode, skip_rows, nullptr, nullptr, nullptr, nullptr, nullptr, rows,
                       hidden, 0.0f, dtype);
    return workspace_needed(c);
}

int skipln_forward_ws(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                      const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                      int64_t rows, int64_t hidden, float eps, int dtype, int variant, void* workspace,
                      int64_t workspace_bytes, skipln_stream_t stream) {
    if (workspace_bytes < 0) return SKIPLN_ERR_WORKSPACE;
    const Workspace ws{workspace, workspace_bytes};
    return run(make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                         dtype),
               variant, nullptr, stream, &ws);
}

int skipln_forward_variant(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                           const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                           int64_t rows, int64_t hidden, float eps, int dtype, int variant, skipln_stream_t stream) {
    return run(make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                         dtype),
               variant, nullptr, stream);
}

int skipln_forward_config(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                          const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                          int64_t rows, int64_t hidden, float eps, int dtype, int geometry, int64_t tiles_per_block,
                          int tiling, skipln_stream_t stream) {
    if (tiles_per_block < 0) return SKIPLN_ERR_SHAPE;
    if (tiling != SKIPLN_TILE_CONTIGUOUS && tiling != SKIPLN_TILE_STRIDED && tiling != SKIPLN_TILE_SKIP_STATIONARY)
        return SKIPLN_ERR_VARIANT;
    const bool elem = geometry >= SKIPLN_VARIANT_ELEMENT_GEOMETRY;
    if (elem ? geometry >= SKIPLN_VARIANT_ELEMENT_GEOMETRY + skipln::elem_count()
             : (geometry < -1 || geometry >= skipln::rowtile_count()))
        return SKIPLN_ERR_VARIANT;
    skipln::Tiling t;
    t.tiles_per_block = tiles_per_block;
    t.mode = tiling;
    const int variant = elem ? geometry : geometry < 0 ? SKIPLN_VARIANT_ROWTILE : SKIPLN_VARIANT_GEOMETRY + geometry;
    return run(make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                         dtype),
               variant, &t, stream);
}

int skipln_forward(const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
                   const void* beta, const void* bias, void* out, void* residual_out, int64_t rows, int64_t hidden,
                   float eps, int dtype, skipln_stream_t stream) {
    return skipln_forward_variant(SKIPLN_OP_LAYER_NORM, input, skip, skip_mode, skip_rows, gamma, beta, bias, out,
                                  residual_out, rows, hidden, eps, dtype, SKIPLN_VARIANT_AUTO, stream);
}

int skipln_forward_simplified(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                              const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                              int64_t rows, int64_t hidden, float eps, int dtype, skipln_stream_t stream) {
    return skipln_forward_variant(SKIPLN_OP_SIMPLIFIED, input, skip, skip_mode, skip_rows, gamma, beta, bias, out,
                                  residual_out, rows, hidden, eps, dtype, SKIPLN_VARIANT_AUTO, stream);
}

int skipln_bias_add(const void* x, const void* bias, const void* skip, void* y, int64_t rows, int64_t channels,
                    int dtype, skipln_stream_t stream) {
    return skipln_forward_variant(SKIPLN_OP_BIAS_ADD, x, skip, SKIPLN_SKIP_EXACT, 0, nullptr, nullptr, bias, y,
                                  nullptr, rows, channels, 0.0f, dtype, SKIPLN_VARIANT_AUTO, stream);
}

int skipln_bias_softmax(const void* data, const void* bias, void* out, int64_t batch_count, int64_t block_size,
                        int64_t bias_batch_count, int is_inner_broadcast, int dtype, void* workspace,
                        int64_t workspace_bytes, skipln_stream_t stream) {
    if (batch_count < 0 || block_size < 0 || bias_batch_count < 0) return SKIPLN_ERR_SHAPE;
    // `biasContract`: empty data with an empty bias is valid and does nothing.
    if ((batch_count == 0 || block_size == 0) && (bias_batch_count == 0 || block_size == 0)) {
        if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return SKIPLN_ERR_DTYPE;
        return SKIPLN_OK;
    }
    if (block_size == 0 || bias_batch_count == 0 || bias_batch_count > batch_count ||
        batch_count % bias_batch_count != 0)
        return SKIPLN_ERR_SHAPE;
    // One bias row per data row: both reuse forms read bias row r.
    const int mode = bias_batch_count == batch_count
                         ? SKIPLN_SKIP_EXACT
                         : (is_inner_broadcast ? SKIPLN_SKIP_BROADCAST_INNER : SKIPLN_SKIP_BROADCAST);
    if (workspace == nullptr)
        return skipln_forward_variant(SKIPLN_OP_BIAS_SOFTMAX, data, bias, mode, bias_batch_count, nullptr, nullptr,
                                      nullptr, out, nullptr, batch_count, block_size, 0.0f, dtype, SKIPLN_VARIANT_AUTO,
                                      stream);
    return skipln_forward_ws(SKIPLN_OP_BIAS_SOFTMAX, data, bias, mode, bias_batch_count, nullptr, nullptr, nullptr,
                             out, nullptr, batch_count, block_size, 0.0f, dtype, SKIPLN_VARIANT_AUTO, workspace,
                             workspace_bytes, stream);
}

int skipln_copy(void* dst, const void* src, int64_t bytes, skipln_stream_t stream) {
    if (bytes < 0 || bytes % 16 != 0) return SKIPLN_ERR_SHAPE;
    if (bytes == 0) return SKIPLN_OK;
    if (!dst || !src) return SKIPLN_ERR_NULL;
    if (!aligned16(dst) || !aligned16(src)) return SKIPLN_ERR_SHAPE;
    if (overlap(span(dst, bytes), span(src, bytes))) return SKIPLN_ERR_ALIAS;
    return status_of(skipln::launch_copy(dst, src, bytes / 16, reinterpret_cast<hipStream_t>(stream)));
}

int skipln_stream(const void* src0, const void* src1, void* dst0, void* dst1, int64_t bytes, int block,
                  int chunks_per_lane, int64_t xcd_granule, int store_through, skipln_stream_t stream) {
    if (!skipln::stream_shape_ok(block, chunks_per_lane)) return SKIPLN_ERR_VARIANT;
    if (xcd_granule < 1 || xcd_granule > skipln::kMaxStreamGranule) return SKIPLN_ERR_VARIANT;
    if (bytes < 0 || bytes % 16 != 0) return SKIPLN_ERR_SHAPE;
    if (src1 && !src0) return SKIPLN_ERR_NULL;   // inputs fill src0 first
    if (dst1 && !dst0) return SKIPLN_ERR_NULL;   // outputs fill dst0 first
    const int reads = (src0 != nullptr) + (src1 != nullptr);
    const int writes = (dst0 != nullptr) + (dst1 != nullptr);
    if (reads + writes == 0) return SKIPLN_ERR_NULL;
    if (bytes == 0) return SKIPLN_OK;
    for (const void* p : {src0, src1, static_cast<const void*>(dst0), static_cast<const void*>(dst1)})
        if (p && !aligned16(p)) return SKIPLN_ERR_SHAPE;
    const Range r[4] = {span(src0, src0 ? bytes : 0), span(src1, src1 ? bytes : 0), span(dst0, dst0 ? bytes : 0),
                        span(dst1, dst1 ? bytes : 0)};
    for (int o = 2; o < 4; ++o)
        for (int i = 0; i < 4; ++i)
            if (i != o && overlap(r[o], r[i])) return SKIPLN_ERR_ALIAS;
    return status_of(skipln::launch_stream(reads, writes, block, chunks_per_lane, xcd_granule, store_through != 0, src0,
                                           src1, dst0, dst1, bytes / 16, reinterpret_cast<hipStream_t>(stream)));
}

int skipln_rowtile_geometries(void) { return skipln::rowtile_count(); }

int skipln_element_geometries(void) { return skipln::elem_count(); }

const char* skipln_kernel_name(int kernel_id) { return skipln::kernel_name(kernel_id); }

const char* skipln_status_string(int status) {
    switch (status) {
        case SKIPLN_OK: return "ok";
        case SKIPLN_ERR_NULL: return "a required pointer is NULL";
        case SKIPLN_ERR_SHAPE: return "invalid shape (rows, hidden, skip_rows or bias rows)";
        case SKIPLN_ERR_DTYPE: return "unsupported element type";
        case SKIPLN_ERR_MODE: return "unknown or unsupported skip mode";
        case SKIPLN_ERR_EPS: return "epsilon must be a non-negative number";
        case SKIPLN_ERR_ALIAS: return "an output overlaps an input or the other output";
        case SKIPLN_ERR_UNSUPPORTED: return "the forced kernel family cannot run this shape or alignment";
        case SKIPLN_ERR_LAUNCH: return "kernel launch failed";
        case SKIPLN_ERR_DEVICE: return "no usable HIP device";
        case SKIPLN_ERR_VARIANT: return "unknown variant, geometry or tiling";
        case SKIPLN_ERR_OP: return "unknown operation";
        case SKIPLN_ERR_WORKSPACE: return "the workspace is missing, misaligned or too small";
        default: return "unknown status";
    }
}

int skipln_version(void) { return 1; }

}  // extern "C"
