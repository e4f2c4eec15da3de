// Host logic of libskipln shared by both C ABIs: argument checks, kernel
// choice and launch.
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
#include "skipln_core.h"

#include <atomic>

static_assert(SKIPLN_OP_LAYER_NORM == skipln::kOpLayerNorm && SKIPLN_OP_SIMPLIFIED == skipln::kOpSimplified &&
                  SKIPLN_OP_BIAS_ADD == skipln::kOpBiasAdd && SKIPLN_OP_BIAS_SOFTMAX == skipln::kOpBiasSoftmax,
              "operations of the ABI and the kernels agree");

namespace skipln {
namespace core {
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

bool normalizing(int op) { return op == SKIPLN_OP_LAYER_NORM || op == SKIPLN_OP_SIMPLIFIED; }

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

// Many long RMS rows (past the register-resident kernel's 65,536 values):
// the generic kernel's chunk form (one 1024-lane workgroup per row, the
// row's first 40,832 sums parked in LDS, no workspace) outruns the split-row
// kernels once there is a row for every compute unit.  Measured on MI355X
// (256 CUs), generic / split-row time: RMS 0.80-0.93 for 256 to 2048 rows of
// 65,536 to 262,144 values (either type; 0.99 at 128 rows); layer norm
// 0.92-1.08 beyond 65,536 values (the split-row kernels kept).
bool generic_outruns_split(int op, int64_t rows, int cus) {
    if (rows < 0 || cus <= 0 || rows < cus) return false;
    return op == SKIPLN_OP_SIMPLIFIED;
}

// Tiling of the automatic launch.  Streaming rows (exact skip): one tile per
// block, so blocks are dispatched in address order and the set of rows in
// flight stays compact; this reached the 2-read/2-write streaming rate on
// MI355X.  A cyclic broadcast skip is shared by every batch: each block of a
// normalization keeps its skip rows (and gamma/beta) in registers and walks a
// few batches (the launcher's default).  BiasSoftmax has no parameters to
// keep: it streams its rows in address order, its bias rows served by the
// caches, as long as the bias fits them (and always with grouped (inner)
// reuse, whose consecutive rows share a bias row).  A cyclic bias of 16 MiB
// or more (a per-head position bias of a long sequence) is re-read from HBM
// by every batch when streamed, so those launches keep it stationary too,
// walking every batch (up to 8) once it exceeds the last-level cache.
// Measured on MI355X, float16 attention scores of 8 batches x 16 heads:
// 1024 / 2048 / 8192 keys (bias of 32 / 128 / 512 MiB) 113.9 / 436.7 /
// 2078.8 us streamed, 95.5 / 360.0 / 1747.3 stationary over 3 batches,
// 1631.3 over 8 at 8192 keys (365.8 at 2048); float32 4096 keys 2103.2 ->
// 1630.2.  An 8 MiB bias streamed 1.5 % faster (91.3 against 92.7).
// Normalizations with a skip of 16 MiB or more walk 8 batches per block
// instead of 3, re-reading the skip less often: layer norm float16 (32, 2048,
// 8192) / (64, 1024, 8192) / (32, 4096, 4096) 403.4 / 402.9 / 380.7 ->
// 366.7 / 365.4 / 359.9 us, float32 (16, 4096, 4096) 375.6 -> 366.7, RMS
// float16 (32, 2048, 8192) 370.7 -> 366.3; with the 8 MiB skip of (64, 512,
// 4096) float32 the two were within 1 % (182.2 / 183.6).
Tiling auto_tiling(int op, int skip_mode, int64_t skip_bytes) {
    const bool softmax = op == SKIPLN_OP_BIAS_SOFTMAX;
    const bool big = skip_bytes >= (int64_t{16} << 20);
    const bool cyclic = skip_mode == SKIPLN_SKIP_BROADCAST && (!softmax || big);
    const bool walk_all = softmax ? skip_bytes >= (int64_t{256} << 20) : big;
    Tiling t;
    t.tiles_per_block = cyclic ? (walk_all ? 8 : 0) : 1;
    t.mode = cyclic ? kTileSkipStationary : kTileStrided;
    return t;
}

Args make_args(const Call& c, int store) {
    Args a;
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
    a.tiling = kTileStrided;
    // Bytes the launch writes: the output, and the residual when emitted.
    // The system-scope store policy serves large launches of rows of whole
    // 128-byte lines only: where rows end inside a line (so every row's
    // first and last line are written partly), it measured 14-19 % slower
    // than non-temporal stores on MI355X (2 GiB launches: float16 rows of
    // 2056 / 4104 / 8200 values 500 / 489 / 485 against 431 / 417 / 391 us,
    // float32 rows of 1028 values 511 against 420), while on whole-line rows
    // it is the faster one (float16 rows of 2048 values: 367 against 375).
    const int64_t row_bytes = c.hidden * (c.dtype == SKIPLN_F32 ? 4 : 2);
    const int64_t written = c.rows * row_bytes * (c.residual ? 2 : 1);
    a.store_through = store == kStoreAuto ? (written >= kStoreThroughBytes && row_bytes % 128 == 0 ? 1 : 0)
                                          : (store == kStoreThrough);
    return a;
}

// Whether the workspace serves the call: present, aligned, large enough and
// overlapping no tensor (SKIPLN_OK when it does).
int check_workspace(const Call& c, const Workspace* ws, int index) {
    if (!ws || !ws->ptr || !aligned16(ws->ptr) || ws->bytes < workspace_needed(c, index)) return SKIPLN_ERR_WORKSPACE;
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
    return SKIPLN_OK;
}

}  // namespace

bool known_op(int op) {
    return op == SKIPLN_OP_LAYER_NORM || op == SKIPLN_OP_SIMPLIFIED || op == SKIPLN_OP_BIAS_ADD ||
           op == SKIPLN_OP_BIAS_SOFTMAX;
}

// Skip forms an operation accepts: grouped (inner) reuse is BiasSoftmax's.
bool mode_ok(int op, int skip_mode) {
    if (skip_mode == SKIPLN_SKIP_EXACT) return true;
    if (skip_mode == SKIPLN_SKIP_BROADCAST) return op != SKIPLN_OP_BIAS_ADD;
    if (skip_mode == SKIPLN_SKIP_BROADCAST_INNER) return op == SKIPLN_OP_BIAS_SOFTMAX;
    return false;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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

int select(int op, int64_t hidden, int dtype, bool broadcast, bool vec_ok, bool elem_ok, int variant,
           bool with_workspace, int64_t rows, int cus) {
    const int base = (op * 2 + dtype) * kIdsPerType;
    const int v = dtype == SKIPLN_F32 ? 4 : 8;  // elements per 16-byte chunk
    const bool chunked = vec_ok && hidden % v == 0;
    if (variant == kVariantGeneric) return base + kGenericIndex;
    if (variant == kVariantElement) {
        const int g = elem_ok ? elem_pick(op, hidden) : -1;
        return g >= 0 ? base + kElemFirst + g : -SKIPLN_ERR_UNSUPPORTED;
    }
    if (variant == kVariantSpan) {
        const int g = vec_ok ? span_fit(op, hidden, dtype) : -1;
        return g >= 0 ? base + kSpanFirst + g : -SKIPLN_ERR_UNSUPPORTED;
    }
    if (variant >= kVariantSpanGeometry && variant < kVariantSpanGeometry + span_count()) {
        const int g = variant - kVariantSpanGeometry;
        if (!vec_ok || !span_holds(g, hidden, dtype)) return -SKIPLN_ERR_UNSUPPORTED;
        return base + kSpanFirst + g;
    }
    if (variant >= kVariantElementGeometry && variant < kVariantElementGeometry + elem_count()) {
        const int g = variant - kVariantElementGeometry;
        if (!elem_ok || !elem_holds(g, hidden)) return -SKIPLN_ERR_UNSUPPORTED;
        return base + kElemFirst + g;
    }
    const bool lds_ok = vec_ok && ldsrow_holds(op, hidden, dtype);
    const bool split_ok = vec_ok && split_holds(op, hidden, dtype);
    const bool reg_ok = vec_ok && regrow_holds(op, hidden, dtype);
    if (variant == kVariantLdsRow) return lds_ok ? base + kLdsRowIndex : -SKIPLN_ERR_UNSUPPORTED;
    if (variant == kVariantSplitRow) return split_ok ? base + kSplitRowIndex : -SKIPLN_ERR_UNSUPPORTED;
    if (variant == kVariantRegRow) return reg_ok ? base + kRegRowIndex : -SKIPLN_ERR_UNSUPPORTED;
    // Long rows of the reducing operations: staged in LDS; beyond its
    // capacity held in registers, or split across workgroups when a
    // workspace is at hand.
    if (variant == kVariantAuto && hidden / v > kRowtileMaxAutoChunks) {
        // Large launches of normalization rows of up to 3072 chunks (whole
        // cache lines): 1024-lane row tiles in the single-tile form outrun
        // the LDS-staged kernel.  Measured on MI355X, 2 GiB launches (rows x
        // (input, skip, residual, output)): float32 rows of 8224 / 8448 /
        // 10240 / 11264 / 12288 values 447.9 / 439.0 / 413.2 / 405.3 / 397.9
        // -> 373.3 / 371.5 / 363.2 / 373.7 / 376.1 us; float16 rows of 22528
        // / 24576 values 427.1 / 418.2 -> 413.6 / 404.0; float16 rows of
        // 20480 values 431.3 against 436.2, so float16 layer norm stays on
        // the LDS kernel below 2689 chunks.  float16 RMS (58 VGPRs, two
        // blocks per CU where layer norm holds one) gains from 2304 chunks:
        // rows of 18432 / 20480 values 436.9 / 465.4 -> 422.0 / 437.9 us at
        // 16384 rows.  float32 rows of 3073-4096 chunks run 1024 x 4 tiles
        // (32768 rows of 14336 / 16384 values: layer norm 1420.4 / 1927.1 ->
        // 1360 / 1706 us, RMS of 16384 values 1794.0 -> 1604.9; 16384 rows:
        // 692.8 / 961.8 -> 680.3 / 930.1, RMS 937.5 -> 906.0), though layer
        // norm at the size threshold itself (8192 rows of 16384 values) ran
        // 408.1 against 382.3; float16 rows of that length stay on the LDS
        // kernel.
        const int64_t hv = hidden / v;
        const int64_t hv_min = dtype == SKIPLN_F32 ? 2049 : op == SKIPLN_OP_SIMPLIFIED ? 2304 : 2689;
        const int64_t hv_max = dtype == SKIPLN_F32 ? 4096 : 3072;
        if (chunked && !broadcast && (op == SKIPLN_OP_LAYER_NORM || op == SKIPLN_OP_SIMPLIFIED) && hv >= hv_min &&
            hv <= hv_max && single_tile_launch(rows, hidden, dtype == SKIPLN_F32 ? 4 : 2)) {
            const int g = rowtile_pick(op, hidden, dtype, false, false);
            if (g >= 0) return base + kRowtileFirst + g;
        }
        if (lds_ok) return base + kLdsRowIndex;
        // Register-resident rows (measured on MI355X against the generic and
        // split-row kernels, 65,536-value rows: float16 11-27 % faster from
        // 128 to 4096 rows; float32 7-19 % faster at 256-512 and 2048-4096
        // rows, within 5 % at 1024).
        if (reg_ok) return base + kRegRowIndex;
        if (split_ok && with_workspace && !generic_outruns_split(op, rows, cus))
            return base + kSplitRowIndex;
    }
    if (variant == kVariantAuto || variant == kVariantRowtile || variant == kVariantMultiwave) {
        const int g = chunked ? rowtile_pick(op, hidden, dtype, broadcast, variant == kVariantMultiwave, rows) : -1;
        if (g >= 0) return base + kRowtileFirst + g;
        if (variant != kVariantAuto) return -SKIPLN_ERR_UNSUPPORTED;
        // Rows that are not whole chunks: span row tiles (16-byte aligned
        // tensors), else element-wise row tiles, then the generic kernel.
        const int sp = vec_ok && !chunked ? span_pick(op, hidden, dtype, broadcast) : -1;
        if (sp >= 0) return base + kSpanFirst + sp;
        const int e = elem_ok && !chunked ? elem_pick(op, hidden) : -1;
        if (e >= 0) return base + kElemFirst + e;
        return base + kGenericIndex;
    }
    if (variant >= kVariantGeometry && variant < kVariantGeometry + rowtile_count()) {
        const int g = variant - kVariantGeometry;
        // The geometry must hold the whole row.
        if (!chunked || !rowtile_holds(g, hidden, dtype)) return -SKIPLN_ERR_UNSUPPORTED;
        return base + kRowtileFirst + g;
    }
    return -SKIPLN_ERR_VARIANT;
}

int64_t workspace_needed(const Call& c, int index) {
    if (index != kSplitRowIndex) return 0;
    return split_workspace_bytes(make_args(c, kStoreAuto), c.dtype);
}

int64_t auto_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode, int64_t skip_rows) {
    if (!known_op(op)) return -SKIPLN_ERR_OP;
    if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return -SKIPLN_ERR_DTYPE;
    if (!mode_ok(op, skip_mode)) return -SKIPLN_ERR_MODE;
    if (rows < 0 || hidden <= 0 || hidden > INT32_MAX) return -SKIPLN_ERR_SHAPE;
    if (skip_mode != SKIPLN_SKIP_EXACT && (skip_rows <= 0 || rows % skip_rows != 0)) return -SKIPLN_ERR_SHAPE;
    // With a workspace and as few rows as no device has compute units, the
    // automatic choice takes the split-row pair wherever it may.
    const int id =
        select(op, hidden, dtype, skip_mode != SKIPLN_SKIP_EXACT, true, true, kVariantAuto, true, -1, 0);
    if (id < 0) return id;
    if (id % kIdsPerType != kSplitRowIndex || rows == 0) return 0;
    const Call c = make_call(op, nullptr, nullptr, skip_mode, skip_rows, nullptr, nullptr, nullptr, nullptr, nullptr,
                             rows, hidden, 0.0f, dtype);
    return workspace_needed(c, kSplitRowIndex);
}

hipError_t device_cus(int* cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::atomic<int> cache[64];
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return hipSuccess;
}

int status_of(hipError_t e) {
    if (e == hipSuccess) return SKIPLN_OK;
    if (e == hipErrorInvalidDevice || e == hipErrorNoDevice) return SKIPLN_ERR_DEVICE;
    return SKIPLN_ERR_LAUNCH;
}

int run(const Call& c, int variant, const Tiling* tiling, skipln_stream_t stream, const Workspace* ws, int store) {
    const int st = validate(c);
    if (st != SKIPLN_OK) return st;
    const bool vec = all_aligned16(c), elem = all_element_aligned(c), bcast = c.skip_mode != SKIPLN_SKIP_EXACT;
    // First the choice for a device of any size (the row count decides only
    // the large-launch rule); where that is the split-row pair the workspace
    // must serve (checked before any HIP call), and the device's compute
    // units decide between it and the generic kernel.
    int id = select(c.op, c.hidden, c.dtype, bcast, vec, elem, variant, ws != nullptr, c.rows, 0);
    if (id < 0) return -id;
    if (c.rows == 0) return SKIPLN_OK;
    if (id % kIdsPerType == kSplitRowIndex && variant == kVariantAuto) {
        const bool residual_aliases = c.residual && (c.residual == c.input || c.residual == c.skip);
        if (!residual_aliases) {
            const int w = check_workspace(c, ws, kSplitRowIndex);
            if (w != SKIPLN_OK) return w;
        }
        int cus = 0;
        const hipError_t e = device_cus(&cus);
        if (e != hipSuccess) return status_of(e);
        id = select(c.op, c.hidden, c.dtype, bcast, vec, elem, variant, true, c.rows, cus);
        if (id < 0) return -id;
    }
    const Args a = make_args(c, store);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int index = id % kIdsPerType;
    if (index == kSplitRowIndex && c.residual && (c.residual == c.input || c.residual == c.skip)) {
        // The split-row kernels read x and skip twice, so a residual written
        // over either cannot take them: the generic kernel can.
        if (variant != kVariantAuto) return SKIPLN_ERR_UNSUPPORTED;
        return status_of(launch_generic(a, c.op, c.dtype, s));
    }
    if (index == kSplitRowIndex) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;  // the split-row kernels have no tiling
        const int w = check_workspace(c, ws, index);
        if (w != SKIPLN_OK) return w;
        return status_of(launch_split(a, c.op, c.dtype, ws->ptr, s));
    }
    if (index == kGenericIndex) return status_of(launch_generic(a, c.op, c.dtype, s));
    if (index == kRegRowIndex) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;
        return status_of(launch_regrow(a, c.op, c.dtype, s));
    }
    if (index == kLdsRowIndex) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;  // the long-row kernel has no tiling
        return status_of(launch_ldsrow(a, c.op, c.dtype, s));
    }
    if (index >= kSpanFirst && index < kSpanFirst + span_count()) {
        if (tiling) return SKIPLN_ERR_UNSUPPORTED;  // one tile of rows per block
        return status_of(launch_span(a, c.op, c.dtype, index - kSpanFirst, s));
    }
    if (index >= kElemFirst) {
        const int g = index - kElemFirst;
        return status_of(launch_elem(a, c.op, c.dtype, g, tiling ? *tiling : elem_tiling(g), s));
    }
    const int64_t skip_bytes =
        c.skip_mode == SKIPLN_SKIP_BROADCAST ? c.skip_rows * c.hidden * (c.dtype == SKIPLN_F32 ? 4 : 2) : 0;
    const Tiling t = tiling ? *tiling : auto_tiling(c.op, c.skip_mode, skip_bytes);
    return status_of(launch_rowtile(a, c.op, c.dtype, index - kRowtileFirst, t, s));
}

}  // namespace core
}  // namespace skipln
