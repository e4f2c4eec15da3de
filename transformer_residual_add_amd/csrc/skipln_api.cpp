// C ABI of the operator library (include/skipln.h): each entry point builds
// the call, and the shared host logic (skipln_core.cpp) validates it, picks
// the kernel and launches it.  Every other symbol of the library is hidden.
#include "../../include/skipln.h"
#include "skipln_core.h"

using skipln::core::Call;
using skipln::core::make_call;
using skipln::core::run;
using skipln::core::Workspace;

extern "C" {

SKIPLN_API int skipln_forward(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                              const void* gamma, const void* beta, const void* bias, void* out, void* residual_out,
                              int64_t rows, int64_t hidden, float eps, int dtype, skipln_stream_t stream) {
    return run(make_call(SKIPLN_OP_LAYER_NORM, input, skip, skip_mode, skip_rows, gamma, beta, bias, out,
                         residual_out, rows, hidden, eps, dtype),
               skipln::core::kVariantAuto, nullptr, stream);
}

SKIPLN_API int skipln_forward_simplified(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                         const void* gamma, const void* beta, const void* bias, void* out,
                                         void* residual_out, int64_t rows, int64_t hidden, float eps, int dtype,
                                         skipln_stream_t stream) {
    return run(make_call(SKIPLN_OP_SIMPLIFIED, input, skip, skip_mode, skip_rows, gamma, beta, bias, out,
                         residual_out, rows, hidden, eps, dtype),
               skipln::core::kVariantAuto, nullptr, stream);
}

SKIPLN_API int skipln_bias_add(const void* x, const void* bias, const void* skip, void* y, int64_t rows,
                               int64_t channels, int dtype, skipln_stream_t stream) {
    return run(make_call(SKIPLN_OP_BIAS_ADD, x, skip, SKIPLN_SKIP_EXACT, 0, nullptr, nullptr, bias, y, nullptr, rows,
                         channels, 0.0f, dtype),
               skipln::core::kVariantAuto, nullptr, stream);
}

SKIPLN_API int skipln_bias_softmax(const void* data, const void* bias, void* out, int64_t batch_count,
                                   int64_t block_size, int64_t bias_batch_count, int is_inner_broadcast, int dtype,
                                   void* workspace, int64_t workspace_bytes, skipln_stream_t stream) {
    if (batch_count < 0 || block_size < 0 || bias_batch_count < 0) return SKIPLN_ERR_SHAPE;
    // `biasContract`: empty data with an empty bias is valid and does nothing.
    if ((batch_count == 0 || block_size == 0) && (bias_batch_count == 0 || block_size == 0)) {
        if (dtype != SKIPLN_F32 && dtype != SKIPLN_F16) return SKIPLN_ERR_DTYPE;
        return SKIPLN_OK;
    }
    if (block_size == 0 || bias_batch_count == 0 || bias_batch_count > batch_count ||
        batch_count % bias_batch_count != 0)
        return SKIPLN_ERR_SHAPE;
    if (workspace_bytes < 0) return SKIPLN_ERR_WORKSPACE;
    // One bias row per data row: both reuse forms read bias row r.
    const int mode = bias_batch_count == batch_count
                         ? SKIPLN_SKIP_EXACT
                         : (is_inner_broadcast ? SKIPLN_SKIP_BROADCAST_INNER : SKIPLN_SKIP_BROADCAST);
    const Call c = make_call(SKIPLN_OP_BIAS_SOFTMAX, data, bias, mode, bias_batch_count, nullptr, nullptr, nullptr,
                             out, nullptr, batch_count, block_size, 0.0f, dtype);
    if (workspace == nullptr) return run(c, skipln::core::kVariantAuto, nullptr, stream);
    const Workspace ws{workspace, workspace_bytes};
    return run(c, skipln::core::kVariantAuto, nullptr, stream, &ws);
}

SKIPLN_API int skipln_forward_ws(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                                 const void* gamma, const void* beta, const void* bias, void* out,
                                 void* residual_out, int64_t rows, int64_t hidden, float eps, int dtype,
                                 void* workspace, int64_t workspace_bytes, skipln_stream_t stream) {
    if (workspace_bytes < 0) return SKIPLN_ERR_WORKSPACE;
    const Workspace ws{workspace, workspace_bytes};
    return run(make_call(op, input, skip, skip_mode, skip_rows, gamma, beta, bias, out, residual_out, rows, hidden, eps,
                         dtype),
               skipln::core::kVariantAuto, nullptr, stream, &ws);
}

SKIPLN_API int64_t skipln_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode,
                                          int64_t skip_rows) {
    return skipln::core::auto_workspace_bytes(op, rows, hidden, dtype, skip_mode, skip_rows);
}

SKIPLN_API int skipln_validate(const void* input, const void* skip, int skip_mode, int64_t skip_rows,
                               const void* gamma, const void* beta, const void* bias, const void* out,
                               const void* residual_out, int64_t rows, int64_t hidden, float eps, int dtype) {
    return skipln::core::validate(make_call(SKIPLN_OP_LAYER_NORM, input, skip, skip_mode, skip_rows, gamma, beta, bias,
                                            out, residual_out, rows, hidden, eps, dtype));
}

SKIPLN_API const char* skipln_status_string(int status) {
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

SKIPLN_API int skipln_version(void) { return 2; }

}  // extern "C"
