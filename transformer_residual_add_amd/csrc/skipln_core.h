// Host logic shared by the two C ABIs (the operator library, skipln_api.cpp,
// and the tuning library, skipln_tune_api.cpp): argument checks, kernel choice
// and launch.  Not installed; not part of either ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/skipln.h"
#include "skipln_internal.h"

namespace skipln {
namespace core {

// Kernel families (the tuning library's SKIPLN_VARIANT_* values).
constexpr int kVariantAuto = 0;
constexpr int kVariantGeneric = 1;
constexpr int kVariantRowtile = 2;
constexpr int kVariantMultiwave = 3;
constexpr int kVariantLdsRow = 4;
constexpr int kVariantSplitRow = 5;
constexpr int kVariantElement = 6;
constexpr int kVariantRegRow = 7;
constexpr int kVariantSpan = 8;
constexpr int kVariantGeometry = 64;
constexpr int kVariantElementGeometry = 128;
constexpr int kVariantSpanGeometry = 192;

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

// A caller's workspace: device memory for partial results.
struct Workspace {
    void* ptr;
    int64_t bytes;
};

// Output store policy of the row-tile and register-resident kernels:
// automatic (by the bytes a launch writes), non-temporal, or non-temporal
// with system-scope coherence.
constexpr int kStoreAuto = -1;
constexpr int kStoreStream = 0;
constexpr int kStoreThrough = 1;

bool known_op(int op);
bool mode_ok(int op, int skip_mode);
bool aligned16(const void* p);

Call make_call(int op, const void* input, const void* skip, int skip_mode, int64_t skip_rows, const void* gamma,
               const void* beta, const void* bias, const void* out, const void* residual_out, int64_t rows,
               int64_t hidden, float eps, int dtype);

// SKIPLN_OK or the status of the first failed check; host code only.
int validate(const Call& c);

// Kernel id (>= 0) for this variant, or -status.  vec_ok: tensors 16-byte
// aligned; elem_ok: aligned to their element size; with_workspace: the call
// brings a workspace, so the automatic choice may take the split-row kernels;
// rows: the call's row count (< 0: unknown, taken as fewer than `cus`); cus:
// the device's compute units (the automatic choice sends calls of at least
// that many long rows of some operations to the generic kernel instead of
// the split-row pair).
int select(int op, int64_t hidden, int dtype, bool broadcast, bool vec_ok, bool elem_ok, int variant,
           bool with_workspace, int64_t rows, int cus);

// Workspace bytes a launch of kernel `index` (per type) needs for this call.
int64_t workspace_needed(const Call& c, int index);

// Workspace bytes the automatic choice may need for these arguments on any
// device (the split-row pair's, when it can run the rows; 0 otherwise), or
// -status.  Host code only.
int64_t auto_workspace_bytes(int op, int64_t rows, int64_t hidden, int dtype, int skip_mode, int64_t skip_rows);

// Compute units of the current device (HIP call; cached per device).
hipError_t device_cus(int* cus);

// Validate, choose and launch.  `tiling` == nullptr: automatic tiling;
// `ws` == nullptr: the call brings no workspace; `store`: kStore*.
int run(const Call& c, int variant, const Tiling* tiling, skipln_stream_t stream, const Workspace* ws = nullptr,
        int store = kStoreAuto);

int status_of(hipError_t e);

}  // namespace core
}  // namespace skipln
