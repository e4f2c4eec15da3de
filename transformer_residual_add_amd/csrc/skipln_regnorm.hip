// Register-resident long rows of the normalizations: SkipLayerNormalization
// and its root-mean-square form (SkipLayerNormalization manifest:
// `description`, `inputs`, `outputs`, `attributes.epsilon`) for rows longer
// than one workgroup's LDS holds, up to 65,536 values.
//
// One 1024-lane block per row at a time, persistent over rows.  Lane t keeps
// the binary32 sums s = (x + skip) + bias of its chunks t, t + 1024, ... in
// VGPRs (64 values per lane at 65,536 values per row), so every input crosses
// HBM once:
//   pass 1: every x and skip load of the row is issued at once (float16
//           skip chunks into registers; float32 ones, twice as wide, mostly
//           straight into LDS with direct-to-LDS buffer loads, the rest into
//           registers); the bias goes through a short register ring; s is
//           formed slab by slab;
//   statistics from the registers, exactly two-pass: the mean, then the sum
//           of squared deviations from it (the mean square for the
//           root-mean-square form), each merged across the block through LDS;
//   pass 2: residual (s rounded once) and output, gamma and beta through a
//           ring; once every store of the row is issued, the next row's loads
//           go out.
// Chunks past the row's end are read as zeros through the buffer range check
// and kept out of the statistics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skipln_device.h"
#include "skipln_internal.h"
#include "skipln_rowtile.h"

namespace skipln {
namespace {
using namespace device;

constexpr int kNormBlock = 1024;
constexpr int kNormSlabBytes = kNormBlock * 16;
constexpr int kNormMaxValues = 64;       // binary32 sums per lane
constexpr int kNormPastRow = 0x40000000; // lane offset beyond every row
constexpr int kNormNonTemporal = 2;      // cache policy of the streamed loads
constexpr int kParamAhead = 2;           // bias / gamma / beta slabs loaded ahead
constexpr int kLdsSkipSlabs = 9;         // float32 skip slabs loaded straight into LDS (144 KiB)

template <typename T, int OP, int CH>
__global__ void __launch_bounds__(kNormBlock) regnorm_kernel(const Args a) {
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr int W = kNormBlock / 64;
    static_assert(CH * V <= kNormMaxValues, "row held in registers");
    // Every load of a row is issued at once.  float16 skip chunks are as
    // small as the sums they become: they load into registers.  float32 ones
    // would double the row's registers: the first LS slabs load straight
    // into LDS (16-byte direct-to-LDS buffer loads), the rest into registers.
    constexpr int LS = sizeof(T) == 4 ? (kLdsSkipSlabs < CH ? kLdsSkipSlabs : CH) : 0;
    constexpr int SA = CH - LS;  // skip slabs in registers
    // The longest float32 rows leave room for one parameter slab ahead only.
    constexpr int PA = sizeof(T) == 4 && CH >= 16 ? 1 : (kParamAhead < CH ? kParamAhead : CH);
    __shared__ float4 red[2][W];
    extern __shared__ u32x4 lskip[];  // LS slabs of kNormBlock chunks

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int hv = a.hidden / V;
    const int row_bytes = hv * 16;
    const int lane_off = tid * 16;
    const int nk_lane = (hv - tid + kNormBlock - 1) / kNormBlock;
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const bool through = a.store_through != 0;
    const float inv_h = 1.0f / static_cast<float>(a.hidden);
    const u32x4* X = static_cast<const u32x4*>(a.input);
    const u32x4* S = static_cast<const u32x4*>(a.skip);
    // Absent beta / bias: a resource of size 0, whose loads read zeros.
    const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(a.gamma, row_bytes);
    const __amdgpu_buffer_rsrc_t betar = buffer_rsrc(a.beta, a.beta ? row_bytes : 0);
    const __amdgpu_buffer_rsrc_t biasr = buffer_rsrc(a.bias, a.bias ? row_bytes : 0);

    // Lane offset of chunk k (this lane's, or one the range check refuses);
    // re-read through an empty asm at each pass so that the offsets are
    // formed where they are used rather than kept live.
    int lofs = lane_off, nk = nk_lane;
    auto refresh = [&]() {
        lofs = lane_off;
        nk = nk_lane;
        asm volatile("" : "+v"(lofs), "+v"(nk));
    };
    auto lo = [&](int k) { return k < nk ? lofs : kNormPastRow; };
    refresh();

    u32x4 xq[CH];
    u32x4 sq[SA > 0 ? SA : 1];
    int64_t row = blockIdx.x;
    int64_t srow = 0;  // skip row of the row whose loads are in flight
    auto issue_row = [&](int64_t r) {
        // r >= rows: an empty range, no memory access.
        const bool live = r < a.rows;
        srow = live ? skip_row_of(r, a, small_rows) : 0;
        const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(X + (live ? r : 0) * hv, live ? row_bytes : 0);
        const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(S + srow * hv, live ? row_bytes : 0);
#pragma unroll
        for (int k = 0; k < CH; ++k)
            xq[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, lo(k), k * kNormSlabBytes, kNormNonTemporal);
        // Lane t of wavefront w writes its chunk at LDS chunk k * kNormBlock +
        // 64 w + t: every lane later reads back only its own chunk.
        // (The direct-to-LDS builtin exists for the device pass only; the
        // host pass, which emits just the launch stub, must not see it.)
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int k = 0; k < LS; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                sr, (__attribute__((address_space(3))) void*)(lskip + k * kNormBlock + wave * 64), 16, lo(k),
                k * kNormSlabBytes, 0, kNormNonTemporal);
#endif
#pragma unroll
        for (int k = 0; k < SA; ++k)
            sq[k] = __builtin_amdgcn_raw_buffer_load_b128(sr, lo(LS + k), (LS + k) * kNormSlabBytes,
                                                          kNormNonTemporal);
    };
    issue_row(row);

    int buf = 0;
    for (; row < a.rows; row += gridDim.x) {
        refresh();
        // Pass 1: s = (x + skip) + bias in binary32.
        u32x4 bq[PA];
#pragma unroll
        for (int j = 0; j < PA; ++j) bq[j] = __builtin_amdgcn_raw_buffer_load_b128(biasr, lo(j), j * kNormSlabBytes, 0);
        // The skip slabs in LDS are read back once every load of the row
        // has landed (all were issued together; the bias just after).
        if constexpr (LS > 0) __builtin_amdgcn_s_waitcnt(0);
        float s[CH][V];
        // Layer norm sums s - sh, sh = the wavefront's first sum (chunk 0 of
        // its lane 0 always lies in the row), so that rounding scales with
        // the row's spread rather than its offset from zero.
        float acc = 0.0f, sh = 0.0f;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const u32x4 sk = k < LS ? lskip[k * kNormBlock + tid] : sq[k - LS];
            const u32x4 bk = bq[k % PA];
            if (k + PA < CH)
                bq[k % PA] = __builtin_amdgcn_raw_buffer_load_b128(biasr, lo(k + PA), (k + PA) * kNormSlabBytes, 0);
            float xf[V], sf[V], bf[V];
            E::widen(xq[k], xf);
            E::widen(sk, sf);
            E::widen(bk, bf);
            // Chunks past the row's end (whatever their sums) contribute
            // nothing; their stores are dropped by the range check.
#pragma unroll
            for (int e = 0; e < V; ++e) s[k][e] = (xf[e] + sf[e]) + bf[e];
            if constexpr (OP != kOpSimplified)
                if (k == 0) sh = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s[0][0])));
            const bool valid = k < nk;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if constexpr (OP == kOpSimplified)
                    acc += valid ? s[k][e] * s[k][e] : 0.0f;
                else
                    acc += valid ? s[k][e] - sh : 0.0f;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Statistics: per wavefront, then across the block through LDS.
        // Layer norm: the mean relative to wavefront 0's shift sh0,
        //   dmean = sum_w (n_w (sh_w - sh0) + sum_w (s - sh_w)) / H,
        // then the squared deviations ((s - sh0) - dmean)^2 from registers.
        // off: what to subtract from s - sh0 (0 for the root-mean-square form).
        float sh0 = 0.0f, off = 0.0f, var;
        const float wacc = wave_sum(acc);
        if constexpr (OP == kOpSimplified) {
            if ((tid & 63) == 0) red[buf][wave] = make_float4(wacc, 0.0f, 0.0f, 0.0f);
            __syncthreads();
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) tot += red[buf][w].x;
            buf ^= 1;
            var = tot * inv_h;
        } else {
            const float wn = wave_sum(static_cast<float>(nk * V));
            if ((tid & 63) == 0) red[buf][wave] = make_float4(sh, wacc, wn, 0.0f);
            __syncthreads();
            sh0 = red[buf][0].x;
            float dsum = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float4 p = red[buf][w];
                dsum += p.z * (p.x - sh0) + p.y;
            }
            buf ^= 1;
            off = dsum * inv_h;
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const bool valid = k < nk;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float d = (s[k][e] - sh0) - off;
                    q += valid ? d * d : 0.0f;
                }
            }
            const float wq = wave_sum(q);
            if ((tid & 63) == 0) red[buf][wave] = make_float4(wq, 0.0f, 0.0f, 0.0f);
            __syncthreads();
            float m2 = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) m2 += red[buf][w].x;
            buf ^= 1;
            var = m2 * inv_h;
        }
        const float rstd = rsqrtf(var + a.eps);

        // Pass 2: residual and output.
        const __amdgpu_buffer_rsrc_t orow = buffer_rsrc(static_cast<char*>(a.out) + row * row_bytes, row_bytes);
        const __amdgpu_buffer_rsrc_t rrow = buffer_rsrc(a.residual ? static_cast<char*>(a.residual) + row * row_bytes
                                                                   : nullptr,
                                                        a.residual ? row_bytes : 0);
        refresh();
        u32x4 gq[PA], eq[PA];
#pragma unroll
        for (int j = 0; j < PA; ++j) {
            gq[j] = __builtin_amdgcn_raw_buffer_load_b128(gr, lo(j), j * kNormSlabBytes, 0);
            eq[j] = __builtin_amdgcn_raw_buffer_load_b128(betar, lo(j), j * kNormSlabBytes, 0);
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const u32x4 gk = gq[k % PA], ek = eq[k % PA];
            if (k + PA < CH) {
                gq[k % PA] = __builtin_amdgcn_raw_buffer_load_b128(gr, lo(k + PA), (k + PA) * kNormSlabBytes, 0);
                eq[k % PA] = __builtin_amdgcn_raw_buffer_load_b128(betar, lo(k + PA), (k + PA) * kNormSlabBytes, 0);
            }
            // s again, not the deviations the statistics formed: keeping
            // those alive as well would double the row's registers.
#pragma unroll
            for (int e = 0; e < V; ++e) asm volatile("" : "+v"(s[k][e]));
            // Stores take their whole offset in the vector offset (a scalar
            // slab offset leaves the data registers unguarded against the
            // next instruction's writes).
            const int voff = lo(k) + k * kNormSlabBytes;
            if (a.residual) E::store(E::narrow(s[k]), rrow, voff, 0, through);
            float t[V], y[V];
#pragma unroll
            for (int e = 0; e < V; ++e) t[e] = ((s[k][e] - sh0) - off) * rstd;
            E::widen_fma(t, gk, ek, y);
            E::store(E::narrow(y), orow, voff, 0, through);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The next row's loads, after every store of this one.
        refresh();
        issue_row(row + gridDim.x);
    }
}

template <typename T, int OP, int CH>
hipError_t launch_ch(const Args& a, hipStream_t st) {
    auto kernel = regnorm_kernel<T, OP, CH>;
    constexpr size_t lds = sizeof(T) == 4 ? static_cast<size_t>(kLdsSkipSlabs < CH ? kLdsSkipSlabs : CH) * kNormSlabBytes
                                          : 0;
    static int occ_cache = 0;
    int occ = __atomic_load_n(&occ_cache, __ATOMIC_RELAXED);
    if (occ <= 0) {
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kNormBlock, lds);
        if (e != hipSuccess) return e;
        if (occ < 1) return hipErrorInvalidConfiguration;
        __atomic_store_n(&occ_cache, occ, __ATOMIC_RELAXED);
    }
    int cus = 0;
    const hipError_t e = rowtile::cu_count(&cus);
    if (e != hipSuccess) return e;
    int64_t blocks = static_cast<int64_t>(cus) * occ;
    if (a.rows < blocks) blocks = a.rows;
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)),
                           dim3(kNormBlock), params, lds, st);
}

// Slab counts compiled: the smallest that covers the row.
template <typename T, int OP>
hipError_t launch_t(const Args& a, hipStream_t st) {
    const int hv = a.hidden / Elem<T>::kPerChunk;
    const int n = (hv + kNormBlock - 1) / kNormBlock;
    if constexpr (sizeof(T) == 4) {
        if (n <= 10) return launch_ch<T, OP, 10>(a, st);
        if (n <= 12) return launch_ch<T, OP, 12>(a, st);
        if (n <= 14) return launch_ch<T, OP, 14>(a, st);
        if (n <= 16) return launch_ch<T, OP, 16>(a, st);
    } else {
        if (n <= 5) return launch_ch<T, OP, 5>(a, st);
        if (n <= 6) return launch_ch<T, OP, 6>(a, st);
        if (n <= 7) return launch_ch<T, OP, 7>(a, st);
        if (n <= 8) return launch_ch<T, OP, 8>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool regnorm_holds(int op, int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    // Rows the compiled slab counts cover: at most 64 values per lane, and
    // long enough for the smallest count (shorter rows have the LDS kernel).
    const int64_t min_slabs = dtype == 0 ? 10 : 5;
    return (op == kOpLayerNorm || op == kOpSimplified) && hidden > 0 && hidden % v == 0 &&
           hidden <= static_cast<int64_t>(kNormBlock) * kNormMaxValues &&
           hidden / v > (min_slabs - 1) * static_cast<int64_t>(kNormBlock);
}

hipError_t launch_regnorm(const Args& a, int op, int dtype, hipStream_t st) {
    if (op == kOpLayerNorm)
        return dtype == 0 ? launch_t<float, kOpLayerNorm>(a, st) : launch_t<_Float16, kOpLayerNorm>(a, st);
    if (op == kOpSimplified)
        return dtype == 0 ? launch_t<float, kOpSimplified>(a, st) : launch_t<_Float16, kOpSimplified>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace skipln
