// Row kernels for gfx950 (CDNA4, wave64): SkipLayerNormalization, its
// root-mean-square form, BiasAdd and BiasSoftmax.
//
// SkipLayerNormalization (com.microsoft SkipLayerNormalization WebGPU
// manifest): `description` (skip addition fused with a layer normalization
// over the hidden axis), `inputs[skip]` (exact, or broadcast over the batch
// with numel(skip)/H rows, the `Params.skipRows` of the broadcast binding
// set), `inputs[bias]` (joins input + skip before the normalization),
// `inputs[gamma]` / `inputs[beta]`, `outputs[input_skip_bias_sum]`,
// `attributes.epsilon`.  Statistics are the population mean and variance of
// the binary32 sum; all arithmetic is binary32, float16 only at load/store.
// BiasAdd (com.microsoft BiasAdd manifest) is the same sum without the
// normalization, in the order (x + bias) + skip.  BiasSoftmax (com.microsoft
// BiasSoftmax manifest) is a softmax over each row of data + bias, the bias
// rows arriving through the skip slot (exact, cyclic, or grouped reuse).
//
// The work is bound by HBM bandwidth (about 1 flop per byte moved), so the
// kernels are organised around moving each byte once:
//   * rowtile_kernel: a group of G lanes owns one row at a time and keeps the
//     whole row in VGPRs between the reduction and the output, so x and skip
//     are read from HBM exactly once.  Every access is a 16-byte vector
//     load/store (4 fp32 or 8 fp16), coalesced across the group.  G is 4..32
//     (several rows per wavefront, short rows), 64 (one wavefront per row)
//     or 128..1024 (several wavefronts per row, partial results combined
//     through LDS with one barrier per row).  Each block walks row tiles
//     (contiguous, strided, or skip-stationary), loads gamma/beta/bias into
//     registers once, and issues the loads of its next tile before it
//     reduces and stores the current one, keeping HBM requests in flight
//     across the reduction.  Streaming tensors use non-temporal accesses so
//     they do not displace the broadcast skip and the parameters in L2.
//   * ldsrow_kernel: rows too long for registers, staged in LDS (160 KiB per
//     workgroup on gfx950), one 1024-lane block per row.
//   * generic_kernel: any H and any alignment, one 256-lane block per row,
//     several passes over the row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdio>
#include <utility>

#include "skipln_device.h"
#include "skipln_internal.h"

namespace skipln {
namespace {
using namespace device;

// ------------------------------------------------------------------------
// Row-tile kernel.
// ------------------------------------------------------------------------
// Thread t of a row group owns chunks k*G + t (k < CH) of the row; a chunk
// past the row end (ragged hidden size) is skipped.  Number of elements of
// wavefront w of the group, for the cross-wave combine.
template <int G, int CH, int V>
__device__ __forceinline__ float wave_elems(int hv, int w) {
    int n = 0;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        int left = hv - (k * G + 64 * w);
        n += left <= 0 ? 0 : (left >= 64 ? 64 : left);
    }
    return static_cast<float>(n * V);
}

template <typename T, int OP, int G, int CH, int BLOCK>
__global__ void __launch_bounds__(BLOCK) rowtile_kernel(const Args a) {
    static_assert(OP == kOpLayerNorm || OP == kOpSimplified || OP == kOpBiasAdd || OP == kOpBiasSoftmax,
                  "operation");
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr bool kNorm = OP == kOpLayerNorm || OP == kOpSimplified;  // gamma/beta
    constexpr bool kParams = OP != kOpBiasSoftmax;                       // any per-column parameter
    constexpr int RPB = BLOCK / G;                  // rows per block per tile
    constexpr int WPR = G > 64 ? G / 64 : 1;        // wavefronts per row
    static_assert(BLOCK % G == 0 && BLOCK % 64 == 0, "block of whole groups and wavefronts");
    __shared__ float4 partial[2][RPB][WPR];

    const int tid = threadIdx.x;
    // Row of the tile handled by this group; wave-uniform when G >= 64, and
    // said so, so that row addresses live in scalar registers.
    const int slot = G >= 64 ? __builtin_amdgcn_readfirstlane(tid / G) : tid / G;
    const int lt = tid - slot * G; // lane within the group
    const int hv = a.hidden / V;   // chunks per row
    const float h = static_cast<float>(a.hidden);

    const u32x4* __restrict__ X = static_cast<const u32x4*>(a.input);
    const u32x4* __restrict__ S = static_cast<const u32x4*>(a.skip);
    u32x4* __restrict__ R = static_cast<u32x4*>(a.residual);
    u32x4* __restrict__ O = static_cast<u32x4*>(a.out);
    const bool has_bias = kParams && a.bias != nullptr;
    const bool has_beta = a.beta != nullptr;
    const bool bcast = a.skip_rows > 0 || a.skip_group > 0;
    const bool small_rows = a.rows <= 0xFFFFFFFFll;

    bool ok[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) ok[k] = k * G + lt < hv;

    // Parameters: loaded once per block, kept in registers (raw T bits).
    u32x4 gam[CH], bet[CH], bia[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        gam[k] = u32x4{0, 0, 0, 0};
        bet[k] = u32x4{0, 0, 0, 0};
        bia[k] = u32x4{0, 0, 0, 0};
    }
    auto load_params = [&]() {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int c = k * G + lt;
            if (ok[k]) {
                if constexpr (kNorm) {
                    gam[k] = static_cast<const u32x4*>(a.gamma)[c];
                    if (has_beta) bet[k] = static_cast<const u32x4*>(a.beta)[c];
                }
                if (has_bias) bia[k] = static_cast<const u32x4*>(a.bias)[c];
            }
        }
    };

    float nw[WPR];
#pragma unroll
    for (int w = 0; w < WPR; ++w) nw[w] = wave_elems<G, CH, V>(hv, w);
    const float own_n = wave_elems<G, CH, V>(hv, lt / 64);
    // Reciprocals once per block: the per-row statistics multiply (<= 1.5 ulp)
    // instead of dividing, which shortens the latency of short launches.
    const float inv_h = 1.0f / h;
    const float inv_own_n = own_n > 0.0f ? 1.0f / own_n : 0.0f;

    // Tiles (RPB consecutive rows each) of this block, T = tiles_per_block:
    //   contiguous:      b*T, b*T + 1, ..., b*T + T - 1
    //   strided:         b, b + grid, b + 2*grid, ...
    //   skip-stationary: with P = skip_rows / RPB tiles per batch, block b
    //                    owns tile column p = b mod P (the same skip rows in
    //                    every batch) and batches [c*T, c*T + T), c = b div P:
    //                    tiles p + n*P.  Its skip rows are loaded once.
    const int64_t n_tiles = (a.rows + RPB - 1) / RPB;
    int64_t t_first, stride, t_end;
    const bool stationary = a.tiling == kTileSkipStationary;
    if (a.tiling == kTileContiguous) {
        t_first = blockIdx.x * a.tiles_per_block;
        stride = 1;
        t_end = t_first + a.tiles_per_block < n_tiles ? t_first + a.tiles_per_block : n_tiles;
    } else if (a.tiling == kTileStrided) {
        t_first = blockIdx.x;
        stride = gridDim.x;
        t_end = n_tiles;
    } else {
        const int64_t P = a.skip_rows / RPB;
        const int64_t batches = a.rows / a.skip_rows;
        const int64_t n0 = (blockIdx.x / P) * a.tiles_per_block;
        const int64_t n1 = n0 + a.tiles_per_block < batches ? n0 + a.tiles_per_block : batches;
        t_first = n0 * P + blockIdx.x % P;
        stride = P;
        t_end = n1 * P;
    }

    u32x4 xr[CH], sr[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        xr[k] = u32x4{0, 0, 0, 0};
        sr[k] = u32x4{0, 0, 0, 0};
    }
    auto issue_loads = [&](int64_t tile, bool with_skip) {
        const int64_t row = tile * RPB + slot;
        if (row < a.rows) {
            const int64_t srow = skip_row_of(row, a, small_rows);
            const u32x4* xp = X + row * hv + lt;
            const u32x4* sp = S + srow * hv + lt;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
                    xr[k] = __builtin_nontemporal_load(xp + k * G);
                    // The broadcast skip is re-read by every batch: keep it cached.
                    if (with_skip) sr[k] = bcast ? sp[k * G] : __builtin_nontemporal_load(sp + k * G);
                }
            }
        }
    };

    // Order of the first loads (measured): a block that handles one tile
    // needs bias as soon as x and skip arrive, so parameters go first; a
    // long-lived skip-stationary block gets its first tile moving first.
    int64_t tile = t_first;
    if (stationary) {
        if (tile < t_end) issue_loads(tile, true);
        load_params();
    } else {
        load_params();
        if (tile < t_end) issue_loads(tile, true);
    }

    int parity = 0;

    for (; tile < t_end; tile += stride) {
        const int64_t row = tile * RPB + slot;
        const bool live = row < a.rows;
        if constexpr (V == 8 && kParams) {
            // Keep gamma/beta/bias packed (2 fp16 per VGPR): without this the
            // compiler hoists their widening out of the loop and triples
            // their register footprint, which costs occupancy.
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                asm volatile("" : "+v"(gam[k]), "+v"(bet[k]), "+v"(bia[k]));
            }
        }

        // s = (x + skip) + bias in binary32 (BiasAdd: (x + bias) + skip;
        // BiasSoftmax: data + bias, the bias arriving through the skip slot).
        float s[CH][V];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            float xf[V], sf[V], bf[V];
            E::widen(xr[k], xf);
            E::widen(sr[k], sf);
            E::widen(bia[k], bf);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float v;
                if constexpr (OP == kOpBiasAdd) {
                    v = xf[e] + bf[e];
                    v = v + sf[e];
                } else {
                    v = xf[e] + sf[e];
                    if (has_bias) v = v + bf[e];
                }
                s[k][e] = v;
            }
        }

        // Registers of x/skip are free again: start the next tile's loads.
        if (tile + stride < t_end) issue_loads(tile + stride, !stationary);

        if constexpr (OP == kOpBiasSoftmax) {
            // Softmax over the row: exponentials relative to a reference
            // value r taken from the row, computed as 2^((z - r) log2 e), so
            // that the rounding of the exponent scales with z - r (small for
            // the terms that matter) rather than with z.
            //   one wavefront or less per row: r = the row maximum M and
            //     y = e / sum(e);
            //   several wavefronts: each wavefront w uses its own maximum m_w
            //     and its own sum s_w, exchanged through LDS (one barrier);
            //     then M = max m_w, S = sum_w s_w 2^((m_w - M) log2 e) and
            //     y = e 2^((m_w - M) log2 e) / S.
            // Chunks past the row end take part as -inf / 0.  Special values
            // follow the definition: any NaN in the row, a +inf, or a row
            // that is -inf throughout makes the whole row NaN; a wavefront
            // whose elements are all -inf contributes zeros.
            constexpr float kLog2e = 1.4426950408889634f;
            constexpr float kNegInf = -__builtin_inff();
            float mx = kNegInf;
#pragma unroll
            for (int k = 0; k < CH; ++k)
                if (ok[k])
#pragma unroll
                    for (int e = 0; e < V; ++e) mx = __builtin_fmaxf(mx, s[k][e]);
            float m, r;
            if constexpr (WPR == 1) {
                m = group_reduce<MaxOp, G>(mx);
                r = m;
            } else {
                m = wave_max(mx);
                r = m != kNegInf ? m : 0.0f;
            }
            float part = 0.0f;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        s[k][e] = __builtin_amdgcn_exp2f((s[k][e] - r) * kLog2e);
                        part += s[k][e];
                    }
                }
            }
            float scale;
            if constexpr (WPR == 1) {
                scale = 1.0f / group_sum<G>(part);
            } else {
                const float ws = wave_sum(part);
                if ((lt & 63) == 0) partial[parity][slot][lt >> 6] = make_float4(m, ws, 0.0f, 0.0f);
                __syncthreads();
                float row_max = kNegInf;
#pragma unroll
                for (int w = 0; w < WPR; ++w) row_max = __builtin_fmaxf(row_max, partial[parity][slot][w].x);
                float total = 0.0f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    const float4 p = partial[parity][slot][w];
                    const float f = p.x == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((p.x - row_max) * kLog2e);
                    total += p.y * f;
                }
                const float own = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m - row_max) * kLog2e);
                scale = own / total;
                parity ^= 1;
            }
            if (live) {
                u32x4* op = O + row * hv + lt;
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    if (ok[k]) {
                        float y[V];
#pragma unroll
                        for (int e = 0; e < V; ++e) y[e] = s[k][e] * scale;
                        __builtin_nontemporal_store(E::narrow(y), op + k * G);
                    }
                }
            }
            continue;
        }

        if constexpr (OP == kOpBiasAdd) {
            // BiasAdd ends here: the sum is the output.
            if (live) {
                u32x4* op = O + row * hv + lt;
#pragma unroll
                for (int k = 0; k < CH; ++k)
                    if (ok[k]) __builtin_nontemporal_store(E::narrow(s[k]), op + k * G);
            }
            continue;
        }

        if (R != nullptr && live) {
            u32x4* rp = R + row * hv + lt;
#pragma unroll
            for (int k = 0; k < CH; ++k)
                if (ok[k]) __builtin_nontemporal_store(E::narrow(s[k]), rp + k * G);
        }

        // Statistics are taken relative to a value of the row itself (lane
        // 0's first element), subtracted from s in place once the residual is
        // out: the mean is kept as shift + dmean and the row normalized as
        // (s - shift) - dmean, so rounding scales with the row's spread, not
        // with its offset from zero (s - shift is exact when both are near the
        // row mean; a binary32 mean near 1000 could not be held to better than
        // 3e-5).  Lane 0 of a group always holds chunk 0; with several
        // wavefronts per row each uses its own lane 0.  This lane's partial
        // sum (of squares, for the simplified form) follows.
        const float shift = OP == kOpLayerNorm ? group_first<G>(s[0][0]) : 0.0f;
        float part = 0.0f;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (ok[k]) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    if constexpr (OP == kOpSimplified) {
                        part += s[k][e] * s[k][e];
                    } else {
                        s[k][e] = s[k][e] - shift;
                        part += s[k][e];
                    }
                }
            }
        }

        // off: what to subtract from the shifted s to center it on the row mean.
        float off = 0.0f, var;
        if constexpr (OP == kOpSimplified) {
            // Root mean square: no mean; the mean square takes the variance's place.
            if constexpr (WPR == 1) {
                var = group_sum<G>(part) * inv_h;
            } else {
                const float wsq = wave_sum(part);
                if ((lt & 63) == 0) partial[parity][slot][lt >> 6] = make_float4(wsq, 0.0f, 0.0f, 0.0f);
                __syncthreads();
                float tot = 0.0f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) tot += partial[parity][slot][w].x;
                var = tot * inv_h;
                parity ^= 1;
            }
        } else if constexpr (WPR == 1) {
            const float dmean = group_sum<G>(part) * inv_h;
            off = dmean;
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float d = s[k][e] - dmean;
                        q += d * d;
                    }
                }
            }
            var = group_sum<G>(q) * inv_h;
        } else {
            // Per wavefront: shift_w, the mean relative to it, and the squared
            // deviations from the wavefront mean; merged across wavefronts by
            // Chan et al.'s pairwise update (M2 = sum_w M2_w + n_w d_w^2)
            // relative to wavefront 0's shift (wavefront 0 always has
            // elements), so the merge only adds small numbers.
            const float wd = wave_sum(part) * inv_own_n;
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        const float d = s[k][e] - wd;
                        q += d * d;
                    }
                }
            }
            const float wm2 = wave_sum(q);
            if ((lt & 63) == 0) partial[parity][slot][lt >> 6] = make_float4(shift, wd, wm2, 0.0f);
            __syncthreads();
            const float row_shift = partial[parity][slot][0].x;
            float dsum = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                if (nw[w] > 0.0f) {
                    const float4 p = partial[parity][slot][w];
                    dsum += nw[w] * ((p.x - row_shift) + p.y);
                }
            }
            const float dmean = dsum * inv_h;
            float m2 = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                if (nw[w] > 0.0f) {
                    const float4 p = partial[parity][slot][w];
                    const float dm = ((p.x - row_shift) + p.y) - dmean;
                    m2 += p.z + nw[w] * dm * dm;
                }
            }
            var = m2 * inv_h;
            // s holds s - shift_w; the row is centered by subtracting
            // dmean - (shift_w - row_shift) (both small).
            off = dmean - (shift - row_shift);
            parity ^= 1;
        }
        const float rstd = rsqrtf(var + a.eps);

        if (live) {
            u32x4* op = O + row * hv + lt;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
                    float gf[V], bf[V], y[V];
                    E::widen(gam[k], gf);
                    E::widen(bet[k], bf);
#pragma unroll
                    for (int e = 0; e < V; ++e) y[e] = (s[k][e] - off) * rstd * gf[e] + bf[e];
                    __builtin_nontemporal_store(E::narrow(y), op + k * G);
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// Long-row kernel: the row is staged in LDS.
// ------------------------------------------------------------------------
// One 1024-lane block per row at a time (persistent over rows).  Lane t owns
// chunks t, t + 1024, ...; it loads them (kLdsBatch chunks in flight per
// lane), forms the binary32 sums, stores the residual, and parks its sums in
// LDS -- up to 160 KiB, i.e. rows of up to ~40K values whatever T is -- so x
// and skip cross HBM once.  Each lane re-reads only the LDS words it wrote,
// so the row data needs no barrier; only the block reductions do.
constexpr int kLdsBlock = 1024;
constexpr int kLdsBatch = 4;

template <typename T, int OP>
__global__ void __launch_bounds__(kLdsBlock) ldsrow_kernel(const Args a) {
    static_assert(OP == kOpLayerNorm || OP == kOpSimplified || OP == kOpBiasSoftmax, "row-reducing operations");
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr int Q = V / 4;  // float4 words of binary32 sums per chunk
    constexpr int W = kLdsBlock / 64;
    extern __shared__ float4 srow[];
    __shared__ float red[2][W];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int hv = a.hidden / V;
    const float h = static_cast<float>(a.hidden);
    const bool has_bias = OP != kOpBiasSoftmax && a.bias != nullptr;
    const bool has_beta = a.beta != nullptr;
    const bool bcast = a.skip_rows > 0 || a.skip_group > 0;
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const u32x4* __restrict__ X = static_cast<const u32x4*>(a.input);
    const u32x4* __restrict__ S = static_cast<const u32x4*>(a.skip);
    const u32x4* __restrict__ Bz = static_cast<const u32x4*>(a.bias);
    const u32x4* __restrict__ Gm = static_cast<const u32x4*>(a.gamma);
    const u32x4* __restrict__ Bt = static_cast<const u32x4*>(a.beta);
    u32x4* __restrict__ R = static_cast<u32x4*>(a.residual);
    u32x4* __restrict__ O = static_cast<u32x4*>(a.out);

    // Block reduction (SumOp or MaxOp); `buf` alternates so that a slot is
    // rewritten only after a barrier every lane passes after reading it.
    auto block_reduce = [&](float v, int buf, auto op) {
        using Op = decltype(op);
        const float ws = wave_reduce<Op>(v);
        if ((tid & 63) == 0) red[buf][wave] = ws;
        __syncthreads();
        float t = Op::id();
#pragma unroll
        for (int w = 0; w < W; ++w) t = Op::apply(t, red[buf][w]);
        return t;
    };
    auto block_sum = [&](float v, int buf) { return block_reduce(v, buf, SumOp{}); };

    int rms_buf = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t srow_i = skip_row_of(row, a, small_rows);
        const u32x4* xp = X + row * hv;
        const u32x4* sp = S + srow_i * hv;

        if constexpr (OP == kOpBiasSoftmax) {
            // Softmax over the row of z = data + bias (bias through the skip
            // slot): z parked in LDS while the block finds the maximum M, then
            // replaced by 2^((z - M) log2 e) while the block sums them, then
            // scaled by 1 / sum.  Special values as in the row-tile kernel
            // (one reference, the row maximum).
            constexpr float kLog2e = 1.4426950408889634f;
            float mx = -__builtin_inff();
            for (int c0 = tid; c0 < hv; c0 += kLdsBlock * kLdsBatch) {
                u32x4 xr[kLdsBatch], sr[kLdsBatch];
#pragma unroll
                for (int b = 0; b < kLdsBatch; ++b) {
                    const int c = c0 + b * kLdsBlock;
                    xr[b] = sr[b] = u32x4{0, 0, 0, 0};
                    if (c < hv) {
                        xr[b] = __builtin_nontemporal_load(xp + c);
                        sr[b] = bcast ? sp[c] : __builtin_nontemporal_load(sp + c);
                    }
                }
#pragma unroll
                for (int b = 0; b < kLdsBatch; ++b) {
                    const int c = c0 + b * kLdsBlock;
                    if (c < hv) {
                        float xf[V], sf[V], zv[V];
                        E::widen(xr[b], xf);
                        E::widen(sr[b], sf);
#pragma unroll
                        for (int e = 0; e < V; ++e) {
                            zv[e] = xf[e] + sf[e];
                            mx = __builtin_fmaxf(mx, zv[e]);
                        }
#pragma unroll
                        for (int q = 0; q < Q; ++q)
                            srow[c * Q + q] = make_float4(zv[4 * q], zv[4 * q + 1], zv[4 * q + 2], zv[4 * q + 3]);
                    }
                }
            }
            const float m = block_reduce(mx, 0, MaxOp{});
            float part = 0.0f;
            for (int c = tid; c < hv; c += kLdsBlock) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    float4 v = srow[c * Q + q];
                    v.x = __builtin_amdgcn_exp2f((v.x - m) * kLog2e);
                    v.y = __builtin_amdgcn_exp2f((v.y - m) * kLog2e);
                    v.z = __builtin_amdgcn_exp2f((v.z - m) * kLog2e);
                    v.w = __builtin_amdgcn_exp2f((v.w - m) * kLog2e);
                    part += v.x + v.y + v.z + v.w;
                    srow[c * Q + q] = v;
                }
            }
            const float scale = 1.0f / block_sum(part, 1);
            for (int c = tid; c < hv; c += kLdsBlock) {
                float y[V];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 v = srow[c * Q + q];
                    y[4 * q] = v.x * scale;
                    y[4 * q + 1] = v.y * scale;
                    y[4 * q + 2] = v.z * scale;
                    y[4 * q + 3] = v.w * scale;
                }
                __builtin_nontemporal_store(E::narrow(y), O + row * hv + c);
            }
            continue;
        }
        // Shift of the sums (see the row-tile kernel): the row's first sum,
        // formed by every lane with the same operations, hence the same bits.
        float shift = 0.0f;
        if constexpr (OP == kOpLayerNorm) {
            shift = E::load1(a.input, row * a.hidden) + E::load1(a.skip, srow_i * a.hidden);
            if (has_bias) shift = shift + E::load1(a.bias, 0);
        }

        float part = 0.0f;
        for (int c0 = tid; c0 < hv; c0 += kLdsBlock * kLdsBatch) {
            u32x4 xr[kLdsBatch], sr[kLdsBatch], br[kLdsBatch];
#pragma unroll
            for (int b = 0; b < kLdsBatch; ++b) {
                const int c = c0 + b * kLdsBlock;
                xr[b] = sr[b] = br[b] = u32x4{0, 0, 0, 0};
                if (c < hv) {
                    xr[b] = __builtin_nontemporal_load(xp + c);
                    sr[b] = bcast ? sp[c] : __builtin_nontemporal_load(sp + c);
                    if (has_bias) br[b] = Bz[c];
                }
            }
#pragma unroll
            for (int b = 0; b < kLdsBatch; ++b) {
                const int c = c0 + b * kLdsBlock;
                if (c < hv) {
                    float xf[V], sf[V], bf[V], sv[V];
                    E::widen(xr[b], xf);
                    E::widen(sr[b], sf);
                    E::widen(br[b], bf);
#pragma unroll
                    for (int e = 0; e < V; ++e) {
                        float v = xf[e] + sf[e];
                        if (has_bias) v = v + bf[e];
                        sv[e] = v;
                        if constexpr (OP == kOpSimplified)
                            part += v * v;
                        else
                            part += v - shift;
                    }
                    if (R != nullptr) __builtin_nontemporal_store(E::narrow(sv), R + row * hv + c);
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        srow[c * Q + q] = make_float4(sv[4 * q], sv[4 * q + 1], sv[4 * q + 2], sv[4 * q + 3]);
                }
            }
        }

        // The mean is kept as shift + dmean (see the row-tile kernel).
        float dmean = 0.0f, var;
        if constexpr (OP == kOpSimplified) {
            var = block_sum(part, rms_buf) / h;
            rms_buf ^= 1;
        } else {
            dmean = block_sum(part, 0) / h;
            float q2 = 0.0f;
            for (int c = tid; c < hv; c += kLdsBlock) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 v = srow[c * Q + q];
                    const float d0 = (v.x - shift) - dmean, d1 = (v.y - shift) - dmean;
                    const float d2 = (v.z - shift) - dmean, d3 = (v.w - shift) - dmean;
                    q2 += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
                }
            }
            var = block_sum(q2, 1) / h;
        }
        const float rstd = rsqrtf(var + a.eps);

        for (int c = tid; c < hv; c += kLdsBlock) {
            float gf[V], bf[V], y[V];
            E::widen(Gm[c], gf);
            if (has_beta) {
                E::widen(Bt[c], bf);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) bf[e] = 0.0f;
            }
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float4 v = srow[c * Q + q];
                y[4 * q] = ((v.x - shift) - dmean) * rstd * gf[4 * q] + bf[4 * q];
                y[4 * q + 1] = ((v.y - shift) - dmean) * rstd * gf[4 * q + 1] + bf[4 * q + 1];
                y[4 * q + 2] = ((v.z - shift) - dmean) * rstd * gf[4 * q + 2] + bf[4 * q + 2];
                y[4 * q + 3] = ((v.w - shift) - dmean) * rstd * gf[4 * q + 3] + bf[4 * q + 3];
            }
            __builtin_nontemporal_store(E::narrow(y), O + row * hv + c);
        }
    }
}

// ------------------------------------------------------------------------
// Generic kernel: any hidden size and alignment.
// ------------------------------------------------------------------------
constexpr int kGenericBlock = 256;

template <typename T, int OP>
__global__ void __launch_bounds__(kGenericBlock) generic_kernel(const Args a) {
    using E = Elem<T>;
    constexpr int W = kGenericBlock / 64;
    __shared__ float red[2][W];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int64_t H = a.hidden;
    const float h = static_cast<float>(a.hidden);
    int rms_slot = 0;

    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    // Block reduction (SumOp or MaxOp) through LDS slot `buf`.
    auto block_reduce = [&](float v, int buf, auto op) {
        using Op = decltype(op);
        const float ws = wave_reduce<Op>(v);
        if ((tid & 63) == 0) red[buf][wave] = ws;
        __syncthreads();
        float t = Op::id();
#pragma unroll
        for (int w = 0; w < W; ++w) t = Op::apply(t, red[buf][w]);
        return t;
    };

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const int64_t srow = skip_row_of(row, a, small_rows);
        const int64_t xo = row * H, so = srow * H;
        // The same binary32 operations in every pass, hence the same bits.
        auto sum_at = [&](int64_t c) {
            float v;
            if constexpr (OP == kOpBiasAdd) {
                v = E::load1(a.input, xo + c) + E::load1(a.bias, c);
                v = v + E::load1(a.skip, so + c);
            } else {
                v = E::load1(a.input, xo + c) + E::load1(a.skip, so + c);
                if (OP != kOpBiasSoftmax && a.bias != nullptr) v = v + E::load1(a.bias, c);
            }
            return v;
        };

        if constexpr (OP == kOpBiasAdd) {
            for (int64_t c = tid; c < H; c += kGenericBlock) E::store1(a.out, xo + c, sum_at(c));
            continue;
        }
        if constexpr (OP == kOpBiasSoftmax) {
            // Softmax over the row of z = data + bias (bias through the skip
            // slot): the maximum M, then the sum of 2^((z - M) log2 e), then
            // the scaled exponentials, recomputed from the same bits in each
            // pass.  Slot 0 holds the maximum, slot 1 the sum: a slot is
            // rewritten only after the other slot's barrier, which every lane
            // passes after reading it.
            constexpr float kLog2e = 1.4426950408889634f;
            float mx = -__builtin_inff();
            for (int64_t c = tid; c < H; c += kGenericBlock) mx = __builtin_fmaxf(mx, sum_at(c));
            const float m = block_reduce(mx, 0, MaxOp{});
            float part = 0.0f;
            for (int64_t c = tid; c < H; c += kGenericBlock) part += __builtin_amdgcn_exp2f((sum_at(c) - m) * kLog2e);
            const float scale = 1.0f / block_reduce(part, 1, SumOp{});
            for (int64_t c = tid; c < H; c += kGenericBlock)
                E::store1(a.out, xo + c, __builtin_amdgcn_exp2f((sum_at(c) - m) * kLog2e) * scale);
            continue;
        }
        if constexpr (OP == kOpSimplified) {
            float sq = 0.0f;
            for (int64_t c = tid; c < H; c += kGenericBlock) {
                const float v = sum_at(c);
                sq += v * v;
            }
            // One barrier per row: consecutive rows use alternate LDS slots,
            // and a slot is rewritten two rows later, after a barrier that
            // every lane reaches only once it has read the slot.
            const float wsq = wave_sum(sq);
            if ((tid & 63) == 0) red[rms_slot][wave] = wsq;
            __syncthreads();
            float tot = 0.0f;
#pragma unroll
            for (int w = 0; w < W; ++w) tot += red[rms_slot][w];
            rms_slot ^= 1;
            const float rstd = rsqrtf(tot / h + a.eps);
            for (int64_t c = tid; c < H; c += kGenericBlock) {
                const float v = sum_at(c);
                if (a.residual != nullptr) E::store1(a.residual, xo + c, v);
                const float g = E::load1(a.gamma, c);
                const float b = a.beta != nullptr ? E::load1(a.beta, c) : 0.0f;
                E::store1(a.out, xo + c, v * rstd * g + b);
            }
            continue;
        }

        // Sums relative to the row's first sum (see the row-tile kernel).
        const float shift = sum_at(0);
        float part = 0.0f;
        for (int64_t c = tid; c < H; c += kGenericBlock) part += sum_at(c) - shift;
        float ws = wave_sum(part);
        if ((tid & 63) == 0) red[0][wave] = ws;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) tot += red[0][w];
        const float dmean = tot / h;  // the mean is shift + dmean (see the row-tile kernel)

        float q = 0.0f;
        for (int64_t c = tid; c < H; c += kGenericBlock) {
            const float d = (sum_at(c) - shift) - dmean;
            q += d * d;
        }
        ws = wave_sum(q);
        if ((tid & 63) == 0) red[1][wave] = ws;
        __syncthreads();
        tot = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) tot += red[1][w];
        const float rstd = rsqrtf(tot / h + a.eps);

        // Each element is read and then written by the same lane, so exact
        // aliasing of an output with input or skip is safe.
        for (int64_t c = tid; c < H; c += kGenericBlock) {
            const float v = sum_at(c);
            if (a.residual != nullptr) E::store1(a.residual, xo + c, v);
            const float g = E::load1(a.gamma, c);
            const float b = a.beta != nullptr ? E::load1(a.beta, c) : 0.0f;
            E::store1(a.out, xo + c, ((v - shift) - dmean) * rstd * g + b);
        }
    }
}

// ------------------------------------------------------------------------
// Streaming copy (bandwidth reference): 16-byte chunks, persistent grid.
// ------------------------------------------------------------------------
constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(kCopyBlock) copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                          int64_t chunks) {
    const int64_t step = static_cast<int64_t>(gridDim.x) * kCopyBlock;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyBlock + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * step < chunks; i += kCopyUnroll * step) {
        u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * step);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * step);
    }
    for (; i < chunks; i += step) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// ------------------------------------------------------------------------
// Host side: geometry table, occupancy-sized persistent grids.
// ------------------------------------------------------------------------
struct Geom {
    int g, ch, block;
};

// Auto order (increasing capacity G*CH chunks) first, then geometries only
// reachable through the multi-wavefront variant.
constexpr Geom kGeoms[] = {
    {16, 1, 256},  {32, 1, 256},  {64, 1, 256},   {64, 2, 256},   {64, 3, 256},
    {64, 4, 256},  {128, 4, 256}, {256, 3, 256},  {256, 4, 256},  {512, 3, 512},
    {512, 4, 512}, {1024, 3, 1024}, {1024, 4, 1024}, {128, 1, 256}, {256, 1, 256},
    {512, 2, 512}, {128, 8, 256},  {256, 2, 512},  {256, 4, 512},  {64, 2, 64},
    {64, 3, 64},   {32, 6, 256},  {192, 1, 192},  {192, 2, 192},  {512, 1, 512},
    {1024, 1, 1024}, {1024, 2, 1024}, {256, 2, 256}, {4, 1, 256},   {8, 1, 256},
    {4, 2, 256},   {8, 2, 256},   {8, 4, 256},    {16, 2, 256},   {16, 4, 256},
    {32, 2, 256},  {128, 2, 256}, {32, 4, 256},   {16, 8, 256},
};
constexpr int kNumGeoms = sizeof(kGeoms) / sizeof(kGeoms[0]);
static_assert(kRowtileFirst + kNumGeoms <= kSplitRowIndex, "kernel index ranges are disjoint");

// Automatic choice: the first entry whose capacity holds the row's chunks.
// Short rows are latency bound: one chunk per lane spreads a row over more
// lanes and shortens the per-lane load/reduce chain; rows of 8 chunks or
// fewer (e.g. attention rows of a few keys) pack 32 or 64 rows into a
// 256-lane block instead of leaving most of a 16-lane group idle.  Long rows use 256-lane
// groups (4 wavefronts; 1024-lane groups pay for 16-wavefront barriers).
// A broadcast skip uses the same geometries with skip-stationary tiling.
struct AutoEntry {
    int max_chunks, geom;
};
constexpr AutoEntry kAutoExact[] = {
    {4, 28}, {8, 29}, {16, 0}, {32, 1}, {64, 2}, {128, 13}, {192, 22}, {256, 14}, {512, 27},
    {768, 7}, {1024, 8}, {1536, 9}, {2048, 10}, {3072, 11}, {4096, 12},
};
constexpr AutoEntry kAutoBroadcast[] = {
    {4, 28}, {8, 29}, {16, 0}, {32, 1}, {64, 2}, {128, 13}, {192, 22}, {256, 14}, {512, 27},
    {768, 7}, {1024, 8}, {1536, 9}, {2048, 10}, {3072, 11}, {4096, 12},
};
// BiasSoftmax streams one tensor in and one out and has no per-column
// parameters; on MI355X it runs fastest with two to four chunks per lane
// (more independent loads in flight per lane, fewer lanes per reduction)
// until a row needs several wavefronts (measured over 2..2048 chunks).
constexpr AutoEntry kAutoSoftmax[] = {
    {4, 28},   {8, 29},   {16, 31},  {32, 33},   {64, 35},   {128, 37},  {256, 5},
    {512, 6},  {1024, 15}, {2048, 10}, {3072, 11}, {4096, 12},
};

hipError_t cu_count(int* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::atomic<int> cache[64];
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

// Blocks of `kernel` the device holds at once (occupancy limit x CUs); the
// per-kernel occupancy is cached after the first query.
template <typename K>
hipError_t resident_blocks(K kernel, int block, int* occupancy_cache, int64_t* out) {
    int cus = 0;
    hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    int occ = __atomic_load_n(occupancy_cache, __ATOMIC_RELAXED);
    if (occ <= 0) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, 0);
        if (e != hipSuccess) return e;
        if (occ < 1) occ = 1;
        __atomic_store_n(occupancy_cache, occ, __ATOMIC_RELAXED);
    }
    *out = static_cast<int64_t>(cus) * occ;
    return hipSuccess;
}

template <typename K>
hipError_t launch_grid(K kernel, int block, int64_t blocks, const Args& a, hipStream_t st) {
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks)),
                           dim3(block), params, 0, st);
}

constexpr int64_t kMaxGrid = 0x7FFFFFFF;

template <typename T, int OP, int I>
hipError_t launch_geom(const Args& a0, Tiling tiling, hipStream_t st) {
    constexpr Geom g = kGeoms[I];
    static int occ = 0;
    auto kernel = rowtile_kernel<T, OP, g.g, g.ch, g.block>;
    const int64_t rpb = g.block / g.g;
    const int64_t tiles = (a0.rows + rpb - 1) / rpb;
    Args a = a0;
    int mode = tiling.mode;
    int64_t per = tiling.tiles_per_block;
    // Skip-stationary needs a broadcast skip whose rows split into whole tiles.
    if (mode == kTileSkipStationary && (a.skip_rows <= 0 || a.skip_rows % rpb != 0 || a.skip_rows / rpb > kMaxGrid))
        mode = kTileStrided;
    int64_t resident = 0;
    if (per <= 0) {
        const hipError_t e = resident_blocks(kernel, g.block, &occ, &resident);
        if (e != hipSuccess) return e;
    }
    int64_t blocks = 1;
    if (mode == kTileSkipStationary) {
        const int64_t P = a.skip_rows / rpb;
        const int64_t batches = a.rows / a.skip_rows;
        if (per <= 0) {
            // Enough batch chunks per tile column to fill the resident grid.
            const int64_t chunks = resident > P ? resident / P : 1;
            per = (batches + chunks - 1) / chunks;
        }
        if (P * ((batches + per - 1) / per) > kMaxGrid) per = (batches * P + kMaxGrid - 1) / kMaxGrid;
        blocks = P * ((batches + per - 1) / per);
    } else {
        if (per <= 0) {
            // Persistent: one wave of resident blocks walks all tiles, strided.
            per = (tiles + resident - 1) / resident;
            mode = kTileStrided;
        }
        if ((tiles + per - 1) / per > kMaxGrid) per = (tiles + kMaxGrid - 1) / kMaxGrid;
        blocks = (tiles + per - 1) / per;
    }
    a.tiles_per_block = per;
    a.tiling = mode;
    return launch_grid(kernel, g.block, blocks < 1 ? 1 : blocks, a, st);
}

template <typename T, int OP, int... I>
hipError_t launch_geom_dispatch(int idx, const Args& a, Tiling t, hipStream_t st, std::integer_sequence<int, I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((idx == I ? (r = launch_geom<T, OP, I>(a, t, st), 0) : 0), ...);
    return r;
}

template <typename T, int OP>
hipError_t launch_generic_t(const Args& a, hipStream_t st) {
    static int occ = 0;
    int64_t resident = 0;
    const hipError_t e = resident_blocks(generic_kernel<T, OP>, kGenericBlock, &occ, &resident);
    if (e != hipSuccess) return e;
    const int64_t blocks = a.rows < resident ? a.rows : resident;
    return launch_grid(generic_kernel<T, OP>, kGenericBlock, blocks < 1 ? 1 : blocks, a, st);
}

// Kernel names: "<op>generic_<t>" and "<op>rowtile_<t>_g<G>_c<CH>", with
// "_b<block>" when the block is not the default max(256, G); <op> is empty
// for layer normalization, "rms_" for the simplified form, "biasadd_",
// "softmax_".
struct NameTable {
    char name[kNumOps][2][kIdsPerType][48];
    NameTable() {
        const char* op_prefix[kNumOps] = {"", "rms_", "biasadd_", "softmax_"};
        const char* tn[2] = {"f32", "f16"};
        for (int op = 0; op < kNumOps; ++op) {
            for (int t = 0; t < 2; ++t) {
                for (int i = 0; i < kIdsPerType; ++i) {
                    char* dst = name[op][t][i];
                    const int gi = i - kRowtileFirst;
                    if (i == kGenericIndex) {
                        snprintf(dst, 48, "%sgeneric_%s", op_prefix[op], tn[t]);
                    } else if (i == kLdsRowIndex) {
                        snprintf(dst, 48, "%sldsrow_%s", op_prefix[op], tn[t]);
                    } else if (i == kSplitRowIndex) {
                        snprintf(dst, 48, "%ssplitrow_%s", op_prefix[op], tn[t]);
                    } else if (gi >= 0 && gi < kNumGeoms) {
                        const Geom& g = kGeoms[gi];
                        const int default_block = g.g > 256 ? g.g : 256;
                        if (g.block == default_block)
                            snprintf(dst, 48, "%srowtile_%s_g%d_c%d", op_prefix[op], tn[t], g.g, g.ch);
                        else
                            snprintf(dst, 48, "%srowtile_%s_g%d_c%d_b%d", op_prefix[op], tn[t], g.g, g.ch, g.block);
                    } else {
                        snprintf(dst, 48, "unknown");
                    }
                }
            }
        }
    }
};

}  // namespace

int rowtile_count() { return kNumGeoms; }

int rowtile_pick(int op, int64_t hidden, int dtype, bool broadcast, bool multiwave_only) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    if (hidden <= 0 || hidden % v != 0) return -1;
    const int64_t hv = hidden / v;
    if (!multiwave_only) {
        if (op == kOpBiasSoftmax) {
            for (const AutoEntry& e : kAutoSoftmax)
                if (hv <= e.max_chunks) return e.geom;
            return -1;
        }
        for (const AutoEntry& e : (broadcast ? kAutoBroadcast : kAutoExact))
            if (hv <= e.max_chunks) return e.geom;
        return -1;
    }
    int best = -1;  // smallest capacity among groups of two or more wavefronts
    for (int i = 0; i < kNumGeoms; ++i) {
        if (kGeoms[i].g < 128) continue;
        const int64_t cap = static_cast<int64_t>(kGeoms[i].g) * kGeoms[i].ch;
        if (cap < hv) continue;
        if (best < 0 || cap < static_cast<int64_t>(kGeoms[best].g) * kGeoms[best].ch) best = i;
    }
    return best;
}

bool rowtile_holds(int geometry, int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    if (geometry < 0 || geometry >= kNumGeoms || hidden <= 0 || hidden % v != 0) return false;
    return hidden / v <= static_cast<int64_t>(kGeoms[geometry].g) * kGeoms[geometry].ch;
}

const char* kernel_name(int kernel_id) {
    static const NameTable table;  // built once, thread-safe initialization
    if (kernel_id < 0 || kernel_id >= kNumOps * 2 * kIdsPerType) return "unknown";
    const int op = kernel_id / (2 * kIdsPerType), t = kernel_id / kIdsPerType % 2;
    return table.name[op][t][kernel_id % kIdsPerType];
}

hipError_t launch_copy(void* dst, const void* src, int64_t chunks, hipStream_t st) {
    static int occ = 0;
    int64_t blocks = 0;
    const hipError_t e = resident_blocks(copy_kernel, kCopyBlock, &occ, &blocks);
    if (e != hipSuccess) return e;
    const int64_t need = (chunks + kCopyBlock - 1) / kCopyBlock;
    if (need < blocks) blocks = need;
    if (blocks < 1) blocks = 1;
    u32x4* d = static_cast<u32x4*>(dst);
    const u32x4* s = static_cast<const u32x4*>(src);
    void* params[] = {&d, &s, &chunks};
    return hipLaunchKernel(reinterpret_cast<const void*>(copy_kernel), dim3(static_cast<unsigned>(blocks)),
                           dim3(kCopyBlock), params, 0, st);
}

template <typename T, int OP>
hipError_t launch_ldsrow_t(const Args& a, hipStream_t st) {
    auto kernel = ldsrow_kernel<T, OP>;
    const size_t lds = static_cast<size_t>(a.hidden) * sizeof(float);
    int cus = 0;
    hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    int occ = 0;  // depends on the row's LDS footprint, so it is not cached
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kLdsBlock, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) return hipErrorInvalidConfiguration;
    int64_t blocks = static_cast<int64_t>(cus) * occ;
    if (a.rows < blocks) blocks = a.rows;
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)),
                           dim3(kLdsBlock), params, lds, st);
}

template <typename T>
hipError_t launch_generic_op(const Args& a, int op, hipStream_t st) {
    switch (op) {
        case kOpLayerNorm: return launch_generic_t<T, kOpLayerNorm>(a, st);
        case kOpSimplified: return launch_generic_t<T, kOpSimplified>(a, st);
        case kOpBiasAdd: return launch_generic_t<T, kOpBiasAdd>(a, st);
        case kOpBiasSoftmax: return launch_generic_t<T, kOpBiasSoftmax>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ldsrow(const Args& a, int op, int dtype, hipStream_t st) {
    if (op == kOpLayerNorm)
        return dtype == 0 ? launch_ldsrow_t<float, kOpLayerNorm>(a, st) : launch_ldsrow_t<_Float16, kOpLayerNorm>(a, st);
    if (op == kOpSimplified)
        return dtype == 0 ? launch_ldsrow_t<float, kOpSimplified>(a, st)
                          : launch_ldsrow_t<_Float16, kOpSimplified>(a, st);
    if (op == kOpBiasSoftmax)
        return dtype == 0 ? launch_ldsrow_t<float, kOpBiasSoftmax>(a, st)
                          : launch_ldsrow_t<_Float16, kOpBiasSoftmax>(a, st);
    return hipErrorInvalidValue;
}

bool ldsrow_holds(int op, int64_t hidden, int dtype) {
    const int v = dtype == 0 ? Elem<float>::kPerChunk : Elem<_Float16>::kPerChunk;
    return (op == kOpLayerNorm || op == kOpSimplified || op == kOpBiasSoftmax) && hidden > 0 && hidden % v == 0 &&
           hidden * static_cast<int64_t>(sizeof(float)) <= kLdsRowBytes;
}

hipError_t launch_generic(const Args& a, int op, int dtype, hipStream_t st) {
    return dtype == 0 ? launch_generic_op<float>(a, op, st) : launch_generic_op<_Float16>(a, op, st);
}

template <typename T>
hipError_t launch_rowtile_op(const Args& a, int op, int geometry, Tiling tiling, hipStream_t st) {
    auto seq = std::make_integer_sequence<int, kNumGeoms>{};
    switch (op) {
        case kOpLayerNorm: return launch_geom_dispatch<T, kOpLayerNorm>(geometry, a, tiling, st, seq);
        case kOpSimplified: return launch_geom_dispatch<T, kOpSimplified>(geometry, a, tiling, st, seq);
        case kOpBiasAdd: return launch_geom_dispatch<T, kOpBiasAdd>(geometry, a, tiling, st, seq);
        case kOpBiasSoftmax: return launch_geom_dispatch<T, kOpBiasSoftmax>(geometry, a, tiling, st, seq);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rowtile(const Args& a, int op, int dtype, int geometry, Tiling tiling, hipStream_t st) {
    if (geometry < 0 || geometry >= kNumGeoms) return hipErrorInvalidValue;
    return dtype == 0 ? launch_rowtile_op<float>(a, op, geometry, tiling, st)
                      : launch_rowtile_op<_Float16>(a, op, geometry, tiling, st);
}

}  // namespace skipln
