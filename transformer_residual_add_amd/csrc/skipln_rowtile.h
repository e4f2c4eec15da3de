// Row-tile kernels of 16-byte chunks or single elements, their geometry
// tables and their launch templates; shared by the sources that instantiate
// them (one translation unit per operation, compiled in parallel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>
#include <utility>

#include "skipln_device.h"
#include "skipln_internal.h"

namespace skipln {
namespace rowtile {
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

// Static LDS of a row-tile kernel: the cross-wavefront partials, double
// buffered.
template <int G, int BLOCK>
constexpr int partial_bytes() {
    return 2 * (BLOCK / G) * (G > 64 ? G / 64 : 1) * 16;
}

// FORM (kForm* in skipln_internal.h): kFormWalk blocks walk the tiles the
// launch gives them, each tile's loads issued while the previous tile
// finishes, gamma/beta/bias held in registers throughout; kFormOneTile
// blocks take exactly tile blockIdx.x (the launcher's guarantee) and load
// gamma and beta only once the sum is formed, so far fewer registers are
// live; kFormStreamSkip is kFormOneTile with the exact skip read by
// non-temporal loads (the launcher's choice for one wave of resident blocks).
// Otherwise the skip goes through the caches.
template <typename E, int OP, int G, int CH, int BLOCK, int FORM>
__global__ void __launch_bounds__(BLOCK) rowtile_kernel(const Args a) {
    static_assert(OP == kOpLayerNorm || OP == kOpSimplified || OP == kOpBiasAdd || OP == kOpBiasSoftmax,
                  "operation");
    using Raw = typename E::Raw;
    constexpr int V = E::kPerChunk;
    constexpr bool kNorm = OP == kOpLayerNorm || OP == kOpSimplified;  // gamma/beta
    constexpr bool kParams = OP != kOpBiasSoftmax;                       // any per-column parameter
    constexpr int RPB = BLOCK / G;                  // rows per block per tile
    constexpr int WPR = G > 64 ? G / 64 : 1;        // wavefronts per row
    static_assert(BLOCK % G == 0 && BLOCK % 64 == 0, "block of whole groups and wavefronts");
    static_assert(FORM >= kFormWalk && FORM <= kFormStreamSkip, "kernel form");
    constexpr bool SS = FORM == kFormStreamSkip;
    constexpr bool ONE = FORM != kFormWalk;
    // One tile per block: gamma and beta are loaded after the sum is formed
    // (their registers are not held through the loads of x and skip).
    constexpr bool LP = kNorm && ONE;
    __shared__ float4 partial[2][RPB][WPR];
    static_assert(sizeof(partial) == partial_bytes<G, BLOCK>(), "static LDS of the kernel");

    const int tid = threadIdx.x;
    // Row of the tile handled by this group; wave-uniform when G >= 64, and
    // said so, so that row addresses live in scalar registers.
    const int slot = G >= 64 ? __builtin_amdgcn_readfirstlane(tid / G) : tid / G;
    const int lt = tid - slot * G; // lane within the group
    const int hv = a.hidden / V;   // chunks per row
    const float h = static_cast<float>(a.hidden);

    const Raw* __restrict__ X = static_cast<const Raw*>(a.input);
    const Raw* __restrict__ S = static_cast<const Raw*>(a.skip);
    Raw* __restrict__ R = static_cast<Raw*>(a.residual);
    Raw* __restrict__ O = static_cast<Raw*>(a.out);
    const bool has_bias = kParams && a.bias != nullptr;
    const bool has_beta = a.beta != nullptr;
    const bool bcast = a.skip_rows > 0 || a.skip_group > 0;
    const bool small_rows = a.rows <= 0xFFFFFFFFll;
    const bool through = a.store_through != 0;

    bool ok[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) ok[k] = k * G + lt < hv;

    // Parameters: loaded once per block, kept in registers (raw T bits).
    Raw gam[CH], bet[CH], bia[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        gam[k] = E::zero();
        bet[k] = E::zero();
        bia[k] = E::zero();
    }
    auto load_params = [&]() {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int c = k * G + lt;
            if (ok[k]) {
                if constexpr (kNorm && !LP) {
                    gam[k] = static_cast<const Raw*>(a.gamma)[c];
                    if (has_beta) bet[k] = static_cast<const Raw*>(a.beta)[c];
                }
                if (has_bias) bia[k] = static_cast<const Raw*>(a.bias)[c];
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
    // (The single-tile forms are never launched skip-stationary: left out, so
    // that the streamed first loads cannot be merged with cached ones.)
    const bool stationary = !ONE && a.tiling == kTileSkipStationary;
    if constexpr (ONE) {
        // One tile per block (the launcher's guarantee for these forms).
        t_first = blockIdx.x;
        stride = 1;
        t_end = t_first + 1;
    } else if (a.tiling == kTileContiguous) {
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

    Raw xr[CH], sr[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
        xr[k] = E::zero();
        sr[k] = E::zero();
    }
    // `stream`: std::true_type for a block's first tile in an SS kernel.
    auto issue_loads = [&](int64_t tile, bool with_skip, auto stream) {
        const int64_t row = tile * RPB + slot;
        if (row < a.rows) {
            const int64_t srow = skip_row_of(row, a, small_rows);
            const Raw* xp = X + row * hv + lt;
            const Raw* sp = S + srow * hv + lt;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
                    xr[k] = __builtin_nontemporal_load(xp + k * G);
                    // The broadcast skip is re-read by every batch: keep it
                    // cached.  (The compiler merges the two loads of one
                    // address below into one and drops the non-temporal hint,
                    // so an exact skip is a cached load too; the streaming
                    // form is a separate instantiation of this body.)
                    if (with_skip) {
                        if constexpr (decltype(stream)::value)
                            sr[k] = __builtin_nontemporal_load(sp + k * G);
                        else
                            sr[k] = bcast ? sp[k * G] : __builtin_nontemporal_load(sp + k * G);
                    }
                }
            }
        }
    };

    // Order of the first loads (measured): a block that handles one tile
    // needs bias as soon as x and skip arrive, so parameters go first; a
    // long-lived skip-stationary block gets its first tile moving first.
    int64_t tile = t_first;
    if (stationary) {
        if (tile < t_end) issue_loads(tile, true, std::false_type{});
        load_params();
    } else {
        load_params();
        if (tile < t_end) issue_loads(tile, true, std::integral_constant<bool, SS>{});
    }

    int parity = 0;

    for (; tile < t_end; tile += stride) {
        const int64_t row = tile * RPB + slot;
        const bool live = row < a.rows;
        // Outputs go through buffer resources over this tile's rows (base
        // and size uniform, in scalar registers): a lane's element offset in
        // the tile in one register, chunk k's offset k * G as a scalar.
        const int64_t row0 = tile * RPB;
        const int tile_bytes =
            static_cast<int>((a.rows - row0 < RPB ? a.rows - row0 : RPB) * hv * static_cast<int>(sizeof(Raw)));
        const int voff = (slot * hv + lt) * static_cast<int>(sizeof(Raw));
        auto put = [&](Raw* base, int k, const Raw& v) {
            E::store(v, buffer_rsrc(base + row0 * hv, tile_bytes), voff, k * G * static_cast<int>(sizeof(Raw)),
                     through);
        };
        if constexpr (V == 8 && kParams) {
            // Keep gamma/beta/bias packed (2 fp16 per VGPR): without this the
            // compiler hoists their widening out of the loop and triples
            // their register footprint, which costs occupancy.
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if constexpr (LP)
                    asm volatile("" : "+v"(bia[k]));
                else
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
        if constexpr (!ONE)
            if (tile + stride < t_end) issue_loads(tile + stride, !stationary, std::false_type{});

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
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    if (ok[k]) {
                        float y[V];
#pragma unroll
                        for (int e = 0; e < V; ++e) y[e] = s[k][e] * scale;
                        put(O, k, E::narrow(y));
                    }
                }
            }
            continue;
        }

        if constexpr (OP == kOpBiasAdd) {
            // BiasAdd ends here: the sum is the output.
            if (live) {
#pragma unroll
                for (int k = 0; k < CH; ++k)
                    if (ok[k]) put(O, k, E::narrow(s[k]));
            }
            continue;
        }

        if (R != nullptr && live) {
#pragma unroll
            for (int k = 0; k < CH; ++k)
                if (ok[k]) put(R, k, E::narrow(s[k]));
        }
        if constexpr (LP) {
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                const int c = k * G + lt;
                if (ok[k]) {
                    gam[k] = static_cast<const Raw*>(a.gamma)[c];
                    if (has_beta) bet[k] = static_cast<const Raw*>(a.beta)[c];
                }
            }
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
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (ok[k]) {
                    float t[V], y[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) t[e] = (s[k][e] - off) * rstd;
                    E::widen_fma(t, gam[k], bet[k], y);
                    put(O, k, E::narrow(y));
                }
            }
        }
    }
}

// ------------------------------------------------------------------------
// Host side: geometry table, occupancy-sized persistent grids.
// ------------------------------------------------------------------------
struct Geom {
    int g, ch, block;
};

// Every geometry is the automatic choice of some row length, operation or
// skip form (the tables in skipln_kernels.hip), measured fastest there on
// MI355X in sweeps over a wider set: 16-1024-lane groups, 1-8 chunks per
// lane, 64-1024-lane blocks.  The forced-variant and tuning entry points
// reach the same kernels.
constexpr Geom kGeoms[] = {
    {16, 1, 256}, {32, 1, 256}, {64, 1, 256}, {64, 2, 256}, {64, 4, 256}, {128, 4, 256}, {256, 3, 256},
    {256, 4, 256}, {512, 3, 512}, {512, 4, 512}, {1024, 3, 1024}, {1024, 4, 1024}, {128, 1, 256},
    {256, 1, 256}, {512, 2, 512}, {192, 1, 192}, {256, 2, 256}, {4, 1, 256}, {8, 1, 256}, {8, 2, 256},
    {16, 2, 256}, {32, 2, 256}, {32, 4, 256},
};
constexpr int kNumGeoms = sizeof(kGeoms) / sizeof(kGeoms[0]);
static_assert(kRowtileFirst + kNumGeoms <= kElemFirst, "kernel index ranges are disjoint");

// Element-wise row tiles (one element per access): rows that are not whole
// 16-byte chunks, or tensors aligned to their element size only.  Four to
// sixteen elements per lane keep several loads in flight per lane; each is
// the automatic choice for some row length.
constexpr Geom kElemGeoms[] = {
    {4, 1, 256}, {4, 2, 256}, {8, 2, 256}, {8, 4, 256}, {16, 4, 256}, {32, 4, 256}, {64, 4, 256},
    {128, 4, 256}, {128, 8, 256}, {256, 8, 256}, {512, 8, 512}, {1024, 8, 1024}, {1024, 16, 1024},
};
constexpr int kNumElemGeoms = sizeof(kElemGeoms) / sizeof(kElemGeoms[0]);
static_assert(kElemFirst + kNumElemGeoms <= kRegRowIndex, "kernel index ranges are disjoint");

inline hipError_t cu_count(int* out) {
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
hipError_t launch_grid(K kernel, int block, int64_t blocks, const Args& a, hipStream_t st, size_t lds = 0) {
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(blocks)),
                           dim3(block), params, lds, st);
}

// LDS of a compute unit (160 KiB on gfx950), cached per device.
inline hipError_t lds_per_cu(int* out) {
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
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

// Largest number of blocks per compute unit a launch can be held to.
constexpr int kMaxBlocksCap = 16;

// Dynamic LDS that holds a compute unit to at most `cap` resident blocks of
// `kernel` (0: no limit): the least LDS for which the runtime's occupancy
// calculation (which knows the LDS allocation granule) gives `cap` or fewer,
// found by bisection once per kernel and cap (`cache`: kMaxBlocksCap + 1
// entries, LDS + 1, 0 = not computed) and assumed alike on every device.
template <typename K>
hipError_t cap_lds(K kernel, int block, int cap, int static_bytes, std::atomic<int>* cache, size_t* out) {
    *out = 0;
    if (cap <= 0) return hipSuccess;
    if (cap > kMaxBlocksCap) cap = kMaxBlocksCap;
    const int known = cache[cap].load(std::memory_order_relaxed);
    if (known > 0) {
        *out = static_cast<size_t>(known - 1);
        return hipSuccess;
    }
    int lds = 0;
    hipError_t e = lds_per_cu(&lds);
    if (e != hipSuccess) return e;
    if (lds <= static_bytes + 1) return hipSuccess;
    auto occupancy = [&](int dyn, int* occ) {
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, reinterpret_cast<const void*>(kernel), block,
                                                           static_cast<size_t>(dyn));
    };
    int occ = 0;
    e = occupancy(0, &occ);
    if (e != hipSuccess) return e;
    int lo = 0, hi = lds - static_bytes;  // occupancy(lo) > cap, occupancy(hi) <= cap
    if (occ > cap) {
        while (hi - lo > 1) {
            const int mid = lo + (hi - lo) / 2;
            e = occupancy(mid, &occ);
            if (e != hipSuccess) return e;
            (occ > cap ? lo : hi) = mid;
        }
    } else {
        hi = 0;
    }
    cache[cap].store(hi + 1, std::memory_order_relaxed);
    *out = static_cast<size_t>(hi);
    return hipSuccess;
}

// Large launches of cache-line rows (single_tile_launch()) of one tile per
// block take the single-tile form where single_tile_blocks() says so.  Measured on MI355X, one block
// per tile, graph replay: at 2 GiB per launch the single-tile form was 4-12 %
// faster on the geometries below; at 1 GiB within -7..+3 %, and on launches
// of 134-268 MB the walking form was as fast or faster (16384 rows of 1024
// float16 values: 23.1 against 23.2-23.6 us).
//
// Blocks per compute unit of the single-tile form for the normalizations
// (0: as many as the registers allow), or -1 where the walking form stays.
// Measured at 2 GiB per launch, layer norm, walking form against the best
// cap: float16 rows of 1024 (64-lane groups, 2 chunks) 350.6 -> 337.0 us at
// 4 blocks; 2048 (256 x 1) 390.1 -> 362.2 at 6; 4096 (256 x 2) 358.2 ->
// 344.2 at 4; 16384 (512 x 4; the walking form holds one block per CU)
// 404.3 -> 356.4 with no cap; float32 rows of 512 361.1 -> 339.6 at 3, 1024
// 386.8 -> 358.5 at 5, 2048 360.5 -> 340.1 at 4; RMS alike (float16 2048:
// 386.6 -> 362.0, 4096: 359.7 -> 347.0).  Rows of 1536, 3072-6144 and 8192
// float16 values (and 768, 3072-5120, 4096 and 8192 float32) gained under 3 %
// or lost, as did BiasAdd and BiasSoftmax: those keep the walking form.
// 1024-lane tiles of 3 chunks per lane (rows of up to 3072 chunks, which the
// automatic choice gives them only in large launches) hold one block per CU
// in either form; the single form was faster (float16 20480: 446.6 -> 436.2
// us; float32 12288: 403.8 -> 376.1).  float32 rows of 3073-4096 chunks take
// 1024 x 4 tiles in large launches, one block per CU (against the LDS-staged
// kernel at 32768 rows: layer norm 14336 / 16384 values 1420.4 / 1927.1 ->
// 1360 / 1706 us, RMS 16384 values 1794.0 -> 1604.9; with no limit RMS ran
// 1668.8).
// Geometries whose single-tile form ran faster at every launch size
// measured, not only in large launches: float16 layer norm rows of
// 1537-2048 chunks (512 x 4; the walking form holds one block per CU).
// Walking -> single-tile form at 1024 / 2048 / 4096 / 8192 rows: 14336
// values 30.8 / 53.2 / 99.2 / 196.2 -> 26.3 / 44.1 / 80.7 / 155.9 us, 16384
// values 32.3 / 56.7 / 109.5 / 207.3 -> 29.0 / 49.8 / 93.5 / 177.8; 12352
// values at 1024 / 4096 rows 28.2 / 95.7 -> 23.7 / 72.7; at 256 rows the two
// forms are equal.  RMS (fewer
// registers) lost at 1024 rows (27.7 against 29.3) and float32 layer norm at
// 32768 (3.6 %): both keep the large-launch rule.  float32 layer norm rows
// of 1537-2048 chunks take 1024 x 3 tiles in this form instead (the
// automatic choice in skipln_kernels.hip), and so does every other launch of
// that tile (its walking form spills).  Rows must be whole 128-byte lines,
// as for large launches.
template <typename E, int OP, int G, int CH>
constexpr bool single_tile_always() {
    return OP == kOpLayerNorm && ((E::kPerChunk == 8 && G == 512 && CH == 4) ||
                                  (E::kPerChunk == 4 && G == 1024 && CH == 3));
}

template <typename E, int OP, int G, int CH>
constexpr int single_tile_blocks() {
    // float16 BiasSoftmax rows of 513-1024 chunks (512 x 2 tiles): large
    // launches of 262144 rows of 8192 keys with a padding mask ran 1354 /
    // 1431 us in the single-tile form against about 1500 / 1507 walking on two
    // boxes.  float32 rows on 512 x 2 and 512 x 4 tiles gained 5-6 % on one box
    // and lost 1-10 % on the other, and stay walking.
    if constexpr (OP == kOpBiasSoftmax) return E::kPerChunk == 8 && G == 512 && CH == 2 ? 0 : -1;
    if constexpr (OP != kOpLayerNorm && OP != kOpSimplified) return -1;
    constexpr bool half = E::kPerChunk == 8;
    if constexpr (G == 64 && CH == 2) return half ? 4 : 3;
    if constexpr (G == 256 && CH == 1) return half ? 6 : 5;
    if constexpr (G == 256 && CH == 2) return 4;
    if constexpr (G == 512 && CH == 4) return half ? 0 : -1;
    if constexpr (G == 1024 && CH == 3) return 0;
    if constexpr (G == 1024 && CH == 4) return half ? -1 : 1;
    return -1;
}

constexpr int64_t kMaxGrid = 0x7FFFFFFF;
// Batches a skip-stationary block walks when the launch does not say.
constexpr int64_t kStationaryBatches = 3;
// A dispatch counts its work-items in 32 bits: blocks x block stays below 2^32.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;

// The single-tile form's blocks per CU for a launch that asks for `cap`
// (kBlocksAuto: the table's, or no limit where the table keeps the walking
// form), and the dynamic LDS that enforces it.
template <typename E, int OP, int GG, int CH, int BLOCK>
hipError_t one_tile_lds(int cap, size_t* lds) {
    static std::atomic<int> cache[kMaxBlocksCap + 1];
    constexpr int table = single_tile_blocks<E, OP, GG, CH>();
    if (cap < 0) cap = table > 0 ? table : 0;
    return cap_lds(rowtile_kernel<E, OP, GG, CH, BLOCK, kFormOneTile>, BLOCK, cap, partial_bytes<GG, BLOCK>(), cache,
                   lds);
}

// Blocks of a geometry's kernel a compute unit holds at once in kernel form
// `form` (kFormWalk, or kFormOneTile held to `blocks_per_cu` as a launch of
// that form is).
template <typename E, int OP, int GG, int CH, int BLOCK>
hipError_t occupancy_geom(int form, int blocks_per_cu, int* out) {
    if (form == kFormWalk)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
            out, reinterpret_cast<const void*>(rowtile_kernel<E, OP, GG, CH, BLOCK, kFormWalk>), BLOCK, 0);
    size_t lds = 0;
    const hipError_t e = one_tile_lds<E, OP, GG, CH, BLOCK>(blocks_per_cu, &lds);
    if (e != hipSuccess) return e;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        out, reinterpret_cast<const void*>(rowtile_kernel<E, OP, GG, CH, BLOCK, kFormOneTile>), BLOCK, lds);
}

template <typename E, int OP, int GG, int CH, int BLOCK>
hipError_t launch_geom(const Args& a0, Tiling tiling, hipStream_t st) {
    constexpr Geom g = {GG, CH, BLOCK};
    static int occ = 0;
    auto kernel = rowtile_kernel<E, OP, g.g, g.ch, g.block, kFormWalk>;
    const int64_t rpb = g.block / g.g;
    const int64_t tiles = (a0.rows + rpb - 1) / rpb;
    Args a = a0;
    int mode = tiling.mode;
    int64_t per = tiling.tiles_per_block;
    const int64_t max_blocks = kMaxWorkItems / g.block < kMaxGrid ? kMaxWorkItems / g.block : kMaxGrid;
    // Skip-stationary needs a broadcast skip whose rows split into whole tiles.
    if (mode == kTileSkipStationary &&
        (a.skip_rows <= 0 || a.skip_rows % rpb != 0 || a.skip_rows / rpb > max_blocks))
        mode = kTileStrided;
    int64_t resident = 0;
    if (per <= 0 && mode != kTileSkipStationary) {
        const hipError_t e = resident_blocks(kernel, g.block, &occ, &resident);
        if (e != hipSuccess) return e;
    }
    int64_t blocks = 1;
    if (mode == kTileSkipStationary) {
        const int64_t P = a.skip_rows / rpb;
        const int64_t batches = a.rows / a.skip_rows;
        if (per <= 0) {
            // Each block keeps its skip rows for kStationaryBatches batches.
            // Measured on MI355X over seven broadcast shapes (64-512
            // batches of 64-2048 skip rows, 768-8192 values, both types,
            // layer norm and RMS): 3 batches per block was the fastest or
            // within 2 % of it on every shape, and 8-15 % faster on six of
            // them than a grid sized to the resident blocks; that grid's
            // speed also swung with the block count (on 64 batches of 512
            // float32 rows of 4096: 175 us at 512 blocks, 190-205 us at
            // 1024-2048, 178 us at 3 batches per block).
            per = kStationaryBatches < batches ? kStationaryBatches : batches;
        }
        // At most max_blocks / P batch chunks per tile column.
        const int64_t chunks_max = max_blocks / P;
        if ((batches + per - 1) / per > chunks_max) per = (batches + chunks_max - 1) / chunks_max;
        blocks = P * ((batches + per - 1) / per);
    } else {
        if (per <= 0) {
            // Persistent: one wave of resident blocks walks all tiles, strided.
            per = (tiles + resident - 1) / resident;
            mode = kTileStrided;
        }
        if ((tiles + per - 1) / per > max_blocks) per = (tiles + max_blocks - 1) / max_blocks;
        blocks = (tiles + per - 1) / per;
    }
    a.tiles_per_block = per;
    a.tiling = mode;
    // An exact skip streams its first tile (the SS kernel) when the launch is
    // one wave of resident blocks with one tile each: measured 4.15 against
    // 4.28 us on 1024 rows of 768 float32 values, 3.7 against 3.8 us on 1024
    // rows of 768 float16 values.  Launches whose blocks walk several tiles,
    // or whose grid runs in several waves, measured slower with it (25
    // against 23 us on 16384 rows of 1024 float16 values).  Element-wise
    // kernels (odd row lengths) keep one form.
    if constexpr (E::kPerChunk > 1) {
        if (tiling.form == kFormAuto && mode != kTileSkipStationary && a.skip_rows <= 0 && a.skip_group <= 0 &&
            per <= 1) {
            static int occ_ss = 0;
            auto kernel_ss = rowtile_kernel<E, OP, g.g, g.ch, g.block, kFormStreamSkip>;
            int64_t resident_ss = 0;
            const hipError_t e = resident_blocks(kernel_ss, g.block, &occ_ss, &resident_ss);
            if (e != hipSuccess) return e;
            if (blocks <= resident_ss) return launch_grid(kernel_ss, g.block, blocks < 1 ? 1 : blocks, a, st);
        }
    }
    if constexpr (E::kPerChunk > 1) {
        if (mode != kTileSkipStationary && per <= 1) {
            // The single-tile form when forced, or for a large launch (or a
            // geometry that takes it at any size) where the table gives it
            // blocks per CU (>= 0).
            bool single = false;
            int cap = kBlocksAuto;
            if (tiling.form == kFormOneTile) {
                single = true;
                cap = tiling.blocks_per_cu;
            } else if (tiling.form == kFormAuto) {
                const int eb = static_cast<int>(16 / E::kPerChunk);
                const bool lines = a.hidden * eb % 128 == 0;
                if (single_tile_launch(a.rows, a.hidden, eb) || (single_tile_always<E, OP, g.g, g.ch>() && lines)) {
                    cap = single_tile_blocks<E, OP, g.g, g.ch>();
                    single = cap >= 0;
                }
            }
            if (single) {
                size_t lds = 0;
                const hipError_t e = one_tile_lds<E, OP, g.g, g.ch, g.block>(cap, &lds);
                if (e != hipSuccess) return e;
                return launch_grid(rowtile_kernel<E, OP, g.g, g.ch, g.block, kFormOneTile>, g.block,
                                   blocks < 1 ? 1 : blocks, a, st, lds);
            }
        }
    }
    return launch_grid(kernel, g.block, blocks < 1 ? 1 : blocks, a, st);
}

template <typename T, int OP, int... I>
hipError_t launch_geom_dispatch(int idx, const Args& a, Tiling t, hipStream_t st, std::integer_sequence<int, I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((idx == I ? (r = launch_geom<Elem<T>, OP, kGeoms[I].g, kGeoms[I].ch, kGeoms[I].block>(a, t, st), 0) : 0), ...);
    return r;
}

template <typename T, int OP, int... I>
hipError_t occupancy_geom_dispatch(int idx, int form, int blocks_per_cu, int* out, std::integer_sequence<int, I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((idx == I ? (r = occupancy_geom<Elem<T>, OP, kGeoms[I].g, kGeoms[I].ch, kGeoms[I].block>(form, blocks_per_cu, out),
                  0)
               : 0),
     ...);
    return r;
}

template <typename T, int OP, int... I>
hipError_t launch_elem_dispatch(int idx, const Args& a, Tiling t, hipStream_t st, std::integer_sequence<int, I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((idx == I ? (r = launch_geom<Single<T>, OP, kElemGeoms[I].g, kElemGeoms[I].ch, kElemGeoms[I].block>(a, t, st),
                  0)
               : 0),
     ...);
    return r;
}

}  // namespace rowtile
}  // namespace skipln
