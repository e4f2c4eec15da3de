// Span row tiles: the row operations (SkipLayerNormalization and its
// root-mean-square form, BiasAdd, BiasSoftmax; SkipLayerNormalization
// manifest `description`, `inputs`, `outputs`; BiasAdd manifest
// `description`; BiasSoftmax manifest `description`) on rows whose length is
// not a whole number of 16-byte chunks (a softmax over 77, 197 or 1500 keys),
// with every tensor 16-byte aligned at its base.
//
// The tensors are read as arrays of aligned 16-byte chunks: a group of G
// lanes owns one row and lane t loads the chunks k*G + t (k < CH) of the span
// of chunks that the row's bytes touch, so every load is a 16-byte access
// whatever the row's offset.  The first and last chunk of a span also hold
// elements of the neighbouring rows: those elements take no part in the row's
// arithmetic, and in those two chunks the outputs are stored element by
// element (another lane stores the neighbour's elements, which are other
// bytes), in every other chunk as one 16-byte store.
//
// Per-column vectors (gamma, beta, bias) and a broadcast skip row start at
// other offsets within their chunks than the data row does.  The offset
// between the two is the same for every chunk of a row, so a lane loads the
// two aligned chunks that cover its 16 bytes and shifts them into place
// (dword select, then a byte align).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skipln_device.h"
#include "skipln_internal.h"
#include "skipln_rowtile.h"

namespace skipln {
namespace {
using namespace device;

struct SpanGeom {
    int g, ch, block;
};

// Each geometry holds rows spanning up to g * ch chunks; the automatic
// choice takes the first that holds the row.
constexpr SpanGeom kSpanGeoms[] = {
    {8, 2, 256}, {16, 2, 256}, {32, 2, 256}, {64, 2, 256}, {64, 4, 256}, {128, 4, 256}, {256, 4, 256}, {512, 4, 512},
    {64, 3, 256}, {128, 3, 256}, {256, 3, 256}, {512, 3, 512},
};
constexpr int kNumSpanGeoms = sizeof(kSpanGeoms) / sizeof(kSpanGeoms[0]);
static_assert(kSpanFirst + kNumSpanGeoms <= kRegRowIndex, "kernel index ranges are disjoint");

// Chunks a row of `hidden` values of `elem_bytes` each can touch: its bytes
// plus up to 15 before its first chunk boundary.
inline int64_t span_chunks(int64_t hidden, int elem_bytes) { return (hidden * elem_bytes + 15) / 16 + 1; }

// The 16 bytes at byte `sigma` (0-15) of the 32-byte pair lo:hi: a dword
// select (a uniform branch when every lane of the wavefront shifts alike,
// selects otherwise), then one byte align per dword.
template <bool UNIFORM>
__device__ __forceinline__ u32x4 realign(const u32x4& lo, const u32x4& hi, int sigma) {
    if constexpr (UNIFORM) sigma = __builtin_amdgcn_readfirstlane(sigma);
    const int ds = sigma >> 2;
    const unsigned bs = static_cast<unsigned>(sigma & 3);
    unsigned s0, s1, s2, s3, s4;
    if constexpr (UNIFORM) {
        switch (ds) {
            case 0: s0 = lo.x; s1 = lo.y; s2 = lo.z; s3 = lo.w; s4 = hi.x; break;
            case 1: s0 = lo.y; s1 = lo.z; s2 = lo.w; s3 = hi.x; s4 = hi.y; break;
            case 2: s0 = lo.z; s1 = lo.w; s2 = hi.x; s3 = hi.y; s4 = hi.z; break;
            default: s0 = lo.w; s1 = hi.x; s2 = hi.y; s3 = hi.z; s4 = hi.w; break;
        }
    } else {
        const unsigned w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        unsigned s[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) s[k] = ds == 0 ? w[k] : ds == 1 ? w[k + 1] : ds == 2 ? w[k + 2] : w[k + 3];
        s0 = s[0]; s1 = s[1]; s2 = s[2]; s3 = s[3]; s4 = s[4];
    }
    u32x4 r;
    r.x = __builtin_amdgcn_alignbyte(s1, s0, bs);
    r.y = __builtin_amdgcn_alignbyte(s2, s1, bs);
    r.z = __builtin_amdgcn_alignbyte(s3, s2, bs);
    r.w = __builtin_amdgcn_alignbyte(s4, s3, bs);
    return r;
}

// Bytes 0 .. dx-1 of `head` followed by bytes dx .. 15 of `rest`.
__device__ __forceinline__ u32x4 splice(const u32x4& head, const u32x4& rest, int dx) {
    const unsigned h[4] = {head.x, head.y, head.z, head.w};
    const unsigned r[4] = {rest.x, rest.y, rest.z, rest.w};
    unsigned o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cut = dx - 4 * q;  // bytes of dword q taken from head
        const unsigned m = cut >= 4 ? 0xFFFFFFFFu : cut <= 0 ? 0u : (1u << (cut * 8)) - 1u;
        o[q] = (h[q] & m) | (r[q] & ~m);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// A vector of `chunks` whole or partial 16-byte chunks seen from a row:
// chunk i of the row's span needs the vector's chunks q0 + i and q0 + i + 1,
// shifted by `sig` bytes; chunks outside the vector read as zeros.  A partial
// last chunk lies within the same 4 KiB page as the vector's last byte (the
// base is 16-byte aligned), so reading all of it is safe; its bytes past the
// vector are never used.
struct VecView {
    const u32x4* p;  // the vector's chunk q0
    int lo, hi;      // span chunks i whose vector chunk q0 + i exists: lo <= i < hi
    int sig;
    __device__ VecView(const void* base, int64_t q0, int64_t chunks, int s) : sig(s) {
        p = static_cast<const u32x4*>(base) + q0;
        lo = q0 < 0 ? static_cast<int>(-q0) : 0;
        const int64_t h = chunks - q0;
        hi = h > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(h);
    }
    template <bool UNIFORM>
    __device__ __forceinline__ u32x4 chunk(int i) const {
        const u32x4 z{0, 0, 0, 0};
        const u32x4 a = i >= lo && i < hi ? p[i] : z;
        const u32x4 b = i + 1 >= lo && i + 1 < hi ? p[i + 1] : z;
        return realign<UNIFORM>(a, b, sig);
    }
};

template <typename T, int OP, int G, int CH, int BLOCK>
__global__ void __launch_bounds__(BLOCK) span_kernel(const Args a) {
    static_assert(OP == kOpLayerNorm || OP == kOpSimplified || OP == kOpBiasAdd || OP == kOpBiasSoftmax,
                  "operation");
    using E = Elem<T>;
    constexpr int V = E::kPerChunk;
    constexpr int SZ = 16 / V;                         // bytes per element
    constexpr bool kNorm = OP == kOpLayerNorm || OP == kOpSimplified;
    constexpr int RPB = BLOCK / G;                     // rows per block
    constexpr int WPR = G > 64 ? G / 64 : 1;           // wavefronts per row
    static_assert(BLOCK % G == 0 && BLOCK % 64 == 0 && G >= 8, "block of whole groups and wavefronts");
    __shared__ float4 partial[2][RPB][WPR];
    // Seams: the chunk that holds the end of one row and the start of the
    // next.  Where both rows lie in one wavefront (all but every (64/G)th
    // row), the two rows' lanes park their copies of it here and the later
    // row's first lane stores the spliced chunk whole, instead of both
    // storing their elements one by one.  One wavefront writes and reads each
    // entry, so no barrier is needed: its LDS operations complete in order.
    // Taken for softmax rows of 8 and 16 lanes: over 77 / 197 float16 keys
    // 127-136 / 64-66 against 151 / 70-71 us, 121 float32 keys 138-139
    // against 142-143.  Elsewhere the few registers it holds cost more than
    // the stores save (32-lane softmax rows over 255 keys, the
    // normalizations and BiasAdd: 2-7 % slower; some lost a wavefront of
    // occupancy).  Outputs: out, and the normalizations' residual.
    constexpr int NOUT = kNorm ? 2 : 1;
    constexpr bool kSeams = OP == kOpBiasSoftmax && G <= 16;
    constexpr int kSeamRows = kSeams ? RPB : 1;
    __shared__ u32x4 seam_head[NOUT][kSeamRows];  // from the earlier row
    __shared__ u32x4 seam_rest[NOUT][kSeamRows];  // from the later row

    const int tid = threadIdx.x;
    const int slot = G >= 64 ? __builtin_amdgcn_readfirstlane(tid / G) : tid / G;
    const int lt = tid - slot * G;
    const int64_t H = a.hidden;
    // Tiles of RPB rows, one per block unless the rows outnumber what one
    // dispatch can hold (2^32 work-items): then blocks walk tiles strided,
    // the partials double-buffered so one barrier per tile suffices.
    const int64_t n_tiles = (a.rows + RPB - 1) / RPB;
    auto tile = [&](const int64_t row0, const int par) {
        const int64_t row = row0 + slot;
        const bool live = row < a.rows;
        const float h = static_cast<float>(a.hidden);
        const float inv_h = 1.0f / h;

        // The row's bytes [rb, rb + H*SZ) span chunks c0 .. c0 + n - 1; its first
        // element is element d of chunk c0 (byte dx).
        const int64_t rb = row * H * SZ;
        const int dx = static_cast<int>(rb & 15);
        const int d = dx / SZ;
        const int64_t c0 = rb >> 4;
        const int n = live ? static_cast<int>(((rb + H * SZ + 15) >> 4) - c0) : 0;

        const u32x4* X = static_cast<const u32x4*>(a.input);
        const u32x4* S = static_cast<const u32x4*>(a.skip);
        const bool bcast = a.skip_rows > 0 || a.skip_group > 0;
        const bool has_bias = OP != kOpBiasSoftmax && a.bias != nullptr;
        const bool has_beta = kNorm && a.beta != nullptr;
        const bool small_rows = a.rows <= 0xFFFFFFFFll;

        // Byte offset between the data row and a row of a per-column vector or
        // of a broadcast skip, taken as floor chunk `q0` and remainder `sig`:
        // for chunk i of the span the vector's bytes are at 16 * (q0 + i) + sig.
        const int psig = (16 - dx) & 15;        // per-column vectors (row 0 at their base)
        const int64_t pq0 = dx > 0 ? -1 : 0;
        const int64_t pchunks = (H * SZ + 15) >> 4;
        int64_t sq0 = 0, schunks = 0;
        int ssig = 0;
        if (bcast) {
            const int64_t sb = skip_row_of(live ? row : 0, a, small_rows) * H * SZ - dx;
            sq0 = sb >= 0 ? sb >> 4 : -((15 - sb) >> 4);
            ssig = static_cast<int>(sb - sq0 * 16);
            const int64_t srows = a.skip_group > 0 ? a.rows / a.skip_group : a.skip_rows;
            schunks = (srows * H * SZ + 15) >> 4;
        }
        // One row per wavefront or more: every lane shifts alike.
        constexpr bool kUniform = G >= 64;
        auto vec_chunk = [&](const VecView& v, int i) -> u32x4 { return v.template chunk<kUniform>(i); };
        const VecView skip_view(a.skip, sq0, schunks, ssig);
        const VecView bias_view(a.bias, pq0, pchunks, psig);

        // Loads: the data row's chunks (non-temporal), the skip's (the same
        // chunks for an exact skip; shifted into place for a broadcast one), and
        // the bias's.  Rows of fewer than 64 lanes load their two end chunks,
        // which the neighbouring rows load too, through the caches, so that the
        // second load finds the line: softmax over 77 / 197 float16 keys 150 /
        // 71 against 212 / 79 us non-temporal (with the end-chunk store policy
        // below); at 64 lanes and more it gained nothing.
        u32x4 xr[CH], sr[CH], br[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int i = k * G + lt;
            const bool in = i < n;
            const bool cached = G < 64 && (i == 0 || i == n - 1);
            xr[k] = in ? (cached ? X[c0 + i] : __builtin_nontemporal_load(X + c0 + i)) : E::zero();
            if (!bcast)
                sr[k] = in ? (cached ? S[c0 + i] : __builtin_nontemporal_load(S + c0 + i)) : E::zero();
            else
                sr[k] = in ? vec_chunk(skip_view, i) : E::zero();
            br[k] = in && has_bias ? vec_chunk(bias_view, i) : E::zero();
        }

        // Element e of chunk i holds column i*V + e - d; it belongs to the row
        // when that column lies in [0, H).
        const int hid = a.hidden;
        auto valid = [&](int k, int e) {
            const int col = (k * G + lt) * V + e - d;
            return col >= 0 && col < hid;
        };
        // Whether chunk k of this lane lies wholly inside the row: only the
        // two end chunks of a span (and chunks past it) need per-element
        // masks, so the arithmetic masks just those, behind a branch that
        // most wavefronts skip.
        auto inside = [&](int k) {
            const int first = (k * G + lt) * V - d;
            return first >= 0 && first + V <= hid;
        };

        // Outputs through a buffer resource over the tile's chunks (base and
        // size uniform): whole chunks of the row as one 16-byte store, the two
        // end chunks element by element.  Offsets stay in the vector offset.
        const int64_t rows_in = a.rows - row0 < RPB ? a.rows - row0 : RPB;
        const int64_t t0 = (row0 * H * SZ) >> 4;
        const int64_t t1 = ((row0 + rows_in) * H * SZ + 15) >> 4;
        const int tile_bytes = static_cast<int>((t1 - t0) * 16);
        const int lane_base = static_cast<int>(c0 - t0);
        const bool through = a.store_through != 0;
        // Rows longer than one chunk have distinct first and last chunks, so
        // a seam holds the ends of exactly two rows.  Seam j (the start of
        // slot j) joins two rows of one wavefront unless slot j starts one.
        const bool seams = kSeams && H * SZ > 16;
        auto joined = [&](int j) { return j % (64 / G) != 0; };
        const int tail_bytes = static_cast<int>((rb + H * SZ) & 15);  // of the row in its last chunk; 0: whole
        auto put = [&](void* base, int o, int k, const u32x4& v) {
            const __amdgpu_buffer_rsrc_t r = buffer_rsrc(static_cast<char*>(base) + t0 * 16, tile_bytes);
            const int i = k * G + lt;
            const int voff = (lane_base + i) * 16;
            const int first = i * V - d;  // column of element 0
            if (first >= 0 && first + V <= hid) {
                E::store(v, r, voff, 0, through);
                return;
            }
            if (seams) {
                if (i == 0 && dx != 0 && joined(slot)) {
                    seam_rest[o][slot] = v;
                    return;
                }
                if (i == n - 1 && tail_bytes != 0 && slot + 1 < rows_in && joined(slot + 1)) {
                    seam_head[o][slot + 1] = v;
                    return;
                }
            }
            // End chunks: the neighbouring row writes the chunk's other
            // elements, so these stores take the default (write-back) policy,
            // which lets the cache merge the two rows' halves of a line:
            // layer norm over 1,048,576 rows of 77 float16 values 286 against
            // 422 us with non-temporal stores, BiasAdd over 121 float32
            // values 155 against 192 (with the end-chunk loads above); 1-2 %
            // at 1001 values.
            const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < V; ++e) {
                if (!valid(k, e)) continue;
                if constexpr (SZ == 4) {
                    __builtin_amdgcn_raw_buffer_store_b32(w[e], r, voff + e * 4, 0, 0);
                } else {
                    const unsigned short hv = static_cast<unsigned short>(w[e >> 1] >> ((e & 1) * 16));
                    __builtin_amdgcn_raw_buffer_store_b16(hv, r, voff + e * 2, 0, 0);
                }
            }
        };

        // The joined seams, once the wavefront's rows have parked their ends:
        // the later row's first lane stores each.
        auto flush_seams = [&]() {
            if (!seams) return;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lt == 0 && live && dx != 0 && joined(slot)) {
#pragma unroll
                for (int o = 0; o < NOUT; ++o) {
                    void* base = o == 0 ? a.out : a.residual;
                    if (base == nullptr) continue;
                    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(static_cast<char*>(base) + t0 * 16, tile_bytes);
                    E::store(splice(seam_head[o][slot], seam_rest[o][slot], dx), r, lane_base * 16, 0, through);
                }
            }
        };

        // s = (x + skip) + bias in binary32 (BiasAdd: (x + bias) + skip;
        // BiasSoftmax: data + bias, the bias arriving through the skip slot).
        float s[CH][V];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            float xf[V], sf[V], bf[V];
            E::widen(xr[k], xf);
            E::widen(sr[k], sf);
            E::widen(br[k], bf);
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

        if constexpr (OP == kOpBiasAdd) {
#pragma unroll
            for (int k = 0; k < CH; ++k)
                if (k * G + lt < n) put(a.out, 0, k, E::narrow(s[k]));
            flush_seams();
            return;
        }

        if constexpr (OP == kOpBiasSoftmax) {
            // As the row tiles: exponentials relative to the row maximum (one
            // wavefront or less per row) or to each wavefront's maximum merged
            // through LDS; elements outside the row enter as -inf.
            constexpr float kLog2e = 1.4426950408889634f;
            constexpr float kNegInf = -__builtin_inff();
            float mx = kNegInf;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (!inside(k)) {
#pragma unroll
                    for (int e = 0; e < V; ++e) s[k][e] = valid(k, e) ? s[k][e] : kNegInf;
                }
#pragma unroll
                for (int e = 0; e < V; ++e) mx = __builtin_fmaxf(mx, s[k][e]);
            }
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
            for (int k = 0; k < CH; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    // -inf (outside the row) gives 0; a row of -inf only is
                    // NaN throughout, as the definition has it.
                    s[k][e] = __builtin_amdgcn_exp2f((s[k][e] - r) * kLog2e);
                    part += s[k][e];
                }
            float scale;
            if constexpr (WPR == 1) {
                scale = 1.0f / group_sum<G>(part);
            } else {
                const float ws = wave_sum(part);
                if ((lt & 63) == 0) partial[par][slot][lt >> 6] = make_float4(m, ws, 0.0f, 0.0f);
                __syncthreads();
                float row_max = kNegInf;
#pragma unroll
                for (int w = 0; w < WPR; ++w) row_max = __builtin_fmaxf(row_max, partial[par][slot][w].x);
                float total = 0.0f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    const float4 p = partial[par][slot][w];
                    const float f = p.x == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((p.x - row_max) * kLog2e);
                    total += p.y * f;
                }
                const float own = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f((m - row_max) * kLog2e);
                scale = own / total;
            }
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (k * G + lt < n) {
                    float y[V];
#pragma unroll
                    for (int e = 0; e < V; ++e) y[e] = s[k][e] * scale;
                    put(a.out, 0, k, E::narrow(y));
                }
            }
            flush_seams();
            return;
        }

        if (a.residual != nullptr) {
#pragma unroll
            for (int k = 0; k < CH; ++k)
                if (k * G + lt < n) put(a.residual, 1, k, E::narrow(s[k]));
        }
        // gamma and beta once the residual is out (their registers are not held
        // through the sum).
        const VecView gamma_view(a.gamma, pq0, pchunks, psig);
        const VecView beta_view(a.beta, pq0, pchunks, psig);
        u32x4 gr[CH], er[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int i = k * G + lt;
            const bool in = i < n;
            gr[k] = in ? vec_chunk(gamma_view, i) : E::zero();
            er[k] = in && has_beta ? vec_chunk(beta_view, i) : E::zero();
        }

        // Statistics as the row tiles take them: relative to a value of the row
        // (the first element in each wavefront's first chunk), merged across
        // wavefronts with Chan et al.'s update; RMS: the mean square.
        float first = s[0][0];
#pragma unroll
        for (int e = 1; e < V; ++e) first = (lt == 0 && e == d) ? s[0][e] : first;
        float shift = 0.0f;
        if constexpr (OP == kOpLayerNorm) shift = group_first<G>(first);
        // Elements outside the row (in the end chunks only) are set to the
        // shift (RMS: 0), so they add nothing to the sums, and before the
        // second pass to the mean, so they add nothing to the squared
        // deviations either.
        float part = 0.0f;
        int outside = 0;
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (!inside(k)) {
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const bool ok = valid(k, e);
                    outside += ok ? 0 : 1;
                    s[k][e] = ok ? s[k][e] : shift;
                }
            }
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
        const float outside_f = static_cast<float>(outside);
        auto park = [&](float value) {
#pragma unroll
            for (int k = 0; k < CH; ++k)
                if (!inside(k))
#pragma unroll
                    for (int e = 0; e < V; ++e) s[k][e] = valid(k, e) ? s[k][e] : value;
        };
        float off = 0.0f, var;
        if constexpr (OP == kOpSimplified) {
            if constexpr (WPR == 1) {
                var = group_sum<G>(part) * inv_h;
            } else {
                const float wsq = wave_sum(part);
                if ((lt & 63) == 0) partial[par][slot][lt >> 6] = make_float4(wsq, 0.0f, 0.0f, 0.0f);
                __syncthreads();
                float tot = 0.0f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) tot += partial[par][slot][w].x;
                var = tot * inv_h;
            }
        } else if constexpr (WPR == 1) {
            const float dmean = group_sum<G>(part) * inv_h;
            off = dmean;
            park(dmean);
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < CH; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float dv = s[k][e] - dmean;
                    q += dv * dv;
                }
            var = group_sum<G>(q) * inv_h;
        } else {
            // Per wavefront: its own first value as the shift (wavefront w's
            // lane 0 holds chunk 64 w, whose element 0 is in the row whenever
            // the wavefront holds any), its mean and squared deviations; merged
            // relative to wavefront 0's shift.
            const float wn = wave_sum(static_cast<float>(CH * V) - outside_f);
            const float wd = wn > 0.0f ? wave_sum(part) / wn : 0.0f;
            park(wd);
            float q = 0.0f;
#pragma unroll
            for (int k = 0; k < CH; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float dv = s[k][e] - wd;
                    q += dv * dv;
                }
            const float wm2 = wave_sum(q);
            if ((lt & 63) == 0) partial[par][slot][lt >> 6] = make_float4(shift, wd, wm2, wn);
            __syncthreads();
            const float row_shift = partial[par][slot][0].x;
            float dsum = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const float4 p = partial[par][slot][w];
                if (p.w > 0.0f) dsum += p.w * ((p.x - row_shift) + p.y);
            }
            const float dmean = dsum * inv_h;
            float m2 = 0.0f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const float4 p = partial[par][slot][w];
                if (p.w > 0.0f) {
                    const float dm = ((p.x - row_shift) + p.y) - dmean;
                    m2 += p.z + p.w * dm * dm;
                }
            }
            var = m2 * inv_h;
            off = dmean - (shift - row_shift);
        }
        const float rstd = rsqrtf(var + a.eps);
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (k * G + lt < n) {
                float t[V], y[V];
#pragma unroll
                for (int e = 0; e < V; ++e) t[e] = (s[k][e] - off) * rstd;
                E::widen_fma(t, gr[k], er[k], y);
                put(a.out, 0, k, E::narrow(y));
            }
        }
        flush_seams();
    };
    int par = 0;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x, par ^= 1) tile(t * RPB, par);
}

template <typename T, int OP, int I>
hipError_t launch_span_geom(const Args& a, hipStream_t st) {
    constexpr SpanGeom g = kSpanGeoms[I];
    constexpr int rpb = g.block / g.g;
    // One tile per block, within a dispatch's 2^32 work-items.
    constexpr int64_t kMaxBlocks = 0xFFFFFFFFll / g.block;
    int64_t blocks = (a.rows + rpb - 1) / rpb;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    Args arg = a;
    void* params[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void*>(span_kernel<T, OP, g.g, g.ch, g.block>),
                           dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks)), dim3(g.block), params, 0, st);
}

template <typename T, int OP, int... I>
hipError_t launch_span_dispatch(int idx, const Args& a, hipStream_t st, std::integer_sequence<int, I...>) {
    hipError_t r = hipErrorInvalidValue;
    ((idx == I ? (r = launch_span_geom<T, OP, I>(a, st), 0) : 0), ...);
    return r;
}

template <int OP>
hipError_t launch_span_op(const Args& a, int dtype, int geometry, hipStream_t st) {
    auto seq = std::make_integer_sequence<int, kNumSpanGeoms>{};
    return dtype == 0 ? launch_span_dispatch<float, OP>(geometry, a, st, seq)
                      : launch_span_dispatch<_Float16, OP>(geometry, a, st, seq);
}

}  // namespace

int span_count() { return kNumSpanGeoms; }

bool span_geometry(int geometry, int* g, int* ch, int* block) {
    if (geometry < 0 || geometry >= kNumSpanGeoms) return false;
    *g = kSpanGeoms[geometry].g;
    *ch = kSpanGeoms[geometry].ch;
    *block = kSpanGeoms[geometry].block;
    return true;
}

bool span_holds(int geometry, int64_t hidden, int dtype) {
    if (geometry < 0 || geometry >= kNumSpanGeoms || hidden <= 0) return false;
    const int64_t cap = static_cast<int64_t>(kSpanGeoms[geometry].g) * kSpanGeoms[geometry].ch;
    return span_chunks(hidden, dtype == 0 ? 4 : 2) <= cap;
}

int span_fit(int /*op*/, int64_t hidden, int dtype) {
    // The geometry of least capacity (lanes x chunks) that holds the row.
    int best = -1;
    for (int i = 0; i < kNumSpanGeoms; ++i)
        if (span_holds(i, hidden, dtype) &&
            (best < 0 || kSpanGeoms[i].g * kSpanGeoms[i].ch < kSpanGeoms[best].g * kSpanGeoms[best].ch))
            best = i;
    return best;
}

int span_pick(int op, int64_t hidden, int dtype, bool broadcast) {
    const int g = span_fit(op, hidden, dtype);
    if (g < 0) return -1;
    // Measured on MI355X against the element-wise tiles (graph replay, exact
    // skip or bias, 128 MiB per tensor; span / element us):
    //  - BiasSoftmax: faster from 8 chunks touched on -- float16 keys 77 /
    //    197 / 300 / 500 / 1001 / 1500 / 3001 / 4095: 93 / 80 / 84 / 74 / 68 /
    //    67 / 69 / 86 against 145 / 126 / 157 / 110 / 86 / 111 / 125 / 103;
    //    float32 keys 77 / 500 / 2047: 77 / 65 / 67 against 83 / 70 / 74 --
    //    and slower on rows of a chunk or two (13 keys: 338 against 149).
    //  - BiasAdd: faster from 64 chunks on -- float16 500 / 1001 / 3001
    //    values: 71 / 74 / 80 against 87 / 84 / 92; float32 1001 / 2047: 79 /
    //    76 against 83 / 85 -- mixed below (float16 121 / 255: 96 / 118
    //    against 105 / 91; float32 77 / 121: 98 / 83 against 84 / 85).
    //  - Layer norm and RMS: slower on short rows (float16 13 / 77 / 255
    //    values: 543 / 222 / 212 against 183 / 184 / 133), within -15 % to
    //    +50 % from 64 chunks on (500: 133 against 154, 2047: 207 against
    //    136), so the normalizations keep the element-wise tiles.
    // With a broadcast skip or bias, whose rows must be shifted into place
    // chunk by chunk, the span tiles lost more often than they won (softmax
    // over 77 / 121 / 2047 / 4095 float16 keys with bias rows shared by many
    // rows: 90 / 112 / 197 / 209 against 82 / 100 / 173 / 191 us).
    if (broadcast) return -1;
    const int64_t touched = span_chunks(hidden, dtype == 0 ? 4 : 2);
    if (op == kOpBiasSoftmax) return touched >= 8 ? g : -1;
    if (op == kOpBiasAdd) return touched >= 64 ? g : -1;
    return -1;
}

hipError_t launch_span(const Args& a, int op, int dtype, int geometry, hipStream_t st) {
    if (geometry < 0 || geometry >= kNumSpanGeoms) return hipErrorInvalidValue;
    switch (op) {
        case kOpLayerNorm: return launch_span_op<kOpLayerNorm>(a, dtype, geometry, st);
        case kOpSimplified: return launch_span_op<kOpSimplified>(a, dtype, geometry, st);
        case kOpBiasAdd: return launch_span_op<kOpBiasAdd>(a, dtype, geometry, st);
        case kOpBiasSoftmax: return launch_span_op<kOpBiasSoftmax>(a, dtype, geometry, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace skipln
