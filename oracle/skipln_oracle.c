/*
 * CPU oracle for the SkipLayerNormalization row operator -- TEST
 * INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It is a plain, slow, obviously correct reading of
 * the operator and shares no code, header, table or constant with the HIP
 * implementation.
 *
 * Source of the definition: the com.microsoft SkipLayerNormalization WebGPU
 * kernel-package manifest (page "com.microsoft.SkipLayerNormalization ...
 * manifest.json"):
 *   - `description` and `inputs[input]`: a skip addition fused with a layer
 *     normalization over the last (hidden) axis;
 *   - `inputs[skip]`: skip is exact-shape, or (1,S,H) / (S,H) broadcast over
 *     the batch; `bindingSets.vec4_beta_broadcast_output_only` `Params.skipRows`
 *     is numel(skip)/H;
 *   - `inputs[bias]`: the optional bias is added to the sum input + skip,
 *     before normalization;
 *   - `inputs[gamma]`, `inputs[beta]`: per-column scale and (optional) shift;
 *   - `outputs[input_skip_bias_sum]`: the optional pre-normalization sum;
 *   - `attributes.epsilon`, `attributeDescriptions.epsilon`: a non-negative
 *     epsilon added to the variance under the square root; the `Params`
 *     structs carry it as an f32 value;
 *   - `typeConstraints.T`: float32 or float16 for every tensor.
 *
 * Readings where the manifest is silent (each is listed in the design notes):
 *   - the variance is the population variance (divide by H);
 *   - the sum is formed in IEEE binary32, in the order (input + skip) + bias,
 *     one rounding per add; the residual output is that sum rounded once to T
 *     (identity for float32, one round-to-nearest-even for float16);
 *   - normalization reads the binary32 sum (not its float16 rounding);
 *   - broadcast skip: logical row r reads skip row r mod S;
 *   - statistics and the affine step are evaluated in binary64 and the
 *     normalized output is returned unrounded, as binary64.
 *
 * fp16 <-> fp32 conversion is written out below from the IEEE 754 binary16
 * format definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits; subnormals at 2^-24 spacing; round-to-nearest, ties-to-even).
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fPIC -shared -pthread
 * (no -ffast-math, no -march=native).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_F16 1

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16                                                         */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary16 -> binary32; exact for every finite value. */
float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t m = h & 0x3FFu;
    if (e == 0x1Fu) /* infinity or NaN: keep the fraction bits */
        return bits_f32(sign | 0x7F800000u | (m << 13));
    if (e == 0) { /* zero or subnormal: m * 2^-24, exact in binary32 */
        float v = ldexpf((float)m, -24);
        return sign ? -v : v;
    }
    return bits_f32(sign | ((e - 15u + 127u) << 23) | (m << 13));
}

/* Round an integer quotient q with remainder rem (of a power-of-two divisor
 * whose half is `half`) to nearest, ties to even. */
static uint32_t round_nearest_even(uint32_t q, uint32_t rem, uint32_t half) {
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;
    return q;
}

/* binary32 -> binary16, round to nearest, ties to even.  Overflow gives
 * +-infinity; NaN gives a quiet NaN of the same sign. */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e = (u >> 23) & 0xFFu;
    uint32_t m = u & 0x7FFFFFu;

    if (e == 0xFFu)
        return (uint16_t)(sign | (m ? 0x7E00u : 0x7C00u));
    if (e == 0) /* zero, or a binary32 subnormal (< 2^-126): far below half of 2^-24 */
        return sign;

    int ue = (int)e - 127;            /* value = (2^23 + m) * 2^(ue - 23) */
    uint32_t full = 0x800000u | m;    /* 24-bit significand */
    if (ue > 15)
        return (uint16_t)(sign | 0x7C00u);
    if (ue >= -14) {
        /* Normal binary16 range: quantum 2^(ue - 10), i.e. drop 13 bits. */
        uint32_t q = round_nearest_even(full >> 13, full & 0x1FFFu, 0x1000u);
        if (q == 0x800u) { /* carried into the next binade */
            q = 0x400u;
            ue += 1;
        }
        if (ue > 15)
            return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | ((uint32_t)(ue + 15) << 10) | (q - 0x400u));
    }
    /* Subnormal binary16 range: quantum 2^-24, value / 2^-24 = full * 2^(ue + 1). */
    int shift = -(ue + 1); /* >= 14 */
    if (shift > 24)        /* value < 2^-25: below half the smallest subnormal */
        return sign;
    uint32_t q = round_nearest_even(full >> shift, full & ((1u << shift) - 1u), 1u << (shift - 1));
    /* q == 0x400 encodes the smallest normal number, as it should. */
    return (uint16_t)(sign | q);
}

void oracle_f16_to_f32_array(const uint16_t* h, float* f, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        f[i] = oracle_f16_to_f32(h[i]);
}

void oracle_f32_to_f16_array(const float* f, uint16_t* h, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        h[i] = oracle_f32_to_f16(f[i]);
}

/* ------------------------------------------------------------------------ */
/* Element access                                                            */
/* ------------------------------------------------------------------------ */

static float load_t(const void* p, int64_t i, int dtype) {
    if (dtype == ORACLE_F32)
        return ((const float*)p)[i];
    return oracle_f16_to_f32(((const uint16_t*)p)[i]);
}

static void store_t(void* p, int64_t i, float v, int dtype) {
    if (dtype == ORACLE_F32)
        ((float*)p)[i] = v;
    else
        ((uint16_t*)p)[i] = oracle_f32_to_f16(v);
}

/* ------------------------------------------------------------------------ */
/* SkipLayerNormalization                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void* input;
    const void* skip;
    int64_t skip_rows; /* 0: exact skip (row i reads skip row i) */
    const void* gamma;
    const void* beta;  /* may be NULL: treated as 0 */
    const void* bias;  /* may be NULL: treated as 0 */
    int dtype;
    int64_t hidden;
    int64_t row_offset; /* logical index of row 0 (broadcast indexing) */
    double eps;
    int simplified;     /* 1: root-mean-square normalization (no mean) */
    void* residual_out; /* T, may be NULL */
    double* y_out;      /* binary64, may be NULL */
    double* mean_out;   /* per row, may be NULL */
    double* var_out;    /* per row, may be NULL (mean square when simplified) */
    int64_t r0, r1;
    int status;
} sln_job;

static void sln_rows(sln_job* J) {
    const int64_t H = J->hidden;
    float* s = (float*)malloc((size_t)H * sizeof(float));
    if (!s) {
        J->status = -2;
        return;
    }
    for (int64_t i = J->r0; i < J->r1; ++i) {
        /* Skip row read by this row. */
        int64_t j = J->skip_rows > 0 ? (J->row_offset + i) % J->skip_rows : i;

        /* Pre-normalization sum in binary32: (input + skip) + bias. */
        for (int64_t c = 0; c < H; ++c) {
            float a = load_t(J->input, i * H + c, J->dtype) + load_t(J->skip, j * H + c, J->dtype);
            if (J->bias)
                a = a + load_t(J->bias, c, J->dtype);
            s[c] = a;
            if (J->residual_out)
                store_t(J->residual_out, i * H + c, a, J->dtype);
        }

        /* Row statistics in binary64, two passes. */
        double mean = 0.0;
        if (!J->simplified) {
            double sum = 0.0;
            for (int64_t c = 0; c < H; ++c)
                sum += (double)s[c];
            mean = sum / (double)H;
        }
        double ss = 0.0;
        for (int64_t c = 0; c < H; ++c) {
            double d = (double)s[c] - mean;
            ss += d * d;
        }
        double var = ss / (double)H;
        double denom = sqrt(var + J->eps);

        if (J->mean_out)
            J->mean_out[i] = mean;
        if (J->var_out)
            J->var_out[i] = var;
        if (J->y_out) {
            for (int64_t c = 0; c < H; ++c) {
                double g = (double)load_t(J->gamma, c, J->dtype);
                double b = J->beta ? (double)load_t(J->beta, c, J->dtype) : 0.0;
                J->y_out[i * H + c] = ((double)s[c] - mean) / denom * g + b;
            }
        }
    }
    free(s);
    J->status = 0;
}

static void* sln_thread(void* arg) {
    sln_rows((sln_job*)arg);
    return NULL;
}

/*
 * Reference SkipLayerNormalization over `rows` rows of `hidden` elements.
 *
 * input        rows x hidden, type T (row-major, contiguous)
 * skip         rows x hidden when skip_rows == 0 (exact); otherwise
 *              skip_rows x hidden, and logical row (row_offset + i) reads skip
 *              row (row_offset + i) mod skip_rows
 * gamma        hidden, type T; beta and bias: hidden or NULL
 * eps          binary32 epsilon (>= 0), widened exactly to binary64
 * residual_out rows x hidden of T, or NULL
 * y_out        rows x hidden binary64, or NULL
 * mean_out / var_out: rows binary64 each, or NULL
 * simplified   0: layer normalization; 1: root-mean-square normalization
 *              (no mean subtraction; the "variance" is the mean square)
 * Returns 0, or -1 on invalid arguments, -2 if memory ran out.
 */
int oracle_skip_norm(const void* input, const void* skip, int64_t skip_rows,
                     const void* gamma, const void* beta, const void* bias,
                     int dtype, int64_t rows, int64_t hidden, int64_t row_offset,
                     float eps, int simplified, void* residual_out, double* y_out,
                     double* mean_out, double* var_out, int nthreads) {
    if (rows < 0 || hidden <= 0 || skip_rows < 0 || row_offset < 0 || !(eps >= 0.0f))
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16)
        return -1;
    if (rows == 0)
        return 0;
    if (!input || !skip || !gamma)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > rows)
        nthreads = (int)rows;

    sln_job base;
    base.input = input;
    base.skip = skip;
    base.skip_rows = skip_rows;
    base.gamma = gamma;
    base.beta = beta;
    base.bias = bias;
    base.dtype = dtype;
    base.hidden = hidden;
    base.row_offset = row_offset;
    base.eps = (double)eps;
    base.simplified = simplified ? 1 : 0;
    base.residual_out = residual_out;
    base.y_out = y_out;
    base.mean_out = mean_out;
    base.var_out = var_out;
    base.status = 0;

    sln_job* jobs = (sln_job*)calloc((size_t)nthreads, sizeof(sln_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    char* spawned = (char*)calloc((size_t)nthreads, 1);
    if (!jobs || !tids || !spawned) {
        free(jobs);
        free(tids);
        free(spawned);
        return -2;
    }
    /* Contiguous row ranges; thread 0 is the calling thread. */
    int64_t per = (rows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].r0 = t * per < rows ? t * per : rows;
        jobs[t].r1 = (t + 1) * per < rows ? (t + 1) * per : rows;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, sln_thread, &jobs[t]) == 0)
            spawned[t] = 1;
        else
            sln_rows(&jobs[t]); /* no thread available: run it here */
    }
    sln_rows(&jobs[0]);
    int status = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (spawned[t])
            pthread_join(tids[t], NULL);
        if (jobs[t].status != 0 && status == 0)
            status = jobs[t].status;
    }
    free(jobs);
    free(tids);
    free(spawned);
    return status;
}

/* ------------------------------------------------------------------------ */
/* BiasAdd                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * Reference BiasAdd (com.microsoft BiasAdd WebGPU manifest, `description`
 * and `outputs[Y]`): the channel bias is added to X first and the residual
 * skip second, Y = (X + bias) + skip, per element of an (N, S, C) tensor
 * flattened to rows x hidden (hidden = C).  Each add is one IEEE binary32
 * add; Y is that binary32 value rounded once to T.
 * y_exact (optional, binary64): X + bias + skip evaluated in binary64.
 */
int oracle_bias_add(const void* x, const void* bias, const void* skip, int dtype,
                    int64_t rows, int64_t hidden, void* y_out, double* y_exact) {
    if (rows < 0 || hidden <= 0)
        return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16)
        return -1;
    if (rows == 0)
        return 0;
    if (!x || !bias || !skip)
        return -1;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t c = 0; c < hidden; ++c) {
            float xv = load_t(x, i * hidden + c, dtype);
            float bv = load_t(bias, c, dtype);
            float sv = load_t(skip, i * hidden + c, dtype);
            float a = xv + bv;
            a = a + sv;
            if (y_out)
                store_t(y_out, i * hidden + c, a, dtype);
            if (y_exact)
                y_exact[i * hidden + c] = (double)xv + (double)bv + (double)sv;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* BiasSoftmax                                                               */
/* ------------------------------------------------------------------------ */

/*
 * Reference BiasSoftmax (com.microsoft BiasSoftmax WebGPU manifest,
 * `description`, `attributeDescriptions`, `derive`): the data is
 * batch_count rows of block_size values (the dimensions from `axis` on,
 * flattened); bias holds bias_rows rows of block_size values, bias_rows
 * dividing batch_count.  Data row r adds bias row r / (batch_count /
 * bias_rows) when inner != 0 (consecutive groups of rows share a bias row)
 * and bias row r mod bias_rows otherwise (cyclic reuse).  z = data + bias is
 * one IEEE binary32 add; y = exp(z - max z) / sum exp(z - max z) over the row
 * in binary64, returned unrounded.
 */
int oracle_bias_softmax(const void* data, const void* bias, int dtype, int64_t batch_count, int64_t block_size,
                        int64_t bias_rows, int inner, double* y_out) {
    if (batch_count < 0 || block_size <= 0 || bias_rows <= 0 || bias_rows > batch_count ||
        batch_count % bias_rows != 0)
        return batch_count == 0 ? 0 : -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16)
        return -1;
    if (!data || !bias || !y_out)
        return -1;
    const int64_t repeat = batch_count / bias_rows;
    double* z = (double*)malloc((size_t)block_size * sizeof(double));
    if (!z)
        return -2;
    for (int64_t r = 0; r < batch_count; ++r) {
        const int64_t j = inner ? r / repeat : r % bias_rows;
        /* The row maximum; a NaN never compares greater, and then makes every
         * exp() below, and so the whole row, NaN. */
        double m = -INFINITY;
        for (int64_t c = 0; c < block_size; ++c) {
            float zf = load_t(data, r * block_size + c, dtype) + load_t(bias, j * block_size + c, dtype);
            z[c] = (double)zf;
            if (z[c] > m)
                m = z[c];
        }
        double sum = 0.0;
        for (int64_t c = 0; c < block_size; ++c)
            sum += exp(z[c] - m);
        for (int64_t c = 0; c < block_size; ++c)
            y_out[r * block_size + c] = exp(z[c] - m) / sum;
    }
    free(z);
    return 0;
}

int oracle_version(void) { return 1; }
