/*
 * Drives every entry point of the CPU oracle (oracle/skipln_oracle.c) for a
 * build under AddressSanitizer and UndefinedBehaviorSanitizer: both element
 * types, exact and broadcast skips, every optional tensor present or absent,
 * the root-mean-square form, several threads, row offsets, BiasAdd,
 * BiasSoftmax with exact, cyclic and grouped bias rows and special values,
 * every binary16 pattern through the converters, and rejected arguments.
 * Exits 0 when every internal consistency check holds; the sanitizers abort
 * the run on any memory or undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { F32 = 0, F16 = 1 };

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);
void oracle_f16_to_f32_array(const uint16_t* h, float* f, int64_t n);
void oracle_f32_to_f16_array(const float* f, uint16_t* h, int64_t n);
int oracle_skip_norm(const void* input, const void* skip, int64_t skip_rows, const void* gamma, const void* beta,
                     const void* bias, int dtype, int64_t rows, int64_t hidden, int64_t row_offset, float eps,
                     int simplified, void* residual_out, double* y_out, double* mean_out, double* var_out,
                     int nthreads);
int oracle_bias_add(const void* x, const void* bias, const void* skip, int dtype, int64_t rows, int64_t hidden,
                    void* y_out, double* y_exact);
int oracle_bias_softmax(const void* data, const void* bias, int dtype, int64_t batch_count, int64_t block_size,
                        int64_t bias_rows, int inner, double* y_out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64 (Steele, Lea and Flood, 2014) */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)((next_u64() >> 40) * (1.0 / 16777216.0)); }

static int failures = 0;
#define CHECK(cond, what)                                        \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "check failed: %s (%s)\n", what, #cond); \
            ++failures;                                          \
        }                                                        \
    } while (0)

/* Fill n elements of type dtype with uniform values in [lo, hi). */
static void* fill(int dtype, int64_t n, float lo, float hi) {
    if (n == 0) return malloc(1);
    if (dtype == F32) {
        float* p = (float*)malloc((size_t)n * sizeof(float));
        for (int64_t i = 0; i < n; ++i) p[i] = uniform(lo, hi);
        return p;
    }
    uint16_t* p = (uint16_t*)malloc((size_t)n * sizeof(uint16_t));
    for (int64_t i = 0; i < n; ++i) p[i] = oracle_f32_to_f16(uniform(lo, hi));
    return p;
}

static size_t esize(int dtype) { return dtype == F32 ? 4 : 2; }

static void skip_norm_case(int dtype, int64_t rows, int64_t hidden, int64_t skip_rows, int beta, int bias,
                           int residual, int simplified, float eps) {
    const int64_t srows = skip_rows > 0 ? skip_rows : rows;
    void* x = fill(dtype, rows * hidden, -3.0f, 3.0f);
    void* s = fill(dtype, srows * hidden, -3.0f, 3.0f);
    void* g = fill(dtype, hidden, 0.5f, 1.5f);
    void* b = beta ? fill(dtype, hidden, -0.1f, 0.1f) : NULL;
    void* bi = bias ? fill(dtype, hidden, -0.1f, 0.1f) : NULL;
    void* r1 = residual ? malloc((size_t)(rows * hidden) * esize(dtype) + 1) : NULL;
    void* r4 = residual ? malloc((size_t)(rows * hidden) * esize(dtype) + 1) : NULL;
    double* y1 = (double*)malloc((size_t)(rows * hidden) * sizeof(double) + 8);
    double* y4 = (double*)malloc((size_t)(rows * hidden) * sizeof(double) + 8);
    double* m = (double*)malloc((size_t)rows * sizeof(double) + 8);
    double* v = (double*)malloc((size_t)rows * sizeof(double) + 8);
    CHECK(oracle_skip_norm(x, s, skip_rows, g, b, bi, dtype, rows, hidden, 0, eps, simplified, r1, y1, m, v, 1) == 0,
          "skip_norm, one thread");
    CHECK(oracle_skip_norm(x, s, skip_rows, g, b, bi, dtype, rows, hidden, 0, eps, simplified, r4, y4, NULL, NULL, 4) ==
              0,
          "skip_norm, four threads");
    CHECK(memcmp(y1, y4, (size_t)(rows * hidden) * sizeof(double)) == 0, "threads agree on y");
    if (residual) CHECK(memcmp(r1, r4, (size_t)(rows * hidden) * esize(dtype)) == 0, "threads agree on residual");
    for (int64_t i = 0; i < rows; ++i) CHECK(v[i] >= 0.0, "variance non-negative");
    /* rows handed over from a row offset: the broadcast index continues */
    if (rows >= 2 && skip_rows > 0) {
        const int64_t half = rows / 2;
        double* yb = (double*)malloc((size_t)((rows - half) * hidden) * sizeof(double) + 8);
        CHECK(oracle_skip_norm((const char*)x + (size_t)(half * hidden) * esize(dtype), s, skip_rows, g, b, bi, dtype,
                               rows - half, hidden, half, eps, simplified, NULL, yb, NULL, NULL, 2) == 0,
              "skip_norm with a row offset");
        CHECK(memcmp(yb, y1 + half * hidden, (size_t)((rows - half) * hidden) * sizeof(double)) == 0,
              "row offset continues the broadcast");
        free(yb);
    }
    free(x), free(s), free(g), free(b), free(bi), free(r1), free(r4), free(y1), free(y4), free(m), free(v);
}

static void softmax_case(int dtype, int64_t rows, int64_t cols, int64_t bias_rows, int inner, int specials) {
    void* d = fill(dtype, rows * cols, -6.0f, 6.0f);
    void* b = fill(dtype, bias_rows * cols, -1.0f, 1.0f);
    if (specials && rows >= 3 && cols >= 2) {
        const float nan = nanf(""), inf = INFINITY;
        if (dtype == F32) {
            ((float*)d)[0] = nan;
            ((float*)d)[cols] = inf;
            for (int64_t c = 0; c < cols; ++c) ((float*)d)[2 * cols + c] = -inf;
        } else {
            ((uint16_t*)d)[0] = oracle_f32_to_f16(nan);
            ((uint16_t*)d)[cols] = oracle_f32_to_f16(inf);
            for (int64_t c = 0; c < cols; ++c) ((uint16_t*)d)[2 * cols + c] = oracle_f32_to_f16(-inf);
        }
    }
    double* y = (double*)malloc((size_t)(rows * cols) * sizeof(double) + 8);
    CHECK(oracle_bias_softmax(d, b, dtype, rows, cols, bias_rows, inner, y) == 0, "bias_softmax");
    for (int64_t r = specials ? 3 : 0; r < rows; ++r) {
        double sum = 0.0;
        for (int64_t c = 0; c < cols; ++c) sum += y[r * cols + c];
        CHECK(fabs(sum - 1.0) < 1e-12, "softmax rows sum to one");
    }
    if (specials && rows >= 3 && cols >= 2)
        for (int r = 0; r < 3; ++r) CHECK(isnan(y[r * cols]), "special rows are NaN");
    free(d), free(b), free(y);
}

int main(void) {
    /* every binary16 pattern widens and narrows back (NaNs stay NaN) */
    for (uint32_t h = 0; h < 65536; ++h) {
        const float f = oracle_f16_to_f32((uint16_t)h);
        const uint16_t back = oracle_f32_to_f16(f);
        if (isnan(f))
            CHECK(isnan(oracle_f16_to_f32(back)), "NaN stays NaN");
        else
            CHECK(back == (uint16_t)h, "binary16 round trip");
    }
    {
        uint16_t hs[7];
        float fs[7] = {0.0f, -0.0f, 65504.0f, 65520.0f, 5.9604645e-8f, 1e-9f, -3.0f};
        float back[7];
        oracle_f32_to_f16_array(fs, hs, 7);
        oracle_f16_to_f32_array(hs, back, 7);
        CHECK(isinf(back[3]), "65520 rounds to infinity");
        CHECK(back[5] == 0.0f, "tiny values flush to zero");
    }

    /* SkipLayerNormalization and its simplified form over the flag matrix */
    const int64_t hiddens[] = {1, 2, 3, 8, 63, 768, 1000};
    for (int dtype = F32; dtype <= F16; ++dtype)
        for (unsigned flags = 0; flags < 32; ++flags)
            for (size_t h = 0; h < sizeof(hiddens) / sizeof(hiddens[0]); ++h) {
                const int beta = flags & 1, bias = (flags >> 1) & 1, residual = (flags >> 2) & 1;
                const int bcast = (flags >> 3) & 1, simplified = (flags >> 4) & 1;
                skip_norm_case(dtype, 12, hiddens[h], bcast ? 4 : 0, beta, bias, residual, simplified,
                               dtype == F32 ? 1e-12f : 1e-5f);
            }
    skip_norm_case(F32, 5, 64, 0, 1, 1, 1, 0, 0.0f);

    /* BiasAdd */
    for (int dtype = F32; dtype <= F16; ++dtype) {
        const int64_t rows = 9, cols = 77;
        void* x = fill(dtype, rows * cols, -2.0f, 2.0f);
        void* s = fill(dtype, rows * cols, -2.0f, 2.0f);
        void* b = fill(dtype, cols, -1.0f, 1.0f);
        void* y = malloc((size_t)(rows * cols) * esize(dtype));
        double* ye = (double*)malloc((size_t)(rows * cols) * sizeof(double));
        CHECK(oracle_bias_add(x, b, s, dtype, rows, cols, y, ye) == 0, "bias_add");
        CHECK(oracle_bias_add(x, b, s, dtype, rows, cols, y, NULL) == 0, "bias_add without the exact sum");
        free(x), free(s), free(b), free(y), free(ye);
    }

    /* BiasSoftmax: exact, cyclic and grouped bias rows; special values */
    for (int dtype = F32; dtype <= F16; ++dtype) {
        softmax_case(dtype, 12, 77, 12, 0, 1);
        softmax_case(dtype, 12, 64, 4, 0, 0);
        softmax_case(dtype, 12, 64, 3, 1, 1);
        softmax_case(dtype, 8, 1, 1, 1, 0);
    }

    /* rejected arguments return an error without touching memory */
    {
        float one = 1.0f;
        double yd = 0.0;
        CHECK(oracle_skip_norm(&one, &one, 0, &one, NULL, NULL, F32, 1, 0, 0, 1e-5f, 0, NULL, &yd, NULL, NULL, 1) < 0,
              "hidden 0 rejected");
        CHECK(oracle_skip_norm(&one, &one, 0, &one, NULL, NULL, F32, 1, 1, 0, -1.0f, 0, NULL, &yd, NULL, NULL, 1) < 0,
              "negative eps rejected");
        CHECK(oracle_skip_norm(&one, &one, 0, &one, NULL, NULL, 7, 1, 1, 0, 1e-5f, 0, NULL, &yd, NULL, NULL, 1) < 0,
              "unknown type rejected");
        CHECK(oracle_skip_norm(NULL, NULL, 0, NULL, NULL, NULL, F32, 0, 1, 0, 1e-5f, 0, NULL, NULL, NULL, NULL, 1) == 0,
              "no rows is a no-op");
        CHECK(oracle_bias_add(&one, &one, &one, F32, 1, 0, &one, NULL) < 0, "bias_add hidden 0 rejected");
        CHECK(oracle_bias_softmax(&one, &one, F32, 4, 1, 3, 0, &yd) < 0, "bias rows not dividing rejected");
        CHECK(oracle_bias_softmax(&one, &one, F32, 0, 1, 0, 0, &yd) == 0, "empty softmax is a no-op");
    }

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle under sanitizers: all checks passed\n");
    return 0;
}
