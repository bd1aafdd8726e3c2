/* Drives every entry point of oracle/fp8_oracle.c on small inputs, for a
 * build under AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure; see tests/test_oracle_sanitize.py).  Every buffer is
 * allocated at exactly the size the call may touch: a strided matrix ends
 * with its last row's last element, not at rows * ld.  Inputs mix normal
 * values with NaN, +-Inf, zeros and subnormals, and the KV calls use slots
 * outside the cache.  Exit status 0 means every call returned; the
 * sanitizers abort on the first report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* entry points (oracle/fp8_oracle.c has no header of its own) */
double or_decode(int fmt, uint8_t code);
void or_decode_table(int fmt, double* out256);
double or_format_max(int fmt);
uint8_t or_encode(int fmt, float v);
void or_encode_array(int fmt, const float* v, int64_t n, uint8_t* out);
int64_t or_num_groups(int gran, int64_t rows, int64_t cols);
void or_amax(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, int gran, float* amax_out);
void or_scale(float amax, int fmt, int pow2, float* s_out, float* s_inv_out);
void or_quantize_with_scales(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, int gran,
                             int fmt, const float* scales, uint8_t* q, int64_t ldq, int64_t* counts3);
void or_quantize(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, int gran, int fmt,
                 int pow2, uint8_t* q, int64_t ldq, float* amax_out, float* scale_out, float* scale_inv_out,
                 int64_t* counts3);
typedef struct {
    float amax[16];
    int32_t len, pos, count;
} or_ring;
void or_ring_init(or_ring* r, int32_t len);
float or_ring_window_max(const or_ring* r);
void or_delayed_step(or_ring* r, const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld, int fmt,
                     uint8_t* q, int64_t ldq, float spike_threshold, float* out4, int64_t* counts3);
void or_gemm_sampled(const uint8_t* A, int fa, int64_t lda, const uint8_t* B, int fb, int64_t ldb, int64_t K,
                     const float* a_inv, int a_per_row, const float* b_inv, int b_per_row, const int64_t* ms,
                     const int64_t* ns, int64_t n, float* y32, double* p64);
void or_gemm(const uint8_t* A, int fa, int64_t lda, const uint8_t* B, int fb, int64_t ldb, int64_t M, int64_t N,
             int64_t K, const float* a_inv, int a_per_row, const float* b_inv, int b_per_row, float* Y32,
             int64_t ldy, double* P, int64_t ldp);
void or_blockgemm_sampled(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t K,
                          const float* a_inv, const float* b_inv, const int64_t* ms, const int64_t* ns, int64_t n,
                          float* y32, double* p64);
void or_blockgemm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M, int64_t N, int64_t K,
                  const float* a_inv, const float* b_inv, float* Y32, int64_t ldy, double* P, int64_t ldp);
void or_gemm_exact_sampled(const uint8_t* A, int fa, int64_t lda, const uint8_t* B, int fb, int64_t ldb,
                           int64_t K, const float* a_inv, int a_per_row, const float* b_inv, int b_per_row,
                           int block_mode, const int64_t* ms, const int64_t* ns, int64_t n, double* y_exact);
uint16_t or_f32_to_bf16(float v);
void or_f32_to_bf16_array(const float* v, int64_t n, uint16_t* out);
void or_kv_store(const void* x, int in_dtype, int64_t n, int64_t heads, int64_t head_dim, int64_t ld,
                 const int64_t* slots, int64_t capacity, int storage, int scaling, int pow2, void* cache,
                 float* scale_inv, int64_t* counts3);
void or_kv_load(const void* cache, int storage, int scaling, const float* scale_inv, int64_t n, int64_t heads,
                int64_t head_dim, const int64_t* slots, int64_t capacity, int out_bf16, void* out, int64_t ld_out);
int or_num_threads(void);
void or_set_num_threads(int n);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {           /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float next_value(void) {
    uint64_t r = next_u64();
    switch (r % 16) {
        case 0: return NAN;
        case 1: return (r & 16) ? INFINITY : -INFINITY;
        case 2: return (r & 16) ? 0.0f : -0.0f;
        case 3: return ldexpf((float)(r >> 40) / 16777216.0f, -140);     /* subnormal */
        case 4: return ldexpf((float)((int64_t)(r >> 40) - (1 << 23)), 20);  /* far past fmax */
        default: return ((float)(int64_t)(r >> 40) / 16777216.0f - 0.5f) * 40.0f;
    }
}
static void* exact_alloc(size_t bytes) { return malloc(bytes ? bytes : 1); }
static uint8_t finite_code(int fmt) {      /* a random finite code */
    for (;;) {
        uint8_t c = (uint8_t)next_u64();
        if (isfinite(or_decode(fmt, c))) return c;
    }
}

static void quantize_cases(int64_t rows, int64_t cols, int64_t ld) {
    const int64_t n_in = rows ? (rows - 1) * ld + cols : 0;
    float* xf = exact_alloc((size_t)n_in * 4);
    uint16_t* xb = exact_alloc((size_t)n_in * 2);
    for (int64_t i = 0; i < n_in; ++i) xf[i] = next_value();
    or_f32_to_bf16_array(xf, n_in, xb);
    for (int dt = 0; dt < 2; ++dt) {
        const void* x = dt == 0 ? (const void*)xf : (const void*)xb;
        for (int gran = 0; gran < 4; ++gran)
            for (int fmt = 0; fmt < 2; ++fmt) {
                const int64_t ng = or_num_groups(gran, rows, cols);
                const int64_t ldq = cols + (gran & 1);
                const int64_t n_q = rows ? (rows - 1) * ldq + cols : 0;
                uint8_t* q = exact_alloc((size_t)n_q);
                float* am = exact_alloc((size_t)ng * 4);
                float* s = exact_alloc((size_t)ng * 4);
                float* si = exact_alloc((size_t)ng * 4);
                int64_t c3[3];
                or_amax(x, dt, rows, cols, ld, gran, am);
                or_quantize(x, dt, rows, cols, ld, gran, fmt, gran == 1, q, ldq, am, s, si, c3);
                or_quantize_with_scales(x, dt, rows, cols, ld, gran, fmt, s, q, ldq, c3);
                free(q); free(am); free(s); free(si);
            }
        /* delayed scaling: 20 steps on a ring of 16 (and one of 3), guard on */
        for (int len = 3; len <= 16; len += 13) {
            or_ring r;
            or_ring_init(&r, len);
            uint8_t* q = exact_alloc((size_t)n_in);
            for (int step = 0; step < 20; ++step) {
                float out4[4];
                int64_t c3[3];
                or_delayed_step(&r, x, dt, rows, cols, ld, step & 1, q, ld, step > 5 ? 4.0f : 0.0f, out4, c3);
                (void)or_ring_window_max(&r);
            }
            free(q);
        }
    }
    free(xf); free(xb);
}

static void gemm_cases(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    for (int fa = 0; fa < 2; ++fa)
        for (int fb = 0; fb < 2; ++fb) {
            const int64_t na = M ? (M - 1) * lda + K : 0, nb = N ? (N - 1) * ldb + K : 0;
            uint8_t* A = exact_alloc((size_t)na);
            uint8_t* B = exact_alloc((size_t)nb);
            for (int64_t i = 0; i < na; ++i) A[i] = finite_code(fa);
            for (int64_t i = 0; i < nb; ++i) B[i] = finite_code(fb);
            float* sa = exact_alloc((size_t)M * 4);
            float* sb = exact_alloc((size_t)N * 4);
            for (int64_t i = 0; i < M; ++i) sa[i] = ldexpf(1.0f, (int)(next_u64() % 9) - 4);
            for (int64_t i = 0; i < N; ++i) sb[i] = ldexpf(1.0f, (int)(next_u64() % 9) - 4);
            const int64_t ldy = N + 1;
            float* Y = exact_alloc((size_t)(M ? (M - 1) * ldy + N : 0) * 4);
            double* P = exact_alloc((size_t)(M ? (M - 1) * ldy + N : 0) * 8);
            or_gemm(A, fa, lda, B, fb, ldb, M, N, K, sa, 1, sb, 0, Y, ldy, P, ldy);
            const int64_t ns_ = 37;
            int64_t* ms = exact_alloc(ns_ * 8);
            int64_t* nsv = exact_alloc(ns_ * 8);
            for (int64_t i = 0; i < ns_; ++i) {
                ms[i] = (int64_t)(next_u64() % (uint64_t)M);
                nsv[i] = (int64_t)(next_u64() % (uint64_t)N);
            }
            float* y = exact_alloc(ns_ * 4);
            double* p = exact_alloc(ns_ * 8);
            double* ye = exact_alloc(ns_ * 8);
            or_gemm_sampled(A, fa, lda, B, fb, ldb, K, sa, 0, sb, 1, ms, nsv, ns_, y, p);
            or_gemm_exact_sampled(A, fa, lda, B, fb, ldb, K, sa, 1, sb, 1, 0, ms, nsv, ns_, ye);
            if (fa == 0 && fb == 0 && K % 128 == 0) {
                const int64_t kb = K / 128, nblk = (N + 127) / 128;
                float* ba = exact_alloc((size_t)(M * kb) * 4);
                float* bb = exact_alloc((size_t)(nblk * kb) * 4);
                for (int64_t i = 0; i < M * kb; ++i) ba[i] = ldexpf(1.0f, (int)(next_u64() % 5) - 2);
                for (int64_t i = 0; i < nblk * kb; ++i) bb[i] = ldexpf(1.0f, (int)(next_u64() % 5) - 2);
                or_blockgemm_sampled(A, lda, B, ldb, K, ba, bb, ms, nsv, ns_, y, p);
                or_blockgemm(A, lda, B, ldb, M, N, K, ba, bb, Y, ldy, P, ldy);
                or_gemm_exact_sampled(A, 0, lda, B, 0, ldb, K, ba, 1, bb, 1, 1, ms, nsv, ns_, ye);
                free(ba); free(bb);
            }
            free(A); free(B); free(sa); free(sb); free(Y); free(P); free(ms); free(nsv); free(y); free(p); free(ye);
        }
}

static void kv_cases(int64_t n, int64_t heads, int64_t head_dim, int64_t capacity) {
    const int64_t ld = heads * head_dim + 3;
    const int64_t n_in = (n - 1) * ld + heads * head_dim;
    float* xf = exact_alloc((size_t)n_in * 4);
    for (int64_t i = 0; i < n_in; ++i) xf[i] = next_value();
    int64_t* slots = exact_alloc((size_t)n * 8);
    for (int64_t t = 0; t < n; ++t)
        slots[t] = (t % 5 == 4) ? capacity + t : (t % 7 == 6 ? -1 : (t * 3) % capacity);
    for (int storage = 0; storage < 3; ++storage)
        for (int scaling = 0; scaling < 2; ++scaling) {
            const size_t esz = storage == 2 ? 2 : 1;
            void* cache = exact_alloc((size_t)(capacity * heads * head_dim) * esz);
            memset(cache, 0, (size_t)(capacity * heads * head_dim) * esz);
            const int64_t nsc = scaling == 0 ? capacity * heads : heads;
            float* sinv = exact_alloc((size_t)nsc * 4);
            for (int64_t i = 0; i < nsc; ++i) sinv[i] = 0.25f;
            int64_t c3[3];
            or_kv_store(xf, 0, n, heads, head_dim, ld, slots, capacity, storage, scaling, scaling == 0, cache,
                        sinv, c3);
            const int64_t ldo = heads * head_dim + 1;
            for (int ob = 0; ob < 2; ++ob) {
                void* out = exact_alloc((size_t)((n - 1) * ldo + heads * head_dim) * (ob ? 2 : 4));
                or_kv_load(cache, storage, scaling, sinv, n, heads, head_dim, slots, capacity, ob, out, ldo);
                free(out);
            }
            free(cache); free(sinv);
        }
    free(xf); free(slots);
}

int main(void) {
    double t[256];
    for (int fmt = 0; fmt < 2; ++fmt) {
        or_decode_table(fmt, t);
        (void)or_format_max(fmt);
        for (int c = 0; c < 256; ++c) (void)or_encode(fmt, (float)t[c]);
        float v[1000];
        uint8_t out[1000];
        for (int i = 0; i < 1000; ++i) v[i] = next_value();
        or_encode_array(fmt, v, 1000, out);
        for (int i = 0; i < 1000; ++i) {
            float s, si;
            or_scale(v[i], fmt, i & 1, &s, &si);
            (void)or_f32_to_bf16(v[i]);
        }
    }
    or_set_num_threads(2);
    (void)or_num_threads();
    static const int64_t shapes[][3] = {{1, 1, 1}, {3, 130, 131}, {129, 257, 260}, {200, 64, 64}, {0, 5, 5}};
    for (unsigned i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        quantize_cases(shapes[i][0], shapes[i][1], shapes[i][2]);
    gemm_cases(1, 1, 16, 16, 16);
    gemm_cases(37, 45, 80, 83, 81);
    gemm_cases(130, 140, 256, 256, 260);
    kv_cases(11, 3, 40, 9);
    kv_cases(1, 1, 8, 1);
    printf("oracle sanitize driver: ok\n");
    return 0;
}
