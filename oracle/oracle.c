/*
 * Plain fp64 CPU oracle for the pipelined tiled GEMM and its grouped and broadcast forms.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file; only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark load it.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes, and from where:
 *   - The GEMM is the plain definition of the standard tiled matmul that the pages start
 *     from (How We Built TLX: "Introducing TLX", listing 1, the synchronous Triton loop):
 *     C[i][j] = sum over k of A[i][k] * B[k][j].  The pipelined version in listing 2 is said
 *     to keep the same computation and change only the orchestration ("Introducing TLX",
 *     the paragraph after listing 1), so the oracle never pipelines, tiles or reorders.
 *   - The grouped form is one such GEMM per expert over that expert's contiguous row range
 *     (How We Built TLX: "Case Study 3: Distributed Grouped GEMM for LLM Pretraining").
 *   - The broadcast form is the GEMM on the explicitly materialised row [Xu[idx[r]] | Xc[r]]
 *     (How We Built TLX: "Case Study 2: In-Kernel Broadcast Optimization for RecSys", where
 *     the kernel is said to perform this broadcast implicitly; the oracle performs it
 *     literally).
 *   - The weight gradient of the grouped form, dW_g = X_g^T . dY_g over each expert's rows,
 *     is the same definition with the sum running over the expert's rows (same case study;
 *     the gradient products of its pretraining use).
 *   - IKBO attention: each candidate's query attends to its user's keys and values, the
 *     attention form of the same broadcast (case study 2), as the textbook softmax attention.
 *   - Epilogue: optional per-column bias, then optional SiLU(v) = v / (1 + exp(-v)).
 *
 * Arithmetic: inputs are the same bfloat16 bit patterns the GPU receives, decoded exactly;
 * every product of two bfloat16 values is exact in double; sums run in double in ascending
 * k.  Outputs are the double values v; rounding to float32 or bfloat16 (nearest, ties to
 * even, directly from the double) is offered as separate functions.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared oracle.c -o liboracle.so -lm
 * Rows are independent and are spread over OpenMP threads; that does not change any sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_B_KN = 0, OR_B_NK = 1 };
enum { OR_EPI_NONE = 0, OR_EPI_BIAS = 1, OR_EPI_SILU = 2, OR_EPI_BIAS_SILU = 3 };
enum { OR_OK = 0, OR_BAD_ARG = 1, OR_BAD_OFFSETS = 2, OR_BAD_INDEX = 3, OR_NO_MEMORY = 4 };

/* ---- scalar helpers ------------------------------------------------------------------ */

static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* SiLU as its definition: v * sigmoid(v) = v / (1 + e^-v).  For v < -709 exp overflows to
 * +inf and the quotient is -0.0, which is the correctly signed limit. */
double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

static double apply_epilogue(double acc, int epi, const float* bias, int64_t j) {
    double v = acc;
    if (epi == OR_EPI_BIAS || epi == OR_EPI_BIAS_SILU) v += (double)bias[j];
    if (epi == OR_EPI_SILU || epi == OR_EPI_BIAS_SILU) v = oracle_silu(v);
    return v;
}

/* Round a double to the nearest bfloat16 (ties to even) in one step, without passing
 * through float32.  bfloat16 keeps 8 significant bits and float32's exponent range:
 * normal numbers below 2^e (with 2^(e-1) <= |v|) have spacing 2^(e-8); below 2^-126 the
 * spacing is fixed at 2^-133; results of magnitude 2^128 or more are infinite. */
uint16_t oracle_round_bf16(double v) {
    uint32_t u;
    float f;
    if (isnan(v)) return (uint16_t)0x7FC0;
    if (isinf(v)) return v > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
    double q;
    if (v == 0.0) {
        q = v;
    } else {
        int e;
        frexp(v, &e);                 /* |v| = m * 2^e, 0.5 <= m < 1 */
        int step_exp = e - 8;
        if (step_exp < -133) step_exp = -133;
        double step = ldexp(1.0, step_exp);
        q = nearbyint(v / step) * step; /* division by a power of two is exact */
        if (q == 0.0) q = copysign(0.0, v);
    }
    if (fabs(q) >= ldexp(1.0, 128)) return q > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
    f = (float)q;                     /* exact: q is a bfloat16 value */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_round_bf16_array(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(v[i]);
}

void oracle_round_f32_array(const double* v, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (float)v[i]; /* C conversion: nearest, ties even */
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- one output row of a plain GEMM --------------------------------------------------- */

/* out[j] = sum_k a[k] * B(k, j), ascending k, for j in [0, N).  `a` holds K decoded values. */
static void row_times_matrix(const double* a, int64_t N, int64_t K, const uint16_t* B,
                             int64_t ldb, int b_layout, double* out) {
    if (b_layout == OR_B_KN) {
        for (int64_t j = 0; j < N; ++j) out[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double ak = a[k];
            const uint16_t* brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) out[j] += ak * bf16_value(brow[j]);
        }
    } else {
        for (int64_t j = 0; j < N; ++j) {
            const uint16_t* bcol = B + j * ldb;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += a[k] * bf16_value(bcol[k]);
            out[j] = s;
        }
    }
}

static int check_common(int64_t M, int64_t N, int64_t K, int epi, int layout) {
    if (M < 0 || N < 0 || K < 0) return OR_BAD_ARG;
    if (epi < OR_EPI_NONE || epi > OR_EPI_BIAS_SILU) return OR_BAD_ARG;
    if (layout != OR_B_KN && layout != OR_B_NK) return OR_BAD_ARG;
    return OR_OK;
}

/* ---- gemm ------------------------------------------------------------------------------ *
 * out[t][j] = epi(sum_k A[r][k] * B(k, j) + bias[j]) for r = rows[t] (or r = t when rows is
 * NULL and nrows == M).  A is M x K with row stride lda; B is K x N (stride ldb) for layout
 * KN or N x K (stride ldb) for layout NK.  out is nrows x N, dense. */
int oracle_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                const uint16_t* B, int64_t ldb, int b_layout, const float* bias, int epi,
                const int64_t* rows, int64_t nrows, double* out) {
    int st = check_common(M, N, K, epi, b_layout);
    if (st) return st;
    if ((epi == OR_EPI_BIAS || epi == OR_EPI_BIAS_SILU) && !bias && N > 0) return OR_BAD_ARG;
    if (!rows && nrows != M) return OR_BAD_ARG;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= M) return OR_BAD_ARG;
    int failed = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!a || !acc) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            {
                const int64_t r = rows ? rows[t] : t;
                for (int64_t k = 0; k < K; ++k) a[k] = bf16_value(A[r * lda + k]);
                row_times_matrix(a, N, K, B, ldb, b_layout, acc);
                for (int64_t j = 0; j < N; ++j) out[t * N + j] = apply_epilogue(acc[j], epi, bias, j);
            }
        }
        free(a);
        free(acc);
    }
    return failed ? OR_NO_MEMORY : OR_OK;
}

/* ---- grouped gemm ---------------------------------------------------------------------- *
 * Group g owns rows [off[g], off[g+1]) of X and Y.  Requires off[0] = 0, off nondecreasing,
 * off[G] = M_total.  W holds G matrices back to back, each K x N (KN) or N x K (NK).
 * bias, when used, is G x N. */
int oracle_grouped_gemm(int32_t G, int64_t M_total, int64_t N, int64_t K, const uint16_t* X,
                        const uint16_t* W, int w_layout, const int32_t* off, const float* bias,
                        int epi, const int64_t* rows, int64_t nrows, double* out) {
    int st = check_common(M_total, N, K, epi, w_layout);
    if (st) return st;
    if (G <= 0 || !off) return OR_BAD_ARG;
    if ((epi == OR_EPI_BIAS || epi == OR_EPI_BIAS_SILU) && !bias && N > 0) return OR_BAD_ARG;
    if (off[0] != 0 || (int64_t)off[G] != M_total) return OR_BAD_OFFSETS;
    for (int32_t g = 0; g < G; ++g)
        if (off[g + 1] < off[g]) return OR_BAD_OFFSETS;
    if (!rows && nrows != M_total) return OR_BAD_ARG;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= M_total) return OR_BAD_ARG;
    const int64_t wsize = K * N;
    const int64_t ldw = (w_layout == OR_B_KN) ? N : K;
    int failed = 0;
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!a || !acc) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            {
                const int64_t r = rows ? rows[t] : t;
                int32_t g = 0; /* the one group whose (nonempty) range holds row r */
                while (!((int64_t)off[g] <= r && r < (int64_t)off[g + 1])) ++g;
                for (int64_t k = 0; k < K; ++k) a[k] = bf16_value(X[r * K + k]);
                row_times_matrix(a, N, K, W + (int64_t)g * wsize, ldw, w_layout, acc);
                const float* bg = bias ? bias + (int64_t)g * N : NULL;
                for (int64_t j = 0; j < N; ++j) out[t * N + j] = apply_epilogue(acc[j], epi, bg, j);
            }
        }
        free(a);
        free(acc);
    }
    return failed ? OR_NO_MEMORY : OR_OK;
}

/* ---- broadcast gemm -------------------------------------------------------------------- *
 * Row r of the (never shared) materialised input is z = [Xu[idx[r]] | Xc[r]], of width
 * Ku + Kc; Y[r] = epi(z . W + bias).  W is (Ku + Kc) x N (KN) or N x (Ku + Kc) (NK); rows
 * 0..Ku-1 of W (KN) meet the user features.  Requires 0 <= idx[r] < U. */
int oracle_broadcast_gemm(int64_t U, int64_t Mc, int64_t Ku, int64_t Kc, int64_t N,
                          const uint16_t* Xu, const uint16_t* Xc, const int32_t* idx,
                          const uint16_t* W, int w_layout, const float* bias, int epi,
                          const int64_t* rows, int64_t nrows, double* out) {
    const int64_t K = Ku + Kc;
    int st = check_common(Mc, N, K, epi, w_layout);
    if (st) return st;
    if (U < 0 || Ku < 0 || Kc < 0) return OR_BAD_ARG;
    if ((epi == OR_EPI_BIAS || epi == OR_EPI_BIAS_SILU) && !bias && N > 0) return OR_BAD_ARG;
    for (int64_t r = 0; r < Mc; ++r)
        if (idx[r] < 0 || (int64_t)idx[r] >= U) return OR_BAD_INDEX;
    if (!rows && nrows != Mc) return OR_BAD_ARG;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= Mc) return OR_BAD_ARG;
    const int64_t ldw = (w_layout == OR_B_KN) ? N : K;
    int failed = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!z || !acc) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            {
                const int64_t r = rows ? rows[t] : t;
                const int64_t u = idx[r];
                for (int64_t k = 0; k < Ku; ++k) z[k] = bf16_value(Xu[u * Ku + k]);
                for (int64_t k = 0; k < Kc; ++k) z[Ku + k] = bf16_value(Xc[r * Kc + k]);
                row_times_matrix(z, N, K, W, ldw, w_layout, acc);
                for (int64_t j = 0; j < N; ++j) out[t * N + j] = apply_epilogue(acc[j], epi, bias, j);
            }
        }
        free(z);
        free(acc);
    }
    return failed ? OR_NO_MEMORY : OR_OK;
}

/* ---- grouped weight gradient ----------------------------------------------------------- *
 * The backward pass of the expert GEMM Y_g = X_g . W_g with respect to the weights (How We
 * Built TLX: "Case Study 3: Distributed Grouped GEMM for LLM Pretraining" names the grouped
 * expert products of pretraining; their weight gradient is the textbook product below):
 *     dW[g][i][j] = sum over r in [off[g], off[g+1]) of X[r][i] * dY[r][j],
 * i.e. dW_g = X_g^T . dY_g, summed in ascending r.  A group with no rows has dW_g = 0.
 * X is M_total x K, dY is M_total x N (both dense row-major); dW is G x K x N.  Output rows
 * are selected by their flat index q = g * K + i in [0, G * K) (all of them, in order, when
 * rows is NULL and nrows == G * K); out is nrows x N, dense. */
int oracle_grouped_wgrad(int32_t G, int64_t M_total, int64_t K, int64_t N, const uint16_t* X,
                         const uint16_t* dY, const int32_t* off, const int64_t* rows,
                         int64_t nrows, double* out) {
    if (G <= 0 || M_total < 0 || K < 0 || N < 0 || !off) return OR_BAD_ARG;
    if (off[0] != 0 || (int64_t)off[G] != M_total) return OR_BAD_OFFSETS;
    for (int32_t g = 0; g < G; ++g)
        if (off[g + 1] < off[g]) return OR_BAD_OFFSETS;
    const int64_t total = (int64_t)G * K;
    if (!rows && nrows != total) return OR_BAD_ARG;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= total) return OR_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < nrows; ++t) {
        const int64_t q = rows ? rows[t] : t;
        const int64_t g = q / K, i = q % K;
        double* acc = out + t * N;
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t r = off[g]; r < (int64_t)off[g + 1]; ++r) {
            const double x = bf16_value(X[r * K + i]);
            const uint16_t* dyrow = dY + r * N;
            for (int64_t j = 0; j < N; ++j) acc[j] += x * bf16_value(dyrow[j]);
        }
    }
    return OR_OK;
}

/* ---- IKBO attention --------------------------------------------------------------------- *
 * The attention form of the in-kernel broadcast (How We Built TLX: "Case Study 2: In-Kernel
 * Broadcast Optimization for RecSys" states that for FlashAttention the co-design amortises
 * the K/V reads across the candidates sharing one user context).  Candidates are contiguous
 * by user: user u owns candidates [off[u], off[u+1]).  For candidate c of user u and head h:
 *     s_j = scale * sum_e Q[c][h][e] * K[u][j][h][e]          (j = 0 .. L-1)
 *     p_j = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)
 *     O[c][h][e] = sum_j p_j * V[u][j][h][e]
 * Q and O are [Mc][H][D], K and V are [U][L][H][D] (all dense).  Every sum runs in double in
 * ascending index order.  Output rows are selected by candidate index (all of them when rows is
 * NULL and nrows == Mc); out is nrows x H x D. */
int oracle_ikbo_attention(int64_t U, int64_t Mc, int64_t H, int64_t D, int64_t L, double scale,
                          const int32_t* off, const uint16_t* Q, const uint16_t* K,
                          const uint16_t* V, const int64_t* rows, int64_t nrows, double* out) {
    if (U <= 0 || Mc < 0 || H <= 0 || D <= 0 || L <= 0 || !off) return OR_BAD_ARG;
    if (off[0] != 0 || (int64_t)off[U] != Mc) return OR_BAD_OFFSETS;
    for (int64_t u = 0; u < U; ++u)
        if (off[u + 1] < off[u]) return OR_BAD_OFFSETS;
    if (!rows && nrows != Mc) return OR_BAD_ARG;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= Mc) return OR_BAD_ARG;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        double* q = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!s || !q) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            const int64_t c = rows ? rows[t] : t;
            int64_t u = 0; /* the user whose (nonempty) range holds candidate c */
            while (!((int64_t)off[u] <= c && c < (int64_t)off[u + 1])) ++u;
            for (int64_t h = 0; h < H; ++h) {
                for (int64_t e = 0; e < D; ++e) q[e] = bf16_value(Q[(c * H + h) * D + e]);
                double mx = -INFINITY;
                for (int64_t j = 0; j < L; ++j) {
                    const uint16_t* kr = K + ((u * L + j) * H + h) * D;
                    double acc = 0.0;
                    for (int64_t e = 0; e < D; ++e) acc += q[e] * bf16_value(kr[e]);
                    s[j] = scale * acc;
                    if (s[j] > mx) mx = s[j];
                }
                double den = 0.0;
                for (int64_t j = 0; j < L; ++j) {
                    s[j] = exp(s[j] - mx);
                    den += s[j];
                }
                double* o = out + (t * H + h) * D;
                for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
                for (int64_t j = 0; j < L; ++j) {
                    const uint16_t* vr = V + ((u * L + j) * H + h) * D;
                    const double p = s[j] / den;
                    for (int64_t e = 0; e < D; ++e) o[e] += p * bf16_value(vr[e]);
                }
            }
        }
        free(s);
        free(q);
    }
    return failed ? OR_NO_MEMORY : OR_OK;
}
