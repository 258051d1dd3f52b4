/*
 * moe_ref.c - a second CPU implementation of the routed-MoE layer, in plain C
 * (TEST INFRASTRUCTURE).  Only the tests, the smoke entry and the benchmark's
 * CPU-baseline leg load it; the product path never does.  It shares no code
 * with the NumPy oracle (moe_oracle.py) or with the HIP library: it is
 * written again from the same definitions so that the two CPU
 * implementations can be checked against each other on small layers, and it
 * is the oracle the benchmark times on the host's cores (OpenMP over output
 * rows and router rows; no -ffast-math).
 *
 * What it computes (pages cited by title and section):
 *   - Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना", section "implemented
 *     features": the DeepSeek-V3-style sigmoid router with the noaux_tc
 *     correction, routed_scaling_factor and the shared expert; row-scaled
 *     int8 / packed int4 / packed int2 weights dequantised on use.
 *   - ideipro.ru, "Энтузиаст запустил GLM-5.2 на ноутбуке с 25 ГБ RAM": 8
 *     experts per token per layer.
 * The points the pages leave open take the same readings as the NumPy
 * oracle: a group scores the sum of its two largest corrected scores; the
 * corrected scores c = s + b select, the sigmoid scores s weigh; ties go to
 * the lower index; a NaN corrected or group score ranks as -inf; w_k =
 * s_k / (sum of the chosen s in slot order) * rsf; shared experts weigh 1;
 * experts are SwiGLU without biases; codes are two's complement, column c of
 * a row in field c % (8/bits) of byte c / (8/bits), lowest field first; one
 * scale per output row.
 *
 * Precision: the router dot products and every expert product in double
 * (each weight = code * scale, exact in double); the routing decisions in
 * float (the scores rounded once to float), as the GPU takes them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_OK 0
#define REF_ERR_ARG 1
#define REF_ERR_MISSING_EXPERT 2

/* Code of column c of a packed row (two's complement, sign-extended). */
static int code_at(const uint8_t* row, int c, int bits) {
    const int per = 8 / bits;
    const int field = (row[c / per] >> ((c % per) * bits)) & ((1 << bits) - 1);
    return field >= (1 << (bits - 1)) ? field - (1 << bits) : field;
}

/* Dequantised row: out[c] = code * scale, in double. */
static void dequant_row(const uint8_t* row, float scale, int n, int bits, double* out) {
    for (int c = 0; c < n; ++c) out[c] = (double)code_at(row, c, bits) * (double)scale;
}

/* Rank keys: a larger value first; NaN counts as -inf; equal values by index. */
static float rank_value(float v) { return isnan(v) ? -INFINITY : v; }

static int before(float va, int ia, float vb, int ib) {
    va = rank_value(va);
    vb = rank_value(vb);
    if (va != vb) return va > vb;
    return ia < ib;
}

/*
 * Routing of one token from its float scores s[E] and the bias b[E]:
 * chosen[K] in slot order and their weights.
 */
static void route_token(const float* s, const float* b, int E, int n_group, int topk_group, int top_k, float rsf,
                        int32_t* chosen, float* weight) {
    const int per = E / n_group;
    float* c = (float*)malloc(sizeof(float) * (size_t)E);
    float* gs = (float*)malloc(sizeof(float) * (size_t)n_group);
    int* kept = (int*)malloc(sizeof(int) * (size_t)n_group);
    for (int e = 0; e < E; ++e) c[e] = rank_value(s[e] + b[e]);
    for (int g = 0; g < n_group; ++g) {
        /* two largest values of the group by the rank order */
        int i1 = -1, i2 = -1;
        for (int e = g * per; e < (g + 1) * per; ++e) {
            if (i1 < 0 || before(c[e], e, c[i1], i1)) {
                i2 = i1;
                i1 = e;
            } else if (i2 < 0 || before(c[e], e, c[i2], i2)) {
                i2 = e;
            }
        }
        gs[g] = rank_value(c[i1] + c[i2]);
    }
    /* keep the topk_group best groups: selection by repeated best-remaining */
    for (int g = 0; g < n_group; ++g) kept[g] = 0;
    for (int r = 0; r < topk_group; ++r) {
        int best = -1;
        for (int g = 0; g < n_group; ++g)
            if (!kept[g] && (best < 0 || before(gs[g], g, gs[best], best))) best = g;
        kept[best] = 1;
    }
    /* the top_k best experts of the kept groups, best first */
    char* taken = (char*)calloc((size_t)E, 1);
    for (int k = 0; k < top_k; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (!kept[e / per] || taken[e]) continue;
            if (best < 0 || before(c[e], e, c[best], best)) best = e;
        }
        taken[best] = 1;
        chosen[k] = best;
    }
    float total = 0.0f;
    for (int k = 0; k < top_k; ++k) total = total + s[chosen[k]];
    for (int k = 0; k < top_k; ++k) {
        const float q = s[chosen[k]] / total;
        weight[k] = q * rsf;
    }
    free(taken);
    free(kept);
    free(gs);
    free(c);
}

/*
 * One layer on T tokens.
 *   x        : float [T][H]
 *   router_w : float [E][H];  bias : float [E]
 *   q_gate[e], q_up[e] : packed codes [I][H*bits/8] of expert e (e < E + S);
 *   q_down[e]          : packed codes [H][I*bits/8];
 *   s_gate[e], s_up[e] : float [I];  s_down[e] : float [H]
 *   (the pointers of experts no token selects may be NULL)
 * Outputs:
 *   scores64 : double [T][E]   sigmoid scores
 *   idx      : int32 [T][K]    chosen experts in slot order
 *   w        : float [T][K]    their weights
 *   h        : double [T*(K+S)][I]  h of assignment t*(K+S)+slot
 *   y        : double [T][H]
 * Returns REF_OK, REF_ERR_ARG, or REF_ERR_MISSING_EXPERT (a selected expert's
 * pointers are NULL).
 */
int moe_ref_layer(const float* x, int T, int H, int I, int E, int n_group, int topk_group, int top_k, int n_shared,
                  float rsf, int bits, const float* router_w, const float* bias, const uint8_t* const* q_gate,
                  const uint8_t* const* q_up, const uint8_t* const* q_down, const float* const* s_gate,
                  const float* const* s_up, const float* const* s_down, int nthreads, double* scores64,
                  int32_t* idx, float* w, double* h, double* y) {
    if (T < 1 || H < 1 || I < 1 || E < 2 || n_group < 1 || E % n_group || E / n_group < 2) return REF_ERR_ARG;
    if (topk_group < 1 || topk_group > n_group || top_k < 1 || top_k > topk_group * (E / n_group)) return REF_ERR_ARG;
    if (n_shared < 0 || (bits != 8 && bits != 4 && bits != 2) || H % (8 / bits) || I % (8 / bits)) return REF_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
#ifdef _OPENMP
    omp_set_num_threads(nthreads);
#endif
    const int slots = top_k + n_shared;

    /* router: sigmoid of the fp64 dot products, one row per expert */
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
        for (int t = 0; t < T; ++t) {
            double z = 0.0;
            for (int k = 0; k < H; ++k) z += (double)router_w[(size_t)e * H + k] * (double)x[(size_t)t * H + k];
            scores64[(size_t)t * E + e] = 1.0 / (1.0 + exp(-z));
        }
    }
    float* s32 = (float*)malloc(sizeof(float) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) s32[e] = (float)scores64[(size_t)t * E + e];
        route_token(s32, bias, E, n_group, topk_group, top_k, rsf, idx + (size_t)t * top_k, w + (size_t)t * top_k);
    }
    free(s32);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < slots; ++k) {
            const int e = k < top_k ? idx[(size_t)t * top_k + k] : E + (k - top_k);
            if (!q_gate[e] || !q_up[e] || !q_down[e] || !s_gate[e] || !s_up[e] || !s_down[e])
                return REF_ERR_MISSING_EXPERT;
        }

    /* experts: every (token, slot) in turn, the products row by row */
    memset(y, 0, sizeof(double) * (size_t)T * H);
    const size_t rbg = (size_t)H * bits / 8, rbd = (size_t)I * bits / 8;
    for (int t = 0; t < T; ++t) {
        const float* xt = x + (size_t)t * H;
        for (int k = 0; k < slots; ++k) {
            const int e = k < top_k ? idx[(size_t)t * top_k + k] : E + (k - top_k);
            const double coef = k < top_k ? (double)w[(size_t)t * top_k + k] : 1.0;
            double* ha = h + ((size_t)t * slots + k) * I;
#pragma omp parallel
            {
                double* row = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
#pragma omp for schedule(static)
                for (int i = 0; i < I; ++i) {
                    double g = 0.0, v = 0.0;
                    dequant_row(q_gate[e] + (size_t)i * rbg, s_gate[e][i], H, bits, row);
                    for (int c = 0; c < H; ++c) g += row[c] * (double)xt[c];
                    dequant_row(q_up[e] + (size_t)i * rbg, s_up[e][i], H, bits, row);
                    for (int c = 0; c < H; ++c) v += row[c] * (double)xt[c];
                    ha[i] = g / (1.0 + exp(-g)) * v;
                }
#pragma omp for schedule(static)
                for (int r = 0; r < H; ++r) {
                    double o = 0.0;
                    dequant_row(q_down[e] + (size_t)r * rbd, s_down[e][r], I, bits, row);
                    for (int i = 0; i < I; ++i) o += row[i] * ha[i];
                    y[(size_t)t * H + r] += coef * o;
                }
                free(row);
            }
        }
    }
    return REF_OK;
}

/* Threads the OpenMP runtime would use by default (the host's cores). */
int moe_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
