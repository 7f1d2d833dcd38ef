/*
 * gdn_oracle.c -- CPU oracle for the gated delta rule with dynamic per-tile
 * FP8-E4M3 fake quantize-dequantize (QDQ) of the recurrent state.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product (the HIP
 * library) never calls, links or includes anything from here, and nothing
 * here is shared with it.
 *
 * What it computes (plain definitions, written out token by token):
 *
 *  - Gated delta rule recurrence, the "recurrent updates" of Gated DeltaNet
 *    that the pages build their state QAT on (#2519 page, "What does this PR
 *    do?", step 2-3; #2506 page "Additional Information" on the recurrent
 *    inference mode).  For one sequence and one head, with state S (dv x dk,
 *    row = value channel, column = key channel):
 *        decay      S <- a_t * S              a_t = exp(g_t)   (scalar gate)
 *                   S <- S * diag(exp(g_t))                     (per-key-channel
 *                   gate, "per-key-channel retention", #2506 page)
 *        delta      u = beta_t * (v_t - S k_t);  S <- S + u k_t^T
 *        output     o_t = S q_t
 *    which is S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 *    All of it in fp64.
 *
 *  - State QDQ (#2497 page "What does this PR do?": dynamic FP8 E4M3, one
 *    scalar scale amax/448 with a zero guard per full-key x 64-value-column
 *    tile, recomputed at every boundary independently per sequence and head).
 *    The method keeps its state in fp32 storage, so the quantization decision
 *    is taken in fp32: the state is stored to fp32, amax is the largest |x| of
 *    the tile, s = amax / 448 (IEEE fp32 division; s = 1 when that is not
 *    positive -- the zero guard), y = x / s (IEEE fp32 division), the code is
 *    y rounded to the nearest E4M3FN value with ties to the even code, and the
 *    stored value is code * s rounded to fp32.  Only the E4M3 rounding itself
 *    is a search over the grid, written out below from the format definition.
 *
 *  - QDQ placement (#2497 page: 64-token chunks, QDQ at each boundary; #2519
 *    page step 3: QDQ at the prefill->decode handoff and after every later
 *    recurrent write, output taken from the working state before the QDQ).
 *    With prefix length P and valid length L (1 <= t <= L):
 *        ORC_QDQ_CHUNK : QDQ after token t when t <= P and (t % 64 == 0 or t == P)
 *        ORC_QDQ_WRITE : QDQ after token t when t >= max(P, 1)
 *    A token that satisfies both is quantized once.  A supplied initial state
 *    is used as given.
 *
 *  - Log-retention grid (#2509 page "What does this PR do?": an optional
 *    rounding of the log-retention among the per-token decode policies; its
 *    pilot selected a grid of 1/256).  The page gives no formula; this
 *    oracle's reading: with grid_log2 = k > 0 every recurrent write (token
 *    t > P) decays with g rounded to the nearest multiple of 2^-k, ties to
 *    even (per key channel for the per-channel gate); the chunked prefix
 *    t <= P is unchanged.
 *
 *  - INT8 block-32 state QDQ (#2519 page: dynamic INT8 state recipes, one of
 *    them with 32-element blocks; the page gives no formula, so what follows
 *    is this oracle's reading): with ORC_QDQ_INT8 every QDQ of the state
 *    quantizes each block of 32 consecutive key columns of a state row on
 *    its own: s = amax / 127 (IEEE fp32; s = 1 when that is not positive),
 *    code = x / s (IEEE fp32 division) rounded half to even, clamped to
 *    [-127, 127], stored value code * s in fp32.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off (no fast-math), so
 * float expressions are evaluated in IEEE binary32 and double ones in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_QDQ_CHUNK 1u
#define ORC_QDQ_WRITE 2u
#define ORC_QDQ_INT8 8u
#define ORC_INT8_BLOCK 32
#define ORC_CHUNK 64
#define ORC_TILE_ROWS 64

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.  No      */
/* infinities; S.1111.111 is NaN; largest finite magnitude 448 (S.1111.110); */
/* subnormals m/8 * 2^-6.                                                    */
/* ------------------------------------------------------------------------ */

double orc_e4m3_decode(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Magnitudes of codes 0x00..0x7E; increasing with the code. */
static double g_grid[127];
static int g_grid_ready = 0;

static void grid_init(void)
{
    if (g_grid_ready) return;
    for (int c = 0; c < 127; ++c) g_grid[c] = orc_e4m3_decode(c);
    g_grid_ready = 1;
}

/* Nearest E4M3FN code to y (an fp32 value).  Ties go to the code with an
 * even mantissa LSB.  Magnitudes at or above 448 saturate to 448.  NaN maps to
 * the NaN code.  Bisection finds the two grid neighbours, then the distances
 * decide; at an exact midpoint both differences are exact in fp64. */
int orc_e4m3_encode(float yf)
{
    grid_init();
    double y = (double)yf;
    if (isnan(y)) return 0x7F;
    int sign = signbit(y) ? 0x80 : 0;
    double a = fabs(y);
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 126;               /* grid[lo] <= a < grid[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_grid[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - g_grid[lo], dhi = g_grid[hi] - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo & 1) == 0 ? lo : hi;
    return sign | c;
}

/* The same rounding by exhaustive search over every finite code, used by the
 * tests to pin the bisection above. */
int orc_e4m3_encode_bruteforce(float yf)
{
    double y = (double)yf;
    if (isnan(y)) return 0x7F;
    int sign = signbit(y) ? 0x80 : 0;
    double a = fabs(y);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 127; ++c) {
        double d = fabs(a - orc_e4m3_decode(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return sign | best;
}

void orc_e4m3_encode_array(const float* y, int64_t n, uint8_t* codes)
{
    for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_encode(y[i]);
}

/* QDQ of one tile of n fp32 values (decision in fp32, see header).
 * out may alias x.  scale and codes may be NULL. */
void orc_qdq_tile_f32(const float* x, int64_t n, float* out, float* scale, uint8_t* codes)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float ax = fabsf(x[i]);
        if (ax > amax) amax = ax;
    }
    float s = amax / 448.0f;
    if (!(s > 0.0f)) s = 1.0f;
    for (int64_t i = 0; i < n; ++i) {
        float y = x[i] / s;
        int c = orc_e4m3_encode(y);
        float cv = (float)orc_e4m3_decode(c);
        if (codes) codes[i] = (uint8_t)c;
        out[i] = cv * s;
    }
    if (scale) *scale = s;
}

/* QDQ of n_rows rows of row_len fp32 values, each row one group with its
 * own scale: the per-(token, head) grouping of the W quantizer (#2497 page,
 * Usage: the W quantizer keeps axes (0, 1, 2) of W [batch, token, head, key],
 * so its amax runs over the key axis alone).  scales: [n_rows] or NULL. */
void orc_qdq_rows_f32(const float* x, int64_t n_rows, int row_len,
                      float* out, float* scales, uint8_t* codes)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t off = r * row_len;
        orc_qdq_tile_f32(x + off, row_len, out + off, scales ? scales + r : NULL,
                         codes ? codes + off : NULL);
    }
}

/* Round half to even of an fp32 value to an integral value (|y| < 2^22),
 * from the definition: the nearer integer, the even one on a tie; a zero
 * result keeps the operand's sign (IEEE 754 roundToIntegralTiesToEven). */
static float round_half_even(float y)
{
    float f = floorf(y);
    float d = y - f;                 /* exact: y and f share the binade's ulp */
    float r;
    if (d > 0.5f) r = f + 1.0f;
    else if (d < 0.5f) r = f;
    else r = (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
    return copysignf(r, y);
}

/* INT8 QDQ of n_blocks blocks of `block` consecutive fp32 values, each block
 * one group (reading above).  out may alias x; scales [n_blocks] and codes
 * may be NULL. */
void orc_qdq_int8_blocks_f32(const float* x, int64_t n_blocks, int block, float* out,
                             float* scales, int8_t* codes)
{
    for (int64_t b = 0; b < n_blocks; ++b) {
        const float* xb = x + b * block;
        float* ob = out + b * block;
        float amax = 0.0f;
        for (int i = 0; i < block; ++i) {
            float ax = fabsf(xb[i]);
            if (ax > amax) amax = ax;
        }
        float s = amax / 127.0f;
        if (!(s > 0.0f)) s = 1.0f;
        for (int i = 0; i < block; ++i) {
            float c = round_half_even(xb[i] / s);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            if (codes) codes[b * block + i] = (int8_t)c;
            ob[i] = c * s;
        }
        if (scales) scales[b] = s;
    }
}

/* QDQ of n_states states of dv x dk fp32 values, one tile per 64 rows
 * (rows = value channels).  scales: [n_states][dv/64] or NULL. */
void orc_qdq_states_f32(const float* x, int64_t n_states, int dv, int dk,
                        float* out, float* scales, uint8_t* codes)
{
    int tiles = dv / ORC_TILE_ROWS;
    int64_t tile_elems = (int64_t)ORC_TILE_ROWS * dk;
    for (int64_t s = 0; s < n_states; ++s)
        for (int j = 0; j < tiles; ++j) {
            int64_t off = (s * tiles + j) * tile_elems;
            orc_qdq_tile_f32(x + off, tile_elems, out + off,
                             scales ? scales + s * tiles + j : NULL,
                             codes ? codes + off : NULL);
        }
}

/* QDQ of an fp64 state: stored to fp32 first, then quantized; the result is
 * written back widened to fp64.  scales: [dv/64] or NULL. */
static void qdq_state_f64(double* S, int dv, int dk, float* tmp, float* scales)
{
    int64_t n = (int64_t)dv * dk;
    for (int64_t i = 0; i < n; ++i) tmp[i] = (float)S[i];
    orc_qdq_states_f32(tmp, 1, dv, dk, tmp, scales, NULL);
    for (int64_t i = 0; i < n; ++i) S[i] = (double)tmp[i];
}

/* Log-gate on the grid 2^-k: the nearest multiple, ties to even (k = 0: g). */
double orc_grid_gate(double g, int k)
{
    if (k <= 0) return g;
    return ldexp(nearbyint(ldexp(g, k)), -k);   /* default rounding: to nearest, ties to even */
}

/* ------------------------------------------------------------------------ */
/* Recurrence for one (sequence, head).                                     */
/*   q, k : [L][dk]   v : [L][dv]   beta : [L]   g : [L] or [L][dk]         */
/*   S0   : [dv][dk] or NULL (zero state)                                    */
/*   o    : [L][dv]   S_out : [dv][dk]                                       */
/* Optional boundary record (any pointer may be NULL): for every chunked-     */
/* prefix boundary b (t <= P and t % 64 == 0 or t == P), bound_pre[b] is the  */
/* state after token t before QDQ, bound_post[b] after it (equal to pre when  */
/* CHUNK QDQ is off), bound_scales[b][dv/64] the scales (1 when no QDQ).     */
/* grid_log2 > 0: tokens t > P decay with orc_grid_gate(g, grid_log2).       */
/* Returns the number of prefix boundaries (ceil(P/64)), or -1 on bad args.  */
/* ------------------------------------------------------------------------ */
int orc_gdn_sequence(int L, int P, int dk, int dv, int per_channel, unsigned flags,
                     const double* q, const double* k, const double* v,
                     const double* beta, const double* g, const double* S0,
                     double* o, double* S_out,
                     int max_bounds, double* bound_pre, double* bound_post,
                     float* bound_scales, int grid_log2)
{
    if (L < 0 || P < 0 || P > L || dk <= 0 || dv <= 0) return -1;
    if (flags && dv % ORC_TILE_ROWS) return -1;     /* QDQ tiles are 64 value rows */
    if ((flags & ORC_QDQ_INT8) && dk % ORC_INT8_BLOCK) return -1;
    int64_t n = (int64_t)dv * dk;
    int tiles = dv / ORC_TILE_ROWS > 0 ? dv / ORC_TILE_ROWS : 1;
    double* S = (double*)malloc(sizeof(double) * (size_t)n);
    double* dec = (double*)malloc(sizeof(double) * (size_t)dk);
    float* tmp = (float*)malloc(sizeof(float) * (size_t)n);
    float* sc = (float*)malloc(sizeof(float) * (size_t)tiles);
    if (!S || !dec || !tmp || !sc) { free(S); free(dec); free(tmp); free(sc); return -1; }
    if (S0) memcpy(S, S0, sizeof(double) * (size_t)n);
    else    memset(S, 0, sizeof(double) * (size_t)n);

    int nb = 0;
    for (int t = 1; t <= L; ++t) {
        const double* qt = q + (int64_t)(t - 1) * dk;
        const double* kt = k + (int64_t)(t - 1) * dk;
        const double* vt = v + (int64_t)(t - 1) * dv;
        double bt = beta[t - 1];

        /* decay (a recurrent write t > P on the log-retention grid when one is set) */
        int kg = (t > P) ? grid_log2 : 0;
        if (per_channel) {
            for (int c = 0; c < dk; ++c) dec[c] = exp(orc_grid_gate(g[(int64_t)(t - 1) * dk + c], kg));
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c) S[(int64_t)r * dk + c] *= dec[c];
        } else {
            double a = exp(orc_grid_gate(g[t - 1], kg));
            for (int64_t i = 0; i < n; ++i) S[i] *= a;
        }
        /* delta correction against the decayed state */
        for (int r = 0; r < dv; ++r) {
            double* Sr = S + (int64_t)r * dk;
            double y = 0.0;
            for (int c = 0; c < dk; ++c) y += Sr[c] * kt[c];
            double u = bt * (vt[r] - y);
            for (int c = 0; c < dk; ++c) Sr[c] += u * kt[c];
        }
        /* output from the working state */
        for (int r = 0; r < dv; ++r) {
            const double* Sr = S + (int64_t)r * dk;
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += Sr[c] * qt[c];
            o[(int64_t)(t - 1) * dv + r] = acc;
        }
        /* boundaries */
        int is_bound = (t <= P) && (t % ORC_CHUNK == 0 || t == P);
        int do_qdq = ((flags & ORC_QDQ_CHUNK) && is_bound) ||
                     ((flags & ORC_QDQ_WRITE) && t >= (P > 1 ? P : 1));
        if (is_bound && nb < max_bounds && bound_pre)
            memcpy(bound_pre + (int64_t)nb * n, S, sizeof(double) * (size_t)n);
        if (do_qdq && (flags & ORC_QDQ_INT8)) {
            for (int64_t i = 0; i < n; ++i) tmp[i] = (float)S[i];
            orc_qdq_int8_blocks_f32(tmp, n / ORC_INT8_BLOCK, ORC_INT8_BLOCK, tmp, NULL, NULL);
            for (int64_t i = 0; i < n; ++i) S[i] = (double)tmp[i];
            for (int j = 0; j < tiles; ++j) sc[j] = 1.0f;    /* the record's scales are the FP8 codec's */
        } else if (do_qdq) {
            qdq_state_f64(S, dv, dk, tmp, sc);
        } else {
            for (int j = 0; j < tiles; ++j) sc[j] = 1.0f;
        }
        if (is_bound && nb < max_bounds) {
            if (bound_post) memcpy(bound_post + (int64_t)nb * n, S, sizeof(double) * (size_t)n);
            if (bound_scales) memcpy(bound_scales + (int64_t)nb * tiles, sc, sizeof(float) * (size_t)tiles);
        }
        if (is_bound) ++nb;
    }
    memcpy(S_out, S, sizeof(double) * (size_t)n);
    free(S); free(dec); free(tmp); free(sc);
    return nb;
}
