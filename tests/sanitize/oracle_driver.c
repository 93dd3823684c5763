/*
 * oracle_driver.c -- runs every function of the CPU oracle (oracle/ssm_oracle.c)
 * on small inputs and edge cases, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Test infrastructure
 * only: it checks memory safety and defined behaviour of the oracle, not its
 * values (the pins do that). Inputs come from a fixed linear congruential
 * sequence; every buffer is sized exactly to what the call may touch, so an
 * out-of-bounds index in the oracle is reported.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_gdn_step(int B, int H, int HV, int K, int V, int num_slots, const double *qkv, long qkv_stride,
                 const double *a, const double *b, const double *A_log, const double *dt_bias, double *state,
                 const int32_t *idx, double *out, double scale, int use_l2, double l2eps, const double *norm_gate,
                 const double *norm_w, double norm_eps, int norm_act, int state_fmt);
int orc_gdn_step_f32(int B, int H, int HV, int K, int V, int num_slots, const float *qkv, long qkv_stride,
                     const float *a, const float *b, const float *A_log, const float *dt_bias, float *state,
                     const int32_t *idx, float *out, float scale, int use_l2, float l2eps);
int orc_gdn_multi(int B, int T, int H, int HV, int K, int V, int num_slots, const double *qkv, long qkv_stride,
                  const double *a, const double *b, const double *A_log, const double *dt_bias, double *state,
                  const int32_t *idx, const int32_t *lengths, double *out, double scale, int use_l2, double l2eps,
                  const double *norm_gate, const double *norm_w, double norm_eps, int norm_act);
int orc_gdn_step_buffered(int B, int H, int HV, int K, int V, int num_slots, const double *qkv, long qkv_stride,
                          const double *a, const double *b, const double *A_log, const double *dt_bias,
                          double *state, const int32_t *idx, double *out, double scale, int use_l2, double l2eps,
                          const double *norm_gate, const double *norm_w, double norm_eps, int norm_act,
                          double *d_cache, double *k_cache, double *g_cache, const int32_t *write_pos, int L,
                          int ring_fmt);
int orc_conv1d_update(int T, int C, int W, int num_slots, const double *x, const double *w, const double *bias,
                      double *conv_state, const int32_t *idx, int skip_slot0, double *y, int act_silu);
int orc_kda_decode(int T, int H, int D, int W, int num_slots, const double *x, const double *conv_w,
                   const double *conv_bias, double *conv_state, const double *raw_g, const double *raw_beta,
                   double lower_bound, double *state, const int32_t *idx, double *out, const double *gate,
                   const double *norm_w, double norm_eps, double scale, int use_l2, double l2eps, double *y_scratch);
int orc_gdn_step_conv(int B, int H, int HV, int K, int V, int W, int num_slots, const double *x,
                      const double *conv_w, const double *conv_b, double *conv_state, const double *a,
                      const double *b, const double *A_log, const double *dt_bias, double *state, const int32_t *idx,
                      double *out, double scale, int use_l2, double l2eps, const double *norm_gate,
                      const double *norm_w, double norm_eps, int norm_act, double *y_scratch);
int orc_mamba_step(int B, int Dm, int N, int num_slots, const double *x, const double *dt, const double *A,
                   const double *Bm, const double *Cm, const double *Dv, const double *z, double *hpool,
                   const int32_t *idx, double *y);
int orc_mamba_scan(int B, int T, int Dm, int N, int num_slots, const double *x, const double *dt, const double *A,
                   const double *Bm, const double *Cm, const double *Dv, const double *z, double *hpool,
                   const int32_t *idx, const int32_t *lengths, int zero_init, double *y);
double orc_round_fmt(double x, int fmt);
double orc_softplus(double x);
double orc_kda_gate(double raw_g, double lb);

static uint64_t lcg = 12345;
static double rnd(void) {
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((double)(lcg >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}
/* exactly n doubles from the sequence (a fresh heap block of that size) */
static double *vec(size_t n) {
    double *p = malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i)
        p[i] = rnd();
    return p;
}
static float *vecf(size_t n) {
    float *p = malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i)
        p[i] = (float)rnd();
    return p;
}
static int fails = 0;
#define CHECK(x) do { if (!(x)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #x); ++fails; } } while (0)

static void gdn(int H, int HV, int K, int V, int with_norm, int state_fmt) {
    const int B = 5, slots = 4;
    const long C = 2L * H * K + (long)HV * V;
    const int32_t idx[5] = {2, -1, 0, 4, 3}; /* a negative and an out-of-range pad */
    double *qkv = vec((size_t)B * C), *a = vec((size_t)B * HV), *b = vec((size_t)B * HV);
    double *Al = vec(HV), *db = vec(HV), *st = vec((size_t)slots * HV * V * K), *out = vec((size_t)B * HV * V);
    double *ng = with_norm ? vec((size_t)B * HV * V) : NULL, *nw = with_norm ? vec(V) : NULL;
    CHECK(orc_gdn_step(B, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, out, 0.3, 1, 1e-6, ng, nw, 1e-5, 0,
                       state_fmt) == 0);
    CHECK(orc_gdn_step(0, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, out, 0.3, 1, 1e-6, NULL, NULL, 1e-5, 1,
                       state_fmt) == 0);
    if (H > 1) /* HV + 1 is then not a multiple of H: rejected before anything is read */
        CHECK(orc_gdn_step(B, H, HV + 1, K, V, slots, qkv, C, a, b, Al, db, st, idx, out, 0.3, 1, 1e-6, NULL,
                           NULL, 1e-5, 0, state_fmt) != 0);
    free(qkv); free(a); free(b); free(Al); free(db); free(st); free(out); free(ng); free(nw);
}

static void gdn_f32(void) {
    const int B = 3, H = 1, HV = 2, K = 8, V = 5, slots = 3;
    const long C = 2L * H * K + (long)HV * V;
    const int32_t idx[3] = {1, 7, 0};
    float *qkv = vecf((size_t)B * C), *a = vecf((size_t)B * HV), *b = vecf((size_t)B * HV);
    float *Al = vecf(HV), *db = vecf(HV), *st = vecf((size_t)slots * HV * V * K), *out = vecf((size_t)B * HV * V);
    CHECK(orc_gdn_step_f32(B, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, out, 0.35f, 1, 1e-6f) == 0);
    free(qkv); free(a); free(b); free(Al); free(db); free(st); free(out);
}

static void gdn_multi(void) {
    const int B = 3, T = 5, H = 2, HV = 4, K = 8, V = 6, slots = 4;
    const long C = 2L * H * K + (long)HV * V;
    const int32_t idx[3] = {3, -2, 1}, len[3] = {5, 2, 0};
    double *qkv = vec((size_t)B * T * C), *a = vec((size_t)B * T * HV), *b = vec((size_t)B * T * HV);
    double *Al = vec(HV), *db = vec(HV), *st = vec((size_t)slots * HV * V * K), *out = vec((size_t)B * T * HV * V);
    double *ng = vec((size_t)B * T * HV * V), *nw = vec(V);
    CHECK(orc_gdn_multi(B, T, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, len, out, 0.3, 1, 1e-6, ng, nw,
                        1e-5, 1) == 0);
    CHECK(orc_gdn_multi(B, T, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, NULL, out, 0.3, 0, 0.0, NULL,
                        NULL, 1e-5, 0) == 0);
    CHECK(orc_gdn_multi(B, 0, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, NULL, out, 0.3, 1, 1e-6, NULL,
                        NULL, 1e-5, 0) == 0);
    free(qkv); free(a); free(b); free(Al); free(db); free(st); free(out); free(ng); free(nw);
}

static void buffered(int L, int fmt) {
    const int B = 4, H = 2, HV = 4, K = 8, V = 7, slots = 5;
    const long C = 2L * H * K + (long)HV * V;
    const int32_t idx[4] = {4, 0, -1, 2};
    int32_t wp[4] = {0, L - 1, 0, L}; /* first phase, flush, padded slot, out-of-range phase */
    double *qkv = vec((size_t)B * C), *a = vec((size_t)B * HV), *b = vec((size_t)B * HV);
    double *Al = vec(HV), *db = vec(HV), *st = vec((size_t)slots * HV * V * K), *out = vec((size_t)B * HV * V);
    double *dc = vec((size_t)slots * HV * L * V), *kc = vec((size_t)slots * H * L * K), *gc = vec((size_t)slots * HV * L);
    double *ng = vec((size_t)B * HV * V);
    for (int p = 0; p < L; ++p) {
        wp[0] = p;
        CHECK(orc_gdn_step_buffered(B, H, HV, K, V, slots, qkv, C, a, b, Al, db, st, idx, out, 0.3, 1, 1e-6,
                                    p % 2 ? ng : NULL, NULL, 1e-5, 0, dc, kc, gc, wp, L, fmt) == 0);
    }
    free(qkv); free(a); free(b); free(Al); free(db); free(st); free(out); free(dc); free(kc); free(gc); free(ng);
}

static void kda(int D, int W, int with_gate) {
    const int T = 4, H = 2, slots = 5, C = 3 * H * D;
    const int32_t idx[4] = {0, 3, 5, 1}; /* NULL block, live, out of range, live */
    double *x = vec((size_t)T * C), *cw = vec((size_t)C * W), *cb = vec(C), *cs = vec((size_t)slots * C * (W - 1));
    double *rg = vec((size_t)T * H * D), *rb = vec((size_t)T * H), *st = vec((size_t)slots * H * D * D);
    double *out = vec((size_t)T * H * D), *g = with_gate ? vec((size_t)T * H * D) : NULL, *nw = vec(D);
    double *y = vec((size_t)T * C);
    CHECK(orc_kda_decode(T, H, D, W, slots, x, cw, with_gate ? cb : NULL, cs, rg, rb, -5.0, st, idx, out, g, nw,
                         1e-5, 0.2, 1, 1e-6, y) == 0);
    free(x); free(cw); free(cb); free(cs); free(rg); free(rb); free(st); free(out); free(g); free(nw); free(y);
}

static void gdn_conv(int W) {
    const int B = 3, H = 1, HV = 2, K = 8, V = 6, slots = 3;
    const int C = 2 * H * K + HV * V;
    const int32_t idx[3] = {0, 9, 2};
    double *x = vec((size_t)B * C), *cw = vec((size_t)C * W), *cb = vec(C), *cs = vec((size_t)slots * C * (W - 1));
    double *a = vec((size_t)B * HV), *b = vec((size_t)B * HV), *Al = vec(HV), *db = vec(HV);
    double *st = vec((size_t)slots * HV * V * K), *out = vec((size_t)B * HV * V), *y = vec((size_t)B * C);
    CHECK(orc_gdn_step_conv(B, H, HV, K, V, W, slots, x, cw, cb, cs, a, b, Al, db, st, idx, out, 0.3, 1, 1e-6, NULL,
                            NULL, 1e-5, 0, y) == 0);
    free(x); free(cw); free(cb); free(cs); free(a); free(b); free(Al); free(db); free(st); free(out); free(y);
}

static void mamba(int N) {
    const int B = 3, T = 6, Dm = 5, slots = 3;
    const int32_t idx[3] = {2, -1, 0}, len[3] = {6, 3, 0};
    double *x = vec((size_t)B * T * Dm), *dt = vec((size_t)B * T * Dm), *A = vec((size_t)Dm * N);
    double *Bm = vec((size_t)B * T * N), *Cm = vec((size_t)B * T * N), *Dv = vec(Dm), *z = vec((size_t)B * T * Dm);
    double *h = vec((size_t)slots * Dm * N), *y = vec((size_t)B * T * Dm);
    for (size_t i = 0; i < (size_t)B * T * Dm; ++i)
        dt[i] = fabs(dt[i]) * 0.1;
    CHECK(orc_mamba_step(B, Dm, N, slots, x, dt, A, Bm, Cm, Dv, z, h, idx, y) == 0);
    CHECK(orc_mamba_step(B, Dm, N, slots, x, dt, A, Bm, Cm, NULL, NULL, h, idx, y) == 0);
    CHECK(orc_mamba_scan(B, T, Dm, N, slots, x, dt, A, Bm, Cm, Dv, z, h, idx, len, 0, y) == 0);
    CHECK(orc_mamba_scan(B, T, Dm, N, slots, x, dt, A, Bm, Cm, NULL, NULL, h, idx, NULL, 1, y) == 0);
    free(x); free(dt); free(A); free(Bm); free(Cm); free(Dv); free(z); free(h); free(y);
}

int main(void) {
    /* scalar helpers over the formats' edges */
    const double edge[] = {0.0, -0.0, 1e-310, 3.5e38, -3.5e38, 65520.0, 1e300, -1e300, 1.0 + 1.0 / 256};
    for (size_t i = 0; i < sizeof edge / sizeof edge[0]; ++i)
        for (int f = 0; f < 4; ++f)
            (void)orc_round_fmt(edge[i], f);
    CHECK(orc_softplus(1000.0) == 1000.0);
    CHECK(orc_kda_gate(0.0, -5.0) == -2.5);
    gdn(2, 4, 16, 5, 0, 3);
    gdn(1, 3, 4, 9, 1, 1);
    gdn(2, 2, 8, 3, 1, 2);
    gdn_f32();
    gdn_multi();
    buffered(1, 1);
    buffered(3, 1);
    buffered(4, 3);
    kda(8, 4, 1);
    kda(4, 2, 0);
    gdn_conv(4);
    gdn_conv(2);
    mamba(1);
    mamba(4);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ORACLE_DRIVER_OK\n");
    return 0;
}
