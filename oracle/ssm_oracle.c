/*
 * ssm_oracle.c -- plain, slow fp64 CPU oracle for the single-token recurrent
 * decode step of gated linear-attention / SSM layers.
 *
 * TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and
 * the cpu_baseline leg of bench.py may load this library. It shares no code,
 * header, table or helper with the HIP library under
 * ssm_recurrent_decode_gated_amd/csrc, and neither side includes the other.
 *
 * Sources (web pages; cited by title and section):
 *   [MBU]    "Triton decode kernel + MBU analysis" (Mamba-1 decode write-up)
 *   [REPLAY] "Microbenchmark: buffered output-only GDN decode (ReplaySSM
 *            Part A) vs. the existing packed GDN decode kernel" (script)
 *   [KDA]    "Microbenchmark for the fused Kimi-K3 KDA decode kernel on ROCm"
 *            (script)
 *   [LOG]    "Optimization Log: Qwen3.5-27B Dense on B200"
 *
 * Arithmetic: every value is IEEE fp64, computed in plain scalar loops in the
 * order the method states it, on the full V x K matrix of each head. No
 * blocking, no fusion, no reassociation. Inputs arrive already decoded to fp64
 * (bf16/f16/f32 -> fp64 is exact). Rounding to a storage format happens only
 * where the method stores a value in that format (the buffered ring).
 * OpenMP only spreads independent (row, head) units over host threads; it does
 * not change any arithmetic.
 *
 * Parity pins (closed forms, invariants, a hand-worked 4x4 case) live in
 * tests/test_oracle_pins.py; every function here is pinned by at least one
 * of them. One choice is a reading rather than a formula the pages print:
 * L2-normalising q/k in the KDA step (optional, as in the GDN step, whose
 * arithmetic it shares and whose pins cover it).
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD (-1)

/* storage formats for rounding */
#define ORC_FMT_F32 0
#define ORC_FMT_BF16 1
#define ORC_FMT_F16 2
#define ORC_FMT_NONE 3 /* keep fp64 */

#define ORC_ACT_SILU 0
#define ORC_ACT_SIGMOID 1

/* ------------------------------------------------------------------ */
/* scalar helpers                                                      */
/* ------------------------------------------------------------------ */

/* softplus(x) = log(1 + e^x); for x > 20 the correction e^-x < 2e-9 is
 * below fp64 relevance for the gate, and x is returned. */
double orc_softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }

double orc_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

double orc_silu(double x) { return x * orc_sigmoid(x); }

/* Round-to-nearest-even of x to a binary format with p significand bits
 * (hidden bit included), minimum normal exponent emin and maximum exponent
 * emax. Subnormals use the fixed spacing 2^(emin-p+1); results beyond the
 * largest finite value become +-inf (IEEE 754 roundTiesToEven overflow). */
static double round_binary(double x, int p, int emin, int emax)
{
    if (x != x || isinf(x) || x == 0.0)
        return x;
    int e;
    frexp(x, &e);        /* x = m 2^e, 0.5 <= |m| < 1 */
    int lead = e - 1;    /* exponent of the leading bit */
    if (lead < emin)
        lead = emin;
    double ulp = ldexp(1.0, lead - (p - 1));
    double r = nearbyint(x / ulp) * ulp; /* default mode: ties to even */
    double maxv = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxv)
        return copysign(INFINITY, x);
    return r;
}

double orc_round_fmt(double x, int fmt)
{
    switch (fmt) {
    case ORC_FMT_F32: return round_binary(x, 24, -126, 127);
    case ORC_FMT_BF16: return round_binary(x, 8, -126, 127);
    case ORC_FMT_F16: return round_binary(x, 11, -14, 15);
    default: return x;
    }
}

/* GDN gates ([REPLAY] argument list a, b, A_log, dt_bias; the gate formula is
 * the plain reading that matches [MBU] "Kernel design": decay = exp(dt*A) with
 * A = -exp(A_log) and dt = softplus(a + dt_bias)):
 *   g    = -exp(A_log) * softplus(a + dt_bias)   (log of the decay)
 *   beta = sigmoid(b)                                                  */
void orc_gdn_gates(double a, double b, double A_log, double dt_bias,
                   double *g, double *beta)
{
    *g = -exp(A_log) * orc_softplus(a + dt_bias);
    *beta = orc_sigmoid(b);
}

/* KDA per-channel gate, as the fused-op workload fixes it: g = lb *
 * sigmoid(raw_g) with lb = -5 [KDA, constants and the `fused` call:
 * lower_bound]. The pages also pass A_log[H] and dt_bias[H*D] to the op
 * without saying how they enter the gate, so no form using them is computed
 * here (the library refuses them). */
double orc_kda_gate(double raw_g, double lb)
{
    return lb * orc_sigmoid(raw_g);
}

/* ------------------------------------------------------------------ */
/* one head of the gated delta rule                                    */
/* ------------------------------------------------------------------ */

/* [LOG] "Kernel 4: Fused DeltaNet Recurrent", Math, written for a state
 * stored as S[V][K] (row = value index, column = key index, the layout of
 * [REPLAY] `_bench_cfg`: state randn(num_slots, HV, V, K)). In that layout the
 * page's S^T k and S^T q are the matrix-vector products S k and S q:
 *   S <- S diag(decay)         (GDN: every decay[c] = exp(g); KDA: per key channel)
 *   u <- S k
 *   delta <- beta (v - u)
 *   S <- S + delta k^T
 *   o <- S q
 * Each line runs over the whole matrix before the next starts. */
static void delta_rule_head(double *S, int V, int K, const double *decay,
                            const double *k, const double *q, const double *v,
                            double beta, double *o, double *delta, double *u)
{
    for (int r = 0; r < V; ++r)
        for (int c = 0; c < K; ++c)
            S[(size_t)r * K + c] *= decay[c];
    for (int r = 0; r < V; ++r) {
        double acc = 0.0;
        for (int c = 0; c < K; ++c)
            acc += S[(size_t)r * K + c] * k[c];
        u[r] = acc;
    }
    for (int r = 0; r < V; ++r)
        delta[r] = beta * (v[r] - u[r]);
    for (int r = 0; r < V; ++r)
        for (int c = 0; c < K; ++c)
            S[(size_t)r * K + c] += delta[r] * k[c];
    for (int r = 0; r < V; ++r) {
        double acc = 0.0;
        for (int c = 0; c < K; ++c)
            acc += S[(size_t)r * K + c] * q[c];
        o[r] = acc;
    }
}

/* q/k preparation: optional L2 normalisation x / sqrt(sum x^2 + eps), then q
 * is multiplied by `scale` ([REPLAY] `_bench_cfg`: scale = K**-0.5,
 * use_qk_l2norm_in_kernel=True). k is not scaled. */
static void prep_qk(const double *qin, const double *kin, int K, double scale,
                    int use_l2, double l2eps, double *q, double *k)
{
    double qn = 1.0, kn = 1.0;
    if (use_l2) {
        double sq = 0.0, sk = 0.0;
        for (int c = 0; c < K; ++c) {
            sq += qin[c] * qin[c];
            sk += kin[c] * kin[c];
        }
        qn = 1.0 / sqrt(sq + l2eps);
        kn = 1.0 / sqrt(sk + l2eps);
    }
    for (int c = 0; c < K; ++c) {
        q[c] = qin[c] * qn * scale;
        k[c] = kin[c] * kn;
    }
}

/* Gated RMSNorm over one head's V outputs ([KDA] `_gated_rmsnorm`; [LOG]
 * "Kernel 2: Triton RMSNormGated" gives the silu-gated form):
 *   o <- o / sqrt(mean(o^2) + eps) * w * act(gate)                       */
static void gated_rmsnorm(double *o, int V, const double *gate,
                          const double *w, double eps, int act)
{
    double ss = 0.0;
    for (int r = 0; r < V; ++r)
        ss += o[r] * o[r];
    double inv = 1.0 / sqrt(ss / V + eps);
    for (int r = 0; r < V; ++r) {
        double gz = act == ORC_ACT_SIGMOID ? orc_sigmoid(gate[r]) : orc_silu(gate[r]);
        o[r] = o[r] * inv * (w ? w[r] : 1.0) * gz;
    }
}

/* ------------------------------------------------------------------ */
/* packed GDN decode step                                              */
/* ------------------------------------------------------------------ */

/* One packed GDN decode step over B batch rows ([REPLAY] module docstring and
 * `_make_static`/`_bench_cfg`: packed mixed_qkv = [q heads | k heads | v heads]
 * with qk_dim = 2*H*K before v_dim = HV*V; state pool [num_slots, HV, V, K]
 * indexed by ssm_state_indices; out [B, 1, HV, V]).
 * Value head hv reads q/k head hv / (HV/H) (contiguous GQA groups).
 * Row b is padded, and touches nothing, when idx[b] < 0 or >= num_slots.
 * state is fp64 and updated in place; out receives unrounded fp64.
 * state_fmt: the format the pool stores the state in (ORC_FMT_NONE keeps fp64;
 * ORC_FMT_BF16 / F16 model the 16-bit per-head state of [LOG] "Kernel 4": the
 * updated state is rounded once when stored, after this step's output has
 * been formed from the unrounded update). */
int orc_gdn_step(int B, int H, int HV, int K, int V, int num_slots,
                 const double *qkv, long qkv_stride, const double *a,
                 const double *b, const double *A_log, const double *dt_bias,
                 double *state, const int32_t *idx, double *out, double scale,
                 int use_l2, double l2eps, const double *norm_gate,
                 const double *norm_w, double norm_eps, int norm_act, int state_fmt)
{
    if (B < 0 || H < 1 || HV < 1 || HV % H || K < 1 || V < 1 || num_slots < 1)
        return ORC_BAD;
    const int G = HV / H;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int bi = 0; bi < B; ++bi) {
        for (int hv = 0; hv < HV; ++hv) {
            const int s = idx[bi];
            if (s < 0 || s >= num_slots)
                continue;
            const int h = hv / G;
            const double *row = qkv + (size_t)bi * qkv_stride;
            double *q = malloc(sizeof(double) * (3 * (size_t)K + 3 * (size_t)V));
            double *k = q + K, *decay = k + K, *o = decay + K, *delta = o + V, *u = delta + V;
            prep_qk(row + (size_t)h * K, row + (size_t)H * K + (size_t)h * K, K,
                    scale, use_l2, l2eps, q, k);
            double g, beta;
            orc_gdn_gates(a[(size_t)bi * HV + hv], b[(size_t)bi * HV + hv],
                          A_log[hv], dt_bias[hv], &g, &beta);
            for (int c = 0; c < K; ++c)
                decay[c] = exp(g);
            double *S = state + ((size_t)s * HV + hv) * (size_t)V * K;
            const double *v = row + 2 * (size_t)H * K + (size_t)hv * V;
            delta_rule_head(S, V, K, decay, k, q, v, beta, o, delta, u);
            if (state_fmt != ORC_FMT_NONE)
                for (size_t e = 0; e < (size_t)V * K; ++e)
                    S[e] = orc_round_fmt(S[e], state_fmt);
            if (norm_gate)
                gated_rmsnorm(o, V, norm_gate + ((size_t)bi * HV + hv) * V,
                              norm_w, norm_eps, norm_act);
            memcpy(out + ((size_t)bi * HV + hv) * V, o, sizeof(double) * V);
            free(q);
        }
    }
    return ORC_OK;
}

/* The packed GDN step once more, every value in IEEE fp32 (float, no
 * wider intermediates: each operation rounds to float). A sanity build of
 * the oracle, not a second oracle: it runs the same method in the same order
 * (gates, optional q/k L2 norm and scale, decay, S k, delta, rank-1 update,
 * S q) without the output norm, so the fp64 oracle can be held against a
 * float computation of the same recurrence (the fp32 tolerance of [MBU]
 * "Correctness" is the bar). state is fp32 [num_slots][HV][V][K], updated in
 * place; out is fp32 [B][HV][V]. */
int orc_gdn_step_f32(int B, int H, int HV, int K, int V, int num_slots,
                     const float *qkv, long qkv_stride, const float *a_in,
                     const float *b_in, const float *A_log, const float *dt_bias,
                     float *state, const int32_t *idx, float *out, float scale,
                     int use_l2, float l2eps)
{
    if (B < 0 || H < 1 || HV < 1 || HV % H || K < 1 || V < 1 || num_slots < 1)
        return ORC_BAD;
    const int grp = HV / H;
    float *qs = malloc(sizeof(float) * (2 * (size_t)K + 2 * (size_t)V));
    float *ks = qs + K, *sk = ks + K, *dl = sk + V;
    for (int bi = 0; bi < B; ++bi) {
        const int slot = idx[bi];
        if (slot < 0 || slot >= num_slots)
            continue;
        const float *x = qkv + (size_t)bi * qkv_stride;
        for (int hv = 0; hv < HV; ++hv) {
            const float *xq = x + (size_t)(hv / grp) * K;
            const float *xk = x + (size_t)H * K + (size_t)(hv / grp) * K;
            const float *xv = x + 2 * (size_t)H * K + (size_t)hv * V;
            float nq = 1.0f, nk = 1.0f;
            if (use_l2) {
                float s2q = 0.0f, s2k = 0.0f;
                for (int i = 0; i < K; ++i) {
                    s2q += xq[i] * xq[i];
                    s2k += xk[i] * xk[i];
                }
                nq = 1.0f / sqrtf(s2q + l2eps);
                nk = 1.0f / sqrtf(s2k + l2eps);
            }
            for (int i = 0; i < K; ++i) {
                qs[i] = xq[i] * nq * scale;
                ks[i] = xk[i] * nk;
            }
            const float z = a_in[(size_t)bi * HV + hv] + dt_bias[hv];
            const float sp = z > 20.0f ? z : log1pf(expf(z));
            const float gl = -expf(A_log[hv]) * sp;
            const float bt = 1.0f / (1.0f + expf(-b_in[(size_t)bi * HV + hv]));
            const float ed = expf(gl);
            float *M = state + ((size_t)slot * HV + hv) * (size_t)V * K;
            for (size_t e = 0; e < (size_t)V * K; ++e)
                M[e] = M[e] * ed;
            for (int r = 0; r < V; ++r) {
                float dot = 0.0f;
                for (int i = 0; i < K; ++i)
                    dot += M[(size_t)r * K + i] * ks[i];
                sk[r] = dot;
            }
            for (int r = 0; r < V; ++r)
                dl[r] = bt * (xv[r] - sk[r]);
            for (int r = 0; r < V; ++r)
                for (int i = 0; i < K; ++i)
                    M[(size_t)r * K + i] = M[(size_t)r * K + i] + dl[r] * ks[i];
            float *o = out + ((size_t)bi * HV + hv) * V;
            for (int r = 0; r < V; ++r) {
                float dot = 0.0f;
                for (int i = 0; i < K; ++i)
                    dot += M[(size_t)r * K + i] * qs[i];
                o[r] = dot;
            }
        }
    }
    free(qs);
    return ORC_OK;
}

/* GDN over T tokens per sequence: the packed step above applied to tokens
 * 0..len-1 of each row in order, the state carried from token to token (the
 * recurrent form of [LOG] "Kernel 4" run over a token axis; [MBU] "Prefill
 * path" for the multi-token use). Row b, token t reads mixed_qkv row
 * b*T + t (stride qkv_stride), a/b [B][T][HV], norm_gate [B][T][HV][V], and
 * writes out [B][T][HV][V]; tokens t >= len (lengths[b], clamped to [0, T];
 * NULL: T) and padded rows write nothing. */
int orc_gdn_multi(int B, int T, int H, int HV, int K, int V, int num_slots,
                  const double *qkv, long qkv_stride, const double *a,
                  const double *b, const double *A_log, const double *dt_bias,
                  double *state, const int32_t *idx, const int32_t *lengths,
                  double *out, double scale, int use_l2, double l2eps,
                  const double *norm_gate, const double *norm_w, double norm_eps,
                  int norm_act)
{
    if (B < 0 || T < 0)
        return ORC_BAD;
    int32_t *idx_t = malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
    double *a_t = malloc(sizeof(double) * ((size_t)B * HV + 1));
    double *b_t = malloc(sizeof(double) * ((size_t)B * HV + 1));
    double *ng_t = norm_gate ? malloc(sizeof(double) * ((size_t)B * HV * V + 1)) : NULL;
    double *o_t = malloc(sizeof(double) * ((size_t)B * HV * V + 1));
    int rc = ORC_OK;
    for (int t = 0; t < T && rc == ORC_OK; ++t) {
        for (int bi = 0; bi < B; ++bi) {
            int len = lengths ? lengths[bi] : T;
            len = len < 0 ? 0 : (len > T ? T : len);
            idx_t[bi] = t < len ? idx[bi] : -1;
            const size_t bt = (size_t)bi * T + t;
            memcpy(a_t + (size_t)bi * HV, a + bt * HV, sizeof(double) * HV);
            memcpy(b_t + (size_t)bi * HV, b + bt * HV, sizeof(double) * HV);
            if (ng_t)
                memcpy(ng_t + (size_t)bi * HV * V, norm_gate + bt * HV * V, sizeof(double) * HV * V);
        }
        rc = orc_gdn_step(B, H, HV, K, V, num_slots, qkv + (size_t)t * qkv_stride,
                          qkv_stride * T, a_t, b_t, A_log, dt_bias, state, idx_t, o_t,
                          scale, use_l2, l2eps, ng_t, norm_w, norm_eps, norm_act,
                          ORC_FMT_NONE);
        for (int bi = 0; bi < B; ++bi)
            if (idx_t[bi] >= 0 && idx_t[bi] < num_slots)
                memcpy(out + ((size_t)bi * T + t) * HV * V, o_t + (size_t)bi * HV * V,
                       sizeof(double) * HV * V);
    }
    free(idx_t);
    free(a_t);
    free(b_t);
    free(ng_t);
    free(o_t);
    return rc;
}

/* ------------------------------------------------------------------ */
/* buffered (L-step write-back) GDN decode step                        */
/* ------------------------------------------------------------------ */

/* [REPLAY] module docstring, `_bench_cfg` and `_state_bytes_per_step`: the pool
 * holds a checkpoint S_ck that is written only once every L steps; every step
 * appends a ring record (d: [HV, V] in the activation dtype, k: [H, K] in the
 * activation dtype shared by the HV/H value heads of a q/k head, g: [HV] fp32)
 * at position p = write_pos[b]; at p == L-1 the ring is folded into the
 * checkpoint and the state is written back.
 *
 * Reading used here (the pages give no formula): a record holds this step's
 * delta-rule update -- d = delta, k = the normalised key, g = the log decay --
 * so replaying records 0..p-1 on the checkpoint, one by one,
 *     S <- exp(g_j) S + d_j k_j^T ,
 * reproduces the state after step p-1. Step p is then the packed step above,
 * run from that state with this step's full-precision delta and k; the stored
 * copies are rounded to the ring's formats. write_pos is read, never advanced.
 * A row whose write_pos is outside [0, L) is treated as padded.
 * ring_fmt is the storage format of d and k (ORC_FMT_*); g is stored as fp32. */
int orc_gdn_step_buffered(int B, int H, int HV, int K, int V, int num_slots,
                          const double *qkv, long qkv_stride, const double *a,
                          const double *b, const double *A_log,
                          const double *dt_bias, double *state,
                          const int32_t *idx, double *out, double scale,
                          int use_l2, double l2eps, const double *norm_gate,
                          const double *norm_w, double norm_eps, int norm_act,
                          double *d_cache, double *k_cache, double *g_cache,
                          const int32_t *write_pos, int L, int ring_fmt)
{
    if (B < 0 || H < 1 || HV < 1 || HV % H || K < 1 || V < 1 || num_slots < 1 || L < 1)
        return ORC_BAD;
    const int G = HV / H;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int bi = 0; bi < B; ++bi) {
        for (int hv = 0; hv < HV; ++hv) {
            const int s = idx[bi];
            const int p = write_pos[bi];
            if (s < 0 || s >= num_slots || p < 0 || p >= L)
                continue;
            const int h = hv / G;
            const double *row = qkv + (size_t)bi * qkv_stride;
            double *S = malloc(sizeof(double) * ((size_t)V * K + 3 * (size_t)K + 3 * (size_t)V));
            double *q = S + (size_t)V * K, *k = q + K, *decay = k + K;
            double *o = decay + K, *delta = o + V, *u = delta + V;
            double *ck = state + ((size_t)s * HV + hv) * (size_t)V * K;
            double *dring = d_cache + ((size_t)s * HV + hv) * (size_t)L * V;
            double *kring = k_cache + ((size_t)s * H + h) * (size_t)L * K;
            double *gring = g_cache + ((size_t)s * HV + hv) * (size_t)L;

            /* replay the ring on a copy of the checkpoint */
            memcpy(S, ck, sizeof(double) * (size_t)V * K);
            for (int j = 0; j < p; ++j) {
                const double dj = exp(gring[j]);
                for (int r = 0; r < V; ++r)
                    for (int c = 0; c < K; ++c)
                        S[(size_t)r * K + c] = dj * S[(size_t)r * K + c] +
                                               dring[(size_t)j * V + r] * kring[(size_t)j * K + c];
            }

            /* this step, from the replayed state */
            prep_qk(row + (size_t)h * K, row + (size_t)H * K + (size_t)h * K, K,
                    scale, use_l2, l2eps, q, k);
            double g, beta;
            orc_gdn_gates(a[(size_t)bi * HV + hv], b[(size_t)bi * HV + hv],
                          A_log[hv], dt_bias[hv], &g, &beta);
            for (int c = 0; c < K; ++c)
                decay[c] = exp(g);
            const double *v = row + 2 * (size_t)H * K + (size_t)hv * V;
            delta_rule_head(S, V, K, decay, k, q, v, beta, o, delta, u);
            if (norm_gate)
                gated_rmsnorm(o, V, norm_gate + ((size_t)bi * HV + hv) * V,
                              norm_w, norm_eps, norm_act);
            memcpy(out + ((size_t)bi * HV + hv) * V, o, sizeof(double) * V);

            /* append this step's record at position p */
            for (int r = 0; r < V; ++r)
                dring[(size_t)p * V + r] = orc_round_fmt(delta[r], ring_fmt);
            gring[p] = orc_round_fmt(g, ORC_FMT_F32);
            if (hv % G == 0)
                for (int c = 0; c < K; ++c)
                    kring[(size_t)p * K + c] = orc_round_fmt(k[c], ring_fmt);

            /* fold: the last phase of the cycle writes the state back */
            if (p == L - 1)
                memcpy(ck, S, sizeof(double) * (size_t)V * K);
            free(S);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* KDA: causal conv1d update, per-channel delta rule, gated RMSNorm     */
/* ------------------------------------------------------------------ */

/* Causal depthwise conv1d update for one decode token per row ([KDA]
 * `triton_chain`: causal_conv1d_update(..., activation="silu",
 * conv_state_indices=...); [LOG] "Kernel 5: Fused Causal Conv1d Update"
 * describes the same update as one fused kernel). Per channel c the window is
 * [cs[0], ..., cs[W-2], x] (oldest first); y = act(sum_j w[c][j] window[j] +
 * bias[c]); the state becomes window[1..W-1]. conv_state is the logical
 * [num_slots][C][W-1] array. A row is skipped when its slot is < 0, >=
 * num_slots, or == 0 with skip_slot0 (the fused KDA op's NULL block, [KDA]
 * `Inputs`). act_silu = 0 leaves y linear. */
int orc_conv1d_update(int T, int C, int W, int num_slots, const double *x,
                      const double *w, const double *bias, double *conv_state,
                      const int32_t *idx, int skip_slot0, double *y, int act_silu)
{
    if (T < 0 || C < 1 || W < 2 || num_slots < 1)
        return ORC_BAD;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const int s = idx[t];
        if (s < 0 || s >= num_slots || (skip_slot0 && s == 0))
            continue;
        double *win = malloc(sizeof(double) * (size_t)W);
        for (int c = 0; c < C; ++c) {
            double *cs = conv_state + ((size_t)s * C + c) * (size_t)(W - 1);
            for (int j = 0; j < W - 1; ++j)
                win[j] = cs[j];
            win[W - 1] = x[(size_t)t * C + c];
            double acc = bias ? bias[c] : 0.0;
            for (int j = 0; j < W; ++j)
                acc += w[(size_t)c * W + j] * win[j];
            y[(size_t)t * C + c] = act_silu ? orc_silu(acc) : acc;
            for (int j = 0; j < W - 1; ++j)
                cs[j] = win[j + 1];
        }
        free(win);
    }
    return ORC_OK;
}

/* KDA recurrent step on the post-conv activations y [T][3*H*D] = [q | k | v]
 * ([KDA] `triton_chain`: the conv output feeds fused_recurrent_kda_packed_decode
 * as mixed_qkv). Per token t and head h:
 *   q, k <- L2-normalised, q *= scale          (optional; a reading: the
 *                                               pages' chain shows no norm)
 *   g[c] <- orc_kda_gate(raw_g[t,h,c], lb)     (per key channel)
 *   beta <- sigmoid(raw_beta[t,h])
 *   delta rule with decay[c] = exp(g[c])
 *   o <- gated RMSNorm with a sigmoid gate ([KDA] `_gated_rmsnorm`) if gate
 * A token is skipped when its slot is <= 0 or >= num_slots (slot 0 is the
 * NULL block, [KDA] `Inputs`). */
int orc_kda_step(int T, int H, int D, int num_slots, const double *y,
                 const double *raw_g, const double *raw_beta, double lower_bound,
                 double *state, const int32_t *idx, double *out,
                 const double *gate, const double *norm_w, double norm_eps,
                 double scale, int use_l2, double l2eps)
{
    if (T < 0 || H < 1 || D < 1 || num_slots < 1)
        return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            const int s = idx[t];
            if (s <= 0 || s >= num_slots)
                continue;
            const size_t C = 3 * (size_t)H * D;
            const double *row = y + (size_t)t * C;
            double *q = malloc(sizeof(double) * 6 * (size_t)D);
            double *k = q + D, *decay = k + D, *o = decay + D, *delta = o + D, *u = delta + D;
            prep_qk(row + (size_t)h * D, row + (size_t)H * D + (size_t)h * D, D,
                    scale, use_l2, l2eps, q, k);
            for (int c = 0; c < D; ++c) {
                double gc = orc_kda_gate(raw_g[((size_t)t * H + h) * D + c], lower_bound);
                decay[c] = exp(gc);
            }
            const double beta = orc_sigmoid(raw_beta[(size_t)t * H + h]);
            double *S = state + ((size_t)s * H + h) * (size_t)D * D;
            const double *v = row + 2 * (size_t)H * D + (size_t)h * D;
            delta_rule_head(S, D, D, decay, k, q, v, beta, o, delta, u);
            if (gate)
                gated_rmsnorm(o, D, gate + ((size_t)t * H + h) * D, norm_w,
                              norm_eps, ORC_ACT_SIGMOID);
            memcpy(out + ((size_t)t * H + h) * D, o, sizeof(double) * D);
            free(q);
        }
    }
    return ORC_OK;
}

/* The fused KDA decode op: conv1d update + SiLU, then the KDA step, then the
 * gated norm, in one call ([KDA] module docstring and `fused`: one launch
 * replacing the conv -> recurrent decode -> gated RMSNorm chain). The conv
 * output is kept at fp64 (the fusion removes the intermediate QKV round trip,
 * so it is not rounded to bf16). y_scratch is [T][3*H*D]. */
int orc_kda_decode(int T, int H, int D, int W, int num_slots, const double *x,
                   const double *conv_w, const double *conv_bias,
                   double *conv_state, const double *raw_g,
                   const double *raw_beta, double lower_bound, double *state,
                   const int32_t *idx, double *out, const double *gate,
                   const double *norm_w, double norm_eps, double scale,
                   int use_l2, double l2eps, double *y_scratch)
{
    int rc = orc_conv1d_update(T, 3 * H * D, W, num_slots, x, conv_w, conv_bias,
                               conv_state, idx, 1, y_scratch, 1);
    if (rc)
        return rc;
    return orc_kda_step(T, H, D, num_slots, y_scratch, raw_g, raw_beta,
                        lower_bound, state, idx, out, gate, norm_w,
                        norm_eps, scale, use_l2, l2eps);
}

/* GDN with its causal conv1d update fused in front (the KDA fused op's
 * pattern, [KDA] module docstring and `triton_chain`, applied to the GDN step
 * of [REPLAY]; [LOG] "Integration" lists the DeltaNet forward as projection +
 * conv1d + recurrent + gated norm): the pre-conv activations x [B][2HK+HV*V]
 * go through orc_conv1d_update (SiLU, conv state per slot, padded rows
 * skipped by the GDN rule), and the fp64 conv output is the step's mixed_qkv.
 * y_scratch is [B][2HK+HV*V]. */
int orc_gdn_step_conv(int B, int H, int HV, int K, int V, int W, int num_slots,
                      const double *x, const double *conv_w,
                      const double *conv_b, double *conv_state,
                      const double *a, const double *b, const double *A_log,
                      const double *dt_bias, double *state, const int32_t *idx,
                      double *out, double scale, int use_l2, double l2eps,
                      const double *norm_gate, const double *norm_w,
                      double norm_eps, int norm_act, double *y_scratch)
{
    const int C = 2 * H * K + HV * V;
    int rc = orc_conv1d_update(B, C, W, num_slots, x, conv_w, conv_b, conv_state,
                               idx, 0, y_scratch, 1);
    if (rc)
        return rc;
    return orc_gdn_step(B, H, HV, K, V, num_slots, y_scratch, C, a, b, A_log,
                        dt_bias, state, idx, out, scale, use_l2, l2eps,
                        norm_gate, norm_w, norm_eps, norm_act, ORC_FMT_NONE);
}

/* ------------------------------------------------------------------ */
/* Mamba-1 selective-scan decode step                                  */
/* ------------------------------------------------------------------ */

/* [MBU] "Kernel design": per (batch row, channel d) with state row h[N]:
 *   dA = exp(dt * A[d,:]);  dB = dt * B[b,:]
 *   h  <- dA * h + dB * x
 *   y  = sum_n C[b,n] h[n]  (+ D[d] x if D)  (* silu(z) if z)
 * dt is an input (already positive). The state row lives at slot idx[b] of a
 * pool [num_slots][Dm][N]; idx < 0 or >= num_slots pads the row. */
int orc_mamba_step(int B, int Dm, int N, int num_slots, const double *x,
                   const double *dt, const double *A, const double *Bm,
                   const double *Cm, const double *Dv, const double *z,
                   double *hpool, const int32_t *idx, double *y)
{
    if (B < 0 || Dm < 1 || N < 1 || num_slots < 1)
        return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(static)
    for (int bi = 0; bi < B; ++bi) {
        for (int d = 0; d < Dm; ++d) {
            const int s = idx[bi];
            if (s < 0 || s >= num_slots)
                continue;
            const double xv = x[(size_t)bi * Dm + d];
            const double dtv = dt[(size_t)bi * Dm + d];
            double *h = hpool + ((size_t)s * Dm + d) * (size_t)N;
            double acc = 0.0;
            for (int n = 0; n < N; ++n) {
                const double dA = exp(dtv * A[(size_t)d * N + n]);
                const double dB = dtv * Bm[(size_t)bi * N + n];
                h[n] = dA * h[n] + dB * xv;
                acc += Cm[(size_t)bi * N + n] * h[n];
            }
            if (Dv)
                acc += Dv[d] * xv;
            if (z)
                acc *= orc_silu(z[(size_t)bi * Dm + d]);
            y[(size_t)bi * Dm + d] = acc;
        }
    }
    return ORC_OK;
}

/* Mamba-1 over T tokens (prefill): the step above applied to tokens
 * 0..len-1 of each row in order, the state carried between them ([MBU]
 * "Prefill path": the multi-token scan over the same recurrence). Per row b
 * with slot s = idx[b] in [0, num_slots) and len = lengths ? lengths[b] : T:
 *   h = zero_init ? 0 : hpool[s]
 *   for t < len: h <- exp(dt[b,t,d] A[d,:]) h + dt[b,t,d] B[b,t,:] x[b,t,d]
 *                y[b,t,d] = sum_n C[b,t,n] h[n] (+ D[d] x) (* silu(z[b,t,d]))
 *   hpool[s] = h
 * x, dt, z, y are [B][T][Dm]; Bm, Cm are [B][T][N]; y rows t >= len and
 * padded rows are not written. */
int orc_mamba_scan(int B, int T, int Dm, int N, int num_slots, const double *x,
                   const double *dt, const double *A, const double *Bm,
                   const double *Cm, const double *Dv, const double *z,
                   double *hpool, const int32_t *idx, const int32_t *lengths,
                   int zero_init, double *y)
{
    if (B < 0 || T < 0 || Dm < 1 || N < 1 || num_slots < 1)
        return ORC_BAD;
#pragma omp parallel for collapse(2) schedule(static)
    for (int bi = 0; bi < B; ++bi) {
        for (int d = 0; d < Dm; ++d) {
            const int s = idx[bi];
            if (s < 0 || s >= num_slots)
                continue;
            int len = lengths ? lengths[bi] : T;
            if (len < 0)
                len = 0;
            if (len > T)
                len = T;
            double *h = hpool + ((size_t)s * Dm + d) * (size_t)N;
            if (zero_init)
                for (int n = 0; n < N; ++n)
                    h[n] = 0.0;
            for (int t = 0; t < len; ++t) {
                const size_t bt = (size_t)bi * T + t;
                const double xv = x[bt * Dm + d];
                const double dtv = dt[bt * Dm + d];
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    const double dA = exp(dtv * A[(size_t)d * N + n]);
                    const double dB = dtv * Bm[bt * N + n];
                    h[n] = dA * h[n] + dB * xv;
                    acc += Cm[bt * N + n] * h[n];
                }
                if (Dv)
                    acc += Dv[d] * xv;
                if (z)
                    acc *= orc_silu(z[bt * Dm + d]);
                y[bt * Dm + d] = acc;
            }
        }
    }
    return ORC_OK;
}

/* thread count for the parallel loops above (timing runs only: the
   arithmetic of every unit is the same at any count); n < 1 is ignored */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* number of OpenMP threads the parallel loops above use */
int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
