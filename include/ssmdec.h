/*
 * ssmdec.h -- C ABI of the MI355X (gfx950) single-token recurrent decode
 * library for gated linear-attention layers: the gated delta rule (GDN /
 * DeltaNet / KDA) over an fp32 state pool, updated in place.
 *
 * Sources (web pages, cited by title and section):
 *   [REPLAY] "Microbenchmark: buffered output-only GDN decode (ReplaySSM
 *            Part A) vs. the existing packed GDN decode kernel"
 *   [KDA]    "Microbenchmark for the fused Kimi-K3 KDA decode kernel on ROCm"
 *   [LOG]    "Optimization Log: Qwen3.5-27B Dense on B200"
 *   [MBU]    "Triton decode kernel + MBU analysis"
 *
 * Conventions for every call:
 *   - Every pointer argument is a DEVICE pointer (memory of the current HIP
 *     device), except where stated. The caller allocates and owns all
 *     buffers (mamba_scan's optional workspace included); the library never
 *     allocates, frees or keeps memory between calls.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream). No
 *     call synchronises, reads device memory on the host or allocates, so
 *     every call can be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is launched. On
 *     error nothing is launched, the call returns a negative SSMD_ERR_* code
 *     and ssmd_last_error() describes it.
 *   - Out-of-range slot indices are not errors: they mark padded rows, which
 *     read and write nothing (their `out` rows are left as they were). Two
 *     active rows naming the same slot in one call is a precondition
 *     violation with an undefined result.
 *   - Activation tensors (dtype SSMD_BF16 / SSMD_F16 / SSMD_F32) have no
 *     alignment requirement beyond their element size; rows aligned to 4
 *     elements take a faster vector-load path. fp32 states must be 16-byte
 *     aligned.
 *   - Calls are reentrant; the only global state is the thread-local error
 *     string.
 */
#ifndef SSMDEC_H
#define SSMDEC_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SSMD_OK 0
#define SSMD_ERR_NULL_ARG (-1)    /* a required pointer is NULL */
#define SSMD_ERR_BAD_SHAPE (-2)   /* sizes, strides or alignment are inconsistent */
#define SSMD_ERR_BAD_DTYPE (-3)   /* unknown dtype or activation code */
#define SSMD_ERR_UNSUPPORTED (-4) /* head size not compiled in, or an input with no defined meaning */
#define SSMD_ERR_LAUNCH (-5)      /* the HIP runtime refused the launch */

/* element types */
#define SSMD_F32 0
#define SSMD_BF16 1
#define SSMD_F16 2

/* gate activation of the output gated RMSNorm */
#define SSMD_ACT_SILU 0
#define SSMD_ACT_SIGMOID 1

/*
 * gdn_decode_step -- one packed GDN decode step for B rows.
 *
 * Defines ([REPLAY] module docstring, `_make_static`, `_bench_cfg`; [LOG]
 * "Kernel 4: Fused DeltaNet Recurrent", Math): for every row b whose slot
 * s = ssm_state_indices[b] is in [0, num_slots), and every value head hv
 * (q/k head h = hv / (HV/H)):
 *   q, k  = the h-th K-slices of the q and k blocks of mixed_qkv[b];
 *   v     = the hv-th V-slice of its v block;
 *   if use_qk_l2norm: q <- q / sqrt(|q|^2 + l2norm_eps), same for k;
 *   q    <- scale * q;
 *   g     = -exp(A_log[hv]) * softplus(a[b,hv] + dt_bias[hv]);
 *   beta  = sigmoid(b[b,hv]);
 *   S     = state[s, hv]                (V x K, row = value index)
 *   S    <- exp(g) S;  delta = beta (v - S k);  S <- S + delta k^T;  o = S q;
 *   if norm_gate: o <- o / sqrt(mean(o^2) + norm_eps) * w * act(norm_gate[b,hv])
 *                 (w = norm_weight, or ones when NULL; act per norm_act);
 *   out[b, 0, hv, :] = o (rounded to out_dtype, RNE).
 *
 * Arguments and layouts (row-major):
 *   mixed_qkv  [B, row stride qkv_row_stride >= 2*H*K + HV*V] act_dtype:
 *              q heads (H*K) | k heads (H*K) | v heads (HV*V)
 *   a, b       [B, HV] act_dtype gate logits (contiguous)
 *   A_log      [HV] fp32;  dt_bias [HV] fp32
 *   state      [num_slots, HV, V, K] fp32, updated in place
 *   ssm_state_indices [B] int32
 *   out        [B, 1, HV, V] out_dtype
 *   norm_gate  [B, HV, V] act_dtype or NULL (no output norm)
 *   norm_weight [V] fp32 or NULL (ones)
 *   K in {16, 32, 64, 128, 256}; 1 <= V <= 1024; HV % H == 0; B >= 0 (B == 0
 *   is a no-op).
 */
int gdn_decode_step(const void* mixed_qkv, int64_t qkv_row_stride,
                    const void* a, const void* b,
                    const float* A_log, const float* dt_bias,
                    float* state, int32_t num_slots,
                    const int32_t* ssm_state_indices,
                    void* out,
                    int32_t B, int32_t H, int32_t HV, int32_t K, int32_t V,
                    int32_t act_dtype, int32_t out_dtype,
                    float scale, int32_t use_qk_l2norm, float l2norm_eps,
                    const void* norm_gate, const float* norm_weight,
                    float norm_eps, int32_t norm_act,
                    hipStream_t stream);

/*
 * gdn_decode_step_state16 -- gdn_decode_step on a state pool stored in 16-bit
 * floats. "Optimization Log: Qwen3.5-27B Dense on B200" ("Kernel 4: Fused
 * DeltaNet Recurrent") sizes the per-head state as a 16-bit [128, 128] tile;
 * storing it so halves the dominant traffic of the step.
 *
 * Computes exactly what gdn_decode_step computes, in fp32, from the state
 * read as 16-bit values; the updated rows are rounded (RNE) to state_dtype
 * once, when they are stored, and this step's output is formed from the
 * unrounded update. state is [num_slots, HV, V, K] of state_dtype
 * (SSMD_BF16 or SSMD_F16), 16-byte aligned. All other arguments, layouts and
 * conventions are those of gdn_decode_step.
 */
int gdn_decode_step_state16(const void* mixed_qkv, int64_t qkv_row_stride,
                            const void* a, const void* b,
                            const float* A_log, const float* dt_bias,
                            void* state, int32_t state_dtype, int32_t num_slots,
                            const int32_t* ssm_state_indices,
                            void* out,
                            int32_t B, int32_t H, int32_t HV, int32_t K, int32_t V,
                            int32_t act_dtype, int32_t out_dtype,
                            float scale, int32_t use_qk_l2norm, float l2norm_eps,
                            const void* norm_gate, const float* norm_weight,
                            float norm_eps, int32_t norm_act,
                            hipStream_t stream);

/*
 * gdn_decode_step_buffered -- the GDN step with the state written back only
 * once every L steps ([REPLAY] module docstring, `_bench_cfg`,
 * `_state_bytes_per_step`, `_amortize`).
 *
 * The pool `state` holds a checkpoint. Per row b with phase p = write_pos[b]
 * (0 <= p < L; other values pad the row), the ring holds the records of
 * phases 0..p-1 of the current cycle:
 *   d_cache [num_slots, HV, L, V] act_dtype  -- that step's delta
 *   k_cache [num_slots, H,  L, K] act_dtype  -- that step's normalised key
 *                                               (one per q/k head)
 *   g_cache [num_slots, HV, L]    fp32       -- that step's log decay g
 * The call computes this step's output exactly as gdn_decode_step would from
 * the state S_{p-1} obtained by replaying records 0..p-1 on the checkpoint
 * (S <- exp(g_j) S + d_j k_j^T). For p < L-1 it appends this step's record
 * at position p (delta and k rounded RNE to act_dtype, g as fp32) and
 * leaves `state` as it is; for p == L-1 it writes the folded state S_p back
 * to `state` and appends no record (the next cycle starts at position 0, so
 * a record at L-1 would never be read). write_pos is read only: the caller
 * advances it to (p + 1) % L between calls. With L == 1 the call computes
 * what gdn_decode_step computes. Ring entries past p, and the whole ring
 * after a flush, are don't-care; a zeroed ring with write_pos = 0 is a cold
 * start.
 * L is 1..64 (else SSMD_ERR_BAD_SHAPE), and the ring's staging must fit the
 * kernel's shared memory: 4 ((L-1)(K + R + 4) + 1 + 2R) <= 61440 bytes, with
 * R = V when norm_gate is given and otherwise the row-tile height (128 rows
 * for K = 64 and 128, 64 for K = 16, 32 and 256); past it the call returns
 * SSMD_ERR_UNSUPPORTED (without the norm: L <= 59 at K = 128, L <= 48 at
 * K = 256).
 * All other arguments are those of gdn_decode_step.
 */
int gdn_decode_step_buffered(const void* mixed_qkv, int64_t qkv_row_stride,
                             const void* a, const void* b,
                             const float* A_log, const float* dt_bias,
                             float* state, int32_t num_slots,
                             const int32_t* ssm_state_indices,
                             void* out,
                             int32_t B, int32_t H, int32_t HV, int32_t K, int32_t V,
                             int32_t act_dtype, int32_t out_dtype,
                             float scale, int32_t use_qk_l2norm, float l2norm_eps,
                             const void* norm_gate, const float* norm_weight,
                             float norm_eps, int32_t norm_act,
                             void* d_cache, void* k_cache, float* g_cache,
                             const int32_t* write_pos, int32_t L,
                             hipStream_t stream);

/*
 * gdn_fused_recurrent -- the GDN step over T tokens per sequence: for every
 * row b with slot s = ssm_state_indices[b] in [0, num_slots) and
 * len = lengths[b] clamped to [0, T] (lengths NULL: len = T), tokens
 * t = 0..len-1 are each one gdn_decode_step, in order, on the same state
 * ([LOG] "Kernel 4: Fused DeltaNet Recurrent", Math, run over a token axis;
 * the multi-token use of [MBU] "Prefill path"). The state is read and
 * written once per call, not once per token; the result is that of len
 * consecutive gdn_decode_step calls up to rounding. Tokens t >= len and
 * padded rows write no output; a row with len = 0 leaves its state as it is.
 *   mixed_qkv  [B*T rows, row stride qkv_row_stride >= 2*H*K + HV*V]
 *              act_dtype; token t of row b is row b*T + t
 *   a, b       [B, T, HV] act_dtype
 *   out        [B, T, HV, V] out_dtype
 *   norm_gate  [B, T, HV, V] act_dtype or NULL; with it V must not exceed
 *              what one 8-wave block holds: 256 for K = 64 and 128, 128
 *              for K = 16, 32 and 256
 *   T >= 0. All other arguments, layouts and conventions are those of
 *   gdn_decode_step.
 */
int gdn_fused_recurrent(const void* mixed_qkv, int64_t qkv_row_stride,
                        const void* a, const void* b,
                        const float* A_log, const float* dt_bias,
                        float* state, int32_t num_slots,
                        const int32_t* ssm_state_indices, const int32_t* lengths,
                        void* out,
                        int32_t B, int32_t T, int32_t H, int32_t HV, int32_t K, int32_t V,
                        int32_t act_dtype, int32_t out_dtype,
                        float scale, int32_t use_qk_l2norm, float l2norm_eps,
                        const void* norm_gate, const float* norm_weight,
                        float norm_eps, int32_t norm_act,
                        hipStream_t stream);

/*
 * gdn_chunk_prefill -- what gdn_fused_recurrent computes (the GDN step over T
 * tokens per row, state read and written once), in chunked form for long
 * sequences: tokens in chunks of 64, each chunk's effect reduced to dense
 * products (the Gram products and M = (I + A)^-1 of the chunk's unit
 * lower-triangular system) that run in parallel over chunks, then one pass
 * per tile of state rows walks the chunks in order (Delta^T = M (beta v -
 * beta e^gamma k S^T), o = e^gamma q S^T + P Delta^T, S <- e^gamma_C S +
 * Delta e^(gamma_C - gamma) k). [LOG] "Kernel 4: Fused DeltaNet
 * Recurrent", Math, unrolled over a chunk; [MBU] "Prefill path". The result
 * equals that of gdn_fused_recurrent up to rounding.
 *   Arguments, layouts and conventions: those of gdn_fused_recurrent, plus
 *   workspace (device, 16-byte aligned, caller-owned, contents don't-care
 *   on entry and exit) of at least gdn_chunk_workspace_bytes(B, T, HV, K, V,
 *   norm_gate != NULL) bytes. K in {64, 128}; V a multiple of 16, <= 256.
 */
int64_t gdn_chunk_workspace_bytes(int32_t B, int32_t T, int32_t HV, int32_t K, int32_t V, int32_t with_norm);
int gdn_chunk_prefill(const void* mixed_qkv, int64_t qkv_row_stride,
                      const void* a, const void* b,
                      const float* A_log, const float* dt_bias,
                      float* state, int32_t num_slots,
                      const int32_t* ssm_state_indices, const int32_t* lengths,
                      void* out,
                      int32_t B, int32_t T, int32_t H, int32_t HV, int32_t K, int32_t V,
                      int32_t act_dtype, int32_t out_dtype,
                      float scale, int32_t use_qk_l2norm, float l2norm_eps,
                      const void* norm_gate, const float* norm_weight,
                      float norm_eps, int32_t norm_act,
                      void* workspace, int64_t workspace_bytes,
                      hipStream_t stream);

/*
 * gdn_chunk_prefill_noalloc -- gdn_chunk_prefill for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, arguments,
 * layouts and conventions, without the workspace arguments. The workspace is
 * instead a fixed array of SSMD_CHUNK_SCRATCH_BYTES in device memory that the
 * library holds on each device it runs on until the process ends; the call
 * allocates and frees nothing. Limits and behaviour:
 *   - a call needing more than SSMD_CHUNK_SCRATCH_BYTES of workspace
 *     (gdn_chunk_workspace_bytes of its sizes) returns SSMD_ERR_BAD_SHAPE
 *     and launches nothing; 128 MiB holds the records of, e.g., one
 *     4096-token row at HV = 32, or one 2048-token row with the gated norm;
 *   - every call on a device shares that device's array: calls that can run
 *     at the same time on one device (other streams, other threads) race on
 *     it and must be ordered by the caller; the array's contents are
 *     don't-care on entry and exit, so nothing needs clearing;
 *   - the first call on a device looks up the array's device address
 *     (hipGetSymbolAddress); make that first call outside stream capture.
 */
#define SSMD_CHUNK_SCRATCH_BYTES (128LL << 20)
int gdn_chunk_prefill_noalloc(const void* mixed_qkv, int64_t qkv_row_stride,
                              const void* a, const void* b,
                              const float* A_log, const float* dt_bias,
                              float* state, int32_t num_slots,
                              const int32_t* ssm_state_indices, const int32_t* lengths,
                              void* out,
                              int32_t B, int32_t T, int32_t H, int32_t HV, int32_t K, int32_t V,
                              int32_t act_dtype, int32_t out_dtype,
                              float scale, int32_t use_qk_l2norm, float l2norm_eps,
                              const void* norm_gate, const float* norm_weight,
                              float norm_eps, int32_t norm_act,
                              hipStream_t stream);

/*
 * gdn_decode_step_conv -- gdn_decode_step with the causal conv1d update + SiLU
 * of its q, k and v channels fused in front, in one launch (the fused op of
 * [KDA] module docstring and `triton_chain` applied to the GDN step; [LOG]
 * "Kernel 5: Fused Causal Conv1d Update" and "Integration" place the conv
 * between the input projection and the recurrence).
 *
 * For every row b whose slot s = ssm_state_indices[b] is in [0, num_slots)
 * and every channel c < C = 2*H*K + HV*V:
 *   window = [conv_state[s, c, 0..W-2], x[b, c]]  (oldest first)
 *   y[c]   = silu(sum_j conv_weight[c, j] window[j] + conv_bias[c])
 *   conv_state[s, c, :] <- window[1..W-1]         (bit-exact shift)
 * then gdn_decode_step on mixed_qkv[b] = y (kept in fp32, never rounded to
 * act_dtype). Padded rows touch neither state nor conv_state nor out.
 *   x            [B, row stride x_row_stride >= C] act_dtype, pre-conv,
 *                q heads | k heads | v heads as mixed_qkv of gdn_decode_step
 *   conv_weight  [C, W] fp32; conv_bias [C] fp32 or NULL
 *   conv_state   logical [num_slots, C, W-1] act_dtype at element strides
 *                (cs_slot_stride, cs_chan_stride, cs_tap_stride), as in
 *                kda_decode_step (SD and DS layouts alike)
 *   2 <= W <= 8; HV / H <= 16 and (HV / H) * V <= 4096 (one block holds a
 *   q/k head's whole group of value heads). All other arguments, layouts and
 *   conventions are those of gdn_decode_step.
 */
int gdn_decode_step_conv(const void* x, int64_t x_row_stride,
                         const float* conv_weight, const float* conv_bias,
                         void* conv_state, int64_t cs_slot_stride,
                         int64_t cs_chan_stride, int64_t cs_tap_stride, int32_t W,
                         const void* a, const void* b,
                         const float* A_log, const float* dt_bias,
                         float* state, int32_t num_slots,
                         const int32_t* ssm_state_indices,
                         void* out,
                         int32_t B, int32_t H, int32_t HV, int32_t K, int32_t V,
                         int32_t act_dtype, int32_t out_dtype,
                         float scale, int32_t use_qk_l2norm, float l2norm_eps,
                         const void* norm_gate, const float* norm_weight,
                         float norm_eps, int32_t norm_act,
                         hipStream_t stream);

/*
 * kda_decode_step -- the fused KDA decode op: causal conv1d update + SiLU,
 * per-key-channel gated delta rule, sigmoid-gated RMSNorm, in one launch
 * ([KDA] module docstring, `triton_chain` and `fused`, `_gated_rmsnorm`;
 * [LOG] "Kernel 5: Fused Causal Conv1d Update").
 *
 * Per token t with slot s = state_indices[t] in [1, num_slots) (slot 0 is the
 * NULL block and is skipped, as are out-of-range slots), channel
 * c < C = 3*H*D:
 *   window = [conv_state[s, c, 0..W-2], x[t, c]]  (oldest first)
 *   y[c]   = silu(sum_j conv_weight[c, j] window[j] + conv_bias[c])
 *   conv_state[s, c, :] <- window[1..W-1]
 * y = [q | k | v], each [H, D]. Per head h:
 *   if use_qk_l2norm: q, k L2-normalised (eps l2norm_eps); q <- scale * q;
 *   g[i]  = lower_bound * sigmoid(raw_g[t,h,i])   (per key channel i; the
 *           workload's gate, lower_bound = -5);
 *   beta  = sigmoid(raw_beta[t, h]);
 *   S = state[s, h] (D x D, row = value index):
 *   S <- S diag(exp(g)); delta = beta (v - S k); S <- S + delta k^T; o = S q;
 *   if output_gate: o <- o / sqrt(mean(o^2) + norm_eps) * w * sigmoid(output_gate[t,h])
 *   out[t, h, :] = o (bf16 when out_dtype = SSMD_BF16, etc.)
 *
 *   x            [T, C] act_dtype (contiguous)
 *   conv_weight  [C, W] fp32; conv_bias [C] fp32 or NULL
 *   conv_state   logical [num_slots, C, W-1] act_dtype at element strides
 *                (cs_slot_stride, cs_chan_stride, cs_tap_stride): the SD
 *                layout [num_slots, W-1, C] has strides ((W-1)*C, 1, C),
 *                the DS layout [num_slots, C, W-1] has (C*(W-1), W-1, 1)
 *   raw_g        [T, H, D] act_dtype; raw_beta [T, H] act_dtype
 *   A_log, dt_bias: must be NULL. [KDA] `Inputs` and `fused` pass an A_log
 *                [H] and a dt_bias [H*D] to the op without stating how they
 *                enter the gate; rather than give them a meaning no page
 *                fixes, a call with either non-NULL returns
 *                SSMD_ERR_UNSUPPORTED and launches nothing.
 *   state        [num_slots, H, D, D] fp32, in place
 *   out          [T, H, D] out_dtype
 *   output_gate  [T, H, D] act_dtype or NULL (no norm); norm_weight [D] fp32 or NULL
 *   D in {16, 32, 64, 128, 256}; 2 <= W <= 8; T >= 0.
 */
int kda_decode_step(const void* x,
                    const float* conv_weight, const float* conv_bias,
                    void* conv_state, int64_t cs_slot_stride,
                    int64_t cs_chan_stride, int64_t cs_tap_stride,
                    const void* raw_g, const void* raw_beta,
                    const float* A_log, const float* dt_bias,
                    float lower_bound,
                    float* state, int32_t num_slots,
                    const int32_t* state_indices,
                    void* out,
                    const void* output_gate, const float* norm_weight,
                    float norm_eps,
                    int32_t T, int32_t H, int32_t D, int32_t W,
                    int32_t act_dtype, int32_t out_dtype,
                    float scale, int32_t use_qk_l2norm, float l2norm_eps,
                    hipStream_t stream);

/*
 * mamba_decode_step -- one Mamba-1 selective-scan decode step (the diagonal
 * relative of the delta rule), "Triton decode kernel + MBU analysis",
 * "Kernel design". For every row b whose slot s = state_indices[b] is in
 * [0, num_slots), and every channel d < Dm, with h = state[s, d, :] (N wide):
 *   dA = exp(dt[b,d] * A[d,:]);  dB = dt[b,d] * Bm[b,:]
 *   h <- dA * h + dB * x[b,d]                    (state updated in place)
 *   y  = sum_n Cm[b,n] h[n] + Dvec[d] x[b,d]     (Dvec NULL: no skip term)
 *   y *= silu(z[b,d])                            (z NULL: no gate)
 *   out[b,d] = y (out_dtype, RNE)
 * dt is taken as given (already positive). The page's kernel allocates a
 * fresh state each call; here the state is a slot pool updated in place, as
 * in the other calls.
 *   x, dt, z [B, Dm] act_dtype;  Bm, Cm [B, N] act_dtype;  A [Dm, N] fp32
 *   (16-byte aligned);  Dvec [Dm] fp32;  state [num_slots, Dm, N] fp32;
 *   out [B, Dm] out_dtype;  N in {16, 32, 64, 128, 256}; B >= 0.
 */
int mamba_decode_step(const void* x, const void* dt, const float* A,
                      const void* Bm, const void* Cm, const float* Dvec,
                      const void* z, float* state, int32_t num_slots,
                      const int32_t* state_indices, void* out,
                      int32_t B, int32_t Dm, int32_t N,
                      int32_t act_dtype, int32_t out_dtype,
                      hipStream_t stream);

/*
 * mamba_scan -- Mamba-1 over T tokens per row (prefill): the recurrence of
 * mamba_decode_step applied to tokens 0..len-1 of each row in order, the
 * state carried from token to token ([MBU] "Prefill path", a multi-token scan
 * of the "Kernel design" recurrence). For every row b whose slot
 * s = state_indices[b] is in [0, num_slots), with len = lengths[b] clamped to
 * [0, T] (lengths NULL: len = T) and every channel d:
 *   h = zero_init ? 0 : state[s, d, :]
 *   for t < len:  h <- exp(dt[b,t,d] A[d,:]) h + dt[b,t,d] Bm[b,t,:] x[b,t,d]
 *                 out[b,t,d] = (Cm[b,t,:] . h + Dvec[d] x[b,t,d]) * silu(z[b,t,d])
 *                 (Dvec NULL: no skip term; z NULL: no gate)
 *   state[s, d, :] = h
 * out rows t >= len are not written; padded rows touch nothing.
 *   x, dt, z [B, T, Dm] act_dtype;  Bm, Cm [B, T, N] act_dtype;
 *   A [Dm, N] fp32 (16-byte aligned);  Dvec [Dm] fp32;
 *   state [num_slots, Dm, N] fp32 (16-byte aligned), in place;
 *   lengths [B] int32 or NULL;  out [B, T, Dm] out_dtype;
 *   N in {16, 32, 64, 128, 256};  0 <= B <= 65535;  T >= 0.
 * workspace (device, 16-byte aligned, caller-owned, contents don't-care on
 * entry and exit) lets the scan split T into chunks that run in parallel
 * (scan each chunk from zero, carry the chunk boundaries in order, rescan
 * each chunk from its true start): mamba_scan_workspace_bytes() gives the
 * size that reaches full parallelism on the current device. With less (or
 * NULL / 0) the call uses as many chunks as fit, down to one sequential pass;
 * the result is the same up to rounding.
 */
int64_t mamba_scan_workspace_bytes(int32_t B, int32_t T, int32_t Dm, int32_t N);
int mamba_scan(const void* x, const void* dt, const float* A,
               const void* Bm, const void* Cm, const float* Dvec,
               const void* z, float* state, int32_t num_slots,
               const int32_t* state_indices, const int32_t* lengths,
               int32_t zero_init, void* out,
               void* workspace, int64_t workspace_bytes,
               int32_t B, int32_t T, int32_t Dm, int32_t N,
               int32_t act_dtype, int32_t out_dtype,
               hipStream_t stream);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* ssmd_last_error(void);

/*
 * ssmd_stream_copy -- measurement aid: copies `bytes` (a multiple of 16) from
 * src to dst with the same 128-bit load/store pattern as the decode kernels.
 * A read-once/write-once stream of equal sizes gives the practical HBM
 * ceiling a decode step (equal state read and write) can be compared with.
 */
int ssmd_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/*
 * ssmd_check_slot_indices -- debug check of a slot-index vector before a
 * decode call. Every step above reads and writes the slot its row names, so
 * two active rows naming one slot in a call race on it (the result is
 * undefined); the pages' pools ([REPLAY] `_bench_cfg`, [KDA] `Inputs`) give
 * each active row its own slot. This counts the active rows whose slot an
 * earlier active row already names and writes the count to *dup_count
 * (0: the vector is valid).
 *
 *   slot_indices [B] int32 (device); 0 <= B <= 65536 (B == 0 writes 0)
 *   num_slots    pool size: indices outside [0, num_slots) are padded rows
 *   null_slot_zero  non-zero for kda_decode_step's convention, where slot 0
 *                is the NULL block and pads the row too
 *   dup_count    [1] int32 (device), written by the kernel on `stream`
 *
 * One workgroup compares each row with every earlier one (O(B^2)): a debug
 * aid, not meant for the timed path. Enqueued asynchronously like the
 * steps; the caller reads *dup_count after synchronising. Errors:
 * SSMD_ERR_NULL_ARG, SSMD_ERR_BAD_SHAPE (B outside [0, 65536], num_slots < 1,
 * misaligned pointers), SSMD_ERR_LAUNCH.
 */
int ssmd_check_slot_indices(const int32_t* slot_indices, int32_t B, int32_t num_slots,
                            int32_t null_slot_zero, int32_t* dup_count, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSMDEC_H */
