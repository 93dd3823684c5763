// ssmd_api.hip -- the extern "C" entry points declared in include/ssmdec.h:
// host-side validation, launch-shape choice, and the stream-copy
// measurement aid. Nothing here touches device memory from the host,
// synchronises or allocates.
#include <atomic>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SSMD_OK;
}

bool valid_dtype(int d) { return d == SSMD_F32 || d == SSMD_BF16 || d == SSMD_F16; }
int dtype_bytes(int d) { return d == SSMD_F32 ? 4 : 2; }
bool head_size_ok(int k) { return k == 16 || k == 32 || k == 64 || k == 128 || k == 256; }
bool aligned(const void* p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

// Launch shape of the state-streaming kernels: 4 waves per block. The packed
// step without a norm runs persistent prefetching blocks, one per CU; the
// other kernels run one block per work unit. SSMD_TUNE="wpb[,grid_cap]"
// overrides it (read once) for launch-shape sweeps.
ssmd::Launch launch_for() {
  // read once; a function-local static is initialised exactly once even
  // when several host threads make their first call together
  static const ssmd::Launch l = [] {
    const char* e = getenv("SSMD_TUNE");
    int wpb = 0, cap = 0;
    const int n = e ? sscanf(e, "%d,%d", &wpb, &cap) : 0;
    return (n >= 1 && wpb >= 1 && wpb <= 8 && cap >= 0) ? ssmd::Launch{wpb, cap, 1} : ssmd::Launch{4, 0, 0};
  }();
  return l;
}

// Compute units of the current device, cached per device (a host-side query;
// nothing is enqueued, so it is safe under stream capture).
int cu_count(int* n) {
  // per-device cache; concurrent first calls store the same value
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(SSMD_ERR_LAUNCH, "hipGetDevice failed");
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *n = c;
      return SSMD_OK;
    }
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
    return fail(SSMD_ERR_LAUNCH, "cannot read the compute-unit count of device %d", dev);
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  *n = v;
  return SSMD_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSMD_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Checks shared by the two GDN entry points. Returns SSMD_OK or an error.
int check_gdn(const char* fn, const void* qkv, int64_t stride, const void* a, const void* b,
              const float* A_log, const float* dt_bias, const void* state, int32_t num_slots,
              const int32_t* idx, const void* out, int32_t B, int32_t H, int32_t HV, int32_t K,
              int32_t V, int32_t act, int32_t odt, const void* norm_gate, int32_t norm_act) {
  if (B < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: B = %d < 0", fn, B);
  if (H < 1 || HV < 1 || HV % H)
    return fail(SSMD_ERR_BAD_SHAPE, "%s: need H >= 1, HV >= 1 and HV %% H == 0 (H=%d HV=%d)", fn, H, HV);
  if (!head_size_ok(K)) return fail(SSMD_ERR_UNSUPPORTED, "%s: K = %d not in {16,32,64,128,256}", fn, K);
  if (V < 1 || V > 1024) return fail(SSMD_ERR_BAD_SHAPE, "%s: V = %d outside [1, 1024]", fn, V);
  if (num_slots < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: num_slots = %d < 1", fn, num_slots);
  if (!valid_dtype(act) || !valid_dtype(odt))
    return fail(SSMD_ERR_BAD_DTYPE, "%s: bad act/out dtype (%d, %d)", fn, act, odt);
  if (norm_act != SSMD_ACT_SILU && norm_act != SSMD_ACT_SIGMOID)
    return fail(SSMD_ERR_BAD_DTYPE, "%s: bad norm_act %d", fn, norm_act);
  if (B == 0) return SSMD_OK;
  if (!qkv || !a || !b || !A_log || !dt_bias || !state || !idx || !out)
    return fail(SSMD_ERR_NULL_ARG, "%s: a required pointer is NULL", fn);
  const int64_t need = 2LL * H * K + (int64_t)HV * V;
  if (stride < need)
    return fail(SSMD_ERR_BAD_SHAPE, "%s: qkv_row_stride %lld < 2*H*K + HV*V = %lld", fn, (long long)stride,
                (long long)need);
  if (!aligned(state, 16)) return fail(SSMD_ERR_BAD_SHAPE, "%s: state must be 16-byte aligned", fn);
  if ((int64_t)B * HV * ((V + 7) / 8) >= (1LL << 31))
    return fail(SSMD_ERR_BAD_SHAPE, "%s: B*HV too large for one launch", fn);
  (void)norm_gate;
  return SSMD_OK;
}

ssmd::GdnParams gdn_params(const void* qkv, int64_t stride, const void* a, const void* b,
                           const float* A_log, const float* dt_bias, void* state, int32_t num_slots,
                           const int32_t* idx, void* out, int32_t B, int32_t H, int32_t HV, int32_t K,
                           int32_t V, int32_t act, int32_t odt, float scale, int32_t use_l2,
                           float l2eps, const void* norm_gate, const float* norm_w, float norm_eps,
                           int32_t norm_act) {
  ssmd::GdnParams p{};
  p.qkv = qkv;
  p.qkv_stride = stride;
  p.qkv_vec = stride % 4 == 0 && aligned(qkv, 4 * dtype_bytes(act));
  p.a = a;
  p.b = b;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.state = state;
  p.state_dt = SSMD_F32;
  p.num_slots = num_slots;
  p.idx = idx;
  p.out = out;
  p.B = B;
  p.H = H;
  p.HV = HV;
  p.K = K;
  p.V = V;
  p.act_dt = act;
  p.out_dt = odt;
  p.scale = scale;
  p.use_l2 = use_l2 ? 1 : 0;
  p.l2eps = l2eps;
  p.norm_gate = norm_gate;
  p.norm_w = norm_w;
  p.norm_eps = norm_eps;
  p.norm_act = norm_act;
  return p;
}

// ------------------------------------------------------------- stream copy
// One 128-bit non-temporal load and store per iteration over a grid of a few
// blocks per CU: the fastest same-mix copy found on MI355X (a 2 GiB sweep of
// unroll depth, grid size and temporal/non-temporal access).
__global__ __launch_bounds__(256) void stream_copy_kernel(const ssmd::f4* __restrict__ src,
                                                          ssmd::f4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    ssmd::st4<true>(reinterpret_cast<float*>(dst + i), ssmd::ld4<true>(reinterpret_cast<const float*>(src + i)));
}

// Debug check of a slot-index vector: one block counts the active rows
// (lo <= idx < num_slots) whose slot an earlier active row already names,
// by direct comparison with every earlier row (O(B^2), a debug aid), and
// writes the count to *dups (no pre-zeroed memory needed).
__global__ __launch_bounds__(256) void check_slot_indices_kernel(const int32_t* __restrict__ idx, int32_t B,
                                                                 int32_t num_slots, int32_t lo,
                                                                 int32_t* __restrict__ dups) {
  __shared__ int total;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  int mine = 0;
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int s = idx[i];
    if (s < lo || s >= num_slots) continue;  // padded row
    for (int j = 0; j < i; ++j)
      if (idx[j] == s) {
        ++mine;
        break;
      }
  }
  if (mine) atomicAdd(&total, mine);  // LDS atomic
  __syncthreads();
  if (threadIdx.x == 0) *dups = total;
}

}  // namespace

namespace ssmd {
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int n_cu, hipStream_t st) {
  const int64_t n = bytes / 16;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4LL * n_cu) blocks = 4LL * n_cu;
  stream_copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(static_cast<const f4*>(src),
                                                                  static_cast<f4*>(dst), n);
  return hipGetLastError();
}
}  // namespace ssmd

extern "C" {

const char* ssmd_last_error(void) { return g_err; }

int gdn_decode_step(const void* mixed_qkv, int64_t qkv_row_stride, const void* a, const void* b,
                    const float* A_log, const float* dt_bias, float* state, int32_t num_slots,
                    const int32_t* ssm_state_indices, void* out, int32_t B, int32_t H, int32_t HV,
                    int32_t K, int32_t V, int32_t act_dtype, int32_t out_dtype, float scale,
                    int32_t use_qk_l2norm, float l2norm_eps, const void* norm_gate,
                    const float* norm_weight, float norm_eps, int32_t norm_act, hipStream_t stream) {
  int rc = check_gdn("gdn_decode_step", mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state,
                     num_slots, ssm_state_indices, out, B, H, HV, K, V, act_dtype, out_dtype,
                     norm_gate, norm_act);
  if (rc) return rc;
  if (B == 0) return ok();
  ssmd::GdnParams p = gdn_params(mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots,
                                 ssm_state_indices, out, B, H, HV, K, V, act_dtype, out_dtype, scale,
                                 use_qk_l2norm, l2norm_eps, norm_gate, norm_weight, norm_eps, norm_act);
  const ssmd::Launch l = launch_for();
  if (!norm_gate) {
    int n_cu = 0;
    if (int rc2 = cu_count(&n_cu)) return rc2;
    return launch_status(ssmd::launch_gdn_pf(p, l, n_cu, stream), "gdn_decode_step");
  }
  return launch_status(ssmd::launch_gdn(p, l, stream), "gdn_decode_step");
}

int gdn_decode_step_state16(const void* mixed_qkv, int64_t qkv_row_stride, const void* a, const void* b,
                            const float* A_log, const float* dt_bias, void* state, int32_t state_dtype,
                            int32_t num_slots, const int32_t* ssm_state_indices, void* out, int32_t B,
                            int32_t H, int32_t HV, int32_t K, int32_t V, int32_t act_dtype,
                            int32_t out_dtype, float scale, int32_t use_qk_l2norm, float l2norm_eps,
                            const void* norm_gate, const float* norm_weight, float norm_eps,
                            int32_t norm_act, hipStream_t stream) {
  const char* fn = "gdn_decode_step_state16";
  int rc = check_gdn(fn, mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots,
                     ssm_state_indices, out, B, H, HV, K, V, act_dtype, out_dtype, norm_gate, norm_act);
  if (rc) return rc;
  if (state_dtype != SSMD_BF16 && state_dtype != SSMD_F16)
    return fail(SSMD_ERR_BAD_DTYPE, "%s: state_dtype must be SSMD_BF16 or SSMD_F16 (got %d)", fn, state_dtype);
  if (B == 0) return ok();
  ssmd::GdnParams p = gdn_params(mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots,
                                 ssm_state_indices, out, B, H, HV, K, V, act_dtype, out_dtype, scale,
                                 use_qk_l2norm, l2norm_eps, norm_gate, norm_weight, norm_eps, norm_act);
  p.state_dt = state_dtype;
  int n_cu = 0;
  if (int rc2 = cu_count(&n_cu)) return rc2;
  return launch_status(ssmd::launch_gdn_s16(p, launch_for(), n_cu, stream), fn);
}

int gdn_decode_step_buffered(const void* mixed_qkv, int64_t qkv_row_stride, const void* a,
                             const void* b, const float* A_log, const float* dt_bias, float* state,
                             int32_t num_slots, const int32_t* ssm_state_indices, void* out,
                             int32_t B, int32_t H, int32_t HV, int32_t K, int32_t V,
                             int32_t act_dtype, int32_t out_dtype, float scale,
                             int32_t use_qk_l2norm, float l2norm_eps, const void* norm_gate,
                             const float* norm_weight, float norm_eps, int32_t norm_act,
                             void* d_cache, void* k_cache, float* g_cache, const int32_t* write_pos,
                             int32_t L, hipStream_t stream) {
  const char* fn = "gdn_decode_step_buffered";
  int rc = check_gdn(fn, mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots,
                     ssm_state_indices, out, B, H, HV, K, V, act_dtype, out_dtype, norm_gate, norm_act);
  if (rc) return rc;
  if (L < 1 || L > 64) return fail(SSMD_ERR_BAD_SHAPE, "%s: L = %d outside [1, 64]", fn, L);
  const ssmd::Launch l = launch_for();
  const int rpt = ssmd::buffered_rows_per_tile(K, V, norm_gate != nullptr, l);
  const size_t lds = ssmd::buffered_lds_bytes(K, rpt, L);
  if (lds > 60 * 1024)
    return fail(SSMD_ERR_UNSUPPORTED, "%s: ring staging needs %zu bytes of LDS (> 60 KiB); lower L", fn, lds);
  if (B == 0) return ok();
  if (!d_cache || !k_cache || !g_cache || !write_pos)
    return fail(SSMD_ERR_NULL_ARG, "%s: a ring pointer is NULL", fn);
  ssmd::GdnParams p = gdn_params(mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots,
                                 ssm_state_indices, out, B, H, HV, K, V, act_dtype, out_dtype, scale,
                                 use_qk_l2norm, l2norm_eps, norm_gate, norm_weight, norm_eps, norm_act);
  p.d_cache = d_cache;
  p.k_cache = k_cache;
  p.g_cache = g_cache;
  p.write_pos = write_pos;
  p.L = L;
  int n_cu = 0;
  if (int rc2 = cu_count(&n_cu)) return rc2;
  // the block width can only narrow here, so the LDS bound checked above holds
  const ssmd::Launch lb = ssmd::buffered_launch(K, norm_gate != nullptr, L, (int64_t)B * HV, n_cu, l);
  return launch_status(ssmd::launch_gdn_buffered(p, lb, stream), fn);
}

int gdn_decode_step_conv(const void* x, int64_t x_row_stride, const float* conv_weight,
                         const float* conv_bias, void* conv_state, int64_t cs_slot_stride,
                         int64_t cs_chan_stride, int64_t cs_tap_stride, int32_t W, const void* a,
                         const void* b, const float* A_log, const float* dt_bias, float* state,
                         int32_t num_slots, const int32_t* ssm_state_indices, void* out, int32_t B,
                         int32_t H, int32_t HV, int32_t K, int32_t V, int32_t act_dtype,
                         int32_t out_dtype, float scale, int32_t use_qk_l2norm, float l2norm_eps,
                         const void* norm_gate, const float* norm_weight, float norm_eps,
                         int32_t norm_act, hipStream_t stream) {
  const char* fn = "gdn_decode_step_conv";
  int rc = check_gdn(fn, x, x_row_stride, a, b, A_log, dt_bias, state, num_slots, ssm_state_indices,
                     out, B, H, HV, K, V, act_dtype, out_dtype, norm_gate, norm_act);
  if (rc) return rc;
  if (W < 2 || W > 8) return fail(SSMD_ERR_BAD_SHAPE, "%s: conv width W = %d outside [2, 8]", fn, W);
  if (HV / H > 16 || (int64_t)(HV / H) * V > 4096)
    return fail(SSMD_ERR_UNSUPPORTED, "%s: HV/H = %d > 16 or (HV/H)*V = %lld > 4096", fn, HV / H,
                (long long)(HV / H) * V);
  if (cs_slot_stride < 1 || cs_chan_stride < 1 || cs_tap_stride < 1)
    return fail(SSMD_ERR_BAD_SHAPE, "%s: conv-state strides must be positive", fn);
  if ((int64_t)B * H >= (1LL << 31)) return fail(SSMD_ERR_BAD_SHAPE, "%s: B*H too large", fn);
  if (B == 0) return ok();
  if (!conv_weight || !conv_state) return fail(SSMD_ERR_NULL_ARG, "%s: conv_weight or conv_state is NULL", fn);
  ssmd::GdnConvParams cp{};
  cp.g = gdn_params(x, x_row_stride, a, b, A_log, dt_bias, state, num_slots, ssm_state_indices, out, B,
                    H, HV, K, V, act_dtype, out_dtype, scale, use_qk_l2norm, l2norm_eps, norm_gate,
                    norm_weight, norm_eps, norm_act);
  cp.conv_w = conv_weight;
  cp.conv_b = conv_bias;
  cp.conv_state = conv_state;
  cp.cs_slot = cs_slot_stride;
  cp.cs_chan = cs_chan_stride;
  cp.cs_tap = cs_tap_stride;
  cp.W = W;
  int n_cu = 0;
  if (int rc2 = cu_count(&n_cu)) return rc2;
  return launch_status(ssmd::launch_gdn_conv(cp, launch_for(), n_cu, stream), fn);
}

int gdn_fused_recurrent(const void* mixed_qkv, int64_t qkv_row_stride, const void* a, const void* b,
                        const float* A_log, const float* dt_bias, float* state, int32_t num_slots,
                        const int32_t* ssm_state_indices, const int32_t* lengths, void* out, int32_t B,
                        int32_t T, int32_t H, int32_t HV, int32_t K, int32_t V, int32_t act_dtype,
                        int32_t out_dtype, float scale, int32_t use_qk_l2norm, float l2norm_eps,
                        const void* norm_gate, const float* norm_weight, float norm_eps, int32_t norm_act,
                        hipStream_t stream) {
  const char* fn = "gdn_fused_recurrent";
  if (T < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: T = %d < 0", fn, T);
  if (B < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: B = %d < 0", fn, B);
  const int64_t rows = (int64_t)B * T;
  if (rows >= (1LL << 31)) return fail(SSMD_ERR_BAD_SHAPE, "%s: B*T too large", fn);
  int rc = check_gdn(fn, mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots, ssm_state_indices,
                     out, (int32_t)rows, H, HV, K, V, act_dtype, out_dtype, norm_gate, norm_act);
  if (rc) return rc;
  if ((int64_t)T * qkv_row_stride >= (1LL << 31) || (int64_t)T * HV * V >= (1LL << 31))
    return fail(SSMD_ERR_BAD_SHAPE, "%s: one row's T tokens exceed 2^31 elements", fn);
  if (norm_gate && V > ssmd::gdn_multi_max_norm_rows(K))
    return fail(SSMD_ERR_UNSUPPORTED, "%s: with the gated norm V = %d exceeds %d for K = %d", fn, V,
                ssmd::gdn_multi_max_norm_rows(K), K);
  if (rows == 0) return ok();
  int n_cu = 0;
  if (int rc2 = cu_count(&n_cu)) return rc2;
  ssmd::GdnMultiParams mp{};
  mp.g = gdn_params(mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots, ssm_state_indices, out, B,
                    H, HV, K, V, act_dtype, out_dtype, scale, use_qk_l2norm, l2norm_eps, norm_gate, norm_weight,
                    norm_eps, norm_act);
  mp.T = T;
  mp.lengths = lengths;
  return launch_status(ssmd::launch_gdn_multi(mp, launch_for(), n_cu, stream), fn);
}

int64_t gdn_chunk_workspace_bytes(int32_t B, int32_t T, int32_t HV, int32_t K, int32_t V, int32_t with_norm) {
  if (B < 0 || T < 0 || HV < 1 || V < 1) return fail(SSMD_ERR_BAD_SHAPE, "gdn_chunk_workspace_bytes: bad sizes");
  ok();
  return 4 * ssmd::gdn_chunk_workspace_floats(B, T, HV, K, V, with_norm != 0);
}

namespace {

// Body of the two chunked-prefill entry points: `workspace` is the caller's
// buffer, or (static_ws) NULL, meaning the library's static array.
int chunk_prefill(const char* fn, const void* mixed_qkv, int64_t qkv_row_stride, const void* a, const void* b,
                  const float* A_log, const float* dt_bias, float* state, int32_t num_slots,
                  const int32_t* ssm_state_indices, const int32_t* lengths, void* out, int32_t B, int32_t T,
                  int32_t H, int32_t HV, int32_t K, int32_t V, int32_t act_dtype, int32_t out_dtype, float scale,
                  int32_t use_qk_l2norm, float l2norm_eps, const void* norm_gate, const float* norm_weight,
                  float norm_eps, int32_t norm_act, void* workspace, int64_t workspace_bytes, bool static_ws,
                  hipStream_t stream) {
  if (T < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: T = %d < 0", fn, T);
  if (B < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: B = %d < 0", fn, B);
  const int64_t rows = (int64_t)B * T;
  if (rows >= (1LL << 31)) return fail(SSMD_ERR_BAD_SHAPE, "%s: B*T too large", fn);
  int rc = check_gdn(fn, mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots, ssm_state_indices,
                     out, (int32_t)rows, H, HV, K, V, act_dtype, out_dtype, norm_gate, norm_act);
  if (rc) return rc;
  if (K != 64 && K != 128) return fail(SSMD_ERR_UNSUPPORTED, "%s: K = %d not in {64, 128}", fn, K);
  if (V % 16 || V > 256) return fail(SSMD_ERR_UNSUPPORTED, "%s: V = %d must be a multiple of 16, <= 256", fn, V);
  if (rows == 0) return ok();
  if ((int64_t)B * HV * ((T + 63) / 64) >= (1LL << 31)) return fail(SSMD_ERR_BAD_SHAPE, "%s: too many chunks", fn);
  const int64_t need = 4 * ssmd::gdn_chunk_workspace_floats(B, T, HV, K, V, norm_gate != nullptr);
  if (static_ws) {
    if (need > (int64_t)SSMD_CHUNK_SCRATCH_BYTES)
      return fail(SSMD_ERR_BAD_SHAPE,
                  "%s: this call needs %lld bytes of workspace, more than the library's static %lld "
                  "(B * HV * ceil(T / 64) too large; use gdn_chunk_prefill with a workspace)",
                  fn, (long long)need, (long long)SSMD_CHUNK_SCRATCH_BYTES);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(SSMD_ERR_BAD_SHAPE, "%s: workspace of %lld bytes needed (got %lld)", fn, (long long)need,
                  (long long)workspace_bytes);
    if (!aligned(workspace, 16)) return fail(SSMD_ERR_BAD_SHAPE, "%s: workspace must be 16-byte aligned", fn);
  }
  int n_cu = 0;
  if (int rc2 = cu_count(&n_cu)) return rc2;
  if (static_ws) {
    const hipError_t e = ssmd::gdn_chunk_scratch(&workspace);
    if (e != hipSuccess)
      return fail(SSMD_ERR_LAUNCH, "%s: cannot find the static workspace on this device: %s", fn, hipGetErrorString(e));
  }
  ssmd::GdnChunkParams cp{};
  cp.g = gdn_params(mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots, ssm_state_indices, out, B,
                    H, HV, K, V, act_dtype, out_dtype, scale, use_qk_l2norm, l2norm_eps, norm_gate, norm_weight,
                    norm_eps, norm_act);
  cp.T = T;
  cp.lengths = lengths;
  cp.nck = (T + 63) / 64;
  cp.ws = static_cast<float*>(workspace);
  cp.obuf = norm_gate ? cp.ws + (ssmd::gdn_chunk_workspace_floats(B, T, HV, K, V, false)) : nullptr;
  return launch_status(ssmd::launch_gdn_chunk(cp, n_cu, stream), fn);
}

}  // namespace

int gdn_chunk_prefill(const void* mixed_qkv, int64_t qkv_row_stride, const void* a, const void* b,
                      const float* A_log, const float* dt_bias, float* state, int32_t num_slots,
                      const int32_t* ssm_state_indices, const int32_t* lengths, void* out, int32_t B,
                      int32_t T, int32_t H, int32_t HV, int32_t K, int32_t V, int32_t act_dtype,
                      int32_t out_dtype, float scale, int32_t use_qk_l2norm, float l2norm_eps,
                      const void* norm_gate, const float* norm_weight, float norm_eps, int32_t norm_act,
                      void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return chunk_prefill("gdn_chunk_prefill", mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state, num_slots,
                       ssm_state_indices, lengths, out, B, T, H, HV, K, V, act_dtype, out_dtype, scale,
                       use_qk_l2norm, l2norm_eps, norm_gate, norm_weight, norm_eps, norm_act, workspace,
                       workspace_bytes, false, stream);
}

int gdn_chunk_prefill_noalloc(const void* mixed_qkv, int64_t qkv_row_stride, const void* a, const void* b,
                              const float* A_log, const float* dt_bias, float* state, int32_t num_slots,
                              const int32_t* ssm_state_indices, const int32_t* lengths, void* out, int32_t B,
                              int32_t T, int32_t H, int32_t HV, int32_t K, int32_t V, int32_t act_dtype,
                              int32_t out_dtype, float scale, int32_t use_qk_l2norm, float l2norm_eps,
                              const void* norm_gate, const float* norm_weight, float norm_eps, int32_t norm_act,
                              hipStream_t stream) {
  return chunk_prefill("gdn_chunk_prefill_noalloc", mixed_qkv, qkv_row_stride, a, b, A_log, dt_bias, state,
                       num_slots, ssm_state_indices, lengths, out, B, T, H, HV, K, V, act_dtype, out_dtype, scale,
                       use_qk_l2norm, l2norm_eps, norm_gate, norm_weight, norm_eps, norm_act, nullptr, 0, true,
                       stream);
}

int kda_decode_step(const void* x, const float* conv_weight, const float* conv_bias, void* conv_state,
                    int64_t cs_slot_stride, int64_t cs_chan_stride, int64_t cs_tap_stride,
                    const void* raw_g, const void* raw_beta, const float* A_log, const float* dt_bias,
                    float lower_bound, float* state, int32_t num_slots, const int32_t* state_indices,
                    void* out, const void* output_gate, const float* norm_weight, float norm_eps,
                    int32_t T, int32_t H, int32_t D, int32_t W, int32_t act_dtype, int32_t out_dtype,
                    float scale, int32_t use_qk_l2norm, float l2norm_eps, hipStream_t stream) {
  const char* fn = "kda_decode_step";
  if (T < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: T = %d < 0", fn, T);
  if (H < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: H = %d < 1", fn, H);
  if (!head_size_ok(D)) return fail(SSMD_ERR_UNSUPPORTED, "%s: D = %d not in {16,32,64,128,256}", fn, D);
  if (W < 2 || W > 8) return fail(SSMD_ERR_BAD_SHAPE, "%s: conv width W = %d outside [2, 8]", fn, W);
  if (num_slots < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: num_slots = %d < 1", fn, num_slots);
  if (!valid_dtype(act_dtype) || !valid_dtype(out_dtype))
    return fail(SSMD_ERR_BAD_DTYPE, "%s: bad act/out dtype (%d, %d)", fn, act_dtype, out_dtype);
  if (cs_slot_stride < 1 || cs_chan_stride < 1 || cs_tap_stride < 1)
    return fail(SSMD_ERR_BAD_SHAPE, "%s: conv-state strides must be positive", fn);
  if ((int64_t)T * H >= (1LL << 31)) return fail(SSMD_ERR_BAD_SHAPE, "%s: T*H too large", fn);
  // The pages pass A_log and dt_bias to the fused op but state no formula for
  // them; the gate computed here is the workload's lower_bound *
  // sigmoid(raw_g), and a call that supplies either tensor is refused rather
  // than given a meaning no page fixes.
  if (A_log || dt_bias)
    return fail(SSMD_ERR_UNSUPPORTED,
                "%s: A_log / dt_bias must be NULL (no formula for them is defined; the gate is "
                "lower_bound * sigmoid(raw_g))", fn);
  if (T == 0) return ok();
  if (!x || !conv_weight || !conv_state || !raw_g || !raw_beta || !state || !state_indices || !out)
    return fail(SSMD_ERR_NULL_ARG, "%s: a required pointer is NULL", fn);
  if (!aligned(state, 16)) return fail(SSMD_ERR_BAD_SHAPE, "%s: state must be 16-byte aligned", fn);
  ssmd::KdaParams p{};
  p.x = x;
  p.conv_w = conv_weight;
  p.conv_b = conv_bias;
  p.conv_state = conv_state;
  p.cs_slot = cs_slot_stride;
  p.cs_chan = cs_chan_stride;
  p.cs_tap = cs_tap_stride;
  p.raw_g = raw_g;
  p.raw_g_vec = aligned(raw_g, 4 * dtype_bytes(act_dtype));
  p.raw_beta = raw_beta;
  p.lower_bound = lower_bound;
  p.state = state;
  p.num_slots = num_slots;
  p.idx = state_indices;
  p.out = out;
  p.gate = output_gate;
  p.norm_w = norm_weight;
  p.norm_eps = norm_eps;
  p.T = T;
  p.H = H;
  p.D = D;
  p.W = W;
  p.act_dt = act_dtype;
  p.out_dt = out_dtype;
  p.scale = scale;
  p.use_l2 = use_qk_l2norm ? 1 : 0;
  p.l2eps = l2norm_eps;
  if (ssmd::kda_pf_supported(p) && aligned(conv_weight, 16))
    return launch_status(ssmd::launch_kda_pf(p, launch_for(), stream), fn);
  return launch_status(ssmd::launch_kda(p, launch_for(), stream), fn);
}

int mamba_decode_step(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                      const float* Dvec, const void* z, float* state, int32_t num_slots,
                      const int32_t* state_indices, void* out, int32_t B, int32_t Dm, int32_t N,
                      int32_t act_dtype, int32_t out_dtype, hipStream_t stream) {
  const char* fn = "mamba_decode_step";
  if (B < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: B = %d < 0", fn, B);
  if (Dm < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: D = %d < 1", fn, Dm);
  if (!head_size_ok(N)) return fail(SSMD_ERR_UNSUPPORTED, "%s: N = %d not in {16,32,64,128,256}", fn, N);
  if (num_slots < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: num_slots = %d < 1", fn, num_slots);
  if (!valid_dtype(act_dtype) || !valid_dtype(out_dtype))
    return fail(SSMD_ERR_BAD_DTYPE, "%s: bad act/out dtype (%d, %d)", fn, act_dtype, out_dtype);
  if ((int64_t)B * ((Dm + 63) / 64) >= (1LL << 31)) return fail(SSMD_ERR_BAD_SHAPE, "%s: B*D too large", fn);
  if (B == 0) return ok();
  if (!x || !dt || !A || !Bm || !Cm || !state || !state_indices || !out)
    return fail(SSMD_ERR_NULL_ARG, "%s: a required pointer is NULL", fn);
  if (!aligned(A, 16) || !aligned(state, 16))
    return fail(SSMD_ERR_BAD_SHAPE, "%s: A and state must be 16-byte aligned", fn);
  ssmd::MambaParams p{};
  p.x = x;
  p.dt = dt;
  p.A = A;
  p.Bm = Bm;
  p.Cm = Cm;
  p.Dvec = Dvec;
  p.z = z;
  p.state = state;
  p.num_slots = num_slots;
  p.idx = state_indices;
  p.out = out;
  p.B = B;
  p.Dm = Dm;
  p.N = N;
  p.act_dt = act_dtype;
  p.out_dt = out_dtype;
  int n_cu = 0;
  if (int rc2 = cu_count(&n_cu)) return rc2;
  return launch_status(ssmd::launch_mamba(p, launch_for(), n_cu, stream), fn);
}

int64_t mamba_scan_workspace_bytes(int32_t B, int32_t T, int32_t Dm, int32_t N) {
  const char* fn = "mamba_scan_workspace_bytes";
  if (B < 0 || T < 0 || Dm < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: need B >= 0, T >= 0, D >= 1", fn);
  if (!head_size_ok(N)) return fail(SSMD_ERR_UNSUPPORTED, "%s: N = %d not in {16,32,64,128,256}", fn, N);
  int n_cu = 0;
  if (int rc = cu_count(&n_cu)) return rc;
  int Lc = 0, nck = 0;
  ssmd::mamba_scan_chunking(B, T, Dm, N, n_cu, INT64_MAX, &Lc, &nck);
  ok();
  return nck > 1 ? 2LL * B * nck * Dm * N * 4 : 0;
}

int mamba_scan(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
               const float* Dvec, const void* z, float* state, int32_t num_slots,
               const int32_t* state_indices, const int32_t* lengths, int32_t zero_init, void* out,
               void* workspace, int64_t workspace_bytes, int32_t B, int32_t T, int32_t Dm, int32_t N,
               int32_t act_dtype, int32_t out_dtype, hipStream_t stream) {
  const char* fn = "mamba_scan";
  if (B < 0 || B > 65535) return fail(SSMD_ERR_BAD_SHAPE, "%s: B = %d outside [0, 65535]", fn, B);
  if (T < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: T = %d < 0", fn, T);
  if (Dm < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: D = %d < 1", fn, Dm);
  if (!head_size_ok(N)) return fail(SSMD_ERR_UNSUPPORTED, "%s: N = %d not in {16,32,64,128,256}", fn, N);
  if (num_slots < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: num_slots = %d < 1", fn, num_slots);
  if (!valid_dtype(act_dtype) || !valid_dtype(out_dtype))
    return fail(SSMD_ERR_BAD_DTYPE, "%s: bad act/out dtype (%d, %d)", fn, act_dtype, out_dtype);
  if (workspace_bytes < 0) return fail(SSMD_ERR_BAD_SHAPE, "%s: workspace_bytes < 0", fn);
  if ((int64_t)T * Dm >= (1LL << 40)) return fail(SSMD_ERR_BAD_SHAPE, "%s: T*D too large", fn);
  if (B == 0) return ok();
  if (!A || !state || !state_indices) return fail(SSMD_ERR_NULL_ARG, "%s: A, state or state_indices is NULL", fn);
  if (T > 0 && (!x || !dt || !Bm || !Cm || !out))
    return fail(SSMD_ERR_NULL_ARG, "%s: x, dt, Bm, Cm or out is NULL", fn);
  if (!aligned(A, 16) || !aligned(state, 16))
    return fail(SSMD_ERR_BAD_SHAPE, "%s: A and state must be 16-byte aligned", fn);
  if (workspace_bytes > 0 && (!workspace || !aligned(workspace, 16)))
    return fail(SSMD_ERR_BAD_SHAPE, "%s: workspace must be a 16-byte aligned pointer when workspace_bytes > 0", fn);
  int n_cu = 0;
  if (int rc = cu_count(&n_cu)) return rc;
  ssmd::MambaScanParams p{};
  ssmd::mamba_scan_chunking(B, T, Dm, N, n_cu, workspace ? workspace_bytes : 0, &p.Lc, &p.nck);
  if (p.nck > 65535) return fail(SSMD_ERR_BAD_SHAPE, "%s: too many chunks (%d)", fn, p.nck);
  p.x = x;
  p.dt = dt;
  p.A = A;
  p.Bm = Bm;
  p.Cm = Cm;
  p.Dvec = Dvec;
  p.z = z;
  p.state = state;
  p.num_slots = num_slots;
  p.idx = state_indices;
  p.lengths = lengths;
  p.zero_init = zero_init ? 1 : 0;
  p.out = out;
  p.ws_P = static_cast<float*>(workspace);
  p.ws_h = p.nck > 1 ? p.ws_P + (int64_t)B * p.nck * Dm * N : nullptr;
  p.B = B;
  p.T = T;
  p.Dm = Dm;
  p.N = N;
  p.act_dt = act_dtype;
  p.out_dt = out_dtype;
  return launch_status(ssmd::launch_mamba_scan(p, n_cu, stream), fn);
}

int ssmd_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst) return fail(SSMD_ERR_NULL_ARG, "ssmd_stream_copy: NULL pointer");
  if (bytes < 0 || bytes % 16) return fail(SSMD_ERR_BAD_SHAPE, "ssmd_stream_copy: bytes must be a multiple of 16");
  if (!aligned(src, 16) || !aligned(dst, 16))
    return fail(SSMD_ERR_BAD_SHAPE, "ssmd_stream_copy: pointers must be 16-byte aligned");
  if (bytes == 0) return ok();
  int n_cu = 0;
  if (int rc = cu_count(&n_cu)) return rc;
  return launch_status(ssmd::launch_stream_copy(src, dst, bytes, n_cu, stream), "ssmd_stream_copy");
}

int ssmd_check_slot_indices(const int32_t* slot_indices, int32_t B, int32_t num_slots, int32_t null_slot_zero,
                            int32_t* dup_count, hipStream_t stream) {
  const char* fn = "ssmd_check_slot_indices";
  // one workgroup compares every pair: 65536 rows is about 2^31 comparisons
  if (B < 0 || B > 65536) return fail(SSMD_ERR_BAD_SHAPE, "%s: B = %d outside [0, 65536]", fn, B);
  if (num_slots < 1) return fail(SSMD_ERR_BAD_SHAPE, "%s: num_slots = %d < 1", fn, num_slots);
  if (!dup_count) return fail(SSMD_ERR_NULL_ARG, "%s: dup_count is NULL", fn);
  if (B > 0 && !slot_indices) return fail(SSMD_ERR_NULL_ARG, "%s: slot_indices is NULL", fn);
  if (!aligned(dup_count, 4) || (B > 0 && !aligned(slot_indices, 4)))
    return fail(SSMD_ERR_BAD_SHAPE, "%s: int32 pointers must be 4-byte aligned", fn);
  check_slot_indices_kernel<<<dim3(1), dim3(256), 0, stream>>>(slot_indices, B, num_slots, null_slot_zero ? 1 : 0,
                                                                dup_count);
  return launch_status(hipGetLastError(), fn);
}

}  // extern "C"
