// gdn_conv_decode_pf.hip -- conv-fused GDN decode step, persistent form:
// 8-wave blocks walk the (batch row, q/k head) groups with a grid stride and,
// while one group's conv and state rows are computed and stored, hold the
// next group's state rows, conv windows, conv weights and gates in flight
// (the launcher picks one block per CU or, for many groups, one per group). Same arithmetic, row layout and conv-state roll as
// gdn_conv_decode.hip, which handles every shape this kernel does not.
//
// The group is still the unit of work (its conv state is rolled in place by
// exactly one block), so the block covers a whole group: 8 waves x RG row
// groups x RPI rows = 256 rows, the G V rows of a group at G = 2, V = 128
// (or G V = 256 at K = 64), and its 2K + G V conv channels at one per thread.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

constexpr int GCPF_WAVES = 8;
constexpr int GCPF_THREADS = 64 * GCPF_WAVES;
constexpr int GCPF_RG = 4;  // row groups per wave per group: 32 rows at RPI = 8
constexpr int GCPF_GMAX = 16;  // largest GQA group G = HV / H

template <int K, int ACT, int WT>
__global__ __launch_bounds__(GCPF_THREADS) void gdn_conv_pf_kernel(GdnConvParams cp, int n_units) {
  const GdnParams& p = cp.g;
  using RL = RowLayout<K>;
  using T = typename std::conditional<ACT == SSMD_F32, float, uint16_t>::type;
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, RG = GCPF_RG;
  constexpr int ROWS = GCPF_WAVES * RG * RPI;  // rows of one group
  constexpr int NCH = 2 * K + ROWS;            // conv channels of one group
  static_assert(NCH <= GCPF_THREADS, "one conv channel per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  const int G = p.HV / p.H;
  const int V = p.V;
  // y[buffer][channel]: SiLU conv outputs of a group at fp32; consecutive
  // groups alternate buffers, so one barrier per group orders the writes of a
  // group after every read of the group two back
  __shared__ float y[2][NCH];
  __shared__ float gdecay[2][GCPF_GMAX], gbeta[2][GCPF_GMAX];

  T* const cs = static_cast<T*>(cp.conv_state);
  float* const pool = static_cast<float*>(p.state);
  // group-local channel ci -> channel of x: q of head h | k of head h | v of heads h G .. h G + G - 1
  auto chan = [&](int h, int ci) {
    return ci < K ? h * K + ci : (ci < 2 * K ? (p.H + h) * K + (ci - K) : 2 * p.H * K + h * ROWS + (ci - 2 * K));
  };
  // this thread's rows of a group: row R = (i * waves + wave) * RPI + rr, value head R / V
  auto row_of = [&](int i) { return (i * GCPF_WAVES + wave) * RPI + rr; };
  auto to_f = [](T v) -> float {
    if constexpr (ACT == SSMD_F32) return v;
    else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(v);
    else return f16_bits_to_f32(v);
  };

  struct Unit {
    int slot, bi, h;
    T raw[WT];       // conv window: taps 0 .. WT - 2 from the conv state, then x
    float wf[WT], cb;
    float av, bv, A_log, dt_bias;
    f4 s[RG][NV];
  };
  auto fetch = [&](int unit, Unit& U) {
    U.h = unit % p.H;
    U.bi = unit / p.H;
    U.slot = p.idx[U.bi];
    if (U.slot < 0 || U.slot >= p.num_slots) return;  // padded row: touch nothing
    const int gc = chan(U.h, min(tid, NCH - 1));
    const int64_t cso = (int64_t)U.slot * cp.cs_slot + (int64_t)gc * cp.cs_chan;
#pragma unroll
    for (int j = 0; j < WT - 1; ++j) U.raw[j] = cs[cso + (int64_t)j * cp.cs_tap];
    U.raw[WT - 1] = static_cast<const T*>(p.qkv)[(int64_t)U.bi * p.qkv_stride + gc];
#pragma unroll
    for (int j = 0; j < WT; ++j) U.wf[j] = cp.conv_w[(int64_t)gc * WT + j];
    U.cb = cp.conv_b ? cp.conv_b[gc] : 0.f;
    const int gh = U.h * G + min(tid, G - 1);
    const int64_t gidx = (int64_t)U.bi * p.HV + gh;
    U.av = ld_act<ACT>(p.a, gidx);
    U.bv = ld_act<ACT>(p.b, gidx);
    U.A_log = p.A_log[gh];
    U.dt_bias = p.dt_bias[gh];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int R = row_of(i);
      const int g = R / V;
      const float* S = pool + (((int64_t)U.slot * p.HV + U.h * G + g) * V + (R - g * V)) * (int64_t)K;
#pragma unroll
      for (int j = 0; j < NV; ++j) U.s[i][j] = ld4<true>(S + RL::col(c, j));
    }
  };
  auto compute = [&](Unit& U, int buf) {
    if (U.slot < 0 || U.slot >= p.num_slots) {  // uniform over the block
      __syncthreads();  // still one barrier per group: it orders the buffer reuse
      return;
    }
    float* const yb = y[buf];
    // conv output -> LDS, and roll the window: tap j <- window[j + 1], the newest tap <- x
    if (tid < NCH) {
      const int64_t cso = (int64_t)U.slot * cp.cs_slot + (int64_t)chan(U.h, tid) * cp.cs_chan;
      float acc = U.cb;
#pragma unroll
      for (int j = 0; j < WT; ++j) acc += U.wf[j] * to_f(U.raw[j]);
#pragma unroll
      for (int j = 0; j < WT - 1; ++j) cs[cso + (int64_t)j * cp.cs_tap] = U.raw[j + 1];
      yb[tid] = silu_f(acc);
    }
    if (tid < G) {
      const float g = -expf(U.A_log) * softplus_f(U.av + U.dt_bias);
      gdecay[buf][tid] = expf(g);
      gbeta[buf][tid] = sigmoid_f(U.bv);
    }
    __syncthreads();
    float qf[NV * 4], kf[NV * 4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[4 * j + e] = yb[RL::col(c, j) + e];
        kf[4 * j + e] = yb[K + RL::col(c, j) + e];
      }
    }
    float qs = p.scale, ks = 1.f;
    if (p.use_l2) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < NV * 4; ++e) {
        sq += qf[e] * qf[e];
        sk += kf[e] * kf[e];
      }
      sq = group_sum<LPR>(sq);
      sk = group_sum<LPR>(sk);
      qs *= rsqrtf(sq + p.l2eps);
      ks = rsqrtf(sk + p.l2eps);
    }
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < NV * 4; ++e) {
      qf[e] *= qs;
      kf[e] *= ks;
      kq += kf[e] * qf[e];
    }
    kq = group_sum<LPR>(kq);
    const int64_t obase = ((int64_t)U.bi * p.HV + U.h * G) * V;  // output row R of the group is obase + R
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int R = row_of(i);
      const int g = R / V;
      const float decay = gdecay[buf][g], beta = gbeta[buf][g];
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        dk += U.s[i][j].x * kf[4 * j] + U.s[i][j].y * kf[4 * j + 1] + U.s[i][j].z * kf[4 * j + 2] +
              U.s[i][j].w * kf[4 * j + 3];
        dq += U.s[i][j].x * qf[4 * j] + U.s[i][j].y * qf[4 * j + 1] + U.s[i][j].z * qf[4 * j + 2] +
              U.s[i][j].w * qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const float delta = beta * (yb[2 * K + R] - decay * dk);
      const float o = decay * dq + delta * kq;
      float* S = pool + (((int64_t)U.slot * p.HV + U.h * G + g) * V + (R - g * V)) * (int64_t)K;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        f4 n;
        n.x = decay * U.s[i][j].x + delta * kf[4 * j];
        n.y = decay * U.s[i][j].y + delta * kf[4 * j + 1];
        n.z = decay * U.s[i][j].z + delta * kf[4 * j + 2];
        n.w = decay * U.s[i][j].w + delta * kf[4 * j + 3];
        st4<true>(S + RL::col(c, j), n);
      }
      if (c == 0) store_act1(p.out, obase + R, p.out_dt, o);
    }
  };

  Unit A, B;
  int u = blockIdx.x;
  const int gs = gridDim.x;
  if (u < n_units) fetch(u, A);
  while (u < n_units) {
    if (u + gs < n_units) fetch(u + gs, B);
    compute(A, 0);
    if (u + gs >= n_units) break;
    if (u + 2 * gs < n_units) fetch(u + 2 * gs, A);
    compute(B, 1);
    u += 2 * gs;
  }
}

namespace {

template <int K, int ACT>
hipError_t launch_gcpf_k(const GdnConvParams& cp, int64_t blocks, int n_units, hipStream_t st) {
  gdn_conv_pf_kernel<K, ACT, 4><<<dim3((unsigned)blocks), dim3(GCPF_THREADS), 0, st>>>(cp, n_units);
  return hipGetLastError();
}

template <int K>
hipError_t launch_gcpf_act(const GdnConvParams& cp, int64_t blocks, int n_units, hipStream_t st) {
  switch (cp.g.act_dt) {
    case SSMD_F32: return launch_gcpf_k<K, SSMD_F32>(cp, blocks, n_units, st);
    case SSMD_BF16: return launch_gcpf_k<K, SSMD_BF16>(cp, blocks, n_units, st);
    default: return launch_gcpf_k<K, SSMD_F16>(cp, blocks, n_units, st);
  }
}

}  // namespace

bool gdn_conv_pf_fits(const GdnConvParams& cp) {
  const GdnParams& p = cp.g;
  const int rows_per_block = GCPF_WAVES * GCPF_RG * RowLayout<128>::RPI;
  static_assert(RowLayout<128>::RPI == RowLayout<64>::RPI, "one row count for both head sizes");
  return !p.norm_gate && cp.W == 4 && (p.K == 64 || p.K == 128) && (int64_t)(p.HV / p.H) * p.V == rows_per_block;
}

hipError_t launch_gdn_conv_pf(const GdnConvParams& cp, int64_t blocks, hipStream_t st) {
  if (!gdn_conv_pf_fits(cp) || blocks < 1) return hipErrorInvalidValue;
  const int64_t units = (int64_t)cp.g.B * cp.g.H;
  if (blocks > units) blocks = units;
  return cp.g.K == 64 ? launch_gcpf_act<64>(cp, blocks, (int)units, st)
                      : launch_gcpf_act<128>(cp, blocks, (int)units, st);
}

}  // namespace ssmd
