// kda_decode_pf.hip -- the fused KDA decode op (conv1d update + SiLU, KDA
// delta rule, sigmoid-gated RMSNorm) as blocks that, when they walk several
// (token, head) units, prefetch the next one while computing the current
// one: the structure of gdn_decode_pf.hip applied to kda_decode.hip, for the common shapes (head
// size 64 or 128, conv width 4).
//
// Same computation as kda_decode_kernel ("Microbenchmark for the fused
// Kimi-K3 KDA decode kernel on ROCm": module docstring, `triton_chain`,
// `_gated_rmsnorm`, `Inputs`; "Optimization Log: Qwen3.5-27B Dense on B200",
// "Kernel 4: Fused DeltaNet Recurrent", Math). Blocks of 4 waves walk
// (token, head) units with a grid stride (by default the grid has one block
// per unit, which measured faster; see the launcher): each wave holds D/4 state
// rows, each thread up to two conv channels (window, weights, bias) and one
// gate column and output row. Everything a unit needs from HBM is fetched
// one unit ahead (activation values kept raw until used), so the compute of
// a unit never waits on a load issued after the next unit's and the memory
// queue stays full across units. One barrier per unit: after the conv
// output and the per-column decay; the gated RMSNorm epilogue of a unit
// (which needs every wave's o^2) runs after the next unit's barrier. LDS
// buffers alternate with the parity of the units a block computes (skipped
// units do not count), so no buffer is rewritten before every wave has
// passed the barrier that follows its last read.
#include <type_traits>

#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

constexpr int KPF_WAVES = 4;

template <int D, bool NORM, int ACT>
__global__ __launch_bounds__(64 * KPF_WAVES) void kda_decode_pf_kernel(KdaParams p, int n_units) {
  using RL = RowLayout<D>;
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI;
  constexpr int NT = 64 * KPF_WAVES;
  constexpr int RG = D / (KPF_WAVES * RPI);  // row groups per wave
  static_assert(RG >= 1 && RG * KPF_WAVES * RPI == D, "rows must tile the head");
  static_assert(D <= NT, "one gate column and one output row per thread");
  constexpr int CPT = (3 * D + NT - 1) / NT;  // conv channels per thread
  constexpr int W = 4;
  using T = typename std::conditional<ACT == SSMD_F32, float, uint16_t>::type;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  const int col = min(tid, D - 1);  // this thread's gate column and output row
  const int C = 3 * p.H * D;
  // double buffered by the parity of the block's computed units
  __shared__ float y_lds[2][3 * D];
  __shared__ float dec_lds[2][D];
  __shared__ float o_lds[2][NORM ? D : 1];
  __shared__ float red[2][KPF_WAVES];
  T* const cs = static_cast<T*>(p.conv_state);
  const float* const cb = p.conv_b ? p.conv_b : p.conv_w;  // bias, or any valid address times 0
  const float cb_on = p.conv_b ? 1.f : 0.f;
  const float nw = NORM && p.norm_w ? p.norm_w[col] : 1.f;
  auto row_of = [&](int i) { return (i * KPF_WAVES + wave) * RPI + rr; };
  auto chan = [&](int h, int ci) {  // global channel of head-local channel ci (q, k, v slices)
    const int part = ci / D;
    return part * p.H * D + h * D + (ci - part * D);
  };

  struct Unit {
    int t, h, slot;
    T win[CPT][W];  // conv windows: state taps 0..W-2 (oldest first), then x
    float wv[CPT][W], bias[CPT];
    T graw, rbeta, z;  // raw activation values, converted when used
    f4 s[RG][NV];
  };
  auto valid = [&](const Unit& U) { return U.slot > 0 && U.slot < p.num_slots; };  // slot 0: NULL block
  auto fetch = [&](int unit, Unit& U) {
    U.t = unit / p.H;
    U.h = unit - U.t * p.H;
    U.slot = p.idx[U.t];
    if (!valid(U)) return;  // uniform over the block
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int gc = chan(U.h, min(tid + m * NT, 3 * D - 1));
      const int64_t cso = (int64_t)U.slot * p.cs_slot + (int64_t)gc * p.cs_chan;
#pragma unroll
      for (int j = 0; j < W - 1; ++j) U.win[m][j] = cs[cso + (int64_t)j * p.cs_tap];
      U.win[m][W - 1] = static_cast<const T*>(p.x)[(int64_t)U.t * C + gc];
      const f4 wq = *reinterpret_cast<const f4*>(p.conv_w + (int64_t)gc * W);
      U.wv[m][0] = wq.x; U.wv[m][1] = wq.y; U.wv[m][2] = wq.z; U.wv[m][3] = wq.w;
      U.bias[m] = cb[gc];
    }
    const int64_t hoff = ((int64_t)U.t * p.H + U.h) * D;
    U.graw = static_cast<const T*>(p.raw_g)[hoff + col];
    U.rbeta = static_cast<const T*>(p.raw_beta)[(int64_t)U.t * p.H + U.h];
    if constexpr (NORM) U.z = static_cast<const T*>(p.gate)[hoff + col];
    const float* S = p.state + ((int64_t)U.slot * p.H + U.h) * (int64_t)D * D;
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
      for (int j = 0; j < NV; ++j) U.s[i][j] = ld4<true>(S + (int64_t)row_of(i) * D + RL::col(c, j));
  };
  auto to_f = [](T v) -> float {
    if constexpr (ACT == SSMD_F32) return v;
    else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(v);
    else return f16_bits_to_f32(v);
  };

  // Gated RMSNorm epilogue of a computed unit (its o and partial sums in
  // buffer pb), run after the next barrier: one output row per thread.
  struct Pending {
    int64_t hoff;
    T z;
    int pb;
    bool on;
  };
  Pending pend{0, T(0), 0, false};
  auto epilogue = [&]() {
    if constexpr (NORM) {
      if (pend.on && tid < D) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < KPF_WAVES; ++w) tot += red[pend.pb][w];
        const float inv = rsqrtf(tot / (float)D + p.norm_eps);
        store_act1(p.out, pend.hoff + tid, p.out_dt, o_lds[pend.pb][tid] * inv * nw * sigmoid_f(to_f(pend.z)));
      }
      pend.on = false;
    }
  };

  int buf = 0;
  auto compute = [&](Unit& U) {
    if (!valid(U)) return;  // uniform: no barrier is skipped by part of the block
    float* const y = y_lds[buf];
    float* const dl = dec_lds[buf];
    // ---- conv update of the unit's q, k, v channels -> y; roll the windows
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ci = tid + m * NT;
      if (ci < 3 * D) {
        float acc = cb_on * U.bias[m];
#pragma unroll
        for (int j = 0; j < W; ++j) acc += U.wv[m][j] * to_f(U.win[m][j]);
        const int64_t cso = (int64_t)U.slot * p.cs_slot + (int64_t)chan(U.h, ci) * p.cs_chan;
#pragma unroll
        for (int j = 0; j < W - 1; ++j) cs[cso + (int64_t)j * p.cs_tap] = U.win[m][j + 1];
        y[ci] = silu_f(acc);
      }
    }
    // ---- per-column decay, one column per thread
    if (tid < D) dl[tid] = expf(p.lower_bound * sigmoid_f(to_f(U.graw)));
    __syncthreads();
    epilogue();  // the previous unit's outputs (its o and sums are complete)
    // ---- q, k fragments, norms, the decay of this lane's columns
    float qf[NV * 4], kf[NV * 4], dec[NV * 4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const f4 qv = *reinterpret_cast<const f4*>(y + RL::col(c, j));
      const f4 kv = *reinterpret_cast<const f4*>(y + D + RL::col(c, j));
      const f4 dv = *reinterpret_cast<const f4*>(dl + RL::col(c, j));
      qf[4 * j] = qv.x; qf[4 * j + 1] = qv.y; qf[4 * j + 2] = qv.z; qf[4 * j + 3] = qv.w;
      kf[4 * j] = kv.x; kf[4 * j + 1] = kv.y; kf[4 * j + 2] = kv.z; kf[4 * j + 3] = kv.w;
      dec[4 * j] = dv.x; dec[4 * j + 1] = dv.y; dec[4 * j + 2] = dv.z; dec[4 * j + 3] = dv.w;
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
    const float beta = sigmoid_f(to_f(U.rbeta));
    const int64_t hoff = ((int64_t)U.t * p.H + U.h) * D;
    float* const S = p.state + ((int64_t)U.slot * p.H + U.h) * (int64_t)D * D;
    // ---- the unit's state rows
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        U.s[i][j].x *= dec[4 * j];
        U.s[i][j].y *= dec[4 * j + 1];
        U.s[i][j].z *= dec[4 * j + 2];
        U.s[i][j].w *= dec[4 * j + 3];
        dk += U.s[i][j].x * kf[4 * j] + U.s[i][j].y * kf[4 * j + 1] + U.s[i][j].z * kf[4 * j + 2] +
              U.s[i][j].w * kf[4 * j + 3];
        dq += U.s[i][j].x * qf[4 * j] + U.s[i][j].y * qf[4 * j + 1] + U.s[i][j].z * qf[4 * j + 2] +
              U.s[i][j].w * qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const int row = row_of(i);
      const float delta = beta * (y[2 * D + row] - dk);
      const float o = dq + delta * kq;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        f4 n;
        n.x = U.s[i][j].x + delta * kf[4 * j];
        n.y = U.s[i][j].y + delta * kf[4 * j + 1];
        n.z = U.s[i][j].z + delta * kf[4 * j + 2];
        n.w = U.s[i][j].w + delta * kf[4 * j + 3];
        st4<true>(S + (int64_t)row * D + RL::col(c, j), n);
      }
      if (c == 0) {
        if constexpr (NORM) {
          o_lds[buf][row] = o;
          ss += o * o;
        } else {
          store_act1(p.out, hoff + row, p.out_dt, o);
        }
      }
    }
    if constexpr (NORM) {
      ss = wave_sum(ss);
      if (lane == 0) red[buf][wave] = ss;
      pend = Pending{hoff, U.z, buf, true};
    }
    buf ^= 1;
  };

  // units u = (token u / H, head u % H) with a grid stride
  Unit A, B;
  int u = blockIdx.x;
  const int g = gridDim.x;
  if (u < n_units) fetch(u, A);
  while (u < n_units) {
    if (u + g < n_units) fetch(u + g, B);
    compute(A);
    if (u + g >= n_units) break;
    if (u + 2 * g < n_units) fetch(u + 2 * g, A);
    compute(B);
    u += 2 * g;
  }
  if constexpr (NORM) {
    __syncthreads();
    epilogue();
  }
}

namespace {

// One block per (token, head) unit unless a grid cap is given (launch-shape
// sweeps; the blocks then walk the units with a grid stride). Measured at
// T = 64, D = 128, conv width 4, gated norm: 12 / 24 / 48 / 96 heads in
// 20.5 / 37.4 / 71.6 / 143.6 us, against 22.1 / 41.5 / 77.4 / 151.4 with one
// block per CU walking the units: several resident blocks per CU, each with
// all its loads issued at once, keep more bytes in flight than one walking
// block's one-unit-ahead prefetch.
template <int D, bool NORM, int ACT>
hipError_t launch_kpf(const KdaParams& p, int cap, hipStream_t st) {
  const int64_t units = (int64_t)p.T * p.H;
  const int64_t blocks = cap > 0 && units > cap ? cap : units;
  kda_decode_pf_kernel<D, NORM, ACT><<<dim3((unsigned)blocks), dim3(64 * KPF_WAVES), 0, st>>>(p, (int)units);
  return hipGetLastError();
}

template <int D, bool NORM>
hipError_t launch_kpf_act(const KdaParams& p, int cap, hipStream_t st) {
  switch (p.act_dt) {
    case SSMD_F32: return launch_kpf<D, NORM, SSMD_F32>(p, cap, st);
    case SSMD_BF16: return launch_kpf<D, NORM, SSMD_BF16>(p, cap, st);
    default: return launch_kpf<D, NORM, SSMD_F16>(p, cap, st);
  }
}

template <int D>
hipError_t launch_kpf_norm(const KdaParams& p, int cap, hipStream_t st) {
  return p.gate ? launch_kpf_act<D, true>(p, cap, st) : launch_kpf_act<D, false>(p, cap, st);
}

}  // namespace

bool kda_pf_supported(const KdaParams& p) {
  return (p.D == 64 || p.D == 128) && p.W == 4;
}

hipError_t launch_kda_pf(const KdaParams& p, const Launch& l, hipStream_t st) {
  const int cap = l.grid_cap;  // > 0 only for launch-shape sweeps
  switch (p.D) {
    case 64: return launch_kpf_norm<64>(p, cap, st);
    case 128: return launch_kpf_norm<128>(p, cap, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
