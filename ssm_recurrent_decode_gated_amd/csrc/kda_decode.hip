// kda_decode.hip -- fused KDA decode on gfx950: causal conv1d update + SiLU,
// per-key-channel gated delta rule, sigmoid-gated RMSNorm, in one launch.
//
// Follows "Microbenchmark for the fused Kimi-K3 KDA decode kernel on ROCm"
// (module docstring; `triton_chain` gives the three steps the fused op
// replaces: conv update with SiLU, the KDA recurrent step with a lower-bounded
// gate, and `_gated_rmsnorm`; `Inputs` gives the layouts and the NULL slot 0),
// with the delta-rule order of "Optimization Log: Qwen3.5-27B Dense on B200"
// ("Kernel 4: Fused DeltaNet Recurrent", Math).
//
// One block per (token, head). The block first runs the conv update for the
// head's 3*D channels (q, k and v slices), writing the rolled conv state back
// and keeping the SiLU outputs in LDS at fp32 (the conv output never goes
// through HBM). The state rows then stream exactly as in the GDN kernel, with
// the decay a per-column vector (lane constants, since a lane's columns are
// fixed). The gated RMSNorm needs the whole head, so the block owns all D
// rows. The gate inputs and the first pass of state loads are issued before
// the conv prologue, so the state stream is in flight while the conv runs.
#include <type_traits>

#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int D>
constexpr int kda_rg() {
  return D == 16 ? 1 : (D == 32 ? 2 : (D == 256 ? 2 : 4));
}

template <int D, bool NORM, int ACT, bool VEC>
__global__ __launch_bounds__(512) void kda_decode_kernel(KdaParams p) {
  using RL = RowLayout<D>;
  constexpr int RG = kda_rg<D>();
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, ROWS = RG * RPI;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  const int h = blockIdx.x % p.H;
  const int t = blockIdx.x / p.H;
  const int slot = p.idx[t];
  if (slot <= 0 || slot >= p.num_slots) return;  // NULL block or padding
  float* S = p.state + ((int64_t)slot * p.H + h) * (int64_t)D * D;
  auto row_of = [&](int pass, int i) { return pass + (i * nwaves + wave) * RPI + rr; };
  const int64_t hoff = ((int64_t)t * p.H + h) * D;

  // ---- small loads first (this thread's conv channels: state taps and x;
  // the gate inputs), then the first pass of state loads: waiting for the
  // small ones never waits for the state stream.
  using T = typename std::conditional<ACT == SSMD_F32, float, uint16_t>::type;
  constexpr int CPT = 4;   // conv channels per thread held in registers (3*D <= CPT*blockDim)
  constexpr int WMAX = 8;  // widest conv accepted by the host
  const int C = 3 * p.H * D;
  const int W = p.W;
  const int nch = 3 * D;
  T* cs = static_cast<T*>(p.conv_state);
  const T* xr = static_cast<const T*>(p.x) + (int64_t)t * C;
  const int64_t cs_base = (int64_t)slot * p.cs_slot;
  auto chan = [&](int ci) {  // global channel of head-local channel ci (q, k, v slices)
    const int part = ci / D;
    return part * p.H * D + h * D + (ci - part * D);
  };
  T raw[CPT][WMAX];  // window = [state taps 0..W-2 (oldest first), x]
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int gc = chan(min(tid + m * (int)blockDim.x, nch - 1));
    const int64_t cso = cs_base + (int64_t)gc * p.cs_chan;
#pragma unroll
    for (int j = 0; j < WMAX - 1; ++j)
      if (j < W - 1) raw[m][j] = cs[cso + (int64_t)j * p.cs_tap];
    raw[m][WMAX - 1] = xr[gc];
  }
  float rg[NV * 4];
#pragma unroll
  for (int j = 0; j < NV; ++j) ld_act4<ACT, VEC>(p.raw_g, hoff + RL::col(c, j), &rg[4 * j]);
  const float rbeta = ld_act<ACT>(p.raw_beta, (int64_t)t * p.H + h);
  f4 s[RG][NV];
  auto load_group = [&](int pass, int i) {
    const int row = min(row_of(pass, i), D - 1);
#pragma unroll
    for (int j = 0; j < NV; ++j) s[i][j] = ld4<true>(S + (int64_t)row * D + RL::col(c, j));
  };
  int pass = 0;
#pragma unroll
  for (int i = 0; i < RG; ++i) load_group(pass, i);

  // ---- conv update of this head's q, k, v channels -> y (LDS, fp32)
  __shared__ float y[3 * D];
  __shared__ float o_lds[NORM ? D : 1];
  __shared__ float red_lds[1];
  auto to_f = [](T v) -> float {
    if constexpr (ACT == SSMD_F32) return v;
    else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(v);
    else return f16_bits_to_f32(v);
  };
  auto conv_channel = [&](int ci, const T* win_state, T xv) {
    const int gc = chan(ci);
    const float* wr = p.conv_w + (int64_t)gc * W;
    const int64_t cso = cs_base + (int64_t)gc * p.cs_chan;
    float acc = p.conv_b ? p.conv_b[gc] : 0.f;
#pragma unroll
    for (int j = 0; j < WMAX - 1; ++j)
      if (j < W - 1) acc += wr[j] * to_f(win_state[j]);
    acc += wr[W - 1] * to_f(xv);
    // roll: tap j <- window[j + 1]; the newest tap takes x
#pragma unroll
    for (int j = 0; j < WMAX - 2; ++j)
      if (j < W - 2) cs[cso + (int64_t)j * p.cs_tap] = win_state[j + 1];
    cs[cso + (int64_t)(W - 2) * p.cs_tap] = xv;
    y[ci] = silu_f(acc);
  };
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int ci = tid + m * (int)blockDim.x;
    if (ci < nch) conv_channel(ci, raw[m], raw[m][WMAX - 1]);
  }
  for (int ci = tid + CPT * (int)blockDim.x; ci < nch; ci += blockDim.x) {  // only with tiny blocks
    T win[WMAX];
    const int64_t cso = cs_base + (int64_t)chan(ci) * p.cs_chan;
    for (int j = 0; j < W - 1; ++j) win[j] = cs[cso + (int64_t)j * p.cs_tap];
    conv_channel(ci, win, xr[chan(ci)]);
  }
  __syncthreads();

  // ---- q/k fragments, L2 norms, per-column decay, beta
  float qf[NV * 4], kf[NV * 4], dec[NV * 4];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[4 * j + e] = y[RL::col(c, j) + e];
      kf[4 * j + e] = y[D + RL::col(c, j) + e];
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
#pragma unroll
  for (int e = 0; e < NV * 4; ++e) dec[e] = expf(p.lower_bound * sigmoid_f(rg[e]));
  const float beta = sigmoid_f(rbeta);

  // ---- stream the state rows
  while (true) {
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        s[i][j].x *= dec[4 * j];
        s[i][j].y *= dec[4 * j + 1];
        s[i][j].z *= dec[4 * j + 2];
        s[i][j].w *= dec[4 * j + 3];
        dk += s[i][j].x * kf[4 * j] + s[i][j].y * kf[4 * j + 1] + s[i][j].z * kf[4 * j + 2] +
              s[i][j].w * kf[4 * j + 3];
        dq += s[i][j].x * qf[4 * j] + s[i][j].y * qf[4 * j + 1] + s[i][j].z * qf[4 * j + 2] +
              s[i][j].w * qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const int row = row_of(pass, i);
      const float vrow = y[2 * D + min(row, D - 1)];
      const float delta = beta * (vrow - dk);
      const float o = dq + delta * kq;
      if (row < D) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          f4 n;
          n.x = s[i][j].x + delta * kf[4 * j];
          n.y = s[i][j].y + delta * kf[4 * j + 1];
          n.z = s[i][j].z + delta * kf[4 * j + 2];
          n.w = s[i][j].w + delta * kf[4 * j + 3];
          st4<true>(S + (int64_t)row * D + RL::col(c, j), n);
        }
        if (c == 0) {
          if constexpr (NORM) o_lds[row] = o;
          else store_act1(p.out, hoff + row, p.out_dt, o);
        }
      }
    }
    pass += nwaves * ROWS;
    if (pass >= D) break;
#pragma unroll
    for (int i = 0; i < RG; ++i) load_group(pass, i);
  }

  if constexpr (NORM) {
    __syncthreads();
    if (wave == 0) {
      float ss = 0.f;
      for (int r = lane; r < D; r += 64) ss += o_lds[r] * o_lds[r];
      ss = wave_sum(ss);
      if (lane == 0) red_lds[0] = ss;
    }
    __syncthreads();
    const float inv = rsqrtf(red_lds[0] / (float)D + p.norm_eps);
    for (int r = tid; r < D; r += blockDim.x) {
      const float gz = sigmoid_f(ld_act<ACT>(p.gate, hoff + r));
      const float w = p.norm_w ? p.norm_w[r] : 1.f;
      store_act1(p.out, hoff + r, p.out_dt, o_lds[r] * inv * w * gz);
    }
  }
}

namespace {

template <int D, bool NORM, int ACT, bool VEC>
hipError_t launch_kk(const KdaParams& p, const Launch& l, hipStream_t st) {
  constexpr int RPI = RowLayout<D>::RPI;
  const int wave_rows = kda_rg<D>() * RPI;
  const int need = (D + wave_rows - 1) / wave_rows;
  const int wpb = l.wpb > need ? need : l.wpb;
  const dim3 grid((unsigned)((int64_t)p.T * p.H));
  kda_decode_kernel<D, NORM, ACT, VEC><<<grid, dim3(64 * wpb), 0, st>>>(p);
  return hipGetLastError();
}

template <int D, bool NORM>
hipError_t launch_kact(const KdaParams& p, const Launch& l, hipStream_t st) {
  const bool vec = p.raw_g_vec;
  switch (p.act_dt) {
    case SSMD_F32: return vec ? launch_kk<D, NORM, SSMD_F32, true>(p, l, st) : launch_kk<D, NORM, SSMD_F32, false>(p, l, st);
    case SSMD_BF16: return vec ? launch_kk<D, NORM, SSMD_BF16, true>(p, l, st) : launch_kk<D, NORM, SSMD_BF16, false>(p, l, st);
    default: return vec ? launch_kk<D, NORM, SSMD_F16, true>(p, l, st) : launch_kk<D, NORM, SSMD_F16, false>(p, l, st);
  }
}

template <int D>
hipError_t launch_knorm(const KdaParams& p, const Launch& l, hipStream_t st) {
  return p.gate ? launch_kact<D, true>(p, l, st) : launch_kact<D, false>(p, l, st);
}

}  // namespace

hipError_t launch_kda(const KdaParams& p, const Launch& l, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_knorm<16>(p, l, st);
    case 32: return launch_knorm<32>(p, l, st);
    case 64: return launch_knorm<64>(p, l, st);
    case 128: return launch_knorm<128>(p, l, st);
    case 256: return launch_knorm<256>(p, l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
