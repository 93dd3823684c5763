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
// rows. The first pass of state loads is issued before the conv prologue.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int D, int RG, bool NORM>
__global__ __launch_bounds__(512) void kda_decode_kernel(KdaParams p) {
  using RL = RowLayout<D>;
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

  // ---- first pass of state loads
  int base = wave * ROWS;
  f4 s[RG][NV];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int row = base + i * RPI + rr;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      s[i][j] = row < D ? ld4<false>(S + (int64_t)row * D + RL::col(c, j)) : f4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- conv update of this head's q, k, v channels -> y (LDS, fp32)
  __shared__ float y[3 * D];
  __shared__ float o_lds[NORM ? D : 1];
  __shared__ float red_lds[1];
  const int C = 3 * p.H * D;
  const int W = p.W;
  {
    const int64_t xrow = (int64_t)t * C;
    uint16_t* cs16 = static_cast<uint16_t*>(p.conv_state);
    float* cs32 = static_cast<float*>(p.conv_state);
    const int64_t cs_base = (int64_t)slot * p.cs_slot;
    for (int ci = tid; ci < 3 * D; ci += blockDim.x) {
      const int part = ci / D;  // 0 = q, 1 = k, 2 = v
      const int gc = part * p.H * D + h * D + (ci - part * D);
      const float* wr = p.conv_w + (int64_t)gc * W;
      const int64_t cso = cs_base + (int64_t)gc * p.cs_chan;
      // window = [state taps 0..W-2 (oldest first), x]; raw bits kept for the roll
      uint32_t raw[8];
      float win[8];
      for (int j = 0; j < W - 1; ++j) {
        const int64_t o = cso + (int64_t)j * p.cs_tap;
        if (p.act_dt == SSMD_F32) {
          win[j] = cs32[o];
          raw[j] = __float_as_uint(win[j]);
        } else {
          raw[j] = cs16[o];
          win[j] = p.act_dt == SSMD_BF16 ? bf16_bits_to_f32(raw[j]) : f16_bits_to_f32(raw[j]);
        }
      }
      if (p.act_dt == SSMD_F32) {
        win[W - 1] = static_cast<const float*>(p.x)[xrow + gc];
        raw[W - 1] = __float_as_uint(win[W - 1]);
      } else {
        raw[W - 1] = static_cast<const uint16_t*>(p.x)[xrow + gc];
        win[W - 1] = p.act_dt == SSMD_BF16 ? bf16_bits_to_f32(raw[W - 1]) : f16_bits_to_f32(raw[W - 1]);
      }
      float acc = p.conv_b ? p.conv_b[gc] : 0.f;
      for (int j = 0; j < W; ++j) acc += wr[j] * win[j];
      for (int j = 0; j < W - 1; ++j) {  // roll: tap j <- window[j + 1]
        const int64_t o = cso + (int64_t)j * p.cs_tap;
        if (p.act_dt == SSMD_F32) cs32[o] = __uint_as_float(raw[j + 1]);
        else cs16[o] = (uint16_t)raw[j + 1];
      }
      y[ci] = silu_f(acc);
    }
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
  const int64_t hoff = ((int64_t)t * p.H + h) * D;
  const float ea = p.A_log ? expf(p.A_log[h]) : 1.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float rg[4];
    load_act4(p.raw_g, hoff + RL::col(c, j), p.act_dt, p.raw_g_vec, rg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float db = p.dt_bias ? p.dt_bias[h * D + RL::col(c, j) + e] : 0.f;
      dec[4 * j + e] = expf(p.lower_bound * sigmoid_f(ea * (rg[e] + db)));
    }
  }
  const float beta = sigmoid_f(load_act1(p.raw_beta, (int64_t)t * p.H + h, p.act_dt));

  // ---- stream the state rows
  while (base < D) {
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
      const int row = base + i * RPI + rr;
      const float vrow = row < D ? y[2 * D + row] : 0.f;
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
          st4<false>(S + (int64_t)row * D + RL::col(c, j), n);
        }
        if (c == 0) {
          if constexpr (NORM) o_lds[row] = o;
          else store_act1(p.out, hoff + row, p.out_dt, o);
        }
      }
    }
    base += nwaves * ROWS;
    if (base < D) {
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int row = base + i * RPI + rr;
#pragma unroll
        for (int j = 0; j < NV; ++j)
          s[i][j] = row < D ? ld4<false>(S + (int64_t)row * D + RL::col(c, j)) : f4{0.f, 0.f, 0.f, 0.f};
      }
    }
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
      const float gz = sigmoid_f(load_act1(p.gate, hoff + r, p.act_dt));
      const float w = p.norm_w ? p.norm_w[r] : 1.f;
      store_act1(p.out, hoff + r, p.out_dt, o_lds[r] * inv * w * gz);
    }
  }
}

namespace {

template <int D, int RG>
hipError_t launch_kk(const KdaParams& p, int wpb, hipStream_t st) {
  constexpr int RPI = RowLayout<D>::RPI;
  const int wave_rows = RG * RPI;
  const int need = (D + wave_rows - 1) / wave_rows;
  if (wpb > need) wpb = need;
  const dim3 grid((unsigned)((int64_t)p.T * p.H));
  const dim3 block(64 * wpb);
  if (p.gate)
    kda_decode_kernel<D, RG, true><<<grid, block, 0, st>>>(p);
  else
    kda_decode_kernel<D, RG, false><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_krg(const KdaParams& p, const Launch& l, hipStream_t st) {
  switch (l.rg) {
    case 1: return launch_kk<D, 1>(p, l.wpb, st);
    case 2: return launch_kk<D, 2>(p, l.wpb, st);
    case 4: return launch_kk<D, 4>(p, l.wpb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_kda(const KdaParams& p, const Launch& l, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_krg<16>(p, l, st);
    case 32: return launch_krg<32>(p, l, st);
    case 64: return launch_krg<64>(p, l, st);
    case 128: return launch_krg<128>(p, l, st);
    case 256: return launch_krg<256>(p, l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
