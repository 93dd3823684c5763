// gdn_multi.hip -- GDN over T tokens per sequence on gfx950: the packed step
// of gdn_decode.hip applied token after token with the state held in
// registers, so each state row is read and written once per call instead of
// once per token (T tokens of speculative verification or a short prompt
// cost one state round trip).
//
// Each state row v evolves independently once the token's k, q, v_v, g and
// beta are known ("Optimization Log: Qwen3.5-27B Dense on B200", "Kernel 4:
// Fused DeltaNet Recurrent", Math, in the single-pass row form):
//   dk = S_v . k, dq = S_v . q;  delta = beta (v_v - e^g dk)
//   o_v = e^g dq + delta (k . q);  S_v <- e^g S_v + delta k
// so a wave keeps its rows (RG groups of RPI rows, K/LPR columns per lane)
// in registers for the whole call and walks the tokens, normalising each
// token's q and k from registers (no LDS). Rows of a head are split into
// tiles over blocks when there are few (row, head) units. The gated RMSNorm
// needs a token's whole head: with it, one block holds the head and each
// token takes one barrier (per-wave partial sums of o^2 in LDS, double
// buffered by token parity).
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int K>
constexpr int gmulti_rg() {
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 2 : 4));
}

template <int K, bool NORM, int ACT, bool VEC>
__global__ __launch_bounds__(512) void gdn_multi_kernel(GdnMultiParams mp) {
  const GdnParams& p = mp.g;
  using RL = RowLayout<K>;
  constexpr int RG = gmulti_rg<K>();
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  __shared__ float red[2][NORM ? 8 : 1];

  int bid = blockIdx.x;
  const int tile = bid % mp.tiles;
  bid /= mp.tiles;
  const int hv = bid % p.HV;
  const int bi = bid / p.HV;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;  // padded row: touch nothing
  const int T = mp.T;
  const int len = mp.lengths ? min(max(mp.lengths[bi], 0), T) : T;
  if (len == 0) return;  // nothing to do: the state stays as it is
  const int h = hv / (p.HV / p.H);
  const int V = p.V;
  const int r0 = tile * mp.rows_per_tile;
  const int r1 = min(V, r0 + mp.rows_per_tile);
  float* const S = static_cast<float*>(p.state) + ((int64_t)slot * p.HV + hv) * (int64_t)V * K;
  int rowc[RG];  // this lane's rows, clamped into the tile (rows past it are computed, never stored)
#pragma unroll
  for (int i = 0; i < RG; ++i) rowc[i] = min(r0 + (i * nwaves + wave) * RPI + rr, r1 - 1);

  struct Tok {
    float qf[NV * 4], kf[NV * 4], vv[RG], zz[RG], av, bv;
  };
  auto fetch = [&](int t, Tok& X) {
    const int64_t bt = (int64_t)bi * T + min(t, len - 1);
    const int64_t qrow = bt * p.qkv_stride;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)h * K + RL::col(c, j), &X.qf[4 * j]);
      ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)(p.H + h) * K + RL::col(c, j), &X.kf[4 * j]);
    }
    const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)hv * V;
    const int64_t gbase = (bt * p.HV + hv) * V;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      X.vv[i] = ld_act<ACT>(p.qkv, vbase + rowc[i]);
      X.zz[i] = NORM ? ld_act<ACT>(p.norm_gate, gbase + rowc[i]) : 0.f;
    }
    X.av = ld_act<ACT>(p.a, bt * p.HV + hv);
    X.bv = ld_act<ACT>(p.b, bt * p.HV + hv);
  };

  // ---- the tile's rows, held for the whole call
  f4 s[RG][NV];
  Tok A;
  fetch(0, A);
#pragma unroll
  for (int i = 0; i < RG; ++i)
#pragma unroll
    for (int j = 0; j < NV; ++j) s[i][j] = ld4<true>(S + (int64_t)rowc[i] * K + RL::col(c, j));
  const float A_log = p.A_log[hv];
  const float dt_bias = p.dt_bias[hv];

  auto compute = [&](int t, Tok& X) {
    float qs = p.scale, ks = 1.f;
    if (p.use_l2) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < NV * 4; ++e) {
        sq += X.qf[e] * X.qf[e];
        sk += X.kf[e] * X.kf[e];
      }
      sq = group_sum<LPR>(sq);
      sk = group_sum<LPR>(sk);
      qs *= rsqrtf(sq + p.l2eps);
      ks = rsqrtf(sk + p.l2eps);
    }
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < NV * 4; ++e) {
      X.qf[e] *= qs;
      X.kf[e] *= ks;
      kq += X.kf[e] * X.qf[e];
    }
    kq = group_sum<LPR>(kq);
    const float g = -expf(A_log) * softplus_f(X.av + dt_bias);
    const float beta = sigmoid_f(X.bv);
    const float decay = expf(g);
    const int64_t obase = (((int64_t)bi * T + t) * p.HV + hv) * V;
    float o[RG];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        dk += s[i][j].x * X.kf[4 * j] + s[i][j].y * X.kf[4 * j + 1] + s[i][j].z * X.kf[4 * j + 2] +
              s[i][j].w * X.kf[4 * j + 3];
        dq += s[i][j].x * X.qf[4 * j] + s[i][j].y * X.qf[4 * j + 1] + s[i][j].z * X.qf[4 * j + 2] +
              s[i][j].w * X.qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const float delta = beta * (X.vv[i] - decay * dk);
      o[i] = decay * dq + delta * kq;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        s[i][j].x = decay * s[i][j].x + delta * X.kf[4 * j];
        s[i][j].y = decay * s[i][j].y + delta * X.kf[4 * j + 1];
        s[i][j].z = decay * s[i][j].z + delta * X.kf[4 * j + 2];
        s[i][j].w = decay * s[i][j].w + delta * X.kf[4 * j + 3];
      }
      const int row = r0 + (i * nwaves + wave) * RPI + rr;
      if constexpr (NORM) {
        if (c == 0 && row < r1) ss += o[i] * o[i];
      } else {
        if (c == 0 && row < r1) store_act1(p.out, obase + row, p.out_dt, o[i]);
      }
    }
    if constexpr (NORM) {
      ss = wave_sum(ss);
      if (lane == 0) red[t & 1][wave] = ss;
      __syncthreads();
      float tot = 0.f;
      for (int w = 0; w < nwaves; ++w) tot += red[t & 1][w];
      const float inv = rsqrtf(tot / (float)V + p.norm_eps);
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int row = r0 + (i * nwaves + wave) * RPI + rr;
        if (c == 0 && row < r1) {
          const float z = X.zz[i];
          const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
          const float w = p.norm_w ? p.norm_w[row] : 1.f;
          store_act1(p.out, obase + row, p.out_dt, o[i] * inv * w * gz);
        }
      }
    }
  };

  // ---- tokens. The next token's inputs are not prefetched into a second
  // register set (that pushes the K = 128 kernel past 256 VGPRs into
  // scratch); at ~170 VGPRs, 2-3 waves per SIMD hide each other's loads.
  for (int t = 0; t < len; ++t) {
    if (t > 0) fetch(t, A);
    compute(t, A);
  }

#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int row = r0 + (i * nwaves + wave) * RPI + rr;
    if (row < r1) {
#pragma unroll
      for (int j = 0; j < NV; ++j) st4<true>(S + (int64_t)row * K + RL::col(c, j), s[i][j]);
    }
  }
}

namespace {

template <int K, bool NORM, int ACT, bool VEC>
hipError_t launch_gm_k(const GdnMultiParams& mp0, const Launch& l, int n_cu, hipStream_t st) {
  GdnMultiParams mp = mp0;
  const GdnParams& p = mp.g;
  const int wave_rows = gmulti_rg<K>() * RowLayout<K>::RPI;
  int wpb;
  if (NORM) {
    wpb = (p.V + wave_rows - 1) / wave_rows;  // the whole head in one block (host-checked <= 8 waves)
    mp.tiles = 1;
  } else {
    wpb = min(l.wpb, (p.V + wave_rows - 1) / wave_rows);
    // few (row, head) units: smaller blocks, more of them
    while (wpb > 1 && (int64_t)p.B * p.HV * ((p.V + wpb * wave_rows - 1) / (wpb * wave_rows)) < 2LL * n_cu) wpb /= 2;
    mp.tiles = (p.V + wpb * wave_rows - 1) / (wpb * wave_rows);
  }
  mp.rows_per_tile = wpb * wave_rows;
  const int64_t blocks = (int64_t)p.B * p.HV * mp.tiles;
  gdn_multi_kernel<K, NORM, ACT, VEC><<<dim3((unsigned)blocks), dim3(64 * wpb), 0, st>>>(mp);
  return hipGetLastError();
}

template <int K, bool NORM>
hipError_t launch_gm_act(const GdnMultiParams& mp, const Launch& l, int n_cu, hipStream_t st) {
  const bool vec = mp.g.qkv_vec;
  switch (mp.g.act_dt) {
    case SSMD_F32:
      return vec ? launch_gm_k<K, NORM, SSMD_F32, true>(mp, l, n_cu, st) : launch_gm_k<K, NORM, SSMD_F32, false>(mp, l, n_cu, st);
    case SSMD_BF16:
      return vec ? launch_gm_k<K, NORM, SSMD_BF16, true>(mp, l, n_cu, st) : launch_gm_k<K, NORM, SSMD_BF16, false>(mp, l, n_cu, st);
    default:
      return vec ? launch_gm_k<K, NORM, SSMD_F16, true>(mp, l, n_cu, st) : launch_gm_k<K, NORM, SSMD_F16, false>(mp, l, n_cu, st);
  }
}

template <int K>
hipError_t launch_gm_norm(const GdnMultiParams& mp, const Launch& l, int n_cu, hipStream_t st) {
  return mp.g.norm_gate ? launch_gm_act<K, true>(mp, l, n_cu, st) : launch_gm_act<K, false>(mp, l, n_cu, st);
}

}  // namespace

int gdn_multi_max_norm_rows(int K) {
  switch (K) {
    case 16: return 8 * gmulti_rg<16>() * RowLayout<16>::RPI;
    case 32: return 8 * gmulti_rg<32>() * RowLayout<32>::RPI;
    case 64: return 8 * gmulti_rg<64>() * RowLayout<64>::RPI;
    case 128: return 8 * gmulti_rg<128>() * RowLayout<128>::RPI;
    default: return 8 * gmulti_rg<256>() * RowLayout<256>::RPI;
  }
}

hipError_t launch_gdn_multi(const GdnMultiParams& mp, const Launch& l, int n_cu, hipStream_t st) {
  switch (mp.g.K) {
    case 16: return launch_gm_norm<16>(mp, l, n_cu, st);
    case 32: return launch_gm_norm<32>(mp, l, n_cu, st);
    case 64: return launch_gm_norm<64>(mp, l, n_cu, st);
    case 128: return launch_gm_norm<128>(mp, l, n_cu, st);
    case 256: return launch_gm_norm<256>(mp, l, n_cu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
