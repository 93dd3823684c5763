// gdn_decode.hip -- packed GDN decode step on gfx950.
//
// Computes, per (batch row, value head), the gated delta rule of
// "Optimization Log: Qwen3.5-27B Dense on B200" ("Kernel 4: Fused DeltaNet
// Recurrent", Math) on the fp32 state pool of the packed GDN decode in
// "Microbenchmark: buffered output-only GDN decode (ReplaySSM Part A) vs. the
// existing packed GDN decode kernel" (`_bench_cfg`: state [slots, HV, V, K],
// mixed_qkv q|k|v, gates a, b, A_log, dt_bias, slot indices).
//
// Design (HBM-bound: ~0.9 flop per state byte, far below the fp32 ridge, so
// no MFMA): every state row v is independent once k, q, g and beta are known:
//   dk = S_v . k,  dq = S_v . q                      (one pass over the row)
//   u = e^g dk;  delta_v = beta (v_v - u);  o_v = e^g dq + delta_v (k . q)
//   S_v <- e^g S_v + delta_v k
// so each row is read once and written once, with both dot products reduced
// over the row's lanes by DPP in the same pass. A row of K fp32 is spread
// over LPR lanes (8 for K >= 32) with 128-bit accesses, so one wave-wide
// access covers 8 rows x 128 contiguous bytes. q and k are normalised by
// every wave from registers (the 8 lanes of a row hold the whole vector), so
// the kernel needs no LDS and no barrier unless the gated RMSNorm epilogue
// is on. The first pass of state loads is issued before the prologue so its
// latency overlaps the gate/normalisation arithmetic.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int K, int RG, bool NORM, bool NT>
__global__ __launch_bounds__(512) void gdn_decode_kernel(GdnParams p, int tiles_per_head,
                                                         int rows_per_tile) {
  using RL = RowLayout<K>;
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, ROWS = RG * RPI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  int bid = blockIdx.x;
  const int tile = bid % tiles_per_head;
  bid /= tiles_per_head;
  const int hv = bid % p.HV;
  const int bi = bid / p.HV;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;  // padded row: touch nothing
  const int h = hv / (p.HV / p.H);
  const int V = p.V;
  float* S = p.state + ((int64_t)slot * p.HV + hv) * (int64_t)V * K;
  const int r0 = tile * rows_per_tile;
  const int r1 = min(V, r0 + rows_per_tile);
  const int64_t qrow = (int64_t)bi * p.qkv_stride;
  const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)hv * V;

  // ---- first pass of state loads (independent of the prologue)
  int base = r0 + wave * ROWS;
  f4 s[RG][NV];
  float vv[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int row = base + i * RPI + rr;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      s[i][j] = row < r1 ? ld4<NT>(S + (int64_t)row * K + RL::col(c, j)) : f4{0.f, 0.f, 0.f, 0.f};
    vv[i] = row < r1 ? load_act1(p.qkv, vbase + row, p.act_dt) : 0.f;
  }

  // ---- prologue: q/k fragments, L2 norms, gates
  float qf[NV * 4], kf[NV * 4];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    load_act4(p.qkv, qrow + (int64_t)h * K + RL::col(c, j), p.act_dt, p.qkv_vec, &qf[4 * j]);
    load_act4(p.qkv, qrow + (int64_t)(p.H + h) * K + RL::col(c, j), p.act_dt, p.qkv_vec, &kf[4 * j]);
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
  const int64_t gidx = (int64_t)bi * p.HV + hv;
  const float av = load_act1(p.a, gidx, p.act_dt);
  const float bv = load_act1(p.b, gidx, p.act_dt);
  const float g = -expf(p.A_log[hv]) * softplus_f(av + p.dt_bias[hv]);
  const float beta = sigmoid_f(bv);
  const float decay = expf(g);

  __shared__ float o_lds[NORM ? 1024 : 1];
  __shared__ float red_lds[1];
  const int64_t obase = gidx * V;

  // ---- stream the rows
  while (base < r1) {
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        dk += s[i][j].x * kf[4 * j] + s[i][j].y * kf[4 * j + 1] + s[i][j].z * kf[4 * j + 2] +
              s[i][j].w * kf[4 * j + 3];
        dq += s[i][j].x * qf[4 * j] + s[i][j].y * qf[4 * j + 1] + s[i][j].z * qf[4 * j + 2] +
              s[i][j].w * qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const float delta = beta * (vv[i] - decay * dk);
      const float o = decay * dq + delta * kq;
      const int row = base + i * RPI + rr;
      if (row < r1) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          f4 n;
          n.x = decay * s[i][j].x + delta * kf[4 * j];
          n.y = decay * s[i][j].y + delta * kf[4 * j + 1];
          n.z = decay * s[i][j].z + delta * kf[4 * j + 2];
          n.w = decay * s[i][j].w + delta * kf[4 * j + 3];
          st4<NT>(S + (int64_t)row * K + RL::col(c, j), n);
        }
        if (c == 0) {
          if constexpr (NORM) o_lds[row] = o;
          else store_act1(p.out, obase + row, p.out_dt, o);
        }
      }
    }
    base += nwaves * ROWS;
    if (base < r1) {
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int row = base + i * RPI + rr;
#pragma unroll
        for (int j = 0; j < NV; ++j)
          s[i][j] = row < r1 ? ld4<NT>(S + (int64_t)row * K + RL::col(c, j)) : f4{0.f, 0.f, 0.f, 0.f};
        vv[i] = row < r1 ? load_act1(p.qkv, vbase + row, p.act_dt) : 0.f;
      }
    }
  }

  if constexpr (NORM) {
    // gated RMSNorm over the head's V outputs (the whole head is this block)
    __syncthreads();
    if (wave == 0) {
      float ss = 0.f;
      for (int r = lane; r < V; r += 64) ss += o_lds[r] * o_lds[r];
      ss = wave_sum(ss);
      if (lane == 0) red_lds[0] = ss;
    }
    __syncthreads();
    const float inv = rsqrtf(red_lds[0] / (float)V + p.norm_eps);
    for (int r = threadIdx.x; r < V; r += blockDim.x) {
      const float z = load_act1(p.norm_gate, obase + r, p.act_dt);
      const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
      const float w = p.norm_w ? p.norm_w[r] : 1.f;
      store_act1(p.out, obase + r, p.out_dt, o_lds[r] * inv * w * gz);
    }
  }
}

// ------------------------------------------------------------- host side
namespace {

template <int K, int RG, bool NT>
hipError_t launch_k(const GdnParams& p, int wpb, hipStream_t st) {
  constexpr int RPI = RowLayout<K>::RPI;
  const int wave_rows = RG * RPI;
  const bool norm = p.norm_gate != nullptr;
  int tiles, rows_per_tile;
  if (norm) {
    tiles = 1;
    rows_per_tile = p.V;
  } else {
    rows_per_tile = wpb * wave_rows;
    tiles = (p.V + rows_per_tile - 1) / rows_per_tile;
  }
  // never launch more waves than a tile has row passes
  int need = (min(p.V, rows_per_tile) + wave_rows - 1) / wave_rows;
  if (wpb > need) wpb = need;
  const dim3 grid((unsigned)((int64_t)p.B * p.HV * tiles));
  const dim3 block(64 * wpb);
  if (norm)
    gdn_decode_kernel<K, RG, true, NT><<<grid, block, 0, st>>>(p, tiles, rows_per_tile);
  else
    gdn_decode_kernel<K, RG, false, NT><<<grid, block, 0, st>>>(p, tiles, rows_per_tile);
  return hipGetLastError();
}

template <int K, bool NT>
hipError_t launch_rg(const GdnParams& p, const Launch& l, hipStream_t st) {
  switch (l.rg) {
    case 1: return launch_k<K, 1, NT>(p, l.wpb, st);
    case 2: return launch_k<K, 2, NT>(p, l.wpb, st);
    case 4: return launch_k<K, 4, NT>(p, l.wpb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gdn_supported(int K, int rg) {
  return (K == 16 || K == 32 || K == 64 || K == 128 || K == 256) && (rg == 1 || rg == 2 || rg == 4);
}

hipError_t launch_gdn(const GdnParams& p, const Launch& l, hipStream_t st) {
  const bool nt = l.nt != 0;
  switch (p.K) {
    case 16: return nt ? launch_rg<16, true>(p, l, st) : launch_rg<16, false>(p, l, st);
    case 32: return nt ? launch_rg<32, true>(p, l, st) : launch_rg<32, false>(p, l, st);
    case 64: return nt ? launch_rg<64, true>(p, l, st) : launch_rg<64, false>(p, l, st);
    case 128: return nt ? launch_rg<128, true>(p, l, st) : launch_rg<128, false>(p, l, st);
    case 256: return nt ? launch_rg<256, true>(p, l, st) : launch_rg<256, false>(p, l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
