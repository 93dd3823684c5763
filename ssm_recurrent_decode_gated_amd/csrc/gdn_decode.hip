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
// is on. The small activation loads are issued first and the state loads
// right after, with no branch between them, so a wave keeps its whole pass
// (16 KB at K = 128) in flight while the gates and norms are computed.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

// Row groups per wave pass: enough that a wave holds 32 rows of K = 64/128
// (16 KB of state in flight per wave), fewer for the widest head.
template <int K>
constexpr int gdn_rg() {
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 2 : 4));
}

// ACT: activation dtype (compile time, so no dtype branch sits between the
// state loads); VEC: mixed_qkv rows are 4-element aligned. A wave keeps all
// RG row groups of its pass in flight (measured: issuing fewer at a time is
// slower on MI355X); row groups are interleaved across the block's waves, so
// at each step the waves of a block touch one contiguous span of rows. Each
// block walks work units (batch row, value head, row tile) with a grid
// stride, so the grid can be capped below the unit count. State rows are
// loaded and stored non-temporally: each is touched exactly once per step.
template <int K, bool NORM, int ACT, bool VEC>
__global__ __launch_bounds__(512) void gdn_decode_kernel(GdnParams p, int tiles_per_head,
                                                         int rows_per_tile, int n_units) {
  using RL = RowLayout<K>;
  constexpr int RG = gdn_rg<K>();
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, ROWS = RG * RPI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  __shared__ float o_lds[NORM ? 1024 : 1];
  __shared__ float red_lds[1];

  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    int bid = unit;
    const int tile = bid % tiles_per_head;
    bid /= tiles_per_head;
    const int hv = bid % p.HV;
    const int bi = bid / p.HV;
    const int slot = p.idx[bi];
    if (slot < 0 || slot >= p.num_slots) continue;  // padded row: touch nothing
    const int h = hv / (p.HV / p.H);
    const int V = p.V;
    float* S = static_cast<float*>(p.state) + ((int64_t)slot * p.HV + hv) * (int64_t)V * K;
    const int r0 = tile * rows_per_tile;
    const int r1 = min(V, r0 + rows_per_tile);
    const int64_t qrow = (int64_t)bi * p.qkv_stride;
    const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)hv * V;
    const int64_t gidx = (int64_t)bi * p.HV + hv;
    // row of this lane in group i of the pass starting at row `pass`
    auto row_of = [&](int pass, int i) {
      return pass + (i * nwaves + wave) * RPI + rr;
    };

    // ---- small activation loads first, then the state stream: waiting for
    // the former never has to wait for the latter
    float qf[NV * 4], kf[NV * 4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)h * K + RL::col(c, j), &qf[4 * j]);
      ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)(p.H + h) * K + RL::col(c, j), &kf[4 * j]);
    }
    const float av = ld_act<ACT>(p.a, gidx);
    const float bv = ld_act<ACT>(p.b, gidx);
    const float A_log = p.A_log[hv];
    const float dt_bias = p.dt_bias[hv];
    f4 s[RG][NV];
    float vv[RG];
    // rows past the tile end re-read its last row (never stored): no branch
    auto load_group = [&](int pass, int i) {
      const int row = min(row_of(pass, i), r1 - 1);
      vv[i] = ld_act<ACT>(p.qkv, vbase + row);
#pragma unroll
      for (int j = 0; j < NV; ++j) s[i][j] = ld4<true>(S + (int64_t)row * K + RL::col(c, j));
    };
    int pass = r0;
#pragma unroll
    for (int i = 0; i < RG; ++i) load_group(pass, i);

    // ---- prologue: L2 norms, scale, gates
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
    const float g = -expf(A_log) * softplus_f(av + dt_bias);
    const float beta = sigmoid_f(bv);
    const float decay = expf(g);
    const int64_t obase = gidx * V;

    // ---- stream the rows
    while (true) {
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
        const int row = row_of(pass, i);
        if (row < r1) {
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            f4 n;
            n.x = decay * s[i][j].x + delta * kf[4 * j];
            n.y = decay * s[i][j].y + delta * kf[4 * j + 1];
            n.z = decay * s[i][j].z + delta * kf[4 * j + 2];
            n.w = decay * s[i][j].w + delta * kf[4 * j + 3];
            st4<true>(S + (int64_t)row * K + RL::col(c, j), n);
          }
          if (c == 0) {
            if constexpr (NORM) o_lds[row] = o;
            else store_act1(p.out, obase + row, p.out_dt, o);
          }
        }
      }
      pass += nwaves * ROWS;
      if (pass >= r1) break;
#pragma unroll
      for (int i = 0; i < RG; ++i) load_group(pass, i);
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
        const float z = ld_act<ACT>(p.norm_gate, obase + r);
        const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
        const float w = p.norm_w ? p.norm_w[r] : 1.f;
        store_act1(p.out, obase + r, p.out_dt, o_lds[r] * inv * w * gz);
      }
      __syncthreads();  // o_lds / red_lds are reused by the next unit
    }
  }  // unit loop
}

// ------------------------------------------------------------- host side
namespace {

template <int K, bool NORM, int ACT, bool VEC>
hipError_t launch_k(const GdnParams& p, const Launch& l, hipStream_t st) {
  constexpr int RPI = RowLayout<K>::RPI;
  const int wave_rows = gdn_rg<K>() * RPI;
  int wpb = l.wpb;
  int tiles, rows_per_tile;
  if (NORM) {
    tiles = 1;
    rows_per_tile = p.V;
  } else {
    rows_per_tile = wpb * wave_rows;
    tiles = (p.V + rows_per_tile - 1) / rows_per_tile;
  }
  // never launch more waves than a tile has row passes
  const int need = (min(p.V, rows_per_tile) + wave_rows - 1) / wave_rows;
  if (wpb > need) wpb = need;
  const int64_t units = (int64_t)p.B * p.HV * tiles;
  int64_t blocks = units;
  if (l.grid_cap > 0 && blocks > l.grid_cap) blocks = l.grid_cap;
  gdn_decode_kernel<K, NORM, ACT, VEC><<<dim3((unsigned)blocks), dim3(64 * wpb), 0, st>>>(p, tiles, rows_per_tile,
                                                                                       (int)units);
  return hipGetLastError();
}

template <int K, bool NORM>
hipError_t launch_act(const GdnParams& p, const Launch& l, hipStream_t st) {
  const bool vec = p.qkv_vec;
  switch (p.act_dt) {
    case SSMD_F32: return vec ? launch_k<K, NORM, SSMD_F32, true>(p, l, st) : launch_k<K, NORM, SSMD_F32, false>(p, l, st);
    case SSMD_BF16: return vec ? launch_k<K, NORM, SSMD_BF16, true>(p, l, st) : launch_k<K, NORM, SSMD_BF16, false>(p, l, st);
    default: return vec ? launch_k<K, NORM, SSMD_F16, true>(p, l, st) : launch_k<K, NORM, SSMD_F16, false>(p, l, st);
  }
}

template <int K>
hipError_t launch_norm(const GdnParams& p, const Launch& l, hipStream_t st) {
  return p.norm_gate ? launch_act<K, true>(p, l, st) : launch_act<K, false>(p, l, st);
}

}  // namespace

hipError_t launch_gdn(const GdnParams& p, const Launch& l, hipStream_t st) {
  switch (p.K) {
    case 16: return launch_norm<16>(p, l, st);
    case 32: return launch_norm<32>(p, l, st);
    case 64: return launch_norm<64>(p, l, st);
    case 128: return launch_norm<128>(p, l, st);
    case 256: return launch_norm<256>(p, l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
