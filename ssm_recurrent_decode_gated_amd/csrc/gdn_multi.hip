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
// A wave keeps its rows (RG groups of RPI rows, K/LPR columns per lane) in
// registers for the whole call. The block stages the inputs of a chunk of
// tokens in LDS (coalesced loads spread over all its threads, the next
// chunk's loads in flight while the current chunk is computed); a prep pass
// then computes each token's per-head scalars once (normalised q and k,
// k . q, e^g, beta: one wave per token) instead of once per wave, and every
// wave streams its rows through the chunk's tokens. Rows of a head are split
// into tiles over blocks. The gated RMSNorm needs a token's whole head: with
// it, one block holds the head and each token takes one more barrier
// (per-wave partial sums of o^2 in LDS, double buffered by token parity).
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

// Row groups per wave (RG rows groups of RPI rows). Without the norm: two
// (one for K = 16), or one for small batches (twice the blocks per head, so
// a few heads still fill the GPU); deeper groups push K = 128 past 168
// VGPRs, below 3 waves per SIMD. With the norm a head must fit one block of
// at most 8 waves: the packed kernels' depth.
template <int K>
constexpr int gmulti_rg_plain() {
  return K == 16 ? 1 : 2;
}
template <int K>
constexpr int gmulti_rg_norm() {
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 2 : 4));
}
template <int K>
constexpr int gmulti_tc() {  // tokens staged per chunk
  return K == 256 ? 4 : 8;
}

// Token inputs of one chunk live in LDS as fp32, per token
//   [ q (K) | k (K) | v of the block's rows (R) | norm gate (R, NORM) | a | b | . ]
// padded to a multiple of 4 floats (pt), two chunk buffers. A prep pass then
// normalises q and k in place and turns a, b, . into e^g, beta, k . q.
template <int K, bool NORM, int ACT, int RG>
__global__ __launch_bounds__(512) void gdn_multi_kernel(GdnMultiParams mp) {
  const GdnParams& p = mp.g;
  using RL = RowLayout<K>;
  using E = typename std::conditional<ACT == SSMD_F32, float, uint16_t>::type;
  constexpr int TC = gmulti_tc<K>();
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI;
  constexpr int R4 = 4 * RG * RPI;  // rows of a 4-wave block
  extern __shared__ float lds[];
  __shared__ float red[2][NORM ? 8 : 1];
  const int tid = threadIdx.x;
  const int bd = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = bd >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  int bi, hv, tile;
  xcd_unit(blockIdx.x, p.B, p.H, p.HV, mp.tiles, bi, hv, tile);
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;  // padded row: touch nothing
  const int T = mp.T;
  const int len = mp.lengths ? min(max(mp.lengths[bi], 0), T) : T;
  if (len == 0) return;  // nothing to do: the state stays as it is
  const int h = hv / (p.HV / p.H);
  const int V = p.V;
  const int R = mp.rows_per_tile;
  const int r0 = tile * R;
  const int r1 = min(V, r0 + R);
  const int pt = mp.tok_floats;
  const int o_a = 2 * K + (NORM ? 2 : 1) * R;  // a, then b
  float* const S = static_cast<float*>(p.state) + ((int64_t)slot * p.HV + hv) * (int64_t)V * K;
  int rowc[RG];  // this lane's rows, clamped into the tile (rows past it are computed, never stored)
#pragma unroll
  for (int i = 0; i < RG; ++i) rowc[i] = min(r0 + (i * nwaves + wave) * RPI + rr, r1 - 1);

  // ---- staging: chunk t0 .. t0 + TC - 1 (tokens clamped into the row).
  // Each region is read from a block-uniform base with 32-bit element
  // offsets, so a pending load holds one offset register, not a 64-bit
  // address (the host keeps T * row stride below 2^31 elements).
  // Counts per thread for a block of 256 threads: every launch of this
  // kernel uses 4 to 8 waves, so one pass of these covers the chunk.
  constexpr int SQK = (TC * 2 * K + 255) / 256;  // q and k values per thread
  constexpr int SV = (TC * R4 + 255) / 256;      // v (and norm gate) values per thread
  E rq[SQK], rv[SV], rz[NORM ? SV : 1], rab;
  const E* const xq = static_cast<const E*>(p.qkv) + (int64_t)bi * T * p.qkv_stride;
  const E* const xz = NORM ? static_cast<const E*>(p.norm_gate) + ((int64_t)bi * T * p.HV + hv) * V : nullptr;
  const E* const xa = static_cast<const E*>(p.a) + (int64_t)bi * T * p.HV + hv;
  const E* const xb = static_cast<const E*>(p.b) + (int64_t)bi * T * p.HV + hv;
  const uint32_t stride = (uint32_t)p.qkv_stride;
  const uint32_t vcol = 2u * p.H * K + (uint32_t)hv * V;
  auto tok_of = [&](int t0, int u) { return (uint32_t)min(t0 + u, len - 1); };
  auto stage_load = [&](int t0) {
#pragma unroll
    for (int m = 0; m < SQK; ++m) {
      const int i = min(tid + m * bd, TC * 2 * K - 1);
      const int u = i / (2 * K), o = i - u * 2 * K;
      const uint32_t col = o < K ? (uint32_t)(h * K + o) : (uint32_t)((p.H + h) * K + (o - K));
      rq[m] = xq[tok_of(t0, u) * stride + col];
    }
#pragma unroll
    for (int m = 0; m < SV; ++m) {
      const int i = min(tid + m * bd, TC * R - 1);
      const int u = i / R, r = i - u * R;
      const uint32_t row = (uint32_t)min(r0 + r, r1 - 1);
      rv[m] = xq[tok_of(t0, u) * stride + vcol + row];
      if constexpr (NORM) rz[m] = xz[tok_of(t0, u) * (uint32_t)(p.HV * V) + row];
    }
    const int u = min(tid >> 1, TC - 1);
    rab = (tid & 1 ? xb : xa)[tok_of(t0, u) * (uint32_t)p.HV];
  };
  auto to_f = [](E x) -> float {
    if constexpr (ACT == SSMD_F32) return x;
    else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(x);
    else return f16_bits_to_f32(x);
  };
  auto stage_store = [&](int buf) {
    float* dst = lds + buf * TC * pt;
#pragma unroll
    for (int m = 0; m < SQK; ++m) {
      const int i = min(tid + m * bd, TC * 2 * K - 1);
      const int u = i / (2 * K);
      dst[u * pt + (i - u * 2 * K)] = to_f(rq[m]);
    }
#pragma unroll
    for (int m = 0; m < SV; ++m) {
      const int i = min(tid + m * bd, TC * R - 1);
      const int u = i / R, r = i - u * R;
      dst[u * pt + 2 * K + r] = to_f(rv[m]);
      if constexpr (NORM) dst[u * pt + 2 * K + R + r] = to_f(rz[m]);
    }
    if (tid < 2 * TC) dst[(tid >> 1) * pt + o_a + (tid & 1)] = to_f(rab);
  };

  // ---- first chunk's inputs, then the tile's rows (held for the whole call)
  stage_load(0);
  f4 s[RG][NV];
#pragma unroll
  for (int i = 0; i < RG; ++i)
#pragma unroll
    for (int j = 0; j < NV; ++j) s[i][j] = ld4<true>(S + (int64_t)rowc[i] * K + RL::col(c, j));
  const float A_log = p.A_log[hv];
  const float dt_bias = p.dt_bias[hv];
  stage_store(0);
  __syncthreads();

  // Per-token scalars, once per block: one wave per token L2-normalises q
  // (and scales it) and k in place in LDS and replaces a, b by the decay
  // e^g and beta, with k . q after them.
  auto prep = [&](int n, float* chunk) {
    constexpr int KM = (K + 63) / 64;
    for (int u = wave; u < n; u += nwaves) {
      float* tk = chunk + u * pt;
      float qv[KM], kv[KM];
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const int e = lane + 64 * m;
        qv[m] = e < K ? tk[e] : 0.f;
        kv[m] = e < K ? tk[K + e] : 0.f;
        sq += qv[m] * qv[m];
        sk += kv[m] * kv[m];
      }
      float qs = p.scale, ks = 1.f;
      if (p.use_l2) {
        qs *= rsqrtf(wave_sum(sq) + p.l2eps);
        ks = rsqrtf(wave_sum(sk) + p.l2eps);
      }
      float kq = 0.f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        const int e = lane + 64 * m;
        qv[m] *= qs;
        kv[m] *= ks;
        kq += qv[m] * kv[m];
        if (e < K) {
          tk[e] = qv[m];
          tk[K + e] = kv[m];
        }
      }
      kq = wave_sum(kq);
      if (lane == 0) {
        const float g = -expf(A_log) * softplus_f(tk[o_a] + dt_bias);
        tk[o_a] = expf(g);
        tk[o_a + 1] = sigmoid_f(tk[o_a + 1]);
        tk[o_a + 2] = kq;
      }
    }
  };

  auto compute = [&](int t, const float* tok) {
    float qf[NV * 4], kf[NV * 4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const f4 qv = *reinterpret_cast<const f4*>(tok + RL::col(c, j));
      const f4 kv = *reinterpret_cast<const f4*>(tok + K + RL::col(c, j));
      qf[4 * j] = qv.x; qf[4 * j + 1] = qv.y; qf[4 * j + 2] = qv.z; qf[4 * j + 3] = qv.w;
      kf[4 * j] = kv.x; kf[4 * j + 1] = kv.y; kf[4 * j + 2] = kv.z; kf[4 * j + 3] = kv.w;
    }
    const float decay = tok[o_a], beta = tok[o_a + 1], kq = tok[o_a + 2];
    const int64_t obase = (((int64_t)bi * T + t) * p.HV + hv) * V;
    float o[RG];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        dk += s[i][j].x * kf[4 * j] + s[i][j].y * kf[4 * j + 1] + s[i][j].z * kf[4 * j + 2] + s[i][j].w * kf[4 * j + 3];
        dq += s[i][j].x * qf[4 * j] + s[i][j].y * qf[4 * j + 1] + s[i][j].z * qf[4 * j + 2] + s[i][j].w * qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const float delta = beta * (tok[2 * K + (rowc[i] - r0)] - decay * dk);
      o[i] = decay * dq + delta * kq;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        s[i][j].x = decay * s[i][j].x + delta * kf[4 * j];
        s[i][j].y = decay * s[i][j].y + delta * kf[4 * j + 1];
        s[i][j].z = decay * s[i][j].z + delta * kf[4 * j + 2];
        s[i][j].w = decay * s[i][j].w + delta * kf[4 * j + 3];
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
          const float z = tok[2 * K + R + (rowc[i] - r0)];
          const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
          const float w = p.norm_w ? p.norm_w[row] : 1.f;
          store_act1(p.out, obase + row, p.out_dt, o[i] * inv * w * gz);
        }
      }
    }
  };

  // ---- chunks of TC tokens: the next chunk's loads are in flight while this
  // one is computed, then written to the other buffer and prepped (two
  // barriers a chunk)
  prep(min(TC, len), lds);
  __syncthreads();
  int buf = 0;
  for (int t0 = 0; t0 < len; t0 += TC) {
    const bool more = t0 + TC < len;
    if (more) stage_load(t0 + TC);
    const int n = min(TC, len - t0);
#pragma unroll 1
    for (int u = 0; u < n; ++u) compute(t0 + u, lds + buf * TC * pt + u * pt);
    if (more) {
      stage_store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      prep(min(TC, len - t0 - TC), lds + buf * TC * pt);
      __syncthreads();
    }
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

template <int K, bool NORM, int ACT, int RG>
hipError_t launch_gm_k(GdnMultiParams mp, int wpb, hipStream_t st) {
  const GdnParams& p = mp.g;
  mp.rows_per_tile = wpb * RG * RowLayout<K>::RPI;
  mp.tiles = NORM ? 1 : (p.V + mp.rows_per_tile - 1) / mp.rows_per_tile;
  mp.tok_floats = (2 * K + (NORM ? 2 : 1) * mp.rows_per_tile + 3 + 3) / 4 * 4;
  const size_t lds = 2 * (size_t)gmulti_tc<K>() * mp.tok_floats * sizeof(float);
  const int64_t blocks = (int64_t)p.B * p.HV * mp.tiles;
  gdn_multi_kernel<K, NORM, ACT, RG><<<dim3((unsigned)blocks), dim3(64 * wpb), lds, st>>>(mp);
  return hipGetLastError();
}

// Block shape: 4 waves, or (gated norm) enough waves for the whole head, up
// to 8. Without the norm, row groups drop to one per wave when the plain
// depth would give fewer than two blocks per CU.
template <int K, bool NORM, int ACT>
hipError_t launch_gm_shape(const GdnMultiParams& mp, const Launch& l, int n_cu, hipStream_t st) {
  const GdnParams& p = mp.g;
  if constexpr (NORM) {
    constexpr int RG = gmulti_rg_norm<K>();
    const int wave_rows = RG * RowLayout<K>::RPI;
    const int wpb = max(4, (p.V + wave_rows - 1) / wave_rows);
    return launch_gm_k<K, true, ACT, RG>(mp, wpb, st);
  } else {
    constexpr int RG = gmulti_rg_plain<K>();
    const int rows = 4 * RG * RowLayout<K>::RPI;
    const int64_t blocks = (int64_t)p.B * p.HV * ((p.V + rows - 1) / rows);
    // launch-shape sweeps: the staging above spreads a chunk's q, k and v
    // over at least 256 threads, so a fixed shape takes 4 to 8 waves
    if (l.fixed) return launch_gm_k<K, false, ACT, RG>(mp, min(max(l.wpb, 4), 8), st);
    if (RG == 1 || blocks >= 2LL * n_cu) return launch_gm_k<K, false, ACT, RG>(mp, 4, st);
    return launch_gm_k<K, false, ACT, 1>(mp, 4, st);
  }
}

template <int K, bool NORM>
hipError_t launch_gm_act(const GdnMultiParams& mp, const Launch& l, int n_cu, hipStream_t st) {
  switch (mp.g.act_dt) {
    case SSMD_F32: return launch_gm_shape<K, NORM, SSMD_F32>(mp, l, n_cu, st);
    case SSMD_BF16: return launch_gm_shape<K, NORM, SSMD_BF16>(mp, l, n_cu, st);
    default: return launch_gm_shape<K, NORM, SSMD_F16>(mp, l, n_cu, st);
  }
}

template <int K>
hipError_t launch_gm_norm(const GdnMultiParams& mp, const Launch& l, int n_cu, hipStream_t st) {
  return mp.g.norm_gate ? launch_gm_act<K, true>(mp, l, n_cu, st) : launch_gm_act<K, false>(mp, l, n_cu, st);
}

}  // namespace

int gdn_multi_max_norm_rows(int K) {
  switch (K) {
    case 16: return 8 * gmulti_rg_norm<16>() * RowLayout<16>::RPI;
    case 32: return 8 * gmulti_rg_norm<32>() * RowLayout<32>::RPI;
    case 64: return 8 * gmulti_rg_norm<64>() * RowLayout<64>::RPI;
    case 128: return 8 * gmulti_rg_norm<128>() * RowLayout<128>::RPI;
    default: return 8 * gmulti_rg_norm<256>() * RowLayout<256>::RPI;
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
