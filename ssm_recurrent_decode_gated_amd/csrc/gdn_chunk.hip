// gdn_chunk.hip -- the GDN step over T tokens per sequence in chunked form
// (prefill), on gfx950.
//
// Tokens are grouped in chunks of C = 64. Within a chunk with cumulative log
// decay gamma_i = g_1 + ... + g_i and entering state S0 ([V, K], row = value
// index), unrolling the delta rule of "Optimization Log: Qwen3.5-27B Dense on
// B200" ("Kernel 4: Fused DeltaNet Recurrent", Math) gives
//   delta_i + beta_i sum_{j<i} e^(gamma_i - gamma_j) (k_i . k_j) delta_j
//       = beta_i (v_i - e^(gamma_i) S0 k_i)
// a unit lower-triangular system. With A_ij = beta_i e^(gamma_i - gamma_j)
// (k_i . k_j) for j < i and Tm = (I + A)^-1 diag(beta):
//   Delta^T = U - W S0^T,          U = Tm V,   W = Tm (e^gamma k)
//   O       = (e^gamma q) S0^T + P Delta^T,    P_ij = e^(gamma_i - gamma_j) (q_i . k_j), j <= i
//   S_C     = e^(gamma_C) S0 + Delta (e^(gamma_C - gamma) k)
// ("Triton decode kernel + MBU analysis", "Prefill path", leaves prefill to a
// chunked scan; this is its delta-rule form). Two passes:
//   1. prep, one block per (row, value head, chunk), state-free: q and k
//      normalised, gamma, beta, the Gram products, the triangular solve, W,
//      U, e^gamma q, e^(gamma_C - gamma) k and P, written to a workspace;
//   2. state, one block per (row, value head, 16 state rows), walking the
//      chunks in order with its 16 rows in LDS: Delta, O and the new rows.
//      The 16-row tiles of one head are mapped to one XCD, so their shared
//      per-chunk operands are read from that XCD's L2.
// With the gated RMSNorm (over a token's V outputs, split across tiles) pass
// 2 writes fp32 outputs to the workspace and a third pass normalises them.
// All arithmetic is fp32 (the products are small dense ones on the VALU).
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

constexpr int GCH = 64;  // tokens per chunk
constexpr int GCH_VT = 16;  // state rows per pass-2 block

// Per (row, value head, chunk) workspace record, in floats.
__host__ __device__ inline int64_t gch_rec_floats(int K, int V) {
  return 3LL * GCH * K + (int64_t)GCH * V + GCH * GCH + 4;
}

template <int K, int ACT>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  constexpr int KP = K + 1;  // padded row (LDS banks)
  const int V = p.V;
  const int VP = V + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  extern __shared__ float lds[];
  float* const Qs = lds;                  // [64][KP]; later V rows [64][VP]
  float* const Ks = Qs + GCH * (VP > KP ? VP : KP);
  float* const As = Ks + GCH * KP;        // [64][65]
  float* const Ts = As + GCH * 65;        // [64][65]
  float* const gam = Ts + GCH * 65;       // [64]
  float* const bet = gam + GCH;           // [64]

  const int c = blockIdx.x % cp.nck;
  const int bh = blockIdx.x / cp.nck;
  const int hv = bh % p.HV;
  const int bi = bh / p.HV;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;
  const int len = cp.lengths ? min(max(cp.lengths[bi], 0), cp.T) : cp.T;
  const int t0 = c * GCH;
  if (t0 >= len) return;
  const int n = min(GCH, len - t0);  // valid tokens; the rest act as absent (beta = g = 0, k = q = 0)
  const int h = hv / (p.HV / p.H);
  float* const rec = cp.ws + ((int64_t)bh * cp.nck + c) * gch_rec_floats(K, V);
  float* const Wg = rec;
  float* const Ug = Wg + GCH * K;
  float* const Qg = Ug + GCH * V;
  float* const Kg = Qg + GCH * K;
  float* const Pg = Kg + GCH * K;
  float* const gC = Pg + GCH * GCH;

  // ---- q, k of the chunk's tokens -> LDS (fp32)
  for (int e = tid; e < GCH * K; e += 256) {
    const int i = e / K, col = e - i * K;
    const int64_t row = ((int64_t)bi * cp.T + t0 + min(i, n - 1)) * p.qkv_stride;
    const bool ok = i < n;
    Qs[i * KP + col] = ok ? ld_act<ACT>(p.qkv, row + (int64_t)h * K + col) : 0.f;
    Ks[i * KP + col] = ok ? ld_act<ACT>(p.qkv, row + (int64_t)(p.H + h) * K + col) : 0.f;
  }
  // gates of token tid (wave 0), inclusive prefix sum of g
  if (wave == 0) {
    float g = 0.f, be = 0.f;
    if (lane < n) {
      const int64_t gi = ((int64_t)bi * cp.T + t0 + lane) * p.HV + hv;
      g = -expf(p.A_log[hv]) * softplus_f(ld_act<ACT>(p.a, gi) + p.dt_bias[hv]);
      be = sigmoid_f(ld_act<ACT>(p.b, gi));
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(g, d);
      if (lane >= d) g += o;
    }
    gam[lane] = g;
    bet[lane] = be;
  }
  __syncthreads();

  // ---- L2 norms (wave w: tokens 16w .. 16w + 15), q scale
  for (int i = wave * 16; i < wave * 16 + 16; ++i) {
    float sq = 0.f, sk = 0.f;
    for (int col = lane; col < K; col += 64) {
      sq += Qs[i * KP + col] * Qs[i * KP + col];
      sk += Ks[i * KP + col] * Ks[i * KP + col];
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    const float qs = p.scale * (p.use_l2 ? rsqrtf(sq + p.l2eps) : 1.f);
    const float ks = p.use_l2 ? rsqrtf(sk + p.l2eps) : 1.f;
    for (int col = lane; col < K; col += 64) {
      Qs[i * KP + col] *= qs;
      Ks[i * KP + col] *= ks;
    }
  }
  __syncthreads();

  // ---- Gram products, 4x4 blocks per thread (lower triangle only):
  //      A_ij = beta_i e^(g_i - g_j) (k_i . k_j), j < i;  P_ij = e^(g_i - g_j) (q_i . k_j), j <= i
  {
    const int bi4 = tid >> 4, bj4 = tid & 15;
    float qk[4][4] = {}, kk[4][4] = {};
    if (bj4 <= bi4) {
      for (int col = 0; col < K; ++col) {
        float qa[4], ka[4], kb[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          qa[x] = Qs[(4 * bi4 + x) * KP + col];
          ka[x] = Ks[(4 * bi4 + x) * KP + col];
          kb[x] = Ks[(4 * bj4 + x) * KP + col];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            qk[x][y] += qa[x] * kb[y];
            kk[x][y] += ka[x] * kb[y];
          }
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = 4 * bi4 + x, j = 4 * bj4 + y;
        const float dec = j <= i ? expf(gam[i] - gam[j]) : 0.f;
        As[i * 65 + j] = j < i ? bet[i] * dec * kk[x][y] : 0.f;
        Pg[i * GCH + j] = j <= i ? dec * qk[x][y] : 0.f;
      }
  }
  // e^gamma q and e^(gamma_C - gamma) k to the workspace
  const float gl = gam[GCH - 1];
  for (int e = tid; e < GCH * K; e += 256) {
    const int i = e / K, col = e - i * K;
    Qg[e] = expf(gam[i]) * Qs[i * KP + col];
    Kg[e] = expf(gl - gam[i]) * Ks[i * KP + col];
  }
  if (tid == 0) gC[0] = gl;
  __syncthreads();

  // ---- V rows into the q buffer; Tm = (I + A)^-1 diag(beta) by forward
  // substitution: wave w owns columns 16w .. 16w + 15, four lanes per column
  // splitting the sum over j
  for (int e = tid; e < GCH * V; e += 256) {
    const int i = e / V, col = e - i * V;
    const int64_t row = ((int64_t)bi * cp.T + t0 + min(i, n - 1)) * p.qkv_stride;
    Qs[i * VP + col] = i < n ? ld_act<ACT>(p.qkv, row + 2 * (int64_t)p.H * K + (int64_t)hv * V + col) : 0.f;
  }
  {
    const int m = wave * 16 + (lane & 15);
    const int part = lane >> 4;
    for (int i = 0; i < GCH; ++i) {
      float acc = 0.f;
      for (int j = part; j < i; j += 4) acc += As[i * 65 + j] * Ts[j * 65 + m];
      acc += __shfl_xor(acc, 16);
      acc += __shfl_xor(acc, 32);
      if (part == 0) Ts[i * 65 + m] = m <= i ? (m == i ? bet[i] : 0.f) - acc : 0.f;
    }
  }
  __syncthreads();

  // ---- W = Tm (e^gamma k), U = Tm V: 4 rows x 8 columns per thread
  {
    const int i4 = tid >> 4, c8 = tid & 15;
    for (int cb = c8 * 8; cb < K; cb += 128) {
      float w[4][8] = {};
      for (int j = 0; j <= 4 * i4 + 3; ++j) {
        const float ej = expf(gam[j]);
        float kr[8];
#pragma unroll
        for (int y = 0; y < 8; ++y) kr[y] = ej * Ks[j * KP + cb + y];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float tv = Ts[(4 * i4 + x) * 65 + j];
#pragma unroll
          for (int y = 0; y < 8; ++y) w[x][y] += tv * kr[y];
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y) Wg[(4 * i4 + x) * K + cb + y] = w[x][y];
    }
    for (int cb = c8 * 8; cb < V; cb += 128) {
      float u[4][8] = {};
      for (int j = 0; j <= 4 * i4 + 3; ++j) {
        float vr[8];
#pragma unroll
        for (int y = 0; y < 8; ++y) vr[y] = cb + y < V ? Qs[j * VP + cb + y] : 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float tv = Ts[(4 * i4 + x) * 65 + j];
#pragma unroll
          for (int y = 0; y < 8; ++y) u[x][y] += tv * vr[y];
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y)
          if (cb + y < V) Ug[(4 * i4 + x) * V + cb + y] = u[x][y];
    }
  }
}

// Pass 2: one block per (row, value head, 16 state rows), chunks in order.
template <int K, bool NORM>
__global__ __launch_bounds__(256) void gdn_chunk_state_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  const int V = p.V;
  const int nvt = V / GCH_VT;
  const int tid = threadIdx.x;
  __shared__ float Ss[GCH_VT][K + 4];
  __shared__ float Ds[GCH][GCH_VT + 1];
  __shared__ float Kh[GCH][K + 4];

  // XCD-aware block order: the tiles of one (row, head) share blockIdx % 8
  const int BH = p.B * p.HV;
  const int id = blockIdx.x;
  const int lo = id % 8, rest = id / 8;
  const int vt = rest % nvt;
  const int bh = (rest / nvt) * 8 + lo;
  if (bh >= BH) return;
  const int hv = bh % p.HV;
  const int bi = bh / p.HV;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;
  const int len = cp.lengths ? min(max(cp.lengths[bi], 0), cp.T) : cp.T;
  if (len == 0) return;
  const int v0 = vt * GCH_VT;
  float* const Sg = static_cast<float*>(p.state) + (((int64_t)slot * p.HV + hv) * V + v0) * (int64_t)K;
  for (int e = tid; e < GCH_VT * K; e += 256) Ss[e / K][e % K] = Sg[e];
  __syncthreads();

  const int nchunks = (len + GCH - 1) / GCH;
  for (int c = 0; c < nchunks; ++c) {
    const float* const rec = cp.ws + ((int64_t)bh * cp.nck + c) * gch_rec_floats(K, V);
    const float* const Wg = rec;
    const float* const Ug = Wg + GCH * K;
    const float* const Qg = Ug + GCH * V;
    const float* const Kg = Qg + GCH * K;
    const float* const Pg = Kg + GCH * K;
    const float gl = Pg[GCH * GCH];
    const int t0 = c * GCH;
    for (int e = tid; e < GCH * K; e += 256) Kh[e / K][e % K] = Kg[e];
    // X = W S^T, Y = (e^gamma q) S^T: token i, state rows 4 rg .. 4 rg + 3
    const int i = tid >> 2, rg = tid & 3;
    float x[4] = {}, y[4] = {};
    for (int col = 0; col < K; col += 4) {
      const f4 wv = *reinterpret_cast<const f4*>(Wg + i * K + col);
      const f4 qv = *reinterpret_cast<const f4*>(Qg + i * K + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* s = &Ss[4 * rg + r][col];
        x[r] += wv.x * s[0] + wv.y * s[1] + wv.z * s[2] + wv.w * s[3];
        y[r] += qv.x * s[0] + qv.y * s[1] + qv.z * s[2] + qv.w * s[3];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) Ds[i][4 * rg + r] = Ug[i * V + v0 + 4 * rg + r] - x[r];
    __syncthreads();
    // O = Y + P Delta^T (P lower triangular)
    float o[4] = {y[0], y[1], y[2], y[3]};
    for (int j = 0; j <= i; ++j) {
      const float pj = Pg[i * GCH + j];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] += pj * Ds[j][4 * rg + r];
    }
    if (t0 + i < len) {
      const int64_t orow = (((int64_t)bi * cp.T + t0 + i) * p.HV + hv) * V + v0 + 4 * rg;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (NORM) cp.obuf[orow + r] = o[r];
        else store_act1(p.out, orow + r, p.out_dt, o[r]);
      }
    }
    // S <- e^(gamma_C) S + Delta (e^(gamma_C - gamma) k): row r, 8 columns per thread
    {
      const int r = tid >> 4, cb = (tid & 15) * (K / 16);
      const float eg = expf(gl);
      float acc[K / 16];
#pragma unroll
      for (int q = 0; q < K / 16; ++q) acc[q] = eg * Ss[r][cb + q];
      for (int j = 0; j < GCH; ++j) {
        const float d = Ds[j][r];
#pragma unroll
        for (int q = 0; q < K / 16; ++q) acc[q] += d * Kh[j][cb + q];
      }
      __syncthreads();  // every thread is done reading the old rows and Delta
#pragma unroll
      for (int q = 0; q < K / 16; ++q) Ss[r][cb + q] = acc[q];
    }
    __syncthreads();
  }
  for (int e = tid; e < GCH_VT * K; e += 256) Sg[e] = Ss[e / K][e % K];
}

// Pass 3 (gated RMSNorm): one wave per (row, token, value head).
__global__ __launch_bounds__(256) void gdn_chunk_norm_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  const int V = p.V;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (int64_t)p.B * cp.T * p.HV) return;
  const int hv = (int)(wid % p.HV);
  const int64_t bt = wid / p.HV;
  const int bi = (int)(bt / cp.T);
  const int t = (int)(bt - (int64_t)bi * cp.T);
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;
  const int len = cp.lengths ? min(max(cp.lengths[bi], 0), cp.T) : cp.T;
  if (t >= len) return;
  const int64_t base = wid * V;
  float ss = 0.f;
  for (int r = lane; r < V; r += 64) ss += cp.obuf[base + r] * cp.obuf[base + r];
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)V + p.norm_eps);
  for (int r = lane; r < V; r += 64) {
    const float z = load_act1(p.norm_gate, base + r, p.act_dt);
    const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
    const float w = p.norm_w ? p.norm_w[r] : 1.f;
    store_act1(p.out, base + r, p.out_dt, cp.obuf[base + r] * inv * w * gz);
  }
}

int64_t gdn_chunk_workspace_floats(int B, int T, int HV, int K, int V, bool norm) {
  const int64_t nck = (T + GCH - 1) / GCH;
  return (int64_t)B * HV * nck * gch_rec_floats(K, V) + (norm ? (int64_t)B * T * HV * V : 0);
}

namespace {

template <int K, int ACT>
hipError_t launch_gch_k(const GdnChunkParams& cp, hipStream_t st) {
  const GdnParams& p = cp.g;
  const int KP = K + 1, VP = p.V + 1;
  const size_t lds = sizeof(float) * ((size_t)GCH * (VP > KP ? VP : KP) + (size_t)GCH * KP + 2 * GCH * 65 + 2 * GCH);
  const int64_t prep_blocks = (int64_t)p.B * p.HV * cp.nck;
  gdn_chunk_prep_kernel<K, ACT><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
  const int nvt = p.V / GCH_VT;
  const int64_t bh8 = ((int64_t)p.B * p.HV + 7) / 8 * 8;
  const int64_t state_blocks = bh8 * nvt;
  if (p.norm_gate) {
    gdn_chunk_state_kernel<K, true><<<dim3((unsigned)state_blocks), dim3(256), 0, st>>>(cp);
    const int64_t waves = (int64_t)p.B * cp.T * p.HV;
    gdn_chunk_norm_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st>>>(cp);
  } else {
    gdn_chunk_state_kernel<K, false><<<dim3((unsigned)state_blocks), dim3(256), 0, st>>>(cp);
  }
  return hipGetLastError();
}

template <int K>
hipError_t launch_gch_act(const GdnChunkParams& cp, hipStream_t st) {
  switch (cp.g.act_dt) {
    case SSMD_F32: return launch_gch_k<K, SSMD_F32>(cp, st);
    case SSMD_BF16: return launch_gch_k<K, SSMD_BF16>(cp, st);
    default: return launch_gch_k<K, SSMD_F16>(cp, st);
  }
}

}  // namespace

hipError_t launch_gdn_chunk(const GdnChunkParams& cp, hipStream_t st) {
  switch (cp.g.K) {
    case 64: return launch_gch_act<64>(cp, st);
    case 128: return launch_gch_act<128>(cp, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
