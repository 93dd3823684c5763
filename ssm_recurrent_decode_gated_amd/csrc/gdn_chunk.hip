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
// All arithmetic is fp32; the dense products run on the matrix cores
// (v_mfma_f32_16x16x4_f32), the triangular solve on the VALU.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

constexpr int GCH = 64;  // tokens per chunk
constexpr int GCH_VT = 16;  // state rows per pass-2 block

// Per (row, value head, chunk) workspace record, in floats:
//   W [64][K] | U [64][V] | e^gamma q [64][K] | (e^(gamma_C - gamma) k)^T [K][64] | P [64][64] | gamma_C
__host__ __device__ inline int64_t gch_rec_floats(int K, int V) {
  return 3LL * GCH * K + (int64_t)GCH * V + GCH * GCH + 4;
}

// The dense products run on the matrix cores: v_mfma_f32_16x16x4_f32 (fp32
// in and out). Lane l = x + 16 kk supplies A[x][k] and B[k][x] for one k of
// each step and holds D[4 kk + r][x] in register r. Four steps cover 16
// contraction indices; step e takes index k0 + 4 kk + e on lane group kk, so
// a lane's four A (and B) values are 4 consecutive elements of one row: one
// 128-bit load.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4v mma16(const f4 a, const f4 b, f4v c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f4 ld4s(const float* p) { return *reinterpret_cast<const f4*>(p); }

// Loads a [64][L] block of activations (row i = token row rbase + i * stride,
// columns coff .. coff + L - 1) into LDS at row stride ds, as fp32; rows
// i >= n are written as zeros. Groups of 4 elements, UM groups per thread
// (64 L / 4 <= 256 UM): every load of a thread is issued before its LDS
// writes, so the block waits one memory latency, not one per element.
template <int ACT, bool VEC, int UM>
__device__ __forceinline__ void gch_stage(const void* src, int64_t rbase, int64_t stride, int n, int64_t coff, int L,
                                          float* dst, int ds) {
  const int tid = threadIdx.x;
  const int total = GCH * L / 4;
  float v[UM][4];
#pragma unroll
  for (int m = 0; m < UM; ++m) {
    const int e = min(tid + 256 * m, total - 1);
    const int i = (4 * e) / L, col = 4 * e - i * L;
    ld_act4<ACT, VEC>(src, rbase + (int64_t)min(i, n - 1) * stride + coff + col, v[m]);
  }
#pragma unroll
  for (int m = 0; m < UM; ++m) {
    const int e = tid + 256 * m;
    if (e < total) {
      const int i = (4 * e) / L, col = 4 * e - i * L;
      const bool ok = i < n;
      float* d = dst + i * ds + col;
#pragma unroll
      for (int q = 0; q < 4; ++q) d[q] = ok ? v[m][q] : 0.f;
    }
  }
}

template <int K, int ACT, bool VEC>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  constexpr int KP = K + 4;  // row stride: 16-byte aligned rows, staggered banks
  constexpr int TP = GCH + 4;
  const int V = p.V;
  const int VP = V + 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15, kk = lane >> 4;
  extern __shared__ float lds[];
  float* const Qs = lds;                  // [64][KP]; later the V rows [64][VP]
  float* const Ks = Qs + GCH * (VP > KP ? VP : KP);
  float* const As = Ks + GCH * KP;        // [64][TP]
  float* const Ts = As + GCH * TP;        // [64][TP]
  float* const gam = Ts + GCH * TP;       // [64]
  float* const bet = gam + GCH;           // [64]
  float* const egam = bet + GCH;          // [64] e^gamma

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
  float* const Kg = Qg + GCH * K;  // transposed: [K][64]
  float* const Pg = Kg + GCH * K;
  float* const gC = Pg + GCH * GCH;

  // ---- q, k of the chunk's tokens -> LDS (fp32)
  const int64_t rbase = ((int64_t)bi * cp.T + t0) * p.qkv_stride;
  gch_stage<ACT, VEC, K / 16>(p.qkv, rbase, p.qkv_stride, n, (int64_t)h * K, K, Qs, KP);
  gch_stage<ACT, VEC, K / 16>(p.qkv, rbase, p.qkv_stride, n, (int64_t)(p.H + h) * K, K, Ks, KP);
  // gates of token `lane` (wave 0), inclusive prefix sum of g
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
    egam[lane] = expf(g);
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

  // ---- Gram products on the matrix cores, one 16x16 tile (ti, tj) at a time:
  //      A_ij = beta_i e^(g_i - g_j) (k_i . k_j), j < i;  P_ij = e^(g_i - g_j) (q_i . k_j), j <= i
  for (int t = wave; t < 16; t += 4) {
    const int ti = t >> 2, tj = t & 3;
    f4v qk = {0.f, 0.f, 0.f, 0.f}, kkm = {0.f, 0.f, 0.f, 0.f};
    if (tj <= ti) {
      for (int k0 = 0; k0 < K; k0 += 16) {
        const f4 bq = ld4s(Ks + (16 * tj + x) * KP + k0 + 4 * kk);
        qk = mma16(ld4s(Qs + (16 * ti + x) * KP + k0 + 4 * kk), bq, qk);
        kkm = mma16(ld4s(Ks + (16 * ti + x) * KP + k0 + 4 * kk), bq, kkm);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r, j = 16 * tj + x;
      const float dec = j <= i ? expf(gam[i] - gam[j]) : 0.f;
      As[i * TP + j] = j < i ? bet[i] * dec * kkm[r] : 0.f;
      Pg[i * GCH + j] = j <= i ? dec * qk[r] : 0.f;
    }
  }
  // e^gamma q and (e^(gamma_C - gamma) k)^T to the workspace
  const float gl = gam[GCH - 1];
  for (int e = tid; e < GCH * K; e += 256) {
    const int i = e / K, col = e - i * K;
    Qg[e] = egam[i] * Qs[i * KP + col];
    const int kc = e / GCH, j = e - kc * GCH;
    Kg[e] = expf(gl - gam[j]) * Ks[j * KP + kc];
  }
  if (tid == 0) gC[0] = gl;
  __syncthreads();

  // ---- V rows into the q buffer; M = (I + A)^-1 blockwise (Tm = M diag(beta),
  // with beta folded into the W and U products below). 16x16 blocks: the
  // diagonal blocks by forward substitution (wave b, lane m: column m of
  // block b, held in registers), then row block by row block
  //   M_ij = -M_ii sum_{k=j}^{i-1} A_ik M_kj   (i > j)
  // on the matrix cores, one (i, j) per wave. An MFMA result in lane layout
  // (lane x + 16 kk holds D[4 kk + r][x]) is exactly the B operand of the
  // next product, so Z = sum A_ik M_kj feeds -M_ii Z without a round trip.
  gch_stage<ACT, VEC, 16>(p.qkv, rbase, p.qkv_stride, n, 2 * (int64_t)p.H * K + (int64_t)hv * V, V, Qs, VP);
  if (lane < 16) {
    const int b0 = 16 * wave;
    float mc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float sacc = i == lane ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) sacc -= As[(b0 + i) * TP + b0 + j] * mc[j];
      mc[i] = sacc;
      Ts[(b0 + i) * TP + b0 + lane] = sacc;
    }
  }
  __syncthreads();
  for (int ib = 1; ib < 4; ++ib) {
    if (wave < ib) {
      const int jb = wave;
      f4v z = {0.f, 0.f, 0.f, 0.f};
      for (int kb = jb; kb < ib; ++kb) {  // Z += A_(ib,kb) M_(kb,jb)
        f4 bm;
        const float* mcol = Ts + (16 * kb + 4 * kk) * TP + 16 * jb + x;
        bm.x = mcol[0];
        bm.y = mcol[TP];
        bm.z = mcol[2 * TP];
        bm.w = mcol[3 * TP];
        z = mma16(ld4s(As + (16 * ib + x) * TP + 16 * kb + 4 * kk), bm, z);
      }
      f4v mij = {0.f, 0.f, 0.f, 0.f};
      mij = mma16(ld4s(Ts + (16 * ib + x) * TP + 16 * ib + 4 * kk), f4{z[0], z[1], z[2], z[3]}, mij);
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[(16 * ib + 4 * kk + r) * TP + 16 * jb + x] = -mij[r];
    }
    if (wave >= ib) {  // the blocks above the diagonal of this row block are zero
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jb = wave;  // column blocks ib .. 3 of rows 16 ib ..: only jb > ib are outside the solve
        if (jb > ib) Ts[(16 * ib + 4 * kk + r) * TP + 16 * jb + x] = 0.f;
      }
    }
    __syncthreads();
  }
  if (wave > 0) {  // row block 0: column blocks 1 .. 3 are zero
#pragma unroll
    for (int r = 0; r < 4; ++r) Ts[(4 * kk + r) * TP + 16 * wave + x] = 0.f;
  }
  __syncthreads();

  // ---- W = M diag(beta) (e^gamma k) and U = M diag(beta) V on the matrix
  // cores; M is lower triangular, so row tile ti only contracts over tokens
  // < 16 (ti + 1)
  const int ntk = K / 16, ntv = V / 16;
  for (int t = wave; t < 4 * (ntk + ntv); t += 4) {
    const bool isw = t < 4 * ntk;
    const int tt = isw ? t : t - 4 * ntk;
    const int ti = tt & 3, tc = tt >> 2;
    const float* Bm = isw ? Ks : Qs;
    const int bs = isw ? KP : VP;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < 16 * (ti + 1); j0 += 16) {
      f4 b;
      const int j = j0 + 4 * kk;
      const float* col = Bm + 16 * tc + x;
      b.x = col[(j + 0) * bs] * bet[j + 0] * (isw ? egam[j + 0] : 1.f);
      b.y = col[(j + 1) * bs] * bet[j + 1] * (isw ? egam[j + 1] : 1.f);
      b.z = col[(j + 2) * bs] * bet[j + 2] * (isw ? egam[j + 2] : 1.f);
      b.w = col[(j + 3) * bs] * bet[j + 3] * (isw ? egam[j + 3] : 1.f);
      acc = mma16(ld4s(Ts + (16 * ti + x) * TP + j), b, acc);
    }
    float* dst = isw ? Wg : Ug;
    const int ld = isw ? K : V;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * ti + 4 * kk + r) * ld + 16 * tc + x] = acc[r];
  }
}

// Pass 2: one block per (row, value head, 16 state rows), chunks in order.
// Wave w takes token tile w (16 tokens) for Delta and O, and column tiles
// w, w + 4 of the new rows. (Fetching a wave's next-chunk operands ahead
// was measured: 6% faster at one sequence, 45% slower at eight, from the
// registers it costs.)
template <int K, bool NORM>
__global__ __launch_bounds__(256) void gdn_chunk_state_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  const int V = p.V;
  const int nvt = V / GCH_VT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15, kk = lane >> 4;
  constexpr int SP = K + 4;
  __shared__ float Ss[GCH_VT * SP];
  __shared__ float Ds[GCH][GCH_VT + 1];

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
  for (int e = tid; e < GCH_VT * K; e += 256) Ss[(e / K) * SP + e % K] = Sg[e];
  __syncthreads();

  const int ti = wave;
  const int nchunks = (len + GCH - 1) / GCH;
  for (int c = 0; c < nchunks; ++c) {
    const float* const rec = cp.ws + ((int64_t)bh * cp.nck + c) * gch_rec_floats(K, V);
    const float* const Wg = rec;
    const float* const Ug = Wg + GCH * K;
    const float* const Qg = Ug + GCH * V;
    const float* const Kg = Qg + GCH * K;
    const float* const Pg = Kg + GCH * K;
    const float eg = expf(Pg[GCH * GCH]);
    const int t0 = c * GCH;
    // X = W S^T, Y = (e^gamma q) S^T for this wave's 16 tokens
    f4v X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += 16) {
      const f4 b = ld4s(Ss + x * SP + k0 + 4 * kk);
      X = mma16(ld4s(Wg + (16 * ti + x) * K + k0 + 4 * kk), b, X);
      Y = mma16(ld4s(Qg + (16 * ti + x) * K + k0 + 4 * kk), b, Y);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      Ds[i][x] = Ug[i * V + v0 + x] - X[r];  // Delta^T
    }
    __syncthreads();
    // O = Y + P Delta^T (P lower triangular: tokens < 16 (ti + 1))
    for (int j0 = 0; j0 < 16 * (ti + 1); j0 += 16) {
      const int j = j0 + 4 * kk;
      f4 b;
      b.x = Ds[j][x];
      b.y = Ds[j + 1][x];
      b.z = Ds[j + 2][x];
      b.w = Ds[j + 3][x];
      Y = mma16(ld4s(Pg + (16 * ti + x) * GCH + j), b, Y);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      if (t0 + i < len) {
        const int64_t o = (((int64_t)bi * cp.T + t0 + i) * p.HV + hv) * V + v0 + x;
        if constexpr (NORM) cp.obuf[o] = Y[r];
        else store_act1(p.out, o, p.out_dt, Y[r]);
      }
    }
    // S <- e^(gamma_C) S + Delta (e^(gamma_C - gamma) k): column tiles wave, wave + 4
    f4v Sn[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tc = wave + 4 * q;
      if (tc < K / 16) {
        f4v acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = eg * Ss[(4 * kk + r) * SP + 16 * tc + x];
        for (int j0 = 0; j0 < GCH; j0 += 16) {
          const int j = j0 + 4 * kk;
          f4 a;
          a.x = Ds[j][x];
          a.y = Ds[j + 1][x];
          a.z = Ds[j + 2][x];
          a.w = Ds[j + 3][x];
          acc = mma16(a, ld4s(Kg + (16 * tc + x) * GCH + j), acc);
        }
        Sn[q] = acc;
      }
    }
    __syncthreads();  // every wave is done reading the old rows and Delta
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tc = wave + 4 * q;
      if (tc < K / 16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Ss[(4 * kk + r) * SP + 16 * tc + x] = Sn[q][r];
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < GCH_VT * K; e += 256) Sg[e] = Ss[(e / K) * SP + e % K];
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
  const int KP = K + 4, VP = p.V + 4, TP = GCH + 4;
  const size_t lds = sizeof(float) * ((size_t)GCH * (VP > KP ? VP : KP) + (size_t)GCH * KP + 2 * GCH * TP + 3 * GCH);
  const int64_t prep_blocks = (int64_t)p.B * p.HV * cp.nck;
  if (p.qkv_vec)
    gdn_chunk_prep_kernel<K, ACT, true><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
  else
    gdn_chunk_prep_kernel<K, ACT, false><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
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
