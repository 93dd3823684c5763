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
#include <type_traits>

#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

constexpr int GCH = 64;  // tokens per chunk

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

// Staged activations keep their input encoding in LDS: raw 16-bit words for
// bf16/f16 inputs (half the LDS of fp32, so two blocks share a CU), fp32
// otherwise. Normalisation scales and gate factors are kept per token and
// applied to products, so the staged values stay the inputs' own.
template <int ACT>
using stg_t = typename std::conditional<ACT == SSMD_F32, float, uint16_t>::type;
template <int ACT>
using raw4_t = typename std::conditional<ACT == SSMD_F32, f4, uint2>::type;

template <int ACT, bool VEC>
__device__ __forceinline__ raw4_t<ACT> ld_raw4(const void* base, int64_t off) {
  if constexpr (ACT == SSMD_F32) {
    const float* p = static_cast<const float*>(base) + off;
    if constexpr (VEC) return *reinterpret_cast<const f4*>(p);
    else return f4{p[0], p[1], p[2], p[3]};
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if constexpr (VEC) return *reinterpret_cast<const uint2*>(p);
    else return uint2{p[0] | ((uint32_t)p[1] << 16), p[2] | ((uint32_t)p[3] << 16)};
  }
}

template <int ACT>
__device__ __forceinline__ float raw_to_f(uint32_t h) {
  if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(h);
  else return f16_bits_to_f32(h);
}

template <int ACT>
__device__ __forceinline__ f4 raw4_to_f4(raw4_t<ACT> v) {
  if constexpr (ACT == SSMD_F32) return v;
  else return f4{raw_to_f<ACT>(v.x & 0xffffu), raw_to_f<ACT>(v.x >> 16), raw_to_f<ACT>(v.y & 0xffffu),
                 raw_to_f<ACT>(v.y >> 16)};
}

template <int ACT>
__device__ __forceinline__ float stg_ld1(const stg_t<ACT>* p) {
  if constexpr (ACT == SSMD_F32) return *p;
  else return raw_to_f<ACT>(*p);
}

template <int ACT>
__device__ __forceinline__ void stg_st4(stg_t<ACT>* p, raw4_t<ACT> v) {
  if constexpr (ACT == SSMD_F32) *reinterpret_cast<f4*>(p) = v;
  else *reinterpret_cast<uint2*>(p) = v;
}

// One 16-index step of a Gram tile from two staged rows (each pointer at
// column k0 + 4 kk of its lane's row): fp32 storage takes four fp32 MFMAs,
// 16-bit storage one v_mfma_f32_16x16x16 on the raw words (products of 16-bit
// values are exact in fp32, so this matches the fp32 product up to summation
// order).
typedef short s4v __attribute__((ext_vector_type(4)));
typedef _Float16 h4v __attribute__((ext_vector_type(4)));
template <int ACT>
__device__ __forceinline__ f4v gram16(const stg_t<ACT>* a, const stg_t<ACT>* b, f4v c) {
  if constexpr (ACT == SSMD_F32) {
    return mma16(ld4s(a), ld4s(b), c);
  } else {
    const uint2 ua = *reinterpret_cast<const uint2*>(a), ub = *reinterpret_cast<const uint2*>(b);
    if constexpr (ACT == SSMD_BF16)
      return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v, ua), __builtin_bit_cast(s4v, ub), c,
                                                        0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4v, ua), __builtin_bit_cast(h4v, ub), c, 0,
                                                    0, 0);
  }
}

// Issues the loads of rows i < n of a [64][L] activation block (row i = element
// rbase + i * stride, columns coff .. coff + L - 1): 4 elements per group,
// group e = tid + 256 m, token e / (L / 4). Rows past n re-read row n - 1 (in
// bounds) and are zeroed when stored.
template <int ACT, bool VEC, int UM>
__device__ __forceinline__ void gch_load(const void* src, int64_t rbase, int64_t stride, int n, int64_t coff, int L,
                                         raw4_t<ACT> (&v)[UM]) {
  const int g = L / 4;
#pragma unroll
  for (int m = 0; m < UM; ++m) {
    const int e = threadIdx.x + 256 * m;
    const int i = e / g, col = 4 * (e - i * g);
    v[m] = ld_raw4<ACT, VEC>(src, rbase + (int64_t)min(i, n - 1) * stride + coff + col);
  }
}

template <int ACT, int UM>
__device__ __forceinline__ void gch_store(const raw4_t<ACT> (&v)[UM], int n, int L, stg_t<ACT>* dst, int ds) {
  const int g = L / 4;
#pragma unroll
  for (int m = 0; m < UM; ++m) {
    const int e = threadIdx.x + 256 * m;
    const int i = e / g, col = 4 * (e - i * g);
    raw4_t<ACT> w = v[m];
    if (i >= n) w = raw4_t<ACT>{};
    stg_st4<ACT>(dst + i * ds + col, w);
  }
}

// Per-token norm scale of a staged q or k block held in registers (L = K, so
// a token's K / 4 groups sit on K / 4 consecutive lanes of one wave):
// mul * rsqrt(|x|^2 + eps) with the L2 norm, else mul.
template <int ACT, int K, int UM>
__device__ __forceinline__ void gch_norm_scale(const raw4_t<ACT> (&v)[UM], const GdnParams& p, float mul,
                                               float* sc) {
  constexpr int g = K / 4;
#pragma unroll
  for (int m = 0; m < UM; ++m) {
    const f4 f = raw4_to_f4<ACT>(v[m]);
    float s = f.x * f.x + f.y * f.y + f.z * f.z + f.w * f.w;
    s = group_sum<16>(s);
    if constexpr (g == 32) s += __shfl_xor(s, 16);
    const int e = threadIdx.x + 256 * m;
    if ((e & (g - 1)) == 0) sc[e / g] = mul * (p.use_l2 ? rsqrtf(s + p.l2eps) : 1.f);
  }
}

template <int K, int ACT, bool VEC>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(GdnChunkParams cp) {
  using ST = stg_t<ACT>;
  const GdnParams& p = cp.g;
  constexpr int KS = K + 4;  // staged row stride (elements): aligned rows, staggered banks
  constexpr int TP = GCH + 4;
  const int V = p.V;
  const int VS = V + 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15, kk = lane >> 4;
  extern __shared__ float lds[];
  float* const AT = lds;                 // [64][TP]: A, then M (see the inverse below)
  float* const gam = AT + GCH * TP;      // per token: gamma_i
  float* const bet = gam + GCH;          //   beta_i
  float* const egam = bet + GCH;         //   e^gamma_i
  float* const ekc = egam + GCH;         //   e^(gamma_C - gamma_i)
  float* const qsc = ekc + GCH;          //   q scale (norm * K^-1/2)
  float* const ksc = qsc + GCH;          //   k scale (norm)
  float* const fq = ksc + GCH;           //   e^gamma_i q scale
  float* const fk = fq + GCH;            //   e^(gamma_C - gamma_i) k scale
  float* const fw = fk + GCH;            //   beta_i e^gamma_i k scale
  ST* const Qr = reinterpret_cast<ST*>(fw + GCH);  // [64][KS] raw q
  ST* const Kr = Qr + GCH * KS;                    // [64][KS] raw k
  ST* const Vr = Kr + GCH * KS;                    // [64][VS] raw v

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

  // ---- q, k, v of the chunk's tokens: every load issued before any store
  const int64_t rbase = ((int64_t)bi * cp.T + t0) * p.qkv_stride;
  {
    raw4_t<ACT> rq[K / 16], rk[K / 16];
    gch_load<ACT, VEC>(p.qkv, rbase, p.qkv_stride, n, (int64_t)h * K, K, rq);
    gch_load<ACT, VEC>(p.qkv, rbase, p.qkv_stride, n, (int64_t)(p.H + h) * K, K, rk);
    // gates of token `lane` (wave 0): inclusive prefix sum of g, beta, decay factors
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
      const float gl = __shfl(g, 63);
      gam[lane] = g;
      bet[lane] = be;
      egam[lane] = expf(g);
      ekc[lane] = expf(gl - g);
      if (lane == 0) gC[0] = gl;
    }
    gch_norm_scale<ACT, K>(rq, p, p.scale, qsc);
    gch_norm_scale<ACT, K>(rk, p, 1.f, ksc);
    gch_store<ACT>(rq, n, K, Qr, KS);
    gch_store<ACT>(rk, n, K, Kr, KS);
  }
  {
    raw4_t<ACT> rv[16];  // V <= 256: at most 16 groups per thread
    const int uv = V / 16;
#pragma unroll
    for (int m = 0; m < 16; ++m)
      if (m < uv) {
        const int e = tid + 256 * m, g = V / 4;
        const int i = e / g, col = 4 * (e - i * g);
        rv[m] = ld_raw4<ACT, VEC>(p.qkv, rbase + (int64_t)min(i, n - 1) * p.qkv_stride +
                                             2 * (int64_t)p.H * K + (int64_t)hv * V + col);
      }
#pragma unroll
    for (int m = 0; m < 16; ++m)
      if (m < uv) {
        const int e = tid + 256 * m, g = V / 4;
        const int i = e / g, col = 4 * (e - i * g);
        stg_st4<ACT>(Vr + i * VS + col, i < n ? rv[m] : raw4_t<ACT>{});
      }
  }
  __syncthreads();

  if (wave == 0) {
    fq[lane] = egam[lane] * qsc[lane];
    fk[lane] = ekc[lane] * ksc[lane];
    fw[lane] = bet[lane] * egam[lane] * ksc[lane];
  }
  // ---- Gram tiles (ti, tj), tj <= ti: 10 tiles over 4 waves.
  //      A_ij = beta_i e^(g_i - g_j) (k_i . k_j), j < i;  P_ij = e^(g_i - g_j) (q_i . k_j), j <= i
  for (int t = wave; t < 10; t += 4) {
    const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int tj = t - ti * (ti + 1) / 2;
    f4v qk = {0.f, 0.f, 0.f, 0.f}, kkm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k0 = 0; k0 < K; k0 += 16) {
      const ST* bk = Kr + (16 * tj + x) * KS + k0 + 4 * kk;
      qk = gram16<ACT>(Qr + (16 * ti + x) * KS + k0 + 4 * kk, bk, qk);
      kkm = gram16<ACT>(Kr + (16 * ti + x) * KS + k0 + 4 * kk, bk, kkm);
    }
    const int j = 16 * tj + x;
    const float gj = gam[j], kj = ksc[j];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      const float dec = j <= i ? expf(gam[i] - gj) * kj : 0.f;
      AT[i * TP + j] = j < i ? bet[i] * ksc[i] * dec * kkm[r] : 0.f;
      Pg[i * GCH + j] = qsc[i] * dec * qk[r];
    }
  }
  __syncthreads();

  // ---- M = (I + A)^-1 in 16x16 blocks, in place. The diagonal blocks by
  // forward substitution (wave b, lane m: column m of block b, held in
  // registers; row i is overwritten only after every lane has read it). The
  // blocks below the diagonal, row block by row block,
  //   M_ij = -M_ii sum_{k=j}^{i-1} A_ik M_kj   (i > j),
  // on the matrix cores, one (i, j) per wave; M_ij is stored in the unused
  // block above the diagonal, at block position (j, i), so A stays readable.
  // Hence the rows 16 j + r, columns 16 i + c of AT hold M_ij[r][c] for every
  // j <= i. An MFMA result in lane layout (lane x + 16 kk holds D[4 kk + r][x])
  // is exactly the B operand of the next product.
  if (lane < 16) {
    const int b0 = 16 * wave;
    float mc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = i == lane ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= AT[(b0 + i) * TP + b0 + j] * mc[j];
      mc[i] = s;
      AT[(b0 + i) * TP + b0 + lane] = s;
    }
  }
  // e^gamma q and (e^(gamma_C - gamma) k)^T to the workspace (scaled inputs)
  for (int e = tid; e < GCH * K / 4; e += 256) {
    const int i = e / (K / 4), col = 4 * (e - i * (K / 4));
    const float f = fq[i];
    const ST* s = Qr + i * KS + col;
    *reinterpret_cast<f4*>(Qg + i * K + col) =
        f4{f * stg_ld1<ACT>(s), f * stg_ld1<ACT>(s + 1), f * stg_ld1<ACT>(s + 2), f * stg_ld1<ACT>(s + 3)};
    const int kc = e / (GCH / 4), j = 4 * (e - kc * (GCH / 4));
    const ST* kr = Kr + j * KS + kc;
    *reinterpret_cast<f4*>(Kg + kc * GCH + j) = f4{fk[j] * stg_ld1<ACT>(kr), fk[j + 1] * stg_ld1<ACT>(kr + KS),
                                                   fk[j + 2] * stg_ld1<ACT>(kr + 2 * KS),
                                                   fk[j + 3] * stg_ld1<ACT>(kr + 3 * KS)};
  }
  __syncthreads();
  for (int ib = 1; ib < 4; ++ib) {
    if (wave < ib) {
      const int jb = wave;
      f4v z = {0.f, 0.f, 0.f, 0.f};
      for (int kb = jb; kb < ib; ++kb) {  // Z += A_(ib,kb) M_(kb,jb)
        const float* mcol = AT + (16 * jb + 4 * kk) * TP + 16 * kb + x;
        const f4 bm = {mcol[0], mcol[TP], mcol[2 * TP], mcol[3 * TP]};
        z = mma16(ld4s(AT + (16 * ib + x) * TP + 16 * kb + 4 * kk), bm, z);
      }
      f4v mij = {0.f, 0.f, 0.f, 0.f};
      mij = mma16(ld4s(AT + (16 * ib + x) * TP + 16 * ib + 4 * kk), f4{z[0], z[1], z[2], z[3]}, mij);
#pragma unroll
      for (int r = 0; r < 4; ++r) AT[(16 * jb + 4 * kk + r) * TP + 16 * ib + x] = -mij[r];
    }
    __syncthreads();
  }

  // ---- W = M diag(beta e^gamma) k and U = M diag(beta) V on the matrix
  // cores, one 16-column tile of W or U per task, all four row tiles at once:
  // the B tile of token block jb is built once and feeds row tiles ti >= jb
  // (M is lower triangular).
  const int ntk = K / 16, nt = ntk + V / 16;
  for (int tc0 = wave; tc0 < nt; tc0 += 4) {
    const bool isw = tc0 < ntk;
    const int tc = isw ? tc0 : tc0 - ntk;
    const ST* const Bm = (isw ? Kr : Vr) + 16 * tc + x;
    const int bs = isw ? KS : VS;
    const float* const fac = isw ? fw : bet;
    f4v acc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) acc[ti] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const int j = 16 * jb + 4 * kk;
      const f4 fj = ld4s(fac + j);
      const f4 b = {fj.x * stg_ld1<ACT>(Bm + j * bs), fj.y * stg_ld1<ACT>(Bm + (j + 1) * bs),
                    fj.z * stg_ld1<ACT>(Bm + (j + 2) * bs), fj.w * stg_ld1<ACT>(Bm + (j + 3) * bs)};
#pragma unroll
      for (int ti = jb; ti < 4; ++ti) acc[ti] = mma16(ld4s(AT + (16 * jb + x) * TP + 16 * ti + 4 * kk), b, acc[ti]);
    }
    float* dst = isw ? Wg : Ug;
    const int ld = isw ? K : V;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * ti + 4 * kk + r) * ld + 16 * tc + x] = acc[ti][r];
  }
}

// LDS bytes of one prep block.
inline size_t gch_prep_lds_bytes(int K, int V, int act) {
  const size_t es = act == SSMD_F32 ? 4 : 2;
  return sizeof(float) * ((size_t)GCH * (GCH + 4) + 9 * GCH) + es * ((size_t)2 * GCH * (K + 4) + (size_t)GCH * (V + 4));
}

// Pass 2: one block per (row, value head, VT state rows), chunks in order,
// the block's rows held in LDS. Wave w takes token tile w (16 tokens) for
// Delta and O, over all VT / 16 row tiles, so each W, e^gamma q and P operand
// it loads feeds VT / 16 products; for the new rows it takes column tiles w,
// w + 4 over all row tiles, each K-hat operand likewise shared. Larger VT
// reads the per-chunk operands fewer times (V / VT blocks per head read
// them), smaller VT gives more blocks; the host picks VT from the grid size.
// (Fetching a wave's next-chunk operands ahead was measured: 6% faster at one
// sequence, 45% slower at eight, from the registers it costs.)
template <int K, int VT, bool NORM>
__global__ __launch_bounds__(256) void gdn_chunk_state_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  constexpr int NRT = VT / 16;       // row tiles
  constexpr int NCT = K / 16;        // column tiles of the state
  constexpr int CPW = (NCT + 3) / 4; // column tiles per wave
  const int V = p.V;
  const int nvt = V / VT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15, kk = lane >> 4;
  constexpr int SP = K + 4;
  constexpr int DP = VT + 1;
  __shared__ float Ss[VT * SP];
  __shared__ float Ds[GCH * DP];  // Delta^T: [token][state row]

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
  const int v0 = vt * VT;
  float* const Sg = static_cast<float*>(p.state) + (((int64_t)slot * p.HV + hv) * V + v0) * (int64_t)K;
  for (int e = tid; e < VT * K / 4; e += 256) {
    const int r = e / (K / 4), col = 4 * (e - r * (K / 4));
    *reinterpret_cast<f4*>(Ss + r * SP + col) = *reinterpret_cast<const f4*>(Sg + r * K + col);
  }
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
    // X = W S^T and Y = (e^gamma q) S^T for this wave's 16 tokens, every row tile
    f4v X[NRT], Y[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) X[rt] = Y[rt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k0 = 0; k0 < K; k0 += 16) {
      const f4 aw = ld4s(Wg + (16 * ti + x) * K + k0 + 4 * kk);
      const f4 aq = ld4s(Qg + (16 * ti + x) * K + k0 + 4 * kk);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const f4 b = ld4s(Ss + (16 * rt + x) * SP + k0 + 4 * kk);
        X[rt] = mma16(aw, b, X[rt]);
        Y[rt] = mma16(aq, b, Y[rt]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * kk + r;
        Ds[i * DP + 16 * rt + x] = Ug[i * V + v0 + 16 * rt + x] - X[rt][r];  // Delta^T
      }
    __syncthreads();
    // O = Y + P Delta^T (P lower triangular: tokens < 16 (ti + 1))
    for (int j0 = 0; j0 < 16 * (ti + 1); j0 += 16) {
      const int j = j0 + 4 * kk;
      const f4 a = ld4s(Pg + (16 * ti + x) * GCH + j);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float* d = Ds + j * DP + 16 * rt + x;
        Y[rt] = mma16(a, f4{d[0], d[DP], d[2 * DP], d[3 * DP]}, Y[rt]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      if (t0 + i < len) {
        const int64_t o = (((int64_t)bi * cp.T + t0 + i) * p.HV + hv) * V + v0 + x;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          if constexpr (NORM) cp.obuf[o + 16 * rt] = Y[rt][r];
          else store_act1(p.out, o + 16 * rt, p.out_dt, Y[rt][r]);
        }
      }
    }
    // S <- e^(gamma_C) S + Delta (e^(gamma_C - gamma) k): column tiles wave + 4 q, every row tile
    f4v Sn[CPW][NRT];
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int tc = wave + 4 * q;
      if (tc < NCT) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) Sn[q][rt][r] = eg * Ss[(16 * rt + 4 * kk + r) * SP + 16 * tc + x];
      }
    }
#pragma unroll
    for (int j0 = 0; j0 < GCH; j0 += 16) {
      const int j = j0 + 4 * kk;
      f4 bk[CPW];
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
        const int tc = wave + 4 * q;
        if (tc < NCT) bk[q] = ld4s(Kg + (16 * tc + x) * GCH + j);
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float* d = Ds + j * DP + 16 * rt + x;
        const f4 a = {d[0], d[DP], d[2 * DP], d[3 * DP]};
#pragma unroll
        for (int q = 0; q < CPW; ++q)
          if (wave + 4 * q < NCT) Sn[q][rt] = mma16(a, bk[q], Sn[q][rt]);
      }
    }
    __syncthreads();  // every wave is done reading the old rows and Delta
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int tc = wave + 4 * q;
      if (tc < NCT) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) Ss[(16 * rt + 4 * kk + r) * SP + 16 * tc + x] = Sn[q][rt][r];
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < VT * K / 4; e += 256) {
    const int r = e / (K / 4), col = 4 * (e - r * (K / 4));
    *reinterpret_cast<f4*>(Sg + r * K + col) = *reinterpret_cast<const f4*>(Ss + r * SP + col);
  }
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
hipError_t launch_gch_k(const GdnChunkParams& cp, int n_cu, hipStream_t st) {
  const GdnParams& p = cp.g;
  const size_t lds = gch_prep_lds_bytes(K, p.V, ACT);
  const int64_t prep_blocks = (int64_t)p.B * p.HV * cp.nck;
  if (p.qkv_vec)
    gdn_chunk_prep_kernel<K, ACT, true><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
  else
    gdn_chunk_prep_kernel<K, ACT, false><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
  // state rows per block: the largest of 64 / 32 / 16 dividing V that still
  // gives two blocks per CU (16 otherwise)
  const int64_t bh8 = ((int64_t)p.B * p.HV + 7) / 8 * 8;
  int vt = 16;
  for (int c : {64, 32})
    if (p.V % c == 0 && bh8 * (p.V / c) >= 2LL * n_cu) {
      vt = c;
      break;
    }
  const dim3 sg((unsigned)(bh8 * (p.V / vt)));
  const bool nrm = p.norm_gate != nullptr;
  switch (vt * 2 + (nrm ? 1 : 0)) {
    case 128: gdn_chunk_state_kernel<K, 64, false><<<sg, dim3(256), 0, st>>>(cp); break;
    case 129: gdn_chunk_state_kernel<K, 64, true><<<sg, dim3(256), 0, st>>>(cp); break;
    case 64: gdn_chunk_state_kernel<K, 32, false><<<sg, dim3(256), 0, st>>>(cp); break;
    case 65: gdn_chunk_state_kernel<K, 32, true><<<sg, dim3(256), 0, st>>>(cp); break;
    case 32: gdn_chunk_state_kernel<K, 16, false><<<sg, dim3(256), 0, st>>>(cp); break;
    default: gdn_chunk_state_kernel<K, 16, true><<<sg, dim3(256), 0, st>>>(cp); break;
  }
  if (nrm) {
    const int64_t waves = (int64_t)p.B * cp.T * p.HV;
    gdn_chunk_norm_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st>>>(cp);
  }
  return hipGetLastError();
}

template <int K>
hipError_t launch_gch_act(const GdnChunkParams& cp, int n_cu, hipStream_t st) {
  switch (cp.g.act_dt) {
    case SSMD_F32: return launch_gch_k<K, SSMD_F32>(cp, n_cu, st);
    case SSMD_BF16: return launch_gch_k<K, SSMD_BF16>(cp, n_cu, st);
    default: return launch_gch_k<K, SSMD_F16>(cp, n_cu, st);
  }
}

}  // namespace

hipError_t launch_gdn_chunk(const GdnChunkParams& cp, int n_cu, hipStream_t st) {
  switch (cp.g.K) {
    case 64: return launch_gch_act<64>(cp, n_cu, st);
    case 128: return launch_gch_act<128>(cp, n_cu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
