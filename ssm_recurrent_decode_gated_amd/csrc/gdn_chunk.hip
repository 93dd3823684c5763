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
// (k_i . k_j) for j < i and M = (I + A)^-1:
//   Delta^T = M R,     R = diag(beta) V - diag(beta e^gamma) K S0^T
//   O       = diag(e^gamma) Q S0^T + P Delta^T,    P_ij = e^(gamma_i - gamma_j) (q_i . k_j), j <= i
//   S_C     = e^(gamma_C) S0 + Delta diag(e^(gamma_C - gamma)) K
// (q, k normalised; "Triton decode kernel + MBU analysis", "Prefill path",
// leaves prefill to a chunked scan; this is its delta-rule form). Two passes:
//   1. prep, one block per (row, value head, chunk), state-free: q and k
//      norms, gamma, beta, the Gram products, M by a blockwise triangular
//      inverse, and P, written to a small per-chunk record (M, P and five
//      per-token factors, 34 KB);
//   2. state, one block per (row, value head, VT state rows), walking the
//      chunks in order with its rows in LDS: R, Delta, O and the new rows,
//      from the raw q, k, v and the record. The row tiles of one head are
//      mapped to one XCD, so their shared per-chunk operands are read from
//      that XCD's L2.
// With the gated RMSNorm (over a token's V outputs, split across tiles) pass
// 2 writes fp32 outputs to the workspace and a third pass normalises them.
// All arithmetic is fp32 (16-bit inputs enter products exactly); the dense
// products run on the matrix cores, the diagonal blocks of the inverse on
// the VALU.
#include <atomic>
#include <type_traits>

#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

// Workspace of gdn_chunk_prefill_noalloc, for callers that cannot allocate:
// a fixed array in device memory, one per device (each device that loads
// this code holds its own copy until the process ends), shared by every
// call on that device. In host code `scratch` only names the symbol; its
// device address comes from hipGetSymbolAddress (gdn_chunk_scratch below).
static __device__ __align__(256) unsigned char scratch[SSMD_CHUNK_SCRATCH_BYTES];

constexpr int GCH = 64;  // tokens per chunk

// Per (row, value head, chunk) workspace record, in floats:
//   M [64][64] (blocks on and below the diagonal) | P [64][64] (likewise) |
//   fq [64] = e^gamma q-scale | fk [64] = e^(gamma_C - gamma) k-scale |
//   fw [64] = beta e^gamma k-scale | beta [64] | gamma_C, 3 spare
// Per-token factors are zero past the chunk's last valid token.
constexpr int GCH_M = 0, GCH_P = GCH * GCH, GCH_F = 2 * GCH * GCH;
constexpr int64_t GCH_REC = 2 * GCH * GCH + 4 * GCH + 4;

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

// gfx950's v_mfma_f32_16x16x32 (bf16 / f16 in, fp32 out): twice the
// contraction indices of the 16x16x16 form per instruction, at the part's full
// 16-bit matrix rate. Lane x + 16 kk supplies A[x][k] and B[k][x] for the 8
// indices k0 + 8 kk .. k0 + 8 kk + 7 (the same element order in A and B, so
// the sum over them is the contraction) and holds D[4 kk + r][x] in register r,
// as in the 16x16x16 form.
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
template <int ACT>
__device__ __forceinline__ f4v mma32(uint4 a, uint4 b, f4v c) {
  if constexpr (ACT == SSMD_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8v, a), __builtin_bit_cast(b8v, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, a), __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}
// 8 consecutive 16-bit values from LDS rows whose stride keeps them 8-byte
// (not 16-byte) aligned: two 64-bit reads.
__device__ __forceinline__ uint4 ld8h(const uint16_t* p) {
  const uint2 lo = *reinterpret_cast<const uint2*>(p), hi = *reinterpret_cast<const uint2*>(p + 4);
  return uint4{lo.x, lo.y, hi.x, hi.y};
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

template <int ACT>
__device__ __forceinline__ f4 stg_ld4(const stg_t<ACT>* p) {
  if constexpr (ACT == SSMD_F32) return ld4s(p);
  else return raw4_to_f4<ACT>(*reinterpret_cast<const uint2*>(p));
}

template <int K, int ACT, bool VEC>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(GdnChunkParams cp) {
  using ST = stg_t<ACT>;
  const GdnParams& p = cp.g;
  constexpr int KS = K + 4;  // staged row stride (elements): aligned rows, staggered banks
  constexpr int TP = GCH + 4;
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
  ST* const Qr = reinterpret_cast<ST*>(ksc + GCH);  // [64][KS] raw q
  ST* const Kr = Qr + GCH * KS;                     // [64][KS] raw k

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
  float* const rec = cp.ws + ((int64_t)bh * cp.nck + c) * GCH_REC;
  float* const Mg = rec + GCH_M;
  float* const Pg = rec + GCH_P;
  float* const Fg = rec + GCH_F;

  // ---- q, k of the chunk's tokens: every load issued before any store
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
      if (lane < 4) Fg[4 * GCH + lane] = lane == 0 ? gl : 0.f;
    }
    gch_norm_scale<ACT, K>(rq, p, p.scale, qsc);
    gch_norm_scale<ACT, K>(rk, p, 1.f, ksc);
    gch_store<ACT>(rq, n, K, Qr, KS);
    gch_store<ACT>(rk, n, K, Kr, KS);
  }
  __syncthreads();

  if (wave == 0) {  // the record's per-token factors, zero past the last valid token
    const bool ok = lane < n;
    Fg[lane] = ok ? egam[lane] * qsc[lane] : 0.f;
    Fg[GCH + lane] = ok ? ekc[lane] * ksc[lane] : 0.f;
    Fg[2 * GCH + lane] = ok ? bet[lane] * egam[lane] * ksc[lane] : 0.f;
    Fg[3 * GCH + lane] = ok ? bet[lane] : 0.f;
  }
  // ---- Gram tiles (ti, tj), tj <= ti: 10 tiles over 4 waves.
  //      A_ij = beta_i e^(g_i - g_j) (k_i . k_j), j < i;  P_ij = e^(g_i - g_j) (q_i . k_j), j <= i
  for (int t = wave; t < 10; t += 4) {
    const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int tj = t - ti * (ti + 1) / 2;
    f4v qk = {0.f, 0.f, 0.f, 0.f}, kkm = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ACT == SSMD_F32) {
#pragma unroll 4
      for (int k0 = 0; k0 < K; k0 += 16) {
        const ST* bk = Kr + (16 * tj + x) * KS + k0 + 4 * kk;
        qk = mma16(ld4s(Qr + (16 * ti + x) * KS + k0 + 4 * kk), ld4s(bk), qk);
        kkm = mma16(ld4s(Kr + (16 * ti + x) * KS + k0 + 4 * kk), ld4s(bk), kkm);
      }
    } else {  // raw 16-bit words, 32 indices per instruction
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += 32) {
        const uint4 bk = ld8h(Kr + (16 * tj + x) * KS + k0 + 8 * kk);
        qk = mma32<ACT>(ld8h(Qr + (16 * ti + x) * KS + k0 + 8 * kk), bk, qk);
        kkm = mma32<ACT>(ld8h(Kr + (16 * ti + x) * KS + k0 + 8 * kk), bk, kkm);
      }
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
  // ---- M to the workspace, row-major, the 10 blocks on and below the diagonal
  for (int e = tid; e < 10 * 64; e += 256) {
    const int t = e >> 6;
    const int ib = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int jb = t - ib * (ib + 1) / 2;
    const int r = (e & 63) >> 2, c4 = 4 * (e & 3);
    *reinterpret_cast<f4*>(Mg + (16 * ib + r) * GCH + 16 * jb + c4) = ld4s(AT + (16 * jb + r) * TP + 16 * ib + c4);
  }
}

// LDS bytes of one prep block.
inline size_t gch_prep_lds_bytes(int K, int act) {
  const size_t es = act == SSMD_F32 ? 4 : 2;
  return sizeof(float) * ((size_t)GCH * (GCH + 4) + 6 * GCH) + es * 2 * (size_t)GCH * (K + 4);
}

// Pass 2: one block per (row, value head, VT state rows), chunks in order,
// the block's rows in LDS. Per chunk: the chunk's raw k and the record's
// factors are staged in LDS; wave w takes token tile w (16 tokens) for
//   Z = K S^T, Y = Q S^T (q from memory, k from LDS), R = diag(beta) V - diag(fw) Z,
//   Delta^T = M R, O = diag(fq) Y + P Delta^T
// over every row tile, so each q, M and P operand it loads feeds VT / 16
// products; for the new rows S <- e^(gamma_C) S + Delta diag(fk) K it takes
// column tiles w, w + 4 over every row tile. Larger VT reads the per-chunk
// operands fewer times (V / VT blocks per head read them), smaller VT gives
// more blocks; the host picks VT from the grid size.
template <int K, int VT, bool NORM, int ACT>
__global__ __launch_bounds__(256) void gdn_chunk_state_kernel(GdnChunkParams cp) {
  using ST = stg_t<ACT>;
  const GdnParams& p = cp.g;
  constexpr int NRT = VT / 16;       // row tiles
  constexpr int NCT = K / 16;        // column tiles of the state
  constexpr int CPW = (NCT + 3) / 4; // column tiles per wave
  constexpr int SP = K + 4;
  constexpr int DP = VT + 1;
  constexpr int KS = K + 4;
  const int V = p.V;
  const int nvt = V / VT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15, kk = lane >> 4;
  __shared__ __attribute__((aligned(16))) float Ss[VT * SP];
  __shared__ __attribute__((aligned(16))) float Rs[GCH * DP];  // R, then Delta^T: [token][state row]
  __shared__ __attribute__((aligned(16))) ST Kst[GCH * KS];    // the chunk's raw k
  __shared__ __attribute__((aligned(16))) float Fs[4 * GCH + 4];  // fq | fk | fw | beta | gamma_C

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
  const int h = hv / (p.HV / p.H);
  const bool vec = p.qkv_vec;
  const int v0 = vt * VT;
  float* const Sg = static_cast<float*>(p.state) + (((int64_t)slot * p.HV + hv) * V + v0) * (int64_t)K;
  for (int e = tid; e < VT * K / 4; e += 256) {
    const int r = e / (K / 4), col = 4 * (e - r * (K / 4));
    *reinterpret_cast<f4*>(Ss + r * SP + col) = *reinterpret_cast<const f4*>(Sg + r * K + col);
  }

  const int ti = wave;
  const int nchunks = (len + GCH - 1) / GCH;
  for (int c = 0; c < nchunks; ++c) {
    const float* const rec = cp.ws + ((int64_t)bh * cp.nck + c) * GCH_REC;
    const int t0 = c * GCH;
    const int n = min(GCH, len - t0);
    const int64_t rbase = ((int64_t)bi * cp.T + t0) * p.qkv_stride;
    {
      raw4_t<ACT> rk[K / 16];
      if (vec) gch_load<ACT, true>(p.qkv, rbase, p.qkv_stride, n, (int64_t)(p.H + h) * K, K, rk);
      else gch_load<ACT, false>(p.qkv, rbase, p.qkv_stride, n, (int64_t)(p.H + h) * K, K, rk);
      f4 fv;
      if (tid < GCH + 1) fv = ld4s(rec + GCH_F + 4 * tid);
      gch_store<ACT>(rk, n, K, Kst, KS);
      if (tid < GCH + 1) *reinterpret_cast<f4*>(Fs + 4 * tid) = fv;
    }
    // this wave's rows of M and P (blocks on and below the diagonal)
    f4 mA[4], pA[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      if (jb <= ti) {
        mA[jb] = ld4s(rec + GCH_M + (16 * ti + x) * GCH + 16 * jb + 4 * kk);
        pA[jb] = ld4s(rec + GCH_P + (16 * ti + x) * GCH + 16 * jb + 4 * kk);
      }
    __syncthreads();  // Kst, Fs and the rows of S in place
    const float* const fq = Fs;
    const float* const fk = Fs + GCH;
    const float* const fw = Fs + 2 * GCH;
    const float* const bt = Fs + 3 * GCH;
    const float eg = expf(Fs[4 * GCH]);

    // Z = K S^T and Y = Q S^T for this wave's 16 tokens, every row tile
    f4v Y[NRT], Z[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) Y[rt] = Z[rt] = f4v{0.f, 0.f, 0.f, 0.f};
    const int64_t qoff = rbase + (int64_t)min(16 * ti + x, n - 1) * p.qkv_stride + (int64_t)h * K + 4 * kk;
    const ST* const krow = Kst + (16 * ti + x) * KS + 4 * kk;
#pragma unroll 4
    for (int k0 = 0; k0 < K; k0 += 16) {
      const f4 aq = vec ? raw4_to_f4<ACT>(ld_raw4<ACT, true>(p.qkv, qoff + k0))
                        : raw4_to_f4<ACT>(ld_raw4<ACT, false>(p.qkv, qoff + k0));
      const f4 ak = stg_ld4<ACT>(krow + k0);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const f4 b = ld4s(Ss + (16 * rt + x) * SP + k0 + 4 * kk);
        Y[rt] = mma16(aq, b, Y[rt]);
        Z[rt] = mma16(ak, b, Z[rt]);
      }
    }
    // R = diag(beta) V - diag(fw) Z (rows past n are zero: beta = fw = 0)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      const float fqi = fq[i], fwi = fw[i], bti = bt[i];
      const int64_t vo = rbase + (int64_t)min(i, n - 1) * p.qkv_stride + 2 * (int64_t)p.H * K + (int64_t)hv * V +
                         v0 + x;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        Rs[i * DP + 16 * rt + x] = bti * ld_act<ACT>(p.qkv, vo + 16 * rt) - fwi * Z[rt][r];
        Y[rt][r] *= fqi;
      }
    }
    __syncthreads();
    // Delta^T = M R (M lower triangular: tokens < 16 (ti + 1))
    f4v D[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) D[rt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      if (jb <= ti) {
        const int j = 16 * jb + 4 * kk;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const float* d = Rs + j * DP + 16 * rt + x;
          D[rt] = mma16(mA[jb], f4{d[0], d[DP], d[2 * DP], d[3 * DP]}, D[rt]);
        }
      }
    __syncthreads();  // every wave has read R
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Rs[(16 * ti + 4 * kk + r) * DP + 16 * rt + x] = D[rt][r];
    __syncthreads();
    // O = Y + P Delta^T
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      if (jb <= ti) {
        const int j = 16 * jb + 4 * kk;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const float* d = Rs + j * DP + 16 * rt + x;
          Y[rt] = mma16(pA[jb], f4{d[0], d[DP], d[2 * DP], d[3 * DP]}, Y[rt]);
        }
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      if (i < n) {
        const int64_t o = (((int64_t)bi * cp.T + t0 + i) * p.HV + hv) * V + v0 + x;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          if constexpr (NORM) cp.obuf[o + 16 * rt] = Y[rt][r];
          else store_act1(p.out, o + 16 * rt, p.out_dt, Y[rt][r]);
        }
      }
    }
    // S <- e^(gamma_C) S + Delta diag(fk) K: column tiles wave + 4 q, every row tile
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
        if (tc < NCT) {
          const ST* kc = Kst + j * KS + 16 * tc + x;
          bk[q] = f4{fk[j] * stg_ld1<ACT>(kc), fk[j + 1] * stg_ld1<ACT>(kc + KS),
                     fk[j + 2] * stg_ld1<ACT>(kc + 2 * KS), fk[j + 3] * stg_ld1<ACT>(kc + 3 * KS)};
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float* d = Rs + j * DP + 16 * rt + x;
        const f4 a = {d[0], d[DP], d[2 * DP], d[3 * DP]};
#pragma unroll
        for (int q = 0; q < CPW; ++q)
          if (wave + 4 * q < NCT) Sn[q][rt] = mma16(a, bk[q], Sn[q][rt]);
      }
    }
    __syncthreads();  // every wave is done reading the old rows, Delta, Kst and Fs
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
  }
  __syncthreads();
  for (int e = tid; e < VT * K / 4; e += 256) {
    const int r = e / (K / 4), col = 4 * (e - r * (K / 4));
    *reinterpret_cast<f4*>(Sg + r * K + col) = *reinterpret_cast<const f4*>(Ss + r * SP + col);
  }
}

// ---- bf16 inputs: three-way split products
// An fp32 value v splits exactly into three bf16 values, v = h + m + l: h is v
// rounded to bf16, m the remainder rounded, l the rest (at most 8 significant
// bits, so exact). A product of a bf16 operand with v is then the sum of three
// exact bf16 x bf16 products, accumulated in fp32: fp32 accuracy at the bf16
// matrix-core rate (v_mfma_f32_16x16x32_bf16 covers 32 contraction indices;
// v_mfma_f32_16x16x4_f32 covers 4, at a lower rate).
__device__ __forceinline__ void split3(float v, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = f32_to_bf16_bits(v);
  const float r1 = v - bf16_bits_to_f32(h);
  m = f32_to_bf16_bits(r1);
  l = f32_to_bf16_bits(r1 - bf16_bits_to_f32(m));
}

__device__ __forceinline__ f4v mma_bf16(uint4 a, uint4 b, f4v c) { return mma32<SSMD_BF16>(a, b, c); }

// A (bf16, one lane's 8 values) times B given as three bf16 planes.
__device__ __forceinline__ f4v mma_x3(uint4 a, uint4 bh, uint4 bm, uint4 bl, f4v c) {
  c = mma_bf16(a, bl, c);
  c = mma_bf16(a, bm, c);
  return mma_bf16(a, bh, c);
}

// Pass 2 for bf16 inputs: the pass above with Z = K S^T, Y = Q S^T and the row
// update (Delta diag(fk)) K as three-way split products. The block's rows live
// in registers across chunks (the row-update accumulators: lane x + 16 kk
// holds rows 16 rt + 4 kk + r, column 16 tc + x) and in LDS only as their
// three bf16 planes, the B operand of Z and Y; Delta diag(fk) is written as
// three planes too, row-major over tokens, the A operand of the row update.
template <int K, int VT, bool NORM>
__global__ __launch_bounds__(256) void gdn_chunk_state_x3_kernel(GdnChunkParams cp) {
  const GdnParams& p = cp.g;
  constexpr int NRT = VT / 16;       // row tiles
  constexpr int NCT = K / 16;        // column tiles of the state
  constexpr int CPW = (NCT + 3) / 4; // column tiles per wave
  constexpr int SB = K + 4;          // plane row stride (16-bit elements)
  constexpr int DB = GCH + 4;        // Delta-plane row stride
  constexpr int DP = VT + 1;
  constexpr int KS = K + 4;
  const int V = p.V;
  const int nvt = V / VT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15, kk = lane >> 4;
  __shared__ __attribute__((aligned(16))) uint16_t Sp[3][VT * SB];  // the rows of S as bf16 planes
  __shared__ __attribute__((aligned(16))) uint16_t Dq[3][VT * DB];  // Delta diag(fk) as bf16 planes: [state row][token]
  __shared__ __attribute__((aligned(16))) float Rs[GCH * DP];  // R, then Delta^T: [token][state row]
  __shared__ __attribute__((aligned(16))) uint16_t Kst[GCH * KS];  // the chunk's raw k
  __shared__ __attribute__((aligned(16))) float Fs[4 * GCH + 4];  // fq | fk | fw | beta | gamma_C

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
  const int h = hv / (p.HV / p.H);
  const bool vec = p.qkv_vec;
  const int v0 = vt * VT;
  float* const Sg = static_cast<float*>(p.state) + (((int64_t)slot * p.HV + hv) * V + v0) * (int64_t)K;

  // this wave's part of S: column tiles wave + 4 q, every row tile, in registers
  f4v Sn[CPW][NRT];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int tc = wave + 4 * q;
    if (tc < NCT) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sn[q][rt][r] = Sg[(16 * rt + 4 * kk + r) * K + 16 * tc + x];
    }
  }
  auto put_planes = [&]() {
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      const int tc = wave + 4 * q;
      if (tc < NCT) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint32_t a, b, c;
            split3(Sn[q][rt][r], a, b, c);
            const int o = (16 * rt + 4 * kk + r) * SB + 16 * tc + x;
            Sp[0][o] = (uint16_t)a;
            Sp[1][o] = (uint16_t)b;
            Sp[2][o] = (uint16_t)c;
          }
      }
    }
  };
  put_planes();

  const int ti = wave;
  const int nchunks = (len + GCH - 1) / GCH;
  for (int c = 0; c < nchunks; ++c) {
    const float* const rec = cp.ws + ((int64_t)bh * cp.nck + c) * GCH_REC;
    const int t0 = c * GCH;
    const int n = min(GCH, len - t0);
    const int64_t rbase = ((int64_t)bi * cp.T + t0) * p.qkv_stride;
    // every global load of the chunk is issued here, before the first wait:
    // raw k (to LDS), the factors, this wave's rows of M and P, its q operands
    // and the v values of its R entries
    const int64_t qoff = rbase + (int64_t)min(16 * ti + x, n - 1) * p.qkv_stride + (int64_t)h * K + 8 * kk;
    uint4 qa[K / 32];
    uint32_t vr[4][NRT];
    f4 mA[4], pA[4];
    {
      raw4_t<SSMD_BF16> rk[K / 16];
      if (vec) gch_load<SSMD_BF16, true>(p.qkv, rbase, p.qkv_stride, n, (int64_t)(p.H + h) * K, K, rk);
      else gch_load<SSMD_BF16, false>(p.qkv, rbase, p.qkv_stride, n, (int64_t)(p.H + h) * K, K, rk);
      f4 fv;
      if (tid < GCH + 1) fv = ld4s(rec + GCH_F + 4 * tid);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        if (jb <= ti) {
          mA[jb] = ld4s(rec + GCH_M + (16 * ti + x) * GCH + 16 * jb + 4 * kk);
          pA[jb] = ld4s(rec + GCH_P + (16 * ti + x) * GCH + 16 * jb + 4 * kk);
        }
#pragma unroll
      for (int m = 0; m < K / 32; ++m) {
        const uint2 lo = vec ? ld_raw4<SSMD_BF16, true>(p.qkv, qoff + 32 * m)
                             : ld_raw4<SSMD_BF16, false>(p.qkv, qoff + 32 * m);
        const uint2 hi = vec ? ld_raw4<SSMD_BF16, true>(p.qkv, qoff + 32 * m + 4)
                             : ld_raw4<SSMD_BF16, false>(p.qkv, qoff + 32 * m + 4);
        qa[m] = uint4{lo.x, lo.y, hi.x, hi.y};
      }
      const uint16_t* const vq = static_cast<const uint16_t*>(p.qkv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t vo = rbase + (int64_t)min(16 * ti + 4 * kk + r, n - 1) * p.qkv_stride +
                           2 * (int64_t)p.H * K + (int64_t)hv * V + v0 + x;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) vr[r][rt] = vq[vo + 16 * rt];
      }
      gch_store<SSMD_BF16>(rk, n, K, Kst, KS);
      if (tid < GCH + 1) *reinterpret_cast<f4*>(Fs + 4 * tid) = fv;
    }
    __syncthreads();  // Kst, Fs and the planes of S in place
    const float* const fq = Fs;
    const float* const fk = Fs + GCH;
    const float* const fw = Fs + 2 * GCH;
    const float* const bt = Fs + 3 * GCH;
    const float eg = expf(Fs[4 * GCH]);

    // Z = K S^T and Y = Q S^T, three-way split in S
    f4v Y[NRT], Z[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) Y[rt] = Z[rt] = f4v{0.f, 0.f, 0.f, 0.f};
    const uint16_t* const krow = Kst + (16 * ti + x) * KS + 8 * kk;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32) {
      const uint4 aq = qa[k0 / 32];
      const uint4 ak = ld8h(krow + k0);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int o = (16 * rt + x) * SB + k0 + 8 * kk;
        const uint4 bh = ld8h(&Sp[0][o]), bm = ld8h(&Sp[1][o]), bl = ld8h(&Sp[2][o]);
        Y[rt] = mma_x3(aq, bh, bm, bl, Y[rt]);
        Z[rt] = mma_x3(ak, bh, bm, bl, Z[rt]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      const float fqi = fq[i], fwi = fw[i], bti = bt[i];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        Rs[i * DP + 16 * rt + x] = bti * bf16_bits_to_f32(vr[r][rt]) - fwi * Z[rt][r];
        Y[rt][r] *= fqi;
      }
    }
    __syncthreads();
    // Delta^T = M R
    f4v D[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) D[rt] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      if (jb <= ti) {
        const int j = 16 * jb + 4 * kk;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const float* d = Rs + j * DP + 16 * rt + x;
          D[rt] = mma16(mA[jb], f4{d[0], d[DP], d[2 * DP], d[3 * DP]}, D[rt]);
        }
      }
    __syncthreads();  // every wave has read R
    {
      // Delta^T into Rs; Delta diag(fk) as planes: lane x + 16 kk holds tokens
      // 16 ti + 4 kk .. + 3 of state row 16 rt + x, one 64-bit store per plane
      const f4 fk4 = ld4s(fk + 16 * ti + 4 * kk);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        uint32_t a[4], b[4], cc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Rs[(16 * ti + 4 * kk + r) * DP + 16 * rt + x] = D[rt][r];
          split3(D[rt][r] * fk4[r], a[r], b[r], cc[r]);
        }
        const int o = (16 * rt + x) * DB + 16 * ti + 4 * kk;
        *reinterpret_cast<uint2*>(&Dq[0][o]) = uint2{a[0] | (a[1] << 16), a[2] | (a[3] << 16)};
        *reinterpret_cast<uint2*>(&Dq[1][o]) = uint2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        *reinterpret_cast<uint2*>(&Dq[2][o]) = uint2{cc[0] | (cc[1] << 16), cc[2] | (cc[3] << 16)};
      }
    }
    __syncthreads();
    // O = Y + P Delta^T
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      if (jb <= ti) {
        const int j = 16 * jb + 4 * kk;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const float* d = Rs + j * DP + 16 * rt + x;
          Y[rt] = mma16(pA[jb], f4{d[0], d[DP], d[2 * DP], d[3 * DP]}, Y[rt]);
        }
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * kk + r;
      if (i < n) {
        const int64_t o = (((int64_t)bi * cp.T + t0 + i) * p.HV + hv) * V + v0 + x;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          if constexpr (NORM) cp.obuf[o + 16 * rt] = Y[rt][r];
          else store_act1(p.out, o + 16 * rt, p.out_dt, Y[rt][r]);
        }
      }
    }
    // S <- e^(gamma_C) S + (Delta diag(fk)) K, three-way split in Delta diag(fk)
#pragma unroll
    for (int q = 0; q < CPW; ++q)
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Sn[q][rt] *= eg;
#pragma unroll
    for (int j0 = 0; j0 < GCH; j0 += 32) {
      const int j = j0 + 8 * kk;
      uint4 bk[CPW];
#pragma unroll
      for (int q = 0; q < CPW; ++q) {
        const int tc = wave + 4 * q;
        if (tc < NCT) {
          const uint16_t* kc = Kst + j * KS + 16 * tc + x;
          bk[q] = uint4{kc[0] | ((uint32_t)kc[KS] << 16), kc[2 * KS] | ((uint32_t)kc[3 * KS] << 16),
                        kc[4 * KS] | ((uint32_t)kc[5 * KS] << 16), kc[6 * KS] | ((uint32_t)kc[7 * KS] << 16)};
        }
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int o = (16 * rt + x) * DB + j;
        const uint4 ah = ld8h(&Dq[0][o]), am = ld8h(&Dq[1][o]), al = ld8h(&Dq[2][o]);
#pragma unroll
        for (int q = 0; q < CPW; ++q)
          if (wave + 4 * q < NCT) {
            Sn[q][rt] = mma_bf16(al, bk[q], Sn[q][rt]);
            Sn[q][rt] = mma_bf16(am, bk[q], Sn[q][rt]);
            Sn[q][rt] = mma_bf16(ah, bk[q], Sn[q][rt]);
          }
      }
    }
    __syncthreads();  // every wave is done reading the planes, Delta, Kst and Fs
    put_planes();
  }
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int tc = wave + 4 * q;
    if (tc < NCT) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sg[(16 * rt + 4 * kk + r) * K + 16 * tc + x] = Sn[q][rt][r];
    }
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

hipError_t gdn_chunk_scratch(void** ptr) {
  // device address of `scratch`, looked up once per device with that device
  // current (concurrent first calls store the same value)
  static std::atomic<void*> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    void* c = cache[dev].load(std::memory_order_acquire);
    if (c) {
      *ptr = c;
      return hipSuccess;
    }
  }
  void* a = nullptr;
  e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!a) return hipErrorInvalidSymbol;
  if (dev >= 0 && dev < 64) cache[dev].store(a, std::memory_order_release);
  *ptr = a;
  return hipSuccess;
}

int64_t gdn_chunk_workspace_floats(int B, int T, int HV, int K, int V, bool norm) {
  (void)K;
  const int64_t nck = (T + GCH - 1) / GCH;
  return (int64_t)B * HV * nck * GCH_REC + (norm ? (int64_t)B * T * HV * V : 0);
}

namespace {

template <int K, int VT, int ACT>
void launch_gch_state(const GdnChunkParams& cp, dim3 grid, hipStream_t st) {
  if (cp.g.norm_gate) gdn_chunk_state_kernel<K, VT, true, ACT><<<grid, dim3(256), 0, st>>>(cp);
  else gdn_chunk_state_kernel<K, VT, false, ACT><<<grid, dim3(256), 0, st>>>(cp);
}

template <int K, int ACT>
hipError_t launch_gch_k(const GdnChunkParams& cp, int n_cu, hipStream_t st) {
  const GdnParams& p = cp.g;
  const size_t lds = gch_prep_lds_bytes(K, ACT);
  const int64_t prep_blocks = (int64_t)p.B * p.HV * cp.nck;
  if (p.qkv_vec)
    gdn_chunk_prep_kernel<K, ACT, true><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
  else
    gdn_chunk_prep_kernel<K, ACT, false><<<dim3((unsigned)prep_blocks), dim3(256), lds, st>>>(cp);
  // state rows per block: the largest of 64 / 32 / 16 (32 / 16 for the bf16
  // split kernel, whose LDS holds one block per CU at 64) dividing V that
  // still gives two blocks per CU (16 otherwise)
  const int64_t bh8 = ((int64_t)p.B * p.HV + 7) / 8 * 8;
  int vt = 16;
  for (int c : {64, 32})
    if ((ACT != SSMD_BF16 || c < 64) && p.V % c == 0 && bh8 * (p.V / c) >= 2LL * n_cu) {
      vt = c;
      break;
    }
  const dim3 sg((unsigned)(bh8 * (p.V / vt)));
  if constexpr (ACT == SSMD_BF16) {
    const bool nrm = p.norm_gate != nullptr;
    if (vt == 32) {
      if (nrm) gdn_chunk_state_x3_kernel<K, 32, true><<<sg, dim3(256), 0, st>>>(cp);
      else gdn_chunk_state_x3_kernel<K, 32, false><<<sg, dim3(256), 0, st>>>(cp);
    } else {
      if (nrm) gdn_chunk_state_x3_kernel<K, 16, true><<<sg, dim3(256), 0, st>>>(cp);
      else gdn_chunk_state_x3_kernel<K, 16, false><<<sg, dim3(256), 0, st>>>(cp);
    }
  } else if (vt == 64) {
    launch_gch_state<K, 64, ACT>(cp, sg, st);
  } else if (vt == 32) {
    launch_gch_state<K, 32, ACT>(cp, sg, st);
  } else {
    launch_gch_state<K, 16, ACT>(cp, sg, st);
  }
  if (p.norm_gate) {
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
