// gdn_buffered.hip -- GDN decode with the state written back once every L
// steps, on gfx950.
//
// Follows "Microbenchmark: buffered output-only GDN decode (ReplaySSM Part A)
// vs. the existing packed GDN decode kernel" (module docstring,
// `_bench_cfg`, `_state_bytes_per_step`): the pool holds a checkpoint S_ck
// that every step reads; each step appends a ring record (delta [V], the
// normalised key [K] shared by a q/k head, and g) at its phase p =
// write_pos[b]; only the phase p == L-1 writes the state back.
//
// The step's inputs need S_{p-1} k and S_{p-1} q, not S_{p-1} itself. With
// records j < p replayed as S <- e^{g_j} S + d_j k_j^T,
//   S_{p-1} = c_ck S_ck + sum_j c_j d_j k_j^T,
//   c_ck = exp(sum_{i<p} g_i),  c_j = exp(sum_{j<i<p} g_i),
// so per state row v:
//   (S_{p-1} k)_v = c_ck (S_ck k)_v + sum_j c_j (k_j . k) d_j[v]
// and the same with q. A non-flush step therefore streams S_ck once (read
// only) and adds p cheap ring terms per row; the flush step also materialises
// S_p = e^g (c_ck S_ck + sum_j c_j d_j k_j^T) + delta k^T and writes it.
// Ring records and the coefficients are staged in LDS once per block; the
// fold loops over records outermost so each record's key fragment is read
// from LDS once per row pass.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int K, int RG, bool NORM>
__global__ __launch_bounds__(512) void gdn_buffered_kernel(GdnParams p, int tiles_per_head,
                                                           int rows_per_tile) {
  using RL = RowLayout<K>;
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, ROWS = RG * RPI;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  int bid = blockIdx.x;
  const int tile = bid % tiles_per_head;
  bid /= tiles_per_head;
  const int hv = bid % p.HV;
  const int bi = bid / p.HV;
  const int slot = p.idx[bi];
  const int pos = p.write_pos[bi];
  if (slot < 0 || slot >= p.num_slots || pos < 0 || pos >= p.L) return;  // padded row
  const bool flush = pos == p.L - 1;
  const int G = p.HV / p.H;
  const int h = hv / G;
  const int V = p.V;
  float* S = p.state + ((int64_t)slot * p.HV + hv) * (int64_t)V * K;
  const int r0 = tile * rows_per_tile;
  const int r1 = min(V, r0 + rows_per_tile);
  const int64_t qrow = (int64_t)bi * p.qkv_stride;
  const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)hv * V;

  // LDS: kr [pos][K] ring keys, dr [pos][rows_per_tile] ring deltas of this
  // tile, cf [pos + 1] coefficients (c_j, then c_ck), ca / cg [pos] = c_j
  // times the record's dot with k / q.
  extern __shared__ float lds[];
  float* kr = lds;
  float* dr = kr + pos * K;
  float* cf = dr + pos * rows_per_tile;
  float* ca = cf + pos + 1;
  float* cg = ca + pos;
  __shared__ float o_lds[NORM ? 1024 : 1];
  __shared__ float red_lds[1];

  // ---- first pass of checkpoint loads
  int base = r0 + wave * ROWS;
  f4 s[RG][NV];
  float vv[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int row = base + i * RPI + rr;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      s[i][j] = row < r1 ? ld4<false>(S + (int64_t)row * K + RL::col(c, j)) : f4{0.f, 0.f, 0.f, 0.f};
    vv[i] = row < r1 ? load_act1(p.qkv, vbase + row, p.act_dt) : 0.f;
  }

  // ---- stage the ring records of this cycle (j < pos)
  const int64_t kr_g = ((int64_t)slot * p.H + h) * p.L * K;
  for (int e = tid; e < pos * K; e += blockDim.x) kr[e] = load_act1(p.k_cache, kr_g + e, p.act_dt);
  const int tr = r1 - r0;
  const int64_t dr_g = ((int64_t)slot * p.HV + hv) * p.L * V;
  for (int e = tid; e < pos * tr; e += blockDim.x) {
    const int j = e / tr, r = e - j * tr;
    dr[j * rows_per_tile + r] = load_act1(p.d_cache, dr_g + (int64_t)j * V + r0 + r, p.act_dt);
  }
  const float* gr = p.g_cache + ((int64_t)slot * p.HV + hv) * p.L;
  if (tid <= pos) {
    float sum = 0.f;
    for (int i = (tid < pos ? tid + 1 : 0); i < pos; ++i) sum += gr[i];
    cf[tid] = expf(sum);
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
  __syncthreads();

  // ---- record dots: lane group (wave, rr) takes records j = wave*RPI + rr + m*nwaves*RPI
  for (int j = wave * RPI + rr; j < pos; j += nwaves * RPI) {
    float al = 0.f, ga = 0.f;
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) {
      const f4 kv = *reinterpret_cast<const f4*>(kr + j * K + RL::col(c, jj));
      al += kv.x * kf[4 * jj] + kv.y * kf[4 * jj + 1] + kv.z * kf[4 * jj + 2] + kv.w * kf[4 * jj + 3];
      ga += kv.x * qf[4 * jj] + kv.y * qf[4 * jj + 1] + kv.z * qf[4 * jj + 2] + kv.w * qf[4 * jj + 3];
    }
    al = group_sum<LPR>(al);
    ga = group_sum<LPR>(ga);
    if (c == 0) {
      ca[j] = cf[j] * al;
      cg[j] = cf[j] * ga;
    }
  }
  __syncthreads();
  const float cck = cf[pos];
  const int64_t obase = gidx * V;
  const int64_t dw = dr_g + (int64_t)pos * V;  // this step's delta record

  // ---- stream the checkpoint rows
  while (base < r1) {
    float delta[RG];
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
      const int row = base + i * RPI + rr;
      float sk = cck * dk, sqv = cck * dq;
      if (row < r1) {
        const float* dcol = dr + (row - r0);
        for (int j = 0; j < pos; ++j) {
          const float d = dcol[j * rows_per_tile];
          sk += ca[j] * d;
          sqv += cg[j] * d;
        }
      }
      delta[i] = beta * (vv[i] - decay * sk);
      const float o = decay * sqv + delta[i] * kq;
      if (row < r1 && c == 0) {
        store_act1(p.d_cache, dw + row, p.act_dt, delta[i]);
        if constexpr (NORM) o_lds[row] = o;
        else store_act1(p.out, obase + row, p.out_dt, o);
      }
    }
    if (flush) {
      // fold the ring into the checkpoint rows, then apply this step
#pragma unroll
      for (int i = 0; i < RG; ++i)
#pragma unroll
        for (int j = 0; j < NV; ++j) s[i][j] *= cck;
      for (int j = 0; j < pos; ++j) {
        f4 kv[NV];
#pragma unroll
        for (int jj = 0; jj < NV; ++jj) kv[jj] = *reinterpret_cast<const f4*>(kr + j * K + RL::col(c, jj));
        const float cj = cf[j];
#pragma unroll
        for (int i = 0; i < RG; ++i) {
          const int row = base + i * RPI + rr;
          const float e = row < r1 ? cj * dr[j * rows_per_tile + row - r0] : 0.f;
#pragma unroll
          for (int jj = 0; jj < NV; ++jj) s[i][jj] += e * kv[jj];
        }
      }
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int row = base + i * RPI + rr;
        if (row < r1) {
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            f4 n;
            n.x = decay * s[i][j].x + delta[i] * kf[4 * j];
            n.y = decay * s[i][j].y + delta[i] * kf[4 * j + 1];
            n.z = decay * s[i][j].z + delta[i] * kf[4 * j + 2];
            n.w = decay * s[i][j].w + delta[i] * kf[4 * j + 3];
            st4<false>(S + (int64_t)row * K + RL::col(c, j), n);
          }
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
          s[i][j] = row < r1 ? ld4<false>(S + (int64_t)row * K + RL::col(c, j)) : f4{0.f, 0.f, 0.f, 0.f};
        vv[i] = row < r1 ? load_act1(p.qkv, vbase + row, p.act_dt) : 0.f;
      }
    }
  }

  // ---- append this step's key (once per q/k head) and g
  if (tile == 0 && hv % G == 0 && wave == 0 && rr == 0) {
    const int64_t kw = kr_g + (int64_t)pos * K;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) store_act1(p.k_cache, kw + RL::col(c, j) + e, p.act_dt, kf[4 * j + e]);
  }
  if (tile == 0 && tid == 0) p.g_cache[((int64_t)slot * p.HV + hv) * p.L + pos] = g;

  if constexpr (NORM) {
    __syncthreads();
    if (wave == 0) {
      float ss = 0.f;
      for (int r = lane; r < V; r += 64) ss += o_lds[r] * o_lds[r];
      ss = wave_sum(ss);
      if (lane == 0) red_lds[0] = ss;
    }
    __syncthreads();
    const float inv = rsqrtf(red_lds[0] / (float)V + p.norm_eps);
    for (int r = tid; r < V; r += blockDim.x) {
      const float z = load_act1(p.norm_gate, obase + r, p.act_dt);
      const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
      const float w = p.norm_w ? p.norm_w[r] : 1.f;
      store_act1(p.out, obase + r, p.out_dt, o_lds[r] * inv * w * gz);
    }
  }
}

namespace {

template <int K, int RG>
hipError_t launch_bk(const GdnParams& p, int wpb, hipStream_t st) {
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
  int need = (min(p.V, rows_per_tile) + wave_rows - 1) / wave_rows;
  if (wpb > need) wpb = need;
  const int pmax = p.L - 1;
  const size_t lds = sizeof(float) * ((size_t)pmax * K + (size_t)pmax * rows_per_tile + 3 * (size_t)pmax + 1);
  const dim3 grid((unsigned)((int64_t)p.B * p.HV * tiles));
  const dim3 block(64 * wpb);
  if (norm)
    gdn_buffered_kernel<K, RG, true><<<grid, block, lds, st>>>(p, tiles, rows_per_tile);
  else
    gdn_buffered_kernel<K, RG, false><<<grid, block, lds, st>>>(p, tiles, rows_per_tile);
  return hipGetLastError();
}

template <int K>
hipError_t launch_brg(const GdnParams& p, const Launch& l, hipStream_t st) {
  switch (l.rg) {
    case 1: return launch_bk<K, 1>(p, l.wpb, st);
    case 2: return launch_bk<K, 2>(p, l.wpb, st);
    case 4: return launch_bk<K, 4>(p, l.wpb, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gdn_buffered(const GdnParams& p, const Launch& l, hipStream_t st) {
  switch (p.K) {
    case 16: return launch_brg<16>(p, l, st);
    case 32: return launch_brg<32>(p, l, st);
    case 64: return launch_brg<64>(p, l, st);
    case 128: return launch_brg<128>(p, l, st);
    case 256: return launch_brg<256>(p, l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
