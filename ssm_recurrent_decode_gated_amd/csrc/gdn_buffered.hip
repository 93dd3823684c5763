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

// 4-element ring loads per thread in the staging pass issued ahead of the
// state stream
constexpr int BUF_RU4 = 2;

template <int K>
constexpr int buf_rg() {
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 2 : 4));
}

template <int K, bool NORM, int ACT, bool VEC, int RG, int RU4>
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

  int bi, hv, tile;
  xcd_unit(blockIdx.x, p.B, p.H, p.HV, tiles_per_head, bi, hv, tile);
  const int slot = p.idx[bi];
  const int pos = p.write_pos[bi];
  if (slot < 0 || slot >= p.num_slots || pos < 0 || pos >= p.L) return;  // padded row
  const bool flush = pos == p.L - 1;
  const int G = p.HV / p.H;
  const int h = hv / G;
  const int V = p.V;
  float* S = static_cast<float*>(p.state) + ((int64_t)slot * p.HV + hv) * (int64_t)V * K;
  const int r0 = tile * rows_per_tile;
  const int r1 = min(V, r0 + rows_per_tile);
  const int64_t qrow = (int64_t)bi * p.qkv_stride;
  const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)hv * V;
  const int64_t gidx = (int64_t)bi * p.HV + hv;
  // rows of a pass are interleaved across the block's waves
  auto row_of = [&](int pass, int i) { return pass + (i * nwaves + wave) * RPI + rr; };

  // LDS: kr [pos][K] ring keys, dr [pos][rows_per_tile] ring deltas of this
  // tile, gl [pos] ring log decays, cf [pos + 1] coefficients (c_j, then
  // c_ck), ca / cg [pos] = c_j times the record's dot with k / q, rk / rq
  // [rows_per_tile] = the ring's share of (S_{p-1} k) and (S_{p-1} q) per row.
  extern __shared__ float lds[];
  float* kr = lds;
  float* dr = kr + pos * K;
  float* gl = dr + pos * rows_per_tile;
  float* cf = gl + pos;
  float* ca = cf + pos + 1;
  float* cg = ca + pos;
  float* rk = cg + pos;
  float* rq = rk + rows_per_tile;
  // this tile's outputs and deltas, written out as contiguous runs at the end
  // (scattered 2-byte stores inside a read-only stream cost far more than
  // their bytes); a tile has at most 256 rows without the norm, V <= 1024
  // with it
  __shared__ float o_lds[NORM ? 1024 : 256];
  __shared__ float d_lds[NORM ? 1024 : 256];
  __shared__ float red_lds[1];

  // ---- small loads first (activations, then this cycle's ring records
  // j < pos), then the checkpoint stream: waiting for the small ones never
  // waits for the stream. The ring staging issues up to RING_U loads per
  // thread before its first LDS store.
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
  const int64_t kr_g = ((int64_t)slot * p.H + h) * p.L * K;
  const int tr = r1 - r0;
  const int64_t dr_g = ((int64_t)slot * p.HV + hv) * p.L * V;
  const float* gr = p.g_cache + ((int64_t)slot * p.HV + hv) * p.L;
  const int nk = pos * K, nd = pos * tr, bd = blockDim.x;
  constexpr int RING_U = 8;
  float kt[RING_U], dt[RING_U];
  float gt = 0.f;
  // 16-bit rings with 8-byte aligned bases (the common case): 4 elements per
  // load, RU4 loads per thread (4 RU4 blockDim elements of each), issued
  // unconditionally (indices clamped into record 0 when the ring is empty)
  // and kept raw until the LDS stores, so nothing waits on them before the
  // state stream is issued.
  constexpr bool R16 = ACT != SSMD_F32;
  const bool rvec = R16 && (((reinterpret_cast<uintptr_t>(p.k_cache) | reinterpret_cast<uintptr_t>(p.d_cache)) & 7) == 0) &&
                    V % 4 == 0 && tr % 4 == 0;
  uint2 kt4[RU4], dt4[RU4];
  if (rvec) {
    const uint16_t* const kc = static_cast<const uint16_t*>(p.k_cache);
    const uint16_t* const dc = static_cast<const uint16_t*>(p.d_cache);
    const int nk4 = max(nk, 4), nd4 = max(nd, 4);
#pragma unroll
    for (int m = 0; m < RU4; ++m) {
      const int e = min(4 * (tid + m * bd), nk4 - 4);
      kt4[m] = *reinterpret_cast<const uint2*>(kc + kr_g + e);
    }
#pragma unroll
    for (int m = 0; m < RU4; ++m) {
      const int e = min(4 * (tid + m * bd), nd4 - 4);
      const int j = e / tr;
      dt4[m] = *reinterpret_cast<const uint2*>(dc + dr_g + (int64_t)j * V + r0 + (e - j * tr));
    }
    gt = gr[min(tid, max(pos - 1, 0))];
    __builtin_amdgcn_sched_barrier(0);  // ring loads ahead of the state stream
  } else if (pos > 0) {  // uniform: clamped indices, no per-element branch
#pragma unroll
    for (int m = 0; m < RING_U; ++m) kt[m] = ld_act<ACT>(p.k_cache, kr_g + min(tid + m * bd, nk - 1));
#pragma unroll
    for (int m = 0; m < RING_U; ++m) {
      const int e = min(tid + m * bd, nd - 1);
      const int j = e / tr;
      dt[m] = ld_act<ACT>(p.d_cache, dr_g + (int64_t)j * V + r0 + (e - j * tr));
    }
    gt = gr[min(tid, pos - 1)];
  }
  f4 s[RG][NV];
  float vv[RG];
  auto load_group = [&](int pass, int i) {
    const int row = min(row_of(pass, i), r1 - 1);  // past-the-end rows re-read the last one
    vv[i] = ld_act<ACT>(p.qkv, vbase + row);
#pragma unroll
    for (int j = 0; j < NV; ++j) s[i][j] = ld4<true>(S + (int64_t)row * K + RL::col(c, j));
  };
  int pass = r0;
#pragma unroll
  for (int i = 0; i < RG; ++i) load_group(pass, i);
  if (rvec) __builtin_amdgcn_sched_barrier(0);  // the ring's LDS stores behind it

  // ---- ring records to LDS (rare long rings finish with a plain loop)
  auto raw4 = [](uint2 v, float o[4]) {
    if constexpr (ACT == SSMD_BF16) {
      o[0] = __uint_as_float(v.x << 16);
      o[1] = __uint_as_float(v.x & 0xffff0000u);
      o[2] = __uint_as_float(v.y << 16);
      o[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
      o[0] = f16_bits_to_f32(v.x & 0xffffu);
      o[1] = f16_bits_to_f32(v.x >> 16);
      o[2] = f16_bits_to_f32(v.y & 0xffffu);
      o[3] = f16_bits_to_f32(v.y >> 16);
    }
  };
  if (rvec && pos > 0) {
#pragma unroll
    for (int m = 0; m < RU4; ++m) {
      const int e = 4 * (tid + m * bd);
      float f[4];
      if (e < nk) {
        raw4(kt4[m], f);
        *reinterpret_cast<f4*>(kr + e) = f4{f[0], f[1], f[2], f[3]};
      }
      if (e < nd) {
        const int j = e / tr;
        raw4(dt4[m], f);
        float* d = dr + j * rows_per_tile + (e - j * tr);
        d[0] = f[0];
        d[1] = f[1];
        d[2] = f[2];
        d[3] = f[3];
      }
    }
    for (int e = tid + 4 * RU4 * bd; e < nk; e += bd) kr[e] = ld_act<ACT>(p.k_cache, kr_g + e);
    for (int e = tid + 4 * RU4 * bd; e < nd; e += bd) {
      const int j = e / tr;
      dr[j * rows_per_tile + (e - j * tr)] = ld_act<ACT>(p.d_cache, dr_g + (int64_t)j * V + r0 + (e - j * tr));
    }
    if (tid < pos) gl[tid] = gt;
    for (int e = tid + bd; e < pos; e += bd) gl[e] = gr[e];
  } else if (pos > 0) {
#pragma unroll
    for (int m = 0; m < RING_U; ++m) {
      const int e = tid + m * bd;
      if (e < nk) kr[e] = kt[m];
      if (e < nd) {
        const int j = e / tr;
        dr[j * rows_per_tile + (e - j * tr)] = dt[m];
      }
    }
    for (int e = tid + RING_U * bd; e < nk; e += bd) kr[e] = ld_act<ACT>(p.k_cache, kr_g + e);
    for (int e = tid + RING_U * bd; e < nd; e += bd) {
      const int j = e / tr;
      dr[j * rows_per_tile + (e - j * tr)] = ld_act<ACT>(p.d_cache, dr_g + (int64_t)j * V + r0 + (e - j * tr));
    }
    if (tid < pos) gl[tid] = gt;
    for (int e = tid + bd; e < pos; e += bd) gl[e] = gr[e];
  }

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
  __syncthreads();

  // ---- replay coefficients: c_j = exp(sum_{j<i<pos} g_i), c_ck = exp(sum_{i<pos} g_i)
  if (tid <= pos) {
    float sum = 0.f;
    for (int i = (tid < pos ? tid + 1 : 0); i < pos; ++i) sum += gl[i];
    cf[tid] = expf(sum);
  }
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

  // ---- the ring's share of S_{p-1} k and S_{p-1} q, once per row
  for (int e = tid; e < 2 * tr; e += bd) {
    const int r = e < tr ? e : e - tr;
    const float* coef = e < tr ? ca : cg;
    float acc = 0.f;
    for (int j = 0; j < pos; ++j) acc += coef[j] * dr[j * rows_per_tile + r];
    (e < tr ? rk : rq)[r] = acc;
  }
  __syncthreads();
  const float cck = cf[pos];
  const int64_t obase = gidx * V;
  const int64_t dw = dr_g + (int64_t)pos * V;  // this step's delta record

  // ---- stream the checkpoint rows
  while (true) {
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
      const int row = row_of(pass, i);
      const int rowc = min(row, r1 - 1);
      const float sk = cck * dk + rk[rowc - r0];
      const float sqv = cck * dq + rq[rowc - r0];
      delta[i] = beta * (vv[i] - decay * sk);
      const float o = decay * sqv + delta[i] * kq;
      if (row < r1 && c == 0) {
        // a flush streams the state out anyway: its outputs go straight out
        // (the norm epilogue needs them in LDS); non-flush steps stage theirs
        if (NORM || !flush) o_lds[row - r0] = o;
        else store_act1(p.out, obase + row, p.out_dt, o);
        d_lds[row - r0] = delta[i];
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
          const int rowc = min(row_of(pass, i), r1 - 1);
          const float e = cj * dr[j * rows_per_tile + rowc - r0];
#pragma unroll
          for (int jj = 0; jj < NV; ++jj) s[i][jj] += e * kv[jj];
        }
      }
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int row = row_of(pass, i);
        if (row < r1) {
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            f4 n;
            n.x = decay * s[i][j].x + delta[i] * kf[4 * j];
            n.y = decay * s[i][j].y + delta[i] * kf[4 * j + 1];
            n.z = decay * s[i][j].z + delta[i] * kf[4 * j + 2];
            n.w = decay * s[i][j].w + delta[i] * kf[4 * j + 3];
            st4<true>(S + (int64_t)row * K + RL::col(c, j), n);
          }
        }
      }
    }
    pass += nwaves * ROWS;
    if (pass >= r1) break;
#pragma unroll
    for (int i = 0; i < RG; ++i) load_group(pass, i);
  }

  // ---- this step's record at position p: delta (this tile's rows), the key
  // (once per q/k head) and g. A flush appends none: the next cycle starts at
  // position 0, and a record at L-1 would never be read.
  if (!flush) {  // uniform over the block
    __syncthreads();
    // outputs (without the norm: the norm epilogue writes them) and this
    // step's delta record, in one pass
    const StoreRun ro{p.out, obase + r0, p.out_dt, o_lds, NORM ? 0 : r1 - r0};
    const StoreRun rd{p.d_cache, dw + r0, ACT, d_lds, r1 - r0};
    store_runs(ro, rd, tid, bd);
    if (tile == 0 && hv % G == 0 && wave == 0 && rr == 0) {
      const int64_t kw = kr_g + (int64_t)pos * K;
#pragma unroll
      for (int j = 0; j < NV; ++j) store4(p.k_cache, kw + RL::col(c, j), ACT, &kf[4 * j]);
    }
    if (tile == 0 && tid == 0) p.g_cache[((int64_t)slot * p.HV + hv) * p.L + pos] = g;
  }

  if constexpr (NORM) {
    if (flush) __syncthreads();  // (non-flush steps passed one above)
    if (wave == 0) {
      float ss = 0.f;
      for (int r = lane; r < V; r += 64) ss += o_lds[r] * o_lds[r];
      ss = wave_sum(ss);
      if (lane == 0) red_lds[0] = ss;
    }
    __syncthreads();
    const float inv = rsqrtf(red_lds[0] / (float)V + p.norm_eps);
    for (int r = tid; r < V; r += blockDim.x) {
      const float z = ld_act<ACT>(p.norm_gate, obase + r);
      const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
      const float w = p.norm_w ? p.norm_w[r] : 1.f;
      o_lds[r] = o_lds[r] * inv * w * gz;
    }
    __syncthreads();
    store_runs(StoreRun{p.out, obase, p.out_dt, o_lds, V}, StoreRun{p.out, obase, p.out_dt, o_lds, 0}, tid, bd);
  }
}

namespace {

template <int K, bool NORM, int ACT, bool VEC, int RG, int RU4>
hipError_t launch_bk_rg(const GdnParams& p, const Launch& l, hipStream_t st) {
  constexpr int RPI = RowLayout<K>::RPI;
  const int wave_rows = RG * RPI;
  int wpb = l.wpb;
  int tiles, rows_per_tile;
  if (NORM) {
    tiles = 1;
    rows_per_tile = p.V;
  } else {
    rows_per_tile = wpb * wave_rows;
    tiles = (p.V + rows_per_tile - 1) / rows_per_tile;
  }
  const int need = (min(p.V, rows_per_tile) + wave_rows - 1) / wave_rows;
  if (wpb > need) wpb = need;
  const size_t lds = buffered_lds_bytes(K, rows_per_tile, p.L);
  const dim3 grid((unsigned)((int64_t)p.B * p.HV * tiles));
  gdn_buffered_kernel<K, NORM, ACT, VEC, RG, RU4><<<grid, dim3(64 * wpb), lds, st>>>(p, tiles, rows_per_tile);
  return hipGetLastError();
}

// Full-height tiles by default (4 waves, or the launch's width): 16-row waves
// over 64-row tiles measured a faster flush phase (B = 64, L = 8: 50.0
// against 54.0 us) but slower non-flush phases (every tile repeats the ring
// staging and record dots), a slower cycle overall. buffered_launch below
// narrows the block instead where that measured faster.
template <int K, bool NORM, int ACT, bool VEC>
hipError_t launch_bk(const GdnParams& p, const Launch& l, hipStream_t st) {
  constexpr int RG = buf_rg<K>();
  if constexpr (K == 128 && !NORM) {
    if (!l.fixed && l.wpb == 1) {
      // L = 1: every step flushes with no record to fold, a plain in-place
      // stream: 1-wave blocks over 8-row tiles, as the packed step
      if (p.L == 1) return launch_bk_rg<K, NORM, ACT, VEC, 1, BUF_RU4>(p, l, st);
      // small batches: 1-wave blocks over 16-row tiles, so that a few heads
      // still spread over every CU; the staging pass ahead of the state
      // stream is made deep enough for the ring's L - 1 keys (64 threads x
      // 4 RU4 elements: 512, 1024 or 2048)
      const int64_t keys = (int64_t)(p.L - 1) * K;
      if (keys > 4LL * 2 * BUF_RU4 * 64) return launch_bk_rg<K, NORM, ACT, VEC, 2, 4 * BUF_RU4>(p, l, st);
      if (keys > 4LL * BUF_RU4 * 64) return launch_bk_rg<K, NORM, ACT, VEC, 2, 2 * BUF_RU4>(p, l, st);
      return launch_bk_rg<K, NORM, ACT, VEC, 2, BUF_RU4>(p, l, st);
    }
    // 2-wave blocks whose ring outgrows the default staging pass: a pass twice
    // as deep (the kernel's registers peak elsewhere: 162 VGPRs either way)
    if (!l.fixed && l.wpb == 2 && (int64_t)(p.L - 1) * K > 4LL * BUF_RU4 * 128)
      return launch_bk_rg<K, NORM, ACT, VEC, RG, 2 * BUF_RU4>(p, l, st);
  }
  return launch_bk_rg<K, NORM, ACT, VEC, RG, BUF_RU4>(p, l, st);
}

template <int K, bool NORM>
hipError_t launch_bact(const GdnParams& p, const Launch& l, hipStream_t st) {
  const bool vec = p.qkv_vec;
  switch (p.act_dt) {
    case SSMD_F32: return vec ? launch_bk<K, NORM, SSMD_F32, true>(p, l, st) : launch_bk<K, NORM, SSMD_F32, false>(p, l, st);
    case SSMD_BF16: return vec ? launch_bk<K, NORM, SSMD_BF16, true>(p, l, st) : launch_bk<K, NORM, SSMD_BF16, false>(p, l, st);
    default: return vec ? launch_bk<K, NORM, SSMD_F16, true>(p, l, st) : launch_bk<K, NORM, SSMD_F16, false>(p, l, st);
  }
}

template <int K>
hipError_t launch_bnorm(const GdnParams& p, const Launch& l, hipStream_t st) {
  return p.norm_gate ? launch_bact<K, true>(p, l, st) : launch_bact<K, false>(p, l, st);
}

}  // namespace

// LDS of the ring staging for a tile of `rows` rows: kr, dr, gl, cf, ca, cg,
// rk, rq (see the kernel); the host checks it against the budget.
size_t buffered_lds_bytes(int K, int rows, int L) {
  const size_t pm = (size_t)(L - 1);
  return sizeof(float) * (pm * (size_t)K + pm * (size_t)rows + 4 * pm + 1 + 2 * (size_t)rows);
}

// Block width of a buffered launch. 2-wave blocks (64-row tiles of 32-row
// waves at K = 128) for large batches (at least four heads per CU) whose ring
// of L - 1 records fits the staging pass issued ahead of the state stream
// (4 x RU4 elements per thread of 128; RU4 = 2 BUF_RU4 where BUF_RU4 does not
// suffice). Measured on MI355X (HV = 32, K = V = 128, bf16), cycle means:
// B = 64, L = 8 29.7 against 30.7 us with 4-wave blocks; L = 16 29.6 against
// 30.5 (33.0 with 2-wave blocks and a per-element loop for the records past
// the staging pass); B = 256, L = 8 / 16 99.8 / 96.4 against 101.4 / 99.4.
// The deeper pass costs a little where it is not needed (B = 64, L = 8: 30.0),
// and B = 16 stays faster with 4 waves. Below one head per CU, 1-wave blocks
// over 16-row tiles (8-row at L = 1) spread the few heads over every CU.
Launch buffered_launch(int K, bool norm, int L, int64_t heads, int n_cu, const Launch& l) {
  if (l.fixed || norm || K != 128) return l;
  // L = 1: 1-wave blocks over 8-row tiles (measured: B = 64 46.3 against 50.5 us
  // with the wide tiles, B = 256 170.8 against 187.3)
  if (L == 1 && heads >= 4LL * n_cu) return Launch{1, 0, 0};
  // small batches (fewer heads than CUs): 1-wave blocks over 16-row tiles
  // (8-row at L = 1). HV = 32, B = 1: L = 1 / 8 / 16 cycles 4.2 / 5.5 / 6.4
  // against 6.3 / 6.9 / 7.2 us with whole-head 4-wave blocks; from one head
  // per CU up the wider blocks are as fast or faster (B = 8: 8.6 / 8.6 / 8.8
  // against 9.4 / 8.6 / 10.2)
  if (heads < n_cu) return Launch{1, 0, 0};
  const int64_t deepest_pass = 4LL * 2 * BUF_RU4 * 128;
  if ((int64_t)(L - 1) * K <= deepest_pass && heads >= 4LL * n_cu) return Launch{2, 0, 0};
  return l;
}

int buffered_rows_per_tile(int K, int V, bool norm, const Launch& l) {
  if (norm) return V;
  switch (K) {
    case 16: return l.wpb * buf_rg<16>() * RowLayout<16>::RPI;
    case 32: return l.wpb * buf_rg<32>() * RowLayout<32>::RPI;
    case 64: return l.wpb * buf_rg<64>() * RowLayout<64>::RPI;
    case 128: return l.wpb * buf_rg<128>() * RowLayout<128>::RPI;
    default: return l.wpb * buf_rg<256>() * RowLayout<256>::RPI;
  }
}

hipError_t launch_gdn_buffered(const GdnParams& p, const Launch& l, hipStream_t st) {
  switch (p.K) {
    case 16: return launch_bnorm<16>(p, l, st);
    case 32: return launch_bnorm<32>(p, l, st);
    case 64: return launch_bnorm<64>(p, l, st);
    case 128: return launch_bnorm<128>(p, l, st);
    case 256: return launch_bnorm<256>(p, l, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
