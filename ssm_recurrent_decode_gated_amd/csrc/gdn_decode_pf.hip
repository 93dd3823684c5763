// gdn_decode_pf.hip -- packed GDN decode (no output norm). Same arithmetic
// and row layout as gdn_decode.hip. Blocks take work units (batch row, value
// head, row tile); where the grid is smaller than the unit count they walk
// the units with a grid stride, each wave holding the next unit's state pass
// in registers while it computes and stores the current one.
//
// Launch shape (measured on MI355X, HV = 32, K = V = 128; see the
// launcher): at large batches one 1-wave block per 8-row tile, so every block
// is a single short read-then-write burst (B = 256: 170.6 us, 6.29 TB/s of
// state). In-place streams on this part run faster the less each block and
// wave holds: many short bursts in flight at once keep HBM busier than a few
// long ones (a plain in-place copy: 5.6 TB/s with 64 KB per block, 6.3 with
// 8 KB, 6.6 with 4 KB). Small batches launch one block per 16-row tile (up
// to B = 8 at HV = 32) or per 128-row unit (at most two per CU).
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

// Rows per wave per unit: 32 for K = 64/128 (16 KB of state), fewer where a
// second unit would not fit the register file.
template <int K>
constexpr int pf_rg() {
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 1 : 4));
}

// VF: the unit's v values are loaded ahead of its state rows, so the
// conversion of v waits for nothing but v and each row group is computed and
// stored as it arrives (used at small batches, a few 1-wave blocks per CU).
template <int K, int ACT, bool VEC, int RG, bool VF>
__global__ __launch_bounds__(512) void gdn_decode_pf_kernel(GdnParams p, int tiles_per_head,
                                                            int rows_per_tile, int n_units) {
  using RL = RowLayout<K>;
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;

  struct Unit {
    int slot, bi, hv, h, r0, r1;
    float qf[NV * 4], kf[NV * 4], vv[RG], av, bv, A_log, dt_bias;
    f4 s[RG][NV];
  };
  auto fetch = [&](int unit, Unit& U) {
    int tile;
    xcd_unit(unit, p.B, p.H, p.HV, tiles_per_head, U.bi, U.hv, tile);
    U.h = U.hv / (p.HV / p.H);
    U.slot = p.idx[U.bi];
    if (U.slot < 0 || U.slot >= p.num_slots) return;
    U.r0 = tile * rows_per_tile;
    U.r1 = min(p.V, U.r0 + rows_per_tile);
    const int64_t qrow = (int64_t)U.bi * p.qkv_stride;
    const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)U.hv * p.V;
    const int64_t gidx = (int64_t)U.bi * p.HV + U.hv;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)U.h * K + RL::col(c, j), &U.qf[4 * j]);
      ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)(p.H + U.h) * K + RL::col(c, j), &U.kf[4 * j]);
    }
    U.av = ld_act<ACT>(p.a, gidx);
    U.bv = ld_act<ACT>(p.b, gidx);
    U.A_log = p.A_log[U.hv];
    U.dt_bias = p.dt_bias[U.hv];
    const float* S = static_cast<float*>(p.state) + ((int64_t)U.slot * p.HV + U.hv) * (int64_t)p.V * K;
    if constexpr (VF) {
#pragma unroll
      for (int i = 0; i < RG; ++i)
        U.vv[i] = ld_act<ACT>(p.qkv, vbase + min(U.r0 + (i * nwaves + wave) * RPI + rr, U.r1 - 1));
    }
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int row = min(U.r0 + (i * nwaves + wave) * RPI + rr, U.r1 - 1);
      if constexpr (!VF) U.vv[i] = ld_act<ACT>(p.qkv, vbase + row);
#pragma unroll
      for (int j = 0; j < NV; ++j) U.s[i][j] = ld4<true>(S + (int64_t)row * K + RL::col(c, j));
    }
  };
  auto compute = [&](Unit& U) {
    if (U.slot < 0 || U.slot >= p.num_slots) return;
    float qs = p.scale, ks = 1.f;
    if (p.use_l2) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < NV * 4; ++e) {
        sq += U.qf[e] * U.qf[e];
        sk += U.kf[e] * U.kf[e];
      }
      sq = group_sum<LPR>(sq);
      sk = group_sum<LPR>(sk);
      qs *= rsqrtf(sq + p.l2eps);
      ks = rsqrtf(sk + p.l2eps);
    }
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < NV * 4; ++e) {
      U.qf[e] *= qs;
      U.kf[e] *= ks;
      kq += U.kf[e] * U.qf[e];
    }
    kq = group_sum<LPR>(kq);
    const float g = -expf(U.A_log) * softplus_f(U.av + U.dt_bias);
    const float beta = sigmoid_f(U.bv);
    const float decay = expf(g);
    float* S = static_cast<float*>(p.state) + ((int64_t)U.slot * p.HV + U.hv) * (int64_t)p.V * K;
    const int64_t obase = ((int64_t)U.bi * p.HV + U.hv) * p.V;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float dk = 0.f, dq = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        dk += U.s[i][j].x * U.kf[4 * j] + U.s[i][j].y * U.kf[4 * j + 1] + U.s[i][j].z * U.kf[4 * j + 2] +
              U.s[i][j].w * U.kf[4 * j + 3];
        dq += U.s[i][j].x * U.qf[4 * j] + U.s[i][j].y * U.qf[4 * j + 1] + U.s[i][j].z * U.qf[4 * j + 2] +
              U.s[i][j].w * U.qf[4 * j + 3];
      }
      dk = group_sum<LPR>(dk);
      dq = group_sum<LPR>(dq);
      const float delta = beta * (U.vv[i] - decay * dk);
      const float o = decay * dq + delta * kq;
      const int row = U.r0 + (i * nwaves + wave) * RPI + rr;
      if (row < U.r1) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          f4 n;
          n.x = decay * U.s[i][j].x + delta * U.kf[4 * j];
          n.y = decay * U.s[i][j].y + delta * U.kf[4 * j + 1];
          n.z = decay * U.s[i][j].z + delta * U.kf[4 * j + 2];
          n.w = decay * U.s[i][j].w + delta * U.kf[4 * j + 3];
          st4<true>(S + (int64_t)row * K + RL::col(c, j), n);
        }
        if (c == 0) store_act1(p.out, obase + row, p.out_dt, o);
      }
    }
  };

  Unit A, B;
  int u = blockIdx.x;
  const int g = gridDim.x;
  if (u < n_units) fetch(u, A);
  while (u < n_units) {
    if (u + g < n_units) fetch(u + g, B);
    compute(A);
    if (u + g >= n_units) break;
    if (u + 2 * g < n_units) fetch(u + 2 * g, A);
    compute(B);
    u += 2 * g;
  }
}

namespace {

template <int K, int ACT, bool VEC, int RG, bool VF = false>
hipError_t launch_pf_rg(const GdnParams& p, int wpb, int64_t cap, hipStream_t st) {
  const int wave_rows = RG * RowLayout<K>::RPI;
  const int rows_per_tile = wpb * wave_rows;
  const int tiles = (p.V + rows_per_tile - 1) / rows_per_tile;
  // never launch more waves than a tile has rows for
  const int need = (min(p.V, rows_per_tile) + wave_rows - 1) / wave_rows;
  if (wpb > need) wpb = need;
  const int64_t units = (int64_t)p.B * p.HV * tiles;
  const int64_t blocks = units < cap ? units : cap;
  gdn_decode_pf_kernel<K, ACT, VEC, RG, VF><<<dim3((unsigned)blocks), dim3(64 * wpb), 0, st>>>(
      p, tiles, rows_per_tile, (int)units);
  return hipGetLastError();
}

template <int K, int ACT, bool VEC>
hipError_t launch_pf_k(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  constexpr int RG = pf_rg<K>();
  if (l.fixed) return launch_pf_rg<K, ACT, VEC, RG>(p, l.wpb, l.grid_cap > 0 ? l.grid_cap : n_cu, st);
  auto units_for = [&](int w, int rg) {
    const int rpt = w * rg * RowLayout<K>::RPI;
    return (int64_t)p.B * p.HV * ((p.V + rpt - 1) / rpt);
  };
  // Large batches (more than two full-height units per CU): one 1-wave block
  // per tile of one row group (8 rows of K = 64/128, 4 KB), no walk. Many
  // short read-then-write bursts in flight at once keep HBM busier than a few
  // long streams: at B = 256 (HV = 32, K = V = 128) 170.6 us, against 171.2
  // with 2-wave and 171.6 with 4-wave blocks over tiles of 2 and 4 row groups
  // (all three hold 64 KB of state loads per CU at this kernel's 4 waves per
  // SIMD; 8-wave blocks 180), 185.5 us for the persistent walk below (32 rows
  // per wave, one block per CU) and 190.6 us for 16-row waves; B = 64: 45.7 us
  // against 46.1 (4-wave) and 49.9 (walk). The persistent walk at one row
  // group per wave measured 197-272 us, so small tiles go with one block each.
  if constexpr (RG > 1) {
    if (units_for(4, RG) > 2LL * n_cu) return launch_pf_rg<K, ACT, VEC, 1>(p, 1, units_for(1, 1), st);
  }
  // Small batches (measured at HV = 32, K = V = 128, graph replay): up to
  // four 1-wave units of the full row-group depth per CU (B <= 8), 1-wave
  // blocks of half the rows per wave, one per unit, with v loaded ahead of the
  // state (B = 1 / 2 / 4 / 8: 3.6 / 4.3 / 5.1 / 7.2 us, against 3.6 / 5.2 /
  // 5.9 / 7.5 with 32-row 1- or 2-wave blocks; B = 1 with 8-row tiles 3.8,
  // with v loaded beside each row group 4.1, with 4-wave blocks 5.5; the
  // same shape at B = 16 15.2 against 12.6). Beyond that, narrower blocks
  // until every CU has a unit; one block per unit, all state loads in flight
  // at once, while that is at most two per CU (B = 16: 12.5 us against 13.9
  // persistent; 2-wave or 1-wave blocks, or v ahead of the state, 12.6-13.1);
  // beyond that one persistent block per CU (B = 64: 50.2 us against 52.1
  // with one block per unit).
  auto grid_for = [&](int64_t u) { return u <= 2LL * n_cu ? u : (int64_t)n_cu; };
  if constexpr (RG >= 2) {
    if (units_for(1, RG) <= 4LL * n_cu)
      return launch_pf_rg<K, ACT, VEC, RG / 2, true>(p, 1, units_for(1, RG / 2), st);
  }
  int wpb = 4;
  while (wpb > 1 && units_for(wpb, RG) < n_cu) wpb /= 2;
  return launch_pf_rg<K, ACT, VEC, RG>(p, wpb, grid_for(units_for(wpb, RG)), st);
}

template <int K>
hipError_t launch_pf_act(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  const bool vec = p.qkv_vec;
  switch (p.act_dt) {
    case SSMD_F32: return vec ? launch_pf_k<K, SSMD_F32, true>(p, l, n_cu, st) : launch_pf_k<K, SSMD_F32, false>(p, l, n_cu, st);
    case SSMD_BF16: return vec ? launch_pf_k<K, SSMD_BF16, true>(p, l, n_cu, st) : launch_pf_k<K, SSMD_BF16, false>(p, l, n_cu, st);
    default: return vec ? launch_pf_k<K, SSMD_F16, true>(p, l, n_cu, st) : launch_pf_k<K, SSMD_F16, false>(p, l, n_cu, st);
  }
}

}  // namespace

hipError_t launch_gdn_pf(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  if (p.norm_gate) return hipErrorInvalidValue;
  switch (p.K) {
    case 16: return launch_pf_act<16>(p, l, n_cu, st);
    case 32: return launch_pf_act<32>(p, l, n_cu, st);
    case 64: return launch_pf_act<64>(p, l, n_cu, st);
    case 128: return launch_pf_act<128>(p, l, n_cu, st);
    case 256: return launch_pf_act<256>(p, l, n_cu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
