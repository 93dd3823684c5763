// gdn_decode_s16.hip -- packed GDN decode step with the state pool stored in
// 16-bit floats (bf16 or f16) and every operation in fp32.
//
// "Optimization Log: Qwen3.5-27B Dense on B200" ("Kernel 4: Fused DeltaNet
// Recurrent") sizes the per-head state as a 16-bit [128, 128] tile; with the
// state the dominant traffic, 16-bit storage halves the bytes of a step. The
// arithmetic is that of gdn_decode.hip: per row, dk = S.k and dq = S.q in one
// pass, delta = beta (v - e^g dk), o = e^g dq + delta (k.q), and the new row
// e^g S + delta k is rounded (RNE) once, when it is stored. The step's own
// output comes from the unrounded row.
//
// Launch structure: at large batches one 1-wave block per row tile holding a
// single unit (WALK = false); otherwise persistent blocks, two per CU, each
// wave holding the next unit's state pass while it computes the current one.
// Units go in XCD-aware order (xcd_unit). A row of K 16-bit values is spread
// over LPR lanes with 128-bit accesses of 8 elements. With the gated-RMSNorm
// epilogue on, a unit is a whole head: the block walks all V rows (the first
// pass prefetched), keeps o in LDS and reduces across waves.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int K>
constexpr int s16_rg() {  // row groups per wave pass: 32 rows at K = 64/128
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 2 : 4));
}

template <int K, int ST, int ACT, bool VEC, bool NORM, int RG, bool WALK>
__global__ __launch_bounds__(512) void gdn_decode_s16_kernel(GdnParams p, int tiles_per_head,
                                                             int rows_per_tile, int n_units) {
  using RL = RowLayout16<K>;
  constexpr int EV = RL::EV, LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, ROWS = RG * RPI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  __shared__ float o_lds[NORM ? 1024 : 1];
  __shared__ float red_lds[1];
  uint16_t* const pool = static_cast<uint16_t*>(p.state);
  auto row_of = [&](int pass, int i) { return pass + (i * nwaves + wave) * RPI + rr; };

  struct Unit {
    int slot, bi, hv, h, r0, r1;
    float qf[NV * EV], kf[NV * EV], vv[RG], av, bv, A_log, dt_bias;
    u4 s[RG][NV];  // first pass of state rows, packed
  };
  auto fetch = [&](int unit, Unit& U) {
    int tile;
    xcd_unit(unit, p.B, p.H, p.HV, tiles_per_head, U.bi, U.hv, tile);
    U.slot = p.idx[U.bi];
    if (U.slot < 0 || U.slot >= p.num_slots) return;
    U.h = U.hv / (p.HV / p.H);
    U.r0 = tile * rows_per_tile;
    U.r1 = min(p.V, U.r0 + rows_per_tile);
    const int64_t qrow = (int64_t)U.bi * p.qkv_stride;
    const int64_t vbase = qrow + 2 * (int64_t)p.H * K + (int64_t)U.hv * p.V;
    const int64_t gidx = (int64_t)U.bi * p.HV + U.hv;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
      for (int half = 0; half < EV / 4; ++half) {
        ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)U.h * K + RL::col(c, j) + 4 * half, &U.qf[EV * j + 4 * half]);
        ld_act4<ACT, VEC>(p.qkv, qrow + (int64_t)(p.H + U.h) * K + RL::col(c, j) + 4 * half,
                          &U.kf[EV * j + 4 * half]);
      }
    }
    U.av = ld_act<ACT>(p.a, gidx);
    U.bv = ld_act<ACT>(p.b, gidx);
    U.A_log = p.A_log[U.hv];
    U.dt_bias = p.dt_bias[U.hv];
    const uint16_t* S = pool + ((int64_t)U.slot * p.HV + U.hv) * (int64_t)p.V * K;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int row = min(row_of(U.r0, i), U.r1 - 1);
      U.vv[i] = ld_act<ACT>(p.qkv, vbase + row);
#pragma unroll
      for (int j = 0; j < NV; ++j) U.s[i][j] = ld16x8<true>(S + (int64_t)row * K + RL::col(c, j));
    }
  };

  auto process = [&](Unit& U) {
    if (U.slot < 0 || U.slot >= p.num_slots) return;  // uniform over the block
    float qs = p.scale, ks = 1.f;
    if (p.use_l2) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < NV * EV; ++e) {
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
    for (int e = 0; e < NV * EV; ++e) {
      U.qf[e] *= qs;
      U.kf[e] *= ks;
      kq += U.kf[e] * U.qf[e];
    }
    kq = group_sum<LPR>(kq);
    const float g = -expf(U.A_log) * softplus_f(U.av + U.dt_bias);
    const float beta = sigmoid_f(U.bv);
    const float decay = expf(g);
    uint16_t* S = pool + ((int64_t)U.slot * p.HV + U.hv) * (int64_t)p.V * K;
    const int64_t obase = ((int64_t)U.bi * p.HV + U.hv) * p.V;
    const int64_t vbase = (int64_t)U.bi * p.qkv_stride + 2 * (int64_t)p.H * K + (int64_t)U.hv * p.V;

    int pass = U.r0;
    while (true) {
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        float sv[NV][EV];
        float dk = 0.f, dq = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          unpack8<ST>(U.s[i][j], sv[j]);
#pragma unroll
          for (int e = 0; e < EV; ++e) {
            dk += sv[j][e] * U.kf[EV * j + e];
            dq += sv[j][e] * U.qf[EV * j + e];
          }
        }
        dk = group_sum<LPR>(dk);
        dq = group_sum<LPR>(dq);
        const float delta = beta * (U.vv[i] - decay * dk);
        const float o = decay * dq + delta * kq;
        const int row = row_of(pass, i);
        if (row < U.r1) {
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            float n[EV];
#pragma unroll
            for (int e = 0; e < EV; ++e) n[e] = decay * sv[j][e] + delta * U.kf[EV * j + e];
            st16x8<true>(S + (int64_t)row * K + RL::col(c, j), pack8<ST>(n));
          }
          if (c == 0) {
            if constexpr (NORM) o_lds[row] = o;
            else store_act1(p.out, obase + row, p.out_dt, o);
          }
        }
      }
      pass += nwaves * ROWS;
      if (pass >= U.r1) break;
#pragma unroll
      for (int i = 0; i < RG; ++i) {  // later passes of a long head load here
        const int row = min(row_of(pass, i), U.r1 - 1);
        U.vv[i] = ld_act<ACT>(p.qkv, vbase + row);
#pragma unroll
        for (int j = 0; j < NV; ++j) U.s[i][j] = ld16x8<true>(S + (int64_t)row * K + RL::col(c, j));
      }
    }

    if constexpr (NORM) {
      __syncthreads();
      if (wave == 0) {
        float ss = 0.f;
        for (int r = lane; r < p.V; r += 64) ss += o_lds[r] * o_lds[r];
        ss = wave_sum(ss);
        if (lane == 0) red_lds[0] = ss;
      }
      __syncthreads();
      const float inv = rsqrtf(red_lds[0] / (float)p.V + p.norm_eps);
      for (int r = threadIdx.x; r < p.V; r += blockDim.x) {
        const float z = ld_act<ACT>(p.norm_gate, obase + r);
        const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
        const float w = p.norm_w ? p.norm_w[r] : 1.f;
        store_act1(p.out, obase + r, p.out_dt, o_lds[r] * inv * w * gz);
      }
      __syncthreads();  // o_lds / red_lds are reused by the next unit
    }
  };

  if constexpr (!WALK) {
    Unit A;
    for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
      fetch(u, A);
      process(A);
    }
  } else {
    Unit A, B;
    int u = blockIdx.x;
    const int gs = gridDim.x;
    if (u < n_units) fetch(u, A);
    while (u < n_units) {
      if (u + gs < n_units) fetch(u + gs, B);
      process(A);
      if (u + gs >= n_units) break;
      if (u + 2 * gs < n_units) fetch(u + 2 * gs, A);
      process(B);
      u += 2 * gs;
    }
  }
}

namespace {

template <int K, int ST, int ACT, bool VEC, bool NORM, int RG>
hipError_t launch_s16_rg(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  const int wave_rows = RG * RowLayout16<K>::RPI;
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
  const int64_t units = (int64_t)p.B * p.HV * tiles;
  // two blocks per CU: 16-bit rows halve the bytes per unit but not the ALU
  // work, so a second wave per SIMD is needed to hide the arithmetic latency
  // (measured at B = 256: 111 us with 2 blocks per CU, 139 us with 1)
  const int64_t cap = l.grid_cap > 0 ? l.grid_cap : 2 * (int64_t)n_cu;
  const int64_t blocks = units < cap ? units : cap;
  gdn_decode_s16_kernel<K, ST, ACT, VEC, NORM, RG, true><<<dim3((unsigned)blocks), dim3(64 * wpb), 0, st>>>(
      p, tiles, rows_per_tile, (int)units);
  return hipGetLastError();
}

// One block per tile (as many waves as the tile has row groups of RG x RPI
// rows, at most 4), no walk: the kernel holds a single unit, so its registers
// admit five waves per SIMD, and the hardware dispatcher refills each CU as
// its blocks finish.
template <int K, int ST, int ACT, bool VEC, int RG>
hipError_t launch_s16_tiles(const GdnParams& p, int64_t units, int rows_per_tile, int tiles, hipStream_t st) {
  const int wave_rows = RG * RowLayout16<K>::RPI;
  const int wpb = (min(p.V, rows_per_tile) + wave_rows - 1) / wave_rows;
  gdn_decode_s16_kernel<K, ST, ACT, VEC, false, RG, false><<<dim3((unsigned)units), dim3(64 * wpb), 0, st>>>(
      p, tiles, rows_per_tile, (int)units);
  return hipGetLastError();
}

// Large batches (more than four 4-wave tiles of half the walk's rows per wave
// per CU): one 1-wave block per tile of one wave's rows (16 at K = 128).
// Measured on MI355X at HV = 32, K = V = 128, bf16 state, same session: B =
// 256 94.2 us with 4-wave blocks against 103.9 us for the walk (5.77 TB/s),
// B = 64 27.3 against 28.8; then 1-wave blocks 93.7 / 27.0 against 94.7 /
// 27.6 for 4-wave and 95.0 / 27.2 for 2-wave blocks. With no compute at all
// the walk's loads and stores take 100 us at B = 256: its limit is how its
// two units per wave issue, not the arithmetic. A third block per CU for the
// walk, or a capped grid-stride loop over single units (102 us), measured
// slower. Small batches keep the walk (B = 16: 8.3 against 9.2 us for 4-wave
// tiles, 9.7 for 1-wave ones): with few tiles, its register use, two blocks
// per CU, spreads them evenly over the CUs. Below one whole-head tile per CU
// the walk leaves CUs idle, and the 1-wave tiles spread the few heads over all
// of them (B = 1 / 2 / 4: 3.9 / 4.3 / 4.7 against 5.0 / 5.3 / 5.6 us).
template <int K, int ST, int ACT, bool VEC, bool NORM>
hipError_t launch_s16_k(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  constexpr int RG = s16_rg<K>();
  if constexpr (!NORM) {
    constexpr int RG1 = RG / 2 > 1 ? RG / 2 : 1;
    const int rows4 = 4 * RG1 * RowLayout16<K>::RPI;
    const int64_t units4 = (int64_t)p.B * p.HV * ((p.V + rows4 - 1) / rows4);
    // the walk's whole-head tiles (4 waves of RG row groups) per CU
    const int rows_w = 4 * RG * RowLayout16<K>::RPI;
    const int64_t units_w = (int64_t)p.B * p.HV * ((p.V + rows_w - 1) / rows_w);
    if (!l.fixed && (units4 > 4LL * n_cu || units_w < n_cu)) {
      const int rows_per_tile = RG1 * RowLayout16<K>::RPI;
      const int tiles = (p.V + rows_per_tile - 1) / rows_per_tile;
      return launch_s16_tiles<K, ST, ACT, VEC, RG1>(p, (int64_t)p.B * p.HV * tiles, rows_per_tile, tiles, st);
    }
  }
  return launch_s16_rg<K, ST, ACT, VEC, NORM, RG>(p, l, n_cu, st);
}

template <int K, int ST, bool NORM>
hipError_t launch_s16_act(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  const bool vec = p.qkv_vec;
  switch (p.act_dt) {
    case SSMD_F32: return vec ? launch_s16_k<K, ST, SSMD_F32, true, NORM>(p, l, n_cu, st) : launch_s16_k<K, ST, SSMD_F32, false, NORM>(p, l, n_cu, st);
    case SSMD_BF16: return vec ? launch_s16_k<K, ST, SSMD_BF16, true, NORM>(p, l, n_cu, st) : launch_s16_k<K, ST, SSMD_BF16, false, NORM>(p, l, n_cu, st);
    default: return vec ? launch_s16_k<K, ST, SSMD_F16, true, NORM>(p, l, n_cu, st) : launch_s16_k<K, ST, SSMD_F16, false, NORM>(p, l, n_cu, st);
  }
}

template <int K>
hipError_t launch_s16_st(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  const bool norm = p.norm_gate != nullptr;
  if (p.state_dt == SSMD_BF16)
    return norm ? launch_s16_act<K, SSMD_BF16, true>(p, l, n_cu, st) : launch_s16_act<K, SSMD_BF16, false>(p, l, n_cu, st);
  return norm ? launch_s16_act<K, SSMD_F16, true>(p, l, n_cu, st) : launch_s16_act<K, SSMD_F16, false>(p, l, n_cu, st);
}

}  // namespace

hipError_t launch_gdn_s16(const GdnParams& p, const Launch& l, int n_cu, hipStream_t st) {
  switch (p.K) {
    case 16: return launch_s16_st<16>(p, l, n_cu, st);
    case 32: return launch_s16_st<32>(p, l, n_cu, st);
    case 64: return launch_s16_st<64>(p, l, n_cu, st);
    case 128: return launch_s16_st<128>(p, l, n_cu, st);
    case 256: return launch_s16_st<256>(p, l, n_cu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
