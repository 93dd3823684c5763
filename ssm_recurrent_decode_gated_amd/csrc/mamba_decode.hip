// mamba_decode.hip -- Mamba-1 selective-scan decode step on gfx950.
//
// "Triton decode kernel + MBU analysis" ("Kernel design"): per batch row b
// and channel d, with the N-wide state row h = state[slot, d, :],
//   dA = exp(dt * A[d, :]),  dB = dt * B[b, :]
//   h <- dA * h + dB * x
//   y = sum_n C[b, n] h[n]  (+ D[d] x)  (* silu(z))
// The state row is the only per-(b, d) stream (8N bytes read + written); A is
// shared by every row b and B, C by every channel d, so they come from cache.
// Layout as in the GDN kernels: a row of N fp32 is spread over LPR lanes with
// 128-bit accesses (N = 16: 4 lanes, 16 rows per wave-wide access, 1 KB
// contiguous), the y dot product reduces over those lanes with DPP, and the
// per-row scalars (x, dt, z) are loaded by every lane of the row.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

template <int N>
constexpr int mamba_rg() {
  return N <= 32 ? 4 : 2;
}

template <int N, int ACT, int RG>
__global__ __launch_bounds__(256) void mamba_decode_kernel(MambaParams p, int blocks_per_row) {
  using RL = RowLayout<N>;
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  const int bi = blockIdx.x / blocks_per_row;
  const int chunk = blockIdx.x - bi * blocks_per_row;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;  // padded row: touch nothing
  const int Dm = p.Dm;
  const int d0 = chunk * nwaves * RG * RPI;
  float* Hs = p.state + (int64_t)slot * Dm * N;

  // B and C of this row at the lane's columns (shared by every channel)
  float bf[NV * 4], cf[NV * 4];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf[4 * j + e] = ld_act<ACT>(p.Bm, (int64_t)bi * N + RL::col(c, j) + e);
      cf[4 * j + e] = ld_act<ACT>(p.Cm, (int64_t)bi * N + RL::col(c, j) + e);
    }
  }
  float xv[RG], dtv[RG], zv[RG], dv[RG];
  f4 h[RG][NV], a[RG][NV];
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int d = min(d0 + (i * nwaves + wave) * RPI + rr, Dm - 1);  // past-the-end rows re-read the last
    const int64_t bd = (int64_t)bi * Dm + d;
    xv[i] = ld_act<ACT>(p.x, bd);
    dtv[i] = ld_act<ACT>(p.dt, bd);
    zv[i] = p.z ? ld_act<ACT>(p.z, bd) : 0.f;
    dv[i] = p.Dvec ? p.Dvec[d] : 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      a[i][j] = *reinterpret_cast<const f4*>(p.A + (int64_t)d * N + RL::col(c, j));
      h[i][j] = ld4<true>(Hs + (int64_t)d * N + RL::col(c, j));
    }
  }
  // exp(dt A) = exp2(dt log2(e) A): one v_exp_f32 (about 1 ulp) per element
  // instead of expf's longer sequence (B=256, D=4096, N=16: 28.4 -> 27.3 us;
  // B=8, D=1536: 3.76 -> 3.45 us)
  constexpr float LOG2E = 1.44269504088896341f;
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    const int d = d0 + (i * nwaves + wave) * RPI + rr;
    const float dl = dtv[i] * LOG2E;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      f4 n;
      n.x = __builtin_amdgcn_exp2f(dl * a[i][j].x) * h[i][j].x + dtv[i] * bf[4 * j] * xv[i];
      n.y = __builtin_amdgcn_exp2f(dl * a[i][j].y) * h[i][j].y + dtv[i] * bf[4 * j + 1] * xv[i];
      n.z = __builtin_amdgcn_exp2f(dl * a[i][j].z) * h[i][j].z + dtv[i] * bf[4 * j + 2] * xv[i];
      n.w = __builtin_amdgcn_exp2f(dl * a[i][j].w) * h[i][j].w + dtv[i] * bf[4 * j + 3] * xv[i];
      acc += cf[4 * j] * n.x + cf[4 * j + 1] * n.y + cf[4 * j + 2] * n.z + cf[4 * j + 3] * n.w;
      if (d < Dm) st4<true>(Hs + (int64_t)d * N + RL::col(c, j), n);
    }
    acc = group_sum<LPR>(acc);
    float y = acc + dv[i] * xv[i];
    if (p.z) y *= silu_f(zv[i]);
    if (d < Dm && c == 0) store_act1(p.out, (int64_t)bi * Dm + d, p.out_dt, y);
  }
}

namespace {

template <int N, int ACT, int RG>
hipError_t launch_m_rg(const MambaParams& p, int wpb, hipStream_t st) {
  const int rows_per_block = wpb * RG * RowLayout<N>::RPI;
  const int blocks_per_row = (p.Dm + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)((int64_t)p.B * blocks_per_row));
  mamba_decode_kernel<N, ACT, RG><<<grid, dim3(64 * wpb), 0, st>>>(p, blocks_per_row);
  return hipGetLastError();
}

// 2-wave blocks of mamba_rg row groups per wave where that gives every CU a
// block (measured at N = 16: B = 256, D = 4096 25.9 us against 26.6 with
// 1-wave blocks, 26.7 with half the rows per wave and 27.4 with 4 waves);
// below that, 1-wave blocks and then half and a quarter of the rows per wave
// until every CU has one (the finest otherwise): B = 1 / 8, D = 1536, N = 16
// 2.93 / 3.41 us with 2-wave blocks against 2.29 / 2.98 with 1-wave blocks of
// half the rows.
template <int N, int ACT>
hipError_t launch_m(const MambaParams& p, const Launch& l, int n_cu, hipStream_t st) {
  constexpr int RG = mamba_rg<N>();
  if (l.fixed) return launch_m_rg<N, ACT, RG>(p, min(l.wpb, 4), st);
  auto blocks = [&](int wpb, int rg) {
    const int rows = wpb * rg * RowLayout<N>::RPI;
    return (int64_t)p.B * ((p.Dm + rows - 1) / rows);
  };
  if (blocks(2, RG) >= n_cu) return launch_m_rg<N, ACT, RG>(p, 2, st);
  if (blocks(1, RG) >= n_cu) return launch_m_rg<N, ACT, RG>(p, 1, st);
  constexpr int RG2 = RG / 2 > 1 ? RG / 2 : 1;
  if constexpr (RG2 < RG) {
    if (blocks(1, RG2) >= n_cu) return launch_m_rg<N, ACT, RG2>(p, 1, st);
  }
  constexpr int RG4 = RG2 / 2 > 1 ? RG2 / 2 : 1;
  return launch_m_rg<N, ACT, RG4>(p, 1, st);
}

template <int N>
hipError_t launch_mact(const MambaParams& p, const Launch& l, int n_cu, hipStream_t st) {
  switch (p.act_dt) {
    case SSMD_F32: return launch_m<N, SSMD_F32>(p, l, n_cu, st);
    case SSMD_BF16: return launch_m<N, SSMD_BF16>(p, l, n_cu, st);
    default: return launch_m<N, SSMD_F16>(p, l, n_cu, st);
  }
}

}  // namespace

hipError_t launch_mamba(const MambaParams& p, const Launch& l, int n_cu, hipStream_t st) {
  switch (p.N) {
    case 16: return launch_mact<16>(p, l, n_cu, st);
    case 32: return launch_mact<32>(p, l, n_cu, st);
    case 64: return launch_mact<64>(p, l, n_cu, st);
    case 128: return launch_mact<128>(p, l, n_cu, st);
    case 256: return launch_mact<256>(p, l, n_cu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
