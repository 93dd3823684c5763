// gdn_conv_decode.hip -- GDN decode step with the causal conv1d update + SiLU
// fused in front, on gfx950.
//
// The fused KDA op of "Microbenchmark for the fused Kimi-K3 KDA decode kernel
// on ROCm" (conv update then recurrent step in one launch, the conv output
// kept on chip) applied to the packed GDN step of "Microbenchmark: buffered
// output-only GDN decode (ReplaySSM Part A) vs. the existing packed GDN decode
// kernel"; "Optimization Log: Qwen3.5-27B Dense on B200" ("Kernel 5: Fused
// Causal Conv1d Update", "Integration") puts the conv between the input
// projection and the recurrence.
//
// The conv state is rolled in place, so each channel must be updated by
// exactly one block. The G = HV/H value heads of a q/k head share its q and k
// channels, so a block owns one (batch row, q/k head) group: it runs the conv
// over the group's 2K + G V channels once (SiLU outputs kept in LDS at fp32),
// then streams the G value heads' states as G V rows, each row taking its own
// head's gates. Every small load (conv windows, conv weights, gates) is
// issued before the first pass of state rows, so the conv and the gates are
// computed while that pass is in flight.
#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

// Row groups per wave pass. K = 128: 8 (64 rows per wave, 256 per block), so
// the G = 2 value heads of a group are one pass with every state load issued
// up front (measured at B = 256, HV = 32: 207.5 us against 210.5 with two
// passes, the second issued only after the first was computed).
template <int K>
constexpr int gconv_rg() {
  return K == 16 ? 1 : (K == 32 ? 2 : (K == 256 ? 2 : (K == 128 ? 8 : 4)));
}

constexpr int GCONV_THREADS = 256;
constexpr int GCONV_GMAX = 16;                  // largest GQA group G = HV / H
constexpr int GCONV_YMAX = 2 * 256 + 16 * 256;  // conv outputs of one group, 2K + G V
constexpr int GCONV_OMAX = 16 * 256;            // outputs of one group, G V

// WT: the conv width when it is 4 (compile time), 0 for any width in [2, 8].
template <int K, bool NORM, int ACT, int WT>
__global__ __launch_bounds__(GCONV_THREADS) void gdn_conv_decode_kernel(GdnConvParams cp) {
  const GdnParams& p = cp.g;
  using RL = RowLayout<K>;
  using T = typename std::conditional<ACT == SSMD_F32, float, uint16_t>::type;
  constexpr int RG = gconv_rg<K>();
  constexpr int LPR = RL::LPR, NV = RL::NV, RPI = RL::RPI, ROWS = RG * RPI;
  constexpr int CPT = 2;              // conv channels per thread per chunk
  constexpr int WM = WT ? WT : 8;     // register window
  const int W = WT ? WT : cp.W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int nwaves = GCONV_THREADS / 64;
  const int c = lane % LPR;
  const int rr = lane / LPR;
  __shared__ float y[GCONV_YMAX];
  __shared__ float gdecay[GCONV_GMAX], gbeta[GCONV_GMAX];
  __shared__ float o_lds[NORM ? GCONV_OMAX : 1];
  __shared__ float red_lds[NORM ? GCONV_GMAX : 1];

  const int h = blockIdx.x % p.H;
  const int bi = blockIdx.x / p.H;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;  // padded row: touch nothing
  const int G = p.HV / p.H;
  const int V = p.V;
  const int rows = G * V;  // row R of the group: value head h G + R / V, state row R % V
  const int nch = 2 * K + rows;
  // group-local channel ci -> channel of x: q of head h | k of head h | v of heads h G .. h G + G - 1
  auto chan = [&](int ci) {
    return ci < K ? h * K + ci
                  : (ci < 2 * K ? (p.H + h) * K + (ci - K) : 2 * p.H * K + h * rows + (ci - 2 * K));
  };
  float* const pool = static_cast<float*>(p.state);
  auto row_ptr = [&](int R) {
    const int g = R / V;
    return pool + (((int64_t)slot * p.HV + h * G + g) * V + (R - g * V)) * (int64_t)K;
  };
  auto row_of = [&](int pass, int i) { return pass + (i * nwaves + wave) * RPI + rr; };

  // ---- small loads: conv windows and weights of this thread's first channels, gates
  T* const cs = static_cast<T*>(cp.conv_state);
  const T* const xr = static_cast<const T*>(p.qkv) + (int64_t)bi * p.qkv_stride;
  const int64_t cs_base = (int64_t)slot * cp.cs_slot;
  T raw[CPT][WM];
  float wf[CPT][WM], cb[CPT];
  auto conv_load = [&](int base) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int gc = chan(min(base + tid + m * GCONV_THREADS, nch - 1));
      const int64_t cso = cs_base + (int64_t)gc * cp.cs_chan;
#pragma unroll
      for (int j = 0; j < WM - 1; ++j)
        if (j < W - 1) raw[m][j] = cs[cso + (int64_t)j * cp.cs_tap];
      raw[m][WM - 1] = xr[gc];
#pragma unroll
      for (int j = 0; j < WM; ++j)
        if (j < W) wf[m][j] = cp.conv_w[(int64_t)gc * W + j];
      cb[m] = cp.conv_b ? cp.conv_b[gc] : 0.f;
    }
  };
  auto to_f = [](T v) -> float {
    if constexpr (ACT == SSMD_F32) return v;
    else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(v);
    else return f16_bits_to_f32(v);
  };
  // conv output -> y, and roll the window: tap j <- window[j + 1], the newest tap <- x
  auto conv_do = [&](int base) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int ci = base + tid + m * GCONV_THREADS;
      if (ci < nch) {
        const int64_t cso = cs_base + (int64_t)chan(ci) * cp.cs_chan;
        float acc = cb[m];
#pragma unroll
        for (int j = 0; j < WM - 1; ++j)
          if (j < W - 1) acc += wf[m][j] * to_f(raw[m][j]);
#pragma unroll
        for (int j = 0; j < WM; ++j)  // the current input sits at tap W - 1
          if (j == W - 1) acc += wf[m][j] * to_f(raw[m][WM - 1]);
#pragma unroll
        for (int j = 0; j < WM - 1; ++j)
          if (j < W - 1) cs[cso + (int64_t)j * cp.cs_tap] = j + 1 < W - 1 ? raw[m][j + 1] : raw[m][WM - 1];
        y[ci] = silu_f(acc);
      }
    }
  };
  conv_load(0);
  const int gh = h * G + min(tid, G - 1);  // value head whose gates this thread computes
  const int64_t gidx = (int64_t)bi * p.HV + gh;
  const float av = ld_act<ACT>(p.a, gidx);
  const float bv = ld_act<ACT>(p.b, gidx);
  const float A_log = p.A_log[gh];
  const float dt_bias = p.dt_bias[gh];

  // ---- first pass of state rows (rows past the end re-read the last row, never stored)
  f4 s[RG][NV];
  auto load_group = [&](int pass, int i) {
    const float* S = row_ptr(min(row_of(pass, i), rows - 1));
#pragma unroll
    for (int j = 0; j < NV; ++j) s[i][j] = ld4<true>(S + RL::col(c, j));
  };
  int pass = 0;
#pragma unroll
  for (int i = 0; i < RG; ++i) load_group(pass, i);

  // ---- conv (remaining chunks load after the state pass was issued), gates
  conv_do(0);
  for (int base = CPT * GCONV_THREADS; base < nch; base += CPT * GCONV_THREADS) {
    conv_load(base);
    conv_do(base);
  }
  if (tid < G) {
    const float g = -expf(A_log) * softplus_f(av + dt_bias);
    gdecay[tid] = expf(g);
    gbeta[tid] = sigmoid_f(bv);
  }
  __syncthreads();

  // ---- q, k of the group from LDS; L2 norms and scale
  float qf[NV * 4], kf[NV * 4];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[4 * j + e] = y[RL::col(c, j) + e];
      kf[4 * j + e] = y[K + RL::col(c, j) + e];
    }
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
  const int64_t obase = ((int64_t)bi * p.HV + h * G) * V;  // output row R of the group is obase + R

  // ---- stream the group's rows; each row takes its own head's decay and beta
  while (true) {
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int R = row_of(pass, i);
      const int Rc = min(R, rows - 1);
      const int g = Rc / V;
      const float decay = gdecay[g], beta = gbeta[g];
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
      const float delta = beta * (y[2 * K + Rc] - decay * dk);
      const float o = decay * dq + delta * kq;
      if (R < rows) {
        float* S = row_ptr(R);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          f4 n;
          n.x = decay * s[i][j].x + delta * kf[4 * j];
          n.y = decay * s[i][j].y + delta * kf[4 * j + 1];
          n.z = decay * s[i][j].z + delta * kf[4 * j + 2];
          n.w = decay * s[i][j].w + delta * kf[4 * j + 3];
          st4<true>(S + RL::col(c, j), n);
        }
        if (c == 0) {
          if constexpr (NORM) o_lds[R] = o;
          else store_act1(p.out, obase + R, p.out_dt, o);
        }
      }
    }
    pass += nwaves * ROWS;
    if (pass >= rows) break;
#pragma unroll
    for (int i = 0; i < RG; ++i) load_group(pass, i);
  }

  if constexpr (NORM) {
    // gated RMSNorm of each value head over its V outputs
    __syncthreads();
    for (int g = wave; g < G; g += nwaves) {
      float ss = 0.f;
      for (int r = lane; r < V; r += 64) ss += o_lds[g * V + r] * o_lds[g * V + r];
      ss = wave_sum(ss);
      if (lane == 0) red_lds[g] = ss;
    }
    __syncthreads();
    for (int R = tid; R < rows; R += GCONV_THREADS) {
      const int g = R / V;
      const float inv = rsqrtf(red_lds[g] / (float)V + p.norm_eps);
      const float z = ld_act<ACT>(p.norm_gate, obase + R);
      const float gz = p.norm_act == SSMD_ACT_SIGMOID ? sigmoid_f(z) : silu_f(z);
      const float w = p.norm_w ? p.norm_w[R - g * V] : 1.f;
      store_act1(p.out, obase + R, p.out_dt, o_lds[R] * inv * w * gz);
    }
  }
}

namespace {

template <int K, bool NORM, int ACT>
hipError_t launch_gc(const GdnConvParams& cp, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)cp.g.B * cp.g.H));
  if (cp.W == 4)
    gdn_conv_decode_kernel<K, NORM, ACT, 4><<<grid, dim3(GCONV_THREADS), 0, st>>>(cp);
  else
    gdn_conv_decode_kernel<K, NORM, ACT, 0><<<grid, dim3(GCONV_THREADS), 0, st>>>(cp);
  return hipGetLastError();
}

template <int K, bool NORM>
hipError_t launch_gc_act(const GdnConvParams& cp, hipStream_t st) {
  switch (cp.g.act_dt) {
    case SSMD_F32: return launch_gc<K, NORM, SSMD_F32>(cp, st);
    case SSMD_BF16: return launch_gc<K, NORM, SSMD_BF16>(cp, st);
    default: return launch_gc<K, NORM, SSMD_F16>(cp, st);
  }
}

template <int K>
hipError_t launch_gc_norm(const GdnConvParams& cp, hipStream_t st) {
  return cp.g.norm_gate ? launch_gc_act<K, true>(cp, st) : launch_gc_act<K, false>(cp, st);
}

}  // namespace

// One block of GCONV_THREADS threads per (batch row, q/k head). The host has
// checked G <= GCONV_GMAX and G V <= GCONV_OMAX (so 2K + G V <= GCONV_YMAX).
// Shapes the 8-wave kernel of gdn_conv_decode_pf.hip covers (width 4, no
// output norm, G V = 256 at K = 64 or 128) take it: with fewer than four
// groups per CU one block per CU walks them (or one per group if there are
// fewer groups than CUs), from four up one block per group. Measured at
// H = 16, HV = 32, K = V = 128: B = 8 / 16 / 32 / 64 / 256 in 9.0 / 13.2 /
// 25.6 / 52.3 / 200.1 us, against 10.7 / 14.1 / 27.1 / 56.3 / 207.1 with this
// kernel; walking at B = 64 / 256 took 53.3 / 202.7 us, one block per group
// at B = 32 (two per CU) 27.4. A fixed launch shape with a grid cap forces
// the 8-wave kernel with that many blocks, one without forces this kernel.
hipError_t launch_gdn_conv(const GdnConvParams& cp, const Launch& l, int n_cu, hipStream_t st) {
  if (gdn_conv_pf_fits(cp)) {
    if (l.fixed && l.grid_cap > 0) return launch_gdn_conv_pf(cp, l.grid_cap, st);
    if (!l.fixed) {
      const int64_t groups = (int64_t)cp.g.B * cp.g.H;
      return launch_gdn_conv_pf(cp, groups >= 4LL * n_cu ? groups : (int64_t)n_cu, st);
    }
  }
  switch (cp.g.K) {
    case 16: return launch_gc_norm<16>(cp, st);
    case 32: return launch_gc_norm<32>(cp, st);
    case 64: return launch_gc_norm<64>(cp, st);
    case 128: return launch_gc_norm<128>(cp, st);
    case 256: return launch_gc_norm<256>(cp, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
