// mamba_scan.hip -- Mamba-1 selective scan over T tokens (prefill) on gfx950.
//
// "Triton decode kernel + MBU analysis" ("Prefill path") leaves prefill to a
// fused chunked scan over the recurrence of "Kernel design":
//   h_t = exp(dt_t A) h_{t-1} + dt_t B_t x_t,   y_t = C_t . h_t (+ D x_t) (* silu(z_t))
// per (row b, channel d) with an N-wide diagonal state. The recurrence is
// diagonal, so a chunk of tokens acts on its starting state as
//   h_end = P h_start + h_loc,   P = prod_t exp(dt_t A) = exp(A sum_t dt_t),
// with h_loc the chunk's scan from zero. That gives the chunked form:
//   1. summary: every (row, chunk, channel) scans its chunk from zero,
//      storing P and h_loc (workspace);
//   2. carry: per (row, channel, n), walk the chunks in order, replacing
//      each h_loc by the chunk's true starting state and writing the final
//      state to the pool;
//   3. output: every (row, chunk, channel) rescans its chunk from its
//      starting state and writes y.
// With one chunk (no workspace, or enough rows and channels to fill the
// GPU) a single pass does 3 alone from the pool state.
//
// Layout: a channel's N-wide state is split over LPN = N/16 lanes of 16
// consecutive elements each (registers for the whole chunk); y reduces over
// those lanes with DPP. A block of 256 threads holds 256/LPN consecutive
// channels of one row and one chunk: x, dt, z are per-lane loads coalesced
// over channels, prefetched one group of 8 tokens ahead; B and C of a token
// group are shared by the block's channels and staged through LDS (double
// buffered, one barrier per group). A rows stay in registers.
#include <type_traits>

#include "ssmd_device.h"
#include "ssmd_internal.h"

namespace ssmd {

constexpr int MSCAN_THREADS = 256;
constexpr int MSCAN_SUB = 8;   // tokens per prefetch group
constexpr int MSCAN_NPL = 16;  // state elements per lane (chunked passes)

enum MScanMode { MSCAN_SUMMARY = 0, MSCAN_OUTPUT = 1, MSCAN_SINGLE = 2 };

// One activation value as loaded, converted when staged: a conversion (or a
// load under a branch) right at the load makes the wave wait for it there,
// which turns the one-group-ahead prefetch into a wait per token.
template <int ACT>
struct ScanRaw {
  typename std::conditional<ACT == SSMD_F32, float, uint32_t>::type v;
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    if constexpr (ACT == SSMD_F32) v = static_cast<const float*>(base)[off];
    else v = static_cast<const uint16_t*>(base)[off];
  }
  __device__ __forceinline__ float get() const {
    if constexpr (ACT == SSMD_F32) return v;
    else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(v);
    else return f16_bits_to_f32(v);
  }
};

// NPL: state elements per lane (16; 4 for a single pass that would leave
// SIMDs idle).
template <int N, int ACT, int MODE, int NPL = MSCAN_NPL>
__global__ __launch_bounds__(MSCAN_THREADS) void mamba_scan_kernel(MambaScanParams p) {
  constexpr int LPN = N / NPL;
  constexpr int CPB = MSCAN_THREADS / LPN;            // channels per block
  constexpr int BCV = MSCAN_SUB * N * 2;              // B and C values of a token group
  constexpr int BCT = (BCV + MSCAN_THREADS - 1) / MSCAN_THREADS;  // per thread
  __shared__ float bc_lds[2][BCV];  // [group token][B | C][N]
  const int tid = threadIdx.x;
  const int j = tid % LPN;   // which 16 state elements
  const int bi = blockIdx.z;
  const int chunk = blockIdx.y;
  const int d_raw = blockIdx.x * CPB + tid / LPN;
  const int d = min(d_raw, p.Dm - 1);  // lanes past the end compute a copy of the last channel, store nothing
  const bool live = d_raw < p.Dm;
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;  // padded row: touch nothing
  const int len = p.lengths ? min(max(p.lengths[bi], 0), p.T) : p.T;
  const int t0 = chunk * p.Lc;
  const int t1 = min(t0 + p.Lc, len);
  const int64_t ws_off = (((int64_t)bi * p.nck + chunk) * p.Dm + d) * N + NPL * j;

  // a2 = A log2(e): exp(dt A) = exp2(dt a2), one multiply and one v_exp_f32
  // (about 1 ulp) per element and token instead of the ~14 instructions of
  // expf; the scan is bound by this arithmetic, not by memory.
  constexpr float LOG2E = 1.44269504088896341f;
  float h[NPL], a2[NPL];
#pragma unroll
  for (int q = 0; q < NPL / 4; ++q) {
    const f4 av = *reinterpret_cast<const f4*>(p.A + (int64_t)d * N + NPL * j + 4 * q);
    a2[4 * q] = av.x * LOG2E; a2[4 * q + 1] = av.y * LOG2E; a2[4 * q + 2] = av.z * LOG2E; a2[4 * q + 3] = av.w * LOG2E;
  }
  float dt_sum = 0.f;  // chunk decay: prod_t exp(dt_t A) = exp2(a2 sum_t dt_t)
  float* const hs = p.state + ((int64_t)slot * p.Dm + d) * N + NPL * j;

  // ---- token groups: x, dt, z in registers and B, C in LDS, one group ahead
  const float Dd = (MODE != MSCAN_SUMMARY && p.Dvec) ? p.Dvec[d] : 0.f;
  const bool has_z = MODE != MSCAN_SUMMARY && p.z != nullptr;
  float xc[MSCAN_SUB], dc[MSCAN_SUB], zc[MSCAN_SUB];
  ScanRaw<ACT> xn[MSCAN_SUB], dn[MSCAN_SUB], zn[MSCAN_SUB], bcn[BCT];
  const void* const zsrc = has_z ? p.z : p.x;  // without a gate: a harmless in-bounds load, unused
  auto load_group = [&](int g0) {  // tokens g0 .. g0 + SUB - 1 (clamped into the row)
#pragma unroll
    for (int u = 0; u < MSCAN_SUB; ++u) {
      const int t = min(g0 + u, p.T - 1);
      const int64_t o = ((int64_t)bi * p.T + t) * p.Dm + d;
      xn[u].load(p.x, o);
      dn[u].load(p.dt, o);
      zn[u].load(zsrc, o);
    }
#pragma unroll
    for (int e = 0; e < BCT; ++e) {
      const int i = min(tid + e * MSCAN_THREADS, BCV - 1);
      const int u = i / (2 * N), w = (i / N) & 1, n = i % N;
      const int t = min(g0 + u, p.T - 1);
      bcn[e].load(w ? p.Cm : p.Bm, ((int64_t)bi * p.T + t) * N + n);
    }
  };
  auto stage_group = [&](int buf) {
#pragma unroll
    for (int e = 0; e < BCT; ++e) {
      const int i = tid + e * MSCAN_THREADS;
      if (i < BCV) bc_lds[buf][i] = bcn[e].get();
    }
#pragma unroll
    for (int u = 0; u < MSCAN_SUB; ++u) {
      xc[u] = xn[u].get();
      dc[u] = dn[u].get();
      zc[u] = zn[u].get();
    }
  };

  int buf = 0;
  if (t0 < t1) {
    load_group(t0);
    stage_group(0);
    __syncthreads();
  }
  // the entering state, loaded after the (conditional) first staging so that
  // on every path into the loop these are the latest loads: the first use
  // then waits for them alone, not for the group prefetched ahead of it
  if constexpr (MODE == MSCAN_SUMMARY) {
#pragma unroll
    for (int n = 0; n < NPL; ++n) h[n] = 0.f;
  } else {
    const float* src = MODE == MSCAN_OUTPUT ? p.ws_h + ws_off : hs;
    const bool zero = MODE == MSCAN_SINGLE && p.zero_init;
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const f4 v = zero ? f4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f4*>(src + 4 * q);
      h[4 * q] = v.x; h[4 * q + 1] = v.y; h[4 * q + 2] = v.z; h[4 * q + 3] = v.w;
    }
    // settle them here (s_waitcnt vmcnt(0), expcnt and lgkmcnt untouched):
    // left pending into the loop, the compiler waits for everything in
    // flight, the next group's prefetch included, at their first use
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  for (int g0 = t0; g0 < t1; g0 += MSCAN_SUB) {
    if (g0 + MSCAN_SUB < t1) load_group(g0 + MSCAN_SUB);
    const float* bc = bc_lds[buf];
#pragma unroll
    for (int u = 0; u < MSCAN_SUB; ++u) {
      const int t = g0 + u;
      if (t < t1) {  // uniform over the block
        const float dtv = dc[u], xv = xc[u];
        const float dtx = dtv * xv;
        const float* Bt = bc + u * 2 * N + NPL * j;
        const float* Ct = Bt + N;
        float acc = 0.f;
        if constexpr (MODE == MSCAN_SUMMARY) dt_sum += dtv;
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          const float dA = __builtin_amdgcn_exp2f(dtv * a2[n]);
          h[n] = dA * h[n] + dtx * Bt[n];
          if constexpr (MODE != MSCAN_SUMMARY) acc += Ct[n] * h[n];
        }
        if constexpr (MODE != MSCAN_SUMMARY) {
          if constexpr (LPN > 1) acc = group_sum<LPN>(acc);
          float y = acc + Dd * xv;
          if (has_z) y *= silu_f(zc[u]);
          if (live && j == 0) store_act1(p.out, ((int64_t)bi * p.T + t) * p.Dm + d, p.out_dt, y);
        }
      }
    }
    if (g0 + MSCAN_SUB < t1) {
      stage_group(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (!live) return;
  if constexpr (MODE == MSCAN_SUMMARY) {
    float P[NPL];
#pragma unroll
    for (int n = 0; n < NPL; ++n) P[n] = __builtin_amdgcn_exp2f(dt_sum * a2[n]);
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      *reinterpret_cast<f4*>(p.ws_P + ws_off + 4 * q) = f4{P[4 * q], P[4 * q + 1], P[4 * q + 2], P[4 * q + 3]};
      *reinterpret_cast<f4*>(p.ws_h + ws_off + 4 * q) = f4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
    }
  } else if constexpr (MODE == MSCAN_SINGLE) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q)
      *reinterpret_cast<f4*>(hs + 4 * q) = f4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
  }
}

// Carry pass: one thread per (row, channel, element), walking the chunks.
// ws_h[c] <- the state entering chunk c; the pool gets the state after the
// last chunk. Empty chunks (past the row's length) hold P = 1, h_loc = 0.
__global__ __launch_bounds__(256) void mamba_scan_carry_kernel(MambaScanParams p) {
  const int64_t per_row = (int64_t)p.Dm * p.N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.B * per_row) return;
  const int bi = (int)(i / per_row);
  const int64_t e = i - bi * per_row;  // d * N + n
  const int slot = p.idx[bi];
  if (slot < 0 || slot >= p.num_slots) return;
  float* hs = p.state + (int64_t)slot * per_row + e;
  float h = p.zero_init ? 0.f : *hs;
  // Chunks in groups of CG: the group's loads are all issued before its
  // stores (a store to ws_h ahead of the next chunk's load would make every
  // chunk wait a full memory round trip), then the short FMA chain runs.
  constexpr int CG = 16;
  const int64_t base = (int64_t)bi * p.nck * per_row + e;
  for (int c0 = 0; c0 < p.nck; c0 += CG) {
    float hl[CG], P[CG];
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const int64_t o = base + (int64_t)min(c0 + j, p.nck - 1) * per_row;
      hl[j] = p.ws_h[o];
      P[j] = p.ws_P[o];
    }
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      if (c0 + j < p.nck) {
        p.ws_h[base + (int64_t)(c0 + j) * per_row] = h;
        h = P[j] * h + hl[j];
      }
    }
  }
  *hs = h;
}

namespace {

template <int N, int ACT>
hipError_t launch_ms(const MambaScanParams& p, int n_cu, hipStream_t st) {
  constexpr int CPB = MSCAN_THREADS / (N / MSCAN_NPL);
  const dim3 grid((unsigned)((p.Dm + CPB - 1) / CPB), (unsigned)p.nck, (unsigned)p.B);
  if (p.nck == 1) {
    // A single pass over few rows and channels: 4 elements per lane (N/4
    // lanes per channel) while 16 would leave SIMDs without 4 waves (one
    // 2048-token prompt, D = 1536, N = 16: 1014 -> 739 us). The chunked
    // passes keep 16 (at 4 they measured 3% slower for one prompt and 52%
    // for eight: the lanes of a channel repeat its x, dt, z loads).
    constexpr int NPL4 = 4;
    if constexpr (N / NPL4 <= 16) {
      const int64_t waves16 = (int64_t)p.B * p.Dm * (N / MSCAN_NPL) / 64;
      if (waves16 < 16LL * n_cu) {
        constexpr int CPB4 = MSCAN_THREADS / (N / NPL4);
        const dim3 grid4((unsigned)((p.Dm + CPB4 - 1) / CPB4), 1u, (unsigned)p.B);
        mamba_scan_kernel<N, ACT, MSCAN_SINGLE, NPL4><<<grid4, dim3(MSCAN_THREADS), 0, st>>>(p);
        return hipGetLastError();
      }
    }
    mamba_scan_kernel<N, ACT, MSCAN_SINGLE><<<grid, dim3(MSCAN_THREADS), 0, st>>>(p);
    return hipGetLastError();
  }
  mamba_scan_kernel<N, ACT, MSCAN_SUMMARY><<<grid, dim3(MSCAN_THREADS), 0, st>>>(p);
  const int64_t lanes = (int64_t)p.B * p.Dm * p.N;
  mamba_scan_carry_kernel<<<dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st>>>(p);
  mamba_scan_kernel<N, ACT, MSCAN_OUTPUT><<<grid, dim3(MSCAN_THREADS), 0, st>>>(p);
  return hipGetLastError();
}

template <int N>
hipError_t launch_ms_act(const MambaScanParams& p, int n_cu, hipStream_t st) {
  switch (p.act_dt) {
    case SSMD_F32: return launch_ms<N, SSMD_F32>(p, n_cu, st);
    case SSMD_BF16: return launch_ms<N, SSMD_BF16>(p, n_cu, st);
    default: return launch_ms<N, SSMD_F16>(p, n_cu, st);
  }
}

}  // namespace

// Chunk length for a scan of B rows x T tokens x Dm channels: enough chunks
// that the summary and output passes give every SIMD of the device a few
// waves, chunks of at least 32 tokens, and no more chunks than the
// workspace holds (0 bytes: one chunk).
void mamba_scan_chunking(int B, int T, int Dm, int N, int n_cu, int64_t ws_bytes, int* Lc, int* nck) {
  const int64_t lanes = (int64_t)B * Dm * (N / MSCAN_NPL);
  const int64_t target = (int64_t)n_cu * 4 * 4 * 64;  // 4 waves per SIMD
  int64_t want = lanes >= target ? 1 : (target + lanes - 1) / lanes;
  const int64_t max_by_len = T <= 32 ? 1 : (T + 31) / 32;
  if (want > max_by_len) want = max_by_len;
  const int64_t per_chunk = 2LL * B * Dm * N * 4;
  const int64_t fit = ws_bytes / per_chunk;
  if (want > fit) want = fit;
  if (want < 1) want = 1;
  int L = (int)((T + want - 1) / want);
  L = (L + MSCAN_SUB - 1) / MSCAN_SUB * MSCAN_SUB;
  if (L < MSCAN_SUB) L = MSCAN_SUB;
  *Lc = L;
  *nck = T == 0 ? 1 : (T + L - 1) / L;
}

hipError_t launch_mamba_scan(const MambaScanParams& p, int n_cu, hipStream_t st) {
  switch (p.N) {
    case 16: return launch_ms_act<16>(p, n_cu, st);
    case 32: return launch_ms_act<32>(p, n_cu, st);
    case 64: return launch_ms_act<64>(p, n_cu, st);
    case 128: return launch_ms_act<128>(p, n_cu, st);
    case 256: return launch_ms_act<256>(p, n_cu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssmd
