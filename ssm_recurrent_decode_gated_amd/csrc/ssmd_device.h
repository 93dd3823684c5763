// ssmd_device.h -- device-side building blocks shared by the decode kernels
// (gfx950 / CDNA4, wave64): element conversion, lane-group reductions over
// DPP, and the row-group lane layout used to stream fp32 state rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssmdec.h"

namespace ssmd {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16, round-to-nearest-even (the default rounding mode), NaN stays
// NaN: gfx950 converts natively (v_cvt_pk_bf16_f32, two values per
// instruction), with no per-element branch.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // RNE
}

__device__ __forceinline__ float load_act1(const void* base, int64_t off, int dt);

// Load 4 consecutive activation elements (element offset `off`) as fp32.
// With `vec` (base aligned to 4 elements and `off` a multiple of 4) this is
// one 64/128-bit load; otherwise four element loads. `dt` and `vec` are
// uniform across the wave.
__device__ __forceinline__ void load_act4(const void* base, int64_t off, int dt, bool vec, float out[4]) {
  if (!vec) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = load_act1(base, off + e, dt);
    return;
  }
  if (dt == SSMD_F32) {
    f4 v = *reinterpret_cast<const f4*>(static_cast<const float*>(base) + off);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    if (dt == SSMD_BF16) {
      out[0] = __uint_as_float(v.x << 16);
      out[1] = __uint_as_float(v.x & 0xffff0000u);
      out[2] = __uint_as_float(v.y << 16);
      out[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
      out[0] = f16_bits_to_f32(v.x & 0xffffu);
      out[1] = f16_bits_to_f32(v.x >> 16);
      out[2] = f16_bits_to_f32(v.y & 0xffffu);
      out[3] = f16_bits_to_f32(v.y >> 16);
    }
  }
}

__device__ __forceinline__ float load_act1(const void* base, int64_t off, int dt) {
  if (dt == SSMD_F32) return static_cast<const float*>(base)[off];
  uint32_t h = static_cast<const uint16_t*>(base)[off];
  return dt == SSMD_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

__device__ __forceinline__ void store_act1(void* base, int64_t off, int dt, float v) {
  if (dt == SSMD_F32) {
    static_cast<float*>(base)[off] = v;
  } else {
    static_cast<uint16_t*>(base)[off] = dt == SSMD_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
  }
}

// Compile-time-typed activation loads: no dtype branch in the kernel body, so
// the compiler can keep every state load in flight across them.
template <int ACT>
__device__ __forceinline__ float ld_act(const void* base, int64_t off) {
  if constexpr (ACT == SSMD_F32) return static_cast<const float*>(base)[off];
  else if constexpr (ACT == SSMD_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[off]);
  else return f16_bits_to_f32(static_cast<const uint16_t*>(base)[off]);
}

// 4 consecutive elements; VEC: `base + off` is aligned to 4 elements.
template <int ACT, bool VEC>
__device__ __forceinline__ void ld_act4(const void* base, int64_t off, float out[4]) {
  if constexpr (!VEC) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = ld_act<ACT>(base, off + e);
  } else if constexpr (ACT == SSMD_F32) {
    f4 v = *reinterpret_cast<const f4*>(static_cast<const float*>(base) + off);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    if constexpr (ACT == SSMD_BF16) {
      out[0] = __uint_as_float(v.x << 16);
      out[1] = __uint_as_float(v.x & 0xffff0000u);
      out[2] = __uint_as_float(v.y << 16);
      out[3] = __uint_as_float(v.y & 0xffff0000u);
    } else {
      out[0] = f16_bits_to_f32(v.x & 0xffffu);
      out[1] = f16_bits_to_f32(v.x >> 16);
      out[2] = f16_bits_to_f32(v.y & 0xffffu);
      out[3] = f16_bits_to_f32(v.y >> 16);
    }
  }
}

template <int ACT>
__device__ __forceinline__ void st_act(void* base, int64_t off, float v) {
  if constexpr (ACT == SSMD_F32) static_cast<float*>(base)[off] = v;
  else if constexpr (ACT == SSMD_BF16) static_cast<uint16_t*>(base)[off] = f32_to_bf16_bits(v);
  else static_cast<uint16_t*>(base)[off] = f32_to_f16_bits(v);
}

// A run of n consecutive fp32 values src[0..n) (in LDS or registers) bound
// for base[off .. off + n) in dtype dt.
struct StoreRun {
  void* base;
  int64_t off;
  int dt;
  const float* src;
  int n;
};

// One 16-byte piece of a run: `per` values from sv to q, converted to dt.
__device__ __forceinline__ void store_piece16(void* q, int dt, const float* sv) {
  if (dt == SSMD_F32) {
    *reinterpret_cast<f4*>(q) = f4{sv[0], sv[1], sv[2], sv[3]};
  } else {
    u4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = dt == SSMD_BF16 ? f32_to_bf16_bits(sv[2 * k]) : f32_to_f16_bits(sv[2 * k]);
      const uint32_t hi = dt == SSMD_BF16 ? f32_to_bf16_bits(sv[2 * k + 1]) : f32_to_f16_bits(sv[2 * k + 1]);
      w[k] = lo | (hi << 16);
    }
    *reinterpret_cast<u4*>(q) = w;
  }
}

// Unaligned head and tail of a run as element stores; returns the byte
// address of its first 16-byte-aligned element and the number of 16-byte
// pieces after it (head elements come first).
__device__ __forceinline__ char* run_edges(const StoreRun& r, int tid, int bd, int* head, int* nvec) {
  const int esz = r.dt == SSMD_F32 ? 4 : 2;
  char* d = static_cast<char*>(r.base) + r.off * esz;
  *head = min(r.n, (int)(((16 - ((uintptr_t)d & 15)) & 15) / esz));
  *nvec = (r.n - *head) / (16 / esz);
  const int tail0 = *head + *nvec * (16 / esz);
  for (int e = tid; e < *head; e += bd) store_act1(r.base, r.off + e, r.dt, r.src[e]);
  for (int e = tail0 + tid; e < r.n; e += bd) store_act1(r.base, r.off + e, r.dt, r.src[e]);
  return d + (int64_t)*head * esz;
}

// Writes two runs, spread over a block's threads (tid of bd): their
// 16-byte-aligned parts as 16-byte stores in one combined pass (both runs'
// pieces issued together), the unaligned head and tail of each as element
// stores. Runs written this way reach memory as whole lines instead of
// scattered 2-byte pieces, which inside a read-only stream cost far more
// than their bytes. A run with n = 0 writes nothing.
__device__ __forceinline__ void store_runs(const StoreRun& a, const StoreRun& b, int tid, int bd) {
  int ha, na, hb, nb;
  char* const da = run_edges(a, tid, bd, &ha, &na);
  char* const db = run_edges(b, tid, bd, &hb, &nb);
  const int pa = a.dt == SSMD_F32 ? 4 : 8, pb = b.dt == SSMD_F32 ? 4 : 8;  // values per piece
  for (int v = tid; v < na + nb; v += bd) {
    const bool first = v < na;
    const int i = first ? v : v - na;
    const int per = first ? pa : pb;
    char* const q = (first ? da : db) + (int64_t)i * 16;
    const float* const sv = (first ? a.src + ha : b.src + hb) + i * per;
    store_piece16(q, first ? a.dt : b.dt, sv);
  }
}

// Stores 4 consecutive fp32 values to base[off .. off + 4) in dtype dt from
// one lane: one 8-byte (16-bit types) or 16-byte (fp32) store where aligned,
// element stores otherwise.
__device__ __forceinline__ void store4(void* base, int64_t off, int dt, const float v[4]) {
  if (dt == SSMD_F32) {
    float* d = static_cast<float*>(base) + off;
    if (((uintptr_t)d & 15) == 0) {
      *reinterpret_cast<f4*>(d) = f4{v[0], v[1], v[2], v[3]};
      return;
    }
  } else {
    uint16_t* d = static_cast<uint16_t*>(base) + off;
    if (((uintptr_t)d & 7) == 0) {
      uint32_t h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) h[k] = dt == SSMD_BF16 ? f32_to_bf16_bits(v[k]) : f32_to_f16_bits(v[k]);
      *reinterpret_cast<uint2*>(d) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) store_act1(base, off + k, dt, v[k]);
}

// ------------------------------------------------------------- math
__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// ------------------------------------------------------------- reductions
// DPP lane moves within a row of 16 lanes (gfx9 encodings). Every pattern
// below reads a lane of the caller's own group, and groups are active or
// inactive as a whole, so no lane reads a disabled or out-of-row source and
// bound_ctrl never takes effect; setting it lets the compiler fold the move
// into the add that consumes it (one v_add_f32_dpp per step).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <- lane 15-i within 16

// Sum over aligned groups of LPR lanes (LPR in {2,4,8,16}); every lane of the
// group receives the group total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "lane group");
  x += dpp_mov<DPP_XOR1>(x);
  if constexpr (LPR >= 4) x += dpp_mov<DPP_XOR2>(x);
  if constexpr (LPR >= 8) x += dpp_mov<DPP_HALF_MIRROR>(x);
  if constexpr (LPR >= 16) x += dpp_mov<DPP_ROW_MIRROR>(x);
  return x;
}

// Sum over the whole wave (64 lanes); every lane receives the total.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// ------------------------------------------------------------- unit order
// Work unit -> (batch row bi, value head hv, row tile), XCD-aware: the
// G * tiles units that share one q/k head (its G = HV/H value heads, all
// their tiles) get unit indices that are equal mod 8. Workgroups go to the 8
// XCDs round robin, so with one block per unit they run on one XCD and read
// that head's q and k from its L2 rather than from HBM once per XCD. Groups
// past the last whole set of 8 map in order. A bijection for any B, H, HV,
// tiles.
__device__ __forceinline__ void xcd_unit(int unit, int B, int H, int HV, int tiles, int& bi, int& hv, int& tile) {
  const int G = HV / H;
  const int n_share = G * tiles;
  const int n_groups = B * H;
  const int in_sets = (n_groups / 8) * 8 * n_share;
  int gi, m;
  if (unit < in_sets) {
    const int sx = unit >> 3;
    gi = (sx / n_share) * 8 + (unit & 7);
    m = sx % n_share;
  } else {
    const int r = unit - in_sets;
    gi = (n_groups / 8) * 8 + r / n_share;
    m = r % n_share;
  }
  tile = m % tiles;
  bi = gi / H;
  hv = (gi - bi * H) * G + m / tiles;
}

// ------------------------------------------------------------- row layout
// A head's state is V rows of K fp32 (row = value index). A row is split
// over LPR lanes; lane c of a row owns the float4 columns c, c+LPR, c+2*LPR,
// ... so each wave-wide 128-bit access covers (64/LPR) rows x 16*LPR
// contiguous bytes. q and k fragments follow the same columns, so they are
// lane constants for the whole head.
template <int K>
struct RowLayout {
  static_assert(K == 16 || K == 32 || K == 64 || K == 128 || K == 256, "head size");
  static constexpr int LPR = K >= 32 ? 8 : K / 4;  // lanes per row
  static constexpr int NV = K / (4 * LPR);         // float4 per lane per row
  static constexpr int RPI = 64 / LPR;             // rows per wave-wide access
  __device__ static __forceinline__ int col(int c, int j) { return 4 * (c + LPR * j); }
};

// Row layout for a state of 16-bit elements: a lane's 128-bit access holds
// EV = 8 consecutive elements, so lane c of a row owns columns
// 8(c + LPR j) .. 8(c + LPR j) + 7; one wave-wide access covers RPI rows x 128
// contiguous bytes, as in the fp32 layout.
template <int K>
struct RowLayout16 {
  static_assert(K == 16 || K == 32 || K == 64 || K == 128 || K == 256, "head size");
  static constexpr int EV = 8;
  static constexpr int LPR = K / EV >= 8 ? 8 : K / EV;  // lanes per row
  static constexpr int NV = K / (EV * LPR);            // 128-bit accesses per lane per row
  static constexpr int RPI = 64 / LPR;                  // rows per wave-wide access
  __device__ static __forceinline__ int col(int c, int j) { return EV * (c + LPR * j); }
};

template <bool NT>
__device__ __forceinline__ u4 ld16x8(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  else return *reinterpret_cast<const u4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st16x8(void* p, u4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u4*>(p));
  else *reinterpret_cast<u4*>(p) = v;
}

// 8 packed 16-bit values <-> fp32 (ST = SSMD_BF16 or SSMD_F16; RNE on packing)
template <int ST>
__device__ __forceinline__ void unpack8(u4 v, float out[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = v[w];
    if constexpr (ST == SSMD_BF16) {
      out[2 * w] = __uint_as_float(x << 16);
      out[2 * w + 1] = __uint_as_float(x & 0xffff0000u);
    } else {
      out[2 * w] = f16_bits_to_f32(x & 0xffffu);
      out[2 * w + 1] = f16_bits_to_f32(x >> 16);
    }
  }
}

// Eight fp32 values to eight 16-bit ones (RNE), two per 32-bit word, low
// half first. Converting pairs as vectors lets gfx950 round both halves of a
// word in one v_cvt_pk_bf16_f32 instead of two single conversions and a merge.
template <int ST>
__device__ __forceinline__ u4 pack8(const float in[8]) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  u4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f2v x = {in[2 * w], in[2 * w + 1]};
    if constexpr (ST == SSMD_BF16) v[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2v));
    else v[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, h2v));
  }
  return v;
}

template <bool NT>
__device__ __forceinline__ f4 ld4(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
  else return *reinterpret_cast<const f4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st4(float* p, f4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
  else *reinterpret_cast<f4*>(p) = v;
}

}  // namespace ssmd
