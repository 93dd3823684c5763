// ssmd_internal.h -- parameter blocks passed from the validated C entry points
// to the kernel launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssmdec.h"

namespace ssmd {

struct GdnParams {
  const void* qkv;
  int64_t qkv_stride;
  bool qkv_vec;  // rows are 4-element aligned: q/k fragments use vector loads
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  void* state;       // fp32 pool, or 16-bit for the state16 entry point
  int32_t state_dt;  // SSMD_F32, SSMD_BF16 or SSMD_F16
  int32_t num_slots;
  const int32_t* idx;
  void* out;
  int32_t B, H, HV, K, V;
  int32_t act_dt, out_dt;
  float scale;
  int32_t use_l2;
  float l2eps;
  const void* norm_gate;
  const float* norm_w;
  float norm_eps;
  int32_t norm_act;
  // buffered form only
  void* d_cache;
  void* k_cache;
  float* g_cache;
  const int32_t* write_pos;
  int32_t L;
};

// GDN over T tokens per sequence: g.qkv / g.a / g.b / g.norm_gate / g.out
// hold B*T token rows (token t of row b is row b*T + t).
struct GdnMultiParams {
  GdnParams g;
  int32_t T;
  const int32_t* lengths;  // [B] or NULL (all T)
  int32_t tiles, rows_per_tile, tok_floats;  // set by the launcher
};

// Chunked GDN over T tokens: ws holds one record per (row, value head,
// chunk of 64 tokens), then (gated norm only) fp32 outputs [B][T][HV][V] at obuf.
struct GdnChunkParams {
  GdnParams g;
  int32_t T;
  const int32_t* lengths;
  int32_t nck;
  float* ws;
  float* obuf;
};

// GDN step with the causal conv1d update in front: g.qkv is the pre-conv row
// x (stride g.qkv_stride); the conv state holds the last W - 1 inputs of each
// channel in the activation dtype.
struct GdnConvParams {
  GdnParams g;
  const float* conv_w;  // [C][W], C = 2 H K + HV V
  const float* conv_b;  // [C] or NULL
  void* conv_state;
  int64_t cs_slot, cs_chan, cs_tap;
  int32_t W;
};

struct KdaParams {
  const void* x;
  const float* conv_w;
  const float* conv_b;
  void* conv_state;
  int64_t cs_slot, cs_chan, cs_tap;
  const void* raw_g;
  bool raw_g_vec;  // raw_g is 4-element aligned: vector loads
  const void* raw_beta;
  float lower_bound;
  float* state;
  int32_t num_slots;
  const int32_t* idx;
  void* out;
  const void* gate;
  const float* norm_w;
  float norm_eps;
  int32_t T, H, D, W;
  int32_t act_dt, out_dt;
  float scale;
  int32_t use_l2;
  float l2eps;
};

struct MambaParams {
  const void* x;
  const void* dt;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dvec;
  const void* z;
  float* state;
  int32_t num_slots;
  const int32_t* idx;
  void* out;
  int32_t B, Dm, N;
  int32_t act_dt, out_dt;
};

// Mamba-1 scan over T tokens; ws_P / ws_h: [B][nck][Dm][N] fp32 each (nck > 1).
struct MambaScanParams {
  const void* x;
  const void* dt;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dvec;
  const void* z;
  float* state;
  int32_t num_slots;
  const int32_t* idx;
  const int32_t* lengths;
  int32_t zero_init;
  void* out;
  float* ws_P;
  float* ws_h;
  int32_t B, T, Dm, N;
  int32_t Lc, nck;  // chunk length (a multiple of 8) and chunk count
  int32_t act_dt, out_dt;
};

// Launch shape of the state-streaming kernels, chosen on the host.
struct Launch {
  int wpb;       // waves per workgroup
  int grid_cap;  // > 0: at most this many blocks, each walking units with a grid stride
  int fixed;     // 1: wpb and grid_cap as given; 0: a launcher with a shape policy picks its own
};

// Launchers: return a hipError_t from the launch.
hipError_t launch_gdn(const GdnParams& p, const Launch& l, hipStream_t s);
// Persistent prefetching form of the packed step (no output norm); the grid
// is n_cu blocks unless Launch.grid_cap says otherwise.
hipError_t launch_gdn_pf(const GdnParams& p, const Launch& l, int n_cu, hipStream_t s);
// The packed step on a 16-bit state pool (persistent prefetching blocks).
hipError_t launch_gdn_s16(const GdnParams& p, const Launch& l, int n_cu, hipStream_t s);
hipError_t launch_gdn_buffered(const GdnParams& p, const Launch& l, hipStream_t s);
hipError_t launch_kda(const KdaParams& p, const Launch& l, hipStream_t s);
// Persistent prefetching form of the KDA op for head size 64/128 and conv
// width 4 (16-byte aligned conv weights); kda_pf_supported says whether a
// call qualifies.
bool kda_pf_supported(const KdaParams& p);
hipError_t launch_kda_pf(const KdaParams& p, const Launch& l, hipStream_t s);
hipError_t launch_gdn_conv(const GdnConvParams& p, const Launch& l, int n_cu, hipStream_t s);
// Persistent conv-fused step: whether it covers the shape, and its launch with
// the given number of blocks (each walking groups with a grid stride).
bool gdn_conv_pf_fits(const GdnConvParams& p);
hipError_t launch_gdn_conv_pf(const GdnConvParams& p, int64_t blocks, hipStream_t s);
hipError_t launch_gdn_multi(const GdnMultiParams& p, const Launch& l, int n_cu, hipStream_t s);
hipError_t launch_gdn_chunk(const GdnChunkParams& p, int n_cu, hipStream_t s);
int64_t gdn_chunk_workspace_floats(int B, int T, int HV, int K, int V, bool norm);
// Device address of the chunked prefill's static workspace on the current
// device (SSMD_CHUNK_SCRATCH_BYTES bytes).
hipError_t gdn_chunk_scratch(void** ptr);
// Largest V the multi-token kernel takes with the gated RMSNorm (one block per head).
int gdn_multi_max_norm_rows(int K);
hipError_t launch_mamba(const MambaParams& p, const Launch& l, int n_cu, hipStream_t s);
hipError_t launch_mamba_scan(const MambaScanParams& p, int n_cu, hipStream_t s);
// Chunking of a Mamba scan on a device of n_cu compute units with ws_bytes of
// workspace: chunk length *Lc and count *nck (1 when ws_bytes is too small).
void mamba_scan_chunking(int B, int T, int Dm, int N, int n_cu, int64_t ws_bytes, int* Lc, int* nck);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int n_cu, hipStream_t s);

// Rows of one buffered-kernel tile, and the LDS its ring staging needs.
int buffered_rows_per_tile(int K, int V, bool norm, const Launch& l);
Launch buffered_launch(int K, bool norm, int L, int64_t heads, int n_cu, const Launch& l);
size_t buffered_lds_bytes(int K, int rows, int L);


}  // namespace ssmd
