// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mea {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const int32_t* seqstart_q;
  const int32_t* seqstart_k;
  const float* slopes;
  const int32_t* kv_lens;  // dense mode only, nullable: per-batch key count (clamped to N)
  int B, M, N, Hq, Hkv, group;
  int causal, varlen, alibi;
  float scale_log2;      // scale * log2(e)
  int n_qtiles;          // dense: q tiles per (batch, head); packed: bound on tiles over all segments
  int total_wg;          // logical work-groups
  int wg_per_xcd;        // ceil(total_wg / 8)
  long long q_bstride;   // elements between batch rows (dense)
  long long kv_bstride;
  int q_rstride;         // elements between consecutive tokens: Hq * D
  int kv_rstride;        // Hkv * D
};

struct DecParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* ctx;
  uint16_t* out;
  const float* slopes;
  float* ws_o;           // [B][Hq][nchunk][D] unnormalised partial outputs
  float* ws_ml;          // [B][Hq][nchunk][2] partial (row max in log2 units, row sum)
  int B, Hq, Hkv, group, S_max, nchunk, nhb;
  int alibi;
  float scale_log2;
};

// Query rows per forward work-group and the decode chunk length.
int fwd_block_m(int D, bool causal);
constexpr int kDecodeChunk = 512;

struct AppendParams {
  uint16_t* kc;
  uint16_t* vc;
  const uint16_t* kn;
  const uint16_t* vn;
  const int32_t* ctx;
  int B, S_max, T, row_elems;  // row_elems = Hkv * D
};

hipError_t launch_fwd(int dtype, int D, const FwdParams& p, hipStream_t stream);
hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_decode(int dtype, int D, const DecParams& p, hipStream_t stream);

}  // namespace mea
