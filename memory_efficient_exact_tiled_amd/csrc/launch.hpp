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
  const uint8_t* block_mask;  // dense mode only, nullable: [ceil(M/64)][nkb] block-sparse mask
  int nkb;                 // key blocks per mask row: ceil(N/64)
  int B, M, N, Hq, Hkv, group;
  int causal, varlen, alibi;
  int wide;              // dense D=64 without mask: 256-row work-groups (else 128)
  int gq;                // causal, group % 4 == 0: 32-row work-groups of 4 query heads (one per wave)
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
  int* plan;             // [B + 2]: prefix sums of the clamped ctx, then the span L
  float* ws_o;           // [rows][Hq][D] unnormalised partial outputs; row = w + b
  float* ws_ml;          // [rows][Hq][2] partial (row max in log2 units, row sum)
  int B, Hq, Hkv, group, S_max, nhb;
  int grid;              // split work-groups along x: min(compute units, kDecodeMaxSplit)
  int alibi;
  float scale_log2;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;      // natural log, [B][Hq][M] (packed: [Hq][M])
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* lse2;           // workspace: lse * log2(e), +inf for rows with no key; layout of lse
  float* delta;          // workspace: rowsum(dO * O); layout of lse
  const int32_t* seqstart_q;
  const int32_t* seqstart_k;
  const float* slopes;
  const uint8_t* block_mask;   // dense mode only, nullable: [ceil(M/64)][nkb] block-sparse mask
  int nkb;
  int B, M, N, Hq, Hkv, group;
  int causal, varlen, alibi;
  float scale;           // as given
  float scale_log2;      // scale * log2(e)
  long long rows;        // query rows over all batch entries (dense B*M, packed M)
  int n_qtiles, total_wg_q, wg_per_xcd_q;   // dQ kernel: 128-row query tiles
  int n_ktiles, total_wg_k, wg_per_xcd_k;   // dK/dV kernel: 128-key tiles
  long long q_bstride;
  long long kv_bstride;
  int q_rstride;
  int kv_rstride;
};

// Query rows per forward work-group (wide: the 256-row dense D=64 tiles) and
// the shortest span of keys of a decode split work-group.
int fwd_block_m(int D, bool causal, bool block_sparse, bool wide, bool gq);
constexpr int kSparseBlock = 64;   // block edge of block-sparse masks
constexpr int kDecodeChunk = 64;        // shortest span of keys of a split work-group
constexpr int kDecodeMaxSplit = 1024;   // most split work-groups (the workspace holds that many + B rows)

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
hipError_t launch_bwd(int dtype, int D, const BwdParams& p, hipStream_t stream);
constexpr int kBwdTileQ = 128;   // query rows per dQ work-group
constexpr int kBwdTileK = 128;   // keys per dK/dV work-group

}  // namespace mea
