// C ABI of libmea.so (declared in include/mea.h): host-side validation,
// launch geometry, status codes. Validation happens before any HIP call, so
// an invalid call touches neither the device nor the runtime.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/mea.h"
#include "launch.hpp"

namespace {

bool mea_debug() {
  static const bool on = [] {
    const char* e = std::getenv("MEA_DEBUG");
    return e != nullptr && std::strcmp(e, "0") != 0;
  }();
  return on;
}

bool dtype_ok(int dtype) { return dtype == MEA_FP16 || dtype == MEA_BF16; }

constexpr int kMaxDevices = 64;

// Device a call's work runs on: the device of its stream (the current device
// for the null stream). -1 if the runtime cannot tell.
int stream_device(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return -1;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return -1;
  }
  return dev;
}

// Compute units of the device a call's stream runs on, queried once per
// device (256 if the query fails). Called only after a call's arguments have
// been validated. Calls from several host threads may race to fill an entry;
// they store the same value, and the entries are atomics so that race is well
// defined.
int device_compute_units(hipStream_t stream) {
  static std::atomic<int> cached[kMaxDevices];
  const int dev = stream_device(stream);
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}
bool dim_ok(int D) { return D == 64 || D == 128; }

// Validates device-resident index arrays with a synchronous copy (MEA_DEBUG=1 only).
int debug_check_seqstart(const int32_t* st, int B, int total, hipStream_t stream) {
  int32_t* h = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (size_t)(B + 1)));
  if (h == nullptr) return MEA_EINVAL;
  int rc = MEA_OK;
  if (hipMemcpyAsync(h, st, sizeof(int32_t) * (size_t)(B + 1), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    rc = MEA_EHIP;
  } else {
    if (h[0] != 0 || h[B] != total) rc = MEA_EINVAL;
    for (int s = 0; s < B && rc == MEA_OK; ++s)
      if (h[s + 1] < h[s]) rc = MEA_EINVAL;
  }
  std::free(h);
  return rc;
}

int debug_check_ctx(const int32_t* ctx, int B, int S_max, hipStream_t stream) {
  int32_t* h = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (size_t)B));
  if (h == nullptr) return MEA_EINVAL;
  int rc = MEA_OK;
  if (hipMemcpyAsync(h, ctx, sizeof(int32_t) * (size_t)B, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    rc = MEA_EHIP;
  } else {
    for (int b = 0; b < B && rc == MEA_OK; ++b)
      if (h[b] < 0 || h[b] > S_max) rc = MEA_EINVAL;
  }
  std::free(h);
  return rc;
}

}  // namespace

extern "C" {

const char* mea_strerror(int status) {
  switch (status) {
    case MEA_OK: return "success";
    case MEA_EINVAL: return "invalid argument";
    case MEA_EUNSUPPORTED: return "unsupported dtype or head dimension";
    case MEA_EWORKSPACE: return "workspace missing, too small or misaligned";
    case MEA_EHIP: return "HIP runtime error";
    case MEA_ESCRATCH: return "problem too large for the library's static decode scratch (mea_decode_noalloc)";
    default: return "unknown status";
  }
}

int mea_supported(int dtype, int D) { return (dtype_ok(dtype) && dim_ok(D)) ? 1 : 0; }

int mea_decode_chunk(void) { return mea::kDecodeChunk; }

}  // extern "C"

namespace {

// Shared by mea_fwd and mea_fwd_kvcache: validates, fills FwdParams, launches.
int fwd_impl(const void* q, const void* k, const void* v, void* out, int B, int M, int N, int Hq, int Hkv, int D,
             float scale, unsigned bias_kind, const int32_t* seqstart_q, const int32_t* seqstart_k,
             const float* alibi_slopes, int dtype, float* lse, const int32_t* kv_lens, const uint8_t* block_mask,
             void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return MEA_EINVAL;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return MEA_EINVAL;
  if (Hq % Hkv != 0) return MEA_EINVAL;
  if ((bias_kind & ~(MEA_MASK_CAUSAL | MEA_MASK_BLOCKDIAG | MEA_BIAS_ALIBI)) != 0u) return MEA_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return MEA_EINVAL;
  const bool varlen = (bias_kind & MEA_MASK_BLOCKDIAG) != 0u;
  const bool causal = (bias_kind & MEA_MASK_CAUSAL) != 0u;
  const bool alibi = (bias_kind & MEA_BIAS_ALIBI) != 0u;
  if (alibi && alibi_slopes == nullptr) return MEA_EINVAL;
  if (varlen) {
    if (seqstart_q == nullptr) return MEA_EINVAL;
    if (seqstart_k == nullptr && M != N) return MEA_EINVAL;
  }
  if (!mea_supported(dtype, D)) return MEA_EUNSUPPORTED;
  // Row strides and per-row offsets are int32 inside the kernel; whole-tensor
  // offsets are 64-bit.
  const long long q_rstride = (long long)Hq * D, kv_rstride = (long long)Hkv * D;
  if (q_rstride > 0x7fffffffLL || kv_rstride > 0x7fffffffLL) return MEA_EINVAL;
  if (block_mask != nullptr && (varlen || kv_lens != nullptr)) return MEA_EINVAL;
  // Work-group counts are int32; checked here at the smallest tile height
  // (128 rows of one head, or 32 rows of 4 heads), and exactly below.
  const long long t128 = varlen ? ((long long)M + 127) / 128 + B : ((long long)M + 127) / 128 * B;
  if (t128 * Hq > 0x7fffffffLL - 8) return MEA_EINVAL;
  // Dense D=64 without mask takes 256-row work-groups when there are enough
  // of them for two per compute unit; otherwise 128-row ones keep the GPU
  // full (measured +13 to +39 % at M <= 1024, B=4, H=16).
  bool wide = false;
  if (D == 64 && !causal && block_mask == nullptr) {
    const long long t256 = varlen ? ((long long)M + 255) / 256 + B : ((long long)M + 255) / 256 * B;
    wide = t256 * Hq >= 2LL * device_compute_units(static_cast<hipStream_t>(stream));
  }
  // Causal launches whose KV heads serve a multiple of 4 query heads use
  // 32-row work-groups of 4 query heads (one per wave) sharing one KV head.
  const bool gq = causal && block_mask == nullptr && (Hq / Hkv) % 4 == 0;
  const int BM = mea::fwd_block_m(D, causal, block_mask != nullptr, wide, gq);

  mea::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.seqstart_q = seqstart_q;
  p.seqstart_k = seqstart_k != nullptr ? seqstart_k : seqstart_q;
  p.slopes = alibi_slopes;
  p.kv_lens = kv_lens;
  p.block_mask = block_mask;
  p.nkb = (N + mea::kSparseBlock - 1) / mea::kSparseBlock;
  p.B = B;
  p.M = M;
  p.N = N;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.group = Hq / Hkv;
  p.causal = causal;
  p.varlen = varlen;
  p.alibi = alibi;
  p.wide = wide;
  p.gq = gq;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.q_rstride = (int)q_rstride;
  p.kv_rstride = (int)kv_rstride;
  long long tiles, total;
  if (varlen) {
    tiles = ((long long)M + BM - 1) / BM + B;   // each segment wastes at most one partial tile
    total = tiles * (gq ? Hq / 4 : Hq);
    p.q_bstride = 0;
    p.kv_bstride = 0;
  } else {
    tiles = ((long long)M + BM - 1) / BM;
    total = tiles * (gq ? Hq / 4 : Hq) * (long long)B;
    p.q_bstride = (long long)M * q_rstride;
    p.kv_bstride = (long long)N * kv_rstride;
  }
  if (total > 0x7fffffffLL - 8) return MEA_EINVAL;
  p.n_qtiles = (int)tiles;
  p.total_wg = (int)total;
  p.wg_per_xcd = (int)((total + 7) / 8);

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mea_debug() && varlen) {
    int rc = debug_check_seqstart(seqstart_q, B, M, st);
    if (rc == MEA_OK && seqstart_k != nullptr) rc = debug_check_seqstart(seqstart_k, B, N, st);
    if (rc != MEA_OK) return rc;
  }
  if (mea_debug() && kv_lens != nullptr) {
    const int rc = debug_check_ctx(kv_lens, B, N, st);
    if (rc != MEA_OK) return rc;
  }
  return mea::launch_fwd(dtype, D, p, st) == hipSuccess ? MEA_OK : MEA_EHIP;
}

}  // namespace

extern "C" {

int mea_fwd(const void* q, const void* k, const void* v, void* out, int B, int M, int N, int Hq, int Hkv, int D,
            float scale, unsigned bias_kind, const int32_t* seqstart_q, const int32_t* seqstart_k,
            const float* alibi_slopes, int dtype, float* lse, void* stream) {
  return fwd_impl(q, k, v, out, B, M, N, Hq, Hkv, D, scale, bias_kind, seqstart_q, seqstart_k, alibi_slopes, dtype,
                  lse, nullptr, nullptr, stream);
}

int mea_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, int B, int M, int N, int Hq, int Hkv,
                        int D, float scale, unsigned bias_kind, const uint8_t* block_mask, const float* alibi_slopes,
                        int dtype, float* lse, void* stream) {
  if (block_mask == nullptr) return MEA_EINVAL;
  if ((bias_kind & MEA_MASK_BLOCKDIAG) != 0u) return MEA_EINVAL;
  return fwd_impl(q, k, v, out, B, M, N, Hq, Hkv, D, scale, bias_kind, nullptr, nullptr, alibi_slopes, dtype, lse,
                  nullptr, block_mask, stream);
}

int mea_block_sparse_block(void) { return mea::kSparseBlock; }

int mea_fwd_kvcache(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out,
                    int B, int M, int Hq, int Hkv, int D, int S_max, float scale, unsigned bias_kind,
                    const float* alibi_slopes, int dtype, float* lse, void* stream) {
  if (ctx_lens == nullptr) return MEA_EINVAL;
  if ((bias_kind & MEA_MASK_BLOCKDIAG) != 0u) return MEA_EINVAL;
  return fwd_impl(q, kcache, vcache, out, B, M, S_max, Hq, Hkv, D, scale, bias_kind, nullptr, nullptr, alibi_slopes,
                  dtype, lse, ctx_lens, nullptr, stream);
}

int mea_kv_append(void* kcache, void* vcache, const void* k_new, const void* v_new, const int32_t* ctx_lens, int B,
                  int S_max, int Hkv, int D, int T, int dtype, void* stream) {
  if (kcache == nullptr || vcache == nullptr || k_new == nullptr || v_new == nullptr || ctx_lens == nullptr)
    return MEA_EINVAL;
  if (B <= 0 || S_max <= 0 || Hkv <= 0 || D <= 0 || T < 0) return MEA_EINVAL;
  if (!mea_supported(dtype, D)) return MEA_EUNSUPPORTED;
  if ((long long)Hkv * D > 0x7fffffffLL || B > 65535) return MEA_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mea_debug()) {
    const int rc = debug_check_ctx(ctx_lens, B, S_max, st);
    if (rc != MEA_OK) return rc;
  }
  if (T == 0) return MEA_OK;
  mea::AppendParams p{};
  p.kc = static_cast<uint16_t*>(kcache);
  p.vc = static_cast<uint16_t*>(vcache);
  p.kn = static_cast<const uint16_t*>(k_new);
  p.vn = static_cast<const uint16_t*>(v_new);
  p.ctx = ctx_lens;
  p.B = B;
  p.S_max = S_max;
  p.T = T;
  p.row_elems = Hkv * D;
  return mea::launch_kv_append(p, st) == hipSuccess ? MEA_OK : MEA_EHIP;
}

size_t mea_bwd_workspace_bytes(int B, int M, int Hq, unsigned bias_kind) {
  if (B <= 0 || M <= 0 || Hq <= 0) return 0;
  const size_t rows = ((bias_kind & MEA_MASK_BLOCKDIAG) != 0u ? 1u : (size_t)B) * (size_t)M;
  const size_t one = ((rows * (size_t)Hq * sizeof(float)) + 255) & ~(size_t)255;
  return 2 * one;
}

}  // extern "C"

namespace {

int bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int M, int N, int Hq, int Hkv, int D, float scale,
             unsigned bias_kind, const int32_t* seqstart_q, const int32_t* seqstart_k, const float* alibi_slopes,
             const uint8_t* block_mask, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return MEA_EINVAL;
  if (B <= 0 || M <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return MEA_EINVAL;
  if (Hq % Hkv != 0) return MEA_EINVAL;
  if ((bias_kind & ~(MEA_MASK_CAUSAL | MEA_MASK_BLOCKDIAG | MEA_BIAS_ALIBI)) != 0u) return MEA_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return MEA_EINVAL;
  const bool varlen = (bias_kind & MEA_MASK_BLOCKDIAG) != 0u;
  const bool causal = (bias_kind & MEA_MASK_CAUSAL) != 0u;
  const bool alibi = (bias_kind & MEA_BIAS_ALIBI) != 0u;
  if (alibi && alibi_slopes == nullptr) return MEA_EINVAL;
  if (varlen) {
    if (seqstart_q == nullptr) return MEA_EINVAL;
    if (seqstart_k == nullptr && M != N) return MEA_EINVAL;
  }
  if (varlen && block_mask != nullptr) return MEA_EINVAL;
  if (!mea_supported(dtype, D)) return MEA_EUNSUPPORTED;
  const long long q_rstride = (long long)Hq * D, kv_rstride = (long long)Hkv * D;
  if (q_rstride > 0x7fffffffLL || kv_rstride > 0x7fffffffLL) return MEA_EINVAL;
  const size_t need = mea_bwd_workspace_bytes(B, M, Hq, bias_kind);
  if (workspace == nullptr || workspace_bytes < need) return MEA_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0u) return MEA_EWORKSPACE;

  mea::BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.lse2 = static_cast<float*>(workspace);
  p.delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2);
  p.seqstart_q = seqstart_q;
  p.seqstart_k = seqstart_k != nullptr ? seqstart_k : seqstart_q;
  p.slopes = alibi_slopes;
  p.block_mask = block_mask;
  p.nkb = (N + mea::kSparseBlock - 1) / mea::kSparseBlock;
  p.B = B;
  p.M = M;
  p.N = N;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.group = Hq / Hkv;
  p.causal = causal;
  p.varlen = varlen;
  p.alibi = alibi;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.q_rstride = (int)q_rstride;
  p.kv_rstride = (int)kv_rstride;
  const long long TQ = mea::kBwdTileQ, TK = mea::kBwdTileK;
  long long qt, kt, tq, tk;
  if (varlen) {
    p.rows = M;
    qt = ((long long)M + TQ - 1) / TQ + B;   // each segment wastes at most one partial tile
    kt = ((long long)N + TK - 1) / TK + B;
    tq = qt * Hq;
    tk = kt * Hkv;
    p.q_bstride = 0;
    p.kv_bstride = 0;
  } else {
    p.rows = (long long)B * M;
    qt = ((long long)M + TQ - 1) / TQ;
    kt = ((long long)N + TK - 1) / TK;
    tq = qt * Hq * (long long)B;
    tk = kt * Hkv * (long long)B;
    p.q_bstride = (long long)M * q_rstride;
    p.kv_bstride = (long long)N * kv_rstride;
  }
  if (tq > 0x7fffffffLL - 8 || tk > 0x7fffffffLL - 8) return MEA_EINVAL;
  p.n_qtiles = (int)qt;
  p.total_wg_q = (int)tq;
  p.wg_per_xcd_q = (int)((tq + 7) / 8);
  p.n_ktiles = (int)kt;
  p.total_wg_k = (int)tk;
  p.wg_per_xcd_k = (int)((tk + 7) / 8);

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mea_debug() && varlen) {
    int rc = debug_check_seqstart(seqstart_q, B, M, st);
    if (rc == MEA_OK && seqstart_k != nullptr) rc = debug_check_seqstart(seqstart_k, B, N, st);
    if (rc != MEA_OK) return rc;
  }
  return mea::launch_bwd(dtype, D, p, st) == hipSuccess ? MEA_OK : MEA_EHIP;
}

}  // namespace

extern "C" {

int mea_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
            void* dq, void* dk, void* dv, int B, int M, int N, int Hq, int Hkv, int D, float scale,
            unsigned bias_kind, const int32_t* seqstart_q, const int32_t* seqstart_k, const float* alibi_slopes,
            int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, B, M, N, Hq, Hkv, D, scale, bias_kind, seqstart_q, seqstart_k,
                  alibi_slopes, nullptr, dtype, workspace, workspace_bytes, stream);
}

int mea_bwd_blocksparse(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int M, int N, int Hq, int Hkv, int D,
                        float scale, unsigned bias_kind, const uint8_t* block_mask, const float* alibi_slopes,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (block_mask == nullptr) return MEA_EINVAL;
  if ((bias_kind & MEA_MASK_BLOCKDIAG) != 0u) return MEA_EINVAL;
  return bwd_impl(q, k, v, out, dout, lse, dq, dk, dv, B, M, N, Hq, Hkv, D, scale, bias_kind, nullptr, nullptr,
                  alibi_slopes, block_mask, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Decode workspace: the plan ([B + 2] int32: prefix sums of ctx, then the span
// of keys per split work-group), then the partial outputs [R][Hq][D] and the
// (max, sum) pairs [R][Hq][2], R = G_max + B rows, each part 256-byte
// aligned. Split work-group w writes its partial of sequence b to row w + b:
// the sequences of a work-group are consecutive and so are the work-groups of
// a sequence, so w + b is unique and below G + B for G <= G_max split
// work-groups, whatever S_max is. A caller's workspace is sized for G_max =
// kDecodeMaxSplit (any device); the static scratch of mea_decode_noalloc for
// the split work-groups of the device it runs on.
struct DecLayout {
  size_t plan, o, ml, total;
};

DecLayout dec_layout(int B, int Hq, int D, int max_split) {
  DecLayout l{};
  const size_t rows = (size_t)max_split + (size_t)B;
  const size_t slots = rows * (size_t)Hq;
  l.plan = ((size_t)(B + 2) * sizeof(int32_t) + 255) & ~(size_t)255;
  l.o = (slots * (size_t)D * sizeof(float) + 255) & ~(size_t)255;
  l.ml = slots * 2 * sizeof(float);
  l.total = l.plan + l.o + l.ml;
  return l;
}

// Host-side checks shared by mea_decode and mea_decode_noalloc.
int decode_check(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, const void* out,
                 int B, int Hq, int Hkv, int D, int S_max, float scale, int dtype) {
  if (q == nullptr || kcache == nullptr || vcache == nullptr || ctx_lens == nullptr || out == nullptr)
    return MEA_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S_max <= 0) return MEA_EINVAL;
  if (Hq % Hkv != 0) return MEA_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale)) return MEA_EINVAL;
  if (!mea_supported(dtype, D)) return MEA_EUNSUPPORTED;
  if ((long long)Hkv * D > 0x7fffffffLL) return MEA_EINVAL;
  // Context prefix sums are int32 on the device.
  if ((long long)B * (long long)S_max > 0x7fffffffLL) return MEA_EINVAL;
  const int nhb = (Hq / Hkv + 15) / 16;
  if ((long long)Hkv * nhb > 65535 || B > 65535) return MEA_EINVAL;
  return MEA_OK;
}

// Fills DecParams over the workspace ws (laid out by lay) and launches.
int decode_launch(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out, int B,
                  int Hq, int Hkv, int D, int S_max, float scale, const float* alibi_slopes, int dtype, char* ws,
                  const DecLayout& lay, int grid, hipStream_t st) {
  mea::DecParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.kc = static_cast<const uint16_t*>(kcache);
  p.vc = static_cast<const uint16_t*>(vcache);
  p.ctx = ctx_lens;
  p.out = static_cast<uint16_t*>(out);
  p.slopes = alibi_slopes;
  p.plan = reinterpret_cast<int*>(ws);
  p.ws_o = reinterpret_cast<float*>(ws + lay.plan);
  p.ws_ml = reinterpret_cast<float*>(ws + lay.plan + lay.o);
  p.grid = grid;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.group = Hq / Hkv;
  p.S_max = S_max;
  p.nhb = (p.group + 15) / 16;
  p.alibi = alibi_slopes != nullptr;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (mea_debug()) {
    const int rc = debug_check_ctx(ctx_lens, B, S_max, st);
    if (rc != MEA_OK) return rc;
  }
  return mea::launch_decode(dtype, D, p, st) == hipSuccess ? MEA_OK : MEA_EHIP;
}

// Split work-groups of a decode step: one per compute unit of the stream's
// device (8 waves fill one), at most kDecodeMaxSplit.
int decode_grid(hipStream_t st) {
  const int cus = device_compute_units(st);
  return cus < mea::kDecodeMaxSplit ? cus : mea::kDecodeMaxSplit;
}

// Scratch of mea_decode_noalloc: the decode workspace in a static device
// array, one copy per device the library runs on, kept until the process
// ends. Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[MEA_DECODE_NOALLOC_SCRATCH_BYTES];

char* scratch_ptr(int dev) {
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = ptrs[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return static_cast<char*>(ptr);
  std::lock_guard<std::mutex> lock(mu);
  ptr = ptrs[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return static_cast<char*>(ptr);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* found = nullptr;
  const hipError_t e = hipGetSymbolAddress(&found, HIP_SYMBOL(scratch));
  if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
  if (e != hipSuccess || found == nullptr) return nullptr;
  ptrs[dev].store(found, std::memory_order_release);
  return static_cast<char*>(found);
}

}  // namespace

extern "C" {

size_t mea_decode_workspace_bytes(int B, int Hq, int D, int S_max) {
  if (B <= 0 || Hq <= 0 || D <= 0 || S_max <= 0) return 0;
  return dec_layout(B, Hq, D, mea::kDecodeMaxSplit).total;
}

int mea_decode(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out, int B,
               int Hq, int Hkv, int D, int S_max, float scale, const float* alibi_slopes, int dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = decode_check(q, kcache, vcache, ctx_lens, out, B, Hq, Hkv, D, S_max, scale, dtype);
  if (rc != MEA_OK) return rc;
  const DecLayout lay = dec_layout(B, Hq, D, mea::kDecodeMaxSplit);
  if (workspace == nullptr || workspace_bytes < lay.total) return MEA_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0u) return MEA_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return decode_launch(q, kcache, vcache, ctx_lens, out, B, Hq, Hkv, D, S_max, scale, alibi_slopes, dtype,
                       static_cast<char*>(workspace), lay, decode_grid(st), st);
}

int mea_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out,
                       int B, int Hq, int Hkv, int D, int S_max, float scale, const float* alibi_slopes, int dtype,
                       void* stream) {
  const int rc = decode_check(q, kcache, vcache, ctx_lens, out, B, Hq, Hkv, D, S_max, scale, dtype);
  if (rc != MEA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int grid = decode_grid(st);
  const DecLayout lay = dec_layout(B, Hq, D, grid);
  if (lay.total > (size_t)MEA_DECODE_NOALLOC_SCRATCH_BYTES) return MEA_ESCRATCH;
  char* ws = scratch_ptr(stream_device(st));
  if (ws == nullptr) return MEA_EHIP;
  return decode_launch(q, kcache, vcache, ctx_lens, out, B, Hq, Hkv, D, S_max, scale, alibi_slopes, dtype, ws, lay,
                       grid, st);
}

}  // extern "C"
