// KV-cache append for gfx950: copies T new key/value rows of every sequence
// into its cache at positions ctx .. ctx+T-1 (the decode phase appends the
// newest token's key and value before attending: "Transformer : comprendre
// l'entrainement et l'inference", briefia.fr, section on the simple KV cache).
//
// A pure copy, bound by HBM bandwidth: each thread moves 16-byte chunks of K
// and V, consecutive threads consecutive chunks of a row, so reads of the new
// rows and writes into the cache are both coalesced. Rows that would land at
// or past S_max are dropped (the kernel bounds every write by S_max).
#include "common.hpp"
#include "launch.hpp"

namespace mea {

namespace {

__global__ void __launch_bounds__(256) kv_append_kernel(const AppendParams p) {
  const int b = blockIdx.y;
  const int ctx = min(max(p.ctx[b], 0), p.S_max);
  const int rows = min(p.T, p.S_max - ctx);            // rows that fit
  const int cpr = p.row_elems / 8;                      // 16-byte chunks per row
  const long long total = (long long)rows * cpr;
  const long long src0 = (long long)b * p.T * p.row_elems;
  const long long dst0 = ((long long)b * p.S_max + ctx) * p.row_elems;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long e = i * 8;
    *reinterpret_cast<uint4*>(p.kc + dst0 + e) = *reinterpret_cast<const uint4*>(p.kn + src0 + e);
    *reinterpret_cast<uint4*>(p.vc + dst0 + e) = *reinterpret_cast<const uint4*>(p.vn + src0 + e);
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
  const long long chunks = (long long)p.T * (p.row_elems / 8);
  const int blocks = (int)((chunks + 255) / 256 < 1024 ? (chunks + 255) / 256 : 1024);
  hipLaunchKernelGGL(kv_append_kernel, dim3(blocks > 0 ? blocks : 1, p.B), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mea
