// Shared device helpers for the gfx950 attention kernels: vector types, MFMA
// wrappers and the LDS transpose read.
//
// Operand layouts used throughout (wave64, verified on gfx950):
//   v_mfma_f32_32x32x16_{bf16,f16}: A lane l holds row l%32, k = (l/32)*8 + 0..7;
//     B lane l holds column l%32, same k; C/D lane l holds column l%32 and
//     rows (r/4)*8 + (l/32)*4 + r%4 for r = 0..15.
//   v_mfma_f32_16x16x32_{bf16,f16}: A lane l holds row l%16, k = (l/16)*8 + 0..7;
//     B lane l holds column l%16, same k; C/D lane l holds column l%16 and rows
//     (l/16)*4 + r for r = 0..3.
//   v_mfma_f32_16x16x16{bf16_1k,f16}: as above with k = (l/16)*4 + 0..3.
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane s addresses 8 bytes
//     (4 elements); lane s of the result receives element (s % 4) of the
//     addresses given by lanes 4*j + s/4, j = 0..3, i.e. when the 16 lanes
//     address a 4-row x 16-column block of a row-major tile (lane s: row s/4,
//     columns 4*(s%4)..+3), lane s gets column s of rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ f32x16 mma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16k16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                     c, 0, 0, 0);
  }
};

template <>
struct Mfma<_Float16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x16 mma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16k16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

// Eight elements from two transpose reads of LDS (see the layout note above).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::v8 lds_tr_x8(const uint16_t* p0, const uint16_t* p1) {
  typedef typename Mfma<T>::v4 v4;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  v4 x = __builtin_bit_cast(v4, a);
  v4 y = __builtin_bit_cast(v4, b);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::v4 lds_tr_x4(const uint16_t* p0) {
  return __builtin_bit_cast(typename Mfma<T>::v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0)));
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::v8 load_v8(const uint16_t* p) {
  return __builtin_bit_cast(typename Mfma<T>::v8, *reinterpret_cast<const uint4*>(p));
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::v8 zero_v8() {
  return __builtin_bit_cast(typename Mfma<T>::v8, make_uint4(0u, 0u, 0u, 0u));
}

// Raw buffer resource over [base, base + bytes): 16-byte loads at offsets at
// or past `bytes` return zeros instead of touching memory, which is how row
// ranges (segment ends, context lengths) are enforced without branches.
// Word 3 is the gfx9-family default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Streaming variant: the non-temporal cache policy (bit 1 of the policy
// operand) for data read exactly once, such as a KV cache scanned by one
// decode step; it measured 9 % faster than the default policy there.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2));
}

// LDS DMA (buffer_load_dwordx4 ... lds): lane i of the wave copies 16 bytes
// from the buffer at voff to lds_dst + 16 * i; lds_dst is wave-uniform. The
// copy completes asynchronously (vmcnt), ahead of any barrier that publishes it.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds_dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 0);
}

// Byte count of rows [0, n) of a row-major tensor, clamped to the 32-bit
// range of a buffer resource (n <= 0 gives 0).
__device__ __forceinline__ uint32_t rows_bytes(long long n, long long row_bytes) {
  const long long b = n > 0 ? n * row_bytes : 0;
  return b > 0xffffffffLL ? 0xffffffffu : (uint32_t)b;
}

// Work-group skip lists of block-sparse masks. The tiles [0, n) are
// evaluated 256 at a time: each of the work-group's 256 threads tests one
// tile with pred, a ballot per wave packs the results into a 256-bit set in
// LDS, and the next tile that is on is then found with bit scans. Every
// thread must call next_on with the same arguments (it holds barriers).
struct TileSkipList {
  uint64_t* lds;      // 4 words of LDS
  int win = -1;       // window (tile / 256) held in bits
  uint64_t bits[4];

  template <typename Pred>
  __device__ __forceinline__ int next_on(int t, int n, Pred pred) {
    while (t < n) {
      const int w = t >> 8;
      if (w != win) {
        __syncthreads();                        // readers of the previous window are done
        const int tt = (w << 8) + (int)threadIdx.x;
        const unsigned long long b = __ballot(tt < n && pred(tt));
        if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = b;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) bits[i] = lds[i];
        win = w;
      }
      const int pos = t & 255;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < (pos >> 6)) continue;
        uint64_t m = bits[i];
        if (i == (pos >> 6)) m &= ~0ull << (pos & 63);
        if (m != 0) return (w << 8) + i * 64 + __builtin_ctzll(m);
      }
      t = (w + 1) << 8;
    }
    return n;
  }
};

// Packed batches: segment s of the prefix sums st (clamped to [0, total])
// owns the logical tiles [base(s), base(s) + ntile(s)) of height bt, with
// base(s) = floor(st[s] / bt) + s and ntile(s) = ceil(len(s) / bt). Since
// floor(st[s+1] / bt) - floor(st[s] / bt) + 1 >= ceil(len(s) / bt), these
// ranges are disjoint and in segment order, and they end at or before
// ceil(total / bt) + B. The segment of logical tile t is then the last s with
// base(s) <= t, found by binary search: O(log B) reads of st whatever the
// number of segments (a serial scan costs O(B) per work-group). Returns that
// segment and the tile's rank in it, or B when t falls in the gap after a
// segment's last tile (that work-group has nothing to do). Malformed prefix
// sums give wrong segments but every returned row range stays in [0, total].
__device__ __forceinline__ int find_segment_tile(const int32_t* st, int B, int total, int bt, int t, int& rank,
                                                 int& a0, int& a1, int& ntile) {
  auto base = [&](int s) { return min(max(st[s], 0), total) / bt + s; };
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base(mid) <= t) lo = mid; else hi = mid - 1;
  }
  const int b0 = base(lo);
  a0 = min(max(st[lo], 0), total);
  a1 = min(max(st[lo + 1], a0), total);
  ntile = (a1 - a0 + bt - 1) / bt;
  rank = t - b0;
  return (rank >= 0 && rank < ntile) ? lo : B;
}

// Launch order of causal launches: logical work-group pid -> (tile rank t,
// head slot bh), tile rank major (longest tiles first) with the head slots
// innermost. A head slot is bh = stream * group + r, where a stream is one
// (batch row, KV head) whose group query heads read the same K/V. Work-group
// p runs on XCD p % 8, and every XCD has its own L2: when the streams split
// evenly over the 8 XCDs, stream s is pinned to XCD s % 8, so all query heads
// reading one K/V stream share one L2 (each K/V byte is then fetched from HBM
// once, not once per XCD its query heads were dealt to). Otherwise the head
// slots are dealt round-robin over the XCDs.
__host__ __device__ inline void causal_order(int pid, int nbh, int group, int& t, int& bh) {
  const int nstreams = nbh / group;
  if ((nstreams & 7) != 0 || group == 1) {
    t = pid / nbh;                       // with group == 1 this is the same pinning
    bh = pid - t * nbh;
    return;
  }
  const int x = pid & 7;
  const int hpx = nbh >> 3;              // head slots per XCD per tile rank
  const int slot = pid >> 3;
  t = slot / hpx;
  const int rem = slot - t * hpx;
  bh = (x + 8 * (rem / group)) * group + rem % group;
}

// 2^x on the transcendental unit (v_exp_f32): exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_xor(float x, int mask) { return fmaxf(x, __shfl_xor(x, mask)); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling: the running row maximum is only raised when a block's
// maximum exceeds it by more than this many powers of two, so P <= 2^8.
constexpr float kRescaleThreshold = 8.0f;

}  // namespace mea
