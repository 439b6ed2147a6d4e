// KV-cache decode step for gfx950: split-KV partial softmax plus combine.
//
// Each sequence has one new query per head; its key and value are already
// appended to the cache and it attends to cache rows 0..ctx-1 ("Transformer :
// comprendre l'entrainement et l'inference", briefia.fr, prefill vs decode and
// the simple KV cache). Decode reads every cached K/V byte once and does
// little arithmetic per byte, so it is bound by HBM bandwidth; the design
// goal is to keep enough loads in flight and to read each K/V row once for
// all query heads that share it.
//
// decode_split: one work-group per (sequence b, KV head g, block of up to 16
//   of g's query heads, chunk of kDecodeChunk keys); chunks at or past ctx
//   exit at once. Its 4 waves split the chunk; each wave walks 32 keys per
//   step:
//     * K rows are loaded from HBM straight into the A-operand layout of
//       v_mfma_f32_16x16x32 (row = key, k = head dim), the query heads of the
//       group form the B operand (one column per head), so S^T = K Q^T reads
//       each key once for all heads of the group;
//     * the online softmax runs per head (one head per lane column);
//     * V rows go HBM -> LDS (a per-wave region) and come back transposed
//       through ds_read_b64_tr_b16 as the A operand of O^T = V^T P^T;
//     * slots at or past ctx are never loaded (zero-filled), so whatever the
//       cache holds there (NaN included) cannot reach the result.
//   The 4 wave partials are merged in LDS and the work-group writes one
//   partial (row max m in log2 units, row sum l, unnormalised O) per head.
// decode_combine: per (b, query head) merges the partials of all chunks by
//   their maxima: O = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c, which
//   is the block update of the online softmax ("FlashAttention (2022)",
//   paithon.it, section on the softmax that needs not see the whole row).
#include "common.hpp"
#include "launch.hpp"

namespace mea {

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 32;                          // keys per wave step
constexpr int kWaveKeys = kDecodeChunk / kWaves;   // keys per wave per chunk

template <int D>
struct DecShape {
  static constexpr int LDS = D + 16;               // padded row stride of a V block (elements)
  static constexpr int VTILE = kStep * LDS;        // elements per wave's V block
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int NLD = kStep * CPR / 64;     // chunks per lane per step
  static constexpr int SMEM_BYTES = kWaves * VTILE * 2;
  static constexpr int MERGE_BYTES = (2 * kWaves * 16 + kWaves * 16 * D) * 4;
  static_assert(MERGE_BYTES <= SMEM_BYTES, "merge buffer must fit in the V region");
};

template <typename T, int D>
__global__ void __launch_bounds__(256) decode_split_kernel(const DecParams p) {
  using S = DecShape<D>;
  using MF = Mfma<T>;
  typedef typename MF::v8 v8;
  constexpr int LDS = S::LDS, VTILE = S::VTILE, CPR = S::CPR, NLD = S::NLD;
  constexpr int DS = D / 32;     // k-steps of the score product (16x16x32)
  constexpr int DB = D / 16;     // 16-row output blocks

  __shared__ __attribute__((aligned(16))) uint16_t smem[S::SMEM_BYTES / 2];

  const int chunk = blockIdx.x;
  const int g = blockIdx.y / p.nhb;
  const int hb = blockIdx.y - g * p.nhb;
  const int b = blockIdx.z;
  const int ctx = min(max(p.ctx[b], 0), p.S_max);
  const int start = chunk * kDecodeChunk;
  if (start >= ctx) return;
  const int end = min(start + kDecodeChunk, ctx);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;     // query head within the block (MFMA column)
  const int grp = lane >> 4;
  const int nh = min(16, p.group - hb * 16);
  const int h = g * p.group + hb * 16 + col;
  const bool real = col < nh;

  const float c = p.scale_log2;
  const float slope = (p.alibi && real) ? p.slopes[h] * kLog2e : 0.f;

  v8 qf[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st)
    qf[st] = real ? load_v8<T>(p.q + ((long long)b * p.Hq + h) * D + st * 32 + grp * 8) : zero_v8<T>();

  const long long rstride = (long long)p.Hkv * D;
  const uint16_t* kbase = p.kc + (long long)b * p.S_max * rstride + (long long)g * D;
  const uint16_t* vbase = p.vc + (long long)b * p.S_max * rstride + (long long)g * D;
  uint16_t* Vw = smem + wave * VTILE;

  const int w0 = start + wave * kWaveKeys;
  const int w1 = min(w0 + kWaveKeys, end);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[db][r] = 0.f;

  const int ll = lane & 15;
  const int vrow = grp * 4 + (ll >> 2);
  const int vcol = 4 * (ll & 3);

  for (int key0 = w0; key0 < w1; key0 += kStep) {
    // K in the A-operand layout, V rows staged for LDS.
    v8 kf[2][DS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = key0 + kb * 16 + col;
#pragma unroll
      for (int st = 0; st < DS; ++st)
        kf[kb][st] = key < w1 ? load_v8<T>(kbase + (long long)key * rstride + st * 32 + grp * 8) : zero_v8<T>();
    }
    uint4 vst[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = lane + i * 64;
      const int r = ch / CPR;
      const int cc = (ch - r * CPR) * 8;
      const int key = key0 + r;
      vst[i] = key < w1 ? *reinterpret_cast<const uint4*>(vbase + (long long)key * rstride + cc)
                        : make_uint4(0u, 0u, 0u, 0u);
    }

    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int st = 0; st < DS; ++st) s[kb] = MF::mma16(kf[kb][st], qf[st], s[kb]);
    }

    // Scores in log2 units; keys past the wave's range are masked.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + kb * 16 + grp * 4 + r;
        float x = s[kb][r] * c;
        if (p.alibi) x -= slope * (float)(ctx - 1 - key);
        x = key < w1 ? x : -INFINITY;
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    if (__any(mx > m_run + kRescaleThreshold)) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - (mn == -INFINITY ? 0.f : mn));
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
      m_run = mn;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    v8 pf;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = fast_exp2(s[kb][r] - mu);
        psum += pv;
        pf[kb * 4 + r] = (T)pv;
      }
    l_run += psum;

    // V block -> this wave's LDS region, then O^T += V^T P^T. LDS operations
    // of one wave complete in order; the compiler barriers keep the program
    // order of stores and transpose reads.
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = lane + i * 64;
      const int r = ch / CPR;
      const int cc = (ch - r * CPR) * 8;
      *reinterpret_cast<uint4*>(Vw + r * LDS + cc) = vst[i];
    }
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* a0 = Vw + vrow * LDS + db * 16 + vcol;
      const v8 vf = lds_tr_x8<T>(a0, a0 + 16 * LDS);
      o[db] = MF::mma16(vf, pf, o[db]);
    }
    __asm__ volatile("" ::: "memory");
  }

  // ---- merge the 4 wave partials, write the chunk partial ------------------
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  __syncthreads();
  float* wm = reinterpret_cast<float*>(smem);
  float* wl = wm + kWaves * 16;
  float* wo = wl + kWaves * 16;
  if (grp == 0) {
    wm[wave * 16 + col] = m_run;
    wl[wave * 16 + col] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) wo[(wave * 16 + col) * D + db * 16 + grp * 4 + r] = o[db][r];
  __syncthreads();

  for (int idx = tid; idx < nh * D; idx += kWaves * 64) {
    const int hc = idx / D;
    const int d = idx - hc * D;
    float mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, wm[w * 16 + hc]);
    const float mref = mstar == -INFINITY ? 0.f : mstar;
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(wm[w * 16 + hc] - mref);
      acc += e * wo[(w * 16 + hc) * D + d];
      lsum += e * wl[w * 16 + hc];
    }
    const int hh = g * p.group + hb * 16 + hc;
    const long long slot = ((long long)b * p.Hq + hh) * p.nchunk + chunk;
    p.ws_o[slot * D + d] = acc;
    if (d == 0) {
      p.ws_ml[slot * 2 + 0] = mstar;
      p.ws_ml[slot * 2 + 1] = lsum;
    }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(const DecParams p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx = min(max(p.ctx[b], 0), p.S_max);
  const int n = (ctx + kDecodeChunk - 1) / kDecodeChunk;
  const long long base = ((long long)b * p.Hq + h) * p.nchunk;
  float mstar = -INFINITY;
  for (int i = 0; i < n; ++i) mstar = fmaxf(mstar, p.ws_ml[(base + i) * 2]);
  const float mref = mstar == -INFINITY ? 0.f : mstar;
  float acc = 0.f, lsum = 0.f;
  for (int i = 0; i < n; ++i) {
    const float e = fast_exp2(p.ws_ml[(base + i) * 2] - mref);
    acc += e * p.ws_o[(base + i) * D + d];
    lsum += e * p.ws_ml[(base + i) * 2 + 1];
  }
  // A row with no keys has lsum == 0 and returns 0; NaN inputs stay NaN.
  const float r = lsum != 0.f ? acc / lsum : 0.f;
  const T w = (T)r;
  p.out[((long long)b * p.Hq + h) * D + d] = __builtin_bit_cast(uint16_t, w);
}

template <typename T, int D>
hipError_t launch_typed(const DecParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(p.nchunk, p.Hkv * p.nhb, p.B), dim3(kWaves * 64), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.Hq, p.B), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int D, const DecParams& p, hipStream_t stream) {
  if (dtype == 0) return D == 64 ? launch_typed<_Float16, 64>(p, stream) : launch_typed<_Float16, 128>(p, stream);
  return D == 64 ? launch_typed<__bf16, 64>(p, stream) : launch_typed<__bf16, 128>(p, stream);
}

}  // namespace mea
