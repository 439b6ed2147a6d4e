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
// decode_plan: prefix sums of the context lengths and the span L of keys per
//   split work-group, L = max(kDecodeChunk, ceil(sum ctx / G)) for G split
//   work-groups (one per compute unit), into the workspace header. Every
//   split work-group then gets the same amount of work whatever the length
//   mix, so no last round of long chunks runs on a mostly idle GPU, and a
//   short batch (one sequence of a few thousand keys) still spreads over the
//   whole GPU.
// decode_split: work-group w takes the keys [w L, (w+1) L) of the sequences
//   laid end to end, for 8 consecutive (KV head g, block of up to 16 of g's
//   query heads) units, one per wave: the 8 waves read the same cache rows
//   (all KV heads of a position sit side by side) at the same time. A range
//   that spans several sequences yields one partial per sequence, in
//   workspace row w + b (unique: a work-group's sequences are consecutive,
//   and so are a sequence's work-groups). A wave walks its keys 16 per
//   step with two register stages (the next step's loads are in flight while
//   the current one is computed):
//     * K rows are loaded from HBM straight into the A-operand layout of
//       v_mfma_f32_16x16x32 (row = key, k = head dim), the query heads of the
//       group form the B operand (one column per head), so S^T = K Q^T reads
//       each key once for all heads of the group;
//     * the online softmax runs per head (one head per lane column); P is
//       rounded to the input type and the row sum is taken over the rounded
//       values, so the normaliser matches the weights P.V uses;
//     * V rows go HBM -> registers -> the wave's LDS region and come back
//       transposed through ds_read_b64_tr_b16 as the A operand of
//       O^T = V^T P^T (v_mfma_f32_16x16x16);
//     * all K/V loads are buffer loads whose resource ends at the last key
//       of the sequence's part of the span: cache slots at or past ctx read
//       as zeros and are masked, so whatever the cache holds there (NaN
//       included) cannot reach the result;
//       they use the non-temporal cache policy, since each cache row is read
//       once per step;
//   Each wave writes its partial (row max m in log2 units, row sum l,
//   unnormalised O) per head to the workspace.
// decode_combine: per (b, query head) merges the partials of the work-groups
//   that covered the sequence by their maxima: O = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c, which
//   is the block update of the online softmax ("FlashAttention (2022)",
//   paithon.it, section on the softmax that needs not see the whole row).
#include "common.hpp"
#include "launch.hpp"

namespace mea {

namespace {

constexpr int kWaves = 8;      // (KV head, head block) units per work-group
constexpr int kKStep = 16;     // keys per wave step
constexpr int kStages = 2;     // register stages of K/V per wave
constexpr int kInlinePlan = 512;   // batches up to this size are planned inside the split kernel

template <int D, int KSTEP>
struct DecShape {
  static constexpr int LDS = D + 16;               // padded row stride of a V block (elements)
  static constexpr int VTILE = KSTEP * LDS;        // elements per wave's V block
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int NLD = KSTEP * CPR / 64;     // V chunks per lane per step
};

// One wave: prefix sums of the clamped context lengths, then the span L,
// into dst[0 .. B + 1]. Lane i takes sequences [i * per, (i + 1) * per): it
// sums them, a wave-wide shuffle scan gives each lane its starting offset,
// and a second pass writes the running sums (no LDS, no barrier).
__device__ __forceinline__ void plan_wave(const DecParams& p, int* dst, int lane) {
  const int per = (p.B + 63) / 64;
  const int b0 = lane * per;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < p.B) sum += min(max(p.ctx[b], 0), p.S_max);
  }
  int x = sum;   // inclusive scan over the lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  int run = x - sum;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < p.B) {
      run += min(max(p.ctx[b], 0), p.S_max);
      dst[b + 1] = run;
    }
  }
  if (lane == 0) dst[0] = 0;
  if (lane == 63) {
    const long long per_wg = ((long long)x + p.grid - 1) / p.grid;   // x: the total at the last lane
    const long long L = max((long long)kDecodeChunk, (per_wg + 15) / 16 * 16);
    dst[p.B + 1] = (int)min(L, (long long)0x7fffffff);
  }
}

// The plan as a kernel of its own (batches of more than kInlinePlan
// sequences; smaller ones are planned inside the split kernel).
__global__ void __launch_bounds__(64) decode_plan_kernel(const DecParams p) {
  plan_wave(p, p.plan, threadIdx.x);
}

// One wave = one (KV head g, block of up to 16 of g's query heads) over the
// work-group's span of keys; the waves of a work-group take consecutive
// units, so they read the same cache rows at the same time. KSTEP keys per step (16 or 32);
// STAGES register stages of K/V: the loads of the next STAGES-1 steps are in
// flight while the current step is computed.
template <typename T, int D, int KSTEP, int STAGES, bool INLINE_PLAN>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_split_kernel(const DecParams p) {
  using S = DecShape<D, KSTEP>;
  using MF = Mfma<T>;
  typedef typename MF::v8 v8;
  typedef typename MF::v4 v4;
  constexpr int LDS = S::LDS, VTILE = S::VTILE, CPR = S::CPR, NLD = S::NLD;
  constexpr int DS = D / 32;     // k-steps of the score product (16x16x32)
  constexpr int DB = D / 16;     // 16-row output blocks
  constexpr int KB = KSTEP / 16; // 16-key blocks per step

  __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * VTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is made visibly wave-uniform: the K/V buffer resources
  // depend on it (through the KV head), and a resource the compiler takes
  // for divergent turns every load into a loop over lanes (readfirstlane,
  // compare, exec mask) whose pending loads its wait counting then
  // overestimates, so each step waited for the loads of the next.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // [B + 1] prefix sums of ctx, then L: from the plan kernel, or (small
  // batches) computed here by wave 0 into LDS, work-group (0, 0) also
  // storing it for the combine.
  const int* prefix = p.plan;
  if constexpr (INLINE_PLAN) {
    __shared__ int splan[kInlinePlan + 2];
    if (wave == 0) {
      plan_wave(p, splan, lane);
      if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = lane; i < p.B + 2; i += 64) p.plan[i] = splan[i];
    }
    __syncthreads();
    prefix = splan;
  }
  const int unit = blockIdx.y * kWaves + wave;
  if (unit >= p.Hkv * p.nhb) return;
  const int g = unit / p.nhb;
  const int hb = unit - g * p.nhb;
  const int total = prefix[p.B];
  const int L = prefix[p.B + 1];
  const long long lo64 = (long long)blockIdx.x * L;
  if (lo64 >= total) return;
  const int lo = (int)lo64;
  const int hi = (int)min(lo64 + L, (long long)total);
  // First sequence with keys at or past lo: the last b with prefix[b] <= lo
  // whose prefix grows after it (binary search over the prefix sums).
  int bl = 0, bh = p.B - 1;
  while (bl < bh) {
    const int mid = (bl + bh + 1) >> 1;
    if (prefix[mid] <= lo) bl = mid; else bh = mid - 1;
  }
  for (int b = bl; b < p.B && prefix[b] < hi; ++b) {
  const int ctx = prefix[b + 1] - prefix[b];
  const int w0 = max(lo - prefix[b], 0);
  const int w1 = min(hi - prefix[b], ctx);
  if (w1 <= w0) continue;
  const long long prow = (long long)blockIdx.x + b;   // workspace row of this partial

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

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[db][r] = 0.f;

  const int ll = lane & 15;
  const int vrow = grp * 4 + (ll >> 2);
  const int vcol = 4 * (ll & 3);

  struct Stage {
    v8 kf[KB][DS];    // K, A-operand layout (row = key, k = head dim)
    uint4 vst[NLD];   // V rows, bound for LDS
  };
  // Per-lane byte offsets inside one step's rows; the buffer resource is
  // rebased on each step and ends at the last key of this sequence's part of
  // the span, so rows past it read as zeros.
  const uint32_t row_bytes = (uint32_t)rstride * 2u;
  const uint32_t koff_lane = (uint32_t)col * row_bytes + (uint32_t)grp * 16u;
  uint32_t voff_lane[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int ch = lane + i * 64;
    const int r = ch / CPR;
    voff_lane[i] = (uint32_t)r * row_bytes + (uint32_t)(ch - r * CPR) * 16u;
  }
  auto load = [&](Stage& sg, int key0) {
    const uint32_t bytes = rows_bytes(w1 - key0, row_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (long long)key0 * rstride, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + (long long)key0 * rstride, bytes);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int st = 0; st < DS; ++st)
        sg.kf[kb][st] = __builtin_bit_cast(v8, buf_load16_nt(rk, koff_lane + kb * 16 * row_bytes + st * 64));
#pragma unroll
    for (int i = 0; i < NLD; ++i) sg.vst[i] = buf_load16_nt(rv, voff_lane[i]);
  };
  auto compute = [&](const Stage& sg, int key0) {
    f32x4 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int st = 0; st < DS; ++st) s[kb] = MF::mma16(sg.kf[kb][st], qf[st], s[kb]);
    }

    // Scores in log2 units; keys past the sequence's part of the span are masked.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
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
    T pv[KB * 4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[kb * 4 + r] = (T)fast_exp2(s[kb][r] - mu);
    // Row sum of the rounded P (the weights P.V uses, as in the forward), two
    // at a time.
    typedef T T2 __attribute__((ext_vector_type(2)));
    const T2 one2 = {(T)1.f, (T)1.f};
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < KB * 4; u += 2) {
      const T2 pp = {pv[u], pv[u + 1]};
      if constexpr (__is_same(T, __bf16))
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, psum, false);
      else
        psum = __builtin_amdgcn_fdot2(pp, one2, psum, false);
    }
    l_run += psum;

    // V block -> this wave's LDS region, then O^T += V^T P^T. LDS operations
    // of one wave complete in order; the compiler barriers keep the program
    // order of stores and transpose reads.
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = lane + i * 64;
      const int r = ch / CPR;
      const int cc = (ch - r * CPR) * 8;
      *reinterpret_cast<uint4*>(Vw + r * LDS + cc) = sg.vst[i];
    }
    __asm__ volatile("" ::: "memory");
    if constexpr (KSTEP == 32) {
      v8 pf;
#pragma unroll
      for (int u = 0; u < 8; ++u) pf[u] = pv[u];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* a0 = Vw + vrow * LDS + db * 16 + vcol;
        o[db] = MF::mma16(lds_tr_x8<T>(a0, a0 + 16 * LDS), pf, o[db]);
      }
    } else {
      v4 pf;
#pragma unroll
      for (int u = 0; u < 4; ++u) pf[u] = pv[u];
#pragma unroll
      for (int db = 0; db < DB; ++db)
        o[db] = MF::mma16k16(lds_tr_x4<T>(Vw + vrow * LDS + db * 16 + vcol), pf, o[db]);
    }
    __asm__ volatile("" ::: "memory");
  };

  // The next stages' loads are issued unconditionally: a step at or past w1
  // gets an empty buffer resource, so its loads return zeros without
  // touching memory. A conditional prefetch leaves the compiler unsure
  // whether those loads are in flight, and its wait counts then assume they
  // are not: each step waited for the loads of the next one as well.
  if constexpr (STAGES == 3) {
    Stage s0, s1, s2;
    int key0 = w0;
    load(s0, key0);
    load(s1, key0 + KSTEP);
    while (true) {
      load(s2, key0 + 2 * KSTEP);
      compute(s0, key0);
      key0 += KSTEP;
      if (key0 >= w1) break;
      load(s0, key0 + 2 * KSTEP);
      compute(s1, key0);
      key0 += KSTEP;
      if (key0 >= w1) break;
      load(s1, key0 + 2 * KSTEP);
      compute(s2, key0);
      key0 += KSTEP;
      if (key0 >= w1) break;
    }
  } else if constexpr (STAGES == 2) {
    Stage sa, sb;
    int key0 = w0;
    load(sa, key0);
    while (true) {
      load(sb, key0 + KSTEP);
      compute(sa, key0);
      key0 += KSTEP;
      if (key0 >= w1) break;
      load(sa, key0 + KSTEP);
      compute(sb, key0);
      key0 += KSTEP;
      if (key0 >= w1) break;
    }
  } else {
    for (int key0 = w0; key0 < w1; key0 += KSTEP) {
      Stage sg;
      load(sg, key0);
      compute(sg, key0);
    }
  }

  // ---- this wave's partial for the sequence's part of the span -----------------
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (real) {
    const long long ws = prow * p.Hq + h;
    float* dst = p.ws_o + ws * D + grp * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(dst + db * 16) = o[db];
    if (grp == 0) {
      p.ws_ml[ws * 2 + 0] = m_run;
      p.ws_ml[ws * 2 + 1] = l_tot;
    }
  }
  }   // sequences of the range
}

// One work-group of 256 threads per (sequence, query head). A partial's
// output row (D floats) is read by D / 4 threads, 16 bytes each, so a pass
// merges 1024 / D partials at once: thread t takes the float4 t % (D / 4) of
// partials t / (D / 4), t / (D / 4) + 1024 / D, ... (independent loads, no
// chain through memory even for the hundreds of partials of one long
// sequence), and the 1024 / D groups are summed through LDS at the end.
template <typename T, int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(const DecParams p) {
  constexpr int NT = 256, TPR = D / 4, RPP = NT / TPR;   // threads per row, rows per pass
  __shared__ f32x4 red[NT];
  __shared__ float lred[RPP];
  __shared__ float wmax[NT / 64];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int* prefix = p.plan;
  const int L = prefix[p.B + 1];
  const int ctx = prefix[b + 1] - prefix[b];
  // Partials of the work-groups w = floor(prefix[b] / L) .. floor((prefix[b] +
  // ctx - 1) / L), in workspace rows w + b.
  const int w0 = prefix[b] / L;
  const int n = ctx > 0 ? (prefix[b] + ctx - 1) / L - w0 + 1 : 0;
  const long long base = (long long)w0 + b;

  float m = -INFINITY;
  for (int i = tid; i < n; i += NT) m = fmaxf(m, p.ws_ml[((base + i) * p.Hq + h) * 2]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  float mstar = wmax[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) mstar = fmaxf(mstar, wmax[w]);
  const float mref = mstar == -INFINITY ? 0.f : mstar;

  const int sub = tid % TPR;   // float4 column group
  const int rg = tid / TPR;    // partial within a pass
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
#pragma unroll 4
  for (int i = rg; i < n; i += RPP) {
    const long long r = (base + i) * p.Hq + h;
    const float e = fast_exp2(p.ws_ml[r * 2] - mref);
    const f32x4 o4 = *reinterpret_cast<const f32x4*>(p.ws_o + r * D + sub * 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += e * o4[u];
    lsum += e * p.ws_ml[r * 2 + 1];
  }
  red[tid] = acc;
  if (sub == 0) lred[rg] = lsum;
  __syncthreads();
  if (rg == 0) {
#pragma unroll
    for (int g = 1; g < RPP; ++g) {
      const f32x4 x = red[g * TPR + sub];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += x[u];
      lsum += lred[g];
    }
    // A row with no keys has lsum == 0 and returns 0; NaN inputs stay NaN.
    typename Mfma<T>::v4 w;
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = (T)(lsum != 0.f ? acc[u] / lsum : 0.f);
    *reinterpret_cast<uint2*>(p.out + ((long long)b * p.Hq + h) * D + sub * 4) = __builtin_bit_cast(uint2, w);
  }
}

template <typename T, int D>
hipError_t launch_typed(const DecParams& p, hipStream_t stream) {
  const int units = p.Hkv * p.nhb;
  const dim3 grid(p.grid, (units + kWaves - 1) / kWaves);
  hipError_t e;
  if (p.B <= kInlinePlan) {
    hipLaunchKernelGGL((decode_split_kernel<T, D, kKStep, kStages, true>), grid, dim3(kWaves * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_split_kernel<T, D, kKStep, kStages, false>), grid, dim3(kWaves * 64), 0, stream, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(p.Hq, p.B), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int D, const DecParams& p, hipStream_t stream) {
  if (dtype == 0) return D == 64 ? launch_typed<_Float16, 64>(p, stream) : launch_typed<_Float16, 128>(p, stream);
  return D == 64 ? launch_typed<__bf16, 64>(p, stream) : launch_typed<__bf16, 128>(p, stream);
}

}  // namespace mea
