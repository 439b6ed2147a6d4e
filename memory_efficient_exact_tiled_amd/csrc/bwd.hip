// Tiled exact attention backward pass for gfx950 (MI355X).
//
// Method: the score matrix is recomputed block by block from q, k and the
// row log-sum-exp the forward stored, never read back from memory ("FlashAttention
// (2022): l'attenzione che non satura la memoria", paithon.it, section on the
// softmax that needs not see the whole row: the backward recomputes the scores
// on the fly instead of keeping them). With P = exp(s - lse) the gradients are
// the derivative of softmax(s) v, written with the softmax Jacobian:
//   dP = dO V^T,   dS = P * (dP - Delta),   Delta_i = sum_d dO_id O_id,
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
//
// Three kernels, no atomics (every output element has a single writer, so
// the result is deterministic):
//   * bwd_prep_kernel: Delta and lse * log2(e) per (row, query head) into the
//     caller's workspace (+inf for a row with no allowed key, so its P is 0);
//   * bwd_dq_kernel: the forward's shape. A work-group owns 128 query rows of
//     one (segment, query head), keeps Q and dO in registers and streams K/V
//     blocks of 64 keys through LDS (loaded two blocks ahead without a
//     block-sparse mask). S^T = K Q^T and dP^T = V dO^T leave one
//     query per lane, so lse and Delta are per-lane scalars; dS^T is rounded
//     to the input type and fed as the B operand of dQ^T += K^T dS^T, with K^T
//     read from the row-major K block by ds_read_b64_tr_b16;
//   * bwd_dkdv_kernel: the mirror image. A work-group owns 128 keys of one
//     (segment, KV head) (32 per wave, K and V in registers) and streams
//     64-query blocks of Q, dO, lse and Delta through LDS, for every query
//     head that shares the KV head (grouped-query attention sums over them
//     inside the work-group). S = Q K^T and dP = dO V^T leave one key per
//     lane; P and dS, rounded, are the B operands of dV^T += dO^T P and
//     dK^T += Q^T dS, with dO^T and Q^T from transpose reads.
// Masks (causal bottom-right, segment ends) and ALiBi come from indices as in
// the forward; blocks entirely above the diagonal are skipped. Under a
// block-sparse mask (BS = 1, 64 x 64 blocks) each work-group walks only the
// blocks some of its rows or keys need, and a wave skips the blocks that are
// off for its own rows or keys.
#include "common.hpp"
#include "launch.hpp"

namespace mea {

namespace {

constexpr int kWaves = 4;
// Waves per SIMD the register budget is tuned for: two at D=64; at D=128 the
// resident K, V and both accumulators need the whole register file of one.
template <int D>
constexpr int kBwdWpe = D == 64 ? 2 : 1;

// LDS tiles are row-major with rows padded to D + 8 elements: the 16-row
// ds_read_b128 operand reads are then conflict-free; the transpose reads
// conflict two ways on half their banks. An XOR swizzle of the 16-byte chunks
// removes those conflicts too, but measured slower on both kernels: the extra
// address arithmetic lands on the VALU, which bounds them.
template <int D>
__device__ __forceinline__ int lds_at(int row, int col) {
  return row * (D + 8) + col;
}

template <typename T>
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  typedef T T2 __attribute__((ext_vector_type(2)));
  const T2* x = reinterpret_cast<const T2*>(&a);
  const T2* y = reinterpret_cast<const T2*>(&b);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (__is_same(T, __bf16))
      acc = __builtin_amdgcn_fdot2_f32_bf16(x[i], y[i], acc, false);
    else
      acc = __builtin_amdgcn_fdot2(x[i], y[i], acc, false);
  }
  return acc;
}

// ---- Delta and lse in log2 units --------------------------------------------
// D/8 lanes per (row, head): each loads 16 bytes of O and dO. Items run in
// the lse layout ([batch][head][query], query fastest), so the lse reads and
// the Delta / lse2 writes of a wave are contiguous (the (row, head) order
// fetched twice the algorithmic bytes through those scattered 4-byte
// accesses).
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const BwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int IPB = 256 / CPR;   // items per block per sweep
  const int sub = threadIdx.x % CPR;
  const long long n_items = p.rows * p.Hq;
  for (long long item = (long long)blockIdx.x * IPB + threadIdx.x / CPR; item < n_items;
       item += (long long)gridDim.x * IPB) {
    const long long bh = item / p.M;
    const long long i = item - bh * p.M;
    const long long b = bh / p.Hq;
    const int h = (int)(bh - b * p.Hq);
    const long long e = (b * p.M + i) * p.q_rstride + (long long)h * D + sub * 8;
    float acc = dot8<T>(*reinterpret_cast<const uint4*>(p.out + e), *reinterpret_cast<const uint4*>(p.dout + e));
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (sub == 0) {
      const float l = p.lse[item];
      p.delta[item] = acc;
      p.lse2[item] = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
  }
}

// ---- dQ ------------------------------------------------------------------------
template <typename T, int D, int CS, int AL, int BS = 0>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kBwdWpe<D>, kBwdWpe<D>))) bwd_dq_kernel(const BwdParams p) {
  using MF = Mfma<T>;
  typedef typename MF::v8 v8;
  const bool ALIBI = AL == 2 ? (p.alibi != 0) : AL == 1;
  const bool CAUSAL = CS == 2 ? (p.causal != 0) : CS == 1;
  constexpr int QW = 32, BM = kWaves * QW, BN = 64;
  constexpr int TILE = BN * (D + 8);     // K and V blocks in LDS (lds_at)
  constexpr int CPR = D / 8, NLD = BN * CPR / (kWaves * 64);
  constexpr int DB = D / 32, DS = D / 16;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: masks branch, not select
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Launch order as in the forward: causal launches are tile index major
  // with the heads innermost, round-robin over the XCDs (dense: longest tiles
  // first over all (batch, head) pairs; packed: segment by segment); the
  // others give each XCD a contiguous range of (batch, head, tile).
  const int pid = blockIdx.x;
  int bh, t;
  if (CS == 1) {
    if (pid >= p.total_wg_q) return;
    const int nbh = p.varlen ? p.Hq : p.B * p.Hq;
    causal_order(pid, nbh, p.group, t, bh);
  } else {
    const int lid = (pid & 7) * p.wg_per_xcd_q + (pid >> 3);
    if (lid >= p.total_wg_q) return;
    bh = lid / p.n_qtiles;
    t = lid - bh * p.n_qtiles;
  }
  const int h = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = h / p.group;

  int M_s, N_s, tile;
  long long qoff, koff, st_off;
  if (!p.varlen) {
    M_s = p.M;
    N_s = p.N;
    tile = CAUSAL ? (p.n_qtiles - 1 - t) : t;
    qoff = (long long)b * p.q_bstride + (long long)h * D;
    koff = (long long)b * p.kv_bstride + (long long)g * D;
    st_off = ((long long)b * p.Hq + h) * p.M;
  } else {
    int rank, a0 = 0, a1 = 0, ntile = 0;
    const int s = find_segment_tile(p.seqstart_q, p.B, p.M, BM, t, rank, a0, a1, ntile);
    if (s >= p.B) return;
    tile = CAUSAL ? (ntile - 1 - rank) : rank;
    const int k0 = min(max(p.seqstart_k[s], 0), p.N);
    const int k1 = min(max(p.seqstart_k[s + 1], k0), p.N);
    M_s = a1 - a0;
    N_s = k1 - k0;
    qoff = (long long)a0 * p.q_rstride + (long long)h * D;
    koff = (long long)k0 * p.kv_rstride + (long long)g * D;
    st_off = (long long)h * p.M + a0;
  }

  const int i0 = tile * BM;
  const int off = N_s - M_s;
  int kend = N_s;
  if (CAUSAL) kend = min(N_s, i0 + BM + off);
  kend = max(kend, 0);
  const int ntiles = (kend + BN - 1) / BN;

  const int wq0 = i0 + wave * QW;
  const int wlast = min(wq0 + QW, M_s) - 1;
  int wkend = 0;
  if (wlast >= wq0) wkend = CAUSAL ? max(min(N_s, wlast + off + 1), 0) : N_s;

  const float c = p.scale_log2;
  const float slope = ALIBI ? p.slopes[h] * kLog2e : 0.f;
  const int qi = wq0 + l32;
  const bool qin = qi < M_s;
  const float lse2 = qin ? p.lse2[st_off + qi] : INFINITY;
  const float dlt = qin ? p.delta[st_off + qi] : 0.f;

  v8 qf[DS], df[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) {
    const long long e = qoff + (long long)qi * p.q_rstride + st * 16 + hi * 8;
    qf[st] = qin ? load_v8<T>(p.q + e) : zero_v8<T>();
    df[st] = qin ? load_v8<T>(p.dout + e) : zero_v8<T>();
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  uint4 kst[2][NLD], vst[2][NLD];
  const uint32_t row_bytes = (uint32_t)p.kv_rstride * 2u;
  uint32_t ld_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int ch = tid + i * (kWaves * 64);
    const int r = ch / CPR;
    ld_off[i] = (uint32_t)r * row_bytes + (uint32_t)(ch - r * CPR) * 16u;
  }
  // A block index outside [0, ntiles) gives an empty resource: the loads
  // are still issued but return zeros without touching memory.
  auto gload = [&](int kt, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const bool in = kt >= 0 && kt < ntiles;
    const long long o = in ? koff + (long long)kt * BN * p.kv_rstride : 0;
    const uint32_t bytes = in ? rows_bytes(N_s - kt * BN, row_bytes) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + o, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + o, bytes);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[i] = buf_load16(rk, ld_off[i]);
      vr[i] = buf_load16(rv, ld_off[i]);
    }
  };
  auto lstore = [&](int buf, const uint4 (&kr)[NLD], const uint4 (&vr)[NLD]) {
    uint16_t* ks = smem + buf * 2 * TILE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = tid + i * (kWaves * 64);
      const int r = ch / CPR;
      const int cc = (ch - r * CPR) * 8;
      *reinterpret_cast<uint4*>(ks + lds_at<D>(r, cc)) = kr[i];
      *reinterpret_cast<uint4*>(ks + TILE + lds_at<D>(r, cc)) = vr[i];
    }
  };

  const int g16 = lane >> 4;
  const int ll = lane & 15;
  const int trow = (g16 >> 1) * 4 + (ll >> 2);
  const int tcol = (g16 & 1) * 16 + 4 * (ll & 3);

  // Block-sparse skip list over key blocks (K tiles are the mask's key blocks).
  int qblo = 0, qbhi = -1, wqblk = -1;
  if (BS) {
    qblo = i0 >> 6;
    qbhi = min(i0 + BM, M_s) - 1;
    qbhi = qbhi >= i0 ? (qbhi >> 6) : qblo - 1;
    wqblk = (wq0 < M_s) ? (wq0 >> 6) : -1;
  }
  __shared__ uint64_t skip_bits[4];
  TileSkipList skip{skip_bits};
  auto tile_on = [&](int kt) {
    bool on = false;
    for (int r = qblo; r <= qbhi; ++r) on |= p.block_mask[(long long)r * p.nkb + kt] != 0;
    return on;
  };
  auto next_tile = [&](int kt) { return BS ? skip.next_on(kt, ntiles, tile_on) : kt; };
  // One key block on LDS buffer buf.
  auto compute = [&](const int kt, const int buf) {
    const int key_base = kt * BN;
    if (key_base >= wkend) return;
    if (BS && (wqblk < 0 || p.block_mask[(long long)wqblk * p.nkb + kt] == 0)) return;
    const uint16_t* Ks = smem + buf * 2 * TILE;
    const uint16_t* Vs = Ks + TILE;

    // S^T = K Q^T and dP^T = V dO^T (one query per lane, 32 keys per block)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = 0.f;
        dp[kb][r] = 0.f;
      }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const int a = lds_at<D>(kb * 32 + l32, st * 16 + hi * 8);
        s[kb] = MF::mma32(load_v8<T>(Ks + a), qf[st], s[kb]);
        dp[kb] = MF::mma32(load_v8<T>(Vs + a), df[st], dp[kb]);
      }
    __builtin_amdgcn_s_setprio(0);

    // P = 2^(s c + bias - lse2), dS = P (dP - Delta), rounded to T. The
    // exponent is formed in s: explicitly (bias, mask) only on blocks that
    // need it.
    const bool need_mask = (key_base + BN > N_s) || (CAUSAL && key_base + BN - 1 > wq0 + off);
    if (ALIBI || need_mask) {
      const int rel = key_base + hi * 4;
      const int lim_n = N_s - rel;
      const int lim_c = CAUSAL ? (qi + off - rel) : 0x7fffffff;
      const float dist0 = (float)(qi + off - rel);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = kb * 32 + (r >> 2) * 8 + (r & 3);
          float x = fmaf(s[kb][r], c, -lse2);
          if (ALIBI) x -= slope * fabsf(dist0 - (float)kr);
          s[kb][r] = (kr < lim_n && kr <= lim_c) ? x : -INFINITY;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], c, -lse2);
    }
    v8 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dsf[kb * 2 + (r >> 3)][r & 7] = (T)(fast_exp2(s[kb][r]) * (dp[kb][r] - dlt));

    // dQ^T += K^T dS^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int c0 = db * 32 + tcol;
        acc[db] = MF::mma32(lds_tr_x8<T>(Ks + lds_at<D>(tt * 16 + trow, c0), Ks + lds_at<D>(tt * 16 + trow + 8, c0)),
                            dsf[tt], acc[db]);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  int kt0 = next_tile(0), nkt = 0;
  if constexpr (BS == 0) {
    // Two blocks ahead, in two register sets, over pairs of blocks, as in the
    // forward (every path back to the loop head has issued both sets' loads).
    gload(kt0, kst[0], vst[0]);
    __builtin_amdgcn_sched_barrier(0);
    gload(kt0 + 1, kst[1], vst[1]);
    int kt = kt0;
    for (; kt + 1 < ntiles; kt += 2) {
      lstore(0, kst[0], vst[0]);
      __syncthreads();
      gload(kt + 2, kst[0], vst[0]);
      compute(kt, 0);
      lstore(1, kst[1], vst[1]);
      __syncthreads();
      gload(kt + 3, kst[1], vst[1]);
      compute(kt + 1, 1);
    }
    if (kt < ntiles) {
      lstore(0, kst[0], vst[0]);
      __syncthreads();
      compute(kt, 0);
    }
  } else {
    if (kt0 < ntiles) gload(kt0, kst[0], vst[0]);
    for (int kt = kt0, n = 0; kt < ntiles; kt = nkt, ++n) {
      const int buf = n & 1;
      nkt = next_tile(kt + 1);
      lstore(buf, kst[0], vst[0]);
      __syncthreads();
      if (nkt < ntiles) gload(nkt, kst[0], vst[0]);
      compute(kt, buf);
    }
  }

  // dQ is staged through the (then free) K/V buffers and stored as whole
  // rows, 16 bytes per lane, as in the forward's epilogue.
  __syncthreads();
  constexpr int OS = D + 8;
  static_assert(kWaves * QW * OS <= 2 * 2 * TILE, "the staged dQ must fit the K/V buffers");
  uint16_t* ob = smem + wave * (QW * OS);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      typename MF::v4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = (T)(acc[db][rg * 4 + u] * p.scale);
      *reinterpret_cast<uint2*>(ob + l32 * OS + db * 32 + rg * 8 + hi * 4) = __builtin_bit_cast(uint2, w);
    }
  __builtin_amdgcn_wave_barrier();   // each wave reads back only its own rows
  constexpr int CPO = D / 8;
#pragma unroll
  for (int i = 0; i < QW * CPO / 64; ++i) {
    const int ch = lane + i * 64;
    const int r = ch / CPO;
    const int cc = (ch - r * CPO) * 8;
    const int q = wq0 + r;
    const uint4 v = *reinterpret_cast<const uint4*>(ob + r * OS + cc);
    if (q < M_s) *reinterpret_cast<uint4*>(p.dq + qoff + (long long)q * p.q_rstride + cc) = v;
  }
}

// ---- dK, dV ----------------------------------------------------------------------
template <typename T, int D, int CS, int AL, int BS = 0>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kBwdWpe<D>, kBwdWpe<D>))) bwd_dkdv_kernel(const BwdParams p) {
  using MF = Mfma<T>;
  typedef typename MF::v8 v8;
  const bool ALIBI = AL == 2 ? (p.alibi != 0) : AL == 1;
  const bool CAUSAL = CS == 2 ? (p.causal != 0) : CS == 1;
  constexpr int KW = 32, BNK = kWaves * KW, BQ = 64;
  constexpr int TILE = BQ * (D + 8);     // Q and dO blocks in LDS (lds_at)
  constexpr int CPR = D / 8, NLD = BQ * CPR / (kWaves * 64);
  constexpr int DB = D / 32, DS = D / 16;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) float sstat[2][2][BQ];   // [buf][lse2, Delta][row]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: masks branch, not select
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Under a causal mask key tile 0 sees the most queries: causal launches
  // are tile index major with the KV heads innermost, round-robin over the
  // XCDs, as in the dQ kernel.
  const int pid = blockIdx.x;
  int bg, t;
  if (CS == 1) {
    if (pid >= p.total_wg_k) return;
    const int nbg = p.varlen ? p.Hkv : p.B * p.Hkv;
    causal_order(pid, nbg, 1, t, bg);
  } else {
    const int lid = (pid & 7) * p.wg_per_xcd_k + (pid >> 3);
    if (lid >= p.total_wg_k) return;
    bg = lid / p.n_ktiles;
    t = lid - bg * p.n_ktiles;
  }
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;

  int M_s, N_s, tile;
  long long qbase, koff, st_base;   // qbase: row 0 of the segment, head 0
  if (!p.varlen) {
    M_s = p.M;
    N_s = p.N;
    tile = t;
    qbase = (long long)b * p.q_bstride;
    koff = (long long)b * p.kv_bstride + (long long)g * D;
    st_base = (long long)b * p.Hq * p.M;
  } else {
    int rank, a0 = 0, a1 = 0, ntile = 0;
    const int s = find_segment_tile(p.seqstart_k, p.B, p.N, BNK, t, rank, a0, a1, ntile);
    if (s >= p.B) return;
    tile = rank;
    const int q0 = min(max(p.seqstart_q[s], 0), p.M);
    const int q1 = min(max(p.seqstart_q[s + 1], q0), p.M);
    M_s = q1 - q0;
    N_s = a1 - a0;
    qbase = (long long)q0 * p.q_rstride;
    koff = (long long)a0 * p.kv_rstride + (long long)g * D;
    st_base = q0;
  }
  // Statistics are [B][Hq][M] (packed: [Hq][M]); one head spans M rows.
  const float c = p.scale_log2;
  const int off = N_s - M_s;
  const int j0 = tile * BNK;
  const int wj0 = j0 + wave * KW;        // first key of this wave
  const int kj = wj0 + l32;              // this lane's key
  const bool kin = kj < N_s;

  // Queries that can see keys >= j0: i >= j0 - off under the causal mask.
  int qfirst = 0;
  if (CAUSAL) qfirst = max(j0 - off, 0);
  qfirst = (qfirst / BQ) * BQ;
  const int nqt = M_s > qfirst ? (M_s - qfirst + BQ - 1) / BQ : 0;
  const int niter = nqt * p.group;

  v8 kf[DS], vf[DS];
#pragma unroll
  for (int st = 0; st < DS; ++st) {
    const long long e = koff + (long long)kj * p.kv_rstride + st * 16 + hi * 8;
    kf[st] = kin ? load_v8<T>(p.k + e) : zero_v8<T>();
    vf[st] = kin ? load_v8<T>(p.v + e) : zero_v8<T>();
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[db][r] = 0.f;
      dva[db][r] = 0.f;
    }

  uint4 qst[NLD], dst[NLD];
  float stv = 0.f;
  const uint32_t row_bytes = (uint32_t)p.q_rstride * 2u;
  uint32_t ld_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int ch = tid + i * (kWaves * 64);
    const int r = ch / CPR;
    ld_off[i] = (uint32_t)r * row_bytes + (uint32_t)(ch - r * CPR) * 16u;
  }
  auto gload = [&](int it) {
    const int hh = it / nqt;
    const int qt = it - hh * nqt;
    const int h = g * p.group + hh;
    const int r0 = qfirst + qt * BQ;
    const uint32_t bytes = rows_bytes(M_s - r0, row_bytes);
    const long long base = qbase + (long long)r0 * p.q_rstride + (long long)h * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dout + base, bytes);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      qst[i] = buf_load16(rq, ld_off[i]);
      dst[i] = buf_load16(rd, ld_off[i]);
    }
    if (tid < 2 * BQ) {
      const int r = tid & (BQ - 1);
      const long long si = st_base + (long long)h * p.M + r0 + r;
      const bool in = r0 + r < M_s;
      stv = tid < BQ ? (in ? p.lse2[si] : INFINITY) : (in ? p.delta[si] : 0.f);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* qs = smem + buf * 2 * TILE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = tid + i * (kWaves * 64);
      const int r = ch / CPR;
      const int cc = (ch - r * CPR) * 8;
      *reinterpret_cast<uint4*>(qs + lds_at<D>(r, cc)) = qst[i];
      *reinterpret_cast<uint4*>(qs + TILE + lds_at<D>(r, cc)) = dst[i];
    }
    if (tid < 2 * BQ) sstat[buf][tid >> 6][tid & (BQ - 1)] = stv;
  };

  const int g16 = lane >> 4;
  const int ll = lane & 15;
  const int trow = (g16 >> 1) * 4 + (ll >> 2);
  const int tcol = (g16 & 1) * 16 + 4 * (ll & 3);
  const bool wave_has_keys = wj0 < N_s;

  // Block-sparse skip list over query tiles (64 rows = one mask row): a tile
  // is visited if either of the work-group's key blocks is on for it.
  const int kblo = j0 >> 6;
  const int kbhi = BS ? (min(j0 + BNK, N_s) - 1) >> 6 : kblo;
  const int wkblk = wj0 >> 6;
  __shared__ uint64_t skip_bits[4];
  TileSkipList skip{skip_bits};
  auto qtile_on = [&](int qt) {
    const long long qrow = (qfirst + qt * BQ) >> 6;
    bool on = false;
    for (int c = kblo; c <= kbhi; ++c) on |= p.block_mask[qrow * p.nkb + c] != 0;
    return on;
  };
  // Iterations run over (query head of the group, query tile); the skip list
  // is over query tiles and the same for every head.
  auto next_it = [&](int it) {
    if (BS) {
      while (it < niter) {
        const int hh = it / nqt;
        const int qt = skip.next_on(it - hh * nqt, nqt, qtile_on);
        if (qt < nqt) return hh * nqt + qt;
        it = (hh + 1) * nqt;
      }
    }
    return it;
  };
  int it0 = next_it(0), nit = 0;
  if (it0 < niter) gload(it0);
  for (int it = it0, n = 0; it < niter; it = nit, ++n) {
    const int buf = BS ? (n & 1) : (it & 1);
    nit = next_it(it + 1);
    lstore(buf);
    __syncthreads();
    const int hh = it / nqt;
    const int qt = it - hh * nqt;
    if (nit < niter) gload(nit);
    if (!wave_has_keys) continue;
    if (BS && p.block_mask[(long long)((qfirst + qt * BQ) >> 6) * p.nkb + wkblk] == 0) continue;

    const int h = g * p.group + hh;
    const float slope = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const uint16_t* Qs = smem + buf * 2 * TILE;
    const uint16_t* Os = Qs + TILE;
    const int r0 = qfirst + qt * BQ;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qb0 = r0 + qs * 32;      // first query of this 32-row block
      // Under the causal mask the block's last query sees keys <= qb0 + 31 + off.
      if (CAUSAL && qb0 + 31 + off < wj0) continue;
      if (qb0 >= M_s) continue;
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const int a = lds_at<D>(qs * 32 + l32, st * 16 + hi * 8);
        s = MF::mma32(load_v8<T>(Qs + a), kf[st], s);
        dp = MF::mma32(load_v8<T>(Os + a), vf[st], dp);
      }
      __builtin_amdgcn_s_setprio(0);

      // This lane's key kj; its 16 queries qb0 + rg*8 + hi*4 + u (r = rg*4 + u).
      // The exponent s c + bias - lse2 is formed in s; bias and mask only on
      // blocks that need them.
      const bool need_mask = CAUSAL && (qb0 + off < wj0 + KW - 1);
      f32x4 d4[4];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int rr = qs * 32 + rg * 8 + hi * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sstat[buf][0][rr]);
        d4[rg] = *reinterpret_cast<const f32x4*>(&sstat[buf][1][rr]);
#pragma unroll
        for (int u = 0; u < 4; ++u) s[rg * 4 + u] = fmaf(s[rg * 4 + u], c, -l4[u]);
      }
      if (ALIBI || need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dist = qb0 + (r >> 2) * 8 + hi * 4 + (r & 3) + off - kj;   // query position - key
          float x = s[r];
          if (ALIBI) x -= slope * fabsf((float)dist);
          s[r] = (!need_mask || dist >= 0) ? x : -INFINITY;
        }
      }
      v8 pf[2], dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(s[r]);
        pf[r >> 3][r & 7] = (T)pr;
        dsf[r >> 3][r & 7] = (T)(pr * (dp[r] - d4[r >> 2][r & 3]));
      }

      // dV^T += dO^T P,  dK^T += Q^T dS
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int r0 = qs * 32 + tt * 16 + trow, c0 = db * 32 + tcol;
          const int a0 = lds_at<D>(r0, c0), a1 = lds_at<D>(r0 + 8, c0);
          dva[db] = MF::mma32(lds_tr_x8<T>(Os + a0, Os + a1), pf[tt], dva[db]);
          dka[db] = MF::mma32(lds_tr_x8<T>(Qs + a0, Qs + a1), dsf[tt], dka[db]);
        }
      __builtin_amdgcn_s_setprio(0);
    }
  }

  // dK and dV are staged through the (then free) Q/dO buffers and stored as
  // whole rows, 16 bytes per lane, as in the forward's epilogue.
  __syncthreads();
  constexpr int OS = D + 8;
  static_assert(kWaves * 2 * KW * OS <= 2 * 2 * TILE, "the staged dK, dV must fit the Q/dO buffers");
  uint16_t* obk = smem + wave * (2 * KW * OS);
  uint16_t* obv = obk + KW * OS;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      typename MF::v4 wk, wv;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wk[u] = (T)(dka[db][rg * 4 + u] * p.scale);
        wv[u] = (T)dva[db][rg * 4 + u];
      }
      const int col = db * 32 + rg * 8 + hi * 4;
      *reinterpret_cast<uint2*>(obk + l32 * OS + col) = __builtin_bit_cast(uint2, wk);
      *reinterpret_cast<uint2*>(obv + l32 * OS + col) = __builtin_bit_cast(uint2, wv);
    }
  __builtin_amdgcn_wave_barrier();   // each wave reads back only its own rows
  constexpr int CPO = D / 8;
#pragma unroll
  for (int i = 0; i < KW * CPO / 64; ++i) {
    const int ch = lane + i * 64;
    const int r = ch / CPO;
    const int cc = (ch - r * CPO) * 8;
    const int kk = wj0 + r;
    const uint4 vk = *reinterpret_cast<const uint4*>(obk + r * OS + cc);
    const uint4 vv = *reinterpret_cast<const uint4*>(obv + r * OS + cc);
    if (kk < N_s) {
      const long long e = koff + (long long)kk * p.kv_rstride + cc;
      *reinterpret_cast<uint4*>(p.dk + e) = vk;
      *reinterpret_cast<uint4*>(p.dv + e) = vv;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const BwdParams& p, hipStream_t stream) {
  {
    constexpr int IPB = 256 / (D / 8);
    const long long items = p.rows * p.Hq;
    long long blocks = (items + IPB - 1) / IPB;
    if (blocks > 8192) blocks = 8192;
    if (blocks > 0) hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  const dim3 gq(p.wg_per_xcd_q * 8), gk(p.wg_per_xcd_k * 8), blk(kWaves * 64);
  if (p.block_mask != nullptr) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 2, 2, 1>), gk, blk, 0, stream, p);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, 2, 2, 1>), gq, blk, 0, stream, p);
  } else if (!p.causal) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 0, 2>), gk, blk, 0, stream, p);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, 0, 2>), gq, blk, 0, stream, p);
  } else if (p.alibi) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 1, 1>), gk, blk, 0, stream, p);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, 1, 1>), gq, blk, 0, stream, p);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 1, 0>), gk, blk, 0, stream, p);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, 1, 0>), gq, blk, 0, stream, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(int D, const BwdParams& p, hipStream_t stream) {
  return D == 64 ? launch_typed<T, 64>(p, stream) : launch_typed<T, 128>(p, stream);
}

}  // namespace

hipError_t launch_bwd(int dtype, int D, const BwdParams& p, hipStream_t stream) {
  return dtype == 0 ? launch_dtype<_Float16>(D, p, stream) : launch_dtype<__bf16>(D, p, stream);
}

}  // namespace mea
