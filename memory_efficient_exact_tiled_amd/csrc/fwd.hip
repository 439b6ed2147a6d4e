// Tiled exact attention forward pass for gfx950 (MI355X).
//
// Method: the score matrix is never formed. Each work-group keeps a block of
// queries on chip, streams K/V blocks of the same (segment, KV head) through
// LDS, and folds every block into an online softmax: a running row maximum
// and row sum, with the accumulated output rescaled when the maximum grows.
// Only the output (and optionally the row log-sum-exp) is written back.
// ("FlashAttention (2022): l'attenzione che non satura la memoria",
// paithon.it, sections on tiling and on the online softmax.)
//
// Work decomposition (one work-group = 4 waves = 256 threads):
//   * a work-group owns BM = 4 * 32 * QB query rows of one (batch or packed
//     segment, query head); wave w owns 32 * QB consecutive rows (QB = 2 for
//     dense D=64 when that still gives two work-groups per compute unit,
//     else 1); two waves (three at QB=1, D=64) share each SIMD, so one
//     wave's softmax overlaps another's matrix-core work; the P.V products
//     (and at D=64 the score products) run at raised wave priority;
//   * K/V blocks of BN = 64 keys are copied to LDS with buffer loads whose
//     resource ends at the segment's last key (rows past it read as zeros):
//     straight into LDS (LDS DMA) at D=128, through registers at D=64 (the
//     faster of the two for each); double buffered so one barrier per block
//     suffices, with the next block's copies in flight during the current
//     block's compute (two blocks ahead for the register staging of
//     launches without a block-sparse mask);
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q held in
//     registers for the whole kernel). With this orientation each lane holds
//     one query's scores for 32 of the 64 keys, so the row max needs a single
//     cross-lane step (v_permlane32_swap between lanes l and l^32) and the
//     row sum none until the end;
//   * P^T is rounded to the input type in registers; the row sum is taken
//     over those rounded values, two at a time with v_dot2_f32_{bf16,f16}
//     (so the normaliser matches the weights P.V actually uses), and P^T is
//     fed straight back as the B operand of O^T = V^T P^T; V^T comes from the
//     row-major V block with ds_read_b64_tr_b16, which matches the key order
//     P^T has in the score accumulators, so V is never transposed in memory;
//   * causal and block-diagonal masks are index predicates evaluated only on
//     blocks that straddle the diagonal or the segment end; blocks entirely
//     above the diagonal are never visited (per work-group) or computed (per
//     wave); ALiBi is computed from the indices. Under the causal mask the
//     ALiBi bias of a key block is linear in the key's index within the block,
//     so it is added by the score MFMA itself: one more k-step whose K column
//     is that index (exact in 16-bit floats) and whose Q column is slope /
//     scale split into two 16-bit parts; what is left per (row, block) is a
//     constant folded into the exponent's offset (heads with steep slopes,
//     where fp32 accumulation would blur the scores, add the bias per score);
//   * grouped-query attention: query head h reads KV head h / (Hq / Hkv) in
//     place; the heads sharing a KV head are adjacent in the launch order;
//   * block-sparse masks (64 x 64 blocks of query rows and keys): the
//     work-group walks only the key blocks at least one of its query blocks
//     has on (a skip list read from the mask), and a wave skips the blocks
//     that are off for its own query block.
//   * the normalised output is staged through LDS and stored as whole rows.
//
// Launch order: work-group p runs on XCD p % 8. Without a causal mask each
// XCD is given a contiguous range of logical work-groups, so the query tiles
// of one head (which read the same K/V) share that XCD's L2. Under a causal
// mask the tiles differ in length by up to the sequence length, and the
// launch is tile index major with the heads innermost (causal_order): dense
// launches issue every (batch, head)'s longest tile before any second-longest
// one (measured 13-31 % faster at M = 1024..4096 than per-head order with XCD
// ranges); packed launches go segment by segment, each segment's tiles
// longest first (+5-8 % on 8 segments of 64..2048 tokens; a strict
// longest-first order over all segments measured slower). The query heads of
// one KV head are pinned to one XCD, so under grouped-query attention each
// K/V byte is fetched once (the packed 8-segment GQA batch: 154 -> 74 MB).
// Packed work-groups find their segment by a binary search over the
// segments' tile ranges (find_segment_tile), whatever the segment count.
#include "common.hpp"
#include "launch.hpp"

namespace mea {

namespace {

constexpr int kWaves = 4;
constexpr int kBN = 64;

// Query rows per wave = 32 * QB. Dense D=64 uses QB=2 (each K/V fragment read
// from LDS feeds two query blocks); under a causal mask and at D=128 QB=1,
// which halves the rows a diagonal block masks off and keeps a wave within
// the register budget of several waves per SIMD.
template <int D, int QB_, int GQ = 0>
struct FwdShape {
  static constexpr int QB = QB_;
  static constexpr int QW = 32 * QB;            // query rows per wave
  // Query rows per work-group: GQ = 1 (grouped-query work-groups) gives the
  // four waves the same rows of four query heads sharing one KV head.
  static constexpr int BM = GQ ? QW : kWaves * QW;
  // Padded LDS row strides (elements). K rows are read 16 rows x 16 bytes at
  // a time: a stride of 4 banks mod 64 keeps those 16 rows on distinct banks.
  // The transpose read of V covers 4 rows x 2 chunks of 32 bytes per 32
  // lanes: a stride of 16 or 48 banks mod 64 puts the 8 chunks on 8 disjoint
  // bank ranges (D + 16 left two of them on the same banks; D + 32 measured
  // 1-2 % faster).
  static constexpr int LDSK = D + 8;
  static constexpr int LDS = D + 32;            // V
  static constexpr int TILEK = kBN * LDSK;
  static constexpr int TILE = TILEK + kBN * LDS;  // elements per buffer: the K block, then the V block
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int NLD = kBN * CPR / (kWaves * 64);  // chunks per thread per tensor
  // Waves per SIMD the register budget is tuned for.
  static constexpr int WPE = (D == 64 && QB == 1) ? 3 : 2;
};

// CS and AL select how the causal and ALiBi flags are known: 0 = off, 1 = on
// (compile-time constants), 2 = read from p at run time. Causal launches
// specialise both; the dense launch reads both at run time, which the
// compiler schedules better than the fully specialised form. BS = 1 reads a
// block-sparse mask (p.block_mask). GQ = 1 (causal launches whose KV heads
// serve a multiple of 4 query heads): a work-group takes 32 query rows of 4
// query heads that share one KV head, one head per wave, so its waves stop at
// the same diagonal and one LDS copy of each K/V block serves 4 heads.
template <typename T, int D, int QB_, int CS, int AL, int BS = 0, int GQ = 0>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(FwdShape<D, QB_>::WPE, FwdShape<D, QB_>::WPE))) fwd_kernel(const FwdParams p) {
  using S = FwdShape<D, QB_, GQ>;
  static_assert(!GQ || (CS == 1 && BS == 0 && QB_ == 1), "grouped-query work-groups are causal, QB = 1");
  using MF = Mfma<T>;
  const bool ALIBI = AL == 2 ? (p.alibi != 0) : AL == 1;
  const bool CAUSAL = CS == 2 ? (p.causal != 0) : CS == 1;
  typedef typename MF::v8 v8;
  constexpr int QB = S::QB, QW = S::QW, BM = S::BM, LDS = S::LDS, LDSK = S::LDSK, TILE = S::TILE, TILEK = S::TILEK;
  constexpr int CPR = S::CPR, NLD = S::NLD;
  constexpr int DB = D / 32;   // 32-wide output column blocks
  constexpr int DS = D / 16;   // k-steps of the score product
  constexpr bool kFastSum = D == 64 && BS == 0 && ((QB_ == 1 && CS == 1 && AL == 0) || QB_ == 2);

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Under a causal mask the wave index is made visibly wave-uniform, so the
  // per-wave mask decisions compile to scalar branches (measured faster
  // there; the dense D=64 launch schedules better without it). At D=128 it
  // also keeps the LDS DMA copies, whose LDS address (M0) and count depend
  // on the wave, out of divergent branches and lane loops.
  const int wave = (CS == 1 || D == 128) ? __builtin_amdgcn_readfirstlane(tid >> 6) : (tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work decomposition -------------------------------------------------
  const int pid = blockIdx.x;
  int bh, t;
  if (CS == 1) {
    // Causal: tile index major, heads innermost, dealt round-robin over the
    // XCDs. Dense: every (batch, head)'s longest tile is issued before any
    // second-longest one. Packed: segment by segment, each segment's tiles
    // longest first, for all heads at once.
    if (pid >= p.total_wg) return;
    const int nbh = (p.varlen ? p.Hq : p.B * p.Hq) / (GQ ? kWaves : 1);
    causal_order(pid, nbh, GQ ? p.group / kWaves : p.group, t, bh);
  } else {
    const int lid = (pid & 7) * p.wg_per_xcd + (pid >> 3);
    if (lid >= p.total_wg) return;
    bh = lid / p.n_qtiles;
    t = lid - bh * p.n_qtiles;
  }
  // GQ: bh counts groups of 4 consecutive query heads (one KV head's, since
  // the group size is a multiple of 4); wave w takes the w-th of them.
  const int hq = GQ ? p.Hq / kWaves : p.Hq;
  const int h = GQ ? (bh % hq) * kWaves + wave : bh % p.Hq;
  const int b = bh / hq;
  const int g = h / p.group;

  int M_s, N_s, tile;
  long long qoff, koff, lse_off;
  if (!p.varlen) {
    M_s = p.M;
    N_s = p.kv_lens != nullptr ? min(max(p.kv_lens[b], 0), p.N) : p.N;
    tile = CAUSAL ? (p.n_qtiles - 1 - t) : t;
    qoff = (long long)b * p.q_bstride + (long long)h * D;
    koff = (long long)b * p.kv_bstride + (long long)g * D;
    lse_off = ((long long)b * p.Hq + h) * p.M;
  } else {
    // Locate (segment, tile) by a binary search over the segment boundaries,
    // which are clamped to the tensor extents so no row index can leave them.
    int in = 0, a0 = 0, a1 = 0, ntile = 0;
    const int s = find_segment_tile(p.seqstart_q, p.B, p.M, BM, t, in, a0, a1, ntile);
    if (s >= p.B) return;
    tile = CAUSAL ? (ntile - 1 - in) : in;
    const int* sk = p.seqstart_k;
    const int k0 = min(max(sk[s], 0), p.N);
    const int k1 = min(max(sk[s + 1], k0), p.N);
    M_s = a1 - a0;
    N_s = k1 - k0;
    qoff = (long long)a0 * p.q_rstride + (long long)h * D;
    koff = (long long)k0 * p.kv_rstride + (long long)g * D;
    lse_off = (long long)h * p.M + a0;
  }

  const int i0 = tile * BM;            // first query row of the work-group (segment-local)
  const int off = N_s - M_s;           // bottom-right causal alignment
  int kend = N_s;
  if (CAUSAL) kend = min(N_s, i0 + BM + off);
  kend = max(kend, 0);
  const int ntiles = (kend + kBN - 1) / kBN;

  const int wq0 = i0 + (GQ ? 0 : wave * QW);   // first query row of this wave
  const int wlast = min(wq0 + QW, M_s) - 1;
  int wkend = 0;                       // keys this wave needs
  if (wlast >= wq0) wkend = CAUSAL ? max(min(N_s, wlast + off + 1), 0) : N_s;

  const float c = p.scale_log2;
  const float slope = ALIBI ? p.slopes[h] * kLog2e : 0.f;

  // ---- Q fragments (B operand: column = query, k = head dim) ---------------
  v8 qf[QB][DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wq0 + qb * 32 + l32;
#pragma unroll
    for (int st = 0; st < DS; ++st)
      qf[qb][st] = (row < M_s) ? load_v8<T>(p.q + qoff + (long long)row * p.q_rstride + st * 16 + hi * 8)
                               : zero_v8<T>();
  }

  // Causal ALiBi through the MFMA (see the header): A rows = keys of the
  // block (index kb * 32 + l32 in lanes with hi = 0, twice), B = slope / scale
  // as hi + lo parts in lanes with hi = 0; zeros elsewhere.
  v8 kx[2], qx;
  // The fold is exact to fp32 accumulation: the bias term kl * r rounds with
  // the score at about 63 * |slope| * 2^-24 (log2 units), independent of the
  // scale. Heads with |slope| > 16 (log2 units) take the explicit bias instead.
  const bool fold = (CS == 1 && AL == 1) && fabsf(slope) <= 16.f;
  if constexpr (CS == 1 && AL == 1) {
    // r = slope / scale (both in log2 units). fp16 holds at most 65504, so a
    // power of two 2^e moves from the Q column to the K column (index * 2^e
    // stays exact for index < 64 and e <= 10).
    const float r = fold ? slope / c : 0.f;
    int e = 0;
    if constexpr (__is_same(T, _Float16)) e = min(max(ilogbf(fabsf(r)) - 14, 0), 10);
    const float rs = ldexpf(r, -e);
    const T rh = (T)rs;
    const T rl = (T)(rs - (float)rh);
    qx = zero_v8<T>();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kx[kb] = zero_v8<T>();
    if (hi == 0) {
      qx[0] = rh;
      qx[1] = rl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        kx[kb][0] = (T)ldexpf((float)(kb * 32 + l32), e);
        kx[kb][1] = kx[kb][0];
      }
    }
  }

  f32x16 o[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
  }

  // ---- K/V staging ---------------------------------------------------------
  // D=64: K/V staging through registers (HBM -> VGPRs -> LDS), which measured
  // faster there than the LDS DMA the D=128 kernels use.
  constexpr bool kDma = D == 128;
  uint4 kst[2][NLD], vst[2][NLD];
  const uint32_t row_bytes = (uint32_t)p.kv_rstride * 2u;
  uint32_t ld_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int ch = tid + i * (kWaves * 64);
    const int r = ch / CPR;
    ld_off[i] = (uint32_t)r * row_bytes + (uint32_t)(ch - r * CPR) * 16u;
  }
  // A block index outside [0, ntiles) gives an empty resource: the loads are
  // still issued (so every iteration has the same loads in flight) but
  // return zeros without touching memory.
  auto gload = [&](int kt, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) {
    const bool in = kt >= 0 && kt < ntiles;
    const long long o = in ? koff + (long long)kt * kBN * p.kv_rstride : 0;
    const uint32_t bytes = in ? rows_bytes(N_s - kt * kBN, row_bytes) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + o, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + o, bytes);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[i] = buf_load16(rk, ld_off[i]);
      vr[i] = buf_load16(rv, ld_off[i]);
    }
  };
  auto lstore = [&](int buf, const uint4 (&kr)[NLD], const uint4 (&vr)[NLD]) {
    uint16_t* ks = smem + buf * TILE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int ch = tid + i * (kWaves * 64);
      const int r = ch / CPR;
      const int cc = (ch - r * CPR) * 8;
      *reinterpret_cast<uint4*>(ks + r * LDSK + cc) = kr[i];
      *reinterpret_cast<uint4*>(ks + TILEK + r * LDS + cc) = vr[i];
    }
  };

  // D=128: K/V staging by LDS DMA (buffer_load ... lds). One wave-instruction
  // writes 64 consecutive 16-byte chunks of a padded block, lane i the i-th;
  // wave w issues instructions w, w + 4, ... of the K block (LDSK / 8 chunks
  // per row) and of the V block (LDS / 8). Pad chunks re-load their row's
  // first chunk (an in-range address). Rows past the segment end read as
  // zeros (buffer range).
  constexpr int KCH = LDSK / 8, VCH = LDS / 8;
  constexpr int NKI = kBN * KCH / 64, NVI = kBN * VCH / 64;
  constexpr int MKI = (NKI + kWaves - 1) / kWaves, MVI = (NVI + kWaves - 1) / kWaves;
  static_assert(kBN * KCH % 64 == 0 && kBN * VCH % 64 == 0, "blocks must be whole wave-instructions");
  uint32_t koffs[MKI], voffs[MVI];
#pragma unroll
  for (int i = 0; i < MKI; ++i) {
    const int q = (wave + i * kWaves) * 64 + lane;
    const int row = q / KCH, cch = q - row * KCH;
    koffs[i] = (uint32_t)row * row_bytes + (cch < D / 8 ? (uint32_t)cch * 16u : 0u);
  }
#pragma unroll
  for (int i = 0; i < MVI; ++i) {
    const int q = (wave + i * kWaves) * 64 + lane;
    const int row = q / VCH, cch = q - row * VCH;
    voffs[i] = (uint32_t)row * row_bytes + (cch < D / 8 ? (uint32_t)cch * 16u : 0u);
  }
  auto dma = [&](int kt, int buf) {
    const uint32_t bytes = rows_bytes(N_s - kt * kBN, row_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + koff + (long long)kt * kBN * p.kv_rstride, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + koff + (long long)kt * kBN * p.kv_rstride, bytes);
    uint16_t* kdst = smem + buf * TILE;
    uint16_t* vdst = kdst + TILEK;
#pragma unroll
    for (int i = 0; i < MKI; ++i) {
      const int j = wave + i * kWaves;
      if (j < NKI)
        lds_dma16(rk, kdst + j * 512, koffs[i]);
    }
#pragma unroll
    for (int i = 0; i < MVI; ++i) {
      const int j = wave + i * kWaves;
      if (j < NVI)
        lds_dma16(rv, vdst + j * 512, voffs[i]);
    }
  };

  // Lane coordinates of the V^T transpose reads.
  const int g16 = lane >> 4;
  const int ll = lane & 15;
  const int vrow = (g16 >> 1) * 4 + (ll >> 2);
  const int vcol = (g16 & 1) * 16 + 4 * (ll & 3);

  // Under ALiBi the bias grows towards the diagonal, so blocks are walked
  // from the last one back to the first: the running maximum is then set by
  // the first block and the lazy rescale almost never fires. Otherwise
  // blocks go in order, so the work-groups of a head read the same K/V
  // blocks at about the same time (L2 reuse).
  // (Block-sparse launches walk forward: their skip list is over key blocks.)
  const bool rev = CS == 1 && AL == 1 && BS == 0;
  // Block-sparse skip list: key block kt is visited if any query block of the
  // work-group has it on (the mask row of query block r is p.block_mask + r *
  // p.nkb; K tiles are exactly the mask's key blocks).
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
  auto next_tile = [&](int it) { return BS ? skip.next_on(it, ntiles, tile_on) : it; };
  int it0 = next_tile(0), nit = 0;
  constexpr bool k2 = !kDma && BS == 0;
  if constexpr (k2) {
    // Blocks it0 and it0 + 1 into the two staging sets, in that order.
    gload(it0 < ntiles ? (rev ? ntiles - 1 - it0 : it0) : -1, kst[0], vst[0]);
    __builtin_amdgcn_sched_barrier(0);
    gload(it0 + 1 < ntiles ? (rev ? ntiles - 2 - it0 : it0 + 1) : -1, kst[1], vst[1]);
  } else if (it0 < ntiles) {
    if constexpr (kDma) dma(rev ? ntiles - 1 - it0 : it0, 0);
    else gload(rev ? ntiles - 1 - it0 : it0, kst[0], vst[0]);
  }
  // One key block: scores, softmax update, P.V, on LDS buffer buf.
  auto compute = [&](const int kt, const int buf) {
    const int key_base = kt * kBN;
    if (key_base >= wkend) return;   // the whole block is masked for this wave
    if (BS && (wqblk < 0 || p.block_mask[(long long)wqblk * p.nkb + kt] == 0)) return;
    const uint16_t* Ks = smem + buf * TILE;
    const uint16_t* Vs = Ks + TILEK;

    // S^T = K Q^T
    f32x16 s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
    // Raised priority for the score products at D=64 only: at D=128 it
    // measured 2-3 % slower than raising it for the P.V products alone.
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int st = 0; st < DS; ++st) {
        const v8 kf = load_v8<T>(Ks + (kb * 32 + l32) * LDSK + st * 16 + hi * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = MF::mma32(kf, qf[qb][st], s[qb][kb]);
      }
      if constexpr (CS == 1 && AL == 1) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = MF::mma32(kx[kb], qx, s[qb][kb]);
      }
    }
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);

    const bool need_mask = (key_base + kBN > N_s) || (CAUSAL && key_base + kBN - 1 > wq0 + off);
    typename MF::v8 pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = wq0 + qb * 32 + l32;
      float cc = c, bb = 0.f;   // exponent of P = s * cc + bb - (running max)
      if constexpr (CS == 1 && AL == 1) {
        // s already holds slope/scale * (key - key_base); the rest of the bias,
        // -slope * (query position - key_base), is constant per row and block.
        // Under the causal rule every allowed key is inside the segment.
        bb = -slope * (float)(qi + off - key_base);
        if (need_mask || !fold) {
          const int lim_c = qi + off - key_base - hi * 4;   // kr <= lim_c : causal
          // Unfolded, the bias comes from the exact distance (query position -
          // key = lim_c - kr, exact as a float difference of integers below
          // 2^24): a product of the large per-block part and a separate
          // in-block part would not cancel exactly at steep slopes.
          const float dl = (float)lim_c;
          const float sl = fold ? 0.f : slope;
          const float b0 = fold ? bb : 0.f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kr = kb * 32 + (r >> 2) * 8 + (r & 3);
              const float bias = fmaf(sl, (float)kr - dl, b0);
              s[qb][kb][r] = (!need_mask || kr <= lim_c) ? fmaf(s[qb][kb][r], c, bias) : -INFINITY;
            }
          cc = 1.f;
          bb = 0.f;
        }
      } else if (ALIBI || need_mask) {
        // Explicit scores in log2 units: scale, ALiBi from indices, mask.
        const int rel = key_base + hi * 4;           // key = rel + kr
        const int lim_n = N_s - rel;                 // kr <  lim_n : inside the segment
        const int lim_c = CAUSAL ? (qi + off - rel) : 0x7fffffff;  // kr <= lim_c : causal
        const float dist0 = (float)(qi + off - rel); // query position - key, at kr = 0
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = kb * 32 + (r >> 2) * 8 + (r & 3);
            float x = s[qb][kb][r] * c;
            if (ALIBI) x -= slope * fabsf(dist0 - (float)kr);
            // Under a compile-time causal mask every allowed key of a real row
            // is inside the segment, so only the causal bound is tested.
            x = ((CS == 1 || kr < lim_n) && kr <= lim_c) ? x : -INFINITY;
            s[qb][kb][r] = x;
          }
        cc = 1.f;
      }
      // At D=64 without ALiBi or a block mask (the causal QB=1 kernel, and
      // the dense QB=2 kernel when its ALiBi flag is off), P is first tried
      // with the running max as the offset, before this
      // block's max is known. If every rounded P of the lane is below 2^7
      // (lane row sum below 128; NaN and inf fail the test), no score is
      // more than the rescale threshold above the running max, so the full
      // step below would keep that max and produce this same P. Only the
      // order of the row-sum additions differs. The full step runs directly
      // while a row has no running max yet (its first block), and when the
      // test fails. Measured 3-5 % faster on the causal and 2.4 % on the
      // dense B=4 M=4096 launch; slower at D=128 and with ALiBi, whose
      // rising bias fails the test on most blocks.
      float psum = 0.f;
      bool full = true;
      if (kFastSum && !ALIBI && __all(m_run[qb] > -INFINITY)) {
        const float nb = bb - m_run[qb];
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
          for (int u = 0; u < 8; ++u) pf[qb][tt][u] = (T)fast_exp2(fmaf(s[qb][tt >> 1][(tt & 1) * 8 + u], cc, nb));
          typedef T T2 __attribute__((ext_vector_type(2)));
          const T2 one2 = {(T)1.f, (T)1.f};
#pragma unroll
          for (int u = 0; u < 8; u += 2) {
            const T2 pp = {pf[qb][tt][u], pf[qb][tt][u + 1]};
            float& acc = (tt & 1) ? ps1 : ps0;
            if constexpr (sizeof(T) == 2 && __is_same(T, __bf16))
              acc = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, acc, false);
            else
              acc = __builtin_amdgcn_fdot2(pp, one2, acc, false);
          }
        }
        psum = ps0 + ps1;
        full = !__all(psum < 128.f);
      }
      if (full) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        {
          const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
        }
        const float mt = fmaf(mx, cc, bb);
        if (__any(mt > m_run[qb] + kRescaleThreshold)) {
          const float mn = fmaxf(m_run[qb], mt);
          const float alpha = fast_exp2(m_run[qb] - (mn == -INFINITY ? 0.f : mn));
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
          m_run[qb] = mn;
        }
        const float mu = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[qb][kb][r] = fast_exp2(fmaf(s[qb][kb][r], cc, bb - mu));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int u = 0; u < 8; ++u) pf[qb][tt][u] = (T)s[qb][tt >> 1][(tt & 1) * 8 + u];
        // Row sum of the rounded P (the values P.V uses), two at a time.
        psum = 0.f;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          typedef T T2 __attribute__((ext_vector_type(2)));
          const T2 one2 = {(T)1.f, (T)1.f};
#pragma unroll
          for (int u = 0; u < 8; u += 2) {
            const T2 pp = {pf[qb][tt][u], pf[qb][tt][u + 1]};
            if constexpr (sizeof(T) == 2 && __is_same(T, __bf16))
              psum = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, psum, false);
            else
              psum = __builtin_amdgcn_fdot2(pp, one2, psum, false);
          }
        }
      }
      l_run[qb] += psum;
    }

    // O^T += V^T P^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const uint16_t* a0 = Vs + (tt * 16 + vrow) * LDS + db * 32 + vcol;
        const v8 vf = lds_tr_x8<T>(a0, a0 + 8 * LDS);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = MF::mma32(vf, pf[qb][tt], o[qb][db]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto tile_at = [&](int i) { return rev ? ntiles - 1 - i : i; };
  // Register staging without a block-sparse skip list prefetches two blocks
  // ahead: block i + 2 is loaded into the staging set block i just left, so
  // a load has two blocks of compute to arrive. In-kernel timestamps showed
  // loads issued one block ahead still arriving late (their wait was a fifth
  // of a block); two ahead measured 3 % faster on the dense B=4 M=4096 launch.
  if constexpr (k2) {
    // Blocks in pairs (set 0, then set 1), so every path back to the loop
    // head has issued both sets' loads; an odd last block runs after it.
    int it = it0;
    for (; it + 1 < ntiles; it += 2) {
      lstore(0, kst[0], vst[0]);
      __syncthreads();
      gload(it + 2 < ntiles ? tile_at(it + 2) : -1, kst[0], vst[0]);
      compute(tile_at(it), 0);
      lstore(1, kst[1], vst[1]);
      __syncthreads();
      gload(it + 3 < ntiles ? tile_at(it + 3) : -1, kst[1], vst[1]);
      compute(tile_at(it + 1), 1);
    }
    if (it < ntiles) {
      lstore(0, kst[0], vst[0]);
      __syncthreads();
      compute(tile_at(it), 0);
    }
  } else {
    for (int it = it0, n = 0; it < ntiles; it = nit, ++n) {
      const int kt = tile_at(it);
      const int buf = n & 1;
      nit = next_tile(it + 1);
      if constexpr (kDma) {
        __builtin_amdgcn_s_waitcnt(0);   // this wave's block copies have landed in LDS
        __syncthreads();                 // ... and every wave's
        if (nit < ntiles) dma(tile_at(nit), buf ^ 1);
      } else {
        lstore(buf, kst[0], vst[0]);
        __syncthreads();
        if (nit < ntiles) gload(tile_at(nit), kst[0], vst[0]);
      }
      compute(kt, buf);
    }
  }

  // ---- epilogue --------------------------------------------------------------
  // The normalised tile is staged through LDS (the K/V buffers, free once
  // every wave has left the loop) so that the stores to HBM are whole rows,
  // 16 bytes per lane, instead of 8-byte pieces of 32 rows per instruction:
  // the same bytes, half the store instructions (measured 1-5 % faster, most
  // on packed batches of short tiles).
  __syncthreads();
  constexpr int OS = D + 8;   // staged row stride (elements)
  static_assert(kWaves * QW * OS <= 2 * TILE, "the staged output must fit the K/V buffers");
  uint16_t* ob = smem + wave * (QW * OS);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32);
    const int qi = wq0 + qb * 32 + l32;
    const float inv = lt != 0.f ? 1.f / lt : 0.f;   // no allowed key -> 0; NaN stays NaN
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        typename MF::v4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = (T)(o[qb][db][rg * 4 + u] * inv);
        *reinterpret_cast<uint2*>(ob + (qb * 32 + l32) * OS + db * 32 + rg * 8 + hi * 4) = __builtin_bit_cast(uint2, w);
      }
    if (qi < M_s && p.lse != nullptr && hi == 0)
      p.lse[lse_off + qi] = lt != 0.f ? (m_run[qb] + __log2f(lt)) * kLn2 : -INFINITY;
  }
  __builtin_amdgcn_wave_barrier();   // each wave reads back only its own rows
  constexpr int CPO = D / 8;         // 16-byte chunks per output row
#pragma unroll
  for (int i = 0; i < QW * CPO / 64; ++i) {
    const int ch = lane + i * 64;
    const int r = ch / CPO;
    const int cc = (ch - r * CPO) * 8;
    const int qi = wq0 + r;
    const uint4 v = *reinterpret_cast<const uint4*>(ob + r * OS + cc);
    if (qi < M_s) *reinterpret_cast<uint4*>(p.out + qoff + (long long)qi * p.q_rstride + cc) = v;
  }
}

template <typename T, int D, int QB, int CS, int AL, int BS, int GQ = 0>
hipError_t launch_k(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<T, D, QB, CS, AL, BS, GQ>), dim3(p.wg_per_xcd * 8), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

// Launch shapes (fwd_block_m must agree): the dense D=64 launch runs QB=2
// (256-row work-groups) when that still gives every compute unit two
// work-groups (p.wide, set by the host), else QB=1; causal and block-sparse
// launches run QB=1 (128-row work-groups), which halves the rows a diagonal
// block masks off and keeps the skip list of a work-group close to what each
// wave needs. Causal launches, block-sparse ones included, take the
// kernels specialised for the causal mask (measured 7 % faster than reading
// the flag at run time on the block-sparse window pattern).
template <typename T, int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  if (p.block_mask != nullptr) {
    if (p.causal) return p.alibi ? launch_k<T, D, 1, 1, 1, 1>(p, stream) : launch_k<T, D, 1, 1, 0, 1>(p, stream);
    return launch_k<T, D, 1, 2, 2, 1>(p, stream);
  }
  if (!p.causal) {
    if constexpr (D == 64) {
      if (p.wide) return launch_k<T, D, 2, 2, 2, 0>(p, stream);
    }
    return launch_k<T, D, 1, 2, 2, 0>(p, stream);
  }
  if (p.gq) return p.alibi ? launch_k<T, D, 1, 1, 1, 0, 1>(p, stream) : launch_k<T, D, 1, 1, 0, 0, 1>(p, stream);
  return p.alibi ? launch_k<T, D, 1, 1, 1, 0>(p, stream) : launch_k<T, D, 1, 1, 0, 0>(p, stream);
}

template <typename T>
hipError_t launch_dtype(int D, const FwdParams& p, hipStream_t stream) {
  return D == 64 ? launch_d<T, 64>(p, stream) : launch_d<T, 128>(p, stream);
}

}  // namespace

int fwd_block_m(int D, bool causal, bool block_sparse, bool wide, bool gq) {
  if (gq) return FwdShape<64, 1, 1>::BM;
  if (D == 64) return (wide && !causal && !block_sparse) ? FwdShape<64, 2>::BM : FwdShape<64, 1>::BM;
  return FwdShape<128, 1>::BM;
}

hipError_t launch_fwd(int dtype, int D, const FwdParams& p, hipStream_t stream) {
  return dtype == 0 ? launch_dtype<_Float16>(D, p, stream) : launch_dtype<__bf16>(D, p, stream);
}

}  // namespace mea
