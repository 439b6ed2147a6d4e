/*
 * mea.h - memory-efficient exact attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmea.so. Every entry point takes plain pointers and sizes; no
 * torch or HIP types appear in the signatures (a stream is passed as the
 * hipStream_t value cast to void*, NULL meaning the null stream).
 *
 * Conventions shared by all entry points
 *   - Tensor pointers are DEVICE pointers, owned by the caller; the library
 *     never allocates, frees or keeps device memory, and keeps no state
 *     between calls.
 *   - Work is enqueued asynchronously on `stream`; no call synchronises.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error the call returns a nonzero status and launches nothing. Contents
 *     of device arrays (seqstart_*, ctx_lens) cannot be checked without a
 *     sync; they are a documented precondition, and the kernels clamp every
 *     row index they derive from them to the tensor bounds, so malformed
 *     contents give wrong numbers, never out-of-bounds accesses.
 *   - fp16/bf16 tensors are contiguous, row-major, element strides as stated.
 *   - Accumulation is fp32; P (the softmax numerators) is rounded to the
 *     input type before the P.V product; outputs are rounded to nearest even.
 *   - Stateless and reentrant: calls from several host threads are safe.
 */
#ifndef MEA_H
#define MEA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MEA_OK 0
#define MEA_EINVAL 1       /* null pointer, non-positive size, inconsistent heads, bad scale */
#define MEA_EUNSUPPORTED 2 /* (dtype, head dim) combination without a kernel */
#define MEA_EWORKSPACE 3   /* workspace missing, too small or not 256-byte aligned */
#define MEA_EHIP 4         /* the HIP runtime rejected a launch */
#define MEA_ESCRATCH 5     /* mea_decode_noalloc: the step needs more than its static scratch */

/* Element types of q, k, v, caches and outputs. */
#define MEA_FP16 0
#define MEA_BF16 1

/* bias_kind bit flags. */
#define MEA_MASK_CAUSAL 1u    /* query i of a segment with M queries, N keys sees key j iff j <= i + N - M */
#define MEA_MASK_BLOCKDIAG 2u /* packed segments; each query segment sees only its own key segment */
#define MEA_BIAS_ALIBI 4u     /* adds -slope[h] * |(i + N - M) - j| to the scaled score */

/*
 * mea_fwd - exact scaled-dot-product attention forward pass that never forms
 * the M x N score matrix: Q tiles stay on chip while K/V tiles stream through
 * LDS and an online softmax (running row max and row sum, rescaled as each
 * new block arrives) accumulates the output.
 *
 * The method: "FlashAttention (2022): l'attenzione che non satura la
 * memoria" (paithon.it), sections on tiling ("L'idea: non scrivere mai la
 * matrice intera") and on the online softmax; its API shape and variants
 * (causal lower-triangular mask, packed variable-length batches under a
 * block-diagonal mask, grouped-query attention, ALiBi): "Come costruire
 * Transformer efficienti in memoria con xFormers..." (chipsbuilder.com).
 *
 *   out[b,i,h,:] = sum_j softmax_j( scale * q[b,i,h,:].k[b,j,g,:] + bias ) v[b,j,g,:]
 *   with g = h / (Hq / Hkv), over the keys j the mask allows.
 *
 * Layout (dense, bias_kind without MEA_MASK_BLOCKDIAG):
 *   q, out  [B, M, Hq,  D]      k, v  [B, N, Hkv, D]
 * Layout (packed, MEA_MASK_BLOCKDIAG): the batch is one physical row,
 *   q, out  [M, Hq, D]  (M = total packed queries)
 *   k, v    [N, Hkv, D] (N = total packed keys)
 *   B is the number of segments; seqstart_q / seqstart_k are int32 device
 *   arrays of B+1 non-decreasing prefix sums with seqstart_q[0] = 0,
 *   seqstart_q[B] = M (resp. N). seqstart_k may be NULL: then it equals
 *   seqstart_q (self-attention, requires M == N).
 *   Causal alignment is bottom-right within each segment.
 * scale         > 0 and finite (typically 1/sqrt(D)); used as given in fp32.
 * alibi_slopes  fp32 device array [Hq], required iff MEA_BIAS_ALIBI is set.
 * dtype         MEA_FP16 or MEA_BF16 for q, k, v and out.
 * lse           optional fp32 device array: log-sum-exp of each row's scaled,
 *               biased scores, natural log; layout [B, Hq, M] (dense) or
 *               [Hq, M] (packed). -inf for a row with no allowed key. NULL to skip.
 * Rows with no allowed key get out = 0.
 * Supported D: 64, 128 (see mea_supported). Hq % Hkv == 0.
 * Returns MEA_OK or an error status (nothing launched on error).
 */
int mea_fwd(const void* q, const void* k, const void* v, void* out,
            int B, int M, int N, int Hq, int Hkv, int D, float scale,
            unsigned bias_kind, const int32_t* seqstart_q, const int32_t* seqstart_k,
            const float* alibi_slopes, int dtype, float* lse, void* stream);

/*
 * mea_fwd_blocksparse - mea_fwd restricted to a block-sparse pattern: the
 * (query row, key) index space of every batch row and head is cut into
 * blocks of mea_block_sparse_block() x mea_block_sparse_block() (64 x 64),
 * and a pair is allowed only if its block is on (and, with MEA_MASK_CAUSAL,
 * the causal rule allows it). Blocks that are off are never loaded or
 * computed: each work-group walks a skip list of the key blocks its query
 * blocks need. The FlashAttention page names this block-sparse variant as
 * what reached 64K-element sequences ("FlashAttention (2022): l'attenzione
 * che non satura la memoria", paithon.it, section on what the numbers
 * showed); the pages give no pattern, so the mask is the caller's.
 *
 *   q, out [B, M, Hq, D]; k, v [B, N, Hkv, D] (dense layout of mea_fwd)
 *   block_mask  uint8 device array [ceil(M/64)][ceil(N/64)], row-major, shared
 *               by all batch rows and heads; nonzero = block on. Required.
 * bias_kind  MEA_MASK_CAUSAL and/or MEA_BIAS_ALIBI (MEA_MASK_BLOCKDIAG is
 *            MEA_EINVAL). Rows whose blocks are all off get out = 0, lse = -inf.
 * Other arguments, lse layout and errors as mea_fwd.
 */
int mea_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, int B, int M, int N, int Hq, int Hkv,
                        int D, float scale, unsigned bias_kind, const uint8_t* block_mask, const float* alibi_slopes,
                        int dtype, float* lse, void* stream);

/* Block edge (query rows and keys) of mea_fwd_blocksparse masks: 64. */
int mea_block_sparse_block(void);

/*
 * mea_bwd - backward pass of mea_fwd: the gradients dq, dk, dv of the loss
 * sum(dout * out) for the same (q, k, v, masks, bias). The scores are
 * recomputed block by block from q, k and the forward's lse, never stored
 * ("FlashAttention (2022): l'attenzione che non satura la memoria",
 * paithon.it, section on the softmax that needs not see the whole row: the
 * backward recomputes the score matrix on the fly). With P = exp(s - lse):
 *
 *   dP = dout v^T,  dS = P * (dP - rowsum(dout * out)),
 *   dq = scale dS k,  dk = scale dS^T q,  dv = P^T dout
 *
 * (the derivative of mea_fwd's definition through the softmax). Under
 * grouped-query attention dk, dv of a KV head sum over its query heads.
 * Training context: the xFormers tutorial's mixed-precision training section
 * (chipsbuilder.com page above).
 *
 *   q, out, dout, dq   layout of mea_fwd's q      k, v, dk, dv  layout of k
 *   lse     the fp32 log-sum-exp mea_fwd wrote for this (q, k, v) (required)
 *   out     mea_fwd's output for the same inputs
 * B, M, N, Hq, Hkv, D, scale, bias_kind, seqstart_q, seqstart_k,
 * alibi_slopes, dtype: exactly as in the mea_fwd call.
 * dq, dk, dv are fully overwritten (keys no query sees get 0); they must not
 * alias any input.
 * workspace  device buffer of at least mea_bwd_workspace_bytes(B, M, Hq,
 *            bias_kind) bytes, 256-byte aligned, owned by the caller;
 *            contents on entry ignored. Concurrent calls must not share it.
 * Accumulation is fp32; P and dS are rounded to the input type before their
 * products (as P in the forward); every gradient element has one writer, so
 * results are deterministic run to run.
 * Returns MEA_OK or an error status (nothing launched on error).
 */
size_t mea_bwd_workspace_bytes(int B, int M, int Hq, unsigned bias_kind);
int mea_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
            void* dq, void* dk, void* dv, int B, int M, int N, int Hq, int Hkv, int D, float scale,
            unsigned bias_kind, const int32_t* seqstart_q, const int32_t* seqstart_k, const float* alibi_slopes,
            int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mea_bwd_blocksparse - mea_bwd for a mea_fwd_blocksparse call: the same
 * arguments as that call (block_mask included) plus its out and lse, the
 * upstream gradient, the gradient outputs and the workspace of mea_bwd.
 * Blocks that are off are never loaded or computed; keys whose blocks are all
 * off get dk = dv = 0.
 */
int mea_bwd_blocksparse(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int M, int N, int Hq, int Hkv, int D,
                        float scale, unsigned bias_kind, const uint8_t* block_mask, const float* alibi_slopes,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mea_fwd_kvcache - chunked prefill / multi-token decode over a KV cache:
 * the M newest queries of every sequence attend to that sequence's cached
 * keys and values, whose rows for those M tokens are already appended. The
 * causal mask is aligned bottom-right (query row i, at position
 * ctx_lens[b]-M+i, sees cache rows j <= i + ctx_lens[b] - M), which is the
 * mask the simple KV cache builds: a lower triangle shifted by the number of
 * cached tokens ("Transformer : comprendre l'entrainement et l'inference",
 * briefia.fr, section on the simple KV cache; the prefill vs decode section).
 * Same kernels as mea_fwd, with each sequence's key count read from ctx_lens.
 *
 *   q, out   [B, M, Hq, D]
 *   kcache   [B, S_max, Hkv, D]     vcache same
 *   ctx_lens int32 device array [B], 0 <= ctx_lens[b] <= S_max; rows at or
 *            past ctx_lens[b] are never read. If ctx_lens[b] < M under the
 *            causal mask, the first M - ctx_lens[b] rows have no key: out 0.
 * bias_kind  MEA_MASK_CAUSAL and/or MEA_BIAS_ALIBI (MEA_MASK_BLOCKDIAG is
 *            MEA_EINVAL). lse, if given: [B, Hq, M].
 * Other arguments and errors as mea_fwd. With M = 1 this is the decode step
 * computed by the forward kernels (mea_decode is the faster path for it).
 */
int mea_fwd_kvcache(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out,
                    int B, int M, int Hq, int Hkv, int D, int S_max, float scale, unsigned bias_kind,
                    const float* alibi_slopes, int dtype, float* lse, void* stream);

/*
 * mea_kv_append - appends T new key/value rows per sequence to a KV cache:
 * rows k_new[b, t], v_new[b, t] go to cache row ctx_lens[b] + t, t < T
 * (each decode step concatenates the newest key and value to the cache:
 * briefia.fr page above, section on the simple KV cache). Rows that would
 * land at or past S_max are dropped. ctx_lens is read, not updated: the
 * caller adds T to its lengths.
 *
 *   kcache, vcache [B, S_max, Hkv, D] (written);  k_new, v_new [B, T, Hkv, D]
 *   ctx_lens int32 device array [B], 0 <= ctx_lens[b] <= S_max.
 *   T >= 0 (T = 0 is a no-op). dtype as mea_fwd; a bit-exact copy.
 * Returns MEA_OK or an error status (nothing launched on error).
 */
int mea_kv_append(void* kcache, void* vcache, const void* k_new, const void* v_new, const int32_t* ctx_lens, int B,
                  int S_max, int Hkv, int D, int T, int dtype, void* stream);

/*
 * mea_decode - one KV-cache decode step: each sequence's newest query
 * attends to all of its cached keys (its own key and value already
 * appended). Split-KV: the cached keys of all sequences, laid end to end,
 * are cut into equal spans (one per split work-group, at least
 * mea_decode_chunk() keys each), each span yields one partial (row max, row
 * sum, unnormalised output) per sequence it touches for all query heads of
 * one KV head, and a combine kernel merges a sequence's partials by their
 * log-sum-exp. The step itself: "Transformer : comprendre l'entrainement et
 * l'inference" (briefia.fr), sections on prefill vs decode and the simple
 * KV cache; the single-query equivalence: "Transformerを実装して少し理解した
 * 気になる会(その4)" (scrapbox.io), section "KV Cache"; the merge rule is
 * the block update of the online softmax (paithon.it page above).
 *
 *   q, out   [B, Hq, D]             (one query per sequence)
 *   kcache   [B, S_max, Hkv, D]     vcache same
 *   ctx_lens int32 device array [B], 0 <= ctx_lens[b] <= S_max (larger
 *            values are clamped to S_max, negative ones to 0), and
 *            B * S_max < 2^31 (else MEA_EINVAL). Slots
 *            >= ctx_lens[b] are never read and may hold anything (NaN).
 *            ctx_lens[b] == 0 gives out = 0.
 *   The query of sequence b sits at position ctx_lens[b]-1 (ALiBi distance
 *   ctx_lens[b]-1-j).
 * alibi_slopes  fp32 device array [Hq] or NULL (no bias).
 * workspace     device buffer of at least mea_decode_workspace_bytes(B, Hq, D,
 *               S_max) bytes, 256-byte aligned, owned by the caller; its
 *               contents on entry are ignored. Concurrent calls must not
 *               share a workspace. Its size does not depend on S_max: the
 *               partials take (1024 + B) * Hq * (D + 2) fp32 values (at most
 *               1024 split work-groups, one row per (work-group, sequence)
 *               pair), after a header of B + 2 int32.
 * Returns MEA_OK or an error status (nothing launched on error).
 */
size_t mea_decode_workspace_bytes(int B, int Hq, int D, int S_max);
int mea_decode(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens,
               void* out, int B, int Hq, int Hkv, int D, int S_max, float scale,
               const float* alibi_slopes, int dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * mea_decode_noalloc - mea_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same step, the same kernels and the same results
 * as mea_decode, with the workspace taken from a static device array of
 * MEA_DECODE_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * device it runs on until the process ends. The call allocates and frees
 * nothing. Arguments and errors as mea_decode, without the workspace.
 *
 * Limit: the step needs P + O + L bytes of scratch, P = (B + 2) * 4 rounded
 * up to 256, O = (G + B) * Hq * D * 4 rounded up to 256, L = (G + B) * Hq * 8,
 * with G the compute units of the stream's device (256 on MI355X); a larger
 * step returns MEA_ESCRATCH and launches nothing. (B=32, Hq=32, D=128 needs
 * 4.8 MB.)
 * The scratch is shared by every call on a device and keeps the last call's
 * contents (each call writes every byte it reads before reading it): calls
 * on one device whose work may overlap in time (different streams, or
 * different host threads without ordering) race on it and must be
 * serialised by the caller.
 */
#define MEA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int mea_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens,
                       void* out, int B, int Hq, int Hkv, int D, int S_max, float scale,
                       const float* alibi_slopes, int dtype, void* stream);

/* Human-readable text of a status code (static storage, never NULL). */
const char* mea_strerror(int status);

/* 1 if (dtype, head dim D) has kernels, else 0 (what xFormers' info listing
 * of supported kernels answers in the tutorial's setup section). */
int mea_supported(int dtype, int D);

/* Shortest span of keys of one decode split work-group. */
int mea_decode_chunk(void);

#ifdef __cplusplus
}
#endif

#endif /* MEA_H */
