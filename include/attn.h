/*
 * attn.h: C ABI of the MI355X (gfx950) fused attention library (forward in bf16
 * and FP8, backward, decode).
 *
 * The operation.  Scaled dot-product attention forward with the log-sum-exp
 * of every score row:
 *
 *     O   = softmax(scale * Q K^T  [+ causal mask]) V
 *     LSE = ln( sum_j exp(scale * q_i . k_j) )      over the allowed keys j
 *
 * as defined on page "GPU注意力算子性能优化" (QiMeng-Attention), section 1
 * (softmax(Q K^T / sqrt(d_k)) V, scores of shape [batch, heads, seq, seq]) and
 * page "注意力机制的本质与计算挑战", section 1 (scores, softmax, weighted sum of
 * V).  The mask is the causal one of page "AVO算法优化Transformer注意力机制性能
 * 解析", section 2.2: query i sees keys 0..i.  K/V heads are shared by
 * contiguous groups of query heads (GQA; MQA when H_kv = 1, MHA when
 * H_kv = H_q), per the QiMeng page, section 3.2.  The score matrix is never
 * written to memory: scores live in registers and an online softmax merges
 * key tiles (page "从硬件视角看注意力机制优化", section 2.1; the QiMeng page,
 * section 3.1.1: local computation plus a global reduction).
 *
 * Everything here is plain C: no HIP, torch or vendor bf16 types.  bf16 data
 * is passed as raw 16-bit storage behind void pointers.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every argument error is reported synchronously, before any
 * work is enqueued; nothing is launched when the status is not ATTN_OK. */
typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,      /* a required pointer is NULL                              */
    ATTN_ERR_SHAPE = 2,     /* B, H_q, H_kv, N or D <= 0, or a size overflows         */
    ATTN_ERR_GQA = 3,       /* H_q is not a multiple of H_kv                          */
    ATTN_ERR_HEAD_DIM = 4,  /* D is not a supported head size (this build: 128)        */
    ATTN_ERR_SCALE = 5,     /* scale is NaN or infinite                               */
    ATTN_ERR_ALIGN = 6,     /* a pointer is not 16-byte aligned                        */
    ATTN_ERR_ALIAS = 7,     /* an output range overlaps an input or the other output   */
    ATTN_ERR_LAUNCH = 8,    /* the HIP runtime rejected the kernel launch              */
    ATTN_ERR_DEVICE = 9,    /* the current device is not a gfx950 (MI350-series) GPU   */
    ATTN_ERR_WORKSPACE = 10,/* the workspace is smaller than the call needs            */
    ATTN_ERR_SCRATCH = 11   /* the call needs more than the library's fixed scratch    */
} attn_status;

/*
 * attn_fwd: enqueue the attention forward pass on `stream`.
 *
 * q    device pointer, bf16 [B, H_q, N, D], contiguous row-major (D fastest).
 * k, v device pointers, bf16 [B, H_kv, N, D], contiguous row-major.
 * o    device pointer, bf16 [B, H_q, N, D], written: O rounded to nearest even.
 * lse  device pointer, fp32 [B, H_q, N], written: natural-log LSE of each
 *      score row (scale included, masked keys excluded).  May be NULL when
 *      the caller does not need it.
 * B, H_q, H_kv, N, D   sizes; N is both the query and the key length.
 *      Query head h reads K/V head h / (H_q / H_kv).
 * causal   0: every query sees all N keys.  Non-zero: query i sees keys 0..i.
 * scale    multiplies the scores (1/sqrt(D) for the standard attention).
 * stream   a hipStream_t, or NULL for the default stream of the current
 *          device.  The pointers must belong to that device.
 *
 * Ownership: the caller allocates and frees every buffer; the library keeps no
 * pointer after the call returns, allocates no memory and keeps no global
 * state beyond a per-process cache of the device architecture check.  It does
 * not synchronise: the work runs in stream order and its results are visible
 * after the caller synchronises with the stream.  o and lse must not overlap
 * q, k, v or each other.  Results are bitwise reproducible for identical
 * inputs.  Thread-safe.
 *
 * Non-finite inputs propagate as the formula does in IEEE arithmetic, over the
 * keys each row sees: a NaN or +inf score makes its row NaN (O and LSE), a -inf
 * score gives its key weight 0, a row whose scores are all -inf is NaN, and a
 * NaN or infinity in V row j reaches O of exactly the rows that see key j.
 * The call enqueues two kernels: the fast one, and an exact one that redoes
 * only the query tiles whose masked key blocks (causal diagonal, ragged end)
 * hold a NaN or infinity in V; its other workgroups exit at once.
 *
 * Errors: returns a status code (see above).  A fault inside the kernel (for
 * example a pointer to too little memory) is reported by the HIP runtime at
 * the caller's next synchronisation, not by this call.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                     void* stream);

/*
 * attn_fwd_varlen: attn_fwd over a packed batch of variable-length sequences,
 * with an optional sliding window.
 *
 * The operation.  Sequences are concatenated along the token axis and never
 * attend across a boundary (variable sequence lengths: future work on the AVO
 * page, section 6).  Row i of a sequence sees key j of the same sequence when
 * i - window_left <= j <= i + window_right (a negative bound is unbounded), and
 * with `causal` also j <= i: the local-window and band attention of page
 * "注意力机制的本质与计算挑战", section 2.1.  Each row's O and LSE are attn_fwd's
 * over those keys.
 *
 * q, o     device pointers, bf16 [H_q, total, D] (head-major: the dense layout
 *          with B = 1 and N = total).
 * k, v     device pointers, bf16 [H_kv, total, D].
 * lse      device pointer, fp32 [H_q, total], or NULL.
 * cu_seqlens device pointer, int32 [n_seq + 1]: cu_seqlens[0] = 0, non-decreasing,
 *          cu_seqlens[n_seq] = total; sequence s is tokens cu[s] .. cu[s+1]-1.
 *          Every sequence must be at most max_seqlen tokens long: rows past
 *          max_seqlen are not written.  Offsets are clamped to [0, total], so
 *          malformed offsets cannot make the kernel access memory out of range.
 * window_left, window_right   the window (negative: no bound on that side).
 * Other arguments, precision, ownership and errors as for attn_fwd; cu_seqlens
 * must be 4-byte aligned and must not overlap o or lse.
 */
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens, int n_seq, int max_seqlen, int total,
                            int H_q, int H_kv, int D, int causal, int window_left,
                            int window_right, float scale, void* stream);

/*
 * attn_fwd_blocksparse: attn_fwd with a block-sparse mask.
 *
 * The operation.  Query rows and keys are cut into blocks of 128 (the last may
 * be short).  Query block qb of mask head mh attends to the key blocks listed in
 * kb_idx[kb_ptr[mh * n_blk + qb] .. kb_ptr[mh * n_blk + qb + 1] - 1], with
 * n_blk = ceil(N / 128), in block-compressed-row form (block-sparse patterns and
 * a compressed storage format for them: future work on page "AVO算法优化
 * Transformer注意力机制性能解析", section 6).  Row i of query head h sees key j
 * when j's block is listed for i's block of mask head (mask_heads == 1 ? 0 : h)
 * and, with `causal`, j <= i.  O and LSE are attn_fwd's over those keys; a row
 * that sees no key gets O = 0 and LSE = -inf.  Indices outside [0, n_blk) are
 * ignored and an index listed twice counts once.  The mask is shared by all
 * batch entries.
 *
 * kb_ptr   device pointer, int32 [mask_heads * n_blk + 1], non-decreasing
 *          offsets into kb_idx; they are clamped to [0, nnz] on the device, so
 *          malformed offsets cannot make the kernel read out of range.
 * kb_idx   device pointer, int32 [nnz] key-block indices (may be NULL if nnz = 0).
 * nnz      number of entries of kb_idx.
 * mask_heads  1 (one mask for every head) or H_q (one per query head).
 * Other arguments, precision, ownership and errors as for attn_fwd.  N may be
 * at most 2048 * 128 = 262144 (ATTN_ERR_SHAPE otherwise, as for mask_heads not
 * 1 or H_q and nnz < 0); kb_ptr, kb_idx must be 4-byte aligned and must not
 * overlap o or lse.
 */
attn_status attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int* kb_ptr, const int* kb_idx, int nnz, int mask_heads,
                                 int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                                 void* stream);

/*
 * attn_fwd_fp8: attn_fwd on FP8 (e4m3) inputs with per-tensor descales.
 *
 * The operation.  q8, k8 and v8 hold OCP e4m3 codes (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals, NaN at 0x7F/0xFF, largest finite
 * value 448); the tensors they stand for are Q = descale_q * q8, K = descale_k *
 * k8, V = descale_v * v8.  O and LSE are attn_fwd's on those tensors.  Both
 * matrix products run in FP8 with fp32 accumulation and the softmax runs in
 * fp32 (page "注意力机制的本质与计算挑战", section 3: FP16/FP8 matrix products,
 * fp32 softmax and accumulation; page "GPU注意力算子性能优化" (QiMeng-Attention),
 * section 3.1.1; FP8 storage with wider accumulation: page "从硬件视角看注意力
 * 机制优化", section 2.3).  The softmax weights are rounded to e4m3 for the
 * second product: each row's weights of a block of 64 keys are first
 * multiplied by the power of two that puts their largest one in (224, 448],
 * the top binade of e4m3 (so none overflows and none is rounded more coarsely
 * than 2^-10 / 224 of the largest), and the matrix core's E8M0 operand scale
 * takes the power of two back exactly.  O is normalised by the sum of the
 * rounded weights; the LSE uses the fp32 weights.  NaN codes propagate as in
 * attn_fwd (e4m3 has no infinity).
 *
 * q8       device pointer, uint8 [B, H_q, N, D] codes, contiguous row-major.
 * k8, v8   device pointers, uint8 [B, H_kv, N, D] codes.
 * o        device pointer, bf16 [B, H_q, N, D], written.
 * lse      device pointer, fp32 [B, H_q, N], or NULL.
 * descale_q, descale_k, descale_v   finite fp32 factors (ATTN_ERR_SCALE
 *          otherwise, or when |scale * descale_q * descale_k| overflows fp32).
 * Other arguments, ownership and errors as for attn_fwd (D must be 128; q8,
 * k8, v8, o 16-byte aligned, lse 4-byte aligned).
 */
attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse,
                         int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                         float descale_q, float descale_k, float descale_v, void* stream);

/*
 * attn_bwd: enqueue the attention backward pass on `stream`: the gradients of
 * a scalar loss with respect to q, k and v, given its gradient dout with
 * respect to the forward output.
 *
 * The operation.  The chain rule through the forward above, with the
 * probabilities recomputed from the forward's LSE rather than stored (page
 * "AVO算法优化Transformer注意力机制性能解析", section 2.2: recomputation and
 * gradient reuse in the backward pass; page "GPU注意力算子性能优化"
 * (QiMeng-Attention), section 2.2.2: the backward's gradients).  With
 * P_ij = exp(scale * q_i.k_j - LSE_i) over the allowed keys:
 *
 *     delta_i = dO_i . O_i
 *     dS_ij   = P_ij (dO_i . v_j - delta_i)
 *     dQ_i    = scale * sum_j dS_ij k_j
 *     dK_j    = scale * sum_i dS_ij q_i      (summed over the query heads
 *     dV_j    = sum_i P_ij dO_i               of the K/V head's group)
 *
 * q, dout  device pointers, bf16 [B, H_q, N, D] (dout: dL/dO).
 * k, v     device pointers, bf16 [B, H_kv, N, D].
 * o, lse   the forward's outputs for these q, k, v, causal and scale: bf16
 *          [B, H_q, N, D] and fp32 [B, H_q, N] (natural log).
 * dq       device pointer, bf16 [B, H_q, N, D], written.
 * dk, dv   device pointers, bf16 [B, H_kv, N, D], written.
 * delta    device pointer, fp32 [B, H_q, N], written with delta_i above (the
 *          dK/dV kernel reads it back; its value after the call is the row sum
 *          dO_i . O_i in fp32).
 * B, H_q, H_kv, N, D, causal, scale, stream: as for attn_fwd.
 *
 * Precision: P and dS are rounded to bf16 (nearest even) as matrix-core
 * operands (for dK, dS is formed from the bf16 P; for dQ from the fp32 P),
 * every sum is accumulated in fp32, and the three gradients are rounded to
 * bf16 (nearest even) once at the end.  No atomics: results are bitwise
 * reproducible.
 *
 * Ownership and errors as for attn_fwd.  No output may overlap an input or
 * another output (ATTN_ERR_ALIAS); q, k, v, o, dout, dq, dk, dv must be
 * 16-byte aligned and lse, delta 4-byte aligned (ATTN_ERR_ALIGN).
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     float* delta, int B, int H_q, int H_kv, int N, int D, int causal,
                     float scale, void* stream);

/*
 * attn_bwd_dq and attn_bwd_dkdv: the two kernels of attn_bwd as separate
 * calls (attn_bwd enqueues exactly these two, in this order).  attn_bwd_dq
 * writes dq and delta; attn_bwd_dkdv reads delta (as written by attn_bwd_dq
 * for the same q, k, v, o, dout, lse, causal and scale, earlier in stream
 * order) and writes dk, dv.  Arguments, layouts, precision, ownership and
 * errors as for attn_bwd; for attn_bwd_dkdv, delta is an input.
 */
attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, float* delta,
                        int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                        void* stream);
attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, const float* delta, void* dk, void* dv,
                          int B, int H_q, int H_kv, int N, int D, int causal, float scale,
                          void* stream);

/*
 * attn_bwd_ws: attn_bwd with the dK/dV step split over the query heads of
 * each K/V head's group.  The dK/dV step runs one workgroup per 128 keys of a
 * K/V head, so with few K/V heads (MQA, small GQA batches) it has fewer
 * workgroups than the GPU has compute units.  Here each of n_splits parts of a
 * group's query heads writes fp32 partial dK and dV into `workspace`, and a
 * third kernel adds the parts in part order and rounds once to bf16.
 *
 * n_splits   parts per group, or <= 0 to let the library choose
 *            (attn_bwd_splits); it is reduced to a divisor of H_q / H_kv.  With
 *            one part this is exactly attn_bwd and `workspace` is not used (it
 *            may be NULL).
 * workspace  device memory of at least attn_bwd_workspace_bytes(B, H_q, H_kv,
 *            N, D, n_splits) bytes, 16-byte aligned, owned by the caller,
 *            disjoint from every argument, and not used by other work until
 *            the call's work has finished.  Its contents on entry do not matter.
 * Other arguments, layouts and errors as for attn_bwd, plus
 * ATTN_ERR_WORKSPACE (too small).  Precision as for attn_bwd, except that dK
 * and dV are the fp32 sums of the parts' fp32 sums, still reproducible
 * bitwise for a given n_splits.
 */
attn_status attn_bwd_ws(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, int B, int H_q, int H_kv, int N, int D, int causal,
                        float scale, int n_splits, void* workspace, size_t workspace_bytes,
                        void* stream);

/* attn_bwd_splits: the parts attn_bwd_ws uses for these arguments (n_splits <=
 * 0: the library's choice, the smallest divisor of H_q / H_kv that gives at
 * least 256 dK/dV workgroups, causal: 1024, or 2048 from N = 8192, at most
 * 16), or 0 if they are invalid.  Host-only arithmetic. */
int attn_bwd_splits(int B, int H_q, int H_kv, int N, int D, int causal, int n_splits);

/* attn_bwd_workspace_bytes: bytes of workspace attn_bwd_ws needs for these
 * arguments: 2 * parts * B * H_kv * N * D * 4 when it splits, else 0 (also 0 if
 * they are invalid).  Host-only arithmetic. */
size_t attn_bwd_workspace_bytes(int B, int H_q, int H_kv, int N, int D, int causal, int n_splits);

/*
 * attn_decode: enqueue split-KV decode attention on `stream`.
 *
 * The operation.  M query rows per (batch, query head) are the last M
 * positions of a sequence whose L keys and values are cached.  Each row gets
 * the forward's result (attn_fwd above) over its allowed keys: all L keys, or
 * with `causal` keys 0 .. L - M + i for row i (0 <= i < M).  The key range is
 * cut into splits computed in parallel, whose partial results are then merged
 * exactly by their log-sum-exp (the "local computation plus global reduction"
 * of the QiMeng page, section 3.1.1; see attn_lse_merge below).
 *
 * q      device pointer, bf16 [B, H_q, M, D].
 * k, v   device pointers, bf16 [B, H_kv, L, D] (the cache).
 * o      device pointer, bf16 [B, H_q, M, D], written (round to nearest even).
 * lse    device pointer, fp32 [B, H_q, M], written (natural log), or NULL.
 * causal 0: every row sees all L keys; non-zero: as above (needs M <= L).
 * scale  multiplies the scores.
 * n_splits   number of key splits, or <= 0 to let the library choose (about
 *        2048 waves of work); it is reduced to at most one split per 32 keys.
 * workspace  device memory of at least attn_decode_workspace_bytes(B, H_q,
 *        H_kv, M, L, D, n_splits) bytes, 16-byte aligned, owned by the caller;
 *        it holds the partial results between the two kernels of the call and
 *        must not be used by other work until the call's work has finished.
 * stream as for attn_fwd.
 *
 * Precision: scores and P V accumulate in fp32 on the matrix cores with P
 * rounded to bf16; each partial O is divided by the sum of the bf16 weights
 * it applied; partials and the merge are fp32; O is rounded to bf16 once.
 * Non-finite inputs propagate as the formula does: a NaN or +inf score, or
 * scores that are all -inf, make the row's O and LSE NaN; a non-finite V
 * element reaches exactly the rows that see its key (keys a row does not see
 * never enter its products).
 * Errors as for attn_fwd, plus ATTN_ERR_WORKSPACE.  q, k, v and workspace must
 * be 16-byte aligned, o and lse 4-byte aligned.
 */
attn_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H_q, int H_kv, int M, int L, int D, int causal, float scale,
                        int n_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_noalloc: attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops with a fixed memory
 * plan, harnesses that forbid hipMalloc.  It takes no workspace and calls no
 * allocator: the partial results live in a fixed array inside the library,
 * ATTN_DECODE_SCRATCH_BYTES per GPU, which each GPU the library runs on holds
 * until the process ends.  The array's address on a device is looked up
 * (hipGetSymbolAddress) on the first call with that device current.
 *
 * Every call on one GPU uses that GPU's one array and leaves its partial
 * results there.  Calls whose work can overlap on one GPU (streams with no
 * ordering between them) race on it; calls in one stream, or ordered by
 * events, are safe.  No part of the array needs to start at zero: a call
 * writes every entry it reads.
 *
 * Arguments, precision and errors as for attn_decode, without workspace and
 * workspace_bytes, plus ATTN_ERR_SCRATCH when attn_decode_workspace_bytes()
 * for these arguments exceeds ATTN_DECODE_SCRATCH_BYTES (checked before any
 * HIP call).  o and lse must be 4-byte aligned.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H_q, int H_kv, int M, int L, int D, int causal,
                                float scale, int n_splits, void* stream);

/*
 * attn_decode_partial: only the local half of attn_decode: the partial result
 * of every key split, for a caller that merges them itself (attn_lse_merge, or
 * a merge across devices).  Split s covers keys [32*floor(s*nb/n_splits),
 * 32*floor((s+1)*nb/n_splits)) with nb = ceil(L/32); n_splits must be in
 * [1, nb].
 *
 * o_part   device pointer, fp32 [B*H_q*M, n_splits, D], 16-byte aligned,
 *          written: each split's softmax-weighted mean of V over its allowed
 *          keys (0 where it has none; where they all scored -inf, the sum of
 *          0 * V over them: 0, or NaN where such a V element is not finite).
 * lse_part device pointer, fp32 [B*H_q*M, n_splits], written: each split's
 *          natural-log LSE (-inf where it has no allowed key or they all
 *          scored -inf; NaN where one scored NaN or +inf).
 * Other arguments as for attn_decode.
 */
attn_status attn_decode_partial(const void* q, const void* k, const void* v, float* o_part,
                                float* lse_part, int B, int H_q, int H_kv, int M, int L, int D,
                                int causal, float scale, int n_splits, void* stream);

/* attn_decode_splits: the number of key splits attn_decode uses for these
 * arguments (n_splits <= 0: the library's choice), or 0 if they are invalid.
 * Host-only arithmetic. */
int attn_decode_splits(int B, int H_q, int H_kv, int M, int L, int D, int n_splits);

/* attn_decode_workspace_bytes: bytes of workspace attn_decode needs for these
 * arguments (0 if they are invalid).  Host-only arithmetic. */
size_t attn_decode_workspace_bytes(int B, int H_q, int H_kv, int M, int L, int D, int n_splits);

/*
 * attn_lse_merge: combine partial attention results over disjoint key sets,
 * exactly: LSE = ln sum_p exp(LSE_p) and O = sum_p exp(LSE_p - LSE) O_p (the
 * QiMeng page, section 3.1.1: the global reduction of local results).  This is
 * also the step that merges per-GPU partials when keys are sharded.
 *
 * o_part   device pointer, fp32 [rows, n_parts, D], 16-byte aligned.
 * lse_part device pointer, fp32 [rows, n_parts]; -inf marks a part of weight
 *          0 (no keys, or keys that all scored -inf): its O_p is multiplied
 *          by that 0, so a NaN there reaches O.  A NaN or +inf LSE_p makes
 *          the row's O and LSE NaN.
 * o        device pointer, bf16 [rows, D], written (round to nearest even).
 * lse      device pointer, fp32 [rows], written, or NULL.  A row whose parts
 *          are all -inf gets O = 0 and LSE = -inf (attn_decode, whose rows
 *          always have keys, makes such a row NaN instead).
 * D        128 in this build.
 */
attn_status attn_lse_merge(const float* o_part, const float* lse_part, int rows, int n_parts,
                           int D, void* o, float* lse, void* stream);

/* attn_decode_flops: 4 * D flops per allowed (row, key) pair, summed over
 * B * H_q heads.  Host-only arithmetic. */
double attn_decode_flops(int B, int H_q, int M, int L, int D, int causal);

/* attn_status_string: a static, human-readable description of a status code. */
const char* attn_status_string(int status);

/*
 * attn_fwd_flops: the throughput convention of the benchmarks,
 * 4 * B * H_q * N^2 * D, halved when causal.  Host-only arithmetic.
 */
double attn_fwd_flops(int B, int H_q, int N, int D, int causal);

/*
 * attn_bwd_flops: 10 * B * H_q * N^2 * D (the five N x N x D products S, dP,
 * dV, dK, dQ), halved when causal.  Host-only arithmetic.
 */
double attn_bwd_flops(int B, int H_q, int N, int D, int causal);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
