/*
 * fa2.h — C ABI of the gfx950 exact-softmax-attention library (libfa2.so): forward and
 * backward.
 *
 * The operation (per head, per sequence):
 *     S = scale * Q K^T,  S[i][j] = -inf where causal and j > i,
 *     P = row-softmax(S),  O = P V,  LSE[i] = log(sum_j exp(S[i][j]))  (natural log)
 * computed without writing S or P to memory, as in the FlashAttention-2 forward:
 *   - definition S = QK^T, P = softmax(S), O = PV: "FlashAttention 2: Faster Attention with
 *     Better Parallelism and Work Partitioning" reading notes (papers.chlience.com), section 1;
 *     the 1/sqrt(d) scale inside the score: "FlashAttention" (llm-infra-atlas), section 1;
 *   - the one-pass recurrence with an unscaled accumulator and a single final division, and
 *     the logsumexp L = m + log(l) as the second output: chlience notes, section 5.2;
 *     "FlashAttention-2: ..." summary (paper-graph-ui), section 3.4, "Algorithm 1 Walkthrough"
 *     and "Tweak 2: Store Logsumexp";
 *   - causal semantics (column index greater than row index is masked) and skipping of tiles
 *     that lie wholly above the diagonal: paper-graph-ui section 3.4, "Causal masking
 *     optimization"; chlience notes, section 5.6;
 *   - packed variable-length batches addressed by cu_seqlens offsets: llm-infra-atlas,
 *     section 0 (the engineering-interface entry of its reading table).
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers (HIP device memory). bf16 tensors are passed as raw 16-bit
 *     words (bfloat16 bit patterns). q, k, v, o must be 16-byte aligned; lse 4-byte aligned.
 *   - Ownership: the caller allocates and frees every buffer. The library never allocates,
 *     frees or retains a pointer, and keeps no mutable global state; calls are reentrant.
 *     Two exceptions use static device arrays of the library. fa2_fwd_splitkv_noalloc keeps
 *     its partials in one (see there). The persistent kernels, which fa2_fwd_varlen uses at
 *     d = 72..128 and fa2_bwd_varlen at d = 72..256, take their work-queue counters from a
 *     pool of sets that every launch returns to zero (see fa2_fwd_varlen).
 *   - On success every element of o and lse covered by the call is overwritten (for the
 *     varlen entry: the rows of every sequence, see below). Inputs are never written.
 *   - stream is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously;
 *     the call returns without synchronising. A call enqueues kernel launches only (no
 *     allocation, memset, copy or host synchronisation), so it may be captured in a HIP
 *     graph and replayed.
 *   - Arguments are validated on the host before any HIP call. On any error nothing is
 *     launched and nothing is written; the return value says why (FA2_* codes below).
 *   - Problems with zero rows (N == 0, total_tokens == 0 or num_seqs == 0) succeed without a
 *     launch; their pointers may then be NULL.
 *   - Results are deterministic: no arithmetic uses atomics, so a call with the same inputs
 *     and variant gives bitwise-identical outputs, independent of B and H. (The persistent
 *     kernels' work queues hand out blocks in a varying order; each block is computed the
 *     same way whichever workgroup takes it.)
 */
#ifndef FA2_H_
#define FA2_H_

#ifdef __cplusplus
extern "C" {
#endif

enum fa2_status {
  FA2_OK = 0,
  FA2_ERR_NULL_PTR = 1,            /* a required pointer is NULL */
  FA2_ERR_BAD_SHAPE = 2,           /* B, H or H_kv <= 0, H_kv not dividing H, N < 0, ... */
  FA2_ERR_UNSUPPORTED_HEADDIM = 3, /* d not a multiple of 8 in [8, 256] */
  FA2_ERR_MISALIGNED = 4,          /* q/k/v/o not 16-byte aligned, or lse not 4-byte aligned */
  FA2_ERR_BAD_SCALE = 5,           /* scale is NaN or infinite */
  FA2_ERR_NO_DEVICE = 6,           /* no usable HIP device is current */
  FA2_ERR_LAUNCH = 7,              /* the kernel launch failed (HIP error) */
  FA2_ERR_BAD_VARIANT = 8,         /* variant index out of range for this d */
  FA2_ERR_TOO_LARGE = 9,           /* the grid or an index would overflow 31 bits */
  FA2_ERR_SCRATCH_TOO_SMALL = 10   /* fa2_fwd_splitkv_noalloc: the partials exceed the
                                      static scratch (FA2_STATIC_SCRATCH_BYTES) */
};

/* Size of the static device scratch that fa2_fwd_splitkv_noalloc uses (per device). */
#define FA2_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * Fixed-length forward.
 *   q, k, v : bf16 [B, H, N, d], contiguous (d fastest), read only.
 *   o       : bf16 [B, H, N, d], contiguous; written with round-to-nearest-even.
 *   lse     : fp32 [B, H, N]; natural-log logsumexp of each row of S.
 *   d       : any multiple of 8 from 8 to 256 (64, 128 and 256 run natively; other
 *             values run on the next of those widths with the extra columns padded, at the
 *             padded width's matrix cost).  causal: 0 or 1 (mask key j > query i).
 *   scale   : any finite float (typically 1/sqrt(d)); applied to QK^T before the softmax.
 * Returns FA2_OK or an error code (see above).
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int N, int d, int causal, float scale, void* stream);

/*
 * Packed variable-length forward: num_seqs sequences concatenated along the token axis.
 *   q, k, v, o : bf16 [H, total_tokens, d] contiguous (each head holds all tokens of all
 *                sequences back to back).
 *   lse        : fp32 [H, total_tokens].
 *   cu_seqlens : DEVICE int32 [num_seqs + 1]; sequence s owns tokens [cu[s], cu[s+1]).
 *                Expected: cu[0] = 0, non-decreasing, cu[num_seqs] = total_tokens and every
 *                length <= max_seqlen. The contents are not checked on the host; the kernel
 *                clamps every offset into [0, total_tokens], so bad offsets never cause an
 *                out-of-bounds access, but rows outside [0, max_seqlen) of a sequence, and
 *                tokens covered by no sequence, are then left unwritten.
 *   max_seqlen : upper bound on the sequence lengths (sizes the grid).
 *   causal     : mask within each sequence with sequence-local indices.
 * At head dimensions that run on the d = 128 kernels (72..128) this call uses the persistent
 * variant (d128_w8_bc64_persist): one workgroup per CU takes row blocks from a work queue,
 * so the row blocks past the end of shorter sequences cost no workgroup launch. Its queue
 * counters live in a static per-device pool of 1024 sets, one set per launch in turn, each
 * returned to zero by its launch: the pool allocates nothing, and launches in flight at
 * the same time on one device use different sets as long as fewer than 1024 of them run
 * at once. A call made while its stream is being captured into a graph launches the
 * ordinary one-workgroup-per-row-block kernel instead, which gives the same results.
 * Other head dimensions use variant 0.
 */
int fa2_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                   int H, int d, int causal, float scale, void* stream);

/*
 * Same as fa2_fwd / fa2_fwd_varlen, with an explicit kernel variant (tile configuration).
 * variant 0 is the default that fa2_fwd uses; 1 .. fa2_num_variants(d)-1 are alternatives
 * with identical results up to rounding order. Used by tuning sweeps and tests.
 */
int fa2_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, int causal, float scale, int variant,
                    void* stream);
int fa2_fwd_varlen_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int* cu_seqlens, int num_seqs, int max_seqlen,
                           int total_tokens, int H, int d, int causal, float scale,
                           int variant, void* stream);

/*
 * Grouped-query and multi-query forward: H query heads share H_kv key/value heads, query
 * head h reading key/value head floor(h / g) with g = H / H_kv, and no copy of K or V is
 * made ("FlashAttention 2: ..." reading notes, papers.chlience.com, section 5.6, the head
 * index mapping for MQA/GQA; paper-graph-ui summary, section 3.4, "The Backward Pass:
 * Simpler Statistics, Same Structure", its paragraph on multi-query and grouped-query
 * attention).
 *   q, o : bf16 [B, H, N, d];  k, v : bf16 [B, H_kv, N, d];  lse : fp32 [B, H, N].
 *   varlen: q, o [H, total_tokens, d]; k, v [H_kv, total_tokens, d]; lse [H, total_tokens].
 *   H_kv must divide H (else FA2_ERR_BAD_SHAPE); H_kv == H is ordinary multi-head attention
 *   and H_kv == 1 is multi-query attention. variant as for fa2_fwd_variant (0 = the
 *   fixed-length default; for the varlen call, fa2_fwd_varlen_default_variant(d) is the
 *   variant fa2_fwd_varlen runs).
 * Everything else (validation, ownership, asynchrony, zero-size calls) is as for fa2_fwd.
 */
int fa2_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int H_kv, int N, int d, int causal, float scale, int variant,
                void* stream);
int fa2_fwd_varlen_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                       int H, int H_kv, int d, int causal, float scale, int variant,
                       void* stream);

/*
 * Forward of a query block against one key/value chunk, with separate query and key
 * lengths: the building block of split-KV (several chunks, then fa2_lse_merge) and of
 * sharding the key sequence across devices ("FlashAttention", llm-infra-atlas, section 5:
 * each step of context parallelism is one call with the right mask).
 *   q, o : bf16 [B, H, N_q, d];  k, v : bf16 [B, H_kv, N_k, d];  lse : fp32 [B, H, N_q].
 *   causal: query i (0-based within q) may attend key j (0-based within k) iff
 *           j <= i + diag. diag = 0 with N_q == N_k is fa2_fwd's mask; diag = N_k - N_q
 *           aligns the last query with the last key; for the chunk [a, b) of a sequence
 *           whose queries start at position q_start, diag = q_start - a. |diag| <= 2^30.
 *   Rows with no allowed key (N_k == 0, or all keys masked) get O = 0 and LSE = -inf.
 *   k and v are not read when N_k == 0 and may then be NULL.
 * H_kv, variant and everything else as for fa2_fwd_gqa; fa2_fwd_gqa is this call with
 * N_q = N_k = N and diag = 0.
 */
int fa2_fwd_chunk(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int H_kv, int N_q, int N_k, int d, int causal, int diag,
                  float scale, int variant, void* stream);

/*
 * Split-KV forward: fa2_fwd_chunk's result computed with the keys cut into up to num_splits
 * contiguous pieces that run in the same launch (more workgroups when B*H*ceil(N_q/128) is
 * small, e.g. few query rows over a long key sequence), followed by fa2_lse_merge of the
 * pieces. Arguments as fa2_fwd_chunk, plus:
 *   num_splits : >= 1. The pieces are ceil(N_k / num_splits) keys rounded up to the key tile
 *                of the variant, so fewer pieces than num_splits may be used.
 *   o_parts    : bf16 [num_splits, B, H, N_q, d] workspace, lse_parts : fp32
 *                [num_splits, B, H, N_q] workspace (caller-provided; overwritten; unused and
 *                may be NULL when num_splits == 1 or N_k == 0).
 * Results equal fa2_fwd_chunk's up to rounding (each piece's O is rounded to bf16 once
 * before the merge).
 */
int fa2_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int H_kv, int N_q, int N_k, int d, int causal, int diag,
                    float scale, int num_splits, void* o_parts, float* lse_parts, int variant,
                    void* stream);

/*
 * fa2_fwd_splitkv without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The per-piece partial O and LSE live in a static device array of the library,
 * FA2_STATIC_SCRATCH_BYTES per device (each device the library runs on holds its own copy
 * until the process ends). The call allocates nothing and frees nothing.
 *   Arguments, results and validation as fa2_fwd_splitkv (minus o_parts / lse_parts).
 *   The pieces need P * B * H * N_q * (2 d + 4) bytes (P pieces, the bf16 part rounded up to
 *   256 bytes); above FA2_STATIC_SCRATCH_BYTES the call returns FA2_ERR_SCRATCH_TOO_SMALL and
 *   launches nothing. With one piece (num_splits == 1, or N_k == 0) it is fa2_fwd_chunk and
 *   the scratch is not used.
 *   The first call on a device looks up that device's copy of the array (hipGetSymbolAddress,
 *   with the device current) and keeps the address for the life of the process;
 *   FA2_ERR_NO_DEVICE if that fails. A device reset (hipDeviceReset) unloads the array, so the
 *   kept address is not valid afterwards: do not call this entry point on a device after
 *   resetting it in the same process.
 *   Every call on one device shares that device's scratch, which keeps the last call's
 *   partials (every partial row read by the merge is written by the same call first, so
 *   nothing needs clearing). Calls that overlap on one device (two streams, or two host
 *   threads, before the first has finished on the GPU) race on the scratch and may return
 *   wrong results: serialise them.
 */
int fa2_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N_q, int N_k, int d, int causal,
                            int diag, float scale, int num_splits, int variant, void* stream);

/*
 * Merge of partial results by their logsumexp (the "LSE mix"):
 *     LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s
 * which recovers attention over the union of the parts' key sets exactly (up to rounding).
 * ("FlashAttention", llm-infra-atlas: section 5 on context parallelism, and its section 0
 * reading table on mixing the LSEs of two variable-length calls.)
 *   o_parts   : bf16 [num_parts, rows, d] (part s is the contiguous block s), read only.
 *   lse_parts : fp32 [num_parts, rows] (natural log; -inf marks a row with no key in part s).
 *   o         : bf16 [rows, d]; lse : fp32 [rows]; written. rows is any count, e.g.
 *               B * H * N_q for fa2_fwd_chunk outputs. o/lse must not alias the parts.
 *   d         : a multiple of 8 from 8 to 256.  num_parts >= 1.
 * A row whose LSE_s are all -inf gets O = 0 and LSE = -inf. rows == 0 succeeds without a
 * launch. Validation, ownership and asynchrony as for fa2_fwd.
 */
int fa2_lse_merge(const void* o_parts, const float* lse_parts, int num_parts, long long rows,
                  int d, void* o, float* lse, void* stream);

/*
 * Backward: gradients of O = softmax(scale * Q K^T [causal]) V with respect to Q, K and V,
 * given dO, the forward's O and LSE. P is recomputed from LSE rather than stored, and
 *     D = rowsum(dO o O),  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
 *     dQ = scale * dS K,   dK = scale * dS^T Q
 * ("FlashAttention 2: ..." reading notes, papers.chlience.com, sections 5.2 and 5.3;
 * paper-graph-ui summary, section 3.4, "The Backward Pass: Simpler Statistics, Same
 * Structure"; the pages state dQ and dK for an unscaled score, the factor scale follows from
 * S = scale * Q K^T). With grouped-query attention dK and dV of a key/value head are summed
 * over its query heads (chlience notes, section 5.6).
 *   q, o, dout, dq : bf16 [B, H, N, d];  k, v, dk, dv : bf16 [B, H_kv, N, d];
 *   lse            : fp32 [B, H, N], the forward's logsumexp (natural log);
 *   delta          : fp32 [B, H, N] caller-provided buffer, overwritten with D (it is the
 *                    only intermediate; the library allocates nothing).
 *   H_kv must divide H. d is a multiple of 8 up to 256 (64, 128 and 256 natively, others
 *   padded as in the forward); causal and scale as for the forward (same scale as the
 *   forward).
 *   dq, dk, dv and delta are fully overwritten on success; they must not alias the inputs.
 * Two kernels run in order on stream (dQ and D, then dK and dV); no arithmetic uses atomics,
 * so the gradients are bitwise reproducible. Validation, ownership and zero-size rules as
 * fa2_fwd.
 * Varlen: q, o, dout, dq [H, T, d]; k, v, dk, dv [H_kv, T, d]; lse, delta [H, T];
 * cu_seqlens as for fa2_fwd_varlen (tokens covered by no sequence are left unwritten). At
 * head dimensions 72..256 both kernels run in their persistent forms, which take blocks
 * from work queues whose counters come from the pool described at fa2_fwd_varlen (two sets
 * per call); under stream capture the ordinary kernels run instead. Results are the same
 * bits either way.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* delta,
            int B, int H, int H_kv, int N, int d, int causal, float scale, void* stream);
int fa2_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* delta,
                   const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                   int H, int H_kv, int d, int causal, float scale, void* stream);

/*
 * Backward of a fixed-length call with the query heads of each group split over several
 * dK/dV workgroups, for grouped- and multi-query attention. The gradients of a key/value head
 * are sums over the query heads that share it (chlience notes, section 5.6); fa2_bwd forms
 * them in one dK/dV workgroup per (key/value head, 128-key block), which with few key/value
 * heads leaves the GPU half idle (B=1, H_kv=2, N=16384: 1024 waves, where two per SIMD take
 * 2048). Here each group's g query heads are split over S workgroups, S the smallest divisor
 * of g that gives the dK/dV kernel as many waves as its occupancy fills on 256 CUs, four
 * times that when causal (causal key blocks carry unequal work), else g.
 * Each split writes fp32 partial dK and dV to the workspace, and a third kernel adds them in
 * split order and rounds to bf16.
 *   Arguments and results as fa2_bwd, plus:
 *   workspace       : device memory, 16-byte aligned, caller-owned, overwritten; may be NULL
 *                     when fa2_bwd_workspace_bytes(B, H, H_kv, N, d, causal) is 0.
 *   workspace_bytes : its size; below fa2_bwd_workspace_bytes(): FA2_ERR_SCRATCH_TOO_SMALL
 *                     (NULL when needed: FA2_ERR_NULL_PTR; misaligned: FA2_ERR_MISALIGNED).
 * When no split is needed (H_kv == H, or enough key/value heads and keys) the call is fa2_bwd,
 * bit for bit. With a split, dK and dV are the same sums taken in another order, so their
 * bits can differ from fa2_bwd's within rounding; repeated calls give the same bits.
 */
int fa2_bwd_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int H_kv,
               int N, int d, int causal, float scale, void* workspace, long long workspace_bytes,
               void* stream);

/* Workspace bytes fa2_bwd_ws needs for this shape and mask: S * 2 * B * H_kv * N * d * 4
 * (fp32 partial dK and dV per split), 0 when it does not split or the shape is invalid. Host
 * only; touches no device. */
long long fa2_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d, int causal);

/*
 * The same query-head splits for packed variable-length batches: arguments and results as
 * fa2_bwd_varlen, plus a workspace as for fa2_bwd_ws (S * 2 * H_kv * total_tokens * d * 4
 * bytes, from fa2_bwd_varlen_workspace_bytes; S chosen as for fa2_bwd_ws with total_tokens
 * keys per key/value head). The reduce visits each sequence's rows only, so tokens covered by
 * no sequence stay unwritten in dk and dv, as in fa2_bwd_varlen.
 */
int fa2_bwd_varlen_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta,
                      const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                      int H, int H_kv, int d, int causal, float scale, void* workspace,
                      long long workspace_bytes, void* stream);
long long fa2_bwd_varlen_workspace_bytes(int num_seqs, int max_seqlen, int total_tokens, int H,
                                         int H_kv, int d, int causal);

/* Number of kernel variants for head dimension d (0 if d is unsupported; a padded d has
 * the variants of its padded width). Host only. */
int fa2_num_variants(int d);

/*
 * Launch geometry of a fixed-length call, computed on the host without touching the GPU:
 * *num_workgroups = B*H*ceil(N/block_rows), *block_rows = query rows per workgroup,
 * *block_cols = keys per K/V tile, *lds_bytes = LDS per workgroup. Returns a status code;
 * outputs may be NULL.
 */
int fa2_fwd_geometry(int B, int H, int N, int d, int causal, int variant,
                     int* num_workgroups, int* block_rows, int* block_cols, int* lds_bytes);

/* Static, human-readable text for a status code (never NULL). */
const char* fa2_status_str(int status);

/* Static name of a kernel variant (e.g. "d128_w8_bc64_opt_la4"), or "" if out of range. */
const char* fa2_variant_name(int d, int variant);

/* The variant fa2_fwd_varlen runs for head dimension d (0 if d is unsupported). Host only. */
int fa2_fwd_varlen_default_variant(int d);

/* ABI version of this header; bumped on any incompatible change. */
int fa2_abi_version(void);

#define FA2_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* FA2_H_ */
