/*
 * mla.h -- C ABI of the MI355X (gfx950) absorbed-MLA decode library with decode
 * context parallelism (DCP).
 *
 * The operations are the ones the vLLM pages describe:
 *  - "vllm.v1.attention.backends.mla.flashattn_mla" API page, _forward_decode:
 *    absorbed MLA decode over a paged latent cache (q_pe against k_pe, q_nope
 *    against the latent c_kv, c_kv as the value, one softmax scale, causal),
 *    returning the output and the per-(token, head) LSE in [tokens, heads] order.
 *  - PR #24453 ("add DCP support for FLASH_ATTN_MLA backend"), review thread:
 *    global token p is stored on DCP rank p mod W, and with more than one query
 *    row per request each row gets its own per-rank seqlen_k (the interleaved
 *    causal mask; a row may see no key on a rank).  The same thread mentions the
 *    layout that gives each rank contiguous blocks of tokens (whole pages); the
 *    calls take both as runs of cp_interleave tokens dealt to the ranks in turn.
 *  - PR #48196 ("DCP sparse MLA output-merge optimizations"): the exact
 *    LSE-weighted merge of per-rank partials with per-row valid counts, the
 *    W_UV up-projection, which commutes with the merge, and the exchange that
 *    projects each rank's partial before the all-to-all (the pack by
 *    destination head slice and the receiving rank's combine; the transport
 *    between GPUs is the caller's).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps a pointer after the call returns, and it
 *    keeps no state between calls except a per-device "is this gfx950" flag.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without waiting.  No call reads device memory on the
 *    host (except mla_decode_partial in the MLA_DEBUG=1 mode described with
 *    it), so all calls can be captured in a HIP graph.
 *  - bf16 tensors are passed as `const void*` holding IEEE bfloat16 bits.
 *  - Errors are returned as mla_status codes; the library never aborts.  Host-
 *    visible argument errors are detected before anything is enqueued.
 *    Device-side preconditions (listed per call) are the caller's contract.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mla_status;

#define MLA_OK               0
#define MLA_ERR_NULL        -1  /* a required pointer is NULL                      */
#define MLA_ERR_SHAPE       -2  /* a size, stride or rank argument is out of range  */
#define MLA_ERR_UNSUPPORTED -3  /* current device is not gfx950                     */
#define MLA_ERR_WORKSPACE   -4  /* workspace too small for the requested splits      */
#define MLA_ERR_HIP         -5  /* a HIP runtime call or kernel launch failed        */
#define MLA_ERR_CAPTURE     -6  /* MLA_DEBUG checks asked for on a capturing stream  */

/* Element types of the per-rank partial outputs (mla_decode_partial's out,
 * the merges' outs).  bf16 is the default path; fp32 partials keep the merge's
 * inputs unrounded, so a merged row carries one bf16 rounding instead of two
 * (at twice the partials' bytes). */
#define MLA_DTYPE_BF16 0
#define MLA_DTYPE_F32  1
/* Element type of an FP8 latent cache (mla_decode_partial's kv_dtype): OCP
 * FP8 E4M3 ("fn": exponent bias 7, no infinities, largest finite 448) codes,
 * one fp32 scale per cache, element value = code value * kv_scale.  The pages
 * leave the convention open (they reject FP8 caches as unsupported); this is the
 * reading this library implements. */
#define MLA_DTYPE_FP8_E4M3 2

/* Which keys a query row sees (mask_mode of the decode calls).
 * MLA_MASK_CAUSAL: row i of a request, at global position p = S_b - Q_b + i,
 *   sees the keys at positions 0..p (on a DCP rank: the ones it stores; the
 *   interleaved causal mask of the PR #24453 thread).
 * MLA_MASK_CONTEXT: every row of the request sees the keys at positions
 *   0..S_b-Q_b-1, its tokens before the query tokens, without a causal mask:
 *   the context stage of the two-stage decode the same thread proposes for
 *   query_len > 1 (context KV with causal=False, query KV with causal=True).
 *   The query stage is an ordinary MLA_MASK_CAUSAL call with cp_world = 1 over
 *   the query tokens' own KV rows: for example kv_cache = those rows as
 *   [T, 1, 576] (page_size 1), block_table[b][j] = query_start_loc[b] + j and
 *   seq_lens[b] = Q_b.  Merging the cp_world context partials and the query
 *   partial with mla_lse_merge gives the unsharded result. */
#define MLA_MASK_CAUSAL  0
#define MLA_MASK_CONTEXT 1

/* Fixed head dimensions of the absorbed form. */
#define MLA_D_LATENT 512   /* kv_lora_rank: c_kv, q_nope and output width */
#define MLA_D_ROPE    64   /* qk_rope_head_dim: k_pe and q_pe width       */
#define MLA_D_ROW    576   /* one cache row: c_kv | k_pe                  */
#define MLA_D_V      128   /* v_head_dim: width after W_UV                */
#define MLA_MAX_HEADS 128

/* Human-readable name of a status code (static string, never NULL). */
const char* mla_status_string(mla_status status);

/*
 * mla_decode_partial -- one DCP rank's absorbed-MLA attention over its shard of
 * the paged latent cache ("flashattn_mla" _forward_decode with the PR #24453
 * interleaved mask).
 *
 * Requests b = 0..B-1 own the query tokens t in [query_start_loc[b],
 * query_start_loc[b+1]); Q_b is their count and T = query_start_loc[B].
 * seq_lens[b] = S_b is the request's GLOBAL token count, its own Q_b query
 * tokens included; query row i of b sits at global position p = S_b - Q_b + i.
 * Shard layout: runs of I = cp_interleave consecutive tokens are dealt to the W
 * ranks in turn, so token p is stored on rank (p div I) mod W (I = 1: rank
 * p mod W, the interleaved layout; I = page_size: whole pages per rank).  Rank
 * r stores its tokens in ascending position, local token j = (p div WI)*I +
 * p mod I living in physical block block_table[b*bt_stride + j / page_size],
 * slot j % page_size.  Row p sees the rank's first
 *   L = (n div WI)*I + min(max(n mod WI - rI, 0), I),   n = p + 1,
 * local tokens (its per-rank seqlen_k; with I = 1, ceil((p + 1 - r) / W), 0 if
 * p < r).
 *
 * For every token t and head h, with the visible local keys j:
 *   s_j  = scale * (q_nope[t,h,:] . c_kv_j + q_pe[t,h,:] . k_pe_j)
 *   lse  = ln sum_j exp(s_j)                       (natural log, fp32)
 *   out  = sum_j exp(s_j - lse) * c_kv_j           (bf16, round to nearest even)
 * A row that sees no key on this rank gets out = 0 and lse = -inf.  With
 * mask_mode = MLA_MASK_CONTEXT every row of request b sees instead the rank's
 * first Lx_b local keys, Lx_b = the count above for n = S_b - Q_b (the context
 * stage of the two-stage decode; only those keys need to be in the cache).
 *
 * Layouts (all last dimensions contiguous):
 *   q_nope   bf16 [T,H,512], element (t,h,d) at q_nope + t*qn_stride_t + h*qn_stride_h + d
 *            (strides in elements)
 *   q_pe     bf16 [T,H,64], strides qp_stride_t / qp_stride_h in elements; may
 *            alias q_nope + 512 when q is one [T,H,576] tensor
 *   kv_cache [num_blocks, page_size, 576] of element type kv_dtype: bf16
 *            (MLA_DTYPE_BF16; kv_scale is ignored) or FP8 E4M3 codes
 *            (MLA_DTYPE_FP8_E4M3: every value is code * kv_scale, kv_scale
 *            finite and > 0; only for H <= 16, the bandwidth-bound decode:
 *            more heads return MLA_ERR_UNSUPPORTED); block stride
 *            kv_block_stride elements (>= page_size*576, a multiple of 16
 *            bytes); row stride 576 elements
 *   block_table int32 [B, bt_stride]; entries past a request's last block are
 *            never read (may be -1)
 *   seq_lens int32 [B]; query_start_loc int32 [B+1], query_start_loc[0] = 0,
 *            nondecreasing
 *   out      [T,H,512] contiguous, bf16 (out_dtype = MLA_DTYPE_BF16, rounded
 *            to nearest even) or fp32 (MLA_DTYPE_F32, the normalised fp32
 *            accumulator);  lse fp32 [T,H] contiguous
 *   row_keys int32 [T] or NULL: when given, receives every row's L (the count
 *            of visible local keys above, under mask_mode), the values
 *            mla_dcp_local_seqlens writes for this rank and the merges take
 *            as valid counts; written by the launches of this call (no
 *            further launch)
 *
 * Host integers: max_query_len >= every Q_b and max_seq_len >= every S_b are
 * upper bounds that size the launch grid (nothing is read back from the
 * device).  num_splits caps how many workgroups split one row's keys
 * ("num_splits" of the varlen kernel call on the flashattn_mla page):
 * 0 = choose automatically, 1 = never split, k = at most k.  Splitting needs
 * `workspace` of at least mla_decode_workspace_size(...) bytes (any
 * alignment); with workspace == NULL the call runs unsplit.  The workspace
 * holds the split partials and the split tickets of the in-kernel combine,
 * and, for H = 64 or 128, the order in which the call dispatches its work
 * (longest rows first, computed on the device by the call itself; without a
 * workspace the rows run in token order, with the same results).  It must be
 * zero-filled before its first use, every call leaves it ready for the next
 * (tickets back at zero), and calls that overlap in time (e.g. on two
 * streams) must not share one workspace.
 *
 * Returns MLA_OK, or MLA_ERR_NULL / MLA_ERR_SHAPE (B<0, T<0, H outside
 * [1,128], page_size<1, cp_world<1, cp_rank outside [0,cp_world),
 * cp_interleave<1 or cp_world*cp_interleave > 2^30, strides
 * smaller than the data, scale not finite or not positive, out_dtype,
 * mask_mode or kv_dtype not one of theirs, an FP8 kv_scale not finite or
 * not positive) / MLA_ERR_WORKSPACE /
 * MLA_ERR_UNSUPPORTED / MLA_ERR_HIP.  B == 0 or T == 0 enqueues nothing and
 * returns MLA_OK (the grid is sized from host ints and may be empty).
 * Device-side contract: Q_b <= S_b <= max_seq_len, Q_b <= max_query_len,
 * block ids valid for every stored local token.
 *
 * Debug mode: with the environment variable MLA_DEBUG=1 the call first copies
 * seq_lens, query_start_loc and block_table to host memory on hip_stream,
 * waits for the stream, and checks the device-side contract with
 * mla_check_decode_metadata (block ids against the device allocation that
 * holds kv_cache).  A violation is reported on stderr and the call returns
 * MLA_ERR_SHAPE with nothing enqueued.  The wait makes debug mode unusable
 * inside HIP graph capture: on a capturing stream the call returns
 * MLA_ERR_CAPTURE.  Without MLA_DEBUG=1 nothing is read back.
 */
mla_status mla_decode_partial(
    const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
    const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
    const void* kv_cache, int32_t kv_dtype, float kv_scale, int64_t kv_block_stride, int32_t page_size,
    const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    int32_t B, int32_t T, int32_t H, int32_t max_query_len, int32_t max_seq_len,
    int32_t cp_world, int32_t cp_rank, int32_t cp_interleave, int32_t mask_mode, float scale,
    int32_t num_splits,
    void* out, int32_t out_dtype, float* lse, int32_t* row_keys,
    void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * mla_decode_partial_noalloc -- mla_decode_partial for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results and errors as
 * mla_decode_partial (with the same split plan, bit for bit the same
 * outputs), without the workspace: the split partials, split tickets and the
 * 128-head dispatch order live in a device array of the library,
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU it runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no hipFree, no
 * host allocation; MLA_DEBUG does not apply to it).  Its first call on a
 * device looks up that device's copy of the array.
 *   Returns MLA_ERR_WORKSPACE when the call's plan needs more than
 *   MLA_NOALLOC_SCRATCH_BYTES (mla_decode_workspace_size of the same
 *   arguments tells: it fits when that is at most the limit; long rows split
 *   many ways, e.g. a few 128-head tokens with num_splits in the hundreds, do
 *   not), otherwise as mla_decode_partial.
 * All calls on one GPU share its array, which keeps the last call's contents
 * (what must start at zero, the split tickets, is cleared by the calls that
 * use them): calls that overlap in time on one GPU (two streams, two host
 * threads) race and must not be issued.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

mla_status mla_decode_partial_noalloc(
    const void* q_nope, int64_t qn_stride_t, int64_t qn_stride_h,
    const void* q_pe, int64_t qp_stride_t, int64_t qp_stride_h,
    const void* kv_cache, int32_t kv_dtype, float kv_scale, int64_t kv_block_stride, int32_t page_size,
    const int32_t* block_table, int32_t bt_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    int32_t B, int32_t T, int32_t H, int32_t max_query_len, int32_t max_seq_len,
    int32_t cp_world, int32_t cp_rank, int32_t cp_interleave, int32_t mask_mode, float scale,
    int32_t num_splits,
    void* out, int32_t out_dtype, float* lse, int32_t* row_keys, void* hip_stream);

/*
 * mla_check_decode_metadata -- the device-side contract of mla_decode_partial,
 * checked on HOST copies of its metadata (what MLA_DEBUG=1 runs).  All
 * pointers are host pointers: seq_lens [B], query_start_loc [B+1],
 * block_table [B * bt_stride].  Checks, in order:
 *   query_start_loc[0] == 0, nondecreasing, query_start_loc[B] == T;
 *   per request: 0 <= Q_b <= max_query_len, Q_b <= S_b <= max_seq_len;
 *   the ceil(Lc_b / page_size) blocks that hold the Lc_b local tokens the call
 *   reads (rank cp_rank's share of all S_b tokens, or with MLA_MASK_CONTEXT of
 *   the first S_b - Q_b) fit in the row (<= bt_stride) and have ids in
 *   [0, num_blocks) (num_blocks < 0: only ids >= 0 are required).
 * Returns MLA_OK, MLA_ERR_NULL, or MLA_ERR_SHAPE for the first violation,
 * whose description goes to `reason` (NUL-terminated, truncated to
 * reason_len; may be NULL).  Pure host code: no device access.
 */
mla_status mla_check_decode_metadata(const int32_t* seq_lens, const int32_t* query_start_loc,
                                     const int32_t* block_table, int32_t bt_stride, int32_t B, int32_t T,
                                     int32_t max_query_len, int32_t max_seq_len, int32_t page_size,
                                     int32_t cp_world, int32_t cp_rank, int32_t cp_interleave,
                                     int32_t mask_mode, int64_t num_blocks, char* reason, size_t reason_len);

/*
 * Bytes of workspace mla_decode_partial needs for the same host arguments
 * (0 when the plan neither splits nor, for H = 64 or 128, orders its work).  Pure
 * host arithmetic, no device access.
 * Returns (size_t)-1 for invalid arguments.
 */
size_t mla_decode_workspace_size(int32_t B, int32_t T, int32_t H, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t cp_world, int32_t cp_interleave,
                                 int32_t num_splits);

/*
 * mla_lse_merge -- exact LSE-weighted merge of W per-rank partials
 * (PR #48196, _dcp_lse_merge, with per-row valid counts).
 *
 *   outs  [W,T,H,512] contiguous (rank r's partial at outs + r*T*H*512), of
 *         element type outs_dtype (MLA_DTYPE_BF16 or MLA_DTYPE_F32)
 *   lses  fp32 [W,T,H] contiguous (natural-log LSE, -inf for empty rows)
 *   valid int32 [W,T] per-row key counts, or NULL.  Rank w takes part in row t
 *         iff valid[w*T+t] > 0 (with NULL: iff its lse is > -inf).  What a
 *         rank that does not take part holds never reaches the result; with
 *         counts given its partial and LSE are not even read (without counts
 *         every rank's row is read and its LSE decides).
 *   out   bf16 [T,H,512]:  out = sum_w exp(lse_w - LSE) * outs_w
 *   out_lse fp32 [T,H] or NULL:  LSE = ln sum_w exp(lse_w)
 * A row with no participating rank gets out = 0 and LSE = -inf.
 * Returns MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE (W<1, T<0, H outside [1,128],
 * outs_dtype not one of the two), MLA_ERR_UNSUPPORTED or MLA_ERR_HIP; T == 0
 * is a no-op.
 */
mla_status mla_lse_merge(const void* outs, int32_t outs_dtype, const float* lses, const int32_t* valid,
                         int32_t W, int32_t T, int32_t H,
                         void* out, float* out_lse, void* hip_stream);

/*
 * mla_merge_v_up_proj -- the merge fused with the per-head W_UV up-projection
 * (PR #48196, _dcp_merge_and_v_up_proj; exact because the merge is linear in
 * the partials and the projection is linear).
 *
 *   outs, outs_dtype, lses, valid, W, T, H   as in mla_lse_merge
 *   W_UV  bf16 [H,512,128] contiguous:  y[t,h,:] = merged_out[t,h,:] @ W_UV[h]
 *   out   bf16 [T,H,128] contiguous
 *   out_lse fp32 [T,H] or NULL
 * The merged latent row is rounded to bf16 before the projection (fp32
 * accumulation).  Returns as mla_lse_merge.
 */
mla_status mla_merge_v_up_proj(const void* outs, int32_t outs_dtype, const float* lses, const int32_t* valid,
                               int32_t W, int32_t T, int32_t H, const void* W_UV,
                               void* out, float* out_lse, void* hip_stream);

/*
 * mla_dcp_a2a_pack -- one rank's side of the projected exchange before the
 * merge (PR #48196: each rank projects its partial through W_UV before the
 * all-to-all, and empty rows are handled in the pack from the valid counts).
 * Destination q owns the contiguous heads q*Hs .. q*Hs+Hs-1, Hs = H / cp_world.
 *
 *   out_r   [T,H,512] contiguous: this rank's partial (mla_decode_partial), of
 *           element type out_dtype (MLA_DTYPE_BF16 or MLA_DTYPE_F32)
 *   lse_r   fp32 [T,H]
 *   valid_r int32 [T] this rank's per-row counts, or NULL (then a row takes part
 *           iff its lse is > -inf).  A row that takes no part is sent as y = 0,
 *           lse = -inf and its partial is not read.
 *   W_UV    bf16 [H,512,128] contiguous
 *   send_y  bf16 [cp_world,T,Hs,128]: send_y[q,t,j] = out_r[t,qHs+j] @ W_UV[qHs+j]
 *           (fp32 accumulation, rounded to bf16)
 *   send_lse fp32 [cp_world,T,Hs]
 * Requires H % cp_world == 0.  Returns MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE,
 * MLA_ERR_UNSUPPORTED or MLA_ERR_HIP; T == 0 is a no-op.
 */
mla_status mla_dcp_a2a_pack(const void* out_r, int32_t out_dtype, const float* lse_r, const int32_t* valid_r,
                            int32_t T, int32_t H, int32_t cp_world, const void* W_UV,
                            void* send_y, float* send_lse, void* hip_stream);

/*
 * mla_dcp_a2a_combine -- the receiving rank's side: the LSE-weighted merge of
 * the cp_world projected slices it received (one from every rank, its own
 * included), rows of 128 values.
 *
 *   recv_y   bf16: source s's slice [T,Hs,128] (contiguous) at
 *            recv_y + s*recv_y_stride elements (stride >= T*Hs*128, a multiple of 8)
 *   recv_lse fp32: source s's [T,Hs] at recv_lse + s*recv_lse_stride (>= T*Hs)
 *   out      bf16 [T,Hs,128]:  out = sum_s exp(lse_s - LSE) * y_s over the
 *            sources whose lse is > -inf
 *   out_lse  fp32 [T,Hs] or NULL:  LSE = ln sum_s exp(lse_s)
 * A row no source takes part in gets out = 0 and LSE = -inf.  The strides let
 * the slices sit wherever the transport put them (for example every rank's
 * send buffer in one allocation).  Returns MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE,
 * MLA_ERR_UNSUPPORTED or MLA_ERR_HIP; T == 0 is a no-op.
 */
mla_status mla_dcp_a2a_combine(const void* recv_y, int64_t recv_y_stride, const float* recv_lse,
                               int64_t recv_lse_stride, int32_t cp_world, int32_t T, int32_t Hs,
                               void* out, float* out_lse, void* hip_stream);

/*
 * mla_dcp_local_seqlens -- the per-row, per-rank seqlen_k of the DCP mask
 * (PR #24453 review thread; shard layout with runs of cp_interleave tokens as
 * for mla_decode_partial), computed on the device by the same device function
 * the decode kernel uses.  row_seqlen int32 [T] (row t's visible key
 * count on rank cp_rank under mask_mode; usable directly as `valid[cp_rank]`
 * of the merge) and
 * shard_len int32 [B] (request b's tokens stored on the rank), either may be
 * NULL.  Returns MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED or
 * MLA_ERR_HIP.
 */
mla_status mla_dcp_local_seqlens(const int32_t* seq_lens, const int32_t* query_start_loc,
                                 int32_t B, int32_t T, int32_t cp_world, int32_t cp_rank,
                                 int32_t cp_interleave, int32_t mask_mode, int32_t* row_seqlen,
                                 int32_t* shard_len, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
