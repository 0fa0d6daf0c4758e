/*
 * libmla_decode: absorbed-weight sparse multi-head latent attention decode
 * step for MI355X (gfx950), as a C ABI.
 *
 * The step (DeepSeek-V3.2-Exp pages, decode mode):
 *   1. mla_absorb_q       q~[b,h,:] = q_nope[b,h,:] W_UK,h          (128 -> 512)
 *      "Query-key similarity" page, decode-branch code excerpt: the query is
 *      absorbed through the first 128 rows of each head's wkv_b slice.
 *   2. mla_sparse_decode  s[b,h,t] = scale * (q~ . c[b,t] + q_pe . k_pe[b,t])
 *      over the selected positions only, softmax over keys, and the latent
 *      mix O~[b,h,:] = sum_t A[b,h,t] c[b,t,:]
 *      "Query-key similarity" page, formula S_i and the index mask in the code
 *      excerpt (-inf off the indexer's selection, shared by all heads);
 *      "Softmax" page, formula for A (normalisation over key positions).
 *   3. mla_combine        merges split-K partials of step 2 (log-sum-exp).
 *   4. mla_value_up       O[b,h,:] = O~[b,h,:] W_UV,h^T               (512 -> 128)
 *      "Apply value weights" page, formula O_i = O~_i W_UV,i.
 *
 * Fixed dimensions (Queries page, init excerpt and shapes): 128 heads,
 * 128 non-rotary and 64 rotary query dims (qk_head_dim 192), latent rank 512,
 * value dim 128.  wkv_b is the [128*256, 512] matrix of the key-value
 * up-projection; per head h, rows h*256 .. h*256+127 are W_UK,h and rows
 * h*256+128 .. h*256+255 are W_UV,h, each stored [d][c] with c contiguous.
 *
 * Conventions
 *  - bf16 tensors are passed as raw 16-bit storage (void*).  All strides are
 *    in elements.  Every tensor pointer is GPU device memory owned by the
 *    caller; the library allocates and frees nothing and keeps no pointer
 *    after a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and never synchronise.  Inputs must not alias outputs.
 *  - Every entry point returns MLA_OK (0) or a positive mla_status.  Argument
 *    errors are detected on the host before anything is enqueued.  No C++
 *    exception crosses this interface and the library never aborts.
 *  - The library is reentrant.  Its only global state is the static scratch
 *    array of mla_sparse_decode_noalloc (one per GPU, with its address looked
 *    up once per device).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2

#define MLA_HEADS 128
#define MLA_NOPE_DIM 128
#define MLA_ROPE_DIM 64
#define MLA_LATENT_DIM 512
#define MLA_VALUE_DIM 128

/* Most index slots one split may hold in sparse mode (indices != NULL). */
#define MLA_MAX_SLOTS_PER_SPLIT 2048
#define MLA_MAX_SPLITS 64

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL                     */
  MLA_ERR_BAD_DIM = 2,             /* B, k_max, max_len or splits invalid */
  MLA_ERR_ALIGNMENT = 3,           /* base not 16-byte aligned / stride not 8 elements */
  MLA_ERR_WORKSPACE_TOO_SMALL = 4, /* ws_bytes below what the call's *_workspace_bytes gives */
  MLA_ERR_UNSUPPORTED = 5,         /* a stride too small for the fixed row widths, or a head count other than 16/32/64/128 */
  MLA_ERR_HIP = 6,                 /* a HIP call failed: see mla_last_hip_error()     */
  MLA_ERR_RANGE = 7,               /* one sequence's cache or q_pe span exceeds 2 GiB */
  MLA_ERR_SCRATCH_LIMIT = 8        /* partials larger than the static scratch (noalloc) */
} mla_status;

/* Flags of mla_sparse_decode. */
#define MLA_FLAG_VALIDATE 1u      /* range/duplicate/empty checks + attended bitmap */
#define MLA_FLAG_WRITE_SCORES 2u  /* write the scaled scores of every index slot   */

/* Bits OR-ed into *status_dev by the device-side checks (MLA_FLAG_VALIDATE). */
#define MLA_DEV_INDEX_OUT_OF_RANGE 1u /* an index >= L_b, or negative and not -1 */
#define MLA_DEV_DUPLICATE_INDEX 2u    /* a position appears twice in one row     */
#define MLA_DEV_EMPTY_SELECTION 4u    /* a sequence selects no position          */

int mla_abi_version(void);
const char* mla_status_string(int status);
/* The hipError_t of the most recent MLA_ERR_HIP on this thread (0 if none). */
int mla_last_hip_error(void);

/*
 * Launch plan for mla_sparse_decode: how many key splits per sequence (one
 * workgroup per (sequence, split), each covering all 128 heads).
 * `dense` is nonzero when no index list is passed.  num_cus <= 0 means 256.
 * Pure host function.  Returns MLA_ERR_BAD_DIM for B < 1 or k_max < 1.
 */
int mla_plan(int32_t B, int32_t k_max, int32_t dense, int32_t num_cus, int32_t* num_splits);

/*
 * Bytes of workspace mla_sparse_decode needs for `num_splits` splits: 0 when
 * num_splits == 1 (the normalised result is written directly), otherwise the
 * per-split unnormalised latent sums sum_t 2^(u_t - m_s) c_t, bf16
 * [S][B][128][512], followed by the per-split (m_s, l_s = sum_t 2^(u_t - m_s))
 * pairs, fp32 [S][B][128][2]; u_t is the score in log2 units and m_s the
 * split's reference maximum (within 8 of its largest u_t; -inf for no key).
 * Returns 0 for invalid arguments.
 */
size_t mla_workspace_bytes(int32_t B, int32_t num_splits);

/*
 * Step 1: q_abs[b][h][c] = sum_d q_nope[b][h][d] * W_UK,h[d][c].
 *   q_nope  bf16, element (b, h, d) at q_nope[b*q_nope_sb + h*q_nope_sh + d]
 *           (d contiguous; the [B,1,128,128] layout has sb = 16384, sh = 128).
 *   wkv_b   bf16 [32768][512], contiguous.
 *   q_abs   bf16 [B][128][512], contiguous (written).
 * Requires 1 <= B <= 65536, 16-byte aligned bases, strides multiples of 8,
 * non-negative strides and (B - 1) * q_nope_sb * 2 + 256 below 4 GiB
 * (MLA_ERR_RANGE).  fp32 accumulation, one rounding to bf16.
 */
int mla_absorb_q(const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh,
                 const void* wkv_b, void* q_abs, int32_t B, void* stream);

/*
 * Step 2: sparse flash-decode over the selected cache rows.
 *   q_abs    bf16 [B][128][512] contiguous (from mla_absorb_q).
 *   q_pe     bf16, element (b, h, r) at q_pe[b*q_pe_sb + h*q_pe_sh + r], r < 64.
 *   kv       latent cache: row (b, t) at kv + b*kv_sb + t*kv_st, 512 values.
 *   pe       rotary-key cache: row (b, t) at pe + b*pe_sb + t*pe_st, 64 values.
 *            Two buffers as in the pages' code, or one packed 576-value row
 *            (pe = kv + 512, pe_st = kv_st) -- both are plain strides here.
 *   seq_lens int32 [B], device: L_b, the cached positions of sequence b
 *            (clamped to [0, max_len]).
 *   max_len  host upper bound on every L_b.
 *   indices  int32 [B][k_max], device, any order: the selected positions of
 *            each sequence, shared by all heads; -1 is padding and is skipped.
 *            Positions must be distinct and < L_b (a top-k's output).  NULL
 *            selects every t < L_b (dense decode; then k_max >= max_len).
 *   k_max    index slots per sequence.
 *   scale    softmax scale (qk_head_dim^-1/2 for this model).
 *   num_splits  from mla_plan (1 <= S <= 64).  Split s takes index slots
 *            [s * chunk, (s + 1) * chunk), chunk = ceil(k_max / S) rounded up
 *            to 32; in sparse mode chunk <= MLA_MAX_SLOTS_PER_SPLIT.
 *   workspace, ws_bytes       device scratch, >= mla_workspace_bytes(B, S);
 *            unused (may be NULL) when S == 1.
 *   o_latent bf16 [B][128][512], lse fp32 [B][128] (natural log; may be NULL):
 *            written here when S == 1, by mla_combine when S > 1.
 *   flags    MLA_FLAG_*.
 *   attended_bitmap uint32 [B][bitmap_words], zeroed by the caller: with
 *            VALIDATE, bit t of row b is set for every selected in-range
 *            position (written by the gather itself).  bitmap_words >=
 *            ceil(max_len / 32).
 *   scores_out fp32 [B][128][k_max]: with WRITE_SCORES, scale * (q~ . c +
 *            q_pe . k_pe) of each slot's position, -inf for masked slots.
 *   status_dev uint32, device, zeroed by the caller: MLA_DEV_* bits (VALIDATE).
 * Without VALIDATE, rows with repeated indices are attended once per repeat
 * and out-of-range indices are skipped; both are caller errors.
 * Each sequence's cache span (max_len * row stride * 2 bytes, for kv and pe)
 * and its q_pe span ((127 * q_pe_sh + 64) * 2 bytes) must be below 2 GiB
 * (MLA_ERR_RANGE).
 */
int mla_sparse_decode(const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                      const void* kv, int64_t kv_sb, int64_t kv_st,
                      const void* pe, int64_t pe_sb, int64_t pe_st,
                      const int32_t* seq_lens, int32_t max_len,
                      const int32_t* indices, int32_t k_max, float scale, int32_t B,
                      int32_t num_splits, void* workspace, size_t ws_bytes,
                      void* o_latent, float* lse,
                      uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                      float* scores_out, uint32_t* status_dev, void* stream);

/*
 * Step 2 (and 3) for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same decode as mla_sparse_decode, with the same arguments except that
 * there is no workspace.  With num_splits > 1 the split partials go to a
 * static device array inside the library (mla_noalloc_scratch_bytes() bytes
 * per GPU, held until the process ends) and this call also merges them, as
 * mla_combine does, into o_latent and lse; with num_splits == 1 it is
 * mla_sparse_decode.  It calls no allocator.
 * Errors: those of mla_sparse_decode, and MLA_ERR_SCRATCH_LIMIT when
 * mla_workspace_bytes(B, num_splits) exceeds the scratch (40 MiB: e.g.
 * B = 64 with 4 splits needs 33.8 MB).  The first call on a device looks up
 * the scratch address (MLA_ERR_HIP if that fails).
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller.  Nothing in the scratch needs clearing between calls: the
 * decode overwrites every partial it merges.
 */
size_t mla_noalloc_scratch_bytes(void);
int mla_sparse_decode_noalloc(const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                              const void* kv, int64_t kv_sb, int64_t kv_st,
                              const void* pe, int64_t pe_sb, int64_t pe_st,
                              const int32_t* seq_lens, int32_t max_len,
                              const int32_t* indices, int32_t k_max, float scale, int32_t B,
                              int32_t num_splits, void* o_latent, float* lse,
                              uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                              float* scores_out, uint32_t* status_dev, void* stream);

/*
 * Step 3: merge the S partials of step 2 ("Softmax" page: the normalisation
 * over all selected keys, assembled from per-split maxima and sums):
 *   O~ = sum_s w_s acc_s / sum_s w_s l_s,  w_s = 2^(m_s - max_s m_s),
 *   lse = ln 2 * (max_s m_s + log2 sum_s w_s l_s).
 * A no-op returning MLA_OK when num_splits == 1.  An empty selection gives
 * NaN in o_latent and -inf in lse; with status_dev non-NULL it also sets
 * MLA_DEV_EMPTY_SELECTION.
 */
int mla_combine(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                void* o_latent, float* lse, uint32_t* status_dev, void* stream);

/*
 * Step 4: out[b][h][d] = sum_c o_latent[b][h][c] * W_UV,h[d][c].
 *   o_latent bf16 [B][128][512] contiguous; wkv_b as in mla_absorb_q;
 *   out bf16, element (b, h, d) at out[b*out_sb + h*out_sh + d] (the
 *   [B,1,128,128] layout has sb = 16384, sh = 128).
 * fp32 accumulation, one rounding to bf16.
 */
int mla_value_up(const void* o_latent, const void* wkv_b, void* out,
                 int64_t out_sb, int64_t out_sh, int32_t B, void* stream);

/*
 * Steps 3 and 4 in one launch, for num_splits >= 2: the value-up of step 4
 * reads its O~ operand merged on the fly from the split partials in
 * `workspace` (the same merge as mla_combine), so O~ is never stored.
 * out as in mla_value_up; lse fp32 [B][128] (may be NULL); status_dev as in
 * mla_combine (may be NULL).  MLA_ERR_RANGE when the partials' (max, sum)
 * array (num_splits * B * 128 * 8 bytes) exceeds 2 GiB.
 */
int mla_combine_value_up(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                         const void* wkv_b, void* out, int64_t out_sb, int64_t out_sh, float* lse,
                         uint32_t* status_dev, void* stream);

/*
 * Head-sharded step: the same calls for one GPU's share of the heads when
 * the heads are split across GPUs ("Queries" page, init excerpt: wkv_b is a
 * column-parallel layer and each rank holds n_local_heads heads; the decode
 * excerpt on the "Query-key similarity" page views wkv_b per local head).
 * n_heads is 16, 32, 64 or 128 (MLA_ERR_UNSUPPORTED otherwise) and every
 * per-head array has n_heads heads: q_nope [B, n_heads, 128] and q_pe
 * [B, n_heads, 64] (strides as in the 128-head calls), wkv_b
 * [n_heads*256][512] (the rank's rows of the weight), q_abs and o_latent
 * [B][n_heads][512], lse [B][n_heads], scores_out [B][n_heads][k_max], out
 * [B, n_heads, 128], workspace >= mla_workspace_bytes_heads(n_heads, B, S).
 * The selection and the latent cache are shared by all heads, so every rank
 * reads every selected row; the decode launches the same workgroups as for
 * 128 heads.  Otherwise each call is the 128-head call of the same name.
 */
size_t mla_workspace_bytes_heads(int32_t n_heads, int32_t B, int32_t num_splits);
int mla_absorb_q_heads(int32_t n_heads, const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh,
                       const void* wkv_b, void* q_abs, int32_t B, void* stream);
int mla_sparse_decode_heads(int32_t n_heads, const void* q_abs, const void* q_pe, int64_t q_pe_sb, int64_t q_pe_sh,
                            const void* kv, int64_t kv_sb, int64_t kv_st,
                            const void* pe, int64_t pe_sb, int64_t pe_st,
                            const int32_t* seq_lens, int32_t max_len,
                            const int32_t* indices, int32_t k_max, float scale, int32_t B,
                            int32_t num_splits, void* workspace, size_t ws_bytes,
                            void* o_latent, float* lse,
                            uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                            float* scores_out, uint32_t* status_dev, void* stream);
int mla_combine_heads(int32_t n_heads, const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                      void* o_latent, float* lse, uint32_t* status_dev, void* stream);
int mla_value_up_heads(int32_t n_heads, const void* o_latent, const void* wkv_b, void* out, int64_t out_sb,
                       int64_t out_sh, int32_t B, void* stream);
int mla_combine_value_up_heads(int32_t n_heads, const void* workspace, size_t ws_bytes, int32_t B,
                               int32_t num_splits, const void* wkv_b, void* out, int64_t out_sb, int64_t out_sh,
                               float* lse, uint32_t* status_dev, void* stream);

/*
 * Sparse prefill ("Queries" page, prefill mode, mla-prefill excerpt): for
 * every query token s of a prompt of T tokens, attention over the prompt's
 * own positions t <= s (the causal mask) that the indexer selected for that
 * token (the index mask), per head, with keys [W_UK,h c_t | k_pe_t] and
 * values W_UV,h c_t:
 *   O[b,s,h,:] = sum_t softmax_t(scale * (q_nope[b,s,h] . W_UK,h c_t +
 *                                q_pe[b,s,h] . k_pe_t)) W_UV,h c_t.
 * Computed in the absorbed form, which equals it exactly in real arithmetic
 * (the "Apply value weights" page, Explanation): mla_absorb_q over the B*T
 * query rows, the sparse attention of mla_sparse_decode with row r = token
 * r % T of prompt r / T attending the prompt's latent rows up to its own
 * position, then the merge and value-up -- three launches on `stream`.
 *   q_nope  bf16, element (r, h, d) at q_nope[r*q_nope_st + h*q_nope_sh + d]
 *           for the query rows r = b*T + s ([B,T,128,128] contiguous has
 *           st = 16384, sh = 128); q_pe likewise with 64 values.
 *   kv, pe  latent and rotary key of position t of prompt b at
 *           kv + b*kv_sb + t*kv_st and pe + b*pe_sb + t*pe_st (t < T).
 *   wkv_b   bf16 [32768][512] as in mla_absorb_q.
 *   indices int32 [B*T][k_max]: the selection of each query token, any
 *           order, -1 padding; entries t with s < t < T are removed by the
 *           causal mask; NULL selects every causal key (then k_max >= T).
 *   num_splits  key splits per query row (mla_plan(B*T, k_max, ...)).
 *   workspace   >= mla_prefill_workspace_bytes(B, T, num_splits) bytes.
 *   out     bf16, element (r, h, d) at out[r*out_st + h*out_sh + d].
 *   lse     fp32 [B*T][128] (natural log), may be NULL.
 *   flags   MLA_FLAG_VALIDATE only (attended_bitmap [B*T][bitmap_words],
 *           bitmap_words >= ceil(T / 32), zeroed by the caller; status_dev:
 *           an index >= T or below -1 sets MLA_DEV_INDEX_OUT_OF_RANGE);
 *           MLA_FLAG_WRITE_SCORES returns MLA_ERR_BAD_DIM.
 * Requires 1 <= B*T <= 65536 and the alignment and span rules of
 * mla_absorb_q and mla_sparse_decode.
 */
size_t mla_prefill_workspace_bytes(int32_t B, int32_t T, int32_t num_splits);
int mla_sparse_prefill(const void* q_nope, int64_t q_nope_st, int64_t q_nope_sh,
                       const void* q_pe, int64_t q_pe_st, int64_t q_pe_sh,
                       const void* kv, int64_t kv_sb, int64_t kv_st,
                       const void* pe, int64_t pe_sb, int64_t pe_st,
                       const void* wkv_b, const int32_t* indices, int32_t k_max, float scale,
                       int32_t B, int32_t T, int32_t num_splits, void* workspace, size_t ws_bytes,
                       void* out, int64_t out_st, int64_t out_sh, float* lse,
                       uint32_t flags, uint32_t* attended_bitmap, int64_t bitmap_words,
                       uint32_t* status_dev, void* stream);

/*
 * One-time set-up ("Query-key similarity" page, code excerpt: a quantised
 * wkv_b is dequantised once and the dense copy reused):
 *   w_bf16[i][j] = bf16(e4m3(w_fp8[i][j]) * scales[i/128][j/128]), rounded to
 * nearest even from the exact product.
 *   w_fp8   uint8 [32768][512] OCP E4M3FN codes; scales fp32 [256][4];
 *   w_bf16  bf16 [32768][512] (written).
 */
int mla_dequant_wkv_b_fp8(const void* w_fp8, const float* scales, void* w_bf16, void* stream);

/*
 * Steps 1 and 4 reading the block-scaled fp8 weight directly instead of a
 * bf16 copy ("Query-key similarity" page, code excerpt: a quantised wkv_b is
 * dequantised through its block scale before the absorption).  Each call
 * dequantises the slices it uses in registers, to exactly the values
 * mla_dequant_wkv_b_fp8 writes (bf16 rounded to nearest even from the exact
 * product e4m3(w[i][j]) * scale[i/128][j/128]), and so reads 16.8 MB of
 * weight codes per step instead of 33.5 MB of bf16.
 *   w_fp8    uint8 [32768][512] OCP E4M3FN codes, 16-byte aligned.
 *   w_scale  fp32 [256][4] block scales, 4-byte aligned.
 *   w_formed NULL, or bf16 [32768][512] (16-byte aligned): a test hook; the
 *            call also writes the weights exactly as it formed them in
 *            registers (the W_UK rows for absorb, the W_UV rows for value-up).
 * The other arguments, the results and the errors are those of mla_absorb_q,
 * mla_value_up and mla_combine_value_up.
 */
int mla_absorb_q_fp8(const void* q_nope, int64_t q_nope_sb, int64_t q_nope_sh, const void* w_fp8,
                     const float* w_scale, void* q_abs, int32_t B, void* w_formed, void* stream);
int mla_value_up_fp8(const void* o_latent, const void* w_fp8, const float* w_scale, void* out,
                     int64_t out_sb, int64_t out_sh, int32_t B, void* w_formed, void* stream);
int mla_combine_value_up_fp8(const void* workspace, size_t ws_bytes, int32_t B, int32_t num_splits,
                             const void* w_fp8, const float* w_scale, void* out, int64_t out_sb, int64_t out_sh,
                             float* lse, uint32_t* status_dev, void* stream);

/*
 * Output projection, the step after the value-up ("Attention update" page,
 * mla-output excerpt: the head outputs are flattened per sequence and the
 * output linear layer maps them to the model width):
 *   out[b][o] = sum_i x[b][i] * wo[o][i],  i < 16384 = 128 heads x 128, o < 7168.
 *   x    bf16 [B][x_sb]: row b's first 16384 values are head h's 128 outputs
 *        at 128 h .. (the [B][1][128][128] value-up output, contiguous, has
 *        x_sb = 16384); x_sb >= 16384, a multiple of 8; 16-byte aligned.
 *   wo   bf16 [7168][16384], contiguous (a linear layer's weight), 16-byte aligned.
 *   out  bf16 [B][out_sb], out_sb >= 7168: the first 7168 values of each row
 *        are written; 2-byte aligned.
 * fp32 accumulation, one rounding to bf16.  Launches one kernel per 64 rows
 * of the batch.  Errors: MLA_ERR_NULL_POINTER, MLA_ERR_BAD_DIM (B outside
 * 1 .. 65536, a row stride below the row width), MLA_ERR_ALIGNMENT,
 * MLA_ERR_RANGE ((63 * x_sb + 16384) * 2 bytes must stay below 4 GiB),
 * MLA_ERR_HIP.
 */
int mla_output_proj(const void* x, int64_t x_sb, const void* wo, void* out, int64_t out_sb, int32_t B,
                    void* stream);

/*
 * The output projection on a repacked weight (the same "Attention update"
 * passage; a layout of the same linear weight, made once at set-up like the
 * fp8 dequantisation).  mla_output_proj reads, per chunk of 256 inputs, a
 * 512-byte piece of each of 7168 weight rows 32 KB apart; the packed layout
 * stores each group of 28 output rows chunk by chunk, so the same bytes are
 * read as one contiguous stream per group.  Since the workgroups of
 * mla_output_proj start their walk over the inputs at different chunks, the
 * two reach about the same rate at every batch (measured within a few
 * percent either way).
 *   mla_output_proj_pack: wo_packed[g][c][r][k] = wo[28 g + r][256 c + k]
 *     for g < 256, c < 64, r < 28, k < 256; wo and wo_packed bf16, 7168 x 16384
 *     elements each (235 MB), 16-byte aligned, not overlapping.
 *   mla_output_proj_packed: arguments, results and errors as
 *     mla_output_proj, with wo_packed from mla_output_proj_pack; the result
 *     is bit-identical to mla_output_proj on the unpacked weight.
 */
int mla_output_proj_pack(const void* wo, void* wo_packed, void* stream);
int mla_output_proj_packed(const void* x, int64_t x_sb, const void* wo_packed, void* out, int64_t out_sb,
                           int32_t B, void* stream);

/*
 * The output projection with its inputs split in four (the same "Attention
 * update" passage and result up to fp32 rounding order): each quarter of
 * i = 0 .. 16383 is summed by its own workgroups into an fp32 partial, and a
 * second launch adds the four partials in quarter order and rounds to bf16
 * once.  Each CU then reads a quarter of x instead of all of it, which is
 * what limits mla_output_proj at large batches (measured faster from about
 * 32 rows on; no faster below).
 *   x, wo, out, x_sb, out_sb, B: as mla_output_proj.
 *   workspace  device memory of at least mla_output_proj_split_workspace_bytes(B)
 *              bytes (4 x min(B, 64) x 7168 fp32 partial sums), 16-byte aligned,
 *              owned by the caller; its contents on entry do not matter, and it
 *              must not be in use by another call until this one's launches
 *              have completed on `stream`.
 * Launches two kernels per 64 rows of the batch.  Errors: those of
 * mla_output_proj, MLA_ERR_NULL_POINTER for a NULL workspace, MLA_ERR_ALIGNMENT
 * for a misaligned one, MLA_ERR_WORKSPACE_TOO_SMALL.
 * mla_output_proj_split_workspace_bytes: pure host function; 0 for B outside
 * 1 .. 65536.
 */
size_t mla_output_proj_split_workspace_bytes(int32_t B);
int mla_output_proj_split(const void* x, int64_t x_sb, const void* wo, void* out, int64_t out_sb, int32_t B,
                          void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
