/*
 * mla_decode.h -- C ABI of libmla.so: absorbed ("MQA mode") Multi-head Latent
 * Attention decode on AMD Instinct MI355X (gfx950).
 *
 * The method (itwiki article "Multi-head latent attention", section
 * "Structure"): each token caches only its compressed latent c^KV (d_c values)
 * and one decoupled-RoPE key k^R (d_r values) shared by all heads.  In MQA
 * mode the key up-projection W^UK is folded into the query, every head's
 * latent query is dotted directly with the cached c^KV, the position term
 * q^R . k^R is added, scores are scaled by 1/sqrt(d_h + d_h^R) and softmaxed
 * causally, the softmax weights sum the c^KV rows, and W^UV is applied to that
 * latent output afterwards.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains memory; it keeps no state between calls
 *    apart from a per-device cache of kernel attributes (compute-unit count,
 *    raised LDS limits).  Whatever one call leaves for a later one (a split
 *    plan, partial results) lives in a caller-owned workspace.
 *  - Every call enqueues work on `stream` (a hipStream_t passed as void*; NULL
 *    is the default stream) and returns without synchronising.
 *  - Tensors are row-major with the last dimension contiguous.  Strides are
 *    in elements.
 *  - Return value: MLA_OK or a negative MLA_ERR_* code.  On an error return
 *    nothing has been enqueued, except for MLA_ERR_LAUNCH, which reports a
 *    failed kernel launch (hipGetLastError) and may leave earlier kernels of
 *    the same call enqueued.
 *  - Weights follow the nn.Linear storage convention [out, in]:
 *    W^UK and W^UV are [n_h*d_h, d_c]; head i owns rows i*d_h .. (i+1)*d_h-1.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define MLA_F32 0      /* IEEE binary32 */
#define MLA_BF16 1     /* bfloat16 */
#define MLA_FP8_E4M3 2 /* OCP 8-bit float E4M3 ("fn": max 448, no infinities) */
/* low-bit latent-cache formats (kv_dtype of mla_decode_absorbed only) */
#define MLA_INT4 3     /* 4-bit content codes + 4-bit RoPE codes, grouped fp16 scale/min */
#define MLA_INT2 4     /* 2-bit content codes + 4-bit RoPE codes, grouped fp16 scale/min */

/* status codes */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, bad dtype code */
#define MLA_ERR_UNSUPPORTED (-2) /* valid but not implemented combination */
#define MLA_ERR_MISALIGNED (-3)  /* a pointer/stride breaks the 16-byte alignment rule */
#define MLA_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */
#define MLA_ERR_LAUNCH (-5)      /* the HIP runtime rejected a kernel launch */
#define MLA_ERR_TOO_LARGE (-6)   /* more than the fixed scratch of mla_decode_step_noalloc */

/* flags for mla_decode_absorbed */
#define MLA_FLAG_FORCE_GENERIC 1 /* use the portable fp32 kernel even when the
                                    MFMA kernel applies (for cross-checks) */

/*
 * mla_absorb_q -- fold W^UK into the query (absorption identity
 * q^T W^UK c = (W^UK^T q)^T c; itwiki "Multi-head latent attention", section
 * "Matrix absorption"; lecture "MHA · GQA · MQA · MLA", section "Why
 * Projection Absorption Helps").
 *
 *   q_lat[t, i, c] = sum_k q_nope[t, i, k] * w_uk[i*d_h + k, c]
 *
 *  q_nope  [T_q, n_h, d_h], token stride q_stride_t (>= n_h*d_h), dtype act_dtype
 *  w_uk    [n_h*d_h, d_c],  dtype w_dtype
 *  q_lat   [T_q, n_h, d_c], token stride qlat_stride_t (>= n_h*d_c), dtype out_dtype
 *  act_dtype, w_dtype in {MLA_F32, MLA_BF16}; out_dtype in {MLA_F32, MLA_BF16}.
 *  Accumulation is fp32.  bf16 activations and weights with d_h <= 128 take
 *  the MFMA kernel (which then needs d_h % 16 == 0, d_c % 32 == 0, and
 *  16-byte aligned rows of q_nope, w_uk and q_lat, else MLA_ERR_MISALIGNED);
 *  other combinations take a plain fp32 kernel.  T_q == 0 is a no-op.
 */
int mla_absorb_q(const void* q_nope, int64_t q_stride_t, const void* w_uk, void* q_lat,
                 int64_t qlat_stride_t, int T_q, int n_h, int d_h, int d_c, int act_dtype,
                 int w_dtype, int out_dtype, void* stream);

/*
 * mla_decode_workspace_bytes -- size of the scratch buffer mla_decode_absorbed
 * needs for the given batch shape (split-KV partial outputs, their
 * log-sum-exps and the work list).  max_blocks_per_seq and num_splits as in
 * mla_decode_absorbed.  Uses the current HIP device's compute-unit count.
 * Returns 0 on invalid arguments.
 */
size_t mla_decode_workspace_bytes(int B, int s_q, int n_h, int d_c, int max_blocks_per_seq,
                                  int num_splits);

/*
 * mla_decode_absorbed -- MQA-mode attention of s_q new tokens per sequence
 * over a paged latent cache (itwiki "Multi-head latent attention", sections
 * "Decoupled RoPE" and "Matrix absorption").
 *
 * For sequence b of length L = seq_lens[b], query token i (0 <= i < s_q)
 * sits at position L - s_q + i and sees keys j = 0 .. L - s_q + i:
 *   s[j]  = softmax_scale * (q_lat[b,i,h,:] . c_j + q_rope[b,i,h,:] . kR_j)
 *   o_lat[b,i,h,:] = sum_j softmax(s)[j] * c_j
 *   lse[b,i,h]     = log(sum_j exp(s[j]))          (natural log)
 * The caller passes softmax_scale = 1/sqrt(d_h + d_h^R).
 *
 *  q_lat    [B, s_q, n_h, d_c], dtype q_dtype (MLA_BF16 or MLA_F32), contiguous
 *  q_rope   [B, s_q, n_h, d_r], dtype q_dtype, contiguous
 *  kv_cache paged cache, block_size tokens per block, physical block p at
 *           byte offset p * block_bytes:
 *           kv_dtype MLA_BF16 / MLA_F32: [num_blocks, block_size, d_c + d_r],
 *             each token row = [c^KV | k^R];
 *           kv_dtype MLA_FP8_E4M3: per block [block_size*d_c e4m3fn content |
 *             block_size*d_r bf16 k^R | block_size fp32 per-token scales];
 *             c_j = e4m3(code) * scale_j (the RoPE key stays bf16).
 *           kv_dtype MLA_INT4 / MLA_INT2 (the QuantMLA review's INT4 content +
 *             INT4 RoPE and INT2 content + INT4 RoPE; the grouping and packing
 *             are this library's): per block [block_size x content codes
 *             (d_c*b/8 bytes, b = 4 or 2) | block_size x RoPE codes (d_r/2
 *             bytes) | block_size x (d_c+d_r)/32 pairs (fp16 scale, fp16
 *             min)]; each group of 32 consecutive values of a token (content
 *             groups first, then RoPE groups) decodes as code * scale + min.
 *             Codes are packed in little-endian 32-bit words of 32/b values:
 *             value 2k at bit k*b, value 2k+1 at bit 16 + k*b.  Needs
 *             d_c % 32 == 0 and d_r % 32 == 0.  The MFMA kernel decodes to
 *             fp16 and multiplies fp16 operands (queries and softmax weights
 *             rounded to fp16, fp32 accumulation): queries and decoded values
 *             must lie inside the fp16 range (|x| < 65504); the portable
 *             kernel decodes to fp32.
 *  block_table [B, max_blocks_per_seq] int32: logical block k of sequence b
 *           is physical block block_table[b*max_blocks_per_seq + k].
 *  seq_lens [B] int32 (device).
 *  o_lat    [B, s_q, n_h, d_c], dtype out_dtype (MLA_F32 or MLA_BF16).
 *  lse      [B, s_q, n_h] fp32, or NULL.
 *  num_splits  0 = automatic split-KV planning from the lengths and the
 *           device's compute-unit count; k > 0 = each sequence is cut into
 *           min(k, its block count) contiguous partitions, raised where a
 *           partition would exceed 512 blocks.
 *  workspace   device buffer of at least mla_decode_workspace_bytes(...)
 *           bytes; its contents need no initialisation and are clobbered.
 *  flags    0 or MLA_FLAG_FORCE_GENERIC.
 *
 * Kernel selection: bf16 queries, a bf16, fp8, int4 or int2 cache, n_h == 128,
 * d_c == 512, d_r == 64, block_size == 64 and 16-byte aligned cache/query
 * pointers take the MFMA kernel; everything else (fp32, other shapes) takes a
 * portable fp32 kernel.  Constraints: 1 <= s_q <= 16, d_c <= 2048, d_r <= 256,
 * d_c % 4 == 0.
 * Device-side preconditions (not checked, they would need a synchronisation):
 *   s_q <= seq_lens[b] <= max_blocks_per_seq*block_size, and every table
 *   entry a sequence uses names a valid block.  Slots of the last block past
 *   seq_lens[b] are never read into the result (they may hold NaN).
 * Concurrent calls must use distinct workspaces.
 */
int mla_decode_absorbed(const void* q_lat, const void* q_rope, const void* kv_cache,
                        const int32_t* block_table, int max_blocks_per_seq,
                        const int32_t* seq_lens, int B, int s_q, int n_h, int d_c, int d_r,
                        int block_size, float softmax_scale, int q_dtype, int kv_dtype,
                        int out_dtype, int num_splits, void* workspace, size_t workspace_bytes,
                        void* o_lat, float* lse, int flags, void* stream);

/*
 * mla_combine_lse -- merge split-KV partial results (log-sum-exp combine):
 *   lse[n] = log sum_s exp(lse_part[n,s]),
 *   out[n,:] = sum_s exp(lse_part[n,s] - lse[n]) * o_part[n,s,:]
 * Each o_part[n,s,:] is normalised over its own keys.  Splits with
 * lse_part = -inf carry no weight; a row whose splits are all -inf gets
 * out = 0, lse = -inf.
 *
 *  o_part   [N, S, D] fp32
 *  lse_part [N, S] fp32
 *  splits_per_row [N] int32 (device) with 0 <= value <= S, or NULL for S
 *  out      [N, D], dtype out_dtype (MLA_F32 or MLA_BF16)
 *  lse_out  [N] fp32, or NULL
 *  Requires D % 4 == 0 and 16-byte aligned o_part/out.  N == 0 is a no-op.
 */
int mla_combine_lse(const float* o_part, const float* lse_part, const int32_t* splits_per_row,
                    int N, int S, int D, void* out, float* lse_out, int out_dtype, void* stream);

/*
 * mla_up_proj_v -- apply W^UV after the weighted latent sum (itwiki
 * "Multi-head latent attention", section "Matrix absorption"):
 *
 *   o[t, i, k] = sum_c w_uv[i*d_h + k, c] * o_lat[t, i, c]
 *
 *  o_lat [T_q, n_h, d_c], token stride olat_stride_t, dtype act_dtype
 *  w_uv  [n_h*d_h, d_c], dtype w_dtype
 *  o     [T_q, n_h, d_h], token stride o_stride_t, dtype out_dtype
 *  bf16 activations and weights take the MFMA kernel (needs d_c % 64 == 0,
 *  d_c <= 512, d_h % 32 == 0, 16-byte aligned o_lat/w_uv rows, and o
 *  aligned to two elements with an even o_stride_t, else
 *  MLA_ERR_MISALIGNED); other combinations a plain fp32 kernel.
 *  Accumulation is fp32.  T_q == 0 is a no-op.
 */
int mla_up_proj_v(const void* o_lat, int64_t olat_stride_t, const void* w_uv, void* o,
                  int64_t o_stride_t, int T_q, int n_h, int d_c, int d_h, int act_dtype,
                  int w_dtype, int out_dtype, void* stream);

/* mla_cache_append -- the cache producer, the step before decode (itwiki
 * "Multi-head latent attention", sections "Joint KV compression" and
 * "Decoupled RoPE"): for each new token t
 *     c^KV_t = W^DKV h_t,   k^R_t = RoPE(W^KR h_t, positions[t])
 * written into the paged cache at slot slot_mapping[t]: block slot/block_size,
 * row slot%block_size.  A negative slot skips the token (padding).
 *
 *  h            [T, d], token stride h_stride_t (elements), dtype in_dtype
 *               (MLA_F32 or MLA_BF16)
 *  w_dkv_kr     [d_c + d_r, d], dtype in_dtype: the d_c rows of W^DKV then
 *               the d_r rows of W^KR ([out, in])
 *  positions    [T] int32, the tokens' positions in their sequences
 *  slot_mapping [T] int32, physical slot or < 0
 *  kv_cache     the cache mla_decode_absorbed reads, kv_dtype MLA_F32 /
 *               MLA_BF16 rows [d_c | d_r], or MLA_FP8_E4M3 blocks (needs
 *               in_dtype MLA_BF16, d_c % 16 == 0, d_r % 8 == 0): the content
 *               is stored as e4m3fn codes of c / s with s = amax|c| / 448 as
 *               fp32 (1 for an all-zero row), round to nearest even; k^R bf16.
 *  rope_base    RoPE base (pairs (x_k, x_{k+d_r/2}) rotated by
 *               positions[t] * rope_base^(-2k/d_r); angles in fp64); d_r <= 128
 *  workspace    >= mla_cache_append_workspace_bytes(T, d, d_c, d_r) bytes,
 *               16-byte aligned, caller-owned (fp32 partial sums).
 * Accumulation is fp32; stored rows round to nearest even.  bf16 inputs with
 * d % 512 == 0, (d_c + d_r) % 32 == 0 and 16-byte aligned rows take the MFMA
 * projection, everything else a plain fp32 kernel.  Two tokens mapping to
 * the same slot race.  T == 0 is a no-op. */
int mla_cache_append(const void* h, int64_t h_stride_t, const void* w_dkv_kr, const int32_t* positions,
                     const int32_t* slot_mapping, void* kv_cache, int T, int d, int d_c, int d_r,
                     int block_size, float rope_base, int in_dtype, int kv_dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* mla_cache_append_workspace_bytes -- workspace size for mla_cache_append
 * (0 for invalid sizes). */
size_t mla_cache_append_workspace_bytes(int T, int d, int d_c, int d_r);

/* mla_decode_step -- one whole absorbed decode step in three launches
 * (itwiki "Multi-head latent attention", section "Matrix absorption"):
 * q_lat = W^UK_h^T q_nope (as mla_absorb_q), the attention of
 * mla_decode_absorbed over the paged cache, and the split-KV merge fused
 * with o = W^UV_h o_lat (as mla_up_proj_v).  Same results as those three
 * calls with bf16 q_lat / o_lat, without the o_lat round trip through memory.
 *
 *  q_nope [B, s_q, n_h, d_h] bf16, q_rope [B, s_q, n_h, d_r] bf16, contiguous
 *  w_uk, w_uv [n_h*d_h, d_c] bf16 ([out, in], head h = rows h*d_h ..)
 *  kv_cache, block_table, seq_lens, kv_dtype, num_splits: as mla_decode_absorbed
 *  o [B, s_q, n_h, d_h] bf16; lse [B, s_q, n_h] fp32 or NULL
 *  workspace >= mla_decode_step_workspace_bytes(...), 16-byte aligned
 * Needs the MFMA path of mla_decode_absorbed (n_h = 128, d_c = 512,
 * d_r = 64, block_size = 64, kv bf16 / fp8 / int4 / int2) and d_h = 128,
 * else MLA_ERR_UNSUPPORTED; all pointers 16-byte aligned. */
int mla_decode_step(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                    const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens, const void* w_uv,
                    int B, int s_q, int n_h, int d_h, int d_c, int d_r, int block_size, float softmax_scale,
                    int kv_dtype, int num_splits, void* workspace, size_t workspace_bytes, void* o, float* lse,
                    void* stream);

/* mla_decode_step_stages -- mla_decode_step one stage (or several) per
 * call, for callers that put their own work or timing between the stages:
 *   MLA_STAGE_ABSORB  q_lat = W^UK_h^T q_nope into the workspace, with the
 *                     split plan of the batch (from seq_lens)
 *   MLA_STAGE_ATTEND  the attention kernel over the paged cache: partial rows
 *                     of split sequences, final latent rows of unsplit ones
 *                     and their lse, all in the workspace (lse also in `lse`)
 *   MLA_STAGE_MERGE   merge of the partitions fused with o = W^UV_h o_lat
 * Stages run in this order within a call.  Arguments, alignment, workspace
 * size and status codes are those of mla_decode_step, which equals one call
 * with MLA_STAGE_ALL.  Every piece of state a stage leaves for the next
 * (q_lat, plan, partial rows) is in the caller's workspace, so the stages
 * of one step must be given the same workspace and arguments, in order, on
 * one stream (or ordered by the caller); nothing is kept by the library.
 * ATTEND without a preceding ABSORB on that workspace, or MERGE without a
 * preceding ATTEND, gives meaningless results; the kernels check every plan
 * entry against the call's shapes and the sequences' current lengths, so no
 * access leaves the buffers.
 * stages == 0 or bits outside MLA_STAGE_ALL: MLA_ERR_INVALID_ARG. */
#define MLA_STAGE_ABSORB 1
#define MLA_STAGE_ATTEND 2
#define MLA_STAGE_MERGE 4
#define MLA_STAGE_ALL 7
int mla_decode_step_stages(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                           const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                           const void* w_uv, int B, int s_q, int n_h, int d_h, int d_c, int d_r, int block_size,
                           float softmax_scale, int kv_dtype, int num_splits, void* workspace,
                           size_t workspace_bytes, void* o, float* lse, int stages, void* stream);

/* mla_decode_step_noalloc -- mla_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same step with no workspace
 * argument.  Its plan, bf16 partial rows and absorbed queries live in one
 * fixed device array of MLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * and frees nothing.
 *  - Arguments, requirements and status codes as mla_decode_step, and
 *    MLA_ERR_TOO_LARGE (nothing enqueued) when the step needs more scratch:
 *    bf16 q_lat (B*s_q*n_h*d_c*2 bytes) plus room for the partial rows of
 *    max(compute units / s_q, B * ceil(max_blocks_per_seq / 512)) partitions
 *    (B * max(num_splits, that ceil) with explicit splits), each
 *    s_q*n_h*d_c*2 bytes.  That covers B = 64 at 8K or 16K context with
 *    s_q <= 2, B = 128 up to 32K and B = 4 at 128K on a 256-unit GPU.
 *  - Automatic planning is limited to one wave of partitions (at most one
 *    per compute unit and query token, unless the 512-page cap per
 *    partition needs more), so its plan, and with it the rounding of the
 *    merge, can differ from mla_decode_step's where that one would plan
 *    more; with an explicit num_splits the results are bit-identical.
 *  - Every call on a GPU shares that GPU's scratch and leaves its contents
 *    there: calls that overlap on one GPU (two streams, two host threads)
 *    race and must be ordered by the caller.  No part of the scratch needs
 *    to start at zero: every byte a call reads is written earlier in the
 *    same call. */
#define MLA_NOALLOC_SCRATCH_BYTES (64ull << 20)
int mla_decode_step_noalloc(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                            const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                            const void* w_uv, int B, int s_q, int n_h, int d_h, int d_c, int d_r, int block_size,
                            float softmax_scale, int kv_dtype, int num_splits, void* o, float* lse, void* stream);

/* mla_decode_step_workspace_bytes -- workspace of mla_decode_step (the
 * decode workspace plus a bf16 q_lat buffer); 0 on bad sizes. */
size_t mla_decode_step_workspace_bytes(int B, int s_q, int n_h, int d_c, int max_blocks_per_seq, int num_splits);

/* mla_expand_kv -- MHA-mode keys and values from the latent (itwiki
 * "Multi-head latent attention", section "Joint KV compression"), the input
 * of prefill: k_c[t,i,:] = W^UK_i c_kv[t,:], v_c[t,i,:] = W^UV_i c_kv[t,:].
 *
 *  c_kv      [T, d_c], token stride c_stride_t, dtype act_dtype
 *  w_uk/w_uv [n_h*d_h, d_c] ([out, in]; head i = rows i*d_h ..), dtype w_dtype
 *  k_c, v_c  [T, n_h, d_h] contiguous, dtype out_dtype
 *  bf16 inputs with n_h*d_h a multiple of 256, d_c a multiple of 32, the
 *  token stride a multiple of 8 elements and 16-byte aligned pointers (8 for
 *  bf16 outputs) take the expansion GEMM kernel (both products in one
 *  launch); other bf16 shapes the MFMA up-projection kernel (same limits and
 *  alignment rules as mla_up_proj_v), other combinations a plain fp32
 *  kernel.  T == 0 is a no-op. */
int mla_expand_kv(const void* c_kv, int64_t c_stride_t, const void* w_uk, const void* w_uv, void* k_c,
                  void* v_c, int T, int n_h, int d_c, int d_h, int act_dtype, int w_dtype, int out_dtype,
                  void* stream);

/* mla_prefill_mha -- causal MHA-mode attention of one sequence (prefill; the
 * itwiki article's layer equation with k = [k^C; k^R], k^R shared by the
 * heads): o[t,i,:] = sum_{j<=t} softmax_j(softmax_scale * (q[t,i,:d_h] .
 * k_c[j,i,:] + q[t,i,d_h:] . k_r[j,:])) v_c[j,i,:].
 *
 *  q    [T, n_h, d_h + d_r] (q^C then q^R per head), contiguous
 *  k_c  [T, n_h, d_h], k_r [T, d_r], v_c [T, n_h, d_h], contiguous; dtype
 *       in_dtype (MLA_F32 or MLA_BF16)
 *  o    [T, n_h, d_h], dtype out_dtype; lse [T, n_h] fp32 (natural log) or NULL
 *  bf16 with d_h == 128, d_r == 64 and 16-byte aligned buffers takes the MFMA
 *  kernel (fp32 accumulation, exp2-domain online softmax); everything else
 *  (d_h + d_r <= 256) a plain fp32 kernel.  T == 0 is a no-op. */
int mla_prefill_mha(const void* q, const void* k_c, const void* k_r, const void* v_c, void* o, float* lse,
                    int T, int n_h, int d_h, int d_r, float softmax_scale, int in_dtype, int out_dtype,
                    void* stream);

/* mla_gqa_decode -- GQLA's GQA decode path (chatpaper page on GQLA,
 * abstract: the same weights decode either in MQA-absorb form, as
 * mla_decode_absorbed, or in GQA form over a cache expanded per group of
 * heads).  n_g groups of n_h/n_g consecutive heads; group g's keys and
 * values are k^C_{j,g} = W^UK_g c_j, v^C_{j,g} = W^UV_g c_j; the RoPE key is
 * shared:
 *   s[j] = softmax_scale * (q_c[b,i,h,:] . k^C_{j,g(h)} + q_r[b,i,h,:] . kR_j),
 *          j <= seq_lens[b] - s_q + i
 *   o[b,i,h,:] = sum_j softmax(s)[j] v^C_{j,g(h)},  lse[b,i,h] = log sum_j exp(s[j])
 *
 *  q_c  [B, s_q, n_h, d_h], q_r [B, s_q, n_h, d_r], dtype q_dtype, contiguous
 *  kv_cache paged, block_size tokens per block, physical block p at byte
 *           offset p * block_size * (2*n_g*d_h + d_r) * elem; per block
 *           [n_g][block_size][d_h] k^C | [n_g][block_size][d_h] v^C |
 *           [block_size][d_r] k^R, dtype kv_dtype (MLA_BF16 or MLA_F32)
 *  block_table / seq_lens as for mla_decode_absorbed (1 <= s_q <= seq_lens[b])
 *  o    [B, s_q, n_h, d_h], dtype out_dtype; lse [B, s_q, n_h] fp32 or NULL
 *  bf16 with d_h = 128, d_r = 64, block_size = 64, s_q * n_h / n_g = 32 and
 *  16-byte aligned buffers takes the MFMA kernel (one workgroup per
 *  (sequence, group), no workspace); everything else (d_h + d_r <= 256) a
 *  portable fp32 kernel.  flags: MLA_FLAG_FORCE_GENERIC or 0. */
int mla_gqa_decode(const void* q_c, const void* q_r, const void* kv_cache, const int32_t* block_table,
                   int max_blocks_per_seq, const int32_t* seq_lens, int B, int s_q, int n_h, int n_g, int d_h,
                   int d_r, int block_size, float softmax_scale, int q_dtype, int kv_dtype, int out_dtype, void* o,
                   float* lse, int flags, void* stream);

/* mla_status_string -- static, human-readable text for a status code. */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
