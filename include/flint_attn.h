/*
 * flint_attn.h - C ABI of the Flint sink-aware attention on AMD Instinct
 * MI355X (gfx950): the prefill forward, its backward, and decode with a KV
 * cache.
 *
 * What one call computes, for every valid token t of sequence s, query head
 * h (0..31) and its key/value head g = h / 8 (grouped-query attention,
 * 32 query heads over 4 key/value heads, head dimension 128 - "flint" page of
 * NeMo AutoModel, section "Model Architecture"):
 *
 *   qhat = RMSNorm(q[t,h,:]) * q_norm_w,  khat = RMSNorm(k[t',g,:]) * k_norm_w
 *       weight-form RMSNorm, x / sqrt(mean(x^2) + eps) * w, over the 128
 *       channels of one head (Hugging Face discussion #26 on RecursiveSI/flint,
 *       "What was unusually easy": plain weight form, not 1+w);
 *   if use_rope: NeoX rotation of channel c with channel c+64 by the angle
 *       pos * theta^(-c/64), on all 128 channels, after the norm
 *       ("Model Architecture": query/key normalization precedes RoPE;
 *       flint.layers API page, FlintAttention._apply_rope);
 *   z(t') = qhat . khat(t') / sqrt(128) over the allowed keys t' of the same
 *       sequence: not padding, not after t, and when window > 0 at most
 *       window-1 tokens before t (window 513 = the current token and the 512
 *       before it, "Model Architecture"; window 0 = full causal attention,
 *       flint.layers page, FlintAttention.forward);
 *   out[t,h,:] = sum_t' exp(z(t') - m) v[t',g,:] / (exp(sink[h] - m) + sum_t' exp(z(t') - m)),
 *       m = max(sink[h], max z): the sink is a per-query-head FP32 logit in
 *       natural-log units, not scaled by 1/sqrt(128), that joins the max and
 *       the denominator with zero value and is not a token (discussion #26,
 *       "What was unusually easy" and "Configuration oddities" item 5;
 *       flint.layers page, _FlintSinkParameters).
 *
 * Padded query rows (index in sequence >= seqused[s]) are written as exact
 * zeros: padded queries and keys leave real attention and only the zero-value
 * sink stays valid (flint.layers page, FlintAttention.forward, attention_mask).
 * A row whose sink is -INF and whose key set is empty is also written as 0.
 *
 * Layout. BSHD [B, S, H, D] tensors are the THD [T, H, D] form with T = B*S
 * and cu_seqlens = {0, S, 2S, ..., B*S}; THD packs documents back to back with
 * document-local positions (flint.layers page, _apply_rope and forward:
 * "[batch, sequence, heads, head_dim] or THD [tokens, heads, head_dim]").
 *
 * Ownership and threading. Every pointer is caller-owned. The library keeps no
 * state and allocates nothing; it is reentrant. Two calls that share a
 * workspace must not overlap on the device.
 *
 * Asynchrony. flint_attn_fwd validates its host arguments synchronously,
 * enqueues two kernels on `stream` and returns. Argument errors return a
 * negative status and launch nothing. Errors in device-resident data
 * (cu_seqlens, seqused) are detected on the device: the call then writes
 * nothing to `out` and records the error in the workspace, where
 * flint_attn_device_status() reads it. With the environment variable
 * FLINT_ATTN_DEBUG=1, flint_attn_fwd synchronizes and returns that status.
 */
#ifndef FLINT_ATTN_H
#define FLINT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flint_status {
  FLINT_OK = 0,
  FLINT_ERR_NULL = -1,        /* a required pointer is NULL                      */
  FLINT_ERR_SHAPE = -2,       /* negative or inconsistent sizes                  */
  FLINT_ERR_UNSUPPORTED = -3, /* heads / head_dim other than 32 / 4 / 128         */
  FLINT_ERR_VALUE = -4,       /* window < 0, eps <= 0, theta <= 0 with RoPE, NaN  */
  FLINT_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required          */
  FLINT_ERR_ALIGN = -6,       /* tensor pointers not 16-byte aligned, workspace
                                 not 256-byte aligned, int32 arrays not 4-byte    */
  FLINT_ERR_HIP = -7,         /* a HIP runtime call or kernel launch failed        */
  FLINT_ERR_DEVICE_DATA = -8, /* cu_seqlens / seqused / mask content is invalid    */
  FLINT_ERR_TOO_LARGE = -9    /* flint_attn_fwd_static: the sizes need more than its
                                 static scratch (FLINT_ATTN_STATIC_SCRATCH_BYTES)   */
} flint_status;

/* Device-data error bits reported by flint_attn_device_status(). */
#define FLINT_DEV_CU_START 1     /* cu_seqlens[0] != 0                          */
#define FLINT_DEV_CU_ORDER 2     /* cu_seqlens decreases somewhere              */
#define FLINT_DEV_CU_END 4       /* cu_seqlens[n_seqs] != total_tokens          */
#define FLINT_DEV_MAX_SEQLEN 8   /* a sequence is longer than max_seqlen        */
#define FLINT_DEV_SEQUSED 16     /* seqused[s] < 0 or > the sequence length     */
#define FLINT_DEV_CACHE 32       /* decode: cache_len[b] < 0, or a full layer's cache
                                    cannot hold the token (cache_len[b] >= cache_cap) */

/* Longest sequence (tokens) the prefill forward and backward take: 2^21. */
#define FLINT_MAX_SEQLEN 2097152

/*
 * Bytes of device workspace flint_attn_fwd needs for these sizes; 0 when the
 * sizes are invalid (negative, max_seqlen above FLINT_MAX_SEQLEN, or heads /
 * head_dim unsupported). The value
 * only grows with each argument. It holds the work schedule and the
 * normalized, rotated K and the V tiles of every sequence, laid out for the
 * attention kernel (about 2 KiB per token and 256 KiB per sequence, rounded
 * up to whole 64-token tiles).
 */
size_t flint_attn_workspace_bytes(int32_t total_tokens, int32_t n_seqs, int32_t max_seqlen,
                                  int32_t num_kv_heads, int32_t head_dim);

/*
 * The attention forward. All tensor pointers are device pointers.
 *
 *   q          bf16 [T, num_q_heads, head_dim], contiguous, 16-byte aligned
 *   k, v       bf16 [T, num_kv_heads, head_dim], contiguous, 16-byte aligned
 *   q_norm_w   fp32 [head_dim] RMSNorm weight of the query heads (shared)
 *   k_norm_w   fp32 [head_dim] RMSNorm weight of the key heads (shared)
 *   sink       fp32 [num_q_heads] sink logits, natural-log units; -INF allowed
 *   positions  int32 [T] RoPE positions (document-local for THD), or NULL for
 *              the index inside the sequence; never read when use_rope == 0
 *   cu_seqlens int32 [n_seqs + 1]: cu[0] = 0, non-decreasing, cu[n_seqs] = T
 *   seqused    int32 [n_seqs] valid prefix length of each sequence (trailing
 *              padding), or NULL when every token is valid
 *   n_seqs, max_seqlen, total_tokens (T): sizes; max_seqlen bounds every
 *              cu[s+1] - cu[s] and is at most FLINT_MAX_SEQLEN (else
 *              FLINT_ERR_UNSUPPORTED)
 *   num_q_heads, num_kv_heads, head_dim: must be 32, 4, 128
 *   window     keys per query including the current token (513 on Flint's
 *              sliding layers), or 0 for full causal attention
 *   use_rope   non-zero on sliding (RoPE) layers, 0 on full (NoPE) layers
 *   rope_theta RoPE base (> 0 when use_rope)
 *   eps        RMSNorm epsilon (> 0; Flint uses 1e-6)
 *   workspace  device buffer of workspace_bytes >= flint_attn_workspace_bytes(),
 *              256-byte aligned; its content on entry is ignored
 *   out        bf16 [T, num_q_heads, head_dim], 16-byte aligned; every row is
 *              written (padded rows as zeros)
 *   stream     hipStream_t to enqueue on (NULL = the default stream)
 *
 * Returns FLINT_OK or a negative flint_status. T == 0 returns FLINT_OK
 * without launching anything.
 */
int flint_attn_fwd(const void* q, const void* k, const void* v, const float* q_norm_w,
                   const float* k_norm_w, const float* sink, const int32_t* positions,
                   const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                   int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t window, int32_t use_rope,
                   float rope_theta, float eps, void* workspace, size_t workspace_bytes, void* out,
                   void* stream);

/*
 * flint_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a static array of
 * FLINT_ATTN_STATIC_SCRATCH_BYTES in the library's device memory, one per
 * GPU, held from the library's first call on that GPU until the process
 * ends; its address is looked up once per device. The call allocates
 * nothing and runs the same kernels as flint_attn_fwd, with the same
 * arguments otherwise and the same results. Limits and caveats:
 *   - sizes whose flint_attn_workspace_bytes() exceeds the scratch return
 *     FLINT_ERR_TOO_LARGE and launch nothing (64 MiB: about 31,000 tokens
 *     of one sequence);
 *   - every call on a GPU uses that GPU's one array: calls that overlap on
 *     one GPU (other streams, other threads) race and must be serialized by
 *     the caller; each call rewrites what it reads, so the content a previous
 *     call left does not matter;
 *   - device-data errors (cu_seqlens, seqused) cannot be read back with
 *     flint_attn_device_status; with FLINT_ATTN_DEBUG=1 the call synchronizes
 *     and returns FLINT_ERR_DEVICE_DATA itself.
 */
#define FLINT_ATTN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int flint_attn_fwd_static(const void* q, const void* k, const void* v, const float* q_norm_w,
                          const float* k_norm_w, const float* sink, const int32_t* positions,
                          const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                          int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t window,
                          int32_t use_rope, float rope_theta, float eps, void* out, void* stream);

/* Phases of flint_attn_fwd, in the order they must run on one stream
 * (SCHEDULE and KV run in one launch when both are asked for). */
#define FLINT_PHASE_SCHEDULE 1 /* check cu_seqlens/seqused; lay out the query blocks
                                  and the padded rows                                */
#define FLINT_PHASE_KV 2       /* normalize + rotate K, transpose V into the workspace */
#define FLINT_PHASE_ATTEND 4   /* the attention kernel; writes every row of out
                                  (padded rows as zeros)                             */
#define FLINT_PHASE_ALL 7

/*
 * flint_attn_fwd split into its phases: the same arguments plus a bit set of
 * FLINT_PHASE_* values; the selected phases are enqueued in order. Running
 * the phases of one call in several calls (same arguments and workspace, same
 * stream, in phase order) gives the same result as flint_attn_fwd; this lets
 * a caller time or overlap the phases. FLINT_PHASE_KV and FLINT_PHASE_ATTEND
 * read what the earlier phases left in the workspace. phases outside 1..7
 * return FLINT_ERR_VALUE.
 */
int flint_attn_fwd_phases(const void* q, const void* k, const void* v, const float* q_norm_w,
                          const float* k_norm_w, const float* sink, const int32_t* positions,
                          const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                          int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t window,
                          int32_t use_rope, float rope_theta, float eps, void* workspace,
                          size_t workspace_bytes, void* out, void* stream, int32_t phases);

/*
 * Turns a binary BSHD attention mask into per-sequence valid lengths. The
 * mask is uint8 [batch, seqlen] (device), non-zero = valid token. TE's BSHD
 * form supports trailing padding only and arbitrary padding takes THD
 * packing (flint.layers page, FlintAttention.forward, attention_mask), so
 * each row must be ones followed by zeros. Writes seqused[b] (device int32
 * [batch]) and *n_bad (device int32) = the number of rows that are not of that
 * form. Such a row gets seqused = -1, which flint_attn_fwd reports as the
 * device-data error FLINT_DEV_SEQUSED (out untouched), so the lengths can go
 * to the forward without the host reading n_bad first. Asynchronous on
 * `stream`.
 */
int flint_attn_seqused_from_mask(const uint8_t* mask, int32_t batch, int32_t seqlen,
                                 int32_t* seqused, int32_t* n_bad, void* stream);

/*
 * Synchronizes `stream` and reads the device-data error bits that the last
 * flint_attn_fwd using this workspace recorded (FLINT_DEV_* bits, 0 if none)
 * into *flags. Returns FLINT_OK if flags == 0, FLINT_ERR_DEVICE_DATA if not,
 * or another negative status if the arguments or the HIP calls fail.
 */
int flint_attn_device_status(const void* workspace, void* stream, int32_t* flags);

/*
 * Which attention kernel flint_attn_fwd (and flint_attn_fwd_lse) launches for
 * a call of total_tokens tokens in n_seqs sequences; a host-side query that
 * launches nothing. Problems with fewer 32-token query blocks than CUs run on
 * two 4-wave workgroups per work item (four query heads each), so that twice
 * the CUs take part; larger ones on one 8-wave workgroup per item that shares
 * every key/value tile among the kv head's eight query heads. Both compute
 * the same layer. Returns FLINT_KERNEL_WIDE or FLINT_KERNEL_SPLIT, 0 when
 * total_tokens == 0, FLINT_ERR_SHAPE for negative sizes or n_seqs < 1 with
 * tokens. (The FP16 variant always runs the 8-wave kernel.)
 */
#define FLINT_KERNEL_WIDE 1
#define FLINT_KERNEL_SPLIT 2
int flint_attn_fwd_kernel(int32_t total_tokens, int32_t n_seqs);

/* A static, human-readable name of a flint_status value. */
const char* flint_attn_strerror(int status);

/* ------------------------------------------------------------------------
 * Decode with a per-layer KV cache.
 *
 * One new token per sequence attends to the cached keys of its layer. The
 * cache honours the layer's window (Hugging Face discussion #26, "Minor": a
 * hybrid KV cache in which the per-layer window sizes must be honoured): a
 * sliding layer keeps the last `window` tokens in a ring, a full layer keeps
 * all of them. The result for the new token t = cache_len[b] is exactly row t
 * of flint_attn_fwd over the sequence's tokens 0..t with the same weights,
 * sinks, window, positions and flags.
 *
 * Cache layout (caller-owned device memory, one pair per layer), head-major so
 * that every (sequence, kv head) streams one contiguous region, in blocks of
 * 32 slots stored in the order the decode products read them (each 8 KiB
 * block is read as eight contiguous 1 KiB loads):
 *   k_cache [batch][4][cache_cap/32][2][4][64][8] bf16: RMSNorm-ed,
 *           RoPE-rotated keys (as flint_attn_fwd forms them before its bf16
 *           rounding). Element [b][g][blk][kh][ds][l][e] is channel
 *           32 ds + 8 (l / 16) + e of the key in slot 32 blk + 16 kh + l % 16.
 *   vt_cache [batch][4][cache_cap/32][8][64][8] bf16: values. Element
 *           [b][g][blk][db][l][e] is channel 16 db + l % 16 of the value in
 *           slot 32 blk + 4 (l / 16) + e for e < 4 and
 *           32 blk + 16 + 4 (l / 16) + e - 4 for e >= 4.
 * Token t of a sequence sits in slot t of a full layer (window = 0) and in
 * slot t % cache_cap of a sliding layer, which needs cache_cap >= window.
 * cache_cap must be a positive multiple of 32; both pointers 16-byte aligned.
 * The caller owns cache_len (tokens already in the cache, per sequence) and
 * advances it after a call; the library never writes it.
 * ------------------------------------------------------------------------ */

/* Workspace size in bytes for flint_attn_kv_append / flint_attn_decode with
 * `batch` sequences and a cache of `cache_cap` slots. */
size_t flint_attn_decode_workspace_bytes(int32_t batch, int32_t cache_cap);

/* Appends n_new tokens to each sequence's cache: token cache_len[b] + i of
 * sequence b, for i < n_new, from k/v [batch][n_new][4][128] bf16 (projected,
 * before RMSNorm). positions [batch][n_new] int32 gives the RoPE position of
 * each (NULL: the token index cache_len[b] + i; read only when use_rope).
 * Fills a cache from a prompt, or adds the current token. A sliding layer
 * takes n_new <= cache_cap. Errors: FLINT_ERR_NULL, FLINT_ERR_SHAPE
 * (batch < 1, n_new < 1, cache_cap not a positive multiple of 32, a sliding
 * cache smaller than the window), FLINT_ERR_UNSUPPORTED (head layout),
 * FLINT_ERR_VALUE, FLINT_ERR_ALIGN, FLINT_ERR_WORKSPACE, FLINT_ERR_HIP.
 * Device-data errors (FLINT_DEV_CACHE) leave that sequence's cache unchanged
 * and are read with flint_attn_device_status(workspace, ...). */
int flint_attn_kv_append(const void* k, const void* v, const float* k_norm_w,
                         const int32_t* positions, const int32_t* cache_len, int32_t batch,
                         int32_t n_new, void* k_cache, void* vt_cache, int32_t cache_cap,
                         int32_t num_kv_heads, int32_t head_dim, int32_t window,
                         int32_t use_rope, float rope_theta, float eps, void* workspace,
                         size_t workspace_bytes, void* stream);

/* One decode step: appends the new token (q [batch][32][128], k/v
 * [batch][4][128] bf16, projected, before RMSNorm; positions [batch] or NULL
 * = cache_len[b]) to the cache as flint_attn_kv_append does, then writes its
 * attention output out [batch][32][128] bf16 over tokens
 * max(0, t - window + 1) .. t (window > 0) or 0 .. t (window = 0),
 * t = cache_len[b], with the sink. Split over the keys (64 to 512 per split,
 * chosen from the batch and cache size) and merged, so one sequence spreads
 * over the GPU. Errors as for
 * flint_attn_kv_append; a sequence with a device-data error gets zero rows. */
int flint_attn_decode(const void* q, const void* k, const void* v, const float* q_norm_w,
                      const float* k_norm_w, const float* sink, const int32_t* positions,
                      const int32_t* cache_len, int32_t batch, void* k_cache, void* vt_cache,
                      int32_t cache_cap, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t window, int32_t use_rope, float rope_theta,
                      float eps, void* workspace, size_t workspace_bytes, void* out,
                      void* stream);

/* ------------------------------------------------------------------------
 * Projections around the layer ([layers page] FlintAttention: separate q_proj,
 * k_proj, v_proj and o_proj, nn.Linear without bias, y = x W^T with W
 * [out, in]; [config page] hidden_size 2048). bf16 in and out, FP32
 * accumulation, row-major, device pointers, asynchronous on `stream`.
 *
 * flint_proj_qkv: x [T][hidden]; w_q [32*128][hidden], w_k and w_v
 * [4*128][hidden]; writes q [T][32][128], k and v [T][4][128] (channel
 * h*128 + d of a projection is channel d of head h). One launch over the
 * concatenated 5120 output channels. hidden must be a multiple of 64.
 *
 * flint_proj_out: o [T][32*128] (the layer's output), w_o [hidden][32*128];
 * writes y [T][hidden]. hidden must be a multiple of 256.
 *
 * Errors: FLINT_ERR_UNSUPPORTED for other head layouts or hidden sizes,
 * FLINT_ERR_NULL, FLINT_ERR_ALIGN (16-byte alignment of every pointer),
 * FLINT_ERR_HIP. T = 0 does nothing.
 * ------------------------------------------------------------------------ */

int flint_proj_qkv(const void* x, const void* w_q, const void* w_k, const void* w_v,
                   int32_t total_tokens, int32_t hidden, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, void* q, void* k, void* v,
                   void* stream);

int flint_proj_out(const void* o, const void* w_o, int32_t total_tokens, int32_t hidden,
                   int32_t num_q_heads, int32_t head_dim, void* y, void* stream);

/* ------------------------------------------------------------------------
 * BSHD input with document ids and arbitrary padding ([layers page]
 * FlintAttention.forward: attention_mask [B, S] marks valid tokens, padded
 * queries and keys leave attention while the sink stays valid, arbitrary
 * padding is THD packing; integer document_ids [B, S] give a block-diagonal
 * mask). Documents are the maximal runs of equal id among a row's valid
 * tokens; the window counts a document's valid tokens; default positions are
 * the index in the document.
 *
 * flint_attn_bshd_plan turns the mask (uint8 [B][S], nonzero = valid, or NULL:
 * all valid) and the ids (int32 [B][S], or NULL: one document per row) into a
 * THD description, written to `plan`, an int32 array of
 * flint_attn_bshd_plan_bytes(B, S) bytes with N = B*S:
 *   info     [8]   at 0        n_seqs, max_seqlen, total_tokens, packed,
 *                              valid tokens, documents, 0, 0
 *   cu       [N+1] at 8        cu_seqlens, n_seqs + 1 entries used
 *   seqused  [N]   at 9+N      valid length of each sequence
 *   pack     [N]   at 9+2N     packed mode: source token (b*S+s) of each stream token
 *   unpack   [N]   at 9+3N     stream token of each source token, -1 on padding
 *   scratch  [2N+2+3*ceil(N/1024)]
 * packed = 0: the B*S tokens in memory are the THD stream (no document has a
 * padded token inside it): pass q, k, v, positions and out as they are, with
 * total_tokens = N. packed = 1: the stream is the valid tokens in order; gather
 * q, k, v (and positions) with flint_attn_copy_rows(src, pack, total_tokens,
 * ...), run the layer, and scatter the output with
 * flint_attn_copy_rows(packed_out, unpack, N, ..., fill 0, out).
 * The plan is device data: read info after the stream has reached it.
 * Asynchronous on `stream`; errors as for flint_attn_fwd (host checks only:
 * every mask and id array is valid input). N must be below 2^30.
 * ------------------------------------------------------------------------ */

size_t flint_attn_bshd_plan_bytes(int32_t batch, int32_t seqlen);

int flint_attn_bshd_plan(const uint8_t* attention_mask, const int32_t* document_ids,
                         int32_t batch, int32_t seqlen, void* plan, size_t plan_bytes,
                         void* stream);

/* dst row r = src row index[r] for r in [0, n_rows), or rows of the 32-bit
 * word `fill` where index[r] < 0. row_bytes is a multiple of 4 (16-byte
 * vectors when it is a multiple of 16 and both pointers are 16-byte aligned).
 * Device pointers; index entries must name rows that exist in src (the
 * caller's contract, not checked). Asynchronous on `stream`. */
int flint_attn_copy_rows(const void* src, const int32_t* index, int32_t n_rows, int32_t row_bytes,
                         uint32_t fill, void* dst, void* stream);

/* ------------------------------------------------------------------------
 * FP16 attention-compute variant ([flint page] Numerical comparison:
 * attention_compute_dtype = fp16 casts the normalized, rotated Q/K/V to FP16
 * at the attention boundary and restores FP32 before the output projection;
 * the projections stay FP32).
 *
 * q [T][32][128], k and v [T][4][128] are FP32 (the projections); RMSNorm and
 * RoPE run in FP32, q', k' and v are rounded to fp16 once, the products run on
 * fp16 MFMA with FP32 accumulation, and out [T][32][128] is FP32 holding the
 * fp16-rounded output (0 on padded rows). Everything else - flags, sequence
 * description, errors, asynchrony - is as for flint_attn_fwd. Meant for
 * comparison and inference: the pages note fp16 underflow of tiny gradients
 * without loss scaling, so the training path stays bf16.
 * ------------------------------------------------------------------------ */

/* Workspace size in bytes for flint_attn_fwd_f16 (it adds the fp16 query
 * rows, 8 KiB per token, to flint_attn_workspace_bytes). */
size_t flint_attn_f16_workspace_bytes(int32_t total_tokens, int32_t n_seqs, int32_t max_seqlen,
                                      int32_t num_kv_heads, int32_t head_dim);

int flint_attn_fwd_f16(const float* q, const float* k, const float* v, const float* q_norm_w,
                       const float* k_norm_w, const float* sink, const int32_t* positions,
                       const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                       int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t window, int32_t use_rope,
                       float rope_theta, float eps, void* workspace, size_t workspace_bytes,
                       float* out, void* stream);

/* ------------------------------------------------------------------------
 * Training: forward with the row normalizer, and the backward.
 *
 * The backward is what the pages' training recipes need (Hugging Face
 * discussion #26 on RecursiveSI/flint, "Where other stacks fail": sinks in
 * backward and the sink gradient). With z the scaled logits, W the sink
 * softmax weights and p_sink the sink's weight of a row, for an upstream
 * gradient dO of out:
 *   Dr[t,h]   = dO[t,h,:] . out[t,h,:]
 *   dZ        = W * (dO V^T - Dr)            (per row, over its allowed keys)
 *   dv[t',g]  = sum over t and the 8 heads h of g of W[t,h,t'] dO[t,h,:]
 *   dq'[t,h]  = sum_t' dZ[t,h,t'] khat(t') / sqrt(128)
 *   dk'[t',g] = sum over t, h of g of dZ[t,h,t'] qhat(t) / sqrt(128)
 *   dsink[h]  = - sum_t p_sink[t,h] Dr[t,h]  (the sink has value 0)
 * then the adjoint of the rotation (the opposite turn) and of the weight-form
 * RMSNorm: for y = x r w with r = 1/sqrt(mean(x^2) + eps),
 *   dx = r (dy w - x r mean(x r dy w)),  dw += dy x r over tokens and heads.
 * The softmax weights are recomputed from the forward's lse (W = exp(z - lse)).
 * ------------------------------------------------------------------------ */

/* flint_attn_fwd that also writes lse [total_tokens][32] float32 (16-byte
 * aligned): the natural-log normalizer of each row,
 * log(exp(sink[h]) + sum_t' exp(z(t'))), -INF on padded rows. Same errors as
 * flint_attn_fwd; lse NULL with total_tokens > 0 is FLINT_ERR_NULL. */
int flint_attn_fwd_lse(const void* q, const void* k, const void* v, const float* q_norm_w,
                       const float* k_norm_w, const float* sink, const int32_t* positions,
                       const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                       int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t window,
                       int32_t use_rope, float rope_theta, float eps, void* workspace,
                       size_t workspace_bytes, void* out, float* lse, void* stream);

/* Workspace size in bytes for flint_attn_bwd (0 for invalid sizes,
 * max_seqlen above FLINT_MAX_SEQLEN or an unsupported head layout). It holds the normalized operands, per-chunk FP32
 * partial sums of dk and dv, and the per-block terms of the parameter
 * gradients. */
size_t flint_attn_bwd_workspace_bytes(int32_t total_tokens, int32_t n_seqs, int32_t max_seqlen,
                                      int32_t num_kv_heads, int32_t head_dim);

/* Gradients of the layer. Inputs are the forward's arguments (same layout,
 * flags and sequence description) plus out and lse of flint_attn_fwd_lse on
 * those inputs and dout = dL/dout [total_tokens][32][128] bf16. Outputs
 * (caller-owned, written, not accumulated): dq [T][32][128], dk [T][4][128],
 * dv [T][4][128] bf16, zero on padded tokens; dq_norm_w, dk_norm_w [128] and
 * dsink [32] float32, sums over every valid token and head formed in a fixed
 * order, so repeated calls give identical bits. All device pointers; tensors
 * 16-byte aligned, float arrays 4-byte aligned. Errors as for flint_attn_fwd
 * (FLINT_ERR_NULL also for a missing out, lse, dout or output). Device-data
 * errors (cu_seqlens, seqused) leave dq, dk and dv unwritten, set the three
 * parameter gradients to zero and are read with flint_attn_device_status.
 * Asynchronous on `stream`. */
int flint_attn_bwd(const void* q, const void* k, const void* v, const float* q_norm_w,
                   const float* k_norm_w, const float* sink, const int32_t* positions,
                   const int32_t* cu_seqlens, const int32_t* seqused, int32_t n_seqs,
                   int32_t max_seqlen, int32_t total_tokens, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t window, int32_t use_rope,
                   float rope_theta, float eps, const void* out, const float* lse,
                   const void* dout, void* workspace, size_t workspace_bytes, void* dq, void* dk,
                   void* dv, float* dq_norm_w, float* dk_norm_w, float* dsink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_ATTN_H */
