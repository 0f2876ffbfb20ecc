/*
 * gqap — paged grouped-query attention for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels:
 *   - single-token decode over a paged KV cache with grouped-query heads
 *     (split over the key axis, then a combine pass), KV in fp32, bf16 or
 *     OCP fp8 e4m3fn with a per-tensor scale;
 *   - ragged causal prefill on bf16 matrix cores, with the MLA split head
 *     (a 128-wide per-head key part plus a 64-wide rope key shared by all
 *     heads) and an optional 64x64 block-sparse mask;
 *   - the same prefill with the nope parts of Q and K in fp8 e4m3fn, one
 *     scale per tensor or one per row of a head, on the fp8 matrix cores;
 *   - the MLA prefill with the shared rope key in fp8 e4m3fn, one scale per
 *     rope row;
 *   - chunked prefill against the paged cache (append the chunk's keys and
 *     values, then attend to the cached prefix and the chunk), with a bf16
 *     cache or an fp8 e4m3fn cache with per-tensor scales; short chunks
 *     (multi-token decode) run on the paged-decode workers;
 *   - the decode without a caller workspace, for callers that cannot
 *     allocate;
 *   - the padded block table built from a CSR page list;
 *   - plan / validation calls that run on the host only;
 *   - a debug gather that exposes the decode kernels' page addressing.
 *
 * Conventions for every call
 *   - Ownership: the caller owns every buffer (device tensors, plan structs,
 *     workspace).  The library never allocates or frees device memory, never
 *     synchronises a stream and never reads device memory from the host.
 *     Inputs are never modified.
 *   - Pointers named "device" must be device-accessible addresses on the
 *     current HIP device; pointers named "host" are ordinary host memory.
 *   - Strides are in elements of the tensor's own dtype.
 *   - Index tensors are int32.
 *   - Errors: every call validates before it launches anything.  On error it
 *     returns a non-zero gqap_status, launches nothing, and records a message
 *     readable with gqap_last_error() (per host thread).  Faults caused by
 *     invalid device-side data that the caller did not validate (for example
 *     a block id outside the pool) are the caller's responsibility; they may
 *     only surface as GQAP_ERR_HIP if the launch itself reports an error.
 *   - Streams: `stream` is a hipStream_t passed as void*; NULL means the null
 *     stream.  All device work is asynchronous on that stream.
 *
 * Sources for the operations (pages of the reference material):
 *   FlashMLA "Tensor Shapes Reference" (flash_mla_with_kvcache,
 *   get_mla_metadata, flash_mla_prefill, the layout diagrams and the shape
 *   error table); MATE msa_interface (plan/execute split, int32 metadata,
 *   cu_seqlens, causal offset, fp8 e4m3fn with k_scale/v_scale, num_splits,
 *   optional LSE output); Modular flare_mla_prefill (ragged MLA prefill with a
 *   shared rope key and reduced output width, explicit float scale).
 */
#ifndef GQAP_H_
#define GQAP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQAP_BLOCK_SIZE 64      /* paged-cache block rows; fixed at 64 on the pages */
#define GQAP_PLAN_MAGIC 0x47514150u

typedef enum gqap_status {
  GQAP_OK = 0,
  GQAP_ERR_INVALID_ARGUMENT = 1, /* shape, value, stride, pointer or size problem */
  GQAP_ERR_DTYPE = 2,            /* dtype or dtype combination not allowed */
  GQAP_ERR_UNSUPPORTED = 3,      /* valid request this library does not implement */
  GQAP_ERR_HIP = 4               /* a HIP runtime call or launch failed */
} gqap_status;

typedef enum gqap_dtype {
  GQAP_F32 = 0,
  GQAP_BF16 = 1,
  GQAP_FP8_E4M3FN = 2,           /* OCP fp8 E4M3FN (bias 7, no inf, 0x7F/0xFF NaN) */
  GQAP_F16 = 3                   /* reserved: always GQAP_ERR_UNSUPPORTED */
} gqap_dtype;

/* ------------------------------------------------------------------------ */
/* Paged decode                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Shapes (FlashMLA tensor-shape reference, section 1, with a shared pool):
 *   q            [B, Hq, D]            dtype q_dtype; strides q_stride_batch,
 *                                      q_stride_head; D contiguous.
 *   k_pool,v_pool[NB, Hk, 64, D]       dtype kv_dtype; strides kv_stride_block,
 *                                      kv_stride_head; the 64 x D slab of one
 *                                      (block, head) is contiguous (row stride D).
 *   block_table  [B, Nblk] int32       row stride block_table_stride; entry
 *                                      [b, j] is the pool block holding logical
 *                                      tokens 64j .. 64j+63 of sequence b; only
 *                                      entries j < ceil(seq_lens[b] / 64) are read.
 *   seq_lens     [B] int32             0 <= seq_lens[b] <= min(Nblk*64, max_seq_len);
 *                                      a length outside [0, max_seq_len] is
 *                                      not truncated: that sequence is treated
 *                                      as empty (out = 0, lse = -inf).
 *   out          [B, Hq, D]            dtype q_dtype; strides out_stride_*.
 *   lse          [B, Hq] float32       optional, contiguous, natural log.
 * Query head h reads KV head h / (Hq / Hk).  The decode query is the newest
 * token: it sees all seq_lens[b] keys.  seq_lens[b] == 0 gives out = 0 and
 * lse = -inf.
 *
 * Dtype combinations (q / kv): F32/F32, BF16/BF16, BF16/FP8_E4M3FN.
 * For FP8 KV the value of a stored code c is e4m3fn(c) * k_scale (keys) or
 * e4m3fn(c) * v_scale (values); for other KV dtypes both scales must be 1.
 * Supported head_dim: 64 or 128.
 */
typedef struct gqap_decode_desc_t {
  int32_t batch;               /* B >= 0 */
  int32_t num_q_heads;         /* Hq > 0 */
  int32_t num_kv_heads;        /* Hk > 0, Hq % Hk == 0 */
  int32_t head_dim;            /* D */
  int32_t block_size;          /* must be 64 */
  int32_t max_blocks_per_seq;  /* Nblk: block_table row width, >= 1 */
  int32_t num_pool_blocks;     /* NB >= 1 */
  int32_t max_seq_len;         /* capacity the grid is sized for; <= Nblk*64 */
  int32_t q_dtype;             /* gqap_dtype; the output has the same dtype */
  int32_t kv_dtype;            /* gqap_dtype */
  int64_t q_stride_batch;      /* elements */
  int64_t q_stride_head;
  int64_t out_stride_batch;
  int64_t out_stride_head;
  int64_t kv_stride_block;     /* elements between pool blocks */
  int64_t kv_stride_head;      /* elements between heads of one block, >= 64*D */
  int64_t block_table_stride;  /* int32 elements between block_table rows, >= Nblk */
  int32_t num_workers;         /* 0 = choose automatically; else the worker count */
  int32_t num_cus;             /* compute units to plan for; 0 = 256 (MI355X) */
} gqap_decode_desc_t;

/*
 * Plain-old-data plan, filled by gqap_decode_plan and read by the other calls.
 *
 * Schedule: the key blocks of all (sequence, KV head) pairs form one list of
 * work units; a device pre-pass reads seq_lens and cuts that list into
 * num_workers contiguous, equal-length ranges, one per persistent wave.  A
 * worker's range covers pieces of one or more key axes; each piece leaves a
 * normalised partial output and its log-sum-exp, and a combine pass merges
 * the pieces of every (sequence, query head).  The piece count of a sequence
 * plays the role of the split count (num_splits) of split-KV decoding.
 */
typedef struct gqap_decode_plan_t {
  gqap_decode_desc_t desc;
  int32_t num_workers;         /* persistent waves sharing the key blocks evenly */
  int32_t ratio;               /* Hq / Hk */
  int32_t head_chunks;         /* ceil(ratio / 16) */
  int32_t max_pieces;          /* partial-result slots: B*Hk*head_chunks + num_workers */
  uint64_t workspace_bytes;    /* device workspace the decode needs */
  uint32_t magic;              /* GQAP_PLAN_MAGIC when valid */
  uint32_t kernel;             /* internal kernel variant */
} gqap_decode_plan_t;

/*
 * Validate a decode request and choose its split schedule.  Pure host code:
 * touches no device and no tensor (get_mla_metadata on the FlashMLA page is
 * likewise shape/stride validation only).  The schedule depends only on the
 * descriptor's capacities, never on live lengths, so one plan serves every
 * call with the same shapes.
 * Errors: INVALID_ARGUMENT (non-positive sizes, Hq % Hk != 0, max_seq_len >
 * Nblk*64, strides that overlap or break 16-byte alignment, bad num_workers),
 * DTYPE (dtype pair not in the list above), UNSUPPORTED (block_size != 64,
 * head_dim not 64/128, F16, batch * Hq * 64 >= 2^32: one combine launch).
 */
gqap_status gqap_decode_plan(const gqap_decode_desc_t* desc, gqap_decode_plan_t* plan);

/*
 * Optional deep check of host copies of the metadata (the "coverage up to
 * max seq_lens" requirement of get_mla_metadata): 0 <= seq_lens[b] <=
 * min(Nblk*64, max_seq_len), and every entry block_table[b, j] with
 * j < ceil(seq_lens[b]/64) lies in [0, NB).  Padding entries are not checked.
 * block_table_host uses the plan's block_table_stride.  Errors:
 * INVALID_ARGUMENT naming the first offending entry.
 */
gqap_status gqap_decode_validate_host(const gqap_decode_plan_t* plan,
                                      const int32_t* block_table_host,
                                      const int32_t* seq_lens_host);

/*
 * Decode attention for one query token per sequence.
 *   scale:    multiplies q.k (e.g. 1/sqrt(D)); required, no default.
 *   k_scale, v_scale: per-tensor dequantisation scales (1.0 unless FP8 KV).
 *   workspace: device buffer of at least plan->workspace_bytes bytes, 256-byte
 *              aligned; its contents on entry do not matter.
 * All device pointers must be 16-byte aligned.  Asynchronous on `stream`.
 */
gqap_status gqap_paged_decode(const gqap_decode_plan_t* plan,
                              const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              float scale, float k_scale, float v_scale,
                              void* out, float* lse,
                              void* workspace, uint64_t workspace_bytes,
                              void* stream);

/*
 * The decode of gqap_paged_decode without a caller workspace and without any
 * allocation: for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * partial results live in a scratch array inside the library, one per GPU,
 * GQAP_NOALLOC_SCRATCH_BYTES long and held from the first call on that GPU
 * (whose address lookup is the call's only set-up) until the process ends.
 * The caller still passes every input and output, as for gqap_paged_decode.
 * Errors: those of gqap_paged_decode, and UNSUPPORTED when the plan's
 * workspace_bytes exceeds GQAP_NOALLOC_SCRATCH_BYTES (checked first, before
 * any device call).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (different streams, or threads without ordering) race
 * and must not be issued; calls in one stream are ordered and safe.  Nothing
 * in the array needs to start at zero.  Asynchronous on `stream`.
 */
#define GQAP_NOALLOC_SCRATCH_BYTES (32u << 20)

gqap_status gqap_paged_decode_noalloc(const gqap_decode_plan_t* plan,
                                      const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      float scale, float k_scale, float v_scale,
                                      void* out, float* lse, void* stream);

/*
 * Copy logical rows [0, num_rows) of KV head `kv_head` of sequence `b` from a
 * paged pool into dst [num_rows, D] (same dtype as the pool, contiguous),
 * using the same address arithmetic as the decode kernels.  Rows at or past
 * seq_lens[b] (read on the device) are left untouched.  num_rows is a host
 * value <= Nblk*64.  Exposed for bit-exact tests of the page addressing.
 */
gqap_status gqap_debug_gather_kv(const gqap_decode_plan_t* plan, const void* pool,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 int32_t b, int32_t kv_head, int32_t num_rows,
                                 void* dst, void* stream);

/* ------------------------------------------------------------------------ */
/* Ragged causal prefill (GQA, optional MLA rope key, optional block mask)   */
/* ------------------------------------------------------------------------ */

/*
 * Token-major ragged layout (Modular flare_mla_prefill; MATE cu_seqlens):
 *   q       [T, Hq, Dqk]   Dqk = Dn + Dr; strides q_stride_token, q_stride_head
 *   k       [T, Hk, Dn]    per-head key part (Dn = 128)
 *   v       [T, Hk, Dv]    Dv = 128
 *   k_rope  [T, 1, Dr]     shared rope key (Dr = 64), broadcast to every head;
 *                          NULL iff Dr == 0
 *   cu_seqlens [B + 1] int32 device: [0, cumsum(seq_len)]; cu_seqlens[B] <= T
 *   block_mask [B, nb, nb] uint8 device, optional (has_block_mask): entry
 *                          [b, i, j] != 0 lets query block i see key block j;
 *                          nb = mask_blocks >= ceil(max_seq_len/64), row
 *                          stride nb; entries above the diagonal are ignored.
 *   out     [T, Hq, Dv]    bf16; strides out_stride_*
 *   lse     [T, Hq] float32 optional, contiguous, natural log
 * Query i of a sequence sees key j iff j <= i (equal query and key lengths,
 * so the causal offset is 0) and, with a mask, mask[b, i/64, j/64] != 0.
 * score(i, j, h) = scale * (q[i,h,:Dn] . k[j,h/(Hq/Hk),:] + q[i,h,Dn:] . k_rope[j,0,:]).
 * A row with no visible key gets out = 0 and lse = -inf.
 */
typedef struct gqap_prefill_desc_t {
  int32_t batch;               /* B >= 0 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hk, Hq % Hk == 0 */
  int32_t head_dim_qk;         /* Dqk: 128 (Dr = 0) or 192 (Dr = 64) */
  int32_t head_dim_rope;       /* Dr: 0 or 64 */
  int32_t head_dim_v;          /* Dv: 128 */
  int32_t total_tokens;        /* T: rows of q/k/v/out */
  int32_t max_seq_len;         /* capacity the grid is sized for */
  int32_t dtype;               /* GQAP_BF16 */
  int32_t causal;              /* must be 1 */
  int32_t has_block_mask;      /* 0 or 1 */
  int32_t mask_blocks;         /* nb when has_block_mask */
  int64_t q_stride_token, q_stride_head;
  int64_t k_stride_token, k_stride_head;
  int64_t v_stride_token, v_stride_head;
  int64_t kr_stride_token;
  int64_t out_stride_token, out_stride_head;
  int32_t num_cus;             /* 0 = 256 */
  int32_t num_splits;          /* key-axis splits: 0 = chosen by the plan, 1..16 forced */
  int64_t qr_stride_token;     /* fp8 only: q_rope strides (bf16 elements) */
  int64_t qr_stride_head;
} gqap_prefill_desc_t;

typedef struct gqap_prefill_plan_t {
  gqap_prefill_desc_t desc;
  int32_t ratio;               /* Hq / Hk */
  int32_t q_tiles;             /* ceil(max_seq_len / q_tile_rows) */
  int32_t q_tile_rows;         /* query rows per workgroup and head: 128, or 64 when a
                                  block mask is given and Hq / Hk is even (a workgroup
                                  then takes two heads of one KV group, so that all its
                                  waves follow the same mask row) */
  int32_t kernel;
  uint64_t workspace_bytes;    /* 0 unless num_splits > 1 */
  uint32_t magic;
  uint32_t num_splits;         /* key-axis splits the calls will use */
} gqap_prefill_plan_t;

/*
 * Key-axis splits (prefill and chunked prefill).  When the grid (one
 * workgroup per 128-row query tile and head) would leave more than a quarter
 * of the compute units idle, the plan gives each query tile num_splits
 * workgroups, each taking one contiguous range of the tile's key tiles, so
 * the GPU is filled.  They write normalised fp32 partial outputs and their
 * LSEs into the caller's workspace, and a merge pass combines them with
 * weights exp(lse_s - max):  out = sum_s w_s o_s / sum_s w_s.  This is the
 * split-KV scheme of split decoding applied to query tiles (MATE msa:
 * num_splits).  Auto choice, for grid < 3/4 * num_cus: ceil(2 * num_cus /
 * grid), at most 4, and at most a quarter of the key tiles of the longest
 * sequence; otherwise 1.  num_splits > 0 in the descriptor forces a count.  workspace_bytes = num_splits * T * Hq * 129 * 4
 * when num_splits > 1; the workspace must then be 16-byte aligned and at
 * least that large.  Results equal the unsplit ones up to fp32 rounding.
 *
 * dtype GQAP_FP8_E4M3FN plans the fp8 prefill (gqap_prefill_fp8): q holds
 * only the nope part [T, Hq, Dn] and k [T, Hk, Dn], both e4m3fn codes with
 * strides in bytes (multiples of 16); the rope part of the query is a
 * separate bf16 tensor q_rope [T, Hq, Dr] with strides qr_stride_token,
 * qr_stride_head; v, k_rope and out are bf16 as above.  head_dim_qk still
 * counts Dn + Dr.
 *
 * Validate a prefill request.  Pure host code.  Errors: INVALID_ARGUMENT
 * (sizes, strides, Hq % Hk, mask_blocks too small), DTYPE (not bf16 or fp8),
 * UNSUPPORTED (causal == 0, head widths other than 128/192 with rope 0/64,
 * Dv != 128, Hq * batch * ceil(max_seq_len/128) * num_splits >= 2^24
 * workgroups, or with splits T * Hq * 64 >= 2^32: one merge launch);
 * INVALID_ARGUMENT also for num_splits outside 0..16.  A plan with batch > 0
 * has q_tiles >= 1 (the last query tile of a sequence clears its rows past
 * the capacity).
 */
gqap_status gqap_prefill_plan(const gqap_prefill_desc_t* desc, gqap_prefill_plan_t* plan);

/*
 * Ragged causal prefill.  All device pointers 16-byte aligned.  workspace may
 * be NULL when plan->workspace_bytes == 0.  Asynchronous on `stream`.
 * Capacity: the rows of a sequence past the plan's max_seq_len are not
 * computed; they get out = 0 and lse = -inf (the rows below it are exact,
 * since a causal row never sees a later key).  Only
 * rows inside each sequence are read: a key tile that runs past the end
 * repeats the sequence's last row, whose probability is then exactly 0, so
 * K/V are expected to be finite (an infinite value in a sequence's last V
 * row would also reach the other rows of its last 64-key tile).
 */
gqap_status gqap_prefill(const gqap_prefill_plan_t* plan,
                         const void* q, const void* k, const void* v, const void* k_rope,
                         const int32_t* cu_seqlens, const uint8_t* block_mask,
                         float scale, void* out, float* lse,
                         void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * Ragged causal prefill with the per-head (nope) parts of Q and K in fp8
 * (Modular flare_mla_prefill, the overload that takes q_nope, q_rope, q_scale
 * and k_scales).  The plan must have dtype GQAP_FP8_E4M3FN (layout above).
 * The value of a code c is e4m3fn(c) * q_scale (query) or e4m3fn(c) * k_scale
 * (key), one scale per tensor, host floats; the score is
 *   scale * (q_scale * k_scale * (q_nope codes . k codes) + q_rope . k_rope).
 * q_rope and k_rope are both NULL iff head_dim_rope == 0.  Masking, ragged
 * rows, lse and the rows past a sequence's end behave as in gqap_prefill.
 * Errors: INVALID_ARGUMENT (null or misaligned pointers, non-finite scales,
 * rope tensors that do not match the plan), DTYPE (a bf16 plan), HIP.
 */
gqap_status gqap_prefill_fp8(const gqap_prefill_plan_t* plan,
                             const void* q_nope, const void* q_rope, const void* k, const void* v,
                             const void* k_rope, const int32_t* cu_seqlens, const uint8_t* block_mask,
                             float scale, float q_scale, float k_scale, void* out, float* lse,
                             void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * The fp8 prefill with blockwise scales: one fp32 scale per row of a head,
 * i.e. per 1 x Dn block of q_nope and of k (the page leaves the layout of
 * q_scale and k_scales open; this is the finest one that keeps a row in a
 * single scale).  q_scales [T, Hq] and k_scales [T, Hk] are contiguous fp32
 * device arrays (4-byte aligned); the score is
 *   scale * (q_scales[i,h] * k_scales[j,g] * (q_nope[i,h] codes . k[j,g] codes)
 *            + q_rope[i,h] . k_rope[j]).
 * Everything else as gqap_prefill_fp8.  Errors: those of gqap_prefill_fp8,
 * and INVALID_ARGUMENT for a null or misaligned scale array.
 */
gqap_status gqap_prefill_fp8_blockwise(const gqap_prefill_plan_t* plan,
                                       const void* q_nope, const void* q_rope, const void* k, const void* v,
                                       const void* k_rope, const int32_t* cu_seqlens, const uint8_t* block_mask,
                                       float scale, const float* q_scales, const float* k_scales,
                                       void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                                       void* stream);

/*
 * Ragged causal MLA prefill with the shared rope key quantised (Modular
 * flare_mla_prefill, the overload that takes k_rope together with
 * k_rope_scales).  The plan is a bf16 plan with head_dim_rope 64 (layout as
 * gqap_prefill); q, k and v are bf16.  k_rope [T, 1, 64] holds e4m3fn codes,
 * its token stride kr_stride_token counted in bytes (a multiple of 16, at
 * least 64); k_rope_scales [T] float32 holds one scale per rope row (the page
 * leaves the scale layout open: one per row is the finest that keeps a row
 * under one scale; a per-tensor scale is the case of equal entries).  The
 * value of a code c of row j is e4m3fn(c) * k_rope_scales[j], so
 *   score = scale * (q[i,h,:128] . k[j,g,:] + k_rope_scales[j] * (q[i,h,128:] . codes of k_rope[j])).
 * Masking, ragged rows, lse, capacity and key-axis splits behave as in
 * gqap_prefill.  Errors: INVALID_ARGUMENT (null or misaligned pointers, a
 * plan without the rope part, a bad rope stride, non-finite scale), DTYPE (an
 * fp8 plan), HIP.
 */
gqap_status gqap_prefill_rope_fp8(const gqap_prefill_plan_t* plan,
                                  const void* q, const void* k, const void* v,
                                  const void* k_rope, const float* k_rope_scales,
                                  const int32_t* cu_seqlens, const uint8_t* block_mask,
                                  float scale, void* out, float* lse,
                                  void* workspace, uint64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Chunked prefill against a paged KV cache                                  */
/* ------------------------------------------------------------------------ */

/*
 * A chunk of new tokens of every sequence attends to the keys already in the
 * paged cache and to itself.  A prefill with a KV cache writes the chunk's
 * keys and values into the cache, tokens 64j .. 64j+63 of a sequence going to
 * block_table[b, j] (FlashMLA tensor-shape reference, section 4, and its
 * "Prefill to Cache Mapping"); the chunk is aligned to the end of the keys,
 * so with kv_len keys in all, the last q_len of them the chunk's own, query i
 * uses the keys up to kv_len - q_len + i (MATE msa_interface,
 * _normalize_qo_offset and _resolve_seqused_k).
 *
 * Shapes (bf16 tensors, D = 128 contiguous, Dr = head_dim_rope):
 *   q             [T, Hq, D + Dr]  strides q_stride_token, q_stride_head
 *   k_new, v_new  [T, Hk, D]       the chunk's keys and values; strides
 *                                  new_stride_token, new_stride_head
 *   k_rope_new    [T, 1, Dr]       MLA only: the chunk's rope keys, token
 *                                  stride kr_new_stride_token
 *   k_pool,v_pool [NB, Hk, 64, D]  strides kv_stride_block, kv_stride_head;
 *                                  each (block, head) 64 x D slab contiguous
 *   kr_pool       [NB, 1, 64, Dr]  MLA only: the rope cache on the same pages,
 *                                  block stride kr_stride_block, 64 x Dr slab
 *                                  contiguous (flare_mla_prefill, overload A:
 *                                  the rope keys come from a paged cache)
 *   block_table   [B, Nblk] int32  row stride block_table_stride; entries
 *                                  j < ceil(kv_lens[b] / 64) are used
 *   cu_seqlens_q  [B + 1] int32    chunk b is rows cu[b] .. cu[b+1]-1 of q,
 *                                  k_new, v_new and out; cu[B] <= T
 *   kv_lens       [B] int32        keys of sequence b with its chunk included:
 *                                  q_len_b = cu[b+1] - cu[b] <= kv_lens[b] <=
 *                                  max_kv_len, q_len_b <= max_q_len
 *   out           [T, Hq, D]       strides out_stride_*
 *   lse           [T, Hq] float32  optional, contiguous, natural log
 * Query i of chunk b sees key j iff j <= kv_lens[b] - q_len_b + i; query head
 * h reads KV head h / (Hq / Hk).  With Dr = 64 (MLA) the score adds
 * q[i, h, D:] . kr[j], the one rope key row of token j shared by every head.
 */
typedef struct gqap_chunk_desc_t {
  int32_t batch;               /* B >= 0 */
  int32_t num_q_heads;         /* Hq > 0 */
  int32_t num_kv_heads;        /* Hk > 0, Hq % Hk == 0 */
  int32_t head_dim;            /* D: 128 */
  int32_t block_size;          /* must be 64 */
  int32_t max_blocks_per_seq;  /* Nblk >= ceil(max_kv_len / 64) */
  int32_t num_pool_blocks;     /* NB >= 1 */
  int32_t total_q_tokens;      /* T: rows of q, k_new, v_new, out */
  int32_t max_q_len;           /* capacity the grid is sized for */
  int32_t max_kv_len;          /* capacity; <= Nblk * 64 */
  int32_t dtype;               /* GQAP_BF16 */
  int32_t head_dim_rope;       /* Dr: 0, or 64 for MLA */
  int64_t q_stride_token, q_stride_head;
  int64_t new_stride_token, new_stride_head;
  int64_t out_stride_token, out_stride_head;
  int64_t kv_stride_block;     /* elements between pool blocks */
  int64_t kv_stride_head;      /* elements between heads of a block, >= 64*D */
  int64_t block_table_stride;  /* int32 elements between rows, >= Nblk */
  int64_t kr_new_stride_token; /* MLA: elements between rope rows of k_rope_new, >= Dr */
  int64_t kr_stride_block;     /* MLA: elements between rope-cache blocks, >= 64*Dr */
  int32_t num_splits;          /* key-axis splits: 0 = chosen by the plan, 1..16 forced */
  int32_t kv_dtype;            /* storage of k_pool / v_pool: GQAP_BF16, or GQAP_FP8_E4M3FN
                                  for an fp8 cache with per-tensor scales (the calls
                                  gqap_append_kv_fp8 / gqap_chunk_prefill_fp8kv); 0, as a
                                  zero-filled descriptor leaves it, means GQAP_BF16.  With
                                  fp8 the kv_stride_* count bytes */
} gqap_chunk_desc_t;

typedef struct gqap_chunk_plan_t {
  gqap_chunk_desc_t desc;
  int32_t ratio;               /* Hq / Hk */
  int32_t q_tiles;             /* ceil(max_q_len / q_tile_rows) */
  int32_t q_tile_rows;         /* query rows per workgroup and head: 128 */
  int32_t kernel;             /* 1..4: prefill kernel (2, 4: with rope; 3, 4: fp8 cache);
                                  5, 6: decode workers, with the rope cache
                                  when Dr = 64 (6: fp8 cache) */
  uint64_t workspace_bytes;    /* prefill kernel: 0 unless num_splits > 1 */
  uint32_t magic;
  uint32_t num_splits;         /* key-axis splits the calls will use (1 on the decode workers) */
  int32_t num_workers;         /* decode workers: one-wave workers per call, else 0 */
  int32_t head_chunks;         /* decode workers: 16-column tiles per KV head, else 0 */
} gqap_chunk_plan_t;

/*
 * Validate a chunked-prefill request.  Pure host code.  Errors:
 * INVALID_ARGUMENT (sizes, strides that overlap or break 16-byte alignment,
 * Hq % Hk, max_kv_len > Nblk * 64, max_q_len > max_kv_len), DTYPE (dtype
 * not bf16, kv_dtype not 0, bf16 or fp8 e4m3fn),
 * UNSUPPORTED (block_size != 64, D != 128, Dr not 0 or 64, Hq * batch *
 * ceil(max_q_len / 128) * num_splits >= 2^24 workgroups, T * Hk * 16 >= 2^32
 * (one append launch), with splits T * Hq * 64 >= 2^32); INVALID_ARGUMENT
 * also for num_splits outside 0..16.  Key-axis splits as for the prefill.
 *
 * Short chunks: with num_splits = 0, a plan whose chunk rows times Hq / Hk
 * (the (token, query head) pairs of one KV head, max_q_len * Hq / Hk) fit in
 * as many 16-wide tiles as the Hq / Hk heads of one token (for Hq / Hk <= 16:
 * max_q_len * Hq / Hk <= 16; multi-token decode, e.g. speculative
 * verification) runs the calls below on the paged-decode workers, plain or
 * MLA (Dr = 64: the rope rows come from kr_pool): the keys and values of a
 * KV head are then read once per tile instead of once per query head.  The
 * results are the same attention; workspace_bytes is then the decode
 * workers' workspace (never 0).
 *
 * Capacity (both calls below): a chunk whose kv_lens[b] exceeds max_kv_len,
 * or is smaller than its own length q_len_b, is outside the plan: it is not
 * appended and all its rows get out = 0 and lse = -inf.  A chunk longer than
 * max_q_len keeps its causal offset kv_lens[b] - q_len_b; its first max_q_len
 * rows are computed and the rest get out = 0 and lse = -inf.
 */
gqap_status gqap_chunk_plan(const gqap_chunk_desc_t* desc, gqap_chunk_plan_t* plan);

/*
 * Optional deep check of host copies of the metadata: cu_seqlens_q starts at
 * 0, never decreases and ends at most at T; 0 <= q_len_b <= min(kv_lens[b],
 * max_q_len); kv_lens[b] <= max_kv_len; every used block_table entry lies in
 * [0, NB).  Errors: INVALID_ARGUMENT naming the first offending entry.
 */
gqap_status gqap_chunk_validate_host(const gqap_chunk_plan_t* plan, const int32_t* block_table_host,
                                     const int32_t* cu_seqlens_q_host, const int32_t* kv_lens_host);

/*
 * Write the chunk's keys and values into the paged cache: token i of chunk b
 * goes to logical position p = kv_lens[b] - q_len_b + i, i.e. row p % 64 of
 * pool block block_table[b, p / 64], for every KV head, and with Dr = 64 its
 * rope row to the same row of kr_pool (k_rope_new and kr_pool are NULL iff
 * Dr == 0).  Nothing else in the pools changes.  Asynchronous on `stream`;
 * 16-byte aligned pointers.
 */
gqap_status gqap_append_kv(const gqap_chunk_plan_t* plan, const void* k_new, const void* v_new,
                           const void* k_rope_new, void* k_pool, void* v_pool, void* kr_pool,
                           const int32_t* block_table, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                           void* stream);

/*
 * Attention of each chunk to its sequence's cached keys (the chunk's own
 * included, so gqap_append_kv runs first).  kr_pool is NULL iff Dr == 0.  Only key rows j < kv_lens[b] are
 * used; a key tile that runs past kv_lens[b] repeats row kv_lens[b] - 1,
 * whose probability is then exactly 0.  A query with no visible key gets
 * out = 0 and lse = -inf.  workspace may be NULL when plan->workspace_bytes
 * == 0.  Asynchronous on `stream`; 16-byte aligned pointers (lse, cu_seqlens_q
 * and kv_lens 4-byte).
 */
gqap_status gqap_chunk_prefill(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                               const void* v_pool, const void* kr_pool, const int32_t* block_table,
                               const int32_t* cu_seqlens_q, const int32_t* kv_lens, float scale,
                               void* out, float* lse, void* workspace, uint64_t workspace_bytes,
                               void* stream);

/*
 * The same two calls over an fp8 e4m3fn KV cache (plan kv_dtype
 * GQAP_FP8_E4M3FN; the plain calls reject such a plan with DTYPE and these
 * reject a bf16 one).  The cache is the per-tensor scaled fp8 cache that the
 * paged decode reads (MATE msa_interface: k_scale / v_scale dequantisation
 * scales; FlashMLA tensor-shape reference: FP8 caches): a stored code c
 * stands for e4m3fn(c) * k_scale in k_pool and e4m3fn(c) * v_scale in v_pool.
 * k_pool and v_pool are [NB, Hk, 64, D] bytes; q, k_new, v_new, the rope
 * tensors, out and lse are as above (bf16 / float32), and the rope cache
 * stays bf16.
 *
 * gqap_append_kv_fp8 writes the code of k_new / k_scale (v_new / v_scale),
 * the quotient taken in float32, rounded to the nearest e4m3fn value with
 * ties to the even code, magnitudes past 448 saturating to +-448 and NaN
 * giving a NaN code; positions as gqap_append_kv.
 * gqap_chunk_prefill_fp8kv computes the attention of gqap_chunk_prefill with
 * the dequantised keys and values; queries stay bf16 and are never
 * quantised.  k_scale and v_scale must be finite and > 0.
 */
gqap_status gqap_append_kv_fp8(const gqap_chunk_plan_t* plan, const void* k_new, const void* v_new,
                               const void* k_rope_new, void* k_pool, void* v_pool, void* kr_pool,
                               const int32_t* block_table, const int32_t* cu_seqlens_q, const int32_t* kv_lens,
                               float k_scale, float v_scale, void* stream);

gqap_status gqap_chunk_prefill_fp8kv(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                                     const void* v_pool, const void* kr_pool, const int32_t* block_table,
                                     const int32_t* cu_seqlens_q, const int32_t* kv_lens, float scale,
                                     float k_scale, float v_scale, void* out, float* lse, void* workspace,
                                     uint64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* CSR page input                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Padded block table from a flat page list (MATE msa_interface,
 * _build_page_table_from_flat_kv_indices): the pages of sequence b are
 * kv_indices[kv_page_indptr[b] .. kv_page_indptr[b+1]), in order.  Writes
 * block_table[b, j] = kv_indices[kv_page_indptr[b] + j] for j < min(pages of b,
 * max_blocks_per_seq) and -1 for the rest of the row up to max_blocks_per_seq
 * (pages past the row width are not represented).  The page's own builder
 * pads with 0 into a table as wide as the longest page list; here the width
 * is the caller's and the padding -1, which no valid page id equals, so a
 * stray read of padding cannot alias block 0.  No attention call reads
 * padding entries, so results do not depend on the choice.  With it, every
 * call that takes a block table also takes CSR page input.
 *   kv_indices      [total pages] int32 device
 *   kv_page_indptr  [batch + 1] int32 device, non-decreasing, starting at 0
 *   block_table     [batch, >= max_blocks_per_seq] int32 device, row stride
 *                   block_table_stride (elements), written
 * Errors: INVALID_ARGUMENT (null pointer, batch < 0, max_blocks_per_seq < 1,
 * block_table_stride < max_blocks_per_seq, misaligned pointer), UNSUPPORTED
 * (batch * max_blocks_per_seq >= 2^32 entries: one launch), HIP.
 * Asynchronous on `stream`.
 */
gqap_status gqap_block_table_from_csr(const int32_t* kv_indices, const int32_t* kv_page_indptr, int32_t batch,
                                      int32_t max_blocks_per_seq, int64_t block_table_stride,
                                      int32_t* block_table, void* stream);

/* ------------------------------------------------------------------------ */

/* Message of the last non-OK status on this host thread ("" if none). */
const char* gqap_last_error(void);

/* Library version string. */
const char* gqap_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQAP_H_ */
