/*
 * nomas_attn.h -- C ABI of the action-aware causal attention library (gfx950).
 *
 * The operation.  Hy-Nomas generates video segment by segment; each segment's
 * keys and values join a permanent, growing cache that later segments attend
 * to ("Tencent's Hy-Nomas Steers a 60-Second Video World ..." (gpts24.com),
 * section "One World, Generated Segment by Segment").  Attention is joint over
 * video and text tokens of 16 heads x 128 dims ("Summary (Overview)" page,
 * Theoretical Foundation) and masked by these rules ("Summary (Overview)",
 * Model Architecture: Segment-wise Causal Attention and Action-Aware Causal
 * Attention, Figure 6b; onedev.kr review, section "무엇과 다른가"):
 *   - a query of segment j sees segments 0..j of its own video (both ways
 *     inside segment j, nothing later);
 *   - every segment's descriptive head stays visible to later segments;
 *   - an action tail a_k is visible only inside its own segment, to video
 *     queries whose latent frame lies in a_k's window [lo, hi), and (text-query
 *     reading "R") to a_k's own tokens;
 *   - packed videos never see each other; padding is never visible.
 * Hidden pairs get -inf logits; the library computes exact softmax attention
 * O = softmax(scale * Q K^T + M) V (and its gradient for training packs).
 * The unmasked-pair count A of a call is the "A_i" of the FLOPs-based packing
 * estimate ("Summary (Overview)", Training Infrastructure, Eq. 6; xyznot.com
 * guide, "Dağıtık Paketleme FLOP Tahmini").
 *
 * Token order inside a segment record (a convention of this library):
 *   [video tokens, frame-major | head | a_0 | a_1 | ... | n_pad padding]
 *
 * Conventions for every call:
 *   - every function returns a nomas_status and never aborts or throws; on
 *     failure nomas_last_error() holds a thread-local description;
 *   - Q, K, V, O, dO, dQ, dK, dV are bf16 (dQ, dK, dV fp32 on request),
 *     token-major [tokens][heads][128] with the 128 dims contiguous and a
 *     caller-given token stride (elements, >= heads*128, multiple of 8, at
 *     most 2^24: larger ones return INVALID_ARGUMENT); device pointers must
 *     be 16-byte aligned;
 *   - LSE is fp32 [heads][queries] (natural log; -inf for a row that sees no
 *     key); such rows (padding) get O = 0 and dQ = 0 whatever their inputs
 *     hold, and finite values in them change no other result (in the
 *     forward not even non-finite ones);
 *   - device work is enqueued on the caller's HIP stream (NULL = default
 *     stream) and is not waited for;
 *   - plans and caches are library-owned handles; K/V cache storage, outputs
 *     and workspaces are caller-owned device memory.
 * Objects are not safe for concurrent mutation; nomas_attn_fwd may be called
 * concurrently with distinct outputs and workspaces.
 */
#ifndef NOMAS_ATTN_H
#define NOMAS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NOMAS_MAX_ACTIONS 32
#define NOMAS_HEAD_DIM 128

typedef int32_t nomas_status;
enum {
  NOMAS_OK = 0,
  NOMAS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or option        */
  NOMAS_ERR_LAYOUT = 2,           /* malformed segment records               */
  NOMAS_ERR_UNSUPPORTED = 3,      /* head_dim != 128, unsupported tile size  */
  NOMAS_ERR_CAPACITY = 4,         /* cache append would exceed capacity      */
  NOMAS_ERR_STALE_PLAN = 5,       /* cache changed since the plan was built  */
  NOMAS_ERR_ALIGNMENT = 6,        /* pointer or stride misaligned            */
  NOMAS_ERR_HIP = 7               /* HIP runtime or launch failure           */
};

/* One action tail: n_tokens text tokens, visible to the segment's video
 * queries whose latent frame f satisfies frame_lo <= f < frame_hi. */
typedef struct {
  int32_t n_tokens;
  int32_t frame_lo;
  int32_t frame_hi;
} nomas_action;

/* One segment.  (video, index) identifies it: segments of one video see the
 * segments of the same video with index <= their own.  Sizes:
 * n_frames * tokens_per_frame video tokens (the latent grid of Eq. 1), n_head
 * head tokens, the action tails, then n_pad padding tokens.  Requirements:
 * video >= 0, index >= 0, all counts >= 0, at least one token,
 * 0 <= n_actions <= 32, each action n_tokens >= 1 and
 * 0 <= frame_lo < frame_hi <= n_frames. */
typedef struct {
  int32_t video;
  int32_t index;
  int32_t n_frames;
  int32_t tokens_per_frame;
  int32_t n_head;
  int32_t n_actions;
  int32_t n_pad;
  int32_t reserved; /* set to 0 */
  nomas_action actions[NOMAS_MAX_ACTIONS];
} nomas_segment;

/* Tokens of a list of segments, concatenated in order.  A (video, index)
 * may appear at most once per layout; a segment named in both the query and
 * the key layout must carry identical records. */
typedef struct {
  int32_t n_segments;
  const nomas_segment* segments;
} nomas_layout;

/* What text (head / tail) queries see of action tails; the pages only state
 * the rule for video queries.  R: a tail's tokens see that tail, heads see
 * none.  K: no text query sees a tail.  H: as R, and heads also see every
 * tail of their own segment. */
enum { NOMAS_TEXT_QUERY_R = 0, NOMAS_TEXT_QUERY_K = 1, NOMAS_TEXT_QUERY_H = 2 };

/* Plan flags. */
enum {
  NOMAS_PLAN_HOST_ONLY = 1, /* build host tables only (no device upload);
                               such a plan cannot run nomas_attn_fwd/bwd */
  NOMAS_PLAN_GRAD_F32 = 2,  /* nomas_attn_bwd writes dq, dk, dv as fp32
                               (same layouts and element strides as the
                               bf16 gradients); without it they are bf16 */
  NOMAS_PLAN_KV_HEAD_MAJOR = 4 /* the new-token keys and values are head-major:
                               k_new / v_new of nomas_attn_fwd and k, v, dk,
                               dv of nomas_attn_bwd are [H][n][128], row r of
                               head h at element h * kv_stride + r * 128, and
                               kv_stride (>= n * 128, a multiple of 8) is the
                               stride between heads.  Without it they are
                               token-major [n][H][128] with token stride
                               kv_stride.  Queries, outputs and dO are
                               token-major either way.  Head-major rows make
                               each 64-key tile one contiguous 16 KB block
                               per head, which streams faster from HBM. */
};

typedef struct {
  int32_t num_heads;       /* >= 1                                        */
  int32_t head_dim;        /* must be 128                                 */
  int32_t block_q;         /* 0 = 128; the kernels support 128            */
  int32_t block_k;         /* 0 = 64; the kernels support 64              */
  int32_t text_query_mode; /* NOMAS_TEXT_QUERY_*                          */
  int32_t flags;           /* NOMAS_PLAN_*                                */
  int32_t window_segments; /* sliding window over segments: 0 = none; W >= 1:
                              a query of segment index s sees keys of
                              segment indices s - W + 1 .. s of its video
                              only (older segments, their heads included,
                              become invisible and their tiles EMPTY).  The
                              pages list sliding-window attention among the
                              single-GPU inference optimisations ("Summary
                              (Overview)", Inference) without its unit; a
                              whole-segment window is the reading taken.  */
  int32_t video_keep_percent; /* video-block sparsity: 0 = dense; P in
                              1..100: in every (head, query-tile pair) unit
                              only ceil(P% of its video key tiles) are
                              attended -- those with the highest block score
                              (below) -- while key tiles holding any head,
                              tail or padding token are always kept.  The
                              pages keep 25% of video blocks after the first
                              two denoising steps ("Summary (Overview)",
                              Inference) without stating the selection; the
                              score taken is the dot product of the unit's
                              query sum and the tile's key sum,
                              s = sum_d (sum_q Q[q,d]) * (sum_k K[k,d]),
                              i.e. the sum of the unit's logits over the
                              tile (up to the softmax scale); ties go to the
                              lower key tile.  The library evaluates s in
                              fp32 (row sums in groups of 16 rows, then the
                              group sums; products and adds rounded
                              separately; ascending d), deterministically, so
                              its ranking can differ from the exact one only
                              between tiles whose scores lie within that
                              evaluation's rounding error of each other.
                              Lists of any length (up to 4096 key tiles are
                              ranked by a sort in LDS, longer ones by a
                              radix select; the kept sets are the same).
                              Forward only.                                */
} nomas_plan_opts;

typedef struct nomas_plan nomas_plan;
typedef struct nomas_kvcache nomas_kvcache;
typedef struct nomas_kvcache_int8 nomas_kvcache_int8;

/* Tile classes as exported by nomas_plan_export_classes. */
enum { NOMAS_TILE_EMPTY = 0, NOMAS_TILE_FULL = 1, NOMAS_TILE_PARTIAL = 2 };

typedef struct {
  int64_t n_queries;
  int64_t n_keys;          /* cached + new                                 */
  int64_t n_cached_keys;
  int64_t n_q_tiles;
  int64_t n_k_tiles;
  int64_t n_empty_tiles;
  int64_t n_full_tiles;
  int64_t n_partial_tiles;
  int64_t unmasked_pairs;  /* A: number of visible (query, key) pairs      */
  int64_t executed_pairs;  /* pairs inside FULL + PARTIAL tiles (in range) */
  double effective_flop;   /* forward: 4 * head_dim * num_heads * A        */
  int32_t block_q;
  int32_t block_k;
  int32_t num_heads;
  int32_t text_query_mode;
  int64_t sparse_list_entries; /* per head: key tiles the units of a sparse
                                  plan attend (sum over units); 0 if dense */
  int32_t video_keep_percent;
  int32_t window_segments;
} nomas_plan_info;

/* --------------------------------------------------------------------------
 * Plans
 * ------------------------------------------------------------------------ */

/* Build a plan for one attention call shape.
 *   q       query tokens.
 *   kv_new  key/value tokens passed to each call (k_new / v_new).
 *   cache   NULL, or a KV cache whose committed segments precede kv_new in
 *           key order: keys = cache tokens (in append order) ++ kv_new.
 *           The plan remembers the cache's current contents (its segment
 *           records, in order) and is valid with any cache of the same head
 *           count holding exactly those segments -- this one, or another
 *           layer's cache with the same history; after an append or truncate
 *           that changes them, calls return NOMAS_ERR_STALE_PLAN.
 * Expands the records into per-token descriptors, classifies every
 * block_q x block_k tile as EMPTY, FULL or PARTIAL, builds per-q-tile and
 * per-k-tile lists of non-empty tiles and counts A, then (unless
 * NOMAS_PLAN_HOST_ONLY) copies the tables to the current HIP device
 * (synchronously).  *out is owned by the caller until nomas_plan_destroy.
 * Errors: INVALID_ARGUMENT, LAYOUT, UNSUPPORTED, HIP. */
nomas_status nomas_attn_plan(const nomas_layout* q, const nomas_layout* kv_new,
                             const nomas_kvcache* cache,
                             const nomas_plan_opts* opts, nomas_plan** out);

nomas_status nomas_plan_get_info(const nomas_plan* plan, nomas_plan_info* info);

/* Dense tile class map, row-major [n_q_tiles][n_k_tiles] of NOMAS_TILE_*.
 * n must be >= n_q_tiles * n_k_tiles. */
nomas_status nomas_plan_export_classes(const nomas_plan* plan, uint8_t* host_buf,
                                       size_t n);

nomas_status nomas_plan_destroy(nomas_plan* plan);

/* --------------------------------------------------------------------------
 * Forward
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace nomas_attn_fwd needs for this plan (may be 0). */
nomas_status nomas_attn_fwd_workspace_size(const nomas_plan* plan, size_t* bytes);

/* O = softmax(scale * Q K^T + M) V for the plan's queries.
 *   q, o          [n_queries][H][128], token strides q_stride / o_stride.
 *   k_new, v_new  [n_new_keys][H][128], token stride kv_stride.
 *   cache         a cache holding the plan's cached segments (NULL iff the
 *                 plan has none); its K/V buffers supply keys
 *                 [0, n_cached_keys).
 *   lse           NULL or fp32 [H][n_queries].
 *   workspace     device memory of nomas_attn_fwd_workspace_size bytes
 *                 (may be NULL when that size is 0).
 * Errors: INVALID_ARGUMENT (host-only plan, missing pointer or workspace),
 * STALE_PLAN, ALIGNMENT, HIP. */
nomas_status nomas_attn_fwd(const nomas_plan* plan, const nomas_kvcache* cache,
                            const void* q, int64_t q_stride,
                            const void* k_new, const void* v_new, int64_t kv_stride,
                            void* o, int64_t o_stride, float* lse, float scale,
                            void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/* The same forward for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: no workspace argument, and the call allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine).  Its workspace is a
 * fixed device array of the library, 64 MiB (NOMAS_NOALLOC_SCRATCH_BYTES),
 * which each device the library runs on holds until the process ends (its
 * address is resolved when a plan is first built on that device).  Results
 * are those of nomas_attn_fwd, bit for bit.  Every call on a device shares
 * that device's array, so calls that overlap on one device (concurrent
 * streams, threads) race; serialise them.  A plan whose
 * nomas_attn_fwd_workspace_size exceeds the array is rejected with
 * UNSUPPORTED before anything is enqueued.
 * Errors: as nomas_attn_fwd, and UNSUPPORTED (workspace above 64 MiB). */
#define NOMAS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
nomas_status nomas_attn_fwd_noalloc(const nomas_plan* plan, const nomas_kvcache* cache,
                                    const void* q, int64_t q_stride,
                                    const void* k_new, const void* v_new, int64_t kv_stride,
                                    void* o, int64_t o_stride, float* lse, float scale,
                                    void* hip_stream);

/* --------------------------------------------------------------------------
 * Backward (plans without a cache: training packs)
 * ------------------------------------------------------------------------ */

/* Workspace of nomas_attn_bwd: two fp32 row statistics per head and padded
 * query row, then 256 bytes of work-queue counters (never zero bytes).  A
 * workspace serves one backward call at a time: calls that overlap on the
 * device need one workspace each. */
nomas_status nomas_attn_bwd_workspace_size(const nomas_plan* plan, size_t* bytes);

/* Gradients of O = attention(Q, K, V) for upstream dO:
 *   dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)), dQ = scale dS K,
 *   dK = scale dS^T Q,
 * (the calculus of the softmax attention defined above) with P recomputed as
 * exp(scale * (Q K^T) - lse) from Q and K as given and lse from
 * nomas_attn_fwd on the same inputs.  q, o, d_o, dq share q_stride; k, v, dk,
 * dv share kv_stride (elements).  dq, dk, dv are written (not accumulated):
 * bf16, or fp32 if the plan was built with NOMAS_PLAN_GRAD_F32.  Workgroups
 * claim their units (key-tile pairs, query-tile pairs) from counters in the
 * workspace, but each unit is summed by one workgroup in a fixed order, with
 * no atomic adds on values: equal inputs give bit-identical gradients.
 * Errors: INVALID_ARGUMENT (plan with a cache, host-only plan, missing
 * pointer or workspace), UNSUPPORTED (video-block sparse plan), ALIGNMENT,
 * HIP. */
nomas_status nomas_attn_bwd(const nomas_plan* plan,
                            const void* q, const void* k, const void* v,
                            const void* o, const void* d_o, const float* lse,
                            int64_t q_stride, int64_t kv_stride,
                            void* dq, void* dk, void* dv, float scale,
                            void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/* --------------------------------------------------------------------------
 * KV cache ("One World, Generated Segment by Segment": each segment's K/V is
 * appended to a permanent, growing cache)
 * ------------------------------------------------------------------------ */

/* k_buf / v_buf: caller-owned device memory, bf16 [heads][capacity][128]
 * (head-major, so one head's keys are contiguous).  The handle (segment
 * records, lengths) is library-owned. */
nomas_status nomas_kvcache_create(int32_t heads, int32_t head_dim, int64_t capacity,
                                  void* k_buf, void* v_buf, nomas_kvcache** out);

/* Append one segment: k_new / v_new hold its tokens' K/V, [tokens][H][128]
 * (token stride kv_stride) in the segment's token order.  The cache keeps the
 * rows a later segment can see -- the video and head tokens, which come first
 * -- and copies them behind the cached rows on hip_stream; the action-tail
 * and padding rows are not stored (action tails are visible only inside their
 * own segment, "Model Architecture": Action-Aware Causal Attention).
 * Capacity is counted in stored rows.  Over capacity: NOMAS_ERR_CAPACITY and
 * nothing is written or recorded.  A segment already in the cache:
 * NOMAS_ERR_LAYOUT. */
nomas_status nomas_kvcache_append(nomas_kvcache* cache, const nomas_segment* seg,
                                  const void* k_new, const void* v_new,
                                  int64_t kv_stride, void* hip_stream);

/* Drop segments so that n_segments remain (rollback).  Plans built when the
 * cache held exactly those segments become valid again. */
nomas_status nomas_kvcache_truncate(nomas_kvcache* cache, int32_t n_segments);

/* Resume a cache: an empty handle (just created, or reset) takes on the
 * segments whose rows are already in its buffers -- written by appends to a
 * cache over the same buffers, or saved and restored by the caller -- in
 * append order, segment i's stored rows (video and head tokens) following
 * those of segments 0 .. i-1 from row 0 of every head.  Nothing is copied or
 * launched; plans built for these segments are valid with it.  The pages'
 * cache is permanent and grows segment by segment ("One World, Generated
 * Segment by Segment"); this lets a session continue in a new process.
 * Errors: INVALID_ARGUMENT (NULL, cache not empty), LAYOUT (malformed record,
 * a segment listed twice), CAPACITY (rows beyond capacity); on error nothing
 * is recorded. */
nomas_status nomas_kvcache_adopt(nomas_kvcache* cache, const nomas_segment* segments,
                                 int32_t n_segments);

nomas_status nomas_kvcache_reset(nomas_kvcache* cache);
/* n_tokens: stored rows (video + head tokens of the cached segments). */
nomas_status nomas_kvcache_len(const nomas_kvcache* cache, int64_t* n_tokens,
                               int32_t* n_segments);
nomas_status nomas_kvcache_destroy(nomas_kvcache* cache);

/* --------------------------------------------------------------------------
 * INT8 KV cache ("Summary (Overview)", Inference: INT8 KV-cache quantization
 * among the single-GPU optimisations; the scheme is not given)
 *
 * Rows are kept as the bf16 cache keeps them (each segment's video and head
 * tokens, head-major), but quantized: a (head, token) row of 128 values x is
 * stored as 128 int8 codes q and one int8 exponent e, where e is the smallest
 * integer with max |x| <= 127 * 2^e (0 for a zero row, at least -127) and
 * q = x / 2^e rounded to the nearest integer, ties to even.  The stored value
 * q * 2^e is exact in bf16, so attention over it is exact attention over the
 * dequantized cache.  Inputs must be finite.  About half the bytes of a bf16
 * cache (129 B per row instead of 256).
 *
 * The attention kernels read bf16 tiles: nomas_kvcache_int8_expand writes the
 * dequantized rows into a bf16 working cache once per (layer, segment step),
 * and the four denoising calls of the step run on it; the INT8 caches are the
 * resident archive of every layer.
 * ------------------------------------------------------------------------ */

/* k_codes / v_codes: caller-owned device memory, int8 [heads][capacity][128];
 * k_exp / v_exp: int8 [heads][capacity]; all 16-byte aligned.  The handle is
 * library-owned.  Errors: INVALID_ARGUMENT, UNSUPPORTED (head_dim != 128),
 * ALIGNMENT. */
nomas_status nomas_kvcache_int8_create(int32_t heads, int32_t head_dim, int64_t capacity,
                                       void* k_codes, void* v_codes, void* k_exp,
                                       void* v_exp, nomas_kvcache_int8** out);

/* As nomas_kvcache_append, quantizing the stored rows on hip_stream. */
nomas_status nomas_kvcache_int8_append(nomas_kvcache_int8* cache, const nomas_segment* seg,
                                       const void* k_new, const void* v_new,
                                       int64_t kv_stride, void* hip_stream);

/* Make dst (a bf16 cache of the same head count) hold the dequantized rows
 * and the segment records of cache: rows [0, len) of every head are written
 * on hip_stream, dst's previous contents are replaced.  A plan built for
 * these segments is valid with dst afterwards (also across layers).
 * Errors: INVALID_ARGUMENT (NULL, head counts differ), CAPACITY (dst too
 * small; nothing written), HIP. */
nomas_status nomas_kvcache_int8_expand(const nomas_kvcache_int8* cache, nomas_kvcache* dst,
                                       void* hip_stream);

/* As nomas_kvcache_adopt, for codes and exponents already in an INT8
 * cache's buffers. */
nomas_status nomas_kvcache_int8_adopt(nomas_kvcache_int8* cache, const nomas_segment* segments,
                                      int32_t n_segments);

nomas_status nomas_kvcache_int8_truncate(nomas_kvcache_int8* cache, int32_t n_segments);
nomas_status nomas_kvcache_int8_len(const nomas_kvcache_int8* cache, int64_t* n_tokens,
                                    int32_t* n_segments);
nomas_status nomas_kvcache_int8_destroy(nomas_kvcache_int8* cache);

/* --------------------------------------------------------------------------
 * Camera cross-attention ("Summary (Overview)", Model Architecture:
 * Camera-Trajectory Conditioning, Eq. 3; gpts24.com, "Inside the
 * Architecture: Dual Stream, Language Encoder, and Explicit Camera Math")
 *
 * Video tokens are the queries, camera tokens the keys and values; the
 * result is what Eq. 3 adds to the video tokens.  A camera token stands for
 * a group of four frames, i.e. one latent frame, so a segment of n_frames
 * latent frames has n_frames camera tokens; the camera tokens of a layout
 * are its segments' tokens concatenated in segment order (segment i's
 * frame g is camera token c_i + g, c_i = sum of n_frames before i).
 * Visibility (the pages state none; the reading taken): a video token of
 * latent frame f in segment i sees camera tokens c_i + g of its own segment
 * with |f - g| <= radius_frames; radius_frames < 0 means every camera token
 * of segment i, and 0 the time-aligned reading (its own frame only).  Text
 * and padding tokens are not queries: their output rows are written as 0.
 * The projections (64-dim camera vectors to heads x 128, and of the output)
 * are the caller's.
 * ------------------------------------------------------------------------ */

typedef struct nomas_camera_plan nomas_camera_plan;

typedef struct {
  int64_t n_queries;          /* tokens of the layout (rows of q and o)    */
  int64_t n_video_queries;
  int64_t n_camera_tokens;    /* sum of n_frames                           */
  int64_t visible_pairs;      /* visible (video token, camera token) pairs */
  double effective_flop;      /* 4 * 128 * heads * visible_pairs           */
  double algorithmic_bytes;   /* q and o rows + k_cam and v_cam rows, bf16 */
  int32_t num_heads;
  int32_t radius_frames;      /* -1 = whole segment                        */
} nomas_camera_plan_info;

/* Build the per-token camera ranges of a query layout (records validated as
 * for nomas_attn_plan) and, unless flags holds NOMAS_PLAN_HOST_ONLY, copy
 * them to the current HIP device (synchronously).  *out is owned by the
 * caller until nomas_camera_plan_destroy.
 * Errors: INVALID_ARGUMENT (NULL pointer, num_heads < 1, unknown flag),
 * LAYOUT, UNSUPPORTED (2^31 tokens or more), HIP. */
nomas_status nomas_camera_attn_plan(const nomas_layout* q, int32_t num_heads,
                                    int32_t radius_frames, int32_t flags,
                                    nomas_camera_plan** out);

nomas_status nomas_camera_plan_get_info(const nomas_camera_plan* plan,
                                        nomas_camera_plan_info* info);

/* Per query token, the camera tokens it sees: host_buf int32
 * [n_queries][2] = {first, end} (first == end: none).  n must be >=
 * 2 * n_queries. */
nomas_status nomas_camera_plan_export_ranges(const nomas_camera_plan* plan,
                                             int32_t* host_buf, size_t n);

nomas_status nomas_camera_plan_destroy(nomas_camera_plan* plan);

/* O = softmax(scale * Q K_cam^T + M) V_cam for every token of the plan's
 * layout (0 for rows that see no camera token).
 *   q, o          [n_queries][H][128] bf16, token strides q_stride / o_stride.
 *   k_cam, v_cam  [n_camera_tokens][H][128] bf16, token stride cam_stride
 *                 (may be NULL when the layout has no camera token).
 * Enqueued on hip_stream; allocates nothing.
 * Errors: INVALID_ARGUMENT (host-only plan, plan of another device, missing
 * pointer, bad stride or scale), ALIGNMENT, HIP. */
nomas_status nomas_camera_attn_fwd(const nomas_camera_plan* plan,
                                   const void* q, int64_t q_stride,
                                   const void* k_cam, const void* v_cam,
                                   int64_t cam_stride, void* o, int64_t o_stride,
                                   float scale, void* hip_stream);

/* --------------------------------------------------------------------------
 * Action windows in latent frames
 * ------------------------------------------------------------------------ */

/* The latent frames an action acts on, from its span in pixel frames.  The
 * video autoencoder compresses time 4x ("Summary (Overview)", Theoretical
 * Foundation, Eq. 1: F pixel frames give floor((F - 1) / 4) + 1 latent
 * frames); the grouping taken is the causal one that count implies: latent
 * frame 0 holds pixel frame 0 alone, latent frame i >= 1 pixel frames
 * 4i - 3 .. 4i, and frames of a trailing incomplete group belong to none.
 * An action over pixel frames [first, end) of a segment of n_pixel_frames
 * frames gets the window [*lo, *hi) of every latent frame holding one of
 * its frames (the frame_lo / frame_hi of nomas_action); *lo == *hi when
 * all of its frames are in the dropped trailing group.
 * Errors: INVALID_ARGUMENT (NULL output, first < 0, end <= first,
 * end > n_pixel_frames). */
nomas_status nomas_action_latent_window(int64_t first, int64_t end, int64_t n_pixel_frames,
                                        int32_t* lo, int32_t* hi);

/* --------------------------------------------------------------------------
 * Errors
 * ------------------------------------------------------------------------ */

const char* nomas_status_string(nomas_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* nomas_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NOMAS_ATTN_H */
