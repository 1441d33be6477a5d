/*
 * wave.h -- C ABI of chunk-wise block-causal "wave" attention on AMD gfx950.
 *
 * What the calls compute
 * ----------------------
 * A streaming video diffusion model denoises B chunks through K levels.  The
 * update of chunk i at level j attends to its own tokens (both directions)
 * and to the K/V of earlier chunks, never later ones; which level of each
 * earlier chunk it reads is set by a context policy phi(j, r) of the level j
 * and the chunk distance r (streaming-video-diffusion design-space paper,
 * thelatestinai.com listing of arXiv 2609.22283: Figure 1, Table 1):
 *   clean        phi = 0             (fully denoised history)
 *   same-level   phi = j
 *   progressive  phi = max(j - r, 0)
 * Run serially, the B*K updates take B*K rounds; pipelined, chunks sit at
 * staggered levels and the same B*K updates take B+K-1 rounds (same paper,
 * Figure 2).  Wave Forcing (aiany.app summary, mechanism paragraph) hands K/V
 * to later chunks early, within the round; Wan-Streamer v0.2 (abstract) writes
 * incoming K/V into a cache and passes language/state to the generator only as
 * a K/V slice (here: an optional per-chunk conditioning slot).
 *
 *   wave_plan   (host)   builds the (chunk, level) nodes, their gather lists
 *                        (context slots in timeline order), the rounds, the
 *                        physical cache slots and a packed device descriptor.
 *   kv_write    (device) copies one round's fresh K/V into the cache slots.
 *   wave_attn   (device) block-causal flash attention of one round: every
 *                        query chunk of the round against exactly the slots of
 *                        its gather list; masked slots are never read.
 *
 * Conventions
 * -----------
 * Levels: 0 = clean, K = pure noise.  Update U(i, j), j = K..1, consumes
 * chunk i at level j and writes slot (i, j).  The clean slot (i, 0) is written
 * by a refresh node R(i) (a forward pass over the finished chunk), created
 * only when some node reads (i, 0).  A conditioning slot C(i) (level
 * WAVE_LEVEL_COND) is written with chunk i's first update when cond_len > 0.
 * A node may read a slot written in an earlier round, or earlier in the same
 * round by a lower chunk: each round's kv_write precedes its wave_attn.
 *
 * All int32 status returns: WAVE_OK or a negative WAVE_ERR_*; the message of
 * the last failure on the calling thread is returned by wave_last_error().
 * No C++ exception crosses this boundary.  The library never allocates or
 * frees device memory: every device buffer belongs to the caller, except the
 * fixed per-device scratch array behind wave_attn_splitkv_noalloc, which
 * comes with the library's code object.
 */
#ifndef WAVE_H
#define WAVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  WAVE_OK = 0,
  WAVE_ERR_INVALID_ARG = -1, /* null pointer, out-of-range value, bad round */
  WAVE_ERR_CAPACITY = -2,    /* cache has fewer slots / shorter lpad than the plan needs */
  WAVE_ERR_UNSUPPORTED = -3, /* head_dim, dtype or q_tile the kernels do not handle */
  WAVE_ERR_HIP = -4,         /* a HIP launch reported an error */
  WAVE_ERR_NOMEM = -5        /* host allocation failed */
};

enum { WAVE_CLEAN = 0, WAVE_SAME_LEVEL = 1, WAVE_PROGRESSIVE = 2 };
enum { WAVE_SCHED_SERIAL = 0, WAVE_SCHED_WAVE = 1 };
enum { WAVE_NODE_UPDATE = 0, WAVE_NODE_REFRESH = 1 };
enum { WAVE_DTYPE_BF16 = 0, WAVE_DTYPE_FP32 = 1 };
#define WAVE_LEVEL_COND (-1)

/* Query rows per attention work item; wave_attn handles this value only. */
#define WAVE_Q_TILE 256
/* Keys per streamed K/V tile; cache lpad must be a multiple of it. */
#define WAVE_KEY_TILE 64

typedef struct wave_plan_params {
  int32_t B;           /* chunks, >= 1 */
  int32_t K;           /* denoising levels (updates per chunk), >= 1 */
  int32_t policy;      /* WAVE_CLEAN / WAVE_SAME_LEVEL / WAVE_PROGRESSIVE */
  int32_t sched;       /* WAVE_SCHED_SERIAL / WAVE_SCHED_WAVE */
  int32_t history_cap; /* H: earlier chunks visible, -1 = all, >= 0 = the last H */
  int32_t chunk_len;   /* tokens per chunk: query rows of a node, length of its slot, >= 1 */
  int32_t cond_len;    /* tokens of each conditioning slot C(i); 0 = no conditioning */
  int32_t q_tile;      /* query rows per work item; 0 = WAVE_Q_TILE */
  int32_t query_len;   /* query rows of every node; 0 = chunk_len.  Fewer rows than the
                          chunk's slot (e.g. only a chunk's audio tokens) give the
                          decode-shaped case: short queries against long contexts. */
} wave_plan_params;

/* One logical cache slot as referenced by a node. */
typedef struct wave_slot_ref {
  int32_t chunk;     /* chunk index */
  int32_t level;     /* 0..K, or WAVE_LEVEL_COND */
  int32_t phys_slot; /* physical slot index in the per-layer cache */
  int32_t len;       /* valid tokens in the slot (chunk_len or cond_len) */
} wave_slot_ref;

typedef struct wave_node {
  int32_t chunk, level, kind, round;
  int32_t q_offset;    /* first row of this node in the round's packed Q / O */
  int32_t q_len;       /* query rows (query_len, else chunk_len) */
  int32_t ctx_begin;   /* gather list: ctx[ctx_begin .. ctx_begin+ctx_count), timeline order, own slot last */
  int32_t ctx_count;
  int32_t write_begin; /* slots this node writes: writes[write_begin ..), conditioning first */
  int32_t write_count;
} wave_node;

/* Attention work item: query rows [q_start, q_start+q_rows) of one node. */
typedef struct wave_work {
  int32_t node;    /* global node index */
  int32_t q_start; /* row offset inside the node */
  int32_t q_rows;  /* <= q_tile */
  int32_t keys;    /* total keys over the node's gather list */
} wave_work;

/* Read-only view of a plan.  All arrays belong to the plan and stay valid
 * until wave_plan_destroy.  Nodes are grouped by round, ascending chunk inside
 * a round; writes and ctx entries are grouped by node in node order; a
 * round's work items are sorted by decreasing cost. */
typedef struct wave_plan_view {
  int32_t num_rounds, num_nodes, num_ctx, num_writes, num_work;
  int32_t num_phys_slots; /* cache slots per layer the plan needs */
  int32_t max_slot_len;   /* longest slot, tokens */
  int32_t q_tile;
  const int32_t* round_node_begin;  /* [num_rounds+1] */
  const int32_t* round_write_begin; /* [num_rounds+1] */
  const int32_t* round_work_begin;  /* [num_rounds+1] */
  const int32_t* round_q_rows;      /* [num_rounds]: rows of the round's packed Q / O */
  const int32_t* round_src_rows;    /* [num_rounds]: rows of the round's packed fresh K/V */
  const wave_node* nodes;
  const wave_slot_ref* ctx;
  const wave_slot_ref* writes;
  const wave_work* work;
} wave_plan_view;

typedef struct wave_plan wave_plan_t;

/* Build a plan on the host.  Deterministic: equal params give an identical
 * view and descriptor.  *out receives a new plan owned by the caller (free
 * with wave_plan_destroy); a plan is immutable and may be shared by threads. */
int32_t wave_plan(const wave_plan_params* params, wave_plan_t** out);
int32_t wave_plan_view_get(const wave_plan_t* plan, wave_plan_view* out);
/* Size in bytes of the packed device descriptor (int32 words). */
int32_t wave_plan_desc_size(const wave_plan_t* plan, size_t* bytes);
/* Write the descriptor into host memory [host_dst, host_dst+bytes); the caller
 * uploads it once to device memory and passes that pointer as d_desc. */
int32_t wave_plan_desc_pack(const wave_plan_t* plan, void* host_dst, size_t bytes);
void wave_plan_destroy(wave_plan_t* plan);

/* Per-layer K/V cache, device memory owned by the caller.
 *   k : bf16 [num_slots][heads][lpad][head_dim]  (token-major per head)
 *   vt: bf16 [num_slots][heads][head_dim][lpad]  (V transposed per head, so
 *       the P.V contraction streams keys contiguously)
 * lpad >= the plan's max_slot_len, a multiple of WAVE_KEY_TILE, and
 * (head_dim-1)*lpad*2 + 2*WAVE_KEY_TILE <= INT32_MAX (about 8.4 M tokens at
 * head_dim 128; WAVE_ERR_UNSUPPORTED above).  Tokens [len, lpad) of a
 * written slot are zero. */
typedef struct wave_kv_cache {
  void* k;
  void* vt;
  int32_t num_slots;
  int32_t heads;
  int32_t head_dim; /* 64 or 128 */
  int32_t lpad;
} wave_kv_cache;

/* Copy the fresh K/V of round `round` into their physical slots and zero
 * each slot's tail [len, lpad).  k_src, v_src: device [src_rows][heads][head_dim]
 * of dtype src_dtype (bf16 copied, fp32 rounded to bf16 to nearest even),
 * token row stride src_row_stride elements (>= heads*head_dim), rows packed in
 * the round's write order (view.writes[round_write_begin[round] ..]).
 * d_desc: device copy of this plan's descriptor.  stream: hipStream_t (NULL =
 * default stream).  Asynchronous; never synchronises.  A round with no writes
 * is a no-op. */
int32_t kv_write(const wave_plan_t* plan, const void* d_desc, int32_t round,
                 const wave_kv_cache* cache, const void* k_src, const void* v_src,
                 int32_t src_dtype, int64_t src_row_stride, void* stream);

/* Workspace of wave_attn's tail balancing for round `round`, `heads` heads of
 * `head_dim` on a device of `compute_units` compute units (0 = the current
 * device).  wave_attn runs one workgroup per (work item, head) in the plan's
 * work order, most key tiles first; when those workgroups do not divide
 * evenly over the compute units, the last of them run on a part-empty chip.
 * The library picks, from a simulation of that in-order dispatch, the number
 * of trailing work items to cut into contiguous key-tile ranges (1 to 4
 * pieces, merged by a second kernel as in wave_attn_splitkv).  *bytes = 0
 * when no cut pays off.  tail_items, tail_splits (may be NULL) receive the
 * choice.  The choice is memoised in the plan; this call is thread-safe. */
int32_t wave_attn_workspace(const wave_plan_t* plan, int32_t round, int32_t heads,
                            int32_t head_dim, int32_t compute_units, size_t* bytes,
                            int32_t* tail_items, int32_t* tail_splits);

/* Block-causal attention of every node of round `round`.
 *   q  : device [round_q_rows][heads][head_dim], dtype q_dtype (bf16, or fp32
 *        rounded to bf16 to nearest even on load), row stride q_row_stride elements.
 *   o  : device bf16 [round_q_rows][heads][head_dim], dense.
 *   lse: device fp32 [heads][round_q_rows] natural-log sum of exp of the scaled
 *        scores, or NULL.
 *   workspace: NULL, or device memory of at least wave_attn_workspace() bytes
 *        (current device), 256-byte aligned, owned by the caller, scratch
 *        after the call: enables tail balancing.
 * scale multiplies Q.K (typically 1/sqrt(head_dim)).  Softmax in fp32, both
 * contractions in bf16 with fp32 accumulation.  Without a workspace, each
 * node's result depends on its query rows and the contents of its gather list
 * only, with a fixed reduction order, so it is bitwise the same in any
 * schedule; with one, the nodes of cut items differ from that by rounding
 * (another reduction order).  The plan's q_tile must be WAVE_Q_TILE.
 * Asynchronous on `stream`; calls that share a workspace must be ordered on
 * one stream. */
int32_t wave_attn(const wave_plan_t* plan, const void* d_desc, int32_t round,
                  const wave_kv_cache* cache, const void* q, int32_t q_dtype,
                  int64_t q_row_stride, void* o, float* lse, float scale,
                  void* workspace, size_t workspace_bytes, void* stream);

/* One wave round of every layer: for each layer l in order, kv_write of the
 * round's fresh K/V into caches[l], then wave_attn of the round's nodes on
 * that cache, all on `stream` with no host synchronisation (a round is one
 * concurrent forward pass over the chunks in flight, with each chunk's K/V in
 * the cache before the attention that reads it: Wave Forcing summary,
 * mechanism paragraph; Wan-Streamer v0.2 abstract).
 *   num_layers: >= 1; caches, k_src, v_src, q, o: arrays of num_layers
 *               entries, one per layer, each as for kv_write / wave_attn;
 *   lse: NULL, or an array of num_layers entries (entries may be NULL).
 *   src_dtype, src_row_stride, q_dtype, q_row_stride, scale: shared by the
 *               layers.
 *   workspace: as for wave_attn (NULL, or >= wave_attn_workspace() bytes);
 *               the layers reuse it one after another on `stream`.
 * Every layer's arguments are checked before anything is enqueued; an error
 * names the layer.  A launch error part-way leaves the earlier layers'
 * launches enqueued.  Results equal those of the separate calls. */
int32_t wave_round(const wave_plan_t* plan, const void* d_desc, int32_t round, int32_t num_layers,
                   const wave_kv_cache* caches, const void* const* k_src, const void* const* v_src,
                   int32_t src_dtype, int64_t src_row_stride, const void* const* q, int32_t q_dtype,
                   int64_t q_row_stride, void* const* o, float* const* lse, float scale,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Split-KV attention for short query chunks against long contexts (the
 * decode-shaped case: e.g. a chunk's 64 audio rows against tens of thousands
 * of cached keys, Wan-Streamer v0.2 abstract and "Latency-Preserving
 * Infrastructure": audio latents are short and handled unsharded).  Each
 * node's key tiles (gather list order) are cut into num_splits contiguous
 * ranges processed by separate workgroups; a second kernel merges them:
 * LSE = log sum_k exp(LSE_k), O = sum_k exp(LSE_k - LSE) O_k.  Results equal
 * wave_attn's up to rounding (the reduction order differs).
 *   num_splits: >= 1, or 0 to let the library choose from the round's work
 *               and the current device's compute-unit count: the most splits
 *               whose workgroups (work items x heads x splits) fill the units
 *               in one dispatch wave, 1..64.
 *   workspace : device memory of at least wave_attn_splitkv_workspace()
 *               bytes, 256-byte aligned, owned by the caller; its contents
 *               need no initialisation and are scratch after the call.
 * Other arguments as for wave_attn.  Asynchronous on `stream`; calls that
 * share a workspace must be ordered on one stream. */
int32_t wave_attn_splitkv_workspace(const wave_plan_t* plan, int32_t round, int32_t heads,
                                    int32_t head_dim, int32_t num_splits, size_t* bytes,
                                    int32_t* splits_used);
int32_t wave_attn_splitkv(const wave_plan_t* plan, const void* d_desc, int32_t round,
                          const wave_kv_cache* cache, const void* q, int32_t q_dtype,
                          int64_t q_row_stride, void* o, float* lse, float scale,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of device scratch behind wave_attn_splitkv_noalloc. */
#define WAVE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* wave_attn_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial results live in a
 * library-owned array of WAVE_NOALLOC_SCRATCH_BYTES per device, created with
 * the library's code object on each device and held until the process ends;
 * this call allocates and frees no device memory.  A call whose split count
 * needs more than that (wave_attn_splitkv_workspace() bytes) fails with
 * WAVE_ERR_CAPACITY before any launch; num_splits = 1 needs none.  Every call
 * on one device shares that device's array and overwrites it: calls that
 * overlap on one device (different streams, or different threads without
 * ordering) race and must not be issued.  Results equal wave_attn_splitkv's
 * with the same split count.  Other arguments as for wave_attn_splitkv. */
int32_t wave_attn_splitkv_noalloc(const wave_plan_t* plan, const void* d_desc, int32_t round,
                                  const wave_kv_cache* cache, const void* q, int32_t q_dtype,
                                  int64_t q_row_stride, void* o, float* lse, float scale,
                                  int32_t num_splits, void* stream);

/* ---- Toy denoiser chain: the steps on either side of the attention ----
 *
 * The pages carry no model weights; a seeded stand-in closes the loop between
 * denoising levels so that a chunk's next node consumes its previous node's
 * result (Wave Forcing summary, mechanism paragraph; design-space paper,
 * Figure 2: a chunk advances one denoising step per round, and the refresh
 * pass consumes the finished chunk).  Per layer of a node:
 *   [Q | K | V] = bf16( (A W^T) / rms(A) ),  rms(a) = sqrt(mean_c a_c^2 + 1e-6)
 * A: the node's input rows [chunk_len][D], D = heads * head_dim; W [3D][D].
 * The chain needs plans with cond_len = 0 and query rows = chunk tokens. */

/* x_layout of qkv_project */
#define WAVE_X_ROUND 0 /* x is [round_q_rows][D], packed like the round's Q (e.g. the previous layer's O) */
#define WAVE_X_CHUNK 1 /* x is per-chunk state [B][chunk_len][D] (chain_store's layout) */

/* wave_attn that also hands the next layer its RMS statistics: row_sq
 * (device fp32 [round_q_rows][heads], 4-byte aligned, or NULL for none)
 * receives, for every output row and head, the sum over head_dim of the
 * squares of the bf16 O values written.  The next layer's qkv_project takes
 * it with x = this o, instead of a pass over x's rows (the per-token
 * normalisation of the toy chain; fused here into the kernel that produces
 * the rows).  Other arguments, results and behaviour as for wave_attn. */
int32_t wave_attn_chain(const wave_plan_t* plan, const void* d_desc, int32_t round,
                        const wave_kv_cache* cache, const void* q, int32_t q_dtype,
                        int64_t q_row_stride, void* o, float* lse, float scale, float* row_sq,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of qkv_project for round `round`: one fp32 per query row. */
int32_t qkv_project_workspace(const wave_plan_t* plan, int32_t round, size_t* bytes);

/* QKV projection of every node of round `round` at one layer.
 *   cache: the layer's cache; each node's K and V^T go into its own slot (the
 *          last entry of its gather list), tokens [chunk_len, lpad) zeroed.
 *          Replaces kv_write for chain rounds.
 *   x    : device bf16 input rows, layout x_layout.
 *   row_sq: NULL, or wave_attn_chain's row_sq of the call whose o is x
 *          (x_layout must then be WAVE_X_ROUND): rms(row) is taken as
 *          sqrt(sum_h row_sq[row][h] / D + 1e-6) instead of from x's rows.
 *   w    : device bf16 [3D][D]; row o holds output column o's weights
 *          (o < D: Q, then K, then V; column = head * head_dim + dim).
 *   q    : device bf16 [round_q_rows][heads][head_dim] (wave_attn's q).
 *   workspace: >= qkv_project_workspace() bytes, 256-byte aligned.
 * D must be a multiple of 128.  Asynchronous on `stream`. */
int32_t qkv_project(const wave_plan_t* plan, const void* d_desc, int32_t round,
                    const wave_kv_cache* cache, const void* x, int32_t x_layout,
                    const float* row_sq, const void* w, void* q, void* workspace,
                    size_t workspace_bytes, void* stream);

/* state[chunk(n)] = o[rows of n] for every node n of round `round`:
 *   o    : device bf16 [round_q_rows][model_dim] (wave_attn's o of the last layer).
 *   state: device bf16 [B][chunk_len][model_dim].
 * model_dim a positive multiple of 8.  Asynchronous on `stream`. */
int32_t chain_store(const wave_plan_t* plan, const void* d_desc, int32_t round, int32_t model_dim,
                    const void* o, void* state, void* stream);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call into this library from the same thread. */
const char* wave_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WAVE_H */
