/*
 * zha.h - C ABI of the ZHA decode hot path on AMD Instinct MI355X (gfx950).
 *
 * ZHA (Zyphra Hierarchical Attention) keeps the full KV cache and builds a
 * tree index over it; a decode query walks the tree top-down with per-level
 * top-p selection and then runs exact attention over the keys it reached.
 *
 * Sources (web pages, cited by title and section):
 *   MTP = "Zyphra AI Introduces Zyphra Hierarchical Attention (ZHA): A Path to
 *         True Subquadratic Attention" (MarkTechPost article with its
 *         explainer widget).
 *   LC  = "Zyphra Hierarchical Attention" (lesscarbs.net), "What happened?".
 *
 * Conventions for every entry point:
 *   - Every pointer argument named *device* is device memory owned by the
 *     caller; the library never allocates, frees or retains device memory and
 *     keeps no global mutable state apart from a thread-local error string
 *     (and, for zha_attend_noalloc, one static scratch array per GPU and a
 *     table of their addresses).
 *   - Calls are asynchronous and ordered on the given HIP stream (a
 *     hipStream_t passed as void*; NULL = the default stream).  No call
 *     synchronises the host.  Device faults surface at the caller's next
 *     synchronisation.  NaN/Inf inputs are not sanitised and propagate.
 *   - All argument checks run on the host before any HIP call; a failed check
 *     returns a negative zha_status and launches nothing.  zha_last_error()
 *     then describes the failure.
 *   - Two calls may run concurrently on different streams when they write to
 *     distinct buffers.
 *
 * Shapes.  B sequences, H KV heads, G query heads per KV head, d head dim,
 * R reference queries, C chunk size, Lv levels, T queries per query head.
 * A "cache" is one (sequence, KV head) pair with its own tree; cache index
 * = b * H + h.  Query index = ((b * H + h) * G + g) * T + t.
 */
#ifndef ZHA_H_
#define ZHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZHA_VERSION 1
#define ZHA_MAX_LEVELS 8

/* Status codes returned by every int-returning entry point. */
enum zha_status {
  ZHA_OK = 0,
  ZHA_ERR_NULL = -1,        /* a required pointer is NULL */
  ZHA_ERR_ARG = -2,         /* bad dimension, p outside (0, 1], T <= 0, n_old mismatch, ... */
  ZHA_ERR_UNSUPPORTED = -3, /* valid but not implemented (head_dim, chunk, n_ref, dtype) */
  ZHA_ERR_CAPACITY = -4,    /* tokens beyond capacity, or a buffer too small */
  ZHA_ERR_ALIGN = -5,       /* a row or base pointer is not 16-byte aligned */
  ZHA_ERR_HIP = -6          /* a HIP call or launch failed (text in zha_last_error) */
};

/* Element types of K, V, Q and of the stored mean keys g. */
enum zha_dtype { ZHA_F32 = 0, ZHA_BF16 = 1 };

/*
 * Storage form of level-1 nodes.
 *   ZHA_LEAF_MEAN: like every other level, the node stores its mean keys
 *     g_j (kv_dtype), L_j and c_j = L_j - r_j . g_j / sqrt(d).
 *   ZHA_LEAF_WEIGHTS: the node stores the softmax weights of its own C keys,
 *     w_ji = exp(z_ji - L_j) ([R][C] fp32), L_j and c_j = L_j - sum_i w_ji z_ji.
 *     Since g_j = sum_i w_ji k_i, the tangent-plane score of a level-1 node is
 *     computed from the raw keys as max_j [c_j + sum_i w_ji q . k_i / sqrt(d)]
 *     (the same plane with g_j unrounded).  A level-1 node then occupies
 *     R*(4C+8) bytes instead of R*(d*esize+8), and routing reads the chunk's
 *     C*d key elements instead of R*d mean-key elements.  Supported with bf16
 *     and chunk in {4, 8, 16}.  Levels >= 2 are the same in both forms.
 *   ZHA_LEAF_WEIGHTS2: level 1 as in ZHA_LEAF_WEIGHTS; a level-2 node
 *     stores its C children's mass shares rho_cj = exp(L_j(child c) - L_j)
 *     ([R][C] fp32; 0 for the children a trailing node lacks), L_j and
 *     c_j = L_j - sum_i w_ji z_ji over its C*C keys, where the node's weight
 *     of key i in child c is rho_cj times the child's own w_ji.  Routing
 *     scores level 2 from its raw keys (the same plane with g unrounded);
 *     with at most 4 queries per cache and routing from level 2 or above,
 *     that pass also forms the level-1 scores of its children (the keys of
 *     a candidate are read once) and keeps the logits when the caller
 *     passes the buffer; that pass reads only the keys: it recomputes the
 *     log masses L of the node and of its children, the weights, shares and
 *     c from the reference queries the tree keeps (ref_offset) and the keys,
 *     to fp32 rounding of the stored ones.  A level-2 node occupies R*(4C+8) bytes instead of
 *     R*(2d+8).  Supported with bf16, chunk 4 and 3..8 levels, with either
 *     g_dtype (ZHA_G_FP8 then stores levels >= 3 in fp8); not with the
 *     prefill calls (zha_build_spine, zha_route_prefill).  Levels >= 3 are
 *     the same in every form.
 */
enum zha_leaf_form { ZHA_LEAF_MEAN = 0, ZHA_LEAF_WEIGHTS = 1, ZHA_LEAF_WEIGHTS2 = 2 };

/*
 * Storage of the mean keys g of the levels that store them (every level but
 * those the leaf form stores as weights).
 *   ZHA_G_KV: kv_dtype.
 *   ZHA_G_FP8: the low-precision router variant (MTP TL;DR, "FP4 router"),
 *     read as OCP FP8 E4M3 with one power-of-two scale per node and
 *     reference query: row j is stored as s_j * e4m3(g_j / s_j), rounded to
 *     nearest even, with s_j = 2^(ceil(log2 max_e |g_je|) - 8) (1 for a zero
 *     row) in the tree's scale block; c_j uses the stored values.  Halves
 *     the bytes routing reads per node.  Needs kv_dtype ZHA_BF16.
 *   ZHA_G_FP4: the same variant read as OCP MXFP4: each row j of g in
 *     blocks of 32 consecutive elements of d, each block an E8M0 scale
 *     2^(floor(log2 max |block|) - 2) (2^-127 for a zero block) times FP4
 *     E2M1 values (round to nearest even, saturating at 6); c_j uses the
 *     stored values.  A quarter of the bf16 bytes plus one scale byte per 32
 *     elements.  Needs kv_dtype ZHA_BF16, head_dim 128 and
 *     ZHA_LEAF_WEIGHTS2 (levels >= 3 store MXFP4).
 */
enum zha_g_dtype { ZHA_G_KV = 0, ZHA_G_FP8 = 2, ZHA_G_FP4 = 4 };

/* Flags of zha_attend. */
enum zha_attend_flags {
  ZHA_SINK = 1,       /* token 0 is always attended (MTP "How does top-p routing pick tokens?") */
  ZHA_LAST_CHUNK = 2, /* tokens [C*floor((N-1)/C), N) are always attended (MTP widget step 5) */
  ZHA_ALL_KEYS = 4,   /* ignore the selection: dense attention over all N keys */
  ZHA_CAUSAL = 8      /* prefill block: query t of each head sits at position
                         N - T + t and sees keys [0, N - T + t] only; the current
                         chunk and the sink are taken relative to it (bf16) */
};

/*
 * Problem configuration.  Supported: head_dim in {64, 128}; n_ref in 1..16;
 * chunk a power of two in 1..256; levels in 1..ZHA_MAX_LEVELS with
 * chunk^levels <= 2^24; kv_dtype ZHA_F32 or ZHA_BF16 (g is stored in the same
 * type); q_per_kv * T <= 1024.  Anything else is ZHA_ERR_UNSUPPORTED.
 */
typedef struct zha_config {
  int32_t batch;           /* B */
  int32_t n_kv_heads;      /* H */
  int32_t q_per_kv;        /* G: query heads sharing one KV head (and its tree) */
  int32_t head_dim;        /* d */
  int32_t n_ref;           /* R: reference queries per KV head */
  int32_t chunk;           /* C: keys per level-1 node; children per upper node */
  int32_t levels;          /* Lv: level 1 = chunks of raw keys, level Lv = top */
  int32_t kv_dtype;        /* enum zha_dtype */
  int32_t leaf_form;       /* enum zha_leaf_form */
  int32_t g_dtype;         /* enum zha_g_dtype (0 = ZHA_G_KV) */
  int64_t capacity_tokens; /* largest N the tree buffer must hold */
} zha_config;

/*
 * Tree buffer layout (computed by zha_get_tree_layout).  Level l (index l-1)
 * holds node_cap[l-1] = ceil(node_cap[l-2] / C) nodes per cache, with
 * node_cap[0] = floor(capacity / C).  Per level, three blocks:
 *   g: [caches][node_cap][g_bytes / element size]: for level 1 in the
 *      weights forms, w as [R][C] fp32; for level 2 in ZHA_LEAF_WEIGHTS2,
 *      rho as [R][C] fp32; otherwise R x d mean keys in kv_dtype.
 *      Within one node the R x d mean
 *      keys are stored d-chunk-interleaved so that one 64-lane load yields a
 *      16 x 32 MFMA operand tile: element (j, e) with 16-byte piece
 *      k = e / E (E = elements per 16 bytes), sub-index e % E, lives at
 *      element offset ((k / 4) * 4 * R + (k % 4) * R + j) * E + e % E.
 *   L: [caches][node_cap][R] fp32, log mass L_j of the node.
 *   c: [caches][node_cap][R] fp32, plane offset c_j = L_j - r_j . g_j / sqrt(d)
 *      with the stored (rounded) g_j.
 * With g_dtype ZHA_G_FP8 the levels that store mean keys hold R x d E4M3
 * bytes per node: element (j, e) with MFMA step s = e / 32 and k-group
 * kg = (e % 32) / 8 lives at byte ((s / 2) * 4 * R + kg * R + j) * 16 +
 * (s % 2) * 8 + e % 8 (one 16-byte load yields two MFMA steps), and a fourth
 * block s: [caches][node_cap][R] fp32 holds the row scales (s_offset).
 * With ZHA_G_FP4 those levels hold R x d / 2 bytes per node: element (j, e)
 * with MFMA step s = e / 32 and k-group kg = (e % 32) / 8 is nibble e % 2
 * (low first) of byte (kg * R + j) * 16 + s * 4 + (e % 8) / 2 (one 16-byte
 * load yields the four steps of d = 128), and the scale block s:
 * [caches][node_cap][R][d / 32] holds the E8M0 block scales (byte b means
 * 2^(b - 127)).
 * Offsets are bytes from the tree base; every block is 256-byte aligned.
 */
typedef struct zha_tree_layout {
  int32_t levels;
  int32_t reserved;
  int64_t node_cap[ZHA_MAX_LEVELS];
  int64_t g_offset[ZHA_MAX_LEVELS];
  int64_t L_offset[ZHA_MAX_LEVELS];
  int64_t c_offset[ZHA_MAX_LEVELS];
  int64_t g_bytes[ZHA_MAX_LEVELS]; /* bytes of one node's g (or w) block, per level */
  int64_t total_bytes;  /* size of the caller's tree buffer */
  int64_t s_offset[ZHA_MAX_LEVELS]; /* fp8 row scales or fp4 block scales per level, or -1 */
  int64_t scratch_offset; /* fp32 children of up to 2 top nodes per cache, used by
                             zha_append to split its spans over more workgroups;
                             -1 when the geometry does not split */
  int64_t ref_offset;     /* ZHA_LEAF_WEIGHTS2: the reference queries the tree was
                             built with, [H][R][d] fp32 (zha_build and zha_append
                             store them; routing recomputes the level-1 and
                             level-2 log masses and weights from them and the
                             keys); else -1 */
} zha_tree_layout;

/*
 * Route output layout (computed by zha_get_route_layout) for n_queries =
 * B*H*G*T queries.  Per level l (index l-1):
 *   sel:   [n_queries][words[l-1]] uint32 bitsets, bit n%32 of word n/32 set
 *          iff node n is kept; starts at sel_offset[l-1] (in uint32 words).
 *   score: [n_queries][score_stride[l-1]] fp32 plane scores of the
 *          candidates (entries >= the level's node count are unused), -inf
 *          for nodes that were not candidates; starts at score_offset[l-1]
 *          (in floats); score_stride = node_cap rounded up to 4.
 *   stats: [n_queries] zha_select_stats; starts at stats_offset[l-1]
 *          (in records).
 * Optional logits (leaf-weights forms only): level-1 scoring computes
 * q . k_i / sqrt(d) for every key of every candidate chunk (in
 * ZHA_LEAF_WEIGHTS2 level-2 scoring does, for every key of every candidate
 * level-2 node, when it also forms the level-1 scores); zha_route can
 * keep them in a [caches][ceil(QC/16)][capacity/4][4][QW] fp32 buffer (4-key
 * quads, 4 keys, QW = min(QC rounded up to 4, 16) queries; QC = G*T queries
 * per cache; rows beyond QC unused) so that zha_attend reads 16 bytes per key
 * and query instead of the keys.
 * Scratch: zha_route accepts any ws_bytes >= workspace_min_bytes (per level
 * and query, the score tiles' candidate key ranges).  With ws_bytes >=
 * workspace_bytes it may also spread the selection of a level with few
 * queries and many candidates over several workgroups per query (same
 * result, bit for bit).
 */
typedef struct zha_route_layout {
  int32_t levels;
  int32_t reserved;
  int64_t n_queries;
  int64_t words[ZHA_MAX_LEVELS];
  int64_t sel_offset[ZHA_MAX_LEVELS];
  int64_t score_offset[ZHA_MAX_LEVELS];
  int64_t score_stride[ZHA_MAX_LEVELS];
  int64_t stats_offset[ZHA_MAX_LEVELS];
  int64_t sel_words_total;    /* uint32 words of the sel buffer */
  int64_t score_floats_total; /* floats of the score buffer */
  int64_t stats_total;        /* records of the stats buffer */
  int64_t workspace_bytes;    /* scratch that enables every select form (see below) */
  int64_t logits_floats;      /* floats of the optional logits buffer (weights forms), else 0 */
  int64_t workspace_min_bytes; /* smallest scratch zha_route accepts */
} zha_route_layout;

/*
 * Per (level, query) record of the top-p selection.  Masses are fixed-point
 * integers m = round(exp(s - max_score) * 2^shift), so sums are exact and
 * independent of summation order.  A candidate is kept iff its order key is
 * > cut_key, or == cut_key and its node id < cut_id (ties go to lower ids).
 */
typedef struct zha_select_stats {
  float max_score;     /* largest candidate score */
  int32_t n_cand;      /* candidates at this level */
  int32_t n_kept;      /* kept candidates */
  uint32_t cut_key;    /* order key of the last kept score */
  int32_t cut_id;      /* tie bound at cut_key (exclusive) */
  int32_t shift;       /* fixed-point shift of the masses */
  uint64_t mass_total; /* sum of candidate masses (M) */
  uint64_t mass_kept;  /* sum of kept masses */
} zha_select_stats;

/*
 * Optional per-kernel timing.  When a call receives a non-NULL zha_profile,
 * it records events[2k] on the stream right before its k-th kernel launch
 * and events[2k+1] right after it, for k < n_pairs, and reports in n_used
 * how many kernels it launched and in kernel[k] which kernel each pair
 * timed (enum zha_kernel_id * 16 + level, level 0 when not per-level).
 * The events are caller-created hipEvent_t handles; the library only
 * records them (no allocation, no synchronisation).
 */
#define ZHA_PROFILE_MAX 32
enum zha_kernel_id {
  ZHA_K_BUILD = 1,   /* tree build over whole top spans */
  ZHA_K_SCORE = 2,   /* plane scores of one level's candidates */
  ZHA_K_SELECT = 3,  /* top-p selection of one level */
  ZHA_K_ATTEND = 4,  /* split-K attention over the routed keys */
  ZHA_K_COMBINE = 5, /* merge of the split-K partials */
  ZHA_K_PROBE = 6    /* zha_stream_probe (level field = its mode) */
};
typedef struct zha_profile {
  void* events[2 * ZHA_PROFILE_MAX]; /* hipEvent_t */
  int32_t n_pairs;                    /* event pairs provided (<= ZHA_PROFILE_MAX) */
  int32_t n_used;                     /* (out) kernels launched by the call */
  int32_t kernel[ZHA_PROFILE_MAX];    /* (out) id * 16 + level of each timed kernel */
} zha_profile;

/* ---- information ------------------------------------------------------- */

int zha_version(void);
/* Static text for a status code. */
const char* zha_status_string(int status);
/* Thread-local description of the last failure of this thread ("" if none). */
const char* zha_last_error(void);

/* ---- sizes and layouts (host only, never touch the GPU) ---------------- */

/* Fills *out for cfg.  Returns ZHA_OK or a validation error. */
int zha_get_tree_layout(const zha_config* cfg, zha_tree_layout* out);
/* Fills *out for cfg and T queries per query head. */
int zha_get_route_layout(const zha_config* cfg, int32_t T, zha_route_layout* out);
/* Scratch bytes zha_attend / zha_dense_decode need for T queries per head. */
int64_t zha_attend_workspace_bytes(const zha_config* cfg, int32_t T);
/* Single-number forms of the layouts above (negative on a validation
 * error): the tree buffer (zha_get_tree_layout total_bytes), the route
 * scratch that enables every select form (zha_get_route_layout
 * workspace_bytes), and the dense decode's scratch (the attend scratch). */
int64_t zha_tree_bytes(const zha_config* cfg);
int64_t zha_route_workspace_bytes(const zha_config* cfg, int32_t T);
int64_t zha_dense_workspace_bytes(const zha_config* cfg, int32_t T);

/* ---- the hot path ------------------------------------------------------- */

/*
 * zha_build - build every tree level for the first n_tokens keys.
 * Defines (MTP "Building the tree"): keys are cut into contiguous chunks of
 * C; each chunk is summarised per reference query r_j by its log attention
 * mass L_j = logsumexp_i (r_j . k_i / sqrt(d)) and the tangent-plane slope
 * g_j = sum_i softmax_i(r_j . k_i / sqrt(d)) k_i; summaries are merged level
 * by level: L(P) = logsumexp_c L(c), g(P) = sum_c exp(L(c) - L(P)) g(c).
 * n_1 = floor(N / C) leaves (a trailing partial chunk is not a node);
 * n_l = ceil(n_{l-1} / C) (a partial upper node merges the children present).
 *   K        device, [B][H][capacity][d] kv_dtype addressed by
 *            k_strides = {batch, head, token} in elements; each token row
 *            is d contiguous elements, 16-byte aligned.
 *   ref      device, [H][R][d] fp32 reference queries.  With kv_dtype
 *            bf16 every value is rounded to bf16 (nearest even) before use:
 *            the tree is that of the bf16-rounded reference queries (the
 *            logits r . k run on bf16 matrix cores).
 *   tree     device, zha_get_tree_layout(cfg).total_bytes bytes; overwritten for
 *            the nodes that exist at n_tokens.
 * Errors: NULL pointers, n_tokens < 0 or > capacity, misalignment.
 */
int zha_build(const zha_config* cfg, const void* K, const int64_t k_strides[3], int64_t n_tokens,
              const float* ref, void* tree, zha_profile* prof, void* stream);

/*
 * zha_append - extend a tree built for n_old tokens to n_old + n_new.
 * The caller has already written K rows [n_old, n_old + n_new).  Only the
 * nodes whose key range meets the new tokens are rewritten (new leaves and
 * the right spine of ancestors); the result is bit-identical to zha_build
 * over n_old + n_new tokens.  MTP "Building the tree" defines the nodes;
 * growth in place follows from nodes being functions of their key range.
 * Errors: as zha_build, plus n_old < 0, n_new < 0, n_old + n_new > capacity.
 */
int zha_append(const zha_config* cfg, const void* K, const int64_t k_strides[3], int64_t n_old,
               int64_t n_new, const float* ref, void* tree, zha_profile* prof, void* stream);

/*
 * zha_route - top-down top-p routing of B*H*G*T decode queries.
 * Defines (MTP "Building the tree", "How does top-p routing pick tokens?",
 * widget "1 . How it works" steps 2-4): a query scores a node by the max
 * over its reference-query tangent planes,
 *   s(q, node) = max_j [ L_j + (q - r_j) . g_j / sqrt(d) ]
 *              = max_j [ c_j + q . g_j / sqrt(d) ];
 * all top-level nodes are candidates; at each level the estimated masses
 * exp(s) are renormalised over the query's candidates, the smallest set
 * holding fraction p is kept (order: score descending, node id ascending;
 * keep a candidate iff the mass ranked before it is < p * M; p >= 1 keeps
 * all), and the children of kept nodes become the next candidates, down to
 * level 1 (raw chunks).
 *   tree      device, built for n_tokens.
 *   Q         device, [B][H][G][T][d] kv_dtype with q_strides = {batch,
 *             kv head, query head, t} in elements; rows contiguous, 16-byte
 *             aligned.
 *   p         in (0, 1]; NaN or <= 0 is ZHA_ERR_ARG.
 *   K         device keys as zha_build (read by the weights-form levels'
 *             scoring; may be NULL, with k_strides, in the mean form).
 *   sel       device, zha_get_route_layout().sel_words_total uint32 (output).
 *   score     device, zha_get_route_layout().score_floats_total fp32 (output).
 *   stats     device, zha_get_route_layout().stats_total records (output).
 *   logits    device, zha_get_route_layout().logits_floats fp32 (optional
 *             output, NULL to skip; leaf-weights forms only).
 *   ws        device scratch of at least workspace_min_bytes (ws_bytes
 *             >= workspace_bytes enables the split selection).
 * Level-1 bits of sel are the routed chunk ids consumed by zha_attend.
 */
int zha_route(const zha_config* cfg, const void* tree, int64_t n_tokens, const void* Q,
              const int64_t q_strides[4], int32_t T, float p, const void* K,
              const int64_t k_strides[3], uint32_t* sel, float* score,
              zha_select_stats* stats, float* logits, void* ws, int64_t ws_bytes,
              zha_profile* prof, void* stream);

/*
 * Chunked prefill (causal).  A block of T consecutive positions
 * [N - T, N) of every sequence is processed at once: query t of a head sits
 * at position N - T + t and decodes against the tree of its own prefix of
 * N - T + t + 1 tokens (the pages' sub-quadratic claim is about this
 * regime, MTP TL;DR).  Complete nodes of that prefix tree are nodes of the
 * tree built over N tokens; the one node per level >= 2 that straddles the
 * query's position is partial and merges the children that exist (R11).
 * zha_build_spine stores those partial nodes for every prefix state of the
 * block; zha_route_prefill routes each query on its prefix tree; zha_attend
 * with ZHA_CAUSAL attends each query over its own keys.  bf16 keys only.
 */
/* Bytes of the spine buffer for blocks of up to T positions (-1 on bad cfg/T). */
int64_t zha_spine_bytes(const zha_config* cfg, int32_t T);

/*
 * zha_build_spine - the partial nodes of the prefix trees of a block.
 *   K, k_strides, ref   as zha_build; keys [0, n_tokens) are read.
 *   n_tokens, T         the block is positions [n_tokens - T, n_tokens).
 *   spine               device, zha_spine_bytes(cfg, T) bytes (output):
 *                       for each state k (complete chunks of a prefix) and
 *                       level >= 2 whose node holding chunk k-1 is partial,
 *                       that node (g in the tree's storage and layout, L, c,
 *                       scale).
 * Errors: as zha_build, plus T outside [1, n_tokens], kv_dtype not bf16.
 */
int zha_build_spine(const zha_config* cfg, const void* K, const int64_t k_strides[3], int64_t n_tokens,
                    int32_t T, const float* ref, void* spine, zha_profile* prof, void* stream);

/*
 * zha_route_prefill - zha_route for a prefill block: query t of each head
 * routes on the tree of its prefix of n_tokens - T + t + 1 tokens (complete
 * nodes from tree, built over n_tokens; the partial ones from spine, built
 * by zha_build_spine for the same n_tokens and T).  Score rows hold -inf
 * beyond each query's prefix; outputs, workspace and errors as zha_route.
 */
int zha_route_prefill(const zha_config* cfg, const void* tree, const void* spine, int64_t n_tokens,
                      const void* Q, const int64_t q_strides[4], int32_t T, float p, const void* K,
                      const int64_t k_strides[3], uint32_t* sel, float* score, zha_select_stats* stats,
                      float* logits, void* ws, int64_t ws_bytes, zha_profile* prof, void* stream);

/*
 * zha_route_levels - zha_route with a depth-aware schedule.
 * Defines (MTP widget "5 . Caveats": top-p must scale with depth, a fixed
 * per-level p shrinks the coverage of deeper trees; the pages' summary of
 * the method: the tree depth can grow iteratively): the same routing, with
 *   p_levels  host, cfg->levels floats; p_levels[l-1] is the fraction kept at
 *             level l, each in (0, 1] (>= 1 keeps all; NaN or <= 0 is
 *             ZHA_ERR_ARG);
 *   top_level the level routing starts from: all its nodes are candidates
 *             and the levels above it are neither read nor written (their
 *             blocks of sel, score and stats keep their contents); 0 means
 *             cfg->levels, otherwise 1..cfg->levels.
 * Every other argument, output and error is as zha_route, which equals
 * zha_route_levels with p at every level and top_level 0.
 */
int zha_route_levels(const zha_config* cfg, const void* tree, int64_t n_tokens, const void* Q,
                     const int64_t q_strides[4], int32_t T, const float* p_levels, int32_t top_level,
                     const void* K, const int64_t k_strides[3], uint32_t* sel, float* score,
                     zha_select_stats* stats, float* logits, void* ws, int64_t ws_bytes,
                     zha_profile* prof, void* stream);

/*
 * zha_attend - exact softmax attention over the routed keys.
 * Defines (MTP widget step 5; "How does top-p routing pick tokens?"):
 *   A = keys of the level-1 chunks whose bit is set in sel1
 *       U {0} (ZHA_SINK) U [C*floor((N-1)/C), N) (ZHA_LAST_CHUNK),
 *   o = sum_{i in A} softmax_i(q . k_i / sqrt(d)) v_i,  lse = logsumexp.
 * With ZHA_ALL_KEYS, A = all N keys (dense decode).
 *   Q         as zha_route.
 *   K, V      device, as zha_build (same kv_strides for both).
 *   sel1      device, [n_queries][sel1_words] uint32 chunk bitsets (the
 *             level-1 block of zha_route's sel, or any set); may be NULL
 *             with ZHA_ALL_KEYS.
 *   logits    device, optional (NULL = compute every logit from K): the
 *             logits zha_route wrote for the same Q, K and n_tokens with
 *             sel1 = its level-1 selection.  Quads holding a routed chunk
 *             read their logits there; other quads (forced keys only) use K.
 *   out       device, [n_queries][d] fp32 (output).
 *   lse       device, [n_queries] fp32 (output, may be NULL).
 *   ws        device scratch of zha_attend_workspace_bytes(cfg, T).
 *   prof      optional per-kernel timing (may be NULL), see zha_profile.
 * Errors: NULL pointers, n_tokens outside [1, capacity], sel1_words <
 * ceil(floor(n_tokens / C) / 32), workspace too small, misalignment.
 */
int zha_attend(const zha_config* cfg, const void* Q, const int64_t q_strides[4], int32_t T,
               const void* K, const void* V, const int64_t kv_strides[3], int64_t n_tokens,
               const uint32_t* sel1, int64_t sel1_words, const float* logits, uint32_t flags,
               float* out, float* lse, void* ws, int64_t ws_bytes, zha_profile* prof,
               void* stream);

/*
 * zha_attend_noalloc - zha_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, argument meanings, outputs and
 * errors as zha_attend, without ws / ws_bytes.  The split-K partials go to a
 * static device array of ZHA_NOALLOC_SCRATCH_BYTES bytes inside the library
 * (one per GPU, held from the first call on that GPU until the process
 * ends); the call allocates nothing.  It uses the array of the calling
 * thread's current device, so `stream` must belong to that device.  Every
 * partial is written before it is read, so no call depends on what an
 * earlier call left there; but all calls on one GPU share the one array, so
 * two calls whose executions overlap on a GPU (different streams, or
 * threads) race and their results are undefined.
 * Errors: as zha_attend, plus ZHA_ERR_CAPACITY when the configuration needs
 * more than ZHA_NOALLOC_SCRATCH_BYTES (zha_attend_workspace_bytes(cfg, T)),
 * and ZHA_ERR_ARG when `stream` belongs to another device.
 */
#define ZHA_NOALLOC_SCRATCH_BYTES (32ll << 20)
int zha_attend_noalloc(const zha_config* cfg, const void* Q, const int64_t q_strides[4], int32_t T,
                       const void* K, const void* V, const int64_t kv_strides[3], int64_t n_tokens,
                       const uint32_t* sel1, int64_t sel1_words, const float* logits, uint32_t flags,
                       float* out, float* lse, zha_profile* prof, void* stream);

/*
 * zha_dense_decode - dense flash-decode over all n_tokens keys, the
 * same-GPU baseline (MTP "How fast is ZHA?" compares against dense
 * attention).  Equivalent to zha_attend with ZHA_ALL_KEYS and no sel1.
 */
int zha_dense_decode(const zha_config* cfg, const void* Q, const int64_t q_strides[4], int32_t T,
                     const void* K, const void* V, const int64_t kv_strides[3], int64_t n_tokens,
                     float* out, float* lse, void* ws, int64_t ws_bytes, zha_profile* prof,
                     void* stream);

/* ---- measurement (not part of the decode path) ------------------------- */

/*
 * zha_stream_probe - one launch of a plain streaming kernel over n_bytes of
 * device memory, timed like any other call through prof: the achievable HBM
 * bandwidth of simple access patterns on the GPU (the ceiling against which
 * the decode kernels' roofline fractions are read) and, as ZHA_PROBE_COPY, a
 * copy of known size that calibrates the byte counters of a profiler.
 * Every mode reads each 16-byte piece of src[0, n_bytes) exactly once:
 *   ZHA_PROBE_READ / _NT   read only (plain / nontemporal loads), grid-stride
 *                          over 4,096 workgroups; dst receives at most one word
 *                          per workgroup (>= 16 KiB needed);
 *   ZHA_PROBE_READ_SLAB / _SLAB_NT  read only, one contiguous 512 KiB slab
 *                          per workgroup (dst as above);
 *   ZHA_PROBE_COPY / _NT   dst[0, n_bytes) = src (plain / nontemporal), one
 *                          contiguous 512 KiB slab per workgroup;
 *   ZHA_PROBE_MIX / _NT    slab by slab, every 16 KiB span of src folded
 *                          (xor of its four 4 KiB quarters) into the matching
 *                          4 KiB span of dst[0, n_bytes / 4): four bytes read
 *                          per byte
 *                          written (plain / nontemporal stores), the mix of
 *                          the scoring passes that read keys and write
 *                          logits;
 *   ZHA_PROBE_TILE_MIX     one 64 KiB tile of src per workgroup (256 rows of
 *                          256 bytes), each load instruction covering 16 rows
 *                          x 64 bytes (the matrix-core operand layout of the
 *                          key-reading passes), then one 16-byte piece per
 *                          256 bytes read written to dst[0, n_bytes / 16)
 *                          (nontemporal): the tile shape and 16:1
 *                          read/write mix of the fused level-2 pass.
 *   src, dst  device, 16-byte aligned, not overlapping; dst_bytes its size.
 *   n_bytes   a positive multiple of 64.
 * Errors: ZHA_ERR_ARG (mode, n_bytes), ZHA_ERR_NULL, ZHA_ERR_ALIGN,
 * ZHA_ERR_CAPACITY (dst_bytes too small), ZHA_ERR_HIP.
 */
enum zha_probe_mode {
  ZHA_PROBE_READ = 0,
  ZHA_PROBE_READ_NT = 1,
  ZHA_PROBE_COPY = 2,
  ZHA_PROBE_COPY_NT = 3,
  ZHA_PROBE_MIX = 4,
  ZHA_PROBE_MIX_NT = 5,
  ZHA_PROBE_READ_SLAB = 6,
  ZHA_PROBE_READ_SLAB_NT = 7,
  ZHA_PROBE_TILE_MIX = 8
};
int zha_stream_probe(int32_t mode, const void* src, void* dst, int64_t n_bytes, int64_t dst_bytes,
                     zha_profile* prof, void* stream);

/* ------------------------------------------------------------------------
 * zha_selected_chunks: the level-1 selection of zha_route as sorted lists of
 * chunk ids (MTP "How does top-p routing pick tokens?": a query attends the
 * raw chunks kept at the bottom level, plus the sink and its current chunk,
 * which zha_attend adds by flag and which are not listed here).
 *   sel1        device, n_queries x sel1_words uint32: bit c of query q's row
 *               (word c / 32, bit c % 32) set when chunk c is kept, as
 *               zha_route writes the level-1 rows (zha_route_layout
 *               sel_offset[0], words[0]); bits at or past n_chunks ignored.
 *   n_chunks    chunks the rows cover (floor(n_tokens / chunk)).
 *   chunk_ids   device, n_queries x cap int32 (output): query q's kept chunk
 *               ids in increasing order at chunk_ids[q * cap ...]; entries
 *               past its count (or past cap) are not written.
 *   chunk_count device, n_queries int32 (output): query q's number of kept
 *               chunks, which may exceed cap (only the first cap ids are
 *               then written).
 * One workgroup per query, stream-ordered, no host sync.
 * Errors: ZHA_ERR_NULL, ZHA_ERR_ALIGN (pointers not 4-byte aligned),
 * ZHA_ERR_ARG (n_queries < 1 or >= 2^31, n_chunks < 0 or >= 2^31, cap < 0),
 * ZHA_ERR_CAPACITY (sel1_words < ceil(n_chunks / 32)), ZHA_ERR_HIP.
 */
int zha_selected_chunks(const uint32_t* sel1, int64_t sel1_words, int64_t n_queries, int64_t n_chunks,
                        int32_t* chunk_ids, int32_t* chunk_count, int64_t cap, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H_ */
