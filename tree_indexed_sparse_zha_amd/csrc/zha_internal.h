// Internal launch interface between the C-ABI layer (zha_api.cpp) and the
// HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/zha.h"

namespace zha {

// Records the caller's timing events around each kernel launch (zha_profile).
struct Prof {
  zha_profile* p;
  hipStream_t s;
  void begin(int id, int level) {
    if (p && p->n_used < p->n_pairs) {
      (void)hipEventRecord(static_cast<hipEvent_t>(p->events[2 * p->n_used]), s);
      p->kernel[p->n_used] = id * 16 + level;
    }
  }
  void end() {
    if (!p) return;
    if (p->n_used < p->n_pairs) (void)hipEventRecord(static_cast<hipEvent_t>(p->events[2 * p->n_used + 1]), s);
    ++p->n_used;
  }
};

constexpr int kMaxLevels = 8;

// Tree geometry for one call.  Offsets are bytes from the tree base.
struct TreeGeom {
  int levels;
  int R;
  int D;
  int C;
  int esize;  // bytes per K/V/g element (2 = bf16, 4 = fp32)
  int H;
  int caches;
  int leaf_weights;  // level 1 stores softmax weights instead of mean keys
  int w2;            // level 2 too stores the weights of its C*C keys ([R][C*C] fp32)
  int64_t node_cap[kMaxLevels];
  int64_t g_off[kMaxLevels];
  int64_t L_off[kMaxLevels];
  int64_t c_off[kMaxLevels];
  int64_t s_off[kMaxLevels];  // fp8 row scales per level, or -1
  uint32_t g8;                // bit l-1: level l stores g as fp8 E4M3 with row scales
  uint32_t g4;                // bit l-1: level l stores g as MXFP4 (E2M1, E8M0 scale per 32 of d)
  int64_t span_len[kMaxLevels + 1];  // span_len[l] = C^l tokens covered by a level-l node
};

struct BuildArgs {
  const void* K;
  int64_t sb, sh, st;  // K strides in elements (batch, head, token)
  const float* ref;    // [H][R][D]
  char* tree;
  TreeGeom geo;
  int64_t n_tokens;    // tree is built for this many tokens
  int64_t first_span;  // first top span to rebuild
  int64_t n_spans;     // number of spans to rebuild
  int64_t span_tokens; // tokens per top span = C^levels
  float inv_sqrt_d;
  // prefill spine (nullptr: normal build).  With a spine the kernel writes
  // no tree node; after every chunk it completes it stores, for each
  // snapshot state k (complete chunks) in [spine_k0, spine_k0 + spine_states),
  // the partial node of every level >= 2 that holds chunk k-1.
  char* spine;
  int64_t spine_k0;
  int64_t spine_states;
  int64_t spine_rec;   // bytes per record: g block, then L, c, scale (R fp32 each)
  // split top spans (appends touching at most 2 spans): the sub-span pass
  // builds the top node's children (top_level = levels - 1) and also stores
  // them as fp32 (m, s, weighted sum) in top_scratch; the merge pass
  // (merge_top) folds them into the top node.
  int top_level;       // level of the launch's top node
  float* top_scratch;  // [caches][2 spans][C children][R][D + 2] fp32, or nullptr
  int64_t scratch_span0;
  int merge_top;
  int mf;  // matrix-core build (k_build_mf) for the tree; the spine keeps k_build_span
};

// Byte offset of the spine record of (cache, state k, level lvl >= 2).
__host__ __device__ inline int64_t spine_record(int64_t cache, int64_t k, int lvl, int64_t k0, int64_t states,
                                                int levels, int64_t rec) {
  return ((cache * states + (k - k0)) * (levels - 1) + (lvl - 2)) * rec;
}

struct ScoreArgs {
  const char* g;         // level base of g
  const float* c;        // level base of c
  const float* gscale;   // level base of the fp8 row scales or MXFP4 block scales, or nullptr (KV dtype)
  int gfmt;              // g storage of this level: 0 KV dtype, 1 fp8, 2 MXFP4
  int64_t node_cap;      // nodes per cache at this level
  int64_t n_nodes;       // valid nodes per cache at this level
  int R, C, D, H, G, T, QC;  // QC = G * T queries per cache
  const void* Q;
  int64_t qsb, qsh, qsg, qst;
  const uint32_t* sel_parent;  // parent level bitsets or nullptr (top level)
  int64_t parent_words;        // words per query row of sel_parent
  float* score;                // [n_queries][score_stride] for this level
  int64_t score_stride;
  uint32_t* keyrange;          // [n_queries][kr_slots][4]: max key, min key, candidate count, 0
  int64_t kr_slots;            // slots per query: one per score tile (plain stores), or 1 (atomics)
  float inv_sqrt_d;
  int leaf_weights;            // a weights-form level: g holds w [R][C] fp32, C keys per node
  int wkeys;                   // weights form: keys per node (C at level 1, C * C at level 2)
  int64_t n_keys;              // weights form: keys of the complete chunks (a trailing node may cover fewer)
  // level 2 holding its children's mass shares (chunk 4): g holds rho
  // [R][4] per node, and its plane sums are rho-weighted sums of the
  // children's level-1 sums, from the level-1 weights w1 [R][4] per chunk
  const float* w1;
  const float* c1;             // level-1 c (fused level-1 scores)
  int64_t node_cap1;           // level-1 nodes per cache
  const float* ref;            // the tree's reference queries [H][R][D] fp32 (fused level 2:
                               // its log masses, weights, shares and offsets are recomputed
                               // from the logits r . k)
  float* score1;               // fused: level-1 score rows the level-2 pass writes, or nullptr
  int64_t score1_stride;
  int fuse1;                   // level 1 after a fused level-2 pass: mask the rows, publish key ranges
  const void* K;               // keys (weights form only)
  int64_t ksb, ksh, kst;
  int64_t causal_n0;           // prefill: query t of a head sits at position causal_n0 + t; -1 = decode
  int64_t lvl_chunks;          // chunks under one node of this level (C^(l-1))
  const char* spine;           // prefill spine records (levels >= 2), or nullptr
  int64_t spine_k0, spine_states, spine_rec;
  int levels, level, top;      // tree depth, this level, routing start level
  int64_t kr_spine_slot;       // key-range slot of the spine score (prefill)
  int64_t n_queries;           // caches * QC
  float* logits;               // optional [caches][ceil(QC/16)][nquads][4][QW] (weights form)
  int64_t nquads;              // 4-key quads per cache in the logits buffer
  int QW;                      // queries per logits row: min(QC rounded up to 4, 16)
};

struct SelectArgs {
  const float* score;  // [n_queries][score_stride]
  int64_t score_stride;
  const uint32_t* keyrange;  // written by the score kernel of the same level
  int64_t kr_slots;          // slot stride per query
  int64_t kr_used;           // slots the score kernel wrote (its tile count, or 1)
  int64_t n_nodes;
  uint32_t* sel;       // [n_queries][words]
  int64_t words;
  void* stats;         // zha_select_stats[n_queries]
  float p;
  int keep_all;
  void* split;      // split-select workspace (select_split_bytes), or null
  int64_t split_S;  // workgroups per query in the split form (set at launch)
  // one-workgroup select: the parent level's bitsets (nullptr at the routing
  // start or when C < 4), whose dropped parents' children it need not read,
  // and how many cut-bin candidates it resolves in LDS (0: radix passes only)
  const uint32_t* sel_parent;
  int64_t parent_words;
  int C;
  int cut_cap;
  int parent_lds;  // parent-bit words of LDS the one-workgroup select is launched with (set at launch)
};

// Split select: per query a state record, and per (query, segment) a slot of
// 2048 histogram bins plus five words; used for at most kSelSplitQueries
// queries when at least two segments of kSelSplitNodes candidates each fit
// within kSelSplitBlocks workgroups.
constexpr int64_t kSelStateBytes = 128;
constexpr int64_t kSelSlotU64 = 2056;
constexpr int64_t kSelSplitBlocks = 2048;
constexpr int64_t kSelSplitNodes = 32768;
constexpr int64_t kSelSplitQueries = 64;
// workgroups per query of the split select for a level (1: no split)
inline int select_segments(int64_t n_queries, int64_t n_nodes) {
  if (n_queries <= 0 || n_queries > kSelSplitQueries) return 1;
  const int64_t s = std::min<int64_t>(kSelSplitBlocks / n_queries, n_nodes / kSelSplitNodes);
  return s >= 2 ? (int)std::min<int64_t>(s, 256) : 1;
}

inline int64_t select_split_bytes(int64_t n_queries, int64_t max_nodes) {
  const int S = select_segments(n_queries, max_nodes);
  if (S < 2) return 0;
  return n_queries * kSelStateBytes + n_queries * S * kSelSlotU64 * 8;
}

// Keys per tile of the weights-form score kernel launched for a level with
// wkeys keys per node: 8-key chunks (the light geometry, whose candidates
// come in 64-key runs) take one wave per 64 keys, so that a tile no query
// reaches ends at once; else 256 keys (also for many queries per cache, mq).
inline int leafw_tile(int wkeys, bool mq) { return wkeys == 8 && !mq ? 64 : 256; }

// key-range slots per query of one level's score kernel, for a level of
// `node_cap` nodes: one per tile for the bf16 kernels (plus one for the
// prefill spine score), 1 for the fp32 one (atomics)
inline int64_t route_kr_slots(int dtype, bool leaf_weights, int64_t node_cap, int wkeys) {
  if (leaf_weights) return (node_cap * wkeys + leafw_tile(wkeys, false) - 1) / leafw_tile(wkeys, false) + 1;
  if (dtype == 1) return (node_cap + 63) / 64 + 1;  // k_score_bf16: 64-node tiles
  return 1;                                         // k_score_generic
}

struct AttendArgs {
  const void* Q;
  int64_t qsb, qsh, qsg, qst;
  const void* K;
  const void* V;
  int64_t sb, sh, st;
  int H, G, T, QC, C, D;
  int64_t n_tokens;
  int64_t n_chunks;  // floor(n_tokens / C): chunks that can carry a selection bit
  const uint32_t* sel1;
  int64_t sel_words;
  uint32_t flags;
  int64_t tile_keys;  // keys per workgroup
  int64_t n_tiles;
  float* partial;     // [n_queries][n_tiles][D + 2]
  int64_t causal_n0;    // prefill: query t of a head sees keys [0, causal_n0 + t]; -1 = decode
  const float* logits;  // optional, see ScoreArgs
  int64_t nquads;
  int QW;
  float* out;
  float* lse;
  float inv_sqrt_d;
};

hipError_t launch_build(const BuildArgs& a, int dtype, Prof& prof);
hipError_t launch_route_init(uint32_t* keyrange, int64_t n, Prof& prof);
hipError_t launch_route_level(const ScoreArgs& sa, const SelectArgs& se, int dtype, int n_caches,
                              int level, Prof& prof);
hipError_t launch_attend(const AttendArgs& a, int dtype, int n_caches, Prof& prof);
// streaming probes (zha_stream_probe); arguments checked by the caller
hipError_t launch_probe(int mode, const void* src, void* dst, int64_t n_bytes, Prof& prof);
// level-1 bitsets -> sorted chunk id lists (zha_selected_chunks); arguments
// checked by the caller
hipError_t launch_selected_chunks(const uint32_t* sel1, int64_t words, int64_t n_queries, int64_t n_chunks,
                                  int32_t* ids, int32_t* count, int64_t cap, hipStream_t s);

}  // namespace zha
