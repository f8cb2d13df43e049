// Top-down top-p routing for ZHA on gfx950: per level, a score kernel and a
// select kernel.
//
// Defines (MTP = "Zyphra AI Introduces Zyphra Hierarchical Attention (ZHA):
// A Path to True Subquadratic Attention"; sections "Building the tree" and
// "How does top-p routing pick tokens?", widget "1 . How it works" steps
// 2-4):
//   s(q, node) = max_j [ c_j + q . g_j / sqrt(d) ]      (tangent-plane score)
//   masses exp(s) renormalised over the query's current candidates;
//   keep the smallest set holding fraction p (score desc, id asc; a candidate
//   is kept iff the mass ranked before it is < p * M); children of kept nodes
//   are the next candidates.
//
// Score design (bf16).  A workgroup takes a tile of 64 nodes of one cache and
// up to 16 queries of that cache (the G query heads of a KV head share its
// tree, so every node is read once for all of them).  A node's R x d mean
// keys are stored d-interleaved, so the 64 lanes load it with fully coalesced
// 16-byte loads straight into MFMA A operands; the queries are the B operand
// and v_mfma_f32_16x16x32_bf16 yields all R x 16 plane dot products.  Nodes
// whose parent no query kept are skipped without touching their bytes.
//
// Select design.  One workgroup per query, or, for levels with few queries
// and many candidates, a chain of kernels that spreads each query's row over
// several workgroups with the same arithmetic.  Masses are fixed-point integers
// round(exp(s - max) * 2^shift) so every sum is exact and order-independent
// (deterministic without float atomics).  The cut is found by a radix select
// on the order key of the score (digits of up to 11 bits below the
// candidates' common key prefix) over mass-weighted histograms in LDS, then
// ties at the cut key are resolved by node id.  The kept set is written as a
// bitset.
#include <algorithm>
#include <climits>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {
namespace {

struct SelStats {  // mirrors zha_select_stats
  float max_score;
  int32_t n_cand;
  int32_t n_kept;
  uint32_t cut_key;
  int32_t cut_id;
  int32_t shift;
  unsigned long long mass_total;
  unsigned long long mass_kept;
};
static_assert(sizeof(SelStats) == 40, "stats layout");

// Candidate key range and count of one score tile for one query, reduced
// over the wave's lanes and stored (plain store, no atomics) into the
// tile's slot; the select kernel reduces the slots.  Every tile writes its
// slot, also when it has no candidate (max 0, min ~0, count 0).
__device__ __forceinline__ void publish_range(uint32_t* slot, bool c, uint32_t k) {
  const unsigned long long bal = __ballot(c);
  uint32_t kmax = c ? k : 0u, kmin = c ? k : 0xffffffffu;
  if (bal != 0ull) {
    for (int o = 1; o < 64; o <<= 1) {
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    }
  }
  if ((threadIdx.x & 63) == 0)
    *reinterpret_cast<uint4*>(slot) = make_uint4(kmax, kmin, (uint32_t)__popcll(bal), 0u);
}

// Prefill (causal): query qi of a cache (qi = head * T + t) sits at position
// n0 + t and routes on the tree of its first n0 + t + 1 tokens, whose level-l
// nodes are the complete nodes below its horizon plus one partial node (the
// spine).  Complete nodes of this level visible to it (all: decode).
__device__ __forceinline__ int64_t causal_horizon(const ScoreArgs& A, int qi) {
  if (A.causal_n0 < 0) return INT64_MAX;
  const int64_t k = (A.causal_n0 + qi % A.T + 1) / A.C;  // complete chunks
  return k / A.lvl_chunks;
}

__global__ void k_route_init(uint32_t* kr, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    kr[4 * i + 0] = 0u;
    kr[4 * i + 1] = 0xffffffffu;
    kr[4 * i + 2] = 0u;
    kr[4 * i + 3] = 0u;
  }
}

// ---------------------------------------------------------------------------
// score, bf16, MFMA

// Candidate bits of 16 consecutive nodes nb0 .. nb0 + 15 of a level (bit u =
// node nb0 + u) for query qi of a cache: nodes that exist whose parent the
// query kept (every node at the top level), and, in prefill, only the
// query's complete nodes (below its horizon).  The nodes' 16 / C parents
// lie in one bitset word when C < 16.
__device__ __forceinline__ uint32_t node_bits16(const ScoreArgs& A, int cache, int qi, int64_t nb0) {
  const int64_t nvalid = A.n_nodes - nb0 < 16 ? (A.n_nodes - nb0 > 0 ? A.n_nodes - nb0 : 0) : 16;
  const uint32_t valid = (uint32_t)((1ull << nvalid) - 1ull);
  uint32_t mb = 0u;
  if (A.sel_parent) {
    const uint32_t* row = A.sel_parent + ((int64_t)cache * A.QC + qi) * A.parent_words;
    if (A.C >= 16) {
      // every node has one of at most two parents; test each node
      for (int u = 0; u < 16; ++u) {
        const int64_t par = (nb0 + u) / A.C;
        if ((row[par >> 5] >> (par & 31)) & 1u) mb |= 1u << u;
      }
    } else {
      const int64_t p0 = nb0 / A.C;
      const uint32_t word = row[p0 >> 5] >> (p0 & 31);
      for (int pi = 0; pi < 16 / A.C; ++pi)
        if ((word >> pi) & 1u) mb |= ((1u << A.C) - 1u) << (pi * A.C);
    }
    mb &= valid;
  } else {
    mb = valid;
  }
  const int64_t hz = causal_horizon(A, qi) - nb0;
  if (hz < 16) mb &= hz > 0 ? (1u << hz) - 1u : 0u;
  return mb;
}

// Candidate bits of the NCH (<= 64) nodes m0 .. m0 + NCH - 1 of a
// weights-form tile for query qi, as node_bits16, with CP children per
// parent (the nodes' NCH / CP parents lie in one bitset word).
template <int NCH, int CP>
__device__ __forceinline__ unsigned long long chunk_bits(const ScoreArgs& A, int cache, int qi, int64_t m0) {
  static_assert(NCH % CP == 0 && NCH / CP <= 32, "whole parents within one word");
  const int64_t nvalid = A.n_nodes - m0 < NCH ? A.n_nodes - m0 : NCH;
  const unsigned long long valid = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1ull);
  unsigned long long mb = 0ull;
  if (A.sel_parent) {
    const int64_t p0 = m0 / CP;
    const uint32_t word = A.sel_parent[((int64_t)cache * A.QC + qi) * A.parent_words + (p0 >> 5)] >> (p0 & 31);
#pragma unroll
    for (int pi = 0; pi < NCH / CP; ++pi)
      if ((word >> pi) & 1u) mb |= ((1ull << CP) - 1ull) << (pi * CP);
    mb &= valid;
  } else {
    mb = valid;
  }
  const int64_t hz = causal_horizon(A, qi) - m0;
  if (hz < 64) mb &= hz > 0 ? (1ull << hz) - 1ull : 0ull;
  return mb;
}

// GF = 1: g stored as fp8 E4M3 with a power-of-two scale per row; each
// 16-byte load holds two MFMA steps, converted to bf16 with the row's scale
// applied (exact: E4M3 values times powers of two are bf16 values).
// GF = 2: g stored as MXFP4; one 16-byte load holds the four steps of
// d = 128, each step's 8 E2M1 codes converted to bf16 times its block's
// E8M0 scale (exact as well).
template <int D, int GF>
__global__ __launch_bounds__(256) void k_score_bf16(ScoreArgs A) {
  constexpr bool G8 = GF == 1;  // fp8 rows with fp32 row scales
  constexpr bool G4 = GF == 2;  // MXFP4: E2M1 codes, an E8M0 scale per 32 values of d
  static_assert(!G4 || D == 128, "MXFP4 rows need d = 128");
  constexpr int NS = D / 32;  // MFMA k-steps of 32 bf16
  constexpr int TILE = 64;
  constexpr int NB = 4;       // nodes per batch
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qg0 = blockIdx.z * 16;
  const int nq = min(16, A.QC - qg0);
  const int64_t n0 = (int64_t)blockIdx.x * TILE;
  const int R = A.R;
  const int qn = lane & 15, kg = lane >> 4;
  __shared__ float sc[16][TILE + 1];

  bf16x8 bq[NS];
  {
    const int qi = qg0 + qn;
    if (qn < nq) {
      const int b = cache / A.H, h = cache % A.H, gq = qi / A.T, t = qi % A.T;
      const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb +
                         (int64_t)h * A.qsh + (int64_t)gq * A.qsg + (int64_t)t * A.qst;
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const int64_t gnode = G4 ? (int64_t)R * D / 2 : (int64_t)R * D * (G8 ? 1 : 2);
  const char* gcache = A.g + (int64_t)cache * A.node_cap * gnode;
  const float* ccache = A.c + (int64_t)cache * A.node_cap * R;
  const int jrow = lane & 15;

  // candidate bits of this wave's 16 nodes for query qn, then per-node "any query"
  const uint32_t mybits = qn < nq ? node_bits16(A, cache, qg0 + qn, n0 + wave * 16) : 0u;
  uint32_t anybits = mybits;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) anybits |= (uint32_t)__shfl_xor((int)anybits, o);

  // raw 16-byte loads per node and lane: NS pieces (bf16), NS / 2 (fp8) or 1
  // (MXFP4: the four steps of lane (row, k-group) in one piece)
  constexpr int NL = G4 ? 1 : (G8 ? NS / 2 : NS);
  const float* scache = G8 ? A.gscale + (int64_t)cache * A.node_cap * R : nullptr;
  // MXFP4: the 4 E8M0 bytes of a row (one per step), as one word
  const uint32_t* s4cache =
      G4 ? reinterpret_cast<const uint32_t*>(A.gscale) + (int64_t)cache * A.node_cap * R : nullptr;
  auto load_batch = [&](int u0, uint4 (*af)[NL], float (*cv)[4], float* sv) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int u = u0 + k;
      const int64_t m = n0 + wave * 16 + u;
      const bool live = (anybits >> u) & 1u;
      const char* gn = gcache + m * gnode;
#pragma unroll
      for (int s = 0; s < NL; ++s)
        // (each node's rows are read once per call: nontemporal)
        af[k][s] = live && jrow < R ? ld16_nt(gn + ((int64_t)(4 * s + kg) * R + jrow) * 16) : make_uint4(0, 0, 0, 0);
      if constexpr (G8) sv[k] = live && jrow < R ? scache[m * R + jrow] : 0.f;
      if constexpr (G4) sv[k] = __uint_as_float(live && jrow < R ? s4cache[m * R + jrow] : 0u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = 4 * kg + i;
        cv[k][i] = live && jj < R ? ccache[m * R + jj] : kNegInf;
      }
    }
  };

  uint4 af[NB][NL], an[NB][NL];
  float cv[NB][4], cn[NB][4];
  float sv[NB], sn[NB];
  load_batch(0, af, cv, sv);
  for (int u0 = 0; u0 < 16; u0 += NB) {
    if (u0 + NB < 16) load_batch(u0 + NB, an, cn, sn);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int u = u0 + k;
      float v = kNegInf;
      if ((anybits >> u) & 1u) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          uint4 op;
          if constexpr (G4) {
            // 8 E2M1 codes of step s (word s of the piece) -> bf16 x 2^(e8 - 127)
            const uint32_t w = s == 0 ? af[k][0].x : s == 1 ? af[k][0].y : s == 2 ? af[k][0].z : af[k][0].w;
            const uint32_t e8 = (__float_as_uint(sv[k]) >> (8 * s)) & 255u;
            const float sf = __uint_as_float(e8 == 0u ? 0x00400000u : e8 << 23);
            op.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 0));
            op.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 1));
            op.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 2));
            op.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sf, 3));
          } else if constexpr (G8) {
            // 8 E4M3 codes of step s (words x, y or z, w of the pair's slot) -> bf16 x scale
            const uint32_t w0 = (s & 1) ? af[k][s / 2].z : af[k][s / 2].x;
            const uint32_t w1 = (s & 1) ? af[k][s / 2].w : af[k][s / 2].y;
            op.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, sv[k], false));
            op.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, sv[k], true));
            op.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, sv[k], false));
            op.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, sv[k], true));
          } else {
            op = af[k][s];
          }
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(op), bq[s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, cv[k][i] + acc[i] * A.inv_sqrt_d);
        v = fmaxf(v, __shfl_xor(v, 16));
        v = fmaxf(v, __shfl_xor(v, 32));
      }
      if (lane < 16) sc[qn][wave * 16 + u] = ((mybits >> u) & 1u) ? v : kNegInf;
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
#pragma unroll
      for (int s = 0; s < NL; ++s) af[k][s] = an[k][s];
#pragma unroll
      for (int i = 0; i < 4; ++i) cv[k][i] = cn[k][i];
      sv[k] = sn[k];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nq * TILE; idx += 256) {
    const int q = idx / TILE, x = idx % TILE;
    const int64_t mm = n0 + x;
    if (mm < A.n_nodes) A.score[((int64_t)cache * A.QC + qg0 + q) * A.score_stride + mm] = sc[q][x];
  }
  // candidate key range and count of this tile, per query (integer atomics)
  for (int q = wave; q < nq; q += 4) {
    const float v = sc[q][lane];
    const bool c = n0 + lane < A.n_nodes && v > kNegInf;
    publish_range(A.keyrange + (((int64_t)cache * A.QC + qg0 + q) * A.kr_slots + blockIdx.x) * 4, c, order_key(v));
  }
}

// Levels >= 2 with few reference queries (R <= 8, bf16 g): the MFMA's 16 A
// rows are (node, plane) pairs, 16 / RP nodes of RP padded planes each, so
// one MFMA chain scores 16 / RP nodes instead of one node with R of its 16
// rows in use (R = 1, the lightweight geometry, fills every row).  Output
// row 4 kg + i of lane (query, kg) is node (4 kg + i) / RP, plane
// (4 kg + i) % RP; the max over a node's planes stays inside the lane for
// RP <= 4 and takes one shuffle for RP = 8.  Tiles, candidate bits, score
// rows and key-range slots as k_score_bf16.
template <int D, int RP>
__global__ __launch_bounds__(256) void k_score_smallr(ScoreArgs A) {
  constexpr int NS = D / 32;
  constexpr int TILE = 64;
  constexpr int NPM = 16 / RP;  // nodes per MFMA chain
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qg0 = blockIdx.z * 16;
  const int nq = min(16, A.QC - qg0);
  const int64_t n0 = (int64_t)blockIdx.x * TILE;
  const int R = A.R;
  const int qn = lane & 15, kg = lane >> 4;
  __shared__ float sc[16][TILE + 1];

  bf16x8 bq[NS];
  {
    const int qi = qg0 + qn;
    if (qn < nq) {
      const int b = cache / A.H, h = cache % A.H, gq = qi / A.T, t = qi % A.T;
      const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb +
                         (int64_t)h * A.qsh + (int64_t)gq * A.qsg + (int64_t)t * A.qst;
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const int64_t gnode = (int64_t)R * D * 2;
  const char* gcache = A.g + (int64_t)cache * A.node_cap * gnode;
  const float* ccache = A.c + (int64_t)cache * A.node_cap * R;

  // candidate bits of this wave's 16 nodes for query qn, then "any query"
  const int64_t nb0 = n0 + wave * 16;
  const uint32_t mybits = qn < nq ? node_bits16(A, cache, qg0 + qn, nb0) : 0u;
  uint32_t anybits = mybits;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) anybits |= (uint32_t)__shfl_xor((int)anybits, o);

  // A row of this lane: node mrow / RP of the chain, plane mrow % RP
  const int mrow = lane & 15, mnode = mrow / RP, mj = mrow % RP;
  uint4 af[RP][NS];
#pragma unroll
  for (int ch = 0; ch < RP; ++ch) {
    const int u = ch * NPM + mnode;
    const bool live = ((anybits >> u) & 1u) && mj < R;
    const char* gn = gcache + (nb0 + u) * gnode;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      af[ch][s] = live ? ld16(gn + ((int64_t)(4 * s + kg) * R + mj) * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int ch = 0; ch < RP; ++ch) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[ch][s]), bq[s], acc, 0, 0, 0);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * kg + i;
      const int u = ch * NPM + row / RP, j = row % RP;
      const bool ok = ((anybits >> u) & 1u) && j < R;
      v[i] = ok ? ccache[(nb0 + u) * R + j] + acc[i] * A.inv_sqrt_d : kNegInf;
    }
    // max over each node's planes; lane writes the nodes it then holds
    if constexpr (RP == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = ch * NPM + 4 * kg + i;
        if (qn < nq) sc[qn][wave * 16 + u] = ((mybits >> u) & 1u) ? v[i] : kNegInf;
      }
    } else if constexpr (RP == 2) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int u = ch * NPM + 2 * kg + h2;
        const float m2 = fmaxf(v[2 * h2], v[2 * h2 + 1]);
        if (qn < nq) sc[qn][wave * 16 + u] = ((mybits >> u) & 1u) ? m2 : kNegInf;
      }
    } else {
      float m4 = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
      if constexpr (RP == 8) m4 = fmaxf(m4, __shfl_xor(m4, 16));
      const int u = ch * NPM + (RP == 4 ? kg : kg / 2);
      if (qn < nq && (RP == 4 || (kg & 1) == 0)) sc[qn][wave * 16 + u] = ((mybits >> u) & 1u) ? m4 : kNegInf;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nq * TILE; idx += 256) {
    const int q = idx / TILE, x = idx % TILE;
    const int64_t mm = n0 + x;
    if (mm < A.n_nodes) A.score[((int64_t)cache * A.QC + qg0 + q) * A.score_stride + mm] = sc[q][x];
  }
  for (int q = wave; q < nq; q += 4) {
    const float v = sc[q][lane];
    const bool c = n0 + lane < A.n_nodes && v > kNegInf;
    publish_range(A.keyrange + (((int64_t)cache * A.QC + qg0 + q) * A.kr_slots + blockIdx.x) * 4, c, order_key(v));
  }
}

// ---------------------------------------------------------------------------
// score of the levels scored from their keys (bf16): level 1 of the weights
// forms (C in {4, 8, 16}), level 2 holding child shares (16-key nodes)
//
// s(q, chunk) = max_j [ c_j + sum_i w_ji (q . k_i) / sqrt(d) ]: the chunk's
// raw keys go through the MFMA (A = 16 keys, B = up to 16 queries) exactly
// as in attention; the MFMA leaves, in each lane, the logits of 4 keys for
// one query, and the lane folds them with the weights of all R planes of
// their chunk (staged once per tile in LDS and read as broadcasts) and takes
// the max itself, so no lane exchange is needed when C = 4.  A tile is KT
// keys (256, or 64 for 8-key chunks: one wave); each wave owns 4 groups of
// 16 keys and skips groups none of whose chunks is a candidate of any query,
// and a tile with no candidate at all ends after writing -inf; weights are
// staged only for candidate chunks.

// RT: R as a compile-time constant (0 = runtime).  Q4: at most 4 queries per
// cache; the MFMA then fills only 4 of its 16 query columns, so the logits
// go through LDS and the plane fold runs with lanes = (chunk, part, query),
// every lane busy.  C is the keys per node.  MODE 1: level 2 under chunk 4
// (16-key nodes, 4 children per parent) holding its children's mass shares
// rho_cj = exp(L_j(chunk c) - L_j(node)): the node's weight of key i in chunk
// c is rho_cj w_ji(chunk c), so its plane sum is sum_c rho_cj times the
// chunk's own sum over its keys, which the fold forms anyway.  MODE 2 (Q4):
// MODE 1, and the chunk sums also give every chunk's level-1 plane
// c_j(chunk) + sum_i w_ji s_i, written to the level-1 score rows, so level 1
// needs neither its keys nor its logits again.
template <int D, int C, int RT, bool Q4, int MODE = 0, int KT = 256>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_score_leafw(ScoreArgs A) {
  static_assert(MODE == 0 || C == 16, "child shares: 16-key nodes of 4 chunks");
  static_assert(MODE < 2 || Q4, "fused level-1 scores: at most 4 queries per cache");
  static_assert(KT == 256 || (KT == 64 && MODE == 0), "tiles of 256 keys, or of 64 (one wave)");
  constexpr int NT = KT;       // threads: one wave per 64 keys
  constexpr int NW = KT / 64;  // waves
  constexpr int CP = MODE ? 4 : C;   // children per parent
  constexpr int GW = MODE ? 4 : C;   // floats per plane of a node's g block (w, or rho)
  constexpr int NS = D / 32;
  constexpr int NCH = KT / C;   // chunks per tile (<= 64)
  constexpr int GPW = 4;        // groups of 16 keys per wave
  constexpr int PARTS = C / 4;  // 4-key lane parts per chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qg0 = blockIdx.z * 16;
  const int nq = min(16, A.QC - qg0);
  const int64_t k0 = (int64_t)blockIdx.x * KT;
  const int64_t m0 = k0 / C;
  const int R = A.R;
  const int qn = lane & 15, kg = lane >> 4;
  const int64_t n_keys = A.n_keys;  // keys of complete chunks
  // padded: the fold's lanes (chunk cx, part) read WROW cx + part, distinct
  // modulo 16 float4s (64 banks), and rl's floats 4 cx + part
  constexpr int WROW = 17 * PARTS;
  // w row order: plane-major in memory order (staged from 16-byte pieces
  // read as [j][part]); MODE 2 writes its own w (lanes (plane, part)) part-
  // major, [part][17 planes], so that 16 lanes of one part store to distinct
  // banks; the folds read either order conflict-free
  auto wix = [](int j, int part) { return MODE == 2 ? part * 17 + j : j * PARTS + part; };
  __shared__ float sc[16][NCH + 1];
  __shared__ float4 wl[NCH][WROW];  // w of chunk x, plane j, 4-key part at [x][wix(j, part)]
  __shared__ float cl[NCH][17];
  // Q4: [wave][quad of the wave][query] logits; rows padded to 5 float4s so
  // that the gather of a key's 4 queries (16 rows of a wave at once) reads
  // distinct banks
  __shared__ float4 zl[Q4 ? NW : 1][16][5];
  __shared__ unsigned long long mbl[16];    // candidate bits per query
  __shared__ float rl[MODE ? NCH : 1][WROW];     // MODE: rho of node x, plane j, chunk part
  __shared__ float c1l[MODE == 2 ? 4 * NCH : 1][17];  // MODE 2: c of the tile's chunks

  bf16x8 bq[NS];
  {
    const int qi = qg0 + qn;
    if (qn < nq) {
      const int b = cache / A.H, h = cache % A.H, gq = qi / A.T, t = qi % A.T;
      const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb +
                         (int64_t)h * A.qsh + (int64_t)gq * A.qsg + (int64_t)t * A.qst;
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const int b = cache / A.H, h = cache % A.H;
  // MODE 2: the tree's reference queries in bf16 (exact: they hold bf16
  // values) in LDS, read per group as a second B operand (column = plane
  // j = qn), so that the log masses, weights, shares and offsets of both
  // levels come from z_ji = r_j . k_i / sqrt(d) instead of memory
  // (loaded here, stored to LDS once the tile's key loads are issued)
  constexpr int RPC = D / 8;  // 16-byte bf16 pieces of a reference row
  __shared__ uint4 refs[MODE == 2 ? 16 : 1][RPC + 1];
  float4 rr4[MODE == 2 ? 2 : 1];
  if constexpr (MODE == 2) {
    const int j = tid / RPC, pc = tid % RPC;
    const bool ok = tid < 16 * RPC && j < R;
    const float4* rp = reinterpret_cast<const float4*>(A.ref + ((int64_t)h * R + (ok ? j : 0)) * D + pc * 8);
    rr4[0] = ok ? rp[0] : make_float4(0.f, 0.f, 0.f, 0.f);
    rr4[1] = ok ? rp[1] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const bf16_t* Kc = reinterpret_cast<const bf16_t*>(A.K) + (int64_t)b * A.ksb + (int64_t)h * A.ksh;
  const float* wcache = reinterpret_cast<const float*>(A.g) + (int64_t)cache * A.node_cap * R * GW;
  const float* ccache = A.c + (int64_t)cache * A.node_cap * R;

  // candidate bits of the tile's chunks for query qn (bit x = chunk m0 + x)
  const unsigned long long mybits = qn < nq ? chunk_bits<NCH, CP>(A, cache, qg0 + qn, m0) : 0ull;
  // chunks that are a candidate of some query (same value in every lane)
  unsigned long long anybits = mybits;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) anybits |= __shfl_xor(anybits, o);
  if (anybits == 0ull) {
    // no chunk of the tile is any query's candidate (same in every wave):
    // -inf scores and empty key ranges, nothing read
    for (int idx = tid; idx < nq * NCH; idx += NT) {
      const int q = idx / NCH, x = idx % NCH;
      if (m0 + x < A.n_nodes) A.score[((int64_t)cache * A.QC + qg0 + q) * A.score_stride + m0 + x] = kNegInf;
    }
    for (int q = wave; q < nq; q += NW)
      publish_range(A.keyrange + (((int64_t)cache * A.QC + qg0 + q) * A.kr_slots + blockIdx.x) * 4, false, 0u);
    return;
  }

  // All loads of the tile are issued together as buffer loads (masked rows
  // read zeros): w and c of the candidate chunks first, then the K rows of
  // this wave's live groups; only the w/c loads are waited for before the
  // LDS stores, the K loads stay in flight across the barrier.
  const int64_t n_valid = min((int64_t)NCH, A.n_nodes - m0);  // chunks of this tile (>= 1)
  const rsrc_t wr = make_rsrc(wcache + m0 * R * GW, (uint32_t)(n_valid * R * GW * 4));
  const rsrc_t cr = make_rsrc(ccache + m0 * R, (uint32_t)(n_valid * R * 4));
  const int64_t rows = min((int64_t)KT, n_keys - k0);  // keys of complete chunks in this tile
  const rsrc_t kr = make_rsrc(Kc + k0 * A.kst, (uint32_t)((rows - 1) * A.kst * 2 + D * 2));
  // MODE: the level-1 rows of the tile's chunks (w1, and c1 in MODE 2)
  const int64_t c0 = m0 * 4;                                    // first chunk of the tile
  const int64_t n1 = n_keys / 4;                                // chunks of level 1
  const int64_t n1v = MODE ? min((int64_t)KT / 4, n1 - c0) : 0;  // the tile's (>= 1)
  const rsrc_t w1r = make_rsrc(MODE ? A.w1 + ((int64_t)cache * A.node_cap1 + c0) * R * 4 : nullptr,
                               (uint32_t)(n1v * R * 16));
  constexpr int ITEMS = NCH * 16 / NT;
  static_assert(ITEMS * NT == NCH * 16, "whole (chunk, plane) items per thread");
  // w as 16-byte pieces in memory order, piece it -> (chunk x, plane j,
  // part pp): with R = 16 consecutive lanes read consecutive bytes (MODE:
  // part pp of node x is chunk 4x + pp, read from its own w1 row, and rho
  // of (node x, plane j, chunk pp) is one float in the same order)
  float4 wst[ITEMS * PARTS];
  float rst[MODE ? ITEMS * PARTS : 1];
  float cst[ITEMS];
  if constexpr (MODE != 2) {
#pragma unroll
  for (int r = 0; r < ITEMS * PARTS; ++r) {
    const int it = tid + NT * r;
    const int x = it / (16 * PARTS), j = (it / PARTS) % 16, pp = it % PARTS;
    const bool ok = ((anybits >> x) & 1ull) && j < R;
    uint4 v;
    if constexpr (MODE) {
      v = bld16(w1r, ok ? (uint32_t)(((4 * x + pp) * R + j) * 16) : kOffNone);
      rst[r] = bld4f(wr, ok ? (uint32_t)(((x * R + j) * 4 + pp) * 4) : kOffNone);
    } else {
      v = bld16(wr, ok ? (uint32_t)((x * R + j) * C * 4 + pp * 16) : kOffNone);
    }
    wst[r] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int it = tid + NT * r;
    const int x = it / 16, j = it % 16;
    const bool ok = ((anybits >> x) & 1ull) && j < R;
    cst[r] = bld4f(cr, ok ? (uint32_t)((x * R + j) * 4) : kOffNone);
  }
  }
  uint4 kf[GPW][NS];
  bool live[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * GPW + gi;
    const unsigned long long gmask = ((1ull << (16 / C)) - 1ull) << (g * 16 / C);
    live[gi] = (anybits & gmask) != 0ull;
    const uint32_t ko = live[gi] ? (uint32_t)((g * 16 + qn) * A.kst * 2) : kOffNone;
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[gi][s] = bld16<0>(kr, ko + (4 * s + kg) * 16);
  }
  if constexpr (MODE == 2) {
    if (tid < 16 * RPC) {
      const float rr[8] = {rr4[0].x, rr4[0].y, rr4[0].z, rr4[0].w, rr4[1].x, rr4[1].y, rr4[1].z, rr4[1].w};
      float dummy[8];
      refs[tid / RPC][tid % RPC] = pack(rr, dummy, bf16_t());
    }
  }
  if constexpr (MODE != 2) {
#pragma unroll
    for (int r = 0; r < ITEMS * PARTS; ++r) {
      const int it = tid + NT * r;
      wl[it / (16 * PARTS)][it % (16 * PARTS)] = wst[r];  // [x][j * PARTS + pp]
      if constexpr (MODE) rl[it / (16 * PARTS)][it % (16 * PARTS)] = rst[r];
    }
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
      const int it = tid + NT * r;
      cl[it / 16][it % 16] = cst[r];
    }
  }
  if (tid < 16) mbl[tid] = mybits;  // lanes 0..15: kg 0, query qn = tid
  __syncthreads();

  const int RR = RT > 0 ? RT : R;
  constexpr int UNR = RT <= 0 ? 1 : RT < 4 ? RT : 4;  // plane loop unroll
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * GPW + gi;
    const int x = (g * 16 + 4 * kg) / C;  // chunk (within the tile) of this lane's 4 keys
    const int part = kg % PARTS;
    if (!live[gi]) {
      if (!Q4 && part == 0) sc[qn][x] = kNegInf;
      continue;
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[gi][s]), bq[s], z, 0, 0, 0);
    float zz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) zz[i] = z[i] * A.inv_sqrt_d;
    const int64_t quad = (k0 + g * 16) / 4 + kg;
    if (!Q4 && A.logits && qn < nq && quad < A.nquads) {
      // keep the attention logits of these 4 keys for query qn (zha_attend
      // reads them): row [quad][key][query], queries innermost
      float* lp = A.logits + (((int64_t)cache * gridDim.z + blockIdx.z) * A.nquads + quad) * 4 * A.QW + qn;
#pragma unroll
      for (int i = 0; i < 4; ++i) st4_nt(lp + i * A.QW, zz[i]);
    }
    if constexpr (MODE == 2) {
      // lane (plane j = qn, chunk kg of node g): z of the chunk's 4 keys; the
      // chunk's log mass L(chunk) = LSE z (formed as the build forms it), its
      // weights w = exp(z - L(chunk)), offset c = L(chunk) - sum w z; the
      // node's log mass L(node) = LSE over its complete chunks of L(chunk)
      // (4 lanes), each chunk's share rho = exp(L(chunk) - L(node)), and the
      // node's offset L(node) - sum over its chunks of rho (L(chunk) - c(chunk)).
      // Nothing of the stored tree is read: both levels come from the keys
      // and the reference queries alone.
      f32x4 zr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        zr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[gi][s]), as_bf16x8(refs[qn][4 * s + kg]), zr, 0, 0, 0);
      const bool ok = qn < R && c0 + 4 * g + kg < n1;
      float zi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) zi[i] = zr[i] * A.inv_sqrt_d;
      const float m1 = fmaxf(fmaxf(zi[0], zi[1]), fmaxf(zi[2], zi[3]));
      float e[4], s1 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = __expf(zi[i] - m1);
        s1 += e[i];
      }
      const float L1 = m1 + __logf(s1);
      const float inv1 = 1.f / s1;
      float w[4], wz = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = ok ? e[i] * inv1 : 0.f;
        wz = fmaf(w[i], zi[i], wz);
      }
      float m2 = ok ? m1 : kNegInf;
      m2 = fmaxf(m2, __shfl_xor(m2, 16));
      m2 = fmaxf(m2, __shfl_xor(m2, 32));
      const float pl = ok ? s1 * __expf(m1 - m2) : 0.f;  // this chunk's mass relative to the node max
      float ps = pl + __shfl_xor(pl, 16);
      ps += __shfl_xor(ps, 32);
      const float L2 = m2 + __logf(ps);
      const float rho = ok ? pl / ps : 0.f;
      float t = rho * wz;
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      if (qn < R) {
        wl[g][wix(qn, kg)] = make_float4(w[0], w[1], w[2], w[3]);
        rl[g][qn * PARTS + kg] = rho;
        c1l[4 * g + kg][qn] = L1 - wz;
        if (kg == 0) cl[g][qn] = L2 - t;
      }
    }
    if constexpr (Q4) {
      if (qn < 4) zl[wave][gi * 4 + kg][qn] = make_float4(zz[0], zz[1], zz[2], zz[3]);
    } else {
      // fold the 4 logits with every plane of the chunk (rows of chunks that
      // are no candidate hold stale LDS data; their result is discarded below)
      float best = kNegInf;
#pragma unroll UNR
      for (int jj = 0; jj < RR; ++jj) {
        const float4 wv = wl[x][wix(jj, part)];
        float v = wv.x * zz[0] + wv.y * zz[1] + wv.z * zz[2] + wv.w * zz[3];
        if constexpr (MODE) v *= rl[x][jj * PARTS + part];  // the chunk's share of the node
#pragma unroll
        for (int o = 16; o < 16 * PARTS; o <<= 1) v += __shfl_xor(v, o);
        best = fmaxf(best, cl[x][jj] + v);
      }
      if (part == 0) sc[qn][x] = ((mybits >> x) & 1ull) ? best : kNegInf;
    }
  }
  if constexpr (Q4) {
    // lanes (query u, part, chunk cx) over the wave's 64 / C chunks; quads of
    // dead groups hold stale LDS data, discarded by the candidate bit
    wave_sync();
    if (A.logits) {
      // the wave's 16 quads as rows [quad][key][query]: lane (quad qq, key
      // kk) gathers the 4 queries' logits of its key and stores them as one
      // 16-byte piece, so the wave writes 1 KiB with one coalesced store
      // (quads of chunks that are no query's candidate are not written:
      // attention reads logits of kept chunks only)
      const int qq = lane >> 2, kk = lane & 3;
      const int xq = (wave * 64 + 4 * qq) / C;  // chunk of the quad within the tile
      const int64_t quad = (k0 + wave * 64) / 4 + qq;
      if (((anybits >> xq) & 1ull) && quad < A.nquads) {
        const float* zr = reinterpret_cast<const float*>(&zl[wave][qq][0]);
        st16_nt(A.logits + ((((int64_t)cache * gridDim.z + blockIdx.z) * A.nquads + quad) * 4 + kk) * 4, zr[kk], zr[4 + kk],
                zr[8 + kk], zr[12 + kk]);
      }
    }
    const int u = lane & 3, part = (lane >> 2) % PARTS, cx = lane / (4 * PARTS);
    const int x = wave * (64 / C) + cx;
    const float4 zv = zl[wave][cx * PARTS + part][u];
    float best = kNegInf, best1 = kNegInf;
#pragma unroll UNR
    for (int jj = 0; jj < RR; ++jj) {
      const float4 wv = wl[x][wix(jj, part)];
      float v = wv.x * zv.x + wv.y * zv.y + wv.z * zv.z + wv.w * zv.w;
      if constexpr (MODE == 2) best1 = fmaxf(best1, c1l[4 * x + part][jj] + v);  // chunk 4x + part's plane
      if constexpr (MODE) v *= rl[x][jj * PARTS + part];  // the chunk's share of the node
      if constexpr (PARTS == 4) {
        v = row_sum_stride4(v);  // lane = u + 4 part + 16 cx: the 4 parts of a row
      } else {
#pragma unroll
        for (int o = 4; o < 4 * PARTS; o <<= 1) v += __shfl_xor(v, o);
      }
      best = fmaxf(best, cl[x][jj] + v);
    }
    if (part == 0 && u < nq) sc[u][x] = ((mbl[u] >> x) & 1ull) ? best : kNegInf;
    if constexpr (MODE == 2) {
      // level-1 score of chunk 4(m0 + x) + part for query u, for every chunk
      // of a node some query has as candidate (the level-1 pass keeps those
      // whose parent is kept)
      const int64_t ch = 4 * (m0 + x) + part;
      if (u < nq && ((anybits >> x) & 1ull) && ch < n_keys / 4)
        A.score1[((int64_t)cache * A.QC + qg0 + u) * A.score1_stride + ch] = best1;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nq * NCH; idx += NT) {
    const int q = idx / NCH, x = idx % NCH;
    const int64_t mm = m0 + x;
    if (mm < A.n_nodes) A.score[((int64_t)cache * A.QC + qg0 + q) * A.score_stride + mm] = sc[q][x];
  }
  for (int q = wave; q < nq; q += NW) {
    const float v = lane < NCH ? sc[q][lane] : kNegInf;
    const bool c = lane < NCH && m0 + lane < A.n_nodes && v > kNegInf;
    publish_range(A.keyrange + (((int64_t)cache * A.QC + qg0 + q) * A.kr_slots + blockIdx.x) * 4, c, order_key(v));
  }
}

// Level-1 score for many queries per cache (QC > 16): a workgroup keeps its
// 256-key tile (K rows in registers, weights and offsets in LDS) and walks up
// to kMqBlocks query blocks of 16 over it, so the tile is read once per
// 16 kMqBlocks queries instead of once per 16.  Per block the arithmetic is
// the one of k_score_leafw (MFMA over the keys, fold in the MFMA layout).
constexpr int kMqBlocks = 16;
// below this many (tile, cache) pairs a level keeps one query block per
// workgroup: walking 16 blocks in one workgroup would leave the GPU idle
constexpr int64_t kMqMinTiles = 256;

template <int D, int C, int RT, int MODE = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_score_leafw_mq(ScoreArgs A) {
  static_assert(MODE == 0 || C == 16, "child shares: 16-key nodes of 4 chunks");
  constexpr int CP = MODE ? 4 : C;  // children per parent
  constexpr int NS = D / 32;
  constexpr int KT = 256;
  constexpr int NCH = KT / C;
  constexpr int GPW = 4;
  constexpr int PARTS = C / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qz0 = blockIdx.z * 16 * kMqBlocks;  // first query of the workgroup
  const int nqb = min(kMqBlocks, (A.QC - qz0 + 15) / 16);
  const int64_t k0 = (int64_t)blockIdx.x * KT;
  const int64_t m0 = k0 / C;
  const int R = A.R;
  const int qn = lane & 15, kg = lane >> 4;
  const int64_t n_keys = A.n_keys;
  constexpr int WROW = 16 * PARTS + 1;
  constexpr int GW = MODE ? 4 : C;  // floats per plane of a node's g block (w, or rho)
  __shared__ float sc[16][NCH + 1];
  __shared__ float4 wl[NCH][WROW];
  __shared__ float cl[NCH][17];
  __shared__ float rl[MODE ? NCH : 1][WROW];

  const int b = cache / A.H, h = cache % A.H;
  const bf16_t* Kc = reinterpret_cast<const bf16_t*>(A.K) + (int64_t)b * A.ksb + (int64_t)h * A.ksh;
  const float* wcache = reinterpret_cast<const float*>(A.g) + (int64_t)cache * A.node_cap * R * GW;
  const float* ccache = A.c + (int64_t)cache * A.node_cap * R;

  // candidate bits of the tile's chunks for query qg0 + qn
  auto block_bits = [&](int qg0) -> unsigned long long {
    return qn < min(16, A.QC - qg0) ? chunk_bits<NCH, CP>(A, cache, qg0 + qn, m0) : 0ull;
  };
  unsigned long long anybits = 0ull;
  for (int qb = 0; qb < nqb; ++qb) anybits |= block_bits(qz0 + 16 * qb);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) anybits |= __shfl_xor(anybits, o);

  const int64_t n_valid = min((int64_t)NCH, A.n_nodes - m0);
  const rsrc_t wr = make_rsrc(wcache + m0 * R * GW, (uint32_t)(n_valid * R * GW * 4));
  const rsrc_t cr = make_rsrc(ccache + m0 * R, (uint32_t)(n_valid * R * 4));
  const int64_t rows = min((int64_t)KT, n_keys - k0);
  const rsrc_t kr = make_rsrc(Kc + k0 * A.kst, (uint32_t)((rows - 1) * A.kst * 2 + D * 2));
  const int64_t c0 = m0 * 4;  // MODE: first level-1 chunk of the tile, and its chunks
  const int64_t n1v = MODE ? min((int64_t)KT / 4, n_keys / 4 - c0) : 0;
  const rsrc_t w1r = make_rsrc(MODE ? A.w1 + ((int64_t)cache * A.node_cap1 + c0) * R * 4 : nullptr,
                               (uint32_t)(n1v * R * 16));
  constexpr int ITEMS = NCH * 16 / 256;
  // w as 16-byte pieces in memory order, piece it -> (chunk x, plane j,
  // part pp): with R = 16 consecutive lanes read consecutive bytes (MODE:
  // chunk 4x + pp's own w1 row, and its share rho of node x)
  float4 wst[ITEMS * PARTS];
  float rst[MODE ? ITEMS * PARTS : 1];
  float cst[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS * PARTS; ++r) {
    const int it = tid + 256 * r;
    const int x = it / (16 * PARTS), j = (it / PARTS) % 16, pp = it % PARTS;
    const bool ok = ((anybits >> x) & 1ull) && j < R;
    uint4 v;
    if constexpr (MODE) {
      v = bld16(w1r, ok ? (uint32_t)(((4 * x + pp) * R + j) * 16) : kOffNone);
      rst[r] = bld4f(wr, ok ? (uint32_t)(((x * R + j) * 4 + pp) * 4) : kOffNone);
    } else {
      v = bld16(wr, ok ? (uint32_t)((x * R + j) * C * 4 + pp * 16) : kOffNone);
    }
    wst[r] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int it = tid + 256 * r;
    const int x = it / 16, j = it % 16;
    const bool ok = ((anybits >> x) & 1ull) && j < R;
    cst[r] = bld4f(cr, ok ? (uint32_t)((x * R + j) * 4) : kOffNone);
  }
  uint4 kf[GPW][NS];
  bool live[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = wave * GPW + gi;
    const unsigned long long gmask = ((1ull << (16 / C)) - 1ull) << (g * 16 / C);
    live[gi] = (anybits & gmask) != 0ull;
    const uint32_t ko = live[gi] ? (uint32_t)((g * 16 + qn) * A.kst * 2) : kOffNone;
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[gi][s] = bld16<0>(kr, ko + (4 * s + kg) * 16);
  }
#pragma unroll
  for (int r = 0; r < ITEMS * PARTS; ++r) {
    const int it = tid + 256 * r;
    wl[it / (16 * PARTS)][it % (16 * PARTS)] = wst[r];  // [x][j * PARTS + pp]
    if constexpr (MODE) rl[it / (16 * PARTS)][it % (16 * PARTS)] = rst[r];
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int it = tid + 256 * r;
    cl[it / 16][it % 16] = cst[r];
  }
  __syncthreads();

  const int RR = RT > 0 ? RT : R;
  constexpr int UNR = RT <= 0 ? 1 : RT < 4 ? RT : 4;
  const int QB = (A.QC + 15) / 16;  // 16-query blocks of the logits rows
  for (int qb = 0; qb < nqb; ++qb) {
    const int qg0 = qz0 + 16 * qb;
    const int nq = min(16, A.QC - qg0);
    const unsigned long long mybits = block_bits(qg0);
    bf16x8 bq[NS];
    {
      const int qi = qg0 + qn;
      if (qn < nq) {
        const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                           (int64_t)(qi / A.T) * A.qsg + (int64_t)(qi % A.T) * A.qst;
#pragma unroll
        for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
      }
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = wave * GPW + gi;
      const int x = (g * 16 + 4 * kg) / C;
      const int part = kg % PARTS;
      if (!live[gi]) {
        if (part == 0) sc[qn][x] = kNegInf;
        continue;
      }
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[gi][s]), bq[s], z, 0, 0, 0);
      float zz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[i] = z[i] * A.inv_sqrt_d;
      const int64_t quad = (k0 + g * 16) / 4 + kg;
      if (A.logits && qn < nq && quad < A.nquads) {
        float* lp = A.logits + (((int64_t)cache * QB + qg0 / 16) * A.nquads + quad) * 4 * A.QW + qn;
#pragma unroll
        for (int i = 0; i < 4; ++i) st4_nt(lp + i * A.QW, zz[i]);
      }
      float best = kNegInf;
#pragma unroll UNR
      for (int jj = 0; jj < RR; ++jj) {
        const float4 wv = wl[x][jj * PARTS + part];
        float v = wv.x * zz[0] + wv.y * zz[1] + wv.z * zz[2] + wv.w * zz[3];
        if constexpr (MODE) v *= rl[x][jj * PARTS + part];  // the chunk's share of the node
#pragma unroll
        for (int o = 16; o < 16 * PARTS; o <<= 1) v += __shfl_xor(v, o);
        best = fmaxf(best, cl[x][jj] + v);
      }
      if (part == 0) sc[qn][x] = ((mybits >> x) & 1ull) ? best : kNegInf;
    }
    __syncthreads();
    for (int idx = tid; idx < nq * NCH; idx += 256) {
      const int q = idx / NCH, x = idx % NCH;
      const int64_t mm = m0 + x;
      if (mm < A.n_nodes) A.score[((int64_t)cache * A.QC + qg0 + q) * A.score_stride + mm] = sc[q][x];
    }
    for (int q = wave; q < nq; q += 4) {
      const float v = lane < NCH ? sc[q][lane] : kNegInf;
      const bool c = lane < NCH && m0 + lane < A.n_nodes && v > kNegInf;
      publish_range(A.keyrange + (((int64_t)cache * A.QC + qg0 + q) * A.kr_slots + blockIdx.x) * 4, c, order_key(v));
    }
    __syncthreads();
  }
}

// Level 1 after a fused level-2 pass (chunk 4, at most 4 queries per cache):
// that pass wrote the plane score of every chunk of its candidates; a chunk
// is a candidate of a query iff the query kept its parent, so the others
// become -inf here, and every (query, workgroup) publishes the candidate key
// range of its kMaskTiles x 64 chunks for the select (one slot per
// workgroup).  Wave w of a workgroup is query w; a workgroup walks
// kMaskTiles consecutive tiles of 64 chunks.
constexpr int kMaskTiles = 16;
__global__ __launch_bounds__(256) void k_score_mask1(ScoreArgs A, int64_t n_tiles) {
  const int qi = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (qi >= A.QC) return;  // whole waves
  const int cache = blockIdx.y;
  const int64_t row = (int64_t)cache * A.QC + qi;
  const uint32_t* prow = A.sel_parent + row * A.parent_words;
  float* srow = A.score + row * A.score_stride;
  // every load first: the parent words of the lane's kMaskTiles chunks,
  // then the row entries of the kept parents' children (buffer loads; the
  // others are masked and move nothing), then the masking and key ranges
  const int64_t m0 = (int64_t)blockIdx.x * kMaskTiles * 64 + lane;
  uint32_t pw[kMaskTiles];
#pragma unroll
  for (int t = 0; t < kMaskTiles; ++t) {
    const int64_t m = m0 + 64 * t;
    pw[t] = m < A.n_nodes ? prow[(m / 4) >> 5] : 0u;
  }
  const int64_t mb = (int64_t)blockIdx.x * kMaskTiles * 64;  // first chunk of the workgroup
  const rsrc_t sr = make_rsrc(srow + mb, (uint32_t)(min((int64_t)kMaskTiles * 64, A.n_nodes - mb) * 4));
  float v[kMaskTiles];
#pragma unroll
  for (int t = 0; t < kMaskTiles; ++t) {
    const int64_t m = m0 + 64 * t;
    const bool kept = (pw[t] >> ((m / 4) & 31)) & 1u;
    const float x = bld4f<0>(sr, kept ? (uint32_t)((lane + 64 * t) * 4) : kOffNone);
    v[t] = kept ? x : kNegInf;
  }
  uint32_t kmax = 0u, kmin = 0xffffffffu, cnt = 0u;
#pragma unroll
  for (int t = 0; t < kMaskTiles; ++t) {
    const int64_t tile = (int64_t)blockIdx.x * kMaskTiles + t;
    if (tile >= n_tiles) break;  // uniform
    const int64_t m = m0 + 64 * t;
    const bool kept = (pw[t] >> ((m / 4) & 31)) & 1u;
    if (!kept && m < A.n_nodes) srow[m] = kNegInf;
    if (v[t] > kNegInf) {
      const uint32_t k = order_key(v[t]);
      kmax = max(kmax, k);
      kmin = min(kmin, k);
      ++cnt;
    }
  }
  for (int o = 1; o < 64; o <<= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    cnt += (uint32_t)__shfl_xor((int)cnt, o);
  }
  if (lane == 0)
    *reinterpret_cast<uint4*>(A.keyrange + (row * A.kr_slots + blockIdx.x) * 4) = make_uint4(kmax, kmin, cnt, 0u);
}

// Levels >= 2 for many queries per cache (QC > 16, bf16 g, R > 8): a
// workgroup takes 64 nodes (16 per wave, in batches of 4 held in registers)
// and walks up to kMqBlocks query blocks of 16 over each batch, so the nodes
// are read once per 16 kMqBlocks queries.  Scores go straight to the rows
// (lane kg writes node kg of the batch); each (query, tile) key-range slot is
// gathered with LDS atomics and written once.
template <int D>
__global__ __launch_bounds__(256) void k_score_bf16_mq(ScoreArgs A) {
  constexpr int NS = D / 32;
  constexpr int TILE = 64;
  constexpr int NB = 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qz0 = blockIdx.z * 16 * kMqBlocks;
  const int nqb = min(kMqBlocks, (A.QC - qz0 + 15) / 16);
  const int64_t n0 = (int64_t)blockIdx.x * TILE;
  const int64_t nb0 = n0 + wave * 16;
  const int R = A.R;
  const int qn = lane & 15, kg = lane >> 4;
  const int b = cache / A.H, h = cache % A.H;
  __shared__ uint32_t krl[kMqBlocks][16][3];  // per (block, query): max key, min key, count

  for (int i = tid; i < kMqBlocks * 16; i += 256) {
    krl[i / 16][i % 16][0] = 0u;
    krl[i / 16][i % 16][1] = 0xffffffffu;
    krl[i / 16][i % 16][2] = 0u;
  }
  const int64_t gnode = (int64_t)R * D * 2;
  const char* gcache = A.g + (int64_t)cache * A.node_cap * gnode;
  const float* ccache = A.c + (int64_t)cache * A.node_cap * R;

  // candidate bits of this wave's 16 nodes for query qg0 + qn
  auto block_bits = [&](int qg0) -> uint32_t {
    return qn < min(16, A.QC - qg0) ? node_bits16(A, cache, qg0 + qn, nb0) : 0u;
  };
  uint32_t anybits = 0u;
  for (int qb = 0; qb < nqb; ++qb) anybits |= block_bits(qz0 + 16 * qb);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) anybits |= (uint32_t)__shfl_xor((int)anybits, o);
  __syncthreads();  // krl initialised

  const int jrow = lane & 15;
  for (int u0 = 0; u0 < 16; u0 += NB) {
    uint4 af[NB][NS];
    float cv[NB][4];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int u = u0 + k;
      const int64_t m = nb0 + u;
      const bool live = (anybits >> u) & 1u;
      const char* gn = gcache + m * gnode;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        af[k][s] = live && jrow < R ? ld16(gn + ((int64_t)(4 * s + kg) * R + jrow) * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = 4 * kg + i;
        cv[k][i] = live && jj < R ? ccache[m * R + jj] : kNegInf;
      }
    }
    for (int qb = 0; qb < nqb; ++qb) {
      const int qg0 = qz0 + 16 * qb;
      const int nq = min(16, A.QC - qg0);
      const uint32_t mybits = block_bits(qg0);
      bf16x8 bq[NS];
      {
        const int qi = qg0 + qn;
        if (qn < nq) {
          const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                             (int64_t)(qi / A.T) * A.qsg + (int64_t)(qi % A.T) * A.qst;
#pragma unroll
          for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
        } else {
#pragma unroll
          for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
        }
      }
      float mine = kNegInf;  // this lane's node: u0 + kg
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int u = u0 + k;
        float v = kNegInf;
        if ((anybits >> u) & 1u) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[k][s]), bq[s], acc, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) v = fmaxf(v, cv[k][i] + acc[i] * A.inv_sqrt_d);
          v = fmaxf(v, __shfl_xor(v, 16));
          v = fmaxf(v, __shfl_xor(v, 32));
        }
        if (k == kg) mine = ((mybits >> u) & 1u) ? v : kNegInf;
      }
      const int64_t m = nb0 + u0 + kg;
      if (qn < nq && m < A.n_nodes) {
        A.score[((int64_t)cache * A.QC + qg0 + qn) * A.score_stride + m] = mine;
        if (mine > kNegInf) {
          const uint32_t key = order_key(mine);
          atomicMax(&krl[qb][qn][0], key);
          atomicMin(&krl[qb][qn][1], key);
          atomicAdd(&krl[qb][qn][2], 1u);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < nqb * 16; i += 256) {
    const int qb = i / 16, q = i % 16;
    const int qg0 = qz0 + 16 * qb;
    if (q < min(16, A.QC - qg0)) {
      uint32_t* slot = A.keyrange + (((int64_t)cache * A.QC + qg0 + q) * A.kr_slots + blockIdx.x) * 4;
      *reinterpret_cast<uint4*>(slot) = make_uint4(krl[qb][q][0], krl[qb][q][1], krl[qb][q][2], 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// prefill spine score (bf16 keys, levels >= 2): one wave per query scores the
// partial node of its own prefix tree at this level, from the spine record of
// its state, when the node is a candidate (top level, or its parent, the
// partial node one level up, was kept).  Lane (j, dg): reference query j,
// the 16-byte pieces dg, dg + 4, ... of d (the node layout of the tree).

template <int D, bool G8>
__global__ __launch_bounds__(256) void k_score_spine(ScoreArgs A) {
  constexpr int NS = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = (int64_t)blockIdx.x * 4 + wave;
  if (q >= A.n_queries) return;  // uniform per wave
  const int cache = (int)(q / A.QC), qi = (int)(q % A.QC);
  const int64_t k = (A.causal_n0 + qi % A.T + 1) / A.C;  // complete chunks of the prefix
  const int64_t sid = k / A.lvl_chunks;                   // the partial node's id
  uint32_t* slot = A.keyrange + (q * A.kr_slots + A.kr_spine_slot) * 4;
  bool cand = (k % A.lvl_chunks) != 0 && k >= A.spine_k0 && k < A.spine_k0 + A.spine_states;
  if (cand && A.level < A.top) {
    const int64_t par = sid / A.C;
    cand = (A.sel_parent[q * A.parent_words + (par >> 5)] >> (par & 31)) & 1u;
  }
  if (!cand) {
    if (lane == 0) *reinterpret_cast<uint4*>(slot) = make_uint4(0u, 0xffffffffu, 0u, 0u);
    return;
  }
  const int R = A.R, j = lane & 15, dg = lane >> 4;
  const char* rec = A.spine + spine_record(cache, k, A.level, A.spine_k0, A.spine_states, A.levels, A.spine_rec);
  const float* f = reinterpret_cast<const float*>(rec + (int64_t)R * D * (G8 ? 1 : 2));
  const int b = cache / A.H, h = cache % A.H;
  const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                     (int64_t)(qi / A.T) * A.qsg + (int64_t)(qi % A.T) * A.qst;
  float dot = 0.f;
  if (j < R) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float qv[8], gv[8];
      unpack(ld16(qp + (4 * s + dg) * 8), qv, bf16_t());
      if constexpr (G8) {
        const uint4 w = ld16(rec + ((int64_t)((s / 2) * 4 + dg) * R + j) * 16);
        const uint32_t w0 = (s & 1) ? w.z : w.x, w1 = (s & 1) ? w.w : w.y;
        const float sc = f[2 * R + j];
        gv[0] = __builtin_amdgcn_cvt_f32_fp8((int)w0, 0) * sc;
        gv[1] = __builtin_amdgcn_cvt_f32_fp8((int)w0, 1) * sc;
        gv[2] = __builtin_amdgcn_cvt_f32_fp8((int)w0, 2) * sc;
        gv[3] = __builtin_amdgcn_cvt_f32_fp8((int)w0, 3) * sc;
        gv[4] = __builtin_amdgcn_cvt_f32_fp8((int)w1, 0) * sc;
        gv[5] = __builtin_amdgcn_cvt_f32_fp8((int)w1, 1) * sc;
        gv[6] = __builtin_amdgcn_cvt_f32_fp8((int)w1, 2) * sc;
        gv[7] = __builtin_amdgcn_cvt_f32_fp8((int)w1, 3) * sc;
      } else {
        unpack(ld16(rec + ((int64_t)(4 * s + dg) / 4 * 4 * R + (int64_t)((4 * s + dg) % 4) * R + j) * 16), gv,
               bf16_t());
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += qv[e] * gv[e];
    }
  }
  dot += __shfl_xor(dot, 16);
  dot += __shfl_xor(dot, 32);
  float v = j < R ? f[R + j] + dot * A.inv_sqrt_d : kNegInf;
  v = wave_max_xor(v, 1, 16);
  if (lane == 0) {
    A.score[q * A.score_stride + sid] = v;
    *reinterpret_cast<uint4*>(slot) = make_uint4(order_key(v), order_key(v), 1u, 0u);
  }
}

// ---------------------------------------------------------------------------
// score, generic (fp32): one wave per node, lane (j, quarter of d)

template <typename T, int D>
__global__ __launch_bounds__(256) void k_score_generic(ScoreArgs A) {
  constexpr int E = Elem<T>::per16;
  constexpr int NS = D / E / 4;
  constexpr int NV = NS * E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, dg = lane >> 4;
  const int cache = blockIdx.y;
  const int64_t m = (int64_t)blockIdx.x * 4 + wave;
  if (m >= A.n_nodes) return;
  const int R = A.R;
  const int64_t gnode = (int64_t)R * D * Elem<T>::size;
  const char* gn = A.g + ((int64_t)cache * A.node_cap + m) * gnode;
  float gv[NV];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint4 v = j < R ? ld16(gn + ((int64_t)(4 * s + dg) * R + j) * 16) : make_uint4(0, 0, 0, 0);
    unpack(v, &gv[s * E], T());
  }
  const float cj = j < R ? A.c[((int64_t)cache * A.node_cap + m) * R + j] : 0.f;
  const int b = cache / A.H, h = cache % A.H;
  for (int qi = 0; qi < A.QC; ++qi) {
    const int64_t qg = (int64_t)cache * A.QC + qi;
    bool cand = true;
    if (A.sel_parent) {
      const int64_t par = m / A.C;
      cand = (A.sel_parent[qg * A.parent_words + (par >> 5)] >> (par & 31)) & 1u;
    }
    float v = kNegInf;
    if (cand) {
      const int gq = qi / A.T, t = qi % A.T;
      const T* qp = reinterpret_cast<const T*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                    (int64_t)gq * A.qsg + (int64_t)t * A.qst;
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float qv[E];
        unpack(ld16(qp + (4 * s + dg) * E), qv, T());
#pragma unroll
        for (int e = 0; e < E; ++e) part += gv[s * E + e] * qv[e];
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      v = j < R ? cj + part * A.inv_sqrt_d : kNegInf;
      v = wave_max_xor(v, 1, 16);
    }
    if (lane == 0) {
      A.score[qg * A.score_stride + m] = v;
      if (v > kNegInf) {
        uint32_t* kr = A.keyrange + qg * A.kr_slots * 4;
        atomicMax(&kr[0], order_key(v));
        atomicMin(&kr[1], order_key(v));
        atomicAdd(&kr[2], 1u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// select

constexpr int kSelThreads = 1024;

__device__ __forceinline__ unsigned long long fixed_mass(float s, float mx, double scale) {
  return (unsigned long long)llrint((double)expf(s - mx) * scale);
}

// Block-wide sum of a 64-bit value (blocks of kSelThreads): within each
// wave by shuffles, then over the waves' totals in LDS (two barriers; the
// integer sum is exact in any order).
__device__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* red) {
  const int tid = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  unsigned long long r = 0ull;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) r += red[w];
  __syncthreads();  // red is free again
  return r;
}

// Finds the bin b (scanning from the highest bin down) whose mass interval
// (above, above + hist[b]] contains P, where `above` starts at *A_io and
// accumulates the bins above b.  Returns b and updates *A_io to the mass
// strictly above bin b.  nbins is a power of two.
__device__ int find_bin(const unsigned long long* hist, int nbins, unsigned long long P,
                        unsigned long long* A_io, unsigned long long* red, int* sh_bin,
                        unsigned long long* sh_above) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = nbins >= kSelThreads ? nbins / kSelThreads : 1;
  const int b0 = tid * per;
  const int nb = b0 < nbins ? per : 0;
  unsigned long long mine = 0;
  for (int i = 0; i < nb; ++i) mine += hist[b0 + i];
  // inclusive suffix sum over the threads' sums: within the wave by
  // shuffles, then the totals of the higher waves from LDS
  unsigned long long suf = mine;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long t = __shfl_down(suf, o);
    if (lane + o < 64) suf += t;
  }
  if (lane == 0) red[wv] = suf;
  if (tid == 0) *sh_bin = -1;
  __syncthreads();
  unsigned long long higher = 0ull;
  for (int w = wv + 1; w < kSelThreads / 64; ++w) higher += red[w];
  unsigned long long cum = *A_io + higher + (suf - mine);  // mass of the bins above this thread's range
  for (int i = nb - 1; i >= 0; --i) {
    const unsigned long long h = hist[b0 + i];
    if (cum < P && P <= cum + h) {
      *sh_bin = b0 + i;
      *sh_above = cum;
    }
    cum += h;
  }
  __syncthreads();
  const int b = *sh_bin;
  if (b >= 0) *A_io = *sh_above;
  __syncthreads();
  return b;
}

// Radix select on the order key.  Candidate keys share their bits above the
// highest bit where the largest and smallest key differ, so the digits
// (11 bits at most, from the top down) start below that common prefix: every
// histogram then spreads over the candidates' actual range instead of piling
// into the few bins a narrow score range occupies.  The steps below serve
// both the one-workgroup-per-query kernel and the split form, where S
// workgroups share a query's row.

// Candidate key range and count of query q, from the score tiles' slots.
__device__ void reduce_slots(const SelectArgs& A, int64_t q, uint32_t* kmax_o, uint32_t* kmin_o,
                             unsigned long long* n_o) {
  const int tid = threadIdx.x;
  uint32_t kmax = 0u, kmin = 0xffffffffu;
  unsigned long long ncand = 0ull;
  const uint4* kr = reinterpret_cast<const uint4*>(A.keyrange) + q * A.kr_slots;
  for (int64_t i = tid; i < A.kr_used; i += kSelThreads) {
    const uint4 v = kr[i];
    kmax = max(kmax, v.x);
    kmin = min(kmin, v.y);
    ncand += v.z;
  }
  for (int o = 1; o < 64; o <<= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    ncand += __shfl_xor(ncand, o);
  }
  __shared__ uint32_t rmax[kSelThreads / 64], rmin[kSelThreads / 64];
  __shared__ unsigned long long rcnt[kSelThreads / 64];
  if ((tid & 63) == 0) {
    rmax[tid >> 6] = kmax;
    rmin[tid >> 6] = kmin;
    rcnt[tid >> 6] = ncand;
  }
  __syncthreads();
  kmax = 0u;
  kmin = 0xffffffffu;
  ncand = 0ull;
  for (int w = 0; w < kSelThreads / 64; ++w) {
    kmax = max(kmax, rmax[w]);
    kmin = min(kmin, rmin[w]);
    ncand += rcnt[w];
  }
  __syncthreads();
  *kmax_o = kmax;
  *kmin_o = kmin;
  *n_o = ncand;
}

// Fixed-point setting of a row of n candidates (masses below 2^62 / n, so
// the total fits in 63 bits) and the start of the digit passes.
struct SelSetup {
  double scale;
  float mx;
  int shift;
  uint32_t want;  // key bits above the first digit
  int lo;         // the first digit ends at bit lo
};
__device__ SelSetup sel_setup(uint32_t kmax, uint32_t kmin, int64_t n) {
  SelSetup s;
  s.mx = key_to_float(kmax);
  int lg = 0;
  while ((1ll << lg) < n) ++lg;
  s.shift = 62 - lg;
  s.scale = ldexp(1.0, s.shift);
  const int hb = kmax == kmin ? 0 : 32 - __clz(kmax ^ kmin);  // low bits that differ
  s.want = hb >= 32 ? 0u : (kmax >> hb);
  s.lo = hb;
  return s;
}

// Visits every candidate score of float4 range [b0, b1) of a row (index,
// score, key): float4 loads, two in flight per thread.
template <typename F>
__device__ __forceinline__ void visit_row(const float4* row4, int64_t n, int64_t b0, int64_t b1, F&& fn) {
  for (int64_t b = b0 + threadIdx.x; b < b1; b += 2 * kSelThreads) {
    const float4 v0 = row4[b];
    const float4 v1 = b + kSelThreads < b1 ? row4[b + kSelThreads] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
    const float a[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int64_t i = (c < 4 ? b : b + kSelThreads) * 4 + (c & 3);
      if (i < n && a[c] > kNegInf) fn(i, a[c], order_key(a[c]));
    }
  }
}

// One digit pass over float4 range [b0, b1): adds into the LDS histogram
// `hist` the mass of each candidate whose key bits [top, 32) equal `want`,
// binned by its bits [lo, lo + w); on the first pass returns this thread's
// share of the total mass of every candidate.
__device__ unsigned long long digit_pass(const float4* row4, int64_t n, int64_t b0, int64_t b1, bool first,
                                         int top, int lo, int w, uint32_t want, float mx, double scale,
                                         unsigned long long* hist) {
  unsigned long long part = 0;
  const uint32_t mask = (uint32_t)((1 << w) - 1);
  visit_row(row4, n, b0, b1, [&](int64_t, float s, uint32_t k) {
    const bool match = top >= 32 || (k >> top) == want;
    if (!first && !match) return;
    const unsigned long long mm = fixed_mass(s, mx, scale);
    if (first) part += mm;
    if (match && w > 0) atomicAdd(&hist[(k >> lo) & mask], mm);
  });
  return part;
}

// With the cut key tau found (mass `above` strictly above it, h_tau at it):
// ties at tau all carry the same mass; returns how many of them are kept
// (the smallest ids) when only some are needed to reach P, else 0 (all
// kept).
__device__ __forceinline__ unsigned long long ties_needed(uint32_t tau, unsigned long long P,
                                                          unsigned long long above, unsigned long long h_tau,
                                                          float mx, double scale) {
  const unsigned long long m_tau = fixed_mass(key_to_float(tau), mx, scale);
  const unsigned long long n_tau = m_tau ? h_tau / m_tau : 0ull;
  const unsigned long long k_tie = m_tau ? (P - above + m_tau - 1ull) / m_tau : n_tau;
  return k_tie < n_tau ? k_tie : 0ull;
}

// Is candidate i of the row a tie at key tau?
__device__ __forceinline__ bool is_tie(const float* row, int64_t i, int64_t i1, uint32_t tau) {
  if (i >= i1) return false;
  const float s = row[i];
  return s > kNegInf && order_key(s) == tau;
}

// Ties at tau in [i0, i1) of a row, counted by the workgroup.
__device__ unsigned long long count_ties(const float* row, int64_t i0, int64_t i1, uint32_t tau,
                                         unsigned long long* red) {
  unsigned long long c = 0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += kSelThreads) c += is_tie(row, i, i1, tau) ? 1ull : 0ull;
  return block_sum_u64(c, red);
}

// One past the id of the need-th tie at tau (need >= 1) in [i0, i1), or
// INT_MAX when the range holds fewer.  The range is walked in steps of 8
// consecutive candidates per thread; the step that reaches `need` is
// resolved with a workgroup prefix sum of the threads' tie counts.
__device__ int tie_find(const float* row, int64_t i0, int64_t i1, uint32_t tau, unsigned long long need) {
  constexpr int PER = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int sh_cut;
  __shared__ uint32_t wsum[kSelThreads / 64];
  if (tid == 0) sh_cut = INT_MAX;
  __syncthreads();
  for (int64_t base = i0; base < i1; base += (int64_t)kSelThreads * PER) {
    const int64_t a = base + (int64_t)tid * PER;
    uint32_t bits = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) bits |= is_tie(row, a + e, i1, tau) ? 1u << e : 0u;
    const uint32_t c = __popc(bits);
    uint32_t x = c;  // inclusive prefix over the wave
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint64_t before = x - c, total = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      const uint32_t v = wsum[w];
      if (w < wave) before += v;
      total += v;
    }
    if (total >= need) {
      if (before < need && need <= before + c) {
        uint32_t left = (uint32_t)(need - before);  // the left-th set bit of this thread's mask
        for (int e = 0; e < PER; ++e)
          if ((bits >> e) & 1u) {
            if (--left == 0u) {
              sh_cut = (int)(a + e + 1);
              break;
            }
          }
      }
      __syncthreads();
      break;
    }
    need -= total;
    __syncthreads();  // wsum is rewritten by the next step
  }
  const int cut = sh_cut;
  __syncthreads();
  return cut;
}

// Bitset words [w0, w1) of the kept candidates (key above tau, or at tau
// with id below cut_id): one word (8 float4 loads) per thread step; adds this
// thread's kept count.  (The kept mass follows from the cut itself, see
// kept_mass.)
__device__ void write_bits(const float4* row4, int64_t n, int64_t w0, int64_t w1, uint32_t tau, int cut_id,
                           uint32_t* srow, unsigned long long* kept) {
  const int64_t n4 = (n + 3) / 4;
  for (int64_t w = w0 + threadIdx.x; w < w1; w += kSelThreads) {
    uint32_t bits = 0u;
    float4 v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int64_t b4 = w * 8 + c;
      v[c] = b4 < n4 ? row4[b4] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float a[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bb = c * 4 + e;
        const int64_t i = w * 32 + bb;
        const float s = a[e];
        if (i < n && s > kNegInf) {
          const uint32_t k = order_key(s);
          if (k > tau || (k == tau && i < (int64_t)cut_id)) bits |= 1u << bb;
        }
      }
    }
    srow[w] = bits;
    *kept += __popc(bits);
  }
}

// Kept fixed-point mass of a selection with cut key tau: every candidate
// when all are kept (M), else the mass strictly above tau plus the kept ties
// at tau, which all carry one mass (need of them, or all h_tau of them when
// need is 0).  Integer sums: equal to adding the kept candidates' masses.
__device__ __forceinline__ unsigned long long kept_mass(bool keep_all, unsigned long long M,
                                                         unsigned long long above, unsigned long long h_tau,
                                                         unsigned long long need, uint32_t tau, float mx,
                                                         double scale) {
  if (keep_all) return M;
  return above + (need ? need * fixed_mass(key_to_float(tau), mx, scale) : h_tau);
}

__device__ __forceinline__ unsigned long long p_target(float p, unsigned long long M) {
  unsigned long long P = (unsigned long long)ceil((double)p * (double)M);
  if (P < 1ull) P = 1ull;
  if (P > M) P = M;
  return P;
}

// ---- the one-workgroup select: two reads of the row in the common case
//
// Pass 1 sums the fixed-point masses (M) and histograms them over a linear
// grid of scores, 2048 bins over [lo, max]: lo is the lowest candidate
// score, or max - span when that is higher, span wide enough that every
// score below it has a fixed-point mass that rounds to 0 (all of them land
// in bin 0).  The bin of a score is monotone in the score, so the cut lies
// in the one bin b whose mass interval holds P, exactly as in a radix digit.
// Pass 2 writes the bitset: every candidate in a bin above b is kept, every
// one below dropped, and the candidates of bin b (key, id, mass) are
// compacted into LDS.  Among those few the keep rule is applied exactly: a
// candidate is kept iff the mass of the bins above b plus the mass of the
// bin-b candidates ranked before it (score descending, id ascending) is
// below P; their bits are or-ed in.  This is the same cut the radix select
// reaches (the fixed-point rule has one answer).  When bin b holds more
// candidates than the LDS list takes, the radix passes run instead.
//
// Both passes read the row as consecutive float4s per thread (four in
// flight).  At levels below the routing start with C >= 4 the parent
// level's bits of the query are first copied to LDS (when they fit), and
// float4s whose parent was not kept are not read: their entries are -inf
// (not candidates).

constexpr int kLinBins = 2048;
constexpr int kCutCap = 1536;
// parent bits held in LDS (dynamic, sized per launch to the words a row
// reaches): levels of up to 163,840 parents (with the static arrays, at
// most 61 KiB of the 160 KiB a workgroup may take)
constexpr int kParentWords = 5120;
constexpr int kSelUnroll = 4;

__device__ __forceinline__ int lin_bin(float s, float lo, float inv_w) {
  const float x = (s - lo) * inv_w;
  return x <= 0.0f ? 0 : (x >= (float)(kLinBins - 1) ? kLinBins - 1 : (int)x);
}

// float4 b of a row (nodes 4b .. 4b+3): -inf past the row's end or, with
// parent bits in LDS, when its parent (node 4b / C = 4b >> lgC) was not kept.
__device__ __forceinline__ float4 row_f4(const float4* row4, int64_t n4, const uint32_t* pbits, int lgC, int64_t b) {
  bool ok = b < n4;
  if (pbits && ok) {
    const int64_t pi = (4 * b) >> lgC;
    ok = (pbits[pi >> 5] >> (pi & 31)) & 1u;
  }
  return ok ? row4[b] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
}

__device__ uint32_t block_minmax_u32(uint32_t v, bool want_max, unsigned long long* red) {
  const int tid = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t u = (uint32_t)__shfl_xor((int)v, o);
    v = want_max ? max(v, u) : min(v, u);
  }
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  uint32_t r = (uint32_t)red[0];
#pragma unroll
  for (int w = 1; w < kSelThreads / 64; ++w) r = want_max ? max(r, (uint32_t)red[w]) : min(r, (uint32_t)red[w]);
  __syncthreads();  // red is free again
  return r;
}

// One workgroup per query.
__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs A) {
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.x;
  const float* row = A.score + q * A.score_stride;  // 16-byte aligned rows
  const float4* row4 = reinterpret_cast<const float4*>(row);
  const int64_t n = A.n_nodes;
  const int64_t n4 = (n + 3) / 4;
  uint32_t* srow = A.sel + q * A.words;
  SelStats* st = reinterpret_cast<SelStats*>(A.stats) + q;
  const int64_t nwords = (n + 31) / 32;

  __shared__ unsigned long long hist[2048];
  __shared__ unsigned long long red[kSelThreads / 64];  // per-wave partials of the block reductions
  __shared__ int sh_bin;
  __shared__ unsigned long long sh_above;
  __shared__ uint32_t l_key[kCutCap];
  __shared__ int l_id[kCutCap];
  __shared__ unsigned long long l_mass[kCutCap];
  extern __shared__ uint32_t l_par[];  // A.parent_lds words
  __shared__ int l_n;

  uint32_t kmax, kmin;
  unsigned long long ncand;
  reduce_slots(A, q, &kmax, &kmin, &ncand);
  if (ncand == 0) {
    for (int64_t w = tid; w < nwords; w += kSelThreads) srow[w] = 0u;
    if (tid == 0) {
      SelStats s0 = {kNegInf, 0, 0, 0u, 0, 0, 0ull, 0ull};
      *st = s0;
    }
    return;
  }
  const SelSetup su = sel_setup(kmax, kmin, n);
  const float mx = su.mx;
  const double scale = su.scale;

  unsigned long long M = 0, P = 0, above = 0, h_tau = 0;
  uint32_t tau = 0u;
  int cut_id = INT_MAX;
  unsigned long long kept = 0, kmass = 0;
  bool done = false;

  if (!A.keep_all && A.cut_cap > 0) {
    // the parent bits of this query, when there are any and they fit
    const uint32_t* pbits = nullptr;
    const int lgC = __ffs(A.C) - 1;  // C is a power of two
    if (A.sel_parent) {
      const int64_t pw = (((n4 - 1) * 4 >> lgC) >> 5) + 1;  // parent words the row's float4s reach
      if (pw <= A.parent_lds) {
        const uint32_t* prow = A.sel_parent + q * A.parent_words;
        for (int64_t i = tid; i < pw; i += kSelThreads) l_par[i] = prow[i];
        pbits = l_par;
      }
    }
    // pass 1: M and the linear-bin histogram, over the candidates' score
    // range down to where the masses reach 0
    const float span = (float)(su.shift + 2) * 0.6931472f;  // exp(-span) * 2^shift < 1/4: mass 0 below
    const float lo = fmaxf(mx - span, key_to_float(kmin));
    const float inv_w = (float)kLinBins / fmaxf(mx - lo, 1e-30f);
    for (int i = tid; i < kLinBins; i += kSelThreads) hist[i] = 0ull;
    if (tid == 0) l_n = 0;
    __syncthreads();
    unsigned long long part = 0;
    for (int64_t b0 = 0; b0 < n4; b0 += (int64_t)kSelThreads * kSelUnroll) {
      float4 v[kSelUnroll];
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) v[u] = row_f4(row4, n4, pbits, lgC, b0 + u * kSelThreads + tid);
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const float a[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const int64_t i0 = (b0 + u * kSelThreads + tid) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (i0 + e < n && a[e] > kNegInf) {
            const unsigned long long m = fixed_mass(a[e], mx, scale);
            part += m;
            if (m) atomicAdd(&hist[lin_bin(a[e], lo, inv_w)], m);
          }
        }
      }
    }
    __syncthreads();
    M = block_sum_u64(part, red);
    P = p_target(A.p, M);
    const int bcut = find_bin(hist, kLinBins, P, &above, red, &sh_bin, &sh_above);
    // the kept mass of the bins above the cut bin is their histogram mass
    // (the same integer masses; every candidate when no bin is cut, M = 0)
    const unsigned long long above_bins = bcut >= 0 ? above : M;
    // pass 2: bits of the bins above the cut bin; the cut bin's candidates to
    // LDS.  Eight consecutive lanes hold one bitset word's 32 candidates.
    for (int64_t b0 = 0; b0 < n4; b0 += (int64_t)kSelThreads * kSelUnroll) {
      float4 v[kSelUnroll];
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) v[u] = row_f4(row4, n4, pbits, lgC, b0 + u * kSelThreads + tid);
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const float a[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const int64_t b = b0 + u * kSelThreads + tid;
        uint32_t nib = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t i = b * 4 + e;
          if (i < n && a[e] > kNegInf) {
            const int bin = lin_bin(a[e], lo, inv_w);
            if (bin > bcut) {
              nib |= 1u << e;
            } else if (bin == bcut) {
              const int j = atomicAdd(&l_n, 1);
              if (j < A.cut_cap) {
                l_key[j] = order_key(a[e]);
                l_id[j] = (int)i;
                l_mass[j] = fixed_mass(a[e], mx, scale);
              }
            }
          }
        }
        kept += __popc(nib);
        uint32_t word = nib << (4 * (tid & 7));
        word |= __shfl_xor(word, 1);
        word |= __shfl_xor(word, 2);
        word |= __shfl_xor(word, 4);
        if ((tid & 7) == 0 && b / 8 < nwords) srow[b / 8] = word;
      }
    }
    __syncthreads();  // the row's words are stored and visible to the workgroup before the or-ed bits
    const int nl = l_n;
    if (nl <= A.cut_cap) {
      // radix digits over the cut bin's candidates in LDS find the cut key,
      // starting below the common prefix of their keys
      uint32_t kl_max = 0u, kl_min = 0xffffffffu;
      for (int j = tid; j < nl; j += kSelThreads) {
        kl_max = max(kl_max, l_key[j]);
        kl_min = min(kl_min, l_key[j]);
      }
      kl_max = block_minmax_u32(kl_max, true, red);
      kl_min = block_minmax_u32(kl_min, false, red);
      const int hb = kl_max == kl_min ? 0 : 32 - __clz(kl_max ^ kl_min);
      uint32_t want = hb >= 32 ? 0u : (kl_max >> hb);
      int lo2 = hb;
      h_tau = hist[bcut];
      __syncthreads();
      while (lo2 > 0) {
        const int w = lo2 < 11 ? lo2 : 11;
        const int nb = 1 << w;
        const int top = lo2;
        lo2 -= w;
        for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0ull;
        __syncthreads();
        const uint32_t mask = (uint32_t)(nb - 1);
        for (int j = tid; j < nl; j += kSelThreads) {
          const uint32_t k = l_key[j];
          if (top >= 32 || (k >> top) == want) atomicAdd(&hist[(k >> lo2) & mask], l_mass[j]);
        }
        __syncthreads();
        const int bsel = find_bin(hist, nb, P, &above, red, &sh_bin, &sh_above);
        want = (w >= 32 ? 0u : (want << w)) | (uint32_t)bsel;
        h_tau = hist[bsel];
        __syncthreads();
      }
      tau = want;
      // ties at tau carry one mass: the lowest `need` ids are kept (0: all)
      const unsigned long long need = ties_needed(tau, P, above, h_tau, mx, scale);
      if (need) {
        __shared__ int sh_cut;
        if (tid == 0) sh_cut = INT_MAX;
        __syncthreads();
        for (int j = tid; j < nl; j += kSelThreads) {
          if (l_key[j] != tau) continue;
          unsigned long long rank = 0ull;  // ties with a lower id
          for (int f = 0; f < nl; ++f) rank += (l_key[f] == tau && l_id[f] < l_id[j]) ? 1ull : 0ull;
          if (rank == need - 1ull) sh_cut = l_id[j] + 1;
        }
        __syncthreads();
        cut_id = sh_cut;
        __syncthreads();
      }
      for (int j = tid; j < nl; j += kSelThreads) {
        const uint32_t k = l_key[j];
        const int id = l_id[j];
        if (k > tau || (k == tau && id < cut_id)) {
          atomicOr(&srow[id >> 5], 1u << (id & 31));
          kmass += l_mass[j];
          ++kept;
        }
      }
      if (tid == 0) kmass += above_bins;
      done = true;
    } else {
      kept = 0ull;
      kmass = 0ull;
      above = 0ull;
    }
  }

  if (!done) {
    // radix digit passes on the order key; the first one also sums M
    uint32_t want = su.want;
    int lo = su.lo;
    bool first = true;
    bool found = false;
    do {
      const int w = lo < 11 ? lo : 11;
      const int nb = 1 << w;
      const int top = lo;  // bits [top, 32) must equal `want`
      lo -= w;
      for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0ull;
      __syncthreads();
      const unsigned long long part = digit_pass(row4, n, 0, n4, first, top, lo, w, want, mx, scale, hist);
      __syncthreads();
      if (first) {
        M = block_sum_u64(part, red);
        first = false;
        if (A.keep_all) break;
        P = p_target(A.p, M);
        if (w == 0) {  // every candidate has the same key
          want = kmax;
          h_tau = M;
          found = true;
          break;
        }
      }
      const int bsel = find_bin(hist, nb, P, &above, red, &sh_bin, &sh_above);
      want = (w >= 32 ? 0u : (want << w)) | (uint32_t)bsel;
      h_tau = hist[bsel];
      __syncthreads();
      found = lo == 0;
    } while (!found);

    unsigned long long need = 0;
    if (!A.keep_all) {
      tau = want;
      need = ties_needed(tau, P, above, h_tau, mx, scale);
      if (need) cut_id = tie_find(row, 0, n, tau, need);
    }
    write_bits(row4, n, 0, nwords, tau, cut_id, srow, &kept);
    kmass = tid == 0 ? kept_mass(A.keep_all, M, above, h_tau, need, tau, mx, scale) : 0ull;
  }
  const unsigned long long nk = block_sum_u64(kept, red);
  const unsigned long long km = block_sum_u64(kmass, red);
  if (tid == 0) {
    SelStats s1;
    s1.max_score = mx;
    s1.n_cand = (int32_t)ncand;
    s1.n_kept = (int32_t)nk;
    s1.cut_key = tau;
    s1.cut_id = cut_id;
    s1.shift = su.shift;
    s1.mass_total = M;
    s1.mass_kept = km;
    *st = s1;
  }
}

// Wave form: one wave per query for rows of at most kWaveRow candidates
// (register i of lane l holds candidate 64i + l, so that the steps past the
// row's end, i >= ceil(n / 64), are skipped by the whole wave; step i's
// ballot is bitset words 2i and 2i + 1).  Same fixed-point masses and the
// same cut as k_select;
// the radix digits are 8 bits wide (a 256-bin histogram per wave in LDS),
// which changes the number of passes, not the key found: each pass narrows
// to the one bin whose mass interval holds P, and the last pass ends at the
// exact cut key.
constexpr int kWaveRow = 2048;
// levels with fewer queries keep one workgroup per query (no gain from
// finer work items there)
constexpr int64_t kWaveQueries = 64;

__global__ __launch_bounds__(256) void k_select_wave(SelectArgs A, int64_t n_queries) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = (int64_t)blockIdx.x * 4 + wave;
  if (q >= n_queries) return;  // uniform per wave; nothing below synchronises waves
  __shared__ unsigned long long hist_all[4][256];
  unsigned long long* hist = hist_all[wave];
  const int64_t n = A.n_nodes;
  const int nit = (int)((n + 63) / 64);  // steps holding candidates (<= 32; the same in every lane)
  const float* row = A.score + q * A.score_stride;
  uint32_t* srow = A.sel + q * A.words;
  SelStats* st = reinterpret_cast<SelStats*>(A.stats) + q;
  const int64_t nwords = (n + 31) / 32;

  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t e = 64 * (int64_t)i + lane;
    v[i] = (i < nit && e < n) ? row[e] : kNegInf;
  }

  // candidate key range and count from the score tiles' slots
  uint32_t kmax = 0u, kmin = 0xffffffffu;
  unsigned long long ncand = 0ull;
  {
    const uint4* kr = reinterpret_cast<const uint4*>(A.keyrange) + q * A.kr_slots;
    for (int64_t i = lane; i < A.kr_used; i += 64) {
      const uint4 s = kr[i];
      kmax = max(kmax, s.x);
      kmin = min(kmin, s.y);
      ncand += s.z;
    }
    for (int o = 1; o < 64; o <<= 1) {
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
      ncand += __shfl_xor(ncand, o);
    }
  }
  if (ncand == 0) {
    if (lane < nwords) srow[lane] = 0u;
    if (lane == 0) {
      SelStats s0 = {kNegInf, 0, 0, 0u, 0, 0, 0ull, 0ull};
      *st = s0;
    }
    return;
  }
  const SelSetup su = sel_setup(kmax, kmin, n);
  const float mx = su.mx;
  const double scale = su.scale;
  auto wsum = [](unsigned long long x) {
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
    return x;
  };

  uint32_t want = su.want;
  int lo = su.lo;
  unsigned long long M = 0, P = 0, above = 0, h_tau = 0;
  bool first = true, found = false;
  do {
    const int w = lo < 8 ? lo : 8;
    const int nb = 1 << w;
    const int top = lo;
    lo -= w;
    for (int i = lane; i < nb; i += 64) hist[i] = 0ull;
    wave_sync();
    unsigned long long part = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float s = i < nit ? v[i] : kNegInf;
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        const bool match = top >= 32 || (k >> top) == want;
        if (first || match) {
          const unsigned long long mm = fixed_mass(s, mx, scale);
          if (first) part += mm;
          if (match && w > 0) atomicAdd(&hist[(k >> lo) & (uint32_t)(nb - 1)], mm);
        }
      }
    }
    wave_sync();
    if (first) {
      M = wsum(part);
      first = false;
      if (A.keep_all) break;
      P = p_target(A.p, M);
      if (w == 0) {  // every candidate has the same key
        want = kmax;
        h_tau = M;
        found = true;
        break;
      }
    }
    // the bin, scanning from the top, whose mass interval holds P: each lane
    // sums nb / 64 bins (or one), an inclusive suffix sum over the lanes
    // gives the mass above each lane's bins
    const int per = nb >= 64 ? nb / 64 : 1;
    const int b0 = lane * per;
    const int cnt = b0 < nb ? per : 0;
    unsigned long long mine = 0;
    for (int i = 0; i < cnt; ++i) mine += hist[b0 + i];
    unsigned long long suf = mine;
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long t = __shfl_down(suf, o);
      if (lane + o < 64) suf += t;
    }
    unsigned long long cum = above + (suf - mine);
    int bin = -1;
    unsigned long long bin_above = 0;
    for (int i = cnt - 1; i >= 0; --i) {
      const unsigned long long hv = hist[b0 + i];
      if (bin < 0 && cum < P && P <= cum + hv) {
        bin = b0 + i;
        bin_above = cum;
      }
      cum += hv;
    }
    const unsigned long long ball = __ballot(bin >= 0);
    const int src = ball ? __ffsll((long long)ball) - 1 : 0;
    const int bsel = __shfl(bin, src);
    if (ball) above = __shfl(bin_above, src);
    want = (w >= 32 ? 0u : (want << w)) | (uint32_t)bsel;
    h_tau = hist[bsel & (nb - 1)];
    wave_sync();
    found = lo == 0;
  } while (!found);

  uint32_t tau = 0u;
  int cut_id = INT_MAX;
  if (!A.keep_all) {
    tau = want;
    const unsigned long long need = ties_needed(tau, P, above, h_tau, mx, scale);
    if (need) {
      // the need-th tie in id order: step i holds ids 64i .. 64i + 63 in
      // lane order, so its ballot lists them in id order
      unsigned long long before = 0;
      int cut = -1;
      unsigned long long cut_b = 0ull;  // ballot of the step holding the cut, lower ties dropped
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i < nit) {
          const unsigned long long b = __ballot(v[i] > kNegInf && order_key(v[i]) == tau);
          const unsigned long long c = (unsigned long long)__popcll(b);
          if (cut < 0 && before < need && need <= before + c) {
            cut = i;
            cut_b = b;
          }
          if (cut < 0) before += c;
        }
      }
      if (cut >= 0) {
        for (unsigned long long left = need - before; left > 1ull; --left) cut_b &= cut_b - 1ull;
        cut_id = 64 * cut + (__ffsll((long long)cut_b) - 1) + 1;
      }
    }
  }

  unsigned long long kmass = 0, nk = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (i < nit) {
      const float s = v[i];
      bool keep = false;
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        if (k > tau || (k == tau && 64 * i + lane < cut_id)) {
          keep = true;
          kmass += fixed_mass(s, mx, scale);
        }
      }
      const unsigned long long b = __ballot(keep);  // words 2i (ids 64i ..) and 2i + 1
      nk += (unsigned long long)__popcll(b);
      if (lane < 2 && 2 * i + lane < nwords) srow[2 * i + lane] = lane == 0 ? (uint32_t)b : (uint32_t)(b >> 32);
    }
  }
  const unsigned long long km = wsum(kmass);
  if (lane == 0) {
    SelStats s1;
    s1.max_score = mx;
    s1.n_cand = (int32_t)ncand;
    s1.n_kept = (int32_t)nk;
    s1.cut_key = tau;
    s1.cut_id = cut_id;
    s1.shift = su.shift;
    s1.mass_total = M;
    s1.mass_kept = km;
    *st = s1;
  }
}

// Row form: one 256-thread workgroup per query for rows of at most
// kRowsRow candidates, register i of thread t holding candidate 256i + t
// (steps past the row's end skipped by the whole workgroup; step i's ballot
// in wave w is bitset words 8i + 2w and 8i + 2w + 1).  The steps of the wave form
// with workgroup-wide sums and scans: 8-bit digits over one LDS histogram,
// each thread owning one bin in the scan.
constexpr int kRowsRow = 8192;

__global__ __launch_bounds__(256) void k_select_rows(SelectArgs A) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t q = blockIdx.x;
  __shared__ unsigned long long hist[256];
  __shared__ unsigned long long wred[4];
  __shared__ uint32_t wmax[4], wmin[4];
  __shared__ int sh_i[2];
  __shared__ unsigned long long sh_u[2];
  __shared__ uint32_t tcnt[4][32];  // ties at the cut key per wave and step
  const int64_t n = A.n_nodes;
  const int nit = (int)((n + 255) / 256);  // steps holding candidates (<= 32)
  const float* row = A.score + q * A.score_stride;
  uint32_t* srow = A.sel + q * A.words;
  SelStats* st = reinterpret_cast<SelStats*>(A.stats) + q;
  const int64_t nwords = (n + 31) / 32;

  // workgroup sum of a 64-bit value (every thread gets it)
  auto bsum = [&](unsigned long long x) {
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
    if (lane == 0) wred[wave] = x;
    __syncthreads();
    const unsigned long long r = (wred[0] + wred[1]) + (wred[2] + wred[3]);
    __syncthreads();
    return r;
  };

  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t e = 256 * (int64_t)i + tid;
    v[i] = (i < nit && e < n) ? row[e] : kNegInf;
  }

  uint32_t kmax = 0u, kmin = 0xffffffffu;
  unsigned long long ncand = 0ull;
  {
    const uint4* kr = reinterpret_cast<const uint4*>(A.keyrange) + q * A.kr_slots;
    for (int64_t i = tid; i < A.kr_used; i += 256) {
      const uint4 s = kr[i];
      kmax = max(kmax, s.x);
      kmin = min(kmin, s.y);
      ncand += s.z;
    }
    for (int o = 1; o < 64; o <<= 1) {
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    }
    if (lane == 0) {
      wmax[wave] = kmax;
      wmin[wave] = kmin;
    }
    __syncthreads();
    kmax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    kmin = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    ncand = bsum(ncand);
  }
  if (ncand == 0) {
    if (tid < nwords) srow[tid] = 0u;
    if (tid == 0) {
      SelStats s0 = {kNegInf, 0, 0, 0u, 0, 0, 0ull, 0ull};
      *st = s0;
    }
    return;
  }
  const SelSetup su = sel_setup(kmax, kmin, n);
  const float mx = su.mx;
  const double scale = su.scale;

  uint32_t want = su.want;
  int lo = su.lo;
  unsigned long long M = 0, P = 0, above = 0, h_tau = 0;
  bool first = true, found = false;
  do {
    const int w = lo < 8 ? lo : 8;
    const int nb = 1 << w;
    const int top = lo;
    lo -= w;
    hist[tid] = 0ull;
    __syncthreads();
    unsigned long long part = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float s = i < nit ? v[i] : kNegInf;
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        const bool match = top >= 32 || (k >> top) == want;
        if (first || match) {
          const unsigned long long mm = fixed_mass(s, mx, scale);
          if (first) part += mm;
          if (match && w > 0) atomicAdd(&hist[(k >> lo) & (uint32_t)(nb - 1)], mm);
        }
      }
    }
    __syncthreads();
    if (first) {
      M = bsum(part);
      first = false;
      if (A.keep_all) break;
      P = p_target(A.p, M);
      if (w == 0) {  // every candidate has the same key
        want = kmax;
        h_tau = M;
        found = true;
        break;
      }
    }
    // bin tid: mass of the bins above it by a suffix sum over the threads
    const unsigned long long mine = tid < nb ? hist[tid] : 0ull;
    unsigned long long suf = mine;
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long t = __shfl_down(suf, o);
      if (lane + o < 64) suf += t;
    }
    if (lane == 0) wred[wave] = suf;  // the wave's total
    __syncthreads();
    unsigned long long hi_waves = 0;
    for (int w2 = wave + 1; w2 < 4; ++w2) hi_waves += wred[w2];
    const unsigned long long cum = above + hi_waves + (suf - mine);  // mass strictly above bin tid
    if (tid == 0) sh_i[0] = -1;
    __syncthreads();
    if (tid < nb && cum < P && P <= cum + mine) {
      sh_i[0] = tid;
      sh_u[0] = cum;
    }
    __syncthreads();
    const int bsel = sh_i[0];
    if (bsel >= 0) above = sh_u[0];
    want = (w >= 32 ? 0u : (want << w)) | (uint32_t)bsel;
    h_tau = hist[bsel & (nb - 1)];
    __syncthreads();
    found = lo == 0;
  } while (!found);

  uint32_t tau = 0u;
  int cut_id = INT_MAX;
  if (!A.keep_all) {
    tau = want;
    const unsigned long long need = ties_needed(tau, P, above, h_tau, mx, scale);
    if (need) {
      // the need-th tie in id order (step, then wave, then lane): the ties
      // per wave and step through LDS, then the wave holding the cut finds
      // its bit in that step's ballot
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i < nit) {
          const unsigned long long b = __ballot(v[i] > kNegInf && order_key(v[i]) == tau);
          if (lane == 0) tcnt[wave][i] = (uint32_t)__popcll(b);
        }
      }
      if (tid == 0) sh_i[1] = INT_MAX;
      __syncthreads();
      unsigned long long before = 0;
      int istar = -1, wstar = -1;
      for (int i = 0; i < nit && istar < 0; ++i)
        for (int w2 = 0; w2 < 4 && istar < 0; ++w2) {
          const unsigned long long c = tcnt[w2][i];
          if (before < need && need <= before + c) {
            istar = i;
            wstar = w2;
          } else {
            before += c;
          }
        }
      if (istar >= 0 && wave == wstar) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i == istar) {
            unsigned long long b = __ballot(v[i] > kNegInf && order_key(v[i]) == tau);
            for (unsigned long long left = need - before; left > 1ull; --left) b &= b - 1ull;  // drop lower ties
            if (lane == 0) sh_i[1] = 256 * i + 64 * wave + (__ffsll((long long)b) - 1) + 1;
          }
        }
      }
      __syncthreads();
      cut_id = sh_i[1];
    }
  }

  unsigned long long kmass = 0, nkeep = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (i < nit) {
      const float s = v[i];
      bool keep = false;
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        if (k > tau || (k == tau && 256 * i + tid < cut_id)) {
          keep = true;
          kmass += fixed_mass(s, mx, scale);
        }
      }
      nkeep += keep ? 1ull : 0ull;
      const unsigned long long b = __ballot(keep);  // words 8i + 2 wave and 8i + 2 wave + 1
      const int64_t wd = 8 * (int64_t)i + 2 * wave + lane;
      if (lane < 2 && wd < nwords) srow[wd] = lane == 0 ? (uint32_t)b : (uint32_t)(b >> 32);
    }
  }
  const unsigned long long nk = bsum(nkeep);
  const unsigned long long km = bsum(kmass);
  if (tid == 0) {
    SelStats s1;
    s1.max_score = mx;
    s1.n_cand = (int32_t)ncand;
    s1.n_kept = (int32_t)nk;
    s1.cut_key = tau;
    s1.cut_id = cut_id;
    s1.shift = su.shift;
    s1.mass_total = M;
    s1.mass_kept = km;
    *st = s1;
  }
}

// Split form: S workgroups per query, each on its share of the row's words,
// for levels with few queries and many candidates.  The per-query state and
// the segments' histograms live in the route workspace; a chain of kernels
// (set-up; per digit a histogram kernel over the segments and a find kernel
// per query; the ties at the cut key counted per segment; the bitset over
// the segments, where the segment holding the last kept tie finds it; the
// statistics) takes the same steps as k_select and reaches bit-identical
// results, since every sum is of integers.
struct SelState {
  double scale;
  unsigned long long ncand, M, P, above, h_tau;
  float mx;
  int32_t shift;
  unsigned long long need_tie;  // ties at tau to keep (smallest ids first), 0: all
  uint32_t kmax, want, tau;
  int32_t lo, first, phase;  // phase 0: digit passes, 1: cut key known, 2: no candidate
};
static_assert(sizeof(SelState) <= kSelStateBytes, "select state size");

__device__ __forceinline__ SelState* sel_state(const SelectArgs& A, int64_t q) {
  return reinterpret_cast<SelState*>(static_cast<char*>(A.split) + q * kSelStateBytes);
}
// Segment slot of (query, segment): histogram bins, then the first pass's
// mass, the kept count, one unused word, the ties at the cut key and the
// segment's cut id.
constexpr int kSlotM = 2048, kSlotKept = 2049, kSlotTies = 2051, kSlotCut = 2052;
__device__ __forceinline__ unsigned long long* sel_slot(const SelectArgs& A, int64_t n_queries, int64_t q,
                                                         int64_t s) {
  return reinterpret_cast<unsigned long long*>(static_cast<char*>(A.split) + n_queries * kSelStateBytes) +
         (q * A.split_S + s) * kSelSlotU64;
}
__device__ __forceinline__ void segment_words(const SelectArgs& A, int64_t s, int64_t* w0, int64_t* w1) {
  const int64_t nwords = (A.n_nodes + 31) / 32;
  const int64_t per = (nwords + A.split_S - 1) / A.split_S;
  *w0 = min(s * per, nwords);
  *w1 = min(*w0 + per, nwords);
}

__global__ __launch_bounds__(kSelThreads) void k_select_setup(SelectArgs A) {
  const int64_t q = blockIdx.x;
  uint32_t kmax, kmin;
  unsigned long long ncand;
  reduce_slots(A, q, &kmax, &kmin, &ncand);
  if (threadIdx.x != 0) return;
  SelState s;
  s.scale = 0.0;
  s.ncand = ncand;
  s.M = s.P = s.above = s.h_tau = 0ull;
  s.mx = kNegInf;
  s.shift = 0;
  s.kmax = kmax;
  s.want = 0u;
  s.tau = 0u;
  s.need_tie = 0ull;
  s.lo = 0;
  s.first = 1;
  s.phase = ncand == 0 ? 2 : 0;
  if (ncand != 0) {
    const SelSetup su = sel_setup(kmax, kmin, A.n_nodes);
    s.scale = su.scale;
    s.mx = su.mx;
    s.shift = su.shift;
    s.want = su.want;
    s.lo = su.lo;
  }
  *sel_state(A, q) = s;
}

__global__ __launch_bounds__(kSelThreads) void k_select_hist(SelectArgs A) {
  const int64_t seg = blockIdx.x, q = blockIdx.y;
  const SelState s = *sel_state(A, q);
  if (s.phase != 0) return;
  __shared__ unsigned long long hist[2048];
  __shared__ unsigned long long red[kSelThreads / 64];  // per-wave partials of the block reductions
  const int w = s.lo < 11 ? s.lo : 11;
  const int nb = 1 << w;
  const int64_t n = A.n_nodes;
  const float4* row4 = reinterpret_cast<const float4*>(A.score + q * A.score_stride);
  int64_t w0, w1;
  segment_words(A, seg, &w0, &w1);
  const int64_t b1 = min(w1 * 8, (n + 3) / 4);
  for (int i = threadIdx.x; i < nb; i += kSelThreads) hist[i] = 0ull;
  __syncthreads();
  const unsigned long long part =
      digit_pass(row4, n, w0 * 8, b1, s.first != 0, s.lo, s.lo - w, w, s.want, s.mx, s.scale, hist);
  __syncthreads();
  unsigned long long* out = sel_slot(A, gridDim.y, q, seg);
  if (w > 0)
    for (int i = threadIdx.x; i < nb; i += kSelThreads) out[i] = hist[i];
  if (s.first) {
    const unsigned long long m = block_sum_u64(part, red);
    if (threadIdx.x == 0) out[kSlotM] = m;
  }
}

__global__ __launch_bounds__(kSelThreads) void k_select_find(SelectArgs A, int64_t n_queries) {
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.x;
  SelState s = *sel_state(A, q);
  if (s.phase != 0) return;
  __shared__ unsigned long long hist[2048];
  __shared__ unsigned long long red[kSelThreads / 64];  // per-wave partials of the block reductions
  __shared__ int sh_bin;
  __shared__ unsigned long long sh_above;
  const int w = s.lo < 11 ? s.lo : 11;
  const int nb = 1 << w;
  bool found = false;
  if (s.first) {
    unsigned long long part = 0;
    for (int64_t g = tid; g < A.split_S; g += kSelThreads) part += sel_slot(A, n_queries, q, g)[kSlotM];
    s.M = block_sum_u64(part, red);
    s.first = 0;
    if (A.keep_all) {
      s.phase = 1;
      if (tid == 0) *sel_state(A, q) = s;
      return;
    }
    s.P = p_target(A.p, s.M);
    if (w == 0) {  // every candidate has the same key
      s.want = s.kmax;
      s.h_tau = s.M;
      found = true;
    }
  }
  if (!found) {
    // bin i summed over the segments, 8 loads in flight per thread
    const unsigned long long* slots = sel_slot(A, n_queries, q, 0);
    const int64_t S = A.split_S;
    for (int i = tid; i < nb; i += kSelThreads) {
      unsigned long long h = 0;
      int64_t g = 0;
      for (; g + 8 <= S; g += 8) {
        unsigned long long v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = slots[(g + u) * kSelSlotU64 + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) h += v[u];
      }
      for (; g < S; ++g) h += slots[g * kSelSlotU64 + i];
      hist[i] = h;
    }
    __syncthreads();
    const int bsel = find_bin(hist, nb, s.P, &s.above, red, &sh_bin, &sh_above);
    s.want = (w >= 32 ? 0u : (s.want << w)) | (uint32_t)bsel;
    s.h_tau = hist[bsel];
    s.lo -= w;
    __syncthreads();
    found = s.lo == 0;
  }
  if (found) {
    s.tau = s.want;
    s.need_tie = ties_needed(s.tau, s.P, s.above, s.h_tau, s.mx, s.scale);
    s.phase = 1;
  }
  if (tid == 0) *sel_state(A, q) = s;
}

// Ties at the cut key per segment, when only some of them are kept.
__global__ __launch_bounds__(kSelThreads) void k_select_ties(SelectArgs A) {
  const int64_t seg = blockIdx.x, q = blockIdx.y;
  const SelState s = *sel_state(A, q);
  if (s.phase != 1 || s.need_tie == 0ull) return;
  __shared__ unsigned long long red[kSelThreads / 64];  // per-wave partials of the block reductions
  int64_t w0, w1;
  segment_words(A, seg, &w0, &w1);
  const unsigned long long c =
      count_ties(A.score + q * A.score_stride, w0 * 32, min(w1 * 32, A.n_nodes), s.tau, red);
  if (threadIdx.x == 0) sel_slot(A, gridDim.y, q, seg)[kSlotTies] = c;
}

__global__ __launch_bounds__(kSelThreads) void k_select_bits(SelectArgs A) {
  const int64_t seg = blockIdx.x, q = blockIdx.y;
  const SelState s = *sel_state(A, q);
  __shared__ unsigned long long red[kSelThreads / 64];  // per-wave partials of the block reductions
  int64_t w0, w1;
  segment_words(A, seg, &w0, &w1);
  uint32_t* srow = A.sel + q * A.words;
  if (s.phase == 2) {
    for (int64_t w = w0 + threadIdx.x; w < w1; w += kSelThreads) srow[w] = 0u;
    return;
  }
  const float* row = A.score + q * A.score_stride;
  unsigned long long* out = sel_slot(A, gridDim.y, q, seg);
  // ties at the cut key kept in this segment: all while the segments before
  // hold fewer than need_tie, none after; the segment that holds the
  // need_tie-th one cuts inside and records its cut id
  int cut = INT_MAX, cut_rec = INT_MAX;
  if (s.phase == 1 && s.need_tie) {
    unsigned long long before = 0;
    for (int64_t g = threadIdx.x; g < seg; g += kSelThreads) before += sel_slot(A, gridDim.y, q, g)[kSlotTies];
    before = block_sum_u64(before, red);
    const unsigned long long mine = out[kSlotTies];
    if (before >= s.need_tie) {
      cut = 0;
    } else if (s.need_tie - before <= mine) {
      cut = tie_find(row, w0 * 32, min(w1 * 32, A.n_nodes), s.tau, s.need_tie - before);
      cut_rec = cut;
    }
  }
  unsigned long long kept = 0;
  write_bits(reinterpret_cast<const float4*>(row), A.n_nodes, w0, w1, A.keep_all ? 0u : s.tau, cut, srow, &kept);
  const unsigned long long nk = block_sum_u64(kept, red);
  if (threadIdx.x == 0) {
    out[kSlotKept] = nk;
    out[kSlotCut] = (unsigned long long)(uint32_t)cut_rec;
  }
}

__global__ __launch_bounds__(64) void k_select_stats(SelectArgs A, int64_t n_queries) {
  const int64_t q = blockIdx.x;
  const SelState s = *sel_state(A, q);
  SelStats* st = reinterpret_cast<SelStats*>(A.stats) + q;
  if (s.phase == 2) {
    if (threadIdx.x == 0) {
      SelStats s0 = {kNegInf, 0, 0, 0u, 0, 0, 0ull, 0ull};
      *st = s0;
    }
    return;
  }
  unsigned long long nk = 0, cut = INT_MAX;
  for (int64_t g = threadIdx.x; g < A.split_S; g += 64) {
    const unsigned long long* slot = sel_slot(A, n_queries, q, g);
    nk += slot[kSlotKept];
    cut = min(cut, slot[kSlotCut]);  // at most one segment cuts inside its ties
  }
  for (int o = 1; o < 64; o <<= 1) {
    nk += __shfl_xor(nk, o);
    cut = min(cut, (unsigned long long)__shfl_xor(cut, o));
  }
  const unsigned long long km = kept_mass(A.keep_all, s.M, s.above, s.h_tau, s.need_tie, s.tau, s.mx, s.scale);
  if (threadIdx.x == 0) {
    SelStats s1;
    s1.max_score = s.mx;
    s1.n_cand = (int32_t)s.ncand;
    s1.n_kept = (int32_t)nk;
    s1.cut_key = A.keep_all ? 0u : s.tau;
    s1.cut_id = (int32_t)cut;
    s1.shift = s.shift;
    s1.mass_total = s.M;
    s1.mass_kept = km;
    *st = s1;
  }
}

}  // namespace

hipError_t launch_route_init(uint32_t* keyrange, int64_t n, Prof& prof) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_route_init, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, prof.s, keyrange, n);
  return hipGetLastError();
}

hipError_t launch_route_level(const ScoreArgs& sa, const SelectArgs& se, int dtype, int n_caches,
                              int level, Prof& prof) {
  const int64_t n_queries = (int64_t)n_caches * sa.QC;
  hipStream_t s = prof.s;
  // weights form: many queries per cache walk 16 query blocks over a tile;
  // the tile's keys
  const bool mq = sa.leaf_weights && sa.QC > 16 && (sa.n_nodes * sa.wkeys + 255) / 256 * n_caches >= kMqMinTiles;
  const int kt = leafw_tile(sa.wkeys, mq);
  if (sa.n_nodes > 0) {
    prof.begin(ZHA_K_SCORE, level);
    // weights-form levels: C keys per node at level 1 (C in {4, 8, 16}), or
    // 16-key nodes of 4 chunks at level 2 holding child shares (MODE 1; MODE
    // 2 also writes the level-1 scores), or level 1 after such a fused pass
    const bool w2lvl = sa.leaf_weights && sa.wkeys == 16 && sa.C == 4;
    const int64_t wtiles = sa.leaf_weights ? (sa.n_nodes * sa.wkeys + kt - 1) / kt : 0;
    if (sa.fuse1) {
      hipLaunchKernelGGL(k_score_mask1, dim3((unsigned)((wtiles + kMaskTiles - 1) / kMaskTiles), (unsigned)n_caches),
                         dim3(256), 0, s, sa, wtiles);
    } else if (mq) {
      dim3 grid((unsigned)wtiles, (unsigned)n_caches, (unsigned)((sa.QC + 16 * kMqBlocks - 1) / (16 * kMqBlocks)));
#define ZHA_LWM(DD, CC, MM)                                                                     \
  do {                                                                                          \
    if (sa.R == 16)                                                                             \
      hipLaunchKernelGGL((k_score_leafw_mq<DD, CC, 16, MM>), grid, dim3(256), 0, s, sa);        \
    else if (sa.R == 1)                                                                         \
      hipLaunchKernelGGL((k_score_leafw_mq<DD, CC, 1, MM>), grid, dim3(256), 0, s, sa);         \
    else                                                                                        \
      hipLaunchKernelGGL((k_score_leafw_mq<DD, CC, 0, MM>), grid, dim3(256), 0, s, sa);         \
  } while (0)
      if (sa.D == 128) {
        if (w2lvl) ZHA_LWM(128, 16, 1);
        else if (sa.wkeys == 4) ZHA_LWM(128, 4, 0);
        else if (sa.wkeys == 8) ZHA_LWM(128, 8, 0);
        else ZHA_LWM(128, 16, 0);
      } else {
        if (w2lvl) ZHA_LWM(64, 16, 1);
        else if (sa.wkeys == 4) ZHA_LWM(64, 4, 0);
        else if (sa.wkeys == 8) ZHA_LWM(64, 8, 0);
        else ZHA_LWM(64, 16, 0);
      }
#undef ZHA_LWM
    } else if (sa.leaf_weights) {
      dim3 grid((unsigned)wtiles, (unsigned)n_caches, (unsigned)((sa.QC + 15) / 16));
#define ZHA_LW_Q(DD, CC, QQ, MM)                                                                      \
  do {                                                                                                \
    constexpr int KTT = (CC) == 8 ? 64 : 256; /* leafw_tile */                                        \
    if (sa.R == 16)                                                                                   \
      hipLaunchKernelGGL((k_score_leafw<DD, CC, 16, QQ, MM, KTT>), grid, dim3(KTT), 0, s, sa);        \
    else if (sa.R == 1)                                                                               \
      hipLaunchKernelGGL((k_score_leafw<DD, CC, 1, QQ, MM, KTT>), grid, dim3(KTT), 0, s, sa);         \
    else                                                                                              \
      hipLaunchKernelGGL((k_score_leafw<DD, CC, 0, QQ, MM, KTT>), grid, dim3(KTT), 0, s, sa);         \
  } while (0)
#define ZHA_LW(DD, CC, MM)               \
  do {                                   \
    if (sa.QC <= 4)                      \
      ZHA_LW_Q(DD, CC, true, MM);        \
    else                                 \
      ZHA_LW_Q(DD, CC, false, MM);       \
  } while (0)
      if (w2lvl && sa.score1) {
        // level 2 with the level-1 scores (<= 4 queries per cache)
        if (sa.D == 128)
          ZHA_LW_Q(128, 16, true, 2);
        else
          ZHA_LW_Q(64, 16, true, 2);
      } else if (sa.D == 128) {
        if (w2lvl) ZHA_LW(128, 16, 1);
        else if (sa.wkeys == 4) ZHA_LW(128, 4, 0);
        else if (sa.wkeys == 8) ZHA_LW(128, 8, 0);
        else ZHA_LW(128, 16, 0);
      } else {
        if (w2lvl) ZHA_LW(64, 16, 1);
        else if (sa.wkeys == 4) ZHA_LW(64, 4, 0);
        else if (sa.wkeys == 8) ZHA_LW(64, 8, 0);
        else ZHA_LW(64, 16, 0);
      }
#undef ZHA_LW
#undef ZHA_LW_Q
    } else if (dtype == 1) {
      dim3 grid((unsigned)((sa.n_nodes + 63) / 64), (unsigned)n_caches, (unsigned)((sa.QC + 15) / 16));
      if (sa.gscale && sa.gfmt == 2) {
        if (sa.D != 128) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_score_bf16<128, 2>), grid, dim3(256), 0, s, sa);
      } else if (sa.gscale) {
        if (sa.D == 128)
          hipLaunchKernelGGL((k_score_bf16<128, 1>), grid, dim3(256), 0, s, sa);
        else
          hipLaunchKernelGGL((k_score_bf16<64, 1>), grid, dim3(256), 0, s, sa);
      } else if (sa.R > 8 && sa.QC > 16 && (sa.n_nodes + 63) / 64 * n_caches >= kMqMinTiles) {
        dim3 gmq((unsigned)((sa.n_nodes + 63) / 64), (unsigned)n_caches,
                 (unsigned)((sa.QC + 16 * kMqBlocks - 1) / (16 * kMqBlocks)));
        if (sa.D == 128)
          hipLaunchKernelGGL((k_score_bf16_mq<128>), gmq, dim3(256), 0, s, sa);
        else
          hipLaunchKernelGGL((k_score_bf16_mq<64>), gmq, dim3(256), 0, s, sa);
      } else if (sa.R <= 8) {
#define ZHA_SR(DD)                                                                          \
  do {                                                                                      \
    if (sa.R == 1)                                                                          \
      hipLaunchKernelGGL((k_score_smallr<DD, 1>), grid, dim3(256), 0, s, sa);               \
    else if (sa.R == 2)                                                                     \
      hipLaunchKernelGGL((k_score_smallr<DD, 2>), grid, dim3(256), 0, s, sa);               \
    else if (sa.R <= 4)                                                                     \
      hipLaunchKernelGGL((k_score_smallr<DD, 4>), grid, dim3(256), 0, s, sa);               \
    else                                                                                    \
      hipLaunchKernelGGL((k_score_smallr<DD, 8>), grid, dim3(256), 0, s, sa);               \
  } while (0)
        if (sa.D == 128)
          ZHA_SR(128);
        else
          ZHA_SR(64);
#undef ZHA_SR
      } else if (sa.D == 128) {
        hipLaunchKernelGGL((k_score_bf16<128, 0>), grid, dim3(256), 0, s, sa);
      } else {
        hipLaunchKernelGGL((k_score_bf16<64, 0>), grid, dim3(256), 0, s, sa);
      }
    } else {
      dim3 grid((unsigned)((sa.n_nodes + 3) / 4), (unsigned)n_caches);
      if (sa.D == 128)
        hipLaunchKernelGGL((k_score_generic<float, 128>), grid, dim3(256), 0, s, sa);
      else
        hipLaunchKernelGGL((k_score_generic<float, 64>), grid, dim3(256), 0, s, sa);
    }
    prof.end();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  SelectArgs sel = se;
  if (sa.n_nodes <= 0)
    sel.kr_used = 0;
  else if (sa.fuse1)  // k_score_mask1: one slot per workgroup of kMaskTiles tiles
    sel.kr_used = ((sa.n_nodes * sa.wkeys + kt - 1) / kt + kMaskTiles - 1) / kMaskTiles;
  else if (sa.leaf_weights)
    sel.kr_used = (sa.n_nodes * sa.wkeys + kt - 1) / kt;
  else if (dtype == 1)
    sel.kr_used = (sa.n_nodes + 63) / 64;
  else
    sel.kr_used = 1;
  if (sa.spine && level >= 2 && sa.n_nodes > 0) {
    if (sa.gfmt == 2) return hipErrorInvalidValue;  // prefill takes no MXFP4 rows
    // prefill: each query's partial node of this level, scored from the spine
    ScoreArgs sp = sa;
    sp.kr_spine_slot = sel.kr_used;
    const dim3 g((unsigned)((sa.n_queries + 3) / 4));
    if (sa.gscale) {
      if (sa.D == 128)
        hipLaunchKernelGGL((k_score_spine<128, true>), g, dim3(256), 0, s, sp);
      else
        hipLaunchKernelGGL((k_score_spine<64, true>), g, dim3(256), 0, s, sp);
    } else if (sa.D == 128) {
      hipLaunchKernelGGL((k_score_spine<128, false>), g, dim3(256), 0, s, sp);
    } else {
      hipLaunchKernelGGL((k_score_spine<64, false>), g, dim3(256), 0, s, sp);
    }
    sel.kr_used += 1;
  }
  prof.begin(ZHA_K_SELECT, level);
  sel.split_S = sel.split ? select_segments(n_queries, sel.n_nodes) : 1;
  if (sel.split_S < 2 && sel.n_nodes <= kWaveRow && n_queries >= kWaveQueries) {
    hipLaunchKernelGGL(k_select_wave, dim3((unsigned)((n_queries + 3) / 4)), dim3(256), 0, s, sel, n_queries);
  } else if (sel.split_S < 2 && sel.n_nodes <= kRowsRow && n_queries >= kWaveQueries) {
    hipLaunchKernelGGL(k_select_rows, dim3((unsigned)n_queries), dim3(256), 0, s, sel);
  } else if (sel.split_S < 2) {
    // LDS for the parent bits the rows reach (the kernel computes the same count)
    sel.parent_lds = 0;
    if (sel.sel_parent && !sel.keep_all && sel.cut_cap > 0 && sel.n_nodes > 0) {
      const int lgC = __builtin_ctz((unsigned)sel.C);
      const int64_t n4 = (sel.n_nodes + 3) / 4;
      const int64_t pw = (((n4 - 1) * 4 >> lgC) >> 5) + 1;
      if (pw <= kParentWords) sel.parent_lds = (int)pw;
    }
    hipLaunchKernelGGL(k_select, dim3((unsigned)n_queries), dim3(kSelThreads), (size_t)sel.parent_lds * 4, s, sel);
  } else {
    const dim3 segs((unsigned)sel.split_S, (unsigned)n_queries);
    hipLaunchKernelGGL(k_select_setup, dim3((unsigned)n_queries), dim3(kSelThreads), 0, s, sel);
    for (int pass = 0; pass < 3; ++pass) {  // 11-bit digits cover the 32-bit key in 3 passes
      hipLaunchKernelGGL(k_select_hist, segs, dim3(kSelThreads), 0, s, sel);
      hipLaunchKernelGGL(k_select_find, dim3((unsigned)n_queries), dim3(kSelThreads), 0, s, sel, n_queries);
    }
    hipLaunchKernelGGL(k_select_ties, segs, dim3(kSelThreads), 0, s, sel);
    hipLaunchKernelGGL(k_select_bits, segs, dim3(kSelThreads), 0, s, sel);
    hipLaunchKernelGGL(k_select_stats, dim3((unsigned)n_queries), dim3(64), 0, s, sel, n_queries);
  }
  prof.end();
  return hipGetLastError();
}

}  // namespace zha
