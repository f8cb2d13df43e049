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
// Select design.  One workgroup per query.  Masses are fixed-point integers
// round(exp(s - max) * 2^shift) so every sum is exact and order-independent
// (deterministic without float atomics).  The cut is found by a three-pass
// radix select on the order key of the score (11 + 11 + 10 bits) over
// mass-weighted histograms in LDS, then ties at the cut key are resolved by
// node id.  The kept set is written as a bitset.
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

// ---------------------------------------------------------------------------
// score, bf16, MFMA

template <int D>
__global__ __launch_bounds__(256) void k_score_bf16(ScoreArgs A) {
  constexpr int NS = D / 32;  // MFMA k-steps of 32 bf16
  constexpr int TILE = 64;
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
  const uint32_t* prow =
      A.sel_parent ? A.sel_parent + ((int64_t)cache * A.QC + qg0 + qn) * A.parent_words : nullptr;
  const int jrow = lane & 15;

  for (int u = 0; u < 16; u += 4) {
    bool cand[4], any[4];
    int64_t m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m[k] = n0 + wave * 16 + u + k;
      bool ok = m[k] < A.n_nodes && qn < nq;
      if (ok && prow) {
        const int64_t par = m[k] / A.C;
        ok = (prow[par >> 5] >> (par & 31)) & 1u;
      }
      cand[k] = ok;
      any[k] = __ballot(ok) != 0;
    }
    uint4 af[4][NS];
    float cv[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (any[k]) {
        const char* gn = gcache + m[k] * gnode;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          af[k][s] = jrow < R ? ld16(gn + ((int64_t)(4 * s + kg) * R + jrow) * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jj = 4 * kg + i;
          cv[k][i] = jj < R ? ccache[m[k] * R + jj] : kNegInf;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v = kNegInf;
      if (any[k]) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[k][s]), bq[s], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, cv[k][i] + acc[i] * A.inv_sqrt_d);
        v = fmaxf(v, __shfl_xor(v, 16));
        v = fmaxf(v, __shfl_xor(v, 32));
      }
      if (lane < 16) sc[qn][wave * 16 + u + k] = cand[k] ? v : kNegInf;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nq * TILE; idx += 256) {
    const int q = idx / TILE, x = idx % TILE;
    const int64_t mm = n0 + x;
    if (mm < A.n_nodes) A.score[((int64_t)cache * A.QC + qg0 + q) * A.node_cap + mm] = sc[q][x];
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
    if (lane == 0) A.score[qg * A.node_cap + m] = v;
  }
}

// ---------------------------------------------------------------------------
// select

constexpr int kSelThreads = 256;

__device__ __forceinline__ unsigned long long fixed_mass(float s, float mx, double scale) {
  return (unsigned long long)llrint((double)expf(s - mx) * scale);
}

// Block-wide sum of a 64-bit value.
__device__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int off = kSelThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const unsigned long long r = red[0];
  __syncthreads();
  return r;
}

// Finds the bin b (scanning from the highest bin down) whose mass interval
// (above, above + hist[b]] contains P, where `above` starts at *A_io and
// accumulates the bins above b.  Returns b and updates *A_io to the mass
// strictly above bin b.
__device__ int find_bin(const unsigned long long* hist, int nbins, unsigned long long P,
                        unsigned long long* A_io, unsigned long long* red, int* sh_bin,
                        unsigned long long* sh_above) {
  const int tid = threadIdx.x;
  const int per = nbins / kSelThreads;
  // thread t owns bins [t*per, (t+1)*per); suffix sums over threads
  unsigned long long mine = 0;
  for (int i = 0; i < per; ++i) mine += hist[tid * per + i];
  red[tid] = mine;
  __syncthreads();
  // inclusive suffix scan (Hillis-Steele) over 256 values
  for (int off = 1; off < kSelThreads; off <<= 1) {
    unsigned long long add = (tid + off < kSelThreads) ? red[tid + off] : 0ull;
    __syncthreads();
    red[tid] += add;
    __syncthreads();
  }
  unsigned long long cum = *A_io + (red[tid] - mine);  // mass of bins above this thread's range
  if (tid == 0) *sh_bin = -1;
  __syncthreads();
  for (int i = per - 1; i >= 0; --i) {
    const int bin = tid * per + i;
    const unsigned long long h = hist[bin];
    if (cum < P && P <= cum + h) {
      *sh_bin = bin;
      *sh_above = cum;
    }
    cum += h;
  }
  __syncthreads();
  const int b = *sh_bin;
  *A_io = *sh_above;
  __syncthreads();
  return b;
}

__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs A) {
  const int tid = threadIdx.x;
  const int64_t q = blockIdx.x;
  const float* row = A.score + q * A.node_cap;
  const int64_t n = A.n_nodes;
  uint32_t* srow = A.sel + q * A.words;
  SelStats* st = reinterpret_cast<SelStats*>(A.stats) + q;
  const int64_t nwords = (n + 31) / 32;

  __shared__ unsigned long long hist[2048];
  __shared__ unsigned long long red[kSelThreads];
  __shared__ float redf[kSelThreads];
  __shared__ int sh_bin;
  __shared__ unsigned long long sh_above;
  __shared__ int sh_cut;

  // pass 0: max score and candidate count
  float mx = kNegInf;
  unsigned long long cnt = 0;
  for (int64_t i = tid; i < n; i += kSelThreads) {
    const float s = row[i];
    if (s > kNegInf) {
      ++cnt;
      mx = fmaxf(mx, s);
    }
  }
  redf[tid] = mx;
  __syncthreads();
  for (int off = kSelThreads / 2; off > 0; off >>= 1) {
    if (tid < off) redf[tid] = fmaxf(redf[tid], redf[tid + off]);
    __syncthreads();
  }
  mx = redf[0];
  __syncthreads();
  const unsigned long long ncand = block_sum_u64(cnt, red);

  if (ncand == 0) {
    for (int64_t w = tid; w < nwords; w += kSelThreads) srow[w] = 0u;
    if (tid == 0) {
      SelStats s0 = {kNegInf, 0, 0, 0u, 0, 0, 0ull, 0ull};
      *st = s0;
    }
    return;
  }
  int lg = 0;
  while ((1ll << lg) < n) ++lg;
  const int shift = 62 - lg;
  const double scale = ldexp(1.0, shift);

  // pass 1: total mass and histogram of the top 11 key bits
  for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0ull;
  __syncthreads();
  unsigned long long part = 0;
  for (int64_t i = tid; i < n; i += kSelThreads) {
    const float s = row[i];
    if (s > kNegInf) {
      const unsigned long long mm = fixed_mass(s, mx, scale);
      part += mm;
      atomicAdd(&hist[order_key(s) >> 21], mm);
    }
  }
  __syncthreads();
  const unsigned long long M = block_sum_u64(part, red);

  uint32_t tau = 0u;
  int cut_id = INT_MAX;
  if (!A.keep_all) {
    unsigned long long P = (unsigned long long)ceil((double)A.p * (double)M);
    if (P < 1ull) P = 1ull;
    if (P > M) P = M;
    unsigned long long above = 0ull;
    const int b1 = find_bin(hist, 2048, P, &above, red, &sh_bin, &sh_above);
    // pass 2: next 11 bits inside bin b1
    for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0ull;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kSelThreads) {
      const float s = row[i];
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        if ((int)(k >> 21) == b1) atomicAdd(&hist[(k >> 10) & 2047u], fixed_mass(s, mx, scale));
      }
    }
    __syncthreads();
    const int b2 = find_bin(hist, 2048, P, &above, red, &sh_bin, &sh_above);
    // pass 3: last 10 bits
    const uint32_t hi22 = ((uint32_t)b1 << 11) | (uint32_t)b2;
    for (int i = tid; i < 2048; i += kSelThreads) hist[i] = 0ull;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kSelThreads) {
      const float s = row[i];
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        if ((k >> 10) == hi22) atomicAdd(&hist[k & 1023u], fixed_mass(s, mx, scale));
      }
    }
    __syncthreads();
    const int b3 = find_bin(hist, 1024, P, &above, red, &sh_bin, &sh_above);
    tau = (hi22 << 10) | (uint32_t)b3;
    // ties at tau all carry the same mass
    const unsigned long long m_tau = fixed_mass(key_to_float(tau), mx, scale);
    const unsigned long long n_tau = hist[b3] / m_tau;
    const unsigned long long k_tie = (P - above + m_tau - 1ull) / m_tau;
    __syncthreads();
    if (k_tie < n_tau) {
      // the k_tie-th smallest id among the ties is the last one kept
      unsigned long long need = k_tie;
      if (tid == 0) sh_cut = INT_MAX;
      __syncthreads();
      for (int64_t base = 0; base < n; base += kSelThreads) {
        const int64_t i = base + tid;
        const bool tie = i < n && row[i] > kNegInf && order_key(row[i]) == tau;
        const int c = __syncthreads_count(tie);
        if ((unsigned long long)c >= need) {
          red[tid] = tie ? 1ull : 0ull;
          __syncthreads();
          unsigned long long before = 0;
          for (int t = 0; t < tid; ++t) before += red[t];
          if (tie && before + 1ull == need) sh_cut = (int)(i + 1);
          __syncthreads();
          break;
        }
        need -= (unsigned long long)c;
      }
      cut_id = sh_cut;
    }
  }

  // pass 5: bitset of kept candidates
  unsigned long long kept = 0, kmass = 0;
  for (int64_t w = tid; w < nwords; w += kSelThreads) {
    uint32_t bits = 0u;
    for (int bb = 0; bb < 32; ++bb) {
      const int64_t i = w * 32 + bb;
      if (i >= n) break;
      const float s = row[i];
      if (s > kNegInf) {
        const uint32_t k = order_key(s);
        if (k > tau || (k == tau && i < (int64_t)cut_id)) {
          bits |= 1u << bb;
          kmass += fixed_mass(s, mx, scale);
        }
      }
    }
    srow[w] = bits;
    kept += __popc(bits);
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
    s1.shift = shift;
    s1.mass_total = M;
    s1.mass_kept = km;
    *st = s1;
  }
}

}  // namespace

hipError_t launch_route_level(const ScoreArgs& sa, const SelectArgs& se, int dtype, int n_caches,
                              int level, Prof& prof) {
  const int64_t n_queries = (int64_t)n_caches * sa.QC;
  hipStream_t s = prof.s;
  if (sa.n_nodes > 0) {
    prof.begin(ZHA_K_SCORE, level);
    if (dtype == 1) {
      dim3 grid((unsigned)((sa.n_nodes + 63) / 64), (unsigned)n_caches, (unsigned)((sa.QC + 15) / 16));
      if (sa.D == 128)
        hipLaunchKernelGGL(k_score_bf16<128>, grid, dim3(256), 0, s, sa);
      else
        hipLaunchKernelGGL(k_score_bf16<64>, grid, dim3(256), 0, s, sa);
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
  prof.begin(ZHA_K_SELECT, level);
  hipLaunchKernelGGL(k_select, dim3((unsigned)n_queries), dim3(kSelThreads), 0, s, se);
  prof.end();
  return hipGetLastError();
}

}  // namespace zha
