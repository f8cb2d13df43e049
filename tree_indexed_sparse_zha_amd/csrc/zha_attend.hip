// Exact attention over routed keys (split-K flash-decode) for ZHA on gfx950.
//
// Defines (MTP = "Zyphra AI Introduces Zyphra Hierarchical Attention (ZHA):
// A Path to True Subquadratic Attention", widget "1 . How it works" step 5
// and section "How does top-p routing pick tokens?"): exact softmax attention
// over the keys of the selected level-1 chunks, plus token 0 (the sink) and
// the current chunk; with all keys selected it is dense decode attention.
//
// Design.  Grid = (key tile, cache, group of up to 4 queries of the cache).
// The queries of one group share every K/V byte they read (the G query heads
// of a KV head are packed together, as dense GQA decode does).  Lanes are
// (key slot, 16-byte piece of the row): each wave step reads 64 x 16 B of K
// and of V, i.e. whole rows of 4 keys (bf16, d = 128), skipping steps no
// query of the group selected, so reads are gathered at chunk granularity.
// q.k is a per-lane partial dot plus a butterfly over the lanes of one row;
// the softmax is online in fp32 with one rescale per 4 key steps.  Each
// workgroup writes (max, sum, weighted V sum) per query; a second kernel
// combines the tiles in a fixed order (deterministic, no atomics).
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {
namespace {

constexpr int kAttThreads = 256;

constexpr int kQG = 4;  // queries per workgroup
constexpr int kU = 4;   // wave steps per batch

__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2, float l2,
                                            const float* acc2, int n) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;
  const float f1 = __expf(m - mn), f2 = __expf(m2 - mn);
  l = l * f1 + l2 * f2;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * f1 + acc2[i] * f2;
  m = mn;
}

template <typename T, int D>
__global__ __launch_bounds__(kAttThreads) void k_attend(AttendArgs A) {
  constexpr int E = Elem<T>::per16;
  constexpr int LPK = D / E;   // lanes per key row
  constexpr int KPS = 64 / LPK;  // keys per wave step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = lane / LPK, pc = lane % LPK;
  const int cache = blockIdx.y, grp = blockIdx.z;
  const int64_t tile = blockIdx.x;
  const int b = cache / A.H, h = cache % A.H;
  const int64_t k_lo = tile * A.tile_keys;
  const int64_t k_hi = min(A.n_tokens, k_lo + A.tile_keys);
  const int64_t per_wave = A.tile_keys / 4;
  const int64_t w_lo = k_lo + wave * per_wave;
  const int64_t w_hi = min(k_hi, w_lo + per_wave);
  const bool all = A.flags & 4u, sink = A.flags & 1u, last = A.flags & 2u;
  const int64_t last_start = (int64_t)A.C * ((A.n_tokens - 1) / A.C);

  float qv[kQG][E];
  const uint32_t* srow[kQG];
  bool qok[kQG];
#pragma unroll
  for (int u = 0; u < kQG; ++u) {
    const int qi = grp * kQG + u;
    qok[u] = qi < A.QC;
    const int qs = qok[u] ? qi : 0;
    const int gq = qs / A.T, t = qs % A.T;
    const T* qp = reinterpret_cast<const T*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                  (int64_t)gq * A.qsg + (int64_t)t * A.qst;
    unpack(ld16(qp + pc * E), qv[u], T());
    srow[u] = A.sel1 ? A.sel1 + ((int64_t)cache * A.QC + qs) * A.sel_words : nullptr;
  }
  const T* Kc = reinterpret_cast<const T*>(A.K) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  const T* Vc = reinterpret_cast<const T*>(A.V) + (int64_t)b * A.sb + (int64_t)h * A.sh;

  float m[kQG], l[kQG], acc[kQG][E];
#pragma unroll
  for (int u = 0; u < kQG; ++u) {
    m[u] = kNegInf;
    l[u] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[u][e] = 0.f;
  }

  for (int64_t k0 = w_lo; k0 < w_hi; k0 += KPS * kU) {
    bool sel[kU][kQG];
    bool lsel[kU];
    bool anysel = false;
#pragma unroll
    for (int x = 0; x < kU; ++x) {
      const int64_t key = k0 + x * KPS + kk;
      const bool valid = key < w_hi;
      const int64_t chunk = key / A.C;
      lsel[x] = false;
#pragma unroll
      for (int u = 0; u < kQG; ++u) {
        bool s = valid && qok[u];
        if (s && !all) {
          bool forced = (sink && key == 0) || (last && key >= last_start);
          bool bit = chunk < A.n_chunks && ((srow[u][chunk >> 5] >> (chunk & 31)) & 1u);
          s = forced || bit;
        }
        sel[x][u] = s;
        lsel[x] = lsel[x] || s;
      }
      anysel = anysel || lsel[x];
    }
    if (!__any(anysel)) continue;
    uint4 kr[kU], vr[kU];
#pragma unroll
    for (int x = 0; x < kU; ++x) {
      const int64_t key = k0 + x * KPS + kk;
      if (lsel[x]) {
        kr[x] = ld16(Kc + key * A.st + pc * E);
        vr[x] = ld16(Vc + key * A.st + pc * E);
      } else {
        kr[x] = make_uint4(0, 0, 0, 0);
        vr[x] = make_uint4(0, 0, 0, 0);
      }
    }
    float z[kU][kQG];
#pragma unroll
    for (int x = 0; x < kU; ++x) {
      float kf[E];
      unpack(kr[x], kf, T());
#pragma unroll
      for (int u = 0; u < kQG; ++u) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) part += kf[e] * qv[u][e];
        part = wave_sum_xor(part, 1, LPK);
        z[x][u] = sel[x][u] ? part * A.inv_sqrt_d : kNegInf;
      }
    }
#pragma unroll
    for (int u = 0; u < kQG; ++u) {
      float mn = m[u];
#pragma unroll
      for (int x = 0; x < kU; ++x) mn = fmaxf(mn, z[x][u]);
      if (mn == kNegInf) continue;
      const float f = __expf(m[u] - mn);
      l[u] *= f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[u][e] *= f;
#pragma unroll
      for (int x = 0; x < kU; ++x) {
        const float pz = __expf(z[x][u] - mn);
        float vf[E];
        unpack(vr[x], vf, T());
        l[u] += pz;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[u][e] += pz * vf[e];
      }
      m[u] = mn;
    }
  }

  // merge the key slots of the wave (lanes kk = 0.. share piece pc)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int u = 0; u < kQG; ++u) {
      const float m2 = __shfl_xor(m[u], off), l2 = __shfl_xor(l[u], off);
      float a2[E];
#pragma unroll
      for (int e = 0; e < E; ++e) a2[e] = __shfl_xor(acc[u][e], off);
      merge_state(m[u], l[u], acc[u], m2, l2, a2, E);
    }
  }
  // merge the 4 waves
  __shared__ float red[4][kQG][D + 2];
  if (kk == 0) {
#pragma unroll
    for (int u = 0; u < kQG; ++u) {
#pragma unroll
      for (int e = 0; e < E; ++e) red[wave][u][pc * E + e] = acc[u][e];
      if (pc == 0) {
        red[wave][u][D] = m[u];
        red[wave][u][D + 1] = l[u];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kQG * D; idx += kAttThreads) {
    const int u = idx / D, d = idx % D;
    const int qi = grp * kQG + u;
    if (qi >= A.QC) continue;
    float mm = kNegInf;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][u][D]);
    float ll = 0.f, o = 0.f;
    if (mm != kNegInf) {
      for (int w = 0; w < 4; ++w) {
        const float mw = red[w][u][D];
        if (mw == kNegInf) continue;
        const float f = __expf(mw - mm);
        ll += red[w][u][D + 1] * f;
        o += red[w][u][d] * f;
      }
    }
    float* part = A.partial + (((int64_t)cache * A.QC + qi) * A.n_tiles + tile) * (D + 2);
    if (d == 0) {
      part[0] = mm;
      part[1] = ll;
    }
    part[2 + d] = o;
  }
}

constexpr int kTileQuadsMax = 2048;                // 8192 keys
constexpr int kQPT = kTileQuadsMax / kAttThreads;  // quads per thread in phase 1 (32 keys)

// Phase 1 of the bf16 kernels.  Thread `tid` covers the 8 quads (32 keys)
// starting at k_lo + 32 tid.  Bit 4u + kk of qmask[i] marks key kk of quad i
// as attended by query u of the group (a routed chunk or a forced key); bit i
// of *routed marks quads that hold a routed chunk of some query.  The 32 keys
// start on a multiple of 32 and C is a power of two, so the bits of their
// chunks lie in one selection word per query: one load per query.
template <int QG>
__device__ __forceinline__ void quad_masks(const AttendArgs& A, int cache, int qg0, int nq, int64_t k_lo,
                                           int64_t k_hi, int tid, unsigned long long* qmask,
                                           uint32_t* routed) {
  const bool all = A.flags & 4u, sink = A.flags & 1u, last = A.flags & 2u;
  const int64_t last_start = (int64_t)A.C * ((A.n_tokens - 1) / A.C);
  const int64_t key0 = k_lo + 32 * (int64_t)tid;
  const int lc = __builtin_ctz((unsigned)A.C);
  const int64_t c0 = key0 >> lc;
  const bool rd = !all && A.sel1 != nullptr && key0 < k_hi && c0 < A.n_chunks;
  const uint32_t* wp = A.sel1 + ((int64_t)cache * A.QC + qg0) * A.sel_words + (c0 >> 5);
  uint32_t wq[QG];
#pragma unroll
  for (int u = 0; u < QG; ++u) wq[u] = (rd && u < nq) ? wp[(int64_t)u * A.sel_words] : 0u;
  const int sh = (int)(c0 & 31);
  const uint32_t qall = (1u << nq) - 1u;  // nq <= 16
  // prefill (causal): query u sits at position pos[u], sees keys <= pos[u]
  // and its own current chunk [C floor(pos[u] / C), pos[u]]
  const bool causal = A.causal_n0 >= 0;
  int64_t pos[QG];
#pragma unroll
  for (int u = 0; u < QG; ++u) pos[u] = causal ? A.causal_n0 + (qg0 + (u < nq ? u : 0)) % A.T : A.n_tokens - 1;
  uint32_t rt = 0u;
#pragma unroll
  for (int i = 0; i < kQPT; ++i) {
    unsigned long long msk = 0ull;
    uint32_t qany = 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int64_t key = key0 + 4 * i + kk;
      const bool in = key < k_hi;
      const int j = (4 * i + kk) >> lc;  // chunk of this key, counted from c0
      uint32_t qb = 0u;                  // bit u: query u routes this key's chunk
#pragma unroll
      for (int u = 0; u < QG; ++u) qb |= ((wq[u] >> (sh + j)) & 1u) << u;
      if (!in || c0 + j >= A.n_chunks) qb = 0u;
      uint32_t qs;
      if (!causal) {
        const bool forced = in && (all || (sink && key == 0) || (last && key >= last_start));
        qs = forced ? qall : qb;
      } else {
        uint32_t vis = 0u, fq = 0u;
#pragma unroll
        for (int u = 0; u < QG; ++u) {
          const bool v = in && u < nq && key <= pos[u];
          vis |= (uint32_t)v << u;
          fq |= (uint32_t)(v && (all || (sink && key == 0) || (last && key >= (int64_t)A.C * (pos[u] / A.C)))) << u;
        }
        qb &= vis;
        qs = fq | qb;
      }
      qany |= qb;
#pragma unroll
      for (int u = 0; u < QG; ++u) msk |= (unsigned long long)((qs >> u) & 1u) << (4 * u + kk);
    }
    qmask[i] = msk;
    if (qany) rt |= 1u << i;
  }
  *routed = rt;
}

// Exclusive scan of `cnt` over the workgroup (256 threads); returns the total.
__device__ __forceinline__ int block_scan_excl(int cnt, int* scan, int* excl) {
  const int tid = threadIdx.x;
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kAttThreads; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  *excl = scan[tid] - cnt;
  return scan[kAttThreads - 1];
}

// Level-1 bitsets to sorted chunk id lists: one workgroup per query walks
// its row in segments of kAttThreads x kIdWords words; each thread counts
// the set bits of its words, an exclusive scan over the workgroup gives each
// thread its first output position, and the ids are written in bit order.
constexpr int kIdWords = 4;
__global__ __launch_bounds__(kAttThreads) void k_selected_chunks(const uint32_t* __restrict__ sel1, int64_t words,
                                                                int64_t n_chunks, int32_t* __restrict__ ids,
                                                                int32_t* __restrict__ count, int64_t cap) {
  __shared__ int scan[kAttThreads];
  const int64_t q = blockIdx.x;
  const uint32_t* row = sel1 + q * words;
  int32_t* out = ids + q * cap;
  const int64_t nw = (n_chunks + 31) / 32;  // words the chunks reach
  int64_t base = 0;
  for (int64_t w0 = 0; w0 < nw; w0 += (int64_t)kAttThreads * kIdWords) {
    uint32_t bits[kIdWords];
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kIdWords; ++k) {
      const int64_t w = w0 + (int64_t)threadIdx.x * kIdWords + k;
      uint32_t b = w < nw ? row[w] : 0u;
      const int64_t lo = w * 32;
      if (lo + 32 > n_chunks) b &= lo >= n_chunks ? 0u : ((1u << (n_chunks - lo)) - 1u);  // bits past n_chunks
      bits[k] = b;
      cnt += __popc(b);
    }
    int excl;
    const int tot = block_scan_excl(cnt, scan, &excl);
    int64_t pos = base + excl;
#pragma unroll
    for (int k = 0; k < kIdWords; ++k) {
      const int64_t w = w0 + (int64_t)threadIdx.x * kIdWords + k;
      uint32_t b = bits[k];
      while (b) {
        const int bit = __ffs(b) - 1;
        b &= b - 1u;
        if (pos < cap) out[pos] = (int32_t)(w * 32 + bit);
        ++pos;
      }
    }
    base += tot;
    __syncthreads();  // scan[] is reused by the next segment
  }
  if (threadIdx.x == 0) count[q] = (int32_t)base;
}

constexpr int kMaxForcedQuads = 16;

// Phase 1 of the bf16 kernels, compaction: the tile's quads with a key some
// query of the group attends, in LDS as (quad index, 4-bit key mask per
// query).  SPLIT puts the quads holding a routed chunk first (*n_r of them)
// and the forced-only quads (sink, current chunk) after them, at most
// kMaxForcedQuads; otherwise all quads are in key order and *n_r = *n_ent.
template <int QG, bool SPLIT>
__device__ __forceinline__ void collect_quads(const AttendArgs& A, int cache, int qg0, int nq, int64_t k_lo,
                                              int64_t k_hi, uint16_t* e_quad, unsigned long long* e_mask,
                                              int* scan, int* n_r, int* n_ent) {
  const int tid = threadIdx.x;
  unsigned long long qmask[kQPT];
  uint32_t routed;
  quad_masks<QG>(A, cache, qg0, nq, k_lo, k_hi, tid, qmask, &routed);
  if constexpr (SPLIT) {
    int cnt = 0;  // routed count in the low 16 bits, forced-only count above
#pragma unroll
    for (int i = 0; i < kQPT; ++i)
      if (qmask[i]) cnt += ((routed >> i) & 1u) ? 1 : (1 << 16);
    int excl;
    const int tot = block_scan_excl(cnt, scan, &excl);
    *n_r = tot & 0xffff;
    *n_ent = *n_r + min(tot >> 16, kMaxForcedQuads);
    int pos_r = excl & 0xffff, pos_f = *n_r + (excl >> 16);
#pragma unroll
    for (int i = 0; i < kQPT; ++i) {
      if (qmask[i]) {
        const int pos = ((routed >> i) & 1u) ? pos_r++ : pos_f++;
        if (pos < *n_ent) {
          e_quad[pos] = (uint16_t)(tid * kQPT + i);
          e_mask[pos] = qmask[i];
        }
      }
    }
  } else {
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kQPT; ++i) cnt += qmask[i] != 0ull;
    int pos;
    *n_ent = block_scan_excl(cnt, scan, &pos);
    *n_r = *n_ent;
#pragma unroll
    for (int i = 0; i < kQPT; ++i) {
      if (qmask[i]) {
        e_quad[pos] = (uint16_t)(tid * kQPT + i);
        e_mask[pos] = qmask[i];
        ++pos;
      }
    }
  }
}

// Phase 1b: logits of the n_f forced-only quads (entries n_r ..), one thread
// per key and query, into f_log[f][query][key].
template <int D, int QG>
__device__ __forceinline__ void forced_logits(const AttendArgs& A, const bf16_t* Kc, int b, int h, int qg0, int nq,
                                              int64_t k_lo, int64_t k_hi, const uint16_t* e_quad, int n_r, int n_f,
                                              float (*f_log)[QG][4]) {
  constexpr int PIECES = D / 8;
  for (int idx = threadIdx.x; idx < n_f * 4 * QG; idx += kAttThreads) {
    const int f = idx / (4 * QG), kk = (idx / QG) % 4, u = idx % QG;
    const int64_t key = k_lo + 4 * (int64_t)e_quad[n_r + f] + kk;
    float z = kNegInf;
    if (u < nq && key < k_hi) {
      const int qi = qg0 + u;
      const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                         (int64_t)(qi / A.T) * A.qsg + (int64_t)(qi % A.T) * A.qst;
      const bf16_t* kp = Kc + key * A.st;
      float dot = 0.f;
#pragma unroll
      for (int pc = 0; pc < PIECES; ++pc) {
        float kv[8], qv[8];
        unpack(ld16(kp + pc * 8), kv, bf16_t());
        unpack(ld16(qp + pc * 8), qv, bf16_t());
#pragma unroll
        for (int x = 0; x < 8; ++x) dot += kv[x] * qv[x];
      }
      z = dot * A.inv_sqrt_d;
    }
    f_log[f][u][kk] = z;
  }
}



// Combines the 4 waves' (max, sum, weighted V sum) per query and writes the
// workgroup's partial result for the tile.
template <int D, int QG>
__device__ __forceinline__ void write_partial(const AttendArgs& A, float (*red)[QG][D + 2], int cache, int qg0,
                                              int nq, int64_t tile) {
  for (int idx = threadIdx.x; idx < QG * D; idx += kAttThreads) {
    const int u = idx / D, d = idx % D;
    if (u >= nq) continue;
    float mm = kNegInf;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][u][D]);
    float ll = 0.f, o = 0.f;
    if (mm != kNegInf) {
      for (int w = 0; w < 4; ++w) {
        const float mw = red[w][u][D];
        if (mw == kNegInf) continue;
        const float f = __expf(mw - mm);
        ll += red[w][u][D + 1] * f;
        o += red[w][u][d] * f;
      }
    }
    float* part = A.partial + (((int64_t)cache * A.QC + qg0 + u) * A.n_tiles + tile) * (D + 2);
    if (d == 0) {
      part[0] = mm;
      part[1] = ll;
    }
    part[2 + d] = o;
  }
}

// One batch of T steps of the streaming kernel for this lane's key: rescale
// the running state once to the batch max, then accumulate exp(z - max) * v.
template <int T, int QG>
__device__ __forceinline__ void absorb(const uint4 (&vv4)[T], const float (&z)[T][QG], float (&m)[QG],
                                       float (&lsum)[QG], float (&acc)[QG][8]) {
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    float bm = z[0][u];
#pragma unroll
    for (int t = 1; t < T; ++t) bm = fmaxf(bm, z[t][u]);
    const float mn = fmaxf(m[u], bm);
    if (mn > m[u]) {
      const float sc = __expf(m[u] - mn);
      lsum[u] *= sc;
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[u][x] *= sc;
      m[u] = mn;
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float vv[8];
    unpack(vv4[t], vv, bf16_t());
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const float pw = z[t][u] == kNegInf ? 0.f : __expf(z[t][u] - m[u]);
      lsum[u] += pw;
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[u][x] += pw * vv[x];
    }
  }
}

// bf16 path without cached logits: compacted quads, QK^T on MFMA, PV in fp32
// FMA.  The non-empty quads are compacted, in key order, into an LDS list
// with a 4-bit key mask per query.  Each wave takes groups of four list
// entries (16 keys); K rows go straight into the A operand of
// v_mfma_f32_16x16x32_bf16 (queries are the B operand), so one MFMA chain
// yields the 16 x 16 logits.  The softmax weights leave the MFMA layout
// through a 1 KiB LDS slot per wave and meet V, which is loaded with fully
// coalesced 16-byte rows and accumulated in fp32.  The next group's K and V
// are in flight while the current one is computed.
template <int D, int QG>
__global__ __launch_bounds__(kAttThreads) void k_attend_mfma(AttendArgs A) {
  constexpr int PIECES = D / 8;    // 16-byte pieces per row
  constexpr int NS = D / 32;       // MFMA k-steps
  constexpr int NVL = PIECES / 4;  // V loads per lane per 16-key group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qg0 = blockIdx.z * QG;
  const int nq = min(QG, A.QC - qg0);
  const int64_t tile = blockIdx.x;
  const int b = cache / A.H, h = cache % A.H;
  const int64_t k_lo = tile * A.tile_keys;
  const int64_t k_hi = min(A.n_tokens, k_lo + A.tile_keys);

  __shared__ uint16_t e_quad[kTileQuadsMax];
  __shared__ unsigned long long e_mask[kTileQuadsMax];
  __shared__ int scan[kAttThreads];
  __shared__ float p_lds[4][16][16];  // [wave][key in group][query]
  __shared__ float sc_lds[4][16];
  __shared__ float red[4][QG][D + 2];

  // ---- phase 1
  int n_r, n_ent;
  collect_quads<QG, false>(A, cache, qg0, nq, k_lo, k_hi, e_quad, e_mask, scan, &n_r, &n_ent);
  __syncthreads();

  // ---- phase 2
  const int r16 = lane & 15, kg = lane >> 4;
  bf16x8 bq[NS];
  {
    const int qi = qg0 + r16;
    if (r16 < nq) {
      const int gq = qi / A.T, t = qi % A.T;
      const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                         (int64_t)gq * A.qsg + (int64_t)t * A.qst;
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const bf16_t* Kc = reinterpret_cast<const bf16_t*>(A.K) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  const bf16_t* Vc = reinterpret_cast<const bf16_t*>(A.V) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  // this tile's rows; offsets past the last key read zeros
  const uint32_t tile_bytes = (uint32_t)((k_hi - k_lo - 1) * A.st * 2 + D * 2);
  const rsrc_t kr = make_rsrc(Kc + k_lo * A.st, tile_bytes);
  const rsrc_t vr = make_rsrc(Vc + k_lo * A.st, tile_bytes);
  const uint32_t row_bytes = (uint32_t)(A.st * 2);

  const int n_groups = (n_ent + 3) / 4;
  // Loads of one 16-key group into KA (K rows, A operand) and VA (V rows,
  // FMA layout).
#define ZHA_LOAD_GROUP(g, KA, VA)                                                                 \
  do {                                                                                            \
    {                                                                                             \
      const int e_ = 4 * (g) + (r16 >> 2);                                                        \
      const uint32_t ro_ = e_ < n_ent ? (4u * e_quad[e_] + (r16 & 3)) * row_bytes : kOffNone;     \
      _Pragma("unroll") for (int s_ = 0; s_ < NS; ++s_) KA[s_] = bld16<0>(kr, ro_ + (4 * s_ + kg) * 16); \
    }                                                                                             \
    _Pragma("unroll") for (int u_ = 0; u_ < NVL; ++u_) {                                          \
      const int pi_ = lane + 64 * u_;                                                             \
      const int kq_ = pi_ / PIECES, pc_ = pi_ % PIECES;                                           \
      const int e_ = 4 * (g) + (kq_ >> 2);                                                        \
      const uint32_t ro_ = e_ < n_ent ? (4u * e_quad[e_] + (kq_ & 3)) * row_bytes : kOffNone;     \
      VA[u_] = bld16(vr, ro_ + pc_ * 16);                                                         \
    }                                                                                             \
  } while (0)

  float m = kNegInf, l = 0.f;  // softmax state of query r16 (MFMA layout)
  float acc[QG][8];            // V accumulators of piece (lane % PIECES) (FMA layout)
#pragma unroll
  for (int u = 0; u < QG; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;

  // each wave walks its own groups (g = wave, wave + 4, ...); the LDS slots
  // it exchanges through are its own, so only wave-scope barriers are needed
  uint4 kf[NS], vf[NVL], kn[NS], vn[NVL];
  if (wave < n_groups) ZHA_LOAD_GROUP(wave, kf, vf);
  for (int g = wave; g < n_groups; g += 4) {
    if (g + 4 < n_groups) ZHA_LOAD_GROUP(g + 4, kn, vn);
    {
      // lane: keys 4*kg + i of the group (entry 4g + kg), query r16
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[s]), bq[s], z, 0, 0, 0);
      const int e = 4 * g + kg;
      const unsigned long long msk = (e < n_ent && r16 < QG) ? e_mask[e] >> (r16 * 4) : 0ull;
      float zz[4];
      float mb = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zz[i] = ((msk >> i) & 1ull) ? z[i] * A.inv_sqrt_d : kNegInf;
        mb = fmaxf(mb, zz[i]);
      }
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float mn = fmaxf(m, mb);
      float sc = 1.f, ps = 0.f;
      float pz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pz[i] = 0.f;
      if (mn != kNegInf) {
        sc = __expf(m - mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pz[i] = __expf(zz[i] - mn);
          ps += pz[i];
        }
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l = l * sc + ps;
      m = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) p_lds[wave][4 * kg + i][r16] = pz[i];
      if (kg == 0) sc_lds[wave][r16] = sc;
    }
    wave_sync();
    {
      float scq[QG];
#pragma unroll
      for (int u = 0; u < QG; ++u) scq[u] = sc_lds[wave][u];
#pragma unroll
      for (int u = 0; u < QG; ++u)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[u][x] *= scq[u];
#pragma unroll
      for (int v = 0; v < NVL; ++v) {
        const int kq = (lane + 64 * v) / PIECES;
        float vv[8];
        unpack(vf[v], vv, bf16_t());
#pragma unroll
        for (int u = 0; u < QG; ++u) {
          const float pw = p_lds[wave][kq][u];
#pragma unroll
          for (int x = 0; x < 8; ++x) acc[u][x] += pw * vv[x];
        }
      }
    }
    wave_sync();
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = kn[s];
#pragma unroll
    for (int v = 0; v < NVL; ++v) vf[v] = vn[v];
  }
#undef ZHA_LOAD_GROUP

  // lanes sharing a piece hold partial V sums of different keys: add them
#pragma unroll
  for (int off = PIECES; off < 64; off <<= 1)
#pragma unroll
    for (int u = 0; u < QG; ++u)
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[u][x] += __shfl_xor(acc[u][x], off);
  if (lane < PIECES) {
#pragma unroll
    for (int u = 0; u < QG; ++u)
#pragma unroll
      for (int x = 0; x < 8; ++x) red[wave][u][lane * 8 + x] = acc[u][x];
  }
  if (kg == 0 && r16 < QG) {
    red[wave][r16][D] = m;
    red[wave][r16][D + 1] = l;
  }
  __syncthreads();
  write_partial<D, QG>(A, red, cache, qg0, nq, tile);
}

// bf16 path with the route's cached level-1 logits: V streaming only.
//
// Phase 1 compacts the selected quads as above, routed quads first, then the
// few quads that hold forced keys only (the sink's quad and the current
// chunk, which lies inside one tile: at most 5 quads; in a prefill block the
// group's queries have up to 3 current chunks, at most 13 quads); the logits
// of those few are computed once into LDS.  Phase 2: lanes are (quad of the step, key of the quad,
// 16-byte piece of the row); each wave takes every 4th step, with 4 steps of
// V (one coalesced 1 KiB load per quad for d = 128) and their cached logits
// in flight at once, and keeps a per-lane online softmax (one rescale per
// batch) in fp32.  No LDS traffic or barrier in the loop.  Groups of 16
// queries go to k_attend_pv16 instead.
template <int D, int QG>
__global__ __launch_bounds__(kAttThreads) __attribute__((amdgpu_waves_per_eu(QG <= 4 ? 5 : 1))) void k_attend_cached(AttendArgs A) {
  constexpr int PIECES = D / 8;   // 16-byte pieces per row
  constexpr int LPQ = 4 * PIECES; // lanes per quad
  constexpr int EPS = 64 / LPQ;   // quads per wave step
  // wave steps in flight: 4 leaves registers for more waves per SIMD, which
  // hides the gathers better than deeper prefetch per wave (8 steps ran the
  // 1M-token decode about 10% slower)
  constexpr int U = QG <= 8 ? 4 : 2;
  constexpr int STRIDE = 4 * EPS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qg0 = blockIdx.z * QG;
  const int nq = min(QG, A.QC - qg0);
  const int64_t tile = blockIdx.x;
  const int b = cache / A.H, h = cache % A.H;
  const int64_t k_lo = tile * A.tile_keys;
  const int64_t k_hi = min(A.n_tokens, k_lo + A.tile_keys);

  __shared__ uint16_t e_quad[kTileQuadsMax];
  __shared__ unsigned long long e_mask[kTileQuadsMax];
  __shared__ int scan[kAttThreads];
  __shared__ float f_log[kMaxForcedQuads][QG][4];
  __shared__ float red[4][QG][D + 2];

  // ---- phase 1: routed quads first, then the forced-only ones
  int n_r, n_ent;
  collect_quads<QG, true>(A, cache, qg0, nq, k_lo, k_hi, e_quad, e_mask, scan, &n_r, &n_ent);
  const int n_f = n_ent - n_r;
  __syncthreads();

  const bf16_t* Kc = reinterpret_cast<const bf16_t*>(A.K) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  const bf16_t* Vc = reinterpret_cast<const bf16_t*>(A.V) + (int64_t)b * A.sb + (int64_t)h * A.sh;

  // ---- phase 1b: logits of the forced-only quads
  if (n_f) {
    forced_logits<D, QG>(A, Kc, b, h, qg0, nq, k_lo, k_hi, e_quad, n_r, n_f, f_log);
    __syncthreads();
  }

  // ---- phase 2
  const int qs = lane / LPQ, kk = (lane % LPQ) / PIECES, pc = lane % PIECES;
  const uint32_t row_bytes = (uint32_t)(A.st * 2);
  const rsrc_t vr = make_rsrc(Vc + k_lo * A.st, (uint32_t)((k_hi - k_lo - 1) * A.st * 2 + D * 2));
  // this tile's cached logits: [quad][QW][4] fp32
  const int nqt = (int)((k_hi - k_lo + 3) / 4);
  const float* ltile = A.logits + (((int64_t)cache * ((A.QC + 15) / 16) + qg0 / 16) * A.nquads + (k_lo >> 2)) * A.QW * 4;
  const rsrc_t lr = make_rsrc(ltile, (uint32_t)(nqt * A.QW * 16));
  // byte offset of (key kk, query 0 of the group) within a quad's row; the
  // group's QG queries are contiguous there (QG <= QW, qg0 % 16 + QG <= QW)
  const uint32_t lq = (uint32_t)(kk * A.QW + qg0 % 16) * 4;
  float m[QG], lsum[QG], acc[QG][8];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    m[u] = kNegInf;
    lsum[u] = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[u][x] = 0.f;
  }
  // routed quads: V and cached logits by buffer loads (unselected read nothing)
  for (int e0 = wave * EPS + qs; e0 < n_r; e0 += STRIDE * U) {
    uint4 vv4[U];
    float z[U][QG];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int e = e0 + t * STRIDE;
      const bool ok = e < n_r;
      const uint32_t quad = ok ? e_quad[e] : 0u;
      const unsigned long long msk = ok ? e_mask[e] >> kk : 0ull;
      vv4[t] = bld16(vr, ok ? (4u * quad + kk) * row_bytes + pc * 16 : kOffNone);
      // the logits of key kk for the group's queries, 4 per 16-byte load
#pragma unroll
      for (int v = 0; v < QG / 4; ++v) {
        const uint4 lz = bld16<0>(lr, ok ? quad * (uint32_t)A.QW * 16 + lq + v * 16 : kOffNone);
        const float l4[4] = {__uint_as_float(lz.x), __uint_as_float(lz.y), __uint_as_float(lz.z), __uint_as_float(lz.w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) z[t][4 * v + i] = ((msk >> (4 * (4 * v + i))) & 1ull) ? l4[i] : kNegInf;
      }
    }
    absorb<U, QG>(vv4, z, m, lsum, acc);
  }
  // forced-only quads: logits from LDS
  for (int f0 = wave * EPS + qs; f0 < n_f; f0 += STRIDE) {
    uint4 vv4[1];
    float z[1][QG];
    const uint32_t quad = e_quad[n_r + f0];
    const unsigned long long msk = e_mask[n_r + f0] >> kk;
    vv4[0] = bld16(vr, (4u * quad + kk) * row_bytes + pc * 16);
#pragma unroll
    for (int u = 0; u < QG; ++u) z[0][u] = ((msk >> (4 * u)) & 1ull) ? f_log[f0][u][kk] : kNegInf;
    absorb<1, QG>(vv4, z, m, lsum, acc);
  }

  // merge the lanes that share a piece (different keys): common max, then sums
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const float mw = wave_max_xor(m[u], PIECES, 64);
    const float f = mw == kNegInf ? 0.f : __expf(m[u] - mw);
    lsum[u] *= f;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[u][x] *= f;
    m[u] = mw;
  }
#pragma unroll
  for (int off = PIECES; off < 64; off <<= 1)
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      lsum[u] += __shfl_xor(lsum[u], off);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[u][x] += __shfl_xor(acc[u][x], off);
    }
  if (lane < PIECES) {
#pragma unroll
    for (int u = 0; u < QG; ++u)
#pragma unroll
      for (int x = 0; x < 8; ++x) red[wave][u][lane * 8 + x] = acc[u][x];
  }
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      red[wave][u][D] = m[u];
      red[wave][u][D + 1] = lsum[u];
    }
  }
  __syncthreads();
  write_partial<D, QG>(A, red, cache, qg0, nq, tile);
}

// Groups of 16 queries (QC > 8): the P V product on the matrix cores.  The
// q.k MFMA (or the cached logits) leaves in lane (query r, key group g) the
// logits of keys 4g .. 4g+3 of a 16-key group for query r, which is the A
// operand layout of v_mfma_f32_16x16x16_bf16 for P (rows = queries, k =
// keys); the group's V rows are staged in LDS and read as the B operand
// (k = keys, columns = 16 values of d).  P is split into three bf16 terms
// (hi + mid + lo, exact to about 2^-26 relative), so the product keeps fp32
// accuracy.  The output rows (4 queries x 16 values of d per lane and block)
// are rescaled per query when the running max moves, as in the FMA kernels.
// Phase 1 is the one of k_attend_cached (CACHED: routed quads read the
// route's logits, forced-only quads get theirs computed once) or of
// k_attend_mfma (logits from K on the fly).
typedef short short4v __attribute__((ext_vector_type(4)));

template <int D, bool CACHED>
__global__ __launch_bounds__(kAttThreads) void k_attend_pv16(AttendArgs A) {
  constexpr int QG = 16;
  constexpr int PIECES = D / 8;     // 16-byte pieces per row
  constexpr int NS = D / 32;        // q.k MFMA k-steps
  constexpr int NVL = PIECES / 4;   // V loads per lane per 16-key group
  constexpr int NB = D / 16;        // output blocks of 16 values of d
  constexpr int VROW = D + 8;       // padded LDS V row (bf16 elements)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cache = blockIdx.y;
  const int qg0 = blockIdx.z * QG;
  const int nq = min(QG, A.QC - qg0);
  const int64_t tile = blockIdx.x;
  const int b = cache / A.H, h = cache % A.H;
  const int64_t k_lo = tile * A.tile_keys;
  const int64_t k_hi = min(A.n_tokens, k_lo + A.tile_keys);

  __shared__ uint16_t e_quad[kTileQuadsMax];
  __shared__ unsigned long long e_mask[kTileQuadsMax];
  __shared__ int scan[kAttThreads];
  __shared__ float f_log[CACHED ? kMaxForcedQuads : 1][QG][4];
  __shared__ uint16_t vs[4][16 * VROW];
  __shared__ float red[4][QG][D + 2];

  // ---- phase 1: the tile's quads with a key some query attends, routed
  // quads first (CACHED) or in key order
  int n_r, n_ent;
  collect_quads<QG, CACHED>(A, cache, qg0, nq, k_lo, k_hi, e_quad, e_mask, scan, &n_r, &n_ent);
  __syncthreads();

  const bf16_t* Kc = reinterpret_cast<const bf16_t*>(A.K) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  const bf16_t* Vc = reinterpret_cast<const bf16_t*>(A.V) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  const int n_f = n_ent - n_r;
  if (CACHED && n_f) {
    forced_logits<D, QG>(A, Kc, b, h, qg0, nq, k_lo, k_hi, e_quad, n_r, n_f, f_log);
    __syncthreads();
  }

  // ---- phase 2
  const int r16 = lane & 15, kg = lane >> 4;
  bf16x8 bq[CACHED ? 1 : NS];
  if constexpr (!CACHED) {
    const int qi = qg0 + r16;
    if (r16 < nq) {
      const bf16_t* qp = reinterpret_cast<const bf16_t*>(A.Q) + (int64_t)b * A.qsb + (int64_t)h * A.qsh +
                         (int64_t)(qi / A.T) * A.qsg + (int64_t)(qi % A.T) * A.qst;
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(ld16(qp + (4 * s + kg) * 8));
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const uint32_t tile_bytes = (uint32_t)((k_hi - k_lo - 1) * A.st * 2 + D * 2);
  const rsrc_t kr = make_rsrc(Kc + k_lo * A.st, tile_bytes);
  const rsrc_t vr = make_rsrc(Vc + k_lo * A.st, tile_bytes);
  const uint32_t row_bytes = (uint32_t)(A.st * 2);
  // the route's logits of this tile and group: [quad][key][QW], queries
  // qg0 .. qg0 + 15 are a whole row block (qg0 % 16 == 0)
  const float* ltile = CACHED ? A.logits + (((int64_t)cache * ((A.QC + 15) / 16) + qg0 / 16) * A.nquads + (k_lo >> 2)) *
                                               A.QW * 4
                              : nullptr;

  const int n_groups = (n_ent + 3) / 4;
  auto load_group = [&](int g, uint4* KA, uint4* VA) {
    if constexpr (!CACHED) {
      const int e = 4 * g + (r16 >> 2);
      const uint32_t ro = e < n_ent ? (4u * e_quad[e] + (r16 & 3)) * row_bytes : kOffNone;
#pragma unroll
      for (int s = 0; s < NS; ++s) KA[s] = bld16<0>(kr, ro + (4 * s + kg) * 16);
    }
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int pi = lane + 64 * u;
      const int kq = pi / PIECES, pc = pi % PIECES;
      const int e = 4 * g + (kq >> 2);
      const uint32_t ro = e < n_ent ? (4u * e_quad[e] + (kq & 3)) * row_bytes : kOffNone;
      VA[u] = bld16(vr, ro + pc * 16);
    }
  };

  float m = kNegInf, l = 0.f;  // softmax state of query r16 (same in its 4 lanes)
  f32x4 O[NB];                 // rows 4 kg + i (queries), column 16 blk + r16 (d)
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) O[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 kf[CACHED ? 1 : NS], kn[CACHED ? 1 : NS], vf[NVL], vn[NVL];
  if (wave < n_groups) load_group(wave, kf, vf);
  for (int g = wave; g < n_groups; g += 4) {
    if (g + 4 < n_groups) load_group(g + 4, kn, vn);
    // logits of query r16 for the 4 keys of entry e
    const int e = 4 * g + kg;
    const unsigned long long msk = (e < n_ent && r16 < nq) ? e_mask[e] >> (4 * r16) : 0ull;
    float zz[4];
    if constexpr (CACHED) {
      if (e < n_r && r16 < nq) {
        const float* lz = ltile + (int64_t)e_quad[e] * 4 * A.QW + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[i] = lz[i * A.QW];
      } else if (e < n_ent && r16 < nq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[i] = f_log[e - n_r][r16][i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) zz[i] = kNegInf;
      }
    } else {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[s]), bq[s], z, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[i] = z[i] * A.inv_sqrt_d;
    }
    float mb = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!((msk >> i) & 1ull)) zz[i] = kNegInf;
      mb = fmaxf(mb, zz[i]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float mn = fmaxf(m, mb);
    float sc = 1.f, ps = 0.f, pz[4] = {0.f, 0.f, 0.f, 0.f};
    if (mn != kNegInf) {
      sc = __expf(m - mn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pz[i] = __expf(zz[i] - mn);
        ps += pz[i];
      }
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * sc + ps;
    m = mn;

    // the group's V rows into this wave's LDS slot
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int pi = lane + 64 * u;
      *reinterpret_cast<uint4*>(&vs[wave][(pi / PIECES) * VROW + (pi % PIECES) * 8]) = vf[u];
    }
    wave_sync();
    // rescale the output rows (query 4 kg + i: its factor is in lane 4 kg + i)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = __shfl(sc, 4 * kg + i);
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) O[blk][i] *= f;
    }
    // P = hi + mid + lo in bf16 (A operand: query r16, keys 4 kg + i)
    short4v ph, pm, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t bh = bf16_bits(pz[i]);
      const float r1 = pz[i] - __uint_as_float(bh << 16);
      const uint32_t bm = bf16_bits(r1);
      const float r2 = r1 - __uint_as_float(bm << 16);
      ph[i] = (short)bh;
      pm[i] = (short)bm;
      pl[i] = (short)bf16_bits(r2);
    }
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      // B operand: V[key 4 kg + i][d = 16 blk + r16]
      short4v vb;
#pragma unroll
      for (int i = 0; i < 4; ++i) vb[i] = (short)vs[wave][(4 * kg + i) * VROW + 16 * blk + r16];
      O[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, O[blk], 0, 0, 0);
      O[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pm, vb, O[blk], 0, 0, 0);
      O[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, O[blk], 0, 0, 0);
    }
    wave_sync();
    if constexpr (!CACHED) {
#pragma unroll
      for (int s = 0; s < NS; ++s) kf[s] = kn[s];
    }
#pragma unroll
    for (int u = 0; u < NVL; ++u) vf[u] = vn[u];
  }

  // this wave's (max, sum, weighted V sum) per query for the workgroup merge
#pragma unroll
  for (int blk = 0; blk < NB; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * kg + i][16 * blk + r16] = O[blk][i];
  if (kg == 0) {
    red[wave][r16][D] = m;
    red[wave][r16][D + 1] = l;
  }
  __syncthreads();
  write_partial<D, QG>(A, red, cache, qg0, nq, tile);
}

// Merges the per-tile partial results of one query: S slices of D threads,
// slice s folding tiles s, s + S, ... with a running max (two tiles in flight
// per step), then slice 0 merging the S slice states in slice order, so the
// result does not depend on timing.
template <int D, int S>
__global__ __launch_bounds__(D * S) void k_combine(AttendArgs A) {
  const int64_t q = blockIdx.x;
  const int d = threadIdx.x % D, sl = threadIdx.x / D;
  const int64_t nt = A.n_tiles;
  const float* base = A.partial + q * nt * (D + 2);
  float m = kNegInf, l = 0.f, o = 0.f;
  auto fold = [&](float mt, float lt, float ot) {
    if (mt == kNegInf) return;
    if (mt > m) {
      const float f = __expf(m - mt);  // 0 while m is -inf
      l = l * f + lt;
      o = o * f + ot;
      m = mt;
    } else {
      const float f = __expf(mt - m);
      l += f * lt;
      o += f * ot;
    }
  };
  int64_t t = sl;
  for (; t + S < nt; t += 2 * S) {
    const float* a = base + t * (D + 2);
    const float* b = a + S * (D + 2);
    const float ma = a[0], la = a[1], oa = a[2 + d];
    const float mb = b[0], lb = b[1], ob = b[2 + d];
    fold(ma, la, oa);
    fold(mb, lb, ob);
  }
  if (t < nt) {
    const float* a = base + t * (D + 2);
    fold(a[0], a[1], a[2 + d]);
  }
  __shared__ float sm[S], sls[S], so[S][D];
  if (d == 0) {
    sm[sl] = m;
    sls[sl] = l;
  }
  so[sl][d] = o;
  __syncthreads();
  if (sl != 0) return;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, sm[s]);
  float L = 0.f, O = 0.f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      if (sm[s] == kNegInf) continue;
      const float f = __expf(sm[s] - M);
      L += f * sls[s];
      O += f * so[s][d];
    }
  }
  A.out[q * D + d] = L > 0.f ? O / L : 0.f;
  if (d == 0 && A.lse) A.lse[q] = L > 0.f ? M + __logf(L) : kNegInf;
}

template <int D, int QG>
void launch_mfma(const AttendArgs& a, int n_caches, hipStream_t s) {
  dim3 grid((unsigned)a.n_tiles, (unsigned)n_caches, (unsigned)((a.QC + QG - 1) / QG));
  hipLaunchKernelGGL((k_attend_mfma<D, QG>), grid, dim3(kAttThreads), 0, s, a);
}

template <int D, int QG>
void launch_cached(const AttendArgs& a, int n_caches, hipStream_t s) {
  dim3 grid((unsigned)a.n_tiles, (unsigned)n_caches, (unsigned)((a.QC + QG - 1) / QG));
  hipLaunchKernelGGL((k_attend_cached<D, QG>), grid, dim3(kAttThreads), 0, s, a);
}

template <int D>
void launch_mfma_qg(const AttendArgs& a, int n_caches, hipStream_t s) {
  if (a.QC > 8) {
    // groups of 16 queries: P V on the matrix cores
    dim3 grid((unsigned)a.n_tiles, (unsigned)n_caches, (unsigned)((a.QC + 15) / 16));
    if (a.logits)
      hipLaunchKernelGGL((k_attend_pv16<D, true>), grid, dim3(kAttThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_attend_pv16<D, false>), grid, dim3(kAttThreads), 0, s, a);
    return;
  }
  if (a.logits) {
    if (a.QC <= 4)
      launch_cached<D, 4>(a, n_caches, s);
    else
      launch_cached<D, 8>(a, n_caches, s);
    return;
  }
  if (a.QC <= 4)
    launch_mfma<D, 4>(a, n_caches, s);
  else
    launch_mfma<D, 8>(a, n_caches, s);
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, int dtype, int n_caches, Prof& prof) {
  const int64_t n_queries = (int64_t)n_caches * a.QC;
  hipStream_t s = prof.s;
  if (a.tile_keys > 4 * kTileQuadsMax || a.tile_keys % 256) return hipErrorInvalidValue;
  prof.begin(ZHA_K_ATTEND, 0);
  if (dtype == 1) {
    if (a.D == 128)
      launch_mfma_qg<128>(a, n_caches, s);
    else
      launch_mfma_qg<64>(a, n_caches, s);
  } else {
    dim3 grid((unsigned)a.n_tiles, (unsigned)n_caches, (unsigned)((a.QC + kQG - 1) / kQG));
    if (a.D == 128)
      hipLaunchKernelGGL((k_attend<float, 128>), grid, dim3(kAttThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_attend<float, 64>), grid, dim3(kAttThreads), 0, s, a);
  }
  prof.end();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof.begin(ZHA_K_COMBINE, 0);
  if (a.D == 128)
    hipLaunchKernelGGL((k_combine<128, 8>), dim3((unsigned)n_queries), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL((k_combine<64, 16>), dim3((unsigned)n_queries), dim3(1024), 0, s, a);
  prof.end();
  return hipGetLastError();
}

hipError_t launch_selected_chunks(const uint32_t* sel1, int64_t words, int64_t n_queries, int64_t n_chunks,
                                  int32_t* ids, int32_t* count, int64_t cap, hipStream_t s) {
  hipLaunchKernelGGL(k_selected_chunks, dim3((unsigned)n_queries), dim3(kAttThreads), 0, s, sel1, words, n_chunks,
                     ids, count, cap);
  return hipGetLastError();
}

}  // namespace zha
