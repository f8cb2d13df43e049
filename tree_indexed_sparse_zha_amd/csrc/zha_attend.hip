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

template <int D>
__global__ __launch_bounds__(D) void k_combine(AttendArgs A) {
  const int64_t q = blockIdx.x;
  const int d = threadIdx.x;
  const float* base = A.partial + q * A.n_tiles * (D + 2);
  float M = kNegInf;
  for (int64_t t = 0; t < A.n_tiles; ++t) M = fmaxf(M, base[t * (D + 2)]);
  float L = 0.f, o = 0.f;
  if (M != kNegInf) {
    for (int64_t t = 0; t < A.n_tiles; ++t) {
      const float mt = base[t * (D + 2)];
      if (mt == kNegInf) continue;
      const float f = __expf(mt - M);
      L += f * base[t * (D + 2) + 1];
      o += f * base[t * (D + 2) + 2 + d];
    }
  }
  A.out[q * D + d] = L > 0.f ? o / L : 0.f;
  if (d == 0 && A.lse) A.lse[q] = L > 0.f ? M + __logf(L) : kNegInf;
}

}  // namespace

hipError_t launch_attend(const AttendArgs& a, int dtype, int n_caches, Prof& prof) {
  const int64_t n_queries = (int64_t)n_caches * a.QC;
  hipStream_t s = prof.s;
  dim3 grid((unsigned)a.n_tiles, (unsigned)n_caches, (unsigned)((a.QC + kQG - 1) / kQG));
  prof.begin(ZHA_K_ATTEND, 0);
  if (dtype == 1) {
    if (a.D == 128)
      hipLaunchKernelGGL((k_attend<bf16_t, 128>), grid, dim3(kAttThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_attend<bf16_t, 64>), grid, dim3(kAttThreads), 0, s, a);
  } else {
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
    hipLaunchKernelGGL(k_combine<128>, dim3((unsigned)n_queries), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(k_combine<64>, dim3((unsigned)n_queries), dim3(64), 0, s, a);
  prof.end();
  return hipGetLastError();
}

}  // namespace zha
