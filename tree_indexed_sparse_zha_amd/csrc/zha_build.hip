// Tree build for ZHA (levels 1..Lv) on gfx950.
//
// Defines (MTP = "Zyphra AI Introduces Zyphra Hierarchical Attention (ZHA):
// A Path to True Subquadratic Attention", section "Building the tree"):
// contiguous chunks of C keys are summarised per reference query r_j by
//   L_j = logsumexp_i z_ji,  g_j = sum_i softmax_i(z_j) k_i,  z_ji = r_j.k_i/sqrt(d),
// and summaries are merged level by level,
//   L_j(P) = logsumexp_c L_j(c),  g_j(P) = sum_c exp(L_j(c) - L_j(P)) g_j(c).
// Stored: g rounded once to the KV dtype, L, and c_j = L_j - r_j.g_j/sqrt(d)
// with the rounded g.
//
// Design.  One workgroup owns one top span (C^Lv tokens) of one cache; each of
// its W waves streams a share of it in blocks of 16 keys.  Lane (j = lane % 16, dg = lane / 16) owns
// reference query j and a quarter of the head dimension (the 16-byte pieces
// dg, dg+4, dg+8, ... of a row), so all merges of g are lane-local fp32
// arithmetic and only the two dot products over d (r.k on MFMA, r.g for c)
// cross lanes.  Open nodes of every level above the leaves are kept as fp32
// flash-style accumulators (running max, mass, weighted sum) in registers;
// a node is written once, when its last child arrives, in the d-interleaved
// layout the routing MFMA reads directly (one coalesced 1 KiB store per
// 16-byte piece group).  Since a wave rebuilds whole top spans and nothing
// else, a rebuild of the spans touched by appended tokens reproduces a fresh
// build bit for bit.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {
namespace {

constexpr int kKeysPerBlock = 16;

__device__ __forceinline__ void absorb(float& am, float& as, float* aacc, bool& used, float mc,
                                       float sc, const float* gc, int nv) {
  // Fold a child with mass sc*exp(mc) and mass-weighted key sum gc*exp(mc)
  // into an open node.
  if (!used) {
    am = mc;
    as = sc;
    for (int v = 0; v < nv; ++v) aacc[v] = gc[v];
    used = true;
    return;
  }
  // explicit fused forms: every kernel that folds nodes rounds alike
  const float mn = fmaxf(am, mc);
  const float fa = __expf(am - mn), fc = __expf(mc - mn);
  as = fmaf(as, fa, sc * fc);
  for (int v = 0; v < nv; ++v) aacc[v] = fmaf(aacc[v], fa, gc[v] * fc);
  am = mn;
}

// W > 1: the workgroup's W waves share one top span (W divides C), wave w
// streaming the w-th W-th of it, i.e. C / W whole children of the top node;
// their open top-level accumulators are merged in LDS, in wave order, by
// wave 0.
template <typename T, int D, int NA, bool LEAF_ACC, int W>
__global__ __launch_bounds__(64 * W) void k_build_span(BuildArgs A) {
  constexpr int E = Elem<T>::per16;
  constexpr int PIECES = D / E;
  constexpr int NS = PIECES / 4;  // 16-byte pieces per lane
  constexpr int NV = NS * E;      // fp32 values per lane = D / 4
  constexpr int KB = kKeysPerBlock;
  constexpr int NAR = NA > 0 ? NA : 1;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15, dg = lane >> 4;
  const TreeGeom& geo = A.geo;
  const int R = geo.R, C = geo.C;
  const int cache = blockIdx.y;
  const int b = cache / geo.H, h = cache % geo.H;
  const int64_t span = A.first_span + blockIdx.x;
  const int64_t ncomplete = (A.n_tokens / C) * C;
  const int64_t t0 = span * A.span_tokens;  // span start: every node boundary is relative to it
  const int64_t tend = min(t0 + A.span_tokens, ncomplete);
  if (t0 >= tend) return;  // uniform over the workgroup
  // this wave's share of the span
  const int64_t sub = A.span_tokens / W;
  const int64_t w0 = t0 + wave * sub;
  const int64_t t1 = min(w0 + sub, tend);
  const float isd = A.inv_sqrt_d;

  // reference query j, this lane's quarter of d (with bf16 keys, rounded
  // to bf16: the tree is that of the bf16-rounded reference queries)
  float rj[NV];
  {
    const float* rp = A.ref + ((int64_t)h * R + (j < R ? j : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float r = (j < R) ? rp[(4 * s + dg) * E + e] : 0.f;
        rj[s * E + e] = sizeof(T) == 2 ? round_bf16f(r) : r;
      }
  }

  __shared__ uint4 Ks_all[W][KB * PIECES];
  __shared__ float zs_all[W][16][KB + 1];
  uint4* Ks = Ks_all[wave];
  float (*zs)[KB + 1] = zs_all[wave];

  const T* Kc = reinterpret_cast<const T*>(A.K) + (int64_t)b * A.sb + (int64_t)h * A.sh;

  // open nodes above the leaves (or of the leaves themselves when C > 16)
  float am[NAR], as[NAR], aacc[NAR][NV];
  bool used[NAR];
#pragma unroll
  for (int a = 0; a < NAR; ++a) used[a] = false;

  // Writes one node: g rounded to its storage (kv dtype, or fp8 with a row
  // scale), L and c = L - r.g/sqrt(d) with the stored g, at the given
  // destinations (a tree level, or a prefill spine record).
  auto emit_at = [&](bool fp8, char* gb, float* Ld, float* cd, float* sd, float L, const float* g) {
    float gr[NV];
    if constexpr (sizeof(T) == 2 && NS % 2 == 0) {
      if (fp8) {
        // fp8 E4M3 with a power-of-two scale per row j: 2^e, e = ceil(log2 max|g_j|) - 8
        float mx = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) mx = fmaxf(mx, fabsf(g[v]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const uint32_t mb = __float_as_uint(mx);
        const int ex = (int)(mb >> 23) & 255;
        const int e = ex == 0 ? 0 : ((mb & 0x7fffffu) == 0u ? ex - 127 : ex - 126) - 8;
        const float scl = ldexpf(1.f, e);
        uint32_t w8[NV / 4];  // 4 E4M3 codes per word, hardware round to nearest even
#pragma unroll
        for (int k = 0; k < NV / 4; ++k) {
          const float a0 = ldexpf(g[4 * k], -e), a1 = ldexpf(g[4 * k + 1], -e);
          const float a2 = ldexpf(g[4 * k + 2], -e), a3 = ldexpf(g[4 * k + 3], -e);
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
          w8[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo, true);
          gr[4 * k + 0] = __builtin_amdgcn_cvt_f32_fp8((int)w8[k], 0) * scl;
          gr[4 * k + 1] = __builtin_amdgcn_cvt_f32_fp8((int)w8[k], 1) * scl;
          gr[4 * k + 2] = __builtin_amdgcn_cvt_f32_fp8((int)w8[k], 2) * scl;
          gr[4 * k + 3] = __builtin_amdgcn_cvt_f32_fp8((int)w8[k], 3) * scl;
        }
        float dot = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) dot += rj[v] * gr[v];
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        const float c = L - dot * isd;
        if (j < R) {
          // this lane's 8-value pieces s = 0..NS-1 are MFMA steps s, k-group dg;
          // steps 2P and 2P+1 share one 16-byte slot
#pragma unroll
          for (int P = 0; P < NS / 2; ++P)
            st16(gb + ((int64_t)(P * 4 + dg) * R + j) * 16,
                 make_uint4(w8[4 * P], w8[4 * P + 1], w8[4 * P + 2], w8[4 * P + 3]));
          if (dg == 0) {
            Ld[j] = L;
            cd[j] = c;
            sd[j] = scl;
          }
        }
        return;
      }
    }
    uint4 pk[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) pk[s] = pack(&g[s * E], &gr[s * E], T());
    float dot = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) dot += rj[v] * gr[v];
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const float c = L - dot * isd;
    if (j < R) {
#pragma unroll
      for (int s = 0; s < NS; ++s) st16(gb + ((int64_t)(s * 4 + dg) * R + j) * 16, pk[s]);
      if (dg == 0) {
        Ld[j] = L;
        cd[j] = c;
      }
    }
  };
  auto emit = [&](int lvl, int64_t node, float L, const float* g) {
    if (A.spine) return;  // spine pass: the tree is already built
    const bool fp8 = (geo.g8 >> (lvl - 1)) & 1u;
    const int64_t nidx = (int64_t)cache * geo.node_cap[lvl - 1] + node;
    const int64_t gnode = (int64_t)R * D * (fp8 ? 1 : Elem<T>::size);
    float* Lb = reinterpret_cast<float*>(A.tree + geo.L_off[lvl - 1]) + nidx * R;
    float* cb = reinterpret_cast<float*>(A.tree + geo.c_off[lvl - 1]) + nidx * R;
    float* sb = fp8 ? reinterpret_cast<float*>(A.tree + geo.s_off[lvl - 1]) + nidx * R : nullptr;
    emit_at(fp8, A.tree + geo.g_off[lvl - 1] + nidx * gnode, Lb, cb, sb, L, g);
  };
  // spine record of (state k, level lvl): g block, then L, c, scale
  auto emit_spine = [&](int64_t k, int lvl, float L, const float* g) {
    const bool fp8 = (geo.g8 >> (lvl - 1)) & 1u;
    char* rec = A.spine + spine_record(cache, k, lvl, A.spine_k0, A.spine_states, geo.levels, A.spine_rec);
    const int64_t gbytes = (int64_t)R * D * (fp8 ? 1 : Elem<T>::size);
    float* f = reinterpret_cast<float*>(rec + gbytes);
    emit_at(fp8, rec, f, f + R, f + 2 * R, L, g);
  };

  // merge pass of a split top span: fold the fp32 children the sub-span pass
  // stored into the top node with the unsplit build's association: the 4
  // waves of a span each fold their C / 4 children in order, then wave 0
  // folds the waves' results in order
  const int64_t rec_floats = (int64_t)R * (D + 2);
  if (A.merge_top) {
    float mm = 0.f, ss = 0.f, gg[NV];
    bool u = false;
    const int64_t sub_tokens = A.span_tokens / C;
    const int per = C / 4;
    for (int w = 0; w < 4; ++w) {
      float wm = 0.f, wsum = 0.f, wg[NV];
      bool wu = false;
      for (int c = w * per; c < (w + 1) * per; ++c) {
        if (t0 + c * sub_tokens >= tend) break;
        const float* rec = A.top_scratch + (((int64_t)cache * 2 + (span - A.scratch_span0)) * C + c) * rec_floats;
        const int jj = j < R ? j : 0;
        float gc[NV];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int e = 0; e < E; ++e) gc[s * E + e] = rec[2 * R + (int64_t)jj * D + (4 * s + dg) * E + e];
        absorb(wm, wsum, wg, wu, rec[jj], rec[R + jj], gc, NV);
      }
      if (wu) absorb(mm, ss, gg, u, wm, wsum, wg, NV);
    }
    if (u) {
      const float L = mm + __logf(ss);
      const float inv = 1.f / ss;
#pragma unroll
      for (int v = 0; v < NV; ++v) gg[v] *= inv;
      emit(geo.levels, span, L, gg);
    }
    return;
  }

  auto load_block = [&](int64_t pos, int nk, uint4* regs) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pi = lane + 64 * u;
      const int key = pi / PIECES, pc = pi % PIECES;
      regs[u] = key < nk ? ld16(Kc + (pos + key) * A.st + pc * E) : make_uint4(0, 0, 0, 0);
    }
  };

  // bf16: reference rows as MFMA A operands (exact: ref holds bf16 values)
  bf16x8 afr[NS];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float rr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rr[e] = rj[s * 8 + e];
      float dummy[8];
      afr[s] = as_bf16x8(pack(rr, dummy, bf16_t()));
    }
  }

  uint4 pre[NS];
  int64_t pos = w0;
  int nk = (int)min<int64_t>(KB, t1 - pos);
  if (pos < t1) load_block(pos, nk, pre);
  const int seg = C < KB ? C : KB;

  while (pos < t1) {
#pragma unroll
    for (int u = 0; u < NS; ++u) Ks[lane + 64 * u] = pre[u];
    wave_sync();
    const int64_t npos = pos + nk;
    const int nnk = (int)min<int64_t>(KB, t1 - npos);
    if (npos < t1) load_block(npos, nnk, pre);

    // z[j][i] = r_j . k_i / sqrt(d) for the 16 keys of the block
    if constexpr (sizeof(T) == 2) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint4 kb = Ks[(lane & 15) * PIECES + 4 * s + (lane >> 4)];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[s], as_bf16x8(kb), acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) zs[4 * (lane >> 4) + i][lane & 15] = acc[i] * isd;
    } else {
      for (int i = 0; i < KB; ++i) {
        float part = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float kv[E];
          unpack(Ks[i * PIECES + 4 * s + dg], kv, T());
#pragma unroll
          for (int e = 0; e < E; ++e) part += rj[s * E + e] * kv[e];
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (dg == 0) zs[j][i] = part * isd;
      }
    }
    wave_sync();

    // leaf segments of this block: seg keys each (a whole leaf when C <= 16)
    for (int sg = 0; sg < nk; sg += seg) {
      float m = kNegInf;
      for (int i = 0; i < seg; ++i) m = fmaxf(m, zs[j][sg + i]);
      float ssum = 0.f;
      float acc[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] = 0.f;
      for (int i = 0; i < seg; ++i) {
        const float e = __expf(zs[j][sg + i] - m);
        ssum += e;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float kv[E];
          unpack(Ks[(sg + i) * PIECES + 4 * s + dg], kv, T());
#pragma unroll
          for (int x = 0; x < E; ++x) acc[s * E + x] += e * kv[x];
        }
      }
      if constexpr (!LEAF_ACC) {
        const float L = m + __logf(ssum);
        const float inv = 1.f / ssum;
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] *= inv;
        if (geo.leaf_weights) {
          if (!A.spine) {
          // weights form: w_ji = exp(z_ji - L_j) and c_j = L_j - sum_i w_ji z_ji
          // (= L_j - r_j . g_j / sqrt(d) with the unrounded g_j = sum_i w_ji k_i)
          const int64_t nidx = (int64_t)cache * geo.node_cap[0] + (pos + sg) / C;
          float wz = 0.f;
          float* wb = reinterpret_cast<float*>(A.tree + geo.g_off[0]) + (nidx * R + j) * C;
          for (int i0 = 0; i0 < seg; i0 += 4) {
            float wv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const float z = zs[j][sg + i0 + x];
              wv[x] = __expf(z - m) * inv;
              wz += wv[x] * z;
            }
            if (j < R && dg == 0) *reinterpret_cast<float4*>(wb + i0) = make_float4(wv[0], wv[1], wv[2], wv[3]);
          }
          if (j < R && dg == 0) {
            reinterpret_cast<float*>(A.tree + geo.L_off[0])[nidx * R + j] = L;
            reinterpret_cast<float*>(A.tree + geo.c_off[0])[nidx * R + j] = L - wz;
          }
          }
        } else {
          emit(1, (pos + sg) / C, L, acc);
        }
        if constexpr (NA > 0) absorb(am[0], as[0], aacc[0], used[0], L, 1.f, acc, NV);
      } else {
        absorb(am[0], as[0], aacc[0], used[0], m, ssum, acc, NV);
      }
      // close every node whose span ends after this segment, bottom-up
      // (with C < 16 several levels can close inside one block)
      const int64_t end = pos + sg + seg;
      const int64_t rel = end - t0;
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const int lvl = a + (LEAF_ACC ? 1 : 2);
        const int64_t sp = geo.span_len[lvl];
        if (used[a] && (rel % sp) == 0 && !(W > 1 && a == NA - 1)) {
          const float L = am[a] + __logf(as[a]);
          const float inv = 1.f / as[a];
          float g[NV];
#pragma unroll
          for (int v = 0; v < NV; ++v) g[v] = aacc[a][v] * inv;
          emit(lvl, (end - sp) / sp, L, g);
          if (a + 1 < NA) absorb(am[a + 1], as[a + 1], aacc[a + 1], used[a + 1], L, 1.f, g, NV);
          used[a] = false;
        }
      }
      // prefill spine: after chunk k-1, the partial node of each level >= 2
      // holding it merges that level's open accumulator with every open one
      // below it (its partial descendants)
      if (A.spine && (end % C) == 0) {
        const int64_t k = end / C;
        if (k >= A.spine_k0 && k < A.spine_k0 + A.spine_states) {
          float sm = 0.f, ss = 0.f, sgc[NV];
          bool su = false;
#pragma unroll
          for (int a = 0; a < NA; ++a) {
            const int lvl = a + (LEAF_ACC ? 1 : 2);
            if (used[a]) absorb(sm, ss, sgc, su, am[a], as[a], aacc[a], NV);
            if (lvl >= 2 && su && (k % (geo.span_len[lvl] / C)) != 0) {
              const float L = sm + __logf(ss);
              const float inv = 1.f / ss;
              float g[NV];
#pragma unroll
              for (int v = 0; v < NV; ++v) g[v] = sgc[v] * inv;
              emit_spine(k, lvl, L, g);
            }
          }
        }
      }
    }
    pos = npos;
    nk = nnk;
    wave_sync();
  }

  // end of the data inside this wave's share: close the partial nodes,
  // bottom-up (with W > 1 the top accumulator is merged across waves below)
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    if (W > 1 && a == NA - 1) break;
    const int lvl = a + (LEAF_ACC ? 1 : 2);
    const int64_t sp = geo.span_len[lvl];
    if (used[a]) {
      const float L = am[a] + __logf(as[a]);
      const float inv = 1.f / as[a];
      float g[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) g[v] = aacc[a][v] * inv;
      emit(lvl, (pos - 1) / sp, L, g);
      if (a + 1 < NA) absorb(am[a + 1], as[a + 1], aacc[a + 1], used[a + 1], L, 1.f, g, NV);
      used[a] = false;
    }
  }
  if constexpr (W > 1 && NA > 0) {
    __shared__ float dep_m[W][64], dep_s[W][64], dep_g[W][NV][64];
    __shared__ int dep_used[W];
    const int top = NA - 1;
    dep_m[wave][lane] = am[top];
    dep_s[wave][lane] = as[top];
#pragma unroll
    for (int v = 0; v < NV; ++v) dep_g[wave][v][lane] = aacc[top][v];
    if (lane == 0) dep_used[wave] = used[top] ? 1 : 0;
    __syncthreads();
    if (wave == 0) {
      float mm = 0.f, ss = 0.f, gg[NV];
      bool u = false;
      for (int w = 0; w < W; ++w) {
        if (!dep_used[w]) continue;
        float gc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) gc[v] = dep_g[w][v][lane];
        absorb(mm, ss, gg, u, dep_m[w][lane], dep_s[w][lane], gc, NV);
      }
      if (u) {
        const int lvl = top + (LEAF_ACC ? 1 : 2);
        const float L = mm + __logf(ss);
        const float inv = 1.f / ss;
#pragma unroll
        for (int v = 0; v < NV; ++v) gg[v] *= inv;
        emit(lvl, t0 / geo.span_len[lvl], L, gg);
        if (A.top_scratch) {
          // sub-span pass: this node is a child of a split top node.  Keep
          // it in fp32 exactly as a top-level accumulator holds a single
          // child (max L, mass 1, mean g), so that the merge pass repeats
          // the unsplit build's arithmetic bit for bit.
          const int64_t top_span = t0 / (A.span_tokens * C);
          float* rec = A.top_scratch +
                       (((int64_t)cache * 2 + (top_span - A.scratch_span0)) * C + (t0 / A.span_tokens) % C) * rec_floats;
          if (j < R) {
            if (dg == 0) {
              rec[j] = L;
              rec[R + j] = 1.f;
            }
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int e = 0; e < E; ++e) rec[2 * R + (int64_t)j * D + (4 * s + dg) * E + e] = gg[s * E + e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core build (bf16 keys, C = 4, g in bf16, >= 3 levels).  Same node definitions as k_build_span, different work split:
//
//  * The 4 waves of a workgroup take the 4 level-2 nodes (16 keys each) of a
//    64-key round of the span, in order.  A level-2 node is computed straight
//    from its 16 keys: the weights P_ji = exp(z_ji - max_i z_ji) of the
//    16 x 16 (plane, key) logits are the B operand and the keys the A operand
//    of v_mfma_f32_16x16x4_f32, so g_j = (sum_i P_ji k_i) / (sum_i P_ji) is an
//    fp32 matrix product (4 MFMAs of K = 4 keys per 16 values of d) instead
//    of a VALU loop.  Lane (j, g) of a wave owns the 4 keys of leaf g for the
//    leaf statistics, supplies them as the K = 4 slice of the product, and
//    receives d = 16b + 4g + i (b < D/16, i < 4) of g_j.  In the mean form
//    each leaf's g is one more such product over its own 4 keys.
//  * The level-3 node of the round is the ordered merge of those 4 fp32
//    level-2 nodes (LSE of L, mass-weighted mean of g), and levels above
//    fold their children in order in flash-style accumulators, as in
//    k_build_span.  Above level 2 the 256 lanes of the workgroup split the
//    R x D values of a node: lane (j, g) of wave w owns the D/16 values of d
//    starting at (4w + g) D/16, so each lane keeps D/16 values per open level
//    instead of D/4.  The dot r_j . g_j that c needs is summed over the
//    waves in LDS, in wave order.
//
// Every node of level >= 3 is the in-order fold of its children's
// (L, mass 1, fp32 mean g); the append split (sub-span pass, then the top
// node from the stored fp32 children) therefore reproduces a fresh build bit
// for bit when both of its passes also run here.
template <int D, int NU, int C, int GF = 0>
__global__ __launch_bounds__(256, NU <= 3 ? 4 : 3) void k_build_mf(BuildArgs A) {
  constexpr bool G8 = GF == 1;  // levels written by put_node hold fp8 rows
  constexpr bool G4 = GF == 2;  // ... or MXFP4 blocks (d = 128)
  static_assert(!G4 || D == 128, "MXFP4 rows need d = 128 (a 32-block is four lanes of a wave)");
  static_assert(C == 4 || C == 8, "chunk of 4 or 8 keys");
  constexpr int RL = C == 4 ? 3 : 2;  // level of a round's node (64 keys)
  constexpr int LPL = C / 4;          // lanes of one plane sharing a leaf
  constexpr int PIECES = D / 8;  // 16-byte pieces of a bf16 key row
  constexpr int NS = PIECES / 4;  // pieces per lane when staging K; z MFMA steps
  constexpr int NB = D / 16;      // 16-wide d blocks of the level-2 product
  constexpr int VPL = D / 16;     // values of d per lane above level 2
  constexpr int KB = 16;
  constexpr int KROW = PIECES + 1;  // padded LDS key row (uint4)
  constexpr int NUR = NU > 0 ? NU : 1;
  // lane indices: lane, j, g and d0 are re-declared opaque at the top of
  // every round (an empty asm that may change them), so that the compiler
  // derives the per-lane addresses inside the round instead of keeping them
  // all live across the loop (about 250 VGPRs and 2 waves per SIMD, against
  // 128-160 and 3-4 waves per SIMD now)
  int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int j = lane & 15, g = lane >> 4;
  const TreeGeom& geo = A.geo;
  const int R = geo.R;
  const int cache = blockIdx.y;
  const int b = cache / geo.H, h = cache % geo.H;
  const int64_t span = A.first_span + blockIdx.x;
  const int64_t t0 = span * A.span_tokens;
  const int64_t tend = min(t0 + A.span_tokens, (A.n_tokens / C) * C);
  if (t0 >= tend) return;  // uniform over the workgroup
  const float isd = A.inv_sqrt_d;
  const int top = A.top_level;
  int d0 = VPL * (4 * wave + g);  // this lane's first d above level 2

  __shared__ uint4 Ks[4][KB * KROW];
  __shared__ float zs[4][16][KB + 1];
  __shared__ float chL[4][16];
  __shared__ s16x4 Wb[4][3][64];  // the round node's weights of each 16-key part (three bf16 terms)
  __shared__ float dotp[kMaxLevels][4][16];
  __shared__ float rmax[kMaxLevels][4][16];  // fp8 levels: the waves' row maxima of a node's g
  __shared__ uint4 refB[16][KROW];          // reference rows in bf16 (MFMA operands and the dots r . g)

  // with bf16 keys the tree is that of the bf16-rounded reference queries
  for (int i = threadIdx.x; i < 16 * PIECES; i += 256) {
    const int jr = i / PIECES, pc = i % PIECES;
    float rr[8], dummy[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rr[e] = jr < R ? round_bf16f(A.ref[((int64_t)h * R + jr) * D + pc * 8 + e]) : 0.f;
    refB[jr][pc] = pack(rr, dummy, bf16_t());
  }
  __syncthreads();
  // r_j[d .. d + 3] (d a multiple of 4) from the bf16 rows
  auto ref4 = [&](int jr, int d) -> float4 {
    const uint2 w = reinterpret_cast<const uint2*>(&refB[jr][d / 8])[(d % 8) / 4];
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  };

  // node writers above level 2: this lane's D/16 values of g (rounded to
  // bf16), the wave's share of r . g into dotp[slot]; L and c are stored by
  // finish() once every wave's share is in.  With fp8 rows (G8: ZHA_G_FP8
  // above levels 1-2 held as weights) row j of g is stored as
  // s_j * e4m3(g_j / s_j), s_j = 2^(ceil(log2 max_d |g_jd|) - 8) (1 for a
  // zero row): the row's maximum is gathered over the four waves through
  // LDS (one barrier; every lane of the workgroup calls put_node together).
  // With MXFP4 (G4) each block of 32 values of d is the four lanes g = 0..3
  // of one wave: its E8M0 scale 2^(floor(log2 max) - 2) comes from two
  // shuffles, and the hardware conversion rounds g / scale to E2M1 (nearest
  // even, saturating at 6).
  auto put_node = [&](int lvl, int64_t node, float L, const float* gv, int slot) {
    uint32_t wd[VPL / 2];  // bf16 pairs, (G8) E4M3 codes in wd[0 .. VPL / 4) or (G4) E2M1 codes in wd[0]
    float gr[VPL];         // the stored values
    float scl = 1.f;
    uint32_t e8 = 0u;      // G4: the E8M0 byte of this lane's block
    if constexpr (G4) {
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) mx = fmaxf(mx, fabsf(gv[e]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const int ex = (int)(__float_as_uint(mx) >> 23) & 255;  // floor(log2 mx) = ex - 127 for normal mx
      const int es = ex == 0 ? -127 : max(ex - 129, -127);
      e8 = (uint32_t)(es + 127);
      scl = __uint_as_float(e8 == 0u ? 0x00400000u : e8 << 23);  // 2^es
      uint32_t w4 = 0u;
      w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, gv[0], gv[1], scl, 0);
      w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, gv[2], gv[3], scl, 1);
      w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, gv[4], gv[5], scl, 2);
      w4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w4, gv[6], gv[7], scl, 3);
      wd[0] = w4;
      const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4, scl, 0);
      const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4, scl, 1);
      const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4, scl, 2);
      const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4, scl, 3);
      gr[0] = (float)p0[0];
      gr[1] = (float)p0[1];
      gr[2] = (float)p1[0];
      gr[3] = (float)p1[1];
      gr[4] = (float)p2[0];
      gr[5] = (float)p2[1];
      gr[6] = (float)p3[0];
      gr[7] = (float)p3[1];
    } else if constexpr (G8) {
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) mx = fmaxf(mx, fabsf(gv[e]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) rmax[slot][wave][j] = mx;
      __syncthreads();
      mx = fmaxf(fmaxf(rmax[slot][0][j], rmax[slot][1][j]), fmaxf(rmax[slot][2][j], rmax[slot][3][j]));
      const uint32_t mb = __float_as_uint(mx);
      const int ex = (int)(mb >> 23) & 255;
      const int es = ex == 0 ? 0 : ((mb & 0x7fffffu) == 0u ? ex - 127 : ex - 126) - 8;
      scl = ldexpf(1.f, es);
#pragma unroll
      for (int k = 0; k < VPL / 4; ++k) {  // hardware E4M3 conversion, round to nearest even
        const float a0 = ldexpf(gv[4 * k], -es), a1 = ldexpf(gv[4 * k + 1], -es);
        const float a2 = ldexpf(gv[4 * k + 2], -es), a3 = ldexpf(gv[4 * k + 3], -es);
        const int lo8 = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        wd[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, lo8, true);
        gr[4 * k + 0] = __builtin_amdgcn_cvt_f32_fp8((int)wd[k], 0) * scl;
        gr[4 * k + 1] = __builtin_amdgcn_cvt_f32_fp8((int)wd[k], 1) * scl;
        gr[4 * k + 2] = __builtin_amdgcn_cvt_f32_fp8((int)wd[k], 2) * scl;
        gr[4 * k + 3] = __builtin_amdgcn_cvt_f32_fp8((int)wd[k], 3) * scl;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VPL / 2; ++e) {
        wd[e] = bf16_pair(gv[2 * e], gv[2 * e + 1]);
        gr[2 * e] = bf16_lo(wd[e]);
        gr[2 * e + 1] = bf16_hi(wd[e]);
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; e += 4) {
      const float4 rv = ref4(j, d0 + e);
      dot = fmaf(rv.x, gr[e], dot);
      dot = fmaf(rv.y, gr[e + 1], dot);
      dot = fmaf(rv.z, gr[e + 2], dot);
      dot = fmaf(rv.w, gr[e + 3], dot);
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    if (g == 0) dotp[slot][wave][j] = dot;
    if (j < R) {
      const int64_t nidx = (int64_t)cache * geo.node_cap[lvl - 1] + node;
      if constexpr (G4) {
        // lane (j, g) of wave w holds d = 32w + 8g .. +7: MFMA step w, k-group g;
        // its 4 code bytes at (g * R + j) * 16 + 4w, its block's scale byte at [j][w]
        char* gb = A.tree + geo.g_off[lvl - 1] + nidx * R * (D / 2) + ((int64_t)g * R + j) * 16 + wave * 4;
        *reinterpret_cast<uint32_t*>(gb) = wd[0];
        if (g == 0) (A.tree + geo.s_off[lvl - 1])[(nidx * R + j) * (D / 32) + wave] = (char)e8;
      } else if constexpr (G8) {
        // byte of (j, d): MFMA step st = d / 32, k-group kg = (d % 32) / 8, at
        // ((st / 2) * 4R + kg * R + j) * 16 + (st % 2) * 8 + d % 8
        const int st = d0 / 32, kg = (d0 % 32) / 8;
        char* gb = A.tree + geo.g_off[lvl - 1] + nidx * R * D + ((int64_t)((st / 2) * 4 + kg) * R + j) * 16 +
                   (st % 2) * 8 + d0 % 8;
        if constexpr (VPL == 8)
          *reinterpret_cast<uint2*>(gb) = make_uint2(wd[0], wd[1]);
        else
          *reinterpret_cast<uint32_t*>(gb) = wd[0];
        if (d0 == 0) reinterpret_cast<float*>(A.tree + geo.s_off[lvl - 1])[nidx * R + j] = scl;
      } else {
        char* gb = A.tree + geo.g_off[lvl - 1] + nidx * R * D * 2 + ((int64_t)(d0 / 8) * R + j) * 16 + (d0 % 8) * 2;
        if constexpr (VPL == 8)
          st16(gb, make_uint4(wd[0], wd[1], wd[2], wd[3]));
        else
          *reinterpret_cast<uint2*>(gb) = make_uint2(wd[0], wd[1]);
      }
      if (lvl == top && A.top_scratch && !A.merge_top) {
        // sub-span pass: the top node is a child of a split top node; keep it
        // in fp32 as (L, mass 1, mean g) for the merge pass
        const int64_t top_span = t0 / (A.span_tokens * C);
        float* rec = A.top_scratch +
                     (((int64_t)cache * 2 + (top_span - A.scratch_span0)) * C + (t0 / A.span_tokens) % C) *
                         ((int64_t)R * (D + 2));
#pragma unroll
        for (int e = 0; e < VPL; ++e) rec[2 * R + (int64_t)j * D + d0 + e] = gv[e];
        if (wave == 0 && g == 0) {
          rec[j] = L;
          rec[R + j] = 1.f;
        }
      }
    }
  };
  auto finish = [&](int lvl, int64_t node, float L, int slot) {
    if (wave == 0 && g == 0 && j < R) {
      const float dot = ((dotp[slot][0][j] + dotp[slot][1][j]) + dotp[slot][2][j]) + dotp[slot][3][j];
      const int64_t nidx = (int64_t)cache * geo.node_cap[lvl - 1] + node;
      reinterpret_cast<float*>(A.tree + geo.L_off[lvl - 1])[nidx * R + j] = L;
      reinterpret_cast<float*>(A.tree + geo.c_off[lvl - 1])[nidx * R + j] = L - dot * isd;
    }
  };

  if (A.merge_top) {
    // merge pass of a split top span: fold the C stored fp32 children in order
    const int64_t sub_tokens = A.span_tokens / C;
    const int jj = j < R ? j : 0;
    float mm = 0.f, ss = 0.f, gg[VPL];
    bool u = false;
    for (int c = 0; c < C; ++c) {
      if (t0 + c * sub_tokens >= tend) break;
      const float* rec = A.top_scratch +
                         (((int64_t)cache * 2 + (span - A.scratch_span0)) * C + c) * ((int64_t)R * (D + 2));
      float gc[VPL];
#pragma unroll
      for (int e = 0; e < VPL; ++e) gc[e] = rec[2 * R + (int64_t)jj * D + d0 + e];
      absorb(mm, ss, gg, u, rec[jj], rec[R + jj], gc, VPL);
    }
    const float L = mm + __logf(ss);
    const float inv = 1.f / ss;
#pragma unroll
    for (int e = 0; e < VPL; ++e) gg[e] *= inv;
    put_node(top, span, L, gg, 0);
    __syncthreads();
    finish(top, span, L, 0);
    return;
  }

  const bf16_t* Kc = reinterpret_cast<const bf16_t*>(A.K) + (int64_t)b * A.sb + (int64_t)h * A.sh;
  const int64_t nkeys = tend - t0;
  const int64_t nrounds = (nkeys + 63) / 64;
  auto block_keys = [&](int64_t r) -> int {
    const int64_t s0 = 64 * r + 16 * wave;
    return (int)max<int64_t>(0, min<int64_t>(16, nkeys - s0));
  };
  auto load_block = [&](int64_t pos, int nk, uint4* regs) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pi = lane + 64 * u;
      const int key = pi / PIECES, pc = pi % PIECES;
      regs[u] = key < nk ? ld16(Kc + (pos + key) * A.st + pc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 pre[NS];
  {
    const int nk0 = block_keys(0);
    if (nk0 > 0) load_block(t0 + 16 * wave, nk0, pre);
  }
  const uint16_t* Ks16 = reinterpret_cast<const uint16_t*>(Ks[wave]);
  // A operand of a 16x16x16 bf16 product over a part's 16 keys: keys
  // 4gg .. 4gg + 3 at column d (exact)
  auto key_operand = [&](const uint16_t* K16, int d, int gg) -> s16x4 {
    uint32_t kw[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint32_t k0 = K16[((4 * gg + 2 * h2) * KROW + d / 8) * 8 + d % 8];
      const uint32_t k1 = K16[((4 * gg + 2 * h2 + 1) * KROW + d / 8) * 8 + d % 8];
      kw[h2] = k0 | (k1 << 16);
    }
    return pack_s16x4(kw[0], kw[1]);
  };
  // four fp32 weights as three bf16 B operands, hi + mid + lo = x to within
  // 2^-27 relative
  auto split3 = [](const float* x, s16x4* pw) {
    float hi[4], mid[4], lo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      hi[s] = round_bf16f(x[s]);
      const float r1 = x[s] - hi[s];
      mid[s] = round_bf16f(r1);
      lo[s] = round_bf16f(r1 - mid[s]);
    }
    pw[0] = pack_s16x4(bf16_pair(hi[0], hi[1]), bf16_pair(hi[2], hi[3]));
    pw[1] = pack_s16x4(bf16_pair(mid[0], mid[1]), bf16_pair(mid[2], mid[3]));
    pw[2] = pack_s16x4(bf16_pair(lo[0], lo[1]), bf16_pair(lo[2], lo[3]));
  };

  // open accumulators of levels RL + 1 .. RL + NU
  float um[NUR], us[NUR], ua[NUR][VPL];
  bool uu[NUR];
#pragma unroll
  for (int a = 0; a < NUR; ++a) uu[a] = false;

  for (int64_t r = 0; r < nrounds; ++r) {
    asm volatile("" : "+v"(lane), "+v"(j), "+v"(g), "+v"(d0));
    const int nk = block_keys(r);
    const int64_t kb0 = t0 + 64 * r + 16 * wave;  // this wave's 16-key block
    if (nk > 0) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int pi = lane + 64 * u;
        Ks[wave][(pi / PIECES) * KROW + pi % PIECES] = pre[u];
      }
    }
    wave_sync();
    {
      const int nnk = block_keys(r + 1);
      if (nnk > 0) load_block(kb0 + 64, nnk, pre);
    }
    float P[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's normalised weights of its 4 keys in the block
    if (nk > 0) {
      // z[j][i] = r_j . k_i / sqrt(d)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(refB[lane & 15][4 * s + g]),
                                                      as_bf16x8(Ks[wave][(lane & 15) * KROW + 4 * s + g]), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) zs[wave][4 * g + i][lane & 15] = acc[i] * isd;
      wave_sync();

      // this lane's keys 4g .. 4g+3 of the block: leaf g (C = 4), or half of
      // leaf g / 2 (C = 8, statistics shared with lane g ^ 1)
      const bool leaf = 4 * g < nk;
      float z[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) z[s] = zs[wave][j][4 * g + s];
      float m1 = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      if constexpr (C == 8) m1 = fmaxf(m1, __shfl_xor(m1, 16));
      float e[4], s1 = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        e[s] = __expf(z[s] - m1);
        s1 += e[s];
      }
      if constexpr (C == 8) s1 += __shfl_xor(s1, 16);
      float Lleaf = 0.f;  // weights form: the log mass of this lane's leaf
      if (!geo.leaf_weights) {
        // mean form: leaf l's g_j = sum_i w_ji k_i over its C keys is C / 4
        // fp32 MFMAs per 16 values of d (K = 4 of the leaf's keys; lane (j, g)
        // supplies keys Cl + 4s + g, whose weights it recomputes from leaf
        // l's max and sum, shuffled from a lane of that leaf)
        const float L1 = m1 + __logf(s1);
        const float inv1 = 1.f / s1;
#pragma unroll
        for (int l = 0; l < 16 / C; ++l) {
          if (C * l >= nk) break;  // uniform: leaves are complete
          const int src = (lane & 15) + 16 * (l * LPL);
          const float ml = __shfl(m1, src), il = __shfl(inv1, src), Ll = __shfl(L1, src);
          float wb[LPL];
#pragma unroll
          for (int s = 0; s < LPL; ++s) wb[s] = __expf(zs[wave][j][C * l + 4 * s + g] - ml) * il;
          float dot = 0.f;
          uint2 pk[NB];
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
            const int d = 16 * blk + (lane & 15);
            f32x4 Gl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < LPL; ++s) {
              const float kv =
                  __uint_as_float((uint32_t)Ks16[((C * l + 4 * s + g) * KROW + d / 8) * 8 + d % 8] << 16);
              Gl = __builtin_amdgcn_mfma_f32_16x16x4f32(kv, wb[s], Gl, 0, 0, 0);
            }
            const float4 rv = ref4(j, 16 * blk + 4 * g);
            pk[blk] = make_uint2(bf16_pair(Gl[0], Gl[1]), bf16_pair(Gl[2], Gl[3]));
            dot = fmaf(rv.x, bf16_lo(pk[blk].x), dot);
            dot = fmaf(rv.y, bf16_hi(pk[blk].x), dot);
            dot = fmaf(rv.z, bf16_lo(pk[blk].y), dot);
            dot = fmaf(rv.w, bf16_hi(pk[blk].y), dot);
          }
          dot += __shfl_xor(dot, 16);
          dot += __shfl_xor(dot, 32);
          if (j < R) {
            const int64_t nidx = (int64_t)cache * geo.node_cap[0] + kb0 / C + l;
            char* gb = A.tree + geo.g_off[0] + nidx * R * D * 2;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
              *reinterpret_cast<uint2*>(gb + ((int64_t)(2 * blk + g / 2) * R + j) * 16 + (g % 2) * 8) = pk[blk];
            if (g == 0) {
              reinterpret_cast<float*>(A.tree + geo.L_off[0])[nidx * R + j] = Ll;
              reinterpret_cast<float*>(A.tree + geo.c_off[0])[nidx * R + j] = Ll - dot * isd;
            }
          }
        }
      } else {
        // weights form: w_ji = exp(z_ji - L_j), c_j = L_j - sum_i w_ji z_ji
        const float L1 = m1 + __logf(s1);
        Lleaf = L1;
        const float inv1 = 1.f / s1;
        float wv[4], wz = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          wv[s] = e[s] * inv1;
          wz += wv[s] * z[s];
        }
        if constexpr (C == 8) wz += __shfl_xor(wz, 16);
        if (leaf && j < R) {
          const int64_t nidx = (int64_t)cache * geo.node_cap[0] + kb0 / C + g / LPL;
          // the tree is written once here and read by later calls: nontemporal stores
          st16_nt(reinterpret_cast<float*>(A.tree + geo.g_off[0]) + (nidx * R + j) * C + 4 * (g % LPL), wv[0], wv[1],
                  wv[2], wv[3]);
          if (g % LPL == 0) {
            st4_nt(reinterpret_cast<float*>(A.tree + geo.L_off[0]) + nidx * R + j, L1);
            st4_nt(reinterpret_cast<float*>(A.tree + geo.c_off[0]) + nidx * R + j, L1 - wz);
          }
        }
      }

      // the block's 16 keys: the level-2 node (C = 4) or a quarter of the
      // round's level-2 node (C = 8); weights relative to the block max
      float m2 = leaf ? m1 : kNegInf;
      m2 = fmaxf(m2, __shfl_xor(m2, 16));
      m2 = fmaxf(m2, __shfl_xor(m2, 32));
      float ps = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        P[s] = leaf ? __expf(z[s] - m2) : 0.f;
        ps += P[s];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      const float L2 = m2 + __logf(ps);
      const float inv2 = 1.f / ps;
#pragma unroll
      for (int s = 0; s < 4; ++s) P[s] *= inv2;  // normalised weights of the block
      // when C = 4 the block is also emitted as the level-2 node: its rounded
      // mean keys (lane: d = 16b + 4g + i of plane j, from the product below),
      // or, when level 2 is scored from its keys, the mass share
      // exp(L(leaf g) - L) of each child (so that the weight of key i of leaf
      // g is that share times the leaf's own w) with c = L - sum_i P_i z_i
      const bool w2 = C == 4 && geo.w2;
      float dot = 0.f;
      uint2 pk[NB];
      if (C == 4 && !w2) {
        // g^T[d][j] = sum over keys k[key][d] P[j][key] on the bf16 matrix
        // cores (v_mfma_f32_16x16x16_bf16, the 16 keys as the contraction):
        // A = keys (row d = 16b + lane % 16, k = key 4g + s: exact in bf16),
        // B = P (k = key 4g + s, column j: this lane's own four weights), P
        // split into three bf16 terms (hi + mid + lo = P to within 2^-27
        // relative), so that the three products accumulate the fp32 sum
        s16x4 pw[3];
        split3(P, pw);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          f32x4 G = {0.f, 0.f, 0.f, 0.f};
          const s16x4 ka = key_operand(Ks16, 16 * blk + (lane & 15), g);
#pragma unroll
          for (int t = 0; t < 3; ++t) G = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, pw[t], G, 0, 0, 0);
          const float4 rv = ref4(j, 16 * blk + 4 * g);
          pk[blk] = make_uint2(bf16_pair(G[0], G[1]), bf16_pair(G[2], G[3]));
          dot = fmaf(rv.x, bf16_lo(pk[blk].x), dot);
          dot = fmaf(rv.y, bf16_hi(pk[blk].x), dot);
          dot = fmaf(rv.z, bf16_lo(pk[blk].y), dot);
          dot = fmaf(rv.w, bf16_hi(pk[blk].y), dot);
        }
      } else if (w2) {
        dot = P[0] * z[0];
#pragma unroll
        for (int s = 1; s < 4; ++s) dot = fmaf(P[s], z[s], dot);
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      if (g == 0) chL[wave][j] = L2;
      if (C == 4 && j < R) {
        const int64_t nidx = (int64_t)cache * geo.node_cap[1] + kb0 / 16;
        if (w2) {
          st4_nt(reinterpret_cast<float*>(A.tree + geo.g_off[1]) + (nidx * R + j) * 4 + g, leaf ? __expf(Lleaf - L2) : 0.f);
        } else {
          char* gb = A.tree + geo.g_off[1] + nidx * R * D * 2;
#pragma unroll
          for (int blk = 0; blk < NB; ++blk)
            *reinterpret_cast<uint2*>(gb + ((int64_t)(2 * blk + g / 2) * R + j) * 16 + (g % 2) * 8) = pk[blk];
        }
        if (g == 0) {
          st4_nt(reinterpret_cast<float*>(A.tree + geo.L_off[1]) + nidx * R + j, L2);
          st4_nt(reinterpret_cast<float*>(A.tree + geo.c_off[1]) + nidx * R + j, w2 ? L2 - dot : L2 - dot * isd);
        }
      }
    }
    __syncthreads();  // the round's four 16-key parts (keys, L) are in LDS

    // the round's node (level 3 when C = 4, level 2 when C = 8) over its up
    // to 64 keys: each 16-key part's share exp(L_c - max) / sum (the max of
    // the parts' L first), and the key weights W = share_c * P (P the part's
    // normalised weights), so that g = sum_i W_i k_i; L is the LSE of the
    // parts' L
    const int nch = (int)min<int64_t>(4, (nkeys - 64 * r + 15) / 16);
    float lc[4], m3 = chL[0][j];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      lc[c] = c < nch ? chL[c][j] : kNegInf;
      m3 = fmaxf(m3, lc[c]);
    }
    float wc[4], s3 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wc[c] = c < nch ? __expf(lc[c] - m3) : 0.f;
      s3 += wc[c];
    }
    const float L3 = m3 + __logf(s3);
    {
      const float inv = 1.f / s3;
#pragma unroll
      for (int c = 0; c < 4; ++c) wc[c] *= inv;
    }
    if (wave < nch) {
      // this wave's part: its weights as the B operand of k-step `wave` of
      // the round's product (lane (j, g): keys 4g + s of the part, plane j)
      const float ws = wave == 0 ? wc[0] : wave == 1 ? wc[1] : wave == 2 ? wc[2] : wc[3];
      float W[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) W[s] = ws * P[s];
      s16x4 pw[3];
      split3(W, pw);
#pragma unroll
      for (int t = 0; t < 3; ++t) Wb[wave][t][lane] = pw[t];
    }
    __syncthreads();  // every part's weights are in
    // g^T[d][j] = sum over the round's keys k[key][d] W[j][key] on the bf16
    // matrix cores, 16 keys (one part) per k-step.  Wave w computes this
    // lane's own values above level 2, d = d0 + 4q + i (q < D / 64, i < 4):
    // A-operand row rr of step q takes d = VPL (4w + rr / 4) + 4q + rr % 4,
    // so that output rows 4g + i land on lane (j, g).
    float a3[VPL];
    {
      f32x4 G3[VPL / 4];
#pragma unroll
      for (int q = 0; q < VPL / 4; ++q) G3[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int rr = lane & 15;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < nch) {
          const uint16_t* Kp = reinterpret_cast<const uint16_t*>(Ks[c]);
          s16x4 wb[3];
#pragma unroll
          for (int t = 0; t < 3; ++t) wb[t] = Wb[c][t][lane];
#pragma unroll
          for (int q = 0; q < VPL / 4; ++q) {
            const s16x4 ka = key_operand(Kp, VPL * (4 * wave + rr / 4) + 4 * q + rr % 4, g);
#pragma unroll
            for (int t = 0; t < 3; ++t) G3[q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, wb[t], G3[q], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < VPL / 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) a3[4 * q + i] = G3[q][i];
    }
    const int64_t rel = min<int64_t>(64 * (r + 1), nkeys);
    const int64_t end = t0 + rel;
    const bool last = rel == nkeys;
    put_node(RL, (t0 + 64 * r) / 64, L3, a3, 0);
    float pL[NUR];
    int64_t pnode[NUR];
    bool pend[NUR];
#pragma unroll
    for (int a = 0; a < NUR; ++a) pend[a] = false;
    if constexpr (NU > 0) absorb(um[0], us[0], ua[0], uu[0], L3, 1.f, a3, VPL);
    // close every level above the round's whose span ends here, bottom-up
#pragma unroll
    for (int a = 0; a < NU; ++a) {
      const int lvl = RL + 1 + a;
      const int sh = (C == 4 ? 2 : 3) * lvl;  // span_len[lvl] = C^lvl = 2^sh
      if (uu[a] && ((rel & ((1ll << sh) - 1)) == 0 || last)) {
        const float L = um[a] + __logf(us[a]);
        const float inv = 1.f / us[a];
        float gv[VPL];
#pragma unroll
        for (int e = 0; e < VPL; ++e) gv[e] = ua[a][e] * inv;
        put_node(lvl, (end - 1) >> sh, L, gv, a + 1);
        pend[a] = true;
        pL[a] = L;
        pnode[a] = (end - 1) >> sh;
        if (a + 1 < NU) absorb(um[a + 1], us[a + 1], ua[a + 1], uu[a + 1], L, 1.f, gv, VPL);
        uu[a] = false;
      }
    }
    __syncthreads();  // every wave's share of r . g is in
    finish(RL, (t0 + 64 * r) / 64, L3, 0);
#pragma unroll
    for (int a = 0; a < NU; ++a)
      if (pend[a]) finish(RL + 1 + a, pnode[a], pL[a], a + 1);
  }
}

// Waves per top span: W = min(C, 4) when the top node has children built by
// the waves (C <= 16 and at least 2 levels); W divides C, so a wave's share
// is a whole number of the top node's children.
template <typename T, int D, int NA, bool LEAF>
hipError_t launch_na(const BuildArgs& a, dim3 grid, hipStream_t s) {
  if (a.spine || a.merge_top) {
    // the spine needs the accumulators in key order: one wave per span
    hipLaunchKernelGGL((k_build_span<T, D, NA, LEAF, 1>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  if constexpr (!LEAF && NA >= 1) {
    if (a.geo.C >= 4) {
      hipLaunchKernelGGL((k_build_span<T, D, NA, LEAF, 4>), grid, dim3(256), 0, s, a);
      return hipGetLastError();
    }
    if (a.geo.C == 2) {
      hipLaunchKernelGGL((k_build_span<T, D, NA, LEAF, 2>), grid, dim3(128), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_build_span<T, D, NA, LEAF, 1>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_leaf(const BuildArgs& a, dim3 grid, hipStream_t s) {
  if (a.geo.C > kKeysPerBlock) {
    // leaves span several blocks: an open node per level, leaves included
    switch (a.top_level) {
      case 1: return launch_na<T, D, 1, true>(a, grid, s);
      case 2: return launch_na<T, D, 2, true>(a, grid, s);
      case 3: return launch_na<T, D, 3, true>(a, grid, s);
      case 4: return launch_na<T, D, 4, true>(a, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.top_level - 1) {
    case 0: return launch_na<T, D, 0, false>(a, grid, s);
    case 1: return launch_na<T, D, 1, false>(a, grid, s);
    case 2: return launch_na<T, D, 2, false>(a, grid, s);
    case 3: return launch_na<T, D, 3, false>(a, grid, s);
    case 4: return launch_na<T, D, 4, false>(a, grid, s);
    case 5: return launch_na<T, D, 5, false>(a, grid, s);
    case 6: return launch_na<T, D, 6, false>(a, grid, s);
    case 7: return launch_na<T, D, 7, false>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int C, int GF>
hipError_t dispatch_mf_c(const BuildArgs& a, dim3 grid, hipStream_t s) {
  const int nu = a.merge_top ? 0 : a.top_level - (C == 4 ? 3 : 2);
  switch (nu) {
    case 0: hipLaunchKernelGGL((k_build_mf<D, 0, C, GF>), grid, dim3(256), 0, s, a); break;
    case 1: hipLaunchKernelGGL((k_build_mf<D, 1, C, GF>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_build_mf<D, 2, C, GF>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_build_mf<D, 3, C, GF>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_build_mf<D, 4, C, GF>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_build_mf<D, 5, C, GF>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// fp8 and MXFP4 rows are built here only above levels 1-2 held as weights
// (chunk 4): then every level k_build_mf writes through put_node holds them
template <int D>
hipError_t dispatch_mf(const BuildArgs& a, dim3 grid, hipStream_t s) {
  if (a.geo.g8 || a.geo.g4) {
    if (a.geo.C != 4 || !a.geo.w2) return hipErrorInvalidValue;
    if (a.geo.g8) return dispatch_mf_c<D, 4, 1>(a, grid, s);
    if constexpr (D == 128) return dispatch_mf_c<D, 4, 2>(a, grid, s);
    return hipErrorInvalidValue;
  }
  if (a.geo.C == 8) return dispatch_mf_c<D, 8, 0>(a, grid, s);
  if (a.geo.C == 4) return dispatch_mf_c<D, 4, 0>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_build(const BuildArgs& a, int dtype, Prof& prof) {
  if (a.n_spans <= 0 || a.geo.caches <= 0) return hipSuccess;
  dim3 grid((unsigned)a.n_spans, (unsigned)a.geo.caches);
  hipStream_t s = prof.s;
  hipError_t e;
  prof.begin(ZHA_K_BUILD, 0);
  if (a.mf && !a.spine) {
    e = a.geo.D == 128 ? dispatch_mf<128>(a, grid, s) : dispatch_mf<64>(a, grid, s);
  } else if (dtype == 1)
    e = a.geo.D == 128 ? dispatch_leaf<bf16_t, 128>(a, grid, s) : dispatch_leaf<bf16_t, 64>(a, grid, s);
  else
    e = a.geo.D == 128 ? dispatch_leaf<float, 128>(a, grid, s) : dispatch_leaf<float, 64>(a, grid, s);
  prof.end();
  return e;
}

}  // namespace zha
