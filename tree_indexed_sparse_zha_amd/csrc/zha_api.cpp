// C-ABI entry points of the ZHA decode path: argument checks, layouts and
// launch geometry.  Every check runs on the host before any HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "zha_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ZHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
int esize(int dtype) { return dtype == ZHA_BF16 ? 2 : 4; }

int check_config(const zha_config* c) {
  if (!c) return fail(ZHA_ERR_NULL, "cfg is NULL");
  if (c->batch < 1 || c->n_kv_heads < 1 || c->q_per_kv < 1)
    return fail(ZHA_ERR_ARG, "batch, n_kv_heads and q_per_kv must be >= 1");
  if (c->head_dim < 1 || c->n_ref < 1 || c->chunk < 1 || c->levels < 1)
    return fail(ZHA_ERR_ARG, "head_dim, n_ref, chunk and levels must be >= 1");
  if (c->capacity_tokens < 1) return fail(ZHA_ERR_ARG, "capacity_tokens must be >= 1");
  if (c->kv_dtype != ZHA_F32 && c->kv_dtype != ZHA_BF16)
    return fail(ZHA_ERR_UNSUPPORTED, "kv_dtype %d unsupported", c->kv_dtype);
  if (c->leaf_form != ZHA_LEAF_MEAN && c->leaf_form != ZHA_LEAF_WEIGHTS && c->leaf_form != ZHA_LEAF_WEIGHTS2)
    return fail(ZHA_ERR_ARG, "leaf_form %d unknown", c->leaf_form);
  if (c->leaf_form == ZHA_LEAF_WEIGHTS2 && (c->kv_dtype != ZHA_BF16 || c->chunk != 4 || c->levels < 3 || c->levels > 8))
    return fail(ZHA_ERR_UNSUPPORTED, "weights at levels 1 and 2 need bf16, chunk 4 and 3..8 levels");
  if (c->leaf_form == ZHA_LEAF_WEIGHTS &&
      (c->kv_dtype != ZHA_BF16 || (c->chunk != 4 && c->chunk != 8 && c->chunk != 16)))
    return fail(ZHA_ERR_UNSUPPORTED, "the leaf weights form needs bf16 and chunk 4, 8 or 16");
  if (c->g_dtype != ZHA_G_KV && c->g_dtype != ZHA_G_FP8 && c->g_dtype != ZHA_G_FP4)
    return fail(ZHA_ERR_ARG, "g_dtype %d unknown", c->g_dtype);
  if (c->g_dtype == ZHA_G_FP8 && c->kv_dtype != ZHA_BF16)
    return fail(ZHA_ERR_UNSUPPORTED, "fp8 g needs bf16 keys");
  if (c->g_dtype == ZHA_G_FP4 && (c->kv_dtype != ZHA_BF16 || c->head_dim != 128 || c->leaf_form != ZHA_LEAF_WEIGHTS2))
    return fail(ZHA_ERR_UNSUPPORTED, "MXFP4 g needs bf16 keys, head_dim 128 and levels 1-2 held as weights");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(ZHA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", c->head_dim);
  if (c->n_ref > 16) return fail(ZHA_ERR_UNSUPPORTED, "n_ref %d unsupported (1..16)", c->n_ref);
  if (!is_pow2(c->chunk) || c->chunk > 256)
    return fail(ZHA_ERR_UNSUPPORTED, "chunk %d unsupported (power of two <= 256)", c->chunk);
  if (c->levels > ZHA_MAX_LEVELS)
    return fail(ZHA_ERR_UNSUPPORTED, "levels %d unsupported (<= %d)", c->levels, ZHA_MAX_LEVELS);
  int64_t span = 1;
  for (int l = 0; l < c->levels; ++l) span *= c->chunk;
  if (span > (int64_t(1) << 24))
    return fail(ZHA_ERR_UNSUPPORTED, "chunk^levels = %lld exceeds 2^24", (long long)span);
  if (c->chunk > 16 && c->levels > 4)
    return fail(ZHA_ERR_UNSUPPORTED, "chunk > 16 supports at most 4 levels");
  if (c->capacity_tokens > (int64_t(1) << 36)) return fail(ZHA_ERR_UNSUPPORTED, "capacity too large");
  if ((int64_t)c->batch * c->n_kv_heads > 65535)
    return fail(ZHA_ERR_UNSUPPORTED, "batch * n_kv_heads must be <= 65535");
  return ZHA_OK;
}

int check_T(const zha_config* c, int32_t T) {
  if (T < 1) return fail(ZHA_ERR_ARG, "T must be >= 1");
  if ((int64_t)c->q_per_kv * T > 1024) return fail(ZHA_ERR_UNSUPPORTED, "q_per_kv * T must be <= 1024");
  return ZHA_OK;
}

int check_ptr16(const void* p, const char* name) {
  if (!p) return fail(ZHA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16) return fail(ZHA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return ZHA_OK;
}

int check_strides(const int64_t* s, int n, int es, const char* name) {
  if (!s) return fail(ZHA_ERR_NULL, "%s is NULL", name);
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(ZHA_ERR_ARG, "%s[%d] is negative", name, i);
    if ((s[i] * es) % 16) return fail(ZHA_ERR_ALIGN, "%s[%d] * element size is not a multiple of 16", name, i);
  }
  return ZHA_OK;
}

// Keys per node of level index l when routing scores that level from its
// keys (level 1 in both weights forms, which store the weights of the C
// keys; level 2 in ZHA_LEAF_WEIGHTS2, which stores its C children's mass
// shares), else 0.
static int weight_keys(const zha_config* c, int l) {
  if (l == 0 && (c->leaf_form == ZHA_LEAF_WEIGHTS || c->leaf_form == ZHA_LEAF_WEIGHTS2)) return c->chunk;
  if (l == 1 && c->leaf_form == ZHA_LEAF_WEIGHTS2) return c->chunk * c->chunk;
  return 0;
}

// Appends split each top span over its C children when the top has at least
// two levels below it and C is in 4..16 (the sub-span pass uses 4 waves).
static bool split_top(const zha_config* c) { return c->levels >= 3 && c->chunk >= 4 && c->chunk <= 16; }

void fill_tree_layout(const zha_config* c, zha_tree_layout* out) {
  std::memset(out, 0, sizeof(*out));
  out->levels = c->levels;
  const int64_t caches = (int64_t)c->batch * c->n_kv_heads;
  int64_t n = c->capacity_tokens / c->chunk;
  int64_t off = 0;
  for (int l = 0; l < c->levels; ++l) {
    if (l > 0) n = cdiv(n, c->chunk);
    const int wk = weight_keys(c, l);
    const bool fp8 = wk == 0 && c->g_dtype == ZHA_G_FP8;
    const bool fp4 = wk == 0 && c->g_dtype == ZHA_G_FP4;
    // weights [R][wk] fp32, or at level 2 of ZHA_LEAF_WEIGHTS2 the child shares [R][C]
    out->g_bytes[l] = wk    ? (int64_t)c->n_ref * (l == 1 ? c->chunk : wk) * 4
                      : fp4 ? (int64_t)c->n_ref * c->head_dim / 2
                            : (int64_t)c->n_ref * c->head_dim * (fp8 ? 1 : esize(c->kv_dtype));
    out->node_cap[l] = n;
    out->g_offset[l] = off;
    off = align256(off + caches * n * out->g_bytes[l]);
    out->L_offset[l] = off;
    off = align256(off + caches * n * c->n_ref * 4);
    out->c_offset[l] = off;
    off = align256(off + caches * n * c->n_ref * 4);
    out->s_offset[l] = -1;
    if (fp8 || fp4) {  // fp32 row scales, or one E8M0 byte per 32 elements of a row
      out->s_offset[l] = off;
      off = align256(off + caches * n * c->n_ref * (fp8 ? 4 : c->head_dim / 32));
    }
  }
  for (int l = c->levels; l < ZHA_MAX_LEVELS; ++l) out->s_offset[l] = -1;
  out->scratch_offset = -1;
  if (split_top(c)) {
    out->scratch_offset = off;
    off = align256(off + caches * 2 * c->chunk * (int64_t)c->n_ref * (c->head_dim + 2) * 4);
  }
  out->ref_offset = -1;
  if (weight_keys(c, 1)) {
    out->ref_offset = off;
    off = align256(off + (int64_t)c->n_kv_heads * c->n_ref * c->head_dim * 4);
  }
  out->total_bytes = off > 0 ? off : 256;
}

void fill_geom(const zha_config* c, const zha_tree_layout& tl, zha::TreeGeom* g) {
  std::memset(g, 0, sizeof(*g));
  g->levels = c->levels;
  g->R = c->n_ref;
  g->D = c->head_dim;
  g->C = c->chunk;
  g->esize = esize(c->kv_dtype);
  g->H = c->n_kv_heads;
  g->caches = c->batch * c->n_kv_heads;
  g->leaf_weights = weight_keys(c, 0) != 0;
  g->w2 = weight_keys(c, 1) != 0;
  for (int l = 0; l < c->levels; ++l) {
    g->node_cap[l] = tl.node_cap[l];
    g->g_off[l] = tl.g_offset[l];
    g->L_off[l] = tl.L_offset[l];
    g->c_off[l] = tl.c_offset[l];
    g->s_off[l] = tl.s_offset[l];
    if (tl.s_offset[l] >= 0) {
      if (c->g_dtype == ZHA_G_FP4)
        g->g4 |= 1u << l;
      else
        g->g8 |= 1u << l;
    }
  }
  g->span_len[0] = 1;
  for (int l = 1; l <= c->levels; ++l) g->span_len[l] = g->span_len[l - 1] * c->chunk;
}

// node counts per level for n tokens
void level_sizes(const zha_config* c, int64_t n_tokens, int64_t* n) {
  n[0] = n_tokens / c->chunk;
  for (int l = 1; l < c->levels; ++l) n[l] = cdiv(n[l - 1], c->chunk);
}

// Keys per attention workgroup, fixed per configuration (from the capacity) so
// that the workspace bound holds for every n_tokens: tiles of >= 256 keys and
// enough workgroups to fill 256 CUs several times at full capacity.
int64_t attend_tile_keys(const zha_config* c, int32_t T) {
  const int64_t caches = (int64_t)c->batch * c->n_kv_heads;
  const int64_t groups = cdiv((int64_t)c->q_per_kv * T, 4);
  int64_t tk = 256;
  while (tk < 8192 && caches * groups * cdiv(c->capacity_tokens, tk * 2) >= 2048) tk *= 2;
  return tk;
}

int64_t attend_ws(const zha_config* c, int32_t T) {
  const int64_t nq = (int64_t)c->batch * c->n_kv_heads * c->q_per_kv * T;
  const int64_t tk = attend_tile_keys(c, T);
  return align256(nq * cdiv(c->capacity_tokens, tk) * (c->head_dim + 2) * 4);
}

// Cut-bin candidates the one-workgroup select resolves in LDS (1536, its
// list size).  The ZHA_SELECT_CUT_CAP environment variable lowers it (0
// makes every level take the radix passes), so that tests can check that
// both ways reach the same bits.
int select_cut_cap() {
  const char* e = std::getenv("ZHA_SELECT_CUT_CAP");
  if (!e || !*e) return 1536;
  const long v = std::strtol(e, nullptr, 10);
  return v < 0 ? 0 : (v > 1536 ? 1536 : (int)v);
}

int check_prof(zha_profile* prof) {
  if (!prof) return ZHA_OK;
  if (prof->n_pairs < 0 || prof->n_pairs > ZHA_PROFILE_MAX)
    return fail(ZHA_ERR_ARG, "prof->n_pairs must be in [0, %d]", ZHA_PROFILE_MAX);
  for (int i = 0; i < 2 * prof->n_pairs; ++i)
    if (!prof->events[i]) return fail(ZHA_ERR_NULL, "prof->events[%d] is NULL", i);
  return ZHA_OK;
}

// Trees built by k_build_mf: bf16 keys, R <= 16, and a 64-key round's node
// at a level of the tree: chunk 4 with 3..8 levels (the round's node is
// level 3) or chunk 8 with 2..7 levels (level 2); g in bf16, or in fp8 when
// levels 1 and 2 are held as weights (fp8 then starts at the round's level).
static bool build_mf(const zha_config* c) {
  if (c->kv_dtype != ZHA_BF16 || c->n_ref > 16) return false;
  if (c->g_dtype != ZHA_G_KV && c->leaf_form != ZHA_LEAF_WEIGHTS2) return false;
  if (c->chunk == 4) return c->levels >= 3 && c->levels <= 8;
  if (c->chunk == 8) return c->levels >= 2 && c->levels <= 7;
  return false;
}

int do_build(const zha_config* cfg, const void* K, const int64_t* ks, int64_t n_old, int64_t n_new,
             const float* ref, void* tree, zha_profile* prof, void* stream, bool append) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_prof(prof))) return rc;
  if (prof) prof->n_used = 0;
  if ((rc = check_ptr16(K, "K"))) return rc;
  if ((rc = check_strides(ks, 3, esize(cfg->kv_dtype), "k_strides"))) return rc;
  if ((rc = check_ptr16(ref, "ref"))) return rc;
  if ((rc = check_ptr16(tree, "tree"))) return rc;
  if (n_old < 0 || n_new < 0) return fail(ZHA_ERR_ARG, "token counts must be >= 0");
  if (n_old + n_new > cfg->capacity_tokens)
    return fail(ZHA_ERR_CAPACITY, "%lld tokens exceed capacity %lld", (long long)(n_old + n_new),
                (long long)cfg->capacity_tokens);
  zha_tree_layout tl;
  fill_tree_layout(cfg, &tl);
  zha::BuildArgs a;
  std::memset(&a, 0, sizeof(a));
  a.K = K;
  a.sb = ks[0];
  a.sh = ks[1];
  a.st = ks[2];
  a.ref = ref;
  a.tree = static_cast<char*>(tree);
  fill_geom(cfg, tl, &a.geo);
  a.n_tokens = n_old + n_new;
  a.span_tokens = a.geo.span_len[cfg->levels];
  a.inv_sqrt_d = 1.0f / std::sqrt((float)cfg->head_dim);
  const int64_t C = cfg->chunk;
  const int64_t end_c = ((n_old + n_new) / C) * C;  // complete-chunk boundary after the call
  if (append) {
    const int64_t old_c = (n_old / C) * C;
    if (end_c <= old_c) return ZHA_OK;  // no new complete chunk: the tree is unchanged
    a.first_span = old_c / a.span_tokens;
    a.n_spans = cdiv(end_c, a.span_tokens) - a.first_span;
  } else {
    a.first_span = 0;
    a.n_spans = cdiv(end_c, a.span_tokens);
  }
  if (a.n_spans <= 0) return ZHA_OK;
  if (a.n_spans > 0x7fffffffll) return fail(ZHA_ERR_UNSUPPORTED, "too many spans");
  zha::Prof pr{prof, static_cast<hipStream_t>(stream)};
  if (tl.ref_offset >= 0) {
    // the reference queries travel with the tree (routing recomputes weights from them)
    hipError_t e = hipMemcpyAsync(static_cast<char*>(tree) + tl.ref_offset, ref,
                                  (size_t)cfg->n_kv_heads * cfg->n_ref * cfg->head_dim * 4, hipMemcpyDeviceToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "reference copy");
  }
  a.top_level = cfg->levels;
  a.mf = build_mf(cfg);
  // on the matrix-core path the split's sub-span pass must itself reach the
  // round's level (3 for chunk 4, 2 for chunk 8)
  if (append && a.n_spans <= 2 && tl.scratch_offset >= 0 && (!a.mf || cfg->levels >= (C == 4 ? 4 : 3))) {
    // few spans: build their children in parallel, then merge the top nodes
    zha::BuildArgs s1 = a;
    s1.top_level = cfg->levels - 1;
    s1.span_tokens = a.span_tokens / C;
    s1.first_span = a.first_span * C;
    s1.n_spans = a.n_spans * C;
    s1.top_scratch = reinterpret_cast<float*>(static_cast<char*>(tree) + tl.scratch_offset);
    s1.scratch_span0 = a.first_span;
    hipError_t e = zha::launch_build(s1, cfg->kv_dtype, pr);
    if (e != hipSuccess) return hip_fail(e, "build launch");
    zha::BuildArgs s2 = a;
    s2.merge_top = 1;
    s2.top_scratch = s1.top_scratch;
    s2.scratch_span0 = a.first_span;
    e = zha::launch_build(s2, cfg->kv_dtype, pr);
    if (e != hipSuccess) return hip_fail(e, "build launch");
    return ZHA_OK;
  }
  hipError_t e = zha::launch_build(a, cfg->kv_dtype, pr);
  if (e != hipSuccess) return hip_fail(e, "build launch");
  return ZHA_OK;
}

// Scratch of zha_attend_noalloc: one static array per GPU (each device
// holds its own copy at its own address from the library's first use of it
// until the process ends).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per
// device, with that device current, and is kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[ZHA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the calling thread's current device, which must be
// the device of `stream` (NULL = the current device's default stream).
int scratch_on_current_device(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ZHA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  if (stream) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sd != dev) return fail(ZHA_ERR_ARG, "stream belongs to device %d, the current device is %d", (int)sd, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(ZHA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ZHA_OK;
}

}  // namespace

extern "C" {

int zha_version(void) { return ZHA_VERSION; }

const char* zha_status_string(int s) {
  switch (s) {
    case ZHA_OK:
      return "ok";
    case ZHA_ERR_NULL:
      return "null pointer";
    case ZHA_ERR_ARG:
      return "invalid argument";
    case ZHA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case ZHA_ERR_CAPACITY:
      return "capacity exceeded or buffer too small";
    case ZHA_ERR_ALIGN:
      return "misaligned pointer or stride";
    case ZHA_ERR_HIP:
      return "HIP error";
    default:
      return "unknown status";
  }
}

const char* zha_last_error(void) { return g_err; }

int zha_get_tree_layout(const zha_config* cfg, zha_tree_layout* out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(ZHA_ERR_NULL, "out is NULL");
  fill_tree_layout(cfg, out);
  return ZHA_OK;
}

// Queries per row of the logits buffer: QC rounded up to 4, at most 16.
static int logits_row(int64_t QC) { return QC >= 16 ? 16 : (int)((QC + 3) / 4 * 4); }

// Key-range slots of every level: offsets (in uint32 units) into the route
// workspace when `off` is given; returns the bytes needed.
static int64_t kr_total(const zha_config* cfg, const zha_tree_layout& tl, int64_t n_queries, int64_t* off) {
  int64_t words = 0;
  for (int l = 0; l < cfg->levels; ++l) {
    const int wk = weight_keys(cfg, l);
    if (off) off[l] = words;
    words += n_queries * zha::route_kr_slots(cfg->kv_dtype, wk != 0, tl.node_cap[l], wk) * 4;
  }
  return words * 4;
}

int zha_get_route_layout(const zha_config* cfg, int32_t T, zha_route_layout* out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_T(cfg, T))) return rc;
  if (!out) return fail(ZHA_ERR_NULL, "out is NULL");
  zha_tree_layout tl;
  fill_tree_layout(cfg, &tl);
  std::memset(out, 0, sizeof(*out));
  out->levels = cfg->levels;
  out->n_queries = (int64_t)cfg->batch * cfg->n_kv_heads * cfg->q_per_kv * T;
  int64_t sw = 0, sf = 0, ss = 0;
  for (int l = 0; l < cfg->levels; ++l) {
    out->words[l] = cdiv(tl.node_cap[l], 32);
    out->sel_offset[l] = sw;
    sw += out->n_queries * out->words[l];
    out->score_offset[l] = sf;
    out->score_stride[l] = (tl.node_cap[l] + 3) / 4 * 4;
    sf += out->n_queries * out->score_stride[l];
    out->stats_offset[l] = ss;
    ss += out->n_queries;
  }
  out->sel_words_total = sw > 0 ? sw : 1;
  out->score_floats_total = sf > 0 ? sf : 1;
  out->stats_total = ss;
  // per level, query and score tile: candidate key range and count, written
  // by the score kernel and reduced by the select kernel
  // (the select kernels' split form uses the bytes after them)
  out->workspace_min_bytes = align256(kr_total(cfg, tl, out->n_queries, nullptr));
  out->workspace_bytes =
      out->workspace_min_bytes + align256(zha::select_split_bytes(out->n_queries, tl.node_cap[0]));
  if (weight_keys(cfg, 0)) {
    const int64_t QC = (int64_t)cfg->q_per_kv * T;
    out->logits_floats = (int64_t)cfg->batch * cfg->n_kv_heads * cdiv(QC, 16) *
                         (tl.node_cap[0] * cfg->chunk / 4) * 4 * logits_row(QC);
  }
  return ZHA_OK;
}

int64_t zha_attend_workspace_bytes(const zha_config* cfg, int32_t T) {
  if (check_config(cfg) || check_T(cfg, T)) return -1;
  return attend_ws(cfg, T);
}

int64_t zha_tree_bytes(const zha_config* cfg) {
  zha_tree_layout tl;
  const int rc = zha_get_tree_layout(cfg, &tl);
  return rc ? rc : tl.total_bytes;
}

int64_t zha_route_workspace_bytes(const zha_config* cfg, int32_t T) {
  zha_route_layout rl;
  const int rc = zha_get_route_layout(cfg, T, &rl);
  return rc ? rc : rl.workspace_bytes;
}

int64_t zha_dense_workspace_bytes(const zha_config* cfg, int32_t T) { return zha_attend_workspace_bytes(cfg, T); }

int zha_build(const zha_config* cfg, const void* K, const int64_t k_strides[3], int64_t n_tokens,
              const float* ref, void* tree, zha_profile* prof, void* stream) {
  return do_build(cfg, K, k_strides, 0, n_tokens, ref, tree, prof, stream, false);
}

int zha_append(const zha_config* cfg, const void* K, const int64_t k_strides[3], int64_t n_old,
               int64_t n_new, const float* ref, void* tree, zha_profile* prof, void* stream) {
  return do_build(cfg, K, k_strides, n_old, n_new, ref, tree, prof, stream, true);
}

// Prefill spine geometry for blocks of up to T query positions: snapshot
// states k (complete chunks of a query's prefix) per cache, and bytes per
// record (one node: g block, then L, c and scale, R fp32 each).
static int64_t spine_states(const zha_config* c, int32_t T) { return (int64_t)T / c->chunk + 2; }
static int64_t spine_rec_bytes(const zha_config* c) {
  const int64_t g = (int64_t)c->n_ref * c->head_dim * (c->g_dtype == ZHA_G_FP8 ? 1 : esize(c->kv_dtype));
  return (g + 12 * c->n_ref + 15) / 16 * 16;
}

static int do_route(const zha_config* cfg, const void* tree, int64_t n_tokens, const void* Q,
                    const int64_t q_strides[4], int32_t T, const float* pl, int32_t top_level, const void* K,
                    const int64_t k_strides[3], uint32_t* sel, float* score, zha_select_stats* stats,
                    float* logits, void* ws, int64_t ws_bytes, zha_profile* prof, void* stream,
                    bool prefill = false, const void* spine = nullptr) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_prof(prof))) return rc;
  if ((rc = check_T(cfg, T))) return rc;
  if ((rc = check_ptr16(tree, "tree"))) return rc;
  if ((rc = check_ptr16(Q, "Q"))) return rc;
  if ((rc = check_strides(q_strides, 4, esize(cfg->kv_dtype), "q_strides"))) return rc;
  const bool leafw = weight_keys(cfg, 0) != 0;
  if (leafw) {
    if ((rc = check_ptr16(K, "K"))) return rc;
    if ((rc = check_strides(k_strides, 3, esize(cfg->kv_dtype), "k_strides"))) return rc;
  }
  if (logits) {
    if (!leafw) return fail(ZHA_ERR_ARG, "logits need a leaf weights form");
    if ((rc = check_ptr16(logits, "logits"))) return rc;
  }
  if ((rc = check_ptr16(sel, "sel"))) return rc;
  if ((rc = check_ptr16(score, "score"))) return rc;
  if ((rc = check_ptr16(stats, "stats"))) return rc;
  if (!pl) return fail(ZHA_ERR_NULL, "p_levels is NULL");
  for (int l = 0; l < cfg->levels; ++l)
    if (!(pl[l] > 0.0f) || std::isnan(pl[l])) return fail(ZHA_ERR_ARG, "p of level %d must be in (0, 1]", l + 1);
  if (top_level < 0 || top_level > cfg->levels)
    return fail(ZHA_ERR_ARG, "top_level %d outside 0..%d", top_level, cfg->levels);
  const int top = top_level == 0 ? cfg->levels : top_level;
  if (n_tokens < 0) return fail(ZHA_ERR_ARG, "n_tokens must be >= 0");
  if (n_tokens > cfg->capacity_tokens) return fail(ZHA_ERR_CAPACITY, "n_tokens exceeds capacity");
  if (prefill) {
    if (cfg->leaf_form == ZHA_LEAF_WEIGHTS2)
      return fail(ZHA_ERR_UNSUPPORTED, "prefill routing does not take level-2 weights");
    if (cfg->levels >= 2 && (rc = check_ptr16(spine, "spine"))) return rc;
    if (cfg->kv_dtype != ZHA_BF16) return fail(ZHA_ERR_UNSUPPORTED, "prefill routing needs bf16 keys");
    if (T > n_tokens) return fail(ZHA_ERR_ARG, "T = %d positions exceed n_tokens", T);
  }
  zha_route_layout rl;
  zha_get_route_layout(cfg, T, &rl);
  if ((rc = check_ptr16(ws, "ws"))) return rc;
  if (ws_bytes < rl.workspace_min_bytes) return fail(ZHA_ERR_CAPACITY, "workspace too small");
  zha_tree_layout tl;
  fill_tree_layout(cfg, &tl);
  int64_t n[ZHA_MAX_LEVELS];
  level_sizes(cfg, n_tokens, n);
  const int caches = cfg->batch * cfg->n_kv_heads;
  const float isd = 1.0f / std::sqrt((float)cfg->head_dim);
  if (prof) prof->n_used = 0;
  zha::Prof pr{prof, static_cast<hipStream_t>(stream)};
  uint32_t* keyrange = static_cast<uint32_t*>(ws);
  int64_t kr_off[ZHA_MAX_LEVELS];
  const int64_t kr_bytes = kr_total(cfg, tl, rl.n_queries, kr_off);
  void* split = rl.workspace_bytes > rl.workspace_min_bytes && ws_bytes >= rl.workspace_bytes
                    ? static_cast<void*>(static_cast<char*>(ws) + rl.workspace_min_bytes)
                    : nullptr;
  // levels 1-2 as weights, level 2 scored in this call and at most 4 queries
  // per cache: the level-2 pass also writes the level-1 scores (and the
  // logits attention reads), and level 1 only masks them by the kept parents
  const bool fuse1 = weight_keys(cfg, 1) && top >= 2 && (int64_t)cfg->q_per_kv * T <= 4;
  if (cfg->kv_dtype != ZHA_BF16) {
    // the fp32 score kernel accumulates its single slot per query with atomics
    hipError_t e = zha::launch_route_init(keyrange, kr_bytes / 16, pr);
    if (e != hipSuccess) return hip_fail(e, "route init launch");
  }
  for (int l = top - 1; l >= 0; --l) {
    zha::ScoreArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.g = static_cast<const char*>(tree) + tl.g_offset[l];
    sa.c = reinterpret_cast<const float*>(static_cast<const char*>(tree) + tl.c_offset[l]);
    sa.gscale = tl.s_offset[l] >= 0
                    ? reinterpret_cast<const float*>(static_cast<const char*>(tree) + tl.s_offset[l])
                    : nullptr;
    sa.gfmt = tl.s_offset[l] < 0 ? 0 : (cfg->g_dtype == ZHA_G_FP4 ? 2 : 1);
    sa.node_cap = tl.node_cap[l];
    sa.n_nodes = n[l];
    sa.R = cfg->n_ref;
    sa.C = cfg->chunk;
    sa.D = cfg->head_dim;
    sa.H = cfg->n_kv_heads;
    sa.G = cfg->q_per_kv;
    sa.T = T;
    sa.QC = cfg->q_per_kv * T;
    sa.Q = Q;
    sa.qsb = q_strides[0];
    sa.qsh = q_strides[1];
    sa.qsg = q_strides[2];
    sa.qst = q_strides[3];
    sa.sel_parent = (l == top - 1) ? nullptr : sel + rl.sel_offset[l + 1];
    sa.parent_words = (l == top - 1) ? 0 : rl.words[l + 1];
    sa.score = score + rl.score_offset[l];
    sa.score_stride = rl.score_stride[l];
    sa.keyrange = keyrange + kr_off[l];
    sa.kr_slots = zha::route_kr_slots(cfg->kv_dtype, weight_keys(cfg, l) != 0, tl.node_cap[l], weight_keys(cfg, l));
    sa.inv_sqrt_d = isd;
    sa.causal_n0 = prefill ? n_tokens - T : -1;
    sa.lvl_chunks = 1;
    for (int i = 0; i < l; ++i) sa.lvl_chunks *= cfg->chunk;
    sa.levels = cfg->levels;
    sa.level = l + 1;
    sa.top = top;
    sa.n_queries = rl.n_queries;
    if (prefill && spine) {
      sa.spine = static_cast<const char*>(spine);
      sa.spine_k0 = (n_tokens - T + 1) / cfg->chunk;
      sa.spine_states = spine_states(cfg, T);
      sa.spine_rec = spine_rec_bytes(cfg);
    }
    sa.wkeys = weight_keys(cfg, l);
    sa.leaf_weights = sa.wkeys != 0;
    if (sa.leaf_weights) {
      sa.K = K;
      sa.ksb = k_strides[0];
      sa.ksh = k_strides[1];
      sa.kst = k_strides[2];
      sa.n_keys = n[0] * cfg->chunk;
      // the logits are written by level 1, or by level 2 when it is fused
      sa.logits = (l == 0) != fuse1 ? logits : nullptr;
      sa.fuse1 = l == 0 && fuse1;
      sa.nquads = tl.node_cap[0] * cfg->chunk / 4;
      sa.QW = logits_row(sa.QC);
      if (l == 1) {  // level 2 holding child shares: the level-1 rows it reads (and fills)
        sa.ref = reinterpret_cast<const float*>(static_cast<const char*>(tree) + tl.ref_offset);
        sa.w1 = reinterpret_cast<const float*>(static_cast<const char*>(tree) + tl.g_offset[0]);
        sa.c1 = reinterpret_cast<const float*>(static_cast<const char*>(tree) + tl.c_offset[0]);
        sa.node_cap1 = tl.node_cap[0];
        sa.score1 = fuse1 ? score + rl.score_offset[0] : nullptr;
        sa.score1_stride = rl.score_stride[0];
      }
    }
    zha::SelectArgs se;
    std::memset(&se, 0, sizeof(se));
    se.score = sa.score;
    se.score_stride = sa.score_stride;
    se.keyrange = sa.keyrange;
    se.kr_slots = sa.kr_slots;
    se.n_nodes = n[l];
    se.sel = sel + rl.sel_offset[l];
    se.words = rl.words[l];
    se.stats = stats + rl.stats_offset[l];
    se.p = pl[l];
    se.keep_all = pl[l] >= 1.0f;
    se.split = split;
    // decode levels below the start: children of dropped parents hold -inf
    // and need not be read (prefill rows also hold each query's partial node)
    se.sel_parent = (!prefill && cfg->chunk >= 4) ? sa.sel_parent : nullptr;
    se.parent_words = sa.parent_words;
    se.C = cfg->chunk;
    se.cut_cap = select_cut_cap();
    hipError_t e = zha::launch_route_level(sa, se, cfg->kv_dtype, caches, l + 1, pr);
    if (e != hipSuccess) return hip_fail(e, "route launch");
  }
  return ZHA_OK;
}

int zha_route(const zha_config* cfg, const void* tree, int64_t n_tokens, const void* Q,
              const int64_t q_strides[4], int32_t T, float p, const void* K,
              const int64_t k_strides[3], uint32_t* sel, float* score,
              zha_select_stats* stats, float* logits, void* ws, int64_t ws_bytes,
              zha_profile* prof, void* stream) {
  float pl[ZHA_MAX_LEVELS];
  for (int l = 0; l < ZHA_MAX_LEVELS; ++l) pl[l] = p;
  return do_route(cfg, tree, n_tokens, Q, q_strides, T, pl, 0, K, k_strides, sel, score, stats, logits, ws,
                  ws_bytes, prof, stream);
}

int64_t zha_spine_bytes(const zha_config* cfg, int32_t T) {
  if (check_config(cfg) || check_T(cfg, T)) return -1;
  if (cfg->levels < 2) return 256;
  return align256((int64_t)cfg->batch * cfg->n_kv_heads * spine_states(cfg, T) * (cfg->levels - 1) *
                  spine_rec_bytes(cfg));
}

int zha_build_spine(const zha_config* cfg, const void* K, const int64_t k_strides[3], int64_t n_tokens,
                    int32_t T, const float* ref, void* spine, zha_profile* prof, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_T(cfg, T))) return rc;
  if ((rc = check_prof(prof))) return rc;
  if (prof) prof->n_used = 0;
  if (cfg->kv_dtype != ZHA_BF16) return fail(ZHA_ERR_UNSUPPORTED, "prefill needs bf16 keys");
  if (cfg->leaf_form == ZHA_LEAF_WEIGHTS2)
    return fail(ZHA_ERR_UNSUPPORTED, "the prefill spine does not take level-2 weights");
  if ((rc = check_ptr16(K, "K"))) return rc;
  if ((rc = check_strides(k_strides, 3, esize(cfg->kv_dtype), "k_strides"))) return rc;
  if ((rc = check_ptr16(ref, "ref"))) return rc;
  if ((rc = check_ptr16(spine, "spine"))) return rc;
  if (n_tokens < T || n_tokens < 1) return fail(ZHA_ERR_ARG, "need 1 <= T <= n_tokens");
  if (n_tokens > cfg->capacity_tokens) return fail(ZHA_ERR_CAPACITY, "n_tokens exceeds capacity");
  if (cfg->levels < 2) return ZHA_OK;  // no node above the chunks: no spine
  zha_tree_layout tl;
  fill_tree_layout(cfg, &tl);
  zha::BuildArgs a;
  std::memset(&a, 0, sizeof(a));
  a.K = K;
  a.sb = k_strides[0];
  a.sh = k_strides[1];
  a.st = k_strides[2];
  a.ref = ref;
  a.tree = nullptr;
  fill_geom(cfg, tl, &a.geo);
  a.n_tokens = n_tokens;
  a.span_tokens = a.geo.span_len[cfg->levels];
  a.inv_sqrt_d = 1.0f / std::sqrt((float)cfg->head_dim);
  a.spine = static_cast<char*>(spine);
  a.spine_k0 = (n_tokens - T + 1) / cfg->chunk;
  a.spine_states = spine_states(cfg, T);
  a.spine_rec = spine_rec_bytes(cfg);
  a.top_level = cfg->levels;
  // states k0 .. k_end (complete chunks of n_tokens): the spans holding chunks k0-1 .. k_end-1
  const int64_t k_end = n_tokens / cfg->chunk;
  if (k_end < 1 || k_end < a.spine_k0) return ZHA_OK;
  const int64_t c_first = a.spine_k0 > 0 ? a.spine_k0 - 1 : 0;
  a.first_span = c_first * cfg->chunk / a.span_tokens;
  a.n_spans = (k_end - 1) * cfg->chunk / a.span_tokens - a.first_span + 1;
  zha::Prof pr{prof, static_cast<hipStream_t>(stream)};
  hipError_t e = zha::launch_build(a, cfg->kv_dtype, pr);
  if (e != hipSuccess) return hip_fail(e, "spine launch");
  return ZHA_OK;
}

int zha_route_prefill(const zha_config* cfg, const void* tree, const void* spine, int64_t n_tokens,
                      const void* Q, const int64_t q_strides[4], int32_t T, float p, const void* K,
                      const int64_t k_strides[3], uint32_t* sel, float* score, zha_select_stats* stats,
                      float* logits, void* ws, int64_t ws_bytes, zha_profile* prof, void* stream) {
  float pl[ZHA_MAX_LEVELS];
  for (int l = 0; l < ZHA_MAX_LEVELS; ++l) pl[l] = p;
  return do_route(cfg, tree, n_tokens, Q, q_strides, T, pl, 0, K, k_strides, sel, score, stats, logits, ws,
                  ws_bytes, prof, stream, true, spine);
}

int zha_route_levels(const zha_config* cfg, const void* tree, int64_t n_tokens, const void* Q,
                     const int64_t q_strides[4], int32_t T, const float* p_levels, int32_t top_level,
                     const void* K, const int64_t k_strides[3], uint32_t* sel, float* score,
                     zha_select_stats* stats, float* logits, void* ws, int64_t ws_bytes,
                     zha_profile* prof, void* stream) {
  return do_route(cfg, tree, n_tokens, Q, q_strides, T, p_levels, top_level, K, k_strides, sel, score, stats,
                  logits, ws, ws_bytes, prof, stream);
}

int zha_attend(const zha_config* cfg, const void* Q, const int64_t q_strides[4], int32_t T,
               const void* K, const void* V, const int64_t kv_strides[3], int64_t n_tokens,
               const uint32_t* sel1, int64_t sel1_words, const float* logits, uint32_t flags,
               float* out, float* lse, void* ws, int64_t ws_bytes, zha_profile* prof,
               void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_prof(prof))) return rc;
  if ((rc = check_T(cfg, T))) return rc;
  const int es = esize(cfg->kv_dtype);
  if ((rc = check_ptr16(Q, "Q"))) return rc;
  if ((rc = check_strides(q_strides, 4, es, "q_strides"))) return rc;
  if ((rc = check_ptr16(K, "K"))) return rc;
  if ((rc = check_ptr16(V, "V"))) return rc;
  if ((rc = check_strides(kv_strides, 3, es, "kv_strides"))) return rc;
  if ((rc = check_ptr16(out, "out"))) return rc;
  if ((rc = check_ptr16(ws, "ws"))) return rc;
  if (flags & ~15u) return fail(ZHA_ERR_ARG, "unknown flags 0x%x", flags);
  if (n_tokens < 1) return fail(ZHA_ERR_ARG, "n_tokens must be >= 1");
  if (flags & ZHA_CAUSAL) {
    if (cfg->kv_dtype != ZHA_BF16) return fail(ZHA_ERR_UNSUPPORTED, "causal attention needs bf16 keys");
    if (T > n_tokens) return fail(ZHA_ERR_ARG, "T = %d positions exceed n_tokens", T);
  }
  if (n_tokens > cfg->capacity_tokens) return fail(ZHA_ERR_CAPACITY, "n_tokens exceeds capacity");
  const int64_t n_chunks = n_tokens / cfg->chunk;
  if (logits) {
    if (!weight_keys(cfg, 0)) return fail(ZHA_ERR_ARG, "logits need a leaf weights form");
    if (flags & ZHA_ALL_KEYS) return fail(ZHA_ERR_ARG, "logits cannot be used with ZHA_ALL_KEYS");
    if ((rc = check_ptr16(logits, "logits"))) return rc;
  }
  if (!(flags & ZHA_ALL_KEYS)) {
    if (!sel1) return fail(ZHA_ERR_NULL, "sel1 is NULL");
    if (sel1_words < cdiv(n_chunks, 32)) return fail(ZHA_ERR_CAPACITY, "sel1_words too small");
  }
  const int64_t need = attend_ws(cfg, T);
  if (ws_bytes < need)
    return fail(ZHA_ERR_CAPACITY, "workspace %lld < %lld bytes", (long long)ws_bytes, (long long)need);
  zha::AttendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.qsb = q_strides[0];
  a.qsh = q_strides[1];
  a.qsg = q_strides[2];
  a.qst = q_strides[3];
  a.K = K;
  a.V = V;
  a.sb = kv_strides[0];
  a.sh = kv_strides[1];
  a.st = kv_strides[2];
  a.H = cfg->n_kv_heads;
  a.G = cfg->q_per_kv;
  a.T = T;
  a.QC = cfg->q_per_kv * T;
  a.C = cfg->chunk;
  a.D = cfg->head_dim;
  a.n_tokens = n_tokens;
  a.n_chunks = n_chunks;
  a.sel1 = (flags & ZHA_ALL_KEYS) ? nullptr : sel1;
  a.sel_words = sel1_words;
  a.flags = flags;
  a.tile_keys = attend_tile_keys(cfg, T);
  a.n_tiles = cdiv(n_tokens, a.tile_keys);
  a.partial = static_cast<float*>(ws);
  a.causal_n0 = (flags & ZHA_CAUSAL) ? n_tokens - T : -1;
  a.logits = logits;
  if (logits) {
    zha_tree_layout tl;
    fill_tree_layout(cfg, &tl);
    a.nquads = tl.node_cap[0] * cfg->chunk / 4;
    a.QW = logits_row(a.QC);
  }
  a.out = out;
  a.lse = lse;
  a.inv_sqrt_d = 1.0f / std::sqrt((float)cfg->head_dim);
  if (prof) prof->n_used = 0;
  zha::Prof pr{prof, static_cast<hipStream_t>(stream)};
  hipError_t e = zha::launch_attend(a, cfg->kv_dtype, cfg->batch * cfg->n_kv_heads, pr);
  if (e != hipSuccess) return hip_fail(e, "attend launch");
  return ZHA_OK;
}

int zha_attend_noalloc(const zha_config* cfg, const void* Q, const int64_t q_strides[4], int32_t T,
                       const void* K, const void* V, const int64_t kv_strides[3], int64_t n_tokens,
                       const uint32_t* sel1, int64_t sel1_words, const float* logits, uint32_t flags,
                       float* out, float* lse, zha_profile* prof, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_T(cfg, T))) return rc;
  const int64_t need = attend_ws(cfg, T);
  if (need > ZHA_NOALLOC_SCRATCH_BYTES)
    return fail(ZHA_ERR_CAPACITY,
                "zha_attend_noalloc: %lld bytes of split-K partials needed, the static scratch holds %lld "
                "(use zha_attend with a workspace)",
                (long long)need, (long long)ZHA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(stream, &ws))) return rc;
  return zha_attend(cfg, Q, q_strides, T, K, V, kv_strides, n_tokens, sel1, sel1_words, logits, flags, out, lse,
                    ws, ZHA_NOALLOC_SCRATCH_BYTES, prof, stream);
}

int zha_dense_decode(const zha_config* cfg, const void* Q, const int64_t q_strides[4], int32_t T,
                     const void* K, const void* V, const int64_t kv_strides[3], int64_t n_tokens,
                     float* out, float* lse, void* ws, int64_t ws_bytes, zha_profile* prof,
                     void* stream) {
  return zha_attend(cfg, Q, q_strides, T, K, V, kv_strides, n_tokens, nullptr, 0, nullptr, ZHA_ALL_KEYS,
                    out, lse, ws, ws_bytes, prof, stream);
}

int zha_stream_probe(int32_t mode, const void* src, void* dst, int64_t n_bytes, int64_t dst_bytes,
                     zha_profile* prof, void* stream) {
  int rc = check_prof(prof);
  if (rc) return rc;
  if (mode < ZHA_PROBE_READ || mode > ZHA_PROBE_TILE_MIX) return fail(ZHA_ERR_ARG, "probe mode %d unknown", mode);
  if (n_bytes < 64 || n_bytes % 64) return fail(ZHA_ERR_ARG, "n_bytes must be a positive multiple of 64");
  if ((rc = check_ptr16(src, "src"))) return rc;
  if ((rc = check_ptr16(dst, "dst"))) return rc;
  const bool read_only = mode <= ZHA_PROBE_READ_NT || mode == ZHA_PROBE_READ_SLAB || mode == ZHA_PROBE_READ_SLAB_NT;
  const int64_t need = read_only                    ? 16384
                       : mode <= ZHA_PROBE_COPY_NT  ? n_bytes
                       : mode == ZHA_PROBE_TILE_MIX ? (n_bytes / 16 + 15) / 16 * 16
                                                    : n_bytes / 4;
  if (dst_bytes < need)
    return fail(ZHA_ERR_CAPACITY, "dst holds %lld bytes, the probe writes up to %lld", (long long)dst_bytes,
                (long long)need);
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + dst_bytes && b < a + n_bytes) return fail(ZHA_ERR_ARG, "src and dst overlap");
  if (prof) prof->n_used = 0;
  zha::Prof pr{prof, static_cast<hipStream_t>(stream)};
  hipError_t e = zha::launch_probe(mode, src, dst, n_bytes, pr);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ZHA_OK;
}

int zha_selected_chunks(const uint32_t* sel1, int64_t sel1_words, int64_t n_queries, int64_t n_chunks,
                        int32_t* chunk_ids, int32_t* chunk_count, int64_t cap, void* stream) {
  if (!sel1) return fail(ZHA_ERR_NULL, "sel1 is NULL");
  if (!chunk_count) return fail(ZHA_ERR_NULL, "chunk_count is NULL");
  if (cap > 0 && !chunk_ids) return fail(ZHA_ERR_NULL, "chunk_ids is NULL");
  if ((reinterpret_cast<uintptr_t>(sel1) | reinterpret_cast<uintptr_t>(chunk_count) |
       reinterpret_cast<uintptr_t>(chunk_ids)) % 4)
    return fail(ZHA_ERR_ALIGN, "pointers must be 4-byte aligned");
  if (n_queries < 1 || n_queries > INT32_MAX) return fail(ZHA_ERR_ARG, "n_queries %lld out of range", (long long)n_queries);
  if (n_chunks < 0 || n_chunks > INT32_MAX) return fail(ZHA_ERR_ARG, "n_chunks %lld out of range", (long long)n_chunks);
  if (cap < 0) return fail(ZHA_ERR_ARG, "cap must be >= 0");
  if (sel1_words < cdiv(n_chunks, 32)) return fail(ZHA_ERR_CAPACITY, "sel1_words too small");
  hipError_t e = zha::launch_selected_chunks(sel1, sel1_words, n_queries, n_chunks, chunk_ids, chunk_count, cap,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selected-chunks launch");
  return ZHA_OK;
}

}  // extern "C"
