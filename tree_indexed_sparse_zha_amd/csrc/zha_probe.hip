// Streaming probes: the HBM bandwidth plain access patterns reach on this
// GPU (the achievable ceiling each kernel's roofline fraction is read
// against) and a copy of known size that calibrates rocprofv3's byte
// counters.  Measurement only; no decode kernel uses them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "zha_internal.h"

namespace zha {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 4096;  // 16 workgroups per CU, grid-stride
constexpr int kUnroll = 4;          // 16-byte pieces in flight per thread

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool NT>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// Read-only stream: every 16-byte piece once; the loads of a step are all
// issued before their values are folded.  The fold is stored only if it
// hits a fixed pattern, so the loads stay live without a write stream.
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const u32x4* __restrict__ src, int64_t n16,
                                                              unsigned int* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  unsigned int acc = 0u;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load16<NT>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = load16<NT>(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// Read-only stream over contiguous slabs: workgroup b reads slab b
// (kSlabIters steps of 256 threads x kSlabUnroll pieces, each step one
// contiguous 32 KiB span), all loads of a step issued before their use.
constexpr int kSlabUnroll = 8;
constexpr int kSlabIters = 16;
constexpr int64_t kSlab16 = (int64_t)kProbeThreads * kSlabUnroll * kSlabIters;  // pieces per workgroup
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void k_probe_read_slab(const u32x4* __restrict__ src, int64_t n16,
                                                                   unsigned int* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kSlab16;
  unsigned int acc = 0u;
  for (int it = 0; it < kSlabIters; ++it) {
    const int64_t i0 = base + (int64_t)it * kProbeThreads * kSlabUnroll + threadIdx.x;
    u32x4 v[kSlabUnroll];
#pragma unroll
    for (int u = 0; u < kSlabUnroll; ++u) {
      const int64_t i = i0 + u * kProbeThreads;
      v[u] = i < n16 ? load16<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kSlabUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x & (kProbeBlocks - 1)] = acc;
}

// Copy over contiguous slabs (as k_probe_read_slab): every piece read once
// and written once, a step's loads all issued before its stores.
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void k_probe_copy(const u32x4* __restrict__ src, int64_t n16,
                                                              u32x4* __restrict__ dst) {
  const int64_t base = (int64_t)blockIdx.x * kSlab16;
  for (int it = 0; it < kSlabIters; ++it) {
    const int64_t i0 = base + (int64_t)it * kProbeThreads * kSlabUnroll + threadIdx.x;
    u32x4 v[kSlabUnroll];
#pragma unroll
    for (int u = 0; u < kSlabUnroll; ++u) {
      const int64_t i = i0 + u * kProbeThreads;
      v[u] = i < n16 ? load16<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kSlabUnroll; ++u) {
      const int64_t i = i0 + u * kProbeThreads;
      if (i < n16) store16<NT>(dst + i, v[u]);
    }
  }
}

// Read four pieces, write one (their xor) over contiguous slabs: a 4:1
// read/write byte mix, the mix of the scoring passes that read keys and
// write logits.  Workgroup b reads slab b of src and writes the matching
// quarter-size slab of dst.
template <bool NT_STORE>
__global__ __launch_bounds__(kProbeThreads) void k_probe_mix(const u32x4* __restrict__ src, int64_t n16,
                                                             u32x4* __restrict__ dst) {
  const int64_t base = (int64_t)blockIdx.x * kSlab16;
  for (int it = 0; it < kSlabIters; ++it) {
    const int64_t i0 = base + (int64_t)it * kProbeThreads * kSlabUnroll + threadIdx.x;
    u32x4 v[kSlabUnroll];
#pragma unroll
    for (int u = 0; u < kSlabUnroll; ++u) {
      const int64_t i = i0 + u * kProbeThreads;
      v[u] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
    // pieces u = 0..3 and 4..7 of the step fold into two output pieces
    const int64_t o0 = (base + (int64_t)it * kProbeThreads * kSlabUnroll) / 4 + threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t o = o0 + h * kProbeThreads;
      if (o < n16 / 4) store16<NT_STORE>(dst + o, v[4 * h] ^ v[4 * h + 1] ^ v[4 * h + 2] ^ v[4 * h + 3]);
    }
  }
}

// Tiles of 256 rows x 256 bytes (64 KiB), one per workgroup, loaded in the
// operand layout of the key-reading score passes (each load instruction
// covers 16 rows x 64 bytes; 16 pieces in flight per lane), folded, and one
// 16-byte piece written per 256 bytes read (nontemporal): the read/write
// mix and tile shape of the fused level-2 pass (4 KiB written per 64 KiB
// tile of keys).  Pieces past n16 read as zero.
__global__ __launch_bounds__(kProbeThreads) void k_probe_tile_mix(const u32x4* __restrict__ src, int64_t n16,
                                                                  u32x4* __restrict__ dst) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qn = lane & 15, kg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 4096;  // first piece of the tile
  u32x4 v[16];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t i = t0 + (int64_t)(64 * wave + 16 * gi + qn) * 16 + 4 * s + kg;
      v[4 * gi + s] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
  u32x4 x = v[0];
#pragma unroll
  for (int t = 1; t < 16; ++t) x ^= v[t];
  const int64_t o = (int64_t)blockIdx.x * kProbeThreads + tid;  // stands for pieces [16 o, 16 o + 16)
  if (16 * o < n16) __builtin_nontemporal_store(x, dst + o);
}

}  // namespace

hipError_t launch_probe(int mode, const void* src, void* dst, int64_t n_bytes, Prof& prof) {
  hipStream_t s = prof.s;
  const int64_t n16 = n_bytes / 16;
  const u32x4* in = static_cast<const u32x4*>(src);
  const int64_t slabs = (n16 + kSlab16 - 1) / kSlab16;  // workgroups of the slab forms
  if (slabs > 0x7fffffff) return hipErrorInvalidValue;
  prof.begin(ZHA_K_PROBE, mode);
  switch (mode) {
    case ZHA_PROBE_READ:
      hipLaunchKernelGGL(k_probe_read<false>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<unsigned int*>(dst));
      break;
    case ZHA_PROBE_READ_NT:
      hipLaunchKernelGGL(k_probe_read<true>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<unsigned int*>(dst));
      break;
    case ZHA_PROBE_READ_SLAB:
      hipLaunchKernelGGL(k_probe_read_slab<false>, dim3((unsigned)slabs), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<unsigned int*>(dst));
      break;
    case ZHA_PROBE_READ_SLAB_NT:
      hipLaunchKernelGGL(k_probe_read_slab<true>, dim3((unsigned)slabs), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<unsigned int*>(dst));
      break;
    case ZHA_PROBE_COPY:
      hipLaunchKernelGGL(k_probe_copy<false>, dim3((unsigned)slabs), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<u32x4*>(dst));
      break;
    case ZHA_PROBE_COPY_NT:
      hipLaunchKernelGGL(k_probe_copy<true>, dim3((unsigned)slabs), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<u32x4*>(dst));
      break;
    case ZHA_PROBE_MIX:
      hipLaunchKernelGGL(k_probe_mix<false>, dim3((unsigned)slabs), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<u32x4*>(dst));
      break;
    case ZHA_PROBE_MIX_NT:
      hipLaunchKernelGGL(k_probe_mix<true>, dim3((unsigned)slabs), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<u32x4*>(dst));
      break;
    case ZHA_PROBE_TILE_MIX: {
      const int64_t tiles = (n16 + 4095) / 4096;
      if (tiles > 0x7fffffff) return hipErrorInvalidValue;
      hipLaunchKernelGGL(k_probe_tile_mix, dim3((unsigned)tiles), dim3(kProbeThreads), 0, s, in, n16,
                         static_cast<u32x4*>(dst));
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  prof.end();
  return hipGetLastError();
}

}  // namespace zha
