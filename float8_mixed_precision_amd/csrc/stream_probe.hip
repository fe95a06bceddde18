// HBM streaming probes (measurement support, not a step of the method): the
// rates a plain kernel reaches when it only reads, only writes, or copies,
// with the access pattern the quantize kernels use (16-byte vector accesses,
// coalesced, several in flight per thread).  They are the practical ceilings
// the amax pass (read only) and the cast (read 2 B, write 2 B per element)
// are measured against, next to the chip's 8 TB/s.
//
// Each thread of a grid-stride loop handles UNROLL 16-byte vectors per
// round (consecutive threads on consecutive vectors, so a wave covers 1 KB
// per instruction); all UNROLL loads of a round are issued before any is
// used.  The index is clamped into the buffer and the value masked, so the
// loads carry no branch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int THREADS = 256;
constexpr int UNROLL = 8;
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// read: OR of every dword (stored per thread so it is not optimised away)
__global__ __launch_bounds__(THREADS) void k_read(const v4u *__restrict__ src, int64_t n16,
                                                  uint32_t *__restrict__ sink) {
  const int64_t per_round = (int64_t)gridDim.x * THREADS * UNROLL;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * THREADS * UNROLL + threadIdx.x; base < n16;
       base += per_round) {
    v4u v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * THREADS;
      v[u] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t keep = base + (int64_t)u * THREADS < n16 ? ~0u : 0u;
      acc |= (v[u].x | v[u].y | v[u].z | v[u].w) & keep;
    }
  }
  sink[(int64_t)blockIdx.x * THREADS + threadIdx.x] = acc;
}

// write: a constant pattern; NT: non-temporal stores
template <bool NT>
__global__ __launch_bounds__(THREADS) void k_write(v4u *__restrict__ dst, int64_t n16,
                                                   uint32_t pattern) {
  const int64_t per_round = (int64_t)gridDim.x * THREADS * UNROLL;
  const v4u v = (v4u){pattern, pattern ^ 1u, pattern ^ 2u, pattern ^ 3u};
  for (int64_t base = (int64_t)blockIdx.x * THREADS * UNROLL + threadIdx.x; base < n16;
       base += per_round) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * THREADS;
      if (i < n16) {
        if (NT)
          __builtin_nontemporal_store(v, dst + i);
        else
          dst[i] = v;
      }
    }
  }
}

// copy: src -> dst, all loads of a round before its stores
template <bool NT>
__global__ __launch_bounds__(THREADS) void k_copy(const v4u *__restrict__ src,
                                                  v4u *__restrict__ dst, int64_t n16) {
  const int64_t per_round = (int64_t)gridDim.x * THREADS * UNROLL;
  for (int64_t base = (int64_t)blockIdx.x * THREADS * UNROLL + threadIdx.x; base < n16;
       base += per_round) {
    v4u v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * THREADS;
      v[u] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * THREADS;
      if (i < n16) {
        if (NT)
          __builtin_nontemporal_store(v[u], dst + i);
        else
          dst[i] = v[u];
      }
    }
  }
}

}  // namespace

// kind: 0 read (src, sink = float-sized words, workgroups * 256 of them),
// 1 write (dst), 2 copy (src -> dst), 3 write non-temporal, 4 copy with
// non-temporal stores.  bytes: a multiple of 16; src / dst 16-byte aligned;
// workgroups >= 1.  Returns 0, 1 for a bad argument (nothing launched), 5
// for a launch failure.
extern "C" __attribute__((visibility("default"))) int fp8_probe_stream(
    int kind, const void *src, void *dst, int64_t bytes, int workgroups, void *sink,
    void *stream) {
  if (bytes <= 0 || (bytes & 15) || workgroups < 1) return 1;
  const bool reads = kind == 0 || kind == 2 || kind == 4;
  const bool writes = kind >= 1;
  if ((reads && (!src || (reinterpret_cast<uintptr_t>(src) & 15))) ||
      (writes && (!dst || (reinterpret_cast<uintptr_t>(dst) & 15))) || (kind == 0 && !sink))
    return 1;
  const int64_t n16 = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)workgroups), b(THREADS);
  const v4u *s = static_cast<const v4u *>(src);
  v4u *d = static_cast<v4u *>(dst);
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_read, g, b, 0, st, s, n16, static_cast<uint32_t *>(sink)); break;
    case 1: hipLaunchKernelGGL(k_write<false>, g, b, 0, st, d, n16, 0x3C3C3C3Cu); break;
    case 2: hipLaunchKernelGGL(k_copy<false>, g, b, 0, st, s, d, n16); break;
    case 3: hipLaunchKernelGGL(k_write<true>, g, b, 0, st, d, n16, 0x3C3C3C3Cu); break;
    case 4: hipLaunchKernelGGL(k_copy<true>, g, b, 0, st, s, d, n16); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
