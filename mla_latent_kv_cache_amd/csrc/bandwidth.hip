// Streaming-read ceiling of the GPU's HBM: kernels that read a large buffer once, with 16-byte loads into
// registers or with 1 KB direct-to-LDS requests, and write (almost) nothing.  Its rate is the practical upper bound of an HBM-bound kernel such as the decode
// attention (which reads each cache row once), reported beside the vendor peak.  A measurement helper only:
// the latent-cache library does not use it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Each lane keeps UNROLL independent 16-byte loads in flight per iteration of a grid-stride loop over the
// buffer (non-temporal loads when NT); the loaded words are folded by xor into one value, which is stored only
// if it equals a constant that random data practically never gives (the store keeps the loads live; the write
// traffic is nil).
template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, size_t n, unsigned* sink,
                                                   unsigned magic) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= src[i];
  const unsigned a = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (a == magic) sink[blockIdx.x] = a;
}

// The same read through direct-to-LDS DMA (global_load_lds_dwordx4 with the non-temporal hint, the load path
// of the decode kernels): each wave streams 1 KB chunks w, w + W, ... (W = all waves of the grid) into an
// NF-slot ring of its own, keeping NF requests in flight; one workgroup of four waves per CU.  Nothing is
// written unless the last slot holds the magic word.
template <int NF>
__global__ __launch_bounds__(256, 1) void stream_dma(const char* __restrict__ src, size_t n_chunks, unsigned* sink,
                                                     unsigned magic) {
  __shared__ __attribute__((aligned(1024))) char ring[4 * NF * 1024];
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const size_t W = (size_t)gridDim.x * 4;
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)ring + w * NF * 1024;
  size_t k = 0;
  for (size_t g = (size_t)blockIdx.x * 4 + w; g < n_chunks; g += W, ++k) {
    const char* p = src + g * 1024;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"((uint32_t)(16 * lane)), "s"(p), "s"(base + (uint32_t)(k % NF) * 1024)
        : "memory");
    if (k + 1 >= NF) __builtin_amdgcn_s_waitcnt(0x0F70 | ((NF - 1) & 0xF) | (((NF - 1) >> 4) << 14));
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every request has landed
  __syncthreads();
  const unsigned v = *(const unsigned*)(ring + 16 * threadIdx.x);
  if (v == magic) sink[blockIdx.x] = v;
}

template <bool NT>
void launch_read(const u32x4* p, size_t n16, unsigned* sink, int blocks, int unroll, hipStream_t st) {
  switch (unroll) {
    case 1: hipLaunchKernelGGL((stream_read<1, NT>), dim3(blocks), dim3(256), 0, st, p, n16, sink, 0x9e3779b9u); break;
    case 2: hipLaunchKernelGGL((stream_read<2, NT>), dim3(blocks), dim3(256), 0, st, p, n16, sink, 0x9e3779b9u); break;
    case 4: hipLaunchKernelGGL((stream_read<4, NT>), dim3(blocks), dim3(256), 0, st, p, n16, sink, 0x9e3779b9u); break;
    default: hipLaunchKernelGGL((stream_read<8, NT>), dim3(blocks), dim3(256), 0, st, p, n16, sink, 0x9e3779b9u); break;
  }
}

}  // namespace

extern "C" {

// Read n16 16-byte words at src (16-byte aligned device memory) with `blocks` workgroups of 256 lanes,
// `unroll` in {1, 2, 4, 8} loads in flight per lane, non-temporal loads when `nontemporal`; sink [blocks]
// (device) receives at most a few words.  Returns 0, or -1 for bad arguments, -6 for a failed launch.
int mla_bw_stream_read(const void* src, size_t n16, unsigned* sink, int blocks, int unroll, int nontemporal,
                       hipStream_t stream) {
  if (!src || !sink || blocks <= 0 || ((uintptr_t)src & 15u) != 0) return -1;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return -1;
  const u32x4* p = (const u32x4*)src;
  if (nontemporal)
    launch_read<true>(p, n16, sink, blocks, unroll, stream);
  else
    launch_read<false>(p, n16, sink, blocks, unroll, stream);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// The same read through LDS DMA (see stream_dma): n1k 1 KB chunks at src (16-byte aligned device memory),
// `blocks` workgroups of four waves, `inflight` in {4, 8, 16} requests in flight per wave.  Returns 0, or -1 for
// bad arguments, -6 for a failed launch.
int mla_bw_stream_dma(const void* src, size_t n1k, unsigned* sink, int blocks, int inflight, hipStream_t stream) {
  if (!src || !sink || blocks <= 0 || ((uintptr_t)src & 15u) != 0) return -1;
  const char* p = (const char*)src;
  switch (inflight) {
    case 4: hipLaunchKernelGGL(stream_dma<4>, dim3(blocks), dim3(256), 0, stream, p, n1k, sink, 0x9e3779b9u); break;
    case 8: hipLaunchKernelGGL(stream_dma<8>, dim3(blocks), dim3(256), 0, stream, p, n1k, sink, 0x9e3779b9u); break;
    case 16: hipLaunchKernelGGL(stream_dma<16>, dim3(blocks), dim3(256), 0, stream, p, n1k, sink, 0x9e3779b9u); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
