// Device-side helpers shared by the gfx950 kernels of the latent-cache library.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l holds A[l%32][8(l/32)..+7], B[8(l/32)..+7][l%32];
// result element e of lane l is D[8(e/4) + 4(l/32) + e%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 MFMA.  Lane l holds A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16];
// result element e of lane l is D[4(l/16) + e][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 fp16 MFMA (same lane layout as mfma16).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j supplies the
// address of 4 consecutive 16-bit elements; lane i receives element (i % 4) of the chunks addressed
// by lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.  With lane j addressing row (r0 + j/4), columns
// (c0 + 4(j%4) .. +3) of a row-major tile, lane i receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Retained-pair index read from caller memory, clamped into [0, half) so that a bad table cannot
// make a kernel index outside the query row or the RoPE tables.
__device__ __forceinline__ int load_pair(const int32_t* pair_idx, int i, int half) {
  int p = pair_idx[i];
  return p < 0 ? 0 : (p >= half ? half - 1 : p);
}

// Workgroup barrier for LDS data exchanged between waves that does not wait for outstanding global or
// LDS-DMA loads (__syncthreads would, draining in-flight prefetches).  This wave's own LDS operations
// complete (lgkmcnt 0) before the barrier; the asm clobbers keep the compiler from moving memory
// accesses across it.  LDS written by DMA is waited for separately with vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// nope_idx[0 .. d_h-2r) = ascending dims of head h whose pair is not retained, built by the first wave
// of the workgroup from two 64-bit ballots (d_h/2 <= 128; kept[] is LDS scratch of d_h/2 ints).  The
// caller synchronises after the call.  Duplicate or out-of-range retained indices cannot push an entry
// outside [0, d_h).
__device__ __forceinline__ void build_nope_idx(const int32_t* pair_idx, int h, int r, int half, int* kept,
                                               int* nope_idx) {
  for (int i = threadIdx.x; i < half; i += blockDim.x) kept[i] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < r; j += blockDim.x) kept[load_pair(pair_idx, h * r + j, half)] = 1;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const bool k0 = l < half && kept[l], k1 = 64 + l < half && kept[64 + l];
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(k0), m1 = __builtin_amdgcn_ballot_w64(k1);
    const uint64_t below = l ? (~0ull >> (64 - l)) : 0ull;
    if (l < half && !k0) {
      const int pos = l - __builtin_popcountll(m0 & below);
      nope_idx[2 * pos] = 2 * l;
      nope_idx[2 * pos + 1] = 2 * l + 1;
    }
    if (64 + l < half && !k1) {
      const int pos = 64 + l - __builtin_popcountll(m0) - __builtin_popcountll(m1 & below);
      nope_idx[2 * pos] = 2 * (64 + l);
      nope_idx[2 * pos + 1] = 2 * (64 + l) + 1;
    }
  }
}

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16 * lane (global_load_lds_dwordx4),
// global address = base (wave-uniform, SGPRs) + voff (per lane, 32-bit).  Written as asm so that the
// compiler does not guard every later LDS read with a full vmcnt(0) drain: the asm has no output
// registers, and its completion is awaited explicitly with MLA_WAIT_VMCNT before the slot it fills is
// read.  (Loads the compiler does not see only make its own vmcnt waits stricter.)
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");  // M0 is rewritten here; no other instruction in these kernels reads M0
}
// As dma16 with the non-temporal hint, for rows a call streams once (the decode's cache rows): a stream of
// 1 KB requests at four waves per CU reaches ~7.15 TB/s with it against ~6.4 TB/s without (same GPU).  (The
// queries of one sequence in a multi-query decode read its rows from several workgroups and would find them
// in L2 without the hint; a per-launch choice measured slower for the single-query decode it serves.)
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
}
// 4 bytes per lane (global_load_lds_dword) into LDS at lds_addr + 4 * lane; otherwise as dma16.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt with only the vector-memory counter constrained (expcnt 7, lgkmcnt 15 = no wait)
#define MLA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | (((n) >> 4) << 14))

// Float equivalents of __shfl_xor for a full 64-lane wave.
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

// ---------------------------------------------------------------- int4 group-32 latent codec
// s = fp16(absmax / 7) with an IEEE fp32 division (infinite s saturates to the largest finite fp16);
// code = clamp(rint(x / s), -7, 7) with an IEEE fp32 division; s == 0 gives code 0.
__device__ __forceinline__ __half int4_scale(float absmax) {
  float s = __fdiv_rn(absmax, 7.0f);
  __half h = __float2half_rn(s);
  if (__hisinf(h)) h = __ushort_as_half((unsigned short)0x7BFF);
  return h;
}
__device__ __forceinline__ int int4_code(float x, float s) {
  if (s == 0.0f) return 0;
  float q = rintf(__fdiv_rn(x, s));
  q = fminf(fmaxf(q, -7.0f), 7.0f);
  return (int)q;
}
__device__ __forceinline__ float int4_dequant(int code, float s) { return (float)code * s; }
// Sign-extend nibble `k` (0 = low) of a byte.
__device__ __forceinline__ int nibble(uint32_t byte, int k) {
  int v = (byte >> (4 * k)) & 0xF;
  return v >= 8 ? v - 16 : v;
}

}  // namespace mla
