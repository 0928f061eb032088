// fa_varlen_device.h -- device helpers shared by the forward and backward
// kernels: vector types, the 16-bit element traits, fast exp2/log2, lane-pair
// reductions, raw buffer resources, direct global -> LDS loads with explicit
// waits, and the register staging of K-style (row-major, swizzled) and
// V-style (transposed) 16-bit tiles into LDS.
//
// Included by the .hip sources only (inside namespace fa, an anonymous
// namespace: every translation unit keeps its own copy).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_varlen_tiling.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

// 16-bit element types of the MFMA path: bf16 and IEEE fp16 share every tile
// layout (2-byte elements, moved as raw bits through LDS); only the MFMA and
// the float conversions (round to nearest even) differ.
template <typename T>
struct Elem16;
template <>
struct Elem16<__bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  __device__ __forceinline__ static f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Elem16<_Float16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  __device__ __forceinline__ static f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// 16x16x32 MFMA of the 16-bit element type
template <typename T>
struct Mfma16;
template <>
struct Mfma16<__bf16> {
  __device__ __forceinline__ static f32x4 run(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma16<_Float16> {
  __device__ __forceinline__ static f32x4 run(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Lanes l and l^32 hold the two halves of one query row.  v_permlane32_swap
// exchanges the halves of a register pair; one result holds the lane's own
// value and the other its partner's, so symmetric reductions need no select.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Raw buffer resource over [base, base + bytes).  Loads at byte offsets at or
// past `bytes` return zeros from the hardware range check, which is how rows
// past the end of a sequence are zero-filled without branches.  Dword 3 selects
// the 32-bit data format that untyped buffer loads need on CDNA.
// Callers pass wave-uniform values; readfirstlane tells the compiler so, and
// keeps the resource in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* p = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// The same descriptor as four scalar dwords, for inline assembly.
__device__ __forceinline__ u32x4 buffer_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu;  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// LDS byte address of a pointer into a __shared__ array (wave-uniform).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// Direct global -> LDS load (buffer_load_dwordx4 ... lds): lane i's 16 bytes
// at byte offset `voffset` of the buffer land at LDS byte address
// lds_base + 16 i, without passing through registers.  It is issued from
// inline assembly so that the compiler does not track it (its wait analysis
// cannot tell LDS buffers apart and would wait for the load before the next
// LDS read of any buffer).  The caller waits for it itself (wait_vmcnt)
// before the barrier after which the destination is read.  A load in flight
// that the compiler does not know of only makes the compiler's own vmcnt
// waits stricter: vector-memory loads complete in order.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N): at most N vector-memory loads of this wave still in
// flight (export and LDS counters untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_offset, 0, 0);
}

using tiling::head_rows_bytes;
using tiling::key_of_arow;
using tiling::k_swz;
using tiling::v_swz;

template <int D, int BN, int NW>
struct Tile16 : tiling::Geom16<D, BN, NW> {
  using G = tiling::Geom16<D, BN, NW>;
  using G::K_PER_THREAD;
  using G::THREADS;
  using G::V_PER_THREAD;

  u32x4 kreg[K_PER_THREAD];
  u32x4 vreg[V_PER_THREAD][4];

  // global -> registers; rows at or beyond Lk read as zero.  The resources
  // start at the tile's first key (head slice) and end exactly at the end of
  // the last valid row's head slice, so offsets stay below BN * row_stride * 2
  // bytes (the host bounds heads * head_dim) and never reach past a tensor.
  __device__ __forceinline__ void load_k(const uint16_t* __restrict__ kbase, int64_t row_stride, int key0, int Lk,
                                         int tid) {
    const int rows = max(0, min(BN, Lk - key0));
    const __amdgpu_buffer_rsrc_t rk =
        buffer_rsrc(kbase + (int64_t)key0 * row_stride, head_rows_bytes(rows, row_stride, D, 2));
#pragma unroll
    for (int i = 0; i < K_PER_THREAD; ++i) {
      const int c = tid + i * THREADS;
      kreg[i] = buffer_load16(rk, ((uint32_t)G::k_row(c) * (uint32_t)row_stride + G::k_chunk(c) * 8) * 2u);
    }
  }
  __device__ __forceinline__ void load_v(const uint16_t* __restrict__ vbase, int64_t row_stride, int key0, int Lk,
                                         int tid) {
    const int rows = max(0, min(BN, Lk - key0));
    const __amdgpu_buffer_rsrc_t rv =
        buffer_rsrc(vbase + (int64_t)key0 * row_stride, head_rows_bytes(rows, row_stride, D, 2));
#pragma unroll
    for (int i = 0; i < V_PER_THREAD; ++i) {
      const int w = tid + i * THREADS;
      const int u = G::v_group(w), dc = G::v_dchunk(w);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (G::v_owned(w)) x = buffer_load16(rv, ((uint32_t)(4 * u + r) * (uint32_t)row_stride + dc * 8) * 2u);
        vreg[i][r] = x;
      }
    }
  }

  // registers -> LDS: K as is, V transposed
  __device__ __forceinline__ void store_k(uint16_t* Ks, int tid) const {
#pragma unroll
    for (int i = 0; i < K_PER_THREAD; ++i) {
      const int c = tid + i * THREADS;
      *(u32x4*)(Ks + G::ks_index(G::k_row(c), G::k_chunk(c))) = kreg[i];
    }
  }
  __device__ __forceinline__ void store_v(uint16_t* Vt, int tid) const {
#pragma unroll
    for (int i = 0; i < V_PER_THREAD; ++i) {
      const int w = tid + i * THREADS;
      if (!G::v_owned(w)) continue;
      const int u = G::v_group(w), dc = G::v_dchunk(w);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        // dims 2*e2 and 2*e2+1 of the chunk, for keys 4u..4u+3
        const uint32_t r0 = vreg[i][0][e2], r1 = vreg[i][1][e2];
        const uint32_t r2 = vreg[i][2][e2], r3 = vreg[i][3][e2];
        u32x2 lo, hi;
        lo[0] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);  // (key0, key1) of dim 2*e2
        lo[1] = __builtin_amdgcn_perm(r3, r2, 0x05040100u);  // (key2, key3)
        hi[0] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);  // dim 2*e2+1
        hi[1] = __builtin_amdgcn_perm(r3, r2, 0x07060302u);
        const int d0 = dc * 8 + 2 * e2;
        *(u32x2*)(Vt + G::vt_index(d0, 4 * u)) = lo;
        *(u32x2*)(Vt + G::vt_index(d0 + 1, 4 * u)) = hi;
      }
    }
  }
};

}  // namespace
}  // namespace fa
