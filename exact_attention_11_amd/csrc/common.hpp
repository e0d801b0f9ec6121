// Device-side building blocks shared by the gfx950 kernels of libfattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the hardware transcendental unit (v_exp_f32): 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the hardware unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
// 1/x on the hardware unit (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Pack two floats into bf16 pairs (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// bf16 -> f32 of the low / high half of a packed pair (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Byte select from two dwords (v_perm_b32): selector bytes 0-3 pick from `a`,
// 4-7 from `b`.
__device__ __forceinline__ uint32_t perm_b32(uint32_t b, uint32_t a, uint32_t sel) {
  return __builtin_amdgcn_perm(b, a, sel);
}
// (a.lo16, b.lo16) and (a.hi16, b.hi16) as packed pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return zero (hardware range check), so tails need no predication.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// Direct HBM -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane i's bytes from byte offset `off` land at LDS byte lds_addr + 16*i
// (lds_addr the same in every lane of the wave); out-of-range lanes write
// zeros.  Written as inline assembly on purpose: the compiler then does not
// model the load's LDS write, so it inserts no vmcnt(0) drain in front of
// later LDS reads it cannot prove disjoint (it cannot for the transposing
// reads).  The caller orders the data with wait_vmem and a barrier.  The
// instruction writes no VGPR; m0 (the LDS base) is saved and restored.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t off) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(off), "s"(r)
      : "memory");
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Wait until this wave's outstanding vector-memory operations (including the
// direct-to-LDS loads) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// output lane i, element t is element (i % 4) of the 8 bytes addressed by
// lane 4t + i/4 of the same group.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// a.lo*b.lo + a.hi*b.hi + c for packed bf16 pairs, f32 result (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
constexpr uint32_t kBf16OnePair = 0x3F803F80u;  // (1.0, 1.0) as bf16
__device__ __forceinline__ void stg8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Value held by lane (lane ^ 32) of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: each lane ends up
// with its own value in one result and its partner's in the other).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

// Work item of this workgroup in a grid of nheads x nblk items, block 0 the
// heaviest.  Dispatch is round-robin over the 8 XCDs in blockIdx order; when
// the grid and the head count divide by 8, each XCD gets its own heads (their
// K/V stay in its L2), takes them `group` at a time and dispatches the
// heaviest blocks of a group first, so the launch ends with light blocks.
// Otherwise items go head by head, heaviest block first, consecutive items on
// one XCD when the grid divides by 8.
__device__ __forceinline__ void grouped_item(int nheads, int nblk, int group, int& head, int& blk) {
  const int G = gridDim.x;
  int w = blockIdx.x;
  if ((G & 7) == 0 && (nheads & 7) == 0) {
    const int hx = nheads >> 3;  // heads of each XCD
    const int u = w >> 3;        // dispatch rank within the XCD
    const int gi = u / (group * nblk);
    const int gs = min(group, hx - gi * group);  // heads in this group
    const int within = u - gi * group * nblk;
    blk = within / gs;
    head = (w & 7) * hx + gi * group + within % gs;
  } else {
    if ((G & 7) == 0) w = (w & 7) * (G >> 3) + (w >> 3);
    blk = w % nblk;
    head = w / nblk;
  }
}

}  // namespace fattn
