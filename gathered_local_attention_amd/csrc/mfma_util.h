// Helpers shared by the matrix-core attention kernels of libclusterattn
// (gfx950): MFMA operand types, bf16/fp16 packing, direct-to-LDS loads with
// explicit vmcnt accounting, the transposing LDS read and the cross-row
// reductions.  Internal; not part of the public ABI.
#pragma once

#include "common.h"

namespace ca {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 32;
constexpr uint32_t kRow = D * 2;   // bytes of one head row (bf16 / fp16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                   __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x2 unpack(uint32_t w) {
    return f32x2{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
  }
};

template <> struct Mfma<f16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                  __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x2 unpack(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(v2, w), f32x2);
  }
};

// two floats -> one dword of T (round to nearest even, one instruction)
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), typename Mfma<T>::v2));
}

template <typename T>
__device__ __forceinline__ uint2 pack4(f32x4 x) {
  return make_uint2(pack2<T>(x[0], x[1]), pack2<T>(x[2], x[3]));
}

__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ uint4 pad(uint2 a) { return make_uint4(a.x, a.y, 0u, 0u); }
__device__ __forceinline__ uint4 sel(bool c, uint4 a) {
  return c ? a : make_uint4(0u, 0u, 0u, 0u);
}

// 16-byte load at a 32-bit byte offset from a (wave-uniform) base pointer
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off);
}
template <typename V>
__device__ __forceinline__ void stv(void* base, uint32_t off, V v) {
  *reinterpret_cast<V*>(reinterpret_cast<char*>(base) + off) = v;
}

// Streaming (non-temporal) 16-byte store for outputs that no later load of
// the same kernel reads: the lines are not kept in the L2, so little dirty
// data is left for the write-back at the kernel's end.  The backward passes
// write dQ, dK and dV this way (high-res backward 203.6 -> 193.8 us, stage-1
// 52.6 -> 51.7 us); the forward's O is faster with ordinary stores (23.2 vs
// 24.1 us at stage-1).
__device__ __forceinline__ void st16_nt(void* base, uint32_t off, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + off));
}


// Reductions over the four 16-lane rows (lanes c, c+16, c+32, c+48) with the
// gfx950 row-swap moves: permlane16_swap(x, x) yields x of rows {0,0,2,2} and
// {1,1,3,3}, permlane32_swap(x, x) x of halves {0,0} and {1,1} (checked on the
// hardware), so two VALU swaps replace two LDS-crossbar shuffles.
__device__ __forceinline__ float xrow16(float v, bool take_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xrow32(float v, bool take_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float shfl_max16_32(float v) { return xrow32(xrow16(v, true), true); }
__device__ __forceinline__ float shfl_sum16_32(float v) { return xrow32(xrow16(v, false), false); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;


__device__ __forceinline__ uint4 lds16(const char* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint2 lds_tr8(const char* base, uint32_t off) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(base + off)));
  return __builtin_bit_cast(uint2, r);
}

// One 16-byte direct-to-LDS load per lane: global (base + voff) -> LDS
// (lds + 16 * lane), lds wave-uniform.  Written as asm with no outputs so that
// the compiler does not guard every later LDS read with a full vmcnt wait;
// the kernels wait for these loads themselves with s_waitcnt vmcnt(n), which
// counts them in issue order together with every other vector-memory op.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// The same for rows that no other item reads again (a cluster's own query
// rows): a streaming (non-temporal) load, so they do not push gathered rows
// that other items still need out of the L2.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// The same with a per-lane 64-bit global address (lanes may read from
// different arrays in one instruction).
__device__ __forceinline__ void dma16v(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(addr), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt with vmcnt = N (0..63) and no wait on the other counters
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}


// Direct-to-LDS 4-byte load per lane: global (base + voff) -> LDS (lds + 4 * lane).
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) for a run-time n from the few values the pipelines use
// (a larger count is never required: any n' <= n is safe, only slower)
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {   // n wave-uniform; above 11 waits as for 11
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    default: wait_vm<11>(); break;
  }
}

// wait for this wave's outstanding LDS reads (before a DMA overwrites them)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace
}  // namespace ca
