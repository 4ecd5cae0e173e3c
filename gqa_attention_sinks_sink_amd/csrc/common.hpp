// Device helpers shared by the sink-attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_sink {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2 (RNE) with the gfx950 conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// MFMA wrappers (gfx950 bf16, fp32 accumulate).
//   16x16x32: A lane l = row l%16, k 8*(l/16)+[0..7]; B lane l = col l%16, same k;
//             C lane l = col l%16, rows 4*(l/16)+[0..3].
//   32x32x16: A lane l = row l%32, k 8*(l/32)+[0..7]; B lane l = col l%32, same k;
//             C reg i of lane l = row 8*(i/4)+4*(l/32)+(i%4), col l%32.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
//   16x16x16: A lane l = row l%16, k 4*(l/16)+[0..3]; B lane l = col l%16, same k;
//             C as 16x16x32.
__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read (ds_read_b64_tr_b16). Within each 16-lane group, lane j supplies
// an 8-byte address holding 4 consecutive bf16 of one row; lane i receives element
// (i % 4) of lane (4*e + i/4)'s data as its element e. With lane j pointing at
// row k0 + j/4, columns c0 + 4*(j%4) .. +3 of a row-major tile, lane i receives column
// c0 + i of rows k0..k0+3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, const_cast<void*>(lds_addr)));
}

// Two transposing reads (keys k0..k0+3 and the next 4 keys) as one 8-element MFMA operand.
__device__ __forceinline__ u32x4 join_tr16(s16x4 lo, s16x4 hi) {
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes return zero
// without touching memory (CDNA buffer range check), so tails need no branches. The range
// check covers the VGPR offset; the SGPR offset is kept at zero so every byte is checked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS (no VGPRs): lane i of the wave writes
// lds_base + 16 * i, where lds_base is wave-uniform. The load is issued so that the compiler
// does not see the LDS write.
// The compiler otherwise makes every later LDS read wait for all outstanding buffer loads
// (it cannot tell the stages of a ring apart), which serialises a prefetch ring. Callers own
// the synchronisation: s_waitcnt vmcnt for their own loads, then lds_barrier().
// The LDS address goes through M0, which the load reads when it is issued (one wait state
// between the M0 write and the load); M0 is saved and restored around it.
__device__ __forceinline__ void buffer_load16_lds_async(__amdgpu_buffer_rsrc_t r, const void* lds_base, uint32_t voff) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)LDS_PTR(void, const_cast<void*>(lds_base));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}

// Buffer resource whose base and size are taken from lane 0 (the caller guarantees they are
// wave-uniform), so that it lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const void* ub = (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return make_rsrc(ub, __builtin_amdgcn_readfirstlane(bytes));
}

// Non-temporal variant (data read once: K/V cache streaming); lds_addr is the wave-uniform
// LDS byte address that lane 0 writes.
__device__ __forceinline__ void buffer_load16_lds_async_nt(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr_in, uint32_t voff) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(lds_addr_in);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}


// Lane index that the compiler can neither hoist nor keep alive across a loop: per-lane
// addresses derived from it are recomputed where they are used.
__device__ __forceinline__ int opaque_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Read of memory that no kernel writes while it runs (page tables): through the constant
// address space, so that a wave-uniform index becomes a scalar load. A plain global load
// here would be a vector load, and the compiler's wait for it would also retire every K/V
// load issued before it.
template <typename T>
__device__ __forceinline__ T load_invariant(const T* base, size_t idx) {
  return ((const __attribute__((address_space(4))) T*)base)[idx];
}

// Workgroup barrier that is also a compiler barrier for memory accesses, without the
// s_waitcnt vmcnt(0) / lgkmcnt(0) that __syncthreads() adds.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(n) (n < 16), leaving the other counters alone.
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8))
// s_waitcnt lgkmcnt(0) alone (the vmcnt field at its maximum, 63).
#define WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14))

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

template <typename T>
__device__ __forceinline__ T clampi(T v, T lo, T hi) { return v < lo ? lo : (v > hi ? hi : v); }

}  // namespace attn_sink
