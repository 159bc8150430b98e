// Device-side helpers shared by the gfx950 kernels: bf16 packing, MFMA operand types,
// cross-lane reductions and launch-geometry constants. CDNA4 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// 16 bytes viewed as raw dwords (what a 128-bit load returns).
struct __attribute__((aligned(16))) U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ U4 ldg16(const void* p) { return *reinterpret_cast<const U4*>(p); }
// 16-byte load and store with the non-temporal hint, for data that is read (written) once.
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
__device__ __forceinline__ U4 ldg16_nt(const void* p) {
  return __builtin_bit_cast(U4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void stg16_nt(void* p, U4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stg16(void* p, U4 v) { *reinterpret_cast<U4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(U4 v) { return __builtin_bit_cast(bf16x8, v); }

// exp2 on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the lane pair (l, l ^ 32) with one v_permlane32_swap: after the swap the two
// results hold x[l % 32] and x[32 + l % 32] in some order, so a symmetric op gives the pair value.
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// 16 bytes per lane straight from global memory into LDS (global_load_lds_dwordx4): lane i's
// bytes land at lds_base + 16 * i, so one wave instruction fills 1 KiB of LDS. lds_base must be
// the same for the whole wave.
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void_t*)lds_base, 16, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_32x32x16_bf16 whose destination is never allocated over
// the A or B operand registers: the compiler may otherwise reuse a source that dies at the
// instruction as its destination, which on gfx950 has given run-to-run different (wrong)
// results. The empty asm keeps both sources live until the result exists; it also pins the
// result to VGPRs, so accumulators the compiler keeps in AGPRs use the plain builtin (the build
// scans the generated code and rejects any remaining overlap).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  asm volatile("" ::"v"(a), "v"(b), "v"(d));
  return d;
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  const f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  asm volatile("" ::"v"(a), "v"(b), "v"(d));
  return d;
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lanes 4j..4j+3 each
// address 4 consecutive 16-bit elements of "row" j (16 elements per row); afterwards lane i holds
// element i of rows 0..3. With a row-major [key][dim] tile this yields 4 consecutive keys of one
// dim per lane: the k-slots of an MFMA operand whose reduction runs over keys.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same 16-byte direct-to-LDS load issued as inline assembly. The compiler then neither knows
// that LDS is written nor waits for it: the caller owns every vmcnt wait for these loads (with
// vmcnt(N) it can keep the newest N loads in flight, e.g. a ring of LDS stages). The LDS base of
// the wave (byte address) goes through M0. kStream adds the non-temporal hint, for rows that are
// read once (the decode caches; it measurably raises the achieved HBM bandwidth there); tiles that
// other work-groups read again (prefill K/V) keep the default policy.
// A global load with the LDS bit must come at least one wait state after a scalar instruction
// that writes M0. The compiler writes M0 for the "{m0}" operand directly in front of the asm and
// does not insert hazard wait states in front of inline assembly, so the s_nop 0 is part of the
// asm itself (the build scans the generated code for any M0 write closer to such a load).
template <bool kStream = true>
__device__ __forceinline__ void load_lds16_async(const void* gptr, const void* lds_base) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  if constexpr (kStream)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(lds_addr) : "memory");
}

// The same load with a wave-uniform base in SGPRs and a 32-bit per-lane byte offset: the
// address needs no vector arithmetic per load. The base must be computed by scalar instructions
// (kernel arguments, block indices, loop counters): the "s" constraint then holds, and the SGPR
// pair is never the result of a vector instruction such as v_readfirstlane. A VMEM instruction
// that reads an SGPR written by a VALU instruction needs 5 wait states, which the compiler does not
// insert in front of inline assembly (the build rejects such sequences in the generated code).
// kStream adds the non-temporal hint (rows read once), as for load_lds16_async.
template <bool kStream = false>
__device__ __forceinline__ void load_lds16_async_sv(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  if constexpr (kStream)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}

// The same, with the 5 wait states that a base pair written by a vector instruction would need
// inside the asm: for loads placed among other work, where a branch target may come right before.
template <bool kStream = false>
__device__ __forceinline__ void load_lds16_async_sv_nop(const void* sbase, uint32_t voff, const void* lds_base) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base;
  if constexpr (kStream)
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
  else
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}

// Work-group barrier without the memory fences of __syncthreads(): for tiles filled by
// load_lds16_async after an explicit vmcnt wait, where the fence's wait for every outstanding
// load (including later stages still in flight) is not wanted.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// vmcnt(0) as a real s_waitcnt the compiler's wait tracking sees (gfx9 encoding: expcnt and
// lgkmcnt fields at their maximum): use it to retire ordinary loads before async LDS loads start,
// so no lazily placed wait for them lands inside a loop and drains the async loads too.
__device__ __forceinline__ void retire_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace attn
