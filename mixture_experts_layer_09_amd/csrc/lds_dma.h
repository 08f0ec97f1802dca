// lds_dma.h -- global->LDS DMA, explicit vmcnt waits and transposing LDS
// reads for gfx950, shared by the grouped GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// One DMA instruction: 16 bytes per lane from sbase + voff to LDS lds_dst +
// 16 * lane (sbase and lds_dst are wave-uniform; lds_dst goes through M0).
// Written as inline asm so that the compiler, which would otherwise make
// every later LDS read wait for all DMA in flight, leaves the waiting to
// wait_vmcnt; the memory clobber keeps LDS reads and other memory operations
// on their side of it, and m0 is declared clobbered so that the compiler
// keeps no value of its own there across the instruction (clang notes that
// m0 is a reserved register, which it only ever sets right before its own
// uses; the clobber is recorded all the same, so the note is silenced here).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, char* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds_dst)));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// As dma16 with the LDS destination given as an LDS address (wave-uniform),
// which spares the generic-to-LDS pointer conversion in a hot loop.
__device__ __forceinline__ void dma16_at(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// The LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// As dma16 with 4 bytes per lane (LDS lds_dst + 4 * lane).
__device__ __forceinline__ void dma4(const char* sbase, uint32_t voff, char* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds_dst)));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

#pragma clang diagnostic pop

// A pointer the compiler may not prove wave-uniform, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Two consecutive int32 at a wave-uniform address, read through the scalar
// cache.  The compiler turns a plain load of memory that the kernel might
// also write into a vector load, and its wait (vmcnt(0)) would drain every
// DMA and store this wave has in flight; this one waits on lgkmcnt only.
__device__ __forceinline__ void scalar_load2(const int32_t* p, int& a, int& b) {
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  a = static_cast<int>(static_cast<uint32_t>(v));
  b = static_cast<int>(static_cast<uint32_t>(v >> 32));
}

// s_waitcnt vmcnt(n) with the other counters left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 16].
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    default: wait_vmcnt<16>(); break;
  }
}

// Wait until at most min(MAXA, after) * OPS DMAs of this wave are in flight,
// for a wave-uniform `after` >= 0: the first test is the steady state, so a
// K-loop stage takes one scalar branch.
template <int OPS, int MAXA>
__device__ __forceinline__ void wait_after(int after) {
  if constexpr (MAXA <= 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= MAXA)
      wait_vmcnt<MAXA * OPS>();
    else
      wait_after<OPS, MAXA - 1>(after);
  }
}

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

__device__ __forceinline__ i16x4_t ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

typedef __attribute__((ext_vector_type(2))) int i32x2v_t;

__device__ __forceinline__ i32x2v_t ds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2v_t*)(p));
}

}  // namespace moe
