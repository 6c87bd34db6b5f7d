// Direct-to-LDS buffer loads for the gfx950 ring kernels (MXFP4 / MoE GEMMs and
// the W4A16 GEMM).
#pragma once

#include "device_common.h"

namespace bsfp4 {

// ---- direct-to-LDS loads ---------------------------------------------------
// buffer_load_dword{,x4} ... lds: every lane fetches 4 / 16 bytes and the wave
// writes them to LDS at M0 + lane * size, so one instruction fills 256 B / 1 KB
// of LDS without passing through VGPRs.  They are issued from inline assembly
// so that the compiler does not add a full vmcnt(0) wait before every LDS read
// (it cannot tell which ring slot an LDS DMA targets); the kernel waits
// explicitly with s_waitcnt vmcnt(n) + s_barrier.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Addressing: a buffer resource (SGPRs), a per-lane 32-bit offset and a
// uniform SGPR offset; lanes whose offset is past the buffer's size read zeros.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buf_lds16(v4u32 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_uniform) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_uniform)
               : "memory");
}

__device__ __forceinline__ void buf_lds4(v4u32 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_uniform) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_uniform)
               : "memory");
}

// Raw buffer resource over [p, p + bytes) (bytes < 2^31), uniform.
__device__ __forceinline__ v4u32 make_rsrc4(const void* p, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return v4u32{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xFFFFu)),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

constexpr uint32_t kBufOOB = 0x80000000u;  // lane offset past every buffer: reads zero

__device__ __forceinline__ v4u32 uniform4(v4u32 v) {
  return v4u32{(uint32_t)__builtin_amdgcn_readfirstlane((int)v.x), (uint32_t)__builtin_amdgcn_readfirstlane((int)v.y),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)v.z), (uint32_t)__builtin_amdgcn_readfirstlane((int)v.w)};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform run-time n (a compile-time constant
// after unrolling where the caller's loops are unrolled); n above 14 waits
// for vmcnt(14), i.e. for more loads than asked, never fewer
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
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
    default: wait_vmcnt<14>(); break;
  }
}

}  // namespace bsfp4
