// LDS-DMA staging and transposing LDS reads on gfx950, shared by the
// streaming MFMA kernels (Hessian Gram, split-bf16 trailing update and the
// factorisation's trailing update).
//
//  * global_load_lds_dwordx4: each lane moves 16 bytes from its own global
//    address to LDS at M0 + 16 * lane, without passing through VGPRs. It is
//    issued from inline asm so that the compiler does not wait for every
//    outstanding DMA before each LDS read; completion is tracked with vmcnt
//    by the kernel, and the wait and the barrier that publishes a stage sit
//    in one asm block so no LDS read can be scheduled between them.
//  * ds_read_b64_tr_b16: within each group of 16 lanes, lane a + 4j supplies
//    the address of 4 consecutive 16-bit elements of row j, and lane 4a + b
//    receives element b of lane a's piece for the 4 rows, i.e. 4 consecutive
//    rows of one column. Two reads give the 8-deep K slice of a bf16 MFMA
//    operand from a row-major [k][column] LDS tile.
#pragma once
#include "common.h"

namespace gq {

// 16 zero bytes: the DMA source of chunks outside the matrix.
static __device__ __align__(16) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

__device__ __forceinline__ int dma_swz(int t) {
  // XOR applied to the 16-byte chunk index of row t (values < 16, so the
  // chunks of a row of 16 or more chunks are permuted among themselves).
  return (0xAC60 >> (4 * (t & 3))) & 15;   // t%4 -> 0, 6, 12, 10
}

// Wait until at most `stages` stages of 8 DMA instructions of this wave are
// outstanding, then barrier.
__device__ __forceinline__ void wait_dma_barrier(int stages) {
  if (stages <= 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if (stages == 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if (stages == 2) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_base) : "memory");
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int v4i32_t __attribute__((ext_vector_type(4)));

// Buffer form of the DMA: lane offset voff plus scalar offset soff into the
// buffer rsrc; offsets at or past the buffer's size read as zeros.
__device__ __forceinline__ void dma16_rsrc(uint32_t voff, v4i32_t rsrc, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds_base), "s"(soff) : "memory");
}

__device__ __forceinline__ v4i32_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  v4i32_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));   // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)(uint32_t)(bytes > 0 ? bytes : 0));
  r.w = 0x00020000;                                                    // raw, 32-bit format
  return r;
}

__device__ __forceinline__ v4i16_t lds_tr16(uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) v4i16_t*>(byte_off));
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace gq
