// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, the bf16 matrix-core instructions, cross-half wave exchange,
// the LDS transpose read, and base-2 exp/log.
//
// Lane layouts used throughout (wave64; l = lane, h = l / 32):
//   v_mfma_f32_32x32x16_bf16  D = A * B + C,  A 32x16, B 16x32, D 32x32
//     A: lane l holds A[m = l % 32][k = 8h .. 8h + 7]
//     B: lane l holds B[k = 8h .. 8h + 7][n = l % 32]
//     D: lane l, register i holds D[m = 8 (i / 4) + 4h + (i % 4)][n = l % 32]
//   ds_read_b64_tr_b16 (per group of 16 lanes, s = l % 16):
//     if source lane s reads the 4 bf16 at row r0 + s / 4, columns
//     c0 + 4 (s % 4) .. + 3 of a row-major matrix, result lane i of the group
//     receives the 4 bf16 at rows r0 .. r0 + 3 of column c0 + i.
// Both were checked on the device against a host matrix product / index dump.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// max(a, b, c) in one v_max3_f32 (the compiler otherwise builds a tree of
// two-input maxima for a long chain).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Combine a per-lane value with the same lane of the other wave half
// (lane l with lane l ^ 32) using v_permlane32_swap: after swapping x with
// itself, the two results hold {x[l], x[l ^ 32]} in some order on every lane.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- direct global -> LDS loads, written as inline assembly so that the
// compiler neither tracks these LDS writes (it would wait for every
// outstanding load before each LDS read) nor counts them in its own waits;
// kernels wait for them explicitly. M0 carries the wave-uniform LDS address.
// Lane i reads base + voff (its own 32-bit offset) and writes LDS at
// lds + 16 i (dma16) or lds + 4 i (dma4).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, FA_LDS char* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(la) : "m0");
}
// The same with the non-temporal hint: for data read once (a decode's K/V
// stream), so the caches do not keep lines no one will read again; on the
// 2 GB decode workload it moves the kernel from 6.0 to 6.7 TB/s.
__device__ __forceinline__ void dma16_nt(const char* base, uint32_t voff, FA_LDS char* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(base), "s"(la) : "m0");
}
// The same through a buffer resource: lane i reads rsrc.base + voff, and a
// lane whose 16 bytes lie past rsrc's size reads zeros instead of memory, so
// a tile that runs past the end of a tensor needs no per-lane clamp. The
// resource must be uniform (scalar registers).
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4_t r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)((uint32_t)(a >> 32) & 0xffffu);  // stride 0: raw byte addressing
  r[2] = (int32_t)bytes;                            // range checked against this
  r[3] = 0x00020000;                                // 32-bit data format
  return r;
}
__device__ __forceinline__ void dma16_buf(i32x4_t rsrc, uint32_t voff, FA_LDS char* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(la) : "m0");
}
__device__ __forceinline__ void dma4(const char* base, uint32_t voff, FA_LDS char* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(base), "s"(la) : "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory operations are still
// outstanding (they complete in issue order) and all of its LDS reads have
// returned, then join the workgroup barrier. No memory fence: LDS
// visibility is all that is needed.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Transposing LDS read of 4 bf16 (see the layout note above).
__device__ __forceinline__ bf16x4_t lds_read_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4_t*)(p));
}
__device__ __forceinline__ bf16x4_t lds_read_tr4(const FA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4_t*)(p));
}

// Workgroup barrier after this wave's LDS accesses have completed, with no
// wait for outstanding global memory operations.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8_t concat8(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even fp32 -> bf16 of a pair.
__device__ __forceinline__ bf16x2_t to_bf16x2(float a, float b) {
  f32x2_t f = {a, b};
  return __builtin_convertvector(f, bf16x2_t);
}

// Chunk swizzles (XOR on the 16-byte chunk index within a row). RPL = rows
// per 256-byte bank line. K: the 16 rows of one 128-bit read phase land on 16
// distinct chunk slots. V: the 4 rows of one transposed read phase land in 4
// distinct 64-byte quarters of the bank line.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  constexpr int RPL = 128 / D;
  return (r / RPL) & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  constexpr int RPL = 128 / D;
  return 4 * ((r / RPL) & (4 / RPL - 1));
}

}  // namespace fa
