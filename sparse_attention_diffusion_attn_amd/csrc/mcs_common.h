// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// LDS swizzles, gathers straight into LDS, and the XCD-aware work mapping.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mcs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).  Lane l holds row/col
// (l % 32) of A/B and the 8 k-slots 8*(l/32)+i; it receives D rows
// 8*(j/4) + 4*(l/32) + (j%4), column l % 32, in accumulator j.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// K/V tiles of 64 rows live in LDS as D/32 "planes": plane T holds columns
// 32T .. 32T+31 of all 64 rows, 64 bytes per row, 4 KiB per plane.  Inside a
// plane the four 16-byte chunks of row r are permuted by XOR with (r >> 2) & 3.
// With 64 four-byte banks this keeps conflict-free both the 16-byte reads of
// 16 consecutive rows at one chunk (QK^T operand) and the transposing 8-byte
// reads of 4 consecutive rows x 2 chunks (PV operand), and every LDS address a
// lane uses is one of a few base registers plus a compile-time offset.
__device__ __forceinline__ int plane_chunk(int row, int chunk4) {
  return (chunk4 ^ (row >> 2)) & 3;
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0; loads past the
// end return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Per-lane 16-byte buffer -> LDS copy from byte offset voff + soff (soff
// uniform) of the resource; lane l's bytes land at lds_base + 16*l (lds_base
// uniform).
__device__ __forceinline__ void gather16_buf(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff,
                                             uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}

// Max / sum of this lane's value and lane (l ^ 32)'s, exchanged in the VALU
// (v_permlane32_swap swaps the two 32-lane halves; the pair it returns is
// {x[l], x[l^32]} in an order that a symmetric operation does not see).
__device__ __forceinline__ float max_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// j receives element (j % 4) of the 8-byte rows addressed by lanes j/4, j/4+4,
// j/4+8 and j/4+12.
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ i32x2 tr_read(const char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)p;
  return __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a));
}

// Workgroups are dealt round-robin to the 8 XCDs.  Map dispatch index i to a
// work item so that, within each run of 8*S dispatch indices, XCD x receives
// the S consecutive work items x*S .. x*S+S-1.  With S = 64 (two resident
// workgroups on each of an XCD's 32 CUs) the groups resident on one XCD are
// neighbours in PDDP order, whose similar queries select overlapping key sets
// that then hit in that XCD's L2, and all XCDs work on the same one or two
// heads, which keeps the K/V rows in flight well inside the 256 MB last-level
// cache.  A final partial run keeps the identity mapping.  (Measured against
// teams of 2 XCDs sharing a head: +1.5 to +2.5% on the 32768- to 118912-token
// layers.)
__device__ __forceinline__ int xcd_remap(int i, int n) {
  constexpr int X = 8, S = 64, SB = X * S;
  const int b = i / SB;
  if ((b + 1) * SB > n) return i;
  const int r = i - b * SB;
  return b * SB + (r % X) * S + r / X;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace mcs
