// Pieces shared by the GEMM kernels (NVFP4 and MXFP4): the XCD-aware tile order, the swizzled
// LDS code layout and the LDS barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t word(const u32x4_t &v, int i) { return v[i]; }

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8).  Map
// them so that each XCD gets a contiguous range of logical tiles, and order tiles in groups of
// kGroupM tile-rows so the tiles that run together on one XCD share A and W panels in its L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ int xcd_logical(int b, int nwg) {
  const int per = nwg / kXcds, rem = nwg % kXcds;
  const int x = b % kXcds, i = b / kXcds;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

// Tile (tm, tn) of workgroup `b` in a grid of tiles_m x tiles_n tiles, in the order above.
__device__ __forceinline__ void tile_of(int b, int nwg, int tiles_m, int tiles_n, int &tm,
                                        int &tn) {
  const int logical = xcd_logical(b, nwg);
  const int in_group = kGroupM * tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  tm = first_m + (logical % in_group) % gsz;
  tn = (logical % in_group) / gsz;
}

// Byte offset of half `h` of a 32-byte code row `row` in an LDS stage.  The two 16-byte halves
// are swapped on rows where bit 2 xor bit 3 of the row is set: a fragment read (one half of 8 or
// 16 consecutive rows per LDS cycle) then covers every bank once, and a store of 16 consecutive
// chunks still fills 256 contiguous bytes.
__device__ __forceinline__ int code_offset(int row, int h) {
  return row * 32 + ((h ^ (row >> 2) ^ (row >> 3)) & 1) * 16;
}

// A global scale read with a vector load.  A uniform read would be a scalar load, which the
// compiler may issue after the operand loads, and scalar loads share their wait counter with
// LDS: the first LDS barrier would then wait for it behind the whole stream of W (the rotated
// weights of a decode loop are not in cache).  Issued before the operand loads, a vector load is
// also waited for before them, since loads complete in order.
__device__ __forceinline__ float load_global_scale(const float *p) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, 4, 0x00020000);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Two floats to bf16, round to nearest even, in one packed conversion (v_cvt_pk_bf16_f32),
// element 0 in the low half.  The kernels keep fp32 denormals, so this equals the bit-level
// rounding (add 0x7FFF plus the kept lsb, shift) for every value that is not a NaN.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// Wait for this wave's LDS stores, then for every wave of the workgroup.  The asm's memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace nvfp4
