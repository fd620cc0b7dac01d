// Measurement program (not part of libnvfp4): the throughput of the matrix-core routes an NVFP4
// W4A4 product could take on gfx950, from registers only (no memory traffic), so the choice of
// route rests on numbers measured on the device rather than on instruction counts alone.
//
// NVFP4 scales every 16 values by an E4M3 factor, which no CDNA4 matrix instruction takes, so
// every route pays vector (VALU) work for the scales besides its MFMAs:
//   f16          : v_mfma_f32_32x32x16_f16 alone (the ceiling of the fp16 route);
//   f16+decode   : the fp16 route as the library's GEMM runs it: per K step a wave decodes 4 A and
//                  4 W fragments (FP4 -> fp16 with the hardware conversion, times the block scale:
//                  exact) and issues 16 MFMAs on a 4 x 4 grid of 32 x 32 tiles;
//   fp8          : v_mfma_f32_32x32x16_fp8_fp8 alone: K = 16 is exactly one NVFP4 block, with
//                  E2M1 codes exact in FP8 E4M3;
//   fp8+rescale  : that MFMA into a fresh tile per block, then the per-block rescale of each of the
//                  lane's 16 results by sbA[row] * sbW[col] into the running sum (16 multiplies
//                  for the scale products, 16 FMAs), plus the FP4 -> FP8 code conversion of the
//                  operands; 2 x 2 tiles per wave (the rescale's temporaries leave no room for
//                  more accumulators);
//   fp8+fma-only : the same with only the 16 FMAs per block (scale products assumed free): the
//                  least VALU the FP8 route can do;
//   fp4-scaled   : v_mfma_scale_f32_32x32x64_f8f6f4 on FP4 operands with unit E8M0 scales (the
//                  MXFP4 product's instruction; it cannot carry E4M3 scales per 16 values).
// Operands are random bits (finite values), since the chip lowers its clock under dense MFMA
// work on random data.  Each route runs 2048 workgroups of 4 waves; TFLOP/s count 2 M N K of
// the MFMAs only (for the fp8 routes: the useful K = 16 per block).
//
//   usage: mfma_routes [iterations]      (prints one line per route)
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

#define CK(x)                                                                          \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);           \
      exit(1);                                                                         \
    }                                                                                  \
  } while (0)

__device__ __forceinline__ uint32_t mix(uint32_t h) {
  h ^= h >> 16; h *= 0x7feb352du; h ^= h >> 15; h *= 0x846ca68bu; h ^= h >> 16;
  return h;
}
// Random finite fp16 pair / E4M3 bytes / E4M3 scale pair from a seed.
__device__ __forceinline__ uint32_t rnd_f16x2(uint32_t h) {
  return (h & 0x83FF83FFu) | (((((h >> 10) & 7u) + 12u) << 10) | ((((h >> 26) & 7u) + 12u) << 26));
}
__device__ __forceinline__ uint32_t rnd_fp8x4(uint32_t h) {
  return (h & 0x87878787u) | 0x20202020u;
}

__device__ __forceinline__ half8_t decode8(uint32_t q, half2_t s) {
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0);
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1);
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2);
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3);
  h0 *= s; h1 *= s; h2 *= s; h3 *= s;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Eight E2M1 codes (one word) -> eight E4M3 bytes: the magnitude (3 bits) indexes the E4M3
// encodings of 0, 0.5, 1, 1.5, 2, 3, 4, 6 through byte permutes; the sign moves to bit 7.
__device__ __forceinline__ uint64_t fp4_to_fp8x8(uint32_t q) {
  const uint32_t lut_lo = 0x3C383000u, lut_hi = 0x4C484440u;  // E4M3 of 0, .5, 1, 1.5 | 2, 3, 4, 6
  const uint32_t lo = q & 0x0F0F0F0Fu, hi = (q >> 4) & 0x0F0F0F0Fu;
  const uint32_t mlo = __builtin_amdgcn_perm(lut_hi, lut_lo, lo & 0x07070707u);
  const uint32_t mhi = __builtin_amdgcn_perm(lut_hi, lut_lo, hi & 0x07070707u);
  const uint32_t slo = (lo & 0x08080808u) << 4, shi = (hi & 0x08080808u) << 4;
  return ((uint64_t)(mhi | shi) << 32) | (uint64_t)(mlo | slo);
}

enum Route { kF16, kF16Decode, kFp8, kFp8Rescale, kFp8FmaOnly, kFp4Scaled };

template <int R>
__global__ __launch_bounds__(256) void k_route(int iters, float *out) {
  const uint32_t tid = blockIdx.x * 256 + threadIdx.x;
  uint32_t s0 = mix(tid * 0x9E3779B9u + 1u), s1 = mix(s0 + 7u), s2 = mix(s1 + 13u), s3 = mix(s2 + 5u);
  float chk = 0.0f;
  if (R == kF16 || R == kF16Decode) {
    floatx16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx16_t{};
    half8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h = mix(s0 + i);
      a[i] = __builtin_bit_cast(half8_t, make_uint4(rnd_f16x2(h), rnd_f16x2(mix(h)), rnd_f16x2(mix(h + 1)), rnd_f16x2(mix(h + 2))));
      const uint32_t g = mix(s1 + i);
      b[i] = __builtin_bit_cast(half8_t, make_uint4(rnd_f16x2(g), rnd_f16x2(mix(g)), rnd_f16x2(mix(g + 1)), rnd_f16x2(mix(g + 2))));
    }
    uint32_t qa = s2, qw = s3;
    const half2_t sc = {(_Float16)1.125f, (_Float16)1.125f};
    for (int it = 0; it < iters; ++it) {
      if (R == kF16Decode) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = decode8(qa + i, sc);
          b[i] = decode8(qw + i, sc);
        }
        qa = qa * 1664525u + 1013904223u;
        qw = qw * 22695477u + 1u;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) chk += acc[i][j][0] + acc[i][j][15];
  } else if (R == kFp8 || R == kFp8Rescale || R == kFp8FmaOnly) {
    floatx16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = floatx16_t{};
    long a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = (long)(((uint64_t)rnd_fp8x4(mix(s0 + i)) << 32) | rnd_fp8x4(mix(s1 + i)));
      b[i] = (long)(((uint64_t)rnd_fp8x4(mix(s2 + i)) << 32) | rnd_fp8x4(mix(s3 + i)));
    }
    uint32_t qa = s2, qw = s3, sbits = s0 & 0x3C3C3C3Cu;
    float sa[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sa[e] = 1.0f + e * 0.0625f;
    // A zero tile kept in registers as the MFMA's C operand (read only), so that a fresh block
    // product needs no zeroing instructions.
    floatx16_t zero = {};
    asm volatile("" : "+v"(zero));
    for (int it = 0; it < iters; ++it) {
      if (R == kFp8) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a[i], b[j], acc[i][j], 0, 0, 0);
        // 4 accumulators give 4 MFMAs per step (the 4 x 4 grid of the fp16 routes needs twice
        // the registers of an fp8 K = 16 step in the rescale forms).
      } else {
        if (R == kFp8Rescale) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            a[i] = (long)fp4_to_fp8x8(qa + i);
            b[i] = (long)fp4_to_fp8x8(qw + i);
          }
          qa = qa * 1664525u + 1013904223u;
          qw = qw * 22695477u + 1u;
        }
        // This block's scales: the lane's column scale, its 16 rows' scales (E4M3 -> fp32).
        const floatx2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sbits, 1.0f, false);
        sbits = sbits * 1103515245u + 12345u;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const floatx16_t p = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a[i], b[j], zero, 0, 0, 0);
            const float sw = j ? w2[1] : w2[0];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float t = (R == kFp8Rescale) ? sa[e] * sw : sw;
              acc[i][j][e] = fmaf(p[e], t, acc[i][j][e]);
            }
          }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) chk += acc[i][j][0] + acc[i][j][15];
  } else {  // kFp4Scaled
    floatx16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx16_t{};
    i32x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = i32x8_t{(int)mix(s0 + i), (int)mix(s1 + i), (int)mix(s2 + i), (int)mix(s3 + i), 0, 0, 0, 0};
      b[i] = i32x8_t{(int)mix(s0 + 9 * i), (int)mix(s1 + 9 * i), (int)mix(s2 + 9 * i), (int)mix(s3 + 9 * i), 0, 0, 0, 0};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, 127, 0, 127);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) chk += acc[i][j][0] + acc[i][j][15];
  }
  if (chk == 1234.5f) out[tid] = chk;  // keeps the work; never true for these inputs in practice
}

template <int R>
static void run(const char *name, int iters, float *out, int mfma_per_iter, double k_useful) {
  const int grid = 2048;
  hipLaunchKernelGGL(k_route<R>, dim3(grid), dim3(256), 0, 0, iters / 8, out);
  CK(hipDeviceSynchronize());
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  CK(hipEventRecord(a, 0));
  hipLaunchKernelGGL(k_route<R>, dim3(grid), dim3(256), 0, 0, iters, out);
  CK(hipEventRecord(b, 0));
  CK(hipEventSynchronize(b));
  CK(hipGetLastError());
  float ms = 0;
  CK(hipEventElapsedTime(&ms, a, b));
  const double flops = 2.0 * 32 * 32 * k_useful * (double)mfma_per_iter * iters * grid * 4;
  printf("%-13s %9.1f us  %8.1f TFLOP/s\n", name, ms * 1e3, flops / (ms * 1e-3) / 1e12);
  CK(hipEventDestroy(a));
  CK(hipEventDestroy(b));
}

int main(int argc, char **argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 200;
  float *out = nullptr;
  CK(hipMalloc(&out, 2048 * 256 * sizeof(float)));
  run<kF16>("f16", iters, out, 16, 16);
  run<kF16Decode>("f16+decode", iters, out, 16, 16);
  run<kFp8>("fp8", iters, out, 4, 16);
  run<kFp8Rescale>("fp8+rescale", iters, out, 4, 16);
  run<kFp8FmaOnly>("fp8+fma-only", iters, out, 4, 16);
  run<kFp4Scaled>("fp4-scaled", iters, out, 16, 64);
  CK(hipFree(out));
  return 0;
}
