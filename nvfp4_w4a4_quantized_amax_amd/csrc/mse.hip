// MSE-observer block scales for offline weight quantization: the global scale stays the amax
// one, and each block takes, among the E4M3 codes c0 - 16 .. c0 + 1 around the amax-derived code
// c0, the scale whose reconstruction has the least squared error ("Accelerating large language
// models with NVFP4 quantization", section "NVFP4 robustness with scale-dependent variability",
// names MSE-based observers as a calibration refinement).  The error is evaluated in fp32 in a
// fixed order so the decision is reproducible:
//   d_i = RN(code value_i * sb * gs) (code value * sb is exact), e_i = RN(x_i - d_i),
//   row error = left-to-right RN sum of RN(e_i * e_i) over 16 consecutive values;
//   a 16x16 tile combines its 16 row errors by a pairwise tree (partner r ^ 1, ^2, ^4, ^8).
// The smallest error wins; among equal errors the code nearest c0, then the smaller code.
// Elements are encoded under each candidate exactly as the quantizer does (nearest E2M1, ties
// to even), with the per-code multipliers of the scale tables.

#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kMseThreads = 256;

struct MseOut {
  uint8_t *codes;
  int64_t ld_codes;
  uint8_t *scales;
  int64_t ld_scales;
};
constexpr int kMseAmaxWgs = 512;

// Pass 1: per-workgroup maxima of |x| (bf16 patterns) into the workspace slots.
__global__ __launch_bounds__(kMseThreads) void k_mse_amax(const uint16_t *__restrict__ x,
                                                          int64_t rows, int64_t cols, int64_t ld,
                                                          uint32_t *__restrict__ slots) {
  __shared__ uint32_t red[kMseThreads / kWave];
  const int64_t cpr = cols / 8, n = rows * cpr;
  uint32_t m = 0;
  for (int64_t u = (int64_t)blockIdx.x * kMseThreads + threadIdx.x; u < n;
       u += (int64_t)gridDim.x * kMseThreads) {
    const int64_t r = u / cpr, c = u - r * cpr;
    m = max(m, absmax8(*(const uint4 *)(x + r * ld + c * 8)));
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) slots[blockIdx.x] = m;
}

// Error of 16 values (two 8-value halves) under scale sb: see the header.
__device__ __forceinline__ float row_error(const uint4 &a, const uint4 &b, uint2 codes, float sb,
                                           float gs) {
  float s = 0.0f;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  const uint32_t v[4] = {b.x, b.y, b.z, b.w};
  const uint32_t q[2] = {codes.x, codes.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx2_t cv = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[h], 1.0f, 0)
                         : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[h], 1.0f, 1)
                         : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[h], 1.0f, 2)
                                  : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[h], 1.0f, 3);
      const uint32_t xw = h == 0 ? w[j] : v[j];
      const float x0 = bf16_lo(xw), x1 = bf16_hi(xw);
      const float d0 = (cv[0] * sb) * gs, d1 = (cv[1] * sb) * gs;
      const float e0 = x0 - d0, e1 = x1 - d1;
      s = s + e0 * e0;
      s = s + e1 * e1;
    }
  }
  return s;
}

// Offsets from c0 in order of preference: 0, -1, +1, -2, -3, ..., -16.
__device__ __forceinline__ int cand_offset(int i) { return i == 0 ? 0 : (i == 1 ? -1 : (i == 2 ? 1 : 1 - i)); }
constexpr int kMseCands = 18;

__device__ __forceinline__ float mse_gs(const uint32_t *slots, int n_slots, QuantTables &tab,
                                        uint32_t *red, float *gs_out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n_slots; i += blockDim.x) m = max(m, slots[i]);
  m = block_max_u32(m, red);
  const float gs = global_scale_from_amax_bits(m);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  build_tables(tab, gs);
  return gs;
}

// 1D blocks: one thread per 16-value block.
__global__ __launch_bounds__(kMseThreads) void k_mse_encode_1d(const uint16_t *__restrict__ x,
                                                               int64_t rows, int64_t cols,
                                                               int64_t ld, MseOut o,
                                                               const uint32_t *__restrict__ slots,
                                                               int n_slots,
                                                               float *__restrict__ gs_out) {
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kMseThreads / kWave];
  const float gs = mse_gs(slots, n_slots, tab, red, gs_out);
  const float inv6gs = tab.inv6gs;
  const int64_t bpr = cols / 16, n = rows * bpr;
  for (int64_t blk = (int64_t)blockIdx.x * kMseThreads + threadIdx.x; blk < n;
       blk += (int64_t)gridDim.x * kMseThreads) {
    const int64_t r = blk / bpr, cb = blk - r * bpr;
    const uint4 *p = (const uint4 *)(x + r * ld + cb * 16);
    const uint4 v0 = p[0], v1 = p[1];
    float k0;
    const int c0 = scale_code(absmax16(v0, v1), tab, inv6gs, &k0);
    int best = c0;
    float best_e = __builtin_inff();
    for (int i = 0; i < kMseCands; ++i) {
      const int c = min(max(c0 + cand_offset(i), 0), kE4M3MaxCode);
      const float kc = __uint_as_float(tab.ent[c].y);
      const uint2 q = encode16(v0, v1, kc, c, gs);
      const float err = row_error(v0, v1, q, e4m3_to_float((uint32_t)c), gs);
      if (err < best_e) {
        best_e = err;
        best = c;
      }
    }
    const uint2 packed = encode16(v0, v1, __uint_as_float(tab.ent[best].y), best, gs);
    ntstore8(o.codes + r * o.ld_codes + cb * 8, packed);
    ntstore_u8(o.scales + r * o.ld_scales + cb, (uint32_t)best);
  }
}

// 16x16 tiles: lane l of a wave holds row l % 16 of tile l / 16 of a group of 4 adjacent tiles
// in one 16-row band; the tile's error is the pairwise tree over its 16 lanes.
__global__ __launch_bounds__(kMseThreads) void k_mse_encode_2d(const uint16_t *__restrict__ w,
                                                               int64_t rows, int64_t cols,
                                                               int64_t ld, MseOut o,
                                                               const uint32_t *__restrict__ slots,
                                                               int n_slots,
                                                               float *__restrict__ gs_out) {
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kMseThreads / kWave];
  const float gs = mse_gs(slots, n_slots, tab, red, gs_out);
  const float inv6gs = tab.inv6gs;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWavesPerWg = kMseThreads / kWave;
  const int64_t tiles_c = cols / 16, groups_c = (tiles_c + 3) / 4;
  const int64_t n_groups = (rows / 16) * groups_c;
  for (int64_t g = (int64_t)blockIdx.x * kWavesPerWg + wave; g < n_groups;
       g += (int64_t)gridDim.x * kWavesPerWg) {
    const int64_t band = g / groups_c;
    const int64_t tc = (g - band * groups_c) * 4 + (lane >> 4);
    const int r = lane & 15;
    const bool valid = tc < tiles_c;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (valid) {
      const uint4 *p = (const uint4 *)(w + (band * 16 + r) * ld + tc * 16);
      v0 = p[0];
      v1 = p[1];
    }
    uint32_t m = absmax16(v0, v1);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, kWave));
    float k0;
    const int c0 = scale_code(m, tab, inv6gs, &k0);
    int best = c0;
    float best_e = __builtin_inff();
    for (int i = 0; i < kMseCands; ++i) {
      const int c = min(max(c0 + cand_offset(i), 0), kE4M3MaxCode);
      const float kc = __uint_as_float(tab.ent[c].y);
      const uint2 q = encode16(v0, v1, kc, c, gs);
      float err = row_error(v0, v1, q, e4m3_to_float((uint32_t)c), gs);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) err = err + __shfl_xor(err, off, kWave);
      if (err < best_e) {
        best_e = err;
        best = c;
      }
    }
    if (!valid) continue;
    const uint2 packed = encode16(v0, v1, __uint_as_float(tab.ent[best].y), best, gs);
    ntstore8(o.codes + (band * 16 + r) * o.ld_codes + tc * 8, packed);
    if (r == 0) ntstore_u8(o.scales + band * o.ld_scales + tc, (uint32_t)best);
  }
}

hipError_t launch_quantize_mse(const void *x, int64_t rows, int64_t cols, int64_t ld_x, bool two_d,
                               uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                               int64_t ld_scales, float *gs_out, void *ws, hipStream_t stream) {
  uint32_t *slots = (uint32_t *)ws;
  const int64_t chunks = rows * (cols / 8);
  int64_t ga = (chunks + kMseThreads * 4 - 1) / (kMseThreads * 4);
  ga = ga < 1 ? 1 : (ga > kMseAmaxWgs ? kMseAmaxWgs : ga);
  static_assert(kMseAmaxWgs <= kMaxAmaxSlots, "slot array too small");
  hipLaunchKernelGGL(k_mse_amax, dim3((unsigned)ga), dim3(kMseThreads), 0, stream,
                     (const uint16_t *)x, rows, cols, ld_x, slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const MseOut o{codes, ld_codes, scales, ld_scales};
  if (two_d) {
    const int64_t groups = (rows / 16) * ((cols / 16 + 3) / 4);
    int64_t g = (groups + 3) / 4;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    hipLaunchKernelGGL(k_mse_encode_2d, dim3((unsigned)g), dim3(kMseThreads), 0, stream,
                       (const uint16_t *)x, rows, cols, ld_x, o, slots, (int)ga, gs_out);
  } else {
    const int64_t blocks = rows * (cols / 16);
    int64_t g = (blocks + kMseThreads - 1) / kMseThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    hipLaunchKernelGGL(k_mse_encode_1d, dim3((unsigned)g), dim3(kMseThreads), 0, stream,
                       (const uint16_t *)x, rows, cols, ld_x, o, slots, (int)ga, gs_out);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
