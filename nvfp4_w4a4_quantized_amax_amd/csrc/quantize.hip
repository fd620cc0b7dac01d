// NVFP4 dynamic quantization kernels for gfx950.
//
// Pass 1 (k_amax): streaming read of the bf16 tensor, |x| max on the bit patterns (exact and
// order independent), one atomicMax per workgroup; the last workgroup to arrive turns amax into
// the FP32 global scale and builds the per-tensor tables (block-scale thresholds and element
// multipliers, see nvfp4_device.hpp), then clears the reduction cells.
// Pass 2 (k_encode_1d / k_encode_2d): re-reads the tensor (same workgroup -> same chunks, in
// reverse order, so the most recently read data is still in that XCD's L2), fits each block's
// E4M3 scale and writes packed codes and scales.
// Small tensors use k_quantize_small: one workgroup does both passes with an LDS barrier.
//
// The format steps follow "NVFP4 Explained: NVIDIA's 4-Bit Format for Faster AI Inference"
// ("How NVFP4 Represents a Value") and "What is NVFP4? 4-bit AI inference on NVIDIA Blackwell
// explained" ("What does NVFP4 mean?", "Why does scaling matter so much?").
#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / kWave;
constexpr int kTileChunks = 64;  // one wave step: 64 x 16 B = 512 bf16 values = 32 blocks

// Chunk c (8 bf16 values) -> element offset in x.
template <bool CONTIG>
__device__ __forceinline__ size_t chunk_x_offset(uint32_t c, FastDiv cpr, int64_t ld_x) {
  if (CONTIG) return (size_t)c * 8u;
  uint32_t r = fdiv(c, cpr);
  uint32_t col8 = c - r * cpr.d;
  return (size_t)r * (size_t)ld_x + (size_t)col8 * 8u;
}

// ---------------------------------------------------------------------------------------------
// Pass 1
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

template <bool CONTIG>
__global__ __launch_bounds__(kQThreads) void k_amax(const uint4 *__restrict__ x, uint32_t n_chunks,
                                                    uint32_t tiles_per_wg, FastDiv cpr,
                                                    int64_t ld_x, WsHeader *__restrict__ ws,
                                                    float *__restrict__ gs_out) {
  __shared__ uint32_t red[kQWaves];
  __shared__ uint32_t last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t t0 = blockIdx.x * tiles_per_wg;
  const uint32_t n_tiles = (n_chunks + kTileChunks - 1) / kTileChunks;
  const uint32_t t1 = min(t0 + tiles_per_wg, n_tiles);
  uint32_t m = 0;
  // Each wave walks tiles t0 + wave, t0 + wave + 4, ...; four tiles in flight per wave.
  uint32_t t = t0 + wave;
  for (; t + 3 * kQWaves < t1; t += 4 * kQWaves) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t c = (t + u * kQWaves) * kTileChunks + lane;
      v[u] = c < n_chunks ? x[chunk_x_offset<CONTIG>(c, cpr, ld_x) / 8u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) m = max(m, absmax8(v[u]));
  }
  for (; t < t1; t += kQWaves) {
    uint32_t c = t * kTileChunks + lane;
    if (c < n_chunks) m = max(m, absmax8(x[chunk_x_offset<CONTIG>(c, cpr, ld_x) / 8u]));
  }
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = red[0];
#pragma unroll
    for (int w = 1; w < kQWaves; ++w) b = max(b, red[w]);
    atomicMax(&ws->amax_bits, b);
    __threadfence();
    uint32_t ticket = atomicAdd(&ws->arrive, 1u);
    last = (ticket == gridDim.x - 1u);
  }
  __syncthreads();
  if (!last) return;
  // Last workgroup: every other workgroup's atomicMax happened before its arrival.
  __threadfence();
  __shared__ float s_gs;
  if (threadIdx.x == 0) {
    uint32_t amax = atomicExch(&ws->amax_bits, 0u);
    ws->arrive = 0u;
    float gs = global_scale_from_amax_bits(amax);
    s_gs = gs;
    ws->tab.gs = gs;
    ws->tab.inv6gs = inv6gs_of(gs);
    *gs_out = gs;
  }
  __syncthreads();
  if (threadIdx.x < 128) build_table_entry(&ws->tab, threadIdx.x, s_gs);
}

// ---------------------------------------------------------------------------------------------
// Pass 2, 1D blocks.  Lane i of a wave step holds chunk base + i; lanes 2j and 2j+1 hold the
// two halves of block base/2 + j and exchange their maxima with one shuffle.
// ---------------------------------------------------------------------------------------------
struct Enc1dOut {
  uint8_t *codes;
  int64_t ld_codes;
  uint8_t *scales;
  int64_t ld_scales;
};

template <bool CONTIG>
__device__ __forceinline__ void encode_chunk_1d(uint4 v, uint32_t c, bool valid, int lane,
                                                FastDiv cpr, const Enc1dOut &o, float gs,
                                                float inv6gs, const uint16_t *thresh,
                                                const float *mult) {
  uint32_t m = valid ? absmax8(v) : 0u;
  uint32_t bam = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
  if (!valid) return;
  int code = scale_code(bam, inv6gs, thresh);
  uint32_t packed = encode8(v, mult[code], code, gs);
  size_t co, so;
  if (CONTIG) {
    co = (size_t)c * 4u;
    so = (size_t)(c >> 1);
  } else {
    uint32_t r = fdiv(c, cpr);
    uint32_t col8 = c - r * cpr.d;
    co = (size_t)r * (size_t)o.ld_codes + (size_t)col8 * 4u;
    so = (size_t)r * (size_t)o.ld_scales + (size_t)(col8 >> 1);
  }
  *(uint32_t *)(o.codes + co) = packed;
  if ((lane & 1) == 0) o.scales[so] = (uint8_t)code;
}

template <bool CONTIG>
__global__ __launch_bounds__(kQThreads) void k_encode_1d(const uint4 *__restrict__ x,
                                                         uint32_t n_chunks, uint32_t tiles_per_wg,
                                                         FastDiv cpr, int64_t ld_x, Enc1dOut o,
                                                         const WsHeader *__restrict__ ws) {
  __shared__ uint16_t s_thresh[128];
  __shared__ float s_mult[128];
  if (threadIdx.x < 128) {
    s_thresh[threadIdx.x] = ws->tab.thresh[threadIdx.x];
    s_mult[threadIdx.x] = ws->tab.mult[threadIdx.x];
  }
  const float gs = ws->tab.gs;
  const float inv6gs = ws->tab.inv6gs;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t t0 = blockIdx.x * tiles_per_wg;
  const uint32_t n_tiles = (n_chunks + kTileChunks - 1) / kTileChunks;
  const uint32_t t1 = min(t0 + tiles_per_wg, n_tiles);
  if (t0 >= t1) return;
  // Walk this wave's tiles in the reverse of pass 1's order, two at a time.
  const uint32_t cnt = (t1 - t0 > (uint32_t)wave) ? (t1 - t0 - wave + kQWaves - 1) / kQWaves : 0u;
  int32_t i = (int32_t)cnt - 1;
  for (; i >= 1; i -= 2) {
    uint32_t ta = t0 + wave + (uint32_t)i * kQWaves;
    uint32_t tb = ta - kQWaves;
    uint32_t ca = ta * kTileChunks + lane, cb = tb * kTileChunks + lane;
    bool va = ca < n_chunks, vb = cb < n_chunks;
    uint4 a = va ? x[chunk_x_offset<CONTIG>(ca, cpr, ld_x) / 8u] : make_uint4(0, 0, 0, 0);
    uint4 b = vb ? x[chunk_x_offset<CONTIG>(cb, cpr, ld_x) / 8u] : make_uint4(0, 0, 0, 0);
    encode_chunk_1d<CONTIG>(a, ca, va, lane, cpr, o, gs, inv6gs, s_thresh, s_mult);
    encode_chunk_1d<CONTIG>(b, cb, vb, lane, cpr, o, gs, inv6gs, s_thresh, s_mult);
  }
  if (i == 0) {
    uint32_t ta = t0 + wave;
    uint32_t ca = ta * kTileChunks + lane;
    bool va = ca < n_chunks;
    uint4 a = va ? x[chunk_x_offset<CONTIG>(ca, cpr, ld_x) / 8u] : make_uint4(0, 0, 0, 0);
    encode_chunk_1d<CONTIG>(a, ca, va, lane, cpr, o, gs, inv6gs, s_thresh, s_mult);
  }
}

// ---------------------------------------------------------------------------------------------
// Pass 2, 16x16 tiles.  A wave covers 4 horizontally adjacent tiles of one 16-row band: lane l
// holds row l % 16 of tile l / 16 (32 bytes = 16 values); the tile maximum is a 16-lane
// butterfly.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kQThreads) void k_encode_2d(const uint16_t *__restrict__ w,
                                                         int64_t rows, int64_t cols, int64_t ld_w,
                                                         Enc1dOut o,
                                                         const WsHeader *__restrict__ ws) {
  __shared__ uint16_t s_thresh[128];
  __shared__ float s_mult[128];
  if (threadIdx.x < 128) {
    s_thresh[threadIdx.x] = ws->tab.thresh[threadIdx.x];
    s_mult[threadIdx.x] = ws->tab.mult[threadIdx.x];
  }
  const float gs = ws->tab.gs;
  const float inv6gs = ws->tab.inv6gs;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tiles_c = cols / 16;
  const int64_t groups_c = (tiles_c + 3) / 4;
  const int64_t n_groups = (rows / 16) * groups_c;
  for (int64_t g = (int64_t)blockIdx.x * kQWaves + wave; g < n_groups;
       g += (int64_t)gridDim.x * kQWaves) {
    const int64_t band = g / groups_c;
    const int64_t tc = (g - band * groups_c) * 4 + (lane >> 4);
    const int r = lane & 15;
    const bool valid = tc < tiles_c;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (valid) {
      const uint4 *p = (const uint4 *)(w + (band * 16 + r) * ld_w + tc * 16);
      v0 = p[0];
      v1 = p[1];
    }
    uint32_t m = max(absmax8(v0), absmax8(v1));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, kWave));
    if (!valid) continue;
    int code = scale_code(m, inv6gs, s_thresh);
    float k = s_mult[code];
    uint2 packed = make_uint2(encode8(v0, k, code, gs), encode8(v1, k, code, gs));
    *(uint2 *)(o.codes + (band * 16 + r) * o.ld_codes + tc * 8) = packed;
    if (r == 0) o.scales[band * o.ld_scales + tc] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------------------------
// Small tensors: one workgroup of 1024 threads runs both passes; tables live in LDS.  Optionally
// also writes the decoded A (code * block scale, fp16, gs not applied) for the small-M GEMM.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;

__global__ __launch_bounds__(kSmallThreads) void k_quantize_small(
    const uint16_t *__restrict__ x, int32_t rows, int32_t cols, int64_t ld_x, Enc1dOut o,
    float *__restrict__ gs_out, _Float16 *__restrict__ dec, int64_t ld_dec) {
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kSmallThreads / kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cpr = cols / 8;
  const int n_chunks = rows * cpr;
  uint32_t m = 0;
  for (int c = threadIdx.x; c < n_chunks; c += kSmallThreads) {
    int r = c / cpr, c8 = c - r * cpr;
    m = max(m, absmax8(*(const uint4 *)(x + (int64_t)r * ld_x + c8 * 8)));
  }
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0;
    for (int w = 0; w < kSmallThreads / kWave; ++w) b = max(b, red[w]);
    float gs = global_scale_from_amax_bits(b);
    tab.gs = gs;
    tab.inv6gs = inv6gs_of(gs);
    *gs_out = gs;
  }
  __syncthreads();
  if (threadIdx.x < 128) build_table_entry(&tab, threadIdx.x, tab.gs);
  __syncthreads();
  const float gs = tab.gs, inv6gs = tab.inv6gs;
  // Chunks are walked in wave-sized runs so that lane pairs always hold one whole block.
  for (int base = wave * kWave; base < n_chunks; base += kSmallThreads) {
    int c = base + lane;
    bool valid = c < n_chunks;
    int r = valid ? c / cpr : 0, c8 = valid ? c - r * cpr : 0;
    uint4 v = valid ? *(const uint4 *)(x + (int64_t)r * ld_x + c8 * 8) : make_uint4(0, 0, 0, 0);
    uint32_t mm = valid ? absmax8(v) : 0u;
    uint32_t bam = max(mm, (uint32_t)__shfl_xor((int)mm, 1, kWave));
    if (!valid) continue;
    int code = scale_code(bam, inv6gs, tab.thresh);
    uint32_t packed = encode8(v, tab.mult[code], code, gs);
    *(uint32_t *)(o.codes + (int64_t)r * o.ld_codes + c8 * 4) = packed;
    if ((lane & 1) == 0) o.scales[(int64_t)r * o.ld_scales + (c8 >> 1)] = (uint8_t)code;
    if (dec) {
      half8_t d = decode8_f16(packed, scale_f16x2((uint32_t)code));
      *(half8_t *)(dec + (int64_t)r * ld_dec + c8 * 8) = d;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------------
static FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1ull);
  return f;
}

int quant_grid_wgs() { return 256 * 4; }

hipError_t launch_amax(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *ws,
                       float *gs_out, int *grid_out, uint32_t *tiles_per_wg_out,
                       hipStream_t stream) {
  const uint32_t cpr = (uint32_t)(cols / 8);
  const uint32_t n_chunks = (uint32_t)(rows * (cols / 8));
  const uint32_t n_tiles = (n_chunks + kTileChunks - 1) / kTileChunks;
  uint32_t grid = (uint32_t)quant_grid_wgs();
  uint32_t tpw = (n_tiles + grid - 1) / grid;
  if (tpw == 0) tpw = 1;
  grid = (n_tiles + tpw - 1) / tpw;
  if (grid == 0) grid = 1;
  *grid_out = (int)grid;
  *tiles_per_wg_out = tpw;
  FastDiv f = make_fastdiv(cpr);
  const bool contig = (ld_x == cols);
  if (contig)
    hipLaunchKernelGGL(k_amax<true>, dim3(grid), dim3(kQThreads), 0, stream, (const uint4 *)x,
                       n_chunks, tpw, f, ld_x, (WsHeader *)ws, gs_out);
  else
    hipLaunchKernelGGL(k_amax<false>, dim3(grid), dim3(kQThreads), 0, stream, (const uint4 *)x,
                       n_chunks, tpw, f, ld_x, (WsHeader *)ws, gs_out);
  return hipGetLastError();
}

hipError_t launch_encode_1d(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                            const void *ws, int grid, uint32_t tpw, hipStream_t stream) {
  const uint32_t cpr = (uint32_t)(cols / 8);
  const uint32_t n_chunks = (uint32_t)(rows * (cols / 8));
  FastDiv f = make_fastdiv(cpr);
  Enc1dOut o{codes, ld_codes, scales, ld_scales};
  const bool contig = (ld_x == cols) && (ld_codes == cols / 2) && (ld_scales == cols / 16);
  if (contig)
    hipLaunchKernelGGL(k_encode_1d<true>, dim3(grid), dim3(kQThreads), 0, stream,
                       (const uint4 *)x, n_chunks, tpw, f, ld_x, o, (const WsHeader *)ws);
  else
    hipLaunchKernelGGL(k_encode_1d<false>, dim3(grid), dim3(kQThreads), 0, stream,
                       (const uint4 *)x, n_chunks, tpw, f, ld_x, o, (const WsHeader *)ws);
  return hipGetLastError();
}

hipError_t launch_encode_2d(const void *w, int64_t rows, int64_t cols, int64_t ld_w,
                            uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                            const void *ws, hipStream_t stream) {
  Enc1dOut o{codes, ld_codes, scales, ld_scales};
  const int64_t groups = (rows / 16) * ((cols / 16 + 3) / 4);
  int64_t grid = (groups + kQWaves - 1) / kQWaves;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(k_encode_2d, dim3((unsigned)grid), dim3(kQThreads), 0, stream,
                     (const uint16_t *)w, rows, cols, ld_w, o, (const WsHeader *)ws);
  return hipGetLastError();
}

hipError_t launch_quantize_small(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                                 int64_t ld_scales, float *gs_out, _Float16 *dec, int64_t ld_dec,
                                 hipStream_t stream) {
  Enc1dOut o{codes, ld_codes, scales, ld_scales};
  hipLaunchKernelGGL(k_quantize_small, dim3(1), dim3(kSmallThreads), 0, stream,
                     (const uint16_t *)x, (int32_t)rows, (int32_t)cols, ld_x, o, gs_out, dec,
                     ld_dec);
  return hipGetLastError();
}

}  // namespace nvfp4
