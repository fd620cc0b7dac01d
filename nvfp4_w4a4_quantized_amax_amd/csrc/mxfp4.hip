// MXFP4 for gfx950: the same E2M1 elements as NVFP4 with one E8M0 (power-of-two) scale per 32
// consecutive values and no tensor scale ("What is NVFP4? 4-bit AI inference on NVIDIA
// Blackwell explained", section "NVFP4 versus MXFP4"; "NVFP4 Explained: NVIDIA's 4-Bit Format
// for Faster AI Inference", section "Why the Block Scale Uses FP8 E4M3").
//
// Scale of a block: X = 2^e, e = floor(log2(bamax)) - 2 clamped to [-127, 127] (the conversion
// rule of the MX specification; 2 is the exponent of E2M1's largest value), stored as e + 127.
// Element: nearest E2M1 value to x / X, ties to even, saturating at 6, sign = signbit(x).
// x / X = x * 2^-e is exact in fp32 for every bf16 x, so the hardware FP4 conversion of that
// product (unit scale: round to nearest even, saturating) gives the code directly.
//
// Unlike NVFP4's E4M3 scales, these scales are what CDNA4's scaled MFMA consumes natively:
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands takes, per lane, 16 code bytes (32
// consecutive K values of one row, element i in nibble i) and the E8M0 byte of that block, so
// a lane's fragment is exactly one MXFP4 block of the packed tensor.

#include "nvfp4_device.hpp"
#include "gemm_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// E8M0 exponent of a block from its largest |bf16| bit pattern.  For a normal maximum,
// floor(log2) is the exponent field minus 127; zero and subnormal maxima (field 0) and the
// smallest normals land below -127 and clamp there.  The field is at most 254, so e <= 125.
__device__ __forceinline__ int mx_exponent(uint32_t bam) { return max((int)(bam >> 7) - 129, -127); }

// 2^-e as a float (e in [-127, 125]: the biased exponent 127 - e is in [2, 254]).
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------------------------------------
// Quantize: lane l of a wave takes the 16-byte chunk (8 values) l of a 1 KiB run, so loads and
// stores are contiguous across the wave; the four lanes of a 32-value block share their maxima
// with two cross-lane steps.  Chunk u of the tensor is row u / (cols / 8), chunk u % (cols / 8).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_mx_quantize(const uint16_t *__restrict__ x, int64_t ld_x,
                                                     uint32_t n_chunks, FastDiv cpr,
                                                     uint8_t *__restrict__ codes, int64_t ld_codes,
                                                     uint8_t *__restrict__ scales,
                                                     int64_t ld_scales) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < n_chunks; u += stride) {
    const uint32_t r = fdiv(u, cpr), c = u - r * cpr.d;
    const uint4 v = *(const uint4 *)(x + (int64_t)r * ld_x + (int64_t)c * 8);
    uint32_t m = absmax8(v);
    // n_chunks and the row length are multiples of 4, so the four lanes of a block are all
    // in the loop together.
    m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
    const int e = mx_exponent(m);
    const uint32_t q = encode8_fast(v, mx_inv_scale(e));
    *(uint32_t *)(codes + (int64_t)r * ld_codes + (int64_t)c * 4) = q;
    if ((c & 3) == 0) scales[(int64_t)r * ld_scales + (c >> 2)] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------------------------
// Dequantize: value = code value * 2^(byte - 127).  bf16 output: one thread = 8 values (one code
// word, 16 bytes out).  fp32 output: one thread = 4 values (16 bits of codes, 16 bytes out), so
// that one store instruction of a wave covers 1 KiB of contiguous output; with 8 values per
// thread the two 16-byte stores of a lane interleave at a 32-byte stride, which wrote at about a
// third of the HBM rate.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float mx_scale_value(uint32_t b) {
  // 2^(b - 127) for b in [0, 254]: b = 0 is the fp32 subnormal 2^-127.
  return b ? __uint_as_float(b << 23) : 0x1p-127f;
}

__global__ __launch_bounds__(256) void k_mx_dequantize_bf16(const uint8_t *__restrict__ codes,
                                                            int64_t ld_codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t ld_scales, uint32_t n_chunks,
                                                            FastDiv cpr,
                                                            uint16_t *__restrict__ y,
                                                            int64_t ld_y) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < n_chunks; u += stride) {
    const uint32_t r = fdiv(u, cpr), c = u - r * cpr.d;
    const uint32_t q = *(const uint32_t *)(codes + (int64_t)r * ld_codes + (int64_t)c * 4);
    const float s = mx_scale_value(scales[(int64_t)r * ld_scales + (c >> 2)]);
    const floatx2_t f[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3)};
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[2 * j] = f32_to_bf16_rne(f[j][0] * s);
      h[2 * j + 1] = f32_to_bf16_rne(f[j][1] * s);
    }
    ntstore16(y + (int64_t)r * ld_y + (int64_t)c * 8,
              make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16)));
  }
}

// n_quads = rows * cols / 4 < 2^32; the loop counter is 64-bit so that the last stride step
// cannot wrap, and the quotient's sum is taken in 64 bits for the same reason.
__global__ __launch_bounds__(256) void k_mx_dequantize_f32(const uint8_t *__restrict__ codes,
                                                           int64_t ld_codes,
                                                           const uint8_t *__restrict__ scales,
                                                           int64_t ld_scales, uint32_t n_quads,
                                                           FastDiv qpr, float *__restrict__ y,
                                                           int64_t ld_y) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t u64 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u64 < n_quads;
       u64 += stride) {
    const uint32_t u = (uint32_t)u64;
    // fdiv's 32-bit sum holds below 2^31 only; u can reach 2^32 here, so sum in 64 bits.
    const uint32_t r = (uint32_t)(((uint64_t)__umulhi(u, qpr.mul) + u) >> qpr.shift);
    const uint32_t c = u - r * qpr.d;
    const uint32_t q = *(const uint16_t *)(codes + (int64_t)r * ld_codes + (int64_t)c * 2);
    const float s = mx_scale_value(scales[(int64_t)r * ld_scales + (c >> 3)]);
    const floatx2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    const floatx2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    ntstore16(y + (int64_t)r * ld_y + (int64_t)c * 4,
              make_uint4(__float_as_uint(f0[0] * s), __float_as_uint(f0[1] * s),
                         __float_as_uint(f1[0] * s), __float_as_uint(f1[1] * s)));
  }
}

// ---------------------------------------------------------------------------------------------
// GEMM Y = A . W^T (both MXFP4, K-contiguous), fp32 accumulation, bf16 out.  The scaled MFMA
// applies both E8M0 scales itself, so there is no decode: fragments go from LDS (or memory)
// straight to the matrix core.
// ---------------------------------------------------------------------------------------------
struct MxArgs {
  const uint8_t *a_codes, *a_scales, *w_codes, *w_scales;
  int64_t ld_ac, ld_as, ld_wc, ld_ws;
  int64_t m, n, k;
  uint16_t *y;
  int64_t ld_y;
  int tiles_m, tiles_n;
  // Activation quantized inside the product (k_gemm_mx_mid, small M): bf16 A, and where
  // workgroup 0 writes its MXFP4 form (null: nowhere).
  const uint16_t *a_bf16;
  int64_t ld_a;
  uint8_t *aq_codes, *aq_scales;
  int64_t ld_aqc, ld_aqs;
};

__device__ __forceinline__ floatx16_t mx_mfma(const u32x4_t &a, const u32x4_t &w, uint32_t sa,
                                              uint32_t sw, const floatx16_t &c) {
  // FP4 operands occupy only the first four registers of the 8-register operand; the rest is
  // left undefined (the instruction does not read it).
  const i32x8_t av = __builtin_shufflevector((i32x4_t)a, (i32x4_t)a, 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8_t wv = __builtin_shufflevector((i32x4_t)w, (i32x4_t)w, 0, 1, 2, 3, -1, -1, -1, -1);
  // cbsz = blgp = 4: both operands FP4 (E2M1); scale byte 0 of each scale register.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, wv, c, 4, 4, 0, (int)sa, 0, (int)sw);
}

// Pipelined 256 x 256 tiles (K a multiple of 64, scale rows 2-byte aligned).  One 64-wide K
// window of a tile is 256 rows x 32 code bytes of A and of W plus 2 scale bytes per row; it is
// loaded into registers two windows ahead, stored to one of two LDS stages one window ahead and
// read back by the waves that use it.  Each wave computes 128 x 128 as 4 x 4 MFMA tiles of
// 32 x 32; per window that is 16 MFMAs, the first 8 before and the last 8 after the barrier
// that publishes the next window, so the LDS reads of the next window hide behind the second
// half.  The scale bytes are read from LDS one by one: extracting them from 16-bit reads made
// the register allocator spill the accumulators.
struct MxStage {
  uint8_t a[256 * 32];
  uint8_t w[256 * 32];
  uint16_t as[256];
  uint16_t ws[256];
};

struct MxWindowRegs {
  u32x4_t a0, a1, w0, w1;
  uint16_t as, ws;
};

struct MxFrags {
  u32x4_t a[4], w[4];
  uint32_t sa[4], sw[4];
};

__device__ __forceinline__ void mx_load_window(MxWindowRegs &r, const uint8_t *const (&ga)[2],
                                               const uint8_t *const (&gw)[2], const uint8_t *gas,
                                               const uint8_t *gws, int64_t win) {
  r.a0 = *(const u32x4_t *)(ga[0] + win * 32);
  r.a1 = *(const u32x4_t *)(ga[1] + win * 32);
  r.w0 = *(const u32x4_t *)(gw[0] + win * 32);
  r.w1 = *(const u32x4_t *)(gw[1] + win * 32);
  r.as = *(const uint16_t *)(gas + win * 2);
  r.ws = *(const uint16_t *)(gws + win * 2);
}

__device__ __forceinline__ void mx_store_window(const MxWindowRegs &r, MxStage &S, int tid) {
  // chunk c = i * 256 + tid is half c % 2 of row c / 2
  const int o0 = code_offset(tid >> 1, tid & 1), o1 = code_offset(128 + (tid >> 1), tid & 1);
  *(u32x4_t *)(S.a + o0) = r.a0;
  *(u32x4_t *)(S.a + o1) = r.a1;
  *(u32x4_t *)(S.w + o0) = r.w0;
  *(u32x4_t *)(S.w + o1) = r.w1;
  S.as[tid] = r.as;
  S.ws[tid] = r.ws;
}

// Lane (row lr, half kh) of fragment f: row wm * 128 + f * 32 + lr of A, K half kh (one 32-value
// block) with its scale byte; likewise for W.
__device__ __forceinline__ void mx_read_frags(const MxStage &S, int wm, int wn, int lr, int kh,
                                              MxFrags &fr) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int ra = wm * 128 + f * 32 + lr, rw = wn * 128 + f * 32 + lr;
    fr.a[f] = *(const u32x4_t *)(S.a + code_offset(ra, kh));
    fr.w[f] = *(const u32x4_t *)(S.w + code_offset(rw, kh));
    fr.sa[f] = ((const uint8_t *)S.as)[ra * 2 + kh];
    fr.sw[f] = ((const uint8_t *)S.ws)[rw * 2 + kh];
  }
}

// Rows f0, f0 + 1 of the 4 x 4 MFMA tiles.
template <int F0>
__device__ __forceinline__ void mx_mfma_half(const MxFrags &fr, floatx16_t (&acc)[4][4]) {
#pragma unroll
  for (int f = F0; f < F0 + 2; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = mx_mfma(fr.a[f], fr.w[g], fr.sa[f], fr.sw[g], acc[f][g]);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx_lds(MxArgs p) {
  __shared__ __align__(16) MxStage st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m_tile = (int64_t)tm * 256, n_tile = (int64_t)tn * 256;

  // This thread's share of every window's loads (rows clamped into the matrix; results of
  // clamped rows are never stored).
  const uint8_t *ga[2], *gw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = i * 256 + tid, row = c >> 1, half = c & 1;
    ga[i] = p.a_codes + min(m_tile + row, p.m - 1) * p.ld_ac + half * 16;
    gw[i] = p.w_codes + min(n_tile + row, p.n - 1) * p.ld_wc + half * 16;
  }
  const uint8_t *gas = p.a_scales + min(m_tile + tid, p.m - 1) * p.ld_as;
  const uint8_t *gws = p.w_scales + min(n_tile + tid, p.n - 1) * p.ld_ws;
  const int64_t nwin = p.k / 64;  // >= 1

  floatx16_t acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = floatx16_t{};

  // Window 0 goes to stage 0 and window 1 stays in registers.  In window w, window w + 1 is
  // stored to stage (w + 1) % 2 (whose previous window every wave read before the last
  // barrier) and window w + 2 is loaded; after the barrier, window w + 1 is read back.
  // Windows past the end are clamped to the last one.
  MxWindowRegs r;
  mx_load_window(r, ga, gw, gas, gws, 0);
  mx_store_window(r, st[0], tid);
  mx_load_window(r, ga, gw, gas, gws, min((int64_t)1, nwin - 1));
  lds_barrier();
  MxFrags fa, fb;
  mx_read_frags(st[0], wm, wn, lr, kh, fa);
  // One window: its first 8 MFMAs overlap the store of window w + 1 and the loads of window
  // w + 2, the last 8 the reads of window w + 1 (the scheduler is asked to alternate them).
  auto window = [&](int64_t w, const MxFrags &cur, MxFrags &nxt) {
    mx_store_window(r, st[(w + 1) & 1], tid);
    mx_load_window(r, ga, gw, gas, gws, min(w + 2, nwin - 1));
    mx_mfma_half<0>(cur, acc);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < 6) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      if (i < 6) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // vector memory read
    }
    lds_barrier();
    mx_read_frags(st[(w + 1) & 1], wm, wn, lr, kh, nxt);
    mx_mfma_half<2>(cur, acc);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Two windows per iteration, so the fragment registers alternate without copies.  The last
  // window also stores, loads and reads a (clamped) window past the end, which is never used.
  int64_t w = 0;
  for (; w + 1 < nwin; w += 2) {
    window(w, fa, fb);
    window(w + 1, fb, fa);
  }
  if (w < nwin) window(w, fa, fb);

  const int64_t m0 = m_tile + wm * 128, n0 = n_tile + wn * 128;
  const bool full = m_tile + 256 <= p.m && n_tile + 256 <= p.n;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {  // rows i and i + 1 are adjacent
        const int64_t row = m0 + f * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
        const uint32_t pk = bf16x2_rne(acc[f][g][i], acc[f][g][i + 1]);
        if (full || (row < p.m && col < p.n)) ntstore_u16(p.y + row * p.ld_y + col, pk);
        if (full || (row + 1 < p.m && col < p.n))
          ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
      }
    }
}

// Wide-window pipeline (K a multiple of 512; 16-byte aligned scale rows; operands addressable
// with 32-bit offsets).  A window is 256 K values: 128 code bytes per row, so the 16-byte loads
// of 8 adjacent lanes cover one whole 128-byte line and each row is fetched once per window.
// Scale bytes travel 16 per row (two windows) per load.  The codes of a row sit in LDS as 8
// chunks of 16 bytes, chunk c at slot c ^ wide_swizzle(row): the fragment reads (one chunk of 8
// or 16 consecutive rows at a time) and the window stores (8 whole rows per wave) then touch
// every bank once.  The scale bytes of a row and window, b0..b7 (block j covers K values
// 32j .. 32j + 31 of the window), are stored as the word b0 b2 b4 b6 followed by b1 b3 b5 b7:
// the lane that feeds K half kh of every 64-wide step reads word kh once per window, and the
// MFMA picks byte s of it for step s through its operand select.
//
// Per window each wave issues 64 MFMAs in four 64-wide steps; the fragments of step s + 1 are
// read from LDS while step s runs.  During step 0 the registers holding window w + 1 are stored
// to the free LDS stage and refilled with window w + 2, one store and one load per MFMA; one
// barrier per window, before step 3, publishes window w + 1.  Rows past the end of A or W are
// read with offsets beyond the buffer, which the hardware answers with zeros and no memory
// access.  (Compared with the 64-wide window, this quarters the cache lines fetched per flop:
// there every window touched each row's line for 32 code bytes and 2 scale bytes.)
constexpr int kMxWideK = 256;

struct MxWideStage {
  uint8_t a[256 * 128];
  uint8_t w[256 * 128];
  uint32_t as[256 * 2];
  uint32_t ws[256 * 2];
};

__device__ __forceinline__ int wide_swizzle(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }

struct MxWideRegs {
  u32x4_t a[8], w[8];
};

struct MxWideFrags {
  u32x4_t a[4], w[4];
};

template <int S>
__device__ __forceinline__ floatx16_t mx_mfma_sel(const u32x4_t &a, const u32x4_t &w, uint32_t sa,
                                                  uint32_t sw, const floatx16_t &c) {
  const i32x8_t av = __builtin_shufflevector((i32x4_t)a, (i32x4_t)a, 0, 1, 2, 3, -1, -1, -1, -1);
  const i32x8_t wv = __builtin_shufflevector((i32x4_t)w, (i32x4_t)w, 0, 1, 2, 3, -1, -1, -1, -1);
  // both operands FP4; byte S of each scale word
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, wv, c, 4, 4, S, (int)sa, S, (int)sw);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx_wide(MxArgs p) {
  __shared__ __align__(16) MxWideStage st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const uint32_t m_tile = (uint32_t)tm * 256, n_tile = (uint32_t)tn * 256;

  const __amdgpu_buffer_rsrc_t bac = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.a_codes, 0, (int)((p.m - 1) * p.ld_ac + p.k / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t bwc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.w_codes, 0, (int)((p.n - 1) * p.ld_wc + p.k / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t bas = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.a_scales, 0, (int)((p.m - 1) * p.ld_as + p.k / 32), 0x00020000);
  const __amdgpu_buffer_rsrc_t bws = __builtin_amdgcn_make_buffer_rsrc(
      (void *)p.w_scales, 0, (int)((p.n - 1) * p.ld_ws + p.k / 32), 0x00020000);

  // Chunk i of this thread's share of a window: row i * 32 + tid / 8, 16-byte part tid % 8.
  const uint32_t lrow = (uint32_t)tid >> 3, part = (uint32_t)tid & 7;
  const uint32_t ga0 = (m_tile + lrow) * (uint32_t)p.ld_ac + part * 16;
  const uint32_t gw0 = (n_tile + lrow) * (uint32_t)p.ld_wc + part * 16;
  const uint32_t ga_step = 32 * (uint32_t)p.ld_ac, gw_step = 32 * (uint32_t)p.ld_wc;
  const uint32_t gas0 = (m_tile + tid) * (uint32_t)p.ld_as;
  const uint32_t gws0 = (n_tile + tid) * (uint32_t)p.ld_ws;
  const int st_code = lrow * 128 + ((part ^ wide_swizzle(lrow)) << 4);
  // Fragment f of A is row wm * 128 + f * 32 + lr; its swizzle depends on lr only.
  const int sz = wide_swizzle(lr);
  const int fa_row = (wm * 128 + lr) * 128, fw_row = (wn * 128 + lr) * 128;
  const int nwin = (int)(p.k / kMxWideK);  // even, >= 2

  floatx16_t acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = floatx16_t{};

  MxWideRegs r;
  u32x4_t sa_pair, sw_pair;  // scale bytes of two windows, this thread's A row and W row
  auto load_codes = [&](int win) {
    const uint32_t o = (uint32_t)win * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(bac, (int)(ga0 + i * ga_step + o), 0, 0);
      r.w[i] = __builtin_amdgcn_raw_buffer_load_b128(bwc, (int)(gw0 + i * gw_step + o), 0, 0);
    }
  };
  auto load_scales = [&](int win) {  // win even: windows win and win + 1
    sa_pair = __builtin_amdgcn_raw_buffer_load_b128(bas, (int)(gas0 + (uint32_t)win * 8), 0, 0);
    sw_pair = __builtin_amdgcn_raw_buffer_load_b128(bws, (int)(gws0 + (uint32_t)win * 8), 0, 0);
  };
  auto store_codes = [&](MxWideStage &S) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(u32x4_t *)(S.a + st_code + i * 4096) = r.a[i];
      *(u32x4_t *)(S.w + st_code + i * 4096) = r.w[i];
    }
  };
  auto store_scales = [&](MxWideStage &S, int odd) {
    const uint32_t alo = odd ? sa_pair[2] : sa_pair[0], ahi = odd ? sa_pair[3] : sa_pair[1];
    const uint32_t wlo = odd ? sw_pair[2] : sw_pair[0], whi = odd ? sw_pair[3] : sw_pair[1];
    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
    *(u32x2_t *)(S.as + tid * 2) = u32x2_t{__builtin_amdgcn_perm(ahi, alo, 0x06040200u),
                                           __builtin_amdgcn_perm(ahi, alo, 0x07050301u)};
    *(u32x2_t *)(S.ws + tid * 2) = u32x2_t{__builtin_amdgcn_perm(whi, wlo, 0x06040200u),
                                           __builtin_amdgcn_perm(whi, wlo, 0x07050301u)};
  };
  auto read_frags = [&](const MxWideStage &S, int s, MxWideFrags &fr) {
    const int o = ((2 * s + kh) ^ sz) << 4;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fr.a[f] = *(const u32x4_t *)(S.a + fa_row + f * 4096 + o);
      fr.w[f] = *(const u32x4_t *)(S.w + fw_row + f * 4096 + o);
    }
  };
  uint32_t sa[4], sw[4];  // scale words of the current window, per fragment
  auto read_scales = [&](const MxWideStage &S, uint32_t (&a)[4], uint32_t (&b)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      a[f] = S.as[(wm * 128 + f * 32 + lr) * 2 + kh];
      b[f] = S.ws[(wn * 128 + f * 32 + lr) * 2 + kh];
    }
  };

  // Prologue: window 0 to stage 0, window 1 in registers.
  load_scales(0);
  load_codes(0);
  store_codes(st[0]);
  store_scales(st[0], 0);
  load_codes(1);
  lds_barrier();
  MxWideFrags fx, fy;
  read_frags(st[0], 0, fx);
  read_scales(st[0], sa, sw);

  // One window: stage `cur` holds window w, registers hold window w + 1 (and the scale pair of
  // windows w and w + 1 if w is even, else of w + 1 and w + 2 ... loaded at the right time).
  auto window = [&](int w, MxWideStage &cur, MxWideStage &nxt, int odd) {
    uint32_t na[4], nb[4];
    // step 0: store window w + 1, issue the loads of window w + 2 (and its scale pair)
    store_codes(nxt);
    store_scales(nxt, !odd);
    const int w2 = min(w + 2, nwin - 1);
    if (!odd) load_scales(w2 & ~1);
    load_codes(w2);
    read_frags(cur, 1, fy);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = mx_mfma_sel<0>(fx.a[f], fx.w[g], sa[f], sw[g], acc[f][g]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // vector memory read
      if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    read_frags(cur, 2, fx);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = mx_mfma_sel<1>(fy.a[f], fy.w[g], sa[f], sw[g], acc[f][g]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_frags(cur, 3, fy);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = mx_mfma_sel<2>(fx.a[f], fx.w[g], sa[f], sw[g], acc[f][g]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    read_frags(nxt, 0, fx);
    read_scales(nxt, na, nb);
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = mx_mfma_sel<3>(fy.a[f], fy.w[g], sa[f], sw[g], acc[f][g]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sa[f] = na[f];
      sw[f] = nb[f];
    }
  };
  for (int w = 0; w < nwin; w += 2) {
    window(w, st[0], st[1], 0);
    window(w + 1, st[1], st[0], 1);
  }

  const int64_t m0 = m_tile + wm * 128, n0 = n_tile + wn * 128;
  const bool full = m_tile + 256 <= p.m && n_tile + 256 <= p.n;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {  // rows i and i + 1 are adjacent
        const int64_t row = m0 + f * 32 + 8 * (i >> 2) + 4 * kh + (i & 3);
        const uint32_t pk = bf16x2_rne(acc[f][g][i], acc[f][g][i + 1]);
        if (full || (row < p.m && col < p.n)) ntstore_u16(p.y + row * p.ld_y + col, pk);
        if (full || (row + 1 < p.m && col < p.n))
          ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
      }
    }
}

// Small and mid-size M (M <= 128): output tiles of 32FM x 32FN, one per workgroup.  The 4 waves
// take the four quarters of K; each computes the whole tile over its quarter (FM x FN MFMA tiles
// of 32 x 32, straight from memory: a lane's operand is one MXFP4 block) with DEPTH 64-wide
// windows of loads in flight, and the four partial tiles are added through LDS.  Scales come
// 8 bytes (4 windows) per row and load: lane half kh shifts the word by 8 kh, and the MFMA's
// scale select picks byte 0 or 2 of each 32-bit half.  K must be a multiple of 256 * DEPTH and
// scale rows 8-byte aligned; W is read once per 32FM-row slice of A.
// FA (one row tile, M * K <= kMxFaMaxValues): A arrives as bf16 and every workgroup quantizes
// all of it into LDS exactly as k_mx_quantize does (8-value chunks, the four lanes of a block
// sharing its maximum); its loads go out before W's, so waiting for them waits for nothing
// else, and workgroup 0 also writes the quantized A when asked to.
template <int FM, int FN>
struct MxMidWin {
  u32x4_t a[FM], w[FN];
};

template <int FM, int FN, int DEPTH>
struct MxMidScales {
  uint2 a[FM][DEPTH / 4], w[FN][DEPTH / 4];
};

constexpr int kMxFaChunks = 8;                        // 8-value chunks of A per thread
constexpr int64_t kMxFaMaxValues = kMxFaChunks * 8 * 256;  // 16384

template <int FM, int FN, int DEPTH, bool FA>
__global__ __launch_bounds__(256) void k_gemm_mx_mid(MxArgs p) {
  static_assert(DEPTH % 4 == 0, "a scale load covers 4 windows");
  static_assert(!FA || FM == 1, "the fused activation is one row tile");
  __shared__ float s_red[4][FM][FN][16][kWave];  // [wave][f][g][register][lane]
  // FA: A's codes (m rows of k / 2 bytes), then its scales (m rows of k / 32 bytes).
  extern __shared__ __align__(16) uint8_t s_fa[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, kh = lane >> 5;
  const uint32_t sh = 8u * kh;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * (32 * FM), n0 = (int64_t)tn * (32 * FN);
  // Rows clamped into the matrices; results of clamped rows are never stored.
  const int64_t wpw = p.k / 256;  // 64-wide windows per wave, a multiple of DEPTH
  const int64_t w_first = wave * wpw;
  const uint8_t *ac[FM], *as[FM], *wc[FN], *ws[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t ra = min(m0 + f * 32 + lr, p.m - 1);
    ac[f] = p.a_codes + ra * p.ld_ac + kh * 16 + w_first * 32;
    as[f] = p.a_scales + ra * p.ld_as + w_first * 2;
  }
#pragma unroll
  for (int g = 0; g < FN; ++g) {
    const int64_t rw = min(n0 + g * 32 + lr, p.n - 1);
    wc[g] = p.w_codes + rw * p.ld_wc + kh * 16 + w_first * 32;
    ws[g] = p.w_scales + rw * p.ld_ws + w_first * 2;
  }
  // FA: this lane's rows of A in LDS (one row tile: m0 = 0).
  const int64_t fa_row = min((int64_t)lr, p.m - 1);
  const uint8_t *lac = s_fa + fa_row * (p.k / 2) + kh * 16 + w_first * 32;
  const uint8_t *las = s_fa + p.m * (p.k / 2) + fa_row * (p.k / 32) + kh + w_first * 2;
  floatx16_t acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) acc[f][g] = floatx16_t{};
  // FA: A's 8-value chunks u = threadIdx.x + 256 t, loaded before any load of W (past the
  // end: the last chunk again, never stored).
  // (fa_n <= 2048: 32-bit arithmetic.)
  const uint32_t fa_cpr = (uint32_t)(p.k / 8), fa_n = (uint32_t)p.m * fa_cpr;
  uint4 xa[FA ? kMxFaChunks : 1];
  if (FA) {
#pragma unroll
    for (int t = 0; t < kMxFaChunks; ++t) {
      const uint32_t u = min(threadIdx.x + 256u * t, fa_n - 1u);
      const uint32_t r = u / fa_cpr, c = u - r * fa_cpr;
      xa[t] = *(const uint4 *)(p.a_bf16 + (int64_t)r * p.ld_a + c * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  auto load = [&](MxMidWin<FM, FN> &r, int64_t win) {
    if (!FA) {
#pragma unroll
      for (int f = 0; f < FM; ++f) r.a[f] = *(const u32x4_t *)(ac[f] + win * 32);
    }
#pragma unroll
    for (int g = 0; g < FN; ++g) r.w[g] = *(const u32x4_t *)(wc[g] + win * 32);
  };
  // scales of windows win .. win + DEPTH - 1
  auto load_scales = [&](MxMidScales<FM, FN, DEPTH> &q, int64_t win) {
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int u = 0; u < DEPTH / 4; ++u)
        if (!FA) q.a[f][u] = *(const uint2 *)(as[f] + (win + 4 * u) * 2);
#pragma unroll
    for (int g = 0; g < FN; ++g)
#pragma unroll
      for (int u = 0; u < DEPTH / 4; ++u) q.w[g][u] = *(const uint2 *)(ws[g] + (win + 4 * u) * 2);
  };
  // window j of the round whose scales are q (window win of the wave's share; FA reads A's
  // operand and scale byte from LDS, the byte moved to where the scale select looks)
  auto compute = [&](const MxMidWin<FM, FN> &r, const MxMidScales<FM, FN, DEPTH> &q, int j,
                     int64_t win) {
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const u32x4_t av = FA ? *(const u32x4_t *)(lac + win * 32) : r.a[f];
      const uint32_t sa = FA ? (uint32_t)las[win * 2] << ((j & 1) ? 16 : 0)
                             : ((j >> 1) & 1 ? q.a[f][j >> 2].y : q.a[f][j >> 2].x) >> sh;
#pragma unroll
      for (int g = 0; g < FN; ++g) {
        const uint32_t sw = ((j >> 1) & 1 ? q.w[g][j >> 2].y : q.w[g][j >> 2].x) >> sh;
        if (j & 1)
          acc[f][g] = mx_mfma_sel<2>(av, r.w[g], sa, sw, acc[f][g]);
        else
          acc[f][g] = mx_mfma_sel<0>(av, r.w[g], sa, sw, acc[f][g]);
      }
    }
  };
  // Full rounds refill every slot after using it (the next round's scales first), the last
  // round only drains; the scheduling barriers keep the loads in window order.
  MxMidWin<FM, FN> ring[DEPTH];
  MxMidScales<FM, FN, DEPTH> cur, nxt;
  load_scales(cur, 0);
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) {
    load(ring[j], j);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (FA) {
    // Quantize A into LDS (and, from workgroup 0, into the caller's buffers).  fa_n and 256 are
    // multiples of 4, so the four lanes of a block are in or out together.
    uint8_t *sac = s_fa, *sas = s_fa + p.m * (p.k / 2);
#pragma unroll
    for (int t = 0; t < kMxFaChunks; ++t) {
      const uint32_t u = threadIdx.x + 256u * t;
      uint32_t mm = absmax8(xa[t]);
      mm = max(mm, (uint32_t)__shfl_xor((int)mm, 1, kWave));
      mm = max(mm, (uint32_t)__shfl_xor((int)mm, 2, kWave));
      if (u < fa_n) {
        const uint32_t r = u / fa_cpr, c = u - r * fa_cpr;
        const int e = mx_exponent(mm);
        const uint32_t qv = encode8_fast(xa[t], mx_inv_scale(e));
        *(uint32_t *)(sac + r * (fa_cpr * 4) + c * 4) = qv;
        if ((c & 3) == 0) sas[r * (fa_cpr / 4) + (c >> 2)] = (uint8_t)(e + 127);
        if (blockIdx.x == 0 && p.aq_codes) {
          *(uint32_t *)(p.aq_codes + (int64_t)r * p.ld_aqc + c * 4) = qv;
          if ((c & 3) == 0) p.aq_scales[(int64_t)r * p.ld_aqs + (c >> 2)] = (uint8_t)(e + 127);
        }
      }
    }
    __syncthreads();
  }
  int64_t i = 0;
  for (; i + DEPTH < wpw; i += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      compute(ring[j], cur, j, i + j);
      __builtin_amdgcn_sched_barrier(0);
      if (j == 0) load_scales(nxt, i + DEPTH);
      load(ring[j], i + j + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
    }
    cur = nxt;
  }
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) compute(ring[j], cur, j, i + j);

  // Add the four quarters.  The tile's FM * FN * 16 accumulator registers (in (f, g, register)
  // order) are shared out 4 * FM * FN to a wave; registers r and r + 1 hold adjacent rows.
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_red[wave][f][g][r][lane] = acc[f][g][r];
  __syncthreads();
  constexpr int kPer = 4 * FM * FN;
#pragma unroll
  for (int j = 0; j < kPer; j += 2) {
    const int t = wave * kPer + j;
    const int f = t / (16 * FN), g = (t / 16) % FN, r = t % 16;
    float v0 = s_red[0][f][g][r][lane], v1 = s_red[0][f][g][r + 1][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      v0 += s_red[w][f][g][r][lane];
      v1 += s_red[w][f][g][r + 1][lane];
    }
    const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    const int64_t col = n0 + g * 32 + lr;
    const uint32_t pk = bf16x2_rne(v0, v1);
    if (row < p.m && col < p.n) ntstore_u16(p.y + row * p.ld_y + col, pk);
    if (row + 1 < p.m && col < p.n) ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
  }
}

// Any shape (K a multiple of 32): each wave computes one 32 x 32 tile straight from memory, one
// 64-wide K window at a time; a missing second block of the last window reads as zero codes.
__global__ __launch_bounds__(256) void k_gemm_mx_simple(MxArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, kh = lane >> 5;
  const int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  if (tile >= (int64_t)p.tiles_m * p.tiles_n) return;
  const int64_t m0 = (tile / p.tiles_n) * 32, n0 = (tile % p.tiles_n) * 32;
  const int64_t ra = min(m0 + lr, p.m - 1), rw = min(n0 + lr, p.n - 1);
  const uint8_t *ac = p.a_codes + ra * p.ld_ac + kh * 16, *as = p.a_scales + ra * p.ld_as + kh;
  const uint8_t *wc = p.w_codes + rw * p.ld_wc + kh * 16, *ws = p.w_scales + rw * p.ld_ws + kh;
  const int64_t nblk = p.k / 32;
  floatx16_t acc = floatx16_t{};
  for (int64_t b0 = 0; b0 < nblk; b0 += 2) {
    const bool in = b0 + kh < nblk;  // this lane's block exists
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const u32x4_t a = in ? *(const u32x4_t *)(ac + b0 * 16) : z;
    const u32x4_t w = in ? *(const u32x4_t *)(wc + b0 * 16) : z;
    const uint32_t sa = in ? as[b0] : 127u, sw = in ? ws[b0] : 127u;
    acc = mx_mfma(a, w, sa, sw, acc);
  }
  const int64_t col = n0 + lr;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t row = m0 + 8 * (i >> 2) + 4 * kh + (i & 3);
    if (row < p.m && col < p.n) ntstore_u16(p.y + row * p.ld_y + col, f32_to_bf16_rne(acc[i]));
  }
}

// ---------------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------------
static FastDiv mx_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1ull);
  return f;
}

static unsigned mx_grid(uint32_t n_chunks) {
  uint32_t g = (n_chunks + 255) / 256;
  if (g > 4096) g = 4096;
  return g < 1 ? 1 : g;
}

hipError_t launch_mx_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                              hipStream_t stream) {
  const uint32_t cpr = (uint32_t)(cols / 8), n = (uint32_t)(rows * (cols / 8));
  hipLaunchKernelGGL(k_mx_quantize, dim3(mx_grid(n)), dim3(256), 0, stream, (const uint16_t *)x,
                     ld_x, n, mx_fastdiv(cpr), codes, ld_codes, scales, ld_scales);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                                int64_t ld_scales, int64_t rows, int64_t cols, void *y,
                                int64_t ld_y, int out_f32, hipStream_t stream) {
  // The caller keeps rows * cols / 8 below 2^31, so rows * cols / 4 fits 32 bits.
  if (out_f32) {
    const uint32_t qpr = (uint32_t)(cols / 4), n = (uint32_t)(rows * (cols / 4));
    hipLaunchKernelGGL(k_mx_dequantize_f32, dim3(mx_grid(n)), dim3(256), 0, stream, codes,
                       ld_codes, scales, ld_scales, n, mx_fastdiv(qpr), (float *)y, ld_y);
  } else {
    const uint32_t cpr = (uint32_t)(cols / 8), n = (uint32_t)(rows * (cols / 8));
    hipLaunchKernelGGL(k_mx_dequantize_bf16, dim3(mx_grid(n)), dim3(256), 0, stream, codes,
                       ld_codes, scales, ld_scales, n, mx_fastdiv(cpr), (uint16_t *)y, ld_y);
  }
  return hipGetLastError();
}

// Launches k_gemm_mx_mid when K suits its ring, the scale rows are 8-byte aligned and the
// shape makes at least 128 tiles (FA: and A fits the fused form); returns whether it did.
template <int FM, int FN, int DEPTH, bool FA = false>
static bool launch_mx_mid(MxArgs &p, hipStream_t stream) {
  const int64_t tiles_m = (p.m + 32 * FM - 1) / (32 * FM), tiles_n = (p.n + 32 * FN - 1) / (32 * FN);
  if (p.k % (256 * DEPTH) != 0 || tiles_m * tiles_n < 128 || (uintptr_t)p.w_scales % 8 ||
      p.ld_ws % 8)
    return false;
  if (!FA && ((uintptr_t)p.a_scales % 8 || p.ld_as % 8)) return false;
  if (FA && (tiles_m != 1 || p.m * p.k > kMxFaMaxValues || (uintptr_t)p.a_bf16 % 16 ||
             p.ld_a % 8 || (p.aq_codes && ((uintptr_t)p.aq_codes % 4 || p.ld_aqc % 4))))
    return false;
  p.tiles_m = (int)tiles_m;
  p.tiles_n = (int)tiles_n;
  const size_t lds = FA ? (size_t)(p.m * (p.k / 2 + p.k / 32)) : 0;
  hipLaunchKernelGGL((k_gemm_mx_mid<FM, FN, DEPTH, FA>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(256), lds, stream, p);
  return true;
}

hipError_t launch_mx_gemm(const uint8_t *a_codes, int64_t ld_ac, const uint8_t *a_scales,
                          int64_t ld_as, const uint8_t *w_codes, int64_t ld_wc,
                          const uint8_t *w_scales, int64_t ld_ws, int64_t m, int64_t n, int64_t k,
                          uint16_t *y, int64_t ld_y, hipStream_t stream) {
  MxArgs p{a_codes, a_scales, w_codes, w_scales, ld_ac, ld_as, ld_wc, ld_ws, m, n, k, y, ld_y, 0, 0};
  // M <= 128: the mid-size kernel.  Deeper rings keep more of W in flight (16 windows, all of a
  // quarter of K = 4096 at once); each M range takes the deepest ring K allows, and 128-row
  // tiles fall back to 64-row ones where they would be too few.
  bool mid = false;
  if (m <= 4)
    mid = launch_mx_mid<1, 1, 16>(p, stream) || launch_mx_mid<1, 1, 8>(p, stream) ||
          launch_mx_mid<1, 1, 4>(p, stream);
  else if (m <= 32)
    mid = launch_mx_mid<1, 2, 16>(p, stream) || launch_mx_mid<1, 2, 8>(p, stream) ||
          launch_mx_mid<1, 2, 4>(p, stream);
  else if (m <= 64)
    mid = launch_mx_mid<2, 2, 8>(p, stream) || launch_mx_mid<2, 2, 4>(p, stream);
  else if (m <= 128)
    mid = launch_mx_mid<4, 2, 8>(p, stream) || launch_mx_mid<4, 2, 4>(p, stream) ||
          launch_mx_mid<2, 2, 4>(p, stream);
  if (mid) return hipGetLastError();
  const bool pipelined = m > 128 && k % 64 == 0 && (uintptr_t)a_scales % 2 == 0 &&
                         (uintptr_t)w_scales % 2 == 0 && ld_as % 2 == 0 && ld_ws % 2 == 0;
  if (pipelined) {
    p.tiles_m = (int)((m + 255) / 256);
    p.tiles_n = (int)((n + 255) / 256);
    const int64_t lim = (int64_t)1 << 31;
    const bool wide = k % 512 == 0 && (uintptr_t)a_scales % 16 == 0 &&
                      (uintptr_t)w_scales % 16 == 0 && ld_as % 16 == 0 && ld_ws % 16 == 0 &&
                      (int64_t)p.tiles_m * 256 * ld_ac < lim && (int64_t)p.tiles_n * 256 * ld_wc < lim &&
                      (int64_t)p.tiles_m * 256 * ld_as < lim && (int64_t)p.tiles_n * 256 * ld_ws < lim;
    if (wide) {
      hipLaunchKernelGGL(k_gemm_mx_wide, dim3((unsigned)p.tiles_m * (unsigned)p.tiles_n),
                         dim3(256), 0, stream, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(k_gemm_mx_lds, dim3((unsigned)p.tiles_m * (unsigned)p.tiles_n), dim3(256),
                       0, stream, p);
    return hipGetLastError();
  }
  p.tiles_m = (int)((m + 31) / 32);
  p.tiles_n = (int)((n + 31) / 32);
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL(k_gemm_mx_simple, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// One launch for small M with bf16 activations: the activation is quantized inside the
// mid-size kernel.  Sets *launched (and returns the launch status) only when the shape fits.
hipError_t launch_mx_gemm_fused(const void *a_bf16, int64_t ld_a, uint8_t *aq_codes,
                                int64_t ld_aqc, uint8_t *aq_scales, int64_t ld_aqs,
                                const uint8_t *w_codes, int64_t ld_wc, const uint8_t *w_scales,
                                int64_t ld_ws, int64_t m, int64_t n, int64_t k, uint16_t *y,
                                int64_t ld_y, hipStream_t stream, bool *launched) {
  *launched = false;
  if (m > 4) return hipSuccess;
  MxArgs p{nullptr, nullptr, w_codes, w_scales, 0, 0, ld_wc, ld_ws, m, n, k, y, ld_y, 0, 0,
           (const uint16_t *)a_bf16, ld_a, aq_codes, aq_scales, ld_aqc, ld_aqs};
  *launched = launch_mx_mid<1, 1, 16, true>(p, stream) || launch_mx_mid<1, 1, 8, true>(p, stream) ||
              launch_mx_mid<1, 1, 4, true>(p, stream);
  return *launched ? hipGetLastError() : hipSuccess;
}

}  // namespace nvfp4
