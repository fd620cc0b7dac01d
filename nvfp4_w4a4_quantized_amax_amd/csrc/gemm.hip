// W4A4 GEMM kernels for gfx950: Y = A . W^T with both operands in NVFP4, FP32 accumulation,
// bf16 output ("NVFP4 Dynamic Quantization in Practice: W4A4 Accelerated Deployment ...",
// section "The Meaning and Advantages of W4A4"; reconstruction from "NVFP4 Explained",
// section "How NVFP4 Represents a Value").
//
// CDNA4's scaled MFMA takes power-of-two E8M0 scales per 32 values, which cannot carry a
// fractional E4M3 scale per 16 values.  Here each packed E2M1 code is decoded to fp16 and
// multiplied by its block scale (both exact: code * scale has at most 6 significant bits and
// lies in [2^-10, 2688]), and the dense contraction runs on the fp16 MFMA with fp32
// accumulators.  Both global scales factor out of the sum and are applied once in the epilogue:
//   Y = RN_bf16(acc * RN_fp32(gsA * gsW)).
//
// The order of the K terms inside one MFMA is free (the dot product does not care), so each
// lane loads 16 contiguous bytes (32 codes, two scale blocks) of one row per 64-wide K window
// straight into registers and feeds them to four K=16 MFMAs; A and W use the same mapping.

#include <mutex>
#include <type_traits>

#include "nvfp4_device.hpp"
#include "gemm_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kGemmThreads = 256;  // 4 waves, 2 (M) x 2 (N)

// ---------------------------------------------------------------------------------------------
// Per-lane operand loads for one 64-wide K window
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint4 load16(const uint8_t *p) { return *(const uint4 *)p; }

// 16 code bytes at p (the lane's K-half offset already applied); `rem` = bytes of the row left
// from p, a multiple of 8.
__device__ __forceinline__ uint4 load16_masked(const uint8_t *p, int64_t rem) {
  if (rem >= 16) return *(const uint4 *)p;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (rem >= 8) {
    uint2 h = *(const uint2 *)p;
    v.x = h.x;
    v.y = h.y;
  }
  return v;
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int FM, int FN>
struct Frags {
  uint4 a[FM];
  uint4 w[FN];
  uint32_t sa[FM];  // two scale bytes (blocks 2*kh, 2*kh+1 of the window)
  uint32_t sw[FN];
};

template <int FM, int FN>
__device__ __forceinline__ void load_window(Frags<FM, FN> &fr, const uint8_t *const (&a_row)[FM],
                                            const uint8_t *const (&a_srow)[FM],
                                            const uint8_t *const (&w_row)[FN],
                                            const uint8_t *const (&w_srow)[FN], int64_t win) {
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    fr.a[f] = load16(a_row[f] + win * 32);
    fr.sa[f] = (uint32_t)a_srow[f][win * 4] | ((uint32_t)a_srow[f][win * 4 + 1] << 8);
  }
#pragma unroll
  for (int g = 0; g < FN; ++g) {
    fr.w[g] = load16(w_row[g] + win * 32);
    fr.sw[g] = (uint32_t)w_srow[g][win * 4] | ((uint32_t)w_srow[g][win * 4 + 1] << 8);
  }
}

// The last, partial window: codes past K read as zero, scales past K/16 are not read.
template <int FM, int FN>
__device__ __forceinline__ void load_window_masked(Frags<FM, FN> &fr,
                                                   const uint8_t *const (&a_row)[FM],
                                                   const uint8_t *const (&a_srow)[FM],
                                                   const uint8_t *const (&w_row)[FN],
                                                   const uint8_t *const (&w_srow)[FN],
                                                   int64_t win, int64_t rem_bytes,
                                                   int64_t rem_blocks) {
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    fr.a[f] = load16_masked(a_row[f] + win * 32, rem_bytes);
    uint32_t s0 = rem_blocks > 0 ? a_srow[f][win * 4] : 0u;
    uint32_t s1 = rem_blocks > 1 ? a_srow[f][win * 4 + 1] : 0u;
    fr.sa[f] = s0 | (s1 << 8);
  }
#pragma unroll
  for (int g = 0; g < FN; ++g) {
    fr.w[g] = load16_masked(w_row[g] + win * 32, rem_bytes);
    uint32_t s0 = rem_blocks > 0 ? w_srow[g][win * 4] : 0u;
    uint32_t s1 = rem_blocks > 1 ? w_srow[g][win * 4 + 1] : 0u;
    fr.sw[g] = s0 | (s1 << 8);
  }
}

template <int FM, int FN>
__device__ __forceinline__ void compute_window(const Frags<FM, FN> &fr,
                                               floatx16_t (&acc)[FM][FN]) {
  half2_t sa[FM], sw[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) sa[f] = scales_f16x2(fr.sa[f]);
#pragma unroll
  for (int g = 0; g < FN; ++g) sw[g] = scales_f16x2(fr.sw[g]);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    half8_t av[FM], bv[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
      av[f] = decode8_f16(word(fr.a[f], kk), kk < 2 ? splat_lo(sa[f]) : splat_hi(sa[f]));
#pragma unroll
    for (int g = 0; g < FN; ++g)
      bv[g] = decode8_f16(word(fr.w[g], kk), kk < 2 ? splat_lo(sw[g]) : splat_hi(sw[g]));
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int g = 0; g < FN; ++g)
        acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[f], bv[g], acc[f][g], 0, 0, 0);
  }
}

// Full K loop of one wave tile (32*FM rows of A by 32*FN rows of W).  Row pointers already
// include the lane's K-half offsets (16 code bytes, 2 scale bytes).
template <int FM, int FN>
__device__ __forceinline__ void wave_tile_kloop(const uint8_t *const (&a_row)[FM],
                                                const uint8_t *const (&a_srow)[FM],
                                                const uint8_t *const (&w_row)[FN],
                                                const uint8_t *const (&w_srow)[FN], int64_t k,
                                                int kh, floatx16_t (&acc)[FM][FN]) {
  const int64_t nwin = k / 64;
  Frags<FM, FN> b0, b1;
  if (nwin > 0) load_window(b0, a_row, a_srow, w_row, w_srow, 0);
  int64_t w = 0;
  for (; w + 2 <= nwin; w += 2) {
    load_window(b1, a_row, a_srow, w_row, w_srow, w + 1);
    compute_window(b0, acc);
    if (w + 2 < nwin) load_window(b0, a_row, a_srow, w_row, w_srow, w + 2);
    compute_window(b1, acc);
  }
  if (w < nwin) compute_window(b0, acc);
  if (k % 64) {
    const int64_t rem_bytes = k / 2 - nwin * 32 - kh * 16;
    const int64_t rem_blocks = k / 16 - nwin * 4 - kh * 2;
    load_window_masked(b1, a_row, a_srow, w_row, w_srow, nwin, rem_bytes, rem_blocks);
    compute_window(b1, acc);
  }
}

// ---------------------------------------------------------------------------------------------
// Dense tile kernel
// ---------------------------------------------------------------------------------------------
struct DenseArgs {
  GemmOperand a, w;
  int64_t m, n, k;
  uint16_t *y;
  int64_t ld_y;
  int tiles_m, tiles_n;
  // Split K (shapes with too few tiles to fill the device): workgroup (tile, blockIdx.y) covers
  // 64-wide K windows [blockIdx.y * wps, (blockIdx.y + 1) * wps) and stores its unscaled fp32
  // sums to part + blockIdx.y * m * n (row-major, m x n); k_splitk_reduce finishes Y.  part is
  // NULL when K is not split.
  float *part;
  int64_t wps;
};

// fp32 partial sums of one wave tile (before the global scales) into this split's slab.
template <int FM, int FN, class InRange>
__device__ __forceinline__ void store_partial(const DenseArgs &p, const floatx16_t (&acc)[FM][FN],
                                              int64_t m0, int64_t n0, int lr, int kh,
                                              InRange in_range) {
  float *dst = p.part + (int64_t)blockIdx.y * p.m * p.n;
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (in_range(row, col)) dst[row * p.n + col] = acc[f][g][r];
      }
    }
}


template <int FM, int FN, bool W2D>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_tile(DenseArgs p) {
  constexpr int BM = 64 * FM, BN = 64 * FN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;

  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const float alpha = load_global_scale(p.a.gs) * load_global_scale(p.w.gs);
  const int in_group = kGroupM * p.tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsz = min(p.tiles_m - first_m, kGroupM);
  const int tm = first_m + (logical % in_group) % gsz;
  const int tn = (logical % in_group) / gsz;
  const int64_t m0 = (int64_t)tm * BM + wm * 32 * FM;
  const int64_t n0 = (int64_t)tn * BN + wn * 32 * FN;

  const uint8_t *a_row[FM], *a_srow[FM], *w_row[FN], *w_srow[FN];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t r = min(m0 + f * 32 + lr, p.m - 1);
    a_row[f] = p.a.codes + r * p.a.ld_codes + kh * 16;
    a_srow[f] = p.a.scales + r * p.a.ld_scales + kh * 2;
  }
#pragma unroll
  for (int g = 0; g < FN; ++g) {
    const int64_t r = min(n0 + g * 32 + lr, p.n - 1);
    w_row[g] = p.w.codes + r * p.w.ld_codes + kh * 16;
    w_srow[g] = p.w.scales + (W2D ? (r >> 4) : r) * p.w.ld_scales + kh * 2;
  }
  int64_t kk = p.k;
  if (p.part) {  // this split's K windows: move the row pointers to its first one
    const int64_t w0 = (int64_t)blockIdx.y * p.wps;
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      a_row[f] += w0 * 32;
      a_srow[f] += w0 * 4;
    }
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      w_row[g] += w0 * 32;
      w_srow[g] += w0 * 4;
    }
    kk = min(p.k - w0 * 64, p.wps * 64);
  }
  floatx16_t acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) acc[f][g] = floatx16_t{};

  wave_tile_kloop<FM, FN>(a_row, a_srow, w_row, w_srow, kk, kh, acc);

  if (p.part) {
    store_partial<FM, FN>(p, acc, m0, n0, lr, kh,
                          [&](int64_t row, int64_t col) { return row < p.m && col < p.n; });
    return;
  }
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {  // rows r and r + 1 are adjacent
        const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const uint32_t pk = bf16x2_rne(acc[f][g][r] * alpha, acc[f][g][r + 1] * alpha);
        if (row < p.m && col < p.n) ntstore_u16(p.y + row * p.ld_y + col, pk);
        if (row + 1 < p.m && col < p.n) ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Pipelined tile kernel (256 x 256 tiles, K a multiple of 64).  Packed codes and scales of each
// 64-wide K window are loaded from HBM into registers two windows ahead, written to one of two
// LDS stages one window ahead, and read back by the waves that use them (each 32-row fragment
// of A or W is used by two of the four waves).  All LDS traffic is ordinary loads and stores,
// so the compiler places the waits for it where the data is first used.
// Per stage: A and W codes [row][32 bytes], A scales [row][4 bytes], W scales [row][4 bytes]
// (1D) or one copy per wave of the 16 band rows (2D).  The two 16-byte halves of a code row
// are swapped on rows where bit 2 xor bit 3 of the row is set: a fragment read (one half of 8
// or 16 consecutive rows per LDS cycle) then covers every bank once, and a store of 16
// consecutive chunks still fills 256 contiguous bytes.
// ---------------------------------------------------------------------------------------------
struct LdsStage {
  uint8_t a[256 * 32];
  uint8_t w[256 * 32];
  uint8_t as[256 * 4];
  uint8_t ws[256 * 4];
};

// One thread's share of a window: chunk c = i * 256 + tid of A and of W (row c / 2, 16-byte
// half c % 2), and the 4 scale bytes of A row tid and of W row tid (1D) or band tid % 16 (2D).
struct WindowRegs {
  u32x4_t a0, a1, w0, w1;
  uint32_t as, ws;
};

__device__ __forceinline__ void load_window_regs(WindowRegs &r, const uint8_t *const (&ga)[2],
                                                 const uint8_t *const (&gw)[2],
                                                 const uint8_t *gas, const uint8_t *gws,
                                                 int64_t win) {
  r.a0 = *(const u32x4_t *)(ga[0] + win * 32);
  r.a1 = *(const u32x4_t *)(ga[1] + win * 32);
  r.w0 = *(const u32x4_t *)(gw[0] + win * 32);
  r.w1 = *(const u32x4_t *)(gw[1] + win * 32);
  r.as = *(const uint32_t *)(gas + win * 4);
  r.ws = *(const uint32_t *)(gws + win * 4);
}


__device__ __forceinline__ void store_window_regs(const WindowRegs &r, LdsStage &S, int tid) {
  // chunk c = i * 256 + tid is half c % 2 of row c / 2
  const int o0 = code_offset(tid >> 1, tid & 1), o1 = code_offset(128 + (tid >> 1), tid & 1);
  *(u32x4_t *)(S.a + o0) = r.a0;
  *(u32x4_t *)(S.a + o1) = r.a1;
  *(u32x4_t *)(S.w + o0) = r.w0;
  *(u32x4_t *)(S.w + o1) = r.w1;
  *(uint32_t *)(S.as + tid * 4) = r.as;
  *(uint32_t *)(S.ws + tid * 4) = r.ws;
}


template <bool W2D, class Stage>
__device__ __forceinline__ void read_stage_frags(const Stage &S, int wave, int wm, int wn,
                                                 int lr, int kh, Frags<4, 4> &fr) {
  const int ra = wm * 128 + lr, rw = wn * 128 + lr;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    fr.a[f] = *(const uint4 *)(S.a + code_offset(ra + f * 32, kh));
    fr.sa[f] = *(const uint16_t *)(S.as + (ra + f * 32) * 4 + kh * 2);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    fr.w[g] = *(const uint4 *)(S.w + code_offset(rw + g * 32, kh));
    fr.sw[g] = W2D ? *(const uint16_t *)(S.ws + wave * 256 + (wn * 8 + g * 2 + (lr >> 4)) * 4 +
                                         kh * 2)
                   : *(const uint16_t *)(S.ws + (rw + g * 32) * 4 + kh * 2);
  }
}

// read_stage_frags for the first NF A fragments only (the tile's rows past them are padding).
template <bool W2D, int NF, class Stage>
__device__ __forceinline__ void read_stage_frags_nf(const Stage &S, int wave, int wn, int lr,
                                                    int kh, Frags<4, 4> &fr) {
  const int ra = lr, rw = wn * 128 + lr;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    fr.a[f] = *(const uint4 *)(S.a + code_offset(ra + f * 32, kh));
    fr.sa[f] = *(const uint16_t *)(S.as + (ra + f * 32) * 4 + kh * 2);
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    fr.w[g] = *(const uint4 *)(S.w + code_offset(rw + g * 32, kh));
    fr.sw[g] = W2D ? *(const uint16_t *)(S.ws + wave * 256 + (wn * 8 + g * 2 + (lr >> 4)) * 4 +
                                         kh * 2)
                   : *(const uint16_t *)(S.ws + (rw + g * 32) * 4 + kh * 2);
  }
}

// Decoded operands of one K=16 step: 4 A fragments then 4 W fragments (8 fp16 each).
struct StepOps {
  half8_t v[8];
};

__device__ __forceinline__ void window_scales(const Frags<4, 4> &fr, half2_t (&sa)[4],
                                              half2_t (&sw)[4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) sa[f] = scales_f16x2(fr.sa[f]);
#pragma unroll
  for (int g = 0; g < 4; ++g) sw[g] = scales_f16x2(fr.sw[g]);
}

// Step kk (0..3) uses code word kk of every fragment; words 0-1 belong to the lane's first
// scale block, words 2-3 to its second.
__device__ __forceinline__ void decode_step(const Frags<4, 4> &fr, const half2_t (&sa)[4],
                                            const half2_t (&sw)[4], int kk, StepOps &d) {
#pragma unroll
  for (int f = 0; f < 4; ++f)
    d.v[f] = decode8_f16(word(fr.a[f], kk), kk < 2 ? splat_lo(sa[f]) : splat_hi(sa[f]));
#pragma unroll
  for (int g = 0; g < 4; ++g)
    d.v[4 + g] = decode8_f16(word(fr.w[g], kk), kk < 2 ? splat_lo(sw[g]) : splat_hi(sw[g]));
}

__device__ __forceinline__ void mfma_step(const StepOps &d, floatx16_t (&acc)[4][4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d.v[f], d.v[4 + g], acc[f][g], 0, 0, 0);
}

// Ask the scheduler to alternate one MFMA with four VALU instructions (the decode of the next
// step), so that the conversions run while the matrix core works.
__device__ __forceinline__ void interleave_step() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
}

// Step with memory work: each of the first `nmem` MFMAs is followed by one instruction of the
// memory kind `mem_mask` (0x020 vector-memory read, 0x100 LDS read, 0x200 LDS write) besides
// its four VALU instructions, so that a burst of memory instructions never blocks the wave.
template <int MEM_MASK, int NMEM, int MEM_MASK2 = 0, int NMEM2 = 0>
__device__ __forceinline__ void interleave_step_mem() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NMEM) __builtin_amdgcn_sched_group_barrier(MEM_MASK, 1, 0);
    if (i < NMEM2) __builtin_amdgcn_sched_group_barrier(MEM_MASK2, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
}

// Ends a step: nothing moves across this point, and the step's operands stay live until here.
// Without this the register allocator hands an MFMA's source registers to the next step's
// decode as soon as the last MFMA reading them has issued; the VALU write then waits for the
// MFMA, and decode and matrix work no longer overlap.
__device__ __forceinline__ void end_step(const StepOps &d) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(d.v[i]));
}

// The same steps for a tile whose first NF 32-row A fragments hold rows (NF < 4: the last
// tile of a group); the fragments past them are neither read, decoded nor multiplied.  A step
// then has 4 NF MFMAs and (NF + 4) decodes of 8 VALU operations each.
template <int NF>
__device__ __forceinline__ void decode_step_nf(const Frags<4, 4> &fr, const half2_t (&sa)[4],
                                               const half2_t (&sw)[4], int kk, StepOps &d) {
#pragma unroll
  for (int f = 0; f < NF; ++f)
    d.v[f] = decode8_f16(word(fr.a[f], kk), kk < 2 ? splat_lo(sa[f]) : splat_hi(sa[f]));
#pragma unroll
  for (int g = 0; g < 4; ++g)
    d.v[4 + g] = decode8_f16(word(fr.w[g], kk), kk < 2 ? splat_lo(sw[g]) : splat_hi(sw[g]));
}

template <int NF>
__device__ __forceinline__ void mfma_step_nf(const StepOps &d, floatx16_t (&acc)[NF][4]) {
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(d.v[f], d.v[4 + g], acc[f][g], 0, 0, 0);
}

template <int NF>
__device__ __forceinline__ void window_scales_nf(const Frags<4, 4> &fr, half2_t (&sa)[4],
                                                 half2_t (&sw)[4]) {
#pragma unroll
  for (int f = 0; f < NF; ++f) sa[f] = scales_f16x2(fr.sa[f]);
#pragma unroll
  for (int g = 0; g < 4; ++g) sw[g] = scales_f16x2(fr.sw[g]);
}

// Interleave for 4 NF MFMAs: after each, its share of the next step's decode VALU and of up
// to two kinds of memory instructions: one per MFMA from the first while they are no more than
// the MFMAs (the full tile's pattern), else spread evenly.
template <int NF, int MEM_MASK = 0, int NMEM = 0, int MEM_MASK2 = 0, int NMEM2 = 0>
__device__ __forceinline__ void interleave_step_nf() {
  constexpr int kSlots = 4 * NF;
  constexpr int kValu = ((NF + 4) * 8 + kSlots - 1) / kSlots;
  constexpr int kPer1 = (NMEM + kSlots - 1) / kSlots, kPer2 = (NMEM2 + kSlots - 1) / kSlots;
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int j = 0; j < kPer1; ++j)
      if (NMEM <= kSlots ? i < NMEM : j < (i + 1) * NMEM / kSlots - i * NMEM / kSlots)
        __builtin_amdgcn_sched_group_barrier(MEM_MASK, 1, 0);
#pragma unroll
    for (int j = 0; j < kPer2; ++j)
      if (NMEM2 <= kSlots ? i < NMEM2 : j < (i + 1) * NMEM2 / kSlots - i * NMEM2 / kSlots)
        __builtin_amdgcn_sched_group_barrier(MEM_MASK2, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
  }
}

template <int NF>
__device__ __forceinline__ void end_step_nf(const StepOps &d) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NF; ++i) asm volatile("" ::"v"(d.v[i]));
#pragma unroll
  for (int i = 4; i < 8; ++i) asm volatile("" ::"v"(d.v[i]));
}

template <bool W2D>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_lds(DenseArgs p) {
  __shared__ __align__(16) LdsStage st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;

  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int in_group = kGroupM * p.tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsz = min(p.tiles_m - first_m, kGroupM);
  const int tm = first_m + (logical % in_group) % gsz;
  const int tn = (logical % in_group) / gsz;
  const int64_t m_tile = (int64_t)tm * 256, n_tile = (int64_t)tn * 256;

  // This thread's share of every window's loads (rows clamped into the matrix; results of
  // clamped rows are never stored).
  // With K split, this workgroup's windows start at w0 (the row pointers move there).
  const int64_t w0 = p.part ? (int64_t)blockIdx.y * p.wps : 0;
  const uint8_t *ga[2], *gw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = i * 256 + tid, row = c >> 1, half = c & 1;
    ga[i] = p.a.codes + min(m_tile + row, p.m - 1) * p.a.ld_codes + half * 16 + w0 * 32;
    gw[i] = p.w.codes + min(n_tile + row, p.n - 1) * p.w.ld_codes + half * 16 + w0 * 32;
  }
  const uint8_t *gas = p.a.scales + min(m_tile + tid, p.m - 1) * p.a.ld_scales + w0 * 4;
  const uint8_t *gws = (W2D ? p.w.scales + min(n_tile / 16 + (lane & 15), p.n / 16 - 1) * p.w.ld_scales
                            : p.w.scales + min(n_tile + tid, p.n - 1) * p.w.ld_scales) + w0 * 4;
  const int64_t nwin = p.part ? min(p.wps, p.k / 64 - w0) : p.k / 64;  // >= 1
  // Window `win` is clamped to the last one so that the loop has no branch (a clamped load is
  // never stored).
  floatx16_t acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = floatx16_t{};

  // Window 0 goes to stage 0 and window 1 stays in registers.  At the start of window w,
  // window w + 1 is stored to stage (w + 1) % 2 (every wave finished reading it before the
  // previous barrier) and window w + 2 is loaded; after the barrier in the middle of window w,
  // window w + 1 is read back.
  WindowRegs r;
  load_window_regs(r, ga, gw, gas, gws, 0);
  store_window_regs(r, st[0], tid);
  load_window_regs(r, ga, gw, gas, gws, min((int64_t)1, nwin - 1));
  lds_barrier();
  Frags<4, 4> cur, nxt;
  read_stage_frags<W2D>(st[0], wave, wm, wn, lr, kh, cur);
  half2_t sa[4], sw[4];
  window_scales(cur, sa, sw);
  StepOps ev, od;
  decode_step(cur, sa, sw, 0, ev);

  for (int64_t w = 0; w + 1 < nwin; ++w) {
    store_window_regs(r, st[(w + 1) & 1], tid);
    load_window_regs(r, ga, gw, gas, gws, min(w + 2, nwin - 1));
    decode_step(cur, sa, sw, 1, od);
    mfma_step(ev, acc);
    interleave_step_mem<0x200, 6, 0x020, 6>();
    end_step(ev);
    lds_barrier();
    read_stage_frags<W2D>(st[(w + 1) & 1], wave, wm, wn, lr, kh, nxt);
    decode_step(cur, sa, sw, 2, ev);
    mfma_step(od, acc);
    interleave_step_mem<0x100, 16>();
    end_step(od);
    decode_step(cur, sa, sw, 3, od);
    mfma_step(ev, acc);
    interleave_step();
    end_step(ev);
    window_scales(nxt, sa, sw);
    decode_step(nxt, sa, sw, 0, ev);
    mfma_step(od, acc);
    interleave_step();
    end_step(od);
    cur = nxt;
  }
  decode_step(cur, sa, sw, 1, od);
  mfma_step(ev, acc);
  interleave_step();
  end_step(ev);
  decode_step(cur, sa, sw, 2, ev);
  mfma_step(od, acc);
  interleave_step();
  end_step(od);
  decode_step(cur, sa, sw, 3, od);
  mfma_step(ev, acc);
  interleave_step();
  end_step(ev);
  mfma_step(od, acc);

  const int64_t m0 = m_tile + wm * 128, n0 = n_tile + wn * 128;
  if (p.part) {
    store_partial<4, 4>(p, acc, m0, n0, lr, kh,
                        [&](int64_t row, int64_t col) { return row < p.m && col < p.n; });
    return;
  }
  const float alpha = (*p.a.gs) * (*p.w.gs);
  const bool full = m_tile + 256 <= p.m && n_tile + 256 <= p.n;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {  // rows r and r + 1 are adjacent
        const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const uint32_t pk = bf16x2_rne(acc[f][g][r] * alpha, acc[f][g][r + 1] * alpha);
        if (full || (row < p.m && col < p.n)) ntstore_u16(p.y + row * p.ld_y + col, pk);
        if (full || (row + 1 < p.m && col < p.n))
          ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Grouped (mixture-of-experts) kernel: a persistent grid walks all (expert, m-tile, n-tile)
// tiles; the tile list is derived on the device from the expert offsets.
// ---------------------------------------------------------------------------------------------
constexpr int kMaxGroups = 1024;

struct GroupedArgs {
  GemmOperand a, w;
  const int32_t *row_index;
  const int32_t *offsets;
  int32_t num_groups;
  int64_t w_group_rows;  // W rows per expert (= n)
  int64_t n, k, total_rows;
  uint16_t *y;
  int64_t ld_y;
  int tiles_n;
};

template <int FM, int FN, bool W2D>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_grouped(GroupedArgs p) {
  constexpr int BM = 64 * FM, BN = 64 * FN;
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_start[kMaxGroups + 1];  // first tile id of each group
  __shared__ int s_part[kGemmThreads];
  const int E = p.num_groups;
  // Offsets, clamped into [0, total_rows] and made non-decreasing against bad input.
  for (int e = threadIdx.x; e <= E; e += kGemmThreads) {
    int v = p.offsets[e];
    s_off[e] = min(max(v, 0), (int)p.total_rows);
  }
  __syncthreads();
  // Per-thread slice of groups -> partial tile counts -> block exclusive scan.
  constexpr int kPer = (kMaxGroups + kGemmThreads - 1) / kGemmThreads;
  int local[kPer];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = threadIdx.x * kPer + j;
    int t = 0;
    if (e < E) {
      const int cnt = max(s_off[e + 1] - s_off[e], 0);
      t = ((cnt + BM - 1) / BM) * p.tiles_n;
    }
    local[j] = t;
    sum += t;
  }
  s_part[threadIdx.x] = sum;
  __syncthreads();
  for (int o = 1; o < kGemmThreads; o <<= 1) {
    int v = threadIdx.x >= o ? s_part[threadIdx.x - o] : 0;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = s_part[threadIdx.x] - sum;  // exclusive prefix
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = threadIdx.x * kPer + j;
    if (e < E) s_start[e] = run;
    run += local[j];
  }
  if (threadIdx.x == kGemmThreads - 1) s_start[E] = s_part[kGemmThreads - 1];
  __syncthreads();
  const int total_tiles = s_start[E];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;

  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    // Expert of tile t: last e with s_start[e] <= t (binary search over E + 1 entries).
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s_start[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int local_t = t - s_start[e];
    const int r_begin = s_off[e], r_end = s_off[e + 1];
    const int mt = (r_end - r_begin + BM - 1) / BM;
    const int tm = local_t % mt, tn = local_t / mt;
    const int64_t m0 = (int64_t)r_begin + (int64_t)tm * BM + wm * 32 * FM;
    const int64_t n0 = (int64_t)tn * BN + wn * 32 * FN;
    const int64_t wbase = (int64_t)e * p.w_group_rows;

    const uint8_t *a_row[FM], *a_srow[FM], *w_row[FN], *w_srow[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int64_t gr = min(m0 + f * 32 + lr, (int64_t)r_end - 1);
      const int64_t r = p.row_index ? (int64_t)p.row_index[gr] : gr;
      a_row[f] = p.a.codes + r * p.a.ld_codes + kh * 16;
      a_srow[f] = p.a.scales + r * p.a.ld_scales + kh * 2;
    }
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      const int64_t r = wbase + min(n0 + g * 32 + lr, p.n - 1);
      w_row[g] = p.w.codes + r * p.w.ld_codes + kh * 16;
      w_srow[g] = p.w.scales + (W2D ? (r >> 4) : r) * p.w.ld_scales + kh * 2;
    }
    floatx16_t acc[FM][FN];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int g = 0; g < FN; ++g) acc[f][g] = floatx16_t{};

    wave_tile_kloop<FM, FN>(a_row, a_srow, w_row, w_srow, p.k, kh, acc);

    const float alpha = (*p.a.gs) * p.w.gs[e];
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int g = 0; g < FN; ++g) {
        const int64_t col = n0 + g * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {  // rows r and r + 1 are adjacent
          const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
          const uint32_t pk = bf16x2_rne(acc[f][g][r] * alpha, acc[f][g][r + 1] * alpha);
          if (row < r_end && col < p.n) ntstore_u16(p.y + row * p.ld_y + col, pk);
          if (row + 1 < r_end && col < p.n) ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
        }
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Grouped kernel with the pipelined K loop (K a multiple of 64, 4-byte aligned scale rows):
// 128 x 256 tiles (tile rows waste less on the small experts than 256), two waves of 128 x 128
// per workgroup, two workgroups per CU.  The K loop is the dense kernel's: windows staged
// through two LDS stages, decode interleaved with the MFMAs.  A rows are gathered through
// row_index while they are loaded.
// ---------------------------------------------------------------------------------------------
struct LdsStageG {
  uint8_t a[128 * 32];
  uint8_t w[256 * 32];
  uint8_t as[128 * 4];
  uint8_t ws[256 * 4];  // 1D: one row per W row; 2D: each wave's copy of the 16 band rows
};

// One thread's share of a window (128 threads): A chunks c = i * 128 + tid (i < 2) and W chunks
// c = i * 128 + tid (i < 4), chunk c being half c % 2 of row c / 2; the scale bytes of A row tid
// and of W rows tid and 128 + tid (1D) or band tid % 16 (2D, ws1 unused).
struct WindowRegsG {
  u32x4_t a0, a1, w0, w1, w2, w3;
  uint32_t as, ws0, ws1;
};

// One tile of the grouped kernel whose first NF 32-row A fragments hold rows of the group
// (NF < 4 only for a group's last tile): the fragments past them would be padding and are
// neither read from LDS, decoded nor multiplied.  (A separate function rather than a lambda in
// the kernel: inside a generic lambda the scheduler bunched the LDS reads that the interleave
// hints spread over the MFMAs.)
template <bool W2D, int NF, class Load, class Store>
__device__ __forceinline__ void grouped_lds_tile(const GroupedArgs &p, LdsStageG (&st)[2],
                                                 const Load &load, const Store &store, int wave,
                                                 int wn, int lr, int kh, int64_t nwin, int e,
                                                 int64_t m_tile, int64_t n_tile, int r_end) {
    floatx16_t acc[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = floatx16_t{};

    __syncthreads();  // the previous tile's last fragment reads are done with both stages
    WindowRegsG r;
    load(0, r);
    store(r, st[0]);
    load(min((int64_t)1, nwin - 1), r);
    lds_barrier();
    Frags<4, 4> cur, nxt;
    read_stage_frags_nf<W2D, NF>(st[0], wave, wn, lr, kh, cur);
    half2_t sa[4], sw[4];
    window_scales_nf<NF>(cur, sa, sw);
    StepOps ev, od;
    decode_step_nf<NF>(cur, sa, sw, 0, ev);
    for (int64_t w = 0; w + 1 < nwin; ++w) {
      store(r, st[(w + 1) & 1]);
      load(min(w + 2, nwin - 1), r);
      decode_step_nf<NF>(cur, sa, sw, 1, od);
      mfma_step_nf<NF>(ev, acc);
      interleave_step_nf<NF, 0x200, 9, 0x020, 9>();
      end_step_nf<NF>(ev);
      lds_barrier();
      read_stage_frags_nf<W2D, NF>(st[(w + 1) & 1], wave, wn, lr, kh, nxt);
      decode_step_nf<NF>(cur, sa, sw, 2, ev);
      mfma_step_nf<NF>(od, acc);
      interleave_step_nf<NF, 0x100, 2 * NF + 8>();
      end_step_nf<NF>(od);
      decode_step_nf<NF>(cur, sa, sw, 3, od);
      mfma_step_nf<NF>(ev, acc);
      interleave_step_nf<NF>();
      end_step_nf<NF>(ev);
      window_scales_nf<NF>(nxt, sa, sw);
      decode_step_nf<NF>(nxt, sa, sw, 0, ev);
      mfma_step_nf<NF>(od, acc);
      interleave_step_nf<NF>();
      end_step_nf<NF>(od);
      cur = nxt;
    }
    decode_step_nf<NF>(cur, sa, sw, 1, od);
    mfma_step_nf<NF>(ev, acc);
    interleave_step_nf<NF>();
    end_step_nf<NF>(ev);
    decode_step_nf<NF>(cur, sa, sw, 2, ev);
    mfma_step_nf<NF>(od, acc);
    interleave_step_nf<NF>();
    end_step_nf<NF>(od);
    decode_step_nf<NF>(cur, sa, sw, 3, od);
    mfma_step_nf<NF>(ev, acc);
    interleave_step_nf<NF>();
    end_step_nf<NF>(ev);
    mfma_step_nf<NF>(od, acc);

    const float alpha = (*p.a.gs) * p.w.gs[e];
    const int64_t n0 = n_tile + wn * 128;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = n0 + g * 32 + lr;
#pragma unroll
        for (int r2 = 0; r2 < 16; r2 += 2) {  // rows r2 and r2 + 1 are adjacent
          const int64_t row = m_tile + f * 32 + 8 * (r2 >> 2) + 4 * kh + (r2 & 3);
          const uint32_t pk = bf16x2_rne(acc[f][g][r2] * alpha, acc[f][g][r2 + 1] * alpha);
          if (row < r_end && col < p.n) ntstore_u16(p.y + row * p.ld_y + col, pk);
          if (row + 1 < r_end && col < p.n)
            ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
        }
      }
}

template <bool W2D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_grouped_lds(GroupedArgs p) {
  constexpr int BM = 128, BN = 256, NT = 128;
  __shared__ __align__(16) LdsStageG st[2];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_start[kMaxGroups + 1];  // first tile id of each group
  __shared__ int s_part[NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave;
  const int lr = lane & 31, kh = lane >> 5;
  const int E = p.num_groups;
  // Tile list: offsets clamped into [0, total_rows] against bad input, per-group tile counts,
  // exclusive scan.
  for (int e = tid; e <= E; e += NT) s_off[e] = min(max(p.offsets[e], 0), (int)p.total_rows);
  __syncthreads();
  constexpr int kPer = (kMaxGroups + NT - 1) / NT;
  int local[kPer];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid * kPer + j;
    int t = 0;
    if (e < E) t = ((max(s_off[e + 1] - s_off[e], 0) + BM - 1) / BM) * p.tiles_n;
    local[j] = t;
    sum += t;
  }
  s_part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < NT; o <<= 1) {
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int run = s_part[tid] - sum;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid * kPer + j;
    if (e < E) s_start[e] = run;
    run += local[j];
  }
  if (tid == NT - 1) s_start[E] = s_part[NT - 1];
  __syncthreads();
  const int total_tiles = s_start[E];
  const int64_t nwin = p.k / 64;  // >= 1

  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    int lo = 0, hi = E;  // last group with s_start[e] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_start[mid] <= t) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int local_t = t - s_start[e];
    const int r_begin = s_off[e], r_end = s_off[e + 1];
    const int mt = (r_end - r_begin + BM - 1) / BM;
    const int tm = local_t % mt, tn = local_t / mt;
    const int64_t m_tile = (int64_t)r_begin + (int64_t)tm * BM, n_tile = (int64_t)tn * BN;
    const int64_t wbase = (int64_t)e * p.w_group_rows;

    // Source rows of this thread's loads (A gathered through row_index; rows clamped into the
    // group / expert, results of clamped rows are never stored).
    auto a_src = [&](int64_t r) __attribute__((always_inline)) {
      const int64_t gr = min(m_tile + r, (int64_t)r_end - 1);
      return p.row_index ? (int64_t)p.row_index[gr] : gr;
    };
    const uint8_t *ga[2], *gw[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = i * NT + tid;
      ga[i] = p.a.codes + a_src(c >> 1) * p.a.ld_codes + (c & 1) * 16;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = i * NT + tid;
      gw[i] = p.w.codes + (wbase + min(n_tile + (c >> 1), p.n - 1)) * p.w.ld_codes + (c & 1) * 16;
    }
    const uint8_t *gas = p.a.scales + a_src(tid) * p.a.ld_scales;
    const uint8_t *gws0, *gws1;
    if (W2D) {
      gws0 = p.w.scales +
             ((wbase + n_tile) / 16 + min((int64_t)(lane & 15), (p.n - n_tile) / 16 - 1)) * p.w.ld_scales;
      gws1 = gws0;
    } else {
      gws0 = p.w.scales + (wbase + min(n_tile + tid, p.n - 1)) * p.w.ld_scales;
      gws1 = p.w.scales + (wbase + min(n_tile + NT + tid, p.n - 1)) * p.w.ld_scales;
    }
    auto load = [&](int64_t win, WindowRegsG &r) __attribute__((always_inline)) {
      r.a0 = *(const u32x4_t *)(ga[0] + win * 32);
      r.a1 = *(const u32x4_t *)(ga[1] + win * 32);
      r.w0 = *(const u32x4_t *)(gw[0] + win * 32);
      r.w1 = *(const u32x4_t *)(gw[1] + win * 32);
      r.w2 = *(const u32x4_t *)(gw[2] + win * 32);
      r.w3 = *(const u32x4_t *)(gw[3] + win * 32);
      r.as = *(const uint32_t *)(gas + win * 4);
      r.ws0 = *(const uint32_t *)(gws0 + win * 4);
      r.ws1 = W2D ? 0u : *(const uint32_t *)(gws1 + win * 4);
    };
    auto store = [&](const WindowRegsG &r, LdsStageG &S) __attribute__((always_inline)) {
      *(u32x4_t *)(S.a + code_offset(tid >> 1, tid & 1)) = r.a0;
      *(u32x4_t *)(S.a + code_offset(64 + (tid >> 1), tid & 1)) = r.a1;
      *(u32x4_t *)(S.w + code_offset(tid >> 1, tid & 1)) = r.w0;
      *(u32x4_t *)(S.w + code_offset(64 + (tid >> 1), tid & 1)) = r.w1;
      *(u32x4_t *)(S.w + code_offset(128 + (tid >> 1), tid & 1)) = r.w2;
      *(u32x4_t *)(S.w + code_offset(192 + (tid >> 1), tid & 1)) = r.w3;
      *(uint32_t *)(S.as + tid * 4) = r.as;
      *(uint32_t *)(S.ws + tid * 4) = r.ws0;  // 2D: wave * 256 + lane * 4
      if (!W2D) *(uint32_t *)(S.ws + (NT + tid) * 4) = r.ws1;
    };

    const int nf = (int)((min((int64_t)BM, (int64_t)r_end - m_tile) + 31) / 32);  // 1..4
    if (nf >= 4)
      grouped_lds_tile<W2D, 4>(p, st, load, store, wave, wn, lr, kh, nwin, e, m_tile, n_tile, r_end);
    else if (nf == 3)
      grouped_lds_tile<W2D, 3>(p, st, load, store, wave, wn, lr, kh, nwin, e, m_tile, n_tile, r_end);
    else if (nf == 2)
      grouped_lds_tile<W2D, 2>(p, st, load, store, wave, wn, lr, kh, nwin, e, m_tile, n_tile, r_end);
    else
      grouped_lds_tile<W2D, 1>(p, st, load, store, wave, wn, lr, kh, nwin, e, m_tile, n_tile, r_end);
  }
}

// ---------------------------------------------------------------------------------------------
// Small-M kernel (m <= 16, decode-shaped): streams W at full width.  A workgroup owns 16 rows of
// W; its 4 waves split K and reduce through LDS.  The MFMA is 16x16x32 with W rows as the M side
// and the (zero-padded) 16 activation rows as the N side.  Both operands arrive packed and are
// decoded in registers with the same K permutation: lane (row r = lane % 16, group q = lane / 16)
// loads 16 code bytes at byte 64 * window + 16 * q of its row, i.e. K values
// 128 * window + 32 * q + [0, 32), which feed four K=32 MFMAs (8 values each).
// Loads of four windows are issued before any of them is used.
// ---------------------------------------------------------------------------------------------
struct SmallMArgs {
  GemmOperand a, w;
  int64_t m, n, k;
  uint16_t *y;
  int64_t ld_y;
  int scale_pairs;  // both scale arrays 2-byte aligned with even row strides
  // Decode kernels, full windows, W with 16x16 tile scales, every wave holding its whole
  // share of windows, scale rows 4-byte aligned: a wave's scale bytes of a band (the same for
  // all its lanes) come in one scalar load (the launcher then takes the kernels' SS form,
  // where nothing touches LDS before the band loop).
  int scalar_scales;
  // Decode kernel with the activation quantization fused in: bf16 A (m x k, row stride ld_a),
  // and where workgroup 0 writes the quantized A (each pointer may be NULL: not written; the
  // row strides are a.ld_codes / a.ld_scales).
  const uint16_t *a_bf16;
  int64_t ld_a;
  uint8_t *aq_codes, *aq_scales;
  float *aq_gs;
};

constexpr int kSmallMWin = 8;

template <bool W2D>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_small_m(SmallMArgs p) {
  __shared__ floatx4_t s_red[4][kWave];
  const float alpha = load_global_scale(p.a.gs) * load_global_scale(p.w.gs);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t wr = min(n0 + i16, p.n - 1);
  const uint8_t *w_row = p.w.codes + wr * p.w.ld_codes + q * 16;
  const uint8_t *w_srow = p.w.scales + (W2D ? (wr >> 4) : wr) * p.w.ld_scales + q * 2;
  const bool a_ok = i16 < p.m;
  const int64_t ar = a_ok ? i16 : 0;
  const uint8_t *a_row = p.a.codes + ar * p.a.ld_codes + q * 16;
  const uint8_t *a_srow = p.a.scales + ar * p.a.ld_scales + q * 2;
  // 128-wide K windows, split contiguously over the 4 waves.
  const int64_t nwin = (p.k + 127) / 128;
  const int64_t per = (nwin + 3) / 4;
  const int64_t w_begin = wave * per, w_end = min(w_begin + per, nwin);
  const int64_t kbytes = p.k / 2, kblocks = p.k / 16;
  floatx4_t acc = floatx4_t{};
  for (int64_t win0 = w_begin; win0 < w_end; win0 += kSmallMWin) {
    uint4 wv[kSmallMWin], av[kSmallMWin];
    uint32_t ws_[kSmallMWin], as_[kSmallMWin];
#pragma unroll
    for (int u = 0; u < kSmallMWin; ++u) {
      const int64_t win = win0 + u;
      const bool in = win < w_end;
      const int64_t rem = in ? kbytes - win * 64 - q * 16 : 0;   // code bytes left for this lane
      const int64_t remb = in ? kblocks - win * 8 - q * 2 : 0;   // scale blocks left
      wv[u] = load16_masked(w_row + win * 64, rem);
      av[u] = a_ok ? load16_masked(a_row + win * 64, rem) : make_uint4(0, 0, 0, 0);
      // Scale pairs as one 16-bit load when both blocks exist and the scale rows are 2-byte
      // aligned (lane offsets are even); otherwise byte by byte.
      uint32_t wsv = 0, asv = 0;
      if (!p.scale_pairs) {
        wsv = (remb > 0 ? w_srow[win * 8] : 0u) | (remb > 1 ? (uint32_t)w_srow[win * 8 + 1] << 8 : 0u);
        if (a_ok)
          asv = (remb > 0 ? a_srow[win * 8] : 0u) | (remb > 1 ? (uint32_t)a_srow[win * 8 + 1] << 8 : 0u);
      } else if (remb > 1) {
        wsv = *(const uint16_t *)(w_srow + win * 8);
        if (a_ok) asv = *(const uint16_t *)(a_srow + win * 8);
      } else if (remb == 1) {
        wsv = w_srow[win * 8];
        if (a_ok) asv = a_srow[win * 8];
      }
      ws_[u] = wsv;
      as_[u] = asv;
    }
#pragma unroll
    for (int u = 0; u < kSmallMWin; ++u) {
      const half2_t swp = scales_f16x2(ws_[u]), sap = scales_f16x2(as_[u]);
      const half2_t sw0 = splat_lo(swp), sw1 = splat_hi(swp);
      const half2_t sa0 = splat_lo(sap), sa1 = splat_hi(sap);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8_t wop = decode8_f16(word(wv[u], kk), kk < 2 ? sw0 : sw1);
        const half8_t aop = decode8_f16(word(av[u], kk), kk < 2 ? sa0 : sa1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc, 0, 0, 0);
      }
    }
  }
  s_red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const floatx4_t s = s_red[0][lane] + s_red[1][lane] + s_red[2][lane] + s_red[3][lane];
    if (i16 < p.m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + 4 * q + r;
        if (n < p.n) ntstore_u16(p.y + (int64_t)i16 * p.ld_y + n, f32_to_bf16_rne(s[r] * alpha));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Decode-shaped kernels (m <= 16, K <= 4096): one workgroup of 16 waves per CU walks the 16-row
// bands of W (bands b, b + G, b + 2G, ... for a grid of G).  Wave w owns the w-th sixteenth of K
// for every band and keeps its slice of A, ready for the MFMA, in registers for the whole call,
// so the loop only streams W.  dec_depth bands of W are in flight per workgroup (4: with the
// launch grid, all of a workgroup's bands for N up to 16384): a band's registers are refilled
// with the band dec_depth steps ahead as soon as they have been multiplied.  The sixteen partial
// sums of each band of a round meet in LDS, one barrier per round.
//
// FULL (K a multiple of 128, scale rows 2-byte aligned with even strides, W's codes and scales
// each under 2 GiB): W is read with buffer loads whose offsets are unsigned 32-bit; windows past
// a wave's share and bands past the last one get an offset beyond the buffer's size, which the
// hardware answers with zeros and no memory access.  No load then sits under control flow, the
// band loop refills its ring unconditionally, and each load stays in flight until its data is
// used.  Other shapes take masked loads from clamped addresses.
// ---------------------------------------------------------------------------------------------
constexpr int kDecWaves = 16;
constexpr int kDecWin = 2;  // 128-wide K windows per wave at most (K <= 16 * 2 * 128)
// Bands of W in flight per workgroup: as many as the 128 registers of a 16-wave workgroup hold
// next to the rest of the kernel (deep: the FULL forms, except the W4A4 one where every wave
// quantizes its slice of A, which measured faster with 3 bands of two windows while its ring
// went out whole, and no slower since the ring goes out in parts).
constexpr int dec_depth(int win, bool deep) { return win == 1 || deep ? 4 : 3; }
constexpr uint32_t kBufOutOfRange = 0x80000000u;  // above every buffer size used here

template <int WIN>
struct DecodeW {
  u32x4_t v[WIN];
  // Two scale bytes per window (the lane's two 16-value blocks), kept 16-bit so that no
  // widening of a loaded value is placed ahead of its use.
  uint16_t s[WIN];
  // The SS form: the wave's 8 WIN scale bytes of the band, as loaded by one scalar load
  // (uniform, so they stay in scalar registers); lane group q's pair is picked at use.
  uint32_t sd[2 * WIN];
};

// Scale pair of window u for lane group q (bits 0-15).
template <bool SS, int WIN>
__device__ __forceinline__ uint32_t scale_pair(const DecodeW<WIN> &w, int u, int q) {
  if (!SS) return w.s[u];
  const uint32_t dw = (q & 2) ? w.sd[2 * u + 1] : w.sd[2 * u];
  return dw >> ((q & 1) * 16);
}

// Buffer resources over W's codes and scales (raw, byte-addressed, sized to the data).
struct WBufs {
  __amdgpu_buffer_rsrc_t codes, scales;
};

__device__ __forceinline__ WBufs make_wbufs(const SmallMArgs &p) {
  const int64_t srows = p.w.block_rows == 16 ? (p.n + 15) / 16 : p.n;
  const int32_t cbytes = (int32_t)((p.n - 1) * p.w.ld_codes + p.k / 2);
  const int32_t sbytes = (int32_t)((srows - 1) * p.w.ld_scales + p.k / 16);
  WBufs b;
  b.codes = __builtin_amdgcn_make_buffer_rsrc((void *)p.w.codes, 0, cbytes, 0x00020000);
  b.scales = __builtin_amdgcn_make_buffer_rsrc((void *)p.w.scales, 0, sbytes, 0x00020000);
  return b;
}

template <bool W2D, bool FULL, int WIN, bool SS = false>
__device__ __forceinline__ void load_decode_w(const SmallMArgs &p, const WBufs &buf, int64_t band,
                                              int64_t nbands, int i16, int q, int64_t win0,
                                              int nw, DecodeW<WIN> &r) {
  if (FULL) {
    const bool valid = band < nbands;
    const int64_t row = min(band * 16 + i16, p.n - 1);
    // 32-bit offsets; the empty asm keeps the adds plain (see gv_load_row).
    uint32_t rc = (uint32_t)row * (uint32_t)p.w.ld_codes;
    uint32_t rs = (uint32_t)(W2D ? band : row) * (uint32_t)p.w.ld_scales;
    asm volatile("" : "+v"(rc), "+v"(rs));
    const uint32_t cb = rc + q * 16, sb = rs + q * 2;
    if (SS) {
      // The wave's 8 WIN scale bytes of the band (bands past the last read the last band's,
      // whose codes load as zeros and whose outputs are never stored): one scalar load; lane
      // group q takes the two bytes of its blocks in each window at use (scale_pair).
      typedef __attribute__((address_space(4))) const u32x4_t cu32x4;
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      typedef __attribute__((address_space(4))) const u32x2 cu32x2;
      const uint32_t off = __builtin_amdgcn_readfirstlane(
          (uint32_t)(min(band, nbands - 1) * p.w.ld_scales + win0 * 8));
      const uint8_t *sp = p.w.scales + off;
      if (WIN == 2) {
        const u32x4_t v = *(cu32x4 *)(uintptr_t)sp;
        r.sd[0] = v[0];
        r.sd[1] = v[1];
        r.sd[2 * WIN - 2] = v[2];
        r.sd[2 * WIN - 1] = v[3];
      } else {
        const u32x2 v = *(cu32x2 *)(uintptr_t)sp;
        r.sd[0] = v[0];
        r.sd[1] = v[1];
      }
#pragma unroll
      for (int u = 0; u < WIN; ++u)
        r.v[u] = __builtin_amdgcn_raw_buffer_load_b128(
            buf.codes, (int)(valid ? cb + (uint32_t)(win0 + u) * 64 : kBufOutOfRange), 0, 0);
      return;
    }
#pragma unroll
    for (int u = 0; u < WIN; ++u) {
      const bool in = valid && u < nw;
      const uint32_t co = in ? cb + (uint32_t)(win0 + u) * 64 : kBufOutOfRange;
      const uint32_t so = in ? sb + (uint32_t)(win0 + u) * 8 : kBufOutOfRange;
      r.v[u] = __builtin_amdgcn_raw_buffer_load_b128(buf.codes, (int)co, 0, 0);
      r.s[u] = __builtin_amdgcn_raw_buffer_load_b16(buf.scales, (int)so, 0, 0);
    }
    return;
  }
  band = min(band, nbands - 1);  // past the last band: a valid address, never used
  const int64_t row = min(band * 16 + i16, p.n - 1);
  const uint8_t *wrow = p.w.codes + row * p.w.ld_codes + q * 16;
  const uint8_t *srow = p.w.scales + (W2D ? band : row) * p.w.ld_scales + q * 2;
  const int64_t kbytes = p.k / 2, kblocks = p.k / 16;
#pragma unroll
  for (int u = 0; u < WIN; ++u) {
    const int64_t win = win0 + u;
    const bool in = u < nw;
    const int64_t rem = in ? kbytes - win * 64 - q * 16 : 0;
    const int64_t remb = in ? kblocks - win * 8 - q * 2 : 0;
    const uint4 v = load16_masked(wrow + win * 64, rem);
    r.v[u] = u32x4_t{v.x, v.y, v.z, v.w};
    uint32_t sv = 0;
    if (p.scale_pairs && remb > 1) {
      sv = *(const uint16_t *)(srow + win * 8);
    } else {
      sv = (remb > 0 ? srow[win * 8] : 0u) | (remb > 1 ? (uint32_t)srow[win * 8 + 1] << 8 : 0u);
    }
    r.s[u] = (uint16_t)sv;
  }
}

// Issues the loads of ring slots J0 .. J1 - 1 (the workgroup's bands J0 .. J1 - 1 of its first
// dec_depth), all of them by default.
template <bool W2D, bool FULL, int WIN, bool SS, int D, int J0 = 0, int J1 = D>
__device__ __forceinline__ void decode_ring_start(const SmallMArgs &p, const WBufs &buf,
                                                  int64_t nbands, int i16, int q, int64_t win0,
                                                  int nw, DecodeW<WIN> (&ring)[D]) {
  static_assert(0 <= J0 && J0 < J1 && J1 <= D, "ring slots");
#pragma unroll
  for (int j = J0; j < J1; ++j)
    load_decode_w<W2D, FULL, WIN, SS>(p, buf, blockIdx.x + (int64_t)j * gridDim.x, nbands, i16, q,
                                  win0, nw, ring[j]);
  // Work on A that follows must not move above these loads (it would wait for A first).
  __builtin_amdgcn_sched_barrier(0);
}

// The band loop, in rounds of D bands (bands base + j G, j < D, for a grid of G).
// mul(ring slot) returns the wave's 16x16 partial product of a band and the slot is refilled with
// the band D G further on.  After a round the D partials of the 16 waves meet in LDS: after one
// barrier, thread t adds the 16 waves' values of output (band t / 256, lane (t / 4) % 64,
// component t % 4) in wave order, and a second barrier frees the buffer for the next round.  The
// main loop runs while all D bands of a round are real, so its refills need no condition (past
// the last band they load nothing in the FULL form); the last, partial round only drains.  The
// scheduler may interleave the W decode of one band with the MFMAs of another; that overlap
// measured faster than keeping each band's waits precise with scheduling barriers.
template <bool W2D, bool FULL, int WIN, bool SS, int D, class Mul>
__device__ __forceinline__ void decode_band_loop(const SmallMArgs &p, const WBufs &buf,
                                                 int64_t nbands, int lane, int wave,
                                                 int64_t win0, int nw, float alpha_a, float alpha_w,
                                                 DecodeW<WIN> (&ring)[D],
                                                 floatx4_t (*s_red)[kDecWaves][kWave], Mul mul) {
  static_assert(D * 256 <= kDecWaves * 64, "at most one output per thread and round");
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t g = gridDim.x;
  const int fj = threadIdx.x >> 8, fl = (threadIdx.x >> 2) & 63, fc = threadIdx.x & 3;
  const int frow = fl & 15;
  auto finish = [&](const floatx4_t (&acc)[D], int64_t base) {
#pragma unroll
    for (int j = 0; j < D; ++j) s_red[j][wave][lane] = acc[j];
    __syncthreads();
    const int64_t band = base + fj * g;
    if (fj < D && band < nbands && frow < p.m) {
      float t = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) t += ((const float *)&s_red[fj][w2][fl])[fc];
      const int64_t n = band * 16 + 4 * (fl >> 4) + fc;
      // A plain store: the end of the kernel waits for it, and a write-back one through L2
      // completes sooner than a streaming one (measured 0.1-0.3 us per call).
      // The W global scale is first used here, after the bands: its load went out before the W
      // ring, and a use hoisted ahead of the loop would wait for the whole ring (the empty asm
      // keeps the multiply in place).
      float aw = alpha_w;
      asm volatile("" : "+v"(aw));
      if (n < p.n) p.y[(int64_t)frow * p.ld_y + n] = (uint16_t)f32_to_bf16_rne(t * (alpha_a * aw));
    }
    __syncthreads();
  };
  floatx4_t acc[D];
  int64_t base = blockIdx.x;
  for (; base + (D - 1) * g < nbands; base += D * g) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      acc[j] = mul(ring[j]);
      load_decode_w<W2D, FULL, WIN, SS>(p, buf, base + (j + D) * g, nbands, i16, q, win0, nw,
                                        ring[j]);
    }
    finish(acc, base);
  }
  if (base < nbands) {
#pragma unroll
    for (int j = 0; j < D; ++j) acc[j] = base + j * g < nbands ? mul(ring[j]) : floatx4_t{};
    finish(acc, base);
  }
}

// W4A4.  FUSED: A arrives as bf16 and every workgroup quantizes it itself (amax over all of A,
// the FP32 global scale and the scale tables, then the codes of every K slice), exactly as
// nvfp4_quantize_1d would; workgroup 0 also writes the quantized A when asked to.  A is at most
// 16 rows, so the redundant work is small and no workgroup waits for another.
// LEAD (FUSED with one activation row): wave 0 alone loads the row, finds its amax, builds the
// tables and encodes every slice, while the other waves' W rings, issued once the row's loads
// are out (a first barrier), are in flight; they meet it at a second barrier.  Otherwise each
// wave loads and encodes its own slice, and its ring goes out in three parts after the amax
// barrier (a W ring issued before it delays the activation loads of the waves that start
// later): one band there, one after the tables, the rest after the encode.  A wave that issues
// loads while the CU's memory pipeline is full of W requests stalls at that instruction until
// earlier requests drain, so with the whole ring issued at the amax barrier the table barrier
// waited for the last wave to get its loads out (the table phase took 3 us at 16 rows, 1.2 us
// with no ring in flight); issued in parts, the quantization runs while the first bands stream
// (1.0-1.6 us faster at 2-16 rows; the whole ring after the tables or after the encode, or two
// bands at the amax barrier, measured in between).
template <bool W2D, bool FUSED, bool FULL, int WIN, bool LEAD = false, bool SS = false>
__global__ __launch_bounds__(kDecWaves * 64) void k_gemm_decode(SmallMArgs p) {
  static_assert(!SS || (W2D && FULL), "one scalar scale load per band needs 2D scales, full windows");
  static_assert(!LEAD || FUSED, "the lead-wave form quantizes A");
  constexpr int D = dec_depth(WIN, FULL && (!FUSED || LEAD));
  __shared__ floatx4_t s_red[D][kDecWaves][kWave];
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kDecWaves];
  // Quantized A slice of each wave (fused form): up to 16 rows x 16 blocks.
  __shared__ __align__(8) uint8_t s_acodes[FUSED ? kDecWaves : 1][16 * 16 * 8];
  __shared__ uint8_t s_ascales[FUSED ? kDecWaves : 1][16 * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t nwin = (p.k + 127) / 128;
  const int64_t per = (nwin + kDecWaves - 1) / kDecWaves;  // <= WIN, checked by the launcher
  const int64_t win0 = wave * per;
  const int nw = (int)max((int64_t)0, min(per, nwin - win0));
  const int64_t kbytes = p.k / 2, kblocks = p.k / 16;
  const int64_t nbands = (p.n + 15) / 16;
  const WBufs buf = make_wbufs(p);
  // Read before any load of A or W is issued, so that waiting for it waits for nothing else.
  const float gs_w = load_global_scale(p.w.gs);
  const float gs_a_in = FUSED ? 0.0f : load_global_scale(p.a.gs);

  // This wave's K slice of A, decoded once: window u, K step kk -> 8 fp16 values of A row i16.
  half8_t aop[WIN][4];
  float gs_a = 0.0f;
  DecodeW<WIN> ring[D];
  if (FUSED) {
    const int64_t kb0 = win0 * 8;                                       // first block of the slice
    const int bps = (int)max((int64_t)0, min(per * 8, kblocks - kb0));  // blocks per row
    uint8_t *lc = s_acodes[wave], *ls = s_ascales[wave];
    if (LEAD) {
      // Wave 0: lane l takes blocks l, l + 64, l + 128, l + 192 of the row (K <= 4096); lanes
      // past the row reload its last block, which leaves the maximum unchanged.  Its own W ring
      // goes out after these loads; the other waves issue theirs at once.
      if (wave == 0) {
        constexpr int kLB = 4;
        const int nb = (int)kblocks;
        uint4 xa[kLB][2];
#pragma unroll
        for (int j = 0; j < kLB; ++j) {
          const uint16_t *src = p.a_bf16 + (int64_t)min(j * 64 + lane, nb - 1) * 16;
          xa[j][0] = *(const uint4 *)src;
          xa[j][1] = *(const uint4 *)(src + 8);
        }
        // The other waves issue their rings only after this barrier, behind the row's loads.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        decode_ring_start<W2D, FULL, WIN, SS>(p, buf, nbands, i16, q, win0, nw, ring);
        uint32_t mx = 0;
#pragma unroll
        for (int j = 0; j < kLB; ++j) mx = max(mx, absmax16(xa[j][0], xa[j][1]));
        mx = wave_max_u32(mx);
        const float g = global_scale_from_amax_bits(mx);
        build_tables_one_wave(tab, g);
        if (p.aq_gs && blockIdx.x == 0 && lane == 0) *p.aq_gs = g;
        const float inv6gs = inv6gs_of(g);
        const int spw = (int)per * 8;  // blocks of one wave's slice
#pragma unroll
        for (int j = 0; j < kLB; ++j) {
          const int b = j * 64 + lane;
          if (b < nb) {
            float kq;
            const int code = scale_code(absmax16(xa[j][0], xa[j][1]), tab, inv6gs, &kq);
            const uint2 e = encode16(xa[j][0], xa[j][1], kq, code, g);
            const int w = b / spw, c = b - w * spw;
            *(uint2 *)(s_acodes[w] + c * 8) = e;
            s_ascales[w][c] = (uint8_t)code;
            if (blockIdx.x == 0) {
              if (p.aq_codes) ntstore8(p.aq_codes + b * 8, e);
              if (p.aq_scales) ntstore_u8(p.aq_scales + b, (uint32_t)code);
            }
          }
        }
      } else {
        __builtin_amdgcn_s_barrier();  // wave 0's row loads are out (measured 0.1 us faster)
        decode_ring_start<W2D, FULL, WIN, SS>(p, buf, nbands, i16, q, win0, nw, ring);
      }
      // Only LDS passes between the waves here; the barrier waits for LDS accesses alone, not
      // for the W rings in flight.
      lds_barrier();
      gs_a = tab.gs;
    } else {
      // Each wave loads its own K slice of all m rows of A, coalesced: step j gives lane l the
      // 16-value block j * 64 + l of the slice (row = block / bps, bps blocks per row); lanes past
      // the slice reload its last block (or A's first block when the slice is empty), which leaves
      // the maximum unchanged; steps wholly past the slice load nothing.  The registers give this
      // workgroup's share of the global amax and are then encoded in place; the codes reach the
      // MFMA layout through the wave's own corner of LDS.  W's ring is issued once every wave
      // holds its A: issued earlier, the A loads of the later waves wait behind the W stream of
      // the whole chip (measured: A of the last wave slot about 2 us after the first), and the
      // amax that every wave needs waits for the last of them.
      const int nblk = (int)p.m * bps;                                    // <= 16 * 16
      uint4 xa[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j == 0 || j * 64 < nblk) {  // steps past the slice (small M) load nothing
          const int blk = min(j * 64 + lane, max(nblk - 1, 0));
          const int r = bps > 0 ? blk / bps : 0, c = bps > 0 ? blk - r * bps : 0;
          const uint16_t *src = p.a_bf16 + r * p.ld_a + (bps > 0 ? kb0 + c : 0) * 16;
          xa[j][0] = *(const uint4 *)src;
          xa[j][1] = *(const uint4 *)(src + 8);
        } else {
          xa[j][0] = xa[j][1] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, absmax16(xa[j][0], xa[j][1]));
      mx = wave_max_u32(mx);
      if (lane == 0) red[wave] = mx;
      __syncthreads();
      decode_ring_start<W2D, FULL, WIN, SS, D, 0, 1>(p, buf, nbands, i16, q, win0, nw, ring);
      mx = red[0];
#pragma unroll
      for (int w2 = 1; w2 < kDecWaves; ++w2) mx = max(mx, red[w2]);
      gs_a = global_scale_from_amax_bits(mx);
      build_tables<true>(tab, gs_a);  // an LDS-only barrier: the W ring is in flight
      decode_ring_start<W2D, FULL, WIN, SS, D, 1, 2>(p, buf, nbands, i16, q, win0, nw, ring);
      if (p.aq_gs && blockIdx.x == 0 && threadIdx.x == 0) *p.aq_gs = gs_a;
      const float inv6gs = tab.inv6gs;
      // Encode; codes and scales of the slice go to this wave's LDS corner (row-major, 16 blocks
      // per row at most) and, for workgroup 0, to the caller's quantized A.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = j * 64 + lane;
        if (blk < nblk) {
          const int r = blk / bps, c = blk - r * bps;
          float kq;
          const int code = scale_code(absmax16(xa[j][0], xa[j][1]), tab, inv6gs, &kq);
          const uint2 e = encode16(xa[j][0], xa[j][1], kq, code, gs_a);
          *(uint2 *)(lc + (r * 16 + c) * 8) = e;
          ls[r * 16 + c] = (uint8_t)code;
          if (blockIdx.x == 0) {
            if (p.aq_codes) ntstore8(p.aq_codes + r * p.a.ld_codes + (kb0 + c) * 8, e);
            if (p.aq_scales) ntstore_u8(p.aq_scales + r * p.a.ld_scales + kb0 + c, (uint32_t)code);
          }
        }
      }
      // Each wave reads back only its own corner, and a wave's LDS accesses complete in order:
      // ordering them at wavefront scope suffices, with no workgroup barrier.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      decode_ring_start<W2D, FULL, WIN, SS, D, 2, D>(p, buf, nbands, i16, q, win0, nw, ring);
    }
    // MFMA layout: lane (i16, q), window u holds blocks 8u + 2q and 8u + 2q + 1 of row i16.
    const bool a_ok = i16 < p.m;
#pragma unroll
    for (int u = 0; u < WIN; ++u) {
      const int c0 = u * 8 + q * 2;
      const bool v0 = a_ok && c0 < bps, v1 = a_ok && c0 + 1 < bps;
      const uint2 e0 = v0 ? *(const uint2 *)(lc + (i16 * 16 + c0) * 8) : make_uint2(0, 0);
      const uint2 e1 = v1 ? *(const uint2 *)(lc + (i16 * 16 + c0 + 1) * 8) : make_uint2(0, 0);
      const uint32_t sv = (v0 ? (uint32_t)ls[i16 * 16 + c0] : 0u) |
                          ((v1 ? (uint32_t)ls[i16 * 16 + c0 + 1] : 0u) << 8);
      const uint4 v = make_uint4(e0.x, e0.y, e1.x, e1.y);
      const half2_t sp = scales_f16x2(sv);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        aop[u][kk] = decode8_f16(word(v, kk), kk < 2 ? splat_lo(sp) : splat_hi(sp));
    }
  } else {
    // Rows past m read row m - 1 (their products land in columns that are not stored).
    const int64_t ar = min((int64_t)i16, p.m - 1);
    const uint8_t *arow = p.a.codes + ar * p.a.ld_codes + q * 16;
    const uint8_t *asrow = p.a.scales + ar * p.a.ld_scales + q * 2;
    uint4 av[WIN];
    uint32_t as[WIN];
#pragma unroll
    for (int u = 0; u < WIN; ++u) {
      if (FULL) {
        const int64_t win = min(win0 + u, nwin - 1);
        av[u] = *(const uint4 *)(arow + win * 64);
        as[u] = *(const uint16_t *)(asrow + win * 8);
      } else {
        const int64_t win = win0 + u;
        const bool in = u < nw;
        const int64_t rem = in ? kbytes - win * 64 - q * 16 : 0;
        const int64_t remb = in ? kblocks - win * 8 - q * 2 : 0;
        av[u] = load16_masked(arow + win * 64, rem);
        as[u] = (remb > 0 ? asrow[win * 8] : 0u) |
                (remb > 1 ? (uint32_t)asrow[win * 8 + 1] << 8 : 0u);
      }
    }
    decode_ring_start<W2D, FULL, WIN, SS>(p, buf, nbands, i16, q, win0, nw, ring);
#pragma unroll
    for (int u = 0; u < WIN; ++u) {
      const half2_t sp = scales_f16x2(as[u]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        aop[u][kk] = decode8_f16(word(av[u], kk), kk < 2 ? splat_lo(sp) : splat_hi(sp));
    }
  }

  decode_band_loop<W2D, FULL, WIN, SS>(
      p, buf, nbands, lane, wave, win0, nw, FUSED ? gs_a : gs_a_in, gs_w, ring, s_red,
      [&](const DecodeW<WIN> &w) {
        floatx4_t acc = floatx4_t{};
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
          if (FULL || u < nw) {  // FULL: W of windows past the share is zero
            const half2_t sp = scales_f16x2(scale_pair<SS>(w, u, q));
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const half8_t wop =
                  decode8_f16(word(w.v[u], kk), kk < 2 ? splat_lo(sp) : splat_hi(sp));
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop[u][kk], acc, 0, 0, 0);
            }
          }
        }
        return acc;
      });
}

// ---------------------------------------------------------------------------------------------
// Weight-only W4A16 ("NVFP4 Dynamic Quantization in Practice", section "The Meaning and
// Advantages of W4A4": the 4-bit weights are reconstructed to 16-bit floating point and multiplied
// with 16-bit activations):  Y = RN_bf16(gsW * sum_k A[m, k] * (cW * sbW)[n, k]),  m <= 16.
// The bf16 activations feed the bf16 MFMA unchanged; W is decoded exactly to bf16 (code * block
// scale); gsW factors out of the sum.  Same lane <-> K mapping as the W4A4 decode kernels: lane
// (row i16, group q) covers K values 128 * window + 32 * q + [0, 32) of its row, step kk the
// eight at + 8 * kk.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bf16x8_t load_a_bf16x8(const uint16_t *row, int64_t k0, int64_t k,
                                                  bool ok) {
  // k % 16 == 0 and k0 % 8 == 0: the eight values are all in the row or all past its end.
  const bf16x8_t z = {};
  return ok && k0 < k ? *(const bf16x8_t *)(row + k0) : z;
}

// K <= 4096: the decode form above with bf16 A held in registers.
template <bool W2D, bool FULL, int WIN, bool SS = false>
__global__ __launch_bounds__(kDecWaves * 64) void k_gemm_w4a16_decode(SmallMArgs p) {
  static_assert(!SS || (W2D && FULL), "one scalar scale load per band needs 2D scales, full windows");
  constexpr int D = dec_depth(WIN, FULL);
  __shared__ floatx4_t s_red[D][kDecWaves][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t nwin = (p.k + 127) / 128;
  const int64_t per = (nwin + kDecWaves - 1) / kDecWaves;  // <= WIN, checked by the launcher
  const int64_t win0 = wave * per;
  const int nw = (int)max((int64_t)0, min(per, nwin - win0));
  const int64_t nbands = (p.n + 15) / 16;
  const WBufs buf = make_wbufs(p);
  const float gs_w = load_global_scale(p.w.gs);  // read before the loads of A and W are issued

  bf16x8_t aop[WIN][4];
  if (FULL) {
    // Rows past m read row m - 1, windows past the share the last window: never used.
    const uint16_t *arow = p.a_bf16 + min((int64_t)i16, p.m - 1) * p.ld_a;
#pragma unroll
    for (int u = 0; u < WIN; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        aop[u][kk] = *(const bf16x8_t *)(arow + min(win0 + u, nwin - 1) * 128 + q * 32 + kk * 8);
  } else {
    const bool a_ok = i16 < p.m;
    const uint16_t *arow = p.a_bf16 + (a_ok ? i16 : 0) * p.ld_a;
#pragma unroll
    for (int u = 0; u < WIN; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        aop[u][kk] = load_a_bf16x8(arow, (win0 + u) * 128 + q * 32 + kk * 8, p.k, a_ok && u < nw);
  }
  DecodeW<WIN> ring[D];
  decode_ring_start<W2D, FULL, WIN, SS>(p, buf, nbands, i16, q, win0, nw, ring);

  decode_band_loop<W2D, FULL, WIN, SS>(
      p, buf, nbands, lane, wave, win0, nw, 1.0f, gs_w, ring, s_red, [&](const DecodeW<WIN> &w) {
        floatx4_t acc = floatx4_t{};
#pragma unroll
        for (int u = 0; u < WIN; ++u) {
          if (FULL || u < nw) {  // FULL: W of windows past the share is zero
            const floatx2_t sf = scales_f32x2(scale_pair<SS>(w, u, q));
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const bf16x8_t wop = decode8_bf16(word(w.v[u], kk), kk < 2 ? sf[0] : sf[1]);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop, aop[u][kk], acc, 0, 0, 0);
            }
          }
        }
        return acc;
      });
}

// ---------------------------------------------------------------------------------------------
// W4A16 GEMV for a single activation row (m == 1, K = 1024 * NB with NB in {2, 4, 8}): no
// MFMA, no LDS reduction and no barrier in the loop.  Each wave owns whole rows of W (rows w,
// w + G, ... for G waves in the grid); lane l covers K values [16 NB l, 16 NB (l + 1)), i.e. NB
// blocks: NB * 8 code bytes and NB scale bytes of the row, and the same K range of A, which it
// holds in registers as packed bf16 pairs (A is read from memory once per workgroup, through
// LDS).  The unscaled W codes are converted to bf16 pairs (exact) and multiplied into fp32 with
// the 2-term dot instruction; each 16-value block's sum takes its W scale with one FMA, and the
// 64 lane partials of a row meet through cross-lane adds.  gv_depth(NB) rows are in flight per
// wave, read with buffer loads: rows past the end get an offset beyond the buffer size (zeros,
// no memory access), so the loads carry no control flow.
// Used for N >= 8192, where it measured faster than the decode form (11.4 against 12.0 us at
// 14336 x 4096, 15.0 against 16.6 at 28672 x 4096); for smaller N its fixed cost (A staged
// through LDS, one row per wave) makes it slower.  A W4A4 form was slower than the decode
// kernels at every size measured, so there is none.
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int gv_depth(int nb) { return nb == 8 ? 2 : 4; }

template <int NB>
struct GvRow {
  u32x4_t c[NB / 2];  // NB * 8 code bytes
  uint32_t s[(NB + 3) / 4];
};

template <bool W2D, int NB>
__device__ __forceinline__ void gv_load_row(const SmallMArgs &p, const WBufs &buf, int64_t row,
                                            int lane, GvRow<NB> &r) {
  const bool valid = row < p.n;
  const int64_t srow = W2D ? row / 16 : row;
  // The offsets fit in 32 bits (buffers under 2 GiB).  The row products pass through an empty
  // asm so that the lane offset is added with a plain 32-bit add: fused into a 64-bit
  // multiply-add, the unused high half of the addend lands in a register that a pending load
  // writes, and the read then waits for that load.
  uint32_t rc = (uint32_t)row * (uint32_t)p.w.ld_codes, rs = (uint32_t)srow * (uint32_t)p.w.ld_scales;
  asm volatile("" : "+v"(rc), "+v"(rs));
  const uint32_t co = valid ? rc + lane * (NB * 8) : kBufOutOfRange;
  const uint32_t so = valid ? rs + lane * NB : kBufOutOfRange;
#pragma unroll
  for (int i = 0; i < NB / 2; ++i)
    r.c[i] = __builtin_amdgcn_raw_buffer_load_b128(buf.codes, (int)(co + (valid ? 16 * i : 0)), 0, 0);
  if (NB == 2) r.s[0] = __builtin_amdgcn_raw_buffer_load_b16(buf.scales, (int)so, 0, 0);
  if (NB == 4) r.s[0] = __builtin_amdgcn_raw_buffer_load_b32(buf.scales, (int)so, 0, 0);
  if (NB == 8) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(buf.scales, (int)so, 0, 0);
    r.s[0] = v[0];
    r.s[1] = v[1];
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <bool W2D, int NB>
__global__ __launch_bounds__(kDecWaves * 64) void k_gemv_w4a16(SmallMArgs p) {
  constexpr int D = gv_depth(NB);
  constexpr int NW = NB * 2;  // code words per lane per row
  // The wave index is uniform; saying so keeps the row logic scalar.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)gridDim.x * kDecWaves;
  const int64_t first = (int64_t)blockIdx.x * kDecWaves + wave;
  const WBufs buf = make_wbufs(p);
  const float alpha = load_global_scale(p.w.gs);

  // A (one row) is read from memory once per workgroup into LDS (thread t copies 16-byte chunk
  // t; its load goes out before the W loads, so waiting for it waits for nothing else); every
  // wave then takes its copy from there.  Lane l's K range: NB blocks of 16 values.
  __shared__ __align__(16) uint8_t s_a[NB * 2048];
  const int tid = threadIdx.x;
  constexpr int kChunks = NB * 128;  // <= 1024 = the workgroup size
  uint4 achunk = make_uint4(0, 0, 0, 0);
  if (tid < kChunks) achunk = *(const uint4 *)(p.a_bf16 + 8 * tid);
  GvRow<NB> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    gv_load_row<W2D, NB>(p, buf, first + j * g, lane, ring[j]);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads in row order: row j waits only for rows <= j
  }
  if (tid < kChunks) *(uint4 *)(s_a + 16 * tid) = achunk;
  lds_barrier();
  // A as packed bf16 pairs.
  uint32_t a2[NW * 4];
#pragma unroll
  for (int i = 0; i < 2 * NB; ++i) {
    const uint4 v = *(const uint4 *)(s_a + lane * (NB * 32) + 16 * i);
    a2[4 * i] = v.x;
    a2[4 * i + 1] = v.y;
    a2[4 * i + 2] = v.z;
    a2[4 * i + 3] = v.w;
  }

  for (int64_t base = first; base < p.n; base += D * g) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int64_t row = base + j * g;
      float acc = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t sbyte = (ring[j].s[b / 4] >> (8 * (b % 4))) & 0xFFu;
        const float sb = scales_f32x2(sbyte)[0];
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const uint32_t q = ring[j].c[b / 2][2 * (b % 2) + w];
          const bf16x2_t wv[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0),
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1),
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2),
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3)};
#pragma unroll
          for (int sel = 0; sel < 4; ++sel)
            sum = __builtin_amdgcn_fdot2_f32_bf16(
                wv[sel], __builtin_bit_cast(bf16x2_t, a2[(2 * b + w) * 4 + sel]), sum, false);
        }
        acc = __builtin_fmaf(sum, sb, acc);
      }
      gv_load_row<W2D, NB>(p, buf, row + D * g, lane, ring[j]);
      const float t = wave_sum(acc);
      if (lane == 0 && row < p.n) ntstore_u16(p.y + row, f32_to_bf16_rne(t * alpha));
    }
  }
}

// Any K: one workgroup of 16 waves per band; wave w takes windows w, w + 16, ..., loading W and
// A for up to kW16Chunk of them at a time (A comes from L2: it is at most 16 rows).
constexpr int kW16Chunk = 4;

template <bool W2D>
__global__ __launch_bounds__(kDecWaves * 64) void k_gemm_w4a16_stream(SmallMArgs p) {
  __shared__ floatx4_t s_red[kDecWaves][kWave];
  const float gs_w = load_global_scale(p.w.gs);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  const int64_t band = blockIdx.x;
  const int64_t row = min(band * 16 + i16, p.n - 1);
  const uint8_t *wrow = p.w.codes + row * p.w.ld_codes + q * 16;
  const uint8_t *srow = p.w.scales + (W2D ? band : row) * p.w.ld_scales + q * 2;
  const bool a_ok = i16 < p.m;
  const uint16_t *arow = p.a_bf16 + (a_ok ? i16 : 0) * p.ld_a;
  const int64_t nwin = (p.k + 127) / 128;
  const int64_t kbytes = p.k / 2, kblocks = p.k / 16;
  floatx4_t acc = floatx4_t{};
  for (int64_t c0 = wave; c0 < nwin; c0 += kDecWaves * kW16Chunk) {
    uint4 wv[kW16Chunk];
    uint32_t ws_[kW16Chunk];
    bf16x8_t av[kW16Chunk][4];
#pragma unroll
    for (int u = 0; u < kW16Chunk; ++u) {
      const int64_t win = c0 + (int64_t)u * kDecWaves;
      const bool in = win < nwin;
      const int64_t rem = in ? kbytes - win * 64 - q * 16 : 0;
      const int64_t remb = in ? kblocks - win * 8 - q * 2 : 0;
      wv[u] = load16_masked(wrow + win * 64, rem);
      uint32_t sv = 0;
      if (p.scale_pairs && remb > 1)
        sv = *(const uint16_t *)(srow + win * 8);
      else
        sv = (remb > 0 ? srow[win * 8] : 0u) | (remb > 1 ? (uint32_t)srow[win * 8 + 1] << 8 : 0u);
      ws_[u] = sv;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        av[u][kk] = load_a_bf16x8(arow, win * 128 + q * 32 + kk * 8, p.k, a_ok && in);
    }
#pragma unroll
    for (int u = 0; u < kW16Chunk; ++u) {
      const floatx2_t sf = scales_f32x2(ws_[u]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t wop = decode8_bf16(word(wv[u], kk), kk < 2 ? sf[0] : sf[1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop, av[u][kk], acc, 0, 0, 0);
      }
    }
  }
  s_red[wave][lane] = acc;
  __syncthreads();
  if (wave < 4 && i16 < p.m) {
    float t = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) t += ((const float *)&s_red[w2][lane])[wave];
    const int64_t n = band * 16 + 4 * q + wave;
    if (n < p.n) ntstore_u16(p.y + (int64_t)i16 * p.ld_y + n, f32_to_bf16_rne(t * gs_w));
  }
}

// ---------------------------------------------------------------------------------------------
// Mid-size M (16 < M <= 128, K a multiple of 1024): output tiles of 32 FM rows by 64 columns
// (the launcher uses FM = 2, and FM = 4 for M > 64 on wide 2D-scaled weights), one per
// workgroup, so a 14336-row W gives 224 workgroups per row slice.  The 4 waves split K in four
// contiguous quarters; each wave computes the whole tile over its quarter (FM x 2 MFMA tiles of
// 32 x 32) with four 64-wide windows of loads in flight, and the four partial tiles are added
// through LDS.  W is read once per row slice of A;
// nothing but Y goes to memory.  FM = 2 leaves room for two workgroups per CU.  SCV (scale rows
// 16-byte aligned): the scales of a round of four windows come in one 16-byte load per
// fragment row (a 32-bit word per window; lane half kh takes its two bytes by a shift), in
// place of a 16-bit load per window.
// ---------------------------------------------------------------------------------------------
constexpr int kMidDepth = 4;

template <int FM, bool W2D, bool SCV>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_mid(DenseArgs p) {
  __shared__ float s_red[4][FM][2][16][kWave];  // [wave][f][g][register][lane]
  const float alpha = load_global_scale(p.a.gs) * load_global_scale(p.w.gs);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, kh = lane >> 5;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * (32 * FM), n0 = (int64_t)tn * 64;

  // Rows clamped into the matrices; results of clamped rows are never stored.
  const int64_t wpw = p.k / 256;  // windows per wave, a multiple of kMidDepth
  const int64_t w_first = wave * wpw;
  const uint8_t *a_row[FM], *a_srow[FM], *w_row[2], *w_srow[2];
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int64_t r = min(m0 + f * 32 + lr, p.m - 1);
    a_row[f] = p.a.codes + r * p.a.ld_codes + kh * 16 + w_first * 32;
    a_srow[f] = p.a.scales + r * p.a.ld_scales + (SCV ? 0 : kh * 2) + w_first * 4;
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int64_t r = min(n0 + g * 32 + lr, p.n - 1);
    w_row[g] = p.w.codes + r * p.w.ld_codes + kh * 16 + w_first * 32;
    w_srow[g] = p.w.scales + (W2D ? (r >> 4) : r) * p.w.ld_scales + (SCV ? 0 : kh * 2) +
                w_first * 4;
  }
  floatx16_t acc[FM][2];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[f][g] = floatx16_t{};

  // Ring of kMidDepth windows: full rounds refill every slot after using it, the last round
  // only drains, so no load sits under a branch.  Two scale bytes per fragment come in one
  // 16-bit load.  The scheduling barriers keep the loads in window order, so that waiting for
  // window j waits for nothing issued after it.
  auto load = [&](Frags<FM, 2> &fr, int64_t win) {
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      fr.a[f] = load16(a_row[f] + win * 32);
      if (!SCV) fr.sa[f] = *(const uint16_t *)(a_srow[f] + win * 4);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      fr.w[g] = load16(w_row[g] + win * 32);
      if (!SCV) fr.sw[g] = *(const uint16_t *)(w_srow[g] + win * 4);
    }
  };
  struct RoundScales {
    uint4 a[FM], w[2];
  };
  static_assert(kMidDepth == 4, "a 16-byte scale load covers four windows");
  auto load_scales = [&](RoundScales &q, int64_t win) {
#pragma unroll
    for (int f = 0; f < FM; ++f) q.a[f] = *(const uint4 *)(a_srow[f] + win * 4);
#pragma unroll
    for (int g = 0; g < 2; ++g) q.w[g] = *(const uint4 *)(w_srow[g] + win * 4);
  };
  const uint32_t ssh = 16u * kh;
  auto set_scales = [&](Frags<FM, 2> &fr, const RoundScales &q, int j) {
#pragma unroll
    for (int f = 0; f < FM; ++f) fr.sa[f] = word(q.a[f], j) >> ssh;
#pragma unroll
    for (int g = 0; g < 2; ++g) fr.sw[g] = word(q.w[g], j) >> ssh;
  };
  Frags<FM, 2> ring[kMidDepth];
  RoundScales cur, nxt;
  if (SCV) load_scales(cur, 0);
#pragma unroll
  for (int j = 0; j < kMidDepth; ++j) {
    load(ring[j], j);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t i = 0; i + kMidDepth < wpw; i += kMidDepth) {
#pragma unroll
    for (int j = 0; j < kMidDepth; ++j) {
      if (SCV) set_scales(ring[j], cur, j);
      compute_window(ring[j], acc);
      __builtin_amdgcn_sched_barrier(0);
      if (SCV && j == 0) load_scales(nxt, i + kMidDepth);
      load(ring[j], i + j + kMidDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (SCV) cur = nxt;
  }
#pragma unroll
  for (int j = 0; j < kMidDepth; ++j) {
    if (SCV) set_scales(ring[j], cur, j);
    compute_window(ring[j], acc);
  }

  // Add the four quarters: every wave stores its tile, then wave q finishes MFMA tiles
  // t = q * FM / 2 .. (q + 1) * FM / 2 - 1 (tile t is (t / 2, t % 2)) from all four copies.
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_red[wave][f][g][r][lane] = acc[f][g][r];
  __syncthreads();
#pragma unroll
  for (int t = 0; t < FM / 2; ++t) {
    const int tile = wave * (FM / 2) + t, f = tile >> 1, g = tile & 1;
    const int64_t col = n0 + g * 32 + lr;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {  // rows r and r + 1 are adjacent
      float v0 = s_red[0][f][g][r][lane], v1 = s_red[0][f][g][r + 1][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        v0 += s_red[w][f][g][r][lane];
        v1 += s_red[w][f][g][r + 1][lane];
      }
      const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      const uint32_t pk = bf16x2_rne(v0 * alpha, v1 * alpha);
      if (row < p.m && col < p.n) ntstore_u16(p.y + row * p.ld_y + col, pk);
      if (row + 1 < p.m && col < p.n) ntstore_u16(p.y + (row + 1) * p.ld_y + col, pk >> 16);
    }
  }
}

// Y = RN_bf16(gsA * gsW * sum over splits of the fp32 partials); four columns per thread
// (n % 4 == 0), the splits added in order.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ part, int splits,
                                                       int64_t m, int64_t n,
                                                       uint16_t *__restrict__ y, int64_t ld_y,
                                                       const float *__restrict__ gsa,
                                                       const float *__restrict__ gsw) {
  const float alpha = (*gsa) * (*gsw);
  const int64_t per_row = n / 4, total = m * per_row, slab = m * n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per_row, c = (i - r * per_row) * 4;
    const float *src = part + r * n + c;
    float4 s = *(const float4 *)src;
    for (int t = 1; t < splits; ++t) {
      const float4 v = *(const float4 *)(src + t * slab);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    uint32_t *dst = (uint32_t *)(y + r * ld_y + c);  // ld_y and y are 2-element aligned
    dst[0] = bf16x2_rne(s.x * alpha, s.y * alpha);
    dst[1] = bf16x2_rne(s.z * alpha, s.w * alpha);
  }
}

// ---------------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------------
static hipError_t launch_splitk_reduce(const DenseArgs &p, int splits, hipStream_t stream) {
  const int64_t total = p.m * (p.n / 4);
  int64_t g = (total + 255) / 256;
  g = g < 1 ? 1 : (g > 2048 ? 2048 : g);
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)g), dim3(256), 0, stream, p.part, splits,
                     p.m, p.n, p.y, p.ld_y, p.a.gs, p.w.gs);
  return hipGetLastError();
}

template <int FM, int FN>
static hipError_t launch_tile_fm(const GemmOperand &a, const GemmOperand &w, int64_t m,
                                 int64_t n, int64_t k, uint16_t *y, int64_t ld_y, float *part,
                                 hipStream_t stream) {
  DenseArgs p{};
  p.a = a;
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.tiles_m = (int)((m + 64 * FM - 1) / (64 * FM));
  p.tiles_n = (int)((n + 64 * FN - 1) / (64 * FN));
  const int splits = part ? gemm_k_splits(m, n, k) : 1;
  if (splits > 1) {
    p.part = part;
    p.wps = ((k + 63) / 64 + splits - 1) / splits;  // splits * wps windows cover k, none empty
  }
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n, (unsigned)splits);
  if (w.block_rows == 16)
    hipLaunchKernelGGL((k_gemm_tile<FM, FN, true>), grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_tile<FM, FN, false>), grid, dim3(kGemmThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(p, splits, stream);
}

static bool aligned4(const void *q) { return ((uintptr_t)q & 3u) == 0; }

hipError_t launch_gemm_tile(const GemmOperand &a, const GemmOperand &w, int64_t m, int64_t n,
                            int64_t k, uint16_t *y, int64_t ld_y, float *part,
                            hipStream_t stream) {
  const bool scales2 = ((uintptr_t)a.scales % 2 == 0) && ((uintptr_t)w.scales % 2 == 0) &&
                       a.ld_scales % 2 == 0 && w.ld_scales % 2 == 0;
  const bool scv = (uintptr_t)a.scales % 16 == 0 && (uintptr_t)w.scales % 16 == 0 &&
                   a.ld_scales % 16 == 0 && w.ld_scales % 16 == 0;
  if ((gemm_uses_mid(m, n, k) && scales2) ||
      (gemm_uses_mid_wide(m, n, k) && w.block_rows == 16 && scv)) {
    DenseArgs p{};
    p.a = a;
    p.w = w;
    p.m = m;
    p.n = n;
    p.k = k;
    p.y = y;
    p.ld_y = ld_y;
    p.tiles_m = (int)((m + 63) / 64);
    p.tiles_n = (int)((n + 63) / 64);
    const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
    // M = 65-384 against a wide weight (2D scales, aligned scale rows): 128-row tiles (W read
    // once per row slice; measured 0.7-1.8 us faster than two 64-row slices at M = 65-128).
    if (w.block_rows == 16 && scv && m > 64 && (n + 63) / 64 >= 128) {
      p.tiles_m = (int)((m + 127) / 128);
      hipLaunchKernelGGL((k_gemm_mid<4, true, true>), dim3((unsigned)p.tiles_m * (unsigned)p.tiles_n),
                         dim3(kGemmThreads), 0, stream, p);
    } else if (w.block_rows == 16 && scv)
      hipLaunchKernelGGL((k_gemm_mid<2, true, true>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
    else if (w.block_rows == 16)
      hipLaunchKernelGGL((k_gemm_mid<2, true, false>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
    else if (scv)
      hipLaunchKernelGGL((k_gemm_mid<2, false, true>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((k_gemm_mid<2, false, false>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
    return hipGetLastError();
  }
  if (m <= 64) return launch_tile_fm<1, 4>(a, w, m, n, k, y, ld_y, part, stream);
  if (m <= 128) return launch_tile_fm<2, 4>(a, w, m, n, k, y, ld_y, part, stream);
  // The pipelined kernel needs whole 64-wide K windows and 4-byte aligned scale rows.
  const bool lds_ok = (k % 64 == 0) && aligned4(a.scales) && aligned4(w.scales) &&
                      (a.ld_scales % 4 == 0) && (w.ld_scales % 4 == 0);
  if (!lds_ok) return launch_tile_fm<4, 4>(a, w, m, n, k, y, ld_y, part, stream);
  DenseArgs p{};
  p.a = a;
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.tiles_m = (int)((m + 255) / 256);
  p.tiles_n = (int)((n + 255) / 256);
  const int splits = part ? gemm_k_splits(m, n, k) : 1;
  if (splits > 1) {
    p.part = part;
    p.wps = (k / 64 + splits - 1) / splits;
  }
  const dim3 grid((unsigned)p.tiles_m * (unsigned)p.tiles_n, (unsigned)splits);
  if (w.block_rows == 16)
    hipLaunchKernelGGL(k_gemm_lds<true>, grid, dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_gemm_lds<false>, grid, dim3(kGemmThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(p, splits, stream);
}

// CU count of the current device, queried once per device (256 if the query fails).
static int device_cus() {
  static std::mutex mu;
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cache[dev] = c;
  }
  return cache[dev];
}

// One workgroup per CU, each taking the same number of 16-row bands.
static unsigned decode_grid(int64_t n) {
  const int64_t nbands = (n + 15) / 16;
  const int64_t slots = device_cus();
  const int64_t per_wg = (nbands + slots - 1) / slots;
  return (unsigned)((nbands + per_wg - 1) / per_wg);
}

// Full windows: K a multiple of 128, 16-bit scale-pair loads allowed, W's codes and scales each
// addressable with 31-bit buffer offsets.
static bool decode_full(const SmallMArgs &p) {
  const int64_t srows = p.w.block_rows == 16 ? (p.n + 15) / 16 : p.n;
  const int64_t lim = (int64_t)1 << 31;
  return p.k % 128 == 0 && p.scale_pairs && (p.n - 1) * p.w.ld_codes + p.k / 2 < lim &&
         (srows - 1) * p.w.ld_scales + p.k / 16 < lim;
}

template <bool FUSED, bool FULL, int WIN, bool LEAD = false>
static void launch_decode_t(const SmallMArgs &p, bool w2d, hipStream_t stream) {
  const dim3 grid(decode_grid(p.n)), block(kDecWaves * 64);
  // Not in the forms that quantize A: scalar loads and LDS accesses share one wait counter, so
  // the activation's LDS work would wait for the ring's scale loads (measured 0.4 us slower).
  if (!FUSED && FULL && w2d && p.scalar_scales)
    hipLaunchKernelGGL((k_gemm_decode<true, FUSED, FULL, WIN, LEAD, !FUSED && FULL>), grid, block,
                       0, stream, p);
  else if (w2d)
    hipLaunchKernelGGL((k_gemm_decode<true, FUSED, FULL, WIN, LEAD>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_decode<false, FUSED, FULL, WIN, LEAD>), grid, block, 0, stream, p);
}

// The fused form with one activation row takes the lead-wave kernel.
template <bool FUSED, bool FULL, int WIN>
static void launch_decode_m(const SmallMArgs &p, bool w2d, hipStream_t stream) {
  if (FUSED && p.m == 1) launch_decode_t<FUSED, FULL, WIN, FUSED>(p, w2d, stream);
  else launch_decode_t<FUSED, FULL, WIN>(p, w2d, stream);
}

// Whether a decode launch can take each wave's scale bytes of a band with one scalar load:
// 16x16 tile scales, full windows, every wave holding WIN windows (K = 16 x 128 x WIN), scale
// rows 4-byte aligned.
static bool decode_scalar_scales(const SmallMArgs &p, bool w2d, bool full) {
  const int64_t nwin = (p.k + 127) / 128;
  return w2d && full && (nwin == kDecWaves || nwin == kDecWaves * kDecWin) &&
         (uintptr_t)p.w.scales % 4 == 0 && p.w.ld_scales % 4 == 0;
}

template <bool FUSED>
static hipError_t launch_decode(const SmallMArgs &args, bool w2d, hipStream_t stream) {
  SmallMArgs p = args;
  const bool full = decode_full(p);
  const bool one = (p.k + 127) / 128 <= kDecWaves;  // one window per wave
  p.scalar_scales = decode_scalar_scales(p, w2d, full) ? 1 : 0;
  if (full && one) launch_decode_m<FUSED, true, 1>(p, w2d, stream);
  if (full && !one) launch_decode_m<FUSED, true, 2>(p, w2d, stream);
  if (!full && one) launch_decode_m<FUSED, false, 1>(p, w2d, stream);
  if (!full && !one) launch_decode_m<FUSED, false, 2>(p, w2d, stream);
  return hipGetLastError();
}

template <bool FULL, int WIN>
static void launch_w4a16_t(const SmallMArgs &p, bool w2d, hipStream_t stream) {
  const dim3 grid(decode_grid(p.n)), block(kDecWaves * 64);
  if (FULL && w2d && p.scalar_scales)
    hipLaunchKernelGGL((k_gemm_w4a16_decode<true, FULL, WIN, FULL>), grid, block, 0, stream, p);
  else if (w2d)
    hipLaunchKernelGGL((k_gemm_w4a16_decode<true, FULL, WIN>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_w4a16_decode<false, FULL, WIN>), grid, block, 0, stream, p);
}

// The GEMV form: m == 1, N >= 8192, K = 1024 * NB (NB 2, 4 or 8), W's scale rows aligned to
// NB bytes, and the buffer offsets of W under 2 GiB.
static int gemv_nb(const SmallMArgs &p) {
  const int64_t nb = p.k / 1024;
  if (p.m != 1 || p.n < 8192 || p.k % 1024 || (nb != 2 && nb != 4 && nb != 8)) return 0;
  if ((uintptr_t)p.w.scales % nb || p.w.ld_scales % nb) return 0;
  const int64_t srows = p.w.block_rows == 16 ? (p.n + 15) / 16 : p.n;
  const int64_t lim = (int64_t)1 << 31;
  if ((p.n - 1) * p.w.ld_codes + p.k / 2 >= lim || (srows - 1) * p.w.ld_scales + p.k / 16 >= lim)
    return 0;
  return (int)nb;
}

static hipError_t launch_gemv_w4a16(const SmallMArgs &p, int nb, hipStream_t stream) {
  const int64_t want = (p.n + kDecWaves - 1) / kDecWaves;
  const int64_t slots = device_cus();
  const dim3 grid((unsigned)(want < slots ? want : slots)), block(kDecWaves * 64);
  const bool w2d = p.w.block_rows == 16;
#define NV_GEMV(NB)                                                                      \
  if (nb == NB) {                                                                        \
    if (w2d) hipLaunchKernelGGL((k_gemv_w4a16<true, NB>), grid, block, 0, stream, p);    \
    else hipLaunchKernelGGL((k_gemv_w4a16<false, NB>), grid, block, 0, stream, p);       \
  }
  NV_GEMV(2)
  NV_GEMV(4)
  NV_GEMV(8)
#undef NV_GEMV
  return hipGetLastError();
}

hipError_t launch_gemm_decode_fused(const void *a_bf16, int64_t ld_a, const GemmOperand &aq,
                                    const GemmOperand &w, int64_t m, int64_t n, int64_t k,
                                    uint16_t *y, int64_t ld_y, hipStream_t stream) {
  if (m < 1 || m > 16 || (k + 127) / 128 > kDecWaves * kDecWin) return hipErrorNotSupported;
  SmallMArgs p;
  p.a = aq;
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.scale_pairs = ((uintptr_t)w.scales % 2 == 0) && (w.ld_scales % 2 == 0);
  p.scalar_scales = 0;
  p.a_bf16 = (const uint16_t *)a_bf16;
  p.ld_a = ld_a;
  p.aq_codes = (uint8_t *)aq.codes;
  p.aq_scales = (uint8_t *)aq.scales;
  p.aq_gs = (float *)aq.gs;
  return launch_decode<true>(p, w.block_rows == 16, stream);
}

hipError_t launch_gemm_w4a16(const void *a_bf16, int64_t ld_a, const GemmOperand &w, int64_t m,
                             int64_t n, int64_t k, uint16_t *y, int64_t ld_y, hipStream_t stream) {
  if (m < 1 || m > 16) return hipErrorNotSupported;
  SmallMArgs p;
  p.a = GemmOperand{nullptr, 0, nullptr, 0, nullptr, 1};
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.scale_pairs = ((uintptr_t)w.scales % 2 == 0) && (w.ld_scales % 2 == 0);
  p.scalar_scales = 0;
  p.a_bf16 = (const uint16_t *)a_bf16;
  p.ld_a = ld_a;
  p.aq_codes = p.aq_scales = nullptr;
  p.aq_gs = nullptr;
  const bool w2d = w.block_rows == 16;
  // One activation row takes the band kernel where its full-window form applies (0.6-0.9 us
  // faster than the GEMV at 14336 x 4096); the GEMV serves the longer K it also covers.
  const bool dec_fits = (k + 127) / 128 <= kDecWaves * kDecWin;
  if (!(dec_fits && decode_full(p)))
    if (const int nb = gemv_nb(p)) return launch_gemv_w4a16(p, nb, stream);
  if (dec_fits) {
    const bool full = decode_full(p);
    const bool one = (k + 127) / 128 <= kDecWaves;
    p.scalar_scales = decode_scalar_scales(p, w2d, full) ? 1 : 0;
    if (full && one) launch_w4a16_t<true, 1>(p, w2d, stream);
    if (full && !one) launch_w4a16_t<true, 2>(p, w2d, stream);
    if (!full && one) launch_w4a16_t<false, 1>(p, w2d, stream);
    if (!full && !one) launch_w4a16_t<false, 2>(p, w2d, stream);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((n + 15) / 16);
  if (w2d)
    hipLaunchKernelGGL(k_gemm_w4a16_stream<true>, dim3(grid), dim3(kDecWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(k_gemm_w4a16_stream<false>, dim3(grid), dim3(kDecWaves * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_small_m(const GemmOperand &a, const GemmOperand &w, int64_t m, int64_t n,
                               int64_t k, uint16_t *y, int64_t ld_y, hipStream_t stream) {
  SmallMArgs p;
  p.a = a;
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.scale_pairs = ((uintptr_t)a.scales % 2 == 0) && (a.ld_scales % 2 == 0) &&
                  ((uintptr_t)w.scales % 2 == 0) && (w.ld_scales % 2 == 0);
  p.scalar_scales = 0;
  p.a_bf16 = nullptr;
  p.ld_a = 0;
  p.aq_codes = p.aq_scales = nullptr;
  p.aq_gs = nullptr;
  const int64_t nbands = (n + 15) / 16;
  if ((k + 127) / 128 <= kDecWaves * kDecWin) {
    return launch_decode<false>(p, w.block_rows == 16, stream);
  }
  const unsigned grid = (unsigned)nbands;
  if (w.block_rows == 16)
    hipLaunchKernelGGL(k_gemm_small_m<true>, dim3(grid), dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_gemm_small_m<false>, dim3(grid), dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmOperand &a, const int32_t *row_index,
                               const int32_t *offsets, int32_t num_groups, const GemmOperand &w,
                               int64_t w_group_rows, int64_t n, int64_t k, int64_t total_rows,
                               uint16_t *y, int64_t ld_y, hipStream_t stream) {
  constexpr int FM = 2, FN = 4;
  GroupedArgs p;
  p.a = a;
  p.w = w;
  p.row_index = row_index;
  p.offsets = offsets;
  p.num_groups = num_groups;
  p.w_group_rows = w_group_rows;
  p.n = n;
  p.k = k;
  p.total_rows = total_rows;
  p.y = y;
  p.ld_y = ld_y;
  p.tiles_n = (int)((n + 64 * FN - 1) / (64 * FN));
  // Upper bound of the tile count: every group may add one partial m-tile.
  const int64_t max_tiles = ((total_rows + 64 * FM - 1) / (64 * FM) + num_groups) * p.tiles_n;
  const bool pipelined = k % 64 == 0 && aligned4(a.scales) && a.ld_scales % 4 == 0 &&
                         aligned4(w.scales) && w.ld_scales % 4 == 0;
  if (pipelined) {
    // Two 2-wave workgroups per CU walk the tile list.
    const int64_t slots = 2 * (int64_t)device_cus();
    const unsigned g = (unsigned)(max_tiles < slots ? (max_tiles < 1 ? 1 : max_tiles) : slots);
    if (w.block_rows == 16)
      hipLaunchKernelGGL((k_gemm_grouped_lds<true>), dim3(g), dim3(128), 0, stream, p);
    else
      hipLaunchKernelGGL((k_gemm_grouped_lds<false>), dim3(g), dim3(128), 0, stream, p);
    return hipGetLastError();
  }
  int64_t grid = max_tiles < 1024 ? max_tiles : 1024;
  if (grid < 1) grid = 1;
  if (w.block_rows == 16)
    hipLaunchKernelGGL((k_gemm_grouped<FM, FN, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                       0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_grouped<FM, FN, false>), dim3((unsigned)grid), dim3(kGemmThreads),
                       0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
