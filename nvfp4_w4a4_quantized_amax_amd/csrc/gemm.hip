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
#include <stddef.h>

#include "nvfp4_device.hpp"
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
};

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

template <int FM, int FN, bool W2D>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_tile(DenseArgs p) {
  constexpr int BM = 64 * FM, BN = 64 * FN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;

  const int logical = xcd_logical(blockIdx.x, gridDim.x);
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
  floatx16_t acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) acc[f][g] = floatx16_t{};

  wave_tile_kloop<FM, FN>(a_row, a_srow, w_row, w_srow, p.k, kh, acc);

  const float alpha = (*p.a.gs) * (*p.w.gs);
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (row < p.m && col < p.n)
          p.y[row * p.ld_y + col] = (uint16_t)f32_to_bf16_rne(acc[f][g][r] * alpha);
      }
    }
}

// ---------------------------------------------------------------------------------------------
// Pipelined tile kernel (256 x 256 tiles, K a multiple of 64).  Packed codes and scales of each
// 64-wide K window travel HBM -> LDS with direct global-to-LDS loads (no registers), kStages
// windows deep; each wave then reads its fragments from LDS and decodes them in registers.
// Per stage: A and W codes [row][32 bytes], A scales [row][4 bytes], W scales [row or band][4].
// Every thread issues exactly kLoadsPerWindow load instructions per window, so the
// vector-memory counter tells each wave when a window has landed.
// ---------------------------------------------------------------------------------------------
constexpr int kStages = 4;
constexpr int kLoadsPerWindow = 6;

struct LdsStage {
  uint8_t a[256 * 32];
  uint8_t w[256 * 32];
  uint8_t as[256 * 4];
  uint8_t ws[256 * 4];
};

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

__device__ __forceinline__ void g2lds16(const uint8_t *g, void *l) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)l, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const uint8_t *g, void *l) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)l, 4, 0, 0);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_windows_left(int left) {
  // loads still allowed in flight: `left` later windows (0 .. kStages - 2)
  if (left >= 2) wait_vm<2 * kLoadsPerWindow>();
  else if (left == 1) wait_vm<kLoadsPerWindow>();
  else wait_vm<0>();
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// All fragments and scales of one window for one wave (4 A and 4 W fragments of 32 rows), read
// from LDS in one asm block that also waits for them: the compiler cannot tell these reads from
// the in-flight global-to-LDS loads of later stages and would otherwise wait for all of those.
// The outputs are early-clobber: a read in flight must not land in a later read's address.
// Fragment f of A is row (wm * 128 + f * 32 + lr), half kh: 1 KiB apart per f; its scale pair
// is 128 bytes apart per f.  W scale pairs (16x16 tiles) are 8 bytes apart per g.
template <bool W2D>
__device__ __forceinline__ void read_stage_frags(const LdsStage &S, int wm, int wn, int lr, int kh,
                                                 Frags<4, 4> &fr) {
  const uint32_t base = (uint32_t)(uintptr_t)&S;
  const uint32_t ra = wm * 128 + lr, rw = wn * 128 + lr;
  const uint32_t pa = base + offsetof(LdsStage, a) + (ra * 2 + kh) * 16;
  const uint32_t pw = base + offsetof(LdsStage, w) + (rw * 2 + kh) * 16;
  const uint32_t pas = base + offsetof(LdsStage, as) + ra * 4 + kh * 2;
  const uint32_t pws = base + offsetof(LdsStage, ws) +
                       (W2D ? (wn * 8 + (lr >> 4)) * 4 + kh * 2 : rw * 4 + kh * 2);
  u32x4_t a0, a1, a2, a3, w0, w1, w2, w3;
  uint32_t sa0, sa1, sa2, sa3, sw0, sw1, sw2, sw3;
  if (W2D) {
    asm volatile(
        "ds_read_b128 %0, %16\n"
        "ds_read_b128 %1, %16 offset:1024\n"
        "ds_read_b128 %2, %16 offset:2048\n"
        "ds_read_b128 %3, %16 offset:3072\n"
        "ds_read_b128 %4, %17\n"
        "ds_read_b128 %5, %17 offset:1024\n"
        "ds_read_b128 %6, %17 offset:2048\n"
        "ds_read_b128 %7, %17 offset:3072\n"
        "ds_read_u16 %8, %18\n"
        "ds_read_u16 %9, %18 offset:128\n"
        "ds_read_u16 %10, %18 offset:256\n"
        "ds_read_u16 %11, %18 offset:384\n"
        "ds_read_u16 %12, %19\n"
        "ds_read_u16 %13, %19 offset:8\n"
        "ds_read_u16 %14, %19 offset:16\n"
        "ds_read_u16 %15, %19 offset:24\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(w0), "=&v"(w1), "=&v"(w2),
          "=&v"(w3), "=&v"(sa0), "=&v"(sa1), "=&v"(sa2), "=&v"(sa3), "=&v"(sw0), "=&v"(sw1),
          "=&v"(sw2), "=&v"(sw3)
        : "v"(pa), "v"(pw), "v"(pas), "v"(pws)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %16\n"
        "ds_read_b128 %1, %16 offset:1024\n"
        "ds_read_b128 %2, %16 offset:2048\n"
        "ds_read_b128 %3, %16 offset:3072\n"
        "ds_read_b128 %4, %17\n"
        "ds_read_b128 %5, %17 offset:1024\n"
        "ds_read_b128 %6, %17 offset:2048\n"
        "ds_read_b128 %7, %17 offset:3072\n"
        "ds_read_u16 %8, %18\n"
        "ds_read_u16 %9, %18 offset:128\n"
        "ds_read_u16 %10, %18 offset:256\n"
        "ds_read_u16 %11, %18 offset:384\n"
        "ds_read_u16 %12, %19\n"
        "ds_read_u16 %13, %19 offset:128\n"
        "ds_read_u16 %14, %19 offset:256\n"
        "ds_read_u16 %15, %19 offset:384\n"
        "s_waitcnt lgkmcnt(0)\n"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(w0), "=&v"(w1), "=&v"(w2),
          "=&v"(w3), "=&v"(sa0), "=&v"(sa1), "=&v"(sa2), "=&v"(sa3), "=&v"(sw0), "=&v"(sw1),
          "=&v"(sw2), "=&v"(sw3)
        : "v"(pa), "v"(pw), "v"(pas), "v"(pws)
        : "memory");
  }
  fr.a[0] = make_uint4(a0[0], a0[1], a0[2], a0[3]);
  fr.a[1] = make_uint4(a1[0], a1[1], a1[2], a1[3]);
  fr.a[2] = make_uint4(a2[0], a2[1], a2[2], a2[3]);
  fr.a[3] = make_uint4(a3[0], a3[1], a3[2], a3[3]);
  fr.w[0] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
  fr.w[1] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
  fr.w[2] = make_uint4(w2[0], w2[1], w2[2], w2[3]);
  fr.w[3] = make_uint4(w3[0], w3[1], w3[2], w3[3]);
  fr.sa[0] = sa0; fr.sa[1] = sa1; fr.sa[2] = sa2; fr.sa[3] = sa3;
  fr.sw[0] = sw0; fr.sw[1] = sw1; fr.sw[2] = sw2; fr.sw[3] = sw3;
}

template <bool W2D>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_lds(DenseArgs p) {
  constexpr int FM = 4, FN = 4, BM = 256, BN = 256;
  static_assert(kStages == 4, "wait_windows_left assumes four stages");
  __shared__ LdsStage st[kStages];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, kh = lane >> 5;

  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int in_group = kGroupM * p.tiles_n;
  const int first_m = (logical / in_group) * kGroupM;
  const int gsz = min(p.tiles_m - first_m, kGroupM);
  const int tm = first_m + (logical % in_group) % gsz;
  const int tn = (logical % in_group) / gsz;
  const int64_t m_tile = (int64_t)tm * BM, n_tile = (int64_t)tn * BN;

  // This thread's share of every window's loads (rows clamped into the matrix; results of
  // clamped rows are never stored).
  const uint8_t *ga[2], *gw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = i * 256 + tid, row = c >> 1, half = c & 1;
    ga[i] = p.a.codes + min(m_tile + row, p.m - 1) * p.a.ld_codes + half * 16;
    gw[i] = p.w.codes + min(n_tile + row, p.n - 1) * p.w.ld_codes + half * 16;
  }
  const uint8_t *gas = p.a.scales + min(m_tile + tid, p.m - 1) * p.a.ld_scales;
  const uint8_t *gws = W2D ? p.w.scales + min(n_tile / 16 + (lane & 15), p.n / 16 - 1) * p.w.ld_scales
                           : p.w.scales + min(n_tile + tid, p.n - 1) * p.w.ld_scales;
  auto issue = [&](int64_t win, int s) {
    LdsStage &S = st[s];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      g2lds16(ga[i] + win * 32, S.a + (i * 256 + wave * 64) * 16);
      g2lds16(gw[i] + win * 32, S.w + (i * 256 + wave * 64) * 16);
    }
    g2lds4(gas + win * 4, S.as + wave * 64 * 4);
    if (W2D) {
      if (lane < 16) g2lds4(gws + win * 4, S.ws);  // every wave writes the same 64 bytes
    } else {
      g2lds4(gws + win * 4, S.ws + wave * 64 * 4);
    }
  };

  floatx16_t acc[FM][FN];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) acc[f][g] = floatx16_t{};

  const int64_t nwin = p.k / 64;
  for (int64_t w = 0; w < kStages - 1 && w < nwin; ++w) issue(w, (int)w);
  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t later = min((int64_t)kStages - 2, nwin - 1 - w);
    // This wave's loads of window w are done once at most `later` windows remain in flight;
    // the barrier then makes window w complete for every wave and frees stage (w - 1).
    // A plain s_barrier (no fence): the compiler's fence would wait for every load in flight.
    wait_windows_left((int)later);
    __builtin_amdgcn_s_barrier();
    if (w + kStages - 1 < nwin) issue(w + kStages - 1, (int)((w + kStages - 1) % kStages));
    Frags<FM, FN> fr;
    read_stage_frags<W2D>(st[w % kStages], wm, wn, lr, kh, fr);
    compute_window(fr, acc);
  }

  const float alpha = (*p.a.gs) * (*p.w.gs);
  const int64_t m0 = m_tile + wm * 32 * FM, n0 = n_tile + wn * 32 * FN;
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int g = 0; g < FN; ++g) {
      const int64_t col = n0 + g * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (row < p.m && col < p.n)
          p.y[row * p.ld_y + col] = (uint16_t)f32_to_bf16_rne(acc[f][g][r] * alpha);
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
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + f * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
          if (row < r_end && col < p.n)
            p.y[row * p.ld_y + col] = (uint16_t)f32_to_bf16_rne(acc[f][g][r] * alpha);
        }
      }
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
};

constexpr int kSmallMWin = 4;

template <bool W2D>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_small_m(SmallMArgs p) {
  __shared__ floatx4_t s_red[4][kWave];
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
      const uint32_t w0 = remb > 0 ? w_srow[win * 8] : 0u, w1 = remb > 1 ? w_srow[win * 8 + 1] : 0u;
      const uint32_t a0 = (a_ok && remb > 0) ? a_srow[win * 8] : 0u;
      const uint32_t a1 = (a_ok && remb > 1) ? a_srow[win * 8 + 1] : 0u;
      ws_[u] = w0 | (w1 << 8);
      as_[u] = a0 | (a1 << 8);
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
    const float alpha = (*p.a.gs) * (*p.w.gs);
    if (i16 < p.m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + 4 * q + r;
        if (n < p.n) p.y[(int64_t)i16 * p.ld_y + n] = (uint16_t)f32_to_bf16_rne(s[r] * alpha);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------------
template <int FM, int FN>
static hipError_t launch_tile_fm(const GemmOperand &a, const GemmOperand &w, int64_t m,
                                 int64_t n, int64_t k, uint16_t *y, int64_t ld_y,
                                 hipStream_t stream) {
  DenseArgs p;
  p.a = a;
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.tiles_m = (int)((m + 64 * FM - 1) / (64 * FM));
  p.tiles_n = (int)((n + 64 * FN - 1) / (64 * FN));
  const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
  if (w.block_rows == 16)
    hipLaunchKernelGGL((k_gemm_tile<FM, FN, true>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_tile<FM, FN, false>), dim3(grid), dim3(kGemmThreads), 0, stream,
                       p);
  return hipGetLastError();
}

static bool aligned4(const void *q) { return ((uintptr_t)q & 3u) == 0; }

hipError_t launch_gemm_tile(const GemmOperand &a, const GemmOperand &w, int64_t m, int64_t n,
                            int64_t k, uint16_t *y, int64_t ld_y, hipStream_t stream) {
  if (m <= 64) return launch_tile_fm<1, 4>(a, w, m, n, k, y, ld_y, stream);
  if (m <= 128) return launch_tile_fm<2, 4>(a, w, m, n, k, y, ld_y, stream);
  // The pipelined kernel needs whole 64-wide K windows and 4-byte aligned scale rows.
  const bool lds_ok = (k % 64 == 0) && aligned4(a.scales) && aligned4(w.scales) &&
                      (a.ld_scales % 4 == 0) && (w.ld_scales % 4 == 0);
  if (!lds_ok) return launch_tile_fm<4, 4>(a, w, m, n, k, y, ld_y, stream);
  DenseArgs p;
  p.a = a;
  p.w = w;
  p.m = m;
  p.n = n;
  p.k = k;
  p.y = y;
  p.ld_y = ld_y;
  p.tiles_m = (int)((m + 255) / 256);
  p.tiles_n = (int)((n + 255) / 256);
  const unsigned grid = (unsigned)p.tiles_m * (unsigned)p.tiles_n;
  if (w.block_rows == 16)
    hipLaunchKernelGGL(k_gemm_lds<true>, dim3(grid), dim3(kGemmThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(k_gemm_lds<false>, dim3(grid), dim3(kGemmThreads), 0, stream, p);
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
  const unsigned grid = (unsigned)((n + 15) / 16);
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
