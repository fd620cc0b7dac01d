// NVFP4 dynamic quantization kernels for gfx950.
//
// Pass 1 (k_amax): streaming read of the bf16 tensor, |x| max on the bit patterns (exact and
// order independent); each workgroup stores its partial maximum in a workspace slot.  No
// device-scope atomics: on MI355X they are resolved past the per-XCD L2s and serialize.
// Pass 2 (k_encode_1d / k_encode_2d): every workgroup reduces the slots, derives the FP32 global
// scale, builds the per-tensor tables in LDS (block-scale thresholds and element multipliers, see
// nvfp4_device.hpp), then re-reads its share of the tensor, fits each block's E4M3 scale and
// writes packed codes and scales.
//
// Work layout: the tensor is cut into 2 KiB tiles (64 blocks of 16 bf16, one block per lane).
// Tile t belongs to wave slot t mod (4 * grid) of both passes, so at any moment the whole chip streams one contiguous
// region, and tile t is read by the same XCD in both passes (workgroup b runs on XCD b mod 8 and
// owns tiles with (t / 4) mod 8 == b mod 8 for any grid that is a multiple of 8).  Pass 2 walks
// the tiles in the reverse order, so it starts with the data pass 1 read last (still in L2).
// Small tensors use k_quantize_small: one workgroup runs both passes with an LDS barrier.
//
// The format steps follow "NVFP4 Explained: NVIDIA's 4-Bit Format for Faster AI Inference"
// ("How NVFP4 Represents a Value") and "What is NVFP4? 4-bit AI inference on NVIDIA Blackwell
// explained" ("What does NVFP4 mean?", "Why does scaling matter so much?").
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "nvfp4_device.hpp"
#include "launch.hpp"

namespace nvfp4 {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / kWave;
constexpr int kTileBlocks = 64;  // one wave step: 64 blocks of 16 bf16 = 2 KiB, one block per lane
constexpr int kAmaxUnroll = 4;   // tiles in flight per wave in pass 1 (8 x 16 B per lane)

// Block b (16 bf16 values) -> uint4 index of its first half in x.
template <bool CONTIG>
__device__ __forceinline__ size_t block_index(uint32_t b, FastDiv bpr, int64_t ld_x8) {
  if (CONTIG) return (size_t)b * 2u;
  uint32_t r = fdiv(b, bpr);
  uint32_t cb = b - r * bpr.d;
  return (size_t)r * (size_t)ld_x8 + (size_t)cb * 2u;
}

// ---------------------------------------------------------------------------------------------
// Pass 1
// ---------------------------------------------------------------------------------------------
template <bool CONTIG>
__global__ __launch_bounds__(kQThreads) void k_amax(const uint4 *__restrict__ x, uint32_t n_blocks,
                                                    FastDiv bpr, int64_t ld_x8,
                                                    uint32_t *__restrict__ slots) {
  __shared__ uint32_t red[kQWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t S = gridDim.x * kQWaves;  // tiles between two visits of one wave
  const uint32_t n_full = n_blocks / kTileBlocks;
  const uint32_t n_tiles = (n_blocks + kTileBlocks - 1) / kTileBlocks;
  uint32_t m = 0;
  uint32_t t = blockIdx.x * kQWaves + wave;
  for (; t + (kAmaxUnroll - 1) * S < n_full; t += kAmaxUnroll * S) {
    uint4 v[2 * kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const size_t i = block_index<CONTIG>((t + u * S) * kTileBlocks + lane, bpr, ld_x8);
      v[2 * u] = x[i];
      v[2 * u + 1] = x[i + 1];
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = max(m, absmax16(v[2 * u], v[2 * u + 1]));
  }
  for (; t < n_tiles; t += S) {
    const uint32_t b = t * kTileBlocks + lane;
    if (b < n_blocks) {
      const size_t i = block_index<CONTIG>(b, bpr, ld_x8);
      m = max(m, absmax16(x[i], x[i + 1]));
    }
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) slots[blockIdx.x] = m;
}

// Prologue of every encode workgroup: global amax from the slots, FP32 global scale, tables.
__device__ __forceinline__ float tables_from_slots(const uint32_t *__restrict__ slots, int n_slots,
                                                   QuantTables &tab,
                                                   uint32_t *red, float *__restrict__ gs_out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n_slots; i += blockDim.x) m = max(m, slots[i]);
  m = block_max_u32(m, red);
  const float gs = global_scale_from_amax_bits(m);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  build_tables(tab, gs);
  return gs;
}

// ---------------------------------------------------------------------------------------------
// Pass 2, 1D blocks: one lane per 16-value block (two 16-byte loads, one 8-byte code store, one
// scale byte).
// ---------------------------------------------------------------------------------------------
struct EncOut {
  uint8_t *codes;
  int64_t ld_codes;
  uint8_t *scales;
  int64_t ld_scales;
};

// Encode one block whose |max| bf16 pattern `bam` is already known; `code_of(bam, &k)` gives
// its scale code and element multiplier (the table search or the direct lookup).
template <bool CONTIG, class CodeOf>
__device__ __forceinline__ void encode_block_1d_with(const uint4 &a, const uint4 &b, uint32_t bam,
                                                     uint32_t blk, FastDiv bpr, const EncOut &o,
                                                     float gs, CodeOf code_of) {
  float k;
  const int code = code_of(bam, &k);
  const uint2 packed = encode16(a, b, k, code, gs);
  size_t co, so;
  if (CONTIG) {
    co = (size_t)blk * 8u;
    so = (size_t)blk;
  } else {
    const uint32_t r = fdiv(blk, bpr);
    const uint32_t cb = blk - r * bpr.d;
    co = (size_t)r * (size_t)o.ld_codes + (size_t)cb * 8u;
    so = (size_t)r * (size_t)o.ld_scales + (size_t)cb;
  }
  ntstore8(o.codes + co, packed);
  ntstore_u8(o.scales + so, (uint32_t)code);
}

template <bool CONTIG>
__device__ __forceinline__ void encode_block_1d_bam(const uint4 &a, const uint4 &b, uint32_t bam,
                                                    uint32_t blk, FastDiv bpr, const EncOut &o,
                                                    const QuantTables &tab, float inv6gs,
                                                    float gs) {
  encode_block_1d_with<CONTIG>(a, b, bam, blk, bpr, o, gs, [&](uint32_t m, float *k) {
    return scale_code(m, tab, inv6gs, k);
  });
}

template <bool CONTIG>
__device__ __forceinline__ void encode_block_1d(const uint4 &a, const uint4 &b, uint32_t blk,
                                                FastDiv bpr, const EncOut &o,
                                                const QuantTables &tab) {
  encode_block_1d_bam<CONTIG>(a, b, absmax16(a, b), blk, bpr, o, tab, tab.inv6gs, tab.gs);
}

template <bool CONTIG>
__global__ __launch_bounds__(kQThreads) void k_encode_1d(const uint4 *__restrict__ x,
                                                         uint32_t n_blocks, FastDiv bpr,
                                                         int64_t ld_x8, EncOut o,
                                                         const uint32_t *__restrict__ slots,
                                                         int n_slots, float *__restrict__ gs_out) {
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kQWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t S = gridDim.x * kQWaves;
  const uint32_t n_tiles = (n_blocks + kTileBlocks - 1) / kTileBlocks;
  const uint32_t first = blockIdx.x * kQWaves + wave;
  // This wave's tiles are first + i * S, i = 0 .. cnt - 1; they are walked from the last, two
  // at a time (four 16-byte loads in flight per lane).  Only the last tile of all can be partial.
  const uint32_t cnt = first < n_tiles ? (n_tiles - first + S - 1) / S : 0u;
  // The slot loads go out first, then the loads of the first two tiles: the tiles do not
  // depend on the global scale, so they are in flight while the slots are reduced and the tables
  // are built (loads complete in order, so waiting for the slots does not wait for the tiles,
  // and the barriers below wait for LDS work only).
  // Every load below is unconditional (indices clamped into range; max is idempotent and the
  // clamped tile loads are never used), so the compiler can wait for the slots alone.
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kMaxAmaxSlots / kQThreads; ++j)
    m = max(m, slots[min(j * kQThreads + (int)threadIdx.x, n_slots - 1)]);
  int32_t i = (int32_t)cnt - 1;
  const uint32_t ba0 = (first + (uint32_t)max(i, 0) * S) * kTileBlocks + lane;
  const bool va = i >= 0 && ba0 < n_blocks;
  const bool vb = i >= 1;
  const uint32_t bb0 = vb ? ba0 - S * kTileBlocks : 0u;
  const size_t ia0 = block_index<CONTIG>(va ? ba0 : 0u, bpr, ld_x8);
  const size_t ib0 = block_index<CONTIG>(bb0, bpr, ld_x8);
  uint4 a0 = x[ia0], a1 = x[ia0 + 1];
  uint4 b0 = x[ib0], b1 = x[ib0 + 1];
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int w = 0; w < kQWaves; ++w) m = max(m, red[w]);
  const float gs = global_scale_from_amax_bits(m);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  build_tables<true>(tab, gs);
  if (va) encode_block_1d<CONTIG>(a0, a1, ba0, bpr, o, tab);
  if (vb) encode_block_1d<CONTIG>(b0, b1, bb0, bpr, o, tab);
  for (i -= 2; i >= 1; i -= 2) {
    const uint32_t ba = (first + (uint32_t)i * S) * kTileBlocks + lane;
    const uint32_t bb = ba - S * kTileBlocks;
    const size_t ia = block_index<CONTIG>(ba, bpr, ld_x8);  // not the last tile: whole
    a0 = x[ia];
    a1 = x[ia + 1];
    const size_t ib = block_index<CONTIG>(bb, bpr, ld_x8);
    b0 = x[ib];
    b1 = x[ib + 1];
    encode_block_1d<CONTIG>(a0, a1, ba, bpr, o, tab);
    encode_block_1d<CONTIG>(b0, b1, bb, bpr, o, tab);
  }
  if (i == 0) {  // a whole tile: the wave has at least three
    const uint32_t ba = first * kTileBlocks + lane;
    const size_t ia = block_index<CONTIG>(ba, bpr, ld_x8);
    encode_block_1d<CONTIG>(x[ia], x[ia + 1], ba, bpr, o, tab);
  }
}

// ---------------------------------------------------------------------------------------------
// Single-read path: one persistent workgroup per CU (all of them resident at once when nothing
// else occupies the device).  Phase 1 reads each wave's tiles once,
// keeping the first RT of them in registers and the next LT in LDS, and publishes the
// workgroup's partial max.  A grid barrier without read-modify-write atomics follows: every
// workgroup stores (epoch << 16 | max) into its own 64-bit slot, and one wave per workgroup polls
// all slots until every slot carries this call's epoch (a per-call 48-bit number, so stale slots
// never match).  The poll is bounded (spin_limit rounds); a workgroup whose poll runs out
// (possible only if the workgroups were not all resident, e.g. next to other work on the
// device) computes the global maximum itself by reading the whole tensor, so the result is the
// same either way, and counts itself in the status word.  Phase 2 builds the tables and
// encodes the resident tiles without touching memory again; tiles beyond RT + LT per wave are
// read a second time.
// ---------------------------------------------------------------------------------------------
constexpr uint32_t kSpinLimit = 1u << 20;

template <int WAVES, int RT, int LT, bool CONTIG>
__global__ __launch_bounds__(WAVES * 64, 1) void k_quantize_persistent(
    const uint4 *__restrict__ x, uint32_t n_blocks, FastDiv bpr, int64_t ld_x8, EncOut o,
    unsigned long long *__restrict__ slots, unsigned long long epoch, uint32_t spin_limit,
    float *__restrict__ gs_out, uint32_t *__restrict__ status) {
  __shared__ QuantTables tab;
  __shared__ CodeLut lut;
  __shared__ uint32_t red[WAVES];
  __shared__ uint32_t s_amax, s_done;
  // LDS-resident tiles: [tile][half][wave][lane], one 16-byte half-block per lane, and each
  // block's |max| pattern (found in phase 1, used again in phase 2).
  __shared__ uint4 s_tiles[LT * 2 * WAVES][kWave];
  __shared__ uint16_t s_bam[LT * WAVES][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t S = gridDim.x * WAVES;
  const uint32_t n_tiles = (n_blocks + kTileBlocks - 1) / kTileBlocks;
  const uint32_t first = blockIdx.x * WAVES + wave;
  const uint32_t cnt = first < n_tiles ? (n_tiles - first + S - 1) / S : 0u;
  // The wave's i-th tile is first + i * S: i < LT live in LDS, LT <= i < LT + RT in registers,
  // the rest (overflow) are read in both phases.
  auto tile_block = [&](uint32_t i) { return (first + i * S) * kTileBlocks + lane; };
  uint32_t m = 0;

  // Phase 1a: LDS tiles, staged through registers in batches of kLdsBatch tiles.
  constexpr int kLdsBatch = (LT % 4 == 0) ? 4 : 3;
  static_assert(LT % kLdsBatch == 0, "LDS tiles come in whole batches");
#pragma unroll 1
  for (int i0 = 0; i0 < LT; i0 += kLdsBatch) {
    uint4 t[2 * kLdsBatch];
#pragma unroll
    for (int u = 0; u < kLdsBatch; ++u) {
      uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
      const uint32_t b = tile_block(i0 + u);
      if ((uint32_t)(i0 + u) < cnt && b < n_blocks) {
        const size_t idx = block_index<CONTIG>(b, bpr, ld_x8);
        lo = ntload16(x + idx);
        hi = ntload16(x + idx + 1);
      }
      t[2 * u] = lo;
      t[2 * u + 1] = hi;
    }
#pragma unroll
    for (int u = 0; u < kLdsBatch; ++u) {
      const uint32_t bm = absmax16(t[2 * u], t[2 * u + 1]);
      m = max(m, bm);
      s_bam[(i0 + u) * WAVES + wave][lane] = (uint16_t)bm;
      s_tiles[(2 * (i0 + u)) * WAVES + wave][lane] = t[2 * u];
      s_tiles[(2 * (i0 + u) + 1) * WAVES + wave][lane] = t[2 * u + 1];
    }
  }
  // Phase 1b: register tiles (all loads issued before any is used), then the overflow tiles.
  uint4 reg[2 * RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    const uint32_t b = tile_block(LT + i);
    if ((uint32_t)(LT + i) < cnt && b < n_blocks) {
      const size_t idx = block_index<CONTIG>(b, bpr, ld_x8);
      lo = ntload16(x + idx);
      hi = ntload16(x + idx + 1);
    }
    reg[2 * i] = lo;
    reg[2 * i + 1] = hi;
  }
  for (uint32_t i = LT + RT; i < cnt; ++i) {
    const uint32_t b = tile_block(i);
    if (b < n_blocks) {
      const size_t idx = block_index<CONTIG>(b, bpr, ld_x8);
      m = max(m, absmax16(x[idx], x[idx + 1]));
    }
  }
  // Block maxima of the register tiles, two 16-bit patterns per register.
  uint32_t bamr[(RT + 1) / 2];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const uint32_t bm = absmax16(reg[2 * i], reg[2 * i + 1]);
    m = max(m, bm);
    if (i % 2 == 0) bamr[i / 2] = bm;
    else bamr[i / 2] |= bm << 16;
  }
  m = block_max_u32(m, red);

  // Grid barrier on per-workgroup slots.  A slot carries its own payload (the partial max), so
  // neither the store nor the polls need to order any other memory: relaxed device-coherent
  // accesses suffice (a release here would force an L2 write-back).
  const unsigned long long tag = (epoch & 0xFFFFFFFFFFFFull) << 16;
  if (threadIdx.x == 0)
    __hip_atomic_store(slots + blockIdx.x, tag | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wave == 0) {
    uint32_t mx = 0;
    bool done = false;
    // Relaxed device-coherent polls until every slot carries this call's epoch.  Lane l watches
    // slots l, l + 64, ...; each round issues all of its loads at once and reloads only the
    // slots it has not yet seen, so the polls put little load on the few lines they share with
    // every other workgroup.
    constexpr int kPoll = (kMaxPersistentSlots + kWave - 1) / kWave;
    uint32_t pending = 0, lm = 0;
#pragma unroll
    for (int r = 0; r < kPoll; ++r)
      if (lane + kWave * r < (int)gridDim.x) pending |= 1u << r;
    for (uint32_t it = 0; it < spin_limit && !done; ++it) {
      unsigned long long v[kPoll];
#pragma unroll
      for (int r = 0; r < kPoll; ++r)
        v[r] = ((pending >> r) & 1u)
                   ? __hip_atomic_load(slots + lane + kWave * r, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0ull;
#pragma unroll
      for (int r = 0; r < kPoll; ++r) {
        if (((pending >> r) & 1u) && (v[r] & ~0xFFFFull) == tag) {
          lm = max(lm, (uint32_t)(v[r] & 0xFFFFu));
          pending &= ~(1u << r);
        }
      }
      if (__all(pending == 0)) {
        mx = wave_max_u32(lm);
        done = true;
      } else {
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (lane == 0) {
      s_amax = mx;
      s_done = done ? 1u : 0u;
    }
  }
  __syncthreads();
  if (s_done == 0u) {
    // The barrier did not complete: read the whole tensor for the global maximum (uniform
    // branch: every thread of the workgroup takes it).
    uint32_t mm = 0;
    for (uint32_t b = threadIdx.x; b < n_blocks; b += WAVES * 64) {
      const size_t idx = block_index<CONTIG>(b, bpr, ld_x8);
      mm = max(mm, absmax16(x[idx], x[idx + 1]));
    }
    mm = block_max_u32(mm, red);
    if (threadIdx.x == 0) {
      s_amax = mm;
      atomicAdd(status, 1u);
    }
    __syncthreads();
  }
  const float gs = global_scale_from_amax_bits(s_amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *gs_out = gs;
  build_tables(tab, gs);
  build_code_lut(lut, tab);
  const int32_t lut_off = __builtin_amdgcn_readfirstlane(lut.off);
  const int32_t lut_top = __builtin_amdgcn_readfirstlane(lut.top);

  // Phase 2: encode the register tiles; each freed register pair immediately starts the re-read
  // of one overflow tile.  Then the LDS tiles, then the prefetched overflow tiles; any further
  // tiles are re-read and encoded one by one.  Block scales come from the direct lookup table.
  auto phase2 = [&](auto code_of) {
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const uint32_t b = tile_block(LT + i);
      if ((uint32_t)(LT + i) < cnt && b < n_blocks)
        encode_block_1d_with<CONTIG>(reg[2 * i], reg[2 * i + 1],
                                     (i % 2 == 0) ? (bamr[i / 2] & 0xFFFFu) : (bamr[i / 2] >> 16),
                                     b, bpr, o, gs, code_of);
      const uint32_t b2 = tile_block(LT + RT + i);
      if ((uint32_t)(LT + RT + i) < cnt && b2 < n_blocks) {
        const size_t idx = block_index<CONTIG>(b2, bpr, ld_x8);
        reg[2 * i] = x[idx];
        reg[2 * i + 1] = x[idx + 1];
      }
    }
#pragma unroll 2
    for (int i = 0; i < LT; ++i) {
      const uint32_t b = tile_block(i);
      if ((uint32_t)i < cnt && b < n_blocks)
        encode_block_1d_with<CONTIG>(s_tiles[(2 * i) * WAVES + wave][lane],
                                     s_tiles[(2 * i + 1) * WAVES + wave][lane],
                                     s_bam[i * WAVES + wave][lane], b, bpr, o, gs, code_of);
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const uint32_t b = tile_block(LT + RT + i);
      if ((uint32_t)(LT + RT + i) < cnt && b < n_blocks)
        encode_block_1d_with<CONTIG>(reg[2 * i], reg[2 * i + 1],
                                     absmax16(reg[2 * i], reg[2 * i + 1]), b, bpr, o, gs, code_of);
    }
    for (uint32_t i = LT + 2 * RT; i < cnt; ++i) {
      const uint32_t b = tile_block(i);
      if (b < n_blocks) {
        const size_t idx = block_index<CONTIG>(b, bpr, ld_x8);
        const uint4 a0 = x[idx], a1 = x[idx + 1];
        encode_block_1d_with<CONTIG>(a0, a1, absmax16(a0, a1), b, bpr, o, gs, code_of);
      }
    }
  };
  phase2([&](uint32_t m, float *k) { return lut_code(m, lut, lut_off, lut_top, k); });
}

// ---------------------------------------------------------------------------------------------
// Pass 2, 16x16 tiles.  A wave covers 4 horizontally adjacent tiles of one 16-row band: lane l
// holds row l % 16 of tile l / 16 (32 bytes = 16 values); the tile maximum is a 16-lane
// butterfly.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kQThreads) void k_encode_2d(const uint16_t *__restrict__ w,
                                                         int64_t rows, int64_t cols, int64_t ld_w,
                                                         EncOut o,
                                                         const uint32_t *__restrict__ slots,
                                                         int n_slots, float *__restrict__ gs_out) {
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kQWaves];
  tables_from_slots(slots, n_slots, tab, red, gs_out);
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
    float k;
    const int code = scale_code(m, tab, &k);
    const uint2 packed = encode16(v0, v1, k, code, tab.gs);
    ntstore8(o.codes + (band * 16 + r) * o.ld_codes + tc * 8, packed);
    if (r == 0) ntstore_u8(o.scales + band * o.ld_scales + tc, (uint32_t)code);
  }
}

// ---------------------------------------------------------------------------------------------
// Small tensors: one workgroup of 1024 threads runs both passes; tables live in LDS.
// ---------------------------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;

__global__ __launch_bounds__(kSmallThreads) void k_quantize_small(const uint16_t *__restrict__ x,
                                                                  int32_t rows, int32_t cols,
                                                                  int64_t ld_x, EncOut o,
                                                                  float *__restrict__ gs_out) {
  __shared__ QuantTables tab;
  __shared__ uint32_t red[kSmallThreads / kWave];
  const int cpr = cols / 8;
  const int n_chunks = rows * cpr;
  uint32_t m = 0;
  for (int c = threadIdx.x; c < n_chunks; c += kSmallThreads) {
    const int r = c / cpr, c8 = c - r * cpr;
    m = max(m, absmax8(*(const uint4 *)(x + (int64_t)r * ld_x + c8 * 8)));
  }
  m = block_max_u32(m, red);
  const float gs = global_scale_from_amax_bits(m);
  if (threadIdx.x == 0) *gs_out = gs;
  build_tables(tab, gs);
  // One lane per 16-value block.
  const int bpr = cols / 16;
  const int n_blocks = rows * bpr;
  for (int blk = threadIdx.x; blk < n_blocks; blk += kSmallThreads) {
    const int r = blk / bpr, cb = blk - r * bpr;
    const uint4 *p = (const uint4 *)(x + (int64_t)r * ld_x + cb * 16);
    const uint4 v0 = p[0], v1 = p[1];
    float k;
    const int code = scale_code(absmax16(v0, v1), tab, &k);
    const uint2 packed = encode16(v0, v1, k, code, tab.gs);
    ntstore8(o.codes + (int64_t)r * o.ld_codes + cb * 8, packed);
    ntstore_u8(o.scales + (int64_t)r * o.ld_scales + cb, (uint32_t)code);
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

// Grid of both passes: a multiple of 8 (one share per XCD), at most one tile per wave slot.
static int quant_grid(uint32_t n_tiles, int max_wgs) {
  int g = (int)((n_tiles + kQWaves - 1) / kQWaves);
  g = (g + 7) / 8 * 8;
  return g < max_wgs ? (g < 8 ? 8 : g) : max_wgs;
}

constexpr int kAmaxWgs = 512;    // two 4-wave workgroups per CU, four 2 KiB tiles in flight each
constexpr int kEncodeWgs = 1024;

hipError_t launch_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, bool two_d,
                           uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                           float *gs_out, void *ws, hipStream_t stream) {
  const uint32_t bpr = (uint32_t)(cols / 16);
  const uint32_t n_blocks = (uint32_t)(rows * (cols / 16));
  const uint32_t n_tiles = (n_blocks + kTileBlocks - 1) / kTileBlocks;
  const FastDiv f = make_fastdiv(bpr);
  const bool contig_in = (ld_x == cols);
  uint32_t *slots = (uint32_t *)ws;
  const int ga = quant_grid(n_tiles, kAmaxWgs);
  static_assert(kAmaxWgs <= kMaxAmaxSlots, "slot array too small");
  if (contig_in)
    hipLaunchKernelGGL(k_amax<true>, dim3(ga), dim3(kQThreads), 0, stream, (const uint4 *)x,
                       n_blocks, f, ld_x / 8, slots);
  else
    hipLaunchKernelGGL(k_amax<false>, dim3(ga), dim3(kQThreads), 0, stream, (const uint4 *)x,
                       n_blocks, f, ld_x / 8, slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const EncOut o{codes, ld_codes, scales, ld_scales};
  if (two_d) {
    const int64_t groups = (rows / 16) * ((cols / 16 + 3) / 4);
    int64_t g = (groups + kQWaves - 1) / kQWaves;
    g = g < kEncodeWgs ? (g < 1 ? 1 : g) : kEncodeWgs;
    hipLaunchKernelGGL(k_encode_2d, dim3((unsigned)g), dim3(kQThreads), 0, stream,
                       (const uint16_t *)x, rows, cols, ld_x, o, slots, ga, gs_out);
    return hipGetLastError();
  }
  const int ge = quant_grid(n_tiles, kEncodeWgs);
  const bool contig = contig_in && (ld_codes == cols / 2) && (ld_scales == cols / 16);
  if (contig)
    hipLaunchKernelGGL(k_encode_1d<true>, dim3(ge), dim3(kQThreads), 0, stream, (const uint4 *)x,
                       n_blocks, f, ld_x / 8, o, slots, ga, gs_out);
  else
    hipLaunchKernelGGL(k_encode_1d<false>, dim3(ge), dim3(kQThreads), 0, stream,
                       (const uint4 *)x, n_blocks, f, ld_x / 8, o, slots, ga, gs_out);
  return hipGetLastError();
}

// Persistent single-read launch (one workgroup per CU).  Returns hipErrorNotSupported, having
// launched nothing, when the device cannot hold one such workgroup per CU, the path is turned
// off or the stream is being captured, so the caller can use the two-kernel path.
// 16 waves per CU; each wave keeps RT tiles in registers (8 VGPRs each) and LT tiles in LDS
// (16 waves x 4 x 2 KiB = 128 KiB).  An 8192 x 8192 bf16 tensor is 16 tiles per wave, so 12 of
// them are read only once.  (Holding every tile needs 8 waves per CU, which leaves the encode
// phase too few waves to hide its latencies: slower overall.)
constexpr int kPWaves = 16;
constexpr int kPResidentC = 8, kPLdsC = 4;
constexpr int kPResidentS = 8, kPLdsS = 4;
#define K_PERSISTENT_C k_quantize_persistent<kPWaves, kPResidentC, kPLdsC, true>
#define K_PERSISTENT_S k_quantize_persistent<kPWaves, kPResidentS, kPLdsS, false>

// How the single-read kernel is started, chosen once per process by NVFP4_QUANT_PATH (a switch
// for measurement and tests).  By default it is an ordinary launch: one workgroup per CU fits
// (the occupancy query says so), so all of them are resident whenever nothing else occupies the
// device, and a workgroup whose bounded barrier runs out still computes the right maximum.
// "cooperative" starts it with HIP's cooperative launch, which guarantees co-residency (on the
// MI355X measured here that call ended in the two-kernel form, 55 us per 8192 x 8192 call
// against 38 us); "two_pass" turns the single-read path off.  NVFP4_QUANT_SPIN_LIMIT overrides
// the barrier's poll bound (a test switch: 0 makes every workgroup take the whole-tensor
// maximum of a barrier that did not complete).
enum class QuantLaunch { kCooperative, kPlain, kOff };

struct DeviceInfo {
  int cus = 0;
  bool coop = false;
  QuantLaunch mode = QuantLaunch::kPlain;
  uint32_t spin_limit = kSpinLimit;
  int fits_contig = 0, fits_strided = 0;
};

static DeviceInfo device_info() {
  static std::mutex mu;
  static DeviceInfo cache[64];
  static bool known[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{};
  std::lock_guard<std::mutex> lock(mu);
  if (!known[dev]) {
    DeviceInfo d;
    int coop = 0;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess) {
      d.coop = coop != 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &d.fits_contig, (const void *)K_PERSISTENT_C,
              kPWaves * 64, 0) != hipSuccess)
        d.fits_contig = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &d.fits_strided, (const void *)K_PERSISTENT_S,
              kPWaves * 64, 0) != hipSuccess)
        d.fits_strided = 0;
    }
    (void)hipGetLastError();
    const char *path = getenv("NVFP4_QUANT_PATH");
    if (path && strcmp(path, "two_pass") == 0) d.mode = QuantLaunch::kOff;
    if (path && strcmp(path, "cooperative") == 0) d.mode = QuantLaunch::kCooperative;
    if (d.mode == QuantLaunch::kCooperative && !d.coop) d.mode = QuantLaunch::kOff;
    const char *spin = getenv("NVFP4_QUANT_SPIN_LIMIT");
    if (spin && *spin) d.spin_limit = (uint32_t)strtoul(spin, nullptr, 10);
    cache[dev] = d;
    known[dev] = true;
  }
  return cache[dev];
}

// Per-call barrier epochs.  They start from an unpredictable 48-bit value, so that slots left in
// a reused workspace by an earlier process never carry a current epoch; the counter is a
// function-local static, whose one-time initialization is thread-safe, so concurrent first calls
// cannot see it before it is seeded.
static unsigned long long initial_epoch() {
  static int anchor;
  const unsigned long long seed =
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() ^
      ((unsigned long long)getpid() << 32) ^ (unsigned long long)(uintptr_t)&anchor;
  // the SplitMix64 finalizer, a published 64-bit mixing function
  unsigned long long z = seed + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static unsigned long long next_epoch() {
  static std::atomic<unsigned long long> counter{initial_epoch()};
  unsigned long long e;
  do {  // epoch 0 would match the zeros of freshly cleared memory
    e = (counter.fetch_add(1) + 1) & 0xFFFFFFFFFFFFull;
  } while (e == 0);
  return e;
}

hipError_t launch_quantize_persistent(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                      uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                                      int64_t ld_scales, float *gs_out, void *ws,
                                      hipStream_t stream) {
  const DeviceInfo d = device_info();
  const bool contig = (ld_x == cols) && (ld_codes == cols / 2) && (ld_scales == cols / 16);
  const int fits = contig ? d.fits_contig : d.fits_strided;
  if (d.mode == QuantLaunch::kOff || d.cus <= 0 || fits < 1 || d.cus > kMaxPersistentSlots)
    return hipErrorNotSupported;
  // A stream being captured into a graph would freeze this call's epoch into the graph, and
  // every replay after the first would find all slots already carrying it and pass the barrier
  // on stale maxima: captured calls take the two-kernel path, which has no grid barrier.  (A
  // failed query, which can leave an error behind, is treated the same way.)
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
    (void)hipGetLastError();
    return hipErrorNotSupported;
  }
  if (capture != hipStreamCaptureStatusNone) return hipErrorNotSupported;
  const uint32_t bpr = (uint32_t)(cols / 16);
  uint32_t n_blocks = (uint32_t)(rows * (cols / 16));
  FastDiv f = make_fastdiv(bpr);
  int64_t ld_x8 = ld_x / 8;
  EncOut o{codes, ld_codes, scales, ld_scales};
  unsigned long long *slots = (unsigned long long *)((uint8_t *)ws + kPersistentSlotOffset);
  unsigned long long epoch = next_epoch();
  uint32_t *status = (uint32_t *)((uint8_t *)ws + kPersistentStatusOffset);
  uint32_t spin = d.spin_limit;
  const uint4 *xp = (const uint4 *)x;
  void *args[] = {(void *)&xp, (void *)&n_blocks, (void *)&f, (void *)&ld_x8, (void *)&o,
                  (void *)&slots, (void *)&epoch, (void *)&spin, (void *)&gs_out,
                  (void *)&status};
  const void *fn = contig ? (const void *)K_PERSISTENT_C : (const void *)K_PERSISTENT_S;
  if (d.mode == QuantLaunch::kCooperative) {
    if (hipLaunchCooperativeKernel(fn, dim3(d.cus), dim3(kPWaves * 64), args, 0, stream) ==
        hipSuccess)
      return hipSuccess;
    // The cooperative launch was refused (nothing ran): clear the error and let the caller take
    // the two-kernel path.
    (void)hipGetLastError();
    return hipErrorNotSupported;
  }
  // Plain launch: the occupancy check above guarantees one workgroup per CU fits, so on a device
  // that is not running other work all of them are resident at once; if they ever are not, the
  // workgroups whose bounded barrier runs out read the whole tensor for the maximum.
  if (contig)
    hipLaunchKernelGGL((K_PERSISTENT_C), dim3(d.cus), dim3(kPWaves * 64), 0, stream, xp, n_blocks,
                       f, ld_x8, o, slots, epoch, spin, gs_out, status);
  else
    hipLaunchKernelGGL((K_PERSISTENT_S), dim3(d.cus), dim3(kPWaves * 64), 0, stream, xp, n_blocks,
                       f, ld_x8, o, slots, epoch, spin, gs_out, status);
  return hipGetLastError();
}

hipError_t launch_quantize_small(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                                 int64_t ld_scales, float *gs_out, hipStream_t stream) {
  const EncOut o{codes, ld_codes, scales, ld_scales};
  hipLaunchKernelGGL(k_quantize_small, dim3(1), dim3(kSmallThreads), 0, stream,
                     (const uint16_t *)x, (int32_t)rows, (int32_t)cols, ld_x, o, gs_out);
  return hipGetLastError();
}

}  // namespace nvfp4
