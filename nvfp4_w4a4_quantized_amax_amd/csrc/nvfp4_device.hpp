// Device-side building blocks shared by the libnvfp4 kernels (gfx950 / CDNA4, wave64).
//
// Format (see include/nvfp4.h for the full statement and the pages it follows):
//   E2M1 codes, OCP E4M3 block scales (1D: 16 consecutive values, 2D: 16x16 tile), FP32 global
//   scale gs = RN_fp32(amax / 2688); reconstruction = code value * block scale * gs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kE4M3MaxCode = 0x7E;  // 448

// ---------------------------------------------------------------------------------------------
// Per-tensor tables, rebuilt from the global scale by every workgroup that encodes.
// ---------------------------------------------------------------------------------------------
struct QuantTables {
  float gs;       // FP32 global scale
  float inv6gs;   // approx 1 / (6 gs), only used to guess a block-scale code
  float pad[2];
  // ent[c], c = 0..127, everything a block whose guessed scale code is c needs, in one 16-byte
  // read:
  //   x = thresh[c + 1], thresh[s] (s = 1..126) being the smallest bf16 magnitude pattern whose
  //       block scale code is >= s (thresh[127] = 0xFFFF, never reached);
  //   y, z = float bits of the element multipliers of codes c and c + 1; w unused.
  // The multiplier k of scale code s is a float with RNE_fp4(RN_fp32(x * k)) equal to the exact
  // nearest-code rule for every bf16 x; a negative value means no such k was found: -khi
  // (finite) selects the two-term multiplier, -infinity the exact slow path (encode16).  Codes
  // 0, -1 and 127 have k = 0.
  uint4 ent[128];
};

// Workspace header (8 KiB).  The two-pass path leaves one partial maximum (|bf16| bit pattern)
// per amax workgroup in the first 4 KiB; the single-read path keeps one 64-bit (epoch, max) slot
// per workgroup in the next 4 KiB, with a status word at its end that counts (across calls) the
// workgroups whose grid barrier gave up waiting and read the whole tensor for the maximum.
// Nothing in it needs to be zero between calls.
constexpr int kMaxAmaxSlots = 1024;
constexpr size_t kWsHeaderBytes = 8192;
constexpr size_t kPersistentSlotOffset = 4096;
constexpr int kMaxPersistentSlots = 504;
constexpr size_t kPersistentStatusOffset = 8192 - 64;
static_assert(kMaxAmaxSlots * 4 <= kPersistentSlotOffset, "two-pass slots overlap");
static_assert(kPersistentSlotOffset + kMaxPersistentSlots * 8 <= kPersistentStatusOffset,
              "persistent slots overlap the status word");

// ---------------------------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------------------------

// Fast unsigned division by a runtime constant d >= 1, valid for n < 2^31 (the published
// division-by-invariant-integers method of Granlund and Montgomery, "Division by Invariant
// Integers using Multiplication", 1994):
// q = (umulhi(n, mul) + n) >> shift with shift = ceil(log2 d), mul = 2^32 (2^shift - d) / d + 1.
struct FastDiv {
  uint32_t d, mul, shift;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.mul) + n) >> f.shift;
}

// 16-byte load with the non-temporal hint (streamed once, not worth keeping in the caches).
// Streaming (nontemporal) stores for outputs the kernel does not read back: such lines do not
// stay dirty in L2, so the end of the kernel has less to write back.
__device__ __forceinline__ void ntstore8(uint8_t *p, uint2 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2{v.x, v.y}, (u32x2 *)p);
}
__device__ __forceinline__ void ntstore16(void *p, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4 *)p);
}
__device__ __forceinline__ void ntstore_u8(uint8_t *p, uint32_t v) {
  __builtin_nontemporal_store((uint8_t)v, p);
}
__device__ __forceinline__ void ntstore_u16(uint16_t *p, uint32_t v) {
  __builtin_nontemporal_store((uint16_t)v, p);
}

__device__ __forceinline__ uint4 ntload16(const uint4 *p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load((const u32x4 *)p);
  return make_uint4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// Packed unsigned 16-bit max of two words (two bf16 magnitudes per word).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  ushort2_t r = __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                          __builtin_bit_cast(ushort2_t, b));
  return __builtin_bit_cast(uint32_t, r);
}

// Largest |bf16| bit pattern among 8 packed bf16 values.
__device__ __forceinline__ uint32_t absmax8(uint4 v) {
  uint32_t m = pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                          pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
  return max(m & 0xFFFFu, m >> 16);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

// Workgroup-wide max (all threads get the result).  Ends with a barrier.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max_u32(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t b = red[0];
  for (int w = 1; w < nw; ++w) b = max(b, red[w]);
  __syncthreads();
  return b;
}

__device__ __forceinline__ uint32_t absmax16(const uint4 &a, const uint4 &b) {
  const uint32_t m = pk_max_u16(pk_max_u16(pk_max_u16(a.x & 0x7FFF7FFFu, a.y & 0x7FFF7FFFu),
                                           pk_max_u16(a.z & 0x7FFF7FFFu, a.w & 0x7FFF7FFFu)),
                                pk_max_u16(pk_max_u16(b.x & 0x7FFF7FFFu, b.y & 0x7FFF7FFFu),
                                           pk_max_u16(b.z & 0x7FFF7FFFu, b.w & 0x7FFF7FFFu)));
  return max(m & 0xFFFFu, m >> 16);
}

// Value of an OCP E4M3 byte (0..0x7E): exponent field e, mantissa m; e = 0 is m * 2^-9.
__device__ __forceinline__ float e4m3_to_float(uint32_t b) {
  uint32_t e = b >> 3;
  return e ? __uint_as_float((b + 960u) << 20) : (float)(b & 7u) * 0x1p-9f;
}

__device__ __forceinline__ double e4m3_to_double(uint32_t b) {
  uint32_t e = b >> 3, m = b & 7u;
  unsigned long long bits = ((unsigned long long)(e + 1016u) << 52) | ((unsigned long long)m << 49);
  return e ? __longlong_as_double((long long)bits) : (double)m * 0x1p-9;
}

// bf16 (round to nearest even) of a float, as 16 bits.  Inputs are finite.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Round a positive double (in the bf16 normal range) down to the bf16 grid; returns the bf16
// bit pattern and whether the value was already on the grid.
__device__ __forceinline__ uint32_t bf16_round_down(double p, bool *exact) {
  unsigned long long b = (unsigned long long)__double_as_longlong(p);
  unsigned long long t = b & ~((1ull << 45) - 1ull);  // keep 7 explicit mantissa bits
  *exact = (t == b);
  float f = (float)__longlong_as_double((long long)t);  // exactly representable
  return __float_as_uint(f) >> 16;
}

// Two E2M1 codes for x0, x1 (x0 -> low nibble) written into byte `sel` of `old`, using the
// hardware conversion with unit scale (the scale operand is a power of two; 1.0 leaves the
// input unscaled).  Round-to-nearest-even with saturation at 6.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float x0, float x1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x0, x1, 1.0f, SEL);
}

// Magnitude code (0..7) the fast path assigns to the bf16 magnitude pattern `bits` under the
// multiplier k: RNE_fp4(RN_fp32(x * k)).  The encode kernels compute exactly this per element.
__device__ __forceinline__ uint32_t fast_code(uint32_t bits, float k) {
  float y = __uint_as_float(bits << 16) * k;
  return cvt_fp4x2<0>(0u, y, y) & 7u;
}

// Two-term multiplier for a scale S whose rounded reciprocal khi = RN_fp32(1/S) fails (no single
// float reproduces the rule; this happens when gs has few significant bits, so that exact ties
// x = midpoint * S occur): klo = RN_fp32((1 - S khi) khi) carries 1/S - khi to about 2^-24 of
// itself (the residual comes from one double FMA: S has <= 28 significant bits, khi 24), and an
// element takes y = RN_fp32(x khi + RN_fp32(x klo)), monotone in x like the single product.
// Scaling S by 2^E scales khi and klo by 2^-E exactly while klo stays a normal float, which
// the global-scale range of two_term_range guarantees for every block-scale code.
__device__ __forceinline__ float two_term_lo(float khi, double S) {
  const double e = fma(-S, (double)khi, 1.0);
  return (float)(e * (double)khi);
}

__device__ __forceinline__ bool two_term_range(double gsd) {
  return gsd >= 0x1p-60 && gsd <= 0x1p60;
}

__device__ __forceinline__ uint32_t fast_code2(uint32_t bits, float khi, float klo) {
  const float x = __uint_as_float(bits << 16);
  const float y = fmaf(x, khi, x * klo);
  return cvt_fp4x2<0>(0u, y, y) & 7u;
}

// ---------------------------------------------------------------------------------------------
// Per-tensor tables, built in LDS by every workgroup that encodes (256 threads, three phases).
// ---------------------------------------------------------------------------------------------

// E2M1 midpoints between magnitude indices i and i+1 (i = 0..6).
__device__ __forceinline__ double e2m1_mid(int i) {
  // 0.25 0.75 1.25 1.75 2.5 3.5 5
  return i < 4 ? 0.25 + 0.5 * i : (i == 4 ? 2.5 : (i == 5 ? 3.5 : 5.0));
}

// Does multiplier k reproduce the exact nearest-magnitude rule (ties to even index, saturate at
// 6) around midpoint i under the exact scale S = sb * gs?  The fast code is monotone in x, so it
// suffices that the largest bf16 that must map to <= i does and the smallest bf16 that must map
// to >= i+1 does; checking all 7 midpoints covers every bf16 input.
// `code_of(bits)` is the per-element rule under test (the single or the two-term multiplier).
template <class CodeOf>
__device__ __forceinline__ bool midpoint_ok(const CodeOf &code_of, double S, int i) {
  double P = e2m1_mid(i) * S;  // exact: <= 3 + 28 significant bits
  bool exact;
  uint32_t rd = bf16_round_down(P, &exact);
  if (rd == 0u || rd >= 0x7F80u) return false;
  bool tie_down = (i & 1) == 0;  // midpoint between an even index i and i+1 goes down
  uint32_t below = exact ? (tie_down ? rd : rd - 1u) : rd;
  uint32_t above = exact ? (tie_down ? rd + 1u : rd) : rd + 1u;
  return code_of(below) <= (uint32_t)i && code_of(above) >= (uint32_t)i + 1u;
}

__device__ __forceinline__ bool multiplier_ok_at(float k, double S, int i) {
  return midpoint_ok([&](uint32_t b) { return fast_code(b, k); }, S, i);
}

__device__ __forceinline__ bool multiplier2_ok_at(float khi, float klo, double S, int i) {
  return midpoint_ok([&](uint32_t b) { return fast_code2(b, khi, klo); }, S, i);
}

// Block-scale threshold for code s (1..126): bamax / (6 gs) is rounded to the nearest E4M3 code,
// ties to even, so code s is reached when bamax >= mu * 6 * gs (s even) or > it (s odd), mu being
// the midpoint between codes s-1 and s; mu * 6 * gs has <= 5 + 2 + 24 bits: exact in double.
__device__ __forceinline__ uint32_t scale_threshold(int s, double gsd) {
  double mu = 0.5 * (e4m3_to_double((uint32_t)s - 1u) + e4m3_to_double((uint32_t)s));
  bool exact;
  uint32_t rd = bf16_round_down(mu * 6.0 * gsd, &exact);
  uint32_t th = (s & 1) ? rd + 1u : (exact ? rd : rd + 1u);
  return min(th, 0xFFFFu);
}

// Scaling a block scale by 2^j scales the critical bf16 values around each midpoint by 2^j and
// RN(1/S) by 2^-j, leaving x * k and every decision unchanged (no value leaves the normal range
// for amax in the supported range).  So the multiplier only has to be checked for the 8 E4M3
// mantissas (1 + m/8) * gs; the multiplier of any code is that of its mantissa times a power of
// two.  Subnormal E4M3 codes normalize onto the same mantissas.
//
// A wave runs the 8 x 7 multiplier checks itself (lane 7m + i checks mantissa m at E2M1
// midpoint i), combines them with a ballot and passes the base multipliers around with
// shuffles, so nothing has to meet in LDS before the entries are written.  When a mantissa's
// rounded reciprocal fails somewhere (about one mantissa in six), its neighbouring floats are
// checked the same way, one midpoint per lane, so the repair costs two more checks rather than
// up to fourteen in a row.

// The lane's base multiplier (lanes 7m, m = 0..7, hold mantissa m's).  A negative value means
// that no single float passed: -khi (finite) when the two-term multiplier (khi, two_term_lo)
// passes every check, -infinity when it does not either (or gs is outside two_term_range); the
// blocks with that mantissa take the two-term or the exact slow path.  Every lane of the wave
// must call it (ballots).
__device__ inline float table_base_multiplier(double gsd, bool usable) {
  const int lane = threadIdx.x & 63;
  const int m = lane / 7, i = lane - m * 7;
  const bool checker = usable && lane < 56;
  const double S = (1.0 + m * 0.125) * gsd;
  float kb = checker ? (float)(1.0 / S) : 0.0f;
  const bool ok = checker ? multiplier_ok_at(kb, S, i) : true;
  const unsigned long long bad = __ballot(!ok);
  if (bad) {  // uniform: the ballot is the same in every lane
    // The rounded reciprocal of some mantissa fails somewhere: try the float above it, then
    // the one below, then the two-term multiplier, else take the exact path.
    const float ku = __uint_as_float(__float_as_uint(kb) + 1u);
    const float kd = __uint_as_float(__float_as_uint(kb) - 1u);
    const unsigned long long bad_u = __ballot(checker && !multiplier_ok_at(ku, S, i));
    const unsigned long long bad_d = __ballot(checker && !multiplier_ok_at(kd, S, i));
    const bool two_ok = two_term_range(gsd);
    const float klo = checker && two_ok ? two_term_lo(kb, S) : 0.0f;
    const unsigned long long bad_2 =
        __ballot(checker && (!two_ok || !multiplier2_ok_at(kb, klo, S, i)));
    const unsigned long long mine = 0x7Full << (7 * m);
    if (checker && (bad & mine))
      kb = !(bad_u & mine) ? ku
                           : (!(bad_d & mine) ? kd : (!(bad_2 & mine) ? -kb : -INFINITY));
  }
  return kb;
}

// Table entry c (0..127) from the wave's base multipliers kb (table_base_multiplier); every lane
// of the wave must call it (shuffles), each with its own c.  The multiplier of block-scale code
// c is its mantissa's base multiplier (held by lane 7m) scaled by 2^-exponent; 0 outside 1..126.
__device__ inline uint4 table_entry(int c, float kb, double gsd, bool usable) {
  auto code_multiplier = [&](int cc) {
    const uint32_t vb = __float_as_uint(e4m3_to_float((uint32_t)min(max(cc, 1), 126)));
    const int mc = (int)((vb >> 20) & 7u);
    const int E = (int)((vb >> 23) & 0xFFu) - 127;
    const float base = __shfl(kb, 7 * mc, kWave);
    return (usable && cc >= 1 && cc <= 126) ? ldexpf(base, -E) : 0.0f;
  };
  const uint32_t th = (c + 1 > 126 || !usable) ? 0xFFFFu : scale_threshold(c + 1, gsd);
  const float k0 = code_multiplier(c), k1 = code_multiplier(c + 1);
  return make_uint4(th, __float_as_uint(k0), __float_as_uint(k1), 0u);
}

__device__ __forceinline__ bool gs_usable(float gs) { return gs > 0.0f && gs < 3.0e38f; }

// Fill `t` (in LDS) for global scale gs.  Must be called by every thread of a workgroup of at
// least 128 threads; ends with a barrier (the only one).  A usable gs lies in (0, 3e38);
// otherwise every block gets scale 0.  Threads 0..127 (two whole waves) each write one entry.
// LDS_ONLY: the barrier waits for the waves' LDS accesses alone, not for their outstanding
// global loads (a workgroup barrier with the usual fence waits for every load in flight).
template <bool LDS_ONLY = false>
__device__ inline void build_tables(QuantTables &t, float gs) {
  const int tid = threadIdx.x;
  const double gsd = (double)gs;
  const bool usable = gs_usable(gs);
  if (tid < 128) {
    const float kb = table_base_multiplier(gsd, usable);
    t.ent[tid] = table_entry(tid, kb, gsd, usable);
  }
  if (tid == 0) {
    t.gs = gs;
    t.inv6gs = usable ? (float)(1.0 / (6.0 * gsd)) : 0.0f;
  }
  if (LDS_ONLY)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    __syncthreads();
}

// The same tables built by one wave alone (all 64 lanes call it; each writes entries lane and
// lane + 64), with no barrier: the calling wave may read them at once (its LDS accesses complete
// in order), other waves only after a barrier that follows this call.
__device__ inline void build_tables_one_wave(QuantTables &t, float gs) {
  const int lane = threadIdx.x & 63;
  const double gsd = (double)gs;
  const bool usable = gs_usable(gs);
  const float kb = table_base_multiplier(gsd, usable);
  t.ent[lane] = table_entry(lane, kb, gsd, usable);
  t.ent[lane + 64] = table_entry(lane + 64, kb, gsd, usable);
  if (lane == 0) {
    t.gs = gs;
    t.inv6gs = usable ? (float)(1.0 / (6.0 * gsd)) : 0.0f;
  }
}

__device__ __forceinline__ float global_scale_from_amax_bits(uint32_t amax_bf16_bits) {
  double amax = (double)__uint_as_float(amax_bf16_bits << 16);
  return (float)(amax / 2688.0);  // correctly rounded: 53 >= 2 * 24 + 2
}

__device__ __forceinline__ float inv6gs_of(float gs) {
  return (gs > 0.0f && gs < 3.0e38f) ? (float)(1.0 / (6.0 * (double)gs)) : 0.0f;
}

// ---------------------------------------------------------------------------------------------
// Block-scale code and element codes
// ---------------------------------------------------------------------------------------------

// E4M3 code of a block whose |max| bf16 pattern is `bam`, and its element multiplier.  The
// guess truncates t = bam * inv6gs to an E4M3 code (top three mantissa bits for normal codes,
// floor(t * 2^9) below 2^-6).  t is within 2^-23 (relative) of the exact bam / (6 gs), so the
// nearest code is the guess or the next one: one comparison with the exact threshold of the
// next code decides, and the same table entry holds both candidate multipliers.
__device__ __forceinline__ int scale_code(uint32_t bam, const QuantTables &tab, float inv6gs,
                                          float *k_out) {
  const float t = __uint_as_float(bam << 16) * inv6gs;
  const int c_norm = (int)(__float_as_uint(t) >> 20) - 960;
  const int c_sub = (int)(t * 512.0f);
  int cand = (t >= 0x1p-6f) ? c_norm : c_sub;
  cand = min(max(cand, 0), kE4M3MaxCode);
  // One 16-byte read (left to itself the compiler turns the selects below into branches around
  // separate 4-byte reads).
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 ev = __builtin_nontemporal_load((const u32x4 *)&tab.ent[cand]);
  const uint4 e = make_uint4(ev[0], ev[1], ev[2], ev[3]);
  const bool up = bam >= e.x;
  *k_out = __uint_as_float(up ? e.z : e.y);
  return cand + (up ? 1 : 0);
}

__device__ __forceinline__ int scale_code(uint32_t bam, const QuantTables &tab, float *k_out) {
  return scale_code(bam, tab, tab.inv6gs, k_out);
}

// Direct block-scale lookup for the encode loops.  Every |max| bf16 pattern p from the first
// scale threshold T1 (the smallest pattern whose code is >= 1) up to the last one T126 gets its
// own entry, filled with scale_code(p) itself, so the lookup is exact by construction:
//   entry 0       : p < T1          -> code 0, multiplier 0
//   entry i       : p = T1 - 1 + i  (1 <= i <= T126 - T1)
//   entry top     : p >= T126       -> code 126 (top = T126 - T1 + 1)
// The thresholds span log2(432 * 2^10) = 18.75 binades of bf16, about 2400 patterns, for every
// global scale of the supported input range (amax in [2^-96, bf16 max]), and fewer where they
// fall among bf16 subnormals.  With gs = 0 (an all-zero tensor) the table is the single entry
// 0 (code 0, multiplier 0) for every pattern.  A block's code is then one subtraction, one
// clamp and two independent LDS reads.
constexpr int kCodeLutEntries = 2432;
struct CodeLut {
  int32_t off;  // T1 - 1
  int32_t top;  // index of the last entry
  uint8_t code[kCodeLutEntries];
  float k[kCodeLutEntries];
};

// Fill `L` from the tables `t` (already built: call after build_tables).  Every thread of the
// workgroup must call it; ends with a barrier.  Returns false (and fills the single zero entry)
// for a global scale without usable thresholds: gs = 0, or outside the supported range, where
// the thresholds leave the table's size (never for the supported range).
__device__ inline bool build_code_lut(CodeLut &L, const QuantTables &t) {
  const float inv6gs = t.inv6gs;
  const int32_t t1 = (int32_t)t.ent[0].x, t126 = (int32_t)t.ent[125].x;
  const int32_t top = t126 - t1 + 1;
  const bool use = inv6gs > 0.0f && t1 >= 1 && top >= 1 && top < kCodeLutEntries;
  if (use) {
    for (int i = threadIdx.x; i <= top; i += blockDim.x) {
      float k;
      const int c = scale_code((uint32_t)(t1 - 1 + i), t, inv6gs, &k);
      L.code[i] = (uint8_t)c;
      L.k[i] = k;
    }
  } else if (threadIdx.x == 0) {
    L.code[0] = 0;
    L.k[0] = 0.0f;
  }
  if (threadIdx.x == 0) {
    L.off = use ? t1 - 1 : 0x7FFF;
    L.top = use ? top : 0;
  }
  __syncthreads();
  return use;
}

// Block-scale code and multiplier from the lookup table; off and top as loaded from L once per
// wave.
__device__ __forceinline__ int lut_code(uint32_t bam, const CodeLut &L, int32_t off, int32_t top,
                                        float *k_out) {
  const int32_t i = min(max((int32_t)bam - off, 0), top);
  *k_out = L.k[i];
  return L.code[i];
}

// Exact magnitude code of |x| (as a float) for block scale value sbv: compare with each
// midpoint * sbv * gs through one FMA (mid * sbv has <= 7 bits, so the product is exact and the
// sign of the FMA result is the sign of the exact difference).
__device__ __forceinline__ uint32_t exact_mag_code(float ax, float sbv, float gs) {
  uint32_t c = 0;
  c += fmaf(-(0.25f * sbv), gs, ax) > 0.0f;
  c += fmaf(-(0.75f * sbv), gs, ax) >= 0.0f;
  c += fmaf(-(1.25f * sbv), gs, ax) > 0.0f;
  c += fmaf(-(1.75f * sbv), gs, ax) >= 0.0f;
  c += fmaf(-(2.5f * sbv), gs, ax) > 0.0f;
  c += fmaf(-(3.5f * sbv), gs, ax) >= 0.0f;
  c += fmaf(-(5.0f * sbv), gs, ax) > 0.0f;
  return c;
}

__device__ __forceinline__ uint32_t exact_code(float x, float sbv, float gs) {
  uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  if (sbv == 0.0f) return sign;
  return sign | exact_mag_code(fabsf(x), sbv, gs);
}

// Exact path for the 8 packed bf16 values of `v` (blocks whose scale has no exact multiplier).
__device__ __noinline__ uint32_t encode8_exact(uint4 v, int code, float gs) {
  const float sbv = e4m3_to_float((uint32_t)code);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r |= exact_code(bf16_lo(w[j]), sbv, gs) << (8 * j);
    r |= exact_code(bf16_hi(w[j]), sbv, gs) << (8 * j + 4);
  }
  return r;
}

// Eight E2M1 codes (one 32-bit word, element 0 in the low nibble) for 8 packed bf16 values,
// for a block whose multiplier k is exact (k >= 0).
__device__ __forceinline__ uint32_t encode8_fast(uint4 v, float k) {
  uint32_t r = 0;
  r = cvt_fp4x2<0>(r, bf16_lo(v.x) * k, bf16_hi(v.x) * k);
  r = cvt_fp4x2<1>(r, bf16_lo(v.y) * k, bf16_hi(v.y) * k);
  r = cvt_fp4x2<2>(r, bf16_lo(v.z) * k, bf16_hi(v.z) * k);
  r = cvt_fp4x2<3>(r, bf16_lo(v.w) * k, bf16_hi(v.w) * k);
  return r;
}

// Eight codes under the two-term multiplier (khi, klo) of the block's scale.
__device__ __forceinline__ uint32_t encode8_two(uint4 v, float khi, float klo) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
    const float ylo = fmaf(lo, khi, lo * klo), yhi = fmaf(hi, khi, hi * klo);
    r |= (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, ylo, yhi, 1.0f, 0) & 0xFFu) << (8 * j);
  }
  return r;
}

// The 16 codes of one block (a: values 0..7, b: values 8..15).  The multiplier path runs
// unconditionally; the rare blocks whose scale has no single exact multiplier (k < 0) are redone
// with the two-term multiplier (k = -khi, finite) or on the exact path (k = -infinity).
__device__ __forceinline__ uint2 encode16(const uint4 &a, const uint4 &b, float k, int code,
                                          float gs) {
  uint2 r = make_uint2(encode8_fast(a, k), encode8_fast(b, k));
  if (k < 0.0f) {
    if (k != -INFINITY) {
      const float khi = -k;
      const float klo = two_term_lo(khi, (double)e4m3_to_float((uint32_t)code) * (double)gs);
      r.x = encode8_two(a, khi, klo);
      r.y = encode8_two(b, khi, klo);
    } else {
      r.x = encode8_exact(a, code, gs);
      r.y = encode8_exact(b, code, gs);
    }
  }
  return r;
}

// ---------------------------------------------------------------------------------------------
// Decode for the GEMM: 8 codes of one word -> 8 fp16 values code * scale (exact: <= 6
// significant bits, magnitudes in [2^-10, 2688]).  The order of the 8 values inside the vector
// is the same for both GEMM operands, which is all the dot product needs.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ half8_t decode8_f16(uint32_t q, half2_t s2) {
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0);
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1);
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2);
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3);
  h0 *= s2;
  h1 *= s2;
  h2 *= s2;
  h3 *= s2;
  half8_t r = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return r;
}

// Same decode into bf16, for products with bf16 operands (weight-only W4A16).  gfx950 has no
// packed bf16 multiply, so the FP4 values are converted to fp32, scaled there and packed to
// bf16; every step is exact for the same reason as above.
__device__ __forceinline__ bf16x8_t decode8_bf16(uint32_t q, float s) {
  const floatx2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  const floatx2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  const floatx2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  const floatx2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  bf16x8_t r = {(__bf16)(f0[0] * s), (__bf16)(f0[1] * s), (__bf16)(f1[0] * s), (__bf16)(f1[1] * s),
                (__bf16)(f2[0] * s), (__bf16)(f2[1] * s), (__bf16)(f3[0] * s), (__bf16)(f3[1] * s)};
  return r;
}

// Two E4M3 scale bytes (low byte first) -> two floats, exact.
__device__ __forceinline__ floatx2_t scales_f32x2(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(two_bytes, 1.0f, false);
}

__device__ __forceinline__ half2_t scale_f16x2(uint32_t b) {
  _Float16 s = (_Float16)e4m3_to_float(b);
  half2_t r = {s, s};
  return r;
}

// Two E4M3 scale bytes (low byte first) -> fp16 pair, exact (OCP E4M3 values are fp16 values),
// with the hardware FP8 conversion (unit scale).
__device__ __forceinline__ half2_t scales_f16x2(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
}

__device__ __forceinline__ half2_t splat_lo(half2_t v) {
  half2_t r = {v[0], v[0]};
  return r;
}
__device__ __forceinline__ half2_t splat_hi(half2_t v) {
  half2_t r = {v[1], v[1]};
  return r;
}

}  // namespace nvfp4
