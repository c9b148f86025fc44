// Shared pieces of the MFMA decode kernels (bf16 and fp8 caches): tile
// geometry, the LDS swizzle, global->LDS DMA, and the MFMA wrappers.
#pragma once
#include "device_util.h"
#include "mla_internal.h"

namespace mla {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) int lds_i32;

constexpr int kHeads = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kBlk = 64;                          // tokens per page
constexpr int kSub = 32;                          // tokens per subtile
constexpr int kRowB = (kDc + kDr) * 2;            // 1152
constexpr int kTileB = kSub * kRowB;              // 36864
constexpr int kBf16Dma = kTileB / (4 * 1024);     // 9 DMA instructions per wave per subtile
// fp8 staging per subtile: e4m3 codes | bf16 k^R (the scales go to a ring)
constexpr int kF8Codes = kSub * kDc;              // 16384
constexpr int kF8Kr = kSub * kDr * 2;             // 4096
constexpr int kF8Dma = 6;                         // 4 code + 1 k^R + 1 scale instruction per wave
constexpr float kTau = 8.0f;                      // lazy-rescale threshold (log2 units)
constexpr int kMaxUnitPages = 512;                // page ids cached in LDS per unit (32768 tokens)

constexpr int kQrStride = kDr * 2 + 16;            // padded bytes per head of the LDS q_rope copy (fp8)

// chunk swizzle of token row t (bits 2, 3, 1 of t -> bits 0, 1, 2): chosen by
// measuring both LDS read patterns of the tile on gfx950
__device__ __forceinline__ int swz_f(int t) { return ((t >> 2) & 1) | (((t >> 3) & 1) << 1) | (((t >> 1) & 1) << 2); }

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

__device__ __forceinline__ i32x4_t make_rsrc(const void* base) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r[2] = -1;                                                        // num_records: no clamping
  r[3] = 0x00020000;                                                // gfx9 raw buffer config
  return r;
}

// A buffer descriptor with no records: every load through it is out of
// range, so the memory system is never touched (a DMA issued through it
// only keeps the instruction count of a loop branch-free).
__device__ __forceinline__ i32x4_t empty_rsrc() {
  i32x4_t r;
  r[0] = 0;
  r[1] = 0;
  r[2] = 0;           // num_records 0
  r[3] = 0x00020000;  // gfx9 raw buffer config
  return r;
}

// 16-byte global -> LDS DMA (buffer_load_dwordx4 ... lds): lane l's 16 bytes
// from rsrc.base + voff land at LDS address m0 + 16*l, m0 being computed with
// scalar arithmetic from a wave-uniform base.  Issued as inline asm so that
// the compiler does not add its own vmcnt waits in front of later LDS reads;
// completion is tracked explicitly with wait_vm<>() + a barrier.  The s_nop
// after the M0 write covers the SALU-writes-M0 -> LDS-DMA hazard; the caller
// issues dma_fence() once after forming the resource descriptor and before
// the first of these.
__device__ __forceinline__ void dma16_m0(i32x4_t rsrc, int voff, int m0v) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v),
      "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// The same DMA for bytes a workgroup reads exactly once (a key/value
// stream): the non-temporal hint marks the lines for early eviction, and on
// gfx950 it also raises the rate of a pure HBM stream into LDS (6.4 -> 7.1
// TB/s with one workgroup of four waves per compute unit).  Data that other
// workgroups re-read through L2 keeps the plain form.
__device__ __forceinline__ void dma16_m0_stream(i32x4_t rsrc, int voff, int m0v) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(m0v),
      "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// wait states between a VALU write of an SGPR (readfirstlane into the
// resource descriptor) and a VMEM instruction that reads it
__device__ __forceinline__ void dma_fence() { asm volatile("s_nop 4" ::: "memory"); }

// byte offset, within a 32-token subtile of a page, of the 16-byte chunk that
// thread slot p (0..2303) of the DMA deposits at LDS chunk p of the tile: the
// swizzle only permutes the low 3 bits of the chunk index inside a row, and a
// row is 72 chunks (a multiple of 8), so the source is p with those bits
// flipped by the row's swizzle
__device__ __forceinline__ int dma_src_offset(int p) { return (p ^ swz_f(p / 72)) << 4; }

// s_waitcnt vmcnt(n) only (gfx9 encoding: expcnt/lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// P.V accumulation with the accumulator pinned to AGPRs (the 16 blocks fill
// the whole AGPR file, leaving every VGPR for queries and temporaries).  The
// s_nop provides the 2 wait states a VALU-written VGPR needs before an MFMA
// reads it as A/B; back-to-back accumulation into the same AGPRs with the same
// opcode needs none.
__device__ __forceinline__ void mfma_acc(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The same two products on fp16 operands (int caches; the bits travel in the
// bf16 vector type), chosen at compile time
__device__ __forceinline__ f32x16_t mfma_f16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ void mfma_acc_f16(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool F16>
__device__ __forceinline__ f32x16_t mfma_op(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  if constexpr (F16)
    return mfma_f16(a, b, c);
  else
    return mfma(a, b, c);
}
template <bool F16>
__device__ __forceinline__ void mfma_acc_op(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if constexpr (F16)
    mfma_acc_f16(acc, a, b);
  else
    mfma_acc(acc, a, b);
}

// Orders VALU/accvgpr access to the AGPR accumulator after (or before) the
// asm MFMAs above: 24 wait states cover the MFMA-writes-AGPR ->
// v_accvgpr_read and v_accvgpr_write -> MFMA-reads-SrcC hazards.
__device__ __forceinline__ void acc_fence(f32x16_t* acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]),
                 "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]), "+a"(acc[10]), "+a"(acc[11]),
                 "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]), "+a"(acc[15]));
}

// Maximum of three scores, one v_max3_f32.  Written as asm because the
// compiler quiets each operand of fmaxf first (a v_max x, x, x per value it
// cannot prove canonical, as MFMA results are), which more than doubles a
// max tree; the scores here are finite or -inf, never NaN.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max / sum of a value with the lane 32 apart (the other half of the wave):
// one VALU permlane swap instead of an LDS-routed shuffle
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// the same with the raw maximum (scores: never NaN)
__device__ __forceinline__ float half_swap_max_raw(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return max3_raw(a, b, b);
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Zero the 16 accumulator blocks with MFMAs whose inputs are zero (AGPR
// destinations, no VALU traffic through the accumulator file)
__device__ __forceinline__ void zero_acc(f32x16_t* acc) {
  bf16x8_t z = {};
  asm volatile("" : "+v"(z));
#pragma unroll
  for (int d = 0; d < 16; ++d) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc[d]) : "v"(z));
}

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
// Renumber them so that consecutive work units (the partitions of one
// sequence, which read the same query rows) run on one XCD.
__device__ __forceinline__ int xcd_slot(int bid, int grid) {
  constexpr int kXcd = 8;
  if (grid % kXcd != 0) return bid;
  return (bid % kXcd) * (grid / kXcd) + bid / kXcd;
}

__device__ __forceinline__ bf16x8_t lds_b128(const lds_u8* p) {
  return *(const __attribute__((address_space(3))) bf16x8_t*)p;
}
__device__ __forceinline__ bf16x4_t lds_tr16(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
}

}  // namespace mla
