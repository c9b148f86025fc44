// Software-pipelined MFMA decode kernel for the DeepSeek-V2/V3 shape of
// absorbed MLA (itwiki "Multi-head latent attention": sections "Decoupled
// RoPE", "Matrix absorption" and the V2/V3 dimension table): n_h = 128 heads
// sharing one latent row [c^KV 512 | k^R 64] per token, 64-token pages, bf16,
// fp8-e4m3 or grouped int4 / int2 content.
//
// Work decomposition
//   * grid.x = persistent workgroups looping over planned units (sequence,
//     contiguous page range); grid.y = query token i of the sequence.
//   * 4 wavefronts, one per SIMD; wavefront w owns heads 32w .. 32w+31 for
//     both contractions: its queries stay in VGPRs, its P.V accumulator
//     (32 heads x 512 dims fp32) fills the AGPRs.
//   * Keys stream through LDS in 32-token subtiles of bf16 rows (36,864 B):
//     16-byte global->LDS DMA straight into a 4-stage ring (bf16 cache), or
//     into an fp8 staging ring that the workgroup expands into one of two
//     bf16 tile slots (fp8 cache; e4m3 -> bf16 is exact).
//   * S^T[token, head] = K[token, 0:576] . Q^T on v_mfma_f32_32x32x16_bf16
//     (A = key rows from LDS via ds_read_b128, B = queries from registers).
//   * O^T[dim, head] += V^T[dim, token] . P^T[token, head]: A = c^KV columns
//     fetched transposed with ds_read_b64_tr_b16, B = P taken straight from
//     the S^T accumulator layout (the lane is the head in both products).
//   * fp8: the per-token scale multiplies the content score (the RoPE part
//     accumulates separately) and P before the P.V product.
//   * Online softmax in the exp2 domain with a lazy reference max: the
//     reference only moves when a subtile's max exceeds it by 2^kTau, so the
//     accumulator is rarely touched outside the MFMAs (numerator and
//     denominator share the reference, so the result is exact).
//
// Pipeline (iteration i; subtile i+1 resident before it starts)
//   phase 1: the last P.V steps of subtile i-1 (value fragments read before
//            the barrier), then QK(i+1) steps 0..19  ||  softmax of subtile
//            i (max, exp2, P)
//   phase 2: QK(i+1) steps 20..35 interleaved with the other P.V steps of
//            subtile i; the DMA of a later subtile rides along
//
// LDS tile layout: row t (token) is 1152 B = 72 chunks of 16 B; logical chunk
// c is stored at chunk (c & ~7) | ((c ^ f(t)) & 7), f(t) = bits 2, 3, 1 of t
// (swz_f), chosen by measuring both read patterns.  The unit's partial (or
// final) output is staged through LDS so each store writes whole rows.
#include "mfma_common.h"

namespace mla {

// bf16 cache: 4 tile stages (tiles i, i+1 in use, i+2, i+3 in flight)
constexpr int kB16Stages = 4;
constexpr int kB16TabOff = kB16Stages * kTileB;             // 147456
// fp8 cache: 3 staging stages (codes + k^R; subtile i+1 being expanded,
// i+2 and i+3 in flight), a ring of per-token scales, two bf16 tile slots,
// and the queries' RoPE part (its own score accumulator takes those registers)
constexpr int kF8StageB = kF8Codes + kF8Kr;                 // 20480 per subtile
constexpr int kF8Stages3 = 3;
constexpr int kF8ScaleSlots = 8;                            // scales of subtile s at slot s % 8
constexpr int kF8ScaleOff = kF8Stages3 * kF8StageB;         // 61440
constexpr int kF8SlotOff = kF8ScaleOff + kF8ScaleSlots * 128;  // 62464
constexpr int kF8QrOff = kF8SlotOff + 2 * kTileB;           // 136192
constexpr int kF8TabOff = kF8QrOff + kHeads * kQrStride;    // 154624
// low-bit caches (int4 / int2 content, int4 RoPE; groups of 32 values with
// an fp16 (scale, min) pair): 3 staging stages of [content codes | RoPE codes
// | parameters] per subtile, decoded into two fp16 tile slots (fp16 keeps 11
// mantissa bits of code * scale + min where bf16 would keep 8; the products
// then run on the fp16 MFMA, queries and P converted to fp16)
constexpr int kFmtBf16 = 0, kFmtFp8 = 1, kFmtInt4 = 2, kFmtInt2 = 3;
constexpr int kIntCodeB(int fmt) { return fmt == kFmtInt4 ? kSub * kDc / 2 : kSub * kDc / 4; }  // 8192 / 4096
constexpr int kIntRopeB = kSub * kDr / 2;                    // 1024
constexpr int kIntGroups = (kDc + kDr) / 32;                 // 18 per token
constexpr int kIntPrmRow = kIntGroups * 4;                   // 72 bytes of parameters per token
constexpr int kIntPrmB = kSub * kIntPrmRow;                  // 2304
constexpr int kIntMiscChunks = (kIntRopeB + kIntPrmB) / 16;  // 208 16-byte chunks: RoPE codes + parameters
constexpr int kIntStageB(int fmt) { return kIntCodeB(fmt) + kIntRopeB + kIntPrmB; }  // 11520 / 7424
constexpr int kIntStages3 = 3;
constexpr int kIntSlotOff(int fmt) { return kIntStages3 * kIntStageB(fmt); }
constexpr int kIntTabOff(int fmt) { return kIntSlotOff(fmt) + 2 * kTileB; }
constexpr int kIntDma(int fmt) { return kIntCodeB(fmt) / 4096 + 1; }  // content instructions + 1
constexpr int kPipeTabOff(int fmt) {
  return fmt == kFmtBf16 ? kB16TabOff : fmt == kFmtFp8 ? kF8TabOff : kIntTabOff(fmt);
}
constexpr int kOutRowF = kDc + 4;                           // padded fp32 row of the output staging
constexpr int kOutRowH = kDc * 2 + 16;                      // padded bf16 row (bytes)
// the finalize stages 64 fp32 rows or 128 bf16 rows through LDS (after every
// tile, staging slot and page id of the unit is consumed)
constexpr int kOutStageB = 64 * kOutRowF * 4 > kHeads * kOutRowH ? 64 * kOutRowF * 4 : kHeads * kOutRowH;
constexpr int kPipeLds(int fmt) {
  return kPipeTabOff(fmt) + kMaxUnitPages * 4 > kOutStageB ? kPipeTabOff(fmt) + kMaxUnitPages * 4 : kOutStageB;
}
static_assert(kPipeLds(kFmtFp8) <= 160 * 1024 && kPipeLds(kFmtInt4) <= 160 * 1024, "LDS budget");
static_assert(kIntMiscChunks <= 256, "one misc DMA instruction per thread");

// fp16 (scale, min) pair of a group, packed in one dword -> the scale in
// both halves of one dword, the minimum in both halves of another
__device__ __forceinline__ void int_params_x2(uint32_t pr, uint32_t& sc2, uint32_t& mn2) {
  sc2 = (pr & 0xffffu) | (pr << 16);
  mn2 = (pr >> 16) | (pr & 0xffff0000u);
}
// Two codes -> two fp16 values code * scale + min.  The codes sit in the low
// bits of each 16-bit half of x (`mask` keeps them); or-ing in the exponent
// of 1024 makes each half the fp16 number 1024 + code (exact: the spacing
// there is 1), subtracting 1024 leaves the code, and one packed fp16 fma
// rounds code * scale + min once.
__device__ __forceinline__ uint32_t dequant_pair(uint32_t x, uint32_t mask, uint32_t sc2, uint32_t mn2) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 c = __builtin_bit_cast(f16x2, (x & mask) | 0x64006400u) - (f16x2){(_Float16)1024, (_Float16)1024};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, __builtin_bit_cast(f16x2, sc2),
                                                                __builtin_bit_cast(f16x2, mn2)));
}
// one packed word of 8 int4 codes (value 2k at bit 4k, 2k+1 at bit 16+4k) ->
// 8 fp16 values in value order: nibble k of both halves is the pair (2k, 2k+1)
__device__ __forceinline__ u32x4_t int4_word_f16(uint32_t wd, uint32_t sc2, uint32_t mn2) {
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = dequant_pair(wd >> (4 * k), 0x000F000Fu, sc2, mn2);
  return o;
}
// one packed word of 16 int2 codes (value 2k at bit 2k, 2k+1 at bit 16+2k)
// -> values 0..7 (a) and 8..15 (b) as fp16
__device__ __forceinline__ void int2_word_f16(uint32_t wd, uint32_t sc2, uint32_t mn2, u32x4_t& a, u32x4_t& b) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k] = dequant_pair(wd >> (2 * k), 0x00030003u, sc2, mn2);
    b[k] = dequant_pair(wd >> (2 * k + 8), 0x00030003u, sc2, mn2);
  }
}
// the 8 bf16 query values of a fragment as fp16 (exact inside the fp16 range)
__device__ __forceinline__ bf16x8_t bf16x8_as_f16(bf16x8_t v) {
  typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (_Float16)(float)v[e];
  return __builtin_bit_cast(bf16x8_t, h);
}
// one operand value of the products: bf16, or fp16 (int caches) carried in
// the bf16 vector type
template <bool F16>
__device__ __forceinline__ __bf16 op16(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(__bf16, (_Float16)x);
  else
    return (__bf16)x;
}

template <int FMT>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_pipe_kernel(DecodeArgs a) {
  constexpr bool FP8 = FMT == kFmtFp8;      // per-token scaled e4m3 content codes
  constexpr bool INT = FMT >= kFmtInt4;     // grouped low-bit codes
  constexpr bool STAGED = FMT != kFmtBf16;  // codes staged, expanded into 16-bit tile slots
  constexpr bool F16 = INT;                 // fp16 operands (tiles, queries, P); bf16 otherwise
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  lds_i32* tab = (lds_i32*)(smem + kPipeTabOff(FMT));
  constexpr int kDma = FP8 ? kF8Dma : INT ? kIntDma(FMT) : kBf16Dma;  // DMA instructions per wave per subtile
  constexpr int kAhead = 2;                           // subtiles in flight beyond the next one
  constexpr int kQReg = FP8 ? 32 : 36;                // query fragments held in registers

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  const int qi = blockIdx.y;
  const int R = a.s_q * kHeads;
  const int head = w * 32 + l32;
  const int n_units = min(((const WsHeader*)a.ws_header)->n_units, a.units_max);
  const float scale2 = a.scale * kLog2e;

  int off_qk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) off_qk[j] = l32 * kRowB + (((2 * j + g) ^ swz_f(l32)) << 4);
  // transposed V reads: rows ta (first 4 k-slots) and ta + 8 (last 4), for
  // even / odd 32-dim blocks
  int off_pv[2][2];
  {
    const int ta = 4 * g + (j16 >> 2);
    const int clo = 2 * (G & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = ta + 8 * h;
        off_pv[p][h] = t * kRowB + (((4 * p + clo) ^ swz_f(t)) << 4) + (j16 & 1) * 8;
      }
  }
  const int w_s = __builtin_amdgcn_readfirstlane(w);  // wave index as a scalar
  for (int unit = xcd_slot(blockIdx.x, gridDim.x); unit < n_units; unit += gridDim.x) {
    const int4 wk = a.work[unit];
    // a plan entry outside this call's shapes (a workspace that holds no
    // plan of this batch) is skipped: wrong results, never a stray access.
    // (first > end is a planned empty partition: it still writes its empty
    // partial result.)
    if (wk.x < 0 || wk.x >= a.B || wk.y < 0 || wk.z > a.max_blocks || wk.z - wk.y > kMaxUnitPages) continue;
    const int b = wk.x;
    const bool final_out = wk.w < 0;           // the sequence is not split
    const int L = final_out ? ~wk.w : wk.w;    // its length
    const int vis = L - a.s_q + qi + 1;
    const int tok0 = wk.y * kBlk;
    const int tok1 = min(wk.z * kBlk, vis);
    const int ntok = tok1 - tok0;
    const int n_sub = ntok > 0 ? (ntok + kSub - 1) / kSub : 0;
    const int n_last = ntok - (n_sub - 1) * kSub;  // valid rows of the last subtile
    auto nvalid_of = [&](int t) { return t == n_sub - 1 ? n_last : kSub; };

    __syncthreads();  // the previous unit is done with LDS
    // the unit's page ids and the sequence's length first, then the queries
    // and their RoPE part: the first DMA waits for the page ids alone and
    // the query rows arrive under it.  Every query load is complete before
    // the subtile loop (an explicit full wait, or for bf16 the compiler's own
    // waits in the first subtile's QK chain, which also cover the DMAs issued
    // after the queries), so the compiler's vmcnt accounting never places a
    // wait in the loop, where it would also wait for the DMA ring.  (Its
    // waits are conservative: it does not count the DMAs, which are all
    // younger than the queries; the loop's explicit waits stay exact.)
    bf16x8_t q[kQReg];
    bf16x8_t qrv[4];
    lds_u8* qr_lds = smem + kF8QrOff;  // fp8: RoPE query rows, kQrStride bytes per head
    {
      static_assert(kMaxUnitPages <= 512, "two page ids per thread");
      const int npg = (n_sub * kSub + kBlk - 1) / kBlk;
      const int32_t* trow = a.table + (long long)b * a.max_blocks + wk.y;
      const int pg0 = tid < npg ? trow[tid] : 0;
      const int pg1 = tid + 256 < npg ? trow[tid + 256] : 0;
      const int len_now = a.seq_lens[b];
      // uniform row base + 32-bit per-lane offset (scalar base addressing)
      const long long row0 = ((long long)b * a.s_q + qi) * kHeads;
      const uint8_t* ql = (const uint8_t*)a.q_lat + row0 * (kDc * 2);
      const uint8_t* qr = (const uint8_t*)a.q_rope + row0 * (kDr * 2);
      // recomputed here rather than kept live across the unit loop
      int hl = threadIdx.x;
      asm volatile("" : "+v"(hl));
      const int hd = (hl >> 6) * 32 + (hl & 31), gg = (hl >> 5) & 1;
      const int ol = hd * (kDc * 2) + gg * 16, orp = hd * (kDr * 2) + gg * 16;
#pragma unroll
      for (int kb = 0; kb < 32; ++kb) q[kb] = *(const bf16x8_t*)(ql + ol + kb * 32);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qrv[kb] = *(const bf16x8_t*)(qr + orp + kb * 32);
      // table slots past the sequence's pages may hold anything: an entry
      // reaching beyond them (not planned from these lengths) is skipped
      if (wk.z > max(1, (len_now + kBlk - 1) / kBlk)) continue;
      if (tid < npg) tab[tid] = pg0;
      if (tid + 256 < npg) tab[tid + 256] = pg1;
    }
    __syncthreads();  // page ids visible
    // the queries in their operand form, after a full wait: below, once the
    // first subtiles are in flight; the int formats (whose fp16 conversion
    // would otherwise stay live across the DMA issue and spill into the
    // loop) before any DMA
    auto place_queries = [&]() {
      if (F16) {  // int caches: the products run on fp16 operands
#pragma unroll
        for (int kb = 0; kb < 32; ++kb) q[kb] = bf16x8_as_f16(q[kb]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qrv[kb] = bf16x8_as_f16(qrv[kb]);
      }
      int hl = threadIdx.x;
      asm volatile("" : "+v"(hl));
      const int hd = (hl >> 6) * 32 + (hl & 31), gg = (hl >> 5) & 1;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (FP8)
          *(__attribute__((address_space(3))) bf16x8_t*)(qr_lds + hd * kQrStride + (2 * kb + gg) * 16) = qrv[kb];
        else
          q[(32 + kb) % kQReg] = qrv[kb];
      }
    };
    if (INT) {
      wait_vm<0>();
      place_queries();
    }
    // DMA instruction i (0 .. kDma-1) of subtile s for this wave; the bf16
    // tile lands swizzled, the fp8 staging (codes, k^R, scales) linear
    // descriptor of subtile s's half of its page pg (a page id read from the
    // unit's table in LDS)
    auto page_rsrc_of = [&](int s, int pg_lds) {
      const int pg = __builtin_amdgcn_readfirstlane(pg_lds);
      const uint8_t* blk = (const uint8_t*)a.kv + (long long)pg * a.block_bytes;
      return make_rsrc(STAGED ? blk : blk + (s & 1) * kTileB);
    };
    auto page_rsrc = [&](int s) { return page_rsrc_of(s, tab[s >> 1]); };
    auto dma_dst = [&](int s) {  // LDS base (scalar) of subtile s's DMA landing area for this wave
      return __builtin_amdgcn_readfirstlane(
          (int)(uint32_t)(uintptr_t)(smem + (FP8   ? (s % kF8Stages3) * kF8StageB
                                             : INT ? (s % kIntStages3) * kIntStageB(FMT)
                                                   : (s % kB16Stages) * kTileB)));
    };
    // tv: the thread index the source offsets derive from (the prologue
    // passes a copy the compiler cannot see through, so that its offsets
    // are computed there instead of being the loop's, one of which the
    // prologue's register pressure would spill and reload between DMAs)
    auto dma_one = [&](const i32x4_t& rs, int m0b, int s, int i, int tv) {
      if (!STAGED) {
        dma16_m0_stream(rs, dma_src_offset(i * 256 + tv), m0b + i * 4096 + w_s * 1024);
      } else if (INT) {
        // block: [64 x content codes | 64 x RoPE codes | 64 x parameters];
        // subtile half s & 1 of each part
        constexpr int cb = kIntCodeB(FMT);
        const int half = s & 1;
        if (i < kDma - 1) {  // content codes, 4 KB per instruction
          dma16_m0_stream(rs, half * cb + ((i * 4 + w) * 64 + lane) * 16, m0b + (i * 4 + w_s) * 1024);
        } else {  // RoPE codes (64 chunks) then parameters (144 chunks), one per thread
          const int p = tid;
          if (p < kIntMiscChunks) {
            const int src = p < kIntRopeB / 16 ? 2 * cb + half * kIntRopeB + p * 16
                                               : 2 * cb + 2 * kIntRopeB + half * kIntPrmB + (p - kIntRopeB / 16) * 16;
            dma16_m0_stream(rs, src, m0b + cb + w_s * 1024);
          }
        }
      } else {
        const int half = s & 1;
        if (i < 4) {         // content codes: 16 KB, 4 x 1 KB per wave
          dma16_m0_stream(rs, half * kF8Codes + ((i * 4 + w) * 64 + lane) * 16, m0b + (i * 4 + w_s) * 1024);
        } else if (i == 4) {  // RoPE keys: 4 KB
          dma16_m0_stream(rs, kBlk * kDc + half * kF8Kr + (w * 64 + lane) * 16, m0b + kF8Codes + w_s * 1024);
        } else if (lane < 8) {  // scales: 128 B to the scale ring (every wave, same bytes)
          const int ring = __builtin_amdgcn_readfirstlane(
              (int)(uint32_t)(uintptr_t)(smem + kF8ScaleOff + (s % kF8ScaleSlots) * 128));
          dma16_m0_stream(rs, kBlk * (kDc + 2 * kDr) + half * (kSub * 4) + lane * 16, ring);
        }
      }
    };
    // past the unit's last subtile the group is issued through a descriptor
    // with no records (no memory traffic; zeros at most land in a ring slot
    // that is free at that point), so every iteration issues the same
    // instructions and every wait below has a constant count
    auto issue = [&](int s, int tv) {
      const i32x4_t rs = s < n_sub ? page_rsrc(s) : empty_rsrc();
      const int m0b = dma_dst(s);
      dma_fence();
#pragma unroll
      for (int i = 0; i < kDma; ++i) dma_one(rs, m0b, s, i, tv);
    };
    auto tile_of = [&](int s) {
      return smem + (FP8 ? kF8SlotOff + (s & 1) * kTileB
                         : INT ? kIntSlotOff(FMT) + (s & 1) * kTileB : (s % kB16Stages) * kTileB);
    };
    // per-token scales of subtile s for this lane's rows 8qd + 4g + 0..3
    auto scales_of = [&](int s, int qd) {
      return *(const __attribute__((address_space(3))) f32x4_t*)(smem + kF8ScaleOff + (s % kF8ScaleSlots) * 128 +
                                                                  16 * g + 32 * qd);
    };
    // int4 / int2: decode staged subtile s into its fp16 tile slot (rows past
    // nv -> 0).  A job is one 16-byte chunk of codes: int4 content 2 per
    // thread (32 values, one group each), int2 content 1 per thread (64
    // values, two groups); the 64 RoPE chunks (int4, one group each) go to
    // the first 64 threads.  All LDS reads are issued before any conversion.
    auto convert_int = [&](int s, int nv) {
      constexpr int cbits = FMT == kFmtInt4 ? 4 : 2;
      constexpr int rowC = kDc * cbits / 8;      // content code bytes per token
      constexpr int cpr = rowC / 16;             // code chunks per token
      constexpr int nj = kSub * cpr / 256;       // content jobs per thread
      const lds_u8* st = smem + (s % kIntStages3) * kIntStageB(FMT);
      const lds_u8* prm = st + kIntCodeB(FMT) + kIntRopeB;
      lds_u8* tl = smem + kIntSlotOff(FMT) + (s & 1) * kTileB;
      typedef __attribute__((address_space(3))) u32x4_t lds_u4;
      typedef __attribute__((address_space(3))) u32x2_t lds_u2;
      typedef __attribute__((address_space(3))) uint32_t lds_u1;
      u32x4_t cw[nj];
      u32x2_t pw[nj];
#pragma unroll
      for (int i = 0; i < nj; ++i) {
        const int job = tid + 256 * i, t = job / cpr, j = job % cpr;
        cw[i] = *(const lds_u4*)(st + t * rowC + j * 16);
        if (cbits == 4)
          pw[i][0] = *(const lds_u1*)(prm + t * kIntPrmRow + j * 4);
        else
          pw[i] = *(const lds_u2*)(prm + t * kIntPrmRow + j * 8);
      }
      const int tr = tid >> 1, jr = tid & 1;  // RoPE job of threads 0..63
      u32x4_t rw = {0, 0, 0, 0};
      uint32_t rp = 0;
      if (tid < 64) {
        rw = *(const lds_u4*)(st + kIntCodeB(FMT) + tr * (kDr / 2) + jr * 16);
        rp = *(const lds_u1*)(prm + tr * kIntPrmRow + (kDc / 32 + jr) * 4);
      }
      auto put = [&](int t, int c, const u32x4_t& v) {  // logical bf16 chunk c of row t
        *(__attribute__((address_space(3))) u32x4_t*)(tl + t * kRowB + ((c ^ swz_f(t)) << 4)) =
            t < nv ? v : u32x4_t{0, 0, 0, 0};
      };
#pragma unroll
      for (int i = 0; i < nj; ++i) {
        const int job = tid + 256 * i, t = job / cpr, j = job % cpr;
        if (cbits == 4) {
          uint32_t sc2, mn2;
          int_params_x2(pw[i][0], sc2, mn2);
#pragma unroll
          for (int k = 0; k < 4; ++k) put(t, 4 * j + k, int4_word_f16(cw[i][k], sc2, mn2));
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t sc2, mn2;
            int_params_x2(pw[i][k >> 1], sc2, mn2);
            u32x4_t va, vb;
            int2_word_f16(cw[i][k], sc2, mn2, va, vb);
            put(t, 8 * j + 2 * k, va);
            put(t, 8 * j + 2 * k + 1, vb);
          }
        }
      }
      if (tid < 64) {
        uint32_t sc2, mn2;
        int_params_x2(rp, sc2, mn2);
#pragma unroll
        for (int k = 0; k < 4; ++k) put(tr, kDc / 8 + 4 * jr + k, int4_word_f16(rw[k], sc2, mn2));
      }
    };
    // fp8: expand staged subtile s into its bf16 tile slot (rows past nv -> 0).
    // Each lane takes 16 codes (one 16-byte read) of row t = 8i + 2w + g per
    // step i and writes the two swizzled 16-byte bf16 chunks; the four reads
    // are issued before any conversion.  e4m3 -> bf16 with a unit scale is
    // exact.
    auto convert = [&](int s, int nv) {
      if constexpr (INT) {
        convert_int(s, nv);
        return;
      }
      const lds_u8* st = smem + (s % kF8Stages3) * kF8StageB;
      lds_u8* tl = smem + kF8SlotOff + (s & 1) * kTileB;
      const int c0 = 2 * l32;  // first of the lane's two 8-code chunks
      u32x4_t cv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 8 * i + 2 * w + g;
        cv[i] = *(const __attribute__((address_space(3))) u32x4_t*)(st + t * kDc + c0 * 8);
      }
      u32x4_t kr = {0, 0, 0, 0};
      const int tr = tid >> 3, cr = tid & 7;  // RoPE: one 16-byte chunk per thread
      if (tr < nv) kr = *(const __attribute__((address_space(3))) u32x4_t*)(st + kF8Codes + tr * 128 + cr * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 8 * i + 2 * w + g;
        const bool ok = t < nv;
        const int f = swz_f(t);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4_t o;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t word = ok ? cv[i][2 * h + j] : 0u;
            const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
            const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true);
            o[2 * j] = __builtin_bit_cast(uint32_t, lo);
            o[2 * j + 1] = __builtin_bit_cast(uint32_t, hi);
          }
          *(__attribute__((address_space(3))) u32x4_t*)(tl + t * kRowB + (((c0 + h) ^ f) << 4)) = o;
        }
      }
      *(__attribute__((address_space(3))) u32x4_t*)(tl + tr * kRowB + ((64 + (cr ^ swz_f(tr))) << 4)) = kr;
    };
    // zero the value rows of a ragged last subtile (they may hold NaN); all threads
    auto zero_tail = [&](int s) {
      lds_u8* t_ = tile_of(s);
      const int nv = nvalid_of(s);
      for (int e = tid; e < (kSub - nv) * 72; e += 256) {
        const int t = nv + e / 72, c = e % 72;
        *(__attribute__((address_space(3))) u32x4_t*)(t_ + t * kRowB + c * 16) = u32x4_t{0, 0, 0, 0};
      }
    };

    f32x16_t acc[16];
    zero_acc(acc);
    acc_fence(acc);
    float m_run = -INFINITY, l_run = 0.f;

    if (n_sub > 0) {
      int tv = threadIdx.x;
      asm volatile("" : "+v"(tv));
#pragma unroll
      for (int s = 0; s <= kAhead; ++s) issue(s, tv);
      if (INT || !STAGED) {
        // the queries (issued first) and subtile 0 landed; subtiles
        // 1 .. kAhead may still fly.  bf16: the first subtile's QK steps
        // start under their arrival (the compiler's own waits before the
        // later query fragments' first uses count only the query loads, so
        // they also wait for the DMAs issued after them: those steps keep
        // pace with the arrivals, and every load is complete by the last
        // step, before the loop)
        wait_vm<kAhead * kDma>();
      } else {
        wait_vm<0>();  // the queries and subtiles 0 .. kAhead landed
        place_queries();
      }
      __syncthreads();  // subtile 0 (and fp8 RoPE queries) visible
      if (STAGED) {
        convert(0, nvalid_of(0));
        __syncthreads();
      } else if (n_last < kSub && n_sub == 1) {
        zero_tail(0);
        __syncthreads();
      }
    }

    // B operand of QK step f: the query fragment (fp8: RoPE steps from LDS)
    auto qfrag = [&](int f) {
      if (FP8 && f >= 32) return lds_b128(qr_lds + head * kQrStride + (2 * (f - 32) + g) * 16);
      return q[f % kQReg];
    };
    // ---- helpers on LDS tiles
    // QK A-operand fragment f (0..35) of a tile: k-block f, slot group g
    auto kfrag = [&](const lds_u8* tile, int f) { return lds_b128(tile + off_qk[f & 3] + (f >> 2) * 128); };
    // PV A-operand fragment of step (db, ks): V^T[dims db*32.., tokens 16ks + {4g..4g+3, 8+4g..}]
    auto vfrag = [&](const lds_u8* tile, int step) {
      const int db = step & 15, ks = step >> 4;  // ks-outer order
      const int kofs = (db >> 1) * 128 + ks * 16 * kRowB;
      const bf16x4_t lo = lds_tr16(tile + off_pv[db & 1][0] + kofs);
      const bf16x4_t hi = lds_tr16(tile + off_pv[db & 1][1] + kofs);
      bf16x8_t v;
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
      v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      return v;
    };
    // raw scores of the token rows past the end of a ragged subtile -> -inf
    // (a uniform branch; full subtiles skip it)
    auto mask_tail = [&](f32x16_t& sv, int nv) {
      if (nv < kSub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 8 * (r >> 2) + 4 * g + (r & 3);
          sv[r] = t < nv ? sv[r] : -INFINITY;
        }
      }
    };
    // max of the 16 raw scores of a lane (tree), then of the two wave halves
    // holding the same head, in the exp2 domain (the scale is positive)
    auto row_max = [&](const f32x16_t& sv) {
      float m8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) m8[i] = fmaxf(sv[2 * i], sv[2 * i + 1]);
#pragma unroll
      for (int w2 = 4; w2 >= 1; w2 >>= 1)
#pragma unroll
        for (int i = 0; i < w2; ++i) m8[i] = fmaxf(m8[i], m8[i + w2]);
      return half_swap_max(m8[0]) * scale2;
    };

    // softmax of the raw scores sp of one subtile against the running max:
    // lazy new reference, exp2 weights in bf16 (P) and their row sum.  The
    // VALU work is split in pieces so it can sit between MFMAs.
    f32x16_t sp;    // raw S of the subtile whose P.V comes next
    f32x16_t sc;    // S of the following subtile, accumulating (content part for fp8)
    f32x16_t sr;    // fp8: its RoPE part
    bf16x8_t P[2];  // P of subtile sp
    int sp_sub = 0; // subtile index of sp (fp8: scales of P)
    // fp8: S = scale_t * content + RoPE for the 16 rows of a lane
    auto form_scores = [&](int s) {
      if (FP8) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4_t ts = scales_of(s, qd);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * qd + e] = __builtin_fmaf(sc[4 * qd + e], ts[e], sr[4 * qd + e]);
        }
      }
    };
    float m_new = -INFINITY, ps0 = 0.f, ps1 = 0.f;
    float m8[8];
    // The softmax of sp is software-pipelined over 11 stages that sit between
    // the first QK steps of the next subtile: max tree (0..3), lane-half
    // exchange and the lazy reference (4), then for groups of 4 rows: scaled
    // shift, exp2, and row sums + bf16 P one stage apart each, so every
    // dependent VALU op issues at least one MFMA after its producer.
    auto sm_fma = [&](int q4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[4 * q4 + e] = __builtin_fmaf(sp[4 * q4 + e], scale2, -m_new);
    };
    auto sm_ex = [&](int q4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[4 * q4 + e] = __builtin_amdgcn_exp2f(sp[4 * q4 + e]);
    };
    auto sm_cvt = [&](int q4) {  // rows 8*q4 + 4g + 0..3 of the subtile
      ps0 += sp[4 * q4] + sp[4 * q4 + 2];
      ps1 += sp[4 * q4 + 1] + sp[4 * q4 + 3];
      if (FP8) {  // the value rows hold raw codes: their scale goes into P
        const f32x4_t ts = scales_of(sp_sub, q4);
        const int t0 = 8 * q4 + 4 * g;  // masked rows may hold any scale
        const int nv = nvalid_of(sp_sub);
#pragma unroll
        for (int e = 0; e < 4; ++e) P[q4 >> 1][(q4 & 1) * 4 + e] = (__bf16)(t0 + e < nv ? sp[4 * q4 + e] * ts[e] : 0.f);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) P[q4 >> 1][(q4 & 1) * 4 + e] = op16<F16>(sp[4 * q4 + e]);
      }
    };
    auto sm_stage = [&](int st) {  // stages 0..10
      // max tree over the 16 scores of the lane as three-input maxima:
      // 16 -> 6 -> 2 -> 1 (stage 3 is left empty: every dependent step
      // stays one MFMA after its producer).  The int4 kernel keeps the
      // two-input tree: with the other its register allocation spills one
      // value inside the loop, and that reload waits for every DMA in flight.
      if (FMT == kFmtInt4) {
        if (st == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) m8[i] = fmaxf(sp[2 * i], sp[2 * i + 1]);
        } else if (st == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) m8[i] = fmaxf(m8[i], m8[i + 4]);
        } else if (st == 2) {
          m8[0] = fmaxf(m8[0], m8[2]);
          m8[1] = fmaxf(m8[1], m8[3]);
        } else if (st == 3) {
          m8[0] = fmaxf(m8[0], m8[1]);
        }
      } else if (st == 0) {
#pragma unroll
        for (int i = 0; i < 5; ++i) m8[i] = max3_raw(sp[3 * i], sp[3 * i + 1], sp[3 * i + 2]);
      } else if (st == 1) {
        m8[0] = max3_raw(m8[0], m8[1], m8[2]);
        m8[1] = max3_raw(m8[3], m8[4], sp[15]);
      } else if (st == 2) {
        m8[0] = max3_raw(m8[0], m8[1], m8[1]);
      }
      if (st == 4) {
        const float mx = (FMT == kFmtInt4 ? half_swap_max(m8[0]) : half_swap_max_raw(m8[0])) * scale2;
        m_new = mx > m_run + kTau ? mx : m_run;  // lazy: keep the reference unless far behind
        ps0 = ps1 = 0.f;
      } else if (st >= 5) {
        const int k = st - 5;  // shift of group k, exp2 of group k-1, sums and P of group k-2
        if (k >= 2) sm_cvt(k - 2);
        if (k >= 1 && k <= 4) sm_ex(k - 1);
        if (k <= 3) sm_fma(k);
      }
    };
    // the reference moved (rare): rescale O and the row sum before new P.V
    auto sm_commit = [&]() {
      if (m_new != m_run) {
        const float f = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= f;
        acc_fence(acc);
#pragma unroll
        for (int d = 0; d < 16; ++d) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[d][r] *= f;
          asm volatile("" : "+a"(acc[d]));
        }
        acc_fence(acc);
        m_run = m_new;
      }
      l_run += ps0 + ps1;
    };

    if (n_sub > 0) {
      // S(0) -> sp, its first reference max
      const lds_u8* tile = tile_of(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; sr[r] = 0.f; }
      bf16x8_t ka[2] = {kfrag(tile, 0), kfrag(tile, 1)};
      // bf16: the RoPE query fragments straight from their loads (placed
      // into the query array after this subtile)
      auto qfrag0 = [&](int f) { return !STAGED && f >= 32 ? qrv[f - 32] : qfrag(f); };
#pragma unroll
      for (int f = 0; f < 36; ++f) {
        if (FP8 && f >= 32) sr = mfma_op<F16>(ka[f & 1], qfrag0(f), sr); else sc = mfma_op<F16>(ka[f & 1], qfrag0(f), sc);
        if (f + 2 < 36) ka[f & 1] = kfrag(tile, f + 2);
      }
      if (!STAGED) place_queries();
      form_scores(0);
      sp = sc;
      sp_sub = 0;
      mask_tail(sp, nvalid_of(0));
      m_run = row_max(sp);
    }

    constexpr int kQkA = 20;  // QK steps overlapped with the softmax
    // The last kCarry P.V steps of a subtile run at the start of the next
    // iteration: their value fragments are read into vc before the barrier,
    // so after it the MFMA pipe has work while the first key fragments of
    // the next subtile come from LDS (alone, the softmax phase's first steps
    // waited out the pipe drain, the barrier and that LDS latency).  Their
    // slot is refilled only in the next P.V phase, after the reads have
    // completed at the barrier.  Zero operands before the first subtile.
    // (The int formats' registers spill with it.)
    constexpr int kCarry = INT ? 0 : 4;
    static_assert(32 - kCarry <= 2 * (36 - kQkA), "at most two P.V steps per QK step of the second phase");
    bf16x8_t vc[kCarry > 0 ? kCarry : 1];
#pragma unroll
    for (int j = 0; j < (kCarry > 0 ? kCarry : 1); ++j) vc[j] = bf16x8_t{};
    P[0] = bf16x8_t{};
    P[1] = bf16x8_t{};
    auto carried_pv = [&]() {
#pragma unroll
      for (int j = 0; j < kCarry; ++j) mfma_acc_op<F16>(acc[(32 - kCarry + j) & 15], vc[j], P[1]);
    };
    // the page id of the loop's DMA one iteration ahead (an LDS read at the
    // top of the iteration that uses it put its latency before the key
    // fragments' reads); entries past the unit's pages are read, not used
    int pg_next = tab[min((kAhead + 1) >> 1, kMaxUnitPages - 1)];
    for (int it = 0; it + 1 < n_sub; ++it) {
      // ---- (A) next subtile resident; refill the stage subtile it-1 used
      wait_vm<(kAhead - 1) * kDma>();  // subtile it+1 landed (one group, it+2, may fly)
      __syncthreads();
      if (STAGED) {  // expand subtile it+1 into the slot subtile it-1 used
        convert(it + 1, nvalid_of(it + 1));
        __syncthreads();
      } else if (it + 1 == n_sub - 1 && n_last < kSub) {
        zero_tail(it + 1);
        __syncthreads();
      }
      // subtile it+kAhead+1 goes to the stage subtile it-1 (bf16) / it (fp8)
      // used; its DMA instructions are spread over the QK steps below
      const int s_dma = it + kAhead + 1;
      const i32x4_t dma_rs = s_dma < n_sub ? page_rsrc_of(s_dma, pg_next) : empty_rsrc();
      pg_next = tab[min((s_dma + 1) >> 1, kMaxUnitPages - 1)];
      const int dma_m0 = dma_dst(s_dma);
      dma_fence();
      const lds_u8* tile = tile_of(it);
      const lds_u8* tile_n = tile_of(it + 1);

      // ---- phase 1: QK(it+1) steps 0..kQkA-1 (one dependent chain) with
      //      the softmax of subtile it in the gaps
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; sr[r] = 0.f; }
      bf16x8_t ka[2] = {kfrag(tile_n, 0), kfrag(tile_n, 1)};
      __builtin_amdgcn_sched_barrier(0);
      carried_pv();  // subtile it's last P.V steps, under the key fragments' latency
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < kQkA; ++f) {
        sc = mfma_op<F16>(ka[f & 1], qfrag(f), sc);
        ka[f & 1] = kfrag(tile_n, f + 2);
        if (f <= 10) sm_stage(f);
        if (f == 8) asm volatile("" : "+v"(P[0]));  // keep the conversions in place
        if (f == 10) asm volatile("" : "+v"(P[1]));
        __builtin_amdgcn_sched_barrier(0);
      }
      sm_commit();

      // ---- phase 2: QK(it+1) steps kQkA..35 interleaved with the first
      //      32 - kCarry P.V steps of subtile it; the DMA of subtile it+3
      //      rides along
      bf16x8_t va[2] = {vfrag(tile, 0), vfrag(tile, 1)};
      int step = 0;
#pragma unroll
      for (int f = kQkA; f < 36; ++f) {
        if (FP8 && f >= 32) sr = mfma_op<F16>(ka[f & 1], qfrag(f), sr); else sc = mfma_op<F16>(ka[f & 1], qfrag(f), sc);
        if (f + 2 < 36) ka[f & 1] = kfrag(tile_n, f + 2);
        // 32 - kCarry P.V steps over the 36 - kQkA QK steps here: two per
        // QK step first, then one
        const int npv = (f - kQkA) < (32 - kCarry) - (36 - kQkA) ? 2 : 1;
#pragma unroll
        for (int u = 0; u < npv; ++u) {
          mfma_acc_op<F16>(acc[step & 15], va[step & 1], P[step >> 4]);
          if (step + 2 < 32 - kCarry) va[step & 1] = vfrag(tile, step + 2);
          ++step;
        }
        // the DMA group: one instruction every kDmaSp QK steps
        constexpr int kDmaSp = 36 - kQkA >= 2 * kDma ? 2 : 1;
        if ((f - kQkA) % kDmaSp == 0 && (f - kQkA) / kDmaSp < kDma)
          dma_one(dma_rs, dma_m0, s_dma, (f - kQkA) / kDmaSp, tid);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < kCarry; ++j) vc[j] = vfrag(tile, 32 - kCarry + j);
      form_scores(it + 1);
      sp = sc;
      sp_sub = it + 1;
      mask_tail(sp, nvalid_of(it + 1));
    }
    if (n_sub > 0) {  // the last subtile: softmax and P.V only
      carried_pv();  // the previous subtile's (before its P is overwritten)
      const lds_u8* tile = tile_of(n_sub - 1);
#pragma unroll
      for (int st = 0; st <= 10; ++st) sm_stage(st);
      sm_commit();
      bf16x8_t va[2] = {vfrag(tile, 0), vfrag(tile, 1)};
#pragma unroll
      for (int step = 0; step < 32; ++step) {
        mfma_acc_op<F16>(acc[step & 15], va[step & 1], P[step >> 4]);
        if (step + 2 < 32) va[step & 1] = vfrag(tile, step + 2);
      }
    }

    // ---- finalize: normalise, stage rows through LDS, store whole rows
    // (the staging overlaps the ring: the empty groups issued past the last
    // subtile complete first)
    wait_vm<0>();
    acc_fence(acc);
    // the finalize's lane indices and addresses derive from a copy of the
    // thread index the compiler cannot see through, so that they are formed
    // here: hoisted to the kernel start they live across the subtile loop
    // and are spilled to scratch
    int tf = threadIdx.x;
    asm volatile("" : "+v"(tf));
    const int wf = tf >> 6, gf = (tf >> 5) & 1, l32f = tf & 31, headf = wf * 32 + l32f;
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    const long long orow0 = ((long long)b * a.s_q + qi) * kHeads;  // first output row of this (b, qi)
    const long long prow0 = (long long)unit * R + qi * kHeads;  // partial slot = unit index
    // rows go to the output when the sequence is not split and an output is
    // given; otherwise to the unit's partial slot (a decode step passes no
    // output: its merge reads unsplit rows from there too)
    const bool to_out = final_out && a.out != nullptr;
    const bool bf16_out = to_out ? a.out_dtype != 0 : a.part_bf16 != 0;
    float* o32 = to_out ? (float*)a.out + orow0 * kDc : a.o_part + prow0 * kDc;
    uint16_t* o16 = to_out ? (uint16_t*)a.out + orow0 * kDc : (uint16_t*)a.o_part + prow0 * kDc;
    if (gf == 0) {
      if (!final_out)
        a.lse_part[prow0 + headf] = lse_v;
      else if (a.lse)
        a.lse[orow0 + headf] = lse_v;
    }
    __syncthreads();  // every wave is done with the tiles
    typedef __attribute__((address_space(3))) f32x4_t lds_f4;
    typedef __attribute__((address_space(3))) u32x2_t lds_u2;
    typedef __attribute__((address_space(3))) u32x4_t lds_u4;
    if (bf16_out) {
      // all 128 rows at once in bf16, then 16-byte stores of whole rows
      lds_u8* rowp = smem + (size_t)(wf * 32 + l32f) * kOutRowH;
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        asm volatile("" : "+a"(acc[db]));  // one block at a time
        const f32x16_t t = acc[db];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          u32x2_t pk;
          pk[0] = pack_bf16x2(t[4 * qd] * inv, t[4 * qd + 1] * inv);
          pk[1] = pack_bf16x2(t[4 * qd + 2] * inv, t[4 * qd + 3] * inv);
          *(lds_u2*)(rowp + (db * 32 + 8 * qd + 4 * gf) * 2) = pk;
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int e = tf; e < kHeads * (kDc / 8); e += 256) {
        const int r = e / (kDc / 8), c8 = e % (kDc / 8);
        const u32x4_t v = *(const lds_u4*)(smem + (size_t)r * kOutRowH + c8 * 16);
        *(u32x4_t*)(o16 + (long long)r * kDc + 8 * c8) = v;
      }
      continue;  // the next unit starts with a barrier before touching LDS
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((wf >> 1) == pass) {
        lds_u8* rowp = smem + (size_t)((wf & 1) * 32 + l32f) * kOutRowF * 4;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          asm volatile("" : "+a"(acc[db]));  // one block at a time
          const f32x16_t t = acc[db];
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            f32x4_t v;
            v[0] = t[4 * qd] * inv; v[1] = t[4 * qd + 1] * inv; v[2] = t[4 * qd + 2] * inv; v[3] = t[4 * qd + 3] * inv;
            *(lds_f4*)(rowp + (db * 32 + 8 * qd + 4 * gf) * 4) = v;
          }
        }
      }
      __syncthreads();
      // 64 staged rows (heads 64*pass ..) x 512 floats: 128 threads per row, 16 B each
#pragma unroll 4
      for (int e = tf; e < 64 * (kDc / 4); e += 256) {
        const int r = e / (kDc / 4), c4 = e % (kDc / 4);
        const f32x4_t v = *(const lds_f4*)(smem + ((size_t)r * kOutRowF + 4 * c4) * 4);
        const long long row = 64 * pass + r;
        *(float4*)(o32 + row * kDc + 4 * c4) = make_float4(v[0], v[1], v[2], v[3]);
      }
      __syncthreads();
    }
  }
}

template <int FMT>
static hipError_t launch_pipe(const DecodeArgs& a, int grid_x, hipStream_t s) {
  static std::atomic<uint64_t> lds_raised{0};
  if (const hipError_t e = ensure_dynamic_lds((const void*)decode_pipe_kernel<FMT>, kPipeLds(FMT), lds_raised);
      e != hipSuccess)
    return e;
  hipLaunchKernelGGL(decode_pipe_kernel<FMT>, dim3(grid_x, a.s_q), dim3(256), kPipeLds(FMT), s, a);
  return hipGetLastError();
}

// kv dtype codes: 1 bf16, 2 fp8, 3 int4, 4 int2
hipError_t launch_decode_mfma(const DecodeArgs& a, int grid_x, hipStream_t s) {
  switch (a.kv_dtype) {
    case 2: return launch_pipe<kFmtFp8>(a, grid_x, s);
    case 3: return launch_pipe<kFmtInt4>(a, grid_x, s);
    case 4: return launch_pipe<kFmtInt2>(a, grid_x, s);
    default: return launch_pipe<kFmtBf16>(a, grid_x, s);
  }
}

int mfma_max_unit_pages() { return kMaxUnitPages; }

}  // namespace mla
