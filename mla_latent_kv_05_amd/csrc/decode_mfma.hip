// Split-KV MFMA decode kernel for the DeepSeek-V2/V3 shape of absorbed MLA:
// n_h = 128 query heads sharing one latent cache row [c^KV 512 | k^R 64]
// (itwiki "Multi-head latent attention": sections "Decoupled RoPE", "Matrix
// absorption", and the V2/V3 dimension table), 64-token pages, bf16 or
// fp8-e4m3 content.  The itwiki page's "Implementation" section notes that
// this shape (576-wide keys, 512-wide values shared by 128 heads) needs a
// dedicated kernel.
//
// Work decomposition
//   * grid.x = persistent workgroups looping over planned units (sequence,
//     contiguous page range); grid.y = query token i of the sequence.
//   * 4 wavefronts, one per SIMD; wavefront w owns heads 32w .. 32w+31 for
//     both contractions, so P never leaves registers.
//   * The unit's keys stream through LDS in 32-token subtiles (36,864 B of
//     bf16 rows), loaded with 16-byte global->LDS DMA into kStages buffers.
//   * S^T[token, head] = K[token, 0:576] . Q^T on v_mfma_f32_32x32x16_bf16
//     (A = key rows from LDS via ds_read_b128, B = queries held in VGPRs).
//   * O^T[dim, head] += V^T[dim, token] . P^T[token, head]: A = c^KV columns
//     fetched transposed with ds_read_tr16_b64, B = P taken straight from the
//     S^T accumulator layout (each lane owns one head in both products).
//   * Online softmax in base 2 with lazy rescaling: the running reference
//     max only moves when a subtile's max exceeds it by more than kTau, so the
//     256-register accumulator is rarely touched outside the MFMAs.  The
//     result is exact: numerator and denominator share the reference.
//   * fp8 content: codes are DMA'd to a staging area and expanded to the
//     bf16 tile layout (e4m3 -> bf16 is exact); the per-token scale is folded
//     into the content score and into P before the P.V product.
//
// LDS tile layout: row t (token) is 1152 B = 72 chunks of 16 B; logical chunk
// c is stored at chunk (c & ~7) | ((c ^ f(t)) & 7), f(t) = ((t&3)<<1)|((t>>2)&1),
// which keeps both the 8-row b128 reads of the QK step and the 4-row
// transposed reads of the PV step free of bank conflicts.
#include "mfma_common.h"

namespace mla {

template <bool FP8>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  lds_i32* tab = (lds_i32*)(smem + kTabOff(FP8));

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  const int qi = blockIdx.y;
  const int R = a.s_q * kHeads;
  const int head = w * 32 + l32;
  const int n_units = ((const WsHeader*)a.ws_header)->n_units;
  const float scale2 = a.scale * kLog2e;

  // ---- lane-constant LDS offsets
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
  // DMA source offsets of this lane within a bf16 subtile (LDS chunk -> global chunk)
  // (16-bit pairs: offsets are < 36864)
  uint32_t goff2[(kBf16Dma + 1) / 2];
#pragma unroll
  for (int i = 0; i < (kBf16Dma + 1) / 2; ++i) goff2[i] = 0;
#pragma unroll
  for (int i = 0; i < kBf16Dma; ++i) {
    const int p = (i * 4 + w) * 64 + lane;
    const int t = p / 72, cp = p - t * 72;
    const int c = (cp & ~7) | ((cp ^ swz_f(t)) & 7);
    goff2[i >> 1] |= (uint32_t)(t * kRowB + c * 16) << (16 * (i & 1));
  }

  for (int unit = xcd_slot(blockIdx.x, gridDim.x); unit < n_units; unit += gridDim.x) {
    const int4 wk = a.work[unit];
    const int b = wk.x;
    const int L = a.seq_lens[b];
    const int vis = L - a.s_q + qi + 1;
    const int tok0 = wk.y * kBlk;
    const int tok1 = min(wk.z * kBlk, vis);
    const int ntok = tok1 - tok0;
    const int n_sub = ntok > 0 ? (ntok + kSub - 1) / kSub : 0;
    const int n_last = ntok - (n_sub - 1) * kSub;  // valid rows of the last subtile

    __syncthreads();  // previous unit finished with LDS
    {
      const int npg = (n_sub * kSub + kBlk - 1) / kBlk;
      const int32_t* trow = a.table + (long long)b * a.max_blocks + wk.y;
      for (int i = tid; i < npg; i += 256) tab[i] = trow[i];
    }
    // queries of this lane's head: B operand slots (l/32)*8 .. +7 of each 16-dim k-block.
    // The fp8 path keeps the RoPE slice in LDS (its extra score accumulator
    // needs those registers).
    constexpr int kQReg = FP8 ? 32 : 36;
    bf16x8_t q[kQReg];
    lds_u8* qr_lds = smem + kQrOff(FP8);
    {
      const long long qrow = ((long long)b * a.s_q + qi) * kHeads + head;
      const bf16x8_t* ql = (const bf16x8_t*)((const uint16_t*)a.q_lat + qrow * kDc);
      const bf16x8_t* qr = (const bf16x8_t*)((const uint16_t*)a.q_rope + qrow * kDr);
#pragma unroll
      for (int kb = 0; kb < 32; ++kb) q[kb] = ql[2 * kb + g];
      if (FP8) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          *(__attribute__((address_space(3))) bf16x8_t*)(qr_lds + head * kQrStride + (2 * kb + g) * 16) =
              qr[2 * kb + g];
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) q[kQReg - 4 + kb] = qr[2 * kb + g];
      }
    }
    wait_vm<0>();
    __syncthreads();  // page ids visible

    auto issue = [&](int s) {
      const int pg = __builtin_amdgcn_readfirstlane(tab[s >> 1]);
      const uint8_t* blk = (const uint8_t*)a.kv + (long long)pg * a.block_bytes;
      const int half = s & 1;
      if (!FP8) {
        lds_u8* dst = smem + (s % kStages) * kTileB + w * 1024;
        const i32x4_t rs = make_rsrc(blk + half * kTileB);
#pragma unroll
        for (int i = 0; i < kBf16Dma; ++i) dma16(rs, (int)((goff2[i >> 1] >> (16 * (i & 1))) & 0xffffu), dst + i * 4096);
      } else {
        lds_u8* dst = smem + (s % kStages) * kF8Stage;
        const i32x4_t rs = make_rsrc(blk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dma16(rs, half * kF8Codes + ((i * 4 + w) * 64 + lane) * 16, dst + (i * 4 + w) * 1024);
        dma16(rs, kBlk * kDc + half * kF8Kr + (w * 64 + lane) * 16, dst + kF8Codes + w * 1024);
        // every wave issues the (identical) scale load so all waves count kF8Dma per subtile
        if (lane < 8)
          dma16(rs, kBlk * (kDc + 2 * kDr) + half * (kSub * 4) + lane * 16, dst + kF8Codes + kF8Kr);
      }
    };

    f32x16_t acc[16];
#pragma unroll
    for (int d = 0; d < 16; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
    acc_fence(acc);
    float m_run = -INFINITY, l_run = 0.f;

    // prologue
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < n_sub) issue(s);

    for (int it = 0; it < n_sub; ++it) {
      const int outstanding = min(kStages - 2, n_sub - 1 - it);
      if (FP8) wait_groups<kF8Dma>(outstanding); else wait_groups<kBf16Dma>(outstanding);
      __syncthreads();
      if (it + kStages - 1 < n_sub) issue(it + kStages - 1);
      const bool ragged = (it == n_sub - 1) && (n_last < kSub);
      const int nvalid = ragged ? n_last : kSub;

      lds_u8* tile;
      if (!FP8) {
        tile = smem + (it % kStages) * kTileB;
        if (ragged) {  // zero the value rows past the end (they may hold NaN)
          for (int e = tid; e < (kSub - nvalid) * 72; e += 256) {
            const int t = nvalid + e / 72, c = e % 72;
            *(__attribute__((address_space(3))) u32x4_t*)(tile + t * kRowB + c * 16) = u32x4_t{0, 0, 0, 0};
          }
          __syncthreads();
        }
      } else {
        const lds_u8* st = smem + (it % kStages) * kF8Stage;
        tile = smem + kStages * kF8Stage;
#pragma unroll 1
        for (int i = 0; i < 8; ++i) {
          const int qd = tid + 256 * i;
          const int t = qd >> 6, c = qd & 63;
          u32x4_t o = {0, 0, 0, 0};
          if (t < nvalid) {
            const u32x2_t cw = *(const __attribute__((address_space(3))) u32x2_t*)(st + t * kDc + c * 8);
            o[0] = fp8x2_to_bf16x2<false>(cw[0]);
            o[1] = fp8x2_to_bf16x2<true>(cw[0]);
            o[2] = fp8x2_to_bf16x2<false>(cw[1]);
            o[3] = fp8x2_to_bf16x2<true>(cw[1]);
          }
          *(__attribute__((address_space(3))) u32x4_t*)(tile + t * kRowB + (((c & ~7) | ((c ^ swz_f(t)) & 7)) << 4)) = o;
        }
        {
          const int t = tid >> 3, cc = tid & 7;
          const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(st + kF8Codes + t * 128 + cc * 16);
          *(__attribute__((address_space(3))) u32x4_t*)(tile + t * kRowB + ((64 + (cc ^ swz_f(t))) << 4)) = v;
        }
        __syncthreads();
      }

      // ---- S^T = K . Q^T  (rolling prefetch: fragment j of the next 4-step
      //      group is requested as soon as the MFMA consuming slot j issues)
      f32x16_t sc, sr;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sc[r] = 0.f; sr[r] = 0.f; }
      {
        const lds_u8* pk[4] = {tile + off_qk[0], tile + off_qk[1], tile + off_qk[2], tile + off_qk[3]};
        bf16x8_t ka[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ka[j] = lds_b128(pk[j]);
#pragma unroll
        for (int k4 = 0; k4 < 9; ++k4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (FP8 && k4 >= 8)
              sr = mfma(ka[j], lds_b128(qr_lds + head * kQrStride + (2 * j + g) * 16), sr);
            else
              sc = mfma(ka[j], q[(4 * k4 + j) % kQReg], sc);
            if (k4 < 8) ka[j] = lds_b128(pk[j] + (k4 + 1) * 128);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---- scores, mask, online softmax (lane: head, 16 tokens 8(r/4)+4g+r%4)
      // fp8: per-token scales of this lane's tokens, 4 groups of 4 consecutive
      const lds_u8* scl = smem + (it % kStages) * kF8Stage + kF8Codes + kF8Kr + 16 * g;
      auto token_scale = [&](int qd) {
        return *(const __attribute__((address_space(3))) f32x4_t*)(scl + 32 * qd);
      };
      float s[16];
      float mx = -INFINITY;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        f32x4_t ts;
        if (FP8) ts = token_scale(qd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * qd + e;
          const int t = 8 * qd + 4 * g + e;
          float v = FP8 ? (sc[r] * ts[e] + sr[r]) : sc[r];
          v *= scale2;
          if (ragged && t >= nvalid) v = -INFINITY;
          s[r] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = half_swap_max(mx);
      if (m_run == -INFINITY) {
        m_run = mx;  // first subtile: the accumulator is still zero
      } else if (mx > m_run + kTau) {
        const float f = __builtin_amdgcn_exp2f(m_run - mx);
        l_run *= f;
        acc_fence(acc);
#pragma unroll
        for (int d = 0; d < 16; ++d) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[d][r] *= f;
          asm volatile("" : "+a"(acc[d]));  // back to AGPRs block by block
        }
        acc_fence(acc);
        m_run = mx;
      }
      float ps = 0.f;
      bf16x8_t P[2];
      if (FP8) asm volatile("" ::: "memory");  // re-read the token scales instead of keeping 16 live
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        f32x4_t ts;
        if (FP8) ts = token_scale(qd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * qd + e;
          float p = __builtin_amdgcn_exp2f(s[r] - m_run);
          ps += p;
          if (FP8) {
            const int t = 8 * qd + 4 * g + e;
            p = (ragged && t >= nvalid) ? 0.f : p * ts[e];  // masked rows may hold any scale
          }
          P[r >> 3][r & 7] = (__bf16)p;
        }
      }
      l_run += ps;

      // ---- O^T += V^T . P^T  (rolling prefetch of the transposed value reads)
      {
        auto load_v = [&](int db, int ks) {
          const int kofs = (db >> 1) * 128 + ks * 16 * kRowB;
          const bf16x4_t lo = lds_tr16(tile + off_pv[db & 1][0] + kofs);
          const bf16x4_t hi = lds_tr16(tile + off_pv[db & 1][1] + kofs);
          bf16x8_t v;
          v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
          v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
          return v;
        };
        bf16x8_t va[2] = {load_v(0, 0), load_v(0, 1)};
#pragma unroll
        for (int db = 0; db < 16; ++db) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            mfma_acc(acc[db], va[ks], P[ks]);
            if (db < 15) va[ks] = load_v(db + 1, ks);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ---- finalize this unit
    acc_fence(acc);
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    const long long orow = ((long long)b * a.s_q + qi) * kHeads + head;
    const bool final_out = wk.w < 0;
    const long long prow = (long long)wk.w * R + qi * kHeads + head;
    // fp32 rows: the partial slot or an fp32 output; bf16 output otherwise
    const bool bf16_out = final_out && a.out_dtype != 0;
    float* o32 = final_out ? (float*)a.out + orow * kDc : a.o_part + prow * kDc;
    uint16_t* o16 = (uint16_t*)a.out + orow * kDc;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      asm volatile("" : "+a"(acc[db]));  // read one block at a time
      const f32x16_t t = acc[db];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = db * 32 + 8 * qd + 4 * g;
        const float v0 = t[4 * qd] * inv, v1 = t[4 * qd + 1] * inv;
        const float v2 = t[4 * qd + 2] * inv, v3 = t[4 * qd + 3] * inv;
        if (bf16_out) {
          uint2 pk;
          pk.x = f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
          pk.y = f32_to_bf16_bits(v2) | ((uint32_t)f32_to_bf16_bits(v3) << 16);
          *(uint2*)(o16 + d0) = pk;
        } else {
          *(float4*)(o32 + d0) = make_float4(v0, v1, v2, v3);
        }
      }
    }
    if (g == 0) {
      if (!final_out)
        a.lse_part[prow] = lse_v;
      else if (a.lse)
        a.lse[orow] = lse_v;
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int grid_x, hipStream_t s) {
  if (a.kv_dtype != 2) return launch_decode_bf16(a, grid_x, s);
  if (a.kv_dtype == 2) return launch_decode_fp8(a, grid_x, s);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_mfma_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes(true));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(grid_x, a.s_q), dim3(256), kLdsBytes(true), s, a);
  return hipGetLastError();
}

int mfma_max_unit_pages() { return kMaxUnitPages; }

}  // namespace mla
