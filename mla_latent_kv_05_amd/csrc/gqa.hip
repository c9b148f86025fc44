// GQLA's GQA decode path (chatpaper page on GQLA, abstract): the same weights
// as the MQA-absorb path, decoded over a cache expanded per group of heads,
//   s_{i,h,j} = scale * (q^C_{i,h} . k^C_{j,g(h)} + q^R_{i,h} . k^R_j),  j <= L - s_q + i
//   o_{i,h}   = sum_j softmax_j(s) v^C_{j,g(h)},   g(h) = h / (n_h / n_g),
// with the RoPE key shared by all groups.  Paged cache, per block of
// block_size tokens: [n_g][bs][d_h] k^C | [n_g][bs][d_h] v^C | [bs][d_r] k^R.
//
// MFMA kernel (bf16, d_h = 128, d_r = 64, 64-token blocks, s_q * n_h / n_g =
// 32 query rows per group): a workgroup takes one (sequence, group); its 32
// rows (query token i, head of the group) are the N = 32 of
// v_mfma_f32_32x32x16_bf16, so every wave holds all of them and the 4 waves
// split the keys into 4 contiguous ranges, each with its own online softmax,
// merged through LDS at the end.  Each wave streams its 32-key subtiles
// (content keys, RoPE keys, values: 20 KB) by 16-byte global->LDS DMA into
// a private 2-stage ring, so the loop needs no workgroup barrier; the LDS
// layout and swizzles are those of the prefill kernel (S^T = K.Q^T in 12
// MFMAs, O^T += V^T.P^T in 8 with transposed value reads).  HBM-bound:
// (2 d_h + d_r) * 2 bytes per token and group (the RoPE key re-read by each
// group's workgroup comes from L2: the groups of a sequence share an XCD).
#include <type_traits>

#include "mfma_common.h"

namespace mla {

namespace {

constexpr int kGqDh = 128, kGqDr = 64, kGqDq = kGqDh + kGqDr;
constexpr int kGqRows = 32;                      // s_q x heads per group
constexpr int kGqSub = 32;                       // keys per subtile (half a 64-token block)
constexpr int kGqBlk = 64;
constexpr int kGqKcB = kGqSub * kGqDh * 2;       // 8192
constexpr int kGqKrB = kGqSub * kGqDr * 2;       // 4096
constexpr int kGqVB = kGqSub * kGqDh * 2;        // 8192
constexpr int kGqStage = kGqKcB + kGqKrB + kGqVB;  // 20480
constexpr int kGqRing = 2;                       // stages per wave
constexpr int kGqLds = 4 * kGqRing * kGqStage;   // 163840
constexpr int kGqDma = 20;                       // DMA instructions per wave per subtile
constexpr float kGqTau = 8.f;

__device__ __forceinline__ int gq_f16(int t) { return 4 * (t & 3) + ((t >> 2) & 3); }
__device__ __forceinline__ int gq_f8(int t) { return (t >> 1) & 7; }

}  // namespace

__global__ __launch_bounds__(256, 1) void gqa_decode_mfma_kernel(const uint16_t* q_c, const uint16_t* q_r,
                                                                 const uint8_t* cache, const int32_t* table,
                                                                 int max_blocks, const int32_t* seq_lens, int n_h,
                                                                 int n_g, int s_q, long long block_bytes,
                                                                 float scale2, void* out, float* lse,
                                                                 int out_bf16) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  const int w_s = __builtin_amdgcn_readfirstlane(w);
  // the n_g groups of a sequence are consecutive workgroups of one XCD
  // (round-robin dealing: workgroup id = 8k + x sits on XCD x)
  int b, grp;
  {
    const int n_wg = gridDim.x;
    const int lin = (n_wg & 7) ? (int)blockIdx.x : (blockIdx.x & 7) * (n_wg >> 3) + (blockIdx.x >> 3);
    b = lin / n_g;  // this workgroup's rank in (sequence, group) order
    grp = lin % n_g;
  }
  const int L = seq_lens[b];
  const int hpg = n_h / n_g;
  // this lane's query row: token i = l32 / hpg, head grp * hpg + l32 % hpg
  const int qi = l32 / hpg, head = grp * hpg + l32 % hpg;
  const long long qrow = ((long long)b * s_q + qi) * n_h + head;
  bf16x8_t qf[kGqDq / 16];
#pragma unroll
  for (int f = 0; f < 8; ++f) qf[f] = *(const bf16x8_t*)(q_c + qrow * kGqDh + 16 * f + 8 * g);
#pragma unroll
  for (int f = 8; f < 12; ++f) qf[f] = *(const bf16x8_t*)(q_r + qrow * kGqDr + 16 * (f - 8) + 8 * g);

  // this wave's contiguous share of the subtiles
  const int n_tot = (L + kGqSub - 1) / kGqSub;
  const int s_begin = (w_s * n_tot) >> 2, s_end = ((w_s + 1) * n_tot) >> 2;
  const int32_t* trow = table + (long long)b * max_blocks;
  const int lds_w = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(smem + w_s * kGqRing * kGqStage));
  const long long grp_off = (long long)grp * kGqBlk * kGqDh * 2;
  const long long v_off = (long long)n_g * kGqBlk * kGqDh * 2;
  const long long kr_off = 2 * v_off;
  // DMA of subtile s into ring slot `slot`: instruction i moves 64 chunks of
  // a region (content keys i = 0..7, values 8..15, RoPE keys 16..19); the
  // lane's chunk p = (i % 8) * 64 + lane lands at LDS chunk p of the region,
  // fetched from the row's logical chunk that the swizzle puts there.  Rows
  // past the sequence end read its last row (finite; their scores are masked).
  auto issue = [&](int s, int slot) {
    const int pg = __builtin_amdgcn_readfirstlane(trow[s >> 1]);
    const uint8_t* blk = cache + (long long)pg * block_bytes;
    const int half = s & 1, last = L - 1 - s * kGqSub;
    const i32x4_t rk = make_rsrc(blk + grp_off + half * kGqKcB);
    const i32x4_t rv = make_rsrc(blk + v_off + grp_off + half * kGqVB);
    const i32x4_t rr = make_rsrc(blk + kr_off + half * kGqKrB);
    const int m0b = lds_w + slot * kGqStage;
    dma_fence();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i * 4 + (lane >> 4);
      const int src = min(t, last) * (kGqDh * 2) + (((lane & 15) ^ gq_f16(t)) << 4);
      dma16_m0_stream(rk, src, m0b + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i * 4 + (lane >> 4);
      const int src = min(t, last) * (kGqDh * 2) + (((lane & 15) ^ gq_f16(t)) << 4);
      dma16_m0_stream(rv, src, m0b + kGqKcB + kGqKrB + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = i * 8 + (lane >> 3);
      const int src = min(t, last) * (kGqDr * 2) + (((lane & 7) ^ gq_f8(t)) << 4);
      dma16_m0(rr, src, m0b + kGqKcB + i * 1024);
    }
  };

  int off_kc[8], off_kr[4];
#pragma unroll
  for (int f = 0; f < 8; ++f) off_kc[f] = l32 * (kGqDh * 2) + ((2 * f + g) ^ gq_f16(l32)) * 16;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) off_kr[bb] = kGqKcB + l32 * (kGqDr * 2) + ((2 * bb + g) ^ gq_f8(l32)) * 16;
  int off_pv[4][2];
  {
    const int ta = 4 * g + (j16 >> 2);
    const int clo = 2 * (G & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int t = ta + 8 * hh;
        off_pv[d][hh] = kGqKcB + kGqKrB + t * (kGqDh * 2) + ((4 * d + clo) ^ gq_f16(t)) * 16 + (j16 & 1) * 8;
      }
  }

  f32x16_t acc[kGqDh / 32];
#pragma unroll
  for (int d = 0; d < kGqDh / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  // a finite floor for the reference max: a wave's key range can hold no
  // visible key for the first query token's rows (its subtile starts past
  // L - s_q), and exp2(score - floor) of masked scores is still 0
  float m_run = -1e30f, l_run = 0.f;
  const int vis_last = L - s_q + qi;  // this row's last visible key

  auto step = [&](int s, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    if (s + 1 < s_end)
      wait_vm<kGqDma>();  // subtile s landed (s + 1 may still be in flight)
    else
      wait_vm<0>();
    const lds_u8* tile = smem + (w_s * kGqRing + SLOT) * kGqStage;
    f32x16_t sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int f = 0; f < kGqDq / 16; ++f) {
      const bf16x8_t ka = f < 8 ? lds_b128(tile + off_kc[f]) : lds_b128(tile + off_kr[f & 3]);
      sc = mfma(ka, qf[f], sc);
    }
    const int j0 = s * kGqSub;
    if (j0 + kGqSub - 1 > L - s_q) {  // scalar branch: the subtile reaches the causal edge or the end
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key > vis_last) sc[r] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = half_swap_max(mx) * scale2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kGqTau)) {  // lazy reference max
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int d = 0; d < kGqDh / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= corr;
      m_run = m_new;
    }
    float ps = 0.f;
    bf16x8_t P[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], scale2, -m_run));
      ps += p;
      P[r >> 3][r & 7] = (__bf16)p;
    }
    l_run += half_swap_sum(ps);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < kGqDh / 32; ++d) {
        const lds_u8* p0 = tile + ks * 16 * (kGqDh * 2);
        const bf16x4_t lo = lds_tr16(p0 + off_pv[d][0]);
        const bf16x4_t hi = lds_tr16(p0 + off_pv[d][1]);
        bf16x8_t va;
        va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
        va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
        acc[d] = mfma(va, P[ks], acc[d]);
      }
    // the slot is free again once its reads have returned; the subtile two
    // ahead goes there
    if (s + 2 < s_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
      issue(s + 2, SLOT);
    }
  };
  wait_vm<0>();  // the query loads are complete before the first DMA
  if (s_begin < s_end) issue(s_begin, 0);
  if (s_begin + 1 < s_end) issue(s_begin + 1, 1);
  for (int s = s_begin; s < s_end; s += kGqRing) {
    step(s, std::integral_constant<int, 0>{});
    if (s + 1 < s_end) step(s + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge the 4 waves: (m, l) per row and O^T in LDS, then each thread
  // finishes 16 dims of one row
  __syncthreads();  // every wave is done with its ring
  float* mrg = (float*)smem_raw;                      // [4][32] m, [4][32] l
  float* ob = (float*)(smem_raw + 1024);              // [4][32 rows][128 + 4]
  constexpr int kRowF = kGqDh + 4;
  if (g == 0) {
    mrg[w * 32 + l32] = m_run;
    mrg[128 + w * 32 + l32] = l_run;
  }
#pragma unroll
  for (int d = 0; d < kGqDh / 32; ++d)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int dim = 32 * d + 8 * qd + 4 * g;
      *(__attribute__((address_space(3))) f32x4_t*)((lds_u8*)(ob + (w * 32 + l32) * kRowF + dim)) =
          f32x4_t{acc[d][4 * qd], acc[d][4 * qd + 1], acc[d][4 * qd + 2], acc[d][4 * qd + 3]};
    }
  __syncthreads();
  {
    const int row = tid >> 3, d0 = (tid & 7) * 16;
    float mw[4], M = -1e30f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mw[k] = mrg[k * 32 + row];
      M = fmaxf(M, mw[k]);
    }
    float wt[4], Lt = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wt[k] = __builtin_amdgcn_exp2f(mw[k] - M);  // 0 for a wave that saw none of this row's keys
      Lt += wt[k] * mrg[128 + k * 32 + row];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    const int ri = row / hpg, rh = grp * hpg + row % hpg;
    const long long orow = ((long long)b * s_q + ri) * n_h + rh;
    float o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4_t v = *(const __attribute__((address_space(3))) f32x4_t*)((const lds_u8*)(ob + (k * 32 + row) * kRowF + d0 + 4 * e4));
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * e4 + e] += wt[k] * v[e];
      }
    if (out_bf16) {
      u32x4_t pk[2];
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e >> 2][e & 3] = pack_bf16x2(o[2 * e] * inv, o[2 * e + 1] * inv);
      *(u32x4_t*)((uint16_t*)out + orow * kGqDh + d0) = pk[0];
      *(u32x4_t*)((uint16_t*)out + orow * kGqDh + d0 + 8) = pk[1];
    } else {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *(f32x4_t*)((float*)out + orow * kGqDh + d0 + 4 * e4) =
            f32x4_t{o[4 * e4] * inv, o[4 * e4 + 1] * inv, o[4 * e4 + 2] * inv, o[4 * e4 + 3] * inv};
    }
    if (lse && (tid & 7) == 0) lse[orow] = Lt > 0.f ? (M + __log2f(Lt)) * kLn2 : -INFINITY;
  }
}

// Portable kernel: one wave per (sequence, query token, head), keys one at a
// time with an exact online softmax in fp32; lanes split the dimensions.
constexpr int kGqMaxD = 4;  // d_h and d_h + d_r up to 256
__global__ __launch_bounds__(256) void gqa_decode_generic_kernel(const void* q_c, const void* q_r,
                                                                 const uint8_t* cache, const int32_t* table,
                                                                 int max_blocks, const int32_t* seq_lens, int B,
                                                                 int s_q, int n_h, int n_g, int d_h, int d_r,
                                                                 int bs, long long block_bytes, float scale,
                                                                 int q_dt, int kv_dt, void* out, float* lse,
                                                                 int out_dt) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * s_q + i) * n_h + h
  if (row >= (long long)B * s_q * n_h) return;
  const int h = (int)(row % n_h), i = (int)((row / n_h) % s_q), b = (int)(row / ((long long)n_h * s_q));
  const int grp = h / (n_h / n_g);
  const int L = seq_lens[b], vis = L - s_q + i + 1;
  const int dq = d_h + d_r;
  float qv[kGqMaxD], acc[kGqMaxD];
#pragma unroll
  for (int k = 0; k < kGqMaxD; ++k) {
    const int e = lane + 64 * k;
    qv[k] = e < d_h ? load_elem(q_c, row * d_h + e, q_dt) : e < dq ? load_elem(q_r, row * d_r + (e - d_h), q_dt) : 0.f;
    acc[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < vis; ++j) {
    const uint8_t* blk = cache + (long long)table[(long long)b * max_blocks + j / bs] * block_bytes;
    const int t = j % bs;
    const long long kc_e = ((long long)grp * bs + t) * d_h;       // element offsets within the block
    const long long v_e = (long long)n_g * bs * d_h + kc_e;
    const long long kr_e = 2LL * n_g * bs * d_h + (long long)t * d_r;
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < kGqMaxD; ++k) {
      const int e = lane + 64 * k;
      float kv = 0.f;
      if (e < d_h)
        kv = load_elem(blk, kc_e + e, kv_dt);
      else if (e < dq)
        kv = load_elem(blk, kr_e + (e - d_h), kv_dt);
      part += qv[k] * kv;
    }
    const float s = wave_sum(part) * scale;
    const float m_new = fmaxf(m, s);
    const float c = __expf(m - m_new), p = __expf(s - m_new);
    l = l * c + p;
#pragma unroll
    for (int k = 0; k < kGqMaxD; ++k) {
      const int e = lane + 64 * k;
      acc[k] = acc[k] * c + (e < d_h ? p * load_elem(blk, v_e + e, kv_dt) : 0.f);
    }
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int k = 0; k < kGqMaxD; ++k) {
    const int e = lane + 64 * k;
    if (e < d_h) store_elem(out, row * d_h + e, acc[k] * inv, out_dt);
  }
  if (lse && lane == 0) lse[row] = l > 0.f ? m + __logf(l) : -INFINITY;
}

bool gqa_mfma_eligible(int s_q, int n_h, int n_g, int d_h, int d_r, int bs, int q_dt, int kv_dt) {
  return q_dt == 1 && kv_dt == 1 && d_h == kGqDh && d_r == kGqDr && bs == kGqBlk && n_g > 0 && n_h % n_g == 0 &&
         s_q * (n_h / n_g) == kGqRows;
}

hipError_t launch_gqa_decode(const void* q_c, const void* q_r, const void* cache, const int32_t* table,
                             int max_blocks, const int32_t* seq_lens, int B, int s_q, int n_h, int n_g, int d_h,
                             int d_r, int bs, long long block_bytes, float scale, int q_dt, int kv_dt, void* out,
                             float* lse, int out_dt, bool mfma, hipStream_t s) {
  if (mfma) {
    static std::atomic<uint64_t> lds_raised{0};
    if (const hipError_t e = ensure_dynamic_lds((const void*)gqa_decode_mfma_kernel, kGqLds, lds_raised);
        e != hipSuccess)
      return e;
    const long long n_wg = (long long)B * n_g;  // one workgroup per (sequence, group)
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gqa_decode_mfma_kernel, dim3((unsigned)n_wg), dim3(256), kGqLds, s, (const uint16_t*)q_c,
                       (const uint16_t*)q_r, (const uint8_t*)cache, table, max_blocks, seq_lens, n_h, n_g, s_q,
                       block_bytes, scale * kLog2e, out, lse, out_dt == 1 ? 1 : 0);
  } else {
    const long long rows = (long long)B * s_q * n_h;
    hipLaunchKernelGGL(gqa_decode_generic_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, q_c, q_r,
                       (const uint8_t*)cache, table, max_blocks, seq_lens, B, s_q, n_h, n_g, d_h, d_r, bs,
                       block_bytes, scale, q_dt, kv_dt, out, lse, out_dt);
  }
  return hipGetLastError();
}

}  // namespace mla
