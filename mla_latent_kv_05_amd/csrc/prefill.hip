// MHA-mode prefill attention (itwiki "Multi-head latent attention": sections
// "Decoupled RoPE" and "Matrix absorption"; the article's implementation
// example runs prefill in MHA mode): per head i and query t,
//   o_{t,i} = sum_{j<=t} softmax_j(scale * (q^C_{t,i}.k^C_{j,i} + q^R_{t,i}.k^R_j)) v^C_{j,i}
// with the RoPE key k^R shared by all heads.  Keys and values are the
// materialised k^C = W^UK c^KV, v^C = W^UV c^KV (the expansion runs in the
// up-projection kernel with one latent row per token feeding every head).
//
// MFMA kernel (bf16, d_h = 128, d_r = 64): a workgroup of 4 waves takes one
// head and 128 query rows, wave w rows 32w .. 32w+31.  Keys stream through a
// 2-stage LDS ring in 32-key subtiles (content keys, RoPE keys and values in
// three swizzled regions), filled by 16-byte global->LDS DMA one subtile
// ahead; one barrier per subtile.  40 KB of LDS and at most 168 registers
// per lane let three workgroups share a compute unit (three waves per SIMD
// hide each other's softmax and DMA waits).  Per subtile and wave:
//   S^T[key, query] = K[key, 0:192] . Q^T  (12 v_mfma_f32_32x32x16_bf16; A =
//                     key rows by ds_read_b128, B = the queries in registers)
//   online softmax per query (the lane is the query; exp2 domain, lazy
//                     reference max), causal mask only where the subtile
//                     reaches the wave's diagonal or the end of the sequence
//   O^T[dim, query] += V^T[dim, key] . P^T[key, query]  (8 MFMAs; A = value
//                     columns by ds_read_b64_tr_b16, B = P from the S layout)
// Workgroups are dealt to the 8 XCDs so that all query blocks of a head run
// on one XCD (its L2 keeps that head's keys and values), in windows of a few
// heads with the longest query blocks first.
#include <type_traits>

#include "mfma_common.h"

namespace mla {

namespace {

constexpr int kPfDh = 128, kPfDr = 64, kPfDq = kPfDh + kPfDr;  // 192
constexpr int kPfQ = 128;                                     // query rows per workgroup
constexpr int kPfSub = 32;                                    // keys per subtile
constexpr int kPfKcB = kPfSub * kPfDh * 2;                     // 8192: content keys, 256-byte rows
constexpr int kPfKrB = kPfSub * kPfDr * 2;                     // 4096: RoPE keys, 128-byte rows
constexpr int kPfVB = kPfSub * kPfDh * 2;                      // 8192: values, 256-byte rows
constexpr int kPfStage = kPfKcB + kPfKrB + kPfVB;              // 20480
constexpr int kPfRing = 2;
constexpr int kPfDma = 5;                                      // DMA instructions per thread per subtile
constexpr float kPfTau = 8.f;                                  // lazy-max slack (log2 units)
// heads per scheduling window: inside a window the query blocks go longest
// first, so the last workgroups dealt are short ones (one head per window
// left its longest block running alone at the end: 710 -> 673 us at 4096
// tokens x 128 heads); 8 heads beat 4 and 16, whose wider key/value working
// set raises the L2 misses
constexpr int kPfWin = 8;

// LDS swizzles (64 banks of 4 bytes: a 256-byte line per cycle).  Content
// key and value rows are 256 bytes (16 chunks of 16 bytes): chunk c of row t
// sits at c ^ f16(t).  f16 is a bijection on the row's low 4 bits, so 16
// consecutive rows reading one logical chunk (ds_read_b128) hit 16 different
// chunk positions, and rows 4a .. 4a+3 get distinct values of bits 2-3, so
// the transposed value reads (4 rows x 4 adjacent chunks per 32 lanes) cover
// all 16 positions too.  RoPE key rows are 128 bytes (two per line): chunk c
// of row t sits at c ^ ((t >> 1) & 7).
__device__ __forceinline__ int pf_f16(int t) { return 4 * (t & 3) + ((t >> 2) & 3); }
__device__ __forceinline__ int pf_f8(int t) { return (t >> 1) & 7; }

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void prefill_mfma_kernel(const uint16_t* q, const uint16_t* kc,
                                                           const uint16_t* kr, const uint16_t* v, void* out,
                                                           float* lse, int T, int n_h, int nqb, float scale2,
                                                           int out_bf16) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[kPfRing * kPfStage];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  // XCD-aware work item: XCD x owns heads x, x + 8, ...; its k-th workgroup
  // takes them in windows of kPfWin heads, and inside a window the query
  // blocks longest first across the window's heads
  int h, qblk;
  {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int hpx = (n_h + 7) >> 3;  // heads per XCD
    const int win = k / (kPfWin * nqb), r = k - win * (kPfWin * nqb);
    const int wh = min(kPfWin, hpx - win * kPfWin);  // heads in this window
    qblk = nqb - 1 - r / wh;
    h = (win * kPfWin + r % wh) * 8 + x;
  }
  if (h >= n_h) return;  // the grid is padded to a multiple of 8 heads
  const int w_s = __builtin_amdgcn_readfirstlane(w);
  const int qb = qblk * kPfQ;
  const int q0 = qb + 32 * w_s;  // this wave's first query (scalar)
  const int qrow = q0 + l32;     // this lane's query
  const long long ldq = (long long)n_h * kPfDq, ldk = (long long)n_h * kPfDh;

  // queries as B fragments: dims 16f + 8g .. +7 of query qrow
  bf16x8_t qf[kPfDq / 16];
  {
    const int qr = min(qrow, T - 1);
    const uint16_t* qp = q + qr * ldq + (long long)h * kPfDq + 8 * g;
#pragma unroll
    for (int f = 0; f < kPfDq / 16; ++f) qf[f] = *(const bf16x8_t*)(qp + 16 * f);
  }
  // the workgroup needs keys 0 .. min(qb + 127, T - 1)
  const int kend = min(qb + kPfQ, T);
  const int n_sub = (kend + kPfSub - 1) / kPfSub;
  const int wave_end = min(q0 + 32, T);  // keys this wave needs: < wave_end

  // DMA sources of this thread: chunk p = i*256 + tid of a region lands at
  // LDS chunk p; content keys and values (rows of 16 chunks) take i = 0, 1,
  // RoPE keys (rows of 8 chunks) i = 0.  Key rows past the sequence end read
  // its last row (finite values; their scores are masked).
  int rw[2], cb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = i * 256 + tid, t = p >> 4;
    rw[i] = t;
    cb[i] = ((p & 15) ^ pf_f16(t)) * 16;
  }
  const int rw_r = tid >> 3, cb_r = ((tid & 7) ^ pf_f8(tid >> 3)) * 16;
  const int kstride = (int)(ldk * 2);  // bytes between key rows of k^C / v^C
  // source offsets of a full subtile (every row inside the sequence): loop
  // invariant, the subtile's position goes into the resource base
  const int vo_c0 = rw[0] * kstride + cb[0], vo_c1 = rw[1] * kstride + cb[1];
  const int vo_r = rw_r * (kPfDr * 2) + cb_r;
  const int lds0 = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)smem);
  auto issue = [&](int s, int slot) {
    const int j0 = s * kPfSub, last = T - 1 - j0;
    const i32x4_t rkc = make_rsrc(kc + (long long)j0 * ldk + (long long)h * kPfDh);
    const i32x4_t rkr = make_rsrc(kr + (long long)j0 * kPfDr);
    const i32x4_t rv = make_rsrc(v + (long long)j0 * ldk + (long long)h * kPfDh);
    const int m0b = lds0 + slot * kPfStage;
    dma_fence();
    int o0 = vo_c0, o1 = vo_c1, orr = vo_r;
    if (last < kPfSub - 1) {  // the sequence's last subtile (uniform): clamp the rows
      o0 = min(rw[0], last) * kstride + cb[0];
      o1 = min(rw[1], last) * kstride + cb[1];
      orr = min(rw_r, last) * (kPfDr * 2) + cb_r;
    }
    dma16_m0(rkc, o0, m0b + w_s * 1024);
    dma16_m0(rkc, o1, m0b + 4096 + w_s * 1024);
    dma16_m0(rkr, orr, m0b + kPfKcB + w_s * 1024);
    dma16_m0(rv, o0, m0b + kPfKcB + kPfKrB + w_s * 1024);
    dma16_m0(rv, o1, m0b + kPfKcB + kPfKrB + 4096 + w_s * 1024);
  };

  // LDS read offsets (relative to a ring slot, which is a compile-time
  // constant in the unrolled loop).  QK step f: this lane's key row l32,
  // logical chunk 2f + g of the content (f < 8) or RoPE (f >= 8) row.
  int off_kc[8], off_kr[4];
#pragma unroll
  for (int f = 0; f < 8; ++f) off_kc[f] = l32 * (kPfDh * 2) + ((2 * f + g) ^ pf_f16(l32)) * 16;
#pragma unroll
  for (int b = 0; b < 4; ++b) off_kr[b] = kPfKcB + l32 * (kPfDr * 2) + ((2 * b + g) ^ pf_f8(l32)) * 16;
  // transposed value reads of dim block d (32 dims = chunks 4d .. 4d+3): rows
  // ta (first 4 k-slots) and ta + 8 (last 4) of a 16-key step (+16 rows for
  // the second step: the swizzle ignores bit 4)
  int off_pv[4][2];
  {
    const int ta = 4 * g + (j16 >> 2);
    const int clo = 2 * (G & 1) + ((j16 & 3) >> 1);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int t = ta + 8 * hh;
        off_pv[d][hh] = kPfKcB + kPfKrB + t * (kPfDh * 2) + ((4 * d + clo) ^ pf_f16(t)) * 16 + (j16 & 1) * 8;
      }
  }

  f32x16_t acc[kPfDh / 32];
#pragma unroll
  for (int d = 0; d < kPfDh / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // one subtile in ring slot SLOT (a compile-time constant, so every LDS
  // offset below folds into the instruction's immediate)
  auto step = [&](int s, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    wait_vm<0>();     // subtile s landed
    __syncthreads();  // subtile s visible; every wave is done with subtile s - 1
    if (s + 1 < n_sub) issue(s + 1, (SLOT + 1) % kPfRing);  // into the slot subtile s - 1 used
    const lds_u8* tile = smem + SLOT * kPfStage;
    const int j0 = s * kPfSub;
    if (j0 < wave_end) {  // scalar branch: some of these keys are visible to this wave
      // ---- S^T = K . Q^T
      f32x16_t sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
      for (int f = 0; f < kPfDq / 16; ++f) {
        const bf16x8_t ka = f < 8 ? lds_b128(tile + off_kc[f & 7]) : lds_b128(tile + off_kr[f & 3]);
        sc = mfma(ka, qf[f], sc);
      }
      // ---- causal mask (only subtiles that reach past the wave's first query
      // or past T) and online softmax in the exp2 domain
      if (j0 + kPfSub - 1 > q0 || j0 + kPfSub > T) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > qrow || key >= T) sc[r] = -INFINITY;
        }
      }
      // row maximum as a tree of raw three-input maxima (scores are finite or
      // -inf, never NaN, so fmaxf's quieting of each operand is not needed)
      const float m0 = max3_raw(sc[0], sc[1], sc[2]), m1 = max3_raw(sc[3], sc[4], sc[5]);
      const float m2 = max3_raw(sc[6], sc[7], sc[8]), m3 = max3_raw(sc[9], sc[10], sc[11]);
      const float m4 = max3_raw(sc[12], sc[13], sc[14]);
      const float m5 = max3_raw(m0, m1, m2), m6 = max3_raw(m3, m4, sc[15]);
      const float mx = half_swap_max_raw(max3_raw(m5, m6, m6)) * scale2;
      // lazy reference: it moves only when some query's max exceeds it by
      // more than 2^kPfTau (numerator and denominator share it, so the result
      // is exact; p stays below 2^kPfTau)
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kPfTau)) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first update
        l_run *= corr;
#pragma unroll
        for (int d = 0; d < kPfDh / 32; ++d)
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
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
        l_run += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      // ---- O^T += V^T . P^T: keys 16ks + {4g..4g+3, 8+4g..8+4g+3}
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int d = 0; d < kPfDh / 32; ++d) {
          const lds_u8* p0 = tile + ks * 16 * (kPfDh * 2);
          const bf16x4_t lo = lds_tr16(p0 + off_pv[d][0]);
          const bf16x4_t hi = lds_tr16(p0 + off_pv[d][1]);
          bf16x8_t va;
          va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
          va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
          acc[d] = mfma(va, P[ks], acc[d]);
        }
    }
  };
  wait_vm<0>();  // the query loads are complete before the first DMA
  issue(0, 0);
  for (int s = 0; s < n_sub; s += kPfRing) {
    step(s, std::integral_constant<int, 0>{});
    if (s + 1 < n_sub) step(s + 1, std::integral_constant<int, 1>{});
  }
  // ---- normalise and store: lane = query, acc[d] rows = dims 32d + 8(r/4) + 4g + r%4
  if (qrow < T) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const long long ob = ((long long)qrow * n_h + h) * kPfDh;
#pragma unroll
    for (int d = 0; d < kPfDh / 32; ++d)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int dim = 32 * d + 8 * qd + 4 * g;
        const float o0 = acc[d][4 * qd] * inv, o1 = acc[d][4 * qd + 1] * inv;
        const float o2 = acc[d][4 * qd + 2] * inv, o3 = acc[d][4 * qd + 3] * inv;
        if (out_bf16) {
          *(u32x2_t*)((uint16_t*)out + ob + dim) = u32x2_t{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        } else {
          *(f32x4_t*)((float*)out + ob + dim) = f32x4_t{o0, o1, o2, o3};
        }
      }
    if (lse && g == 0) lse[(long long)qrow * n_h + h] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// Portable fp32 kernel: one wave per (query, head), keys one at a time with
// an exact online softmax; lanes split the dimensions.
constexpr int kPfMaxD = 4;  // dims per lane: d_qk and d_v up to 256
__global__ __launch_bounds__(256) void prefill_generic_kernel(const void* q, const void* kc, const void* kr,
                                                              const void* v, void* out, float* lse, int T,
                                                              int n_h, int d_h, int d_r, float scale, int dt,
                                                              int out_dt) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * n_h + h
  if (row >= (long long)T * n_h) return;
  const int t = (int)(row / n_h), h = (int)(row % n_h);
  const int dq = d_h + d_r;
  float qv[kPfMaxD], acc[kPfMaxD];
#pragma unroll
  for (int k = 0; k < kPfMaxD; ++k) {
    const int e = lane + 64 * k;
    qv[k] = e < dq ? load_elem(q, row * dq + e, dt) : 0.f;
    acc[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= t; ++j) {
    float part = 0.f;
#pragma unroll
    for (int k = 0; k < kPfMaxD; ++k) {
      const int e = lane + 64 * k;
      float kv = 0.f;
      if (e < d_h)
        kv = load_elem(kc, ((long long)j * n_h + h) * d_h + e, dt);
      else if (e < dq)
        kv = load_elem(kr, (long long)j * d_r + (e - d_h), dt);
      part += qv[k] * kv;
    }
    const float s = wave_sum(part) * scale;
    const float m_new = fmaxf(m, s);
    const float c = __expf(m - m_new), p = __expf(s - m_new);
    l = l * c + p;
#pragma unroll
    for (int k = 0; k < kPfMaxD; ++k) {
      const int e = lane + 64 * k;
      acc[k] = acc[k] * c + (e < d_h ? p * load_elem(v, ((long long)j * n_h + h) * d_h + e, dt) : 0.f);
    }
    m = m_new;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int k = 0; k < kPfMaxD; ++k) {
    const int e = lane + 64 * k;
    if (e < d_h) store_elem(out, row * d_h + e, acc[k] * inv, out_dt);
  }
  if (lse && lane == 0) lse[row] = m + __logf(l);
}

bool prefill_mfma_eligible(int d_h, int d_r, int in_dtype, const void* q, const void* kc, const void* kr,
                           const void* v) {
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  return in_dtype == 1 && d_h == kPfDh && d_r == kPfDr && a16(q) && a16(kc) && a16(kr) && a16(v);
}

hipError_t launch_prefill(const void* q, const void* kc, const void* kr, const void* v, void* out, float* lse,
                          int T, int n_h, int d_h, int d_r, float scale, int in_dtype, int out_dtype,
                          hipStream_t s) {
  if (prefill_mfma_eligible(d_h, d_r, in_dtype, q, kc, kr, v)) {
    const int nqb = (T + kPfQ - 1) / kPfQ;
    const long long grid = (long long)nqb * ((n_h + 7) / 8 * 8);  // heads padded to a multiple of the 8 XCDs
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_mfma_kernel, dim3((unsigned)grid), dim3(256), 0, s, (const uint16_t*)q,
                       (const uint16_t*)kc, (const uint16_t*)kr, (const uint16_t*)v, out, lse, T, n_h, nqb,
                       scale * kLog2e, out_dtype == 1 ? 1 : 0);
  } else {
    const long long rows = (long long)T * n_h;
    hipLaunchKernelGGL(prefill_generic_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, q, kc, kr, v,
                       out, lse, T, n_h, d_h, d_r, scale, in_dtype, out_dtype);
  }
  return hipGetLastError();
}

}  // namespace mla
