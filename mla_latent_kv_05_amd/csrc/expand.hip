// MHA-mode key/value expansion from the latent (itwiki "Multi-head latent
// attention", section "Joint KV compression"): k^C = W^UK c^KV and
// v^C = W^UV c^KV for every token and head, i.e. two plain GEMMs
//   out[t, n] = sum_c W[n, c] * c_kv[t, c],   n = head * d_h + k,
// with the weights stored [n_h*d_h, d_c].  Over a prefill's thousands of
// tokens this is compute-bound (2 * 2 * T * d_c * n_h * d_h flops), so it gets
// a tiled MFMA GEMM.  A workgroup of four waves computes 256 (n) x 256 (t)
// tiles of either output; each wave owns a 128 x 128 quarter as 4 x 4 blocks
// of v_mfma_f32_32x32x16_bf16 with D[n, t] (A = weight rows, B = latent rows,
// so a lane ends up holding 4 consecutive n of one token), accumulated in the
// 256 AGPRs.  The grid is persistent (one workgroup per compute unit, tiles
// dealt round-robin), and both operands stream through a 4-slot LDS ring in
// 32-wide k slices by 16-byte global->LDS DMA three slices ahead, as one
// stream that runs on across tile boundaries, so the next tile's first slices
// are in flight while the current tile's results are stored.  At a tile's
// last slice the ring slot it frees is not refilled at once: each wave stages
// its bf16 results there and stores whole 256-byte row segments (the refill
// catches up one slice later).  Vector memory operations report completion
// in issue order, so the DMA waits count the stores still in flight and the
// stores drain under the next tile's MFMAs.
#include "mfma_common.h"

namespace mla {

namespace {

constexpr int kExN = 256, kExT = 256, kExK = 32;  // workgroup tile and k slice
constexpr int kExWB = kExN * kExK * 2;             // 16384: weight slice, 64-byte rows
constexpr int kExAB = kExT * kExK * 2;             // 16384: latent slice, 64-byte rows
constexpr int kExStage = kExWB + kExAB;            // 32768
constexpr int kExRing = 4;
constexpr int kExLds = kExRing * kExStage;         // 131072
constexpr int kExDma = 8;                          // DMA instructions per thread per slice

// physical chunk (of 4 per 64-byte row) of logical chunk c in row r: rows
// 4 apart land on different banks for the 16-lane phases of ds_read_b128
__device__ __forceinline__ int ex_chunk(int c, int r) { return c ^ ((r >> 2) & 3); }

// s_waitcnt vmcnt(m) for the largest available m <= n (a smaller count only
// waits for more of the oldest operations)
__device__ __forceinline__ void wait_at_most(int n) {
  if (n >= 48)
    wait_vm<48>();
  else if (n >= 40)
    wait_vm<40>();
  else if (n >= 32)
    wait_vm<32>();
  else if (n >= 24)
    wait_vm<24>();
  else if (n >= 16)
    wait_vm<16>();
  else if (n >= 8)
    wait_vm<8>();
  else
    wait_vm<0>();
}

}  // namespace

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void expand_gemm_kernel(const uint16_t* a, long long a_st, const uint16_t* w0,
                                                          const uint16_t* w1, void* out0, void* out1, int T,
                                                          int N, int K) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int w_s = __builtin_amdgcn_readfirstlane(wv);
  const int wn = wv & 1, wt = wv >> 1;  // this wave's 128 n x 128 t quarter
  const int n_tt = (T + kExT - 1) / kExT, n_nt = N / kExN;
  const int G = gridDim.x, nk = K / kExK;
  // tiles blockIdx.x, + G, ... (t fastest, then n, then which weight);
  // the launch keeps G <= the tile count
  const int my_tiles = (n_tt * n_nt * 2 - (int)blockIdx.x + G - 1) / G;
  const int total = my_tiles * nk;  // k slices this workgroup streams

  // DMA side.  Chunk p of a region (4 per 64-byte row) lands at LDS chunk p:
  // rows i*64 + tid/4 for i = 0..3 of the weight and of the latent slice
  // (rows past T read the last token).
  const int cdma = tid & 3, rsub = tid >> 2;
  // the tile being fetched: output rows t0.., weight rows n0.. of weight w
  int is_tile = blockIdx.x, is_ks = 0, n_issued = 0;
  int is_t0 = 0, is_n0 = 0;
  const uint16_t* is_w = w0;
  auto locate = [&](int tile, int& t0, int& n0, bool& second) {
    t0 = (tile % n_tt) * kExT;
    const int rest = tile / n_tt;
    n0 = (rest % n_nt) * kExN;
    second = rest >= n_nt;
  };
  auto fetch_tile = [&]() {
    bool second;
    locate(is_tile, is_t0, is_n0, second);
    is_w = second ? w1 : w0;
  };
  fetch_tile();
  auto issue = [&]() {
    const int k0 = is_ks * kExK;
    const i32x4_t rw = make_rsrc(is_w + (long long)is_n0 * K + k0);
    const i32x4_t ra = make_rsrc(a + (long long)is_t0 * a_st + k0);
    const int last_t = T - 1 - is_t0;
    const int m0b =
        __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(smem + (n_issued % kExRing) * kExStage));
    dma_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 64 + rsub;
      dma16_m0(rw, r * (K * 2) + ex_chunk(cdma, r) * 16, m0b + i * 4096 + w_s * 1024);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 64 + rsub;
      dma16_m0(ra, min(r, last_t) * (int)(a_st * 2) + ex_chunk(cdma, r) * 16, m0b + kExWB + i * 4096 + w_s * 1024);
    }
    ++n_issued;
    if (++is_ks == nk) {
      is_ks = 0;
      is_tile += G;
      fetch_tile();
    }
  };

  // fragment offsets: row l32 of each 32-row block, logical chunk 2kk + g
  int off_c[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) off_c[kk] = l32 * 64 + ex_chunk(2 * kk + g, l32) * 16;
  auto frags = [&](int slot, int kk, bf16x8_t* fa, bf16x8_t* fb) {
    const lds_u8* base = smem + slot * kExStage;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) fa[nb] = lds_b128(base + (wn * 128 + nb * 32) * 64 + off_c[kk]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) fb[tb] = lds_b128(base + kExWB + (wt * 128 + tb * 32) * 64 + off_c[kk]);
  };
  f32x16_t acc[16];  // block (nb, tb) at nb * 4 + tb
  auto mma = [&](const bf16x8_t* fa, const bf16x8_t* fb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) mfma_acc(acc[nb * 4 + tb], fa[nb], fb[tb]);
  };
  // D[n, t]: lane column t = l32 of block tb, rows n = 8(r/4) + 4g + r%4 of
  // block nb.  bf16: per 32-token block row the wave writes its 32 x 128
  // results into 8 KB of the free ring slot as [t][n] rows of 256 bytes
  // (16-byte chunk c of row t at c ^ (t & 15), 8-byte halves swapped for
  // t >= 16: both the 8-byte writes of 32 lanes and the 16-byte reads of 16
  // lanes cover all 64 banks), reads back 16-byte chunks and stores each row
  // segment contiguously: 32 stores per thread per tile.  fp32: 64 direct
  // 16-byte stores.
  auto store_tile = [&](int tile, int stage_slot) {
    int t0, n0;
    bool second;
    locate(tile, t0, n0, second);
    void* out = second ? out1 : out0;
    acc_fence(acc);
    if (OUT_BF16) {
      lds_u8* st = smem + stage_slot * kExStage + wv * 8192;
      const int hsw = (l32 >> 4) & 1;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const f32x16_t& c = acc[nb * 4 + tb];
            const int ch = (nb * 4 + qd) ^ (l32 & 15);
            *(__attribute__((address_space(3))) u32x2_t*)(st + l32 * 256 + ch * 16 + (g ^ hsw) * 8) =
                u32x2_t{pack_bf16x2(c[4 * qd], c[4 * qd + 1]), pack_bf16x2(c[4 * qd + 2], c[4 * qd + 3])};
          }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = i * 4 + (lane >> 4), p = lane & 15;
          u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(st + row * 256 + p * 16);
          if ((row >> 4) & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
          const int t = t0 + wt * 128 + tb * 32 + row;
          if (t < T)  // streamed out: keep L2 for the operands
            __builtin_nontemporal_store(v, (u32x4_t*)((uint16_t*)out + (long long)t * N + n0 + wn * 128 + (p ^ (row & 15)) * 8));
        }
      }
    } else {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int t = t0 + wt * 128 + tb * 32 + l32;
        if (t >= T) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int n = n0 + wn * 128 + nb * 32 + 8 * qd + 4 * g;
            const f32x16_t& c = acc[nb * 4 + tb];
            *(f32x4_t*)((float*)out + (long long)t * N + n) = f32x4_t{c[4 * qd], c[4 * qd + 1], c[4 * qd + 2], c[4 * qd + 3]};
          }
      }
    }
  };
  constexpr int kStores = OUT_BF16 ? 32 : 64;  // store instructions per thread per tile

  zero_acc(acc);
  const int pre = min(total, kExRing);
  for (int p = 0; p < pre; ++p) issue();
  wait_at_most((pre - 1) * kExDma);  // slice 0 landed; the ones issued after it may still fly
  __syncthreads();
  bf16x8_t fa0[4], fb0[4], fa1[4], fb1[4];
  frags(0, 0, fa0, fb0);
  int c_tile = blockIdx.x, c_ks = 0;
  int st_mark = -1;  // slices issued before the last tile's stores
  for (int s = 0; s < total; ++s) {
    const bool tile_end = c_ks == nk - 1;
    frags(s % kExRing, 1, fa1, fb1);
    mma(fa0, fb0);
    // The same straight-line step on every slice, the last included (a
    // branch here leaves the compiler unsure on the join whether the second
    // fragments have landed, and it then waits for the next slice's reads
    // before the second MFMA group); on the last slice the wait covers every
    // outstanding operation, nothing is issued and the fragment reads of the
    // next slot stay inside LDS, unused.
    // Slice s + 1 landed: after it come the DMA of the slices issued later
    // and, if issued after it, the last tile's stores.
    wait_at_most((n_issued - (s + 2)) * kExDma + (st_mark >= s + 2 ? kStores : 0));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of slot s are done
    __syncthreads();                     // ... and every wave's: slot s may be refilled
    // kExRing - 1 slices ahead (slot s % kExRing takes slice s + kExRing),
    // except that at a tile end slot s % kExRing stages the results and is
    // refilled one slice later
    const int target = min(total, s + kExRing + 1 - (tile_end ? 1 : 0));
    while (n_issued < target) issue();
    frags((s + 1) % kExRing, 0, fa0, fb0);
    mma(fa1, fb1);
    if (tile_end) {
      store_tile(c_tile, s % kExRing);
      zero_acc(acc);
      st_mark = n_issued;
      c_ks = 0;
      c_tile += G;
    } else {
      ++c_ks;
    }
  }
}

bool expand_gemm_eligible(long long a_st, int N, int K, int out_dtype, const void* a, const void* w0,
                          const void* w1, const void* o0, const void* o1) {
  auto al = [](const void* p, uintptr_t m) { return ((uintptr_t)p & (m - 1)) == 0; };
  const uintptr_t oa = out_dtype == 1 ? 8 : 16;
  return N % kExN == 0 && K % kExK == 0 && K >= kExK && a_st % 8 == 0 && a_st * 2 * kExT < 0x7fffffffLL &&
         (long long)N * K * 2 < 0x7fffffffLL && al(a, 16) && al(w0, 16) && al(w1, 16) && al(o0, oa) &&
         al(o1, oa);
}

hipError_t launch_expand_gemm(const void* a, long long a_st, const void* w0, const void* w1, void* o0, void* o1,
                              int T, int N, int K, int out_dtype, int n_cu, hipStream_t s) {
  static std::atomic<uint64_t> raised[2];
  const long long n_tiles = (long long)((T + kExT - 1) / kExT) * (N / kExN) * 2;
  const int grid = (int)std::min<long long>(n_tiles, std::max(n_cu, 1));
  const void* fn = out_dtype == 1 ? (const void*)expand_gemm_kernel<true> : (const void*)expand_gemm_kernel<false>;
  if (const hipError_t e = ensure_dynamic_lds(fn, kExLds, raised[out_dtype == 1]); e != hipSuccess) return e;
  if (out_dtype == 1)
    hipLaunchKernelGGL(expand_gemm_kernel<true>, dim3(grid), dim3(256), kExLds, s, (const uint16_t*)a, a_st,
                       (const uint16_t*)w0, (const uint16_t*)w1, o0, o1, T, N, K);
  else
    hipLaunchKernelGGL(expand_gemm_kernel<false>, dim3(grid), dim3(256), kExLds, s, (const uint16_t*)a, a_st,
                       (const uint16_t*)w0, (const uint16_t*)w1, o0, o1, T, N, K);
  return hipGetLastError();
}

}  // namespace mla
