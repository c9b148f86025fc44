// MHA-mode key/value expansion from the latent (itwiki "Multi-head latent
// attention", section "Joint KV compression"): k^C = W^UK c^KV and
// v^C = W^UV c^KV for every token and head, i.e. two plain GEMMs
//   out[t, n] = sum_c W[n, c] * c_kv[t, c],   n = head * d_h + k,
// with the weights stored [n_h*d_h, d_c].  Over a prefill's thousands of
// tokens this is compute-bound (2 * 2 * T * d_c * n_h * d_h flops), so it gets
// a tiled MFMA GEMM: a workgroup computes a 256 (n) x 128 (t) tile of one of
// the two outputs (blockIdx.z), wave w a 128 x 64 quarter as 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 with D[n, t] (A = weight rows, B = latent rows, so
// each lane ends up holding 4 consecutive n of one token: 8- or 16-byte
// stores).  Both operands stream through a 3-stage LDS ring in 32-wide k
// slices by 16-byte global->LDS DMA two slices ahead.
#include "mfma_common.h"

namespace mla {

namespace {

constexpr int kExN = 256, kExT = 128, kExK = 32;  // workgroup tile and k slice
constexpr int kExWB = kExN * kExK * 2;             // 16384: weight slice, 64-byte rows
constexpr int kExAB = kExT * kExK * 2;             // 8192: latent slice, 64-byte rows
constexpr int kExStage = kExWB + kExAB;            // 24576
constexpr int kExRing = 3;
constexpr int kExDma = 6;                          // DMA instructions per thread per slice

// physical chunk (of 4 per 64-byte row) of logical chunk c in row r: rows
// 4 apart land on different banks for the 16-lane phases of ds_read_b128
__device__ __forceinline__ int ex_chunk(int c, int r) { return c ^ ((r >> 2) & 3); }

}  // namespace

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void expand_gemm_kernel(const uint16_t* a, long long a_st, const uint16_t* w0,
                                                          const uint16_t* w1, void* out0, void* out1, int T,
                                                          int N, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[kExRing * kExStage];
  lds_u8* smem = (lds_u8*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int w_s = __builtin_amdgcn_readfirstlane(wv);
  const int t0 = blockIdx.x * kExT, n0 = blockIdx.y * kExN;
  const uint16_t* w = blockIdx.z ? w1 : w0;
  void* out = blockIdx.z ? out1 : out0;
  const int wn = wv & 1, wt = wv >> 1;  // this wave's 128 n x 64 t quarter

  // DMA sources: chunk p of a region (4 per 64-byte row) lands at LDS chunk p.
  // Weight rows p >> 2 for p = i*256 + tid (i = 0..3), latent rows likewise
  // (i = 0, 1; rows past T read the last token).
  const int cdma = tid & 3, rsub = tid >> 2;  // chunk and row within a 64-row group
  const int last_t = T - 1 - t0;
  auto issue = [&](int ks) {
    const int k0 = ks * kExK;
    const i32x4_t rw = make_rsrc(w + (long long)n0 * K + k0);
    const i32x4_t ra = make_rsrc(a + (long long)t0 * a_st + k0);
    const int m0b = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(smem + (ks % kExRing) * kExStage));
    dma_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 64 + rsub;
      dma16_m0(rw, r * (K * 2) + ex_chunk(cdma, r) * 16, m0b + i * 4096 + w_s * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = i * 64 + rsub;
      dma16_m0(ra, min(r, last_t) * (int)(a_st * 2) + ex_chunk(cdma, r) * 16, m0b + kExWB + i * 4096 + w_s * 1024);
    }
  };

  // fragment offsets: row l32 of each 32-row block, logical chunk 2kk + g
  int off_c[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) off_c[kk] = l32 * 64 + ex_chunk(2 * kk + g, l32) * 16;

  f32x16_t acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][tb][r] = 0.f;

  const int nk = K / kExK;
  issue(0);
  if (nk > 1) issue(1);
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk)
      wait_vm<kExDma>();  // slice ks landed (ks + 1 may still be in flight)
    else
      wait_vm<0>();
    __syncthreads();  // slice ks visible; every wave is done with slice ks - 1
    if (ks + 2 < nk) issue(ks + 2);
    const lds_u8* wt_l = smem + (ks % kExRing) * kExStage + wn * 128 * 64;
    const lds_u8* at_l = smem + (ks % kExRing) * kExStage + kExWB + wt * 64 * 64;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t bf[2], af[4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) bf[tb] = lds_b128(at_l + tb * 32 * 64 + off_c[kk]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) af[nb] = lds_b128(wt_l + nb * 32 * 64 + off_c[kk]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = mfma(af[nb], bf[tb], acc[nb][tb]);
    }
  }
  // D[n, t]: lane column t = l32 of block tb, rows n = 8(r/4) + 4g + r%4 of block nb
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + wt * 64 + tb * 32 + l32;
    if (t >= T) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int n = n0 + wn * 128 + nb * 32 + 8 * qd + 4 * g;
        const f32x16_t& c = acc[nb][tb];
        const long long o = (long long)t * N + n;
        if (OUT_BF16)
          *(u32x2_t*)((uint16_t*)out + o) =
              u32x2_t{pack_bf16x2(c[4 * qd], c[4 * qd + 1]), pack_bf16x2(c[4 * qd + 2], c[4 * qd + 3])};
        else
          *(f32x4_t*)((float*)out + o) = f32x4_t{c[4 * qd], c[4 * qd + 1], c[4 * qd + 2], c[4 * qd + 3]};
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
                              int T, int N, int K, int out_dtype, hipStream_t s) {
  dim3 grid((T + kExT - 1) / kExT, N / kExN, 2);
  if (out_dtype == 1)
    hipLaunchKernelGGL(expand_gemm_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)a, a_st,
                       (const uint16_t*)w0, (const uint16_t*)w1, o0, o1, T, N, K);
  else
    hipLaunchKernelGGL(expand_gemm_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)a, a_st,
                       (const uint16_t*)w0, (const uint16_t*)w1, o0, o1, T, N, K);
  return hipGetLastError();
}

}  // namespace mla
