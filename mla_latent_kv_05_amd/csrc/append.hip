// Cache producer, the step before decode (itwiki "Multi-head latent
// attention": sections "Joint KV compression" and "Decoupled RoPE"): for each
// new token t
//   c^KV_t = W^DKV h_t,  k^R_t = RoPE(W^KR h_t, pos_t)
// stored into the paged latent cache at slot_mapping[t] (block = slot /
// block_size, row = slot % block_size) as a bf16 / fp32 row [c^KV | k^R] or,
// for the fp8 cache, as e4m3fn content codes with one fp32 scale per token
// (amax / 448) beside the bf16 RoPE key.
//
// Two kernels.  The projection [T, d] x [d, d_c + d_r] is weight-bound for
// decode batches (the 576 x 7168 bf16 weight is 8.3 MB, the tokens a few
// hundred KB), so it is split over output-column blocks and K ranges until it
// covers the chip: each workgroup reads one [32 x 512] weight slice once and
// writes fp32 partial sums.  The store kernel (one workgroup per token) adds
// the K partials, rotates the RoPE pairs (angles in fp64), quantises and
// writes the row.
#include <cmath>

#include "device_util.h"
#include "mla_internal.h"

namespace mla {

constexpr int kApN = 32;    // output columns per workgroup
constexpr int kApKS = 512;  // K range per workgroup
constexpr int kApM = 64;    // tokens per workgroup (two 32-row MFMA blocks)
constexpr int kApRow = kApKS + 8;  // bf16 elements per staged row (16-byte pad: conflict-free b128 reads)
constexpr size_t kApLds = (size_t)(kApM + kApN) * kApRow * 2;  // 99,840 B

// part[ks][t][n] = sum_{k in range ks} h[t][k] * w[n][k]   (bf16 in, fp32 out)
// grid (N / 32, d / 512, ceil(T / 64)).  The workgroup stages its 64 token
// rows and 32 weight rows of the K range in LDS with whole-row 16-byte loads
// (all issued before any store), then wave w multiplies token block w & 1
// over K half w >> 1 and the two halves meet in LDS.
__global__ __launch_bounds__(256) void append_gemm_mfma_kernel(const uint16_t* h, long long h_st,
                                                               const uint16_t* w, float* part, int T,
                                                               int d, int N) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ap_smem[];
  typedef __attribute__((address_space(3))) uint8_t lds_b;
  typedef __attribute__((address_space(3))) u32x4_t lds_u4;
  lds_b* hs = (lds_b*)ap_smem;
  lds_b* ws = hs + (size_t)kApM * kApRow * 2;
  __shared__ float red[2][32 * 33];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int n0 = blockIdx.x * kApN, k0 = blockIdx.y * kApKS, tb = blockIdx.z * kApM;
  constexpr int kRowChunks = kApKS / 8;                     // 64 16-byte pieces per row
  constexpr int kHL = kApM * kRowChunks / 256;              // 16 per thread
  constexpr int kWL = kApN * kRowChunks / 256;              // 8 per thread
  u32x4_t hv[kHL], wvv[kWL];
#pragma unroll
  for (int j = 0; j < kHL; ++j) {
    const int c = tid + 256 * j, r = c / kRowChunks, p = c % kRowChunks;
    hv[j] = u32x4_t{0, 0, 0, 0};
    if (tb + r < T) hv[j] = *(const u32x4_t*)(h + (long long)(tb + r) * h_st + k0 + 8 * p);
  }
#pragma unroll
  for (int j = 0; j < kWL; ++j) {
    const int c = tid + 256 * j, r = c / kRowChunks, p = c % kRowChunks;
    wvv[j] = *(const u32x4_t*)(w + (long long)(n0 + r) * d + k0 + 8 * p);
  }
#pragma unroll
  for (int j = 0; j < kHL; ++j) {
    const int c = tid + 256 * j, r = c / kRowChunks, p = c % kRowChunks;
    *(lds_u4*)(hs + ((size_t)r * kApRow + 8 * p) * 2) = hv[j];
  }
#pragma unroll
  for (int j = 0; j < kWL; ++j) {
    const int c = tid + 256 * j, r = c / kRowChunks, p = c % kRowChunks;
    *(lds_u4*)(ws + ((size_t)r * kApRow + 8 * p) * 2) = wvv[j];
  }
  __syncthreads();
  const int mrow = (wv & 1) * 32 + l32, kh = (wv >> 1) * (kApKS / 2) + 8 * g;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int st = 0; st < kApKS / 2 / 16; ++st) {
    const bf16x8_t a = *(const __attribute__((address_space(3))) bf16x8_t*)(hs + ((size_t)mrow * kApRow + kh + 16 * st) * 2);
    const bf16x8_t b = *(const __attribute__((address_space(3))) bf16x8_t*)(ws + ((size_t)l32 * kApRow + kh + 16 * st) * 2);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  // D[i = token][j = column]: lane column l32, rows 8(r/4) + 4g + r%4
  if (wv >= 2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wv & 1][(8 * (r >> 2) + 4 * g + (r & 3)) * 33 + l32] = acc[r];
  }
  __syncthreads();
  if (wv < 2) {
    const int t0 = tb + (wv & 1) * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * g + (r & 3);
      const int tt = t0 + i;
      if (tt < T) part[((long long)blockIdx.y * T + tt) * N + n0 + l32] = acc[r] + red[wv][i * 33 + l32];
    }
  }
}

// fp32 / generic shapes: part[0][t][n] = sum_k h[t][k] * w[n][k], one thread
// per output element
__global__ __launch_bounds__(256) void append_gemm_generic_kernel(const void* h, long long h_st,
                                                                  const void* w, float* part, int T,
                                                                  int d, int N, int dt) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * N) return;
  const int t = (int)(idx / N), n = (int)(idx % N);
  float acc = 0.f;
  for (int k = 0; k < d; ++k)
    acc += load_elem(h, (long long)t * h_st + k, dt) * load_elem(w, (long long)n * d + k, dt);
  part[idx] = acc;
}

// One workgroup per token: y = sum of the K partials; RoPE on the last d_r
// values (pairs (k, k + d_r/2), angle pos * base^(-2k/d_r) in fp64); store.
struct RopeFreqs {
  double f[kMaxRopePairs];  // base^(-2k/d_r), computed on the host in fp64
};

__global__ __launch_bounds__(256) void append_store_kernel(const float* part, int n_splits,
                                                           const int32_t* positions,
                                                           const int32_t* slots, void* cache, int T,
                                                           int d_c, int d_r, int block_size,
                                                           long long block_bytes, RopeFreqs fr,
                                                           int kv_dtype) {
  extern __shared__ float y[];  // [d_c + d_r]
  __shared__ float wred[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int slot = slots[t];
  if (slot < 0) return;  // uniform: the token is skipped
  const int N = d_c + d_r;
  // K partials: every load of a column in flight at once (up to kMaxSplits
  // per round trip)
  constexpr int kMaxSplits = 16;
  for (int n = tid; n < N; n += 256) {
    float v = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += kMaxSplits) {
      float p[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s)
        p[s] = s0 + s < n_splits ? part[((long long)(s0 + s) * T + t) * N + n] : 0.f;
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) v += p[s];
    }
    y[n] = v;
  }
  __syncthreads();
  const int half = d_r / 2;
  const double pos = (double)positions[t];
  for (int k = tid; k < half; k += 256) {
    // angle reduced to [-pi, pi] by a two-part 2*pi before the fp64 sine and
    // cosine (positions reach 10^5 radians; the reduction error stays ~1e-11)
    constexpr double kTwoPiHi = 6.283185307179586, kTwoPiLo = 2.4492935982947064e-16;
    const double ang = pos * fr.f[k];
    const double q = rint(ang * (1.0 / kTwoPiHi));
    const double red = fma(-q, kTwoPiLo, fma(-q, kTwoPiHi, ang));
    double sn, cs;
    sincos(red, &sn, &cs);
    const double x1 = y[d_c + k], x2 = y[d_c + k + half];
    y[d_c + k] = (float)(x1 * cs - x2 * sn);
    y[d_c + k + half] = (float)(x2 * cs + x1 * sn);
  }
  __syncthreads();
  const long long blk = slot / block_size, row = slot % block_size;
  uint8_t* base = (uint8_t*)cache + blk * block_bytes;
  if (kv_dtype == 0) {  // fp32 rows
    float* r = (float*)base + row * N;
    for (int n = tid; n < N; n += 256) r[n] = y[n];
  } else if (kv_dtype == 1) {  // bf16 rows
    uint16_t* r = (uint16_t*)base + row * N;
    for (int n = tid; n < N; n += 256) r[n] = f32_to_bf16_bits(y[n]);
  } else {  // fp8 block: codes | bf16 k^R | fp32 scales
    float m = 0.f;
    for (int n = tid; n < d_c; n += 256) m = fmaxf(m, fabsf(y[n]));
    m = wave_max(m);
    if ((tid & 63) == 0) wred[tid >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    uint8_t* codes = base + row * d_c;
    for (int n = 2 * tid; n < d_c; n += 512) {  // two codes per conversion
      const float q0 = fminf(fmaxf(y[n] / scale, -448.f), 448.f);
      const float q1 = n + 1 < d_c ? fminf(fmaxf(y[n + 1] / scale, -448.f), 448.f) : 0.f;
      const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      codes[n] = (uint8_t)(pk & 0xffu);
      if (n + 1 < d_c) codes[n + 1] = (uint8_t)((pk >> 8) & 0xffu);
    }
    uint16_t* kr = (uint16_t*)(base + (long long)block_size * d_c) + row * d_r;
    for (int n = tid; n < d_r; n += 256) kr[n] = f32_to_bf16_bits(y[d_c + n]);
    if (tid == 0) ((float*)(base + (long long)block_size * (d_c + 2 * d_r)))[row] = scale;
  }
}

size_t append_workspace_bytes(int T, int d, int d_c, int d_r) {
  const int N = d_c + d_r;
  const int splits = (d + kApKS - 1) / kApKS;
  return align256((size_t)splits * T * N * 4);
}

bool append_mfma_eligible(int d, int N, int in_dtype, long long h_st, const void* h, const void* w) {
  return in_dtype == 1 && d % kApKS == 0 && N % kApN == 0 && h_st % 8 == 0 &&
         ((uintptr_t)h & 15u) == 0 && ((uintptr_t)w & 15u) == 0;
}

hipError_t launch_append(const void* h, long long h_st, const void* w, const int32_t* positions,
                         const int32_t* slots, void* cache, int T, int d, int d_c, int d_r, int block_size,
                         long long block_bytes, float rope_base, int in_dtype, int kv_dtype, float* part,
                         hipStream_t s) {
  const int N = d_c + d_r;
  int n_splits = 1;
  if (append_mfma_eligible(d, N, in_dtype, h_st, h, w)) {
    static std::atomic<uint64_t> lds_raised{0};
    if (const hipError_t e = ensure_dynamic_lds((const void*)append_gemm_mfma_kernel, (int)kApLds, lds_raised);
        e != hipSuccess)
      return e;
    n_splits = d / kApKS;
    dim3 grid(N / kApN, n_splits, (T + kApM - 1) / kApM);
    hipLaunchKernelGGL(append_gemm_mfma_kernel, grid, dim3(256), kApLds, s, (const uint16_t*)h, h_st,
                       (const uint16_t*)w, part, T, d, N);
  } else {
    const long long total = (long long)T * N;
    hipLaunchKernelGGL(append_gemm_generic_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, h,
                       h_st, w, part, T, d, N, in_dtype);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RopeFreqs fr{};
  for (int k = 0; k < d_r / 2; ++k) fr.f[k] = std::pow((double)rope_base, -2.0 * k / d_r);
  hipLaunchKernelGGL(append_store_kernel, dim3(T), dim3(256), (size_t)N * 4, s, part, n_splits, positions,
                     slots, cache, T, d_c, d_r, block_size, block_bytes, fr, kv_dtype);
  return hipGetLastError();
}

}  // namespace mla
