// Per-head projections around the absorbed decode (itwiki "Multi-head latent
// attention", section "Matrix absorption"; lecture "MHA · GQA · MQA · MLA",
// section "Why Projection Absorption Helps"):
//   absorb:  q_lat[t,i,:] = W^UK_i^T q^C[t,i,:]      W^UK_i = rows i*d_h.. of [n_h*d_h, d_c]
//   up-proj: o[t,i,:]     = W^UV_i  o_lat[t,i,:]
// Both are small batched GEMMs bound by reading the weights (16 MiB bf16 each
// at V3 shapes), so the MFMA kernels read every weight byte exactly once and
// keep each head's weight slice in one workgroup.
#include "device_util.h"
#include "mla_internal.h"

namespace mla {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ f32x16_t mfma16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ generic fp32
// out[t, h, n] = sum_k A[t, h, k] * W(h, k, n); absorb: W(h,k,n) = w[(h*d_h+k)*d_c + n]
// (K = d_h, N = d_c); up-proj: W(h,k,n) = w[(h*d_h+n)*d_c + k] (K = d_c, N = d_h).
template <bool UP>
__global__ __launch_bounds__(256) void proj_generic_kernel(const void* A, long long a_st, const void* w,
                                                           void* out, long long o_st, int T, int n_h,
                                                           int K, int N, int d_h, int d_c, int act_dt,
                                                           int w_dt, int out_dt) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)T * n_h * N;
  if (idx >= total) return;
  const int n = (int)(idx % N);
  const int h = (int)((idx / N) % n_h);
  const int t = (int)(idx / ((long long)N * n_h));
  float acc = 0.f;
  const long long arow = t * a_st + (long long)h * K;
  for (int k = 0; k < K; ++k) {
    const long long wi = UP ? ((long long)(h * d_h + n) * d_c + k) : ((long long)(h * d_h + k) * d_c + n);
    acc += load_elem(A, arow + k, act_dt) * load_elem(w, wi, w_dt);
  }
  store_elem(out, t * o_st + (long long)h * N + n, acc, out_dt);
}

// ------------------------------------------------------------ MFMA absorb
// Workgroup = (head h, 128-column block of d_c).  The weight slice
// W^UK_h[0:d_h, c0:c0+128] is staged in LDS (row stride padded to 144
// elements) and read transposed with ds_read_tr16_b64 as the B operand;
// queries are the A operand straight from global memory.  Wave w covers
// columns c0 + 32w .. +31 for all T_q rows (32-row tiles).
constexpr int kAbsCols = 128;
constexpr int kAbsStride = 144;  // bf16 elements per staged weight row
constexpr int kAbsMaxKb = 8;     // d_h / 16 up to d_h = 128

__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t* q, long long q_st,
                                                          const uint16_t* w, void* out, long long o_st,
                                                          int T, int n_h, int d_h, int d_c, int out_dt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  lds_u8* wl = (lds_u8*)smem_raw;
  const int h = blockIdx.y;
  const int c0 = blockIdx.x * kAbsCols;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  const int ncols = min(kAbsCols, d_c - c0);
  const int cw = 32 * wv;  // this wave's column offset within the block
  const int nkb = d_h / 16;
  // A fragments (query rows t0 + l32) of one 32-row tile; the first tile's
  // loads are issued before the weight staging so the two latencies overlap
  bf16x8_t av[kAbsMaxKb];
  auto load_q = [&](int t0) {
    const int tr = t0 + l32;
#pragma unroll
    for (int kb = 0; kb < kAbsMaxKb; ++kb) {
      if (kb >= nkb) break;
      if (tr < T) av[kb] = *(const bf16x8_t*)(q + tr * q_st + (long long)h * d_h + kb * 16 + g * 8);
      else for (int j = 0; j < 8; ++j) av[kb][j] = (__bf16)0.f;
    }
  };
  load_q(0);
  // stage W rows k = 0..d_h-1, columns c0..c0+ncols (16-byte pieces); the
  // loads of one batch are all issued before any LDS store
  const int pieces = ncols / 8;
  const int total = d_h * pieces;
  for (int e0 = 0; e0 < total; e0 += 256 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + j * 256 + tid;
      if (e < total) v[j] = *(const u32x4_t*)(w + ((long long)(h * d_h + e / pieces)) * d_c + c0 + (e % pieces) * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + j * 256 + tid;
      if (e < total) *(__attribute__((address_space(3))) u32x4_t*)(wl + ((e / pieces) * kAbsStride + (e % pieces) * 8) * 2) = v[j];
    }
  }
  __syncthreads();
  if (cw >= ncols) return;
  // B fragments (this wave's 32 columns, all of K) once from LDS
  bf16x8_t bf[kAbsMaxKb];
#pragma unroll
  for (int kb = 0; kb < kAbsMaxKb; ++kb) {
    if (kb >= nkb) break;
    // B[k][n]: k = kb*16 + g*8 + {0..3 | 4..7}, n = cw + l32 -> two transposed reads
    const int krow = kb * 16 + g * 8 + (j16 >> 2);
    const int col = cw + 16 * (G & 1) + (j16 & 3) * 4;
    const lds_u8* p = wl + (krow * kAbsStride + col) * 2;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t*)(p + 4 * kAbsStride * 2));
    bf[kb][0] = lo[0]; bf[kb][1] = lo[1]; bf[kb][2] = lo[2]; bf[kb][3] = lo[3];
    bf[kb][4] = hi[0]; bf[kb][5] = hi[1]; bf[kb][6] = hi[2]; bf[kb][7] = hi[3];
  }
  for (int t0 = 0; t0 < T; t0 += 32) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < kAbsMaxKb; ++kb) {
      if (kb >= nkb) break;
      acc = mfma16(av[kb], bf[kb], acc);
    }
    if (t0 + 32 < T) load_q(t0 + 32);  // next tile in flight during these stores
    // D[i = t][j = column]: lane column cw + l32, rows 8(r/4) + 4g + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (t < T) store_elem(out, t * o_st + (long long)h * d_c + c0 + cw + l32, acc[r], out_dt);
    }
  }
}

// ------------------------------------------------------------ MFMA up-projection
// Workgroup = (head h, 32-row block k0 of W^UV_h).  The 4 waves split the d_c
// reduction into quarters; each keeps its W slice (32 rows x d_c/4) in
// registers for all T_q tiles, and the quarter sums are added through LDS.
// B[c][k] = W^UV[h*d_h + k][c] is contiguous along c, so both operands load
// straight from global memory.
constexpr int kUpMaxCb = 8;  // d_c / 64 (16-wide k-steps per wave) up to d_c = 512

__global__ __launch_bounds__(256) void up_mfma_kernel(const uint16_t* a, long long a_st, const uint16_t* w,
                                                      void* out, long long o_st, int T, int n_h, int d_c,
                                                      int d_h, int out_dt) {
  __shared__ float red[4][32 * 33];
  const int h = blockIdx.y, k0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ncb = d_c / 64;                  // k-steps of this wave
  const int cbase = wv * ncb * 16;           // first d_c column of this wave
  const uint16_t* wrow = w + ((long long)(h * d_h + k0 + l32)) * d_c + cbase + g * 8;
  bf16x8_t wf[kUpMaxCb];
#pragma unroll
  for (int cb = 0; cb < kUpMaxCb; ++cb)
    if (cb < ncb) wf[cb] = *(const bf16x8_t*)(wrow + cb * 16);
  for (int t0 = 0; t0 < T; t0 += 32) {
    const int tr = t0 + l32;
    const uint16_t* arow = a + (long long)tr * a_st + (long long)h * d_c + cbase + g * 8;
    bf16x8_t af[kUpMaxCb];
#pragma unroll
    for (int cb = 0; cb < kUpMaxCb; ++cb) {
      if (cb < ncb && tr < T) af[cb] = *(const bf16x8_t*)(arow + cb * 16);
      else for (int j = 0; j < 8; ++j) af[cb][j] = (__bf16)0.f;
    }
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int cb = 0; cb < kUpMaxCb; ++cb)
      if (cb < ncb) acc = mfma16(af[cb], wf[cb], acc);
    // D[i = t][j = k]: lane column k0 + l32, rows 8(r/4) + 4g + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wv][(8 * (r >> 2) + 4 * g + (r & 3)) * 33 + l32] = acc[r];
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
      const int i = e >> 5, j = e & 31;
      const int t = t0 + i;
      const float v = red[0][i * 33 + j] + red[1][i * 33 + j] + red[2][i * 33 + j] + red[3][i * 33 + j];
      if (t < T) store_elem(out, (long long)t * o_st + (long long)h * d_h + k0 + j, v, out_dt);
    }
    __syncthreads();
  }
}

hipError_t launch_absorb(const void* q, long long q_st, const void* w, void* out, long long o_st, int T,
                         int n_h, int d_h, int d_c, int act_dt, int w_dt, int out_dt, bool mfma,
                         hipStream_t s) {
  if (mfma) {
    dim3 grid((d_c + kAbsCols - 1) / kAbsCols, n_h);
    const size_t lds = (size_t)d_h * kAbsStride * 2;
    hipLaunchKernelGGL(absorb_mfma_kernel, grid, dim3(256), lds, s, (const uint16_t*)q, q_st,
                       (const uint16_t*)w, out, o_st, T, n_h, d_h, d_c, out_dt);
  } else {
    const long long total = (long long)T * n_h * d_c;
    hipLaunchKernelGGL(proj_generic_kernel<false>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       q, q_st, w, out, o_st, T, n_h, d_h, d_c, d_h, d_c, act_dt, w_dt, out_dt);
  }
  return hipGetLastError();
}

hipError_t launch_up_proj(const void* o_lat, long long a_st, const void* w, void* out, long long o_st,
                          int T, int n_h, int d_c, int d_h, int act_dt, int w_dt, int out_dt, bool mfma,
                          hipStream_t s) {
  if (mfma) {
    hipLaunchKernelGGL(up_mfma_kernel, dim3(d_h / 32, n_h), dim3(256), 0, s, (const uint16_t*)o_lat, a_st,
                       (const uint16_t*)w, out, o_st, T, n_h, d_c, d_h, out_dt);
  } else {
    const long long total = (long long)T * n_h * d_h;
    hipLaunchKernelGGL(proj_generic_kernel<true>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       o_lat, a_st, w, out, o_st, T, n_h, d_c, d_h, d_h, d_c, act_dt, w_dt, out_dt);
  }
  return hipGetLastError();
}

}  // namespace mla
