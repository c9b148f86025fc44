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
#include "plan_body.h"

namespace mla {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ f32x16_t mfma16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ generic fp32
// out[t, h, n] = sum_k A[t, h, k] * W(h, k, n); absorb: W(h,k,n) = w[(h*d_h+k)*d_c + n]
// (K = d_h, N = d_c); up-proj: W(h,k,n) = w[(h*d_h+n)*d_c + k] (K = d_c, N = d_h).
template <bool UP>
__global__ __launch_bounds__(256) void proj_generic_kernel(const void* A, long long a_st, long long a_hs, const void* w,
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
  const long long arow = t * a_st + (long long)h * a_hs;
  for (int k = 0; k < K; ++k) {
    const long long wi = UP ? ((long long)(h * d_h + n) * d_c + k) : ((long long)(h * d_h + k) * d_c + n);
    acc += load_elem(A, arow + k, act_dt) * load_elem(w, wi, w_dt);
  }
  store_elem(out, t * o_st + (long long)h * N + n, acc, out_dt);
}

// ------------------------------------------------------------ MFMA absorb
// Workgroup = (head h, 128-column block of d_c).  The weight slice
// W^UK_h[0:d_h, c0:c0+128] is staged in LDS (row stride padded to 144
// elements) and read transposed with ds_read_tr16_b64 as the B operand.
// Query rows (A operand) are staged 32 at a time in LDS from whole-row
// loads, and each 32 x 128 output tile goes back through LDS (into the
// query area once every wave is done with it) so that global stores write
// whole 16-byte pieces of rows.  Wave w covers columns c0 + 32w .. +31.
// The staging is kept under 53 KB so that three workgroups fit on a compute
// unit: the 4 * n_h tiles of V2/V3 shapes (plus the planner's row when it
// rides along) then run in one wave.
constexpr int kAbsCols = 128;
constexpr int kAbsStride = 144;  // bf16 elements per staged weight row
constexpr int kAbsQStride = 136; // bf16 elements per staged query row
constexpr int kAbsMaxKb = 8;     // d_h / 16 up to d_h = 128

constexpr size_t absorb_lds_bytes(int d_h, bool out_bf16) {
  const size_t q = 32 * kAbsQStride * 2, o = 32 * (kAbsCols + 8) * (out_bf16 ? 2 : 4);
  return (size_t)d_h * kAbsStride * 2 + (q > o ? q : o);
}

// one workgroup's tile: head h, column block cblk
template <bool OUT_BF16>
__device__ __forceinline__ void absorb_tile(const uint16_t* q, long long q_st, const uint16_t* w, void* out,
                                            long long o_st, int T, int n_h, int d_h, int d_c, int h, int cblk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  typedef __attribute__((address_space(3))) u32x4_t lds_u4;
  lds_u8* wl = (lds_u8*)smem_raw;
  lds_u8* ql = wl + d_h * kAbsStride * 2;
  lds_u8* ol = ql;  // the output tile reuses the query rows' space
  constexpr int kOutElem = OUT_BF16 ? 2 : 4;
  constexpr int kORow = (kAbsCols + 8) * kOutElem;  // staged output row (bytes)
  const int c0 = cblk * kAbsCols;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  const int ncols = min(kAbsCols, d_c - c0);
  const int cw = 32 * wv;  // this wave's column offset within the block
  const bool active = cw < ncols;
  const int nkb = d_h / 16;

  // query tile: 32 rows x d_h/8 16-byte pieces (at most 2 per thread)
  const int qpc = d_h / 8;
  u32x4_t qv[2];
  auto load_q = [&](int t0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = j * 256 + tid, row = e / qpc, pc = e % qpc;
      qv[j] = u32x4_t{0, 0, 0, 0};
      if (row < 32 && t0 + row < T) qv[j] = *(const u32x4_t*)(q + (long long)(t0 + row) * q_st + (long long)h * d_h + pc * 8);
    }
  };
  auto store_q = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = j * 256 + tid, row = e / qpc, pc = e % qpc;
      if (row < 32) *(lds_u4*)(ql + (row * kAbsQStride + pc * 8) * 2) = qv[j];
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
      if (e < total) *(lds_u4*)(wl + ((e / pieces) * kAbsStride + (e % pieces) * 8) * 2) = v[j];
    }
  }
  store_q();
  __syncthreads();
  // B fragments (this wave's 32 columns, all of K) once from LDS
  bf16x8_t bf[kAbsMaxKb];
#pragma unroll
  for (int kb = 0; kb < kAbsMaxKb; ++kb) {
    if (kb >= nkb || !active) break;
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
    if (active) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < kAbsMaxKb; ++kb) {
        if (kb >= nkb) break;
        const bf16x8_t av = *(const __attribute__((address_space(3))) bf16x8_t*)(ql + (l32 * kAbsQStride + kb * 16 + g * 8) * 2);
        acc = mfma16(av, bf[kb], acc);
      }
    }
    __syncthreads();  // every wave has read the query rows: their space takes the output tile
    if (active) {
      // D[i = t][j = column]: lane column cw + l32, rows 8(r/4) + 4g + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * g + (r & 3);
        if (OUT_BF16)
          *(__attribute__((address_space(3))) uint16_t*)(ol + i * kORow + (cw + l32) * 2) = f32_to_bf16_bits(acc[r]);
        else
          *(__attribute__((address_space(3))) float*)(ol + i * kORow + (cw + l32) * 4) = acc[r];
      }
    }
    if (t0 + 32 < T) load_q(t0 + 32);  // next tile's rows in flight during the stores
    __syncthreads();  // output tile staged; every wave is done with this query tile
    // 32 rows x ncols of output, 16-byte pieces
    const int opc = ncols * kOutElem / 16;
    for (int e = tid; e < 32 * opc; e += 256) {
      const int row = e / opc, pc = e % opc;
      if (t0 + row < T)
        *(u32x4_t*)((uint8_t*)out + ((long long)(t0 + row) * o_st + (long long)h * d_c + c0) * kOutElem + pc * 16) =
            *(const lds_u4*)(ol + row * kORow + pc * 16);
    }
    if (t0 + 32 < T) {
      __syncthreads();  // every thread has copied the output tile out of the query area
      store_q();
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ MFMA up-projection
// Workgroup = (head h, 32-row block k0 of W^UV_h).  The 4 waves split the d_c
// reduction into quarters; each keeps its W slice (32 rows x d_c/4) in
// registers for all T_q tiles, and the quarter sums are added through LDS.
// B[c][k] = W^UV[h*d_h + k][c] is contiguous along c.  The activation rows
// (A operand) are staged 32 at a time in LDS from whole-row loads.
constexpr int kUpMaxCb = 8;      // d_c / 64 (16-wide k-steps per wave) up to d_c = 512
constexpr int kUpAStride = 520;  // bf16 elements per staged activation row

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void up_mfma_kernel(const uint16_t* a, long long a_st, long long a_hs, const uint16_t* w,
                                                      void* out, long long o_st, int T, int n_h, int d_c,
                                                      int d_h) {
  __shared__ float red[4][32 * 33];
  __shared__ __attribute__((aligned(16))) uint16_t at[32 * kUpAStride];
  typedef __attribute__((address_space(3))) u32x4_t lds_u4;
  lds_u8* al = (lds_u8*)at;
  const int h = blockIdx.y, k0 = blockIdx.x * 32;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int ncb = d_c / 64;                  // k-steps of this wave
  const int cbase = wv * ncb * 16;           // first d_c column of this wave
  const uint16_t* wrow = w + ((long long)(h * d_h + k0 + l32)) * d_c + cbase + g * 8;
  // activation tile: 32 rows x d_c/8 pieces (at most 8 per thread)
  const int apc = d_c / 8;
  u32x4_t av[8];
  auto load_a = [&](int t0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = j * 256 + tid, row = e / apc, pc = e % apc;
      av[j] = u32x4_t{0, 0, 0, 0};
      if (row < 32 && t0 + row < T) av[j] = *(const u32x4_t*)(a + (long long)(t0 + row) * a_st + (long long)h * a_hs + pc * 8);
    }
  };
  auto store_a = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = j * 256 + tid, row = e / apc, pc = e % apc;
      if (row < 32) *(lds_u4*)(al + (row * kUpAStride + pc * 8) * 2) = av[j];
    }
  };
  load_a(0);
  bf16x8_t wf[kUpMaxCb];
#pragma unroll
  for (int cb = 0; cb < kUpMaxCb; ++cb)
    if (cb < ncb) wf[cb] = *(const bf16x8_t*)(wrow + cb * 16);
  store_a();
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 32) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int cb = 0; cb < kUpMaxCb; ++cb)
      if (cb < ncb) {
        const bf16x8_t af = *(const __attribute__((address_space(3))) bf16x8_t*)(al + (l32 * kUpAStride + cbase + cb * 16 + g * 8) * 2);
        acc = mfma16(af, wf[cb], acc);
      }
    if (t0 + 32 < T) load_a(t0 + 32);  // next tile in flight during the reduction
    // D[i = t][j = k]: lane column k0 + l32, rows 8(r/4) + 4g + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wv][(8 * (r >> 2) + 4 * g + (r & 3)) * 33 + l32] = acc[r];
    __syncthreads();  // partial sums written; every wave is done with this activation tile
    for (int e = tid; e < 32 * 16; e += 256) {  // two adjacent columns per thread
      const int i = e >> 4, j = (e & 15) * 2;
      const int t = t0 + i;
      float v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        v[u] = red[0][i * 33 + j + u] + red[1][i * 33 + j + u] + red[2][i * 33 + j + u] + red[3][i * 33 + j + u];
      if (t < T) {
        const long long o = (long long)t * o_st + (long long)h * d_h + k0 + j;
        if (OUT_BF16)
          *(uint32_t*)((uint16_t*)out + o) = pack_bf16x2(v[0], v[1]);
        else
          *(float2*)((float*)out + o) = make_float2(v[0], v[1]);
      }
    }
    if (t0 + 32 < T) store_a();
    __syncthreads();
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t* q, long long q_st, const uint16_t* w,
                                                          void* out, long long o_st, int T, int n_h, int d_h,
                                                          int d_c) {
  absorb_tile<OUT_BF16>(q, q_st, w, out, o_st, T, n_h, d_h, d_c, blockIdx.y, blockIdx.x);
}

// The absorption with the split planner riding along: row 0 of the grid is
// the planner (its first workgroup; the others return), rows 1.. the
// absorption tiles, so the planning overlaps the weight reads instead of
// taking a launch of its own.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void absorb_plan_kernel(const uint16_t* q, long long q_st, const uint16_t* w,
                                                          void* out, long long o_st, int T, int n_h, int d_h,
                                                          int d_c, PlanArgs pa) {
  if (blockIdx.y == 0) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    if (blockIdx.x == 0) plan_body<256>(pa, (lds_u8*)smem_raw);
    return;
  }
  absorb_tile<OUT_BF16>(q, q_st, w, out, o_st, T, n_h, d_h, d_c, blockIdx.y - 1, blockIdx.x);
}

hipError_t launch_absorb_plan(const void* q, long long q_st, const void* w, void* out, long long o_st, int T,
                              int n_h, int d_h, int d_c, const PlanArgs& pa, hipStream_t s) {
  dim3 grid((d_c + kAbsCols - 1) / kAbsCols, n_h + 1);
  const size_t lds = absorb_lds_bytes(d_h, true) > (size_t)plan_lds_bytes(256) ? absorb_lds_bytes(d_h, true)
                                                                                 : (size_t)plan_lds_bytes(256);
  hipLaunchKernelGGL(absorb_plan_kernel<true>, grid, dim3(256), lds, s, (const uint16_t*)q, q_st,
                     (const uint16_t*)w, out, o_st, T, n_h, d_h, d_c, pa);
  return hipGetLastError();
}

hipError_t launch_absorb(const void* q, long long q_st, const void* w, void* out, long long o_st, int T,
                         int n_h, int d_h, int d_c, int act_dt, int w_dt, int out_dt, bool mfma,
                         hipStream_t s) {
  if (mfma) {
    dim3 grid((d_c + kAbsCols - 1) / kAbsCols, n_h);
    if (out_dt == 1)
      hipLaunchKernelGGL(absorb_mfma_kernel<true>, grid, dim3(256), absorb_lds_bytes(d_h, true), s,
                         (const uint16_t*)q, q_st, (const uint16_t*)w, out, o_st, T, n_h, d_h, d_c);
    else
      hipLaunchKernelGGL(absorb_mfma_kernel<false>, grid, dim3(256), absorb_lds_bytes(d_h, false), s,
                         (const uint16_t*)q, q_st, (const uint16_t*)w, out, o_st, T, n_h, d_h, d_c);
  } else {
    const long long total = (long long)T * n_h * d_c;
    hipLaunchKernelGGL(proj_generic_kernel<false>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       q, q_st, (long long)d_h, w, out, o_st, T, n_h, d_h, d_c, d_h, d_c, act_dt, w_dt, out_dt);
  }
  return hipGetLastError();
}

// a_hs: element distance between the heads' activation rows of one token
// (d_c for the up-projection; 0 when one latent row feeds every head, as in
// the MHA-mode key/value expansion)
hipError_t launch_up_proj(const void* o_lat, long long a_st, long long a_hs, const void* w, void* out,
                          long long o_st, int T, int n_h, int d_c, int d_h, int act_dt, int w_dt, int out_dt,
                          bool mfma, hipStream_t s) {
  if (mfma) {
    if (out_dt == 1)
      hipLaunchKernelGGL(up_mfma_kernel<true>, dim3(d_h / 32, n_h), dim3(256), 0, s, (const uint16_t*)o_lat, a_st,
                         a_hs, (const uint16_t*)w, out, o_st, T, n_h, d_c, d_h);
    else
      hipLaunchKernelGGL(up_mfma_kernel<false>, dim3(d_h / 32, n_h), dim3(256), 0, s, (const uint16_t*)o_lat,
                         a_st, a_hs, (const uint16_t*)w, out, o_st, T, n_h, d_c, d_h);
  } else {
    const long long total = (long long)T * n_h * d_h;
    hipLaunchKernelGGL(proj_generic_kernel<true>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       o_lat, a_st, a_hs, w, out, o_st, T, n_h, d_c, d_h, d_h, d_c, act_dt, w_dt, out_dt);
  }
  return hipGetLastError();
}

}  // namespace mla
