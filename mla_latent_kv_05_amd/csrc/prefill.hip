// MHA-mode prefill attention (itwiki "Multi-head latent attention": sections
// "Decoupled RoPE" and "Matrix absorption"; the article's implementation
// example runs prefill in MHA mode): per head i and query t,
//   o_{t,i} = sum_{j<=t} softmax_j(scale * (q^C_{t,i}.k^C_{j,i} + q^R_{t,i}.k^R_j)) v^C_{j,i}
// with the RoPE key k^R shared by all heads.  Keys and values are the
// materialised k^C = W^UK c^KV, v^C = W^UV c^KV (the expansion runs in the
// up-projection kernel with one latent row per token feeding every head).
//
// MFMA kernel (bf16, d_h = 128, d_r = 64): a workgroup of 4 waves takes one
// head and 128 query rows, wave w rows 32w .. 32w+31.  Keys stream through
// LDS in 32-key subtiles (k^C | k^R rows of 192 values, v^C rows of 128),
// double-buffered: the next subtile's global loads are in flight while the
// current one is used.  Per subtile and wave:
//   S^T[key, query] = K[key, 0:192] . Q^T  (12 v_mfma_f32_32x32x16_bf16; A =
//                     key rows by ds_read_b128, B = the queries in registers)
//   online softmax per query (the lane is the query; exp2 domain, exact
//                     rescale), causal mask on the diagonal subtile
//   O^T[dim, query] += V^T[dim, key] . P^T[key, query]  (8 MFMAs; A = value
//                     columns by ds_read_b64_tr_b16, B = P from the S layout)
#include "device_util.h"
#include "mla_internal.h"

namespace mla {

namespace {

typedef __attribute__((address_space(3))) uint8_t pf_lds;
typedef __attribute__((address_space(3))) u32x4_t pf_lds4;

constexpr int kPfDh = 128, kPfDr = 64, kPfDq = kPfDh + kPfDr;  // 192
constexpr int kPfQ = 128;                                     // query rows per workgroup
constexpr int kPfSub = 32;                                    // keys per subtile
constexpr int kPfKRow = kPfDq * 2 + 16;                        // 400 B: padded key row
constexpr int kPfVRow = kPfDh * 2 + 16;                        // 272 B: padded value row
constexpr int kPfKTile = kPfSub * kPfKRow;                     // 12,800 B
constexpr int kPfVTile = kPfSub * kPfVRow;                     // 8,704 B
constexpr int kPfStage = kPfKTile + kPfVTile;                  // 21,504 B
constexpr int kPfChunksK = kPfSub * (kPfDq / 8);               // 768 16-byte pieces
constexpr int kPfChunks = kPfChunksK + kPfSub * (kPfDh / 8);   // 1280
constexpr int kPfLoads = kPfChunks / 256;                      // 5 per thread

__device__ __forceinline__ bf16x4_t pf_tr16(const pf_lds* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
}

}  // namespace

__global__ __launch_bounds__(256) void prefill_mfma_kernel(const uint16_t* q, const uint16_t* kc,
                                                           const uint16_t* kr, const uint16_t* v, void* out,
                                                           float* lse, int T, int n_h, float scale2,
                                                           int out_bf16) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * kPfStage];
  pf_lds* smem = (pf_lds*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, j16 = lane & 15, G = lane >> 4;
  const int h = blockIdx.y;
  const int qb = blockIdx.x * kPfQ;
  const int q0 = qb + 32 * w;  // this wave's first query
  const int qrow = q0 + l32;   // this lane's query
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

  // global -> registers -> LDS staging of subtile s (zeros past T)
  u32x4_t st[kPfLoads];
  auto load_sub = [&](int s) {
#pragma unroll
    for (int i = 0; i < kPfLoads; ++i) {
      const int c = tid + 256 * i;
      st[i] = u32x4_t{0, 0, 0, 0};
      int key, part;
      if (c < kPfChunksK) {
        key = s * kPfSub + c / (kPfDq / 8);
        part = c % (kPfDq / 8);
        if (key < T) {
          if (part < kPfDh / 8)
            st[i] = *(const u32x4_t*)(kc + key * ldk + (long long)h * kPfDh + 8 * part);
          else
            st[i] = *(const u32x4_t*)(kr + (long long)key * kPfDr + 8 * (part - kPfDh / 8));
        }
      } else {
        const int c2 = c - kPfChunksK;
        key = s * kPfSub + c2 / (kPfDh / 8);
        part = c2 % (kPfDh / 8);
        if (key < T) st[i] = *(const u32x4_t*)(v + key * ldk + (long long)h * kPfDh + 8 * part);
      }
    }
  };
  auto store_sub = [&](int buf) {
    pf_lds* base = smem + buf * kPfStage;
#pragma unroll
    for (int i = 0; i < kPfLoads; ++i) {
      const int c = tid + 256 * i;
      if (c < kPfChunksK)
        *(pf_lds4*)(base + (c / (kPfDq / 8)) * kPfKRow + (c % (kPfDq / 8)) * 16) = st[i];
      else {
        const int c2 = c - kPfChunksK;
        *(pf_lds4*)(base + kPfKTile + (c2 / (kPfDh / 8)) * kPfVRow + (c2 % (kPfDh / 8)) * 16) = st[i];
      }
    }
  };

  // value fragment offsets (transposed reads): rows ta (first 4 k-slots) and
  // ta + 8 (last 4) of a 16-key step; dims of block db: 32db + 16(G&1) + 4(j16&3)
  const int ta = 4 * g + (j16 >> 2);
  const int vcol = (16 * (G & 1) + 4 * (j16 & 3)) * 2;

  f32x16_t acc[kPfDh / 32];
#pragma unroll
  for (int d = 0; d < kPfDh / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  load_sub(0);
  store_sub(0);
  __syncthreads();
  for (int s = 0; s < n_sub; ++s) {
    if (s + 1 < n_sub) load_sub(s + 1);  // in flight during this subtile
    const pf_lds* kt = smem + (s & 1) * kPfStage;
    const pf_lds* vt = kt + kPfKTile;
    const int j0 = s * kPfSub;
    if (j0 < wave_end) {  // uniform per wave: some of these keys are visible
      // ---- S^T = K . Q^T
      f32x16_t sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
      for (int f = 0; f < kPfDq / 16; ++f) {
        const bf16x8_t ka = *(const __attribute__((address_space(3))) bf16x8_t*)(kt + l32 * kPfKRow + (16 * f + 8 * g) * 2);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[f], sc, 0, 0, 0);
      }
      // ---- causal mask (diagonal subtile) and online softmax, exp2 domain
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * g + (r & 3);
        sc[r] = key <= qrow && key < T ? sc[r] * scale2 : -INFINITY;
        mx = fmaxf(mx, sc[r]);
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_new = fmaxf(m_run, mx);
      const float corr = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      float ps = 0.f;
      bf16x8_t P[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[r] - m_new);
        ps += p;
        P[r >> 3][r & 7] = (__bf16)p;
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
        ps = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      l_run = l_run * corr + ps;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < kPfDh / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= corr;
      // ---- O^T += V^T . P^T: keys 16ks + {4g..4g+3, 8+4g..8+4g+3}
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int d = 0; d < kPfDh / 32; ++d) {
          const pf_lds* p0 = vt + (16 * ks + ta) * kPfVRow + 32 * d * 2 + vcol;
          const bf16x4_t lo = pf_tr16(p0);
          const bf16x4_t hi = pf_tr16(p0 + 8 * kPfVRow);
          bf16x8_t va;
          va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
          va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[ks], acc[d], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with buffer s & 1
    if (s + 1 < n_sub) {
      store_sub((s + 1) & 1);
      __syncthreads();
    }
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
    dim3 grid((T + kPfQ - 1) / kPfQ, n_h);
    hipLaunchKernelGGL(prefill_mfma_kernel, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)kc,
                       (const uint16_t*)kr, (const uint16_t*)v, out, lse, T, n_h, scale * kLog2e,
                       out_dtype == 1 ? 1 : 0);
  } else {
    const long long rows = (long long)T * n_h;
    hipLaunchKernelGGL(prefill_generic_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, q, kc, kr, v,
                       out, lse, T, n_h, d_h, d_r, scale, in_dtype, out_dtype);
  }
  return hipGetLastError();
}

}  // namespace mla
