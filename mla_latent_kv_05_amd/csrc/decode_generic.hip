// Split planning, the portable fp32 decode kernel, and the log-sum-exp combine.
//
// Method: itwiki "Multi-head latent attention", sections "Decoupled RoPE" and
// "Matrix absorption" -- in MQA mode each head's latent query is dotted with
// the cached c^KV, the RoPE term q^R.k^R is added, scores are scaled by
// 1/sqrt(d_h + d_h^R), softmaxed over the keys j <= t, and the weights sum
// the c^KV rows.  Split-KV partitions and their log-sum-exp merge are this
// library's mechanism for spreading one sequence over many compute units.
#include "device_util.h"
#include "mla_internal.h"
#include "plan_body.h"

namespace mla {

// ============================================================== planner
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[plan_lds_bytes(kPlanThreads)];
  plan_body<kPlanThreads>(a, (__attribute__((address_space(3))) uint8_t*)lds);
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

// ============================================================== generic decode
// One wavefront per query row (query token i, head h), exact online softmax
// token by token in fp32.  Lanes split the d_c + d_r dimensions.  Any shapes
// within the ABI limits, fp32 / bf16 / fp8 / int4 / int2 caches.

constexpr int kMaxQ = 36;  // (2048 + 256) / 64
constexpr int kMaxC = 32;  // 2048 / 64

// value e of a row of packed b-bit codes: 32/b values per little-endian
// 32-bit word, value 2k at bit k*b, value 2k+1 at bit 16 + k*b
__device__ __forceinline__ int packed_code(const uint32_t* words, int e, int b) {
  const int per = 32 / b, i = e % per;
  const int shift = (i & 1) ? 16 + (i >> 1) * b : (i >> 1) * b;
  return (int)((words[e / per] >> shift) & ((1u << b) - 1u));
}

template <int KV>
__device__ __forceinline__ void load_kv_row(const DecodeArgs& a, const uint8_t* blk, int slot,
                                            int lane, int nc, float* cv, float* kr_out) {
  // content dims lane + 64k (k < nc) and RoPE dims lane + 64k (k < 4)
  if (KV == 3 || KV == 4) {  // int4 / int2: [codes | RoPE codes | (scale, min) fp16 per 32 values]
    constexpr int cb = KV == 3 ? 4 : 2;
    const size_t crow = (size_t)a.d_c * cb / 8, rrow = (size_t)a.d_r / 2;
    const int ng = (a.d_c + a.d_r) / 32;
    const uint32_t* cw = (const uint32_t*)(blk + (size_t)slot * crow);
    const uint32_t* rw = (const uint32_t*)(blk + (size_t)a.block_size * crow + (size_t)slot * rrow);
    const _Float16* prm = (const _Float16*)(blk + (size_t)a.block_size * (crow + rrow)) + (size_t)slot * ng * 2;
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      const int d = lane + 64 * k;
      cv[k] = 0.f;
      if (k < nc && d < a.d_c) {
        const int g = d / 32;
        cv[k] = (float)packed_code(cw, d, cb) * (float)prm[2 * g] + (float)prm[2 * g + 1];
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = lane + 64 * k;
      kr_out[k] = 0.f;
      if (d < a.d_r) {
        const int g = (a.d_c + d) / 32;
        kr_out[k] = (float)packed_code(rw, d, 4) * (float)prm[2 * g] + (float)prm[2 * g + 1];
      }
    }
  } else if (KV == 2) {  // fp8: [bs*d_c codes | bs*d_r bf16 | bs fp32 scale]
    const uint8_t* codes = blk + (size_t)slot * a.d_c;
    const uint16_t* kr = (const uint16_t*)(blk + (size_t)a.block_size * a.d_c) + (size_t)slot * a.d_r;
    const float sc = ((const float*)(blk + (size_t)a.block_size * (a.d_c + 2 * a.d_r)))[slot];
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      int d = lane + 64 * k;
      cv[k] = (k < nc && d < a.d_c) ? e4m3fn_to_f32(codes[d]) * sc : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int d = lane + 64 * k;
      kr_out[k] = d < a.d_r ? bf16_bits_to_f32(kr[d]) : 0.f;
    }
  } else {
    const size_t row = (size_t)slot * (a.d_c + a.d_r);
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      int d = lane + 64 * k;
      cv[k] = (k < nc && d < a.d_c) ? load_elem(blk, row + d, KV) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int d = lane + 64 * k;
      kr_out[k] = d < a.d_r ? load_elem(blk, row + a.d_c + d, KV) : 0.f;
    }
  }
}

template <int KV>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int R = a.s_q * a.n_h;
  const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int qi = r / a.n_h, h = r % a.n_h;
  const int nc = (a.d_c + 63) / 64;
  const int n_units = ((const WsHeader*)a.ws_header)->n_units;

  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int4 wk = a.work[unit];
    const int b = wk.x;
    const int L = wk.w < 0 ? ~wk.w : wk.w;
    const int vis = L - a.s_q + qi + 1;
    const int t0 = wk.y * a.block_size;
    const int t1 = min(wk.z * a.block_size, vis);

    const long long qrow = ((long long)b * a.s_q + qi) * a.n_h + h;
    float qc[kMaxC], qr[4], acc[kMaxC];
#pragma unroll
    for (int k = 0; k < kMaxC; ++k) {
      int d = lane + 64 * k;
      qc[k] = (k < nc && d < a.d_c) ? load_elem(a.q_lat, qrow * a.d_c + d, a.q_dtype) : 0.f;
      acc[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int d = lane + 64 * k;
      qr[k] = d < a.d_r ? load_elem(a.q_rope, qrow * a.d_r + d, a.q_dtype) : 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int j = t0; j < t1; ++j) {
      const int pb = a.table[(long long)b * a.max_blocks + j / a.block_size];
      const uint8_t* blk = (const uint8_t*)a.kv + (long long)pb * a.block_bytes;
      float cv[kMaxC], kr[4];
      load_kv_row<KV>(a, blk, j % a.block_size, lane, nc, cv, kr);
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxC; ++k)
        if (k < nc) part += qc[k] * cv[k];
#pragma unroll
      for (int k = 0; k < 4; ++k) part += qr[k] * kr[k];
      const float s = wave_sum(part) * a.scale;
      const float m_new = fmaxf(m, s);
      const float f = expf(m - m_new);  // m = -inf -> 0
      const float p = expf(s - m_new);
      l = l * f + p;
#pragma unroll
      for (int k = 0; k < kMaxC; ++k)
        if (k < nc) acc[k] = acc[k] * f + p * cv[k];
      m = m_new;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse_v = l > 0.f ? m + logf(l) : -INFINITY;
    if (wk.w < 0) {
#pragma unroll
      for (int k = 0; k < kMaxC; ++k) {
        int d = lane + 64 * k;
        if (k < nc && d < a.d_c) store_elem(a.out, qrow * a.d_c + d, acc[k] * inv, a.out_dtype);
      }
      if (lane == 0 && a.lse) a.lse[qrow] = lse_v;
    } else {
      const long long prow = (long long)unit * R + r;  // partial slot = unit index
#pragma unroll
      for (int k = 0; k < kMaxC; ++k) {
        int d = lane + 64 * k;
        if (k < nc && d < a.d_c) a.o_part[prow * a.d_c + d] = acc[k] * inv;
      }
      if (lane == 0) a.lse_part[prow] = lse_v;
    }
  }
}

hipError_t launch_decode_generic(const DecodeArgs& a, int units_max, hipStream_t s) {
  const int R = a.s_q * a.n_h;
  dim3 grid(units_max < 1024 ? units_max : 1024, (R + 3) / 4);
  if (a.kv_dtype == 0)
    hipLaunchKernelGGL(decode_generic_kernel<0>, grid, dim3(256), 0, s, a);
  else if (a.kv_dtype == 1)
    hipLaunchKernelGGL(decode_generic_kernel<1>, grid, dim3(256), 0, s, a);
  else if (a.kv_dtype == 2)
    hipLaunchKernelGGL(decode_generic_kernel<2>, grid, dim3(256), 0, s, a);
  else if (a.kv_dtype == 3)
    hipLaunchKernelGGL(decode_generic_kernel<3>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_generic_kernel<4>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ============================================================== combine
// lse = log sum_s exp(lse_s); out = sum_s exp(lse_s - lse) o_s.  One thread
// per 4 output values.

__device__ __forceinline__ void merge_row(const float* o_base, long long o_stride,
                                          const float* l_base, long long l_stride, int S,
                                          int c4, float4& out, float& lse_out) {
  float m = -INFINITY;
  for (int k = 0; k < S; ++k) m = fmaxf(m, l_base[k * l_stride]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float z = 0.f;
  if (m != -INFINITY) {
    for (int k = 0; k < S; ++k) {
      const float w = expf(l_base[k * l_stride] - m);
      if (w == 0.f) continue;  // an empty split may hold anything in o
      const float4 v = ((const float4*)(o_base + k * o_stride))[c4];
      acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
      z += w;
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  lse_out = z > 0.f ? m + logf(z) : -INFINITY;
}

// the same merge over bf16 partial rows
__device__ __forceinline__ void merge_row_bf16(const uint16_t* o_base, long long o_stride,
                                               const float* l_base, long long l_stride, int S,
                                               int c4, float4& out, float& lse_out) {
  float m = -INFINITY;
  for (int k = 0; k < S; ++k) m = fmaxf(m, l_base[k * l_stride]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float z = 0.f;
  if (m != -INFINITY) {
    for (int k = 0; k < S; ++k) {
      const float w = expf(l_base[k * l_stride] - m);
      if (w == 0.f) continue;
      const uint2 pk = ((const uint2*)(o_base + k * o_stride))[c4];
      acc.x += w * bf16_bits_to_f32((uint16_t)(pk.x & 0xffffu));
      acc.y += w * bf16_bits_to_f32((uint16_t)(pk.x >> 16));
      acc.z += w * bf16_bits_to_f32((uint16_t)(pk.y & 0xffffu));
      acc.w += w * bf16_bits_to_f32((uint16_t)(pk.y >> 16));
      z += w;
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  out = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  lse_out = z > 0.f ? m + logf(z) : -INFINITY;
}

__device__ __forceinline__ void store4(void* out, long long base, float4 v, int dt) {
  if (dt == 0) {
    *(float4*)((float*)out + base) = v;
  } else {
    uint16_t* o = (uint16_t*)out + base;
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
    pk.y = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
    *(uint2*)o = pk;
  }
}

// Merge of a decode call's own partial rows: one thread per 8 consecutive
// elements of a row (16-byte loads of bf16 partials, two of fp32), the loads
// of all partitions issued before they are consumed.
template <bool PBF16>
__global__ __launch_bounds__(256) void combine_units8_kernel(DecodeArgs a) {
  const int bq = blockIdx.y;
  const int b = bq / a.s_q, qi = bq % a.s_q;
  const int2 sq = a.seq[b];
  if (sq.y <= 1) return;
  const int d8 = a.d_c / 8;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int h = idx / d8, c8 = idx % d8;
  if (h >= a.n_h) return;
  const int R = a.s_q * a.n_h;
  const long long prow = (long long)sq.x * R + qi * a.n_h + h;
  const float* lp = a.lse_part + prow;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f, m = -INFINITY;
  auto add = [&](float wk, const u32x4_t& v16, const f32x4_t& lo, const f32x4_t& hi) {
    if (wk == 0.f) return;  // an empty partition may hold anything
    z += wk;
    if constexpr (PBF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += wk * bf16_bits_to_f32((uint16_t)(v16[j] & 0xffffu));
        acc[2 * j + 1] += wk * bf16_bits_to_f32((uint16_t)(v16[j] >> 16));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += wk * lo[j];
        acc[4 + j] += wk * hi[j];
      }
    }
  };
  auto load = [&](int k, u32x4_t& v16, f32x4_t& lo, f32x4_t& hi) {
    const long long e = (prow + (long long)k * R) * a.d_c + 8 * c8;
    if constexpr (PBF16) {
      v16 = *(const u32x4_t*)((const uint16_t*)a.o_part + e);
    } else {
      lo = *(const f32x4_t*)(a.o_part + e);
      hi = *(const f32x4_t*)(a.o_part + e + 4);
    }
  };
  constexpr int kU = 8;
  if (sq.y <= kU) {
    // every load (log-sum-exps and rows) in flight at once: one round trip
    float l[kU];
    u32x4_t v16[kU];
    f32x4_t lo[kU], hi[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k)
      if (k < sq.y) {
        l[k] = lp[(long long)k * R];
        load(k, v16[k], lo[k], hi[k]);
      }
#pragma unroll
    for (int k = 0; k < kU; ++k)
      if (k < sq.y) m = fmaxf(m, l[k]);
    if (m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kU; ++k)
        if (k < sq.y) add(expf(l[k] - m), v16[k], lo[k], hi[k]);
    }
  } else {
    for (int k = 0; k < sq.y; ++k) m = fmaxf(m, lp[(long long)k * R]);
    if (m != -INFINITY) {
      for (int k0 = 0; k0 < sq.y; k0 += 4) {
        float wk[4];
        u32x4_t v16[4];
        f32x4_t lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k = k0 + u;
          wk[u] = k < sq.y ? expf(lp[(long long)k * R] - m) : 0.f;
          if (k < sq.y) load(k, v16[u], lo[u], hi[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) add(wk[u], v16[u], lo[u], hi[u]);
      }
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const long long orow = ((long long)b * a.s_q + qi) * a.n_h + h;
  const long long ob = orow * a.d_c + 8 * c8;
  if (a.out_dtype == 0) {
    *(f32x4_t*)((float*)a.out + ob) = f32x4_t{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *(f32x4_t*)((float*)a.out + ob + 4) = f32x4_t{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  } else {
    u32x4_t pk;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pk[j] = (uint32_t)f32_to_bf16_bits(acc[2 * j] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * j + 1] * inv) << 16);
    *(u32x4_t*)((uint16_t*)a.out + ob) = pk;
  }
  if (c8 == 0 && a.lse) a.lse[orow] = z > 0.f ? m + logf(z) : -INFINITY;
}

__global__ __launch_bounds__(256) void combine_units_kernel(DecodeArgs a) {
  const int bq = blockIdx.y;
  const int b = bq / a.s_q, qi = bq % a.s_q;
  const int2 sq = a.seq[b];
  if (sq.y <= 1) return;
  const int d4 = a.d_c / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int h = idx / d4, c4 = idx % d4;
  if (h >= a.n_h) return;
  const int R = a.s_q * a.n_h;
  const int r = qi * a.n_h + h;
  const long long prow = (long long)sq.x * R + r;
  float4 o;
  float lse_v;
  if (a.part_bf16)
    merge_row_bf16((const uint16_t*)a.o_part + prow * a.d_c, (long long)R * a.d_c, a.lse_part + prow, R, sq.y,
                   c4, o, lse_v);
  else
    merge_row(a.o_part + prow * a.d_c, (long long)R * a.d_c, a.lse_part + prow, R, sq.y, c4, o, lse_v);
  const long long orow = ((long long)b * a.s_q + qi) * a.n_h + h;
  store4(a.out, orow * a.d_c + 4 * c4, o, a.out_dtype);
  if (c4 == 0 && a.lse) a.lse[orow] = lse_v;
}

// Merge for sequences cut into many partitions (long contexts): one
// workgroup per output row; its four wavefronts take every fourth partition
// (one 8-element piece of the row per lane) and add their sums through LDS.
constexpr int kWideMaxS = 1024;
template <bool PBF16>
__global__ __launch_bounds__(256) void combine_units_wide_kernel(DecodeArgs a) {
  __shared__ float wsh[kWideMaxS];
  __shared__ float part[4][64][9];
  __shared__ float rsh[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int R = a.s_q * a.n_h;
  const int row = blockIdx.x;                 // (b, qi, h)
  const int b = row / R, r = row % R;
  const int2 sq = a.seq[b];
  if (sq.y <= 1) return;
  const int S = sq.y;
  const long long prow = (long long)sq.x * R + r;
  // partition weights exp(lse_s - max) and their sum
  float m = -INFINITY;
  for (int k = tid; k < S; k += 256) m = fmaxf(m, a.lse_part[prow + (long long)k * R]);
  m = wave_max(m);
  if (lane == 0) rsh[wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(rsh[0], rsh[1]), fmaxf(rsh[2], rsh[3]));
  const bool cached = S <= kWideMaxS;  // weights kept in LDS, else recomputed
  float zl = 0.f;
  for (int k = tid; k < S; k += 256) {
    const float wk = m == -INFINITY ? 0.f : expf(a.lse_part[prow + (long long)k * R] - m);
    if (cached) wsh[k] = wk;
    zl += wk;
  }
  zl = wave_sum(zl);
  __syncthreads();  // wsh complete; rsh reads done
  if (lane == 0) rsh[wv] = zl;
  // this lane's 8 elements, partitions wv, wv+4, ...
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int pieces = a.d_c / 8;
  if (lane < pieces) {
    for (int k = wv; k < S; k += 4) {
      const float wk = cached ? wsh[k] : (m == -INFINITY ? 0.f : expf(a.lse_part[prow + (long long)k * R] - m));
      if (wk == 0.f) continue;  // an empty partition may hold anything
      const long long e = (prow + (long long)k * R) * a.d_c + 8 * lane;
      if constexpr (PBF16) {
        const u32x4_t v = *(const u32x4_t*)((const uint16_t*)a.o_part + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += wk * bf16_bits_to_f32((uint16_t)(v[j] & 0xffffu));
          acc[2 * j + 1] += wk * bf16_bits_to_f32((uint16_t)(v[j] >> 16));
        }
      } else {
        const f32x4_t lo = *(const f32x4_t*)(a.o_part + e), hi = *(const f32x4_t*)(a.o_part + e + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] += wk * lo[j];
          acc[4 + j] += wk * hi[j];
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[wv][lane][j] = acc[j];
  __syncthreads();
  if (wv == 0 && lane < pieces) {
    const float z = rsh[0] + rsh[1] + rsh[2] + rsh[3];
    const float inv = z > 0.f ? 1.f / z : 0.f;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (part[0][lane][j] + part[1][lane][j] + part[2][lane][j] + part[3][lane][j]) * inv;
    const long long orow = (long long)b * R + r;
    const long long ob = orow * a.d_c + 8 * lane;
    if (a.out_dtype == 0) {
      *(f32x4_t*)((float*)a.out + ob) = f32x4_t{o[0], o[1], o[2], o[3]};
      *(f32x4_t*)((float*)a.out + ob + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
    } else {
      *(u32x4_t*)((uint16_t*)a.out + ob) =
          u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    }
    if (lane == 0 && a.lse) a.lse[orow] = z > 0.f ? m + logf(z) : -INFINITY;
  }
}

hipError_t launch_combine_units(const DecodeArgs& a, hipStream_t s, int expect_splits) {
  // many partitions per sequence: spread each row's partitions over a
  // workgroup (the kernel itself handles up to kWideMaxS partitions)
  if (expect_splits > 8 && a.d_c % 8 == 0 && a.d_c <= 512) {
    dim3 grid(a.B * a.s_q * a.n_h);
    if (a.part_bf16)
      hipLaunchKernelGGL(combine_units_wide_kernel<true>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(combine_units_wide_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // 8-wide path when rows split into 16-byte pieces (d_c % 8 == 0 keeps every
  // fp32 / bf16 row start 16-byte aligned given 256-byte aligned buffers)
  if (a.d_c % 8 == 0) {
    const int per = a.n_h * (a.d_c / 8);
    dim3 grid((per + 255) / 256, a.B * a.s_q);
    if (a.part_bf16)
      hipLaunchKernelGGL(combine_units8_kernel<true>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(combine_units8_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int per = a.n_h * (a.d_c / 4);
  dim3 grid((per + 255) / 256, a.B * a.s_q);
  hipLaunchKernelGGL(combine_units_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void combine_lse_kernel(const float* o_part, const float* lse_part,
                                                          const int32_t* splits, int N, int S, int D,
                                                          void* out, float* lse_out, int out_dt) {
  const int d4 = D / 4;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)N * d4) return;
  const int n = (int)(idx / d4), c4 = (int)(idx % d4);
  int cnt = splits ? splits[n] : S;
  cnt = cnt < 0 ? 0 : (cnt > S ? S : cnt);
  float4 o;
  float lse_v;
  merge_row(o_part + (long long)n * S * D, D, lse_part + (long long)n * S, 1, cnt, c4, o, lse_v);
  store4(out, (long long)n * D + 4 * c4, o, out_dt);
  if (c4 == 0 && lse_out) lse_out[n] = lse_v;
}

hipError_t launch_combine_lse(const float* o_part, const float* lse_part, const int32_t* splits,
                              int N, int S, int D, void* out, float* lse_out, int out_dtype,
                              hipStream_t s) {
  long long total = (long long)N * (D / 4);
  dim3 grid((unsigned)((total + 255) / 256));
  hipLaunchKernelGGL(combine_lse_kernel, grid, dim3(256), 0, s, o_part, lse_part, splits, N, S, D,
                     out, lse_out, out_dtype);
  return hipGetLastError();
}

}  // namespace mla
