// Fused tail of a decode step: the split-KV merge of the attention kernel's
// partial rows (log-sum-exp combine) and the W^UV up-projection (itwiki
// "Multi-head latent attention", section "Matrix absorption": values are
// up-projected after the weighted latent sum) in one launch, so the merged
// latent rows never leave the chip:
//   o_lat[t,h,:] = sum_s exp(lse_s - lse) o_part_s[t,h,:],  lse = log sum_s exp(lse_s)
//   o[t,h,:]     = W^UV_h o_lat[t,h,:]
// A workgroup takes one head and 32 query tokens.  The merged rows go to LDS
// as bf16 (the up-projection's operand type, as in the unfused path, where
// the merged o_lat is stored in bf16); each wave then computes 32 output
// dims: O^T[n, t] = W^UV_h[n, :] . o_lat[t, :] on v_mfma_f32_32x32x16_bf16
// (A = weight rows straight from global memory, B = merged rows from LDS).
#include "device_util.h"
#include "mla_internal.h"

namespace mla {

namespace {
typedef __attribute__((address_space(3))) uint8_t cu_lds;
constexpr int kCuDc = 512, kCuDh = 128;
constexpr int kCuRow = kCuDc + 8;  // bf16 elements per staged row (1040 bytes)
constexpr int kCuMaxS = 4;         // partitions merged with all loads in flight
}  // namespace

// 8 waves: waves 0-3 load their 32 weight rows (the A fragments) while
// waves 4-7 merge the partial rows (every load of both issued up front), then
// waves 0-3 run the MFMAs on the merged rows in LDS.
__global__ __launch_bounds__(512) void combine_up_kernel(CombineUpArgs c) {
  __shared__ __attribute__((aligned(16))) uint16_t at[32 * kCuRow];
  const int h = blockIdx.x, t0 = blockIdx.y * 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int R = c.s_q * c.n_h;
  const int T = c.B * c.s_q;
  bf16x8_t wf[kCuDc / 16];
  if (w < 4) {
    // weight rows n = 32w + l32 as A fragments (c = 16kk + 8g ..)
    const uint16_t* wr = c.w_uv + ((long long)h * kCuDh + 32 * w + l32) * kCuDc + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kCuDc / 16; ++kk) wf[kk] = *(const bf16x8_t*)(wr + 16 * kk);
  } else {
    // merge: wave 4 + q takes rows j*4 + q (j = 0..7), lane = 16-byte chunk
    const int q = w - 4;
    int2 sq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + j * 4 + q;
      sq[j] = t < T ? c.seq[t / c.s_q] : make_int2(0, 0);
    }
    u32x4_t pv[8][kCuMaxS];
    float lv[8][kCuMaxS];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + j * 4 + q;
      const long long first = (long long)sq[j].x * R + (t % c.s_q) * c.n_h + h;
#pragma unroll
      for (int k = 0; k < kCuMaxS; ++k) {
        lv[j][k] = -INFINITY;
        pv[j][k] = u32x4_t{0, 0, 0, 0};
      }
      if (t >= T) continue;
      if (sq[j].y <= 1) {  // unsplit: the attention kernel wrote the final row
        pv[j][0] = *(const u32x4_t*)(c.o_fin + ((long long)t * c.n_h + h) * kCuDc + 8 * lane);
      } else if (sq[j].y <= kCuMaxS) {
#pragma unroll
        for (int k = 0; k < kCuMaxS; ++k)
          if (k < sq[j].y) {
            lv[j][k] = c.lse_part[first + (long long)k * R];
            pv[j][k] = *(const u32x4_t*)(c.o_part + (first + (long long)k * R) * kCuDc + 8 * lane);
          }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = j * 4 + q, t = t0 + r;
      const int n = sq[j].y;
      u32x4_t v = pv[j][0];
      if (t < T && n > 1) {
        const long long first = (long long)sq[j].x * R + (t % c.s_q) * c.n_h + h;
        float m = -INFINITY, z = 0.f;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        auto add = [&](float wt, const u32x4_t& x) {
          if (wt == 0.f) return;  // an empty partition may hold anything
          z += wt;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += wt * bf16_bits_to_f32((uint16_t)(x[e] & 0xffffu));
            acc[2 * e + 1] += wt * bf16_bits_to_f32((uint16_t)(x[e] >> 16));
          }
        };
        if (n <= kCuMaxS) {
#pragma unroll
          for (int k = 0; k < kCuMaxS; ++k) m = fmaxf(m, lv[j][k]);
          if (m != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kCuMaxS; ++k)
              if (k < n) add(expf(lv[j][k] - m), pv[j][k]);
          }
        } else {  // many partitions (long contexts): one at a time
          for (int k = 0; k < n; ++k) m = fmaxf(m, c.lse_part[first + (long long)k * R]);
          if (m != -INFINITY)
            for (int k = 0; k < n; ++k)
              add(expf(c.lse_part[first + (long long)k * R] - m),
                  *(const u32x4_t*)(c.o_part + (first + (long long)k * R) * kCuDc + 8 * lane));
        }
        const float iz = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(acc[2 * e] * iz, acc[2 * e + 1] * iz);
        if (c.lse && lane == 0) c.lse[(long long)t * c.n_h + h] = z > 0.f ? m + logf(z) : -INFINITY;
      }
      *(__attribute__((address_space(3))) u32x4_t*)((cu_lds*)at + (r * kCuRow + 8 * lane) * 2) = v;
    }
  }
  __syncthreads();
  if (w >= 4) return;
  // O^T[n = 32w + rows, t = l32] over d_c
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < kCuDc / 16; ++kk) {
    const bf16x8_t bv = *(const __attribute__((address_space(3))) bf16x8_t*)((const cu_lds*)at + (l32 * kCuRow + 16 * kk + 8 * g) * 2);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk], bv, acc, 0, 0, 0);
  }
  const int t = t0 + l32;
  if (t < T) {
    uint16_t* orow = c.out + ((long long)t * c.n_h + h) * kCuDh + 32 * w;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      *(u32x2_t*)(orow + 8 * qd + 4 * g) =
          u32x2_t{pack_bf16x2(acc[4 * qd], acc[4 * qd + 1]), pack_bf16x2(acc[4 * qd + 2], acc[4 * qd + 3])};
  }
}

hipError_t launch_combine_up(const CombineUpArgs& c, hipStream_t s) {
  const int T = c.B * c.s_q;
  hipLaunchKernelGGL(combine_up_kernel, dim3(c.n_h, (T + 31) / 32), dim3(512), 0, s, c);
  return hipGetLastError();
}

}  // namespace mla
