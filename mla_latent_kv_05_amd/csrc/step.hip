// Fused tail of a decode step: the split-KV merge of the attention kernel's
// partial rows (log-sum-exp combine) and the W^UV up-projection (itwiki
// "Multi-head latent attention", section "Matrix absorption": values are
// up-projected after the weighted latent sum) in one launch, so the merged
// latent rows never leave the chip:
//   o_lat[t,h,:] = sum_s exp(lse_s - lse) o_part_s[t,h,:],  lse = log sum_s exp(lse_s)
//   o[t,h,:]     = W^UV_h o_lat[t,h,:]
// A workgroup takes one head and a share of the 32-token blocks (one
// workgroup per compute unit; the head's weight block stays in LDS across
// its blocks).  The merged rows go to LDS
// as bf16 (the up-projection's operand type, as in the unfused path, where
// the merged o_lat is stored in bf16); each of four waves then computes 32
// output dims: O^T[n, t] = W^UV_h[n, :] . o_lat[t, :] on
// v_mfma_f32_32x32x16_bf16 (A = weight rows, B = merged rows, both from LDS).
#include <type_traits>

#include "mfma_common.h"

namespace mla {

namespace {
typedef __attribute__((address_space(3))) uint8_t cu_lds;
constexpr int kCuDc = 512, kCuDh = 128;
constexpr int kCuMaxS = 4;         // partitions merged with all loads in flight
constexpr int kCuBatch = 8;        // partitions per batch beyond that
}  // namespace

// 8 waves.  Each wave loads 16 whole rows of the head's weight block W^UV_h
// (128 x 512 bf16; one 1 KB row per load instruction) while all waves merge
// the partial rows of the 32 tokens into a bf16 tile in LDS; the weight rows
// follow into LDS, then waves 0-3 run the MFMAs from LDS.  Both blocks use 1 KB rows
// whose 16-byte chunk c sits at c ^ (row & 15), so the 16 rows one
// ds_read_b128 phase touches fall on 16 different bank groups.
constexpr int kCuWB = kCuDh * kCuDc * 2;  // 131072
constexpr int kCuAB = 32 * kCuDc * 2;     // 32768
constexpr int kCuLds = kCuWB + kCuAB;     // 163840
__device__ __forceinline__ int cu_chunk(int c, int row) { return c ^ (row & 15); }

__global__ __launch_bounds__(512) void combine_up_kernel(CombineUpArgs c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  cu_lds* wl = (cu_lds*)smem_raw;
  cu_lds* al = wl + kCuWB;
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int R = c.s_q * c.n_h;
  const int T = c.B * c.s_q;
  const int nblk = (T + 31) / 32;
  // one 32-token block; the first block of a workgroup also brings the
  // head's weight block into LDS (a separate instantiation, so its 64
  // registers are not held across the loop)
  auto block = [&](int tb, auto with_w) __attribute__((always_inline)) {
    constexpr bool kW = decltype(with_w)::value;
    const int t0 = tb * 32;
    // the tokens' partition lists first (their round trip gates the partial
    // loads)
    int2 sq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + j * 8 + w;
      sq[j] = t < T ? c.seq[t / c.s_q] : make_int2(0, 0);
      // a partition list outside the workspace (no plan of this batch there):
      // read the unsplit row instead
      if (sq[j].x < 0 || sq[j].y < 0 || sq[j].x > c.units_max - sq[j].y) sq[j] = make_int2(0, 1);
    }
    u32x4_t wv[16];
    if constexpr (kW) {  // then the weight rows 16w .. 16w+15 (lane = 16-byte chunk)
      const uint16_t* wr = c.w_uv + ((long long)h * kCuDh + 16 * w) * kCuDc + 8 * lane;
#pragma unroll
      for (int i = 0; i < 16; ++i) wv[i] = *(const u32x4_t*)(wr + i * kCuDc);
    }
    u32x4_t pv[4][kCuMaxS];
    float lv[4][kCuMaxS];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + j * 8 + w;
      const long long first = (long long)sq[j].x * R + (t % c.s_q) * c.n_h + h;
#pragma unroll
      for (int k = 0; k < kCuMaxS; ++k) {
        lv[j][k] = -INFINITY;
        pv[j][k] = u32x4_t{0, 0, 0, 0};
      }
      if (t >= T) continue;
      if (sq[j].y <= 1) {  // unsplit: the attention kernel wrote the final row into the unit's slot
        pv[j][0] = *(const u32x4_t*)(c.o_part + first * kCuDc + 8 * lane);
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
    for (int j = 0; j < 4; ++j) {
      const int r = j * 8 + w, t = t0 + r;
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
        } else {  // many partitions (long contexts): online over batches of
                  // kCuBatch with every load of a batch in flight
          for (int k0 = 0; k0 < n; k0 += kCuBatch) {
            float lb[kCuBatch];
            u32x4_t xb[kCuBatch];
#pragma unroll
            for (int i = 0; i < kCuBatch; ++i) {  // past the end: the last partition again, weight 0
              const long long p = first + (long long)min(k0 + i, n - 1) * R;
              lb[i] = c.lse_part[p];
              xb[i] = *(const u32x4_t*)(c.o_part + p * kCuDc + 8 * lane);
            }
            float mb = m;
#pragma unroll
            for (int i = 0; i < kCuBatch; ++i)
              if (k0 + i < n) mb = fmaxf(mb, lb[i]);
            if (mb == -INFINITY) continue;  // only empty partitions so far
            const float sc = expf(m - mb);  // 0 while nothing has been added
            z *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= sc;
            m = mb;
#pragma unroll
            for (int i = 0; i < kCuBatch; ++i)
              if (k0 + i < n) add(expf(lb[i] - m), xb[i]);
          }
        }
        const float iz = z > 0.f ? 1.f / z : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(acc[2 * e] * iz, acc[2 * e + 1] * iz);
        if (c.lse && lane == 0) c.lse[(long long)t * c.n_h + h] = z > 0.f ? m + logf(z) : -INFINITY;
      }
      *(__attribute__((address_space(3))) u32x4_t*)(al + r * (kCuDc * 2) + (cu_chunk(lane, r) << 4)) = v;
    }
    if constexpr (kW) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 16 * w + i;
        *(__attribute__((address_space(3))) u32x4_t*)(wl + row * (kCuDc * 2) + (cu_chunk(lane, row) << 4)) = wv[i];
      }
    }
    __syncthreads();  // every weight row and merged row visible
    if (w < 4) {
      // O^T[n = 32w + rows, t = l32] over d_c: A = weight row n, B = merged row t
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const int nrow = 32 * w + l32;
#pragma unroll
      for (int kk = 0; kk < kCuDc / 16; ++kk) {
        const int ch = 2 * kk + g;
        const bf16x8_t av = *(const __attribute__((address_space(3))) bf16x8_t*)(wl + nrow * (kCuDc * 2) + (cu_chunk(ch, nrow) << 4));
        const bf16x8_t bv = *(const __attribute__((address_space(3))) bf16x8_t*)(al + l32 * (kCuDc * 2) + (cu_chunk(ch, l32) << 4));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
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
    __syncthreads();  // the merged tile is free for the next token block
  };
  if (blockIdx.y >= nblk) return;
  block(blockIdx.y, std::true_type{});
  for (int tb = blockIdx.y + gridDim.y; tb < nblk; tb += gridDim.y) block(tb, std::false_type{});
}

hipError_t launch_combine_up(const CombineUpArgs& c, int n_cu, hipStream_t s) {
  static std::atomic<uint64_t> lds_raised{0};
  if (const hipError_t e = ensure_dynamic_lds((const void*)combine_up_kernel, kCuLds, lds_raised); e != hipSuccess)
    return e;
  // one workgroup per compute unit (the LDS allows no more): heads x token
  // groups, each workgroup looping over its share of the 32-token blocks
  const int T = c.B * c.s_q;
  const int nblk = (T + 31) / 32;
  int gy = n_cu > c.n_h ? n_cu / c.n_h : 1;
  if (gy > nblk) gy = nblk;
  hipLaunchKernelGGL(combine_up_kernel, dim3(c.n_h, gy), dim3(512), kCuLds, s, c);
  return hipGetLastError();
}

}  // namespace mla
