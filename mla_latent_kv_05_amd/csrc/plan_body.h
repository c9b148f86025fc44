// Split planner (shared by the planning kernel and the absorption launch
// that carries it).  Cuts each sequence into contiguous block ranges
// ("units"); automatic mode picks the partition length c (in blocks) that
// minimises an estimated makespan  waves(c) * (c + overhead)  over
// 1..max_waves waves of `slots_per_wave` concurrent units, where overhead
// stands for the partial-result write and merge of a split sequence.
#pragma once
#include "device_util.h"
#include "mla_internal.h"

namespace mla {

constexpr int kPlanLdsSeqs = 8192;  // sequence block counts cached in LDS up to this batch
// LDS of the planner: block counts, per-wave reduction slots, the result
constexpr int plan_lds_bytes(int nt) { return kPlanLdsSeqs * 4 + (nt / 64) * 8 + (nt / 64) * 4 + 16; }

__device__ __forceinline__ int nblocks_of(const PlanArgs& a, int b) {
  int L = a.seq_lens[b];
  int n = (L + a.block_size - 1) / a.block_size;
  return n < 1 ? 1 : n;
}

// Sum or maximum over the 64 lanes of a wave, in registers only: two quad
// permutes, the half-row and row mirrors (DPP) give every lane the total of
// its 16-lane row, then the 16- and 32-lane swaps (permlane) combine the
// rows.  Every lane returns the total.  (The LDS-routed shuffles a generic
// reduction uses cost far more per step, and the search below chains many
// of these reductions.)
template <typename Op>
__device__ __forceinline__ int wave_reduce_i32(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true));  // row_mirror
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  v = op((int)r16[0], (int)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return op((int)r32[0], (int)r32[1]);
}
struct OpAdd {
  __device__ int operator()(int x, int y) const { return x + y; }
};
struct OpMax {
  __device__ int operator()(int x, int y) const { return x > y ? x : y; }
};

// ceil(n / c) for 0 < n, c < 2^23 through a float reciprocal plus one correction
__device__ __forceinline__ int ceil_div_small(int n, int c, float rc) {
  int q = (int)((float)(n + c - 1) * rc);
  const int num = n + c - 1;
  if ((q + 1) * c <= num) ++q;
  if (q * c > num) --q;
  return q;
}

// partitions of a sequence with n blocks: explicit count (raised where a
// partition would exceed max_chunk blocks) or ceil(n / chunk)
__device__ __forceinline__ int units_of(const PlanArgs& a, int n, int chunk) {
  if (a.num_splits > 0) {
    int u = min(a.num_splits, n);
    int need = (n + a.max_chunk - 1) / a.max_chunk;
    return max(u, need);
  }
  return (n + chunk - 1) / chunk;
}

// Every candidate partition length c in [lo, hi] (at most 2048 of them) is
// scored in parallel: units(c) = sum_b ceil(n_b / c), waves = ceil(units /
// slots), cost = waves * (c + overhead), overhead charged when any sequence
// is split.  The cheapest c with waves <= max_waves wins (ties: larger c,
// i.e. fewer partial results); if none fits, c = hi.
// The planner's body for a workgroup of NT threads (NT / 64 >= kMaxAutoWaves + 1
// waves); `lds` points at plan_lds_bytes(NT) bytes of the workgroup's LDS
// (a local-memory pointer: every access is a plain LDS instruction).
template <int NT>
__device__ __forceinline__ void plan_body(const PlanArgs& a, __attribute__((address_space(3))) uint8_t* lds) {
  typedef __attribute__((address_space(3))) int pl_int;
  typedef __attribute__((address_space(3))) unsigned long long pl_u64;
  constexpr int kPlanThreads = NT;
  static_assert(NT / 64 >= kMaxAutoWaves + 1, "one wave per wave-count search plus one");
  pl_int* nb = (pl_int*)lds;
  pl_u64* red = (pl_u64*)(lds + kPlanLdsSeqs * 4);
  pl_int* scan = (pl_int*)(lds + kPlanLdsSeqs * 4 + (NT / 64) * 8);
  pl_int& s_chunk = *(pl_int*)(lds + kPlanLdsSeqs * 4 + (NT / 64) * 12);
  pl_int& s_waves = *(pl_int*)(lds + kPlanLdsSeqs * 4 + (NT / 64) * 12 + 4);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool in_lds = a.B <= kPlanLdsSeqs;

  int max_n = 0;
  for (int b = tid; b < a.B; b += kPlanThreads) {
    const int n = nblocks_of(a, b);
    if (in_lds) nb[b] = n;
    max_n = max(max_n, n);
  }
  max_n = wave_reduce_i32(max_n, OpMax());
  if (lane == 0) red[wv] = (unsigned long long)max_n;
  __syncthreads();
  max_n = 0;
  for (int i = 0; i < kPlanThreads / 64; ++i) max_n = max(max_n, (int)red[i]);
  __syncthreads();

  if (a.num_splits <= 0) {
    const int hi = min(max_n, a.max_chunk);
    const int lo = max(1, min(a.min_chunk, hi));
    const int overhead = 4;
    // waves(c) does not grow with c and the cost grows with c inside each
    // interval of equal waves, except where the split overhead drops (c >=
    // the longest sequence).  So the cheapest c is the smallest c reaching
    // waves <= w for some w in 1..max_waves (a binary search each, one
    // wave per w), or c = min(hi, max_n), or the forced fallback c = hi.
    unsigned long long best = ~0ull;  // key = cost << 32 | (0xffff - c) << 8 | waves
    const int nb_lane = (in_lds && lane < a.B) ? nb[lane] : 0;
    auto units_at = [&](int c) {
      const float rc = 1.0f / (float)c;
      int v = 0;
      if (a.B <= 64)
        v = lane < a.B ? ceil_div_small(nb_lane, c, rc) : 0;
      else
        for (int b = lane; b < a.B; b += 64) v += ceil_div_small(in_lds ? nb[b] : nblocks_of(a, b), c, rc);
      return wave_reduce_i32(v, OpAdd());  // uniform result
    };
    auto consider = [&](int c, int u) {
      const int waves = (u + a.slots_per_wave - 1) / a.slots_per_wave;
      if (waves > a.max_waves && c != hi) return;
      const unsigned long long cost = (unsigned long long)waves * (unsigned)(c + (u > a.B ? overhead : 0));
      // ties on cost go to the larger c; the low byte carries waves (diagnostic)
      const unsigned long long key = (cost << 32) | ((unsigned long long)(0xffffu - (unsigned)c) << 8) |
                                     (unsigned)min(waves, 255);
      best = key < best ? key : best;
    };
    if (wv < a.max_waves) {
      const long long cap = (long long)(wv + 1) * a.slots_per_wave;
      int l = lo, h = hi;  // smallest c in [l, h] with units(c) <= cap, if units(hi) <= cap
      if (units_at(hi) <= cap) {
        while (l < h) {
          const int mid = (l + h) >> 1;
          if (units_at(mid) <= cap) h = mid; else l = mid + 1;
        }
        consider(l, units_at(l));
      }
    } else if (wv == kMaxAutoWaves) {
      const int c1 = min(hi, max_n);
      consider(c1, units_at(c1));
      consider(hi, units_at(hi));
    }
    if (lane == 0) red[wv] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long m = ~0ull;
      for (int i = 0; i < kPlanThreads / 64; ++i) m = red[i] < m ? red[i] : m;
      s_chunk = (int)(0xffffu - (unsigned)((m >> 8) & 0xffffu));
      s_waves = (int)(m & 0xffu);
    }
  } else if (tid == 0) {
    s_chunk = 0;
    s_waves = 0;
  }
  __syncthreads();
  const int chunk = s_chunk;

  // per-thread run of consecutive sequences for the prefix sum
  const int per = (a.B + kPlanThreads - 1) / kPlanThreads;
  const int b0 = tid * per, b1 = min(a.B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += units_of(a, in_lds ? nb[b] : nblocks_of(a, b), chunk);
  // inclusive scan: within each wave by shuffles, then across the waves
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) scan[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += scan[i];
  const int total = [&] { int t = 0; for (int i = 0; i < kPlanThreads / 64; ++i) t += scan[i]; return t; }();
  incl += before;
  int first = incl - local;
  for (int b = b0; b < b1; ++b) {
    const int n = in_lds ? nb[b] : nblocks_of(a, b);
    const int u = units_of(a, n, chunk);
    const int len = (n + u - 1) / u;
    const int Lb = max(a.seq_lens[b], 0);
    a.seq[b] = make_int2(first, u);
    for (int k = 0; k < u; ++k) {
      const int s0 = k * len, s1 = min(n, s0 + len);
      // .w: the sequence length, bit-inverted (negative) when it is not split
      a.work[first + k] = make_int4(b, s0, s1, u > 1 ? Lb : ~Lb);
    }
    first += u;
  }
  if (tid == kPlanThreads - 1) {
    WsHeader* h = (WsHeader*)a.ws_header;
    h->n_units = total;
    h->chunk_blocks = chunk;
    h->waves = s_waves;
  }
}


}  // namespace mla
