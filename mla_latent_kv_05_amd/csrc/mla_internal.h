// Internal declarations shared by the HIP translation units of libmla.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mla {

// Raises a kernel's dynamic-LDS limit on the current device the first time
// the kernel is launched there (the attribute is per device); `done` holds
// one bit per device id below 64 (beyond that the call is made every time).
inline hipError_t ensure_dynamic_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// ---------------------------------------------------------------- workspace
// Layout of the decode workspace (all offsets 256-byte aligned):
//   [0]           WsHeader
//   work          int4[units_max]    (b, first_block, end_block, L or ~L); a split
//                                    unit's partial rows sit at slot = its index
//   seq           int2[B]            (first unit, unit count)
//   lse_part      float[units_max * R]
//   o_part        float[units_max * R * d_c]  (bf16 rows when the decode kernel
//                 writes bf16 partials; the space is sized for fp32)
// with R = s_q * n_h rows per sequence.  slot = -1 marks a sequence that has
// a single unit: that unit writes the final output directly.
struct WsHeader {
  int n_units;
  int chunk_blocks;  // planned partition length in blocks (diagnostic)
  int waves;         // planned waves of units (diagnostic)
  int pad[61];
};

struct WsLayout {
  size_t work, seq, lse_part, o_part, total;
  int units_max;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Upper bound on work units: explicit splits -> B*splits; automatic planning
// -> up to `max_waves` waves of `slots` units plus one rounding unit per sequence.
constexpr int kMaxAutoWaves = 3;

// layout for room for `units` plan entries, partial rows of `part_elem`
// bytes per value
inline WsLayout ws_layout_units(int B, int s_q, int n_h, int d_c, long long units, int part_elem) {
  WsLayout L{};
  L.units_max = (int)units;
  size_t R = (size_t)s_q * n_h;
  size_t off = align256(sizeof(WsHeader));
  L.work = off; off = align256(off + (size_t)units * 16);
  L.seq = off; off = align256(off + (size_t)B * 8);
  L.lse_part = off; off = align256(off + (size_t)units * R * 4);
  L.o_part = off; off = align256(off + (size_t)units * R * d_c * part_elem);
  L.total = off;
  return L;
}

inline WsLayout ws_layout(int B, int s_q, int n_h, int d_c, int num_splits, int n_cu) {
  const long long units = num_splits > 0 ? (long long)B * num_splits : (long long)kMaxAutoWaves * n_cu + B;
  return ws_layout_units(B, s_q, n_h, d_c, units, 4);
}

// ---------------------------------------------------------------- parameters
struct DecodeArgs {
  const void* q_lat;
  const void* q_rope;
  const void* kv;
  const int32_t* table;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  int* ws_header;  // -> WsHeader
  const int4* work;
  const int2* seq;
  float* lse_part;
  float* o_part;       // fp32 rows, or bf16 rows when part_bf16
  int part_bf16;
  long long block_bytes;
  int max_blocks;
  int units_max;  // plan entries the workspace has room for
  int B, s_q, n_h, d_c, d_r, block_size;
  float scale;
  int q_dtype, kv_dtype, out_dtype;
};

struct PlanArgs {
  const int32_t* seq_lens;
  int* ws_header;
  int4* work;
  int2* seq;
  int B, block_size, num_splits;
  int slots_per_wave;  // concurrent units per wave of the decode kernel
  int min_chunk;       // smallest partition (blocks) automatic planning uses
  int max_chunk;       // largest partition (blocks) any unit may have
  int units_max;
  int max_waves;       // automatic planning: at most this many waves of units
                       // (1 .. kMaxAutoWaves) unless even the largest partition needs more
};

// fused merge + W^UV up-projection of a decode step (bf16 partial rows,
// d_c = 512, d_h = 128)
struct CombineUpArgs {
  const int2* seq;
  const float* lse_part;
  const uint16_t* o_part;  // bf16 rows [unit][s_q * n_h][512]: partial rows of split
                           // sequences, final rows of unsplit ones
  const uint16_t* w_uv;    // [n_h * 128, 512]
  uint16_t* out;           // [B * s_q][n_h][128]
  float* lse;              // [B * s_q][n_h] or null
  int units_max;           // plan entries the workspace has room for
  int B, s_q, n_h;
};

// launchers (return hipError_t of the launch)
hipError_t launch_combine_up(const CombineUpArgs& c, int n_cu, hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs& a, int units_max, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int grid_x, hipStream_t s);
// expect_splits: the host's estimate of partitions per sequence (only picks
// between the two merge kernels; both handle any count)
hipError_t launch_combine_units(const DecodeArgs& a, hipStream_t s, int expect_splits);
hipError_t launch_combine_lse(const float* o_part, const float* lse_part, const int32_t* splits,
                              int N, int S, int D, void* out, float* lse_out, int out_dtype,
                              hipStream_t s);
hipError_t launch_absorb(const void* q, long long q_st, const void* w, void* out, long long o_st,
                         int T, int n_h, int d_h, int d_c, int act_dt, int w_dt, int out_dt,
                         bool mfma, hipStream_t s);
// bf16 absorption with the split planner in the same launch
hipError_t launch_absorb_plan(const void* q, long long q_st, const void* w, void* out, long long o_st, int T,
                              int n_h, int d_h, int d_c, const PlanArgs& pa, hipStream_t s);
hipError_t launch_prefill(const void* q, const void* kc, const void* kr, const void* v, void* out, float* lse,
                          int T, int n_h, int d_h, int d_r, float scale, int in_dtype, int out_dtype,
                          hipStream_t s);
bool expand_gemm_eligible(long long a_st, int N, int K, int out_dtype, const void* a, const void* w0,
                          const void* w1, const void* o0, const void* o1);
hipError_t launch_expand_gemm(const void* a, long long a_st, const void* w0, const void* w1, void* o0, void* o1,
                              int T, int N, int K, int out_dtype, int n_cu, hipStream_t s);
bool gqa_mfma_eligible(int s_q, int n_h, int n_g, int d_h, int d_r, int bs, int q_dt, int kv_dt);
hipError_t launch_gqa_decode(const void* q_c, const void* q_r, const void* cache, const int32_t* table,
                             int max_blocks, const int32_t* seq_lens, int B, int s_q, int n_h, int n_g, int d_h,
                             int d_r, int bs, long long block_bytes, float scale, int q_dt, int kv_dt, void* out,
                             float* lse, int out_dt, bool mfma, hipStream_t s);
constexpr int kMaxRopePairs = 64;  // d_r <= 128 for the cache producer
size_t append_workspace_bytes(int T, int d, int d_c, int d_r);
hipError_t launch_append(const void* h, long long h_st, const void* w, const int32_t* positions,
                         const int32_t* slots, void* cache, int T, int d, int d_c, int d_r, int block_size,
                         long long block_bytes, float rope_base, int in_dtype, int kv_dtype, float* part,
                         hipStream_t s);
hipError_t launch_up_proj(const void* o_lat, long long a_st, long long a_hs, const void* w, void* out,
                          long long o_st, int T, int n_h, int d_c, int d_h, int act_dt,
                          int w_dt, int out_dt, bool mfma, hipStream_t s);

}  // namespace mla
