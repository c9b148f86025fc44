// C ABI of libmla.so: argument validation, kernel selection and launch.
// Declarations and contracts: include/mla_decode.h.
#include "mla_decode.h"
#include "mla_internal.h"
#include <algorithm>

#include <atomic>
#include <mutex>

namespace mla {
int mfma_max_unit_pages();
}

using namespace mla;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// compute units of the current device (cached; 0 on failure)
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool act_dtype_ok(int d) { return d == MLA_F32 || d == MLA_BF16; }

int launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

struct DecodeShape {
  int B, s_q, n_h, d_c, d_r, block_size, max_blocks, num_splits;
};

bool mfma_eligible(const DecodeShape& s, int q_dtype, int kv_dtype) {
  return q_dtype == MLA_BF16 && kv_dtype >= MLA_BF16 && kv_dtype <= MLA_INT2 && s.n_h == 128 &&
         s.d_c == 512 && s.d_r == 64 && s.block_size == 64;
}

// upper bound on planned units for this shape
WsLayout layout_for(const DecodeShape& s, int n_cu) {
  WsLayout L = ws_layout(s.B, s.s_q, s.n_h, s.d_c, s.num_splits, n_cu);
  // partitions are capped at mfma_max_unit_pages() pages
  const long long cap = mfma_max_unit_pages();
  const long long per_seq_min = (s.max_blocks + cap - 1) / cap;
  const long long need = (long long)s.B * per_seq_min;
  if (need > L.units_max) {
    WsLayout M = ws_layout(s.B, s.s_q, s.n_h, s.d_c, (int)per_seq_min, n_cu);
    if (M.total > L.total) L = M;
  }
  return L;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or dtype code)";
    case MLA_ERR_UNSUPPORTED: return "unsupported combination of shapes/dtypes";
    case MLA_ERR_MISALIGNED: return "pointer or stride is not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_TOO_LARGE: return "problem needs more than the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

int mla_absorb_q(const void* q_nope, int64_t q_stride_t, const void* w_uk, void* q_lat,
                 int64_t qlat_stride_t, int T_q, int n_h, int d_h, int d_c, int act_dtype, int w_dtype,
                 int out_dtype, void* stream) {
  if (T_q < 0 || n_h <= 0 || d_h <= 0 || d_c <= 0) return MLA_ERR_INVALID_ARG;
  if (!act_dtype_ok(act_dtype) || !act_dtype_ok(w_dtype) || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (T_q == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_INVALID_ARG;
  if (q_stride_t < (int64_t)n_h * d_h || qlat_stride_t < (int64_t)n_h * d_c) return MLA_ERR_INVALID_ARG;
  const bool mfma = act_dtype == MLA_BF16 && w_dtype == MLA_BF16 && d_h <= 128;
  if (mfma) {
    if (d_h % 16 != 0 || d_c % 32 != 0) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(q_nope) || !aligned16(w_uk) || q_stride_t % 8 != 0) return MLA_ERR_MISALIGNED;
    // output rows are written in 16-byte pieces
    const int64_t oe = out_dtype == MLA_F32 ? 4 : 2;
    if (!aligned16(q_lat) || (qlat_stride_t * oe) % 16 != 0) return MLA_ERR_MISALIGNED;
  }
  return launch_status(launch_absorb(q_nope, q_stride_t, w_uk, q_lat, qlat_stride_t, T_q, n_h, d_h, d_c,
                                     act_dtype, w_dtype, out_dtype, mfma, (hipStream_t)stream));
}

int mla_up_proj_v(const void* o_lat, int64_t olat_stride_t, const void* w_uv, void* o, int64_t o_stride_t,
                  int T_q, int n_h, int d_c, int d_h, int act_dtype, int w_dtype, int out_dtype,
                  void* stream) {
  if (T_q < 0 || n_h <= 0 || d_h <= 0 || d_c <= 0) return MLA_ERR_INVALID_ARG;
  if (!act_dtype_ok(act_dtype) || !act_dtype_ok(w_dtype) || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (T_q == 0) return MLA_OK;
  if (!o_lat || !w_uv || !o) return MLA_ERR_INVALID_ARG;
  if (olat_stride_t < (int64_t)n_h * d_c || o_stride_t < (int64_t)n_h * d_h) return MLA_ERR_INVALID_ARG;
  const bool mfma = act_dtype == MLA_BF16 && w_dtype == MLA_BF16;
  if (mfma) {
    if (d_c % 64 != 0 || d_c > 512 || d_h % 32 != 0) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(o_lat) || !aligned16(w_uv) || olat_stride_t % 8 != 0) return MLA_ERR_MISALIGNED;
    // outputs are written two adjacent elements at a time
    if (((uintptr_t)o % (out_dtype == MLA_F32 ? 8 : 4)) != 0 || o_stride_t % 2 != 0) return MLA_ERR_MISALIGNED;
  }
  return launch_status(launch_up_proj(o_lat, olat_stride_t, d_c, w_uv, o, o_stride_t, T_q, n_h, d_c, d_h,
                                      act_dtype, w_dtype, out_dtype, mfma, (hipStream_t)stream));
}

int mla_expand_kv(const void* c_kv, int64_t c_stride_t, const void* w_uk, const void* w_uv, void* k_c, void* v_c,
                  int T, int n_h, int d_c, int d_h, int act_dtype, int w_dtype, int out_dtype, void* stream) {
  if (T < 0 || n_h <= 0 || d_h <= 0 || d_c <= 0) return MLA_ERR_INVALID_ARG;
  if (!act_dtype_ok(act_dtype) || !act_dtype_ok(w_dtype) || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!c_kv || !w_uk || !w_uv || !k_c || !v_c || c_stride_t < d_c) return MLA_ERR_INVALID_ARG;
  const bool mfma = act_dtype == MLA_BF16 && w_dtype == MLA_BF16;
  if (mfma) {
    if (d_c % 64 != 0 || d_c > 512 || d_h % 32 != 0) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(c_kv) || !aligned16(w_uk) || !aligned16(w_uv) || c_stride_t % 8 != 0) return MLA_ERR_MISALIGNED;
    const uintptr_t oa = out_dtype == MLA_F32 ? 8 : 4;
    if ((uintptr_t)k_c % oa != 0 || (uintptr_t)v_c % oa != 0 || ((int64_t)n_h * d_h) % 2 != 0) return MLA_ERR_MISALIGNED;
  }
  hipStream_t st = (hipStream_t)stream;
  const long long o_st = (long long)n_h * d_h;
  if (mfma && expand_gemm_eligible(c_stride_t, n_h * d_h, d_c, out_dtype, c_kv, w_uk, w_uv, k_c, v_c))
    return launch_status(launch_expand_gemm(c_kv, c_stride_t, w_uk, w_uv, k_c, v_c, T, n_h * d_h, d_c, out_dtype,
                                                 current_cu_count(), st));
  // otherwise the up-projection kernel, one latent row per token feeding
  // every head (activation head stride 0)
  hipError_t e = launch_up_proj(c_kv, c_stride_t, 0, w_uk, k_c, o_st, T, n_h, d_c, d_h, act_dtype, w_dtype, out_dtype,
                                mfma, st);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  return launch_status(launch_up_proj(c_kv, c_stride_t, 0, w_uv, v_c, o_st, T, n_h, d_c, d_h, act_dtype, w_dtype,
                                      out_dtype, mfma, st));
}

int mla_prefill_mha(const void* q, const void* k_c, const void* k_r, const void* v_c, void* o, float* lse, int T,
                    int n_h, int d_h, int d_r, float softmax_scale, int in_dtype, int out_dtype, void* stream) {
  if (T < 0 || n_h <= 0 || d_h <= 0 || d_r < 0 || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  if (!act_dtype_ok(in_dtype) || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!q || !k_c || !v_c || !o || (d_r > 0 && !k_r)) return MLA_ERR_INVALID_ARG;
  if (d_h + d_r > 256 || d_h > 256) return MLA_ERR_UNSUPPORTED;
  if (in_dtype == MLA_BF16 && d_h == 128 && d_r == 64 && !aligned16(o)) return MLA_ERR_MISALIGNED;
  return launch_status(launch_prefill(q, k_c, k_r, v_c, o, lse, T, n_h, d_h, d_r, softmax_scale, in_dtype,
                                      out_dtype, (hipStream_t)stream));
}

int mla_gqa_decode(const void* q_c, const void* q_r, const void* kv_cache, const int32_t* block_table,
                   int max_blocks_per_seq, const int32_t* seq_lens, int B, int s_q, int n_h, int n_g, int d_h,
                   int d_r, int block_size, float softmax_scale, int q_dtype, int kv_dtype, int out_dtype, void* o,
                   float* lse, int flags, void* stream) {
  if (B <= 0 || s_q <= 0 || n_h <= 0 || n_g <= 0 || d_h <= 0 || d_r < 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || n_h % n_g != 0)
    return MLA_ERR_INVALID_ARG;
  if (flags & ~MLA_FLAG_FORCE_GENERIC) return MLA_ERR_INVALID_ARG;
  if (!act_dtype_ok(q_dtype) || !act_dtype_ok(kv_dtype) || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (!q_c || !kv_cache || !block_table || !seq_lens || !o || (d_r > 0 && !q_r)) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return MLA_ERR_INVALID_ARG;
  if (d_h > 256 || d_h + d_r > 256) return MLA_ERR_UNSUPPORTED;
  const long long elem = kv_dtype == MLA_F32 ? 4 : 2;
  const long long block_bytes = (long long)block_size * (2LL * n_g * d_h + d_r) * elem;
  bool fast = !(flags & MLA_FLAG_FORCE_GENERIC) &&
              gqa_mfma_eligible(s_q, n_h, n_g, d_h, d_r, block_size, q_dtype, kv_dtype) && aligned16(q_c) &&
              aligned16(q_r) && aligned16(kv_cache) && aligned16(o);
  return launch_status(launch_gqa_decode(q_c, q_r, kv_cache, block_table, max_blocks_per_seq, seq_lens, B, s_q, n_h,
                                         n_g, d_h, d_r, block_size, block_bytes, softmax_scale, q_dtype, kv_dtype,
                                         o, lse, out_dtype, fast, (hipStream_t)stream));
}

size_t mla_cache_append_workspace_bytes(int T, int d, int d_c, int d_r) {
  if (T <= 0 || d <= 0 || d_c <= 0 || d_r < 0) return 0;
  return append_workspace_bytes(T, d, d_c, d_r);
}

int mla_cache_append(const void* h, int64_t h_stride_t, const void* w_dkv_kr, const int32_t* positions,
                     const int32_t* slot_mapping, void* kv_cache, int T, int d, int d_c, int d_r, int block_size,
                     float rope_base, int in_dtype, int kv_dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (T < 0 || d <= 0 || d_c <= 0 || d_r < 0 || d_r % 2 != 0 || block_size <= 0 || !(rope_base > 0.f))
    return MLA_ERR_INVALID_ARG;
  if (d_r > 2 * kMaxRopePairs) return MLA_ERR_UNSUPPORTED;
  if (!act_dtype_ok(in_dtype) || !(kv_dtype == MLA_F32 || kv_dtype == MLA_BF16 || kv_dtype == MLA_FP8_E4M3))
    return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!h || !w_dkv_kr || !positions || !slot_mapping || !kv_cache) return MLA_ERR_INVALID_ARG;
  if (h_stride_t < d) return MLA_ERR_INVALID_ARG;
  if (kv_dtype == MLA_FP8_E4M3 && (in_dtype != MLA_BF16 || d_c % 16 != 0 || d_r % 8 != 0))
    return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < append_workspace_bytes(T, d, d_c, d_r)) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_MISALIGNED;
  const long long elem = kv_dtype == MLA_F32 ? 4 : 2;
  const long long block_bytes = kv_dtype == MLA_FP8_E4M3 ? (long long)block_size * (d_c + 2 * d_r + 4)
                                                         : (long long)block_size * (d_c + d_r) * elem;
  return launch_status(launch_append(h, h_stride_t, w_dkv_kr, positions, slot_mapping, kv_cache, T, d, d_c, d_r,
                                     block_size, block_bytes, rope_base, in_dtype, kv_dtype, (float*)workspace,
                                     (hipStream_t)stream));
}

size_t mla_decode_workspace_bytes(int B, int s_q, int n_h, int d_c, int max_blocks_per_seq, int num_splits) {
  if (B <= 0 || s_q <= 0 || n_h <= 0 || d_c <= 0 || max_blocks_per_seq <= 0 || num_splits < 0) return 0;
  const int n_cu = current_cu_count();
  if (n_cu <= 0) return 0;
  DecodeShape s{B, s_q, n_h, d_c, 0, 0, max_blocks_per_seq, num_splits};
  return layout_for(s, n_cu).total;
}

// bytes per cached token in each format (the block layouts in the header)
static long long kv_row_bytes(int kv_dtype, int d_c, int d_r) {
  switch (kv_dtype) {
    case MLA_F32: return (long long)(d_c + d_r) * 4;
    case MLA_BF16: return (long long)(d_c + d_r) * 2;
    case MLA_FP8_E4M3: return (long long)d_c + 2 * d_r + 4;
    default: {
      const int cb = kv_dtype == MLA_INT4 ? 4 : 2;
      return (long long)d_c * cb / 8 + d_r / 2 + (d_c + d_r) / 32 * 4;
    }
  }
}

int mla_decode_absorbed(const void* q_lat, const void* q_rope, const void* kv_cache, const int32_t* block_table,
                        int max_blocks_per_seq, const int32_t* seq_lens, int B, int s_q, int n_h, int d_c,
                        int d_r, int block_size, float softmax_scale, int q_dtype, int kv_dtype, int out_dtype,
                        int num_splits, void* workspace, size_t workspace_bytes, void* o_lat, float* lse,
                        int flags, void* stream) {
  if (B <= 0 || s_q <= 0 || n_h <= 0 || d_c <= 0 || d_r < 0 || block_size <= 0 || max_blocks_per_seq <= 0)
    return MLA_ERR_INVALID_ARG;
  if (num_splits < 0 || (flags & ~MLA_FLAG_FORCE_GENERIC)) return MLA_ERR_INVALID_ARG;
  if (!act_dtype_ok(q_dtype) || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (kv_dtype < MLA_F32 || kv_dtype > MLA_INT2) return MLA_ERR_INVALID_ARG;
  if (!q_lat || !kv_cache || !block_table || !seq_lens || !o_lat) return MLA_ERR_INVALID_ARG;
  if (d_r > 0 && !q_rope) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return MLA_ERR_INVALID_ARG;
  if (s_q > 16 || d_c > 2048 || d_r > 256 || d_c % 4 != 0) return MLA_ERR_UNSUPPORTED;
  if (kv_dtype == MLA_FP8_E4M3 && (d_r % 8 != 0 || d_c % 16 != 0)) return MLA_ERR_UNSUPPORTED;
  if ((kv_dtype == MLA_INT4 || kv_dtype == MLA_INT2) && (d_c % 32 != 0 || d_r % 32 != 0)) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(o_lat)) return MLA_ERR_MISALIGNED;
  if (!workspace) return MLA_ERR_WORKSPACE;

  const int n_cu = current_cu_count();
  if (n_cu <= 0) return MLA_ERR_LAUNCH;
  DecodeShape shp{B, s_q, n_h, d_c, d_r, block_size, max_blocks_per_seq, num_splits};
  const WsLayout L = layout_for(shp, n_cu);
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_MISALIGNED;

  bool fast = !(flags & MLA_FLAG_FORCE_GENERIC) && mfma_eligible(shp, q_dtype, kv_dtype);
  if (fast && (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(kv_cache))) fast = false;

  uint8_t* ws = (uint8_t*)workspace;
  DecodeArgs a{};
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.kv = kv_cache;
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.out = o_lat;
  a.lse = lse;
  a.ws_header = (int*)ws;
  a.work = (const int4*)(ws + L.work);
  a.seq = (const int2*)(ws + L.seq);
  a.lse_part = (float*)(ws + L.lse_part);
  a.o_part = (float*)(ws + L.o_part);
  a.block_bytes = (long long)block_size * kv_row_bytes(kv_dtype, d_c, d_r);
  a.max_blocks = max_blocks_per_seq;
  a.units_max = L.units_max;
  a.B = B; a.s_q = s_q; a.n_h = n_h; a.d_c = d_c; a.d_r = d_r; a.block_size = block_size;
  a.scale = softmax_scale;
  a.q_dtype = q_dtype; a.kv_dtype = kv_dtype; a.out_dtype = out_dtype;
  // the MFMA kernels write bf16 partial rows when the merged output is bf16
  // anyway (half the partial-result traffic)
  a.part_bf16 = (fast && out_dtype == MLA_BF16) ? 1 : 0;

  hipStream_t st = (hipStream_t)stream;
  const int grid_x = fast ? (n_cu / s_q > 0 ? n_cu / s_q : 1) : (L.units_max < n_cu ? L.units_max : n_cu);

  PlanArgs p{};
  p.seq_lens = seq_lens;
  p.ws_header = (int*)ws;
  p.work = (int4*)(ws + L.work);
  p.seq = (int2*)(ws + L.seq);
  p.B = B;
  p.block_size = block_size;
  p.num_splits = num_splits;
  p.slots_per_wave = grid_x;
  p.min_chunk = fast ? 8 : 4;
  p.max_chunk = mfma_max_unit_pages();
  p.units_max = L.units_max;
  p.max_waves = kMaxAutoWaves;
  hipError_t e = launch_plan(p, st);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  e = fast ? launch_decode_mfma(a, grid_x, st) : launch_decode_generic(a, grid_x, st);
  if (e != hipSuccess) return MLA_ERR_LAUNCH;
  // partitions per sequence are planned on the device; the host expects about
  // slots / B of them (equal lengths) or the explicit count
  const int expect_splits = num_splits > 0 ? num_splits : (grid_x + B - 1) / B;
  e = launch_combine_units(a, st, expect_splits);
  return launch_status(e);
}

// workgroups of the step's attention launch (one per compute unit and query token)
static int step_grid(int n_cu, int s_q) { return n_cu / s_q > 0 ? n_cu / s_q : 1; }

static size_t step_extra_bytes(int B, int s_q, int n_h, int d_c) {
  return align256((size_t)B * s_q * n_h * d_c * 2);  // the absorbed queries (bf16)
}

size_t mla_decode_step_workspace_bytes(int B, int s_q, int n_h, int d_c, int max_blocks_per_seq, int num_splits) {
  const size_t base = mla_decode_workspace_bytes(B, s_q, n_h, d_c, max_blocks_per_seq, num_splits);
  return base ? align256(base) + step_extra_bytes(B, s_q, n_h, d_c) : 0;
}

}  // extern "C"

namespace {

// Argument checks shared by the step entry points (everything but the
// workspace / scratch).
int step_check(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
               const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens, const void* w_uv, int B,
               int s_q, int n_h, int d_h, int d_c, int d_r, int block_size, float softmax_scale, int kv_dtype,
               int num_splits, const void* o) {
  if (B <= 0 || s_q <= 0 || n_h <= 0 || d_h <= 0 || d_c <= 0 || d_r < 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_splits < 0)
    return MLA_ERR_INVALID_ARG;
  if (!q_nope || !w_uk || !q_rope || !kv_cache || !block_table || !seq_lens || !w_uv || !o)
    return MLA_ERR_INVALID_ARG;
  if (kv_dtype < MLA_F32 || kv_dtype > MLA_INT2) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return MLA_ERR_INVALID_ARG;
  DecodeShape shp{B, s_q, n_h, d_c, d_r, block_size, max_blocks_per_seq, num_splits};
  if (!mfma_eligible(shp, MLA_BF16, kv_dtype) || d_h != 128 || s_q > 16) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_rope) || !aligned16(kv_cache) || !aligned16(w_uv) ||
      !aligned16(o))
    return MLA_ERR_MISALIGNED;
  return MLA_OK;
}

// The step's launches on a checked set of arguments, with its plan, partial
// rows and absorbed queries in `ws` laid out as L (partials in bf16) followed
// by q_lat at dec_bytes.
//   1. absorption into ws (bf16 q_lat), the split planner riding in the same
//      launch (automatic plans of at most max_waves waves of units);
//   2. the attention kernel (every unit writes its rows to its partial slot,
//      final rows for unsplit sequences);
//   3. merge + up-projection.
// Everything one stage leaves for the next lives in ws.
int step_launch(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens, const void* w_uv, int B,
                int s_q, int n_h, int d_h, int d_c, int d_r, int block_size, float softmax_scale, int kv_dtype,
                int num_splits, void* o, float* lse, uint8_t* ws, const WsLayout& L, size_t dec_bytes, int n_cu,
                int max_waves, int stages, hipStream_t st) {
  const int T_q = B * s_q;
  uint16_t* q_lat = (uint16_t*)(ws + dec_bytes);
  DecodeArgs a{};
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.kv = kv_cache;
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.out = nullptr;  // rows of unsplit sequences stay in their partial slots
  a.lse = lse;
  a.ws_header = (int*)ws;
  a.work = (const int4*)(ws + L.work);
  a.seq = (const int2*)(ws + L.seq);
  a.lse_part = (float*)(ws + L.lse_part);
  a.o_part = (float*)(ws + L.o_part);
  a.part_bf16 = 1;
  a.block_bytes = (long long)block_size * kv_row_bytes(kv_dtype, d_c, d_r);
  a.max_blocks = max_blocks_per_seq;
  a.units_max = L.units_max;
  a.B = B; a.s_q = s_q; a.n_h = n_h; a.d_c = d_c; a.d_r = d_r; a.block_size = block_size;
  a.scale = softmax_scale;
  a.q_dtype = MLA_BF16; a.kv_dtype = kv_dtype; a.out_dtype = MLA_BF16;
  const int grid_x = step_grid(n_cu, s_q);
  if (stages & MLA_STAGE_ABSORB) {
    PlanArgs p{};
    p.seq_lens = seq_lens;
    p.ws_header = (int*)ws;
    p.work = (int4*)(ws + L.work);
    p.seq = (int2*)(ws + L.seq);
    p.B = B;
    p.block_size = block_size;
    p.num_splits = num_splits;
    p.slots_per_wave = grid_x;
    p.min_chunk = 8;
    p.max_chunk = mfma_max_unit_pages();
    p.units_max = L.units_max;
    p.max_waves = max_waves;
    if (launch_absorb_plan(q_nope, (long long)n_h * d_h, w_uk, q_lat, (long long)n_h * d_c, T_q, n_h, d_h, d_c, p,
                           st) != hipSuccess)
      return MLA_ERR_LAUNCH;
  }
  if ((stages & MLA_STAGE_ATTEND) && launch_decode_mfma(a, grid_x, st) != hipSuccess) return MLA_ERR_LAUNCH;
  if (stages & MLA_STAGE_MERGE) {
    // merge of the partitions fused with the up-projection
    CombineUpArgs c{};
    c.seq = a.seq;
    c.lse_part = a.lse_part;
    c.o_part = (const uint16_t*)a.o_part;
    c.w_uv = (const uint16_t*)w_uv;
    c.out = (uint16_t*)o;
    c.lse = lse;
    c.units_max = L.units_max;
    c.B = B; c.s_q = s_q; c.n_h = n_h;
    if (launch_combine_up(c, n_cu, st) != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

// ------------------------------------------------ scratch of the no-allocation step
// Device memory of mla_decode_step_noalloc: plan, bf16 partial rows and the
// absorbed queries of one step.  A file-scope device array, so the library
// holds one on every GPU it runs on until the process ends and no call
// allocates.  In host code `scratch` only names the symbol; its device
// address (one per GPU) comes from hipGetSymbolAddress with that GPU current.
constexpr size_t kNoAllocScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// the current device's address of `scratch` (looked up once per device)
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_LAUNCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_LAUNCH;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_step_stages(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                           const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                           const void* w_uv, int B, int s_q, int n_h, int d_h, int d_c, int d_r, int block_size,
                           float softmax_scale, int kv_dtype, int num_splits, void* workspace,
                           size_t workspace_bytes, void* o, float* lse, int stages, void* stream) {
  if (stages <= 0 || (stages & ~MLA_STAGE_ALL)) return MLA_ERR_INVALID_ARG;
  if (const int e = step_check(q_nope, w_uk, q_rope, kv_cache, block_table, max_blocks_per_seq, seq_lens, w_uv, B,
                               s_q, n_h, d_h, d_c, d_r, block_size, softmax_scale, kv_dtype, num_splits, o);
      e != MLA_OK)
    return e;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_MISALIGNED;
  const int n_cu = current_cu_count();
  if (n_cu <= 0) return MLA_ERR_LAUNCH;
  DecodeShape shp{B, s_q, n_h, d_c, d_r, block_size, max_blocks_per_seq, num_splits};
  const WsLayout L = layout_for(shp, n_cu);
  const size_t dec_bytes = align256(L.total);
  if (workspace_bytes < dec_bytes + step_extra_bytes(B, s_q, n_h, d_c)) return MLA_ERR_WORKSPACE;
  return step_launch(q_nope, w_uk, q_rope, kv_cache, block_table, max_blocks_per_seq, seq_lens, w_uv, B, s_q, n_h,
                     d_h, d_c, d_r, block_size, softmax_scale, kv_dtype, num_splits, o, lse, (uint8_t*)workspace, L,
                     dec_bytes, n_cu, kMaxAutoWaves, stages, (hipStream_t)stream);
}

int mla_decode_step(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                    const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens, const void* w_uv,
                    int B, int s_q, int n_h, int d_h, int d_c, int d_r, int block_size, float softmax_scale,
                    int kv_dtype, int num_splits, void* workspace, size_t workspace_bytes, void* o, float* lse,
                    void* stream) {
  return mla_decode_step_stages(q_nope, w_uk, q_rope, kv_cache, block_table, max_blocks_per_seq, seq_lens, w_uv, B,
                                s_q, n_h, d_h, d_c, d_r, block_size, softmax_scale, kv_dtype, num_splits, workspace,
                                workspace_bytes, o, lse, MLA_STAGE_ALL, stream);
}

int mla_decode_step_noalloc(const void* q_nope, const void* w_uk, const void* q_rope, const void* kv_cache,
                            const int32_t* block_table, int max_blocks_per_seq, const int32_t* seq_lens,
                            const void* w_uv, int B, int s_q, int n_h, int d_h, int d_c, int d_r, int block_size,
                            float softmax_scale, int kv_dtype, int num_splits, void* o, float* lse, void* stream) {
  if (const int e = step_check(q_nope, w_uk, q_rope, kv_cache, block_table, max_blocks_per_seq, seq_lens, w_uv, B,
                               s_q, n_h, d_h, d_c, d_r, block_size, softmax_scale, kv_dtype, num_splits, o);
      e != MLA_OK)
    return e;
  const int n_cu = current_cu_count();
  if (n_cu <= 0) return MLA_ERR_LAUNCH;
  // room for every plan the capped planner can make: one wave of units, or
  // one per page-capped partition of each sequence, or the explicit count
  const long long cap = mfma_max_unit_pages();
  const long long per_seq_min = (max_blocks_per_seq + cap - 1) / cap;
  const long long per_seq = num_splits > 0 ? (num_splits > per_seq_min ? num_splits : per_seq_min) : per_seq_min;
  long long units = (long long)B * per_seq;
  if (num_splits <= 0 && units < step_grid(n_cu, s_q)) units = step_grid(n_cu, s_q);
  if (units > (1ll << 30)) return MLA_ERR_TOO_LARGE;
  const WsLayout L = ws_layout_units(B, s_q, n_h, d_c, units, 2);
  const size_t dec_bytes = align256(L.total);
  if (dec_bytes + step_extra_bytes(B, s_q, n_h, d_c) > kNoAllocScratchBytes) return MLA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (const int e = scratch_address(&ws); e != MLA_OK) return e;
  return step_launch(q_nope, w_uk, q_rope, kv_cache, block_table, max_blocks_per_seq, seq_lens, w_uv, B, s_q, n_h,
                     d_h, d_c, d_r, block_size, softmax_scale, kv_dtype, num_splits, o, lse, (uint8_t*)ws, L,
                     dec_bytes, n_cu, 1, MLA_STAGE_ALL, (hipStream_t)stream);
}

int mla_combine_lse(const float* o_part, const float* lse_part, const int32_t* splits_per_row, int N, int S,
                    int D, void* out, float* lse_out, int out_dtype, void* stream) {
  if (N < 0 || S <= 0 || D <= 0 || !act_dtype_ok(out_dtype)) return MLA_ERR_INVALID_ARG;
  if (D % 4 != 0) return MLA_ERR_UNSUPPORTED;
  if (N == 0) return MLA_OK;
  if (!o_part || !lse_part || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_part) || !aligned16(out)) return MLA_ERR_MISALIGNED;
  return launch_status(launch_combine_lse(o_part, lse_part, splits_per_row, N, S, D, out, lse_out, out_dtype,
                                          (hipStream_t)stream));
}

}  // extern "C"
