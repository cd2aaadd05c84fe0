// librbs C ABI: host-side argument checks and dispatch to the HIP launchers.
// Every check runs before anything is enqueued; see include/rbs.h for the
// contract of each call.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "rbs_common.h"

using namespace rbs;

namespace {

bool aligned(const void* p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-branch budget: fraction of the visible blocks, rounded up, at least one.
// Multiply and subtract are kept as two correctly rounded steps.
int host_budget(int n_visible, double rho) {
  volatile double prod = rho * (double)n_visible;
  volatile double x = prod - 1e-6;
  double c = ceil(x);
  int n = c < 1.0 ? 1 : (int)c;
  return n < n_visible ? n : n_visible;
}

bool ratio_ok(double r) { return r > 0.0 && r <= 1.0; }  // false for NaN

// Largest row and total entry count of a selection.
void select_sizes(int nb, double rc, double rr, bool sink, int64_t* total, int* widest) {
  int64_t t = 0;
  int w = 0;
  for (int i = 0; i < nb; ++i) {
    int n = host_budget(i + 1, rc) + host_budget(i + 1, rr) + 1 + (sink ? 1 : 0);
    if (n > i + 1) n = i + 1;
    t += n;
    if (n > w) w = n;
  }
  *total = t;
  *widest = w;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

namespace {
// Key tiles per chunk when the final block's rows are split (see
// block_mask_attn_fwd).
constexpr int kChunkTiles = 64;
}  // namespace

namespace {
rbs_status block_stats_common(rbs_dtype dt, const void* q, const void* k, int32_t seqlen,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              int32_t block, float* k_centroid, float* k_radius, float* q_rep,
                              float* q_rep_norm, float* q_rep_head, float* q_rep_head_norm,
                              void* stream) {
  if (dt != RBS_DT_BF16 && dt != RBS_DT_F32) return RBS_E_ARG;
  if (seqlen < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || block <= 0)
    return RBS_E_ARG;
  if (n_q_heads % n_kv_heads != 0) return RBS_E_ARG;
  if (seqlen > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(k_centroid, 16) ||
                     !aligned(k_radius, 4)))
    return RBS_E_ARG;
  if (seqlen > 0 && q_rep && (!aligned(q_rep, 16) || !aligned(q_rep_norm, 4))) return RBS_E_ARG;
  if (seqlen > 0 && q_rep_head && (!aligned(q_rep_head, 16) || !aligned(q_rep_head_norm, 4)))
    return RBS_E_ARG;
  if (head_dim != 64 && head_dim != 128) return RBS_E_UNSUPPORTED;
  if (block < 16 || block > 256 || block % 16 != 0) return RBS_E_UNSUPPORTED;
  // LDS of the stats kernel grows with the group's row width
  const int esize = dt == RBS_DT_BF16 ? 2 : 4;
  const int epv = 16 / esize;
  const int G = n_q_heads / n_kv_heads;
  const int vr = G * (head_dim / epv);
  const size_t qslots = vr <= 256 ? (size_t)(256 / vr) * vr : (size_t)vr;
  if ((qslots * epv + 16 + 256 * epv + head_dim + (size_t)G * (head_dim / 64)) * 4 > 64 * 1024)
    return RBS_E_UNSUPPORTED;
  if ((int64_t)seqlen * n_q_heads * head_dim > ((int64_t)1 << 40)) return RBS_E_UNSUPPORTED;
  if (seqlen == 0) return RBS_OK;
  return launch_block_stats(dt, q, k, seqlen, n_q_heads, n_kv_heads, head_dim, block, k_centroid,
                            k_radius, q_rep, q_rep_norm, q_rep_head, q_rep_head_norm,
                            as_stream(stream));
}
}  // namespace

namespace {
// One list per row head: n_row_heads = n_kv_heads (a list per GQA group) or
// n_q_heads (a list per query head); q_rep / q_rep_norm are per row head.
rbs_status select_common(const float* k_centroid, const float* k_radius, const float* q_rep,
                         const float* q_rep_norm, const float* beta_in, int32_t n_row_heads,
                         int32_t n_kv_heads, int32_t n_blocks, int32_t head_dim,
                         double keep_ratio_centroid, double keep_ratio_rescue, uint32_t flags,
                         float* beta_out, int32_t* row_ptr, int32_t* col_idx,
                         int64_t col_capacity, void* workspace, size_t* workspace_bytes,
                         void* stream) {
  if (!workspace_bytes) return RBS_E_ARG;
  if (n_kv_heads <= 0 || n_row_heads <= 0 || n_row_heads % n_kv_heads != 0) return RBS_E_ARG;
  if (n_blocks < 0 || head_dim <= 0) return RBS_E_ARG;
  if (!ratio_ok(keep_ratio_centroid) || !ratio_ok(keep_ratio_rescue)) return RBS_E_ARG;
  if ((flags & ~RBS_SEL_FORCE_SINK) != 0) return RBS_E_ARG;
  if (head_dim != 64 && head_dim != 128) return RBS_E_UNSUPPORTED;
  if (n_blocks > 0 && select_rows_per_group(n_blocks, head_dim) <= 0) return RBS_E_UNSUPPORTED;
  const bool sink = (flags & RBS_SEL_FORCE_SINK) != 0;
  int64_t per_head;
  int widest;
  select_sizes(n_blocks, keep_ratio_centroid, keep_ratio_rescue, sink, &per_head, &widest);
  const int64_t rows = (int64_t)n_row_heads * n_blocks;
  const size_t counts_bytes = align256((size_t)rows * 4);
  const size_t partial_bytes = align256((size_t)((rows + 63) / 64) * 4);
  const size_t lists_bytes = align256((size_t)rows * widest * 4);
  const size_t scores_bytes = align256(select_score_workspace(n_row_heads, n_blocks));
  const size_t need = 256 + counts_bytes + partial_bytes + lists_bytes + scores_bytes;
  if (!workspace) {
    *workspace_bytes = need;
    return RBS_OK;
  }
  if (!aligned(row_ptr, 4) || !aligned(workspace, 256)) return RBS_E_ARG;
  if (n_blocks > 0 && (!aligned(k_centroid, 16) || !aligned(q_rep, 16) || !aligned(k_radius, 4) ||
                       !aligned(q_rep_norm, 4) || !aligned(col_idx, 4)))
    return RBS_E_ARG;
  if ((beta_in && !aligned(beta_in, 4)) || (beta_out && !aligned(beta_out, 4))) return RBS_E_ARG;
  if (*workspace_bytes < need) return RBS_E_CAPACITY;
  if (col_capacity < per_head * n_row_heads) return RBS_E_CAPACITY;
  if (per_head * n_row_heads > INT32_MAX) return RBS_E_UNSUPPORTED;
  SelectArgs a;
  a.cen = k_centroid;
  a.rad = k_radius;
  a.qrep = q_rep;
  a.qnorm = q_rep_norm;
  a.beta_in = beta_in;
  a.beta_out = beta_out;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  char* const ws = static_cast<char*>(workspace);
  a.counts = reinterpret_cast<int32_t*>(ws + 256);
  a.partial = reinterpret_cast<int32_t*>(ws + 256 + counts_bytes);
  a.lists = reinterpret_cast<int32_t*>(ws + 256 + counts_bytes + partial_bytes);
  a.scores = reinterpret_cast<float*>(ws + 256 + counts_bytes + partial_bytes + lists_bytes);
  a.rbeta = a.scores + (size_t)n_row_heads * ((size_t)n_blocks * (n_blocks + 1) / 2);
  a.H = n_row_heads;
  a.G = n_row_heads / n_kv_heads;
  a.nb = n_blocks;
  a.D = head_dim;
  a.stride = widest;
  a.rho_c = keep_ratio_centroid;
  a.rho_r = keep_ratio_rescue;
  a.sink = sink ? 1 : 0;
  return launch_select(a, as_stream(stream));
}

}  // namespace

namespace {
// Checks shared by the CSR attention entries (every dtype); fills a.
rbs_status attn_args(const void* q, const void* k, const void* v, int32_t seqlen,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block,
                     const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale,
                     void* out, float* lse, bool per_head, AttnArgs& a) {
  if (seqlen < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || block <= 0)
    return RBS_E_ARG;
  if (n_q_heads % n_kv_heads != 0) return RBS_E_ARG;
  if (seqlen > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
                     !aligned(row_ptr, 4) || !aligned(col_idx, 4) || (lse && !aligned(lse, 4))))
    return RBS_E_ARG;
  if (isnan(softmax_scale) || isinf(softmax_scale)) return RBS_E_ARG;
  if (!((head_dim == 64 || head_dim == 128) && (block == 64 || block == 128)))
    return RBS_E_UNSUPPORTED;
  if ((int64_t)seqlen * n_q_heads * head_dim > ((int64_t)1 << 40)) return RBS_E_UNSUPPORTED;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.S = seqlen;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.D = head_dim;
  a.B = block;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.per_head = per_head ? 1 : 0;
  return RBS_OK;
}

rbs_status attn_common(rbs_dtype dt, const void* q, const void* k, const void* v, int32_t seqlen,
                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block,
                       const int32_t* row_ptr, const int32_t* col_idx, float softmax_scale,
                       void* out, float* lse, bool per_head, void* stream) {
  if (dt != RBS_DT_BF16 && dt != RBS_DT_F32) return RBS_E_ARG;
  AttnArgs a;
  const rbs_status st = attn_args(q, k, v, seqlen, n_q_heads, n_kv_heads, head_dim, block, row_ptr,
                                  col_idx, softmax_scale, out, lse, per_head, a);
  if (st != RBS_OK || seqlen == 0) return st;
  const bool bf = dt == RBS_DT_BF16;
  // bf16 at head dim 128 and block 128 runs on the matrix cores; every other
  // supported shape on the vector-ALU kernel
  if (bf && head_dim == 128 && block == 128) return launch_attn_bf16_csr(a, as_stream(stream));
  return launch_attn_vec_csr(a, bf, as_stream(stream));
}

}  // namespace

extern "C" {

const char* rbs_status_string(rbs_status s) {
  switch (s) {
    case RBS_OK: return "ok";
    case RBS_E_ARG: return "invalid argument";
    case RBS_E_UNSUPPORTED: return "unsupported configuration";
    case RBS_E_CAPACITY: return "output capacity or workspace too small";
    case RBS_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

rbs_status rbs_block_stats(rbs_dtype dt, const void* q, const void* k, int32_t seqlen,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block,
                           float* k_centroid, float* k_radius, float* q_rep, float* q_rep_norm,
                           void* stream) {
  if (seqlen > 0 && (!q_rep || !q_rep_norm)) return RBS_E_ARG;
  return block_stats_common(dt, q, k, seqlen, n_q_heads, n_kv_heads, head_dim, block, k_centroid,
                            k_radius, q_rep, q_rep_norm, nullptr, nullptr, stream);
}

rbs_status rbs_block_stats_per_head(rbs_dtype dt, const void* q, const void* k, int32_t seqlen,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block, float* k_centroid, float* k_radius,
                                    float* q_rep_head, float* q_rep_head_norm, void* stream) {
  if (seqlen > 0 && (!q_rep_head || !q_rep_head_norm)) return RBS_E_ARG;
  return block_stats_common(dt, q, k, seqlen, n_q_heads, n_kv_heads, head_dim, block, k_centroid,
                            k_radius, nullptr, nullptr, q_rep_head, q_rep_head_norm, stream);
}

int64_t rbs_select_capacity(int32_t n_kv_heads, int32_t n_blocks, double keep_ratio_centroid,
                            double keep_ratio_rescue, uint32_t flags) {
  if (n_kv_heads <= 0 || n_blocks < 0 || !ratio_ok(keep_ratio_centroid) ||
      !ratio_ok(keep_ratio_rescue))
    return -1;
  int64_t total;
  int widest;
  select_sizes(n_blocks, keep_ratio_centroid, keep_ratio_rescue, (flags & RBS_SEL_FORCE_SINK) != 0,
               &total, &widest);
  return total * n_kv_heads;
}

rbs_status rbs_select(const float* k_centroid, const float* k_radius, const float* q_rep,
                      const float* q_rep_norm, const float* beta_in, int32_t n_kv_heads,
                      int32_t n_blocks, int32_t head_dim, double keep_ratio_centroid,
                      double keep_ratio_rescue, uint32_t flags, float* beta_out,
                      int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                      void* workspace, size_t* workspace_bytes, void* stream) {
  return select_common(k_centroid, k_radius, q_rep, q_rep_norm, beta_in, n_kv_heads, n_kv_heads,
                       n_blocks, head_dim, keep_ratio_centroid, keep_ratio_rescue, flags, beta_out,
                       row_ptr, col_idx, col_capacity, workspace, workspace_bytes, stream);
}

rbs_status rbs_select_static(const float* k_centroid, const float* k_radius,
                             const float* q_rep, const float* q_rep_norm, const float* beta_in,
                             int32_t n_kv_heads, int32_t n_blocks, int32_t head_dim,
                             double keep_ratio_centroid, double keep_ratio_rescue,
                             uint32_t flags, float* beta_out, int32_t* row_ptr,
                             int32_t* col_idx, int64_t col_capacity, void* stream) {
  // size check first: a call that needs more scratch than the array holds
  // fails before anything device-side is touched
  size_t need = 0;
  rbs_status st = select_common(nullptr, nullptr, nullptr, nullptr, nullptr, n_kv_heads,
                                n_kv_heads, n_blocks, head_dim, keep_ratio_centroid,
                                keep_ratio_rescue, flags, nullptr, nullptr, nullptr, 0, nullptr,
                                &need, nullptr);
  if (st != RBS_OK) return st;
  if (need > RBS_SELECT_STATIC_SCRATCH_BYTES) return RBS_E_CAPACITY;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  st = static_scratch(as_stream(stream), &ws, &ws_bytes);
  if (st != RBS_OK) return st;
  return select_common(k_centroid, k_radius, q_rep, q_rep_norm, beta_in, n_kv_heads, n_kv_heads,
                       n_blocks, head_dim, keep_ratio_centroid, keep_ratio_rescue, flags,
                       beta_out, row_ptr, col_idx, col_capacity, ws, &ws_bytes, stream);
}

rbs_status rbs_select_per_head(const float* k_centroid, const float* k_radius,
                               const float* q_rep_head, const float* q_rep_head_norm,
                               const float* beta_in, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t n_blocks, int32_t head_dim, double keep_ratio_centroid,
                               double keep_ratio_rescue, uint32_t flags, float* beta_out,
                               int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                               void* workspace, size_t* workspace_bytes, void* stream) {
  return select_common(k_centroid, k_radius, q_rep_head, q_rep_head_norm, beta_in, n_q_heads,
                       n_kv_heads, n_blocks, head_dim, keep_ratio_centroid, keep_ratio_rescue,
                       flags, beta_out, row_ptr, col_idx, col_capacity, workspace,
                       workspace_bytes, stream);
}

rbs_status blocksparse_attn_fwd(rbs_dtype dt, const void* q, const void* k, const void* v,
                                int32_t seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, int32_t block, const int32_t* row_ptr,
                                const int32_t* col_idx, float softmax_scale, void* out,
                                float* lse, void* stream) {
  return attn_common(dt, q, k, v, seqlen, n_q_heads, n_kv_heads, head_dim, block, row_ptr,
                     col_idx, softmax_scale, out, lse, false, stream);
}

rbs_status blocksparse_attn_fwd_fp8(const void* q, const void* k, const void* v, int32_t seqlen,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block, const int32_t* row_ptr, const int32_t* col_idx,
                                    float softmax_scale, float q_descale, float k_descale,
                                    float v_descale, void* out, float* lse, void* stream) {
  AttnArgs a;
  const rbs_status st = attn_args(q, k, v, seqlen, n_q_heads, n_kv_heads, head_dim, block, row_ptr,
                                  col_idx, softmax_scale, out, lse, false, a);
  if (st != RBS_OK) return st;
  for (const float d : {q_descale, k_descale, v_descale})
    if (!(d > 0.f) || isinf(d)) return RBS_E_ARG;
  if (head_dim != 128 || block != 128) return RBS_E_UNSUPPORTED;
  if (seqlen == 0) return RBS_OK;
  return launch_attn_fp8_csr(a, q_descale, k_descale, v_descale, as_stream(stream));
}

rbs_status blocksparse_attn_fwd_shared_query(rbs_dtype dt, const void* q, const void* k,
                                             const void* v, int32_t seqlen, int32_t n_q_heads,
                                             int32_t n_kv_heads, int32_t head_dim, int32_t block,
                                             const int32_t* row_ptr, const int32_t* col_idx,
                                             float softmax_scale, void* out, float* lse,
                                             void* stream) {
  if (dt != RBS_DT_BF16 && dt != RBS_DT_F32) return RBS_E_ARG;
  AttnArgs a;
  const rbs_status st = attn_args(q, k, v, seqlen, n_q_heads, n_kv_heads, head_dim, block, row_ptr,
                                  col_idx, softmax_scale, out, lse, false, a);
  if (st != RBS_OK) return st;
  if (dt != RBS_DT_BF16 || head_dim != 128 || block != 128) return RBS_E_UNSUPPORTED;
  if (seqlen == 0) return RBS_OK;
  return launch_attn_bf16_pairs(a, as_stream(stream));
}

rbs_status blocksparse_attn_fwd_per_head(rbs_dtype dt, const void* q, const void* k,
                                         const void* v, int32_t seqlen, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t block,
                                         const int32_t* row_ptr, const int32_t* col_idx,
                                         float softmax_scale, void* out, float* lse,
                                         void* stream) {
  return attn_common(dt, q, k, v, seqlen, n_q_heads, n_kv_heads, head_dim, block, row_ptr,
                     col_idx, softmax_scale, out, lse, true, stream);
}

rbs_status block_mask_attn_fwd(rbs_dtype dt, const void* q, const void* k_cached,
                               const void* v, int32_t seqlen, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t n_segments,
                               const int32_t* seg_start, const int32_t* k_rerotate,
                               float rope_theta, int32_t q_row_begin, float softmax_scale,
                               void* out, float* lse, void* workspace, size_t* workspace_bytes,
                               void* stream) {
  if (dt != RBS_DT_BF16 && dt != RBS_DT_F32) return RBS_E_ARG;
  if (seqlen < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || n_segments <= 0)
    return RBS_E_ARG;
  if (n_q_heads % n_kv_heads != 0) return RBS_E_ARG;
  if (!seg_start || !k_rerotate || !workspace_bytes) return RBS_E_ARG;
  if (!aligned(q, 16) || !aligned(k_cached, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return RBS_E_ARG;
  if (!(rope_theta > 0.f) || isinf(rope_theta)) return RBS_E_ARG;
  if (isnan(softmax_scale) || isinf(softmax_scale)) return RBS_E_ARG;
  if (q_row_begin < 0 || q_row_begin > seqlen) return RBS_E_ARG;
  if (seg_start[0] != 0 || seg_start[n_segments] != seqlen) return RBS_E_ARG;
  for (int p = 0; p < n_segments; ++p) {
    if (seg_start[p + 1] <= seg_start[p]) return RBS_E_ARG;
    if (k_rerotate[p] < 0) return RBS_E_ARG;
  }
  if (dt != RBS_DT_BF16 || head_dim != 128) return RBS_E_UNSUPPORTED;
  if (n_segments > kMaxSegments) return RBS_E_UNSUPPORTED;
  for (int p = 0; p < n_segments; ++p)
    if (seg_start[p] % 128 != 0) return RBS_E_UNSUPPORTED;
  if ((int64_t)seqlen * n_q_heads * head_dim > ((int64_t)1 << 40)) return RBS_E_UNSUPPORTED;
  // Work plan. (1) When any segment has a nonzero offset, the keys are
  // re-encoded once into the workspace and the attention reads that copy.
  // (2) The final block's query tiles see every earlier tile; when they see
  // many, each one's key range is cut into chunks of kChunkTiles tiles run by
  // separate workgroups (placed first in the launch, ahead of the other
  // tiles), whose partial results a second kernel merges; otherwise these
  // few long rows would set the kernel's length.
  bool rotate = false;
  for (int p = 0; p < n_segments; ++p) rotate = rotate || k_rerotate[p] != 0;
  rotate = rotate && q_row_begin < seqlen;
  const int nq = (seqlen + 127) / 128;
  const int qt_begin = q_row_begin / 128;
  const int fs = seg_start[n_segments - 1] / 128;  // first tile of the final block
  const int final_lo = fs > qt_begin ? fs : qt_begin;
  const bool split = seqlen > 0 && q_row_begin < seqlen && final_lo < nq &&
                     final_lo + 1 >= 2 * kChunkTiles;
  const int chunks = split ? (nq + kChunkTiles - 1) / kChunkTiles : 0;
  const size_t keys_bytes =
      rotate ? align256((size_t)seqlen * n_kv_heads * head_dim * 2) : 0;
  const size_t table_bytes = rotate ? align256((size_t)n_segments * (head_dim / 2) * 8) : 0;
  const size_t part_bytes =
      split ? (size_t)(nq - final_lo) * n_q_heads * chunks * 128 * kPartRow * sizeof(float) : 0;
  const size_t need = keys_bytes + table_bytes + part_bytes;
  if (!workspace) {
    *workspace_bytes = need;
    return RBS_OK;
  }
  if (*workspace_bytes < need) return RBS_E_CAPACITY;
  if (need > 0 && !aligned(workspace, 256)) return RBS_E_ARG;
  if (seqlen == 0 || q_row_begin == seqlen) return RBS_OK;
  char* ws = static_cast<char*>(workspace);
  AttnArgs a;
  a.q = q;
  a.k = rotate ? ws : k_cached;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.row_ptr = nullptr;
  a.col_idx = nullptr;
  a.per_head = 0;
  a.S = seqlen;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.D = head_dim;
  a.B = 128;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  SegArgs s;
  memset(&s, 0, sizeof(s));
  s.n_seg = n_segments;
  s.q_row_begin = q_row_begin;
  s.theta = rope_theta;
  for (int p = 0; p <= n_segments; ++p) s.start[p] = seg_start[p];
  for (int p = 0; p < n_segments; ++p) s.rerot[p] = k_rerotate[p];
  hipStream_t st = as_stream(stream);
  if (rotate) {
    rbs_status r = launch_rerotate(k_cached, ws, reinterpret_cast<float2*>(ws + keys_bytes),
                                   seqlen, n_kv_heads, s, st);
    if (r != RBS_OK) return r;
  }
  if (!split) {
    s.rest_lo = qt_begin;
    s.rest_hi = nq;
    return launch_attn_segments(a, s, st);
  }
  s.qt_lo = final_lo;
  s.qt_hi = nq;
  s.chunks = chunks;
  s.chunk_tiles = kChunkTiles;
  s.part = reinterpret_cast<float*>(ws + keys_bytes + table_bytes);
  s.grid_split = attn_split_grid(n_q_heads, n_kv_heads, nq - final_lo, chunks);
  s.rest_lo = qt_begin;
  s.rest_hi = fs < nq ? fs : nq;
  rbs_status r = launch_attn_segments(a, s, st);
  if (r != RBS_OK) return r;
  return launch_attn_combine(a, s, st);
}

}  // extern "C"
