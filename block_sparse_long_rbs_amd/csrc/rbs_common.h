// Internal helpers shared by the librbs HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rbs.h"

namespace rbs {

constexpr int kWave = 64;

// bf16 is carried as raw uint16_t bits; widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

// Launch-error helper for host launchers.
inline rbs_status launch_status() {
  return hipGetLastError() == hipSuccess ? RBS_OK : RBS_E_HIP;
}

// Host launchers (one per kernel family); arguments are validated by the API layer.
// qrep/qnorm (per KV head) and qrep_h/qnorm_h (per query head) may each be
// null; the other outputs are always written.
rbs_status launch_block_stats(rbs_dtype dt, const void* q, const void* k, int S, int Hq, int Hkv,
                              int D, int B, float* cen, float* rad, float* qrep, float* qnorm,
                              float* qrep_h, float* qnorm_h, hipStream_t st);

struct SelectArgs {
  const float* cen;
  const float* rad;
  const float* qrep;
  const float* qnorm;
  const float* beta_in;
  float* beta_out;
  int32_t* row_ptr;
  int32_t* col_idx;
  int32_t* counts;   // workspace: [H*nb]
  int32_t* partial;  // workspace: [ceil(H*nb / 64)] count sums per 64 rows
  int32_t* lists;    // workspace: [H*nb][stride]
  float* scores;     // workspace: packed triangular centroid scores per row head (nb <= 1024)
  float* rbeta;      // workspace: r_j * beta_j per KV head (nb <= 1024)
  // Rows r = h * nb + i for h < H row heads: H = n_kv_heads with G = 1 (one
  // list per GQA group), or H = n_q_heads with G = n_q_heads / n_kv_heads (one
  // list per query head). qrep/qnorm are per row head; cen, rad and beta per
  // KV head h / G.
  int H, G, nb, D, stride;
  double rho_c, rho_r;
  int sink;
};
rbs_status launch_select(const SelectArgs& a, hipStream_t st);
// Device address and size of rbs_select_static's scratch array on the GPU
// that runs stream st (the current GPU for the null stream).
rbs_status static_scratch(hipStream_t st, void** ptr, size_t* bytes);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int S, Hq, Hkv, D, B;
  float scale;
  int per_head;   // CSR rows per query head (h * nb + i) instead of per KV head (g * nb + i)
};
rbs_status launch_attn_bf16_csr(const AttnArgs& a, hipStream_t st);
// Shared-query execution: neighbouring query tiles 2p and 2p + 1 of a head in
// one 8-wave workgroup over the union of their block lists.
rbs_status launch_attn_bf16_pairs(const AttnArgs& a, hipStream_t st);
// fp8 (e4m3) Q, K, V with per-tensor dequantisation factors; bf16 output.
rbs_status launch_attn_fp8_csr(const AttnArgs& a, float q_descale, float k_descale,
                               float v_descale, hipStream_t st);
// Vector-ALU path: fp32 inputs, or bf16 with head dim or block 64.
rbs_status launch_attn_vec_csr(const AttnArgs& a, bool bf16, hipStream_t st);
int select_rows_per_group(int nb, int D);
size_t select_score_workspace(int H, int nb);

constexpr int kMaxSegments = 256;
struct SegArgs {
  int n_seg;
  int q_row_begin;
  float theta;
  // One launch covers two ranges of query tiles. Workgroups [0, grid_split)
  // take tiles [qt_lo, qt_hi), each tile's key range cut into `chunks` pieces
  // of chunk_tiles tiles whose unnormalised partial results go to `part`
  // (merged afterwards by the combine kernel); the remaining workgroups take
  // tiles [rest_lo, rest_hi) whole. grid_split = 0 when nothing is split.
  int qt_lo, qt_hi;
  int chunks, chunk_tiles;
  int rest_lo, rest_hi;
  int grid_split;
  float* part;
  int32_t start[kMaxSegments + 1];
  int32_t rerot[kMaxSegments];
};
// Floats per query row in the partial-result workspace: O (D), m, l, then
// padding to a 16-byte multiple.
constexpr int kPartRow = 128 + 4;
// Workgroups of the split part of a segment launch (a multiple of 8).
int attn_split_grid(int Hq, int Hkv, int n_qt, int chunks);
rbs_status launch_attn_segments(const AttnArgs& a, const SegArgs& s, hipStream_t st);
rbs_status launch_attn_combine(const AttnArgs& a, const SegArgs& s, hipStream_t st);
// Position re-encoding: k_out = k_in with every key of segment p rotated by
// s.rerot[p] positions; `table` receives n_seg * 64 cos/sin pairs.
rbs_status launch_rerotate(const void* k_in, void* k_out, float2* table, int S, int Hkv,
                           const SegArgs& s, hipStream_t st);

}  // namespace rbs
