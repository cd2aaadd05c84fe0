// Dual-branch key-block selection into CSR block lists.
//
// RBS-Attention explainer (techfordev), "The Fix: A Radius-Adaptive Rescue
// Branch": centroid branch q.c_b, rescue branch q.c_b + ||q||_2 r_b beta_b,
// each thresholded on its own, masks combined; the Indonesian explainer's
// "Dual-Branch Selection" section says the same. beta is clamped to [0, 1] and
// derived from the head's radius distribution (the pages give no formula; the
// reading here is clamp((r - mean) / (max - mean), 0, 1)).
//
// Kernel 1 (select): one workgroup per (KV head g, R consecutive query
// blocks). It computes the R x (i+1) centroid scores once into LDS (the c_j
// rows are read once per workgroup, not once per query block), then one wave
// per query block runs two exact top-n selections by a 32-step radix select on
// order-preserving integer keys (ties to the lower block index), ORs the sets
// with the diagonal and the optional sink, and writes the ascending row into a
// fixed-stride workspace slot with its count.
// Kernel 2 (compact): exclusive scan of the counts into row_ptr and a copy of
// each row into col_idx.

#include <math.h>

#include "rbs_common.h"

namespace rbs {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 16;          // query blocks per workgroup
constexpr size_t kLdsBudget = 64 * 1024;  // bytes of LDS per workgroup

__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;  // -0 -> +0 so both zeros tie
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int budget(int n_visible, double rho) {
  // separate correctly rounded multiply and subtract (no fused contraction)
  double x = ceil(__dsub_rn(__dmul_rn(rho, (double)n_visible), 1e-6));
  int n = x < 1.0 ? 1 : (int)x;
  return n < n_visible ? n : n_visible;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// n-th largest key among lane-strided candidates j < nvis (keys from LDS via
// the functor), then the membership of j by (key > T) or (key == T and among
// the first `need` ties by ascending j).
template <typename KeyFn>
__device__ __forceinline__ uint32_t nth_largest(int nvis, int n, KeyFn key) {
  const int lane = threadIdx.x & 63;
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
    for (int j0 = 0; j0 < nvis; j0 += 64) {
      const int j = j0 + lane;
      const bool p = j < nvis && key(j) >= cand;
      cnt += __popcll(__ballot(p));
    }
    if (cnt >= n) T = cand;
  }
  return T;
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a, int R) {
  extern __shared__ float smem[];
  const int g = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int nb = a.nb, D = a.D;
  const int rows = min(R, nb - i0);
  const int imax = i0 + rows - 1;
  const int ncols = imax + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  float* rb = smem;                         // [nb] r_j * beta_j
  float* qrow = rb + nb;                    // [R][D]
  float* red = qrow + R * D;                // [16]
  float* sc = red + 16;                     // [R][ncols_pad]
  const int pitch = (ncols + 3) & ~3;

  const float* rad = a.rad + (size_t)g * nb;
  // ---- rescue coefficient ----
  if (a.beta_in) {
    const float* bi = a.beta_in + (size_t)g * nb;
    for (int j = tid; j < nb; j += kThreads) rb[j] = rad[j] * bi[j];
    if (a.beta_out && blockIdx.x == 0)
      for (int j = tid; j < nb; j += kThreads) a.beta_out[(size_t)g * nb + j] = bi[j];
  } else {
    float s = 0.f, m = 0.f;
    for (int j = tid; j < nb; j += kThreads) {
      s += rad[j];
      m = fmaxf(m, rad[j]);
    }
    s = wave_sum(s);
    m = wave_max(m);
    if (lane == 0) { red[wave] = s; red[4 + wave] = m; }
    __syncthreads();
    const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)nb;
    const float mx = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
    const float spread = mx - mean;
    const bool ok = spread > 1e-6f * mx;
    for (int j = tid; j < nb; j += kThreads) {
      float b = ok ? fminf(fmaxf((rad[j] - mean) / spread, 0.f), 1.f) : 0.f;
      rb[j] = rad[j] * b;
      if (a.beta_out && blockIdx.x == 0) a.beta_out[(size_t)g * nb + j] = b;
    }
  }
  // ---- representative queries of this workgroup's rows ----
  for (int x = tid; x < rows * D; x += kThreads)
    qrow[x] = a.qrep[((size_t)g * nb + i0) * D + x];
  __syncthreads();

  // ---- centroid scores: one column j per thread, all R rows at once ----
  const float* cen = a.cen + (size_t)g * nb * D;
  for (int j = tid; j < ncols; j += kThreads) {
    float acc[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.f;
    const float4* cj = reinterpret_cast<const float4*>(cen + (size_t)j * D);
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 c = cj[d4];
#pragma unroll
      for (int r = 0; r < kMaxRows; ++r) {
        if (r < rows) {
          const float4 qv = reinterpret_cast<const float4*>(qrow + r * D)[d4];
          acc[r] = fmaf(qv.x, c.x, acc[r]);
          acc[r] = fmaf(qv.y, c.y, acc[r]);
          acc[r] = fmaf(qv.z, c.z, acc[r]);
          acc[r] = fmaf(qv.w, c.w, acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r)
      if (r < rows) sc[r * pitch + j] = acc[r];
  }
  __syncthreads();

  // ---- per-row selection, one wave per row ----
  for (int r = wave; r < rows; r += kThreads / 64) {
    const int i = i0 + r;
    const int nvis = i + 1;
    const float qn = a.qnorm[(size_t)g * nb + i];
    const float* s = sc + r * pitch;
    auto keyc = [&](int j) { return order_key(s[j]); };
    auto keyr = [&](int j) { return order_key(fmaf(qn, rb[j], s[j])); };
    const int nc = budget(nvis, a.rho_c);
    const int nr = budget(nvis, a.rho_r);
    const uint32_t Tc = nth_largest(nvis, nc, keyc);
    const uint32_t Tr = nth_largest(nvis, nr, keyr);
    // ties at the threshold: how many are needed, by ascending j
    int gtc = 0, gtr = 0;
    for (int j0 = 0; j0 < nvis; j0 += 64) {
      const int j = j0 + lane;
      gtc += __popcll(__ballot(j < nvis && keyc(j) > Tc));
      gtr += __popcll(__ballot(j < nvis && keyr(j) > Tr));
    }
    int needc = nc - gtc, needr = nr - gtr;
    int base = 0;
    int32_t* out = a.lists + ((size_t)g * nb + i) * a.stride;
    for (int j0 = 0; j0 < nvis; j0 += 64) {
      const int j = j0 + lane;
      const bool in = j < nvis;
      const uint32_t kc = in ? keyc(j) : 0u, kr = in ? keyr(j) : 0u;
      const uint64_t tiec = __ballot(in && kc == Tc);
      const uint64_t tier = __ballot(in && kr == Tr);
      const int rankc = __popcll(tiec & lanemask_lt());
      const int rankr = __popcll(tier & lanemask_lt());
      bool sel = in && ((kc > Tc) || (kc == Tc && rankc < needc) || (kr > Tr) ||
                        (kr == Tr && rankr < needr) || j == i || (a.sink && j == 0));
      needc -= __popcll(tiec);
      needr -= __popcll(tier);
      const uint64_t m = __ballot(sel);
      const int pos = base + __popcll(m & lanemask_lt());
      if (sel && pos < a.stride) out[pos] = j;
      base += __popcll(m);
    }
    if (lane == 0) a.counts[(size_t)g * nb + i] = min(base, a.stride);
  }
}

// Exclusive scan of counts into row_ptr and copy of rows into col_idx.
__global__ __launch_bounds__(kThreads) void compact_kernel(const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ lists,
                                                           int stride, int nrows,
                                                           int32_t* __restrict__ row_ptr,
                                                           int32_t* __restrict__ col_idx) {
  __shared__ int sbuf[kThreads];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * kThreads;
  // base = sum of counts before this workgroup's rows
  int s = 0;
  for (int x = tid; x < r0; x += kThreads) s += counts[x];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  const int base = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  // inclusive scan of this workgroup's counts
  const int row = r0 + tid;
  const int c = row < nrows ? counts[row] : 0;
  int x = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  const int incl = base + off + x;
  if (row < nrows) row_ptr[row + 1] = incl;
  if (row == 0) row_ptr[0] = 0;
  sbuf[tid] = incl - c;  // exclusive start of each row
  __syncthreads();
  // copy: one wave per row
  const int nr = min(kThreads, nrows - r0);
  for (int rr = wave; rr < nr; rr += 4) {
    const int rowi = r0 + rr;
    const int cnt = counts[rowi];
    const int start = sbuf[rr];
    const int32_t* src = lists + (size_t)rowi * stride;
    for (int e = lane; e < cnt; e += 64) col_idx[start + e] = src[e];
  }
}

__global__ void zero_row_ptr_kernel(int32_t* row_ptr) { row_ptr[0] = 0; }

}  // namespace

int select_rows_per_group(int nb, int D) {
  // LDS: rb[nb] + qrow[R*D] + red[16] + sc[R*pitch] floats
  for (int R = kMaxRows; R >= 1; --R) {
    const size_t bytes = ((size_t)nb + (size_t)R * D + 16 + (size_t)R * ((nb + 3) & ~3)) * 4;
    if (bytes <= kLdsBudget) return R;
  }
  return 0;
}

rbs_status launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.nb == 0) {
    hipLaunchKernelGGL(zero_row_ptr_kernel, dim3(1), dim3(1), 0, st, a.row_ptr);
    return launch_status();
  }
  const int R = select_rows_per_group(a.nb, a.D);
  if (R <= 0) return RBS_E_UNSUPPORTED;
  const size_t shmem = ((size_t)a.nb + (size_t)R * a.D + 16 + (size_t)R * ((a.nb + 3) & ~3)) * 4;
  dim3 grid((a.nb + R - 1) / R, a.Hkv);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), shmem, st, a, R);
  rbs_status s = launch_status();
  if (s != RBS_OK) return s;
  const int nrows = a.Hkv * a.nb;
  hipLaunchKernelGGL(compact_kernel, dim3((nrows + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     st, a.counts, a.lists, a.stride, nrows, a.row_ptr, a.col_idx);
  return launch_status();
}

}  // namespace rbs
