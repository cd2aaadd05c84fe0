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
// Launches are XCD-aware: a head's work items run on a fixed subset of the
// eight XCDs, so its statistics and score rows stay in those XCDs' L2.

#include <math.h>

#include <mutex>

#include "rbs_common.h"

namespace rbs {
namespace {

constexpr int kThreads = 256;
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

// Radix select over order-preserving 32-bit keys: the n-th largest key
// among the row's candidates (lane-strided, M per lane; absent candidates
// carry key 0, below every real key). Bits are fixed from the top; it stops
// as soon as exactly n keys are >= the prefix, which then is a valid
// threshold (every key above it is kept, none below).
template <int M>
__device__ __forceinline__ uint32_t nth_largest_regs(const uint32_t (&key)[M], int n) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) cnt += __popcll(__ballot(key[m] >= cand));
    if (cnt >= n) {
      T = cand;
      if (cnt == n) break;
    }
  }
  return T;
}

// Keep the keys > T plus the first (n - #keys > T) keys equal to T in
// ascending index order; returns this lane's membership bits.
template <int M>
__device__ __forceinline__ uint32_t take_top(const uint32_t (&key)[M], int n, uint32_t T) {
  int gt = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) gt += __popcll(__ballot(key[m] > T));
  int need = n - gt;
  uint32_t bits = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint64_t tie = __ballot(key[m] == T);
    const int rank = __popcll(tie & lanemask_lt());
    if (key[m] > T || (key[m] == T && rank < need)) bits |= 1u << m;
    need -= __popcll(tie);
  }
  return bits;
}

// ---------------------------------------------------------------------------
// Two-kernel path for nb <= kTriMaxBlocks.
//
// Kernel A (scores): the centroid scores s[g][i][j] = q_rep[g][i] . c[g][j]
// for j <= i form a lower triangle, cut into 64 x 64 tiles (one workgroup
// each, equal work); every wave computes one 32 x 32 sub-tile with fp32
// matrix-core products (v_mfma_f32_32x32x2_f32, fp32 inputs and
// accumulation), operands staged once per tile in LDS. Scores go to a packed
// triangular workspace (row i starts at i (i + 1) / 2). One extra workgroup
// per KV head derives its rescue coefficients and stores r_j * beta_j.
// Kernel B (rows): one wave per (g, i) ranks the row's keys held in
// registers (centroid key and rescue key per candidate) and writes the
// selected block list.

constexpr int kTriMaxBlocks = 1024;
constexpr int kTile = 64;

__host__ __device__ __forceinline__ size_t tri_off(int i) { return (size_t)i * (i + 1) / 2; }

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Work item (head g, item t) of a launch whose T items per head are spread so
// that each head's items run on a fixed subset of the eight XCDs (workgroup
// x runs on XCD x % 8): the head's statistics and score rows are then
// fetched into one or two XCDs' L2 instead of all eight. Returns false for
// padding workgroups.
__device__ __forceinline__ bool xcd_item(int x, int H, int T, int& g, int& t) {
  const int xcd = x & 7, s = x >> 3;
  if (H % 8 == 0) {                 // H / 8 heads per XCD
    g = xcd + 8 * (s / T);
    t = s % T;
    return g < H;
  }
  if (8 % H == 0) {                 // 8 / H XCDs per head, items interleaved
    const int reps = 8 / H;
    g = xcd % H;
    t = s * reps + xcd / H;
    return t < T;
  }
  g = x / T;                        // any other head count: plain order
  t = x % T;
  return g < H;
}

__host__ __forceinline__ int xcd_grid(int H, int T) {
  if (H % 8 == 0) return H * T;
  if (8 % H == 0) return 8 * ((T + 8 / H - 1) / (8 / H));
  return H * T;
}

template <int D>
__global__ __launch_bounds__(kThreads) void score_tiles_kernel(SelectArgs a) {
  const int nb = a.nb;
  const int nt = (nb + kTile - 1) / kTile;
  const int ntiles = nt * (nt + 1) / 2;
  int g, item;                     // row head, tile (ntiles: the rescue-coefficient item)
  if (!xcd_item(blockIdx.x, a.H, ntiles + 1, g, item)) return;
  const int gk = g / a.G;          // its KV head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (item >= ntiles) {
    // row head 0's item also clears the per-64-row count sums that the row
    // kernel (which runs after this kernel) accumulates
    if (g == 0 && a.partial)
      for (int x = tid; x < (a.H * nb + 63) / 64; x += kThreads) a.partial[x] = 0;
    // rescue coefficients of KV head gk (once, from its first row head):
    // beta = clamp((r - mean) / (max - mean), 0, 1)
    __shared__ float red[8];
    if (g % a.G != 0) return;
    const float* rad = a.rad + (size_t)gk * nb;
    float* rb = a.rbeta + (size_t)gk * nb;
    if (a.beta_in) {
      const float* bi = a.beta_in + (size_t)gk * nb;
      for (int j = tid; j < nb; j += kThreads) {
        rb[j] = rad[j] * bi[j];
        if (a.beta_out) a.beta_out[(size_t)gk * nb + j] = bi[j];
      }
      return;
    }
    float sum = 0.f, mx = 0.f;
    for (int j = tid; j < nb; j += kThreads) {
      sum += rad[j];
      mx = fmaxf(mx, rad[j]);
    }
    sum = wave_sum(sum);
    mx = wave_max(mx);
    if (lane == 0) { red[wave] = sum; red[4 + wave] = mx; }
    __syncthreads();
    const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)nb;
    const float top = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
    const float spread = top - mean;
    const bool ok = spread > 1e-6f * top;
    for (int j = tid; j < nb; j += kThreads) {
      const float b = ok ? fminf(fmaxf((rad[j] - mean) / spread, 0.f), 1.f) : 0.f;
      rb[j] = rad[j] * b;
      if (a.beta_out) a.beta_out[(size_t)gk * nb + j] = b;
    }
    return;
  }
  // tile index -> (row tile ti, column tile tj <= ti), heaviest rows first
  int t = item;
  int ti = nt - 1;
  while (t > ti) { t -= ti + 1; --ti; }
  const int tj = t;
  // the tile's 64 representative-query rows and 64 centroid rows are staged
  // once in LDS (rows padded by 16 bytes against bank conflicts) and shared
  // by the four waves
  constexpr int P = D + 4;
  constexpr int V = D / 4;                     // float4 per row
  constexpr int NL = kTile * V / kThreads;     // float4 per thread per operand
  __shared__ __attribute__((aligned(16))) float qs[kTile * P];
  __shared__ __attribute__((aligned(16))) float cs[kTile * P];
  const int i0 = ti * kTile, j0 = tj * kTile;
  {
    const float* qg = a.qrep + (size_t)g * nb * D;
    const float* cg = a.cen + (size_t)gk * nb * D;
    float4 vq[NL], vc[NL];
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int x = tid + n * kThreads, r = x / V, c4 = x % V;
      vq[n] = *reinterpret_cast<const float4*>(qg + (size_t)min(i0 + r, nb - 1) * D + 4 * c4);
      vc[n] = *reinterpret_cast<const float4*>(cg + (size_t)min(j0 + r, nb - 1) * D + 4 * c4);
    }
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      const int x = tid + n * kThreads, r = x / V, c4 = x % V;
      *reinterpret_cast<float4*>(qs + r * P + 4 * c4) = vq[n];
      *reinterpret_cast<float4*>(cs + r * P + 4 * c4) = vc[n];
    }
  }
  __syncthreads();
  const int i_base = i0 + 32 * (wave >> 1);
  const int j_base = j0 + 32 * (wave & 1);
  if (j_base > i_base + 31) return;  // sub-tile entirely above the diagonal
  const int m32 = lane & 31, hh = lane >> 5;
  const float* qrow = qs + (32 * (wave >> 1) + m32) * P + 4 * hh;
  const float* crow = cs + (32 * (wave & 1) + m32) * P + 4 * hh;
  float4 qa[D / 8], cb[D / 8];
#pragma unroll
  for (int s8 = 0; s8 < D / 8; ++s8) {
    qa[s8] = *reinterpret_cast<const float4*>(qrow + 8 * s8);
    cb[s8] = *reinterpret_cast<const float4*>(crow + 8 * s8);
  }
  f32x16_t acc = (f32x16_t){};
#pragma unroll
  for (int s8 = 0; s8 < D / 8; ++s8) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s8].x, cb[s8].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s8].y, cb[s8].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s8].z, cb[s8].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s8].w, cb[s8].w, acc, 0, 0, 0);
  }
  float* sg = a.scores + (size_t)g * tri_off(nb);
  const int j = j_base + m32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i_base + 8 * (r >> 2) + 4 * hh + (r & 3);
    if (i < nb && j <= i) sg[tri_off(i) + j] = acc[r];
  }
}

// Both branches' radix selects in one loop (independent ballot chains).
template <int M>
__device__ __forceinline__ void nth_largest_pair(const uint32_t (&ka)[M], int na,
                                                 const uint32_t (&kb)[M], int nbr, uint32_t& Ta,
                                                 uint32_t& Tb) {
  Ta = 0;
  Tb = 0;
  bool da = false, db = false;
  for (int bit = 31; bit >= 0 && !(da && db); --bit) {
    const uint32_t ca = Ta | (1u << bit), cbv = Tb | (1u << bit);
    int cnta = 0, cntb = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      cnta += __popcll(__ballot(ka[m] >= ca));
      cntb += __popcll(__ballot(kb[m] >= cbv));
    }
    if (!da && cnta >= na) {
      Ta = ca;
      da = (cnta == na);
    }
    if (!db && cntb >= nbr) {
      Tb = cbv;
      db = (cntb == nbr);
    }
  }
}

constexpr int kSelM = 16;   // candidates per lane held in registers (nb <= 1024)

// The n-th largest key for n <= 64 without a ballot per candidate per bit.
// The n-th largest of the 64 per-lane maxima, T_low, is a lower bound on the
// answer (n distinct keys are >= it), so only the keys >= T_low (n of them
// at least, usually few more) can matter: they are compacted into `buf`
// (this wave's LDS slice, 64 M keys) and the radix search runs on them, one
// or a few per lane. Every key of the row >= the result is among them; a
// result below T_low (possible only when exactly n keys are >= T_low) is
// raised to T_low, which then has exactly n keys at or above it.
template <int M>
__device__ __forceinline__ uint32_t nth_largest_small(const uint32_t (&key)[M], int n,
                                                      uint32_t* buf) {
  const int lane = threadIdx.x & 63;
  uint32_t lm = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) lm = max(lm, key[m]);
  const uint32_t lmv[1] = {lm};
  const uint32_t tlow = nth_largest_regs<1>(lmv, n);
  int c = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool in = key[m] >= tlow;
    const uint64_t msk = __ballot(in);
    if (in) buf[c + __popcll(msk & lanemask_lt())] = key[m];
    c += __popcll(msk);
  }
  uint32_t t;
  if (c <= 64) {
    const uint32_t k1[1] = {lane < c ? buf[lane] : 0u};
    t = nth_largest_regs<1>(k1, n);
  } else if (c <= 256) {
    uint32_t k4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) k4[q] = lane + 64 * q < c ? buf[lane + 64 * q] : 0u;
    t = nth_largest_regs<4>(k4, n);
  } else {
    t = nth_largest_regs<M>(key, n);
  }
  return max(t, tlow);
}

// One row (g, i): its i + 1 candidates, M per lane (64 M >= i + 1).
template <int M>
__device__ __forceinline__ int select_row(const SelectArgs& a, int g, int i, uint32_t* buf) {
  const int nb = a.nb;
  const int lane = threadIdx.x & 63;
  const int nvis = i + 1;
  const float qn = a.qnorm[(size_t)g * nb + i];
  const float* srow = a.scores + (size_t)g * tri_off(nb) + tri_off(i);
  const float* rb = a.rbeta + (size_t)(g / a.G) * nb;
  uint32_t kc[M], kr[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = lane + 64 * m;
    const bool in = j < nvis;
    const float sv = in ? srow[j] : 0.f;
    const float rbj = in ? rb[j] : 0.f;
    kc[m] = in ? order_key(sv) : 0u;
    kr[m] = in ? order_key(fmaf(qn, rbj, sv)) : 0u;
  }
  const int nc = budget(nvis, a.rho_c);
  const int nr = budget(nvis, a.rho_r);
  uint32_t Tc, Tr;
  if (nc <= 64 && nr <= 64) {
    Tc = nth_largest_small(kc, nc, buf);
    Tr = nth_largest_small(kr, nr, buf);
  } else {
    nth_largest_pair(kc, nc, kr, nr, Tc, Tr);
  }
  const uint32_t bits = take_top(kc, nc, Tc) | take_top(kr, nr, Tr);
  int base = 0;
  int32_t* out = a.lists + ((size_t)g * nb + i) * a.stride;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = lane + 64 * m;
    const bool sel = j < nvis && (((bits >> m) & 1u) || j == i || (a.sink && j == 0));
    const uint64_t msk = __ballot(sel);
    const int pos = base + __popcll(msk & lanemask_lt());
    if (sel && pos < a.stride) out[pos] = j;
    base += __popcll(msk);
  }
  const int n = min(base, a.stride);
  if (lane == 0) a.counts[(size_t)g * nb + i] = n;
  return n;
}

__global__ __launch_bounds__(kThreads) void select_rows_kernel(SelectArgs a) {
  __shared__ uint32_t cand[kThreads / 64][64 * kSelM];
  const int nb = a.nb;
  const int wave = threadIdx.x >> 6;
  // 4 rows per workgroup, all of one row head, on that head's XCDs;
  // heaviest rows first
  const int rows_per_g = (nb + 3) / 4;
  int g, item;
  if (!xcd_item(blockIdx.x, a.H, rows_per_g, g, item)) return;
  const int i = nb - 1 - (item * 4 + wave);
  int n = 0;
  if (i >= 0) {
    if (i < 4 * 64) n = select_row<4>(a, g, i, cand[wave]);
    else if (i < 8 * 64) n = select_row<8>(a, g, i, cand[wave]);
    else n = select_row<kSelM>(a, g, i, cand[wave]);
  }
  // the workgroup's row counts go into the per-64-row sums with one atomic
  // per 64-row group touched (the four rows are consecutive)
  __shared__ int wc[4];
  if ((threadIdx.x & 63) == 0) wc[wave] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    int grp = -1, acc = 0;
    for (int w = 3; w >= 0; --w) {   // ascending rows
      const int iw = nb - 1 - (item * 4 + w);
      if (iw < 0) continue;
      const int gr = (int)(((size_t)g * nb + iw) >> 6);
      if (gr != grp) {
        if (grp >= 0 && acc) atomicAdd(a.partial + grp, acc);
        grp = gr;
        acc = 0;
      }
      acc += wc[w];
    }
    if (grp >= 0 && acc) atomicAdd(a.partial + grp, acc);
  }
}

constexpr int kLongRows = 8;  // query blocks per workgroup on the long-row path

// beta_out is written once per KV head, by its first row head
__device__ __forceinline__ bool grp_is_first_head(int g, int G) { return g % G == 0; }

// Generic path for long rows (nb > 1024): keys are recomputed from LDS
// on every pass instead of being held in registers.
template <typename KeyFn>
__device__ uint32_t nth_largest_lds(int nvis, int n, KeyFn key) {
  const int lane = threadIdx.x & 63;
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
    for (int j0 = 0; j0 < nvis; j0 += 64) {
      const int j = j0 + lane;
      cnt += __popcll(__ballot(j < nvis && key(j) >= cand));
    }
    if (cnt >= n) {
      T = cand;
      if (cnt == n) break;
    }
  }
  return T;
}

__global__ __launch_bounds__(kThreads) void select_long_kernel(SelectArgs a, int R) {
  extern __shared__ float smem[];
  const int g = blockIdx.y;        // row head
  const int gk = g / a.G;          // its KV head
  const bool beta_writer = grp_is_first_head(g, a.G);
  const int nb = a.nb, D = a.D;
  const int grp = gridDim.x - 1 - blockIdx.x;
  const int i0 = grp * R;
  const int rows = min(R, nb - i0);
  const int ncols = i0 + rows;
  const int pitch = (ncols + 3) & ~3;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  float* rb = smem;
  float* qrow = rb + ((nb + 3) & ~3);
  float* red = qrow + R * D;
  float* sc = red + 16;
  const float* rad = a.rad + (size_t)gk * nb;
  if (a.beta_in) {
    const float* bi = a.beta_in + (size_t)gk * nb;
    for (int j = tid; j < ncols; j += kThreads) rb[j] = rad[j] * bi[j];
    if (a.beta_out && grp == 0 && beta_writer)
      for (int j = tid; j < nb; j += kThreads) a.beta_out[(size_t)gk * nb + j] = bi[j];
  } else {
    float sum = 0.f, mx = 0.f;
    for (int j = tid; j < nb; j += kThreads) {
      sum += rad[j];
      mx = fmaxf(mx, rad[j]);
    }
    sum = wave_sum(sum);
    mx = wave_max(mx);
    if (lane == 0) { red[wave] = sum; red[4 + wave] = mx; }
    __syncthreads();
    const float mean = (red[0] + red[1] + red[2] + red[3]) / (float)nb;
    const float top = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
    const float spread = top - mean;
    const bool ok = spread > 1e-6f * top;
    const bool write_beta = a.beta_out && grp == 0 && beta_writer;
    const int jend = write_beta ? nb : ncols;
    for (int j = tid; j < jend; j += kThreads) {
      const float b = ok ? fminf(fmaxf((rad[j] - mean) / spread, 0.f), 1.f) : 0.f;
      if (j < ncols) rb[j] = rad[j] * b;
      if (write_beta) a.beta_out[(size_t)gk * nb + j] = b;
    }
  }
  for (int x = tid; x < rows * D; x += kThreads) qrow[x] = a.qrep[((size_t)g * nb + i0) * D + x];
  __syncthreads();
  const float* cen = a.cen + (size_t)gk * nb * D;
  for (int j = tid; j < ncols; j += kThreads) {
    const float4* cj = reinterpret_cast<const float4*>(cen + (size_t)j * D);
    for (int r = 0; r < rows; ++r) {
      float acc = 0.f;
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float4 c = cj[d4];
        const float4 qv = reinterpret_cast<const float4*>(qrow + r * D)[d4];
        acc = fmaf(qv.x, c.x, acc);
        acc = fmaf(qv.y, c.y, acc);
        acc = fmaf(qv.z, c.z, acc);
        acc = fmaf(qv.w, c.w, acc);
      }
      sc[r * pitch + j] = acc;
    }
  }
  __syncthreads();
  for (int r = wave; r < rows; r += kThreads / 64) {
    const int i = i0 + r;
    const int nvis = i + 1;
    const float qn = a.qnorm[(size_t)g * nb + i];
    const float* srow = sc + r * pitch;
    auto keyc = [&](int j) { return order_key(srow[j]); };
    auto keyr = [&](int j) { return order_key(fmaf(qn, rb[j], srow[j])); };
    const int nc = budget(nvis, a.rho_c);
    const int nr = budget(nvis, a.rho_r);
    const uint32_t Tc = nth_largest_lds(nvis, nc, keyc);
    const uint32_t Tr = nth_largest_lds(nvis, nr, keyr);
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
      const uint32_t kcv = in ? keyc(j) : 0u, krv = in ? keyr(j) : 0u;
      const uint64_t tiec = __ballot(in && kcv == Tc);
      const uint64_t tier = __ballot(in && krv == Tr);
      const int rankc = __popcll(tiec & lanemask_lt());
      const int rankr = __popcll(tier & lanemask_lt());
      const bool sel = in && ((kcv > Tc) || (kcv == Tc && rankc < needc) || (krv > Tr) ||
                              (krv == Tr && rankr < needr) || j == i || (a.sink && j == 0));
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

// CSR assembly: one workgroup per 16 rows. The row offsets are the sum of all
// earlier counts plus a scan inside the group; the copies are independent.
// The sum of all earlier counts is taken from the per-64-row sums when the
// row kernel produced them (partial != null), else from the counts.
constexpr int kCompactRows = 16;

__device__ __forceinline__ int wave_isum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(kThreads) void compact_kernel(const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ partial,
                                                           const int32_t* __restrict__ lists,
                                                           int stride, int nrows,
                                                           int32_t* __restrict__ row_ptr,
                                                           int32_t* __restrict__ col_idx) {
  __shared__ int start[kCompactRows];
  __shared__ int cnt_s[kCompactRows];
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * kCompactRows;
  const int nr = min(kCompactRows, nrows - r0);
  // sum of the counts of all earlier rows
  int s = 0;
  const int c0 = partial ? (r0 & ~63) : 0;   // earlier rows summed from the counts
  if (partial)
    for (int x = tid; x < (r0 >> 6); x += kThreads) s += partial[x];
  for (int x = c0 + tid; x < r0; x += kThreads) s += counts[x];
  s = wave_isum(s);
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  const int base = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  // inclusive scan of this group's counts (wave 0)
  if (wave == 0) {
    const int c = lane < nr ? counts[r0 + lane] : 0;
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane < nr) {
      start[lane] = base + x - c;
      cnt_s[lane] = c;
      row_ptr[r0 + lane + 1] = base + x;
    }
    if (r0 == 0 && lane == 0) row_ptr[0] = 0;
  }
  __syncthreads();
  // copy: wave w moves rows w, w + 4, w + 8, w + 12, 64 entries per pass;
  // the four rows' loads are issued together
  const int per = kCompactRows / 4;
  int c[per], st[per];
  int cmax = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int rr = wave + 4 * k;
    c[k] = rr < nr ? cnt_s[rr] : 0;
    st[k] = rr < nr ? start[rr] : 0;
    cmax = max(cmax, c[k]);
  }
  for (int e0 = 0; e0 < cmax; e0 += 64) {
    const int e = e0 + lane;
    int v[per];
#pragma unroll
    for (int k = 0; k < per; ++k)
      v[k] = e < c[k] ? lists[(size_t)(r0 + wave + 4 * k) * stride + e] : 0;
#pragma unroll
    for (int k = 0; k < per; ++k)
      if (e < c[k]) col_idx[st[k] + e] = v[k];
  }
}

__global__ void zero_row_ptr_kernel(int32_t* row_ptr) { row_ptr[0] = 0; }

}  // namespace

int select_rows_per_group(int nb, int D) {
  // LDS: rb[nb] + qrow[R*D] + red[16] + sc[R*pitch] floats
  for (int R = kLongRows; R >= 1; --R) {
    const size_t bytes =
        ((size_t)((nb + 3) & ~3) + (size_t)R * D + 16 + (size_t)R * ((nb + 3) & ~3)) * 4;
    if (bytes <= kLdsBudget) return R;
  }
  return 0;
}

size_t select_score_workspace(int H, int nb) {
  return nb <= kTriMaxBlocks ? (size_t)H * (tri_off(nb) + nb) * sizeof(float) : 0;
}

// Scratch of rbs_select_static: a file-scope device array, so that the call
// allocates nothing. Each GPU holds its own copy until the process ends;
// host code uses only the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[RBS_SELECT_STATIC_SCRATCH_BYTES];

rbs_status static_scratch(hipStream_t st, void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return RBS_E_HIP;
  dev = cur;
  if (st && hipStreamGetDevice(st, &dev) != hipSuccess) return RBS_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RBS_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the array's address on this device, taken with the device current
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return RBS_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return RBS_E_HIP;
    if (e != hipSuccess || !p) return RBS_E_HIP;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = RBS_SELECT_STATIC_SCRATCH_BYTES;
  return RBS_OK;
}

rbs_status launch_select(const SelectArgs& a, hipStream_t st) {
  if (a.nb == 0) {
    hipLaunchKernelGGL(zero_row_ptr_kernel, dim3(1), dim3(1), 0, st, a.row_ptr);
    return launch_status();
  }
  if (a.nb <= kTriMaxBlocks) {
    const int nt = (a.nb + kTile - 1) / kTile;
    dim3 g1(xcd_grid(a.H, nt * (nt + 1) / 2 + 1));
    if (a.D == 64)
      hipLaunchKernelGGL(score_tiles_kernel<64>, g1, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL(score_tiles_kernel<128>, g1, dim3(kThreads), 0, st, a);
    rbs_status s = launch_status();
    if (s != RBS_OK) return s;
    const int rows_per_g = (a.nb + 3) / 4;
    hipLaunchKernelGGL(select_rows_kernel, dim3(xcd_grid(a.H, rows_per_g)), dim3(kThreads), 0, st,
                       a);
  } else {
    const int R = select_rows_per_group(a.nb, a.D);
    if (R <= 0) return RBS_E_UNSUPPORTED;
    const size_t shmem =
        ((size_t)((a.nb + 3) & ~3) + (size_t)R * a.D + 16 + (size_t)R * ((a.nb + 3) & ~3)) * 4;
    dim3 grid((a.nb + R - 1) / R, a.H);
    hipLaunchKernelGGL(select_long_kernel, grid, dim3(kThreads), shmem, st, a, R);
  }
  rbs_status s = launch_status();
  if (s != RBS_OK) return s;
  const int nrows = a.H * a.nb;
  // the per-64-row sums exist on the score-tile path (its kernel clears them)
  const int32_t* partial = a.nb <= kTriMaxBlocks ? a.partial : nullptr;
  hipLaunchKernelGGL(compact_kernel, dim3((nrows + kCompactRows - 1) / kCompactRows),
                     dim3(kThreads), 0, st, a.counts, partial, a.lists, a.stride, nrows,
                     a.row_ptr, a.col_idx);
  return launch_status();
}

}  // namespace rbs
