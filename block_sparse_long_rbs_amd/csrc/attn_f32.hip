// Block-sparse causal GQA attention on the vector ALUs, fp32 arithmetic: the
// path for fp32 inputs and for the bf16 shapes the matrix-core kernel does not
// take (head dim or block 64).
//
// Same computation as the bf16 matrix-core kernel (RBS-Attention explainer,
// "The Fix": the combined block mask runs through a block-sparse attention),
// with every product, exponential and sum in fp32. bf16 inputs are widened
// exactly; a bf16 output is rounded to nearest even.
// One workgroup = 64 query rows of one query head inside one query block;
// four lanes share a row, each owning D/4 dimensions. Key tiles of 64 keys are
// staged into LDS; each tile is folded into the running softmax after its 64
// scores are known (one exponential per score plus one rescale per tile).

#include <math.h>

#include "rbs_common.h"

namespace rbs {
namespace {

constexpr int kThreads = 256;
constexpr int QROWS = 64;
constexpr int KT = 64;

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, size_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// T: float or uint16_t (bf16 bits).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_vec_kernel(AttnArgs a) {
  constexpr int DQ = D / 4;
  __shared__ float Ksh[KT][D];
  __shared__ float Vsh[KT][D];
  const int B = a.B;
  const int nb = (a.S + B - 1) / B;
  const int sub_per_block = B / QROWS;
  const int G = a.Hq / a.Hkv;
  // grid.x = Hq * nb * sub_per_block; heaviest query blocks first
  const int x = blockIdx.x;
  const int h = x % a.Hq;
  const int rest = x / a.Hq;
  const int sub = rest % sub_per_block;
  const int i = nb - 1 - rest / sub_per_block;
  const int g = h / G;
  const int tid = threadIdx.x;
  const int rloc = tid >> 2, quarter = tid & 3;
  const int t = i * B + sub * QROWS + rloc;
  const T* Q = static_cast<const T*>(a.q);
  const T* K = static_cast<const T*>(a.k);
  const T* V = static_cast<const T*>(a.v);
  float q[DQ], o[DQ];
#pragma unroll
  for (int d = 0; d < DQ; ++d) {
    q[d] = t < a.S ? ld(Q, ((size_t)t * a.Hq + h) * D + quarter * DQ + d) : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int row = (a.per_head ? h : g) * nb + i;
  const int e0 = a.row_ptr[row], e1 = a.row_ptr[row + 1];
  for (int e = e0; e < e1; ++e) {
    const int j = a.col_idx[e];
    if (j < 0 || j > i) continue;
    for (int kt0 = j * B; kt0 < min((j + 1) * B, a.S); kt0 += KT) {
      __syncthreads();
      for (int x2 = tid; x2 < KT * D; x2 += kThreads) {
        const int kr = x2 / D, d = x2 % D;
        const int u = kt0 + kr;
        const bool ok = u < a.S && u < (j + 1) * B;
        Ksh[kr][d] = ok ? ld(K, ((size_t)u * a.Hkv + g) * D + d) : 0.f;
        Vsh[kr][d] = ok ? ld(V, ((size_t)u * a.Hkv + g) * D + d) : 0.f;
      }
      __syncthreads();
      float s[KT];
      float mx = -INFINITY;
#pragma unroll 8
      for (int kr = 0; kr < KT; ++kr) {
        float p = 0.f;
#pragma unroll
        for (int d = 0; d < DQ; ++d) p = fmaf(q[d], Ksh[kr][quarter * DQ + d], p);
        p += __shfl_xor(p, 1, 64);
        p += __shfl_xor(p, 2, 64);
        const int u = kt0 + kr;
        const bool ok = u <= t && u < a.S && u < (j + 1) * B;
        s[kr] = ok ? p * a.scale : -INFINITY;
        mx = fmaxf(mx, s[kr]);
      }
      const float mnew = fmaxf(m, mx);
      if (mnew == -INFINITY) continue;  // nothing visible yet for this row
      const float alpha = expf(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DQ; ++d) o[d] *= alpha;
#pragma unroll 4
      for (int kr = 0; kr < KT; ++kr) {
        const float p = expf(s[kr] - mnew);
        l += p;
#pragma unroll
        for (int d = 0; d < DQ; ++d) o[d] = fmaf(p, Vsh[kr][quarter * DQ + d], o[d]);
      }
    }
  }
  if (t >= a.S) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* O = static_cast<T*>(a.out);
#pragma unroll
  for (int d = 0; d < DQ; ++d) st(O, ((size_t)t * a.Hq + h) * D + quarter * DQ + d, o[d] * inv);
  if (a.lse && quarter == 0) a.lse[(size_t)h * a.S + t] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

rbs_status launch_attn_vec_csr(const AttnArgs& a, bool bf16, hipStream_t stream) {
  const int nb = (a.S + a.B - 1) / a.B;
  const int grid = a.Hq * nb * (a.B / QROWS);
  if (bf16) {
    if (a.D == 64)
      hipLaunchKernelGGL((attn_vec_kernel<uint16_t, 64>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_vec_kernel<uint16_t, 128>), dim3(grid), dim3(kThreads), 0, stream, a);
  } else {
    if (a.D == 64)
      hipLaunchKernelGGL((attn_vec_kernel<float, 64>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_vec_kernel<float, 128>), dim3(grid), dim3(kThreads), 0, stream, a);
  }
  return launch_status();
}

}  // namespace rbs
