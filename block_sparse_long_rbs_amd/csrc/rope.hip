// Position re-encoding of cached keys for Block-attention.
//
// Block-attention page, section 2.3 "Position Re-encoding": a block's keys
// were encoded from position 0; before the final block attends to them they
// are rotated on to their position in the prompt. Here every key of segment p
// is rotated by k_rerotate[p] positions with the rotate-half RoPE pairing
// (x_i, x_{i+D/2}) and angle k_rerotate[p] * theta^(-2i/D), formed in double
// precision. The rotated keys are written once to a workspace copy that the
// attention kernel then reads like ordinary keys.
//
// Kernel 1: cos/sin table [n_seg][D/2] (float2), one thread per entry.
// Kernel 2: one thread per (token, KV head, 8 frequency pairs): reads the
// 16-byte chunks (x_i..x_{i+7}) and (x_{i+64}..x_{i+71}), writes both rotated,
// rounded to bf16. HBM bound: 2 x S x Hkv x D x 2 bytes.

#include <math.h>

#include "rbs_common.h"

namespace rbs {
namespace {

constexpr int D = 128;
constexpr int kThreads = 256;

__global__ void rope_table_kernel(SegArgs s, float2* __restrict__ table) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= s.n_seg * (D / 2)) return;
  const int p = x / (D / 2), i = x % (D / 2);
  const double inv = pow((double)s.theta, -2.0 * (double)i / (double)D);
  double sn, cs;
  sincos((double)s.rerot[p] * inv, &sn, &cs);
  table[x] = make_float2((float)cs, (float)sn);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__global__ __launch_bounds__(kThreads) void rope_rerotate_kernel(const uint16_t* __restrict__ k_in,
                                                                uint16_t* __restrict__ k_out,
                                                                int S, int Hkv, SegArgs s,
                                                                const float2* __restrict__ table) {
  const size_t x = (size_t)blockIdx.x * kThreads + threadIdx.x;  // (token, head, chunk pair)
  const int cp = (int)(x & 7);
  const size_t row = x >> 3;                                      // token * Hkv + head
  if (row >= (size_t)S * Hkv) return;
  const int t = (int)(row / Hkv);
  int lo = 0, hi = s.n_seg - 1;  // segment of token t: last p with start[p] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const uint16_t* src = k_in + row * D + 8 * cp;
  uint16_t* dst = k_out + row * D + 8 * cp;
  const uint4 A = *reinterpret_cast<const uint4*>(src);
  const uint4 B = *reinterpret_cast<const uint4*>(src + D / 2);
  if (s.rerot[lo] == 0) {  // already at its position
    *reinterpret_cast<uint4*>(dst) = A;
    *reinterpret_cast<uint4*>(dst + D / 2) = B;
    return;
  }
  const float2* cs = table + (size_t)lo * (D / 2) + 8 * cp;
  const uint32_t aw[4] = {A.x, A.y, A.z, A.w}, bw[4] = {B.x, B.y, B.z, B.w};
  uint32_t ya[4], yb[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x1a = bf16_lo(aw[w]), x1b = bf16_hi(aw[w]);
    const float x2a = bf16_lo(bw[w]), x2b = bf16_hi(bw[w]);
    const float2 c0 = cs[2 * w], c1 = cs[2 * w + 1];
    ya[w] = pack2(x1a * c0.x - x2a * c0.y, x1b * c1.x - x2b * c1.y);
    yb[w] = pack2(x2a * c0.x + x1a * c0.y, x2b * c1.x + x1b * c1.y);
  }
  *reinterpret_cast<uint4*>(dst) = make_uint4(ya[0], ya[1], ya[2], ya[3]);
  *reinterpret_cast<uint4*>(dst + D / 2) = make_uint4(yb[0], yb[1], yb[2], yb[3]);
}

}  // namespace

rbs_status launch_rerotate(const void* k_in, void* k_out, float2* table, int S, int Hkv,
                           const SegArgs& s, hipStream_t st) {
  const int nt = s.n_seg * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((nt + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     st, s, table);
  rbs_status r = launch_status();
  if (r != RBS_OK) return r;
  const size_t items = (size_t)S * Hkv * 8;
  hipLaunchKernelGGL(rope_rerotate_kernel, dim3((unsigned)((items + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, static_cast<const uint16_t*>(k_in),
                     static_cast<uint16_t*>(k_out), S, Hkv, s, table);
  return launch_status();
}

}  // namespace rbs
