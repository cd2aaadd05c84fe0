// Block statistics for dual-branch key-block selection.
//
// RBS-Attention explainer (techfordev), "The Standard Approach and Its Blind
// Spot": a key block is summarised by its centroid (mean key) and radius
// (largest key-to-centroid distance); "The Fix" scores blocks with a query q
// and ||q||_2. One workgroup handles one (KV head g, block b) and makes a
// single pass over HBM: the group's query rows of block b are summed into the
// representative query (one per group, and optionally one per query head for
// per-head selection), and the key tile stays in registers between the mean
// and the distance pass.
//
// Bound: HBM. Algorithmic bytes per (g, b): B*(G+1)*D*sizeof(T) read,
// (2*D + 2)*4 written.

#include "rbs_common.h"

namespace rbs {
namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec16;  // 16 bytes of T widened to floats
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const uint4& w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(const uint4& w, float* f) {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
};

// T: uint16_t (bf16 bits) or float. D: head dim. MAXV: key vectors (16 B) per
// thread, >= ceil(B * D * sizeof(T) / 16 / 256).
template <typename T, int D, int MAXV>
__global__ __launch_bounds__(kThreads) void block_stats_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int S, int Hq, int Hkv, int B,
    float* __restrict__ cen, float* __restrict__ rad, float* __restrict__ qrep,
    float* __restrict__ qnorm, float* __restrict__ qrep_h, float* __restrict__ qnorm_h) {
  constexpr int EPV = Vec16<T>::N;        // elements per 16-byte vector
  constexpr int KVEC = D / EPV;           // vectors per key row (divides 256)
  extern __shared__ float smem[];

  const int b = blockIdx.x;
  const int g = blockIdx.y;
  const int nb = gridDim.x;
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int t0 = b * B;
  const int L = min(B, S - t0);

  // ---------------- representative query: mean over L tokens x G heads ----
  const int VR = G * KVEC;                            // vectors per token row of the group
  // LDS: qred [qslots][EPV] | red [16] | kred [256][EPV] | cvec [D] | hsq [G D / 64]
  const int qslots = VR <= kThreads ? (kThreads / VR) * VR : VR;
  float* qred = smem;
  float* red = qred + qslots * EPV;
  float* kred = red + 16;
  float* cvec = kred + kThreads * EPV;
  float* hsq = cvec + D;  // per 64-element chunk of the per-head means: sum of squares
  {
    const int TP = VR <= kThreads ? kThreads / VR : 1;   // tokens per pass
    const int NV = VR <= kThreads ? 1 : (VR + kThreads - 1) / kThreads;
    const T* qg = q + ((size_t)t0 * Hq + (size_t)g * G) * D;
    const size_t row_stride = (size_t)Hq * D;
    for (int n = 0; n < NV; ++n) {
      int to, vi;
      if (NV == 1) { to = tid / VR; vi = tid % VR; } else { to = 0; vi = tid + n * kThreads; }
      float acc[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
      const bool active = (NV == 1) ? (tid < TP * VR) : (vi < VR);
      if (active) {
        const T* p = qg + (size_t)to * row_stride + (size_t)vi * EPV;
        const size_t step = (size_t)TP * row_stride;
        int tt = to;
#pragma unroll 32
        for (; tt < L; tt += TP) {
          // streamed once: non-temporal loads keep Q from displacing cached data
          const u32x4_t wv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
          const uint4 w = make_uint4(wv.x, wv.y, wv.z, wv.w);
          float f[EPV];
          Vec16<T>::widen(w, f);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[e] += f[e];
          p += step;
        }
        const int slot = (NV == 1) ? tid : vi;    // = to*VR + vi when NV == 1
#pragma unroll
        for (int e = 0; e < EPV; ++e) qred[slot * EPV + e] = acc[e];
      }
    }
  }
  __syncthreads();
  {
    const int TP = VR <= kThreads ? kThreads / VR : 1;
    float qd = 0.f;
    if (tid < D) {
      float s = 0.f;
      for (int to = 0; to < TP; ++to)
        for (int hh = 0; hh < G; ++hh) {
          const int slot = to * VR + hh * KVEC + tid / EPV;
          s += qred[slot * EPV + (tid % EPV)];
        }
      qd = s / (float)(G * L);
      if (qrep) qrep[((size_t)g * nb + b) * D + tid] = qd;
    }
    float sq = wave_sum(qd * qd);
    if ((tid & 63) == 0) red[tid >> 6] = sq;
    if (qrep_h) {
      // per query head hl of the group: the mean over the block's tokens; a
      // wave's 64 elements belong to one head (64 divides D)
      for (int x = tid; x < G * D; x += kThreads) {
        const int hl = x / D, d = x % D;
        float sh = 0.f;
        for (int to = 0; to < TP; ++to) sh += qred[(to * VR + hl * KVEC + d / EPV) * EPV + d % EPV];
        const float m = sh / (float)L;
        qrep_h[((size_t)(g * G + hl) * nb + b) * D + d] = m;
        const float w2 = wave_sum(m * m);
        if ((tid & 63) == 0) hsq[x >> 6] = w2;
      }
    }
  }
  __syncthreads();
  if (tid == 0 && qnorm) {
    float s = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) s += red[w];
    qnorm[(size_t)g * nb + b] = sqrtf(s);
  }
  if (qrep_h)
    for (int x = tid; x < G; x += kThreads) {
      float s2 = 0.f;
      for (int c = 0; c < D / 64; ++c) s2 += hsq[x * (D / 64) + c];
      qnorm_h[(size_t)(g * G + x) * nb + b] = sqrtf(s2);
    }

  // ---------------- key centroid and radius --------------------------------
  const int dv = tid % KVEC;                 // this thread's vector column
  const int tok0 = tid / KVEC;               // first token, then + 256/KVEC
  constexpr int TSTEP = kThreads / KVEC;
  uint4 kv[MAXV];
  float part[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) part[e] = 0.f;
  const T* kg = k + ((size_t)t0 * Hkv + g) * D + dv * EPV;
  const size_t krow = (size_t)Hkv * D;
#pragma unroll
  for (int n = 0; n < MAXV; ++n) {
    const int tok = tok0 + n * TSTEP;
    kv[n] = make_uint4(0u, 0u, 0u, 0u);
    if (tok < L) {
      kv[n] = *reinterpret_cast<const uint4*>(kg + (size_t)tok * krow);
      float f[EPV];
      Vec16<T>::widen(kv[n], f);
#pragma unroll
      for (int e = 0; e < EPV; ++e) part[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < EPV; ++e) kred[tid * EPV + e] = part[e];
  __syncthreads();
  if (tid < D) {
    const int col = tid / EPV, e = tid % EPV;
    float s = 0.f;
    for (int r = 0; r < TSTEP; ++r) s += kred[(r * KVEC + col) * EPV + e];
    const float c = s / (float)L;
    cvec[tid] = c;
    cen[((size_t)g * nb + b) * D + tid] = c;
  }
  __syncthreads();
  float cme[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) cme[e] = cvec[dv * EPV + e];
  float best = 0.f;
#pragma unroll
  for (int n = 0; n < MAXV; ++n) {
    const int tok = tok0 + n * TSTEP;
    float f[EPV];
    Vec16<T>::widen(kv[n], f);
    float d2 = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float dd = f[e] - cme[e];
      d2 = fmaf(dd, dd, d2);
    }
    // full squared distance of this token: sum over its KVEC consecutive lanes
#pragma unroll
    for (int o = 1; o < KVEC; o <<= 1) d2 += __shfl_xor(d2, o, kWave);
    if (tok < L) best = fmaxf(best, d2);
  }
  best = wave_max(best);
  if ((tid & 63) == 0) red[8 + (tid >> 6)] = best;
  __syncthreads();
  if (tid == 0) {
    float m = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) m = fmaxf(m, red[8 + w]);
    rad[(size_t)g * nb + b] = sqrtf(m);
  }
}

template <typename T, int D>
rbs_status launch_typed(const void* q, const void* k, int S, int Hq, int Hkv, int B, float* cen,
                        float* rad, float* qrep, float* qnorm, float* qrep_h, float* qnorm_h,
                        hipStream_t st) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int KVEC = D / EPV;
  const int nb = (S + B - 1) / B;
  const int need = (B * KVEC + kThreads - 1) / kThreads;
  dim3 grid(nb, Hkv);
  const int VR = (Hq / Hkv) * KVEC;
  const int qslots = VR <= kThreads ? (kThreads / VR) * VR : VR;
  const size_t shmem =
      ((size_t)qslots * EPV + 16 + kThreads * EPV + D + (Hq / Hkv) * (D / 64)) * sizeof(float);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), shmem, st, (const T*)q, (const T*)k, S, Hq,
                       Hkv, B, cen, rad, qrep, qnorm, qrep_h, qnorm_h);
    return launch_status();
  };
  if (need <= 2) return go(block_stats_kernel<T, D, 2>);
  if (need <= 4) return go(block_stats_kernel<T, D, 4>);
  if (need <= 8) return go(block_stats_kernel<T, D, 8>);
  if (need <= 16) return go(block_stats_kernel<T, D, 16>);
  return go(block_stats_kernel<T, D, 32>);
}

}  // namespace

rbs_status launch_block_stats(rbs_dtype dt, const void* q, const void* k, int S, int Hq, int Hkv,
                              int D, int B, float* cen, float* rad, float* qrep, float* qnorm,
                              float* qrep_h, float* qnorm_h, hipStream_t st) {
  if (dt == RBS_DT_BF16) {
    if (D == 64)
      return launch_typed<uint16_t, 64>(q, k, S, Hq, Hkv, B, cen, rad, qrep, qnorm, qrep_h, qnorm_h, st);
    return launch_typed<uint16_t, 128>(q, k, S, Hq, Hkv, B, cen, rad, qrep, qnorm, qrep_h, qnorm_h, st);
  }
  if (D == 64)
    return launch_typed<float, 64>(q, k, S, Hq, Hkv, B, cen, rad, qrep, qnorm, qrep_h, qnorm_h, st);
  return launch_typed<float, 128>(q, k, S, Hq, Hkv, B, cen, rad, qrep, qnorm, qrep_h, qnorm_h, st);
}

}  // namespace rbs
