// Pieces shared by the matrix-core attention kernels (bf16 and fp8 inputs):
// one workgroup = 4 waves = one query head and a 128-row query tile, each
// wave owning 32 query rows; 128-key tiles; transposed products so that a
// lane holds one query row in both the score and the output accumulators of
// a 32x32 MFMA block (lanes l and l^32 share a row).
#pragma once

#include <math.h>

#include "rbs_common.h"

namespace rbs {
namespace tiles {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int D = 128;
constexpr int TILE = 128;            // keys per tile and query rows per workgroup
constexpr int kThreads = 256;
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Workgroup barrier for LDS hand-offs: this wave's LDS reads/writes are
// complete, then s_barrier. No memory fence, so tile DMAs (vector-memory
// writes into LDS) stay in flight across it; their completion is awaited
// explicitly with wait_vmcnt before the barrier that publishes them.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 16-byte-per-lane DMA from global memory (uniform base + per-lane 32-bit
// byte offset) into LDS at lds_addr + 16*lane (the LDS address goes in M0,
// which the compiler loads for the statement). Issued as inline asm so that
// the compiler does not treat it as a pending LDS write (it would otherwise
// wait for every in-flight tile before each LDS read); completion is awaited
// explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Lanes l and l^32 hold the same query row: combine their values.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work unit decode: XCD-aware, heaviest (highest) query tiles first. The G
// heads (times the key-range chunks, if any) of one (KV head, query tile)
// unit get neighbouring slots on one XCD.
struct Unit {
  int g, h, qt, c;
};
__device__ __forceinline__ bool decode_unit(int x, int G, int Hkv, int qt_lo, int qt_hi, int C,
                                            Unit& u) {
  const int per = G * C;
  const int xcd = x & 7;
  const int slot = x >> 3;
  const int hg = slot % per;
  const int uo = (slot / per) * 8 + xcd;
  const int n_units = Hkv * (qt_hi - qt_lo);
  if (uo >= n_units) return false;
  u.qt = qt_hi - 1 - uo / Hkv;
  u.g = uo % Hkv;
  u.h = u.g * G + hg % G;
  u.c = hg / G;
  return true;
}

// Normalised output of one query tile (bf16, O / l times out_scale) and the
// row's log-sum-exp (natural log; -inf for a row that saw no key), through
// LDS (buf: 32 KB, 16-byte aligned, free when called; `wave` = the wave's
// 32-row slot in the tile): each lane writes its
// 4-value groups into its row (16-byte chunks swizzled by row), then each
// wave reads back its own 32 rows as whole 16-byte chunks, so that the stores
// to O cover 256 contiguous bytes per row instead of 8 bytes of 64 different
// rows. Only the wave's own rows are touched: no workgroup barrier.
__device__ __forceinline__ void store_out_lds(uint16_t* __restrict__ O, float* __restrict__ lse,
                                              int S, int Hq, int h, int qt, int row_begin,
                                              const f32x16_t* o, float m_run, float l_run,
                                              float out_scale, char* buf, int wave) {
  const int lane = threadIdx.x & 63;
  const int m32 = lane & 31, hh = lane >> 5;
  const float l = pair_sum(l_run);
  const float inv = l > 0.f ? out_scale / l : 0.f;
  constexpr int kRowBytes = D * 2;  // one bf16 output row
  {
    const int r = wave * 32 + m32;
    char* rowp = buf + r * kRowBytes;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int chunk = db * 4 + rg;  // 8 head dims from db * 32 + 8 rg; this lane's 4 at + 4 hh
        const uint2 v = make_uint2(cvt_pk_bf16(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv),
                                   cvt_pk_bf16(o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv));
        *reinterpret_cast<uint2*>(rowp + ((chunk ^ (r & 15)) << 4) + 8 * hh) = v;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const int t_lse = qt * TILE + wave * 32 + m32;
  if (lse && hh == 0 && t_lse < S && t_lse >= row_begin)
    lse[(size_t)h * S + t_lse] = l > 0.f ? (m_run + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = wave * 32 + it * 4 + (lane >> 4), chunk = lane & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(buf + r * kRowBytes + ((chunk ^ (r & 15)) << 4));
    const int t = qt * TILE + r;
    if (t < S && t >= row_begin)
      *reinterpret_cast<uint4*>(O + ((size_t)t * Hq + h) * D + chunk * 8) = v;
  }
}

// Key tiles of one unit in CSR mode: the row's block list, staged in LDS 256
// entries at a time (a vector load inside the tile loop would make every wait
// drain the in-flight tile DMAs); entries outside 0..qt are skipped.
struct CsrTiles {
  const int32_t* col_idx;
  int e, e1, cb, qt;
  int* lst;
  __device__ int next(int e_from) {
    for (e = e_from; e < e1; ++e) {
      if (e - cb >= kThreads) {  // refill: every wave reaches this point together
        lds_barrier();
        cb = e;
        lst[threadIdx.x] = (cb + (int)threadIdx.x < e1) ? col_idx[cb + threadIdx.x] : -1;
        lds_barrier();
      }
      const int j = lst[e - cb];
      if (j >= 0 && j <= qt) return j;
    }
    return -1;
  }
};


inline int attn_grid(int Hq, int Hkv, int n_qt, int chunks) {
  const int G = Hq / Hkv;
  const int units = Hkv * (n_qt > 0 ? n_qt : 0);
  return ((units + 7) / 8) * 8 * G * chunks;
}

}  // namespace tiles
}  // namespace rbs
