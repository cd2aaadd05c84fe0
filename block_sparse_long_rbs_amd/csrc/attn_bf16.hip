// Block-sparse causal GQA attention, bf16 inputs, head dim 128, key tile =
// block = 128 tokens, on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Two tile iterators share one kernel body:
//  * CSR mode: the key blocks of row (g, i) come from the selection's CSR
//    lists (RBS-Attention explainer, "The Fix": the combined block mask runs
//    through a standard block-sparse attention).
//  * Segment mode (Block-attention page, sections 2.1-2.5): a query tile of a
//    non-final segment visits its own segment's key tiles up to the diagonal,
//    a query tile of the final segment visits every key tile up to the
//    diagonal; cached keys are rotated by their segment's RoPE offset once
//    their tile has landed in LDS.
//
// Work decomposition. One workgroup = 4 waves = one query head h and one
// query tile of 128 tokens; each wave owns 32 query rows; two workgroups
// share a CU so one's vector work overlaps the other's matrix work. Per key
// tile:
//   S^T = K Q^T    (A = K from LDS, B = Q held in registers)
//   online softmax in fp32, base 2, one query row per lane pair
//   O^T += V^T P^T (A = V^T read from LDS with the transposing load
//                   ds_read_b64_tr_b16, B = P straight from the S registers)
// Computing the transposed products leaves every lane holding one query row
// (lane % 32) in both the score and the output accumulators; lanes l and l^32
// share a row and combine through v_permlane32_swap. The running max is taken
// from the row's first tile and kept while no exponential exceeds 2^64 (seen
// through the tile's row sum), so the hot loop computes no per-tile max.
//
// Data movement. K and V tiles (32 KB each, 16-byte chunks XOR-swizzled per
// row) go from HBM straight into LDS with global_load_lds_dwordx4, issued as
// inline asm and awaited with explicit vector-memory counts: the next tile's
// K streams in during this tile's softmax and P.V, the next V during the next
// Q.K^T. The CSR row is staged in LDS. The heads of one GQA group run on the
// same XCD at neighbouring slots, so a K/V tile is fetched from HBM once and
// served from that XCD's L2 to the other heads.
//
// Bound: matrix cores. Algorithmic flops per (query row, key) pair: 4*D.

#include <math.h>

#include "rbs_common.h"

namespace rbs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr int D = 128;
constexpr int TILE = 128;            // keys per tile and query rows per workgroup
constexpr int kThreads = 256;
constexpr int ROWB = D * 2;          // bytes per K or V row in LDS

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

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
// byte offset) into LDS at lds_addr + 16*lane. Issued as inline asm so that
// the compiler does not treat it as a pending LDS write (it would otherwise
// wait for every in-flight tile before each LDS read); completion is awaited
// explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16-byte chunk swizzles: K rows are read 16 rows x one chunk per matrix
// fragment, V rows 4 rows x four chunks per transposing read.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

// DMA one 128 x 128 bf16 tile (tokens key0.., one KV head; src points at that
// head's token 0) into LDS. Each of the 4 waves issues 8 loads of 1 KB (4
// rows); lane l of a load lands at base + 16 l, so each lane fetches the
// logical chunk that the swizzle puts there. Rows past the sequence end
// repeat the last row (finite values; their scores are masked).
template <bool IS_V>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, size_t rs, int S,
                                         int key0, char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r4 = lane >> 4, pc = lane & 15;
  const uint32_t dst = lds_u32(lds) + wave * 8 * 1024;
  const int row0 = key0 + wave * 32;
  const uint32_t rsb = (uint32_t)rs * 2;  // bytes per token row
  if (row0 + 32 <= S) {
    const uint16_t* base = src + (size_t)row0 * rs;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int lc = IS_V ? (pc ^ (r4 << 2)) : (pc ^ (((it & 3) << 2) | r4));
      dma16(base + (size_t)(it * 4) * rs, r4 * rsb + lc * 16, dst + it * 1024);
    }
  } else {
    // ragged end: rows are clamped to S - 1, offsets taken from min(row0, S - 1)
    const int r0 = min(row0, S - 1);
    const uint16_t* cbase = src + (size_t)r0 * rs;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int lc = IS_V ? (pc ^ (r4 << 2)) : (pc ^ (((it & 3) << 2) | r4));
      const int tok = min(row0 + it * 4 + r4, S - 1);
      dma16(cbase, (uint32_t)(tok - r0) * rsb + lc * 16, dst + it * 1024);
    }
  }
}

// Rotate a landed K tile in place by one RoPE offset (rotate-half pairs
// (d, d + 64); cos/sin per frequency in `rope`). Thread tid takes chunk pair
// (8cp.., 64 + 8cp..) of rows tid/8 + 32 it, in the swizzled layout.
__device__ __forceinline__ void rotate_k_tile(char* Ks, const float2* rope) {
  const int tid = threadIdx.x;
  const int cp = tid & 7, rr = tid >> 3;
  float2 cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = rope[8 * cp + e];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = rr + 32 * it;
    const int sw = k_swz(row);
    uint4* pa = reinterpret_cast<uint4*>(Ks + row * ROWB + ((cp ^ sw) << 4));
    uint4* pb = reinterpret_cast<uint4*>(Ks + row * ROWB + (((cp + 8) ^ sw) << 4));
    const uint4 A = *pa, B = *pb;
    const uint32_t aw[4] = {A.x, A.y, A.z, A.w};
    const uint32_t bw[4] = {B.x, B.y, B.z, B.w};
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float x10 = bf16_lo(aw[w]), x11 = bf16_hi(aw[w]);
      const float x20 = bf16_lo(bw[w]), x21 = bf16_hi(bw[w]);
      const float2 c0 = cs[2 * w], c1 = cs[2 * w + 1];
      ya[w] = cvt_pk_bf16(x10 * c0.x - x20 * c0.y, x11 * c1.x - x21 * c1.y);
      yb[w] = cvt_pk_bf16(x20 * c0.x + x10 * c0.y, x21 * c1.x + x11 * c1.y);
    }
    *pa = make_uint4(ya[0], ya[1], ya[2], ya[3]);
    *pb = make_uint4(yb[0], yb[1], yb[2], yb[3]);
  }
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
// heads of one (KV head, query tile) unit get neighbouring slots on one XCD.
struct Unit {
  int g, h, qt;
};
__device__ __forceinline__ bool decode_unit(int G, int Hkv, int n_qt, int qt_begin, Unit& u) {
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int slot = x >> 3;
  const int hg = slot % G;
  const int uo = (slot / G) * 8 + xcd;
  const int n_units = Hkv * (n_qt - qt_begin);
  if (uo >= n_units) return false;
  u.qt = n_qt - 1 - uo / Hkv;
  u.g = uo % Hkv;
  u.h = u.g * G + hg;
  return true;
}

__device__ __forceinline__ void load_q(const uint16_t* __restrict__ Q, int S, int Hq, int h,
                                       int qt, bf16x8_t* qf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = qt * TILE + wave * 32 + (lane & 31);
  const int hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (t < S) u = *reinterpret_cast<const uint4*>(Q + ((size_t)t * Hq + h) * D + 16 * c + 8 * hh);
    qf[c] = as_bf16x8(u);
  }
}

__device__ __forceinline__ void store_out(uint16_t* __restrict__ O, float* __restrict__ lse, int S,
                                          int Hq, int h, int qt, int row_begin, const f32x16_t* o,
                                          float m_run, float l_run) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  const int t = qt * TILE + wave * 32 + m32;
  const float l = pair_sum(l_run);
  if (t >= S || t < row_begin) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = O + ((size_t)t * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * hh;
      const uint2 v = make_uint2(cvt_pk_bf16(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv),
                                 cvt_pk_bf16(o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv));
      *reinterpret_cast<uint2*>(orow + d) = v;
    }
  if (lse && hh == 0)
    lse[(size_t)h * S + t] = l > 0.f ? (m_run + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
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

// Key tiles of one unit in segment mode: jlo..qt.
struct SegTiles {
  int qt;
  __device__ int next_after(int j) const { return j < qt ? j + 1 : -1; }
};

__device__ __forceinline__ int segment_of_tile(const SegArgs& s, int tile) {
  const int tok = tile * TILE;
  int lo = 0, hi = s.n_seg - 1;  // last p with start[p] <= tok
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.start[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool SEG>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a,
                                                                const int32_t* __restrict__ row_ptr,
                                                                const int32_t* __restrict__ col_idx,
                                                                SegArgs seg, float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char Ks[TILE * ROWB];
  __shared__ __attribute__((aligned(1024))) char Vs[TILE * ROWB];
  __shared__ int lst[SEG ? 1 : kThreads];
  __shared__ float2 rope[SEG ? D / 2 : 1];
  const int G = a.Hq / a.Hkv;
  const int nq = (a.S + TILE - 1) / TILE;
  Unit u;
  if (!decode_unit(G, a.Hkv, nq, SEG ? seg.q_row_begin / TILE : 0, u)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  const size_t rs = (size_t)a.Hkv * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (size_t)u.g * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + (size_t)u.g * D;

  // tile iteration state
  CsrTiles csr{col_idx, 0, 0, 0, u.qt, lst};
  int jseg_lo = 0;
  if (!SEG) {
    const int row = u.g * nq + u.qt;
    csr.e = row_ptr[row];
    csr.e1 = row_ptr[row + 1];
    csr.cb = csr.e;
    lst[threadIdx.x] = (csr.e + (int)threadIdx.x < csr.e1) ? col_idx[csr.e + threadIdx.x] : -1;
    lds_barrier();
  } else {
    const int p = segment_of_tile(seg, u.qt);
    jseg_lo = (p == seg.n_seg - 1) ? 0 : seg.start[p] / TILE;
  }
  SegTiles segt{u.qt};
  // Segment mode: cached keys of a segment with a nonzero offset are rotated
  // in LDS once their tile has landed; the cos/sin table follows the offset.
  int cur_off = 0, pj = 0;
  auto offset_of = [&](int j) {
    while (pj + 1 < seg.n_seg && seg.start[pj + 1] <= j * TILE) ++pj;
    return seg.rerot[pj];
  };

  bf16x8_t qf[8];
  load_q(static_cast<const uint16_t*>(a.q), a.S, a.Hq, u.h, u.qt, qf);
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16_t){};
  float m_run = 0.f, l_run = 0.f;
  bool first = true;

  // per-lane LDS offsets
  const int kx = m32 & 15;
  const int sr = lane & 15, half = (lane >> 4) & 1, y = sr >> 2;
  const int v_lane = (4 * hh + y) * ROWB + (sr & 1) * 8;
  const int vx = 2 * half + ((sr & 3) >> 1);
  const int qq = wave * 32 + m32;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  int j = SEG ? jseg_lo : csr.next(csr.e);
  wait_vmcnt<0>();  // Q fragments and the CSR chunk are in registers before any tile DMA
  if (j >= 0) {
    if (SEG) pj = segment_of_tile(seg, j);
    dma_tile<false>(Kg, rs, a.S, j * TILE, Ks);
    dma_tile<true>(Vg, rs, a.S, j * TILE, Vs);
  }
  while (j >= 0) {
    const int jn = SEG ? segt.next_after(j) : csr.next(csr.e + 1);
    wait_vmcnt<8>();  // K(j) has landed (V(j) may still be in flight)
    lds_barrier();
    if (SEG) {
      const int off = offset_of(j);
      if (off != 0) {
        if (off != cur_off) {
          if (threadIdx.x < D / 2) {
            const double inv = pow((double)seg.theta, -2.0 * (double)threadIdx.x / (double)D);
            double sn, cs;
            sincos((double)off * inv, &sn, &cs);
            rope[threadIdx.x] = make_float2((float)cs, (float)sn);
          }
          lds_barrier();
          cur_off = off;
        }
        rotate_k_tile(Ks, rope);
        lds_barrier();
      }
    }
    // ---- S^T = K Q^T (four independent accumulators in turn) ----
    // Wave priority: matrix phases win issue over the other workgroup's
    // softmax on the same SIMD (P.V highest, so a tile's output accumulation
    // is not held up behind the next tile's scores).
    __builtin_amdgcn_s_setprio(1);
    f32x16_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) s[kb] = (f32x16_t){};
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint4 af = *reinterpret_cast<const uint4*>(Ks + (kb * 32 + m32) * ROWB +
                                                         (((2 * c + hh) ^ kx) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), qf[c], s[kb], 0, 0, 0);
      }
    // keep up to 8 fragment reads in flight ahead of the matrix instructions
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();  // every wave is done with Ks
    if (jn >= 0) dma_tile<false>(Kg, rs, a.S, jn * TILE, Ks);
    // ---- online softmax (base 2) ----
    if (j == u.qt) {
      // causal mask inside the diagonal tile; t is made opaque so that the
      // per-element predicates are not hoisted out of the tile loop
      int t = qq - 4 * hh;
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > t) s[kb][r] = -INFINITY;
    }
    // The running max comes from the row's first tile; later tiles keep it
    // as long as no exponential exceeds 2^64 (seen through the row sum, which
    // also catches inf), else the max is raised and O rescaled (rare path).
    auto tile_max = [&]() {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      return pair_max(mx) * scale_log2;
    };
    if (first) {
      m_run = tile_max();
      first = false;
    }
    uint32_t pk[4][8];
    auto exps = [&]() {
      const float neg = -m_run;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, neg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], scale_log2, neg));
          const uint32_t w = cvt_pk_bf16(p0, p1);
          pk[kb][r >> 1] = w;
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, ls, false);
        }
      return ls;
    };
    float ls = exps();
    if (__ballot(!(ls <= 0x1p64f))) {
      const float m_new = fmaxf(m_run, tile_max());
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      ls = exps();
    }
    l_run += ls;
    if (jn >= 0) wait_vmcnt<8>(); else wait_vmcnt<0>();  // V(j) has landed
    lds_barrier();
    // ---- O^T += V^T P^T (four independent accumulators in turn) ----
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const char* vb = Vs + v_lane + ((((db ^ y) << 2) + vx) << 4) + c * 16 * ROWB;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)vb);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vb + 8 * ROWB));
        const uint4 av = make_uint4((uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                                    (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                                    (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                                    (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
        const int kb = c >> 1, base = (c & 1) * 4;
        const uint4 b = make_uint4(pk[kb][base], pk[kb][base + 1], pk[kb][base + 2],
                                   pk[kb][base + 3]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(b), o[db], 0, 0, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();  // every wave is done with Vs
    if (jn >= 0) dma_tile<true>(Vg, rs, a.S, jn * TILE, Vs);
    j = jn;
  }
  store_out(static_cast<uint16_t*>(a.out), a.lse, a.S, a.Hq, u.h, u.qt,
            SEG ? seg.q_row_begin : 0, o, m_run, l_run);
}

inline int attn_grid(int Hq, int Hkv, int n_qt) {
  const int G = Hq / Hkv;
  const int units = Hkv * n_qt;
  return ((units + 7) / 8) * 8 * G;
}

}  // namespace

rbs_status launch_attn_bf16_csr(const AttnArgs& a, hipStream_t st) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int nq = (a.S + TILE - 1) / TILE;
  SegArgs none;
  none.n_seg = 0;
  none.q_row_begin = 0;
  none.theta = 0.f;
  hipLaunchKernelGGL(attn_bf16_kernel<false>, dim3(attn_grid(a.Hq, a.Hkv, nq)), dim3(kThreads), 0,
                     st, a, a.row_ptr, a.col_idx, none, scale_log2);
  return launch_status();
}

rbs_status launch_attn_segments(const AttnArgs& a, const SegArgs& s, hipStream_t st) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int nq = (a.S + TILE - 1) / TILE;
  const int n_qt = nq - s.q_row_begin / TILE;
  if (n_qt <= 0) return RBS_OK;
  hipLaunchKernelGGL(attn_bf16_kernel<true>, dim3(attn_grid(a.Hq, a.Hkv, n_qt)), dim3(kThreads),
                     0, st, a, nullptr, nullptr, s, scale_log2);
  return launch_status();
}

}  // namespace rbs
