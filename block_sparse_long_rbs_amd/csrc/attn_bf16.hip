// Block-sparse causal GQA attention, bf16 inputs, head dim 128, key tile =
// block = 128 tokens, on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Two tile iterators share one core:
//  * CSR mode: the key blocks of row (g, i) come from the selection's CSR
//    lists (RBS-Attention explainer, "The Fix": the combined mask runs through
//    a standard block-sparse attention).
//  * Segment mode (Block-attention, sections 2.1-2.5): a query tile of a
//    non-final segment visits its own segment's key tiles up to the diagonal,
//    a query tile of the final segment visits every key tile up to the
//    diagonal; cached keys are rotated by their segment's RoPE offset while
//    they are staged into LDS.
//
// Work decomposition. One workgroup = 4 waves = one query head h and one
// query tile of 128 tokens; each wave owns 32 query rows. Per key tile:
//   S^T = K Q^T   (A = K from LDS, B = Q held in registers)
//   online softmax in fp32, base 2, per query row (one row per lane pair)
//   O^T += V^T P^T (A = V^T from LDS, B = P straight from the S registers)
// Computing the transposed products leaves every lane holding one query row
// (lane % 32) in both the score and the output accumulators, so the row max,
// the rescale and the final normalisation need only one cross-half exchange.
// LDS per workgroup: K tile 32 KB (16-byte chunks XOR-swizzled by row) and
// V^T tile 32 KB (8-byte units XOR-swizzled by d), single-buffered; two
// workgroups per CU overlap one's staging with the other's matrix work.
// The heads of one GQA group run on the same XCD at neighbouring slots, so a
// K/V tile is fetched from HBM once and served from that XCD's L2.
//
// Bound: matrix cores. Algorithmic flops per (query row, key) pair: 4*D.

#include <math.h>

#include "rbs_common.h"

namespace rbs {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int TILE = 128;            // keys per tile and query rows per workgroup
constexpr int kThreads = 256;
constexpr int ROWB = D * 2;          // bytes per K row / V^T row in LDS

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Work unit decode: XCD-aware, heaviest (highest) query tiles first.
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

// Stage K tile (rows j*128..) of KV head g into LDS, optionally rotating by a
// cos/sin table (64 frequencies), and V tile transposed.
template <bool ROTATE>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V, int S, int Hkv, int g,
                                           int j, char* Ks, char* Vt, const float2* rope) {
  const int tid = threadIdx.x;
  const size_t rs = (size_t)Hkv * D;  // elements between token rows
  const int key0 = j * TILE;
  // K: chunk pair cp (d 8cp..8cp+7 and 64+8cp..), rows rr + 32*it
  {
    const int cp = tid & 7, rr = tid >> 3;
    uint4 lo[4], hi[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = rr + 32 * it;
      const int tok = key0 + row;
      if (tok < S) {
        const uint16_t* p = K + (size_t)tok * rs + (size_t)g * D + 8 * cp;
        lo[it] = *reinterpret_cast<const uint4*>(p);
        hi[it] = *reinterpret_cast<const uint4*>(p + 64);
      } else {
        lo[it] = make_uint4(0, 0, 0, 0);
        hi[it] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int row = rr + 32 * it;
      uint4 a = lo[it], b = hi[it];
      if (ROTATE) {
        uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float2 cs0 = rope[8 * cp + 2 * w], cs1 = rope[8 * cp + 2 * w + 1];
          const float x10 = bf16_lo(aw[w]), x11 = bf16_hi(aw[w]);
          const float x20 = bf16_lo(bw[w]), x21 = bf16_hi(bw[w]);
          const float y10 = x10 * cs0.x - x20 * cs0.y, y20 = x20 * cs0.x + x10 * cs0.y;
          const float y11 = x11 * cs1.x - x21 * cs1.y, y21 = x21 * cs1.x + x11 * cs1.y;
          aw[w] = pack_bf16x2(y10, y11);
          bw[w] = pack_bf16x2(y20, y21);
        }
        a = make_uint4(aw[0], aw[1], aw[2], aw[3]);
        b = make_uint4(bw[0], bw[1], bw[2], bw[3]);
      }
      const int sw = row & 15;
      *reinterpret_cast<uint4*>(Ks + row * ROWB + ((cp ^ sw) << 4)) = a;
      *reinterpret_cast<uint4*>(Ks + row * ROWB + (((cp + 8) ^ sw) << 4)) = b;
    }
  }
  // V^T: d-octet od, key quads kq and kq + 16
  {
    const int od = tid & 15, kqa = tid >> 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kq = kqa + 16 * half;
      uint4 r[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int tok = key0 + 4 * kq + x;
        r[x] = tok < S ? *reinterpret_cast<const uint4*>(V + (size_t)tok * rs + (size_t)g * D + 8 * od)
                       : make_uint4(0, 0, 0, 0);
      }
      const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
      const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
      const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
      const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) ? 16 : 0;
        const int wi = e >> 1;
        const uint32_t k0 = (w0[wi] >> sh) & 0xFFFFu, k1 = (w1[wi] >> sh) & 0xFFFFu;
        const uint32_t k2 = (w2[wi] >> sh) & 0xFFFFu, k3 = (w3[wi] >> sh) & 0xFFFFu;
        const int d = 8 * od + e;
        uint2 val = make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
        *reinterpret_cast<uint2*>(Vt + d * ROWB + ((kq ^ (d & 31)) << 3)) = val;
      }
    }
  }
}

struct Softmax {
  float m;   // running max (log2 units), same in both lane halves
  float l;   // this lane's partial sum
};

// One key tile of work for this wave.
__device__ __forceinline__ void tile_compute(const char* Ks, const char* Vt, const bf16x8_t* qf,
                                             f32x16_t* o, Softmax& sm, float scale_log2,
                                             bool diag) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  f32x16_t s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = (f32x16_t){};
    const char* rowp = Ks + (kb * 32 + m32) * ROWB;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(rowp + (((2 * c + hh) ^ (m32 & 15)) << 4));
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[c], s[kb], 0, 0, 0);
    }
  }
  // scale, causal mask on the diagonal tile, row max
  const int qq = wave * 32 + m32;
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[kb][r] * scale_log2;
      if (diag) {
        const int kk = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (kk > qq) x = -INFINITY;
      }
      s[kb][r] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mnew = fmaxf(sm.m, mx);
  const float alpha = __builtin_amdgcn_exp2f(sm.m - mnew);
  sm.m = mnew;
  float lsum = 0.f;
  uint32_t pk[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s[kb][r] - mnew);
      const float p1 = __builtin_amdgcn_exp2f(s[kb][r + 1] - mnew);
      lsum += p0 + p1;
      pk[kb][r >> 1] = pack_bf16x2(p0, p1);
    }
  sm.l = sm.l * alpha + lsum;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  // O^T += V^T P^T
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + m32;
    const char* rowp = Vt + d * ROWB;
    const int sw = d & 31;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint2 lo = *reinterpret_cast<const uint2*>(rowp + (((4 * c + hh) ^ sw) << 3));
      const uint2 hi = *reinterpret_cast<const uint2*>(rowp + (((4 * c + 2 + hh) ^ sw) << 3));
      const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
      const int kb = c >> 1, base = (c & 1) * 4;
      const uint4 b = make_uint4(pk[kb][base], pk[kb][base + 1], pk[kb][base + 2], pk[kb][base + 3]);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), o[db], 0, 0, 0);
    }
  }
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
                                          const Softmax& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  const int t = qt * TILE + wave * 32 + m32;
  const float l = sm.l + __shfl_xor(sm.l, 32, 64);
  if (t >= S || t < row_begin) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = O + ((size_t)t * Hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * hh;
      const uint2 v = make_uint2(pack_bf16x2(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv),
                                 pack_bf16x2(o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv));
      *reinterpret_cast<uint2*>(orow + d) = v;
    }
  if (lse && hh == 0)
    lse[(size_t)h * S + t] = l > 0.f ? (sm.m + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

__global__ __launch_bounds__(kThreads, 2) void attn_csr_bf16_kernel(AttnArgs a, float scale_log2) {
  __shared__ __attribute__((aligned(16))) char Ks[TILE * ROWB];
  __shared__ __attribute__((aligned(16))) char Vt[D * ROWB];
  const int G = a.Hq / a.Hkv;
  const int nq = (a.S + TILE - 1) / TILE;
  Unit u;
  if (!decode_unit(G, a.Hkv, nq, 0, u)) return;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  bf16x8_t qf[8];
  load_q(Q, a.S, a.Hq, u.h, u.qt, qf);
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16_t){};
  Softmax sm{-1e30f, 0.f};
  const int row = u.g * nq + u.qt;
  const int e0 = a.row_ptr[row], e1 = a.row_ptr[row + 1];
  for (int e = e0; e < e1; ++e) {
    const int j = a.col_idx[e];
    if (j < 0 || j > u.qt) continue;
    __syncthreads();
    stage_tile<false>(K, V, a.S, a.Hkv, u.g, j, Ks, Vt, nullptr);
    __syncthreads();
    tile_compute(Ks, Vt, qf, o, sm, scale_log2, j == u.qt);
  }
  store_out(static_cast<uint16_t*>(a.out), a.lse, a.S, a.Hq, u.h, u.qt, 0, o, sm);
}

// ---------------------------------------------------------------------------
// CSR core, version 2: K and V tiles go straight from global memory into
// swizzled LDS with global_load_lds_dwordx4 (no staging registers), V^T
// fragments are read with the transposing LDS load ds_read_b64_tr_b16, and the
// K and V buffers are refilled separately: the next tile's K streams in
// during this tile's softmax and P.V, the next V during the next Q.K^T.

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// 16-byte chunk swizzles: K rows are read 16 rows x one chunk per MFMA
// fragment, V rows 4 rows x four chunks per transposing read.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

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

// DMA one 128 x 128 bf16 tile (tokens key0.., one KV head; src already points
// at that head) into LDS. Each of the 4 waves issues 8 loads of 1 KB (4 rows);
// lane l of a load lands at base + 16 l, so each lane fetches the logical
// chunk that the swizzle puts there. Rows past the sequence end repeat the
// last row (finite values; their scores are masked).
// One 16-byte-per-lane DMA from global memory into LDS at lds_addr + 16*lane.
// Issued as inline asm so that the compiler does not treat it as a pending
// LDS write (it would otherwise wait for every in-flight tile before each LDS
// read); completion is awaited explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

template <bool IS_V>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, size_t rs, int S,
                                         int key0, char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r4 = lane >> 4, pc = lane & 15;
  const uint32_t dst = lds_u32(lds) + wave * 8 * 1024;
  const int row0 = key0 + wave * 32;
  if (row0 + 32 <= S) {
    // whole 32-row slice present: scalar row base + per-lane offset
    const uint16_t* base = src + (size_t)row0 * rs;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int lc = IS_V ? (pc ^ (r4 << 2)) : (pc ^ (((it & 3) << 2) | r4));
      dma16(base + (size_t)(it * 4) * rs + (r4 * rs + lc * 8), dst + it * 1024);
    }
  } else {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int lc = IS_V ? (pc ^ (r4 << 2)) : (pc ^ (((it & 3) << 2) | r4));
      const int tok = min(row0 + it * 4 + r4, S - 1);
      dma16(src + (size_t)tok * rs + lc * 8, dst + it * 1024);
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_csr_bf16_v2_kernel(
    AttnArgs a, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    float scale_log2) {
  __shared__ __attribute__((aligned(1024))) char Ks[TILE * ROWB];
  __shared__ __attribute__((aligned(1024))) char Vs[TILE * ROWB];
  const int G = a.Hq / a.Hkv;
  const int nq = (a.S + TILE - 1) / TILE;
  Unit u;
  if (!decode_unit(G, a.Hkv, nq, 0, u)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  const size_t rs = (size_t)a.Hkv * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (size_t)u.g * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + (size_t)u.g * D;

  // CSR row, staged through LDS 256 entries at a time (a vector load inside the
  // tile loop would make every wait drain the in-flight tile DMAs)
  __shared__ int lst[kThreads];
  const int row = u.g * nq + u.qt;
  const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
  int cb = e0;
  lst[threadIdx.x] = (e0 + (int)threadIdx.x < e1) ? col_idx[e0 + threadIdx.x] : -1;
  lds_barrier();
  auto next_valid = [&](int e, int& j) {
    for (; e < e1; ++e) {
      if (e - cb >= kThreads) {  // refill: every wave reaches this point together
        lds_barrier();
        cb = e;
        lst[threadIdx.x] = (cb + (int)threadIdx.x < e1) ? col_idx[cb + threadIdx.x] : -1;
        lds_barrier();
      }
      j = lst[e - cb];
      if (j >= 0 && j <= u.qt) return e;
    }
    j = -1;
    return e1;
  };

  bf16x8_t qf[8];
  load_q(static_cast<const uint16_t*>(a.q), a.S, a.Hq, u.h, u.qt, qf);
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16_t){};
  float m_run = -1e30f, l_run = 0.f;

  // per-lane LDS offsets
  const int kx = m32 & 15;
  const int sr = lane & 15, half = (lane >> 4) & 1, y = sr >> 2;
  const int v_lane = (4 * hh + y) * ROWB + (sr & 1) * 8;
  const int vx = 2 * half + ((sr & 3) >> 1);
  const int qq = wave * 32 + m32;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  int j;
  int e = next_valid(e0, j);
  wait_vmcnt<0>();  // Q fragments and the CSR chunk are in registers before any tile DMA
  if (e < e1) {
    dma_tile<false>(Kg, rs, a.S, j * TILE, Ks);
    dma_tile<true>(Vg, rs, a.S, j * TILE, Vs);
  }
  while (e < e1) {
    int jn;
    const int en = next_valid(e + 1, jn);
    wait_vmcnt<8>();  // K(j) has landed (V(j) may still be in flight)
    lds_barrier();
    // ---- S^T = K Q^T ----
    f32x16_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const char* rowp = Ks + (kb * 32 + m32) * ROWB;
      s[kb] = (f32x16_t){};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 af = *reinterpret_cast<const uint4*>(rowp + (((2 * c + hh) ^ kx) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), qf[c], s[kb], 0, 0, 0);
      }
    }
    // keep up to 8 fragment reads in flight ahead of the matrix instructions
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    lds_barrier();  // every wave is done with Ks
    if (jn >= 0) dma_tile<false>(Kg, rs, a.S, jn * TILE, Ks);
    // ---- online softmax (base 2), lazy rescale by at most 2^8 ----
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
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mt = mx * scale_log2;
    const bool grow = mt > m_run + 8.f;
    if (__ballot(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
      m_run = grow ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    const float neg = -m_run;
    uint32_t pk[4][8];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, neg));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], scale_log2, neg));
        const uint32_t w = cvt_pk_bf16(p0, p1);
        pk[kb][r >> 1] = w;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, l_run,
                                                false);
      }
    if (jn >= 0) wait_vmcnt<8>(); else wait_vmcnt<0>();  // V(j) has landed
    lds_barrier();
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const char* vb = Vs + v_lane + ((((db ^ y) << 2) + vx) << 4);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(vb + c * 16 * ROWB));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(vb + c * 16 * ROWB + 8 * ROWB));
        const uint4 av = make_uint4(
            (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
            (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
            (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
            (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
        const int kb = c >> 1, base = (c & 1) * 4;
        const uint4 b = make_uint4(pk[kb][base], pk[kb][base + 1], pk[kb][base + 2],
                                   pk[kb][base + 3]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(b), o[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    lds_barrier();  // every wave is done with Vs
    if (jn >= 0) dma_tile<true>(Vg, rs, a.S, jn * TILE, Vs);
    e = en;
    j = jn;
  }
  Softmax sm{m_run, l_run};
  store_out(static_cast<uint16_t*>(a.out), a.lse, a.S, a.Hq, u.h, u.qt, 0, o, sm);
}

__device__ __forceinline__ int segment_of_tile(const SegArgs& s, int tile) {
  const int tok = tile * TILE;
  int lo = 0, hi = s.n_seg - 1;  // last p with start[p] <= tok
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.start[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads, 2) void attn_seg_bf16_kernel(AttnArgs a, SegArgs s,
                                                                    float scale_log2) {
  __shared__ __attribute__((aligned(16))) char Ks[TILE * ROWB];
  __shared__ __attribute__((aligned(16))) char Vt[D * ROWB];
  __shared__ float2 rope[D / 2];
  const int G = a.Hq / a.Hkv;
  const int nq = (a.S + TILE - 1) / TILE;
  Unit u;
  if (!decode_unit(G, a.Hkv, nq, s.q_row_begin / TILE, u)) return;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* K = static_cast<const uint16_t*>(a.k);
  const uint16_t* V = static_cast<const uint16_t*>(a.v);
  bf16x8_t qf[8];
  load_q(Q, a.S, a.Hq, u.h, u.qt, qf);
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16_t){};
  Softmax sm{-1e30f, 0.f};
  const int p = segment_of_tile(s, u.qt);
  const int jlo = (p == s.n_seg - 1) ? 0 : s.start[p] / TILE;
  int cur_off = -1;
  int pj = segment_of_tile(s, jlo);
  for (int j = jlo; j <= u.qt; ++j) {
    while (pj + 1 < s.n_seg && s.start[pj + 1] <= j * TILE) ++pj;
    const int off = s.rerot[pj];
    __syncthreads();
    if (off != cur_off) {
      if (threadIdx.x < D / 2) {
        const double inv = pow((double)s.theta, -2.0 * (double)threadIdx.x / (double)D);
        double sn, cs;
        sincos((double)off * inv, &sn, &cs);
        rope[threadIdx.x] = make_float2((float)cs, (float)sn);
      }
      __syncthreads();
      cur_off = off;
    }
    stage_tile<true>(K, V, a.S, a.Hkv, u.g, j, Ks, Vt, rope);
    __syncthreads();
    tile_compute(Ks, Vt, qf, o, sm, scale_log2, j == u.qt);
  }
  store_out(static_cast<uint16_t*>(a.out), a.lse, a.S, a.Hq, u.h, u.qt, s.q_row_begin, o, sm);
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
  hipLaunchKernelGGL(attn_csr_bf16_v2_kernel, dim3(attn_grid(a.Hq, a.Hkv, nq)), dim3(kThreads), 0,
                     st, a, a.row_ptr, a.col_idx, scale_log2);
  return launch_status();
}

rbs_status launch_attn_segments(const AttnArgs& a, const SegArgs& s, hipStream_t st) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int nq = (a.S + TILE - 1) / TILE;
  const int n_qt = nq - s.q_row_begin / TILE;
  if (n_qt <= 0) return RBS_OK;
  hipLaunchKernelGGL(attn_seg_bf16_kernel, dim3(attn_grid(a.Hq, a.Hkv, n_qt)), dim3(kThreads), 0,
                     st, a, s, scale_log2);
  return launch_status();
}

}  // namespace rbs
