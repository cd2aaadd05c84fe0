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
//    diagonal (the keys arrive already re-encoded, see rope.hip). The final
//    segment's long rows can be cut into key-range chunks whose partial
//    results attn_combine_kernel merges.
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
// served from that XCD's L2 to the other heads. In segment mode the Q tile
// also comes by DMA (through Vs, free until the first V tile), so it lands in
// the same memory round trip as the first K tile. The normalised output tile
// goes through LDS so that each row is written as 256 contiguous bytes.
//
// Bound: matrix cores. Algorithmic flops per (query row, key) pair: 4*D.

#include "attn_tiles.h"

namespace rbs {
namespace {

using namespace tiles;

constexpr int ROWB = D * 2;          // bytes per K or V row in LDS

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// 16-byte chunk swizzles in LDS: chunk c of K row r sits at slot c ^ (r & 15)
// (fragments read 16 rows x one chunk), chunk c of V row r at c ^ ((r & 3) << 2)
// (transposing reads take 4 rows x four chunks).

// DMA one 128 x 128 bf16 tile (tokens key0.., one KV head; src points at that
// head's token 0) into LDS. Each of the 4 waves issues 8 loads of 1 KB (4
// rows); lane l of a load lands at base + 16 l, so each lane fetches the
// logical chunk that the swizzle puts there. Rows past the sequence end
// repeat the last row (finite values; their scores are masked).
template <bool IS_V, int NW = 4>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, size_t rs, int S,
                                         int key0, char* lds) {
  constexpr int kLoads = 32 / NW;  // 1 KB loads (4 rows) per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r4 = lane >> 4, pc = lane & 15;
  const uint32_t dst = lds_u32(lds) + wave * kLoads * 1024;
  const int row0 = key0 + wave * 4 * kLoads;
  const uint32_t rsb = (uint32_t)rs * 2;  // bytes per token row
  if (row0 + 4 * kLoads <= S) {
    const uint16_t* base = src + (size_t)row0 * rs;
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int lc = IS_V ? (pc ^ (r4 << 2)) : (pc ^ (((it & 3) << 2) | r4));
      dma16(base + (size_t)(it * 4) * rs, r4 * rsb + lc * 16, dst + it * 1024);
    }
  } else {
    // ragged end: rows are clamped to S - 1, offsets taken from min(row0, S - 1)
    const int r0 = min(row0, S - 1);
    const uint16_t* cbase = src + (size_t)r0 * rs;
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int lc = IS_V ? (pc ^ (r4 << 2)) : (pc ^ (((it & 3) << 2) | r4));
      const int tok = min(row0 + it * 4 + r4, S - 1);
      dma16(cbase, (uint32_t)(tok - r0) * rsb + lc * 16, dst + it * 1024);
    }
  }
}

__device__ __forceinline__ void load_q(const uint16_t* __restrict__ Q, int S, int Hq, int h,
                                       int qt, int wave, bf16x8_t* qf) {
  const int lane = threadIdx.x & 63;
  const int t = qt * TILE + wave * 32 + (lane & 31);
  const int hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (t < S) u = *reinterpret_cast<const uint4*>(Q + ((size_t)t * Hq + h) * D + 16 * c + 8 * hh);
    qf[c] = as_bf16x8(u);
  }
}

// Unnormalised partial result of one key-range chunk: for each of the tile's
// 128 query rows, O (D floats, not yet divided by the row sum), the running
// max m (base 2, scaled) and the row sum l.
__device__ __forceinline__ void store_part(float* __restrict__ part, const f32x16_t* o, float m_run,
                                           float l_run) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  const float l = pair_sum(l_run);
  float* row = part + (size_t)(wave * 32 + m32) * kPartRow;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * hh;
      *reinterpret_cast<float4*>(row + d) =
          make_float4(o[db][4 * rg], o[db][4 * rg + 1], o[db][4 * rg + 2], o[db][4 * rg + 3]);
    }
  if (hh == 0) {
    row[D] = m_run;
    row[D + 1] = l;
  }
}

// Merge the key-range chunks of one (query tile, head): per row, with M the
// largest chunk max, O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c. One
// workgroup takes 16 rows of the tile; 16 threads share a row, 8 outputs each.
constexpr int kCombineRows = 16;
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(AttnArgs a, SegArgs seg) {
  const int per_tile = TILE / kCombineRows;
  const int item = blockIdx.x / per_tile;  // (qt - qt_lo) * Hq + h
  const int r = (blockIdx.x % per_tile) * kCombineRows + (threadIdx.x >> 4);
  const int d0 = (threadIdx.x & 15) * 8;
  const int h = item % a.Hq;
  const int qt = seg.qt_lo + item / a.Hq;
  const int t = qt * TILE + r;
  if (t >= a.S || t < seg.q_row_begin) return;
  int lo = 0, hi = seg.n_seg - 1;  // segment of the tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg.start[mid] <= qt * TILE) lo = mid; else hi = mid - 1;
  }
  const int jlo = (lo == seg.n_seg - 1) ? 0 : seg.start[lo] / TILE;
  const int nc = min(seg.chunks, (qt - jlo + seg.chunk_tiles) / seg.chunk_tiles);
  const size_t cstride = (size_t)TILE * kPartRow;
  const float* base = seg.part + ((size_t)item * seg.chunks * TILE + r) * kPartRow;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[c * cstride + D]);
  float L = 0.f;
  float acc[8] = {};
  for (int c = 0; c < nc; ++c) {
    const float* pc = base + c * cstride;
    const float w = __builtin_amdgcn_exp2f(pc[D] - M);
    L += w * pc[D + 1];
    const float4 x0 = *reinterpret_cast<const float4*>(pc + d0);
    const float4 x1 = *reinterpret_cast<const float4*>(pc + d0 + 4);
    acc[0] += w * x0.x;
    acc[1] += w * x0.y;
    acc[2] += w * x0.z;
    acc[3] += w * x0.w;
    acc[4] += w * x1.x;
    acc[5] += w * x1.y;
    acc[6] += w * x1.z;
    acc[7] += w * x1.w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((size_t)t * a.Hq + h) * D + d0;
  *reinterpret_cast<uint4*>(orow) =
      make_uint4(cvt_pk_bf16(acc[0] * inv, acc[1] * inv), cvt_pk_bf16(acc[2] * inv, acc[3] * inv),
                 cvt_pk_bf16(acc[4] * inv, acc[5] * inv), cvt_pk_bf16(acc[6] * inv, acc[7] * inv));
  if (a.lse && d0 == 0)
    a.lse[(size_t)h * a.S + t] =
        L > 0.f ? (M + __log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

// Key tiles of one unit in segment mode: jlo..jhi.
struct SegTiles {
  int jhi;
  __device__ int next_after(int j) const { return j < jhi ? j + 1 : -1; }
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

// Key tiles of a pair unit (shared-query mode): the merged walk over two CSR
// rows, those of query tiles qt[0] and qt[1] of one head, each staged in LDS
// 256 entries at a time. Every wave evaluates the walk identically, so list
// reloads (which need a workgroup barrier) happen in step. A tile listed in
// both rows is visited once with both halves members; entries outside
// 0..qt[h] are skipped; unsorted rows are walked correctly (each half visits
// exactly its own entries), sorted rows share every common tile.
struct PairTiles {
  const int32_t* col_idx;
  int e[2], e1[2], cb[2], qt[2], cur[2];
  int* lst;
  __device__ int head(int h) {
    for (; e[h] < e1[h]; ++e[h]) {
      if (e[h] - cb[h] >= kThreads) {  // reload: every wave reaches this point together
        lds_barrier();
        cb[h] = e[h];
        if (threadIdx.x < kThreads)
          lst[h * kThreads + threadIdx.x] =
              (cb[h] + (int)threadIdx.x < e1[h]) ? col_idx[cb[h] + threadIdx.x] : -1;
        lds_barrier();
      }
      const int j = lst[h * kThreads + e[h] - cb[h]];
      if (j >= 0 && j <= qt[h]) return j;
    }
    return -1;
  }
  // the walk's next tile (-1 at the end) and which halves list it
  __device__ int next(bool& m0, bool& m1) {
    const int a0 = cur[0], a1 = cur[1];
    const int j = a0 < 0 ? a1 : (a1 < 0 ? a0 : min(a0, a1));
    m0 = j >= 0 && a0 == j;
    m1 = j >= 0 && a1 == j;
    if (m0) { ++e[0]; cur[0] = head(0); }
    if (m1) { ++e[1]; cur[1] = head(1); }
    return j;
  }
};

// The kernel body. PAIR (shared-query execution): one workgroup of 8 waves
// takes query tiles 2p and 2p + 1 of one head, one 4-wave half each, and
// walks the union of their block lists: each key tile is moved into LDS once
// for both halves, and a half skips the products of a tile its own list does
// not hold.
template <bool SEG, bool PAIR>
__device__ __forceinline__ void attn_bf16_body(const AttnArgs& a,
                                               const int32_t* __restrict__ row_ptr,
                                               const int32_t* __restrict__ col_idx,
                                               const SegArgs& seg, float scale_log2) {
  constexpr int NW = PAIR ? 8 : 4;  // waves per workgroup
  __shared__ __attribute__((aligned(1024))) char Ks[TILE * ROWB];
  __shared__ __attribute__((aligned(1024))) char Vs[TILE * ROWB];
  __shared__ int lst[SEG ? 1 : (PAIR ? 2 * kThreads : kThreads)];
  const int G = a.Hq / a.Hkv;
  const int nq = (a.S + TILE - 1) / TILE;
  // segment mode: workgroups [0, grid_split) run key-range chunks
  const bool chunked = SEG && (int)blockIdx.x < seg.grid_split;
  Unit u;
  if (PAIR) {
    if (!decode_unit(blockIdx.x, G, a.Hkv, 0, (nq + 1) / 2, 1, u)) return;
  } else if (!SEG) {
    if (!decode_unit(blockIdx.x, G, a.Hkv, 0, nq, 1, u)) return;
  } else if (chunked) {
    if (!decode_unit(blockIdx.x, G, a.Hkv, seg.qt_lo, seg.qt_hi, seg.chunks, u)) return;
  } else {
    if (!decode_unit(blockIdx.x - seg.grid_split, G, a.Hkv, seg.rest_lo, seg.rest_hi, 1, u)) return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = (threadIdx.x >> 6) & 3;       // the wave's 32-row slot in its query tile
  const int hq = PAIR ? (int)(threadIdx.x >> 8) : 0;  // pair mode: the wave's half
  const int qt_me = PAIR ? 2 * u.qt + hq : u.qt;  // the wave's query tile
  const int m32 = lane & 31, hh = lane >> 5;
  const size_t rs = (size_t)a.Hkv * D;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (size_t)u.g * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + (size_t)u.g * D;

  // tile iteration state
  CsrTiles csr{col_idx, 0, 0, 0, u.qt, lst};
  PairTiles pt;
  if (PAIR) {
    pt.col_idx = col_idx;
    pt.lst = lst;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pt.qt[h] = 2 * u.qt + h;
      const int row = (a.per_head ? u.h : u.g) * nq + pt.qt[h];
      pt.e[h] = pt.qt[h] < nq ? row_ptr[row] : 0;
      pt.e1[h] = pt.qt[h] < nq ? row_ptr[row + 1] : 0;
      pt.cb[h] = pt.e[h];
    }
    const int hl = threadIdx.x >> 8, tl = threadIdx.x & (kThreads - 1);
    lst[threadIdx.x] = (pt.e[hl] + tl < pt.e1[hl]) ? col_idx[pt.e[hl] + tl] : -1;
    lds_barrier();
    pt.cur[0] = pt.head(0);
    pt.cur[1] = pt.head(1);
  }
  int jseg_lo = 0;
  if (!SEG && !PAIR) {
    const int row = (a.per_head ? u.h : u.g) * nq + u.qt;
    csr.e = row_ptr[row];
    csr.e1 = row_ptr[row + 1];
    csr.cb = csr.e;
    lst[threadIdx.x] = (csr.e + (int)threadIdx.x < csr.e1) ? col_idx[csr.e + threadIdx.x] : -1;
    lds_barrier();
  }
  SegTiles segt{u.qt};
  if (SEG) {
    const int p = segment_of_tile(seg, u.qt);
    jseg_lo = (p == seg.n_seg - 1) ? 0 : seg.start[p] / TILE;
    if (chunked) {  // this workgroup's piece of the key range
      jseg_lo += u.c * seg.chunk_tiles;
      if (jseg_lo > u.qt) return;  // nothing left for this chunk
      segt.jhi = min(jseg_lo + seg.chunk_tiles - 1, u.qt);
    }
  }

  bf16x8_t qf[8];
  if (!SEG) load_q(static_cast<const uint16_t*>(a.q), a.S, a.Hq, u.h, qt_me, wave, qf);
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

  bool mem0 = true, mem1 = true;  // pair mode: which halves list tile j
  int j = SEG ? jseg_lo : (PAIR ? pt.next(mem0, mem1) : csr.next(csr.e));
  if (SEG) {
    // The Q tile goes to LDS by DMA (into Vs, which is free until the first
    // V tile) together with the first K tile, so the two land in one memory
    // round trip; the fragments are then read from LDS.
    dma_tile<true>(static_cast<const uint16_t*>(a.q) + (size_t)u.h * D, (size_t)a.Hq * D, a.S,
                   u.qt * TILE, Vs);
    dma_tile<false>(Kg, rs, a.S, j * TILE, Ks);
    wait_vmcnt<8>();  // Q has landed (K may still be in flight)
    lds_barrier();
    const int r = wave * 32 + m32;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[c] = as_bf16x8(*reinterpret_cast<const uint4*>(Vs + r * ROWB +
                                                         (((2 * c + hh) ^ ((r & 3) << 2)) << 4)));
    lds_barrier();  // every wave holds its Q fragments: Vs is free
    dma_tile<true>(Vg, rs, a.S, j * TILE, Vs);
  } else {
    wait_vmcnt<0>();  // Q fragments and the CSR chunk are in registers before any tile DMA
    if (j >= 0) {
      dma_tile<false, NW>(Kg, rs, a.S, j * TILE, Ks);
      dma_tile<true, NW>(Vg, rs, a.S, j * TILE, Vs);
    }
  }
  while (j >= 0) {
    bool mn0 = false, mn1 = false;
    const int jn = SEG ? segt.next_after(j) : (PAIR ? pt.next(mn0, mn1) : csr.next(csr.e + 1));
    // pair mode: a half computes only on the tiles its own list holds (the
    // test is uniform over the half's waves; barriers stay outside it)
    const bool me = !PAIR || (hq ? mem1 : mem0);
    wait_vmcnt<32 / NW>();  // K(j) has landed (V(j) may still be in flight)
    lds_barrier();
    f32x16_t s[4];
    if (me) {
    // ---- S^T = K Q^T (four independent accumulators in turn) ----
    // Wave priority: matrix phases win issue over the other workgroup's
    // softmax on the same SIMD (P.V highest, so a tile's output accumulation
    // is not held up behind the next tile's scores).
    __builtin_amdgcn_s_setprio(1);
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
    }
    lds_barrier();  // every wave is done with Ks
    if (jn >= 0) dma_tile<false, NW>(Kg, rs, a.S, jn * TILE, Ks);
    uint32_t pk[4][8];
    if (me) {
    // ---- online softmax (base 2) ----
    if (j == qt_me) {
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
    }
    if (jn >= 0) wait_vmcnt<32 / NW>(); else wait_vmcnt<0>();  // V(j) has landed
    lds_barrier();
    if (me) {
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
    }
    lds_barrier();  // every wave is done with Vs
    if (jn >= 0) dma_tile<true, NW>(Vg, rs, a.S, jn * TILE, Vs);
    j = jn;
    mem0 = mn0;
    mem1 = mn1;
  }
  if (chunked)
    store_part(seg.part + ((((size_t)(u.qt - seg.qt_lo) * a.Hq + u.h) * seg.chunks + u.c) * TILE) *
                              kPartRow,
               o, m_run, l_run);
  else if (!PAIR || qt_me < nq)
    store_out_lds(static_cast<uint16_t*>(a.out), a.lse, a.S, a.Hq, u.h, qt_me,
                  SEG ? seg.q_row_begin : 0, o, m_run, l_run, 1.0f, hq ? Vs : Ks, wave);
}

template <bool SEG>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a,
                                                                const int32_t* __restrict__ row_ptr,
                                                                const int32_t* __restrict__ col_idx,
                                                                SegArgs seg, float scale_log2) {
  attn_bf16_body<SEG, false>(a, row_ptr, col_idx, seg, scale_log2);
}

__global__ __launch_bounds__(2 * kThreads, 1) void attn_bf16_pair_kernel(
    AttnArgs a, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    SegArgs seg, float scale_log2) {
  attn_bf16_body<false, true>(a, row_ptr, col_idx, seg, scale_log2);
}

}  // namespace

int attn_split_grid(int Hq, int Hkv, int n_qt, int chunks) {
  return chunks > 0 ? attn_grid(Hq, Hkv, n_qt, chunks) : 0;
}

rbs_status launch_attn_bf16_csr(const AttnArgs& a, hipStream_t st) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int nq = (a.S + TILE - 1) / TILE;
  SegArgs none;
  none.n_seg = 0;
  none.q_row_begin = 0;
  none.theta = 0.f;
  none.qt_lo = 0;
  none.qt_hi = nq;
  none.chunks = 0;
  none.chunk_tiles = 0;
  none.rest_lo = 0;
  none.rest_hi = nq;
  none.grid_split = 0;
  none.part = nullptr;
  hipLaunchKernelGGL(attn_bf16_kernel<false>, dim3(attn_grid(a.Hq, a.Hkv, nq, 1)), dim3(kThreads),
                     0, st, a, a.row_ptr, a.col_idx, none, scale_log2);
  return launch_status();
}

rbs_status launch_attn_bf16_pairs(const AttnArgs& a, hipStream_t st) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int nq = (a.S + TILE - 1) / TILE;
  SegArgs none;
  none.n_seg = 0;
  none.q_row_begin = 0;
  none.theta = 0.f;
  none.qt_lo = 0;
  none.qt_hi = nq;
  none.chunks = 0;
  none.chunk_tiles = 0;
  none.rest_lo = 0;
  none.rest_hi = nq;
  none.grid_split = 0;
  none.part = nullptr;
  hipLaunchKernelGGL(attn_bf16_pair_kernel, dim3(attn_grid(a.Hq, a.Hkv, (nq + 1) / 2, 1)),
                     dim3(2 * kThreads), 0, st, a, a.row_ptr, a.col_idx, none, scale_log2);
  return launch_status();
}

rbs_status launch_attn_segments(const AttnArgs& a, const SegArgs& s, hipStream_t st) {
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int grid = s.grid_split + attn_grid(a.Hq, a.Hkv, s.rest_hi - s.rest_lo, 1);
  if (grid == 0) return RBS_OK;
  hipLaunchKernelGGL(attn_bf16_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a, nullptr, nullptr,
                     s, scale_log2);
  return launch_status();
}

rbs_status launch_attn_combine(const AttnArgs& a, const SegArgs& s, hipStream_t st) {
  const int n_qt = s.qt_hi - s.qt_lo;
  if (n_qt <= 0) return RBS_OK;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(n_qt * a.Hq * (TILE / kCombineRows)),
                     dim3(kThreads), 0, st, a, s);
  return launch_status();
}

}  // namespace rbs
