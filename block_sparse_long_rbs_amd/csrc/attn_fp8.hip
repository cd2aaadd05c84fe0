// Block-sparse causal GQA attention with fp8 inputs: Q, K and V in the OCP
// e4m3 format, each with one dequantisation factor, and a bf16 output; head
// dim 128, key tile = block = 128 tokens, on gfx950 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4: fp8 x fp8 products of depth 64, fp32 sums).
// RBS-Attention explainer, "The Fix": the selection's CSR block lists drive a
// standard block-sparse attention; this is that attention for fp8 caches.
//
// Work decomposition, CSR iteration, online softmax and XCD-aware grid are
// those of the bf16 kernel (attn_bf16.hip). Per key tile, in two 64-key
// halves (only one half's scores are live at a time):
//   S^T = K Q^T: per 32-key block, two products of depth 64. A lane holds 32
//     consecutive head-dim bytes of its key row and of its query row, both
//     read from LDS (two 16-byte reads each). The MFMA pairs A and B bytes by
//     the same (lane half, byte) position, so one common byte order serves
//     both.
//   P' = 2^(s - m - e) rounded to e4m3 (nearest even) straight from the
//     score registers, with one power-of-two exponent e per (query row,
//     32-key block) chosen so that the block's largest P' lies in (128, 256]:
//     every block's probabilities use e4m3's whole range (a long tail of small
//     P is neither pushed into the subnormal range nor flushed to zero by a
//     large P elsewhere in the row), and the scaled matrix instruction
//     restores 2^e exactly (its B operand takes one E8M0 exponent per 32-deep
//     block of each column). The row sum is one more scaled product of the
//     same bytes with an all-ones operand. The reference m is lazy, as in the
//     bf16 kernel: raised only when a score passes it by more than 64.
//   O^T += V^T P^T: per 32-wide slice of the head dim and 64-key half, one
//     product. The V^T operand comes from 8-bit transposing LDS reads
//     (ds_read_b64_tr_b8), ordered so that byte j of a lane pairs with the
//     key that byte j of the P operand holds.
// Scores are scaled by softmax_scale * q_descale * k_descale, the output by
// v_descale. Q, K and V tiles are 16 KB each (128 bytes per row), moved HBM
// -> LDS by global_load_lds_dwordx4 with explicit vector-memory counts as in
// the bf16 kernel (4 loads per wave per tile instead of 8).
//
// The softmax's vector instructions, not the matrix products, set the pace.
// The per-block exponents need each block's largest score (a max over the
// lane's 16 values and one cross-lane exchange) on top of the exponentials;
// held to 168 VGPRs for three waves per SIMD the kernel spills, so it runs at
// 229 VGPRs and two waves per SIMD (49 KB of LDS per workgroup).
//
// Bound: matrix cores. Algorithmic flops per (query row, key) pair: 4*D.

#include "attn_tiles.h"

namespace rbs {
namespace {

using namespace tiles;

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;

constexpr int ROW8 = D;  // bytes per K or V row in LDS

// 32x32 block += A (32 x 64, e4m3) * B (64 x 32, e4m3). Constant zero scale
// operands select the plain (unscaled) instruction.
__device__ __forceinline__ f32x16_t mfma_fp8(const v8i_t& a, const v8i_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with B scaled by E8M0 exponent bytes (2^(sb - 127)), one
// per 32-deep block of each column. Checked on the GPU with one-wave probes:
// block 0 of column c is bytes 0-15 of lanes c and c + 32 and takes lane c's
// byte, block 1 is bytes 16-31 of both and takes lane c + 32's byte; a
// constant zero operand selects the unscaled instruction, a runtime 0 means
// 2^-127.
__device__ __forceinline__ f32x16_t mfma_fp8_bscaled(const v8i_t& a, const v8i_t& b,
                                                     const f32x16_t& c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// 16-byte chunk swizzles in LDS (8 chunks per 128-byte row): chunk c of K row
// r sits at slot c ^ ((r >> 1) & 7) (fragment reads take 32 rows x one chunk),
// chunk c of V row r at c ^ (((r >> 1) & 3) << 1) (transposing reads take 16
// rows x two neighbouring chunks). Either way each read spreads evenly over
// the LDS banks.
__device__ __forceinline__ int k_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v_swz(int r) { return ((r >> 1) & 3) << 1; }

// DMA one 128 x 128 e4m3 tile (tokens key0.., one KV head; src points at that
// head's token 0) into LDS. Each of the 4 waves issues 4 loads of 1 KB (8
// rows); lane l of a load lands at slot l & 7 of row l >> 3, so it fetches
// the logical chunk that the swizzle puts there. Rows past the sequence end
// repeat the last row (finite values; their scores are masked).
template <bool IS_V>
__device__ __forceinline__ void dma_tile8(const uint8_t* __restrict__ src, size_t rs, int S,
                                          int key0, char* lds) {
  // the lane's offsets are recomputed at every call from an opaque copy of
  // the thread id, so that none of them has to stay live across the tile loop
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r8 = lane >> 3, pc = lane & 7;
  const uint32_t dst = lds_u32(lds) + wave * 4 * 1024;
  const int row0 = key0 + wave * 32;
  const uint32_t rsb = (uint32_t)rs;  // bytes per token row
  if (row0 + 32 <= S) {
    const uint8_t* base = src + (size_t)row0 * rs;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = wave * 32 + it * 8 + r8;  // row within the tile
      const int lc = pc ^ (IS_V ? v_swz(r) : k_swz(r));
      dma16(base + (size_t)(it * 8) * rs, r8 * rsb + lc * 16, dst + it * 1024);
    }
  } else {
    // ragged end: rows are clamped to S - 1, offsets taken from min(row0, S - 1)
    const int r0 = min(row0, S - 1);
    const uint8_t* cbase = src + (size_t)r0 * rs;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = wave * 32 + it * 8 + r8;
      const int lc = pc ^ (IS_V ? v_swz(r) : k_swz(r));
      const int tok = min(row0 + it * 8 + r8, S - 1);
      dma16(cbase, (uint32_t)(tok - r0) * rsb + lc * 16, dst + it * 1024);
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_fp8_kernel(AttnArgs a,
                                                               const int32_t* __restrict__ row_ptr,
                                                               const int32_t* __restrict__ col_idx,
                                                               float scale_log2, float out_scale) {
  // K and V tiles side by side: together they stage the 32 KB output tile
  __shared__ __attribute__((aligned(1024))) char KVs[2 * TILE * ROW8];
  __shared__ __attribute__((aligned(1024))) char Qs[TILE * ROW8];
  char* const Ks = KVs;
  char* const Vs = KVs + TILE * ROW8;
  __shared__ int lst[kThreads];
  const int G = a.Hq / a.Hkv;
  const int nq = (a.S + TILE - 1) / TILE;
  Unit u;
  if (!decode_unit(blockIdx.x, G, a.Hkv, 0, nq, 1, u)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m32 = lane & 31, hh = lane >> 5;
  const size_t rs = (size_t)a.Hkv * D;
  const uint8_t* Kg = static_cast<const uint8_t*>(a.k) + (size_t)u.g * D;
  const uint8_t* Vg = static_cast<const uint8_t*>(a.v) + (size_t)u.g * D;

  CsrTiles csr{col_idx, 0, 0, 0, u.qt, lst};
  {
    const int row = (a.per_head ? u.h : u.g) * nq + u.qt;
    csr.e = row_ptr[row];
    csr.e1 = row_ptr[row + 1];
    csr.cb = csr.e;
    lst[threadIdx.x] = (csr.e + (int)threadIdx.x < csr.e1) ? col_idx[csr.e + threadIdx.x] : -1;
    lds_barrier();
  }

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16_t){};
  float m_run = 0.f, l_run = 0.f;
  bool first = true;

  // per-lane LDS offsets. K fragment of key block kb, depth chunk kc: row
  // kb * 32 + m32, logical chunks 4 kc + 2 hh and 4 kc + 2 hh + 1.
  const int kswz = k_swz(m32);  // rows kb * 32 + m32 share bits 1..3 with m32
  // V^T fragment, read q of 4 for depth slice db and key chunk kc: this lane
  // supplies row 64 kc + 16 q + vrow (q's two bits put 32 (q >> 1) + 16 (q & 1)
  // = 16 q) and byte 32 db + 16 (g & 1) + 8 (s & 1) of it, with g = lane / 16,
  // s = lane % 16 (a transposing read hands lane i of a 16-lane group byte
  // i & 7 of the 8 bytes addressed by lane 2 k + (i >> 3), for k = 0..7).
  const int g16 = lane >> 4, s16 = lane & 15;
  const int vrow = 8 * (s16 >> 3) + 4 * (g16 >> 1) + ((s16 >> 1) & 3);
  const int vswz = v_swz(vrow);  // rows 64 kc + 16 q + vrow share bits 1..2 with vrow
  const int v_lane = vrow * ROW8 + 8 * (s16 & 1);
  const int qq = wave * 32 + m32;

  int j = csr.next(csr.e);
  wait_vmcnt<0>();  // the CSR chunk is in registers before any tile DMA
  if (j >= 0) {
    // the query tile is staged like a K tile (same swizzle); rows past the
    // end repeat the last row and their outputs are never stored
    dma_tile8<false>(static_cast<const uint8_t*>(a.q) + (size_t)u.h * D, (size_t)a.Hq * D, a.S,
                     u.qt * TILE, Qs);
    dma_tile8<false>(Kg, rs, a.S, j * TILE, Ks);
    dma_tile8<true>(Vg, rs, a.S, j * TILE, Vs);
  }
  // 16-byte LDS reads of a fragment: chunks 4 kc + 2 hh and 4 kc + 2 hh + 1
  // of a row stored with the K swizzle (query rows and key rows alike)
  auto read_frag = [&](const char* rowp, int kc) {
    const uint4 c0 = *reinterpret_cast<const uint4*>(rowp + (((4 * kc + 2 * hh) ^ kswz) << 4));
    const uint4 c1 = *reinterpret_cast<const uint4*>(rowp + (((4 * kc + 2 * hh + 1) ^ kswz) << 4));
    return (v8i_t){(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w,
                   (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
  };
  const char* const qrow = Qs + qq * ROW8;
  const char* const krow = Ks + m32 * ROW8;
  // Probabilities in e4m3 with one power-of-two scale per 32-key block and
  // query row. The B operand of the P.V product carries one exponent per
  // 32-deep block of each column, and the blocks are exactly the key blocks
  // kb of a half (lanes l and l ^ 32 hold 16 keys of each). So for each key
  // block the pair takes the largest score, x (base 2, relative to the row's
  // reference m_run), picks e = ceil(x) - 8 and packs P' = 2^(s - m_run - e),
  // whose largest value lies in (128, 256]: every block's probabilities use
  // e4m3's whole range (relative error <= 2^-4 down to 2^-13 of the block's
  // largest), whatever the other blocks hold, and the product restores 2^e
  // exactly. The row sum comes from the same scaled bytes, as one more
  // product with an all-ones A operand.
  // The reference itself is lazy, as in the bf16 kernel: taken from the
  // row's first half tile and raised only when a score passes it by more
  // than 64 (so that sums stay far inside fp32's range). A raise moves it by
  // a whole number k of powers of two: O and the row sum are multiplied by
  // 2^-k exactly and a half already packed only needs its exponents lowered
  // by k, so nothing is recomputed.
  const v8i_t ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};
  while (j >= 0) {
    const int jn = csr.next(csr.e + 1);
    wait_vmcnt<4>();  // K(j) (and at the first tile Q) has landed; V(j) may be in flight
    lds_barrier();
    const bool diag = j == u.qt;
    // causal mask inside the diagonal tile; t is made opaque so that the
    // per-element predicates are not hoisted out of the tile loop
    int t = qq - 4 * hh;
    asm volatile("" : "+v"(t));
    // P' in e4m3, packed as the B operand of the P.V products: byte j of
    // dword w of key block kb is the lane's score element r = 4 w + j; sb
    // holds each half's exponent byte (of key block 2 half in lanes 0-31, of
    // key block 2 half + 1 in lanes 32-63).
    int pk[4][4];
    int sb[2];
    float k_raise = 0.f;
    f32x16_t s[2];
    // S^T = K Q^T for the 64-key half `half` (key blocks 2 half, 2 half + 1),
    // in the order (depth chunk, key block) so that one Q fragment is live
    auto scores = [&](int half) {
      __builtin_amdgcn_s_setprio(1);
      v8i_t kf = read_frag(krow + (2 * half) * 32 * ROW8, 0);
      v8i_t qc = read_frag(qrow, 0);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int kc = x >> 1, kk = x & 1;
        const v8i_t cur = kf;
        if (x < 3) kf = read_frag(krow + (2 * half + ((x + 1) & 1)) * 32 * ROW8, (x + 1) >> 1);
        s[kk] = mfma_fp8(cur, qc, kc ? s[kk] : (f32x16_t){});
        if (x == 1) qc = read_frag(qrow, 1);
      }
      __builtin_amdgcn_s_setprio(0);
      if (diag) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((2 * half + kk) * 32 + 8 * (r >> 2) + (r & 3) > t) s[kk][r] = -INFINITY;
      }
    };
    auto exps = [&](int half) {
      float mb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kk][r]);
        mb[kk] = pair_max(mx) * scale_log2;  // the key block's largest score
      }
      const float hm = fmaxf(mb[0], mb[1]);
      // reference: the first half's max; later raised by a whole number k of
      // powers of two when a score passes it by more than 64 (rare; O and
      // the row sum are rescaled before this tile's products are added, and
      // the first half's exponents lowered by k)
      if (first) {
        m_run = hm;
        first = false;
      } else if (__ballot(hm - m_run > 64.f)) {
        const float k = fmaxf(ceilf(hm - m_run), 0.f);
        m_run += k;
        k_raise += k;
        if (half == 1) sb[0] = max(sb[0] - (int)k, 1);
      }
      // block exponent e = ceil(x) - 8, x the block's largest score over the
      // reference, kept to [-126, 56] (a block whose scores all lie more than
      // 118 below the reference contributes nothing measurable)
      float neg[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const float e = ceilf(fminf(fmaxf(mb[kk] - m_run, -118.f), 64.f)) - 8.f;
        neg[kk] = -(m_run + e);
        if (kk == hh) sb[half] = (int)e + 127;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kk][4 * w], scale_log2, neg[kk]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kk][4 * w + 1], scale_log2, neg[kk]));
          const float p2 = __builtin_amdgcn_exp2f(fmaf(s[kk][4 * w + 2], scale_log2, neg[kk]));
          const float p3 = __builtin_amdgcn_exp2f(fmaf(s[kk][4 * w + 3], scale_log2, neg[kk]));
          int xw = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          xw = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, xw, true);
          pk[2 * half + kk][w] = xw;
        }
    };
    scores(0);
    exps(0);
    scores(1);
    exps(1);
    lds_barrier();  // every wave is done with Ks
    if (jn >= 0) dma_tile8<false>(Kg, rs, a.S, jn * TILE, Ks);
    if (jn >= 0) wait_vmcnt<4>(); else wait_vmcnt<0>();  // V(j) has landed
    lds_barrier();
    if (__ballot(k_raise > 0.f)) {
      const float alpha = __builtin_amdgcn_exp2f(-k_raise);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    // ---- O^T += V^T P^T (fragments read one step ahead) and the row sum ----
    __builtin_amdgcn_s_setprio(2);
    auto read_v = [&](int kc, int db, v8i_t& f) {
      const char* vb = Vs + v_lane + (((2 * db + (g16 & 1)) ^ vswz) << 4) + kc * 64 * ROW8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v2i_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(vb + 16 * q * ROW8));
        f[2 * q] = x[0];
        f[2 * q + 1] = x[1];
      }
    };
    v8i_t vf[2];
    read_v(0, 0, vf[0]);
    f32x16_t rsum = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int kc = st >> 2, db = st & 3;
      if (st < 7) read_v((st + 1) >> 2, (st + 1) & 3, vf[(st + 1) & 1]);
      const v8i_t b = {pk[2 * kc][0], pk[2 * kc][1], pk[2 * kc][2], pk[2 * kc][3],
                       pk[2 * kc + 1][0], pk[2 * kc + 1][1], pk[2 * kc + 1][2], pk[2 * kc + 1][3]};
      // every row of this product holds the column sums: element 0 is the
      // lane's full row sum over the tile's keys
      if (db == 0) rsum = mfma_fp8_bscaled(ones, b, rsum, sb[kc]);
      o[db] = mfma_fp8_bscaled(vf[st & 1], b, o[db], sb[kc]);
    }
    __builtin_amdgcn_s_setprio(0);
    // lanes l and l ^ 32 both hold the full sum; their shares are added at the end
    l_run += 0.5f * rsum[0];
    lds_barrier();  // every wave is done with Vs
    if (jn >= 0) dma_tile8<true>(Vg, rs, a.S, jn * TILE, Vs);
    j = jn;
  }
  store_out_lds(static_cast<uint16_t*>(a.out), a.lse, a.S, a.Hq, u.h, u.qt, 0, o, m_run, l_run,
                out_scale, KVs, wave);
}

}  // namespace

rbs_status launch_attn_fp8_csr(const AttnArgs& a, float q_descale, float k_descale,
                               float v_descale, hipStream_t st) {
  const float scale_log2 = a.scale * q_descale * k_descale * 1.4426950408889634f;
  const int nq = (a.S + TILE - 1) / TILE;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3(attn_grid(a.Hq, a.Hkv, nq, 1)), dim3(kThreads), 0, st, a,
                     a.row_ptr, a.col_idx, scale_log2, v_descale);
  return launch_status();
}

}  // namespace rbs
