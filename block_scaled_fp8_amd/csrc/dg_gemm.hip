// Block-scaled FP8 GEMM kernels for gfx950 (MI355X, CDNA4).
//
// D = C + A . B^T with E4M3 operands; A carries one scale per row and 128-long
// K block, B one per 128x128 block ("1d2d") or per row and K block ("1d1d").
// Each 128-K block's partial product is promoted into an FP32 accumulator as
// final += scale_a * scale_b * partial (page "02 · DeepGEMM 技术解析" §2.2;
// page "第13章 DeepGEMM" §13.3 algorithm box).
//
// Design (gfx950-first, not the Hopper design the pages describe):
//  * One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-long K block of a
//    16x16 output sub-tile, so the block partial is one MFMA result written
//    from a zero accumulator; the VALU then does final = fma(s, partial, final).
//    No full-tile second accumulator set is needed.
//  * The MFMA is issued with the weight fragment as its first operand and the
//    activation fragment as its second, so each lane ends up owning one output
//    row and four consecutive output columns: one activation scale per lane and
//    fragment, and 8- or 16-byte contiguous stores in the epilogue.
//  * A and B tiles go HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging), 2 LDS stages, each 128-byte row stored with its 16-byte chunks
//    XOR-swizzled by (row & 7) ^ ((row >> 3) & 1): measured with the LDS
//    bank-conflict counter on gfx950, this key makes the fragment reads (16
//    rows x one 16-byte chunk per lane group) conflict free, where plain
//    (row & 7) or ((row >> 1) & 7) keys are 2-way conflicted.
//  * The pipeline runs across tiles: the first stage of a workgroup's next tile
//    is enqueued during the current tile's last K block, and barriers wait on
//    explicit vmcnt values, so epilogue stores do not block the next loads.
//  * Persistent workgroups walk output tiles with stride gridDim.x (page
//    "02 · DeepGEMM 技术解析" §4.3); logical workgroup ids are remapped so
//    consecutive ids share an XCD (and its L2), and tiles are ordered in
//    super-rows of m tiles so concurrently running tiles share A and B.
//  * When a wave's N range straddles two 128-wide weight-scale blocks, the
//    number of leading 16-column fragments that use the first block's scale is
//    a template parameter, selected once per tile: the choice per fragment is
//    resolved at compile time (page "02 · DeepGEMM 技术解析" §2.3).
#include "dg_internal.h"

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
#define DG_LDS __attribute__((address_space(3)))

constexpr int BK = 128;     // K values per scale block and per MFMA
constexpr int STAGES = 2;   // LDS stages

template <int BM, int BN, int WM, int WN>
struct Shape {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM;
  static constexpr int TN = BN / WN;
  static constexpr int FM = TM / 16;
  static constexpr int FN = TN / 16;
  static constexpr int STAGE_BYTES = (BM + BN) * BK;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LOADS = (BM + BN) / 8;           // 1 KiB wave-loads per stage
  static constexpr int LPW = (LOADS + NW - 1) / NW;     // wave-loads per wave
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(TN <= 128, "a wave's N range may touch at most two weight-scale blocks");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "rows are loaded 8 per wave-load");
};

struct Tile {
  int g;        // group
  int m0, n0;   // first row (within the group for masked) and first column
  int m_valid;  // rows < m_valid exist
  bool skip;
};

// LDS slot of 16-byte chunk c of stage row r is c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Persistent scheduler: logical tile index -> (group, m0, n0).
template <int GRP, int BM, int BN>
__device__ __forceinline__ bool get_tile(const GemmParams& p, int t, Tile& tl) {
  tl.skip = false;
  if (GRP == GRP_MASKED) {
    // Groups in order; within a group n tiles outer, m tiles inner, so the m tiles
    // that share a weight slice run next to each other.
    int base = 0;
    for (int g = 0; g < p.num_groups; ++g) {
      const int mg = clampi(p.masked_m[g], 0, p.m);
      const int mt = (mg + BM - 1) / BM;
      const int cnt = mt * p.num_n_tiles;
      if (t < base + cnt) {
        const int loc = t - base;
        tl.g = g;
        tl.n0 = (loc / mt) * BN;
        tl.m0 = (loc % mt) * BM;
        tl.m_valid = mg;
        return true;
      }
      base += cnt;
    }
    return false;
  }
  if (t >= p.total_tiles) return false;
  // super-rows of swizzle_m m tiles, walked column by column
  const int per_super = p.swizzle_m * p.num_n_tiles;
  const int sr = t / per_super;
  const int rem = t - sr * per_super;
  const int rows = min(p.swizzle_m, p.num_m_tiles - sr * p.swizzle_m);
  const int mt = sr * p.swizzle_m + rem % rows;
  const int nt = rem / rows;
  tl.m0 = mt * BM;
  tl.n0 = nt * BN;
  tl.m_valid = p.m;
  tl.g = 0;
  if (GRP == GRP_CONTIG) {
    const int g = p.grouped_layout[tl.m0];
    tl.g = g;
    tl.skip = g < 0 || g >= p.num_groups;
  }
  return true;
}

__device__ __forceinline__ float ue8m0_byte(unsigned int word, int byte) {
  return __uint_as_float(((word >> (8 * byte)) & 0xFFu) << 23);
}

__device__ __forceinline__ unsigned int pack_bf16x2(float x, float y) {
  v2bf v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(unsigned int, v);
}

// Scales of one K block as this lane needs them.
//  1d2d FP32: the lane's activation scale per fragment row, and the (at most two)
//             weight-block scales of the wave's N range.
//  1d1d FP32: the activation scales; weight scales are read per column fragment
//             at promotion time.
//  1d1d UE8M0: raw UE8M0 codes of the lane's activation rows and weight rows; the
//             power-of-two scaling is applied by the MFMA itself.
template <int SFM, int FM, int FN>
struct BlockScales {
  float sa[FM];
  float sb0, sb1;
  int ea[SFM == SF_1D1D_UE8M0 ? FM : 1];
  int eb[SFM == SF_1D1D_UE8M0 ? FN : 1];
};

// Where one wave's share of a tile's stage loads comes from: wave-load q covers 8
// stage rows of 128 bytes; lane L fills LDS bytes [16L, 16L+16) of it = stage row
// r = 8q + L/8, slot L%8, which holds 16-byte chunk (L%8) ^ swz(r) of that row, and
// swz(8q + L/8) = (L/8) ^ (q & 1).  The wave-uniform part of each address lives in
// scalar registers; the per-lane part is one 32-bit offset per chunk parity.  Rows
// past the end of A or B are not loaded (their LDS rows keep stale bytes, which only
// reach output rows or columns that are never stored).
template <int BM, int BN, int WM, int WN>
struct Loader {
  const uint8_t* a_tile;  // row tile.m0 of A (this tile's group)
  const uint8_t* b_tile;  // row tile.n0 of B
  int a_rows, b_rows;     // rows that exist from there on
};

template <int BM, int BN, int WM, int WN, int GRP>
__device__ __forceinline__ void make_loader(const GemmParams& p, const Tile& tl, Loader<BM, BN, WM, WN>& ld) {
  const uint8_t* A = p.a + (GRP == GRP_MASKED ? (int64_t)tl.g * p.a_gstride : 0);
  const uint8_t* B = p.b + (GRP != GRP_DENSE ? (int64_t)tl.g * p.b_gstride : 0);
  ld.a_tile = A + (int64_t)tl.m0 * p.lda;
  ld.b_tile = B + (int64_t)tl.n0 * p.ldb;
  ld.a_rows = p.m - tl.m0;  // m_max rows when masked
  ld.b_rows = p.n - tl.n0;
}

// Enqueue the HBM -> LDS copy of K block kb of a tile into stage s.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void issue_stage(const GemmParams& p, const Loader<BM, BN, WM, WN>& ld, uint8_t* smem,
                                            int kb, int s, const int wave, const int lane) {
  using S = Shape<BM, BN, WM, WN>;
  static_assert((BM / 8) % S::NW == 0, "A and B wave-loads must split at a fixed u");
  constexpr int UA = BM / 8 / S::NW;  // wave-loads u < UA fill A rows, the rest B rows
  const int lr8 = lane >> 3;
  const int lda = (int)p.lda, ldb = (int)p.ldb;
  const bool full = ld.a_rows >= BM && ld.b_rows >= BN;  // uniform: no row to skip
  // per-lane address parts, opaque to the optimiser so it rebuilds each address from a
  // scalar base every K block instead of keeping 64-bit per-lane pointers live
  uint32_t off_a = (uint32_t)(lr8 * lda), off_b = (uint32_t)(lr8 * ldb);
  uint32_t chunk_off = (uint32_t)((lane & 7) ^ lr8) << 4;
  asm volatile("" : "+v"(off_a), "+v"(off_b), "+v"(chunk_off));
#pragma unroll
  for (int u = 0; u < S::LPW; ++u) {
    const int q = wave + u * S::NW;
    if (q < S::LOADS) {
      const int par = (S::NW % 2 == 0) ? (wave & 1) : (u & 1);
      const bool is_a = u < UA;
      const int ld_rows = is_a ? lda : ldb;
      const int row0 = 8 * q - (is_a ? 0 : BM);  // first row of this wave-load (uniform)
      const uint8_t* base = (is_a ? ld.a_tile : ld.b_tile) + (int64_t)kb * BK + (int64_t)row0 * ld_rows;
      const uint32_t lane_off = (is_a ? off_a : off_b) + (chunk_off ^ ((uint32_t)par << 4));
      if (full || lr8 < (is_a ? ld.a_rows : ld.b_rows) - row0)
        __builtin_amdgcn_global_load_lds((const void*)(base + lane_off),
                                         (DG_LDS void*)(smem + s * S::STAGE_BYTES + q * 1024), 16, 0, 0);
    }
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding and no
// LDS operation is, then synchronise the workgroup.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}

// One output tile: the K loop over 128-long blocks, then the epilogue.  K block 0 of
// this tile is already in flight into stage `stage0`; during the last K block the
// first stage of the next tile (if any) is enqueued into the other stage, so it
// overlaps this tile's last block and epilogue.  `vm_after_prefetch` is a lower bound
// on this wave's vector-memory operations issued after that prefetch, before this
// tile's first wait (the previous tile's epilogue stores).
template <int BM, int BN, int WM, int WN, int SFM, int GRP, int OUT, int NF>
__device__ __forceinline__ int gemm_tile(const GemmParams& p, uint8_t* smem, const Tile& tl,
                                         const Loader<BM, BN, WM, WN>& ld, const bool has_next,
                                         const Loader<BM, BN, WM, WN>& ld_next, const int stage0,
                                         const int vm_after_prefetch, const int wave, const int lane) {
  using S = Shape<BM, BN, WM, WN>;
  constexpr int FM = S::FM, FN = S::FN, TM = S::TM, TN = S::TN;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lg = lane >> 4;
  const int nkb = p.sf_k;
  const int g = tl.g;
  const int a_rows = p.m;  // addressable rows of A (m_max for masked)

  // ---- scales
  const int row0 = tl.m0 + wm * TM + lr;       // lane's row in fragment 0
  const int nw0 = tl.n0 + wn * TN;             // wave's first column
  const int64_t sfa_goff = (GRP == GRP_MASKED) ? (int64_t)g * p.sfa_gstride : 0;
  const int64_t sfb_goff = (GRP != GRP_DENSE) ? (int64_t)g * p.sfb_gstride : 0;
  int sa_idx[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) sa_idx[i] = min(row0 + 16 * i, a_rows - 1);
  const int nb = (p.n + 127) / 128;
  const int blk0 = min(nw0 / 128, nb - 1), blk1 = min(nw0 / 128 + 1, nb - 1);
  const int n_a4 = (p.n + 3) & ~3;
  int sb_col[FN];   // 1d1d FP32: first of the lane's four columns in fragment j
  int sb_row[FN];   // 1d1d UE8M0: the weight row the lane feeds to the MFMA in fragment j
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    sb_col[j] = min(nw0 + 16 * j + 4 * lg, n_a4 - 4);
    sb_row[j] = min(nw0 + 16 * j + lr, p.n - 1);
  }

  auto load_scales = [&](int kb, BlockScales<SFM, FM, FN>& sc) {
    if (SFM == SF_1D1D_UE8M0) {
      const unsigned int* sa = (const unsigned int*)p.sfa + sfa_goff + (int64_t)(kb >> 2) * p.sfa_stride;
      const unsigned int* sb = (const unsigned int*)p.sfb + sfb_goff + (int64_t)(kb >> 2) * p.sfb_stride;
      const int sh = 8 * (kb & 3);
#pragma unroll
      for (int i = 0; i < FM; ++i) sc.ea[i] = (sa[sa_idx[i]] >> sh) & 0xFF;
#pragma unroll
      for (int j = 0; j < FN; ++j) sc.eb[j] = (sb[sb_row[j]] >> sh) & 0xFF;
    } else {
      const float* sa = (const float*)p.sfa + sfa_goff + (int64_t)kb * p.sfa_stride;
#pragma unroll
      for (int i = 0; i < FM; ++i) sc.sa[i] = sa[sa_idx[i]];
      if (SFM == SF_1D2D_F32) {
        const float* sb = (const float*)p.sfb + sfb_goff;
        sc.sb0 = sb[(int64_t)blk0 * p.sfb_stride + kb];
        sc.sb1 = (NF < FN) ? sb[(int64_t)blk1 * p.sfb_stride + kb] : sc.sb0;
      }
    }
  };

  float fin[FM][FN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) fin[i][j][v] = 0.f;

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const int sw = swz(lr);  // fragment rows start on multiples of 16: swz(row) == swz(lr)
  const int off_lo = ((2 * lg) ^ sw) * 16, off_hi = ((2 * lg + 1) ^ sw) * 16;

  BlockScales<SFM, FM, FN> cur, nxt;
  load_scales(0, cur);

  for (int kb = 0; kb < nkb; ++kb) {
    const int s = (stage0 + kb) & 1;
    // stage s has landed everywhere and nobody still reads stage s^1
    if (kb == 0) {
      if (vm_after_prefetch >= FM * FN) wait_and_barrier<FM * FN>();
      else wait_and_barrier<0>();
    } else {
      wait_and_barrier<0>();
    }
    if (kb + 1 < nkb) {
      issue_stage(p, ld, smem, kb + 1, s ^ 1, wave, lane);
      load_scales(kb + 1, nxt);
    } else if (has_next) {
      issue_stage(p, ld_next, smem, 0, s ^ 1, wave, lane);
    }
    const uint8_t* st = smem + s * S::STAGE_BYTES;
    // promotion factors for this block
    float s0[FM], s1[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (SFM == SF_1D2D_F32) {
        s0[i] = cur.sa[i] * cur.sb0;
        s1[i] = (NF < FN) ? cur.sa[i] * cur.sb1 : s0[i];
      } else {
        s0[i] = s1[i] = cur.sa[i];
      }
    }
    const float* sb_blk = (const float*)p.sfb + sfb_goff + (int64_t)kb * p.sfb_stride;  // 1d1d FP32

    v8i af[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint8_t* rp = st + (wm * TM + 16 * i + lr) * BK;
      const v4i lo = *(const v4i*)(rp + off_lo);
      const v4i hi = *(const v4i*)(rp + off_hi);
      af[i] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    auto read_b = [&](int j) -> v8i {
      const uint8_t* rp = st + (BM + wn * TN + 16 * j + lr) * BK;
      const v4i lo = *(const v4i*)(rp + off_lo);
      const v4i hi = *(const v4i*)(rp + off_hi);
      return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    auto promote = [&](int i, int j, const v4f& acc) {
      if (SFM == SF_1D2D_F32) {
        const float sc = (j < NF) ? s0[i] : s1[i];  // compile-time choice
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] = __builtin_fmaf(sc, acc[v], fin[i][j][v]);
      } else if (SFM == SF_1D1D_F32) {
        const v4f w = *(const v4f*)(sb_blk + sb_col[j]);
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] = __builtin_fmaf(s0[i] * w[v], acc[v], fin[i][j][v]);
      } else {
        // UE8M0: the MFMA already multiplied by 2^(ea-127) * 2^(eb-127)
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] += acc[v];
      }
    };
    auto mfma = [&](const v8i& bfr, int i, int j) -> v4f {
      if (SFM == SF_1D1D_UE8M0)
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr, af[i], zero, 0, 0, 0, cur.eb[j], 0,
                                                                cur.ea[i]);
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr, af[i], zero, 0, 0, 0, 0, 0, 0);
    };
    // Software pipeline: the partial of MFMA t is promoted while MFMA t+1 runs.
    // The weight fragment is the first MFMA operand, so the lane owns row lr and
    // columns 4*lg + v of each 16x16 block.
    v8i bf = read_b(0);
    v4f acc_prev = zero;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      v8i bf_next = bf;
      if (j + 1 < FN) bf_next = read_b(j + 1);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v4f acc = mfma(bf, i, j);
        if (i > 0) promote(i - 1, j, acc_prev);
        else if (j > 0) promote(FM - 1, j - 1, acc_prev);
        acc_prev = acc;
      }
      bf = bf_next;
    }
    promote(FM - 1, FN - 1, acc_prev);
    cur = nxt;
  }

  // ---- epilogue: lane owns row (m0 + wm*TM + 16i + lr), columns (nw0 + 16j + 4lg .. +3).
  // Returns a lower bound on the vector-memory operations this wave issued here: FM*FN
  // vector stores when the whole tile is inside D and rows need no group check, else 0.
  const bool interior = (GRP != GRP_CONTIG) && (OUT != OUT_F32_C || p.c_vec) && p.d_vec &&
                        tl.m0 + BM <= tl.m_valid && tl.n0 + BN <= p.n;
  char* Dg = (char*)p.d;
  const int esz = (OUT == OUT_BF16) ? 2 : 4;
  if (GRP == GRP_MASKED) Dg += (int64_t)g * p.d_gstride * esz;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = row0 + 16 * i;
    bool row_ok = row < tl.m_valid;
    if (GRP == GRP_CONTIG && row_ok) row_ok = p.grouped_layout[row] == g;
    if (!row_ok) continue;
    char* drow = Dg + (int64_t)row * p.ldd * esz;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = nw0 + 16 * j + 4 * lg;
      if (col >= p.n) continue;
      float o[4] = {fin[i][j][0], fin[i][j][1], fin[i][j][2], fin[i][j][3]};
      const bool full4 = col + 3 < p.n;
      if (OUT == OUT_F32_C) {
        const float* crow = p.c + (int64_t)row * p.ldc;
        if (full4 && p.c_vec) {
          const v4f cv = *(const v4f*)(crow + col);
          o[0] += cv.x; o[1] += cv.y; o[2] += cv.z; o[3] += cv.w;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (col + v < p.n) o[v] += crow[col + v];
        }
      }
      if (OUT == OUT_BF16) {
        unsigned short* dp = (unsigned short*)drow + col;
        const unsigned int w0 = pack_bf16x2(o[0], o[1]), w1 = pack_bf16x2(o[2], o[3]);
        if (full4 && p.d_vec) {
          *(v2u*)dp = (v2u){w0, w1};
        } else {
          const unsigned short h[4] = {(unsigned short)w0, (unsigned short)(w0 >> 16),
                                       (unsigned short)w1, (unsigned short)(w1 >> 16)};
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (col + v < p.n) dp[v] = h[v];
        }
      } else {
        float* dp = (float*)drow + col;
        if (full4 && p.d_vec) {
          *(v4f*)dp = (v4f){o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (col + v < p.n) dp[v] = o[v];
        }
      }
    }
  }
  return interior ? FM * FN : 0;
}

template <int BM, int BN, int WM, int WN, int SFM, int GRP, int OUT>
__global__ void __launch_bounds__(WM* WN * 64, 1) gemm_kernel(const GemmParams p) {
  using S = Shape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS_BYTES];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wn = wave % WN;
  int bid = blockIdx.x;
  if (p.xcd_remap) {  // workgroups are dealt round-robin to the 8 XCDs
    const int per = gridDim.x / 8;
    bid = (bid % 8) * per + bid / 8;
  }
  // next non-skipped tile at or after logical index t
  auto advance = [&](int& t, Tile& tl) -> bool {
    for (;; t += gridDim.x) {
      if (!get_tile<GRP, BM, BN>(p, t, tl)) return false;
      if (!tl.skip) return true;
    }
  };
  int t = bid;
  Tile cur;
  if (!advance(t, cur)) return;
  Loader<BM, BN, WM, WN> ld_cur, ld_next;
  make_loader<BM, BN, WM, WN, GRP>(p, cur, ld_cur);
  issue_stage(p, ld_cur, smem, 0, 0, wave, lane);
  int stage0 = 0;
  int vm_after = 0;
  for (;;) {
    Tile nxt;
    int tn = t + gridDim.x;
    const bool has_next = advance(tn, nxt);
    if (has_next) make_loader<BM, BN, WM, WN, GRP>(p, nxt, ld_next);
    if (SFM == SF_1D2D_F32) {
      // leading 16-column fragments of this wave that use the first weight-scale block
      const int ph = ((cur.n0 + wn * S::TN) & 127) >> 4;
      const int nf = min(S::FN, 8 - ph);
      switch (nf) {
#define DG_NF_CASE(X)                                                                                  \
  case X:                                                                                              \
    if constexpr (X <= S::FN)                                                                          \
      vm_after = gemm_tile<BM, BN, WM, WN, SFM, GRP, OUT, X>(p, smem, cur, ld_cur, has_next, ld_next,  \
                                                             stage0, vm_after, wave, lane);            \
    break;
        DG_NF_CASE(1) DG_NF_CASE(2) DG_NF_CASE(3) DG_NF_CASE(4)
        DG_NF_CASE(5) DG_NF_CASE(6) DG_NF_CASE(7) DG_NF_CASE(8)
#undef DG_NF_CASE
        default: break;
      }
    } else {
      vm_after = gemm_tile<BM, BN, WM, WN, SFM, GRP, OUT, S::FN>(p, smem, cur, ld_cur, has_next, ld_next,
                                                                stage0, vm_after, wave, lane);
    }
    if (!has_next) break;
    stage0 = (stage0 + p.sf_k) & 1;
    cur = nxt;
    ld_cur = ld_next;
    t = tn;
  }
}

// ------------------------------------------------------------------ dispatch
// The file is compiled once per tile shape with DG_TILE_ID set (so the kernel
// instantiations build in parallel) and once without it for the dispatch table.
template <int BM, int BN, int WM, int WN, int SFM, int GRP, int OUT>
static hipError_t launch_one(const GemmParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, SFM, GRP, OUT>), dim3(grid), dim3(WM * WN * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_tile(const GemmParams& p, int sfm, int grp, int out, int grid, hipStream_t s) {
#define DG_CASE(SF, G, O) \
  if (sfm == SF && grp == G && out == O) return launch_one<BM, BN, WM, WN, SF, G, O>(p, grid, s);
  DG_CASE(SF_1D2D_F32, GRP_DENSE, OUT_BF16)
  DG_CASE(SF_1D2D_F32, GRP_DENSE, OUT_F32)
  DG_CASE(SF_1D2D_F32, GRP_DENSE, OUT_F32_C)
  DG_CASE(SF_1D1D_F32, GRP_DENSE, OUT_BF16)
  DG_CASE(SF_1D1D_F32, GRP_DENSE, OUT_F32)
  DG_CASE(SF_1D1D_F32, GRP_DENSE, OUT_F32_C)
  DG_CASE(SF_1D1D_UE8M0, GRP_DENSE, OUT_BF16)
  DG_CASE(SF_1D1D_UE8M0, GRP_DENSE, OUT_F32)
  DG_CASE(SF_1D1D_UE8M0, GRP_DENSE, OUT_F32_C)
  if constexpr (BM <= 128) {
    DG_CASE(SF_1D2D_F32, GRP_CONTIG, OUT_BF16)
    DG_CASE(SF_1D2D_F32, GRP_CONTIG, OUT_F32)
    DG_CASE(SF_1D1D_F32, GRP_CONTIG, OUT_BF16)
    DG_CASE(SF_1D1D_UE8M0, GRP_CONTIG, OUT_BF16)
  }
  DG_CASE(SF_1D2D_F32, GRP_MASKED, OUT_BF16)
  DG_CASE(SF_1D2D_F32, GRP_MASKED, OUT_F32)
  DG_CASE(SF_1D1D_F32, GRP_MASKED, OUT_BF16)
  DG_CASE(SF_1D1D_UE8M0, GRP_MASKED, OUT_BF16)
  DG_CASE(SF_1D1D_UE8M0, GRP_MASKED, OUT_F32)
#undef DG_CASE
  return hipErrorInvalidValue;
}

#define DG_TILE_LAUNCHER(ID, BM, BN, WM, WN)                                                     \
  hipError_t launch_tile_##ID(const GemmParams& p, int sfm, int grp, int out, int grid, hipStream_t s) { \
    return launch_tile<BM, BN, WM, WN>(p, sfm, grp, out, grid, s);                               \
  }

#if defined(DG_TILE_ID)
#if DG_TILE_ID == 0
DG_TILE_LAUNCHER(0, 256, 224, 4, 2)
#elif DG_TILE_ID == 1
DG_TILE_LAUNCHER(1, 256, 256, 4, 2)
#elif DG_TILE_ID == 2
DG_TILE_LAUNCHER(2, 128, 224, 2, 2)
#elif DG_TILE_ID == 3
DG_TILE_LAUNCHER(3, 128, 256, 2, 2)
#elif DG_TILE_ID == 4
DG_TILE_LAUNCHER(4, 128, 128, 2, 2)
#elif DG_TILE_ID == 5
DG_TILE_LAUNCHER(5, 64, 128, 1, 2)
#elif DG_TILE_ID == 6
DG_TILE_LAUNCHER(6, 128, 192, 2, 2)
#elif DG_TILE_ID == 7
DG_TILE_LAUNCHER(7, 256, 192, 4, 2)
#elif DG_TILE_ID == 8
DG_TILE_LAUNCHER(8, 64, 32, 1, 1)
#endif
#else  // dispatch table

const TileCfg kTiles[kNumTiles] = {
    {256, 224, 4, 2}, {256, 256, 4, 2}, {128, 224, 2, 2}, {128, 256, 2, 2}, {128, 128, 2, 2},
    {64, 128, 1, 2},  {128, 192, 2, 2}, {256, 192, 4, 2}, {64, 32, 1, 1}};

#define DG_DECL(ID) hipError_t launch_tile_##ID(const GemmParams&, int, int, int, int, hipStream_t);
DG_DECL(0) DG_DECL(1) DG_DECL(2) DG_DECL(3) DG_DECL(4) DG_DECL(5) DG_DECL(6) DG_DECL(7) DG_DECL(8)
#undef DG_DECL

bool gemm_instantiated(int tile, int sfm, int grp, int out) {
  if (tile < 0 || tile >= kNumTiles) return false;
  if (sfm < 0 || sfm > 2 || out < 0 || out > 2) return false;
  if (grp == GRP_CONTIG) {
    if (kTiles[tile].bm > 128) return false;
    if (out == OUT_F32_C) return false;
    if (out == OUT_F32 && sfm != SF_1D2D_F32) return false;
    return true;
  }
  if (grp == GRP_MASKED) {
    if (out == OUT_F32_C) return false;
    if (out == OUT_F32 && sfm == SF_1D1D_F32) return false;
    return true;
  }
  return grp == GRP_DENSE;
}

int gemm_lds_bytes(int tile) {
  const TileCfg& t = kTiles[tile];
  return STAGES * (t.bm + t.bn) * BK;
}

hipError_t launch_gemm(const GemmParams& p, int tile, int sfm, int grp, int out, int grid,
                       hipStream_t stream) {
  if (!gemm_instantiated(tile, sfm, grp, out)) return hipErrorInvalidValue;
  switch (tile) {
    case 0: return launch_tile_0(p, sfm, grp, out, grid, stream);
    case 1: return launch_tile_1(p, sfm, grp, out, grid, stream);
    case 2: return launch_tile_2(p, sfm, grp, out, grid, stream);
    case 3: return launch_tile_3(p, sfm, grp, out, grid, stream);
    case 4: return launch_tile_4(p, sfm, grp, out, grid, stream);
    case 5: return launch_tile_5(p, sfm, grp, out, grid, stream);
    case 6: return launch_tile_6(p, sfm, grp, out, grid, stream);
    case 7: return launch_tile_7(p, sfm, grp, out, grid, stream);
    case 8: return launch_tile_8(p, sfm, grp, out, grid, stream);
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace dg
