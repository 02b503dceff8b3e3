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
#include <utility>

#include "dg_internal.h"

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
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
  static constexpr int AB_BYTES = (BM + BN) * BK;       // A rows, then B rows, 128 bytes each
  static constexpr int SA_OFF = AB_BYTES;               // activation scales of the K block (<= 1 KiB)
  static constexpr int SB_OFF = AB_BYTES + 1024;        // per-row weight scales of the K block (<= 1 KiB)
  static constexpr int STAGE_BYTES = AB_BYTES + 2048;
  static constexpr int TRASH_OFF = STAGES * STAGE_BYTES;  // 1 KiB sink for loads that are not needed
  static constexpr int LDS_BYTES = TRASH_OFF + 1024;
  static constexpr int LOADS = (BM + BN) / 8;           // 1 KiB row wave-loads per stage
  // wave-load slots per wave: every wave issues LPW per stage; slot q = wave + u*NW is a
  // row load for q < LOADS, the activation scales for q == LOADS, the per-row weight
  // scales for q == LOADS + 1, and a load into the trash region otherwise
  static constexpr int LPW = (LOADS + 2 + NW - 1) / NW;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(TN <= 128, "a wave's N range may touch at most two weight-scale blocks");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "rows are loaded 8 per wave-load");
  static_assert(BM <= 256 && BN <= 256, "one scale wave-load covers at most 256 rows");
};

struct Tile {
  int g;        // group
  int m0, n0;   // first row (within the group for masked) and first column
  int m_valid;  // rows < m_valid exist
  int kb0;      // K-grouped: the group's first 128-long K block
  int nkb;      // K blocks of this tile
  bool skip;
};

// gfx950's transposing LDS read: in each group of 16 lanes, lane 2r + h names an 8-byte row and
// lane 8h + c receives byte c of rows 0..7 of its half h (measured lane layout of
// ds_read_b64_tr_b8): 8 K values of one M (or N) column of an MN-major tile in one lane.
__device__ __forceinline__ v2i read_tr8(const uint8_t* smem, uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((DG_LDS v2i*)(smem + addr));
}

// LDS slot of 16-byte chunk c of stage row r is c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Wave-uniform read of kernel input that no launch writes (scales, group tables), through
// the constant address space: it becomes a scalar load, which is not counted in vmcnt, so
// using its value never waits for the HBM -> LDS copies in flight.
template <class T>
__device__ __forceinline__ T load_uniform(const T* base, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)base)[i];
}

// Persistent scheduler: logical tile index -> (group, m0, n0).
template <int GRP, int BM, int BN>
__device__ __forceinline__ bool get_tile(const GemmParams& p, int t, Tile& tl) {
  tl.skip = false;
  tl.kb0 = 0;
  tl.nkb = p.sf_k;
  if (GRP == GRP_KGROUP) {
    // K-grouped: the non-empty groups one after another, each walked like a dense problem
    const int per_group = p.num_m_tiles * p.num_n_tiles;
    const int gi = t / per_group;
    if (gi >= p.kg_count) return false;
    t -= gi * per_group;
    tl.g = p.kg_group[gi];
    tl.kb0 = p.kg_kb0[gi];
    tl.nkb = p.kg_nkb[gi];
    const int per_super = p.swizzle_m * p.num_n_tiles;
    const int sr = t / per_super;
    const int rem = t - sr * per_super;
    const int rows = min(p.swizzle_m, p.num_m_tiles - sr * p.swizzle_m);
    tl.m0 = (sr * p.swizzle_m + rem % rows) * BM;
    tl.n0 = (rem / rows) * BN;
    tl.m_valid = p.m;
    return true;
  }
  if (GRP == GRP_MASKED) {
    // Groups in order; within a group n tiles outer, m tiles inner, so the m tiles
    // that share a weight slice run next to each other.
    int base = 0;
    for (int g = 0; g < p.num_groups; ++g) {
      const int mg = clampi(load_uniform(p.masked_m, g), 0, p.m);
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
    const int g = load_uniform(p.grouped_layout, tl.m0);
    tl.g = g;
    tl.skip = g < 0 || g >= p.num_groups;
  }
  return true;
}

__device__ __forceinline__ unsigned int pack_bf16x2(float x, float y) {
  v2bf v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(unsigned int, v);
}

// Where a tile's stage loads come from (all wave-uniform).  Row wave-load q covers 8
// stage rows of 128 bytes: lane L fills LDS bytes [16L, 16L+16) = stage row
// r = 8q + L/8, slot L%8, which holds 16-byte chunk (L%8) ^ swz(r) of that row, and
// swz(8q + L/8) = (L/8) ^ (q & 1).  Rows past the end of A or B are not loaded (their
// LDS rows keep stale bytes, which only reach output rows or columns that are never
// stored).  The K block's scales are copied into the same stage:
//  * activation scales of rows m0..m0+BM-1 (FP32, or the UE8M0 word holding the
//    block), contiguous in the MN-major layout: lane L copies rows 4L..4L+3;
//  * per-row weight scales of columns n0..n0+BN-1 the same way, or, for 128x128
//    weight blocks, the (at most three) block scales the tile touches, 4 bytes each.
template <int BM, int BN, int WM, int WN>
struct Loader {
  const uint8_t* a_tile;  // row tile.m0 of A (this tile's group)
  const uint8_t* b_tile;  // row tile.n0 of B
  const uint8_t* sa;      // activation scale of row tile.m0, K block 0
  const uint8_t* sb;      // per-row: weight scale of row tile.n0, K block 0; 1d2d: block scale (n0/128, 0)
  int a_rows, b_rows;     // rows of A / B that exist from the tile start (MN-major: columns)
  int a_krows, b_krows;   // MN-major operands: K rows from the tile's first K row to the operand's end
  int sa_rows, sb_rows;   // scale entries that exist from the tile start (align4 padded)
  int sb_blocks;          // 1d2d: weight-scale blocks that exist from n0/128
};

template <int BM, int BN, int WM, int WN, int SFM, int GRP, int LAY = 0>
__device__ __forceinline__ void make_loader(const GemmParams& p, const Tile& tl, Loader<BM, BN, WM, WN>& ld) {
  const uint8_t* A = p.a + (GRP == GRP_MASKED ? (int64_t)tl.g * p.a_gstride : 0);
  const uint8_t* B = p.b + (GRP == GRP_CONTIG || GRP == GRP_MASKED ? (int64_t)tl.g * p.b_gstride : 0);
  // (K-grouped: the group's K range starts kb0 blocks into every row, and its scales kb0
  // scale rows into the [blocks, mn] scale arrays)
  const int64_t kofs = (GRP == GRP_KGROUP) ? (int64_t)tl.kb0 * BK : 0;
  ld.a_tile = A + (int64_t)tl.m0 * p.lda + kofs;
  ld.b_tile = B + (int64_t)tl.n0 * p.ldb + kofs;
  // MN-major operands (K rows of M or N bytes): the tile starts at K row kofs, column m0 / n0
  if (LAY & LAYOUT_A_MN) ld.a_tile = A + kofs * p.lda + tl.m0;
  if (LAY & LAYOUT_B_MN) ld.b_tile = B + kofs * p.ldb + tl.n0;
  ld.a_krows = p.k - (int)kofs;
  ld.b_krows = p.k - (int)kofs;
  ld.a_rows = p.m - tl.m0;  // m_max rows when masked
  ld.b_rows = p.n - tl.n0;
  const int64_t sfa_goff = (GRP == GRP_MASKED) ? (int64_t)tl.g * p.sfa_gstride
                           : (GRP == GRP_KGROUP ? (int64_t)tl.kb0 * p.sfa_stride : 0);
  const int64_t sfb_goff = (GRP == GRP_CONTIG || GRP == GRP_MASKED) ? (int64_t)tl.g * p.sfb_gstride
                           : (GRP == GRP_KGROUP ? (int64_t)tl.kb0 * p.sfb_stride : 0);
  ld.sa = (const uint8_t*)p.sfa + 4 * (sfa_goff + tl.m0);
  ld.sa_rows = (int)p.sfa_stride - tl.m0;
  if (SFM == SF_1D2D_F32) {
    const int blk0 = tl.n0 / 128;
    ld.sb = (const uint8_t*)p.sfb + 4 * (sfb_goff + (int64_t)blk0 * p.sfb_stride);
    ld.sb_blocks = (p.n + 127) / 128 - blk0;
    ld.sb_rows = 4;  // unused: 128x128 block scales are read with scalar loads
  } else {
    ld.sb = (const uint8_t*)p.sfb + 4 * (sfb_goff + tl.n0);
    ld.sb_rows = (int)p.sfb_stride - tl.n0;
  }
}

// Per-lane byte offsets of the buffer loads, fixed for the whole kernel.  A row wave-load
// covers 8 stage rows of 128 bytes: lane L fills LDS bytes [16L, 16L+16) = stage row
// 8q + L/8, slot L%8, which holds 16-byte chunk (L%8) ^ swz(row) of that row, and
// swz(8q + L/8) = (L/8) ^ (q & 1).  So the source offset is (L/8) * ld + 16 * chunk,
// with one variant per parity of q.
// The parity of q = wave + U * NW is the wave's own parity, flipped by U when NW is odd,
// so each wave keeps the offsets for its own parity ("same") and the other ("flip"), and
// every load picks one at compile time.  (Plain scalar members chosen at compile time: a
// runtime choice between members can turn into a memory access.)
struct LaneOffsets {
  uint32_t a_same, a_flip, b_same, b_flip;
  uint32_t a_rx0, a_rx1, b_rx0, b_rx1;  // row-XOR staging: parts whose key bit is 0 / 1
  uint32_t s;  // scale wave-loads: lane L copies 4-byte entries 4L..4L+3
};

// An MN-major operand 256 columns wide with 8 waves sits in its stage region row-XOR'd
// instead: K row r is stored whole at byte 256 r, its 16-byte chunk c at position c ^ key(r),
// key(r) = (r & 7) | (bit 5 of r) << 3.  Wave-load q fills K rows 4q .. 4q+3 and lane L
// copies chunk (L % 16) ^ key(r) of row r = 4q + L/16, so consecutive lanes read consecutive
// bytes of a K row.  With q = wave + 8U, r & 7 = 4 (wave & 1) + L/16 and bit 5 of r is U & 1,
// so a lane needs one offset per parity of U.  The 16 K rows one transposing read takes in a
// pass (8 per lane group, the two groups differing in bit 5) land on 16 different 4-bank groups.
template <int LAY, int W, int NW>
constexpr bool row_xor = LAY != 0 && W == 256 && NW == 8;
__device__ __forceinline__ uint32_t rx_lane_offset(int lane, int wave, int64_t ld, uint32_t ubit) {
  const uint32_t j = (uint32_t)lane >> 4, c = (uint32_t)lane & 15u;
  const uint32_t key = (4u * ((uint32_t)wave & 1u) + j) | (ubit << 3);
  return (4u * (uint32_t)wave + j) * (uint32_t)ld + 16u * (c ^ key);
}

// An operand stored MN-major (K rows of M or N bytes) sits in its stage region as 16-column
// strips of 128 rows x 16 bytes; K row k is stored at row position k ^ 8 * (bit 5 of k), which
// spreads the transposing fragment reads of the two lane groups served together over all banks.
// Wave-load q fills strip q/2, row positions 64 (q % 2) + [0, 64): lane L copies 16 bytes of K
// row 64 (q % 2) + (L ^ 8 * (bit 5 of L)), so the lane offset depends on the parity of q only.
__device__ __forceinline__ uint32_t mn_lane_row(int lane, uint32_t parity) {
  return 64u * parity + ((uint32_t)lane ^ ((((uint32_t)lane >> 5) & 1u) << 3));
}

template <int LAY = 0>
__device__ __forceinline__ LaneOffsets make_lane_offsets(const GemmParams& p, int wave, int lane) {
  LaneOffsets o;
  const uint32_t r = (uint32_t)lane >> 3, c = (uint32_t)lane & 7, w = (uint32_t)wave & 1;
  o.a_same = r * (uint32_t)p.lda + ((c ^ r ^ w) << 4);
  o.a_flip = r * (uint32_t)p.lda + ((c ^ r ^ w ^ 1u) << 4);
  o.b_same = r * (uint32_t)p.ldb + ((c ^ r ^ w) << 4);
  o.b_flip = r * (uint32_t)p.ldb + ((c ^ r ^ w ^ 1u) << 4);
  o.a_rx0 = o.a_rx1 = o.b_rx0 = o.b_rx1 = 0;
  if (LAY & LAYOUT_A_MN) {
    o.a_same = mn_lane_row(lane, w) * (uint32_t)p.lda;
    o.a_flip = mn_lane_row(lane, w ^ 1u) * (uint32_t)p.lda;
    o.a_rx0 = rx_lane_offset(lane, wave, p.lda, 0u);
    o.a_rx1 = rx_lane_offset(lane, wave, p.lda, 1u);
  }
  if (LAY & LAYOUT_B_MN) {
    o.b_same = mn_lane_row(lane, w) * (uint32_t)p.ldb;
    o.b_flip = mn_lane_row(lane, w ^ 1u) * (uint32_t)p.ldb;
    o.b_rx0 = rx_lane_offset(lane, wave, p.ldb, 0u);
    o.b_rx1 = rx_lane_offset(lane, wave, p.ldb, 1u);
  }
  o.s = (uint32_t)lane << 4;
  return o;
}

// Buffer descriptor over [base, base + bytes): loads at offsets >= bytes return zeros
// without touching memory, which is how rows past the end of A or B are handled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  // the values are wave-uniform; say so, so that the descriptor is built in scalar registers
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Enqueue part U of the HBM -> LDS copy of K block kb of a tile into stage s.  Wave-load
// slot q = wave + U * NW is a row load for q < LOADS, the activation scales for
// q == LOADS, the per-row weight scales for q == LOADS + 1, and otherwise an empty load
// (zero bytes: no memory access) into the trash region, so every wave runs the same
// branch-free instruction stream.  Which kind a slot is depends on the wave only in the
// last slot; all address arithmetic is on wave-uniform values and the only per-lane term
// is the fixed lane offset.
template <int U, int BM, int BN, int WM, int WN, int SFM, int LAY = 0>
__device__ __forceinline__ void issue_part(const GemmParams& p, const Loader<BM, BN, WM, WN>& ld, uint8_t* smem,
                                           int kb, int s, const int wave, const LaneOffsets lo) {
  using S = Shape<BM, BN, WM, WN>;
  static_assert((BM / 8) % S::NW == 0, "A and B wave-loads must split at a fixed slot");
  constexpr int UA = BM / 8 / S::NW;                         // slots U < UA fill A rows
  constexpr bool ALL_B = U >= UA && (S::NW - 1) + U * S::NW < S::LOADS;  // every wave loads B rows
  const int q = wave + U * S::NW;
  constexpr bool FLIP = (S::NW & 1) && (U & 1);  // parity of q differs from the wave's
  const uint8_t* base;
  int bytes;
  uint32_t voff;
  int dst;
  if constexpr (U < UA) {  // A rows 8q .. 8q+7 of the tile
    const int rem = ld.a_rows - 8 * q;
    base = ld.a_tile + (int64_t)(8 * q) * p.lda + kb * BK;
    bytes = rem > 0 ? min(rem, 8) * (int)p.lda - kb * BK : 0;
    voff = FLIP ? lo.a_flip : lo.a_same;
    if constexpr ((LAY & LAYOUT_A_MN) != 0 && row_xor<LAY & LAYOUT_A_MN, BM, S::NW>) {
      // K rows kb*128 + 4q .. of all BM columns; the range runs to the operand's end as for strips
      base = ld.a_tile + (int64_t)kb * BK * p.lda;
      bytes = (int)((((int64_t)(ld.a_krows - kb * BK - 1)) * p.lda + ld.a_rows + 15) & ~(int64_t)15);
      voff = ((U & 1) ? lo.a_rx1 : lo.a_rx0) + (uint32_t)(32 * U) * (uint32_t)p.lda;
    } else if constexpr ((LAY & LAYOUT_A_MN) != 0) {
      // strip q/2: K rows kb*128.. of columns 16 (q/2).. ; the range ends with the 16-byte
      // granule holding the operand's last byte (columns past the end only feed outputs that
      // are never stored; a range ending inside a copy would drop its valid dwords)
      base = ld.a_tile + (int64_t)kb * BK * p.lda + 16 * (q >> 1);
      bytes = (int)((((int64_t)(ld.a_krows - kb * BK - 1)) * p.lda + ld.a_rows - 16 * (q >> 1) + 15) & ~(int64_t)15);
    }
    dst = s * S::STAGE_BYTES + q * 1024;
  } else {
    // B rows 8q - BM .. 8q - BM + 7 of the tile
    const int r0 = 8 * q - BM;
    const int rem = ld.b_rows - r0;
    const uint8_t* b_base = ld.b_tile + (int64_t)r0 * p.ldb + kb * BK;
    int b_bytes = rem > 0 ? min(rem, 8) * (int)p.ldb - kb * BK : 0;
    uint32_t b_voff = FLIP ? lo.b_flip : lo.b_same;
    if constexpr ((LAY & LAYOUT_B_MN) != 0 && row_xor<LAY & LAYOUT_B_MN, BN, S::NW>) {
      constexpr int UB = U - UA;  // B row loads q - BM/8 = wave + 8 UB
      b_base = ld.b_tile + (int64_t)kb * BK * p.ldb;
      b_bytes = (int)((((int64_t)(ld.b_krows - kb * BK - 1)) * p.ldb + ld.b_rows + 15) & ~(int64_t)15);
      b_voff = ((UB & 1) ? lo.b_rx1 : lo.b_rx0) + (uint32_t)(32 * UB) * (uint32_t)p.ldb;
    } else if constexpr ((LAY & LAYOUT_B_MN) != 0) {
      const int st = (q - BM / 8) >> 1;  // (BM / 8 is even: the parity of q is the strip half)
      b_base = ld.b_tile + (int64_t)kb * BK * p.ldb + 16 * st;
      b_bytes = (int)((((int64_t)(ld.b_krows - kb * BK - 1)) * p.ldb + ld.b_rows - 16 * st + 15) & ~(int64_t)15);
    }
    if constexpr (ALL_B) {
      base = b_base;
      bytes = b_bytes;
      voff = b_voff;
      dst = s * S::STAGE_BYTES + q * 1024;
    } else {
      // scale parts: 4-byte entries, K block kb at kb * stride (FP32) or (kb / 4) * stride
      // (UE8M0 words); entries exist up to the padded (multiple of 4) scale length
      const int64_t kb_row = (SFM == SF_1D1D_UE8M0) ? (kb >> 2) : kb;
      const bool is_row = q < S::LOADS;
      const bool is_sa = q == S::LOADS;
      const bool is_sb = (SFM != SF_1D2D_F32) && q == S::LOADS + 1;
      const uint8_t* sa_base = ld.sa + 4 * kb_row * p.sfa_stride;
      const uint8_t* sb_base = ld.sb + 4 * kb_row * p.sfb_stride;
      const int sa_bytes = 4 * max(0, min(ld.sa_rows, BM));
      const int sb_bytes = 4 * max(0, min(ld.sb_rows, BN));
      base = is_row ? b_base : (is_sa ? sa_base : sb_base);
      bytes = is_row ? b_bytes : (is_sa ? sa_bytes : (is_sb ? sb_bytes : 0));
      voff = is_row ? b_voff : lo.s;
      dst = is_row ? s * S::STAGE_BYTES + q * 1024
                   : (is_sa ? s * S::STAGE_BYTES + S::SA_OFF
                            : (is_sb ? s * S::STAGE_BYTES + S::SB_OFF : S::TRASH_OFF));
    }
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), (DG_LDS void*)(smem + dst), 16, voff, 0, 0, 0);
}

template <int BM, int BN, int WM, int WN, int SFM, int LAY, int... Us>
__device__ __forceinline__ void issue_parts(const GemmParams& p, const Loader<BM, BN, WM, WN>& ld, uint8_t* smem,
                                            int kb, int s, const int wave, const LaneOffsets lo,
                                            std::integer_sequence<int, Us...>) {
  (issue_part<Us, BM, BN, WM, WN, SFM, LAY>(p, ld, smem, kb, s, wave, lo), ...);
}

// The whole copy of K block kb into stage s at once (prologue and tile hand-over).
template <int BM, int BN, int WM, int WN, int SFM, int LAY = 0>
__device__ __forceinline__ void issue_stage(const GemmParams& p, const Loader<BM, BN, WM, WN>& ld, uint8_t* smem,
                                            int kb, int s, const int wave, const LaneOffsets lo) {
  using S = Shape<BM, BN, WM, WN>;
  issue_parts<BM, BN, WM, WN, SFM, LAY>(p, ld, smem, kb, s, wave, lo, std::make_integer_sequence<int, S::LPW>{});
}

// Wait until at most N vector-memory operations of this wave are outstanding and no
// LDS operation is, then synchronise the workgroup.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}

// One output tile: the K loop over 128-long blocks, then the epilogue.
//  * K block 0 of this tile (and K block 1 when `pre2`) is already in flight into
//    stage `stage0` (and the other stage).
//  * `vm_after` is a lower bound on this wave's vector-memory operations issued after
//    those prefetches (the previous tile's epilogue stores), so the first waits can
//    leave the stores in flight.
//  * During the last K block the first stage of the next tile is enqueued; after it,
//    once every wave has read the last stage, the next tile's second stage too.
// Returns the number of vector-memory operations this wave's epilogue issued (a lower
// bound) and sets `next_pre2`.
template <int BM, int BN, int WM, int WN, int SFM, int GRP, int OUT, int NF, int LAY = 0>
__device__ __forceinline__ int gemm_tile(const GemmParams& p, uint8_t* smem, const Tile& tl,
                                         const Loader<BM, BN, WM, WN>& ld, const bool has_next,
                                         const Loader<BM, BN, WM, WN>& ld_next, const int nkb_next, const int stage0,
                                         const bool pre2, const int vm_after, bool& next_pre2, const int wave,
                                         const int lane, const LaneOffsets lo) {
  using S = Shape<BM, BN, WM, WN>;
  constexpr int FM = S::FM, FN = S::FN, TM = S::TM, TN = S::TN;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lg = lane >> 4;
  const int nkb = tl.nkb;
  const int g = tl.g;
  const int row0 = tl.m0 + wm * TM + lr;  // lane's row in fragment 0
  const int nw0 = tl.n0 + wn * TN;        // wave's first column
  // 1d2d: the (at most two) weight-scale blocks of the wave's N range
  const int nb = (p.n + 127) / 128;
  const int blk0 = min(nw0 / 128, nb - 1), blk1 = min(nw0 / 128 + 1, nb - 1);

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
  // MN-major strips: lane 2b + h of lane group lg reads 8 bytes (columns 8h..) of the row
  // position holding K row 32 lg + 8 r + b (read r = 0 at mn_lo, r = 1 at mn_hi, r = 2 and 3
  // 16 rows further)
  const int l16 = lane & 15, flip = lg & 1;
  const uint32_t mn_lo = (uint32_t)(16 * (32 * lg + 8 * flip + (l16 >> 1)) + 8 * (l16 & 1));
  const uint32_t mn_hi = (uint32_t)(16 * (32 * lg + 8 * (flip ^ 1) + (l16 >> 1)) + 8 * (l16 & 1));
  // row-XOR regions: lane 2b + h of lane group lg reads 8 bytes (columns 8h..) of K rows
  // 32 lg + b + {0, 8, 16, 24}, whose XOR key is the same: b | (lg & 1) << 3
  const uint32_t rx_lo = (uint32_t)((32 * lg + (l16 >> 1)) * 256 + 8 * (l16 & 1));
  const uint32_t rx_key = (uint32_t)(16 * ((l16 >> 1) | ((lg & 1) << 3)));
  constexpr bool RXA = (LAY & LAYOUT_A_MN) != 0 && row_xor<LAY & LAYOUT_A_MN, BM, S::NW>;
  constexpr bool RXB = (LAY & LAYOUT_B_MN) != 0 && row_xor<LAY & LAYOUT_B_MN, BN, S::NW>;

  // One K block.  SPREAD: the copy of K block kb+1 of this tile into the other stage goes
  // out spread evenly over the block's MFMAs (the memory pipe is the scarcest unit).
  // Otherwise the block issues no loads, except that the last block of a tile starts by
  // enqueueing the next tile's first K block into the free stage.
  auto run_block = [&]<bool SPREAD>(const int kb) {
    const int s = (stage0 + kb) & 1;
    // stage s has landed everywhere and nobody still reads stage s^1
    if ((kb == 0 || (kb == 1 && pre2)) && vm_after >= FM * FN) wait_and_barrier<FM * FN>();
    else wait_and_barrier<0>();
    if (!SPREAD && kb + 1 >= nkb && has_next) issue_stage<BM, BN, WM, WN, SFM, LAY>(p, ld_next, smem, 0, s ^ 1, wave, lo);
    // slot U goes out just before MFMA number U * FM * FN / LPW of the block
    auto issue_before = [&]<int U>(const int t) {
      if constexpr (SPREAD) {
        if ((U * FM * FN) / S::LPW == t) issue_part<U, BM, BN, WM, WN, SFM, LAY>(p, ld, smem, kb + 1, s ^ 1, wave, lo);
      }
    };
    auto issue_all_before = [&]<int... Us>(const int t, std::integer_sequence<int, Us...>) {
      (issue_before.template operator()<Us>(t), ...);
    };
    const uint8_t* st = smem + s * S::STAGE_BYTES;
    auto read_frag = [&](int row) -> v8i {
      const uint8_t* rp = st + row * BK;
      const v4i lo4 = *(const v4i*)(rp + off_lo);
      const v4i hi4 = *(const v4i*)(rp + off_hi);
      return (v8i){lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
    };
    // MN-major region at byte `region`: fragment of the 16 columns of strip `strip`, four
    // transposing reads of 8 K each (lane group lg holds K [32 lg, +32), as the K-major reads)
    auto read_frag_mn = [&](int region, int strip) -> v8i {
      const uint32_t a0 = (uint32_t)(s * S::STAGE_BYTES + region + strip * 2048) + mn_lo;
      const uint32_t a1 = (uint32_t)(s * S::STAGE_BYTES + region + strip * 2048) + mn_hi;
      const v2i x0 = read_tr8(smem, a0), x1 = read_tr8(smem, a1);
      const v2i x2 = read_tr8(smem, a0 + 256), x3 = read_tr8(smem, a1 + 256);
      return (v8i){x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
    };
    // row-XOR region at byte `region`: fragment of the 16 columns starting at byte c16 of the
    // rows, four transposing reads 8 K rows apart
    auto read_frag_rx = [&](int region, int c16) -> v8i {
      // (the key is re-read at each use, so the compiler computes each fragment's address where
      // it is needed instead of keeping one register per fragment live through the loop)
      uint32_t key = rx_key;
      asm volatile("" : "+v"(key));
      const uint32_t a = (uint32_t)(s * S::STAGE_BYTES + region) + rx_lo + ((uint32_t)c16 ^ key);
      const v2i x0 = read_tr8(smem, a), x1 = read_tr8(smem, a + 2048);
      const v2i x2 = read_tr8(smem, a + 4096), x3 = read_tr8(smem, a + 6144);
      return (v8i){x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
    };
    // fragments needed by the first MFMA first, so it waits for as few reads as possible
    // (the K-major reads are written out at each use: routing them through a helper that also
    // holds the MN-major form costs the K-grouped kernel about 45 registers)
    v8i af[FM];
    v8i bf;
    if constexpr (RXB) bf = read_frag_rx(BM * BK, wn * TN);
    else if constexpr ((LAY & LAYOUT_B_MN) != 0) bf = read_frag_mn(BM * BK, (wn * TN) / 16);
    else bf = read_frag(BM + wn * TN + lr);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (RXA) af[i] = read_frag_rx(0, wm * TM + 16 * i);
      else if constexpr ((LAY & LAYOUT_A_MN) != 0) af[i] = read_frag_mn(0, (wm * TM) / 16 + i);
      else af[i] = read_frag(wm * TM + 16 * i + lr);
    }

    // promotion factors for this block: activation scales from the stage's scale region,
    // 128x128 weight-block scales (two per wave at most) by scalar loads
    float sb_blk0 = 0.f, sb_blk1 = 0.f;
    if (SFM == SF_1D2D_F32) {
      const float* sbg = (const float*)p.sfb + (GRP != GRP_DENSE ? (int64_t)g * p.sfb_gstride : 0);
      sb_blk0 = load_uniform(sbg, __builtin_amdgcn_readfirstlane(blk0 * (int)p.sfb_stride + kb));
      if (NF < FN) sb_blk1 = load_uniform(sbg, __builtin_amdgcn_readfirstlane(blk1 * (int)p.sfb_stride + kb));
    }
    float s0[FM], s1[FM];
    int ea[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const float* sa_l = (const float*)(st + S::SA_OFF);
      const float sa = sa_l[wm * TM + 16 * i + lr];
      if (SFM == SF_1D2D_F32) {
        s0[i] = sa * sb_blk0;
        s1[i] = (NF < FN) ? sa * sb_blk1 : s0[i];
      } else if (SFM == SF_1D1D_F32) {
        s0[i] = s1[i] = sa;
      } else {
        ea[i] = (int)((__float_as_uint(sa) >> (8 * (kb & 3))) & 0xFFu);
      }
    }
    auto weight_code = [&](int j) -> int {  // UE8M0 code of the weight row the lane feeds in fragment j
      const unsigned int* sbw = (const unsigned int*)(st + S::SB_OFF);
      return (int)((sbw[wn * TN + 16 * j + lr] >> (8 * (kb & 3))) & 0xFFu);
    };
    auto promote = [&](int i, int j, const v4f& acc) {
      if (SFM == SF_1D2D_F32) {
        const float sc = (j < NF) ? s0[i] : s1[i];  // compile-time choice
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] = __builtin_fmaf(sc, acc[v], fin[i][j][v]);
      } else if (SFM == SF_1D1D_F32) {
        const v4f w = *(const v4f*)(st + S::SB_OFF + 4 * (wn * TN + 16 * j + 4 * lg));
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] = __builtin_fmaf(s0[i] * w[v], acc[v], fin[i][j][v]);
      } else {
        // UE8M0: the MFMA already multiplied by 2^(ea-127) * 2^(eb-127)
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] += acc[v];
      }
      // keep the promotion at this point of the instruction stream (the compiler would
      // otherwise gather all of a block's promotions after its MFMAs, keeping every
      // partial alive at once)
      asm volatile("" : "+v"(fin[i][j][0]), "+v"(fin[i][j][1]), "+v"(fin[i][j][2]), "+v"(fin[i][j][3]));
    };
    // Software pipeline: the partial of MFMA t is promoted while MFMA t+1 runs, and each
    // step (loads, MFMA, promotion of the previous partial) is pinned in program order.
    // The weight fragment is the first MFMA operand, so the lane owns row lr and
    // columns 4*lg + v of each 16x16 block.
    v4f acc_prev = zero;
    int eb = (SFM == SF_1D1D_UE8M0) ? weight_code(0) : 0;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      v8i bf_next = bf;
      int eb_next = eb;
      if (j + 1 < FN) {
        if constexpr (RXB) bf_next = read_frag_rx(BM * BK, wn * TN + 16 * (j + 1));
        else if constexpr ((LAY & LAYOUT_B_MN) != 0) bf_next = read_frag_mn(BM * BK, (wn * TN) / 16 + j + 1);
        else bf_next = read_frag(BM + wn * TN + 16 * (j + 1) + lr);
        if (SFM == SF_1D1D_UE8M0) eb_next = weight_code(j + 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        issue_all_before(j * FM + i, std::make_integer_sequence<int, S::LPW>{});
        v4f acc;
        if (SFM == SF_1D1D_UE8M0)
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, eb, 0, ea[i]);
        else
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, 0, 0, 0);
        asm volatile("" : "+v"(acc));  // the MFMA stays in this step
        if (i > 0) promote(i - 1, j, acc_prev);
        else if (j > 0) promote(FM - 1, j - 1, acc_prev);
        acc_prev = acc;
        __builtin_amdgcn_sched_barrier(0);
      }
      bf = bf_next;
      eb = eb_next;
    }
    promote(FM - 1, FN - 1, acc_prev);
  };

  // K block 0 prefetches block 1 unless the previous tile already did; the last block
  // prefetches the next tile's first block
  if (pre2 || nkb == 1) run_block.template operator()<false>(0);
  else run_block.template operator()<true>(0);
  for (int kb = 1; kb + 1 < nkb; ++kb) run_block.template operator()<true>(kb);
  if (nkb >= 2) run_block.template operator()<false>(nkb - 1);

  // the next tile's second stage goes into the stage this tile read last, once every
  // wave is done with it
  next_pre2 = false;
  if (has_next && nkb >= 2 && nkb_next >= 2) {
    wait_and_barrier<63>();
    issue_stage<BM, BN, WM, WN, SFM, LAY>(p, ld_next, smem, 1, (stage0 + nkb - 1) & 1, wave, lo);
    next_pre2 = true;
  }

  // ---- epilogue: lane owns row (m0 + wm*TM + 16i + lr), columns (nw0 + 16j + 4lg .. +3).
  // Returns a lower bound on the vector-memory operations this wave issued here: FM*FN
  // vector stores when the whole tile is inside D and rows need no group check, else 0.
  const bool interior = (GRP != GRP_CONTIG) && (OUT != OUT_F32_C || p.c_vec) && p.d_vec &&
                        tl.m0 + BM <= tl.m_valid && tl.n0 + BN <= p.n;
  char* Dg = (char*)p.d;
  const int esz = (OUT == OUT_BF16) ? 2 : 4;
  if (GRP == GRP_MASKED || GRP == GRP_KGROUP) Dg += (int64_t)g * p.d_gstride * esz;
  const float* Cg = p.c + (GRP == GRP_KGROUP ? (int64_t)g * p.c_gstride : 0);
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
        const float* crow = Cg + (int64_t)row * p.ldc;
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

template <int BM, int BN, int WM, int WN, int SFM, int GRP, int OUT, int LAY = 0>
__global__ void __launch_bounds__(WM* WN * 64, 1) gemm_kernel(const GemmParams p) {
  using S = Shape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS_BYTES];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wn = wave % WN;
  const LaneOffsets lo = make_lane_offsets<LAY>(p, wave, lane);
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
  make_loader<BM, BN, WM, WN, SFM, GRP, LAY>(p, cur, ld_cur);
  issue_stage<BM, BN, WM, WN, SFM, LAY>(p, ld_cur, smem, 0, 0, wave, lo);
  int stage0 = 0;
  int vm_after = 0;
  bool pre2 = false;
  for (;;) {
    Tile nxt;
    int tn = t + gridDim.x;
    const bool has_next = advance(tn, nxt);
    if (has_next) make_loader<BM, BN, WM, WN, SFM, GRP, LAY>(p, nxt, ld_next);
    const int nkb_next = has_next ? nxt.nkb : 0;
    bool next_pre2 = false;
    if (SFM == SF_1D2D_F32) {
      // leading 16-column fragments of this wave that use the first weight-scale block
      const int ph = ((cur.n0 + wn * S::TN) & 127) >> 4;
      const int nf = min(S::FN, 8 - ph);
      switch (nf) {
#define DG_NF_CASE(X)                                                                                   \
  case X:                                                                                               \
    if constexpr (X <= S::FN)                                                                           \
      vm_after = gemm_tile<BM, BN, WM, WN, SFM, GRP, OUT, X, LAY>(p, smem, cur, ld_cur, has_next, ld_next, \
                                                             nkb_next, stage0, pre2, vm_after,          \
                                                             next_pre2, wave, lane, lo);                \
    break;
        DG_NF_CASE(1) DG_NF_CASE(2) DG_NF_CASE(3) DG_NF_CASE(4)
        DG_NF_CASE(5) DG_NF_CASE(6) DG_NF_CASE(7) DG_NF_CASE(8)
#undef DG_NF_CASE
        default: break;
      }
    } else {
      vm_after = gemm_tile<BM, BN, WM, WN, SFM, GRP, OUT, S::FN, LAY>(p, smem, cur, ld_cur, has_next, ld_next,
                                                                     nkb_next, stage0, pre2, vm_after, next_pre2,
                                                                     wave, lane, lo);
    }
    if (!has_next) break;
    stage0 = (stage0 + cur.nkb) & 1;
    pre2 = next_pre2;
    cur = nxt;
    ld_cur = ld_next;
    t = tn;
  }
}

// ------------------------------------------------------------------ dispatch
// The file is compiled once per tile shape with DG_TILE_ID set (so the kernel
// instantiations build in parallel) and once without it for the dispatch table.
template <int BM, int BN, int WM, int WN, int SFM, int GRP, int OUT, int LAY = 0>
static hipError_t launch_one(const GemmParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, SFM, GRP, OUT, LAY>), dim3(grid), dim3(WM * WN * 64), 0,
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
  if constexpr (BN >= 224) {
    // K-grouped: NT, or both operands stored K-outermost (TN, the weight-gradient storage; on the
    // 224-wide tiles, and on 256x256, where both operands are row-XOR staged)
    if (sfm == SF_1D1D_F32 && grp == GRP_KGROUP && out == OUT_F32_C) {
      if constexpr (BN == 224 || (BM == 256 && BN == 256)) {
        if (p.layout == (LAYOUT_A_MN | LAYOUT_B_MN))
          return launch_one<BM, BN, WM, WN, SF_1D1D_F32, GRP_KGROUP, OUT_F32_C, LAYOUT_A_MN | LAYOUT_B_MN>(p, grid, s);
      }
      if (p.layout == 0) return launch_one<BM, BN, WM, WN, SF_1D1D_F32, GRP_KGROUP, OUT_F32_C>(p, grid, s);
      return hipErrorInvalidValue;
    }
  }
  if (p.layout != 0) return hipErrorInvalidValue;
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

bool gemm_instantiated(int tile, int sfm, int grp, int out, int layout) {
  if (tile < 0 || tile >= kNumTiles) return false;
  if (sfm < 0 || sfm > 2 || out < 0 || out > 2) return false;
  if (grp == GRP_KGROUP) {
    if (layout == (LAYOUT_A_MN | LAYOUT_B_MN))
      return sfm == SF_1D1D_F32 && out == OUT_F32_C &&
             (kTiles[tile].bn == 224 || (kTiles[tile].bm == 256 && kTiles[tile].bn == 256));
    return layout == 0 && sfm == SF_1D1D_F32 && out == OUT_F32_C && kTiles[tile].bn >= 224;
  }
  if (layout != 0) return false;
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
  if (!gemm_instantiated(tile, sfm, grp, out, p.layout)) return hipErrorInvalidValue;
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
