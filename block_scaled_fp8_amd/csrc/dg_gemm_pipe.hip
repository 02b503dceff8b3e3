// Deep-pipelined block-scaled FP8 GEMM main loop for gfx950 (MI355X, CDNA4): dense and
// contiguous-grouped problems with K >= 256, masked-grouped problems with K >= 384.
//
// Computes D = C + A . B^T exactly as the kernels in dg_gemm.hip do (E4M3 operands, one
// activation scale per row and 128-long K block, weight scales per 128x128 block or per
// row; each 128-K block's partial product promoted into an FP32 accumulator as
// final += scale_a * scale_b * partial: page "02 · DeepGEMM 技术解析" §2.2, page
// "第13章 DeepGEMM" §13.3 algorithm box).  What differs is how the work is pipelined:
//
//  * LDS holds three A stages and two B stages (256x224 tile: 96 + 56 KiB).  During K
//    block g the copy of A block g+2 streams in, spread over the block's MFMAs; B block
//    g+2 goes out in one burst right after the block's single workgroup barrier.  Every
//    copy therefore has at least one full K block of time to land, and A (the larger
//    operand) about two.
//  * The barrier sits at the start of the block's last 16-column group, after the last
//    LDS read of the block's B stage: it certifies both that block g+1 has landed (each
//    wave first waits for its own copies with an explicit vmcnt) and that B stage g may
//    be overwritten.  Right after it every wave reads block g+1's first B fragment and,
//    one after each of its last MFMAs, the A fragments of block g+1, so the next block
//    starts with its operands already in registers instead of a burst of LDS reads.
//  * Promotion runs two MFMAs behind: the FMAs after MFMA t consume the partial of
//    MFMA t-2, which has finished by then, so no wave stalls on a matrix result; the
//    scale of a partial is the one of its own K block, also across block boundaries.
//  * LDS fragment reads use one per-lane base per operand half plus immediate offsets,
//    so the inner loop spends no VALU on addresses.
//  * The 16-column fragments of a wave that straddle two 128-wide weight-scale blocks
//    take the second block's scale from a compile-time split chosen once per tile
//    (page "02 · DeepGEMM 技术解析" §2.3).
//  * FP4 (E2M1) weights (page "第13章 DeepGEMM" §13.5) go into the same scaled MFMA as the
//    FP8 activations, which takes mixed operand formats; a weight row then holds 64 bytes per
//    K block, and its four power-of-two scales per block (one per 32 K) are applied by the
//    matrix unit, lane group g supplying the scale of K [32g, 32g+32).
#include <utility>

#include "dg_internal.h"

namespace dg {
namespace pipe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
#define DG_LDS __attribute__((address_space(3)))

constexpr int BK = 128;  // K values per scale block and per MFMA
constexpr int NA = 3;    // A stages

// NB_: B stages (2 for dense and contiguous problems; masked problems, which stream their
// weights from HBM with little reuse, keep 3 in flight; up to 4 are supported)
template <int BM, int BN, int WM, int WN, int SFM, int NB_ = 2>
struct Geo {
  static constexpr bool FP4B = SFM == SF_FP4_UE8M0;
  static constexpr int BKB = FP4B ? BK / 2 : BK;  // bytes of a weight row per K block
  static constexpr int NB = NB_;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int A_SLOT = BM * BK, B_SLOT = BN * BKB;
  static constexpr int SA_SLOT = (BM * 4 + 1023) / 1024 * 1024;
  static constexpr int SB_SLOT = (SFM == SF_1D2D_F32) ? 0 : (BN * 4 + 1023) / 1024 * 1024;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = A_OFF + NA * A_SLOT;
  static constexpr int SA_OFF = B_OFF + NB * B_SLOT;
  static constexpr int SB_OFF = SA_OFF + NA * SA_SLOT;
  static constexpr int TRASH_OFF = SB_OFF + NB * SB_SLOT;  // 1 KiB sink for padding copies
  static constexpr int LDS_BYTES = TRASH_OFF + 1024;
  static constexpr int A_ROWL = BM / 8;  // 1 KiB wave-loads of A rows per block
  static constexpr int B_ROWL = BN * BKB / 1024;
  // wave-loads per wave and block: A rows + activation scales; B rows (+ per-row weight scales)
  static constexpr int LA = (A_ROWL + 1 + NW - 1) / NW;
  static constexpr int LB = (B_ROWL + (SFM == SF_1D2D_F32 ? 0 : 1) + NW - 1) / NW;
  static constexpr int STEPS = FM * FN;
  static constexpr int TB = (FN - 1) * FM;  // step that holds the barrier
  static_assert(NW % 2 == 0, "the swizzle parity of a wave's copies must not depend on the copy index");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tiles are made of 16x16 fragments");
  static_assert(TN <= 128, "a wave's N range may touch at most two weight-scale blocks");
  static_assert(BM <= 256 && BN <= 256, "one scale wave-load covers at most 256 rows");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(TB >= LA, "the A copies are spread over the steps before the barrier");
  static_assert(NB >= 2 && NB <= 4, "B stages");
};

// LDS slot of 16-byte chunk c of row r (rows counted within an operand stage) is
// c ^ swz(r).  gfx950's LDS has 64 four-byte banks; a 16-byte read (ds_read_b128) is served
// 16 lanes at a time, and a probe of every lane pair on the box showed which 16: lanes whose
// index has the same bit 5 and the same parity of bits 2..4 (lanes 0-3, 12-15, 20-23 and 24-27
// go together).  Those 16 lanes must touch 16 different 16-byte bank groups.  An FP8 fragment
// read (chunks 2g and 2g + 1 of rows r..r+15 in lane group g) is conflict-free under swz;
// next to FP4 weights the activation reads chunks g and g + 4, which swz4a keeps apart.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz4a(int r) { return (r & 7) ^ (((r >> 3) & 1) << 1); }

template <class T>
__device__ __forceinline__ T load_uniform(const T* base, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)base)[i];
}

__device__ __forceinline__ unsigned int pack_bf16x2(float x, float y) {
  v2bf v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(unsigned int, v);
}

// Buffer descriptor over [base, base + bytes): reads at offsets >= bytes return zeros
// without touching memory (rows past the end of A or B, padding copies).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ void copy_to_lds(const void* base, int bytes, uint32_t voff, uint8_t* smem, int dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), (DG_LDS void*)(smem + dst), 16, voff, 0, 0, 0);
}

typedef int v2i __attribute__((ext_vector_type(2)));

// gfx950's transposing LDS read: in each group of 16 lanes, lane 2r + h names an 8-byte row
// (r = 0..7, h = 0..1) and lane 8h + c receives byte c of rows 0..7 of its half h, so eight
// bytes that sit one per row come back in one lane (measured lane layout of
// ds_read_b64_tr_b8).  With rows = 8 consecutive K of an MN-major tile and the 16 bytes of a
// row pair = 16 consecutive M, lane l gets 8 consecutive K of row l: an MFMA fragment piece.
__device__ __forceinline__ v2i read_tr8(const uint8_t* smem, uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((DG_LDS v2i*)(smem + addr));
}

// Keep a promoted fragment at this point of the instruction stream: its FMAs are pure
// arithmetic that the compiler would otherwise sink to the end of the block, keeping every
// block partial alive at once.
__device__ __forceinline__ void pin(float (&f)[4]) {
  asm volatile("" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]));
}

// A copy of v that the compiler cannot compute earlier: per-lane values derived from it stay
// where they are used (the epilogue) instead of being hoisted to the kernel start and held
// in registers through the whole main loop.
__device__ __forceinline__ int fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most N vector-memory operations of this wave are outstanding and no
// LDS or scalar-memory operation is, then synchronise the workgroup.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}

// Output tile t of the workgroup's persistent walk.
//  * Dense: super-rows of swizzle_m m tiles, walked column by column, so the tiles that run
//    at the same time share A and B rows.
//  * Contiguous groups (page "02 · DeepGEMM 技术解析" §5.1): the dense walk over all rows;
//    a tile's group is the one of its first row.  A tile whose first row is padding (or
//    names no group) gets no rows: its copies are empty, it issues no MFMAs and stores
//    nothing.  The rows of a tile whose last row is in another group than its first (the
//    padding at the end of a group's last block) are checked one by one when stored.
//  * Masked (page "02 · DeepGEMM 技术解析" §5.2): only the tiles holding valid rows exist.
//    Groups in order; within a group n tiles outer and m tiles inner, so the m tiles that
//    read the same weight slice run next to each other.  masked_m is read on the device and
//    clamped to [0, M_max].
struct TilePos {
  int g;       // group (contiguous, masked)
  int m0, n0;  // first row (within the group) and first column
  int mv;      // rows that exist: M (dense, contiguous; 0 for a skipped contiguous tile) or
               // the group's valid rows (masked)
  bool valid;  // false past the last tile: its copies are empty
  bool chk;    // contiguous: store only the rows whose group is g
};

template <int BM, int BN, int GRP>
__device__ __forceinline__ TilePos tile_pos(const GemmParams& p, int t) {
  TilePos r;
  r.g = 0;
  r.chk = false;
  if (GRP == GRP_MASKED) {
    r.valid = false;
    r.m0 = r.n0 = r.mv = 0;
    int base = 0;
    for (int g = 0; g < p.num_groups; ++g) {
      const int mg = min(max(load_uniform(p.masked_m, g), 0), p.m);
      const int mt = (mg + BM - 1) / BM;
      const int cnt = mt * p.num_n_tiles;
      if (t < base + cnt) {
        const int loc = t - base;
        r.g = g;
        r.n0 = (loc / mt) * BN;
        r.m0 = (loc % mt) * BM;
        r.mv = mg;
        r.valid = true;
        break;
      }
      base += cnt;
    }
    return r;
  }
  r.valid = t < p.total_tiles;
  if (!r.valid) t = 0;
  const int per_super = p.swizzle_m * p.num_n_tiles;
  const int sr = t / per_super;
  const int rem = t - sr * per_super;
  const int rows = min(p.swizzle_m, p.num_m_tiles - sr * p.swizzle_m);
  r.m0 = (sr * p.swizzle_m + rem % rows) * BM;
  r.n0 = (rem / rows) * BN;
  r.mv = p.m;
  if (GRP == GRP_CONTIG) {
    const int g = load_uniform(p.grouped_layout, r.m0);
    const int last = load_uniform(p.grouped_layout, min(r.m0 + BM, p.m) - 1);
    const bool ok = g >= 0 && g < p.num_groups;
    r.g = ok ? g : 0;
    r.mv = ok ? p.m : 0;
    r.chk = ok && last != g;
  }
  return r;
}

// Wave-uniform source of the copies of one K block of one operand: its rows (buffer range
// over the rows that exist, so copies of missing rows return zeros without touching
// memory) and its scales.  Kept as plain 32-bit values so that they can be computed early
// and pinned in scalar registers.
struct Src {
  uint32_t lo, hi;    // row r0, byte kb * 128
  int bytes;
  uint32_t slo, shi;  // scale entry of row r0, K block kb
  int sbytes;
};

// (SC = false: an operand without staged scales; only its row fields are kept)
template <bool SC = true>
__device__ __forceinline__ void pin_src(Src& s) {
  if constexpr (SC) asm volatile("" : "+s"(s.lo), "+s"(s.hi), "+s"(s.bytes), "+s"(s.slo), "+s"(s.shi), "+s"(s.sbytes));
  else asm volatile("" : "+s"(s.lo), "+s"(s.hi), "+s"(s.bytes));
}

// K-major operand (rows of K bytes): the block starts at byte kb * bkb of row r0 and the
// range covers the tile's rows.  MN-major operand (mn: K rows of rows_total bytes, the tile
// being columns r0..r0+R-1): the block starts at K row kb * 128, column r0, and the range ends
// with the 16-byte granule that holds the last byte of the operand, so columns past rows_total
// read the next K row (they only feed outputs that are never stored) or, past the end, zeros.
// (The range check drops every dword that does not fit whole, so a range ending inside a
// 16-byte copy would lose the valid bytes at its start; the granule shares its page with them.)
__device__ __forceinline__ Src make_src(const uint8_t* X, int64_t ld, int r0, int rows_total, int R, int kb,
                                        bool valid, const void* sf, int64_t sf_stride, int64_t sf_row,
                                        bool has_scales, int bkb, bool mn = false, int k = 0) {
  const int rows = valid ? max(0, min(rows_total - r0, R)) : 0;
  const uint64_t base = mn ? (uint64_t)(X + (int64_t)kb * BK * ld + r0) : (uint64_t)(X + (int64_t)r0 * ld + kb * bkb);
  const uint64_t sbase = (uint64_t)((const uint8_t*)sf + 4 * (sf_row * sf_stride + r0));
  // (MN-major: k * ld < 2^31, checked on the host)
  const int mn_bytes = (int)(((int64_t)(k - kb * BK - 1) * ld + rows_total - r0 + 15) & ~(int64_t)15);
  Src s;
  s.lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  s.hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  s.bytes = __builtin_amdgcn_readfirstlane(rows > 0 ? (mn ? mn_bytes : rows * (int)ld - kb * bkb) : 0);
  s.slo = __builtin_amdgcn_readfirstlane((uint32_t)sbase);
  s.shi = __builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32));
  s.sbytes = __builtin_amdgcn_readfirstlane((has_scales && valid) ? 4 * max(0, min((int)sf_stride - r0, R)) : 0);
  return s;
}

__device__ __forceinline__ const void* src_ptr(uint32_t lo, uint32_t hi) {
  return (const void*)(((uint64_t)hi << 32) | lo);
}

// Source of K block k (counted from the start of tile `c`; k >= nkb lies in the next tile
// `n`) from the two tiles' block-0 sources: rows advance by k * kstep bytes (the bytes of a
// K block: BKB along a K-major row, 128 rows of an MN-major operand), scales by srow(k) scale
// rows of `sstep` bytes (srow = k, or k / 4 for words that pack four K blocks).  A few scalar
// instructions instead of rebuilding the source from the tile position every block.
template <bool PACK4>
__device__ __forceinline__ Src src_at(const Src& c, const Src& n, int k, int nkb, uint32_t sstep, uint32_t kstep) {
  const bool same = k < nkb;
  const int kk = same ? k : k - nkb;
  const uint64_t base = ((uint64_t)(same ? c.hi : n.hi) << 32 | (same ? c.lo : n.lo)) + (uint32_t)kk * kstep;
  const int srow = PACK4 ? kk >> 2 : kk;
  const uint64_t sbase = ((uint64_t)(same ? c.shi : n.shi) << 32 | (same ? c.slo : n.slo)) + (uint32_t)srow * sstep;
  Src s;
  s.lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  s.hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  // (a tile with rows has bytes > (nkb-1) * kstep)
  s.bytes = __builtin_amdgcn_readfirstlane(max((same ? c.bytes : n.bytes) - kk * (int)kstep, 0));
  s.slo = __builtin_amdgcn_readfirstlane((uint32_t)sbase);
  s.shi = __builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32));
  s.sbytes = __builtin_amdgcn_readfirstlane(same ? c.sbytes : n.sbytes);
  return s;
}

// Block-0 sources of the current and the next tile, and (1d2d) the weight-scale indices
// of their block 0.
struct Bases {
  Src ac, an, bc, bn;
  int wc0, wc1, wn0, wn1;  // (wn0, wn1: minus the current tile's block count)
};

// State carried from one K block to the next (and across tiles).
template <int FM>
struct Carry {
  v8i af[FM];           // A fragments of the block about to run
  v8i bf;               // its first B fragment
  float sa[FM];         // its activation scales (UE8M0 mode: the packed words, as bits)
  float sbw0, sbw1;     // 1d2d: its weight-block scales
  v4f acc1, acc2;       // partials of the previous block's last two MFMAs, not yet promoted
  float pscale[2];      // their promotion factors (1d2d)
  unsigned int ebw;     // UE8M0: packed weight-scale word of the lane's row in the first B fragment
};

template <int BM, int BN, int WM, int WN, int SFM, int OUT, int GRP, int NB, int LAY>
struct Kernel {
  // Per-row FP32 weight scales run on the generic kernel: here the B stage that holds a
  // block's scales is refilled before its last two partials are promoted.
  static_assert(SFM == SF_1D2D_F32 || SFM == SF_1D1D_UE8M0 || SFM == SF_FP4_UE8M0,
                "1d2d FP32, 1d1d UE8M0 or FP4-weight UE8M0 scales only");
  using G = Geo<BM, BN, WM, WN, SFM, NB>;
  static constexpr bool FP4B = G::FP4B;
  // power-of-two scales applied by the matrix unit itself (no VALU promotion)
  static constexpr bool UE = SFM == SF_1D1D_UE8M0 || FP4B;
  // operands stored MN-major (K rows of M or N bytes): staged as 32-column strips (or row-XOR,
  // below) and read back with the transposing LDS read
  static constexpr bool AMN = (LAY & LAYOUT_A_MN) != 0, BMN = (LAY & LAYOUT_B_MN) != 0;
  static_assert(!(BMN && FP4B), "FP4 weights are K-major");
  static constexpr int FBA = FP4B ? 4 : 5, FBB = 5;  // row-permutation bit of an MN-major stage
  // MN-major operands 128 or 256 columns wide are staged row-major with an XOR key per K row
  // (the copies then read whole row segments); other widths as 32-column strips.  (Measured
  // on 4096x7168x2048 at the sustained clock: tt 70.2 us with row-XOR A against 74.4 with
  // strips; with both operands MN-major and B in strips, row-XOR A took 117.0 against 104.8,
  // so that case keeps strips.)
  static constexpr bool ARX = AMN && !BMN && (BM == 256 || BM == 128), BRX = BMN && (BN == 256 || BN == 128);
  // Row-XOR staging of an MN-major operand W columns wide: wave-load q fills K rows
  // q * (1024 / W) + [0, 1024 / W), and the XOR key of row r has bit FB of r as its top bit.
  // Which copy offset wave-load part U uses: -1 when that bit of q comes from the wave index
  // (the lane offset already holds it), else the bit of U it comes from.
  template <int W, int FB>
  static constexpr int rx_ubit(int U) {
    constexpr int sh = W == 256 ? 2 : 3;  // log2 of the K rows per wave-load
    constexpr int lnw = NW == 8 ? 3 : 2;
    return FB - sh < lnw ? -1 : (U >> (FB - sh - lnw)) & 1;
  }
  static constexpr int FM = G::FM, FN = G::FN, TM = G::TM, TN = G::TN, STEPS = G::STEPS;
  static constexpr int NW = G::NW;
  static __device__ __forceinline__ int next_b(int b) { return b == NB - 1 ? 0 : b + 1; }

  const GemmParams& p;
  uint8_t* smem;
  int wave, lane, wm, wn, lr, lg;
  // per-lane source offsets of the copies.  Row copy q (q = wave + u*NW) fills 1 KiB of
  // LDS: lane L writes row 8q + L/8, slot L%8, which holds 16-byte chunk
  // (L%8) ^ swz(8q + L/8) = (L%8) ^ (L/8) ^ (q&1) of that row; NW is even, so q&1 = wave&1.
  uint32_t off_a, off_b;  // part 0; part u adds u * 8 * NW * ld
  uint32_t off_s;         // scale copies: lane L copies the 4-byte entries 4L..4L+3
  uint32_t a_lo, a_hi, b_lo, b_hi;  // per-lane LDS fragment bases (stage 0)
  uint32_t sa_lds;                  // per-lane LDS address of its rows' activation scales (stage 0)
  uint32_t ww_lds;                  // UE8M0: per-lane LDS address of its B row's packed weight scales (stage 0)
  int wshift;                       // FP4 weights: bit offset of this lane's 32-K block scale in the packed word
  int ustep_a, ustep_b;             // 8 * NW * ld (MN-major: 8 * NW)
  uint32_t kstep_a, kstep_b;        // bytes of one K block along the source (BK or BKB; MN-major: BK * ld)
  uint32_t off_a1, off_b1;          // row-XOR staging: the copy offsets of parts whose key bit comes from U = 1
  uint32_t sstep_a, sstep_b;        // bytes per K-block row of the activation / per-row weight scales
  // masked groups (at most 64): lane g holds group g's valid rows and the inclusive prefix
  // sum of the tiles of groups 0..g, so a tile index maps to its group with one ballot
  int grp_rows = 0, grp_incl = 0;

  __device__ __forceinline__ Kernel(const GemmParams& p_, uint8_t* smem_) : p(p_), smem(smem_) {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lane = threadIdx.x & 63;
    wm = wave / WN;
    wn = wave % WN;
    lr = lane & 15;
    lg = lane >> 4;
    const uint32_t r = (uint32_t)lane >> 3, c = (uint32_t)lane & 7, w = (uint32_t)wave & 1;
    const uint32_t chunk = (c ^ r ^ w) << 4;
    // (next to FP4 weights the activation rows use swz4a: (L%8) ^ (L/8) ^ 2 (q&1))
    off_a = (8u * (uint32_t)wave + r) * (uint32_t)p.lda + (FP4B ? (c ^ r ^ (w << 1)) << 4 : chunk);
    off_s = (uint32_t)lane << 4;
    ustep_a = __builtin_amdgcn_readfirstlane(8 * NW * (int)p.lda);
    if constexpr (FP4B) {
      // 64-byte weight rows: wave-load q fills rows 16q..16q+15; lane L writes row 16q + L/4,
      // slot L%4, which holds chunk (L%4) ^ swz4b(16q + L/4) = (L%4) ^ 2 ((L/16) & 1)
      off_b = (16u * (uint32_t)wave + ((uint32_t)lane >> 2)) * (uint32_t)p.ldb +
              ((((uint32_t)lane & 3u) ^ ((((uint32_t)lane >> 4) & 1u) << 1)) << 4);
      ustep_b = __builtin_amdgcn_readfirstlane(16 * NW * (int)p.ldb);
    } else {
      off_b = (8u * (uint32_t)wave + r) * (uint32_t)p.ldb + chunk;
      ustep_b = __builtin_amdgcn_readfirstlane(8 * NW * (int)p.ldb);
    }
    sstep_a = __builtin_amdgcn_readfirstlane(4u * (uint32_t)p.sfa_stride);
    sstep_b = __builtin_amdgcn_readfirstlane(4u * (uint32_t)p.sfb_stride);
    const int sw = FP4B ? swz4a(lr) : swz(lr);
    // An FP8 operand of the 16x16x128 MFMA holds, in lane group lg, K [16 lg, +16) in its
    // first four registers and K [64 + 16 lg, +16) in its last four (chunks lg and lg + 4 of a
    // 128-byte row); an FP4 operand holds K [32 lg, +32) (chunk lg of a 64-byte row).  With FP8
    // on both sides any assignment shared by the two operands gives the same dot products, and
    // the kernel reads chunks 2 lg and 2 lg + 1; next to FP4 weights it must be the true one.
    const int c_lo = FP4B ? lg : 2 * lg, c_hi = FP4B ? lg + 4 : 2 * lg + 1;
    const uint32_t lo = (uint32_t)((c_lo ^ sw) * 16), hi = (uint32_t)((c_hi ^ sw) * 16);
    a_lo = G::A_OFF + (wm * TM + lr) * BK + lo;
    a_hi = G::A_OFF + (wm * TM + lr) * BK + hi;
    if constexpr (FP4B) {
      // rows r..r+15 of chunk lg sit in slots lg ^ swz4b(r), swz4b(r) = 2 ((r >> 2) & 1): of the
      // 16 lanes served together (see swz), the four that share a bank group (r mod 4) then take
      // four different slots
      b_lo = b_hi = G::B_OFF + (wn * TN + lr) * G::BKB + ((lg ^ (((lr >> 2) & 1) << 1)) * 16);
    } else {
      b_lo = G::B_OFF + (wn * TN + lr) * BK + lo;
      b_hi = G::B_OFF + (wn * TN + lr) * BK + hi;
    }
    kstep_a = BK;
    kstep_b = G::BKB;
    // MN-major operands.  A K block of a tile W columns wide sits in LDS as W/32 strips of
    // 32 columns, strip s at byte 4096 s, each strip 128 K rows of 32 bytes; the 16-column
    // half h of K row k is stored at 32 k + 16 (h ^ bit FB of k).  The fragment reads of one
    // 16-lane group take 8 K rows of one half-strip, and the two groups served together take
    // rows whose bit FB differs, so the swap puts them on the other half of the banks.  FB is 5
    // when a lane group holds K [32 lg, +32) (FP8 next to FP8) and 4 when it holds K [16 lg, +16)
    // and K [64 + 16 lg, +16) (next to FP4 weights).  Wave-load q (1 KiB) fills strip q/4, K rows
    // 32 (q % 4) + [0, 32): lane L copies 16 bytes of K row 32 (q % 4) + L/2, so lane pairs read
    // whole 32-byte row segments.  (q % 4 = wave % 4, and part U adds 8 NW bytes of columns.)
    auto mn_copy = [&](int64_t ld, int fb) -> uint32_t {
      const uint32_t L = (uint32_t)lane, w = (uint32_t)wave;
      const uint32_t row = 32u * (w & 3u) + (L >> 1);
      const uint32_t sh = fb == 5 ? ((L & 1u) ^ (w & 1u)) : ((L & 1u) ^ ((L >> 5) & 1u));
      return row * (uint32_t)ld + 32u * (w >> 2) + 16u * sh;
    };
    // the transposing reads: lane 2b + h of lane group lg reads columns 8h.. of K row k0 + b
    // (+ 8, 16, 24 rows for reads 1-3; FB = 4: + 8, 64, 72) of one 16-column half; a wave whose
    // first 16-column chunk is c0 keeps one base for its even and one for its odd fragments
    auto mn_read = [&](int off, int c0, int fb, bool odd) -> uint32_t {
      const int l = lane & 15;
      const int k0 = (fb == 5 ? 32 * lg : 16 * lg) + (l >> 1);
      const int p0 = c0 & 1;
      const int strip = (c0 >> 1) + (odd ? p0 : 0), half = odd ? 1 - p0 : p0;
      return (uint32_t)(off + strip * 4096 + 32 * k0 + 16 * (half ^ (lg & 1)) + 8 * (l & 1));
    };
    // Row-XOR staging (W = 128 or 256 columns): K row r sits at LDS row r, W bytes, its
    // 16-byte chunk s at position s ^ key(r): key = (r & 7) | bit_FB(r) << 3 for W = 256,
    // ((r >> 1) & 3) | bit_FB(r) << 2 for W = 128.  The 16 K rows one transposing read takes in
    // a cycle (8 per lane group, the two groups differing in bit FB) then land on 16 different
    // 4-bank groups.  Lane L of wave-load q copies chunk (L % C) ^ key(r) of row
    // r = q * (1024 / W) + L / C (C = W / 16): consecutive lanes read consecutive bytes of a row.
    auto rx_copy = [&](int64_t ld, int w, int fb, int ubit) -> uint32_t {
      const uint32_t C = (uint32_t)w / 16, rw = 1024u / (uint32_t)w, L = (uint32_t)lane;
      const uint32_t r = (uint32_t)wave * rw + L / C;  // (part U adds U * NW * rw rows)
      const uint32_t bfb = ubit < 0 ? (r >> fb) & 1u : (uint32_t)ubit;
      const uint32_t key = w == 256 ? (r & 7u) | (bfb << 3) : ((r >> 1) & 3u) | (bfb << 2);
      return r * (uint32_t)ld + 16u * ((L % C) ^ key);
    };
    // the transposing reads: lane 2b + h of lane group g reads columns 8h.. of K row k0(g) + b
    // (+ 8, 16, 24 rows for reads 1-3; FB = 4: + 8, 64, 72), chunk (s0 + i) ^ key
    auto rx_base = [&](int off, int w, int fb) -> uint32_t {
      const int l = lane & 15, k0 = fb == 5 ? 32 * lg : 16 * lg;
      return (uint32_t)(off + (k0 + (l >> 1)) * w + 8 * (l & 1));
    };
    auto rx_key16 = [&](int w) -> uint32_t {
      const int b = (lane & 15) >> 1;
      return (uint32_t)(16 * (w == 256 ? (b | ((lg & 1) << 3)) : (((b >> 1) & 3) | ((lg & 1) << 2))));
    };
    if constexpr (AMN) {
      off_a = mn_copy(p.lda, FBA);
      ustep_a = 8 * NW;
      kstep_a = __builtin_amdgcn_readfirstlane(BK * (uint32_t)p.lda);
      a_lo = mn_read(G::A_OFF, wm * TM / 16, FBA, false);
      a_hi = mn_read(G::A_OFF, wm * TM / 16, FBA, true);
      if constexpr (ARX) {
        constexpr bool from_u = rx_ubit<BM, FBA>(0) >= 0 || rx_ubit<BM, FBA>(1) >= 0;
        off_a = rx_copy(p.lda, BM, FBA, from_u ? 0 : -1);
        off_a1 = from_u ? rx_copy(p.lda, BM, FBA, 1) : off_a;
        ustep_a = __builtin_amdgcn_readfirstlane(NW * (1024 / BM) * (int)p.lda);
        a_lo = rx_base(G::A_OFF, BM, FBA);
        a_hi = rx_key16(BM);
      }
    }
    if constexpr (BMN) {
      off_b = mn_copy(p.ldb, FBB);
      ustep_b = 8 * NW;
      kstep_b = __builtin_amdgcn_readfirstlane(BK * (uint32_t)p.ldb);
      b_lo = mn_read(G::B_OFF, wn * TN / 16, FBB, false);
      b_hi = mn_read(G::B_OFF, wn * TN / 16, FBB, true);
      if constexpr (BRX) {
        constexpr bool from_u = rx_ubit<BN, FBB>(0) >= 0 || rx_ubit<BN, FBB>(1) >= 0;
        off_b = rx_copy(p.ldb, BN, FBB, from_u ? 0 : -1);
        off_b1 = from_u ? rx_copy(p.ldb, BN, FBB, 1) : off_b;
        ustep_b = __builtin_amdgcn_readfirstlane(NW * (1024 / BN) * (int)p.ldb);
        b_lo = rx_base(G::B_OFF, BN, FBB);
        b_hi = rx_key16(BN);
      }
    }
    wshift = 8 * lg;
    sa_lds = G::SA_OFF + 4 * (wm * TM + lr);
    ww_lds = G::SB_OFF + 4 * (wn * TN + lr);
    if (GRP == GRP_MASKED && p.num_groups <= 64) {
      const int mg = lane < p.num_groups ? min(max(p.masked_m[lane], 0), p.m) : 0;
      int incl = ((mg + BM - 1) / BM) * p.num_n_tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      grp_rows = mg;
      grp_incl = incl;
    }
  }

  __device__ __forceinline__ TilePos tile_at(int t) const {
    if (GRP == GRP_MASKED && p.num_groups <= 64) {
      TilePos r;
      const uint64_t hit = __ballot(grp_incl > t);
      r.valid = hit != 0;
      const int g = r.valid ? (int)__builtin_ctzll(hit) : 0;
      const int mg = __builtin_amdgcn_readlane(grp_rows, g);
      const int mt = max(1, (mg + BM - 1) / BM);
      const int loc = t - (__builtin_amdgcn_readlane(grp_incl, g) - ((mg + BM - 1) / BM) * p.num_n_tiles);
      r.g = g;
      r.mv = r.valid ? mg : 0;
      r.n0 = r.valid ? (loc / mt) * BN : 0;
      r.m0 = r.valid ? (loc % mt) * BM : 0;
      return r;
    }
    return tile_pos<BM, BN, GRP>(p, t);
  }

  // ---- copies HBM -> LDS --------------------------------------------------------------
  __device__ __forceinline__ Src a_src(const TilePos& t, int kb) const {
    const int64_t srow = UE ? (kb >> 2) : kb;  // UE8M0 words hold four K blocks
    const uint8_t* A = p.a;
    const uint8_t* SA = (const uint8_t*)p.sfa;
    if (GRP == GRP_MASKED) {
      A += (int64_t)t.g * p.a_gstride;
      SA += 4 * (int64_t)t.g * p.sfa_gstride;
    }
    return make_src(A, p.lda, t.m0, t.mv, BM, kb, t.valid, SA, p.sfa_stride, srow, true, BK, AMN, p.k);
  }
  __device__ __forceinline__ Src b_src(const TilePos& t, int kb) const {
    // (FP4 weights: one word per K block, holding its four 32-K scales)
    const int64_t srow = SFM == SF_1D1D_UE8M0 ? (kb >> 2) : kb;
    const uint8_t* B = p.b;
    const uint8_t* SB = (const uint8_t*)p.sfb;
    if (GRP != GRP_DENSE) {
      B += (int64_t)t.g * p.b_gstride;
      SB += 4 * (int64_t)t.g * p.sfb_gstride;
    }
    // (a skipped contiguous tile reads no weights either)
    const bool valid = GRP == GRP_CONTIG ? t.valid && t.mv > 0 : t.valid;
    return make_src(B, p.ldb, t.n0, p.n, BN, kb, valid, SB, p.sfb_stride, srow, SFM != SF_1D2D_F32, G::BKB, BMN,
                    p.k);
  }

  // Part U of the copy of one operand block into the stage at LDS offset `dst` (its scales
  // into `sdst`): rows for the waves whose copy index is below the row-copy count ROWL, the
  // scales for the one right after (when the operand carries them), empty otherwise.  Which
  // case applies is fixed at compile time except for the one part that straddles them.
  template <int U, int ROWL, bool SCALES>
  __device__ __forceinline__ void copy_part(const Src& s, int dst, int sdst, uint32_t off, int ustep,
                                            uint32_t off1 = 0, bool use1 = false) const {
    constexpr int Q0 = U * NW;
    const int q = wave + Q0;
    const int row_dst = dst + q * 1024;
    const uint32_t row_off = (use1 ? off1 : off) + (uint32_t)U * (uint32_t)ustep;
    if constexpr (Q0 + NW <= ROWL) {
      copy_to_lds(src_ptr(s.lo, s.hi), s.bytes, row_off, smem, row_dst);
    } else if constexpr (Q0 >= ROWL) {
      const bool is_s = SCALES && q == ROWL;
      if constexpr (SCALES) {
        copy_to_lds(src_ptr(s.slo, s.shi), is_s ? s.sbytes : 0, off_s, smem, is_s ? sdst : (int)G::TRASH_OFF);
      } else {
        copy_to_lds(src_ptr(s.lo, s.hi), 0, off_s, smem, (int)G::TRASH_OFF);  // (empty: keeps the copy count)
      }
    } else {
      const bool is_row = q < ROWL, is_s = SCALES && q == ROWL;
      if (SCALES) {
        copy_to_lds(src_ptr(is_row ? s.lo : s.slo, is_row ? s.hi : s.shi), is_row ? s.bytes : (is_s ? s.sbytes : 0),
                    is_row ? row_off : off_s, smem, is_row ? row_dst : (is_s ? sdst : (int)G::TRASH_OFF));
      } else {
        copy_to_lds(src_ptr(s.lo, s.hi), is_row ? s.bytes : 0, row_off, smem, is_row ? row_dst : (int)G::TRASH_OFF);
      }
    }
  }
  template <int U>
  __device__ __forceinline__ void copy_a(const Src& s, int slot) const {
    constexpr bool use1 = ARX && rx_ubit<BM, FBA>(U) == 1;
    copy_part<U, G::A_ROWL, true>(s, G::A_OFF + slot * G::A_SLOT, G::SA_OFF + slot * G::SA_SLOT, off_a, ustep_a,
                                  off_a1, use1);
  }
  template <int U>
  __device__ __forceinline__ void copy_b(const Src& s, int slot) const {
    constexpr bool use1 = BRX && rx_ubit<BN, FBB>(U) == 1;
    copy_part<U, G::B_ROWL, SFM != SF_1D2D_F32>(s, G::B_OFF + slot * G::B_SLOT, G::SB_OFF + slot * G::SB_SLOT,
                                                 off_b, ustep_b, off_b1, use1);
  }
  template <int... Us>
  __device__ __forceinline__ void copy_a_all(const Src& s, int slot, std::integer_sequence<int, Us...>) const {
    (copy_a<Us>(s, slot), ...);
  }
  template <int... Us>
  __device__ __forceinline__ void copy_b_all(const Src& s, int slot, std::integer_sequence<int, Us...>) const {
    (copy_b<Us>(s, slot), ...);
  }
  __device__ __forceinline__ void copy_a_block(const TilePos& t, int kb, int slot) const {
    copy_a_all(a_src(t, kb), slot, std::make_integer_sequence<int, G::LA>{});
  }
  __device__ __forceinline__ void copy_b_block(const TilePos& t, int kb, int slot) const {
    copy_b_all(b_src(t, kb), slot, std::make_integer_sequence<int, G::LB>{});
  }

  // ---- LDS -> registers ---------------------------------------------------------------
  __device__ __forceinline__ v8i frag(uint32_t lo, uint32_t hi, int off) const {
    const v4i l4 = *(const v4i*)(smem + lo + off);
    const v4i h4 = *(const v4i*)(smem + hi + off);
    return (v8i){l4.x, l4.y, l4.z, l4.w, h4.x, h4.y, h4.z, h4.w};
  }
  // MN-major strip stage: four transposing reads of 8 K each, 8 K rows apart (FB = 5) or 8
  // and 64 apart (FB = 4), from the lane's base for the fragment's half-strip
  template <int FB>
  __device__ __forceinline__ v8i frag_tr(uint32_t base, int off) const {
    constexpr int D2 = FB == 5 ? 16 * 32 : 64 * 32, D3 = D2 + 8 * 32;
    const v2i x0 = read_tr8(smem, base + off), x1 = read_tr8(smem, base + off + 8 * 32);
    const v2i x2 = read_tr8(smem, base + off + D2), x3 = read_tr8(smem, base + off + D3);
    return (v8i){x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
  }
  // row-XOR stage W bytes wide: the fragment of chunk c (16 columns) is four transposing reads
  // at base + ((16 c) ^ key16), 8 K rows apart (FB = 5) or 8 and 64 apart (FB = 4)
  template <int FB, int W>
  __device__ __forceinline__ v8i frag_rx(uint32_t base, uint32_t key16, uint32_t c16) const {
    const uint32_t a = base + (c16 ^ key16);
    constexpr int R1 = 8 * W, R2 = (FB == 5 ? 16 : 64) * W, R3 = (FB == 5 ? 24 : 72) * W;
    const v2i x0 = read_tr8(smem, a), x1 = read_tr8(smem, a + R1);
    const v2i x2 = read_tr8(smem, a + R2), x3 = read_tr8(smem, a + R3);
    return (v8i){x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
  }
  __device__ __forceinline__ v8i a_frag(int aslot, int i) const {
    const uint32_t so = (uint32_t)(aslot * G::A_SLOT);
    // (a 16-row fragment is 16 rows x 128 bytes; an MN-major strip holds two fragments)
    if constexpr (ARX) return frag_rx<FBA, BM>(a_lo + so, a_hi, (uint32_t)(wm * TM + 16 * i));
    if constexpr (AMN) return frag_tr<FBA>(((i & 1) ? a_hi : a_lo) + so, 4096 * (i >> 1));
    return frag(a_lo + so, a_hi + so, i * 16 * BK);
  }
  __device__ __forceinline__ v8i b_frag(int bslot, int j) const {
    const uint32_t so = (uint32_t)(bslot * G::B_SLOT);
    if constexpr (FP4B) {
      // 32 E2M1 codes in the first four registers; the MFMA does not read the others
      const v4i x = *(const v4i*)(smem + b_lo + so + j * 16 * G::BKB);
      return (v8i){x.x, x.y, x.z, x.w, 0, 0, 0, 0};
    }
    if constexpr (BRX) return frag_rx<FBB, BN>(b_lo + so, b_hi, (uint32_t)(wn * TN + 16 * j));
    if constexpr (BMN) return frag_tr<FBB>(((j & 1) ? b_hi : b_lo) + so, 4096 * (j >> 1));
    return frag(b_lo + so, b_hi + so, j * 16 * BK);
  }
  // UE8M0: the packed weight-scale word of the lane's B row in fragment j of B stage bslot
  __device__ __forceinline__ unsigned int weight_word(int bslot, int j) const {
    return *(const unsigned int*)(smem + ww_lds + (uint32_t)(bslot * G::SB_SLOT) + 64 * j);
  }
  __device__ __forceinline__ void read_scales(Carry<FM>& c, int aslot) const {
    const uint32_t a = sa_lds + (uint32_t)(aslot * G::SA_SLOT);
#pragma unroll
    for (int i = 0; i < FM; ++i) c.sa[i] = *(const float*)(smem + a + 64 * i);
  }

  // 1d2d: indices of the weight-block scales of this wave's (at most two) 128-wide column
  // blocks for K block kb of tile t
  __device__ __forceinline__ void weight_block_index(const TilePos& t, int kb, int& i0, int& i1) const {
    const int nw0 = t.n0 + wn * TN;
    const int nb = (p.n + 127) / 128;
    const int blk0 = min(nw0 / 128, nb - 1), blk1 = min(nw0 / 128 + 1, nb - 1);
    const int gofs = GRP != GRP_DENSE ? t.g * (int)p.sfb_gstride : 0;
    i0 = __builtin_amdgcn_readfirstlane(gofs + blk0 * (int)p.sfb_stride + kb);
    i1 = __builtin_amdgcn_readfirstlane(gofs + blk1 * (int)p.sfb_stride + kb);
  }
  __device__ __forceinline__ void weight_block_scales(const TilePos& t, int kb, float& s0, float& s1) const {
    int i0, i1;
    weight_block_index(t, kb, i0, i1);
    s0 = load_uniform((const float*)p.sfb, i0);
    s1 = load_uniform((const float*)p.sfb, i1);
  }

  // ---- one K block ------------------------------------------------------------------
  // Block g = (tile cur, K index kb) runs out of A stage `as` and B stage `bs`; nxt is the
  // tile after cur.  `stores`: lower bound on the vector stores the previous epilogue issued
  // stores since the last barrier.
  // NF: leading 16-column fragments that use the wave's first weight-scale block (1d2d);
  // 0 means the split is only known at run time (`nf`).  FA: this wave's 16-row fragments
  // that hold rows of the problem (masked groups: the others are padding, and their MFMAs,
  // promotions and stores are skipped).
  template <int NF, int FA>
  __device__ __forceinline__ void block(Carry<FM>& c, float (&fin)[FM][FN][4], const Bases& sb, int kb, int nkb,
                                        int as, int bs, int stores, int nf) const {
    // promotion factor of fragment (i, j) of this block: activation scale of row i times the
    // weight-block scale of column fragment j (the first block's for j < nf, else the second's;
    // both wave-uniform)
    float sa[FM];
    int ea[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      sa[i] = c.sa[i];
      ea[i] = (int)((__float_as_uint(c.sa[i]) >> (8 * (kb & 3))) & 0xFFu);
    }
    // 1d2d: the factors of fragments j < NF (first weight block) and of the others
    float f0[FM], f1[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      f0[i] = SFM == SF_1D2D_F32 ? sa[i] * c.sbw0 : sa[i];
      f1[i] = SFM == SF_1D2D_F32 && NF < FN ? sa[i] * c.sbw1 : f0[i];
    }
    auto factor = [&](int i, int j) -> float {
      if constexpr (NF == 0) return j < nf ? f0[i] : f1[i];
      else return j < NF ? f0[i] : f1[i];
    };

    // copies of A block g+2 go out spread over the steps before the barrier (in the first
    // block of a tile: right after the barrier, because their stage served as the previous
    // tile's epilogue scratch until every wave has passed it); their source,
    // the B source of block g+2 and the weight-scale indices of block g+1 are computed in the
    // first steps (in the shadow of the MFMAs) and pinned, so the scalar work does not pile
    // up right after the barrier
    Src asrc = {}, bsrc = {};
    uint32_t wo0 = 0, wo1 = 0;  // 1d2d: byte offsets in sfb of the weight-block scales of block g+1
    const int as2 = as >= NA - 2 ? as - (NA - 2) : as + 2;
    const int as1 = as >= NA - 1 ? as - (NA - 1) : as + 1;
    const int bs1 = next_b(bs);
    const int kshift = 8 * (kb & 3);  // UE8M0: byte of this K block in the packed words

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    v4f r1 = c.acc1, r2 = c.acc2;  // partials of MFMAs t-1 and t-2
    v8i bf = c.bf, bfn = c.bf;
    unsigned int ebw = c.ebw, ebwn = c.ebw;
    float sbn0 = 0.f, sbn1 = 0.f;

    auto step = [&]<int t>() {
      constexpr int j = t / FM, i = t % FM;
      // A copies for block g+2
      [&]<int... Us>(std::integer_sequence<int, Us...>) {
        ((t == 1 + (Us * (G::TB - 1)) / G::LA ? (kb != 0 ? copy_a<Us>(asrc, as2) : void()) : void()), ...);
      }(std::make_integer_sequence<int, G::LA>{});
      if constexpr (t == G::TB) {
        // Block g+1 has landed everywhere and B stage bs is no longer read by anyone.  Each
        // wave first waits until its own copies of block g+1 have landed; what it issued after
        // the last of them may stay in flight:
        //  * 2 B stages: the last is B(g+1) (previous barrier); after it come the A copies of
        //    block g+2 (LA), or, in a tile's first block (whose A copies wait for the barrier),
        //    only the previous epilogue's stores (a lower bound is counted);
        //  * NB = 3 or 4 B stages: the last is A(g+1) (previous block); after it come
        //    B(g+NB-1) (LB) and A(g+2) (LA); in a tile's first block B(g+NB-1) and the stores;
        //    in its second block only A(g+2), because the first block issued A(g+1) after
        //    B(g+NB).  (In the very first block the prologue's later B blocks are also waited
        //    for: stricter than needed.)
        // (Only the vmcnt wait depends on the branch: the LDS wait and the barrier stay in
        // straight-line code, so the compiler knows every earlier LDS read has landed.)
        if (kb > 1 || (kb == 1 && NB == 2)) {
          wait_vm<(NB == 2 ? G::LA : G::LA + G::LB)>();
        } else if (kb == 1) {
          wait_vm<G::LA>();
        } else if (stores >= STORES_N) {
          wait_vm<(NB == 2 ? 0 : G::LB) + STORES_N>();
        } else if (stores > 0) {
          if constexpr (TRANSPOSE) wait_vm<(NB == 2 ? 0 : G::LB) + STORES_T>();
          else wait_vm<(NB == 2 ? 0 : G::LB)>();
        } else {
          wait_vm<(NB == 2 ? 0 : G::LB)>();
        }
        wait_and_barrier<63>();
        // (the copies and reads that the barrier releases follow this step's MFMA, so the
        // matrix unit is fed first)
      } else if constexpr (i == 0 && j + 1 < FN) {
        bfn = b_frag(bs, j + 1);
        if (UE) ebwn = weight_word(bs, j + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      v4f acc = zero;
      if constexpr (i < FA) {
        if constexpr (UE) {
          // power-of-two scales: the matrix unit applies 2^(e_b + e_a) to the block's products
          // and adds them to the FP32 accumulator itself, so the promotion needs no VALU work.
          // FP4 weights carry one scale per 32 K: lane group lg passes the one of its K range.
          const int eb = (int)((ebw >> (FP4B ? wshift : kshift)) & 0xFFu);
          const v4f cin = {fin[i][j][0], fin[i][j][1], fin[i][j][2], fin[i][j][3]};
          const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, c.af[i], cin, FP4B ? 4 : 0, 0, 0, eb, 0,
                                                                         ea[i]);
#pragma unroll
          for (int v = 0; v < 4; ++v) fin[i][j][v] = r[v];
        } else {
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, c.af[i], zero, 0, 0, 0, 0, 0, 0);
          asm volatile("" : "+v"(acc));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (t == G::TB) {
        // B block g+NB into the stage block g used
        copy_b_all(bsrc, bs, std::make_integer_sequence<int, G::LB>{});
        if (kb == 0) copy_a_all(asrc, as2, std::make_integer_sequence<int, G::LA>{});
        // first B fragment and scales of block g+1
        bfn = b_frag(bs1, 0);
        if (UE) ebwn = weight_word(bs1, 0);
        if (SFM == SF_1D2D_F32) {
          const __attribute__((address_space(4))) uint8_t* sfb = (const __attribute__((address_space(4))) uint8_t*)p.sfb;
          sbn0 = *(const __attribute__((address_space(4))) float*)(sfb + wo0);
          sbn1 = *(const __attribute__((address_space(4))) float*)(sfb + wo1);
        }
        read_scales(c, as1);
      }
      if constexpr (t == 0) {
        asrc = src_at<UE>(sb.ac, sb.an, kb + 2, nkb, sstep_a, kstep_a);
        pin_src(asrc);
      }
      if constexpr (t == 1) {
        bsrc = src_at<SFM == SF_1D1D_UE8M0>(sb.bc, sb.bn, kb + NB, nkb, sstep_b, kstep_b);
        pin_src<SFM != SF_1D2D_F32>(bsrc);
        if (SFM == SF_1D2D_F32) {
          // (the next tile's indices are stored minus nkb, so both count blocks from this tile's start)
          const bool same = kb + 1 < nkb;
          wo0 = 4u * (uint32_t)__builtin_amdgcn_readfirstlane((same ? sb.wc0 : sb.wn0) + kb + 1);
          wo1 = 4u * (uint32_t)__builtin_amdgcn_readfirstlane((same ? sb.wc1 : sb.wn1) + kb + 1);
          asm volatile("" : "+s"(wo0), "+s"(wo1));
        }
      }
      // after its last use, fragment i of A is replaced by block g+1's
      if constexpr (t >= G::TB) c.af[i] = a_frag(as1, i);
      // promote the partial of MFMA t-2 (for t < 2: of the previous block, with its factor)
      if constexpr (!UE && t >= 2 && (t - 2) % FM < FA) {
        constexpr int tp = t - 2, jp = tp / FM, ip = tp % FM;
        const float sc = factor(ip, jp);
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[ip][jp][v] = __builtin_fmaf(sc, r2[v], fin[ip][jp][v]);
        pin(fin[ip][jp]);
      } else if constexpr (t < 2 && SFM == SF_1D2D_F32 && (t - 2 + STEPS) % FM < FA) {
        constexpr int tp = t - 2 + STEPS, jp = tp / FM, ip = tp % FM;
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[ip][jp][v] = __builtin_fmaf(c.pscale[t], r2[v], fin[ip][jp][v]);
        pin(fin[ip][jp]);
      }
      if constexpr (!UE) {
        r2 = r1;
        r1 = acc;
      }
      if constexpr (i == FM - 1) {
        bf = bfn;
        ebw = ebwn;
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... Ts>(std::integer_sequence<int, Ts...>) {
      (step.template operator()<Ts>(), ...);
    }(std::make_integer_sequence<int, STEPS>{});

    c.bf = bfn;
    c.ebw = ebwn;
    c.sbw0 = sbn0;
    c.sbw1 = sbn1;
    c.acc1 = UE ? zero : r1;
    c.acc2 = UE ? zero : r2;
    constexpr int t0 = STEPS - 2, t1 = STEPS - 1;
    c.pscale[0] = SFM == SF_1D2D_F32 ? factor(t0 % FM, t0 / FM) : 0.f;
    c.pscale[1] = SFM == SF_1D2D_F32 ? factor(t1 % FM, t1 / FM) : 0.f;
  }

  // Promote the two partials still pending (end of a tile).
  __device__ __forceinline__ void flush(Carry<FM>& c, float (&fin)[FM][FN][4]) const {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    if (SFM == SF_1D2D_F32) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tp = STEPS - 2 + s, jp = tp / FM, ip = tp % FM;
        const v4f a = s == 0 ? c.acc2 : c.acc1;
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[ip][jp][v] = __builtin_fmaf(c.pscale[s], a[v], fin[ip][jp][v]);
      }
    }
    c.acc1 = zero;
    c.acc2 = zero;
    c.pscale[0] = c.pscale[1] = 0.f;
  }

  // Store the tile.  Returns a lower bound on the vector-memory operations every lane of
  // this wave issued (0 when it cannot tell).
  //
  // BF16 interior tiles go through LDS: a lane holds 4 consecutive columns of one row per
  // fragment, so storing straight from registers makes every 16 lanes of a store touch 16
  // different rows.  Instead each wave writes one 16-row fragment row at a time into 4 KiB
  // of scratch (the A stage of the tile's last K block, which no wave reads any more), reads
  // it back row-major, 16 bytes per lane, and stores it with consecutive lanes on
  // consecutive addresses.
  // Scratch row r holds 16-byte chunk c at position c ^ ekey(r), with its two 8-byte halves
  // swapped when hkey(r) is 1: ekey(r) = (r mod 16) * PX / 16 with PX the largest power of two
  // (at most 8) that divides the chunk count, so the XOR stays inside the row, and hkey(r) is
  // the bit of r just below the ones ekey uses.  The 8-byte writes (16 consecutive lanes,
  // rows 0..15 of one chunk half) are served 128 bytes at a time (measured), and these keys
  // give the 16 lanes 16 different 8-byte slots of a 128-byte window; the read-back gives
  // each group of 16 lanes that LDS serves together (same bit 5, same parity of bits 2..4)
  // 16 consecutive chunks of the fragment row.  Both are conflict-free.
  static constexpr int RS = 2 * TN;            // scratch row stride in bytes
  static constexpr int CH = TN / 8;            // 16-byte chunks per scratch row
  static constexpr int PX = CH % 8 == 0 ? 8 : CH % 4 == 0 ? 4 : CH % 2 == 0 ? 2 : 1;
  static constexpr int PXB = PX == 8 ? 3 : PX == 4 ? 2 : PX == 2 ? 1 : 0;
  static __device__ __forceinline__ int ekey(int r) { return ((r & 15) * PX) >> 4; }
  static __device__ __forceinline__ int hkey(int r) { return PX > 1 ? (r >> (3 - PXB)) & 1 : 0; }
  static constexpr int SCR = G::A_SLOT / NW;   // scratch bytes per wave
  static constexpr bool TRANSPOSE = OUT == OUT_BF16 && 16 * RS <= SCR && TN % 8 == 0;
  static constexpr int RD = (16 * CH + 63) / 64;  // read-back rounds per fragment row
  static constexpr int STORES_T = TRANSPOSE ? FM * (16 * CH / 64) : 0;  // rounds with every lane active
  static constexpr int STORES_N = FM * FN < 63 ? FM * FN : 63;
  static_assert(STORES_T < STORES_N && STORES_N < 64, "vmcnt is a 6-bit field; the two store counts must differ");

  __device__ __forceinline__ int epilogue(const float (&fin)[FM][FN][4], const TilePos& tr, int aslot) const {
    const int ln = fresh(lane);
    const int lr = ln & 15, lg = ln >> 4;  // (shadow the members: see fresh)
    const bool interior = tr.m0 + BM <= tr.mv && tr.n0 + BN <= p.n && !(GRP == GRP_CONTIG && tr.chk);
    const int esz = (OUT == OUT_BF16) ? 2 : 4;
    char* Dg = (char*)p.d;
    if (GRP == GRP_MASKED) Dg += (int64_t)tr.g * p.d_gstride * esz;
    // (tiles with missing rows take this path only for masked groups, where nearly every
    // tile has some; dense edge tiles use the element path below)
    if (TRANSPOSE && tr.n0 + BN <= p.n && p.d_vec16 && (GRP == GRP_MASKED || interior)) {
      const uint32_t scr = G::A_OFF + aslot * G::A_SLOT + wave * SCR;
      uint8_t* drow0 = (uint8_t*)Dg + ((int64_t)(tr.m0 + wm * TM) * p.ldd + tr.n0 + wn * TN) * 2;
      // the lane's chunk in each 64-chunk round of the read-back: lane group b = ln / 4 is served
      // with the groups of the same bit 3 and parity of bits 0..2, and takes 4 of their 16
      // consecutive chunks
      const int lb = ln >> 2;
      const int lpos = 16 * (2 * (lb >> 3) + (__builtin_popcount(lb & 7) & 1)) + 4 * ((lb & 7) >> 1) + (ln & 3);
      // rows of this wave's part that exist (all of them for interior tiles)
      const int rows = interior ? TM : tr.mv - tr.m0 - wm * TM;
      auto store_rows = [&]<bool ALL>() {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v2u w = {pack_bf16x2(fin[i][j][0], fin[i][j][1]), pack_bf16x2(fin[i][j][2], fin[i][j][3])};
            *(v2u*)(smem + scr + lr * RS + 16 * ((2 * j + (lg >> 1)) ^ ekey(lr)) + 8 * ((lg & 1) ^ hkey(lr))) = w;
          }
#pragma unroll
          for (int k = 0; k < RD; ++k) {
            const int cidx = lpos + 64 * k;
            const int r = cidx / CH, cc = cidx - r * CH;
            if (cidx < 16 * CH && (ALL || 16 * i + r < rows)) {
              v4i x = *(const v4i*)(smem + scr + r * RS + 16 * (cc ^ ekey(r)));
              if (hkey(r)) x = (v4i){x.z, x.w, x.x, x.y};
              *(v4i*)(drow0 + ((int64_t)(16 * i + r) * p.ldd + 8 * cc) * 2) = x;
            }
          }
        }
      };
      if (interior) {
        store_rows.template operator()<true>();
        return STORES_T;
      }
      if constexpr (GRP == GRP_MASKED) store_rows.template operator()<false>();
      return 0;
    }
    const bool vec = (OUT != OUT_F32_C || p.c_vec) && p.d_vec && interior;
    const int row0 = tr.m0 + wm * TM + lr;
    const int nw0 = tr.n0 + wn * TN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // (one fragment row at a time: batching every row's C loads ahead of the adds would
      // hold a second tile of values in registers)
      __builtin_amdgcn_sched_barrier(0);
      const int row = row0 + 16 * i;
      if (row >= tr.mv) continue;
      if (GRP == GRP_CONTIG && tr.chk && p.grouped_layout[row] != tr.g) continue;
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
            const unsigned short h[4] = {(unsigned short)w0, (unsigned short)(w0 >> 16), (unsigned short)w1,
                                         (unsigned short)(w1 >> 16)};
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
    return vec ? STORES_N : 0;
  }

  // All K blocks of one tile, then its epilogue.
  __device__ __forceinline__ void tile(Carry<FM>& c, const TilePos& cur, const TilePos& nxt, int nkb, int& as,
                                       int& bs, int& stores) const {
    float fin[FM][FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) fin[i][j][v] = 0.f;
    // leading 16-column fragments of this wave that use its first weight-scale block: a
    // compile-time split, so each fragment's factor is chosen without any instruction
    const int nf = SFM == SF_1D2D_F32 ? min(FN, 8 - (((cur.n0 + wn * TN) & 127) >> 4)) : FN;
    Bases sb;
    sb.ac = a_src(cur, 0);
    sb.an = a_src(nxt, 0);
    sb.bc = b_src(cur, 0);
    sb.bn = b_src(nxt, 0);
    sb.wc0 = sb.wc1 = sb.wn0 = sb.wn1 = 0;
    if (SFM == SF_1D2D_F32) {
      weight_block_index(cur, 0, sb.wc0, sb.wc1);
      weight_block_index(nxt, 0, sb.wn0, sb.wn1);
      sb.wn0 -= nkb;
      sb.wn1 -= nkb;
    }
    auto run = [&]<int NF, int FA>() {
      for (int kb = 0; kb < nkb; ++kb) {
        block<NF, FA>(c, fin, sb, kb, nkb, as, bs, stores, nf);
        stores = 0;
        as = as == NA - 1 ? 0 : as + 1;
        bs = next_b(bs);
      }
    };
    if constexpr (GRP == GRP_CONTIG) {
      // a skipped tile runs its K blocks without MFMAs (its copies are empty).  With a single
      // wave row (128 rows per wave) that third copy of the block loop pushes the kernel past
      // 256 VGPRs into scratch, so there a skipped tile runs the ordinary loop on its empty
      // (zero) copies instead; it stores nothing either way.
      if (WM > 1 && cur.mv == 0) {
        if constexpr (WM > 1) run.template operator()<FN, 0>();
      } else {
        [&]<int... Ns>(std::integer_sequence<int, Ns...>) {
          ((nf == Ns + 1 ? run.template operator()<Ns + 1, FM>() : void()), ...);
        }(std::make_integer_sequence<int, FN>{});
      }
    } else if constexpr (GRP == GRP_MASKED) {
      // 16-row fragments of this wave that hold valid rows of the group
      const int live = min(FM, max(0, (cur.mv - cur.m0 - wm * TM + 15) / 16));
      [&]<int... Fs>(std::integer_sequence<int, Fs...>) {
        ((live == Fs ? run.template operator()<SFM == SF_1D2D_F32 ? 0 : FN, Fs>() : void()), ...);
      }(std::make_integer_sequence<int, FM + 1>{});
    } else {
      [&]<int... Ns>(std::integer_sequence<int, Ns...>) {
        ((nf == Ns + 1 ? run.template operator()<Ns + 1, FM>() : void()), ...);
      }(std::make_integer_sequence<int, FN>{});
    }
    flush(c, fin);
    stores = epilogue(fin, cur, as == 0 ? NA - 1 : as - 1);
  }
};

template <int BM, int BN, int WM, int WN, int SFM, int OUT, int GRP, int NB, int LAY = 0>
__global__ void __launch_bounds__(WM* WN * 64, 1) pipe_kernel(const GemmParams p) {
  using G = Geo<BM, BN, WM, WN, SFM, NB>;
  using K = Kernel<BM, BN, WM, WN, SFM, OUT, GRP, NB, LAY>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[G::LDS_BYTES];
  const K k(p, smem);
  int bid = blockIdx.x;
  if (p.xcd_remap) {  // workgroups are dealt round-robin to the 8 XCDs
    const int per = gridDim.x / 8;
    bid = (bid % 8) * per + bid / 8;
  }
  int t = bid;
  TilePos cur = k.tile_at(t);
  if (!cur.valid) return;
  TilePos nxt = k.tile_at(t + gridDim.x);
  const int nkb = p.sf_k;  // >= NB

  // prologue: A blocks 0 and 1 and B blocks 0..NB-1 of the first tile, then block 0's
  // operands into registers
  k.copy_a_block(cur, 0, 0);
  k.copy_b_block(cur, 0, 0);
  k.copy_a_block(cur, 1, 1);
  k.copy_b_block(cur, 1, 1);
  if (NB >= 3) k.copy_b_block(cur, 2, 2);
  if (NB >= 4) k.copy_b_block(cur, 3, 3);
  Carry<K::FM> c;
  c.sbw0 = c.sbw1 = 0.f;
  if (SFM == SF_1D2D_F32) k.weight_block_scales(cur, 0, c.sbw0, c.sbw1);
  wait_and_barrier<G::LA + (NB - 1) * G::LB>();
#pragma unroll
  for (int i = 0; i < K::FM; ++i) c.af[i] = k.a_frag(0, i);
  c.bf = k.b_frag(0, 0);
  c.ebw = K::UE ? k.weight_word(0, 0) : 0u;
  k.read_scales(c, 0);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  c.acc1 = zero;
  c.acc2 = zero;
  c.pscale[0] = c.pscale[1] = 0.f;

  int as = 0, bs = 0;
  int stores = 0;
  for (;;) {
    k.tile(c, cur, nxt, nkb, as, bs, stores);
    if (!nxt.valid) break;
    cur = nxt;
    t += gridDim.x;
    nxt = k.tile_at(t + gridDim.x);
  }
  // no copy may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));
}

template <int BM, int BN, int WM, int WN, int SFM, int OUT, int GRP, int NB, int LAY = 0>
static hipError_t launch_one(const GemmParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((pipe_kernel<BM, BN, WM, WN, SFM, OUT, GRP, NB, LAY>), dim3(grid), dim3(WM * WN * 64), 0, stream,
                     p);
  return hipGetLastError();
}

// dense tiles that also run UE8M0 scales and FP4 weights (the planner's choices for large problems)
constexpr bool dense_ue8m0_tile(int bm, int bn) { return (bm == 256 && bn == 224) || (bm == 128 && bn == 192); }

// OUTS: the outputs instantiated on this wave layout (bit OUT_x set)
template <int BM, int BN, int WM, int WN, int OUTS = 7>
static hipError_t launch_dense(const GemmParams& p, int sfm, int out, int grid, hipStream_t s) {
#define DG_CASE(SF, O) \
  if constexpr ((OUTS >> O) & 1)  \
    if (sfm == SF && out == O) return launch_one<BM, BN, WM, WN, SF, O, GRP_DENSE, 2>(p, grid, s);
  DG_CASE(SF_1D2D_F32, OUT_BF16)
  DG_CASE(SF_1D2D_F32, OUT_F32)
  DG_CASE(SF_1D2D_F32, OUT_F32_C)
  if constexpr (dense_ue8m0_tile(BM, BN)) {
    DG_CASE(SF_1D1D_UE8M0, OUT_BF16)
    DG_CASE(SF_1D1D_UE8M0, OUT_F32)
  }
#undef DG_CASE
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_contig(const GemmParams& p, int sfm, int out, int grid, hipStream_t s) {
#define DG_CASE(SF, O) \
  if (sfm == SF && out == O) return launch_one<BM, BN, WM, WN, SF, O, GRP_CONTIG, 2>(p, grid, s);
  DG_CASE(SF_1D2D_F32, OUT_BF16)
  DG_CASE(SF_1D2D_F32, OUT_F32)
  DG_CASE(SF_1D1D_UE8M0, OUT_BF16)
#undef DG_CASE
  return hipErrorInvalidValue;
}

// Operands stored MN-major: dense problems on the two tiles the planner uses for large and
// for small FP8 problems, FP4 weights next to an MN-major A (fp8_fp4 tt), and contiguous groups
// with MN-major weights (m_grouped nn).
template <int LAY>
static hipError_t launch_layout(const GemmParams& p, int bm, int bn, int sfm, int grp, int out, int grid,
                                hipStream_t s) {
#define DG_CASE(BM_, BN_, WM_, WN_, SF, O, GR)                           \
  if (bm == BM_ && bn == BN_ && sfm == SF && out == O && grp == GR) \
    return launch_one<BM_, BN_, WM_, WN_, SF, O, GR, 2, LAY>(p, grid, s);
  DG_CASE(256, 224, 4, 2, SF_1D2D_F32, OUT_BF16, GRP_DENSE)
  DG_CASE(256, 224, 4, 2, SF_1D2D_F32, OUT_F32, GRP_DENSE)
  DG_CASE(256, 224, 4, 2, SF_1D1D_UE8M0, OUT_BF16, GRP_DENSE)
  DG_CASE(256, 224, 4, 2, SF_1D1D_UE8M0, OUT_F32, GRP_DENSE)
  DG_CASE(128, 192, 2, 2, SF_1D2D_F32, OUT_BF16, GRP_DENSE)
  DG_CASE(128, 192, 2, 2, SF_1D2D_F32, OUT_F32, GRP_DENSE)
  DG_CASE(128, 192, 2, 2, SF_1D2D_F32, OUT_F32_C, GRP_DENSE)
  DG_CASE(128, 192, 2, 2, SF_1D1D_UE8M0, OUT_BF16, GRP_DENSE)
  DG_CASE(128, 192, 2, 2, SF_1D1D_UE8M0, OUT_F32, GRP_DENSE)
  if constexpr (LAY == LAYOUT_A_MN) {
    DG_CASE(256, 224, 4, 2, SF_FP4_UE8M0, OUT_BF16, GRP_DENSE)
    DG_CASE(256, 224, 4, 2, SF_FP4_UE8M0, OUT_F32, GRP_DENSE)
    DG_CASE(128, 192, 2, 2, SF_FP4_UE8M0, OUT_BF16, GRP_DENSE)
    DG_CASE(128, 192, 2, 2, SF_FP4_UE8M0, OUT_F32, GRP_DENSE)
    DG_CASE(128, 192, 2, 2, SF_FP4_UE8M0, OUT_F32_C, GRP_DENSE)
  }
  if constexpr (LAY == LAYOUT_B_MN) {
    // (contiguous nn on 128x256 with 8 waves as 1x8, like dense nn below: 839 us against 1084
    // as 2x4 and 1822 with 4 waves, on 32 groups of 4096 x 7168 weights at the sustained clock)
    DG_CASE(128, 224, 2, 2, SF_1D2D_F32, OUT_BF16, GRP_CONTIG)
    DG_CASE(128, 224, 2, 2, SF_1D2D_F32, OUT_F32, GRP_CONTIG)
    DG_CASE(128, 224, 2, 2, SF_1D1D_UE8M0, OUT_BF16, GRP_CONTIG)
    DG_CASE(128, 256, 1, 8, SF_1D2D_F32, OUT_BF16, GRP_CONTIG)
    DG_CASE(128, 256, 1, 8, SF_1D2D_F32, OUT_F32, GRP_CONTIG)
    DG_CASE(128, 256, 1, 8, SF_1D1D_UE8M0, OUT_BF16, GRP_CONTIG)
  }
  if constexpr (LAY == LAYOUT_B_MN) {
    // nn on a 256-wide tile, where B takes the row-XOR staging, with 8 waves as 1x8, each wave
    // 128 rows x 32 columns: a wave reads the B columns of its own N range once per block with
    // the transposing read, and with a single wave row no two waves transpose the same columns
    // (every wave reads all 128 A rows with plain 16-byte reads instead).  91.9 us against 110.5
    // as 2x4 and 115.0 for 256x224 (4x2) on 4096x7168x2048 at the sustained clock.  (tn on this tile, 2x4:
    // 116.3 us with A in strips, 113.1 with both operands row-XOR, against 104.4 on 256x224.)
    DG_CASE(128, 256, 1, 8, SF_1D2D_F32, OUT_BF16, GRP_DENSE)
    DG_CASE(128, 256, 1, 8, SF_1D2D_F32, OUT_F32, GRP_DENSE)
  }
#undef DG_CASE
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN, int NB>
static hipError_t launch_masked(const GemmParams& p, int sfm, int out, int grid, hipStream_t s) {
#define DG_CASE(SF, O) \
  if (sfm == SF && out == O) return launch_one<BM, BN, WM, WN, SF, O, GRP_MASKED, NB>(p, grid, s);
  DG_CASE(SF_1D2D_F32, OUT_BF16)
  DG_CASE(SF_1D1D_UE8M0, OUT_BF16)
#undef DG_CASE
  return hipErrorInvalidValue;
}

}  // namespace pipe

// The file is compiled once per part (DG_PIPE_PART: dense, contiguous, masked, FP4 weights, and
// the three MN-major layouts) so the instantiations build in parallel, and once without it for
// the dispatch functions.
#if defined(DG_PIPE_PART)
#if DG_PIPE_PART == 0
hipError_t launch_pipe_dense(const GemmParams& p, int bm, int bn, int sfm, int out, int grid, hipStream_t s) {
  if (bm == 256 && bn == 224) return pipe::launch_dense<256, 224, 4, 2>(p, sfm, out, grid, s);
  if (bm == 256 && bn == 192) return pipe::launch_dense<256, 192, 4, 2>(p, sfm, out, grid, s);
  // (the 128x192 tile: 4 waves with BF16 output, whose LDS-transposed stores need each wave's
  // 4 KiB share of the scratch; 8 waves, 32x96 each, with FP32 output, where their lighter
  // register load and the second wave per SIMD measured 8% faster on FP32 + C)
  if (bm == 128 && bn == 192) {
    if (out == OUT_BF16) return pipe::launch_dense<128, 192, 2, 2, 1 << OUT_BF16>(p, sfm, out, grid, s);
    return pipe::launch_dense<128, 192, 4, 2, (1 << OUT_F32) | (1 << OUT_F32_C)>(p, sfm, out, grid, s);
  }
  if (bm == 128 && bn == 224) return pipe::launch_dense<128, 224, 2, 2>(p, sfm, out, grid, s);
  if (bm == 128 && bn == 256) return pipe::launch_dense<128, 256, 2, 2>(p, sfm, out, grid, s);
  if (bm == 128 && bn == 128) return pipe::launch_dense<128, 128, 2, 2>(p, sfm, out, grid, s);
  return hipErrorInvalidValue;
}
#elif DG_PIPE_PART == 1
hipError_t launch_pipe_contig(const GemmParams& p, int bm, int bn, int sfm, int out, int grid, hipStream_t s) {
  if (bm == 128 && bn == 224) return pipe::launch_contig<128, 224, 2, 2>(p, sfm, out, grid, s);
  if (bm == 128 && bn == 256) return pipe::launch_contig<128, 256, 2, 4>(p, sfm, out, grid, s);
  return hipErrorInvalidValue;
}
#elif DG_PIPE_PART == 2
hipError_t launch_pipe_masked(const GemmParams& p, int bm, int bn, int sfm, int out, int grid, hipStream_t s) {
  if (bm == 128 && bn == 224) return pipe::launch_masked<128, 224, 2, 2, 3>(p, sfm, out, grid, s);
  if (bm == 256 && bn == 224) return pipe::launch_masked<256, 224, 4, 2, 2>(p, sfm, out, grid, s);
  return hipErrorInvalidValue;
}
#elif DG_PIPE_PART == 3
hipError_t launch_pipe_fp4(const GemmParams& p, int bm, int bn, int grp, int out, int grid, hipStream_t s) {
  using namespace pipe;
  if (grp == GRP_DENSE) {
    if (bm == 256 && bn == 224 && out == OUT_BF16) return launch_one<256, 224, 4, 2, SF_FP4_UE8M0, OUT_BF16, GRP_DENSE, 2>(p, grid, s);
    if (bm == 256 && bn == 224 && out == OUT_F32) return launch_one<256, 224, 4, 2, SF_FP4_UE8M0, OUT_F32, GRP_DENSE, 2>(p, grid, s);
    if (bm == 256 && bn == 224 && out == OUT_F32_C) return launch_one<256, 224, 4, 2, SF_FP4_UE8M0, OUT_F32_C, GRP_DENSE, 2>(p, grid, s);
    if (bm == 128 && bn == 192 && out == OUT_BF16) return launch_one<128, 192, 2, 2, SF_FP4_UE8M0, OUT_BF16, GRP_DENSE, 2>(p, grid, s);
    if (bm == 128 && bn == 192 && out == OUT_F32) return launch_one<128, 192, 2, 2, SF_FP4_UE8M0, OUT_F32, GRP_DENSE, 2>(p, grid, s);
    if (bm == 128 && bn == 192 && out == OUT_F32_C) return launch_one<128, 192, 2, 2, SF_FP4_UE8M0, OUT_F32_C, GRP_DENSE, 2>(p, grid, s);
  } else if (grp == GRP_CONTIG && out == OUT_BF16) {
    if (bm == 128 && bn == 224) return launch_one<128, 224, 2, 2, SF_FP4_UE8M0, OUT_BF16, GRP_CONTIG, 2>(p, grid, s);
    if (bm == 128 && bn == 256) return launch_one<128, 256, 2, 2, SF_FP4_UE8M0, OUT_BF16, GRP_CONTIG, 2>(p, grid, s);
  } else if (grp == GRP_MASKED && out == OUT_BF16) {
    if (bm == 128 && bn == 224) return launch_one<128, 224, 2, 2, SF_FP4_UE8M0, OUT_BF16, GRP_MASKED, 3>(p, grid, s);
    if (bm == 256 && bn == 224) return launch_one<256, 224, 4, 2, SF_FP4_UE8M0, OUT_BF16, GRP_MASKED, 2>(p, grid, s);
  }
  return hipErrorInvalidValue;
}
#elif DG_PIPE_PART == 4
hipError_t launch_pipe_layout(const GemmParams& p, int bm, int bn, int sfm, int grp, int out, int grid, hipStream_t s) {
  return p.layout == LAYOUT_A_MN ? pipe::launch_layout<LAYOUT_A_MN>(p, bm, bn, sfm, grp, out, grid, s)
                                 : hipErrorInvalidValue;
}
#elif DG_PIPE_PART == 5
hipError_t launch_pipe_layout_b(const GemmParams& p, int bm, int bn, int sfm, int grp, int out, int grid,
                                hipStream_t s) {
  return pipe::launch_layout<LAYOUT_B_MN>(p, bm, bn, sfm, grp, out, grid, s);
}
#elif DG_PIPE_PART == 6
hipError_t launch_pipe_layout_ab(const GemmParams& p, int bm, int bn, int sfm, int grp, int out, int grid,
                                 hipStream_t s) {
  return pipe::launch_layout<LAYOUT_A_MN | LAYOUT_B_MN>(p, bm, bn, sfm, grp, out, grid, s);
}
#endif
#else  // dispatch

// Shapes with a deep-pipelined instantiation: dense problems (1d2d FP32 scales, any output;
// UE8M0 scales with BF16 or FP32 output on two tiles), contiguous groups (1d2d FP32 scales
// with BF16 or FP32 output, UE8M0 scales with BF16), and masked problems (1d2d FP32 or UE8M0
// scales, BF16) on a 128-row tile streaming B through three stages or a 256-row tile with two.
// FP4 weights: dense on the two UE8M0 tiles (BF16, FP32 or FP32 + C out), contiguous and
// masked groups on the same tiles as FP8 (BF16 out).
bool pipe_instantiated(int bm, int bn, int sfm, int grp, int out, int layout) {
  if (layout != 0) {
    // (launch_layout's list)
    if (grp == GRP_DENSE && layout == LAYOUT_B_MN && bm == 128 && bn == 256)
      return sfm == SF_1D2D_F32 && (out == OUT_BF16 || out == OUT_F32);
    const bool big = bm == 256 && bn == 224, small = bm == 128 && bn == 192;
    if (grp == GRP_DENSE && (sfm == SF_1D2D_F32 || sfm == SF_1D1D_UE8M0))
      return (big && (out == OUT_BF16 || out == OUT_F32)) ||
             (small && (out == OUT_BF16 || out == OUT_F32 || (out == OUT_F32_C && sfm == SF_1D2D_F32)));
    if (grp == GRP_DENSE && sfm == SF_FP4_UE8M0 && layout == LAYOUT_A_MN)
      return (big && (out == OUT_BF16 || out == OUT_F32)) || (small && out >= OUT_BF16 && out <= OUT_F32_C);
    if (grp == GRP_CONTIG && layout == LAYOUT_B_MN && bm == 128 && (bn == 224 || bn == 256))
      return (sfm == SF_1D2D_F32 && (out == OUT_BF16 || out == OUT_F32)) || (sfm == SF_1D1D_UE8M0 && out == OUT_BF16);
    return false;
  }
  if (sfm == SF_FP4_UE8M0) {
    if (grp == GRP_DENSE) return out >= OUT_BF16 && out <= OUT_F32_C && pipe::dense_ue8m0_tile(bm, bn);
    if (grp == GRP_CONTIG) return out == OUT_BF16 && bm == 128 && (bn == 224 || bn == 256);
    if (grp == GRP_MASKED) return out == OUT_BF16 && (bm == 128 || bm == 256) && bn == 224;
    return false;
  }
  if (grp == GRP_CONTIG) {
    const bool ok = (sfm == SF_1D2D_F32 && (out == OUT_BF16 || out == OUT_F32)) ||
                    (sfm == SF_1D1D_UE8M0 && out == OUT_BF16);
    return ok && bm == 128 && (bn == 224 || bn == 256);
  }
  if (grp == GRP_DENSE) {
    if (sfm == SF_1D1D_UE8M0) return (out == OUT_BF16 || out == OUT_F32) && pipe::dense_ue8m0_tile(bm, bn);
    if (sfm != SF_1D2D_F32 || out < OUT_BF16 || out > OUT_F32_C) return false;
    return (bm == 256 && bn == 224) || (bm == 128 && bn == 192) || (bm == 256 && bn == 192) ||
           (bm == 128 && bn == 224) || (bm == 128 && bn == 256) || (bm == 128 && bn == 128);
  }
  if (grp == GRP_MASKED) {
    if ((sfm != SF_1D2D_F32 && sfm != SF_1D1D_UE8M0) || out != OUT_BF16) return false;
    return (bm == 128 || bm == 256) && bn == 224;
  }
  return false;
}

// (the 256-row masked tile holds a whole group of up to 256 rows, so each weight slice is
// streamed once; its A stages leave room for two B stages only)
int pipe_stages_b(int bm, int bn, int grp) { return grp == GRP_MASKED && bm == 128 ? 3 : 2; }

int pipe_lds_bytes(int bm, int bn, int sfm, int grp) {
  const int sa_slot = (bm * 4 + 1023) / 1024 * 1024;
  const int sb_slot = sfm == SF_1D2D_F32 ? 0 : (bn * 4 + 1023) / 1024 * 1024;
  const int bkb = sfm == SF_FP4_UE8M0 ? pipe::BK / 2 : pipe::BK;
  return pipe::NA * (bm * pipe::BK + sa_slot) + pipe_stages_b(bm, bn, grp) * (bn * bkb + sb_slot) + 1024;
}

hipError_t launch_pipe(const GemmParams& p, int bm, int bn, int sfm, int grp, int out, int grid,
                       hipStream_t stream) {
  if (!pipe_instantiated(bm, bn, sfm, grp, out, p.layout)) return hipErrorInvalidValue;
  if (p.layout == LAYOUT_A_MN) return launch_pipe_layout(p, bm, bn, sfm, grp, out, grid, stream);
  if (p.layout == LAYOUT_B_MN) return launch_pipe_layout_b(p, bm, bn, sfm, grp, out, grid, stream);
  if (p.layout == (LAYOUT_A_MN | LAYOUT_B_MN)) return launch_pipe_layout_ab(p, bm, bn, sfm, grp, out, grid, stream);
  if (sfm == SF_FP4_UE8M0) return launch_pipe_fp4(p, bm, bn, grp, out, grid, stream);
  if (grp == GRP_MASKED) return launch_pipe_masked(p, bm, bn, sfm, out, grid, stream);
  if (grp == GRP_CONTIG) return launch_pipe_contig(p, bm, bn, sfm, out, grid, stream);
  return launch_pipe_dense(p, bm, bn, sfm, out, grid, stream);
}
#endif

}  // namespace dg
