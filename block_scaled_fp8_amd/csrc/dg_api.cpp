// C ABI of libdg.so: argument validation, tile heuristic, persistent-grid sizing
// and launch.  Validation runs before any HIP call, so every error path can be
// exercised on a machine without a GPU.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/dg.h"
#include "dg_internal.h"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_num_sms_override{0};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DG_OK;
}

int64_t align4(int64_t x) { return (x + 3) / 4 * 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

// ---------------------------------------------------------------- tile heuristic
// Relative throughput of a tile shape: the operand bytes a workgroup moves per MFMA
// fall with its arithmetic intensity BM*BN/(BM+BN), so efficiency is modelled as
// AI / (AI + 30).  Used only to rank candidates.
double tile_efficiency(const dg::TileCfg& t) {
  const double ai = double(t.bm) * t.bn / double(t.bm + t.bn);
  return ai / (ai + 30.0);
}

// generic kernel, tile kTiles[tile]
int tile_occupancy(int tile) {
  const dg::TileCfg& t = dg::kTiles[tile];
  // workgroups per CU: limited by the 160 KiB of LDS and by one wave per SIMD (4 SIMDs)
  const int lds = dg::gemm_lds_bytes(tile);
  const int by_lds = (160 * 1024) / lds;
  const int waves = t.wm * t.wn;
  const int by_simd = waves >= 4 ? 1 : 4 / waves;
  const int occ = by_lds < by_simd ? by_lds : by_simd;
  return occ < 1 ? 1 : occ;
}

struct Plan {
  int tile = -1;
  int num_m_tiles = 0, num_n_tiles = 0, tiles = 0, grid = 0;
};

// kind: 0 dense, 1 contiguous, 2 masked.  m: rows (masked: expected rows per group).
Plan plan_gemm(int kind, int m, int n, int k, int groups, int m_max, int sfm, int out, int num_sms, int layout = 0) {
  Plan best;
  double best_cost = 1e300;
  const char* force = getenv("DG_FORCE_TILE");
  int fbm = 0, fbn = 0;
  if (force && sscanf(force, "%dx%d", &fbm, &fbn) != 2) fbm = fbn = 0;
  // dense and contiguous K-major problems: whether some tile runs on the pipelined kernel (see below)
  bool any_pipe = false;
  if ((kind == 0 || kind == 1) && !layout)
    for (int t = 0; t < dg::kNumTiles; ++t)
      any_pipe = any_pipe || (dg::gemm_instantiated(t, sfm, kind, out) && k / 128 >= dg::pipe_stages_b(dg::kTiles[t].bm, dg::kTiles[t].bn, kind) &&
                              dg::pipe_instantiated(dg::kTiles[t].bm, dg::kTiles[t].bn, sfm, kind, out, 0));
  for (int t = 0; t < dg::kNumTiles; ++t) {
    const dg::TileCfg& c = dg::kTiles[t];
    // (operands stored MN-major: the pipelined kernel, except for the K-grouped form)
    if (layout && kind == dg::GRP_KGROUP) {
      if (!dg::gemm_instantiated(t, sfm, kind, out, layout)) continue;
    } else if (!layout && !dg::gemm_instantiated(t, sfm, kind, out)) {
      continue;
    }
    if (fbm && (c.bm != fbm || c.bn != fbn)) continue;
    // operands stored MN-major run on the pipelined kernel only
    if (layout && kind != dg::GRP_KGROUP &&
        (!dg::pipe_instantiated(c.bm, c.bn, sfm, kind, out, layout) || k / 128 < dg::pipe_stages_b(c.bm, c.bn, kind)))
      continue;
    // the 256-row pipelined tiles (1d2d scales) run out of registers with FP32 + C output
    // (the compiler spills them to scratch); they stay reachable only when forced
    if (!fbm && kind == 0 && out == dg::OUT_F32_C && sfm == dg::SF_1D2D_F32 && c.bm > 128) continue;
    const int64_t mt = (kind == 2) ? (m + c.bm - 1) / c.bm : (m + c.bm - 1) / c.bm;
    const int64_t nt = (n + c.bn - 1) / c.bn;
    // (masked and K-grouped: every group has its own mt x nt tiles)
    const int64_t tiles = (kind == 2 || kind == dg::GRP_KGROUP) ? int64_t(groups) * mt * nt : mt * nt;
    const int occ = tile_occupancy(t);
    const int64_t slots = int64_t(num_sms) * occ;
    const int64_t waves = (tiles + slots - 1) / slots;
    // compute time per wave of tiles ~ tile area / efficiency; occupancy shares a CU
    double cost = double(waves) * c.bm * c.bn * occ / tile_efficiency(c);
    // padding waste along M when the tile is much taller than the rows present
    if (kind == 2 && m_max > 0) {
      const double rows_done = double(mt) * c.bm;
      cost *= 1.0 + 0.15 * (rows_done / (m > 0 ? m : 1) - 1.0);
    }
    // dense and contiguous problems that the pipelined kernel can run: a tile only the generic
    // kernel has is much slower than the area model says.  Measured: dense at M = 128..256 with
    // N = 2048..7168, the generic 64x32 tile 18.9-64.6 us against 13.1-42.4 us for the
    // pipelined 128x128; contiguous groups of 640 to 2688 rows, the generic 128x128 and 64x128
    // tiles 30.1-92.3 us against 20.1-59.6 us for the pipelined 128x256.
    if (any_pipe && !dg::pipe_instantiated(c.bm, c.bn, sfm, kind, out, 0)) cost *= 3.0;
    // masked problems stream their weights: the pipelined kernel is worth some extra tiles,
    // and a pipelined tile that holds a whole group (m_max rows) streams each weight slice
    // exactly once whatever the group's row count, while its padding fragments issue no
    // MFMAs.  The area model above cannot see that (with rows spread over 0..m_max the
    // 128-row tile re-streams the weights of every group above 128 rows): measured
    // 136 against 143 us for 32 groups of up to 256 rows, so such a tile is taken outright.
    if (kind == 2 && k / 128 >= dg::pipe_stages_b(c.bm, c.bn, kind) && dg::pipe_instantiated(c.bm, c.bn, sfm, kind, out))
      cost *= c.bm >= m_max ? 0.01 : 0.8;
    // B stored [K, N] (nn): every B fragment costs four transposing LDS reads; the 256-wide
    // tile stages B row-XOR and runs 8 waves as one wave row, so each B column is transposed
    // once per block, which the area model cannot see.  Measured against the planner's other
    // tiles: 91.9 against 115.0 us (256x224) on 4096x7168x2048, 24.2 against 39.7 us (128x192,
    // 4 waves) on 512x7168x2048, 86.5 against 168.8 us on 768x4096x7168; so nn takes it, and
    // so do contiguous groups with weights stored [K, N] (839 us against 1822 with 4 waves).
    if ((kind == 0 || kind == 1) && layout == dg::LAYOUT_B_MN && c.bm == 128 && c.bn == 256) cost *= 0.4;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best.tile = t;
      best.num_m_tiles = int(mt);
      best.num_n_tiles = int(nt);
      best.tiles = int(tiles);
      const int64_t g = tiles < slots ? tiles : slots;
      best.grid = int(g < 1 ? 1 : g);
    }
  }
  return best;
}

int sf_mode_of(int32_t sf_format, int32_t gran_n) {
  if (sf_format == DG_SF_UE8M0X4) return dg::SF_1D1D_UE8M0;
  return gran_n == 128 ? dg::SF_1D2D_F32 : dg::SF_1D1D_F32;
}

// Checks shared by the three GEMM entry points.
// layout: dg::LayoutBits of the operands (m: rows of D, for an A stored [k, m]).
int check_common(int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa, const void* b,
                 int64_t ldb, const void* sfb, int64_t sfb_stride, int32_t sf_format, int32_t gran_n,
                 const void* d, int64_t ldd, int32_t d_dtype, bool empty, int layout = 0, int32_t m = 0) {
  if (d_dtype != DG_OUT_BF16 && d_dtype != DG_OUT_F32) return fail(DG_ERR_DTYPE, "d_dtype %d is not DG_OUT_BF16 or DG_OUT_F32", d_dtype);
  if (sf_format != DG_SF_F32 && sf_format != DG_SF_UE8M0X4) return fail(DG_ERR_DTYPE, "sf_format %d is not DG_SF_F32 or DG_SF_UE8M0X4", sf_format);
  if (gran_n != 1 && gran_n != 128) return fail(DG_ERR_UNSUPPORTED, "gran_n %d: weight scales are per 128x128 block (128) or per row (1)", gran_n);
  if (sf_format == DG_SF_UE8M0X4 && gran_n != 1)
    return fail(DG_ERR_UNSUPPORTED, "packed UE8M0 weight scales must be broadcast per row (gran_n == 1)");
  if (k <= 0 || k % 128 != 0) return fail(DG_ERR_SHAPE, "k = %d must be a positive multiple of 128", k);
  if (n < 0) return fail(DG_ERR_SHAPE, "n = %d is negative", n);
  if (empty) return DG_OK;  // nothing is read or written: pointers may be NULL
  if (!a || !sfa || !b || !sfb || !d) return fail(DG_ERR_NULL, "a, sfa, b, sfb and d must not be NULL");
  const bool amn = (layout & dg::LAYOUT_A_MN) != 0, bmn = (layout & dg::LAYOUT_B_MN) != 0;
  if (amn) {
    if (lda < m || lda % 16 != 0) return fail(DG_ERR_LAYOUT, "lda = %lld must be >= m (A stored [k, m]) and a multiple of 16", (long long)lda);
  } else if (lda < k || lda % 16 != 0) {
    return fail(DG_ERR_LAYOUT, "lda = %lld must be >= k and a multiple of 16", (long long)lda);
  }
  if (bmn) {
    if (ldb < n || ldb % 16 != 0) return fail(DG_ERR_LAYOUT, "ldb = %lld must be >= n (B stored [k, n]) and a multiple of 16", (long long)ldb);
  } else if (ldb < k || ldb % 16 != 0) {
    return fail(DG_ERR_LAYOUT, "ldb = %lld must be >= k and a multiple of 16", (long long)ldb);
  }
  // a tile's byte range (up to 256 rows of ld bytes) is a 32-bit signed count
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23)) return fail(DG_ERR_LAYOUT, "lda and ldb must be < 2^23 (tile byte ranges are 32-bit)");
  // an MN-major operand's byte range runs to its end
  if ((amn && int64_t(k) * lda >= (int64_t(1) << 31)) || (bmn && int64_t(k) * ldb >= (int64_t(1) << 31)))
    return fail(DG_ERR_LAYOUT, "an operand stored [k, m] or [k, n] must span less than 2^31 bytes (k * ld)");
  if (!aligned16(a) || !aligned16(b)) return fail(DG_ERR_LAYOUT, "a and b must be 16-byte aligned");
  if (!aligned16(sfa) || !aligned16(sfb)) return fail(DG_ERR_LAYOUT, "sfa and sfb must be 16-byte aligned");
  const int64_t sf_k = k / 128;
  if (gran_n == 128) {
    if (sfb_stride < sf_k) return fail(DG_ERR_LAYOUT, "sfb_stride = %lld must be >= sf_k = %lld for 128x128 weight scales", (long long)sfb_stride, (long long)sf_k);
  } else if (sfb_stride != align4(n)) {
    return fail(DG_ERR_LAYOUT, "per-row weight scales must be MN-major with stride align4(n) = %lld, got %lld", (long long)align4(n), (long long)sfb_stride);
  }
  if (ldd < n) return fail(DG_ERR_LAYOUT, "ldd = %lld must be >= n", (long long)ldd);
  const uintptr_t esz = d_dtype == DG_OUT_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(d) & (esz - 1)) != 0) return fail(DG_ERR_LAYOUT, "d is not aligned to its element size");
  return DG_OK;
}

int do_launch(dg::GemmParams& p, int kind, int32_t m_rows_for_plan, int32_t m_max, int sfm, int out,
              hipStream_t stream) {
  int num_sms = g_num_sms_override.load();
  if (num_sms <= 0) num_sms = device_cu_count();
  if (num_sms <= 0) return fail(DG_ERR_HIP, "could not query the device's compute-unit count");
  Plan pl = plan_gemm(kind, m_rows_for_plan, p.n, p.k, p.num_groups, m_max, sfm, out, num_sms, p.layout);
  if (pl.tile < 0) return fail(DG_ERR_UNSUPPORTED, "no tile configuration for this combination (check DG_FORCE_TILE)");
  const dg::TileCfg& c = dg::kTiles[pl.tile];
  p.num_n_tiles = pl.num_n_tiles;
  if (kind == 2) {
    // masked: the tile count is known on the device only; plan for every row present
    const int64_t mt = (m_max + c.bm - 1) / c.bm;
    p.num_m_tiles = int(mt);
    const int64_t upper = int64_t(p.num_groups) * mt * p.num_n_tiles;
    const int64_t slots = int64_t(num_sms) * tile_occupancy(pl.tile);
    pl.grid = int(upper < slots ? (upper < 1 ? 1 : upper) : slots);
  } else {
    p.num_m_tiles = pl.num_m_tiles;
  }
  p.total_tiles = pl.tiles;
  const int sw_default = 8;
  int sw = env_int("DG_SWIZZLE_M", sw_default);
  if (sw < 1) sw = 1;
  p.swizzle_m = sw < p.num_m_tiles ? sw : (p.num_m_tiles > 0 ? p.num_m_tiles : 1);
  p.xcd_remap = (pl.grid % 8 == 0) ? 1 : 0;
  // vector epilogue accesses need every row (and group) start 16-byte aligned
  const int esz = out == dg::OUT_BF16 ? 2 : 4;
  p.d_vec = (p.ldd % 4 == 0 && (p.d_gstride * esz) % 16 == 0 && aligned16(p.d)) ? 1 : 0;
  p.c_vec = (p.c && p.ldc % 4 == 0 && aligned16(p.c)) ? 1 : 0;
  p.d_vec16 = ((p.ldd * esz) % 16 == 0 && (p.d_gstride * esz) % 16 == 0 && aligned16(p.d)) ? 1 : 0;
  // decode-shaped dense problems (at most 64 rows, 1d2d scales) stream B with the skinny
  // kernel: 16 or 32 columns per workgroup, so the grid covers the chip
  if (kind == dg::GRP_DENSE && p.m <= 64 && sfm == dg::SF_1D2D_F32 && p.layout == 0 && !getenv("DG_FORCE_TILE") &&
      !env_int("DG_NO_SKINNY", 0)) {
    // (32 columns measured faster than 16 at n = 7168 even with 224 workgroups on 256 CUs: every
    // workgroup reads all of A, which is most of its traffic; 16 only when 32 leaves most CUs idle)
    const int bn = env_int("DG_SKINNY_BN", 2 * ((p.n + 31) / 32) >= num_sms ? 32 : 16);
    if (env_int("DG_PRINT_CONFIGS", 0)) fprintf(stderr, "[dg] skinny kernel bn=%d grid=%d\n", bn, (p.n + bn - 1) / bn);
    const hipError_t e = dg::launch_skinny(p, bn, out, stream);
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  if (env_int("DG_PRINT_CONFIGS", 0))
    fprintf(stderr, "[dg] kind=%d m=%d n=%d k=%d groups=%d sf_mode=%d out=%d -> tile %dx%d (waves %dx%d) tiles=%d grid=%d swizzle_m=%d\n",
            kind, p.m, p.n, p.k, p.num_groups, sfm, out, c.bm, c.bn, c.wm, c.wn, p.total_tiles, pl.grid,
            p.swizzle_m);
  // problems with at least as many K blocks as the deep-pipelined kernel keeps B stages run
  // that kernel when it has the chosen tile (one workgroup per CU: its LDS stages take most
  // of the 160 KiB)
  // (the planner only offers pipelined tiles for operands stored MN-major)
  const bool use_pipe = p.sf_k >= dg::pipe_stages_b(c.bm, c.bn, kind) && (p.layout || !env_int("DG_NO_PIPE", 0)) &&
                        dg::pipe_instantiated(c.bm, c.bn, sfm, kind, out, p.layout);
  if (use_pipe) {
    const int occ = (160 * 1024) / dg::pipe_lds_bytes(c.bm, c.bn, sfm, kind);
    const int64_t slots = int64_t(num_sms) * (occ < 1 ? 1 : occ);
    // masked: the tile count is known on the device only; size for every row present
    const int64_t want = kind == dg::GRP_MASKED ? int64_t(p.num_groups) * p.num_m_tiles * p.num_n_tiles : pl.tiles;
    pl.grid = int(want < slots ? (want < 1 ? 1 : want) : slots);
    p.xcd_remap = (pl.grid % 8 == 0) ? 1 : 0;
  }
  if (env_int("DG_PRINT_CONFIGS", 0) && use_pipe) fprintf(stderr, "[dg] deep-pipelined kernel, grid %d\n", pl.grid);
  const hipError_t e = use_pipe ? dg::launch_pipe(p, c.bm, c.bn, sfm, kind, out, pl.grid, stream)
                                : dg::launch_gemm(p, pl.tile, sfm, kind, out, pl.grid, stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------- FP8 x FP4
// Tiles of the pipelined kernel that take FP4 weights, ranked with the same area model as
// plan_gemm (one workgroup per CU: the LDS stages take most of the 160 KiB).
struct Fp4Tile {
  int bm, bn;
};

int launch_fp8_fp4(dg::GemmParams& p, int kind, int m_plan, int m_max, int out, hipStream_t stream) {
  int num_sms = g_num_sms_override.load();
  if (num_sms <= 0) num_sms = device_cu_count();
  if (num_sms <= 0) return fail(DG_ERR_HIP, "could not query the device's compute-unit count");
  static const Fp4Tile dense_tiles[] = {{256, 224}, {128, 192}};
  static const Fp4Tile contig_tiles[] = {{128, 256}, {128, 224}};
  static const Fp4Tile masked_tiles[] = {{256, 224}, {128, 224}};
  const Fp4Tile* cand = kind == dg::GRP_DENSE ? dense_tiles : kind == dg::GRP_CONTIG ? contig_tiles : masked_tiles;
  const char* force = getenv("DG_FORCE_TILE");
  int fbm = 0, fbn = 0;
  if (force && sscanf(force, "%dx%d", &fbm, &fbn) != 2) fbm = fbn = 0;
  int best = -1;
  double best_cost = 1e300;
  for (int i = 0; i < 2; ++i) {
    const Fp4Tile& t = cand[i];
    if (fbm && (t.bm != fbm || t.bn != fbn)) continue;
    if (!dg::pipe_instantiated(t.bm, t.bn, dg::SF_FP4_UE8M0, kind, out, p.layout)) continue;
    if (p.sf_k < dg::pipe_stages_b(t.bm, t.bn, kind)) continue;
    const int64_t mt = (m_plan + t.bm - 1) / t.bm, nt = (p.n + t.bn - 1) / t.bn;
    const int64_t tiles = (kind == dg::GRP_MASKED ? int64_t(p.num_groups) : 1) * mt * nt;
    const int64_t waves = (tiles + num_sms - 1) / num_sms;
    const double ai = double(t.bm) * t.bn / double(t.bm + t.bn);
    double cost = double(waves) * t.bm * t.bn * (ai + 30.0) / ai;
    // a masked tile that holds a whole group streams each weight slice once (see plan_gemm)
    if (kind == dg::GRP_MASKED) cost *= t.bm >= m_max ? 0.01 : 1.0;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = i;
    }
  }
  if (best < 0) return fail(DG_ERR_UNSUPPORTED, "no FP4-weight tile for this problem (k must be >= 256; check DG_FORCE_TILE)");
  const Fp4Tile& t = cand[best];
  p.num_n_tiles = (p.n + t.bn - 1) / t.bn;
  p.num_m_tiles = ((kind == dg::GRP_MASKED ? m_max : p.m) + t.bm - 1) / t.bm;
  const int64_t tiles = (kind == dg::GRP_MASKED ? int64_t(p.num_groups) : 1) * p.num_m_tiles * p.num_n_tiles;
  p.total_tiles = int(tiles);
  int sw = env_int("DG_SWIZZLE_M", 8);
  if (sw < 1) sw = 1;
  p.swizzle_m = sw < p.num_m_tiles ? sw : (p.num_m_tiles > 0 ? p.num_m_tiles : 1);
  const int grid = int(tiles < num_sms ? (tiles < 1 ? 1 : tiles) : num_sms);
  p.xcd_remap = (grid % 8 == 0) ? 1 : 0;
  const int esz = out == dg::OUT_BF16 ? 2 : 4;
  p.d_vec = (p.ldd % 4 == 0 && (p.d_gstride * esz) % 16 == 0 && aligned16(p.d)) ? 1 : 0;
  p.c_vec = (p.c && p.ldc % 4 == 0 && aligned16(p.c)) ? 1 : 0;
  p.d_vec16 = ((p.ldd * esz) % 16 == 0 && (p.d_gstride * esz) % 16 == 0 && aligned16(p.d)) ? 1 : 0;
  if (env_int("DG_PRINT_CONFIGS", 0))
    fprintf(stderr, "[dg] fp8 x fp4 kind=%d m=%d n=%d k=%d groups=%d out=%d -> tile %dx%d tiles=%d grid=%d\n", kind, p.m,
            p.n, p.k, p.num_groups, out, t.bm, t.bn, p.total_tiles, grid);
  const hipError_t e = dg::launch_pipe(p, t.bm, t.bn, dg::SF_FP4_UE8M0, kind, out, grid, stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Checks shared by the three FP8 x FP4 entry points.
int check_fp8_fp4(int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa, const void* b, int64_t ldb,
                  const void* sfb, int64_t sfb_stride, const void* d, int64_t ldd, int32_t d_dtype, bool empty,
                  int layout = 0, int32_t m = 0) {
  if (d_dtype != DG_OUT_BF16 && d_dtype != DG_OUT_F32) return fail(DG_ERR_DTYPE, "d_dtype %d is not DG_OUT_BF16 or DG_OUT_F32", d_dtype);
  if (k <= 0 || k % 128 != 0) return fail(DG_ERR_SHAPE, "k = %d must be a positive multiple of 128", k);
  if (k < 256) return fail(DG_ERR_UNSUPPORTED, "the FP8 x FP4 GEMM needs k >= 256 (two K blocks), got %d", k);
  if (n < 0) return fail(DG_ERR_SHAPE, "n = %d is negative", n);
  if (empty) return DG_OK;
  if (!a || !sfa || !b || !sfb || !d) return fail(DG_ERR_NULL, "a, sfa, b, sfb and d must not be NULL");
  if (layout & dg::LAYOUT_A_MN) {
    if (lda < m || lda % 16 != 0) return fail(DG_ERR_LAYOUT, "lda = %lld must be >= m (A stored [k, m]) and a multiple of 16", (long long)lda);
    if (int64_t(k) * lda >= (int64_t(1) << 31)) return fail(DG_ERR_LAYOUT, "an A stored [k, m] must span less than 2^31 bytes (k * lda)");
  } else if (lda < k || lda % 16 != 0) {
    return fail(DG_ERR_LAYOUT, "lda = %lld must be >= k and a multiple of 16", (long long)lda);
  }
  if (ldb < k / 2 || ldb % 16 != 0) return fail(DG_ERR_LAYOUT, "ldb = %lld (bytes of packed FP4) must be >= k / 2 and a multiple of 16", (long long)ldb);
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23)) return fail(DG_ERR_LAYOUT, "lda and ldb must be < 2^23 (tile byte ranges are 32-bit)");
  if (!aligned16(a) || !aligned16(b)) return fail(DG_ERR_LAYOUT, "a and b must be 16-byte aligned");
  if (!aligned16(sfa) || !aligned16(sfb)) return fail(DG_ERR_LAYOUT, "sfa and sfb must be 16-byte aligned");
  if (sfb_stride != align4(n)) return fail(DG_ERR_LAYOUT, "sfb must be MN-major with stride align4(n) = %lld, got %lld", (long long)align4(n), (long long)sfb_stride);
  if (ldd < n) return fail(DG_ERR_LAYOUT, "ldd = %lld must be >= n", (long long)ldd);
  const uintptr_t esz = d_dtype == DG_OUT_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(d) & (esz - 1)) != 0) return fail(DG_ERR_LAYOUT, "d is not aligned to its element size");
  return DG_OK;
}

}  // namespace

// The four operand layouts of the dense FP8 GEMM (layout: dg::LayoutBits).
static int fp8_gemm(int layout, int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                    int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                    int32_t sf_format, int32_t gran_n, const float* c, int64_t ldc, void* d, int64_t ldd,
                    int32_t d_dtype, hipStream_t stream) {
  if (m < 0) return fail(DG_ERR_SHAPE, "m = %d is negative", m);
  int st = check_common(n, k, a, lda, sfa, b, ldb, sfb, sfb_stride, sf_format, gran_n, d, ldd, d_dtype,
                        m == 0 || n == 0, layout, m);
  if (st != DG_OK) return st;
  if (layout && k < 256) return fail(DG_ERR_UNSUPPORTED, "operands stored [k, m] or [k, n] need k >= 256 (two K blocks), got %d", k);
  if (layout && sf_format == DG_SF_F32 && gran_n == 1)
    return fail(DG_ERR_UNSUPPORTED, "operands stored [k, m] or [k, n] take 128x128 FP32 or per-row UE8M0 weight scales, not per-row FP32");
  if (m == 0 || n == 0) return ok();
  if (sfa_stride != align4(m)) return fail(DG_ERR_LAYOUT, "sfa must be MN-major with stride align4(m) = %lld, got %lld", (long long)align4(m), (long long)sfa_stride);
  if (c) {
    if (d_dtype != DG_OUT_F32) return fail(DG_ERR_UNSUPPORTED, "a C term requires an FP32 output");
    if (ldc < n || (reinterpret_cast<uintptr_t>(c) & 3u) != 0) return fail(DG_ERR_LAYOUT, "c needs ldc >= n and 4-byte alignment");
    if ((const void*)c == d && ldc != ldd) return fail(DG_ERR_LAYOUT, "c aliases d, so ldc must equal ldd");
  }
  dg::GemmParams p{};
  p.a = (const uint8_t*)a; p.lda = lda;
  p.sfa = sfa; p.sfa_stride = sfa_stride;
  p.b = (const uint8_t*)b; p.ldb = ldb;
  p.sfb = sfb; p.sfb_stride = sfb_stride;
  p.c = c; p.ldc = ldc;
  p.d = d; p.ldd = ldd;
  p.m = m; p.n = n; p.k = k; p.num_groups = 1; p.sf_k = k / 128;
  p.layout = layout;
  const int out = c ? dg::OUT_F32_C : (d_dtype == DG_OUT_BF16 ? dg::OUT_BF16 : dg::OUT_F32);
  return do_launch(p, dg::GRP_DENSE, m, 0, sf_mode_of(sf_format, gran_n), out, stream);
}

// M-grouped contiguous GEMM with K-major (layout 0) or MN-major (dg::LAYOUT_B_MN) weights.
static int m_grouped_contiguous(int layout, int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                                const void* b, int64_t ldb, int64_t b_group_stride,
                                const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                int32_t sf_format, int32_t gran_n, void* d, int64_t ldd,
                                int32_t d_dtype, const int32_t* grouped_layout, hipStream_t stream) {
  if (m_total < 0) return fail(DG_ERR_SHAPE, "m_total = %d is negative", m_total);
  if (num_groups <= 0) return fail(DG_ERR_SHAPE, "num_groups = %d must be positive", num_groups);
  int st = check_common(n, k, a, lda, sfa, b, ldb, sfb, sfb_stride, sf_format, gran_n, d, ldd, d_dtype,
                        m_total == 0 || n == 0, layout, m_total);
  if (st != DG_OK) return st;
  if (layout && k < 256) return fail(DG_ERR_UNSUPPORTED, "weights stored [k, n] need k >= 256 (two K blocks), got %d", k);
  if (layout && sf_format == DG_SF_F32 && gran_n == 1)
    return fail(DG_ERR_UNSUPPORTED, "weights stored [k, n] take 128x128 FP32 or per-row UE8M0 scales, not per-row FP32");
  if (m_total == 0 || n == 0) return ok();
  if (!grouped_layout) return fail(DG_ERR_NULL, "grouped_layout must not be NULL");
  if (sfa_stride != align4(m_total)) return fail(DG_ERR_LAYOUT, "sfa must be MN-major with stride align4(m_total) = %lld, got %lld", (long long)align4(m_total), (long long)sfa_stride);
  const int64_t b_rows = layout ? int64_t(k) : int64_t(n);
  if (b_group_stride < b_rows * ldb || b_group_stride % 16 != 0) return fail(DG_ERR_LAYOUT, "b_group_stride must be >= (n or k)*ldb and a multiple of 16");
  const int64_t sfb_min = gran_n == 128 ? int64_t((n + 127) / 128) * sfb_stride
                                        : (sf_format == DG_SF_UE8M0X4 ? int64_t((k / 128 + 3) / 4) : int64_t(k / 128)) * sfb_stride;
  if (sfb_group_stride < sfb_min || (gran_n == 1 && sfb_group_stride % 4 != 0)) return fail(DG_ERR_LAYOUT, "sfb_group_stride = %lld is smaller than one group's scales (%lld) or misaligned", (long long)sfb_group_stride, (long long)sfb_min);
  dg::GemmParams p{};
  p.a = (const uint8_t*)a; p.lda = lda;
  p.sfa = sfa; p.sfa_stride = sfa_stride;
  p.b = (const uint8_t*)b; p.ldb = ldb; p.b_gstride = b_group_stride;
  p.sfb = sfb; p.sfb_stride = sfb_stride; p.sfb_gstride = sfb_group_stride;
  p.d = d; p.ldd = ldd;
  p.grouped_layout = grouped_layout;
  p.m = m_total; p.n = n; p.k = k; p.num_groups = num_groups; p.sf_k = k / 128;
  p.layout = layout;
  const int out = d_dtype == DG_OUT_BF16 ? dg::OUT_BF16 : dg::OUT_F32;
  return do_launch(p, dg::GRP_CONTIG, m_total, 0, sf_mode_of(sf_format, gran_n), out, stream);
}

// Dense FP8 x FP4 GEMM with A stored [m, k] (layout 0) or [k, m] (dg::LAYOUT_A_MN).
static int fp8_fp4_gemm(int layout, int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                        int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                        const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream) {
  if (m < 0) return fail(DG_ERR_SHAPE, "m = %d is negative", m);
  int st = check_fp8_fp4(n, k, a, lda, sfa, b, ldb, sfb, sfb_stride, d, ldd, d_dtype, m == 0 || n == 0, layout, m);
  if (st != DG_OK) return st;
  if (m == 0 || n == 0) return ok();
  if (sfa_stride != align4(m)) return fail(DG_ERR_LAYOUT, "sfa must be MN-major with stride align4(m) = %lld, got %lld", (long long)align4(m), (long long)sfa_stride);
  if (c) {
    if (d_dtype != DG_OUT_F32) return fail(DG_ERR_UNSUPPORTED, "a C term requires an FP32 output");
    if (ldc < n || (reinterpret_cast<uintptr_t>(c) & 3u) != 0) return fail(DG_ERR_LAYOUT, "c needs ldc >= n and 4-byte alignment");
    if ((const void*)c == d && ldc != ldd) return fail(DG_ERR_LAYOUT, "c aliases d, so ldc must equal ldd");
  }
  dg::GemmParams p{};
  p.a = (const uint8_t*)a; p.lda = lda;
  p.sfa = sfa; p.sfa_stride = sfa_stride;
  p.b = (const uint8_t*)b; p.ldb = ldb;
  p.sfb = sfb; p.sfb_stride = sfb_stride;
  p.c = c; p.ldc = ldc;
  p.d = d; p.ldd = ldd;
  p.m = m; p.n = n; p.k = k; p.num_groups = 1; p.sf_k = k / 128;
  p.layout = layout;
  const int out = c ? dg::OUT_F32_C : (d_dtype == DG_OUT_BF16 ? dg::OUT_BF16 : dg::OUT_F32);
  return launch_fp8_fp4(p, dg::GRP_DENSE, m, 0, out, stream);
}

// K-grouped contiguous GEMM: operands K-major (layout 0, A [m, sum K], B [n, sum K]) or both
// stored K-outermost (dg::LAYOUT_A_MN | dg::LAYOUT_B_MN: A [sum K, m], B [sum K, n]).
static int k_grouped(int layout, int32_t num_groups, int32_t m, int32_t n, const int32_t* ks, const void* a,
                     int64_t lda, const float* sfa, const void* b, int64_t ldb, const float* sfb, const float* c,
                     float* d, hipStream_t stream) {
  if (num_groups <= 0) return fail(DG_ERR_SHAPE, "num_groups = %d must be positive", num_groups);
  if (m < 0 || n < 0) return fail(DG_ERR_SHAPE, "m = %d and n = %d must not be negative", m, n);
  if (!ks) return fail(DG_ERR_NULL, "ks (host array of num_groups K sizes) must not be NULL");
  int64_t sum_k = 0;
  for (int g = 0; g < num_groups; ++g) {
    if (ks[g] < 0 || ks[g] % 128 != 0) return fail(DG_ERR_SHAPE, "ks[%d] = %d must be a non-negative multiple of 128", g, ks[g]);
    sum_k += ks[g];
  }
  if (m % 4 != 0 || n % 4 != 0) return fail(DG_ERR_SHAPE, "m = %d and n = %d must be multiples of 4", m, n);
  if (m == 0 || n == 0) return ok();
  if (!c || !d) return fail(DG_ERR_NULL, "c and d must not be NULL (c may equal d)");
  if ((reinterpret_cast<uintptr_t>(c) & 3u) != 0 || (reinterpret_cast<uintptr_t>(d) & 3u) != 0)
    return fail(DG_ERR_LAYOUT, "c and d must be 4-byte aligned");
  const int64_t mn = (int64_t)m * n;
  if (sum_k > 0) {
    if (!a || !b || !sfa || !sfb) return fail(DG_ERR_NULL, "a, sfa, b and sfb must not be NULL");
    if (sum_k >= (int64_t(1) << 31)) return fail(DG_ERR_SHAPE, "sum(ks) must be < 2^31");
    if (layout) {
      if (lda < m || ldb < n) return fail(DG_ERR_LAYOUT, "A stored [sum(ks), m] and B stored [sum(ks), n] need lda >= m and ldb >= n");
      if (sum_k * lda >= (int64_t(1) << 31) || sum_k * ldb >= (int64_t(1) << 31))
        return fail(DG_ERR_LAYOUT, "operands stored [sum(ks), x] must span less than 2^31 bytes (sum(ks) * ld)");
    } else if (lda < sum_k || ldb < sum_k) {
      return fail(DG_ERR_LAYOUT, "lda and ldb must be >= sum(ks) = %lld", (long long)sum_k);
    }
    if (lda % 16 != 0 || ldb % 16 != 0) return fail(DG_ERR_LAYOUT, "lda and ldb must be multiples of 16");
    if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23)) return fail(DG_ERR_LAYOUT, "lda and ldb must be < 2^23 (tile byte ranges are 32-bit)");
    if (!aligned16(a) || !aligned16(b) || !aligned16(sfa) || !aligned16(sfb))
      return fail(DG_ERR_LAYOUT, "a, b, sfa and sfb must be 16-byte aligned");
  }
  // everything is validated above, so an error below is a launch failure only
  for (int g = 0; g < num_groups; ++g) {
    if (ks[g] == 0 && c != d) {   // an empty group is D = C
      const hipError_t e = hipMemcpyAsync(d + g * mn, c + g * mn, mn * sizeof(float), hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) return fail(DG_ERR_HIP, "copy of C into D failed: %s", hipGetErrorString(e));
    }
  }
  if (sum_k == 0) return ok();
  int num_sms = g_num_sms_override.load();
  if (num_sms <= 0) num_sms = device_cu_count();
  if (num_sms <= 0) return fail(DG_ERR_HIP, "could not query the device's compute-unit count");
  int nonempty = 0;
  for (int g = 0; g < num_groups; ++g) nonempty += ks[g] > 0;
  // tile choice: the area model over the tiles of one launch (up to kMaxKGroups groups)
  const int plan_groups = nonempty < dg::kMaxKGroups ? nonempty : dg::kMaxKGroups;
  Plan pl = plan_gemm(dg::GRP_KGROUP, m, n, (int)(sum_k / nonempty), plan_groups, 0, dg::SF_1D1D_F32, dg::OUT_F32_C,
                      num_sms, layout);
  if (pl.tile < 0) return fail(DG_ERR_UNSUPPORTED, "no tile configuration for the K-grouped GEMM");
  const dg::TileCfg& tc = dg::kTiles[pl.tile];
  // One launch over the tiles of up to kMaxKGroups non-empty groups (the groups share the
  // scheduler, page "02 · DeepGEMM 技术解析" §5.2); more groups take more launches.
  const int per_launch = env_int("DG_KGROUP_LOOP", 0) ? 1 : dg::kMaxKGroups;
  int g = 0, kb = 0;
  while (g < num_groups) {
    dg::GemmParams p{};
    p.a = (const uint8_t*)a; p.lda = lda;
    p.sfa = sfa; p.sfa_stride = m;
    p.b = (const uint8_t*)b; p.ldb = ldb;
    p.sfb = sfb; p.sfb_stride = n;
    p.c = c; p.ldc = n; p.c_gstride = mn;
    p.d = d; p.ldd = n; p.d_gstride = mn;
    p.m = m; p.n = n; p.k = (int32_t)sum_k; p.num_groups = num_groups;
    p.layout = layout;
    int max_nkb = 0;
    for (; g < num_groups && p.kg_count < per_launch; ++g) {
      const int nkb = ks[g] / 128;
      if (nkb > 0) {
        p.kg_group[p.kg_count] = g;
        p.kg_kb0[p.kg_count] = kb;
        p.kg_nkb[p.kg_count] = nkb;
        ++p.kg_count;
      }
      kb += nkb;
      max_nkb = nkb > max_nkb ? nkb : max_nkb;
    }
    if (p.kg_count == 0) break;
    p.sf_k = max_nkb;
    p.num_m_tiles = (m + tc.bm - 1) / tc.bm;
    p.num_n_tiles = (n + tc.bn - 1) / tc.bn;
    const int64_t tiles = int64_t(p.kg_count) * p.num_m_tiles * p.num_n_tiles;
    p.total_tiles = int(tiles);
    const int sw = env_int("DG_SWIZZLE_M", 8);
    p.swizzle_m = sw < 1 ? 1 : (sw < p.num_m_tiles ? sw : p.num_m_tiles);
    const int64_t slots = int64_t(num_sms) * tile_occupancy(pl.tile);
    const int grid = int(tiles < slots ? tiles : slots);
    p.xcd_remap = (grid % 8 == 0) ? 1 : 0;
    p.d_vec = (n % 4 == 0 && aligned16(d)) ? 1 : 0;
    p.c_vec = (n % 4 == 0 && aligned16(c)) ? 1 : 0;
    p.d_vec16 = p.d_vec;
    if (env_int("DG_PRINT_CONFIGS", 0))
      fprintf(stderr, "[dg] k-grouped (layout %d): %d non-empty groups, tile %dx%d, %lld tiles, grid %d\n", layout,
              p.kg_count, tc.bm, tc.bn, (long long)tiles, grid);
    const hipError_t e = dg::launch_gemm(p, pl.tile, dg::SF_1D1D_F32, dg::GRP_KGROUP, dg::OUT_F32_C, grid, stream);
    if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

extern "C" {

int dg_fp8_gemm_nt(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                   int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                   int32_t sf_format, int32_t gran_n, const float* c, int64_t ldc, void* d, int64_t ldd,
                   int32_t d_dtype, hipStream_t stream) {
  return fp8_gemm(0, m, n, k, a, lda, sfa, sfa_stride, b, ldb, sfb, sfb_stride, sf_format, gran_n, c, ldc, d, ldd,
                  d_dtype, stream);
}

int dg_fp8_gemm_nn(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                   int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                   int32_t sf_format, int32_t gran_n, const float* c, int64_t ldc, void* d, int64_t ldd,
                   int32_t d_dtype, hipStream_t stream) {
  return fp8_gemm(dg::LAYOUT_B_MN, m, n, k, a, lda, sfa, sfa_stride, b, ldb, sfb, sfb_stride, sf_format, gran_n, c, ldc, d, ldd,
                  d_dtype, stream);
}

int dg_fp8_gemm_tn(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                   int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                   int32_t sf_format, int32_t gran_n, const float* c, int64_t ldc, void* d, int64_t ldd,
                   int32_t d_dtype, hipStream_t stream) {
  return fp8_gemm(dg::LAYOUT_A_MN | dg::LAYOUT_B_MN, m, n, k, a, lda, sfa, sfa_stride, b, ldb, sfb, sfb_stride, sf_format, gran_n, c, ldc, d, ldd,
                  d_dtype, stream);
}

int dg_fp8_gemm_tt(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                   int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                   int32_t sf_format, int32_t gran_n, const float* c, int64_t ldc, void* d, int64_t ldd,
                   int32_t d_dtype, hipStream_t stream) {
  return fp8_gemm(dg::LAYOUT_A_MN, m, n, k, a, lda, sfa, sfa_stride, b, ldb, sfb, sfb_stride, sf_format, gran_n, c, ldc, d, ldd,
                  d_dtype, stream);
}

int dg_m_grouped_fp8_gemm_nt_contiguous(int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                        const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                                        const void* b, int64_t ldb, int64_t b_group_stride,
                                        const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                        int32_t sf_format, int32_t gran_n, void* d, int64_t ldd,
                                        int32_t d_dtype, const int32_t* grouped_layout, hipStream_t stream) {
  return m_grouped_contiguous(0, m_total, n, k, num_groups, a, lda, sfa, sfa_stride, b, ldb, b_group_stride, sfb,
                              sfb_stride, sfb_group_stride, sf_format, gran_n, d, ldd, d_dtype, grouped_layout, stream);
}

int dg_m_grouped_fp8_gemm_nn_contiguous(int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                        const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                                        const void* b, int64_t ldb, int64_t b_group_stride,
                                        const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                        int32_t sf_format, int32_t gran_n, void* d, int64_t ldd,
                                        int32_t d_dtype, const int32_t* grouped_layout, hipStream_t stream) {
  return m_grouped_contiguous(dg::LAYOUT_B_MN, m_total, n, k, num_groups, a, lda, sfa, sfa_stride, b, ldb, b_group_stride, sfb,
                              sfb_stride, sfb_group_stride, sf_format, gran_n, d, ldd, d_dtype, grouped_layout, stream);
}

int dg_m_grouped_fp8_gemm_nt_masked(int32_t num_groups, int32_t m_max, int32_t n, int32_t k, const void* a,
                                    int64_t lda, int64_t a_group_stride, const void* sfa, int64_t sfa_stride,
                                    int64_t sfa_group_stride, const void* b, int64_t ldb, int64_t b_group_stride,
                                    const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride,
                                    int32_t sf_format, int32_t gran_n, void* d, int64_t ldd, int64_t d_group_stride,
                                    int32_t d_dtype, const int32_t* masked_m, int32_t expected_m,
                                    hipStream_t stream) {
  if (num_groups <= 0) return fail(DG_ERR_SHAPE, "num_groups = %d must be positive", num_groups);
  if (m_max < 0) return fail(DG_ERR_SHAPE, "m_max = %d is negative", m_max);
  int st = check_common(n, k, a, lda, sfa, b, ldb, sfb, sfb_stride, sf_format, gran_n, d, ldd, d_dtype,
                        m_max == 0 || n == 0);
  if (st != DG_OK) return st;
  if (m_max == 0 || n == 0) return ok();
  if (!masked_m) return fail(DG_ERR_NULL, "masked_m must not be NULL");
  if (sfa_stride != align4(m_max)) return fail(DG_ERR_LAYOUT, "sfa must be MN-major with stride align4(m_max) = %lld, got %lld", (long long)align4(m_max), (long long)sfa_stride);
  if (a_group_stride < int64_t(m_max) * lda || a_group_stride % 16 != 0) return fail(DG_ERR_LAYOUT, "a_group_stride must be >= m_max*lda and a multiple of 16");
  if (b_group_stride < int64_t(n) * ldb || b_group_stride % 16 != 0) return fail(DG_ERR_LAYOUT, "b_group_stride must be >= n*ldb and a multiple of 16");
  const int64_t sf_rows = sf_format == DG_SF_UE8M0X4 ? (k / 128 + 3) / 4 : k / 128;
  if (sfa_group_stride < sf_rows * sfa_stride || sfa_group_stride % 4 != 0) return fail(DG_ERR_LAYOUT, "sfa_group_stride is smaller than one group's scales or not a multiple of 4");
  const int64_t sfb_min = gran_n == 128 ? int64_t((n + 127) / 128) * sfb_stride : sf_rows * sfb_stride;
  if (sfb_group_stride < sfb_min || (gran_n == 1 && sfb_group_stride % 4 != 0)) return fail(DG_ERR_LAYOUT, "sfb_group_stride is smaller than one group's scales or misaligned");
  if (d_group_stride < int64_t(m_max) * ldd) return fail(DG_ERR_LAYOUT, "d_group_stride must be >= m_max*ldd");
  dg::GemmParams p{};
  p.a = (const uint8_t*)a; p.lda = lda; p.a_gstride = a_group_stride;
  p.sfa = sfa; p.sfa_stride = sfa_stride; p.sfa_gstride = sfa_group_stride;
  p.b = (const uint8_t*)b; p.ldb = ldb; p.b_gstride = b_group_stride;
  p.sfb = sfb; p.sfb_stride = sfb_stride; p.sfb_gstride = sfb_group_stride;
  p.d = d; p.ldd = ldd; p.d_gstride = d_group_stride;
  p.masked_m = masked_m;
  p.m = m_max; p.n = n; p.k = k; p.num_groups = num_groups; p.sf_k = k / 128;
  const int out = d_dtype == DG_OUT_BF16 ? dg::OUT_BF16 : dg::OUT_F32;
  const int em = (expected_m > 0 && expected_m < m_max) ? expected_m : m_max;
  return do_launch(p, dg::GRP_MASKED, em, m_max, sf_mode_of(sf_format, gran_n), out, stream);
}

int dg_k_grouped_fp8_gemm_nt_contiguous(int32_t num_groups, int32_t m, int32_t n, const int32_t* ks,
                                        const void* a, int64_t lda, const float* sfa, const void* b, int64_t ldb,
                                        const float* sfb, const float* c, float* d, hipStream_t stream) {
  return k_grouped(0, num_groups, m, n, ks, a, lda, sfa, b, ldb, sfb, c, d, stream);
}

int dg_k_grouped_fp8_gemm_tn_contiguous(int32_t num_groups, int32_t m, int32_t n, const int32_t* ks,
                                        const void* a, int64_t lda, const float* sfa, const void* b, int64_t ldb,
                                        const float* sfb, const float* c, float* d, hipStream_t stream) {
  return k_grouped(dg::LAYOUT_A_MN | dg::LAYOUT_B_MN, num_groups, m, n, ks, a, lda, sfa, b, ldb, sfb, c, d, stream);
}

int dg_fp8_fp4_gemm_nt(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                       int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                       const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream) {
  return fp8_fp4_gemm(0, m, n, k, a, lda, sfa, sfa_stride, b, ldb, sfb, sfb_stride, c, ldc, d, ldd, d_dtype, stream);
}

int dg_fp8_fp4_gemm_tt(int32_t m, int32_t n, int32_t k, const void* a, int64_t lda, const void* sfa,
                       int64_t sfa_stride, const void* b, int64_t ldb, const void* sfb, int64_t sfb_stride,
                       const float* c, int64_t ldc, void* d, int64_t ldd, int32_t d_dtype, hipStream_t stream) {
  return fp8_fp4_gemm(dg::LAYOUT_A_MN, m, n, k, a, lda, sfa, sfa_stride, b, ldb, sfb, sfb_stride, c, ldc, d, ldd, d_dtype, stream);
}

int dg_m_grouped_fp8_fp4_gemm_nt_contiguous(int32_t m_total, int32_t n, int32_t k, int32_t num_groups,
                                            const void* a, int64_t lda, const void* sfa, int64_t sfa_stride,
                                            const void* b, int64_t ldb, int64_t b_group_stride, const void* sfb,
                                            int64_t sfb_stride, int64_t sfb_group_stride, void* d, int64_t ldd,
                                            int32_t d_dtype, const int32_t* grouped_layout, hipStream_t stream) {
  if (m_total < 0) return fail(DG_ERR_SHAPE, "m_total = %d is negative", m_total);
  if (num_groups <= 0) return fail(DG_ERR_SHAPE, "num_groups = %d must be positive", num_groups);
  int st = check_fp8_fp4(n, k, a, lda, sfa, b, ldb, sfb, sfb_stride, d, ldd, d_dtype, m_total == 0 || n == 0);
  if (st != DG_OK) return st;
  if (m_total == 0 || n == 0) return ok();
  if (d_dtype != DG_OUT_BF16) return fail(DG_ERR_UNSUPPORTED, "the grouped FP8 x FP4 GEMMs write BF16");
  if (!grouped_layout) return fail(DG_ERR_NULL, "grouped_layout must not be NULL");
  if (sfa_stride != align4(m_total)) return fail(DG_ERR_LAYOUT, "sfa must be MN-major with stride align4(m_total) = %lld, got %lld", (long long)align4(m_total), (long long)sfa_stride);
  if (b_group_stride < int64_t(n) * ldb || b_group_stride % 16 != 0) return fail(DG_ERR_LAYOUT, "b_group_stride must be >= n*ldb and a multiple of 16");
  if (sfb_group_stride < int64_t(k / 128) * sfb_stride || sfb_group_stride % 4 != 0) return fail(DG_ERR_LAYOUT, "sfb_group_stride is smaller than one group's scales or not a multiple of 4");
  dg::GemmParams p{};
  p.a = (const uint8_t*)a; p.lda = lda;
  p.sfa = sfa; p.sfa_stride = sfa_stride;
  p.b = (const uint8_t*)b; p.ldb = ldb; p.b_gstride = b_group_stride;
  p.sfb = sfb; p.sfb_stride = sfb_stride; p.sfb_gstride = sfb_group_stride;
  p.d = d; p.ldd = ldd;
  p.grouped_layout = grouped_layout;
  p.m = m_total; p.n = n; p.k = k; p.num_groups = num_groups; p.sf_k = k / 128;
  return launch_fp8_fp4(p, dg::GRP_CONTIG, m_total, 0, dg::OUT_BF16, stream);
}

int dg_m_grouped_fp8_fp4_gemm_nt_masked(int32_t num_groups, int32_t m_max, int32_t n, int32_t k, const void* a,
                                        int64_t lda, int64_t a_group_stride, const void* sfa, int64_t sfa_stride,
                                        int64_t sfa_group_stride, const void* b, int64_t ldb, int64_t b_group_stride,
                                        const void* sfb, int64_t sfb_stride, int64_t sfb_group_stride, void* d,
                                        int64_t ldd, int64_t d_group_stride, int32_t d_dtype, const int32_t* masked_m,
                                        int32_t expected_m, hipStream_t stream) {
  if (num_groups <= 0) return fail(DG_ERR_SHAPE, "num_groups = %d must be positive", num_groups);
  if (m_max < 0) return fail(DG_ERR_SHAPE, "m_max = %d is negative", m_max);
  int st = check_fp8_fp4(n, k, a, lda, sfa, b, ldb, sfb, sfb_stride, d, ldd, d_dtype, m_max == 0 || n == 0);
  if (st != DG_OK) return st;
  if (m_max == 0 || n == 0) return ok();
  if (d_dtype != DG_OUT_BF16) return fail(DG_ERR_UNSUPPORTED, "the grouped FP8 x FP4 GEMMs write BF16");
  if (!masked_m) return fail(DG_ERR_NULL, "masked_m must not be NULL");
  if (sfa_stride != align4(m_max)) return fail(DG_ERR_LAYOUT, "sfa must be MN-major with stride align4(m_max) = %lld, got %lld", (long long)align4(m_max), (long long)sfa_stride);
  if (a_group_stride < int64_t(m_max) * lda || a_group_stride % 16 != 0) return fail(DG_ERR_LAYOUT, "a_group_stride must be >= m_max*lda and a multiple of 16");
  if (b_group_stride < int64_t(n) * ldb || b_group_stride % 16 != 0) return fail(DG_ERR_LAYOUT, "b_group_stride must be >= n*ldb and a multiple of 16");
  if (sfa_group_stride < int64_t((k / 128 + 3) / 4) * sfa_stride || sfa_group_stride % 4 != 0) return fail(DG_ERR_LAYOUT, "sfa_group_stride is smaller than one group's scales or not a multiple of 4");
  if (sfb_group_stride < int64_t(k / 128) * sfb_stride || sfb_group_stride % 4 != 0) return fail(DG_ERR_LAYOUT, "sfb_group_stride is smaller than one group's scales or not a multiple of 4");
  if (d_group_stride < int64_t(m_max) * ldd) return fail(DG_ERR_LAYOUT, "d_group_stride must be >= m_max*ldd");
  dg::GemmParams p{};
  p.a = (const uint8_t*)a; p.lda = lda; p.a_gstride = a_group_stride;
  p.sfa = sfa; p.sfa_stride = sfa_stride; p.sfa_gstride = sfa_group_stride;
  p.b = (const uint8_t*)b; p.ldb = ldb; p.b_gstride = b_group_stride;
  p.sfb = sfb; p.sfb_stride = sfb_stride; p.sfb_gstride = sfb_group_stride;
  p.d = d; p.ldd = ldd; p.d_gstride = d_group_stride;
  p.masked_m = masked_m;
  p.m = m_max; p.n = n; p.k = k; p.num_groups = num_groups; p.sf_k = k / 128;
  const int em = (expected_m > 0 && expected_m < m_max) ? expected_m : m_max;
  return launch_fp8_fp4(p, dg::GRP_MASKED, em, m_max, dg::OUT_BF16, stream);
}

int dg_transform_sf(const float* sf_in, int32_t num_groups, int32_t mn, int32_t sf_k, int32_t gran_mn,
                    int32_t pack_ue8m0, void* sf_out, int32_t* nonpow2_count, hipStream_t stream) {
  if (num_groups <= 0 || mn < 0 || sf_k <= 0) return fail(DG_ERR_SHAPE, "need num_groups > 0, mn >= 0, sf_k > 0");
  if (gran_mn != 1 && gran_mn != 128) return fail(DG_ERR_UNSUPPORTED, "gran_mn %d must be 1 or 128", gran_mn);
  if (pack_ue8m0 != 0 && pack_ue8m0 != 1) return fail(DG_ERR_DTYPE, "pack_ue8m0 must be 0 or 1");
  if (mn == 0) return ok();  // nothing is read or written
  if (!sf_in || !sf_out) return fail(DG_ERR_NULL, "sf_in and sf_out must not be NULL");
  if (!aligned16(sf_out)) return fail(DG_ERR_LAYOUT, "sf_out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(sf_in) & 3u) != 0) return fail(DG_ERR_LAYOUT, "sf_in must be 4-byte aligned");
  const hipError_t e = dg::launch_transform_sf(sf_in, num_groups, mn, sf_k, gran_mn, pack_ue8m0, sf_out,
                                               nonpow2_count, stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "transform launch failed: %s", hipGetErrorString(e));
  return ok();
}

int dg_per_token_group_cast_fp8(int32_t m, int32_t k, const void* x, int64_t ldx, int32_t x_dtype, void* q,
                                int64_t ldq, void* sf, int64_t sf_stride, int32_t sf_format, hipStream_t stream) {
  if (x_dtype != DG_IN_BF16 && x_dtype != DG_IN_F32) return fail(DG_ERR_DTYPE, "x_dtype %d is not DG_IN_BF16 or DG_IN_F32", x_dtype);
  if (sf_format != DG_SF_F32 && sf_format != DG_SF_UE8M0X4) return fail(DG_ERR_DTYPE, "sf_format %d is not DG_SF_F32 or DG_SF_UE8M0X4", sf_format);
  if (m < 0) return fail(DG_ERR_SHAPE, "m = %d is negative", m);
  if (k <= 0 || k % 128 != 0) return fail(DG_ERR_SHAPE, "k = %d must be a positive multiple of 128", k);
  if (m == 0) return ok();  // nothing is read or written: pointers may be NULL
  if (!x || !q || !sf) return fail(DG_ERR_NULL, "x, q and sf must not be NULL");
  const int64_t esz = x_dtype == DG_IN_BF16 ? 2 : 4;
  if (ldx < k || (ldx * esz) % 16 != 0 || !aligned16(x)) return fail(DG_ERR_LAYOUT, "x needs ldx >= k, 16-byte aligned rows and start");
  if (ldq < k || ldq % 8 != 0 || (reinterpret_cast<uintptr_t>(q) & 7u) != 0) return fail(DG_ERR_LAYOUT, "q needs ldq >= k, ldq a multiple of 8 and an 8-byte aligned start");
  if (sf_stride != align4(m)) return fail(DG_ERR_LAYOUT, "sf must be MN-major with stride align4(m) = %lld, got %lld", (long long)align4(m), (long long)sf_stride);
  if ((reinterpret_cast<uintptr_t>(sf) & 3u) != 0) return fail(DG_ERR_LAYOUT, "sf must be 4-byte aligned");
  const hipError_t e = dg::launch_cast(x, ldx, x_dtype == DG_IN_BF16, (uint8_t*)q, ldq, sf, sf_stride,
                                       sf_format == DG_SF_UE8M0X4, m, k, stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "cast launch failed: %s", hipGetErrorString(e));
  return ok();
}

int64_t dg_get_tma_aligned_size(int64_t mn, int32_t elem_bytes) {
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16) return -1;
  const int64_t al = 16 / elem_bytes;
  return (mn + al - 1) / al * al;
}

int32_t dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

int dg_set_num_sms(int32_t n) {
  if (n < 0) return fail(DG_ERR_SHAPE, "num_sms %d is negative", n);
  g_num_sms_override.store(n);
  return ok();
}

int32_t dg_get_num_sms(void) {
  const int o = g_num_sms_override.load();
  return o > 0 ? o : device_cu_count();
}

int dg_get_gemm_config(int32_t kind, int32_t m, int32_t n, int32_t k, int32_t num_groups, int32_t expected_m,
                       int32_t sf_format, int32_t gran_n, int32_t d_dtype, int32_t num_sms, int32_t* block_m,
                       int32_t* block_n, int32_t* num_tiles, int32_t* grid) {
  if (kind < 0 || kind > 2) return fail(DG_ERR_UNSUPPORTED, "kind %d must be 0, 1 or 2", kind);
  if (m < 0 || n <= 0 || k <= 0 || k % 128 != 0 || num_sms <= 0) return fail(DG_ERR_SHAPE, "bad sizes");
  if (d_dtype != DG_OUT_BF16 && d_dtype != DG_OUT_F32) return fail(DG_ERR_DTYPE, "bad d_dtype");
  if (sf_format != DG_SF_F32 && sf_format != DG_SF_UE8M0X4) return fail(DG_ERR_DTYPE, "bad sf_format");
  const int groups = kind == 0 ? 1 : (num_groups > 0 ? num_groups : 1);
  const int em = kind == 2 ? ((expected_m > 0 && expected_m < m) ? expected_m : m) : m;
  const int out = d_dtype == DG_OUT_BF16 ? dg::OUT_BF16 : dg::OUT_F32;
  Plan pl = plan_gemm(kind, em, n, k, groups, kind == 2 ? m : 0, sf_mode_of(sf_format, gran_n), out, num_sms);
  if (pl.tile < 0) return fail(DG_ERR_UNSUPPORTED, "no tile configuration");
  if (block_m) *block_m = dg::kTiles[pl.tile].bm;
  if (block_n) *block_n = dg::kTiles[pl.tile].bn;
  if (num_tiles) *num_tiles = pl.tiles;
  if (grid) *grid = pl.grid;
  return ok();
}

const char* dg_get_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
