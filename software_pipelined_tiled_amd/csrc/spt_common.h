// Internal definitions shared by the host plan code and the gfx950 kernels.
//
// The tile scheduler and the LDS swizzle are written once here as host+device functions, so
// the host-only introspection entry points in gemm.h report exactly what the kernels do.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPT_HD __host__ __device__ __forceinline__

namespace spt {

constexpr int kNumXcd = 8;  // MI355X: 256 CUs in 8 XCDs; workgroups are dealt round-robin over XCDs

// ---------------------------------------------------------------------------------------------
// Tile scheduler ("GEMM II — pipelining with TMA", Step 6: a fixed pool of workgroups, each
// walking many output tiles; l2_group_size groups tiles that share operands).
//
// 1. XCD remap: workgroup w runs on XCD w % 8. Logical worker ids are handed out so that the
//    workgroups of one XCD hold a contiguous range of ids, hence a contiguous run of tiles in
//    raster order, hence a compact block of the output that shares A rows and B rows in that
//    XCD's L2.
// 2. Round r of worker u processes tile t = r * grid + u (a static, precomputed assignment).
// 3. Grouped raster: tiles are ordered in bands of group_m tile-rows; inside a band the order
//    is column-major, so consecutive tiles share the same B column band and group_m A row bands.
// ---------------------------------------------------------------------------------------------
SPT_HD int xcd_remap(int w, int grid) {
  const int x = w % kNumXcd, j = w / kNumXcd;
  const int q = grid / kNumXcd, r = grid % kNumXcd;
  return x * q + (x < r ? x : r) + j;
}

SPT_HD void grouped_raster(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gm = rows_left < group_m ? rows_left : group_m;
  const int local = t - g * per_group;
  tm = first_m + local % gm;
  tn = local / gm;
}

// ---------------------------------------------------------------------------------------------
// LDS operand layout ("Async Data Movement: TMA", How TMA Writes a Swizzled Layout and The
// 128-Byte Swizzle Grouping Requirement). A tile of R rows x BK elements (16-bit) is stored as
// BK/64 groups of [R rows x 128 bytes]; each 128-byte row is eight 16-byte chunks, and logical
// chunk c of row r sits at physical chunk c XOR f(r).
//
// f(r) = r mod 8, the pages' 128-byte swizzle. Measured on gfx950 with SQ_LDS_BANK_CONFLICT
// for the MFMA operand read (16 consecutive rows at one chunk per 64-lane ds_read_b128), it is
// conflict-free, where the unswizzled layout is 4-way conflicted.
//
// A 32-element K-tile has 64-byte rows of four chunks (the pages' narrower swizzle widths for a
// box under 128 bytes). There f(r) = (r / 4) mod 4: the 16 rows one MFMA operand read touches
// then fall on 16 distinct 16-byte bank groups of a 256-byte window for every chunk, so the read
// is conflict-free however the hardware splits the 64 lanes into passes.
SPT_HD int swz(int r) { return r & 7; }
SPT_HD int swz64(int r) { return (r >> 2) & 3; }

// byte offset of logical chunk c (0 .. BK/8-1) of row r in an R-row tile with K-tile depth bk
SPT_HD int lds_chunk_offset(int R, int r, int c, int bk = 64) {
  if (bk == 32) return r * 64 + (((c & 3) ^ swz64(r)) << 4);
  return (c >> 3) * (R * 128) + r * 128 + (((c & 7) ^ swz(r)) << 4);
}

// B rows are staged in a permuted order so that, after the MFMA (which hands each lane four
// consecutive output columns per 16x16 block), a lane holds eight consecutive output columns
// across the two blocks of a pair, enabling one 16-byte store. Within each 32-row group, LDS row
// (h, g, i) = 16h + 4g + i holds global row 8g + 4h + i.
SPT_HD int b_row_perm(int rho) {
  const int base = rho & ~31, h = (rho >> 4) & 1, g = (rho >> 2) & 3, i = rho & 3;
  return base + 8 * g + 4 * h + i;
}

// The same for the 32x32 MFMA, which hands lane l the output columns 8g + 4(l/32) + e (g, e < 4) of a
// 32-column block: within each 32-row group, LDS row 8g + 4h + i holds global row
// 16(g/2) + 8h + 4(g mod 2) + i, so groups g = 0, 1 (and 2, 3) give a lane 8 consecutive columns.
SPT_HD int b_row_perm32(int rho) {
  const int base = rho & ~31, g = (rho >> 3) & 3, h = (rho >> 2) & 1, i = rho & 3;
  return base + 16 * (g >> 1) + 8 * h + 4 * (g & 1) + i;
}

// The two-group kernel's B layout. With the A fragment as the MFMA's first operand, the
// 16x16x32 MFMA hands lane l column l mod 16 of a 16x16 block, rows 4(l/16) .. 4(l/16)+3. Within
// each 128-row group, LDS row 16f + c holds global row 8c + f, so column c of B fragment f is
// output column 8c + f: a lane holds columns 8c .. 8c+7 of four rows across the eight fragments of
// its wave tile, and the 16 lanes of a quarter-wave hold one 256-byte row segment. The store path
// writes that about four times faster per CU than a quarter-wave spread over 16 rows, 16 bytes
// each, which is what the other layouts give.
SPT_HD int b_row_perm128(int rho) {
  const int base = rho & ~127, f = (rho >> 4) & 7, c = rho & 15;
  return base + 8 * c + f;
}

// Split-K work units. With `splits` K ranges per output tile, a launch has tiles_m * tiles_n *
// splits work units; unit t computes K range s = t / (tiles_m * tiles_n) of output tile number
// t mod (tiles_m * tiles_n) in the grouped raster, so units of one K range run side by side and
// share operand bands in L2 just as whole tiles do. Range s covers K-tiles [s*kt_per, (s+1)*kt_per).
SPT_HD void unit_decode(int t, int tiles_m, int tiles_n, int group_m, int& tm, int& tn, int& s) {
  const int per = tiles_m * tiles_n;
  s = t / per;
  grouped_raster(t - s * per, tiles_m, tiles_n, group_m, tm, tn);
}

// ---------------------------------------------------------------------------------------------
// The pipeline protocol's counts ("GEMM II — pipelining with TMA", Step 5: loads run ahead of the
// math through a ring of stages; "Multi-Stage Software Pipelining", Prefill and Main loop). Each
// wave issues its share of every operand tile as 1 KiB direct global->LDS loads; a wave knows a
// K-tile has landed when at most `n` of its own loads are outstanding (s_waitcnt vmcnt(n)), and the
// barrier after that wait publishes every wave's share. The kernels take every wait threshold and
// every refill count from these functions, and the host-only introspection returns the same
// values, so the CPU replays of the protocol check the numbers the kernels run with.
//
// The 4-wave DMA kernel (waves <= 4), per K-tile k:
//   prologue: the first S K-tiles (split ring: operand tiles A0 B0 A1 B1 A2) are loaded, then the
//             wave waits until K-tile 0 has landed: vmcnt(prologue_wait);
//   hand-over (before the last k-step of K-tile k): vmcnt(handover_wait) = K-tile k+1 landed, with
//             only later K-tiles in flight; then the barrier frees K-tile k's slots, and the refill
//             (K-tile k+S, or the split ring's next operand tiles) is issued: `refill_now` loads in
//             the hand-over k-step and `refill_later` in k-step 0 of the next K-tile.
// The two-group kernel (waves = 8, bm = bn = 256, bk = 64): an operand tile is `la` loads of one
// group; G0 waits vmcnt(pp_g0_prologue_wait) after its prologue (A0, B0, A1) and vmcnt(0) after each
// compute phase; G1 waits vmcnt(pp_g1_wait) after the memory phase in which it loaded A(g+2), else 0.
struct PipeProtocol {
  int la, lb, lw;       // loads per wave: an A tile, a B tile, a stage
  int split;            // five operand slots of one K-tile each (bk 64, S 5, square tile)
  int prologue_wait;
  int handover_wait;
  int refill_now, refill_later;
  int pp_g0_prologue_wait, pp_g1_wait;
  int max_wait;         // the largest threshold (vmcnt is a 6-bit counter)
};

SPT_HD constexpr PipeProtocol pipe_protocol(int bm, int bn, int bk, int s, int waves) {
  PipeProtocol p{};
  const int issuers = waves == 8 ? 4 : waves;  // two-group kernel: one group of four loads a tile
  p.la = bm * bk * 2 / 1024 / issuers;
  p.lb = bn * bk * 2 / 1024 / issuers;
  p.lw = p.la + p.lb;
  p.split = (bk == 64 && s == 5 && bm == bn) ? 1 : 0;
  const int nsub = bk / 32;  // MFMA k-steps per K-tile
  if (p.split) {
    p.prologue_wait = 2 * p.la + p.lb;  // A1 and B1 ... beyond A0 B0: only tiles after K-tile 0 outstanding
    p.handover_wait = p.la;             // only the next-but-one K-tile's A tile may be in flight
    p.refill_now = p.lb;
    p.refill_later = p.la;
  } else {
    p.prologue_wait = p.lw * (s > 1 ? s - 1 : 0);
    p.handover_wait = s > 1 ? p.lw * (s - 2) : 0;
    p.refill_now = s > 2 && nsub > 1 ? p.lw / 2 : (s >= 2 ? p.lw : 0);
    p.refill_later = s >= 2 ? p.lw - p.refill_now : 0;
  }
  p.pp_g0_prologue_wait = p.split ? p.la : 0;
  p.pp_g1_wait = p.split ? p.la : 0;
  p.max_wait = p.prologue_wait;
  return p;
}

// Kernel arguments (passed by value).
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;  // output, or the fp32 partial planes of a split-K run
  int M, N, K;
  int lda, ldb, ldc;
  int tiles_m, tiles_n, num_tiles;  // num_tiles: work units, tiles_m * tiles_n * splits
  int group_m;
  int grid;
  int out_dtype;  // 0 f16, 1 bf16, 2 f32
  int splits;     // K ranges per output tile (1: the whole K in one unit)
  int kt_per;     // K-tiles per work unit
  long long split_stride;  // bytes from the partial plane of K range s to that of s + 1
  // Dynamic schedule (4-wave kernel only): null for the static rounds. Else two counters in the
  // plan's workspace, zero at launch: [0] hands out the units after each workgroup's first one,
  // [1] counts finished workgroups; the last workgroup to finish sets both back to zero.
  int* queue;
};

}  // namespace spt
