// C ABI of the GEMM library: plan creation (argument checks, device query, configuration choice),
// launch, and the host-only introspection entry points declared in include/gemm.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "gemm.h"
#include "spt_common.h"
#include "spt_kernels.h"

struct gemm_plan_s {
  int64_t M, N, K, lda, ldb, ldc;
  gemm_dtype_t in_dtype, out_dtype;
  gemm_config_t cfg;       // what gemm_run launches on the preferred path
  const void* fn_main;     // mainloop kernel for cfg (DMA or REG; fp32 output when K is split)
  gemm_config_t cfg_reg;   // register-staged fallback used when pointers are misaligned
  const void* fn_reg;
  int tiles_m, tiles_n;
  int tiles_m_reg, tiles_n_reg;
  // workspace (device memory owned by the plan): staged operands, then the split-K partial planes
  int dev;
  char* ws;
  int64_t kp;              // K as the mainloop sees it: K, or K rounded up to 8 when staged
  int64_t stage_a_off, stage_b_off, part_off;  // byte offsets inside ws
  int64_t queue_off;       // the dynamic schedule's two counters (persistent 2), inside ws
  int64_t ldw;             // row length of a partial plane (elements)
  const void* fn_reduce;
  const void* fn_stage;
  // A plan cut in two (wave quantisation): part[0] covers output columns (split_dim 1) or rows
  // (split_dim 0) [0, split_at), part[1] the rest; each is a plan of its own over the operands this
  // plan's kernels read (its staged copies when it stages). split_dim -1: one part, this plan.
  int split_dim;
  int64_t split_at;
  gemm_plan_s* part[2];
};

namespace {

constexpr int kMaxLds = 160 * 1024;
constexpr int kGfx950Cus = 256;  // MI355X
constexpr int kMaxSplits = 16;
constexpr int64_t kMaxCutRounds = 16;  // rounds of tiles beyond which no two-part cut is tried
constexpr int kMinKtPerSplit = 8;                           // K-tiles a split-K unit keeps at least
constexpr int64_t kMaxPartialBytes = (int64_t)1 << 30;      // fp32 partial planes of a split-K plan
constexpr int64_t kMaxStageBytes = (int64_t)3 << 30;        // staged copies of A and B

bool valid_in(gemm_dtype_t d) { return d == GEMM_F16 || d == GEMM_BF16; }
bool valid_out(gemm_dtype_t d) { return d == GEMM_F16 || d == GEMM_BF16 || d == GEMM_F32; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
bool is_dma(int path) { return path == GEMM_LOAD_DMA || path == GEMM_LOAD_STAGED; }

// Workspace layout: staged A (M rows of kp elements), staged B (N rows), then `splits` fp32 planes
// of M rows of ldw = N rounded up to 8 elements, then, for a dynamic schedule, the two queue
// counters; each part starts on a 256-byte boundary.
struct WsLayout {
  int64_t stage_a, stage_b, part, queue, total, kp, ldw;
};
WsLayout ws_layout(int64_t M, int64_t N, int64_t K, int path, int splits, bool queue = false) {
  WsLayout w{};
  const bool staged = path == GEMM_LOAD_STAGED;
  w.kp = staged ? round_up(K, 8) : K;
  w.ldw = round_up(N, 8);
  const int64_t a_bytes = staged ? round_up(M * w.kp * 2, 256) : 0;
  const int64_t b_bytes = staged ? round_up(N * w.kp * 2, 256) : 0;
  w.stage_a = 0;
  w.stage_b = a_bytes;
  w.part = a_bytes + b_bytes;
  const int64_t planes_end = w.part + (splits > 1 ? (int64_t)splits * M * w.ldw * 4 : 0);
  w.queue = round_up(planes_end, 256);
  w.total = queue ? w.queue + 256 : planes_end;
  return w;
}
int64_t stage_bytes(int64_t M, int64_t N, int64_t K) { return ws_layout(M, N, K, GEMM_LOAD_STAGED, 1).total; }
int64_t partial_bytes(int64_t M, int64_t N, int splits) { return splits > 1 ? (int64_t)splits * M * round_up(N, 8) * 4 : 0; }


gemm_status_t check_args(int64_t M, int64_t N, int64_t K, gemm_dtype_t a, gemm_dtype_t b, gemm_dtype_t c,
                         int64_t lda, int64_t ldb, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return GEMM_ERR_INVALID;
  if (lda < K || ldb < K || ldc < N || lda < 1 || ldb < 1 || ldc < 1) return GEMM_ERR_INVALID;
  if (lda > INT32_MAX || ldb > INT32_MAX || ldc > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
  if (!valid_in(a) || !valid_in(b) || !valid_out(c)) return GEMM_ERR_UNSUPPORTED;
  if (a != b) return GEMM_ERR_UNSUPPORTED;
  return GEMM_OK;
}

// Offsets inside one tile are 32-bit: a tile's rows must span less than 2^31 bytes.
// The staging copy addresses a source operand through one buffer descriptor with 32-bit byte
// offsets, and reads up to 20 bytes around each 16-byte chunk (from the dword holding its first byte).
bool stage_source_fits(int64_t rows, int64_t ld, int64_t K) {
  return rows <= 0 || 4 + ((rows - 1) * ld + K) * 2 + 20 < ((int64_t)1 << 31);
}

bool offsets_fit(const gemm_config_t& c, int64_t lda, int64_t ldb, int64_t ldc, gemm_dtype_t out) {
  const int64_t es = out == GEMM_F32 ? 4 : 2;
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)c.bm * lda * 2 < lim && (int64_t)c.bn * ldb * 2 < lim && (int64_t)c.bm * ldc * es < lim;
}

const spt::KernelEntry* find_entry(const spt::KernelEntry* t, int n, const gemm_config_t& c) {
  for (int i = 0; i < n; ++i)
    if (t[i].bm == c.bm && t[i].bn == c.bn && t[i].bk == c.bk && t[i].stages == c.stages && t[i].waves == c.waves &&
        t[i].mfma == c.mfma)
      return &t[i];
  return nullptr;
}

const spt::KernelEntry* find_entry_for_path(const gemm_config_t& c) {
  int n = 0;
  if (!is_dma(c.load_path)) {
    const spt::KernelEntry* t = spt::reg_kernel_table(&n);
    return find_entry(t, n, c);
  }
  const spt::KernelEntry* t = spt::dma_kernel_table(&n);
  if (const spt::KernelEntry* e = find_entry(t, n, c)) return e;
  t = spt::pp_kernel_table(&n);
  return find_entry(t, n, c);
}

// LDS bytes of a configuration's ring: S stages of an A and a B K-tile, or, for the split ring
// (bk 64, five slots, square tile), five operand slots of one K-tile each.
int ring_bytes(const gemm_config_t& c) {
  const bool split = c.load_path != GEMM_LOAD_REG && c.bk == 64 && c.stages == 5 && c.bm == c.bn;
  return split ? c.stages * c.bm * c.bk * 2 : c.stages * (c.bm + c.bn) * c.bk * 2;
}

bool dma_eligible(int64_t K, int64_t lda, int64_t ldb) { return K % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0; }

// Workgroups one CU holds for a config: LDS-bound (registers allow one 4-wave group per CU for the
// large tiles; the small tiles fit two).
int groups_per_cu(const gemm_config_t& c, int lds_bytes) {
  int by_lds = c.lds_bytes > 0 ? lds_bytes / c.lds_bytes : 1;
  int by_regs = (c.bm * c.bn >= 128 * 128) ? 1 : 2;
  int g = by_lds < by_regs ? by_lds : by_regs;
  return g < 1 ? 1 : g;
}

// K ranges per output tile (split-K): enough work units (tiles x splits) to give every workgroup
// slot of the device one, while each range keeps at least kMinKtPerSplit K-tiles, no range is empty
// and the fp32 partial planes stay under kMaxPartialBytes. 1 when the tiles alone fill the device.
int pick_splits(const gemm_config_t& c, int64_t M, int64_t N, int64_t K, int cu_count, int lds_bytes) {
  if (!is_dma(c.load_path) || K == 0) return 1;
  const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
  const int64_t slots = (int64_t)cu_count * groups_per_cu(c, lds_bytes);
  if (tiles == 0 || tiles >= slots) return 1;  // no output (M or N is 0): nothing to split
  const int64_t kt = ceil_div(K, c.bk);
  int64_t s = slots / tiles;
  if (s > kt / kMinKtPerSplit) s = kt / kMinKtPerSplit;
  if (s > kMaxSplits) s = kMaxSplits;
  while (s > 1 && ((s - 1) * ceil_div(kt, s) >= kt || partial_bytes(M, N, (int)s) > kMaxPartialBytes)) --s;
  return s < 1 ? 1 : (int)s;
}

bool has_stream_variants(const gemm_config_t& c) {
  if (!is_dma(c.load_path)) return false;
  const spt::KernelEntry* e = find_entry_for_path(c);
  return e && e->fn_stream[0][0][0] && e->fn_stream[1][0][0];
}

// The streaming hint of the built-in choice. When all M rows fit one tile row, every B tile is read
// by one workgroup and only A is shared; B is then loaded non-temporally when it spans at least
// kStreamOnceBytes (more than the 32 MB of L2 could keep anyway), so that it takes the streaming
// replacement policy and does not displace A, and the ring is deepened to 8 stages. Likewise A when
// N fits one tile column. Measured on 32 x 8192 x 8192 f16 with B cold: 30.1 us without the hint
// (4 or 8 stages alike), 28.1 us with it at 4 stages and 26.8 us at 8. The hinted lines are not
// kept in the MALL either: a launch that repeats on a B still cached from the last one (warm) slows
// from 22.0 to 25.7 us, the price of streaming every distinct B faster.
constexpr int64_t kStreamOnceBytes = (int64_t)64 << 20;
void apply_stream_hint(gemm_config_t& c, int64_t M, int64_t N, int64_t K) {
  c.stream = 0;
  if (!has_stream_variants(c)) return;
  if (M <= c.bm && 2 * N * K >= kStreamOnceBytes)
    c.stream = 2;
  else if (N <= c.bn && 2 * M * K >= kStreamOnceBytes)
    c.stream = 1;
  if (c.stream != 0) {
    gemm_config_t deep = c;
    deep.stages = 8;
    if (has_stream_variants(deep)) c.stages = 8;
  }
}

// The tile menu, with each kernel's sustained MFMA rate per CU relative to the two-wave-group
// 256x256 kernel (measured on large square problems: about 1450, 1160, 1020 and 500 TFLOP/s). The
// 64x64 tile with 128-deep K-tiles keeps twice the bytes of the 64-deep one in flight: it is there
// for the skinny shapes, whose time is the operand stream rather than the MFMAs. Its rate is set
// above the streaming bounds below (on 32 x 8192 x 8192 it measured 0.52 of the 256x256 kernel's
// per-CU rate while streaming B at 5.8 TB/s), so that the model takes those bounds for it.
struct Candidate { int bm, bn, bk, stages, waves; double rate; };
const Candidate kDmaMenu[] = {{256, 256, 64, 5, 8, 1.0}, {256, 128, 64, 3, 4, 0.8}, {128, 128, 64, 4, 4, 0.7},
                              {64, 64, 64, 4, 4, 0.35}, {64, 64, 128, 4, 4, 0.6}, {32, 32, 128, 4, 2, 0.3}};
const Candidate kRegMenu[] = {{128, 128, 64, 2, 4, 0.35}, {64, 64, 64, 2, 4, 0.2}};
constexpr int kDmaMenuSize = (int)(sizeof(kDmaMenu) / sizeof(kDmaMenu[0]));
constexpr int kRegMenuSize = (int)(sizeof(kRegMenu) / sizeof(kRegMenu[0]));

// Modelled time of a configuration (seconds), the largest of three bounds, plus the reduction:
//   * MFMA: the rounds of work units every workgroup slot runs, each unit its MFMA work at the
//     kernel's rate plus about one K-tile of fill and store;
//   * ring: each unit streams (bm + bn) rows of its K range through a ring that holds S-1 of its S
//     K-tiles in flight, and a load takes about kLoadLatency to land, so a workgroup moves at most
//     (S-1)/S of its ring bytes per kLoadLatency;
//   * HBM: A, B and C once each at the sustained streaming rate;
// and, for a split K, the fp32 partial planes written and read back by the reduction. The ring and
// HBM bounds decide only the skinny shapes (few flops per operand byte); on the others the MFMA
// bound is several times larger.
constexpr double kCuFlops = 1450e12 / 256;  // two-wave-group kernel, per CU
constexpr double kHbmBytes = 4.5e12;        // streaming rate of the reduction
constexpr double kHbmStream = 6.0e12;       // operand streaming rate of a whole launch
constexpr double kLoadLatency = 1.0e-6;     // fitted: a 64x64 tile streams about 48 KiB/us per 64 KiB of ring
double model_time(const gemm_config_t& c, double rate, int64_t M, int64_t N, int64_t K, int cu_count,
                  int lds_bytes) {
  const int gpc = groups_per_cu(c, lds_bytes);
  const int64_t units = ceil_div(M, c.bm) * ceil_div(N, c.bn) * c.splits;
  const int64_t rounds = ceil_div(units, (int64_t)cu_count * gpc);
  const int64_t kt_per = ceil_div(ceil_div(K, c.bk), c.splits);
  const double unit = 2.0 * c.bm * c.bn * (double)(kt_per + 1) * c.bk / (rate * kCuFlops / gpc);
  const double unit_bytes = 2.0 * (c.bm + c.bn) * (double)kt_per * c.bk;
  const double in_flight = (double)ring_bytes(c) * (c.stages > 1 ? c.stages - 1 : 1) / c.stages;
  const double ring = rounds * unit_bytes * kLoadLatency / in_flight;
  const double hbm = (2.0 * (double)(M + N) * K + 4.0 * (double)M * N) / kHbmStream;
  const double reduce = c.splits > 1 ? (2.0 * partial_bytes(M, N, c.splits) + 2.0 * M * N) / kHbmBytes : 0.0;
  double t = rounds * unit;
  if (ring > t) t = ring;
  if (hbm > t) t = hbm;
  return t + reduce;
}

// Workgroups of a configuration that run at once: its work units, up to the device's slots.
int64_t active_groups(const gemm_config_t& c, int64_t M, int64_t N, int cu_count, int lds_bytes) {
  const int64_t units = ceil_div(M, c.bm) * ceil_div(N, c.bn) * c.splits;
  const int64_t slots = (int64_t)cu_count * groups_per_cu(c, lds_bytes);
  return units < slots ? units : slots;
}

// The candidate of least modelled time, each with K unsplit and with K split as pick_splits says. A
// tile whose padded grid is more than half padding is passed over (unless it is the last). Where the
// operand stream bounds the time (the skinny shapes) several tiles model alike; within 1 % the one
// that keeps more workgroups streaming is taken: on 32 x 8192 x 8192, 256 workgroups of 32x32 tiles
// streamed B from HBM 1.2x faster than 128 of 64x64 (30.0 against 36.3 us with B cold, 21.9 against
// 25.4 us warm), at the same modelled time.
gemm_config_t choose(int64_t M, int64_t N, int64_t K, const Candidate* menu, int n, int path, int cu_count,
                     int lds_bytes) {
  gemm_config_t best{};
  double best_t = 0.0;
  int64_t best_active = 0;
  bool have = false;
  for (int i = 0; i < n; ++i) {
    const Candidate& c = menu[i];
    const int64_t tm = ceil_div(M, c.bm), tn = ceil_div(N, c.bn);
    if (i + 1 < n && 2 * M * N < tm * c.bm * tn * c.bn) continue;
    gemm_config_t cfg{};
    cfg.bm = c.bm; cfg.bn = c.bn; cfg.bk = c.bk; cfg.stages = c.stages; cfg.waves = c.waves; cfg.mfma = 16;
    cfg.persistent = 1; cfg.group_m = 8; cfg.load_path = path;
    cfg.lds_bytes = ring_bytes(cfg);
    const int split = pick_splits(cfg, M, N, K, cu_count, lds_bytes);
    for (int sp : {1, split}) {
      cfg.splits = sp;
      const double t = model_time(cfg, c.rate, M, N, K, cu_count, lds_bytes);
      const int64_t active = active_groups(cfg, M, N, cu_count, lds_bytes);
      const bool alike = have && t <= 1.01 * best_t && best_t <= 1.01 * t;
      if (!have || (alike ? active > best_active : t < best_t)) {
        best = cfg;
        best_t = t;
        best_active = active;
        have = true;
      }
    }
  }
  apply_stream_hint(best, M, N, K);
  return best;
}

// Relative MFMA rate of a configuration: its menu entry's, else that of the same tile at another ring
// depth (the streaming hint deepens the 32x32 ring), else 0.2.
double rate_of(const gemm_config_t& c) {
  const bool reg = c.load_path == GEMM_LOAD_REG;
  const Candidate* menu = reg ? kRegMenu : kDmaMenu;
  const int n = reg ? kRegMenuSize : kDmaMenuSize;
  double same_tile = 0.0;
  for (int i = 0; i < n; ++i) {
    if (menu[i].bm != c.bm || menu[i].bn != c.bn || menu[i].bk != c.bk || menu[i].waves != c.waves) continue;
    if (menu[i].stages == c.stages) return menu[i].rate;
    if (same_tile == 0.0) same_tile = menu[i].rate;
  }
  return same_tile > 0.0 ? same_tile : 0.2;
}

// The single configuration `choose` picks and its modelled time.
double best_single(int64_t M, int64_t N, int64_t K, int path, int cu_count, int lds_bytes, gemm_config_t* out) {
  *out = choose(M, N, K, kDmaMenu, kDmaMenuSize, path, cu_count, lds_bytes);
  return model_time(*out, rate_of(*out), M, N, K, cu_count, lds_bytes);
}

// Wave quantisation: with T tiles on G workgroup slots, a last round of T mod G tiles runs at a
// fraction of the device. Cutting the output in two, a first part of whole rounds of one tile size
// and the rest planned on its own (the same menu and model: smaller tiles, or K split), can cost
// less than the rounds of the single choice. Each menu tile and each cut along N or M that gives
// the first part k whole rounds is modelled; a cut is taken when it is modelled at least 10 %
// faster than the single choice, counting one more kernel launch.
struct Parts {
  int dim;     // 1: columns cut at `at`; 0: rows
  int64_t at;
  gemm_config_t first, second;
};
constexpr double kLaunchSeconds = 5e-6;
bool choose_parts(int64_t M, int64_t N, int64_t K, int cu_count, int lds_bytes, Parts* out) {
  if (M <= 0 || N <= 0 || K <= 0) return false;
  gemm_config_t single;
  const double t_single = best_single(M, N, K, GEMM_LOAD_DMA, cu_count, lds_bytes, &single);
  double best = 0.9 * t_single;
  bool have = false;
  for (const Candidate& c : kDmaMenu) {
    gemm_config_t cfg{};
    cfg.bm = c.bm; cfg.bn = c.bn; cfg.bk = c.bk; cfg.stages = c.stages; cfg.waves = c.waves; cfg.mfma = 16;
    cfg.persistent = 1; cfg.group_m = 8; cfg.load_path = GEMM_LOAD_DMA; cfg.splits = 1;
    cfg.lds_bytes = ring_bytes(cfg);
    const int64_t tm = ceil_div(M, c.bm), tn = ceil_div(N, c.bn), T = tm * tn;
    const int64_t G = (int64_t)cu_count * groups_per_cu(cfg, lds_bytes);
    // a cut only pays for the idle part of the last round; past kMaxCutRounds rounds that is under the
    // 10 % the cut must save, and the search over the rounds would only cost host time
    if (T <= G || T % G == 0 || T / G > kMaxCutRounds) continue;
    for (int dim = 1; dim >= 0; --dim) {
      for (int64_t k = 1; k <= T / G; ++k) {
        const int64_t lines = dim == 1 ? (k * G) / tm : (k * G) / tn;  // tile columns (rows) of part 0
        if (lines < 1 || lines >= (dim == 1 ? tn : tm)) continue;
        const int64_t at = lines * (dim == 1 ? c.bn : c.bm);
        const int64_t M0 = dim == 1 ? M : at, N0 = dim == 1 ? at : N;
        const int64_t M1 = dim == 1 ? M : M - at, N1 = dim == 1 ? N - at : N;
        const double t0 = model_time(cfg, c.rate, M0, N0, K, cu_count, lds_bytes);
        gemm_config_t second;
        const double t1 = best_single(M1, N1, K, GEMM_LOAD_DMA, cu_count, lds_bytes, &second);
        const double t = t0 + t1 + kLaunchSeconds;
        if (t < best) {
          best = t;
          have = true;
          out->dim = dim;
          out->at = at;
          out->first = cfg;
          apply_stream_hint(out->first, M0, N0, K);
          out->second = second;
        }
      }
    }
  }
  return have;
}

void finish_config(gemm_config_t& c, int64_t M, int64_t N, int cu_count, int lds_bytes, int& tm, int& tn) {
  tm = (int)ceil_div(M, c.bm);
  tn = (int)ceil_div(N, c.bn);
  if (c.splits < 1) c.splits = 1;
  const int64_t units = (int64_t)tm * tn * c.splits;
  c.lds_bytes = ring_bytes(c);
  if (c.group_m < 1) c.group_m = 8;
  // a band of group_m tile rows taller than the grid orders the tiles exactly as one of tm rows; the
  // clamp also keeps group_m * tn, which the raster computes in 32 bits, within tm * tn
  if (tm >= 1 && c.group_m > tm) c.group_m = tm;
  if (c.persistent) {
    int64_t g = c.grid > 0 ? c.grid : (int64_t)cu_count * groups_per_cu(c, lds_bytes);
    if (g > units) g = units;
    c.grid = (int)(g < 1 ? 1 : g);
  } else {
    c.grid = (int)(units < 1 ? 1 : units);
  }
}

gemm_status_t validate_override(const gemm_config_t& c) {
  if (c.mfma != 16 && c.mfma != 32 && c.mfma != 0) return GEMM_ERR_INVALID;
  if (c.persistent < 0 || c.persistent > 2) return GEMM_ERR_INVALID;
  if (c.load_path < GEMM_LOAD_AUTO || c.load_path > GEMM_LOAD_STAGED) return GEMM_ERR_INVALID;
  if (c.group_m < 0 || c.grid < 0) return GEMM_ERR_INVALID;
  if (c.splits < 0 || c.splits > kMaxSplits) return GEMM_ERR_INVALID;
  if (c.stream < 0 || c.stream > 2) return GEMM_ERR_INVALID;
  return GEMM_OK;
}

gemm_status_t select_impl(int64_t M, int64_t N, int64_t K, gemm_dtype_t a, gemm_dtype_t b, gemm_dtype_t c,
                          int64_t lda, int64_t ldb, int64_t ldc, int cu_count, int lds_bytes,
                          const gemm_config_t* ovr, gemm_config_t* out, gemm_config_t* out_reg) {
  gemm_status_t st = check_args(M, N, K, a, b, c, lda, ldb, ldc);
  if (st != GEMM_OK) return st;
  if (cu_count < 1 || lds_bytes < 1) return GEMM_ERR_INVALID;
  const bool dma_ok = dma_eligible(K, lda, ldb);
  const bool stage_ok = stage_bytes(M, N, K) <= kMaxStageBytes && stage_source_fits(M, lda, K) &&
                        stage_source_fits(N, ldb, K);
  gemm_config_t cfg;
  if (ovr) {
    st = validate_override(*ovr);
    if (st != GEMM_OK) return st;
    cfg = *ovr;
    if (cfg.mfma == 0) cfg.mfma = 16;
    if (cfg.splits == 0) cfg.splits = 1;
    if (cfg.load_path == GEMM_LOAD_AUTO)
      cfg.load_path = dma_ok ? GEMM_LOAD_DMA : (stage_ok ? GEMM_LOAD_STAGED : GEMM_LOAD_REG);
    if (cfg.load_path == GEMM_LOAD_DMA && !dma_ok) return GEMM_ERR_INVALID;
    if (cfg.load_path == GEMM_LOAD_STAGED && !stage_ok) return GEMM_ERR_UNSUPPORTED;
    if (cfg.load_path == GEMM_LOAD_REG && cfg.splits > 1) return GEMM_ERR_INVALID;
    if (partial_bytes(M, N, cfg.splits) > kMaxPartialBytes) return GEMM_ERR_UNSUPPORTED;
    cfg.lds_bytes = ring_bytes(cfg);
    if (!find_entry_for_path(cfg)) return GEMM_ERR_INVALID;
    if (cfg.lds_bytes > lds_bytes) return GEMM_ERR_INVALID;
    // the dynamic queue is built into the 4-wave DMA kernel, for rings that leave it 16 bytes of LDS
    if (cfg.persistent == 2 && (cfg.waves == 8 || cfg.load_path == GEMM_LOAD_REG || cfg.lds_bytes + 16 > kMaxLds))
      return GEMM_ERR_UNSUPPORTED;
    if (cfg.stream != 0 && !has_stream_variants(cfg)) return GEMM_ERR_UNSUPPORTED;
  } else if (dma_ok) {
    cfg = choose(M, N, K, kDmaMenu, kDmaMenuSize, GEMM_LOAD_DMA, cu_count, lds_bytes);
  } else if (stage_ok) {
    cfg = choose(M, N, round_up(K, 8), kDmaMenu, kDmaMenuSize, GEMM_LOAD_STAGED, cu_count, lds_bytes);
  } else {
    cfg = choose(M, N, K, kRegMenu, kRegMenuSize, GEMM_LOAD_REG, cu_count, lds_bytes);
  }
  const int group_m_in = cfg.group_m < 1 ? 8 : cfg.group_m;  // before the clamp to this tile grid
  int tm, tn;
  finish_config(cfg, M, N, cu_count, lds_bytes, tm, tn);
  if ((int64_t)tm * tn * cfg.splits > INT32_MAX) return GEMM_ERR_UNSUPPORTED;  // units are numbered in 32 bits
  // the mainloop reads staged operands with rows of kp elements, and a split run writes fp32
  // planes with rows of ldw elements
  const WsLayout w = ws_layout(M, N, K, cfg.load_path, cfg.splits);
  const bool staged = cfg.load_path == GEMM_LOAD_STAGED;
  if (!offsets_fit(cfg, staged ? w.kp : lda, staged ? w.kp : ldb, ldc, c)) return GEMM_ERR_UNSUPPORTED;
  if (cfg.splits > 1 && !offsets_fit(cfg, staged ? w.kp : lda, staged ? w.kp : ldb, w.ldw, GEMM_F32))
    return GEMM_ERR_UNSUPPORTED;
  *out = cfg;
  if (out_reg) {
    gemm_config_t r = choose(M, N, K, kRegMenu, kRegMenuSize, GEMM_LOAD_REG, cu_count, lds_bytes);
    r.persistent = cfg.persistent;
    r.group_m = group_m_in;
    finish_config(r, M, N, cu_count, lds_bytes, tm, tn);
    if ((int64_t)tm * tn > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (!offsets_fit(r, lda, ldb, ldc, c)) return GEMM_ERR_UNSUPPORTED;
    *out_reg = r;
  }
  return GEMM_OK;
}

const void* kernel_fn(const gemm_config_t& c, gemm_dtype_t in, gemm_dtype_t out) {
  const spt::KernelEntry* e = find_entry_for_path(c);
  if (!e) return nullptr;
  if (c.stream == 1 || c.stream == 2) return e->fn_stream[c.stream - 1][in == GEMM_BF16 ? 1 : 0][(int)out];
  return e->fn[in == GEMM_BF16 ? 1 : 0][(int)out];
}

}  // namespace

extern "C" {

const char* gemm_status_string(gemm_status_t s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID: return "GEMM_ERR_INVALID";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
    case GEMM_ERR_NOMEM: return "GEMM_ERR_NOMEM";
  }
  return "GEMM_ERR_UNKNOWN";
}

gemm_status_t gemm_select_config(int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype, gemm_dtype_t b_dtype,
                                 gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc, int cu_count,
                                 int lds_bytes, const gemm_config_t* config, gemm_config_t* out) {
  if (!out) return GEMM_ERR_INVALID;
  return select_impl(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count, lds_bytes, config, out, nullptr);
}

}  // extern "C"

namespace {

// Where a plan's parts and workspace come from: the heap and hipMalloc (gemm_plan_create), or,
// for gemm_run_noalloc, plan records supplied by the caller and the static scratch array.
struct PlanArena {
  gemm_plan_s* spare;   // records for the parts of a plan cut in two
  int spare_left;
  char* scratch;        // device address of the scratch array (per device)
  int64_t cap, used;    // its size and the bytes handed out so far (256-byte aligned pieces)
};

// Fill *p for C[M,N] = A[M,K]·B[N,K]ᵀ on device `dev` (cu compute units, lds bytes of LDS per
// workgroup). Arguments are already checked. With arena == nullptr, parts are allocated on the heap
// and the workspace with hipMalloc (freed by gemm_plan_destroy); with an arena, nothing is
// allocated and a workspace beyond the scratch left is GEMM_ERR_UNSUPPORTED.
gemm_status_t plan_build(gemm_plan_s* p, int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype,
                         gemm_dtype_t b_dtype, gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc,
                         const gemm_config_t* config, int dev, int cu, int lds, PlanArena* arena) {
  p->M = M; p->N = N; p->K = K; p->lda = lda; p->ldb = ldb; p->ldc = ldc;
  p->in_dtype = a_dtype; p->out_dtype = c_dtype;
  p->dev = dev;
  p->split_dim = -1;
  p->queue_off = -1;
  p->ws = nullptr;
  p->part[0] = p->part[1] = nullptr;
  gemm_status_t st =
      select_impl(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu, lds, config, &p->cfg, &p->cfg_reg);
  if (st != GEMM_OK) return st;
  // the built-in choice may cut the output in two (wave quantisation); each part is a plan over
  // the operands the kernels read: the staged copies (rows of K rounded up to 8) or A and B
  const bool staged_path = p->cfg.load_path == GEMM_LOAD_STAGED;
  Parts parts;
  if (!config && is_dma(p->cfg.load_path) &&
      choose_parts(M, N, staged_path ? round_up(K, 8) : K, cu, lds, &parts)) {
    const int64_t kk = staged_path ? round_up(K, 8) : K;
    const int64_t la = staged_path ? kk : lda, lb = staged_path ? kk : ldb;
    const int64_t M0 = parts.dim == 1 ? M : parts.at, N0 = parts.dim == 1 ? parts.at : N;
    const int64_t M1 = parts.dim == 1 ? M : M - parts.at, N1 = parts.dim == 1 ? N - parts.at : N;
    const int64_t mm[2] = {M0, M1}, nn[2] = {N0, N1};
    const gemm_config_t* pc[2] = {&parts.first, &parts.second};
    for (int i = 0; i < 2 && st == GEMM_OK; ++i) {
      gemm_plan_s* q = nullptr;
      if (arena) {
        if (arena->spare_left < 1) return GEMM_ERR_UNSUPPORTED;
        q = arena->spare++;
        --arena->spare_left;
      } else {
        q = new (std::nothrow) gemm_plan_s();
        if (!q) { st = GEMM_ERR_NOMEM; break; }
      }
      p->part[i] = q;
      st = plan_build(q, mm[i], nn[i], kk, a_dtype, b_dtype, c_dtype, la, lb, ldc, pc[i], dev, cu, lds, arena);
    }
    if (st != GEMM_OK) return st;
    p->split_dim = parts.dim;
    p->split_at = parts.at;
    p->cfg.splits = 1;  // this plan only stages (when it does); the parts run the mainloops
  }
  const bool split = p->cfg.splits > 1;
  p->fn_main = kernel_fn(p->cfg, a_dtype, split ? GEMM_F32 : c_dtype);
  p->fn_reg = kernel_fn(p->cfg_reg, a_dtype, c_dtype);
  p->fn_reduce = split ? spt::splitk_reduce_fn((int)c_dtype) : nullptr;
  p->fn_stage = p->cfg.load_path == GEMM_LOAD_STAGED ? spt::stage_fn() : nullptr;
  p->tiles_m = (int)ceil_div(M, p->cfg.bm);
  p->tiles_n = (int)ceil_div(N, p->cfg.bn);
  p->tiles_m_reg = (int)ceil_div(M, p->cfg_reg.bm);
  p->tiles_n_reg = (int)ceil_div(N, p->cfg_reg.bn);
  if (!p->fn_main) return GEMM_ERR_UNSUPPORTED;
  const WsLayout w = ws_layout(M, N, K, p->cfg.load_path, p->split_dim >= 0 ? 1 : p->cfg.splits,
                               p->split_dim < 0 && p->cfg.persistent == 2);
  p->queue_off = p->split_dim < 0 && p->cfg.persistent == 2 ? w.queue : -1;
  p->kp = w.kp;
  p->ldw = w.ldw;
  p->stage_a_off = w.stage_a;
  p->stage_b_off = w.stage_b;
  p->part_off = w.part;
  if (w.total > 0 && M > 0 && N > 0) {
    if (arena) {
      // only the built-in choice runs here, and it never takes the dynamic queue, whose counters
      // would have to start at zero; every other workspace byte a launch reads it has written
      if (p->queue_off >= 0) return GEMM_ERR_UNSUPPORTED;
      const int64_t at = round_up(arena->used, 256);
      if (at + w.total > arena->cap) return GEMM_ERR_UNSUPPORTED;
      p->ws = arena->scratch + at;
      arena->used = at + w.total;
      return GEMM_OK;
    }
    void* ws = nullptr;
    if (hipMalloc(&ws, (size_t)w.total) != hipSuccess) {
      (void)hipGetLastError();
      return GEMM_ERR_NOMEM;
    }
    p->ws = (char*)ws;
    // the queue counters start at zero; each launch leaves them at zero again
    if (p->queue_off >= 0 && hipMemset(p->ws + p->queue_off, 0, 8) != hipSuccess) {
      (void)hipGetLastError();
      return GEMM_ERR_HIP;
    }
  }
  return GEMM_OK;
}

// The current device, its CU count and LDS per workgroup; GEMM_ERR_HIP unless it is a gfx950.
gemm_status_t device_info(int* dev, int* cu, int* lds) {
  if (hipGetDevice(dev) != hipSuccess) return GEMM_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, *dev) != hipSuccess) return GEMM_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_HIP;
  *cu = prop.multiProcessorCount;
  *lds = (int)(prop.sharedMemPerBlock < (size_t)kMaxLds ? prop.sharedMemPerBlock : (size_t)kMaxLds);
  return GEMM_OK;
}

}  // namespace

extern "C" {

gemm_status_t gemm_plan_create(gemm_plan_t* out, int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype,
                               gemm_dtype_t b_dtype, gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc,
                               const gemm_config_t* config) {
  if (!out) return GEMM_ERR_INVALID;
  *out = nullptr;
  gemm_status_t st = check_args(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc);
  if (st != GEMM_OK) return st;
  if (config) {
    // An override is validated before the device query, against the CU count and LDS of the
    // device the kernels are built for, so a bad configuration reports its own status on any host.
    gemm_config_t checked;
    st = select_impl(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, kGfx950Cus, kMaxLds, config, &checked,
                     nullptr);
    if (st != GEMM_OK) return st;
  }
  int dev = 0, cu = 0, lds = 0;
  st = device_info(&dev, &cu, &lds);
  if (st != GEMM_OK) return st;
  gemm_plan_s* p = new (std::nothrow) gemm_plan_s();
  if (!p) return GEMM_ERR_NOMEM;
  st = plan_build(p, M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, config, dev, cu, lds, nullptr);
  if (st != GEMM_OK) {
    (void)gemm_plan_destroy(p);
    return st;
  }
  *out = p;
  return GEMM_OK;
}

gemm_status_t gemm_plan_destroy(gemm_plan_t plan) {
  if (!plan) return GEMM_OK;
  gemm_status_t st = GEMM_OK;
  for (gemm_plan_s* part : plan->part) {
    const gemm_status_t sp = gemm_plan_destroy(part);
    if (sp != GEMM_OK) st = sp;
  }
  if (plan->ws) {
    int cur = 0;
    const bool switched = hipGetDevice(&cur) == hipSuccess && cur != plan->dev && hipSetDevice(plan->dev) == hipSuccess;
    if (hipFree(plan->ws) != hipSuccess) {
      (void)hipGetLastError();
      st = GEMM_ERR_HIP;
    }
    if (switched) (void)hipSetDevice(cur);
  }
  delete plan;
  return st;
}

gemm_status_t gemm_plan_describe(gemm_plan_t plan, gemm_config_t* out) {
  if (!plan || !out) return GEMM_ERR_INVALID;
  *out = plan->cfg;
  if (plan->part[0]) {  // part 0's mainloop, on this plan's load path
    *out = plan->part[0]->cfg;
    out->load_path = plan->cfg.load_path;
  }
  return GEMM_OK;
}

gemm_status_t gemm_plan_parts(gemm_plan_t plan, int* dim, int64_t* at, gemm_config_t* first, gemm_config_t* second) {
  if (!plan || !dim || !at) return GEMM_ERR_INVALID;
  *dim = plan->split_dim;
  *at = plan->split_dim >= 0 ? plan->split_at : 0;
  if (first) *first = plan->part[0] ? plan->part[0]->cfg : plan->cfg;
  if (second && plan->part[1]) *second = plan->part[1]->cfg;
  return GEMM_OK;
}

gemm_status_t gemm_select_parts(int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype, gemm_dtype_t b_dtype,
                                gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc, int cu_count,
                                int lds_bytes, int* dim, int64_t* at, gemm_config_t* first, gemm_config_t* second) {
  if (!dim || !at) return GEMM_ERR_INVALID;
  gemm_config_t single;
  const gemm_status_t st =
      select_impl(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count, lds_bytes, nullptr, &single, nullptr);
  if (st != GEMM_OK) return st;
  *dim = -1;
  *at = 0;
  if (first) *first = single;
  Parts parts;
  const bool staged = single.load_path == GEMM_LOAD_STAGED;
  if (!is_dma(single.load_path) || !choose_parts(M, N, staged ? round_up(K, 8) : K, cu_count, lds_bytes, &parts))
    return GEMM_OK;
  *dim = parts.dim;
  *at = parts.at;
  gemm_config_t c0 = parts.first, c1 = parts.second;
  int tm, tn;
  finish_config(c0, parts.dim == 1 ? M : parts.at, parts.dim == 1 ? parts.at : N, cu_count, lds_bytes, tm, tn);
  finish_config(c1, parts.dim == 1 ? M : M - parts.at, parts.dim == 1 ? N - parts.at : N, cu_count, lds_bytes, tm,
                tn);
  if (first) *first = c0;
  if (second) *second = c1;
  return GEMM_OK;
}

gemm_status_t gemm_plan_workspace_bytes(gemm_plan_t plan, int64_t* out) {
  if (!plan || !out) return GEMM_ERR_INVALID;
  *out = plan->ws ? ws_layout(plan->M, plan->N, plan->K, plan->cfg.load_path, plan->split_dim >= 0 ? 1 : plan->cfg.splits,
                              plan->queue_off >= 0).total
                 : 0;
  for (gemm_plan_s* part : plan->part) {
    int64_t b = 0;
    if (part && gemm_plan_workspace_bytes(part, &b) == GEMM_OK) *out += b;
  }
  return GEMM_OK;
}

static gemm_status_t launch(const void* fn, int grid, int threads, void* arg, void* stream) {
  void* kargs[] = {arg};
  if (hipLaunchKernel(fn, dim3(grid), dim3(threads), kargs, 0, (hipStream_t)stream) != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

// blocks of 256 threads for a streaming pass over `chunks` 8-element chunks: one chunk per thread,
// at most 16 blocks per CU's worth (the kernels loop over the rest)
static int stream_grid(int64_t chunks) {
  const int64_t b = ceil_div(chunks, 256);
  return (int)(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

gemm_status_t gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, void* stream) {
  if (!plan) return GEMM_ERR_INVALID;
  if (plan->M == 0 || plan->N == 0) return GEMM_OK;
  if (!C || (plan->K > 0 && (!A || !B))) return GEMM_ERR_INVALID;
  const bool aligned = ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
  const gemm_config_t* cfg = &plan->cfg;
  const void* fn = plan->fn_main;
  int tm = plan->tiles_m, tn = plan->tiles_n;
  int64_t K = plan->K, lda = plan->lda, ldb = plan->ldb;
  gemm_status_t st;
  if (cfg->load_path == GEMM_LOAD_STAGED) {
    if (K > 0) {
      spt::StageArgs g;
      g.A = A; g.B = B;
      g.dA = plan->ws + plan->stage_a_off;
      g.dB = plan->ws + plan->stage_b_off;
      g.rows_a = (int)plan->M; g.rows_b = (int)plan->N; g.K = (int)K;
      g.lda = (int)lda; g.ldb = (int)ldb; g.ldd = (int)plan->kp;
      st = launch(plan->fn_stage, stream_grid((plan->M + plan->N) * (plan->kp / 8)), 256, &g, stream);
      if (st != GEMM_OK) return st;
      A = g.dA;
      B = g.dB;
      K = lda = ldb = plan->kp;
    }
  }
  if (plan->split_dim >= 0) {
    // the two parts, over the same (possibly staged) operands: part 1 starts `split_at` columns
    // (rows) into B and C (A and C)
    st = gemm_run(plan->part[0], A, B, C, stream);
    if (st != GEMM_OK) return st;
    const int64_t es = plan->out_dtype == GEMM_F32 ? 4 : 2, at = plan->split_at;
    const char* A1 = (const char*)A + (plan->split_dim == 0 ? at * lda * 2 : 0);
    const char* B1 = (const char*)B + (plan->split_dim == 1 ? at * ldb * 2 : 0);
    char* C1 = (char*)C + (plan->split_dim == 1 ? at * es : at * plan->ldc * es);
    return gemm_run(plan->part[1], A1, B1, C1, stream);
  }
  if (cfg->load_path == GEMM_LOAD_DMA && !aligned) {
    if (!plan->fn_reg) return GEMM_ERR_UNSUPPORTED;
    cfg = &plan->cfg_reg;
    fn = plan->fn_reg;
    tm = plan->tiles_m_reg;
    tn = plan->tiles_n_reg;
  }
  const int splits = cfg->splits > 1 ? cfg->splits : 1;
  spt::GemmArgs args;
  args.A = A; args.B = B; args.C = C;
  args.M = (int)plan->M; args.N = (int)plan->N; args.K = (int)K;
  args.lda = (int)lda; args.ldb = (int)ldb; args.ldc = (int)plan->ldc;
  args.tiles_m = tm; args.tiles_n = tn; args.num_tiles = tm * tn * splits;
  args.group_m = cfg->group_m;
  args.grid = cfg->grid;
  args.out_dtype = (int)plan->out_dtype;
  args.splits = splits;
  args.kt_per = (int)ceil_div(ceil_div(K, cfg->bk), splits);
  args.split_stride = 0;
  args.queue = cfg == &plan->cfg && plan->queue_off >= 0 ? (int*)(plan->ws + plan->queue_off) : nullptr;
  if (splits > 1) {
    args.C = plan->ws + plan->part_off;
    args.ldc = (int)plan->ldw;
    args.out_dtype = (int)GEMM_F32;
    args.split_stride = (long long)plan->M * plan->ldw * 4;
  }
  st = launch(fn, cfg->grid, 64 * cfg->waves, &args, stream);
  if (st != GEMM_OK || splits == 1) return st;
  spt::ReduceArgs r;
  r.W = (const float*)(plan->ws + plan->part_off);
  r.plane = (long long)plan->M * plan->ldw;
  r.splits = splits;
  r.M = (int)plan->M; r.N = (int)plan->N; r.ldw = (int)plan->ldw;
  r.C = C;
  r.ldc = (int)plan->ldc;
  return launch(plan->fn_reduce, stream_grid(plan->M * ceil_div(plan->N, 8)), 256, &r, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// The no-allocation entry point. Its workspace (staged operand copies, split-K partial planes) is
// this file-scope device array: each device that runs it holds its own copy from the library's
// first use on that device until the process ends. Host code reaches a device's copy only through
// the address hipGetSymbolAddress returns with that device current (the array's name is a host-side
// stand-in, not a device address).
constexpr int64_t kScratchBytes = GEMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
struct ScratchDevice {
  bool ready;
  int cu, lds;
  char* ptr;  // this device's copy of `scratch`
};
ScratchDevice g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's properties and scratch address, found on its first use.
gemm_status_t scratch_device(int* dev, int* cu, int* lds, char** ptr) {
  if (hipGetDevice(dev) != hipSuccess) return GEMM_ERR_HIP;
  if (*dev < 0 || *dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDevice& d = g_scratch_dev[*dev];
  if (!d.ready) {
    int dv = 0;
    const gemm_status_t st = device_info(&dv, &d.cu, &d.lds);
    if (st != GEMM_OK) return st;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return GEMM_ERR_HIP;
    }
    d.ptr = (char*)p;
    d.ready = true;
  }
  *cu = d.cu;
  *lds = d.lds;
  *ptr = d.ptr;
  return GEMM_OK;
}

}  // namespace

extern "C" {

gemm_status_t gemm_run_noalloc(int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype, gemm_dtype_t b_dtype,
                               gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc, const void* A,
                               const void* B, void* C, void* stream) {
  gemm_status_t st = check_args(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  if (!C || (K > 0 && (!A || !B))) return GEMM_ERR_INVALID;
  int dev = 0, cu = 0, lds = 0;
  char* sp = nullptr;
  st = scratch_device(&dev, &cu, &lds, &sp);
  if (st != GEMM_OK) return st;
  gemm_plan_s plans[3] = {};  // the plan and the two parts of a plan cut in two, on this stack
  PlanArena arena{plans + 1, 2, sp, kScratchBytes, 0};
  st = plan_build(&plans[0], M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, nullptr, dev, cu, lds, &arena);
  if (st != GEMM_OK) return st;
  return gemm_run(&plans[0], A, B, C, stream);
}

int gemm_schedule_tile(int64_t tiles_m, int64_t tiles_n, int splits, int group_m, int grid, int wg, int round,
                       int64_t* tm, int64_t* tn, int* split) {
  if (tiles_m < 1 || tiles_n < 1 || splits < 1 || group_m < 1 || grid < 1 || wg < 0 || wg >= grid || round < 0 ||
      !tm || !tn || !split)
    return -1;
  if (tiles_m * tiles_n * splits > INT32_MAX) return -1;
  const int64_t t = (int64_t)round * grid + spt::xcd_remap(wg, grid);
  if (t >= tiles_m * tiles_n * splits) return 0;
  if (group_m > tiles_m) group_m = (int)tiles_m;  // the same order; keeps group_m * tiles_n in 32 bits
  int m, n, s;
  spt::unit_decode((int)t, (int)tiles_m, (int)tiles_n, group_m, m, n, s);
  *tm = m;
  *tn = n;
  *split = s;
  return 1;
}

int gemm_pipeline_protocol(int bm, int bn, int bk, int stages, int waves, int* out, int n_out) {
  if (!out || n_out < 10) return -1;
  gemm_config_t c{};
  c.bm = bm; c.bn = bn; c.bk = bk; c.stages = stages; c.waves = waves; c.mfma = 16; c.load_path = GEMM_LOAD_DMA;
  if (!find_entry_for_path(c)) return -1;
  const spt::PipeProtocol p = spt::pipe_protocol(bm, bn, bk, stages, waves);
  const int v[10] = {p.la, p.lb, p.lw, p.split, p.prologue_wait, p.handover_wait, p.refill_now, p.refill_later,
                     p.pp_g0_prologue_wait, p.pp_g1_wait};
  for (int i = 0; i < 10; ++i) out[i] = v[i];
  return 10;
}

int64_t gemm_lds_chunk_offset(int rows, int bk, int row, int chunk) {
  if ((bk != 32 && bk != 64 && bk != 128) || rows < 1 || row < 0 || row >= rows || chunk < 0 || chunk >= bk / 8)
    return -1;
  return spt::lds_chunk_offset(rows, row, chunk, bk);
}

}  // extern "C"
