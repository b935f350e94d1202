// C ABI of the GEMM library: plan creation (argument checks, device query, configuration choice),
// launch, and the host-only introspection entry points declared in include/gemm.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>

#include "gemm.h"
#include "spt_common.h"
#include "spt_kernels.h"

struct gemm_plan_s {
  int64_t M, N, K, lda, ldb, ldc;
  gemm_dtype_t in_dtype, out_dtype;
  gemm_config_t cfg;       // what gemm_run launches on the preferred path
  const void* fn_main;     // kernel for cfg (DMA or REG)
  gemm_config_t cfg_reg;   // register-staged fallback used when pointers are misaligned
  const void* fn_reg;
  int tiles_m, tiles_n;
  int tiles_m_reg, tiles_n_reg;
};

namespace {

constexpr int kMaxLds = 160 * 1024;

bool valid_in(gemm_dtype_t d) { return d == GEMM_F16 || d == GEMM_BF16; }
bool valid_out(gemm_dtype_t d) { return d == GEMM_F16 || d == GEMM_BF16 || d == GEMM_F32; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

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
bool offsets_fit(const gemm_config_t& c, int64_t lda, int64_t ldb, int64_t ldc, gemm_dtype_t out) {
  const int64_t es = out == GEMM_F32 ? 4 : 2;
  const int64_t lim = (int64_t)1 << 31;
  return (int64_t)c.bm * lda * 2 < lim && (int64_t)c.bn * ldb * 2 < lim && (int64_t)c.bm * ldc * es < lim;
}

const spt::KernelEntry* find_entry(const spt::KernelEntry* t, int n, const gemm_config_t& c) {
  for (int i = 0; i < n; ++i)
    if (t[i].bm == c.bm && t[i].bn == c.bn && t[i].bk == c.bk && t[i].stages == c.stages && t[i].waves == c.waves)
      return &t[i];
  return nullptr;
}

const spt::KernelEntry* find_entry_for_path(const gemm_config_t& c) {
  int n = 0;
  if (c.load_path == GEMM_LOAD_REG) {
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

// Preferred tiles, largest first; the first that yields at least one tile per CU wins. The 256x256
// tile runs on the two-wave-group kernel (8 waves) with the split ring of five operand slots.
struct Candidate { int bm, bn, bk, stages, waves; };
const Candidate kDmaMenu[] = {{256, 256, 64, 5, 8}, {256, 128, 64, 3, 4}, {128, 128, 64, 4, 4}, {64, 64, 64, 4, 4}};
const Candidate kRegMenu[] = {{128, 128, 64, 2, 4}, {64, 64, 64, 2, 4}};

gemm_config_t choose(int64_t M, int64_t N, const Candidate* menu, int n, int path, int cu_count, int lds_bytes) {
  gemm_config_t best{};
  int64_t best_tiles = -1;
  for (int i = 0; i < n; ++i) {
    const Candidate& c = menu[i];
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    gemm_config_t cfg{};
    cfg.bm = c.bm; cfg.bn = c.bn; cfg.bk = c.bk; cfg.stages = c.stages; cfg.waves = c.waves; cfg.mfma = 16;
    cfg.persistent = 1; cfg.group_m = 8; cfg.load_path = path;
    cfg.lds_bytes = ring_bytes(cfg);
    if (tiles >= cu_count) return cfg;
    if (tiles > best_tiles) { best = cfg; best_tiles = tiles; }
  }
  return best;
}

void finish_config(gemm_config_t& c, int64_t M, int64_t N, int cu_count, int lds_bytes, int& tm, int& tn) {
  tm = (int)ceil_div(M, c.bm);
  tn = (int)ceil_div(N, c.bn);
  const int64_t tiles = (int64_t)tm * tn;
  c.lds_bytes = ring_bytes(c);
  if (c.group_m < 1) c.group_m = 8;
  if (c.persistent) {
    int64_t g = c.grid > 0 ? c.grid : (int64_t)cu_count * groups_per_cu(c, lds_bytes);
    if (g > tiles) g = tiles;
    c.grid = (int)(g < 1 ? 1 : g);
  } else {
    c.grid = (int)(tiles < 1 ? 1 : tiles);
  }
}

gemm_status_t validate_override(const gemm_config_t& c) {
  if (c.mfma != 16 && c.mfma != 0) return GEMM_ERR_INVALID;
  if (c.load_path < GEMM_LOAD_AUTO || c.load_path > GEMM_LOAD_REG) return GEMM_ERR_INVALID;
  if (c.group_m < 0 || c.grid < 0) return GEMM_ERR_INVALID;
  return GEMM_OK;
}

gemm_status_t select_impl(int64_t M, int64_t N, int64_t K, gemm_dtype_t a, gemm_dtype_t b, gemm_dtype_t c,
                          int64_t lda, int64_t ldb, int64_t ldc, int cu_count, int lds_bytes,
                          const gemm_config_t* ovr, gemm_config_t* out, gemm_config_t* out_reg) {
  gemm_status_t st = check_args(M, N, K, a, b, c, lda, ldb, ldc);
  if (st != GEMM_OK) return st;
  if (cu_count < 1 || lds_bytes < 1) return GEMM_ERR_INVALID;
  const bool dma_ok = dma_eligible(K, lda, ldb);
  gemm_config_t cfg;
  if (ovr) {
    st = validate_override(*ovr);
    if (st != GEMM_OK) return st;
    cfg = *ovr;
    if (cfg.mfma == 0) cfg.mfma = 16;
    if (cfg.load_path == GEMM_LOAD_AUTO) cfg.load_path = dma_ok ? GEMM_LOAD_DMA : GEMM_LOAD_REG;
    if (cfg.load_path == GEMM_LOAD_DMA && !dma_ok) return GEMM_ERR_INVALID;
    cfg.lds_bytes = ring_bytes(cfg);
    if (!find_entry_for_path(cfg)) return GEMM_ERR_INVALID;
    if (cfg.lds_bytes > lds_bytes) return GEMM_ERR_INVALID;
  } else if (dma_ok) {
    cfg = choose(M, N, kDmaMenu, 4, GEMM_LOAD_DMA, cu_count, lds_bytes);
  } else {
    cfg = choose(M, N, kRegMenu, 2, GEMM_LOAD_REG, cu_count, lds_bytes);
  }
  int tm, tn;
  finish_config(cfg, M, N, cu_count, lds_bytes, tm, tn);
  if (!offsets_fit(cfg, lda, ldb, ldc, c)) return GEMM_ERR_UNSUPPORTED;
  *out = cfg;
  if (out_reg) {
    gemm_config_t r = choose(M, N, kRegMenu, 2, GEMM_LOAD_REG, cu_count, lds_bytes);
    r.persistent = cfg.persistent;
    r.group_m = cfg.group_m;
    finish_config(r, M, N, cu_count, lds_bytes, tm, tn);
    if (!offsets_fit(r, lda, ldb, ldc, c)) return GEMM_ERR_UNSUPPORTED;
    *out_reg = r;
  }
  return GEMM_OK;
}

const void* kernel_fn(const gemm_config_t& c, gemm_dtype_t in, gemm_dtype_t out) {
  const spt::KernelEntry* e = find_entry_for_path(c);
  if (!e) return nullptr;
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
                                 int lds_bytes, gemm_config_t* out) {
  if (!out) return GEMM_ERR_INVALID;
  return select_impl(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu_count, lds_bytes, nullptr, out, nullptr);
}

gemm_status_t gemm_plan_create(gemm_plan_t* out, int64_t M, int64_t N, int64_t K, gemm_dtype_t a_dtype,
                               gemm_dtype_t b_dtype, gemm_dtype_t c_dtype, int64_t lda, int64_t ldb, int64_t ldc,
                               const gemm_config_t* config) {
  if (!out) return GEMM_ERR_INVALID;
  *out = nullptr;
  gemm_status_t st = check_args(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc);
  if (st != GEMM_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_HIP;
  const int cu = prop.multiProcessorCount;
  const int lds = (int)(prop.sharedMemPerBlock < (size_t)kMaxLds ? prop.sharedMemPerBlock : (size_t)kMaxLds);

  gemm_plan_s* p = new (std::nothrow) gemm_plan_s();
  if (!p) return GEMM_ERR_NOMEM;
  p->M = M; p->N = N; p->K = K; p->lda = lda; p->ldb = ldb; p->ldc = ldc;
  p->in_dtype = a_dtype; p->out_dtype = c_dtype;
  st = select_impl(M, N, K, a_dtype, b_dtype, c_dtype, lda, ldb, ldc, cu, lds, config, &p->cfg, &p->cfg_reg);
  if (st != GEMM_OK) { delete p; return st; }
  p->fn_main = kernel_fn(p->cfg, a_dtype, c_dtype);
  p->fn_reg = kernel_fn(p->cfg_reg, a_dtype, c_dtype);
  p->tiles_m = (int)ceil_div(M, p->cfg.bm);
  p->tiles_n = (int)ceil_div(N, p->cfg.bn);
  p->tiles_m_reg = (int)ceil_div(M, p->cfg_reg.bm);
  p->tiles_n_reg = (int)ceil_div(N, p->cfg_reg.bn);
  if (!p->fn_main) { delete p; return GEMM_ERR_UNSUPPORTED; }
  *out = p;
  return GEMM_OK;
}

gemm_status_t gemm_plan_destroy(gemm_plan_t plan) {
  delete plan;
  return GEMM_OK;
}

gemm_status_t gemm_plan_describe(gemm_plan_t plan, gemm_config_t* out) {
  if (!plan || !out) return GEMM_ERR_INVALID;
  *out = plan->cfg;
  return GEMM_OK;
}

gemm_status_t gemm_run(gemm_plan_t plan, const void* A, const void* B, void* C, void* stream) {
  if (!plan) return GEMM_ERR_INVALID;
  if (plan->M == 0 || plan->N == 0) return GEMM_OK;
  if (!C || (plan->K > 0 && (!A || !B))) return GEMM_ERR_INVALID;
  const bool aligned = ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
  const gemm_config_t* cfg = &plan->cfg;
  const void* fn = plan->fn_main;
  int tm = plan->tiles_m, tn = plan->tiles_n;
  if (plan->cfg.load_path == GEMM_LOAD_DMA && !aligned) {
    if (!plan->fn_reg) return GEMM_ERR_UNSUPPORTED;
    cfg = &plan->cfg_reg;
    fn = plan->fn_reg;
    tm = plan->tiles_m_reg;
    tn = plan->tiles_n_reg;
  }
  spt::GemmArgs args;
  args.A = A; args.B = B; args.C = C;
  args.M = (int)plan->M; args.N = (int)plan->N; args.K = (int)plan->K;
  args.lda = (int)plan->lda; args.ldb = (int)plan->ldb; args.ldc = (int)plan->ldc;
  args.tiles_m = tm; args.tiles_n = tn; args.num_tiles = tm * tn;
  args.group_m = cfg->group_m;
  args.grid = cfg->grid;
  args.out_dtype = (int)plan->out_dtype;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3(cfg->grid), dim3(64 * cfg->waves), kargs, 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

int gemm_schedule_tile(int64_t tiles_m, int64_t tiles_n, int group_m, int grid, int wg, int round, int64_t* tm,
                       int64_t* tn) {
  if (tiles_m < 1 || tiles_n < 1 || group_m < 1 || grid < 1 || wg < 0 || wg >= grid || round < 0 || !tm || !tn)
    return -1;
  if (tiles_m * tiles_n > INT32_MAX) return -1;
  const int64_t t = (int64_t)round * grid + spt::xcd_remap(wg, grid);
  if (t >= tiles_m * tiles_n) return 0;
  int m, n;
  spt::grouped_raster((int)t, (int)tiles_m, (int)tiles_n, group_m, m, n);
  *tm = m;
  *tn = n;
  return 1;
}

int64_t gemm_lds_chunk_offset(int rows, int bk, int row, int chunk) {
  if ((bk != 32 && bk != 64 && bk != 128) || rows < 1 || row < 0 || row >= rows || chunk < 0 || chunk >= bk / 8)
    return -1;
  return spt::lds_chunk_offset(rows, row, chunk, bk);
}

}  // extern "C"
