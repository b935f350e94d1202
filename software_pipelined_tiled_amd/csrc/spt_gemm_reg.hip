// Register-staged variant of the pipelined GEMM (the "vectorized thread copy" path that the
// "B200 TMA Pipeline Designer" checklist keeps for copies a bulk engine cannot describe).
//
// Used when K, lda or ldb is not a multiple of 8 elements, or when A or B is not 16-byte
// aligned: 16-byte direct-to-LDS loads would then straddle rows or read past K. Each thread
// copies 16-byte chunks global -> VGPR -> LDS (same swizzled layout, same B row order, same
// MFMA loop and epilogue as the DMA kernel); a chunk that crosses K is loaded element by
// element and zero-filled past K. Two LDS stages: tile k+1 is written from registers at the
// end of tile k, and tile k+2's global loads are issued right after the hand-over barrier, so
// they are in flight while tile k+1 is computed. One barrier per K-tile.
// One stage (S = 1) is the synchronous relay of "GEMM II — pipelining with TMA" (Forced move:
// every thread loads, writes the tile and waits, then the tile is computed): per K-tile the global
// loads, the LDS writes, a barrier, the MFMAs, and a second barrier before the slot is rewritten.
// It is kept as the first rung of the stage-count ablation.
#include "spt_device.h"
#include "spt_kernels.h"

namespace spt {

// 8 consecutive 16-bit elements starting at element k of a row whose first element is at byte
// `row_off` of `r`; elements at k' >= K are zero. Any 2-byte alignment.
__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t r, bool row_ok, unsigned row_off, int k, int K) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (!row_ok || k >= K) return v;
  if (k + 8 <= K) return __builtin_amdgcn_raw_buffer_load_b128(r, row_off + 2u * (unsigned)k, 0, 0);
  unsigned h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    h[e] = (k + e < K) ? (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, row_off + 2u * (unsigned)(k + e), 0, 0) : 0u;
  v[0] = h[0] | (h[1] << 16);
  v[1] = h[2] | (h[3] << 16);
  v[2] = h[4] | (h[5] << 16);
  v[3] = h[6] | (h[7] << 16);
  return v;
}

template <int BM, int BN, int BK, int S, int WM, int WN, typename TIn, int OUT>
__global__ void __launch_bounds__(WM* WN * 64, 1) gemm_reg_kernel(GemmArgs args) {
  static_assert(S == 1 || S == 2, "one stage (serial) or two");
  using T = TileShape<BM, BN, BK, S, WM, WN>;
  constexpr int CPR = BK / 8;                          // chunks per row
  constexpr int CA = BM * CPR / T::NT, CB = BN * CPR / T::NT;  // chunks per thread per stage
  static_assert(BM * CPR % T::NT == 0 && BN * CPR % T::NT == 0, "chunks divide evenly over threads");
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int M = args.M, N = args.N, K = args.K;
  const int KT = (K + BK - 1) / BK;

  int a_rd[T::NSUB], b_rd[T::NSUB];
#pragma unroll
  for (int s = 0; s < T::NSUB; ++s) {
    a_rd[s] = lds_chunk_offset(BM, wm * T::TM + (lane & 15), 4 * s + (lane >> 4));
    b_rd[s] = T::A_BYTES + lds_chunk_offset(BN, wn * T::TN + (lane & 15), 4 * s + (lane >> 4));
  }

  const int u = xcd_remap(blockIdx.x, args.grid);
  bool first_tile = true;
  for (int t = u; t < args.num_tiles; t += args.grid) {
    int tm, tn;
    grouped_raster(t, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int row0 = tm * BM, col0 = tn * BN;
    const int rows_left = M - row0, cols_left = N - col0;
    const bool full_tile = rows_left >= BM && cols_left >= BN;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc((const char*)args.A + (size_t)row0 * args.lda * 2, ((uint64_t)(rows_left - 1) * args.lda + K) * 2);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc((const char*)args.B + (size_t)col0 * args.ldb * 2, ((uint64_t)(cols_left - 1) * args.ldb + K) * 2);

    u32x4 sa[CA], sb[CB];  // staged chunks of the next K-tile
    auto gload = [&](int kt) {
      const int k0 = kt * BK;
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int q = tid + T::NT * i, row = q / CPR, c = q % CPR;
        sa[i] = load_chunk(ra, row < rows_left, (unsigned)(row * args.lda) * 2u, k0 + 8 * c, K);
      }
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int q = tid + T::NT * i, rho = q / CPR, c = q % CPR;
        const int row = b_row_perm(rho);
        sb[i] = load_chunk(rb, row < cols_left, (unsigned)(row * args.ldb) * 2u, k0 + 8 * c, K);
      }
    };
    auto lstore = [&](int slot) {
      char* base = smem + slot * T::STAGE;
#pragma unroll
      for (int i = 0; i < CA; ++i) {
        const int q = tid + T::NT * i;
        *(u32x4*)(base + lds_chunk_offset(BM, q / CPR, q % CPR)) = sa[i];
      }
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const int q = tid + T::NT * i;
        *(u32x4*)(base + T::A_BYTES + lds_chunk_offset(BN, q / CPR, q % CPR)) = sb[i];
      }
    };

    u32x4 xf[2][T::FN], yf[2][T::FM];
    auto read_frags = [&](int slot, int sub, int buf) {
      const char* base = smem + slot * T::STAGE;
#pragma unroll
      for (int f = 0; f < T::FN; ++f) xf[buf][f] = *(const u32x4*)(base + b_rd[sub] + f * 2048);
#pragma unroll
      for (int f = 0; f < T::FM; ++f) yf[buf][f] = *(const u32x4*)(base + a_rd[sub] + f * 2048);
    };

    f32x4 acc[T::FN][T::FM];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    auto k_tile = [&](int k, int slot, auto first_c) {
      constexpr bool kFirst = decltype(first_c)::value;
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub) {
        const int buf = sub & 1;
        if (sub + 1 < T::NSUB) {
          read_frags(slot, sub + 1, buf ^ 1);
        } else if (k + 1 < KT) {
          lstore(slot ^ 1);  // tile k+1: its slot was released at the previous hand-over
          wait_lgkmcnt0();   // own LDS writes and reads of `slot` complete
          barrier_sync();    // tile k+1 visible everywhere; `slot` released everywhere
          if (k + 2 < KT) gload(k + 2);
          read_frags(slot ^ 1, 0, buf ^ 1);
        }
#pragma unroll
        for (int i = 0; i < T::FN; ++i)
#pragma unroll
          for (int j = 0; j < T::FM; ++j)
            acc[i][j] = mfma16<TIn>(xf[buf][i], yf[buf][j], (kFirst && sub == 0) ? zero4 : acc[i][j]);
      }
    };

    const int es = OUT == 2 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc((char*)args.C + (size_t)row0 * args.ldc * es, ((uint64_t)(rows_left - 1) * args.ldc + N) * es);
    if (KT == 0) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int pu = 0; pu < T::FN / 2; ++pu)
        for (int j = 0; j < T::FM; ++j)
          store8<OUT, true>(z, rc, wm * T::TM + 16 * j + (lane & 15), rows_left,
                            col0 + wn * T::TN + 32 * pu + 8 * (lane >> 4), N, args.ldc);
      continue;
    }

    if (!first_tile) {
      wait_lgkmcnt0();
      barrier_sync();
    }
    first_tile = false;
    if constexpr (S == 1) {
      // the synchronous relay: load, write, wait, compute, then free the slot for the next K-tile
      auto serial_tile = [&](int k, auto first_c) {
        constexpr bool kFirst = decltype(first_c)::value;
        if (k > 0) {
          wait_lgkmcnt0();  // this wave's reads of the slot are done
          barrier_sync();   // ... and every other wave's
        }
        gload(k);
        lstore(0);
        wait_lgkmcnt0();
        barrier_sync();  // the tile is in LDS for every wave
        read_frags(0, 0, 0);
#pragma unroll
        for (int sub = 0; sub < T::NSUB; ++sub) {
          const int buf = sub & 1;
          if (sub + 1 < T::NSUB) read_frags(0, sub + 1, buf ^ 1);
#pragma unroll
          for (int i = 0; i < T::FN; ++i)
#pragma unroll
            for (int j = 0; j < T::FM; ++j)
              acc[i][j] = mfma16<TIn>(xf[buf][i], yf[buf][j], (kFirst && sub == 0) ? zero4 : acc[i][j]);
        }
      };
      serial_tile(0, std::true_type{});
      for (int k = 1; k < KT; ++k) serial_tile(k, std::false_type{});
    } else {
      gload(0);
      lstore(0);
      wait_lgkmcnt0();
      barrier_sync();
      if (KT > 1) gload(1);
      read_frags(0, 0, 0);
      k_tile(0, 0, std::true_type{});
      for (int k = 1; k < KT; ++k) k_tile(k, k & 1, std::false_type{});
    }

    auto epilogue = [&](auto edge_c) {
      constexpr bool kEdge = decltype(edge_c)::value;
#pragma unroll
      for (int pu = 0; pu < T::FN / 2; ++pu) {
#pragma unroll
        for (int j = 0; j < T::FM; ++j) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[2 * pu][j][e];
            v[4 + e] = acc[2 * pu + 1][j][e];
          }
          store8<OUT, kEdge>(v, rc, wm * T::TM + 16 * j + (lane & 15), rows_left,
                             col0 + wn * T::TN + 32 * pu + 8 * (lane >> 4), N, args.ldc);
        }
      }
    };
    if (full_tile) epilogue(std::false_type{});
    else epilogue(std::true_type{});
  }
}

template <int BM, int BN, int BK, int S, int WM, int WN>
static KernelEntry make_reg_entry() {
  using T = TileShape<BM, BN, BK, S, WM, WN>;
  KernelEntry e;
  e.bm = BM; e.bn = BN; e.bk = BK; e.stages = S; e.waves = T::W; e.load_path = 2;
  e.lds_bytes = T::LDS;
  e.mfma = 16;
  e.fn[0][0] = (const void*)&gemm_reg_kernel<BM, BN, BK, S, WM, WN, _Float16, 0>;
  e.fn[0][1] = (const void*)&gemm_reg_kernel<BM, BN, BK, S, WM, WN, _Float16, 1>;
  e.fn[0][2] = (const void*)&gemm_reg_kernel<BM, BN, BK, S, WM, WN, _Float16, 2>;
  e.fn[1][0] = (const void*)&gemm_reg_kernel<BM, BN, BK, S, WM, WN, __bf16, 0>;
  e.fn[1][1] = (const void*)&gemm_reg_kernel<BM, BN, BK, S, WM, WN, __bf16, 1>;
  e.fn[1][2] = (const void*)&gemm_reg_kernel<BM, BN, BK, S, WM, WN, __bf16, 2>;
  return e;
}

const KernelEntry* reg_kernel_table(int* count) {
  static const KernelEntry table[] = {
      make_reg_entry<128, 128, 64, 2, 2, 2>(),
      make_reg_entry<64, 64, 64, 2, 2, 2>(),
      make_reg_entry<128, 128, 64, 1, 2, 2>(),  // the serial rung of the stage-count ablation
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace spt
