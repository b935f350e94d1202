// Software-pipelined, persistent, tiled GEMM  C = A·Bᵀ  for gfx950 (MI355X).
//
// Method: "GEMM II — pipelining with TMA" (Steps 4–6 and the TMA-store epilogue) and
// "Multi-Stage Software Pipelining" (Prefill, Main loop): operand tiles stream through a ring
// of S LDS stages that is kept S-1 tiles ahead of the math, and a persistent pool of
// workgroups walks a grouped tile raster. The gfx950 realisation differs from the pages'
// Hopper/Blackwell one:
//   * loads: direct global->LDS buffer loads (buffer_load_dwordx4 ... lds), 64 lanes x 16 B per
//     instruction, issued by every wave for its share of the tile (there is no single-issuer
//     copy engine). The XOR swizzle is applied on the source side: lane l of an instruction
//     lands at LDS byte 16*l, so it fetches the global chunk that belongs there.
//   * "full": each wave waits for its own loads with s_waitcnt vmcnt(n) and then s_barrier
//     publishes every wave's part (a barrier alone does not wait for in-flight loads, just as
//     a thread barrier cannot see a TMA transfer). "free": each wave drains its ds_reads of a
//     slot (lgkmcnt(0)) before that same barrier, and only then is the slot refilled. One
//     barrier per K-tile. The steady-state vmcnt threshold is an immediate; the ring slot only
//     moves the LDS base address (one scalar add), so the loop is not unrolled by S.
//   * compute: v_mfma_f32_16x16x32_{bf16,f16} with fp32 accumulators in registers; operands are
//     swapped (the B tile feeds the MFMA's row operand) so each lane holds output columns.
//   * epilogue: fp32 -> output type (round to nearest even), 16-byte stores of 8 consecutive
//     columns per lane straight from registers; M/N tails masked per element.
#include "spt_device.h"
#include "spt_kernels.h"

namespace spt {

template <int BM, int BN, int BK, int S, int WM, int WN, typename TIn, int OUT>
__global__ void __launch_bounds__(WM* WN * 64, 1) gemm_dma_kernel(GemmArgs args) {
  using T = TileShape<BM, BN, BK, S, WM, WN>;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int M = args.M, N = args.N, K = args.K;
  const int KT = (K + BK - 1) / BK;

  // DMA address map. A instruction j of this wave fills LDS bytes [(wave*LA + j) * 1024, +1024)
  // of the stage's A region: rows rho = 8*rb + lane/8 of 64-wide group g; the lane's physical
  // chunk lane%8 must hold logical chunk c = (lane%8) XOR swz(rho), so it fetches that chunk.
  auto a_map = [&](int j, int& row, int& kc) {
    const int q = wave * T::LA + j, g = q / (BM / 8), rb = q % (BM / 8);
    const int rho = 8 * rb + (lane >> 3);
    row = rho;
    kc = 8 * (8 * g + ((lane & 7) ^ swz(rho)));
  };
  auto b_map = [&](int j, int& row, int& kc) {
    const int q = wave * T::LB + j, g = q / (BN / 8), rb = q % (BN / 8);
    const int rho = 8 * rb + (lane >> 3);
    row = b_row_perm(rho);
    kc = 8 * (8 * g + ((lane & 7) ^ swz(rho)));
  };
  // fragment read offsets for k-step `sub` at f = 0 (fragment f adds 16 rows = 2048 bytes)
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

    // byte offset of each lane's chunk at k = 0, or kOOB for rows past the matrix edge
    unsigned a_off[T::LA], b_off[T::LB];
#pragma unroll
    for (int j = 0; j < T::LA; ++j) {
      int row, kc;
      a_map(j, row, kc);
      a_off[j] = row < rows_left ? (unsigned)(row * args.lda + kc) * 2u : kOOB;
    }
#pragma unroll
    for (int j = 0; j < T::LB; ++j) {
      int row, kc;
      b_map(j, row, kc);
      b_off[j] = row < cols_left ? (unsigned)(row * args.ldb + kc) * 2u : kOOB;
    }

    // issue this wave's share of K-tile kt into ring slot `slot`
    auto issue = [&](int slot, int kt) {
      const int k0 = kt * BK;
      char* sa = smem + slot * T::STAGE + wave * T::LA * 1024;
      char* sb = smem + slot * T::STAGE + T::A_BYTES + wave * T::LB * 1024;
      if (full_tile && k0 + BK <= K) {  // interior: every chunk valid, the k offset rides in soffset
#pragma unroll
        for (int j = 0; j < T::LA; ++j)
          dma16(ra, sa + j * 1024, a_off[j], 2u * k0);
#pragma unroll
        for (int j = 0; j < T::LB; ++j)
          dma16(rb, sb + j * 1024, b_off[j], 2u * k0);
      } else {  // edge tile or K tail: chunks past K or past the last row read zeros
#pragma unroll
        for (int j = 0; j < T::LA; ++j) {
          int row, kc;
          a_map(j, row, kc);
          const unsigned vo = (k0 + kc < K && a_off[j] != kOOB) ? a_off[j] + 2u * k0 : kOOB;
          dma16(ra, sa + j * 1024, vo, 0u);
        }
#pragma unroll
        for (int j = 0; j < T::LB; ++j) {
          int row, kc;
          b_map(j, row, kc);
          const unsigned vo = (k0 + kc < K && b_off[j] != kOOB) ? b_off[j] + 2u * k0 : kOOB;
          dma16(rb, sb + j * 1024, vo, 0u);
        }
      }
    };

    u32x4 xf[2][T::FN], yf[2][T::FM];  // fragment double buffer: B side (x), A side (y)
    auto read_frags = [&](int slot, int sub, int buf) {
      const char* base = smem + slot * T::STAGE;
#pragma unroll
      for (int f = 0; f < T::FN; ++f) xf[buf][f] = *(const u32x4*)(base + b_rd[sub] + f * 2048);
#pragma unroll
      for (int f = 0; f < T::FM; ++f) yf[buf][f] = *(const u32x4*)(base + a_rd[sub] + f * 2048);
    };

    // Accumulators. The first K-tile is peeled: its first MFMA of every chain takes a zero
    // accumulator (the analogue of accum = (k != 0)), so each accumulator's first value is a
    // distinct MFMA result rather than one shared zero register.
    f32x4 acc[T::FN][T::FM];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // one K-tile: k-steps 0 .. NSUB-1 of `slot`; the last k-step hands over to tile k+1
    auto k_tile = [&](int k, int slot, auto first_tile_c) {
      constexpr bool kFirst = decltype(first_tile_c)::value;
      const int next_slot = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub) {
        const int buf = sub & 1;
        if (sub + 1 < T::NSUB) {
          read_frags(slot, sub + 1, buf ^ 1);
        } else if (k + 1 < KT) {
          wait_lgkmcnt0();  // this wave's reads of `slot` are done
          if constexpr (S == 1) {
            // serial: the only slot is refilled once everyone has read it, then waited on
            barrier_sync();
            issue(0, k + 1);
            wait_vmcnt<0>();
          } else {
            // tiles issued so far: 0 .. min(k+S-1, KT-1); tile k+1 must have landed
            const int ahead = (k + S - 1 < KT - 1 ? k + S - 1 : KT - 1) - (k + 1);
            if (ahead >= S - 2) wait_vmcnt<T::LW * (S - 2)>();
            else wait_vmcnt_tiles<T::LW, (S > 2 ? S - 3 : 0)>(ahead);
          }
          barrier_sync();  // tile k+1 visible to all waves; `slot` free in all waves
          if constexpr (S > 1)
            if (k + S < KT) issue(slot, k + S);
          read_frags(next_slot, 0, buf ^ 1);
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

    if (KT == 0) {  // empty sum: C = 0
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int pu = 0; pu < T::FN / 2; ++pu)
        for (int j = 0; j < T::FM; ++j)
          store8<OUT, true>(z, rc, wm * T::TM + 16 * j + (lane & 15), rows_left,
                            col0 + wn * T::TN + 32 * pu + 8 * (lane >> 4), N, args.ldc);
      continue;
    }

    // the previous tile's fragment reads must be finished everywhere before its slots are refilled
    if (!first_tile) {
      wait_lgkmcnt0();
      barrier_sync();
    }
    first_tile = false;
    // ---- prologue: fill the ring with tiles 0 .. min(S, KT) - 1 ----
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < KT) issue(s, s);
    wait_vmcnt_tiles<T::LW, S - 1>((KT < S ? KT : S) - 1);  // this wave's part of tile 0 landed
    barrier_sync();                                          // ... and every wave's
    read_frags(0, 0, 0);

    // ---- steady state and drain: one barrier per K-tile ----
    k_tile(0, 0, std::true_type{});
    int slot = S > 1 ? 1 : 0;
    for (int k = 1; k < KT; ++k) {
      k_tile(k, slot, std::false_type{});
      slot = slot + 1 == S ? 0 : slot + 1;
    }

    // ---- epilogue: fp32 -> output type, 8 consecutive columns per lane ----
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
          const int m_rel = wm * T::TM + 16 * j + (lane & 15);
          const int n = col0 + wn * T::TN + 32 * pu + 8 * (lane >> 4);
          store8<OUT, kEdge>(v, rc, m_rel, rows_left, n, N, args.ldc);
        }
      }
    };
    if (full_tile) epilogue(std::false_type{});
    else epilogue(std::true_type{});
  }
}

// ------------------------------------------------------------------------------ instantiation table
template <int BM, int BN, int BK, int S, int WM, int WN>
static KernelEntry make_entry() {
  using T = TileShape<BM, BN, BK, S, WM, WN>;
  KernelEntry e;
  e.bm = BM; e.bn = BN; e.bk = BK; e.stages = S; e.waves = T::W; e.load_path = 1;
  e.lds_bytes = T::LDS;
  e.fn[0][0] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, _Float16, 0>;
  e.fn[0][1] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, _Float16, 1>;
  e.fn[0][2] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, _Float16, 2>;
  e.fn[1][0] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, __bf16, 0>;
  e.fn[1][1] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, __bf16, 1>;
  e.fn[1][2] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, __bf16, 2>;
  return e;
}

const KernelEntry* dma_kernel_table(int* count) {
  static const KernelEntry table[] = {
      make_entry<256, 256, 64, 2, 2, 2>(),
      make_entry<256, 256, 64, 1, 2, 2>(),
      make_entry<256, 128, 64, 3, 2, 2>(),
      make_entry<256, 128, 64, 2, 2, 2>(),
      make_entry<256, 128, 64, 1, 2, 2>(),
      make_entry<128, 128, 64, 4, 2, 2>(),
      make_entry<128, 128, 64, 3, 2, 2>(),
      make_entry<128, 128, 64, 2, 2, 2>(),
      make_entry<128, 128, 64, 1, 2, 2>(),
      make_entry<64, 64, 64, 4, 2, 2>(),
      make_entry<64, 64, 64, 2, 2, 2>(),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace spt
