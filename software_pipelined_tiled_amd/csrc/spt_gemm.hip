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
//     lands at LDS byte 16*l, so it fetches the global chunk that belongs there. STREAM = 1 or 2
//     loads A or B with the non-temporal hint (skinny shapes, where one workgroup reads each
//     tile of that operand once).
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

struct Regions {
  int a, b;  // LDS byte offsets of a K-tile's A and B tiles
};

template <int BM, int BN, int BK, int S, int WM, int WN, typename TIn, int OUT, int STREAM>
__global__ void __launch_bounds__(WM* WN * 64, 1) gemm_dma_kernel(GemmArgs args) {
  using T = TileShape<BM, BN, BK, S, WM, WN>;
  // 16 bytes past the ring hold the dynamic schedule's next unit, where the ring leaves room for them
  // (the host enables the queue only for those configurations)
  constexpr int kQueueSlot = T::LDS + 16 <= 160 * 1024 ? 16 : 0;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS + kQueueSlot];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int M = args.M, N = args.N, K = args.K;
  const int KT = args.kt_per;  // K-tiles per work unit (all of K unless K is split)

  // DMA address map. A instruction j of this wave fills LDS bytes [(wave*LA + j) * 1024, +1024)
  // of the stage's A region: rows rho = RPI*rb + lane/CPR of row group g (RPI = 8 rows of 128
  // bytes, or 16 rows of 64 bytes for a 32-deep K-tile); the lane's physical chunk lane%CPR must
  // hold logical chunk (lane%CPR) XOR swizzle(rho). The swizzle has period RPI in the row, so it
  // depends on lane/CPR alone and the chunk depends on the lane alone; the group g is
  // wave-uniform. Element offset of the lane's chunk inside the K-tile: GK*g + lane_kc.
  const int lane_kc = T::RB == 128 ? 8 * ((lane & 7) ^ swz(lane >> 3)) : 8 * ((lane & 3) ^ swz64(lane >> 2));
  auto a_map = [&](int j, int& row, int& g) {
    const int q = wave * T::LA + j, rb = q % (BM / T::RPI);
    g = q / (BM / T::RPI);
    row = T::RPI * rb + lane / T::CPR;
  };
  auto b_map = [&](int j, int& row, int& g) {
    const int q = wave * T::LB + j, rb = q % (BN / T::RPI);
    g = q / (BN / T::RPI);
    row = b_row_perm(T::RPI * rb + lane / T::CPR);
  };
  // fragment read offsets for k-step `sub` at f = 0 (fragment f adds 16 rows = FRAG bytes)
  int a_rd[T::NSUB], b_rd[T::NSUB];
#pragma unroll
  for (int s = 0; s < T::NSUB; ++s) {
    a_rd[s] = lds_chunk_offset(BM, wm * T::TM + (lane & 15), 4 * s + (lane >> 4), BK);
    b_rd[s] = lds_chunk_offset(BN, wn * T::TN + (lane & 15), 4 * s + (lane >> 4), BK);
  }

  // Ring positions. Plain ring: position = stage, the A tile at its start and the B tile after it.
  // Split ring: position = the A tile's slot; the B tile is in the next slot, and the next K-tile
  // starts two slots on.
  auto regions = [&](int pos) {
    if constexpr (T::SPLIT) return Regions{pos * T::SLOT, (pos + 1 == S ? 0 : pos + 1) * T::SLOT};
    else return Regions{pos * T::STAGE, pos * T::STAGE + T::A_BYTES};
  };
  auto pos_next = [&](int pos) {
    if constexpr (T::SPLIT) return pos + 2 >= S ? pos + 2 - S : pos + 2;
    else return pos + 1 == S ? 0 : pos + 1;
  };
  auto pos_prev = [&](int pos) {
    if constexpr (T::SPLIT) return pos < 2 ? pos + S - 2 : pos - 2;
    else return pos == 0 ? S - 1 : pos - 1;
  };

  const int u = xcd_remap(blockIdx.x, args.grid);
  bool first_tile = true;
  // The next work unit: the static schedule's next round, or, with a queue, the next unit nobody has
  // taken yet (every workgroup's first unit is its static one). One lane takes it with an atomic
  // add and hands it to the other waves through LDS; the second barrier keeps the slot from being
  // overwritten before every wave has read it. Each unit is handed out once, so every workgroup
  // ends its loop after at most num_tiles takes.
  auto next = [&](int t) {
    if constexpr (kQueueSlot == 0) {
      return t + args.grid;
    } else {
      if (args.queue == nullptr) return t + args.grid;
      int* const slot = (int*)(smem + T::LDS);
      if (threadIdx.x == 0) *slot = args.grid + atomicAdd(&args.queue[0], 1);
      wait_lgkmcnt0();  // the slot write has reached LDS before any wave passes the barrier
      barrier_sync();
      const int n = *slot;
      wait_lgkmcnt0();  // every wave's read of the slot is done before the next take may overwrite it
      barrier_sync();
      return n;
    }
  };
  for (int t = u; t < args.num_tiles; t = next(t)) {
    int tm, tn, ks;
    unit_decode(t, args.tiles_m, args.tiles_n, args.group_m, tm, tn, ks);
    const int row0 = tm * BM, col0 = tn * BN;
    const int kbase = ks * KT * BK;  // first K element of this unit's range
    const int rows_left = M - row0, cols_left = N - col0;
    const bool full_tile = rows_left >= BM && cols_left >= BN;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc((const char*)args.A + (size_t)row0 * args.lda * 2, ((uint64_t)(rows_left - 1) * args.lda + K) * 2);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc((const char*)args.B + (size_t)col0 * args.ldb * 2, ((uint64_t)(cols_left - 1) * args.ldb + K) * 2);

    // byte offset of each lane's chunk at k = 0; rows past the matrix edge get an offset beyond
    // num_records (it stays beyond it after adding 2*k0 < 2^31), so they read zeros
    unsigned a_off[T::LA], b_off[T::LB];
#pragma unroll
    for (int j = 0; j < T::LA; ++j) {
      int row, g;
      a_map(j, row, g);
      a_off[j] = row < rows_left ? (unsigned)(row * args.lda + T::GK * g + lane_kc) * 2u : kOOB;
    }
#pragma unroll
    for (int j = 0; j < T::LB; ++j) {
      int row, g;
      b_map(j, row, g);
      b_off[j] = row < cols_left ? (unsigned)(row * args.ldb + T::GK * g + lane_kc) * 2u : kOOB;
    }

    // DMA instruction d (0 .. LW-1: A loads first, then B) of this wave's share of K-tile kt of
    // the unit's range (absolute K offset k0 = kbase + kt*BK). The K offset rides in the scalar soffset; the per-lane voffset is a
    // constant, replaced by one past num_records (reads zero) when the lane's chunk lies at or past
    // K (lane_kc >= K - k0 - GK*g: one compare per group and K-tile). K-tiles past the end are
    // therefore zero-filling dummies, and every hand-over issues exactly LW loads per wave, which
    // keeps every vmcnt threshold constant. (kOOB + soffset stays past num_records: soffset < 2^31.)
    // `dst` gives the LDS byte offsets of the A and B tiles' destinations.
    auto dma_one = [&](Regions dst, int kt, int d) {
      const int k0 = kt * BK + kbase;
      if (d < T::LA) {
        const int g = (wave * T::LA + d) / (BM / T::RPI);
        char* sa = smem + dst.a + (wave * T::LA + d) * 1024;
        if constexpr (STREAM == 1) dma16_stream(ra, sa, lane_kc < K - k0 - T::GK * g ? a_off[d] : kOOB, 2u * k0);
        else dma16(ra, sa, lane_kc < K - k0 - T::GK * g ? a_off[d] : kOOB, 2u * k0);
      } else {
        const int j = d - T::LA;
        const int g = (wave * T::LB + j) / (BN / T::RPI);
        char* sb = smem + dst.b + (wave * T::LB + j) * 1024;
        if constexpr (STREAM == 2) dma16_stream(rb, sb, lane_kc < K - k0 - T::GK * g ? b_off[j] : kOOB, 2u * k0);
        else dma16(rb, sb, lane_kc < K - k0 - T::GK * g ? b_off[j] : kOOB, 2u * k0);
      }
    };
    auto issue = [&](Regions dst, int kt) {
#pragma unroll
      for (int d = 0; d < T::LW; ++d) dma_one(dst, kt, d);
    };

    u32x4 xf[2][T::FN], yf[2][T::FM];  // fragment double buffer: B side (x), A side (y)
    // fragment r of k-step `sub` (r < FN: B side, else A side) into buffer `buf`
    auto read_frag = [&](Regions src, int sub, int buf, int r) {
      if (r < T::FN) xf[buf][r] = *(const u32x4*)(smem + src.b + b_rd[sub] + r * T::FRAG);
      else yf[buf][r - T::FN] = *(const u32x4*)(smem + src.a + a_rd[sub] + (r - T::FN) * T::FRAG);
    };
    auto read_frags = [&](Regions src, int sub, int buf) {
#pragma unroll
      for (int f = 0; f < T::FN; ++f) xf[buf][f] = *(const u32x4*)(smem + src.b + b_rd[sub] + f * T::FRAG);
#pragma unroll
      for (int f = 0; f < T::FM; ++f) yf[buf][f] = *(const u32x4*)(smem + src.a + a_rd[sub] + f * T::FRAG);
    };

    // Accumulators. The first K-tile is peeled: its first MFMA of every chain takes a zero
    // accumulator (the analogue of accum = (k != 0)), so each accumulator's first value is a
    // distinct MFMA result rather than one shared zero register.
    f32x4 acc[T::FN][T::FM];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // One k-step: the FN x FM MFMAs on fragment buffer `buf`, with NR fragment reads (for the next
    // k-step) and ND DMA loads (for a later K-tile) threaded between them, each kind spread
    // evenly over the MFMA slots. The order is pinned (sched_barrier) so the loads drain through the
    // vector-memory and LDS pipes while the MFMA pipe stays busy, instead of arriving in a burst.
    constexpr int NM = T::FN * T::FM;
    auto kstep = [&](int buf, auto zero_c, auto nr_c, auto nd_c, auto&& rd, auto&& dm) {
      constexpr bool kZero = decltype(zero_c)::value;
      constexpr int NR = decltype(nr_c)::value, ND = decltype(nd_c)::value;
      static_for<NM>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        constexpr int i = m / T::FM, j = m % T::FM;
        acc[i][j] = mfma16<TIn>(xf[buf][i], yf[buf][j], kZero ? zero4 : acc[i][j]);
        // load slots: the reads, and separately the DMAs, are spread evenly over the MFMA slots. With
        // more of them than MFMAs (the small skinny tiles) slot m takes reads [m*NR/NM, (m+1)*NR/NM)
        if constexpr (NR > 0 && NR <= NM) {
          constexpr int sr = NM / NR;
          if constexpr (m % sr == 0 && m / sr < NR) rd(m / sr);
        } else if constexpr (NR > NM) {
          static_for<NR>([&](auto r_c) {
            if constexpr (decltype(r_c)::value * NM / NR == m) rd(decltype(r_c)::value);
          });
        }
        if constexpr (ND > 0 && ND <= NM) {
          constexpr int sd = NM / ND;
          if constexpr (m % sd == sd / 2 && m / sd < ND) dm(m / sd);
        } else if constexpr (ND > NM) {
          static_for<ND>([&](auto d_c) {
            if constexpr (decltype(d_c)::value * NM / ND == m) dm(decltype(d_c)::value);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto no_load = [](int) {};

    // One K-tile: k-steps 0 .. NSUB-1 of the tile at ring position `pos`. Before the last k-step of
    // every tile but the last (kHandover, a compile-time flag so that the K-loop body is one
    // straight-line block whose accumulators never meet at a join): wait for tile k+1, sync, then,
    // threaded through the MFMAs, read tile k+1's first fragments and refill the freed slots.
    // Plain ring: tile k+S goes into tile k's stage. With two stages, or one k-step per K-tile,
    // the whole refill goes into the hand-over k-step (LW1 = LW). Otherwise it is split in half so
    // the loads spread over a whole K-tile: the first half in the hand-over k-step, the second in
    // k-step 0 of the next tile (kDefer). The stage stays free from this hand-over's barrier to the
    // next one, and by the next hand-over every load of tile k+S has been issued, so the vmcnt
    // thresholds are unchanged.
    // Split ring: tile k's two slots free up at its hand-over; the hand-over k-step loads tile
    // k+2's B tile into tile k's A slot, and k-step 0 of tile k+1 loads tile k+3's A tile into tile
    // k's B slot. Every k-step then issues one operand tile's loads. At a hand-over, tile k+1 must
    // have landed and only tile k+2's A tile may still be in flight: vmcnt(LA).
    // kFirst: the first tile, whose MFMA chains start from zero. b0_c: the fragment buffer the
    // tile's k-step 0 uses (the k-step parity; it alternates per tile when a tile is one k-step).
    constexpr int LW1 = T::P.refill_now;
    constexpr int LWD = T::P.refill_later;  // deferred loads, in k-step 0 of the next tile
    auto k_tile = [&](int k, int pos, auto first_c, auto handover_c, auto b0_c) {
      constexpr bool kFirst = decltype(first_c)::value;
      constexpr bool kHandover = decltype(handover_c)::value;
      constexpr bool kDefer = !kFirst && (T::SPLIT || S > 2) && T::NSUB > 1;
      const Regions cur = regions(pos), nxt = regions(pos_next(pos)), prv = regions(pos_prev(pos));
      static_for<T::NSUB>([&](auto sub_c) {
        constexpr int sub = decltype(sub_c)::value;
        constexpr int buf = (decltype(b0_c)::value + sub) & 1;
        auto zero_c = std::integral_constant<bool, kFirst && (sub == 0)>{};
        auto nr_c = std::integral_constant<int, T::FN + T::FM>{};
        // second half of the refill started at the previous hand-over
        auto nd_def = std::integral_constant<int, (kDefer && sub == 0) ? LWD : 0>{};
        auto dm_def = [&](int d) {
          if constexpr (T::SPLIT) dma_one(Regions{prv.b, prv.b}, k + 2, d);  // A of tile (k-1)+3
          else dma_one(prv, k - 1 + S, LW1 + d);
        };
        if constexpr (sub + 1 < T::NSUB) {
          kstep(buf, zero_c, nr_c, nd_def, [&](int r) { read_frag(cur, sub + 1, buf ^ 1, r); }, dm_def);
        } else if constexpr (kHandover) {
          wait_lgkmcnt0();  // this wave's reads of tile k are done
          if constexpr (S == 1) {
            // serial: the only slot is refilled once everyone has read it, then waited on
            barrier_sync();
            issue(cur, k + 1);
            wait_vmcnt<0>();
            barrier_sync();
            kstep(buf, zero_c, nr_c, std::integral_constant<int, 0>{},
                  [&](int r) { read_frag(cur, 0, buf ^ 1, r); }, no_load);
          } else {
            // plain ring: every hand-over issued LW loads, so exactly tiles k+2 .. k+S-1 may still be
            // in flight; split ring: tile k+2's A tile
            wait_vmcnt<T::P.handover_wait>();
            barrier_sync();  // tile k+1 visible to all waves; tile k's slots free in all waves
            static_assert(T::NSUB >= 2 || LW1 == T::LW, "the deferred half needs a k-step before the hand-over");
            kstep(buf, zero_c, nr_c, std::integral_constant<int, LW1>{},
                  [&](int r) { read_frag(nxt, 0, buf ^ 1, r); },
                  [&](int d) {
                    if constexpr (T::SPLIT) dma_one(Regions{cur.a, cur.a}, k + 2, T::LA + d);  // B of tile k+2
                    else dma_one(cur, k + S, d);
                  });
          }
        } else {
          kstep(buf, zero_c, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, no_load, no_load);
        }
      });
    };

    const int es = OUT == 2 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((char*)args.C + (size_t)ks * args.split_stride + (size_t)row0 * args.ldc * es,
                                                ((uint64_t)(rows_left - 1) * args.ldc + N) * es);

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
    // ---- prologue: fill the ring (tiles past K are zero-filling dummies) ----
    if constexpr (T::SPLIT) {
      // A0, B0, A1, B1, A2 into slots 0 .. 4
#pragma unroll
      for (int h = 0; h < S; ++h)
#pragma unroll
        for (int d = 0; d < (h % 2 ? T::LB : T::LA); ++d)
          dma_one(Regions{h * T::SLOT, h * T::SLOT}, h / 2, (h % 2 ? T::LA : 0) + d);
      wait_vmcnt<T::P.prologue_wait>();  // this wave's part of tile 0 landed
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) issue(regions(s), s);
      wait_vmcnt<T::P.prologue_wait>();  // this wave's part of tile 0 landed
    }
    barrier_sync();  // ... and every wave's
    read_frags(regions(0), 0, 0);

    // ---- steady state and drain: one barrier per K-tile; the last K-tile is peeled ----
    using t_ = std::true_type;
    using f_ = std::false_type;
    using b0_ = std::integral_constant<int, 0>;
    using b1_ = std::integral_constant<int, 1>;
    if (KT == 1) {
      k_tile(0, 0, t_{}, f_{}, b0_{});
    } else {
      k_tile(0, 0, t_{}, t_{}, b0_{});
      int slot = pos_next(0);
      auto advance = [&]() { slot = pos_next(slot); };
      if constexpr (T::NSUB % 2 == 0) {
        for (int k = 1; k < KT - 1; ++k) {
          k_tile(k, slot, f_{}, t_{}, b0_{});
          advance();
        }
        k_tile(KT - 1, slot, f_{}, f_{}, b0_{});
      } else {
        // one k-step per K-tile: tile k uses fragment buffer k mod 2, so tiles go in pairs
        int k = 1;
        for (; k + 1 < KT - 1; k += 2) {
          k_tile(k, slot, f_{}, t_{}, b1_{});
          advance();
          k_tile(k + 1, slot, f_{}, t_{}, b0_{});
          advance();
        }
        if (k < KT - 1) {
          k_tile(k, slot, f_{}, t_{}, b1_{});
          advance();
          ++k;
        }
        if (k & 1) k_tile(k, slot, f_{}, f_{}, b1_{});
        else k_tile(k, slot, f_{}, f_{}, b0_{});
      }
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
          __builtin_amdgcn_sched_barrier(0);  // one 8-value chunk of accumulators live at a time
        }
      }
    };
    if (full_tile) epilogue(std::false_type{});
    else epilogue(std::true_type{});
  }
  if (kQueueSlot != 0 && args.queue != nullptr && threadIdx.x == 0) {
    // this workgroup takes no more units; the last one to get here resets the queue for the next launch
    if (atomicAdd(&args.queue[1], 1) == args.grid - 1) {
      atomicExch(&args.queue[0], 0);
      atomicExch(&args.queue[1], 0);
    }
  }
}

// ------------------------------------------------------------------------------ instantiation table
template <int BM, int BN, int BK, int S, int WM, int WN, int STREAM>
static void fill_fns(const void* (&fn)[2][3]) {
  fn[0][0] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, _Float16, 0, STREAM>;
  fn[0][1] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, _Float16, 1, STREAM>;
  fn[0][2] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, _Float16, 2, STREAM>;
  fn[1][0] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, __bf16, 0, STREAM>;
  fn[1][1] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, __bf16, 1, STREAM>;
  fn[1][2] = (const void*)&gemm_dma_kernel<BM, BN, BK, S, WM, WN, __bf16, 2, STREAM>;
}

// HINTS: also instantiate the variants that load A (fn_stream[0]) or B (fn_stream[1]) with the
// non-temporal hint
template <int BM, int BN, int BK, int S, int WM, int WN, bool HINTS = false>
static KernelEntry make_entry() {
  using T = TileShape<BM, BN, BK, S, WM, WN>;
  KernelEntry e;
  e.bm = BM; e.bn = BN; e.bk = BK; e.stages = S; e.waves = T::W; e.load_path = 1;
  e.lds_bytes = T::LDS;
  e.mfma = 16;
  fill_fns<BM, BN, BK, S, WM, WN, 0>(e.fn);
  if constexpr (HINTS) {
    fill_fns<BM, BN, BK, S, WM, WN, 1>(e.fn_stream[0]);
    fill_fns<BM, BN, BK, S, WM, WN, 2>(e.fn_stream[1]);
  }
  return e;
}

const KernelEntry* dma_kernel_table(int* count) {
  static const KernelEntry table[] = {
      make_entry<256, 256, 64, 2, 2, 2>(),
      make_entry<256, 256, 64, 5, 2, 2>(),
      make_entry<256, 256, 32, 4, 2, 2>(),
      make_entry<256, 256, 64, 1, 2, 2>(),
      make_entry<256, 128, 64, 3, 2, 2>(),
      make_entry<256, 128, 64, 2, 2, 2>(),
      make_entry<256, 128, 64, 1, 2, 2>(),
      make_entry<128, 128, 64, 4, 2, 2>(),
      make_entry<128, 128, 64, 3, 2, 2>(),
      make_entry<128, 128, 64, 2, 2, 2>(),
      make_entry<128, 128, 64, 1, 2, 2>(),
      make_entry<64, 64, 64, 4, 2, 2>(),
      make_entry<64, 64, 128, 4, 2, 2>(),
      make_entry<64, 64, 64, 2, 2, 2>(),
      // skinny shapes (M of a few dozen rows): a 32x32 tile with 128-deep K-tiles and two waves keeps
      // one workgroup per 32 columns streaming, with up to seven 8 KiB operand tiles of B in flight;
      // the operand only one workgroup reads can be streamed with the non-temporal hint
      make_entry<32, 32, 128, 4, 2, 1, true>(),
      make_entry<32, 32, 128, 8, 2, 1, true>(),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace spt
