// Software-pipelined, persistent, tiled GEMM  C = A·Bᵀ  for gfx950: the two-wave-group
// ("ping-pong") form of the mainloop.
//
// The method is the one of spt_gemm.hip ("GEMM II — pipelining with TMA", Steps 4–6; "Multi-Stage
// Software Pipelining", Prefill / Main loop): a ring of LDS stages filled ahead of the math by
// direct global->LDS loads, a persistent pool of workgroups over a grouped raster. What changes
// is who issues what, which is the step "Multi-Stage Software Pipelining" (What's Next) names
// after the multi-stage ring: separate the loading role from the computing role.
//
// On gfx950 a wave issues at most one instruction per issue cycle, so with one wave per SIMD
// every load and LDS read takes an issue slot from the MFMA stream. Here a workgroup has eight
// waves, two per SIMD, in two groups of four (G0 = waves 0-3, G1 = waves 4-7; wave w runs on SIMD
// w mod 4, so each SIMD holds one wave of each group). Time is cut into phases separated by
// workgroup barriers; in every phase one group runs a block of MFMAs (a compute phase) while the
// other group issues its LDS fragment reads and, for G0, the DMA loads of the next K-tile (a
// memory phase). The two groups are one phase apart, so each SIMD's matrix core is fed by one
// wave while its partner's memory instructions issue beside it.
//
// Tile 256x256, K-tile 64. G0 computes output rows [0, 128) of the tile and G1 rows [128, 256);
// inside a group the four waves form a 2x2 grid of 64x128 wave tiles (128 fp32 accumulators per
// lane).
//
// The phases run on without a break from one work unit (an output tile, or one K range of it when
// K is split) to the next: number the K-tiles a workgroup computes g = 0, 1, ..., G-1 across all
// its units (KT per unit). K-tile g is read in phases 2g (G0) and 2g+1 (G1) and computed in phases
// 2g+1 (G0) and 2g+2 (G1). Loads run ahead into the next unit the same way they run ahead inside
// one, so there is no prologue per unit: the pages' overlap of the next tile's loads with the
// current math and the previous tile's stores, carried across tiles.
// A group stores a finished output tile in its next memory phase, with the next K-tile's fragment
// reads spread between the stores (16-bit outputs); after the last K-tile G0 stores in phase 2G,
// beside G1's last MFMAs, and G1 after the last barrier. Both groups pass 2G + 2 barriers.
//
// Ring, S = 2: two 64 KiB stages (stage g mod 2). In phase 2g G0 loads all of K-tile g+1 and waits
// for it at the end of phase 2g+1: loads are issued in bursts, every other phase.
// Ring, S = 5 (split): five 32 KiB operand slots; K-tile g's A tile sits in slot 2g mod 5 and its
// B tile in slot 2g+1 mod 5. Every memory phase issues one operand tile: G0 loads B(g+1) in phase
// 2g (into the slot A(g-1) left) and waits for it at the end of phase 2g+1; G1 loads A(g+2) in
// phase 2g+1 (into the slot B(g-1) left) and waits for it two phases later, with A(g+3) possibly
// still in flight. The kernel starts by loading A(0), B(0) and A(1). Each load has two (B) or three
// (A) phases to land, and the CU's fill path is busy in every phase.
//
// Inside a memory phase the eight loads are spread between the 24 fragment reads (one load, then
// three reads). A CU stages about 150 bytes of L2-resident data per ns through direct
// global->LDS loads; with the four waves of a group issuing, each gets a 1 KiB load through
// about every 28 ns, so eight loads hold a wave for some 350 cycles. Issued as one burst they
// held the reads behind them and the memory phase outlasted the 64 MFMAs of the other group.
// Interleaved, the LDS serves the reads while the loads issue.
//
// Epilogue: with the A fragment as the MFMA's first operand and B staged in the b_row_perm128
// order, a lane holds 8 consecutive output columns of 4 rows, and each store instruction writes
// four rows of 256 bytes (a quarter-wave per row).
#include "spt_device.h"
#include "spt_kernels.h"

namespace spt {

// One work unit: an output tile of the raster and the K range it covers (t >= num_tiles: past the
// end of this workgroup's list).
struct PpTile {
  int t;
  int row0, col0, rows_left, cols_left;
  int ks, kb;  // K range index and its first K element
};

// MF: the MFMA shape, 16 (v_mfma_f32_16x16x32) or 32 (v_mfma_f32_32x32x16). A fragment is MF rows of
// the K-tile at the MFMA's depth (32 or 16 elements): 8 values per lane either way, one ds_read_b128.
template <int S, int MF, typename TIn, int OUT>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel(GemmArgs args) {
  constexpr int BM = 256, BN = 256, BK = 64;
  constexpr bool SPLIT = S == 5;
  constexpr int TM = 64, TN = 128;                   // wave tile
  constexpr int MK = MF == 16 ? 32 : 16;             // K depth of one MFMA
  constexpr int FM = TM / MF, FN = TN / MF;          // A and B fragments per k-step (4, 8 or 2, 4)
  constexpr int NSUB = BK / MK;                      // k-steps per K-tile (2 or 4)
  constexpr int FRAG = MF * 128;                     // bytes between fragments
  using Acc = std::conditional_t<MF == 16, f32x4, f32x16>;
  static_assert(MF == 16 || MF == 32, "16x16x32 or 32x32x16 MFMA");
  constexpr int A_BYTES = BM * BK * 2, STAGE = (BM + BN) * BK * 2;
  constexpr int LDS = SPLIT ? S * A_BYTES : S * STAGE;
  constexpr PipeProtocol P = pipe_protocol(BM, BN, BK, S, 8);
  constexpr int LA = P.la, LB = P.lb;                // DMA instructions per wave for one operand tile
  static_assert(LA == A_BYTES / 1024 / 4 && LB == LA, "one group of four waves loads an operand tile");
  static_assert(S == 2 || S == 5, "two 64 KiB stages or five 32 KiB operand slots");
  static_assert(LDS <= 160 * 1024, "LDS ring fits the 160 KiB of a CU");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  const unsigned smem_base = lds_addr(smem);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, v = wave & 3;
  const int wm = v >> 1, wn = v & 1;
  const int M = args.M, N = args.N, K = args.K;
  const int KT = args.kt_per;  // K-tiles per work unit
  const int es = OUT == 2 ? 4 : 2;
  const int m_base = 128 * grp + TM * wm;  // this wave's first output row inside a tile

  auto tile_at = [&](int t) SPT_INLINE {
    PpTile tl;
    tl.t = t;
    int tm = 0, tn = 0, ks = 0;
    if (t < args.num_tiles) unit_decode(t, args.tiles_m, args.tiles_n, args.group_m, tm, tn, ks);
    tl.ks = ks;
    tl.kb = ks * KT * BK;
    tl.row0 = tm * BM;
    tl.col0 = tn * BN;
    tl.rows_left = M - tl.row0;
    tl.cols_left = N - tl.col0;
    return tl;
  };
  auto c_rsrc = [&](const PpTile& tl) SPT_INLINE {
    return make_rsrc((char*)args.C + (size_t)tl.ks * args.split_stride + (size_t)tl.row0 * args.ldc * es,
                     ((uint64_t)(tl.rows_left - 1) * args.ldc + N) * es);
  };

  const int u0 = xcd_remap(blockIdx.x, args.grid);
  if (KT == 0) {  // empty sum: C = 0 (no barriers: every wave takes this branch)
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t = u0; t < args.num_tiles; t += args.grid) {
      const PpTile tl = tile_at(t);
      const __amdgpu_buffer_rsrc_t rc = c_rsrc(tl);
      for (int pu = 0; pu < TN / 32; ++pu)
        for (int j = 0; j < TM / 16; ++j)
          store8<OUT, true>(z, rc, m_base + 16 * j + (lane & 15), tl.rows_left,
                            tl.col0 + TN * wn + 32 * pu + 8 * (lane >> 4), N, args.ldc);
    }
    return;
  }

  // DMA. Wave v's instruction j of an operand tile fills LDS rows 8q .. 8q+7 (q = LA*v + j) of the
  // tile; lane l lands at row 8q + l/8, physical chunk l%8, which holds logical chunk (l%8) XOR
  // swz(l/8) (the swizzle has period 8 in the row, so it depends on the lane alone). The row
  // splits into a wave-uniform part 8q and a lane part l/8; B rows are staged permuted, and both
  // permutations split the same way (they permute within aligned 32-row groups, and rows 8q .. 8q+7
  // keep their offsets 8(r/4) + r%4 relative to the image of 8q).
  auto bperm = [](int rho) SPT_INLINE { return MF == 16 ? b_row_perm128(rho) : b_row_perm32(rho); };
  const int lrow = lane >> 3;
  const int lane_kc = 8 * ((lane & 7) ^ swz(lrow));
  const int a_lrow = lrow, b_lrow = bperm(lrow);
  auto a_urow = [&](int j) SPT_INLINE { return 8 * (LA * v + j); };
  auto b_urow = [&](int j) SPT_INLINE { return bperm(8 * (LB * v + j)); };
  // fragment read offsets inside an operand tile, k-step s (fragment f adds MF rows): lane l reads
  // row l mod MF, the 8-element chunk l / MF of the k-step's MK elements
  int a_rd[NSUB], b_rd[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    a_rd[s] = lds_chunk_offset(BM, 128 * grp + TM * wm + lane % MF, (MK / 8) * s + lane / MF);
    b_rd[s] = lds_chunk_offset(BN, TN * wn + lane % MF, (MK / 8) * s + lane / MF);
  }

  // A position in the K-tile stream: an output tile, a K-tile inside it, and the buffer descriptors
  // of the tile's A rows and B rows. advance() moves to the next K-tile, into the next output tile
  // after the last. All of it is wave-uniform and lives in scalar registers. The tile change is
  // kept a branch: if-converted, the raster decode (two divisions) and the 64-bit descriptor
  // arithmetic ran in every K-tile, and the scalar work a memory phase issues lengthens it (made
  // once per tile, 2 % faster on 8192^3).
  struct Cursor {
    PpTile tl;
    int u;
    __amdgpu_buffer_rsrc_t ra, rb;
  };
  auto set_rsrc = [&](Cursor& c) SPT_INLINE {
    c.ra = make_rsrc((const char*)args.A + (size_t)c.tl.row0 * args.lda * 2, ((uint64_t)(c.tl.rows_left - 1) * args.lda + K) * 2);
    c.rb = make_rsrc((const char*)args.B + (size_t)c.tl.col0 * args.ldb * 2, ((uint64_t)(c.tl.cols_left - 1) * args.ldb + K) * 2);
  };
  auto cursor_at = [&](int t) SPT_INLINE {
    Cursor c;
    c.tl = tile_at(t);
    c.u = 0;
    set_rsrc(c);
    return c;
  };
  auto advance = [&](Cursor& c) SPT_INLINE {
    if (__builtin_expect(++c.u == KT, 0)) {
      c.u = 0;
      c.tl = tile_at(c.tl.t + args.grid);
      set_rsrc(c);
    }
  };
  auto valid = [&](const Cursor& c) SPT_INLINE { return c.tl.t < args.num_tiles; };

  // This wave's share of the A (or B) tile of the cursor's K-tile into the LDS tile at byte offset
  // `dst`. The lane's offset is its row times ld plus its chunk; a row past the matrix edge then
  // lies at or beyond the descriptor's num_records and reads zero. A chunk at or past K is moved
  // beyond num_records explicitly (one select per call); the K offset rides in the scalar offset.
  // An operand tile's loads, prepared once (the cursor's descriptor, the K offset, the lane's
  // offset, the LDS base) and then issued one instruction at a time, so that a memory phase can
  // spread them between its fragment reads.
  struct OpLoads {
    __amdgpu_buffer_rsrc_t r;
    unsigned v0, lds;
    int k0, ld;
  };
  auto prep_a = [&](const Cursor& c, int dst) SPT_INLINE {
    OpLoads o;
    o.k0 = __builtin_amdgcn_readfirstlane(c.u) * BK + __builtin_amdgcn_readfirstlane(c.tl.kb);
    o.r = c.ra;
    o.v0 = lane_kc < K - o.k0 ? (unsigned)(a_lrow * args.lda + lane_kc) * 2u : kOOB;
    o.lds = smem_base + (unsigned)__builtin_amdgcn_readfirstlane(dst) + LA * v * 1024;
    o.ld = args.lda;
    return o;
  };
  auto prep_b = [&](const Cursor& c, int dst) SPT_INLINE {
    OpLoads o;
    o.k0 = __builtin_amdgcn_readfirstlane(c.u) * BK + __builtin_amdgcn_readfirstlane(c.tl.kb);
    o.r = c.rb;
    o.v0 = lane_kc < K - o.k0 ? (unsigned)(b_lrow * args.ldb + lane_kc) * 2u : kOOB;
    o.lds = smem_base + (unsigned)__builtin_amdgcn_readfirstlane(dst) + LB * v * 1024;
    o.ld = args.ldb;
    return o;
  };
  // load j (< LA) of this wave's share of an A tile / a B tile
  auto load_a = [&](const OpLoads& o, int j) SPT_INLINE {
    dma16_unseen(o.r, o.lds + j * 1024, add_in_place(o.v0, (unsigned)(a_urow(j) * o.ld) * 2u), 2u * o.k0);
  };
  auto load_b = [&](const OpLoads& o, int j) SPT_INLINE {
    dma16_unseen(o.r, o.lds + j * 1024, add_in_place(o.v0, (unsigned)(b_urow(j) * o.ld) * 2u), 2u * o.k0);
  };
  auto issue_a = [&](const Cursor& c, int dst) SPT_INLINE {
    const OpLoads o = prep_a(c, dst);
#pragma unroll
    for (int j = 0; j < LA; ++j) load_a(o, j);
  };
  auto issue_b = [&](const Cursor& c, int dst) SPT_INLINE {
    const OpLoads o = prep_b(c, dst);
#pragma unroll
    for (int j = 0; j < LB; ++j) load_b(o, j);
  };
  // LDS byte offsets of the A and B tiles of K-tile g, from ring position p = 2g mod 5 (split) or
  // g mod 2 (stages)
  auto a_at = [&](int p) SPT_INLINE { return SPLIT ? p * A_BYTES : p * STAGE; };
  auto b_at = [&](int p) SPT_INLINE { return SPLIT ? (p + 1 == S ? 0 : p + 1) * A_BYTES : p * STAGE + A_BYTES; };
  auto pos_step = [&](int p, int n) SPT_INLINE {  // ring position of K-tile g+n
    const int q = SPLIT ? p + 2 * n : p + n;  // n <= 2, so q < 2S
    return q >= S ? q - S : q;
  };

  u32x4 xf[NSUB][FN], yf[NSUB][FM];  // the K-tile's fragments: B side (x), A side (y)
  Acc acc[FN][FM];
  Acc zero_acc;
#pragma unroll
  for (int e = 0; e < (int)(sizeof(Acc) / sizeof(float)); ++e) zero_acc[e] = 0.f;

  // The K-tile's fragment reads in a fixed order (k-step s: the FN B fragments, then the FM A
  // fragments); read i of NR.
  constexpr int NR = NSUB * (FN + FM);
  auto frag_bases = [&](int p, const char*& pa, const char*& pb) SPT_INLINE {
    const int pu = __builtin_amdgcn_readfirstlane(p);
    pa = smem + opaque_s32(a_at(pu));
    pb = smem + opaque_s32(b_at(pu));
  };
  auto read_one = [&](auto i_c, const char* pa, const char* pb) SPT_INLINE {
    constexpr int i = decltype(i_c)::value, s = i / (FN + FM), f = i % (FN + FM);
    if constexpr (f < FN) xf[s][f] = *(const u32x4*)(pb + b_rd[s] + f * FRAG);
    else yf[s][f - FN] = *(const u32x4*)(pa + a_rd[s] + (f - FN) * FRAG);
  };
  auto read_frags = [&](int p) SPT_INLINE {
    const char *pa, *pb;
    frag_bases(p, pa, pb);
    static_for<NR>([&](auto i_c) { read_one(i_c, pa, pb); });
    wait_lgkmcnt0();
  };
  // The same reads with NL loads spread evenly between them: load l goes out just before read
  // floor(l * NR / NL). A wave issues its LDS-DMA loads at a limited rate, so in a burst the
  // reads queued behind them would wait; interleaved, the LDS serves the reads while the loads
  // issue.
  auto read_frags_with_loads = [&](int p, auto nl_c, auto&& load) SPT_INLINE {
    constexpr int NL = decltype(nl_c)::value;
    const char *pa, *pb;
    frag_bases(p, pa, pb);
    static_for<NR>([&](auto i_c) {
      constexpr int i = decltype(i_c)::value;
      static_for<NL>([&](auto l_c) {
        constexpr int l = decltype(l_c)::value;
        if constexpr (l * NR / NL == i) load(l);
      });
      read_one(i_c, pa, pb);
    });
    wait_lgkmcnt0();
  };
  // the MFMAs of one K-tile; kFirst starts every chain from zero (accumulate = (k != 0)). Within a
  // k-step the blocks go row by row in a snake (the A fragment index runs up, then down), so one
  // operand carries over at every row change; the chip runs at its power limit here, and fewer
  // operand bits changing between MFMAs measured about 1 % faster.
  auto compute = [&](auto first_c) SPT_INLINE {
    constexpr bool kFirst = decltype(first_c)::value;
    __builtin_amdgcn_s_setprio(1);
    static_for<NSUB>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      static_for<FN * FM>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value, i = m / FM, j = ((i + s) & 1) ? FM - 1 - m % FM : m % FM;
        if constexpr (MF == 16) acc[i][j] = mfma16<TIn>(yf[s][j], xf[s][i], (kFirst && s == 0) ? zero_acc : acc[i][j]);
        else acc[i][j] = mfma32<TIn>(xf[s][i], yf[s][j], (kFirst && s == 0) ? zero_acc : acc[i][j]);
      });
    });
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Store this wave's part of output tile `tl` from the accumulators: fp32 -> output type, 8
  // consecutive columns per lane. The lane index is re-read through an opaque move, so the address
  // arithmetic stays here instead of being hoisted into registers held across the K-loop.
  // With kReads, the 24 fragment reads of the K-tile at ring position p go out between the stores
  // (one or two after each), so that the reads do not queue behind all sixteen stores; the reads
  // are then complete on return. Only for 16-bit outputs: with fp32 ones (split-K partial planes)
  // the accumulators live beside the fragments being read spilled registers.
  auto epilogue = [&](const PpTile& tl_in, auto reads_c, int p) SPT_INLINE {
    constexpr bool kReads = decltype(reads_c)::value;
    PpTile tl;
    tl.t = tl_in.t;
    tl.row0 = __builtin_amdgcn_readfirstlane(tl_in.row0);
    tl.col0 = __builtin_amdgcn_readfirstlane(tl_in.col0);
    tl.rows_left = __builtin_amdgcn_readfirstlane(tl_in.rows_left);
    tl.cols_left = __builtin_amdgcn_readfirstlane(tl_in.cols_left);
    tl.ks = __builtin_amdgcn_readfirstlane(tl_in.ks);
    tl.kb = 0;
    const __amdgpu_buffer_rsrc_t rc = c_rsrc(tl);
    const int ln = (int)opaque_u32((unsigned)lane);
    // MF = 16: lane l holds rows 4(l/16) + e of each A block, columns 8(l mod 16) .. +7 (one per B
    // fragment). MF = 32: rows l mod 32, 8 consecutive columns per pair of accumulator groups.
    const int m_lane = MF == 16 ? m_base + 4 * (ln / 16) : m_base + ln % MF;
    const int n_lane = MF == 16 ? tl.col0 + TN * wn + 8 * (ln % 16) : tl.col0 + TN * wn + 8 * (ln / MF);
    const bool full = tl.rows_left >= BM && tl.cols_left >= BN;
    // A finished output tile is not read again by this launch: its interior stores go out
    // non-temporal (measured 1-2 % faster on 4096^3 .. 16384^2 x 1024). Split-K partial planes, which
    // the reduction reads back next, keep the default policy (1.4 % slower non-temporal), and so do
    // the MF = 32 stores, whose quarter-waves cover 16 rows of 16 bytes rather than whole 128-byte
    // lines (non-temporal, 16384^2 x 1024 ran 30 % slower).
    const bool nt = MF == 16 && args.splits == 1;
    const unsigned voff = (unsigned)(m_lane * args.ldc + n_lane) * (unsigned)es;
    // The tile's stores in one of three forms, chosen once per tile rather than at every store:
    // 0 interior, non-temporal; 1 interior, default policy; 2 edge tile, masked per element.
    auto stores = [&](auto mode_c) SPT_INLINE {
      constexpr int kMode = decltype(mode_c)::value;
      // 8 consecutive outputs at (m_lane + dm, n_lane + dn)
      auto put8 = [&](const float (&vv)[8], int dm, int dn) SPT_INLINE {
        if constexpr (kMode == 0) store8_at<OUT, kStoreNonTemporal>(vv, rc, voff, (unsigned)((dm * args.ldc + dn) * es));
        else if constexpr (kMode == 1) store8_at<OUT>(vv, rc, voff, (unsigned)((dm * args.ldc + dn) * es));
        else store8<OUT, true>(vv, rc, m_lane + dm, tl.rows_left, n_lane + dn, N, args.ldc);
        __builtin_amdgcn_sched_barrier(0);
      };
      const char *pa = nullptr, *pb = nullptr;
      if constexpr (kReads) frag_bases(p, pa, pb);
      // MF = 16: store s is A block j = s/4, row e = s%4, columns 8c .. 8c+7 from the FN = 8 B
      // fragments. MF = 32: store s is block (i, j) = (s/(2FM), (s/2) mod FM), half h = s%2, whose
      // elements 8h .. 8h+7 hold columns 32i + 16h + 8(l/32) + 0..7.
      constexpr int NS = MF == 16 ? FM * 4 : FN * FM * 2;
      static_for<NS>([&](auto s_c) {
        constexpr int st = decltype(s_c)::value;
        float vv[8];
        if constexpr (MF == 16) {
          constexpr int j = st / 4, e = st % 4;
#pragma unroll
          for (int f = 0; f < FN; ++f) vv[f] = acc[f][j][e];
          put8(vv, 16 * j + e, 0);
        } else {
          constexpr int i = st / (2 * FM), j = (st / 2) % FM, h = st % 2;
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = acc[i][j][8 * h + e];
          put8(vv, 32 * j, 32 * i + 16 * h);
        }
        if constexpr (kReads) {
          static_for<NR>([&](auto r_c) {
            if constexpr (decltype(r_c)::value * NS / NR == st) read_one(r_c, pa, pb);
          });
        }
      });
      if constexpr (kReads) wait_lgkmcnt0();
    };
    if (full && nt) stores(std::integral_constant<int, 0>{});
    else if (full) stores(std::integral_constant<int, 1>{});
    else stores(std::integral_constant<int, 2>{});
  };

  using t_ = std::true_type;
  using f_ = std::false_type;
  PpTile prev;  // the output tile whose stores are pending
  prev.t = args.num_tiles;

  if (grp == 0) {
    // --------------------------------------------------------------------------- G0
    Cursor cur = cursor_at(u0);  // K-tile g
    Cursor nx = cur;             // K-tile g+1
    advance(nx);
    issue_a(cur, a_at(0));
    issue_b(cur, b_at(0));
    if (SPLIT && valid(nx)) {
      issue_a(nx, a_at(pos_step(0, 1)));
      wait_vmcnt<P.pp_g0_prologue_wait>();  // K-tile 0 landed; A(1) may be in flight
    } else {
      wait_vmcnt<0>();
    }
    barrier_sync();  // K-tile 0 visible
    int p = 0;       // ring position of K-tile g
    auto step = [&](auto first_c) SPT_INLINE {
      // phase 2g: memory. Load ahead, store the previous output tile, read K-tile g.
      if constexpr (decltype(first_c)::value || !SPLIT) {
        if (valid(nx)) {
          const int q = pos_step(p, 1);
          if constexpr (!SPLIT) issue_a(nx, a_at(q));
          issue_b(nx, b_at(q));
        }
        if (decltype(first_c)::value && prev.t < args.num_tiles) {
          if constexpr (OUT == 2) {
            epilogue(prev, std::false_type{}, 0);
            read_frags(p);
          } else {
            epilogue(prev, std::true_type{}, p);
          }
        } else {
          read_frags(p);
        }
      } else {
        if (valid(nx)) {
          const OpLoads o = prep_b(nx, b_at(pos_step(p, 1)));
          read_frags_with_loads(p, std::integral_constant<int, LB>{}, [&](int j) SPT_INLINE { load_b(o, j); });
        } else {
          read_frags(p);
        }
      }
      barrier_sync();
      // phase 2g+1: compute K-tile g, then make sure this group's loads for K-tile g+1 (and the
      // stores issued after them) are done
      compute(first_c);
      wait_vmcnt<0>();
      barrier_sync();
      p = pos_step(p, 1);
      advance(nx);
    };
    for (; valid(cur); cur.tl = tile_at(cur.tl.t + args.grid)) {
      step(t_{});
      for (int u = 1; u < KT; ++u) step(f_{});
      prev = cur.tl;
    }
    // phase 2G: the last tile's stores, beside G1's last compute phase
    epilogue(prev, std::false_type{}, 0);
    barrier_sync();
  } else {
    // --------------------------------------------------------------------------- G1
    Cursor cur = cursor_at(u0);  // K-tile g
    Cursor n2 = cur;             // K-tile g+2
    advance(n2);
    advance(n2);
    barrier_sync();  // K-tile 0 visible
    barrier_sync();  // phase 0: idle
    int p = 0;
    auto step = [&](auto first_c) SPT_INLINE {
      constexpr bool kFirst = decltype(first_c)::value;
      // phase 2g+1: memory. Load A(g+2), read K-tile g, and make sure A(g+1) has landed, with
      // A(g+2) possibly still in flight. In the first K-tile of an output tile the previous tile's
      // stores go out here too; the wait then comes before them, so that the count of loads
      // issued after A(g+1) stays exact.
      bool loaded = false;
      if constexpr (SPLIT && kFirst) {
        if (valid(n2)) {
          issue_a(n2, a_at(pos_step(p, 2)));
          loaded = true;
        }
      }
      // A(g+1) landed: only the loads of A(g+2) may still be in flight
      auto wait_a = [&]() SPT_INLINE {
        if constexpr (SPLIT) {
          if (loaded) wait_vmcnt<P.pp_g1_wait>();
          else wait_vmcnt<0>();
        }
      };
      if constexpr (kFirst) {
        wait_a();
        if (prev.t < args.num_tiles) {
          if constexpr (OUT == 2) {
            epilogue(prev, std::false_type{}, 0);
            read_frags(p);
          } else {
            epilogue(prev, std::true_type{}, p);
          }
        } else {
          read_frags(p);
        }
      } else if constexpr (SPLIT) {
        if (valid(n2)) {
          const OpLoads o = prep_a(n2, a_at(pos_step(p, 2)));
          read_frags_with_loads(p, std::integral_constant<int, LA>{}, [&](int j) SPT_INLINE { load_a(o, j); });
          loaded = true;
        } else {
          read_frags(p);
        }
        wait_a();
      } else {
        read_frags(p);
      }
      barrier_sync();
      // phase 2g+2: compute
      compute(first_c);
      barrier_sync();
      p = pos_step(p, 1);
      advance(n2);
    };
    for (; valid(cur); cur.tl = tile_at(cur.tl.t + args.grid)) {
      step(t_{});
      for (int u = 1; u < KT; ++u) step(f_{});
      prev = cur.tl;
    }
    epilogue(prev, std::false_type{}, 0);  // after the last barrier
  }
}

template <int S, int MF>
static KernelEntry make_pp_entry() {
  KernelEntry k;
  k.bm = 256; k.bn = 256; k.bk = 64; k.stages = S; k.waves = 8; k.load_path = 1;
  k.lds_bytes = S == 5 ? 5 * 256 * 64 * 2 : S * (256 + 256) * 64 * 2;
  k.mfma = MF;
  k.fn[0][0] = (const void*)&gemm_pp_kernel<S, MF, _Float16, 0>;
  k.fn[0][1] = (const void*)&gemm_pp_kernel<S, MF, _Float16, 1>;
  k.fn[0][2] = (const void*)&gemm_pp_kernel<S, MF, _Float16, 2>;
  k.fn[1][0] = (const void*)&gemm_pp_kernel<S, MF, __bf16, 0>;
  k.fn[1][1] = (const void*)&gemm_pp_kernel<S, MF, __bf16, 1>;
  k.fn[1][2] = (const void*)&gemm_pp_kernel<S, MF, __bf16, 2>;
  return k;
}

const KernelEntry* pp_kernel_table(int* count) {
  static const KernelEntry table[] = {make_pp_entry<5, 16>(), make_pp_entry<2, 16>(), make_pp_entry<5, 32>()};
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace spt
