// Device-side helpers shared by the gfx950 GEMM kernels: vector types, wait-count and barrier
// wrappers, buffer descriptors, the MFMA wrapper, the epilogue store and the tile geometry.
#pragma once

#include <type_traits>
#include <utility>

#include "spt_common.h"

// Lambdas inside kernels are marked with this: an out-of-line call would pass the accumulator array
// through scratch memory.
#define SPT_INLINE __attribute__((always_inline))

namespace spt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr unsigned kOOB = 0x80000000u;       // voffset beyond every num_records: loads give 0, stores drop
constexpr unsigned kMaxRecords = 0x7FFFFFF0u;
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data format

// ------------------------------------------------------------------------------ waits, barrier
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// wait until at most t*LW of this wave's vector-memory operations are outstanding (t clamped to [0, T])
template <int LW, int T>
__device__ __forceinline__ void wait_vmcnt_tiles(int t) {
  if constexpr (T <= 0) {
    wait_vmcnt<0>();
  } else {
    if (t >= T) wait_vmcnt<LW * T>();
    else wait_vmcnt_tiles<LW, T - 1>(t);
  }
}

__device__ __forceinline__ void barrier_sync() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const unsigned n = bytes > kMaxRecords ? kMaxRecords : (unsigned)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

// One direct global->LDS load: 64 lanes x 16 bytes from `r` at per-lane byte offset
// voffset + soffset into the 1 KiB of LDS starting at `lds` (lane l lands at lds + 16*l).
// Offsets at or beyond the descriptor's num_records read as zero.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, unsigned voffset, unsigned soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voffset, soffset, 0, 0);
}

// The same load with the non-temporal hint (the nt bit of the instruction's cache policy): the
// lines take the streaming replacement policy and are not kept for reuse, for an operand every
// byte of which one workgroup reads once, so that it does not displace the operand the others share.
__device__ __forceinline__ void dma16_stream(__amdgpu_buffer_rsrc_t r, void* lds, unsigned voffset, unsigned soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voffset, soffset, 0, 2);
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(uintptr_t)(const lds_void_t*)p; }

// The same load issued through inline assembly (the LDS address travels in M0), so the compiler
// does not see an LDS write: otherwise it guards every later LDS read that might alias the
// destination with a wait for this load, which serialises fragment reads behind the loads in
// flight. A kernel using it orders its LDS reads after its own loads explicitly (s_waitcnt vmcnt,
// then s_barrier) before any wave reads a tile.
// `lds` is the destination's LDS byte address (wave-uniform). hipcc warns that M0, a reserved
// register, is on the clobber list: the compiler neither saves it around the statement nor knows
// the value left in it, so a kernel using this must not rely on M0 anywhere else (the compiler's
// own code included; tests/test_generated_code.py reads the built kernels back and checks that).
__device__ __forceinline__ void dma16_unseen(__amdgpu_buffer_rsrc_t r, unsigned lds, unsigned voffset,
                                             unsigned soffset) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(r), "s"(soffset)
               : "memory", "m0");
}

// v + c (c wave-uniform), computed where it is written: the compiler may not hoist it, so a loop
// that issues many loads keeps one temporary instead of one precomputed register per load.
__device__ __forceinline__ unsigned add_in_place(unsigned v, unsigned c) {
  unsigned r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(c), "v"(v));
  return r;
}

// x, through a move the compiler cannot see into: values derived from the result are computed
// after this point rather than hoisted above it.
__device__ __forceinline__ unsigned opaque_u32(unsigned x) {
  unsigned r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// The same for a wave-uniform value (kept in a scalar register). Used for ring offsets, so the
// compiler does not turn every address derived from them into an induction variable of its own.
__device__ __forceinline__ int opaque_s32(int x) {
  int r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "s"(x));
  return r;
}

// static_for<N>(f): f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}),
// so loop indices that select code paths are compile-time constants.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------------------ MFMA
template <typename TIn>
__device__ __forceinline__ f32x4 mfma16(u32x4 x, u32x4 y, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16<__bf16>(u32x4 x, u32x4 y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<_Float16>(u32x4 x, u32x4 y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c,
                                                0, 0, 0);
}

// v_mfma_f32_32x32x16: D[i][j] += sum_k X[i][k] Y[j][k] over a 32x32 block and 16 k. Lane l supplies
// row l mod 32 of X and of Y (8 values of k each; both operands use the same lane-to-k map, so the
// pairing of products does not depend on it) and holds D[8g + 4(l/32) + e][l mod 32] in element
// 4g + e of the result (g < 4, e < 4).
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <typename TIn>
__device__ __forceinline__ f32x16 mfma32(u32x4 x, u32x4 y, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<__bf16>(u32x4 x, u32x4 y, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<_Float16>(u32x4 x, u32x4 y, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c,
                                                0, 0, 0);
}

// ------------------------------------------------------------------------------ epilogue
// Two fp32 values rounded to nearest-even and packed, a in the low half. Converting them as one
// two-element vector gives gfx950's two-source conversions (v_cvt_pk_bf16_f32 and v_cvt_pk_f16_f32,
// one instruction per pair); two scalar conversions cost a conversion per value plus a shift and an
// or per pair, four times the VALU work of an output tile's epilogue.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ unsigned pack_f16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Store the 8 consecutive outputs v[0..7] at row m_rel (relative to the tile's first row),
// column n (absolute). OUT: 0 f16, 1 bf16, 2 f32. With EDGE, rows >= rows_left and columns
// >= N are skipped element by element; without it the whole 8-wide segment is in range.
template <int OUT, bool EDGE>
__device__ __forceinline__ void store8(const float (&v)[8], __amdgpu_buffer_rsrc_t rc, int m_rel, int rows_left,
                                      int n, int N, int ldc) {
  if (EDGE && (m_rel >= rows_left || n >= N)) return;
  if constexpr (OUT == 2) {
    const unsigned off = (unsigned)(m_rel * ldc + n) * 4u;
    if (!EDGE || n + 8 <= N) {
      u32x4 lo = {__builtin_bit_cast(unsigned, v[0]), __builtin_bit_cast(unsigned, v[1]),
                  __builtin_bit_cast(unsigned, v[2]), __builtin_bit_cast(unsigned, v[3])};
      u32x4 hi = {__builtin_bit_cast(unsigned, v[4]), __builtin_bit_cast(unsigned, v[5]),
                  __builtin_bit_cast(unsigned, v[6]), __builtin_bit_cast(unsigned, v[7])};
      __builtin_amdgcn_raw_buffer_store_b128(lo, rc, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(hi, rc, off + 16u, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[e]), rc, off + 4u * e, 0, 0);
    }
  } else {
    const unsigned off = (unsigned)(m_rel * ldc + n) * 2u;
    unsigned p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = OUT == 1 ? pack_bf16(v[2 * e], v[2 * e + 1]) : pack_f16(v[2 * e], v[2 * e + 1]);
    if (!EDGE || n + 8 <= N) {
      u32x4 q = {p[0], p[1], p[2], p[3]};
      __builtin_amdgcn_raw_buffer_store_b128(q, rc, off, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(p[e >> 1] >> (16 * (e & 1))), rc, off + 2u * e, 0, 0);
    }
  }
}

// Cache-policy operand of a buffer store that marks the data non-temporal (the nt bit on gfx950).
constexpr int kStoreNonTemporal = 2;

// Store the 8 consecutive outputs v[0..7] at byte offset voffset + soffset of `rc` (an interior
// segment: no masking), with cache policy CPOL (0, or kStoreNonTemporal).
template <int OUT, int CPOL = 0>
__device__ __forceinline__ void store8_at(const float (&v)[8], __amdgpu_buffer_rsrc_t rc, unsigned voffset,
                                         unsigned soffset) {
  if constexpr (OUT == 2) {
    u32x4 lo = {__builtin_bit_cast(unsigned, v[0]), __builtin_bit_cast(unsigned, v[1]),
                __builtin_bit_cast(unsigned, v[2]), __builtin_bit_cast(unsigned, v[3])};
    u32x4 hi = {__builtin_bit_cast(unsigned, v[4]), __builtin_bit_cast(unsigned, v[5]),
                __builtin_bit_cast(unsigned, v[6]), __builtin_bit_cast(unsigned, v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(lo, rc, voffset, soffset, CPOL);
    __builtin_amdgcn_raw_buffer_store_b128(hi, rc, voffset, soffset + 16u, CPOL);
  } else {
    unsigned p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = OUT == 1 ? pack_bf16(v[2 * e], v[2 * e + 1]) : pack_f16(v[2 * e], v[2 * e + 1]);
    u32x4 q = {p[0], p[1], p[2], p[3]};
    __builtin_amdgcn_raw_buffer_store_b128(q, rc, voffset, soffset, CPOL);
  }
}

// ------------------------------------------------------------------------------ the kernel
template <int BM, int BN, int BK, int S, int WM, int WN>
struct TileShape {
  static constexpr int W = WM * WN, NT = 64 * W;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16-row fragments per wave (A side, B side)
  static constexpr int NSUB = BK / 32;              // MFMA k-steps per K-tile
  // LDS rows: 64-element groups of 128-byte rows, or one 64-byte row for a 32-deep K-tile
  static constexpr int GK = BK == 32 ? 32 : 64;     // elements per LDS row
  static constexpr int RB = 2 * GK;                 // bytes per LDS row
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;             // rows one DMA instruction fills
  static constexpr int FRAG = 16 * RB;              // bytes between consecutive 16-row fragments
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  // Split ring (S = 5 with 64-deep K-tiles): five operand slots; K-tile k's A tile sits in slot
  // 2k mod 5 and its B tile in slot 2k+1 mod 5, i.e. two and a half stages.
  static constexpr bool SPLIT = BK == 64 && S == 5;
  static constexpr int SLOT = A_BYTES;
  static constexpr int LDS = SPLIT ? S * SLOT : S * STAGE;
  static constexpr int A_INSTR = A_BYTES / 1024, B_INSTR = B_BYTES / 1024;  // 1 KiB per DMA instruction
  static constexpr PipeProtocol P = pipe_protocol(BM, BN, BK, S, W);
  static constexpr int LA = P.la, LB = P.lb, LW = P.lw;   // per wave, per stage
  static constexpr int MAX_VM = P.max_wait;               // largest vmcnt threshold
  static_assert(LA == A_INSTR / W && LB == B_INSTR / W && (P.split != 0) == SPLIT, "protocol and tile agree");
  static_assert(BK == 32 || BK == 64 || BK == 128, "K-tile is one 64-byte row or one or two 128-byte groups");
  static_assert(S >= 1 && S <= (BK == 128 ? 8 : 5), "1..5 stages (up to 8 for 128-deep K-tiles)");
  static_assert(!SPLIT || A_BYTES == B_BYTES, "split ring: A and B tiles fill equal slots");
  static_assert(TM % 16 == 0 && TN % 32 == 0, "wave tile: 16-row A fragments, pairs of 16-row B fragments");
  static_assert(A_INSTR % W == 0 && B_INSTR % W == 0, "every wave issues the same number of loads");
  static_assert(BM % RPI == 0 && BN % 32 == 0, "tile rows");
  static_assert(MAX_VM < 64, "vmcnt thresholds fit the 6-bit counter");
  static_assert(LDS <= 160 * 1024, "LDS ring fits the 160 KiB of a CU");
  static_assert(NSUB % 2 == 0 || NSUB == 1, "fragment double buffer parity");
};

}  // namespace spt
