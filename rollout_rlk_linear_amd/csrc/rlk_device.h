// rlk_device.h — device building blocks for the gfx950 linear log-prob kernels.
//
// * LDS-DMA fed bf16 MFMA mainloops (v_mfma_f32_16x16x32_bf16, and
//   v_mfma_f32_32x32x16_bf16 for dH) computing a BM x BN fp32 tile with K
//   walked in ascending steps of 32: AsyncGemmP for two K-contiguous operands
//   (A * B^T), AsyncGemmKN for a K-major B (A * B) and AsyncGemmKK for two
//   K-major operands (A^T * B), the last two with fragments assembled by
//   transposing LDS reads.
// * The fixed-order reductions that make every output row independent of the
//   batch: a 16-lane DPP tree, the (m, R, B, zy) merge algebra, bf16 RNE.
//
// Every kernel that produces the same quantity goes through these helpers,
// so the per-element arithmetic, and hence the bits, are identical whatever
// the tile shape or grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rlk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int GROUP = 256;     // vocabulary columns per group (one forward tile width)

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Wave index within the workgroup, as a value the compiler knows is uniform
// across the wave (so choices made from it stay scalar).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------- bf16 --

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, by the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// fp32 -> bf16 bits (same rounding).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// ---------------------------------------------------------- fast exp ----

// exp(x) through the hardware base-2 exponential. Used for the per-element
// terms; the same instruction sequence is used everywhere.
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ------------------------------------------------- 16-lane DPP tree -----
// Pairings per level: rotate-by-8 within a row of 16 lanes, mirror within 8,
// reverse within 4, swap within 2. Each level pairs every lane with a unique
// partner, and after four levels every lane of the 16-lane row holds the
// reduction of all 16 inputs, with identical bits in every lane (IEEE add
// and max are commutative).

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                              0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_3210 = 0x1B;
constexpr int DPP_QUAD_1032 = 0xB1;

__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp_f<DPP_ROW_ROR8>(x);
  x = x + dpp_f<DPP_ROW_HALF_MIRROR>(x);
  x = x + dpp_f<DPP_QUAD_3210>(x);
  x = x + dpp_f<DPP_QUAD_1032>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<DPP_ROW_ROR8>(x));
  x = fmaxf(x, dpp_f<DPP_ROW_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f<DPP_QUAD_3210>(x));
  x = fmaxf(x, dpp_f<DPP_QUAD_1032>(x));
  return x;
}
__device__ __forceinline__ int row16_sum_i(int x) {
  x = x + dpp_i<DPP_ROW_ROR8>(x);
  x = x + dpp_i<DPP_ROW_HALF_MIRROR>(x);
  x = x + dpp_i<DPP_QUAD_3210>(x);
  x = x + dpp_i<DPP_QUAD_1032>(x);
  return x;
}

// ------------------------------------------------ row statistics --------
// Partial softmax statistics of a set of vocabulary columns of one row:
//   m = max z, R = sum over the set minus one arg-max entry of exp(z - m),
//   B = sum over the set of exp(z - m)(z - m), zy = target logit or -inf.
struct Part {
  float m, R, B, zy;
};

__device__ __forceinline__ Part part_empty() { return Part{neg_inf(), 0.f, 0.f, neg_inf()}; }

// Merge of two partials over disjoint column sets. The side with the larger
// max is the base (the left one on a tie); with d = m_other - m_base <= 0,
//   R = R_base + e^d (1 + R_other),  B = B_base + e^d (B_other + (1 + R_other) d).
// An empty side (m = -inf) contributes nothing: its terms are masked to +0,
// and R_base, B_base come out unchanged (they are never -0: every record's
// sums include the +0 of its max column). Straight-line on
// purpose: with an early return for the empty side the compiler branches
// around the exponential, and the merge chains of the combine serialise.
// Accurate expf; contraction is disabled for the whole library, so the
// arithmetic is exactly as written.
__device__ __forceinline__ Part part_merge(const Part& l, const Part& r) {
  const bool left_base = !(r.m > l.m);
  const float bm = left_base ? l.m : r.m, bR = left_base ? l.R : r.R, bB = left_base ? l.B : r.B;
  const float om = left_base ? r.m : l.m, oR = left_base ? r.R : l.R, oB = left_base ? r.B : l.B;
  Part out;
  out.m = bm;
  out.zy = fmaxf(l.zy, r.zy);
  const float d = om - bm;
  const float e = expf(d);
  const float one_r = 1.f + oR;
  const uint32_t keep = om == neg_inf() ? 0u : 0xFFFFFFFFu;
  out.R = bR + __uint_as_float(__float_as_uint(e * one_r) & keep);
  out.B = bB + __uint_as_float(__float_as_uint(e * (oB + one_r * d)) & keep);
  return out;
}

// ------------------------------------------------ rolled epilogues -----
// Copies row block i of an accumulator array into blk through a chain of
// uniform branches, so epilogues can loop over i without unrolling (a fully
// unrolled epilogue does not fit the instruction cache).
template <int K, int MI, int NJ>
__device__ __forceinline__ void acc_row_block(const f32x4 (&acc)[MI][NJ], int i,
                                              f32x4 (&blk)[NJ]) {
  if constexpr (K < MI) {
    if (i == K) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) blk[j] = acc[K][j];
      return;
    }
    acc_row_block<K + 1>(acc, i, blk);
  }
}

// ------------------------------------------------ async (LDS-DMA) mainloop
//
// gfx950 buffer loads can write straight into LDS: `buffer_load_dwordx4 ...
// lds` stores lane i's 16 bytes at (LDS base + 16 i), so one instruction
// fills 1 KB. Operand rows are staged as 64-byte rows (32 bf16 = one MFMA
// k-step) in a ring of stages; the 16-byte pieces of each row are stored
// rotated by the row index (row_slot below), which keeps the 16-row fragment
// reads free of bank conflicts. Rows past the valid range read as
// zero through the buffer's hardware range check (num_records), which tests
// the vector offset alone: every row offset therefore sits in the vector
// offset and only the k offset of a stage, which stays inside a valid row,
// travels in the scalar offset.

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// Buffer resource (V#) for a raw byte buffer: base, stride 0, num_records =
// bytes (loads at or past it return zero), gfx9 dword 3.
// All arguments must be wave-uniform; the words are passed through
// readfirstlane so they live in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 32-bit LDS address of a shared-memory pointer (what M0 expects).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

// Piece placement of a staged 64-byte row: row r (within its 16-row block)
// keeps logical 16-byte piece c at slot (c + r / 2) mod 4, and slot s holds
// piece (s - r / 2) mod 4. A 16-byte fragment read (lane l: row l % 16,
// piece l / 16) is then free of bank conflicts on gfx950 (measured with the
// LDS bank-conflict counter: 0 cycles per ds_read_b128, where XOR placements
// such as c ^ ((r / 2) ^ (r / 8)) cost 4 and a linear row layout 12).
__device__ __forceinline__ int row_slot(int c, int r) { return (c + (r >> 1)) & 3; }
__device__ __forceinline__ int row_piece(int s, int r) { return (s - (r >> 1)) & 3; }

// One 1 KB LDS-DMA block: lane i's 16 bytes from (base + voff + soff) land at
// LDS (addr + 16 i). Written as inline asm so that the compiler does not
// track these LDS writes: its own conservative waits (vmcnt(0) before every
// LDS read) would drain the prefetch pipeline. Ordering is the caller's:
// explicit vmcnt waits and barriers (all with memory clobbers).
// The compiler's hazard checks do not look inside inline asm, so the asm
// keeps two gfx9 rules itself: M0 written by the SALU needs 1 wait state
// before the LDS-DMA reads it, and an SGPR written by a VALU instruction
// needs 5 before a buffer instruction reads it. The descriptor and offsets
// pass through readfirstlane (a no-op where the compiler knows them to be
// uniform); where it does not, it parks them in VGPRs and reads them back
// with a v_readfirstlane just before the asm. SETTLE = true (s_nop 4, 5 wait
// states in all) is for the call sites where it does that; the test suite
// scans the built code for the pattern, so a site that needs it and lacks it
// does not go unnoticed.
// NT = true marks the load non-temporal (the nt cache bit: lines it brings in
// are not retained), for a stream that would otherwise push out data a
// later kernel reads; it always settles.
template <bool SETTLE = false, bool NT = false>
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t addr, int voff, int soff) {
  const i32x4 rs = {__builtin_amdgcn_readfirstlane(rsrc[0]), __builtin_amdgcn_readfirstlane(rsrc[1]),
                    __builtin_amdgcn_readfirstlane(rsrc[2]), __builtin_amdgcn_readfirstlane(rsrc[3])};
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane((int)addr)), "v"(voff), "s"(rs),
          "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory", "m0");
  else if constexpr (SETTLE)
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane((int)addr)), "v"(voff), "s"(rs),
          "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane((int)addr)), "v"(voff), "s"(rs),
          "s"(__builtin_amdgcn_readfirstlane(soff))
        : "memory", "m0");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// C[BM x BN] += A[BM x K] * B[BN x K]^T, both operands K-contiguous
// (element (r, k) at base[r * ld + k]), rows past a_rows / b_rows reading as
// zero. k runs over [k_begin, k_end) in ascending MFMA steps of 32;
// (k_end - k_begin) must be a multiple of 64 and every valid row must hold
// k_end elements. WM x WN = 4 waves; wave (wm, wn) owns rows wm*WTM.. and
// columns wn*WTN.. of the tile, and acc[i][j][r] is element
// (row wm*WTM + 16 i + 4 (lane / 16) + r, col wn*WTN + 16 j + lane % 16).
//
// k-steps are staged in pairs: a slot holds 128 bytes of each operand row
// (two k-steps), so each group of eight 16-byte DMA pieces of a row is one
// whole 128-byte line and every L2 request carries a full line (with
// 64-byte rows each line takes two requests). A has a ring of two pair slots
// and B one of NSB (2 or 3): with 3, B's pair p + 2 is in flight while pair
// p is multiplied, so the operand that streams from HBM (W) has twice the
// lookahead of the one that stays in L2 (hidden) within the same LDS (for the
// 256 x 256 forward the staging alone runs at 13.4 instead of 11.6 TB/s, but
// the whole kernel is no faster, so the kernels use 2). The DMA blocks of a
// pair go out between the first k-step's MFMAs,
// A's pair p + 1 before B's pair p + NSB - 1, so that in-order completion
// lets the wait for pair p leave B's newest pair in flight. The 16-byte
// pieces of row r are rotated by r (slot = (piece + r) mod 8), which keeps
// the 16-row fragment reads of both k-steps free of bank conflicts. Within a
// k-step all B fragments and two A fragments are read first, then A fragment
// i+2 is read while the MFMAs of row block i run (scheduling group barriers
// pin the order).
// BNT: B's loads are non-temporal (dma16's NT).
template <int BM, int BN, int WM, int WN, int NSB = 2, bool BNT = false>
struct AsyncGemmP {
  static constexpr int NW = WM * WN;
  static_assert(NW == 4, "4 waves per tile");
  static_assert(BM % 8 == 0 && BN % 8 == 0, "8-row DMA blocks");
  static_assert(NSB == 2 || NSB == 3, "2 or 3 pair slots for B");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 16, NJ = WTN / 16;
  static constexpr int ROWB = 128;
  static constexpr int SLOT_A = BM * ROWB, SLOT_B = BN * ROWB;
  static constexpr int LDS_BYTES = 2 * SLOT_A + NSB * SLOT_B;
  static constexpr int NI_A = BM / 8, NI_B = BN / 8;  // 1 KB blocks = 8 rows
  static constexpr int NI = NI_A + NI_B;
  static_assert(NI_A % NW == 0 && NI % NW == 0, "DMA blocks divide among the waves");
  static constexpr int NB = NI / NW;  // blocks per wave per pair
  static constexpr int NB_A = NI_A / NW, NB_B = NI_B / NW;
  // 128-byte staged rows: logical piece c of row r sits at slot (c + r) mod 8
  // (conflict-free 16-byte fragment reads for both k-steps of the pair)
  static __device__ __forceinline__ int slot(int c, int r) { return (c + r) & 7; }
  static __device__ __forceinline__ int piece_at(int s, int r) { return (s - r) & 7; }

  f32x4 acc[MI][NJ];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The first pairs of a run (B's pair 0, A's pair 0, then B's pair 1 with 3
  // slots), issued on their own: a persistent caller issues the next tile's
  // while it finishes the current one (its epilogue must then keep out of
  // A's and B's pair-0 slots, and B's pair-1 slot with 3), and passes
  // prefetched = true to run().
  __device__ __forceinline__ void prologue(unsigned char* lds, const uint16_t* A, int64_t lda,
                                           int a_rows, const uint16_t* B, int64_t ldb, int b_rows,
                                           int k_begin, int k_end) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int npairs = (k_end - k_begin) / 64;
    if (npairs <= 0) return;
    const uint32_t lds0 = lds_addr(lds);
    const int ar = a_rows < 0 ? 0 : (a_rows > BM ? BM : a_rows);
    const int br = b_rows < 0 ? 0 : (b_rows > BN ? BN : b_rows);
    const i32x4 rsA = make_rsrc(A, (uint32_t)(ar * lda * 2));
    const i32x4 rsB = make_rsrc(B, (uint32_t)(br * ldb * 2));
    const i32x4 rsNull = make_rsrc(A, 0u);
    const int row0 = 8 * wave + (lane >> 3);
    const int piece = piece_at(lane & 7, row0 & 15);
    const int voffA = (int)(row0 * lda * 2) + 16 * piece;
    const int voffB = (int)(row0 * ldb * 2) + 16 * piece;
    const int kb0 = k_begin * 2;
#pragma unroll
    for (int ii = 0; ii < NB_B; ++ii)
      dma16<false, BNT>(rsB, lds0 + (uint32_t)(2 * SLOT_A) + 1024u * wave + 1024u * NW * ii,
            voffB + (int)(ii * 64 * ldb), kb0);
#pragma unroll
    for (int ii = 0; ii < NB_A; ++ii)
      dma16(rsA, lds0 + 1024u * wave + 1024u * NW * ii, voffA + (int)(ii * 64 * lda), kb0);
    if constexpr (NSB == 3) {
      const i32x4 rb1 = npairs > 1 ? rsB : rsNull;
#pragma unroll
      for (int ii = 0; ii < NB_B; ++ii)
        dma16<false, BNT>(rb1, lds0 + (uint32_t)(2 * SLOT_A + SLOT_B) + 1024u * wave + 1024u * NW * ii,
              voffB + (int)(ii * 64 * ldb), kb0 + 128);
    }
  }

  // YOUNG > 0 with young_pending: the caller issued the prologue, then at
  // least YOUNG more vector-memory operations of its own in every wave (e.g.
  // the previous tile's stores), which need not have completed for pair 0:
  // with in-order completion, YOUNG pending operations at most mean that
  // everything older, the prologue included, has landed.
  // UNROLL: the pair's two k-steps as straight-line code (the refill test
  // becomes a constant instead of a branch after every row block). The
  // register allocator keeps each accumulator chain in place only when the
  // first pair has code of its own, which a young first wait (YOUNG > 0
  // with young_pending) gives it; without that it splits the chains through
  // VGPRs, so the callers that unroll also pass a young first wait.
  template <int YOUNG = 0, bool UNROLL = false>
  __device__ __forceinline__ void run(unsigned char* lds, const uint16_t* A, int64_t lda,
                                      int a_rows, const uint16_t* B, int64_t ldb, int b_rows,
                                      int k_begin, int k_end, bool prefetched = false,
                                      bool young_pending = false) {
    static_assert(YOUNG >= 0 && YOUNG + NB_B < 64, "vmcnt range");
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wm = wave % WM, wn = wave / WM;
    const int npairs = (k_end - k_begin) / 64;
    if (npairs <= 0) return;
    const uint32_t lds0 = lds_addr(lds);
    const int ar = a_rows < 0 ? 0 : (a_rows > BM ? BM : a_rows);
    const int br = b_rows < 0 ? 0 : (b_rows > BN ? BN : b_rows);
    const i32x4 rsA = make_rsrc(A, (uint32_t)(ar * lda * 2));
    const i32x4 rsB = make_rsrc(B, (uint32_t)(br * ldb * 2));
    // DMA: block j of an operand's slot holds its rows 8 j .. 8 j + 7; lane ->
    // row 8 j + lane / 8, physical piece lane % 8, which holds the logical
    // piece piece_at(lane % 8, row). Block wave + NW ii is row 8 wave + lane / 8
    // plus 32 ii rows (same row % 16). The buffer range check covers the vector
    // offset only (the scalar offset is added after it), so the whole row
    // offset, 32 ii rows included, travels in the vector offset and only the k
    // offset in the scalar one: a row at or past a_rows / b_rows then fails the
    // check and is never fetched.
    const int row0 = 8 * wave + (lane >> 3);
    const int piece = piece_at(lane & 7, row0 & 15);
    const int voffA = (int)(row0 * lda * 2) + 16 * piece;
    const int voffB = (int)(row0 * ldb * 2) + 16 * piece;
    // A pair past the last reads through an empty resource: its blocks land
    // zeros in a slot nobody reads and touch no memory, so the refill needs no
    // branch inside the MFMA sequence.
    const i32x4 rsNull = make_rsrc(A, 0u);
    auto a_dst = [&](int p) { return lds0 + (uint32_t)((p & 1) * SLOT_A) + 1024u * wave; };
    auto b_dst = [&](int p) {
      return lds0 + (uint32_t)(2 * SLOT_A + (p % NSB) * SLOT_B) + 1024u * wave;
    };
    // block ii < NB_A: A's block ii (address a, k offset ka, resource ra);
    // else B's block ii - NB_A
    auto issue_block = [&](int ii, uint32_t a, int ka, const i32x4& ra, uint32_t b, int kb,
                           const i32x4& rb) {
      if (ii < NB_A)
        dma16(ra, a + 1024u * NW * ii, voffA + (int)(ii * 64 * lda), ka);
      else
        dma16<false, BNT>(rb, b + 1024u * NW * (ii - NB_A), voffB + (int)((ii - NB_A) * 64 * ldb), kb);
    };
    // fragment offsets of this lane in a slot for half h (k-step 2 p + h):
    // row l % 16 of the block, logical piece 4 h + l / 16
    const int fr = lane & 15;
    const uint32_t foff0 = fr * ROWB + 16 * slot(lane >> 4, fr);
    const uint32_t foff1 = fr * ROWB + 16 * slot(4 + (lane >> 4), fr);

    // prologue, in the order pairs are needed: B 0, A 0, then B 1 (3 slots)
    if (!prefetched) prologue(lds, A, lda, a_rows, B, ldb, b_rows, k_begin, k_end);
    for (int p = 0; p < npairs; ++p) {
      // this wave's part of pairs p of A and B has landed: with 3 B slots
      // everything but B's pair p + 1 (issued after A's pair p), if any
      if (YOUNG > 0 && p == 0 && prefetched && young_pending) {
        if (NSB == 3 && p + 1 < npairs)
          wait_vmcnt<NB_B + YOUNG>();
        else
          wait_vmcnt<YOUNG>();
      } else if (NSB == 3 && p + 1 < npairs) {
        wait_vmcnt<NB_B>();
      } else {
        wait_vmcnt<0>();
      }
      barrier_only();  // everyone's has; the slots of A's pair p - 1 and B's p - 1 are free
      const int pa = p + 1, pb = p + NSB - 1;  // pairs refilled during this one
      const uint32_t da = a_dst(pa), db = b_dst(pb);
      const int ka = (k_begin + 64 * pa) * 2, kb = (k_begin + 64 * pb) * 2;
      const i32x4 ra = pa < npairs ? rsA : rsNull;
      const i32x4 rb = pb < npairs ? rsB : rsNull;
      const unsigned char* sa = lds + (p & 1) * SLOT_A;
      const unsigned char* sb = lds + 2 * SLOT_A + (p % NSB) * SLOT_B;
      constexpr int HSTEPS = UNROLL ? 2 : 1;
#pragma unroll HSTEPS
      for (int h = 0; h < 2; ++h) {
        constexpr int A0 = MI < 2 ? MI : 2;
        const uint32_t fo = h ? foff1 : foff0;
        bf16x8 af[MI], bfr[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bfr[j] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(sb + (wn * WTN + 16 * j) * ROWB + fo));
#pragma unroll
        for (int i = 0; i < A0; ++i)
          af[i] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(sa + (wm * WTM + 16 * i) * ROWB + fo));
        __builtin_amdgcn_sched_group_barrier(0x100, NJ + A0, 0);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (i + A0 < MI)
            af[i + A0] = __builtin_bit_cast(
                bf16x8,
                *reinterpret_cast<const u32x4*>(sa + (wm * WTM + 16 * (i + A0)) * ROWB + fo));
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          if (i + A0 < MI) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NJ - 1, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NJ, 0);
          }
          // the refill's DMA blocks go out during the first k-step's MFMAs
          if (h == 0) {
#pragma unroll
            for (int ii = (i * NB) / MI; ii < ((i + 1) * NB) / MI; ++ii)
              issue_block(ii, da, ka, ra, db, kb, rb);
          }
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
};

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;


typedef __attribute__((ext_vector_type(16))) float f32x16;

// C[BM x BN] += A[BM x K] * B[K x BN] with A K-contiguous (element (r, k) at
// A[r * lda + k]) and B K-major (element (k, n) at B[k * ldb + n]): the
// contraction over the vocabulary, where B is W in its natural layout.
// A is staged in 64-byte rows, pieces placed by a_slot. A B stage is 32
// rows k of BN columns copied verbatim by LDS-DMA, the 16-byte pieces of row
// k permuted by XOR with bswz(k), which spreads the transposing reads below
// over all banks. B fragments come from
// ds_read_b64_tr_b16: inside a 16-lane group, lane i returns element i % 4 of
// what source lanes i / 4 + 4 j (j = 0..3) point at, so source lane s points
// at row k0 + s / 4, columns n0 + 4 (s % 4) .. + 3, and lane i receives
// B[k0 + j][n0 + i], j = 0..3; two reads make a fragment of 8 k.
//
// M32 selects the MFMA: false = v_mfma_f32_16x16x32_bf16 (accumulator layout
// as AsyncGemmP); true = v_mfma_f32_32x32x16_bf16, two per 32-k stage, which
// one wave per SIMD issues at the full matrix-core rate (the 16x16x32 form
// needs two waves per SIMD for that): acc[i][j][e] is element
// (row wm*WTM + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, col wn*WTN + 32 j + lane % 32),
// the A fragment of k16-step q is row lane % 32, k 16 q + 8 (lane / 32) .. + 7,
// and the B fragment column lane % 32, the same k.
// k runs over [k_begin, k_end) in ascending steps of 32 (in two MFMA steps
// of 16 each with M32); the span must be a multiple of 32 and every valid
// row of A must hold k_end elements. Rows of B at or past kb_valid, and
// columns at or past nb_valid in its last valid row, read as zero; other
// columns past nb_valid read whatever follows in memory and only reach output
// columns the caller discards.
template <int BM, int BN, int WM, int WN, int NSTG = 4, bool M32 = false>
struct AsyncGemmKN {
  static constexpr int NW = WM * WN;
  static_assert(NW == 4, "4 waves per workgroup");
  static_assert(BN == 128 || BN == 256, "B rows of 256 or 512 bytes");
  static constexpr int FR = M32 ? 32 : 16;  // rows / columns of one MFMA block
  static_assert(BM % FR == 0, "whole A blocks");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / FR, NJ = WTN / FR;
  static_assert(MI >= 1 && NJ >= 1 && WTM % FR == 0 && WTN % FR == 0, "whole MFMA blocks per wave");
  static constexpr int NST = NSTG;
  static_assert(NST == 3 || NST == 4, "3- or 4-slot ring");
  static constexpr int ROWB_A = 64;
  static constexpr int ROWB_B = BN * 2;
  static constexpr int PPR = BN / 8;    // 16-byte pieces per B row
  static constexpr int RPB = 64 / PPR;  // B rows per 1 KB DMA block
  static constexpr int STAGE_A = BM * ROWB_A;
  static constexpr int STAGE_B = 32 * ROWB_B;
  static constexpr int STAGE_BYTES = STAGE_A + STAGE_B;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static constexpr int NI_A = STAGE_A / 1024, NI_B = STAGE_B / 1024;
  static constexpr int NI = NI_A + NI_B;
  static constexpr int NI_W_MAX = (NI + NW - 1) / NW;
  static constexpr int NI_W_MIN = NI / NW;
  static constexpr int KSUB = M32 ? 2 : 1;  // MFMA steps per 32-k stage
  typedef typename std::conditional<M32, f32x16, f32x4>::type acc_t;
  static constexpr int ACC_N = M32 ? 16 : 4;

  acc_t acc[MI][NJ];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < ACC_N; ++e) acc[i][j][e] = 0.f;
  }

  // Piece placements, measured with the LDS bank-conflict counter (cycles
  // per read, 0 = none). B (K-major, transposing reads): piece p of row k at
  // p ^ bswz(k); the 16x16x32 reads (rows k0 + 8 g + 0..3) take
  // 2 (k % 4) + 8 ((k / 8) % 2): 0; the 32x32x16 reads (rows k0 + 0..3 and
  // k0 + 8..11, two 32-byte column groups) take 4 (k % 4): 0, where the
  // 16x16 placement costs 2. A (64-byte rows, 16-byte reads): the 16-row
  // reads take row_slot (rotation by r / 2): 0; the 32-row reads take a
  // rotation by r / 4: 0, where row_slot costs 4.
  static __device__ __forceinline__ int bswz(int k) {
    return M32 ? 4 * (k & 3) : 2 * (k & 3) + 8 * ((k >> 3) & 1);
  }
  static __device__ __forceinline__ int a_slot(int c, int r) {
    return M32 ? (c + (r >> 2)) & 3 : row_slot(c, r);
  }
  static __device__ __forceinline__ int a_piece(int s, int r) {
    return M32 ? (s - (r >> 2)) & 3 : row_piece(s, r);
  }

  static __device__ __forceinline__ acc_t mfma(const bf16x8& a, const bf16x8& b, const acc_t& c) {
    if constexpr (M32)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }

  __device__ __forceinline__ void run(unsigned char* lds, const uint16_t* A, int64_t lda,
                                      int a_rows, const uint16_t* B, int64_t ldb, int kb_valid,
                                      int nb_valid, int k_begin, int k_end) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wm = wave % WM, wn = wave / WM;
    const int nsteps = (k_end - k_begin) / 32;
    if (nsteps <= 0) return;
    const int ar = a_rows < 0 ? 0 : (a_rows > BM ? BM : a_rows);
    const i32x4 rsA_all = make_rsrc(A, (uint32_t)(ar * lda * 2));
    const uint32_t lds0 = lds_addr(lds);

    const int drow = lane >> 2;
    const int dpiece = a_piece(lane & 3, lane >> 2);
    const int brow = lane / PPR, bslot = lane % PPR;
    int voff[NI_W_MAX];
#pragma unroll
    for (int ii = 0; ii < NI_W_MAX; ++ii) {
      const int j = wave + NW * ii;
      if (j < NI_A) {
        voff[ii] = (int)((16 * j + drow) * lda * 2) + 16 * dpiece;
      } else {
        const int k = RPB * (j - NI_A) + brow;
        voff[ii] = (int)(k * ldb * 2) + 16 * (bslot ^ bswz(k));
      }
    }

    auto issue = [&](int s) {
      const uint32_t st = lds0 + (uint32_t)((s % NST) * STAGE_BYTES);
      const int k0 = k_begin + 32 * s;
      int brows = kb_valid - k0;
      brows = brows < 0 ? 0 : (brows > 32 ? 32 : brows);
      // the resource ends at column nb_valid of the stage's last valid row
      const uint32_t bbytes = brows > 0 ? (uint32_t)(((brows - 1) * ldb + nb_valid) * 2) : 0u;
      const i32x4 rsB = make_rsrc(B + (int64_t)k0 * ldb, bbytes);
      // a stage past the last (padded issue below) reads through empty
      // resources: A's k offset travels in the scalar offset, which the
      // range check does not cover, so A's resource is emptied too
      const i32x4 rsA = s < nsteps ? rsA_all : make_rsrc(A, 0u);
      if constexpr (NI_A % NW == 0 && NI % NW == 0) {
        // block wave + NW ii is an A block iff ii < NI_A / NW (known at compile time)
#pragma unroll
        for (int ii = 0; ii < NI / NW; ++ii) {
          if (ii < NI_A / NW)
            dma16<true>(rsA, st + (wave + NW * ii) * 1024, voff[ii], k0 * 2);
          else
            dma16<true>(rsB, st + (wave + NW * ii) * 1024, voff[ii], 0);
        }
      } else {
#pragma unroll
        for (int ii = 0; ii < NI_W_MAX; ++ii) {
          const int j = wave + NW * ii;
          if (j < NI) {
            if (j < NI_A)
              dma16<true>(rsA, st + j * 1024, voff[ii], k0 * 2);
            else
              dma16<true>(rsB, st + j * 1024, voff[ii], 0);
          }
        }
      }
    };

    // A fragment offsets (MFMA step q of a stage): row lane % FR of the
    // block, logical piece lane / 16 (16x16x32) or 2 q + lane / 32 (32x32x16)
    uint32_t foff[KSUB];
#pragma unroll
    for (int q = 0; q < KSUB; ++q) {
      const int r = lane % FR;
      const int c = M32 ? 2 * q + (lane >> 5) : (lane >> 4);
      foff[q] = (uint32_t)(r * ROWB_A + 16 * a_slot(c, r));
    }
    // transposing reads: 16-lane group g, source lane sl; read t of MFMA step
    // q covers rows k0 + 4 t + sl / 4 at columns n0 + 4 (sl % 4) .. + 3, with
    // (16x16x32) k0 = 8 g, n0 = the block's column; (32x32x16) k0 = 16 q +
    // 8 (g / 2), n0 = the block's column + 16 (g % 2)
    const int g = lane >> 4, sl = lane & 15;
    uint32_t boff[KSUB][2][NJ];
#pragma unroll
    for (int q = 0; q < KSUB; ++q)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int k = (M32 ? 16 * q + 8 * (g >> 1) : 8 * g) + 4 * t + (sl >> 2);
          const int col = wn * WTN + FR * j + (M32 ? 16 * (g & 1) : 0) + 4 * (sl & 3);
          boff[q][t][j] =
              (uint32_t)(STAGE_A + k * ROWB_B + 16 * ((col >> 3) ^ bswz(k)) + 2 * (col & 7));
        }


    // The DMA blocks of the stage being refilled go out one per MFMA row
    // block when they divide evenly (which operand each is: compile time).
    constexpr bool SPLIT = NI_A % NW == 0 && NI % NW == 0 && NI / NW <= MI * KSUB;
    // the first block of each operand in a stage settles the descriptor's
    // SGPRs (the compiler reads them back from VGPRs once per stage)
    auto issue_block = [&](int ii, uint32_t dst, int k0, const i32x4& rsA, const i32x4& rsB) {
      if (ii == 0)
        dma16<true>(rsA, dst, voff[0], k0 * 2);
      else if (ii < NI_A / NW)
        dma16(rsA, dst + 1024u * NW * ii, voff[ii], k0 * 2);
      else if (ii == NI_A / NW)
        dma16<true>(rsB, dst + 1024u * NW * ii, voff[ii], 0);
      else
        dma16(rsB, dst + 1024u * NW * ii, voff[ii], 0);
    };
    auto stage_rsrc_b = [&](int k0) {
      int brows = kb_valid - k0;
      brows = brows < 0 ? 0 : (brows > 32 ? 32 : brows);
      const uint32_t bbytes = brows > 0 ? (uint32_t)(((brows - 1) * ldb + nb_valid) * 2) : 0u;
      return make_rsrc(B + (int64_t)k0 * ldb, bbytes);
    };

    // a ring of NST single-k-step slots; A fragments read two row blocks ahead
    // Every step issues one stage, past the last through empty resources
    // (no memory touched, zeros into a slot no later step reads): no branch
    // sits between the MFMAs, and the wait is the constant NST - 2 stages
    // behind (a count clamped at the end takes a branch per step). Where
    // waves issue unequal block counts the wait counts the smaller, which
    // waits a little longer in the others.
    for (int s = 0; s < NST - 1; ++s) issue(s);
    for (int s = 0; s < nsteps; ++s) {
      wait_vmcnt<(NST - 2) * NI_W_MIN>();
      barrier_only();
      const bool refill = s + NST - 1 < nsteps;
      if (!SPLIT) issue(s + NST - 1);
      const int k3 = k_begin + 32 * (s + NST - 1);
      const uint32_t dst =
          lds0 + (uint32_t)(((s + NST - 1) % NST) * STAGE_BYTES) + 1024u * (uint32_t)wave;
      const i32x4 rsB3 = stage_rsrc_b(k3);
      const i32x4 rsA3 = refill ? rsA_all : make_rsrc(A, 0u);
      unsigned char* st = lds + (s % NST) * STAGE_BYTES;
      constexpr int A0 = MI < 2 ? MI : 2;
#pragma unroll
      for (int q = 0; q < KSUB; ++q) {
        bf16x8 af[MI], bfr[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const s16x4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(st + boff[q][0][j]));
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(st + boff[q][1][j]));
          bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < A0; ++i)
          af[i] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(st + (wm * WTM + FR * i) * ROWB_A + foff[q]));
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NJ + A0, 0);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (i + A0 < MI)
            af[i + A0] = __builtin_bit_cast(
                bf16x8,
                *reinterpret_cast<const u32x4*>(st + (wm * WTM + FR * (i + A0)) * ROWB_A + foff[q]));
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma(af[i], bfr[j], acc[i][j]);
          if (i + A0 < MI) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NJ - 1, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NJ, 0);
          }
          if constexpr (SPLIT) {
            if (q * MI + i < NI / NW) issue_block(q * MI + i, dst, k3, rsA3, rsB3);
          }
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
};

}  // namespace rlk

namespace rlk {

// C[BM x BN] += A^T B with both operands K-major: element (k, m) of A at
// A[k * lda + m] and element (k, n) of B at B[k * ldb + n] (e.g. dW = G^T h
// with G stored [t][v] and h stored [t][h], contracting over t). Each stage is
// 32 rows k of A (BM columns) and of B (BN columns), copied verbatim by
// LDS-DMA with the 16-byte pieces of row k permuted as in AsyncGemmKN; both
// MFMA fragments come from transposing reads (lane i of a 16-lane group
// receives rows k0..k0+3 of column n0 + i). k runs over [k_begin, k_end) in
// ascending MFMA steps of 32 (the span a multiple of 32). Rows at or past
// ka_valid / kb_valid read as zero, and so do columns at or past na_valid /
// nb_valid in the last valid row; other columns past them read what follows
// in memory and only reach outputs the caller discards. WM x WN = 4 waves,
// same accumulator layout as AsyncGemmP (rows = A columns, cols = B columns).
template <int BM, int BN, int WM, int WN, int NSTG>
struct AsyncGemmKK {
  static constexpr int NW = WM * WN;
  static_assert(NW == 4, "4 waves per workgroup");
  static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "rows of 256 or 512 bytes");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 16, NJ = WTN / 16;
  static constexpr int NST = NSTG;
  static_assert(NST >= 2 && NST <= 4, "2- to 4-slot ring");
  static constexpr int ROWB_A = BM * 2, ROWB_B = BN * 2;
  static constexpr int PPR_A = BM / 8, RPB_A = 64 / PPR_A;  // pieces per row, rows per 1 KB block
  static constexpr int PPR_B = BN / 8, RPB_B = 64 / PPR_B;
  static constexpr int STAGE_A = 32 * ROWB_A, STAGE_B = 32 * ROWB_B;
  static constexpr int STAGE_BYTES = STAGE_A + STAGE_B;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static constexpr int NI_A = STAGE_A / 1024, NI_B = STAGE_B / 1024, NI = NI_A + NI_B;
  static_assert(NI_A % NW == 0 && NI % NW == 0, "DMA blocks divide among the waves");
  static constexpr int NB = NI / NW;  // DMA blocks per wave per stage
  static_assert(NB <= MI, "one DMA block per MFMA row block");

  f32x4 acc[MI][NJ];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  static __device__ __forceinline__ int bswz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }

  // Resource over rows [k0, k0 + 32) of a K-major operand: rows at or past
  // k_valid, and columns at or past n_valid in the last valid row, read zero.
  static __device__ __forceinline__ i32x4 stage_rsrc(const uint16_t* base, int64_t ld, int k0,
                                                     int k_valid, int n_valid) {
    int rows = k_valid - k0;
    rows = rows < 0 ? 0 : (rows > 32 ? 32 : rows);
    const uint32_t bytes = rows > 0 ? (uint32_t)(((rows - 1) * ld + n_valid) * 2) : 0u;
    return make_rsrc(base + (int64_t)k0 * ld, bytes);
  }

    // PAD: every step issues one stage, past the last one through empty
  // resources (no memory touched, zeros into a slot no later step reads),
  // so no branch sits between the MFMAs and each wait is the constant
  // NST - 2 stages behind. The empty stages cost their latency once at the
  // end; with only 1-2 steps that outweighs the branches saved.
  template <bool PAD = false>
  __device__ __forceinline__ void run(unsigned char* lds, const uint16_t* A, int64_t lda,                                     int ka_valid, int na_valid, const uint16_t* B, int64_t ldb,
                                      int kb_valid, int nb_valid, int k_begin, int k_end) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wm = wave % WM, wn = wave / WM;
    const int nsteps = (k_end - k_begin) / 32;
    if (nsteps <= 0) return;
    const uint32_t lds0 = lds_addr(lds);

    // DMA: block j of a stage holds rows RPB j + lane / PPR, lane % PPR the
    // physical piece slot, loading logical piece slot ^ bswz(row)
    int voff[NB];
#pragma unroll
    for (int ii = 0; ii < NB; ++ii) {
      const int j = wave + NW * ii;
      if (ii < NI_A / NW) {
        const int k = RPB_A * j + lane / PPR_A;
        voff[ii] = (int)(k * lda * 2) + 16 * ((lane % PPR_A) ^ bswz(k));
      } else {
        const int k = RPB_B * (j - NI_A) + lane / PPR_B;
        voff[ii] = (int)(k * ldb * 2) + 16 * ((lane % PPR_B) ^ bswz(k));
      }
    }
    auto issue_block = [&](int ii, uint32_t dst, const i32x4& ra, const i32x4& rb) {
      dma16(ii < NI_A / NW ? ra : rb, dst + 1024u * NW * ii, voff[ii], 0);
    };
    auto stage_dst = [&](int s) {
      return lds0 + (uint32_t)((s % NST) * STAGE_BYTES) + 1024u * (uint32_t)wave;
    };
    auto issue = [&](int s) {
      const int k0 = k_begin + 32 * s;
      const i32x4 ra = stage_rsrc(A, lda, k0, ka_valid, na_valid);
      const i32x4 rb = stage_rsrc(B, ldb, k0, kb_valid, nb_valid);
#pragma unroll
      for (int ii = 0; ii < NB; ++ii) issue_block(ii, stage_dst(s), ra, rb);
    };

    // transposing reads: 16-lane group g, source lane sl; read q covers rows
    // 8 g + 4 q + sl / 4 at columns c0 + 4 (sl % 4) .. + 3
    const int g = lane >> 4, sl = lane & 15;
    uint32_t aoff[2][MI], boff[2][NJ];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = 8 * g + 4 * q + (sl >> 2);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int col = wm * WTM + 16 * i + 4 * (sl & 3);
        aoff[q][i] = (uint32_t)(k * ROWB_A + 16 * ((col >> 3) ^ bswz(k)) + 2 * (col & 7));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = wn * WTN + 16 * j + 4 * (sl & 3);
        boff[q][j] = (uint32_t)(STAGE_A + k * ROWB_B + 16 * ((col >> 3) ^ bswz(k)) + 2 * (col & 7));
      }
    }
    auto frag = [&](const unsigned char* st, uint32_t o0, uint32_t o1) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(st + o0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(st + o1));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto wait_stage = [&](int want, int last) {
      last = last < nsteps - 1 ? last : nsteps - 1;
      const int after = last - want;
      if (after >= 3)
        wait_vmcnt<3 * NB>();
      else if (after == 2)
        wait_vmcnt<2 * NB>();
      else if (after == 1)
        wait_vmcnt<NB>();
      else
        wait_vmcnt<0>();
    };

    for (int s = 0; s < NST - 1 && (PAD || s < nsteps); ++s) issue(s);
    for (int s = 0; s < nsteps; ++s) {
      if constexpr (PAD)
        wait_vmcnt<(NST - 2) * NB>();
      else
        wait_stage(s, s + NST - 2);
      barrier_only();
      // refill the slot of stage s-1 (every wave is past its reads) with
      // stage s+NST-1, one DMA block per MFMA row block (past the end the
      // stage's resources are empty: stage_rsrc clamps the rows to none)
      const bool refill = s + NST - 1 < nsteps;
      const int kr = k_begin + 32 * (s + NST - 1);
      const i32x4 ra = stage_rsrc(A, lda, kr, ka_valid, na_valid);
      const i32x4 rb = stage_rsrc(B, ldb, kr, kb_valid, nb_valid);
      // the slot once per step (the fragment addresses and the refill's
      // destination derive from it; computed apart, the compiler spent two
      // VALU operations on each of the step's 24 fragment addresses)
      const int slot = s % NST;
      const uint32_t dst =
          lds0 + (uint32_t)(((slot + NST - 1) % NST) * STAGE_BYTES) + 1024u * (uint32_t)wave;
      const unsigned char* st = lds + slot * STAGE_BYTES;
      constexpr int A0 = MI < 2 ? MI : 2;
      bf16x8 af[MI], bfr[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = frag(st, boff[0][j], boff[1][j]);
#pragma unroll
      for (int i = 0; i < A0; ++i) af[i] = frag(st, aoff[0][i], aoff[1][i]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (NJ + A0), 0);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (i + A0 < MI) af[i + A0] = frag(st, aoff[0][i + A0], aoff[1][i + A0]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        if (i + A0 < MI) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NJ - 1, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, NJ, 0);
        }
        if (i < NB && (PAD || refill)) issue_block(i, dst, ra, rb);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
};

}  // namespace rlk
