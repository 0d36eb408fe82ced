// rlk_device.cuh — device building blocks for the gfx950 linear log-prob kernels.
//
// * An LDS-tiled bf16 MFMA mainloop (v_mfma_f32_16x16x32_bf16) that computes
//   a BM x BN fp32 tile of A * B^T with K walked in ascending blocks of 32.
//   Either operand may be stored K-contiguous ("row-major [rows][K]") or
//   K-strided ("row-major [K][rows]"); K-strided operands are transposed in
//   registers (8x8 blocks) on their way into LDS so that every MFMA fragment
//   is one 16-byte LDS read.
// * The fixed-order reductions that make every output row independent of the
//   batch: a 16-lane DPP tree, the (m, R, B, zy) merge algebra, bf16 RNE.
//
// Every kernel that produces the same quantity goes through these helpers,
// so the per-element arithmetic, and hence the bits, are identical whatever
// the tile shape or grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kThreads = 256;  // 4 wave64 per workgroup
constexpr int BK = 64;         // K extent of one LDS stage
constexpr int LDK = BK + 8;    // padded LDS row, in bf16 elements (144 B): conflict-free
                               // 16-byte fragment reads for 16 consecutive rows
constexpr int GROUP = 256;     // vocabulary columns per group (one forward tile width)
constexpr int CHUNK = 32;      // vocabulary columns per chunk (unit of the row statistics)
constexpr int CHUNKS_PER_GROUP = GROUP / CHUNK;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// ---------------------------------------------------------------- bf16 --

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

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
// An empty side (m = -inf) contributes nothing. Accurate expf; contraction is
// disabled for the whole library, so the arithmetic is exactly as written.
__device__ __forceinline__ Part part_merge(const Part& l, const Part& r) {
  const bool left_base = !(r.m > l.m);
  const Part& b = left_base ? l : r;
  const Part& o = left_base ? r : l;
  Part out;
  out.m = b.m;
  out.zy = fmaxf(l.zy, r.zy);
  if (o.m == neg_inf()) {
    out.R = b.R;
    out.B = b.B;
    return out;
  }
  const float d = o.m - b.m;
  const float e = expf(d);
  const float one_r = 1.f + o.R;
  out.R = b.R + e * one_r;
  out.B = b.B + e * (o.B + one_r * d);
  return out;
}

// ------------------------------------------------------ global loads ----

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void sts16(uint16_t* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// One operand tile of ROWS rows x BK of K, staged global -> registers -> LDS.
//   TRANS == false: element (r, k) at src[r * ld + k]  (K contiguous).
//     Thread t moves the 16-byte piece (k = 8 (t % 8)) of rows t / 8 + 32 i.
//   TRANS == true:  element (r, k) at src[k * ld + r]  (rows contiguous).
//     Thread t moves the 8 x 8 block (k = 8 (t % 8) + 0..7, r = 8 (t / 8 + 32 i) + 0..7),
//     transposing it in registers.
// Rows >= rows_valid and k >= k_valid read as zero. For TRANS the row test is
// per 8-row block (rows_valid must be a multiple of 8); for !TRANS the k test
// is per 8-element piece (k_valid must be a multiple of 8).
template <int ROWS, bool TRANS>
struct OperandTile {
  static_assert(ROWS % 32 == 0, "tile rows must be a multiple of 32");
  static constexpr int NPIECE = TRANS ? 0 : ROWS * BK / 8 / kThreads;  // 16-B pieces per thread
  static constexpr int NBLK = TRANS ? (ROWS / 8 * BK / 8 + kThreads - 1) / kThreads : 0;
  static constexpr int NREG = TRANS ? NBLK * 8 : NPIECE;
  u32x4 reg[NREG > 0 ? NREG : 1];

  __device__ __forceinline__ void load(const uint16_t* src, int64_t ld, int rows_valid, int k0,
                                       int k_valid, int tid) {
    if constexpr (!TRANS) {
      const int c = tid & 7;
      const int k = k0 + 8 * c;
#pragma unroll
      for (int i = 0; i < NPIECE; ++i) {
        const int r = (tid >> 3) + 32 * i;
        if (r < rows_valid && k < k_valid)
          reg[i] = ldg16(src + (int64_t)r * ld + k);
        else
          reg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      const int kb = tid & 7;
#pragma unroll
      for (int bi = 0; bi < NBLK; ++bi) {
        const int rb = (tid >> 3) + 32 * bi;
        const bool rows_ok = (rb < ROWS / 8) && (8 * rb + 8 <= rows_valid);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + 8 * kb + j;
          if (rows_ok && k < k_valid)
            reg[bi * 8 + j] = ldg16(src + (int64_t)k * ld + 8 * rb);
          else
            reg[bi * 8 + j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  // Write the registers into an LDS stage laid out [ROWS][LDK] (K contiguous).
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    if constexpr (!TRANS) {
      const int c = tid & 7;
#pragma unroll
      for (int i = 0; i < NPIECE; ++i) {
        const int r = (tid >> 3) + 32 * i;
        sts16(lds + r * LDK + 8 * c, reg[i]);
      }
    } else {
      const int kb = tid & 7;
#pragma unroll
      for (int bi = 0; bi < NBLK; ++bi) {
        const int rb = (tid >> 3) + 32 * bi;
        if (rb >= ROWS / 8) continue;
        // in[j] holds rows 8rb..8rb+7 at k = 8kb + j (two rows per dword);
        // out[q] holds k = 8kb..8kb+7 at row 8rb + q (two k per dword).
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          u32x4 o;
          const int dw = q >> 1;
          const int sh = (q & 1) * 16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (reg[bi * 8 + 2 * e][dw] >> sh) & 0xffffu;
            const uint32_t hi = (reg[bi * 8 + 2 * e + 1][dw] >> sh) & 0xffffu;
            o[e] = lo | (hi << 16);
          }
          sts16(lds + (8 * rb + q) * LDK + 8 * kb, o);
        }
      }
    }
  }
};

// C[BM x BN] (fp32, in registers) += A[BM x K] * B[BN x K]^T over k in
// [k_begin, k_end), in ascending MFMA steps of 32 starting at k_begin. Waves
// form a WM x WN grid; wave (wm, wn) owns rows wm*WTM.. and cols wn*WTN.. of
// the tile. Accumulator layout (16x16 MFMA): acc[i][j][r] is element
//   row = wm*WTM + 16 i + 4 (lane / 16) + r,   col = wn*WTN + 16 j + lane % 16.
template <int BM, int BN, int WM, int WN, bool AT, bool BT>
struct TileGemm {
  static_assert(WM * WN == 4, "4 waves per workgroup");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 16, NJ = WTN / 16;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static constexpr int STAGE = (BM + BN) * LDK;        // bf16 elements per LDS stage
  static constexpr int LDS_BYTES = 2 * STAGE * 2;      // two stages

  f32x4 acc[MI][NJ];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  __device__ __forceinline__ void compute_stage(const uint16_t* As, const uint16_t* Bs, int wm,
                                                int wn, int lane) {
    const int fr = lane & 15;
    const int fk = 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      bf16x8 af[MI], bfr[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = lds_frag(As + (wm * WTM + 16 * i + fr) * LDK + kk * 32 + fk);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = lds_frag(Bs + (wn * WTN + 16 * j + fr) * LDK + kk * 32 + fk);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // A: base of the tile's row 0 (layout per AT), lda; a_rows valid rows.
  // B: likewise. k is absolute: element k of the K-contiguous layout sits at
  // column k, of the K-strided layout at row k.
  __device__ __forceinline__ void run(uint16_t* lds, const uint16_t* A, int64_t lda, int a_rows,
                                      const uint16_t* B, int64_t ldb, int b_rows, int k_begin,
                                      int k_end) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    OperandTile<BM, AT> ta;
    OperandTile<BN, BT> tb;
    const int nsteps = (k_end - k_begin + BK - 1) / BK;
    if (nsteps <= 0) return;
    ta.load(A, lda, a_rows, k_begin, k_end, tid);
    tb.load(B, ldb, b_rows, k_begin, k_end, tid);
    ta.store(lds, tid);
    tb.store(lds + BM * LDK, tid);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      uint16_t* cur = lds + (s & 1) * STAGE;
      uint16_t* nxt = lds + ((s + 1) & 1) * STAGE;
      const bool more = s + 1 < nsteps;
      if (more) {
        ta.load(A, lda, a_rows, k_begin + (s + 1) * BK, k_end, tid);
        tb.load(B, ldb, b_rows, k_begin + (s + 1) * BK, k_end, tid);
      }
      compute_stage(cur, cur + BM * LDK, wm, wn, lane);
      if (more) {
        ta.store(nxt, tid);
        tb.store(nxt + BM * LDK, tid);
      }
      __syncthreads();
    }
  }
};

}  // namespace rlk
