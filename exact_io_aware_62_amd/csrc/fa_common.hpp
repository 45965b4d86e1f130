// Device-side building blocks shared by the forward and backward kernels:
// vector types, the gfx950 bf16 matrix-core op, bf16 packing, and the
// global -> LDS tile staging used by every kernel.
//
// Matrix-core fragment layout used throughout (v_mfma_f32_32x32x16_bf16,
// one 64-lane wavefront; lane l, r = l % 32, g = l / 32):
//   A (32 x 16):  lane l holds row m = r, eight k values indexed by (g, j)
//   B (16 x 32):  lane l holds column n = r, the same eight (g, j) k values
//   C (32 x 32):  lane l, register i holds C[(i/4)*8 + g*4 + i%4][r]
// Only the C layout and "A and B agree on (g, j) -> k" are relied on, so the
// order in which a contraction visits its k index is free; the kernels use
// that freedom to feed a C fragment straight back in as a B operand.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no score seen yet" in the running maximum: keeps
// exp2(m_old - m_new) and exp2(-inf - m) free of inf - inf.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                               const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 bf16x8_from_halves(const u32x2& lo, const u32x2& hi) {
  u32x4 u;
  u[0] = lo[0];
  u[1] = lo[1];
  u[2] = hi[0];
  u[3] = hi[1];
  return __builtin_bit_cast(bf16x8, u);
}

// Eight fp32 values -> bf16x8, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Four fp32 -> four bf16 in two dwords (RNE).
__device__ __forceinline__ u32x2 pack_bf16x4(float a0, float a1, float a2, float a3) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

// ---------------------------------------------------------------------------
// Tile staging.  A tile is ROWS consecutive rows (tokens) x D columns of one
// head of a BHND tensor.  Rows at or beyond `n_valid` are filled with zeros,
// so a partial last tile never feeds stale bits (possibly NaN) to the matrix
// cores.  Two LDS layouts:
//   natural    [ROWS][D + 8]   row-major, 16-byte pad per row
//   transposed [D][ROWS + 4]   column-major copy, 8-byte pad per row
// Loads go HBM -> VGPR first (so they overlap compute of the previous tile),
// then VGPR -> LDS after the compute.
// ---------------------------------------------------------------------------

template <int ROWS, int D, int NT>
struct NaturalStage {
  static constexpr int kChunks = ROWS * D / 8;            // 16-byte chunks
  static constexpr int kPerThread = (kChunks + NT - 1) / NT;
  static constexpr int kStride = D + 8;                   // bf16 elements
  static constexpr int kElems = ROWS * kStride;
  u32x4 reg[kPerThread];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int row0,
                                       int n_valid, int tid) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      if ((kChunks % NT == 0 || c < kChunks) && row0 + row < n_valid)
        reg[i] = ldg16(src + (size_t)(row0 + row) * D + col);
      else
        reg[i] = zero_u32x4();
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks) {
        const int row = c / (D / 8);
        const int col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(lds + row * kStride + col) = reg[i];
      }
    }
  }
};

// Transposed staging: a unit is 4 rows x 8 columns; the thread loads the
// four 16-byte row pieces and writes eight 8-byte column pieces.
template <int ROWS, int D, int NT>
struct TransposedStage {
  static constexpr int kUnits = (ROWS / 4) * (D / 8);
  static constexpr int kPerThread = (kUnits + NT - 1) / NT;
  static constexpr int kStride = ROWS + 4;                // bf16 elements
  static constexpr int kElems = D * kStride;
  u32x4 reg[kPerThread][4];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int row0,
                                       int n_valid, int tid) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int u = tid + i * NT;
      const int rg = u / (D / 8);
      const int col = (u % (D / 8)) * 8;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = rg * 4 + rr;
        if ((kUnits % NT == 0 || u < kUnits) && row0 + row < n_valid)
          reg[i][rr] = ldg16(src + (size_t)(row0 + row) * D + col);
        else
          reg[i][rr] = zero_u32x4();
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int u = tid + i * NT;
      if (kUnits % NT == 0 || u < kUnits) {
        const int rg = u / (D / 8);
        const int col = (u % (D / 8)) * 8;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          // columns col + 2p (low halves) and col + 2p + 1 (high halves)
          const uint32_t a = reg[i][0][p], b = reg[i][1][p];
          const uint32_t c = reg[i][2][p], e = reg[i][3][p];
          u32x2 lo, hi;
          lo[0] = (a & 0xffffu) | (b << 16);
          lo[1] = (c & 0xffffu) | (e << 16);
          hi[0] = (a >> 16) | (b & 0xffff0000u);
          hi[1] = (c >> 16) | (e & 0xffff0000u);
          *reinterpret_cast<u32x2*>(lds + (col + 2 * p) * kStride + rg * 4) = lo;
          *reinterpret_cast<u32x2*>(lds + (col + 2 * p + 1) * kStride + rg * 4) = hi;
        }
      }
    }
  }
};

// Fragment reads from staged tiles.
// A/B operand from a natural tile: row `row`, eight consecutive columns at col.
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* lds, int stride, int row, int col) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(lds + row * stride + col));
}

// A/B operand from a transposed tile over the contraction index: row `row`
// (the free index), contraction positions c0..c0+3 and c1..c1+3.
__device__ __forceinline__ bf16x8 lds_tr8(const uint16_t* lds, int stride, int row, int c0,
                                          int c1) {
  const u32x2 lo = *reinterpret_cast<const u32x2*>(lds + row * stride + c0);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(lds + row * stride + c1);
  return bf16x8_from_halves(lo, hi);
}

// Block index -> (query/key block, batch*head).  Consecutive block ids are
// spread round-robin over the 8 XCDs, so with bid = blk * BH + bh every
// block of one head lands on the same XCD (bh % 8) whenever BH % 8 == 0 and
// they share that XCD's L2 for K and V.
struct BlockCoord {
  int blk;
  int bh;
};

__device__ __forceinline__ BlockCoord block_coord(int BH) {
  BlockCoord c;
  c.bh = blockIdx.x % BH;
  c.blk = blockIdx.x / BH;
  return c;
}

}  // namespace fa
