// Device-side building blocks shared by the forward and backward kernels:
// vector types, the gfx950 bf16 matrix-core op, bf16 packing, and the LDS
// tile format with its HBM -> LDS copy and operand reads.
//
// Matrix-core fragment layout used throughout (v_mfma_f32_32x32x16_bf16,
// one 64-lane wavefront; lane l, r = l % 32, g = l / 32):
//   A (32 x 16):  lane l holds row m = r, eight k values indexed by (g, j)
//   B (16 x 32):  lane l holds column n = r, the same eight (g, j) k values
//   C (32 x 32):  lane l, register i holds C[(i/4)*8 + g*4 + i%4][r]
// Only the C layout and "A and B agree on (g, j) -> k" are relied on, so the
// order in which a contraction visits its k index is free.  The kernels use
// that freedom to feed a C fragment straight back in as a B operand: for
// k-step s of a 32-wide C block, registers 8s .. 8s+7 of lane group g hold
// C rows (2s + j/4)*8 + g*4 + j%4, j = 0..7, and the A operand is gathered
// in exactly that row order (see lds_tr_operand).

#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

// Lambdas that capture by reference must be inlined: an out-of-line call
// would place every captured variable in scratch memory.
#define FA_INLINE __attribute__((always_inline))

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource on gfx9-family GPUs: 32-bit data format,
// no swizzle; the range check then compares each lane's byte offset with
// the resource's num_records.
constexpr int kBufferWord3 = 0x00020000;
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

// Eight consecutive registers of a C fragment -> bf16x8 B operand.
__device__ __forceinline__ bf16x8 pack_c8(const f32x16& c, int base) {
  return pack_bf16x8(c[base + 0], c[base + 1], c[base + 2], c[base + 3], c[base + 4],
                     c[base + 5], c[base + 6], c[base + 7]);
}

// Four fp32 -> four bf16 in two dwords (RNE).
__device__ __forceinline__ u32x2 pack_bf16x4(float a0, float a1, float a2, float a3) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  return __builtin_bit_cast(u32x2, r);
}

// This lane's index in its wavefront, recomputed where it is used (two
// vector ops; asm so the compiler neither hoists nor keeps it in a register).
__device__ __forceinline__ int lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds; each multiplies counter words 0 and 2
// by two odd constants and mixes the high and low halves of the products with
// words 1 and 3 and the round key, which advances by two Weyl constants per
// round.  The key words are wavefront-uniform in every use here, so the key
// schedule runs on the scalar unit.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input XOR in one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  u32x4 out;
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
  return out;
}

// Dropout stream of one head.  One Philox draw, on the counter
// (j / 4, i / 2, bh, offset), decides the block of queries i = 2 ig, 2 ig + 1 and
// keys j = 4 jg .. 4 jg + 3: element e = 4 (i % 2) + j % 4 of the block takes the
// 16-bit half e % 2 (low half first) of output word e / 2, and is kept iff that
// value is >= thresh (floor(p 2^16)).  keep8 returns the block's keep bits, bit e
// for element e: bits 0..3 are query 2 ig, bits 4..7 query 2 ig + 1.
struct DropoutStream {
  uint32_t seed_lo, seed_hi, bh, offset, thresh;
  __device__ __forceinline__ uint32_t keep8(uint32_t jg, uint32_t ig) const {
    const u32x4 w = philox4x32_10(jg, ig, bh, offset, seed_lo, seed_hi);
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
      bits |= (uint32_t)(h >= thresh) << e;
    }
    return bits;
  }
};

// The keep rule on a packed pair: for each 16-bit half h of a Philox output
// word w, 0xFFFF if h >= thresh (kept) and 0 otherwise (thresh = 0 keeps
// everything).  Three packed 16-bit instructions: the saturating difference
// thresh - h (0 exactly when kept), its minimum with 1, and that minus 1.
// ANDed with a packed bf16 pair it zeroes the dropped entries.  tt holds
// thresh in both halves, ones 0x00010001.  Written as asm: the compiler turns
// the same expression into two compares, two selects and a byte permute.
__device__ __forceinline__ uint32_t drop_mask(uint32_t w, uint32_t tt, uint32_t ones) {
  uint32_t d, m, r;
  asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "s"(tt), "v"(w));
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(m) : "v"(d), "s"(ones));
  asm("v_pk_sub_u16 %0, %1, %2" : "=v"(r) : "v"(m), "s"(ones));
  return r;
}

// Value of lane l ^ 1 (DPP quad permute 1, 0, 3, 2).
__device__ __forceinline__ uint32_t pair_swap(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 1 | (0 << 2) | (3 << 4) | (2 << 6), 0xF, 0xF,
                                            false);
}

// Value of lane t (0..3) of this lane's group of four (DPP quad permute).
template <int T>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, T | (T << 2) | (T << 4) | (T << 6), 0xF,
                                            0xF, false);
}

// f(std::integral_constant<int, I>{}) for I = B .. E-1, in order, each call
// with a compile-time index (a loop the compiler cannot fail to unroll).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Keeps the computation of x at this point of the program.  An empty asm
// statement with side effects takes x in registers and hands it back, so the
// compiler can neither sink the work that produced x into a later basic
// block (next to its first real use) nor move it across a neighbouring
// scheduling barrier.  Costs no instruction.
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Two- and three-input maxima as single v_max_f32 / v_max3_f32.  fmaxf on
// values the compiler cannot prove canonical (matrix-core results, lane
// exchanges) first canonicalises each input, one more instruction per input,
// and it may regroup a tree of fmaxf; none of these values is a signalling NaN.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max over lanes l and l ^ 32 (the two halves of a wavefront), without LDS:
// v_permlane32_swap exchanges the upper half of one operand with the lower
// half of the other, so the two results are {x[l], x[l ^ 32]} in some order.
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

// Wait for every outstanding vector-memory operation.  The asm form also
// covers copies issued as asm; the builtin tells the compiler's wait-count
// tracking that nothing is outstanding any more (vmcnt 0, expcnt and lgkmcnt
// left at their "don't wait" maxima).
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Per-lane byte offsets of a tile copy, one per copy segment of a wavefront.
template <int NSEG>
struct LaneOffsets {
  int v[NSEG];
};

// ---------------------------------------------------------------------------
// LDS tile: ROWS x D bf16 (one head, consecutive tokens), row-major with no
// padding; the sixteen-byte chunks of each row are XOR-permuted so that the
// two access patterns the kernels use are free of bank conflicts:
//   * operand rows: 16 lanes read the same chunk of 16 consecutive rows;
//   * transposed operands: 16 lanes read two chunks of 4 consecutive rows.
// The copy from HBM uses global_load_lds_dwordx4: each wavefront instruction
// writes 64 x 16 contiguous bytes of LDS, lane l at byte 16*l, so lane l
// fetches whichever logical chunk lives at that physical position.  Rows at
// or past `n_valid` lie beyond the buffer resource's size, so the hardware
// range check returns zeros for them: finite values, which matters because a
// masked probability of 0 times such a row must stay 0 in the P V product
// (0 * inf or 0 * NaN would not).
// ---------------------------------------------------------------------------
// D = 32 serves rows of 64 one-byte values (the FP8 kernel at head dim 64):
// only the byte size of a row matters to the layout.
template <int ROWS, int D>
struct LdsTile {
  static_assert(D == 32 || D == 64 || D == 128, "row size");
  static constexpr int kRows = ROWS;
  static constexpr int kD = D;
  static constexpr int kCPR = D / 8;                 // chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = ROWS * kRowBytes;
  static constexpr int kSegs = ROWS * kCPR / 64;     // 1 KB copy segments

  __device__ static __forceinline__ int swz(int row) {
    if constexpr (D == 128)
      return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (D == 64)
      return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else
      return (row >> 2) & 3;   // four chunks per row
  }
  // byte offset of logical 16-byte chunk `chunk` of row `row`
  __device__ static __forceinline__ int off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }

  // Per-lane part of the copy: byte offset of the 16 bytes that lane `lane`
  // of wavefront `wave` fetches for copy segment i, relative to the tile's
  // first row.  Loop-invariant, so a kernel computes it once.
  template <int NW>
  __device__ static __forceinline__ LaneOffsets<kSegs / NW> lane_offsets(int wave, int lane) {
    static_assert(kSegs % NW == 0, "segments per wavefront");
    LaneOffsets<kSegs / NW> o;
#pragma unroll
    for (int i = 0; i < kSegs / NW; ++i) {
      const int P = (wave + i * NW) * 64 + lane;
      const int row = P / kCPR;
      o.v[i] = row * kRowBytes + (((P % kCPR) ^ swz(row)) << 4);
    }
    return o;
  }

  // The NW wavefronts of a workgroup copy rows [row0, row0 + ROWS) of `src`
  // (row stride D, rows valid below n_valid) into `lds`, with buffer loads
  // that write LDS directly.  The buffer resource spans only the valid rows
  // of the tile, so the hardware range check turns rows at or past n_valid
  // into zeros (finite values; every kernel masks those rows).  Asynchronous:
  // wait_vmem() + a barrier before the data is read.
  template <int NW>
  __device__ static __forceinline__ void copy(const uint16_t* __restrict__ src, int row0,
                                              int n_valid, char* lds, int wave,
                                              const LaneOffsets<kSegs / NW>& o) {
#if defined(__HIP_DEVICE_COMPILE__)   // the buffer builtins exist only for the GPU target
    const int rows = min(n_valid - row0, ROWS);
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src + (size_t)row0 * D), (short)0, rows * kRowBytes, kBufferWord3);
#pragma unroll
    for (int i = 0; i < kSegs / NW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (wave + i * NW) * 1024),
                                               16, o.v[i], 0, 0, 0);
#endif
  }
};

// LDS address (32-bit offset in the LDS aperture) of a __shared__ object.
__device__ __forceinline__ int lds_addr(const void* p) {
  return (int)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// Copy of rows [row0, row0 + ROWS) of `src` into the LDS tile at LDS address
// `dst` (see LdsTile::copy), issued as asm.  The compiler then sees no LDS
// write, so it neither makes later LDS reads wait for the copy nor needs to
// know which buffer a read touches: that lets a kernel pick its LDS stage at
// run time.  The caller must wait_vmem() and pass a barrier before any
// wavefront reads the tile (as it has to anyway for the other wavefronts'
// parts).  M0 is saved and restored around the copies.
template <class T, int NW>
__device__ __forceinline__ void copy_async(const uint16_t* __restrict__ src, int row0, int n_valid,
                                           int dst, int wave, const LaneOffsets<T::kSegs / NW>& o) {
  const int rows = min(n_valid - row0, T::kRows);
  const unsigned long long a = (unsigned long long)(src + (size_t)row0 * T::kD);
  u32x4 rs;
  rs[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  rs[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);   // stride 0
  rs[2] = __builtin_amdgcn_readfirstlane((unsigned)(rows * T::kRowBytes));
  rs[3] = (unsigned)kBufferWord3;
#pragma unroll
  for (int i = 0; i < T::kSegs / NW; ++i) {
    const int seg = __builtin_amdgcn_readfirstlane(dst + (wave + i * NW) * 1024);
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(o.v[i]), "s"(rs), "s"(seg)
        : "memory");
  }
}

// Operand read, contraction over the tile's columns: row `row`, logical chunk
// `chunk` (eight consecutive columns) -> bf16x8.
template <class T>
__device__ __forceinline__ bf16x8 lds_row_operand(const char* lds, int row, int chunk) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(lds + T::off(row, chunk)));
}

// Transposed operand read, contraction over the tile's rows.  Returns, for
// lane l (r = l % 32, g = l / 32), the eight values
//   tile[k0 + (j/4)*8 + g*4 + j%4][col0 + r],  j = 0..7
// which is the A operand whose (g, j) -> k order matches a C fragment's
// registers 8s..8s+7 (rows (2s + j/4)*8 + g*4 + j%4 of the C block, with
// k0 = 16 s + block offset).  Uses ds_read_b64_tr_b16: within each 16-lane
// group, lane i receives element i%4 of the 8-byte pieces addressed by lanes
// 4e + i/4 (e = 0..3), so lanes addressing rows k0+4g+(s/4), columns
// col0 + 16*((l/16)%2) + 4*(s%4) (s = l % 16) deliver a 4 x 16 transpose.
template <class T>
__device__ __forceinline__ int tr_offset(int k0, int col0, int lane, int half) {
  const int s = lane & 15, gi = (lane >> 4) & 1, g = lane >> 5;
  const int row = k0 + half * 8 + g * 4 + (s >> 2);
  const int col = col0 + 16 * gi + 4 * (s & 3);
  return T::off(row, col >> 3) + ((col & 7) << 1);
}

__device__ __forceinline__ u32x2 lds_tr_b64(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}
// Reads at LDS byte address a + off, with off a compile-time constant that
// goes into the instruction's offset field: the transpose read above, and a
// plain 16-byte read.
__device__ __forceinline__ u32x2 lds_tr_b64_at(int a, int off) {
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* p = reinterpret_cast<lds_char*>((size_t)(uint32_t)a) + off;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x4 lds_read_b128_at(int a, int off) {
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_char* p = reinterpret_cast<lds_char*>((size_t)(uint32_t)a) + off;
  const u32x4 v = *reinterpret_cast<lds_u32x4*>(p);
  return v;
}

// (a ^ b) + c in one v_xad_u32.  Written as asm so that loop-invariant
// address arithmetic is recomputed where it is used instead of being hoisted
// into long-lived registers (which a kernel near its register limit would
// spill, and a spill reload waits for every earlier vector-memory load).
__device__ __forceinline__ int xad(int a, int b, int c) {
  int d;
  asm volatile("v_xad_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
  return d;
}

// Lane-dependent parts of the two operand reads of a swizzled tile T, such
// that (with k-step kk and 32-column block db of the tile):
//   row read  lds_row_operand<T>(base, r, 2*kk + g) == base + xad(xr, kk << 5, ar)
//   tr read   tr_offset<T>(0, db*32, lane, half)    == xad(xt, db << 6, at[half])
// The XOR swizzle only permutes chunks inside a row, and its bits above the
// two lowest chunk bits do not depend on the tr-read half, which is what
// makes both forms exact (checked against the direct formulas on the host).
template <class T>
struct OperandAddr {
  int ar, xr;        // row read
  int at0, at1, xt;  // transposed read, halves 0 and 1
};

template <class T>
__device__ __forceinline__ OperandAddr<T> operand_addr(int lane) {
  OperandAddr<T> o;
  const int r = lane & 31, g = lane >> 5;
  o.ar = r * T::kRowBytes;
  o.xr = (g ^ T::swz(r)) << 4;
  const int s = lane & 15, gi = (lane >> 4) & 1;
  const int lo = 2 * gi + ((s & 3) >> 1);
  int at[2], xt = 0;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = half * 8 + g * 4 + (s >> 2);
    const int sw = T::swz(row);
    at[half] = row * T::kRowBytes + ((lo ^ (sw & 3)) << 4) + ((s & 1) << 3);
    xt = (sw & ~3) << 4;
  }
  o.at0 = at[0];
  o.at1 = at[1];
  o.xt = xt;
  return o;
}

// Writes a wavefront's 32 output rows of D bf16 values, held in the 32x32
// accumulator layout (lane r + 32 g holds row r; register qd*4 + e of column
// block db is column db*32 + qd*8 + g*4 + e), times `mul`, to rows
// dst[0 .. valid) of a row-major global array with row stride D.
//
// Written straight from that layout, one store instruction touches 32 rows
// with 16 bytes each.  Instead the values go through `stage`, an LDS area of
// 32 * 2D bytes that only this wavefront uses: each lane writes its 8-byte
// pieces, then reads back 16 consecutive bytes of one row, so that a store
// instruction covers 64 / (D/8) whole consecutive rows.  The 16-byte chunks
// of a staged row are XOR-swizzled by the index of the row's 256-byte bank
// line (the row itself at D = 128, row / 2 at D = 64, where two rows share
// the 64 banks), which spreads both the writes and the row reads over all
// LDS banks.  The caller guarantees that no
// other wavefront touches `stage` meanwhile and that no copy into it is
// outstanding.
template <int D>
__device__ __forceinline__ void store_rows_staged(char* stage, const f32x16 (&acc)[D / 32],
                                                  float mul, uint16_t* dst, int valid, int lane) {
  constexpr int NDB = D / 32, CPR = D / 8, RB = 2 * D, RPI = 64 / CPR, SH = D == 64 ? 1 : 0;
  const int r = lane & 31, g = lane >> 5;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      *reinterpret_cast<u32x2*>(stage + r * RB + (((db * 4 + qd) ^ ((r >> SH) & (CPR - 1))) << 4) +
                                g * 8) =
          pack_bf16x4(acc[db][qd * 4 + 0] * mul, acc[db][qd * 4 + 1] * mul,
                      acc[db][qd * 4 + 2] * mul, acc[db][qd * 4 + 3] * mul);
  // the reads below take values other lanes wrote: keep them after the writes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  constexpr int NI = 32 / RPI;
  const int ch = lane % CPR, row0 = lane / CPR;
  u32x4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = i * RPI + row0;
    v[i] = *reinterpret_cast<const u32x4*>(stage + row * RB + ((ch ^ ((row >> SH) & (CPR - 1))) << 4));
  }
  uint16_t* d0 = dst + (size_t)row0 * D + ch * 8;
  if (valid >= 32) {
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(d0 + (size_t)i * RPI * D) = v[i];
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (i * RPI + row0 < valid) *reinterpret_cast<u32x4*>(d0 + (size_t)i * RPI * D) = v[i];
  }
  // a later write to `stage` must not overtake these reads
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Active blocks of one row (or column) of the block mask, 64 at a time: bit i
// of `bits` tells whether block base + i is active.  A window is filled with
// one byte load per lane and a ballot, only when a query moves past the
// current 64-block window.  The kernels ask right after their per-tile wait
// and barrier, when no copy is in flight, so that load costs its own latency
// and nothing more; between refills a query is a few scalar bit operations
// instead of one dependent mask load per skipped tile.  Wavefront-uniform.
struct MaskWindow {
  unsigned long long bits = 0;
  int base = -64;
  // first active block >= b among blocks [0, nb), or nb; at(blk) returns the
  // mask byte of block blk (blk < nb)
  template <class At>
  __device__ __forceinline__ int next(int b, int nb, const At& at) {
    while (b < nb) {
      const int wb = b & ~63;
      if (wb != base) {
        const int lb = wb + lane_id();
        bits = __builtin_amdgcn_ballot_w64(lb < nb && at(lb) != 0);
        base = wb;
      }
      const unsigned long long m = bits >> (b - wb);
      if (m) return b + (int)__builtin_ctzll(m);
      b = wb + 64;
    }
    return nb;
  }
};

// Next tile t' >= t (tiles of TILE rows along the masked axis) whose mask block
// is active, or `ntiles`: the block of t itself if active, else the first tile
// of the next active block.
template <int TILE, class At>
__device__ __forceinline__ int next_active_tile(MaskWindow& w, int t, int ntiles, int mask_block,
                                                int nb, const At& at) {
  if (t >= ntiles) return ntiles;
  const int b = (t * TILE) / mask_block;
  const int b2 = w.next(b, nb, at);
  if (b2 != b) t = b2 * (mask_block / TILE);
  return min(t, ntiles);
}

// Block index -> (query/key block, batch*head).  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2), so id mod 8 picks the
// XCD.  Every head's blocks go to one XCD (bh mod 8 = id mod 8), and within an
// XCD the heads are taken four at a time: all blocks of four heads, block 0
// (the longest under the causal order of the kernels) first, before the next
// four.  Each XCD then has about four heads' K and V (or Q and dO) in flight,
// which its 4 MB L2 can hold, and still starts the long blocks first.
// Without `grouped`, or when B*H is not a multiple of 32, the order is plain
// block-major (the first BH ids take block 0 of every head, the next BH block
// 1, ...): every head's longest block starts first, which measured better for
// the causal query-block kernels, whose blocks differ most in length.
struct BlockCoord {
  int blk;
  int bh;
};

__device__ __forceinline__ BlockCoord block_coord(int nblk, bool grouped) {
  const int BH = (int)gridDim.x / nblk;
  const int id = (int)blockIdx.x;
  BlockCoord c;
  if (grouped && BH % 32 == 0) {
    constexpr int kXcd = 8, kGroup = 4;
    const int x = id % kXcd, l = id / kXcd;           // XCD, position on it
    const int g = l / (kGroup * nblk), rem = l - g * (kGroup * nblk);
    c.blk = rem / kGroup;
    c.bh = (g * kGroup + (rem - c.blk * kGroup)) * kXcd + x;
  } else {
    c.blk = id / BH;
    c.bh = id - c.blk * BH;
  }
  return c;
}

}  // namespace fa
