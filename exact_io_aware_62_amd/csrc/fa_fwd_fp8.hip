// FP8 forward: O = softmax(scale * Q K^T + mask) V and LSE, with Q, K and V
// given as E4M3 codes and one fp32 descale per tensor (element = code value
// times descale).  Both products run on the gfx950 8-bit matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation); P is rounded to E4M3 for
// the P V product.
//
// The FlashAttention-2 wiki ("与后续版本的比较", FlashAttention-3) names 8-bit
// floating point as the next step in speed; the rest is the bf16 forward's
// method unchanged (FlashAttention-NeurIPS22 digest, "核心方法": tiling,
// online softmax, fused mask; FlashAttention-2 wiki, "技术架构与工作原理":
// grid over query block x head, rows owned by one wavefront, 1/l deferred).
//
// What changes against the bf16 kernel:
//   * one matrix op covers 64 values of the contraction index (32 bytes per
//     lane and operand), so a 64-key tile takes 2 * D/64 score products and
//     D/32 P V products per wavefront instead of 2 * D/16 and D/8;
//   * the scale and the Q and K descales are folded into the exp2 factor,
//     and the V descale into the epilogue's 1/l;
//   * P is formed as exp2(S c - m + kOff) with the running maximum allowed to
//     lag the true one by at most kSlack, so every P value lies in
//     (0, 2^(kOff + kSlack)] = (0, 256], inside E4M3's finite range (448),
//     and the row's largest value is at least 2^kOff = 16: values down to
//     2^-10 of the row maximum keep three mantissa bits before E4M3's
//     subnormal range starts.  The row sum l is taken over the fp32 values,
//     so LSE is that of the exact scores; only O sees P's rounding;
//   * the V^T operand is read with the 8-bit LDS transpose read
//     (ds_read_b64_tr_b8), whose eight bytes per lane come from eight rows
//     that each lane pair addresses freely; the rows are chosen to match the
//     key order in which the score fragment holds P.
//
// Operand byte order.  For the 8-bit 32x32x64 op, lane l (r = l % 32,
// g = l / 32) holds row (A) or column (B) r and 32 bytes j = 0..31; the
// hardware pairs byte j of lane group g of A with byte j of lane group g of B,
// so any one map (g, j) -> contraction index serves both operands.  Scores:
// bytes j of group g are head-dim columns kk*64 + 32 g + j of Q and K.  P V:
// bytes j of group g are keys 32 (j/16) + 8 ((j%16)/4) + 4 g + j%4, which is
// the key of register j%16 of score block j/16 in that lane (C layout).

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// A (32 x 64) * B (64 x 32) + C with A and B E4M3 (format code 0), no block scales
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b,
                                                   const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16b(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 8-bit transpose read: lane i of each 16-lane group receives byte i % 8 of
// the 8-byte pieces addressed by lanes 2e + i / 8 of the group, e = 0..7.
__device__ __forceinline__ i32x2 lds_tr8_b64(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
}

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(FwdParams p) {
  constexpr int BQ = 128, BK = 64, NW = 4;
  constexpr float kSlack = 4.0f, kOff = 4.0f;
  constexpr int NDB = D / 32;   // 32-wide column blocks of O^T
  constexpr int NKK = D / 64;   // 64-wide steps over the head dimension
  // a row of D one-byte codes occupies the tile format of D/2 two-byte values
  using T = LdsTile<BK, D / 2>;
  constexpr int RB = T::kRowBytes;
  constexpr int TB = T::kBytes;
  static_assert(RB == D, "one byte per code");
  __shared__ __attribute__((aligned(1024))) char kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockCoord bc = block_coord(p.nqb, !CAUSAL);
  const int qb = CAUSAL ? (p.nqb - 1 - bc.blk) : bc.blk;   // heaviest blocks first
  const int N = p.Nq;
  const size_t head = (size_t)bc.bh * N * D;
  const uint8_t* __restrict__ Qh = reinterpret_cast<const uint8_t*>(p.Q) + head;
  const uint16_t* __restrict__ Kh = reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const uint8_t*>(p.K) + head);
  const uint16_t* __restrict__ Vh = reinterpret_cast<const uint16_t*>(
      reinterpret_cast<const uint8_t*>(p.V) + head);

  const int q0w = qb * BQ + wave * 32;
  const int qrow = q0w + r;

  // Q fragments (B operand of S^T = K Q^T): row qrow, bytes kk*64 + 32 g .. +31
  i32x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const uint8_t* src = Qh + (size_t)qrow * D + kk * 64 + g * 32;
    const u32x4 lo = qrow < N ? ldg16b(src) : zero_u32x4();
    const u32x4 hi = qrow < N ? ldg16b(src + 16) : zero_u32x4();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[kk][e] = (int)lo[e];
      qf[kk][4 + e] = (int)hi[e];
    }
  }

  const int kend = CAUSAL ? min(N, (qb + 1) * BQ) : N;
  const int ntiles = (kend + BK - 1) / BK;
  const int mrow = SPARSE ? (qb * BQ) / p.mask_block : 0;
  MaskWindow mw;
  auto next_tile = [&](int t) FA_INLINE -> int {
    if constexpr (SPARSE) {
      const uint8_t* mr = p.blockmask + (size_t)mrow * p.nbm;
      return next_active_tile<BK>(mw, t, ntiles, p.mask_block, p.nbm,
                                  [&](int b) FA_INLINE { return mr[b]; });
    }
    return t;
  };
  auto needs_mask = [&](int t) FA_INLINE {
    return (CAUSAL && t * BK + BK - 1 > q0w) || (t * BK + BK > N);
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float m_run = kNegBig;
  float l_run = 0.f;
  const float c = p.scale_log2;   // scale * q_descale * k_descale * log2(e)

  const auto lofs = T::template lane_offsets<NW>(wave, lane);
  auto load_k = [&](int t, int buf) FA_INLINE {
    T::template copy<NW>(Kh, t * BK, N, buf ? kbuf1 : kbuf0, wave, lofs);
  };
  auto load_v = [&](int t, int buf) FA_INLINE {
    T::template copy<NW>(Vh, t * BK, N, buf ? vbuf1 : vbuf0, wave, lofs);
  };

  f32x16 sc[2];   // scores of the current tile, key blocks 0 and 1
  // P of a tile as the B operand of the P V product; two sets, by tile parity
  i32x8 pb[2];

  auto mask = [&](int tc) FA_INLINE {
    if (needs_mask(tc)) {
      const int ln = lane_id();
      const int kl = tc * BK + (ln >> 5) * 4;
      const int lim = CAUSAL ? min(N - 1, q0w + (ln & 31)) - kl : N - 1 - kl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sc[kb][i] = -INFINITY;
    }
  };
  // Row max as in the bf16 forward: 32 values -> 12 -> 4 in part 1, then
  // 4 -> 1 and the lane-half exchange in part 2, with raw max instructions.
  float mx4[4];
  auto rowmax_part1 = [&]() FA_INLINE {
    float t[12];
#pragma unroll
    for (int u = 0; u < 10; ++u) {
      const int e = 3 * u;
      t[u] = max3_raw(sc[e >> 4][e & 15], sc[(e + 1) >> 4][(e + 1) & 15],
                      sc[(e + 2) >> 4][(e + 2) & 15]);
    }
    t[10] = sc[1][14];
    t[11] = sc[1][15];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      mx4[u] = max3_raw(t[3 * u], t[3 * u + 1], t[3 * u + 2]);
      pin(mx4[u]);
    }
  };
  // Moves the running maximum only when the tile's exceeds it by more than
  // kSlack; returns the factor for the accumulated O (1 if unmoved).
  auto rowmax_part2 = [&]() FA_INLINE -> float {
    const float mx = max_raw(max3_raw(mx4[0], mx4[1], mx4[2]), mx4[3]);
    const float mxc = max_xor32(mx) * c;
    float alpha = 1.f;
    if (mxc > m_run + kSlack) {
      alpha = exp2_fast(m_run - mxc);
      m_run = mxc;
      l_run *= alpha;
    }
    pin(m_run);
    pin(alpha);
    return alpha;
  };
  // P of element e (key block e / 16, register e % 16)
  auto pexp = [&](int e, float moff) FA_INLINE -> float {
    return exp2_fast(__builtin_fmaf(sc[e >> 4][e & 15], c, moff));
  };
  // dword w of the P operand: registers 4(w%4) .. +3 of key block w/4, as E4M3
  auto pack_word = [&](int w) FA_INLINE -> int {
    const int kb = w >> 2, i0 = 4 * (w & 3);
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(sc[kb][i0], sc[kb][i0 + 1], 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(sc[kb][i0 + 2], sc[kb][i0 + 3], x, true);
  };

  // Lane-dependent parts of the operand reads.
  //   K (A operand of the scores): row r of key block kb, 16-byte chunks
  //   4 kk + 2 g + h (h = 0, 1); the chunk swizzle depends on r only.
  const int sr = T::swz(r);
  const int kx = (2 * g) ^ sr;
  const int kr = r * RB;
  //   V^T (A operand of P V): the lane pair 2e, 2e+1 of a 16-lane group
  //   addresses row 8(e/4) + 4 g + e%4 of the 16-row part of read t, bytes
  //   col0 + 8 (lane % 2) with col0 = 32 db + 16 ((lane / 16) % 2).
  const int s16 = lane & 15, gi = (lane >> 4) & 1, e8 = s16 >> 1;
  const int vrl = 8 * (e8 >> 2) + 4 * g + (e8 & 3);
  const int vl = vrl * RB + 8 * (s16 & 1);
  const int vx = (gi ^ T::swz(vrl)) << 4;

  auto kread = [&](const char* kt, int j) FA_INLINE -> i32x8 {
    const int kb = j & 1, kk = j >> 1;
    const char* a = kt + kb * 32 * RB + kr;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(a + (((4 * kk) ^ kx) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(a + (((4 * kk + 1) ^ kx) << 4));
    i32x8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = (int)lo[e];
      v[4 + e] = (int)hi[e];
    }
    return v;
  };
  auto vread = [&](const char* vt, int db) FA_INLINE -> i32x8 {
    i32x8 v;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const char* a = vt + (32 * (t >> 1) + 16 * (t & 1)) * RB + vl + ((db << 5) ^ vx);
      const i32x2 x = lds_tr8_b64(a);
      v[2 * t] = x[0];
      v[2 * t + 1] = x[1];
    }
    return v;
  };

  // scores of the tile in K buffer kt; K fragments read PF products ahead
  auto phaseA = [&](const char* kt) FA_INLINE {
    constexpr int NJ = 2 * NKK, PF = 2;
    i32x8 kfr[NJ];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) kfr[j] = kread(kt, j);
    sc[0] = zero16();
    sc[1] = zero16();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sc[j & 1] = mfma32x32x64_fp8(kfr[j], qf[j >> 1], sc[j & 1]);
      if (j + PF < NJ) kfr[j + PF] = kread(kt, j + PF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P of the current tile into pb[PB], its fp32 row sum returned
  auto softmax_all = [&](auto pbc) FA_INLINE -> float {
    constexpr int PB = decltype(pbc)::value;
    const float moff = kOff - m_run;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float pe = pexp(e, moff);
      sc[e >> 4][e & 15] = pe;
      if (e & 1) a1 += pe;
      else a0 += pe;
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) pb[PB][w] = pack_word(w);
    return a0 + a1;
  };
  // O += P_prev V_prev (P in pb[PP], V in vt) on the matrix cores, with the
  // current tile's row max, exponentials, row sum and packing (into pb[1-PP])
  // between the products.
  auto phaseB = [&](auto ppc, const char* vt, float& alpha) FA_INLINE -> float {
    constexpr int PP = decltype(ppc)::value;
    constexpr int PF = 2;
    i32x8 vfr[NDB];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) vfr[j] = vread(vt, j);
    float a0 = 0.f, a1 = 0.f, moff = 0.f;
    // exponentials of elements [E0(j), E0(j + 1)) after product j (j >= 1)
    auto E0 = [](int j) { return j < 1 ? 0 : (j - 1) * 32 / (NDB - 1); };
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
      oacc[j] = mfma32x32x64_fp8(vfr[j], pb[PP], oacc[j]);
      if (j + PF < NDB) vfr[j + PF] = vread(vt, j + PF);
      if (j == 0) {
        rowmax_part1();
        alpha = rowmax_part2();
        moff = kOff - m_run;
      } else {
        const int e0 = E0(j), e1 = j + 1 == NDB ? 32 : E0(j + 1);
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          float pe = pexp(e, moff);
          pin(pe);
          sc[e >> 4][e & 15] = pe;
          if (e & 1) a1 += pe;
          else a0 += pe;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) pb[1 - PP][w] = pack_word(w);
    return a0 + a1;
  };
  auto pv_only = [&](auto ppc, const char* vt) FA_INLINE {
    constexpr int PP = decltype(ppc)::value;
    i32x8 vfr[NDB];
#pragma unroll
    for (int j = 0; j < NDB; ++j) vfr[j] = vread(vt, j);
#pragma unroll
    for (int j = 0; j < NDB; ++j) oacc[j] = mfma32x32x64_fp8(vfr[j], pb[PP], oacc[j]);
  };
  auto rescale = [&](float alpha) FA_INLINE {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
  };

  // Iteration for tile tc, whose K is in K buffer PAR; the previous tile's V
  // is in V buffer 1 - PAR and its P in pb[1 - PAR].  The current tile's P
  // goes to pb[PAR].
  auto iteration = [&](auto parc, auto firstc, int& tc, int& tn) FA_INLINE {
    constexpr int PAR = decltype(parc)::value;
    constexpr bool FIRST = decltype(firstc)::value;
    wait_vmem();
    __syncthreads();
    const int tn2 = tn < ntiles ? next_tile(tn + 1) : ntiles;
    if (tn < ntiles) load_k(tn, 1 - PAR);
    load_v(tc, PAR);
    phaseA(PAR ? kbuf1 : kbuf0);
    mask(tc);
    if constexpr (FIRST) {
      rowmax_part1();
      rowmax_part2();
      l_run += softmax_all(std::integral_constant<int, PAR>{});
    } else {
      float alpha;
      const float psum =
          phaseB(std::integral_constant<int, 1 - PAR>{}, PAR ? vbuf0 : vbuf1, alpha);
      l_run += psum;
      rescale(alpha);
    }
    tc = tn;
    tn = tn2;
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int tc = next_tile(0);
  int tn = tc < ntiles ? next_tile(tc + 1) : ntiles;
  if (tc < ntiles) {
    load_k(tc, 0);
    iteration(P0{}, std::true_type{}, tc, tn);
    while (tn < ntiles) {
      iteration(P1{}, std::false_type{}, tc, tn);
      iteration(P0{}, std::false_type{}, tc, tn);
    }
    const bool odd = tc < ntiles;
    if (odd) iteration(P1{}, std::false_type{}, tc, tn);
    wait_vmem();
    __syncthreads();
    if (odd) pv_only(P1{}, vbuf1);
    else pv_only(P0{}, vbuf0);
    // every wavefront is done with the V tile before the epilogue reuses it
    __syncthreads();
  }

  // epilogue: O = O_acc * v_descale / l, LSE of the exact scores
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? p.v_descale / l_tot : 0.f;
  // O (bf16, 32 rows of 2D bytes per wavefront) leaves through one of the
  // four 8-bit tile buffers (64 rows of D bytes each) per wavefront
  if (q0w < N) {
    char* stage = wave == 0 ? kbuf0 : wave == 1 ? kbuf1 : wave == 2 ? vbuf0 : vbuf1;
    store_rows_staged<D>(stage, oacc, inv, p.O + (size_t)bc.bh * N * D + (size_t)q0w * D, N - q0w,
                         lane);
  }
  if (qrow < N && g == 0)
    p.LSE[(size_t)bc.bh * N + qrow] =
        l_tot > 0.f ? (m_run - kOff + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D>
static hipError_t launch_fwd_fp8_t(const FwdParams& p, bool causal, bool sparse,
                                   hipStream_t stream) {
  const dim3 grid((unsigned)((long long)p.nqb * p.BH));
  if (causal) {
    if (sparse)
      hipLaunchKernelGGL((fwd_fp8_kernel<D, true, true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_fp8_kernel<D, true, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (sparse)
      hipLaunchKernelGGL((fwd_fp8_kernel<D, false, true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_fp8_kernel<D, false, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, bool sparse,
                          hipStream_t stream) {
  if (d == 64) return launch_fwd_fp8_t<64>(p, causal, sparse, stream);
  if (d == 128) return launch_fwd_fp8_t<128>(p, causal, sparse, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
