// Backward kernels: recompute S and P from Q, K and the saved LSE and form
// dQ, dK, dV (FlashAttention-NeurIPS22 digest, "核心方法", Backward
// recomputation: only O and the softmax normalisers are kept from the
// forward, S and P are rebuilt on chip).
//
// With P = softmax(S), S = scale * Q K^T (+ mask), and L = sum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = sum_k dO_ik O_ik,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three kernels, all deterministic (no atomics; FlashAttention-2 wiki,
// "性能与效率": exact and deterministic):
//   1. dsum_kernel   D_i from the O actually handed in (bf16) and dO;
//   2. dkdv_kernel   one workgroup per 128 keys of one head, looping over
//                    query tiles: dV and dK accumulate in registers and are
//                    written once;
//   3. dq_kernel     one workgroup per 128 query rows, looping over key
//                    tiles: dQ accumulates in registers and is written once.
// The full backward runs dq_kernel first with D formed inside it (bitwise
// the value dsum_kernel gives), then dkdv_kernel: two launches.
// Both main kernels split the sequence over workgroups the way the forward
// does (FlashAttention-2 wiki, "技术架构与工作原理", item 2).

#include <atomic>
#include <mutex>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// log2-domain LSE with the empty-row convention folded in: an empty row
// (LSE = -inf) maps to +inf so that exp2(s - lse2) is exactly 0.
__device__ __forceinline__ float lse_to_log2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

// ---------------------------------------------------------------------------
// 1. D_i = sum_k dO_ik * O_ik  (fp32 accumulation, fixed order)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void dsum_kernel(BwdParams p, long long rows) {
  constexpr int LPR = D / 8;                 // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;             // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = ldg16(p.O + row * D + part * 8);
    const u32x4 g = ldg16(p.dO + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o0 = __uint_as_float(o[i] << 16), o1 = __uint_as_float(o[i] & 0xffff0000u);
      const float g0 = __uint_as_float(g[i] << 16), g1 = __uint_as_float(g[i] & 0xffff0000u);
      acc = __builtin_fmaf(o0, g0, acc);
      acc = __builtin_fmaf(o1, g1, acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) p.Dsum[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  Workgroup = 4 wavefronts = 128 keys; wavefront w owns keys
//    kw .. kw+31: their V rows in registers, the workgroup's K rows in LDS
//    (copied once).  Query tiles of 32 rows (Q and dO, natural layout) are
//    copied HBM -> LDS asynchronously, double-buffered.  S = Q K^T and
//    dP = dO V^T contract over d (row operands); dV^T += dO^T P and
//    dK^T += Q^T dS contract over queries, with dO^T and Q^T read by the LDS
//    transpose read.  Scores are formed as S (queries x keys) so each lane
//    owns one key and the P / dS fragments feed the dV / dK products as B
//    operands directly.  K in LDS and 32-row tiles keep every live value in
//    at most 256 vector registers (two wavefronts per SIMD, no accumulator
//    registers), and the LDS footprint lets two workgroups share a CU.
// ---------------------------------------------------------------------------
//    DROPOUT: dV^T += dO^T (P keep / (1 - p)) and dS = P (dP keep / (1 - p) - D),
//    computed as dV = (1 / (1 - p)) (P keep)^T dO and dS = (1 / (1 - p)) P (dP keep -
//    D (1 - p)): the loop only zeroes dropped elements and takes D times 1 - p,
//    and the factor 1 / (1 - p) is applied to dV and dK once, at the store.
//    A lane holds one key and 16 queries, while one Philox draw covers two
//    consecutive queries by four consecutive keys; so the four lanes of a
//    quad (keys 4c .. 4c+3) each draw two query pairs and exchange the 8-bit
//    results with DPP quad broadcasts: two draws per lane and tile.
//    The dropout draws need registers beyond the 256 the d=128 kernel fills;
//    that instantiation spills 2-6 of them to scratch, which measured faster
//    than one workgroup per CU without spills.
template <int D, bool CAUSAL, bool SPARSE, bool DROPOUT>
__global__ __launch_bounds__(256, 2) void dkdv_kernel(BwdParams p) {
  constexpr int BKB = 128, BQ = 32, NW = 4;
  constexpr int NDB = D / 32, NKK = D / 16;
  using TQ = LdsTile<BQ, D>;    // a query tile of Q or dO
  using TK = LdsTile<BKB, D>;   // the workgroup's K rows
  constexpr int RB = TQ::kRowBytes;
  // K rows of the workgroup; two stages of the Q and dO tiles and of the
  // per-query lse2 / D values.  The tiles are filled by copy_async, and the
  // stage is chosen at run time, so one loop body serves both stages.
  __shared__ __attribute__((aligned(1024))) char kbuf[TK::kBytes];
  // stage s: its Q tile at 2 s kBytes, its dO tile right after it
  __shared__ __attribute__((aligned(1024))) char qobuf[4 * TQ::kBytes];
  __shared__ __attribute__((aligned(16))) float rowbuf[2 * 2 * BQ];   // lse2, then D (-D without dropout)

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockCoord bc = block_coord(p.nkb, true);
  const int kb = bc.blk;
  // Nq queries, Nk keys; causal: query i sees key j iff j <= i + dlt
  const int Nq = p.Nq, Nk = p.Nk, dlt = Nk - Nq;
  const size_t qhead = (size_t)bc.bh * Nq * D, khead = (size_t)bc.bh * Nk * D;
  const uint16_t* __restrict__ Qh = p.Q + qhead;
  const uint16_t* __restrict__ dOh = p.dO + qhead;
  const float* __restrict__ lseh = p.LSE + (size_t)bc.bh * Nq;
  const float* __restrict__ Dh = p.Dsum + (size_t)bc.bh * Nq;

  const int kw = kb * BKB + wave * 32;   // first key of this wavefront
  const int key = kw + r;                // this lane's key
  copy_async<TK, NW>(p.K + khead, kb * BKB, Nk, lds_addr(kbuf), wave,
                     TK::template lane_offsets<NW>(wave, lane));
  bf16x8 vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    vf[kk] = as_bf16x8(key < Nk ? ldg16(p.V + khead + (size_t)key * D + kk * 16 + g * 8)
                                : zero_u32x4());

  // query tiles: causal => only rows i >= (first key of the block) - dlt
  const int nqt = (Nq + BQ - 1) / BQ;
  const int t_begin = CAUSAL ? max(0, kb * BKB - dlt) / BQ : 0;
  const int mcol = SPARSE ? (kb * BKB) / p.mask_block : 0;
  MaskWindow mw;
  auto next_tile = [&](int t) FA_INLINE -> int {
    if constexpr (SPARSE) {
      // column mcol of the mask, one byte per block of query rows
      t = next_active_tile<BQ>(mw, t, nqt, p.mask_block, (Nq + p.mask_block - 1) / p.mask_block,
                               [&](int b) FA_INLINE {
                                 return p.blockmask[(size_t)b * p.nbm + mcol];
                               });
    } else {
      // opaque to the optimizer: with a visible t + 1 sequence it reshapes
      // the tile loop and the dK / dV accumulators end up copied between
      // register sets
      t = __builtin_amdgcn_readfirstlane(t);
      asm volatile("" : "+s"(t));
    }
    return t;
  };

  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv[db] = zero16();
    dk[db] = zero16();
  }
  const float c = p.scale_log2;
  DropoutStream drs;
  if constexpr (DROPOUT) {
    drs.seed_lo = p.seed_lo;
    drs.seed_hi = p.seed_hi;
    drs.bh = (uint32_t)bc.bh;
    drs.offset = p.drop_offset;
    drs.thresh = p.drop_thresh;
  }

  // Thread tid < 2*BQ carries one LSE / D value of the next tile: it is
  // loaded before that tile's LDS-DMA copies are issued (vector-memory waits
  // complete in issue order, so waiting for it then does not wait for the
  // copies) and converted and stored only after the current tile's compute.
  // (Spreading the 2 BQ values over all four wavefronts measured 1-1.5%
  // slower: every wavefront then waits for its copies at this point.)
  float rowv = 0.f;
  int rowq = 0;
  const auto lofs = TQ::template lane_offsets<NW>(wave, lane);
  auto issue = [&](int t, int bufi) FA_INLINE {
    if (tid < 2 * BQ) {
      rowq = t * BQ + (tid % BQ);
      const int qc = min(rowq, Nq - 1);
      rowv = tid < BQ ? lseh[qc] : Dh[qc];
    }
    copy_async<TQ, NW>(Qh, t * BQ, Nq, lds_addr(qobuf) + bufi * 2 * TQ::kBytes, wave, lofs);
    copy_async<TQ, NW>(dOh, t * BQ, Nq, lds_addr(qobuf) + (bufi * 2 + 1) * TQ::kBytes, wave,
                       lofs);
  };
  auto finish_issue = [&](int bufi) FA_INLINE {
    __builtin_amdgcn_sched_barrier(0);
    if (tid < 2 * BQ) {
      float v;
      if (tid < BQ) v = rowq < Nq ? lse_to_log2(rowv) : INFINITY;
      else v = rowq < Nq ? (DROPOUT ? rowv * p.drop_keep : -rowv) : 0.f;
      rowbuf[bufi * 2 * BQ + tid] = v;
    }
  };

  // LDS addresses of this lane's operand reads.  qa[kk]: row read of k-step
  // kk in the Q tile of the stage in use (the dO tile lies kBytes further);
  // ta[db][h]: half h of the transposed read for output column block db, at
  // k-step 0 of that Q tile (k-step ks2 lies 16 ks2 rows further); ka[kk]:
  // row read of k-step kk in this wavefront's 32 K rows.  Each is the full
  // swizzled address, formed once: when the stage flips, qa and ta move by
  // 2 kBytes (2 NKK adds per tile in all), and every read is one address
  // register plus a compile-time immediate.  xad() is opaque, so the
  // compiler keeps these registers rather than redoing the lane arithmetic
  // of each read.
  const OperandAddr<TQ> oa = operand_addr<TQ>(lane);
  int qa[NKK], ka[NKK], ta[NDB][2];
  {
    const int q0a = lds_addr(qobuf), k0a = lds_addr(kbuf) + wave * 32 * RB;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qa[kk] = xad(oa.xr, kk << 5, oa.ar + q0a);
      ka[kk] = xad(oa.xr, kk << 5, oa.ar + k0a);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      ta[db][0] = xad(oa.xt, db << 6, oa.at0 + q0a);
      ta[db][1] = xad(oa.xt, db << 6, oa.at1 + q0a);
    }
  }
  // row operand (contraction over d) of k-step kk at LDS address a[kk] + off
  auto row_read = [&](const int (&a)[NKK], int kk, int off) FA_INLINE {
    return as_bf16x8(lds_read_b128_at(a[kk], off));
  };
  // transposed operand (contraction over queries) for product j of a dV / dK
  // step: k-step ks2 = j / NDB (queries 16 ks2 ..), output column block db;
  // off = 0 for Q^T, kBytes for dO^T
  auto tr_read = [&](int j, int off) FA_INLINE {
    const int ks2 = j / NDB, db = j % NDB;
    const int o = off + 16 * ks2 * RB;
    return bf16x8_from_halves(lds_tr_b64_at(ta[db][0], o), lds_tr_b64_at(ta[db][1], o));
  };

  // One query tile, in four steps of 2 NDB products each; LDS operands are
  // read ahead and each product is fenced, so issue order = program order:
  //   1. S = Q K^T               (both operands from LDS)
  //   2. dP = dO V^T             || P = exp2(S c - lse2), packed to bf16
  //   3. dV^T += dO^T P          || dS = P (dP - D), packed to bf16
  //   4. dK^T += Q^T dS
  // Dropout keep bits: bit i for register i (query q0 + (i/4)*8 + g*4 + i%4,
  // key `key`) of the current tile; the next tile's are drawn during the
  // current tile's last step, where the fewest registers are live.
  uint32_t keep_cur = 0xFFFFFFFFu, keep_next = 0xFFFFFFFFu;
  // A quad of lanes holds four consecutive keys (key group (kw + r) / 4) and,
  // per lane group g, the 16 queries of registers i (query q0 + (i/4)*8 +
  // g*4 + i%4), eight query pairs p = (i/4)*2 + (i%4)/2.  One draw decides a
  // pair for the quad's four keys.  Lane c = r % 4 draws pairs c (h = 0) and
  // c + 4 (h = 1) of the tile at query q0; finish_keep then collects, from
  // each quad lane's two draws, the bits of this lane's key.
  uint32_t keep_mine = 0;
  auto draw_keep = [&](int q0, int h) FA_INLINE {
    const int pr = (r & 3) + 4 * h;
    const uint32_t ig = (uint32_t)((q0 + (pr >> 1) * 8 + g * 4 + (pr & 1) * 2) >> 1);
    keep_mine |= drs.keep8((uint32_t)((kw >> 2) + (r >> 2)), ig) << (8 * h);
    pin(keep_mine);
  };
  auto finish_keep = [&]() FA_INLINE {
    const int c = r & 3;
    uint32_t kb = 0;
    static_for<0, 4>([&](auto tc) FA_INLINE {
      constexpr int T = decltype(tc)::value;
      // lane T's draws: pair T in bits 0..7, pair T + 4 in bits 8..15; this
      // key's bits c and 4 + c of each go to registers i0, i0 + 1 and
      // i0 + 8, i0 + 9
      constexpr int i0 = (T >> 1) * 4 + (T & 1) * 2;
      const uint32_t y = (quad_bcast<T>(keep_mine) >> c) & 0x1111u;
      kb |= ((y & 0x101u) | ((y >> 3) & 0x202u)) << i0;
    });
    keep_next = kb;
    keep_mine = 0;
    pin(keep_next);
  };

  auto compute = [&](int stage, int t, int tn) FA_INLINE {
    constexpr int NJ = NKK;   // products per step (= 2 NDB)
    const float* lse2 = rowbuf + stage * 2 * BQ;
    const float* dsum = lse2 + BQ;
    const int q0 = t * BQ;
    f32x16 s, dp;
    bf16x8 pb[2], sb[2];
    const uint32_t keepbits = keep_cur;
    bf16x8 fa[NJ], fb[NJ];
    constexpr int PF = 2;

    // 1. S = Q K^T
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      fa[j] = row_read(qa, j, 0);
      fb[j] = row_read(ka, j, 0);
    }
    s = zero16();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      s = mfma32x32x16(fa[j], fb[j], s);
      if (j + PF < NJ) {
        fa[j + PF] = row_read(qa, j + PF, 0);
        fb[j + PF] = row_read(ka, j + PF, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // mask: causal diagonal, ragged query or key ends (rare tiles only)
    const bool need_mask = (CAUSAL && q0 + dlt < kw + 31) || (q0 + BQ > Nq) || (kw + 32 > Nk);
    if (need_mask) {
      // register i holds query q0 + (i/4)*8 + g*4 + i%4; this lane's key
      const int ln = lane_id();
      const int kl = kw + (ln & 31);
      const int qg = q0 + (ln >> 5) * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = qg + (i >> 2) * 8 + (i & 3);
        if ((CAUSAL && kl > q + dlt) || q >= Nq || kl >= Nk) s[i] = -INFINITY;
      }
    }

    // 2. dP = dO V^T || P
    u32x4 l4;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) fa[j] = row_read(qa, j, TQ::kBytes);
    if constexpr (DROPOUT) {
      dp = zero16();
    } else {
      // the dP accumulator starts at -D of each register's query, so the
      // products leave dP - D (this form's row buffer holds -D)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(dsum + k * 8 + g * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * k + e] = __uint_as_float(v[e]);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      dp = mfma32x32x16(fa[j], vf[j], dp);
      if (j + PF < NJ) fa[j + PF] = row_read(qa, j + PF, TQ::kBytes);
#pragma unroll
      for (int i = j * 16 / NJ; i < (j + 1) * 16 / NJ; ++i) {
        // LSE (log2 units) of the four queries of registers (i/4)*4 .. +3,
        // one 16-byte read per four registers
        if ((i & 3) == 0) l4 = *reinterpret_cast<const u32x4*>(lse2 + (i >> 2) * 8 + g * 4);
        s[i] = exp2_fast(__builtin_fmaf(s[i], c, -__uint_as_float(l4[i & 3])));
        if ((i & 7) == 7) {
          if constexpr (DROPOUT) {
            // dV takes the kept, rescaled probabilities; dS below takes P
            float t8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              t8[e] = ((keepbits >> (i - 7 + e)) & 1u) ? s[i - 7 + e] : 0.f;
            pb[i >> 3] = pack_bf16x8(t8[0], t8[1], t8[2], t8[3], t8[4], t8[5], t8[6], t8[7]);
          } else {
            pb[i >> 3] = pack_c8(s, i - 7);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // 3. dV^T += dO^T P || dS
    // (issue priority 1 here: of the two wavefronts of a SIMD, the one forming
    // dS under its products goes first; measured about 1% faster, where the
    // same in step 2 or in dQ's mixed products measured slower or no change)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < PF; ++j) fa[j] = tr_read(j, TQ::kBytes);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      dv[j % NDB] = mfma32x32x16(fa[j], pb[j / NDB], dv[j % NDB]);
      if (j + PF < NJ) fa[j + PF] = tr_read(j + PF, TQ::kBytes);
#pragma unroll
      for (int i = j * 16 / NJ; i < (j + 1) * 16 / NJ; ++i) {
        if constexpr (DROPOUT) {
          const float* dq4 = dsum + (i >> 2) * 8 + g * 4;
          const float dpv = ((keepbits >> i) & 1u) ? dp[i] : 0.f;
          dp[i] = s[i] * (dpv - dq4[i & 3]);
        } else {
          dp[i] = s[i] * dp[i];
        }
        if ((i & 7) == 7) sb[i >> 3] = pack_c8(dp, i - 7);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // 4. dK^T += Q^T dS
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) fa[j] = tr_read(j, 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      dk[j % NDB] = mfma32x32x16(fa[j], sb[j / NDB], dk[j % NDB]);
      if (j + PF < NJ) fa[j + PF] = tr_read(j + PF, 0);
      if constexpr (DROPOUT) {
        // the next tile's two draws (unused after the last tile)
        if (j % (NJ / 2) == 0) draw_keep(tn * BQ, j / (NJ / 2));
        if (j == NJ - 1) finish_keep();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int t_first = next_tile(t_begin);
  int t = t_first;
  int stage = 0;
  if (t < nqt) {
    issue(t, 0);
    finish_issue(0);
    if constexpr (DROPOUT) {
      draw_keep(t * BQ, 0);
      draw_keep(t * BQ, 1);
      finish_keep();
    }
  }
  // one loop body for both stages keeps the dK / dV accumulators in one
  // register set
  while (t < nqt) {
    wait_vmem();
    __syncthreads();
    const int tn = next_tile(t + 1);
    if (tn < nqt) issue(tn, stage ^ 1);
    if constexpr (DROPOUT) keep_cur = keep_next;
    // a query tile entirely before this wavefront's first key's diagonal
    // contributes 0 (the dropout form draws the next tile's bits in there)
    if (DROPOUT || !(CAUSAL && t * BQ + BQ - 1 + dlt < kw)) compute(stage, t, tn);
    if (tn < nqt) finish_issue(stage ^ 1);
    t = tn;
    // to the other stage's tiles
    const int flip = stage ? -2 * TQ::kBytes : 2 * TQ::kBytes;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qa[kk] += flip;
      pin(qa[kk]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      ta[db][0] += flip;
      ta[db][1] += flip;
      pin(ta[db][0]);
      pin(ta[db][1]);
    }
    stage ^= 1;
  }

  // epilogue: dV and dK (lane r + 32 g holds key kw + r) leave through this
  // wavefront's own 32 rows of the K buffer, which no other wavefront reads.
  // Without a single query tile the K copy was never waited for: wait for
  // it (every wavefront fills part of every row block) before overwriting.
  if (t_first >= nqt) {
    wait_vmem();
    __syncthreads();
  }
  if (kw < Nk) {
    char* stage = kbuf + wave * 32 * RB;
    const float ds = DROPOUT ? p.drop_scale : 1.f;
    store_rows_staged<D>(stage, dv, ds, p.dV + khead + (size_t)kw * D, Nk - kw, lane);
    store_rows_staged<D>(stage, dk, p.scale * ds, p.dK + khead + (size_t)kw * D, Nk - kw, lane);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ.  Workgroup = 4 wavefronts = 128 query rows (32 per wavefront, held
//    in registers with their dO rows).  Key tiles of 64 rows (K and V,
//    natural layout) are copied HBM -> LDS asynchronously, double-buffered:
//    S^T = K Q^T and dP^T = V dO^T use row operands, dQ^T += K^T dS^T reads
//    K^T with the LDS transpose read.  Same transposed-score arrangement as
//    the forward: each lane owns one query row, so LSE and D are per-lane
//    scalars.
//
//    Per tile the 4 NKK + 4 NDB matrix products are issued in a fixed order
//    (S^T of key block 0, of block 1, dP^T of block 0, of block 1, dQ of
//    block 0, of block 1), and the vector work runs under them, each piece
//    two products after the last product whose result it reads:
//    P = exp2(S c - lse2) of block 0 under S^T of block 1, of block 1 under
//    dP^T of block 0, dS = P (dP - D) of block 0 under dP^T of block 1, of
//    block 1 under dQ of block 0.
//
//    FUSED_D: the workgroup also forms D_i = sum_k dO_ik O_ik for its rows
//    and stores it, in exactly the order dsum_kernel uses (per eight-column
//    chunk a sequential fused multiply-add, then a pairwise tree over the
//    chunks whose index differs in bit D/16, D/32, ..., 1), so the result is
//    the same to the bit; the dK/dV kernel then reads it.
// ---------------------------------------------------------------------------
//    DROPOUT: dS = P (dP keep / (1 - p) - D), with the keep bits of the tile
//    drawn (as in the forward) while its scores are on the matrix cores; the
//    loop forms P (dP keep - D (1 - p)) and the factor 1 / (1 - p) joins the
//    scale of dQ at the store.
template <int D, bool CAUSAL, bool SPARSE, bool FUSED_D, bool DROPOUT>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdParams p) {
  constexpr int BQ = 128, BK = 64, NW = 4;
  constexpr int NDB = D / 32, NKK = D / 16;
  using T = LdsTile<BK, D>;
  constexpr int RB = T::kRowBytes;
  // two stages of the K and V tiles, filled by copy_async; the stage is
  // chosen at run time so one loop body serves both.  Stage s: its K tile at
  // 2 s kBytes, its V tile right after it.
  __shared__ __attribute__((aligned(1024))) char kvbuf[4 * T::kBytes];
  constexpr int KB = T::kBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockCoord bc = block_coord(p.nqb, !CAUSAL);
  const int qb = CAUSAL ? (p.nqb - 1 - bc.blk) : bc.blk;
  // Nq queries, Nk keys; causal: query i sees key j iff j <= i + dlt
  const int Nq = p.Nq, Nk = p.Nk, dlt = Nk - Nq;
  const size_t qhead = (size_t)bc.bh * Nq * D, khead = (size_t)bc.bh * Nk * D;
  const uint16_t* __restrict__ Kh = p.K + khead;
  const uint16_t* __restrict__ Vh = p.V + khead;

  const int q0w = qb * BQ + wave * 32;
  const int qrow = q0w + r;
  // Q, dO (and O for D) fragments: row qrow, columns kk*16 + g*8 .. +7,
  // filled from LDS before the first tile (see below)
  bf16x8 qf[NKK], of[NKK];
  const float lse2 = qrow < Nq ? lse_to_log2(p.LSE[(size_t)bc.bh * Nq + qrow]) : INFINITY;
  float dsum = 0.f;
  const OperandAddr<T> oa = operand_addr<T>(lane);
  // D for this lane's row from the O rows at `orow` (this wavefront's 32 rows
  // in the LDS tile format) and of[]
  auto form_d = [&](const char* orow) FA_INLINE {
    if constexpr (FUSED_D) {
      // chunk c = 2 kk + g of the row (columns 8c .. 8c+7) is in of[kk]
      float part[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 o = qrow < Nq ? *reinterpret_cast<const u32x4*>(orow + (oa.xr ^ (kk << 5)) + oa.ar)
                                  : zero_u32x4();
        const u32x4 gd = __builtin_bit_cast(u32x4, of[kk]);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = __builtin_fmaf(__uint_as_float(o[i] << 16), __uint_as_float(gd[i] << 16), acc);
          acc = __builtin_fmaf(__uint_as_float(o[i] & 0xffff0000u),
                               __uint_as_float(gd[i] & 0xffff0000u), acc);
        }
        part[kk] = acc;
      }
      // tree over chunk bits D/16 .. 2 inside the lane (kk bits NKK/2 .. 1),
      // then chunk bit 1 (= g) across the two lane halves
#pragma unroll
      for (int off = NKK / 2; off > 0; off >>= 1)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          if (!(kk & off)) part[kk] = part[kk] + part[kk | off];
      dsum = sum_xor32(part[0]);
      if (g == 0 && qrow < Nq) p.Dsum[(size_t)bc.bh * Nq + qrow] = dsum;
    } else {
      dsum = qrow < Nq ? p.Dsum[(size_t)bc.bh * Nq + qrow] : 0.f;
    }
  };

  const int kend = CAUSAL ? max(0, min(Nk, (qb + 1) * BQ + dlt)) : Nk;
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

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();
  const float c = p.scale_log2;
  DropoutStream drs;
  if constexpr (DROPOUT) {
    drs.seed_lo = p.seed_lo;
    drs.seed_hi = p.seed_hi;
    drs.bh = (uint32_t)bc.bh;
    drs.offset = p.drop_offset;
    drs.thresh = p.drop_thresh;
  }

  const auto lofs = T::template lane_offsets<NW>(wave, lane);
  auto issue = [&](int t, int stage) FA_INLINE {
    copy_async<T, NW>(Kh, t * BK, Nk, lds_addr(kvbuf) + 2 * stage * KB, wave, lofs);
    copy_async<T, NW>(Vh, t * BK, Nk, lds_addr(kvbuf) + (2 * stage + 1) * KB, wave, lofs);
  };

  constexpr int NS = 4 * NKK + 4 * NDB;   // products per tile
  constexpr int PF = 3;                   // operand reads issued this many products ahead
  // LDS addresses of this lane's operand reads in the K tile of the stage in
  // use (the V tile lies kBytes further): ra[kk], row read of k-step kk in
  // key rows 0..31 (rows 32..63 lie 32 rows further); ta[db][h], half h of
  // the transposed read for output column block db at keys 0..15.  Each is
  // the full swizzled address, formed once (xad() is opaque, so the compiler
  // keeps these registers rather than redoing the lane arithmetic of each
  // read); when the stage flips they move by 2 kBytes, and every read is
  // one address register plus a compile-time immediate.
  int ra[NKK], ta[NDB][2];
  {
    const int a0 = lds_addr(kvbuf);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) ra[kk] = xad(oa.xr, kk << 5, oa.ar + a0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      ta[db][0] = xad(oa.xt, db << 6, oa.at0 + a0);
      ta[db][1] = xad(oa.xt, db << 6, oa.at1 + a0);
    }
  }
  // operand of product j (see the schedule above)
  auto operand = [&](int j) FA_INLINE -> bf16x8 {
    if (j < 4 * NKK) {
      const int kb = (j / NKK) & 1, kk = j % NKK;
      return as_bf16x8(lds_read_b128_at(ra[kk], (j < 2 * NKK ? 0 : KB) + kb * 32 * RB));
    }
    const int jj = j - 4 * NKK, kb = jj / (2 * NDB), ks2 = (jj / NDB) & 1, db = jj % NDB;
    const int o = (kb * 32 + 16 * ks2) * RB;
    return bf16x8_from_halves(lds_tr_b64_at(ta[db][0], o), lds_tr_b64_at(ta[db][1], o));
  };

  // D as the loop uses it: times 1 - p with dropout (see the kernel comment);
  // set once D is known, after the rows are read below
  float dsum_k = 0.f;
  // At d = 128 without dropout the dP^T products of each key block start
  // from -D (this register block, the same value in all 16 entries) instead
  // of 0, so they leave dP - D.  At d = 64 the 16 extra registers would cost
  // a wavefront per SIMD, and with dropout dropped entries need D alone; those
  // forms start from 0 and subtract D.
  constexpr bool kFoldD = !DROPOUT && D == 128;
  f32x16 negd = zero16();
  auto compute = [&](int t) FA_INLINE {
    const int k0 = t * BK;
    const bool need_mask = (CAUSAL && k0 + BK - 1 > q0w + dlt) || (k0 + BK > Nk);
    f32x16 s[2], dp[2];
    bf16x8 ds[4];   // dS^T B operands, entry kb * 2 + ks2
    s[0] = zero16(); s[1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
    // keep bits: bit kb*16 + i for register i of key block kb (keys
    // k0 + kb*32 + (i/4)*8 + g*4 + i%4 of this lane's row)
    uint32_t keepbits = 0xFFFFFFFFu, keep_give = 0;
    bf16x8 fr[NS];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) fr[j] = operand(j);
    static_for<0, NS>([&](auto jc) FA_INLINE {
      constexpr int j = decltype(jc)::value;
      if constexpr (j < 2 * NKK) {
        constexpr int kb = j / NKK, kk = j % NKK;
        s[kb] = mfma32x32x16(fr[j], qf[kk], s[kb]);
      } else if constexpr (j < 4 * NKK) {
        constexpr int kb = (j - 2 * NKK) / NKK, kk = j % NKK;
        dp[kb] = mfma32x32x16(fr[j], of[kk], kk == 0 ? negd : dp[kb]);
      } else {
        constexpr int jj = j - 4 * NKK, kb = jj / (2 * NDB), ks2 = (jj / NDB) & 1, db = jj % NDB;
        dq[db] = mfma32x32x16(fr[j], ds[kb * 2 + ks2], dq[db]);
      }
      if constexpr (j + PF < NS) fr[j + PF] = operand(j + PF);
      if constexpr (DROPOUT && j < 2 * NKK && j % (2 * NKK / 4) == 0) {
        // four draws per tile, spread over the S^T products.  One draw decides
        // four keys of this lane's row and of lane r ^ 1's (rows 2 ig, 2 ig + 1:
        // q0w is even); draw v takes key group u = 2v + (row parity), keep bits
        // 4u .. 4u+3 (keys k0 + kb*32 + m*8 + g*4 + 0..3, u = kb*4 + m).
        constexpr int v = j / (2 * NKK / 4);
        const int odd = qrow & 1;
        const int u = 2 * v + odd, kb = u >> 2, m = u & 3;
        const uint32_t bits =
            drs.keep8((uint32_t)(t * (BK / 4) + kb * 8 + m * 2 + g), (uint32_t)qrow >> 1);
        const uint32_t own = ((odd ? bits >> 4 : bits) & 0xFu) << (4 * u);
        const uint32_t give = ((odd ? bits : bits >> 4) & 0xFu) << (4 * u);
        keepbits = v == 0 ? own : keepbits | own;
        keep_give = v == 0 ? give : keep_give | give;
        pin(keepbits);
        pin(keep_give);
        if constexpr (v == 3) {
          // the other row's bits come from the pair's other lane
          keepbits |= pair_swap(keep_give);
          pin(keepbits);
        }
      }
      // vector work of this product slot: unit u in 0..3 (P of block 0, P of
      // block 1, dS of block 0, dS of block 1) runs in slots
      // (u + 1) NKK + 2 .. (u + 2) NKK + 1, 16 / NKK elements per slot
      static_for<0, 4>([&](auto uc) FA_INLINE {
        constexpr int u = decltype(uc)::value;
        constexpr int s0 = (u + 1) * NKK + 2;
        if constexpr (j >= s0 && j < s0 + NKK) {
          constexpr int kb = u & 1;
          if constexpr (j == s0 && u < 2) {
            if (need_mask) {
              // register i holds key k0 + kb*32 + (i/4)*8 + g*4 + i%4
              const int ln = lane_id();
              const int kl = k0 + kb * 32 + (ln >> 5) * 4;
              const int lim = CAUSAL ? min(Nk - 1, q0w + (ln & 31) + dlt) - kl : Nk - 1 - kl;
#pragma unroll
              for (int i = 0; i < 16; ++i)
                if ((i >> 2) * 8 + (i & 3) > lim) s[kb][i] = -INFINITY;
            }
          }
          constexpr int PER = 16 / NKK, i0 = (j - s0) * PER;
          static_for<i0, i0 + PER>([&](auto ic) FA_INLINE {
            constexpr int i = decltype(ic)::value;
            if constexpr (u < 2) {
              float pv = exp2_fast(__builtin_fmaf(s[kb][i], c, -lse2));
              pin(pv);
              s[kb][i] = pv;
            } else {
              float dpv = dp[kb][i];   // dP - D if kFoldD, else dP
              if constexpr (DROPOUT)
                dpv = ((keepbits >> (kb * 16 + i)) & 1u) ? dpv : 0.f;
              float dsv = kFoldD ? s[kb][i] * dpv : s[kb][i] * (dpv - dsum_k);
              pin(dsv);
              dp[kb][i] = dsv;
              if constexpr ((i & 7) == 7) {
                ds[kb * 2 + (i >> 3)] = pack_c8(dp[kb], i - 7);
                pin(ds[kb * 2 + (i >> 3)]);
              }
            }
          });
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // The rows of the workgroup's query block arrive as whole-row copies into
  // LDS (a lane loading its own row would touch 32 rows per load), in two
  // phases that each fill all four tile slots of kvbuf:
  //   1. dO -> the K tiles of both stages, O -> the V tiles; read of[] and
  //      form D;
  //   2. Q -> the K and V tiles of stage 1 while the first key tile goes to
  //      stage 0; read qf[].  The first iteration's barrier orders these
  //      reads before the copy that refills stage 1.
  // Rows 32 w .. 32 w + 31 of the block sit in stage w / 2, rows
  // 32 (w % 2) .. of that stage.
  const int t_first = next_tile(0);
  const int r0 = qb * BQ;
  const bool upper = r0 + 64 < Nq;   // rows 64..127 of the block exist
  const int wrow = (wave & 1) * 32 * RB;
  auto copy_block = [&](const uint16_t* src, int dst0, int dst1) FA_INLINE {
    copy_async<T, NW>(src, r0, Nq, dst0, wave, lofs);
    if (upper) copy_async<T, NW>(src, r0 + 64, Nq, dst1, wave, lofs);
  };
  auto read_rows = [&](const char* rows, bf16x8 (&f)[NKK]) FA_INLINE {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      f[kk] = as_bf16x8(qrow < Nq ? *reinterpret_cast<const u32x4*>(rows + (oa.xr ^ (kk << 5)) + oa.ar)
                                  : zero_u32x4());
  };
  copy_block(p.dO + qhead, lds_addr(kvbuf), lds_addr(kvbuf) + 2 * KB);
  if constexpr (FUSED_D) copy_block(p.O + qhead, lds_addr(kvbuf) + KB, lds_addr(kvbuf) + 3 * KB);
  wait_vmem();
  __syncthreads();
  read_rows(kvbuf + (wave >> 1) * 2 * KB + wrow, of);
  form_d(kvbuf + ((wave >> 1) * 2 + 1) * KB + wrow);
  dsum_k = DROPOUT ? dsum * p.drop_keep : dsum;
  if constexpr (kFoldD) {
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = -dsum;
  }
  if (t_first < ntiles) {
    __syncthreads();   // every wavefront has read its dO and O rows
    copy_async<T, NW>(p.Q + qhead, r0, Nq, lds_addr(kvbuf) + 2 * KB, wave, lofs);
    if (upper) copy_async<T, NW>(p.Q + qhead, r0 + 64, Nq, lds_addr(kvbuf) + 3 * KB, wave, lofs);
    issue(t_first, 0);
    wait_vmem();
    __syncthreads();
    read_rows(kvbuf + (wave < 2 ? 2 : 3) * KB + wrow, qf);
  }
  int t = t_first;
  int stage = 0;
  // one loop body for both stages keeps dQ in one register set
  while (t < ntiles) {
    wait_vmem();
    __syncthreads();
    const int tn = next_tile(t + 1);
    if (tn < ntiles) issue(tn, stage ^ 1);
    // a tile entirely above this wavefront's causal diagonal contributes 0
    if (!(CAUSAL && t * BK > q0w + 31 + dlt)) compute(t);
    t = tn;
    // to the other stage's tiles
    const int flip = stage ? -2 * KB : 2 * KB;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      ra[kk] += flip;
      pin(ra[kk]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      ta[db][0] += flip;
      ta[db][1] += flip;
      pin(ta[db][0]);
      pin(ta[db][1]);
    }
    stage ^= 1;
  }

  // dQ leaves through the stage the loop did not end on: every wavefront
  // passed the barrier of the last tile, so none reads it, and no copy into
  // it is outstanding.  Rows 32 w .. 32 w + 31 of its K tile (w = 0, 1) or V
  // tile (w = 2, 3) serve wavefront w.  Block-sparse grids store straight
  // from the accumulator layout, which measured faster there.
  if constexpr (!SPARSE) {
    // with no key tile there was no loop barrier after the dO and O reads
    if (t_first >= ntiles) __syncthreads();
    if (q0w < Nq) {
      char* st = kvbuf + (2 * stage + (wave < 2 ? 0 : 1)) * KB + (wave & 1) * 32 * RB;
      store_rows_staged<D>(st, dq, DROPOUT ? p.scale * p.drop_scale : p.scale,
                           p.dQ + qhead + (size_t)q0w * D, Nq - q0w, lane);
    }
  } else if (qrow < Nq) {
    uint16_t* dQh = p.dQ + qhead + (size_t)qrow * D;
    const float sc = DROPOUT ? p.scale * p.drop_scale : p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<u32x2*>(dQh + db * 32 + qd * 8 + g * 4) =
            pack_bf16x4(dq[db][qd * 4 + 0] * sc, dq[db][qd * 4 + 1] * sc,
                        dq[db][qd * 4 + 2] * sc, dq[db][qd * 4 + 3] * sc);
  }
}

hipError_t launch_bwd_dsum(const BwdParams& p, int d, hipStream_t stream) {
  const long long rows = (long long)p.BH * p.Nq;
  if (d == 64) {
    constexpr int RPB = 256 / (64 / 8);
    hipLaunchKernelGGL((dsum_kernel<64>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       stream, p, rows);
  } else {
    constexpr int RPB = 256 / (128 / 8);
    hipLaunchKernelGGL((dsum_kernel<128>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                       0, stream, p, rows);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_dkdv_t(const BwdParams& p, bool dropout, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)p.nkb * p.BH));
  if (dropout)
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, SPARSE, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, SPARSE, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_dq_t(const BwdParams& p, bool fused_d, bool dropout,
                              hipStream_t stream) {
  const dim3 grid((unsigned)((long long)p.nqb * p.BH));
  if (dropout)   // only the fused form (fa_bwd's) has a dropout instantiation
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL, SPARSE, true, true>), grid, dim3(256), 0, stream,
                       p);
  else if (fused_d)
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL, SPARSE, true, false>), grid, dim3(256), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL, SPARSE, false, false>), grid, dim3(256), 0, stream,
                       p);
  return hipGetLastError();
}

#define FA_DISPATCH(FN, d, causal, sparse, ...)                                           \
  ((d) == 64 ? ((causal) ? ((sparse) ? FN<64, true, true>(__VA_ARGS__)                    \
                                     : FN<64, true, false>(__VA_ARGS__))                  \
                         : ((sparse) ? FN<64, false, true>(__VA_ARGS__)                   \
                                     : FN<64, false, false>(__VA_ARGS__)))                \
             : ((causal) ? ((sparse) ? FN<128, true, true>(__VA_ARGS__)                   \
                                     : FN<128, true, false>(__VA_ARGS__))                 \
                         : ((sparse) ? FN<128, false, true>(__VA_ARGS__)                  \
                                     : FN<128, false, false>(__VA_ARGS__))))

hipError_t launch_bwd_dkdv(const BwdParams& p, int d, bool causal, bool sparse, bool dropout,
                           hipStream_t stream) {
  return FA_DISPATCH(launch_dkdv_t, d, causal, sparse, p, dropout, stream);
}

hipError_t launch_bwd_dq(const BwdParams& p, int d, bool causal, bool sparse, bool fused_d,
                         bool dropout, hipStream_t stream) {
  if (dropout && !fused_d) return hipErrorInvalidValue;
  return FA_DISPATCH(launch_dq_t, d, causal, sparse, p, fused_d, dropout, stream);
}

// ---------------------------------------------------------------------------
// Scratch of fa_bwd_noalloc: D_i for up to kNoallocMaxRows query rows.  In
// host code the name `scratch` denotes a host-side stand-in, not the device
// array, so host code never passes it to a kernel or a copy: it uses the
// address hipGetSymbolAddress returns, looked up once per device (with that
// device current) and kept.  Every fa_bwd_noalloc call on a GPU shares that
// GPU's array; D is fully written by the dQ launch before the dK/dV launch
// reads it, so nothing needs clearing, and calls that overlap on one GPU
// (other streams) race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kNoallocMaxRows];

hipError_t noalloc_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* a = addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    a = addr[dev].load(std::memory_order_relaxed);
    if (a == nullptr) {
      void* sym = nullptr;
      e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      a = static_cast<float*>(sym);
      addr[dev].store(a, std::memory_order_release);
    }
  }
  *ptr = a;
  return hipSuccess;
}

}  // namespace fa
