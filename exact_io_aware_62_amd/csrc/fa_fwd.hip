// Forward kernel: O = softmax(scale * Q K^T + mask) V and LSE, one fused pass.
//
// Method (FlashAttention-NeurIPS22 digest, "核心方法": tiling + online softmax
// with a running row maximum m and row sum l merged block by block, and
// matmul + mask + softmax + matmul fused in one kernel), organised the way
// FlashAttention-2 does it (FlashAttention-2 wiki, "技术架构与工作原理"):
//   * item 2: the grid runs over (query block x batch*head), so one head is
//     spread over many compute units;
//   * item 3: each wavefront owns whole query rows, so the softmax row
//     reductions never leave the wavefront;
//   * item 1: the 1/l division is deferred to the epilogue and the softmax
//     scale is folded into a single exp2 argument.
//
// Work split (gfx950): a workgroup is 4 wavefronts and 128 query rows; each
// wavefront owns 32 rows, held in registers.  Key/value tiles of 64 rows are
// copied HBM -> LDS asynchronously (global_load_lds), K and V each
// double-buffered.
//
// The scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16
// matrix cores, so that every lane holds one query row (lanes r and r + 32
// share a row and split its keys).  Row max and row sum are then in-lane
// work plus one exchange between the two lane halves.  The probabilities
// stay in registers and feed O^T += V^T P^T as the B operand directly; the
// V^T operand is read from the natural V tile with the LDS transpose read.
//
// Software pipeline.  A matrix-core op runs for 32 cycles, during which the
// same wavefront can issue independent vector ops; the exp2 work of the
// softmax (about half the matrix time at d = 128) therefore hides behind
// matrix work only if the two are interleaved in one instruction stream.
// Iteration i (tile i, K_i in LDS, V_{i-1} and the packed P_{i-1} held over
// from iteration i-1):
//   phase A  S_i^T = K_i Q^T on the matrix cores (operands read ahead);
//            then the mask, if the tile needs one;
//   phase B  O^T += V_{i-1}^T P_{i-1}^T on the matrix cores, interleaved with
//            tile i's softmax: its row max under the first two products,
//            then P_i = exp2(S_i c - m), the fp32 row sum and the bf16
//            packing of P_i under the rest; then the rare rescale of O.
// The last tile's P V product runs alone after the loop.  Masked tiles
// (causal diagonal, ragged end) are the last tiles of a row block, so the
// mask branch sits between the phases, outside the interleaved code.

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// DROPOUT: P is multiplied by keep / (1 - p) before the P V product (the row
// sum, and with it LSE, stays that of the plain softmax).  Inside the loop the
// dropped probabilities are only zeroed; the common factor 1 / (1 - p) is
// applied once, with 1 / l, in the epilogue.  The keep bits of a tile come
// from the head's Philox stream (DropoutStream) and are drawn while the
// tile's scores are on the matrix cores.
// MODE 2 (split-KV): the key tiles of a query block are split into p.nsplit
// ranges of p.tiles_per_split tiles, one workgroup each; a workgroup writes
// its normalised partial O (fp32) and partial LSE to p.Opart / p.LSEpart, and
// combine_kernel merges the ranges with the log-sum-exp rule.
// Two wavefronts per SIMD at d = 128, three at d = 64 (168 registers: left to
// itself the compiler lets the sparse dropout form grow just past that).
template <int D, bool CAUSAL, bool SPARSE, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2))) void fwd_kernel(FwdParams p) {
  constexpr bool DROPOUT = MODE == 1, SPLIT = MODE == 2;
  constexpr int BQ = 128, BK = 64, NW = 4;
  constexpr float kSlack = 8.0f;
  constexpr int NDB = D / 32;   // 32-wide column blocks of O^T
  constexpr int NKK = D / 16;   // k-steps over the head dimension
  using T = LdsTile<BK, D>;
  constexpr int RB = T::kRowBytes;
  constexpr int TB = T::kBytes;
  // K tiles in kbuf0/kbuf1, V tiles in vbuf0/vbuf1.  Four separate arrays,
  // not one: the compiler can then tell that a read of one buffer does not
  // touch the buffer an outstanding LDS-DMA copy is filling, and does not
  // make the read wait for that copy.
  __shared__ __attribute__((aligned(1024))) char kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf0[TB];
  __shared__ __attribute__((aligned(1024))) char vbuf1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockCoord bc = block_coord(SPLIT ? p.nqb * p.nsplit : p.nqb, !CAUSAL);
  const int qblk = SPLIT ? bc.blk / p.nsplit : bc.blk;
  const int split = SPLIT ? bc.blk - qblk * p.nsplit : 0;
  // heaviest query blocks first under the causal mask
  const int qb = CAUSAL ? (p.nqb - 1 - qblk) : qblk;
  // Nq queries, Nk keys; under the causal mask query i sees key j iff
  // j <= i + dlt (the queries are the last Nq positions of the key sequence)
  const int Nq = p.Nq, Nk = p.Nk, dlt = Nk - Nq;
  const size_t qhead = (size_t)bc.bh * Nq * D, khead = (size_t)bc.bh * Nk * D;
  const uint16_t* __restrict__ Qh = p.Q + qhead;
  const uint16_t* __restrict__ Kh = p.K + khead;
  const uint16_t* __restrict__ Vh = p.V + khead;

  const int q0w = qb * BQ + wave * 32;   // first query row of this wavefront
  const int qrow = q0w + r;              // this lane's query row

  // Q fragments (B operand of S^T = K Q^T): row qrow, columns kk*16 + g*8 ..+7,
  // filled from LDS before the first tile
  bf16x8 qf[NKK];

  // key range and tile schedule
  const int kend = CAUSAL ? max(0, min(Nk, (qb + 1) * BQ + dlt)) : Nk;
  // tiles [tbeg, ntiles): all of the visible range, or this workgroup's split of it
  const int tbeg = SPLIT ? split * p.tiles_per_split : 0;
  const int ntiles = SPLIT ? min((kend + BK - 1) / BK, tbeg + p.tiles_per_split)
                           : (kend + BK - 1) / BK;
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
  // wavefront-uniform tile predicates
  auto needs_mask = [&](int t) FA_INLINE {
    return (CAUSAL && t * BK + BK - 1 > q0w + dlt) || (t * BK + BK > Nk);
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float m_run = kNegBig;   // running max of scaled scores (log2 domain)
  float l_run = 0.f;       // running partial row sum (this lane's keys)
  const float c = p.scale_log2;
  DropoutStream ds_;
  if constexpr (DROPOUT) {
    ds_.seed_lo = p.seed_lo;
    ds_.seed_hi = p.seed_hi;
    ds_.bh = (uint32_t)bc.bh;
    ds_.offset = p.drop_offset;
    ds_.thresh = p.drop_thresh;
  }
  // Dropout: one draw decides four keys of this lane's row and of the row of
  // lane r ^ 1 (rows 2 ig, 2 ig + 1: q0w is even).  Key group u = kb*4 + m
  // (keys k0 + kb*32 + m*8 + g*4 + 0..3) is drawn by the lane of the pair
  // whose row parity equals u's: draw v of a tile takes group u = 2v + (r & 1),
  // and each lane hands the other row's two words to its partner.  kx[2u + h]
  // holds drop_mask() for keys 2h, 2h + 1 of group u in this lane's row,
  // which is word q = 2(u % 2) + h of P's packed B operand pb[u / 2].  The
  // previous tile's entries are dead by then (its P was packed in the
  // previous iteration), so the draws write kx in place.
  uint32_t kx[DROPOUT ? 16 : 1];
  auto draw_keep = [&](int tc, int v) FA_INLINE {
    const int odd = qrow & 1;
    const int u = 2 * v + odd, kb = u >> 2, m = u & 3;
    const u32x4 w = philox4x32_10((uint32_t)(tc * (BK / 4) + kb * 8 + m * 2 + g),
                                  (uint32_t)qrow >> 1, ds_.bh, ds_.offset, ds_.seed_lo,
                                  ds_.seed_hi);
    // words 0, 1: the block's even row; words 2, 3: its odd row
    const uint32_t tt = ds_.thresh * 0x10001u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t ev = drop_mask(w[h], tt, 0x10001u), od = drop_mask(w[2 + h], tt, 0x10001u);
      // both lanes of the pair swap both words (a swap under a lane-dependent
      // condition would read a lane that is switched off); then group 2v takes
      // the even lane's draw and group 2v + 1 the odd lane's
      const uint32_t sev = pair_swap(ev), sod = pair_swap(od);
      kx[4 * v + h] = odd ? sod : ev;
      kx[4 * v + 2 + h] = odd ? od : sev;
      pin(kx[4 * v + h]);
      pin(kx[4 * v + 2 + h]);
    }
  };
  // P's packed B operand entry q with the dropped probabilities zeroed (1 / (1 - p)
  // comes at the end)
  auto pack_p = [&](const f32x16& s, int base, int q) FA_INLINE -> bf16x8 {
    bf16x8 r = pack_c8(s, base);
    if constexpr (DROPOUT) {
      u32x4 wv = __builtin_bit_cast(u32x4, r);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] &= kx[4 * q + i];
      r = __builtin_bit_cast(bf16x8, wv);
    }
    return r;
  };

  const auto lofs = T::template lane_offsets<NW>(wave, lane);
  auto load_k = [&](int t, int buf) FA_INLINE {
    T::template copy<NW>(Kh, t * BK, Nk, buf ? kbuf1 : kbuf0, wave, lofs);
  };
  auto load_v = [&](int t, int buf) FA_INLINE {
    T::template copy<NW>(Vh, t * BK, Nk, buf ? vbuf1 : vbuf0, wave, lofs);
  };

  // P = exp2(S c - m), packed to the bf16 B operands of the PV product:
  // k-step ks2 of key block kb uses C registers 8*ks2 .. 8*ks2+7.
  auto exponentiate = [&](f32x16 (&s)[2], bf16x8 (&pb)[4]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = exp2_fast(__builtin_fmaf(s[kb][i], c, -m_run));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) pb[kb * 2 + ks2] = pack_p(s[kb], 8 * ks2, kb * 2 + ks2);
  };
  auto rowsum = [&](const f32x16 (&s)[2]) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        a0 += s[kb][i];
        a1 += s[kb][i + 1];
        a2 += s[kb][i + 2];
        a3 += s[kb][i + 3];
      }
    return (a0 + a1) + (a2 + a3);
  };
  f32x16 sc[2];          // scores of the current tile
  // bf16 probabilities: phase B reads entry q for the previous tile's P V
  // product and then overwrites it with the current tile's packed P.
  bf16x8 pb[4];

  // Scores above this wavefront's causal diagonal or past the last key -> -inf.
  auto mask = [&](int tc) FA_INLINE {
    if (needs_mask(tc)) {
      // register i of key block kb holds key k0 + g*4 + kb*32 + (i/4)*8 + i%4;
      // compare the constant part against one per-lane bound
      // lane id recomputed here (two vector ops) rather than kept live
      const int ln = lane_id();
      const int kl = tc * BK + (ln >> 5) * 4;
      const int lim = CAUSAL ? min(Nk - 1, q0w + (ln & 31) + dlt) - kl : Nk - 1 - kl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sc[kb][i] = -INFINITY;
    }
  };
  // Row max of the tile as a tree of three-input maxima (depth 4 instead of a
  // chain of 16), in two parts so that each part fits under one matrix
  // product: 32 values -> 12 -> 4 in part 1, then 4 -> 1 and the exchange
  // with the other lane half in part 2.  Raw max instructions: no
  // canonicalising of the products' results, no regrouping.
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
  // The running maximum only moves when a score exceeds it by more than
  // kSlack (log2 units): every exp2 argument then stays below kSlack, far
  // inside fp32 and bf16 range, and since the final 1/l and LSE use the
  // same m the result is the same for any such m.  With scores of a few
  // units this rescales O about once per row.  Returns the factor the
  // accumulated O must be scaled by (1 if unmoved).
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

  const OperandAddr<T> oa = operand_addr<T>(lane);
  // V^T operand for product j of the PV step: key block kb = j / (2 NDB),
  // k-step ks2 = (j / NDB) % 2, output column block db = j % NDB.  The
  // lane-dependent offsets are loop-invariant; with compile-time buffers
  // the compiler keeps them in registers and folds the rest into the
  // instruction's immediate offset.
  // The lane parts of those reads, one per output column block and half,
  // computed once (xad is opaque, so the compiler keeps them in registers
  // instead of redoing the add for every read); the buffer, key block and
  // k-step offsets then fold into each read's immediate offset.
  int vofs[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    vofs[db][0] = xad(oa.xt, db << 6, oa.at0);
    vofs[db][1] = xad(oa.xt, db << 6, oa.at1);
  }
  auto vread = [&](const char* vt, int j) FA_INLINE {
    const int kb = j / (2 * NDB), ks2 = (j / NDB) & 1, db = j % NDB;
    const char* vk = vt + (kb * 32 + 16 * ks2) * RB;
    return bf16x8_from_halves(lds_tr_b64(vk + vofs[db][0]), lds_tr_b64(vk + vofs[db][1]));
  };
  // phase B: O += P_prev V_prev on the matrix cores, interleaved with the
  // current tile's softmax: its row max under the first products, then
  // P = exp2(S c - m), its bf16 packing and row sum under the rest.
  // Program order is the issue order (each step is fenced; pin() keeps the
  // vector work where it is placed): V^T fragments are read PF products ahead.
  auto phaseB = [&](const char* vt, float& alpha) FA_INLINE {
    constexpr int NJ = 4 * NDB, PF = 2, J0 = 2;   // exps in products J0 .. NJ-1
    bf16x8 vfr[NJ];
    __builtin_amdgcn_sched_barrier(0);
    // Issue priority 1 while the softmax runs under the products: of the two
    // wavefronts sharing a SIMD, the one interleaving vector work with its
    // P V products goes first, and the other one's score products (phase A,
    // matrix work only) fill the matrix core around it.  Measured 2-3%
    // faster than equal priority; raising phase A instead measured slower.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < PF; ++j) vfr[j] = vread(vt, j);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kb = j / (2 * NDB), ks2 = (j / NDB) & 1, db = j % NDB;
      oacc[db] = mfma32x32x16(vfr[j], pb[kb * 2 + ks2], oacc[db]);
      if (j + PF < NJ) vfr[j + PF] = vread(vt, j + PF);
      if (j == 0) rowmax_part1();
      if (j == 1) alpha = rowmax_part2();
      // P entry q is last read by product NDB q + NDB - 1; its exps come later
      // (entry q's exps end by product J0 + (8q + 8) (NJ - J0) / 32 - 1 >= NDB q + NDB - 1)
      constexpr int NE = NJ - J0;
      // this slot's exponentials first, then their sums and packs: a sum
      // right after the exponential it reads would need a wait state
      constexpr int EMAX = (32 + NE - 1) / NE + 1;
      const int e0 = j < J0 ? 0 : (j - J0) * 32 / NE;
      const int e1 = j < J0 ? 0 : (j + 1 - J0) * 32 / NE;
      float pes[EMAX];
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        const int b = e >> 4, i = e & 15;
        pes[e - e0] = exp2_fast(__builtin_fmaf(sc[b][i], c, -m_run));
        pin(pes[e - e0]);
      }
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        const int b = e >> 4, i = e & 15;
        const float pe = pes[e - e0];
        sc[b][i] = pe;
        // the row sum is taken over the fp32 probabilities: a sum of the
        // bf16-rounded ones would move LSE by up to 2^-9 on short rows
        if (e & 1) {
          a1 = e == 1 ? pe : a1 + pe;
          pin(a1);
        } else {
          a0 = e == 0 ? pe : a0 + pe;
          pin(a0);
        }
        if ((i & 7) == 7) {
          pb[b * 2 + (i >> 3)] = pack_p(sc[b], i - 7, b * 2 + (i >> 3));
          pin(pb[b * 2 + (i >> 3)]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    return a0 + a1;
  };
  // O += P V alone (the last product of a wavefront), same issue order
  auto pv_only = [&](const char* vt) FA_INLINE {
    constexpr int NJ = 4 * NDB, PF = 2;
    bf16x8 vfr[NJ];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) vfr[j] = vread(vt, j);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int kb = j / (2 * NDB), ks2 = (j / NDB) & 1, db = j % NDB;
      oacc[db] = mfma32x32x16(vfr[j], pb[kb * 2 + ks2], oacc[db]);
      if (j + PF < NJ) vfr[j + PF] = vread(vt, j + PF);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // scores of the tile in K buffer kt (phase A); K fragments read PF ahead
  auto phaseA = [&](const char* kt, int tc) FA_INLINE {
    // product j: k-step kk = j / 2 of key block kb = j % 2 (two independent
    // accumulation chains); one address per k-step serves both blocks
    constexpr int NJ = 2 * NKK, PF = 4;
    bf16x8 kfr[NJ];
    auto kread = [&](int j) FA_INLINE {
      const char* a = kt + (j & 1) * 32 * RB + (oa.xr ^ ((j >> 1) << 5)) + oa.ar;
      kfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(a));
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) kread(j);
    sc[0] = zero16();
    sc[1] = zero16();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      sc[j & 1] = mfma32x32x16(kfr[j], qf[j >> 1], sc[j & 1]);
      if (j + PF < NJ) kread(j + PF);
      if constexpr (DROPOUT) {
        // four draws per tile, spread over the score products
        if (j % (NJ / 4) == 0) draw_keep(tc, j / (NJ / 4));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto rescale = [&](float alpha) FA_INLINE {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
  };

  // One iteration for tile tc, whose K is in K buffer PAR; the previous
  // tile's V is in V buffer 1 - PAR and its probabilities in pb.  FIRST:
  // there is no previous tile (O is still zero).
  const bool wave_has_rows = q0w < Nq;
  auto iteration = [&](auto parc, auto firstc, int& tc, int& tn) FA_INLINE {
    constexpr int PAR = decltype(parc)::value;
    constexpr bool FIRST = decltype(firstc)::value;
    wait_vmem();
    __syncthreads();
    const int tn2 = tn < ntiles ? next_tile(tn + 1) : ntiles;
    if (tn < ntiles) load_k(tn, 1 - PAR);
    load_v(tc, PAR);
    // A tile entirely above this wavefront's causal diagonal is processed
    // like any other: the mask sets all its scores to -inf, so its P is 0
    // and O is unchanged.  One code path keeps O in one register set.
    // (Split-KV serves decoding, where a query block has few rows: a
    // wavefront with none only helps copy the tiles.)
    if (!SPLIT || wave_has_rows) {
      phaseA(PAR ? kbuf1 : kbuf0, tc);
      mask(tc);
      if constexpr (FIRST) {
        rowmax_part1();
        rowmax_part2();
        exponentiate(sc, pb);
        l_run += rowsum(sc);
      } else {
        float alpha;
        const float psum = phaseB(PAR ? vbuf0 : vbuf1, alpha);   // scales l_run by alpha
        l_run += psum;
        rescale(alpha);
      }
    }
    tc = tn;
    tn = tn2;
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int tc = next_tile(tbeg);
  int tn = tc < ntiles ? next_tile(tc + 1) : ntiles;
  if (tc < ntiles) {
    // The workgroup's 128 Q rows come in as whole-row copies (a lane reading
    // its own row straight from global memory would touch 32 rows per load)
    // into K buffer 1 (rows 0..63) and V buffer 0 (rows 64..127), both unused
    // until the first tile's copies; each wavefront then reads its 32 rows
    // with the conflict-free row read.  The first iteration's barrier orders
    // these reads before the copies that refill the two buffers.
    T::template copy<NW>(Qh, qb * BQ, Nq, kbuf1, wave, lofs);
    if (qb * BQ + 64 < Nq) T::template copy<NW>(Qh, qb * BQ + 64, Nq, vbuf0, wave, lofs);
    load_k(tc, 0);
    wait_vmem();
    __syncthreads();
    {
      const char* qt = (wave < 2 ? kbuf1 : vbuf0) + (wave & 1) * 32 * RB;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        qf[kk] = as_bf16x8(qrow < Nq ? *reinterpret_cast<const u32x4*>(qt + (oa.xr ^ (kk << 5)) + oa.ar)
                                     : zero_u32x4());
    }
    iteration(P0{}, std::true_type{}, tc, tn);
    // whole pairs of tiles: the loop body has one entry and one exit, which
    // keeps O in one register set across both halves
    while (tn < ntiles) {
      iteration(P1{}, std::false_type{}, tc, tn);
      iteration(P0{}, std::false_type{}, tc, tn);
    }
    const bool odd = tc < ntiles;   // one tile left (parity 1)
    if (odd) iteration(P1{}, std::false_type{}, tc, tn);
    // the last tile's P V product
    wait_vmem();
    __syncthreads();
    if (!SPLIT || wave_has_rows) {
      if (odd) pv_only(vbuf1);
      else pv_only(vbuf0);
    }
  }

  // epilogue: combine the two lane halves' partial sums, divide once
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? (DROPOUT ? p.drop_scale : 1.0f) / l_tot : 0.f;
  if constexpr (SPLIT) {
    if (qrow < Nq) {
      const size_t prow = ((size_t)split * p.BH + bc.bh) * Nq + qrow;
      float* Op = p.Opart + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = oacc[db][qd * 4 + e] * inv;
          *reinterpret_cast<f32x4*>(Op + db * 32 + qd * 8 + g * 4) = v;
        }
      if (g == 0)
        p.LSEpart[prow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  // O leaves through the K buffers, which nothing reads after the last
  // tile's scores (and the barrier before the last P V product): rows
  // 32 w .. 32 w + 31 of the two K tiles for wavefront w
  if (q0w < Nq) {
    char* stage = (wave < 2 ? kbuf0 : kbuf1) + (wave & 1) * 32 * RB;
    store_rows_staged<D>(stage, oacc, inv, p.O + qhead + (size_t)q0w * D, Nq - q0w, lane);
  }
  if (qrow < Nq && g == 0)
    p.LSE[(size_t)bc.bh * Nq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// Merge of the split-KV partial results of one row: LSE = log sum_s exp(LSE_s)
// and O = sum_s exp(LSE_s - LSE) O_s (each O_s is normalised by its own row
// sum), O rounded to bf16.  A row with no visible key in any split gets
// O = 0, LSE = -inf.  Thread = four columns of one row.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(FwdParams p, long long rows) {
  constexpr int TPR = D / 4, RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;
  const int ns = p.nsplit;
  float m = -INFINITY;
  for (int sidx = 0; sidx < ns; ++sidx) m = fmaxf(m, p.LSEpart[(size_t)sidx * rows + row]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int sidx = 0; sidx < ns; ++sidx) {
      const float w = __expf(p.LSEpart[(size_t)sidx * rows + row] - m);
      wsum += w;
      const f32x4 o = *reinterpret_cast<const f32x4*>(p.Opart + ((size_t)sidx * rows + row) * D + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, o[e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<u32x2*>(p.O + row * D + col) =
      pack_bf16x4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (col == 0) p.LSE[row] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_t(const FwdParams& p, int mode, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)p.nqb * p.BH * (mode == 2 ? p.nsplit : 1)));
  if (mode == 1)
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, SPARSE, 1>), grid, dim3(256), 0, stream, p);
  else if (mode == 2)
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, SPARSE, 2>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, SPARSE, 0>), grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mode != 2) return e;
  const long long rows = (long long)p.BH * p.Nq;
  constexpr int RPB = 256 / (D / 4);
  hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, p, rows);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool sparse, bool dropout,
                      hipStream_t stream) {
  const int mode = dropout ? 1 : (p.nsplit > 1 ? 2 : 0);
  if (d == 64) {
    if (causal) return sparse ? launch_fwd_t<64, true, true>(p, mode, stream)
                              : launch_fwd_t<64, true, false>(p, mode, stream);
    return sparse ? launch_fwd_t<64, false, true>(p, mode, stream)
                  : launch_fwd_t<64, false, false>(p, mode, stream);
  }
  if (causal) return sparse ? launch_fwd_t<128, true, true>(p, mode, stream)
                            : launch_fwd_t<128, true, false>(p, mode, stream);
  return sparse ? launch_fwd_t<128, false, true>(p, mode, stream)
                : launch_fwd_t<128, false, false>(p, mode, stream);
}

// Keep mask of the dropout stream, keep[bh][i][j] = 1 or 0, for inspection and
// tests: one thread per block of two queries and four keys (one Philox draw).
__global__ __launch_bounds__(256) void dropout_keep_mask_kernel(FwdParams p, uint8_t* keep,
                                                               long long groups) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= groups) return;
  const int ng = (p.Nk + 3) / 4, nig = (p.Nq + 1) / 2;
  const long long bhig = gid / ng;           // bh * nig + ig
  const int jg = (int)(gid - bhig * ng);
  const int bh = (int)(bhig / nig), ig = (int)(bhig - (long long)bh * nig);
  DropoutStream ds;
  ds.seed_lo = p.seed_lo;
  ds.seed_hi = p.seed_hi;
  ds.bh = (uint32_t)bh;
  ds.offset = p.drop_offset;
  ds.thresh = p.drop_thresh;
  const uint32_t bits = ds.keep8((uint32_t)jg, (uint32_t)ig);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = 2 * ig + h;
    if (i >= p.Nq) break;
    uint8_t* out = keep + ((long long)bh * p.Nq + i) * p.Nk + 4 * jg;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (4 * jg + t < p.Nk) out[t] = (uint8_t)((bits >> (4 * h + t)) & 1u);
  }
}

hipError_t launch_dropout_keep_mask(const FwdParams& p, uint8_t* keep, hipStream_t stream) {
  const long long groups = (long long)p.BH * ((p.Nq + 1) / 2) * ((p.Nk + 3) / 4);
  const long long blocks = (groups + 255) / 256;
  hipLaunchKernelGGL(dropout_keep_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p,
                     keep, groups);
  return hipGetLastError();
}

}  // namespace fa
