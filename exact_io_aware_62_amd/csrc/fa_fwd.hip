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
// copied HBM -> LDS asynchronously (global_load_lds), double-buffered: the
// copy of tile t+1 is in flight while tile t is multiplied.
//
// The scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16
// matrix cores, so that every lane holds one query row (lanes r and r + 32
// share a row and split its keys).  Row max and row sum are then in-lane
// work plus one exchange between the two lane halves.  The probabilities
// stay in registers and feed O^T += V^T P^T as the B operand directly; the
// V^T operand is read from the natural V tile with the LDS transpose read.

#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int BQ = 128, BK = 64, NW = 4;
  constexpr int NDB = D / 32;   // 32-wide column blocks of O^T
  constexpr int NKK = D / 16;   // k-steps over the head dimension
  using T = LdsTile<BK, D>;
  constexpr int RB = T::kRowBytes;
  constexpr int STAGE = 2 * T::kBytes;   // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const BlockCoord bc = block_coord(p.BH);
  // heaviest query blocks first under the causal mask
  const int qb = CAUSAL ? (p.nqb - 1 - bc.blk) : bc.blk;
  const int N = p.N;
  const size_t head = (size_t)bc.bh * N * D;
  const uint16_t* __restrict__ Qh = p.Q + head;
  const uint16_t* __restrict__ Kh = p.K + head;
  const uint16_t* __restrict__ Vh = p.V + head;

  const int q0w = qb * BQ + wave * 32;   // first query row of this wavefront
  const int qrow = q0w + r;              // this lane's query row

  // Q fragments (B operand of S^T = K Q^T): row qrow, columns kk*16 + g*8 ..+7
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = as_bf16x8(qrow < N ? ldg16(Qh + (size_t)qrow * D + kk * 16 + g * 8)
                                : zero_u32x4());

  // key range and tile schedule
  const int kend = CAUSAL ? min(N, (qb + 1) * BQ) : N;
  const int ntiles = (kend + BK - 1) / BK;
  const int mrow = SPARSE ? (qb * BQ) / p.mask_block : 0;
  auto next_tile = [&](int t) -> int {
    if constexpr (SPARSE) {
      const uint8_t* mr = p.blockmask + (size_t)mrow * p.nbm;
      while (t < ntiles && mr[(t * BK) / p.mask_block] == 0) ++t;
    }
    return t;
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float m_run = kNegBig;   // running max of scaled scores (log2 domain)
  float l_run = 0.f;       // running partial row sum (this lane's keys)
  const float c = p.scale_log2;

  auto issue = [&](int t, int bufi) {
    char* st = lds + bufi * STAGE;
    T::template copy<NW>(Kh, t * BK, N, st, wave, lane);
    T::template copy<NW>(Vh, t * BK, N, st + T::kBytes, wave, lane);
  };

  auto compute = [&](auto bufc, int t) {
    constexpr int BUFI = decltype(bufc)::value;
    const char* kt = lds + BUFI * STAGE;
    const char* vt = kt + T::kBytes;
    const int k0 = t * BK;
    // this wavefront skips tiles that lie entirely above its diagonal
    if (CAUSAL && k0 > q0w + 31) return;
    // S^T (64 keys x 32 queries) as two 32x32 blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s[kb] = mfma32x32x16(lds_row_operand<T>(kt + kb * 32 * RB, r, 2 * kk + g), qf[kk],
                             s[kb]);
    }
    // mask: causal diagonal tile, or keys past the end of the sequence
    if ((CAUSAL && k0 + BK - 1 > q0w) || k0 + BK > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          if (key >= N || (CAUSAL && key > qrow)) s[kb][i] = -INFINITY;
        }
    }
    // online softmax update
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = exp2_fast(__builtin_fmaf(s[kb][i], c, -m_new));
        s[kb][i] = e;
        rs += e;
      }
    l_run = l_run * alpha + rs;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    // O^T += V^T P^T; k-step ks2 of key block kb uses C registers 8*ks2..+7
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const bf16x8 pb = pack_c8(s[kb], 8 * ks2);
        const char* vk = vt + (kb * 32 + 16 * ks2) * RB;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = bf16x8_from_halves(lds_tr_b64(vk + tr_offset<T>(0, db * 32, lane, 0)),
                                              lds_tr_b64(vk + tr_offset<T>(0, db * 32, lane, 1)));
          oacc[db] = mfma32x32x16(a, pb, oacc[db]);
        }
      }
  };

  int t = next_tile(0);
  if (t < ntiles) issue(t, 0);
  while (t < ntiles) {
    wait_vmem();
    __syncthreads();
    int tn = next_tile(t + 1);
    if (tn < ntiles) issue(tn, 1);
    compute(std::integral_constant<int, 0>{}, t);
    t = tn;
    if (t >= ntiles) break;
    wait_vmem();
    __syncthreads();
    tn = next_tile(t + 1);
    if (tn < ntiles) issue(tn, 0);
    compute(std::integral_constant<int, 1>{}, t);
    t = tn;
  }

  // epilogue: combine the two lane halves' partial sums, divide once
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* Oh = p.O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const u32x2 v = pack_bf16x4(oacc[db][qd * 4 + 0] * inv, oacc[db][qd * 4 + 1] * inv,
                                    oacc[db][qd * 4 + 2] * inv, oacc[db][qd * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(Oh + db * 32 + qd * 8 + g * 4) = v;
      }
    if (g == 0)
      p.LSE[(size_t)bc.bh * N + qrow] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  const long long blocks = (long long)p.nqb * p.BH;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, SPARSE>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool sparse, hipStream_t stream) {
  if (d == 64) {
    if (causal) return sparse ? launch_fwd_t<64, true, true>(p, stream)
                              : launch_fwd_t<64, true, false>(p, stream);
    return sparse ? launch_fwd_t<64, false, true>(p, stream)
                  : launch_fwd_t<64, false, false>(p, stream);
  }
  if (causal) return sparse ? launch_fwd_t<128, true, true>(p, stream)
                            : launch_fwd_t<128, true, false>(p, stream);
  return sparse ? launch_fwd_t<128, false, true>(p, stream)
                : launch_fwd_t<128, false, false>(p, stream);
}

}  // namespace fa
