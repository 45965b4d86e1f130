// Kernel parameter blocks and launchers, shared by the host entry points
// (fa_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* LSE;
  const uint8_t* blockmask;  // nullptr unless block-sparse
  int BH;                    // batch * heads
  int Nq, Nk;                // query rows, key rows (equal for self attention)
  int nqb;                   // ceil(Nq / 128) query blocks
  int mask_block;            // block-mask granularity (multiple of 128)
  int nbm;                   // ceil(Nk / mask_block): row stride of the block mask
  float scale_log2;          // scale * log2(e) (FP8: scale * q_descale * k_descale * log2(e))
  float v_descale;           // FP8: factor of every V element (1 otherwise)
  // split-KV (nsplit > 1): partial results [nsplit][BH][Nq][D] and [nsplit][BH][Nq]
  int nsplit, tiles_per_split;
  float* Opart;
  float* LSEpart;
  // dropout on P (read only by the dropout kernels): element (i, j) of head bh
  // is kept iff 16-bit half e % 2 of philox4x32_10(j/4, i/2, bh, drop_offset;
  // seed)[e / 2], e = 4 (i % 2) + j % 4, is >= drop_thresh
  uint32_t drop_thresh;      // floor(p * 2^16)
  float drop_scale;          // 1 / (1 - p): the kept probabilities' factor, applied to O at the end
  uint32_t seed_lo, seed_hi, drop_offset;
};

struct BwdParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* O;
  const uint16_t* dO;
  const float* LSE;
  float* Dsum;               // workspace: D_i = sum_k dO_ik O_ik
  uint16_t* dQ;
  uint16_t* dK;
  uint16_t* dV;
  const uint8_t* blockmask;
  int BH;
  int Nq, Nk;                // query rows, key rows
  int nqb;                   // ceil(Nq / 128) query blocks for the dQ kernel
  int nkb;                   // ceil(Nk / 128) key blocks for the dK/dV kernel
  int mask_block;
  int nbm;                   // ceil(Nk / mask_block): row stride of the block mask
  float scale;               // softmax scale
  float scale_log2;          // scale * log2(e)
  // dropout on P (read only by the dropout kernels): element (i, j) of head bh
  // is kept iff 16-bit half e % 2 of philox4x32_10(j/4, i/2, bh, drop_offset;
  // seed)[e / 2], e = 4 (i % 2) + j % 4, is >= drop_thresh
  uint32_t drop_thresh;      // floor(p * 2^16)
  float drop_scale;          // 1 / (1 - p), applied to dV, dK and dQ at the end
  float drop_keep;           // 1 - p: D is taken times this inside the loops
  uint32_t seed_lo, seed_hi, drop_offset;
};

// dropout: the DROPOUT instantiation (p.drop_* and p.seed_* must be set);
// otherwise p.nsplit > 1 selects split-KV (p.Opart / p.LSEpart) plus the merge
hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool sparse, bool dropout,
                      hipStream_t stream);
// FP8 forward (E4M3 Q, K, V; p.scale_log2 and p.v_descale carry the descales); d = 64, 128
hipError_t launch_fwd_fp8(const FwdParams& p, int d, bool causal, bool sparse,
                          hipStream_t stream);
// keep[bh][i][j] (uint8) of the dropout stream set in p (BH, Nq, Nk, drop_*, seed_*)
hipError_t launch_dropout_keep_mask(const FwdParams& p, uint8_t* keep, hipStream_t stream);
hipError_t launch_bwd_dsum(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, bool causal, bool sparse, bool dropout,
                           hipStream_t stream);
// fused_d: also form D_i and store it in p.Dsum (else read it from there);
// dropout: the DROPOUT instantiation, which exists only with fused_d
hipError_t launch_bwd_dq(const BwdParams& p, int d, bool causal, bool sparse, bool fused_d,
                         bool dropout, hipStream_t stream);

// Allocation-free backward: D lives in a static device array of
// kNoallocMaxRows floats (one per query row, 16 MiB) that every GPU the
// library runs on holds until the process ends.  noalloc_scratch() returns
// that array's address on the current device (looked up once per device with
// hipGetSymbolAddress and cached).
constexpr long long kNoallocMaxRows = 1LL << 22;
hipError_t noalloc_scratch(float** ptr);

}  // namespace fa
