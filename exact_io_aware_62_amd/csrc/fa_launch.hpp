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
  int N;                     // sequence length
  int nqb;                   // ceil(N / 128) query blocks
  int mask_block;            // block-mask granularity (multiple of 128)
  int nbm;                   // ceil(N / mask_block)
  float scale_log2;          // scale * log2(e)
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
  int N;
  int nqb;                   // ceil(N / 128)
  int nkb;                   // ceil(N / 128) key blocks for the dK/dV kernel
  int mask_block;
  int nbm;
  float scale;               // softmax scale
  float scale_log2;          // scale * log2(e)
};

hipError_t launch_fwd(const FwdParams& p, int d, bool causal, bool sparse, hipStream_t stream);
hipError_t launch_bwd_dsum(const BwdParams& p, int d, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, int d, bool causal, bool sparse,
                           hipStream_t stream);
// fused_d: also form D_i and store it in p.Dsum (else read it from there)
hipError_t launch_bwd_dq(const BwdParams& p, int d, bool causal, bool sparse, bool fused_d,
                         hipStream_t stream);

}  // namespace fa
