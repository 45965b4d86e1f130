// C entry points of libfa: argument validation and kernel dispatch.
//
// Every check runs before the first HIP call, so invalid arguments never
// launch anything and can be exercised without a GPU.  See include/fa.h for
// the contract of each call.

#include "fa.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "fa_launch.hpp"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr long long kMaxI32 = 2147483647LL;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shapes only (Nq query rows, Nk key rows).  Sets *empty when there is
// nothing to compute (no query rows).
int check_shape(int B, int H, int Nq, int Nk, int d, bool* empty) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  for (const int n : {Nq, Nk}) {
    if ((long long)n * d > kMaxI32) return FA_ERR_UNSUPPORTED;
    const long long nb = ((long long)n + 127) / 128;
    if (nb * B * H > kMaxI32) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * n > kMaxI32) return FA_ERR_UNSUPPORTED;
  }
  *empty = (long long)B * H * Nq == 0;
  return FA_OK;
}

int check_shape(int B, int H, int N, int d, bool* empty) {
  return check_shape(B, H, N, N, d, empty);
}

// Shapes, scale and mask arguments.
int check_common(int B, int H, int Nq, int Nk, int d, float scale, const uint8_t* blockmask,
                 int mask_block, bool* empty) {
  const int rc = check_shape(B, H, Nq, Nk, d, empty);
  if (rc != FA_OK) return rc;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_UNSUPPORTED;
  if (blockmask != nullptr && (mask_block <= 0 || mask_block % 128 != 0))
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_common(int B, int H, int N, int d, float scale, const uint8_t* blockmask,
                 int mask_block, bool* empty) {
  return check_common(B, H, N, N, d, scale, blockmask, mask_block, empty);
}

bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned(p, 16)) return false;
  return true;
}

fa::BwdParams bwd_params(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* LSE, float* Dsum, int B, int H, int Nq,
                         int Nk, float scale, const uint8_t* blockmask, int mask_block, void* dQ,
                         void* dK, void* dV) {
  fa::BwdParams p;
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = static_cast<const uint16_t*>(K);
  p.V = static_cast<const uint16_t*>(V);
  p.O = static_cast<const uint16_t*>(O);
  p.dO = static_cast<const uint16_t*>(dO);
  p.LSE = LSE;
  p.Dsum = Dsum;
  p.dQ = static_cast<uint16_t*>(dQ);
  p.dK = static_cast<uint16_t*>(dK);
  p.dV = static_cast<uint16_t*>(dV);
  p.blockmask = blockmask;
  p.BH = B * H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.nqb = (Nq + 127) / 128;
  p.nkb = (Nk + 127) / 128;
  p.mask_block = blockmask ? mask_block : 128;
  p.nbm = (Nk + p.mask_block - 1) / p.mask_block;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  p.drop_thresh = 0;
  p.drop_scale = 1.f;
  p.drop_keep = 1.f;
  p.seed_lo = p.seed_hi = p.drop_offset = 0;
  return p;
}

fa::BwdParams bwd_params(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* LSE, float* Dsum, int B, int H, int N,
                         float scale, const uint8_t* blockmask, int mask_block, void* dQ,
                         void* dK, void* dV) {
  return bwd_params(Q, K, V, O, dO, LSE, Dsum, B, H, N, N, scale, blockmask, mask_block, dQ, dK,
                    dV);
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Dropout arguments: 0 <= p < 1 (finite).  p == 0 is no dropout at all.
int check_dropout(float p_drop) {
  if (!std::isfinite(p_drop) || p_drop < 0.f || p_drop >= 1.f) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// The kernels' dropout fields: drop iff the element's 16-bit Philox half is
// < floor(p * 2^16);
// kept values are multiplied by 1 / (1 - p) (fp32), which the kernels apply
// once to their accumulated outputs.
void set_dropout_keep(fa::FwdParams&, float) {}
void set_dropout_keep(fa::BwdParams& p, float p_drop) { p.drop_keep = 1.0f - p_drop; }

template <class Params>
void set_dropout(Params& p, float p_drop, uint64_t seed, uint32_t offset) {
  const double t = std::floor((double)p_drop * 65536.0);
  p.drop_thresh = t >= 65535.0 ? 0xFFFFu : (uint32_t)t;
  p.drop_scale = 1.0f / (1.0f - p_drop);
  set_dropout_keep(p, p_drop);
  p.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(seed >> 32);
  p.drop_offset = offset;
}

// Split-KV layout: how many key ranges per query block (1 = no split).  Asked
// for <= 0, the count aims at one workgroup per compute unit (256), with at
// least four and at most 256 64-key tiles per range; the count is then
// trimmed so that no range is empty.  Measured on decoding shapes (one query row per head,
// 2K-64K keys, 16-256 heads), one workgroup per CU read the cache 10-60%
// faster than 2, 4 or 8 per CU: more, shorter ranges spend their time on
// each workgroup's fixed costs, and fewer leave CUs idle.
int splitkv_splits(int B, int H, int Nq, int Nk, int requested, int* tiles_per_split) {
  const long long nqb = ((long long)Nq + 127) / 128;
  const long long tiles = ((long long)Nk + 63) / 64;
  const long long wg = nqb * B * H;
  long long s = requested;
  if (s <= 0) {
    constexpr long long kTargetWorkgroups = 256, kMaxTilesPerRange = 256;
    s = wg > 0 ? (kTargetWorkgroups + wg - 1) / wg : 1;
    s = std::max(s, (tiles + kMaxTilesPerRange - 1) / kMaxTilesPerRange);
    s = std::min(s, (tiles + 3) / 4);
  }
  s = std::max(1LL, std::min(s, std::max(1LL, tiles)));
  const long long tps = (tiles + s - 1) / s;
  s = tps > 0 ? (tiles + tps - 1) / tps : 1;
  *tiles_per_split = (int)std::max(1LL, tps);
  return (int)std::max(1LL, s);
}

size_t splitkv_bytes(int B, int H, int Nq, int d, int splits) {
  if (splits <= 1) return 0;
  return (size_t)splits * B * H * Nq * (size_t)(d + 1) * 4;
}

int fwd_impl(const void* Q, const void* K, const void* V, int B, int H, int Nq, int Nk, int d,
             float scale, int causal, const uint8_t* blockmask, int mask_block, float p_drop,
             uint64_t seed, uint32_t offset, void* O, float* LSE, hipStream_t stream,
             int num_splits = 1, void* workspace = nullptr, size_t workspace_bytes = 0) {
  bool empty = false;
  int rc = check_common(B, H, Nq, Nk, d, scale, blockmask, mask_block, &empty);
  if (rc != FA_OK) return rc;
  rc = check_dropout(p_drop);
  if (rc != FA_OK) return rc;
  if (empty) return FA_OK;
  if (!Q || !O || !LSE) return FA_ERR_NULL;
  if ((long long)B * H * Nk > 0 && (!K || !V)) return FA_ERR_NULL;   // no keys: O = 0
  if (!all_aligned16({Q, K, V, O}) || !aligned(LSE, 4)) return FA_ERR_UNSUPPORTED;

  fa::FwdParams p;
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = static_cast<const uint16_t*>(K);
  p.V = static_cast<const uint16_t*>(V);
  p.O = static_cast<uint16_t*>(O);
  p.LSE = LSE;
  p.blockmask = blockmask;
  p.BH = B * H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.nqb = (Nq + 127) / 128;
  p.mask_block = blockmask ? mask_block : 128;
  p.nbm = (Nk + p.mask_block - 1) / p.mask_block;
  p.scale_log2 = scale * kLog2e;
  p.v_descale = 1.f;
  set_dropout(p, p_drop, seed, offset);
  p.nsplit = 1;
  p.tiles_per_split = 0;
  p.Opart = p.LSEpart = nullptr;
  if (num_splits != 1 && p_drop == 0.f) {
    p.nsplit = splitkv_splits(B, H, Nq, Nk, num_splits, &p.tiles_per_split);
    if (p.nsplit > 1) {
      const size_t need = splitkv_bytes(B, H, Nq, d, p.nsplit);
      if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
      if (!aligned(workspace, 16)) return FA_ERR_UNSUPPORTED;
      p.Opart = static_cast<float*>(workspace);
      p.LSEpart = p.Opart + (size_t)p.nsplit * B * H * Nq * d;
    }
  }
  return status_of(
      fa::launch_fwd(p, d, causal != 0, blockmask != nullptr, p_drop > 0.f, stream));
}

int bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, int B, int H, int Nq, int Nk, int d, float scale, int causal,
             const uint8_t* blockmask, int mask_block, float p_drop, uint64_t seed,
             uint32_t offset, void* dQ, void* dK, void* dV, void* workspace,
             size_t workspace_bytes, hipStream_t stream, bool noalloc = false);

}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "libfa: a required pointer is NULL";
    case FA_ERR_SHAPE: return "libfa: negative dimension";
    case FA_ERR_UNSUPPORTED:
      return "libfa: unsupported arguments (need d in {64,128}, finite scale > 0, "
             "mask_block a multiple of 128, 16-byte aligned tensors, sizes below 2^31)";
    case FA_ERR_WORKSPACE: return "libfa: workspace missing or too small";
    case FA_ERR_HIP: return "libfa: HIP runtime error at kernel launch";
    case FA_ERR_SCRATCH:
      return "libfa: fa_bwd_noalloc supports at most FA_NOALLOC_MAX_ROWS (4194304) query rows "
             "B*H*N in its static scratch";
    default: return "libfa: unknown status";
  }
}

int fa_fwd(const void* Q, const void* K, const void* V, int B, int H, int N, int d, float scale,
           int causal, const uint8_t* blockmask, int mask_block, void* O, float* LSE,
           hipStream_t stream) {
  return fwd_impl(Q, K, V, B, H, N, N, d, scale, causal, blockmask, mask_block, 0.f, 0, 0, O,
                  LSE, stream);
}

int fa_fwd_nqk(const void* Q, const void* K, const void* V, int B, int H, int Nq, int Nk, int d,
               float scale, int causal, const uint8_t* blockmask, int mask_block, void* O,
               float* LSE, hipStream_t stream) {
  return fwd_impl(Q, K, V, B, H, Nq, Nk, d, scale, causal, blockmask, mask_block, 0.f, 0, 0, O,
                  LSE, stream);
}

int fa_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int d) {
  bool empty = false;
  if (check_shape(B, H, Nq, Nk, d, &empty) != FA_OK) return 0;
  int tps = 0;
  return splitkv_splits(B, H, Nq, Nk, 0, &tps);
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  bool empty = false;
  if (check_shape(B, H, Nq, Nk, d, &empty) != FA_OK) return 0;
  int tps = 0;
  return splitkv_bytes(B, H, Nq, d, splitkv_splits(B, H, Nq, Nk, num_splits, &tps));
}

int fa_fwd_splitkv(const void* Q, const void* K, const void* V, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, const uint8_t* blockmask, int mask_block,
                   int num_splits, void* workspace, size_t workspace_bytes, void* O, float* LSE,
                   hipStream_t stream) {
  return fwd_impl(Q, K, V, B, H, Nq, Nk, d, scale, causal, blockmask, mask_block, 0.f, 0, 0, O,
                  LSE, stream, num_splits <= 0 ? 0 : num_splits, workspace, workspace_bytes);
}

int fa_fwd_dropout(const void* Q, const void* K, const void* V, int B, int H, int N, int d,
                   float scale, int causal, const uint8_t* blockmask, int mask_block,
                   float p_drop, uint64_t seed, uint32_t offset, void* O, float* LSE,
                   hipStream_t stream) {
  return fwd_impl(Q, K, V, B, H, N, N, d, scale, causal, blockmask, mask_block, p_drop, seed,
                  offset, O, LSE, stream);
}

int fa_fwd_fp8(const void* Q, const void* K, const void* V, int B, int H, int N, int d,
               float scale, float q_descale, float k_descale, float v_descale, int causal,
               const uint8_t* blockmask, int mask_block, void* O, float* LSE,
               hipStream_t stream) {
  bool empty = false;
  int rc = check_common(B, H, N, d, scale, blockmask, mask_block, &empty);
  if (rc != FA_OK) return rc;
  for (const float x : {q_descale, k_descale, v_descale})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_UNSUPPORTED;
  // the folded score factor must stay a finite, nonzero fp32 number
  const double c = (double)scale * q_descale * k_descale * 1.4426950408889634;
  if (!(c > 1e-30 && c < 1e30)) return FA_ERR_UNSUPPORTED;
  if (empty) return FA_OK;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  if (!all_aligned16({Q, K, V, O}) || !aligned(LSE, 4)) return FA_ERR_UNSUPPORTED;

  fa::FwdParams p;
  p.Q = static_cast<const uint16_t*>(Q);
  p.K = static_cast<const uint16_t*>(K);
  p.V = static_cast<const uint16_t*>(V);
  p.O = static_cast<uint16_t*>(O);
  p.LSE = LSE;
  p.blockmask = blockmask;
  p.BH = B * H;
  p.Nq = p.Nk = N;
  p.nqb = (N + 127) / 128;
  p.mask_block = blockmask ? mask_block : 128;
  p.nbm = (N + p.mask_block - 1) / p.mask_block;
  p.scale_log2 = (float)c;
  p.v_descale = v_descale;
  set_dropout(p, 0.f, 0, 0);
  p.nsplit = 1;
  p.tiles_per_split = 0;
  p.Opart = p.LSEpart = nullptr;
  return status_of(fa::launch_fwd_fp8(p, d, causal != 0, blockmask != nullptr, stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  bool empty = false;
  if (check_shape(B, H, N, d, &empty) != FA_OK) return 0;
  return (size_t)4 * (size_t)B * (size_t)H * (size_t)N;
}

int fa_bwd_dsum(const void* O, const void* dO, int B, int H, int N, int d, float* Dsum,
                hipStream_t stream) {
  bool empty = false;
  int rc = check_shape(B, H, N, d, &empty);
  if (rc != FA_OK) return rc;
  if (empty) return FA_OK;
  if (!O || !dO || !Dsum) return FA_ERR_NULL;
  if (!all_aligned16({O, dO}) || !aligned(Dsum, 4)) return FA_ERR_UNSUPPORTED;
  const fa::BwdParams p = bwd_params(nullptr, nullptr, nullptr, O, dO, nullptr, Dsum, B, H, N,
                                     1.f, nullptr, 128, nullptr, nullptr, nullptr);
  return status_of(fa::launch_bwd_dsum(p, d, stream));
}

int fa_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                const float* Dsum, int B, int H, int N, int d, float scale, int causal,
                const uint8_t* blockmask, int mask_block, void* dK, void* dV,
                hipStream_t stream) {
  bool empty = false;
  int rc = check_common(B, H, N, d, scale, blockmask, mask_block, &empty);
  if (rc != FA_OK) return rc;
  if (empty) return FA_OK;
  if (!Q || !K || !V || !dO || !LSE || !Dsum || !dK || !dV) return FA_ERR_NULL;
  if (!all_aligned16({Q, K, V, dO, dK, dV}) || !aligned(LSE, 4) || !aligned(Dsum, 4))
    return FA_ERR_UNSUPPORTED;
  const fa::BwdParams p = bwd_params(Q, K, V, nullptr, dO, LSE, const_cast<float*>(Dsum), B, H,
                                     N, scale, blockmask, mask_block, nullptr, dK, dV);
  return status_of(fa::launch_bwd_dkdv(p, d, causal != 0, blockmask != nullptr, false, stream));
}

int fa_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
              const float* Dsum, int B, int H, int N, int d, float scale, int causal,
              const uint8_t* blockmask, int mask_block, void* dQ, hipStream_t stream) {
  bool empty = false;
  int rc = check_common(B, H, N, d, scale, blockmask, mask_block, &empty);
  if (rc != FA_OK) return rc;
  if (empty) return FA_OK;
  if (!Q || !K || !V || !dO || !LSE || !Dsum || !dQ) return FA_ERR_NULL;
  if (!all_aligned16({Q, K, V, dO, dQ}) || !aligned(LSE, 4) || !aligned(Dsum, 4))
    return FA_ERR_UNSUPPORTED;
  const fa::BwdParams p = bwd_params(Q, K, V, nullptr, dO, LSE, const_cast<float*>(Dsum), B, H,
                                     N, scale, blockmask, mask_block, dQ, nullptr, nullptr);
  return status_of(
      fa::launch_bwd_dq(p, d, causal != 0, blockmask != nullptr, false, false, stream));
}

int fa_bwd_dq_dsum(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block, float* Dsum, void* dQ,
                   hipStream_t stream) {
  bool empty = false;
  int rc = check_common(B, H, N, d, scale, blockmask, mask_block, &empty);
  if (rc != FA_OK) return rc;
  if (empty) return FA_OK;
  if (!Q || !K || !V || !O || !dO || !LSE || !Dsum || !dQ) return FA_ERR_NULL;
  if (!all_aligned16({Q, K, V, O, dO, dQ}) || !aligned(LSE, 4) || !aligned(Dsum, 4))
    return FA_ERR_UNSUPPORTED;
  const fa::BwdParams p = bwd_params(Q, K, V, O, dO, LSE, Dsum, B, H, N, scale, blockmask,
                                     mask_block, dQ, nullptr, nullptr);
  return status_of(
      fa::launch_bwd_dq(p, d, causal != 0, blockmask != nullptr, true, false, stream));
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, int B, int H, int N, int d, float scale, int causal,
           const uint8_t* blockmask, int mask_block, void* dQ, void* dK, void* dV,
           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, B, H, N, N, d, scale, causal, blockmask, mask_block, 0.f,
                  0, 0, dQ, dK, dV, workspace, workspace_bytes, stream);
}

int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block, void* dQ, void* dK, void* dV,
                   hipStream_t stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, B, H, N, N, d, scale, causal, blockmask, mask_block, 0.f,
                  0, 0, dQ, dK, dV, nullptr, 0, stream, true);
}

int fa_bwd_nqk(const void* Q, const void* K, const void* V, const void* O, const void* dO,
               const float* LSE, int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const uint8_t* blockmask, int mask_block, void* dQ, void* dK, void* dV,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, B, H, Nq, Nk, d, scale, causal, blockmask, mask_block,
                  0.f, 0, 0, dQ, dK, dV, workspace, workspace_bytes, stream);
}

int fa_bwd_dropout(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block, float p_drop, uint64_t seed,
                   uint32_t offset, void* dQ, void* dK, void* dV, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, B, H, N, N, d, scale, causal, blockmask, mask_block,
                  p_drop, seed, offset, dQ, dK, dV, workspace, workspace_bytes, stream);
}

int fa_dropout_keep_mask(int B, int H, int N, float p_drop, uint64_t seed, uint32_t offset,
                         uint8_t* keep, hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  const int rc = check_dropout(p_drop);
  if (rc != FA_OK) return rc;
  if ((long long)B * H * N * N > (long long)1 << 40) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N == 0) return FA_OK;
  if (!keep) return FA_ERR_NULL;
  fa::FwdParams p{};
  p.BH = B * H;
  p.Nq = N;
  p.Nk = N;
  set_dropout(p, p_drop, seed, offset);
  return status_of(fa::launch_dropout_keep_mask(p, keep, stream));
}

}  // extern "C"

namespace {

int bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, int B, int H, int Nq, int Nk, int d, float scale, int causal,
             const uint8_t* blockmask, int mask_block, float p_drop, uint64_t seed,
             uint32_t offset, void* dQ, void* dK, void* dV, void* workspace,
             size_t workspace_bytes, hipStream_t stream, bool noalloc) {
  bool empty = false;
  int rc = check_common(B, H, Nq, Nk, d, scale, blockmask, mask_block, &empty);
  if (rc != FA_OK) return rc;
  rc = check_dropout(p_drop);
  if (rc != FA_OK) return rc;
  // no query rows: dK = dV = 0 still has to be written when there are keys
  const bool no_keys = (long long)B * H * Nk == 0;
  if (empty && no_keys) return FA_OK;
  if (!empty && (!Q || !O || !dO || !LSE || !dQ)) return FA_ERR_NULL;
  if (!no_keys && (!K || !V || !dK || !dV)) return FA_ERR_NULL;
  if (noalloc) {
    // D goes to the library's static scratch instead of a caller workspace
    if ((long long)B * H * Nq > fa::kNoallocMaxRows) return FA_ERR_SCRATCH;
  } else if (!empty && (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, Nq, d))) {
    return FA_ERR_WORKSPACE;
  }
  if (!all_aligned16({Q, K, V, O, dO, dQ, dK, dV}) || !aligned(LSE, 4) || !aligned(workspace, 4))
    return FA_ERR_UNSUPPORTED;
  if (noalloc) {
    // the first HIP call: every argument check above has passed
    float* ws = nullptr;
    if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
    workspace = ws;
  }
  fa::BwdParams p = bwd_params(Q, K, V, O, dO, LSE, static_cast<float*>(workspace), B, H, Nq,
                               Nk, scale, blockmask, mask_block, dQ, dK, dV);
  set_dropout(p, p_drop, seed, offset);
  const bool cz = causal != 0, sp = blockmask != nullptr, dr = p_drop > 0.f;
  // dQ first, forming D on the way (the same bits fa_bwd_dsum writes), then dK, dV
  if (!empty) rc = status_of(fa::launch_bwd_dq(p, d, cz, sp, true, dr, stream));
  if (rc == FA_OK && !no_keys) rc = status_of(fa::launch_bwd_dkdv(p, d, cz, sp, dr, stream));
  return rc;
}

}  // namespace
