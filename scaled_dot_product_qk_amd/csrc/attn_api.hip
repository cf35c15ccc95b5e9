// Host side of the attention library: the C ABI declared in include/attn.h.
// Validates arguments on the host, picks the kernel instance for (dtype,
// head_dim, causal), sizes the grid and launches on the caller's stream.  No
// allocation and no fallback: anything without a kernel is an error.  The
// only state is memoised device queries (compute units, occupancy, the LDS
// attribute set once per kernel), one extra stream and two events per device
// for the backward (created at its first call on the device), and the
// allocation-free decode entry point's static scratch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "attn.h"
#include "bwd_bf16.h"
#include "decode.h"
#include "fwd_bf16.h"
#include "fwd_f32.h"
#include "fwd_fp8.h"

using namespace attn_dev;

namespace {

constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();
constexpr int64_t kGridYMax = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Element strides of every non-innermost dimension must keep rows 16-byte
// aligned and be non-negative.
bool strides_ok(const int64_t* s, int n, int elem_bytes) {
  const int64_t unit = 16 / elem_bytes;
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || s[i] % unit != 0) return false;
  return true;
}

bool fwd_head_dim_supported(int64_t d) { return d == 64 || d == 80 || d == 128; }
bool decode_head_dim_supported(int64_t d) { return d == 64 || d == 80 || d == 128; }

int elem_bytes_of(int32_t dtype) { return dtype == ATTN_F32 ? 4 : 2; }

float effective_scale(float scale, int64_t d) {
  return scale == 0.f ? 1.0f / std::sqrt((float)d) : scale;
}

// Workspace rows per (sequence, query head): the most pieces of the balanced
// decode split one sequence's slots can span (pieces hold at least
// kDecMinPiece slots, so L slots touch at most (L - 1) / kDecMinPiece + 2).
int64_t decode_pieces(int64_t Lmax) { return Lmax > 0 ? (Lmax - 1) / kDecMinPiece + 2 : 0; }

// Compute units of the current device (queried once per device).
int device_cu_count() {
  static std::atomic<int> counts[64];  // zero until queried; racing first calls store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev >= 64) dev = 63;
  int n = counts[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// A second stream of the library's per device, with the two events that fork
// it from a caller's stream and join it back.  Created at the first request
// on the device that is not made while the caller's stream is being captured
// into a graph (creating a stream there could end the capture); until then,
// and if creation fails, there is none.  `m` serialises the fork / launch /
// join sequences of concurrent callers, which share the two events.
struct SideStream {
  std::once_flag once;
  std::atomic<bool> ready{false};
  bool ok = false;
  std::mutex m;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

SideStream* side_stream(hipStream_t caller) {
  static SideStream sides[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  // The second stream lives on the current device: a caller's stream of
  // another device keeps all the work.
  if (caller != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(caller, &sdev) != hipSuccess || sdev != dev) return nullptr;
  }
  SideStream& x = sides[dev];
  if (!x.ready.load(std::memory_order_acquire)) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    std::call_once(x.once, [&x] {
      x.ok = hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) == hipSuccess &&
             hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&x.join, hipEventDisableTiming) == hipSuccess;
      x.ready.store(true, std::memory_order_release);
    });
  }
  return x.ok ? &x : nullptr;
}

}  // namespace

extern "C" attn_status_t attn_validate_fwd(const attn_fwd_args_t* a) {
  if (!a) return ATTN_ERR_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (a->B < 0 || a->Hq < 0 || a->Hkv < 0 || a->Lq < 0 || a->Lk < 0 || a->d < 0)
    return ATTN_ERR_SHAPE;
  if (!std::isfinite(a->scale)) return ATTN_ERR_SHAPE;
  if (!fwd_head_dim_supported(a->d)) return ATTN_ERR_UNSUPPORTED;
  const bool work = a->B > 0 && a->Hq > 0 && a->Lq > 0;
  if (a->Hq > 0 && (a->Hkv == 0 || a->Hq % a->Hkv != 0)) return ATTN_ERR_SHAPE;
  if (!work) return ATTN_OK;
  if (!a->q || !a->o || !a->lse) return ATTN_ERR_NULL;
  if (a->Lk > 0 && (!a->k || !a->v)) return ATTN_ERR_NULL;
  const int eb = elem_bytes_of(a->dtype);
  if (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->lse)) return ATTN_ERR_LAYOUT;
  if (a->Lk > 0 && (!aligned16(a->k) || !aligned16(a->v))) return ATTN_ERR_LAYOUT;
  if (!strides_ok(a->q_strides, 3, eb) || !strides_ok(a->o_strides, 3, eb) ||
      !strides_ok(a->k_strides, 3, eb) || !strides_ok(a->v_strides, 3, eb))
    return ATTN_ERR_LAYOUT;
  // Index ranges the kernels keep in 32 bits, and the grid limits.
  if (a->Lq > kI32Max || a->Lk > kI32Max || a->B * a->Hq > kI32Max) return ATTN_ERR_UNSUPPORTED;
  if (a->dtype == ATTN_BF16 && a->Lk > 0 &&
      (a->k_strides[2] >= attn_dev::kFwdMaxTokenStride || a->v_strides[2] >= attn_dev::kFwdMaxTokenStride))
    return ATTN_ERR_UNSUPPORTED;
  if ((a->Lq + 127) / 128 > kGridYMax || a->B * a->Hq * ((a->Lq + 127) / 128) > kI32Max)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

extern "C" const char* attn_kernel_name(const attn_fwd_args_t* a) {
  if (attn_validate_fwd(a) != ATTN_OK) return "none";
  const bool bf = a->dtype == ATTN_BF16;
  const bool c = a->causal != 0;
  switch (a->d) {
    case 64: return bf ? (c ? "attn_fwd_bf16_d64_causal" : "attn_fwd_bf16_d64")
                       : (c ? "attn_fwd_f32_d64_causal" : "attn_fwd_f32_d64");
    case 80: return bf ? (c ? "attn_fwd_bf16_d80_causal" : "attn_fwd_bf16_d80")
                       : (c ? "attn_fwd_f32_d80_causal" : "attn_fwd_f32_d80");
    case 128: return bf ? (c ? "attn_fwd_bf16_d128_causal" : "attn_fwd_bf16_d128")
                        : (c ? "attn_fwd_f32_d128_causal" : "attn_fwd_f32_d128");
    default: return "none";
  }
}

static attn_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <int D, bool CAUSAL, int MK = 0>
static attn_status_t launch_fwd_bf16(const FwdParams& p, int grid_x, hipStream_t s) {
  constexpr int lds = FwdMaskShape<D, CAUSAL, MK>::kKernelLdsBytes;
  auto kern = attn_fwd_bf16_kernel<D, CAUSAL, MK>;
  static std::atomic<bool> attr_set{false};  // racing first calls set the same value
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
        hipSuccess)
      return ATTN_ERR_HIP;
    attr_set.store(true, std::memory_order_relaxed);
  }
  FwdParams q = p;
  q.n_qtiles = (p.Lq + Bf16FwdShape<D>::kBR - 1) / Bf16FwdShape<D>::kBR;
  hipLaunchKernelGGL(kern, dim3(grid_x * q.n_qtiles), dim3(64 * Bf16FwdShape<D>::kWaves), lds, s, q);
  return launch_status();
}

template <int D, bool CAUSAL>
static attn_status_t launch_fwd_f32(const FwdParams& p, int grid_x, hipStream_t s) {
  constexpr int lds = F32FwdShape<D>::kLdsBytes;
  auto kern = attn_fwd_f32_kernel<D, CAUSAL>;
  static std::atomic<bool> attr_set{false};  // racing first calls set the same value
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
        hipSuccess)
      return ATTN_ERR_HIP;
    attr_set.store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL(kern, dim3(grid_x, (p.Lq + 127) / 128), dim3(256), lds, s, p);
  return launch_status();
}

static FwdParams dense_fwd_params(const attn_fwd_args_t* a) {
  FwdParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.lse = a->lse;
  p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_st = a->q_strides[2];
  p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_st = a->k_strides[2];
  p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_st = a->v_strides[2];
  p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_st = a->o_strides[2];
  p.Hq = (int)a->Hq;
  p.Hkv = (int)a->Hkv;
  p.group = (int)(a->Hq / a->Hkv);
  p.Lq = (int)a->Lq;
  p.Lk = (int)a->Lk;
  p.n_qtiles = (int)((a->Lq + 127) / 128);
  p.lse_sb = a->Hq * a->Lq;
  p.lse_sh = a->Lq;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.total_q = p.total_k = 0;
  p.mask = nullptr;
  p.m_sb = p.m_sh = p.m_sq = 0;
  p.scale_log2 = effective_scale(a->scale, a->d) * kLog2e;
  p.scale_log2_abs = std::fabs(p.scale_log2);
  p.inv_abs_scale = 1.0f / std::fabs(effective_scale(a->scale, a->d));
  p.neg_q = p.scale_log2 < 0.f ? 1 : 0;
  p.o_mul = 1.f;
  return p;
}

extern "C" attn_status_t attn_fwd(const attn_fwd_args_t* a, void* stream) {
  const attn_status_t st = attn_validate_fwd(a);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0 || a->Lq == 0) return ATTN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const FwdParams p = dense_fwd_params(a);
  const int grid_x = (int)(a->B * a->Hq);
  const bool c = a->causal != 0;
  if (a->dtype == ATTN_BF16) {
    switch (a->d) {
      case 64: return c ? launch_fwd_bf16<64, true>(p, grid_x, s) : launch_fwd_bf16<64, false>(p, grid_x, s);
      case 80: return c ? launch_fwd_bf16<80, true>(p, grid_x, s) : launch_fwd_bf16<80, false>(p, grid_x, s);
      case 128: return c ? launch_fwd_bf16<128, true>(p, grid_x, s) : launch_fwd_bf16<128, false>(p, grid_x, s);
    }
  } else {
    switch (a->d) {
      case 64: return c ? launch_fwd_f32<64, true>(p, grid_x, s) : launch_fwd_f32<64, false>(p, grid_x, s);
      case 80: return c ? launch_fwd_f32<80, true>(p, grid_x, s) : launch_fwd_f32<80, false>(p, grid_x, s);
      case 128: return c ? launch_fwd_f32<128, true>(p, grid_x, s) : launch_fwd_f32<128, false>(p, grid_x, s);
    }
  }
  return ATTN_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------------ masked
constexpr int64_t kMaskMaxRowBytes = int64_t(1) << 27;  // 32-bit lane offsets span 16 mask rows

extern "C" attn_status_t attn_validate_fwd_masked(const attn_fwd_args_t* a, const attn_mask_t* m) {
  const attn_status_t st = attn_validate_fwd(a);
  if (st != ATTN_OK) return st;
  if (!m) return ATTN_ERR_NULL;
  if (m->kind != ATTN_MASK_BOOL && m->kind != ATTN_MASK_ADD_BF16) return ATTN_ERR_DTYPE;
  if (a->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  const bool work = a->B > 0 && a->Hq > 0 && a->Lq > 0;
  if (!work || a->Lk == 0) return ATTN_OK;
  if (!m->data) return ATTN_ERR_NULL;
  const int64_t es = m->kind == ATTN_MASK_BOOL ? 1 : 2;
  if (!aligned16(m->data)) return ATTN_ERR_LAYOUT;
  if (m->strides[0] < 0 || m->strides[1] < 0 || m->strides[2] < 0 || (m->strides[2] * es) % 16 != 0)
    return ATTN_ERR_LAYOUT;
  if (a->Lk % (16 / es) != 0) return ATTN_ERR_UNSUPPORTED;  // whole 16-byte chunks per mask row
  if (m->strides[2] * es >= kMaskMaxRowBytes) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

extern "C" attn_status_t attn_fwd_masked(const attn_fwd_args_t* a, const attn_mask_t* m, void* stream) {
  const attn_status_t st = attn_validate_fwd_masked(a, m);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0 || a->Lq == 0) return ATTN_OK;
  if (a->Lk == 0) return attn_fwd(a, stream);  // no keys: the mask has nothing to remove
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  FwdParams p = dense_fwd_params(a);
  p.mask = m->data;
  p.m_sb = m->strides[0];
  p.m_sh = m->strides[1];
  p.m_sq = m->strides[2];
  const int grid_x = (int)(a->B * a->Hq);
  const bool c = a->causal != 0;
  if (m->kind == ATTN_MASK_BOOL) {
    switch (a->d) {
      case 64: return c ? launch_fwd_bf16<64, true, 1>(p, grid_x, s) : launch_fwd_bf16<64, false, 1>(p, grid_x, s);
      case 80: return c ? launch_fwd_bf16<80, true, 1>(p, grid_x, s) : launch_fwd_bf16<80, false, 1>(p, grid_x, s);
      case 128: return c ? launch_fwd_bf16<128, true, 1>(p, grid_x, s) : launch_fwd_bf16<128, false, 1>(p, grid_x, s);
    }
  } else {
    switch (a->d) {
      case 64: return c ? launch_fwd_bf16<64, true, 2>(p, grid_x, s) : launch_fwd_bf16<64, false, 2>(p, grid_x, s);
      case 80: return c ? launch_fwd_bf16<80, true, 2>(p, grid_x, s) : launch_fwd_bf16<80, false, 2>(p, grid_x, s);
      case 128: return c ? launch_fwd_bf16<128, true, 2>(p, grid_x, s) : launch_fwd_bf16<128, false, 2>(p, grid_x, s);
    }
  }
  return ATTN_ERR_UNSUPPORTED;
}

extern "C" attn_status_t attn_validate_fwd_varlen(const attn_fwd_varlen_args_t* a) {
  if (!a) return ATTN_ERR_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (a->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (a->B < 0 || a->Hq < 0 || a->Hkv < 0 || a->total_q < 0 || a->total_k < 0 || a->max_seqlen_q < 0 ||
      a->d < 0)
    return ATTN_ERR_SHAPE;
  if (a->max_seqlen_q > a->total_q) return ATTN_ERR_SHAPE;
  if (!std::isfinite(a->scale)) return ATTN_ERR_SHAPE;
  if (!fwd_head_dim_supported(a->d)) return ATTN_ERR_UNSUPPORTED;
  if (a->Hq > 0 && (a->Hkv == 0 || a->Hq % a->Hkv != 0)) return ATTN_ERR_SHAPE;
  const bool work = a->B > 0 && a->Hq > 0 && a->max_seqlen_q > 0;
  if (!work) return ATTN_OK;
  if (!a->q || !a->o || !a->lse || !a->cu_seqlens_q || !a->cu_seqlens_k) return ATTN_ERR_NULL;
  if (a->total_k > 0 && (!a->k || !a->v)) return ATTN_ERR_NULL;
  if (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->lse)) return ATTN_ERR_LAYOUT;
  if (a->total_k > 0 && (!aligned16(a->k) || !aligned16(a->v))) return ATTN_ERR_LAYOUT;
  if ((reinterpret_cast<uintptr_t>(a->cu_seqlens_q) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(a->cu_seqlens_k) & 3u) != 0)
    return ATTN_ERR_LAYOUT;
  if (!strides_ok(a->q_strides, 2, 2) || !strides_ok(a->o_strides, 2, 2) || !strides_ok(a->k_strides, 2, 2) ||
      !strides_ok(a->v_strides, 2, 2))
    return ATTN_ERR_LAYOUT;
  if (a->total_q > kI32Max || a->total_k > kI32Max || a->B >= kI32Max) return ATTN_ERR_UNSUPPORTED;
  if (a->total_k > 0 &&
      (a->k_strides[0] >= attn_dev::kFwdMaxTokenStride || a->v_strides[0] >= attn_dev::kFwdMaxTokenStride))
    return ATTN_ERR_UNSUPPORTED;
  if (a->B * a->Hq * ((a->max_seqlen_q + 127) / 128) > kI32Max) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

extern "C" attn_status_t attn_fwd_varlen(const attn_fwd_varlen_args_t* a, void* stream) {
  const attn_status_t st = attn_validate_fwd_varlen(a);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0 || a->max_seqlen_q == 0) return ATTN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  FwdParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.lse = a->lse;
  // the batch offset comes from the sequence offsets
  p.q_sb = 0; p.q_sh = a->q_strides[1]; p.q_st = a->q_strides[0];
  p.k_sb = 0; p.k_sh = a->k_strides[1]; p.k_st = a->k_strides[0];
  p.v_sb = 0; p.v_sh = a->v_strides[1]; p.v_st = a->v_strides[0];
  p.o_sb = 0; p.o_sh = a->o_strides[1]; p.o_st = a->o_strides[0];
  p.Hq = (int)a->Hq;
  p.Hkv = (int)a->Hkv;
  p.group = (int)(a->Hq / a->Hkv);
  p.Lq = (int)a->max_seqlen_q;  // sizes the grid; each sequence's own length is read on the device
  p.Lk = 0;
  p.lse_sb = 0;
  p.lse_sh = a->total_q;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.total_q = (int)a->total_q;
  p.total_k = (int)a->total_k;
  p.mask = nullptr;
  p.m_sb = p.m_sh = p.m_sq = 0;
  p.inv_abs_scale = 0.f;
  p.scale_log2 = effective_scale(a->scale, a->d) * kLog2e;
  p.scale_log2_abs = std::fabs(p.scale_log2);
  p.neg_q = p.scale_log2 < 0.f ? 1 : 0;
  p.o_mul = 1.f;
  const int grid_x = (int)(a->B * a->Hq);
  const bool c = a->causal != 0;
  switch (a->d) {
    case 64: return c ? launch_fwd_bf16<64, true>(p, grid_x, s) : launch_fwd_bf16<64, false>(p, grid_x, s);
    case 80: return c ? launch_fwd_bf16<80, true>(p, grid_x, s) : launch_fwd_bf16<80, false>(p, grid_x, s);
    case 128: return c ? launch_fwd_bf16<128, true>(p, grid_x, s) : launch_fwd_bf16<128, false>(p, grid_x, s);
  }
  return ATTN_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------------ FP8
extern "C" attn_status_t attn_validate_fwd_fp8(const attn_fwd_fp8_args_t* a) {
  if (!a) return ATTN_ERR_NULL;
  if (a->B < 0 || a->Hq < 0 || a->Hkv < 0 || a->Lq < 0 || a->Lk < 0 || a->d < 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(a->scale) || !std::isfinite(a->q_descale) || !std::isfinite(a->k_descale) ||
      !std::isfinite(a->v_descale))
    return ATTN_ERR_SHAPE;
  // the score multiplier scale * q_descale * k_descale * log2(e) must be a finite float
  const double mult = (double)effective_scale(a->scale, a->d > 0 ? a->d : 1) * a->q_descale * a->k_descale * kLog2e;
  if (!(std::fabs(mult) <= (double)std::numeric_limits<float>::max())) return ATTN_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return ATTN_ERR_UNSUPPORTED;
  if (a->Hq > 0 && (a->Hkv == 0 || a->Hq % a->Hkv != 0)) return ATTN_ERR_SHAPE;
  const bool work = a->B > 0 && a->Hq > 0 && a->Lq > 0;
  if (!work) return ATTN_OK;
  if (!a->q || !a->o || !a->lse) return ATTN_ERR_NULL;
  if (a->Lk > 0 && (!a->k || !a->v)) return ATTN_ERR_NULL;
  if (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->lse)) return ATTN_ERR_LAYOUT;
  if (a->Lk > 0 && (!aligned16(a->k) || !aligned16(a->v))) return ATTN_ERR_LAYOUT;
  if (!strides_ok(a->q_strides, 3, 1) || !strides_ok(a->k_strides, 3, 1) || !strides_ok(a->v_strides, 3, 1) ||
      !strides_ok(a->o_strides, 3, 2))
    return ATTN_ERR_LAYOUT;
  if (a->Lq > kI32Max || a->Lk > kI32Max || a->B * a->Hq > kI32Max) return ATTN_ERR_UNSUPPORTED;
  if (a->Lk > 0 &&
      (a->k_strides[2] >= attn_dev::kFwdMaxTokenStride || a->v_strides[2] >= attn_dev::kFwdMaxTokenStride))
    return ATTN_ERR_UNSUPPORTED;
  if (a->B * a->Hq * ((a->Lq + 127) / 128) > kI32Max) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

template <int D, bool CAUSAL>
static attn_status_t launch_fwd_fp8(const FwdParams& p, int grid_x, hipStream_t s) {
  using S = Fp8FwdShape<D>;
  constexpr int lds = S::kLdsBytes;
  auto kern = attn_fwd_fp8_kernel<D, CAUSAL>;
  static std::atomic<bool> attr_set{false};  // racing first calls set the same value
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return ATTN_ERR_HIP;
    attr_set.store(true, std::memory_order_relaxed);
  }
  FwdParams q = p;
  q.n_qtiles = (p.Lq + S::kBR - 1) / S::kBR;
  hipLaunchKernelGGL(kern, dim3(grid_x * q.n_qtiles), dim3(64 * S::kWaves), lds, s, q);
  return launch_status();
}

extern "C" attn_status_t attn_fwd_fp8(const attn_fwd_fp8_args_t* a, void* stream) {
  const attn_status_t st = attn_validate_fwd_fp8(a);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0 || a->Lq == 0) return ATTN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  FwdParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.lse = a->lse;
  p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_st = a->q_strides[2];
  p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_st = a->k_strides[2];
  p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_st = a->v_strides[2];
  p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_st = a->o_strides[2];
  p.Hq = (int)a->Hq;
  p.Hkv = (int)a->Hkv;
  p.group = (int)(a->Hq / a->Hkv);
  p.Lq = (int)a->Lq;
  p.Lk = (int)a->Lk;
  p.n_qtiles = (int)((a->Lq + 127) / 128);
  p.lse_sb = a->Hq * a->Lq;
  p.lse_sh = a->Lq;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.total_q = p.total_k = 0;
  p.mask = nullptr;
  p.m_sb = p.m_sh = p.m_sq = 0;
  p.inv_abs_scale = 0.f;
  p.scale_log2 = (float)((double)effective_scale(a->scale, a->d) * a->q_descale * a->k_descale * kLog2e);
  p.scale_log2_abs = std::fabs(p.scale_log2);
  p.neg_q = p.scale_log2 < 0.f ? 1 : 0;
  p.o_mul = a->v_descale;
  const int grid_x = (int)(a->B * a->Hq);
  const bool c = a->causal != 0;
  switch (a->d) {
    case 64: return c ? launch_fwd_fp8<64, true>(p, grid_x, s) : launch_fwd_fp8<64, false>(p, grid_x, s);
    case 128: return c ? launch_fwd_fp8<128, true>(p, grid_x, s) : launch_fwd_fp8<128, false>(p, grid_x, s);
  }
  return ATTN_ERR_UNSUPPORTED;
}

// ------------------------------------------------------------------ backward
bool bwd_head_dim_supported(int64_t d) { return d == 64 || d == 80 || d == 128; }

extern "C" size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq) {
  if (B < 0 || Hq < 0 || Lq < 0) return 0;
  return (size_t)((B * Hq * Lq * 8 + 255) / 256 * 256);
}

extern "C" attn_status_t attn_validate_bwd(const attn_bwd_args_t* a) {
  if (!a) return ATTN_ERR_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (a->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (a->B < 0 || a->Hq < 0 || a->Hkv < 0 || a->Lq < 0 || a->Lk < 0 || a->d < 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(a->scale)) return ATTN_ERR_SHAPE;
  if (!bwd_head_dim_supported(a->d)) return ATTN_ERR_UNSUPPORTED;
  if (a->Hq > 0 && (a->Hkv == 0 || a->Hq % a->Hkv != 0)) return ATTN_ERR_SHAPE;
  const bool work = a->B > 0 && a->Hq > 0 && (a->Lq > 0 || a->Lk > 0);
  if (!work) return ATTN_OK;
  if (a->Lq > 0 && (!a->q || !a->o || !a->dout || !a->lse || !a->dq)) return ATTN_ERR_NULL;
  if (a->Lk > 0 && (!a->k || !a->v || !a->dk || !a->dv)) return ATTN_ERR_NULL;
  if (a->Lq > 0 && (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->dout) || !aligned16(a->dq) ||
                    (reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0))
    return ATTN_ERR_LAYOUT;
  if (a->Lk > 0 && (!aligned16(a->k) || !aligned16(a->v) || !aligned16(a->dk) || !aligned16(a->dv)))
    return ATTN_ERR_LAYOUT;
  const int64_t* st[] = {a->q_strides, a->k_strides, a->v_strides, a->o_strides,
                         a->do_strides, a->dq_strides, a->dk_strides, a->dv_strides};
  for (const int64_t* x : st)
    if (!strides_ok(x, 3, 2)) return ATTN_ERR_LAYOUT;
  if (a->Lq > kI32Max || a->Lk > kI32Max || a->B * a->Hq > kI32Max || a->B * a->Hq * a->Lq > kI32Max * 64)
    return ATTN_ERR_UNSUPPORTED;
  if (a->B * a->Hkv * ((a->Lk + 127) / 128) > kI32Max || a->B * a->Hq * ((a->Lq + 127) / 128) > kI32Max)
    return ATTN_ERR_UNSUPPORTED;
  if (a->Lq > 0 && a->Lk > 0 &&
      (a->q_strides[2] >= attn_dev::kBwdMaxTokenStride || a->do_strides[2] >= attn_dev::kBwdMaxTokenStride ||
       a->k_strides[2] >= attn_dev::kBwdMaxTokenStride || a->v_strides[2] >= attn_dev::kBwdMaxTokenStride))
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

template <int D, bool CAUSAL>
static attn_status_t launch_bwd_dkdv(const BwdParams& p, int grid, hipStream_t s) {
  using S = BwdKvShape<D>;
  auto kern = attn_bwd_dkdv_kernel<D, CAUSAL>;
  static std::atomic<bool> attr_set{false};  // racing first calls set the same value
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, S::kLdsBytes) !=
        hipSuccess)
      return ATTN_ERR_HIP;
    attr_set.store(true, std::memory_order_relaxed);
  }
  // Key blocks per (batch, kv head) that are resident from the start: the
  // grid's first (compute units x workgroups per unit) blocks, key block
  // slowest.  Causal, the later ones walk their query tiles upward.
  static std::atomic<int> per_cu_cache{0};  // racing first calls store the same value
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, 64 * S::kWaves, S::kLdsBytes) !=
            hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  BwdParams q = p;
  q.kv_round1 = (int)((int64_t)device_cu_count() * per_cu / std::max(1, p.B * p.Hkv));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * S::kWaves), S::kLdsBytes, s, q);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <int D, bool CAUSAL>
static attn_status_t launch_bwd_dq(const BwdParams& p, int grid, hipStream_t s) {
  using S = BwdQShape<D>;
  auto kern = attn_bwd_dq_kernel<D, CAUSAL>;
  static std::atomic<bool> attr_set{false};  // racing first calls set the same value
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, S::kLdsBytes) !=
        hipSuccess)
      return ATTN_ERR_HIP;
    attr_set.store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * S::kWaves), S::kLdsBytes, s, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// The dK/dV and dQ kernels read the inputs and the row statistics, not each
// other's results.  At head_dim 64 and 80 the dQ kernel runs on the
// library's second stream, forked from the caller's stream after the
// statistics kernel and joined back into it before attn_bwd returns (events
// only, no host wait): its workgroups take the compute units the dK/dV
// kernel's causal tail frees (and at 64 slots beside its workgroups).  At
// head_dim 128 that measured no gain, and both run on the caller's stream.
template <int D>
static attn_status_t launch_bwd(const BwdParams& p, bool causal, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.Lq;
  if (rows > 0) {
    hipLaunchKernelGGL(attn_bwd_delta_kernel<D>, dim3((unsigned)((rows + kDeltaRowsPerBlock<D> - 1) / kDeltaRowsPerBlock<D>)),
                       dim3(256), 0, s, p);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  }
  const int g_kv = p.B * p.Hkv * ((p.Lk + 127) / 128);
  const int g_q = p.B * p.Hq * ((p.Lq + BwdQShape<D>::kRows - 1) / BwdQShape<D>::kRows);
  SideStream* side = D <= 80 && g_kv > 0 && g_q > 0 ? side_stream(s) : nullptr;
  auto dkdv = [&]() {
    if (g_kv <= 0) return ATTN_OK;
    return causal ? launch_bwd_dkdv<D, true>(p, g_kv, s) : launch_bwd_dkdv<D, false>(p, g_kv, s);
  };
  auto dq = [&](hipStream_t sq) {
    if (g_q <= 0) return ATTN_OK;
    return causal ? launch_bwd_dq<D, true>(p, g_q, sq) : launch_bwd_dq<D, false>(p, g_q, sq);
  };
  if (!side) {
    const attn_status_t st = dkdv();
    return st != ATTN_OK ? st : dq(s);
  }
  std::lock_guard<std::mutex> lock(side->m);
  if (hipEventRecord(side->fork, s) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
    return ATTN_ERR_HIP;
  attn_status_t st = dq(side->s);
  if (st == ATTN_OK) st = dkdv();
  // joined even after a failed launch, so that nothing of this call runs
  // unordered with the caller's later work
  if (hipEventRecord(side->join, side->s) != hipSuccess || hipStreamWaitEvent(s, side->join, 0) != hipSuccess)
    return ATTN_ERR_HIP;
  return st;
}

extern "C" attn_status_t attn_bwd(const attn_bwd_args_t* a, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  const attn_status_t st = attn_validate_bwd(a);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0 || (a->Lq == 0 && a->Lk == 0)) return ATTN_OK;
  const size_t need = attn_bwd_workspace_bytes(a->B, a->Hq, a->Lq);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_LAYOUT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  BwdParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.dout = a->dout; p.lse = a->lse;
  p.stats = reinterpret_cast<float*>(workspace);
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_st = a->q_strides[2];
  p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_st = a->k_strides[2];
  p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_st = a->v_strides[2];
  p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_st = a->o_strides[2];
  p.do_sb = a->do_strides[0]; p.do_sh = a->do_strides[1]; p.do_st = a->do_strides[2];
  p.dq_sb = a->dq_strides[0]; p.dq_sh = a->dq_strides[1]; p.dq_st = a->dq_strides[2];
  p.dk_sb = a->dk_strides[0]; p.dk_sh = a->dk_strides[1]; p.dk_st = a->dk_strides[2];
  p.dv_sb = a->dv_strides[0]; p.dv_sh = a->dv_strides[1]; p.dv_st = a->dv_strides[2];
  p.B = (int)a->B;
  p.Hq = (int)a->Hq;
  p.Hkv = (int)a->Hkv;
  p.group = (int)(a->Hq / a->Hkv);
  p.Lq = (int)a->Lq;
  p.Lk = (int)a->Lk;
  p.kv_round1 = 0;  // set per launch of the dK/dV kernel
  p.scale = effective_scale(a->scale, a->d);
  p.scale_log2 = p.scale * kLog2e;
  const bool c = a->causal != 0;
  switch (a->d) {
    case 64: return launch_bwd<64>(p, c, s);
    case 80: return launch_bwd<80>(p, c, s);
    case 128: return launch_bwd<128>(p, c, s);
  }
  return ATTN_ERR_UNSUPPORTED;
}

extern "C" size_t attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Lmax, int64_t d) {
  if (B < 0 || Hq < 0 || Lmax < 0 || d <= 0) return 0;
  const int64_t rows = B * Hq * decode_pieces(Lmax);
  const int64_t obytes = (rows * d * 4 + 255) / 256 * 256;
  return (size_t)(obytes + rows * 4);
}

extern "C" attn_status_t attn_validate_decode(const attn_decode_args_t* a) {
  if (!a) return ATTN_ERR_NULL;
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (a->B < 0 || a->Hq < 0 || a->Hkv < 0 || a->Lmax < 0 || a->d < 0) return ATTN_ERR_SHAPE;
  if (!std::isfinite(a->scale)) return ATTN_ERR_SHAPE;
  if (a->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!decode_head_dim_supported(a->d)) return ATTN_ERR_UNSUPPORTED;
  if (a->Hq > 0 && (a->Hkv == 0 || a->Hq % a->Hkv != 0)) return ATTN_ERR_SHAPE;
  if (a->B == 0 || a->Hq == 0) return ATTN_OK;
  if (!a->q || !a->o || !a->lse || !a->seqlens) return ATTN_ERR_NULL;
  if (a->Lmax > 0 && (!a->k_cache || !a->v_cache)) return ATTN_ERR_NULL;
  if (!aligned16(a->q) || !aligned16(a->o) || !aligned16(a->lse)) return ATTN_ERR_LAYOUT;
  if (a->Lmax > 0 && (!aligned16(a->k_cache) || !aligned16(a->v_cache))) return ATTN_ERR_LAYOUT;
  if ((reinterpret_cast<uintptr_t>(a->seqlens) & 3u) != 0) return ATTN_ERR_LAYOUT;
  if (!strides_ok(a->q_strides, 2, 2) || !strides_ok(a->o_strides, 2, 2) ||
      !strides_ok(a->k_strides, 3, 2) || !strides_ok(a->v_strides, 3, 2))
    return ATTN_ERR_LAYOUT;
  const int64_t hgroups = (a->Hq / a->Hkv + kDecHeadsPerGroup - 1) / kDecHeadsPerGroup;
  // the lengths' total must fit 32 bits
  if (a->Lmax > kI32Max || a->B * a->Lmax > kI32Max || a->B * a->Hq > kI32Max ||
      a->B * a->Hkv * hgroups > kI32Max)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

template <int D>
static attn_status_t launch_decode(const DecodeParams& p, int B, hipStream_t s) {
  if (p.Lmax > 0) {
    hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3(p.n_wg), dim3(64 * kDecWaves), 0, s, p);
    if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  }
  hipLaunchKernelGGL(attn_decode_merge_kernel<D>, dim3((unsigned)(((int64_t)B * p.Hq + kDecMergeWaves - 1) / kDecMergeWaves)),
                     dim3(64 * kDecMergeWaves), 0, s, p);
  return launch_status();
}

// Enqueues the decode kernels for validated arguments, with the partial
// results in `workspace` (attn_decode_workspace_bytes bytes, 256-byte
// aligned).
static attn_status_t decode_enqueue(const attn_decode_args_t* a, void* workspace, hipStream_t s) {
  DecodeParams p;
  p.q = a->q; p.k = a->k_cache; p.v = a->v_cache; p.seqlens = a->seqlens;
  const int64_t rows = a->B * a->Hq * decode_pieces(a->Lmax);
  p.o_part = reinterpret_cast<float*>(workspace);
  p.lse_part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                        (rows * a->d * 4 + 255) / 256 * 256);
  p.o = a->o; p.lse = a->lse;
  p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1];
  p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_st = a->k_strides[2];
  p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_st = a->v_strides[2];
  p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1];
  p.Hq = (int)a->Hq;
  p.Hkv = (int)a->Hkv;
  p.group = (int)(a->Hq / a->Hkv);
  p.Lmax = (int)a->Lmax;
  p.B = (int)a->B;
  p.n_hgroups = (p.group + kDecHeadsPerGroup - 1) / kDecHeadsPerGroup;
  p.n_pieces = (int)decode_pieces(a->Lmax);
  // One piece per split workgroup, fewer when even the largest
  // possible total (every sequence at Lmax) would leave pieces below the minimum.
  {
    const int64_t most = (a->Hkv * p.n_hgroups * a->B * a->Lmax + kDecMinPiece - 1) / kDecMinPiece;
    const int64_t want = (int64_t)device_cu_count() * kDecGroupsPerCU;
    p.n_wg = (int)(most < want ? (most > 0 ? most : 1) : want);
  }
  p.scale_log2 = effective_scale(a->scale, a->d) * kLog2e;
  switch (a->d) {
    case 64: return launch_decode<64>(p, (int)a->B, s);
    case 80: return launch_decode<80>(p, (int)a->B, s);
    case 128: return launch_decode<128>(p, (int)a->B, s);
  }
  return ATTN_ERR_UNSUPPORTED;
}

extern "C" attn_status_t attn_decode(const attn_decode_args_t* a, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const attn_status_t st = attn_validate_decode(a);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0) return ATTN_OK;
  const size_t need = attn_decode_workspace_bytes(a->B, a->Hq, a->Lmax, a->d);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_LAYOUT;
  return decode_enqueue(a, workspace, reinterpret_cast<hipStream_t>(stream));
}

// ---- attn_decode_noalloc: the decode workspace in a static device array ----
// Every device the library runs on holds its own copy of `scratch` from the
// first launch on it until the process ends.  In host code the array's name
// is only a host-side stand-in, so the device address of each device's copy
// is looked up once per device (with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {nullptr};

// Device address of the current device's scratch array, or nullptr if the
// runtime cannot give it.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}
}  // namespace

extern "C" attn_status_t attn_decode_noalloc(const attn_decode_args_t* a, void* stream) {
  const attn_status_t st = attn_validate_decode(a);
  if (st != ATTN_OK) return st;
  if (a->B == 0 || a->Hq == 0) return ATTN_OK;
  const size_t need = attn_decode_workspace_bytes(a->B, a->Hq, a->Lmax, a->d);
  if (need > (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  void* ws = device_scratch();
  if (ws == nullptr) return ATTN_ERR_HIP;
  return decode_enqueue(a, ws, reinterpret_cast<hipStream_t>(stream));
}

extern "C" const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid shape or argument";
    case ATTN_ERR_DTYPE: return "invalid dtype";
    case ATTN_ERR_LAYOUT: return "misaligned pointer or stride";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch error";
    case ATTN_ERR_SCRATCH: return "sizes need more than the static decode scratch (attn_decode_noalloc)";
  }
  return "unknown status";
}

extern "C" const char* attn_version(void) { return "attn-gfx950 0.1.0"; }

