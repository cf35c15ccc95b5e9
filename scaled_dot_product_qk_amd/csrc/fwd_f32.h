// Prefill attention forward, fp32 inputs, for gfx950.
//
// Same method and orientation as the bf16 kernel (tiled forward with online
// softmax, "Flash Attention原理：分块计算与重计算" (cnblogs) sections 三-五;
// S^T = K Q^T and O^T = V^T P^T so that a lane holds one query), but every
// operand stays in fp32: the products run on the fp32 matrix instruction
// v_mfma_f32_32x32x2_f32 and the probabilities are not rounded.
//
// One workgroup of 4 waves per (batch, query head, 128 query rows); key tiles
// of 32 keys staged in LDS, double buffered.
#pragma once

#include "device_common.h"
#include "fwd_bf16.h"  // FwdParams

namespace attn_dev {

template <int D>
struct F32FwdShape {
  static constexpr int kBR = 128;
  static constexpr int kBC = 32;
  static constexpr int kDP = (D + 31) / 32 * 32;
  static constexpr int kND = kDP / 32;
  static constexpr int kHalf = D / 2;        // k slots: lane half g covers d in [g*D/2, (g+1)*D/2)
  static constexpr int kChunks = D / 4;      // 16-byte chunks per row
  static constexpr int kKPitch = D + 4;      // floats
  static constexpr int kVPitch = kDP + 4;    // floats; columns >= D are zero
  static constexpr int kKElems = kBC * kKPitch;
  static constexpr int kVElems = kBC * kVPitch;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kLdsBytes = 2 * kBufElems * 4;
  static constexpr int kItems = kBC * kChunks;
  static constexpr int kIter = (kItems + 255) / 256;
  static_assert(D % 8 == 0, "head_dim must be a multiple of 8");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdParams p) {
  using S = F32FwdShape<D>;
  extern __shared__ __attribute__((aligned(16))) float ldsf[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane & 31;
  const int g = lane >> 5;

  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int hk = h / p.group;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int q0 = qt * S::kBR;
  const int qrow = q0 + wave * 32 + lq;

  const float* qg = reinterpret_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh;
  const float* kg = reinterpret_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const float* vg = reinterpret_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh;

  // Q^T B operand: k slot kc of lane half g is d = g * D/2 + kc.
  float qop[S::kHalf];
  {
    const bool ok = qrow < p.Lq;
    const float* qr = qg + (int64_t)qrow * p.q_st + g * S::kHalf;
#pragma unroll
    for (int j = 0; j < S::kHalf / 4; ++j) {
      const u32x4 w = ok ? load16(qr + 4 * j) : zero16();
#pragma unroll
      for (int e = 0; e < 4; ++e) qop[4 * j + e] = __uint_as_float(w[e]);
    }
  }

  int kv_end = p.Lk;
  if (CAUSAL) kv_end = min(kv_end, q0 + S::kBR);
  const int n_tiles = (kv_end + S::kBC - 1) / S::kBC;
  const int wave_last_row = q0 + wave * 32 + 31;

  // Padding columns of V (d >= D) are zero in both buffers.
  if (S::kDP != D) {
    for (int i = tid; i < S::kBC * (S::kDP - D); i += 256) {
      const int row = i / (S::kDP - D), col = D + i % (S::kDP - D);
      ldsf[S::kKElems + row * S::kVPitch + col] = 0.f;
      ldsf[S::kBufElems + S::kKElems + row * S::kVPitch + col] = 0.f;
    }
  }

  u32x4 kreg[S::kIter], vreg[S::kIter];
  auto load_tile = [&](int t) {
    const int kv0 = t * S::kBC;
#pragma unroll
    for (int it = 0; it < S::kIter; ++it) {
      const int item = tid + 256 * it;
      const int row = item / S::kChunks;
      const int ch = item - row * S::kChunks;
      const bool ok = item < S::kItems && kv0 + row < p.Lk;
      kreg[it] = ok ? load16(kg + (int64_t)(kv0 + row) * p.k_st + 4 * ch) : zero16();
      vreg[it] = ok ? load16(vg + (int64_t)(kv0 + row) * p.v_st + 4 * ch) : zero16();
    }
  };
  auto store_tile = [&](int buf) {
    float* kl = ldsf + buf * S::kBufElems;
    float* vl = kl + S::kKElems;
#pragma unroll
    for (int it = 0; it < S::kIter; ++it) {
      const int item = tid + 256 * it;
      if (item < S::kItems) {
        const int row = item / S::kChunks;
        const int ch = item - row * S::kChunks;
        *reinterpret_cast<u32x4*>(kl + row * S::kKPitch + 4 * ch) = kreg[it];
        *reinterpret_cast<u32x4*>(vl + row * S::kVPitch + 4 * ch) = vreg[it];
      }
    }
  };

  f32x16 oacc[S::kND];
#pragma unroll
  for (int i = 0; i < S::kND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    __syncthreads();
    const int kv0 = t * S::kBC;
    const float* kl = ldsf + (t & 1) * S::kBufElems;
    const float* vl = kl + S::kKElems;
    if (!CAUSAL || kv0 <= wave_last_row) {
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      const float* krow = kl + lq * S::kKPitch + g * S::kHalf;
#pragma unroll
      for (int j = 0; j < S::kHalf / 4; ++j) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) s = mfma32_f32(__uint_as_float(a[e]), qop[4 * j + e], s);
      }
      const bool need_mask = (kv0 + S::kBC > p.Lk) || (CAUSAL && kv0 + S::kBC - 1 > q0 + wave * 32);
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[r] * p.scale_log2;
        if (need_mask) {
          const int key = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool vis = key < p.Lk && (!CAUSAL || key <= qrow);
          x = vis ? x : kNegInf;
        }
        s[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(s[r] - m_new);
        rs += s[r];
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < S::kND; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        // O^T += V^T P^T, one key pair (key(r, 0), key(r, 1)) per instruction.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * g + (r & 3);
          const float a = vl[key * S::kVPitch + 32 * db + lq];
          oacc[db] = mfma32_f32(a, s[r], oacc[db]);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
  }

  const float l_tot = sum_xor32(l_run);
  if (qrow < p.Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = reinterpret_cast<float*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qrow * p.o_st;
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        if (d < D) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(oacc[db][4 * j + e] * inv);
          *reinterpret_cast<u32x4*>(orow + d) = w;
        }
      }
    if (g == 0) {
      const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
      p.lse[((int64_t)b * p.Hq + h) * p.Lq + qrow] = lse;
    }
  }
}

}  // namespace attn_dev
