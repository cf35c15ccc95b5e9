// Attention backward, bf16 inputs, for gfx950: dQ, dK, dV by recomputation.
//
// Method: "Flash Attention原理：分块计算与重计算" (cnblogs), section 五: the
// forward keeps only the row statistics (here LSE = m + ln l) and the backward
// recomputes the probabilities tile by tile from them, P = exp(S - LSE), never
// storing S or P.  The gradients are the chain rule through S = Q K^T * scale,
// P = softmax(S), O = P V (the pages state that the derivation exists, not its
// steps): dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with D = rowsum(dO * O),
// dQ = scale dS K, dK = scale dS^T Q.
//
// Three kernels:
//   * attn_bwd_delta_kernel: D per query row (fp32, into the workspace);
//   * attn_bwd_dkdv_kernel: one workgroup per (batch, kv head, 128 keys); each
//     wave keeps its 32 keys' K and V in registers and walks the query heads of
//     the group and their 32-query tiles (Q, dO, LSE and D staged in LDS), so
//     dK and dV of a grouped head are summed without atomics;
//   * attn_bwd_dq_kernel: one workgroup per (batch, query head, 128 queries);
//     each wave keeps its 32 queries' Q, dO, LSE and D in registers and walks
//     32-key tiles of K and V staged in LDS.
// Both products of a tile that contract over its rows (dV^T += dO^T P,
// dK^T += Q^T dS, dQ^T += K^T dS^T) take their A operand from the transposing
// LDS read ds_read_b64_tr_b16 on the row-major tile, visiting the rows in the
// order in which the score accumulator holds them, so that P and dS go from
// the accumulator to the B operand without a shuffle.
//
// Matrix layouts (v_mfma_f32_32x32x16_bf16, lane l, half g = l / 32):
//   A[m][k]: lane l holds m = l % 32, k = 8g .. 8g+7;
//   B[k][n]: lane l holds n = l % 32, k = 8g .. 8g+7;
//   C[m][n]: register r of lane l holds m = 8(r/4) + 4g + r%4, n = l % 32.
// Causal is top-left (query i sees keys j <= i).  Rows past Lq and keys past
// Lk are loaded from the last valid row (in bounds, finite) and masked.
#pragma once

#include "device_common.h"

namespace attn_dev {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, Hq, Lq] from the forward
  float* delta;      // workspace [B, Hq, Lq]
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t o_sb, o_sh, o_st;
  int64_t do_sb, do_sh, do_st;
  int64_t dq_sb, dq_sh, dq_st;
  int64_t dk_sb, dk_sh, dk_st;
  int64_t dv_sb, dv_sh, dv_st;
  int B, Hq, Hkv, group, Lq, Lk;
  float scale;       // softmax scale (signed)
  float scale_log2;  // scale * log2(e)
};

constexpr int kBwdRows = 32;  // rows of a staged tile (queries or keys)

template <int D>
struct BwdShape {
  static constexpr int kKC = D / 16;     // k-slices over head_dim
  static constexpr int kND = D / 32;     // 32-row blocks of a transposed gradient
  static constexpr int kPitch = D + 8;   // row pitch in LDS (elements): 16-byte rows, spread banks
  static constexpr int kTile = kBwdRows * kPitch;       // elements of one staged tile
  static constexpr int kChunks = kBwdRows * D / 8;      // 16-byte chunks of one tile
  static constexpr int kIter = (kChunks + 255) / 256;   // per thread, per tensor
  static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
};

// ---------------------------------------------------------------- delta
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= (int64_t)p.B * p.Hq * p.Lq) return;
  const int i = (int)(row % p.Lq);
  const int64_t bh = row / p.Lq;
  const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
  const uint16_t* orow = reinterpret_cast<const uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_st;
  const uint16_t* drow =
      reinterpret_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)i * p.do_st;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 a = load16(orow + 8 * c), d = load16(drow + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(d[e]) + bf16_hi(a[e]) * bf16_hi(d[e]);
  }
  p.delta[row] = acc;
}

// Per-lane byte offset of the A operand X^T (32 head-dim rows of block db x 16
// tile rows of slice cs) read with ds_read_b64_tr_b16 from a row-major tile:
// lane (G = l/16, i = l%16/4, q = l%4) points at tile row 16 cs + 4 g + i,
// head-dim 32 db + 16 (G & 1) + 4 q; the second read is 8 rows further.
template <int D>
__device__ __forceinline__ int bwd_tr_offset(int lane, int db) {
  using S = BwdShape<D>;
  const int g = lane >> 5, G = lane >> 4, i = (lane & 15) >> 2, q = lane & 3;
  return ((4 * g + i) * S::kPitch + 32 * db + 16 * (G & 1) + 4 * q) * 2;
}

template <int D>
__device__ __forceinline__ u32x4 bwd_tr_read(const char* tile, int off, int cs) {
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  using S = BwdShape<D>;
  const char* a0 = tile + off + 16 * cs * S::kPitch * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) const char*)a0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) const char*)(a0 + 8 * S::kPitch * 2));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Stage rows r0 .. r0+31 (clamped to last) of a [rows, D] tensor into a tile.
template <int D>
struct BwdTileLoader {
  using S = BwdShape<D>;
  u32x4 reg[S::kIter];
  __device__ __forceinline__ void load(const uint16_t* base, int64_t st, int r0, int last, int tid) {
#pragma unroll
    for (int it = 0; it < S::kIter; ++it) {
      const int c = tid + 256 * it;
      if (S::kChunks % 256 == 0 || c < S::kChunks) {
        const int row = c / (D / 8), ch = c % (D / 8);
        reg[it] = load16(base + (int64_t)min(r0 + row, last) * st + 8 * ch);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int it = 0; it < S::kIter; ++it) {
      const int c = tid + 256 * it;
      if (S::kChunks % 256 == 0 || c < S::kChunks) {
        const int row = c / (D / 8), ch = c % (D / 8);
        *reinterpret_cast<u32x4*>(tile + row * S::kPitch + 8 * ch) = reg[it];
      }
    }
  }
};

// ---------------------------------------------------------------- dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  using S = BwdShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lq_tile[2][S::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t ldo_tile[2][S::kTile];
  __shared__ __attribute__((aligned(16))) float lstat[2][2][kBwdRows];  // [buf][lse2, delta][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  const int n_kb = (p.Lk + 127) / 128;
  const int kb = blockIdx.x % n_kb;
  const int bh = blockIdx.x / n_kb;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int k0 = kb * 128;
  const int wave_k0 = k0 + 32 * wave;
  const int key = wave_k0 + ln;  // this lane's key column

  // K^T and V^T as B operands of S = Q K^T and dP = dO V^T: lane holds row
  // `key` of K (V), head-dim 16 kc + 8 g .. +8.  Keys past Lk are zero.
  u32x4 kop[S::kKC], vop[S::kKC];
  {
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)key * p.k_st;
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)key * p.v_st;
    const bool ok = key < p.Lk;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc) {
      kop[kc] = ok ? load16(kr + 16 * kc + 8 * g) : zero16();
      vop[kc] = ok ? load16(vr + 16 * kc + 8 * g) : zero16();
    }
  }
  f32x16 dk_acc[S::kND], dv_acc[S::kND];
#pragma unroll
  for (int db = 0; db < S::kND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk_acc[db][r] = dv_acc[db][r] = 0.f;

  const int tr_off0 = bwd_tr_offset<D>(lane, 0);
  const int n_qt = (p.Lq + kBwdRows - 1) / kBwdRows;
  const int qt0 = CAUSAL ? min(k0 / kBwdRows, n_qt) : 0;  // tiles before hold only queries < k0
  const int tiles_per_head = n_qt - qt0;
  const int n_steps = p.group * tiles_per_head;
  const float c = p.scale_log2;
  constexpr float kLog2eF = 1.4426950408889634f;

  BwdTileLoader<D> lq_ld, ldo_ld;
  float st_reg[2] = {0.f, 0.f};  // this thread's LSE (scaled to log2) and D, threads 0..31
  auto load_step = [&](int step) {
    const int hg = step / tiles_per_head, qt = qt0 + step % tiles_per_head;
    const int h = hk * p.group + hg;
    const int r0 = qt * kBwdRows;
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh;
    const uint16_t* db = reinterpret_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh;
    lq_ld.load(qb, p.q_st, r0, p.Lq - 1, tid);
    ldo_ld.load(db, p.do_st, r0, p.Lq - 1, tid);
    if (tid < kBwdRows) {
      const int64_t si = ((int64_t)b * p.Hq + h) * p.Lq + min(r0 + tid, p.Lq - 1);
      st_reg[0] = p.lse[si] * kLog2eF;
      st_reg[1] = p.delta[si];
    }
  };
  auto store_step = [&](int buf) {
    lq_ld.store(lq_tile[buf], tid);
    ldo_ld.store(ldo_tile[buf], tid);
    if (tid < kBwdRows) {
      lstat[buf][0][tid] = st_reg[0];
      lstat[buf][1][tid] = st_reg[1];
    }
  };

  if (n_steps > 0) {
    load_step(0);
    store_step(0);
  }
  for (int step = 0; step < n_steps; ++step) {
    const int buf = step & 1;
    if (step + 1 < n_steps) load_step(step + 1);
    __syncthreads();
    const int qt = qt0 + step % tiles_per_head;
    const int r0 = qt * kBwdRows;
    // A wave whose keys all come after the tile's last query has nothing here.
    if (!CAUSAL || r0 + kBwdRows - 1 >= wave_k0) {
      const uint16_t* qt_l = lq_tile[buf];
      const uint16_t* dt_l = ldo_tile[buf];
      // S = Q K^T and dP = dO V^T: rows = the tile's 32 queries, columns = keys.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) {
        const u32x4 qa = *reinterpret_cast<const u32x4*>(qt_l + ln * S::kPitch + 16 * kc + 8 * g);
        const u32x4 da = *reinterpret_cast<const u32x4*>(dt_l + ln * S::kPitch + 16 * kc + 8 * g);
        s = mfma32(qa, kop[kc], s);
        dp = mfma32(da, vop[kc], dp);
      }
      // The row statistics of this lane's 16 query rows 8 j + 4 g + 0..3.
      f32x4 lse4[4], dl4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lse4[j] = *reinterpret_cast<const f32x4*>(&lstat[buf][0][8 * j + 4 * g]);
        dl4[j] = *reinterpret_cast<const f32x4*>(&lstat[buf][1][8 * j + 4 * g]);
      }
      // P = exp2(c S - LSE log2 e) (recomputed), dS = P (dP - D); both packed
      // as the B operands of the two 16-query slices.
      u32x4 pb[2], dsb[2];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        float pe[8], de[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * cs + e;
          const int qrow = r0 + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool vis = qrow < p.Lq && key < p.Lk && (!CAUSAL || key <= qrow);
          const float pv = vis ? fast_exp2(__builtin_fmaf(s[r], c, -lse4[r >> 2][r & 3])) : 0.f;
          pe[e] = pv;
          de[e] = pv * (dp[r] - dl4[r >> 2][r & 3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[cs][j] = pack_bf16x2(pe[2 * j], pe[2 * j + 1]);
          dsb[cs][j] = pack_bf16x2(de[2 * j], de[2 * j + 1]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS (rows = head_dim, columns = keys).
#pragma unroll
      for (int db = 0; db < S::kND; ++db)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          const u32x4 dta = bwd_tr_read<D>(reinterpret_cast<const char*>(dt_l), tr_off0 + 64 * db, cs);
          const u32x4 qta = bwd_tr_read<D>(reinterpret_cast<const char*>(qt_l), tr_off0 + 64 * db, cs);
          dv_acc[db] = mfma32(dta, pb[cs], dv_acc[db]);
          dk_acc[db] = mfma32(qta, dsb[cs], dk_acc[db]);
        }
    }
    // The other buffer was last read before this iteration's barrier.
    if (step + 1 < n_steps) store_step(buf ^ 1);
  }

  // dK = scale dK_acc, dV = dV_acc: lane = key, registers = head-dim rows.
  if (key < p.Lk) {
    uint16_t* dkr = reinterpret_cast<uint16_t*>(p.dk) + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_st;
    uint16_t* dvr = reinterpret_cast<uint16_t*>(p.dv) + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_st;
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk_acc[db][4 * j + 0] * p.scale, dk_acc[db][4 * j + 1] * p.scale);
        wk[1] = pack_bf16x2(dk_acc[db][4 * j + 2] * p.scale, dk_acc[db][4 * j + 3] * p.scale);
        wv[0] = pack_bf16x2(dv_acc[db][4 * j + 0], dv_acc[db][4 * j + 1]);
        wv[1] = pack_bf16x2(dv_acc[db][4 * j + 2], dv_acc[db][4 * j + 3]);
        *reinterpret_cast<u32x2*>(dkr + d) = wk;
        *reinterpret_cast<u32x2*>(dvr + d) = wv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdParams p) {
  using S = BwdShape<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lk_tile[2][S::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t lv_tile[2][S::kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  const int n_qb = (p.Lq + 127) / 128;
  const int qb = blockIdx.x % n_qb;
  const int bh = blockIdx.x / n_qb;
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / p.group;
  const int q0 = qb * 128;
  const int wave_q0 = q0 + 32 * wave;
  const int qrow = wave_q0 + ln;  // this lane's query column
  const bool qok = qrow < p.Lq;

  // Q^T and dO^T as B operands of S^T = K Q^T and dP^T = V dO^T.
  u32x4 qop[S::kKC], dop[S::kKC];
  {
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)qrow * p.q_st;
    const uint16_t* dr =
        reinterpret_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)qrow * p.do_st;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc) {
      qop[kc] = qok ? load16(qr + 16 * kc + 8 * g) : zero16();
      dop[kc] = qok ? load16(dr + 16 * kc + 8 * g) : zero16();
    }
  }
  constexpr float kLog2eF = 1.4426950408889634f;
  const int64_t si = ((int64_t)b * p.Hq + h) * p.Lq + min(qrow, p.Lq - 1);
  const float lse2 = qok ? p.lse[si] * kLog2eF : 0.f;
  const float dl = qok ? p.delta[si] : 0.f;
  const float c = p.scale_log2;

  f32x16 dq_acc[S::kND];
#pragma unroll
  for (int db = 0; db < S::kND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.f;

  int n_kt = (p.Lk + kBwdRows - 1) / kBwdRows;
  if (CAUSAL) n_kt = min(n_kt, (q0 + 127) / kBwdRows + 1);
  const int tr_off0 = bwd_tr_offset<D>(lane, 0);
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh;
  BwdTileLoader<D> lk_ld, lv_ld;

  if (n_kt > 0) {
    lk_ld.load(kbase, p.k_st, 0, p.Lk - 1, tid);
    lv_ld.load(vbase, p.v_st, 0, p.Lk - 1, tid);
    lk_ld.store(lk_tile[0], tid);
    lv_ld.store(lv_tile[0], tid);
  }
  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_kt) {
      lk_ld.load(kbase, p.k_st, (t + 1) * kBwdRows, p.Lk - 1, tid);
      lv_ld.load(vbase, p.v_st, (t + 1) * kBwdRows, p.Lk - 1, tid);
    }
    __syncthreads();
    const int kv0 = t * kBwdRows;
    if (!CAUSAL || kv0 <= wave_q0 + 31) {
      const uint16_t* kt_l = lk_tile[buf];
      const uint16_t* vt_l = lv_tile[buf];
      // S^T = K Q^T and dP^T = V dO^T: rows = the tile's 32 keys, columns = queries.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(kt_l + ln * S::kPitch + 16 * kc + 8 * g);
        const u32x4 va = *reinterpret_cast<const u32x4*>(vt_l + ln * S::kPitch + 16 * kc + 8 * g);
        s = mfma32(ka, qop[kc], s);
        dp = mfma32(va, dop[kc], dp);
      }
      // dS^T = P^T (dP^T - D), P^T recomputed from the LSE; packed as the B
      // operands of the two 16-key slices.
      u32x4 dsb[2];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        float de[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * cs + e;
          const int kk = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool vis = kk < p.Lk && (!CAUSAL || kk <= qrow);
          const float pv = vis ? fast_exp2(__builtin_fmaf(s[r], c, -lse2)) : 0.f;
          de[e] = pv * (dp[r] - dl);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dsb[cs][j] = pack_bf16x2(de[2 * j], de[2 * j + 1]);
      }
      // dQ^T += K^T dS^T (rows = head_dim, columns = queries).
#pragma unroll
      for (int db = 0; db < S::kND; ++db)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
          dq_acc[db] = mfma32(bwd_tr_read<D>(reinterpret_cast<const char*>(kt_l), tr_off0 + 64 * db, cs), dsb[cs],
                              dq_acc[db]);
    }
    // The other buffer was last read before this iteration's barrier.
    if (t + 1 < n_kt) {
      lk_ld.store(lk_tile[buf ^ 1], tid);
      lv_ld.store(lv_tile[buf ^ 1], tid);
    }
  }

  if (qok) {
    uint16_t* dqr = reinterpret_cast<uint16_t*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)qrow * p.dq_st;
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(dq_acc[db][4 * j + 0] * p.scale, dq_acc[db][4 * j + 1] * p.scale);
        w[1] = pack_bf16x2(dq_acc[db][4 * j + 2] * p.scale, dq_acc[db][4 * j + 3] * p.scale);
        *reinterpret_cast<u32x2*>(dqr + d) = w;
      }
  }
}

}  // namespace attn_dev
