// Prefill attention forward, FP8 (e4m3) inputs, for gfx950.
//
// The FP8 variant of the tiled forward: "Flash Attention原理：分块计算与重计算"
// (cnblogs), section 六 and FAQ Q8, puts both products of the third version on
// 8-bit floating-point matrix units at twice the 16-bit rate.  The pages fix
// no format or scaling; here Q, K and V are e4m3 codes (1 sign, 4 exponent
// bits with bias 7, 3 mantissa bits; no infinity) and each tensor carries one
// fp32 descale, so an element stands for descale * value(code).
//
//   scores     S = (q_descale k_descale scale) Qc Kc^T   on the fp8 matrix core,
//                                                          fp32 accumulation
//   softmax    as in the bf16 kernel (reference max, sum guard, redo), fp32
//   P          each probability rounded to e4m3 (nearest even); the row sum l
//              adds the rounded values, so O is exactly a convex combination
//              of V rows with weights P~ / sum P~
//   O          v_descale (P~ Vc) / l, rounded to bf16; LSE = m + ln l
//
// Everything else follows the bf16 kernel: one workgroup of 4 waves per
// (batch, query head, 128 query rows), each wave 32 rows; transposed products
// S^T = K Q^T and O^T = V^T P^T so a lane owns one query; K/V tiles copied
// global -> LDS without registers, double buffered; XCD-aware work order.
// The FP8 product contracts 64 keys at once, so a key tile holds 128 keys,
// taken as two 64-key halves (the half granularity of the overlap of one
// half's softmax with the other half's products).
//
// Operand layouts of v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8, unit
// scales): lane l holds 32 bytes, A[m = l%32][k] and B[k][n = l%32], with the
// same lane/byte -> k assignment for A and B (so any fixed assignment of k
// slots works, as for the bf16 product); C as for the bf16 32x32 product.
//   Q K^T slice kc (64 head_dim bytes): lane half g holds bytes
//     64 kc + 16 g + 0..15 (dwords 0-3) and 64 kc + 32 + 16 g + 0..15 (4-7).
//   P V (64 keys of a half): P^T byte 16 j + r is accumulator register r of
//     the half's 32-key block j, i.e. key 32 j + 8 (r/4) + 4 g + r%4; the
//     V^T operand gathers the same keys with four byte-transposing LDS reads.
#pragma once

#include "fwd_bf16.h"

namespace attn_dev {

typedef __attribute__((__vector_size__(8 * sizeof(uint32_t)))) uint32_t u32x8;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

// 32x32x64 e4m3 product with fp32 accumulation; the E8M0 block scales are
// 127, i.e. 2^0, so this is a plain product.
__device__ __forceinline__ f32x16 mfma32_fp8(const u32x8& a, const u32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                         c, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 e4m3 product with fp32 accumulation (unit block scales).  Lane l
// holds A row l % 16 and B column l % 16, each with the 32 k values of
// k-group l / 16 (the same lane/byte -> k assignment for A and B); C row
// 4 (l / 16) + i, column l % 16 in register i.
__device__ __forceinline__ f32x4 mfma16_fp8(const u32x8& a, const u32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                          c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 values to e4m3 codes (nearest even) packed low byte first.  The
// first conversion writes the low half-word and keeps the high one of the
// word it is given, which the second conversion overwrites: any word will
// do, and a's bits (dead after this) save the zeroing a literal 0 costs.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int D>
struct Fp8FwdShape {
  static constexpr int kWaves = 4;
  static constexpr int kGroupsPerCU = 8 / kWaves;  // 2 waves per SIMD
  static constexpr int kRowsPerWave = 32;
  static constexpr int kBR = kRowsPerWave * kWaves;  // 128 query rows per workgroup
  static constexpr int kBC = 128;                     // keys per tile: two 64-key halves
  static constexpr int kKC = D / 64;                  // 64-deep slices of Q K^T
  static constexpr int kND = D / 32;                  // 32-row blocks of O^T
  static constexpr int kChunks = D / 16;              // 16-byte chunks per row (no padding)
  static constexpr int kRowBytes = D;
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kBufBytes = 2 * kTileBytes;    // K tile, then V tile
  static constexpr int kLdsBytes = 2 * kBufBytes;     // double buffered
  static constexpr int kRowsPerCopy = 64 / kChunks;   // rows one 1 KB copy fills
  static constexpr int kCopies = 2 * kBC / kRowsPerCopy;
  static constexpr int kCopiesPerWave = kCopies / kWaves;
  static constexpr int kKVar = 16 / kRowsPerCopy;     // copy patterns per 16-row swizzle period
  static_assert(D == 64 || D == 128, "FP8 head_dim is 64 or 128");
  static_assert(kCopiesPerWave % kKVar == 0 && (kWaves / 2) * kCopiesPerWave * kRowsPerCopy == kBC,
                "each wave copies whole swizzle periods of one of the two tiles");
  static_assert(kCopiesPerWave < 16, "the prologue's wait count fits the simple vmcnt encoding");
  static_assert(kBufBytes < 65536, "in-buffer LDS offsets must fit the instruction offset field");
};

// LDS swizzles (16-byte chunk c of row r is stored at chunk c ^ swz(r % 16)),
// chosen so that the operand reads hit distinct banks whether the LDS serves
// 128 or 256 bytes per cycle:
//   K, 16-byte reads of 16 consecutive rows at one logical chunk:
//     128-byte rows: (r & 7) ^ ((r >> 3) & 1); 64-byte rows:
//     ((r >> 2) & 3) ^ (((r >> 1) & 1) << 1).
//   V, byte-transposing reads: 16 lanes take one chunk of rows
//     {0,1,2,3,8,9,10,11} + 4 g (+16 t), and 32 lanes two adjacent chunks:
//     128-byte rows: (r & 3) | ((r >> 1) & 4); 64-byte rows:
//     ((r >> 1) & 1) | ((r >> 2) & 2).
template <int D>
__device__ __forceinline__ int fp8_k_swz(int r) {
  return D == 128 ? ((r & 7) ^ ((r >> 3) & 1)) : (((r >> 2) & 3) ^ (((r >> 1) & 1) << 1));
}
template <int D>
__device__ __forceinline__ int fp8_v_swz(int r) {
  return D == 128 ? ((r & 3) | ((r >> 1) & 4)) : (((r >> 1) & 1) | ((r >> 2) & 2));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * Fp8FwdShape<D>::kWaves, Fp8FwdShape<D>::kGroupsPerCU) void
attn_fwd_fp8_kernel(FwdParams p) {
  using S = Fp8FwdShape<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  lds_char* const lds_b = (lds_char*)(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31;
  const int g = lane >> 5;

  const WorkItem wi = prefill_work_item(p, CAUSAL);
  const int b = wi.b, h = wi.h, hk = wi.hk;
  const int q0 = wi.qt * S::kBR;
  if (q0 >= p.Lq) return;
  const int row0 = q0 + wave * S::kRowsPerWave;
  const int qrow = row0 + lq;

  const uint8_t* qg = reinterpret_cast<const uint8_t*>(p.q) + b * p.q_sb + h * p.q_sh;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + b * p.v_sb + hk * p.v_sh;

  // Q^T B operands (a negative total scale flips Q's sign bits, exactly).
  u32x8 qop[S::kKC];
  {
    const uint32_t flip = p.neg_q ? 0x80808080u : 0u;
    const bool ok = qrow < p.Lq;
    const uint8_t* qr = qg + (int64_t)qrow * p.q_st + 16 * g;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc) {
      const u32x4 lo = ok ? load16(qr + 64 * kc) : zero16();
      const u32x4 hi = ok ? load16(qr + 64 * kc + 32) : zero16();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qop[kc][e] = lo[e] ^ flip;
        qop[kc][4 + e] = hi[e] ^ flip;
      }
    }
  }
  const float c = p.scale_log2_abs;

  int kv_end = p.Lk;
  if (CAUSAL) kv_end = min(kv_end, q0 + S::kBR);
  const int n_tiles = (kv_end + S::kBC - 1) / S::kBC;
  const int n_full = p.Lk / S::kBC;
  const int wave_last_row = row0 + S::kRowsPerWave - 1;

  // ---- tile copies (as in the bf16 kernel: waves 0-1 copy K, 2-3 copy V) ----
  const bool copies_k = wave < S::kWaves / 2;
  const uint8_t* cp_src = copies_k ? kg : vg;
  const int64_t cp_st = copies_k ? p.k_st : p.v_st;
  const int cp_row = lane / S::kChunks;
  const int cp_row0 = S::kRowsPerCopy * ((wave % (S::kWaves / 2)) * S::kCopiesPerWave);
  const uint32_t cp_lds0 = (uint32_t)(uintptr_t)lds_b + (copies_k ? 0 : S::kTileBytes) + cp_row0 * S::kRowBytes;
  int cp_chunk16[S::kKVar];
  uint32_t cp_off[S::kKVar];
  const uint32_t cp_row_bytes = (uint32_t)cp_st;  // < 2^28: token strides are validated
#pragma unroll
  for (int v = 0; v < S::kKVar; ++v) {
    const int r = S::kRowsPerCopy * v + cp_row;  // row modulo the 16-row swizzle period
    const int pc = lane % S::kChunks;
    const int lc = pc ^ (copies_k ? fp8_k_swz<D>(r) : fp8_v_swz<D>(r));
    cp_chunk16[v] = 16 * lc;
    cp_off[v] = (uint32_t)cp_row * cp_row_bytes + 16 * lc;
  }
  auto issue_tile = [&](int t) {
    const int kv0 = t * S::kBC;
    const uint32_t dst = cp_lds0 + (t & 1) * S::kBufBytes;
    if (t < n_full) {
#pragma unroll
      for (int j = 0; j < S::kCopiesPerWave; ++j)
        fwd_copy16(cp_src + (int64_t)(kv0 + cp_row0 + S::kRowsPerCopy * j) * cp_st, cp_off[j % S::kKVar],
                   dst + j * S::kRowsPerCopy * S::kRowBytes);
    } else {
      // the tile holding key Lk - 1 repeats that row past it (masked to -inf)
      const int last = p.Lk - 1;
#pragma unroll
      for (int j = 0; j < S::kCopiesPerWave; ++j) {
        const int r0 = min(kv0 + cp_row0 + S::kRowsPerCopy * j, last);
        const int rr = min(kv0 + cp_row0 + S::kRowsPerCopy * j + cp_row, last);
        fwd_copy16(cp_src + (int64_t)r0 * cp_st, (uint32_t)(rr - r0) * cp_row_bytes + cp_chunk16[j % S::kKVar],
                   dst + j * S::kRowsPerCopy * S::kRowBytes);
      }
    }
    copy_group_end();
  };

  // ---- LDS operand offsets (bytes within a buffer) ----
  // K A operand, block row lq: chunks 4 kc + g (dwords 0-3) and 4 kc + 2 + g
  // (dwords 4-7); the swizzle flips chunk bits only, so both are slice 0's
  // offset with bits 5 and up flipped.
  const int k_rd = lq * S::kRowBytes + 16 * (fp8_k_swz<D>(lq) ^ g);
  // V^T A operand of d-block db, read t (keys 16 t .. 16 t + 15 of a half):
  // lane (G = lane / 16, e = lane % 16 / 2, hh = lane % 2) points at key row
  // 16 t + 8 (e / 4) + 4 (G / 2) + e % 4, head_dim bytes 32 db + 16 (G % 2) +
  // 8 hh; the transposing read hands lane (G, 8 hh' + b') byte e of the row
  // lane 16 G + 2 e + hh' points at, i.e. head_dim 32 db + 16 (G % 2) + 8 hh' +
  // b' of keys 16 t + {0..3, 8..11} + 4 g: P^T bytes 8 t .. 8 t + 7.
  int v_rd[S::kND];
  {
    const int G = lane >> 4, e = (lane & 15) >> 1, hh = lane & 1;
    const int rr = 8 * (e >> 2) + 4 * (G >> 1) + (e & 3);
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
      v_rd[db] = S::kTileBytes + rr * S::kRowBytes + 16 * ((2 * db + (G & 1)) ^ fp8_v_swz<D>(rr)) + 8 * hh;
  }

  f32x16 oacc[S::kND];
#pragma unroll
  for (int i = 0; i < S::kND; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;  // l_run: the whole row's sum, in both lanes of the query

  // Row sums of P~ on the matrix core.  Read as the B operand of a 16x16x128
  // product, the P^T operand of lane l sits in column l % 16, k-group
  // j = l / 16, and holds 32 keys of query l % 32: k-groups 0 and 2 hold the
  // 64 keys of queries 0-15, k-groups 1 and 3 those of queries 16-31.  An A
  // operand whose row m is e4m3 1.0 on the k-groups j with j % 2 ==
  // (m / 4) % 2 (zero on the others) makes C row m, column n the sum over
  // the half's 64 keys of query n + 16 ((m / 4) % 2); register 0 of lane l
  // (row 4 (l / 16), column l % 16) is then the sum for query l % 32.
  u32x8 sum_sel;
  {
    const uint32_t w = ((lane >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum_sel[i] = w;
  }

  u32x8 ka_next[2][S::kKC];  // K operands of the next tile's first half (two 32-key blocks)
  u32x8 va_last[S::kND];     // V^T operands of this tile's second half
  u32x8 pop[2];              // P^T operands of the two halves
  auto read_k = [&](int buf, int sb, u32x8 (&ka)[2][S::kKC]) {
    const lds_char* kb = lds_b + buf * S::kBufBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) {
        const lds_char* row = kb + (64 * sb + 32 * j) * S::kRowBytes;
        const u32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(row + (k_rd ^ (64 * kc)));
        const u32x4 hi =
            *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(row + (k_rd ^ (64 * kc + 32)));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ka[j][kc][e] = lo[e];
          ka[j][kc][4 + e] = hi[e];
        }
      }
  };
  auto pv = [&](int sb, const u32x8 (&va)[S::kND]) {
#pragma unroll
    for (int db = 0; db < S::kND; ++db) oacc[db] = mfma32_fp8(va[db], pop[sb], oacc[db]);
  };
  auto tile_back = [&] {
    __builtin_amdgcn_s_setprio(2);
    pv(1, va_last);
    __builtin_amdgcn_s_setprio(0);
  };
  auto tile_front = [&](auto mask_tag, int buf, int kv0) {
    constexpr bool MASK = decltype(mask_tag)::value;
    lds_char* vb = lds_b + buf * S::kBufBytes;
    f32x16 s[2][2];  // [half][32-key block]
    auto read_v = [&](int sb, u32x8 (&va)[S::kND]) {
#pragma unroll
      for (int db = 0; db < S::kND; ++db)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          lds_char* a = vb + v_rd[db] + (64 * sb + 16 * t) * S::kRowBytes;
          const u32x2 w = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)a));
          const uint32_t w0 = w[0], w1 = w[1];
          va[db][2 * t] = w0;
          va[db][2 * t + 1] = w1;
        }
    };
    auto qk = [&](int sb, const u32x8 (&ka)[2][S::kKC]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][j][r] = 0.f;
#pragma unroll
        for (int kc = 0; kc < S::kKC; ++kc) s[sb][j] = mfma32_fp8(ka[j][kc], qop[kc], s[sb][j]);
      }
    };
    // P~ = e4m3(exp2(c s - m)) for half sb, packed as the P^T operand;
    // returns the half's row sum of P~ for this lane's query, formed on the
    // matrix core from the same rounded values that weight V (fp32
    // accumulation), without unpacking them on the vector ALU: see sum_sel.
    auto exp_half = [&](int sb) {
      const float neg_m = -m_run;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) e[i] = fast_exp2(__builtin_fmaf(s[sb][j][4 * q + i], c, neg_m));
          pop[sb][4 * j + q] = pack_e4m3x4(e[0], e[1], e[2], e[3]);
        }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      return mfma16_fp8(sum_sel, pop[sb], z)[0];
    };
    auto softmax_half = [&](int sb, auto n_mfma_tag) {
      constexpr int N_MFMA = decltype(n_mfma_tag)::value;
      if constexpr (MASK) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 64 * sb + 32 * j + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool vis = key < p.Lk && (!CAUSAL || key <= qrow);
            s[sb][j][r] = vis ? s[sb][j][r] : kNegInf;
          }
      }
      float ls = exp_half(sb);
      const bool redo = !(ls <= kSumGuard);
#pragma unroll
      for (int i = 0; i < N_MFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 80 / N_MFMA, 0);
      }
      if (__builtin_amdgcn_ballot_w64(redo) != 0) {
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][j][r]);
        const float m_new = fmaxf(m_run, max_xor32(mx) * c);
        const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < S::kND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        ls = exp_half(sb);
      }
      l_run += ls;
    };

    constexpr int kQKMfma = 2 * S::kKC, kPVMfma = S::kND;
    u32x8 ka1[2][S::kKC], va0[S::kND];
    read_k(buf, 1, ka1);
    __builtin_amdgcn_s_setprio(2);
    qk(0, ka_next);
    __builtin_amdgcn_s_setprio(0);
    read_v(0, va0);
    qk(1, ka1);
    softmax_half(0, std::integral_constant<int, kQKMfma>{});
    read_v(1, va_last);
    pv(0, va0);
    softmax_half(1, std::integral_constant<int, kPVMfma>{});
  };

  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): Q has landed before the copies start
  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) {
    issue_tile(1);
    __builtin_amdgcn_s_waitcnt(0x0f70 | S::kCopiesPerWave);  // vmcnt: tile 0's copies done
  } else {
    __builtin_amdgcn_s_waitcnt(0x0f70);
  }
  __syncthreads();
  auto active = [&](int t) { return !CAUSAL || t * S::kBC <= wave_last_row; };
  if (n_tiles > 0 && active(0)) read_k(0, 0, ka_next);

  auto step = [&](auto mask_tag, int t) {
    const bool act = active(t);
    if (act) tile_front(mask_tag, t & 1, t * S::kBC);
    if (t + 1 < n_tiles) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      __syncthreads();
      if (t + 2 < n_tiles) issue_tile(t + 2);
      if (active(t + 1)) read_k((t + 1) & 1, 0, ka_next);
    }
    if (act) tile_back();
  };
  int n_plain = min(n_tiles, n_full);
  if (CAUSAL) n_plain = min(n_plain, (q0 + 1) / S::kBC);
  int t = 0;
  for (; t < n_plain; ++t) step(std::false_type{}, t);
  for (; t < n_tiles; ++t) step(std::true_type{}, t);

  // ---- epilogue: O = v_descale O_acc / l, LSE = (m + log2 l) ln 2 ----
  const float l_tot = l_run;
  if (qrow < p.Lq) {
    const float mul = l_tot > 0.f ? p.o_mul / l_tot : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qrow * p.o_st;
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * j + 0] * mul, oacc[db][4 * j + 1] * mul);
        w[1] = pack_bf16x2(oacc[db][4 * j + 2] * mul, oacc[db][4 * j + 3] * mul);
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    if (g == 0) {
      const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
      p.lse[b * p.lse_sb + h * p.lse_sh + qrow] = lse;
    }
  }
}

}  // namespace attn_dev
