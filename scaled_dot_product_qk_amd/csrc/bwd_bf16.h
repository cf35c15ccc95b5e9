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
//   * attn_bwd_delta_kernel: per query row, (LSE log2 e, D) into the workspace
//     (each row read by a group of adjacent lanes, whole rows per load);
//   * attn_bwd_dkdv_kernel: one workgroup per (batch, kv head, 128 keys); each
//     key group of 32 keeps its K and V in registers and walks the 32-query
//     tiles of the group's query heads (Q, dO and the row statistics staged
//     through registers into LDS), so dK and dV of a grouped head are summed
//     without atomics; at head_dim 128 two waves serve a key group, one
//     forming P and dV, the other dS and dK;
//   * attn_bwd_dq_kernel: one workgroup per (batch, query head, 256 queries,
//     128 at head_dim 64);
//     each wave keeps its 32 queries' Q, dO, LSE and D in registers and walks
//     32-key tiles of K and V staged through registers into LDS.
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

#include <type_traits>

#include "device_common.h"

namespace attn_dev {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, Hq, Lq] from the forward
  float* stats;      // workspace [B, Hq, Lq][2]: (LSE log2 e, D = rowsum(dO * O)) per query row
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
  int kv_round1;     // dK/dV: key blocks per (batch, kv head) resident from the start (causal step order)
  float scale;       // softmax scale (signed)
  float scale_log2;  // scale * log2(e)
};

constexpr int kBwdRows = 32;  // rows of a staged tile (queries or keys)

// ---------------------------------------------------------------- delta
// A row's 16-byte chunks are spread over kDeltaLanes<D> adjacent lanes, so
// each load instruction reads whole rows (coalesced); the lanes' partial dot
// products are then summed across the group.
template <int D>
constexpr int kDeltaLanes = D / 8 <= 8 ? 8 : 16;
template <int D>
constexpr int kDeltaRowsPerBlock = 4 * (64 / kDeltaLanes<D>);

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  constexpr int C = D / 8;  // 16-byte chunks of a row
  constexpr int LPR = kDeltaLanes<D>;
  static_assert(C <= LPR, "a row's chunks fit its lane group");
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Lq;
  const int64_t row = (int64_t)blockIdx.x * kDeltaRowsPerBlock<D> + (threadIdx.x >> 6) * (64 / LPR) + lane / LPR;
  float acc = 0.f;
  if (row < nrows && sub < C) {
    const int i = (int)(row % p.Lq);
    const int64_t bh = row / p.Lq;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const u32x4 a = load16(reinterpret_cast<const uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_st +
                           8 * sub);
    const u32x4 d = load16(reinterpret_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh +
                           (int64_t)i * p.do_st + 8 * sub);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(d[e]) + bf16_hi(a[e]) * bf16_hi(d[e]);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (sub == 0 && row < nrows) {
    p.stats[2 * row] = p.lse[row] * kLog2e;
    p.stats[2 * row + 1] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
// Largest Q, dO token stride (elements) the direct copies of the
// single-wave dK/dV kernels allow: a lane's 32-bit offset spans up to 31 rows
// of one 32-row tile.  (K and V are held to the same bound.)
constexpr int64_t kBwdMaxTokenStride = int64_t(1) << 26;

// dK/dV workgroup: 128 keys in 4 groups of 32.  Below head_dim 128 one wave
// serves each group and forms S, dP, P, dS and both gradients.  At head_dim
// 128 that would need more than 256 registers, so each group is served by
// two waves that split the work by gradient: the P wave forms S = Q K^T and
// P, hands P to its partner through LDS and accumulates dV; the dS wave
// forms dP = dO V^T, and after the next barrier takes P, forms dS and
// accumulates dK.  Each product is formed once, and the two waves of a group
// have the same matrix work per step.  Each step moves a 32-row Q tile, a
// 32-row dO tile and the rows' (LSE log2 e, D) pairs into LDS (below).
template <int D>
struct BwdKvShape {
  static constexpr bool kRoles = D == 128;
  static constexpr int kWaves = kRoles ? 8 : 4;
  static constexpr int kKC = D / 16;                  // k-slices over head_dim
  static constexpr int kND = (D + 31) / 32;           // 32-row head_dim blocks (the last padded at d = 80)
  static constexpr int kChunks = D / 8;               // 16-byte chunks of a row in memory
  static constexpr int kPitch = D <= 64 ? 8 : 16;     // 16-byte chunks of a row in LDS
  static constexpr int kRowBytes = 16 * kPitch;
  static constexpr int kTileBytes = kBwdRows * kRowBytes;
  static constexpr int kStatBytes = kBwdRows * 8;
  static constexpr int kStageBytes = 2 * kTileBytes + kStatBytes;  // Q, dO, statistics
  // Tile copies.  With two roles they are staged through registers: loaded
  // two steps before they are written to LDS, written two steps ahead of the
  // one computed (direct global-to-LDS copies made that kernel about a fifth
  // slower).  A single wave copies straight into LDS, three steps ahead: its
  // registers have no room for staging, and there the direct copies measured
  // faster.  Four buffers either way; with two roles the dS wave reads a
  // step's Q tile after the next barrier.
  static constexpr bool kStaged = kRoles;
  static constexpr int kAhead = 3;  // direct copies: steps in flight beyond the one computed
  static constexpr int kStages = 4;
  static constexpr int kPBytes = 64 * 16 * 4;         // one group's fp32 P tile, 16 values per lane
  static constexpr int kXchgBytes = kRoles ? 2 * 4 * kPBytes : 0;  // two slots per key group
  static constexpr int kLdsBytes = kStages * kStageBytes + kXchgBytes;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kCopiesPerTile = kBwdRows / kRowsPerCopy;
  static constexpr int kCopiesPerWave = 2 * kCopiesPerTile / kWaves;  // plus the statistics for wave 0
  static_assert(kCopiesPerWave * kWaves == 2 * kCopiesPerTile, "copies split evenly over the waves");
  static_assert(kCopiesPerTile % kCopiesPerWave == 0, "a wave copies from one tile only");
  static_assert(kChunks <= kPitch, "rows fit their pitch");
};

// LDS layout of a staged Q or dO row r: 16-byte chunk c at c ^ bwd_swz(r).
// The rows are read two ways: 16 consecutive rows at one chunk (A operands of
// S = Q K^T, dP = dO V^T) and, by the transposing read, 4 consecutive rows x
// 2 (or 4) adjacent chunks per 16 (32) lanes; both hit distinct banks.
//   256-byte rows: ((r & 3) << 2) | ((r >> 2) & 3);
//   128-byte rows: (((r >> 1) & 1) << 2) | ((r >> 2) & 3).
// Head_dim 80 rows (10 chunks) take 256-byte rows; chunks 10-15 are padding.
template <int PITCH>
__device__ __forceinline__ int bwd_swz(int r) {
  return PITCH == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * BwdKvShape<D>::kWaves, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  using S = BwdKvShape<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_raw[];
  lds_char* const lds = (lds_char*)lds_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  const int kgrp = wave & 3;
  // With two roles, waves 0-3 are the P waves (dV) and 4-7 the dS waves (dK).
  const bool ds_wave = S::kRoles && wave >= 4;
  const bool p_wave = !ds_wave;
  const bool do_dv = !S::kRoles || p_wave, do_dk = !S::kRoles || ds_wave;
  // Key blocks slowest (heaviest first when causal), (batch, kv head)
  // fastest, so that the key blocks of one kv head run on one XCD.
  const int n_bh = p.B * p.Hkv;
  const int kb = blockIdx.x / n_bh, bh = blockIdx.x % n_bh;
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int k0 = kb * 128;
  const int wave_k0 = k0 + 32 * kgrp;
  const int key = wave_k0 + ln;  // this lane's key column

  // K^T (P wave) and V^T (dS wave) as B operands of S = Q K^T and dP = dO V^T:
  // lane holds row `key` of K (V), head-dim 16 kc + 8 g .. +8.  Keys past Lk
  // are zero.  A single wave holds both.
  u32x4 kop[S::kKC], vop[S::kRoles ? 1 : S::kKC];
  {
    const bool ok = key < p.Lk;
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(ds_wave ? p.v : p.k) +
                         b * (ds_wave ? p.v_sb : p.k_sb) + hk * (ds_wave ? p.v_sh : p.k_sh) +
                         (int64_t)key * (ds_wave ? p.v_st : p.k_st);
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc) kop[kc] = ok ? load16(kr + 16 * kc + 8 * g) : zero16();
    if constexpr (!S::kRoles) {
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)key * p.v_st;
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) vop[kc] = ok ? load16(vr + 16 * kc + 8 * g) : zero16();
    }
  }
  // Accumulators over head_dim blocks: dV^T then dK^T for a single wave; the
  // P wave's dV^T or the dS wave's dK^T with two roles.
  constexpr int kAcc = S::kRoles ? S::kND : 2 * S::kND;
  f32x16 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  // Steps: the query tiles from the first one with a query at or after k0
  // (causal) to the last, the group's query heads within each tile, so that
  // the key blocks of a kv head running together walk the same tiles at the
  // same time and share them through L2.  The key blocks resident from the
  // start walk the tiles from the last down: they all start on the same one.
  // Causal, a later key block starts when an earlier (heavier) one ends, at
  // a time that grows with its index by as much as its own number of tiles
  // shrinks; walking up from its diagonal, each is on tile `time - const`
  // like the others.
  const int n_qt = (p.Lq + kBwdRows - 1) / kBwdRows;
  const int qt_lo = CAUSAL ? min(k0 / kBwdRows, n_qt) : 0;
  const int n_steps = p.group * (n_qt - qt_lo);
  const bool ascend = CAUSAL && kb >= p.kv_round1;
  const int qt_first = ascend ? qt_lo : n_qt - 1, qt_dir = ascend ? 1 : -1;
  const float c = p.scale_log2;

  // ---- copy plan: wave w moves chunks kCopiesPerWave * w .. +kCopiesPerWave-1
  // of a step (Q tile first, then dO); chunk ci covers tile rows
  // kRowsPerCopy * (ci % kCopiesPerTile) ..; lane -> row lane / kPitch.
  // Staged, the lane reads chunk lane % kPitch of its row in memory order and
  // writes it to the chunk's swizzled slot; copied directly, the lane fills
  // slot lane % kPitch and fetches the chunk that the swizzle puts there.
  // Wave 0 also moves the statistics.
  const int ci0 = S::kCopiesPerWave * wave;
  const bool cp_q = ci0 < S::kCopiesPerTile;
  const int cp_row0 = S::kRowsPerCopy * (ci0 % S::kCopiesPerTile);
  const int cp_c = lane % S::kPitch;  // staged: chunk of the row in memory; direct: LDS slot
  int cp_row[S::kCopiesPerWave];      // tile row of the lane
  int cp_chunk[S::kCopiesPerWave];    // chunk of the row the lane reads
  uint32_t cp_dst[S::kCopiesPerWave];  // staged: LDS byte offset of the lane's slot within the stage
#pragma unroll
  for (int j = 0; j < S::kCopiesPerWave; ++j) {
    const int r = cp_row0 + S::kRowsPerCopy * j + lane / S::kPitch;
    cp_row[j] = r;
    cp_chunk[j] = S::kStaged ? cp_c : cp_c ^ bwd_swz<S::kPitch>(r);
    cp_dst[j] = (cp_q ? 0 : S::kTileBytes) + r * S::kRowBytes + 16 * (cp_c ^ bwd_swz<S::kPitch>(r));
  }
  const int64_t cp_st = cp_q ? p.q_st : p.do_st;
  const int64_t cp_sh = cp_q ? p.q_sh : p.do_sh;
  const uint32_t cp_row_bytes = (uint32_t)(2 * cp_st);  // direct copies: < 2^27, token strides are validated
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  // Step st is query head hg = st % group of query tile qt_first + qt_dir * (st / group).
  // The copies and the compute visit the steps in order, so each keeps a
  // cursor (head within the group, query tile, source rows) advanced one step
  // at a time instead of dividing by the runtime group size and multiplying
  // out the strides.
  int iss_hg = 0, iss_qt = qt_first;  // next step to copy
  const uint16_t* iss_src = (cp_q ? reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb
                                  : reinterpret_cast<const uint16_t*>(p.dout) + b * p.do_sb) +
                            (int64_t)(hk * p.group) * cp_sh + (int64_t)(iss_qt * kBwdRows) * cp_st;
  const int64_t iss_wrap = (int64_t)p.group * cp_sh - qt_dir * kBwdRows * cp_st;
  const float* iss_stat = p.stats + 2 * (((int64_t)b * p.Hq + hk * p.group) * p.Lq + iss_qt * kBwdRows);
  const int64_t stat_sh = 2 * (int64_t)p.Lq, stat_wrap = 2 * ((int64_t)p.group * p.Lq - qt_dir * kBwdRows);
  auto advance = [&]() __attribute__((always_inline)) {
    iss_src += cp_sh;
    iss_stat += stat_sh;
    if (++iss_hg == p.group) {
      iss_hg = 0;
      iss_qt += qt_dir;
      iss_src -= iss_wrap;
      iss_stat -= stat_wrap;
    }
  };

  // Direct copies of the next step into buffer iss_buf.
  int iss_buf = 0;
  auto issue_step = [&]() __attribute__((always_inline)) {
    const uint32_t stage = lds0 + iss_buf * S::kStageBytes;
    iss_buf = iss_buf == S::kStages - 1 ? 0 : iss_buf + 1;
    const int r0 = iss_qt * kBwdRows;
    const uint16_t* src = iss_src;
    const float* st_src = iss_stat;
    advance();
    const uint32_t dst = stage + (cp_q ? 0 : S::kTileBytes);
#pragma unroll
    for (int j = 0; j < S::kCopiesPerWave; ++j) {
      const int row = min(r0 + cp_row[j], p.Lq - 1) - r0;  // rows past Lq repeat the last one
      if (S::kChunks == S::kPitch || cp_chunk[j] < S::kChunks)  // slots of padding chunks (head_dim 80) stay idle
        lds_copy16(src, (uint32_t)row * cp_row_bytes + 16u * (uint32_t)cp_chunk[j],
                   dst + (cp_row0 + S::kRowsPerCopy * j) * S::kRowBytes);
    }
    if (wave == 0) {
      const int row = min(r0 + (lane >> 1), p.Lq - 1) - r0;
      lds_copy4(st_src, (uint32_t)(8 * row + 4 * (lane & 1)), stage + 2 * S::kTileBytes);
    }
  };
  // Direct copies: waits until at most `pending` later steps' copies of this
  // wave are in flight.
  auto wait_steps = [&](int pending) __attribute__((always_inline)) {
    if (wave == 0) {
      constexpr int n = S::kCopiesPerWave + 1;
      if (pending >= 2) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * n));
      else if (pending == 1) __builtin_amdgcn_s_waitcnt(0x0f70 | n);
      else __builtin_amdgcn_s_waitcnt(0x0f70);
    } else {
      constexpr int n = S::kCopiesPerWave;
      if (pending >= 2) __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * n));
      else if (pending == 1) __builtin_amdgcn_s_waitcnt(0x0f70 | n);
      else __builtin_amdgcn_s_waitcnt(0x0f70);
    }
  };

  // Staged copies.  Every wave issues the same loads on every call, the
  // statistics included (only wave 0 writes them), and calls past the last
  // step repeat it, so that the compiler's wait before each write counts
  // exactly the loads of the other register set.
  struct Staged {
    u32x4 v[S::kStaged ? S::kCopiesPerWave : 1];
    float st;
  };
  int iss_n = 0;  // steps loaded so far
  auto load_step = [&](Staged& x) __attribute__((always_inline)) {
    const int r0 = iss_qt * kBwdRows;
    const uint16_t* src = iss_src;
    const float* st_src = iss_stat;
    if (++iss_n < n_steps) advance();
#pragma unroll
    for (int j = 0; j < S::kCopiesPerWave; ++j) {
      const int row = min(r0 + cp_row[j], p.Lq - 1) - r0;  // rows past Lq repeat the last one
      // padding chunks (head_dim 80) load nothing
      x.v[j] = S::kChunks == S::kPitch || cp_c < S::kChunks ? load16(src + (int64_t)row * cp_st + 8 * cp_c) : zero16();
    }
    const int row = min(r0 + (lane >> 1), p.Lq - 1) - r0;
    x.st = st_src[2 * row + (lane & 1)];
  };
  auto write_step = [&](const Staged& x, int buf) __attribute__((always_inline)) {
    lds_char* stage = lds + buf * S::kStageBytes;
#pragma unroll
    for (int j = 0; j < S::kCopiesPerWave; ++j) *reinterpret_cast<lds_u32x4*>(stage + cp_dst[j]) = x.v[j];
    if (wave == 0)
      *reinterpret_cast<__attribute__((address_space(3))) float*>(
          stage + 2 * S::kTileBytes + 4 * (32 * (lane & 1) + (lane >> 1))) = x.st;  // all LSE, then all D
  };

  // ---- LDS operand offsets within a tile ----
  // Row reads (A operands of S and dP): row ln, chunk 2 kc + g.
  const int rd_off = ln * S::kRowBytes + 16 * (g ^ bwd_swz<S::kPitch>(ln));
  // Transposing reads (A operands X^T of dV^T, dK^T): lane (G, i, q) points at
  // row 16 cs + 4 g + i (+8), head-dim 32 db + 16 (G & 1) + 4 q; the chunk is
  // 4 db + 2 (G & 1) + q / 2, so block db is block 0's offset with 64 db
  // XOR-ed in.
  int tr_off[2];
  {
    const int G = lane >> 4, i = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 4 * g + i + 8 * hh;
      tr_off[hh] = r * S::kRowBytes + 16 * ((2 * (G & 1) + (q >> 1)) ^ bwd_swz<S::kPitch>(r)) + 8 * (q & 1);
    }
  }
  auto tr_read = [&](const lds_char* tile, int db, int cs) {
    typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
    const lds_char* t = tile + 16 * cs * S::kRowBytes;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (tr_off[0] ^ (64 * db))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + (tr_off[1] ^ (64 * db))));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const uint32_t a0 = l2[0], a1 = l2[1], a2 = h2[0], a3 = h2[1];
    return u32x4{a0, a1, a2, a3};
  };
  // A product of 32 rows (the stage's Q or dO tile) with this lane's key
  // operands: S = Q K^T, dP = dO V^T; rows = the tile's queries, columns = keys.
  auto row_product = [&](const lds_char* tile, const u32x4* bop) __attribute__((always_inline)) {
    f32x16 acc_s;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_s[r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc) {
      const u32x4 a = *reinterpret_cast<const lds_u32x4*>(tile + (rd_off ^ (32 * kc)));
      acc_s = mfma32(a, bop[kc], acc_s);
    }
    return acc_s;
  };
  // Statistics of the rows this lane's accumulator registers hold: row
  // 8 (r / 4) + 4 g + r % 4 of the tile; element 0 is LSE log2 e, 1 is D.
  // (Staged tiles, the two-role kernel: the tile's 32 LSE values, then its
  // 32 D values, so that a role reads its 16 with four 16-byte reads.)
  auto row_stats = [&](const lds_char* stage, int r, int e) __attribute__((always_inline)) {
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>(
        stage + 2 * S::kTileBytes + 4 * (32 * e + 8 * (r >> 2) + 4 * g + (r & 3)));
  };
  // P = exp2(c S - LSE log2 e), zero for pairs that do not take part (rows
  // past Lq, keys past Lk, causal keys after the query).
  auto probs = [&](const f32x16& s, const lds_char* stage, int r0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 pe;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qrow = r0 + 8 * (r >> 2) + 4 * g + (r & 3);
      const bool vis = !MASK || (qrow < p.Lq && key < p.Lk && (!CAUSAL || key <= qrow));
      const float pv = fast_exp2(__builtin_fmaf(s[r], c, -row_stats(stage, r, 0)));
      pe[r] = vis ? pv : 0.f;
    }
    return pe;
  };
  // Packs 16 accumulator values as the B operands of the two 16-query slices.
  auto pack_b = [&](const f32x16& x, u32x4* out) __attribute__((always_inline)) {
#pragma unroll
    for (int cs = 0; cs < 2; ++cs)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[cs][j] = pack_bf16x2(x[8 * cs + 2 * j], x[8 * cs + 2 * j + 1]);
  };
  // dV^T (dK^T) += X^T B over head-dim blocks first .. first + n - 1, X the
  // stage's dO (Q) tile read transposed.
  auto grad_product = [&](const lds_char* tile, const u32x4* bsl, int acc0, int first, int n) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < n; ++i)
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) acc[acc0 + i] = mfma32(tr_read(tile, first + i, cs), bsl[cs], acc[acc0 + i]);
  };
  // Fully visible tiles (all rows below Lq, all keys below Lk and, causal,
  // every query at or after the wave's last key) skip the per-pair test,
  // which is most of them.
  auto all_visible = [&](int r0) {
    return r0 + kBwdRows <= p.Lq && wave_k0 + 32 <= p.Lk && (!CAUSAL || r0 >= wave_k0 + 31);
  };

  Staged stg_a, stg_b;
  if constexpr (S::kStaged) {
    // Steps 0 and 1 go straight to LDS; 2 and 3 wait in registers.
    if (n_steps > 0) {
      load_step(stg_a);
      write_step(stg_a, 0);
      load_step(stg_a);
      write_step(stg_a, 1);
      load_step(stg_a);
      // Keep step 3's loads after step 2's: the waits in the loop count on
      // that order (the scheduler may otherwise swap the two groups).
      __builtin_amdgcn_sched_barrier(0);
      load_step(stg_b);
    }
  } else {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): K and V have landed before the copies start
#pragma unroll
    for (int st = 0; st < S::kAhead; ++st)
      if (st < n_steps) issue_step();
  }

  // P exchange (two roles): slot (step & 1) of this key group, lane-major
  // 16-byte chunks, chunk j of lane l at 16 (64 j + l).
  lds_char* const xchg = lds + S::kStages * S::kStageBytes + kgrp * 2 * S::kPBytes;
  int prev_buf = -1;  // dS wave: buffer of the previous step (-1: nothing to finish)
  // dS wave, for the previous step (its tiles still in their buffer, its P
  // left by the P wave before this barrier): dP = dO V^T, dS = P (dP - D),
  // dK^T += Q^T dS.
  auto finish_prev = [&](int slot) __attribute__((always_inline)) {
    const lds_char* stage = lds + prev_buf * S::kStageBytes;
    const f32x16 dp = row_product(stage + S::kTileBytes, kop);
    f32x16 ds;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 pv = *reinterpret_cast<const lds_f32x4*>(xchg + slot * S::kPBytes + 16 * (64 * j + lane));
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[4 * j + e] = pv[e] * (dp[4 * j + e] - row_stats(stage, 4 * j + e, 1));
    }
    u32x4 dsb[2];
    pack_b(ds, dsb);
    grad_product(stage, dsb, 0, 0, S::kND);
  };

  // A single wave's step: S = Q K^T and dP = dO V^T (their accumulation
  // chains interleaved), P and dS packed as the B operands of the two
  // 16-query slices, then dV^T += dO^T P and dK^T += Q^T dS block by block.
  auto single_step = [&](int buf, int r0) __attribute__((always_inline)) {
    const lds_char* stage = lds + buf * S::kStageBytes;
    const lds_char* qt_l = stage;
    const lds_char* dt_l = stage + S::kTileBytes;
    const float* st_l = (const float*)(stage + 2 * S::kTileBytes);
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc) {
      const u32x4 qa = *reinterpret_cast<const lds_u32x4*>(qt_l + (rd_off ^ (32 * kc)));
      const u32x4 da = *reinterpret_cast<const lds_u32x4*>(dt_l + (rd_off ^ (32 * kc)));
      s = mfma32(qa, kop[kc], s);
      dp = mfma32(da, vop[kc], dp);
    }
    u32x4 pb[2], dsb[2];
    auto scores = [&](auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        float pe[8], de[8];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          // rows rb .. rb + 3: (LSE log2 e, D) pairs of 4 consecutive rows
          const int rb = 8 * (2 * cs + jj) + 4 * g;
          const f32x4 s01 = *reinterpret_cast<const lds_f32x4*>((const lds_char*)st_l + 8 * rb);
          const f32x4 s23 = *reinterpret_cast<const lds_f32x4*>((const lds_char*)st_l + 8 * rb + 16);
          const float l2v[4] = {s01[0], s01[2], s23[0], s23[2]};
          const float dlv[4] = {s01[1], s01[3], s23[1], s23[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * cs + 4 * jj + e;
            const int qrow = r0 + rb + e;
            const bool vis = !MASK || (qrow < p.Lq && key < p.Lk && (!CAUSAL || key <= qrow));
            const float pv = vis ? fast_exp2(__builtin_fmaf(s[r], c, -l2v[e])) : 0.f;
            pe[4 * jj + e] = pv;
            de[4 * jj + e] = pv * (dp[r] - dlv[e]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[cs][j] = pack_bf16x2(pe[2 * j], pe[2 * j + 1]);
          dsb[cs][j] = pack_bf16x2(de[2 * j], de[2 * j + 1]);
        }
      }
    };
    if (all_visible(r0))
      scores(std::false_type{});
    else
      scores(std::true_type{});
#pragma unroll
    for (int i = 0; i < S::kND; ++i)
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        acc[i] = mfma32(tr_read(dt_l, i, cs), pb[cs], acc[i]);
        acc[S::kND + i] = mfma32(tr_read(qt_l, i, cs), dsb[cs], acc[S::kND + i]);
      }
  };

  int cmp_hg = 0, cmp_qt = qt_first, cmp_buf = 0;  // this step's cursor
  // One step.  Staged, `stg` holds step + 2 (even steps stg_a, odd steps
  // stg_b, so that no register copy waits for loads still in flight);
  // copying directly, it is unused.
  auto run_step = [&](int step, Staged& stg) __attribute__((always_inline)) {
    const int buf = cmp_buf;
    cmp_buf = cmp_buf == S::kStages - 1 ? 0 : cmp_buf + 1;
    if constexpr (S::kStaged) {
      lds_barrier();  // step's tiles in LDS; every wave is done with the buffer refilled next
      // Step + 2 from registers into its buffer (free since step - 2), then
      // the loads of step + 4 into the same registers.  Past the last step
      // both move a repeat of it into a buffer no later step reads.
      write_step(stg, buf + 2 < S::kStages ? buf + 2 : buf + 2 - S::kStages);
      load_step(stg);
    } else {
      wait_steps(min(S::kAhead - 1, n_steps - 1 - step));
      lds_barrier();  // step's tiles in LDS; every wave is done with the buffer refilled next
      if (step + S::kAhead < n_steps) issue_step();
    }
    if (ds_wave && prev_buf >= 0) finish_prev((step - 1) & 1);
    prev_buf = -1;
    const int qt = cmp_qt;
    if (++cmp_hg == p.group) {
      cmp_hg = 0;
      cmp_qt += qt_dir;
    }
    const int r0 = qt * kBwdRows;
    // A wave whose keys all come after the tile's last query has nothing here.
    if (!CAUSAL || r0 + kBwdRows - 1 >= wave_k0) {
      if (!S::kRoles) {
        single_step(buf, r0);
      } else if (ds_wave) {
        prev_buf = buf;
      } else {
        // P wave.
        const lds_char* stage = lds + buf * S::kStageBytes;
        const lds_char* qt_l = stage;
        const lds_char* dt_l = stage + S::kTileBytes;
        const f32x16 s = row_product(qt_l, kop);
        const f32x16 pe =
            all_visible(r0) ? probs(s, stage, r0, std::false_type{}) : probs(s, stage, r0, std::true_type{});
        u32x4 pb[2];
        pack_b(pe, pb);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<lds_f32x4*>(xchg + (step & 1) * S::kPBytes + 16 * (64 * j + lane)) =
              f32x4{pe[4 * j], pe[4 * j + 1], pe[4 * j + 2], pe[4 * j + 3]};
        grad_product(dt_l, pb, 0, 0, S::kND);
      }
    }
  };
  // Whole pairs in the loop (so that the compiler sees both register sets
  // loaded on every way round it), an odd last step after.
  int step = 0;
  for (; step + 1 < n_steps; step += 2) {
    run_step(step, stg_a);
    run_step(step + 1, stg_b);
  }
  if (step < n_steps) run_step(step, stg_a);
  if constexpr (S::kRoles) {
    lds_barrier();  // the last step's P is in LDS
    if (ds_wave && prev_buf >= 0) finish_prev((n_steps - 1) & 1);
  }

  // dK = scale dK_acc, dV = dV_acc: lane = key, registers = head-dim rows.
  if (key < p.Lk) {
    uint16_t* dkr = reinterpret_cast<uint16_t*>(p.dk) + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_st;
    uint16_t* dvr = reinterpret_cast<uint16_t*>(p.dv) + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_st;
    auto store = [&](uint16_t* row, int a0, float mul) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < S::kND; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * i + 8 * j + 4 * g;
          if (d >= D) continue;  // padding rows of the last block (head_dim 80)
          u32x2 w;
          w[0] = pack_bf16x2(acc[a0 + i][4 * j + 0] * mul, acc[a0 + i][4 * j + 1] * mul);
          w[1] = pack_bf16x2(acc[a0 + i][4 * j + 2] * mul, acc[a0 + i][4 * j + 3] * mul);
          *reinterpret_cast<u32x2*>(row + d) = w;
        }
    };
    if (do_dv) store(dvr, 0, 1.f);
    if (do_dk) store(dkr, S::kRoles ? 0 : S::kND, p.scale);
  }
}

// ---------------------------------------------------------------- dQ
// dQ workgroup: 32 queries per wave of one (batch, query head), 8 waves (one
// workgroup per CU) from head_dim 80 on and 4 at 64 (two per CU): the larger
// workgroup shares each copied K/V tile among more queries (2-3 % faster at
// head_dim 80 and 128, 1.4 % slower at 64).  32-key tiles of K and V staged
// through registers into LDS (the dK/dV kernel's swizzle: K is read by rows
// and transposed), three steps ahead of their use.
template <int D>
struct BwdQShape {
  static constexpr int kWaves = D >= 80 ? 8 : 4;
  static constexpr int kRows = 32 * kWaves;           // queries per workgroup
  static constexpr int kPerCU = D >= 80 ? 1 : 2;      // workgroups per CU the registers allow
  static constexpr int kKC = D / 16;
  static constexpr int kND = (D + 31) / 32;           // the last block padded at d = 80
  static constexpr int kChunks = D / 8;
  static constexpr int kPitch = D <= 64 ? 8 : 16;     // 16-byte chunks of a row in LDS
  static constexpr int kRowBytes = 16 * kPitch;
  static constexpr int kTileBytes = kBwdRows * kRowBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;  // K, V
  static constexpr int kStages = 4;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kCopiesPerTile = kBwdRows / kRowsPerCopy;
  static constexpr int kCopiesPerWave = 2 * kCopiesPerTile / kWaves;
  static_assert(kCopiesPerWave * kWaves == 2 * kCopiesPerTile, "copies split evenly over the waves");
  static_assert(kCopiesPerTile % kCopiesPerWave == 0, "a wave copies from one tile only");
  static_assert(kChunks <= kPitch, "rows fit their pitch");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * BwdQShape<D>::kWaves, BwdQShape<D>::kPerCU) void attn_bwd_dq_kernel(BwdParams p) {
  using S = BwdQShape<D>;
  typedef __attribute__((address_space(3))) char lds_char;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_raw[];
  lds_char* const lds = (lds_char*)lds_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ln = lane & 31;
  // Work order as in the forward (whole (batch, kv head) units per XCD, so
  // the workgroups that re-read one kv head's K and V share an L2; causal:
  // heaviest query blocks first across the XCD's units).
  const int n_qb = (p.Lq + S::kRows - 1) / S::kRows;
  int h, b, qb;
  {
    const WorkItem it = dense_work_item(blockIdx.x, gridDim.x, n_qb, p.group, p.Hkv, CAUSAL);
    h = it.h;
    b = it.b;
    qb = it.qt;
  }
  const int hk = h / p.group;
  const int q0 = qb * S::kRows;
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
  const int64_t si = ((int64_t)b * p.Hq + h) * p.Lq + min(qrow, p.Lq - 1);
  const float lse2 = qok ? p.stats[2 * si] : 0.f;
  const float dl = qok ? p.stats[2 * si + 1] : 0.f;
  const float c = p.scale_log2;

  f32x16 dq_acc[S::kND];
#pragma unroll
  for (int db = 0; db < S::kND; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.f;

  int n_kt = (p.Lk + kBwdRows - 1) / kBwdRows;
  if (CAUSAL) n_kt = min(n_kt, (q0 + S::kRows - 1) / kBwdRows + 1);

  // ---- copy plan: the first half of the waves move the K tile, the second
  // half the V tile; lane ->
  // row lane / kPitch, 16-byte chunk lane % kPitch of the row, read in memory
  // order and written to its swizzled LDS slot.  A tile is loaded into
  // registers one step before it is written to LDS, three steps ahead of its
  // use; loads past the last tile repeat it. ----
  const int ci0 = S::kCopiesPerWave * wave;
  const bool cp_k = ci0 < S::kCopiesPerTile;
  const int cp_row0 = S::kRowsPerCopy * (ci0 % S::kCopiesPerTile);
  const int cp_c = lane % S::kPitch;
  int cp_row[S::kCopiesPerWave];
  uint32_t cp_dst[S::kCopiesPerWave];
#pragma unroll
  for (int j = 0; j < S::kCopiesPerWave; ++j) {
    const int r = cp_row0 + S::kRowsPerCopy * j + lane / S::kPitch;
    cp_row[j] = r;
    cp_dst[j] = (cp_k ? 0 : S::kTileBytes) + r * S::kRowBytes + 16 * (cp_c ^ bwd_swz<S::kPitch>(r));
  }
  const int64_t cp_st = cp_k ? p.k_st : p.v_st;
  const uint16_t* cp_base = cp_k ? reinterpret_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh
                                 : reinterpret_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh;
  u32x4 stg[S::kCopiesPerWave];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const int r0 = min(t, n_kt - 1) * kBwdRows;
    const uint16_t* src = cp_base + (int64_t)r0 * cp_st + 8 * cp_c;
#pragma unroll
    for (int j = 0; j < S::kCopiesPerWave; ++j) {
      const int row = min(r0 + cp_row[j], p.Lk - 1) - r0;  // keys past Lk repeat the last one
      stg[j] = S::kChunks == S::kPitch || cp_c < S::kChunks ? load16(src + (int64_t)row * cp_st) : zero16();
    }
  };
  auto write_tile = [&](int buf) __attribute__((always_inline)) {
    lds_char* stage = lds + buf * S::kStageBytes;
#pragma unroll
    for (int j = 0; j < S::kCopiesPerWave; ++j)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(stage + cp_dst[j]) = stg[j];
  };

  const int rd_off = ln * S::kRowBytes + 16 * (g ^ bwd_swz<S::kPitch>(ln));
  int tr_off[2];
  {
    const int G = lane >> 4, i = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 4 * g + i + 8 * hh;
      tr_off[hh] = r * S::kRowBytes + 16 * ((2 * (G & 1) + (q >> 1)) ^ bwd_swz<S::kPitch>(r)) + 8 * (q & 1);
    }
  }

  // Tiles 0-2 go straight to LDS; tile 3 waits in registers.
  if (n_kt > 0) {
#pragma unroll
    for (int t = 0; t < S::kStages - 1; ++t) {
      load_tile(t);
      write_tile(t);
    }
    load_tile(S::kStages - 1);
  }

  for (int t = 0; t < n_kt; ++t) {
    lds_barrier();  // tile t in LDS; every wave is done with tile t - 1's buffer
    // Tile t + 3 from registers into tile t - 1's buffer, then the loads of
    // t + 4 (past the last tile, repeats of it into buffers no later step reads).
    write_tile((t + S::kStages - 1) % S::kStages);
    load_tile(t + S::kStages);
    const int kv0 = t * kBwdRows;
    if (!CAUSAL || kv0 <= wave_q0 + 31) {
      const lds_char* kt_l = lds + (t % S::kStages) * S::kStageBytes;
      const lds_char* vt_l = kt_l + S::kTileBytes;
      // S^T = K Q^T and dP^T = V dO^T: rows = the tile's 32 keys, columns = queries.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) {
        const u32x4 ka = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(kt_l + (rd_off ^ (32 * kc)));
        const u32x4 va = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(vt_l + (rd_off ^ (32 * kc)));
        s = mfma32(ka, qop[kc], s);
        dp = mfma32(va, dop[kc], dp);
      }
      // dS^T = P^T (dP^T - D), P^T recomputed from the LSE; packed as the B
      // operands of the two 16-key slices.  Tiles whose every key comes
      // before the wave's first query (or every key, not causal) and lies
      // below Lk skip the per-pair test.
      u32x4 dsb[2];
      const bool all_vis = kv0 + kBwdRows <= p.Lk && (!CAUSAL || kv0 + kBwdRows - 1 <= wave_q0);
      auto dscores = [&](auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          float de[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * cs + e;
            const int kk = kv0 + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool vis = !MASK || (kk < p.Lk && (!CAUSAL || kk <= qrow));
            const float pv = vis ? fast_exp2(__builtin_fmaf(s[r], c, -lse2)) : 0.f;
            de[e] = pv * (dp[r] - dl);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) dsb[cs][j] = pack_bf16x2(de[2 * j], de[2 * j + 1]);
        }
      };
      if (all_vis)
        dscores(std::false_type{});
      else
        dscores(std::true_type{});
      // dQ^T += K^T dS^T (rows = head_dim, columns = queries).
#pragma unroll
      for (int db = 0; db < S::kND; ++db)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
          typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
          const lds_char* tt = kt_l + 16 * cs * S::kRowBytes;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(tt + (tr_off[0] ^ (64 * db))));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(tt + (tr_off[1] ^ (64 * db))));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const uint32_t a0 = l2[0], a1 = l2[1], a2 = h2[0], a3 = h2[1];
          dq_acc[db] = mfma32(u32x4{a0, a1, a2, a3}, dsb[cs], dq_acc[db]);
        }
    }
  }

  if (qok) {
    uint16_t* dqr = reinterpret_cast<uint16_t*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)qrow * p.dq_st;
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        if (d >= D) continue;  // padding rows of the last block (head_dim 80)
        u32x2 w;
        w[0] = pack_bf16x2(dq_acc[db][4 * j + 0] * p.scale, dq_acc[db][4 * j + 1] * p.scale);
        w[1] = pack_bf16x2(dq_acc[db][4 * j + 2] * p.scale, dq_acc[db][4 * j + 3] * p.scale);
        *reinterpret_cast<u32x2*>(dqr + d) = w;
      }
  }
}

}  // namespace attn_dev
