// Prefill attention forward, bf16 inputs, for gfx950.
//
// Method: the tiled forward with online softmax of "Flash Attention原理：分块
// 计算与重计算" (cnblogs), sections 三-五.  Q is split into row tiles, K and V
// into key tiles; for every key tile the kernel forms the score tile, updates
// each row's running maximum m and normaliser l, rescales the partial output by
// exp(m_old - m_new) (section 四) and adds P V.  Only O and the row statistics
// (returned as LSE = m + ln l, section 五) are written.
//
// Work decomposition: one workgroup of 4 waves per (batch, query head, tile
// of 128 query rows); wave w owns 32 rows.  Key/value tiles of 64 keys are
// staged in LDS, double buffered, and shared by the 4 waves.
//
// Orientation: every product is taken transposed, S^T = K Q^T and
// O^T = V^T P^T, so that in both the score accumulator and the output
// accumulator a lane holds one query's values (lane % 32 = query).  Then
//   * the row max and row sum are in-lane reductions plus one exchange with
//     lane ^ 32 (the other half of the keys);
//   * the probabilities leave the score accumulator already in the B-operand
//     layout of the P V product (no LDS round trip);
//   * the rescale of the output by exp(m_old - m_new) is a per-lane scalar.
// The key order inside each 16-key slice of the P V contraction is permuted to
// match the score accumulator's row order; V^T is written to LDS in that
// permuted order so each lane's 8 keys are one 16-byte read.
//
// Causal (top-left, Lq == Lk): key tiles entirely above a wave's last row are
// skipped; tiles that straddle the diagonal or the end of the keys are masked
// to -inf before the max.  Key tile 0 is processed first and always holds a
// visible key for every row, so the running max is finite from the first tile
// on and exp(-inf - m) = 0 never meets exp(-inf - (-inf)).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace attn_dev {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t o_sb, o_sh, o_st;
  int Hq;
  int Hkv;
  int group;  // Hq / Hkv
  int Lq;
  int Lk;
  int n_qtiles;
  float scale_log2;      // scale * log2(e)
  float scale_log2_abs;  // |scale * log2(e)|
  int neg_q;             // scale < 0: Q's sign bits are flipped on load (exact)
};

// Work-item order shared by the prefill kernels.  The hardware hands
// consecutive workgroup ids to the 8 XCDs in turn; this maps them so that each
// XCD receives one contiguous range of work items, and orders work items kv
// head by kv head, so the workgroups that re-read one head's K and V run on
// the same XCD and share its L2.  Within a kv head: query tiles (heaviest
// first when causal), then the query heads of the group.
struct WorkItem {
  int b, h, hk, qt;
};

__device__ __forceinline__ WorkItem prefill_work_item(const FwdParams& p, bool causal) {
  const int L = blockIdx.x;
  const int N = gridDim.x;
  const int full = N & ~7;
  int w = L;
  if (L < full) w = (L & 7) * (full >> 3) + (L >> 3);
  WorkItem it;
  const int hg = w % p.group;
  int r = w / p.group;
  const int qi = r % p.n_qtiles;
  r /= p.n_qtiles;
  it.hk = r % p.Hkv;
  it.b = r / p.Hkv;
  it.h = it.hk * p.group + hg;
  it.qt = causal ? p.n_qtiles - 1 - qi : qi;
  return it;
}

// 32-query column blocks per wave: two at head_dim 64 (each K or V^T read
// from LDS then feeds two matrix instructions), one at larger head_dims where
// the output accumulator alone would not leave room for two waves per SIMD.
__host__ __device__ constexpr int bf16_fwd_blocks_per_wave(int d) { return d <= 64 ? 2 : 1; }
__host__ __device__ constexpr int bf16_fwd_rows_per_workgroup(int d) {
  return 4 * 32 * bf16_fwd_blocks_per_wave(d);
}

template <int D>
struct Bf16FwdShape {
  static constexpr int kWaves = 4;
  static constexpr int kNB = bf16_fwd_blocks_per_wave(D);
  static constexpr int kRowsPerWave = 32 * kNB;
  static constexpr int kBR = kRowsPerWave * kWaves;  // query rows per workgroup
  static constexpr int kBC = 64;                     // keys per tile
  static constexpr int kKC = D / 16;                 // k-slices of the Q K^T product
  static constexpr int kDP = (D + 31) / 32 * 32;     // rows of O^T padded to 32
  static constexpr int kND = kDP / 32;               // 32-row blocks of O^T
  static constexpr int kChunks = D / 8;              // 16-byte chunks per row
  static constexpr int kKPitch = D + 8;              // K row pitch in LDS (elements)
  static constexpr int kVPitch = kBC + 8;            // V^T row pitch in LDS (elements)
  static constexpr int kKElems = kBC * kKPitch;
  static constexpr int kVElems = kDP * kVPitch;
  static constexpr int kBufBytes = (kKElems + kVElems) * 2;
  static constexpr int kLdsBytes = 2 * kBufBytes;
  static constexpr int kKItems = kBC * kChunks;         // 16-byte K loads per tile
  static constexpr int kVItems = (kBC / 2) * kChunks;   // (key pair, chunk) V loads
  static constexpr int kKIter = (kKItems + 255) / 256;
  static constexpr int kVIter = (kVItems + 255) / 256;
  static_assert(D % 16 == 0, "head_dim must be a multiple of 16");
  static_assert(kBufBytes < 65536, "in-buffer LDS offsets must fit the instruction offset field");
};

// Position of key kk (0..15) of a 16-key slice inside V^T's LDS row: the
// score accumulator gives lane half g the keys {4g..4g+3, 8+4g..8+4g+3} of a
// slice, stored contiguously at 8g..8g+7.
__device__ __forceinline__ int vt_pos16(int kk) {
  return ((kk >> 2) & 1) * 8 + (kk >> 3) * 4 + (kk & 3);
}

// Row maxima are tracked in the log2 domain of the scaled scores, as a
// reference m that only moves when it must.  Each tile's probabilities are
// first formed against the current m; only if some lane's share of the tile
// sum exceeds 2^kRescaleLog2 (or is not a number, as before a row's first
// tile, where m is still -inf) does the wave take the tile max, move m,
// rescale O and l, and form the probabilities again.  Every probability
// therefore stays below 2^kRescaleLog2, well inside fp32 and bf16 range, and
// LSE = m + log2(l) is exact for any m.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kSumGuard = 256.f;
static_assert(kSumGuard == float(1 << int(kRescaleLog2)), "guard is 2^kRescaleLog2");

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdParams p) {
  using S = Bf16FwdShape<D>;
  constexpr int NB = S::kNB;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  char* const lds_b = reinterpret_cast<char*>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane & 31;  // query column within a 32-query block (n index)
  const int g = lane >> 5;   // lane half

  const WorkItem wi = prefill_work_item(p, CAUSAL);
  const int b = wi.b, h = wi.h, hk = wi.hk;
  const int q0 = wi.qt * S::kBR;
  const int row0 = q0 + wave * S::kRowsPerWave;  // first query row of this wave
  int qrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) qrow[nb] = row0 + 32 * nb + lq;

  const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh;
  const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh;

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[qrow][16*kc + 8*g .. +8].
  u32x4 qop[NB][S::kKC];
  {
    const uint32_t flip = p.neg_q ? 0x80008000u : 0u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool ok = qrow[nb] < p.Lq;
      const uint16_t* qr = qg + (int64_t)qrow[nb] * p.q_st + 8 * g;
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) {
        qop[nb][kc] = ok ? load16(qr + 16 * kc) : zero16();
#pragma unroll
        for (int e = 0; e < 4; ++e) qop[nb][kc][e] ^= flip;
      }
    }
  }
  const float c = p.scale_log2_abs;

  // Key tiles this workgroup visits.
  int kv_end = p.Lk;
  if (CAUSAL) kv_end = min(kv_end, q0 + S::kBR);
  const int n_tiles = (kv_end + S::kBC - 1) / S::kBC;
  const int n_full = p.Lk / S::kBC;  // tiles with no key beyond Lk
  const int wave_last_row = row0 + S::kRowsPerWave - 1;

  // Zero the padded rows of V^T (head_dim not a multiple of 32) once; the
  // loader never writes them and their products land in discarded O^T rows.
  if (S::kDP != D) {
    for (int i = tid; i < (S::kDP - D) * S::kVPitch; i += 256) {
      lds[S::kKElems + D * S::kVPitch + i] = 0;
      lds[S::kBufBytes / 2 + S::kKElems + D * S::kVPitch + i] = 0;
    }
  }

  // ---- per-thread loader plan ----
  // K: item -> (key row, 16-byte chunk), chunk fastest (coalesced rows).
  // V: item -> (key pair, chunk), key pair fastest, so that the 4-byte V^T
  //    writes of one instruction hit 32 different LDS banks.
  int64_t koff[S::kKIter];
  int kst[S::kKIter];
  int64_t voff[S::kVIter];
  int vst[S::kVIter];
#pragma unroll
  for (int it = 0; it < S::kKIter; ++it) {
    const int item = tid + 256 * it;
    const int row = item / S::kChunks, ch = item - (item / S::kChunks) * S::kChunks;
    koff[it] = (int64_t)row * p.k_st + 8 * ch;
    kst[it] = (row * S::kKPitch + 8 * ch) * 2;
  }
#pragma unroll
  for (int it = 0; it < S::kVIter; ++it) {
    const int item = tid + 256 * it;
    const int pr = item & 31, ch = item >> 5;
    const int key = 2 * pr;
    voff[it] = (int64_t)key * p.v_st + 8 * ch;
    vst[it] = S::kKElems * 2 + (8 * ch * S::kVPitch + (key & ~15) + vt_pos16(key & 15)) * 2;
  }

  u32x4 kreg[S::kKIter] = {};
  u32x4 vreg[S::kVIter][2] = {};

  // Full tiles load without checks; the tile holding key Lk - 1 reads rows
  // beyond it from row Lk - 1 instead (in bounds and finite), and those keys
  // are masked to -inf, so they carry weight 0.
  auto load_tile = [&](int t) {
    const int kv0 = t * S::kBC;
    if (t < n_full) {
      const uint16_t* kt = kg + (int64_t)kv0 * p.k_st;
      const uint16_t* vt = vg + (int64_t)kv0 * p.v_st;
#pragma unroll
      for (int it = 0; it < S::kKIter; ++it)
        if (S::kKItems % 256 == 0 || tid + 256 * it < S::kKItems) kreg[it] = load16(kt + koff[it]);
#pragma unroll
      for (int it = 0; it < S::kVIter; ++it)
        if (S::kVItems % 256 == 0 || tid + 256 * it < S::kVItems) {
          vreg[it][0] = load16(vt + voff[it]);
          vreg[it][1] = load16(vt + voff[it] + p.v_st);
        }
    } else {
      const int last = p.Lk - 1;
#pragma unroll
      for (int it = 0; it < S::kKIter; ++it) {
        const int item = tid + 256 * it;
        if (S::kKItems % 256 == 0 || item < S::kKItems) {
          const int row = item / S::kChunks, ch = item - (item / S::kChunks) * S::kChunks;
          kreg[it] = load16(kg + (int64_t)min(kv0 + row, last) * p.k_st + 8 * ch);
        }
      }
#pragma unroll
      for (int it = 0; it < S::kVIter; ++it) {
        const int item = tid + 256 * it;
        if (S::kVItems % 256 == 0 || item < S::kVItems) {
          const int pr = item & 31, ch = item >> 5;
          vreg[it][0] = load16(vg + (int64_t)min(kv0 + 2 * pr, last) * p.v_st + 8 * ch);
          vreg[it][1] = load16(vg + (int64_t)min(kv0 + 2 * pr + 1, last) * p.v_st + 8 * ch);
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* base = lds_b + buf * S::kBufBytes;
#pragma unroll
    for (int it = 0; it < S::kKIter; ++it)
      if (S::kKItems % 256 == 0 || tid + 256 * it < S::kKItems)
        *reinterpret_cast<u32x4*>(base + kst[it]) = kreg[it];
#pragma unroll
    for (int it = 0; it < S::kVIter; ++it)
      if (S::kVItems % 256 == 0 || tid + 256 * it < S::kVItems) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          // (key, key + 1) pair of head_dim element 8*ch + t: low or high
          // halves of the two rows' words.
          const uint32_t w = __builtin_amdgcn_perm(vreg[it][1][t >> 1], vreg[it][0][t >> 1],
                                                   (t & 1) ? 0x07060302u : 0x05040100u);
          *reinterpret_cast<uint32_t*>(base + vst[it] + t * S::kVPitch * 2) = w;
        }
      }
  };

  // Per-lane LDS read bases: K rows lq (+32 per key block), V^T rows lq (+32
  // per head_dim block); every other offset is a compile-time constant.
  const int k_rd = (lq * S::kKPitch + 8 * g) * 2;
  const int v_rd = S::kKElems * 2 + (lq * S::kVPitch + 8 * g) * 2;

  f32x16 oacc[NB][S::kND];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < S::kND; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nb][i][r] = 0.f;
  float m_run[NB], l_run[NB];  // reference max (log2 domain), this lane's half of l
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
  }

  // One key tile: S^T, online softmax, O^T += V^T P^T.  MASK selects the
  // variant that masks keys beyond Lk and (causal) keys after the query.
  auto process = [&](auto mask_tag, int buf, int kv0) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* kb = lds_b + buf * S::kBufBytes + k_rd;
    const char* vb = lds_b + buf * S::kBufBytes + v_rd;
    f32x16 s[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][sb][r] = 0.f;
    // Matrix-core phases run at raised wave priority, so that of the two
    // waves sharing a SIMD the one with products to issue goes first and the
    // other's softmax fills the vector ALU meanwhile.
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int kc = 0; kc < S::kKC; ++kc) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kb + (32 * sb * S::kKPitch + 16 * kc) * 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[nb][sb] = mfma32(a, qop[nb][kc], s[nb][sb]);
      }
    __builtin_amdgcn_s_setprio(0);

    if constexpr (MASK) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool vis = key < p.Lk && (!CAUSAL || key <= qrow[nb]);
            s[nb][sb][r] = vis ? s[nb][sb][r] : kNegInf;
          }
    }

    // P = exp2(c s - m) for row block nb, packed as the P^T B operands; returns
    // this lane's share of the row sum.
    u32x4 pop[NB][4];
    auto exp_pack = [&](int nb) {
      const float neg_m = -m_run[nb];
      float rs[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            e[i] = fast_exp2(__builtin_fmaf(s[nb][sb][8 * half + i], c, neg_m));
            rs[i & 3] += e[i];
          }
          u32x4 pk;
          pk[0] = pack_bf16x2(e[0], e[1]);
          pk[1] = pack_bf16x2(e[2], e[3]);
          pk[2] = pack_bf16x2(e[4], e[5]);
          pk[3] = pack_bf16x2(e[6], e[7]);
          pop[nb][2 * sb + half] = pk;
        }
      return (rs[0] + rs[1]) + (rs[2] + rs[3]);
    };
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float lsum = exp_pack(nb);
      if (__builtin_amdgcn_ballot_w64(!(lsum <= kSumGuard)) != 0) {
        float mx = kNegInf;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][sb][r]);
        const float m_new = fmaxf(m_run[nb], max_xor32(mx) * c);  // the scale is positive
        const float alpha = m_new == m_run[nb] ? 1.f : fast_exp2(m_run[nb] - m_new);
        m_run[nb] = m_new;
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < S::kND; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][db][r] *= alpha;
        lsum = exp_pack(nb);
      }
      l_run[nb] += lsum;
    }

    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(vb + (32 * db * S::kVPitch + 16 * cs) * 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][db] = mfma32(a, pop[nb][cs], oacc[nb][db]);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  if (n_tiles > 0) {
    // Q must have landed before the loop: the compiler's in-order view of
    // outstanding loads would otherwise make the first use of Q inside the
    // loop wait for the next tile's prefetch as well.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    load_tile(0);
    store_tile(0);
  }

  // Tiles that need no mask for any wave of the workgroup come first (one
  // code path per loop keeps the accumulators in place); the tail of the key
  // range and the diagonal tiles follow with the masked path.
  int n_plain = min(n_tiles, n_full);
  if (CAUSAL) n_plain = min(n_plain, (q0 + 1) / S::kBC);
  int t = 0;
  for (; t < n_plain; ++t) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    __syncthreads();
    process(std::false_type{}, t & 1, t * S::kBC);
    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
  }
  for (; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    __syncthreads();
    const int kv0 = t * S::kBC;
    if (!CAUSAL || kv0 <= wave_last_row) process(std::true_type{}, t & 1, kv0);
    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
  }

  // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2 ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l_tot = sum_xor32(l_run[nb]);
    if (qrow[nb] < p.Lq) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh +
                       (int64_t)qrow[nb] * p.o_st;
#pragma unroll
      for (int db = 0; db < S::kND; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * db + 8 * j + 4 * g;
          if (d < D) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[nb][db][4 * j + 0] * inv, oacc[nb][db][4 * j + 1] * inv);
            w[1] = pack_bf16x2(oacc[nb][db][4 * j + 2] * inv, oacc[nb][db][4 * j + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d) = w;
          }
        }
      if (g == 0) {
        const float lse = l_tot > 0.f ? (m_run[nb] + log2f(l_tot)) * kLn2 : kNegInf;
        p.lse[((int64_t)b * p.Hq + h) * p.Lq + qrow[nb]] = lse;
      }
    }
  }
}

}  // namespace attn_dev
