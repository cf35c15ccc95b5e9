// Split-KV decode for gfx950: one query token per sequence against a ragged
// bf16 KV cache, then a merge of the partial results.
//
// Decode is the inference case of "Flash Attention原理：分块计算与重计算"
// (cnblogs) FAQ Q12-Q13: each new token's query attends to the keys and values
// already in the cache.  "SDPA backend 与 FlashAttention" section 5 notes that
// its bottleneck differs from prefill: here the cache is streamed from HBM
// once and the arithmetic per byte is tiny, so the kernel is built for
// bandwidth.
//
// Work split (balanced over cache slots): a unit is (kv head, group of up to
// 16 query heads sharing it); every sequence b contributes L_b slots to each
// unit.  The slots are laid end to end, unit class by unit class and, within
// one, sequence by sequence, and the whole range is cut into n_wg equal pieces
// of S slots, one per workgroup of the split kernel (n_wg is one workgroup
// of two waves per compute unit, so all of them are resident together and
// finish together whatever the mix of lengths; the cache reads are
// non-temporal, and fewer concurrent streams read HBM faster: two waves per
// compute unit measured above three or four, and one workgroup per compute
// unit above two).  A piece may cover the end of
// one (sequence, unit) and the start of the next; each such segment yields one
// partial (O_s, LSE_s) per query head.  The lengths live on the device, so
// every workgroup derives S and its segments from them (a prefix sum over the
// sequences in each wave).  Slots at or beyond a sequence's length are never
// loaded.
//
// Within a segment the waves take equal shares and walk them 32 keys at a
// time with the tiled online softmax of the cnblogs page's sections 三-四;
// their partial results are combined in LDS and written to the workspace.
//
// Matrix-core use: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the 16 keys on
// the M side and the query heads of the group on the N side; O^T = V^T P^T on
// the same instruction.  K arrives from HBM already in the A-operand layout
// (16 keys x 16-byte slices).  V^T is built in registers: each lane loads 8
// cache rows of 8 consecutive head_dim values (4 full rows per load
// instruction) and transposes them with byte permutes, so O^T row m of the
// product number t is head_dim index 8m + t.  No LDS is used on the way.
//
// Merge kernel: one wave per (b, query head) combines the pieces with the
// cnblogs section 四 identity on (O_s, LSE_s) pairs:
//   M = max_s LSE_s,  LSE = M + ln sum_s e^(LSE_s - M),
//   O = sum_s e^(LSE_s - LSE) O_s.
#pragma once

#include "device_common.h"

namespace attn_dev {

constexpr int kDecMinPiece = 512;              // fewest cache slots per split workgroup
constexpr int kDecWaves = 2;
constexpr int kDecHeadsPerGroup = 16;
constexpr int kDecGroupsPerCU = 1;             // split workgroups (pieces) per compute unit

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seqlens;
  float* o_part;    // [B, Hq, n_pieces, D]
  float* lse_part;  // [B, Hq, n_pieces]
  void* o;          // merge output [B, Hq, D] (strided)
  float* lse;       // [B, Hq]
  int64_t q_sb, q_sh;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t o_sb, o_sh;
  int B, Hq, Hkv, group, Lmax, n_hgroups;
  int n_wg;      // split workgroups (pieces of the slot range)
  int n_pieces;  // workspace rows per (sequence, query head): most pieces one unit can span
  float scale_log2;
};

// Same threshold as the prefill kernels: the output is rescaled only when a
// query's running max grows by more than 2^8.
constexpr float kDecRescaleLog2 = 8.0f;

// Length of sequence b, clamped to [0, Lmax].
__device__ __forceinline__ int dec_len(const DecodeParams& p, int b) {
  const int L = p.seqlens[b];
  return L < 0 ? 0 : (L > p.Lmax ? p.Lmax : L);
}

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan_i32(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Total of the clamped lengths (every lane of the calling wave gets it).
__device__ __forceinline__ int dec_total(const DecodeParams& p, int lane) {
  int s = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) s += wave_sum_i32(b0 + lane < p.B ? dec_len(p, b0 + lane) : 0);
  return __builtin_amdgcn_readfirstlane(s);
}

// Slots per piece: the slot range split into n_wg parts, rounded up to whole
// 32-key steps, never below kDecMinPiece (which bounds the pieces one unit
// can span by its length / kDecMinPiece + 2).
__device__ __forceinline__ int64_t dec_piece(int64_t T, int n_wg) {
  const int64_t s = ((T + n_wg - 1) / n_wg + 31) / 32 * 32;
  return s > kDecMinPiece ? s : kDecMinPiece;
}

// The sequence holding position y (0 <= y < total) of the lengths laid end to
// end: its index, its first position and its length (never 0).  Every lane
// of the calling wave gets the same answer.
__device__ __forceinline__ void dec_find(const DecodeParams& p, int lane, int y, int& b, int& pre, int& L) {
  int base = 0;
  b = 0;
  pre = 0;
  L = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int len = b0 + lane < p.B ? dec_len(p, b0 + lane) : 0;
    const int incl = wave_scan_i32(len, lane);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > y);
    if (hit != 0) {
      const int i = __builtin_ctzll(hit);
      b = b0 + i;
      L = __builtin_amdgcn_readlane(len, i);
      pre = base + __builtin_amdgcn_readlane(incl, i) - L;
      return;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
}


template <int D>
__global__ __launch_bounds__(64 * kDecWaves, kDecGroupsPerCU) void attn_decode_split_kernel(DecodeParams p) {
  static_assert(D % 16 == 0 && D <= 128, "decode head_dim: a multiple of 16, at most 128");
  // k-slices of S^T = K Q^T, 32 head_dim values each; at head_dim 80 the
  // last slice's chunks 10 and 11 are zero in both operands (never loaded).
  constexpr int KC = (D + 31) / 32;
  __shared__ float red_m[kDecWaves][16];
  __shared__ float red_l[kDecWaves][16];
  __shared__ float red_o[kDecWaves][16][D + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // query column / A-operand row
  const int g = lane >> 4;   // 16-lane row

  // This workgroup's piece [x0, x1) of the slot range; pieces past the end
  // (short caches) have nothing to do and the whole workgroup leaves.
  const int total = dec_total(p, lane);
  const int64_t T = (int64_t)p.Hkv * p.n_hgroups * total;
  const int64_t S = dec_piece(T, p.n_wg);
  const int64_t x0 = (int64_t)blockIdx.x * S;
  if (x0 >= T) return;
  const int64_t x1 = x0 + S < T ? x0 + S : T;
  const float c = p.scale_log2;

  // One segment: keys [k0, k1) of sequence b for unit (kv head hkv, head
  // group hg); its partial results go to piece j of the unit.
  auto segment = [&](int b, int hkv, int hg, int k0, int k1, int j) __attribute__((always_inline)) {
    const int hidx = kDecHeadsPerGroup * hg + n;  // head within the kv group
    const bool hvalid = hidx < p.group;
    const int h = hkv * p.group + hidx;

    // Q^T B operand: k slot (g, i) of slice kc is head_dim index 8*(4*kc + g) + i.
    u32x4 qop[KC];
    {
      const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_sb + (int64_t)h * p.q_sh;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        qop[kc] = hvalid && 8 * (4 * kc + g) < D ? load16(qr + 8 * (4 * kc + g)) : zero16();
    }

    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) + b * p.k_sb + hkv * p.k_sh;
    const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v) + b * p.v_sb + hkv * p.v_sh;

    // equal shares of whole 32-key steps for the waves
    const int share = (k1 - k0 + 32 * kDecWaves - 1) / (32 * kDecWaves) * 32;
    const int w0 = k0 + wave * share;
    const int w1 = min(w0 + share, k1);
    const int last = w1 - 1;  // slots beyond it are read from it (in bounds) and masked

    // The cache is streamed once: its rows are read with non-temporal loads,
    // so they do not displace what the caches hold for other work.
    // K rows as the A operand of S^T: lane row n of 16-key block kb.
    auto load_k = [&](int base, u32x4 (&kr)[2][KC]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* row = kg + (int64_t)min(base + 16 * kb + n, last) * p.k_st;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          kr[kb][kc] = 8 * (4 * kc + g) < D ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 8 * (4 * kc + g)))
                                            : zero16();
      }
    };
    // V rows for the transposed A operand: lane (n, g) loads 8 rows, head_dim
    // chunk n (lanes with 8n >= D load nothing).
    auto load_v = [&](int base, u32x4 (&vr)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = min(base + 16 * (i >> 2) + 4 * g + (i & 3), last);
        vr[i] = (8 * n < D) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + (int64_t)key * p.v_st + 8 * n)) : zero16();
      }
    };

    f32x4 oacc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[t][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    u32x4 kreg[2][KC];
    u32x4 vreg[8];
    if (w0 < w1) {
      load_k(w0, kreg);
      load_v(w0, vreg);
    }

    // Each step's loads for the next 32 keys are issued as soon as the
    // registers they land in have been consumed, so cache rows stay in
    // flight while this step computes.  They are issued on the last step too
    // (its rows clamp to the last slot, in bounds and already cached): loads
    // issued on every path keep the load counter's order known, so each wait
    // covers exactly the loads it needs (conditional prefetches made the
    // compiler also wait for the next step's K rows before this step's P V).
    for (int base = w0; base < w1; base += 32) {
      const int nxt = base + 32;

      // S^T (16 keys x 16 query columns) for the two 16-key blocks.
      f32x4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) s[kb] = mfma16(kreg[kb][kc], qop[kc], s[kb]);
      }
      load_k(nxt, kreg);

      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = base + 16 * kb + 4 * g + r;
          const float x = key < w1 ? s[kb][r] * c : kNegInf;
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_xor32(max_xor16(mx));
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kDecRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[t][r] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kb][r] = fast_exp2(s[kb][r] - m_run);
          rs += s[kb][r];
        }
      l_run += rs;
      // P^T B operand: k slot (g, i) is key base + 16*(i/4) + 4*g + i%4.
      u32x4 pop;
      pop[0] = pack_bf16x2(s[0][0], s[0][1]);
      pop[1] = pack_bf16x2(s[0][2], s[0][3]);
      pop[2] = pack_bf16x2(s[1][0], s[1][1]);
      pop[3] = pack_bf16x2(s[1][2], s[1][3]);

      // A operand of product t: lane row n is head_dim 8n + t, k slot (g, i)
      // the key of vreg[i]; element t of each loaded row, paired by key.
      // Each operand is built right before its product, so only one is live.
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u32x4 a;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          a[jj] = __builtin_amdgcn_perm(vreg[2 * jj + 1][t >> 1], vreg[2 * jj][t >> 1],
                                        (t & 1) ? 0x07060302u : 0x05040100u);
        oacc[t] = mfma16(a, pop, oacc[t]);
      }
      load_v(nxt, vreg);
    }

    // Combine the waves' partial results in LDS.
    const float l_wave = sum_xor32(sum_xor16(l_run));
    if (g == 0) {
      red_m[wave][n] = m_run;
      red_l[wave][n] = l_wave;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 8 * (4 * g + r) + t;
        if (d < D) red_o[wave][n][d] = oacc[t][r];
      }
    __syncthreads();

    const int64_t part_row0 = ((int64_t)b * p.Hq + hkv * p.group + kDecHeadsPerGroup * hg) * p.n_pieces;
    for (int idx = tid; idx < 16 * D; idx += 64 * kDecWaves) {
      const int col = idx / D;
      const int d = idx - col * D;
      if (kDecHeadsPerGroup * hg + col >= p.group) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_m[w][col]);
      float lsum = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float wt = fast_exp2(red_m[w][col] - M);  // empty wave: exp2(-inf) = 0
        lsum += wt * red_l[w][col];
        acc += wt * red_o[w][col][d];
      }
      const int64_t row = part_row0 + (int64_t)col * p.n_pieces + j;
      p.o_part[row * D + d] = acc / lsum;
      if (d == 0) p.lse_part[row] = (M + log2f(lsum)) * kLn2;
    }
    __syncthreads();  // the LDS arrays are reused by the next segment
  };

  // Walk the segments of the piece.  Slot x is position y of unit class
  // u = x / total (kv head u / n_hgroups, head group u % n_hgroups) in the
  // lengths laid end to end.
  for (int64_t x = x0; x < x1;) {
    const int u = (int)(x / total);
    const int y = (int)(x - (int64_t)u * total);
    int b, pre, L;
    dec_find(p, lane, y, b, pre, L);
    const int k0 = y - pre;
    const int k1 = (int)((int64_t)L < k0 + (x1 - x) ? (int64_t)L : k0 + (x1 - x));
    // piece index within the unit: pieces are numbered from the one holding
    // the unit's first slot
    const int j = (int)((int64_t)blockIdx.x - ((int64_t)u * total + pre) / S);
    segment(b, u / p.n_hgroups, u % p.n_hgroups, k0, k1, j);
    x += k1 - k0;
  }
}

// Merge: one wave per (sequence, query head), one head_dim value per lane at
// head_dim 64, two at 80 and 128 (lanes 40-63 idle at 80); four (sequence,
// head) pairs per workgroup.
constexpr int kDecMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kDecMergeWaves) void attn_decode_merge_kernel(DecodeParams p) {
  constexpr int E = (D + 63) / 64;  // head_dim values per lane
  static_assert(E == 1 ? D == 64 : (E == 2 && D % 2 == 0), "merge lanes cover head_dim 64, or up to 128 in pairs");
  const bool lane_on = E * (threadIdx.x & 63) < D;  // the lane holds head_dim values
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * kDecMergeWaves + (threadIdx.x >> 6);
  if (bh >= (int64_t)p.B * p.Hq) return;  // whole wave leaves together
  const int b = (int)(bh / p.Hq);
  const int h = (int)(bh - (int64_t)b * p.Hq);
  // One pass over the lengths gives this sequence's length, its first
  // position and the total.  The pieces of unit (kv head, head group) of
  // sequence b are those holding its slots [u * total + pre, u * total + pre + L).
  int L = 0, pre = 0, total = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int len = b0 + lane < p.B ? dec_len(p, b0 + lane) : 0;
    total += wave_sum_i32(len);
    pre += wave_sum_i32(b0 + lane < b ? len : 0);
    if (b >= b0 && b < b0 + 64) L = __builtin_amdgcn_readlane(len, b - b0);
  }
  int ns = 0;
  if (L > 0) {
    const int64_t S = dec_piece((int64_t)p.Hkv * p.n_hgroups * total, p.n_wg);
    const int hkv = h / p.group;
    const int u = hkv * p.n_hgroups + (h - hkv * p.group) / kDecHeadsPerGroup;
    const int64_t first = (int64_t)u * total + pre;
    ns = (int)((first + L - 1) / S - first / S + 1);
  }
  const int64_t row0 = bh * p.n_pieces;

  // Up to 8 pieces per pass, their loads issued together; the running max
  // and sums are rescaled between passes.
  constexpr int kPass = 8;
  float M = kNegInf, wsum = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kPass) {
    float lsv[kPass], ov[kPass][E];
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const bool ok = s0 + j < ns;
      lsv[j] = ok ? p.lse_part[row0 + s0 + j] : kNegInf;
      const float* src = p.o_part + (row0 + s0 + j) * D + E * lane;
      if constexpr (E == 2) {
        const f32x2 v = ok && lane_on ? *reinterpret_cast<const f32x2*>(src) : f32x2{0.f, 0.f};
        ov[j][0] = v[0];
        ov[j][1] = v[1];
      } else {
        ov[j][0] = ok ? src[0] : 0.f;
      }
    }
    float Mc = M;
#pragma unroll
    for (int j = 0; j < kPass; ++j) Mc = fmaxf(Mc, lsv[j]);
    const float sc = expf(M - Mc);  // first pass: exp(-inf) = 0 on zero sums
    wsum *= sc;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= sc;
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const float w = expf(lsv[j] - Mc);
      wsum += w;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * ov[j][e];
    }
    M = Mc;
  }
  uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + b * p.o_sb + (int64_t)h * p.o_sh;
  const float inv = ns > 0 ? 1.f / wsum : 0.f;
  if constexpr (E == 2) {
    if (lane_on) *reinterpret_cast<uint32_t*>(orow + 2 * lane) = pack_bf16x2(acc[0] * inv, acc[1] * inv);  // bf16, RNE
  } else {
    orow[lane] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
  }
  if (lane == 0) p.lse[bh] = ns > 0 ? M + logf(wsum) : kNegInf;
}

}  // namespace attn_dev
