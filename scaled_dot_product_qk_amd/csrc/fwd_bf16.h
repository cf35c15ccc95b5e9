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
// of query rows); wave w owns 64 rows at head_dim 64 and 32 rows otherwise.
// Key/value tiles of 64 keys are copied from global memory straight into LDS,
// double buffered (three buffers for the pipelined schedule below), and
// shared by the 4 waves.
//
// Orientation: every product is taken transposed, S^T = K Q^T and
// O^T = V^T P^T, so that in both the score accumulator and the output
// accumulator a lane holds one query's values (lane % 32 = query).  Then
//   * the row max and row sum are in-lane reductions plus one exchange with
//     lane ^ 32 (the other half of the keys);
//   * the probabilities leave the score accumulator already in the B-operand
//     layout of the P V product (no LDS round trip);
//   * the rescale of the output by exp(m_old - m_new) is a per-lane scalar.
// V stays row-major in LDS; the V^T operands come from the transposing LDS
// read, visiting the keys of each 16-key slice in the score accumulator's row
// order.
//
// Causal (top-left: query i sees keys j <= i, for any Lq and Lk): key tiles
// entirely above a wave's last row are skipped; tiles that straddle the
// diagonal or the end of the keys are masked to -inf.  Key tile 0 is
// processed first and holds a visible key for every row, so the reference max
// is finite after each row's first tile.
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
  // LSE element strides of (batch, head); the token stride is 1.
  int64_t lse_sb, lse_sh;
  // Packed sequences (NULL for the dense layout): sequence b's query rows are
  // cu_q[b] .. cu_q[b+1]-1 of a [total_q, head, d] tensor, its keys cu_k[b] ..
  // cu_k[b+1]-1; Lq then only sizes the grid (the longest sequence).
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  // Attention mask [B, Hq, Lq, Lk] (NULL if none): element strides of
  // (batch, head, query), key stride 1; uint8 (nonzero: the pair takes part)
  // or bf16 (added to the scaled score).
  const void* mask;
  int64_t m_sb, m_sh, m_sq;
  float inv_abs_scale;   // 1 / |scale|: an additive mask enters the raw score as mask / |scale|
  float scale_log2;      // scale * log2(e)
  float scale_log2_abs;  // |scale * log2(e)|
  int neg_q;             // scale < 0: Q's sign bits are flipped on load (exact)
  float o_mul;           // FP8 inputs: V's descale, applied to O with 1 / l
};

// Work-item order shared by the prefill kernels.  The hardware hands
// consecutive workgroup ids to the 8 XCDs in turn; this maps them so that each
// XCD receives whole (batch, kv head) units, so the workgroups that re-read
// one head's K and V run on the same XCD and share its L2.  Not causal:
// unit by unit, then query tiles, then the query heads of the group.  Causal:
// query tiles heaviest first across the XCD's units (see below).
//
// Packed sequences of different lengths make the work per item uneven across
// sequences, so contiguous ranges would load the XCDs unevenly; there the
// items go in hardware order with the query tile slowest, heaviest first
// across all sequences (items past a sequence's end exit at once).
__device__ __forceinline__ WorkItem prefill_work_item(const FwdParams& p, bool causal) {
  const int L = blockIdx.x;
  const int N = gridDim.x;
  if (p.cu_q != nullptr) {
    const int nb = N / (p.n_qtiles * p.Hq);
    WorkItem it;
    if ((p.Hkv & 7) == 0) {
      // XCD x = L % 8 serves kv heads x, x + 8, ... of every sequence, so the
      // XCDs carry equal work whatever the lengths; on one XCD the items go
      // sequence by sequence (heaviest query tile first, the group's query
      // heads together), so one sequence's K/V at a time lives in its L2.
      // i = ((b * (Hkv / 8) + hkl) * n_qtiles + qi) * group + hg.
      const int x = L & 7;
      int i = L >> 3;
      const int hg = i % p.group;
      i /= p.group;
      const int qi = i % p.n_qtiles;
      i /= p.n_qtiles;
      const int hpx = p.Hkv >> 3;
      it.hk = (i % hpx) * 8 + x;
      it.b = i / hpx;
      it.h = it.hk * p.group + hg;
      it.qt = causal ? p.n_qtiles - 1 - qi : qi;
      return it;
    }
    // L = ((qi * B + b) * Hkv + hk) * group + hg, with N = n_qtiles * B * Hq
    const int hg = L % p.group;
    int r = L / p.group;
    it.hk = r % p.Hkv;
    r /= p.Hkv;
    it.b = r % nb;
    const int qi = r / nb;
    it.h = it.hk * p.group + hg;
    it.qt = causal ? p.n_qtiles - 1 - qi : qi;
    return it;
  }
  // A mask shared by every head (head stride 0) gets the causal order too:
  // the heads of an XCD then read a query tile's mask rows at about the same
  // time.
  const bool shared_mask = p.mask != nullptr && p.m_sh == 0;
  return dense_work_item(L, N, p.n_qtiles, p.group, p.Hkv, causal || shared_mask);
}

// 32-query column blocks per wave: two at head_dim 64 (each K or V^T read
// from LDS then feeds two matrix instructions), one at larger head_dims where
// the output accumulator alone would not leave room for two waves per SIMD.
__host__ __device__ constexpr int bf16_fwd_blocks_per_wave(int d) { return d <= 64 ? 2 : 1; }

template <int D>
struct Bf16FwdShape {
  static constexpr int kWaves = 4;
  static constexpr int kGroupsPerCU = 8 / kWaves;  // workgroups resident per CU (2 waves per SIMD)
  static constexpr int kNB = bf16_fwd_blocks_per_wave(D);
  static constexpr int kRowsPerWave = 32 * kNB;
  static constexpr int kBR = kRowsPerWave * kWaves;  // query rows per workgroup
  static constexpr int kBC = 64;                     // keys per tile
  static constexpr int kKC = D / 16;                 // k-slices of the Q K^T product
  static constexpr int kDP = (D + 31) / 32 * 32;     // rows of O^T padded to 32
  static constexpr int kND = kDP / 32;               // 32-row blocks of O^T
  static constexpr int kChunks = D / 8;              // 16-byte chunks of a row in memory
  static constexpr int kPitch = D <= 64 ? 8 : 16;    // 16-byte chunks of a row in LDS
  static constexpr int kRowBytes = 16 * kPitch;
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kBufBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kRowsPerCopy = 64 / kPitch;  // rows one 1 KB copy instruction fills
  static constexpr int kCopies = 2 * kBC / kRowsPerCopy;  // per tile, K then V
  static constexpr int kCopiesPerWave = kCopies / kWaves;
  static constexpr int kKVar = kPitch == 8 ? 2 : 4;  // K swizzle patterns across one wave's copies
  static_assert(D % 16 == 0, "head_dim must be a multiple of 16");
  static_assert(kChunks <= kPitch && 2 * kDP <= kRowBytes, "a padded row must fit its LDS pitch");
  static_assert(kCopiesPerWave % kKVar == 0 && (kWaves / 2) * kCopiesPerWave * kRowsPerCopy == kBC,
                "each wave copies whole swizzle periods of one of the two tiles");
  static_assert(kBufBytes < 65536, "in-buffer LDS offsets must fit the instruction offset field");
};

// Key/value tile buffers in LDS: three for the pipelined schedule (head_dim
// 64, no mask, causal or not; there a tile's V operands are read after the
// barrier at which the copies of the tile two ahead are issued), two
// otherwise.
__host__ __device__ constexpr int bf16_fwd_kv_stages(int d, bool causal, int mk) {
  return d == 64 && mk == 0 ? 3 : 2;
}

// Attention-mask tiles (MK: 1 uint8 boolean, 2 bf16 additive): the
// workgroup's query rows x the 64 keys of a tile, row-major, double buffered
// after the key/value buffers, copied with the key/value tiles.
template <int D, bool CAUSAL, int MK>
struct FwdMaskShape {
  using S = Bf16FwdShape<D>;
  static_assert(S::kCopiesPerWave + (MK == 0 ? 0 : S::kBR / (1024 / (S::kBC * (MK == 1 ? 1 : 2))) / S::kWaves) < 16,
                "copies in flight per wave fit the simple vmcnt encoding");
  static constexpr int kEs = MK == 1 ? 1 : 2;             // bytes per element
  static constexpr int kRowBytes = S::kBC * kEs;           // 64 or 128
  static constexpr int kChunkKeys = 16 / kEs;              // keys per 16-byte chunk
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kTileBytes = S::kBR * kRowBytes;
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;
  static constexpr int kCopies = MK == 0 ? 0 : S::kBR / kRowsPerCopy;
  static constexpr int kCopiesPerWave = kCopies / S::kWaves;
  static constexpr int kLdsBytes = MK == 0 ? 0 : 2 * kTileBytes;
  static_assert(MK == 0 || kCopies % S::kWaves == 0, "mask copies split evenly over the waves");
  // A mask row's 16-byte chunks are XOR-swizzled by the row index: chunk c
  // of row r sits in slot c ^ swz(r), swz(r) = (r / kRowsPerSpan) %
  // kChunksPerRow, kRowsPerSpan being the rows in one pass over the 64 banks
  // (256 bytes).  A mask read takes the same key offset from 32 rows; without
  // the swizzle those fall on 4 (boolean) or 2 (additive) bank positions,
  // with it on 16, so the read is 2-way instead of 8- or 16-way conflicted.
  static constexpr int kRowsPerSpan = 256 / kRowBytes;
  static constexpr int kSwzRows = kRowsPerSpan * kChunksPerRow;  // period of swz
  static constexpr int kSwzVar = kSwzRows > kRowsPerCopy ? kSwzRows / kRowsPerCopy : 1;
  static_assert(MK == 0 || (kCopiesPerWave * kRowsPerCopy) % kSwzRows == 0,
                "each wave's first mask row starts a swizzle period");
  static_assert(MK == 0 || (S::kRowsPerWave % kSwzRows == 0 && 32 % kSwzRows == 0),
                "a query row's swizzle depends on its lane only");
  __device__ static int swz(int r) { return (r / kRowsPerSpan) % kChunksPerRow; }
  // dynamic LDS of the kernel: key/value buffers, then the mask tiles
  static constexpr int kKVBytes = bf16_fwd_kv_stages(D, CAUSAL, MK) * S::kBufBytes;
  static constexpr int kKernelLdsBytes = kKVBytes + kLdsBytes;
};

// LDS layout of a key row: its 16-byte chunks are XOR-swizzled by the row
// index so that the operand reads spread over all banks.
//   K (A operand of S^T = K Q^T, 16 bytes of 32 consecutive rows per read):
//     8-chunk rows: c ^ (r & 7) ^ ((r >> 3) & 1); 16-chunk rows: c ^ (r & 15).
//     Any 8 consecutive rows at one logical chunk use 8 different chunks, and
//     any 16 use 16 different (row parity, chunk) bank groups.
//   V (read with ds_read_b64_tr_b16, 32 bytes of 4 consecutive rows per
//     16-lane group): the 32-byte halves are XOR-ed by r & 3, which puts the 4
//     rows in 4 different bank groups.
template <int PITCH>
__device__ __forceinline__ int fwd_k_swz(int r) {
  return PITCH == 8 ? (r & 7) ^ ((r >> 3) & 1) : (r & 15);
}
template <int PITCH>
__device__ __forceinline__ int fwd_v_swz(int r) {
  return (PITCH / 4) * (r & 3);
}

__device__ __forceinline__ void fwd_copy16(const void* base, uint32_t off, uint32_t lds_base) {
  lds_copy16(base, off, lds_base);
}

// Largest K/V token stride (elements) the copies' 32-bit lane offsets allow:
// a lane's offset spans at most 7 rows plus one row's chunks.
constexpr int64_t kFwdMaxTokenStride = int64_t(1) << 28;

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

template <int D, bool CAUSAL, int MK = 0>
__global__ __launch_bounds__(64 * Bf16FwdShape<D>::kWaves, Bf16FwdShape<D>::kGroupsPerCU) void
attn_fwd_bf16_kernel(FwdParams p_in) {
  using S = Bf16FwdShape<D>;
  using MS = FwdMaskShape<D, CAUSAL, MK>;
  constexpr int NB = S::kNB;
  constexpr int kStages = bf16_fwd_kv_stages(D, CAUSAL, MK);
  constexpr bool kPipe = kStages == 3;  // the pipelined schedule
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  lds_char* const lds_b = (lds_char*)(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31;  // query column within a 32-query block (n index)
  const int g = lane >> 5;   // lane half

  FwdParams p = p_in;
  const WorkItem wi = prefill_work_item(p, CAUSAL);
  const int b = wi.b, h = wi.h, hk = wi.hk;
  const int q0 = wi.qt * S::kBR;
  // Packed sequences: this work item's sequence, its bounds clamped to the
  // packed extents (inconsistent offsets then cannot reach past the buffers).
  // Work items past the end of a shorter sequence have nothing to do.
  if (p.cu_q != nullptr) {
    const int qs = min(max(p.cu_q[b], 0), p.total_q), qe = min(max(p.cu_q[b + 1], qs), p.total_q);
    const int ks = min(max(p.cu_k[b], 0), p.total_k), ke = min(max(p.cu_k[b + 1], ks), p.total_k);
    p.Lq = qe - qs;
    p.Lk = ke - ks;
    p.q = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)qs * p.q_st;
    p.o = reinterpret_cast<uint16_t*>(p.o) + (int64_t)qs * p.o_st;
    p.lse += qs;
    p.k = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)ks * p.k_st;
    p.v = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)ks * p.v_st;
  }
  if (q0 >= p.Lq) return;
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

  // ---- tile copies: global memory straight into LDS, no registers ----
  // Copy instruction ci of a tile fills kRowsPerCopy rows (1 KB, lane l ->
  // row l / kPitch, physical chunk l % kPitch) of the K tile (first half of
  // the ci range) or the V tile; wave w issues kCopiesPerWave consecutive
  // ones, so waves 0-1 copy K and waves 2-3 copy V.  Each lane fetches the
  // logical chunk its slot holds.  A slot of a padding chunk (head_dim 80:
  // chunks 10-15 of a 16-chunk LDS row) fetches chunk c - 8 of its row
  // instead, which a lane of the same instruction already requests: no K
  // read touches the padding, and the V^T rows it feeds are discarded.  So
  // every lane copies and each issue_tile issues exactly kCopiesPerWave
  // copy instructions on every path, which the vmcnt waits below count on.
  // Per-lane offsets repeat with period kKVar copies.
  constexpr int kHalfCopies = S::kCopies / 2;
  const bool copies_k = wave < S::kWaves / 2;
  const uint16_t* cp_src = copies_k ? kg : vg;
  const int64_t cp_st = copies_k ? p.k_st : p.v_st;
  const int cp_row = lane / S::kPitch;  // row within one copy
  const int cp_row0 = S::kRowsPerCopy * ((wave % (S::kWaves / 2)) * S::kCopiesPerWave);
  const uint32_t cp_lds0 = (uint32_t)(uintptr_t)lds_b + (copies_k ? 0 : S::kTileBytes) + cp_row0 * S::kRowBytes;
  int cp_chunk16[S::kKVar];   // byte offset of the chunk the lane fetches
  uint32_t cp_off[S::kKVar];  // byte offset of that chunk within its copy
  const uint32_t cp_row_bytes = (uint32_t)(2 * cp_st);  // < 2^29: token strides are validated
  static_assert(S::kChunks == S::kPitch || (S::kChunks >= 8 && S::kPitch - 8 <= S::kChunks),
                "a padding slot's stand-in chunk c - 8 is a real chunk of the row");
#pragma unroll
  for (int v = 0; v < S::kKVar; ++v) {
    const int r = S::kRowsPerCopy * v + cp_row;  // row index modulo the swizzle period
    const int pc = lane % S::kPitch;
    int lc = pc ^ (copies_k ? fwd_k_swz<S::kPitch>(r) : fwd_v_swz<S::kPitch>(r));
    if (lc >= S::kChunks) lc -= 8;  // padding slot
    cp_chunk16[v] = 16 * lc;
    cp_off[v] = (uint32_t)cp_row * cp_row_bytes + 16 * lc;
  }
  // Mask copy plan: wave w fills mask-tile rows m_row0 .. m_row0 +
  // MS::kCopiesPerWave * MS::kRowsPerCopy - 1; lane l -> row l / chunks-per-row,
  // 16-byte chunk l % chunks-per-row.
  const char* m_base = nullptr;
  int64_t m_row_bytes = 0;
  int m_lrow = 0, m_row0 = 0;
  int m_key[MS::kSwzVar];  // first key, within the tile, of the chunk the lane fetches
  uint32_t m_lds0 = 0;
  if constexpr (MK != 0) {
    m_base = reinterpret_cast<const char*>(p.mask) + (b * p.m_sb + h * p.m_sh) * MS::kEs;
    m_row_bytes = p.m_sq * MS::kEs;
    m_lrow = lane / MS::kChunksPerRow;
    m_row0 = wave * MS::kCopiesPerWave * MS::kRowsPerCopy;
    m_lds0 = (uint32_t)(uintptr_t)lds_b + MS::kKVBytes;
#pragma unroll
    for (int v = 0; v < MS::kSwzVar; ++v)
      m_key[v] = MS::kChunkKeys * ((lane % MS::kChunksPerRow) ^ MS::swz(MS::kRowsPerCopy * v + m_lrow));
  }
  // Full tiles copy without checks; the tile holding key Lk - 1 reads rows
  // beyond it from row Lk - 1 instead (in bounds and finite), and those keys
  // are masked to -inf, so they carry weight 0.
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int kv0 = t * S::kBC;
    const uint32_t dst = cp_lds0 + buf * S::kBufBytes;
    if (t < n_full) {
#pragma unroll
      for (int j = 0; j < S::kCopiesPerWave; ++j) {
        const uint16_t* src = cp_src + (int64_t)(kv0 + cp_row0 + S::kRowsPerCopy * j) * cp_st;
        fwd_copy16(src, cp_off[j % S::kKVar], dst + j * S::kRowsPerCopy * S::kRowBytes);
      }
    } else {
      const int last = p.Lk - 1;
#pragma unroll
      for (int j = 0; j < S::kCopiesPerWave; ++j) {
        const int row0 = min(kv0 + cp_row0 + S::kRowsPerCopy * j, last);
        const int row = min(kv0 + cp_row0 + S::kRowsPerCopy * j + cp_row, last);
        fwd_copy16(cp_src + (int64_t)row0 * cp_st, (uint32_t)(row - row0) * cp_row_bytes + cp_chunk16[j % S::kKVar],
                   dst + j * S::kRowsPerCopy * S::kRowBytes);
      }
    }
    if constexpr (MK != 0) {
      // Mask rows q0 + m_row0 + ... of this tile's 64 keys.  Every lane
      // copies (rows past Lq repeat row Lq - 1, chunks past Lk repeat the
      // last chunk; both are masked anyway), so each wave issues exactly
      // MS::kCopiesPerWave copies per tile.  Lane l fills slot l % chunks-
      // per-row of its row and fetches the chunk the swizzle puts there.
      const uint32_t mdst = m_lds0 + (t & 1) * MS::kTileBytes;
#pragma unroll
      for (int j = 0; j < MS::kCopiesPerWave; ++j) {
        const int kc0 = min(kv0 + m_key[j % MS::kSwzVar], p.Lk - MS::kChunkKeys);
        const int r = q0 + m_row0 + MS::kRowsPerCopy * j;
        const int ra = min(r, p.Lq - 1), rl = min(r + m_lrow, p.Lq - 1);
        fwd_copy16(m_base + (int64_t)ra * m_row_bytes, (uint32_t)(rl - ra) * (uint32_t)m_row_bytes + kc0 * MS::kEs,
                   mdst + (m_row0 + MS::kRowsPerCopy * j) * MS::kRowBytes);
      }
    }
    copy_group_end();
  };

  // ---- LDS operand offsets (bytes within a buffer) ----
  // K A operand of slice kc: row lq (+32 per key half), logical chunk 2 kc + g.
  // The swizzle only flips chunk bits, so slice kc's offset is slice 0's with
  // bits 5 and up flipped by kc.
  const int k_rd = lq * S::kRowBytes + 16 * (fwd_k_swz<S::kPitch>(lq) ^ g);
  // V^T A operand of d-block db, 16-key slice cs, from two transposing reads:
  // lane (G = lane / 16, i = lane % 16 / 4, q = lane % 4) points at key row
  // 16 cs + 4 g + i (+ 8 for the second read), head_dim 32 db + 16 (G & 1) +
  // 4 q, and receives that head_dim index of keys 16 cs + 4 g + 0..3 (+ 8):
  // the key order of the score accumulator's rows, i.e. of P's B operand.
  int v_rd[S::kND];
  {
    const int G = lane >> 4, i = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int db = 0; db < S::kND; ++db) {
      const int d0 = 32 * db + 16 * (G & 1) + 4 * q;  // 4 elements within one chunk
      v_rd[db] = S::kTileBytes + (4 * g + i) * S::kRowBytes +
                 16 * ((d0 >> 3) ^ fwd_v_swz<S::kPitch>(i)) + 2 * (d0 & 7);
    }
  }

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

  // Key tiles are taken as two 32-key halves, each with its own sum guard
  // (the probabilities of a half depend only on its own scores and the
  // reference max, see kSumGuard), so that the products of one half can run
  // on the matrix core while the vector ALU forms the softmax of another.
  //
  // Head_dim 64, no mask, causal or not (kPipe): a software pipeline across
  // tiles.  With S(t, h) the scores of half h of tile t and PV(t, h) its
  // O^T += V^T P^T products,
  //
  //   phase A of tile t:  PV(t-1, 1) + S(t, 1)    beside softmax(t, 0)
  //   (wait for tile t+1, barrier, copy tile t+2, read K of tile t+1)
  //   phase B of tile t:  PV(t, 0)   + S(t+1, 0)  beside softmax(t, 1)
  //
  // so every softmax half runs beside 16 products.  A rescale of O in
  // softmax(t, h) follows, in program order, the products of every earlier
  // half (their probabilities were formed against the old reference), so it
  // scales them too and stays exact.  The second half's V^T operands are
  // read at the end of phase B, after the barrier of tile t: with three LDS
  // buffers, tile t's buffer is refilled only after the barrier of tile t + 1.
  //
  // Causal, every wave runs every key tile of its workgroup, the tiles on
  // the diagonal masked inside the pipeline (fused_half with MASK), so that
  // no wave leaves the shared schedule early.
  //
  // The other instances (head_dim 80 and 128, and every masked one) keep
  // both softmax halves of a tile before its barrier, which needs fewer
  // registers and, with a mask, keeps the mask words of the tile readable
  // from LDS:
  //
  //   S(t, 0) | S(t, 1) + softmax(t, 0) | PV(t, 0) + softmax(t, 1) | barrier | PV(t, 1)
  u32x4 ka_next[S::kKC];     // K operands, first key half of the next tile
  u32x4 ka1[S::kKC];         // K operands, second key half of this tile
  u32x4 va0[S::kND][2];      // V^T operands, first key half of this tile
  u32x4 va_last[S::kND][2];  // V^T operands, second key half of this tile
  u32x4 pop[NB][4];          // P^T B operands, one per 16-key slice
  f32x16 s[NB][2];           // S^T accumulators, one per key half
  // (the buffer's byte offset goes through readfirstlane so that it stays one
  // scalar term of the address and the constant parts fold into the
  // instructions' offset fields)
  auto buf_bytes = [&](int buf) { return __builtin_amdgcn_readfirstlane(buf * S::kBufBytes); };
  auto read_k = [&](int buf, int sb, u32x4 (&ka)[S::kKC]) {
    const lds_char* kb = lds_b + buf_bytes(buf);
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc)
      ka[kc] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          kb + (k_rd ^ (32 * kc)) + 32 * sb * S::kRowBytes);
  };
  auto read_v = [&](int buf, int sb, u32x4 (&va)[S::kND][2]) {
    lds_char* vb = lds_b + buf_bytes(buf);
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        lds_char* a0 = vb + v_rd[db] + 16 * (2 * sb + j) * S::kRowBytes;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)a0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a0 + 8 * S::kRowBytes));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        va[db][j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
  };
  auto qk = [&](int sb, const u32x4 (&ka)[S::kKC]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][sb][r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb][sb] = mfma32(ka[kc], qop[nb][kc], s[nb][sb]);
  };
  // Both halves' scores, the two accumulation chains interleaved.
  auto qk_both = [&](const u32x4 (&k0)[S::kKC], const u32x4 (&k1)[S::kKC]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][0][r] = s[nb][1][r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < S::kKC; ++kc)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        s[nb][0] = mfma32(k0[kc], qop[nb][kc], s[nb][0]);
        s[nb][1] = mfma32(k1[kc], qop[nb][kc], s[nb][1]);
      }
  };
  // (the 16-key slices j outermost, so that consecutive products accumulate
  // into different output blocks even with one row block per wave)
  auto pv = [&](int sb, const u32x4 (&va)[S::kND][2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < S::kND; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][db] = mfma32(va[db][j], pop[nb][2 * sb + j], oacc[nb][db]);
  };
  // P = exp2(c s - m) for half sb of row block nb, packed as two P^T B
  // operands; returns this lane's share of the half's row sum.
  auto exp_half = [&](int sb, int nb) __attribute__((always_inline)) {
    // (with an attention mask a row may still have no visible key: its
    // reference stays -inf and every probability is exp2(-inf) = 0)
    const float neg_m = (MK != 0 && m_run[nb] == kNegInf) ? 0.f : -m_run[nb];
    // four short dependency chains, each started by its first value (an
    // explicit 0 + e is an instruction: the compiler keeps it for signed zeros)
    float rs[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = fast_exp2(__builtin_fmaf(s[nb][sb][8 * half + i], c, neg_m));
        if (half == 0 && i < 4)
          rs[i] = e[i];
        else
          rs[i & 3] += e[i];
      }
      u32x4 pk;
      pk[0] = pack_bf16x2(e[0], e[1]);
      pk[1] = pack_bf16x2(e[2], e[3]);
      pk[2] = pack_bf16x2(e[4], e[5]);
      pk[3] = pack_bf16x2(e[6], e[7]);
      // keep the packs here, among the products: the compiler would
      // otherwise sink them past the guard's branch (the exact path forms
      // them again), where they run with no product beside them
      asm volatile("" : "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]), "+v"(pk[3]));
      pop[nb][2 * sb + half] = pk;
    }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };
  // The end of a half's softmax: if the sum guard failed for some lane, take
  // the half's max, move the reference, rescale O and l and form the
  // probabilities again; then add the half's sums to l.
  auto finish_half = [&](int sb, bool redo, float (&ls)[NB]) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = kNegInf;
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
        ls[nb] = exp_half(sb, nb);
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) l_run[nb] += ls[nb];
  };
  // Softmax of half sb of the tile in buffer buf starting at key kv0; MASK
  // selects the variant that masks keys beyond Lk and (causal) keys after the
  // query.  N_MFMA products issued just before it are spread between its
  // vector instructions.
  auto softmax_half = [&](auto mask_tag, int buf, int kv0, int sb, auto n_mfma_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int N_MFMA = decltype(n_mfma_tag)::value;
    if constexpr (MASK) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool vis = key < p.Lk && (!CAUSAL || key <= qrow[nb]);
          s[nb][sb][r] = vis ? s[nb][sb][r] : kNegInf;
        }
    }
    if constexpr (MK != 0) {
      // Keys 32 sb + 8 j + 4 g + 0..3 of this lane's query row in the mask
      // tile: a boolean removes pairs, an additive mask enters the raw score
      // as mask / |scale| (so the exponent gets scale s + mask, in log2 units).
      // Query row 32 nb + lq of the wave has swizzle swz(lq).
      const lds_char* mt = lds_b + MS::kKVBytes + buf * MS::kTileBytes;
      const int m_x = 16 * MS::swz(lq);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const lds_char* mrow = mt + (wave * S::kRowsPerWave + 32 * nb + lq) * MS::kRowBytes + 4 * g * MS::kEs;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int off = ((32 * sb + 8 * j) * MS::kEs) ^ m_x;  // flips bits 4 and up only
          if constexpr (MK == 1) {
            const uint32_t w = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(mrow + off);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[nb][sb][4 * j + e] = ((w >> (8 * e)) & 0xffu) ? s[nb][sb][4 * j + e] : kNegInf;
          } else {
            const u32x2 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(mrow + off);
            s[nb][sb][4 * j + 0] = __builtin_fmaf(bf16_lo(w[0]), p.inv_abs_scale, s[nb][sb][4 * j + 0]);
            s[nb][sb][4 * j + 1] = __builtin_fmaf(bf16_hi(w[0]), p.inv_abs_scale, s[nb][sb][4 * j + 1]);
            s[nb][sb][4 * j + 2] = __builtin_fmaf(bf16_lo(w[1]), p.inv_abs_scale, s[nb][sb][4 * j + 2]);
            s[nb][sb][4 * j + 3] = __builtin_fmaf(bf16_hi(w[1]), p.inv_abs_scale, s[nb][sb][4 * j + 3]);
          }
        }
      }
    }
    float ls[NB];
    bool redo = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      ls[nb] = exp_half(sb, nb);
      // a row still without a visible key always takes the exact path
      redo = redo || !(ls[nb] <= kSumGuard) || (MK != 0 && m_run[nb] == kNegInf);
    }
    // about 60 vector instructions per row block: one product per share
    if constexpr (N_MFMA > 0) {
#pragma unroll
      for (int i = 0; i < N_MFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 56 * NB / N_MFMA, 0);
      }
    }
    finish_half(sb, redo, ls);
  };

  // Pipelined schedule, tiles without a mask: the 16 products of a phase —
  // P V of the other half ob = 1 - sb, then the scores of the next half ob —
  // and the softmax of half sb in a fixed interleave, one product per two
  // probabilities (two FMAs, two exponentials, two sums, one pack), each
  // group closed by a scheduling barrier.  Left to the scheduler, the
  // products of a phase bunched together and the vector work ran alone after
  // them.  The arithmetic and its order are those of exp_half.
  // MASK: the tile holds keys beyond Lk or (causal) after some query of the
  // wave; those scores are set to -inf as their probabilities are formed
  // (and left so in s, for the exact path).
  auto fused_half = [&](auto mask_tag, int kv0, int sb, const u32x4 (&va)[S::kND][2], const u32x4 (&ka)[S::kKC])
                        __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (kPipe) {
      static_assert(NB == 2 && S::kND == 2 && S::kKC == 4, "one product per two probabilities");
      const int ob = 1 - sb;
      float rs[NB][4];
      u32x4 pk[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][ob][r] = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < 8) {
          const int db = k >> 2, j = (k >> 1) & 1, nb = k & 1;
          oacc[nb][db] = mfma32(va[db][j], pop[nb][2 * ob + j], oacc[nb][db]);
        } else {
          const int kc = (k - 8) >> 1, nb = k & 1;
          s[nb][ob] = mfma32(ka[kc], qop[nb][kc], s[nb][ob]);
        }
        const int nb = k >> 3, w = k & 7;  // probabilities 2w, 2w + 1 of row block nb
        if constexpr (MASK) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 2 * w + e;
            const int key = kv0 + 32 * sb + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool vis = key < p.Lk && (!CAUSAL || key <= qrow[nb]);
            s[nb][sb][r] = vis ? s[nb][sb][r] : kNegInf;
          }
        }
        const float e0 = fast_exp2(__builtin_fmaf(s[nb][sb][2 * w], c, -m_run[nb]));
        const float e1 = fast_exp2(__builtin_fmaf(s[nb][sb][2 * w + 1], c, -m_run[nb]));
        if (w < 2) {
          rs[nb][(2 * w) & 3] = e0;
          rs[nb][(2 * w + 1) & 3] = e1;
        } else {
          rs[nb][(2 * w) & 3] += e0;
          rs[nb][(2 * w + 1) & 3] += e1;
        }
        uint32_t pw = pack_bf16x2(e0, e1);
        asm volatile("" : "+v"(pw));
        pk[nb][w >> 2][w & 3] = pw;
        __builtin_amdgcn_sched_barrier(0);
      }
      float ls[NB];
      bool redo = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        ls[nb] = (rs[nb][0] + rs[nb][1]) + (rs[nb][2] + rs[nb][3]);
        pop[nb][2 * sb] = pk[nb][0];
        pop[nb][2 * sb + 1] = pk[nb][1];
        redo = redo || !(ls[nb] <= kSumGuard);
      }
      finish_half(sb, redo, ls);
    }
  };

  constexpr int kQKMfma = S::kKC * NB, kPVMfma = S::kND * 2 * NB;
  using QKTag = std::integral_constant<int, kQKMfma>;
  using PVTag = std::integral_constant<int, kPVMfma>;
  using BothTag = std::integral_constant<int, kQKMfma + kPVMfma>;
  using NoneTag = std::integral_constant<int, 0>;

  // Q must have landed before the first copy: the copies are invisible to the
  // compiler, and a later wait for Q would not know to let them run on.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  if (n_tiles > 0) issue_tile(0, 0);
  if (n_tiles > 1) {
    issue_tile(1, 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(S::kCopiesPerWave + MS::kCopiesPerWave));  // tile 0's copies done
  } else {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }
  __syncthreads();
  auto active = [&](int t) { return t < n_tiles && (kPipe || !CAUSAL || t * S::kBC <= wave_last_row); };
  if (active(0)) read_k(0, 0, ka_next);

  // Between the halves of tile t: wait for this wave's copies of tile t + 1
  // and barrier (all copies of t + 1 are in LDS, and every wave is done with
  // the buffer that tile t + 2 refills: tile t's with two buffers, tile
  // t - 1's with three), copy tile t + 2 into buffer buf2 and read the first
  // K operands of tile t + 1 from buffer buf1.
  auto turn = [&](int t, int buf1, int buf2) __attribute__((always_inline)) {
    if (t + 1 < n_tiles) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      __syncthreads();
      if (t + 2 < n_tiles) issue_tile(t + 2, buf2);
      if (active(t + 1)) read_k(buf1, 0, ka_next);
    }
  };
  // Tiles that need no mask for any wave of the workgroup come first; the
  // tail of the key range and the diagonal tiles follow with the masked
  // path.
  int n_plain = min(n_tiles, n_full);
  if (CAUSAL) n_plain = min(n_plain, (q0 + 1) / S::kBC);
  if constexpr (kPipe) {
    // Before tile 0 there is no earlier half: its products run on zero
    // probabilities and zero operands and add nothing, which keeps one copy
    // of the step (a separate first step costs registers).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 2; i < 4; ++i) pop[nb][i] = zero16();
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j) va_last[db][j] = zero16();
    if (active(0)) qk(0, ka_next);
    // With no key of tile 0 past Lk, the reference starts at the first half's
    // row max (no key is masked here), so tile 0 does not take the exact
    // path that a reference of -inf would force on both of its halves.
    if (n_plain > 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][0][r]);
        m_run[nb] = max_xor32(mx) * c;  // the scale is positive
      }
    }
    // Phase A of tile t (the wave is active there).  The V^T operands of the
    // first half are read at its end, before the barrier; those of the
    // second half at the end of phase B (the buffer of tile t is refilled
    // only at the barrier of tile t + 1).
    auto phase_a = [&](auto mask_tag, int t, int buf) __attribute__((always_inline)) {
      read_k(buf, 1, ka1);
      fused_half(mask_tag, t * S::kBC, 0, va_last, ka1);
      read_v(buf, 0, va0);
    };
    // Phase B; the products S(t + 1, 0) are issued whether or not the wave
    // is active in tile t + 1 (then on stale operands, and never used), so
    // that they stay in one scheduling region with the softmax.
    auto phase_b = [&](auto mask_tag, int t, int buf) __attribute__((always_inline)) {
      fused_half(mask_tag, t * S::kBC, 1, va0, ka_next);
      read_v(buf, 1, va_last);
      if (!active(t + 1)) pv(1, va_last);  // the wave's last tile
    };
    // Tile t lives in buffer t % 3.  BUF is that buffer when the caller
    // knows it at compile time (then every LDS address of the step is a
    // register plus a constant offset), -1 otherwise.
    auto step = [&](auto mask_tag, int t, auto buf_tag) __attribute__((always_inline)) {
      constexpr int BUF = decltype(buf_tag)::value;
      const int buf = BUF >= 0 ? BUF : (int)((unsigned)t % 3);
      const int buf1 = BUF >= 0 ? (BUF + 1) % 3 : (int)((unsigned)(t + 1) % 3);
      const int buf2 = BUF >= 0 ? (BUF + 2) % 3 : (int)((unsigned)(t + 2) % 3);
      const bool act = active(t);
      if (act) phase_a(mask_tag, t, buf);
      turn(t, buf1, buf2);
      if (act) phase_b(mask_tag, t, buf);
    };
    // Unmasked tiles three at a time (one pass through the three buffers);
    // the last one or two of them run with the masked path, which is exact
    // for them as well.
    int t = 0;
    // Not causal (every work item the same size): the wave priority falls
    // with the share of the key tiles done (3 in the first quarter, 0 in the
    // last), so on a SIMD shared by two workgroups the wave with more work
    // left issues first.  Left to the age order (oldest wave first), the
    // first workgroup on each compute unit ran its tiles 1.6x as fast as the
    // second, the two drifted apart, and the last round of work items ended
    // up to 90 us apart across compute units (34 us with the priority).
    // Causal items differ in size, and the same rule slowed them.
    int prio = 4;
    auto lower_prio = [&](int t) __attribute__((always_inline)) {
      if constexpr (!CAUSAL) {
        const int want = 3 - min(3, (4 * t) / max(n_tiles, 1));
        if (want < prio) {
          prio = want;
          switch (want) {
            case 3: __builtin_amdgcn_s_setprio(3); break;
            case 2: __builtin_amdgcn_s_setprio(2); break;
            case 1: __builtin_amdgcn_s_setprio(1); break;
            default: __builtin_amdgcn_s_setprio(0); break;
          }
        }
      }
    };
    for (; t + 3 <= n_plain; t += 3) {
      lower_prio(t);
      step(std::false_type{}, t, std::integral_constant<int, 0>{});
      step(std::false_type{}, t + 1, std::integral_constant<int, 1>{});
      step(std::false_type{}, t + 2, std::integral_constant<int, 2>{});
    }
    for (; t < n_tiles; ++t) {
      lower_prio(t);
      step(std::true_type{}, t, std::integral_constant<int, -1>{});
    }
    if constexpr (!CAUSAL) __builtin_amdgcn_s_setprio(0);
  } else {
    auto step = [&](auto mask_tag, int t) __attribute__((always_inline)) {
      const bool act = active(t);
      const int buf = t & 1, kv0 = t * S::kBC;
      if (act) {
        read_k(buf, 1, ka1);
        if constexpr (NB == 1) {
          // One row block per wave: both halves' scores first, their two
          // accumulation chains interleaved; the softmax of the first half
          // then runs beside the other wave's products.  (Same speed as
          // the first half's scores alone before it, and no spilled
          // registers at head_dim 128, where that order spilled 9.)
          qk_both(ka_next, ka1);
          read_v(buf, 0, va0);
          softmax_half(mask_tag, buf, kv0, 0, NoneTag{});
        } else {
          __builtin_amdgcn_s_setprio(2);
          qk(0, ka_next);
          __builtin_amdgcn_s_setprio(0);
          read_v(buf, 0, va0);
          qk(1, ka1);
          softmax_half(mask_tag, buf, kv0, 0, QKTag{});
        }
        read_v(buf, 1, va_last);
        pv(0, va0);
        softmax_half(mask_tag, buf, kv0, 1, PVTag{});
      }
      turn(t, (t + 1) & 1, t & 1);
      if (act) {
        __builtin_amdgcn_s_setprio(2);
        pv(1, va_last);
        __builtin_amdgcn_s_setprio(0);
      }
    };
    int t = 0;
    for (; t < n_plain; ++t) step(std::false_type{}, t);
    for (; t < n_tiles; ++t) step(std::true_type{}, t);
  }

  // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2 ----
  // O is written once and not read again by this call, so it bypasses the
  // caches' allocation (non-temporal stores): left dirty in the caches it
  // would be written back later, taking HBM bandwidth from whatever runs
  // next (a decode step, say).  Non-temporal stores must cover whole lines to
  // stay cheap, so at head_dim 64 and 128 each wave first turns its rows
  // around in LDS (16-byte chunks XOR-swizzled by row) and then stores whole
  // rows, 16 bytes per lane.
  constexpr bool kStaged = D == 64 || D == 128;
  constexpr int kCPR = D / 8;  // 16-byte chunks per row
  constexpr int kRowB = 2 * D;
  lds_char* const st = lds_b + wave * S::kRowsPerWave * kRowB;
  if constexpr (kStaged) __syncthreads();  // every wave is done with the key/value buffers
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float l_tot = sum_xor32(l_run[nb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (g == 0 && qrow[nb] < p.Lq) {
      const float lse = l_tot > 0.f ? (m_run[nb] + log2f(l_tot)) * kLn2 : kNegInf;
      __builtin_nontemporal_store(lse, &p.lse[b * p.lse_sb + h * p.lse_sh + qrow[nb]]);
    }
    uint16_t* const orow = reinterpret_cast<uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qrow[nb] * p.o_st;
    const int r = 32 * nb + lq;
#pragma unroll
    for (int db = 0; db < S::kND; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * db + 8 * j + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[nb][db][4 * j + 0] * inv, oacc[nb][db][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[nb][db][4 * j + 2] * inv, oacc[nb][db][4 * j + 3] * inv);
        if constexpr (kStaged) {
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
              st + r * kRowB + 16 * ((d >> 3) ^ (r & (kCPR - 1))) + 8 * g) = w;
        } else if (d < D && qrow[nb] < p.Lq) {
          __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(orow + d));
        }
      }
  }
  if constexpr (kStaged) {
    uint16_t* const obase = reinterpret_cast<uint16_t*>(p.o) + b * p.o_sb + h * p.o_sh;
#pragma unroll
    for (int i = 0; i < S::kRowsPerWave * kCPR / 64; ++i) {
      const int idx = 64 * i + lane;
      const int r = idx / kCPR, c = idx % kCPR;
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          st + r * kRowB + 16 * (c ^ (r & (kCPR - 1))));
      const int row = row0 + r;
      if (row < p.Lq) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (int64_t)row * p.o_st + 8 * c));
    }
  }
}

}  // namespace attn_dev
