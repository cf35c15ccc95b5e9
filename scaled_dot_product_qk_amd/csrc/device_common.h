// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix-core operand layouts used throughout (wave64; l = lane id):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds A[m = l%32][k = 8*(l/32) + i], i < 8
//                             B: lane l holds B[k = 8*(l/32) + i][n = l%32]
//                             C: lane l, reg r < 16 holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
//   v_mfma_f32_16x16x32_bf16  A: lane l holds A[m = l%16][k = 8*(l/16) + i]
//                             B: lane l holds B[k = 8*(l/16) + i][n = l%16]
//                             C: lane l, reg r < 4 holds C[4*(l/16) + r][l%16]
//   v_mfma_f32_32x32x2_f32    A: lane l holds A[m = l%32][k = l/32]
//                             B: lane l holds B[k = l/32][n = l%32]
//                             C: as for 32x32x16.
// Only the m/n placement and the C layout matter to the kernels: the k index
// is contracted, so any fixed assignment of k slots to lanes works as long as
// the A and B operands agree on it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values to packed bf16, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Reductions across lane pairs that need no LDS.  permlane32_swap exchanges
// the two 32-lane halves of its operands and permlane16_swap the odd and even
// 16-lane rows; called with the same value for both operands, its two results
// hold a lane's own value and its partner's (lane ^ 32, respectively lane ^ 16),
// so a symmetric combination of the two is the pair's reduction in every lane.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copies from global memory straight into LDS, 16 (or 4) bytes per lane:
// from base + off (base wave-uniform, off a per-lane byte offset) to lds_base
// + 16 * lane (+ 4 * lane), lds_base wave-uniform.  Inline assembly, so that
// the compiler neither counts the copies among its outstanding loads nor makes
// LDS reads and barriers wait for them: kernels wait for their own copies
// (vmcnt) before the barrier that publishes them.
// Being inline assembly, the copies are also invisible to the compiler's
// hazard checks.  A vector instruction that writes an SGPR (v_readlane when an
// SGPR spill is reloaded, v_readfirstlane) needs 5 wait states before a vector
// memory instruction may read that SGPR as its address, and the compiler may
// place such a write right before a copy, which would then read a stale base.
// So every copy starts with its own s_nop 4.
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_copy4(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_base) : "memory");
}

// Workgroup barrier that orders LDS only: each wave's LDS accesses complete
// before it, nothing else.  __syncthreads() also waits for every global load
// the wave has in flight (its fence covers global memory), which would drain
// loads issued to stage later tiles through registers; the kernels here share
// data within a workgroup only through LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (vmcnt(n), n < 64: bits 3:0 and 15:14) and leaves the
// other counters unconstrained (expcnt 7, lgkmcnt 15).
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }

// Marks the end of one group of copies in the assembly (an assembler
// comment; no instruction).  A kernel that waits with vmcnt(N) for all but
// its last group of N copies relies on every group issuing exactly N copy
// instructions on every way through the code; the marker lets a CPU test
// of the compiled code count them per group.
__device__ __forceinline__ void copy_group_end() { asm volatile(";;#copy-group-end"); }

// A work item of the prefill-shaped kernels (forward, backward dQ).
struct WorkItem {
  int b, h, hk, qt;
};

// Dense layout: workgroup L of N over work items (batch, query head, query
// tile) with n_qtiles tiles per head, Hkv kv heads and `group` query heads
// per kv head.
//
// tile_major: the causal order below (also taken for a mask shared by all
// heads).
__device__ __forceinline__ WorkItem dense_work_item(int L, int N, int n_qtiles, int group, int Hkv, bool tile_major) {
  const bool causal = tile_major;
  // Causal, with the (batch, kv head) units splitting evenly over the 8
  // XCDs: XCD x serves units x U/8 .. (x+1) U/8 - 1, and on it the items go
  // query tile by query tile, heaviest first, across all of its units (the
  // group's query heads fastest).  Unit by unit, each unit's tiles heaviest
  // first, would leave the heavy tiles of the XCD's last units to run alone
  // at the end when an XCD holds many units of few tiles (at B=4, H=16,
  // n=2048: 8 units of 16 tiles, two thirds of the XCD busy on average).
  const int units = N / (n_qtiles * group);
  if (causal && (units & 7) == 0) {
    const int upx = units >> 3;  // units per XCD
    const int i = L >> 3;
    WorkItem it;
    const int hg = i % group;
    const int r = i / group;
    const int unit = (L & 7) * upx + r % upx;
    const int qi = r / upx;
    it.hk = unit % Hkv;
    it.b = unit / Hkv;
    it.h = it.hk * group + hg;
    it.qt = n_qtiles - 1 - qi;
    return it;
  }
  const int full = N & ~7;
  int w = L;
  if (L < full) w = (L & 7) * (full >> 3) + (L >> 3);
  WorkItem it;
  const int hg = w % group;
  int r = w / group;
  const int qi = r % n_qtiles;
  r /= n_qtiles;
  it.hk = r % Hkv;
  it.b = r / Hkv;
  it.h = it.hk * group + hg;
  it.qt = causal ? n_qtiles - 1 - qi : qi;
  return it;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero16() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

}  // namespace attn_dev
