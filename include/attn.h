/*
 * attn.h - fused scaled dot-product attention forward for AMD Instinct MI355X
 * (gfx950): prefill and single-token decode against a KV cache.
 *
 * What is computed (per batch b and query head h, with key/value head
 * hk = h / (Hq / Hkv)):
 *
 *     S   = Q[b,h] K[b,hk]^T * scale           scores, one row per query
 *     S[i,j] = -inf where j > i                 only when causal (top-left)
 *     P   = softmax(S) along the key axis       after subtracting the row max
 *     O   = P V[b,hk]
 *     LSE = m + ln(l) per row                   m = row max, l = sum exp(S - m)
 *
 * This is the attention of "Flash Attention原理：分块计算与重计算" (cnblogs),
 * section 一 (shapes (batch, num_heads, seq_len, head_dim), P = softmax(S /
 * sqrt(d)) over keys, O = P V, default scale head_dim^-1/2), with the step
 * order Q K^T, scale, causal mask, softmax, times V of "PyTorch Profiler 實戰：
 * 五種 Attention 實現的 GPU 核心剖析" ("核心概念").  The library computes it
 * tile by tile with the online softmax of the cnblogs page's section 四, so
 * S and P never reach device memory; only O and the per-row statistics (the
 * m and l of its section 五, returned as one log-sum-exp) are written.
 * Grouped-query heads (several query heads sharing one key/value head) follow
 * "SDPA backend 与 FlashAttention", sections 11-12.  Decode (one query token
 * against the cached keys and values, the inference case of the cnblogs FAQ
 * Q12-Q13 and "SDPA backend 与 FlashAttention" section 5) splits each
 * sequence's keys into chunks and merges the partial results with the same
 * section 四 rescaling identity applied to (O, LSE) pairs.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates no device memory; between calls it keeps only
 *     memoised device queries, attn_decode_noalloc's static scratch and,
 *     per device, the stream and two events attn_bwd forks onto (see
 *     there).  The entry points are thread-safe.
 *   - Sizes and strides are int64 element counts.  The innermost (head_dim)
 *     stride is 1 for every tensor.  Every base pointer must be 16-byte
 *     aligned and every non-innermost stride a multiple of 16 bytes (8 bf16
 *     or 4 fp32 elements), so that each row starts on a 16-byte boundary.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued and the call returns; the status reports argument
 *     validation and kernel launch only (an execution fault surfaces at the
 *     caller's next synchronisation).
 *   - Invalid or unsupported arguments are rejected with an error status
 *     before anything is enqueued.  Nothing falls back to another method.
 *   - Outputs must not overlap inputs.  Inputs are assumed finite.
 *   - Arithmetic: bf16 inputs are multiplied on bf16 matrix cores with fp32
 *     accumulation; the softmax runs in fp32; probabilities are rounded to
 *     bf16 (round-to-nearest-even) before the P V product; O is rounded to
 *     the input dtype (round-to-nearest-even).  fp32 inputs stay in fp32
 *     throughout.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_BF16 = 0, /* bfloat16 Q/K/V/O */
  ATTN_F32 = 1   /* float32 Q/K/V/O */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* negative size, Hkv == 0 with work to do, Hq % Hkv != 0,
                               max_seqlen_q > total_q, non-finite scale */
  ATTN_ERR_DTYPE = 3,       /* dtype not one of attn_dtype_t */
  ATTN_ERR_LAYOUT = 4,      /* misaligned base pointer, stride not a multiple of
                               16 bytes, or negative stride */
  ATTN_ERR_UNSUPPORTED = 5, /* valid arguments with no kernel (head_dim, dtype or
                               group size outside the supported set, sizes past
                               the documented limits) */
  ATTN_ERR_WORKSPACE = 6,   /* decode workspace NULL or smaller than required */
  ATTN_ERR_HIP = 7,         /* the HIP runtime refused the launch */
  ATTN_ERR_SCRATCH = 8      /* attn_decode_noalloc: the sizes need more workspace than
                               its static scratch (ATTN_DECODE_NOALLOC_SCRATCH_BYTES) */
} attn_status_t;

/* Size of the static device array attn_decode_noalloc uses as its workspace
 * (32 MiB per device): enough for attn_decode_workspace_bytes of (for example
 * B = 64, Hq = 32, d = 128 up to Lmax = 15360). */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Prefill: every query row attends to the keys of its (batch, kv head). */
typedef struct {
  const void *q;   /* [B, Hq,  Lq, d] */
  const void *k;   /* [B, Hkv, Lk, d] */
  const void *v;   /* [B, Hkv, Lk, d] */
  void *o;         /* [B, Hq,  Lq, d], same dtype as q */
  float *lse;      /* [B, Hq, Lq] fp32, contiguous; natural-log log-sum-exp of
                      the scaled (and masked) score row */
  int64_t B, Hq, Hkv, Lq, Lk, d;
  int64_t q_strides[3]; /* element strides of (batch, head, token); d stride is 1 */
  int64_t k_strides[3];
  int64_t v_strides[3];
  int64_t o_strides[3];
  int32_t dtype;   /* attn_dtype_t */
  int32_t causal;  /* nonzero: query i sees keys j <= i (top-left, any Lq and Lk) */
  float scale;     /* multiplier of Q K^T; 0 selects 1/sqrt(d) */
} attn_fwd_args_t;

/* Attention mask for attn_fwd_masked ("Flash Attention原理：分块计算与重计算"
 * (cnblogs), FAQ Q11: any boolean mask, applied inside the kernel; the
 * semantics of scaled_dot_product_attention's attn_mask). */
typedef enum {
  ATTN_MASK_BOOL = 1,      /* uint8: nonzero = the (query, key) pair takes part */
  ATTN_MASK_ADD_BF16 = 2   /* bf16, added to the scaled score before the softmax */
} attn_mask_kind_t;

typedef struct {
  const void *data;     /* [B, Hq, Lq, Lk] logical shape, key-contiguous */
  int32_t kind;         /* attn_mask_kind_t */
  int32_t reserved;     /* 0 */
  int64_t strides[3];   /* element strides of (batch, head, query); 0 broadcasts */
} attn_mask_t;

/* Packed variable-length prefill ("Flash Attention原理：分块计算与重计算"
 * (cnblogs), FAQ Q10: several sequences of different lengths packed into one
 * batch through cumulative sequence offsets, no padding; FAQ Q15: queries and
 * keys/values of different lengths, as in cross-attention).  Sequence b owns
 * query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key/value rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1; it attends only to its own keys. */
typedef struct {
  const void *q;   /* [total_q, Hq,  d] */
  const void *k;   /* [total_k, Hkv, d] */
  const void *v;   /* [total_k, Hkv, d] */
  void *o;         /* [total_q, Hq,  d], same dtype as q */
  float *lse;      /* [Hq, total_q] fp32, contiguous */
  const int32_t *cu_seqlens_q;  /* device, B + 1 entries: 0, ..., total_q, non-decreasing */
  const int32_t *cu_seqlens_k;  /* device, B + 1 entries: 0, ..., total_k, non-decreasing */
  int64_t B, Hq, Hkv, total_q, total_k;
  int64_t max_seqlen_q;  /* >= every query length (host-side: sizes the grid) */
  int64_t d;
  int64_t q_strides[2];  /* element strides of (token, head); d stride is 1 */
  int64_t k_strides[2];
  int64_t v_strides[2];
  int64_t o_strides[2];
  int32_t dtype;   /* attn_dtype_t; ATTN_BF16 */
  int32_t causal;  /* nonzero: within each sequence, query i sees keys j <= i */
  float scale;     /* multiplier of Q K^T; 0 selects 1/sqrt(d) */
} attn_fwd_varlen_args_t;

/* Backward of the prefill ("Flash Attention原理：分块计算与重计算" (cnblogs),
 * section 五: the probabilities are recomputed from the stored log-sum-exp). */
typedef struct {
  const void *q;     /* [B, Hq,  Lq, d]  the forward's inputs ... */
  const void *k;     /* [B, Hkv, Lk, d] */
  const void *v;     /* [B, Hkv, Lk, d] */
  const void *o;     /* [B, Hq,  Lq, d]  ... its output O ... */
  const void *dout;  /* [B, Hq,  Lq, d]  ... and the gradient of the loss with respect to O */
  const float *lse;  /* [B, Hq, Lq] fp32 contiguous, as attn_fwd returned it */
  void *dq;          /* [B, Hq,  Lq, d]  outputs, same dtype as q */
  void *dk;          /* [B, Hkv, Lk, d]  a grouped kv head gets the sum over its query heads */
  void *dv;          /* [B, Hkv, Lk, d] */
  int64_t B, Hq, Hkv, Lq, Lk, d;
  int64_t q_strides[3];  /* element strides of (batch, head, token); d stride is 1 */
  int64_t k_strides[3];
  int64_t v_strides[3];
  int64_t o_strides[3];
  int64_t do_strides[3];
  int64_t dq_strides[3];
  int64_t dk_strides[3];
  int64_t dv_strides[3];
  int32_t dtype;   /* attn_dtype_t; ATTN_BF16 */
  int32_t causal;  /* as in the forward (top-left) */
  float scale;     /* as in the forward; 0 selects 1/sqrt(d) */
} attn_bwd_args_t;

/* FP8 prefill ("Flash Attention原理：分块计算与重计算" (cnblogs), section 六
 * and FAQ Q8: the products run on 8-bit floating-point matrix units).  Q, K
 * and V are e4m3 codes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, largest value 448, no infinity; S.1111.111 is NaN), one
 * byte each; every tensor carries one fp32 descale and an element stands for
 * descale * value(code).  Scores are scale * q_descale * k_descale * (codes
 * product); O is written in bf16. */
typedef struct {
  const void *q;   /* [B, Hq,  Lq, d] e4m3 codes */
  const void *k;   /* [B, Hkv, Lk, d] e4m3 codes */
  const void *v;   /* [B, Hkv, Lk, d] e4m3 codes */
  void *o;         /* [B, Hq,  Lq, d] bf16 */
  float *lse;      /* [B, Hq, Lq] fp32, contiguous */
  int64_t B, Hq, Hkv, Lq, Lk, d;
  int64_t q_strides[3];  /* element (= byte) strides of (batch, head, token), multiples of 16 */
  int64_t k_strides[3];
  int64_t v_strides[3];
  int64_t o_strides[3];  /* bf16 element strides, multiples of 8 */
  float q_descale, k_descale, v_descale;  /* finite */
  int32_t causal;  /* nonzero: query i sees keys j <= i (top-left, any Lq and Lk) */
  float scale;     /* multiplier of Q K^T; 0 selects 1/sqrt(d) */
} attn_fwd_fp8_args_t;

/* Decode: one query token per sequence against a ragged KV cache. */
typedef struct {
  const void *q;          /* [B, Hq, d] */
  const void *k_cache;    /* [B, Hkv, Lmax, d]; slots >= seqlens[b] are never read */
  const void *v_cache;    /* [B, Hkv, Lmax, d] */
  const int32_t *seqlens; /* device int32 [B]; sequence b sees slots 0..seqlens[b]-1.
                             Values are clamped to [0, Lmax]; a sequence of length
                             0 yields O = 0 and LSE = -inf. */
  void *o;                /* [B, Hq, d], same dtype as q */
  float *lse;             /* [B, Hq] fp32, contiguous */
  int64_t B, Hq, Hkv, Lmax, d;
  int64_t q_strides[2];   /* (batch, head) */
  int64_t k_strides[3];   /* (batch, head, token) */
  int64_t v_strides[3];
  int64_t o_strides[2];
  int32_t dtype;          /* attn_dtype_t; decode supports ATTN_BF16 */
  float scale;            /* 0 selects 1/sqrt(d) */
} attn_decode_args_t;

/*
 * attn_fwd - prefill attention forward, one kernel launch.
 * Supported: dtype bf16 or f32; d in {64, 80, 128}; Hq % Hkv == 0; Lq and
 * Lk independent (cross-attention), causal or not.  Limits
 * (ATTN_ERR_UNSUPPORTED past them): Lq, Lk and B * Hq below 2^31; bf16 K and
 * V token strides below 2^28 elements.  Any size may be 0: then nothing is
 * launched (rows that see no key -- Lk == 0 -- get O = 0 and LSE = -inf).
 * Returns ATTN_OK or the first error found; on error nothing is enqueued.
 */
attn_status_t attn_fwd(const attn_fwd_args_t *args, void *stream);

/*
 * attn_fwd_masked - attn_fwd with an attention mask, one kernel launch.  The
 * mask combines with causal (a pair takes part only if both allow it); a row
 * left without any key gets O = 0 and LSE = -inf.  Supported: dtype bf16;
 * d in {64, 80, 128}; the mask's data 16-byte aligned, its query stride a
 * multiple of 16 bytes and below 2^27 bytes, Lk a multiple of 16 (boolean)
 * or 8 (additive) keys.  The mask tile of every key tile is read from device
 * memory: a mask with its own values per head adds Lq x Lk elements per head
 * to the traffic (strides 0 share one mask between heads or batches).
 */
attn_status_t attn_fwd_masked(const attn_fwd_args_t *args, const attn_mask_t *mask, void *stream);

/*
 * attn_fwd_fp8 - prefill attention forward on FP8 inputs, one kernel launch.
 * Both products run on the e4m3 matrix cores with fp32 accumulation; the
 * softmax runs in fp32; each probability is rounded to e4m3 (nearest even)
 * before the P V product and the row normaliser sums the rounded values, so
 * O = v_descale * sum_j P~_j V_j / sum_j P~_j exactly up to accumulation,
 * rounded to bf16, and LSE = m + ln(sum_j P~_j).  Supported: d in {64, 128};
 * Hq % Hkv == 0; Lq and Lk independent, causal or not.  Limits as attn_fwd
 * (K and V token strides below 2^28 bytes).  B, Hq or Lq of 0 launches
 * nothing; Lk == 0 gives O = 0 and LSE = -inf.  A non-finite descale or scale, or a
 * score multiplier past the float range, is ATTN_ERR_SHAPE.
 */
attn_status_t attn_fwd_fp8(const attn_fwd_fp8_args_t *args, void *stream);

/*
 * attn_fwd_varlen - packed variable-length prefill, one kernel launch: the
 * same computation as attn_fwd applied to each sequence separately.
 * Supported: dtype bf16; d in {64, 80, 128}; Hq % Hkv == 0;
 * 0 <= max_seqlen_q <= total_q.  Limits as attn_fwd (total_q, total_k below
 * 2^31; K/V token strides below 2^28 elements).  The offsets live in device
 * memory and are not checked on the host: the caller guarantees the form
 * above and max_seqlen_q >= every query length (a longer sequence's rows
 * past max_seqlen_q, rounded up to the kernel's query tile, are not written).
 * Offsets outside [0, total] are
 * clamped on the device, so inconsistent offsets give wrong rows, never an
 * access outside the tensors.  Sequences with no keys get O = 0 and
 * LSE = -inf.  B == 0, Hq == 0 or max_seqlen_q == 0 is a no-op.
 */
attn_status_t attn_fwd_varlen(const attn_fwd_varlen_args_t *args, void *stream);

/*
 * attn_decode_workspace_bytes - bytes of device workspace attn_decode needs
 * for these sizes: fp32 partial outputs and log-sum-exps, for every query
 * head of every sequence, of the (Lmax - 1) / 512 + 2 pieces of the split
 * that one sequence's cache slots can span at most.  Returns 0 for invalid
 * sizes.
 */
size_t attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Lmax, int64_t d);

/*
 * attn_decode - split-KV decode: one kernel lays the cache slots of every
 * (sequence, kv head) end to end, cuts them into equal pieces (one per
 * workgroup, at least 512 slots each) and computes a partial (O, LSE) per
 * query head for each (sequence, kv head) a piece touches; a second kernel
 * merges the partials of each query head.  `workspace` is caller-owned device memory of at least
 * attn_decode_workspace_bytes(B, Hq, Lmax, d) bytes, 256-byte aligned; its
 * contents on entry do not matter and are overwritten.  Calls that share a
 * workspace must be ordered on one stream.
 * Supported: dtype bf16; d in {64, 80, 128}; Hq % Hkv == 0; B * Lmax < 2^31
 * (ATTN_ERR_UNSUPPORTED otherwise).  The query heads of
 * one kv head are served 16 at a time, so a group larger than 16 reads its
 * keys and values once per 16 query heads.  B == 0 or Hq == 0 is a no-op;
 * Lmax == 0 writes O = 0 and LSE = -inf.  Exactly two kernels are enqueued
 * (one when Lmax == 0).
 */
attn_status_t attn_decode(const attn_decode_args_t *args, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same two kernels and results, with the workspace
 * in a static device array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on, from the first call on that
 * device until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); the first call on a device looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.  The caller
 * still owns and passes every input and output.  Sizes whose
 * attn_decode_workspace_bytes exceed the array return ATTN_ERR_SCRATCH
 * before anything is enqueued.  All calls on one device share that device's
 * array and leave their partial results in it: calls that may overlap on one
 * device (different streams, different threads without ordering) race and
 * must be ordered by the caller, e.g. on one stream.  Errors as attn_decode;
 * ATTN_ERR_HIP if the array's address cannot be obtained.
 */
attn_status_t attn_decode_noalloc(const attn_decode_args_t *args, void *stream);

/*
 * attn_bwd_workspace_bytes - bytes of device workspace attn_bwd needs (two
 * fp32 per query row: LSE log2(e) and D = rowsum(dO * O)).  Returns 0 for
 * invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq);

/*
 * attn_bwd - gradients dQ, dK, dV of the prefill attention, recomputing the
 * probabilities from the stored LSE: dV = P^T dO, dP = dO V^T,
 * dS = P * (dP - rowsum(dO * O)), dQ = scale dS K, dK = scale dS^T Q.  Three
 * kernels are enqueued (row sums, dK/dV, dQ); nothing is accumulated with
 * atomics, so results are deterministic.  `workspace` is caller-owned device
 * memory of at least attn_bwd_workspace_bytes(B, Hq, Lq) bytes, 256-byte
 * aligned, contents irrelevant on entry.
 * Supported: dtype bf16; d in {64, 80, 128}; Hq % Hkv == 0; Lq and Lk
 * independent; causal or not; Q, dO, K and V token strides below 2^26 elements
 * (ATTN_ERR_UNSUPPORTED past it).  dK and dV of keys that no query sees are 0;
 * Lq == 0 gives dK = dV = 0.  B == 0, Hq == 0 or Lq == Lk == 0 is a no-op.
 * At d = 64 and 80 the dQ kernel runs on a second stream that the library
 * keeps per device, forked from `stream` after the row sums and joined back
 * into it (events, no host wait) before the call returns, so that it overlaps
 * the dK/dV kernel; all results are then ordered on `stream` as if every
 * kernel ran there.  Concurrent calls on one device take turns (a host lock)
 * for that sequence.  A call made while `stream` is being captured into a
 * graph, before the library has created its stream on the device, runs all
 * three kernels on `stream`.
 */
attn_status_t attn_bwd(const attn_bwd_args_t *args, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Argument checks only (no device work, no HIP call): the status attn_fwd /
 * attn_decode would return before launching.  Usable without a GPU. */
attn_status_t attn_validate_fwd(const attn_fwd_args_t *args);
attn_status_t attn_validate_fwd_masked(const attn_fwd_args_t *args, const attn_mask_t *mask);
attn_status_t attn_validate_fwd_varlen(const attn_fwd_varlen_args_t *args);
attn_status_t attn_validate_fwd_fp8(const attn_fwd_fp8_args_t *args);
attn_status_t attn_validate_bwd(const attn_bwd_args_t *args);
attn_status_t attn_validate_decode(const attn_decode_args_t *args);

/* Static, human-readable name of a status code.  The status codes are the
 * library's answer to the failure "SDPA backend 与 FlashAttention" warns of
 * in sections 3, 7 and 9: an input the fast kernel cannot take silently
 * runs on a slower path instead (there, head_dim 80 missing the alignment
 * the fused kernel needs).  Here such an input is refused with a code the
 * caller can read and print; no call ever falls back to other arithmetic.
 * Returns "unknown status" for a value outside attn_status_t. */
const char *attn_status_str(attn_status_t status);

/* Static name of the kernel attn_fwd would launch for these arguments, or
 * "none" if they are invalid or unsupported.  No device work.  This is the
 * check "SDPA backend 与 FlashAttention" section 11 asks for: record which
 * backend a call actually runs, so that a silent change of kernel shows up
 * in the logs. */
const char *attn_kernel_name(const attn_fwd_args_t *args);

/* Library version string. */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
