/*
 * fa.h — C ABI of libfa.so: exact, fused scaled-dot-product attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is attention as the FlashAttention guide (cxbdf.cn, part 1)
 * defines it, O = softmax(Q·Kᵀ·scale)·V with the softmax taken along each
 * query row, optionally causal (the causal flag of flash_attn_func in the
 * Llama-Factory page's first code sample), computed tile by tile so that the
 * N×N score matrix never reaches device memory (cxbdf.cn guide, part 2:
 * tiling and kernel fusion). The forward also returns the per-row
 * log-sum-exp, the float "softmax_lse" output of the forward kernel in the
 * FlashAttention-2 全解析 page (blog.gitcode.com, core tiling sketch), which
 * the backward uses to recompute the probabilities instead of storing them
 * (cxbdf.cn guide, part 2, item 3: recomputation in the backward pass).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout: all tensors are dense, token-major and contiguous.
 *   q, o, dout, dq : [T, Hq,  d]   element type `dtype`
 *   k, v, dk, dv   : [T, Hkv, d]   element type `dtype`
 *   lse            : [Hq, T]       float32, natural log of the scaled logits
 * Fixed length (cu_seqlens == NULL): T = B·N, tokens ordered (batch, position),
 *   i.e. the (B, N, H, d) layout of flash_attn_func.
 * Variable length (cu_seqlens != NULL): B sequences packed without padding;
 *   cu_seqlens is int32 device memory with B+1 non-decreasing entries,
 *   cu_seqlens[0] = 0, sequence s = tokens [cu_seqlens[s], cu_seqlens[s+1]),
 *   T = cu_seqlens[B], and N must be ≥ the longest sequence (it sizes the
 *   grid). The caller guarantees this; it is not checked on the device.
 *   No token attends across a sequence boundary.
 * Heads: query head h reads KV head h / (Hq/Hkv) (grouped-query attention;
 *   Hq must be a multiple of Hkv).
 * Causal: key j is visible from query i iff j <= i, positions counted from
 *   the start of the sequence.
 * Supported: dtype FA_FP16 or FA_BF16; scale finite and > 0; head dim d = 64,
 *   128 or 256 for fa_fwd, fa_bwd and fa_fwd_kvcache (the pages' envelope
 *   reaches d = 256, Flash Attention 是什麼, adersaytech.com, section
 *   硬體與版本需求). At d = 256 the backward computes dK and dV in two passes
 *   (dV, then dK) so that each pass's accumulators fit the register file.
 *   The window, the soft cap and dropout reach d = 256 in both directions.
 *
 * Alignment: every tensor pointer must be 16-byte aligned (FA_ERR_INVALID_ARG
 *   otherwise); rows are moved as 16-byte vectors.
 * Ownership: every pointer is device memory owned by the caller. The library
 * allocates nothing and keeps no pointer after returning. Its global state
 * is a cache of the decode kernel's occupancy figures, filled on first use by
 * whichever thread gets there (the values are the same for every caller), and
 * the fixed device array that only fa_bwd_noalloc uses (see there); calls on
 * different streams may run concurrently. Outputs must not alias inputs.
 *
 * Errors: arguments are checked on the host before anything is enqueued; on
 * a negative status nothing was enqueued. FA_ERR_UNSUPPORTED marks a valid
 * request outside the supported envelope, so the caller can fall back to
 * another attention implementation. FA_OK means the work was enqueued on
 * `stream` (NULL = the default stream); device faults surface at the caller's
 * next synchronisation (with FA_DEBUG, before the call returns; see
 * fa_check_cu_seqlens). B = 0 or N = 0 is a no-op returning FA_OK.
 * A launching call clears the calling thread's pending HIP error
 * (hipGetLastError) first, so that FA_ERR_HIP reports its own launches only.
 *
 * Determinism: results are bitwise identical from run to run.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

/* The library is built with hidden symbols; what this header declares is its
 * whole exported interface. */
#pragma GCC visibility push(default)
#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,  /* null or misaligned pointer, negative size, bad enum,
                               Hq % Hkv != 0, bad scale */
  FA_ERR_UNSUPPORTED = -2,  /* head dim outside the supported set (see above) */
  FA_ERR_HIP = -3,          /* the HIP runtime refused a launch (e.g. no device) */
  FA_ERR_WORKSPACE = -4     /* workspace missing or smaller than the size function returns */
} fa_status;

typedef enum {
  FA_FP16 = 0,
  FA_BF16 = 1,
  FA_DTYPE_FORCE_INT = 0x7fffffff  /* not a dtype: keeps fa_dtype an int-sized type whose
                                      range covers any int, so a bad code is rejected
                                      (FA_ERR_INVALID_ARG) rather than undefined */
} fa_dtype;

/*
 * Forward: o = softmax(q·kᵀ·scale [causal])·v and lse = ln Σ_j exp(scale·q·k_j)
 * per (query head, token). o is rounded to `dtype` (nearest even), lse is
 * float32. B = batch size (number of sequences), N = sequence length (maximum
 * length for varlen), d = head dim.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal,
           const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream);

/*
 * Backward of fa_fwd for the upstream gradient `dout`, given the forward's
 * o and lse (the probabilities are recomputed from lse, never stored).
 * Writes dq [T, Hq, d], dk and dv [T, Hkv, d] in `dtype` (nearest even);
 * dk and dv of a KV head are summed over the query heads that share it.
 * `workspace` is caller-owned device memory of at least
 * fa_bwd_workspace_size(B, Hq, Hkv, N, d) bytes (float32 rowsum(dout∘o) and
 * the rescaled lse, 8·Hq·(B·N + 64) bytes rounded up to 256).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int N, int d, float scale, int causal,
           const int32_t* cu_seqlens, fa_dtype dtype,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd is a fixed sequence of stages enqueued on one stream:
 *   0  D = rowsum(dout∘o) and lse·log2(e) into the workspace
 *   1  dk, dv            (reads D)
 *   2  dq                (reads D; independent of stage 1)
 * fa_bwd_stage enqueues one stage with fa_bwd's arguments and checks, so a
 * caller can time the stages separately or run stages 1 and 2 on two streams
 * once stage 0 has completed. Running every stage in order equals fa_bwd.
 * A stage index outside [0, fa_bwd_num_stages()) is FA_ERR_INVALID_ARG.
 */
int fa_bwd_num_stages(void);
int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                 const int32_t* cu_seqlens, fa_dtype dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes fa_bwd needs; an upper bound that uses T <= B·N. 0 on bad sizes. */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): fa_bwd with the same arguments and results, minus the
 * workspace. The workspace lives in a fixed device array inside the library,
 * FA_NOALLOC_SCRATCH_BYTES large, one per GPU, held from the library's first
 * use on that GPU until the process ends; its address is looked up once per
 * device on the first call there. The call itself allocates nothing.
 *   Limit: fa_bwd_workspace_size(B, Hq, Hkv, N, d) <= FA_NOALLOC_SCRATCH_BYTES,
 *          i.e. Hq·(B·N + 64) <= 4,194,304; larger sizes return
 *          FA_ERR_WORKSPACE before anything is enqueued (use fa_bwd then).
 *   Concurrency: every call on one GPU shares that GPU's array, so calls
 *          that overlap on one GPU (different streams, or threads without
 *          ordering) race and may give wrong results; calls ordered on one
 *          stream are safe. The array keeps the last call's contents; each
 *          call writes every byte it reads.
 *   FA_ERR_HIP if the array's device address cannot be obtained (no device).
 * Other checks, errors and determinism as fa_bwd (bitwise equal to it).
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream);

/*
 * Sliding-window (band) attention: the forward and backward above with the
 * causal flag replaced by a window. Query i of a sequence sees the keys
 * j of the same sequence with i − window_left <= j <= i + window_right
 * (positions local to the sequence); −1 leaves that side unbounded. This is
 * the band mask the mlqm.cn evaluation page (Flash Attention 落地评估,
 * section 四, mask types) lists among the masks of standard attention.
 *   (−1, −1) is fa_fwd / fa_bwd without a mask, (−1, 0) is causal (both run
 *   the same kernels as those calls); any other pair runs the window kernels.
 * Every query sees at least its own position, so no row is empty.
 * Arguments, layouts, ownership, workspace and errors as for fa_fwd and
 * fa_bwd; a bound below −1 is FA_ERR_INVALID_ARG, and a window other than the
 * two pairs above needs N < 2^30 (else FA_ERR_UNSUPPORTED). The backward needs
 * the lse of fa_fwd_window with the same window. fa_bwd_window_stage runs one
 * stage (or every stage with stage −1), as fa_bwd_stage does.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int N, int d, float scale,
                  int window_left, int window_right,
                  const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream);
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  int B, int Hq, int Hkv, int N, int d, float scale,
                  int window_left, int window_right,
                  const int32_t* cu_seqlens, fa_dtype dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_window_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int Hq, int Hkv, int N, int d, float scale,
                        int window_left, int window_right,
                        const int32_t* cu_seqlens, fa_dtype dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Soft-capped logits: the forward and backward of fa_fwd / fa_bwd with every
 * logit replaced by softcap·tanh(scale·q·k / softcap) before the softmax. The
 * FlashAttention-2 page (blog.gitcode.com, section 2.3, adaptive soft cap)
 * adds a soft-cap step; the formula printed there is neither bounded nor
 * continuous at the cap, so the bounded tanh form is the reading taken. The
 * backward applies the chain rule through it (dS is multiplied by 1 − tanh²).
 *   softcap : 0 = no cap (the plain kernels run, bit-identical results);
 *             otherwise finite and > 0, with scale / softcap finite
 *             (else FA_ERR_INVALID_ARG)
 * Causal or not, fixed length or varlen, GQA; d = 64, 128 or 256 (the head
 * dimension of the soft-capped models). lse is the log-sum-exp of the capped logits; the
 * backward needs the lse of fa_fwd_softcap with the same cap. Everything else
 * (layouts, ownership, workspace, errors, determinism) as for fa_fwd / fa_bwd;
 * fa_bwd_softcap_stage runs one stage (or every stage with stage −1).
 */
int fa_fwd_softcap(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal, float softcap,
                   const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream);
int fa_bwd_softcap(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal, float softcap,
                   const int32_t* cu_seqlens, fa_dtype dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_softcap_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                         float softcap, const int32_t* cu_seqlens, fa_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * A sliding window and a soft cap together (the local-attention layers of
 * soft-capped models): fa_fwd_window / fa_bwd_window with every visible logit
 * replaced by softcap·tanh(scale·q·k / softcap), as fa_fwd_softcap does.
 * Arguments as fa_fwd_window / fa_bwd_window(_stage) plus `softcap` after
 * window_right; the checks of both apply (softcap = 0 runs the window kernels).
 * d = 64, 128 or 256.
 */
int fa_fwd_window_softcap(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, float scale, int window_left,
                          int window_right, float softcap, const int32_t* cu_seqlens, fa_dtype dtype,
                          hipStream_t stream);
int fa_bwd_window_softcap(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int N, int d, float scale, int window_left,
                          int window_right, float softcap, const int32_t* cu_seqlens, fa_dtype dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_window_softcap_stage(int stage, const void* q, const void* k, const void* v,
                                const void* o, const void* dout, const float* lse, void* dq,
                                void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                                float scale, int window_left, int window_right, float softcap,
                                const int32_t* cu_seqlens, fa_dtype dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);


/*
 * Dropout on the softmax weights: the forward and backward of fa_fwd / fa_bwd
 * with O = (P ∘ Z) V, where Z is 256/t for a kept weight and 0 for a dropped
 * one. The FlashAttention-2 page (blog.gitcode.com, API example) shows a
 * dropout_p argument but no random-number semantics; the reading taken:
 *   t = floor(256·(1 − dropout_p) + 1/2), keep probability t/256 (1 <= t <= 256);
 *   keep decisions from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC '11),
 *   one generator call per 4 x 4 block of (query i, key j) of one query head
 *   and sequence (positions local to the sequence): counter
 *   (j/4, i/4, head, sequence), key (seed mod 2^32, seed / 2^32); word i % 4,
 *   byte j % 4 of the output is the element's byte, kept iff byte < t.
 * The LSE is that of the undropped logits. The backward needs the same seed
 * and dropout_p (it regenerates the decisions; nothing is stored).
 *   dropout_p : 0 = none (the plain kernels run, bit-identical results);
 *               otherwise 0 < dropout_p < 1 with t >= 1 (else FA_ERR_INVALID_ARG)
 * Causal or not, fixed length or varlen, GQA; d = 64, 128 or 256. Everything
 * else as for fa_fwd / fa_bwd;
 * fa_bwd_dropout_stage runs one stage (or every stage with stage −1).
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   float dropout_p, uint64_t seed,
                   const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                   float dropout_p, uint64_t seed, const int32_t* cu_seqlens, fa_dtype dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_dropout_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                         float dropout_p, uint64_t seed, const int32_t* cu_seqlens, fa_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One forward and one backward for every mask and extra above, chosen by an
 * options struct instead of by entry point, so that a caller (or a new
 * combination) needs no further pair of symbols. Each call checks the options
 * and then runs exactly the entry point named below, with the same arguments,
 * checks, results (bit for bit), workspace and errors:
 *   mask FA_MASK_NONE / FA_MASK_CAUSAL, no extras ........ fa_fwd / fa_bwd
 *   FA_MASK_WINDOW (window_left, window_right as for
 *     fa_fwd_window) ...................................... fa_fwd_window / fa_bwd_window
 *   softcap > 0, mask NONE or CAUSAL ..................... fa_fwd_softcap / fa_bwd_softcap
 *   softcap > 0 with FA_MASK_WINDOW ...................... fa_fwd_window_softcap / ...
 *   dropout_p > 0, mask NONE or CAUSAL, no soft cap ...... fa_fwd_dropout / fa_bwd_dropout
 *   dropout with a window or a soft cap: FA_ERR_UNSUPPORTED (no kernel has both)
 * opts must point to host memory holding an fa_attn_options whose struct_size
 * is at least sizeof(fa_attn_options) (the struct may grow at its end); a NULL
 * opts, a smaller struct_size or another mask is FA_ERR_INVALID_ARG. The
 * window fields are read only with FA_MASK_WINDOW, dropout_seed only with
 * dropout_p > 0. Nothing in *opts is kept after the call.
 */
typedef enum {
  FA_MASK_NONE = 0,
  FA_MASK_CAUSAL = 1,
  FA_MASK_WINDOW = 2,
  FA_MASK_FORCE_INT = 0x7fffffff   /* not a mask: keeps fa_mask int-sized */
} fa_mask;

typedef struct {
  size_t struct_size;      /* sizeof(fa_attn_options) */
  fa_mask mask;
  int window_left;         /* FA_MASK_WINDOW: as fa_fwd_window's (-1 = unbounded) */
  int window_right;
  float softcap;           /* 0 = none; else as fa_fwd_softcap's */
  float dropout_p;         /* 0 = none; else as fa_fwd_dropout's */
  uint64_t dropout_seed;
} fa_attn_options;

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int N, int d, float scale,
              const fa_attn_options* opts, const int32_t* cu_seqlens, fa_dtype dtype,
              hipStream_t stream);
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* dk, void* dv,
              int B, int Hq, int Hkv, int N, int d, float scale,
              const fa_attn_options* opts, const int32_t* cu_seqlens, fa_dtype dtype,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward with queries and keys of different lengths (chunked prefill: a block
 * of new tokens attending to the cached ones and to itself). The tiling sketch
 * of the FlashAttention-2 全解析 page (blog.gitcode.com, section 2.1) takes
 * seqlen_q and seqlen_k as separate arguments.
 *   fixed length (both cu_seqlens NULL): q, o [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d];
 *     lse [Hq, B·Nq]
 *   varlen (both non-NULL, int32 device arrays of B+1 entries): q, o [Tq, Hq, d]
 *     with cu_seqlens_q, k, v [Tk, Hkv, d] with cu_seqlens_k; lse [Hq, Tq];
 *     Nq bounds every query length (it sizes the grid) and Nk every key length
 *   one NULL and one non-NULL cu_seqlens: FA_ERR_INVALID_ARG
 * The Lq queries of a sequence with Lk keys are its last Lq positions: query i
 * sits at position i + Lk − Lq and, when causal, sees keys j <= i + Lk − Lq
 * (the alignment fa_fwd_kvcache uses; with Lq = Lk it is fa_fwd's causal mask).
 * A query that sees no key (causal with Lq > Lk, or Lk = 0) gets O = 0 and
 * LSE = −inf. d in {64, 128, 256}; mask none or causal; no window, soft cap or
 * dropout. k and v may be NULL when Nk = 0. Other conventions as fa_fwd.
 */
int fa_fwd_kvlen(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, fa_dtype dtype,
                 hipStream_t stream);

/*
 * Backward of fa_fwd_kvlen: queries and keys of different lengths, for
 * training on a chunk of new tokens over a longer context. The layouts,
 * lengths, placement of the queries (the last Lq of a sequence's Lk positions,
 * bottom-right causal alignment) and cu_seqlens conventions are those of
 * fa_fwd_kvlen; o and lse are its outputs. The tiling sketch of the
 * FlashAttention-2 全解析 page (blog.gitcode.com, section 2.1) takes seqlen_q and
 * seqlen_k separately; the backward recomputes the probabilities from lse
 * (cxbdf.cn guide, part 2, item 3).
 *   dq [.., Hq, d] like q; dk, dv [.., Hkv, d] like k, v (summed over the
 *   query heads that share a KV head)
 * A query that sees no key (lse = −inf) gets dq = 0 and adds nothing to dk,
 * dv; a key no query sees gets dk = dv = 0 (with Nq = 0 every dk, dv is 0).
 * Supported: d = 64 or 128 (else FA_ERR_UNSUPPORTED); causal 0 or 1.
 * workspace: at least fa_bwd_workspace_size(B, Hq, Hkv, Nq, d) bytes.
 * Other checks, errors and determinism as fa_bwd; fa_bwd_kvlen_stage runs one
 * stage (0 D, 1 dk/dv, 2 dq) as fa_bwd_stage does.
 */
int fa_bwd_kvlen(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, fa_dtype dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_bwd_kvlen_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, fa_dtype dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 forward: the forward of fa_fwd on e4m3 inputs. The pages name e4m3
 * (torch.float8_e4m3fn) as the 8-bit attention format and credit
 * FlashAttention-3 with an FP8 forward (FlashAttention-2 全解析, blog.gitcode.com,
 * section 4.3; Flash Attention 是什麼, adersaytech.com, FA-1 to FA-4 table and note).
 *   q : [T, Hq, d]   e4m3fn codes (OCP E4M3, finite-only: bias 7, max 448)
 *   k : [T, Hkv, d]  e4m3fn codes
 *   v : [T, Hkv, d]  e4m3fn codes
 *   descale_q, descale_k, descale_v : per-tensor factors, finite and > 0;
 *       the real inputs are code value × descale
 *   o   : [T, Hq, d] out_dtype (FA_FP16 or FA_BF16), nearest even
 *   lse : [Hq, T]    float32, natural log, of scale·(real Q)·(real K)ᵀ
 * The kernel rounds the softmax weights to e4m3 for the P·V product (the
 * matrix instruction takes 8-bit operands) and normalises O by the sum of
 * those rounded weights; LSE uses the unrounded weights. d = 64, 128 or 256,
 * as for fa_fwd (other d: FA_ERR_UNSUPPORTED). Layout, varlen, causal,
 * alignment, ownership, errors and determinism as for fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal,
               const int32_t* cu_seqlens, float descale_q, float descale_k, float descale_v,
               fa_dtype out_dtype, hipStream_t stream);

/*
 * Decode: attention of Nq new queries per batch entry over a key/value cache
 * (the inference use of the method: long-context inference and inference
 * tools, Flash Attention 是什麼, adersaytech.com, sections 原理拆解 and
 * 各推論工具怎麼開).
 *   q       : [B, Nq, Hq, d]   the new queries, `dtype`
 *   k_cache : [B, Nk, Hkv, d]  cache capacity Nk per entry, `dtype`
 *   v_cache : [B, Nk, Hkv, d]
 *   cache_seqlens : int32 device [B], valid positions L_b of entry b
 *                   (0 <= L_b <= Nk; values outside are clamped into range)
 *   o       : [B, Nq, Hq, d]   `dtype` (nearest even)
 *   lse     : [Hq, B·Nq]       float32, column b·Nq + i for query i of entry b
 * The queries are the newest Nq positions of each sequence: query i of entry
 * b sits at position L_b − Nq + i and, when causal, sees the cached keys at
 * or before that position; otherwise it sees all L_b keys. A query that sees
 * no key gets o = 0 and lse = −inf.
 * The cache is split along the keys into `num_splits` ranges per (entry, KV
 * head) processed in parallel and merged exactly by their log-sum-exp;
 * num_splits = 0 picks fa_kvcache_num_splits(...). `workspace` holds the
 * per-split partial results: at least fa_fwd_kvcache_workspace_size(...)
 * bytes for the same sizes and num_splits.
 * Conventions (alignment, ownership, errors, determinism) as above; B = 0 or
 * Nq = 0 is a no-op.
 */
int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* cache_seqlens, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int num_splits, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * fa_fwd_kvcache is two stages on one stream: 0 computes the per-range
 * partial results into the workspace, 1 merges them into o and lse.
 * fa_fwd_kvcache_stage enqueues one of them with fa_fwd_kvcache's arguments
 * and checks (stage 1 reads what stage 0 wrote for the same arguments), so
 * a caller can time them separately. A stage index outside
 * [0, fa_fwd_kvcache_num_stages()) is FA_ERR_INVALID_ARG.
 */
int fa_fwd_kvcache_num_stages(void);
int fa_fwd_kvcache_stage(int stage, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cache_seqlens, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         int num_splits, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Decode with a sliding window and/or a soft cap (the local layers and capped
 * logits of models such as Gemma-2; window: the sliding-window mask named on
 * the mlqm.cn evaluation page, section 四; cap: the FlashAttention-2 page,
 * blog.gitcode.com, section 2.3, bounded reading):
 * fa_fwd_kvcache with
 *   window_left : −1 = none; otherwise query i of entry b (at position
 *                 p = L_b − Nq + i) sees only keys j >= p − window_left (with
 *                 causal also j <= p); < −1 is FA_ERR_INVALID_ARG
 *   softcap     : 0 = none; otherwise logits softcap·tanh(scale·q·k / softcap),
 *                 finite and > 0 with scale / softcap finite (else INVALID_ARG)
 * The key ranges split only the last Nq + window_left positions of each entry,
 * which are all any of its queries can see. 16-bit caches only; the workspace
 * is that of fa_fwd_kvcache (fa_fwd_kvcache_workspace_size suffices with
 * num_splits = 0). Other conventions as fa_fwd_kvcache.
 */
int fa_fwd_kvcache_local(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cache_seqlens, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         int window_left, float softcap, int num_splits, fa_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode over an FP8 key/value cache: fa_fwd_kvcache with k_cache and v_cache
 * holding e4m3fn codes (1 byte each, same [B, Nk, Hkv, d] layout) and
 * per-tensor descales (cached value = code value × descale). This is the FP8
 * KV cache the FlashAttention-2 全解析 page (blog.gitcode.com, section 4.3,
 * kv_cache_dtype = float8_e4m3fn) offers for long sequences that run out of
 * memory; it halves the cache bytes each call reads.
 *   q, o     : `dtype` (FA_FP16 or FA_BF16), as in fa_fwd_kvcache
 *   descale_k, descale_v : finite and > 0, else FA_ERR_INVALID_ARG
 * The result is that of fa_fwd_kvcache on the decoded cache (every e4m3 value
 * is exact in both 16-bit types): scores scale·descale_k·q·k_code, and O
 * multiplied by descale_v. Codes 0x7f and 0xff (NaN) make the rows that see
 * them NaN. Workspace, num_splits, stages and every other convention as for
 * fa_fwd_kvcache (same workspace size function). num_splits = 0 picks
 * fa_kvcache_fp8_num_splits(...) ranges.
 */
int fa_fwd_kvcache_fp8(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cache_seqlens, void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       float descale_k, float descale_v, int num_splits, fa_dtype dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);
int fa_fwd_kvcache_fp8_stage(int stage, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cache_seqlens, void* o, float* lse,
                             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                             int causal, float descale_k, float descale_v, int num_splits,
                             fa_dtype dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* The key-range count fa_fwd_kvcache uses for num_splits = 0 (>= 1); 0 on bad sizes.
 * It is the largest count whose workgroups are all resident on the current device
 * at once (from the runtime's occupancy figure for the decode kernel; a fixed
 * per-CU bound for a 256-CU part when no device is present), at least 256 keys
 * (eight 32-key tiles) per range and at most 256 ranges. */
int fa_kvcache_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d);
/* The count fa_fwd_kvcache_fp8 uses for num_splits = 0: its workgroups need half
 * the LDS, so more are resident, and at d <= 128 the count is the one that fills
 * half of them, rounded up (measured fastest on every shape tried; at d = 256 the
 * full round measured fastest); the same range bounds apply. */
int fa_kvcache_fp8_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/* Workspace bytes for fa_fwd_kvcache and fa_fwd_kvcache_fp8: (d + 1)·4 bytes per
 * (split, entry, query head, query), rounded up to 256; num_splits = 0 means the
 * larger of the two automatic counts. 0 on bad sizes. */
size_t fa_fwd_kvcache_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                     int num_splits);

/* Static, NUL-terminated text for a status code. */
const char* fa_status_string(int status);

/*
 * Host check of a cu_seqlens array: the packed variable-length batch that
 * takes the place of a padding mask (the Variable length convention above).
 * cu_seqlens_host is HOST memory holding a copy of the device array an entry
 * point would take; exactly its B+1 entries are read. It holds when
 * cu_seqlens_host[0] = 0 and every length cu_seqlens_host[s+1] −
 * cu_seqlens_host[s] lies in [0, N] (so the entries are non-decreasing and
 * the last is at most B·N). Returns FA_OK, or FA_ERR_INVALID_ARG for a NULL
 * pointer, B < 0, N < 0 or a violated condition. Nothing else is touched.
 *
 * Builds with FA_DEBUG defined (build.py --debug: libfa_debug.so) run this
 * check on a copy of every cu_seqlens argument (cu_seqlens_q against Nq and
 * cu_seqlens_k against Nk for the kvlen entry points) before launching, and
 * synchronise the stream after every launch, reporting a failed copy, launch
 * or kernel as FA_ERR_HIP. Those synchronisations make a debug build unfit
 * for graph capture. Release builds never read cu_seqlens on the host.
 */
int fa_check_cu_seqlens(const int32_t* cu_seqlens_host, int B, int N);

#ifdef __cplusplus
}
#endif
#pragma GCC visibility pop

#endif /* FA_H_ */
