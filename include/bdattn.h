/*
 * bdattn — clean-plus-corrupted block-diffusion attention on one MI355X (gfx950).
 *
 * The operation is the attention of block-diffusion language-model training
 * described in "Block Parallelism for Efficient Distributed Long-Context
 * Diffusion Language Model Training":
 *
 *  - §3.2 (Block diffusion language models): a clean copy and a corrupted copy
 *    of the sequence, cut into blocks of B tokens. A clean query of block b sees
 *    the clean keys of blocks 0..b (its whole own block: block-causal), or,
 *    with clean_mask = BDATTN_CLEAN_TOKEN_CAUSAL, the clean keys of blocks < b
 *    and those of its own block up to its own position (the section's "causal
 *    access within block b" read token by token). A corrupted query of target
 *    block b sees its own block's corrupted keys (bidirectionally) and the
 *    clean keys of blocks < b, never another block's corrupted keys.
 *  - §4.3 (Context-sharded block parallelism): one rank holds a shard of clean
 *    queries, the clean K/V of the positions its queries need (gathered into
 *    one buffer in original position order), and a set of whole corrupted
 *    blocks. The problem descriptor below expresses exactly that share; the
 *    whole single-GPU problem is the share with one rank.
 *  - Appendix, "Efficient fused operator" (Implementations 1 and 2): the
 *    forward saves the output and the log-sum-exp; the backward reuses them
 *    and returns the query gradients together with the gradients of the local
 *    corrupted K/V and of the clean K/V buffer, the latter summed over every
 *    local query that sees each clean key (§4.3, Backward pass).
 *    Implementation 1 computes the attention as separate launches over
 *    disjoint key sets, the block-diagonal corrupted part and clean K/V given
 *    by original positions, merged through their log-sum-exps: a descriptor
 *    with partial = 1 is one such launch, and bdattn_merge combines them.
 *
 * Softmax attention per query row i and q head h (KV head g = h / (H/Hkv)):
 *   s_ij = scale <q_i, k_j>,  LSE_i = ln sum_{j visible} exp(s_ij),
 *   O_i = sum_j exp(s_ij - LSE_i) v_j.
 * Blocks are 0-indexed on global clean positions: block(p) = p / B.
 *
 * Layouts (all tensors contiguous, token-major, one dtype):
 *   Q, O, dO, dQ : [n, H, d]        K, V, dK, dV : [n, Hkv, d]
 *   LSE          : [H, n] float32, natural log, scale included.
 * Clean query tensors have n = n_clean_q; clean K/V tensors n = n_clean_kv;
 * corrupted tensors n = n_corr_blocks * B, blocks packed in increasing id order.
 *
 * Ownership and execution: every tensor pointer is a DEVICE pointer owned by
 * the caller. bdattn_fwd / bdattn_bwd enqueue work on `hip_stream` (a
 * hipStream_t; NULL = the default stream) and return without waiting; they
 * never allocate device memory. No result is accumulated with atomics (the
 * only atomics are integer counters that hand work items to workgroups, and
 * an item computes the same values whichever workgroup runs it): results are
 * bitwise reproducible for a given problem and inputs. Scratch space is the caller's `workspace`
 * (device memory of at least bdattn_workspace_size bytes, 256-byte aligned),
 * which must not be used by anything else until the enqueued work is done.
 * Outputs are overwritten, never accumulated into. Tensor pointers must be
 * 16-byte aligned. Calls on different streams may run concurrently if they
 * use distinct workspaces and outputs.
 *
 * Errors: every function returns a bdattn_status. Arguments are validated on
 * the host before any GPU work; on failure nothing is enqueued. After the
 * launches a HIP launch error is reported as BDATTN_ERR_HIP. Nothing aborts or
 * throws across this interface. bdattn_last_error() gives a message for the
 * most recent failure on the calling thread.
 */
#ifndef BDATTN_H
#define BDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BDATTN_VERSION 5

typedef enum {
  BDATTN_OK = 0,
  BDATTN_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad enum, bad ids */
  BDATTN_ERR_SHAPE = -2,       /* sizes not multiples of B, H % Hkv != 0, ... */
  BDATTN_ERR_UNSUPPORTED = -3, /* head dim or dtype this build has no kernel for */
  BDATTN_ERR_COVERAGE = -4,    /* clean K/V buffer misses keys a local query sees */
  BDATTN_ERR_WORKSPACE = -5,   /* workspace missing, too small or misaligned */
  BDATTN_ERR_HIP = -6          /* a HIP runtime call or kernel launch failed */
} bdattn_status;

typedef enum { BDATTN_F32 = 0, BDATTN_BF16 = 1 } bdattn_dtype;
/* Output precision of a bf16 problem (bdattn_problem.precision). */
typedef enum {
  BDATTN_PRECISION_DEFAULT = 0,
  BDATTN_PRECISION_F32_OUT = 1,
  BDATTN_PRECISION_SPLIT = 2
} bdattn_precision;

/* What a clean query sees of its own clean block (§3.2): all of it, or the
 * keys at positions up to its own. Corrupted queries are not affected. */
typedef enum {
  BDATTN_CLEAN_BLOCK_CAUSAL = 0, /* clean keys of blocks <= own block */
  BDATTN_CLEAN_TOKEN_CAUSAL = 1  /* clean keys at positions <= own position */
} bdattn_clean_mask;

/* One rank's share of the block-diffusion attention (§4.3), or the whole
 * problem on one GPU. */
typedef struct {
  int32_t B;       /* block size in tokens, >= 1 */
  int32_t H;       /* query heads */
  int32_t Hkv;     /* key/value heads; H % Hkv == 0 (q head h reads KV head h/(H/Hkv)) */
  int32_t d;       /* head dim: 32 or 128 */
  int32_t dtype;   /* bdattn_dtype of every Q/K/V/O/dO/dQ/dK/dV tensor (but see precision) */
  float scale;     /* softmax scale; <= 0 selects 1/sqrt(d) */
  int64_t n_clean_q;      /* local clean queries ...                         */
  int64_t clean_q_start;  /* ... at global clean positions [start, start+n)  */
  int64_t n_clean_kv;     /* clean K/V buffer ...                            */
  int64_t clean_kv_start; /* ... at global positions [start, start+n); must be 0 */
  int64_t n_corr_blocks;  /* local corrupted blocks (each B tokens)          */
  /* HOST array of n_corr_blocks global block ids, non-decreasing, or NULL
   * for ids 0..n_corr_blocks-1. Read during the call only. A repeated id is
   * another corrupted copy of the same block (complementary masking, which
   * trains a block under a mask and its complement, as Fast-dLLM v2 does):
   * each local block sees the clean prefix of its id and only its own
   * corrupted keys. */
  const int32_t* corr_block_ids;
  int32_t clean_mask; /* bdattn_clean_mask; 0 (block-causal) for zero-initialised descriptors */
  /* 0: the complete attention; the clean buffer must start at position 0 and
   * hold every clean key a local query sees (BDATTN_ERR_COVERAGE otherwise).
   * 1: a partial attention over the keys present, in the sense of the
   * appendix's Implementation 1: clean keys at global positions
   * [clean_kv_start, clean_kv_start + n_clean_kv) (clean_kv_start any multiple
   * of B) and, unless omit_corr_keys, the local corrupted keys; the
   * visibility rules are unchanged. The forward then returns O and LSE over
   * the visible keys present (O = 0 and LSE = -inf for a row that sees none);
   * merge such results with bdattn_merge. The backward, given the MERGED O and
   * LSE of the complete attention, returns each gradient's part through the
   * keys present: dQ summed over a partition of the keys is the full dQ;
   * dK/dV of the keys present are complete. */
  int32_t partial;
  int32_t omit_corr_keys; /* 1: the local corrupted keys are absent (partial only) */
  /* Packed documents: several variable-length sequences in one problem (the
   * paper trains on variable sequence lengths, §5.1). HOST array of n_docs
   * start positions, increasing, the first 0, each a multiple of B; document
   * i holds the global positions [doc_starts[i], doc_starts[i+1]), the last
   * one runs to the end. Blocks are counted from each document's start and
   * no (query, key) pair crosses two documents; a corrupted block belongs to
   * the document holding its id. n_docs <= 1 or NULL: one document. Read
   * during the call only. */
  int32_t n_docs;
  const int32_t* doc_starts;
  /* A gathered clean K/V buffer (the appendix's Implementation 1 masks with
   * each gathered key's original clean token position; the context-sharded
   * all-gather of §4.3 delivers the chunks rank by rank, e.g. in zigzag
   * order). 0: the buffer is in position order. > 0: the buffer is
   * n_clean_kv / kv_chunk_len chunks of kv_chunk_len keys (a multiple of 128
   * and of B); chunk i holds the keys at global positions
   * [kv_chunk_pos[i], kv_chunk_pos[i] + kv_chunk_len). HOST array, read
   * during the call only. The chunks, in any order, must together cover
   * exactly [clean_kv_start, clean_kv_start + n_clean_kv)
   * (BDATTN_ERR_INVALID_ARG otherwise; BDATTN_ERR_SHAPE for a length that is
   * not such a multiple). dk_c/dv_c rows follow the buffer's order. */
  int32_t kv_chunk_len;
  const int32_t* kv_chunk_pos;
  /* bdattn_precision (bf16 inputs; ignored for float32 inputs). DEFAULT:
   * every tensor is of `dtype`. F32_OUT: O, dQ, dK and dV are float32 tensors
   * (the backward reads the forward's float32 O; dO stays bf16); the kernels
   * accumulate in float32 either way, so only the final stores change and the
   * float32 O rounds to the default one bit for bit. SPLIT: F32_OUT, and the
   * softmax weights P and the score gradients dS enter their matrix products
   * (P V, dV = P^T dO, dK = dS^T Q, dQ = dS K) as two bf16 terms, a rounded
   * value and its rounded remainder, so those products see them to about 16
   * bits instead of 8; the products with a split operand run twice (26d
   * instead of 18d matrix flops per pair and q head). The measured
   * alternatives selected by BDATTN_DKDV / BDATTN_BWD support DEFAULT only
   * and are not used otherwise. */
  int32_t precision;
} bdattn_problem;

/* BDATTN_VERSION of the loaded library. */
int bdattn_version(void);

/* Static description of a status code. */
const char* bdattn_status_string(int status);

/* Message of the last failure on this thread ("" if none). */
const char* bdattn_last_error(void);

/* Host-only check of a problem descriptor (no HIP calls). Rules: B >= 1;
 * H, Hkv >= 1 and H % Hkv == 0; d in {32, 128}; dtype known;
 * clean_mask known, partial and omit_corr_keys 0 or 1, omit_corr_keys only
 * with partial (BDATTN_ERR_INVALID_ARG);
 * n_clean_q, clean_q_start, n_clean_kv, n_corr_blocks >= 0; clean_q_start,
 * n_clean_q and n_clean_kv multiples of B (BDATTN_ERR_SHAPE); ids
 * non-decreasing and >= 0 (BDATTN_ERR_INVALID_ARG); every row count and global
 * position below 2^31; coverage unless partial: clean_kv_start == 0 and
 * n_clean_kv reaches the end of the last block of the query shard and the
 * start of the last local corrupted block (BDATTN_ERR_COVERAGE); partial:
 * clean_kv_start a multiple of B (BDATTN_ERR_SHAPE); n_docs >= 0, and with
 * n_docs > 0 doc_starts non-NULL, starting at 0, increasing and below 2^31
 * (BDATTN_ERR_INVALID_ARG), each a multiple of B (BDATTN_ERR_SHAPE). */
int bdattn_validate(const bdattn_problem* p);

/* Bytes of workspace needed by bdattn_fwd (pass 0) or bdattn_bwd (pass 1).
 * Host-only. */
int bdattn_workspace_size(const bdattn_problem* p, int pass, size_t* bytes);

/* Dense visibility matrix of the problem, written to HOST memory as uint8
 * (1 = visible), row-major [nq][nk] with queries = clean-local rows then
 * corrupted rows, keys = clean buffer then corrupted keys. `cap` is the size
 * of host_out in bytes; BDATTN_ERR_INVALID_ARG if it is smaller than nq*nk.
 * Computed from the same predicate the GPU kernels compile. Host-only. */
int bdattn_mask_render(const bdattn_problem* p, uint8_t* host_out, size_t cap);

/* Exact number of visible (query, key) pairs of one q head (host-only). The
 * useful work of fwd+bwd is 12*d*H*pairs flops (QK^T, PV forward; dV, dP,
 * dQ, dK backward). */
int bdattn_visible_pairs(const bdattn_problem* p, int64_t* pairs);

/* Planner statistics (host-only), for tests and logs. out[0..7] =
 * {fwd work items, fwd key tiles visited, fwd key tiles needing a mask,
 *  bwd work items, bwd q tiles visited, bwd q tiles needing a mask,
 *  fwd rows per work item, bwd keys per work item}. */
int bdattn_plan_stats(const bdattn_problem* p, int64_t out[8]);

/* The plan cache (host-only, no HIP calls). The library keeps, per distinct
 * problem descriptor, the planned work lists and a pinned host staging copy
 * of them, from which every call copies into its workspace asynchronously.
 * The cache is bounded: least recently used plans are evicted once the
 * plans' host memory plus the pinned staging memory of live plans exceeds
 * the budget (default 256 MiB), or beyond 1024 plans. An evicted plan's
 * staging buffer is reused or freed only after an event recorded behind its
 * last copy has completed. bdattn_plan_cache_info writes out[0..4] = {plans,
 * plan host bytes, pinned staging bytes (live and spare), budget, evictions
 * so far}. bdattn_plan_cache_budget sets the budget in bytes (>= 1 MiB,
 * BDATTN_ERR_INVALID_ARG otherwise); it applies from the next new plan on. */
int bdattn_plan_cache_info(int64_t out[5]);
int bdattn_plan_cache_budget(size_t bytes);

/* Forward (Implementation 1 of the appendix, fused into one launch): writes
 * o_c [n_clean_q,H,d], o_x [n_corr,H,d], lse_c [H,n_clean_q],
 * lse_x [H,n_corr]. Inputs q_c [n_clean_q,H,d], k_c/v_c [n_clean_kv,Hkv,d],
 * q_x [n_corr,H,d], k_x/v_x [n_corr,Hkv,d]. Pointers of empty tensors may be
 * NULL. */
int bdattn_fwd(const bdattn_problem* p,
               const void* q_c, const void* k_c, const void* v_c,
               const void* q_x, const void* k_x, const void* v_x,
               void* o_c, void* o_x, float* lse_c, float* lse_x,
               void* workspace, size_t ws_bytes, void* hip_stream);

/* The forward for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments and results as bdattn_fwd (bitwise: the same kernels), without
 * the workspace: the block ids, document table and work list go into a
 * scratch array the library holds in device memory, one per device, of at
 * most 8 MiB (a problem whose bdattn_workspace_size(pass 0) exceeds it gets
 * BDATTN_ERR_WORKSPACE; 8 MiB holds a 1M-token sequence at 64 q heads). The
 * call allocates no device and no pinned host memory; the first call on a
 * device looks up that device's array, and the first call with a new
 * problem plans it on the host. The work list is copied from pageable host
 * memory, so the call may wait for that copy to be staged. Every call on a
 * device shares the device's array: calls in one stream are ordered and
 * safe, calls that overlap on one device (other streams, other threads)
 * race. */
int bdattn_fwd_noalloc(const bdattn_problem* p,
                       const void* q_c, const void* k_c, const void* v_c,
                       const void* q_x, const void* k_x, const void* v_x,
                       void* o_c, void* o_x, float* lse_c, float* lse_x, void* hip_stream);

/* Backward (Implementation 2 of the appendix): from the forward's saved
 * o_c/o_x and lse_c/lse_x and the upstream do_c/do_x, writes dq_c, dq_x,
 * dk_c/dv_c [n_clean_kv,Hkv,d] (clean keys no local query sees get zeros)
 * and dk_x/dv_x [n_corr,Hkv,d] (not written, and may be NULL, when
 * omit_corr_keys). LSE is not differentiated. With partial = 1, o_c/o_x and
 * lse_c/lse_x must be those of the complete attention (see bdattn_problem). */
int bdattn_bwd(const bdattn_problem* p,
               const void* q_c, const void* k_c, const void* v_c,
               const void* q_x, const void* k_x, const void* v_x,
               const void* o_c, const void* o_x,
               const float* lse_c, const float* lse_x,
               const void* do_c, const void* do_x,
               void* dq_c, void* dq_x, void* dk_c, void* dv_c, void* dk_x, void* dv_x,
               void* workspace, size_t ws_bytes, void* hip_stream);

/* Merge two partial attention results over disjoint key sets (appendix,
 * Implementation 1): per row i and head h, with weights w = exp(LSE - LSE'),
 *   lse[h,i] = ln(exp(lse_a[h,i]) + exp(lse_b[h,i])),
 *   o[i,h,:] = (exp(lse_a - lse) o_a[i,h,:] + exp(lse_b - lse) o_b[i,h,:]).
 * A part with LSE = -inf has weight 0; a row with -inf in both gets o = 0,
 * lse = -inf. o_a/o_b/o are [n_rows, H, d] of `dtype` (32 or 128 for d; float32
 * at d = 128 too, for the float32 outputs of bf16 problems), LSE
 * [H, n_rows] float32; o may alias o_a or o_b and lse lse_a or lse_b (each
 * element is read before it is written by the same thread). Device pointers,
 * 16-byte aligned; enqueued on hip_stream. */
int bdattn_merge(int64_t n_rows, int32_t H, int32_t d, int32_t dtype,
                 const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                 void* o, float* lse, void* hip_stream);

/* Optional instrumentation for benchmarks. With profiling on (per calling
 * thread), bdattn_fwd and bdattn_bwd record a pair of HIP events on the
 * call's stream around each of their main kernels: index 0 = the forward
 * kernel, 1 = the backward dQ kernel, 2 = the backward dK/dV kernel (the
 * backward's D = rowsum(dO*O) kernel is not timed). bdattn_profile_read
 * waits for the recorded events, writes ms[0..2] (summed milliseconds) and
 * launches[0..2] (number of launches) since the last read, and releases the
 * events; either pointer may be NULL. Off by default; costs nothing when off. */
int bdattn_profile_enable(int on);
int bdattn_profile_read(double* ms, int64_t* launches);
/* The same for `count` kernel slots (at most 7): 0..2 as above, then the
 * linear cross-entropy's (include/bdattn_lce.h) 3 logits product, 4 row
 * kernel, 5 dH product, 6 dW product, each recorded once per chunk.
 * BDATTN_ERR_INVALID_ARG for a count outside [0, 7]. */
int bdattn_profile_read_n(int count, double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* BDATTN_H */
