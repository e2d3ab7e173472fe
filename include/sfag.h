/*
 * libsfag: backward pass of top-k sparse flash attention on AMD Instinct MI355X
 * (gfx950).  C ABI, plain pointers and sizes.
 *
 * The operation is the one the operator page "aclnnSparseFlashAttentionGrad"
 * (CANN ops-transformer documentation) defines:
 *   - 功能说明 (function description): for every query token, gather the key
 *     and value rows named by its top-k sparse indices (each index selects a
 *     block of sparseBlockSize consecutive positions), then
 *       stage 1  dP = dO·V_selᵀ,                dV_sel = Pᵀ·dO
 *       stage 2  dS = P ∘ (dP − rowsum(dO ∘ O))
 *       stage 3  dQ = scale·dS·K_sel,           dK_sel = scale·dSᵀ·Q
 *     with P = exp(scale·Q·K_selᵀ − softmaxMax) / softmaxSum recomputed from
 *     the forward statistics; dK and dV rows are summed over every token and
 *     position that selects them;
 *   - GetWorkspaceSize parameter table: tensors, layouts (BSND, TND), dtypes,
 *     the MLA rope parts (Dr = 64) and their gradients;
 *   - 约束说明 (constraints) and its Mask table: sparseMode 0 (no mask) and 3
 *     (causal, diagonal through the bottom-right corner), deterministic mode,
 *     empty query returns at once;
 *   - 函数原型 (prototypes): the two-phase call, a size query that validates
 *     and returns an executor, then an execute call on a stream.
 *
 * Memory: every tensor and the workspace belong to the caller and live in
 * device memory (HBM) of the current HIP device; the library allocates and
 * frees no device memory and keeps no device state between calls, apart from
 * one auxiliary stream and two events per device that it makes on first use
 * when a call runs two kernels side by side and no stream of the caller's is
 * given for that (sfag_options.auxStream), and the opt-in timing records of
 * sfag_profile_*.  Work is enqueued asynchronously on the caller's stream.
 * Nothing reads the environment: every tuning choice is a field of
 * sfag_options, fixed per plan.
 */
#ifndef SFAG_H
#define SFAG_H

#include <stdbool.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: the values of the operator page's 返回值 (return value) table. */
#define SFAG_OK 0
#define SFAG_ERR_NULLPTR 161001       /* a required tensor, data pointer or output pointer is NULL */
#define SFAG_ERR_PARAM_INVALID 161002 /* dtype, contiguity, inconsistent optional tensors, workspace too small, bad scale */
#define SFAG_ERR_RUNTIME 361001       /* a HIP runtime call or kernel launch failed */
#define SFAG_ERR_TILING 561002        /* layout, sparseMode, block size, token limits or a shape outside the supported range */

/* Element types of sfag_tensor.dtype. */
#define SFAG_BF16 1
#define SFAG_FP16 2
#define SFAG_FP32 3
#define SFAG_INT32 4

/* A dense tensor view.  data: device pointer (may be NULL only when the tensor
 * has no elements).  shape/stride: the first ndim entries are used, strides in
 * elements.  Only row-major contiguous tensors are accepted (the parameter
 * table marks every tensor as non-contiguous: unsupported). */
typedef struct sfag_tensor {
  void* data;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} sfag_tensor;

/* Host-side execution plan: copies of the descriptors and attributes (never the
 * data), the derived sizes and the workspace layout.  The analogue of the
 * operator's executor. */
typedef struct sfag_plan sfag_plan;

/* Values of sfag_options fields (0 always means "chosen from the shapes"). */
#define SFAG_SCATTER_AUTO 0
#define SFAG_SCATTER_KEYBLOCK 1  /* key-block contraction over the tokens selecting a block of 256 keys */
#define SFAG_SCATTER_PARTIALS 2  /* per-(token, position) rows summed per key in CSR order */
#define SFAG_SCATTER_ATOMIC 3    /* fp32 atomic adds (deterministic calls use PARTIALS instead) */
#define SFAG_TOKEN_AUTO 0
#define SFAG_TOKEN_FUSED 1       /* one kernel per token for S, P, dP, dS and dQ (up to 64 heads a workgroup) */
#define SFAG_TOKEN_SPLIT 2       /* S/P/dP/dS kernel then dQ kernel (up to 128 heads a workgroup; N1 >= 32) */
#define SFAG_ORDER_AUTO 0
#define SFAG_ORDER_ASCENDING 1   /* token kernels visit a chunk first token first */
#define SFAG_ORDER_DESCENDING 2  /* last token first (the default under sparseMode 3, except
                                    with 128 heads and k_dq on a second stream) */
#define SFAG_CONCURRENT_AUTO 0
#define SFAG_CONCURRENT_OFF 1
#define SFAG_CONCURRENT_ON 2

/*
 * Tuning and debugging choices of one plan.  They are not part of the
 * operator's interface: sfag_workspace_size makes a plan with the defaults
 * (every field 0), and sfag_plan_configure re-plans it with other values.
 * No choice changes what is computed; the deterministic mode's bits depend on
 * keyBlockRanges alone (never on the budget or the chunking).
 *   workspaceBudget  bytes the whole workspace should stay within; query
 *                    tokens are processed in chunks sized to it (0 = 48 GiB
 *                    for the backward pass, 16 GiB for the forward pass).  A
 *                    chunk never drops below one key-block token range, so
 *                    a tiny budget can still give a larger workspace.
 *   chunkTokens      at most this many query tokens per chunk (0 = no limit;
 *                    rounded down to whole token ranges, at least one).
 *   scatter          SFAG_SCATTER_* (how dKey/dValue rows are accumulated).
 *   tokenPath        SFAG_TOKEN_* (FUSED is the default for N1 <= 16).
 *   tokenOrder       SFAG_ORDER_*.
 *   concurrent       SFAG_CONCURRENT_*: run the dQ kernel on a second stream
 *                    beside the key-block kernels, and the key-block
 *                    grouping there beside the S/dP kernel (default on the
 *                    key-block path for 32 <= N1 < 128, and for N1 = 128
 *                    with chunks of at most 4096 tokens).
 *   rowSplit         workgroups sharing one token's positions in the fused
 *                    token kernel (0 = chosen; 1..8; never split when
 *                    deterministic, whose sums must keep a fixed order).
 *   keyBlockRanges   token ranges per default-size chunk of the key-block
 *                    path (0 = 16).  Range boundaries are fixed in absolute
 *                    token coordinates from the shapes and this value.
 *   validate         1: the call also checks its index and length inputs on
 *                    the device (sfag_validation_read reports the result);
 *                    the workspace grows by 256 bytes.
 *   auxStream        the second stream of a concurrent call (a hipStream_t
 *                    of the caller's, on the same device); NULL = one the
 *                    library makes once per device and keeps until the
 *                    process ends.
 */
typedef struct sfag_options {
  uint64_t workspaceBudget;
  int64_t chunkTokens;
  int32_t scatter;
  int32_t tokenPath;
  int32_t tokenOrder;
  int32_t concurrent;
  int32_t rowSplit;
  int32_t keyBlockRanges;
  int32_t validate;
  int32_t reserved;
  void* auxStream;
} sfag_options;

/*
 * Phase 1: validate the arguments, plan the launch and report the workspace
 * size in bytes.  Host only: reads no device memory, launches nothing.
 *
 * Shapes (N2 = 1, G = N1, D = 512, Dr = 64):
 *   BSND: query/dOut/out/dQueryOut (B,S1,N1,D); key/value/dKeyOut/dValueOut
 *         (B,S2,1,D); sparseIndices (B,S1,1,K) int32; softmaxMax/softmaxSum
 *         (B,1,S1,N1) fp32; rope tensors (…,Dr) with the matching leading dims.
 *   TND:  query (T1,N1,D); key/value (T2,1,D); sparseIndices (T1,1,K);
 *         softmaxMax/softmaxSum (1,T1,N1); actualSeqLengthsQuery/Kv (B,) int32
 *         holding per-sequence token counts that sum to T1 / T2 (required).
 * Float tensors share one dtype, bf16 or fp16.  queryRope and keyRope are
 * given together or not at all; with them dQueryRopeOut and dKeyRopeOut are
 * required.  Index entry i selects key positions [i, i + sparseBlockSize) of its
 * sequence; negative entries select nothing; positions at or beyond the key
 * length, or (sparseMode 3) after t + Lk − Lq, are masked.
 * scaleValue: finite; used as float32.  sparseBlockSize ∈ {1, 8, 16, 32, 64}.
 * layoutOptional: "BSND" or "TND" (NULL = "BSND").  sparseMode ∈ {0, 3}.
 * preTokens = nextTokens = 2147483647.  deterministic: when true every
 * output is bitwise reproducible run to run (dKey/dValue from a key-centric
 * reduction in a fixed order; dQuery summed in a fixed order); when false the
 * outputs may differ in the last bits between runs (with N1 <= 16 the token
 * kernel starts each token's walk where its XCD's workgroups are, and a
 * token's positions may be split over workgroups; fp32 atomics where the
 * selection is sparse).
 * On SFAG_OK *workspaceSize and *plan are set; the plan must be passed to
 * sfag_backward (which frees it) or to sfag_plan_destroy.  On error *plan is
 * NULL and sfag_last_error() describes the failure.
 */
int sfag_workspace_size(const sfag_tensor* query, const sfag_tensor* key, const sfag_tensor* value,
                        const sfag_tensor* sparseIndices, const sfag_tensor* dOut, const sfag_tensor* out,
                        const sfag_tensor* softmaxMax, const sfag_tensor* softmaxSum,
                        const sfag_tensor* actualSeqLengthsQueryOptional,
                        const sfag_tensor* actualSeqLengthsKvOptional,
                        const sfag_tensor* queryRopeOptional, const sfag_tensor* keyRopeOptional,
                        double scaleValue, int64_t sparseBlockSize, const char* layoutOptional,
                        int64_t sparseMode, int64_t preTokens, int64_t nextTokens, bool deterministic,
                        const sfag_tensor* dQueryOut, const sfag_tensor* dKeyOut, const sfag_tensor* dValueOut,
                        const sfag_tensor* dQueryRopeOutOptional, const sfag_tensor* dKeyRopeOutOptional,
                        uint64_t* workspaceSize, sfag_plan** plan);

/*
 * Phase 2: enqueue the backward pass on `stream` (a hipStream_t; NULL = the
 * default stream).  workspace: device buffer of at least the phase-1 size
 * (may be NULL when that size is 0).  Every output element is written: rows of
 * dKey/dValue/dKeyRope that no valid position selects become 0.  The plan is
 * consumed and freed, also on error.  Returns SFAG_OK once the work is
 * enqueued; errors found by the kernels are not reported (indices are bounds
 * checked on the device, so bad indices are masked, never dereferenced).
 * When the plan runs the dQ kernel beside the key-block kernels (by default
 * with 32 <= N1 < 128, or N1 = 128 and chunks of at most 4096 tokens;
 * sfag_options.concurrent), that kernel and the key-block grouping go on a
 * second stream (sfag_options.auxStream, or one of the library's: one per
 * device, default priority, made on first use and kept until the process
 * ends) between events recorded on `stream` and events `stream` waits for,
 * so every output is complete once `stream` reaches the end of the call's
 * work: the caller synchronizes `stream` only.  Calls that share the
 * library's second stream on one device are ordered on it.
 */
int sfag_backward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream);

/*
 * The backward pass of `plan` for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the library's own scratch array serves as the workspace.  That
 * array, SFAG_STATIC_SCRATCH_BYTES (256 MiB), is a device global of the
 * library: each GPU the library runs on holds one until the process ends.
 * The plan's workspace must fit in it (re-plan with sfag_plan_configure and
 * workspaceBudget <= SFAG_STATIC_SCRATCH_BYTES); a larger plan is rejected
 * with SFAG_ERR_PARAM_INVALID before anything is enqueued.  The plan is
 * consumed and freed, also on error.  The call allocates nothing (no
 * hipMalloc, hipFree, stream or event; the opt-in timing of
 * sfag_profile_enable aside): a plan that would run kernels on a second
 * stream without a caller stream for it (sfag_options.auxStream) runs them
 * all on `stream` instead.  Every call on one GPU uses that GPU's one
 * array, so calls that overlap on one GPU (other streams, other threads)
 * race: the caller orders them.  The kernels initialise every part of the
 * array they read (the accumulators are zero-filled at the start of each
 * call), so what an earlier call left there does not matter.  Outputs and
 * errors are those of sfag_backward.
 */
#define SFAG_STATIC_SCRATCH_BYTES (256ull << 20)
int sfag_backward_static(sfag_plan* plan, void* stream);

/*
 * Forward pass of the same attention (the producer of the backward's out,
 * softmaxMax and softmaxSum inputs, whose meaning the operator page's
 * parameter table gives): for each query token t and head h, over the valid
 * positions p of t (the decode and mask rules above),
 *   z = scale·(Q[t,h]·K[p] + Qrope[t,h]·Krope[p]),
 *   softmaxMax[t,h] = max_p z,  softmaxSum[t,h] = Σ_p exp(z − softmaxMax),
 *   out[t,h] = Σ_p exp(z − softmaxMax)/softmaxSum · V[p]
 * (fp32 accumulation; out rounded to the input dtype).  A token with no valid
 * position gets softmaxMax = −inf, softmaxSum = 0 and out = 0.
 * Inputs as for sfag_workspace_size; out has query's shape and dtype,
 * softmaxMax/softmaxSum the statistics' shapes, float32.  All three are
 * written in full by sfag_forward.  The two-phase protocol, the plan's
 * ownership and the error behaviour are those of the backward call; a plan
 * from one call cannot be executed by the other (SFAG_ERR_PARAM_INVALID).
 */
int sfag_forward_workspace_size(const sfag_tensor* query, const sfag_tensor* key, const sfag_tensor* value,
                                const sfag_tensor* sparseIndices, const sfag_tensor* actualSeqLengthsQueryOptional,
                                const sfag_tensor* actualSeqLengthsKvOptional, const sfag_tensor* queryRopeOptional,
                                const sfag_tensor* keyRopeOptional, double scaleValue, int64_t sparseBlockSize,
                                const char* layoutOptional, int64_t sparseMode, const sfag_tensor* out,
                                const sfag_tensor* softmaxMax, const sfag_tensor* softmaxSum,
                                uint64_t* workspaceSize, sfag_plan** plan);
int sfag_forward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream);

/*
 * Re-plans a plan from sfag_workspace_size or sfag_forward_workspace_size
 * (not yet executed) with `options` (NULL = the defaults) and reports the new
 * workspace size.  Host only.  Errors: SFAG_ERR_NULLPTR for a NULL plan or
 * size pointer; SFAG_ERR_PARAM_INVALID for a field outside its values
 * (the plan is left as it was); SFAG_ERR_TILING when no chunking fits the
 * 32-bit pair numbering.
 */
int sfag_plan_configure(sfag_plan* plan, const sfag_options* options, uint64_t* workspaceSize);

/*
 * Result of the device-side input checks of a call planned with
 * options.validate = 1, read back from that call's workspace.  flags is an
 * OR of:
 *   SFAG_BAD_LENGTH_NEGATIVE   an actualSeqLengths entry is negative (the
 *                              parameter table warns that negative values
 *                              are invalid; they count as 0);
 *   SFAG_BAD_LENGTH_SUM_Q/_KV  the query / key lengths do not add up to T1 /
 *                              T2 (the parameter table requires that they
 *                              do; tokens past the declared lengths get no
 *                              valid position and keys past them are never
 *                              read);
 *   SFAG_BAD_INDEX_RANGE       an index entry is at or past its sequence's
 *                              key length (such entries are masked).
 * badEntries counts the entries of the last kind.  sfag_validation_read
 * enqueues a copy of the 16-byte result on `stream`, waits for the stream and
 * fills *result; call it with the workspace of a finished validating call
 * before reusing that workspace.  Errors: SFAG_ERR_NULLPTR,
 * SFAG_ERR_RUNTIME for a failed copy.
 */
#define SFAG_BAD_LENGTH_NEGATIVE 1u
#define SFAG_BAD_LENGTH_SUM_Q 2u
#define SFAG_BAD_LENGTH_SUM_KV 4u
#define SFAG_BAD_INDEX_RANGE 8u
typedef struct sfag_validation {
  uint32_t flags;
  uint32_t reserved;
  uint64_t badEntries;
} sfag_validation;
int sfag_validation_read(const void* workspace, void* stream, sfag_validation* result);

/* Frees a plan that will not be executed.  NULL is accepted. */
void sfag_plan_destroy(sfag_plan* plan);

/* Thread-local description of the last failure of a call on this thread. */
const char* sfag_last_error(void);

/*
 * Index inversion on its own (the integer part of the deterministic path),
 * exposed so that it can be checked bit for bit.  Decodes sparseIndices with
 * the mask rules above and builds the key→(token, position) CSR.
 *   sparseIndices: device int32 (T1, K).  seqLensQ/seqLensKv: device int32 (B,)
 *   for layout 1 (TND), ignored for layout 0 (BSND, where T1 = B·S1, T2 = B·S2).
 *   Outputs (device): nValid (T1) int32, the number of valid positions of each
 *   token; rows (T1, K·block) int32, row t holding in its first nValid[t]
 *   entries the global key row of each valid position in position order;
 *   csrOffsets (T2+1) int32; csrPairs (T1·K·block) int32, in its first
 *   csrOffsets[T2] entries the pairs selecting each key row as t·(K·block) + c
 *   (c = rank of the position among the token's valid positions), grouped by
 *   key row and ascending within a key.
 * sfag_index_workspace_size gives the workspace this call needs.
 * Returns SFAG_ERR_TILING when T1·K·block ≥ 2^31.
 */
uint64_t sfag_index_workspace_size(int64_t T1, int64_t T2, int64_t K, int64_t block);
int sfag_build_index(const void* sparseIndices, const void* seqLensQ, const void* seqLensKv, int64_t B,
                     int64_t S1, int64_t S2, int64_t T1, int64_t T2, int64_t K, int64_t block, int32_t layout,
                     int64_t sparseMode, void* workspace, uint64_t workspaceSize, void* nValid, void* rows,
                     void* csrOffsets, void* csrPairs, void* stream);

/*
 * Band (sliding-window or dense) selection written as sparse indices, so that
 * dense and banded attention run through sfag_forward / sfag_backward on the
 * same kernels.  The band is the block-band test of the MindSpore
 * FlashAttention backward page ("flash_attention_bwd.py",
 * compute_in_each_kv_block: query block q meets key block k iff
 * k − next ≤ q ≤ k + prev), taken per query token and aligned, as sparseMode 3
 * is, on the diagonal through the bottom-right corner: query position t of a
 * sequence with Lq query and Lk key tokens covers key positions
 * d − preTokens .. d + nextTokens, d = t + Lk − Lq, clipped to [0, Lk).
 *
 * sfag_band_indices writes sparseIndices (T1, K) int32 (device, row-major):
 * row t holds, ascending, the start (a multiple of sparseBlockSize, local to
 * the sequence) of every block of sparseBlockSize positions that contains a
 * covered position, then −1 up to K entries; rows are cut after K entries.
 * Tokens past the declared TND lengths get rows of −1.  seqLensQ / seqLensKv:
 * device int32 (B,) per-sequence counts for layout 1 (TND, 1 ≤ B ≤ 256),
 * ignored for layout 0 (BSND: T1 = B·S1, keys S2).  preTokens, nextTokens ≥ 0
 * (2147483647 = unbounded); block ≥ 1.  Enqueued on `stream`; writes nothing
 * else.  Errors: SFAG_ERR_TILING for bad layout or sizes, SFAG_ERR_NULLPTR for
 * a missing pointer, SFAG_ERR_RUNTIME for a failed launch.
 *
 * sfag_band_entries(maxKeyLen, ...) is the K that loses no block for any
 * sequence with at most maxKeyLen keys (0 for bad arguments).
 */
int64_t sfag_band_entries(int64_t maxKeyLen, int64_t preTokens, int64_t nextTokens, int64_t block);
int sfag_band_indices(void* sparseIndices, const void* seqLensQ, const void* seqLensKv, int64_t B, int64_t S1,
                      int64_t S2, int64_t T1, int64_t K, int64_t block, int32_t layout, int64_t preTokens,
                      int64_t nextTokens, void* stream);

/*
 * Optional per-kernel timing for measurement.  While enabled, sfag_backward
 * records a pair of HIP events on its stream around each kernel group
 * ("seq_offsets", "delta", "fill", "decode", "row", "col", "csr", "key_reduce",
 * "cast").  sfag_profile_read waits for the recorded events and returns the
 * summed milliseconds and number of launches of one group since the last
 * reset.  Process-wide state guarded by a mutex; off by default.
 */
void sfag_profile_enable(int on);
void sfag_profile_reset(void);
int sfag_profile_read(const char* kernel, double* totalMs, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* SFAG_H */
