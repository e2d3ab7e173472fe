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
 * frees no device memory and keeps no device state between calls (apart from
 * one auxiliary stream and two events per device, see sfag_backward).  Work
 * is enqueued asynchronously on the caller's stream.
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
 * preTokens = nextTokens = 2147483647.  deterministic: when true dKey/dValue
 * are bitwise reproducible run to run (key-centric reduction over a
 * key→(token, position) CSR); when false dKey/dValue may differ in the last
 * bits between runs.
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
 * With 32 <= N1 < 128 the dQ kernel runs on a second stream of the library's
 * (one per device, default priority, made on first use) between an event
 * recorded on `stream` and an event `stream` waits for, so every output is
 * complete once `stream` reaches that point: the caller synchronizes `stream`
 * only.  SFAG_CONCURRENT=0 keeps everything on `stream`.
 */
int sfag_backward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream);

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
