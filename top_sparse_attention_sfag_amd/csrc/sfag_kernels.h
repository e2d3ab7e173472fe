// Launchers of the gfx950 kernels (HIP translation units only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sfag_plan.h"

namespace sfag {

struct RowArgs {
  const uint16_t *q, *qr, *dO, *k, *kr, *v;
  const uint16_t* o;   // forward output (k_sdp computes Delta from it)
  const float *smax, *ssum, *delta;
  const int32_t *rows, *nvalid;
  uint16_t *ds_out, *p_out, *dq, *dqr;
  int64_t t0, ntok, G, Gp, E;
  int32_t n_hb;
  float scale_log2;  // scale·log2(e)
  float ds_scale;    // power of two applied to dS before its 16-bit rounding
  float dq_mul;      // scale / ds_scale
  int32_t n_split;   // k_row: workgroups per token (>1: dQ sums go to dq_acc)
  float* dq_acc;     // (ntok, G, 512 + Dr) fp32, zeroed, when n_split > 1
  int32_t reverse;   // k_sdp / k_dq: visit the chunk's tokens last to first
  int32_t* phase;    // k_row16: per-XCD key-row hint (rotated walks), NULL: walk each token in order
};

constexpr int kKeyBlock = kKeyBlockRows;
constexpr int kMaxColBlocks = 6;

// A block of output columns of the key-centric kernel: `src` 0 contracts dS
// with [Q|Qr] (dK, dKrope), 1 contracts P with dO (dV); `tcol0` is the first
// column in the source rows, `ocol0` the first accumulator column.
struct ColBlock {
  int32_t src, tcol0, ocol0, width;
};

struct KbArgs {
  const uint16_t *q, *qr, *dO; // (T1, N1, 512), (T1, N1, Dr), (T1, N1, 512) as given
  const uint16_t *ds, *p;      // (ntok, E, Gp)
  const int32_t* svals;        // pair ids sorted by (key block, token)
  const int32_t* er;           // key row within its block of each sorted pair
  const int32_t *vis_start, *vis_key, *n_vis;  // visits: first sorted pair, composite key; count
  int32_t* nonempty;           // (nTR, nKB) flags
  float* part;                 // (nTR, T2, AW) partial sums per token range
  int64_t t0, ntok, E, G, Gp, T2, AW, TR;
  int32_t Dr, nKB, nTR, nCB;
  ColBlock cbs[kMaxColBlocks];
};

// Forward pass (out, softmaxMax, softmaxSum) over one chunk of tokens.
struct FwdArgs {
  const uint16_t *q, *qr, *k, *kr, *v;
  const int32_t *rows, *nvalid;
  uint16_t* out;
  float *smax, *ssum;
  int64_t t0, ntok, G, Gp, E;
  int32_t n_hb;   // 64-head blocks per token
  float scale;
  int32_t reverse;   // visit the chunk's tokens last to first
};
void launch_fwd(int32_t dtype, bool rope, const FwdArgs& a, hipStream_t s);

struct ColArgs {
  const uint16_t *q, *qr, *dO, *ds, *p;
  const int32_t *rows, *nvalid;
  float *acc, *partials;
  int64_t t0, ntok, G, Gp, E, AW;
};

void launch_band_indices(int32_t* idx, int64_t T1, int64_t K, int32_t block, int32_t layout, int64_t S1, int64_t S2,
                         const int32_t* lq, const int32_t* lk, int32_t B, int64_t pre, int64_t nxt, hipStream_t s);
void launch_dq_cast(int32_t dtype, const float* acc, int64_t t0, int64_t ntok, int64_t G, int32_t Dr, float mul,
                    void* dq, void* dqr, hipStream_t s);
// status (optional): the 16-byte validation word (flags, reserved, count).
void launch_seq_offsets(const int32_t* lq, const int32_t* lk, int32_t B, int64_t T1, int64_t T2, int32_t* q_off,
                        int32_t* kv_off, uint32_t* status, hipStream_t s);
void launch_delta(int32_t dtype, const void* dO, const void* O, float* delta, int64_t nrows, hipStream_t s);
void launch_fill_u32(void* p, uint64_t n, uint32_t v, hipStream_t s);
// sort_entries: each token's entries in ascending order first (K <= 16384,
// sequences of at most 65536 keys, no key listed twice), for the locality of
// the token kernels' gathers; off where the rows must follow the listing
// (the index inversion exposed on its own).
void launch_decode(const int32_t* idx, int64_t t0, int64_t ntok, const Dims& d, const int32_t* q_off,
                   const int32_t* kv_off, int32_t* rows, int32_t* nvalid, hipStream_t s, uint32_t* status = nullptr,
                   bool sort_entries = false);
// Stable radix sort of the chunk's valid pairs.  key_mode 0: by key row (then
// csr_off gets the per-key offsets); key_mode 1: by (key row / kKeyBlock) *
// ntok + token (csr_off may be NULL).  Invalid positions sort last.
void launch_csr(int64_t n, const int32_t* rows, const int32_t* nvalid, int64_t E, int64_t T2, int32_t sort_bits,
                int32_t* keys[2], int32_t* vals[2], int32_t* hist, int32_t* csr_off, int32_t** sorted_vals,
                hipStream_t s, int key_mode = 0, int64_t ntok = 0, int32_t** sorted_keys = nullptr);
void launch_key_reduce(const int32_t* off, const int32_t* pairs, const float* part, int64_t AW, int64_t T2, float* acc,
                       hipStream_t s);
void launch_cast(int32_t dtype, const float* acc, int64_t T2, int32_t D, int32_t Dr, float kscale, void* dk, void* dkr,
                 void* dv, hipStream_t s);
void launch_row(int32_t dtype, bool rope, const RowArgs& a, hipStream_t s);
// N1 >= 32: the S/P/dP/dS kernel, then the dQ kernel (together they replace launch_row)
void launch_sdp(int32_t dtype, bool rope, const RowArgs& a, hipStream_t s);
// beside: k_dq runs on the second stream beside the key-block kernels
void launch_dq(int32_t dtype, bool rope, const RowArgs& a, hipStream_t s, bool beside);
void launch_keyblock(int32_t dtype, const KbArgs& a, hipStream_t s);
void launch_visits(const int32_t* ck, const int32_t* svals, const int32_t* rows, int64_t n, int64_t ntok,
                   int32_t nkb, int32_t* flags, int32_t* scan_tmp, int32_t* vis_start, int32_t* vis_key, int32_t* er,
                   int32_t* n_vis, hipStream_t s);
void launch_scan_i32(int32_t* a, int64_t n, int32_t* tmp, hipStream_t s);
// Pairs of a chunk grouped by (key block, token) through per-token counting
// (key blocks up to kMaxBinBlocks); fills svals, er and the visit lists.
void launch_kb_bins(const int32_t* rows, const int32_t* nvalid, int64_t E, int32_t nkb, int64_t ntok, int32_t* cnt,
                    int32_t* flg, int32_t* scan_tmp, int32_t* svals, int32_t* er, int32_t* vis_start, int32_t* vis_key,
                    int32_t* n_vis, hipStream_t s);
// The outputs of the last chunk's range reduction: dKey|dKeyRope (scaled by
// kscale) and dValue in the input dtype, columns [0, D), [D, D + Dr) and
// [D + Dr, AW) of the accumulators.
struct KbOut {
  int32_t dtype, D, Dr;
  float kscale;
  void *dk, *dkr, *dv;
};
// acc[row] = (first ? 0 : acc[row]) + the non-empty ranges' partials in
// ascending range order; with `out` the sums go to the outputs instead.
void launch_kb_reduce(const float* part, const int32_t* nonempty, int64_t T2, int64_t AW, int32_t nTR, int32_t nKB,
                      float* acc, bool first, const KbOut* out, hipStream_t s);
void launch_col(int32_t dtype, bool rope, bool partial, const ColArgs& a, hipStream_t s);

}  // namespace sfag
