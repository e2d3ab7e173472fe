// Launchers of the gfx950 kernels (HIP translation units only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sfag_plan.h"

namespace sfag {

struct RowArgs {
  const uint16_t *q, *qr, *dO, *k, *kr, *v;
  const float *smax, *ssum, *delta;
  const int32_t *rows, *nvalid;
  uint16_t *ds_out, *p_out, *dq, *dqr;
  int64_t t0, ntok, G, Gp, E;
  int32_t n_hb;
  float scale_log2;  // scale·log2(e)
  float ds_scale;    // power of two applied to dS before its 16-bit rounding
  float dq_mul;      // scale / ds_scale
};

struct ColArgs {
  const uint16_t *q, *qr, *dO, *ds, *p;
  const int32_t *rows, *nvalid;
  float *acc, *partials;
  int64_t t0, ntok, G, Gp, E, AW;
};

void launch_seq_offsets(const int32_t* lq, const int32_t* lk, int32_t B, int32_t* q_off, int32_t* kv_off,
                        hipStream_t s);
void launch_delta(int32_t dtype, const void* dO, const void* O, float* delta, int64_t nrows, hipStream_t s);
void launch_fill_u32(void* p, uint64_t n, uint32_t v, hipStream_t s);
void launch_decode(const int32_t* idx, int64_t t0, int64_t ntok, const Dims& d, const int32_t* q_off,
                   const int32_t* kv_off, int32_t* rows, int32_t* nvalid, hipStream_t s);
void launch_csr(int64_t n, const int32_t* rows, const int32_t* nvalid, int64_t E, int64_t T2, int32_t sort_bits,
                int32_t* keys[2], int32_t* vals[2], int32_t* hist, int32_t* csr_off, int32_t** sorted_vals,
                hipStream_t s);
void launch_key_reduce(const int32_t* off, const int32_t* pairs, const float* part, int64_t AW, int64_t T2, float* acc,
                       hipStream_t s);
void launch_cast(int32_t dtype, const float* acc, int64_t T2, int32_t D, int32_t Dr, float kscale, void* dk, void* dkr,
                 void* dv, hipStream_t s);
void launch_row(int32_t dtype, bool rope, const RowArgs& a, hipStream_t s);
void launch_col(int32_t dtype, bool rope, bool partial, const ColArgs& a, hipStream_t s);

}  // namespace sfag
