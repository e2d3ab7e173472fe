// MFMA core of the backward pass (gfx950, v_mfma_f32_16x16x32_{bf16,f16}).
//
// Per query token the operator page "aclnnSparseFlashAttentionGrad" (功能说明,
// stages 1-3) needs five contractions over the token's selected key rows:
//   S  = [Q|Qr]·[K|Kr]_selᵀ  (over D+Dr)      dP = dO·V_selᵀ   (over D)
//   dQ = scale·dS·[K|Kr]_sel (over positions)
//   dK_sel = scale·dSᵀ·[Q|Qr] (over heads)    dV_sel = Pᵀ·dO   (over heads)
// with P = exp(scale·S − max)/sum and dS = P ∘ (dP − Delta).
//
// They run in two kernels so that each keeps its stationary operand on chip:
//   k_row  (per token × 64-head block): S, P, dP, dS and dQ.  The token's Q/dO
//          fragments and the fp32 dQ accumulator live in registers; tiles of
//          32 gathered K/Kr/V rows go through LDS.  P and dS leave as 16-bit
//          (token, position, head) rows.
//   k_col  (per token, dK part or dV part): the contraction over heads.  The
//          token's Q (or dO) is staged in LDS once and turned into transposed
//          MFMA fragments with ds_read_b64_tr_b16; P or dS tiles stream in.  The
//          resulting per-(token, position) rows are added into fp32 key-row
//          accumulators with hardware atomics, or stored as partial rows for
//          the deterministic key-centric reduction.
#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

constexpr int kColTile = 16;  // positions per k_col tile

// PART 0: dK|dKr partial rows = dSᵀ·[Q|Qr]; PART 1: dV partial rows = Pᵀ·dO.
template <typename TT, int DR, int PART, bool PARTIAL>
__global__ void __launch_bounds__(256, 1) k_col(ColArgs a) {
  constexpr int WID = PART == 0 ? 512 + DR : 512;  // output columns of this part
  constexpr int CW = WID / 4;                      // columns per wave
  constexpr int NB = CW / 16;
  constexpr int BSTR = WID + 8;
  constexpr int CPR = WID / 8;
  constexpr int MAXKS = 4;                         // up to 128 heads in steps of 32
  typedef typename TT::vec8 V8;

  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * BSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int64_t tl = blockIdx.x;
  const int64_t t = a.t0 + tl;
  const int G = (int)a.G;
  const int G32 = (G + 31) & ~31;
  const int nks = G32 / 32;
  const int nv = a.nvalid[tl];
  if (nv == 0) return;

  for (int i = tid; i < G32 * CPR; i += 256) {
    const int r = i / CPR, j = i - r * CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < G) {
      if (PART == 0) {
        if (j < 64) val = *(const uint4*)(a.q + (t * G + r) * 512 + j * 8);
        else val = *(const uint4*)(a.qr + (t * G + r) * DR + (j - 64) * 8);
      } else {
        val = *(const uint4*)(a.dO + (t * G + r) * 512 + j * 8);
      }
    }
    *(uint4*)(Bs + r * BSTR + j * 8) = val;
  }
  __syncthreads();
  // Transposed fragments: lane (column n of block nb, head group g) holds heads
  // 32ks + 8g .. +7 of its column.
  V8 Bf[NB][MAXKS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int ks = 0; ks < MAXKS; ++ks) {
      if (ks < nks) {
        const uint16_t* p1 = Bs + (32 * ks + 8 * g + (n >> 2)) * BSTR + wave * CW + 16 * nb + 4 * (n & 3);
        Bf[nb][ks] = join_tr<V8>(lds_read_tr(p1), lds_read_tr(p1 + 4 * BSTR));
      } else {
        Bf[nb][ks] = zero_vec8<V8>();
      }
    }
  }
  const uint16_t* Asrc = PART == 0 ? a.ds : a.p;
  const int32_t* rt = a.rows + tl * a.E;
  const int colbase = (PART == 0 ? 0 : 512 + DR) + wave * CW;
  for (int c0 = 0; c0 < nv; c0 += kColTile) {
    V8 A[MAXKS];
    const int cA = c0 + n;
#pragma unroll
    for (int ks = 0; ks < MAXKS; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      const int hA = 32 * ks + 8 * g;
      if (ks < nks && cA < nv && hA < a.Gp) u = *(const uint4*)(Asrc + (tl * a.E + cA) * a.Gp + hA);
      A[ks] = as_vec8<V8>(u);
    }
    f32x4 o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < MAXKS; ++ks)
        if (ks < nks) o[nb] = TT::mfma(A[ks], Bf[nb][ks], o[nb]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 4 * g + i;
      if (c >= nv) continue;
      if (PARTIAL) {
        float* dst = a.partials + (tl * a.E + c) * a.AW + colbase + n;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) dst[16 * nb] = o[nb][i];
      } else {
        float* dst = a.acc + (int64_t)rt[c] * a.AW + colbase + n;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) unsafeAtomicAdd(dst + 16 * nb, o[nb][i]);
      }
    }
  }
}

template <typename TT, int DR, bool PARTIAL>
static void launch_col_t(const ColArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.ntok), block(256);
  hipLaunchKernelGGL((k_col<TT, DR, 0, PARTIAL>), grid, block, 0, s, a);
  hipLaunchKernelGGL((k_col<TT, DR, 1, PARTIAL>), grid, block, 0, s, a);
}

void launch_col(int32_t dtype, bool rope, bool partial, const ColArgs& a, hipStream_t s) {
  if (a.ntok == 0) return;
  if (dtype == SFAG_BF16) {
    if (rope) partial ? launch_col_t<BF16, 64, true>(a, s) : launch_col_t<BF16, 64, false>(a, s);
    else partial ? launch_col_t<BF16, 0, true>(a, s) : launch_col_t<BF16, 0, false>(a, s);
  } else {
    if (rope) partial ? launch_col_t<FP16, 64, true>(a, s) : launch_col_t<FP16, 64, false>(a, s);
    else partial ? launch_col_t<FP16, 0, true>(a, s) : launch_col_t<FP16, 0, false>(a, s);
  }
}

}  // namespace sfag
