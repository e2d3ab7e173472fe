// Key-centric contraction over heads for dK / dKrope / dV (operator page
// "aclnnSparseFlashAttentionGrad", 功能说明 stages 1 and 3: dV = Pᵀ·dO and
// dK = scale·dSᵀ·Q, summed over every (token, position) selecting the key).
//
// Instead of scattering one partial row per (token, position) with atomics,
// a workgroup owns a block of 128 consecutive key rows and a block of output
// columns, and walks, in token order, the tokens of one token range that
// select any of its keys (the pairs are sorted by (key block, token): an
// inversion of the indices at key-block granularity).  For each such token
// it stages that token's P or dS rows for the block's keys in LDS (rows of
// unselected keys are zero) and accumulates
//     C[key][col] += Σ_h A[key][h] · B[h][col]
// with v_mfma_f32_16x16x32, where B is the token's Q (or dO) read from a
// per-token transposed copy so that each lane's 8 consecutive heads of one
// column are one 16-byte load.  C stays in registers for the whole range and
// is written once as an fp32 partial of that token range; a second kernel
// adds the partials of the ranges in ascending order.  Every sum runs in a
// fixed order, so the result is bitwise reproducible.
#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

namespace {

constexpr int kKB = kKeyBlock;   // key rows per block (128)
constexpr int kMB = kKB / 16;    // 16-row MFMA blocks per key block
constexpr int kMaxGroup = 256;   // entries staged per pass (one per thread)

__device__ __forceinline__ int64_t lower_bound_i32(const int32_t* a, int64_t n, int64_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

}  // namespace

// NB: 16-column MFMA blocks per wave (4 for a 256-column block, 1 for the
// 64-column rope block).
template <typename TT, int NB>
__global__ void __launch_bounds__(256, 2) k_keyblock(KbArgs a) {
  typedef typename TT::vec8 V8;
  constexpr int RB = 256;  // LDS bytes per staged row (up to 128 heads)
  __shared__ __attribute__((aligned(16))) unsigned char As[kKB * RB];
  __shared__ int32_t flag[kKB];
  __shared__ int32_t e_row[kMaxGroup];
  __shared__ int32_t e_pair[kMaxGroup];
  __shared__ int32_t e_pending[kMaxGroup];
  __shared__ int32_t s_cnt[4], s_more;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, n = lane & 15;
  // unit order: token range major, then key block, then column block
  const int cb = blockIdx.x % a.nCB;
  const int kb = (blockIdx.x / a.nCB) % a.nKB;
  const int tr = blockIdx.x / (a.nCB * a.nKB);
  const ColBlock c = a.cbs[cb];
  const int64_t t_lo = (int64_t)tr * a.TR, t_hi = min<int64_t>(t_lo + a.TR, a.ntok);
  const int64_t lo = lower_bound_i32(a.skeys, a.n, (int64_t)kb * a.ntok + t_lo);
  const int64_t hi = lower_bound_i32(a.skeys, a.n, (int64_t)kb * a.ntok + t_hi);
  if (tid == 0 && cb == 0) a.nonempty[(int64_t)tr * a.nKB + kb] = hi > lo ? 1 : 0;
  if (hi <= lo) return;

  const int Gp = (int)a.Gp;
  const int nks = (Gp + 31) / 32;
  const uint16_t* Bsrc = c.src == 0 ? a.qT : a.oT;
  const int64_t Bcols = c.src == 0 ? a.Dq : 512;
  const uint16_t* Asrc = c.src == 0 ? a.ds : a.p;
  const int colw = c.tcol0 + wave * 16 * NB;  // first source column of this wave

  f32x4 C[kMB][NB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) C[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t kb_row0 = (int64_t)kb * kKB;
  int64_t i = lo;
  while (i < hi) {
    // ---- the next group: up to 256 consecutive entries of one token -------
    const int32_t key0 = a.skeys[i];
    const int64_t tl = key0 - (int64_t)kb * a.ntok;
    const int64_t ie = i + tid;
    const bool in = ie < hi && a.skeys[ie] == key0;
    const uint64_t bal = __ballot(in);
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    int32_t pr = 0, rw = 0;
    if (in) {
      pr = a.svals[ie];
      rw = (int32_t)(a.rows[pr] - kb_row0);
      e_row[tid] = rw;
      e_pair[tid] = pr;
      e_pending[tid] = 1;
    }
    __syncthreads();
    // entries of one token are contiguous, so the group is a prefix of the
    // 256 candidates
    const int gs = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    // this token's Q (or dO) columns of the wave: B operands of every k-step,
    // fetched now so that their latency overlaps the staging below
    V8 Bp[4][NB];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int hq = 32 * ks + 8 * g;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ks < nks && hq < Gp) v = *(const uint4*)(Bsrc + ((tl * Bcols + colw + 16 * nb + n) * Gp + hq));
        Bp[ks][nb] = as_vec8<V8>(v);
      }
    }
    bool more = true;
    while (more) {
      // zero the staged rows and the per-row owner flags
      for (int x = tid; x < kKB * RB / 16; x += 256) *(uint4*)(As + x * 16) = make_uint4(0, 0, 0, 0);
      if (tid < kKB) flag[tid] = 0x7fffffff;
      if (tid == 0) s_more = 0;
      __syncthreads();
      // a key listed twice by the token: the earliest pending entry goes first
      if (tid < gs && e_pending[tid]) atomicMin(&flag[e_row[tid]], tid);
      __syncthreads();
      // copy the owners' rows (16-byte chunks, XOR-swizzled by row & 7)
      const int CH = Gp / 8;
      for (int x = tid; x < gs * CH; x += 256) {
        const int e = x / CH, q = x - e * CH;
        if (e_pending[e] && flag[e_row[e]] == e) {
          const int r = e_row[e];
          const uint4 v = *(const uint4*)(Asrc + (int64_t)e_pair[e] * Gp + q * 8);
          *(uint4*)(As + r * RB + (((q & ~7) | ((q & 7) ^ (r & 7))) << 4)) = v;
        }
      }
      __syncthreads();
      if (tid < gs && e_pending[tid]) {
        if (flag[e_row[tid]] == tid) e_pending[tid] = 0;
        else s_more = 1;
      }
      // ---- C += A · B over the heads of this token ------------------------
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < nks) {
          const int q = 4 * ks + g;
          const bool hok = 32 * ks + 8 * g < Gp;
          uint4 av[kMB];
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
            const int r = mb * 16 + n;
            av[mb] = hok ? *(const uint4*)(As + r * RB + (((q & ~7) | ((q & 7) ^ (r & 7))) << 4))
                         : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) C[mb][nb] = TT::mfma(as_vec8<V8>(av[mb]), Bp[ks][nb], C[mb][nb]);
        }
      }
      __syncthreads();
      more = s_more != 0;
      __syncthreads();
    }
    i += gs;
  }
  // ---- partial of this token range ----------------------------------------
  float* out = a.part + (int64_t)tr * a.T2 * a.AW;
  const int ocol = c.ocol0 + wave * 16 * NB + n;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t row = kb_row0 + mb * 16 + 4 * g + k;
      if (row < a.T2) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) out[row * a.AW + ocol + 16 * nb] = C[mb][nb][k];
      }
    }
  }
}

// acc[row] += Σ_tr part[tr][row] over the token ranges whose (range, key
// block) was non-empty, in ascending range order.
__global__ void __launch_bounds__(256) k_kb_reduce(const float* __restrict__ part, const int32_t* __restrict__ nonempty,
                                                   int64_t T2, int64_t AW, int32_t nTR, int32_t nKB,
                                                   float* __restrict__ acc) {
  const int64_t row = blockIdx.x;
  const int kb = (int)(row / kKB);
  for (int64_t col = threadIdx.x * 4; col < AW; col += 256 * 4) {
    float4 s = *(const float4*)(acc + row * AW + col);
    for (int tr = 0; tr < nTR; ++tr) {
      if (!nonempty[(int64_t)tr * nKB + kb]) continue;
      const float4 v = *(const float4*)(part + ((int64_t)tr * T2 + row) * AW + col);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    *(float4*)(acc + row * AW + col) = s;
  }
}

// Per-token transposed copies: qT[tl][c][h] = [Q|Qr][t][h][c] and
// oT[tl][c][h] = dO[t][h][c], heads padded with zeros to Gp.  One block per
// (token, 64-column slice).
__global__ void __launch_bounds__(256) k_transpose(const uint16_t* __restrict__ q, const uint16_t* __restrict__ qr,
                                                   const uint16_t* __restrict__ dO, int64_t t0, int64_t G, int64_t Gp,
                                                   int32_t Dr, uint16_t* __restrict__ qT, uint16_t* __restrict__ oT) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][128 + 8];
  const int64_t Dq = 512 + Dr;
  const int nsl_q = (int)(Dq / 64), nsl = nsl_q + 8;
  const int64_t tl = blockIdx.x / nsl;
  const int sl = blockIdx.x % nsl;
  const int64_t t = t0 + tl;
  const bool isq = sl < nsl_q;
  const int c0 = isq ? sl * 64 : (sl - nsl_q) * 64;
  // load [G][64] as 16-byte chunks: thread -> (head, chunk)
  for (int x = threadIdx.x; x < Gp * 8; x += 256) {
    const int hh = x >> 3, ch = x & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hh < G) {
      const int c = c0 + ch * 8;
      if (!isq) v = *(const uint4*)(dO + (t * G + hh) * 512 + c);
      else if (c < 512) v = *(const uint4*)(q + (t * G + hh) * 512 + c);
      else v = *(const uint4*)(qr + (t * G + hh) * Dr + (c - 512));
    }
    const uint16_t* pv = (const uint16_t*)&v;
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[ch * 8 + k][hh] = pv[k];
  }
  __syncthreads();
  uint16_t* dst = isq ? qT + (tl * Dq + c0) * Gp : oT + (tl * 512 + c0) * Gp;
  const int CH = (int)(Gp / 8);
  for (int x = threadIdx.x; x < 64 * CH; x += 256) {
    const int c = x / CH, ch = x - c * CH;
    *(uint4*)(dst + c * Gp + ch * 8) = *(const uint4*)&tile[c][ch * 8];
  }
}

void launch_transpose(const uint16_t* q, const uint16_t* qr, const uint16_t* dO, int64_t t0, int64_t ntok, int64_t G,
                      int64_t Gp, int32_t Dr, uint16_t* qT, uint16_t* oT, hipStream_t s) {
  if (ntok == 0) return;
  const int nsl = (512 + Dr) / 64 + 8;
  hipLaunchKernelGGL(k_transpose, dim3((unsigned)(ntok * nsl)), dim3(256), 0, s, q, qr, dO, t0, G, Gp, Dr, qT, oT);
}

void launch_keyblock(int32_t dtype, const KbArgs& a, bool wide, hipStream_t s) {
  // Column blocks 256 wide run with NB = 4, the 64-wide rope block with
  // NB = 1; each call launches the blocks of one width, so that every kernel
  // instance has a fixed register shape.
  KbArgs w = a;
  int m = 0;
  for (int i = 0; i < a.nCB; ++i)
    if ((a.cbs[i].width == 256) == wide) w.cbs[m++] = a.cbs[i];
  if (m == 0) return;
  w.nCB = m;
  const dim3 grid((unsigned)(w.nTR * w.nKB * w.nCB)), block(256);
  if (dtype == SFAG_BF16) {
    if (wide) hipLaunchKernelGGL((k_keyblock<BF16, 4>), grid, block, 0, s, w);
    else hipLaunchKernelGGL((k_keyblock<BF16, 1>), grid, block, 0, s, w);
  } else {
    if (wide) hipLaunchKernelGGL((k_keyblock<FP16, 4>), grid, block, 0, s, w);
    else hipLaunchKernelGGL((k_keyblock<FP16, 1>), grid, block, 0, s, w);
  }
}

void launch_kb_reduce(const float* part, const int32_t* nonempty, int64_t T2, int64_t AW, int32_t nTR, int32_t nKB,
                      float* acc, hipStream_t s) {
  if (T2 == 0) return;
  hipLaunchKernelGGL(k_kb_reduce, dim3((unsigned)T2), dim3(256), 0, s, part, nonempty, T2, AW, nTR, nKB, acc);
}

}  // namespace sfag
