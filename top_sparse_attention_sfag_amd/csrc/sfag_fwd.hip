// Forward pass of the top-k sparse attention whose backward the rest of the
// library computes.  It produces the three tensors the backward takes from
// the forward (operator page "aclnnSparseFlashAttentionGrad", 功能说明 and the
// parameter table: out, softmaxMax, softmaxSum):
//     z[h][p] = scale · (Q[h]·K[p] + Qrope[h]·Krope[p])   over valid positions p
//     softmaxMax[h] = max_p z,  softmaxSum[h] = Σ_p exp(z − max)
//     out[h] = Σ_p exp(z − max) / softmaxSum · V[p]
// A token without a valid position gets max = −inf, sum = 0 and out = 0.
//
// gfx950 mapping (k_fwd8 below): one workgroup per (token, 64-head block) as
// 8 waves.  Per tile of 32 gathered positions, Sᵀ = K·Qᵀ on
// v_mfma_f32_16x16x32 (positions as M, Q rows resident in registers), an
// online softmax per head (running max and sum; the fp32 output
// accumulators are rescaled when the max grows), and out += P·V with P from
// LDS as the A operand and V read transposed from LDS (ds_read_b64_tr_b16).
// K|Krope|V rows arrive through global_load_lds into a double buffer,
// 16-byte chunks XOR-swizzled by (row & 7).  With fewer than 64 heads the
// block's upper head groups are zero (64-head blocks with 8 waves measured
// faster at 16 heads than 4 waves of which one held the heads: 87.3 -> 63.6
// ms for 2 x 32768 tokens of 512 blocks of 16).
#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

namespace {

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

constexpr int kTile = 32;   // positions per tile
constexpr int kXcds = 8;    // blockIdx % 8 picks the XCD
constexpr int kRun = 16;    // consecutive tokens per XCD run
constexpr bool kFwdSpread = true;   // k_fwd8 issues a tile's copies between the Sᵀ MFMAs

// Asynchronous global -> LDS copy of 16 bytes per lane (lane l writes at the
// wave-uniform LDS address l_base + 16 l).  Inline asm on purpose: the
// compiler's own form of this copy is tracked as a pending LDS write, and
// without alias information it then waits for every outstanding copy before
// the next LDS read, so the next tile's gather would not overlap the current
// tile's MFMAs.  Reads of copied data follow the explicit s_waitcnt and the
// barrier at the top of each tile.  The copy starts with one wait state
// (s_nop 0): on this chip family an LDS DMA that reads M0 right after a scalar
// write of M0 needs one, and the compiler inserts it only for DMA
// instructions it emits itself.
__device__ __forceinline__ void lds_load16(const void* g, void* l) {
  const uint32_t la = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) unsigned char*)l);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(la)) : "memory");
}

}  // namespace

// k_fwd8: one workgroup per (token, 64-head block) as 8 waves, two per SIMD,
// so that one wave's MFMAs run while the other waits.  Wave w = 4 ph + hg forms
// Sᵀ of head group hg (16 heads, Q in registers) over the position half ph
// of each 32-position tile; the two halves' maxima meet in LDS, each wave
// turns its half into P (bf16, into LDS as (head, position) rows) with the
// tile's common running max, and every wave then adds P·V into its own 64
// output columns for all 64 heads (64 fp32 accumulators a lane instead of
// 128, which is what leaves room for a second wave).  The per-head rescale
// factors and the final sums pass through LDS as well.
template <typename TT, int DR, bool VK>
__global__ void __launch_bounds__(512, 1) k_fwd8(FwdArgs a) {
  constexpr int DQK = 512 + DR;
  constexpr int KS_QK = DQK / 32;
  constexpr int KM_BYTES = kTile * 1024;
  constexpr int KR_BYTES = kTile * DR * 2;
  constexpr int V_BYTES = VK ? 0 : kTile * 1024;
  constexpr int BUF = KM_BYTES + KR_BYTES + V_BYTES;
  constexpr int PST = 72;   // bytes per head row of P (32 positions + 8: conflict-free A reads)
  typedef typename TT::vec8 V8;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) unsigned char ps[64 * PST];
  __shared__ float xmax[2][64];   // per position half: the tile's max of each head
  __shared__ __attribute__((aligned(16))) float alpha_s[64];
  __shared__ float lsum[2][64];
  __shared__ __attribute__((aligned(16))) float inv_s[64];

  const int b = blockIdx.x;
  const int xcd = b % kXcds, u = b / kXcds;
  const int hb = u % a.n_hb;
  const int tq = u / a.n_hb;
  int64_t tl = ((int64_t)(tq / kRun) * kXcds + xcd) * kRun + (tq % kRun);
  if (a.reverse) tl = (a.ntok + kXcds * kRun - 1) / (kXcds * kRun) * (kXcds * kRun) - 1 - tl;
  if (tl >= a.ntok) return;
  const int64_t t = a.t0 + tl;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int hg = wave & 3, ph = wave >> 2;
  const int hl = hg * 16 + n;              // head of this lane within the block (Sᵀ column)
  const int h = hb * 64 + hl;
  const bool hv = h < a.G;

  V8 Qf[KS_QK];
#pragma unroll
  for (int ks = 0; ks < KS_QK; ++ks) {
    const int d0 = 32 * ks + 8 * g;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hv) {
      if (d0 < 512) v = *(const uint4*)(a.q + (t * a.G + h) * 512 + d0);
      else v = *(const uint4*)(a.qr + (t * a.G + h) * DR + (d0 - 512));
    }
    Qf[ks] = as_vec8<V8>(v);
  }
  // output accumulators: head block j (heads 16 j + 4 g + i), column block c
  // (columns 64 wave + 16 c + n)
  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[j][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;   // head hl; l_run: this lane's share of this half

  const int nv = a.nvalid[tl];
  const int32_t* rt = a.rows + tl * a.E;

  // Gather of the 32 rows of a tile into buffer `buf` (rows past nv repeat a
  // valid row, masked out of the softmax) in five steps per wave: step j < 4
  // copies K (and V) row 4w + j, step 4 (w < 4) rope rows 8w .. 8w + 7.
  // The key rows of a step's copies are formed for all five steps at once
  // (scalar for the wave's K|V rows, one lane shuffle for the rope rows), so
  // that issuing a step needs no LDS operation and no wait of its own.
  struct TileKeys {
    int32_t row[4];
    int32_t rope;
  };
  auto tile_keys8 = [&](int c0) -> TileKeys {
    const int cl = c0 + (lane & 31);
    const int key_l = rt[cl < nv ? cl : 0];   // lane r & 31: key row of the tile's position r
    TileKeys tk;
#pragma unroll
    for (int j = 0; j < 4; ++j) tk.row[j] = __builtin_amdgcn_readlane(key_l, wave * 4 + j);
    tk.rope = DR > 0 ? __shfl(key_l, (wave & 3) * 8 + (lane >> 3), 64) : 0;
    return tk;
  };
  auto issue_step = [&](int j, const TileKeys& tk, int buf) {
    unsigned char* base = smem + buf * BUF;
    if (j < 4) {
      const int r = wave * 4 + j;
      const int64_t key = tk.row[j];
      const int gc = lane ^ (r & 7);
      lds_load16(a.k + key * 512 + gc * 8, base + r * 1024);
      if (!VK) lds_load16(a.v + key * 512 + gc * 8, base + KM_BYTES + KR_BYTES + r * 1024);
    } else if (DR > 0 && wave < 4) {
      const int r_l = wave * 8 + (lane >> 3);
      const int gc = (lane & 7) ^ (r_l & 7);
      lds_load16(a.kr + (int64_t)tk.rope * DR + gc * 8, base + KM_BYTES + wave * 8 * (DR * 2));
    }
  };

  // Sᵀ operand offsets (rows ph·16 + n; chunk c of row r sits at chunk
  // (c & ~7) | ((c & 7) ^ (r & 7))) and the transposed V reads
  const int x = n & 7;
  const int oA_even = n * 1024 + 16 * (g ^ x) + ph * 16384;
  const int oA_odd = n * 1024 + 16 * ((4 + g) ^ x) + ph * 16384;
  const int oR_even = n * (DR * 2) + 16 * (g ^ x) + ph * 16 * (DR * 2);
  const int oR_odd = n * (DR * 2) + 16 * ((4 + g) ^ x) + ph * 16 * (DR * 2);
  const int r1 = 4 * g + (n >> 2), x1 = r1 & 7;
  const int half = (n & 3) >> 1, hoff = (n & 1) * 8;
  int oT[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) oT[c] = r1 * 1024 + 16 * ((2 * c + half) ^ x1) + hoff + 128 * wave;

  if (nv > 0) {
    const TileKeys k0 = tile_keys8(0);
#pragma unroll
    for (int j = 0; j < 5; ++j) issue_step(j, k0, 0);
  }
  int cur = 0;
  for (int c0 = 0; c0 < nv; c0 += kTile) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the next tile's copies: at once here, or spread between the Sᵀ MFMAs
    const bool more = c0 + kTile < nv;
    const TileKeys tk = tile_keys8(more ? c0 + kTile : c0);
    if (!kFwdSpread && more) {
#pragma unroll
      for (int j = 0; j < 5; ++j) issue_step(j, tk, cur ^ 1);
    }
    const unsigned char* Km = smem + cur * BUF;
    const unsigned char* Kr = Km + KM_BYTES;
    const unsigned char* Vm = VK ? Km : Km + KM_BYTES + KR_BYTES;
    // ---- Sᵀ of positions ph·16 + 4g + i, head hl
    auto kaddr = [&](int ks) -> const unsigned char* {
      if (ks < 16) return Km + ((ks & 1) ? oA_odd : oA_even) + 128 * (ks >> 1);
      return Kr + ((ks & 1) ? oR_odd : oR_even);
    };
    f32x4 sv = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 kb4[4];
#pragma unroll
    for (int i = 0; i < 3; ++i) kb4[i] = *(const uint4*)kaddr(i);
#pragma unroll
    for (int ks = 0; ks < KS_QK; ++ks) {
      if (ks + 3 < KS_QK) kb4[(ks + 3) & 3] = *(const uint4*)kaddr(ks + 3);
      // (step j at k-step 3j + 1: 128 heads, 4096 tokens, top-2048 causal 3.29 ms
      // with a step every other k-step, 3.22 ms every third)
      if (kFwdSpread && more && ks < 14 && (ks % 3) == 1) issue_step(ks / 3, tk, cur ^ 1);
      sv = TT::mfma(as_vec8<V8>(kb4[ks & 3]), Qf[ks], sv);
      __builtin_amdgcn_sched_barrier(0);
    }
    float z[4];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = c0 + ph * 16 + 4 * g + i < nv ? sv[i] * a.scale : -__builtin_inff();
      tmax = fmaxf(tmax, z[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (g == 0) xmax[ph][hl] = tmax;
    __syncthreads();
    // ---- P with the tile's common running max (finite: the tile holds a
    // valid position)
    const float m_new = fmaxf(m_run, fmaxf(xmax[0][hl], xmax[1][hl]));
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * kLog2e);
    float psum = 0.f;
    uint16_t pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f((z[i] - m_new) * kLog2e);
      psum += p;
      pv[i] = TT::from_f(p);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    *(uint2*)(ps + hl * PST + 32 * ph + 8 * g) =
        make_uint2(pv[0] | ((uint32_t)pv[1] << 16), pv[2] | ((uint32_t)pv[3] << 16));
    if (ph == 0 && g == 0) alpha_s[hl] = alpha;
    __syncthreads();
    // ---- out += P·V over this wave's 64 columns, all 64 heads
    V8 A8[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned char* pr = ps + (16 * j + n) * PST + 8 * g;
      const uint2 lo = *(const uint2*)pr, hi = *(const uint2*)(pr + 32);
      A8[j] = as_vec8<V8>(make_uint4(lo.x, lo.y, hi.x, hi.y));
      const float4 al = *(const float4*)(alpha_s + 16 * j + 4 * g);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[j][c][0] *= al.x;
        acc[j][c][1] *= al.y;
        acc[j][c][2] *= al.z;
        acc[j][c][3] *= al.w;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const unsigned char* p1 = Vm + oT[c];
      const V8 B8 = join_tr<V8>(lds_read_tr((const uint16_t*)p1), lds_read_tr((const uint16_t*)(p1 + 16 * 1024)));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j][c] = TT::mfma(A8[j], B8, acc[j][c]);
    }
    cur ^= 1;
  }
  // ---- statistics and out
  float l_half = l_run + __shfl_xor(l_run, 16);
  l_half += __shfl_xor(l_half, 32);
  __syncthreads();
  if (g == 0) lsum[ph][hl] = l_half;
  __syncthreads();
  if (ph == 0 && g == 0) {
    const float l_tot = lsum[0][hl] + lsum[1][hl];
    inv_s[hl] = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (hv) {
      a.smax[t * a.G + h] = m_run;
      a.ssum[t * a.G + h] = l_tot;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 iv = *(const float4*)(inv_s + 16 * j + 4 * g);
    const float ivs[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = hb * 64 + 16 * j + 4 * g + i;
      if (hh < a.G) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          a.out[(t * a.G + hh) * 512 + 64 * wave + 16 * c + n] = TT::from_f(acc[j][c][i] * ivs[i]);
      }
    }
  }
}

void launch_fwd(int32_t dtype, bool rope, const FwdArgs& a, hipStream_t s) {
  if (a.ntok == 0) return;
  const int64_t per = (int64_t)kXcds * kRun;
  const int64_t padded = (a.ntok + per - 1) / per * per;
  const dim3 grid((unsigned)(padded * a.n_hb));
  const bool vk = a.v == a.k;   // value passed as the key tensor: gather each row once
  auto go = [&](auto tt, auto dr) {
    typedef decltype(tt) T;
    constexpr int D = decltype(dr)::value;
    if (vk) hipLaunchKernelGGL((k_fwd8<T, D, true>), grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((k_fwd8<T, D, false>), grid, dim3(512), 0, s, a);
  };
  if (dtype == SFAG_BF16) {
    if (rope) go(BF16(), std::integral_constant<int, 64>());
    else go(BF16(), std::integral_constant<int, 0>());
  } else {
    if (rope) go(FP16(), std::integral_constant<int, 64>());
    else go(FP16(), std::integral_constant<int, 0>());
  }
}

}  // namespace sfag
