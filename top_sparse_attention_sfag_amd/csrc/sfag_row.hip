// Token-centric MFMA kernel: for one query token and a block of 64 of its
// heads, recompute the logits of every selected key, form P, dP, dS
// (operator page "aclnnSparseFlashAttentionGrad", 功能说明 stages 1-2) and
// accumulate dQ = scale·dS·K_sel (stage 3).  P and dS leave as 16-bit
// (token, position, head) rows for the head-contraction kernels.
//
// gfx950 mapping:
//   * 4 waves, each owning 16 heads; v_mfma_f32_16x16x32 with the positions
//     as M for Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ (B operands: the wave's Q / dO rows,
//     resident in registers) and the heads as M for dQ (A operand: dS straight
//     from the Sᵀ accumulator layout; B operand: K read transposed from LDS
//     with ds_read_b64_tr_b16).  The fp32 dQ accumulator stays in registers.
//   * The 32 gathered K | Krope | V rows of the next tile are fetched with
//     global_load_lds_dwordx4 (global -> LDS without registers) into the other
//     half of a double buffer while the current tile is computed.
//   * LDS rows are stored with their 16-byte chunks XOR-swizzled by (row & 7)
//     so that the 16 rows an MFMA operand reads at one column fall into
//     different bank groups.
//   * Work units are ordered so that each XCD (blockIdx % 8) takes runs of 16
//     consecutive tokens: neighbouring tokens share many selected keys, which
//     then hit in that XCD's L2.
#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

namespace {

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

constexpr int kTile = 32;          // positions per tile
constexpr int kXcds = 8;           // XCDs of an MI355X; blockIdx % 8 picks the XCD
constexpr int kRun = 16;           // consecutive tokens per XCD run

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

// VK: value is the key tensor itself; the first 512 columns of each gathered
// K row serve as its V row (one gather per position).
template <typename TT, int DR, bool VK>
__global__ void __launch_bounds__(256, 1) k_row(RowArgs a) {
  constexpr int DQK = 512 + DR;
  constexpr int KS_QK = DQK / 32;
  constexpr int KS_V = 512 / 32;
  constexpr int NB_Q = DQK / 16;
  constexpr int KM_BYTES = kTile * 1024;        // K main part of a tile
  constexpr int KR_BYTES = kTile * DR * 2;      // K rope part
  constexpr int V_BYTES = VK ? 0 : kTile * 1024;
  constexpr int BUF = KM_BYTES + KR_BYTES + V_BYTES;
  constexpr int STAGE = kTile * 64 * 2;         // one 32 x 64 16-bit staging tile
  typedef typename TT::vec8 V8;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF + 2 * STAGE];
  unsigned char* stage_ds = smem + 2 * BUF;
  unsigned char* stage_p = stage_ds + STAGE;

  // ---- work unit: (token, head block), XCD-aware order ---------------------
  const int b = blockIdx.x;
  const int xcd = b % kXcds, u = b / kXcds;
  const int hb = u % a.n_hb;
  const int rest = u / a.n_hb;
  const int sp = rest % a.n_split;   // which share of the token's positions
  const int tq = rest / a.n_split;
  const int64_t tl = ((int64_t)(tq / kRun) * kXcds + xcd) * kRun + (tq % kRun);
  if (tl >= a.ntok) return;
  const int64_t t = a.t0 + tl;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int h0 = hb * 64 + wave * 16;
  const bool wave_on = h0 < a.Gp;
  const int h = h0 + n;
  const bool hv = h < a.G;

  V8 Qf[KS_QK], dOf[KS_V];
#pragma unroll
  for (int ks = 0; ks < KS_QK; ++ks) {
    const int d0 = 32 * ks + 8 * g;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (wave_on && hv) {
      if (d0 < 512) v = *(const uint4*)(a.q + (t * a.G + h) * 512 + d0);
      else v = *(const uint4*)(a.qr + (t * a.G + h) * DR + (d0 - 512));
    }
    Qf[ks] = as_vec8<V8>(v);
  }
#pragma unroll
  for (int ks = 0; ks < KS_V; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (wave_on && hv) v = *(const uint4*)(a.dO + (t * a.G + h) * 512 + 32 * ks + 8 * g);
    dOf[ks] = as_vec8<V8>(v);
  }
  float mlog = 0.f, inv_l = 0.f, dl = 0.f;
  bool live = false;
  if (wave_on && hv) {
    const float m = a.smax[t * a.G + h], l = a.ssum[t * a.G + h];
    live = l > 0.f;
    inv_l = live ? 1.f / l : 0.f;
    mlog = m * kLog2e;
    dl = a.delta[t * a.G + h];
  }
  f32x4 acc[NB_Q];
#pragma unroll
  for (int i = 0; i < NB_Q; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nv = a.nvalid[tl];
  const int32_t* rt = a.rows + tl * a.E;
  // positions [cb, ce) of this workgroup: whole tiles, the last share ending at nv
  int cb = 0, ce = nv;
  if (a.n_split > 1) {
    const int per = (((nv + a.n_split - 1) / a.n_split) + kTile - 1) / kTile * kTile;
    cb = min(nv, sp * per);
    ce = min(nv, cb + per);
  }

  // Gather the 32 rows of tile c0 into buffer `buf`; rows past nv repeat a
  // valid row (their dS is exactly 0).  Wave w loads rows 8w..8w+7.
  auto issue_tile = [&](int c0, int buf) {
    unsigned char* base = smem + buf * BUF;
    const int r_l = wave * 8 + (lane >> 3);  // rope row handled by this lane
    const int c_l = c0 + r_l;
    const int key_l = rt[c_l < nv ? c_l : 0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = wave * 8 + j;
      const int64_t key = __builtin_amdgcn_readfirstlane(__shfl(key_l, j * 8, 64));
      const int gc = lane ^ (r & 7);
      lds_load16(a.k + key * 512 + gc * 8, base + r * 1024);
      if (!VK) lds_load16(a.v + key * 512 + gc * 8, base + KM_BYTES + KR_BYTES + r * 1024);
    }
    if (DR > 0) {
      const int pc = lane & 7;
      const int gc = pc ^ (r_l & 7);
      lds_load16(a.kr + (int64_t)key_l * DR + gc * 8, base + KM_BYTES + wave * 8 * (DR * 2));
    }
  };

  // Per-lane LDS byte offsets (relative to a buffer).  Chunk index c of row r
  // sits at chunk (c & ~7) | ((c & 7) ^ (r & 7)); for the rows and chunks each
  // lane touches this reduces to a few bases plus immediate offsets.
  const int x = n & 7;                                 // (row & 7) of rows mb*16 + n
  const int oA_even = n * 1024 + 16 * (g ^ x);         // chunk 4ks+g, ks even
  const int oA_odd = n * 1024 + 16 * ((4 + g) ^ x);    // ks odd
  const int oR_even = n * (DR * 2) + 16 * (g ^ x);     // rope chunk g
  const int oR_odd = n * (DR * 2) + 16 * ((4 + g) ^ x);  // rope chunk 4+g
  const int r1 = 4 * g + (n >> 2), x1 = r1 & 7;       // dQ B operand rows r1, r1+16
  const int half = (n & 3) >> 1, hoff = (n & 1) * 8;
  int oT[4], oTr[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    oT[w] = r1 * 1024 + 16 * ((2 * w + half) ^ x1) + hoff;
    oTr[w] = r1 * (DR * 2) + 16 * ((2 * w + half) ^ x1) + hoff;
  }

  if (cb < ce) issue_tile(cb, 0);
  int cur = 0;
  for (int c0 = cb; c0 < ce; c0 += kTile) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c0 + kTile < ce) issue_tile(c0 + kTile, cur ^ 1);
    const unsigned char* Km = smem + cur * BUF;
    const unsigned char* Kr = Km + KM_BYTES;
    const unsigned char* Vm = VK ? Km : Km + KM_BYTES + KR_BYTES;
    if (wave_on) {
      // Sᵀ and dPᵀ.  With operand room (no rope, or value passed as the key)
      // the reads run three MFMAs ahead, each step pinned in order; with the
      // rope operands and a separate V that form spills, so the plain loops
      // stay there.
      constexpr bool kAhead = !(DR > 0 && !VK);
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (kAhead) {
        constexpr int NS = 2 * KS_QK, NP = 2 * KS_V;
        auto addr = [&](int i) -> const unsigned char* {
          if (i < NS) {
            const int mb = i / KS_QK, ks = i % KS_QK;
            if (ks < 16) return Km + ((ks & 1) ? oA_odd : oA_even) + 128 * (ks >> 1) + mb * 16384;
            return Kr + ((ks & 1) ? oR_odd : oR_even) + mb * 16 * (DR * 2);
          }
          const int j = i - NS, mb = j / KS_V, ks = j % KS_V;
          return Vm + ((ks & 1) ? oA_odd : oA_even) + 128 * (ks >> 1) + mb * 16384;
        };
        constexpr int RA = 3;
        uint4 ob[4];
#pragma unroll
        for (int i = 0; i < RA; ++i) ob[i] = *(const uint4*)addr(i);
#pragma unroll
        for (int i = 0; i < NS + NP; ++i) {
          if (i + RA < NS + NP) ob[(i + RA) & 3] = *(const uint4*)addr(i + RA);
          if (i < NS) s[i / KS_QK] = TT::mfma(as_vec8<V8>(ob[i & 3]), Qf[i % KS_QK], s[i / KS_QK]);
          else dp[(i - NS) / KS_V] = TT::mfma(as_vec8<V8>(ob[i & 3]), dOf[(i - NS) % KS_V], dp[(i - NS) / KS_V]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
          const unsigned char* ke = Km + oA_even + mb * 16384;
          const unsigned char* ko = Km + oA_odd + mb * 16384;
          const unsigned char* ve = Vm + oA_even + mb * 16384;
          const unsigned char* vo = Vm + oA_odd + mb * 16384;
#pragma unroll
          for (int ks = 0; ks < 16; ++ks) {
            const unsigned char* p = ((ks & 1) ? ko : ke) + 128 * (ks >> 1);
            s[mb] = TT::mfma(as_vec8<V8>(*(const uint4*)p), Qf[ks], s[mb]);
          }
          if (DR > 0) {
            const unsigned char* re = Kr + oR_even + mb * 16 * (DR * 2);
            const unsigned char* ro = Kr + oR_odd + mb * 16 * (DR * 2);
            s[mb] = TT::mfma(as_vec8<V8>(*(const uint4*)re), Qf[KS_QK - 2], s[mb]);
            s[mb] = TT::mfma(as_vec8<V8>(*(const uint4*)ro), Qf[KS_QK - 1], s[mb]);
          }
#pragma unroll
          for (int ks = 0; ks < KS_V; ++ks) {
            const unsigned char* p = ((ks & 1) ? vo : ve) + 128 * (ks >> 1);
            dp[mb] = TT::mfma(as_vec8<V8>(*(const uint4*)p), dOf[ks], dp[mb]);
          }
        }
      }
      // P = exp(scale·S − max)/sum and dS = P ∘ (dP − Delta) for head h and
      // positions 4g+i (block 0) and 16+4g+i (block 1).
      uint16_t pv[8], dsv[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = mb * 16 + 4 * g + i;
          const bool ok = live && (c0 + j < nv);
          const float p = ok ? exp2f(s[mb][i] * a.scale_log2 - mlog) * inv_l : 0.f;
          const float ds = p * (dp[mb][i] - dl);
          pv[mb * 4 + i] = TT::from_f(p);
          dsv[mb * 4 + i] = TT::from_f(ds * a.ds_scale);
          const int so = (j * 64 + wave * 16 + n) * 2;
          *(uint16_t*)(stage_ds + so) = dsv[mb * 4 + i];
          *(uint16_t*)(stage_p + so) = pv[mb * 4 + i];
        }
      }
      const uint4 dsu = make_uint4(dsv[0] | ((uint32_t)dsv[1] << 16), dsv[2] | ((uint32_t)dsv[3] << 16),
                                   dsv[4] | ((uint32_t)dsv[5] << 16), dsv[6] | ((uint32_t)dsv[7] << 16));
      const V8 A8 = as_vec8<V8>(dsu);
      // dQ += dS·K over the tile's 32 positions: B operand = K rows
      // 4g..4g+3 and 16+4g..16+4g+3 of one column, read transposed.
      auto kread = [&](int nb) -> V8 {
        const unsigned char* p1 = nb < 32 ? Km + oT[nb & 3] + 128 * (nb >> 2) : Kr + oTr[nb & 3];
        const unsigned char* p2 = p1 + (nb < 32 ? 16 * 1024 : 16 * (DR * 2));
        return join_tr<V8>(lds_read_tr((const uint16_t*)p1), lds_read_tr((const uint16_t*)p2));
      };
      if constexpr (kAhead) {
        V8 kb[4];
#pragma unroll
        for (int i = 0; i < 3; ++i) kb[i] = kread(i);
#pragma unroll
        for (int nb = 0; nb < NB_Q; ++nb) {
          if (nb + 3 < NB_Q) kb[(nb + 3) & 3] = kread(nb + 3);
          acc[nb] = TT::mfma(A8, kb[nb & 3], acc[nb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB_Q; ++nb) acc[nb] = TT::mfma(A8, kread(nb), acc[nb]);
      }
    }
    __syncthreads();
    // P and dS of the tile: 32 positions x 64 heads each, one 16-byte chunk
    // per thread and array.
    {
      const int j = tid >> 3, q = tid & 7;
      const int hh = hb * 64 + q * 8;
      if (c0 + j < nv && hh < a.Gp) {
        const int64_t o = (tl * a.E + c0 + j) * a.Gp + hh;
        *(uint4*)(a.ds_out + o) = *(const uint4*)(stage_ds + (j * 64 + q * 8) * 2);
        *(uint4*)(a.p_out + o) = *(const uint4*)(stage_p + (j * 64 + q * 8) * 2);
      }
    }
    cur ^= 1;
  }
  if (!wave_on) return;
  if (a.n_split > 1) {
    // this share's dQ|dQrope sums, unscaled; the cast kernel scales and rounds
    if (cb >= ce) return;
#pragma unroll
    for (int nb = 0; nb < NB_Q; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = h0 + 4 * g + i;
        if (hh < a.G) atomicAdd(a.dq_acc + (tl * a.G + hh) * DQK + 16 * nb + n, acc[nb][i]);
      }
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NB_Q; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + 4 * g + i;
      if (hh < a.G) {
        const int col = 16 * nb + n;
        const uint16_t v = TT::from_f(acc[nb][i] * a.dq_mul);
        if (col < 512) a.dq[(t * a.G + hh) * 512 + col] = v;
        else a.dqr[(t * a.G + hh) * DR + (col - 512)] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_row16: the fused token kernel for up to 16 heads (one head block of 16),
// with the work of a tile spread over all four waves and two workgroups per
// CU (one or two tile buffers each, see kSingle).
//
//   * Sᵀ = K·Qᵀ and dPᵀ = V·dOᵀ of a 32-position tile: wave 0 / 1 form Sᵀ of
//     positions 0..15 / 16..31 (Q in registers), wave 2 / 3 dPᵀ of the same
//     halves (dO in registers); dPᵀ goes to the S waves through LDS.
//   * P = exp(scale·S − max)/sum and dS = P ∘ (dP − Delta) in the S waves;
//     dS is staged in LDS as (head, position) rows, the A operand of
//   * dQ += dS·K_tile: wave w owns every fourth block of 16 dQ|dQrope
//     columns (K read transposed from LDS), fp32 accumulators in registers.
//   * Delta = rowsum(dO ∘ O) (功能说明 stage 2) is formed once per token in
//     the prologue by wave 2, which holds dO, and handed over through LDS.
//   * Waves 0..2 issue the tile copies (global_load_lds) and no other
//     vector-memory work inside the loop, so a wait on their copy counter
//     counts copies only.  With two buffers that wait leaves the next tile's
//     copies in flight: the copies of tile i + 2 go out as soon as every
//     wave is done with tile i, while tile i + 1's are still landing; with
//     one, tile i + 1's go out then and are waited for in full.  Wave 3
//     issues no copies; it stores the P and dS rows (staged in LDS, double
//     buffered) and loads the row indices of the tile whose copies go out
//     next into LDS, so the copying waves never wait on a load of their own.
// ---------------------------------------------------------------------------
template <typename TT, int DR, bool VK>
__global__ void __launch_bounds__(256, 2) k_row16(RowArgs a) {
  constexpr int DQK = 512 + DR;
  constexpr int KS_QK = DQK / 32;          // 16x16x32 k-steps of S (rope last)
  constexpr int KS_V = 512 / 32;
  constexpr int NB_Q = DQK / 16;           // 16-column blocks of dQ|dQrope
  constexpr int NBW = NB_Q / 4;            // per wave
  constexpr int KM_BYTES = kTile * 1024;
  constexpr int KR_BYTES = kTile * DR * 2;
  constexpr int V_BYTES = VK ? 0 : kTile * 1024;
  constexpr int BUF = KM_BYTES + KR_BYTES + V_BYTES;
  constexpr int XSTR = 36;                 // floats per head row of the dPᵀ exchange
  constexpr int DSTR = 40;                 // 16-bit elements per head row of the dS staging
  // copy instructions per tile of copying wave w (rows w, w+3, ...; rope
  // groups of 8 rows w, w+3)
  constexpr int kRowOps = VK ? 1 : 2;
  typedef typename TT::vec8 V8;

  // Two workgroups share a CU, each one's phases (and its copies' latency)
  // overlapping the other's: with separate K and V rows (64 KB a tile) or
  // rope rows each workgroup has one tile buffer, with value = key and no
  // rope two (the next tile landing during this one).  Config-4 shape (16
  // heads, 8192 positions, separate V): 74.9 -> 66.5 ms against one
  // double-buffered workgroup per CU; 4 heads with rope: 0.056 -> 0.043 ms.
  constexpr bool kSingle = !VK || DR > 0;
  constexpr int kAhead = kSingle ? kTile : 2 * kTile;   // positions between a tile and its copies' issue
  __shared__ __attribute__((aligned(16))) unsigned char tbuf[kSingle ? 1 : 2][BUF];
  __shared__ __attribute__((aligned(16))) float xdp[16 * XSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dsT[16 * DSTR];
  __shared__ __attribute__((aligned(16))) uint16_t stg[2][2][kTile * 16];   // [buffer][P, dS][position][head]
  __shared__ int32_t keys_s[kTile];
  __shared__ float delta_s[16];
  __shared__ int rot_s;

  // ---- work unit: token (and share of its positions), XCD-aware order ------
  const int b = blockIdx.x;
  const int xcd = b % kXcds, u = b / kXcds;
  const int sp = u % a.n_split;
  const int tq = u / a.n_split;
  const int64_t tl = ((int64_t)(tq / kRun) * kXcds + xcd) * kRun + (tq % kRun);
  if (tl >= a.ntok) return;
  const int64_t t = a.t0 + tl;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const bool hv = n < a.G;                 // head n
  const bool s_wave = wave < 2, copier = wave < 3;
  const int mb = wave & 1;                 // position half of the Sᵀ / dPᵀ waves

  const int nv = a.nvalid[tl];
  const int32_t* rt = a.rows + tl * a.E;
  int cb = 0, ce = nv;
  if (a.n_split > 1) {
    const int per = (((nv + a.n_split - 1) / a.n_split) + kTile - 1) / kTile * kTile;
    cb = min(nv, sp * per);
    ce = min(nv, cb + per);
  }
  // The share's tiles, walked from tile `rot` on and wrapping.  With a phase
  // hint (calls without the deterministic guarantee) the walk starts at the
  // fraction of its tiles that the workgroups of this XCD last announced
  // reaching: the token's rows ascend (the decode sorts them), so the
  // workgroups that run together on the XCD, each starting where the others
  // are, sweep the key rows together and share their gathers through the
  // XCD's L2.  Any start is correct; only dQ's order of sums depends on it.
  // (One thread reads the hint, which other workgroups rewrite at any time,
  // and hands it to the others, so that every wave walks the same order.)
  const int ntl = (ce - cb + kTile - 1) / kTile;
  int rot = 0;
  if (a.phase && ntl > 1) {
    if (tid == 0) {
      const uint32_t frac =
          (uint32_t)__hip_atomic_load(a.phase + 32 * xcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xffffu;
      rot_s = (int)((frac * (uint32_t)ntl) >> 16);
    }
    __syncthreads();
    rot = __builtin_amdgcn_readfirstlane(rot_s);
    if (rot >= ntl) rot = 0;
  }
  auto tile_at = [&](int L) -> int {   // first position of the L-th tile walked (L < ntl)
    const int x = L + rot;
    return cb + (x >= ntl ? x - ntl : x) * kTile;
  };
  constexpr int kAheadTiles = kAhead / kTile;   // tiles between a tile and its copies' issue

  // ---- prologue: operands, statistics, Delta ----------------------------
  V8 Bf[KS_QK > KS_V ? KS_QK : KS_V];      // Q (S waves) or dO (dP waves) of head n
#pragma unroll
  for (int ks = 0; ks < KS_QK; ++ks) {
    const int d0 = 32 * ks + 8 * g;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hv) {
      if (s_wave) {
        if (d0 < 512) v = *(const uint4*)(a.q + (t * a.G + n) * 512 + d0);
        else v = *(const uint4*)(a.qr + (t * a.G + n) * DR + (d0 - 512));
      } else if (ks < KS_V) {
        v = *(const uint4*)(a.dO + (t * a.G + n) * 512 + d0);
      }
    }
    Bf[ks] = as_vec8<V8>(v);
  }
  float mlog = 0.f, inv_l = 0.f;
  bool live = false;
  if (s_wave && hv) {
    const float m = a.smax[t * a.G + n], l = a.ssum[t * a.G + n];
    live = l > 0.f;
    inv_l = live ? 1.f / l : 0.f;
    mlog = m * kLog2e;
  }
  if (wave == 2) {
    float dsum = 0.f;
    if (hv) {
#pragma unroll
      for (int ks = 0; ks < KS_V; ++ks) {
        const uint4 ov = *(const uint4*)(a.o + (t * a.G + n) * 512 + 32 * ks + 8 * g);
        const uint4 dv = __builtin_bit_cast(uint4, Bf[ks]);
        const uint16_t* po = (const uint16_t*)&ov;
        const uint16_t* pd = (const uint16_t*)&dv;
#pragma unroll
        for (int j = 0; j < 8; ++j) dsum = fmaf(TT::to_f(pd[j]), TT::to_f(po[j]), dsum);
      }
    }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    if (g == 0) delta_s[n] = dsum;
  }
  // row indices of the first two tiles (a position past the share's end
  // repeats its first valid position; its P and dS are 0)
  int32_t key0 = 0, key1 = 0;
  if (copier && cb < ce) {
    const int c_0 = tile_at(0) + (lane & 31), c_1 = (ntl > 1 ? tile_at(1) : cb) + (lane & 31);
    key0 = rt[c_0 < ce ? c_0 : cb];
    key1 = rt[c_1 < ce ? c_1 : cb];
  }
  // every prologue load has landed before the first copy goes out, so the
  // copy counter waits below count copies only
  __builtin_amdgcn_s_waitcnt(0);
  f32x4 acc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- tile copies -------------------------------------------------------
  // Copying wave w fetches K (and V) rows w, w + 3, ... of the tile and the
  // rope rows of groups w, w + 3 (8 rows per instruction); chunk c of row r
  // lands at chunk (c & ~7) | ((c & 7) ^ (r & 7)).
  auto issue = [&](int32_t keyv, int buf) {
    unsigned char* base = tbuf[buf];
#pragma unroll
    for (int r0 = 0; r0 < kTile; r0 += 3) {
      const int r = r0 + wave;
      if (r < kTile) {
        const int64_t key = __builtin_amdgcn_readlane(keyv, r);
        const int gc = lane ^ (r & 7);
        lds_load16(a.k + key * 512 + gc * 8, base + r * 1024);
        if (!VK) lds_load16(a.v + key * 512 + gc * 8, base + KM_BYTES + KR_BYTES + r * 1024);
      }
    }
    if (DR > 0) {
#pragma unroll
      for (int gi0 = 0; gi0 < kTile / 8; gi0 += 3) {
        const int gi = gi0 + wave;
        if (gi < kTile / 8) {
          const int r = gi * 8 + (lane >> 3);
          const int64_t key = __shfl(keyv, r);
          const int gc = (lane & 7) ^ (r & 7);
          lds_load16(a.kr + key * DR + gc * 8, base + KM_BYTES + gi * 8 * (DR * 2));
        }
      }
    }
  };
  // wait until at most this wave's copies of one tile are outstanding
  // (s_waitcnt with only the vector-memory count bounded; gfx9 encoding:
  // vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
  auto wait_one_tile = [&]() {
    constexpr int nr0 = (kTile + 2) / 3, nr1 = (kTile + 1) / 3, nr2 = kTile / 3;
    constexpr int g0 = DR > 0 ? 2 : 0, g12 = DR > 0 ? 1 : 0;
    constexpr int n0 = nr0 * kRowOps + g0, n1 = nr1 * kRowOps + g12, n2 = nr2 * kRowOps + g12;
    static_assert(n0 < 64 && n1 < 64 && n2 < 64, "copy counts must fit the 6-bit vmcnt field");
    if (wave == 0) __builtin_amdgcn_s_waitcnt((n0 & 15) | ((n0 >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (wave == 1) __builtin_amdgcn_s_waitcnt((n1 & 15) | ((n1 >> 4) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt((n2 & 15) | ((n2 >> 4) << 14) | (7 << 4) | (15 << 8));
  };

  // Per-lane LDS offsets (see k_row): Sᵀ / dPᵀ A operand rows 16 mb + n.
  const int x = n & 7;
  const int oA_even = n * 1024 + 16 * (g ^ x);
  const int oA_odd = n * 1024 + 16 * ((4 + g) ^ x);
  const int oR_even = n * (DR * 2) + 16 * (g ^ x);
  const int oR_odd = n * (DR * 2) + 16 * ((4 + g) ^ x);
  const int r1 = 4 * g + (n >> 2), x1 = r1 & 7;
  const int half = (n & 3) >> 1, hoff = (n & 1) * 8;
  int oT[4], oTr[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    oT[w] = r1 * 1024 + 16 * ((2 * w + half) ^ x1) + hoff;
    oTr[w] = r1 * (DR * 2) + 16 * ((2 * w + half) ^ x1) + hoff;
  }

  if (copier && cb < ce) {
    issue(key0, 0);
    if (!kSingle && ntl > 1) issue(key1, 1);
  }
  int cur = 0, it = 0;
  for (int L = 0; L < ntl; ++L, cur ^= (kSingle ? 0 : 1), ++it) {
    const int c0 = tile_at(L);
    const bool more = L + 1 < ntl;
    if (copier) {
      if (more && !kSingle) wait_one_tile();
      else __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));
    }
    __syncthreads();
    const unsigned char* Km = tbuf[cur];
    const unsigned char* Kr = Km + KM_BYTES;
    const unsigned char* Vm = VK ? Km : Km + KM_BYTES + KR_BYTES;
    // wave 3: row indices of the tile whose copies go out at the end of this
    // one (the next with one buffer, the one after with two), into LDS for
    // the copiers
    if (wave == 3 && L + kAheadTiles < ntl && lane < kTile) {
      const int c = tile_at(L + kAheadTiles) + lane;
      const int32_t kv = rt[c < ce ? c : cb];
      keys_s[lane] = kv;
      // (announce the fraction of the walk reached, for the workgroups that
      // start next)
      if (a.phase && lane == 0) {
        const int x = (c - lane - cb) / kTile;
        __hip_atomic_store(a.phase + 32 * xcd, (int32_t)(((uint32_t)x << 16) / (uint32_t)ntl), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // ---- Sᵀ (waves 0, 1) or dPᵀ (waves 2, 3) of positions 16 mb .. +15
    f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s_wave) {
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const unsigned char* p = Km + ((ks & 1) ? oA_odd : oA_even) + 128 * (ks >> 1) + mb * 16384;
        r = TT::mfma(as_vec8<V8>(*(const uint4*)p), Bf[ks], r);
      }
      if (DR > 0) {
        r = TT::mfma(as_vec8<V8>(*(const uint4*)(Kr + oR_even + mb * 16 * (DR * 2))), Bf[KS_QK - 2], r);
        r = TT::mfma(as_vec8<V8>(*(const uint4*)(Kr + oR_odd + mb * 16 * (DR * 2))), Bf[KS_QK - 1], r);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS_V; ++ks) {
        const unsigned char* p = Vm + ((ks & 1) ? oA_odd : oA_even) + 128 * (ks >> 1) + mb * 16384;
        r = TT::mfma(as_vec8<V8>(*(const uint4*)p), Bf[ks], r);
      }
      // dPᵀ of head n, positions 16 mb + 4g .. +3
      *(f32x4*)(xdp + n * XSTR + 16 * mb + 4 * g) = r;
    }
    __syncthreads();
    // ---- P and dS (waves 0, 1)
    if (s_wave) {
      const f32x4 dp = *(const f32x4*)(xdp + n * XSTR + 16 * mb + 4 * g);
      const float dl = delta_s[n];
      uint16_t pv[4], dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * mb + 4 * g + i;   // position within the tile
        const bool ok = live && (c0 + j < nv);
        const float p = ok ? exp2f(r[i] * a.scale_log2 - mlog) * inv_l : 0.f;
        pv[i] = TT::from_f(p);
        dsv[i] = TT::from_f(p * (dp[i] - dl) * a.ds_scale);
        stg[it & 1][0][j * 16 + n] = pv[i];
        stg[it & 1][1][j * 16 + n] = dsv[i];
      }
      *(uint2*)(dsT + n * DSTR + 16 * mb + 4 * g) =
          make_uint2(dsv[0] | ((uint32_t)dsv[1] << 16), dsv[2] | ((uint32_t)dsv[3] << 16));
    }
    __syncthreads();
    // ---- P and dS rows of the tile to memory (wave 3)
    if (wave == 3) {
      const int which = lane >> 5, j = lane & 31;
      if (c0 + j < nv) {
        const uint4* src = (const uint4*)(stg[it & 1][which] + j * 16);
        uint16_t* out = (which ? a.ds_out : a.p_out) + (tl * a.E + c0 + j) * 16;
        ((uint4*)out)[0] = src[0];
        ((uint4*)out)[1] = src[1];
      }
    }
    // ---- dQ += dS·K over the tile's 32 positions, this wave's column blocks
    {
      const uint2 lo = *(const uint2*)(dsT + n * DSTR + 4 * g);
      const uint2 hi = *(const uint2*)(dsT + n * DSTR + 16 + 4 * g);
      const V8 A8 = as_vec8<V8>(make_uint4(lo.x, lo.y, hi.x, hi.y));
      auto kread = [&](int nb) -> V8 {
        const unsigned char* p1 = nb < 32 ? Km + oT[nb & 3] + 128 * (nb >> 2) : Kr + oTr[nb & 3];
        const unsigned char* p2 = p1 + (nb < 32 ? 16 * 1024 : 16 * (DR * 2));
        return join_tr<V8>(lds_read_tr((const uint16_t*)p1), lds_read_tr((const uint16_t*)p2));
      };
#pragma unroll
      for (int j = 0; j < NBW; ++j) acc[j] = TT::mfma(A8, kread(wave + 4 * j), acc[j]);
    }
    __syncthreads();
    // every wave is done with this buffer: the copies of the next tile (one
    // buffer) or the one after (two)
    if (copier && L + kAheadTiles < ntl) {
      const int32_t keyv = keys_s[lane & 31];
      issue(keyv, cur);
    }
  }

  // ---- dQ | dQrope: column blocks wave, wave + 4, ... -----------------------
  if (a.n_split > 1) {
    if (cb >= ce) return;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int col = 16 * (wave + 4 * j) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * g + i;
        if (hh < a.G) atomicAdd(a.dq_acc + (tl * a.G + hh) * DQK + col, acc[j][i]);
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int col = 16 * (wave + 4 * j) + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * g + i;
      if (hh < a.G) {
        const uint16_t v = TT::from_f(acc[j][i] * a.dq_mul);
        if (col < 512) a.dq[(t * a.G + hh) * 512 + col] = v;
        else a.dqr[(t * a.G + hh) * DR + (col - 512)] = v;
      }
    }
  }
}

void launch_row(int32_t dtype, bool rope, const RowArgs& a, hipStream_t s) {
  if (a.ntok == 0) return;
  const int64_t per = (int64_t)kXcds * kRun;
  const int64_t padded = (a.ntok + per - 1) / per * per;
  const dim3 grid((unsigned)(padded * a.n_hb * a.n_split)), block(256);
  // value passed as the key tensor itself: gather each row once
  const bool vk = a.v == a.k;
  if (a.Gp == 16) {   // up to 16 heads: all four waves share a token's tiles
    const dim3 grid16((unsigned)(padded * a.n_split));
    auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid16, block, 0, s, a); };
    if (dtype == SFAG_BF16) {
      if (rope) vk ? go(k_row16<BF16, 64, true>) : go(k_row16<BF16, 64, false>);
      else vk ? go(k_row16<BF16, 0, true>) : go(k_row16<BF16, 0, false>);
    } else {
      if (rope) vk ? go(k_row16<FP16, 64, true>) : go(k_row16<FP16, 64, false>);
      else vk ? go(k_row16<FP16, 0, true>) : go(k_row16<FP16, 0, false>);
    }
    return;
  }
  if (dtype == SFAG_BF16) {
    if (rope) {
      if (vk) hipLaunchKernelGGL((k_row<BF16, 64, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_row<BF16, 64, false>), grid, block, 0, s, a);
    } else {
      if (vk) hipLaunchKernelGGL((k_row<BF16, 0, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_row<BF16, 0, false>), grid, block, 0, s, a);
    }
  } else {
    if (rope) {
      if (vk) hipLaunchKernelGGL((k_row<FP16, 64, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_row<FP16, 64, false>), grid, block, 0, s, a);
    } else {
      if (vk) hipLaunchKernelGGL((k_row<FP16, 0, true>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((k_row<FP16, 0, false>), grid, block, 0, s, a);
    }
  }
}

}  // namespace sfag
