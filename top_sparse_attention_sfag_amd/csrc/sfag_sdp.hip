// Token-centric kernels for N1 >= 32 heads (operator page
// "aclnnSparseFlashAttentionGrad", 功能说明 stages 1-3), split so that neither
// holds more registers than the matrix cores can be fed from:
//
//   k_sdp  (token x up to 128 heads): S = Q·Kᵀ and dP = dO·Vᵀ with
//          v_mfma_f32_32x32x16 (32 heads x 32 positions per wave), then
//          P = exp(scale·S − max)/sum and dS = P ∘ (dP − Delta), stored as
//          16-bit (token, position, head) rows straight from registers (each
//          lane holds 4 consecutive heads of one position per group).  Each
//          wave keeps its 32 heads' Q and dO fragments in registers; the 32
//          gathered K|Krope|V rows of a tile arrive in LDS through
//          global_load_lds_dwordx4, double buffered, 16-byte chunks
//          XOR-swizzled by row.
//   k_dq   (token x 128 heads): dQ = scale·dS·K_sel.  Each wave owns every
//          fourth 16-column block of dQ|dQrope for 64 heads, so a tile's K rows
//          and dS rows are both read once per wave: K columns and dS head
//          groups come out of LDS transposed with ds_read_b64_tr_b16.
#include <algorithm>
#include <type_traits>

#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

namespace {

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;
constexpr int kXcds = 8;
constexpr int kRun = 16;

// Asynchronous global -> LDS copy of 16 bytes per lane (lane l writes at the
// wave-uniform LDS address l_base + 16 l).  Inline asm on purpose: the
// compiler does not track it, so it adds no waits of its own before LDS reads
// of the other buffer; reads of copied data follow an explicit s_waitcnt and
// a barrier.  The copy starts with one wait state (s_nop 0): on this chip
// family an LDS DMA that reads M0 right after a scalar write of M0 needs one,
// and the compiler inserts it only for DMA instructions it emits itself.
__device__ __forceinline__ void lds_load16(const void* g, const void* l) {
  const uint32_t la = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) unsigned char*)l);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(la)) : "memory");
}

// Same, with the LDS address given as a 32-bit offset.
__device__ __forceinline__ void lds_load16_at(const void* g, uint32_t la) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(la)) : "memory");
}
__device__ __forceinline__ uint32_t lds_off(const void* l) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) unsigned char*)l);
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its outstanding copies; the signal fences keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4));   // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename TT>
__device__ __forceinline__ f32x16 mfma32(typename TT::vec8 a, typename TT::vec8 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<FP16>(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 64-head blocks in the 4-wave form of k_sdp8 (else k_sdp with 2 waves of 32)
constexpr bool kSdp16x4 = true;
// at most 64 heads on the caller's stream: k_dq as 4 waves (else 8 waves,
// half of them on zero dS)
constexpr bool kDq64x4 = true;

// Maps a block index to (token of the chunk, head block): each XCD takes runs
// of kRun consecutive tokens.
// With `reverse` the last tokens of the chunk come first (under the causal
// mask they hold the most positions, so the longest units start first and the
// shortest fill the end).
__device__ __forceinline__ int64_t unit_token(int b, int n_hb, int& hb, int64_t ntok, int reverse) {
  const int xcd = b % kXcds, u = b / kXcds;
  hb = u % n_hb;
  const int tq = u / n_hb;
  const int64_t tl = ((int64_t)(tq / kRun) * kXcds + xcd) * kRun + (tq % kRun);
  if (!reverse) return tl;
  const int64_t padded = (ntok + kXcds * kRun - 1) / (kXcds * kRun) * (kXcds * kRun);
  return padded - 1 - tl;
}

// Row indices of a tile: lane r & 31 holds the key row of position c0 + r
// (positions past nv repeat position 0; their P and dS are 0).  Loaded a
// tile ahead of the gather that uses them.
__device__ __forceinline__ int32_t tile_keys(const int32_t* rt, int nv, int c0, int lane) {
  const int cl = c0 + (lane & 31);
  return cl < nv ? rt[cl] : (nv > 0 ? rt[0] : 0);
}

// Issue the async gather of one tile (rows of keyv, see tile_keys).  K main
// rows (1024 B) and, when WITH_V, V rows go one row per instruction; rope
// rows (DR*2 bytes) go 8 per instruction.  Every wave of the block takes a
// share.  The lane writing 16-byte position p of row r fetches chunk
// p ^ swz(r): with WIDE, swz = r & 15 for the 1024-byte rows and
// (r >> 1) & 7 for the rope rows (16 consecutive rows then fill all 64 LDS
// banks when read one chunk per row); otherwise r & 7 for both.
template <int DR, bool WITH_V, bool WIDE>
__device__ __forceinline__ void issue_rows(const uint16_t* k, const uint16_t* kr, const uint16_t* v, int32_t keyv,
                                           unsigned char* base, int km_bytes, int kr_bytes, int wave, int nw,
                                           int lane) {
  for (int r = wave; r < kTile; r += nw) {
    const int64_t key = __builtin_amdgcn_readlane(keyv, r);
    const int gc = lane ^ (r & (WIDE ? 15 : 7));
    lds_load16(k + key * 512 + gc * 8, base + r * 1024);
    if (WITH_V) lds_load16(v + key * 512 + gc * 8, base + km_bytes + kr_bytes + r * 1024);
  }
  if (DR > 0) {
    for (int gi = wave; gi < kTile / 8; gi += nw) {
      const int r = gi * 8 + (lane >> 3);
      const int64_t key = __shfl(keyv, r);
      const int gc = (lane & 7) ^ (WIDE ? ((r >> 1) & 7) : (r & 7));
      lds_load16(kr + key * DR + gc * 8, base + km_bytes + gi * 8 * (DR * 2));
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// k_sdp: blockDim = 64 * nw, nw = min(4, Gp / 32); head block = 32 * nw heads.
// ---------------------------------------------------------------------------
template <typename TT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)TT::from_f(lo) | ((uint32_t)TT::from_f(hi) << 16);
}

// VK: value is the key tensor itself (the operator page's supported case):
// one K|Krope row per position is gathered and its first 512 columns serve as
// the V row, read once for both the S and the dP chains.
template <typename TT, int DR, int NW, bool VK>
__global__ void __launch_bounds__(256, 1) k_sdp(RowArgs a) {
  constexpr int DQK = 512 + DR;
  constexpr int KS_QK = DQK / 16;   // k-steps of 16 along D+Dr
  constexpr int KS_V = 512 / 16;
  constexpr int KM_BYTES = kTile * 1024;
  constexpr int KR_BYTES = kTile * DR * 2;
  constexpr int BUF = KM_BYTES + KR_BYTES + (VK ? 0 : kTile * 1024);
  typedef typename TT::vec8 V8;

  // Two tile buffers as separate LDS objects.  With fewer than four waves and
  // a separate V (68 KB per tile) one buffer is used, so that two workgroups
  // share a CU and each hides the other's gathers: a tile's copies are issued
  // once every wave has read the buffer, and land during its P/dS work.
  constexpr bool kSingle = NW < 4 && !VK;
  __shared__ __attribute__((aligned(16))) unsigned char buf0[BUF];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[kSingle ? 16 : BUF];

  constexpr int nw = NW;
  const int HB = 32 * nw;
  int hb;
  const int64_t tl = unit_token(blockIdx.x, a.n_hb, hb, a.ntok, a.reverse);
  if (tl >= a.ntok) return;
  const int64_t t = a.t0 + tl;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hi = lane & 31, kg = lane >> 5;   // row of the A operand, k-group
  const int h0 = hb * HB + wave * 32;
  const int h = h0 + hi;
  const bool hv = h < a.G;

  // Delta = rowsum(dO ∘ O) of head h (功能说明 stage 2): this lane's 256
  // columns (chunks 2ks + kg) against O, fp32, then the other half from lane
  // ^ 32; lanes 0..31 then hold heads h0 .. h0 + 31.
  // (dO is read again here, from L2, a few chunks at a time, so that O and
  // dO are not all held in registers next to the operands)
  float dsum = 0.f;
  if (hv) {
    const uint16_t* orow = a.o + (t * a.G + h) * 512 + 8 * kg;
    const uint16_t* drow = a.dO + (t * a.G + h) * 512 + 8 * kg;
#pragma unroll 2
    for (int ks = 0; ks < KS_V; ++ks) {
      const uint4 ov = *(const uint4*)(orow + 16 * ks);
      const uint4 dv = *(const uint4*)(drow + 16 * ks);
      const uint16_t* po = (const uint16_t*)&ov;
      const uint16_t* pd = (const uint16_t*)&dv;
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum = fmaf(TT::to_f(pd[j]), TT::to_f(po[j]), dsum);
    }
  }
  dsum += __shfl_xor(dsum, 32);
  // A operands: Q and dO rows of head h, 8 consecutive columns per k-step.
  V8 Qf[KS_QK], dOf[KS_V];
#pragma unroll
  for (int ks = 0; ks < KS_QK; ++ks) {
    const int d0 = 16 * ks + 8 * kg;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hv) {
      if (d0 < 512) v = *(const uint4*)(a.q + (t * a.G + h) * 512 + d0);
      else v = *(const uint4*)(a.qr + (t * a.G + h) * DR + (d0 - 512));
    }
    Qf[ks] = as_vec8<V8>(v);
  }
#pragma unroll
  for (int ks = 0; ks < KS_V; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hv) v = *(const uint4*)(a.dO + (t * a.G + h) * 512 + 16 * ks + 8 * kg);
    dOf[ks] = as_vec8<V8>(v);
  }
  // S = Q·Kᵀ and dP = dO·Vᵀ come out as (32 heads x 32 positions): lane l
  // holds position l % 32 and heads h0 + 8(i/4) + 4kg + i%4, i = 0..15.
  // Per head: P = exp2(scale·log2e·S − mb), mb = log2e·max + log2(sum)
  // (+inf for heads past G or with an empty row, which gives P = 0).
  float mb[16], dl[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int hh = h0 + 8 * (i >> 2) + 4 * kg + (i & 3);
    mb[i] = __builtin_inff();
    dl[i] = __shfl(dsum, hh - h0);
    if (hh < a.G) {
      const float m = a.smax[t * a.G + hh], l = a.ssum[t * a.G + hh];
      if (l > 0.f) mb[i] = m * kLog2e + __log2f(l);
    } else {
      dl[i] = 0.f;
    }
  }
  const int nv = a.nvalid[tl];
  const int32_t* rt = a.rows + tl * a.E;
  // B operand rows: position m = lane & 31 of the tile, chunk 2ks + kg.
  const int m = hi;
  const int x = m & 15, xr = (m >> 1) & 7;   // swizzles of the K|V and rope rows
  const int oK = m * 1024;
  const int oR = m * (DR * 2);

  int32_t keys = tile_keys(rt, nv, 0, lane);   // row indices of the next tile to gather
  // P and dS of the previous tile, packed, stored at the start of the next
  // tile (before its gather is issued, so that waiting for that gather also
  // covers these stores, issued a whole tile earlier)
  uint2 pend_p[4], pend_ds[4];
  int pend_pos = -1;
  // store j of 8: P (j even) or dS (j odd) of head group j / 2
  auto store_one = [&](int j) {
    const int q4 = j >> 1;
    const int hh0 = h0 + 8 * q4 + 4 * kg;
    if (pend_pos >= 0 && pend_pos < nv && hh0 < a.Gp) {
      const int64_t o = (tl * a.E + pend_pos) * a.Gp + hh0;
      if (j & 1) *(uint2*)(a.ds_out + o) = pend_ds[q4];
      else *(uint2*)(a.p_out + o) = pend_p[q4];
    }
  };
  auto store_pending = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) store_one(j);
  };
  // Four waves (128 heads, whole rows): P and dS of a tile are staged in LDS
  // as (tensor, position) rows of 256 bytes and leave as 1 KB coalesced
  // stores of 4 rows.  Chunk j of row r sits at chunk j ^ (r & 15), and the
  // two 8-byte halves of a chunk are swapped in rows 16..31, so that the
  // 8-byte writes of 32 lanes (32 rows, one head group) hit distinct banks.
  constexpr bool kStage = NW == 4;
  __shared__ __attribute__((aligned(16))) unsigned char stg[kStage ? 2 * kTile * 256 : 16];
  uint4 pst[4];          // staged rows read back by this wave: tensor wave / 2, rows 16 (wave & 1) + 4 i + lane / 16
  int stg_c0 = -1;       // first position of the staged tile, -1 if none
  const int srow0 = 16 * (wave & 1) + (lane >> 4), sj = lane & 15;
  auto stage_read = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = srow0 + 4 * i;
      uint4 v = *(const uint4*)(stg + ((wave >> 1) * kTile + r) * 256 + ((sj ^ (r & 15)) << 4));
      pst[i] = (wave & 1) ? make_uint4(v.z, v.w, v.x, v.y) : v;
    }
  };
  auto stage_store = [&](int i) {
    const int pos = stg_c0 + srow0 + 4 * i;
    if (stg_c0 >= 0 && pos < nv) {
      uint16_t* out = (wave >> 1) ? a.ds_out : a.p_out;
      *(uint4*)(out + (tl * a.E + pos) * a.Gp + sj * 8) = pst[i];
    }
  };
  auto stage_write = [&]() {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int j = 4 * wave + q4;
      const int o = m * 256 + ((j ^ (m & 15)) << 4) + ((kg ^ (m >> 4)) << 3);
      *(uint2*)(stg + o) = pend_p[q4];
      *(uint2*)(stg + kTile * 256 + o) = pend_ds[q4];
    }
  };
  // The gather of a tile as a fixed list of copy instructions per wave: K
  // and V rows wave + nw*j (two each), then rope groups wave + nw*j (8 rows
  // each); entries past the tile's rows (nw = 3) are skipped.
  constexpr int kPerRow = VK ? 1 : 2;   // copies per K(|V) row
  constexpr int kRowOps = kPerRow * ((kTile + nw - 1) / nw);
  constexpr int kOps = kRowOps + (DR > 0 ? (kTile / 8 + nw - 1) / nw : 0);
  auto issue_op = [&](int i, int32_t keyv, uint32_t base) {
    if (i < kRowOps) {
      const int r = wave + nw * (i / kPerRow);
      if (r < kTile) {
        const int64_t key = __builtin_amdgcn_readlane(keyv, r);
        const int gc = lane ^ (r & 15);
        if (!VK && (i & 1)) lds_load16_at(a.v + key * 512 + gc * 8, base + KM_BYTES + KR_BYTES + r * 1024);
        else lds_load16_at(a.k + key * 512 + gc * 8, base + r * 1024);
      }
    } else {
      const int gi = wave + nw * (i - kRowOps);
      if (gi < kTile / 8) {
        const int r = gi * 8 + (lane >> 3);
        const int64_t key = __shfl(keyv, r);
        const int gc = (lane & 7) ^ ((r >> 1) & 7);
        lds_load16_at(a.kr + key * DR + gc * 8, base + KM_BYTES + gi * 8 * (DR * 2));
      }
    }
  };

  auto tile = [&](int c0, const unsigned char* Km, unsigned char* nxt) {
    // (the previous tile's MFMAs stay above this wait: the wait stalls issue)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kStage && stg_c0 >= 0) stage_read();
    const bool more = c0 + kTile < nv;
    const uint32_t nxt_l = lds_off(nxt);
    // With fewer than four waves (more copies per wave) the copies go out
    // here at once; spreading them would cost registers.
    constexpr bool kSpread = NW == 4;
    if (!kSpread && !kSingle && more)
      issue_rows<DR, !VK, true>(a.k, a.kr, a.v, keys, nxt, KM_BYTES, KR_BYTES, wave, nw, lane);
    // single buffer: the next tile's copies once every wave has read this one
    // (with the row indices of the next tile, taken before `keys` advances)
    const int32_t keys_next = keys;
    auto issue_single = [&]() {
      if (kSingle && more) {
        bar();
        issue_rows<DR, !VK, true>(a.k, a.kr, a.v, keys_next, nxt, KM_BYTES, KR_BYTES, wave, nw, lane);
      }
    };
    const unsigned char* Kr = Km + KM_BYTES;
    const unsigned char* Vm = VK ? Km : Kr + KR_BYTES;
    f32x16 S, P;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = P[i] = 0.f;
    // S over D and dP over D as two interleaved chains (independent MFMAs
    // back to back), operand reads issued two k-steps ahead, then S over Dr
    uint4 kv[3], vv[3];
    auto rd = [&](int ks, int slot) {
      const int ch = 2 * ks + kg;
      kv[slot] = *(const uint4*)(Km + oK + ((ch ^ x) << 4));
      vv[slot] = VK ? kv[slot] : *(const uint4*)(Vm + oK + ((ch ^ x) << 4));
    };
    rd(0, 0);
    rd(1, 1);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      if (ks + 2 < 32) rd(ks + 2, (ks + 2) % 3);
      // the next tile's copies over the first 8 k-steps (two or three per
      // k-step: early enough to land before the next tile, spread enough not
      // to stall the wave) and the previous tile's stores over the last 8,
      // between the MFMAs
      if (kSpread && more && ks < 8)
        #pragma unroll
        for (int i = ks * kOps / 8; i < (ks + 1) * kOps / 8; ++i) issue_op(i, keys, nxt_l);
      if (kStage) {
        if (ks >= 24 && ks < 28) stage_store(ks - 24);
      } else if (ks >= 24) {
        store_one(ks - 24);
      }
      S = mfma32<TT>(Qf[ks], as_vec8<V8>(kv[ks % 3]), S);
      P = mfma32<TT>(dOf[ks], as_vec8<V8>(vv[ks % 3]), P);
      __builtin_amdgcn_sched_barrier(0);
    }
    keys = tile_keys(rt, nv, c0 + 2 * kTile, lane);
    if (DR > 0) {
      uint4 bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 2 * j + kg;
        bv[j] = *(const uint4*)(Kr + oR + ((ch ^ xr) << 4));
      }
      issue_single();
#pragma unroll
      for (int j = 0; j < 4; ++j) S = mfma32<TT>(Qf[32 + j], as_vec8<V8>(bv[j]), S);
    } else {
      issue_single();
    }
    // P and dS of position c0 + m for the lane's 16 heads
    const bool valid = c0 + m < nv;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float pv[4], dv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = 4 * q4 + jj;
        float p = __builtin_amdgcn_exp2f(S[i] * a.scale_log2 - mb[i]);
        p = valid ? p : 0.f;
        pv[jj] = p;
        dv[jj] = p * (P[i] - dl[i]) * a.ds_scale;
      }
      pend_p[q4] = make_uint2(pack2<TT>(pv[0], pv[1]), pack2<TT>(pv[2], pv[3]));
      pend_ds[q4] = make_uint2(pack2<TT>(dv[0], dv[1]), pack2<TT>(dv[2], dv[3]));
    }
    if (kStage) {
      bar();   // every wave has read the previous staged tile back
      stage_write();
      stg_c0 = c0;
    } else {
      pend_pos = c0 + m;
    }
  };

  if (nv > 0) issue_rows<DR, !VK, true>(a.k, a.kr, a.v, keys, buf0, KM_BYTES, KR_BYTES, wave, nw, lane);
  keys = tile_keys(rt, nv, kTile, lane);
  for (int c0 = 0; c0 < nv; c0 += 2 * kTile) {
    if (kSingle) {
      tile(c0, buf0, buf0);
      if (c0 + kTile < nv) tile(c0 + kTile, buf0, buf0);
    } else {
      tile(c0, buf0, buf1);
      if (c0 + kTile < nv) tile(c0 + kTile, buf1, buf0);
    }
  }
  if (kStage) {
    __syncthreads();
    if (stg_c0 >= 0) {
      stage_read();
#pragma unroll
      for (int i = 0; i < 4; ++i) stage_store(i);
    }
  } else {
    store_pending();
  }
}

// ---------------------------------------------------------------------------
// k_sdp8: the same for a block of 128 heads as 8 waves of 16 heads, two waves
// per SIMD.  With 16 heads a wave holds its Q and dO rows in 136 registers
// (32 heads need 272, which leaves one wave per SIMD), so each SIMD has a
// second wave whose MFMAs run while the first waits.  S and dP of a tile
// come from v_mfma_f32_16x16x32 (16 heads x 16 positions, two position
// blocks); lane (g, n) then holds heads 4g .. 4g + 3 of the wave at position
// n of each block.  Every wave reads the whole tile from LDS, twice the LDS
// traffic of 32-head waves.
//
// NW = 4 takes a block of 64 heads the same way (4 waves of 16) with one
// tile buffer, so that two workgroups share a CU (two waves per SIMD again):
// the next tile's copies go out once every wave has read the buffer, and the
// other workgroup's work covers their latency.
// ---------------------------------------------------------------------------
template <typename TT, int DR, bool VK, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) k_sdp8(RowArgs a) {
  constexpr int DQK = 512 + DR;
  constexpr int KS_QK = DQK / 32;   // k-steps of 32 along D+Dr (rope last)
  constexpr int KS_V = 512 / 32;
  constexpr int KM_BYTES = kTile * 1024;
  constexpr int KR_BYTES = kTile * DR * 2;
  constexpr int BUF = KM_BYTES + KR_BYTES + (VK ? 0 : kTile * 1024);
  constexpr bool kOne = NW == 4;        // one tile buffer
  constexpr int SRB = 32 * NW;          // bytes of a staged (tensor, position) row: 16 NW heads
  constexpr int SCM = 2 * NW - 1;       // chunk swizzle mask of the staged rows
  typedef typename TT::vec8 V8;
  __shared__ __attribute__((aligned(16))) unsigned char buf0[BUF];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[kOne ? 16 : BUF];
  // P and dS of a tile as (tensor, position) rows of the block's heads
  // (SRB bytes); 16-byte chunk j of row r sits at chunk j ^ (r & SCM)
  __shared__ __attribute__((aligned(16))) unsigned char stg[2 * kTile * SRB];

  int hb;
  const int64_t tl = unit_token(blockIdx.x, 1, hb, a.ntok, a.reverse);
  if (tl >= a.ntok) return;
  const int64_t t = a.t0 + tl;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int h0 = 16 * wave;
  const int h = h0 + n;
  const bool hv = h < a.G;

  // Delta of head h: lane (g, n) sums columns 128g .. 128g + 127 of dO ∘ O,
  // the four lanes of head n then add up (功能说明 stage 2)
  float dsum = 0.f;
  if (hv) {
    const uint16_t* orow = a.o + (t * a.G + h) * 512 + 128 * g;
    const uint16_t* drow = a.dO + (t * a.G + h) * 512 + 128 * g;
#pragma unroll 4
    for (int c = 0; c < 16; ++c) {
      const uint4 ov = *(const uint4*)(orow + 8 * c);
      const uint4 dv = *(const uint4*)(drow + 8 * c);
      const uint16_t* po = (const uint16_t*)&ov;
      const uint16_t* pd = (const uint16_t*)&dv;
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum = fmaf(TT::to_f(pd[j]), TT::to_f(po[j]), dsum);
    }
  }
  dsum += __shfl_xor(dsum, 16);
  dsum += __shfl_xor(dsum, 32);
  // A operands: Q|Qrope and dO of head h, columns 32ks + 8g .. +8
  V8 Qf[KS_QK], dOf[KS_V];
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
#pragma unroll
  for (int ks = 0; ks < KS_V; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (hv) v = *(const uint4*)(a.dO + (t * a.G + h) * 512 + 32 * ks + 8 * g);
    dOf[ks] = as_vec8<V8>(v);
  }
  // output heads of this lane: h0 + 4g + i
  float mb[4], dl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = h0 + 4 * g + i;
    mb[i] = __builtin_inff();
    dl[i] = __shfl(dsum, 4 * g + i);
    if (hh < a.G) {
      const float m = a.smax[t * a.G + hh], l = a.ssum[t * a.G + hh];
      if (l > 0.f) mb[i] = m * kLog2e + __log2f(l);
    } else {
      dl[i] = 0.f;
    }
  }
  const int nv = a.nvalid[tl];
  const int32_t* rt = a.rows + tl * a.E;
  int32_t keys = tile_keys(rt, nv, 0, lane);   // row indices of the next tile to gather

  // The gather of a tile as a fixed list of copy instructions per wave: K
  // (and V) rows wave + NW j, then rope group `wave` (waves 0..3, 8 rows each).
  constexpr int kPerRow = VK ? 1 : 2;
  constexpr int kRowOps = kPerRow * (kTile / NW);
  constexpr int kOps = kRowOps + (DR > 0 ? 1 : 0);
  // (rkey: this lane's rope row key, rope_key(keyv), formed before the MFMA
  // loop: a lane shuffle there would wait on LDS and so also on the operand
  // reads issued ahead of the MFMAs)
  auto rope_key = [&](int32_t keyv) -> int32_t {
    return DR > 0 ? __shfl(keyv, (wave & 3) * 8 + (lane >> 3)) : 0;
  };
  auto issue_op = [&](int i, int32_t keyv, int32_t rkey, uint32_t base) {
    if (i < kRowOps) {
      const int r = wave + NW * (i / kPerRow);
      const int64_t key = __builtin_amdgcn_readlane(keyv, r);
      const int gc = lane ^ (r & 15);
      if (!VK && (i & 1)) lds_load16_at(a.v + key * 512 + gc * 8, base + KM_BYTES + KR_BYTES + r * 1024);
      else lds_load16_at(a.k + key * 512 + gc * 8, base + r * 1024);
    } else if (wave < kTile / 8) {
      const int r = wave * 8 + (lane >> 3);
      const int gc = (lane & 7) ^ ((r >> 1) & 7);
      lds_load16_at(a.kr + (int64_t)rkey * DR + gc * 8, base + KM_BYTES + wave * 8 * (DR * 2));
    }
  };
  // staged rows stored by this wave: tensor wave / (NW / 2), rows
  // 8 (wave % (NW / 2)) + SR q + lane / (2 NW) (q = 0, 1; SR = 32 / NW rows
  // per instruction), chunk lane % (2 NW)
  int stg_c0 = -1;
  constexpr int SR = 32 / NW;
  const int sten = wave / (NW / 2);
  const int srow0 = 8 * (wave % (NW / 2)) * (8 / NW) + lane / (2 * NW), sj = lane % (2 * NW);
  auto stage_out = [&]() {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = srow0 + SR * q;
      const uint4 v = *(const uint4*)(stg + (sten * kTile + r) * SRB + ((sj ^ (r & SCM)) << 4));
      uint16_t* out = (sten ? a.ds_out : a.p_out) + (tl * a.E + stg_c0 + r) * a.Gp + sj * 8;
      if (stg_c0 + r < nv) *(uint4*)out = v;
    }
  };
  // LDS offsets of this lane's B-operand reads: row 16 nb + n, chunk
  // 4 ks + g (K|V rows, swizzle r & 15) or 4 ks' + g (rope rows, (r >> 1) & 7)
  auto kofs = [&](int nb, int ks) -> int {
    const int r = 16 * nb + n;
    return r * 1024 + (((4 * ks + g) ^ (r & 15)) << 4);
  };
  auto rofs = [&](int nb, int ks) -> int {
    const int r = 16 * nb + n;
    return r * (DR * 2) + (((4 * ks + g) ^ ((r >> 1) & 7)) << 4);
  };

  auto tile = [&](int c0, const unsigned char* Km, unsigned char* nxt) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the previous tile's P and dS rows: read back and stored at once, so
    // that they hold no registers through the MFMA loop
    if (stg_c0 >= 0) stage_out();
    const bool more = c0 + kTile < nv;
    const int32_t rkey = rope_key(keys);
    const uint32_t nxt_l = lds_off(nxt);
    const unsigned char* Kr = Km + KM_BYTES;
    const unsigned char* Vm = VK ? Km : Kr + KR_BYTES;
    f32x4 S[2], P[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) S[nb] = P[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operand reads one k-step ahead with value = key; with separate V rows
    // (twice the operand registers) in the k-step itself, the other wave of
    // the SIMD covering their latency
    constexpr int LA = VK ? 1 : 0;
    uint4 kv[LA + 1][2], vv[LA + 1][2];
    auto rd = [&](int ks, int slot) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        kv[slot][nb] = *(const uint4*)(Km + kofs(nb, ks));
        vv[slot][nb] = VK ? kv[slot][nb] : *(const uint4*)(Vm + kofs(nb, ks));
      }
    };
    if (LA) rd(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS_V; ++ks) {
      if (!LA) rd(ks, 0);
      else if (ks + 1 < KS_V) rd(ks + 1, (ks + 1) & LA);
      // the next tile's copies over the first 8 k-steps (two buffers)
      if (!kOne && more && ks < 8)
#pragma unroll
        for (int i = ks * kOps / 8; i < (ks + 1) * kOps / 8; ++i) issue_op(i, keys, rkey, nxt_l);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        S[nb] = TT::mfma(Qf[ks], as_vec8<V8>(kv[ks & LA][nb]), S[nb]);
        P[nb] = TT::mfma(dOf[ks], as_vec8<V8>(vv[ks & LA][nb]), P[nb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!kOne) keys = tile_keys(rt, nv, c0 + 2 * kTile, lane);
    if constexpr (DR > 0) {
      uint4 bv[KS_QK - KS_V][2];
#pragma unroll
      for (int ks = 0; ks < KS_QK - KS_V; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bv[ks][nb] = *(const uint4*)(Kr + rofs(nb, ks));
#pragma unroll
      for (int ks = 0; ks < KS_QK - KS_V; ++ks)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) S[nb] = TT::mfma(Qf[KS_V + ks], as_vec8<V8>(bv[ks][nb]), S[nb]);
    }
    // P and dS of positions c0 + 16 nb + n, heads h0 + 4g .. +3
    uint2 wp[2], wd[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bool valid = c0 + 16 * nb + n < nv;
      float pv[4], dv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(S[nb][i] * a.scale_log2 - mb[i]);
        p = valid ? p : 0.f;
        pv[i] = p;
        dv[i] = p * (P[nb][i] - dl[i]) * a.ds_scale;
      }
      wp[nb] = make_uint2(pack2<TT>(pv[0], pv[1]), pack2<TT>(pv[2], pv[3]));
      wd[nb] = make_uint2(pack2<TT>(dv[0], dv[1]), pack2<TT>(dv[2], dv[3]));
    }
    bar();   // every wave has read the previous staged tile back (and, with one
             // buffer, is done with this tile's operands)
    if (kOne && more) {
#pragma unroll
      for (int i = 0; i < kOps; ++i) issue_op(i, keys, rkey, nxt_l);
      keys = tile_keys(rt, nv, c0 + 2 * kTile, lane);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int r = 16 * nb + n;
      const int o = r * SRB + (((2 * wave + (g >> 1)) ^ (r & SCM)) << 4) + ((g & 1) << 3);
      *(uint2*)(stg + o) = wp[nb];
      *(uint2*)(stg + kTile * SRB + o) = wd[nb];
    }
    stg_c0 = c0;
  };

  if (nv > 0) {
    const uint32_t b0 = lds_off(buf0);
    const int32_t rkey0 = rope_key(keys);
#pragma unroll
    for (int i = 0; i < kOps; ++i) issue_op(i, keys, rkey0, b0);
  }
  keys = tile_keys(rt, nv, kTile, lane);
  if constexpr (kOne) {
    for (int c0 = 0; c0 < nv; c0 += kTile) tile(c0, buf0, buf0);
  } else {
    for (int c0 = 0; c0 < nv; c0 += 2 * kTile) {
      tile(c0, buf0, buf1);
      if (c0 + kTile < nv) tile(c0 + kTile, buf1, buf0);
    }
  }
  __syncthreads();
  if (stg_c0 >= 0) stage_out();
}

// ---------------------------------------------------------------------------
// k_dq: 512 threads; head block of 128 heads; wave w takes heads
// 64 (w / 4) .. +64 of the block and the 16-column blocks w % 4, w % 4 + 4,
// ... of dQ|dQrope (blocks 32..35 are the rope columns).
// ---------------------------------------------------------------------------
template <typename TT, int DR, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) k_dq(RowArgs a) {
  constexpr int DQK = 512 + DR;
  constexpr int NB = DQK / 64;             // column blocks per wave
  constexpr int KM_BYTES = kTile * 1024;
  constexpr int KR_BYTES = kTile * DR * 2;
  constexpr int HBW = 16 * NW;             // heads per block: 128 (8 waves) or 64 (4 waves)
  constexpr int DSR = 2 * HBW;             // bytes of a dS row
  constexpr int DCM = 2 * NW - 1;          // chunk swizzle mask of the dS rows
  constexpr int DS_BYTES = kTile * DSR;    // 32 positions x the block's heads, 16-bit
  constexpr int BUF = KM_BYTES + KR_BYTES + DS_BYTES;
  typedef typename TT::vec8 V8;

  __shared__ __attribute__((aligned(16))) unsigned char buf0[BUF];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[BUF];

  int hb;
  const int64_t tl = unit_token(blockIdx.x, a.n_hb, hb, a.ntok, a.reverse);
  if (tl >= a.ntok) return;
  const int64_t t = a.t0 + tl;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index(), g = lane >> 4, n = lane & 15;
  const int hw = wave >> 2, wq = wave & 3;    // head half, column group
  const int hmax = (int)(a.Gp - hb * HBW);    // heads of this block present in the dS rows
  const int nv = a.nvalid[tl];
  const int32_t* rt = a.rows + tl * a.E;

  f32x4 acc[4][NB];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[s][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // dS rows of the tile (DSR bytes each), 32 / NW rows per instruction: the
  // lane writing position p of row r fetches chunk p ^ (r & DCM); chunks of
  // rows past nv or of heads past the block are zero-filled instead.
  int32_t keys = tile_keys(rt, nv, 0, lane);   // row indices of the next tile to gather
  auto issue_tile = [&](int c0, unsigned char* base) {
    unsigned char* dsb = base + KM_BYTES + KR_BYTES;
    const int r = wave * (32 / NW) + lane / (2 * NW), cq = lane % (2 * NW);
    const int c = c0 + r;
    const int q = cq ^ (r & DCM);
    const bool live = c < nv && q * 8 < hmax;
    // Zero fill before any asynchronous copy is issued, so that no plain LDS
    // store follows an asynchronous one into the same buffer.
    if (!live) *(uint4*)(dsb + r * DSR + cq * 16) = make_uint4(0, 0, 0, 0);
    issue_rows<DR, false, false>(a.k, a.kr, nullptr, keys, base, KM_BYTES, KR_BYTES, wave, NW, lane);
    keys = tile_keys(rt, nv, c0 + kTile, lane);
    if (live) lds_load16(a.ds_out + (tl * a.E + c) * a.Gp + hb * HBW + q * 8, dsb + wave * 1024);
  };

  // Transposed-read offsets (see lds_read_tr): K rows 4g+(n>>2) and +16, dS
  // rows likewise.  Wave w owns the 16-column blocks wq, wq+4, wq+8, ...
  // (wq = w % 4), so block j of the wave starts at 16-byte chunk 2wq + 8j of
  // a K row and the XOR swizzle touches only the low three chunk bits: every
  // K read is one per-lane base plus a compile-time offset.
  const int r1 = 4 * g + (n >> 2), x1 = r1 & 7;
  const int half = (n & 3) >> 1, hoff = (n & 1) * 8;
  const int sw = ((2 * wq + half) ^ x1) << 4;
  const int offM = r1 * 1024 + sw + hoff;
  const int offR = r1 * (DR * 2) + sw + hoff;
  // dS: heads 64hw + 16s + 4(n & 3) .. +4 sit in chunk 8hw + 2s + half
  int offD[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) offD[s] = r1 * DSR + (((8 * hw + 2 * s + half) ^ (r1 & DCM)) << 4) + hoff;

  auto tile = [&](int c0, int cend, const unsigned char* Km, unsigned char* nxt) {
    // (the previous tile's MFMAs stay above this wait: the wait stalls issue)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c0 + kTile < cend) issue_tile(c0 + kTile, nxt);
    const unsigned char* Kr = Km + KM_BYTES;
    const unsigned char* Ds = Kr + KR_BYTES;
    // A operands: dS of heads 64hw + 16s + n at positions 4g+i and 16+4g+i
    V8 A[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const unsigned char* p1 = Ds + offD[s];
      A[s] = join_tr<V8>(lds_read_tr((const uint16_t*)p1), lds_read_tr((const uint16_t*)(p1 + 16 * DSR)));
    }
#pragma unroll
    for (int nb0 = 0; nb0 < NB; nb0 += 3) {
      s16x4 t1[3], t2[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int nb = nb0 + j;
        if (nb < NB) {
          const unsigned char* p1;
          int rs;
          if (nb < 8) {           // K columns 16(wq + 4nb) ..
            p1 = Km + offM + nb * 128;
            rs = 16 * 1024;
          } else {                // rope columns 16wq ..
            p1 = Kr + offR;
            rs = 16 * (DR * 2);
          }
          t1[j] = lds_read_tr((const uint16_t*)p1);
          t2[j] = lds_read_tr((const uint16_t*)(p1 + rs));
        }
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (nb0 + j < NB) {
          const V8 B = join_tr<V8>(t1[j], t2[j]);
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[s][nb0 + j] = TT::mfma(A[s], B, acc[s][nb0 + j]);
        }
      }
    }
  };

  // Tiles go in pairs (one per buffer); a trailing tile past nv has zero dS
  // and adds nothing.  An unconditional pair keeps the accumulators in one
  // register form across the loop.
  const int nv2 = (nv + 2 * kTile - 1) / (2 * kTile) * (2 * kTile);
  if (nv > 0) issue_tile(0, buf0);
  for (int c0 = 0; c0 < nv2; c0 += 2 * kTile) {
    tile(c0, nv2, buf0, buf1);
    tile(c0 + kTile, nv2, buf1, buf0);
  }
  // dQ[t][h][col] = scale * acc / ds_scale; lane holds heads 16s + 4g + i of
  // its half, column n
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * (wq + 4 * nb) + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = hb * HBW + hw * 64 + 16 * s + 4 * g + i;
        if (hh < a.G) {
          const uint16_t v = TT::from_f(acc[s][nb][i] * a.dq_mul);
          if (col < 512) a.dq[(t * a.G + hh) * 512 + col] = v;
          else a.dqr[(t * a.G + hh) * DR + (col - 512)] = v;
        }
      }
    }
  }
}

void launch_sdp(int32_t dtype, bool rope, const RowArgs& a_in, hipStream_t s) {
  if (a_in.ntok == 0) return;
  const int64_t per = (int64_t)kXcds * kRun;
  const int64_t padded = (a_in.ntok + per - 1) / per * per;
  RowArgs a = a_in;
  // 128 heads: k_sdp8 (8 waves of 16 heads); 64: its 4-wave form
  if (a.Gp == 128 || (kSdp16x4 && a.Gp == 64)) {
    a.n_hb = 1;
    const bool vk8 = a.v == a.k;
    const bool w8 = a.Gp == 128;
    auto go8 = [&](auto tt, auto dr, auto vk) {
      typedef decltype(tt) T;
      constexpr int D = decltype(dr)::value;
      constexpr bool V = decltype(vk)::value;
      if (w8) hipLaunchKernelGGL((k_sdp8<T, D, V, 8>), dim3((unsigned)padded), dim3(512), 0, s, a);
      else hipLaunchKernelGGL((k_sdp8<T, D, V, 4>), dim3((unsigned)padded), dim3(256), 0, s, a);
    };
    auto by_vk = [&](auto tt, auto dr) {
      if (vk8) go8(tt, dr, std::true_type());
      else go8(tt, dr, std::false_type());
    };
    if (dtype == SFAG_BF16) {
      if (rope) by_vk(BF16(), std::integral_constant<int, 64>());
      else by_vk(BF16(), std::integral_constant<int, 0>());
    } else {
      if (rope) by_vk(FP16(), std::integral_constant<int, 64>());
      else by_vk(FP16(), std::integral_constant<int, 0>());
    }
    return;
  }
  // k_sdp: up to 128 heads per block, 32 per wave
  const int nw = (int)std::min<int64_t>(4, a.Gp / 32);
  a.n_hb = (int32_t)((a.Gp + 32 * nw - 1) / (32 * nw));
  const dim3 g1((unsigned)(padded * a.n_hb)), b1(64 * nw);
  // value passed as the key tensor itself (same rows): gather each row once
  const bool vk = a.v == a.k;
  auto go = [&](auto tt, auto dr) {
    typedef decltype(tt) T;
    constexpr int D = decltype(dr)::value;
    if (vk) {
      switch (nw) {
        case 1: hipLaunchKernelGGL((k_sdp<T, D, 1, true>), g1, b1, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_sdp<T, D, 2, true>), g1, b1, 0, s, a); break;
        case 3: hipLaunchKernelGGL((k_sdp<T, D, 3, true>), g1, b1, 0, s, a); break;
        default: hipLaunchKernelGGL((k_sdp<T, D, 4, true>), g1, b1, 0, s, a); break;
      }
    } else {
      switch (nw) {
        case 1: hipLaunchKernelGGL((k_sdp<T, D, 1, false>), g1, b1, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_sdp<T, D, 2, false>), g1, b1, 0, s, a); break;
        case 3: hipLaunchKernelGGL((k_sdp<T, D, 3, false>), g1, b1, 0, s, a); break;
        default: hipLaunchKernelGGL((k_sdp<T, D, 4, false>), g1, b1, 0, s, a); break;
      }
    }
  };
  if (dtype == SFAG_BF16) {
    if (rope) go(BF16(), std::integral_constant<int, 64>());
    else go(BF16(), std::integral_constant<int, 0>());
  } else {
    if (rope) go(FP16(), std::integral_constant<int, 64>());
    else go(FP16(), std::integral_constant<int, 0>());
  }
}

void launch_dq(int32_t dtype, bool rope, const RowArgs& a_in, hipStream_t s, bool beside) {
  if (a_in.ntok == 0) return;
  const int64_t per = (int64_t)kXcds * kRun;
  const int64_t padded = (a_in.ntok + per - 1) / per * per;
  RowArgs a = a_in;
  // k_dq: 128 heads per block (8 waves); at most 64 heads on the caller's
  // stream: one block of 64 as 4 waves, two workgroups per CU (64 heads, 8192
  // tokens: 1.83 -> 1.06 ms).  Beside the key-block kernels the 8-wave form
  // stays: the 4-wave one takes the CUs first and the key-block launch
  // behind it loses more than it gains (step 6.90 -> 7.33 ms).
  const int nw = kDq64x4 && a.Gp <= 64 && !beside ? 4 : 8;
  a.n_hb = (int32_t)((a.Gp + 16 * nw - 1) / (16 * nw));
  const dim3 g2((unsigned)(padded * a.n_hb)), b2(64 * nw);
  auto go = [&](auto kern8, auto kern4) {
    if (nw == 8) hipLaunchKernelGGL(kern8, g2, b2, 0, s, a);
    else hipLaunchKernelGGL(kern4, g2, b2, 0, s, a);
  };
  if (dtype == SFAG_BF16) {
    if (rope) go(k_dq<BF16, 64, 8>, k_dq<BF16, 64, 4>);
    else go(k_dq<BF16, 0, 8>, k_dq<BF16, 0, 4>);
  } else {
    if (rope) go(k_dq<FP16, 64, 8>, k_dq<FP16, 64, 4>);
    else go(k_dq<FP16, 0, 8>, k_dq<FP16, 0, 4>);
  }
}

}  // namespace sfag
