// Bandwidth-bound kernels around the MFMA core: sequence offsets, Delta,
// accumulator fill, index decode, the stable radix sort that inverts the
// indices into a key -> (token, position) CSR, the key-centric reduction of
// per-pair rows, and the final cast.
#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

// ---------------------------------------------------------------------------
// TND: exclusive prefix sums of the per-sequence lengths (parameter table:
// actualSeqLengthsQuery / actualSeqLengthsKv hold the valid tokens of each
// sequence, adding up to T1 / T2).  Negative lengths count as 0; the sums are
// formed in 64 bits and saturate at 2^31 - 1, so offsets never wrap.  With a
// validation word (status != NULL) negative lengths and sums that differ
// from T1 / T2 are flagged there.  One block, B <= 256.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_seq_offsets(const int32_t* lq, const int32_t* lk, int32_t B, int64_t T1,
                                                     int64_t T2, int32_t* q_off, int32_t* kv_off,
                                                     uint32_t* status) {
  __shared__ int64_t sq[257], sk[257];
  __shared__ int32_t neg;
  const int t = threadIdx.x;
  if (t == 0) neg = 0;
  __syncthreads();
  if (t < B) {
    sq[t + 1] = max(lq[t], 0);
    sk[t + 1] = max(lk[t], 0);
    if (lq[t] < 0 || lk[t] < 0) atomicOr(&neg, 1);
  }
  if (t == 0) sq[0] = sk[0] = 0;
  __syncthreads();
  if (t == 0) {
    for (int b = 1; b <= B; ++b) {
      sq[b] += sq[b - 1];
      sk[b] += sk[b - 1];
    }
    if (status) {
      uint32_t f = neg ? SFAG_BAD_LENGTH_NEGATIVE : 0u;
      if (sq[B] != T1) f |= SFAG_BAD_LENGTH_SUM_Q;
      if (sk[B] != T2) f |= SFAG_BAD_LENGTH_SUM_KV;
      if (f) atomicOr(status, f);
    }
  }
  __syncthreads();
  if (t <= B) {
    q_off[t] = (int32_t)min<int64_t>(sq[t], 0x7fffffffLL);
    kv_off[t] = (int32_t)min<int64_t>(sk[t], 0x7fffffffLL);
  }
}

// ---------------------------------------------------------------------------
// Delta[t][h] = Σ_d dO[t][h][d] · O[t][h][d] in fp32 (the page's
// FlashSoftmaxGrad(dO, O), stage 2).  One wave per (token, head) row of 512.
// ---------------------------------------------------------------------------
template <typename TT>
__global__ void __launch_bounds__(256) k_delta(const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
                                               float* __restrict__ delta, int64_t nrows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nrows) return;
  const uint4 a = *(const uint4*)(dO + row * 512 + lane * 8);
  const uint4 b = *(const uint4*)(O + row * 512 + lane * 8);
  const uint16_t* pa = (const uint16_t*)&a;
  const uint16_t* pb = (const uint16_t*)&b;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(TT::to_f(pa[i]), TT::to_f(pb[i]), s);
  s = wave_sum(s);
  if (lane == 0) delta[row] = s;
}

__global__ void __launch_bounds__(256) k_fill_u32(uint32_t* __restrict__ p, uint64_t n, uint32_t v) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 4;
  for (uint64_t i = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      *(uint4*)(p + i) = make_uint4(v, v, v, v);
    } else {
      for (uint64_t j = i; j < n; ++j) p[j] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Index decode (功能说明: gather of sparseBlockSize rows per index; Mask table:
// sparseMode 0 / 3).  Position e = j*block + r of token t is p = idx[t][j] + r,
// valid iff idx[t][j] >= 0, p < Lk and (mode 3) p <= t_loc + Lk - Lq.  The
// valid positions are compacted into rows[tl][c] = kv_base + p, and only rows
// in [0, T2) are ever written.  With nw > 0 the token's in-range entries are
// first put in ascending order, so that the token kernels walk each token's
// keys in ascending order: tokens that run at the same time on one XCD then
// gather from nearby key ranges through its L2.  The sort marks each entry
// in a bitmap of the sequence's keys (nw 32-bit words in LDS, Lk <= 32 nw)
// and reads the set bits back in order (a popcount scan gives each word its
// first slot; the sorted entries follow the bitmap as 16-bit values).  A
// token that lists a key twice keeps the listing's order instead (the
// bitmap holds one bit a key), so the order depends on the entries alone
// and the results stay bitwise reproducible; the sums see the terms in a
// different order than the listing's, which nothing fixes.  With a
// validation word (status != NULL) entries at or past the key length are
// counted there.  One block per token of the chunk.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_decode(const int32_t* __restrict__ idx, int64_t t0, int64_t K, int32_t block,
                                                int32_t mode, int32_t layout, int64_t S1, int64_t S2,
                                                const int32_t* q_off, const int32_t* kv_off, int32_t B, int64_t T2,
                                                int32_t* __restrict__ rows, int32_t* __restrict__ nvalid,
                                                uint32_t* status, int32_t nw) {
  const int64_t tl = blockIdx.x;
  const int64_t t = t0 + tl;
  const int64_t E = K * block;
  extern __shared__ uint32_t dsh[];   // nw bitmap words, then the sorted entries (16-bit)
  __shared__ int32_t warp_tot[4];
  __shared__ int32_t base_s, n_in_s, dup_s;
  const TokenGeo g = token_geo(t, layout, S1, S2, q_off, kv_off, B);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    base_s = 0;
    dup_s = 0;
  }
  int32_t bad = 0;
  // (uniform: one token per block)
  bool srtd = nw > 0 && g.ok && g.Lk > 0 && g.Lk <= 32 * nw;
  uint16_t* srt = (uint16_t*)(dsh + nw);
  int64_t Ew = E;                        // positions walked below
  if (srtd) {
    const int32_t Lk = g.Lk;
    const int nwt = (Lk + 31) >> 5;
    for (int i = tid; i < nwt; i += 256) dsh[i] = 0u;
    __syncthreads();
    bool dup = false;
    for (int j = tid; j < K; j += 256) {
      const int32_t ent = idx[t * K + j];
      if (ent >= Lk) ++bad;
      if (ent >= 0 && ent < Lk) {
        const uint32_t bit = 1u << (ent & 31);
        if (atomicOr(&dsh[ent >> 5], bit) & bit) dup = true;
      }
    }
    if (dup) dup_s = 1;
    __syncthreads();
    srtd = dup_s == 0;
    if (srtd) {
      // first slot of each word: thread tid takes words tid*cw .. +cw
      const int cw = (nwt + 255) / 256;
      const int w0 = min(nwt, tid * cw), w1 = min(nwt, w0 + cw);
      uint32_t sum = 0;
      for (int i = w0; i < w1; ++i) sum += (uint32_t)__popc(dsh[i]);
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (lane == 63) warp_tot[w] = (int32_t)incl;
      __syncthreads();
      uint32_t slot = incl - sum;
      for (int i = 0; i < w; ++i) slot += (uint32_t)warp_tot[i];
      if (tid == 255) n_in_s = (int32_t)(slot + sum);
      for (int i = w0; i < w1; ++i) {
        uint32_t m = dsh[i];
        while (m) {
          const int b = __builtin_ctz(m);
          m &= m - 1;
          srt[slot++] = (uint16_t)(32 * i + b);
        }
      }
      __syncthreads();
      Ew = (int64_t)n_in_s * block;
    } else {
      bad = 0;   // counted again by the walk over the listing below
    }
  }
  int32_t* out = rows + tl * E;
  for (int64_t e0 = 0; e0 < Ew; e0 += 256) {
    const int64_t e = e0 + tid;
    bool valid = false;
    int64_t row = 0;
    if (e < Ew && g.ok) {
      const int64_t j = e / block, r = e - j * block;
      const int32_t ent = srtd ? (int32_t)srt[j] : idx[t * K + j];
      const int64_t p = (int64_t)ent + r;
      valid = ent >= 0 && p < g.Lk && (mode != 3 || p <= g.bound);
      row = g.kv_base + p;
      valid = valid && row >= 0 && row < T2;
      if (!srtd && r == 0 && ent >= g.Lk) ++bad;
    }
    const uint64_t bal = __ballot(valid);
    const int rank = __popcll(bal & ((1ull << lane) - 1));
    if (lane == 0) warp_tot[w] = __popcll(bal);
    __syncthreads();
    int off = base_s;
    for (int i = 0; i < w; ++i) off += warp_tot[i];
    if (valid) out[off + rank] = (int32_t)row;
    __syncthreads();
    if (tid == 0) base_s += warp_tot[0] + warp_tot[1] + warp_tot[2] + warp_tot[3];
    __syncthreads();
  }
  if (tid == 0) nvalid[tl] = base_s;
  if (status && bad) {
    atomicOr(status, SFAG_BAD_INDEX_RANGE);
    atomicAdd((unsigned long long*)(status + 2), (unsigned long long)bad);
  }
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort of (key, value) pairs, 8 bits per pass, used to group
// the valid pairs by key row while keeping ascending pair order inside a key.
// Item i of the chunk is pair (tl = i / E, c = i % E); its key is the key row
// when c < nvalid[tl] and the sentinel T2 otherwise.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_item(int64_t i, int pass, const int32_t* keys_in, const int32_t* vals_in,
                                          const int32_t* rows, const int32_t* nvalid, int64_t E, int32_t sentinel,
                                          int32_t& key, int32_t& val, int key_mode, int64_t ntok) {
  if (pass == 0) {
    const int64_t tl = i / E, c = i - tl * E;
    if (c < nvalid[tl]) key = key_mode == 0 ? rows[i] : rows[i] / kKeyBlock;
    else key = sentinel;
    val = (int32_t)i;
  } else {
    key = keys_in[i];
    val = vals_in[i];
  }
}

__global__ void __launch_bounds__(kSortThreads) k_sort_hist(int64_t n, int pass, const int32_t* keys_in,
                                                            const int32_t* vals_in, const int32_t* rows,
                                                            const int32_t* nvalid, int64_t E, int32_t sentinel,
                                                            int32_t* __restrict__ hist, int64_t nblk, int key_mode,
                                                            int64_t ntok) {
  __shared__ int32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t b0 = (int64_t)blockIdx.x * kSortBlock;
  for (int k = 0; k < kSortItems; ++k) {
    const int64_t i = b0 + (int64_t)k * kSortThreads + threadIdx.x;
    if (i < n) {
      int32_t key, val;
      load_item(i, pass, keys_in, vals_in, rows, nvalid, E, sentinel, key, val, key_mode, ntok);
      atomicAdd(&h[(key >> (8 * pass)) & 255], 1);
    }
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Exclusive scan of n int32 counts in place, in three phases: per-segment
// sums, a scan of the segment sums, and per-segment scans with their offsets.
constexpr int kScanSeg = 4096;  // elements per segment (256 threads x 16)

__device__ __forceinline__ int32_t block_exclusive_scan256(int32_t v, int32_t* sh, int32_t& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int32_t off = 0;
  for (int i = 0; i < w; ++i) off += sh[i];
  total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return off + x - v;
}

__global__ void __launch_bounds__(256) k_scan_sums(const int32_t* __restrict__ a, int64_t n, int32_t* __restrict__ sums) {
  __shared__ int32_t sh[4];
  const int64_t base = (int64_t)blockIdx.x * kScanSeg;
  int32_t s = 0;
  for (int i = threadIdx.x; i < kScanSeg; i += 256)
    if (base + i < n) s += a[base + i];
  int32_t total;
  block_exclusive_scan256(s, sh, total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

__global__ void __launch_bounds__(256) k_scan_segments(int32_t* __restrict__ a, int64_t n,
                                                       const int32_t* __restrict__ offs) {
  __shared__ int32_t sh[4];
  const int64_t base = (int64_t)blockIdx.x * kScanSeg + threadIdx.x * 16;
  int32_t v[16], s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = base + i < n ? a[base + i] : 0;
    s += v[i];
  }
  int32_t total;
  int32_t run = block_exclusive_scan256(s, sh, total) + offs[blockIdx.x];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (base + i < n) a[base + i] = run;
    run += v[i];
  }
}

// Single-block exclusive scan (for the segment sums).
__global__ void __launch_bounds__(1024) k_scan(int32_t* __restrict__ a, int64_t n) {
  __shared__ int32_t part[1024];
  const int64_t per = (n + 1023) / 1024;
  const int64_t s = threadIdx.x * per, e = min(n, s + per);
  int32_t sum = 0;
  for (int64_t i = s; i < e; ++i) sum += a[i];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int32_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - sum;
  for (int64_t i = s; i < e; ++i) {
    const int32_t v = a[i];
    a[i] = run;
    run += v;
  }
}

__global__ void __launch_bounds__(kSortThreads) k_sort_scatter(int64_t n, int pass, const int32_t* keys_in,
                                                               const int32_t* vals_in, const int32_t* rows,
                                                               const int32_t* nvalid, int64_t E, int32_t sentinel,
                                                               const int32_t* __restrict__ hist, int64_t nblk,
                                                               int32_t* __restrict__ keys_out,
                                                               int32_t* __restrict__ vals_out, int key_mode,
                                                               int64_t ntok) {
  __shared__ int32_t run[256];
  __shared__ int32_t cnt[kSortThreads / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  run[tid] = hist[(int64_t)tid * nblk + blockIdx.x];
  for (int i = 0; i < kSortThreads / 64; ++i) cnt[i][tid] = 0;
  __syncthreads();
  const int64_t b0 = (int64_t)blockIdx.x * kSortBlock;
  for (int k = 0; k < kSortItems; ++k) {
    const int64_t i = b0 + (int64_t)k * kSortThreads + tid;
    const bool in = i < n;
    int32_t key = 0, val = 0;
    if (in) load_item(i, pass, keys_in, vals_in, rows, nvalid, E, sentinel, key, val, key_mode, ntok);
    const int d = in ? (key >> (8 * pass)) & 255 : 256;
    // lanes of this wave holding the same digit
    uint64_t peers = __ballot(in);
    for (int b = 0; b < 8; ++b) {
      const uint64_t bal = __ballot(((d >> b) & 1) != 0);
      peers &= ((d >> b) & 1) ? bal : ~bal;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1));
    const bool leader = in && rank == 0;
    if (leader) cnt[w][d] = __popcll(peers);
    __syncthreads();
    if (in) {
      int pos = run[d] + rank;
      for (int ww = 0; ww < w; ++ww) pos += cnt[ww][d];
      keys_out[pos] = key;
      vals_out[pos] = val;
    }
    __syncthreads();
    int add = 0;
    for (int ww = 0; ww < kSortThreads / 64; ++ww) {
      add += cnt[ww][tid];
      cnt[ww][tid] = 0;
    }
    run[tid] += add;
    __syncthreads();
  }
}

// Composite key of the key-block order: block * ntok + token (sentinel past the end).
__global__ void __launch_bounds__(256) k_kb_keys(const int32_t* __restrict__ kb, const int32_t* __restrict__ vals,
                                                 int64_t n, int64_t E, int64_t ntok, int32_t nkb,
                                                 int32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t b = kb[i];
  out[i] = b < nkb ? (int32_t)((int64_t)b * ntok + vals[i] / E) : (int32_t)((int64_t)nkb * ntok);
}

// csr_off[p] = number of sorted keys < p, p in [0, T2].
__global__ void __launch_bounds__(256) k_csr_offsets(const int32_t* __restrict__ keys, int64_t n, int64_t T2,
                                                     int32_t* __restrict__ off) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p > T2) return;
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < p) lo = mid + 1;
    else hi = mid;
  }
  off[p] = (int32_t)lo;
}

// Key-centric reduction (deterministic path): for each key row p, the partial
// rows of its pairs are added to the accumulator one by one in CSR (ascending
// pair) order.  One block per key row; fixed order, so bitwise reproducible.
__global__ void __launch_bounds__(256) k_key_reduce(const int32_t* __restrict__ off, const int32_t* __restrict__ pairs,
                                                    const float* __restrict__ part, int64_t AW,
                                                    float* __restrict__ acc) {
  const int64_t p = blockIdx.x;
  const int32_t s = off[p], e = off[p + 1];
  if (s == e) return;
  // one running sum from the accumulator through every pair in CSR order, so
  // that splitting the tokens into chunks never regroups the additions
  for (int64_t col = threadIdx.x; col < AW; col += 256) {
    float sum = acc[p * AW + col];
    for (int32_t i = s; i < e; ++i) sum += part[(int64_t)pairs[i] * AW + col];
    acc[p * AW + col] = sum;
  }
}

// ---------------------------------------------------------------------------
// Cast: dK = scale·acc[:, :D] / ds_scale, dKrope likewise, dV = acc[:, D+Dr:],
// rounded to the output type (round to nearest even).
// ---------------------------------------------------------------------------
template <typename TT>
__global__ void __launch_bounds__(256) k_cast(const float* __restrict__ acc, int64_t T2, int32_t D, int32_t Dr,
                                              float kscale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dkr,
                                              uint16_t* __restrict__ dv) {
  const int64_t AW = 2 * D + Dr;
  const int64_t n = T2 * AW;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / AW, c = i - r * AW;
    const float x = acc[i];
    if (c < D) dk[r * D + c] = TT::from_f(x * kscale);
    else if (c < D + Dr) dkr[r * Dr + (c - D)] = TT::from_f(x * kscale);
    else dv[r * D + (c - D - Dr)] = TT::from_f(x);
  }
}

// dQ | dQrope of a chunk from the fp32 sums of a split token kernel:
// dq[t0 + r / G][r % G] = RNE(acc[r] · mul), mul = scale / dS factor.
template <typename TT>
__global__ void __launch_bounds__(256) k_dq_cast(const float* __restrict__ acc, int64_t nrows, int64_t row0,
                                                 int32_t Dr, float mul, uint16_t* __restrict__ dq,
                                                 uint16_t* __restrict__ dqr) {
  const int64_t W = 512 + Dr;
  const int64_t n = nrows * W;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / W, c = i - r * W;
    const uint16_t v = TT::from_f(acc[i] * mul);
    if (c < 512) dq[(row0 + r) * 512 + c] = v;
    else dqr[(row0 + r) * Dr + (c - 512)] = v;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned grid_for(uint64_t n, unsigned per_block, unsigned cap = 65536) {
  uint64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

// In-place exclusive scan of n counts; tmp holds ceil(n / kScanSeg) ints.
// ---------------------------------------------------------------------------
// Band selection written as index rows (the block-band test of the MindSpore
// FlashAttention backward page, "flash_attention_bwd.py",
// compute_in_each_kv_block, taken per query token and aligned like
// sparseMode 3 on the bottom-right diagonal): query position t of a sequence
// covers key positions d - pre .. d + nxt (d = t + Lk - Lq) inside [0, Lk);
// its row holds the ascending starts of the blocks that overlap them, then -1.
// One block per token; with TND the per-sequence offsets are formed in LDS
// (B <= 256, negative lengths count as 0).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_band_indices(int32_t* __restrict__ idx, int64_t K, int32_t block,
                                                      int32_t layout, int64_t S1, int64_t S2,
                                                      const int32_t* __restrict__ lq,
                                                      const int32_t* __restrict__ lk, int32_t B, int64_t pre,
                                                      int64_t nxt) {
  __shared__ int32_t sq[257], sk[257];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (layout == 1) {
    if (tid < B) {
      sq[tid + 1] = max(lq[tid], 0);
      sk[tid + 1] = max(lk[tid], 0);
    }
    if (tid == 0) {
      sq[0] = sk[0] = 0;
      for (int b = 1; b <= B; ++b) {
        sq[b] += sq[b - 1];
        sk[b] += sk[b - 1];
      }
    }
    __syncthreads();
  }
  const TokenGeo g = token_geo(t, layout, S1, S2, sq, sk, B);
  const int64_t lo = max<int64_t>(0, (int64_t)g.bound - pre);
  const int64_t hi = min<int64_t>((int64_t)g.Lk - 1, (int64_t)g.bound + nxt);
  int64_t first = 0, nblk = 0;
  if (g.ok && lo <= hi) {
    first = lo / block;
    nblk = hi / block - first + 1;
  }
  int32_t* row = idx + t * K;
  for (int64_t j = tid; j < K; j += 256) row[j] = j < nblk ? (int32_t)((first + j) * block) : -1;
}

void launch_scan_i32(int32_t* a, int64_t n, int32_t* tmp, hipStream_t s) {
  const int64_t nseg = (n + kScanSeg - 1) / kScanSeg;
  if (nseg <= 1) {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, a, n);
    return;
  }
  hipLaunchKernelGGL(k_scan_sums, dim3((unsigned)nseg), dim3(256), 0, s, a, n, tmp);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, tmp, nseg);
  hipLaunchKernelGGL(k_scan_segments, dim3((unsigned)nseg), dim3(256), 0, s, a, n, tmp);
}

void launch_seq_offsets(const int32_t* lq, const int32_t* lk, int32_t B, int64_t T1, int64_t T2, int32_t* q_off,
                        int32_t* kv_off, uint32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_seq_offsets, dim3(1), dim3(256), 0, s, lq, lk, B, T1, T2, q_off, kv_off, status);
}

void launch_delta(int32_t dtype, const void* dO, const void* O, float* delta, int64_t nrows, hipStream_t s) {
  if (nrows == 0) return;
  const dim3 grid((unsigned)((nrows + 3) / 4));
  if (dtype == SFAG_BF16)
    hipLaunchKernelGGL(k_delta<BF16>, grid, dim3(256), 0, s, (const uint16_t*)dO, (const uint16_t*)O, delta, nrows);
  else
    hipLaunchKernelGGL(k_delta<FP16>, grid, dim3(256), 0, s, (const uint16_t*)dO, (const uint16_t*)O, delta, nrows);
}

void launch_fill_u32(void* p, uint64_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 1024, 8192)), dim3(256), 0, s, (uint32_t*)p, n, v);
}

void launch_decode(const int32_t* idx, int64_t t0, int64_t ntok, const Dims& d, const int32_t* q_off,
                   const int32_t* kv_off, int32_t* rows, int32_t* nvalid, hipStream_t s, uint32_t* status,
                   bool sort_entries) {
  if (ntok == 0) return;
  // the sort's LDS: a bit per key of the longest sequence (BSND: S2; TND:
  // at most T2), keys below 65536 so that 16 bits hold a sorted entry
  const int64_t lk_max = d.layout == 0 ? d.S2 : d.T2;
  int32_t nw = 0;
  if (sort_entries && d.K > 1 && d.K <= 16384 && lk_max <= 65536) nw = (int32_t)std::max<int64_t>(1, (lk_max + 31) / 32);
  const size_t lds = nw ? (size_t)nw * 4 + (size_t)(d.K + 1) / 2 * 4 : 0;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)ntok), dim3(256), lds, s, idx, t0, d.K, (int32_t)d.block, d.mode,
                     d.layout, d.S1, d.S2, q_off, kv_off, (int32_t)d.B, d.T2, rows, nvalid, status, nw);
}

void launch_csr(int64_t n, const int32_t* rows, const int32_t* nvalid, int64_t E, int64_t T2, int32_t sort_bits,
                int32_t* keys[2], int32_t* vals[2], int32_t* hist, int32_t* csr_off, int32_t** sorted_vals,
                hipStream_t s, int key_mode, int64_t ntok, int32_t** sorted_keys) {
  const int64_t nblk = (n + kSortBlock - 1) / kSortBlock;
  const int npass = (sort_bits + 7) / 8;
  int32_t* scan_tmp = hist + 256 * nblk;  // the histogram region reserves room for the segment sums
  // key_mode 1 sorts by key block only: items enter in (token, position) order
  // and the sort is stable, so each block's items stay in token order.
  const int32_t nkb = (int32_t)((T2 + kKeyBlock - 1) / kKeyBlock);
  const int32_t sentinel = key_mode == 0 ? (int32_t)T2 : nkb;
  int cur = 0;
  for (int pass = 0; pass < npass; ++pass) {
    const int32_t* kin = pass ? keys[cur] : nullptr;
    const int32_t* vin = pass ? vals[cur] : nullptr;
    const int nxt = pass ? cur ^ 1 : 0;
    hipLaunchKernelGGL(k_sort_hist, dim3((unsigned)nblk), dim3(kSortThreads), 0, s, n, pass, kin, vin, rows, nvalid,
                       E, sentinel, hist, nblk, key_mode, ntok);
    launch_scan_i32(hist, 256 * nblk, scan_tmp, s);
    hipLaunchKernelGGL(k_sort_scatter, dim3((unsigned)nblk), dim3(kSortThreads), 0, s, n, pass, kin, vin, rows,
                       nvalid, E, sentinel, hist, nblk, keys[nxt], vals[nxt], key_mode, ntok);
    cur = nxt;
  }
  if (csr_off)
    hipLaunchKernelGGL(k_csr_offsets, dim3(grid_for(T2 + 1, 256, 1u << 30)), dim3(256), 0, s, keys[cur], n, T2,
                       csr_off);
  *sorted_vals = vals[cur];
  if (key_mode == 1) {
    // composite keys block * ntok + token for the range lookups
    int32_t* ck = keys[cur ^ 1];
    hipLaunchKernelGGL(k_kb_keys, dim3(grid_for(n, 256, 1u << 30)), dim3(256), 0, s, keys[cur], vals[cur], n, E, ntok,
                       nkb, ck);
    cur ^= 1;
  }
  if (sorted_keys) *sorted_keys = keys[cur];
}

void launch_key_reduce(const int32_t* off, const int32_t* pairs, const float* part, int64_t AW, int64_t T2, float* acc,
                       hipStream_t s) {
  if (T2 == 0) return;
  hipLaunchKernelGGL(k_key_reduce, dim3((unsigned)T2), dim3(256), 0, s, off, pairs, part, AW, acc);
}

void launch_cast(int32_t dtype, const float* acc, int64_t T2, int32_t D, int32_t Dr, float kscale, void* dk, void* dkr,
                 void* dv, hipStream_t s) {
  const uint64_t n = (uint64_t)T2 * (2 * D + Dr);
  if (n == 0) return;
  const dim3 grid(grid_for(n, 256 * 8, 16384));
  if (dtype == SFAG_BF16)
    hipLaunchKernelGGL(k_cast<BF16>, grid, dim3(256), 0, s, acc, T2, D, Dr, kscale, (uint16_t*)dk, (uint16_t*)dkr,
                       (uint16_t*)dv);
  else
    hipLaunchKernelGGL(k_cast<FP16>, grid, dim3(256), 0, s, acc, T2, D, Dr, kscale, (uint16_t*)dk, (uint16_t*)dkr,
                       (uint16_t*)dv);
}

void launch_dq_cast(int32_t dtype, const float* acc, int64_t t0, int64_t ntok, int64_t G, int32_t Dr, float mul,
                    void* dq, void* dqr, hipStream_t s) {
  const int64_t nrows = ntok * G;
  if (nrows == 0) return;
  const dim3 grid(grid_for((uint64_t)nrows * (512 + Dr), 1024, 8192));
  if (dtype == SFAG_BF16)
    hipLaunchKernelGGL(k_dq_cast<BF16>, grid, dim3(256), 0, s, acc, nrows, t0 * G, Dr, mul, (uint16_t*)dq,
                       (uint16_t*)dqr);
  else
    hipLaunchKernelGGL(k_dq_cast<FP16>, grid, dim3(256), 0, s, acc, nrows, t0 * G, Dr, mul, (uint16_t*)dq,
                       (uint16_t*)dqr);
}

void launch_band_indices(int32_t* idx, int64_t T1, int64_t K, int32_t block, int32_t layout, int64_t S1, int64_t S2,
                         const int32_t* lq, const int32_t* lk, int32_t B, int64_t pre, int64_t nxt, hipStream_t s) {
  if (T1 == 0 || K == 0) return;
  hipLaunchKernelGGL(k_band_indices, dim3((unsigned)T1), dim3(256), 0, s, idx, K, block, layout, S1, S2, lq, lk, B,
                     pre, nxt);
}

}  // namespace sfag
