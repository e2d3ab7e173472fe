// Key-centric contraction over heads for dK / dKrope / dV (operator page
// "aclnnSparseFlashAttentionGrad", 功能说明 stages 1 and 3: dV = Pᵀ·dO and
// dK = scale·dSᵀ·Q, summed over every (token, position) selecting the key).
//
// Instead of scattering one partial row per (token, position) with atomics,
// a workgroup owns a block of 256 consecutive key rows and a block of output
// columns, and walks, in token order, the tokens of one token range that
// select any of its keys.  The pairs are sorted by (key block, token), and a
// "visit" is the run of one token's pairs inside one key block.  For each
// visit the workgroup accumulates
//     C[key][col] += Σ_h A[key][h] · B[h][col]
// with v_mfma_f32_16x16x32, where A holds the token's dS (or P) rows placed
// at their key rows (rows the token does not select read a zero row) and B is
// the token's Q|Qrope (or dO) rows as they lie in memory (head-major): the
// operand's column-of-heads fragments come out of LDS through the transposing
// read ds_read_b64_tr_b16, so no transposed copy of the token side is made.
//
// A visit runs in stages, one per 32-head step (four at 128 heads).  Both
// operands of a stage reach LDS through global_load_lds, about three stages
// ahead of their use (four stage buffers), so the only waits on memory are
// explicit ones on copies issued about three stages earlier.  At 128 heads
// each stage's barrier sits between its two row groups, so that the reads of
// the next stage's operands overlap MFMAs, and a visit's copy sources are
// formed once per visit.  The key-row slot map of a visit (which rows its
// token selects, how often, and which pair supplies each row) is built two
// visits ahead with LDS atomics from the visit's pairs, which are themselves
// copied into LDS ahead of that.  A key listed k times by one token has k
// identical dS/P rows (same token, same key), so each stage of that visit
// runs k rounds over the row.
//
// C stays in registers (8 waves, two per SIMD, each with a 128-key half of
// the rows and a quarter of the columns) for the whole token range and is
// written once as an fp32 partial of that range; a second kernel adds
// the partials of the ranges in ascending order.  Every sum runs in a fixed
// order, so the result is bitwise reproducible.
#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

namespace sfag {

namespace {

constexpr int kKB = kKeyBlock;             // key rows per block (256)
constexpr int kStageA = kKB * 64;          // 256 rows x 32 heads, 16-bit
constexpr int kStageB = 256 * 64;          // up to 256 columns x 32 heads
constexpr int kStageBytes = kStageA + kStageB;
constexpr int kWin = 256;                  // visits whose metadata sit in LDS at a time
constexpr int kEnt = 256;                  // pairs of a visit copied into LDS
constexpr int kXcds = 8;                   // XCDs of the chip (workgroup b runs on XCD b % 8)

// Asynchronous global -> LDS copies (lane l of the wave writes 16 or 4 bytes
// at the wave-uniform LDS address l_base + l * size).  Written as inline asm
// on purpose: the compiler then does not track them, so it inserts no waits
// of its own for them before unrelated LDS reads; every read of copied data
// is preceded by an explicit wait on the copy (wait_vm) and a barrier.
// Each copy starts with one wait state (s_nop 0): on this chip family an LDS
// DMA that reads M0 right after a scalar write of M0 needs one, and the
// compiler inserts it only for DMA instructions it emits itself.
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) unsigned char*)l);
}
// (LDS destinations are 32-bit LDS addresses, wave-uniform.)
// Copy through a buffer resource: a lane whose offset lies at or past the
// resource's num_records (a raw buffer: stride 0) fails the buffer range
// check, so it fetches nothing and its load returns zero (the AMD Instinct
// CDNA instruction set reference, buffer addressing and range checking), and
// the LDS slot it writes receives zeros: rows that are never used cost no
// memory traffic.
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t l) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(l) : "memory");
}
constexpr uint32_t kOutside = 0x80000000u;   // offset past any resource size used here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, bytes,
                                           0x00020000);
}
__device__ __forceinline__ void dma4(const void* g, uint32_t l) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(l) : "memory");
}
__device__ __forceinline__ void dma16(const void* g, uint32_t l) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(l) : "memory");
}

// 16 zero bytes: the source of B-stage slots of heads past N1.
__device__ __attribute__((aligned(16))) uint4 g_zero16;

// B stage: 32 head rows (the stage's heads) of NB * 64 columns, NB * 128
// bytes each, in 16-byte chunks; chunk j of head row r sits at position
// j ^ (2 * bswz<NB>(r)), which moves 32-byte chunk pairs within an aligned
// group of 8 (NB = 3: 384-byte rows) or 16 (NB = 4) chunks.  The transposing
// reads take one chunk pair from each of 4 consecutive head rows per 16
// lanes (rows 8g + 0..3 or 8g + 4..7 with 32 heads, 4g + 0..3 with 16); the
// swizzle puts the 4 rows of any 16 lanes on distinct 32-byte bank groups of
// a 128-byte line, and the 8 rows of any 32 lanes on distinct groups of a
// 256-byte line (for 384-byte rows counting the 128-byte shift of odd rows).
template <int NB>
__device__ __forceinline__ int bswz(int r) {
  if constexpr (NB == 4) return (r & 7) ^ (((r >> 3) & 1) << 2);
  else return (r & 3) ^ (((r >> 2) ^ (r >> 3)) & 1);
}

// Chunk swizzle of the 64-byte stage rows (4 chunks of 16 bytes): chunk q of
// row r sits at position q ^ swz(r).  The A-operand reads take chunk g of 16
// consecutive rows per 16 lanes; of the row-dependent swizzles measured with
// that access, (r >> 1) & 3 is one that runs it at the full ds_read_b128 rate
// (about 200 bytes per clock per CU with 8 waves, against 128 for r & 3,
// (r >> 2) & 3 or none).  It depends on bits 1..2 of r only.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

__device__ __forceinline__ int64_t lower_bound_i32(const int32_t* a, int64_t n, int64_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Workgroup barrier for LDS data: waits for this wave's LDS operations only,
// not for its outstanding global loads and copies (a fence would wait for
// those as well, draining the copies that are meant to stay in flight).
// The signal fences keep the compiler from moving memory accesses across.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most M stages' copies of this wave are outstanding: KA A
// copies and KB B copies per stage, where the NBI B-copy instructions of a
// stage go to waves w, w + W, ..., so KB is ceil(NBI / W) for waves below
// NBI % W (all of them when W divides NBI) and floor(NBI / W) for the rest.
// (The count has to be an immediate, hence the two forms.)
template <int M, int KA, int NBI, int W>
__device__ __forceinline__ void wait_stages(int wave) {
  constexpr int KH = KA + (NBI + W - 1) / W, KL = KA + NBI / W;
  if (NBI % W == 0 || wave < NBI % W) wait_vm<M * KH>();
  else wait_vm<M * KL>();
}

struct KbShared {
  int32_t cnt[3][kKB];       // per key row: how often the visit's token lists it
  int32_t prim[3][kKB];      // per key row: the pair whose dS/P row is staged
  int32_t rounds[3];         // max over rows of cnt (at least 1)
  int32_t vstart[kWin + 3];  // first sorted pair of visits wb .. wb + kWin + 2
  int32_t vkey[kWin + 2];    // their composite keys
};

// One column block of NB * 64 columns (NB = 4 for 256 columns, 3 for 192),
// W waves (4 or 8).  Wave w takes the column quarter w % 4 (NB 16-column MFMA
// blocks) and, with 4 waves, all 256 key rows (16 MFMA row blocks), with 8
// waves the half w / 4 of them (8 row blocks): two waves per SIMD, each with
// half the accumulators, so that one wave's waits are covered by the other's
// MFMAs.  GP is the padded head count when it is 128 (all strides
// compile-time), else 0 (taken from the args).
template <typename TT, int NB, int GP, int W>
__device__ __forceinline__ void kb_block(const KbArgs& a, const ColBlock c, int tr, int kb, int vlo,
                                         int vhi, unsigned char* __restrict__ st0,
                                         unsigned char* __restrict__ st1, unsigned char* __restrict__ st2,
                                         unsigned char* __restrict__ st3, KbShared* __restrict__ shp,
                                         int32_t* __restrict__ e_pair, int32_t* __restrict__ e_row) {
  // (restrict: lets the compiler tell the asynchronous LDS copies into one
  // buffer from the reads of another, so that those reads need no wait)
  KbShared& sh = *shp;
  typedef typename TT::vec8 V8;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int g = lane >> 4, n = lane & 15;
  const int Gp = GP ? GP : (int)a.Gp, nks = (Gp + 31) >> 5;
  const uint16_t* Bmain = c.src == 0 ? a.q : a.dO;
  const uint16_t* Asrc = c.src == 0 ? a.ds : a.p;
  const int kbase = kb * (int)a.ntok;   // composite keys are int32 by construction
  constexpr int NT = 64 * W;        // threads
  constexpr int RB = 64 / W;        // MFMA row blocks per wave
  constexpr int KA = 16 / W;        // A copy instructions per wave and stage
  // B copy instructions per stage: 4 NB for 32 head rows, 2 NB with 16 heads
  // (GP = 16: rows 16 .. 31 of the stage are never read)
  constexpr int NBI = GP == 16 ? 2 * NB : 4 * NB;
  constexpr int KBM = (NBI + W - 1) / W;
  const int KB = (NBI - wave + W - 1) / W;      // B copy instructions of this wave and stage
  const int mb0 = (wave >> 2) * RB;             // first row block of the wave
  const int cq = wave & 3;                      // column quarter of the wave

  // ---- visit metadata, staged in LDS for a window of visits from wb ------
  int wb = vlo;
  auto load_window = [&]() {
    for (int j = tid; j < kWin + 3; j += NT) {
      const int x = wb + j;
      sh.vstart[j] = x <= vhi ? a.vis_start[x] : 0;
      if (j < kWin + 2) sh.vkey[j] = x < vhi ? a.vis_key[x] : 0;
    }
  };
  auto v_start = [&](int v) -> int { return sh.vstart[v - wb]; };
  auto v_count = [&](int v) -> int { return sh.vstart[v + 1 - wb] - sh.vstart[v - wb]; };
  auto v_token = [&](int v) -> int { return sh.vkey[v - wb] - kbase; };

  f32x4 C[RB][NB];
#pragma unroll
  for (int mb = 0; mb < RB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) C[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- slot maps ----------------------------------------------------------
  auto reset = [&](int b) {
    if (tid < kKB) {
      sh.cnt[b][tid] = 0;
      sh.prim[b][tid] = -1;
    }
    if (tid == 0) sh.rounds[b] = 1;
  };
  auto add_entry = [&](int b, int32_t pair, int row) {
    const int o = atomicAdd(&sh.cnt[b][row], 1);
    if (o == 0) sh.prim[b][row] = pair;
    else atomicMax(&sh.rounds[b], o + 1);
  };
  // map of visit v from its pairs: the first kEnt from the LDS copy, the
  // rest (only with duplicated keys) straight from memory
  // (eh: which of the two entry buffers holds the visit's pairs)
  auto build = [&](int b, int v, int eh) {
    const int cnt = v_count(v);
    if (tid < cnt && tid < kEnt) add_entry(b, e_pair[eh * kEnt + tid], e_row[eh * kEnt + tid]);
    const int s0 = v_start(v);
    for (int j = tid + kEnt; j < cnt; j += NT) add_entry(b, a.svals[s0 + j], a.er[s0 + j]);
  };
  const uint32_t l_pair = lds_addr(e_pair), l_row = lds_addr(e_row);
  // copy of visit v's first kEnt pairs (ids and key rows) into LDS: 8
  // dword-copy instructions, 8 / W per wave; lanes past the visit re-read
  // its first pair
  auto issue_entries = [&](int v, int eh) {
    const int s0 = v_start(v);
    const int cnt = v_count(v);
#pragma unroll
    for (int k = 0; k < 8 / W; ++k) {
      const int ins = wave * (8 / W) + k;    // 0..3 pair ids, 4..7 key rows
      const int part = ins & 3;
      const int e = part * 64 + lane;
      const int src = s0 + (e < cnt ? e : 0);
      if (ins < 4) dma4(a.svals + src, l_pair + eh * kEnt * 4 + part * 256);
      else dma4(a.er + src, l_row + eh * kEnt * 4 + part * 256);
    }
  };

  // ---- stage copies -------------------------------------------------------
  // A of stage (visit, ks): 256 rows x 4 chunks (heads 32ks + 8q .. +8), 16
  // instructions, wave w issuing w, w + W, ...; the lane writing position
  // p of row r fetches chunk p ^ swz(r).  Rows not selected (and
  // chunks past the heads) take an offset outside the resource: they fetch
  // nothing and their slots receive zeros, which the MFMAs read as such.
  // B: the 32 head rows of the block's columns (bswz layout), 4 * NB
  // instructions (2 * NB, rows 0 .. 15, with 16 heads), wave w issuing w,
  // w + W, ...; the lane writing position e of the stage fetches the chunk
  // of head row e / (8 NB) that belongs there, from Q or Qrope (a block may
  // straddle the two) or dO; heads past N1 read 16 zero bytes.
  // The copies of one stage, prepared once (slot-map entries read, sources
  // made) and then issued one A and one B instruction at a time between the
  // MFMAs of the stage being computed: a burst of copies at the top of a
  // stage stalls the issuing wave until the address unit takes them.
  const int G = (int)a.G;
  const int Dr = a.Dr;
  // Address of the zero chunk, made opaque so that it stays in registers: left
  // to the compiler it is reloaded through a scalar load inside the copy
  // code, and the wait for that load also waits for every LDS read in flight.
  uint32_t z_lo = (uint32_t)(uintptr_t)&g_zero16, z_hi = (uint32_t)((uint64_t)(uintptr_t)&g_zero16 >> 32);
  asm volatile("" : "+v"(z_lo), "+v"(z_hi));
  // Per B instruction k, this lane's chunk: element offset from the stage's
  // first head row in Q|dO or Qrope (bits 0..14), head row within the stage
  // (bits 16..20), and whether it is a Qrope chunk (bit 21).
  uint32_t b_chunk[KBM];
#pragma unroll
  for (int k = 0; k < KBM; ++k) {
    const int e = 64 * (wave + W * k) + lane;
    const int hr = e / (8 * NB), pos = e - hr * (8 * NB);
    const int col = c.tcol0 + 8 * (pos ^ (2 * bswz<NB>(hr)));
    const bool rope = c.src == 0 && col >= 512;
    const uint32_t off = rope ? (uint32_t)(hr * Dr + (col - 512)) : (uint32_t)(hr * 512 + col);
    b_chunk[k] = off | ((uint32_t)hr << 16) | ((uint32_t)rope << 21);
  }
  struct StageCopy {
    __amdgpu_buffer_rsrc_t ars;
    const uint16_t *bm, *br;   // rows of head 32ks of the token in Q|dO and Qrope
    int32_t pr[KA];
    int32_t p0;
    int ks;
    uint32_t st;
    bool on;
  };
  auto b_rows = [&](StageCopy& sc, int tl, int ks) {
    const int64_t hrow = (a.t0 + tl) * a.G + 32 * ks;
    sc.bm = Bmain + hrow * 512;
    sc.br = a.qr + hrow * Dr;
  };
  auto b_src = [&](const StageCopy& sc, int k) -> const void* {
    const uint32_t x = b_chunk[k];
    if (32 * sc.ks + (int)((x >> 16) & 31) >= G) return (const void*)(((uint64_t)z_hi << 32) | z_lo);
    return ((x >> 21) ? sc.br : sc.bm) + (x & 0x7fff);
  };
  // the slot-map entries (staged pair of each key row) of this lane's A copies
  auto prim_of = [&](int b, int32_t (&pr)[KA]) {
#pragma unroll
    for (int k = 0; k < KA; ++k) pr[k] = sh.prim[b][16 * (wave + W * k) + (lane >> 2)];
  };
  auto prep_with = [&](StageCopy& sc, bool on, const int32_t (&pr)[KA], int tl, int ks, uint32_t st) {
    sc.on = on;
    if (!on) return;
    // A rows of token tl: pairs tl*E .. tl*E + E - 1
    sc.ars = make_rsrc(Asrc + (int64_t)tl * a.E * Gp, (int)(a.E * Gp * 2));
    b_rows(sc, tl, ks);
    sc.p0 = tl * (int)a.E;
    sc.ks = ks;
    sc.st = st;
#pragma unroll
    for (int k = 0; k < KA; ++k) sc.pr[k] = pr[k];
  };
  auto prep_stage = [&](StageCopy& sc, bool on, int b, int tl, int ks, uint32_t st) {
    int32_t pr[KA];
    if (on) prim_of(b, pr);
    prep_with(sc, on, pr, tl, ks, st);
  };
  auto issue_a = [&](const StageCopy& sc, int k) {
    const int i = wave + W * k;
    const int row = 16 * i + (lane >> 2);
    const int q = (lane & 3) ^ swz(row);
    const int hq = 32 * sc.ks + 8 * q;
    const uint32_t off = (sc.pr[k] >= 0 && hq < Gp) ? (uint32_t)(((sc.pr[k] - sc.p0) * Gp + hq) * 2) : kOutside;
    bdma16(sc.ars, off, sc.st + i * 1024);
  };
  auto issue_b = [&](const StageCopy& sc, int k) {
    dma16(b_src(sc, k), sc.st + kStageA + (wave + W * k) * 1024);
  };
  auto issue_part = [&](const StageCopy& sc, int k) {
    if (!sc.on) return;
    if (k < KA) issue_a(sc, k);
    if (k < KBM && k < KB) issue_b(sc, k);
  };
  auto issue_all = [&](StageCopy& sc) {
    if (sc.on) {
#pragma unroll
      for (int k = 0; k < KA; ++k) issue_a(sc, k);
#pragma unroll
      for (int k = 0; k < KBM; ++k)
        if (k < KB) issue_b(sc, k);
    }
    sc.on = false;
  };
  // All copies of a stage at once, at the top of the stage: the generic path
  // (Gp != 128) waits for every copy at each stage, so spreading its copies
  // over the MFMAs would leave the last ones no time before that wait.
  auto issue_stage = [&](int b, int tl, int ks, uint32_t st) {
    StageCopy sc;
    prep_stage(sc, true, b, tl, ks, st);
    issue_all(sc);
  };
  // Round r of a stage (r >= 1, keys listed more than once by the token):
  // the rows listed exactly r times leave the sum, so their stage rows are
  // cleared (between barriers: other waves may still read the previous
  // round).
  auto drop_rows = [&](unsigned char* st, int b, int r) {
    bar();
    if (tid < kKB && sh.cnt[b][tid] == r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) *(uint4*)(st + tid * 64 + j * 16) = make_uint4(0, 0, 0, 0);
    }
    bar();
  };
  // C += A · B over the 32 heads of one stage
  // B fragments: lane (g, n) of column block nb takes column
  // 16 (NB cq + nb) + n of the block; a transposing read from head row r
  // (lanes 4m .. 4m + 3 of each 16 addressing row r0 + m, columns 4 apart)
  // gives it heads r0 .. r0 + 3.  Byte offset in the B stage of the 8 bytes
  // this lane addresses in head row r:
  auto boff = [&](int r, int nb) -> int {
    return r * (NB * 128) + ((2 * ((NB * cq + nb) ^ bswz<NB>(r)) + ((n & 3) >> 1)) << 4) + 8 * (n & 1);
  };
  // Rows the token does not select, and head chunks past Gp, hold zeros in
  // the stage (their copies fetch nothing and land zeros), so every row is
  // read as it is.
  auto compute = [&](const unsigned char* st, const StageCopy& sc) {
    const int po = (g ^ swz(n)) << 4;            // rows mb*16 + n: swz(r) = swz(n)
    // heads 8g .. 8g + 7: head rows 8g + n / 4 and 4 further
    const int r0 = 8 * g + (n >> 2);
    V8 Bf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const unsigned char* bs = st + kStageA;
      Bf[nb] = join_tr<V8>(lds_read_tr((const uint16_t*)(bs + boff(r0, nb))),
                           lds_read_tr((const uint16_t*)(bs + boff(r0 + 4, nb))));
    }
    uint4 av[2][4];
    auto rd = [&](int h, uint4 (&dst)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mb = mb0 + 4 * h + j;
        dst[j] = *(const uint4*)(st + (mb * 16 + n) * 64 + po);
      }
    };
    // The reads of row group h + 1 go out ahead of the MFMAs of group h (the
    // scheduler would otherwise sink them below most of those MFMAs, leaving
    // the LDS latency exposed at the next group), and the stage copies
    // between the two halves of the group's MFMAs.
    rd(0, av[0]);
#pragma unroll
    for (int h = 0; h < RB / 4; ++h) {
      if (h + 1 < RB / 4) rd(h + 1, av[(h + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          C[4 * h + j][nb] = TT::mfma(as_vec8<V8>(av[h & 1][j]), Bf[nb], C[4 * h + j][nb]);
      __builtin_amdgcn_sched_barrier(0);
      issue_part(sc, h);   // nothing unless the caller prepared copies
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 2; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          C[4 * h + j][nb] = TT::mfma(as_vec8<V8>(av[h & 1][j]), Bf[nb], C[4 * h + j][nb]);
    }
  };

  // The same for 16 heads (Gp = 16: the upper half of every stage row is
  // zero): v_mfma_f32_16x16x16 over the 16 live heads, half the MFMA work
  // and half the operand reads.  Lane group g takes heads 4g .. 4g + 3: the
  // 8-byte half g & 1 of 16-byte chunk g >> 1 of an A row, head rows
  // 4g .. 4g + 3 of the B stage.
  auto compute16 = [&](const unsigned char* st, const StageCopy& sc) {
    typedef typename TT::vec4 V4;
    const int ch = g >> 1, hoff = (g & 1) << 3;
    const int po = ((ch ^ swz(n)) << 4) + hoff;
    V4 Bf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      Bf[nb] = __builtin_bit_cast(V4, lds_read_tr((const uint16_t*)(st + kStageA + boff(4 * g + (n >> 2), nb))));
    uint2 av[2][4];
    auto rd = [&](int h, uint2 (&dst)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mb = mb0 + 4 * h + j;
        dst[j] = *(const uint2*)(st + (mb * 16 + n) * 64 + po);
      }
    };
    rd(0, av[0]);
#pragma unroll
    for (int h = 0; h < RB / 4; ++h) {
      if (h + 1 < RB / 4) rd(h + 1, av[(h + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          C[4 * h + j][nb] = TT::mfma16(__builtin_bit_cast(V4, av[h & 1][j]), Bf[nb], C[4 * h + j][nb]);
      __builtin_amdgcn_sched_barrier(0);
      issue_part(sc, h);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 2; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          C[4 * h + j][nb] = TT::mfma16(__builtin_bit_cast(V4, av[h & 1][j]), Bf[nb], C[4 * h + j][nb]);
    }
  };

  const int nst = 4 * (vhi - vlo);   // stages (four 32-head stages per visit)
  auto stage_buf = [&](int ks) -> unsigned char* { return ks == 0 ? st0 : ks == 1 ? st1 : ks == 2 ? st2 : st3; };
  const uint32_t L0 = lds_addr(st0), L1 = lds_addr(st1), L2 = lds_addr(st2), L3 = lds_addr(st3);
  auto stage_lds = [&](int ks) -> uint32_t { return ks == 0 ? L0 : ks == 1 ? L1 : ks == 2 ? L2 : L3; };

  // ---- prologue ------------------------------------------------------------
  for (int b = 0; b < 3; ++b) reset(b);
  load_window();
  __syncthreads();
  for (int x = 0; x < 2; ++x) {
    const int v = vlo + x;
    if (v < vhi) {
      const int s0 = v_start(v);
      const int cnt = v_count(v);
      for (int j = tid; j < cnt; j += NT) add_entry(x, a.svals[s0 + j], a.er[s0 + j]);
    }
  }
  __syncthreads();

  if constexpr (GP == 128) {
    // 128 heads: four 32-head stages per visit, numbered x = 4 w + ks over
    // the visits w = v - vlo of the range; stage x uses buffer ks.  Each
    // stage's barrier sits between its two row groups: a wave computes row
    // group 0 of stage x, waits for the copies of stage x + 1 and meets the
    // others, and then reads the operands of stage x + 1 while the MFMAs of
    // row group 1 run: row group 0 of A at once, and B one column block at a
    // time, each into the registers of the column block whose row-group-1
    // MFMAs were just issued.  Stage x + 4 is copied into buffer ks (which
    // every wave has finished reading at the barrier) between those MFMAs.
    // So the operand reads that follow a barrier overlap MFMAs, and copies
    // are issued three and a half stages before their use.  Bookkeeping
    // after the barrier of stage 4 w + ks: ks = 0: the map slot of visit
    // w + 2 (last used by visit w - 1) is cleared and the pairs of visit
    // w + 2 are copied; ks = 2: its map is built (those copies are older
    // than the copies this barrier waited for); ks = 3: the round count of
    // visit w + 1 is read.
    typedef typename TT::vec8 V8b;
    const int po = (g ^ swz(n)) << 4;   // A row chunk of this lane (rows 16 mb + n)
    const int r0 = 8 * g + (n >> 2);    // B head rows r0 and r0 + 4
    // (operand reads address a stage through an LDS pointer made opaque per
    // stage, so that the per-lane offsets are shared by the four buffers
    // instead of being kept, precomputed, once per buffer)
    typedef __attribute__((address_space(3))) const unsigned char* lds_p;
    auto lds_base = [&](const unsigned char* st) -> lds_p {
      lds_p b = (lds_p)st;
      asm volatile("" : "+v"(b));
      return b;
    };
    auto rdA = [&](lds_p st, int h, uint4 (&dst)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 x = *(__attribute__((address_space(3))) const u32x4*)(st + ((mb0 + 4 * h + j) * 16 + n) * 64 + po);
        dst[j] = __builtin_bit_cast(uint4, x);
      }
    };
    auto rdB1 = [&](lds_p st, int nb) -> V8b {
      lds_p bs = st + kStageA;
      return join_tr<V8b>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(bs + boff(r0, nb))),
                          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(bs + boff(r0 + 4, nb))));
    };
    auto rdB = [&](lds_p st, V8b (&dst)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) dst[nb] = rdB1(st, nb);
    };
    // MFMAs of row group h with column block nb
    auto mma = [&](const uint4 (&av)[4], const V8b& B, int h, int nb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) C[4 * h + j][nb] = TT::mfma(as_vec8<V8b>(av[j]), B, C[4 * h + j][nb]);
    };
    // Copy sources of one visit, made once per visit and offset per stage:
    // stage ks of the visit reads A at byte offset aoff[k] + 64 ks (rows not
    // selected keep an offset outside the resource for every ks) and B from
    // the token's head rows 32 ks .. 32 ks + 31 in Q|dO (bm) or Qrope (br).
    struct VisitCopy {
      __amdgpu_buffer_rsrc_t ars;
      const unsigned char *bm, *br;
      uint32_t aoff[KA];
      bool on;
    };
    const uint32_t aq0 = (uint32_t)((((lane & 3) ^ swz(16 * wave + (lane >> 2))) * 8) * 2);
    auto make_copy = [&](VisitCopy& vc, bool on, int tl, const int32_t (&pr)[KA]) {
      vc.on = on;
      if (!on) return;
      vc.ars = make_rsrc(Asrc + (int64_t)tl * a.E * 128, (int)(a.E * 128 * 2));
      const int p0 = tl * (int)a.E;
#pragma unroll
      for (int k = 0; k < KA; ++k) {
        // row 16 (wave + W k) + lane / 4: its swizzle equals that of row
        // 16 wave + lane / 4 (16 W k is a multiple of 8)
        vc.aoff[k] = pr[k] >= 0 ? (uint32_t)((pr[k] - p0) * 256) + aq0 : kOutside;
      }
      const int64_t hrow = (a.t0 + tl) * a.G;
      vc.bm = (const unsigned char*)(Bmain + hrow * 512);
      vc.br = (const unsigned char*)(a.qr + hrow * Dr);
    };
    const void* zero16 = (const void*)(((uint64_t)z_hi << 32) | z_lo);
    // copy part k (A instruction k and B instruction k) of stage ks (the
    // stage's offsets enter as opaque scalars, so that no per-stage copy of a
    // lane's addresses is kept; the offset field of an LDS-bound buffer load
    // would move the LDS destination as well)
    auto issue_copy = [&](const VisitCopy& vc, int ks, int k) {
      if (!vc.on) return;
      const uint32_t st = stage_lds(ks);
      if (k < KA) {
        uint32_t ko = 64u * ks;
        asm volatile("" : "+s"(ko));
        bdma16(vc.ars, vc.aoff[k] + ko, st + (wave + W * k) * 1024);
      }
      if (k < KBM && k < KB) {
        const uint32_t x = b_chunk[k];
        const unsigned char* bm = vc.bm + ks * (32 * 512 * 2);
        const unsigned char* br = vc.br + ks * (32 * 2 * Dr);
        asm volatile("" : "+s"(bm), "+s"(br));
        const bool live = 32 * ks + (int)((x >> 16) & 31) < G;
        const void* src = live ? (const void*)((((x >> 21) & 1) ? br : bm) + 2 * (x & 0x7fff)) : zero16;
        dma16(src, st + kStageA + (wave + W * k) * 1024);
      }
    };
    const int nw = vhi - vlo;
    // prologue: the four stages of the first visit (map slot 0)
    {
      int32_t p0r[KA];
      prim_of(0, p0r);
      VisitCopy vc;
      make_copy(vc, true, v_token(vlo), p0r);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        issue_copy(vc, ks, 0);
        issue_copy(vc, ks, 1);
      }
    }
    // stage 0's copies were issued first: 3 later stages' copies may be
    // outstanding
    wait_stages<3, KA, NBI, W>(wave);
    bar();
    V8b Bc[NB];
    uint4 a0[4], a1[4];
    rdB(lds_base(st0), Bc);
    rdA(lds_base(st0), 0, a0);
    int R = sh.rounds[0];
    int su = 0;   // map slot of visit w: w % 3
    for (int w = 0; w < nw; ++w, su = su == 2 ? 0 : su + 1) {
      const int s1 = su == 2 ? 0 : su + 1, s2 = su == 0 ? 2 : su - 1;   // slots of visits w + 1, w + 2
      const bool next = w + 1 < nw;
      // copies of visit w + 1, issued during visit w (its map was built a
      // visit ago and stays unchanged through visit w)
      VisitCopy vc;
      {
        int32_t pn[KA];
        prim_of(s1, pn);
        make_copy(vc, next, next ? v_token(vlo + w + 1) : 0, pn);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        unsigned char* buf = stage_buf(ks);
        const lds_p lb = lds_base(buf);
        // earlier rounds of a visit whose token lists some key more than once
        for (int r = 0; r + 1 < R; ++r) {
          if (r) {
            drop_rows(buf, su, r);
            rdB(lb, Bc);
            rdA(lb, 0, a0);
          }
          rdA(lb, 1, a1);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) mma(a0, Bc[nb], 0, nb);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) mma(a1, Bc[nb], 1, nb);
        }
        if (R > 1) {
          drop_rows(buf, su, R - 1);
          rdB(lb, Bc);
          rdA(lb, 0, a0);
        }
        // last round, with the barrier between the row groups
        rdA(lb, 1, a1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mma(a0, Bc[nb], 0, nb);
        __builtin_amdgcn_sched_barrier(0);
        // stage x + 1 exists unless this is the range's last stage; the
        // copies issued after those of stage x + 1 are those of the stages
        // x + 2 and x + 3 that exist
        if (next || ks < 3) {
          if (next || ks == 0) wait_stages<2, KA, NBI, W>(wave);
          else if (ks == 1) wait_stages<1, KA, NBI, W>(wave);
          else wait_vm<0>();
          bar();
          if (ks == 0) {
            if (vlo + w + 2 - wb + 1 > kWin) {   // visit w + 2 leaves the window
              wb = vlo + w;
              load_window();
              __syncthreads();
            }
            reset(s2);
            if (w + 2 < nw) issue_entries(vlo + w + 2, w & 1);
          } else if (ks == 2) {
            if (w + 2 < nw) build(s2, vlo + w + 2, w & 1);
          } else if (ks == 3) {
            R = sh.rounds[s1];
          }
        }
        // The reads of the next stage's operands run on the last stage as
        // well (of a buffer in LDS, results unused), so that both paths leave
        // the same reads in flight here and the compiler's waits before the
        // MFMAs below stay on the operands those MFMAs use.
        const lds_p nbuf = lds_base(stage_buf((ks + 1) & 3));
        rdA(nbuf, 0, a0);
        // row group 1, one column block at a time; B of stage x + 1 replaces
        // each block's operand once its MFMAs are issued, and the copies of
        // stage x + 4 (visit w + 1, stage ks: none on the last visit) go out
        // between the blocks
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          __builtin_amdgcn_sched_barrier(0);
          mma(a1, Bc[nb], 1, nb);
          __builtin_amdgcn_sched_barrier(0);
          Bc[nb] = rdB1(nbuf, nb);
          if (nb < 2) issue_copy(vc, ks, nb);
        }
      }
    }
  } else if (nks == 1) {
    // Up to 32 heads (one stage per visit): the four stage buffers rotate over
    // visits and stage copies run two visits ahead.  At the top of visit v
    // the map of visit v + 2 is built (its pairs were copied a visit ago) and
    // its stage is copied between the MFMAs of visit v; the pairs of visit
    // v + 3 are copied at the same time.  Each visit waits once, for copies
    // issued one and two visits earlier.
    auto rbuf = [&](int v) -> unsigned char* { return stage_buf((v - vlo) & 3); };
    auto rlds = [&](int v) -> uint32_t { return stage_lds((v - vlo) & 3); };
    auto ehalf = [&](int v) -> int { return (v - vlo) & 1; };
    // issue order: stage(vlo), pairs(vlo + 2), stage(vlo + 1)
    issue_stage(0, v_token(vlo), 0, rlds(vlo));
    if (vlo + 2 < vhi) issue_entries(vlo + 2, ehalf(vlo + 2));
    if (vlo + 1 < vhi) issue_stage(1, v_token(vlo + 1), 0, rlds(vlo + 1));
    for (int v = vlo; v < vhi; ++v) {
      const int u = (v - vlo) % 3;
      const int u2 = u == 0 ? 2 : u - 1;   // map slot of visit v + 2
      if (v - wb + 3 > kWin) {   // visits v .. v + 3 leave the window
        __syncthreads();
        wb = v;
        load_window();
        __syncthreads();
      }
      // stage(v) and pairs(v + 2) have landed once at most stage(v + 1),
      // issued after them, is outstanding
      if (v + 1 < vhi) wait_stages<1, KA, NBI, W>(wave);
      else wait_vm<0>();
      bar();
      const int R = sh.rounds[u];
      if (v + 3 < vhi) issue_entries(v + 3, ehalf(v + 3));
      if (v + 2 < vhi) build(u2, v + 2, ehalf(v + 2));   // slot u2 was cleared after visit v - 1
      bar();
      StageCopy sc;
      prep_stage(sc, v + 2 < vhi, u2, v + 2 < vhi ? v_token(v + 2) : 0, 0, rlds(v + 2));
      for (int r = 0; r < R; ++r) {
        if (r) drop_rows(rbuf(v), u, r);
        if constexpr (GP == 16) compute16(rbuf(v), sc);
        else compute(rbuf(v), sc);
        sc.on = false;
      }
      reset(u);   // this visit's map slot, for visit v + 3
    }
  } else if (nks <= 2) {
    // Up to 64 heads (one or two 32-head stages per visit): visits alternate
    // between the buffer pairs st0|st1 and st2|st3; the stages of visit v + 1
    // are copied while visit v is computed (its slot map was built a visit
    // earlier), so each visit waits once, for copies issued a visit ago.
    auto vbuf = [&](int v, int ks) -> unsigned char* { return stage_buf((((v - vlo) & 1) << 1) + ks); };
    auto vlds = [&](int v, int ks) -> uint32_t { return stage_lds((((v - vlo) & 1) << 1) + ks); };
    auto issue_visit = [&](int b, int v) {
      const int tl = v_token(v);
      for (int ks = 0; ks < nks; ++ks) issue_stage(b, tl, ks, vlds(v, ks));
    };
    // The pairs of visit v + 3 are copied at the top of visit v (the two
    // entry buffers alternate) and its slot map is built at the end of visit
    // v + 1: the top-of-visit wait covers both kinds of copies, each issued a
    // whole visit earlier.
    auto ehalf = [&](int v) -> int { return (v - vlo) & 1; };
    if (vlo + 2 < vhi) issue_entries(vlo + 2, ehalf(vlo + 2));
    issue_visit(0, vlo);
    for (int v = vlo; v < vhi; ++v) {
      const int u = (v - vlo) % 3;
      const int u1 = u == 2 ? 0 : u + 1, u2 = u == 0 ? 2 : u - 1;
      if (v - wb + 3 > kWin) {   // visits v .. v + 3 leave the window
        __syncthreads();
        wb = v;
        load_window();
        __syncthreads();
      }
      wait_vm<0>();   // the stages of visit v and the pairs of visit v + 2
      bar();
      const int R = sh.rounds[u];
      reset(u2);
      if (v + 3 < vhi) issue_entries(v + 3, ehalf(v + 3));
      // stage ks of visit v + 1 is copied between the MFMAs of stage ks of
      // visit v (a burst of copies stalls the issuing wave)
      const bool nxt = v + 1 < vhi;
      const int tl1 = nxt ? v_token(v + 1) : 0;
      for (int ks = 0; ks < nks; ++ks) {
        StageCopy sc;
        prep_stage(sc, nxt, u1, tl1, ks, vlds(v + 1, ks));
        for (int r = 0; r < R; ++r) {
          if (r) drop_rows(vbuf(v, ks), u, r);
          compute(vbuf(v, ks), sc);
          sc.on = false;   // the copies go out during the first round
        }
      }
      if (v + 2 < vhi) {
        bar();   // every thread's reset of map u2 precedes the build
        build(u2, v + 2, ehalf(v + 2));
      }
    }
  } else {
  {
    const int tl = v_token(vlo);
    StageCopy sc;
    prep_stage(sc, true, 0, tl, 0, L0);
    issue_all(sc);
    prep_stage(sc, nks > 1, 0, tl, 1, L1);
    issue_all(sc);
    prep_stage(sc, nks > 2, 0, tl, 2, L2);
    issue_all(sc);
  }

  // ---- one visit per iteration, four stages ---------------------------------
  int u = 0;   // map slot of visit v: (v - vlo) % 3
  for (int v = vlo; v < vhi; ++v, u = u == 2 ? 0 : u + 1) {
    const int u1 = u == 2 ? 0 : u + 1, u2 = u == 0 ? 2 : u - 1;
    if (v - wb + 2 > kWin) {   // visits v .. v + 2 leave the window
      __syncthreads();
      wb = v;
      load_window();
      __syncthreads();
    }
    const int tl = v_token(v);
    const bool more = v + 1 < vhi;
    const int tl1 = more ? v_token(v + 1) : 0;
    // stage 0 (this path waits for every copy at each stage)
    wait_vm<0>();
    bar();
    const int R = sh.rounds[u];
    reset(u2);
    if (v + 2 < vhi) issue_entries(v + 2, 0);
    StageCopy sc;
    sc.on = false;
    if (nks > 3) issue_stage(u, tl, 3, L3);
    for (int r = 0; r < R; ++r) {
      if (r) drop_rows(st0, u, r);
      compute(st0, sc);
      sc.on = false;   // the copies go out during the first round
    }
    // stages 1 .. 3: each issues the copy of the next visit's stage ks - 1
#pragma unroll
    for (int ks = 1; ks < 4; ++ks) {
      {
        wait_vm<0>();
        bar();
        // map of visit v + 2: its pairs were copied during stage 0
        if (ks == 3 && v + 2 < vhi) build(u2, v + 2, 0);
        if (more) issue_stage(u1, tl1, ks - 1, stage_lds(ks - 1));
        if (ks < nks) {
          for (int r = 0; r < R; ++r) {
            if (r) drop_rows(stage_buf(ks), u, r);
            compute(stage_buf(ks), sc);
            sc.on = false;
          }
        }
      }
    }
  }

  }

  // ---- partial of this token range ----------------------------------------
  float* out = a.part + (int64_t)tr * a.T2 * a.AW;
  const int ocol = c.ocol0 + cq * 16 * NB + n;
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = (int64_t)kb * kKB + (mb0 + mb) * 16 + 4 * g + i;
      if (row < a.T2) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) out[row * a.AW + ocol + 16 * nb] = C[mb][nb][i];
      }
    }
  }
}

}  // namespace

// GPK = 16 or 128: the variant for that padded head count only (each its own
// kernel, so that no variant's registers weigh on another's allocation); 0:
// the generic path.
template <typename TT, int GPK>
__global__ void __launch_bounds__(512, 1) k_keyblock(KbArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char st0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st1[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st2[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char st3[kStageBytes];
  __shared__ KbShared sh;
  __shared__ int32_t e_pair[2 * kEnt];   // pairs of the visits whose maps are built next
  __shared__ int32_t e_row[2 * kEnt];

  // XCD-aware unit order.  Workgroup b runs on XCD b % 8.  XCD x takes the
  // token ranges 16p + x and 16p + 15 - x (p = 0, 1, ...; a snake, so that
  // causal workloads, whose later ranges hold more pairs, stay balanced) and
  // runs each as (key block, column block) units in that order: the column
  // blocks of one key block read the same dS/P rows and the key blocks of one
  // range the same Q/dO rows, now through the same L2.
  const int xcd = blockIdx.x % kXcds, u = blockIdx.x / kXcds;
  const int per_tr = a.nKB * a.nCB;
  const int jt = u / per_tr, rem = u - jt * per_tr;
  const int tr = 16 * (jt >> 1) + ((jt & 1) ? 15 - xcd : xcd);
  if (tr >= a.nTR) return;
  const int kb = rem / a.nCB;
  const int cb = rem - kb * a.nCB;
  const ColBlock c = a.cbs[cb];
  const int64_t t_lo = (int64_t)tr * a.TR, t_hi = min<int64_t>(t_lo + a.TR, a.ntok);
  const int64_t nvis = *a.n_vis;
  const int vlo = __builtin_amdgcn_readfirstlane((int)lower_bound_i32(a.vis_key, nvis, (int64_t)kb * a.ntok + t_lo));
  const int vhi = __builtin_amdgcn_readfirstlane((int)lower_bound_i32(a.vis_key, nvis, (int64_t)kb * a.ntok + t_hi));
  if (threadIdx.x == 0 && cb == 0) a.nonempty[(int64_t)tr * a.nKB + kb] = vhi > vlo ? 1 : 0;
  if (vhi <= vlo) return;
  if constexpr (GPK == 16) {
    if (c.width == 256) kb_block<TT, 4, 16, 8>(a, c, tr, kb, vlo, vhi, st0, st1, st2, st3, &sh, e_pair, e_row);
    else kb_block<TT, 3, 16, 8>(a, c, tr, kb, vlo, vhi, st0, st1, st2, st3, &sh, e_pair, e_row);
  } else if constexpr (GPK == 128) {
    if (c.width == 256) kb_block<TT, 4, 128, 8>(a, c, tr, kb, vlo, vhi, st0, st1, st2, st3, &sh, e_pair, e_row);
    else kb_block<TT, 3, 128, 8>(a, c, tr, kb, vlo, vhi, st0, st1, st2, st3, &sh, e_pair, e_row);
  } else {
    if (c.width == 256) kb_block<TT, 4, 0, 8>(a, c, tr, kb, vlo, vhi, st0, st1, st2, st3, &sh, e_pair, e_row);
    else kb_block<TT, 3, 0, 8>(a, c, tr, kb, vlo, vhi, st0, st1, st2, st3, &sh, e_pair, e_row);
  }
}

// Visits of the sorted pairs: a visit starts where the composite key
// (key block * ntok + token) changes.
__global__ void __launch_bounds__(256) k_vis_flags(const int32_t* __restrict__ ck, int64_t n, int32_t sentinel,
                                                   int32_t* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t k = ck[i];
  flags[i] = (k < sentinel && (i == 0 || ck[i - 1] != k)) ? 1 : 0;
}

// vis_start / vis_key of each visit (from the scanned flags), the key row
// within its block of each sorted pair, and the visit count; vis_start[nvis]
// is the number of valid pairs.
__global__ void __launch_bounds__(256) k_vis_write(const int32_t* __restrict__ ck, const int32_t* __restrict__ svals,
                                                   const int32_t* __restrict__ rows, int64_t n, int64_t ntok,
                                                   int32_t sentinel, const int32_t* __restrict__ scan,
                                                   int32_t* __restrict__ vis_start, int32_t* __restrict__ vis_key,
                                                   int32_t* __restrict__ er, int32_t* __restrict__ n_vis) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t k = ck[i];
  if (k >= sentinel) {
    if (i == 0) {
      *n_vis = 0;
      vis_start[0] = 0;
    }
    return;
  }
  const int32_t kb = (int32_t)(k / ntok);
  er[i] = rows[svals[i]] - kb * kKB;
  const bool st = i == 0 || ck[i - 1] != k;
  const int32_t idx = scan[i];
  if (st) {
    vis_start[idx] = (int32_t)i;
    vis_key[idx] = k;
  }
  if (i + 1 == n || ck[i + 1] >= sentinel) {
    const int32_t nv = idx + (st ? 1 : 0);
    vis_start[nv] = (int32_t)(i + 1);
    *n_vis = nv;
  }
}

// Pairs of a chunk grouped by (key block, token) without a global sort: a
// counting sort whose counters sit in the (key block, token) grid, key block
// major.  k_bin_count histograms each token's valid positions over the key
// blocks (LDS atomics) into cnt and flg (count, count > 0); exclusive scans
// of both give every (key block, token) cell its first slot among the sorted
// pairs and its visit number; k_bin_scatter then writes each token's visits
// and places its pairs (pair id tl * E + j, key row within the block) at
// their cells' slots.  Within one cell the pairs land in no fixed order: a
// visit's slot map places each pair's row by key row, and pairs that share a
// key row (one token listing a key twice) hold identical rows, so the sums
// do not depend on that order.  The result matches the stable sort by key
// block (visits in (key block, token) order, vis_start[v + 1] - vis_start[v]
// pairs each).
// Runs of equal key blocks among the active lanes of a wave (the active
// lanes are a prefix: positions j < nvalid): `head` is set on a run's first
// lane, `len` there is the run's length, and `first` on every active lane is
// its run's first lane.  Sorted rows give long runs, so one LDS atomic per
// run replaces one per lane (they would all hit the same counter).
struct Run {
  bool head;
  int len, first;
};
__device__ __forceinline__ Run lane_run(int32_t kb, bool act, int lane) {
  const int32_t prev = __shfl_up(kb, 1);
  const bool head = act && (lane == 0 || prev != kb);
  const uint64_t heads = __ballot(head);
  const int nact = __popcll(__ballot(act));
  const uint64_t above = heads & ~((2ull << lane) - 1);
  const uint64_t upto = heads & ((2ull << lane) - 1);
  Run r;
  r.head = head;
  r.len = min(above ? (int)__builtin_ctzll(above) : 64, nact) - lane;
  r.first = upto ? 63 - (int)__builtin_clzll(upto) : lane;
  return r;
}

__global__ void __launch_bounds__(256) k_bin_count(const int32_t* __restrict__ rows,
                                                   const int32_t* __restrict__ nvalid, int64_t E, int32_t nkb,
                                                   int64_t ntok, int32_t* __restrict__ cnt,
                                                   int32_t* __restrict__ flg) {
  extern __shared__ int32_t hist[];   // nkb
  const int64_t tl = blockIdx.x;
  for (int i = threadIdx.x; i < nkb; i += 256) hist[i] = 0;
  __syncthreads();
  const int nv = nvalid[tl];
  const int32_t* r = rows + tl * E;
  const int lane = threadIdx.x & 63;
  for (int j0 = 0; j0 < nv; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const bool act = j < nv;
    const int32_t kb = act ? r[j] / kKB : -1;
    const Run run = lane_run(kb, act, lane);
    if (run.head) atomicAdd(&hist[kb], run.len);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nkb; i += 256) {
    const int32_t c = hist[i];
    cnt[(int64_t)i * ntok + tl] = c;
    flg[(int64_t)i * ntok + tl] = c > 0 ? 1 : 0;
  }
}

// goff, vidx: the exclusive scans of cnt and flg.
__global__ void __launch_bounds__(256) k_bin_scatter(const int32_t* __restrict__ rows,
                                                     const int32_t* __restrict__ nvalid, int64_t E, int32_t nkb,
                                                     int64_t ntok, const int32_t* __restrict__ goff,
                                                     const int32_t* __restrict__ vidx, int32_t* __restrict__ svals,
                                                     int32_t* __restrict__ er, int32_t* __restrict__ vis_start,
                                                     int32_t* __restrict__ vis_key, int32_t* __restrict__ n_vis) {
  extern __shared__ int32_t sh[];     // hist[nkb], cursor[nkb]
  int32_t* hist = sh;
  int32_t* cursor = sh + nkb;
  const int64_t tl = blockIdx.x;
  for (int i = threadIdx.x; i < nkb; i += 256) hist[i] = 0;
  __syncthreads();
  const int nv = nvalid[tl];
  const int32_t* r = rows + tl * E;
  const int lane = threadIdx.x & 63;
  for (int j0 = 0; j0 < nv; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const bool act = j < nv;
    const int32_t kb = act ? r[j] / kKB : -1;
    const Run run = lane_run(kb, act, lane);
    if (run.head) atomicAdd(&hist[kb], run.len);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nkb; i += 256) {
    const int64_t cell = (int64_t)i * ntok + tl;
    cursor[i] = goff[cell];
    if (hist[i] > 0) {
      const int32_t v = vidx[cell];
      vis_start[v] = goff[cell];
      vis_key[v] = (int32_t)cell;
    }
    if (cell == (int64_t)nkb * ntok - 1) {   // the grid's last cell closes the lists
      const int32_t nvis = vidx[cell] + (hist[i] > 0 ? 1 : 0);
      vis_start[nvis] = goff[cell] + hist[i];
      *n_vis = nvis;
    }
  }
  __syncthreads();
  for (int j0 = 0; j0 < nv; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const bool act = j < nv;
    const int32_t row = act ? r[j] : 0, kb = act ? row / kKB : -1;
    const Run run = lane_run(kb, act, lane);
    int32_t base = 0;
    if (run.head) base = atomicAdd(&cursor[kb], run.len);
    base = __shfl(base, run.first);
    if (act) {
      const int32_t pos = base + (lane - run.first);
      svals[pos] = (int32_t)(tl * E + j);
      er[pos] = row - kb * kKB;
    }
  }
}

void launch_kb_bins(const int32_t* rows, const int32_t* nvalid, int64_t E, int32_t nkb, int64_t ntok, int32_t* cnt,
                    int32_t* flg, int32_t* scan_tmp, int32_t* svals, int32_t* er, int32_t* vis_start, int32_t* vis_key,
                    int32_t* n_vis, hipStream_t s) {
  if (ntok == 0) return;
  hipLaunchKernelGGL(k_bin_count, dim3((unsigned)ntok), dim3(256), (size_t)nkb * 4, s, rows, nvalid, E, nkb, ntok,
                     cnt, flg);
  launch_scan_i32(cnt, (int64_t)nkb * ntok, scan_tmp, s);
  launch_scan_i32(flg, (int64_t)nkb * ntok, scan_tmp, s);
  hipLaunchKernelGGL(k_bin_scatter, dim3((unsigned)ntok), dim3(256), (size_t)nkb * 8, s, rows, nvalid, E, nkb, ntok,
                     cnt, flg, svals, er, vis_start, vis_key, n_vis);
}

// acc[row] += Σ_tr part[tr][row] over the token ranges whose (range, key
// block) was non-empty, in ascending range order.
// (first: the sum starts from 0 rather than acc, which the zero fill made the
// same bits; OUT: the last chunk's sums go straight to the outputs, rounded
// as k_cast rounds them, four columns at a time: D and Dr are multiples of 4)
template <typename TT, bool OUT>
__global__ void __launch_bounds__(256) k_kb_reduce(const float* __restrict__ part, const int32_t* __restrict__ nonempty,
                                                   int64_t T2, int64_t AW, int32_t nTR, int32_t nKB,
                                                   float* __restrict__ acc, int32_t first, int32_t D, int32_t Dr,
                                                   float kscale, uint16_t* __restrict__ dk, uint16_t* __restrict__ dkr,
                                                   uint16_t* __restrict__ dv) {
  const int64_t row = blockIdx.x;
  const int kb = (int)(row / kKB);
  for (int64_t col = threadIdx.x * 4; col < AW; col += 256 * 4) {
    float4 s = first ? make_float4(0.f, 0.f, 0.f, 0.f) : *(const float4*)(acc + row * AW + col);
    for (int tr = 0; tr < nTR; ++tr) {
      if (!nonempty[(int64_t)tr * nKB + kb]) continue;
      const float4 v = *(const float4*)(part + ((int64_t)tr * T2 + row) * AW + col);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    if constexpr (OUT) {
      const int c = (int)col;
      uint16_t* dst;
      float m = kscale;
      if (c < D) dst = dk + row * D + c;
      else if (c < D + Dr) dst = dkr + row * Dr + (c - D);
      else {
        dst = dv + row * D + (c - D - Dr);
        m = 1.f;
      }
      *(uint2*)dst = make_uint2((uint32_t)TT::from_f(s.x * m) | ((uint32_t)TT::from_f(s.y * m) << 16),
                                (uint32_t)TT::from_f(s.z * m) | ((uint32_t)TT::from_f(s.w * m) << 16));
    } else {
      *(float4*)(acc + row * AW + col) = s;
    }
  }
}

void launch_keyblock(int32_t dtype, const KbArgs& a, hipStream_t s) {
  // token ranges per XCD: two per group of 16 (see the unit order above)
  const int64_t per_xcd = 2 * (((int64_t)a.nTR + 15) / 16);
  const dim3 grid((unsigned)(kXcds * per_xcd * a.nKB * a.nCB)), block(512);
  if (a.Gp == 16) {
    if (dtype == SFAG_BF16) hipLaunchKernelGGL((k_keyblock<BF16, 16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_keyblock<FP16, 16>), grid, block, 0, s, a);
  } else if (a.Gp == 128) {
    if (dtype == SFAG_BF16) hipLaunchKernelGGL((k_keyblock<BF16, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_keyblock<FP16, 128>), grid, block, 0, s, a);
  } else {
    if (dtype == SFAG_BF16) hipLaunchKernelGGL((k_keyblock<BF16, 0>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_keyblock<FP16, 0>), grid, block, 0, s, a);
  }
}

void launch_visits(const int32_t* ck, const int32_t* svals, const int32_t* rows, int64_t n, int64_t ntok,
                   int32_t nkb, int32_t* flags, int32_t* scan_tmp, int32_t* vis_start, int32_t* vis_key, int32_t* er,
                   int32_t* n_vis, hipStream_t s) {
  const int32_t sentinel = (int32_t)((int64_t)nkb * ntok);
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_vis_flags, dim3(grid), dim3(256), 0, s, ck, n, sentinel, flags);
  launch_scan_i32(flags, n, scan_tmp, s);
  hipLaunchKernelGGL(k_vis_write, dim3(grid), dim3(256), 0, s, ck, svals, rows, n, ntok, sentinel, flags, vis_start,
                     vis_key, er, n_vis);
}

void launch_kb_reduce(const float* part, const int32_t* nonempty, int64_t T2, int64_t AW, int32_t nTR, int32_t nKB,
                      float* acc, bool first, const KbOut* out, hipStream_t s) {
  if (T2 == 0) return;
  const dim3 grid((unsigned)T2), block(256);
  const int32_t f = first ? 1 : 0;
  if (!out) {
    hipLaunchKernelGGL((k_kb_reduce<BF16, false>), grid, block, 0, s, part, nonempty, T2, AW, nTR, nKB, acc, f, 0, 0,
                       1.f, nullptr, nullptr, nullptr);
    return;
  }
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, part, nonempty, T2, AW, nTR, nKB, acc, f, out->D, out->Dr,
                       out->kscale, (uint16_t*)out->dk, (uint16_t*)out->dkr, (uint16_t*)out->dv);
  };
  if (out->dtype == SFAG_BF16) go(k_kb_reduce<BF16, true>);
  else go(k_kb_reduce<FP16, true>);
}

}  // namespace sfag
