// Host-side plan shared by the validation unit (plain C++) and the launch unit
// (HIP).  Holds copies of the caller's pointers and attributes, the derived
// sizes and the workspace layout; never the data.
#pragma once

#include <cstdint>
#include <string>

#include "sfag.h"

namespace sfag {

// How the per-(token, position) dK/dV contributions reach the key rows:
//   kScatterAtomic   fp32 atomic adds of each pair's row into the accumulators;
//   kScatterPartials each pair's row stored, then summed per key in CSR order;
//   kScatterKeyBlock contraction per block of 256 key rows over the tokens
//                    selecting them (pairs sorted by key block and token).
enum Scatter : int32_t { kScatterAtomic = 0, kScatterPartials = 1, kScatterKeyBlock = 2 };

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WorkspaceLayout {
  uint64_t status = 0;     // validation result (16 bytes) when options.validate; always at offset 0
  uint64_t seq_off = 0;    // TND: int32 q_off[B+1], kv_off[B+1]
  uint64_t delta = 0;      // fp32 (T1, G): rowsum(dO ∘ O)
  uint64_t acc = 0;        // fp32 (T2, AW): dK | dKrope | dV accumulators
  uint64_t nvalid = 0;     // int32 (chunk): valid positions per token of the chunk
  uint64_t rows = 0;       // int32 (chunk, E): global key row of each valid position
  uint64_t ds = 0;         // 16-bit (chunk, E, Gp): dS of each (token, position, head)
  uint64_t p = 0;          // 16-bit (chunk, E, Gp): P
  uint64_t partials = 0;   // fp32 (chunk, E, AW): per-pair dK|dKr|dV rows (partials scatter)
  uint64_t sort_keys[2] = {0, 0};  // int32 (chunk*E): radix sort ping-pong
  uint64_t sort_vals[2] = {0, 0};
  uint64_t sort_hist = 0;  // int32 (256, nblocks)
  uint64_t csr_off = 0;    // int32 (T2 + 1)
  uint64_t kb_part = 0;    // fp32 (nTR, T2, AW): per token-range partial sums
  uint64_t kb_nonempty = 0;  // int32 (nTR, nKB)
  uint64_t vis_flags = 0;  // int32 (chunk*E): visit starts, scanned in place
  uint64_t vis_start = 0;  // int32 (chunk*E + 1): first sorted pair of each visit
  uint64_t vis_key = 0;    // int32 (chunk*E): composite key of each visit
  uint64_t vis_er = 0;     // int32 (chunk*E): key row within its block of each sorted pair
  uint64_t vis_n = 0;      // int32: number of visits
  uint64_t kb_grid = 0;    // int32 (2, nKB, chunk): per (key block, token) counts and visit flags, then their scans
  uint64_t kb_grid_tmp = 0;  // int32: segment sums of the grid scans
  uint64_t dq_acc = 0;     // fp32 (chunk, G, D + Dr): dQ|dQrope sums when a token's positions are split
  uint64_t phase = 0;      // int32 (8 XCDs x 32): key row each XCD's token workgroups last reached (a hint)
  uint64_t total = 0;
};

struct Dims {
  int32_t layout = 0;      // 0 BSND, 1 TND
  int64_t B = 0, S1 = 0, S2 = 0, T1 = 0, T2 = 0;
  int64_t G = 0, D = 512, Dr = 0;
  int64_t K = 0, block = 1, E = 0;
  int32_t mode = 0;
  int64_t Gp = 0;          // heads padded for the dS/P buffers (16 or a multiple of 32)
  int64_t AW = 0;          // accumulator row width 2*D + Dr
  int64_t chunk = 0;       // tokens per chunk
  int32_t sort_bits = 0;   // bits of the CSR sort key (rows < T2, sentinel T2)
  int32_t kb_sort_bits = 0;  // bits of the key-block sort key (sentinel nKB * chunk)
  int64_t nKB = 0;         // key blocks of kKeyBlockRows rows
  int64_t TR = 0;          // tokens per range of the key-block kernel
  int64_t nTR = 0;         // token ranges per chunk
  int32_t row_split = 1;   // workgroups sharing one token's positions in the fused token kernel
};

uint64_t align256(uint64_t x);

// Workspace layout for `d` (chunk and flags already set).
WorkspaceLayout layout_for(const Dims& d, int32_t scatter, bool validate);

// Default workspace budgets of the backward and forward plans.
constexpr uint64_t kDefaultBudget = 48ull << 30;
constexpr uint64_t kDefaultForwardBudget = 16ull << 30;
// Key-block token ranges per default-size chunk.
constexpr int kDefaultRanges = 16;

// Key rows per block of the key-centric dK/dV contraction.
constexpr int kKeyBlockRows = 256;

// Key blocks up to which the key-block path groups pairs by per-token
// counting (counters in LDS) instead of the global radix sort.
constexpr int64_t kMaxBinBlocks = 8192;
inline bool kb_use_bins(const Dims& d) { return d.nKB <= kMaxBinBlocks && d.nKB <= 2 * d.E; }

// Radix-sort block geometry shared by host and kernels.
constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortBlock = kSortThreads * kSortItems;  // items per sort block

void set_error(const std::string& msg);

}  // namespace sfag

struct sfag_plan;
namespace sfag {
// Scatter path, chunking, token ranges and workspace layout of a validated
// plan from its shapes and options (phase 1 and sfag_plan_configure).
int plan_launch(sfag_plan* p);
}  // namespace sfag

struct sfag_plan {
  const void *q = nullptr, *k = nullptr, *v = nullptr, *idx = nullptr, *dout = nullptr, *out = nullptr;
  const void *smax = nullptr, *ssum = nullptr, *lq = nullptr, *lk = nullptr, *qr = nullptr, *kr = nullptr;
  void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dqr = nullptr, *dkr = nullptr;
  int32_t dtype = 0;
  bool deterministic = false;
  float scale = 0.f;
  int32_t scatter = 0;
  sfag_options opt{};      // tuning choices (all 0 = defaults)
  // forward plans: the outputs out / softmaxMax / softmaxSum
  bool forward = false;
  void *out_w = nullptr, *smax_w = nullptr, *ssum_w = nullptr;
  sfag::Dims d;
  sfag::WorkspaceLayout ws;
};
