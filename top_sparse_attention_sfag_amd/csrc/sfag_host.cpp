// Phase 1 of the two-phase call: argument validation, planning and workspace
// layout.  Plain C++ (no HIP headers): it reads no device memory.
//
// The checks follow the operator page "aclnnSparseFlashAttentionGrad":
// GetWorkspaceSize parameter table (dtypes, shapes, N2 = 1, D = 512, Dr = 64,
// sparseBlockSize, layout, sparseMode, preTokens/nextTokens, contiguity), the
// 返回值 table (which status code each failure class returns) and 规格约束
// (B in 1..256, S1/S2 up to 128K).
#include <cmath>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <new>
#include <sstream>
#include <string>

#include "sfag_plan.h"

namespace sfag {

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

static void carve(uint64_t& cursor, uint64_t& field, uint64_t bytes) {
  field = cursor;
  cursor = align256(cursor + bytes);
}

WorkspaceLayout layout_for(const Dims& d, int32_t scatter, bool validate) {
  const bool partials = scatter == kScatterPartials;
  const bool keyblock = scatter == kScatterKeyBlock;
  WorkspaceLayout w;
  uint64_t c = 0;
  const uint64_t ch = (uint64_t)d.chunk, E = (uint64_t)d.E;
  carve(c, w.status, validate ? 16 : 0);
  carve(c, w.seq_off, d.layout == 1 ? 2 * (uint64_t)(d.B + 1) * 4 : 0);
  carve(c, w.delta, (uint64_t)d.T1 * d.G * 4);
  carve(c, w.acc, (uint64_t)d.T2 * d.AW * 4);
  carve(c, w.nvalid, ch * 4);
  carve(c, w.rows, ch * E * 4);
  carve(c, w.ds, ch * E * d.Gp * 2);
  carve(c, w.p, ch * E * d.Gp * 2);
  if (partials) {
    const uint64_t n = ch * E;
    const uint64_t nblk = (n + kSortBlock - 1) / kSortBlock;
    carve(c, w.partials, n * d.AW * 4);
    carve(c, w.sort_keys[0], n * 4);
    carve(c, w.sort_keys[1], n * 4);
    carve(c, w.sort_vals[0], n * 4);
    carve(c, w.sort_vals[1], n * 4);
    carve(c, w.sort_hist, (256 * nblk + 256 * nblk / 4096 + 2) * 4);
    carve(c, w.csr_off, (uint64_t)(d.T2 + 1) * 4);
  }
  if (d.row_split > 1) carve(c, w.dq_acc, ch * (uint64_t)d.G * (d.D + d.Dr) * 4);
  carve(c, w.phase, 8 * 32 * 4);
  if (keyblock) {
    const uint64_t n = ch * E;
    if (kb_use_bins(d)) {
      // per-token counting: sorted pair ids, their key rows, the grid
      const uint64_t cells = (uint64_t)d.nKB * ch;
      carve(c, w.sort_vals[0], n * 4);
      carve(c, w.kb_grid, 2 * cells * 4);
      carve(c, w.kb_grid_tmp, ((cells + 4095) / 4096 + 2) * 4);
    } else {
      const uint64_t nblk = (n + kSortBlock - 1) / kSortBlock;
      carve(c, w.sort_keys[0], n * 4);
      carve(c, w.sort_keys[1], n * 4);
      carve(c, w.sort_vals[0], n * 4);
      carve(c, w.sort_vals[1], n * 4);
      carve(c, w.sort_hist, (256 * nblk + 256 * nblk / 4096 + 2) * 4);
      carve(c, w.vis_flags, n * 4);
    }
    carve(c, w.kb_part, (uint64_t)d.nTR * d.T2 * d.AW * 4);
    carve(c, w.kb_nonempty, (uint64_t)d.nTR * d.nKB * 4);
    carve(c, w.vis_start, (n + 1) * 4);
    carve(c, w.vis_key, n * 4);
    carve(c, w.vis_er, n * 4);
    carve(c, w.vis_n, 4);
  }
  w.total = c;
  return w;
}

}  // namespace sfag

using namespace sfag;

namespace {

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

int64_t numel(const sfag_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

bool contiguous(const sfag_tensor* t) {
  int64_t s = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != s) return false;
    s *= t->shape[i];
  }
  return true;
}

std::string shape_str(const sfag_tensor* t) {
  std::ostringstream o;
  o << "(";
  for (int i = 0; i < t->ndim; ++i) o << (i ? "," : "") << t->shape[i];
  o << ")";
  return o.str();
}

bool shape_is(const sfag_tensor* t, std::initializer_list<int64_t> s) {
  if (t->ndim != (int)s.size()) return false;
  int i = 0;
  for (int64_t v : s) {
    if (t->shape[i++] != v) return false;
  }
  return true;
}

bool same_shape(const sfag_tensor* a, const sfag_tensor* b) {
  if (a->ndim != b->ndim) return false;
  for (int i = 0; i < a->ndim; ++i)
    if (a->shape[i] != b->shape[i]) return false;
  return true;
}

constexpr int64_t kMaxTokensPerSeq = 131072;  // 规格约束: S1, S2 up to 128K
constexpr int64_t kMaxBatch = 256;            // 规格约束: B 1..256
constexpr int64_t kWindow = 2147483647;       // preTokens / nextTokens: only this value

}  // namespace

extern "C" const char* sfag_last_error(void) { return g_error.c_str(); }

extern "C" void sfag_plan_destroy(sfag_plan* plan) { delete plan; }

extern "C" int sfag_workspace_size(
    const sfag_tensor* query, const sfag_tensor* key, const sfag_tensor* value, const sfag_tensor* sparseIndices,
    const sfag_tensor* dOut, const sfag_tensor* out, const sfag_tensor* softmaxMax, const sfag_tensor* softmaxSum,
    const sfag_tensor* lensQ, const sfag_tensor* lensKv, const sfag_tensor* queryRope, const sfag_tensor* keyRope,
    double scaleValue, int64_t sparseBlockSize, const char* layoutOptional, int64_t sparseMode, int64_t preTokens,
    int64_t nextTokens, bool deterministic, const sfag_tensor* dQueryOut, const sfag_tensor* dKeyOut,
    const sfag_tensor* dValueOut, const sfag_tensor* dQueryRopeOut, const sfag_tensor* dKeyRopeOut,
    uint64_t* workspaceSize, sfag_plan** plan) {
  set_error("");
  if (plan) *plan = nullptr;
  // ---- 161001: required arguments present --------------------------------
  struct Named {
    const sfag_tensor* t;
    const char* name;
  };
  const Named required[] = {{query, "query"},        {key, "key"},           {value, "value"},
                            {sparseIndices, "sparseIndices"}, {dOut, "dOut"}, {out, "out"},
                            {softmaxMax, "softmaxMax"}, {softmaxSum, "softmaxSum"}, {dQueryOut, "dQueryOut"},
                            {dKeyOut, "dKeyOut"},    {dValueOut, "dValueOut"}};
  for (const Named& n : required)
    if (!n.t) return fail(SFAG_ERR_NULLPTR, std::string(n.name) + " is NULL");
  if (!workspaceSize || !plan) return fail(SFAG_ERR_NULLPTR, "workspaceSize or plan output pointer is NULL");
  const bool rope = queryRope || keyRope;
  if (rope && !(queryRope && keyRope))
    return fail(SFAG_ERR_PARAM_INVALID, "queryRope and keyRope must be given together");
  if (rope && (!dQueryRopeOut || !dKeyRopeOut))
    return fail(SFAG_ERR_NULLPTR, "dQueryRopeOut and dKeyRopeOut are required when rope inputs are given");

  const Named all[] = {{query, "query"},           {key, "key"},
                       {value, "value"},           {sparseIndices, "sparseIndices"},
                       {dOut, "dOut"},             {out, "out"},
                       {softmaxMax, "softmaxMax"}, {softmaxSum, "softmaxSum"},
                       {lensQ, "actualSeqLengthsQuery"}, {lensKv, "actualSeqLengthsKv"},
                       {queryRope, "queryRope"},   {keyRope, "keyRope"},
                       {dQueryOut, "dQueryOut"},   {dKeyOut, "dKeyOut"},
                       {dValueOut, "dValueOut"},   {rope ? dQueryRopeOut : nullptr, "dQueryRopeOut"},
                       {rope ? dKeyRopeOut : nullptr, "dKeyRopeOut"}};
  for (const Named& n : all) {
    if (!n.t) continue;
    if (n.t->ndim < 1 || n.t->ndim > 4) return fail(SFAG_ERR_PARAM_INVALID, std::string(n.name) + ": ndim must be 1..4");
    for (int i = 0; i < n.t->ndim; ++i)
      if (n.t->shape[i] < 0) return fail(SFAG_ERR_PARAM_INVALID, std::string(n.name) + ": negative extent");
    if (numel(n.t) > 0 && !n.t->data) return fail(SFAG_ERR_NULLPTR, std::string(n.name) + ": data is NULL");
  }
  // ---- 161002: dtypes and contiguity --------------------------------------
  const int32_t ft = query->dtype;
  if (ft != SFAG_BF16 && ft != SFAG_FP16) return fail(SFAG_ERR_PARAM_INVALID, "query dtype must be bf16 or fp16");
  const Named floats[] = {{key, "key"}, {value, "value"}, {dOut, "dOut"}, {out, "out"}, {queryRope, "queryRope"},
                          {keyRope, "keyRope"}, {dQueryOut, "dQueryOut"}, {dKeyOut, "dKeyOut"},
                          {dValueOut, "dValueOut"}, {rope ? dQueryRopeOut : nullptr, "dQueryRopeOut"},
                          {rope ? dKeyRopeOut : nullptr, "dKeyRopeOut"}};
  for (const Named& n : floats)
    if (n.t && n.t->dtype != ft) return fail(SFAG_ERR_PARAM_INVALID, std::string(n.name) + " dtype differs from query");
  if (sparseIndices->dtype != SFAG_INT32) return fail(SFAG_ERR_PARAM_INVALID, "sparseIndices must be int32");
  if (softmaxMax->dtype != SFAG_FP32 || softmaxSum->dtype != SFAG_FP32)
    return fail(SFAG_ERR_PARAM_INVALID, "softmaxMax and softmaxSum must be float32");
  if ((lensQ && lensQ->dtype != SFAG_INT32) || (lensKv && lensKv->dtype != SFAG_INT32))
    return fail(SFAG_ERR_PARAM_INVALID, "actual sequence lengths must be int32");
  for (const Named& n : all)
    if (n.t && !contiguous(n.t)) return fail(SFAG_ERR_PARAM_INVALID, std::string(n.name) + " is not contiguous");
  if (!std::isfinite(scaleValue)) return fail(SFAG_ERR_PARAM_INVALID, "scaleValue must be finite");

  // ---- 561002: attributes -------------------------------------------------
  std::string layout = layoutOptional ? layoutOptional : "BSND";
  Dims d;
  if (layout == "BSND") d.layout = 0;
  else if (layout == "TND") d.layout = 1;
  else return fail(SFAG_ERR_TILING, "layout must be BSND or TND, got '" + layout + "'");
  if (sparseMode != 0 && sparseMode != 3) return fail(SFAG_ERR_TILING, "sparseMode must be 0 or 3");
  if (sparseBlockSize != 1 && sparseBlockSize != 8 && sparseBlockSize != 16 && sparseBlockSize != 32 &&
      sparseBlockSize != 64)
    return fail(SFAG_ERR_TILING, "sparseBlockSize must be one of 1, 8, 16, 32, 64");
  if (preTokens != kWindow || nextTokens != kWindow)
    return fail(SFAG_ERR_TILING, "preTokens and nextTokens must be 2147483647");
  d.mode = (int32_t)sparseMode;
  d.block = sparseBlockSize;

  // ---- 561002: shapes -----------------------------------------------------
  const int qd = d.layout == 0 ? 4 : 3;
  if (query->ndim != qd || key->ndim != qd || value->ndim != qd || dOut->ndim != qd || out->ndim != qd ||
      sparseIndices->ndim != qd)
    return fail(SFAG_ERR_TILING, "query/key/value/dOut/out/sparseIndices must have " + std::to_string(qd) +
                                     " dims for layout " + layout);
  if (d.layout == 0) {
    d.B = query->shape[0];
    d.S1 = query->shape[1];
    d.G = query->shape[2];
    d.D = query->shape[3];
    d.S2 = key->shape[1];
    d.T1 = d.B * d.S1;
    d.T2 = d.B * d.S2;
    if (key->shape[0] != d.B) return fail(SFAG_ERR_TILING, "key batch differs from query batch");
    if (d.B > kMaxBatch) return fail(SFAG_ERR_TILING, "B must be at most 256");
    if (d.S1 > kMaxTokensPerSeq || d.S2 > kMaxTokensPerSeq) return fail(SFAG_ERR_TILING, "S1 and S2 must be at most 128K");
  } else {
    d.T1 = query->shape[0];
    d.G = query->shape[1];
    d.D = query->shape[2];
    d.T2 = key->shape[0];
    if (!lensQ || !lensKv) return fail(SFAG_ERR_TILING, "TND layout needs actualSeqLengthsQuery and actualSeqLengthsKv");
    if (lensQ->ndim != 1 || lensKv->ndim != 1 || lensQ->shape[0] != lensKv->shape[0])
      return fail(SFAG_ERR_TILING, "actual sequence lengths must both have shape (B,)");
    d.B = lensQ->shape[0];
    if (d.B < 1 || d.B > kMaxBatch) return fail(SFAG_ERR_TILING, "B must be in 1..256");
    if (d.T1 > kMaxBatch * kMaxTokensPerSeq || d.T2 > kMaxBatch * kMaxTokensPerSeq)
      return fail(SFAG_ERR_TILING, "T1/T2 exceed 256 sequences of 128K tokens");
  }
  const int64_t N2 = key->shape[qd - 2];
  if (N2 != 1) return fail(SFAG_ERR_TILING, "N2 must be 1 (one shared key/value head)");
  if (d.D != 512) return fail(SFAG_ERR_TILING, "D must be 512");
  if (d.G < 1 || d.G > 128) return fail(SFAG_ERR_TILING, "N1 must be in 1..128");
  if (key->shape[qd - 1] != d.D) return fail(SFAG_ERR_TILING, "key last dim must equal query's (512)");
  if (!same_shape(value, key)) return fail(SFAG_ERR_TILING, "value shape must equal key shape");
  if (!same_shape(dOut, query) || !same_shape(out, query)) return fail(SFAG_ERR_TILING, "dOut and out must have query's shape");
  d.K = sparseIndices->shape[qd - 1];
  const bool idx_ok = d.layout == 0 ? shape_is(sparseIndices, {d.B, d.S1, 1, d.K}) : shape_is(sparseIndices, {d.T1, 1, d.K});
  if (!idx_ok) return fail(SFAG_ERR_TILING, "sparseIndices shape " + shape_str(sparseIndices) + " does not match query");
  const bool st_ok = d.layout == 0 ? shape_is(softmaxMax, {d.B, 1, d.S1, d.G}) && shape_is(softmaxSum, {d.B, 1, d.S1, d.G})
                                   : shape_is(softmaxMax, {1, d.T1, d.G}) && shape_is(softmaxSum, {1, d.T1, d.G});
  if (!st_ok) return fail(SFAG_ERR_TILING, "softmaxMax/softmaxSum must be (B,1,S1,N1) or (1,T1,N1)");
  if (rope) {
    d.Dr = queryRope->shape[queryRope->ndim - 1];
    if (d.Dr != 64) return fail(SFAG_ERR_TILING, "Drope must be 64");
    const bool qr_ok = d.layout == 0 ? shape_is(queryRope, {d.B, d.S1, d.G, 64}) : shape_is(queryRope, {d.T1, d.G, 64});
    const bool kr_ok = d.layout == 0 ? shape_is(keyRope, {d.B, d.S2, 1, 64}) : shape_is(keyRope, {d.T2, 1, 64});
    if (!qr_ok || !kr_ok) return fail(SFAG_ERR_TILING, "queryRope/keyRope shapes do not match query/key");
    if (!same_shape(dQueryRopeOut, queryRope) || !same_shape(dKeyRopeOut, keyRope))
      return fail(SFAG_ERR_TILING, "rope gradient outputs must match the rope inputs");
  }
  if (!same_shape(dQueryOut, query) || !same_shape(dKeyOut, key) || !same_shape(dValueOut, value))
    return fail(SFAG_ERR_TILING, "gradient outputs must match their inputs' shapes");

  d.E = d.K * d.block;
  d.Gp = d.G <= 16 ? 16 : (d.G + 31) / 32 * 32;
  d.AW = 2 * d.D + d.Dr;
  int bits = 1;
  while (((int64_t)1 << bits) <= d.T2) ++bits;
  d.sort_bits = bits;

  auto* p = new (std::nothrow) sfag_plan();
  if (!p) return fail(SFAG_ERR_RUNTIME, "out of host memory");
  p->q = query->data; p->k = key->data; p->v = value->data; p->idx = sparseIndices->data;
  p->dout = dOut->data; p->out = out->data; p->smax = softmaxMax->data; p->ssum = softmaxSum->data;
  p->lq = d.layout == 1 ? lensQ->data : nullptr;
  p->lk = d.layout == 1 ? lensKv->data : nullptr;
  p->qr = rope ? queryRope->data : nullptr; p->kr = rope ? keyRope->data : nullptr;
  p->dq = dQueryOut->data; p->dk = dKeyOut->data; p->dv = dValueOut->data;
  p->dqr = rope ? dQueryRopeOut->data : nullptr; p->dkr = rope ? dKeyRopeOut->data : nullptr;
  p->dtype = ft;
  p->deterministic = deterministic;
  p->scale = (float)scaleValue;

  p->scatter = kScatterAtomic;
  p->d = d;
  const int rc = plan_launch(p);
  if (rc != SFAG_OK) {
    delete p;
    return rc;
  }
  *workspaceSize = p->ws.total;
  *plan = p;
  return SFAG_OK;
}

namespace sfag {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest chunk (a multiple of `tr` tokens, at least `tr`) whose workspace
// fixed + chunk * per_tok + (chunk / tr) * per_range stays within `budget`.
int64_t chunk_within(uint64_t budget, uint64_t fixed, uint64_t per_tok, uint64_t per_range, int64_t tr) {
  const uint64_t unit = (uint64_t)tr * per_tok + per_range;
  if (budget <= fixed || unit == 0) return tr;
  const uint64_t n = (budget - fixed) / unit;
  return (int64_t)std::max<uint64_t>(1, std::min<uint64_t>(n, (uint64_t)1 << 40)) * tr;
}

// Chunk of at most `cmax` tokens (a multiple of tr) that splits T1 into equal
// chunks: as many chunks as cmax forces, each a whole number of ranges.
int64_t balanced_chunk(int64_t T1, int64_t cmax, int64_t tr) {
  const int64_t n = ceil_div(T1, cmax);
  return std::min<int64_t>(cmax, ceil_div(ceil_div(T1, n), tr) * tr);
}

}  // namespace

int plan_launch(sfag_plan* p) {
  Dims& d = p->d;
  const sfag_options& o = p->opt;
  const bool validate = o.validate != 0;
  d.chunk = 0;
  d.TR = d.nTR = 0;
  d.row_split = 1;
  d.kb_sort_bits = 0;
  d.nKB = (d.T2 + kKeyBlockRows - 1) / kKeyBlockRows;
  // Bytes that do not scale with the chunk: validation word, TND offsets,
  // Delta, accumulators (and the CSR offsets of the partials path).
  auto fixed_bytes = [&](bool partials) {
    uint64_t f = (validate ? 256 : 0) + (d.layout == 1 ? align256(2 * (uint64_t)(d.B + 1) * 4) : 0);
    if (!p->forward) f += align256((uint64_t)d.T1 * d.G * 4) + align256((uint64_t)d.T2 * d.AW * 4);
    if (partials) f += align256((uint64_t)(d.T2 + 1) * 4);
    return f + (64u << 10);   // alignment of the remaining regions
  };
  // pair numbering: chunk * E and the key-block sort key stay below 2^31
  const int64_t pair_cap = d.E > 0 ? 0x7fffffffLL / d.E : ((int64_t)1 << 40);

  if (p->forward) {
    p->scatter = kScatterAtomic;
    if (d.T1 == 0) {
      p->ws = WorkspaceLayout();
      if (validate) {
        uint64_t c = 0;
        carve(c, p->ws.status, 16);
        carve(c, p->ws.seq_off, d.layout == 1 ? 2 * (uint64_t)(d.B + 1) * 4 : 0);
        p->ws.total = c;
      }
      return SFAG_OK;
    }
    const uint64_t budget = o.workspaceBudget ? o.workspaceBudget : kDefaultForwardBudget;
    int64_t cmax = chunk_within(budget, fixed_bytes(false), 4 + (uint64_t)d.E * 4, 0, 1);
    if (o.chunkTokens > 0) cmax = std::min<int64_t>(cmax, o.chunkTokens);
    cmax = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(cmax, pair_cap), d.T1));
    d.chunk = balanced_chunk(d.T1, cmax, 1);
    WorkspaceLayout w;
    uint64_t c = 0;
    carve(c, w.status, validate ? 16 : 0);
    carve(c, w.seq_off, d.layout == 1 ? 2 * (uint64_t)(d.B + 1) * 4 : 0);
    carve(c, w.nvalid, (uint64_t)d.chunk * 4);
    carve(c, w.rows, (uint64_t)d.chunk * d.E * 4);
    w.total = c;
    p->ws = w;
    return SFAG_OK;
  }

  // dK/dV path.  When a token selects a sizeable fraction of the keys it can
  // reach (estimated from the shapes alone), the key-block contraction wins:
  // it moves no per-pair rows and is deterministic.  Otherwise the per-pair
  // rows go through the CSR reduction (deterministic) or fp32 atomics.
  {
    double reach;  // average number of key positions a token may select
    if (d.layout == 0) {
      reach = d.mode == 3 ? (double)d.S2 - (double)d.S1 + 0.5 * (double)(d.S1 + 1) : (double)d.S2;
    } else {
      const double lk = d.B > 0 ? (double)d.T2 / (double)d.B : 0.0;
      reach = d.mode == 3 ? 0.5 * lk : lk;
    }
    if (reach < 1.0) reach = 1.0;
    const double density = (double)d.E / reach;
    const int32_t other = p->deterministic ? kScatterPartials : kScatterAtomic;
    int32_t sc = density >= 0.125 ? kScatterKeyBlock : other;
    if (o.scatter == SFAG_SCATTER_KEYBLOCK) sc = kScatterKeyBlock;
    if (o.scatter == SFAG_SCATTER_PARTIALS) sc = kScatterPartials;
    if (o.scatter == SFAG_SCATTER_ATOMIC) sc = other;
    // the key-block kernel addresses one token's dS/P rows (E x Gp halves)
    // through a buffer resource with a 31-bit size, and needs key rows
    if (sc == kScatterKeyBlock && ((uint64_t)d.E * (uint64_t)d.Gp * 2 > 0x7fffffffULL || d.nKB == 0)) sc = other;
    p->scatter = sc;
  }
  const bool partials = p->scatter == kScatterPartials;
  const bool keyblock = p->scatter == kScatterKeyBlock;
  if (d.T1 == 0) {  // empty query: the outputs are zero-filled, no workspace beyond validation
    p->ws = WorkspaceLayout();
    if (validate) {
      uint64_t c = 0;
      carve(c, p->ws.status, 16);
      carve(c, p->ws.seq_off, d.layout == 1 ? 2 * (uint64_t)(d.B + 1) * 4 : 0);
      p->ws.total = c;
    }
    return SFAG_OK;
  }
  // Chunk-sized bytes per token: index rows, dS and P (and for the partials
  // scatter the per-pair rows and the sort buffers; for the key-block path
  // the sort and visit buffers).
  uint64_t per_tok = 4 + (uint64_t)d.E * 4 + 2 * (uint64_t)d.E * d.Gp * 2;
  if (partials) per_tok += (uint64_t)d.E * d.AW * 4 + 4 * (uint64_t)d.E * 4 + 64;
  if (keyblock) per_tok += 8 * (uint64_t)d.E * 4 + 64;
  const uint64_t fixed = fixed_bytes(partials);
  // the key-block sort key (key block * chunk + token) stays below 2^31
  const int64_t cap = keyblock ? std::min<int64_t>(pair_cap, 0x7ffffffeLL / std::max<int64_t>(1, d.nKB)) : pair_cap;
  if (cap < 1) return fail(SFAG_ERR_TILING, "K * sparseBlockSize too large for 32-bit pair indices");
  int64_t tr = 1;
  uint64_t part_bytes = 0;
  if (keyblock) {
    // Token ranges of the key-block kernel, fixed in absolute token
    // coordinates from the shapes alone (never from the budget or the
    // chunking, so that the deterministic sums keep one order): the default
    // chunk (what the default budget holds, balanced over T1) split into
    // keyBlockRanges ranges (16: the XCD snake pairs ranges x and 15 - x),
    // fewer when that would leave under 8 tokens per range or need more than
    // 4 GiB of fp32 range partials per chunk.
    part_bytes = (uint64_t)d.T2 * d.AW * 4;
    int64_t ranges = o.keyBlockRanges > 0 ? o.keyBlockRanges : kDefaultRanges;
    if (part_bytes > 0) ranges = std::min<int64_t>(ranges, std::max<int64_t>(1, (int64_t)((4ull << 30) / part_bytes)));
    int64_t cdef = chunk_within(kDefaultBudget > ranges * part_bytes ? kDefaultBudget - ranges * part_bytes : 0,
                                fixed, per_tok, 0, 1);
    cdef = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(cdef, cap), d.T1));
    cdef = balanced_chunk(d.T1, cdef, 1);
    ranges = std::max<int64_t>(1, std::min<int64_t>(ranges, cdef / 8));
    tr = ceil_div(cdef, ranges);
  }
  const uint64_t budget = o.workspaceBudget ? o.workspaceBudget : kDefaultBudget;
  int64_t cmax = chunk_within(budget, fixed, per_tok, part_bytes, tr);
  if (o.chunkTokens > 0) cmax = std::min<int64_t>(cmax, std::max<int64_t>(tr, o.chunkTokens / tr * tr));
  cmax = std::min<int64_t>(cmax, std::max<int64_t>(tr, cap / tr * tr));
  cmax = std::min<int64_t>(cmax, ceil_div(d.T1, tr) * tr);
  if (cmax > cap) return fail(SFAG_ERR_TILING, "K * sparseBlockSize too large for 32-bit pair indices");
  d.chunk = balanced_chunk(d.T1, cmax, tr);
  // With few tokens (the fused token kernel, N1 <= 16, gives one workgroup
  // per token) a token's positions are split over up to 4 workgroups, each
  // at least 64 positions, which add their dQ|dQrope sums into an fp32
  // buffer (4 heads, 128 tokens, top-1024 of 2048 keys: token kernel 0.200
  // ms unsplit, 0.126 ms in 4 shares, 0.140 ms in 8).  The shares' atomic
  // sums have no fixed order, so deterministic calls never split.
  if (d.Gp < 32 && !p->deterministic) {
    int64_t sp = std::min<int64_t>(4, std::min<int64_t>(ceil_div(1024, d.chunk), d.E / 64));
    if (o.rowSplit > 0) sp = o.rowSplit;
    d.row_split = (int32_t)std::max<int64_t>(1, std::min<int64_t>(8, sp));
  }
  if (keyblock) {
    d.TR = tr;
    d.nTR = ceil_div(d.chunk, tr);
    int kbits = 1;
    while (((int64_t)1 << kbits) <= d.nKB) ++kbits;  // the sort runs over key-block ids only
    d.kb_sort_bits = kbits;
  }
  p->ws = layout_for(d, p->scatter, validate);
  return SFAG_OK;
}

}  // namespace sfag

// Forward pass (produces out, softmaxMax, softmaxSum).  The shared inputs and
// the three outputs obey the same rules as in the backward call, so the
// backward validation runs on them, with the outputs standing in for dOut and
// the statistics and the inputs for the gradient outputs (same shapes and
// dtypes by construction).  The workspace holds the TND offsets and the
// decoded key rows of one chunk of tokens.
extern "C" int sfag_forward_workspace_size(
    const sfag_tensor* query, const sfag_tensor* key, const sfag_tensor* value, const sfag_tensor* sparseIndices,
    const sfag_tensor* lensQ, const sfag_tensor* lensKv, const sfag_tensor* queryRope, const sfag_tensor* keyRope,
    double scaleValue, int64_t sparseBlockSize, const char* layoutOptional, int64_t sparseMode,
    const sfag_tensor* out, const sfag_tensor* softmaxMax, const sfag_tensor* softmaxSum, uint64_t* workspaceSize,
    sfag_plan** plan) {
  if (plan) *plan = nullptr;
  if (!out || !softmaxMax || !softmaxSum) return fail(SFAG_ERR_NULLPTR, "out, softmaxMax and softmaxSum are required");
  if (!workspaceSize || !plan) return fail(SFAG_ERR_NULLPTR, "workspaceSize or plan output pointer is NULL");
  sfag_plan* p = nullptr;
  uint64_t ws = 0;
  const int rc = sfag_workspace_size(query, key, value, sparseIndices, out, out, softmaxMax, softmaxSum, lensQ,
                                     lensKv, queryRope, keyRope, scaleValue, sparseBlockSize, layoutOptional,
                                     sparseMode, kWindow, kWindow, false, query, key, value, queryRope, keyRope,
                                     &ws, &p);
  if (rc != SFAG_OK) return rc;
  p->forward = true;
  p->out_w = out->data;
  p->smax_w = softmaxMax->data;
  p->ssum_w = softmaxSum->data;
  const int rc2 = plan_launch(p);
  if (rc2 != SFAG_OK) {
    delete p;
    return rc2;
  }
  *workspaceSize = p->ws.total;
  *plan = p;
  return SFAG_OK;
}

extern "C" int sfag_plan_configure(sfag_plan* plan, const sfag_options* options, uint64_t* workspaceSize) {
  set_error("");
  if (!plan || !workspaceSize) return fail(SFAG_ERR_NULLPTR, "plan or workspaceSize is NULL");
  const sfag_options o = options ? *options : sfag_options{};
  if (o.scatter < SFAG_SCATTER_AUTO || o.scatter > SFAG_SCATTER_ATOMIC)
    return fail(SFAG_ERR_PARAM_INVALID, "options.scatter must be one of SFAG_SCATTER_*");
  if (o.tokenPath < SFAG_TOKEN_AUTO || o.tokenPath > SFAG_TOKEN_SPLIT)
    return fail(SFAG_ERR_PARAM_INVALID, "options.tokenPath must be one of SFAG_TOKEN_*");
  if (o.tokenOrder < SFAG_ORDER_AUTO || o.tokenOrder > SFAG_ORDER_DESCENDING)
    return fail(SFAG_ERR_PARAM_INVALID, "options.tokenOrder must be one of SFAG_ORDER_*");
  if (o.concurrent < SFAG_CONCURRENT_AUTO || o.concurrent > SFAG_CONCURRENT_ON)
    return fail(SFAG_ERR_PARAM_INVALID, "options.concurrent must be one of SFAG_CONCURRENT_*");
  if (o.rowSplit < 0 || o.rowSplit > 8) return fail(SFAG_ERR_PARAM_INVALID, "options.rowSplit must be 0..8");
  if (o.keyBlockRanges < 0 || o.keyBlockRanges > 1024)
    return fail(SFAG_ERR_PARAM_INVALID, "options.keyBlockRanges must be 0..1024");
  if (o.chunkTokens < 0) return fail(SFAG_ERR_PARAM_INVALID, "options.chunkTokens must be >= 0");
  if (o.validate != 0 && o.validate != 1) return fail(SFAG_ERR_PARAM_INVALID, "options.validate must be 0 or 1");
  const sfag_options old = plan->opt;
  plan->opt = o;
  const int rc = plan_launch(plan);
  if (rc != SFAG_OK) {
    plan->opt = old;
    (void)plan_launch(plan);
    return rc;
  }
  *workspaceSize = plan->ws.total;
  return SFAG_OK;
}
