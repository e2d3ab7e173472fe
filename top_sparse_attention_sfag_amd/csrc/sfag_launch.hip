// Phase 2 of the two-phase call (the operator page's aclnnSparseFlashAttentionGrad
// execute step): carve the caller's workspace and enqueue the kernels on the
// caller's stream.  Also the stand-alone index inversion entry point.
#include <algorithm>
#include <cstdlib>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "sfag_device.h"
#include "sfag_kernels.h"
#include "sfag_plan.h"

using namespace sfag;

namespace {

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SFAG_ERR_RUNTIME, std::string(what) + ": " + hipGetErrorString(e));
  return SFAG_OK;
}

template <typename T>
T* at(void* base, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Optional per-kernel timing: HIP events recorded on the caller's stream
// around each kernel group, read back (and accumulated per name) on demand.
struct PendingTiming {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<PendingTiming> g_prof_pending;
std::map<std::string, std::pair<double, int64_t>> g_prof_acc;

struct TimedScope {
  bool on;
  PendingTiming t;
  hipStream_t s;
  TimedScope(const char* name, hipStream_t stream) : on(false), s(stream) {
    {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      on = g_prof_on;
    }
    if (!on) return;
    t.name = name;
    if (hipEventCreate(&t.start) != hipSuccess || hipEventCreate(&t.stop) != hipSuccess) {
      on = false;
      return;
    }
    (void)hipEventRecord(t.start, s);
  }
  ~TimedScope() {
    if (!on) return;
    (void)hipEventRecord(t.stop, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending.push_back(t);
  }
};

void prof_drain() {
  for (PendingTiming& t : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(t.stop) == hipSuccess && hipEventElapsedTime(&ms, t.start, t.stop) == hipSuccess) {
      auto& a = g_prof_acc[t.name];
      a.first += ms;
      a.second += 1;
    }
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_prof_pending.clear();
}

// A second stream per device (default priority, non-blocking) and its
// events, made on first use and kept for the life of the process: the
// key-block pre-work runs on it beside k_sdp and k_dq beside the key-block
// kernels, so that each fills the other's tail.
// k_row16 walks start where its XCD's workgroups last were (non-deterministic calls)
constexpr bool kRowRotate = true;
enum SideEvent { kEvSdp = 0, kEvDq = 1, kEvDecode = 2, kEvPre = 3, kNumSideEvents = 4 };
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[kNumSideEvents] = {};
};
std::mutex g_side_mu;
std::map<int, SideStream> g_side;

// The library's second stream of the current device (made on first use).
const SideStream* side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_side_mu);
  auto it = g_side.find(dev);
  if (it != g_side.end()) return &it->second;
  SideStream ss;
  if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
  for (hipEvent_t& e : ss.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
  return &(g_side[dev] = ss);
}

}  // namespace

extern "C" void sfag_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
}

extern "C" void sfag_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_drain();
  g_prof_acc.clear();
}

extern "C" int sfag_profile_read(const char* name, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_drain();
  auto it = g_prof_acc.find(name ? name : "");
  if (total_ms) *total_ms = it == g_prof_acc.end() ? 0.0 : it->second.first;
  if (launches) *launches = it == g_prof_acc.end() ? 0 : it->second.second;
  return SFAG_OK;
}

namespace {

// Validating plans: the 16-byte result word at the start of the workspace,
// cleared on the call's stream (a fill kernel, so that the call can be
// captured in a graph).  NULL otherwise.
uint32_t* start_validation(const sfag_plan* plan, void* workspace, hipStream_t s) {
  if (!plan->opt.validate) return nullptr;
  uint32_t* st = at<uint32_t>(workspace, plan->ws.status);
  launch_fill_u32(st, 4, 0u, s);
  return st;
}

}  // namespace

extern "C" int sfag_validation_read(const void* workspace, void* stream, sfag_validation* result) {
  set_error("");
  if (!workspace || !result) return fail(SFAG_ERR_NULLPTR, "workspace or result is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  sfag_validation v{};
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(SFAG_ERR_RUNTIME, "copy of the validation result failed");
  *result = v;
  return SFAG_OK;
}

extern "C" int sfag_forward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream) {
  set_error("");
  std::unique_ptr<sfag_plan> own(plan);
  if (!plan) return fail(SFAG_ERR_NULLPTR, "plan is NULL");
  if (!plan->forward) return fail(SFAG_ERR_PARAM_INVALID, "plan was made for the backward pass");
  const Dims& d = plan->d;
  const WorkspaceLayout& w = plan->ws;
  if (workspaceSize < w.total) return fail(SFAG_ERR_PARAM_INVALID, "workspace smaller than the phase-1 size");
  if (w.total > 0 && !workspace) return fail(SFAG_ERR_NULLPTR, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint32_t* status = start_validation(plan, workspace, s);
  int32_t* q_off = nullptr;
  int32_t* kv_off = nullptr;
  if (d.layout == 1 && (d.T1 > 0 || status)) {
    q_off = at<int32_t>(workspace, w.seq_off);
    kv_off = q_off + (d.B + 1);
    launch_seq_offsets((const int32_t*)plan->lq, (const int32_t*)plan->lk, (int32_t)d.B, d.T1, d.T2, q_off, kv_off,
                       status, s);
  }
  if (d.T1 == 0) return check_launch("validation");
  FwdArgs fa;
  fa.q = (const uint16_t*)plan->q;
  fa.qr = (const uint16_t*)plan->qr;
  fa.k = (const uint16_t*)plan->k;
  fa.kr = (const uint16_t*)plan->kr;
  fa.v = (const uint16_t*)plan->v;
  int32_t* rows = at<int32_t>(workspace, w.rows);
  int32_t* nvalid = at<int32_t>(workspace, w.nvalid);
  fa.rows = rows;
  fa.nvalid = nvalid;
  fa.out = (uint16_t*)plan->out_w;
  fa.smax = (float*)plan->smax_w;
  fa.ssum = (float*)plan->ssum_w;
  fa.G = d.G;
  fa.Gp = d.Gp;
  fa.E = d.E;
  fa.n_hb = (int32_t)((d.Gp + 63) / 64);
  fa.scale = plan->scale;
  // causal rows grow with the token: longest tokens first (128 heads, 4096
  // tokens, top-2048 causal: 3.38 -> 3.32 ms)
  fa.reverse = d.mode == 3 ? 1 : 0;
  for (int64_t t0 = 0; t0 < d.T1; t0 += d.chunk) {
    const int64_t ntok = std::min<int64_t>(d.chunk, d.T1 - t0);
    {
      TimedScope ts("decode", s);
      launch_decode((const int32_t*)plan->idx, t0, ntok, d, q_off, kv_off, rows, nvalid, s, status, true);
    }
    fa.t0 = t0;
    fa.ntok = ntok;
    TimedScope ts("fwd", s);
    launch_fwd(plan->dtype, d.Dr > 0, fa, s);
  }
  return check_launch("forward kernels");
}

namespace {

// The backward pass on `workspace`.  library_stream: whether the call may use
// (and on first use make) the library's second stream.
int run_backward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream, bool library_stream);

constexpr uint64_t kScratchBytes = SFAG_STATIC_SCRATCH_BYTES;

}  // namespace

// Scratch array of sfag_backward_static, one per device.  In host code the
// name `scratch` stands for a host-side handle, not a device address: host
// code reaches the array only through the address hipGetSymbolAddress gives
// for the current device (scratch_address).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;

// Device address of the current device's scratch array, looked up once per
// device (with that device current); NULL if the lookup fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) return it->second;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch[dev] = p;
  return p;
}

}  // namespace

extern "C" int sfag_backward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream) {
  return run_backward(workspace, workspaceSize, plan, stream, true);
}

extern "C" int sfag_backward_static(sfag_plan* plan, void* stream) {
  set_error("");
  if (!plan) return fail(SFAG_ERR_NULLPTR, "plan is NULL");
  if (plan->ws.total > kScratchBytes) {
    const uint64_t need = plan->ws.total;
    delete plan;
    return fail(SFAG_ERR_PARAM_INVALID, "the plan needs a workspace of " + std::to_string(need) +
                                            " bytes, more than the " + std::to_string(kScratchBytes) +
                                            "-byte scratch array: re-plan with sfag_plan_configure and "
                                            "workspaceBudget <= SFAG_STATIC_SCRATCH_BYTES");
  }
  void* ws = scratch_address();
  if (!ws) {
    delete plan;
    return fail(SFAG_ERR_RUNTIME, "the scratch array's device address could not be found");
  }
  return run_backward(ws, kScratchBytes, plan, stream, false);
}

namespace {

int run_backward(void* workspace, uint64_t workspaceSize, sfag_plan* plan, void* stream, bool library_stream) {
  set_error("");
  std::unique_ptr<sfag_plan> own(plan);
  if (!plan) return fail(SFAG_ERR_NULLPTR, "plan is NULL");
  if (plan->forward) return fail(SFAG_ERR_PARAM_INVALID, "plan was made for the forward pass");
  const Dims& d = plan->d;
  const WorkspaceLayout& w = plan->ws;
  if (workspaceSize < w.total) return fail(SFAG_ERR_PARAM_INVALID, "workspace smaller than the phase-1 size");
  if (w.total > 0 && !workspace) return fail(SFAG_ERR_NULLPTR, "workspace is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool rope = d.Dr > 0;

  uint32_t* status = start_validation(plan, workspace, s);
  int32_t* q_off = nullptr;
  int32_t* kv_off = nullptr;
  if (d.layout == 1 && (d.T1 > 0 || status)) {
    q_off = at<int32_t>(workspace, w.seq_off);
    kv_off = q_off + (d.B + 1);
    TimedScope ts("seq_offsets", s);
    launch_seq_offsets((const int32_t*)plan->lq, (const int32_t*)plan->lk, (int32_t)d.B, d.T1, d.T2, q_off, kv_off,
                       status, s);
  }
  if (d.T1 == 0) {  // empty query (约束说明: return directly); dK/dV are still defined as 0
    launch_fill_u32(plan->dk, (uint64_t)d.T2 * d.D / 2, 0u, s);
    launch_fill_u32(plan->dv, (uint64_t)d.T2 * d.D / 2, 0u, s);
    if (rope) launch_fill_u32(plan->dkr, (uint64_t)d.T2 * d.Dr / 2, 0u, s);
    return check_launch("zero fill");
  }
  float* delta = at<float>(workspace, w.delta);
  float* acc = at<float>(workspace, w.acc);
  int32_t* nvalid = at<int32_t>(workspace, w.nvalid);
  int32_t* rows = at<int32_t>(workspace, w.rows);
  uint16_t* ds = at<uint16_t>(workspace, w.ds);
  uint16_t* pb = at<uint16_t>(workspace, w.p);
  // Token side: k_row (fused, 64 heads per workgroup) or k_sdp + k_dq (up to
  // 128 heads per workgroup; N1 >= 32).
  const sfag_options& o = plan->opt;
  bool use_row = d.Gp < 32;
  if (o.tokenPath == SFAG_TOKEN_FUSED) use_row = true;
  if (o.tokenPath == SFAG_TOKEN_SPLIT && d.Gp >= 32) use_row = false;
  if (use_row && d.Gp > 16) {   // k_row reads Delta; k_row16 and k_sdp form it from dO and O themselves
    TimedScope ts("delta", s);
    launch_delta(plan->dtype, plan->dout, plan->out, delta, d.T1 * d.G, s);
  }
  // On the key-block path with positions the range reduction of every chunk
  // covers every key row: the first chunk's writes the accumulators (no
  // zero fill) and the last chunk's writes dKey|dKeyRope|dValue (no cast).
  const bool reduce_out = plan->scatter == kScatterKeyBlock && d.E > 0;
  if (!reduce_out) {
    TimedScope ts("fill", s);
    launch_fill_u32(acc, (uint64_t)d.T2 * d.AW, 0u, s);
  }

  // fp16 keeps dS above its subnormal range by a power-of-two factor that the
  // dQ and dK epilogues divide out again.
  const float ds_scale = plan->dtype == SFAG_FP16 ? 256.f : 1.f;
  const bool partial = plan->scatter == kScatterPartials;
  const bool keyblock = plan->scatter == kScatterKeyBlock;

  RowArgs ra;
  ra.q = (const uint16_t*)plan->q;
  ra.qr = (const uint16_t*)plan->qr;
  ra.dO = (const uint16_t*)plan->dout;
  ra.o = (const uint16_t*)plan->out;
  ra.k = (const uint16_t*)plan->k;
  ra.kr = (const uint16_t*)plan->kr;
  ra.v = (const uint16_t*)plan->v;
  ra.smax = (const float*)plan->smax;
  ra.ssum = (const float*)plan->ssum;
  ra.delta = delta;
  ra.rows = rows;
  ra.nvalid = nvalid;
  ra.ds_out = ds;
  ra.p_out = pb;
  ra.dq = (uint16_t*)plan->dq;
  ra.dqr = (uint16_t*)plan->dqr;
  ra.G = d.G;
  ra.Gp = d.Gp;
  ra.E = d.E;
  ra.n_hb = (int32_t)((d.Gp + 63) / 64);
  ra.scale_log2 = plan->scale * kLog2e;
  ra.ds_scale = ds_scale;
  ra.dq_mul = plan->scale / ds_scale;
  ra.n_split = 1;
  ra.dq_acc = nullptr;
  // Without the deterministic guarantee the N1 <= 16 token kernel starts each
  // token's walk where the workgroups of its XCD last were (the walk order
  // only changes the order of dQ's sums).
  ra.phase = !plan->deterministic && kRowRotate ? at<int32_t>(workspace, w.phase) : nullptr;
  // causal rows grow with the token: longest tokens first
  ra.reverse = d.mode == 3 ? 1 : 0;
  if (o.tokenOrder == SFAG_ORDER_ASCENDING) ra.reverse = 0;
  if (o.tokenOrder == SFAG_ORDER_DESCENDING) ra.reverse = 1;

  ColArgs ca;
  ca.q = ra.q;
  ca.qr = ra.qr;
  ca.dO = ra.dO;
  ca.ds = ds;
  ca.p = pb;
  ca.rows = rows;
  ca.nvalid = nvalid;
  ca.acc = acc;
  ca.partials = partial ? at<float>(workspace, w.partials) : nullptr;
  ca.G = d.G;
  ca.Gp = d.Gp;
  ca.E = d.E;
  ca.AW = d.AW;

  int32_t* keys[2] = {nullptr, nullptr};
  int32_t* vals[2] = {nullptr, nullptr};
  if (partial || keyblock) {
    keys[0] = at<int32_t>(workspace, w.sort_keys[0]);
    keys[1] = at<int32_t>(workspace, w.sort_keys[1]);
    vals[0] = at<int32_t>(workspace, w.sort_vals[0]);
    vals[1] = at<int32_t>(workspace, w.sort_vals[1]);
  }

  // A second stream on the key-block path with the split token kernels:
  // k_dq runs beside the key-block kernels (64 heads, 8192 varlen tokens,
  // top-2048 causal: 9.4 -> 8.4 ms).  With 128 heads it pays only where the
  // key-block launch is short enough that its last round of workgroups
  // leaves CUs idle for k_dq to fill (4096 tokens, top-2048 causal: 6.66 ->
  // 6.55 ms), and costs on long ones (32768 tokens, top-8192: 286 -> 293 ms,
  // in 3 chunks or in one), so by default it is on there for chunks of at
  // most 4096 tokens.  Where the second stream is used, the key-block
  // pre-work (grouping the pairs by key block) runs on it beside k_sdp, off
  // the path from k_sdp to the key-block kernel (128 heads, 4096 tokens:
  // 6.52 -> 6.48 ms; beside k_dq it took 0.33 ms of that path).  The
  // caller's auxiliary stream if it gave one (with events of the call's
  // own), else the library's, whose events this call holds for its whole
  // enqueue sequence.
  const bool kb_work = keyblock && d.E > 0;
  const bool side_pays = d.Gp < 128 || d.chunk <= 4096;
  bool concurrent = kb_work && !use_row &&
                    (o.concurrent == SFAG_CONCURRENT_ON || (o.concurrent == SFAG_CONCURRENT_AUTO && side_pays));
  bool dq_side = concurrent;
  SideStream own_side;
  struct OwnEvents {
    hipEvent_t e[kNumSideEvents] = {};
    ~OwnEvents() {
      for (hipEvent_t x : e)
        if (x) (void)hipEventDestroy(x);
    }
  } own_events;
  const SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  if (concurrent && o.auxStream) {
    own_side.s = static_cast<hipStream_t>(o.auxStream);
    for (int i = 0; i < kNumSideEvents; ++i) {
      if (hipEventCreateWithFlags(&own_events.e[i], hipEventDisableTiming) != hipSuccess)
        return fail(SFAG_ERR_RUNTIME, "events for the auxiliary stream could not be made");
      own_side.ev[i] = own_events.e[i];
    }
    side = &own_side;
  } else if (concurrent && library_stream) {
    side = side_stream();
    if (side) side_lock.lock();
  }
  if (!side) dq_side = false;
  // With 128 heads and k_dq beside the key-block kernels the token kernels
  // visit causal chunks first token first: k_dq's long last tokens then run
  // beside the key-block launch instead of after it (4096 tokens, top-2048
  // causal: 6.37 -> 6.28 ms).  With 64 heads (8192 TND tokens: 6.98 -> 7.08
  // ms) and alone (32768 tokens: unchanged) the longest tokens stay first.
  if (o.tokenOrder == SFAG_ORDER_AUTO && d.mode == 3 && d.Gp == 128 && dq_side) ra.reverse = 0;
  // stream b waits for the work enqueued so far on stream a
  auto order = [&](hipStream_t a, hipStream_t b, SideEvent e) {
    return hipEventRecord(side->ev[e], a) == hipSuccess && hipStreamWaitEvent(b, side->ev[e], 0) == hipSuccess;
  };
  int32_t* skeys = nullptr;
  int32_t* svals = nullptr;
  // sort by key block and visits of one chunk on stream `st`
  auto pre_work = [&](int64_t ntok, hipStream_t st) {
    const int64_t n = ntok * d.E;
    TimedScope ts("kb_sort", st);
    if (kb_use_bins(d)) {
      int32_t* grid = at<int32_t>(workspace, w.kb_grid);
      svals = at<int32_t>(workspace, w.sort_vals[0]);
      launch_kb_bins(rows, nvalid, d.E, (int32_t)d.nKB, ntok, grid, grid + d.nKB * ntok,
                     at<int32_t>(workspace, w.kb_grid_tmp), svals, at<int32_t>(workspace, w.vis_er),
                     at<int32_t>(workspace, w.vis_start), at<int32_t>(workspace, w.vis_key),
                     at<int32_t>(workspace, w.vis_n), st);
      return;
    }
    launch_csr(n, rows, nvalid, d.E, d.T2, d.kb_sort_bits, keys, vals, at<int32_t>(workspace, w.sort_hist),
               nullptr, &svals, st, 1, ntok, &skeys);
    launch_visits(skeys, svals, rows, n, ntok, (int32_t)d.nKB, at<int32_t>(workspace, w.vis_flags),
                  at<int32_t>(workspace, w.sort_hist), at<int32_t>(workspace, w.vis_start),
                  at<int32_t>(workspace, w.vis_key), at<int32_t>(workspace, w.vis_er),
                  at<int32_t>(workspace, w.vis_n), st);
  };
  for (int64_t t0 = 0; t0 < d.T1; t0 += d.chunk) {
    const int64_t ntok = std::min<int64_t>(d.chunk, d.T1 - t0);
    {
      TimedScope ts("decode", s);
      launch_decode((const int32_t*)plan->idx, t0, ntok, d, q_off, kv_off, rows, nvalid, s, status, true);
    }
    ra.t0 = ca.t0 = t0;
    ra.ntok = ca.ntok = ntok;
    const bool pre_side = dq_side && kb_work;   // pre-work beside k_sdp
    if (pre_side) {
      if (!order(s, side->s, kEvDecode)) return fail(SFAG_ERR_RUNTIME, "fork to the second stream failed");
      pre_work(ntok, side->s);
      if (hipEventRecord(side->ev[kEvPre], side->s) != hipSuccess)
        return fail(SFAG_ERR_RUNTIME, "second stream event failed");
    }
    if (!use_row) {
      {
        TimedScope ts("sdp", s);
        launch_sdp(plan->dtype, rope, ra, s);
      }
      if (dq_side) {
        if (!order(s, side->s, kEvSdp)) return fail(SFAG_ERR_RUNTIME, "fork to the second stream failed");
        {
          TimedScope ts("dq", side->s);
          launch_dq(plan->dtype, rope, ra, side->s, true);
        }
        if (hipEventRecord(side->ev[kEvDq], side->s) != hipSuccess)
          return fail(SFAG_ERR_RUNTIME, "second stream event failed");
      } else {
        TimedScope ts("dq", s);
        launch_dq(plan->dtype, rope, ra, s, false);
      }
    } else if (d.row_split > 1) {
      // a token's positions over row_split workgroups: fp32 dQ sums, then a cast
      ra.n_split = d.row_split;
      ra.dq_acc = at<float>(workspace, w.dq_acc);
      TimedScope ts("row", s);
      launch_fill_u32(ra.dq_acc, (uint64_t)ntok * d.G * (d.D + d.Dr), 0u, s);
      launch_row(plan->dtype, rope, ra, s);
      launch_dq_cast(plan->dtype, ra.dq_acc, t0, ntok, d.G, (int32_t)d.Dr, ra.dq_mul, plan->dq, plan->dqr, s);
    } else {
      TimedScope ts("row", s);
      launch_row(plan->dtype, rope, ra, s);
    }
    if (kb_work) {
      if (!pre_side) pre_work(ntok, s);
      else if (hipStreamWaitEvent(s, side->ev[kEvPre], 0) != hipSuccess)
        return fail(SFAG_ERR_RUNTIME, "join of the second stream failed");
      {
        KbArgs ka;
        ka.q = ra.q;
        ka.qr = ra.qr;
        ka.dO = ra.dO;
        ka.ds = ds;
        ka.p = pb;
        ka.svals = svals;
        ka.er = at<int32_t>(workspace, w.vis_er);
        ka.vis_start = at<int32_t>(workspace, w.vis_start);
        ka.vis_key = at<int32_t>(workspace, w.vis_key);
        ka.n_vis = at<int32_t>(workspace, w.vis_n);
        ka.nonempty = at<int32_t>(workspace, w.kb_nonempty);
        ka.part = at<float>(workspace, w.kb_part);
        ka.t0 = t0;
        ka.ntok = ntok;
        ka.E = d.E;
        ka.G = d.G;
        ka.Gp = d.Gp;
        ka.T2 = d.T2;
        ka.AW = d.AW;
        ka.TR = d.TR;
        ka.Dr = (int32_t)d.Dr;
        ka.nKB = (int32_t)d.nKB;
        ka.nTR = (int32_t)((ntok + d.TR - 1) / d.TR);
        // column blocks: dK|dKrope (three of 192 with rope, two of 256
        // without), dV (two of 256)
        int m = 0;
        const int32_t dq = (int32_t)(d.D + d.Dr);
        const int32_t wk = rope ? 192 : 256;
        for (int32_t c0 = 0; c0 < dq; c0 += wk) ka.cbs[m++] = ColBlock{0, c0, c0, wk};
        ka.cbs[m++] = ColBlock{1, 0, dq, 256};
        ka.cbs[m++] = ColBlock{1, 256, dq + 256, 256};
        ka.nCB = m;
        {
          TimedScope ts("keyblock", s);
          launch_keyblock(plan->dtype, ka, s);
        }
        {
          TimedScope ts("kb_reduce", s);
          KbOut ko{plan->dtype, (int32_t)d.D, (int32_t)d.Dr, plan->scale / ds_scale, plan->dk, plan->dkr, plan->dv};
          launch_kb_reduce(ka.part, ka.nonempty, d.T2, d.AW, ka.nTR, ka.nKB, acc, t0 == 0,
                           t0 + ntok >= d.T1 ? &ko : nullptr, s);
        }
      }
    } else if (!keyblock) {
      TimedScope ts("col", s);
      launch_col(plan->dtype, rope, partial, ca, s);
    }
    if (partial && d.E > 0) {
      int32_t* sorted = nullptr;
      int32_t* off = at<int32_t>(workspace, w.csr_off);
      {
        TimedScope ts("csr", s);
        launch_csr(ntok * d.E, rows, nvalid, d.E, d.T2, d.sort_bits, keys, vals,
                   at<int32_t>(workspace, w.sort_hist), off, &sorted, s);
      }
      TimedScope ts("key_reduce", s);
      launch_key_reduce(off, sorted, ca.partials, d.AW, d.T2, acc, s);
    }
    if (dq_side && hipStreamWaitEvent(s, side->ev[kEvDq], 0) != hipSuccess)
      return fail(SFAG_ERR_RUNTIME, "join of the second stream failed");
    const int rc = check_launch("chunk kernels");
    if (rc != SFAG_OK) return rc;
  }
  if (!reduce_out) {
    TimedScope ts("cast", s);
    launch_cast(plan->dtype, acc, d.T2, (int32_t)d.D, (int32_t)d.Dr, plan->scale / ds_scale, plan->dk, plan->dkr,
                plan->dv, s);
  }
  return check_launch("cast");
}

}  // namespace

namespace {

struct IndexLayout {
  uint64_t seq_off, keys0, keys1, vals0, vals1, hist, total;
};

IndexLayout index_layout(int64_t T1, int64_t E) {
  IndexLayout L;
  const uint64_t n = (uint64_t)T1 * E;
  const uint64_t nblk = (n + kSortBlock - 1) / kSortBlock;
  uint64_t c = 0;
  auto carve = [&](uint64_t& f, uint64_t bytes) {
    f = c;
    c = align256(c + bytes);
  };
  carve(L.seq_off, 2 * 257 * 4);
  carve(L.keys0, n * 4);
  carve(L.keys1, n * 4);
  carve(L.vals0, n * 4);
  carve(L.vals1, n * 4);
  carve(L.hist, (256 * nblk + 256 * nblk / 4096 + 2) * 4);
  L.total = c;
  return L;
}

}  // namespace

extern "C" int64_t sfag_band_entries(int64_t maxKeyLen, int64_t preTokens, int64_t nextTokens, int64_t block) {
  if (maxKeyLen <= 0 || preTokens < 0 || nextTokens < 0 || block < 1) return 0;
  const int64_t width = std::min<int64_t>(maxKeyLen, std::min<int64_t>(preTokens, maxKeyLen) +
                                                         std::min<int64_t>(nextTokens, maxKeyLen) + 1);
  return std::min<int64_t>((maxKeyLen + block - 1) / block, (width - 1 + block - 1) / block + 1);
}

extern "C" int sfag_band_indices(void* sparseIndices, const void* seqLensQ, const void* seqLensKv, int64_t B,
                                 int64_t S1, int64_t S2, int64_t T1, int64_t K, int64_t block, int32_t layout,
                                 int64_t preTokens, int64_t nextTokens, void* stream) {
  set_error("");
  if (layout != 0 && layout != 1) return fail(SFAG_ERR_TILING, "layout must be 0 (BSND) or 1 (TND)");
  if (block < 1 || block > (1 << 20) || K < 0 || T1 < 0 || B < 0)
    return fail(SFAG_ERR_TILING, "bad sizes (block >= 1, K, T1, B >= 0)");
  if (preTokens < 0 || nextTokens < 0) return fail(SFAG_ERR_TILING, "preTokens and nextTokens must be >= 0");
  if (layout == 0 && (S1 < 0 || S2 < 0 || S2 > 0x7fffffffLL || B * S1 != T1))
    return fail(SFAG_ERR_TILING, "BSND needs T1 = B*S1 and 0 <= S2 < 2^31");
  if (layout == 1 && (B < 1 || B > 256)) return fail(SFAG_ERR_TILING, "TND needs 1 <= B <= 256");
  if (T1 > 0 && K > 0 && !sparseIndices) return fail(SFAG_ERR_NULLPTR, "sparseIndices is NULL");
  if (layout == 1 && (!seqLensQ || !seqLensKv)) return fail(SFAG_ERR_NULLPTR, "TND needs both length arrays");
  if (T1 > 0x7fffffffLL) return fail(SFAG_ERR_TILING, "T1 must be below 2^31");
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  launch_band_indices((int32_t*)sparseIndices, T1, K, (int32_t)block, layout, S1, S2, (const int32_t*)seqLensQ,
                      (const int32_t*)seqLensKv, (int32_t)B, preTokens, nextTokens, s);
  return check_launch("band indices");
}

extern "C" uint64_t sfag_index_workspace_size(int64_t T1, int64_t T2, int64_t K, int64_t block) {
  (void)T2;
  if (T1 < 0 || K < 0 || block < 1) return 0;
  return index_layout(T1, K * block).total;
}

extern "C" int sfag_build_index(const void* sparseIndices, const void* seqLensQ, const void* seqLensKv, int64_t B,
                                int64_t S1, int64_t S2, int64_t T1, int64_t T2, int64_t K, int64_t block,
                                int32_t layout, int64_t sparseMode, void* workspace, uint64_t workspaceSize,
                                void* nValid, void* rows, void* csrOffsets, void* csrPairs, void* stream) {
  set_error("");
  if (layout != 0 && layout != 1) return fail(SFAG_ERR_TILING, "layout must be 0 (BSND) or 1 (TND)");
  if (sparseMode != 0 && sparseMode != 3) return fail(SFAG_ERR_TILING, "sparseMode must be 0 or 3");
  if (block < 1 || K < 0 || T1 < 0 || T2 < 0 || B < 0 || B > 256) return fail(SFAG_ERR_TILING, "bad sizes");
  if (layout == 0 && (B * S1 != T1 || B * S2 != T2)) return fail(SFAG_ERR_TILING, "BSND needs T1 = B*S1, T2 = B*S2");
  const int64_t E = K * block;
  if ((double)T1 * (double)E >= 2147483648.0) return fail(SFAG_ERR_TILING, "T1*K*block must be below 2^31");
  const IndexLayout L = index_layout(T1, E);
  if (workspaceSize < L.total) return fail(SFAG_ERR_PARAM_INVALID, "workspace too small");
  if (!workspace || !csrOffsets || (T1 > 0 && (!sparseIndices || !nValid || !rows || !csrPairs)) ||
      (layout == 1 && (!seqLensQ || !seqLensKv)))
    return fail(SFAG_ERR_NULLPTR, "NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  Dims d;
  d.layout = layout;
  d.B = B;
  d.S1 = S1;
  d.S2 = S2;
  d.T1 = T1;
  d.T2 = T2;
  d.K = K;
  d.block = block;
  d.E = E;
  d.mode = (int32_t)sparseMode;
  int bits = 1;
  while (((int64_t)1 << bits) <= T2) ++bits;
  int32_t* q_off = nullptr;
  int32_t* kv_off = nullptr;
  if (layout == 1) {
    q_off = at<int32_t>(workspace, L.seq_off);
    kv_off = q_off + (B + 1);
    launch_seq_offsets((const int32_t*)seqLensQ, (const int32_t*)seqLensKv, (int32_t)B, T1, T2, q_off, kv_off,
                       nullptr, s);
  }
  launch_decode((const int32_t*)sparseIndices, 0, T1, d, q_off, kv_off, (int32_t*)rows, (int32_t*)nValid, s);
  const int64_t n = T1 * E;
  if (n == 0) {
    launch_fill_u32(csrOffsets, (uint64_t)T2 + 1, 0u, s);
    return check_launch("index");
  }
  int32_t* keys[2] = {at<int32_t>(workspace, L.keys0), at<int32_t>(workspace, L.keys1)};
  int32_t* vals[2] = {at<int32_t>(workspace, L.vals0), at<int32_t>(workspace, L.vals1)};
  int32_t* sorted = nullptr;
  launch_csr(n, (const int32_t*)rows, (const int32_t*)nValid, E, T2, bits, keys, vals, at<int32_t>(workspace, L.hist),
             (int32_t*)csrOffsets, &sorted, s);
  if (hipMemcpyAsync(csrPairs, sorted, (size_t)n * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return fail(SFAG_ERR_RUNTIME, "copy of the CSR pairs failed");
  return check_launch("index");
}
