// C ABI of the layer engine: argument checks, workspace layout, launches.
// Every check happens on the host before anything is queued on the stream.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/rnn.h"
#include "rnn_internal.hpp"

#define RNN_API extern "C" __attribute__((visibility("default")))

namespace {

using rnn::bf16;

constexpr size_t ALIGN = 256;
constexpr int MAX_CHUNKS = 64;     // bias-gradient partial sums
constexpr double TIMEOUT_S = 10.0;

size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

int gates(const rnn_desc_t* d) { return d->mode == RNN_LSTM ? 4 : 3; }
int cell_of(const rnn_desc_t* d) {
  if (d->mode == RNN_LSTM) return rnn::CELL_LSTM;
  return d->reset_after ? rnn::CELL_GRU_RA : rnn::CELL_GRU_BASIC;
}
long long ldx_of(const rnn_desc_t* d) { return d->ldx ? d->ldx : d->I; }
long long ldy_of(const rnn_desc_t* d) { return d->ldy ? d->ldy : (d->direction == 2 ? 2LL : 1LL) * d->H; }
size_t esz(const rnn_desc_t* d) { return d->dtype == RNN_BF16 ? 2 : 4; }

struct Layout {
  size_t status, flags, partial, gemm, z, c, rh, dg, xb, xb_bytes, gath, attp, wt, wht, dgt, xt, ht, rht, dwp, dwp_bytes,
      total;
  size_t gemm_floats;
  int GZ, GD;
};

// CU count the workspace is sized for (MI355X); a device with more CUs
// simply splits less when the scratch would not fit
constexpr int PLAN_CUS = 256;

bool desc_ok(const rnn_desc_t* d) {
  if (!d) return false;
  if (d->mode != RNN_LSTM && d->mode != RNN_GRU) return false;
  if (d->dtype != RNN_F32 && d->dtype != RNN_BF16) return false;
  if (d->direction < 0 || d->direction > 2) return false;
  if (d->mode == RNN_GRU && d->reset_after != 0 && d->reset_after != 1) return false;
  if (d->att && d->mode != RNN_GRU) return false;  // attention scores scale the GRU update gate
  if (d->recompute != 0 && !(d->recompute == 1 && d->mode == RNN_LSTM)) return false;
  if (d->dw_hh_mode != 0 && d->dw_hh_mode != 1) return false;
  if (d->stepwise != 0 && d->stepwise != 1) return false;
  if (d->T < 1 || d->B < 1 || d->I < 1 || d->H < 1) return false;
  const int G = gates(d);
  int seen = 0;
  for (int k = 0; k < G; ++k) {
    const int g = d->gate_order[k];
    if (g < 0 || g >= G || (seen & (1 << g))) return false;
    seen |= 1 << g;
  }
  if (d->ldx != 0 && d->ldx < d->I) return false;
  if (d->ldy != 0 && d->ldy < (d->direction == 2 ? 2LL : 1LL) * d->H) return false;
  return true;
}

// granularity the kernels need (16-byte chunks along I and H)
bool shape_supported(const rnn_desc_t* d) {
  if (d->I % 8 || d->H % 16) return false;
  if (ldx_of(d) % 8 || ldy_of(d) % 8) return false;
  if ((long long)d->T * d->B > (1LL << 31) / 2) return false;
  if (4LL * d->H > (1LL << 30)) return false;  // gate-row indices in 32 bits
  return true;
}


// Step-counter layout of a plan (see FLAG_LINE): adjacent counters for a
// batch group on one XCD, one line each otherwise; and the count of ints
// from the first counter through the last placement word of nwg workgroups.
void counter_layout(const rnn::RecPlan& plan, int* stride, int* place_off) {
  // (the kernels of 64-row tiles assume one line per counter)
  const bool packed = plan.xcd_span <= 1 && plan.mb < 4;
  *stride = packed ? 1 : rnn::FLAG_LINE;
  *place_off = packed ? rnn::FLAG_SLOTS : 1;
}
long long counter_ints(const rnn::RecPlan& plan) {
  int stride, place;
  counter_layout(plan, &stride, &place);
  const long long nwg = (long long)plan.nGroups * plan.nSlices;
  return std::max((long long)place + nwg, nwg * stride);
}

// shapes whose backward plans can carry the fused dW_hh variant (the fp32
// plans of 4 waves with 8 or 12 k-steps each, and 8 waves with 6: there the
// accumulators fit beside the resident W_hh without spilling)
bool fused_dw_shape(const rnn_desc_t* d) {
  if (d->dtype != RNN_F32 || d->dw_hh_mode != 0 || d->stepwise) return false;
  const int cell = cell_of(d);
  return (cell == rnn::CELL_LSTM && d->H <= 128) || (cell == rnn::CELL_GRU_RA && d->H <= 256);
}

// Weight gradients as products over k-contiguous (transposed) operands, the
// input- and recurrent-side columns of a gate row in one product split at
// column I (a whole number of 256-wide tiles); T*B is then a whole number of
// 16-byte chunks. bf16: always (the direct-load kernel). fp32: for long
// sequences (T*B >= 8192), where the k-contiguous product's gain outweighs
// the transposes, and not where the BPTT kernel may accumulate dW_hh itself.
bool nt_weight_grads(const rnn_desc_t* d) {
  const long long TB = (long long)d->T * d->B;
  if (TB % 8 || d->I % 256) return false;
  return d->dtype == RNN_BF16 || (TB >= 8192 && !fused_dw_shape(d));
}
hipError_t transpose_dt(int dtype, const rnn::RowMap& src, int R, int T, int B, void* out, hipStream_t s) {
  return dtype == RNN_BF16 ? rnn::launch_gather_transpose<bf16>(src, R, T, B, out, s)
                           : rnn::launch_gather_transpose<float>(src, R, T, B, out, s);
}

Layout layout(const rnn_desc_t* d) {
  Layout L{};
  const size_t s = esz(d);
  const size_t TB = (size_t)d->T * d->B, H = d->H;
  const int cell = cell_of(d);
  L.GZ = (cell == rnn::CELL_GRU_RA) ? 4 : gates(d);
  L.GD = (cell == rnn::CELL_GRU_RA) ? 4 : gates(d);
  size_t off = 0;
  L.status = off;
  off += ALIGN;
  L.flags = off;
  off += up(2 * (size_t)rnn::FLAG_PASS * sizeof(int));  // forward and backward passes
  L.partial = off;
  off += up((size_t)MAX_CHUNKS * 4 * H * sizeof(float));
  {
    // GEMM scratch: the largest split-K product (the weight gradients)
    const long long GH = (long long)gates(d) * d->H;
    const long long nmax = d->I > d->H ? d->I : d->H;
    size_t f = rnn::gemm_workspace_floats(GH, nmax, (long long)TB, PLAN_CUS);
    const size_t f2 = rnn::gemm_workspace_floats((long long)TB, GH, d->I, PLAN_CUS);
    const size_t f3 = rnn::gemm_workspace_floats((long long)TB, d->I, GH, PLAN_CUS);
    // the LSTM's two weight gradients as one product with two output parts
    const size_t f4 = rnn::gemm_workspace_floats(GH, (long long)d->I + d->H, (long long)TB, PLAN_CUS);
    if (f2 > f) f = f2;
    if (f3 > f) f = f3;
    if (cell == rnn::CELL_LSTM && f4 > f) f = f4;
    if (cell != rnn::CELL_LSTM) {
      // the GRUs' k-contiguous weight gradients: the r and u rows over
      // [x | h_{t-1}], then the candidate rows (reset-after: each side on its
      // own; basic: one product over [x | r*h_{t-1}])
      const size_t f6 = rnn::gemm_workspace_floats(2LL * d->H, (long long)d->I + d->H, (long long)TB, PLAN_CUS);
      const size_t f7 = rnn::gemm_workspace_floats(d->H, nmax, (long long)TB, PLAN_CUS);
      const size_t f8 = rnn::gemm_workspace_floats(d->H, (long long)d->I + d->H, (long long)TB, PLAN_CUS);
      if (f6 > f) f = f6;
      if (f7 > f) f = f7;
      if (f8 > f) f = f8;
    }
    // the per-step recurrence keeps its carried state here between launches
    const size_t f5 = rnn::stepwise_scratch_floats(cell, d->B, d->H);
    if (f5 > f) f = f5;
    L.gemm = off;
    L.gemm_floats = f;
    off += up(f * sizeof(float));
  }
  L.z = off;
  off += up(TB * L.GZ * H * s);
  L.c = off;
  if (cell == rnn::CELL_LSTM && !d->recompute) off += up(TB * H * s);
  L.rh = off;
  if (cell == rnn::CELL_GRU_BASIC) off += up(TB * H * s);
  L.dg = off;
  off += up(TB * L.GD * H * s);
  // exchange ring of the persistent kernels: two slots of every batch
  // group's operand tiles (16 padded rows per group, groups of >= 4 rows, a
  // contraction of at most 4H)
  L.xb = off;
  L.xb_bytes = 2 * (size_t)16 * ((d->B + 3) / 4) * 4 * H * s;
  off += up(L.xb_bytes);
  // per batch row, the gate gradients of its own first step (direction 1
  // with variable lengths: the weight gradient's h0 term)
  L.gath = off;
  off += up((size_t)d->B * L.GD * H * s);
  // AUGRU: per hidden slice partial score gradients (slices hold >= 16 units)
  L.attp = off;
  if (d->att) off += up(TB * (H / 16) * sizeof(float));
  // W_ih transposed to [I][G*H] for the input gradient (a k-contiguous
  // operand, loaded straight into LDS)
  L.wt = off;
  off += up((size_t)d->I * gates(d) * H * s);
  // W_hh transposed to [H][G*H] in the BPTT kernel's contraction order
  L.wht = off;
  if (cell_of(d) != rnn::CELL_GRU_BASIC) off += up((size_t)H * gates(d) * H * s);
  // bf16 LSTM and reset-after GRU: the weight-gradient products as
  // k-contiguous ones: the gate gradients (all GD lanes), x and h_{t-1}
  // transposed to [.][T*B]
  L.dgt = L.xt = L.ht = off;
  if (nt_weight_grads(d)) {
    L.dgt = off;
    off += up(TB * L.GD * H * s);
    L.xt = off;
    off += up(TB * (size_t)d->I * s);
    L.ht = off;
    off += up(TB * H * s);
  }
  // basic GRU: r*h_{t-1} transposed as well (the candidate rows' activation)
  L.rht = off;
  if (nt_weight_grads(d) && cell == rnn::CELL_GRU_BASIC) off += up(TB * H * s);
  // fp32 reset-after GRU (H <= 256) and LSTM (H <= 128): per batch group
  // (>= 4 rows) partial recurrent-weight gradients of the fused BPTT kernel
  L.dwp = off;
  L.dwp_bytes = 0;
  if (fused_dw_shape(d)) {
    L.dwp_bytes = (size_t)((d->B + 3) / 4) * (cell == rnn::CELL_LSTM ? 4 : 3) * H * (H + 1) * sizeof(float);
    off += up(L.dwp_bytes);
  }
  L.total = off;
  return L;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15) == 0; }

// A bidirectional layer (direction 2) runs as its two single-direction
// halves, each over its own half of the workspace.
rnn_desc_t half_desc(const rnn_desc_t* d, int k) {
  rnn_desc_t h = *d;
  if (d->direction == 2) {
    h.direction = k;
    h.ldy = ldy_of(d);
  }
  return h;
}
size_t ws_total(const rnn_desc_t* d) {
  if (d->direction != 2) return layout(d).total;
  const rnn_desc_t h = half_desc(d, 0);
  return 2 * layout(&h).total;
}
// element offsets into the [2][...] stacked arrays of a bidirectional layer
const void* at(const void* p, long long elems, size_t es) { return p ? (const char*)p + elems * (long long)es : nullptr; }
void* at(void* p, long long elems, size_t es) { return p ? (char*)p + elems * (long long)es : nullptr; }

struct DevInfo {
  int cu = 0;
  long long ticks = 0;  // handshake time-out in wall-clock ticks (< 0: give up at once)
  int rate_khz = 0;
};

// handshake time-out of the persistent kernels (seconds; < 0: no time at all)
double g_timeout_s = TIMEOUT_S;

bool log_on() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("RNN_LOG");
    v = (e && *e && *e != '0') ? 1 : 0;
  }
  return v == 1;
}

int dev_info(DevInfo* out) {
  static DevInfo cache[64];
  int dev = 0;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess || dev < 0 || dev >= 64) {
    if (log_on()) fprintf(stderr, "[rnn] hipGetDevice: %s (device %d)\n", hipGetErrorString(e), dev);
    return RNN_ERR_DEVICE;
  }
  if (cache[dev].cu == 0) {
    int cu = 0, rate_khz = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return RNN_ERR_DEVICE;
    if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate_khz <= 0)
      rate_khz = 100000;
    cache[dev].rate_khz = rate_khz;
    cache[dev].cu = cu;
  }
  *out = cache[dev];
  out->ticks = g_timeout_s < 0 ? -1 : (long long)(g_timeout_s * out->rate_khz * 1000.0);
  return RNN_OK;
}


void inv_perm(const rnn_desc_t* d, int perm[4]) {
  for (int k = 0; k < 4; ++k) perm[k] = 0;
  for (int k = 0; k < gates(d); ++k) perm[d->gate_order[k]] = k;
}

int check_common(const rnn_desc_t* d, const void* ws, size_t ws_bytes) {
  if (!desc_ok(d)) return RNN_ERR_INVALID_ARG;
  if (!shape_supported(d)) return RNN_ERR_UNSUPPORTED;
  if (!ws || !aligned(ws)) return RNN_ERR_INVALID_ARG;
  if (ws_bytes < ws_total(d)) return RNN_ERR_WORKSPACE_TOO_SMALL;
  return RNN_OK;
}

int hip_status_at(hipError_t e, int line) {
  if (e == hipSuccess) return RNN_OK;
  if (log_on()) fprintf(stderr, "[rnn] HIP error %d (%s) at rnn_api.cpp:%d\n", (int)e, hipGetErrorString(e), line);
  return RNN_ERR_DEVICE;
}
#define hip_status(e) hip_status_at((e), __LINE__)

// ---- optional kernel timing (rnn_profile_*) ----
enum Label { L_FILL, L_PROJ, L_RFWD, L_RBWD, L_DX, L_DW, L_DB, L_AUX, L_COUNT };
const char* kLabel[L_COUNT] = {"fill", "proj_gemm", "rec_fwd", "rec_bwd", "dx_gemm", "dw_gemm", "db_colsum", "aux"};
struct Pending {
  int label;
  hipEvent_t a, b;
};
struct Prof {
  bool on = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total[L_COUNT] = {};
  long long count[L_COUNT] = {};
};
Prof& prof() {
  static Prof p;
  return p;
}
hipEvent_t take_event() {
  Prof& p = prof();
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
// Destroys the pooled events (none may be pending): done whenever profiling
// is off and every recorded pair has been read, so that no HIP event of the
// library outlives its use (a process then tears down with none alive).
void release_pool(Prof& p) {
  for (hipEvent_t e : p.pool) (void)hipEventDestroy(e);
  p.pool.clear();
}
// Brackets the kernels queued during its lifetime with two events.
struct ProfScope {
  int label;
  hipStream_t s;
  hipEvent_t a = nullptr;
  ProfScope(int l, hipStream_t st) : label(l), s(st) {
    if (prof().on && (a = take_event())) (void)hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!a) return;
    hipEvent_t b = take_event();
    if (!b) return;
    (void)hipEventRecord(b, s);
    prof().pending.push_back({label, a, b});
  }
};

rnn::RowMap rows(const void* p, long long ld) {
  rnn::RowMap m{};
  m.ptr = p;
  m.ld = ld;
  m.kind = 0;
  return m;
}
rnn::RowMap perm_rows(const void* p, long long ld, int H, const int perm[4]) {
  rnn::RowMap m = rows(p, ld);
  m.kind = 1;
  m.H = H;
  for (int i = 0; i < 4; ++i) m.perm[i] = perm[i];
  return m;
}

int g_cu_count = PLAN_CUS;  // refreshed from the device before every call that launches

hipError_t gemm_dt(int dtype, const rnn::GemmArgs& g, bool ak, bool bk, hipStream_t s) {
  return dtype == RNN_BF16 ? rnn::launch_gemm<bf16>(g, ak, bk, g_cu_count, s)
                           : rnn::launch_gemm<float>(g, ak, bk, g_cu_count, s);
}
hipError_t colsum_dt(int dtype, const void* src, long long lds, long long M, int col0, int ncols, void* out,
                     int out_row0, int H, const int perm[4], int acc, float* partial, hipStream_t s) {
  ProfScope ps(L_DB, s);
  if (dtype == RNN_BF16)
    return rnn::launch_colsum<bf16>(src, lds, M, col0, ncols, out, out_row0, H, perm, acc, partial, MAX_CHUNKS, s);
  return rnn::launch_colsum<float>(src, lds, M, col0, ncols, out, out_row0, H, perm, acc, partial, MAX_CHUNKS, s);
}

// Exchange ring for single row-tile plans; K = contraction length of the
// exchanged vector. Pairs of k-steps share a tile when groups have <= 8 rows.
// Returns 0 (no ring: the kernels read rows of y / dG), 1 (tiled) or 2 (packed).
int ring_kind(const rnn::RecPlan& p, const Layout& L, long long K, size_t esize) {
  if (p.nw == 0 || p.bg > 16 * p.mb) return 0;  // (nw 0: the per-step path)
  if ((K * (long long)esize) % 64 != 0) return 0;  // whole k-steps only
  const long long gbytes = K * 16 * (long long)p.mb * (long long)esize;  // a 1 KiB tile per (k-step, row tile)
  if ((size_t)(2 * p.nGroups * gbytes) > L.xb_bytes) return 0;
  const long long ksteps = K * (long long)esize / 64;
  return (p.mb == 1 && p.bg <= 8 && ksteps % 2 == 0 && p.ki % 2 == 0) ? 2 : 1;
}
void set_xbuf(rnn::RecArgs& a, const rnn::RecPlan& p, const Layout& L, char* ws, long long K, size_t esize) {
  const int kind = ring_kind(p, L, K, esize);
  a.xbuf = kind ? ws + L.xb : nullptr;
  a.xg_bytes = kind ? K * 16 * (long long)p.mb * (long long)esize : 0;
  a.xpacked = kind == 2 ? 1 : 0;
}

// Whether the BPTT kernel of backward plan p accumulates dW_hh for (half)
// descriptor d: a plan with the fused variant on a packed ring, room for the
// partials, and the modelled cost of the extra per-step products (what the
// wait does not hide, plus the partial sums) below that of the separate
// product it replaces (~15 us per launch it saves, at ~50 TFLOP/s).
bool fused_dw(const rnn_desc_t* d, const rnn::RecPlan& p) {
  if (!fused_dw_shape(d) || !p.func_fdw) return false;
  const Layout L = layout(d);
  const long long K = (long long)(cell_of(d) == rnn::CELL_LSTM ? 4 : 3) * d->H;
  if (ring_kind(p, L, K, esz(d)) != 2) return false;
  const double part = (double)p.nGroups * K * (d->H + 1) * sizeof(float);
  if (part > (double)L.dwp_bytes) return false;
  const int launches = cell_of(d) == rnn::CELL_LSTM ? (d->I % 256 == 0 ? 0 : 1) : 2;
  const double saved = 15.0 * launches + 2.0 * K * d->H * (double)d->T * d->B / 50e6;
  const double cost = d->T * p.fdw_us + 5.0 + part / 4e6;
  return cost < saved;
}

// A persistent grid is launched only when every workgroup can be resident at
// once (each waits for the others every step): at most one step counter per
// workgroup, and grid <= (workgroups per CU) x CUs.
int coresidency(const rnn::RecPlan& p, bool dual, int occ, int cu) {
  const long long nwg = (long long)p.nGroups * p.nSlices;
  const long long grid = rnn::launch_blocks(p, dual);
  if (nwg > rnn::FLAG_SLOTS) return RNN_ERR_UNSUPPORTED;
  if (occ < 1 || cu < 1 || grid > (long long)occ * cu) return RNN_ERR_UNSUPPORTED;
  return RNN_OK;
}

int launch_persistent(const rnn::RecPlan& p, const rnn::RecLaunch& Lr, const DevInfo& di, hipStream_t s,
                      const char* what) {
  const long long grid = rnn::launch_blocks(p, Lr.dual != 0);
  const int occ = rnn::max_coresident(p);
  if (coresidency(p, Lr.dual != 0, occ, di.cu) != RNN_OK) {
    if (log_on()) fprintf(stderr, "[rnn] %s: grid %lld not co-resident (occupancy %d x %d CUs)\n", what, grid, occ, di.cu);
    return RNN_ERR_UNSUPPORTED;
  }
  const rnn::RecArgs& a = Lr.d[0];
  if (log_on())
    fprintf(stderr,
            "[rnn] %s: %s%d groups of %d rows x %d slices (%d units), %d waves, mb=%d nt=%d ki=%d, lds=%zu, "
            "ring=%s, counters every %d ints, model %.2f us/step\n",
            what, Lr.dual ? "2 directions x " : "", p.nGroups, p.bg, p.nSlices, p.Hs, p.nw, p.mb, p.nt, p.ki,
            p.lds_bytes, a.xbuf ? (a.xpacked ? "packed" : "tiled") : "off", a.fstride, p.cost_us);
  hipError_t e = rnn::launch_rec(p, Lr, s);
  if (e != hipSuccess) {
    if (log_on()) fprintf(stderr, "[rnn] %s: launch failed: %s\n", what, hipGetErrorString(e));
    return (e == hipErrorCooperativeLaunchTooLarge) ? RNN_ERR_UNSUPPORTED : RNN_ERR_DEVICE;
  }
  return RNN_OK;
}

// Plan of the persistent kernels: a bidirectional layer runs both halves in
// one launch on half the chip each when the plan's workgroups divide over
// the 4 XCDs of a half; otherwise each half gets the whole chip in turn.
template <typename F>
bool choose_plan(F planner, bool bidir, const DevInfo& di, rnn::RecPlan* plan, bool* dual) {
  *dual = false;
  if (bidir && planner(di.cu / 2, 4, plan) && ((plan->nGroups * plan->nSlices) % 4 == 0 || plan->per_xcd > 0)) {
    *dual = true;
    return true;
  }
  return planner(di.cu, 8, plan);
}

// The plan of pass 0 (forward) or 1 (backward through time) for d: a
// persistent plan when one fits with a co-resident grid (occ > 0: that many
// workgroups per CU, else the device's occupancy) and d does not ask for the
// per-step path; otherwise the per-step plan (nw = 0, one slice, no ring).
// Both backward calls decide here, so they agree.
bool persistent_plan(const rnn_desc_t* d, int pass, const DevInfo& di, int occ, rnn::RecPlan* plan, bool* dual) {
  const int cell = cell_of(d);
  *dual = false;
  if (!d->stepwise) {
    auto planner = [&](int cu, int xcds, rnn::RecPlan* p) {
      return pass == 0 ? rnn::plan_fwd(cell, d->dtype, d->B, d->H, cu, xcds, p)
                       : rnn::plan_bwd(cell, d->dtype, d->B, d->H, cu, xcds, p);
    };
    if (choose_plan(planner, d->direction == 2, di, plan, dual) &&
        coresidency(*plan, *dual, occ > 0 ? occ : rnn::max_coresident(*plan), di.cu) == RNN_OK)
      return true;
  }
  *plan = rnn::RecPlan{};
  plan->nGroups = plan->nSlices = 1;
  plan->Hs = d->H;
  plan->bg = d->B;
  plan->xcd_span = 1;
  *dual = false;
  return false;
}

// The per-step recurrence of every half of a layer (scratch: each half's
// GEMM region, free between the products around it).
int run_stepwise(const rnn_desc_t* d, int pass, int halves, const rnn::RecArgs (&args)[2], char* ws, size_t half_bytes,
                 hipStream_t s) {
  const rnn_desc_t h = half_desc(d, 0);
  const Layout L = layout(&h);
  for (int k = 0; k < halves; ++k) {
    float* scratch = (float*)(ws + k * half_bytes + L.gemm);
    const hipError_t e = pass == 0 ? rnn::stepwise_fwd(cell_of(d), d->dtype == RNN_BF16, args[k], scratch, L.gemm_floats, s)
                                   : rnn::stepwise_bwd(cell_of(d), d->dtype == RNN_BF16, args[k], scratch, L.gemm_floats, s);
    if (int st = hip_status(e)) return st;
  }
  if (log_on()) fprintf(stderr, "[rnn] %s: per-step path, %d steps\n", pass ? "bwd" : "fwd", d->T);
  return RNN_OK;
}

int run_persistent(const rnn::RecPlan& plan, bool dual, int halves, const rnn::RecArgs (&args)[2],
                   const DevInfo& di, hipStream_t s, const char* what) {
  if (dual) {
    rnn::RecLaunch Lr{};
    Lr.d[0] = args[0];
    Lr.d[1] = args[1];
    Lr.dual = 1;
    return launch_persistent(plan, Lr, di, s, what);
  }
  for (int k = 0; k < halves; ++k) {
    rnn::RecLaunch Lr{};
    Lr.d[0] = args[k];
    if (int st = launch_persistent(plan, Lr, di, s, what)) return st;
  }
  return RNN_OK;
}

}  // namespace

RNN_API size_t rnn_workspace_bytes(const rnn_desc_t* d) {
  if (!desc_ok(d)) return 0;
  return ws_total(d);
}

RNN_API const char* rnn_status_string(int st) {
  switch (st) {
    case RNN_OK: return "ok";
    case RNN_ERR_INVALID_ARG: return "invalid argument";
    case RNN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RNN_ERR_UNSUPPORTED: return "unsupported shape or launch configuration";
    case RNN_ERR_DEVICE: return "HIP runtime error";
    case RNN_ERR_TIMEOUT: return "step handshake timed out on the device";
    default: return "unknown status";
  }
}

RNN_API int rnn_last_device_status(const void* workspace) {
  if (!workspace) return RNN_ERR_INVALID_ARG;
  int v = 0;
  if (hipMemcpy(&v, workspace, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return RNN_ERR_DEVICE;
  return v;
}

namespace {

struct FwdIO {
  const void *x, *h0, *c0, *W_ih, *W_hh, *b_ih, *b_hh;
  void *y, *hT, *cT;
};

FwdIO fwd_half(const rnn_desc_t* d, const FwdIO& io, int k) {
  if (d->direction != 2) return io;
  const size_t es = esz(d);
  const long long G = gates(d), H = d->H, BH = (long long)d->B * d->H;
  FwdIO o = io;
  o.W_ih = at(io.W_ih, k * G * H * d->I, es);
  o.W_hh = at(io.W_hh, k * G * H * H, es);
  o.b_ih = at(io.b_ih, k * G * H, es);
  o.b_hh = at(io.b_hh, k * G * H, es);
  o.h0 = at(io.h0, k * BH, es);
  o.c0 = at(io.c0, k * BH, es);
  o.hT = at(io.hT, k * BH, es);
  o.cT = at(io.cT, k * BH, es);
  o.y = at(io.y, k * H, es);
  return o;
}

// One direction up to its persistent kernel: the counter fill, the input
// projection and the kernel's arguments.
int fwd_begin(const rnn_desc_t* d, const FwdIO& io, char* ws, const rnn::RecPlan& plan, const DevInfo& di,
              int* status, hipStream_t s, rnn::RecArgs& a) {
  int st;
  const Layout L = layout(d);
  const int cell = cell_of(d);
  int perm[4];
  inv_perm(d, perm);
  const int G = gates(d);

  // status word and the forward step counters start at zero
  {
    // one fill from the status word through the last counter this launch uses
    ProfScope ps(L_FILL, s);
    const long long n = (long long)(L.flags - L.status) / sizeof(int) + counter_ints(plan);
    if ((st = hip_status(rnn::launch_fill_i32((int*)(ws + L.status), 0, n, s)))) return st;
  }

  // input projection for every step: Z[t,b][g*H+j] = x . W_ih[g,j] + biases
  rnn::GemmArgs g{};
  g.a = rows(io.x, ldx_of(d));
  g.b = perm_rows(io.W_ih, d->I, d->H, perm);
  g.M = (long long)d->T * d->B;
  g.N = (long long)G * d->H;
  g.K = d->I;
  g.c = ws + L.z;
  g.ldc = (long long)L.GZ * d->H;
  g.c_kind = 0;
  g.H = d->H;
  for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
  g.bias1 = io.b_ih;
  g.bias2 = io.b_hh;
  g.bias_skip_gate = (cell == rnn::CELL_GRU_RA) ? RNN_GATE_C : -1;
  g.part = (float*)(ws + L.gemm);
  g.ws_floats = (long long)L.gemm_floats;
  {
    ProfScope ps(L_PROJ, s);
    if ((st = hip_status(gemm_dt(d->dtype, g, false, false, s)))) return st;
  }

  a = rnn::RecArgs{};
  a.T = d->T;
  a.B = d->B;
  a.H = d->H;
  a.dir = d->direction;
  a.nGroups = plan.nGroups;
  a.nSlices = plan.nSlices;
  a.Hs = plan.Hs;
  a.bg = plan.bg;
  for (int i = 0; i < 4; ++i) a.perm[i] = perm[i];
  a.W_hh = io.W_hh;
  a.b_hh = io.b_hh;
  a.h0 = io.h0;
  a.c0 = io.c0;
  a.y = io.y;
  a.ldy = ldy_of(d);
  a.z = ws + L.z;
  a.GZ = L.GZ;
  a.cbuf = (cell == rnn::CELL_LSTM && !d->recompute) ? ws + L.c : nullptr;
  a.ldc = d->H;
  a.rh = ws + L.rh;
  a.hT = io.hT;
  a.cT = (d->mode == RNN_LSTM) ? io.cT : nullptr;
  a.GD = L.GD;
  a.flags = (int*)(ws + L.flags);
  counter_layout(plan, &a.fstride, &a.place_off);
  a.status = status;
  a.timeout_ticks = di.ticks;
  a.lengths = d->lengths;
  a.att = d->att;
  if (cell != rnn::CELL_GRU_BASIC) set_xbuf(a, plan, L, ws, d->H, esz(d));
  return RNN_OK;
}

// Past a row's length the kernels keep the latched state in y when it is
// also their exchange buffer; the output there is zero.
int fwd_end(const rnn_desc_t* d, const rnn::RecArgs& a, hipStream_t s) {
  if (d->lengths && !a.xbuf) {
    ProfScope ps(L_AUX, s);
    const hipError_t e = d->dtype == RNN_BF16
                             ? rnn::launch_zero_inactive<bf16>(a.y, a.ldy, d->lengths, d->T, d->B, d->H, s)
                             : rnn::launch_zero_inactive<float>(a.y, a.ldy, d->lengths, d->T, d->B, d->H, s);
    return hip_status(e);
  }
  return RNN_OK;
}

struct BwdIO {
  const void *W_ih, *W_hh, *h0, *c0, *y, *dy, *dhT, *dcT;
  void *dx, *dh0, *dc0, *datt;
};

BwdIO bwd_half(const rnn_desc_t* d, const BwdIO& io, int k) {
  if (d->direction != 2) return io;
  const size_t es = esz(d);
  const long long G = gates(d), H = d->H, BH = (long long)d->B * d->H;
  BwdIO o = io;
  o.W_ih = at(io.W_ih, k * G * H * d->I, es);
  o.W_hh = at(io.W_hh, k * G * H * H, es);
  o.h0 = at(io.h0, k * BH, es);
  o.c0 = at(io.c0, k * BH, es);
  o.y = at(io.y, k * H, es);
  o.dy = at(io.dy, k * H, es);
  o.dhT = at(io.dhT, k * BH, es);
  o.dcT = at(io.dcT, k * BH, es);
  o.dh0 = at(io.dh0, k * BH, es);
  o.dc0 = at(io.dc0, k * BH, es);
  return o;  // dx and datt are shared: the second half adds to them
}

// One direction up to its BPTT kernel: the counter fill, the cell-state
// rebuild (recompute mode) and the kernel's arguments.
int bwd_begin(const rnn_desc_t* d, const BwdIO& io, char* ws, const rnn::RecPlan& plan, const DevInfo& di,
              int* status, hipStream_t s, rnn::RecArgs& a) {
  int st;
  const Layout L = layout(d);
  const int cell = cell_of(d);
  int perm[4];
  inv_perm(d, perm);
  int* flags = (int*)(ws + L.flags) + rnn::FLAG_PASS;
  {
    // one fill from the status word through the last backward counter (the
    // forward counters in between are no longer read)
    ProfScope ps(L_FILL, s);
    const long long n = (long long)(flags - (int*)(ws + L.status)) + counter_ints(plan);
    if ((st = hip_status(rnn::launch_fill_i32((int*)(ws + L.status), 0, n, s)))) return st;
  }

  a = rnn::RecArgs{};
  a.T = d->T;
  a.B = d->B;
  a.H = d->H;
  a.dir = d->direction;
  a.nGroups = plan.nGroups;
  a.nSlices = plan.nSlices;
  a.Hs = plan.Hs;
  a.bg = plan.bg;
  for (int i = 0; i < 4; ++i) a.perm[i] = perm[i];
  a.W_hh = io.W_hh;
  a.h0 = io.h0;
  a.c0 = (d->mode == RNN_LSTM) ? io.c0 : nullptr;
  a.y = (void*)io.y;
  a.ldy = ldy_of(d);
  a.z = ws + L.z;
  a.GZ = L.GZ;
  a.cbuf = ws + L.c;
  a.ldc = d->H;
  if (d->recompute) {
    // cell states rebuilt from the saved gates into the input-gate lane of
    // the gate-gradient rows: step t's lane is read by the BPTT kernel
    // before its own gradients overwrite it, and by no step after that
    ProfScope ps(L_AUX, s);
    const hipError_t e =
        d->dtype == RNN_BF16
            ? rnn::launch_lstm_cell_scan<bf16>(ws + L.z, (long long)L.GZ * d->H, io.c0, d->lengths, d->T, d->B,
                                               d->H, d->direction, ws + L.dg, (long long)L.GD * d->H, s)
            : rnn::launch_lstm_cell_scan<float>(ws + L.z, (long long)L.GZ * d->H, io.c0, d->lengths, d->T, d->B,
                                                d->H, d->direction, ws + L.dg, (long long)L.GD * d->H, s);
    if ((st = hip_status(e))) return st;
    a.cbuf = ws + L.dg;
    a.ldc = (long long)L.GD * d->H;
  }
  a.rh = ws + L.rh;
  a.dy = io.dy;
  a.dhT = io.dhT;
  a.dcT = (d->mode == RNN_LSTM) ? io.dcT : nullptr;
  a.dg = ws + L.dg;
  a.GD = L.GD;
  a.dh0 = io.dh0;
  a.dc0 = (d->mode == RNN_LSTM) ? io.dc0 : nullptr;
  a.flags = flags;
  counter_layout(plan, &a.fstride, &a.place_off);
  a.status = status;
  a.timeout_ticks = di.ticks;
  a.lengths = d->lengths;
  a.att = d->att;
  a.datt_part = (float*)(ws + L.attp);
  if (cell != rnn::CELL_GRU_BASIC) set_xbuf(a, plan, L, ws, (long long)(cell == rnn::CELL_LSTM ? 4 : 3) * d->H, esz(d));
  a.dwp = fused_dw(d, plan) ? (float*)(ws + L.dwp) : nullptr;
  // W_hh transposed into the contraction order of the BPTT kernel (unit-major
  // rows for the bf16 LSTM ring, gate-major otherwise), so that the kernel
  // loads its operands as rows instead of one element per load. Measured: at
  // 8 MiB of W_hh the kernel's start-up falls by 13-17 us for an 8 us
  // transpose; at 4 MiB and below the transpose costs more than it saves.
  a.W_hhT = nullptr;
  const int kq = 16 / (int)esz(d);
  const size_t whh_bytes = (size_t)gates(d) * d->H * d->H * esz(d);
  if (plan.nw > 0 && cell != rnn::CELL_GRU_BASIC && d->H % kq == 0 && whh_bytes >= ((size_t)8 << 20)) {
    const bool umaj = cell == rnn::CELL_LSTM && d->dtype == RNN_BF16 && plan.mb < 4 && a.xbuf != nullptr;
    const int G = gates(d);
    ProfScope ps(L_AUX, s);
    const hipError_t e =
        d->dtype == RNN_BF16
            ? rnn::launch_weight_transpose<bf16>(io.W_hh, G, d->H, d->H, perm, ws + L.wht, (long long)G * d->H, s, umaj)
            : rnn::launch_weight_transpose<float>(io.W_hh, G, d->H, d->H, perm, ws + L.wht, (long long)G * d->H, s,
                                                  umaj);
    if ((st = hip_status(e))) return st;
    a.W_hhT = ws + L.wht;
  }
  return RNN_OK;
}

// After the BPTT kernel: the score-gradient sum and the input gradient.
int bwd_end(const rnn_desc_t* d, const BwdIO& io, char* ws, const rnn::RecPlan& plan, const rnn::RecArgs& a,
            int accumulate, hipStream_t s) {
  int st;
  const Layout L = layout(d);
  int perm[4];
  inv_perm(d, perm);
  const int G = gates(d);
  if (d->att && io.datt) {
    ProfScope ps(L_AUX, s);
    const long long TB = (long long)d->T * d->B;
    const hipError_t e =
        d->dtype == RNN_BF16
            ? rnn::launch_att_reduce<bf16>(a.datt_part, plan.nSlices, TB, io.datt, accumulate ? 1 : 0, s)
            : rnn::launch_att_reduce<float>(a.datt_part, plan.nSlices, TB, io.datt, accumulate ? 1 : 0, s);
    if ((st = hip_status(e))) return st;
  }
  if (io.dx) {
    // dx[t,b] = sum over input-side gate rows of dG[t,b][n] W_ih[n], through
    // W_ih transposed to [I][G*H] (both operands k-contiguous)
    ProfScope ps(L_DX, s);
    {
      const hipError_t e =
          d->dtype == RNN_BF16
              ? rnn::launch_weight_transpose<bf16>(io.W_ih, G, d->H, d->I, perm, ws + L.wt, (long long)G * d->H, s)
              : rnn::launch_weight_transpose<float>(io.W_ih, G, d->H, d->I, perm, ws + L.wt, (long long)G * d->H, s);
      if ((st = hip_status(e))) return st;
    }
    rnn::GemmArgs g{};
    g.a = rows(ws + L.dg, (long long)L.GD * d->H);
    g.b = rows(ws + L.wt, (long long)G * d->H);
    g.M = (long long)d->T * d->B;
    g.N = d->I;
    g.K = (long long)G * d->H;
    g.c = io.dx;
    g.ldc = ldx_of(d);
    g.H = d->H;
    g.accumulate = accumulate ? 1 : 0;
    g.part = (float*)(ws + L.gemm);
    g.ws_floats = (long long)L.gemm_floats;
    if (nt_weight_grads(d)) {
      // the gate gradients transposed for the weight gradients, written
      // from the product's own A tiles
      g.at = ws + L.dgt;
      g.ld_at = g.M;
    }
    if ((st = hip_status(gemm_dt(d->dtype, g, false, false, s)))) return st;
    if (nt_weight_grads(d) && L.GD > G) {
      // reset-after GRU: the lane the input gradient does not read (the
      // candidate gradient times r, for the recurrent side) by a transpose
      ProfScope ps2(L_AUX, s);
      const long long TB = (long long)d->T * d->B;
      const hipError_t e = transpose_dt(d->dtype, 
          rows(ws + L.dg + (size_t)G * d->H * esz(d), (long long)L.GD * d->H), (L.GD - G) * d->H, d->T, d->B,
          ws + L.dgt + (size_t)G * d->H * TB * esz(d), s);
      if ((st = hip_status(e))) return st;
    }
  } else if (nt_weight_grads(d)) {
    ProfScope ps(L_AUX, s);
    const hipError_t e = transpose_dt(d->dtype, rows(ws + L.dg, (long long)L.GD * d->H), L.GD * d->H,
                                                            d->T, d->B, ws + L.dgt, s);
    if ((st = hip_status(e))) return st;
  }
  return RNN_OK;
}

}  // namespace

RNN_API int rnn_fwd(const rnn_desc_t* d, const void* x, const void* h0, const void* c0, const void* W_ih,
                    const void* W_hh, const void* b_ih, const void* b_hh, void* y, void* hT, void* cT,
                    void* workspace, size_t ws_bytes, void* stream) {
  int st = check_common(d, workspace, ws_bytes);
  if (st) return st;
  if (!x || !W_ih || !W_hh || !b_ih || !b_hh || !y) return RNN_ERR_INVALID_ARG;
  const void* ptrs[] = {x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT, d->lengths, d->att};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return RNN_ERR_INVALID_ARG;
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  g_cu_count = di.cu;
  const int cell = cell_of(d);
  const bool bidir = d->direction == 2;
  const int halves = bidir ? 2 : 1;
  rnn::RecPlan plan;
  bool dual;
  const bool pers = persistent_plan(d, 0, di, 0, &plan, &dual);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const rnn_desc_t hd[2] = {half_desc(d, 0), half_desc(d, 1)};
  const size_t half_bytes = layout(&hd[0]).total;
  int* status = (int*)(ws + layout(&hd[0]).status);
  const FwdIO io{x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT};
  rnn::RecArgs args[2]{};
  for (int k = 0; k < halves; ++k)
    if ((st = fwd_begin(&hd[k], fwd_half(d, io, k), ws + k * half_bytes, plan, di, status, s, args[k]))) return st;
  {
    ProfScope ps(L_RFWD, s);
    if (pers) st = run_persistent(plan, dual, halves, args, di, s, "fwd");
    else st = run_stepwise(d, 0, halves, args, ws, half_bytes, s);
    if (st) return st;
  }
  for (int k = 0; k < halves; ++k)
    if ((st = fwd_end(&hd[k], args[k], s))) return st;
  return RNN_OK;
}

// ---- forward with no allocation and no workspace argument ----
// The workspace of rnn_fwd_noalloc is this array. In host code its name is
// a host-side stand-in: the device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever passed to kernels. Every call on a device shares that device's copy;
// each call starts by zeroing its status word and step counters with a fill
// kernel, as rnn_fwd does, and calls that overlap in time on one device race.
static __device__ __align__(256) unsigned char scratch[RNN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RNN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return RNN_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RNN_OK;
}
}  // namespace

RNN_API int rnn_fwd_noalloc(const rnn_desc_t* d, const void* x, const void* h0, const void* c0, const void* W_ih,
                            const void* W_hh, const void* b_ih, const void* b_hh, void* y, void* hT, void* cT,
                            void* stream) {
  // size checks first: a descriptor beyond the array is refused on the host
  if (!desc_ok(d)) return RNN_ERR_INVALID_ARG;
  if (ws_total(d) > (size_t)RNN_NOALLOC_SCRATCH_BYTES) return RNN_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (int st = scratch_ptr(&ws)) return st;
  return rnn_fwd(d, x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT, ws, (size_t)RNN_NOALLOC_SCRATCH_BYTES, stream);
}

RNN_API int rnn_bwd_data(const rnn_desc_t* d, const void* W_ih, const void* W_hh, const void* h0, const void* c0,
                         const void* y, const void* dy, const void* dhT, const void* dcT, void* dx, void* dh0,
                         void* dc0, void* datt, int accumulate, void* workspace, size_t ws_bytes,
                         void* stream) {
  int st = check_common(d, workspace, ws_bytes);
  if (st) return st;
  if (!W_ih || !W_hh || !y || !dy) return RNN_ERR_INVALID_ARG;
  const void* ptrs[] = {W_ih, W_hh, h0, c0, y, dy, dhT, dcT, dx, dh0, dc0, datt, d->lengths, d->att};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return RNN_ERR_INVALID_ARG;
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  g_cu_count = di.cu;
  const int cell = cell_of(d);
  const bool bidir = d->direction == 2;
  const int halves = bidir ? 2 : 1;
  rnn::RecPlan plan;
  bool dual;
  const bool pers = persistent_plan(d, 1, di, 0, &plan, &dual);
  // the score-gradient shares of a workgroup's units sit after its reduction buffer
  if (d->att) plan.lds_bytes += (size_t)plan.mb * 16 * plan.Hs * sizeof(float);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const rnn_desc_t hd[2] = {half_desc(d, 0), half_desc(d, 1)};
  const size_t half_bytes = layout(&hd[0]).total;
  int* status = (int*)(ws + layout(&hd[0]).status);
  const BwdIO io{W_ih, W_hh, h0, c0, y, dy, dhT, dcT, dx, dh0, dc0, datt};
  rnn::RecArgs args[2]{};
  for (int k = 0; k < halves; ++k)
    if ((st = bwd_begin(&hd[k], bwd_half(d, io, k), ws + k * half_bytes, plan, di, status, s, args[k]))) return st;
  {
    ProfScope ps(L_RBWD, s);
    if (pers) st = run_persistent(plan, dual, halves, args, di, s, "bwd");
    else st = run_stepwise(d, 1, halves, args, ws, half_bytes, s);
    if (st) return st;
  }
  // the second half of a bidirectional layer adds its dx and score gradient
  for (int k = 0; k < halves; ++k)
    if ((st = bwd_end(&hd[k], bwd_half(d, io, k), ws + k * half_bytes, plan, args[k], k == 0 ? accumulate : 1, s)))
      return st;
  return RNN_OK;
}

namespace {
// Weight gradients of one direction. fused_groups > 0: the BPTT kernel left
// that many per-group dW_hh partials in the workspace.
int bwd_weights_dir(const rnn_desc_t* d, const void* x, const void* h0, const void* y, void* dW_ih, void* dW_hh,
                    void* db_ih, void* db_hh, int accumulate, void* workspace, void* stream, int fused_groups) {
  int st;
  const Layout L = layout(d);
  const int cell = cell_of(d);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int perm[4];
  inv_perm(d, perm);
  const int G = gates(d);
  const int H = d->H;
  const long long TB = (long long)d->T * d->B;
  const long long GDH = (long long)L.GD * H;
  const char* dg = ws + L.dg;
  const size_t s_el = esz(d);
  float* partial = (float*)(ws + L.partial);
  const int acc = accumulate ? 1 : 0;

  // dW rows [row0, row0+nrows) = dG[:, dg_col..]^T act, plus (optionally)
  // the bias gradient of the same rows = sum over (t,b) of those dG columns
  auto dW = [&](void* out, long long row0, long long nrows, int dg_col, rnn::RowMap act, long long ncols,
                void* bias_out) {
    rnn::GemmArgs g{};
    g.a = rows(dg + dg_col * s_el, GDH);   // k-outer: memory row (t,b), elements along gate rows
    g.b = act;                             // k-outer: memory row (t,b), elements along columns
    g.M = nrows;
    g.N = ncols;
    g.K = TB;
    g.c = out;
    g.ldc = ncols;
    g.c_kind = 1;
    g.c_row0 = row0;
    g.H = H;
    for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
    g.accumulate = acc;
    g.part = (float*)(ws + L.gemm);
    g.ws_floats = (long long)L.gemm_floats;
    g.rowsum_out = bias_out;
    ProfScope ps(L_DW, s);
    return gemm_dt(d->dtype, g, true, true, s);
  };

  rnn::RowMap hprev{};
  hprev.ptr = y;
  hprev.ld = ldy_of(d);
  hprev.kind = 2;
  hprev.h0 = h0;
  hprev.ld0 = H;
  hprev.B = d->B;
  hprev.T = d->T;
  hprev.dir = d->direction;

  // LSTM with both weight gradients: one product over [x | h_{t-1}] with two
  // output parts (dG is read once, one split-K finish); the bias gradients
  // (equal for the two biases) come from its row sums
  const bool fused = fused_groups > 0;
  const bool merged = cell == rnn::CELL_LSTM && dW_ih && dW_hh && d->I % 256 == 0 && !fused;
  // reset-after GRU (bf16): the r and u rows as one product over
  // [x | h_{t-1}] like the LSTM's; the candidate rows take different
  // gradients on the two sides (d_c against x, d_c * r against h_{t-1}), two
  // products of their own
  const bool gra_nt = cell == rnn::CELL_GRU_RA && dW_ih && dW_hh && !fused && nt_weight_grads(d);
  // basic GRU (bf16): the candidate rows see r * h_{t-1} on the recurrent
  // side and the same gradient d_c on both, so they too are one product
  const bool grb_nt = cell == rnn::CELL_GRU_BASIC && dW_ih && dW_hh && !fused && nt_weight_grads(d);
  if (gra_nt) {
    ProfScope ps(L_DW, s);
    hipError_t e = transpose_dt(d->dtype, rows(x, ldx_of(d)), d->I, d->T, d->B, ws + L.xt, s);
    if (e == hipSuccess) e = transpose_dt(d->dtype, hprev, H, d->T, d->B, ws + L.ht, s);
    if ((st = hip_status(e))) return st;
    // A rows [lane*H, ...) of the transposed gate gradients
    auto prod = [&](int lane, long long M, rnn::RowMap b, long long N, void* c, long long ldc, long long row0,
                    void* rs1, void* rs2) {
      rnn::GemmArgs g{};
      g.a = rows(ws + L.dgt + (size_t)lane * H * TB * s_el, TB);
      g.b = b;
      g.M = M;
      g.N = N;
      g.K = TB;
      g.c = c;
      g.ldc = ldc;
      g.c_kind = 1;
      g.c_row0 = row0;
      g.H = H;
      for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
      g.accumulate = acc;
      g.part = (float*)(ws + L.gemm);
      g.ws_floats = (long long)L.gemm_floats;
      g.rowsum_out = rs1;
      g.rowsum_out2 = rs2;
      return g;
    };
    rnn::GemmArgs g = prod(0, 2LL * H, rows(ws + L.xt, TB), (long long)d->I + H, dW_ih, d->I, 0, db_ih ? db_ih : db_hh,
                           db_ih ? db_hh : nullptr);
    g.b2 = rows(ws + L.ht, TB);
    g.n_split = d->I;
    g.c2 = dW_hh;
    g.ldc2 = H;
    if ((st = hip_status(gemm_dt(d->dtype, g, false, false, s)))) return st;
    g = prod(2, H, rows(ws + L.xt, TB), d->I, dW_ih, d->I, 2LL * H, db_ih, nullptr);
    if ((st = hip_status(gemm_dt(d->dtype, g, false, false, s)))) return st;
    g = prod(3, H, rows(ws + L.ht, TB), H, dW_hh, H, 2LL * H, db_hh, nullptr);
    if ((st = hip_status(gemm_dt(d->dtype, g, false, false, s)))) return st;
  } else if (grb_nt) {
    ProfScope ps(L_DW, s);
    hipError_t e = transpose_dt(d->dtype, rows(x, ldx_of(d)), d->I, d->T, d->B, ws + L.xt, s);
    if (e == hipSuccess) e = transpose_dt(d->dtype, hprev, H, d->T, d->B, ws + L.ht, s);
    if (e == hipSuccess) e = transpose_dt(d->dtype, rows(ws + L.rh, H), H, d->T, d->B, ws + L.rht, s);
    if ((st = hip_status(e))) return st;
    // rows [lane*H, lane*H + M) of both weight gradients, one product over
    // [x | act]; the two bias gradients of those rows are equal
    auto prod = [&](int lane, long long M, const char* act) {
      rnn::GemmArgs g{};
      g.a = rows(ws + L.dgt + (size_t)lane * H * TB * s_el, TB);
      g.b = rows(ws + L.xt, TB);
      g.b2 = rows(act, TB);
      g.n_split = d->I;
      g.M = M;
      g.N = (long long)d->I + H;
      g.K = TB;
      g.c = dW_ih;
      g.ldc = d->I;
      g.c2 = dW_hh;
      g.ldc2 = H;
      g.c_kind = 1;
      g.c_row0 = (long long)lane * H;
      g.H = H;
      for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
      g.accumulate = acc;
      g.part = (float*)(ws + L.gemm);
      g.ws_floats = (long long)L.gemm_floats;
      g.rowsum_out = db_ih ? db_ih : db_hh;
      g.rowsum_out2 = db_ih ? db_hh : nullptr;
      return gemm_dt(d->dtype, g, false, false, s);
    };
    if ((st = hip_status(prod(0, 2LL * H, ws + L.ht)))) return st;
    if ((st = hip_status(prod(2, H, ws + L.rht)))) return st;
  } else if (merged && nt_weight_grads(d)) {
    // the same product with k-contiguous operands: dG^T (written by the
    // input-gradient product) against x^T and h_{t-1}^T; the bias gradients
    // from its row sums
    ProfScope ps(L_DW, s);
    rnn::GemmArgs g{};
    hipError_t e = transpose_dt(d->dtype, rows(x, ldx_of(d)), d->I, d->T, d->B, ws + L.xt, s);
    if (e == hipSuccess) e = transpose_dt(d->dtype, hprev, H, d->T, d->B, ws + L.ht, s);
    if ((st = hip_status(e))) return st;
    g.a = rows(ws + L.dgt, TB);
    g.b = rows(ws + L.xt, TB);
    g.b2 = rows(ws + L.ht, TB);
    g.n_split = d->I;
    g.M = (long long)G * H;
    g.N = (long long)d->I + H;
    g.K = TB;
    g.c = dW_ih;
    g.ldc = d->I;
    g.c2 = dW_hh;
    g.ldc2 = H;
    g.c_kind = 1;
    g.c_row0 = 0;
    g.H = H;
    for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
    g.accumulate = acc;
    g.part = (float*)(ws + L.gemm);
    g.ws_floats = (long long)L.gemm_floats;
    g.rowsum_out = db_ih ? db_ih : db_hh;
    g.rowsum_out2 = db_ih ? db_hh : nullptr;
    if ((st = hip_status(gemm_dt(d->dtype, g, false, false, s)))) return st;
  } else if (merged) {
    rnn::GemmArgs g{};
    g.a = rows(dg, GDH);
    g.b = rows(x, ldx_of(d));
    g.b2 = hprev;
    g.n_split = d->I;
    g.M = (long long)G * H;
    g.N = (long long)d->I + H;
    g.K = TB;
    g.c = dW_ih;
    g.ldc = d->I;
    g.c2 = dW_hh;
    g.ldc2 = H;
    g.c_kind = 1;
    g.c_row0 = 0;
    g.H = H;
    for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
    g.accumulate = acc;
    g.part = (float*)(ws + L.gemm);
    g.ws_floats = (long long)L.gemm_floats;
    g.rowsum_out = db_ih ? db_ih : db_hh;
    g.rowsum_out2 = db_ih ? db_hh : nullptr;
    ProfScope ps(L_DW, s);
    if ((st = hip_status(gemm_dt(d->dtype, g, true, true, s)))) return st;
  } else if (dW_ih) {
    if ((st = hip_status(dW(dW_ih, 0, (long long)G * H, 0, rows(x, ldx_of(d)), d->I, db_ih)))) return st;
  } else if (db_ih) {
    if ((st = hip_status(colsum_dt(d->dtype, dg, GDH, TB, 0, G * H, db_ih, 0, H, perm, acc, partial, s)))) return st;
  }
  // recurrent side: lanes of dG_h (LSTM: all; GRU: r,u, then the candidate rows)
  const int ccol = (cell == rnn::CELL_GRU_RA) ? 3 * H : 2 * H;  // candidate lane of dG_h
  if ((dW_hh || db_hh) && fused) {
    // the per-group partials of the BPTT kernel, summed in group order (the
    // kernel used each row's own h_{t-1}, so no direction-1 correction)
    ProfScope ps(L_DW, s);
    const int K = (cell == rnn::CELL_LSTM ? 4 : 3) * H;
    if ((st = hip_status(rnn::launch_dw_partials_finish<float>((const float*)(ws + L.dwp), fused_groups, K, H, perm,
                                                               dW_hh, db_hh, acc, s))))
      return st;
  }
  if (dW_hh && !fused) {
    if (merged || gra_nt || grb_nt) {
      // done above
    } else if (cell == rnn::CELL_LSTM) {
      if ((st = hip_status(dW(dW_hh, 0, 4LL * H, 0, hprev, H, db_hh)))) return st;
    } else {
      if ((st = hip_status(dW(dW_hh, 0, 2LL * H, 0, hprev, H, db_hh)))) return st;
      rnn::RowMap cact = (cell == rnn::CELL_GRU_RA) ? hprev : rows(ws + L.rh, H);
      if ((st = hip_status(dW(dW_hh, 2LL * H, H, ccol, cact, H, db_hh)))) return st;
    }
    // Direction 1 with variable lengths: a row b with 0 < L_b < T starts at
    // step L_b - 1 from h0, where the h_{t-1} map reads y of step L_b (zero
    // there). Add those rows' dG^T h0 terms from a gathered copy of their
    // gate gradients. The basic GRU's candidate rows see r*h_{t-1}, which
    // the forward kept with the right state.
    if (d->direction == 1 && d->lengths && h0) {
      char* gath = ws + L.gath;
      {
        ProfScope ps(L_AUX, s);
        const hipError_t e =
            d->dtype == RNN_BF16
                ? rnn::launch_gather_first_rows<bf16>(dg, GDH, 0, (int)GDH, d->lengths, d->T, d->B, gath, s)
                : rnn::launch_gather_first_rows<float>(dg, GDH, 0, (int)GDH, d->lengths, d->T, d->B, gath, s);
        if ((st = hip_status(e))) return st;
      }
      auto corr = [&](long long row0, long long nrows, int col) {
        rnn::GemmArgs g{};
        g.a = rows(gath + col * s_el, GDH);
        g.b = rows(h0, H);
        g.M = nrows;
        g.N = H;
        g.K = d->B;
        g.c = dW_hh;
        g.ldc = H;
        g.c_kind = 1;
        g.c_row0 = row0;
        g.H = H;
        for (int i = 0; i < 4; ++i) g.perm[i] = perm[i];
        g.accumulate = 1;
        g.part = (float*)(ws + L.gemm);
        g.ws_floats = (long long)L.gemm_floats;
        ProfScope ps(L_DW, s);
        return gemm_dt(d->dtype, g, true, true, s);
      };
      if (cell == rnn::CELL_LSTM) {
        if ((st = hip_status(corr(0, 4LL * H, 0)))) return st;
      } else {
        if ((st = hip_status(corr(0, 2LL * H, 0)))) return st;
        if (cell == rnn::CELL_GRU_RA && (st = hip_status(corr(2LL * H, H, ccol)))) return st;
      }
    }
  }
  if (db_hh && !dW_hh && !fused) {
    if (cell == rnn::CELL_LSTM) {
      if ((st = hip_status(colsum_dt(d->dtype, dg, GDH, TB, 0, 4 * H, db_hh, 0, H, perm, acc, partial, s)))) return st;
    } else {
      if ((st = hip_status(colsum_dt(d->dtype, dg, GDH, TB, 0, 2 * H, db_hh, 0, H, perm, acc, partial, s)))) return st;
      if ((st = hip_status(colsum_dt(d->dtype, dg, GDH, TB, ccol, H, db_hh, 2 * H, H, perm, acc, partial, s))))
        return st;
    }
  }
  return RNN_OK;
}
}  // namespace

RNN_API int rnn_bwd_weights(const rnn_desc_t* d, const void* x, const void* h0, const void* y, void* dW_ih,
                            void* dW_hh, void* db_ih, void* db_hh, int accumulate, void* workspace,
                            size_t ws_bytes, void* stream) {
  int st = check_common(d, workspace, ws_bytes);
  if (st) return st;
  if (!x || !y) return RNN_ERR_INVALID_ARG;
  const void* ptrs[] = {x, h0, y, dW_ih, dW_hh, db_ih, db_hh, d->lengths};
  for (const void* p : ptrs)
    if (p && !aligned(p)) return RNN_ERR_INVALID_ARG;
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  g_cu_count = di.cu;
  const rnn_desc_t h0d = half_desc(d, 0);
  int fused_groups = 0;
  if (fused_dw_shape(&h0d)) {
    rnn::RecPlan plan;
    bool dual;
    if (persistent_plan(d, 1, di, 0, &plan, &dual) && fused_dw(&h0d, plan)) fused_groups = plan.nGroups;
  }
  if (d->direction != 2)
    return bwd_weights_dir(d, x, h0, y, dW_ih, dW_hh, db_ih, db_hh, accumulate, workspace, stream, fused_groups);
  // the two halves in turn, each over its own workspace half and [2][...] slice
  const size_t es = esz(d);
  const long long G = gates(d), H = d->H, BH = (long long)d->B * d->H;
  for (int k = 0; k < 2; ++k) {
    const rnn_desc_t h = half_desc(d, k);
    const size_t hb = layout(&h).total;
    if ((st = bwd_weights_dir(&h, x, at(h0, k * BH, es), at(y, k * H, es), at(dW_ih, k * G * H * d->I, es),
                              at(dW_hh, k * G * H * H, es), at(db_ih, k * G * H, es), at(db_hh, k * G * H, es),
                              accumulate, (char*)workspace + k * hb, stream, fused_groups)))
      return st;
  }
  return RNN_OK;
}

RNN_API int rnn_plan_query(const rnn_desc_t* d, int pass, int cu_count, int wg_per_cu, rnn_plan_t* out) {
  if (!desc_ok(d) || !out || (pass != 0 && pass != 1) || cu_count < 0 || wg_per_cu < 0) return RNN_ERR_INVALID_ARG;
  if (!shape_supported(d)) return RNN_ERR_UNSUPPORTED;
  memset(out, 0, sizeof(*out));
  DevInfo di;
  if (cu_count > 0) {
    di.cu = cu_count;
  } else {
    if (int st = dev_info(&di)) return st;
  }
  const int cell = cell_of(d);
  rnn::RecPlan plan;
  bool dual;
  if (!persistent_plan(d, pass, di, wg_per_cu, &plan, &dual)) {
    out->stepwise = 1;  // no co-resident persistent grid (or asked for): one launch pair per step
    return RNN_OK;
  }
  const long long nwg = (long long)plan.nGroups * plan.nSlices;
  out->groups = plan.nGroups;
  out->rows = plan.bg;
  out->slices = plan.nSlices;
  out->units = plan.Hs;
  out->waves = plan.nw;
  out->workgroups = (int)(dual ? 2 * nwg : nwg);
  out->blocks = (int)rnn::launch_blocks(plan, dual);
  out->dual = dual ? 1 : 0;
  out->xcd_span = plan.xcd_span;
  out->model_us_per_step = plan.cost_us;
  {
    const rnn_desc_t h = half_desc(d, 0);
    const Layout L = layout(&h);
    rnn::RecArgs a{};
    const long long K = pass == 0 ? d->H : (long long)(cell == rnn::CELL_LSTM ? 4 : 3) * d->H;
    if (cell != rnn::CELL_GRU_BASIC) set_xbuf(a, plan, L, nullptr, K, esz(d));
    out->ring = a.xg_bytes ? (a.xpacked ? 2 : 1) : 0;
    out->fused_dw = pass == 1 && fused_dw(&h, plan) ? 1 : 0;
  }
  return RNN_OK;
}

RNN_API int rnn_handshake_probe(const rnn_desc_t* d, int pass, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_common(d, workspace, ws_bytes);
  if (st) return st;
  if (pass != 0 && pass != 1) return RNN_ERR_INVALID_ARG;
  const int cell = cell_of(d);
  if (cell == rnn::CELL_GRU_BASIC || d->stepwise) return RNN_ERR_UNSUPPORTED;  // no exchange ring
  DevInfo di;
  if ((st = dev_info(&di))) return st;
  g_cu_count = di.cu;
  const bool bidir = d->direction == 2;
  const int halves = bidir ? 2 : 1;
  rnn::RecPlan plan;
  bool dual;
  auto planner = [&](int cu, int xcds, rnn::RecPlan* p) {
    return pass == 0 ? rnn::plan_fwd(cell, d->dtype, d->B, d->H, cu, xcds, p)
                     : rnn::plan_bwd(cell, d->dtype, d->B, d->H, cu, xcds, p);
  };
  if (!choose_plan(planner, bidir, di, &plan, &dual)) return RNN_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const rnn_desc_t hd[2] = {half_desc(d, 0), half_desc(d, 1)};
  const size_t half_bytes = layout(&hd[0]).total;
  int* status = (int*)(ws + layout(&hd[0]).status);
  const int G = (cell == rnn::CELL_LSTM) ? 4 : 3;
  const long long K = pass == 0 ? d->H : (long long)G * d->H;
  rnn::RecArgs args[2]{};
  for (int k = 0; k < halves; ++k) {
    char* w = ws + k * half_bytes;
    const Layout L = layout(&hd[k]);
    int* flags = (int*)(w + L.flags) + (pass ? rnn::FLAG_PASS : 0);
    {
      const long long n = (long long)(flags - (int*)(w + L.status)) + counter_ints(plan);
      if ((st = hip_status(rnn::launch_fill_i32((int*)(w + L.status), 0, n, s)))) return st;
    }
    rnn::RecArgs& a = args[k];
    a.T = d->T;
    a.B = d->B;
    a.H = d->H;
    a.dir = hd[k].direction;
    a.nGroups = plan.nGroups;
    a.nSlices = plan.nSlices;
    a.Hs = plan.Hs;
    a.bg = plan.bg;
    a.flags = flags;
    counter_layout(plan, &a.fstride, &a.place_off);
    a.status = status;
    a.timeout_ticks = di.ticks;
    set_xbuf(a, plan, L, w, K, esz(d));
    if (!a.xbuf || plan.mb != 1) return RNN_ERR_UNSUPPORTED;
  }
  const int umaj = (pass == 1 && cell == rnn::CELL_LSTM && d->dtype == RNN_BF16) ? 1 : 0;
  const int gk = pass == 0 ? 1 : G;
  auto go = [&](const rnn::RecLaunch& Lr) -> int {
    const long long nwg = (long long)plan.nGroups * plan.nSlices;
    if (coresidency(plan, Lr.dual != 0, rnn::max_coresident(plan), di.cu) != RNN_OK) return RNN_ERR_UNSUPPORTED;
    return hip_status(rnn::launch_exchange_probe(plan, Lr, d->dtype, (int)K, gk, umaj, s));
  };
  if (dual) {
    rnn::RecLaunch Lr{};
    Lr.d[0] = args[0];
    Lr.d[1] = args[1];
    Lr.dual = 1;
    return go(Lr);
  }
  for (int k = 0; k < halves; ++k) {
    rnn::RecLaunch Lr{};
    Lr.d[0] = args[k];
    if ((st = go(Lr))) return st;
  }
  return RNN_OK;
}

#ifdef RNN_STEP_TIMERS
// Debug build only (include/rnn_debug.h): the per-step timers of the last
// persistent kernel(s), after the caller has synchronised.
RNN_API int rnn_step_timers_read(unsigned long long* timers, unsigned long long* cal) {
  if (!timers || !cal) return RNN_ERR_INVALID_ARG;
  return hip_status(rnn::read_step_timers(timers, cal));
}
RNN_API int rnn_step_timers_reset(void) { return hip_status(rnn::reset_step_timers()); }
RNN_API int rnn_step_timers_shape(int* wgs, int* steps, int* phases) {
  if (!wgs || !steps || !phases) return RNN_ERR_INVALID_ARG;
  *wgs = rnn::TIMER_WGS;
  *steps = rnn::TIMER_STEPS;
  *phases = rnn::TIMER_PHASES;
  return RNN_OK;
}
#endif

RNN_API int rnn_set_handshake_timeout(double seconds) {
  g_timeout_s = seconds == 0 ? TIMEOUT_S : seconds;
  return RNN_OK;
}

RNN_API int rnn_profile_enable(int on) {
  Prof& p = prof();
  p.on = on != 0;
  if (!p.on && p.pending.empty()) release_pool(p);
  return RNN_OK;
}

RNN_API int rnn_profile_read(rnn_kernel_time_t* out, int max, int reset) {
  Prof& p = prof();
  int st = RNN_OK;
  for (const Pending& e : p.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(e.b) != hipSuccess || hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) st = RNN_ERR_DEVICE;
    p.total[e.label] += ms;
    p.count[e.label] += 1;
    p.pool.push_back(e.a);
    p.pool.push_back(e.b);
  }
  p.pending.clear();
  if (!p.on) release_pool(p);
  if (st != RNN_OK) return st;
  int n = 0;
  for (int l = 0; l < L_COUNT; ++l) {
    if (p.count[l] == 0) continue;
    if (out && n < max) {
      memset(&out[n], 0, sizeof(out[n]));
      strncpy(out[n].name, kLabel[l], sizeof(out[n].name) - 1);
      out[n].launches = p.count[l];
      out[n].total_ms = p.total[l];
    }
    ++n;
  }
  if (reset) {
    for (int l = 0; l < L_COUNT; ++l) {
      p.total[l] = 0;
      p.count[l] = 0;
    }
  }
  return n;
}
