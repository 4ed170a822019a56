// C ABI of the fused RNN operator: descriptor, packed-weight layout,
// workspace plan, argument checks and launch sequence.
//
// The call sequence follows the workspace protocol of oneDNN issue #218 "rnn
// training example?" (size query, caller-allocated workspace written by the
// training forward pass and read by the backward pass) and the reserved
// workspace of the MXNet "fused RNN operator" page (Operator Registration):
// intermediates saved by the forward pass are reused by backward, and the
// buffer (not its content) is reused across iterations.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "rnn.h"
#include "rnn_common.h"

using namespace rnnk;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

enum KernelId { K_GEMM_IN = 0, K_FWD = 1, K_BWD = 2, K_GEMM_DX = 3, K_GEMM_DW = 4, K_FILL = 5, K_PREP = 6,
                K_PROBE = 7, K_DROPOUT = 8, K_NKERNELS = 9 };

struct ProfPending {
  hipEvent_t a, b;
  int kernel;
};

// Recurrent launch plan for one sweep kind.
struct SweepPlan {
  RecConfig cfg{};
  int nchunk = 0, Bc = 0;   // batch chunks of Bc rows
  int U = 0, nwg = 0, groups = 0, grid = 0;
  int place = 0;            // 1: XCD-local groups (sweep_grid)
  bool persistent = false;
  size_t lds = 0;   // dynamic LDS for staging ring entries (0: fragments read from global)
};

struct Plan {
  int T = 0, B = 0, training = 0;
  int fslice = 0, bslice = 0, fgran = 0, bgran = 0, bslice2 = 0, bgran2 = 0;
  size_t fring_step = 0, fring_group = 0, bring_step = 0, bring_group = 0;
  size_t bring_step2 = 0, bring_group2 = 0;
  bool wavefront = false;
  bool drop_rings = false;
  SweepPlan fwd, bwd;
  size_t off_err = 0, off_flags = 0, flags_bytes = 0;
  size_t off_xch = 0, xch_bytes = 0;
  size_t off_st = 0, st_bytes = 0;
  size_t off_gx = 0, gx_bytes = 0;
  size_t off_yin = 0, yin_slot = 0;
  int yin_slots = 0;
  size_t off_res = 0, res_layer = 0;
  // gate gradients in the compute type: dG [T*B][dg_ld] (dg_k columns in
  // gg_col order), dG^T [D*G*H][tb_ld] (tb_k columns in tb_k order)
  size_t off_dg = 0, off_dgT = 0, off_dghT = 0, dg_layer = 0, dgT_layer = 0;
  int dg_ld = 0, tb_ld = 0, dg_k = 0, tb_k = 0;
  size_t off_dy = 0, dy_slot = 0;
  // dropped inputs of layers 1..L-1 (training with dropout), slot l-1
  size_t off_xd = 0, xd_slot = 0;
  size_t off_scr = 0, scr_bytes = 0;   // operand preparation for the GEMMs
  size_t total = 0;
  rnn_status_t status = RNN_STATUS_SUCCESS;
};

}  // namespace

struct rnn_desc {
  int mode = 0, L = 0, D = 0, I = 0, H = 0, wtype = 0, G = 0;
  int sched = RNN_SCHED_AUTO;
  const int* lengths = nullptr;   // device [B] valid steps per row, or null
  size_t wbytes = 0, dwbytes = 0;
  std::vector<size_t> off[2][4];  // [grad][which] per layer block offset
  // pending training sequence
  int seq_stage = 0, seq_T = -1, seq_B = -1;
  const void* seq_ws = nullptr;
  const int* seq_lengths = nullptr;
  // inter-layer dropout: current setting, and the one the pending training
  // sequence's forward used
  double drop_p = 0.0;
  unsigned long long drop_seed = 0;
  double seq_drop_p = 0.0;
  unsigned long long seq_drop_seed = 0;
  // profiling
  int prof = 0;
  std::vector<ProfPending> pending;
  std::vector<hipEvent_t> pool;
  long long prof_n[K_NKERNELS] = {};
  double prof_ms[K_NKERNELS] = {};
};

namespace {

int in_width(const rnn_desc* h, int l) { return l == 0 ? h->I : h->D * h->H; }
// GRU flavours whose n reads (r*h) W_hn (two exchanges per step)
bool is_gru2(const rnn_desc* h) { return h->mode == RNN_GRU_TF || h->mode == RNN_GRU_PAPER; }
// the cell type the kernels and the workspace layout see
int kmode(const rnn_desc* h) { return is_gru2(h) ? RNN_GRU : h->mode; }

void layout_weights(rnn_desc* h) {
  for (int grad = 0; grad < 2; ++grad) {
    const size_t es = (grad == 0 && h->wtype == RNN_W_BF16) ? 2 : 4;
    const size_t gh = (size_t)h->G * h->H;
    size_t off = 0;
    for (int w = 0; w < 4; ++w) h->off[grad][w].assign(h->L, 0);
    for (int l = 0; l < h->L; ++l) {
      h->off[grad][RNN_W_IH][l] = off;
      off = align_up(off + h->D * gh * in_width(h, l) * es);
      h->off[grad][RNN_W_HH][l] = off;
      off = align_up(off + h->D * gh * h->H * es);
      h->off[grad][RNN_B_IH][l] = off;
      off = align_up(off + h->D * gh * 4);
      h->off[grad][RNN_B_HH][l] = off;
      off = align_up(off + h->D * gh * 4);
    }
    (grad ? h->dwbytes : h->wbytes) = off;
  }
}

// Candidate kernel configurations, in order of preference.
const RecConfig kFwdCfgs[] = {{1, 1, 8, 4},  {1, 2, 8, 4},  {1, 1, 16, 4}, {1, 2, 16, 4}, {2, 1, 8, 4},
                              {2, 2, 8, 4},  {2, 1, 16, 4}, {2, 2, 16, 4}, {4, 1, 4, 8},  {4, 2, 4, 8},
                              {4, 1, 8, 8},  {4, 2, 8, 8},
                              {1, 2, 32, 4}, {1, 2, 16, 8}, {2, 2, 16, 8}, {4, 2, 16, 8},
                              {8, 1, 8, 4}};
// (measured at the DS2 shapes: eight waves of 16 K chunks beat four waves
// of 32 by 11-13 % in the backward sweep -- half the granules per wave; 32
// chunks on eight waves spill, so fp32 keeps four waves of 64)
const RecConfig kBwdCfgs[] = {{1, 1, 8, 4},  {1, 2, 8, 4},  {1, 1, 16, 4}, {1, 2, 16, 4},
                              {1, 1, 16, 8}, {1, 2, 16, 8}, {1, 1, 32, 4}, {1, 2, 32, 4},
                              {1, 1, 64, 4}, {1, 2, 64, 4}, {1, 2, 32, 8}, {1, 1, 32, 8},
                              {2, 1, 16, 4}, {2, 1, 32, 4}};

// Units per workgroup are a multiple of the per-lane MFMA k run (8 bf16 / 4
// fp32 values, 16 bytes) so that every A fragment of the exchange comes from
// one producer's slice.
int unit_quantum(const rnn_desc* h) { return h->wtype == RNN_W_BF16 ? 8 : 4; }

// CUs of one XCD of an MI355X (256 CUs in 8 XCDs).
constexpr int kCusPerXcd = 32;

// Units per workgroup of an XCD-local group: the fewest that keep one
// group's workgroups within the CUs of one XCD.
int xcd_units(const rnn_desc* h) {
  const int Q = unit_quantum(h);
  return ceil_div(ceil_div(h->H, kCusPerXcd), Q) * Q;
}

// Pick a forward configuration: U so that all groups together use about
// `target_wgs` workgroups, the gate columns of U units fit the MFMA tiles, the
// K chunks fit the registers, and each epilogue thread owns one (row, unit).
// `Ureq` > 0: exactly that many units (XCD-local groups), with the wide
// (eight-column-tile) configurations allowed; 0: the planner's choice.
bool plan_fwd(const rnn_desc* h, int mt, int Bc, int groups, bool inproj, SweepPlan* sp, int Ureq = 0) {
  const int Q = unit_quantum(h);
  const int GB = (h->mode == RNN_GRU && inproj) ? 4 : h->G;
  const int target_wgs = std::max(1, env_int("RNN_FWD_TARGET_WGS", 256));
  int U = ceil_div(ceil_div(h->H * std::max(1, groups), target_wgs), Q) * Q;
  const int Uenv = env_int("RNN_FWD_UNITS", 0);
  if (Uenv > 0) U = ceil_div(Uenv, Q) * Q;
  if (Ureq > 0) U = Ureq;
  U = std::max(Q, std::min(U, ceil_div(h->H, Q) * Q));
  const int Ulow = Ureq > 0 ? U : Q;
  for (int tryU = U; tryU >= Ulow; tryU -= Q) {
    const int nwg = ceil_div(h->H, tryU);
    const int ngr = (inproj ? 2 : 1) * nwg * (tryU / Q);   // K granules
    // (measured: four waves with two load batches beat eight waves with one
    // for the fp32 DS2 forward, so the list order, fewer waves first, stands)
    const int force = env_int("RNN_FWD_CFG", -1);   // tuning: only this list entry
    for (const RecConfig& c : kFwdCfgs) {
      if (force >= 0 && &c != &kFwdCfgs[force % (int)(sizeof(kFwdCfgs) / sizeof(kFwdCfgs[0]))]) continue;
      if (c.mt != mt || (c.nt > 4 && Ureq == 0)) continue;
      if (is_gru2(h) && !rnn_gru2_fwd_config_supported(h->wtype == RNN_W_BF16, c)) continue;
      if (GB * tryU > 16 * c.nt || Bc * tryU > 64 * c.nwaves) continue;
      if (ceil_div(ceil_div(ngr, c.nwaves), 4) > c.kpw) continue;
      sp->cfg = c;
      sp->U = tryU;
      sp->nwg = nwg;
      sp->groups = groups;
      sp->grid = nwg * groups;
      return true;
    }
  }
  return false;
}

bool plan_bwd(const rnn_desc* h, int mt, int Bc, int groups, SweepPlan* sp, int Ureq = 0) {
  const int Q = unit_quantum(h);
  int U = ceil_div(std::max(1, env_int("RNN_BWD_UNITS", 16)), Q) * Q;
  if (Ureq > 0) U = Ureq;
  U = std::max(Q, std::min(U, ceil_div(h->H, Q) * Q));
  const int Ulow = Ureq > 0 ? U : Q;
  for (int tryU = U; tryU >= Ulow; tryU -= Q) {
    const int nwg = ceil_div(h->H, tryU);
    const int ngr = h->G * nwg * (tryU / Q);   // K granules
    // the flavours with two exchanges hold two weight sets: the n gate
    // (nwg*U/Q granules) and r, z (twice that), each within kpw chunks
    const int ngr2 = 2 * nwg * (tryU / Q);
    const int force = env_int("RNN_BWD_CFG", -1);   // tuning: only this list entry
    for (const RecConfig& c : kBwdCfgs) {
      if (force >= 0 && &c != &kBwdCfgs[force % (int)(sizeof(kBwdCfgs) / sizeof(kBwdCfgs[0]))]) continue;
      if (c.mt != mt || (c.kpw > 32 && h->wtype == RNN_W_BF16) || (c.nt > 1 && Ureq == 0)) continue;
      if (is_gru2(h) && !rnn_gru2_bwd_config_supported(h->wtype == RNN_W_BF16, c)) continue;
      if (tryU > 16 * c.nt || Bc * tryU > 64 * c.nwaves) continue;
      if (ceil_div(ceil_div(is_gru2(h) ? ngr2 : ngr, c.nwaves), 4) > c.kpw) continue;
      sp->cfg = c;
      sp->U = tryU;
      sp->nwg = nwg;
      sp->groups = groups;
      sp->grid = nwg * groups;
      return true;
    }
  }
  return false;
}

// Split-K factor of a time-parallel product (weight gradients, and the data
// gradient), from a two-term time model fitted at the DS2 shapes:
//  * the K loop: tiles*split workgroups of K/split each, dealt in rounds of
//    512 (two per CU, 9.3 ns per k each with bf16 operands -- the DS2 LSTM
//    weight gradient, M = 3200, N = 801, K = 6000, split 1/2/3/4: 89/67/82/79
//    us -- and 66 ns with fp32 operands -- the fp32 input projection, data
//    gradient and weight gradients unsplit: 295, 420 and 790 us); a last
//    round of at most 256 runs one per CU, 1.59x faster per workgroup than
//    two sharing a CU;
//  * summing the partials: 2.15 ps per element of the result per split.
// At least 256 k per split, at most 8 splits.
int gemm_split(const rnn_desc* h, int M, int N, int K, int batches) {
  const double us_per_k = h->wtype == RNN_W_BF16 ? 0.00933 : 0.0658;
  const int tiles = ceil_div(M, 128) * ceil_div(N, 128) * std::max(1, batches);
  const int smax = std::min(8, std::max(1, K / 256));
  const int force = env_int("RNN_DW_SPLIT", 0);   // tuning: this split factor
  if (force > 0) return std::min(force, smax);
  const double elems = (double)M * N * std::max(1, batches);
  int best = 1;
  double best_us = 1e30, unsplit_us = 0.0;
  for (int s = 1; s <= smax; ++s) {
    const int n = tiles * s, rem = n % 512;
    const double rounds = 2.0 * (n / 512) + (rem == 0 ? 0.0 : rem <= 256 ? 1.59 : 2.0);
    const double us = rounds * ceil_div(K, s) * us_per_k + (s > 1 ? 2.15e-6 * s * elems : 0.0);
    if (s == 1) unsplit_us = us;
    if (us < best_us - 1e-9) {
      best_us = us;
      best = s;
    }
  }
  // split only for a predicted gain of at least 10 % (the model's error)
  return best_us < 0.9 * unsplit_us ? best : 1;
}

// Widest layer input, rounded up to whole 16-byte bf16 vectors: the row
// count of the transposed-operand scratch (W_ih^T, X^T).
size_t input_pad(const rnn_desc* h) {
  int Imax = h->I;
  for (int l = 1; l < h->L; ++l) Imax = std::max(Imax, in_width(h, l));
  return (size_t)ceil_div(Imax, 8) * 8;
}

// The weight gradients of layer l run as one launch of two products when
// dW_ih and dW_hh have the same shape: one direction, input width = hidden
// width, one product per matrix (not the two-exchange GRU flavours).
bool dw_fused(const rnn_desc* h, int l) {
  return h->D == 1 && in_width(h, l) == h->H && !is_gru2(h) && env_int("RNN_NO_DW_FUSE", 0) == 0;
}

// `drop`: the inter-layer dropout probability of a training pass (0: none)
Plan make_plan(const rnn_desc* h, int T, int B, int training, double drop = 0.0) {
  Plan p;
  p.T = T;
  p.B = B;
  p.training = training;
  const int bf = h->wtype == RNN_W_BF16;
  const size_t es = bf ? 2 : 4;
  const int Bq = std::max(B, 1);
  auto chunk = [&](int max_bc, SweepPlan& sp) {
    max_bc = std::max(1, std::min(32, max_bc));
    sp.nchunk = ceil_div(Bq, max_bc);
    sp.Bc = ceil_div(Bq, sp.nchunk);
  };
  const int Q = unit_quantum(h);
  // rows of a granule: the batch chunk, padded so that a producer's slice
  // (granules_per_slice granules of rows x 16 bytes) is whole 128-byte lines
  auto padded_rows = [&](int Bc, int granules_per_slice) {
    int rows = Bc;
    while ((granules_per_slice * rows) % 8 != 0) ++rows;
    return rows;
  };
  const int sched = h->sched;
  const bool allow_stage = env_int("RNN_NO_STAGE", 0) == 0;
  // XCD-local recurrence groups (persistent sweeps only).  By default the
  // vanilla tanh RNN with bf16 weights takes them: one gate per unit keeps
  // the 32-unit workgroup's MFMA work as small as the 8- or 16-unit slices of
  // the linear placement, so the shorter exchange of one XCD wins (measured
  // at H = 800, T = 300: B = 1 inference 0.56 vs 0.68 ms, B = 20 training
  // step 1.39 vs 1.44 ms, the 5-layer bidirectional step 8.06 vs 8.34 ms);
  // the gated cells, whose slices are three or four times wider, and fp32
  // weights measured slower.  RNN_PLACE=1 forces XCD-local groups.
  const int place_env = env_int("RNN_PLACE", -1);
  const bool place_auto = h->G == 1 && bf;
  // (A stepped sweep takes the same units and chunks on a linear grid, so
  // that both schedules do bitwise the same arithmetic.)
  const bool place_req = place_env == 1 || (place_env < 0 && place_auto);
  // Otherwise runs of consecutive slices per XCD whose units fill one
  // 128-byte line of the fp32 per-unit data (input projection, reserve, dy),
  // so that each line is fetched through one L2 instead of two to four:
  // the default for the one-exchange forward sweeps (DS2 LSTM: inference
  // sweep 503 -> 272 MB fetched, inference 0.835 -> 0.824 ms; GRU forward
  // -1 %) and the LSTM backward (656 -> 530 MB fetched, 801 -> 794 us);
  // the other backward sweeps and the two-exchange GRU flavours (whose
  // forward measured 1.8 % slower) take them only with RNN_PLACE=2 (GRU
  // backward 788 -> 793 us); RNN_PLACE=0 gives the plain linear grid to
  // every sweep.
  auto line_runs = [&](int U, bool fwd) {
    const bool want = place_env == 2 ||
                      (place_env < 0 && !is_gru2(h) && (fwd || h->mode == RNN_LSTM));
    return want && U < 32 && 32 % U == 0 ? 32 / U : 0;
  };
  // co-residency: returns whether every workgroup of the sweep fits on the
  // GPU at once (with LDS staging if it fits, else without)
  auto fit = [&](SweepPlan& sp, bool fwd, size_t stage_bytes) {
    auto res = [&](size_t lds) {
      if (is_gru2(h)) return fwd ? rnn_gru2_fwd_max_resident(bf, sp.cfg) : rnn_gru2_bwd_max_resident(bf, sp.cfg);
      return fwd ? rnn_fwd_max_resident(kmode(h), bf, sp.cfg, lds)
                 : rnn_bwd_max_resident(kmode(h), bf, sp.cfg, lds);
    };
    if (is_gru2(h)) stage_bytes = 0;   // their backward reads fragments from the rings
    size_t lds = allow_stage ? stage_bytes : 0;
    int maxres = lds ? res(lds) : 0;
    if (lds && maxres < sp.grid) lds = 0;
    if (!lds) maxres = res(0);
    sp.lds = lds;
    const bool fits = maxres >= sp.grid && maxres > 0;
    sp.persistent = sched == RNN_SCHED_PERSISTENT || (sched == RNN_SCHED_AUTO && fits);
    return fits;
  };

  // batch-chunk caps to try, smallest first: more, smaller chunks spread the
  // exchange over more CUs (measured at the DS2 shapes: the backward sweep
  // at 4-row chunks runs 11 % faster than at 10, the forward at 10-row
  // chunks 7 % faster than at 20) as long as every workgroup stays resident;
  // 32 rows is the last resort
  auto ladder = [](int pref, std::initializer_list<int> steps) {
    std::vector<int> v;
    pref = std::max(1, std::min(32, pref));
    v.push_back(pref);
    for (int m : steps)
      if (m > v.back()) v.push_back(m);
    return v;
  };

  // ---- forward sweep
  const bool wf0 = h->D == 1 && h->L > 1 && h->L <= kMaxLayersPerLaunch && !is_gru2(h) &&
                   env_int("RNN_NO_WAVEFRONT", 0) == 0;
  // `Ux` > 0: XCD-local groups of Ux units per workgroup
  auto plan_f = [&](int max_bc, int Ux) {
    chunk(max_bc, p.fwd);
    p.wavefront = wf0;
    const int fl = p.wavefront ? h->L : 1;
    const int fmt = ceil_div(p.fwd.Bc, 16);
    if (!plan_fwd(h, fmt, p.fwd.Bc, fl * h->D * p.fwd.nchunk, p.wavefront, &p.fwd, Ux)) {
      // a wavefront layer also holds its W_ih slice (twice the K range):
      // when that fits no configuration, the layers run one launch each
      if (!p.wavefront) return false;
      p.wavefront = false;
      if (!plan_fwd(h, fmt, p.fwd.Bc, h->D * p.fwd.nchunk, false, &p.fwd, Ux)) return false;
    }
    // wavefront: every workgroup polls its own and the layer below's flags
    if (p.wavefront && 2 * p.fwd.nwg > kMaxWaitFlags) p.wavefront = false;
    if (!p.wavefront && p.fwd.groups != h->D * p.fwd.nchunk &&
        !plan_fwd(h, fmt, p.fwd.Bc, h->D * p.fwd.nchunk, false, &p.fwd, Ux))
      return false;
    if (p.fwd.nwg > kMaxWaitFlags) return false;
    p.fwd.place = Ux > 0 ? 1 : line_runs(p.fwd.U, true);
    p.fwd.grid = sweep_grid(p.fwd.place, p.fwd.nwg, p.fwd.groups);
    // exchange rings: one entry per step, entries padded to 1 KB
    const int s_total = T + (p.wavefront ? h->L : 1) - 1;
    p.fgran = padded_rows(p.fwd.Bc, p.fwd.U / Q) * 16;
    p.fslice = (p.fwd.U / Q) * p.fgran;
    p.fring_step = ((size_t)p.fwd.nwg * p.fslice + 1023) / 1024 * 1024;
    p.fring_group = align_up(p.fring_step * (size_t)(s_total + 1));
    return true;
  };
  {
    // bf16 sweeps of the LSTM (training) and of every GRU flavour (training
    // and inference) start at 4-row chunks (16 units and eight waves per
    // workgroup: measured 6-11 % faster training sweeps at the DS2 shapes,
    // the two-exchange GRU flavours 11 %, GRU inference 2 %); LSTM inference
    // and fp32 start at 16 rows (4-row chunks measured 1.5 % slower for LSTM
    // inference and up to 60 % slower with fp32 weights, whose 4-unit
    // granules make the 4-row grids wide)
    const bool gru = h->mode == RNN_GRU || is_gru2(h);
    const int fwd_pref = (bf && h->G >= 3 && (training || gru)) ? 4 : 16;
    bool ok = false, fits = false;
    if (place_req) {   // XCD-local groups: enough batch chunks to give each XCD one group
      const int per = std::max(1, kXcds / ((wf0 ? h->L : 1) * h->D));
      ok = plan_f(env_int("RNN_PLACE_BC", ceil_div(Bq, per)), xcd_units(h));
      fits = ok && fit(p.fwd, true, 0);
      ok = fits;
    }
    for (int mb : ladder(env_int("RNN_FWD_MAX_BC", fwd_pref), {16, 32})) {
      if (fits) break;
      if (ok && Bq <= p.fwd.Bc) break;   // a larger cap changes nothing
      ok = plan_f(mb, 0);
      // the forward reads its fragments straight from the ring
      fits = ok && fit(p.fwd, true, 0);
      if (fits) break;
    }
    if (!ok) {
      p.status = RNN_STATUS_UNSUPPORTED;
      return p;
    }
    if (!fits && sched == RNN_SCHED_PERSISTENT) p.status = RNN_STATUS_NOT_CORESIDENT;
    if (!p.fwd.persistent && p.fwd.place) {
      p.fwd.place = 0;
      p.fwd.grid = sweep_grid(0, p.fwd.nwg, p.fwd.groups);
    }
  }
  // a wavefront with dropout also rings each layer's dropped h for the layer above
  p.drop_rings = p.wavefront && training && drop > 0.0;
  if (is_gru2(h) && !p.fwd.persistent) p.status = RNN_STATUS_NOT_CORESIDENT;

  // ---- backward sweep: the same ladder of batch chunk sizes
  if (training) {
    auto plan_b = [&](int max_bc, int Ux) {
      chunk(max_bc, p.bwd);
      if (!plan_bwd(h, ceil_div(p.bwd.Bc, 16), p.bwd.Bc, h->D * p.bwd.nchunk, &p.bwd, Ux) ||
          p.bwd.nwg > kMaxWaitFlags)
        return false;
      p.bwd.place = Ux > 0 ? 1 : line_runs(p.bwd.U, false);
      p.bwd.grid = sweep_grid(p.bwd.place, p.bwd.nwg, p.bwd.groups);
      // the flavours with two exchanges: da_n (one gate per slice) in the
      // first ring, [da_r, da_z] (two gates) in the second
      const int gpr = is_gru2(h) ? 1 : h->G;
      p.bgran = padded_rows(p.bwd.Bc, gpr * p.bwd.U / Q) * 16;
      p.bslice = gpr * (p.bwd.U / Q) * p.bgran;
      p.bring_step = ((size_t)p.bwd.nwg * p.bslice + 1023) / 1024 * 1024;
      p.bring_group = align_up(p.bring_step * (size_t)(T + 1));
      if (is_gru2(h)) {
        p.bgran2 = padded_rows(p.bwd.Bc, 2 * p.bwd.U / Q) * 16;
        p.bslice2 = 2 * (p.bwd.U / Q) * p.bgran2;
        p.bring_step2 = ((size_t)p.bwd.nwg * p.bslice2 + 1023) / 1024 * 1024;
        p.bring_group2 = align_up(p.bring_step2 * (size_t)(T + 1));
      }
      return true;
    };
    bool ok = false, fits = false;
    if (place_req) {
      const int per = std::max(1, kXcds / h->D);
      ok = plan_b(env_int("RNN_PLACE_BC", ceil_div(Bq, per)), xcd_units(h));
      fits = ok && fit(p.bwd, false, p.bring_step);
      ok = fits;
    }
    for (int mb : ladder(env_int("RNN_BWD_MAX_BC", 4), {5, 7, 10, 16, 32})) {
      if (fits) break;
      if (ok && Bq <= p.bwd.Bc) break;   // a larger cap changes nothing
      ok = plan_b(mb, 0);
      fits = ok && fit(p.bwd, false, p.bring_step);
      if (fits) break;
    }
    if (!ok) {
      p.status = RNN_STATUS_UNSUPPORTED;
      return p;
    }
    if (!fits && sched == RNN_SCHED_PERSISTENT) p.status = RNN_STATUS_NOT_CORESIDENT;
    if (is_gru2(h) && !p.bwd.persistent) p.status = RNN_STATUS_NOT_CORESIDENT;
    if (!p.bwd.persistent && p.bwd.place) {
      p.bwd.place = 0;
      p.bwd.grid = sweep_grid(0, p.bwd.nwg, p.bwd.groups);
    }
  }

  const size_t TB = (size_t)T * B;
  const size_t dgh = (size_t)h->D * h->G * h->H;
  size_t off = 0;
  p.off_err = off;
  off = align_up(off + 256);
  p.off_flags = off;
  p.flags_bytes = (size_t)std::max(p.fwd.grid, p.bwd.grid) * kFlagStride * 4;
  off = align_up(off + p.flags_bytes);
  p.off_xch = off;
  size_t xf = (size_t)p.fwd.groups * p.fring_group * ((is_gru2(h) || p.drop_rings) ? 2 : 1);
  size_t xb = (size_t)p.bwd.groups * (p.bring_group + p.bring_group2);
  p.xch_bytes = std::max(xf, training ? xb : (size_t)0);
  off = align_up(off + p.xch_bytes);
  p.off_st = off;
  const int fl2 = p.wavefront ? h->L : 1;
  p.st_bytes = (size_t)2 * std::max(fl2, 1) * h->D * B * h->H * 4;
  off = align_up(off + p.st_bytes);
  p.off_gx = off;
  p.gx_bytes = TB * dgh * 4;
  off = align_up(off + p.gx_bytes);
  p.off_yin = off;
  p.yin_slot = align_up(TB * h->D * h->H * 4);
  if (h->L > 1) p.yin_slots = (training || p.wavefront) ? h->L - 1 : std::min(2, h->L - 1);
  off += p.yin_slot * p.yin_slots;
  p.off_xd = off;
  if (training && drop > 0.0 && h->L > 1) {
    p.xd_slot = p.yin_slot;
    off += p.xd_slot * (h->L - 1);
  }
  // operand-preparation scratch (fwd: layer input in bf16)
  const size_t Ipad = input_pad(h);
  // reduction extents of the dX and dW products in the backward sweep's
  // store orders (gg_col, tb_k): whole workgroup slices and batch chunks
  p.dg_k = training ? h->D * p.bwd.nwg * h->G * p.bwd.U : (int)dgh;
  p.tb_k = training ? p.bwd.nchunk * T * p.bwd.Bc : (int)TB;
  p.dg_ld = ceil_div(p.dg_k, 8) * 8;
  p.tb_ld = ceil_div(std::max(p.tb_k, 1), 8) * 8;
  size_t scr = bf ? align_up(TB * Ipad * 2) : 0;
  if (training) {
    const int R = reserve_slots(kmode(h));
    p.off_res = off;
    p.res_layer = align_up((size_t)h->D * TB * R * h->H * 4);
    off += p.res_layer * h->L;
    p.dg_layer = align_up(TB * (size_t)p.dg_ld * es);
    p.dgT_layer = align_up(dgh * (size_t)p.tb_ld * es);
    p.off_dg = off;
    off += p.dg_layer * h->L;
    p.off_dgT = off;
    off += p.dgT_layer * h->L;
    p.off_dghT = off;
    if (h->mode == RNN_GRU) off += p.dgT_layer * h->L;
    p.off_dy = off;
    p.dy_slot = align_up(TB * h->D * h->H * 4);
    if (h->L > 1) off += 2 * p.dy_slot;
    // backward_data: W_ih^T [I_l][dg_ld] and the dX split-K partials;
    // backward_weights: X^T, H_prev^T, split-K partials
    size_t part_dx = 0;
    for (int l = 0; l < h->L; ++l) {
      const int I_l = in_width(h, l);
      const int sdx = gemm_split(h, (int)TB, I_l, p.dg_k, 1);
      if (sdx > 1) part_dx = std::max(part_dx, (size_t)sdx * TB * I_l * 4);
    }
    scr = std::max(scr, align_up(Ipad * p.dg_ld * es) + align_up(part_dx));
    size_t wts = align_up(Ipad * p.tb_ld * es) + align_up((size_t)h->D * h->H * p.tb_ld * es);
    if (is_gru2(h)) wts += align_up((size_t)h->D * h->H * p.tb_ld * es);   // (r*H_prev)^T
    size_t part = 0;
    for (int l = 0; l < h->L; ++l) {
      const int I_l = in_width(h, l);
      if (dw_fused(h, l))
        part = std::max(part, (size_t)gemm_split(h, h->G * h->H, h->H + 1, p.tb_k, 2) * 2 *
                                  (size_t)h->G * h->H * (h->H + 1) * 4);
      part = std::max(part, (size_t)gemm_split(h, (int)dgh, I_l + 1, p.tb_k, 1) * dgh * (I_l + 1) * 4);
      part = std::max(part, (size_t)gemm_split(h, h->G * h->H, h->H + 1, p.tb_k, h->D) * h->D *
                                (size_t)h->G * h->H * (h->H + 1) * 4);
      if (is_gru2(h))   // their dW_hh in two products, 2H and H rows
        for (int m = 1; m <= 2; ++m)
          part = std::max(part, (size_t)gemm_split(h, m * h->H, h->H + 1, p.tb_k, h->D) * h->D *
                                    (size_t)m * h->H * (h->H + 1) * 4);
    }
    scr = std::max(scr, wts + align_up(part));
  }
  p.off_scr = off;
  p.scr_bytes = scr;
  off += scr;
  p.total = align_up(off);
  return p;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

// ------------------------------------------------------------- profiling
struct ProfScope {
  rnn_desc* h;
  hipStream_t s;
  int k;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(rnn_desc* h_, hipStream_t s_, int k_) : h(h_), s(s_), k(k_) {
    if (!h->prof) return;
    a = take();
    b = take();
    if (a) (void)hipEventRecord(a, s);
  }
  hipEvent_t take() {
    if (!h->pool.empty()) {
      hipEvent_t e = h->pool.back();
      h->pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  ~ProfScope() {
    if (!h->prof || !a || !b) return;
    (void)hipEventRecord(b, s);
    h->pending.push_back({a, b, k});
  }
};

void prof_collect(rnn_desc* h) {
  for (auto& e : h->pending) {
    if (hipEventSynchronize(e.b) == hipSuccess) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, e.a, e.b) == hipSuccess) {
        h->prof_n[e.kernel] += 1;
        h->prof_ms[e.kernel] += ms;
      }
    }
    h->pool.push_back(e.a);
    h->pool.push_back(e.b);
  }
  h->pending.clear();
}

rnn_status_t dev(hipError_t e) { return e == hipSuccess ? RNN_STATUS_SUCCESS : RNN_STATUS_DEVICE; }
#define RNN_TRY(expr)                          \
  do {                                         \
    rnn_status_t st_ = (expr);                 \
    if (st_ != RNN_STATUS_SUCCESS) return st_; \
  } while (0)

rnn_status_t fill(rnn_desc* h, hipStream_t s, std::initializer_list<std::pair<void*, size_t>> r,
                  uint32_t value = 0u) {
  std::vector<void*> ps;
  std::vector<size_t> ns;
  std::vector<uint32_t> vs;
  for (auto& x : r) {
    ps.push_back(x.first);
    ns.push_back(x.second);
    vs.push_back(value);
  }
  ProfScope ps_(h, s, K_FILL);
  return dev(rnn_launch_fill(ps.data(), ns.data(), vs.data(), (int)ps.size(), s));
}

// The 256-byte head of the workspace: the error word and zeros in [0, 128),
// 16-byte constant vectors for the GEMMs after it: bf16 ones at 128, fp32
// ones at 192.
constexpr size_t kZero16 = 64, kOnesBf16 = 128, kOnesF32 = 192;
// `flags` (optional): the sweep flags, cleared in the same launch.
rnn_status_t fill_head(rnn_desc* h, hipStream_t s, void* head, void* flags = nullptr,
                       size_t flag_bytes = 0) {
  char* c = reinterpret_cast<char*>(head);
  void* ptrs[4] = {c, c + kOnesBf16, c + kOnesF32, flags};
  size_t bytes[4] = {kOnesBf16, 64, 64, flag_bytes};
  uint32_t vals[4] = {0u, 0x3f803f80u, 0x3f800000u, 0u};
  ProfScope ps_(h, s, K_FILL);
  return dev(rnn_launch_fill(ptrs, bytes, vals, flags && flag_bytes ? 4 : 3, s));
}

// The same ranges as fill_head, for a launch that sets them alongside its
// own job.
FillJob head_fill_job(void* head, void* extra = nullptr, size_t extra_bytes = 0) {
  char* c = reinterpret_cast<char*>(head);
  FillJob f{};
  void* ptrs[4] = {c, c + kOnesBf16, c + kOnesF32, extra};
  size_t bytes[4] = {kOnesBf16, 64, 64, extra_bytes};
  uint32_t vals[4] = {0u, 0x3f803f80u, 0x3f800000u, 0u};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && bytes[i]) {
      f.p[f.count] = ptrs[i];
      f.bytes[f.count] = bytes[i];
      f.v[f.count] = vals[i];
      ++f.count;
    }
  return f;
}

// A launch that clears a sweep's flags alongside its own job.
FillJob flags_fill_job(void* flags, size_t bytes) {
  FillJob f{};
  f.p[0] = flags;
  f.bytes[0] = bytes;
  f.v[0] = 0u;
  f.count = 1;
  return f;
}

// Constant vectors and the kernel choice of a GEMM on this workspace.
void gemm_consts(const rnn_desc* h, GemmParams& g, const void* ws, size_t off_head) {
  const char* c = reinterpret_cast<const char*>(ws) + off_head;
  g.zero16 = c + kZero16;
  g.ones16 = c + (h->wtype == RNN_W_BF16 ? kOnesBf16 : kOnesF32);
  g.force_general = env_int("RNN_GEMM_GENERAL", 0);
}


// Polls a bounded wait makes before it expires (RNN_SPIN_LIMIT; 0 expires
// every wait at once, a host-forced timeout for tests).
unsigned spin_limit() {
  const int v = env_int("RNN_SPIN_LIMIT", 1 << 20);
  return (unsigned)std::max(0, v);
}

const void* layer_w(const rnn_desc* h, const void* W, int which, int l) {
  return reinterpret_cast<const char*>(W) + h->off[0][which][l];
}

// Hoisted input projection of layer l: GX[T*B, D*G*H] = in W_ih^T + b_ih + b_hh
// (b_hh not folded into GRU's n gate, which needs it inside r*(.)).  The bf16
// path first rounds the layer input to bf16 (the MFMA operand precision).
// `pre` (bf16 only, optional): ranges the bf16 rounding launch also sets.
rnn_status_t gemm_input(rnn_desc* h, hipStream_t s, const Plan& p, int l, const float* in,
                        const void* W, float* gx, void* ws, const FillJob* pre = nullptr) {
  GemmParams g{};
  const int I_l = in_width(h, l);
  const bool bf = h->wtype == RNN_W_BF16;
  const int EPV = bf ? 8 : 4;
  g.M = p.T * p.B;
  g.N = h->D * h->G * h->H;
  g.K = I_l;
  if (bf) {
    const int ldx = ceil_div(I_l, 8) * 8;
    void* xb = at<void>(ws, p.off_scr);
    {
      ProfScope ps(h, s, K_PREP);
      RNN_TRY(dev(rnn_launch_convert(in, I_l, xb, ldx, g.M, I_l, s, pre)));
    }
    g.A[0] = xb;
    g.lda = ldx;
    g.a_vec = 1;
  } else {
    g.A[0] = in;
    g.lda = I_l;
    g.a_vec = (I_l % EPV == 0) && ((uintptr_t)in % 16 == 0);
  }
  g.B[0] = layer_w(h, W, RNN_W_IH, l);
  g.ldb = I_l;
  // 16-byte row loads of W_ih need whole vectors per row and an aligned base
  // (W may sit at any element offset of a caller's parameter arena)
  g.b_vec = (I_l % EPV == 0) && ((uintptr_t)g.B[0] % 16 == 0);
  g.n_ones = -1;
  g.C[0] = gx;
  g.ldc = g.N;
  g.bias1 = reinterpret_cast<const float*>(layer_w(h, W, RNN_B_IH, l));
  g.bias2 = reinterpret_cast<const float*>(layer_w(h, W, RNN_B_HH, l));
  g.bias2_skip_gate = kmode(h) == RNN_GRU ? 2 : -1;   // b_hn stays inside n
  g.gh = h->G * h->H;
  g.hh = h->H;
  g.split_k = 1;
  ProfScope ps(h, s, K_GEMM_IN);
  gemm_consts(h, g, ws, p.off_err);
  return dev(rnn_launch_gemm(g, bf, EPI_BIAS, 1, s));
}

rnn_status_t check_common(const rnn_desc* h, int T, int B, const void* ws, size_t ws_bytes) {
  if (!h) return RNN_STATUS_INVALID_ARG;
  if (T < 0 || B < 0) return RNN_STATUS_INVALID_ARG;
  if (ws && ((uintptr_t)ws % kAlign) != 0) return RNN_STATUS_INVALID_ARG;
  (void)ws_bytes;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t forward_impl(rnn_desc* h, void* stream, int T, int B, const float* x, const float* h0,
                          const float* c0, const void* W, float* y, float* hy, float* cy, void* ws,
                          size_t ws_bytes, int training) {
  RNN_TRY(check_common(h, T, B, ws, ws_bytes));
  if (h->mode != RNN_LSTM && (c0 || cy)) return RNN_STATUS_INVALID_ARG;
  if (!W || !ws) return RNN_STATUS_INVALID_ARG;
  if (T > 0 && B > 0 && (!x || !y)) return RNN_STATUS_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const double drop = training ? h->drop_p : 0.0;
  Plan p = make_plan(h, T, B, training, drop);
  if (p.status != RNN_STATUS_SUCCESS) return p.status;
  if (ws_bytes < p.total) return RNN_STATUS_WORKSPACE_TOO_SMALL;
  if (h->seq_ws == ws) h->seq_stage = 0;

  // the first persistent sweep's flags are cleared with the head; with bf16
  // operands both are set by the launch that rounds layer 0's input (one
  // launch fewer per call)
  bool flags_clear = p.fwd.persistent && T > 0 && B > 0;
  const bool head_in_convert = h->wtype == RNN_W_BF16 && T > 0 && B > 0;
  const FillJob head_job = head_fill_job(at<void>(ws, p.off_err), flags_clear ? at<void>(ws, p.off_flags) : nullptr,
                                         p.flags_bytes);
  if (!head_in_convert)
    RNN_TRY(fill_head(h, s, at<void>(ws, p.off_err), flags_clear ? at<void>(ws, p.off_flags) : nullptr,
                      p.flags_bytes));
  const FillJob* pre = head_in_convert ? &head_job : nullptr;
  const size_t nstate = (size_t)h->L * h->D * B * h->H;
  if (T == 0 || B == 0) {
    if (hy) RNN_TRY(dev(rnn_copy_state(hy, h0, nstate, s)));
    if (cy) RNN_TRY(dev(rnn_copy_state(cy, c0, nstate, s)));
    if (training) {
      h->seq_stage = 1;
      h->seq_T = T;
      h->seq_B = B;
      h->seq_ws = ws;
      h->seq_lengths = h->lengths;
      h->seq_drop_p = drop;
      h->seq_drop_seed = h->drop_seed;
    }
    return RNN_STATUS_SUCCESS;
  }
  const int bf = h->wtype == RNN_W_BF16;
  float* gx = at<float>(ws, p.off_gx);
  auto yin = [&](int l) { return at<float>(ws, p.off_yin + p.yin_slot * (size_t)((training || p.wavefront) ? l : (l % 2))); };
  auto res = [&](int l) { return training ? at<float>(ws, p.off_res + p.res_layer * l) : nullptr; };

  FwdParams f{};
  f.T = T;
  f.B = B;
  f.H = h->H;
  f.D = h->D;
  f.nchunk = p.fwd.nchunk;
  f.place = p.fwd.place;
  f.ngroups = p.fwd.groups;
  f.Bc = p.fwd.Bc;
  f.U = p.fwd.U;
  f.nwg = p.fwd.nwg;
  f.slice = p.fslice;
  f.gran = p.fgran;
  f.group_poll = env_int("RNN_GROUP_POLL", 0);
  f.ring_step = (long long)p.fring_step;
  f.ring_group = (long long)p.fring_group;
  f.stage = p.fwd.lds > 0 ? 1 : 0;
  f.persistent = p.fwd.persistent ? 1 : 0;
  f.training = training;
  f.lengths = h->lengths;
  f.h0 = h0;
  f.c0 = c0;
  f.hy = hy;
  f.cy = cy;
  f.st_h = at<float>(ws, p.off_st);
  f.st_c = at<float>(ws, p.off_st + p.st_bytes / 2);
  f.xch = at<void>(ws, p.off_xch);
  // the flavours with two exchanges: the r*h ring after the h rings
  f.xch2 = is_gru2(h) ? at<void>(ws, p.off_xch + (size_t)p.fwd.groups * p.fring_group) : nullptr;
  f.paper = h->mode == RNN_GRU_PAPER ? 1 : 0;
  f.flags = at<unsigned>(ws, p.off_flags);
  f.err = at<unsigned>(ws, p.off_err);
  f.spin_limit = spin_limit();

  auto run_sweep = [&](int nlayers) -> rnn_status_t {
    f.nlayers = nlayers;
    f.s_total = T + nlayers - 1;
    const int grid = p.fwd.grid;   // (groups = nlayers * D * nchunk)
    if (f.persistent && !flags_clear) RNN_TRY(fill(h, s, {{at<void>(ws, p.off_flags), p.flags_bytes}}));
    flags_clear = false;
    if (f.persistent) {
      f.s_begin = -1;
      f.s_end = f.s_total;
      ProfScope ps(h, s, K_FWD);
      if (is_gru2(h)) return dev(rnn_launch_gru2_fwd(f, bf, p.fwd.cfg, grid, s));
      return dev(rnn_launch_fwd(f, h->mode, bf, p.fwd.cfg, grid, p.fwd.lds, s));
    }
    if (is_gru2(h)) return RNN_STATUS_NOT_CORESIDENT;
    for (int st = -1; st < f.s_total; ++st) {
      f.s_begin = st;
      f.s_end = st + 1;
      ProfScope ps(h, s, K_FWD);
      RNN_TRY(dev(rnn_launch_fwd(f, h->mode, bf, p.fwd.cfg, grid, p.fwd.lds, s)));
    }
    return RNN_STATUS_SUCCESS;
  };

  if (p.wavefront) {
    RNN_TRY(gemm_input(h, s, p, 0, x, W, gx, ws, pre));
    f.wavefront = 1;
    if (p.drop_rings) {
      f.xch_drop = at<void>(ws, p.off_xch + (size_t)p.fwd.groups * p.fring_group);
      f.drop_thr = (unsigned long long)std::floor(drop * 4294967296.0);
      f.drop_scale = drop < 1.0 ? (float)(1.0 / (1.0 - drop)) : 0.f;
      f.drop_k0 = (unsigned)(h->drop_seed & 0xFFFFFFFFull);
      f.drop_k1 = (unsigned)(h->drop_seed >> 32);
    }
    f.first_layer = 0;
    f.gx = gx;
    for (int l = 0; l < h->L; ++l) {
      f.w_ih[l] = layer_w(h, W, RNN_W_IH, l);
      f.w_hh[l] = layer_w(h, W, RNN_W_HH, l);
      f.b_ih[l] = reinterpret_cast<const float*>(layer_w(h, W, RNN_B_IH, l));
      f.b_hh[l] = reinterpret_cast<const float*>(layer_w(h, W, RNN_B_HH, l));
      f.in_l[l] = in_width(h, l);
      f.y[l] = (l == h->L - 1) ? y : yin(l);
      f.reserve[l] = res(l);
    }
    RNN_TRY(run_sweep(h->L));
    // the dropped inputs of the upper layers, for their weight gradients
    for (int l = 1; l < h->L && drop > 0.0 && training; ++l) {
      ProfScope ps(h, s, K_DROPOUT);
      RNN_TRY(dev(rnn_launch_dropout(yin(l - 1), at<float>(ws, p.off_xd + p.xd_slot * (size_t)(l - 1)), nullptr,
                                     (long long)T * B * h->D * h->H, h->drop_seed, l, drop, s)));
    }
  } else {
    f.wavefront = 0;
    for (int l = 0; l < h->L; ++l) {
      const float* in = (l == 0) ? x : yin(l - 1);
      if (l > 0 && drop > 0.0) {   // layer l reads y_{l-1} * keep / (1 - p)
        float* xd = at<float>(ws, p.off_xd + p.xd_slot * (size_t)(l - 1));
        ProfScope ps(h, s, K_DROPOUT);
        RNN_TRY(dev(rnn_launch_dropout(in, xd, nullptr, (long long)T * B * h->D * h->H,
                                       h->drop_seed, l, drop, s)));
        in = xd;
      }
      // the bf16 rounding of an upper layer's input runs after the sweep
      // below and clears the flags of this layer's sweep in the same launch
      const FillJob flag_job = flags_fill_job(at<void>(ws, p.off_flags), p.flags_bytes);
      const bool fold = l > 0 && bf && f.persistent;
      RNN_TRY(gemm_input(h, s, p, l, in, W, gx, ws, l == 0 ? pre : (fold ? &flag_job : nullptr)));
      if (fold) flags_clear = true;
      f.first_layer = l;
      f.gx = gx;
      f.w_ih[0] = layer_w(h, W, RNN_W_IH, l);
      f.w_hh[0] = layer_w(h, W, RNN_W_HH, l);
      f.b_ih[0] = reinterpret_cast<const float*>(layer_w(h, W, RNN_B_IH, l));
      f.b_hh[0] = reinterpret_cast<const float*>(layer_w(h, W, RNN_B_HH, l));
      f.in_l[0] = in_width(h, l);
      f.y[0] = (l == h->L - 1) ? y : yin(l);
      f.reserve[0] = res(l);
      RNN_TRY(run_sweep(1));
    }
  }
  if (training) {
    h->seq_stage = 1;
    h->seq_T = T;
    h->seq_B = B;
    h->seq_ws = ws;
    h->seq_lengths = h->lengths;
    h->seq_drop_p = drop;
    h->seq_drop_seed = h->drop_seed;
  }
  return RNN_STATUS_SUCCESS;
}

// The forward sweep's launch with only its exchange: the same grid, waits,
// ring stores and flags, no weights, arithmetic or outputs.
rnn_status_t exchange_probe_impl(rnn_desc* h, void* stream, int T, int B, int training, void* ws,
                                 size_t ws_bytes) {
  RNN_TRY(check_common(h, T, B, ws, ws_bytes));
  if (!ws) return RNN_STATUS_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Plan p = make_plan(h, T, B, training ? 1 : 0);
  if (p.status != RNN_STATUS_SUCCESS) return p.status;
  if (ws_bytes < p.total) return RNN_STATUS_WORKSPACE_TOO_SMALL;
  if (!p.fwd.persistent) return RNN_STATUS_NOT_CORESIDENT;
  if (h->seq_ws == ws) h->seq_stage = 0;
  RNN_TRY(fill_head(h, s, at<void>(ws, p.off_err)));
  if (T == 0 || B == 0) return RNN_STATUS_SUCCESS;
  FwdParams f{};
  f.T = T;
  f.B = B;
  f.H = h->H;
  f.D = h->D;
  f.nchunk = p.fwd.nchunk;
  f.place = p.fwd.place;
  f.ngroups = p.fwd.groups;
  f.Bc = p.fwd.Bc;
  f.U = p.fwd.U;
  f.nwg = p.fwd.nwg;
  f.slice = p.fslice;
  f.gran = p.fgran;
  f.ring_step = (long long)p.fring_step;
  f.ring_group = (long long)p.fring_group;
  f.persistent = 1;
  f.probe = 1;
  f.wavefront = p.wavefront ? 1 : 0;
  f.nlayers = p.wavefront ? h->L : 1;
  f.s_total = T + f.nlayers - 1;
  f.s_begin = -1;
  f.s_end = f.s_total;
  for (int l = 0; l < f.nlayers; ++l) f.in_l[l] = in_width(h, l);
  f.xch = at<void>(ws, p.off_xch);
  f.flags = at<unsigned>(ws, p.off_flags);
  f.err = at<unsigned>(ws, p.off_err);
  f.spin_limit = spin_limit();
  const int grid = p.fwd.grid;
  RNN_TRY(fill(h, s, {{at<void>(ws, p.off_flags), p.flags_bytes}}));
  ProfScope ps(h, s, K_PROBE);
  // (the flavours with two exchanges per step probe one of them)
  return dev(rnn_launch_fwd(f, kmode(h), h->wtype == RNN_W_BF16, p.fwd.cfg, grid, p.fwd.lds, s));
}

}  // namespace

// ------------------------------------------------ inference without allocation
// The workspace of rnn_forward_inference_static: a fixed device array of the
// library, one copy per device (the runtime places it when the code object is
// loaded on that device; it is held until the process ends).  Host code never
// uses the array's name as an address: its device address is looked up once
// per device, with that device current, and kept.
static constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

rnn_status_t static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return RNN_STATUS_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return RNN_STATUS_DEVICE;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RNN_STATUS_SUCCESS;
}
}  // namespace


// ================================================================== C ABI
extern "C" {

rnn_status_t rnn_create(rnn_handle_t* out, rnn_mode_t mode, int num_layers, int num_dirs,
                        int input_size, int hidden_size, rnn_wtype_t wtype) {
  if (!out) return RNN_STATUS_INVALID_ARG;
  *out = nullptr;
  if (mode != RNN_TANH && mode != RNN_LSTM && mode != RNN_GRU && mode != RNN_GRU_TF &&
      mode != RNN_GRU_PAPER)
    return RNN_STATUS_INVALID_ARG;
  if (wtype != RNN_W_F32 && wtype != RNN_W_BF16) return RNN_STATUS_INVALID_ARG;
  if (num_layers <= 0 || input_size <= 0 || hidden_size <= 0) return RNN_STATUS_INVALID_ARG;
  if (num_dirs != 1 && num_dirs != 2) return RNN_STATUS_INVALID_ARG;
  rnn_desc* h = new (std::nothrow) rnn_desc();
  if (!h) return RNN_STATUS_INVALID_ARG;
  h->mode = mode;
  h->L = num_layers;
  h->D = num_dirs;
  h->I = input_size;
  h->H = hidden_size;
  h->wtype = wtype;
  h->G = gates_of(kmode(h));
  layout_weights(h);
  *out = h;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_destroy(rnn_handle_t h) {
  if (!h) return RNN_STATUS_SUCCESS;
  prof_collect(h);
  for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
  delete h;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_set_sequence_lengths(rnn_handle_t h, const int* lengths) {
  if (!h) return RNN_STATUS_INVALID_ARG;
  h->lengths = lengths;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_set_dropout(rnn_handle_t h, double p, unsigned long long seed) {
  if (!h || !(p >= 0.0 && p <= 1.0)) return RNN_STATUS_INVALID_ARG;
  h->drop_p = p;
  h->drop_seed = seed;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_dropout_mask(rnn_handle_t h, void* stream, int T, int B, int layer,
                              unsigned char* mask) {
  if (!h || T < 0 || B < 0 || layer < 1 || layer >= h->L) return RNN_STATUS_INVALID_ARG;
  const long long n = (long long)T * B * h->D * h->H;
  if (n == 0) return RNN_STATUS_SUCCESS;
  if (!mask) return RNN_STATUS_INVALID_ARG;
  return dev(rnn_launch_dropout(nullptr, nullptr, mask, n, h->drop_seed, layer, h->drop_p,
                                reinterpret_cast<hipStream_t>(stream)));
}

rnn_status_t rnn_set_schedule(rnn_handle_t h, rnn_schedule_t s) {
  if (!h || (s != RNN_SCHED_AUTO && s != RNN_SCHED_PERSISTENT && s != RNN_SCHED_STEPPED))
    return RNN_STATUS_INVALID_ARG;
  h->sched = s;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_weights_size(rnn_handle_t h, int grad, size_t* bytes) {
  if (!h || !bytes) return RNN_STATUS_INVALID_ARG;
  *bytes = grad ? h->dwbytes : h->wbytes;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_weight_offset(rnn_handle_t h, int grad, int layer, int dir, rnn_param_t which,
                               size_t* byte_offset, size_t* elem_count) {
  if (!h || !byte_offset || !elem_count) return RNN_STATUS_INVALID_ARG;
  if (layer < 0 || layer >= h->L || dir < 0 || dir >= h->D) return RNN_STATUS_INVALID_ARG;
  if (which < RNN_W_IH || which > RNN_B_HH) return RNN_STATUS_INVALID_ARG;
  const int g = grad ? 1 : 0;
  const size_t es = (which <= RNN_W_HH && !g && h->wtype == RNN_W_BF16) ? 2 : 4;
  const size_t gh = (size_t)h->G * h->H;
  size_t count = gh;
  if (which == RNN_W_IH) count = gh * in_width(h, layer);
  if (which == RNN_W_HH) count = gh * h->H;
  *elem_count = count;
  *byte_offset = h->off[g][which][layer] + (size_t)dir * count * es;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_workspace_size(rnn_handle_t h, int T, int B, int training, size_t* bytes) {
  if (!h || !bytes || T < 0 || B < 0) return RNN_STATUS_INVALID_ARG;
  Plan p = make_plan(h, T, B, training ? 1 : 0, training ? h->drop_p : 0.0);
  if (p.status == RNN_STATUS_UNSUPPORTED) return p.status;
  *bytes = p.total;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_plan_info(rnn_handle_t h, int T, int B, int training, int* out) {
  if (!h || !out || T < 0 || B < 0) return RNN_STATUS_INVALID_ARG;
  Plan p = make_plan(h, T, B, training ? 1 : 0, training ? h->drop_p : 0.0);
  if (p.status == RNN_STATUS_UNSUPPORTED) return p.status;
  for (int i = 0; i < 16; ++i) out[i] = 0;
  auto put = [&](int base, const SweepPlan& sp) {
    const int v[8] = {sp.nchunk, sp.Bc, sp.U, sp.nwg, sp.groups, sp.grid, sp.place, sp.persistent ? 1 : 0};
    for (int i = 0; i < 8; ++i) out[base + i] = v[i];
  };
  put(0, p.fwd);
  if (training) put(8, p.bwd);
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_forward_inference(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                   const float* h0, const float* c0, const void* W, float* y,
                                   float* hy, float* cy, void* ws, size_t ws_bytes) {
  return forward_impl(h, stream, T, B, x, h0, c0, W, y, hy, cy, ws, ws_bytes, 0);
}

rnn_status_t rnn_forward_training(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                  const float* h0, const float* c0, const void* W, float* y,
                                  float* hy, float* cy, void* ws, size_t ws_bytes) {
  return forward_impl(h, stream, T, B, x, h0, c0, W, y, hy, cy, ws, ws_bytes, 1);
}

rnn_status_t rnn_backward_data(rnn_handle_t h, void* stream, int T, int B, const float* y,
                               const float* dy, const float* dhy, const float* dcy, const void* W,
                               const float* h0, const float* c0, float* dx, float* dh0,
                               float* dc0, void* ws, size_t ws_bytes) {
  RNN_TRY(check_common(h, T, B, ws, ws_bytes));
  if (h->mode != RNN_LSTM && (dcy || dc0 || c0)) return RNN_STATUS_INVALID_ARG;
  if (!W || !ws) return RNN_STATUS_INVALID_ARG;
  if (T > 0 && B > 0 && (!y || !dy || !dx)) return RNN_STATUS_INVALID_ARG;
  if (h->seq_stage < 1 || h->seq_ws != ws || h->seq_T != T || h->seq_B != B ||
      h->seq_lengths != h->lengths)
    return RNN_STATUS_BAD_CALL_ORDER;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Plan p = make_plan(h, T, B, 1, h->seq_drop_p);
  if (p.status != RNN_STATUS_SUCCESS) return p.status;
  if (ws_bytes < p.total) return RNN_STATUS_WORKSPACE_TOO_SMALL;
  // the head and the first sweep's flags are set by the launch that
  // transposes the top layer's W_ih (it depends on nothing the sweep makes,
  // so it runs before the sweep): one launch fewer per call
  bool flags_clear = p.bwd.persistent && T > 0 && B > 0;
  const bool head_in_transpose = T > 0 && B > 0;
  const FillJob head_job = head_fill_job(at<void>(ws, p.off_err), flags_clear ? at<void>(ws, p.off_flags) : nullptr,
                                         p.flags_bytes);
  if (!head_in_transpose)
    RNN_TRY(fill_head(h, s, at<void>(ws, p.off_err), flags_clear ? at<void>(ws, p.off_flags) : nullptr,
                      p.flags_bytes));
  const size_t nstate = (size_t)h->L * h->D * B * h->H;
  if (T == 0 || B == 0) {
    if (dh0) RNN_TRY(dev(rnn_copy_state(dh0, dhy, nstate, s)));
    if (dc0) RNN_TRY(dev(rnn_copy_state(dc0, dcy, nstate, s)));
    h->seq_stage = 2;
    return RNN_STATUS_SUCCESS;
  }
  const int bf = h->wtype == RNN_W_BF16;
  const size_t lstride = (size_t)h->D * B * h->H;
  const size_t dgh = (size_t)h->D * h->G * h->H;
  auto yl = [&](int l) -> const float* {
    return l == h->L - 1 ? y : at<float>(ws, p.off_yin + p.yin_slot * (size_t)l);
  };
  auto dyslot = [&](int i) { return at<float>(ws, p.off_dy + p.dy_slot * (size_t)(i % 2)); };
  BwdParams b{};
  b.T = T;
  b.B = B;
  b.H = h->H;
  b.D = h->D;
  b.nchunk = p.bwd.nchunk;
  b.place = p.bwd.place;
  b.ngroups = p.bwd.groups;
  b.Bc = p.bwd.Bc;
  b.U = p.bwd.U;
  b.nwg = p.bwd.nwg;
  b.slice = p.bslice;
  b.gran = p.bgran;
  b.group_poll = env_int("RNN_GROUP_POLL", 0);
  b.ring_step = (long long)p.bring_step;
  b.ring_group = (long long)p.bring_group;
  b.stage = p.bwd.lds > 0 ? 1 : 0;
  b.persistent = p.bwd.persistent ? 1 : 0;
  b.lengths = h->lengths;
  b.st_dh = at<float>(ws, p.off_st);
  b.st_dc = at<float>(ws, p.off_st + p.st_bytes / 2);
  b.xch = at<void>(ws, p.off_xch);
  if (is_gru2(h)) {   // [da_r, da_z] rings after the da_n rings
    b.xch2 = at<void>(ws, p.off_xch + (size_t)p.bwd.groups * p.bring_group);
    b.gran2 = p.bgran2;
    b.slice2 = p.bslice2;
    b.ring_step2 = (long long)p.bring_step2;
    b.ring_group2 = (long long)p.bring_group2;
  }
  b.paper = h->mode == RNN_GRU_PAPER ? 1 : 0;
  b.flags = at<unsigned>(ws, p.off_flags);
  b.err = at<unsigned>(ws, p.off_err);
  b.spin_limit = spin_limit();
  // W_ih^T [I_l][dg_ld] in the scratch, the B operand of layer l's dX product
  void* wT = at<void>(ws, p.off_scr);
  auto transpose_w = [&](int l, const FillJob* fill) -> rnn_status_t {
    TransposeParams tp{};
    tp.src = layer_w(h, W, RNN_W_IH, l);
    tp.ld_src = in_width(h, l);
    tp.alt_r0 = tp.alt_r1 = 0;
    tp.out = wT;
    tp.ld_out = p.dg_ld;
    tp.R = p.dg_k;   // columns in the sweep's dG order (gg_col)
    tp.C = in_width(h, l);
    tp.map = 1;
    tp.mU = p.bwd.U;
    tp.mG = h->G;
    tp.mH = h->H;
    tp.mNwg = p.bwd.nwg;
    ProfScope ps(h, s, K_PREP);
    return dev(rnn_launch_transpose(tp, bf, bf, s, fill));
  };
  if (head_in_transpose) RNN_TRY(transpose_w(h->L - 1, &head_job));
  for (int l = h->L - 1; l >= 0; --l) {
    b.w_hh = layer_w(h, W, RNN_W_HH, l);
    b.reserve = at<float>(ws, p.off_res + p.res_layer * l);
    b.y = yl(l);
    b.h0 = h0 ? h0 + l * lstride : nullptr;
    b.c0 = c0 ? c0 + l * lstride : nullptr;
    b.dy = (l == h->L - 1) ? dy : dyslot(l);
    b.dhy = dhy ? dhy + l * lstride : nullptr;
    b.dcy = dcy ? dcy + l * lstride : nullptr;
    b.dg = at<void>(ws, p.off_dg + p.dg_layer * l);
    b.dgT = at<void>(ws, p.off_dgT + p.dgT_layer * l);
    b.dghT = h->mode == RNN_GRU ? at<void>(ws, p.off_dghT + p.dgT_layer * l) : nullptr;
    b.dg_ld = p.dg_ld;
    b.tb_ld = p.tb_ld;
    b.dh0 = dh0 ? dh0 + l * lstride : nullptr;
    b.dc0 = dc0 ? dc0 + l * lstride : nullptr;
    if (b.persistent && !flags_clear) RNN_TRY(fill(h, s, {{at<void>(ws, p.off_flags), p.flags_bytes}}));
    flags_clear = false;
    if (b.persistent) {
      b.s_begin = 0;
      b.s_end = T + 1;
      ProfScope ps(h, s, K_BWD);
      if (is_gru2(h)) RNN_TRY(dev(rnn_launch_gru2_bwd(b, bf, p.bwd.cfg, p.bwd.grid, s)));
      else RNN_TRY(dev(rnn_launch_bwd(b, h->mode, bf, p.bwd.cfg, p.bwd.grid, p.bwd.lds, s)));
    } else {
      if (is_gru2(h)) return RNN_STATUS_NOT_CORESIDENT;
      for (int st = 0; st <= T; ++st) {
        b.s_begin = st;
        b.s_end = st + 1;
        ProfScope ps(h, s, K_BWD);
        RNN_TRY(dev(rnn_launch_bwd(b, h->mode, bf, p.bwd.cfg, p.bwd.grid, p.bwd.lds, s)));
      }
    }
    // dX_l = dG_i W_ih  (both directions in one product, K = D*G*H); B = W_ih^T
    // (the top layer's was transposed before its sweep)
    const int I_l = in_width(h, l);
    // (layer l's transpose runs after its sweep: below the top it also
    // clears the flags of the next sweep, layer l-1's)
    if (!(head_in_transpose && l == h->L - 1)) {
      const FillJob flag_job = flags_fill_job(at<void>(ws, p.off_flags), p.flags_bytes);
      const bool fold = l > 0 && b.persistent;
      RNN_TRY(transpose_w(l, fold ? &flag_job : nullptr));
      if (fold) flags_clear = true;
    }
    GemmParams g{};
    g.M = T * B;
    g.N = I_l;
    g.K = p.dg_k;
    g.A[0] = b.dg;
    g.lda = p.dg_ld;
    g.B[0] = wT;
    g.ldb = p.dg_ld;
    g.n_ones = -1;
    g.C[0] = (l == 0) ? dx : dyslot(l - 1);
    g.ldc = I_l;
    g.a_vec = 1;
    g.b_vec = 1;
    g.split_k = gemm_split(h, g.M, g.N, g.K, 1);
    if (g.split_k > 1)   // partials after W_ih^T in the scratch
      g.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(wT) + align_up(input_pad(h) * p.dg_ld * (bf ? 2 : 4)));
    {
      ProfScope ps(h, s, K_GEMM_DX);
      gemm_consts(h, g, ws, p.off_err);
      RNN_TRY(dev(rnn_launch_gemm(g, bf, EPI_STORE, 1, s)));
    }
    if (l > 0 && h->seq_drop_p > 0.0) {   // d y_{l-1} = d(input of l) * keep / (1 - p)
      float* dyl = dyslot(l - 1);
      ProfScope ps(h, s, K_DROPOUT);
      RNN_TRY(dev(rnn_launch_dropout(dyl, dyl, nullptr, (long long)T * B * h->D * h->H,
                                     h->seq_drop_seed, l, h->seq_drop_p, s)));
    }
  }
  h->seq_stage = 2;
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_backward_weights(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                  const float* h0, const float* y, void* ws, size_t ws_bytes,
                                  float* dW) {
  RNN_TRY(check_common(h, T, B, ws, ws_bytes));
  if (!ws || !dW) return RNN_STATUS_INVALID_ARG;
  if (T > 0 && B > 0 && (!x || !y)) return RNN_STATUS_INVALID_ARG;
  if (h->seq_stage < 2 || h->seq_ws != ws || h->seq_T != T || h->seq_B != B ||
      h->seq_lengths != h->lengths)
    return RNN_STATUS_BAD_CALL_ORDER;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Plan p = make_plan(h, T, B, 1, h->seq_drop_p);
  if (p.status != RNN_STATUS_SUCCESS) return p.status;
  if (ws_bytes < p.total) return RNN_STATUS_WORKSPACE_TOO_SMALL;
  void* wsm = ws;
  if (T == 0 || B == 0) return fill(h, s, {{dW, h->dwbytes}});
  const int bf = h->wtype == RNN_W_BF16;
  const size_t lstride = (size_t)h->D * B * h->H;
  const int GH = h->G * h->H;
  const int dgh = h->D * GH;
  auto yl = [&](int l) -> const float* {
    return l == h->L - 1 ? y : at<float>(wsm, p.off_yin + p.yin_slot * (size_t)l);
  };
  (void)lstride;
  char* dWb = reinterpret_cast<char*>(dW);
  const size_t TB = (size_t)T * B;
  const size_t es = bf ? 2 : 4;
  const size_t Ipad = input_pad(h);
  char* scr = at<char>(wsm, p.off_scr);
  void* xT = scr;
  char* hT = scr + align_up(Ipad * p.tb_ld * es);
  const size_t hT_bytes = align_up((size_t)h->D * h->H * p.tb_ld * es);
  // (r*H_prev)^T [D][H][T*B] for the flavours whose n reads W_hn (r*h)
  char* rhT = is_gru2(h) ? hT + hT_bytes : nullptr;
  float* part = reinterpret_cast<float*>(hT + hT_bytes * (is_gru2(h) ? 2 : 1));
  const int R = reserve_slots(kmode(h));
  for (int l = 0; l < h->L; ++l) {
    const int I_l = in_width(h, l);
    const float* X = (l == 0) ? x
                     : (h->seq_drop_p > 0.0 ? at<float>(wsm, p.off_xd + p.xd_slot * (size_t)(l - 1))
                                            : yl(l - 1));
    const char* dgT = at<char>(wsm, p.off_dgT + p.dgT_layer * l);
    const char* dghT = h->mode == RNN_GRU ? at<char>(wsm, p.off_dghT + p.dgT_layer * l) : dgT;
    {  // X^T [I_l][tb_ld] and H_prev^T [D][H][tb_ld] (shifted one step, h0 at the
       // start), columns in the sweep's dG^T order (tb_k), in as few launches as
       // the batched transpose allows
      ProfScope ps(h, s, K_PREP);
      std::vector<TransposeParams> jobs;
      auto kmap = [&](TransposeParams& q) {
        q.R = p.tb_k;
        q.map = 2;
        q.mBc = p.bwd.Bc;
        q.mT = T;
        q.mB = B;
      };
      TransposeParams tp{};
      tp.src = X;
      tp.ld_src = I_l;
      tp.out = xT;
      tp.ld_out = p.tb_ld;
      tp.C = I_l;
      kmap(tp);
      jobs.push_back(tp);
      for (int d = 0; d < h->D; ++d) {
        TransposeParams th{};
        th.src = yl(l) + (size_t)d * h->H;
        th.ld_src = (long long)h->D * h->H;
        th.shift = d == 0 ? -B : B;
        th.alt = h0 ? h0 + l * lstride + (size_t)d * B * h->H : nullptr;
        th.ld_alt = h->H;
        th.alt_r0 = d == 0 ? 0 : (T - 1) * B;
        th.alt_r1 = th.alt_r0 + B;
        th.out = hT + (size_t)d * h->H * p.tb_ld * es;
        th.ld_out = p.tb_ld;
        th.C = h->H;
        kmap(th);
        if (d == 1) {   // a row's first reverse step starts from h0
          th.lengths = h->lengths;
          th.len_B = B;
          th.len_T = T;
        }
        jobs.push_back(th);
        if (rhT) {   // reserve slot 3 holds r*h_prev of every step
          TransposeParams tr{};
          tr.src = at<float>(wsm, p.off_res + p.res_layer * l) + (size_t)d * TB * R * h->H + 3 * (size_t)h->H;
          tr.ld_src = (long long)R * h->H;
          tr.out = rhT + (size_t)d * h->H * p.tb_ld * es;
          tr.ld_out = p.tb_ld;
          tr.C = h->H;
          kmap(tr);
          jobs.push_back(tr);
        }
      }
      for (size_t j = 0; j < jobs.size(); j += 4)
        RNN_TRY(dev(rnn_launch_transpose_batch(jobs.data() + j, (int)std::min<size_t>(4, jobs.size() - j), 0, bf, s)));
    }
    if (dw_fused(h, l)) {   // dW_ih | db_ih and dW_hh | db_hh: one launch of two same-shape products
      GemmParams g{};
      g.M = GH;
      g.N = h->H + 1;
      g.K = p.tb_k;
      g.A[0] = dgT;
      g.A[1] = dghT;
      g.B[0] = xT;
      g.B[1] = hT;
      g.lda = p.tb_ld;
      g.ldb = p.tb_ld;
      g.n_ones = h->H;
      g.C[0] = reinterpret_cast<float*>(dWb + h->off[1][RNN_W_IH][l]);
      g.C[1] = reinterpret_cast<float*>(dWb + h->off[1][RNN_W_HH][l]);
      g.ldc = h->H;
      g.cbias[0] = reinterpret_cast<float*>(dWb + h->off[1][RNN_B_IH][l]);
      g.cbias[1] = reinterpret_cast<float*>(dWb + h->off[1][RNN_B_HH][l]);
      g.a_vec = g.b_vec = 1;
      g.split_k = gemm_split(h, g.M, g.N, g.K, 2);
      g.partial = part;
      ProfScope ps(h, s, K_GEMM_DW);
      gemm_consts(h, g, ws, p.off_err);
      RNN_TRY(dev(rnn_launch_gemm(g, bf, EPI_DW, 2, s)));
      continue;
    }
    {  // dW_ih | db_ih = dG_i^T [X | 1]
      GemmParams g{};
      g.M = dgh;
      g.N = I_l + 1;
      g.K = p.tb_k;
      g.A[0] = dgT;
      g.lda = p.tb_ld;
      g.B[0] = xT;
      g.ldb = p.tb_ld;
      g.n_ones = I_l;
      g.C[0] = reinterpret_cast<float*>(dWb + h->off[1][RNN_W_IH][l]);
      g.ldc = I_l;
      g.cbias[0] = reinterpret_cast<float*>(dWb + h->off[1][RNN_B_IH][l]);
      g.a_vec = g.b_vec = 1;
      g.split_k = gemm_split(h, g.M, g.N, g.K, 1);
      g.partial = part;
      ProfScope ps(h, s, K_GEMM_DW);
      gemm_consts(h, g, ws, p.off_err);
      RNN_TRY(dev(rnn_launch_gemm(g, bf, EPI_DW, 1, s)));
    }
    // dW_hh | db_hh = dG_h^T [H_prev | 1], per direction; the flavours
    // whose n reads W_hn (r*h) take their n rows against (r*H_prev) instead
    const int parts = rhT ? 2 : 1;
    for (int part_i = 0; part_i < parts; ++part_i) {
      const int row0 = part_i == 0 ? 0 : 2 * h->H;
      const char* Bsrc = part_i == 0 ? hT : rhT;
      GemmParams g{};
      g.M = rhT ? (part_i == 0 ? 2 * h->H : h->H) : GH;
      g.N = h->H + 1;
      g.K = p.tb_k;
      g.lda = p.tb_ld;
      g.ldb = p.tb_ld;
      g.n_ones = h->H;
      g.ldc = h->H;
      for (int d = 0; d < h->D; ++d) {
        g.A[d] = dghT + ((size_t)d * GH + row0) * p.tb_ld * es;
        g.B[d] = Bsrc + (size_t)d * h->H * p.tb_ld * es;
        g.C[d] = reinterpret_cast<float*>(dWb + h->off[1][RNN_W_HH][l]) + ((size_t)d * GH + row0) * h->H;
        g.cbias[d] = reinterpret_cast<float*>(dWb + h->off[1][RNN_B_HH][l]) + (size_t)d * GH + row0;
      }
      g.a_vec = g.b_vec = 1;
      g.split_k = gemm_split(h, g.M, g.N, g.K, h->D);
      g.partial = part;
      ProfScope ps(h, s, K_GEMM_DW);
      gemm_consts(h, g, ws, p.off_err);
      RNN_TRY(dev(rnn_launch_gemm(g, bf, EPI_DW, h->D, s)));
    }
  }
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_forward_inference_static(rnn_handle_t h, void* stream, int T, int B, const float* x,
                                          const float* h0, const float* c0, const void* W, float* y,
                                          float* hy, float* cy) {
  if (!h || T < 0 || B < 0) return RNN_STATUS_INVALID_ARG;
  Plan p = make_plan(h, T, B, 0);
  if (p.status != RNN_STATUS_SUCCESS) return p.status;
  if (p.total > kStaticScratchBytes) return RNN_STATUS_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  RNN_TRY(static_scratch(&ws));
  // per-launch timing events are created on demand: kept off here
  const int prof = h->prof;
  h->prof = 0;
  const rnn_status_t st = forward_impl(h, stream, T, B, x, h0, c0, W, y, hy, cy, ws, kStaticScratchBytes, 0);
  h->prof = prof;
  return st;
}

size_t rnn_static_workspace_bytes(void) { return kStaticScratchBytes; }

rnn_status_t rnn_exchange_floor(rnn_handle_t h, void* stream, int T, int B, int training, void* ws,
                                size_t ws_bytes) {
  return exchange_probe_impl(h, stream, T, B, training, ws, ws_bytes);
}

rnn_status_t rnn_bf16_rounding_check(void* stream, unsigned long long first, unsigned long long count,
                                     unsigned long long* mismatches) {
  if (!mismatches || count > (1ull << 32) || first >= (1ull << 32) || first + count > (1ull << 32))
    return RNN_STATUS_INVALID_ARG;
  if (count == 0) return RNN_STATUS_SUCCESS;
  return dev(rnn_launch_bf16_round_check(first, count, mismatches, reinterpret_cast<hipStream_t>(stream)));
}

rnn_status_t rnn_mfma_peak_probe(void* stream, int kind, int blocks, int iters, float* out) {
  if (kind < 0 || kind > 2 || blocks <= 0 || iters <= 0 || !out) return RNN_STATUS_INVALID_ARG;
  return dev(rnn_launch_mfma_peak(kind, blocks, iters, out, reinterpret_cast<hipStream_t>(stream)));
}

rnn_status_t rnn_device_status(rnn_handle_t h, void* stream, const void* ws, size_t ws_bytes) {
  if (!h || !ws || ws_bytes < 256) return RNN_STATUS_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return RNN_STATUS_DEVICE;
  unsigned err = 0;
  if (hipMemcpy(&err, ws, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return RNN_STATUS_DEVICE;
  return err ? RNN_STATUS_DEVICE_TIMEOUT : RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_set_profiling(rnn_handle_t h, int enable) {
  if (!h) return RNN_STATUS_INVALID_ARG;
  prof_collect(h);
  h->prof = enable ? 1 : 0;
  for (int k = 0; k < K_NKERNELS; ++k) {
    h->prof_n[k] = 0;
    h->prof_ms[k] = 0.0;
  }
  return RNN_STATUS_SUCCESS;
}

rnn_status_t rnn_profile_read(rnn_handle_t h, int kernel, long long* launches, double* total_ms) {
  if (!h || kernel < 0 || kernel >= K_NKERNELS || !launches || !total_ms) return RNN_STATUS_INVALID_ARG;
  prof_collect(h);
  *launches = h->prof_n[kernel];
  *total_ms = h->prof_ms[kernel];
  return RNN_STATUS_SUCCESS;
}

const char* rnn_status_string(rnn_status_t s) {
  switch (s) {
    case RNN_STATUS_SUCCESS: return "success";
    case RNN_STATUS_INVALID_ARG: return "invalid argument";
    case RNN_STATUS_UNSUPPORTED: return "unsupported configuration";
    case RNN_STATUS_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RNN_STATUS_BAD_CALL_ORDER: return "bad call order (backward needs the matching forward_training)";
    case RNN_STATUS_NOT_CORESIDENT: return "persistent schedule cannot keep every workgroup resident";
    case RNN_STATUS_DEVICE: return "HIP runtime error";
    case RNN_STATUS_DEVICE_TIMEOUT: return "bounded device wait expired";
    default: return "unknown status";
  }
}

}  // extern "C"
