// C-ABI entry points of the stacked-LSTM forward library (host side).
//
// lstm_fwd validates its arguments, asks the planner for a schedule, carves
// the caller's workspace and enqueues the kernels on the caller's stream:
//   1. the grouped input-projection GEMM of layer 0 over all timesteps (it
//      also zeroes the error word and the step counters in the workspace);
//   2. LAYERWISE: per layer, the persistent recurrence, then the next layer's
//      input GEMM;  WAVEFRONT: one persistent launch that runs every layer.
// Nothing here synchronises the host.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "lstm_bwd.h"  // include/ is on the include path
#include "lstm_fwd.h"
#include "lstm_params.h"
#include "lstm_plan.h"

namespace lstm {
hipError_t launch_input_gemm(bool bf16, const GemmParams& p, hipStream_t s);
hipError_t rec_prepare(bool bf16, bool stream, bool vec, bool frag, int nwv, int mw, int nw, int lds_bytes,
                       int* max_blocks_per_cu);
hipError_t launch_clear(int* p, long long n, hipStream_t s);
hipError_t launch_rec(bool bf16, bool stream, bool vec, bool frag, int nwv, const RecParams& p, int lds_bytes,
                      bool plain, hipStream_t s);
hipError_t res_prepare(bool bf16, int mw, int nw, int nci, int nrb, bool save, int lds_bytes, int* max_blocks_per_cu);
hipError_t launch_rec_res(bool bf16, int nci, int nrb, const RecParams& p, int lds_bytes, bool plain, hipStream_t s);
hipError_t launch_h0_frag(bool bf16, const void* h0, void* dst, int B, int H, long long tile_elems, hipStream_t s);
}  // namespace lstm

using namespace lstm;

namespace {

constexpr int kMaxDevices = 64;
constexpr long long kDefaultTimeoutUs = 2000000;  // 2 s per step wait

struct DevCache {
  bool ready = false;
  DeviceInfo info;
  long long clock_khz = 100000;  // wall clock (s_memrealtime) rate
};
DevCache g_dev[kMaxDevices];
std::mutex g_dev_mu;

lstm_status_t device_info(DevCache* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LSTM_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevCache& c = g_dev[dev];
  if (!c.ready) {
    int cus = 0, lds = 0, clk = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return LSTM_ERR_HIP;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return LSTM_ERR_HIP;
    if (hipDeviceGetAttribute(&clk, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return LSTM_ERR_HIP;
    c.info.num_cus = cus;
    c.info.lds_per_block = lds;
    c.clock_khz = clk > 0 ? clk : 100000;
    c.ready = true;
  }
  *out = c;
  return LSTM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

lstm_status_t validate(const lstm_desc_t* d, const void* x, const void* W, const void* R, const void* b,
                       const void* y, const void* ws) {
  if (!d) return LSTM_ERR_INVALID_ARG;
  if (d->L < 1 || d->I < 1 || d->H < 1 || d->B < 1 || d->T < 1) return LSTM_ERR_INVALID_ARG;
  if (d->dtype != LSTM_F32 && d->dtype != LSTM_BF16) return LSTM_ERR_INVALID_ARG;
  if (d->cell < LSTM_CELL_LSTM || d->cell > LSTM_CELL_RNN_RELU) return LSTM_ERR_INVALID_ARG;
  if (!x || !W || !R || !b || !y) return LSTM_ERR_INVALID_ARG;
  if (!ws) return LSTM_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return LSTM_ERR_WORKSPACE;
  return LSTM_OK;
}

}  // namespace

extern "C" {

const char* lstm_status_string(lstm_status_t s) {
  switch (s) {
    case LSTM_OK: return "LSTM_OK";
    case LSTM_ERR_INVALID_ARG: return "LSTM_ERR_INVALID_ARG";
    case LSTM_ERR_UNSUPPORTED: return "LSTM_ERR_UNSUPPORTED";
    case LSTM_ERR_WORKSPACE: return "LSTM_ERR_WORKSPACE";
    case LSTM_ERR_HIP: return "LSTM_ERR_HIP";
    case LSTM_ERR_BARRIER_TIMEOUT: return "LSTM_ERR_BARRIER_TIMEOUT";
  }
  return "LSTM_ERR_UNKNOWN";
}

lstm_status_t lstm_fwd_plan(const lstm_desc_t* d, int32_t force_regime, int32_t num_cus, int32_t lds_per_cu,
                            lstm_plan_info_t* out) {
  if (!d || !out) return LSTM_ERR_INVALID_ARG;
  DeviceInfo info;
  if (num_cus > 0) {
    info.num_cus = num_cus;
    info.lds_per_block = lds_per_cu > 0 ? lds_per_cu : 160 * 1024;
  } else {
    DevCache c;
    lstm_status_t st = device_info(&c);
    if (st != LSTM_OK) return st;
    info = c.info;
  }
  Plan p;
  const int rc = make_plan(d->L, d->I, d->H, d->B, d->T, d->dtype, d->cell, force_regime, info, &p);
  if (rc) return (lstm_status_t)rc;
  *out = lstm_plan_info_t();
  out->regime = p.regime;
  out->num_launches = p.num_launches;
  out->grid = p.rec[0].grid;
  out->block = 64 * p.rec[0].nwaves;
  out->lds_bytes = p.rec[0].lds_bytes;
  out->ksplit = p.rec[0].ks;
  int on_chip = 1;
  for (int r = 0; r < p.nrec; ++r)
    for (int k = 0; k < p.rec[r].nlayers; ++k) on_chip &= p.rec[r].layers[k].staged;
  out->weights_on_chip = on_chip;
  out->layers_per_launch = p.rec[0].nlayers;
  for (int k = 0; k < p.rec[0].nlayers && k < 16; ++k) {
    out->wg_per_layer[k] = p.rec[0].layers[k].wg_count;
    out->mtiles_per_wg[k] = p.rec[0].layers[k].mt_per_wg;
  }
  out->tile_groups_m = p.rec[0].ntgm;
  out->tile_groups_n = p.rec[0].ntgn;
  out->wave_tiles_m = p.rec[0].mw;
  out->wave_tiles_n = p.rec[0].nw;
  out->weights_streamed = p.rec[0].stream;
  out->input_gemms = p.ngemm;
  out->weight_blocks_in_registers = p.rec[0].res_nrb;
  const int dv_lds = data_valid_lds(p, p.rec[0], d->H, d->B, info);
  out->data_valid_exchange = dv_lds > 0 ? 1 : 0;
  if (dv_lds > 0) out->lds_bytes = dv_lds;  // two reduction areas
  return LSTM_OK;
}

size_t lstm_fwd_workspace_size(const lstm_desc_t* d) {
  if (!d) return 0;
  // the layout does not depend on the device; any partition fits the same buffers
  DeviceInfo info;
  Plan p;
  if (make_plan(d->L, d->I, d->H, d->B, d->T, d->dtype, d->cell, LSTM_REGIME_LAYERWISE, info, &p)) return 0;
  return p.ws_bytes;
}

lstm_status_t lstm_fwd_validate(const lstm_desc_t* d, const void* x, const void* W, const void* R, const void* b,
                                const void* y, const void* ws, size_t ws_bytes) {
  lstm_status_t st = validate(d, x, W, R, b, y, ws);
  if (st != LSTM_OK) return st;
  const size_t need = lstm_fwd_workspace_size(d);
  if (need == 0) return LSTM_ERR_UNSUPPORTED;
  if (ws_bytes < need) return LSTM_ERR_WORKSPACE;
  return LSTM_OK;
}

lstm_status_t lstm_fwd_last_error(const void* ws, hipStream_t stream) {
  if (!ws) return LSTM_ERR_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return LSTM_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return LSTM_ERR_HIP;
  return v == 0 ? LSTM_OK : LSTM_ERR_BARRIER_TIMEOUT;
}

}  // extern "C"

namespace {

// The forward pass.  `reserve` (training forward, LSTM only) receives every
// layer's activated gates, cell states and hidden states (lstm_bwd.h layout).
lstm_status_t fwd_impl(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                       const void* R, const void* b, void* y, void* hT, float* cT, void* ws, hipStream_t stream,
                       const lstm_fwd_opts_t* opts, void* reserve) {
  lstm_status_t st = validate(d, x, W, R, b, y, ws);
  if (st != LSTM_OK) return st;
  if (reserve && d->cell != LSTM_CELL_LSTM) return LSTM_ERR_UNSUPPORTED;
  DevCache dev;
  st = device_info(&dev);
  if (st != LSTM_OK) return st;
  const int force = opts ? opts->force_regime : LSTM_REGIME_AUTO;
  Plan p;
  const int rc = make_plan(d->L, d->I, d->H, d->B, d->T, d->dtype, d->cell, force, dev.info, &p,
                           aligned16(R) && (!h0 || aligned16(h0)));
  if (rc) return (lstm_status_t)rc;

  const int L = d->L, I = d->I, H = d->H, B = d->B, T = d->T;
  const bool bf16 = p.bf16;
  const size_t ds = p.dsize;
  char* wsb = static_cast<char*>(ws);
  int* err = reinterpret_cast<int*>(wsb + p.err_off);
  int* flags = reinterpret_cast<int*>(wsb + p.flags_off);
  float* G = reinterpret_cast<float*>(wsb + p.G_off);
  char* hist = wsb + p.hist_off;
  const size_t slot = p.slot_elems;  // elements between two steps of an exchange buffer
  const char* Wb = static_cast<const char*>(W);
  const char* Rb = static_cast<const char*>(R);
  const char* bb = static_cast<const char*>(b);
  const size_t ng = p.gates, nbias = p.bias_rows;  // row blocks of W/R and of b
  auto W_l = [&](int l) -> const void* {
    return l == 0 ? Wb : Wb + (ng * H * I + (size_t)(l - 1) * ng * H * H) * ds;
  };
  auto R_l = [&](int l) -> const void* { return Rb + (size_t)l * ng * H * H * ds; };
  auto b_l = [&](int l) -> const void* { return bb + (size_t)l * nbias * H * ds; };
  if (p.cell != LSTM_CELL_LSTM) c0 = nullptr, cT = nullptr;  // no cell state
  auto xbuf = [&](int l) -> void* {  // layer l's exchange buffer: T slots of [B][H]
    return static_cast<void*>(hist + (size_t)l * T * slot * ds);
  };
  auto state = [&](const void* base, int l, size_t esz) -> const void* {
    return base ? static_cast<const char*>(base) + (size_t)l * B * H * esz : nullptr;
  };

  long long timeout_us = (opts && opts->wait_timeout_us > 0) ? opts->wait_timeout_us : kDefaultTimeoutUs;
  if (opts && opts->wait_timeout_us < 0) timeout_us = 0;  // forces every blocked wait to fail (tests)
  const long long timeout_ticks = timeout_us * dev.clock_khz / 1000;

  int nl = 0;
  const int maxl = (opts && opts->max_launches > 0) ? opts->max_launches : 0;
  auto before = [&](int kind) {
    if (nl < maxl) {
      if (opts->launch_kind) opts->launch_kind[nl] = kind;
      if (opts->ev_start && hipEventRecord(opts->ev_start[nl], stream) != hipSuccess) return false;
    }
    return true;
  };
  auto after = [&]() {
    if (nl < maxl && opts->ev_stop && hipEventRecord(opts->ev_stop[nl], stream) != hipSuccess) return false;
    ++nl;
    return true;
  };

  auto gemm = [&](int l, const void* U, long long u_slot, int K, bool zero, void* fill) -> lstm_status_t {
    GemmParams gp{};  // C = null: the forward's G layout
    gp.W = W_l(l);
    gp.U = U;
    gp.u_slot = u_slot;
    gp.bias = b_l(l);
    gp.G = G;
    gp.zero_ptr = zero ? reinterpret_cast<int*>(wsb) : nullptr;
    gp.zero_count = zero ? (int)p.zero_ints : 0;
    gp.fill_ptr = static_cast<unsigned*>(fill);
    gp.fill_count = fill ? (long long)((size_t)T * slot * ds / 4) : 0;
    gp.K = K;
    gp.H = H;
    gp.Mt = p.Mt;
    gp.B = B;
    gp.N = T * B;
    gp.vec_ok_w = aligned16(gp.W) && ((size_t)K * ds) % 16 == 0;
    gp.vec_ok_u = aligned16(U) && ((size_t)K * ds) % 16 == 0 && ((size_t)u_slot * ds) % 16 == 0;
    gp.cell = p.cell;
    gp.num_cus = dev.info.num_cus;
    if (!before(LSTM_KERNEL_INPUT_GEMM)) return LSTM_ERR_HIP;
    if (launch_input_gemm(bf16, gp, stream) != hipSuccess) return LSTM_ERR_HIP;
    if (!after()) return LSTM_ERR_HIP;
    return LSTM_OK;
  };

  // 16-byte loads allowed for every operand row of layer pl (the aligned path)
  auto layer_vec = [&](const LayerPlan& pl) -> bool {
    const int l = pl.layer;
    const void* Wl = pl.hoisted ? nullptr : W_l(l);
    const void* Ul = pl.hoisted ? nullptr : (l == 0 ? x : static_cast<const void*>(xbuf(l - 1)));
    const long long us = pl.hoisted ? 0 : (l == 0 ? (long long)B * I : (long long)slot);
    return ((size_t)H * ds) % 16 == 0 && aligned16(R_l(l)) && aligned16(xbuf(l)) && (!Wl || aligned16(Wl)) &&
           (!Ul || aligned16(Ul)) && (!state(h0, l, ds) || aligned16(state(h0, l, ds))) && (pl.Kin % p.KC) == 0 &&
           ((size_t)us * ds) % 16 == 0;
  };
  auto launch_vec = [&](const LaunchPlan& lp) -> bool {
    bool v = (H % p.KC) == 0;
    for (int k = 0; k < lp.nlayers; ++k) v = v && layer_vec(lp.layers[k]);
    return v;
  };
  // Wavefront launches read each other's exchange buffers (the first layer of
  // a launch reads the last layer of the one before), so they use the
  // load-order exchange only if every one of them is on the aligned path.
  bool wave_vec = true;
  if (p.regime == LSTM_REGIME_WAVEFRONT)
    for (int r = 0; r < p.nrec; ++r) wave_vec = wave_vec && launch_vec(p.rec[r]);

  // Data-valid exchange (lstm_rec.h, data_valid_lds in lstm_plan.h) when the
  // launch's buffers allow it: its LDS bytes, or 0.
  auto sent_lds = [&](const LaunchPlan& lp) -> int {
    const int need = data_valid_lds(p, lp, H, B, dev.info);
    return (need && launch_vec(lp) && (size_t)slot * ds < (1u << 31)) ? need : 0;
  };

  // Every recurrent launch is prepared -- parameters, kernel variant, LDS
  // limit, co-residency -- before the first kernel is enqueued, so a refusal
  // (LSTM_ERR_UNSUPPORTED, LSTM_ERR_HIP) leaves nothing queued.
  struct RecLaunch {
    RecParams rp;
    int lds = 0;
    bool vec = false, frag = false, res = false;
    const LaunchPlan* lp = nullptr;
  };
  std::vector<RecLaunch> launches(p.nrec);
  bool traced = false;  // only the first recurrent launch is traced
  auto rec_prepare_launch = [&](const LaunchPlan& lp, RecLaunch& out) -> lstm_status_t {
    RecParams& rp = out.rp;
    rp.nlayers = lp.nlayers;
    rp.slot = (long long)slot;
    rp.fslot = (long long)slot;
    rp.T = T, rp.B = B, rp.H = H, rp.Mt = p.Mt, rp.ncnt = p.ncnt;
    rp.cell = p.cell;
    rp.ks = lp.ks;
    rp.ntgm = lp.ntgm, rp.ntgn = lp.ntgn, rp.mw = lp.mw, rp.nw = lp.nw;
    rp.red_off = lp.red_off;
    rp.grid = lp.grid;
    rp.xcd_remap = (lp.grid % 8) == 0 ? 1 : 0;
    rp.err = err;
    rp.timeout_ticks = timeout_ticks;
    const bool tr = opts && opts->trace && opts->trace_wgs > 0 && !traced;
    rp.trace = tr ? reinterpret_cast<long long*>(opts->trace) : nullptr;
    rp.trace_wgs = tr ? opts->trace_wgs : 0;
    rp.trace_stride = (tr && opts->trace_stride > 0) ? opts->trace_stride : 1;
    traced = traced || tr;
    int lds = lp.lds_bytes;
    rp.sent = 0, rp.red_stride = 0;
    if (const int need = sent_lds(lp)) {
      rp.sent = 1, rp.red_stride = ((lp.lds_bytes - lp.red_off) + 255) & ~255;
      lds = need;
    }
    for (int k = 0; k < lp.nlayers; ++k) {
      const LayerPlan& pl = lp.layers[k];
      const int l = pl.layer;
      RecLayer& r = rp.layer[k];
      r.W = pl.hoisted ? nullptr : W_l(l);
      r.R = R_l(l);
      r.bias = b_l(l);
      r.G = pl.hoisted ? G : nullptr;
      r.U = pl.hoisted ? nullptr : (l == 0 ? x : xbuf(l - 1));
      r.u_slot = pl.hoisted ? 0 : (l == 0 ? (long long)B * I : (long long)slot);
      r.X = xbuf(l);
      r.F = nullptr;
      r.ufrag = 0;
      r.Yout = (l == L - 1) ? y : nullptr;
      r.h0 = state(h0, l, ds);
      r.c0 = static_cast<const float*>(state(c0, l, sizeof(float)));
      r.hT = hT ? static_cast<char*>(hT) + (size_t)l * B * H * ds : nullptr;
      r.cT = cT ? cT + (size_t)l * B * H : nullptr;
      r.flags = flags + (size_t)l * kFlagsPerLayer * kFlagStride;
      const bool dep_here = !pl.hoisted && k > 0;
      r.dep_flags = dep_here ? flags + (size_t)(l - 1) * kFlagsPerLayer * kFlagStride : nullptr;
      r.dep_count = dep_here ? lp.layers[k - 1].wg_count : 0;
      r.Kin = pl.Kin;
      r.wg_begin = pl.wg_begin;
      r.wg_count = pl.wg_count;
      r.mt_per_wg = pl.mt_per_wg;
      r.staged = pl.staged;
      r.vec_ok = layer_vec(pl) ? 1 : 0;
      r.save_gates = nullptr, r.save_c = nullptr, r.save_h = nullptr;
      if (reserve) {
        const size_t tbh = (size_t)T * B * H;
        char* rb = static_cast<char*>(reserve);
        r.save_gates = reinterpret_cast<float*>(rb + (size_t)l * tbh * 16);
        r.save_c = reinterpret_cast<float*>(rb + (size_t)L * tbh * 16 + (size_t)l * tbh * 4);
        r.save_h = static_cast<void*>(rb + (size_t)L * tbh * 20 + (size_t)l * tbh * ds);
      }
    }
    for (int k = lp.nlayers; k < kMaxLayersPerLaunch; ++k) rp.layer[k] = RecLayer();
    // aligned fast path: whole chunks and 16-byte aligned rows in every layer of the launch
    const bool vec = launch_vec(lp);
    // On the aligned path h_t is exchanged in load order when the batch fills
    // at least one 16-column tile (below that a load-order read would fetch
    // mostly padding; the register-resident kernel always uses it).
    // Wavefront: each layer's exchange buffer holds it (read by the layer
    // itself and, as its fused input, by the layer above).  Layerwise: the
    // one-layer load-order region holds it, and the row-major slots keep a
    // copy for the next layer's input GEMM (none for the top layer, whose
    // copy is y).
    const bool frag = vec && (p.regime != LSTM_REGIME_WAVEFRONT || wave_vec) && (B >= 16 || lp.res_nrb > 0);
    if (frag) {
      for (int k = 0; k < lp.nlayers; ++k) {
        RecLayer& r = rp.layer[k];
        const LayerPlan& pl = lp.layers[k];
        const int l = pl.layer;
        if (p.regime == LSTM_REGIME_WAVEFRONT) {
          r.F = xbuf(l);
          r.X = nullptr;
          if (!pl.hoisted && l > 0) r.ufrag = 1;  // U = xbuf(l - 1), now in load order
        } else {
          r.F = static_cast<void*>(wsb + p.xf_off);
          r.X = (l < L - 1) ? xbuf(l) : nullptr;
        }
      }
    }
    int per_cu = 0;
    const bool res = lp.res_nrb > 0;
    if (res && !vec) return LSTM_ERR_UNSUPPORTED;  // planned only for aligned rows
    hipError_t pe = res ? res_prepare(bf16, lp.mw, lp.nw, lp.res_nci, lp.res_nrb, reserve != nullptr, lp.lds_bytes, &per_cu)
                        : rec_prepare(bf16, lp.stream, vec, frag, lp.nwaves, lp.mw, lp.nw, lds, &per_cu);
    if (pe == hipSuccess && rp.sent && (long long)per_cu * dev.info.num_cus < lp.grid) {
      // the second reduction area costs co-residency: step counters instead
      // (the filled slots are then simply overwritten)
      rp.sent = 0, rp.red_stride = 0, lds = lp.lds_bytes;
      pe = rec_prepare(bf16, lp.stream, vec, frag, lp.nwaves, lp.mw, lp.nw, lds, &per_cu);
    }
    if (pe != hipSuccess) return LSTM_ERR_HIP;
    if ((long long)per_cu * dev.info.num_cus < lp.grid) return LSTM_ERR_UNSUPPORTED;  // not co-resident
    out.lds = lds, out.vec = vec, out.frag = frag, out.res = res, out.lp = &lp;
    return LSTM_OK;
  };
  for (int r = 0; r < p.nrec; ++r) {
    st = rec_prepare_launch(p.rec[r], launches[r]);
    if (st != LSTM_OK) return st;
  }
  auto rec = [&](const RecLaunch& rl) -> lstm_status_t {
    const LaunchPlan& lp = *rl.lp;
    if (!before(LSTM_KERNEL_RECURRENT)) return LSTM_ERR_HIP;
    // the register-resident kernel reads h_{t-1} from load-order slot t: h0
    // goes to slot 0 first (counted as part of the recurrence)
    if (rl.res && rl.rp.layer[0].h0 &&
        launch_h0_frag(bf16, rl.rp.layer[0].h0, rl.rp.layer[0].F, B, H, (long long)(H / p.KC) * (2048 / (long long)ds),
                       stream) != hipSuccess)
      return LSTM_ERR_HIP;
    const bool plain = opts && opts->plain_launch;
    const hipError_t le = rl.res ? launch_rec_res(bf16, lp.res_nci, lp.res_nrb, rl.rp, lp.lds_bytes, plain, stream)
                                 : launch_rec(bf16, lp.stream, rl.vec, rl.frag, lp.nwaves, rl.rp, rl.lds, plain, stream);
    if (le != hipSuccess) return LSTM_ERR_HIP;
    if (!after()) return LSTM_ERR_HIP;
    return LSTM_OK;
  };
  // the data-valid exchange of launch r (its slots are filled by the input GEMM before it)
  auto sent_of = [&](int r) -> bool { return launches[r].rp.sent != 0; };

  if (p.ngemm > 0) {
    // layer 0 input projection (+ zeroing of the error word and step counters)
    st = gemm(0, x, (long long)B * I, I, true, (p.regime != LSTM_REGIME_WAVEFRONT && sent_of(0)) ? xbuf(0) : nullptr);
    if (st != LSTM_OK) return st;
  } else {
    // every input product is fused into the steps: only the counters need clearing
    if (!before(LSTM_KERNEL_CLEAR)) return LSTM_ERR_HIP;
    if (launch_clear(reinterpret_cast<int*>(wsb), (long long)p.zero_ints, stream) != hipSuccess) return LSTM_ERR_HIP;
    if (!after()) return LSTM_ERR_HIP;
  }
  if (p.regime == LSTM_REGIME_WAVEFRONT) {
    for (int r = 0; r < p.nrec; ++r) {
      st = rec(launches[r]);
      if (st != LSTM_OK) return st;
    }
  } else {
    for (int l = 0; l < L; ++l) {
      if (l > 0) {
        st = gemm(l, xbuf(l - 1), (long long)slot, H, false, sent_of(l) ? xbuf(l) : nullptr);
        if (st != LSTM_OK) return st;
      }
      st = rec(launches[l]);
      if (st != LSTM_OK) return st;
    }
  }
  if (opts && opts->num_launches) *opts->num_launches = nl;
  return LSTM_OK;
}

}  // namespace

extern "C" {

lstm_status_t lstm_fwd_ex(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                          const void* R, const void* b, void* y, void* hT, float* cT, void* ws, hipStream_t stream,
                          const lstm_fwd_opts_t* opts) {
  return fwd_impl(d, x, h0, c0, W, R, b, y, hT, cT, ws, stream, opts, nullptr);
}

size_t lstm_train_reserve_size(const lstm_desc_t* d) {
  if (!d || d->cell != LSTM_CELL_LSTM || lstm_fwd_workspace_size(d) == 0) return 0;
  const size_t tbh = (size_t)d->L * d->T * d->B * d->H;
  return (tbh * (16 + 4 + (d->dtype == LSTM_BF16 ? 2 : 4)) + 255) & ~(size_t)255;
}

lstm_status_t lstm_fwd_train_ex(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                                const void* R, const void* b, void* y, void* hT, float* cT, void* reserve, void* ws,
                                hipStream_t stream, const lstm_fwd_opts_t* opts) {
  if (!reserve) return LSTM_ERR_INVALID_ARG;
  return fwd_impl(d, x, h0, c0, W, R, b, y, hT, cT, ws, stream, opts, reserve);
}

lstm_status_t lstm_fwd_train(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                             const void* R, const void* b, void* y, void* hT, float* cT, void* reserve, void* ws,
                             hipStream_t stream) {
  return lstm_fwd_train_ex(d, x, h0, c0, W, R, b, y, hT, cT, reserve, ws, stream, nullptr);
}

lstm_status_t lstm_fwd(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                       const void* R, const void* b, void* y, void* hT, float* cT, void* ws, hipStream_t stream) {
  return lstm_fwd_ex(d, x, h0, c0, W, R, b, y, hT, cT, ws, stream, nullptr);
}

}  // extern "C"
