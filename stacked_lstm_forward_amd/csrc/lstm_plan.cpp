// Host planner of the stacked-LSTM forward pass (pure C++, no HIP calls).
//
// Two schedules:
//   LAYERWISE  per layer: one input GEMM over all T*B columns, then one
//              persistent recurrent launch for that layer.  Used when the
//              layers' weights cannot all stay on chip at once (large H) or L = 1.
//   WAVEFRONT  one input GEMM for layer 0, then one persistent launch in which
//              every layer owns its own workgroups and its own weight rows in
//              LDS; layer l+1 fuses its input product W_{l+1} h^l_t into the
//              step and starts step t as soon as layer l has published it.
// The wavefront is the network-level overlap of layers ("Optimizing
// Performance of Recurrent Neural Networks on GPUs", proposed method and key
// results on layer overlap); keeping each workgroup's rows in LDS across all
// steps is the persistent-kernel idea ("Persistent RNNs").  The per-layer
// workgroup partition plays the role of the pages' hand-tuned kernel choice
// under concurrency: each concurrently running layer gets a share of the CUs
// sized to its work instead of the whole GPU.
#include "lstm_plan.h"

#include <algorithm>

namespace lstm {

namespace {

constexpr int kStatusOk = 0, kInvalid = 1, kUnsupported = 2;
constexpr int kRegimeAuto = 0, kRegimeLayerwise = 1, kRegimeWavefront = 2;
constexpr int kFragBytes = 32;  // one lane's fragment
constexpr int kLdsReserve = 256;  // static LDS of the kernel

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// Choose the K split and the tile groups of a launch whose largest workgroup
// owns `mmax` M-tiles; fills ks/ntgm/ntgn/mw/nw/red_off/lds_bytes.  `staged_bytes`
// is the LDS the weight rows need (0 when streamed); `nch` the K chunks of the
// longest tile row.  Returns false if nothing fits.
//
// 8-wave launches take the widest split that still leaves every wave at
// least kMinChunksPerWave chunks (else the widest that fits): the split's
// combine costs a barrier that waits for the slowest wave, which a wave with
// only a chunk or two does not pay back.  Measured on the 8-layer bf16
// H = 256, B = 64 stack (8 chunks): 4-way 0.848 ms, 2-way 0.802, 1-way 1.133;
// the 4-layer fp32 H = 512 stack (32 chunks) is fastest 4-way.
constexpr int kMinChunksPerWave = 4;

bool choose_split(int mmax, int ncnt, int nch, int staged_bytes, int lds_limit, int nwaves, LaunchPlan* lp) {
  static const int ks_order[4] = {8, 4, 2, 1};
  LaunchPlan widest;
  bool have_widest = false;
  // prefer at most 4 tiles per wave, fall back to 8, then 16; with two waves
  // per SIMD a wave has 256 registers and larger tile sets spill, so 8-wave
  // workgroups take 4 at most
  const int npass = nwaves == 8 ? 1 : 3;
  for (int pass = 0; pass < npass; ++pass) {
    const int tile_cap = pass == 0 ? 4 : (pass == 1 ? 8 : 16);
    for (int ks : ks_order) {
      if (ks > nwaves) continue;
      const int ntg = nwaves / ks;
      int best_ntgm = -1, best_cost = 1 << 30;
      for (int ntgm = 1; ntgm <= ntg; ntgm *= 2) {
        const int ntgn = ntg / ntgm;
        const int mw = cdiv(mmax, ntgm), nw = cdiv(ncnt, ntgn);
        if (mw > 4 || nw > 4 || mw * nw > tile_cap) continue;
        if (ntgm > mmax || ntgn > ncnt) continue;  // a tile group with nothing to do
        // re-read cost: tile groups that share column tiles each read those
        // activations from global memory (x ntgm); tile groups that share M-tiles
        // each read those weight rows, from LDS when staged (cheap) or from
        // global memory when streamed (x ntgn)
        const int w_act = 4, w_wgt = staged_bytes > 0 ? 1 : 4;
        const int cost = w_act * ntgm * ncnt + w_wgt * ntgn * mmax;
        if (cost < best_cost) best_cost = cost, best_ntgm = ntgm;
      }
      if (best_ntgm < 0) continue;
      const int ntgm = best_ntgm, ntgn = ntg / ntgm;
      const int mw = cdiv(mmax, ntgm), nw = cdiv(ncnt, ntgn);
      // one 1 KiB partial per (tile, non-finalising K-group)
      const int red = ks > 1 ? ntg * mw * nw * (ks - 1) * 64 * 16 : 0;
      const int red_off = (staged_bytes + 255) & ~255;
      if (red_off + red + kLdsReserve > lds_limit) continue;
      LaunchPlan c = *lp;
      c.nwaves = nwaves;
      c.ks = ks, c.ntgm = ntgm, c.ntgn = ntgn, c.mw = mw, c.nw = nw;
      c.red_off = red_off;
      c.lds_bytes = red_off + red;
      if (nwaves != 8 || cdiv(nch, ks) >= kMinChunksPerWave) {
        *lp = c;
        return true;
      }
      if (!have_widest) widest = c, have_widest = true;
    }
    if (have_widest) {
      *lp = widest;
      return true;
    }
  }
  return false;
}

int round_grid(int g) { return (g + 7) & ~7; }

// Register-resident launch of one layer: the weight rows stay on chip, split
// between the registers and the LDS of each workgroup.  Only the shapes the
// kernel is instantiated for (kResShape): the workgroup's M-tiles, 4 K-groups
// of exactly nci chunks each, at most kResMaxNW 16-column batch tiles.
// Returns the entry of kResShape, or -1.
int resident_shape(bool bf16, int m, int nch, int ncnt) {
  if (ncnt > kResMaxNW) return -1;
  for (int k = 0; k < kResShapes; ++k) {
    const ResShape& r = kResShape[k];
    if ((r.bf16 != 0) == bf16 && r.mw == m && 4 * r.nci == nch) return k;
  }
  return -1;
}

bool plan_resident(int m, int nch, int ncnt, bool bf16, bool aligned, const DeviceInfo& dev, LaunchPlan* lp) {
  const int k = aligned ? resident_shape(bf16, m, nch, ncnt) : -1;
  if (k < 0) return false;
  const ResShape& r = kResShape[k];
  const int nlb = r.mw * r.nci - r.nrb;  // LDS blocks per wave
  const int red = r.mw * 4 * 64 * 16;    // one 1 KiB partial per (M-tile, K-group)
  const int red_off = 4 * nlb * 64 * kFragBytes;
  if (red_off + red + kLdsReserve > dev.lds_per_block) return false;
  lp->res_nrb = r.nrb, lp->res_nci = r.nci;
  lp->nwaves = 4, lp->ks = 4, lp->ntgm = 1, lp->ntgn = 1, lp->mw = r.mw, lp->nw = ncnt;
  lp->red_off = red_off, lp->lds_bytes = red_off + red;
  lp->stream = 0;
  return true;
}

// Single-layer persistent launch (hoisted input).
bool plan_single(int layer, int Mt, int nch, int ncnt, bool bf16, bool aligned, const DeviceInfo& dev,
                 LaunchPlan* lp) {
  const int gmax = dev.num_cus;
  int m = std::max(1, cdiv(Mt, gmax));
  if (m > 16) return false;
  const int wgs = cdiv(Mt, m);
  LayerPlan& L = lp->layers[0];
  L = LayerPlan();
  L.layer = layer, L.hoisted = 1, L.Kin = 0, L.nch = nch;
  L.wg_begin = 0, L.wg_count = wgs, L.mt_per_wg = m;
  lp->nlayers = 1;
  const int staged_bytes = m * nch * 64 * kFragBytes;
  // one wave per SIMD: a single layer's waves are not limited by a layer below
  if (choose_split(m, ncnt, nch, staged_bytes, dev.lds_per_block, 4, lp)) {
    L.staged = 1;
    lp->stream = 0;
  } else if (plan_resident(m, nch, ncnt, bf16, aligned, dev, lp)) {
    L.staged = 1;
  } else if (choose_split(m, ncnt, nch, 0, dev.lds_per_block, 4, lp)) {
    L.staged = 0;
    lp->stream = 1;
  } else {
    return false;
  }
  lp->grid = round_grid(wgs);
  return wgs <= kFlagsPerLayer && lp->grid <= std::max(gmax, 8);
}

// Wavefront launch over layers [l0, l0+n).  Layers >= 1 fuse their input
// product; layer 0 fuses it too when fuse0 (K = I + H), else its input is
// hoisted into the input GEMM.
bool plan_wavefront(int l0, int n, int Mt, int nch_h, int nch_x, int I, int H, bool fuse0, int ncnt,
                    const DeviceInfo& dev, LaunchPlan* lp) {
  const int gmax = dev.num_cus;
  int nchl[kMaxLayersPerLaunch];
  for (int k = 0; k < n; ++k) {
    const int l = l0 + k;
    // fused layers: input chunks + recurrent chunks
    nchl[k] = (l == 0) ? (fuse0 ? nch_x + nch_h : nch_h) : nch_h + nch_h;
  }
  // smallest per-workgroup budget (chunks x M-tiles) whose partition fits the grid
  int best_budget = -1;
  int budgets[kMaxLayersPerLaunch * 16];
  int nb = 0;
  for (int k = 0; k < n; ++k)
    for (int m = 1; m <= 16; ++m) budgets[nb++] = m * nchl[k];
  std::sort(budgets, budgets + nb);
  int mt[kMaxLayersPerLaunch];
  for (int bi = 0; bi < nb; ++bi) {
    const int wb = budgets[bi];
    int tot = 0;
    bool ok = true;
    for (int k = 0; k < n; ++k) {
      const int m = std::min(16, std::max(1, wb / nchl[k]));
      if (m * nchl[k] > wb && m > 1) { ok = false; break; }
      mt[k] = m;
      tot += cdiv(Mt, m);
    }
    if (ok && tot <= gmax) { best_budget = wb; break; }
  }
  if (best_budget < 0) return false;
  // Equal M-tiles per workgroup in every layer when the grid has room: a wave
  // then owns the same tile set in every layer and none of its tiles is empty
  // (layers with fewer rows per workgroup only finish their steps sooner).
  {
    int mmin = 16;
    for (int k = 0; k < n; ++k) mmin = std::min(mmin, mt[k]);
    int tot = 0;
    for (int k = 0; k < n; ++k) tot += cdiv(Mt, mmin);
    if (tot <= gmax)
      for (int k = 0; k < n; ++k) mt[k] = mmin;
  }
  int mmax = 1, staged_max = 0, nch_max = 1, begin = 0;
  lp->nlayers = n;
  for (int k = 0; k < n; ++k) {
    LayerPlan& L = lp->layers[k];
    L = LayerPlan();
    L.layer = l0 + k;
    L.hoisted = (l0 + k == 0 && !fuse0) ? 1 : 0;
    L.Kin = L.hoisted ? 0 : (l0 + k == 0 ? I : H);
    L.nch = nchl[k];
    L.mt_per_wg = mt[k];
    L.wg_count = cdiv(Mt, mt[k]);
    L.wg_begin = begin;
    L.staged = 1;
    begin += L.wg_count;
    mmax = std::max(mmax, mt[k]);
    nch_max = std::max(nch_max, nchl[k]);
    staged_max = std::max(staged_max, mt[k] * nchl[k] * 64 * kFragBytes);
  }
  // two waves per SIMD: a wave waiting on one dependency leaves the SIMD to its partner
  if (!choose_split(mmax, ncnt, nch_max, staged_max, dev.lds_per_block, 8, lp) &&
      !choose_split(mmax, ncnt, nch_max, staged_max, dev.lds_per_block, 4, lp))
    return false;
  lp->stream = 0;
  lp->grid = round_grid(begin);
  for (int k = 0; k < n; ++k)
    if (lp->layers[k].wg_count > kFlagsPerLayer) return false;
  return lp->grid <= std::max(gmax, 8);
}

}  // namespace

int make_plan(const int32_t L, const int32_t I, const int32_t H, const int32_t B, const int32_t T,
              const int32_t dtype, const int32_t cell, int force_regime, const DeviceInfo& dev, Plan* out,
              bool aligned) {
  if (L < 1 || I < 1 || H < 1 || B < 1 || T < 1) return kInvalid;
  if (dtype != 0 && dtype != 1) return kInvalid;
  if (cell < 0 || cell > 3) return kInvalid;
  if (force_regime < kRegimeAuto || force_regime > kRegimeWavefront) return kInvalid;
  if (dev.num_cus < 1) return kInvalid;
  Plan& p = *out;
  p = Plan();
  p.bf16 = dtype == 1;
  p.cell = cell;
  p.gates = cell == 0 ? 4 : (cell == 1 ? 3 : 1);
  p.bias_rows = cell <= 1 ? 4 : 1;
  p.KC = p.bf16 ? 64 : 32;
  p.dsize = p.bf16 ? 2 : 4;
  p.Mt = cdiv(H, cell >= 2 ? 16 : 4);  // 16-row tiles: 4 units x 4 rows, or 16 units x 1 row
  p.ncnt = cdiv(B, 16);
  if (p.ncnt > 16) return kUnsupported;                     // B > 256
  if ((long long)L > 64) return kUnsupported;
  if ((long long)T * B > (1LL << 31) / 16 || (long long)H * 4 > (1LL << 30)) return kUnsupported;
  // one step's h (a row-major exchange slot) stays below 4 GiB: kernels address it with 32-bit byte offsets
  if ((long long)B * H * 4 >= (1LL << 32) || (long long)B * I * 4 >= (1LL << 32)) return kUnsupported;

  const int nch_h = cdiv(H, p.KC);
  const int nch_x = cdiv(I, p.KC);

  bool wave = false;
  if (force_regime == kRegimeWavefront || (force_regime == kRegimeAuto && L >= 2)) {
    // try the wavefront: groups of up to 16 layers per launch; layer 0's input
    // product fused into its steps when that fits, else hoisted into one GEMM
    for (int fuse0 = 1; fuse0 >= 0 && !wave; --fuse0) {
      int nrec = 0;
      bool ok = true;
      for (int l0 = 0; l0 < L; l0 += kMaxLayersPerLaunch) {
        const int n = std::min(kMaxLayersPerLaunch, L - l0);
        if (!plan_wavefront(l0, n, p.Mt, nch_h, nch_x, I, H, fuse0 != 0, p.ncnt, dev, &p.rec[nrec])) {
          ok = false;
          break;
        }
        ++nrec;
      }
      if (ok) {
        wave = true;
        p.nrec = nrec;
        p.ngemm = fuse0 ? 0 : 1;
        p.nclear = fuse0 ? 1 : 0;
      }
    }
    if (!wave && force_regime == kRegimeWavefront) return kUnsupported;
  }
  if (!wave) {
    p.nrec = L;
    p.ngemm = L;
    p.nclear = 0;
    for (int l = 0; l < L; ++l)
      if (!plan_single(l, p.Mt, nch_h, p.ncnt, p.bf16 != 0, aligned && (H % p.KC) == 0, dev, &p.rec[l]))
        return kUnsupported;
  }
  p.regime = wave ? kRegimeWavefront : kRegimeLayerwise;
  p.num_launches = p.nrec + p.ngemm + p.nclear;

  // workspace: [error word | step counters L x kFlagsPerLayer, one 128-byte line each |
  //             G (one layer) | exchange buffers of all L layers, T slots each]
  size_t off = 0;
  p.err_off = off;
  off += 256;
  p.flags_off = off;
  off += align256((size_t)L * kFlagsPerLayer * kFlagStride * sizeof(int));
  p.zero_ints = off / sizeof(int);
  p.G_off = off;
  off += align256((size_t)T * p.Mt * B * 16 * sizeof(float));
  // exchange slots hold h_t of one step either row-major ([B][H]) or in load
  // order (ncnt column tiles x nch chunks of 16 x KC), whichever is larger
  p.hist_off = off;
  const size_t slot_raw = std::max((size_t)B * H, (size_t)p.ncnt * 16 * nch_h * p.KC) * p.dsize;
  const size_t slot_bytes = (slot_raw + kSlotAlign - 1) / kSlotAlign * kSlotAlign;
  p.slot_elems = slot_bytes / p.dsize;
  off += (size_t)L * T * slot_bytes;
  // one layer's load-order exchange for layerwise runs (the row-major slots
  // above then feed the next layer's input GEMM); one set of slots, reused
  // layer after layer: T, plus one in front for the register-resident
  // kernel's h0 (it reads slot t and writes slot t + 1)
  p.xf_off = off;
  off += (size_t)(T + 1) * slot_bytes;
  p.ws_bytes = off;
  return kStatusOk;
}

int data_valid_lds(const Plan& p, const LaunchPlan& lp, int H, int B, const DeviceInfo& dev) {
  if (p.regime == kRegimeWavefront || lp.nlayers != 1 || lp.res_nrb > 0 || lp.stream || lp.ks < 2) return 0;
  if (lp.nwaves != 4 || lp.mw != 1 || lp.nw != 1) return 0;  // the one instantiation that has it
  const LayerPlan& pl = lp.layers[0];
  if (!pl.hoisted || !pl.staged || B >= 16 || pl.wg_count > kSentMaxWgs) return 0;
  if (H % p.KC != 0 || ((size_t)H * p.dsize) % 16 != 0 || cdiv(pl.nch, lp.ks) > 6) return 0;
  const int red = lp.lds_bytes - lp.red_off;
  const int need = lp.red_off + ((red + 255) & ~255) + red;
  return need + kLdsReserve <= dev.lds_per_block ? need : 0;
}

}  // namespace lstm
