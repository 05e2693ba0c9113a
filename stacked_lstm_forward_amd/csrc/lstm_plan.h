// Host planner: decides the schedule, the workgroup partition and the
// workspace layout of one lstm_fwd call.  Pure host code (no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lstm_params.h"

namespace lstm {

struct DeviceInfo {
  int num_cus = 256;        // compute units
  int lds_per_block = 160 * 1024;
};

struct LayerPlan {
  int layer = 0;        // network layer index
  int hoisted = 1;      // 1: input product from the input GEMM; 0: fused W_l u_t per step
  int Kin = 0;          // fused input width (0 when hoisted)
  int nch = 0;          // K chunks per tile row (fused input + recurrent)
  int wg_begin = 0, wg_count = 0, mt_per_wg = 0;
  int staged = 0;
};

struct LaunchPlan {
  int nlayers = 0;
  LayerPlan layers[kMaxLayersPerLaunch];
  int stream = 0;       // 1: weight rows streamed from global memory every step
  int res_nrb = 0;      // > 0: register-resident kernel; weight blocks per wave in registers
  int res_nci = 0;      // ... and chunks per wave (K-group)
  int nwaves = 4;       // waves per workgroup (4: one per SIMD, 8: two per SIMD)
  int ks = 4, ntgm = 1, ntgn = 1, mw = 1, nw = 1;
  int lds_bytes = 0, red_off = 0;
  int grid = 0;
};

struct Plan {
  int regime = 0;       // lstm_regime_t
  int cell = 0;         // lstm_cell_t
  int gates = 4;        // weight-row blocks of H rows (4 LSTM, 3 GRU, 1 simple RNN)
  int bias_rows = 4;    // bias blocks of H (4 LSTM, 4 GRU, 1 simple RNN)
  int bf16 = 0;
  int KC = 32;          // K columns per chunk
  int dsize = 4;
  int Mt = 0, ncnt = 0;
  int nrec = 0;         // recurrent launches
  LaunchPlan rec[64];   // layerwise: one per layer; wavefront: one per group of up to 16 layers
  int ngemm = 0;        // input-GEMM launches
  int nclear = 0;       // 1: a clear kernel zeroes the error word and step counters (no input GEMM does)
  int num_launches = 0;
  // workspace layout (bytes)
  size_t err_off = 0, flags_off = 0, G_off = 0, hist_off = 0, ws_bytes = 0;
  size_t slot_elems = 0;  // elements between two steps of an exchange buffer
  size_t xf_off = 0;    // one layer's load-order exchange (layerwise runs), T slots of slot_elems
  size_t zero_ints = 0; // ints zeroed at the start (error word + all step counters)
};

// Data-valid exchange (lstm_rec.h): recurrent launch `lp` qualifies when it
// runs one hoisted layer whose weight rows stay in LDS, splits the K range
// over waves (the split's barrier is the step's only one), loads all of a
// wave's chunks at once (at most 6 per wave with one column tile), exchanges
// h in row-major slots (batch below one 16-column tile, whole 16-byte rows)
// and has at most kSentMaxWgs workgroups: every reader re-reads the whole
// slot until it is complete, which measured faster than step counters up to
// 64 workgroups and slower from 128 (one layer, B = 4 and 8, bf16 and fp32).
// Returns the launch's LDS bytes (its reduction area once per step parity) or
// 0.  The caller adds the conditions on its buffers (16-byte aligned rows).
constexpr int kSentMaxWgs = 64;
int data_valid_lds(const Plan& p, const LaunchPlan& lp, int H, int B, const DeviceInfo& dev);

// Returns 0 on success, else an lstm_status_t.
// `aligned`: the caller's R (and h0) allow 16-byte loads; the register-resident
// kernel needs it.
int make_plan(const int32_t L, const int32_t I, const int32_t H, const int32_t B, const int32_t T,
              const int32_t dtype, const int32_t cell, int force_regime, const DeviceInfo& dev, Plan* out,
              bool aligned = true);

}  // namespace lstm
