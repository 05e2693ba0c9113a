// Kernel parameter blocks shared by the host planner and the device kernels.
#pragma once

#include <stdint.h>

namespace lstm {

constexpr int kMaxLayersPerLaunch = 16;  // layers one recurrent launch can run as a wavefront
constexpr int kFlagsPerLayer = 1024;     // step-counter slots per layer (max workgroups per layer)
constexpr int kFlagStride = 32;          // ints between two step counters: one 128-byte line each
constexpr int kGemmThreads = 256;
constexpr int kGemmTileM = 256;          // rows (16 M-tiles) per input-GEMM workgroup
constexpr int kGemmTileN = 128;          // columns (time x batch) per input-GEMM workgroup
constexpr int kSlotAlign = 256;          // bytes: exchange slots never share a cache line
// Register-resident recurrent kernel (one layer, weights in registers + LDS):
// 4 waves = 4 K-groups; per shape the dtype, mw M-tiles per workgroup, nci
// chunks per K-group (H = 4 nci chunks of 64 bf16 or 32 fp32 columns exactly)
// and nrb of each wave's mw * nci weight blocks in registers, the rest in LDS;
// up to kResMaxNW 16-column batch tiles.
struct ResShape {
  int bf16, mw, nci, nrb;
};
constexpr int kResShapes = 3;
constexpr ResShape kResShape[kResShapes] = {
    {1, 4, 16, 48},  // bf16 H = 4096 (R_l 128 MiB): 48 blocks in registers, 16 in LDS
    {1, 3, 12, 36},  // bf16 H = 3072 (72 MiB): all 36 in registers
    {0, 2, 16, 16},  // fp32 H = 2048 (64 MiB): 16 blocks in registers, 16 in LDS
};
constexpr int kResMaxNW = 4;

// Input projection G = W_l U^T + b_l over all T*B columns (hoisted out of the recurrence).
// Output layout [T][Mt][B][16] fp32: for step t, M-tile mt, batch b, the 16
// gate-interleaved rows of the tile (see cell_row).
struct GemmParams {
  const void* W;     // [4H][K] (caller layout, gate blocks)
  const void* U;     // input sequence: step t, batch b at U + t*u_slot + b*K (elements)
  const void* bias;  // [4H]
  float* G;          // [T][Mt][B][16]
  int* zero_ptr;     // if non-null: workgroup 0 zeroes zero_count ints first (flags, error word)
  unsigned* fill_ptr;     // if non-null: fill_count words set to all ones first (the exchange
  long long fill_count;   // slots of the data-valid recurrent launch that follows)
  long long u_slot;  // elements between two steps of U
  int zero_count;
  int K, H, Mt, B, N;  // N = T*B
  int vec_ok_w, vec_ok_u;
  int cell;            // lstm_cell_t
  int num_cus;         // compute units of the device (tile-shape choice; 0: 256)
  // plain product (the backward pass's weight and input gradients): C[m][n] =
  // sum over k of W[m][k] U[n][k], rows m < H, fp32, row stride ldc; no bias.
  // With ksplit > 1 the K range is split in ksplit equal chunk ranges: range 0
  // writes C, range z > 0 writes C2 + (z - 1) split_stride (same row stride),
  // and the launcher adds them into C afterwards, in order.
  float* C;
  long long ldc;
  float* C2;
  long long split_stride;
  int ksplit;
  // direct-to-LDS kernel, mixed column-tile widths: nblk column blocks per
  // M-block, the first nbig of NT column tiles, the rest of NT - 2 (0: all NT)
  int nbig, nblk;
};

// One layer of a recurrent launch.
struct RecLayer {
  const void* W;          // fused input weights W_l [4H][Kin], or null when the input is hoisted
  const void* R;          // R_l [4H][H]
  const void* bias;       // b_l [4H] (fused input only; hoisted G already holds the bias)
  const float* G;         // hoisted pre-activations [T][Mt][B][16], or null
  const void* U;          // fused input: step t, batch b at U + t*u_slot + b*Kin (the layer
                          // below's exchange buffer, or x for layer 0), or null
  void* X;                // row-major h_t, [T] slots of [B][H]: the exchange buffer itself
                          // when F is null, else a copy for a later input GEMM, or null
  void* F;                // aligned path: h_t in load order (fragment blocks, see
                          // lstm_rec.h), [T] slots of fslot elements, or null
  void* Yout;             // caller's y [T][B][H] (top layer), or null
  const void* h0;         // [B][H] or null (zeros)
  const float* c0;        // [B][H] or null (zeros)
  void* hT;               // [B][H] or null
  float* cT;              // [B][H] or null
  int* flags;             // per-workgroup step counters of this layer, kFlagStride apart
  const int* dep_flags;   // step counters of the producer of U in this launch, or null
  int dep_count;          // workgroups of that producer
  long long u_slot;       // elements between two steps of U
  int ufrag;              // 1: U is the layer below's F (load order), else row-major
  int Kin;                // fused input width (0 when hoisted)
  int wg_begin, wg_count; // virtual workgroup ids owned by this layer
  int mt_per_wg;          // M-tiles per workgroup
  int staged;             // 1: weight rows kept in LDS for the whole sequence
  int vec_ok;             // 16-byte loads allowed on W/R/U/X/h0 rows
  // training forward (LSTM only; null otherwise): per step, the activated
  // gates [T][B][4H] fp32 (blocks i, f, g, o), c_t [T][B][H] fp32 and h_t
  // [T][B][H] (dtype) of this layer, for the backward pass
  float* save_gates;
  float* save_c;
  void* save_h;
};

struct RecParams {
  RecLayer layer[kMaxLayersPerLaunch];
  long long slot;         // elements between two steps of an exchange buffer
  long long fslot;        // elements between two steps of F
  int nlayers;
  int T, B, H, Mt, ncnt;  // ncnt = ceil(B/16) column tiles
  int cell;               // lstm_cell_t
  int ks;                 // waves splitting the K chunks of one tile (1, 2, 4 or 8)
  int ntgm, ntgn;         // tile groups: ntgm*ntgn = waves/ks; group g -> (g%ntgm, g/ntgm)
  int mw, nw;             // tiles per wave in M and N (<= the kernel's MW, NW)
  int red_off;            // LDS byte offset of the cross-wave reduction area
  int grid;               // launched workgroups
  int xcd_remap;          // 1: map blockIdx round-robin over 8 XCDs to contiguous virtual ids
  int* err;               // device error word (0 ok, 1 step-wait timeout)
  long long timeout_ticks;  // per-wait limit in wall-clock ticks
  long long* trace;       // optional per-step phase timestamps (see lstm_fwd_opts_t), or null
  int trace_wgs, trace_stride;
  int sent;               // 1: data-valid exchange (single hoisted layer, row-major slots): the
                          // slots start filled with all-ones words, h_t is written without a step
                          // counter and readers poll the data itself (see lstm_rec.h)
  int red_stride;         // bytes between the two step-parity copies of the reduction area (sent)
};

}  // namespace lstm
