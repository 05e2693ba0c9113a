/*
 * lstm_fwd.h -- C ABI of the MI355X (gfx950) stacked-LSTM forward library.
 *
 * What one call computes: the forward pass of a stack of L LSTM layers over T
 * timesteps for B independent sequences, h_t, c_t = LSTM(x_t, h_{t-1}, c_{t-1}),
 * where layer l's output sequence is layer l+1's input (the network level of
 * "Optimizing Performance of Recurrent Neural Networks on GPUs", abstract and
 * proposed method).  Per layer and step, with u_t = x_t (l = 0) or h^{l-1}_t:
 *
 *     p   = W_l u_t + R_l h_{t-1} + b_l      (4H rows, gate blocks i, f, g, o)
 *     i   = sigmoid(p_i)  f = sigmoid(p_f)  g = tanh(p_g)  o = sigmoid(p_o)
 *     c_t = f * c_{t-1} + i * g               (fp32)
 *     h_t = o * tanh(c_t)
 *
 * The four per-gate matrices are grouped into one 4H-row matrix per weight
 * (same page, proposed method: gate grouping).
 *
 * The same page applies the method to GRU cells (three grouped matrices) and
 * to the simple RNN (one matrix); desc.cell selects them, read as cuDNN v5's
 * cells (the pages print their equations nowhere):
 *   LSTM_CELL_GRU       W_l [3H][I_l], R_l [3H][H], gate blocks r, z, n;
 *                       b_l [4H] = b_r, b_z, b_Wn, b_Rn
 *                         r = sigmoid(W_r u + R_r h + b_r)
 *                         z = sigmoid(W_z u + R_z h + b_z)
 *                         n = tanh(W_n u + b_Wn + r * (R_n h + b_Rn))
 *                         h_t = (1 - z) * n + z * h_{t-1}
 *   LSTM_CELL_RNN_TANH  W_l [H][I_l], R_l [H][H], b_l [H]:  h_t = tanh(W u + R h + b)
 *   LSTM_CELL_RNN_RELU  the same with max(0, .)
 * These cells have no cell state: c0 and cT are ignored (may be NULL).  With
 * G = 4, 3, 1 weight-row blocks and NB = 4, 4, 1 bias blocks, the layouts below
 * read G*H for 4H in W and R and NB*H for 4H in b.  How the library schedules the
 * work (hoisted input projection, persistent recurrent kernel with weights kept
 * on chip -- "Persistent RNNs: Stashing Recurrent Weights On-Chip" -- and the
 * layer wavefront -- first page, proposed method: layer overlap) is not part of
 * the contract; only the results are.
 *
 * Layouts (all dense, row-major, no padding):
 *   x   [T][B][I]                      dtype
 *   W   W_0 [4H][I] then W_1..W_{L-1}, each [4H][H]     dtype
 *   R   [L][4H][H]                     dtype
 *   b   [L][4H]                        dtype  (one bias per layer)
 *   h0  [L][B][H]                      dtype  (NULL: zeros)
 *   c0  [L][B][H]                      fp32   (NULL: zeros)
 *   y   [T][B][H]                      dtype  (top layer's h_1..h_T)
 *   hT  [L][B][H]                      dtype  (NULL: not written)
 *   cT  [L][B][H]                      fp32   (NULL: not written)
 * Within W, R and b the row blocks are the gates i, f, g, o: row k*H + j is
 * gate k of hidden unit j.  "dtype" is LSTM_F32 (IEEE fp32) or LSTM_BF16
 * (bfloat16 bits); arithmetic is fp32 (fp32 accumulation and cell state) in
 * both cases.  With LSTM_BF16 the h that feeds the next step is the bf16 value
 * stored in y / the layer-to-layer buffers.  A NaN in h may come back as the
 * canonical quiet NaN (its payload is not kept).
 *
 * Ownership: every tensor pointer is a device pointer owned by the caller.  The
 * library allocates no device memory and keeps no state between calls outside
 * the caller's workspace `ws` (lstm_fwd_noalloc instead uses one fixed device
 * array of the library's, described at its declaration), which must hold at least
 * lstm_fwd_workspace_size(desc) bytes, 256-byte aligned.  Its contents on entry
 * are ignored.  All work is enqueued on `stream`, asynchronously; nothing syncs
 * the host.  Concurrent calls must not share a workspace.
 *
 * Errors: every entry point returns a status; nothing throws across the ABI.
 * Argument checks run before anything is enqueued.
 */
#ifndef LSTM_FWD_H
#define LSTM_FWD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LSTM_F32 = 0, LSTM_BF16 = 1 } lstm_dtype_t;

/* Recurrent cell of every layer (0, the LSTM, when the field is left zeroed). */
typedef enum {
  LSTM_CELL_LSTM = 0,
  LSTM_CELL_GRU = 1,
  LSTM_CELL_RNN_TANH = 2,
  LSTM_CELL_RNN_RELU = 3
} lstm_cell_t;

/* Problem description.  L, I, H, B, T >= 1. dtype is an lstm_dtype_t, cell an lstm_cell_t. */
typedef struct {
  int32_t L, I, H, B, T;
  int32_t dtype;
  int32_t cell;
} lstm_desc_t;

typedef enum {
  LSTM_OK = 0,
  LSTM_ERR_INVALID_ARG = 1,     /* bad desc field or a required pointer is NULL      */
  LSTM_ERR_UNSUPPORTED = 2,     /* valid but beyond the library's limits            */
  LSTM_ERR_WORKSPACE = 3,       /* workspace missing, misaligned or too small       */
  LSTM_ERR_HIP = 4,             /* a HIP runtime call or kernel launch failed       */
  LSTM_ERR_BARRIER_TIMEOUT = 5  /* a device-side step wait exceeded its time limit  */
} lstm_status_t;

/* Schedules the planner can choose (or a caller can force, for testing). */
typedef enum {
  LSTM_REGIME_AUTO = 0,
  LSTM_REGIME_LAYERWISE = 1,   /* per layer: input GEMM over all T, then the persistent recurrence */
  LSTM_REGIME_WAVEFRONT = 2    /* layer 0 input GEMM, then one persistent launch running all layers
                                  as a wavefront (layer l step t beside layer l+1 step t-1)          */
} lstm_regime_t;

/* Kinds of kernel launch reported through lstm_fwd_opts_t. */
typedef enum {
  LSTM_KERNEL_INPUT_GEMM = 1, /* grouped input projection of one layer over all steps            */
  LSTM_KERNEL_RECURRENT = 2,  /* persistent recurrence (one layer, or several as a wavefront)     */
  LSTM_KERNEL_CLEAR = 3       /* clears the error word and step counters when no input GEMM
                                 runs first (every layer's input product fused into the steps)   */
} lstm_kernel_kind_t;

/* Size in bytes of the workspace lstm_fwd needs for `d`; 0 if `d` is invalid or unsupported. */
size_t lstm_fwd_workspace_size(const lstm_desc_t *d);

/*
 * Forward pass.  See the file comment for layouts, ownership and errors.
 * x, W, R, b, y and ws are required; h0, c0, hT, cT may be NULL.
 * Returns LSTM_OK once everything is enqueued.  A device-side wait that times
 * out is reported by lstm_fwd_last_error, not here (the call does not sync).
 */
lstm_status_t lstm_fwd(const lstm_desc_t *d,
                       const void *x, const void *h0, const float *c0,
                       const void *W, const void *R, const void *b,
                       void *y, void *hT, float *cT,
                       void *ws, hipStream_t stream);

/* Options for lstm_fwd_ex.  Zero-initialise and set what you need. */
typedef struct {
  int32_t force_regime;       /* lstm_regime_t; LSTM_REGIME_AUTO lets the planner decide          */
  int32_t max_launches;       /* capacity of ev_start / ev_stop / launch_kind (0: no events)       */
  hipEvent_t *ev_start;       /* if non-NULL: recorded on `stream` right before launch k           */
  hipEvent_t *ev_stop;        /* if non-NULL: recorded on `stream` right after launch k            */
  int32_t *launch_kind;       /* out (optional): lstm_kernel_kind_t of launch k                    */
  int32_t *num_launches;      /* out (optional): number of kernel launches enqueued                */
  int64_t wait_timeout_us;    /* device step-wait limit in microseconds; 0 selects the default (2 s);
                                 negative makes every wait that is not already satisfied fail at once
                                 (exercises the timeout path without waiting)                       */
  int64_t *trace;             /* optional device buffer: per-step phase timestamps (wall-clock ticks)
                                 of the first recurrent launch, for workgroups v = 0, s, 2s, ...
                                 (s = trace_stride): trace[((v/s)*T + t)*8 + k], k = 0 step start,
                                 1 dependencies met, 2 products done, 3 partial sums combined,
                                 4 gates/stores issued, 5 step published (100 MHz wall clock);
                                 6 and 7: shader-clock counter at 0 and at 2, so (7-6)/(2-0)
                                 gives the core clock; trace_wgs*T*8 entries                       */
  int32_t trace_wgs;          /* number of traced workgroups (0: no trace)                        */
  int32_t trace_stride;       /* virtual workgroup stride between traced workgroups (>= 1)         */
  int32_t plain_launch;       /* 1: launch the persistent kernel with an ordinary launch instead of a
                                 cooperative one (for profilers that do not handle cooperative
                                 launches, and for HIP graph capture: a forward enqueued this way
                                 on a capturing stream replays to the same bits; it records no
                                 memset nodes).  Co-residency is still checked against the
                                 occupancy limit; a grid that is not co-resident ends with
                                 LSTM_ERR_BARRIER_TIMEOUT rather than a hang.                      */
} lstm_fwd_opts_t;

/* lstm_fwd with options (opts may be NULL, which equals lstm_fwd). */
lstm_status_t lstm_fwd_ex(const lstm_desc_t *d,
                          const void *x, const void *h0, const float *c0,
                          const void *W, const void *R, const void *b,
                          void *y, void *hT, float *cT,
                          void *ws, hipStream_t stream, const lstm_fwd_opts_t *opts);

/* Human-readable name of a status code (static storage; never NULL). */
const char *lstm_status_string(lstm_status_t s);

/*
 * Host-only argument check, the same one lstm_fwd runs before enqueueing:
 * desc fields, required pointers and the workspace size `ws_bytes`.  Makes no
 * HIP call, so it can run on a machine without a GPU.
 */
lstm_status_t lstm_fwd_validate(const lstm_desc_t *d, const void *x, const void *W,
                                const void *R, const void *b, const void *y,
                                const void *ws, size_t ws_bytes);

/*
 * Waits for `stream`, then reads the device-side error word that the last
 * lstm_fwd on workspace `ws` left (LSTM_OK or LSTM_ERR_BARRIER_TIMEOUT).
 */
lstm_status_t lstm_fwd_last_error(const void *ws, hipStream_t stream);

/*
 * lstm_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The workspace is a fixed device array inside the
 * library, LSTM_FWD_NOALLOC_MAX_WORKSPACE bytes on each device the library
 * runs on, held until the process ends.  A problem whose
 * lstm_fwd_workspace_size exceeds it returns LSTM_ERR_WORKSPACE before
 * anything is enqueued (64 MiB holds, e.g., a 1-layer H = 128, B = 8, T = 16
 * problem or a 1-layer bf16 H = 1536, B = 4, T = 256 one; the 4-layer
 * H = 512, B = 64, T = 100 problem needs 113 MiB).  The call allocates
 * nothing; the other arguments, layouts, results and errors are lstm_fwd's.
 * Every call on one device shares that device's array and finds the previous
 * call's contents in it (the kernels clear what must start at zero): calls
 * that overlap on one device -- on two streams, or from two host threads --
 * race, and their results are undefined; calls ordered on one stream are safe.
 * dev_status: optional device int32 (NULL: not written).  After the call's
 * kernels it holds LSTM_OK or LSTM_ERR_BARRIER_TIMEOUT: what
 * lstm_fwd_last_error reports for a call with a caller's workspace.
 */
#define LSTM_FWD_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
lstm_status_t lstm_fwd_noalloc(const lstm_desc_t *d,
                               const void *x, const void *h0, const float *c0,
                               const void *W, const void *R, const void *b,
                               void *y, void *hT, float *cT,
                               int32_t *dev_status, hipStream_t stream);

/* What the planner decided for a problem (for logging and tests). */
typedef struct {
  int32_t regime;            /* lstm_regime_t actually used                                   */
  int32_t num_launches;      /* kernel launches per call                                       */
  int32_t grid;              /* workgroups of each recurrent launch                            */
  int32_t block;             /* threads per workgroup of the recurrent kernel                  */
  int32_t lds_bytes;         /* dynamic LDS per workgroup of the recurrent kernel              */
  int32_t ksplit;            /* waves that split the K dimension of one output tile            */
  int32_t weights_on_chip;   /* 1 if every recurrent workgroup keeps its weight rows on chip for
                                the whole sequence (in LDS, or in LDS plus registers)         */
  int32_t layers_per_launch; /* layers one recurrent launch runs concurrently                  */
  int32_t wg_per_layer[16];  /* workgroups given to each layer of the first recurrent launch   */
  int32_t mtiles_per_wg[16]; /* 16-row tiles (4 units x 4 gates) per workgroup, per layer      */
  int32_t tile_groups_m;     /* waves of a K-group that split the M-tiles (x tile_groups_n = 4/ksplit) */
  int32_t tile_groups_n;     /* ... that split the 16-column batch tiles                      */
  int32_t wave_tiles_m;      /* most M-tiles one wave computes                                 */
  int32_t wave_tiles_n;      /* most column tiles one wave computes                            */
  int32_t weights_streamed;  /* 1 if the first recurrent launch reads weights from HBM per step */
  int32_t input_gemms;       /* input-projection GEMM launches per call; 0 when every layer's
                                input product W_l u_t is fused into its recurrent steps          */
  int32_t weight_blocks_in_registers; /* 2 KiB weight blocks each wave of the first recurrent
                                launch keeps in registers (0: weights in LDS only, or streamed) */
  int32_t data_valid_exchange; /* 1 if the first recurrent launch exchanges h_t without step
                                counters: its slots start filled with all-ones words and readers
                                re-read h_{t-1} until no element holds that pattern (small
                                single-layer grids; assumes 16-byte aligned caller buffers)     */
} lstm_plan_info_t;

/*
 * Runs the planner only (no HIP call when num_cus > 0): num_cus and
 * lds_per_cu describe the device (0 queries the current HIP device).
 */
lstm_status_t lstm_fwd_plan(const lstm_desc_t *d, int32_t force_regime, int32_t num_cus,
                            int32_t lds_per_cu, lstm_plan_info_t *out);

#ifdef __cplusplus
}
#endif

#endif /* LSTM_FWD_H */
