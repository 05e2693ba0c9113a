/*
 * lstm_bwd.h -- C ABI of the stacked-LSTM training passes on MI355X (gfx950):
 * a forward pass that keeps what the backward pass needs, and the backward
 * pass (backpropagation through time) itself.
 *
 * The backward pass is the chain rule through the forward definition of
 * lstm_fwd.h (LSTM cell only).  Per layer from the top down and per step from
 * the last to the first, with dh_rec and dc_rec the gradients reaching h_t and
 * c_t through step t+1 (dhT and dcT at the last step):
 *     dh    = dY[t] + dh_rec                       (dY: dy for the top layer,
 *                                                  else the layer above's input gradient)
 *     dc    = dh o (1 - tanh(c_t)^2) + dc_rec
 *     dp    = [dc g i(1-i), dc c_{t-1} f(1-f), dc i (1-g^2), dh tanh(c_t) o(1-o)]
 *     dh_rec = dp R_l ,   dc_rec = dc f
 * and then, once the dp of every step are known, the weight and input
 * gradients as single products over all T*B columns
 *     dW_l = dP^T U ,  dR_l = dP^T H_prev ,  db_l = sum of dP over the columns ,
 *     dU = dP W_l  (the layer below's dY, or dx)
 * ("Optimizing Performance of Recurrent Neural Networks on GPUs", proposed
 * method: the weight update done as one large product, and the layers'
 * backward passes able to follow one another).
 *
 * Layouts (dense, row-major): the forward tensors as in lstm_fwd.h.
 *   reserve  written by lstm_fwd_train, read by lstm_bwd; lstm_train_reserve_size
 *            bytes: for every layer l, the activated gates [T][B][4H] fp32 (blocks
 *            i, f, g, o), then for every layer c_t [T][B][H] fp32, then for every
 *            layer h_t [T][B][H] in dtype.  Its contents are meaningful only
 *            between an lstm_fwd_train and the lstm_bwd of the same inputs.
 *   dy [T][B][H], dhT, dcT [L][B][H]                         fp32 (dhT, dcT: NULL = zero)
 *   dx [T][B][I], dh0, dc0 [L][B][H]                         fp32 (NULL: not written)
 *   dW like W, dR like R, db like b                          fp32 (required)
 * Arithmetic: the per-step gate derivatives in fp32; every product in the
 * workload's dtype with fp32 accumulation (bf16 workloads multiply bf16
 * operands, as their forward does).
 *
 * Ownership: every pointer is a device pointer owned by the caller.  `ws` must
 * hold lstm_bwd_workspace_size(desc) bytes, 256-byte aligned; its contents on
 * entry are ignored.  Work is enqueued on `stream` asynchronously.
 *
 * Errors: status codes as in lstm_fwd.h, checked on the host before anything
 * is enqueued; a cell other than the LSTM returns LSTM_ERR_UNSUPPORTED.
 *
 * Recurrent chain: for H = 128, 256, 512, 1024, 1536, 2048, 3072 or 4096 in
 * bf16 and H = 128, 256, 512 or 1024 in fp32, with B <= 64 (32 at H = 4096), it
 * runs as one persistent launch per layer that keeps R_l^T on chip (when its
 * workgroups fit on the device at once and dy, reserve and the state
 * tensors are 16-byte aligned): H / 16 workgroups per batch group (up to four
 * groups, each an independent copy over part of the batch), each finishing
 * 16 units, over all of K (H <= 512) or a quarter of it with partial sums
 * added across four workgroups; dp_t and the partial sums go through `ws`
 * with per-workgroup step counters, and a step wait longer than 2 s sets the
 * error word that lstm_bwd_last_error reports.  Other shapes run it as two
 * launches per step that stream R_l^T from memory.  Either way the results
 * are deterministic: every sum is taken in a fixed order.
 */
#ifndef LSTM_BWD_H
#define LSTM_BWD_H

#include "lstm_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the reserve buffer for `d` (0: invalid, or a cell other than the LSTM). */
size_t lstm_train_reserve_size(const lstm_desc_t *d);

/* lstm_fwd that also fills `reserve` (required); `ws` as for lstm_fwd. */
lstm_status_t lstm_fwd_train(const lstm_desc_t *d,
                             const void *x, const void *h0, const float *c0,
                             const void *W, const void *R, const void *b,
                             void *y, void *hT, float *cT,
                             void *reserve, void *ws, hipStream_t stream);

/* lstm_fwd_train with the options of lstm_fwd_ex (opts may be NULL). */
lstm_status_t lstm_fwd_train_ex(const lstm_desc_t *d,
                                const void *x, const void *h0, const float *c0,
                                const void *W, const void *R, const void *b,
                                void *y, void *hT, float *cT,
                                void *reserve, void *ws, hipStream_t stream, const lstm_fwd_opts_t *opts);

/* Options for lstm_bwd_ex.  Zero-initialise and set what you need. */
typedef struct {
  int32_t plain_launch;     /* 1: start the on-chip recurrent chain with an ordinary launch instead of a
                               cooperative one (for profilers that do not handle cooperative launches);
                               co-residency is still checked against the occupancy limit          */
  int32_t reserved0;        /* zero */
  int64_t wait_timeout_us;  /* the on-chip chain's step-wait limit in microseconds; 0 selects the
                               default (2 s); negative makes every wait that is not already
                               satisfied fail at once (exercises the timeout path without waiting) */
  int32_t reserved[4];      /* zero */
} lstm_bwd_opts_t;

/* Bytes of the workspace lstm_bwd needs for `d` (0: invalid or unsupported). */
size_t lstm_bwd_workspace_size(const lstm_desc_t *d);

/* 1 if lstm_bwd runs the recurrent chain of `d` as the persistent on-chip
 * launch described above, 0 if it streams R_l^T (or `d` is invalid).  Host
 * only, no HIP calls; at run time the on-chip chain also needs its
 * workgroups co-resident on the device and dy, reserve, c0, dhT, dcT, dh0 and
 * dc0 16-byte aligned (it moves them 16 bytes at a time), else the streamed
 * chain runs. */
int lstm_bwd_chain_on_chip(const lstm_desc_t *d);

/* Status of the last lstm_bwd on `ws`: synchronises `stream`, then reads the
 * workspace's error word (LSTM_ERR_BARRIER_TIMEOUT if a step wait of the
 * on-chip recurrent chain ran out).  lstm_bwd zeroes that word on entry. */
lstm_status_t lstm_bwd_last_error(const void *ws, hipStream_t stream);

/* Backward pass: gradients of every forward input from dy, dhT and dcT. */
lstm_status_t lstm_bwd(const lstm_desc_t *d,
                       const void *x, const void *h0, const float *c0,
                       const void *W, const void *R, const void *reserve,
                       const float *dy, const float *dhT, const float *dcT,
                       float *dx, float *dh0, float *dc0,
                       float *dW, float *dR, float *db,
                       void *ws, hipStream_t stream);

/* lstm_bwd with options (opts may be NULL, which equals lstm_bwd). */
lstm_status_t lstm_bwd_ex(const lstm_desc_t *d,
                          const void *x, const void *h0, const float *c0,
                          const void *W, const void *R, const void *reserve,
                          const float *dy, const float *dhT, const float *dcT,
                          float *dx, float *dh0, float *dc0,
                          float *dW, float *dR, float *db,
                          void *ws, hipStream_t stream, const lstm_bwd_opts_t *opts);

#ifdef __cplusplus
}
#endif

#endif /* LSTM_BWD_H */
