// Persistent recurrent kernel of the stacked-LSTM forward pass (template
// definitions; instantiated by lstm_rec_inst.hip once per dtype / weight source).
#pragma once

#include "lstm_common.h"
#include "lstm_params.h"

namespace lstm {

// ----------------------------------------------------------------------------
// Step ordering
// ----------------------------------------------------------------------------
// Protocol between workgroups (no cache-wide fences):
//  * a layer's h_t is written to slot t of its exchange buffer with agent-scope
//    atomic stores, which write through to the device-wide coherence point;
//    every slot is written once per launch and starts on its own 256-byte
//    boundary, so no cache can hold a copy of it from before it was written
//    (kernel start drops stale lines from previous launches);
//  * the writer waits for those stores to complete (s_waitcnt 0), then one
//    thread bumps the workgroup's step counter (agent-scope atomic store);
//  * a reader polls the counters it depends on (one 128-byte line each, all
//    polled with one batch of loads), then reads the slot with ordinary loads.
// Every wait is bounded: past `timeout` wall-clock ticks the error word is set
// and all workgroups leave the kernel.

// One poll of flags[0..min(count, 256)) by one whole wave: lane i loads
// counters i, i+64, i+128, i+192 (indices clamped, so all loads are
// unconditional and in flight together).
__device__ __forceinline__ void poll_issue(const int* flags, int count, int (&v)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = min(lane + 64 * k, count - 1);
    v[k] = __hip_atomic_load(flags + (long)i * kFlagStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Executed by one whole wave: true once every counter of a[0..na) is >= ta
// and every counter of b[0..nb) is >= tb (b may be null).  Both sets are
// polled with one batch of loads, so a satisfied wait costs one round trip.
// False if another workgroup reported an error or the wait timed out.
// One poll at a time (the register-resident kernel, which has no registers
// for a second batch in flight, uses it directly).
__device__ bool wait_counts_serial(const int* a, int na, int ta, const int* b, int nb, int tb, int* err,
                                   long long timeout);

// The same wait with two polls in flight while at most 256 counters per set
// are polled (measured: the 1-layer bf16 H = 1536, B = 4, T = 2048 recurrence
// 7.43 -> 7.38 ms; the 4-layer fp32 H = 512 wavefront about 1% faster).
__device__ bool wait_counts(const int* a, int na, int ta, const int* b, int nb, int tb, int* err,
                            long long timeout) {
  const int lane = threadIdx.x & 63;
  const long long start = wall_clock64();
  if (max(na, b ? nb : 0) <= 256) {
    // Two polls in flight, each batch also reading the error word: a change
    // is seen about half a round trip after it lands, instead of up to two
    // round trips (a poll, then a dependent read of the error word).
    int va[2][4], vb[2][4], ve[2];
    auto issue = [&](int k) {
      poll_issue(a, na, va[k]);
      if (b) poll_issue(b, nb, vb[k]);
      ve[k] = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    issue(0);
    while (true) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        issue(k ^ 1);
        int ok = 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ok &= (va[k][i] >= ta) ? 1 : 0;
          if (b) ok &= (vb[k][i] >= tb) ? 1 : 0;
        }
        if (__all(ok)) return true;
        if (ve[k] != 0) return false;
        if (wall_clock64() - start > timeout) {
          if (lane == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return false;
        }
      }
    }
  }
  return wait_counts_serial(a, na, ta, b, nb, tb, err, timeout - (wall_clock64() - start));
}

__device__ bool wait_counts_serial(const int* a, int na, int ta, const int* b, int nb, int tb, int* err,
                                   long long timeout) {
  const int lane = threadIdx.x & 63;
  const long long start = wall_clock64();
  while (true) {
    int ok = 1;
    const int n = max(na, b ? nb : 0);
    // the error word is read with the first batch of counters, not after them
    const int e = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int base = 0; base < n; base += 256) {
      int va[4], vb[4];
      if (base < na) poll_issue(a + (long)base * kFlagStride, na - base, va);
      if (b && base < nb) poll_issue(b + (long)base * kFlagStride, nb - base, vb);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (base < na) ok &= (va[k] >= ta) ? 1 : 0;
        if (b && base < nb) ok &= (vb[k] >= tb) ? 1 : 0;
      }
    }
    if (__all(ok)) return true;
    if (e != 0) return false;
    if (wall_clock64() - start > timeout) {
      if (lane == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

template <bool BF16>
__device__ __forceinline__ void store_coherent(typename Dt<BF16>::T* p, typename Dt<BF16>::T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One lane's gate non-linearities and state update.  p holds the lane's four
// pre-activation rows of its tile (LSTM: i, f, g, o of one unit; GRU: r, z and
// the input and recurrent halves of n; simple RNN: four consecutive units).
// `st` is the lane's fp32 state: the LSTM's cell c, the GRU's h_{t-1}; unused
// by the simple RNN.  emit(k, h) receives the new hidden value of the lane's
// unit + k (k = 0 except for the simple RNN, which emits min(4, left) units).
template <class Emit>
__device__ __forceinline__ void cell_update(int cell, const f32x4 p, float& st, int left, Emit&& emit) {
  if (cell == kCellLstm) {
    const float ig = sigmoid_f(p[0]);
    const float fg = sigmoid_f(p[1]);
    const float gg = tanh_f(p[2]);
    const float og = sigmoid_f(p[3]);
    const float cn = fg * st + ig * gg;
    st = cn;
    emit(0, og * tanh_f(cn));
  } else if (cell == kCellGru) {
    const float rg = sigmoid_f(p[0]);
    const float zg = sigmoid_f(p[1]);
    const float ng = tanh_f(p[2] + rg * p[3]);
    const float hn = (1.f - zg) * ng + zg * st;
    st = hn;
    emit(0, hn);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < left) emit(k, cell == kCellRnnRelu ? fmaxf(p[k], 0.f) : tanh_f(p[k]));
  }
}

// Training forward: the LSTM step's activated gates (the same functions of
// the same pre-activations as in cell_update, so the same values) and the new
// cell state of (batch column b, unit j), saved for the backward pass.
__device__ __forceinline__ void save_lstm_step(float* gates, float* cs, const f32x4 p, float c, int t, int B, int H,
                                               int b, int j) {
  const long r = (long)t * B + b;
  float* g = gates + r * 4 * H + j;
  g[0] = sigmoid_f(p[0]);
  g[H] = sigmoid_f(p[1]);
  g[2L * H] = tanh_f(p[2]);
  g[3L * H] = sigmoid_f(p[3]);
  cs[r * H + j] = c;
}

// ----------------------------------------------------------------------------
// Persistent recurrence (optionally several layers as a wavefront)
// ----------------------------------------------------------------------------
// Waves: wave w -> K-group w % ks, tile group w / ks.  The ks waves of a tile
// group split the K chunks of the same output tiles and combine them through
// LDS; tile group g covers M-tiles g%ntgm (+ntgm ...) and column tiles
// g/ntgm (+ntgn ...).  MW x NW is the most tiles one wave holds; STREAM means
// the weight rows are read from global memory every step instead of LDS.
//
// VEC (the fast path): every K range is a whole number of chunks and every row
// starts on a 16-byte boundary, so each fragment is two unconditional 16-byte
// loads; rows past the end are clamped to a valid row (their products are
// never used).  With no branch around a load, the compiler's wait counting
// stays exact and a wave keeps PD chunks of loads in flight ahead of its
// MFMAs.  !VEC handles ragged sizes with per-element loads (slow, correct).
// PD: chunks of loads in flight per wave, from a budget of 48 registers for the
// ring (two waves share a SIMD, so a wave has at most 256 registers in all);
// even, so that the two LDS weight buffers alternate with the ring slot.  A
// deeper ring measured slower: every wave's burst of loads at the start of a
// step then queues in front of the first chunk everybody waits for.
template <int MW, int NW, bool STREAM>
struct RecShape {
  static constexpr int kRegsPerChunk = 8 * NW + (STREAM ? 8 * MW : 0);
  static constexpr int kBudget = 48;
  static constexpr int kFit = kBudget / kRegsPerChunk;
  static constexpr int PD = kFit < 2 ? 2 : (kFit > 8 ? 8 : (kFit & ~1));
};

// FRAG (aligned path only): h_t is exchanged in load order through the F
// buffers (see the addressing note below) instead of the row-major slots.
template <bool BF16, int MW, int NW, bool STREAM, bool VEC, int NWV, bool FRAG>
__global__ void __launch_bounds__(64 * NWV) lstm_rec_kernel(const RecParams P) {
  static_assert(VEC || !FRAG, "the load-order exchange needs the aligned path");
  typedef typename Dt<BF16>::T T;
  constexpr int KC = Dt<BF16>::KC;
  constexpr int PD = RecShape<MW, NW, STREAM>::PD;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_ok;
  __shared__ int s_abort[2];  // data-valid exchange: a wave gave up waiting in a step of this parity

  // The layer table is read in place from the kernel-argument segment with a
  // wave-uniform index (scalar loads); copying one entry out of the by-value
  // array with a runtime index would spill.
  typedef const __attribute__((address_space(4))) RecParams KP;
  KP* pp = (KP*)(__builtin_amdgcn_kernarg_segment_ptr());
  const int bid = blockIdx.x;
  const int v = P.xcd_remap ? ((bid & 7) * (P.grid >> 3) + (bid >> 3)) : bid;
  int li = -1;
  for (int i = 0; i < P.nlayers; ++i)
    if (v >= pp->layer[i].wg_begin && v < pp->layer[i].wg_begin + pp->layer[i].wg_count) li = i;
  if (li < 0) return;
  li = __builtin_amdgcn_readfirstlane(li);
#define LY(f) (pp->layer[li].f)

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a provably wave-uniform value: everything derived from it
  // (K-group, tile group, chunk counts, tile validity) lives in scalar
  // registers and its branches are scalar, so no load sits behind a divergent branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = P.ks;
  const int kg = wave % ks, tg = wave / ks;
  const int gm = tg % P.ntgm, gn = tg / P.ntgm;
  const int wl = v - LY(wg_begin);
  const int mt0 = wl * LY(mt_per_wg);
  const int mcnt = min(LY(mt_per_wg), P.Mt - mt0);
  const int H = P.H, B = P.B, T_ = P.T, Kin = LY(Kin);
  const long slot = P.slot;
  const int nch_u = (Kin + KC - 1) / KC;
  const int nch_h = (H + KC - 1) / KC;
  const int nch = nch_u + nch_h;
  const bool vec = LY(vec_ok);
  const int q = lane >> 4;
  const int cell = P.cell;
  uint4* As = reinterpret_cast<uint4*>(smem);  // fragment block (m, c) at As + (m * nch + c) * 128
  // Data-valid exchange (one hoisted layer, row-major slots, every chunk of a
  // wave loaded at once): no step counters.  The host fills the slots with
  // all-ones words; a reader re-reads its chunks of h_{t-1} with coherent
  // loads until none holds that pattern, a writer stores h_t (NaNs made
  // canonical) and moves on without waiting for its stores.  The K-split
  // partial sums alternate between two LDS areas by step parity, so no
  // barrier closes a step.
  constexpr bool kSentCode = VEC && !STREAM && !FRAG && NWV == 4 && MW == 1 && NW == 1;
  const bool sent = kSentCode && P.sent && ks > 1 && Kin == 0 && LY(staged) && (nch + ks - 1) / ks <= PD;
  if (tid == 0) s_abort[0] = s_abort[1] = 0;

  // ---- keep this workgroup's weight rows on chip for the whole sequence
  if (!STREAM && LY(staged)) {
    const int total = mcnt * nch * 64;
    for (int f = tid; f < total; f += 64 * NWV) {
      const int ln = f & 63;
      const int c = (f >> 6) % nch;
      const int m = (f >> 6) / nch;
      const CellRow cr = cell_row(cell, mt0 + m, ln & 15, H);
      const int qq = ln >> 4;
      Frag fr = zero_frag();
      if (c < nch_u) {
        if (cr.w >= 0) fr = load_frag<BF16>(LY(W), Kin, cr.w, c * KC, qq, Kin, vec);
      } else {
        if (cr.r >= 0) fr = load_frag<BF16>(LY(R), H, cr.r, (c - nch_u) * KC, qq, H, vec);
      }
      lds_put(As + (long)(f >> 6) * 128, ln, fr);
    }
    __syncthreads();
  }

  // ---- per-wave tile bookkeeping
  bool mval[MW], nval[NW];
  int mloc[MW];
  int mblk[MW];   // LDS block row of M-tile i, clamped to a valid one (reads stay unconditional)
  long arow[MW];  // caller weight row this lane loads for M-tile i (streamed weights; clamped)
  uint32_t mw_[MW], mr_[MW];  // 0 where that row has no input / recurrent weights (streamed fragment zeroed)
  int unit[MW], bcol[NW];     // first unit of this lane's rows; batch column
  // B-operand (h, u) addressing.  A row-major source (x, h0, and every source
  // off the aligned path): lane offset row * K + q * KC/8, chunk stride KC,
  // half 1 at +KC/2.  A load-order source (the F buffers): lane offset
  // lane * EPH, column tile n's blocks from n * nch_part * FB, chunk stride FB,
  // half 1 at +FB/2 -- one load reads 1 KiB in one piece.
  constexpr int FB = 2048 / Dt<BF16>::SZ;  // elements of one 2 KiB fragment block
  constexpr int EPH = 16 / Dt<BF16>::SZ;   // elements of one lane's 16-byte half
  // row-major byte offsets of this lane's two halves in h and u (rows clamped
  // to valid ones; the planner keeps a slot below 4 GiB)
  uint32_t hrow0[NW], hrow1[NW], urow0[NW], urow1[NW];
  long boff[NW], uoff[NW];  // row-major element offsets of this lane's rows of h and u (!FRAG)
  int nlc[NW];              // column tile of j, clamped (wave-uniform)
  int fpos[MW];             // load-order position of this lane's unit in column tile 0
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    mloc[i] = gm + i * P.ntgm;
    mval[i] = i < P.mw && mloc[i] < mcnt;
    mblk[i] = min(mloc[i], mcnt - 1);
    const CellRow cr = cell_row(cell, mt0 + mloc[i], lane & 15, H);
    const long r = mval[i] ? (cr.w >= 0 ? cr.w : cr.r) : -1;  // LSTM, RNN: w == r; GRU n: one of them
    mw_[i] = (mval[i] && cr.w >= 0) ? 0xffffffffu : 0u;
    mr_[i] = (mval[i] && cr.r >= 0) ? 0xffffffffu : 0u;
    arow[i] = VEC ? (r >= 0 ? r : 0) : r;
    // LSTM / GRU: the lane's four rows are the four rows of unit 4*mt + q;
    // simple RNN: they are units 16*mt + 4*q + k, k = 0..3
    unit[i] = cell >= kCellRnnTanh ? 16 * (mt0 + mloc[i]) + 4 * q : 4 * (mt0 + mloc[i]) + q;
    // (the simple RNN's four units share one 16-byte group and follow it)
    const int kc = unit[i] % KC;
    fpos[i] = (unit[i] / KC) * FB + (kc / (KC / 2)) * (FB / 2) + (((kc % (KC / 2)) / EPH) * 16 + (lane & 15)) * EPH +
              kc % EPH;
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int nloc = gn + j * P.ntgn;
    nval[j] = j < P.nw && nloc < P.ncnt;
    bcol[j] = 16 * nloc + (lane & 15);
    nlc[j] = min(nloc, P.ncnt - 1);
    hrow0[j] = (uint32_t)(min(bcol[j], B - 1) * H + q * (KC / 8)) * (uint32_t)Dt<BF16>::SZ;
    hrow1[j] = hrow0[j] + (KC / 2) * Dt<BF16>::SZ;
    urow0[j] = (uint32_t)(min(bcol[j], B - 1) * Kin + q * (KC / 8)) * (uint32_t)Dt<BF16>::SZ;
    urow1[j] = urow0[j] + (KC / 2) * Dt<BF16>::SZ;
    boff[j] = (long)min(bcol[j], B - 1) * H;
    uoff[j] = (long)min(bcol[j], B - 1) * Kin;
  }
  auto fin = [&](int i, int j) { return ((i * P.nw + j) % ks) == kg; };
  // Branch-free MFMA chains on the aligned path with two waves per SIMD: a
  // tile the wave does not own (past the layer's last M-tile or column tile,
  // or beyond mw x nw when the instantiation rounds up) multiplies clamped
  // rows and its sum is never used.  Measured: the 4-layer fp32 H = 512
  // wavefront 1.297 -> 1.272 ms, the 8-layer bf16 H = 256 one 0.853 -> 0.835.
  // One wave per SIMD keeps the branches (the single-layer bf16 H = 1536
  // launch was 0.7% slower without them), and so does choosing between both
  // forms at run time (2-3% slower: the loop then carries both).
  constexpr bool dense = VEC && NWV == 8;
  auto live = [&](int i, int j) { return mval[i] && nval[j] && fin(i, j) && unit[i] < H && bcol[j] < B; };

  // per-lane state in registers, fp32: the LSTM's cell state c, the GRU's
  // previous h (for z * h_{t-1}); and the bias of fused-input layers
  float creg[MW][NW];
  f32x4 breg[MW];
  const T* bias = reinterpret_cast<const T*>(LY(bias));
  const T* h0p = reinterpret_cast<const T*>(LY(h0));
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    breg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (Kin && mval[i]) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int bi = cell_row(cell, mt0 + mloc[i], 4 * q + k, H).bi;
        if (bi >= 0) breg[i][k] = to_float(bias[bi]);
      }
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      creg[i][j] = 0.f;
      if (live(i, j)) {
        const long o = (long)bcol[j] * H + unit[i];
        if (cell == kCellLstm && LY(c0)) creg[i][j] = LY(c0)[o];
        if (cell == kCellGru && h0p) creg[i][j] = to_float(h0p[o]);
      }
    }
  }

  // optional phase trace of this workgroup (thread 0 writes wall-clock stamps)
  long long* trc = nullptr;
  if (P.trace && v % P.trace_stride == 0 && v / P.trace_stride < P.trace_wgs)
    trc = P.trace + (long)(v / P.trace_stride) * T_ * 8;
  auto stamp = [&](int t, int k) {
    if (trc && tid == 0) trc[t * 8 + k] = wall_clock64();
  };
  // shader-clock counter next to wall-clock stamps 0 and 2 (gives the core clock)
  auto stamp_clk = [&](int t, int k) {
    if (trc && tid == 0) trc[t * 8 + k] = clock64();
  };

  const T* Wp = reinterpret_cast<const T*>(LY(W));
  const T* Rp = reinterpret_cast<const T*>(LY(R));
  T* Xp = reinterpret_cast<T*>(LY(X));
  T* Fp = FRAG ? reinterpret_cast<T*>(LY(F)) : nullptr;
  const bool ufrag = FRAG && LY(ufrag);
  // u's byte offsets for the whole launch (u's layout is fixed)
  uint32_t ulo0[NW], ulo1[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    ulo0[j] = ufrag ? (uint32_t)(lane * 16) : urow0[j];
    ulo1[j] = ufrag ? (uint32_t)(lane * 16 + 1024) : urow1[j];
  }
  const T* Up = reinterpret_cast<const T*>(LY(U));
  const float* Gp = LY(G);
  // G offsets of this lane's tiles (clamped so every load is valid)
  long goff[MW][NW];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j)
      goff[i][j] = ((long)min(mt0 + mloc[i], P.Mt - 1) * B + min(bcol[j], B - 1)) * 16 + 4 * q;

  for (int t = 0; t < T_; ++t) {
    stamp(t, 0);
    stamp_clk(t, 6);
    // ---- hoisted pre-activations of this wave's tiles (do not depend on the wait)
    f32x4 gq[MW][NW];
    if (Gp) {
      const float* gt = Gp + (long)t * P.Mt * B * 16;
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j)  // (non-temporal: read once)
          gq[i][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gt + goff[i][j]));
    }

    // ---- wait for h^l_{t-1} (own layer) and h^{l-1}_t (producer in this launch)
    const int* own = (t > 0 && !sent) ? LY(flags) : nullptr;
    const int* dep = LY(dep_flags);
    if (own || dep) {
      if (wave == 0) {
        const bool ok = own ? wait_counts(own, LY(wg_count), t, dep, LY(dep_count), t + 1, P.err, P.timeout_ticks)
                            : wait_counts(dep, LY(dep_count), t + 1, nullptr, 0, 0, P.err, P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s_ok) return;
    }
    stamp(t, 1);

    f32x4 acc[MW][NW];
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int j = 0; j < NW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // h_{t-1}: the load-order buffer on the aligned path, else the row-major
    // slot; at t = 0 the caller's row-major h0 (null: zero, no h part)
    const bool hfrag = FRAG && t > 0;
    const T* hsrc = t > 0 ? (hfrag ? Fp + (long)(t - 1) * P.fslot : Xp + (long)(t - 1) * slot)
                          : reinterpret_cast<const T*>(LY(h0));
    const T* usrc = Kin ? Up + (long)t * LY(u_slot) : nullptr;
    uint32_t hlo0[NW], hlo1[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      hlo0[j] = hfrag ? (uint32_t)(lane * 16) : hrow0[j];
      hlo1[j] = hfrag ? (uint32_t)(lane * 16 + 1024) : hrow1[j];
    }

    Frag rb[PD][NW];
    Frag ra[STREAM ? PD : 1][MW];
    // loads of chunk c (c < nch_u: input part, else recurrent part)
    auto issue = [&](Frag (&b)[NW], Frag (&a)[MW], int c) {
      const bool is_u = c < nch_u;
      const int Kseg = is_u ? Kin : H;
      const int kk = (is_u ? c : c - nch_u) * KC;  // first column of the chunk
      const T* bsrc = is_u ? usrc : hsrc;
      const T* asrc = is_u ? Wp : Rp;
      if (VEC && !FRAG) {
#pragma unroll
        for (int j = 0; j < NW; ++j) b[j] = load_frag_vec<BF16>(bsrc + (is_u ? uoff[j] : boff[j]) + kk, q);
      } else if (VEC) {
        // a wave-uniform base per column tile plus per-lane byte offsets, so
        // each half is one 16-byte load (base in scalar registers)
        const bool fr = is_u ? ufrag : hfrag;
        const int cc = is_u ? c : c - nch_u;
        const int npart = is_u ? nch_u : nch_h;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          const char* pj = reinterpret_cast<const char*>(bsrc + (fr ? (long)(nlc[j] * npart + cc) * FB : (long)kk));
          const uint32_t o0 = is_u ? ulo0[j] : hlo0[j], o1 = is_u ? ulo1[j] : hlo1[j];
          b[j].v[0] = *reinterpret_cast<const uint4*>(pj + o0);
          b[j].v[1] = *reinterpret_cast<const uint4*>(pj + o1);
        }
      }
      if (VEC) {
        if (STREAM) {
#pragma unroll
          for (int i = 0; i < MW; ++i) {
            a[i] = load_frag_vec<BF16>(asrc + arow[i] * Kseg + kk, q);
            frag_mask(a[i], is_u ? mw_[i] : mr_[i]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NW; ++j)
          if (nval[j]) b[j] = bcol[j] < B ? load_frag_off<BF16>(bsrc, (long)bcol[j] * Kseg, kk, q, Kseg, false) : zero_frag();
        if (STREAM) {
#pragma unroll
          for (int i = 0; i < MW; ++i)
            if (mval[i]) {
              a[i] = arow[i] >= 0 ? load_frag<BF16>(asrc, Kseg, arow[i], kk, q, Kseg, false) : zero_frag();
              frag_mask(a[i], is_u ? mw_[i] : mr_[i]);
            }
        }
      }
    };
    // this wave's chunks of one part: c = c0 + ci * ks for ci < n
    auto products = [&](int c0, int n) {
      // Weight fragments from LDS are read one chunk ahead into the other of
      // two buffers (chunk ci uses al[ci & 1], and ci & 1 == s & 1 because PD
      // is even), so their latency hides behind the MFMAs and nothing is copied.
      // The reads are unconditional (clamped tile rows): with no branch around
      // them the compiler's LDS wait counts stay exact instead of draining.
      Frag al[STREAM ? 1 : 2][MW];
      auto lds_a = [&](Frag (&dst)[MW], int ci) {
        const int c = c0 + min(ci, n - 1) * ks;
#pragma unroll
        for (int i = 0; i < MW; ++i) dst[i] = lds_get(As + (mblk[i] * nch + c) * 128, lane);
      };
      auto compute = [&](int s, int ci) {
        if (!STREAM) lds_a(al[STREAM ? 0 : ((s + 1) & 1)], ci + 1);
        Frag (&a)[MW] = STREAM ? ra[STREAM ? s : 0] : al[STREAM ? 0 : (s & 1)];
        if (dense) {
          // every tile of the instantiation is one of the wave's (a tile past
          // the layer's last M-tile multiplies clamped rows; its sum is never
          // used): no branch between the MFMA chains
#pragma unroll
          for (int i = 0; i < MW; ++i)
#pragma unroll
            for (int j = 0; j < NW; ++j) mfma_frag<BF16>(acc[i][j], a[i], rb[s][j]);
        } else {
#pragma unroll
          for (int i = 0; i < MW; ++i)
#pragma unroll
            for (int j = 0; j < NW; ++j)
              if (mval[i] && nval[j]) mfma_frag<BF16>(acc[i][j], a[i], rb[s][j]);
        }
      };
      if (n > 0 && n <= PD) {
        // burst: every chunk of this wave in flight at once
#pragma unroll
        for (int s = 0; s < PD; ++s) issue(rb[s], ra[STREAM ? s : 0], c0 + min(s, n - 1) * ks);
        if (!STREAM) lds_a(al[0], 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < PD; ++s)
          if (s < n) compute(s, s);
      } else if (n > PD) {
        // ring: every issue is unconditional (chunk index clamped to the last one)
        // and the loop runs to a multiple of PD, so the load stream has no
        // branches; only the MFMAs of the padded tail are skipped.  The
        // scheduling barriers keep each refill where it is written instead of
        // next to its use.
        const int n_pad = (n + PD - 1) / PD * PD;
#pragma unroll
        for (int s = 0; s < PD; ++s) issue(rb[s], ra[STREAM ? s : 0], c0 + s * ks);
        if (!STREAM) lds_a(al[0], 0);
        __builtin_amdgcn_sched_barrier(0);
        for (int i0 = 0; i0 < n_pad; i0 += PD) {
#pragma unroll
          for (int s = 0; s < PD; ++s) {
            const int ci = i0 + s;
            if (ci < n) compute(s, ci);
            issue(rb[s], ra[STREAM ? s : 0], c0 + min(ci + PD, n - 1) * ks);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };

    // a null h_{t-1} (t = 0 without h0) is zero: only the input chunks remain
    const int c_end = hsrc ? nch : nch_u;
    if (kSentCode && sent && t > 0) {
      // this wave's chunks c = kg + s * ks, s < n (n <= PD), re-read until
      // every element of every one has been written, then multiplied
      const int n = nch > kg ? (nch - kg + ks - 1) / ks : 0;
      Frag hb[PD][NW];
      if (n > 0) {
        const long long t0 = wall_clock64();
        const __amdgpu_buffer_rsrc_t hb_rsrc = raw_buffer(hsrc, (int)(slot * (long)sizeof(T)));
        while (true) {
#pragma unroll
          for (int s = 0; s < PD; ++s)
            if (s < n) {
              const int c = kg + s * ks;
#pragma unroll
              for (int j = 0; j < NW; ++j) {
                const int e = (int)boff[j] + c * KC;  // element offset of the chunk in this lane's row
                hb[s][j].v[0] = load16_coherent(hb_rsrc, (e + frag_col<BF16>(q, 0)) * (int)sizeof(T));
                hb[s][j].v[1] = load16_coherent(hb_rsrc, (e + frag_col<BF16>(q, 1)) * (int)sizeof(T));
              }
            }
          int ok = 1;
#pragma unroll
          for (int s = 0; s < PD; ++s)
            if (s < n) {
#pragma unroll
              for (int j = 0; j < NW; ++j) ok &= written16<BF16>(hb[s][j].v[0]) & written16<BF16>(hb[s][j].v[1]);
            }
          if (__all(ok)) break;
          if (__hip_atomic_load(P.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
              wall_clock64() - t0 > P.timeout_ticks) {
            // give up: the workgroup leaves together after the combine barrier
            if (lane == 0) {
              __hip_atomic_store(P.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              s_abort[t & 1] = 1;
            }
            break;
          }
        }
#pragma unroll
        for (int s = 0; s < PD; ++s)
          if (s < n) {
            const int c = kg + s * ks;
            Frag a[MW];
#pragma unroll
            for (int i = 0; i < MW; ++i) a[i] = lds_get(As + (mblk[i] * nch + c) * 128, lane);
#pragma unroll
            for (int i = 0; i < MW; ++i)
#pragma unroll
              for (int j = 0; j < NW; ++j)
                if (mval[i] && nval[j]) mfma_frag<BF16>(acc[i][j], a[i], hb[s][j]);
          }
      }
    } else {
      products(kg, c_end > kg ? (c_end - kg + ks - 1) / ks : 0);
    }
    stamp(t, 2);
    stamp_clk(t, 7);

    // ---- combine the K-split partial sums: tile e is finalised by K-group
    // e % ks; every other K-group of its tile group leaves one partial in LDS
    if (ks > 1) {
      f32x4* red = reinterpret_cast<f32x4*>(smem + P.red_off + (sent ? (t & 1) * P.red_stride : 0));
      const int tpg = P.mw * P.nw;
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          if (!(mval[i] && nval[j]) || fin(i, j)) continue;
          const int e = i * P.nw + j;
          const int f = e % ks;
          const int slot_r = kg < f ? kg : kg - 1;
          red[((tg * tpg + e) * (ks - 1) + slot_r) * 64 + lane] = acc[i][j];
        }
      __syncthreads();
      if (sent && s_abort[t & 1]) return;
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          if (!(mval[i] && nval[j]) || !fin(i, j)) continue;
          const int e = i * P.nw + j;
          for (int r = 0; r < ks - 1; ++r) acc[i][j] += red[((tg * tpg + e) * (ks - 1) + r) * 64 + lane];
        }
    }
    stamp(t, 3);

    // ---- gates, cell update, outputs
    // the exchange: the load-order buffer (plus the row-major copy when a
    // later input GEMM reads it), else the row-major slot itself
    T* fout = Fp ? Fp + (long)t * P.fslot : nullptr;
    T* xout = FRAG ? (Xp ? Xp + (long)t * slot : nullptr) : Xp + (long)t * slot;
    T* yout = LY(Yout) ? reinterpret_cast<T*>(LY(Yout)) + (long)t * B * H : nullptr;
    const bool last = (t == T_ - 1);
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        if (!live(i, j)) continue;
        const f32x4 p = acc[i][j] + (Gp ? gq[i][j] : breg[i]);
        const long o = (long)bcol[j] * H + unit[i];
        // the exchange (write-through) and, beside a load-order exchange, the
        // row-major copy a later input GEMM reads
        T* const dst = FRAG ? fout + (long)(bcol[j] >> 4) * nch_h * FB + fpos[i] : xout + o;
        T* const cpy = FRAG ? xout : nullptr;
        auto emit = [&](int k, float h) {  // h_t to the exchange, y and (last step) hT
          const T hv = sent ? canon_nan<BF16>(from_float<BF16>(h)) : from_float<BF16>(h);
          store_coherent<BF16>(dst + k, hv);
          if (cpy) cpy[o + k] = hv;
          if (yout) yout[o + k] = hv;
          if (last && LY(hT)) reinterpret_cast<T*>(LY(hT))[o + k] = hv;
          if (LY(save_h)) reinterpret_cast<T*>(LY(save_h))[(long)t * B * H + o + k] = hv;
        };
        cell_update(cell, p, creg[i][j], H - unit[i], emit);
        if (cell == kCellLstm && last && LY(cT)) LY(cT)[o] = creg[i][j];
        if (cell == kCellLstm && LY(save_gates)) save_lstm_step(LY(save_gates), LY(save_c), p, creg[i][j], t, B, H, bcol[j], unit[i]);
      }
    stamp(t, 4);

    // ---- publish step t: stores complete, then the step counter (the
    // data-valid exchange publishes by the stores themselves)
    if (!sent) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(LY(flags) + (long)wl * kFlagStride, t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    stamp(t, 5);
  }
#undef LY
}

}  // namespace lstm
