// Device kernels of the stacked-LSTM forward pass for gfx950 (CDNA4).
//
//  * lstm_input_gemm: the grouped input projection for all timesteps at once,
//    G = W_l [u_1 .. u_T] + b_l over the four gates ("Optimizing Performance of
//    Recurrent Neural Networks on GPUs", proposed method: gate grouping, and
//    the input-weight product being independent of the recurrence).  MFMA,
//    LDS-staged operands, fp32 output in the tile layout the recurrence reads.
//
//  * lstm_rec_kernel: the recurrence.  One cooperative launch runs all T steps
//    ("Persistent RNNs: Stashing Recurrent Weights On-Chip": one launch for the
//    whole sequence, weights kept on chip across steps).  Each workgroup owns a
//    set of hidden units of one layer (all four gate rows of each), keeps its
//    weight rows in LDS when they fit, computes R_l h_{t-1} (plus W_l u_t when
//    the input product is not hoisted) with MFMA, and applies the gate
//    non-linearities and the fp32 cell update in registers.  Several layers can
//    share one launch: layer l+1 consumes layer l's step t as soon as it is
//    published, so layer l step t runs beside layer l+1 step t-1 (first page,
//    proposed method: overlapping layers).  Steps are ordered with per-workgroup
//    step counters (agent-scope release/acquire), polled with a time limit so a
//    wait can never hang.
#include "lstm_common.h"
#include "lstm_params.h"

namespace lstm {

// ----------------------------------------------------------------------------
// Input projection GEMM
// ----------------------------------------------------------------------------
template <bool BF16>
__global__ void __launch_bounds__(kGemmThreads) lstm_input_gemm(const GemmParams P) {
  constexpr int KC = Dt<BF16>::KC;
  constexpr int FQ = KC / 4;
  __shared__ Frag As[8 * 64];
  __shared__ Frag Bs[8 * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (P.zero_ptr && blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = tid; i < P.zero_count; i += kGemmThreads) P.zero_ptr[i] = 0;
  }
  const int mtb = blockIdx.y * 8;             // first M-tile of this workgroup
  const int n0 = blockIdx.x * kGemmTileN;     // first column
  const int nch = (P.K + KC - 1) / KC;
  const bool vw = P.vec_ok_w, vu = P.vec_ok_u;

  // per-thread staging slots: 2 A fragments and 2 B fragments per chunk
  long arow[2];
  long bcol[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int f = tid + s * kGemmThreads;
    const int ln = f & 63;
    const int mtl = f >> 6;
    arow[s] = (mtb + mtl < P.Mt) ? tile_row(mtb + mtl, ln & 15, P.H) : -1;
    const long col = n0 + 16 * mtl + (ln & 15);
    bcol[s] = col < P.N ? col : -1;
  }
  const int q = lane >> 4;  // same for f = tid and f = tid + 256 (256 is a multiple of 64)

  Frag ra[2], rb[2];
  auto fetch = [&](int c) {
    const int k0 = c * KC + q * FQ;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      ra[s] = arow[s] >= 0 ? load_frag<BF16>(P.W, P.K, arow[s], k0, P.K, vw) : zero_frag();
      rb[s] = bcol[s] >= 0 ? load_frag<BF16>(P.U, P.K, bcol[s], k0, P.K, vu) : zero_frag();
    }
  };

  const int wm = wave & 1, wn = wave >> 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nch > 0) fetch(0);
  for (int c = 0; c < nch; ++c) {
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      As[tid + s * kGemmThreads] = ra[s];
      Bs[tid + s * kGemmThreads] = rb[s];
    }
    __syncthreads();
    if (c + 1 < nch) fetch(c + 1);
    Frag a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = As[(4 * wm + i) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = Bs[(4 * wn + j) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_frag<BF16>(acc[i][j], a[i], b[j]);
  }

  // epilogue: add bias, write [T][Mt][B][16]
  typedef typename Dt<BF16>::T T;
  const T* bias = reinterpret_cast<const T*>(P.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mt = mtb + 4 * wm + i;
    const int unit = 4 * mt + (lane >> 4);
    if (mt >= P.Mt || unit >= P.H) continue;
    f32x4 bv;
    bv[0] = to_float(bias[0 * P.H + unit]);
    bv[1] = to_float(bias[1 * P.H + unit]);
    bv[2] = to_float(bias[2 * P.H + unit]);
    bv[3] = to_float(bias[3 * P.H + unit]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long col = n0 + 16 * (4 * wn + j) + (lane & 15);
      if (col >= P.N) continue;
      const long t = col / P.B, bb = col % P.B;
      float* dst = P.G + ((t * P.Mt + mt) * P.B + bb) * 16 + 4 * (lane >> 4);
      *reinterpret_cast<f32x4*>(dst) = acc[i][j] + bv;
    }
  }
}

// ----------------------------------------------------------------------------
// Step ordering
// ----------------------------------------------------------------------------
// Executed by one whole wave: true once every counter in flags[0..count) is
// >= target.  False if another workgroup already reported an error, or if the
// wait exceeds `timeout` wall-clock ticks (then it reports the error itself).
__device__ bool wait_counts(const int* flags, int count, int target, int* err, long long timeout) {
  const int lane = threadIdx.x & 63;
  const long long start = wall_clock64();
  while (true) {
    int ok = 1;
    for (int i = lane; i < count; i += 64) {
      const int v = __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok &= (v >= target) ? 1 : 0;
    }
    if (__all(ok)) return true;
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    if (wall_clock64() - start > timeout) {
      if (lane == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ----------------------------------------------------------------------------
// Persistent recurrence (optionally several layers as a wavefront)
// ----------------------------------------------------------------------------
// Waves: wave w -> K-group w % KS, tile group w / KS.  The KS waves of a tile
// group split the K chunks of the same output tiles and combine them through
// LDS; tile group g covers M-tiles g%ntgm (+ntgm ...) and column tiles
// g/ntgm (+ntgn ...).
template <bool BF16, int KS>
__global__ void __launch_bounds__(kRecThreads) lstm_rec_kernel(const RecParams P) {
  typedef typename Dt<BF16>::T T;
  constexpr int KC = Dt<BF16>::KC;
  constexpr int FQ = KC / 4;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_ok;

  const int bid = blockIdx.x;
  const int v = P.xcd_remap ? ((bid & 7) * (P.grid >> 3) + (bid >> 3)) : bid;
  RecLayer Ly;
  int found = 0;
#pragma unroll
  for (int i = 0; i < kMaxLayersPerLaunch; ++i) {
    if (i < P.nlayers && v >= P.layer[i].wg_begin && v < P.layer[i].wg_begin + P.layer[i].wg_count) {
      Ly = P.layer[i];
      found = 1;
    }
  }
  if (!found) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave % KS, tg = wave / KS;
  const int gm = tg % P.ntgm, gn = tg / P.ntgm;
  const int wl = v - Ly.wg_begin;
  const int mt0 = wl * Ly.mt_per_wg;
  const int mcnt = min(Ly.mt_per_wg, P.Mt - mt0);
  const int H = P.H, B = P.B, T_ = P.T, Kin = Ly.Kin;
  const int nch_u = (Kin + KC - 1) / KC;
  const int nch_h = (H + KC - 1) / KC;
  const int nch = nch_u + nch_h;
  const bool vec = Ly.vec_ok;
  const int q = lane >> 4;
  Frag* As = reinterpret_cast<Frag*>(smem);

  // ---- keep this workgroup's weight rows on chip for the whole sequence
  if (Ly.staged) {
    const int total = mcnt * nch * 64;
    for (int f = tid; f < total; f += kRecThreads) {
      const int ln = f & 63;
      const int c = (f >> 6) % nch;
      const int m = (f >> 6) / nch;
      const long row = tile_row(mt0 + m, ln & 15, H);
      const int qq = ln >> 4;
      Frag fr = zero_frag();
      if (row >= 0) {
        if (c < nch_u)
          fr = load_frag<BF16>(Ly.W, Kin, row, c * KC + qq * FQ, Kin, vec);
        else
          fr = load_frag<BF16>(Ly.R, H, row, (c - nch_u) * KC + qq * FQ, H, vec);
      }
      As[f] = fr;
    }
    __syncthreads();
  }

  // ---- per-wave tile bookkeeping
  bool mval[4], nval[4];
  int mloc[4], nloc[4];
  long arow[4];  // caller weight row this lane loads for M-tile i (streamed weights)
  int unit[4], bcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mloc[i] = gm + i * P.ntgm;
    mval[i] = mloc[i] < mcnt;
    arow[i] = mval[i] ? tile_row(mt0 + mloc[i], lane & 15, H) : -1;
    unit[i] = 4 * (mt0 + mloc[i]) + q;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    nloc[j] = gn + j * P.ntgn;
    nval[j] = nloc[j] < P.ncnt;
    bcol[j] = 16 * nloc[j] + (lane & 15);
  }
  auto fin = [&](int i, int j) { return ((i * P.nw + j) % KS) == kg; };

  // cell state (fp32, registers) and bias of fused-input layers
  float creg[4][4];
  f32x4 breg[4];
  const T* bias = reinterpret_cast<const T*>(Ly.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    breg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (Kin && mval[i] && unit[i] < H) {
#pragma unroll
      for (int k = 0; k < 4; ++k) breg[i][k] = to_float(bias[k * H + unit[i]]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      creg[i][j] = 0.f;
      if (Ly.c0 && mval[i] && nval[j] && unit[i] < H && bcol[j] < B) creg[i][j] = Ly.c0[(long)bcol[j] * H + unit[i]];
    }
  }

  const T* Wp = reinterpret_cast<const T*>(Ly.W);
  const T* Rp = reinterpret_cast<const T*>(Ly.R);
  T* Yp = reinterpret_cast<T*>(Ly.Y);

  for (int t = 0; t < T_; ++t) {
    // ---- wait for h^l_{t-1} (own layer) and h^{l-1}_t (producer in this launch)
    const bool need_own = t > 0;
    const bool need_dep = Ly.dep_flags != nullptr;
    if (need_own || need_dep) {
      if (wave == 0) {
        bool ok = true;
        if (need_own) ok = wait_counts(Ly.flags, Ly.wg_count, t, P.err, P.timeout_ticks);
        if (ok && need_dep) ok = wait_counts(Ly.dep_flags, Ly.dep_count, t + 1, P.err, P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
      if (!s_ok) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }

    // ---- hoisted pre-activations for the tiles this wave finalises (issued early)
    f32x4 gq[4][4];
    if (Ly.G) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          gq[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (mval[i] && nval[j] && fin(i, j) && unit[i] < H && bcol[j] < B)
            gq[i][j] = *reinterpret_cast<const f32x4*>(
                Ly.G + (((long)t * P.Mt + mt0 + mloc[i]) * B + bcol[j]) * 16 + 4 * q);
        }
    }

    // ---- grouped products: [W_l | R_l] (rows of this workgroup) x [u_t ; h_{t-1}]
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const T* hsrc = t > 0 ? Yp + (long)(t - 1) * B * H : reinterpret_cast<const T*>(Ly.h0);
    const T* usrc = Kin ? reinterpret_cast<const T*>(Ly.U) + (long)t * B * Kin : nullptr;
    const int c_end = hsrc ? nch : nch_u;
    for (int c = kg; c < c_end; c += KS) {
      const bool is_u = c < nch_u;
      const int Kseg = is_u ? Kin : H;
      const int k0 = (is_u ? c : c - nch_u) * KC + q * FQ;
      const T* bsrc = is_u ? usrc : hsrc;
      Frag a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!mval[i]) continue;
        if (Ly.staged)
          a[i] = As[(mloc[i] * nch + c) * 64 + lane];
        else
          a[i] = arow[i] >= 0 ? load_frag<BF16>(is_u ? (const void*)Wp : (const void*)Rp, Kseg, arow[i], k0, Kseg, vec)
                              : zero_frag();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!nval[j]) continue;
        b[j] = bcol[j] < B ? load_frag<BF16>(bsrc, Kseg, bcol[j], k0, Kseg, vec) : zero_frag();
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (mval[i] && nval[j]) mfma_frag<BF16>(acc[i][j], a[i], b[j]);
    }

    // ---- combine the K-split partial sums
    if (KS > 1) {
      f32x4* red = reinterpret_cast<f32x4*>(smem + P.red_off);
      const int tpg = P.mw * P.nw;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!(mval[i] && nval[j]) || fin(i, j)) continue;
          const int e = i * P.nw + j;
          red[((tg * tpg + e) * KS + kg) * 64 + lane] = acc[i][j];
        }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!(mval[i] && nval[j]) || !fin(i, j)) continue;
          const int e = i * P.nw + j;
#pragma unroll
          for (int k2 = 0; k2 < KS; ++k2)
            if (k2 != kg) acc[i][j] += red[((tg * tpg + e) * KS + k2) * 64 + lane];
        }
    }

    // ---- gates, cell update, outputs
    T* yout = Yp + (long)t * B * H;
    const bool last = (t == T_ - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!(mval[i] && nval[j]) || !fin(i, j)) continue;
        if (unit[i] >= H || bcol[j] >= B) continue;
        const f32x4 p = acc[i][j] + (Ly.G ? gq[i][j] : breg[i]);
        const float ig = sigmoid_f(p[0]);
        const float fg = sigmoid_f(p[1]);
        const float gg = tanh_f(p[2]);
        const float og = sigmoid_f(p[3]);
        const float cn = fg * creg[i][j] + ig * gg;
        creg[i][j] = cn;
        const T hv = from_float<BF16>(og * tanh_f(cn));
        const long o = (long)bcol[j] * H + unit[i];
        yout[o] = hv;
        if (last) {
          if (Ly.hT) reinterpret_cast<T*>(Ly.hT)[o] = hv;
          if (Ly.cT) Ly.cT[o] = cn;
        }
      }

    // ---- publish step t
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(Ly.flags + wl, t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ----------------------------------------------------------------------------
// Host-side launchers (the only code outside this file that touches the kernels)
// ----------------------------------------------------------------------------
namespace {
template <bool BF16>
const void* rec_fn(int ks) {
  if (ks == 1) return reinterpret_cast<const void*>(&lstm_rec_kernel<BF16, 1>);
  if (ks == 2) return reinterpret_cast<const void*>(&lstm_rec_kernel<BF16, 2>);
  return reinterpret_cast<const void*>(&lstm_rec_kernel<BF16, 4>);
}
const void* rec_kernel_fn(bool bf16, int ks) { return bf16 ? rec_fn<true>(ks) : rec_fn<false>(ks); }
}  // namespace

hipError_t launch_input_gemm(bool bf16, const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.N + kGemmTileN - 1) / kGemmTileN, (p.Mt + 7) / 8);
  if (bf16)
    hipLaunchKernelGGL(lstm_input_gemm<true>, grid, dim3(kGemmThreads), 0, s, p);
  else
    hipLaunchKernelGGL(lstm_input_gemm<false>, grid, dim3(kGemmThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t rec_prepare(bool bf16, int ks, int lds_bytes, int* max_blocks_per_cu) {
  const void* fn = rec_kernel_fn(bf16, ks);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(max_blocks_per_cu, fn, kRecThreads, lds_bytes);
}

hipError_t launch_rec(bool bf16, int ks, const RecParams& p, int lds_bytes, hipStream_t s) {
  const void* fn = rec_kernel_fn(bf16, ks);
  void* args[] = {const_cast<RecParams*>(&p)};
  return hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kRecThreads), args, (unsigned)lds_bytes, s);
}

}  // namespace lstm
