// Backward pass (backpropagation through time) of the stacked LSTM for
// gfx950: kernels and the lstm_bwd entry point (include/lstm_bwd.h).
//
// Per layer, from the top:
//   1. the recurrent chain, strictly serial in t: for t = T-1 .. 0 an
//      elementwise kernel turns dh = dY[t] + dh_rec and dc_rec into the gate
//      derivatives dp_t (fp32, and a copy in the workload's dtype) and the next
//      dc_rec; then dh_rec = dp_t R_l, an MFMA product over K = 4H split across
//      workgroups so it fills the GPU (the K-split partial sums are added by the
//      next step's elementwise kernel, in a fixed order);
//   2. once every step's dp is known, the weight and input gradients as single
//      MFMA products over all T*B columns -- dW_l = dP^T U, dR_l = dP^T H_prev,
//      dU = dP W_l ("Optimizing Performance of Recurrent Neural Networks on
//      GPUs", proposed method: the weight update as one large product) -- and
//      db_l as column sums of dP.
// Products take operands in the workload's dtype (bf16 or fp32) with fp32
// accumulation; both operands of every product are laid out K-contiguous by
// LDS-tiled transposes, so each lane's fragment is two 16-byte loads.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "lstm_bwd.h"  // include/ is on the include path
#include "lstm_common.h"
#include "lstm_params.h"

namespace lstm {
namespace {

constexpr int kBwdThreads = 256;

template <typename D>
__device__ __forceinline__ D to_dt(float v);
template <>
__device__ __forceinline__ float to_dt<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_dt<uint16_t>(float v) { return f32_to_bf16(v); }

// dst[c][r] = row r of the source, element c, for r < rows, c < cols, where
// row r is first[r] (r < nfirst; zeros when first is null) or main[r - nfirst].
template <typename S, typename D>
__global__ void __launch_bounds__(kBwdThreads) bwd_transpose(const S* main, long ldm, const S* first, long ldf,
                                                            int nfirst, int rows, int cols, D* dst, long ldd) {
  __shared__ float tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = r0 + ty + 4 * k, c = c0 + tx;
    float v = 0.f;
    if (r < rows && c < cols) {
      if (r < nfirst)
        v = first ? to_float(first[(long)r * ldf + c]) : 0.f;
      else
        v = to_float(main[(long)(r - nfirst) * ldm + c]);
    }
    tile[ty + 4 * k][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = c0 + ty + 4 * k, r = r0 + tx;
    if (r < rows && c < cols) dst[(long)c * ldd + r] = to_dt<D>(tile[tx][ty + 4 * k]);
  }
}

// C[m][n] = sum over k of A[m][k] B[n][k] (fp32 accumulation), both operands
// K-contiguous rows.  Workgroup tile (32 WM) x (32 WN): 4 waves in a 2 x 2
// grid, each WM x WN MFMA tiles of 16 x 16.  blockIdx.z = K split z takes
// chunks [z cps, (z+1) cps) and writes its partial sums at C + z * split_stride.
template <bool BF16, int WM, int WN>
__global__ void __launch_bounds__(kBwdThreads) bwd_gemm_nt(const void* A, long lda, const void* Bm, long ldb, float* C,
                                                          long ldc, long split_stride, int M, int N, int K, int cps,
                                                          int vec) {
  typedef typename Dt<BF16>::T T;
  constexpr int KC = Dt<BF16>::KC;
  const int lane = threadIdx.x & 63, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.y * 32 * WM + 16 * WM * wm, n0 = blockIdx.x * 32 * WN + 16 * WN * wn;
  const int nch = (K + KC - 1) / KC;
  const int cb = blockIdx.z * cps, ce = min(nch, cb + cps);
  const T* Ap = reinterpret_cast<const T*>(A);
  const T* Bp = reinterpret_cast<const T*>(Bm);
  long aoff[WM], boff[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) aoff[i] = (long)min(m0 + 16 * i + (lane & 15), M - 1) * lda;
#pragma unroll
  for (int j = 0; j < WN; ++j) boff[j] = (long)min(n0 + 16 * j + (lane & 15), N - 1) * ldb;
  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag a[2][WM], b[2][WN];
  auto load = [&](int s, int c) {
#pragma unroll
    for (int i = 0; i < WM; ++i) a[s][i] = load_frag_off<BF16>(Ap, aoff[i], c * KC, q, K, vec != 0);
#pragma unroll
    for (int j = 0; j < WN; ++j) b[s][j] = load_frag_off<BF16>(Bp, boff[j], c * KC, q, K, vec != 0);
  };
  if (cb < ce) load(0, cb);
  for (int c = cb; c < ce; ++c) {
    const int s = (c - cb) & 1;
    if (c + 1 < ce) load(s ^ 1, c + 1);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) mfma_frag<BF16>(acc[i][j], a[s][i], b[s][j]);
  }
  float* Cz = C + (long)blockIdx.z * split_stride;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int col = n0 + 16 * j + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 16 * i + 4 * q + r;
        if (row < M) Cz[(long)row * ldc + col] = acc[i][j][r];
      }
    }
}

struct StepArgs {
  const float* dY;      // [B][H] gradient reaching h_t from above (dy, or the upper layer's dU)
  const float* dhp;     // [S][B][H] K-split partials of dh_rec (null at the last step)
  long sstride;
  int S;
  const float* dhT;     // [B][H] or null: dh_rec at the last step
  const float* dcT;     // [B][H] or null: dc_rec at the last step
  const float* gates;   // [B][4H] activated gates of step t
  const float* c_t;     // [B][H]
  const float* c_prev;  // [B][H] or null (zeros)
  float* dcrec;         // [B][H] in: dc_rec of step t+1; out: dc f
  float* dP;            // [B][4H] fp32 gate derivatives of step t
  void* dPh;            // [B][4H] the same in the workload's dtype
  float* dc0;           // [B][H] or null: written at step 0
  int B, H, last;
};

// One step of the recurrent chain for every (sequence, unit).
template <bool BF16>
__global__ void __launch_bounds__(kBwdThreads) bwd_step(const StepArgs a) {
  typedef typename Dt<BF16>::T T;
  const long n = (long)a.B * a.H;
  for (long idx = (long)blockIdx.x * kBwdThreads + threadIdx.x; idx < n; idx += (long)gridDim.x * kBwdThreads) {
    const int bb = (int)(idx / a.H), j = (int)(idx % a.H);
    float dh = a.dY ? a.dY[idx] : 0.f;
    float dcr;
    if (a.last) {
      dh += a.dhT ? a.dhT[idx] : 0.f;
      dcr = a.dcT ? a.dcT[idx] : 0.f;
    } else {
      float s = 0.f;
      for (int z = 0; z < a.S; ++z) s += a.dhp[z * a.sstride + idx];
      dh += s;
      dcr = a.dcrec[idx];
    }
    const float* g = a.gates + (long)bb * 4 * a.H + j;
    const float ig = g[0], fg = g[a.H], gg = g[2L * a.H], og = g[3L * a.H];
    const float ct = a.c_t[idx], cp = a.c_prev ? a.c_prev[idx] : 0.f;
    const float tc = tanhf(ct);
    const float dc = dh * og * (1.f - tc * tc) + dcr;
    const float d[4] = {dc * gg * ig * (1.f - ig), dc * cp * fg * (1.f - fg), dc * ig * (1.f - gg * gg),
                        dh * tc * og * (1.f - og)};
    float* dp = a.dP + (long)bb * 4 * a.H + j;
    T* dph = reinterpret_cast<T*>(a.dPh) + (long)bb * 4 * a.H + j;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      dp[(long)k * a.H] = d[k];
      dph[(long)k * a.H] = from_float<BF16>(d[k]);
    }
    const float dcn = dc * fg;
    a.dcrec[idx] = dcn;
    if (a.dc0) a.dc0[idx] = dcn;
  }
}

// db[k] = sum over the rows r < rows of dP[r][k] (in row order).
__global__ void __launch_bounds__(kBwdThreads) bwd_colsum(const float* dP, int rows, int cols, float* db) {
  const int k = blockIdx.x * kBwdThreads + threadIdx.x;
  if (k >= cols) return;
  float s = 0.f;
  for (int r = 0; r < rows; ++r) s += dP[(long)r * cols + k];
  db[k] = s;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t rt, wt, dp, dph, dpt, ut, ht, dy0, dy1, dhp, dcrec, total;
  int S;  // K splits of the per-step product
};

constexpr int kStepWM = 1, kStepWN = 4;  // per-step product tile: 32 x 128
constexpr int kBigWM = 2, kBigWN = 2;    // weight-gradient products: 64 x 64

// K splits of the per-step product: enough workgroups to fill 256 CUs.  The
// count returned is the one the launch makes (chunks per split rounded up),
// which the step kernel sums.
int step_splits(int B, int H, int K, bool bf16) {
  const int blocks = ((B + 32 * kStepWM - 1) / (32 * kStepWM)) * ((H + 32 * kStepWN - 1) / (32 * kStepWN));
  const int nch = (K + (bf16 ? 64 : 32) - 1) / (bf16 ? 64 : 32);
  const int want = std::max(1, std::min(nch, 256 / std::max(1, blocks)));
  const int cps = (nch + want - 1) / want;
  return (nch + cps - 1) / cps;
}

bool bwd_layout(const lstm_desc_t* d, BwdLayout* o) {
  if (!d || d->cell != LSTM_CELL_LSTM || lstm_fwd_workspace_size(d) == 0) return false;
  const size_t s = d->dtype == LSTM_BF16 ? 2 : 4;
  const size_t H = d->H, B = d->B, TB = (size_t)d->T * d->B, G = 4 * H;
  const size_t Imax = std::max<size_t>(d->I, H);
  o->S = step_splits(d->B, d->H, 4 * d->H, d->dtype == LSTM_BF16);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  o->rt = take(H * G * s);
  o->wt = take(Imax * G * s);
  o->dp = take(TB * G * 4);
  o->dph = take(TB * G * s);
  o->dpt = take(G * TB * s);
  o->ut = take(Imax * TB * s);
  o->ht = take(H * TB * s);
  o->dy0 = take(TB * H * 4);
  o->dy1 = take(TB * H * 4);
  o->dhp = take((size_t)o->S * B * H * 4);
  o->dcrec = take(B * H * 4);
  o->total = off;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool BF16>
hipError_t transpose(const void* main, long ldm, const void* first, long ldf, int nfirst, int rows, int cols, void* dst,
                     long ldd, hipStream_t s) {
  typedef typename Dt<BF16>::T T;
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  hipLaunchKernelGGL((bwd_transpose<T, T>), grid, dim3(kBwdThreads), 0, s, static_cast<const T*>(main), ldm,
                     static_cast<const T*>(first), ldf, nfirst, rows, cols, static_cast<T*>(dst), ldd);
  return hipGetLastError();
}

template <bool BF16, int WM, int WN>
hipError_t gemm_nt(const void* A, long lda, const void* Bm, long ldb, float* C, long ldc, long split_stride, int M,
                   int N, int K, int splits, hipStream_t s) {
  const int KC = BF16 ? 64 : 32;
  const int nch = (K + KC - 1) / KC;
  const int cps = (nch + splits - 1) / splits;
  const int sz = BF16 ? 2 : 4;
  const int vec = aligned16(A) && aligned16(Bm) && (lda * sz) % 16 == 0 && (ldb * sz) % 16 == 0;
  const dim3 grid((N + 32 * WN - 1) / (32 * WN), (M + 32 * WM - 1) / (32 * WM), (nch + cps - 1) / cps);
  hipLaunchKernelGGL((bwd_gemm_nt<BF16, WM, WN>), grid, dim3(kBwdThreads), 0, s, A, lda, Bm, ldb, C, ldc,
                     split_stride, M, N, K, cps, vec);
  return hipGetLastError();
}

template <bool BF16>
lstm_status_t bwd_run(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                      const void* R, const void* reserve, const float* dy, const float* dhT, const float* dcT,
                      float* dx, float* dh0, float* dc0, float* dW, float* dR, float* db, void* ws, const BwdLayout& o,
                      hipStream_t st) {
  const int L = d->L, I = d->I, H = d->H, B = d->B, T = d->T;
  const long TB = (long)T * B, G = 4L * H;
  const size_t s = BF16 ? 2 : 4;
  char* w = static_cast<char*>(ws);
  void* RT = w + o.rt;
  void* WT = w + o.wt;
  float* dP = reinterpret_cast<float*>(w + o.dp);
  void* dPh = w + o.dph;
  void* dPT = w + o.dpt;
  void* UT = w + o.ut;
  void* HT = w + o.ht;
  float* dYbuf[2] = {reinterpret_cast<float*>(w + o.dy0), reinterpret_cast<float*>(w + o.dy1)};
  float* dhp = reinterpret_cast<float*>(w + o.dhp);
  float* dcrec = reinterpret_cast<float*>(w + o.dcrec);
  const char* rsv = static_cast<const char*>(reserve);
  const size_t tbh = (size_t)T * B * H;
  const float* dY = dy;
  int next = 0;
#define CHECK(e)                             \
  do {                                       \
    if ((e) != hipSuccess) return LSTM_ERR_HIP; \
  } while (0)
  for (int l = L - 1; l >= 0; --l) {
    const int Il = l == 0 ? I : H;
    const char* Wl = static_cast<const char*>(W) + (l == 0 ? 0 : (G * I + (size_t)(l - 1) * G * H)) * s;
    const char* Rl = static_cast<const char*>(R) + (size_t)l * G * H * s;
    const float* gates = reinterpret_cast<const float*>(rsv + (size_t)l * tbh * 16);
    const float* cs = reinterpret_cast<const float*>(rsv + (size_t)L * tbh * 16 + (size_t)l * tbh * 4);
    const char* hs = rsv + (size_t)L * tbh * 20 + (size_t)l * tbh * s;
    // R_l^T [H][4H]: the per-step product's second operand, K = 4H contiguous
    CHECK(transpose<BF16>(Rl, H, nullptr, 0, 0, (int)G, H, RT, G, st));
    for (int t = T - 1; t >= 0; --t) {
      StepArgs a;
      a.dY = dY + (size_t)t * B * H;
      a.dhp = t < T - 1 ? dhp : nullptr;
      a.sstride = (long)B * H;
      a.S = o.S;
      a.dhT = dhT ? dhT + (size_t)l * B * H : nullptr;
      a.dcT = dcT ? dcT + (size_t)l * B * H : nullptr;
      a.gates = gates + (size_t)t * B * G;
      a.c_t = cs + (size_t)t * B * H;
      a.c_prev = t > 0 ? cs + (size_t)(t - 1) * B * H : (c0 ? c0 + (size_t)l * B * H : nullptr);
      a.dcrec = dcrec;
      a.dP = dP + (size_t)t * B * G;
      a.dPh = static_cast<char*>(dPh) + (size_t)t * B * G * s;
      a.dc0 = (t == 0 && dc0) ? dc0 + (size_t)l * B * H : nullptr;
      a.B = B, a.H = H, a.last = t == T - 1;
      const int blocks = (int)std::min<long>(((long)B * H + kBwdThreads - 1) / kBwdThreads, 1024);
      hipLaunchKernelGGL(bwd_step<BF16>, dim3(blocks), dim3(kBwdThreads), 0, st, a);
      CHECK(hipGetLastError());
      const void* dpt = static_cast<const char*>(dPh) + (size_t)t * B * G * s;
      if (t > 0) {
        // dh_rec = dp_t R_l, as o.S partial sums over slices of K = 4H
        CHECK((gemm_nt<BF16, kStepWM, kStepWN>(dpt, G, RT, G, dhp, H, (long)B * H, B, H, (int)G, o.S, st)));
      } else if (dh0) {
        CHECK((gemm_nt<BF16, kStepWM, kStepWN>(dpt, G, RT, G, dh0 + (size_t)l * B * H, H, 0, B, H, (int)G, 1, st)));
      }
    }
    // db_l: column sums of dP over all steps and sequences
    hipLaunchKernelGGL(bwd_colsum, dim3((unsigned)((G + kBwdThreads - 1) / kBwdThreads)), dim3(kBwdThreads), 0, st, dP,
                       (int)TB, (int)G, db + (size_t)l * G);
    CHECK(hipGetLastError());
    // the K = T*B contiguous operands of the weight-gradient products
    CHECK(transpose<BF16>(dPh, G, nullptr, 0, 0, (int)TB, (int)G, dPT, TB, st));
    const void* U = l == 0 ? x : static_cast<const void*>(rsv + (size_t)L * tbh * 20 + (size_t)(l - 1) * tbh * s);
    CHECK(transpose<BF16>(U, Il, nullptr, 0, 0, (int)TB, Il, UT, TB, st));
    const void* h0l = h0 ? static_cast<const char*>(h0) + (size_t)l * B * H * s : nullptr;
    CHECK(transpose<BF16>(hs, H, h0l, H, B, (int)TB, H, HT, TB, st));  // row t*B+b: h_{t-1}[b] (h0 at t = 0)
    float* dWl = dW + (l == 0 ? 0 : (G * I + (size_t)(l - 1) * G * H));
    CHECK((gemm_nt<BF16, kBigWM, kBigWN>(dPT, TB, UT, TB, dWl, Il, 0, (int)G, Il, (int)TB, 1, st)));
    CHECK((gemm_nt<BF16, kBigWM, kBigWN>(dPT, TB, HT, TB, dR + (size_t)l * G * H, H, 0, (int)G, H, (int)TB, 1, st)));
    if (l > 0 || dx) {
      // dU = dP W_l: the layer below's dY, or dx
      CHECK(transpose<BF16>(Wl, Il, nullptr, 0, 0, (int)G, Il, WT, G, st));
      float* dU = l > 0 ? dYbuf[next] : dx;
      CHECK((gemm_nt<BF16, kBigWM, kBigWN>(dPh, G, WT, G, dU, Il, 0, (int)TB, Il, (int)G, 1, st)));
      dY = dU;
      next ^= 1;
    }
  }
#undef CHECK
  return LSTM_OK;
}

}  // namespace
}  // namespace lstm

using namespace lstm;

extern "C" {

size_t lstm_bwd_workspace_size(const lstm_desc_t* d) {
  BwdLayout o;
  return bwd_layout(d, &o) ? o.total : 0;
}

lstm_status_t lstm_bwd(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                       const void* R, const void* reserve, const float* dy, const float* dhT, const float* dcT,
                       float* dx, float* dh0, float* dc0, float* dW, float* dR, float* db, void* ws,
                       hipStream_t stream) {
  if (!d || d->L < 1 || d->I < 1 || d->H < 1 || d->B < 1 || d->T < 1) return LSTM_ERR_INVALID_ARG;
  if (d->dtype != LSTM_F32 && d->dtype != LSTM_BF16) return LSTM_ERR_INVALID_ARG;
  if (d->cell < LSTM_CELL_LSTM || d->cell > LSTM_CELL_RNN_RELU) return LSTM_ERR_INVALID_ARG;
  if (d->cell != LSTM_CELL_LSTM) return LSTM_ERR_UNSUPPORTED;
  if (!x || !W || !R || !reserve || !dy || !dW || !dR || !db) return LSTM_ERR_INVALID_ARG;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) return LSTM_ERR_WORKSPACE;
  BwdLayout o;
  if (!bwd_layout(d, &o)) return LSTM_ERR_UNSUPPORTED;
  // the products address their operands with 32-bit tile indices and 64-bit offsets;
  // keep every dimension below 2^31 elements
  if ((long long)d->T * d->B * 4 * d->H >= (1LL << 31)) return LSTM_ERR_UNSUPPORTED;
  return d->dtype == LSTM_BF16
             ? bwd_run<true>(d, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db, ws, o, stream)
             : bwd_run<false>(d, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db, ws, o, stream);
}

}  // extern "C"
