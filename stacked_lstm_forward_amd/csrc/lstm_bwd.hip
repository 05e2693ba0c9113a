// Backward pass (backpropagation through time) of the stacked LSTM for
// gfx950: kernels and the lstm_bwd entry point (include/lstm_bwd.h).
//
// Per layer, from the top:
//   1. the recurrent chain, strictly serial in t = T-1 .. 0: dh = dY[t] +
//      dh_rec and dc_rec give the gate derivatives dp_t (fp32, and copies in
//      the workload's dtype) and the next dc_rec; dh_rec = dp_t R_l, an MFMA
//      product over K = 4H.  For the shapes lstm_bwd_res.h is built for, one
//      persistent launch per layer runs the whole chain with R_l^T on chip
//      (R_l^T rewritten once per layer in MFMA load order, K unit-major).
//      Otherwise (the streamed chain) each step is an elementwise kernel and
//      the product split over K across workgroups so it fills the GPU (the
//      K-split partial sums are added by the next step's elementwise kernel,
//      in a fixed order); that product reads all of R_l every step, so it is
//      bound by memory: R_l^T and dp_t are laid out in the order the MFMA
//      fragments are loaded (every wave-wide load reads 1 KiB in one piece),
//      each workgroup keeps its slice of dp_t in LDS and streams its slice of
//      R_l^T with eight chunks of loads in flight per wave;
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

#include <mutex>
#include <vector>

#include "lstm_bwd.h"  // include/ is on the include path
#include "lstm_bwd_res.h"
#include "lstm_common.h"
#include "lstm_params.h"

namespace lstm {

// lstm_kernels.hip
hipError_t prepare_fn(const void* fn, int lds_bytes, int block, int* blocks_per_cu);
hipError_t launch_gemm_plain(bool bf16, const void* A, const void* B, float* C, long long ldc, int M, int N, int K,
                             int num_cus, float* C2, long long c2_floats, hipStream_t s);
// lstm_bwd_res_inst.hip: the on-chip chain kernel of kBwdResShape[k] for nw batch tiles
const void* bwd_res_kernel_ptr_shape0(int nw);
const void* bwd_res_kernel_ptr_shape1(int nw);
const void* bwd_res_kernel_ptr_shape2(int nw);
const void* bwd_res_kernel_ptr_shape3(int nw);
const void* bwd_res_kernel_ptr_shape4(int nw);
const void* bwd_res_kernel_ptr_shape5(int nw);
const void* bwd_res_kernel_ptr_shape6(int nw);
const void* bwd_res_kernel_ptr_shape7(int nw);
const void* bwd_res_kernel_ptr_shape8(int nw);
const void* bwd_res_kernel_ptr_shape9(int nw);
const void* bwd_res_kernel_ptr_shape10(int nw);
const void* bwd_res_kernel_ptr_shape11(int nw);
const void* bwd_res_kernel_ptr_shape12(int nw);
const void* bwd_res_kernel_ptr_shape13(int nw);
const void* bwd_res_kernel_ptr_shape14(int nw);
const void* bwd_res_kernel_ptr_shape15(int nw);

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

// The same transpose for T-typed source and destination with 16-byte global
// loads and stores on whole 64 x 64 tiles (rows 16-byte aligned: the host
// checks the bases and leading dimensions); partial tiles go element by element.
template <typename T>
__global__ void __launch_bounds__(kBwdThreads) bwd_transpose_v(const T* main, long ldm, const T* first, long ldf,
                                                              int nfirst, int rows, int cols, T* dst, long ldd) {
  constexpr int EPV = 16 / sizeof(T), PR = 64 / EPV;  // elements per 16 bytes, pieces per tile row
  __shared__ __align__(16) T tile[64][64 + EPV];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  auto src_row = [&](int r) -> const T* {
    return r < nfirst ? (first ? first + (long)r * ldf : nullptr) : main + (long)(r - nfirst) * ldm;
  };
  if (r0 + 64 > rows || c0 + 64 > cols) {
    for (int i = threadIdx.x; i < 64 * 64; i += kBwdThreads) {
      const int r = i / 64, c = i % 64;
      const T* row = r0 + r < rows ? src_row(r0 + r) : nullptr;
      tile[r][c] = (row && c0 + c < cols) ? row[c0 + c] : T(0);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += kBwdThreads) {
      const int c = i / 64, r = i % 64;
      if (c0 + c < cols && r0 + r < rows) dst[(long)(c0 + c) * ldd + r0 + r] = tile[r][c];
    }
    return;
  }
  for (int i = threadIdx.x; i < 64 * PR; i += kBwdThreads) {
    const int r = i / PR, pc = i % PR;
    const T* row = src_row(r0 + r);
    *reinterpret_cast<uint4*>(&tile[r][pc * EPV]) =
        row ? *reinterpret_cast<const uint4*>(row + c0 + pc * EPV) : uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * PR; i += kBwdThreads) {
    const int c = i / PR, pr = i % PR;
    T v[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) v[e] = tile[pr * EPV + e][c];
    *reinterpret_cast<uint4*>(dst + (long)(c0 + c) * ldd + r0 + pr * EPV) = *reinterpret_cast<const uint4*>(v);
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

// Element offset of (row r, column k) of a matrix stored in MFMA load order
// with nch chunks of KC columns per row tile: block (r / 16, chunk) of 2 KiB,
// half h at +1 KiB, lane q * 16 + r % 16 at +16 bytes per lane, holding the
// lane's fragment columns frag_col(q, h) .. + KC / 8 - 1 of that chunk.
template <bool BF16>
__device__ __forceinline__ long frag_off(int r, int k, int nch) {
  constexpr int KC = Dt<BF16>::KC, EPH = KC / 8;
  const int c = k / KC, kc = k % KC;
  const int h = kc / (KC / 2), q = (kc % (KC / 2)) / EPH, e = kc % EPH;
  return (((long)(r >> 4) * nch + c) * 2 + h) * (64 * EPH) + (q * 16 + (r & 15)) * EPH + e;
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
  void* dPf;            // the same in MFMA load order (nch chunks per 16 rows)
  float* dc0;           // [B][H] or null: written at step 0
  int B, H, last, nch;
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
    T* dpf = reinterpret_cast<T*>(a.dPf);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const T v = from_float<BF16>(d[k]);
      dp[(long)k * a.H] = d[k];
      dph[(long)k * a.H] = v;
      dpf[frag_off<BF16>(bb, k * a.H + j, a.nch)] = v;
    }
    const float dcn = dc * fg;
    a.dcrec[idx] = dcn;
    if (a.dc0) a.dc0[idx] = dcn;
  }
}

// db[k] = sum over the rows r < rows of dP[r][k], in two passes with a fixed
// order: slab z (rows kColSlab z .. kColSlab z + kColSlab - 1, in order) into
// part[z][k], then the slabs in order.
constexpr int kColSlab = 64;
__global__ void __launch_bounds__(kBwdThreads) bwd_colsum_slab(const float* dP, int rows, int cols, float* part) {
  const int k = blockIdx.x * kBwdThreads + threadIdx.x, z = blockIdx.y;
  if (k >= cols) return;
  const int r1 = min(rows, (z + 1) * kColSlab);
  float s = 0.f;
#pragma unroll 8
  for (int r = z * kColSlab; r < r1; ++r) s += dP[(long)r * cols + k];
  part[(long)z * cols + k] = s;
}
__global__ void __launch_bounds__(kBwdThreads) bwd_colsum_final(const float* part, int slabs, int cols, float* db) {
  const int k = blockIdx.x * kBwdThreads + threadIdx.x;
  if (k >= cols) return;
  float s = 0.f;
#pragma unroll 8
  for (int z = 0; z < slabs; ++z) s += part[(long)z * cols + k];
  db[k] = s;
}

// R_l^T in load order: element (n, k) = R_l[k][n] for n < H, k < 4H, zero in
// the padding.  Workgroup (x, c): columns n of R 64 x .. 64 x + 63 and rows k
// of chunk c, through an LDS tile.  UNIT_MAJOR orders K as k = 4 u + g (gate g
// of unit u, row g H + u of R_l), the order of the on-chip chain's exchange.
// Rows are read in 16-byte pieces (each tile row is one 128- or 256-byte run of
// R_l) when every row of R_l starts 16-byte aligned (`vec`: the host checks the
// base and that H is a multiple of 16 / size of an element), element by
// element otherwise.
template <bool BF16, bool UNIT_MAJOR>
__global__ void __launch_bounds__(kBwdThreads) bwd_block_rt(const void* R, int H, int nch, int vec, uint4* out) {
  typedef typename Dt<BF16>::T T;
  constexpr int KC = Dt<BF16>::KC, EPH = KC / 8, VE = 16 / sizeof(T), RV = 64 / VE;
  __shared__ __align__(16) T tile[KC][64 + VE];
  const int n0 = blockIdx.x * 64, c = blockIdx.y, G = 4 * H;
  const T* Rp = static_cast<const T*>(R);
  for (int i = threadIdx.x; i < KC * RV; i += kBwdThreads) {
    const int kr = i / RV, nc = (i % RV) * VE, k = c * KC + kr, n = n0 + nc;
    const long row = UNIT_MAJOR ? (long)(k % 4) * H + k / 4 : (long)k;
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (k < G && n < H) {
      if (vec) {
        v = *reinterpret_cast<const uint4*>(Rp + row * H + n);
      } else {
        T t[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) t[e] = n + e < H ? Rp[row * H + n + e] : T(0);
        __builtin_memcpy(&v, t, 16);
      }
    }
    *reinterpret_cast<uint4*>(&tile[kr][nc]) = v;
  }
  __syncthreads();
  // 4 row tiles x 2 halves x 64 lanes of 16 bytes
  for (int i = threadIdx.x; i < 4 * 2 * 64; i += kBwdThreads) {
    const int t16 = i / 128, h = (i / 64) % 2, lane = i % 64, q = lane >> 4;
    const int nl = 16 * t16 + (lane & 15), n = n0 + nl;
    if (n >= ((H + 15) & ~15)) continue;
    T v[EPH];
#pragma unroll
    for (int e = 0; e < EPH; ++e) v[e] = tile[frag_col<BF16>(q, h) + e][nl];
    out[frag_off<BF16>(n, c * KC + frag_col<BF16>(q, h), nch) / EPH] = *reinterpret_cast<const uint4*>(v);
  }
}

// Zeroes n 16-byte words (a fill kernel, so the call stays capturable).
__global__ void __launch_bounds__(kBwdThreads) bwd_zero(uint4* p, long n) {
  for (long i = (long)blockIdx.x * kBwdThreads + threadIdx.x; i < n; i += (long)gridDim.x * kBwdThreads)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// dst[i] = sum over z < S of part[z * pstride + i], in order (dh0 from the
// K-split partial sums of step 0).
__global__ void __launch_bounds__(kBwdThreads) bwd_sum_parts(const float* part, long pstride, int S, long n,
                                                             float* dst) {
  for (long i = (long)blockIdx.x * kBwdThreads + threadIdx.x; i < n; i += (long)gridDim.x * kBwdThreads) {
    float v = 0.f;
    for (int z = 0; z < S; ++z) v += part[z * pstride + i];
    dst[i] = v;
  }
}

constexpr int kRecWaves = 8;   // waves per workgroup of the per-step product: one column tile each
constexpr int kRecDepth = 8;   // chunks of R^T loads in flight per wave
constexpr int kRecLdsBlocks = 64;  // dp blocks (2 KiB) a workgroup stages: 128 KiB

// The per-step product dh_rec partials: part[z][b][n] = sum over the chunks c
// of split z of dp_t[b][c-th chunk] . R^T[n][c-th chunk], for b < B, n < H.
// Workgroup (x, z, y): column tiles 8 x + w (wave w), chunks
// [z cps, min(nch, (z + 1) cps)), batch tiles NBT y .. NBT y + NBT - 1.  Its
// dp blocks go to LDS first; each wave then streams its R^T blocks (each
// read once per step by one wave) kRecDepth chunks ahead.
template <bool BF16, int NBT>
__global__ void __launch_bounds__(64 * kRecWaves) bwd_rec_product(const uint4* RTf, const uint4* DPf, float* part,
                                                                   long pstride, int B, int H, int nch, int cps,
                                                                   int nbt) {
  extern __shared__ __align__(16) uint4 sdp[];  // [NBT][cps] blocks of 128 x 16 bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = blockIdx.x * kRecWaves + wave, z = blockIdx.y, bt0 = blockIdx.z * NBT;
  const int c0 = z * cps, ncs = min(nch, c0 + cps) - c0;
  // R^T prefetch first (it comes from memory), then stage dp (mostly in L2)
  const bool live = n16 * 16 < H && ncs > 0;
  const uint4* rt = RTf + ((long)n16 * nch + c0) * 128 + lane;
  Frag ring[kRecDepth];
  if (live) {
#pragma unroll
    for (int s = 0; s < kRecDepth; ++s)
      if (s < ncs) {
        ring[s].v[0] = rt[(long)s * 128];
        ring[s].v[1] = rt[(long)s * 128 + 64];
      }
  }
  const int nblk = NBT * ncs * 128;
  for (int i = tid; i < nblk; i += 64 * kRecWaves) {
    const int bt = i / (ncs * 128), rem = i % (ncs * 128), cc = rem / 128, w = rem % 128;
    sdp[(bt * cps + cc) * 128 + w] =
        bt0 + bt < nbt ? DPf[((long)(bt0 + bt) * nch + c0 + cc) * 128 + w] : uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  if (!live) return;
  f32x4 acc[NBT];
#pragma unroll
  for (int bt = 0; bt < NBT; ++bt) acc[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int cb = 0; cb < ncs; cb += kRecDepth) {
#pragma unroll
    for (int s = 0; s < kRecDepth; ++s) {
      const int cc = cb + s;
      if (cc < ncs) {
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
          const Frag d = lds_get(sdp + (bt * cps + cc) * 128, lane);
          mfma_frag<BF16>(acc[bt], ring[s], d);
        }
        if (cc + kRecDepth < ncs) {
          ring[s].v[0] = rt[(long)(cc + kRecDepth) * 128];
          ring[s].v[1] = rt[(long)(cc + kRecDepth) * 128 + 64];
        }
      }
    }
  }
  // acc[bt]: batch row 16 (bt0 + bt) + lane % 16, columns n .. n + 3
  const int n = 16 * n16 + 4 * (lane >> 4);
  float* pz = part + (long)z * pstride;
#pragma unroll
  for (int bt = 0; bt < NBT; ++bt) {
    const int b = 16 * (bt0 + bt) + (lane & 15);
    if (b >= B) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < H) pz[(long)b * H + n + r] = acc[bt][r];
  }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Shape of the per-step product launch for a (B, H, dtype).
struct RecShape {
  int nch;      // chunks of K = 4H
  int nt16;     // column tiles of 16 (n < H)
  int nbt;      // batch tiles of 16
  int NBT;      // batch tiles per workgroup (1, 2, 4 or 8)
  int ngroups;  // workgroups across the columns (kRecWaves tiles each)
  int bgroups;  // ... across the batch
  int cps;      // chunks per K split
  int S;        // K splits (partial sums the step kernel adds)
};

// Enough K splits for about 256 workgroups, each staging at most
// kRecLdsBlocks dp blocks; batch tiles go to as few workgroup groups as
// possible, since every group streams all of R^T.
RecShape rec_shape(int B, int H, bool bf16) {
  RecShape r;
  const int KC = bf16 ? 64 : 32;
  r.nch = (4 * H + KC - 1) / KC;
  r.nt16 = (H + 15) / 16;
  r.nbt = (B + 15) / 16;
  const int m = std::min(r.nbt, 8);
  r.NBT = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
  r.bgroups = (r.nbt + r.NBT - 1) / r.NBT;
  r.ngroups = (r.nt16 + kRecWaves - 1) / kRecWaves;
  const int want = std::max(1, 256 / (r.ngroups * r.bgroups));
  r.cps = std::max(1, std::min((r.nch + want - 1) / want, kRecLdsBlocks / r.NBT));
  r.S = (r.nch + r.cps - 1) / r.cps;
  return r;
}

struct BwdLayout {
  size_t ctl, flg, dpx, prt, rtf, dpf, wt, dp, dph, dpt, ut, ht, dy0, dy1, dhp, dcrec, colp, spl, total;
  RecShape rs;
  int res_nci;  // > 0: the chain runs in lstm_bwd_res_kernel with this many chunks per wave,
  int res_mw;   // ... this many M-tiles per workgroup (4 over a K quarter, 1 over all of K)
  int res_nw;   // ... and this many batch tiles (1, 2 or 4; 3 runs as 4)
  size_t spl_floats;
};

// Floats of the buffer for the extra K ranges' partial sums of the gradient
// products (launch_gemm_plain splits K when a product has too few tiles to
// fill the GPU; each extra range needs a copy of C): one copy of the largest
// T*B-row result (the input gradient), or up to 15 copies of the largest
// weight gradient (4H x max(I, H)) within 64 MiB.
size_t bwd_spl_floats(size_t TB, size_t G, size_t Imax) {
  return std::max(TB * Imax, std::min(15 * G * Imax, (size_t)1 << 24));
}

// Batch tiles the on-chip chain runs for B sequences (its instantiations take
// 1, 2 or 4; a third tile runs as a fourth, all padding).
int bwd_res_nw(int B) {
  const int nbt = (B + 15) / 16;
  return nbt <= 2 ? nbt : 4;
}

bool bwd_res_listed(bool bf16, int nci, int mw) {
  for (const BwdResShape& sh : kBwdResShape)
    if (sh.bf16 == (bf16 ? 1 : 0) && sh.nci == nci && sh.mw == mw) return true;
  return false;
}

// The on-chip chain's shape for a problem, when kBwdResShape has it: one
// M-tile per workgroup over all of K (NCI = H / KC chunks per wave, every
// block in LDS; H a multiple of KC) when its R_l^T rows fit in LDS, else four
// M-tiles over a K quarter (NCI = H / (4 KC); H a multiple of 256, whole unit
// groups of 64 per quarter); *mw = 0 otherwise (the streamed chain runs).  B
// at most 64 (32 with four M-tiles and NCI = 16).
int bwd_resident_nci(const lstm_desc_t* d, int* mw) {
  const bool bf16 = d->dtype == LSTM_BF16;
  const int KC = bf16 ? 64 : 32;
  *mw = 0;
  if (d->cell != LSTM_CELL_LSTM || d->H % KC != 0 || d->B > 64) return 0;
  const int nw = bwd_res_nw(d->B);
  int nci = d->H / KC;
  if (bwd_res_listed(bf16, nci, 1)) {
    *mw = 1;
  } else {
    if (d->H % 256 != 0) return 0;
    nci = d->H / (4 * KC);
    if (!bwd_res_listed(bf16, nci, 4) || nw > (nci >= 16 ? 2 : 4)) return 0;
    *mw = 4;
  }
  // the kernel's per-step offsets are 32-bit: T + 1 slots of the dp exchange
  // (nw tiles x 4H / KC chunks x 2 KiB) and the T B 4H saved gates
  const long long xslot = (long long)nw * (4LL * d->H / KC) * (2048 / (bf16 ? 2 : 4));
  if ((long long)(d->T + 1) * xslot >= (1LL << 31) || (long long)d->T * d->B * 4 * d->H >= (1LL << 31)) return 0;
  return nci;
}
int bwd_res_wgs(int H) { return H / 16; }

const void* bwd_res_fn(bool bf16, int nci, int mw, int nw) {
  const void* (*const per_shape[kBwdResShapes])(int) = {
      bwd_res_kernel_ptr_shape0, bwd_res_kernel_ptr_shape1,  bwd_res_kernel_ptr_shape2,  bwd_res_kernel_ptr_shape3,
      bwd_res_kernel_ptr_shape4, bwd_res_kernel_ptr_shape5,  bwd_res_kernel_ptr_shape6,  bwd_res_kernel_ptr_shape7,
      bwd_res_kernel_ptr_shape8, bwd_res_kernel_ptr_shape9,  bwd_res_kernel_ptr_shape10, bwd_res_kernel_ptr_shape11,
      bwd_res_kernel_ptr_shape12, bwd_res_kernel_ptr_shape13, bwd_res_kernel_ptr_shape14, bwd_res_kernel_ptr_shape15};
  static_assert(kBwdResShapes == 16, "one compile unit per shape");
  for (int k = 0; k < kBwdResShapes; ++k)
    if (kBwdResShape[k].bf16 == (bf16 ? 1 : 0) && kBwdResShape[k].nci == nci && kBwdResShape[k].mw == mw)
      return per_shape[k](nw);
  return nullptr;
}

// Compute units and wall-clock rate (kHz) of the current device, once per device.
hipError_t bwd_device(int* cus, int* clk_khz) {
  struct Info {
    int dev, cus, clk;
  };
  static std::mutex mu;
  static std::vector<Info> seen;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const Info& i : seen)
    if (i.dev == dev) {
      *cus = i.cus, *clk_khz = i.clk;
      return hipSuccess;
    }
  Info i{dev, 0, 0};
  if ((e = hipDeviceGetAttribute(&i.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&i.clk, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
  seen.push_back(i);
  *cus = i.cus, *clk_khz = i.clk;
  return hipSuccess;
}

constexpr long long kBwdTimeoutUs = 2000000;  // 2 s per step wait

constexpr int kBigWM = 2, kBigWN = 2;  // weight-gradient products when the direct-to-LDS kernel does not fit

bool bwd_layout(const lstm_desc_t* d, BwdLayout* o) {
  if (!d || d->cell != LSTM_CELL_LSTM || lstm_fwd_workspace_size(d) == 0) return false;
  const size_t s = d->dtype == LSTM_BF16 ? 2 : 4;
  const size_t H = d->H, B = d->B, TB = (size_t)d->T * d->B, G = 4 * H;
  const size_t Imax = std::max<size_t>(d->I, H);
  o->rs = rec_shape(d->B, d->H, d->dtype == LSTM_BF16);
  o->res_nci = bwd_resident_nci(d, &o->res_mw);
  o->res_nw = bwd_res_nw(d->B);
  const bool resident = o->res_nci > 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  o->ctl = take(256);  // the error word first, as in the forward's workspace
  // the on-chip chain: two sets of step counters, the dp exchange, the partial sums
  const int rwgs = bwd_res_wgs(d->H);
  // (counters for up to res_nw batch groups of rwgs workgroups)
  o->flg = take(resident ? (size_t)2 * o->res_nw * rwgs * kFlagStride * 4 : 0);
  o->dpx = take(resident ? (size_t)d->T * o->res_nw * o->rs.nch * 2048 : 0);
  o->prt = take(resident && o->res_mw > 1 ? (size_t)(d->T + 1) * bwd_res_part_floats(rwgs, o->res_nw) * 4 : 0);
  o->rtf = take((size_t)o->rs.nt16 * o->rs.nch * 2048);
  o->dpf = take((size_t)o->rs.nbt * o->rs.nch * 2048);
  o->wt = take(Imax * G * s);
  o->dp = take(TB * G * 4);
  o->dph = take(TB * G * s);
  o->dpt = take(G * TB * s);
  o->ut = take(Imax * TB * s);
  o->ht = take(H * TB * s);
  o->dy0 = take(TB * H * 4);
  o->dy1 = take(TB * H * 4);
  o->dhp = take((size_t)o->rs.S * B * H * 4);
  o->dcrec = take(B * H * 4);
  o->colp = take((TB + kColSlab - 1) / kColSlab * G * 4);
  o->spl_floats = bwd_spl_floats(TB, G, Imax);
  o->spl = take(o->spl_floats * 4);  // partial sums of the products' extra K ranges
  o->total = off;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool BF16>
hipError_t transpose(const void* main, long ldm, const void* first, long ldf, int nfirst, int rows, int cols, void* dst,
                     long ldd, hipStream_t s) {
  typedef typename Dt<BF16>::T T;
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  const long epv = 16 / (long)sizeof(T);
  if (aligned16(main) && aligned16(first) && aligned16(dst) && ldm % epv == 0 && ldf % epv == 0 && ldd % epv == 0) {
    hipLaunchKernelGGL((bwd_transpose_v<T>), grid, dim3(kBwdThreads), 0, s, static_cast<const T*>(main), ldm,
                       static_cast<const T*>(first), ldf, nfirst, rows, cols, static_cast<T*>(dst), ldd);
    return hipGetLastError();
  }
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

template <bool BF16, int NBT>
const void* rec_product_fn() {
  return reinterpret_cast<const void*>(&bwd_rec_product<BF16, NBT>);
}

template <bool BF16>
hipError_t rec_product(const RecShape& r, const void* RTf, const void* DPf, float* part, int B, int H, hipStream_t st) {
  const void* fn = r.NBT == 1   ? rec_product_fn<BF16, 1>()
                   : r.NBT == 2 ? rec_product_fn<BF16, 2>()
                   : r.NBT == 4 ? rec_product_fn<BF16, 4>()
                                : rec_product_fn<BF16, 8>();
  const int lds = r.NBT * r.cps * 2048;
  hipError_t e = prepare_fn(fn, lds, 64 * kRecWaves, nullptr);
  if (e != hipSuccess) return e;
  const uint4* rt = static_cast<const uint4*>(RTf);
  const uint4* dp = static_cast<const uint4*>(DPf);
  long pstride = (long)B * H;
  int nch = r.nch, cps = r.cps, nbt = r.nbt;
  void* args[] = {&rt, &dp, &part, &pstride, &B, &H, &nch, &cps, &nbt};
  return hipLaunchKernel(fn, dim3(r.ngroups, r.S, r.bgroups), dim3(64 * kRecWaves), args, (unsigned)lds, st);
}

// C = A B^T (see gemm_nt) on the direct-to-LDS kernel when the operands suit
// it (K-contiguous rows of whole chunks, 16-byte aligned), else gemm_nt.
template <bool BF16>
hipError_t big_product(const void* A, const void* Bm, float* C, long ldc, int M, int N, int K, float* spare,
                       long long spare_floats, hipStream_t st) {
  const hipError_t e = launch_gemm_plain(BF16, A, Bm, C, ldc, M, N, K, 0, spare, spare_floats, st);
  if (e != hipErrorNotSupported) return e;
  return gemm_nt<BF16, kBigWM, kBigWN>(A, K, Bm, K, C, ldc, 0, M, N, K, 1, st);
}

template <bool BF16>
lstm_status_t bwd_run(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                      const void* R, const void* reserve, const float* dy, const float* dhT, const float* dcT,
                      float* dx, float* dh0, float* dc0, float* dW, float* dR, float* db, void* ws, const BwdLayout& o,
                      bool plain, long long timeout_us, hipStream_t st) {
  const int L = d->L, I = d->I, H = d->H, B = d->B, T = d->T;
  const long TB = (long)T * B, G = 4L * H;
  const size_t s = BF16 ? 2 : 4;
  char* w = static_cast<char*>(ws);
  const RecShape& rs = o.rs;
  void* RTf = w + o.rtf;
  void* DPf = w + o.dpf;
  void* WT = w + o.wt;
  float* dP = reinterpret_cast<float*>(w + o.dp);
  void* dPh = w + o.dph;
  void* dPT = w + o.dpt;
  void* UT = w + o.ut;
  void* HT = w + o.ht;
  float* dYbuf[2] = {reinterpret_cast<float*>(w + o.dy0), reinterpret_cast<float*>(w + o.dy1)};
  float* dhp = reinterpret_cast<float*>(w + o.dhp);
  float* dcrec = reinterpret_cast<float*>(w + o.dcrec);
  float* colp = reinterpret_cast<float*>(w + o.colp);
  float* spl = reinterpret_cast<float*>(w + o.spl);  // partial sums of split products
  const long long spl_floats = (long long)o.spl_floats;
  const char* rsv = static_cast<const char*>(reserve);
  const size_t tbh = (size_t)T * B * H;
  const float* dY = dy;
  int next = 0;
#define CHECK(e)                             \
  do {                                       \
    if ((e) != hipSuccess) return LSTM_ERR_HIP; \
  } while (0)
  // the on-chip chain needs every workgroup resident at once: checked (and
  // the kernel's LDS limit set) before anything is enqueued, else the
  // streamed chain runs
  int cus = 0, clk_khz = 0;
  CHECK(bwd_device(&cus, &clk_khz));
  // (its per-step loads and stores are 16 bytes wide: the caller's per-step
  // tensors must be 16-byte aligned, as torch allocations are)
  bool resident = o.res_nci > 0 && aligned16(dy) && aligned16(reserve) && aligned16(c0) && aligned16(dhT) &&
                  aligned16(dcT) && aligned16(dh0) && aligned16(dc0);
  const int res_nw = o.res_nw;
  const int res_wgs = bwd_res_wgs(H);
  // batch groups: the most (of res_nw, res_nw / 2, .., 1; each group runs
  // res_nw / groups column tiles on its own res_wgs workgroups) whose grid
  // is co-resident
  int res_groups = 0, res_lds = 0;
  const void* res_fn = nullptr;
  for (int g = res_nw; resident && g >= 1 && !res_groups; g /= 2) {
    const void* fn = bwd_res_fn(BF16, o.res_nci, o.res_mw, res_nw / g);
    const int lds = bwd_res_lds_bytes(res_nw / g, o.res_nci, o.res_mw);
    int per_cu = 0;
    if (fn && prepare_fn(fn, lds, 64 * kBwdResWaves, &per_cu) == hipSuccess && (long)per_cu * cus >= (long)g * res_wgs) {
      res_groups = g, res_fn = fn, res_lds = lds;
    } else {
      (void)hipGetLastError();
    }
  }
  if (!res_groups) resident = false;
  const int res_all = res_groups * res_wgs;  // workgroups in all
  // the error word
  hipLaunchKernelGGL(bwd_zero, dim3(1), dim3(kBwdThreads), 0, st, reinterpret_cast<uint4*>(w + o.ctl), 16L);
  CHECK(hipGetLastError());
  // the padding of dp's load-order copy (rows >= B, columns >= 4H) stays zero
  {
    const long n16 = (long)rs.nbt * rs.nch * 128;
    hipLaunchKernelGGL(bwd_zero, dim3((unsigned)std::min<long>((n16 + kBwdThreads - 1) / kBwdThreads, 1024)),
                       dim3(kBwdThreads), 0, st, static_cast<uint4*>(DPf), n16);
    CHECK(hipGetLastError());
  }
  for (int l = L - 1; l >= 0; --l) {
    const int Il = l == 0 ? I : H;
    const char* Wl = static_cast<const char*>(W) + (l == 0 ? 0 : (G * I + (size_t)(l - 1) * G * H)) * s;
    const char* Rl = static_cast<const char*>(R) + (size_t)l * G * H * s;
    const float* gates = reinterpret_cast<const float*>(rsv + (size_t)l * tbh * 16);
    const float* cs = reinterpret_cast<const float*>(rsv + (size_t)L * tbh * 16 + (size_t)l * tbh * 4);
    const char* hs = rsv + (size_t)L * tbh * 20 + (size_t)l * tbh * s;
    // R_l^T in load order: the per-step product's streamed operand
    // (K unit-major for the on-chip chain)
    const int rt_vec = aligned16(Rl) && H % (16 / (BF16 ? 2 : 4)) == 0;
    if (resident)
      hipLaunchKernelGGL((bwd_block_rt<BF16, true>), dim3((H + 63) / 64, rs.nch), dim3(kBwdThreads), 0, st,
                         static_cast<const void*>(Rl), H, rs.nch, rt_vec, static_cast<uint4*>(RTf));
    else
      hipLaunchKernelGGL((bwd_block_rt<BF16, false>), dim3((H + 63) / 64, rs.nch), dim3(kBwdThreads), 0, st,
                         static_cast<const void*>(Rl), H, rs.nch, rt_vec, static_cast<uint4*>(RTf));
    CHECK(hipGetLastError());
    if (resident) {
      const long nflag = (long)2 * res_all * kFlagStride * 4 / 16;
      hipLaunchKernelGGL(bwd_zero, dim3((unsigned)std::min<long>((nflag + kBwdThreads - 1) / kBwdThreads, 64)),
                         dim3(kBwdThreads), 0, st, reinterpret_cast<uint4*>(w + o.flg), nflag);
      CHECK(hipGetLastError());
      BwdResParams P{};
      P.RTf = static_cast<const uint4*>(RTf);
      P.DPx = w + o.dpx;
      P.xslot = (long long)res_nw * rs.nch * 2048 / (long long)s;
      P.dY = dY;
      P.gates = gates;
      P.cs = cs;
      P.c0 = c0 ? c0 + (size_t)l * B * H : nullptr;
      P.dhT = dhT ? dhT + (size_t)l * B * H : nullptr;
      P.dcT = dcT ? dcT + (size_t)l * B * H : nullptr;
      P.dP = dP;
      P.dPh = dPh;
      P.dh0 = dh0 ? dh0 + (size_t)l * B * H : nullptr;
      P.dc0 = dc0 ? dc0 + (size_t)l * B * H : nullptr;
      P.part = reinterpret_cast<float*>(w + o.prt);
      P.flags_d = reinterpret_cast<int*>(w + o.flg);
      P.flags_p = P.flags_d + (long)res_all * kFlagStride;
      P.err = reinterpret_cast<int*>(w + o.ctl);
      P.timeout_ticks = timeout_us * clk_khz / 1000;
      P.T = T, P.B = B, P.H = H, P.nch = rs.nch, P.wgs = res_all, P.groups = res_groups;
      P.grid = (res_all + 7) & ~7;
      P.xcd_remap = 1;
      void* args[] = {&P};
      if (plain)
        CHECK(hipLaunchKernel(res_fn, dim3(P.grid), dim3(64 * kBwdResWaves), args, (unsigned)res_lds, st));
      else
        CHECK(hipLaunchCooperativeKernel(res_fn, dim3(P.grid), dim3(64 * kBwdResWaves), args,
                                         (unsigned)res_lds, st));
    }
    for (int t = T - 1; t >= 0 && !resident; --t) {
      StepArgs a;
      a.dY = dY + (size_t)t * B * H;
      a.dhp = t < T - 1 ? dhp : nullptr;
      a.sstride = (long)B * H;
      a.S = rs.S;
      a.dhT = dhT ? dhT + (size_t)l * B * H : nullptr;
      a.dcT = dcT ? dcT + (size_t)l * B * H : nullptr;
      a.gates = gates + (size_t)t * B * G;
      a.c_t = cs + (size_t)t * B * H;
      a.c_prev = t > 0 ? cs + (size_t)(t - 1) * B * H : (c0 ? c0 + (size_t)l * B * H : nullptr);
      a.dcrec = dcrec;
      a.dP = dP + (size_t)t * B * G;
      a.dPh = static_cast<char*>(dPh) + (size_t)t * B * G * s;
      a.dPf = DPf;
      a.nch = rs.nch;
      a.dc0 = (t == 0 && dc0) ? dc0 + (size_t)l * B * H : nullptr;
      a.B = B, a.H = H, a.last = t == T - 1;
      const int blocks = (int)std::min<long>(((long)B * H + kBwdThreads - 1) / kBwdThreads, 1024);
      hipLaunchKernelGGL(bwd_step<BF16>, dim3(blocks), dim3(kBwdThreads), 0, st, a);
      CHECK(hipGetLastError());
      if (t > 0 || dh0) {
        // dh_rec = dp_t R_l, as rs.S partial sums over slices of K = 4H
        CHECK(rec_product<BF16>(rs, RTf, DPf, dhp, B, H, st));
        if (t == 0) {
          const long n = (long)B * H;
          hipLaunchKernelGGL(bwd_sum_parts, dim3((unsigned)std::min<long>((n + kBwdThreads - 1) / kBwdThreads, 1024)),
                             dim3(kBwdThreads), 0, st, static_cast<const float*>(dhp), n, rs.S, n,
                             dh0 + (size_t)l * B * H);
          CHECK(hipGetLastError());
        }
      }
    }
    // db_l: column sums of dP over all steps and sequences
    {
      const int slabs = (int)((TB + kColSlab - 1) / kColSlab);
      const unsigned gx = (unsigned)((G + kBwdThreads - 1) / kBwdThreads);
      hipLaunchKernelGGL(bwd_colsum_slab, dim3(gx, slabs), dim3(kBwdThreads), 0, st, dP, (int)TB, (int)G, colp);
      CHECK(hipGetLastError());
      hipLaunchKernelGGL(bwd_colsum_final, dim3(gx), dim3(kBwdThreads), 0, st, static_cast<const float*>(colp), slabs,
                         (int)G, db + (size_t)l * G);
      CHECK(hipGetLastError());
    }
    // the K = T*B contiguous operands of the weight-gradient products
    CHECK(transpose<BF16>(dPh, G, nullptr, 0, 0, (int)TB, (int)G, dPT, TB, st));
    const void* U = l == 0 ? x : static_cast<const void*>(rsv + (size_t)L * tbh * 20 + (size_t)(l - 1) * tbh * s);
    CHECK(transpose<BF16>(U, Il, nullptr, 0, 0, (int)TB, Il, UT, TB, st));
    const void* h0l = h0 ? static_cast<const char*>(h0) + (size_t)l * B * H * s : nullptr;
    CHECK(transpose<BF16>(hs, H, h0l, H, B, (int)TB, H, HT, TB, st));  // row t*B+b: h_{t-1}[b] (h0 at t = 0)
    float* dWl = dW + (l == 0 ? 0 : (G * I + (size_t)(l - 1) * G * H));
    CHECK(big_product<BF16>(dPT, UT, dWl, Il, (int)G, Il, (int)TB, spl, spl_floats, st));
    CHECK(big_product<BF16>(dPT, HT, dR + (size_t)l * G * H, H, (int)G, H, (int)TB, spl, spl_floats, st));
    if (l > 0 || dx) {
      // dU = dP W_l: the layer below's dY, or dx
      CHECK(transpose<BF16>(Wl, Il, nullptr, 0, 0, (int)G, Il, WT, G, st));
      float* dU = l > 0 ? dYbuf[next] : dx;
      CHECK(big_product<BF16>(dPh, WT, dU, Il, (int)TB, Il, (int)G, spl, spl_floats, st));
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

lstm_status_t lstm_bwd_last_error(const void* ws, hipStream_t stream) {
  if (!ws) return LSTM_ERR_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return LSTM_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, ws, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return LSTM_ERR_HIP;
  return v == 0 ? LSTM_OK : LSTM_ERR_BARRIER_TIMEOUT;
}

size_t lstm_bwd_workspace_size(const lstm_desc_t* d) {
  BwdLayout o;
  return bwd_layout(d, &o) ? o.total : 0;
}

int lstm_bwd_chain_on_chip(const lstm_desc_t* d) {
  BwdLayout o;
  return bwd_layout(d, &o) && o.res_nci > 0 ? 1 : 0;
}

lstm_status_t lstm_bwd_ex(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                          const void* R, const void* reserve, const float* dy, const float* dhT, const float* dcT,
                          float* dx, float* dh0, float* dc0, float* dW, float* dR, float* db, void* ws,
                          hipStream_t stream, const lstm_bwd_opts_t* opts) {
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
  const bool plain = opts && opts->plain_launch;
  // the step-wait limit: the default, the caller's, or (negative) none at all
  const long long timeout_us = (opts && opts->wait_timeout_us > 0) ? opts->wait_timeout_us
                               : (opts && opts->wait_timeout_us < 0) ? 0
                                                                     : kBwdTimeoutUs;
  return d->dtype == LSTM_BF16 ? bwd_run<true>(d, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db,
                                               ws, o, plain, timeout_us, stream)
                               : bwd_run<false>(d, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db,
                                                ws, o, plain, timeout_us, stream);
}

lstm_status_t lstm_bwd(const lstm_desc_t* d, const void* x, const void* h0, const float* c0, const void* W,
                       const void* R, const void* reserve, const float* dy, const float* dhT, const float* dcT,
                       float* dx, float* dh0, float* dc0, float* dW, float* dR, float* db, void* ws,
                       hipStream_t stream) {
  return lstm_bwd_ex(d, x, h0, c0, W, R, reserve, dy, dhT, dcT, dx, dh0, dc0, dW, dR, db, ws, stream, nullptr);
}

}  // extern "C"
