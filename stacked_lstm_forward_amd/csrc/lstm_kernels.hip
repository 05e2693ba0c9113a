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
#include <algorithm>
#include <mutex>
#include <vector>

#include "lstm_common.h"
#include "lstm_params.h"

namespace lstm {

// ----------------------------------------------------------------------------
// Input projection GEMM
// ----------------------------------------------------------------------------
// Workgroup tile: MTW M-tiles x NTW column tiles (kGemmTileM x kGemmTileN, or
// 64 x 64 when the large tile would leave most CUs idle); wave (wm, wn) of the
// 2 x 2 waves computes MTW/2 M-tiles x NTW/2 column tiles.
// Per K chunk (128 bytes of every row) the workgroup stages 24 fragment blocks
// of 2 KiB in LDS, double-buffered (one barrier per chunk), while the next
// chunk's global loads are already in registers.
//
// VEC: K is a whole number of chunks and rows are 16-byte aligned, so every
// fragment load is unconditional (rows past the end are clamped to a valid row
// and their results dropped); the ragged path loads element by element.
// (k0: first column of the chunk; q: the lane's quad)
template <bool BF16, bool VEC>
__device__ __forceinline__ Frag gemm_load_a(const GemmParams& P, long arow, int k0, int q) {
  typedef typename Dt<BF16>::T T;
  if (VEC) return load_frag_vec<BF16>(reinterpret_cast<const T*>(P.W) + arow * P.K + k0, q);
  return arow >= 0 ? load_frag<BF16>(P.W, P.K, arow, k0, q, P.K, P.vec_ok_w) : zero_frag();
}

template <bool BF16, bool VEC>
__device__ __forceinline__ Frag gemm_load_b(const GemmParams& P, long boff, bool bval, int k0, int q) {
  typedef typename Dt<BF16>::T T;
  if (VEC) return load_frag_vec<BF16>(reinterpret_cast<const T*>(P.U) + boff + k0, q);
  return bval ? load_frag_off<BF16>(P.U, boff, k0, q, P.K, P.vec_ok_u) : zero_frag();
}

template <bool BF16, bool VEC, int MTW, int NTW>
__global__ void __launch_bounds__(kGemmThreads) lstm_input_gemm(const GemmParams P) {
  constexpr int KC = Dt<BF16>::KC;
  static_assert(MTW % 4 == 0 && NTW % 4 == 0, "every thread stages whole fragments");
  constexpr int WM = MTW / 2, WN = NTW / 2;    // M-tiles and column tiles per wave
  constexpr int NA = MTW * 64 / kGemmThreads;  // A fragments staged per thread per chunk
  constexpr int NB = NTW * 64 / kGemmThreads;  // B fragments staged per thread per chunk
  constexpr int STAGE = (MTW + NTW) * 128;     // 16-byte halves per LDS stage
  extern __shared__ __align__(16) unsigned char gsmem[];
  uint4* lds = reinterpret_cast<uint4*>(gsmem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (P.zero_ptr) {  // grid-stride zeroing of the error word and step counters
    const long nwg = (long)gridDim.x * gridDim.y;
    const long wg = (long)blockIdx.y * gridDim.x + blockIdx.x;
    for (long i = wg * kGemmThreads + tid; i < P.zero_count; i += nwg * kGemmThreads) P.zero_ptr[i] = 0;
  }
  if (P.fill_ptr) {  // grid-stride: the unwritten pattern of a data-valid exchange
    const long nwg = (long)gridDim.x * gridDim.y;
    const long wg = (long)blockIdx.y * gridDim.x + blockIdx.x;
    for (long i = wg * kGemmThreads + tid; i < P.fill_count; i += nwg * kGemmThreads) P.fill_ptr[i] = kSentinelWord;
  }
  const int mtb = blockIdx.y * MTW;        // first M-tile of this workgroup
  const int n0 = blockIdx.x * NTW * 16;    // first column
  const int nch = (P.K + KC - 1) / KC;
  const int q = lane >> 4;                 // same for every staging slot (256 is a multiple of 64)

  // staging slots of this thread: fragment f = tid + s * 256 of the A and B blocks
  long arow[NA];
  uint32_t amask[NA];  // 0 where the tile row has no input-weight row (its fragment is zero)
  long boff[NB];
  bool bval[NB];
#pragma unroll
  for (int s = 0; s < NA; ++s) {
    const int f = tid + s * kGemmThreads;
    const int mtl = f >> 6;
    long r = (mtb + mtl < P.Mt) ? cell_row(P.cell, mtb + mtl, f & 15, P.H).w : -1;
    amask[s] = r >= 0 ? 0xffffffffu : 0u;
    if (VEC && r < 0) r = 0;
    arow[s] = r;
  }
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    const int f = tid + s * kGemmThreads;
    const long col = n0 + 16 * (f >> 6) + (f & 15);
    bval[s] = col < P.N;
    const long cc = bval[s] ? col : P.N - 1;
    boff[s] = (cc / P.B) * P.u_slot + (cc % P.B) * P.K;  // column n: step n / B, sequence n % B
  }

  const int wm = wave & 1, wn = wave >> 1;
  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag ra[NA], rb[NB];
  if (nch > 0) {
#pragma unroll
    for (int s = 0; s < NA; ++s) ra[s] = gemm_load_a<BF16, VEC>(P, arow[s], 0, q);
#pragma unroll
    for (int s = 0; s < NB; ++s) rb[s] = gemm_load_b<BF16, VEC>(P, boff[s], bval[s], 0, q);
    if (P.cell == kCellGru) {
#pragma unroll
      for (int s = 0; s < NA; ++s) frag_mask(ra[s], amask[s]);
    }
#pragma unroll
    for (int s = 0; s < NA; ++s) lds_put(lds + (tid / 64 + s * (kGemmThreads / 64)) * 128, lane, ra[s]);
#pragma unroll
    for (int s = 0; s < NB; ++s) lds_put(lds + (MTW + tid / 64 + s * (kGemmThreads / 64)) * 128, lane, rb[s]);
    __syncthreads();
  }
  for (int c = 0; c < nch; ++c) {
    // next chunk's loads go out before this chunk's MFMAs (clamped, unconditional)
    const int cn = min(c + 1, nch - 1);
#pragma unroll
    for (int s = 0; s < NA; ++s) ra[s] = gemm_load_a<BF16, VEC>(P, arow[s], cn * KC, q);
#pragma unroll
    for (int s = 0; s < NB; ++s) rb[s] = gemm_load_b<BF16, VEC>(P, boff[s], bval[s], cn * KC, q);
    __builtin_amdgcn_sched_barrier(0);
    const uint4* st = lds + (c & 1) * STAGE;
    Frag b[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) b[j] = lds_get(st + (MTW + WN * wn + j) * 128, lane);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const Frag a = lds_get(st + (WM * wm + i) * 128, lane);
#pragma unroll
      for (int j = 0; j < WN; ++j) mfma_frag<BF16>(acc[i][j], a, b[j]);
    }
    if (c + 1 < nch) {
      uint4* nx = lds + ((c + 1) & 1) * STAGE;
      if (P.cell == kCellGru) {  // rows with no input weights (the recurrent half of n)
#pragma unroll
        for (int s = 0; s < NA; ++s) frag_mask(ra[s], amask[s]);
      }
#pragma unroll
      for (int s = 0; s < NA; ++s) lds_put(nx + (tid / 64 + s * (kGemmThreads / 64)) * 128, lane, ra[s]);
#pragma unroll
      for (int s = 0; s < NB; ++s) lds_put(nx + (MTW + tid / 64 + s * (kGemmThreads / 64)) * 128, lane, rb[s]);
    }
    __syncthreads();
  }

  // epilogue: add bias, write [T][Mt][B][16]
  typedef typename Dt<BF16>::T T;
  const T* bias = reinterpret_cast<const T*>(P.bias);
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int mt = mtb + WM * wm + i;
    if (mt >= P.Mt) continue;
    f32x4 bv;  // this lane's four rows 4*(lane/16) + k of the tile (rows past H are never read)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int bi = cell_row(P.cell, mt, 4 * (lane >> 4) + k, P.H).bi;
      bv[k] = bi >= 0 ? to_float(bias[bi]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const long col = n0 + 16 * (WN * wn + j) + (lane & 15);
      if (col >= P.N) continue;
      const long t = col / P.B, bb = col % P.B;
      float* dst = P.G + ((t * P.Mt + mt) * P.B + bb) * 16 + 4 * (lane >> 4);
      *reinterpret_cast<f32x4*>(dst) = acc[i][j] + bv;
    }
  }
}

// Fast path of the input projection (K a whole number of chunks, every row
// 16-byte aligned, operands below 2^31 elements): a 256 x (16 NT) workgroup
// tile, 8 waves (two per SIMD) of 64 x (8 NT) -- 4 x NT/2 MFMA tiles, the
// accumulators in the accumulation registers.  Operands go from global memory
// straight into LDS with gfx950's direct-to-LDS loads (a wave-wide 16-byte load
// lands lane l at byte 16 l of its LDS destination).
//
// Pipeline.  The W rows (A operand) have three LDS stages and the U columns
// (B operand) two: W comes from HBM (every layer's 128 MiB W is read once per
// forward and does not stay in the last-level cache), U mostly from the L2 or
// the last-level cache, so W's loads get two chunks of lead and U's one.  One
// barrier per chunk, in its middle:
//   1. read the fragments of the chunk's second K-half from LDS, interleaved
//      with the MFMAs of its first half (fragments read during the previous
//      chunk);
//   2. wait for this wave's loads of the next chunk, and for the reads of 1;
//   3. barrier: the next chunk is in LDS and nobody reads this chunk's stages
//      any more;
//   4. issue the loads of chunk c + 2 (U) and c + 3 (W) into those stages;
//   5. read the next chunk's first-half fragments, interleaved with the MFMAs
//      of this chunk's second half.
// The loads are issued from inline assembly.  The compiler cannot tell which
// LDS bytes a direct-to-LDS load writes, so after a builtin one it makes every
// later LDS read wait for all loads in flight -- which would wait for the loads
// just issued in 4.  Here their completion is tracked by hand (the vmcnt
// waits in 2; loads complete in issue order).
constexpr int kDmaTiles = 16;             // M-tiles per workgroup (and at most column tiles)
constexpr int kDmaWaves = 8;
constexpr int kDmaThreads = 64 * kDmaWaves;
constexpr int kDmaAStages = 3, kDmaBStages = 2;
constexpr int kDmaALoads = 2 * kDmaTiles / kDmaWaves;  // direct-to-LDS loads of W per wave per chunk
constexpr int kDmaBLoads = 2 * kDmaTiles / kDmaWaves;  // ... of U (at most; NT < 16 repeats the last)

__host__ __device__ constexpr unsigned dma_lds_bytes(int nt) {
  return (kDmaAStages * kDmaTiles + kDmaBStages * nt) * 2048u;
}

template <bool BF16>
__device__ __forceinline__ void mfma_half(f32x4& acc, const uint4& a, const uint4& b);
template <>
__device__ __forceinline__ void mfma_half<true>(f32x4& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0,
                                                0, 0);
}
template <>
__device__ __forceinline__ void mfma_half<false>(f32x4& acc, const uint4& a, const uint4& b) {
  const float* fa = reinterpret_cast<const float*>(&a);
  const float* fb = reinterpret_cast<const float*>(&b);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], acc, 0, 0, 0);
}

// One workgroup tile of the direct-to-LDS product: M-tiles mtb .. mtb + 15,
// NT column tiles from column n0, K chunks c_first .. c_first + nch - 1; the
// stage layout is that of NTS column tiles (NT <= NTS), so tiles of two widths
// can share one launch.  Each of the two column-halves of waves takes NT / 2.
// PLAIN: rows in order (row m of tile mt is 16 mt + m, rows >= H unused) and
// the product written to C[m][n] without bias (the backward pass's gradient
// products); z > 0 selects partial-sum buffer z - 1 of a split K.
template <bool BF16, int NT, int NTS, bool PLAIN>
__device__ __forceinline__ void dma_tile(const GemmParams& P, int mtb, long n0, int z, int c_first, int nch) {
  static_assert(NT % 2 == 0 && NT <= NTS && NTS <= kDmaTiles, "column tiles per workgroup");
  constexpr int WM = kDmaTiles / 4;          // M-tiles per wave (4 M-quarters x 2 column halves)
  constexpr int WN = NT / 2;                 // column tiles per wave
  typedef typename Dt<BF16>::T T;
  constexpr int KC = Dt<BF16>::KC;
  constexpr uint32_t kABytes = kDmaTiles * 2048, kBBytes = NTS * 2048;  // one stage
  extern __shared__ __align__(16) unsigned char gsmem[];
  const uint4* lds = reinterpret_cast<const uint4*>(gsmem);
  // LDS byte address of the dynamic area (M0 takes LDS addresses, not generic ones)
  typedef __attribute__((address_space(3))) unsigned char lds_byte_t;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_byte_t*)gsmem;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Staging.  A block holds its 16 rows' 128-byte chunks row by row, 8 pieces
  // of 16 bytes each, piece p of row r in slot p ^ ((r >> 1) & 7).  One
  // wave-wide load fills half a block: 8 whole rows, lane l row 8i + l/8, slot
  // l%8, so every load reads whole 128-byte lines (a load of 16 rows x 64 bytes
  // costs the texture path several times more), and the swizzle keeps the
  // fragment reads below free of bank conflicts.  Rows and columns past the
  // end are clamped to valid ones (results unused).
  // Wave w loads W load-slots w*kDmaALoads + k and U load-slots w*kDmaBLoads + k
  // (slot j: block j/2, half j%2; U slots past 2 NT repeat the last one).
  constexpr int EPH = 16 / Dt<BF16>::SZ;  // elements of one 16-byte piece
  const T* Wg = reinterpret_cast<const T*>(P.W) + (long)c_first * KC;
  const T* Ug = reinterpret_cast<const T*>(P.U) + (long)c_first * KC;
  uint32_t srcA[kDmaALoads], srcB[kDmaBLoads];  // byte offsets (the launcher keeps them below 2^32)
  uint32_t dstA[kDmaALoads], dstB[kDmaBLoads];  // byte offsets inside a stage (wave-uniform)
#pragma unroll
  for (int k = 0; k < kDmaALoads; ++k) {
    const int j = wave * kDmaALoads + k, blk = j / 2, i = j % 2;
    const int r = 8 * i + (lane >> 3);
    const long piece = (lane & 7) ^ ((r >> 1) & 7);
    const int mt = mtb + blk;
    const long row = mt >= P.Mt ? -1 : PLAIN ? (16 * mt + r < P.H ? 16 * mt + r : -1) : cell_row(P.cell, mt, r, P.H).w;
    srcA[k] = (uint32_t)(((row < 0 ? 0 : row) * P.K + piece * EPH) * (long)sizeof(T));
    dstA[k] = blk * 2048 + i * 1024;
  }
#pragma unroll
  for (int k = 0; k < kDmaBLoads; ++k) {
    const int j = min(wave * kDmaBLoads + k, 2 * NT - 1), blk = j / 2, i = j % 2;
    const int r = 8 * i + (lane >> 3);
    const long piece = (lane & 7) ^ ((r >> 1) & 7);
    long col = n0 + 16 * blk + r;
    col = col < P.N ? col : P.N - 1;
    // column n: step n / B, sequence n % B
    srcB[k] = (uint32_t)(((col / P.B) * P.u_slot + (col % P.B) * P.K + piece * EPH) * (long)sizeof(T));
    dstB[k] = blk * 2048 + i * 1024;
  }
  // chunk indices are clamped, so every iteration issues the same loads
  // (the chunk's column offset goes into the scalar base address)
  auto load_A = [&](int c) {
    const uint32_t st = lds_base + (uint32_t)(c % kDmaAStages) * kABytes;
    const T* base = Wg + (long)min(c, nch - 1) * KC;
#pragma unroll
    for (int k = 0; k < kDmaALoads; ++k) dma16(base, srcA[k], st + dstA[k]);
  };
  auto load_B = [&](int c) {
    const uint32_t st = lds_base + kDmaAStages * kABytes + (uint32_t)(c % kDmaBStages) * kBBytes;
    const T* base = Ug + (long)min(c, nch - 1) * KC;
#pragma unroll
    for (int k = 0; k < kDmaBLoads; ++k) dma16(base, srcB[k], st + dstB[k]);
  };

  // this lane's fragment halves (row lane%16, piece 4h + lane/16) in a block
  const int fr_ = lane & 15, fsw = (fr_ >> 1) & 7;
  const int foff0 = fr_ * 8 + ((0 + q) ^ fsw), foff1 = fr_ * 8 + ((4 + q) ^ fsw);
  const int wm = wave & 3, wn = wave >> 2;
  uint4 fa[2][WM], fb[2][WN];  // fragment halves: [K-half][tile]
  auto read_half = [&](int c, int h) {
    const uint4* sa = lds + (c % kDmaAStages) * (kABytes / 16);
    const uint4* sb = lds + (kDmaAStages * kABytes + (c % kDmaBStages) * kBBytes) / 16;
    const int fo = h ? foff1 : foff0;
#pragma unroll
    for (int j = 0; j < WN; ++j) fb[h][j] = sb[(WN * wn + j) * 128 + fo];
#pragma unroll
    for (int i = 0; i < WM; ++i) fa[h][i] = sa[(WM * wm + i) * 128 + fo];
  };

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_phase = [&](int h) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) mfma_half<BF16>(acc[i][j], fa[h][i], fb[h][j]);
  };
  // one fragment read, then a few MFMAs (the reads fill the other register
  // set, so no wait separates them from these MFMAs)
  constexpr int kReads = WM + WN;                       // fragment reads per K-half
  constexpr int kMfmas = WM * WN * (BF16 ? 1 : 4);      // MFMAs per K-half
  constexpr int kPer = kMfmas / kReads;
  auto interleave = [&]() {
#pragma unroll
    for (int k = 0; k < kReads; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);  // then MFMAs
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kPer * kReads, 0);
  };

  // prologue: W chunks 0 and 1, U chunk 0 in flight; wait for chunk 0
  load_A(0);
  load_B(0);
  load_A(1);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaALoads) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  load_B(1);
  load_A(2);
  read_half(0, 0);
  for (int c = 0; c < nch; ++c) {
    // 1. second-half fragments of chunk c while the first half multiplies
    read_half(c, 1);
    mfma_phase(0);
    interleave();
    // 2. this wave's loads of chunk c + 1 have landed (only W's chunk c + 2
    //    may still be in flight), and so have the reads above
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kDmaALoads) : "memory");
    // 3. everybody's have; nobody reads chunk c's stages any more
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // 4. refill them: U chunk c + 2, W chunk c + 3
    load_B(c + 2);
    load_A(c + 3);
    // 5. first-half fragments of chunk c + 1 while the second half multiplies
    read_half(c + 1, 0);
    mfma_phase(1);
    interleave();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last (redundant) loads have landed

  if constexpr (PLAIN) {
    float* const C = z == 0 ? P.C : P.C2 + (long)(z - 1) * P.split_stride;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int mt = mtb + WM * wm + i;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const long col = n0 + 16 * (WN * wn + j) + (lane & 15);
        if (col >= P.N) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int row = 16 * mt + 4 * q + k;
          if (row < P.H) C[(long)row * P.ldc + col] = acc[i][j][k];
        }
      }
    }
    return;
  }

  // epilogue: add bias, write [T][Mt][B][16]
  const T* bias = reinterpret_cast<const T*>(P.bias);
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int mt = mtb + WM * wm + i;
    if (mt >= P.Mt) continue;
    f32x4 bv;       // this lane's four rows 4*(lane/16) + k of the tile (rows past H are never read)
    bool wrow[4];   // false: the row has no input weights (the GRU's recurrent half of n), so its
                    // product (of a clamped stand-in row) is dropped and G holds the bias alone
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const CellRow cr = cell_row(P.cell, mt, 4 * q + k, P.H);
      bv[k] = cr.bi >= 0 ? to_float(bias[cr.bi]) : 0.f;
      wrow[k] = cr.w >= 0;
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const long col = n0 + 16 * (WN * wn + j) + (lane & 15);
      if (col >= P.N) continue;
      const long t = col / P.B, bb = col % P.B;
      float* dst = P.G + ((t * P.Mt + mt) * P.B + bb) * 16 + 4 * q;
      f32x4 g;
#pragma unroll
      for (int k = 0; k < 4; ++k) g[k] = wrow[k] ? acc[i][j][k] + bv[k] : bv[k];
      // streamed past the caches: the recurrence reads each step's rows once,
      // long after, and the caches keep serving this product's operands
      __builtin_nontemporal_store(g, reinterpret_cast<f32x4*>(dst));
    }
  }
}

// The grouped input projection (or a plain product) on the direct-to-LDS
// kernel.  NT column tiles per workgroup (16, or 14 when that packs the
// columns into fewer rounds of workgroups than 16 would: see launch_dma);
// with P.nbig > 0 (NT = 14 only) the column blocks of every M-block are
// P.nblk tiles, the first P.nbig of them NT wide and the others NT - 2 (fewer
// idle CUs in the last round: the 1600 columns of a 4096-wide layer at
// B = 32, T = 50 make 2 x 14 + 6 x 12 column tiles per M-block; 0.196 ->
// 0.189 ms per layer).
template <bool BF16, int NT, bool PLAIN>
__global__ void __launch_bounds__(kDmaThreads) lstm_input_gemm_dma(const GemmParams P) {
  constexpr int KC = Dt<BF16>::KC;
  const int tid = threadIdx.x;
  if (P.zero_ptr) {  // grid-stride zeroing of the error word and step counters
    const long nwg = (long)gridDim.x * gridDim.y;
    const long wg = (long)blockIdx.y * gridDim.x + blockIdx.x;
    for (long i = wg * kDmaThreads + tid; i < P.zero_count; i += nwg * kDmaThreads) P.zero_ptr[i] = 0;
  }
  if (P.fill_ptr) {  // grid-stride: the unwritten pattern of a data-valid exchange
    const long nwg = (long)gridDim.x * gridDim.y;
    const long wg = (long)blockIdx.y * gridDim.x + blockIdx.x;
    for (long i = wg * kDmaThreads + tid; i < P.fill_count; i += nwg * kDmaThreads) P.fill_ptr[i] = kSentinelWord;
  }
  // Tile order: the 1-D grid (a multiple of 8) goes round-robin over the 8
  // XCDs, so workgroup ids are first regrouped into one contiguous range per
  // XCD, and that range walks the (M, N) tile grid in groups of 4 M-blocks
  // with N inner: the ~32 workgroups an XCD runs at once share 4 blocks of W
  // rows and 8 blocks of U columns through their L2 instead of each pulling
  // its own from memory.
  const int nM = (P.Mt + kDmaTiles - 1) / kDmaTiles;
  const bool mixed = P.nbig > 0;
  const int nN = mixed ? P.nblk : (P.N + NT * 16 - 1) / (NT * 16);
  const int total = nM * nN;
  const int per_xcd = (int)gridDim.x >> 3;
  const int vs = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  // plain products may split K: workgroup vs takes chunk range vs / total
  const int ks = (PLAIN && P.ksplit > 1) ? P.ksplit : 1;
  if (vs >= total * ks) return;
  const int z = vs / total, v = vs % total;
  constexpr int kGroupM = 4;
  const int in_group = kGroupM * nN;
  const int first_m = (v / in_group) * kGroupM;
  const int gsize = min(nM - first_m, kGroupM);
  const int mblk = first_m + (v % in_group) % gsize;
  const int nblk = (v % in_group) / gsize;
  const int mtb = mblk * kDmaTiles;                  // first M-tile
  const int c_first = z * (P.K / KC) / ks;           // this workgroup's chunk range of K
  const int nch = (z + 1) * (P.K / KC) / ks - c_first;
  if constexpr (NT == 14) {  // (a second body in the 16-wide kernel measured slower: 0.157 -> 0.168 ms)
    if (mixed && nblk >= P.nbig) {
      const long n0 = ((long)P.nbig * NT + (long)(nblk - P.nbig) * (NT - 2)) * 16;
      dma_tile<BF16, NT - 2, NT, PLAIN>(P, mtb, n0, z, c_first, nch);
      return;
    }
  }
  dma_tile<BF16, NT, NT, PLAIN>(P, mtb, (long)nblk * NT * 16, z, c_first, nch);
}

// C[m][n] += C2[z S + m ldc + n] for z = 0 .. parts - 1, in that order: the
// partial sums of a plain product whose K range was split.
__global__ void __launch_bounds__(256) gemm_split_sum(float* C, const float* C2, long long S, int parts, int M, int N,
                                                      long long ldc) {
  const long long n = (long long)M * N;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long o = (i / N) * ldc + i % N;
    float v = C[o];
#pragma unroll 4
    for (int z = 0; z < parts; ++z) v += C2[z * S + o];
    C[o] = v;
  }
}

// Zeroes n ints (the error word and the step counters) when no input GEMM
// runs before the recurrence to do it.  A fill kernel rather than a memset, so
// the call stays capturable in a HIP graph.
__global__ void __launch_bounds__(256) lstm_clear(int* p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0;
}

// h0 of one layer, row-major [B][H], rewritten in the order the register-
// resident kernel loads its recurrent operand (lstm_rec_res.h: for column tile
// j and chunk c a block of FB elements, half hh at +FB/2, lane qq*16 + r at
// +EPH (qq*16 + r)), so that its first step reads h0 like every later h_{t-1}.
// Rows >= B of the last column tile are not written (their sums are never
// finished).
template <typename T, int KC>
__global__ void __launch_bounds__(256) lstm_h0_frag(const T* __restrict__ h0, T* __restrict__ dst, int B, int H,
                                                    long long tile_elems) {
  constexpr int EPH = 16 / (int)sizeof(T), FB = 2048 / (int)sizeof(T);
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)B * H) return;
  const int b = (int)(i / H), k = (int)(i % H);
  const int c = k / KC, kc = k % KC;
  const int hh = kc / (KC / 2), qq = (kc % (KC / 2)) / EPH, e = kc % EPH;
  dst[(b >> 4) * tile_elems + (long long)c * FB + hh * (FB / 2) + (qq * 16 + (b & 15)) * EPH + e] = h0[i];
}

// ----------------------------------------------------------------------------
// Host-side launchers (the only code outside this directory's kernels that
// touches them).  The recurrent kernel's instantiations live in
// lstm_rec_inst.hip, compiled once per (dtype, weight source).
// ----------------------------------------------------------------------------
#define LSTM_DECL(d, s, w) const void* rec_kernel_ptr_##d##_##s##_w##w(int mw, int nw, bool vec, bool frag);
LSTM_DECL(f32, lds, 4) LSTM_DECL(f32, stream, 4) LSTM_DECL(bf16, lds, 4) LSTM_DECL(bf16, stream, 4)
LSTM_DECL(f32, lds, 8) LSTM_DECL(f32, stream, 8) LSTM_DECL(bf16, lds, 8) LSTM_DECL(bf16, stream, 8)
#undef LSTM_DECL

const void* rec_res_kernel_ptr_shape0(int nw, bool save);
const void* rec_res_kernel_ptr_shape1(int nw, bool save);
const void* rec_res_kernel_ptr_shape2(int nw, bool save);
static_assert(kResShapes == 3, "one instantiation unit per resident shape");

const void* rec_res_kernel_ptr(bool bf16, int mw, int nw, int nci, int nrb, bool save) {
  const void* (*const per_shape[kResShapes])(int, bool) = {rec_res_kernel_ptr_shape0, rec_res_kernel_ptr_shape1,
                                                      rec_res_kernel_ptr_shape2};
  for (int k = 0; k < kResShapes; ++k) {
    const ResShape& r = kResShape[k];
    if ((r.bf16 != 0) == bf16 && r.mw == mw && r.nci == nci && r.nrb == nrb) return per_shape[k](nw, save);
  }
  return nullptr;
}

namespace {
const void* rec_kernel_fn(bool bf16, bool stream, bool vec, int nwv, int mw, int nw, bool frag) {
  if (nwv == 8) {
    if (bf16)
      return stream ? rec_kernel_ptr_bf16_stream_w8(mw, nw, vec, frag) : rec_kernel_ptr_bf16_lds_w8(mw, nw, vec, frag);
    return stream ? rec_kernel_ptr_f32_stream_w8(mw, nw, vec, frag) : rec_kernel_ptr_f32_lds_w8(mw, nw, vec, frag);
  }
  if (bf16)
    return stream ? rec_kernel_ptr_bf16_stream_w4(mw, nw, vec, frag) : rec_kernel_ptr_bf16_lds_w4(mw, nw, vec, frag);
  return stream ? rec_kernel_ptr_f32_stream_w4(mw, nw, vec, frag) : rec_kernel_ptr_f32_lds_w4(mw, nw, vec, frag);
}
}  // namespace

// A kernel's dynamic-LDS limit and its occupancy for a given LDS size and
// block do not change between calls: set and query them once per process and
// device instead of on every forward call (each is a runtime call on the host
// path of every launch).  The limit only ever grows, to the largest size any
// launch of that kernel has asked for.  blocks_per_cu may be null.
hipError_t prepare_fn(const void* fn, int lds_bytes, int block, int* blocks_per_cu) {
  struct Limit {
    const void* fn;
    int dev, lds;  // largest dynamic LDS set for fn on dev
  };
  struct Occ {
    const void* fn;
    int dev, lds, block, blocks;
  };
  static std::mutex mu;
  static std::vector<Limit> limits;
  static std::vector<Occ> occ;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  Limit* lim = nullptr;
  for (Limit& l : limits)
    if (l.fn == fn && l.dev == dev) lim = &l;
  if (!lim || lim->lds < lds_bytes) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    if (lim)
      lim->lds = lds_bytes;
    else
      limits.push_back(Limit{fn, dev, lds_bytes});
  }
  if (!blocks_per_cu) return hipSuccess;
  for (const Occ& o : occ)
    if (o.fn == fn && o.dev == dev && o.lds == lds_bytes && o.block == block) {
      *blocks_per_cu = o.blocks;
      return hipSuccess;
    }
  int b = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, block, lds_bytes);
  if (e != hipSuccess) return e;
  occ.push_back(Occ{fn, dev, lds_bytes, block, b});
  *blocks_per_cu = b;
  return hipSuccess;
}

template <int MTW, int NTW>
const void* input_gemm_fn(bool bf16, bool vec) {
  if (bf16)
    return vec ? reinterpret_cast<const void*>(&lstm_input_gemm<true, true, MTW, NTW>)
               : reinterpret_cast<const void*>(&lstm_input_gemm<true, false, MTW, NTW>);
  return vec ? reinterpret_cast<const void*>(&lstm_input_gemm<false, true, MTW, NTW>)
             : reinterpret_cast<const void*>(&lstm_input_gemm<false, false, MTW, NTW>);
}

const void* dma_kernel(bool bf16, int nt, bool plain) {
  if (plain)
    return nt == 14 ? (bf16 ? reinterpret_cast<const void*>(&lstm_input_gemm_dma<true, 14, true>)
                            : reinterpret_cast<const void*>(&lstm_input_gemm_dma<false, 14, true>))
                    : (bf16 ? reinterpret_cast<const void*>(&lstm_input_gemm_dma<true, 16, true>)
                            : reinterpret_cast<const void*>(&lstm_input_gemm_dma<false, 16, true>));
  return nt == 14 ? (bf16 ? reinterpret_cast<const void*>(&lstm_input_gemm_dma<true, 14, false>)
                          : reinterpret_cast<const void*>(&lstm_input_gemm_dma<false, 14, false>))
                  : (bf16 ? reinterpret_cast<const void*>(&lstm_input_gemm_dma<true, 16, false>)
                          : reinterpret_cast<const void*>(&lstm_input_gemm_dma<false, 16, false>));
}

// Byte offsets of the direct-to-LDS kernel are 32-bit: whether p's operands
// stay below 2^32 bytes and every row is whole 16-byte pieces of whole chunks.
bool dma_fits(bool bf16, const GemmParams& p) {
  const bool whole = (p.K % (bf16 ? Dt<true>::KC : Dt<false>::KC)) == 0;
  const long long esz = bf16 ? 2 : 4;
  const long long w_bytes = (long long)p.Mt * 16 * p.K * esz;  // at most G*H rows (tile rows past H are clamped)
  const long long u_bytes = ((long long)((p.N - 1) / p.B) * p.u_slot + (long long)p.B * p.K) * esz;
  return p.vec_ok_w && p.vec_ok_u && whole && w_bytes < (1LL << 32) && u_bytes < (1LL << 32);
}

hipError_t launch_dma(bool bf16, const GemmParams& p, hipStream_t s) {
  // 14 column tiles per workgroup instead of 16 when that needs no more
  // rounds of one workgroup per CU: each round then loads 30 fragment
  // blocks per chunk instead of 32 (the 16384 x 1600 projection of a
  // 4096-wide bf16 layer at B = 32, T = 50: 448 tiles in 2 rounds become 512
  // in 2 rounds)
  const int nM = (p.Mt + kDmaTiles - 1) / kDmaTiles;
  auto rounds = [&](int nt) {
    const int cus = p.num_cus > 0 ? p.num_cus : 256;
    return (nM * ((p.N + nt * 16 - 1) / (nt * 16)) + cus - 1) / cus;
  };
  int nt = rounds(14) * (kDmaTiles + 14) < rounds(16) * (kDmaTiles + 16) ? 14 : 16;
  if (p.ksplit > 1) nt = 16;  // (the split was chosen for 16)
  GemmParams q = p;
  q.nbig = 0, q.nblk = 0;
  if (p.ksplit <= 1 && nt == 14) {
    // Mixed widths when they shorten the busiest CU: the tiles of each
    // XCD's range go, in launch order, to whichever of its CUs frees first
    // (a tile costs its load blocks per chunk, 16 + width); compare with
    // uniform tiles of the chosen width.
    const int cus = p.num_cus > 0 ? p.num_cus : 256;
    const int nct = (p.N + 15) / 16;
    auto makespan = [&](int nblk, int nbig, int wbig, int wsmall) {
      const int total = nM * nblk;
      const int grid = (total + 7) & ~7, per_xcd = grid / 8, cpx = std::max(1, cus / 8);
      long long worst = 0;
      std::vector<long long> busy(cpx);
      for (int x = 0; x < 8; ++x) {
        std::fill(busy.begin(), busy.end(), 0LL);
        for (int v = x * per_xcd; v < std::min(total, (x + 1) * per_xcd); ++v) {
          const int in_group = 4 * nblk, first_m = (v / in_group) * 4, gsize = std::min(nM - first_m, 4);
          const int nb = (v % in_group) / gsize;
          const int w = nb < nbig ? wbig : wsmall;
          auto it = std::min_element(busy.begin(), busy.end());
          *it += kDmaTiles + w;
        }
        worst = std::max(worst, *std::max_element(busy.begin(), busy.end()));
      }
      return worst;
    };
    // (the choice is a function of the shape: made once per process)
    struct Seen {
      int Mt, N, cus, nbig, nblk;
    };
    static std::mutex mu;
    static std::vector<Seen> seen;
    std::lock_guard<std::mutex> lock(mu);
    auto hit = std::find_if(seen.begin(), seen.end(),
                            [&](const Seen& e) { return e.Mt == p.Mt && e.N == p.N && e.cus == cus; });
    if (hit == seen.end()) {
      Seen e{p.Mt, p.N, cus, 0, 0};
      const int nblk_u = (nct + nt - 1) / nt;
      const long long uniform = makespan(nblk_u, nblk_u, nt, nt);
      // the fewest blocks of widths nt and nt - 2 that cover the columns
      const int k = (nct + nt - 1) / nt;
      const int need = nct - (nt - 2) * k;  // columns beyond k narrow blocks
      const int nbig = need <= 0 ? 0 : (need + 1) / 2;
      if (nbig > 0 && nbig < k && makespan(k, nbig, nt, nt - 2) < uniform) e.nbig = nbig, e.nblk = k;
      seen.push_back(e);
      hit = seen.end() - 1;
    }
    q.nbig = hit->nbig, q.nblk = hit->nblk;
  }
  auto kernel_of = [&](int n) { return dma_kernel(bf16, n, p.C != nullptr); };
  const void* fn = kernel_of(nt);
  // 16 column tiles take all 160 KiB of a CU's LDS; a device that gives a
  // workgroup less falls back to 14 (152 KiB)
  hipError_t e = prepare_fn(fn, (int)dma_lds_bytes(nt), kDmaThreads, nullptr);
  if (e != hipSuccess && nt == 16) {
    (void)hipGetLastError();
    nt = 14;
    fn = kernel_of(nt);
    e = prepare_fn(fn, (int)dma_lds_bytes(nt), kDmaThreads, nullptr);
  }
  if (e != hipSuccess) return e;
  const unsigned lds = dma_lds_bytes(nt);
  const int nblk = q.nbig > 0 ? q.nblk : (p.N + nt * 16 - 1) / (nt * 16);
  const int tiles = nblk * nM * (p.ksplit > 1 ? p.ksplit : 1);
  const dim3 grid((tiles + 7) & ~7);  // a multiple of the 8 XCDs (extra workgroups only help zeroing)
  void* args[] = {&q};
  return hipLaunchKernel(fn, grid, dim3(kDmaThreads), args, lds, s);
}

hipError_t launch_input_gemm(bool bf16, const GemmParams& p, hipStream_t s) {
  constexpr int kMTW = kGemmTileM / 16, kNTW = kGemmTileN / 16;
  // the 256 x 256 direct-to-LDS kernel pays off on long K (measured: 0.45 vs
  // 0.53 ms at K = 4096, 0.33 vs 0.35 ms at K = 1536); short K keeps the
  // register-staged 256 x 128 kernel, whose smaller tiles fill more CUs
  if (p.K >= 1024 && dma_fits(bf16, p)) return launch_dma(bf16, p, s);
  const bool vec = p.vec_ok_w && p.vec_ok_u && (p.K % (bf16 ? Dt<true>::KC : Dt<false>::KC)) == 0;
  // A problem the 256 x 128 tile covers with fewer than kGemmSmallGrid
  // workgroups (a short sequence, a small batch) leaves most CUs idle while
  // each workgroup runs its whole K loop: 64 x 64 tiles spread it further
  // (1-layer H = 128, B = 8, T = 16, fp32: 2 workgroups and 33 us, 16).
  constexpr int kGemmSmallGrid = 64;
  const int big = ((p.N + kGemmTileN - 1) / kGemmTileN) * ((p.Mt + kMTW - 1) / kMTW);
  const bool small = big < kGemmSmallGrid;
  const int mtw = small ? 4 : kMTW, ntw = small ? 4 : kNTW;
  const unsigned lds = 2 * (mtw + ntw) * 64 * sizeof(Frag);
  const dim3 grid((p.N + ntw * 16 - 1) / (ntw * 16), (p.Mt + mtw - 1) / mtw);
  const void* fn = small ? input_gemm_fn<4, 4>(bf16, vec) : input_gemm_fn<kMTW, kNTW>(bf16, vec);
  hipError_t e = prepare_fn(fn, (int)lds, kGemmThreads, nullptr);
  if (e != hipSuccess) return e;
  void* args[] = {const_cast<GemmParams*>(&p)};
  return hipLaunchKernel(fn, grid, dim3(kGemmThreads), args, lds, s);
}

// C[m][n] = sum over k of A[m][k] B[n][k] for m < M, n < N (A [M][K] and
// B [N][K] row-major in the workload's dtype, C fp32 with row stride ldc) on
// the direct-to-LDS kernel.  hipErrorNotSupported when the operands do not
// suit it (the caller then uses another kernel); nothing is enqueued then.
hipError_t launch_gemm_plain(bool bf16, const void* A, const void* B, float* C, long long ldc, int M, int N, int K,
                             int num_cus, float* C2, long long c2_floats, hipStream_t s) {
  const long long esz = bf16 ? 2 : 4;
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  GemmParams p{};
  p.W = A, p.U = B, p.C = C, p.ldc = ldc;
  p.K = K, p.H = M, p.Mt = (M + 15) / 16, p.B = N, p.N = N, p.u_slot = 0;
  p.vec_ok_w = al16(A) && (K * esz) % 16 == 0;
  p.vec_ok_u = al16(B) && (K * esz) % 16 == 0;
  p.cell = kCellRnnTanh;
  p.num_cus = num_cus;
  if (M < 1 || N < 1 || K < 1 || !dma_fits(bf16, p)) return hipErrorNotSupported;
  // A product of few 256 x 256 tiles with a long K (the input gradient
  // dP W_l: 1600 x 4096 x 16384 makes 112 tiles on 256 CUs; a small layer's
  // weight gradients, 4H x H x T B, a handful) splits K so the tiles fill the
  // chip: up to 16 ranges of at least 8 chunks, as many as the spare buffer
  // holds, the partial sums added in order afterwards.
  const int cus = num_cus > 0 ? num_cus : 256;
  const int tiles16 = ((p.Mt + kDmaTiles - 1) / kDmaTiles) * ((N + 255) / 256);
  const int nch = K / (bf16 ? Dt<true>::KC : Dt<false>::KC);
  const long long cfl = (long long)M * ldc;
  int ks = 1;
  while (ks < 16 && tiles16 * (ks + 1) <= cus && nch / (ks + 1) >= 8 && C2 && (long long)ks * cfl <= c2_floats &&
         ldc >= N)
    ++ks;
  if (ks > 1) p.C2 = C2, p.split_stride = cfl, p.ksplit = ks;
  hipError_t e = launch_dma(bf16, p, s);
  if (e != hipSuccess || ks == 1) return e;
  const long long n = (long long)M * N;
  hipLaunchKernelGGL(gemm_split_sum, dim3((unsigned)std::min<long long>((n + 255) / 256, 4096)), dim3(256), 0, s, C,
                     static_cast<const float*>(C2), cfl, ks - 1, M, N, ldc);
  return hipGetLastError();
}

hipError_t launch_clear(int* p, long long n, hipStream_t s) {
  const long long blocks = std::min<long long>((n + 255) / 256, 1024);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lstm_clear, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_h0_frag(bool bf16, const void* h0, void* dst, int B, int H, long long tile_elems, hipStream_t s) {
  const long long n = (long long)B * H;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL((lstm_h0_frag<uint16_t, 64>), dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(h0), static_cast<uint16_t*>(dst), B, H, tile_elems);
  else
    hipLaunchKernelGGL((lstm_h0_frag<float, 32>), dim3(blocks), dim3(256), 0, s, static_cast<const float*>(h0),
                       static_cast<float*>(dst), B, H, tile_elems);
  return hipGetLastError();
}

hipError_t rec_prepare(bool bf16, bool stream, bool vec, bool frag, int nwv, int mw, int nw, int lds_bytes,
                       int* max_blocks_per_cu) {
  const void* fn = rec_kernel_fn(bf16, stream, vec, nwv, mw, nw, frag);
  if (!fn) return hipErrorInvalidValue;
  return prepare_fn(fn, lds_bytes, 64 * nwv, max_blocks_per_cu);
}

hipError_t res_prepare(bool bf16, int mw, int nw, int nci, int nrb, bool save, int lds_bytes, int* max_blocks_per_cu) {
  const void* fn = rec_res_kernel_ptr(bf16, mw, nw, nci, nrb, save);
  if (!fn) return hipErrorInvalidValue;
  return prepare_fn(fn, lds_bytes, 64 * 4, max_blocks_per_cu);
}

hipError_t launch_rec_res(bool bf16, int nci, int nrb, const RecParams& p, int lds_bytes, bool plain, hipStream_t s) {
  const void* fn = rec_res_kernel_ptr(bf16, p.mw, p.nw, nci, nrb, p.layer[0].save_gates != nullptr);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<RecParams*>(&p)};
  if (plain) return hipLaunchKernel(fn, dim3(p.grid), dim3(64 * 4), args, (unsigned)lds_bytes, s);
  return hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(64 * 4), args, (unsigned)lds_bytes, s);
}

hipError_t launch_rec(bool bf16, bool stream, bool vec, bool frag, int nwv, const RecParams& p, int lds_bytes,
                      bool plain, hipStream_t s) {
  const void* fn = rec_kernel_fn(bf16, stream, vec, nwv, p.mw, p.nw, frag);
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {const_cast<RecParams*>(&p)};
  if (plain) return hipLaunchKernel(fn, dim3(p.grid), dim3(64 * nwv), args, (unsigned)lds_bytes, s);
  return hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(64 * nwv), args, (unsigned)lds_bytes, s);
}

}  // namespace lstm
