// Shared definitions of the stacked-LSTM forward kernels (gfx950 / CDNA4).
//
// Tile convention used by every kernel.  The four per-gate weight matrices are
// grouped into one 4H-row matrix ("Optimizing Performance of Recurrent Neural
// Networks on GPUs", proposed method: gate grouping).  Kernels walk that matrix
// in 16-row "M-tiles" whose rows are gate-interleaved:
//
//     tile mt, row rho (0..15)  <->  hidden unit j = 4*mt + rho/4, gate k = rho%4
//     caller row                 =   k*H + j           (gate blocks i, f, g, o)
//
// With the 16x16 MFMA output layout (lane l holds rows 4*(l/16)+r, column
// l%16, r = 0..3) each lane ends up holding the four gate pre-activations of
// one (unit, column) pair, so the gate non-linearities and the cell update run
// in registers straight after the product.
//
// Operand fragments: a "chunk" is 128 bytes of every row of a 16-row tile
// (32 fp32 or 64 bf16 K columns).  Lane l serves row l%16 and quad q = l/16;
// it holds two 16-byte halves: half h covers the chunk's columns
// [h*KC/2 + q*KC/8, h*KC/2 + (q+1)*KC/8).  The four quads' halves h together
// cover 64 contiguous bytes of the row, so every 16-byte load (global or LDS)
// of a wave touches whole 64-byte pieces.  The weight fragment and the
// activation fragment of a lane cover the same K indices, so the sum over K is
// exact whatever order the hardware uses inside one MFMA.  In LDS a block of
// 64 fragments is stored half-major (all lanes' half 0, then all lanes' half
// 1), so a wave's 16-byte LDS access is 1 KiB contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lstm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Frag {
  uint4 v[2];  // two 16-byte halves of one row's chunk (see above)
};

template <bool BF16>
struct Dt;
template <>
struct Dt<false> {
  typedef float T;
  static constexpr int KC = 32;  // K columns per chunk
  static constexpr int SZ = 4;
};
template <>
struct Dt<true> {
  typedef uint16_t T;
  static constexpr int KC = 64;
  static constexpr int SZ = 2;
};

__device__ __forceinline__ Frag zero_frag() {
  Frag f;
  f.v[0] = make_uint4(0, 0, 0, 0);
  f.v[1] = make_uint4(0, 0, 0, 0);
  return f;
}

// acc += A(16 x 32-byte K slice) * B(32-byte K slice x 16)
template <bool BF16>
__device__ __forceinline__ void mfma_frag(f32x4& acc, const Frag& a, const Frag& b);

template <>
__device__ __forceinline__ void mfma_frag<true>(f32x4& acc, const Frag& a, const Frag& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[0]),
                                                __builtin_bit_cast(bf16x8, b.v[0]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[1]),
                                                __builtin_bit_cast(bf16x8, b.v[1]), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_frag<false>(f32x4& acc, const Frag& a, const Frag& b) {
  const float* fa0 = reinterpret_cast<const float*>(&a.v[0]);
  const float* fb0 = reinterpret_cast<const float*>(&b.v[0]);
  const float* fa1 = reinterpret_cast<const float*>(&a.v[1]);
  const float* fb1 = reinterpret_cast<const float*>(&b.v[1]);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa0[e], fb0[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa1[e], fb1[e], acc, 0, 0, 0);
}

// Column of half h of quad q's fragment, relative to the chunk start.
template <bool BF16>
__device__ __forceinline__ int frag_col(int q, int h) {
  return h * (Dt<BF16>::KC / 2) + q * (Dt<BF16>::KC / 8);
}

// Quad q's fragment of the chunk that starts at element p of a row (16-byte
// aligned): two unconditional 16-byte loads.
template <bool BF16>
__device__ __forceinline__ Frag load_frag_vec(const typename Dt<BF16>::T* p, int q) {
  Frag f;
  f.v[0] = *reinterpret_cast<const uint4*>(p + frag_col<BF16>(q, 0));
  f.v[1] = *reinterpret_cast<const uint4*>(p + frag_col<BF16>(q, 1));
  return f;
}

// Quad q's fragment of the chunk starting at column k0 of the row at element
// offset `off` (row length K), zero-filling columns >= K.  `vec_ok` says
// 16-byte loads are aligned (every row start is a multiple of 16 bytes).
template <bool BF16>
__device__ __forceinline__ Frag load_frag_off(const void* base, long off, int k0, int q, int K, bool vec_ok) {
  typedef typename Dt<BF16>::T T;
  constexpr int N = 16 / Dt<BF16>::SZ;  // elements per half
  const T* row = reinterpret_cast<const T*>(base) + off;
  Frag f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = k0 + frag_col<BF16>(q, h);
    if (vec_ok && k + N <= K) {
      f.v[h] = *reinterpret_cast<const uint4*>(row + k);
    } else {
      T tmp[N];
#pragma unroll
      for (int e = 0; e < N; ++e) tmp[e] = (k + e < K) ? row[k + e] : T(0);
      __builtin_memcpy(&f.v[h], tmp, 16);
    }
  }
  return f;
}

// Same for row `row` of a row-major [rows][ld] matrix.
template <bool BF16>
__device__ __forceinline__ Frag load_frag(const void* base, long ld, long row, int k0, int q, int K, bool vec_ok) {
  return load_frag_off<BF16>(base, row * ld, k0, q, K, vec_ok);
}

// One wave-wide direct-to-LDS load of 16 bytes per lane: global
// `base` + `voff` (base wave-uniform, in scalar registers; voff this lane's byte
// offset) -> LDS byte `lds_off` + 16 * lane.  Written as inline assembly so
// that the compiler, which cannot tell which LDS bytes such a load writes,
// does not make every later LDS read wait for all of them; the kernels that
// use it track its completion themselves (s_waitcnt vmcnt; loads complete in
// issue order).  M0 carries the LDS address (those kernels use M0 for nothing
// else); its write needs one wait state before the load reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(voff), "s"(base)
               : "memory");
}

// f &= mask on every 32-bit word (mask 0 zeroes a fragment without a branch)
__device__ __forceinline__ void frag_mask(Frag& f, uint32_t m) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f.v[h].x &= m;
    f.v[h].y &= m;
    f.v[h].z &= m;
    f.v[h].w &= m;
  }
}

// A block of 64 fragments in LDS, half-major: lane l's half h at [h * 64 + l].
__device__ __forceinline__ void lds_put(uint4* blk, int lane, const Frag& f) {
  blk[lane] = f.v[0];
  blk[64 + lane] = f.v[1];
}
__device__ __forceinline__ Frag lds_get(const uint4* blk, int lane) {
  Frag f;
  f.v[0] = blk[lane];
  f.v[1] = blk[64 + lane];
  return f;
}

// Cells (lstm_cell_t).  LSTM and GRU tiles hold 4 units x 4 rows; the GRU's
// four rows per unit are r, z, the input half of n and the recurrent half of
// n, kept apart because the reset gate multiplies only the recurrent half
// ("three matrix groups" with the n group split in two).  A simple-RNN tile
// holds 16 units of one row each.
constexpr int kCellLstm = 0, kCellGru = 1, kCellRnnTanh = 2, kCellRnnRelu = 3;

__device__ __host__ __forceinline__ int cell_units_per_tile(int cell) { return cell >= kCellRnnTanh ? 16 : 4; }

struct CellRow {
  long w;  // input-weight row (-1: none -- past H, or the GRU's recurrent half of n)
  long r;  // recurrent-weight row (-1: none -- past H, or the GRU's input half of n)
  int bi;  // bias element (-1: past H)
};

// Rows behind tile row rho of M-tile mt (gate-interleaved order).
__device__ __forceinline__ CellRow cell_row(int cell, int mt, int rho, int H) {
  CellRow c{-1, -1, -1};
  if (cell >= kCellRnnTanh) {
    const int j = 16 * mt + rho;
    if (j < H) c.w = c.r = c.bi = j;
    return c;
  }
  const int j = 4 * mt + (rho >> 2), k = rho & 3;
  if (j >= H) return c;
  if (cell == kCellGru) {
    if (k < 2) {
      c.w = c.r = c.bi = (long)k * H + j;
    } else if (k == 2) {
      c.w = c.bi = 2L * H + j;  // W_n u + b_Wn
    } else {
      c.r = 2L * H + j;         // R_n h + b_Rn
      c.bi = 3 * H + j;
    }
    return c;
  }
  c.w = c.r = c.bi = (long)k * H + j;
  return c;
}

// Logistic function from its definition 1 / (1 + e^{-z}), with the hardware
// base-2 exponential (v_exp_f32) and reciprocal (v_rcp_f32).  Saturates to
// exactly 1.0 (e^{-z} underflows to 0) and 0.0 (e^{-z} overflows to +inf).
__device__ __forceinline__ float sigmoid_f(float z) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * z);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// tanh(z) = 2 sigmoid(2z) - 1; exact +-1 at saturation, absolute error ~1e-7 near 0.
__device__ __forceinline__ float tanh_f(float z) { return 2.0f * sigmoid_f(2.0f * z) - 1.0f; }

__device__ __forceinline__ float to_float(float v) { return v; }
__device__ __forceinline__ float to_float(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Data-valid exchange: a slot starts as all-ones words, which no stored value
// can equal once NaNs are canonical, so a reader knows an element has been
// written when it no longer holds the all-ones pattern.
// ---------------------------------------------------------------------------
constexpr uint32_t kSentinelWord = 0xffffffffu;

// A raw buffer over `bytes` bytes at p (loads past the end return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// 16 bytes at byte offset `off` of the buffer with the agent-coherence bit
// (sc1), the cache policy of agent-scope atomic loads: a re-read sees the
// writers' later stores instead of a stale cached copy.  One wave-wide load
// of contiguous lanes is still coalesced.
__device__ __forceinline__ uint4 load16_coherent(__amdgpu_buffer_rsrc_t r, int off) {
  constexpr int kSc1 = 16;  // cache-policy operand bit of sc1
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

// 1 if no element of the 16 bytes still holds the unwritten pattern
template <bool BF16>
__device__ __forceinline__ int written16(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  int ok = 1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (BF16)
      ok &= ((w[e] & 0xffffu) != 0xffffu && (w[e] >> 16) != 0xffffu) ? 1 : 0;
    else
      ok &= (w[e] != kSentinelWord) ? 1 : 0;
  }
  return ok;
}

template <bool BF16>
__device__ __forceinline__ typename Dt<BF16>::T from_float(float f);
template <>
__device__ __forceinline__ float from_float<false>(float f) { return f; }
template <>
__device__ __forceinline__ uint16_t from_float<true>(float f) { return f32_to_bf16(f); }

// the value with any NaN replaced by the canonical quiet NaN (never all ones)
template <bool BF16>
__device__ __forceinline__ typename Dt<BF16>::T canon_nan(typename Dt<BF16>::T v);
template <>
__device__ __forceinline__ float canon_nan<false>(float v) { return v == v ? v : __uint_as_float(0x7fc00000u); }
template <>
__device__ __forceinline__ uint16_t canon_nan<true>(uint16_t v) {
  return (v & 0x7fffu) > 0x7f80u ? (uint16_t)0x7fc0u : v;
}

}  // namespace lstm
