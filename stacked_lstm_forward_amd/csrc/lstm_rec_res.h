// Persistent recurrent kernel of one layer whose recurrent weights do not fit
// in LDS but do fit in LDS plus the register file (template definitions;
// instantiated by lstm_rec_res_inst.hip).
//
// The persistent-kernel idea ("Persistent RNNs") is to read R_l from memory
// once per sequence and keep it on chip for all T steps.  A 4H x H layer with
// H = 4096 in bf16 is 128 MiB: more than the 40 MiB of LDS of the whole chip,
// less than LDS plus the 128 MiB of vector registers.  Here each of the four
// waves of a workgroup (one per SIMD, so a wave may use all 512 registers)
// holds NRB fragment blocks of its K share in registers for the whole launch
// and the rest of its blocks in LDS; per step only h_{t-1} and the hoisted
// pre-activations are read from memory.
//
// Work split: wave w is K-group w of 4.  It owns chunks c = w, w + 4, ... of
// every M-tile of the workgroup (MW tiles) for every column tile (NW tiles),
// so it reads a quarter of h_{t-1} and the four waves together read it once.
// The launcher guarantees H = 4 * NCI chunks exactly (aligned rows), so every
// wave has NCI chunks and all its offsets are compile-time constants.
// Block b of a wave is (chunk index ci = b / MW, M-tile b % MW).  The last
// LPC = (NB - NRB) / NCI M-tiles of every chunk live in LDS, the others in
// registers.  A chunk's products take its LDS M-tiles first and then read the
// next chunk's LDS blocks into the same registers, so each LDS read has three
// register M-tiles' products to land (with all LDS blocks in the last chunks,
// each read only one block ahead, those chunks stalled on LDS and a pass took
// about twice its matrix-core time; two buffers read a whole chunk ahead cost
// the registers a deeper h ring needs more).  The NW column tiles are done
// one after the other (MW accumulators and one h fragment per chunk in
// registers); after each, the four K-groups' partial sums meet in LDS and
// K-group i finishes M-tile i of that column tile.  Multiplying both tiles of
// B = 32 in one pass (each weight block feeding two accumulators) was
// measured no faster: the passes are bound by how many h loads each wave
// keeps in flight, not by the hand-over between tiles.
//
// Exchange layout.  A wave's load of one fragment half touches 16 batch rows
// of h; from a row-major [B][H] buffer that is 16 pieces of 64 bytes 2H bytes
// apart, which the vector memory path serves several times slower than 1 KiB
// of contiguous memory.  So h_t also goes to Xf in exactly the order its
// readers load it: for column tile j and chunk c a 2 KiB block, half h at
// +1 KiB, lane l's 16 bytes at +16 l:
//     Xf[t][((j * nch + c) * 2 + h) * 64 + lane][8 bf16]
// and every load instruction of a step reads 1 KiB in one piece.  The row-major
// copy (the next layer's input, or y) is still written.  Step t reads slot t
// and writes slot t + 1; slot 0 holds h0, rewritten in this order before the
// launch (lstm_h0_frag), so every step takes the same path.  The loads are
// buffer loads whose only per-lane operand is one 32-bit offset: tile, chunk
// and half are compile-time offsets, which keeps registers for the ring.
// The step protocol (write-through stores, step counters, bounded waits) is the
// one of lstm_rec_kernel.  SAVE adds the training forward's stores (gates,
// cell and hidden states of every step); without them the inference kernel
// has the registers for one more chunk of h loads in flight.
#pragma once

#include "lstm_rec.h"

namespace lstm {

constexpr int kResWaves = 4;  // waves per workgroup = K-groups
// Register blocks defined as accumulation-register values.  Weights that only
// outgrow the architectural VGPRs are parked in the accumulation registers as
// spill slots and copied back before every MFMA (about four register moves per
// product); a value that is an accumulation register from its definition is
// read by the MFMA in place.  30 blocks (240 registers) leave room for the
// accumulators.
constexpr int kResAgprBlocks = 30;

// One register weight block (a wave's fragment of 16 rows x one chunk) in the
// MFMA operand type, and the products of one chunk into one accumulator: bf16
// two 16x16x32 MFMAs, fp32 eight 16x16x4 MFMAs, back to back (each takes the
// previous one's result without a register read).
template <bool BF16>
struct ResOps;
template <>
struct ResOps<true> {
  typedef bf16x8 V;
  static __device__ __forceinline__ V cast(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
  static __device__ __forceinline__ void chunk(f32x4& acc, const V& a0, const V& a1, const V& x0, const V& x1) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, x0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, x1, acc, 0, 0, 0);
  }
};
template <>
struct ResOps<false> {
  typedef f32x4 V;
  static __device__ __forceinline__ V cast(const uint4& u) { return __builtin_bit_cast(f32x4, u); }
  static __device__ __forceinline__ void chunk(f32x4& acc, const V& a0, const V& a1, const V& x0, const V& x1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[e], x0[e], acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[e], x1[e], acc, 0, 0, 0);
  }
};

template <bool BF16, int MW, int NW, int NCI, int NRB, bool SAVE>
__global__ void __launch_bounds__(64 * kResWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
lstm_rec_res_kernel(const RecParams P) {
  typedef typename Dt<BF16>::T T;
  constexpr int KC = Dt<BF16>::KC;
  constexpr int KS = kResWaves;
  constexpr int NB = MW * NCI;     // fragment blocks per wave
  constexpr int NLB = NB - NRB;    // ... of which in LDS
  constexpr int LPC = NLB / NCI;   // LDS M-tiles per chunk
  constexpr int RPC = MW - LPC;    // register M-tiles per chunk
  static_assert(NLB % NCI == 0, "LDS blocks spread evenly over the chunks");
  // h load chunks in flight per wave (bf16 H = 4096, B = 32: 2 -> 0.51 ms per
  // layer, 4 -> 0.42 (later 0.356), 5 -> 0.342 once the addressing and the
  // single LDS buffer below freed the registers, 6 spills; 3 with more than
  // two column tiles, whose per-tile state takes the registers).  A shape
  // with at most 36 register blocks has registers for a deeper ring.
  constexpr bool kRoomy = BF16 && NRB <= 36;
  constexpr int PD = kRoomy ? (NW <= 2 ? 8 : 6) : (NW <= 2 ? 5 : 3);
  static_assert(NRB >= 0 && NRB <= NB, "register blocks");
  static_assert(MW <= KS, "one finishing K-group per M-tile");
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_ok;

  const RecLayer& Lr = P.layer[0];
  const int bid = blockIdx.x;
  const int v = P.xcd_remap ? ((bid & 7) * (P.grid >> 3) + (bid >> 3)) : bid;
  if (v >= Lr.wg_count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4;
  const int H = P.H, B = P.B, T_ = P.T, cell = P.cell;
  const long slot = P.slot;
  constexpr int NCH = KS * NCI;           // chunks of a row of h
  constexpr int FB = 2048 / Dt<BF16>::SZ;  // elements of one 2 KiB fragment block
  constexpr int EPH = 16 / Dt<BF16>::SZ;   // elements of one lane's 16-byte half
  const int mt0 = v * Lr.mt_per_wg;
  const int mcnt = min(Lr.mt_per_wg, P.Mt - mt0);
  uint4* As = reinterpret_cast<uint4*>(smem) + (long)kg * NLB * 128;  // this wave's LDS blocks
  f32x4* red = reinterpret_cast<f32x4*>(smem + P.red_off);

  bool mval[MW];
  long arow[MW];
  uint32_t mr_[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    mval[i] = i < mcnt;
    const CellRow cr = cell_row(cell, mt0 + min(i, mcnt - 1), lane & 15, H);
    mr_[i] = (mval[i] && cr.r >= 0) ? 0xffffffffu : 0u;
    arow[i] = cr.r >= 0 ? cr.r : 0;
  }
  // byte offset of this lane's 16 bytes in its first block of a slot; tile j,
  // chunk slot ci and half hh add the compile-time (j NCH + ci KS) FB + hh FB/2
  // elements, so every h load of a step takes this one register
  const int hlane = (kg * FB + lane * EPH) * Dt<BF16>::SZ;

  // ---- this wave's weight blocks: M-tile i < RPC of chunk slot ci is
  // register block ci * RPC + i, M-tile i >= RPC is LDS block ci * LPC + i - RPC
  const T* Rp = reinterpret_cast<const T*>(Lr.R) + kg * KC;
  typedef ResOps<BF16> Ops;
  typedef typename Ops::V V;
  struct WB {
    V h[2];
  };
  WB wreg[NRB > 0 ? NRB : 1];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int ci = b / MW, i = b % MW;
    Frag f = load_frag_vec<BF16>(Rp + arow[i] * H + ci * KS * KC, q);
    frag_mask(f, mr_[i]);
    if (i < RPC) {
      const int r = ci * RPC + (i < RPC ? i : 0);
      WB w{{Ops::cast(f.v[0]), Ops::cast(f.v[1])}};
      if (r < kResAgprBlocks) {
        asm volatile("" : "+a"(w.h[0]));
        asm volatile("" : "+a"(w.h[1]));
      }
      wreg[r] = w;
    } else
      lds_put(As + (ci * LPC + i - RPC) * 128, lane, f);
  }

  // ---- per column tile j: this wave finishes M-tile kg (if it exists)
  const bool fm = kg < mcnt;
  const int funit = cell >= kCellRnnTanh ? 16 * (mt0 + kg) + 4 * q : 4 * (mt0 + kg) + q;
  // Xf position of this lane's unit in column tile 0 (the simple RNN's four
  // units funit..funit+3 share one 16-byte group, so they follow it)
  uint32_t fpos;
  {
    const int c = funit / KC, kc = funit % KC;
    const int hh = kc / (KC / 2), qq = (kc % (KC / 2)) / EPH, e = kc % EPH;
    fpos = c * FB + hh * (FB / 2) + (qq * 16 + (lane & 15)) * EPH + e;
  }
  bool flive[NW];
  float st[NW];
  const T* h0p = reinterpret_cast<const T*>(Lr.h0);
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int bc = 16 * j + (lane & 15);
    flive[j] = fm && j < P.ncnt && funit < H && bc < B;
    st[j] = 0.f;
    if (flive[j]) {
      const long o = (long)bc * H + funit;
      if (cell == kCellLstm && Lr.c0) st[j] = Lr.c0[o];
      if (cell == kCellGru && h0p) st[j] = to_float(h0p[o]);
    }
  }

  long long* trc = nullptr;
  if (P.trace && v % P.trace_stride == 0 && v / P.trace_stride < P.trace_wgs)
    trc = P.trace + (long)(v / P.trace_stride) * T_ * 8;
  auto stamp = [&](int t, int k) {
    if (trc && tid == 0) trc[t * 8 + k] = wall_clock64();
  };
  auto stamp_clk = [&](int t, int k) {
    if (trc && tid == 0) trc[t * 8 + k] = clock64();
  };

  T* Xp = reinterpret_cast<T*>(Lr.X);
  T* Xf = reinterpret_cast<T*>(Lr.F);
  const float* Gp = Lr.G;

  for (int t = 0; t < T_; ++t) {
    stamp(t, 0);
    stamp_clk(t, 6);
    // hoisted pre-activations of this lane's unit in column tile j: with up
    // to two tiles all are loaded before the wait, with more each one at the
    // start of its pass (registers).  Non-temporal: read once, they would
    // otherwise crowd h out of the caches.
    const float* gt = Gp + (long)t * P.Mt * B * 16;
    auto gload = [&](int j) {
      const long off = ((long)min(mt0 + kg, P.Mt - 1) * B + min(16 * j + (lane & 15), B - 1)) * 16 + 4 * q;
      return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gt + off));
    };
    constexpr bool kEarlyG = NW <= 2;
    f32x4 gq[kEarlyG ? NW : 1];
    if constexpr (kEarlyG) {
#pragma unroll
      for (int j = 0; j < NW; ++j) gq[j] = gload(j);
    }

    if (t > 0) {
      if (kg == 0) {
        const bool ok = wait_counts_serial(Lr.flags, Lr.wg_count, t, nullptr, 0, 0, P.err, P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s_ok) return;
    }
    // The pre-activations are needed in registers from here on: left alone
    // the compiler moves their loads after the next pass's h loads, and the
    // first gate phase then waits for those (loads complete in order).
    if constexpr (kEarlyG) {
#pragma unroll
      for (int j = 0; j < NW; ++j) asm volatile("" : "+v"(gq[j]));
    }
    stamp(t, 1);

    // h_{t-1} is load-order slot t (slot 0: h0, written there before the
    // launch); a null h0 is zero: nothing to multiply at t = 0
    const T* hsrc = (t > 0 || h0p) ? Xf + (long)t * P.fslot : nullptr;
    const __amdgpu_buffer_rsrc_t hrs = raw_buffer(hsrc, (int)(P.fslot * Dt<BF16>::SZ));
    T* fout = Xf + (long)(t + 1) * P.fslot;
    // row-major copy: y for the top layer, else the next layer's input
    T* rout = Lr.Yout ? reinterpret_cast<T*>(Lr.Yout) + (long)t * B * H : Xp + (long)t * slot;
    // (the host gives every resident layer either y or a row-major X)
    const bool last = (t == T_ - 1);

    T hl[4];      // the last tile's new h values (up to four units: the simple RNN)
    int nl = 0;   // ... how many
    f32x4 pl{};   // ... its pre-activations (training saves)
    // The h loads of the step form one stream over all column tiles, PD
    // chunks ahead: the next tile's first chunks are in flight while this
    // tile's sums are combined and its gates computed.  Load g is chunk slot
    // g % NCI of column tile g / NCI.
    Frag rb[PD];
    // One LDS buffer: a chunk's products take its LDS M-tiles first, and the
    // next chunk's LDS blocks are read into the same registers right after
    // them, three register M-tiles (six products) ahead of their use.  With
    // three column tiles two buffers, the next chunk's blocks read a whole
    // chunk ahead, time the same and are kept; with four, one buffer and
    // ordinary loads (below) spill least and run fastest.
    constexpr bool kLdsAhead = NW == 3;
    Frag al[kLdsAhead ? 2 : 1][LPC > 0 ? LPC : 1];
    auto issue = [&](Frag& dst, int g) {
      const int o = ((g / NCI) * NCH + (g % NCI) * KS) * FB * Dt<BF16>::SZ;
      if constexpr (NW == 4) {
        // (four column tiles: ordinary loads measured faster, 0.75 against
        // 0.88 ms per layer at bf16 H = 4096, B = 64)
        const char* pc = reinterpret_cast<const char*>(hsrc) + o + hlane;
        dst.v[0] = *reinterpret_cast<const uint4*>(pc);
        dst.v[1] = *reinterpret_cast<const uint4*>(pc + 1024);
      } else {
        dst.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(hrs, hlane, o, 0));
        dst.v[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(hrs, hlane, o + 1024, 0));
      }
    };
    if (hsrc) {
#pragma unroll
      for (int g = 0; g < PD && g < NW * NCI; ++g) issue(rb[g], g);
#pragma unroll
      for (int e = 0; e < LPC; ++e) al[0][e] = lds_get(As + e * 128, lane);
    }

#pragma unroll
    for (int j = 0; j < NW; ++j) {
      f32x4 acc[MW];
#pragma unroll
      for (int i = 0; i < MW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (hsrc) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ci = 0; ci < NCI; ++ci) {
          const int g = j * NCI + ci, s = g % PD;
          if constexpr (kLdsAhead) {
            if (ci + 1 < NCI || j + 1 < NW) {
              const int cn = (ci + 1) % NCI;
#pragma unroll
              for (int e = 0; e < LPC; ++e) al[cn & 1][e] = lds_get(As + (cn * LPC + e) * 128, lane);
            }
          }
#pragma unroll
          for (int ii = 0; ii < MW; ++ii) {
            const int i = kLdsAhead ? ii : (ii + RPC) % MW;  // one buffer: the LDS M-tiles (i >= RPC) first
            if constexpr (!kLdsAhead) {
              if (ii == LPC && (ci + 1 < NCI || j + 1 < NW)) {
                const int cn = (ci + 1) % NCI;
#pragma unroll
                for (int e = 0; e < LPC; ++e) al[0][e] = lds_get(As + (cn * LPC + e) * 128, lane);
              }
            }
            // no branch: a missing M-tile has zero weights and a missing
            // column tile a clamped h row; their sums are never finished
            const V x0 = Ops::cast(rb[s].v[0]), x1 = Ops::cast(rb[s].v[1]);
            V a0, a1;
            if (i < RPC) {
              a0 = wreg[ci * RPC + (i < RPC ? i : 0)].h[0];
              a1 = wreg[ci * RPC + (i < RPC ? i : 0)].h[1];
            } else {
              a0 = Ops::cast(al[kLdsAhead ? (ci & 1) : 0][i < RPC ? 0 : i - RPC].v[0]);
              a1 = Ops::cast(al[kLdsAhead ? (ci & 1) : 0][i < RPC ? 0 : i - RPC].v[1]);
            }
            // one accumulator's products back to back (bf16: a pair issues
            // every 16.9 cycles, alternating accumulators every 22.9, which
            // the scheduler would otherwise choose)
            Ops::chunk(acc[i], a0, a1, x0, x1);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (g + PD < NW * NCI) issue(rb[s], g + PD);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (j == 0) {
        stamp(t, 2);
        stamp_clk(t, 7);
      }

      // ---- every K-group leaves its partial sums of the column tile in LDS;
      // K-group kg then adds the four partials of M-tile kg in a fixed order
#pragma unroll
      for (int i = 0; i < MW; ++i) red[(i * KS + kg) * 64 + lane] = acc[i];
      __syncthreads();
      if (j == 0) stamp(t, 3);
      if (flive[j]) {
        f32x4 p = kEarlyG ? gq[kEarlyG ? j : 0] : gload(j);
#pragma unroll
        for (int r = 0; r < KS; ++r) p += red[(kg * KS + r) * 64 + lane];
        const long o = (long)(16 * j + (lane & 15)) * H + funit;
        const long fo = (long)j * NCH * FB + fpos;
        // The last tile's stores that no other workgroup reads in this launch
        // (the row-major copy, hT, the training saves) wait until the step is
        // published: the step counter then waits only for the exchange.
        const bool later = j == NW - 1;
        cell_update(cell, p, st[j], H - funit, [&](int u, float h) {
          const T hv = from_float<BF16>(h);
          store_coherent<BF16>(fout + fo + u, hv);
          if (later) {
            hl[u] = hv;
            nl = u + 1;
            return;
          }
          rout[o + u] = hv;
          if (last && Lr.hT) reinterpret_cast<T*>(Lr.hT)[o + u] = hv;
          if constexpr (SAVE) reinterpret_cast<T*>(Lr.save_h)[(long)t * B * H + o + u] = hv;
        });
        if (cell == kCellLstm && last && Lr.cT) Lr.cT[o] = st[j];
        if constexpr (SAVE) {
          if (later)
            pl = p;
          else if (cell == kCellLstm)
            save_lstm_step(Lr.save_gates, Lr.save_c, p, st[j], t, B, H, 16 * j + (lane & 15), funit);
        }
      }
      // the next column tile reuses the partial-sum area
      if (j + 1 < NW) __syncthreads();
    }
    stamp(t, 4);

    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(Lr.flags + (long)v * kFlagStride, t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stamp(t, 5);
    if (flive[NW - 1]) {
      const long o = (long)(16 * (NW - 1) + (lane & 15)) * H + funit;
      for (int u = 0; u < nl; ++u) {
        rout[o + u] = hl[u];
        if (last && Lr.hT) reinterpret_cast<T*>(Lr.hT)[o + u] = hl[u];
        if constexpr (SAVE) reinterpret_cast<T*>(Lr.save_h)[(long)t * B * H + o + u] = hl[u];
      }
      if constexpr (SAVE) {
        if (cell == kCellLstm)
          save_lstm_step(Lr.save_gates, Lr.save_c, pl, st[NW - 1], t, B, H, 16 * (NW - 1) + (lane & 15), funit);
      }
    }
  }
}

}  // namespace lstm
