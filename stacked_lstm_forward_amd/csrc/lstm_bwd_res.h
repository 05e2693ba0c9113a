// Persistent kernel of one layer's recurrent chain in the backward pass, with
// R_l^T kept on chip (template definitions; instantiated in
// lstm_bwd_res_inst.hip).
//
// The chain runs t = T-1 .. 0: dh_t = dY[t] + dh_rec, dc_t = dh_t o (1 -
// tanh(c_t)^2) + dc_rec, the gate derivatives dp_t, dc_rec <- dc_t f_t and
// dh_rec <- dp_t R_l (a product over K = 4H).  Streaming R_l from memory for
// that product every step reads 128 MiB per step at bf16 H = 4096; here, as in
// the forward's resident kernel, R_l^T stays in registers and LDS for the
// whole chain, and per step only dp_{t+1} is read.
//
// Work split (H a multiple of 256: H / 16 workgroups per batch group, one
// per CU; 256 at H = 4096).  The K index of the product is ordered unit-major, k = 4 u + g
// for gate g of unit u (R_l^T and the exchanged dp use the same order, so the
// product is unchanged).  Workgroup v = 4 ug + kq (of its group) owns output units 64 ug ..
// 64 ug + 63 (four M-tiles of 16) and the K quarter kq: input units H / 4 kq
// .. H / 4 (kq + 1) - 1, all four gates.  So it reads a quarter of dp_{t+1}
// per step (256 KiB at bf16 H = 4096, B = 32, not all of it: one workgroup per
// 16 units reading all 1 MiB took 18.5 us a step, bound by those reads), and
// the four workgroups of a unit group add their partial sums: each leaves its
// sums in a per-step slot, then workgroup (ug, kq) adds the four partials of
// M-tile kq in a fixed order and finishes those 16 units (the elementwise
// part) for every sequence.
// Inside a workgroup, as in the forward: wave w is K-group w of 4 and owns
// chunks w, w + 4, ... of the quarter (NCI = H / (4 KC) chunks of KC: 16 at
// bf16 H = 4096) of every M-tile: NRB fragment blocks in registers and the
// others in LDS, spread evenly over the chunks (at H = 4096: 48 and one per
// chunk, 16; smaller layers: three M-tiles of every chunk in registers, one
// in LDS); the column tiles run one after the other with one stream of dp
// loads five chunks ahead; the four waves' sums meet in LDS.
// Batch groups: sequences are independent, so when the GPU has room the
// column tiles are split over `groups` copies of this grid (group jg takes
// tiles NW jg .. NW jg + NW - 1, holds its own copy of R_l^T and runs its own
// chain with its own counters); a small layer then spreads its products over
// more CUs.
//
// One M-tile per workgroup over all of K (MW = 1, small layers whose R_l^T
// rows fit in LDS) is the same with one unit group per workgroup and no K
// split: no partial sums, the four waves' sums go straight into the
// elementwise part.
//
// Step protocol, per workgroup one counter (two with K quarters; agent-scope
// stores, bounded waits with the error word):
//   flags_d[v] = s + 1 once iteration s's dp (of step T - 1 - s) is written;
//   flags_p[v] = s + 1 once iteration s's partial sums are written (MW = 4).
// Iteration s > 0 waits for flags_d >= s of the workgroups of its batch group
// that finish its K part's units (H / 64 of them per quarter: 64 kq .. 64 kq
// + 63 at H = 4096; all H / 16 with MW = 1), multiplies, and with K quarters
// publishes its partials and waits for flags_p >= s + 1 of its unit group's
// four workgroups.  The iteration after the last step computes
// dh0 = dp_0 R_l.
#pragma once

#include "lstm_rec_res.h"

namespace lstm {

struct BwdResParams {
  const uint4* RTf;     // R_l^T in load order, K unit-major: block (M-tile, chunk) of 128 x 16 bytes
  void* DPx;            // dp_t in load order (K unit-major), [T] slots of xslot elements (dtype)
  long long xslot;
  float* part;          // partial sums: [T + 1][wgs][NW][4 M-tiles][64 lanes][4] per iteration
  const float* dY;      // [T][B][H] gradient reaching h_t from above
  const float* gates;   // [T][B][4H] activated gates (i, f, g, o)
  const float* cs;      // [T][B][H] cell states
  const float* c0;      // [B][H] or null (zeros)
  const float* dhT;     // [B][H] or null
  const float* dcT;     // [B][H] or null
  float* dP;            // [T][B][4H] gate derivatives
  void* dPh;            // [T][B][4H] the same in the dtype
  float* dh0;           // [B][H] or null
  float* dc0;           // [B][H] or null
  int* flags_d;         // per-workgroup counters, kFlagStride apart (zero on entry)
  int* flags_p;         // ... of the partial sums
  int* err;             // device error word
  long long timeout_ticks;
  int T, B, H, nch;
  int wgs;     // workgroups in all: groups x H / 16
  int groups;  // batch groups: group jg takes column tiles NW jg .. NW jg + NW - 1 (an independent chain)
  int grid, xcd_remap;
};

constexpr int kBwdResWaves = 4;
constexpr int kBwdResMW = 4;  // M-tiles (of 16 output units) per workgroup
constexpr int kBwdResPf = 7;  // per-step inputs of one (unit, sequence): dY, i, f, g, o, c_t, c_{t-1}

// Fragment blocks (of each wave's MW NCI) kept in registers, for NCI chunks
// per wave: with four M-tiles (K quarters), 48 of 64 at NCI = 16 (bf16
// H = 4096), else three of the four M-tiles of every chunk; with one M-tile
// (all of K) none, every block in LDS.
__host__ __device__ constexpr int bwd_res_nrb(int nci, int mw) { return mw == 1 ? 0 : nci >= 16 ? 48 : 3 * nci; }

// The instantiated shapes, (bf16, NCI, MW).  MW = 4: each workgroup four
// M-tiles over a K quarter, NCI = H / (4 KC): H = 4096, 256, 512, 1024, 1536,
// 2048 and 3072 in bf16, 256, 512 and 1024 in fp32 (fp32 at H = 2048 would
// hold 48 blocks in registers and spills).  MW = 1: each workgroup one
// M-tile over all of K, its R_l^T rows in LDS (64 H x size of an element
// bytes), NCI = H / KC: H = 128, 256 and 512 in both dtypes.  Each is built
// with 1, 2 and 4 batch tiles (MW = 4, NCI = 16: 1 and 2), one compile unit
// per shape (lstm_bwd_res_inst.hip).
struct BwdResShape {
  int bf16, nci, mw;
};
constexpr int kBwdResShapes = 16;
constexpr BwdResShape kBwdResShape[kBwdResShapes] = {
    {1, 16, 4}, {1, 1, 4}, {1, 2, 4},  {1, 4, 4}, {1, 6, 4},  {1, 8, 4}, {0, 2, 4},  {0, 4, 4},
    {0, 8, 4},  {1, 4, 1}, {1, 8, 1},  {0, 8, 1}, {0, 16, 1}, {1, 2, 1}, {0, 4, 1}, {1, 12, 4}};

// LDS bytes: the LDS weight blocks, one tile's K-group sums, the parked inputs.
__host__ __device__ constexpr int bwd_res_lds_bytes(int nw, int nci, int mw) {
  return kBwdResWaves * (mw * nci - bwd_res_nrb(nci, mw)) * 2048 + mw * kBwdResWaves * 64 * 16 +
         nw * kBwdResPf * 256 * 4;
}

// A 16-byte store written through to the device-wide coherence point (the
// cache policy of an agent-scope atomic store), for data other workgroups
// read after a step counter says it is there.
__device__ __forceinline__ void store16_coherent(__amdgpu_buffer_rsrc_t r, int off, const f32x4& v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int kSc1 = 16;  // cache-policy operand bit of sc1
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kSc1);
}

// Floats of one iteration's partial-sum slot.
__host__ __device__ constexpr long long bwd_res_part_floats(int wgs, int nw) {
  return (long long)wgs * nw * kBwdResMW * 64 * 4;
}

template <bool BF16, int NW, int NCI, int MW>
__global__ void __launch_bounds__(64 * kBwdResWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
lstm_bwd_res_kernel(const BwdResParams P) {
  typedef typename Dt<BF16>::T T;
  typedef ResOps<BF16> Ops;
  typedef typename Ops::V V;
  constexpr int SZ = Dt<BF16>::SZ, KC = Dt<BF16>::KC;
  static_assert(MW == 1 || MW == kBwdResMW, "four M-tiles over a K quarter, or one over all of K");
  constexpr int KS = kBwdResWaves, NRB = bwd_res_nrb(NCI, MW);
  constexpr int NB = MW * NCI, NLB = NB - NRB, LPC = NLB / NCI, RPC = MW - LPC;
  static_assert(NLB % NCI == 0 && LPC >= 1, "LDS blocks spread evenly over the chunks");
  constexpr int FB = 2048 / SZ, EPH = 16 / SZ;
  constexpr int PD = 5;  // chunks of dp loads in flight per wave
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_ok;

  const int bid = blockIdx.x;
  const int v = P.xcd_remap ? ((bid & 7) * (P.grid >> 3) + (bid >> 3)) : bid;
  if (v >= P.wgs) return;
  // batch group jg, and within it unit group ug (MW M-tiles) and K part kq
  // (of MW: quarters, or all of K)
  const int wgs0 = P.wgs / P.groups, jg = v / wgs0, v0 = v - jg * wgs0;
  const int ug = v0 / MW, kq = v0 % MW;
  const int gw0 = jg * wgs0;  // the group's first workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = P.H, B = P.B, T_ = P.T, nch = P.nch;
  uint4* As = reinterpret_cast<uint4*>(smem) + (long)kg * NLB * 128;
  f32x4* red = reinterpret_cast<f32x4*>(smem + KS * NLB * 2048);
  f32x4* pf = reinterpret_cast<f32x4*>(smem + KS * NLB * 2048 + MW * KS * 64 * 16);
  // LDS byte address of this wave's input area (M0 takes LDS addresses)
  typedef __attribute__((address_space(3))) unsigned char lds_byte_t;
  const uint32_t pf_lds = (uint32_t)(uintptr_t)(lds_byte_t*)(smem + KS * NLB * 2048 + MW * KS * 64 * 16) +
                          (uint32_t)(kg * kBwdResPf) * 1024;

  // ---- this wave's blocks of R_l^T: M-tile 4 ug + i, chunk 64 kq + kg + 4 ci
  // (M-tile i < RPC of chunk slot ci in register block ci RPC + i, the others
  // in LDS block ci LPC + i - RPC)
  struct WB {
    V h[2];
  };
  WB wreg[NRB > 0 ? NRB : 1];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int ci = b / MW, i = b % MW;
    const uint4* blk = P.RTf + ((long)(MW * ug + i) * nch + NCI * KS * kq + kg + KS * ci) * 128;
    Frag f;
    f.v[0] = blk[lane];
    f.v[1] = blk[64 + lane];
    if (i < RPC) {
      const int r = ci * RPC + (i < RPC ? i : 0);
      WB w{{Ops::cast(f.v[0]), Ops::cast(f.v[1])}};
      if (r < kResAgprBlocks) {
        asm volatile("" : "+a"(w.h[0]));
        asm volatile("" : "+a"(w.h[1]));
      }
      wreg[r] = w;
    } else {
      lds_put(As + (ci * LPC + i - RPC) * 128, lane, f);
    }
  }

  // ---- what this thread finishes: wave kg < NW finishes column tile kg of
  // M-tile kq, lane `lane` the four units u0 .. u0 + 3 of sequence fb (the
  // lane's four sums of that tile, so every per-step load and store is 16
  // bytes); the other waves only multiply
  const int u0 = 16 * (MW * ug + kq) + 4 * (lane >> 4);
  const int jt = NW * jg + kg;                       // its column tile
  const int fb = min(16 * jt + (lane & 15), B - 1);  // clamped for the loads of padding lanes
  const bool fwave = kg < NW;                        // wave-uniform
  const bool fin = fwave && 16 * jt + (lane & 15) < B;
  f32x4 dcrec = f32x4{0.f, 0.f, 0.f, 0.f};
  if (fin && P.dcT) dcrec = *reinterpret_cast<const f32x4*>(P.dcT + (long)fb * H + u0);
  // dp of the four units in load order: k = 4 u0 .. 4 u0 + 15 lie in chunk
  // 4 u0 / KC from column kc0 = 4 u0 % KC: half kc0 / (KC / 2), quads from
  // (kc0 % (KC / 2)) / EPH on, each quad one lane's 16 bytes (two units' four
  // gates in bf16, one unit's in fp32), 256 bytes apart; byte offset of the
  // first in column tile kg's part of an exchange slot:
  const int xkc = (4 * u0) % KC;
  const int xoff = ((jt * nch + (4 * u0) / KC) * FB + (xkc / (KC / 2)) * (FB / 2) +
                    (((xkc % (KC / 2)) / EPH) * 16 + (fb & 15)) * EPH) *
                   SZ;
  const int xbytes = (int)(P.xslot * SZ);

  T* DPx = reinterpret_cast<T*>(P.DPx);
  T* dPh = reinterpret_cast<T*>(P.dPh);
  // byte offset of this lane's 16 bytes in its wave's first dp block of a
  // column tile; tile, chunk slot and half are compile-time offsets
  const int hlane = (kg * FB + lane * EPH) * SZ;
  const long long pslot = bwd_res_part_floats(P.wgs, NW);

  for (int s = 0; s <= T_; ++s) {
    const int t = T_ - 1 - s;  // step whose dp this iteration computes (-1: dh0 only)
    if (t < 0 && !P.dh0) break;
    // per-step inputs of this thread's units, loaded before the waits
    // straight into this wave's LDS area (no registers held across the
    // waits; read after a vmcnt wait): dY, i, f, g, o, c_t, c_{t-1}.  Bases
    // per step (wave-uniform), 32-bit byte offsets within a step's rows.
    if (t >= 0 && fwave) {
      const long tb = (long)t * B;
      const uint32_t rh = (uint32_t)(fb * H + u0) * 4, rg = (uint32_t)(fb * 4 * H + u0) * 4;
      dma16(P.dY + tb * H, rh, pf_lds);
#pragma unroll
      for (int k = 0; k < 4; ++k) dma16(P.gates + tb * 4 * H, rg + (uint32_t)(k * H) * 4, pf_lds + (1 + k) * 1024);
      dma16(P.cs + tb * H, rh, pf_lds + 5 * 1024);
      if (t > 0)
        dma16(P.cs + (tb - B) * H, rh, pf_lds + 6 * 1024);
      else if (P.c0)
        dma16(P.c0, rh, pf_lds + 6 * 1024);
      else
        pf[(kg * kBwdResPf + 6) * 64 + lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (s > 0) {
      // dp_{t+1} of this K part's units: finished by the part's workgroups in
      // this batch group (H / 64 of them per quarter: 64 kq .. 64 kq + 63 at
      // H = 4096; all H / 16 with one M-tile per workgroup)
      if (kg == 0) {
        const int nq = wgs0 / MW;
        const bool ok = wait_counts_serial(P.flags_d + (long)(gw0 + nq * kq) * kFlagStride, nq, s, nullptr, 0, 0, P.err,
                                           P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s_ok) return;
    }
    f32x4 dhr = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s > 0) {
      // ---- this workgroup's partial dh_rec = dp_{t+1} R_l over its K quarter
      const T* src = DPx + (long)(t + 1) * P.xslot + ((long)NW * jg * nch + NCI * KS * kq) * FB;
      const __amdgpu_buffer_rsrc_t drs = raw_buffer(src, (int)((long)NW * nch * FB * SZ));
      Frag rb[PD];
      Frag al[MW == 1 ? 2 : LPC];  // (one M-tile: this chunk's and the next chunk's LDS block)
      auto issue = [&](Frag& dst, int g) {
        const int o = ((g / NCI) * nch + (g % NCI) * KS) * FB * SZ;
        dst.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(drs, hlane, o, 0));
        dst.v[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(drs, hlane, o + 1024, 0));
      };
#pragma unroll
      for (int g = 0; g < PD && g < NW * NCI; ++g) issue(rb[g], g);
#pragma unroll
      for (int e = 0; e < LPC; ++e) al[e] = lds_get(As + e * 128, lane);
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        f32x4 acc[MW];
#pragma unroll
        for (int i = 0; i < MW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ci = 0; ci < NCI; ++ci) {
          const int g = j * NCI + ci, sl = g % PD;
          if constexpr (MW == 1) {
            // every block in LDS: the next chunk's read into the other buffer
            // while this chunk's MFMAs run
            if (ci + 1 < NCI || j + 1 < NW) al[(g + 1) & 1] = lds_get(As + ((ci + 1) % NCI) * 128, lane);
            Ops::chunk(acc[0], Ops::cast(al[g & 1].v[0]), Ops::cast(al[g & 1].v[1]), Ops::cast(rb[sl].v[0]),
                       Ops::cast(rb[sl].v[1]));
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int ii = 0; ii < (MW == 1 ? 0 : MW); ++ii) {
            // the LDS M-tiles first; the next chunk's LDS blocks are then
            // read into the same registers, three products ahead of use
            const int i = (ii + RPC) % MW;
            if (ii == LPC && (ci + 1 < NCI || j + 1 < NW)) {
              const int cn = (ci + 1) % NCI;
#pragma unroll
              for (int e = 0; e < LPC; ++e) al[e] = lds_get(As + (cn * LPC + e) * 128, lane);
            }
            const V x0 = Ops::cast(rb[sl].v[0]), x1 = Ops::cast(rb[sl].v[1]);
            V a0, a1;
            if (i < RPC) {
              a0 = wreg[ci * RPC + (i < RPC ? i : 0)].h[0];
              a1 = wreg[ci * RPC + (i < RPC ? i : 0)].h[1];
            } else {
              a0 = Ops::cast(al[i < RPC ? 0 : i - RPC].v[0]);
              a1 = Ops::cast(al[i < RPC ? 0 : i - RPC].v[1]);
            }
            Ops::chunk(acc[i], a0, a1, x0, x1);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (g + PD < NW * NCI) issue(rb[sl], g + PD);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the four K-groups' sums of the tile meet in LDS; K-group kg adds
        // those of M-tile kg in a fixed order and leaves them in the slot
        // (one M-tile: wave j, which finishes tile j, adds them into dh_rec)
#pragma unroll
        for (int i = 0; i < MW; ++i) red[(i * KS + kg) * 64 + lane] = acc[i];
        __syncthreads();
        if (MW > 1 || kg == j) {
          f32x4 p = red[((MW > 1 ? kg : 0) * KS) * 64 + lane];
#pragma unroll
          for (int r = 1; r < KS; ++r) p += red[((MW > 1 ? kg : 0) * KS + r) * 64 + lane];
          if constexpr (MW > 1) {
            const __amdgpu_buffer_rsrc_t prs =
                raw_buffer(P.part + (long)s * pslot + (long)v * (NW * MW * 256), NW * MW * 1024);
            store16_coherent(prs, ((j * MW + kg) * 64 + lane) * 16, p);
          } else {
            dhr = p;
          }
        }
        if (j + 1 < NW) __syncthreads();  // the next tile reuses the area
      }
    }
    if (s > 0 && MW > 1) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(P.flags_p + (long)v * kFlagStride, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // ---- the unit group's four partial sums of M-tile kq, in a fixed order
      if (kg == 0) {
        const bool ok = wait_counts_serial(P.flags_p + (long)(gw0 + 4 * ug) * kFlagStride, 4, s + 1, nullptr, 0, 0, P.err,
                                           P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s_ok) return;
      if (fwave) {
        const f32x4* pin = reinterpret_cast<const f32x4*>(P.part + (long)s * pslot + (long)(gw0 + 4 * ug) * (NW * MW * 256)) +
                           (kg * MW + kq) * 64 + lane;
        dhr = pin[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) dhr += pin[w * (NW * MW * 64)];
      }
    }

    // ---- the elementwise part of this thread's units (the exchange copy of
    // dp first: the step counter waits only for it; dP and its dtype copy,
    // read by later kernels, are stored after the counter)
    f32x4 dps[4];  // dps[g][e]: gate g of unit u0 + e
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS input loads
    if (fin) {
      const long fbh = (long)fb * H + u0;
      if (t < 0) {
        *reinterpret_cast<f32x4*>(P.dh0 + fbh) = dhr;
      } else {
        const f32x4* x = pf + kg * kBwdResPf * 64 + lane;
        const f32x4 ig = x[1 * 64], fg = x[2 * 64], gg = x[3 * 64], og = x[4 * 64], ct = x[5 * 64], cp = x[6 * 64];
        const f32x4 dh =
            x[0] + (s > 0 ? dhr : (P.dhT ? *reinterpret_cast<const f32x4*>(P.dhT + fbh) : f32x4{0.f, 0.f, 0.f, 0.f}));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float tc = tanh_f(ct[e]);
          const float dc = dh[e] * og[e] * (1.f - tc * tc) + dcrec[e];
          dps[0][e] = dc * gg[e] * ig[e] * (1.f - ig[e]);
          dps[1][e] = dc * cp[e] * fg[e] * (1.f - fg[e]);
          dps[2][e] = dc * ig[e] * (1.f - gg[e] * gg[e]);
          dps[3][e] = dh[e] * tc * og[e] * (1.f - og[e]);
          dcrec[e] = dc * fg[e];
        }
        // the exchange: unit u0 + e's four gates are elements 4 e .. 4 e + 3
        // of the 16 (EPH per 16-byte quad)
        const __amdgpu_buffer_rsrc_t xrs = raw_buffer(DPx + (long)t * P.xslot, xbytes);
        if constexpr (BF16) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            unsigned w[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const int e = 2 * p + h / 2, g = 2 * (h % 2);
              w[h] = (unsigned)from_float<true>(dps[g][e]) | ((unsigned)from_float<true>(dps[g + 1][e]) << 16);
            }
            store16_coherent(xrs, xoff + p * 256, __builtin_bit_cast(f32x4, make_uint4(w[0], w[1], w[2], w[3])));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            store16_coherent(xrs, xoff + e * 256, f32x4{dps[0][e], dps[1][e], dps[2][e], dps[3][e]});
        }
        if (t == 0 && P.dc0) *reinterpret_cast<f32x4*>(P.dc0 + fbh) = dcrec;
      }
    }
    if (t < 0) break;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(P.flags_d + (long)v * kFlagStride, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (fin) {
      const unsigned row = (unsigned)(t * B + fb) * 4 * H + u0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        *reinterpret_cast<f32x4*>(P.dP + row + (unsigned)(g * H)) = dps[g];
        if constexpr (BF16) {
          const unsigned lo = (unsigned)from_float<true>(dps[g][0]) | ((unsigned)from_float<true>(dps[g][1]) << 16);
          const unsigned hi = (unsigned)from_float<true>(dps[g][2]) | ((unsigned)from_float<true>(dps[g][3]) << 16);
          *reinterpret_cast<uint2*>(dPh + row + (unsigned)(g * H)) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<f32x4*>(dPh + row + (unsigned)(g * H)) = dps[g];
        }
      }
    }
  }
}

}  // namespace lstm
