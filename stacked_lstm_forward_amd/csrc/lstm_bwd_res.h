// Persistent kernel of one layer's recurrent chain in the backward pass, with
// R_l^T kept on chip (template definitions; instantiated in lstm_bwd.hip).
//
// The chain runs t = T-1 .. 0: dh_t = dY[t] + dh_rec, dc_t = dh_t o (1 -
// tanh(c_t)^2) + dc_rec, the gate derivatives dp_t, dc_rec <- dc_t f_t and
// dh_rec <- dp_t R_l (a product over K = 4H).  Streaming R_l from memory for
// that product every step reads 128 MiB per step at bf16 H = 4096; here, as in
// the forward's resident kernel, R_l^T stays in registers and LDS for the
// whole chain, and per step only dp_{t+1} is read.
//
// Work split (H = 4096: 256 workgroups, one per CU).  The K index of the
// product is ordered unit-major, k = 4 u + g for gate g of unit u (R_l^T and
// the exchanged dp use the same order, so the product is unchanged).
// Workgroup v = 4 ug + kq owns output units 64 ug .. 64 ug + 63 (four M-tiles
// of 16) and the K quarter kq: input units 1024 kq .. 1024 kq + 1023, all four
// gates.  So it reads a quarter of dp_{t+1} per step (256 KiB at B = 32, not
// all of it: one workgroup per 16 units reading all 1 MiB took 18.5 us a
// step, bound by those reads), and the four workgroups of a unit group add
// their partial sums: each leaves its sums in a per-step slot, then
// workgroup (ug, kq) adds the four partials of M-tile kq in a fixed order and
// finishes those 16 units (the elementwise part) for every sequence.
// Inside a workgroup, as in the forward: wave w is K-group w of 4 and owns
// chunks w, w + 4, ... of the quarter (16 chunks of 64) of every M-tile: 48
// fragment blocks in registers, one per chunk (16) in LDS; the column tiles
// run one after the other with one stream of dp loads five chunks ahead; the
// four waves' sums meet in LDS.
//
// Step protocol, two counters per workgroup (agent-scope stores, bounded
// waits with the error word):
//   flags_d[v] = s + 1 once iteration s's dp (of step T - 1 - s) is written;
//   flags_p[v] = s + 1 once iteration s's partial sums are written.
// Iteration s > 0 waits for flags_d >= s of the 64 workgroups that finish its
// K quarter's units (workgroups 64 kq .. 64 kq + 63), multiplies, publishes
// its partials and waits for flags_p >= s + 1 of its unit group's four
// workgroups.  The iteration after the last step computes dh0 = dp_0 R_l.
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
  int T, B, H, nch, wgs, grid, xcd_remap;
};

constexpr int kBwdResWaves = 4;
constexpr int kBwdResMW = 4;    // M-tiles (of 16 output units) per workgroup
constexpr int kBwdResNCI = 16;  // chunks of the K quarter per wave (H = 4096)
constexpr int kBwdResNRB = 48;  // ... of whose blocks in registers
constexpr int kBwdResPf = 7;    // per-step inputs of one (unit, sequence): dY, i, f, g, o, c_t, c_{t-1}

// LDS bytes: the LDS weight blocks, one tile's partial sums, the parked inputs.
__host__ __device__ constexpr int bwd_res_lds_bytes(int nw) {
  return kBwdResWaves * (kBwdResMW * kBwdResNCI - kBwdResNRB) * 2048 + kBwdResMW * kBwdResWaves * 64 * 16 +
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

template <bool BF16, int NW>
__global__ void __launch_bounds__(64 * kBwdResWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
lstm_bwd_res_kernel(const BwdResParams P) {
  typedef typename Dt<BF16>::T T;
  typedef ResOps<BF16> Ops;
  typedef typename Ops::V V;
  constexpr int SZ = Dt<BF16>::SZ;
  constexpr int KS = kBwdResWaves, MW = kBwdResMW, NCI = kBwdResNCI, NRB = kBwdResNRB;
  constexpr int NB = MW * NCI, NLB = NB - NRB, LPC = NLB / NCI, RPC = MW - LPC;
  static_assert(NLB % NCI == 0 && LPC >= 1, "LDS blocks spread evenly over the chunks");
  constexpr int FB = 2048 / SZ, EPH = 16 / SZ;
  constexpr int PD = 5;  // chunks of dp loads in flight per wave
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_ok;

  const int bid = blockIdx.x;
  const int v = P.xcd_remap ? ((bid & 7) * (P.grid >> 3) + (bid >> 3)) : bid;
  if (v >= P.wgs) return;
  const int ug = v >> 2, kq = v & 3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = P.H, B = P.B, T_ = P.T, nch = P.nch;
  uint4* As = reinterpret_cast<uint4*>(smem) + (long)kg * NLB * 128;
  f32x4* red = reinterpret_cast<f32x4*>(smem + KS * NLB * 2048);
  float* pf = reinterpret_cast<float*>(smem + KS * NLB * 2048 + MW * KS * 64 * 16);

  // ---- this wave's blocks of R_l^T: M-tile 4 ug + i, chunk 64 kq + kg + 4 ci
  // (M-tile i < RPC of chunk slot ci in register block ci RPC + i, the others
  // in LDS block ci LPC + i - RPC)
  struct WB {
    V h[2];
  };
  WB wreg[NRB];
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

  // ---- the (unit, sequence) pair this thread finishes in column tile j:
  // element kg of lane `lane`'s sums of M-tile kq, i.e. unit
  // 64 ug + 16 kq + 4 (lane >> 4) + kg, sequence 16 j + (lane & 15)
  const int unit = 64 * ug + 16 * kq + 4 * (lane >> 4) + kg;
  const int bl = lane & 15;
  float dcrec[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int b = 16 * j + bl;
    dcrec[j] = (b < B && P.dcT) ? P.dcT[(long)b * H + unit] : 0.f;
  }
  // dp of this pair's unit in load order: k = 4 unit + g is chunk unit / 16,
  // half (lane >> 4) >> 1, quad 2 ((lane >> 4) & 1) + kg / 2, element
  // 4 (kg & 1) + g: the four gates are four consecutive elements
  const unsigned xunit = (unsigned)(unit / 16) * FB + ((lane >> 4) >> 1) * (FB / 2) +
                         ((2 * ((lane >> 4) & 1) + kg / 2) * 16) * EPH + 4 * (kg & 1);

  T* DPx = reinterpret_cast<T*>(P.DPx);
  T* dPh = reinterpret_cast<T*>(P.dPh);
  // byte offset of this lane's 16 bytes in its wave's first dp block of a
  // column tile; tile, chunk slot and half are compile-time offsets
  const int hlane = (kg * FB + lane * EPH) * SZ;
  const long long pslot = bwd_res_part_floats(P.wgs, NW);

  for (int s = 0; s <= T_; ++s) {
    const int t = T_ - 1 - s;  // step whose dp this iteration computes (-1: dh0 only)
    if (t < 0 && !P.dh0) break;
    // per-step inputs of this thread's pairs, loaded before the waits
    float in[NW][kBwdResPf];
    if (t >= 0) {
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        // (32-bit offsets from the arguments' base addresses: the host keeps
        // T B 4H and every exchange and partial-sum offset below 2^31)
        const int b = min(16 * j + bl, B - 1);
        const unsigned bh = (unsigned)(t * B + b) * H + unit, g4 = (unsigned)(t * B + b) * 4 * H + unit;
        in[j][0] = P.dY[bh];
#pragma unroll
        for (int k = 0; k < 4; ++k) in[j][1 + k] = P.gates[g4 + (unsigned)(k * H)];
        in[j][5] = P.cs[bh];
        in[j][6] = t > 0 ? P.cs[bh - (unsigned)(B * H)] : (P.c0 ? P.c0[(unsigned)(b * H + unit)] : 0.f);
      }
    }
    if (s > 0) {
      // dp_{t+1} of this quarter's units: finished by the quarter's workgroups
      // (wgs / 4 of them: 64 kq .. 64 kq + 63 at H = 4096)
      if (kg == 0) {
        const int nq = P.wgs / 4;
        const bool ok = wait_counts_serial(P.flags_d + (long)nq * kq * kFlagStride, nq, s, nullptr, 0, 0, P.err,
                                           P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s_ok) return;
    }
    if (t >= 0) {
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int k = 0; k < kBwdResPf; ++k) pf[(j * kBwdResPf + k) * 256 + tid] = in[j][k];
    }

    float dhr[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) dhr[j] = 0.f;
    if (s > 0) {
      // ---- this workgroup's partial dh_rec = dp_{t+1} R_l over its K quarter
      const T* src = DPx + (long)(t + 1) * P.xslot + (long)(NCI * KS * kq) * FB;
      const __amdgpu_buffer_rsrc_t drs = raw_buffer(src, (int)((long)NW * nch * FB * SZ));
      const __amdgpu_buffer_rsrc_t prs = raw_buffer(P.part + (long)s * pslot + (long)v * (NW * MW * 256), NW * MW * 1024);
      Frag rb[PD];
      Frag al[LPC];
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
#pragma unroll
          for (int ii = 0; ii < MW; ++ii) {
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
#pragma unroll
        for (int i = 0; i < MW; ++i) red[(i * KS + kg) * 64 + lane] = acc[i];
        __syncthreads();
        f32x4 p = red[(kg * KS) * 64 + lane];
#pragma unroll
        for (int r = 1; r < KS; ++r) p += red[(kg * KS + r) * 64 + lane];
        store16_coherent(prs, ((j * MW + kg) * 64 + lane) * 16, p);
        if (j + 1 < NW) __syncthreads();  // the next tile reuses the area
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(P.flags_p + (long)v * kFlagStride, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // ---- the unit group's four partial sums of M-tile kq, in a fixed order
      if (kg == 0) {
        const bool ok = wait_counts_serial(P.flags_p + (long)(4 * ug) * kFlagStride, 4, s + 1, nullptr, 0, 0, P.err,
                                           P.timeout_ticks);
        if (lane == 0) s_ok = ok ? 1 : 0;
      }
      __syncthreads();
      if (!s_ok) return;
      const float* pin = P.part + (long)s * pslot + (long)(4 * ug) * (NW * MW * 256);
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) dhr[j] += pin[(long)w * (NW * MW * 256) + ((j * MW + kq) * 64 + lane) * 4 + kg];
    }

    // ---- the elementwise part of this thread's pairs (the exchange copy of
    // dp first: the step counter waits only for it; dP and its dtype copy,
    // read by later kernels, are stored after the counter)
    float dps[NW][4];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int b = 16 * j + bl;
      if (b >= B) continue;
      const unsigned bh = (unsigned)(b * H + unit);
      if (t < 0) {
        P.dh0[bh] = dhr[j];
        continue;
      }
      const float* x = pf + j * kBwdResPf * 256 + tid;
      const float ig = x[1 * 256], fg = x[2 * 256], gg = x[3 * 256], og = x[4 * 256];
      const float ct = x[5 * 256], cp = x[6 * 256];
      const float dh = x[0] + (s > 0 ? dhr[j] : (P.dhT ? P.dhT[bh] : 0.f));
      const float tc = tanh_f(ct);
      const float dc = dh * og * (1.f - tc * tc) + dcrec[j];
      const float d[4] = {dc * gg * ig * (1.f - ig), dc * cp * fg * (1.f - fg), dc * ig * (1.f - gg * gg),
                          dh * tc * og * (1.f - og)};
      dcrec[j] = dc * fg;
      T hv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dps[j][k] = d[k];
        hv[k] = from_float<BF16>(d[k]);
      }
      // the four gates' dp as one 8-byte word of the exchange
      const unsigned xo = (unsigned)t * (unsigned)P.xslot + (unsigned)((b >> 4) * nch) * FB + xunit + (b & 15) * EPH;
      if constexpr (BF16) {
        const unsigned long long wv = (unsigned long long)hv[0] | ((unsigned long long)hv[1] << 16) |
                                      ((unsigned long long)hv[2] << 32) | ((unsigned long long)hv[3] << 48);
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(DPx + xo), wv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) store_coherent<BF16>(DPx + xo + k, hv[k]);
      }
      if (t == 0 && P.dc0) P.dc0[bh] = dcrec[j];
    }
    if (t < 0) break;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(P.flags_d + (long)v * kFlagStride, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int b = 16 * j + bl;
      if (b >= B) continue;
      const unsigned row = (unsigned)(t * B + b) * 4 * H + unit;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        P.dP[row + (unsigned)(k * H)] = dps[j][k];
        dPh[row + (unsigned)(k * H)] = from_float<BF16>(dps[j][k]);
      }
    }
  }
}

}  // namespace lstm
