// Persistent kernel of one layer's recurrent chain in the backward pass, with
// R_l^T kept on chip (template definitions; instantiated in lstm_bwd.hip).
//
// The chain runs t = T-1 .. 0: dh_t = dY[t] + dh_rec, dc_t = dh_t o (1 -
// tanh(c_t)^2) + dc_rec, the gate derivatives dp_t, dc_rec <- dc_t f_t and
// dh_rec <- dp_t R_l (a product over K = 4H).  Streaming R_l from memory for
// that product every step reads 128 MiB per step at bf16 H = 4096; here, as in
// the forward's resident kernel, each workgroup keeps its rows of R_l^T (its
// 16 hidden units, all 4H columns) in registers and LDS for the whole chain,
// and per step reads only dp_{t+1}, which every workgroup publishes in the
// order its readers load it.
//
// Work split: workgroup v owns units 16 v .. 16 v + 15 (one M-tile); wave w is
// K-group w of 4 and owns chunks c = w, w + 4, ... of the 4H columns (NCI
// chunks): one fragment block per chunk, in registers except every fourth
// chunk's (ci % 4 == 3), which sits in LDS.  The NW batch column tiles are
// multiplied one after the other with one stream of dp loads running PD chunks
// ahead; each tile's four partial sums meet in LDS and the 256 threads of the
// workgroup finish one (unit, sequence) pair each.  The per-step inputs of
// those pairs (dY, the saved gates and cell states) are loaded before the wait
// and parked in LDS, so the products keep their registers.
//
// Step protocol: one counter per workgroup, s + 1 once iteration s (dp of step
// T - 1 - s) is in memory; iteration s > 0 waits for every counter >= s.  The
// iteration after the last step computes dh0 = dp_0 R_l.
#pragma once

#include "lstm_rec_res.h"

namespace lstm {

struct BwdResParams {
  const uint4* RTf;     // R_l^T in load order: block (unit tile, chunk) of 128 x 16 bytes
  void* DPx;            // dp_t in load order, [T] slots of xslot elements (dtype)
  long long xslot;
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
  int* flags;           // per-workgroup counters, kFlagStride apart (zero on entry)
  int* err;             // device error word
  long long timeout_ticks;
  int T, B, H, nch, wgs, grid, xcd_remap;
};

constexpr int kBwdResWaves = 4;
constexpr int kBwdResPf = 7;  // per-step inputs of one (unit, sequence): dY, i, f, g, o, c_t, c_{t-1}

// LDS bytes: the LDS weight blocks, one tile's partial sums, the parked inputs.
__host__ __device__ constexpr int bwd_res_lds_bytes(int nci, int nrb, int nw) {
  return kBwdResWaves * (nci - nrb) * 2048 + kBwdResWaves * 64 * 16 + nw * kBwdResPf * 256 * 4;
}

template <bool BF16, int NW, int NCI, int NRB>
__global__ void __launch_bounds__(64 * kBwdResWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
lstm_bwd_res_kernel(const BwdResParams P) {
  typedef typename Dt<BF16>::T T;
  typedef ResOps<BF16> Ops;
  typedef typename Ops::V V;
  constexpr int KC = Dt<BF16>::KC;
  constexpr int KS = kBwdResWaves;
  constexpr int NLB = NCI - NRB;  // LDS blocks per wave: chunks ci % 4 == 3
  static_assert(NLB * 4 == NCI, "every fourth chunk's block in LDS");
  constexpr int PD = 4;  // chunks of dp loads in flight per wave
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_ok;

  const int bid = blockIdx.x;
  const int v = P.xcd_remap ? ((bid & 7) * (P.grid >> 3) + (bid >> 3)) : bid;
  if (v >= P.wgs) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = P.H, B = P.B, T_ = P.T, nch = P.nch;
  uint4* As = reinterpret_cast<uint4*>(smem) + (long)kg * NLB * 128;
  f32x4* red = reinterpret_cast<f32x4*>(smem + KS * NLB * 2048);
  float* pf = reinterpret_cast<float*>(smem + KS * NLB * 2048 + KS * 64 * 16);

  // ---- this wave's blocks of R_l^T: chunk slot ci is chunk kg + KS ci
  struct WB {
    V h[2];
  };
  WB wreg[NRB];
#pragma unroll
  for (int ci = 0; ci < NCI; ++ci) {
    const uint4* blk = P.RTf + ((long)v * nch + kg + KS * ci) * 128;
    Frag f;
    f.v[0] = blk[lane];
    f.v[1] = blk[64 + lane];
    if (ci % 4 == 3) {
      lds_put(As + (ci / 4) * 128, lane, f);
    } else {
      const int r = (ci / 4) * 3 + ci % 4;
      WB w{{Ops::cast(f.v[0]), Ops::cast(f.v[1])}};
      if (r < kResAgprBlocks) {
        asm volatile("" : "+a"(w.h[0]));
        asm volatile("" : "+a"(w.h[1]));
      }
      wreg[r] = w;
    }
  }

  // ---- the (unit, sequence) pair this thread finishes in column tile j:
  // unit 16 v + (tid >> 4), sequence 16 j + (tid & 15).  In a wave's
  // accumulator that element is lane 16 (u >> 2) + (tid & 15), row u & 3.
  const int u = tid >> 4, unit = 16 * v + u;
  const int alane = 16 * (u >> 2) + (tid & 15), arow = u & 3;
  float dcrec[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int b = 16 * j + (tid & 15);
    dcrec[j] = (b < B && P.dcT) ? P.dcT[(long)b * H + unit] : 0.f;
  }

  T* DPx = reinterpret_cast<T*>(P.DPx);
  T* dPh = reinterpret_cast<T*>(P.dPh);
  constexpr int FB = 2048 / Dt<BF16>::SZ;  // elements of one 2 KiB block
  constexpr int EPH = 16 / Dt<BF16>::SZ;

  for (int s = 0; s <= T_; ++s) {
    const int t = T_ - 1 - s;  // step whose dp this iteration computes (-1: dh0 only)
    if (t < 0 && !P.dh0) break;
    // per-step inputs of this thread's pairs, loaded before the wait
    float in[NW][kBwdResPf];
    if (t >= 0) {
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        // (32-bit offsets from the arguments' base addresses: the host keeps
        // T B 4H and every exchange offset below 2^31)
        const int b = min(16 * j + (tid & 15), B - 1);
        const unsigned bh = (unsigned)(t * B + b) * H + unit, g4 = (unsigned)(t * B + b) * 4 * H + unit;
        in[j][0] = P.dY[bh];
#pragma unroll
        for (int k = 0; k < 4; ++k) in[j][1 + k] = P.gates[g4 + (unsigned)(k * H)];
        in[j][5] = P.cs[bh];
        in[j][6] = t > 0 ? P.cs[bh - (unsigned)(B * H)] : (P.c0 ? P.c0[(unsigned)(b * H + unit)] : 0.f);
      }
    }
    if (s > 0) {
      if (kg == 0) {
        const bool ok = wait_counts_serial(P.flags, P.wgs, s, nullptr, 0, 0, P.err, P.timeout_ticks);
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

    // ---- dh_rec = dp_{t+1} R_l for every column tile (none at s = 0: dhT)
    const T* src = DPx + (long)(t + 1) * P.xslot;
    Frag rb[PD];
    Frag al;
    auto issue = [&](Frag& dst, int g) {
      const int jj = g / NCI, ci = g % NCI;
      const uint4* blk = reinterpret_cast<const uint4*>(src + ((long)jj * nch + kg + KS * ci) * FB);
      dst.v[0] = blk[lane];
      dst.v[1] = blk[64 + lane];
    };
    if (s > 0) {
#pragma unroll
      for (int g = 0; g < PD; ++g) issue(rb[g], g);
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s > 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ci = 0; ci < NCI; ++ci) {
          const int g = j * NCI + ci, sl = g % PD;
          if (ci % 4 == 0) al = lds_get(As + (ci / 4) * 128, lane);  // the block of chunk ci + 3
          const V x0 = Ops::cast(rb[sl].v[0]), x1 = Ops::cast(rb[sl].v[1]);
          V a0, a1;
          if (ci % 4 == 3) {
            a0 = Ops::cast(al.v[0]);
            a1 = Ops::cast(al.v[1]);
          } else {
            const int r = (ci / 4) * 3 + ci % 4;
            a0 = wreg[r].h[0];
            a1 = wreg[r].h[1];
          }
          Ops::chunk(acc, a0, a1, x0, x1);
          __builtin_amdgcn_sched_barrier(0);
          if (g + PD < NW * NCI) issue(rb[sl], g + PD);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- the four K-groups' partial sums, added in a fixed order
      red[kg * 64 + lane] = acc;
      __syncthreads();
      const int b = 16 * j + (tid & 15);
      const bool live = b < B && unit < H;
      float dhr = 0.f;
      if (s > 0) {
#pragma unroll
        for (int w = 0; w < KS; ++w) dhr += red[w * 64 + alane][arow];
      }
      if (live) {
        const unsigned bh = (unsigned)(b * H + unit);
        if (t < 0) {
          if (P.dh0) P.dh0[bh] = dhr;
        } else {
          const float* x = pf + j * kBwdResPf * 256 + tid;
          const float ig = x[1 * 256], fg = x[2 * 256], gg = x[3 * 256], og = x[4 * 256];
          const float ct = x[5 * 256], cp = x[6 * 256];
          const float dh = x[0] + (s > 0 ? dhr : (P.dhT ? P.dhT[bh] : 0.f));
          const float tc = tanhf(ct);
          const float dc = dh * og * (1.f - tc * tc) + dcrec[j];
          const float d[4] = {dc * gg * ig * (1.f - ig), dc * cp * fg * (1.f - fg), dc * ig * (1.f - gg * gg),
                              dh * tc * og * (1.f - og)};
          dcrec[j] = dc * fg;
          const unsigned row = (unsigned)(t * B + b) * 4 * H + unit;
          // load order of dp_t: row b, column k H + unit (H is whole chunks,
          // so the place inside a chunk is the same for the four gates)
          const int kc = unit % KC, hh = kc / (KC / 2), qq = (kc % (KC / 2)) / EPH, e = kc % EPH;
          const unsigned xo = (unsigned)t * (unsigned)P.xslot +
                              ((unsigned)((b >> 4) * nch + unit / KC) * 2 + hh) * (FB / 2) + (qq * 16 + (b & 15)) * EPH + e;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const T hv = from_float<BF16>(d[k]);
            P.dP[row + (unsigned)(k * H)] = d[k];
            dPh[row + (unsigned)(k * H)] = hv;
            store_coherent<BF16>(DPx + xo + (unsigned)(k * (H / KC) * FB), hv);
          }
          if (t == 0 && P.dc0) P.dc0[bh] = dcrec[j];
        }
      }
      // the next tile's partial sums reuse the area
      if (j + 1 < NW) __syncthreads();
    }
    if (t < 0) break;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(P.flags + (long)v * kFlagStride, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace lstm
