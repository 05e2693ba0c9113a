// Measured-peak microbenchmarks for gfx950 (see include/lstm_peaks.h).
//
// Each kernel isolates one limit the stacked-LSTM forward kernels run into:
//   * the matrix cores (register operands, 8 independent accumulators per wave,
//     so issue and not dependence sets the rate);
//   * HBM (a grid-stride read, and a copy);
//   * LDS (conflict-free 16-byte reads, a wave reading 1 KiB contiguous);
//   * the step exchange between workgroups: write a slice of the step's slot,
//     wait for the stores, publish a step counter, poll every counter, read the
//     whole slot -- the protocol of the persistent recurrent kernels -- either
//     with device-coherent operations (works across the 8 XCDs, whose L2s are
//     not coherent with each other) or with L2-level operations among
//     workgroups that share one XCD.
// Results feed only the reported fractions; nothing on the forward path calls
// these kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lstm_peaks.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// ---------------------------------------------------------------- matrix cores
// One round: 8 independent MFMAs, accumulating in place.  The accumulators
// are tied to the instruction's destination by the asm constraints, so the
// loop carries no copies between rounds (plain builtins let the register
// allocator rotate the accumulators through moves in a loop this small).
template <int KIND>
__global__ void __launch_bounds__(kThreads) peak_mfma_kernel(float* out, int iters, int sink) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
  if (KIND == 0 || KIND == 1) {
    // bf16 operand bits near 1.0 (8 per lane, packed in 4 words)
    const u32x4 ua = {0x3f803f80u + lane, 0x3f813f7fu, 0x3f7f3f82u, 0x3f803f80u ^ lane};
    const u32x4 ub = {0x3f803f81u, 0x3f7e3f80u + lane, 0x3f803f80u, 0x3f823f80u};
    if (KIND == 0) {
      f32x4 acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(ua), "v"(ub));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][3];
    } else {
      f32x16 acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
      for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(ua), "v"(ub));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][15];
    }
  } else {
    const float a = 1.0f + 1e-3f * lane, b = 0.5f - 1e-3f * lane;
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(acc[k]) : "v"(a), "v"(b));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][3];
  }
  // the compiler does not see the asm MFMAs' latency: let the last ones
  // retire before the accumulators are read back (the sum is only a sink)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
  if (sink) out[0] = s;  // a run-time flag keeps every product live
}

// ---------------------------------------------------------------- HBM
__global__ void __launch_bounds__(kThreads) peak_read_kernel(const uint4* p, long n, uint4* out, int sink) {
  const long stride = (long)gridDim.x * kThreads;
  long i = (long)blockIdx.x * kThreads + threadIdx.x;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc.x ^= a.x ^ b.x ^ c.x ^ d.x;
    acc.y ^= a.y ^ b.y ^ c.y ^ d.y;
    acc.z ^= a.z ^ b.z ^ c.z ^ d.z;
    acc.w ^= a.w ^ b.w ^ c.w ^ d.w;
  }
  for (; i < n; i += stride) {
    const uint4 a = p[i];
    acc.x ^= a.x, acc.y ^= a.y, acc.z ^= a.z, acc.w ^= a.w;
  }
  if (sink) out[0] = acc;
}

__global__ void __launch_bounds__(kThreads) peak_copy_kernel(const uint4* src, uint4* dst, long n) {
  const long stride = (long)gridDim.x * kThreads;
  long i = (long)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a, dst[i + stride] = b, dst[i + 2 * stride] = c, dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// ---------------------------------------------------------------- LDS
constexpr int kLdsUnits = 4096;  // 64 KiB of 16-byte units per workgroup

__global__ void __launch_bounds__(kThreads) peak_lds_kernel(uint4* out, int iters, int sink) {
  __shared__ uint4 buf[kLdsUnits];
  for (int i = threadIdx.x; i < kLdsUnits; i += kThreads) buf[i] = make_uint4(i, 3 * i, 5 * i, 7 * i);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // each read: 64 consecutive 16-byte units (1 KiB, no bank conflict)
      const uint4 v = buf[((it * 8 + k) * 64 + wave * 1024 + lane) & (kLdsUnits - 1)];
      acc.x ^= v.x, acc.y ^= v.y, acc.z ^= v.z, acc.w ^= v.w;
    }
    asm volatile("" ::: "memory");  // the next round reads LDS again
  }
  if (sink) out[0] = acc;
}

// ---------------------------------------------------------------- step exchange
constexpr int kCounterStride = 32;  // ints: one 128-byte line per counter
constexpr int kMaxActive = 256;

struct StepArgs {
  int* err;
  int* cnt;
  char* slots;
  int* xcc;
  long long timeout;
  int stride, scope, slice, steps, nact, sink;
};

__device__ __forceinline__ int xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

__global__ void __launch_bounds__(kThreads) peak_step_clear(int* p, long n) {
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads) p[i] = 0;
}

__global__ void __launch_bounds__(kThreads) peak_step_kernel(const StepArgs a) {
  const int bid = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (a.xcc && tid == 0) a.xcc[bid] = xcc_id();
  if (bid % a.stride) return;
  const int me = bid / a.stride;
  __shared__ int s_ok;
  const long slot_bytes = (long)a.nact * a.slice;
  const int nu = a.slice / 16;                  // 16-byte units of my slice
  const long nslot = slot_bytes / 16;           // ... of the whole slot
  // L2-level polls (sc0: the L1 is bypassed, the XCD's L2 is not)
  const __amdgpu_buffer_rsrc_t crs = rsrc_of(a.cnt, kMaxActive * kCounterStride * 4);
  uint32_t acc = 0;
  for (int t = 0; t < a.steps; ++t) {
    uint4* slot = reinterpret_cast<uint4*>(a.slots + (long)t * slot_bytes);
    uint4* mine = slot + (long)me * nu;
    for (int i = tid; i < nu; i += kThreads) {
      const uint32_t w[4] = {(uint32_t)t, (uint32_t)me, (uint32_t)i, 1u};
      uint32_t* d = reinterpret_cast<uint32_t*>(mine + i);
      if (a.scope == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) __hip_atomic_store(d + e, w[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        mine[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      if (a.scope == 0)
        __hip_atomic_store(a.cnt + (long)me * kCounterStride, t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_store(a.cnt + (long)me * kCounterStride, t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (tid < 64) {
      const long long start = wall_clock64();
      bool ok = true;
      while (true) {
        int good = 1;
        const int e0 = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = min(lane + 64 * k, a.nact - 1);
          const int c = a.scope == 0
                            ? __hip_atomic_load(a.cnt + (long)i * kCounterStride, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : (int)__builtin_amdgcn_raw_buffer_load_b32(crs, i * kCounterStride * 4, 0, 1);
          good &= (c >= t + 1) ? 1 : 0;
        }
        if (__all(good)) break;
        if (e0 != 0) {
          ok = false;
          break;
        }
        if (wall_clock64() - start > a.timeout) {
          if (lane == 0) __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = false;
          break;
        }
      }
      if (lane == 0) s_ok = ok ? 1 : 0;
    }
    __syncthreads();
    if (!s_ok) return;
    // every workgroup reads the whole slot with ordinary loads (never read
    // before in this launch, so no cache holds an older copy)
    for (long i = tid; i < nslot; i += kThreads) {
      const uint4 v = slot[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (a.sink) a.err[1 + (bid & 31)] = (int)acc;
}

int g_wallclock_khz = 0;

int launch_error(hipError_t e) { return e == hipSuccess ? 0 : 2; }

}  // namespace

extern "C" {

int lstm_peak_mfma(int kind, int grid, int iters, float* out, int sink, hipStream_t stream, hipEvent_t ev0,
                   hipEvent_t ev1) {
  if (kind < 0 || kind > 2 || grid < 1 || iters < 1 || !out) return 1;
  if (hipEventRecord(ev0, stream) != hipSuccess) return 2;
  if (kind == 0)
    hipLaunchKernelGGL(peak_mfma_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, out, iters, sink);
  else if (kind == 1)
    hipLaunchKernelGGL(peak_mfma_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, out, iters, sink);
  else
    hipLaunchKernelGGL(peak_mfma_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, out, iters, sink);
  if (hipGetLastError() != hipSuccess) return 2;
  return launch_error(hipEventRecord(ev1, stream));
}

int lstm_peak_memory(int mode, void* buf, size_t bytes, int grid, void* out, int sink, hipStream_t stream,
                     hipEvent_t ev0, hipEvent_t ev1) {
  if ((mode != 0 && mode != 1) || !buf || !out || grid < 1 || bytes < 32 || bytes % 32 != 0) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return 1;
  if (hipEventRecord(ev0, stream) != hipSuccess) return 2;
  if (mode == 0) {
    hipLaunchKernelGGL(peak_read_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<const uint4*>(buf),
                       (long)(bytes / 16), static_cast<uint4*>(out), sink);
  } else {
    const long half = (long)(bytes / 32);
    const uint4* src = static_cast<const uint4*>(buf);
    hipLaunchKernelGGL(peak_copy_kernel, dim3(grid), dim3(kThreads), 0, stream, src,
                       static_cast<uint4*>(buf) + half, half);
  }
  if (hipGetLastError() != hipSuccess) return 2;
  return launch_error(hipEventRecord(ev1, stream));
}

int lstm_peak_lds(int grid, int iters, void* out, int sink, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (grid < 1 || iters < 1 || !out) return 1;
  if (hipEventRecord(ev0, stream) != hipSuccess) return 2;
  hipLaunchKernelGGL(peak_lds_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<uint4*>(out), iters, sink);
  if (hipGetLastError() != hipSuccess) return 2;
  return launch_error(hipEventRecord(ev1, stream));
}

size_t lstm_peak_step_ws_bytes(int grid, int stride, int slice_bytes, int steps) {
  if (grid < 1 || stride < 1 || slice_bytes < 0 || slice_bytes % 16 != 0 || steps < 1) return 0;
  const long nact = (grid + stride - 1) / stride;
  if (nact > kMaxActive) return 0;
  return 256 + (size_t)kMaxActive * kCounterStride * 4 + (size_t)steps * nact * slice_bytes;
}

int lstm_peak_step(int grid, int stride, int scope, int slice_bytes, int steps, int64_t timeout_us, void* ws,
                   int* xcc, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const size_t need = lstm_peak_step_ws_bytes(grid, stride, slice_bytes, steps);
  if (!need || !ws || (scope != 0 && scope != 1) || timeout_us < 1) return 1;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return 1;
  if (!g_wallclock_khz) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 2;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 2;
    g_wallclock_khz = khz > 0 ? khz : 100000;
  }
  StepArgs a;
  char* base = static_cast<char*>(ws);
  a.err = reinterpret_cast<int*>(base);
  a.cnt = reinterpret_cast<int*>(base + 256);
  a.slots = base + 256 + (size_t)kMaxActive * kCounterStride * 4;
  a.xcc = xcc;
  a.timeout = (long long)timeout_us * g_wallclock_khz / 1000;
  a.stride = stride, a.scope = scope, a.slice = slice_bytes, a.steps = steps;
  a.nact = (grid + stride - 1) / stride;
  a.sink = 0;
  const long nclear = (long)((256 + (size_t)kMaxActive * kCounterStride * 4) / 4);
  hipLaunchKernelGGL(peak_step_clear, dim3(64), dim3(kThreads), 0, stream, a.err, nclear);
  if (hipGetLastError() != hipSuccess) return 2;
  // every workgroup of the exchange must be resident at once: a cooperative launch
  int per_cu = 0, cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 2;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&peak_step_kernel),
                                                   kThreads, 0) != hipSuccess)
    return 2;
  if ((long)per_cu * cus < grid) return 1;
  if (hipEventRecord(ev0, stream) != hipSuccess) return 2;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&peak_step_kernel), dim3(grid), dim3(kThreads), args,
                                 0, stream) != hipSuccess)
    return 2;
  return launch_error(hipEventRecord(ev1, stream));
}

}  // extern "C"
