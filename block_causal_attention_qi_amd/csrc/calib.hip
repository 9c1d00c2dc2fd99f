// Calibration microbenchmarks (include/qi_calib.h): register-only MFMA
// throughput, device copy bandwidth, and the LDS cost of the GEMM's K-loop
// instruction mixes on the running MI355X.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qi_calib.h"
#include "common.hpp"

namespace {

template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float *out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0];
  } else {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0];
  }
  if (s == 1.2345e30f) out[threadIdx.x] = s;  // keeps the loop alive; never true
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ a, u32x4 *__restrict__ b, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) b[i] = a[i];
}

// Read-only stream: each thread sums 8 independent 16-byte loads per
// iteration of a grid-stride loop; one word per thread is written to out
// (gridDim.x * 256 words) only if the sum is a value random data never gives.
__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ a, int64_t n, unsigned *out) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x, nt = (int64_t)gridDim.x * 256;
  unsigned s = 0;
  for (int64_t base = tid; base < n; base += 8 * nt) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = base + u * nt;
      v[u] = i < n ? a[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (s == 0x9E3779B9u) out[tid] = s;
}

// One 512-thread workgroup per CU (8 waves, two per SIMD), 128 KB of LDS;
// each iteration every wave issues the MODE's mix (qi_calib.h), every fourth
// iteration ends with a barrier.  Wave 0 of each workgroup adds its shader
// cycles to clk[0] and 1 to clk[1].  Every LDS index stays below 8192 slots;
// copy sources stay below 4096 slots of src.
template <int MODE>
__global__ __launch_bounds__(512, 1) void lds_mix_kernel(float *out, int iters, unsigned long long *clk,
                                                         const u32x4 *src) {
  __shared__ u32x4 s[8192];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 8192; i += 512) s[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  // the GEMM's patterns: staging store slot of row tid/8, chunk tid%8; fragment
  // read of row (wave&1)*128 + lane%32 at a swizzled chunk
  const int lrow = tid >> 3, lc = tid & 7;
  const int wslot = lrow * 8 + (lc ^ ((lrow >> 1) & 7));
  const int fr = lane & 31, half = lane >> 5, sw = (fr >> 1) & 7;
  const int rowA = (wave & 1) * 128 + fr;
  u32x4 acc4 = {0, 0, 0, 0};
  const u32x4 wv = {(uint32_t)tid, 7u, 9u, 11u};
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(lane * 0.01f);
    b[i] = (__bf16)0.5f;
  }
  constexpr bool kMfma = MODE >= 2, kReads = MODE == 0 || MODE >= 3;
  constexpr int kNr = MODE == 0 ? 8 : 6;
  for (int it = 0; it < iters; ++it) {
    const int ch = ((it & 3) * 2 + half) ^ sw;
    const int buf = (it & 1) * 4096;
    if constexpr (kReads) {
#pragma unroll
      for (int r = 0; r < kNr; ++r) acc4 += s[buf + ((rowA + 32 * r) * 8) % 4096 + ch];
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int r = 0; r < 8; ++r) s[buf + (wslot + 512 * r) % 4096] = wv + (uint32_t)(r + it);
    }
    if constexpr (MODE == 3) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        s[(4096 - buf) + (wslot + 512 * (r + 2 * (it & 3))) % 4096] = wv + (uint32_t)(r + it);
    }
    if constexpr (MODE == 4) {
#if __HIP_DEVICE_COMPILE__
#pragma unroll
      for (int r = 0; r < 2; ++r)
        __builtin_amdgcn_global_load_lds((const void *)(src + ((wave * 64 + lane + 512 * r) & 4095)),
                                         (__attribute__((address_space(3))) void *)&s[(4096 - buf) +
                                             ((wave * 64 + 512 * (r + 2 * (it & 3))) % 4096)],
                                         16, 0, 0);
#endif
    }
    if constexpr (kMfma) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    if constexpr (MODE >= 3) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i < 2) __builtin_amdgcn_sched_group_barrier(MODE == 3 ? 0x200 : 0x020, 1, 0);
      }
    }
    if ((it & 3) == 3) __syncthreads();
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  float sum = (float)acc4[0] + (float)acc4[1] + (float)s[(tid * 3 + iters) & 8191][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += acc[j][0];
  // keeps the work alive: the compiler cannot decide this (practically never true)
  if (__float_as_uint(sum) == (uint32_t)iters * 2654435761u) out[tid] = sum;
  if (tid == 0) {
    atomicAdd(&clk[0], (unsigned long long)(t1 - t0));
    atomicAdd(&clk[1], 1ull);
  }
}

// One workgroup per CU with W waves per SIMD (waves w and w + 4 share a SIMD
// when W = 2).  ROLE of a wave: 1 = 8 MFMAs per iteration, 2 = 32 VALU
// instructions (KIND 1: v_fma_f32, 2: v_exp_f32) on 8 independent chains,
// 3 = both, four VALU instructions after each MFMA.  SPLIT: waves 0-3 take
// role 1, waves 4-7 role 2.  Timed from the host with events (wall clock).
template <int W, int KIND, int ROLE, int SPLIT>
__global__ __launch_bounds__(256 * W, 1) void valu_mix_kernel(float *out, int iters) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int role = SPLIT ? (wave < 4 ? 1 : 2) : ROLE;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = -1.f - 0.01f * (float)(lane + j);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(lane * 0.01f);
    b[i] = (__bf16)0.5f;
  }
  auto valu = [&](int j) {
    if constexpr (KIND == 1) v[j] = __builtin_fmaf(v[j], 0.999f, 0.001f);
    else v[j] = __builtin_amdgcn_exp2f(v[j]);
  };
  if (role == 1) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
  } else if (role == 2) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 32; ++r) valu(r & 7);
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) valu((4 * m + r) & 7);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // then four VALU / transcendental
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += v[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) sum += acc[j][0];
  // keeps the work alive: the compiler cannot decide this (practically never true)
  if (__float_as_uint(sum) == (uint32_t)iters * 2654435761u) out[tid] = sum;
}

}  // namespace

extern "C" {

qi_status qi_calib_mfma_tflops(int32_t shape, int32_t iters, double *tflops) {
  if (!tflops) return QI_ERR_NULL;
  if ((shape != 0 && shape != 1) || iters < 1 || iters > 10000000) return QI_ERR_RANGE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QI_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return QI_ERR_HIP;
  float *out = nullptr;
  hipStream_t st;
  hipEvent_t e0, e1;
  if (hipStreamCreate(&st) != hipSuccess) return QI_ERR_HIP;
  qi_status rc = QI_OK;
  const int blocks = cus * 8;
  if (hipMalloc(&out, 256 * sizeof(float)) != hipSuccess) rc = QI_ERR_HIP;
  if (rc == QI_OK && (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)) rc = QI_ERR_HIP;
  if (rc == QI_OK) {
    auto run = [&]() {
      if (shape == 0)
        hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, st, out, iters);
      else
        hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, st, out, iters);
    };
    run();  // warm-up
    (void)hipEventRecord(e0, st);
    run();
    (void)hipEventRecord(e1, st);
    float ms = 0.f;
    if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess ||
        hipGetLastError() != hipSuccess)
      rc = QI_ERR_HIP;
    const double per = shape == 0 ? 32.0 * 32 * 16 * 2 : 16.0 * 16 * 32 * 2;
    *tflops = rc == QI_OK ? (double)blocks * 4 * iters * 8 * per / (ms * 1e-3) / 1e12 : 0.0;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  if (out) (void)hipFree(out);
  (void)hipStreamDestroy(st);
  return rc;
}

// Best of `reps` timed launches of one stream kernel for each grid size in
// grids (workgroups of 256 threads); returns the best time in ms.
}  // extern "C"
template <class Launch>
static qi_status best_ms(int32_t reps, const int *grids, int ngrids, Launch &&launch, float *best_out) {
  hipStream_t st;
  hipEvent_t e0, e1;
  if (hipStreamCreate(&st) != hipSuccess) return QI_ERR_HIP;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    (void)hipStreamDestroy(st);
    return QI_ERR_HIP;
  }
  float best = 1e30f;
  qi_status rc = QI_OK;
  for (int gi = 0; gi < ngrids && rc == QI_OK; ++gi)
    for (int r = 0; r <= reps && rc == QI_OK; ++r) {
      (void)hipEventRecord(e0, st);
      launch(grids[gi], st);
      (void)hipEventRecord(e1, st);
      float ms = 0.f;
      if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) rc = QI_ERR_HIP;
      if (r > 0 && ms < best) best = ms;  // r == 0 is a warm-up
    }
  *best_out = best;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipStreamDestroy(st);
  return rc;
}

// grid sizes tried by the stream measurements: 4 to 16 workgroups per CU
static const int kStreamGrids[] = {1024, 2048, 4096};

extern "C" {

qi_status qi_calib_copy_gbs(const void *src, void *dst, int64_t bytes, int32_t reps, double *gbs) {
  if (!src || !dst || !gbs) return QI_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || reps < 1 || reps > 1000) return QI_ERR_RANGE;
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return QI_ERR_ALIGN;
  const int64_t n = bytes / 16;
  float best = 0.f;
  const qi_status rc = best_ms(reps, kStreamGrids, 3, [&](int grid, hipStream_t st) {
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, st, (const u32x4 *)src, (u32x4 *)dst, n);
  }, &best);
  *gbs = rc == QI_OK ? 2.0 * (double)bytes / (best * 1e-3) / 1e9 : 0.0;
  return rc;
}

qi_status qi_calib_read_gbs(const void *src, int64_t bytes, void *scratch, int32_t reps, double *gbs) {
  if (!src || !scratch || !gbs) return QI_ERR_NULL;
  if (bytes < 16 || bytes % 16 != 0 || reps < 1 || reps > 1000) return QI_ERR_RANGE;
  if ((uintptr_t)src & 15) return QI_ERR_ALIGN;
  const int64_t n = bytes / 16;
  float best = 0.f;
  const qi_status rc = best_ms(reps, kStreamGrids, 3, [&](int grid, hipStream_t st) {
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, st, (const u32x4 *)src, n, (unsigned *)scratch);
  }, &best);
  *gbs = rc == QI_OK ? (double)bytes / (best * 1e-3) / 1e9 : 0.0;
  return rc;
}

qi_status qi_calib_lds_cycles(int32_t mode, int32_t iters, double *cycles) {
  if (!cycles) return QI_ERR_NULL;
  if (mode < 0 || mode > 4 || iters < 4 || iters > 10000000) return QI_ERR_RANGE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QI_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return QI_ERR_HIP;
  float *out = nullptr;
  unsigned long long *clk = nullptr;
  u32x4 *src = nullptr;
  hipStream_t st;
  if (hipStreamCreate(&st) != hipSuccess) return QI_ERR_HIP;
  qi_status rc = QI_OK;
  if (hipMalloc(&out, 512 * sizeof(float)) != hipSuccess || hipMalloc(&clk, 2 * sizeof(unsigned long long)) != hipSuccess ||
      hipMalloc(&src, 4096 * sizeof(u32x4)) != hipSuccess)
    rc = QI_ERR_HIP;
  if (rc == QI_OK && hipMemsetAsync(src, 0, 4096 * sizeof(u32x4), st) != hipSuccess) rc = QI_ERR_HIP;
  auto run = [&](int n) {
    switch (mode) {
      case 0: hipLaunchKernelGGL(lds_mix_kernel<0>, dim3(cus), dim3(512), 0, st, out, n, clk, src); break;
      case 1: hipLaunchKernelGGL(lds_mix_kernel<1>, dim3(cus), dim3(512), 0, st, out, n, clk, src); break;
      case 2: hipLaunchKernelGGL(lds_mix_kernel<2>, dim3(cus), dim3(512), 0, st, out, n, clk, src); break;
      case 3: hipLaunchKernelGGL(lds_mix_kernel<3>, dim3(cus), dim3(512), 0, st, out, n, clk, src); break;
      default: hipLaunchKernelGGL(lds_mix_kernel<4>, dim3(cus), dim3(512), 0, st, out, n, clk, src); break;
    }
  };
  unsigned long long h[2] = {0, 0};
  if (rc == QI_OK) {
    run(100);  // warm-up
    if (hipMemsetAsync(clk, 0, 2 * sizeof(unsigned long long), st) != hipSuccess) rc = QI_ERR_HIP;
  }
  if (rc == QI_OK) {
    run(iters);
    if (hipMemcpyAsync(h, clk, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess || hipGetLastError() != hipSuccess)
      rc = QI_ERR_HIP;
  }
  *cycles = (rc == QI_OK && h[1]) ? (double)h[0] / (double)h[1] / iters : 0.0;
  if (out) (void)hipFree(out);
  if (clk) (void)hipFree(clk);
  if (src) (void)hipFree(src);
  (void)hipStreamDestroy(st);
  return rc;
}

qi_status qi_calib_valu_ns(int32_t mode, int32_t iters, double *ns) {
  if (!ns) return QI_ERR_NULL;
  if (mode < 0 || mode > 9 || iters < 4 || iters > 10000000) return QI_ERR_RANGE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QI_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return QI_ERR_HIP;
  float *out = nullptr;
  hipStream_t st;
  hipEvent_t e0, e1;
  if (hipStreamCreate(&st) != hipSuccess) return QI_ERR_HIP;
  qi_status rc = QI_OK;
  if (hipMalloc(&out, 1024 * sizeof(float)) != hipSuccess) rc = QI_ERR_HIP;
  if (rc == QI_OK && (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)) rc = QI_ERR_HIP;
  if (rc == QI_OK) {
    auto run = [&](int n) {
      switch (mode) {
        case 0: hipLaunchKernelGGL((valu_mix_kernel<2, 2, 2, 0>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 1: hipLaunchKernelGGL((valu_mix_kernel<2, 1, 2, 0>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 2: hipLaunchKernelGGL((valu_mix_kernel<2, 2, 3, 0>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 3: hipLaunchKernelGGL((valu_mix_kernel<2, 1, 3, 0>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 4: hipLaunchKernelGGL((valu_mix_kernel<2, 1, 1, 0>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 5: hipLaunchKernelGGL((valu_mix_kernel<2, 2, 0, 1>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 6: hipLaunchKernelGGL((valu_mix_kernel<2, 1, 0, 1>), dim3(cus), dim3(512), 0, st, out, n); break;
        case 7: hipLaunchKernelGGL((valu_mix_kernel<1, 1, 1, 0>), dim3(cus), dim3(256), 0, st, out, n); break;
        case 8: hipLaunchKernelGGL((valu_mix_kernel<1, 2, 2, 0>), dim3(cus), dim3(256), 0, st, out, n); break;
        default: hipLaunchKernelGGL((valu_mix_kernel<1, 1, 2, 0>), dim3(cus), dim3(256), 0, st, out, n); break;
      }
    };
    run(200);  // warm-up
    (void)hipEventRecord(e0, st);
    run(iters);
    (void)hipEventRecord(e1, st);
    float ms = 0.f;
    if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess ||
        hipGetLastError() != hipSuccess)
      rc = QI_ERR_HIP;
    *ns = rc == QI_OK ? (double)ms * 1e6 / iters : 0.0;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  if (out) (void)hipFree(out);
  (void)hipStreamDestroy(st);
  return rc;
}

}  // extern "C"
