// Calibration kernels: what one gfx950 GPU delivers for a streaming HBM read,
// for the merges' pattern of several read streams and one write stream, and
// for a register-resident bf16 MFMA loop.  The decode and merge kernels'
// roofline fractions are quoted against the vendor peaks (8 TB/s HBM, 2.5
// PFLOP/s dense bf16) and against these measured ceilings.  Contracts in
// include/mla_calib.h.
#include <hip/hip_runtime.h>

#include "mla.h"
#include "mla_calib.h"
#include "mla_common.h"

namespace mla {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// Every thread streams 16-byte words with a grid stride, kReadUnroll loads in
// flight, and folds them with xor so that no load is dead; one word per thread
// goes to the sink at the end (a few hundred KiB against GiB read).
template <bool kNT>
__global__ __launch_bounds__(kReadThreads) void calib_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                                  uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = kNT ? __builtin_nontemporal_load(buf + i + u * stride) : buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= buf[i];
  const int64_t gid = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  if (gid < MLA_CALIB_SINK_WORDS) sink[gid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// The merges' access pattern: R input streams read once, one output stream
// written once (16-byte words, two per thread and input in flight, grid
// stride); the output is the xor of the inputs so that no load is dead.
template <int R>
__global__ __launch_bounds__(kReadThreads) void calib_gather_kernel(const u32x4* __restrict__ in, int64_t n16,
                                                                    u32x4* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads * 2;
  for (int64_t base = (int64_t)blockIdx.x * kReadThreads * 2 + threadIdx.x; base < n16; base += stride) {
    u32x4 acc[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t i = base + u * kReadThreads;
        if (i < n16) acc[u] ^= in[r * n16 + i];
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t i = base + u * kReadThreads;
      if (i < n16) out[i] = acc[u];
    }
  }
}

// Each wave runs `iters` rounds of kMfmaChains independent MFMA 16x16x32 bf16
// accumulation chains on operands that stay in registers.
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(MLA_CALIB_MFMA_THREADS) void calib_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  f32x4 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  const int gid = (int)blockIdx.x * MLA_CALIB_MFMA_THREADS + (int)threadIdx.x;
  if (gid < MLA_CALIB_SINK_WORDS) sink[gid] = s;
}

}  // namespace mla

extern "C" {

mla_status mla_calib_hbm_read(const void* buf, size_t bytes, int32_t nontemporal, uint32_t* sink,
                              void* hip_stream) {
  if (bytes == 0) return MLA_OK;
  if (!buf || !sink) return MLA_ERR_NULL;
  if (bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0) return MLA_ERR_SHAPE;
  const int64_t n16 = (int64_t)(bytes / 16);
  // Sixteen 256-thread workgroups per CU of the 256-CU part; at most one
  // thread per 16-byte word.
  int64_t grid = 256 * 16;
  const int64_t need = (n16 + mla::kReadThreads - 1) / mla::kReadThreads;
  if (grid > need) grid = need;
  hipStream_t s = (hipStream_t)hip_stream;
  if (nontemporal)
    hipLaunchKernelGGL(mla::calib_read_kernel<true>, dim3((unsigned)grid), dim3(mla::kReadThreads), 0, s,
                       (const mla::u32x4*)buf, n16, sink);
  else
    hipLaunchKernelGGL(mla::calib_read_kernel<false>, dim3((unsigned)grid), dim3(mla::kReadThreads), 0, s,
                       (const mla::u32x4*)buf, n16, sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_calib_hbm_gather(const void* in, size_t bytes_per_input, int32_t inputs, void* out,
                                void* hip_stream) {
  if (bytes_per_input == 0) return MLA_OK;
  if (!in || !out) return MLA_ERR_NULL;
  if (bytes_per_input % 16 != 0 || ((uintptr_t)in & 15) != 0 || ((uintptr_t)out & 15) != 0 ||
      (inputs != 1 && inputs != 2 && inputs != 4 && inputs != 8))
    return MLA_ERR_SHAPE;
  const int64_t n16 = (int64_t)(bytes_per_input / 16);
  // Four 256-thread workgroups per CU of the 256-CU part (measured best of
  // 1024..8192 for eight inputs).
  int64_t grid = 1024;
  const int64_t need = (n16 + 2 * mla::kReadThreads - 1) / (2 * mla::kReadThreads);
  if (grid > need) grid = need;
  hipStream_t s = (hipStream_t)hip_stream;
  const mla::u32x4* pi = (const mla::u32x4*)in;
  mla::u32x4* po = (mla::u32x4*)out;
  switch (inputs) {
    case 1: hipLaunchKernelGGL(mla::calib_gather_kernel<1>, dim3((unsigned)grid), dim3(mla::kReadThreads), 0, s, pi, n16, po); break;
    case 2: hipLaunchKernelGGL(mla::calib_gather_kernel<2>, dim3((unsigned)grid), dim3(mla::kReadThreads), 0, s, pi, n16, po); break;
    case 4: hipLaunchKernelGGL(mla::calib_gather_kernel<4>, dim3((unsigned)grid), dim3(mla::kReadThreads), 0, s, pi, n16, po); break;
    default: hipLaunchKernelGGL(mla::calib_gather_kernel<8>, dim3((unsigned)grid), dim3(mla::kReadThreads), 0, s, pi, n16, po); break;
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

double mla_calib_mfma_flops(int32_t iters) {
  return iters < 0 ? -1.0
                   : (double)MLA_CALIB_MFMA_GROUPS * (MLA_CALIB_MFMA_THREADS / 64) * (double)iters *
                         mla::kMfmaChains * (2.0 * 16 * 16 * 32);
}

mla_status mla_calib_mfma_bf16(int32_t iters, float* sink, void* hip_stream) {
  if (iters < 0) return MLA_ERR_SHAPE;
  if (!sink) return MLA_ERR_NULL;
  hipLaunchKernelGGL(mla::calib_mfma_kernel, dim3(MLA_CALIB_MFMA_GROUPS), dim3(MLA_CALIB_MFMA_THREADS), 0,
                     (hipStream_t)hip_stream, (int)iters, sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
