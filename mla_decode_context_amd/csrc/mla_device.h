// Device helpers shared by the gfx950 decode kernels: MFMA wrappers, LDS-DMA
// loads, transposed LDS reads, wait-count operands, device-scope workspace
// accesses, lane-swap reductions and the split-slot map.
#pragma once

#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

constexpr int kRowBytes = kRow * 2;              // 1152: one cache row

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed 64-bit LDS read: within each 16-lane group, lane i receives
// element (i & 3) of the four-element chunk addressed by lane 4e + (i >> 2),
// for e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16_at(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uint8_t*)p);
}

// Direct-to-LDS load (gfx950 global_load_lds_dwordx4): each lane fetches 16
// bytes from its own global address and the wave's 64 results fill the 1 KiB of
// LDS starting at lds_block (wave-uniform; passed in M0).  The 16-head decode
// loads cache rows with the non-temporal hint (dma_16B_to_lds_stream and the
// SGPR-base form with kNT): there one workgroup reads each row once per call,
// and with the hint a 340 MB cache decoded 8 % faster from a flushed
// last-level cache.  The 128-head decode shares every row among the
// workgroups of a request's rows and head blocks through L2, so it loads
// without the hint.  Issued through asm so
// that the compiler adds no wait of its own: the kernel orders these loads with
// explicit vmcnt waits and barriers.  The asm is volatile with a memory clobber,
// so no other memory access moves across it.  A write of M0 needs one wait state
// before an LDS-DMA instruction reads it, hence the s_nop.  M0 is not named as
// a clobber: LLVM reserves it and ignores it in clobber lists, so it is this
// asm's to use only because the compiled kernels read M0 nowhere else (a CPU
// test scans the gfx950 assembly of every kernel source for that).
__device__ __forceinline__ void dma_16B_to_lds(const void* src, const uint8_t* lds_block) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds_block);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory");
}

// The same load with the non-temporal hint, for cache rows (see below).
__device__ __forceinline__ void dma_16B_to_lds_stream(const void* src, const uint8_t* lds_block) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)lds_block);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(lds), "v"(src)
               : "memory");
}

// Two FP8 E4M3 codes (bytes 0-1 of `w`, or bytes 2-3 with kHi) -> two bf16
// (low half = the lower byte's value).  Exact: every E4M3 value is a bf16
// value; the scale operand is 1.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// Empty asm that "uses" a pointer, extending its registers' live range.
__device__ __forceinline__ void keep_live(const void* p) { asm volatile("" : : "v"(p)); }

// Device-scope (all-XCD coherent) accesses to the split workspace: relaxed
// atomics at agent scope, which the compiler emits as plain loads and stores
// with the device-coherence cache policy and no fences.
__device__ __forceinline__ void store_device(float* p, float x, float y) {
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float* p) {
  return __uint_as_float(__hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ f32x4 load_device4(const float* p) {
  const uint64_t lo = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load((const uint64_t*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
               __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
}

// Splits of a row with L visible keys: ceil(L / chunk), at least 1, at most the
// grid's split extent.
__device__ __forceinline__ int num_splits_of(int L, int chunk, int max_splits) {
  const int n = L > 0 ? (L + chunk - 1) / chunk : 1;
  return n < max_splits ? n : max_splits;
}

// Where the partials of a split row live: piece k of the row (k = 0..np-1)
// stores its heads at workspace row base + k*stride (+ adj0 for k = 0); a
// workspace row holds H heads of 512 fp32 plus H LSEs.
struct SlotMap {
  int base, stride, adj0;
  __device__ __forceinline__ int64_t row(int k) const {
    return (int64_t)base + (int64_t)k * stride + (k == 0 ? adj0 : 0);
  }
};

// vmcnt(n) operand of s_waitcnt (expcnt and lgkmcnt left at their maxima).
#define MLA_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// s_waitcnt operand: lgkmcnt(0), vmcnt and expcnt left at their maxima.
#define MLA_LGKMCNT0 (15 | (3 << 14) | (7 << 4))

// Direct-to-LDS loads with a wave-uniform 64-bit base in SGPRs and a per-lane
// 32-bit byte offset; see dma_16B_to_lds.
//
// make_sbase() assembles the base in SGPRs: each 32-bit half comes from the
// first lane (the value is uniform).  readfirstlane returns int: the low half
// is widened through uint32_t so that it is zero-extended, never
// sign-extended into the high half.  The readfirstlanes are VALU writes of the
// SGPRs, and a VMEM instruction may read an SGPR only five wait states after a
// VALU wrote it; the compiler inserts no wait states inside inline asm, so
// make_sbase() ends with an s_nop 4 that names the new SGPRs as operands (it
// is ordered after their writes and before the loads, which are volatile asm
// too).  Every load of the stage then uses the settled base and needs only
// the one wait state for M0.  A CPU test checks the compiled kernels for a
// VALU write of a base SGPR closer than five wait states to a load.
__device__ __forceinline__ uint64_t make_sbase(const void* base) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sbase = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_nop 4" : : "s"(sbase));
  return sbase;
}

// Block-table entry p[0], the same for every lane, read with a scalar load:
// both halves of the address go through readfirstlane, so the compiler sees a
// wave-uniform address even when it keeps the row pointer in VGPRs.  (A vector
// load would be waited for with vmcnt, i.e. behind every stage load in flight.)
__device__ __forceinline__ int load_uniform_i32(const int32_t* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

template <bool kNT>
__device__ __forceinline__ void dma_16B_to_lds_sbase(uint32_t lds_off, uint32_t voff, uint64_t sbase) {
  if (kNT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_off), "v"(voff), "s"(sbase)
                 : "memory");
}

// Output stores of the decode kernels: dims d .. d+3 (or d+7) of output row
// `row` (= t*H + h), as bf16 (round to nearest even) or, when the caller asked
// for fp32 partials, as fp32.  The branch is uniform (a kernel argument).
__device__ __forceinline__ void store_out4(const DecodeParams& a, size_t row, int d, f32x4 x) {
  if (a.out_f)
    *(f32x4*)(a.out_f + row * kLatent + d) = x;
  else
    *(u32x2*)(a.out + row * kLatent + d) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}
__device__ __forceinline__ void store_out8(const DecodeParams& a, size_t row, int d, f32x4 x, f32x4 y) {
  if (a.out_f) {
    *(f32x4*)(a.out_f + row * kLatent + d) = x;
    *(f32x4*)(a.out_f + row * kLatent + d + 4) = y;
  } else {
    *(u32x4*)(a.out + row * kLatent + d) = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                 pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  }
}
__device__ __forceinline__ void zero_out8(const DecodeParams& a, size_t row, int d) {
  store_out8(a, row, d, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f});
}

// max / sum over the four lanes l, l^16, l^32, l^48 (one MFMA column) with the
// gfx950 lane-swap instructions (VALU, no LDS round trip).
__device__ __forceinline__ float col_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


}  // namespace mla
