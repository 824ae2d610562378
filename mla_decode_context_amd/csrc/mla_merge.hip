// Exact LSE-weighted merge of per-rank DCP partials, alone and fused with the
// per-head W_UV up-projection, for gfx950 (CDNA4).
//
// What is computed follows PR #48196 ("DCP sparse MLA output-merge
// optimizations"): the merge weights each rank's partial by exp(lse_r - LSE)
// with LSE = ln sum_r exp(lse_r), ranks whose per-row valid count is zero take
// no part (their buffers are not read), and the W_UV projection is linear, so
// projecting the merged latent row equals merging the projected partials.
//
// Both kernels stream the partials once from HBM (the merge is bandwidth-bound:
// about W*1 KiB read per (token, head) against 1 KiB or 256 B written).
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

// Rank w takes part in row t iff valid[w,t] > 0, or, without counts, iff its
// LSE is above -inf (a NaN LSE is treated as not taking part).  With counts,
// nothing else of a rank that does not take part is read.
__device__ __forceinline__ bool takes_part(const MergeParams& a, int w, int t, size_t lse_idx,
                                           float& lse_w) {
  if (a.valid && a.valid[(size_t)w * a.T + t] <= 0) return false;
  lse_w = a.lses[lse_idx];
  return a.valid ? true : (lse_w > -INFINITY);
}

// Merge weights of row (t, h): fills LSE and returns false when no rank takes part.
__device__ __forceinline__ bool merge_lse(const MergeParams& a, int t, int h, float& lse_tot) {
  const size_t plane = (size_t)a.T * a.H;
  const size_t row = (size_t)t * a.H + h;
  float mx = -INFINITY;
  bool any = false;
  for (int w = 0; w < a.W; ++w) {
    float l;
    if (takes_part(a, w, t, w * plane + row, l)) {
      mx = any ? fmaxf(mx, l) : l;
      any = true;
    }
  }
  if (!any) {
    lse_tot = -INFINITY;
    return false;
  }
  float sum = 0.f;
  for (int w = 0; w < a.W; ++w) {
    float l;
    if (takes_part(a, w, t, w * plane + row, l)) sum += fast_exp2((l - mx) * kLog2e);
  }
  lse_tot = mx + fast_log2(sum) * kLn2;
  return true;
}

// Workgroup = (token t, 16 heads); thread (head 16*blockIdx.y + tid / 16, dims
// 32*(tid % 16) .. +32).  Whether rank w takes part in row t is the same for
// every thread of the workgroup, so valid[w, t] comes through scalar loads;
// the LSEs and partials of up to eight participating ranks are then loaded
// together and combined online (running max, rescaled sum), ranks in order.
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams a) {
  const int t = blockIdx.x;
  const int h = 16 * blockIdx.y + (threadIdx.x >> 4);
  const int d0 = 32 * (threadIdx.x & 15);
  const bool hok = h < a.H;
  const int hc = hok ? h : a.H - 1;
  const size_t plane = (size_t)a.T * a.H;
  const size_t row = (size_t)t * a.H + hc;
  const int32_t* vcol = a.valid;
  float m = -INFINITY, ssum = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int w0 = 0; w0 < a.W; w0 += 8) {
    float l[8];
    u32x4 x[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int w = w0 + u;
      bool take = w < a.W;
      if (take && vcol)
        take = ((const __attribute__((address_space(4))) int32_t*)vcol)[(size_t)w * a.T + t] > 0;
      l[u] = -INFINITY;
      if (take) {
        l[u] = a.lses[w * plane + row];
        const u32x4* src = (const u32x4*)(a.outs + (w * plane + row) * kLatent + d0);
        if (vcol || l[u] > -INFINITY) {
#pragma unroll
          for (int k = 0; k < 4; ++k) x[u][k] = src[k];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // A rank whose LSE is -inf (or NaN, without counts) adds nothing.
      const float mn = fmaxf(m, l[u]);
      if (l[u] > -INFINITY && mn > -INFINITY) {
        const float c_old = m == -INFINITY ? 0.f : fast_exp2((m - mn) * kLog2e);
        const float c_new = fast_exp2((l[u] - mn) * kLog2e);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = acc[2 * k] * c_old + f32x4{bf16_lo(x[u][k][0]), bf16_hi(x[u][k][0]),
                                                  bf16_lo(x[u][k][1]), bf16_hi(x[u][k][1])} * c_new;
          acc[2 * k + 1] = acc[2 * k + 1] * c_old + f32x4{bf16_lo(x[u][k][2]), bf16_hi(x[u][k][2]),
                                                          bf16_lo(x[u][k][3]), bf16_hi(x[u][k][3])} * c_new;
        }
        ssum = ssum * c_old + c_new;
        m = mn;
      }
    }
  }
  if (!hok) return;
  const float inv = ssum > 0.f ? 1.f / ssum : 0.f;
  uint16_t* op = a.out + row * kLatent + d0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *(u32x4*)(op + 8 * k) = u32x4{pack_bf16x2(acc[2 * k][0] * inv, acc[2 * k][1] * inv),
                                  pack_bf16x2(acc[2 * k][2] * inv, acc[2 * k][3] * inv),
                                  pack_bf16x2(acc[2 * k + 1][0] * inv, acc[2 * k + 1][1] * inv),
                                  pack_bf16x2(acc[2 * k + 1][2] * inv, acc[2 * k + 1][3] * inv)};
  if (a.out_lse && (threadIdx.x & 15) == 0) a.out_lse[row] = ssum > 0.f ? m + fast_log2(ssum) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Merge fused with W_UV.  Workgroup = (head h, 64 tokens); wave w owns tokens
// 16w .. 16w+15 of the block.  For each 32-wide k-step the wave forms the
// merged latent slice of its 16 tokens directly in the MFMA operand layout
// (lane (token lr, group g) holds dims 32s + 8g .. +8), rounds it to bf16 and
// multiplies it with W_UV[h]^T, which the workgroup stages in LDS transposed
// ([n][k]) 128 k-rows at a time.  y^T[n][token] accumulates in 8 tiles of
// 16 n x 16 tokens.
// ---------------------------------------------------------------------------
constexpr int kProjTok = 64;       // tokens per workgroup
constexpr int kKChunk = 128;       // k rows of W_UV staged per pass
constexpr int kWtStride = kKChunk + 8;   // LDS row stride (bf16) of W_UV^T: 272 B

__global__ __launch_bounds__(256) void merge_v_up_kernel(const MergeParams a) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kVHead * kWtStride];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;
  const int h = blockIdx.y;
  const int t = blockIdx.x * kProjTok + 16 * w + lr;
  const bool row_ok = t < a.T;
  const size_t plane = (size_t)a.T * a.H;
  const size_t rowi = (size_t)(row_ok ? t : 0) * a.H + h;

  float lse_tot = -INFINITY;
  const bool any = row_ok && merge_lse(a, row_ok ? t : 0, h, lse_tot);

  f32x4 y[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) y[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* wsrc = a.wuv + (size_t)h * kLatent * kVHead;
  for (int kc = 0; kc < kLatent; kc += kKChunk) {
    __syncthreads();
    // Stage W_UV[h][kc .. kc+128][0 .. 128] transposed: thread takes k = idx % 128
    // and eight consecutive n, writes them down column k of rows n .. n+7.
#pragma unroll
    for (int it = 0; it < (kKChunk * kVHead / 8) / 256; ++it) {
      const int idx = it * 256 + threadIdx.x;
      const int k = idx & (kKChunk - 1);
      const int n0 = (idx / kKChunk) * 8;
      const u32x4 v = *(const u32x4*)(wsrc + (size_t)(kc + k) * kVHead + n0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wt[(n0 + 2 * e) * kWtStride + k] = (uint16_t)(v[e] & 0xFFFFu);
        wt[(n0 + 2 * e + 1) * kWtStride + k] = (uint16_t)(v[e] >> 16);
      }
    }
    __syncthreads();

#pragma unroll
    for (int s = 0; s < kKChunk / 32; ++s) {
      const int d0 = kc + 32 * s + 8 * g;
      float m8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (any) {
        for (int wr = 0; wr < a.W; ++wr) {
          float l;
          if (takes_part(a, wr, t, wr * plane + rowi, l)) {
            const float wgt = fast_exp2((l - lse_tot) * kLog2e);
            const u32x4 v = *(const u32x4*)(a.outs + (wr * plane + rowi) * kLatent + d0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              m8[2 * e] += wgt * bf16_lo(v[e]);
              m8[2 * e + 1] += wgt * bf16_hi(v[e]);
            }
          }
        }
      }
      const u32x4 mb = u32x4{pack_bf16x2(m8[0], m8[1]), pack_bf16x2(m8[2], m8[3]),
                             pack_bf16x2(m8[4], m8[5]), pack_bf16x2(m8[6], m8[7])};
      const bf16x8 bop = __builtin_bit_cast(bf16x8, mb);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const u32x4 av = *(const u32x4*)(wt + (16 * nt + lr) * kWtStride + 32 * s + 8 * g);
        y[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bop, y[nt], 0, 0, 0);
      }
    }
  }

  // y^T tile nt: lane (token lr, group g) holds n = 16nt + 4g + (0..3).
  if (row_ok) {
    uint16_t* op = a.out + ((size_t)t * a.H + h) * kVHead + 4 * g;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      *(u32x2*)(op + 16 * nt) = u32x2{pack_bf16x2(y[nt][0], y[nt][1]), pack_bf16x2(y[nt][2], y[nt][3])};
    if (a.out_lse && g == 0) a.out_lse[rowi] = lse_tot;
  }
}

hipError_t launch_lse_merge(const MergeParams& p, hipStream_t stream) {
  if (p.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)p.T, (unsigned)((p.H + 15) / 16)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge_v_up(const MergeParams& p, hipStream_t stream) {
  if (p.T <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.T + kProjTok - 1) / kProjTok), (unsigned)p.H);
  hipLaunchKernelGGL(merge_v_up_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
