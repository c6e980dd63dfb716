// la_decode.hip -- single-token decode step, HBM-streaming.
//
// Per (b, h): S <- lambda S + k v^T, then o = q^T S (the recurrent form of
// Lightning Attention used for generation; Ling & Ring 2.6 pages, "Hybrid
// Linear Attention" section: O(n) training and decoding).
//
// The d x d fp32 state dominates the traffic (2 * 4 * d^2 bytes per (b, h)
// against 8 * d bytes of token data), so the kernel is a streaming
// read-modify-write: one workgroup per (b, h); each thread owns 4 adjacent
// value columns and every (256*4/d)-th key row, issues all its 16-byte state
// loads before any arithmetic, writes the updated rows back with 16-byte
// stores (64 consecutive lanes cover whole 512-byte rows), and the partial
// q^T S column sums of the row groups are reduced through LDS.
#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {

template <typename T>
__device__ __forceinline__ float ld_tok(const T* p, int i);
template <>
__device__ __forceinline__ float ld_tok<float>(const float* p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_tok<uint16_t>(const uint16_t* p, int i) {
  return bf2f(p[i]);
}

template <int D, typename T>
__global__ __launch_bounds__(256) void decode_kernel(int H, const T* __restrict__ q,
                                                    const T* __restrict__ k,
                                                    const T* __restrict__ v,
                                                    const float* __restrict__ slope,
                                                    float* __restrict__ state, T* __restrict__ o) {
  constexpr int CG = D / 4;        // float4 column groups
  constexpr int RG = (256 / CG < D) ? 256 / CG : D;  // row groups
  constexpr int ROWS = D / RG;     // rows per thread
  __shared__ float qs[D], ks[D], vs[D];
  __shared__ f32x4_t red[RG][CG];

  const int bh = blockIdx.x;
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  float* S = state + (size_t)bh * D * D;

  const bool active = tid < CG * RG;  // all 256 threads unless d < 32

  // issue the state loads first: they are the whole cost
  f32x4_t sv[ROWS];
  if (active) {
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
      sv[m] = *reinterpret_cast<const f32x4_t*>(S + (size_t)(rg + RG * m) * D + 4 * cg);
  }

  if (tid < D) {
    qs[tid] = ld_tok(q + (size_t)bh * D, tid);
    ks[tid] = ld_tok(k + (size_t)bh * D, tid);
    vs[tid] = ld_tok(v + (size_t)bh * D, tid);
  }
  const float lam = expf(-slope[h]);
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
  const f32x4_t v4 = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
#pragma unroll
  for (int m = 0; m < ROWS; ++m) {
    const int i = rg + RG * m;
    const float ki = ks[i], qi = qs[i];
    f32x4_t s;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s[c] = fmaf(lam, sv[m][c], ki * v4[c]);
      acc[c] = fmaf(qi, s[c], acc[c]);
    }
    *reinterpret_cast<f32x4_t*>(S + (size_t)i * D + 4 * cg) = s;
  }
  red[rg][cg] = acc;
  }
  __syncthreads();
  if (tid < CG) {
    f32x4_t t = red[0][tid];
#pragma unroll
    for (int g = 1; g < RG; ++g) {
      const f32x4_t u = red[g][tid];
      t[0] += u[0];
      t[1] += u[1];
      t[2] += u[2];
      t[3] += u[3];
    }
    T* ob = o + (size_t)bh * D + 4 * tid;
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<f32x4_t*>(ob) = t;
    } else {
      *reinterpret_cast<u32x2_t*>(ob) = u32x2_t{pack2(t[0], t[1]), pack2(t[2], t[3])};
    }
  }
}

template <int D>
hipError_t launch_d(bool bf16, int B, int H, const void* q, const void* k, const void* v,
                    const float* slope, float* state, void* o, hipStream_t s) {
  const dim3 grid((unsigned)(B * H)), block(256);
  if (bf16)
    hipLaunchKernelGGL((decode_kernel<D, uint16_t>), grid, block, 0, s, H,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, slope, state,
                       (uint16_t*)o);
  else
    hipLaunchKernelGGL((decode_kernel<D, float>), grid, block, 0, s, H, (const float*)q,
                       (const float*)k, (const float*)v, slope, state, (float*)o);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(bool bf16, int B, int H, int D, const void* q, const void* k,
                         const void* v, const float* slope, float* state, void* o,
                         hipStream_t s) {
  switch (D) {
    case 16: return launch_d<16>(bf16, B, H, q, k, v, slope, state, o, s);
    case 32: return launch_d<32>(bf16, B, H, q, k, v, slope, state, o, s);
    case 64: return launch_d<64>(bf16, B, H, q, k, v, slope, state, o, s);
    case 128: return launch_d<128>(bf16, B, H, q, k, v, slope, state, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
