// la_decode.hip -- decode steps (one token, or a few tokens per call),
// HBM-streaming.
//
// Per (b, h) and token: S <- lambda S + k v^T, then o = q^T S (the recurrent
// form of Lightning Attention used for generation; Ling & Ring 2.6 pages,
// "Hybrid Linear Attention" section: O(n) training and decoding).  With K
// tokens per call the state makes one round trip for all K.
//
// The d x d fp32 state dominates the traffic (2 * 4 * d^2 bytes per (b, h)
// against 8 * d bytes of token data), so the kernel is a streaming
// read-modify-write: one workgroup per (b, h); each thread owns 4 adjacent
// value columns and every (256*4/d)-th key row, issues all its 16-byte state
// loads before any arithmetic, writes the updated rows back with 16-byte
// stores (64 consecutive lanes cover whole 512-byte rows), and the partial
// q^T S column sums of the row groups are reduced across lanes and then
// through LDS.
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

// K tokens (1 <= K <= KMAX) per (b, h): token j updates the state and reads
// o_j = q_j^T S_j, the K steps of the recurrence on a state held in
// registers, so the state is streamed once for all K tokens.
template <int D, typename T, int KMAX>
__global__ __launch_bounds__(256) void decode_kernel(int H, int K, const T* __restrict__ q,
                                                    const T* __restrict__ k,
                                                    const T* __restrict__ v,
                                                    const float* __restrict__ slope,
                                                    float* __restrict__ state, T* __restrict__ o) {
  constexpr int CG = D / 4;        // float4 column groups
  constexpr int RG = (256 / CG < D) ? 256 / CG : D;  // row groups
  constexpr int ROWS = D / RG;     // rows per thread
  constexpr int NWV = (CG * RG + 63) / 64;           // active waves
  __shared__ float qs[KMAX][D], ks[KMAX][D], vs[KMAX][D];
  __shared__ f32x4_t red[KMAX][NWV][CG];

  const int bh = blockIdx.x;
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int lane = tid & 63, wv = tid >> 6;
  float* S = state + (size_t)bh * D * D;

  const bool active = tid < CG * RG;  // all 256 threads unless d < 32

  // issue the state loads first: they are the whole cost
  f32x4_t sv[ROWS];
  if (active) {
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
      sv[m] = *reinterpret_cast<const f32x4_t*>(S + (size_t)(rg + RG * m) * D + 4 * cg);
  }

  const size_t tok0 = (size_t)bh * K * D;
  for (int e = tid; e < K * D; e += 256) {
    const int j = e / D, c = e - j * D;
    qs[j][c] = ld_tok(q + tok0, e);
    ks[j][c] = ld_tok(k + tok0, e);
    vs[j][c] = ld_tok(v + tok0, e);
  }
  const float lam = expf(-slope[h]);
  __syncthreads();

  if (active) {
    for (int j = 0; j < K; ++j) {
      const f32x4_t v4 = {vs[j][4 * cg], vs[j][4 * cg + 1], vs[j][4 * cg + 2], vs[j][4 * cg + 3]};
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < ROWS; ++m) {
        const int i = rg + RG * m;
        const float ki = ks[j][i], qi = qs[j][i];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sv[m][c] = fmaf(lam, sv[m][c], ki * v4[c]);
          acc[c] = fmaf(qi, sv[m][c], acc[c]);
        }
      }
      // sum over the row groups of this wave (lanes CG apart), then one
      // partial per wave through LDS
#pragma unroll
      for (int off = CG; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
      if (lane < CG) red[j][wv][cg] = acc;
    }
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
      *reinterpret_cast<f32x4_t*>(S + (size_t)(rg + RG * m) * D + 4 * cg) = sv[m];
  }
  __syncthreads();
  for (int e = tid; e < K * CG; e += 256) {
    const int j = e / CG, c4 = e - j * CG;
    f32x4_t t = red[j][0][c4];
#pragma unroll
    for (int g = 1; g < NWV; ++g) {
      const f32x4_t u = red[j][g][c4];
      t[0] += u[0];
      t[1] += u[1];
      t[2] += u[2];
      t[3] += u[3];
    }
    T* ob = o + tok0 + (size_t)j * D + 4 * c4;
    if constexpr (sizeof(T) == 4) {
      *reinterpret_cast<f32x4_t*>(ob) = t;
    } else {
      *reinterpret_cast<u32x2_t*>(ob) = u32x2_t{pack2(t[0], t[1]), pack2(t[2], t[3])};
    }
  }
}

template <int D, int KMAX>
hipError_t launch_d(bool bf16, int B, int H, int K, const void* q, const void* k, const void* v,
                    const float* slope, float* state, void* o, hipStream_t s) {
  const dim3 grid((unsigned)(B * H)), block(256);
  if (bf16)
    hipLaunchKernelGGL((decode_kernel<D, uint16_t, KMAX>), grid, block, 0, s, H, K,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, slope, state,
                       (uint16_t*)o);
  else
    hipLaunchKernelGGL((decode_kernel<D, float, KMAX>), grid, block, 0, s, H, K,
                       (const float*)q, (const float*)k, (const float*)v, slope, state,
                       (float*)o);
  return hipGetLastError();
}

template <int KMAX>
hipError_t launch_k(bool bf16, int B, int H, int K, int D, const void* q, const void* k,
                    const void* v, const float* slope, float* state, void* o, hipStream_t s) {
  switch (D) {
    case 16: return launch_d<16, KMAX>(bf16, B, H, K, q, k, v, slope, state, o, s);
    case 32: return launch_d<32, KMAX>(bf16, B, H, K, q, k, v, slope, state, o, s);
    case 64: return launch_d<64, KMAX>(bf16, B, H, K, q, k, v, slope, state, o, s);
    case 128: return launch_d<128, KMAX>(bf16, B, H, K, q, k, v, slope, state, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(bool bf16, int B, int H, int D, const void* q, const void* k,
                         const void* v, const float* slope, float* state, void* o,
                         hipStream_t s) {
  return launch_k<1>(bf16, B, H, 1, D, q, k, v, slope, state, o, s);
}

hipError_t launch_decode_tokens(bool bf16, int B, int H, int K, int D, const void* q,
                                const void* k, const void* v, const float* slope, float* state,
                                void* o, hipStream_t s) {
  // the smallest token capacity that holds K keeps the LDS footprint, and
  // so the loss of occupancy, to what K needs
  static_assert(kDecodeTokensMax == 16, "capacities below");
  if (K < 1 || K > kDecodeTokensMax) return hipErrorInvalidValue;
  if (K <= 2) return launch_k<2>(bf16, B, H, K, D, q, k, v, slope, state, o, s);
  if (K <= 4) return launch_k<4>(bf16, B, H, K, D, q, k, v, slope, state, o, s);
  if (K <= 8) return launch_k<8>(bf16, B, H, K, D, q, k, v, slope, state, o, s);
  return launch_k<16>(bf16, B, H, K, D, q, k, v, slope, state, o, s);
}

}  // namespace la
