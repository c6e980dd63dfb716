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
// read-modify-write:
//  * a workgroup owns one (b, h) (the columns could split across workgroups
//    with no reduction between them, since o_t[j] = sum_i q_t[i] S_t[i][j]
//    needs only column j, but measured one workgroup of 1024 threads per
//    (b, h) is fastest, below);
//  * each thread owns 4 adjacent value columns and every RG-th key row,
//    issues all its 16-byte state loads before any arithmetic and writes the
//    updated rows back with 16-byte stores;
//  * the state is read with non-temporal loads and written with stores that
//    carry the sc1 cache-policy bit and not nt.  A streaming read-modify-write
//    of a 134 MB buffer, timed over all 64 combinations of the sc0/sc1/nt
//    bits, is fast both when the buffer was written just before (0.87 of the
//    HBM peak: the Infinity Cache serves it) and when it comes from HBM
//    (0.75) only with nt loads and sc1 stores without nt.  Plain accesses
//    reach 0.85 and 0.65, nt loads and stores 0.76 and 0.75;
//  * the partial q^T S column sums of the row groups are reduced across
//    lanes and then through LDS;
//  * with one token per call each thread loads the q and k entries of its
//    rows and the v entries of its columns itself, so no barrier stands
//    between a wave's state loads and its stores (measured 1% faster than
//    staging the token in LDS first, with the state from HBM or not); with
//    several tokens they are staged in LDS once for the workgroup, and the
//    wave partials of o go through LDS in rounds of at most 8 tokens (4
//    above 8), so that two workgroups still fit on a CU at 16 tokens
//    (16-token call 82 against 101 us with all 16 partials at once).
// On the B=64, H=32, d=128 step (one machine, best of three rounds), state
// from HBM / state in the Infinity Cache: 1024 threads per (b, h) 45.0 /
// 39.2 us; 512 threads per (b, h) 45.1 / 39.7 us; 1024 threads per half of
// the columns 44.2 / 41.6 us; 512 threads per half 47.2 / 41.0 us.
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

// 16-byte state accesses: non-temporal loads; stores through a buffer
// resource over the workgroup's state slice, at byte offset off, with the
// sc1 cache-policy bit.
__device__ __forceinline__ f32x4_t ld_state(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}
__device__ __forceinline__ void st_state(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kCpolSc1);
}

// Value columns per workgroup: all of them.
template <int D>
constexpr int decode_cols() { return D; }
// Threads per workgroup: one per (4 columns, row) up to 1024.
template <int D>
constexpr int dec_threads() { return D / 4 * D < 1024 ? D / 4 * D : 1024; }

// K tokens (1 <= K <= KMAX) per (b, h): token j updates the state and reads
// o_j = q_j^T S_j, the K steps of the recurrence on a state held in
// registers, so the state is streamed once for all K tokens.  Workgroup
// (b h) * SPLIT + part owns value columns part * COLS .. +COLS-1.
template <int D, typename T, int KMAX>
__global__ __launch_bounds__(dec_threads<D>()) void decode_kernel(int H, int K, const T* __restrict__ q,
                                                    const T* __restrict__ k,
                                                    const T* __restrict__ v,
                                                    const float* __restrict__ slope,
                                                    float* __restrict__ state, T* __restrict__ o) {
  constexpr int kDecThreads = dec_threads<D>();
  constexpr int COLS = decode_cols<D>();
  constexpr int SPLIT = D / COLS;  // workgroups per (b, h)
  constexpr int CG = COLS / 4;     // float4 column groups
  constexpr int RG = (kDecThreads / CG < D) ? kDecThreads / CG : D;  // row groups
  constexpr int ROWS = D / RG;     // rows per thread
  constexpr int NWV = (CG * RG + 63) / 64;           // active waves
  __shared__ __attribute__((aligned(16))) float qs[KMAX][D], ks[KMAX][D], vs[KMAX][COLS];
  // cross-wave partial sums of o, for up to KR tokens at a time: rounds of
  // 4 tokens above 8 keep the workgroup's LDS below half of the CU's, so
  // that two workgroups of 1024 threads still fit
  constexpr int KR = KMAX <= 8 ? KMAX : 4;
  __shared__ f32x4_t red[KR][NWV][CG];

  const int bh = blockIdx.x / SPLIT;
  const int c_base = (blockIdx.x % SPLIT) * COLS;  // first value column
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int lane = tid & 63, wv = tid >> 6;
  float* Sw = state + (size_t)bh * D * D + c_base;  // the workgroup's slice
  float* S = Sw + 4 * cg;

  const bool active = tid < CG * RG;  // every thread: the workgroup has CG * RG

  // issue the state loads first: they are the whole cost
  f32x4_t sv[ROWS];
  if (active) {
#pragma unroll
    for (int m = 0; m < ROWS; ++m) sv[m] = ld_state(S + (size_t)(rg + RG * m) * D);
  }

  const size_t tok0 = (size_t)bh * K * D;
  // o for tokens j0 .. j0 + nk - 1 from the waves' partials in red
  auto reduce_store = [&](int j0, int nk) {
    for (int e = tid; e < nk * CG; e += kDecThreads) {
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
      T* ob = o + tok0 + (size_t)(j0 + j) * D + c_base + 4 * c4;
      if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<f32x4_t*>(ob) = t;
      } else {
        *reinterpret_cast<u32x2_t*>(ob) = u32x2_t{pack2(t[0], t[1]), pack2(t[2], t[3])};
      }
    }
  };
  const float lam = expf(-slope[h]);
  if constexpr (KMAX == 1) {
    // one token: each thread loads the q and k entries of its rows and the v
    // entries of its columns itself, so that no barrier stands between a
    // wave's state loads and its stores
    if (active) {
      float qv[ROWS], kv[ROWS];
#pragma unroll
      for (int m = 0; m < ROWS; ++m) {
        qv[m] = ld_tok(q + tok0, rg + RG * m);
        kv[m] = ld_tok(k + tok0, rg + RG * m);
      }
      f32x4_t v4;
#pragma unroll
      for (int c = 0; c < 4; ++c) v4[c] = ld_tok(v + tok0, c_base + 4 * cg + c);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < ROWS; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sv[m][c] = fmaf(lam, sv[m][c], kv[m] * v4[c]);
          acc[c] = fmaf(qv[m], sv[m][c], acc[c]);
        }
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(Sw);
#pragma unroll
      for (int m = 0; m < ROWS; ++m)
        st_state(rs, (uint32_t)(((rg + RG * m) * D + 4 * cg) * sizeof(float)), sv[m]);
#pragma unroll
      for (int off = CG; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
      if (lane < CG) red[0][wv][cg] = acc;
    }
  } else {
  // q and k entries stored by row group: row rg + RG m at rg ROWS + m, so
  // that a thread reads its ROWS entries of a token as one vector
  for (int e = tid; e < K * D; e += kDecThreads) {
    const int j = e / D, c = e - j * D;
    const int x = (c % RG) * ROWS + c / RG;
    qs[j][x] = ld_tok(q + tok0, e);
    ks[j][x] = ld_tok(k + tok0, e);
  }
  for (int e = tid; e < K * COLS; e += kDecThreads) {
    const int j = e / COLS, c = e - j * COLS;
    vs[j][c] = ld_tok(v + tok0, j * D + c_base + c);
  }
  __syncthreads();

  // tokens in rounds of KR; a round's partials are reduced before the next
  // round writes its own (all but the last round end in two barriers, after
  // the state loads have all been waited for)
  for (int j0 = 0; j0 < K; j0 += KR) {
  const int nk = K - j0 < KR ? K - j0 : KR;
  if (active) {
    for (int j = j0; j < j0 + nk; ++j) {
      const f32x4_t v4 = {vs[j][4 * cg], vs[j][4 * cg + 1], vs[j][4 * cg + 2], vs[j][4 * cg + 3]};
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < ROWS; ++m) {
        const float ki = ks[j][ROWS * rg + m], qi = qs[j][ROWS * rg + m];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // in place (scale, then accumulate k v): the state keeps its
          // registers from token to token, with no copies between them
          sv[m][c] *= lam;
          sv[m][c] = fmaf(ki, v4[c], sv[m][c]);
          acc[c] = fmaf(qi, sv[m][c], acc[c]);
        }
      }
      // sum over the row groups of this wave (lanes CG apart), then one
      // partial per wave through LDS
#pragma unroll
      for (int off = CG; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
      if (lane < CG) red[j - j0][wv][cg] = acc;
    }
    if (j0 + nk == K) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(Sw);
#pragma unroll
      for (int m = 0; m < ROWS; ++m)
        st_state(rs, (uint32_t)(((rg + RG * m) * D + 4 * cg) * sizeof(float)), sv[m]);
    }
  }
  if (j0 + nk < K) {
    __syncthreads();
    reduce_store(j0, nk);
    __syncthreads();
  }
  }
  }
  __syncthreads();
  const int last = KMAX == 1 ? 0 : (K - 1) / KR * KR;  // the last round's first token
  reduce_store(last, K - last);
}

template <int D, int KMAX>
hipError_t launch_d(bool bf16, int B, int H, int K, const void* q, const void* k, const void* v,
                    const float* slope, float* state, void* o, hipStream_t s) {
  const dim3 grid((unsigned)(B * H * (D / decode_cols<D>()))), block(dec_threads<D>());
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
