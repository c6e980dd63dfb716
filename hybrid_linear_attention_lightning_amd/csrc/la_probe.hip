// la_probe.hip -- a streaming read-modify-write kernel for measuring the HBM
// rate the decode step's access pattern can reach on this GPU: x <- a x over
// n floats in place, 16-byte buffer accesses, each element read once and
// written once (the decode step's state traffic without its arithmetic),
// with the cache-policy bits of the loads and of the stores chosen
// separately.  Measurement only; no part of the layer uses it.
#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {

// LP, SP: cache-policy bits (sc0 = 1, nt = 2, sc1 = 16) of the loads and the
// stores.  Workgroup w covers float4 elements 1024 w .. 1024 w + 1023.
template <int LP, int SP>
__global__ __launch_bounds__(256) void stream_rmw_kernel(float* __restrict__ x, size_t n4, float a) {
  constexpr int PER = 4;  // float4 per thread, all loads issued before the stores
  const size_t blk = (size_t)blockIdx.x * 256 * PER;
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(x + 4 * blk);
  f32x4_t v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x + 256u * j;
    if (blk + i < n4)
      v[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * i, 0, LP));
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t i = threadIdx.x + 256u * j;
    if (blk + i < n4)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v[j] * a), r, 16u * i, 0,
                                             SP);
  }
}

template <int LP, int SP>
void launch(float* x, size_t n4, float a, hipStream_t s) {
  hipLaunchKernelGGL((stream_rmw_kernel<LP, SP>), dim3((unsigned)((n4 + 1023) / 1024)), dim3(256),
                     0, s, x, n4, a);
}

}  // namespace

hipError_t launch_stream_rmw(float* x, size_t n, float a, int load_policy, int store_policy,
                             hipStream_t s) {
  const size_t n4 = n / 4;
  const bool lnt = load_policy == kCpolNt;
  switch (store_policy) {
    case 0: lnt ? launch<kCpolNt, 0>(x, n4, a, s) : launch<0, 0>(x, n4, a, s); break;
    case kCpolNt:
      lnt ? launch<kCpolNt, kCpolNt>(x, n4, a, s) : launch<0, kCpolNt>(x, n4, a, s);
      break;
    case kCpolSc1:
      lnt ? launch<kCpolNt, kCpolSc1>(x, n4, a, s) : launch<0, kCpolSc1>(x, n4, a, s);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace la
