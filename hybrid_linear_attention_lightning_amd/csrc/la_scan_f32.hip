// la_scan_f32.hip -- segment start states, and the fp32 reference-precision
// forward.
//
// Segment start states.  The "Context Parallel for Lightning Attention"
// section of the Ling & Ring 2.6 pages computes each shard's hidden state
// from a zero start (local recursion) and then corrects every shard with the
// states of the shards before it (global correction).  On one GPU the same
// algebra gives parallelism along the sequence: with segments of L tokens and
// pieces of Lp tokens (Lp divides L), the state entering segment r is
//
//   S_in(r) = lambda^L S_in(r-1) + sum_{pieces p in segment r-1}
//                                  lambda^(rL - end_p) P_p,       S_in(0) = S0
//
// where P_p = sum_{t in p} lambda^(end_p - 1 - t) k_t v_t^T and end_p is one
// past the piece's last token.  A piece whose decay to the next segment start
// is below 2^-kSkipLog2 is neither computed nor added (its contribution is
// below fp32 resolution by a factor of more than 2^40).
//
// fp32 forward.  The chunked recursion evaluated with fp32 FMAs on the vector
// units, one workgroup per (b, h), chunks of at most 64 (d <= 64) or 32
// (d = 128) rows so that Q, K, V, the scores and the d x d state fit in LDS.
#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {

__global__ __launch_bounds__(256) void scan_kernel(ScanPass p, const SeqTable st) {
  // grid: rows x (D*D/4/256 blocks); each thread owns one float4 of the state
  const int D = p.D;
  if (blockIdx.x == 0 && threadIdx.x < kTagWords) p.tag[threadIdx.x] = p.tag_value.w[threadIdx.x];
  const int per_head = D * D / 4;
  const int r_idx = blockIdx.x / ((per_head + 255) / 256);
  const int e4 = (blockIdx.x % ((per_head + 255) / 256)) * 256 + threadIdx.x;
  if (e4 >= per_head) return;
  const int ppseg = p.seg_len / p.piece_len;
  const Row row = st.nseq > 0 ? packed_row(st, r_idx / p.H, r_idx % p.H, p.H, p.G, ppseg)
                              : uniform_row(r_idx, p.H, p.N, p.nseg, p.npiece);
  if (row.nseg < 2) return;
  const float sl2 = p.slope[row.h] * kLog2e;
  const size_t dd = (size_t)D * D;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  if (p.state_in) s = reinterpret_cast<const f32x4_t*>(p.state_in + row.st * dd)[e4];
  const float gL = exp2f(-sl2 * (float)p.seg_len);
  // Every segment but the last is full, so the pieces that segment r-1
  // contributes to the start of segment r are the same ranks for every r:
  // rank k (k pieces between it and the segment end) is at distance k * Lp,
  // and it was computed iff lambda^(k Lp) >= 2^-kSkipLog2 (the test the piece
  // kernel makes, in the same arithmetic).
  int nneed = 0;
  while (nneed < ppseg && !(sl2 * (float)(nneed * p.piece_len) >= kSkipLog2)) ++nneed;
  const f32x4_t* pc4 = reinterpret_cast<const f32x4_t*>(p.pieces + (size_t)row.piecebase * dd);
  // entry 0: the row's initial state, read by its first segment
  reinterpret_cast<f32x4_t*>(p.seg_states + (size_t)row.segbase * dd)[e4] = s;
  for (int r = 1; r < row.nseg; ++r) {
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] *= gL;
    const int last = r * ppseg - 1;  // piece of rank 0
    for (int k0 = 0; k0 < nneed; k0 += 8) {
      // eight independent loads in flight, then the weighted sum
      f32x4_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = k0 + j < nneed ? pc4[(size_t)(last - k0 - j) * (dd / 4) + e4]
                              : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float f = exp2f(-sl2 * (float)((k0 + j) * p.piece_len));
#pragma unroll
        for (int c = 0; c < 4; ++c) s[c] = fmaf(f, v[j][c], s[c]);
      }
    }
    reinterpret_cast<f32x4_t*>(p.seg_states + ((size_t)row.segbase + r) * dd)[e4] = s;
  }
}

// EPI: the output epilogue (per-head RMSNorm, per-channel weight, sigmoid
// gate) on each block's fp32 output rows, staged in LDS, before the store.
template <int D, int CS, bool EPI>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdPass p, const SeqTable st) {
  constexpr int DS = D + 1;  // padded row stride
  __shared__ float Sm[D * D];
  __shared__ float Qm[CS * DS], Km[CS * DS], Vm[CS * DS];
  __shared__ float Pm[CS * (CS + 1)];
  __shared__ float bj[CS];
  __shared__ float Om[EPI ? CS * DS : 1], rn[EPI ? CS : 1];
  const int tid = threadIdx.x;
  // one (sequence, head) row per workgroup
  const Row row = st.nseq > 0 ? packed_row(st, blockIdx.x / p.H, blockIdx.x % p.H, p.H, 0, 0)
                              : uniform_row(blockIdx.x, p.H, p.N, 1, 0);
  const int N = row.len;
  const float sl2 = p.slope[row.h] * kLog2e;
  const size_t head_off = row.tok * D;
  const float* qg = (const float*)p.q + head_off;
  const float* kg = (const float*)p.k + head_off;
  const float* vg = (const float*)p.v + head_off;
  float* og = (float*)p.o + head_off;
  for (int e = tid; e < D * D; e += 256)
    Sm[e] = p.state_in ? p.state_in[(size_t)row.st * D * D + e] : 0.f;
  auto tok = [&](int tau) { return p.reverse ? (N - 1 - tau) : tau; };
  for (int t0 = 0; t0 < N; t0 += CS) {
    const int n = min(CS, N - t0);
    __syncthreads();
    for (int e = tid; e < CS * D; e += 256) {
      const int r = e / D, c = e % D;
      const bool ok = r < n;
      const size_t g = ok ? (size_t)tok(t0 + r) * D + c : 0;
      Qm[r * DS + c] = ok ? qg[g] : 0.f;
      Km[r * DS + c] = ok ? kg[g] : 0.f;
      Vm[r * DS + c] = ok ? vg[g] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < CS * CS; e += 256) {
      const int i = e / CS, j = e % CS;
      float acc = 0.f;
      if (j <= i) {
        for (int x = 0; x < D; ++x) acc = fmaf(Qm[i * DS + x], Km[j * DS + x], acc);
        acc *= exp2f(-sl2 * (float)(i - j));
      }
      Pm[i * (CS + 1) + j] = acc;
    }
    __syncthreads();
    for (int e = tid; e < CS * D; e += 256) {
      const int i = e / D, c = e % D;
      if (i >= n) continue;
      float intra = 0.f, inter = 0.f;
      for (int j = 0; j <= i; ++j) intra = fmaf(Pm[i * (CS + 1) + j], Vm[j * DS + c], intra);
      for (int x = 0; x < D; ++x) inter = fmaf(Qm[i * DS + x], Sm[x * D + c], inter);
      const float out = intra + exp2f(-sl2 * (float)(i + 1)) * inter;
      if constexpr (EPI)
        Om[i * DS + c] = out;
      else
        og[(size_t)tok(t0 + i) * D + c] = out;
    }
    __syncthreads();
    if constexpr (EPI) {
      const float* gt = (const float*)p.gate + head_off;
      if (tid < n) {
        float ss = 0.f;
        for (int c = 0; c < D; ++c) ss = fmaf(Om[tid * DS + c], Om[tid * DS + c], ss);
        rn[tid] = 1.f / sqrtf(ss / (float)D + p.eps);
      }
      __syncthreads();
      for (int e = tid; e < CS * D; e += 256) {
        const int i = e / D, c = e % D;
        if (i >= n) continue;
        const size_t g = (size_t)tok(t0 + i) * D + c;
        const float sig = 1.f / (1.f + expf(-gt[g]));
        og[g] = Om[i * DS + c] * rn[i] * p.norm_w[(size_t)row.h * D + c] * sig;
      }
    }
    const float g = exp2f(-sl2 * (float)n);
    if (tid < CS) bj[tid] = tid < n ? exp2f(-sl2 * (float)(n - 1 - tid)) : 0.f;
    __syncthreads();
    for (int e = tid; e < D * D; e += 256) {
      const int x = e / D, c = e % D;
      float acc = 0.f;
      for (int j = 0; j < n; ++j) acc = fmaf(bj[j] * Km[j * DS + x], Vm[j * DS + c], acc);
      Sm[e] = fmaf(g, Sm[e], acc);
    }
  }
  __syncthreads();
  if (p.state_out)
    for (int e = tid; e < D * D; e += 256) p.state_out[(size_t)row.st * D * D + e] = Sm[e];
}

template <int D, int CS>
hipError_t launch_f32(const FwdPass& p, const SeqTable& t, hipStream_t s) {
  const unsigned grid = (unsigned)((t.nseq > 0 ? t.nseq : p.B) * p.H);
  if (p.gate)
    hipLaunchKernelGGL((fwd_f32_kernel<D, CS, true>), dim3(grid), dim3(256), 0, s, p, t);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, CS, false>), dim3(grid), dim3(256), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const ScanPass& p, const SeqTable& t, hipStream_t s) {
  const int per_head = p.D * p.D / 4;
  const unsigned grid = (unsigned)((t.nseq > 0 ? t.nseq : p.B) * p.H * ((per_head + 255) / 256));
  hipLaunchKernelGGL(scan_kernel, dim3(grid), dim3(256), 0, s, p, t);
  return hipGetLastError();
}

// Chunks are evaluated in blocks of at most min(C, 64) rows (32 for d = 128);
// the result does not depend on the blocking beyond rounding.
hipError_t launch_fwd_f32(const FwdPass& p, const SeqTable& t, hipStream_t s) {
  const int cs = p.C;
  switch (p.D) {
    case 16: return cs >= 64 ? launch_f32<16, 64>(p, t, s) : cs >= 32 ? launch_f32<16, 32>(p, t, s) : launch_f32<16, 16>(p, t, s);
    case 32: return cs >= 64 ? launch_f32<32, 64>(p, t, s) : cs >= 32 ? launch_f32<32, 32>(p, t, s) : launch_f32<32, 16>(p, t, s);
    case 64: return cs >= 64 ? launch_f32<64, 64>(p, t, s) : cs >= 32 ? launch_f32<64, 32>(p, t, s) : launch_f32<64, 16>(p, t, s);
    case 128: return cs >= 32 ? launch_f32<128, 32>(p, t, s) : launch_f32<128, 16>(p, t, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
