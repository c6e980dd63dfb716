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
// below the fp32 resolution of the sum, which holds the segment's last,
// undecayed piece as well).
//
// fp32 forward.  The chunked recursion evaluated with fp32 FMAs on the vector
// units, one workgroup per (row, slice of value columns); see fwd_f32_kernel.
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

// fp32 forward, one workgroup per (row, slice of W value columns): the
// outputs and state of a column depend on all keys but only on that column of
// V, so the columns split across workgroups with no exchange; the masked
// scores of a block are recomputed by each slice (W = D for the epilogue,
// whose norm needs whole rows).  Per block of CS <= C rows:
//   P = (Q K^T) * M                        (CS x CS, 4 x 4 / 2 x 2 / 1 x 1 register tiles)
//   O[:, cols] = P V[:, cols] + diag(a) Q S[:, cols]
//   S[:, cols] = lambda^n S[:, cols] + K^T diag(b) V[:, cols]
// Each thread keeps its rows x 4 columns of the state slice in registers; a
// copy in LDS serves the block's inter-block products.  All LDS reads are
// 16-byte vectors along the contraction (rows padded by 4 floats).
template <int D, int CS, int W, bool EPI>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdPass p, const SeqTable st) {
  static_assert(CS == 16 || CS == 32 || CS == 64, "block rows");
  constexpr int DP = D + 4;             // padded row of Q and K
  constexpr int WP = W + 4;             // padded row of V and of the state slice
  constexpr int CP = CS + 4;            // padded row of P
  constexpr int TC = W / 4;             // float4 column groups of the slice
  constexpr int RG = 256 / TC;          // row groups (outputs and state)
  constexpr int OR = CS / RG > 0 ? CS / RG : 1;  // output rows per thread
  constexpr int SR = D / RG > 0 ? D / RG : 1;    // state rows per thread
  constexpr int PB = CS / 16;           // score tile per thread: PB x PB
  static_assert(RG * OR >= CS || RG >= CS, "output rows");
  __shared__ __attribute__((aligned(16))) float Qm[CS * DP], Km[CS * DP], Vm[CS * WP];
  __shared__ __attribute__((aligned(16))) float Pm[CS * CP], Sm[D * WP];
  __shared__ float bj[CS];
  __shared__ float ssq[EPI ? CS : 1][EPI ? TC : 1];
  const int tid = threadIdx.x;
  constexpr int SPLIT = D / W;
  const int r_idx = blockIdx.x / SPLIT;
  const int c0 = (blockIdx.x % SPLIT) * W;  // first value column of the slice
  const Row row = st.nseq > 0 ? packed_row(st, r_idx / p.H, r_idx % p.H, p.H, 0, 0)
                              : uniform_row(r_idx, p.H, p.N, 1, 0);
  const int N = row.len;
  const float sl2 = p.slope[row.h] * kLog2e;
  const size_t head_off = row.tok * D;
  const float* qg = (const float*)p.q + head_off;
  const float* kg = (const float*)p.k + head_off;
  const float* vg = (const float*)p.v + head_off;
  float* og = (float*)p.o + head_off;
  auto tok = [&](int tau) { return p.reverse ? (N - 1 - tau) : tau; };

  // this thread's outputs: rows orow(m) = rg + RG m, columns 4 cg .. +3 of
  // the slice; its state: rows srow(m) = rg + RG m, same columns
  const int cg = tid % TC, rg = tid / TC;
  f32x4_t sv[SR];
#pragma unroll
  for (int m = 0; m < SR; ++m) {
    const int x = rg + RG * m;
    sv[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (p.state_in && x < D)
      sv[m] = *reinterpret_cast<const f32x4_t*>(p.state_in + (size_t)row.st * D * D +
                                                (size_t)x * D + c0 + 4 * cg);
    if (x < D) *reinterpret_cast<f32x4_t*>(Sm + x * WP + 4 * cg) = sv[m];
  }
  // score tile of this thread: rows PB (tid / 16) .., columns PB (tid % 16) ..
  const int pi0 = PB * (tid >> 4), pj0 = PB * (tid & 15);

  // Q, K (all features) and V (the slice) of a block move global ->
  // registers -> LDS; the next block's loads are issued as soon as the
  // current block is in LDS, so they are in flight during its arithmetic.
  constexpr int QK_IT = (CS * (D / 4) + 255) / 256;  // float4 per thread
  constexpr int V_IT = (CS * TC + 255) / 256;
  f32x4_t qr[QK_IT], kr[QK_IT], vr[V_IT];
  auto fetch = [&](int t0) {
    const int n = min(CS, N - t0);
#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
      const int e = tid + 256 * it, r = e / (D / 4), c4 = e % (D / 4);
      qr[it] = kr[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (e < CS * (D / 4) && r < n) {
        const size_t g = (size_t)tok(t0 + r) * D + 4 * c4;
        qr[it] = *reinterpret_cast<const f32x4_t*>(qg + g);
        kr[it] = *reinterpret_cast<const f32x4_t*>(kg + g);
      }
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
      const int e = tid + 256 * it, r = e / TC, c4 = e % TC;
      vr[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (e < CS * TC && r < n)
        vr[it] = *reinterpret_cast<const f32x4_t*>(vg + (size_t)tok(t0 + r) * D + c0 + 4 * c4);
    }
  };
  if (N > 0) fetch(0);

  for (int t0 = 0; t0 < N; t0 += CS) {
    const int n = min(CS, N - t0);
    __syncthreads();  // the previous block is done with Q, K, V, P and S
    // ---- stage this block's Q, K, V; start the next block's loads ----
#pragma unroll
    for (int it = 0; it < QK_IT; ++it) {
      const int e = tid + 256 * it, r = e / (D / 4), c4 = e % (D / 4);
      if (e < CS * (D / 4)) {
        *reinterpret_cast<f32x4_t*>(Qm + r * DP + 4 * c4) = qr[it];
        *reinterpret_cast<f32x4_t*>(Km + r * DP + 4 * c4) = kr[it];
      }
    }
#pragma unroll
    for (int it = 0; it < V_IT; ++it) {
      const int e = tid + 256 * it, r = e / TC, c4 = e % TC;
      if (e < CS * TC) *reinterpret_cast<f32x4_t*>(Vm + r * WP + 4 * c4) = vr[it];
    }
    if (t0 + CS < N) fetch(t0 + CS);
    if (tid < CS) bj[tid] = tid < n ? exp2f(-sl2 * (float)(n - 1 - tid)) : 0.f;
    __syncthreads();
    // ---- scores ----
    {
      float acc[PB][PB];
#pragma unroll
      for (int a = 0; a < PB; ++a)
#pragma unroll
        for (int b = 0; b < PB; ++b) acc[a][b] = 0.f;
#pragma unroll 2
      for (int x = 0; x < D; x += 4) {
        f32x4_t qa[PB], kb[PB];
#pragma unroll
        for (int a = 0; a < PB; ++a) qa[a] = *reinterpret_cast<const f32x4_t*>(Qm + (pi0 + a) * DP + x);
#pragma unroll
        for (int b = 0; b < PB; ++b) kb[b] = *reinterpret_cast<const f32x4_t*>(Km + (pj0 + b) * DP + x);
#pragma unroll
        for (int a = 0; a < PB; ++a)
#pragma unroll
          for (int b = 0; b < PB; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[a][b] = fmaf(qa[a][e], kb[b][e], acc[a][b]);
      }
#pragma unroll
      for (int a = 0; a < PB; ++a)
#pragma unroll
        for (int b = 0; b < PB; ++b) {
          const int i = pi0 + a, j = pj0 + b;
          Pm[i * CP + j] = j <= i ? acc[a][b] * exp2f(-sl2 * (float)(i - j)) : 0.f;
        }
    }
    __syncthreads();
    // ---- outputs of the slice ----
    f32x4_t ov[OR];
#pragma unroll
    for (int m = 0; m < OR; ++m) {
      const int i = rg + RG * m;
      f32x4_t intra = {0.f, 0.f, 0.f, 0.f}, inter = intra;
      if (i < CS) {
#pragma unroll 2
        for (int j = 0; j <= i; j += 4) {
          const f32x4_t pr = *reinterpret_cast<const f32x4_t*>(Pm + i * CP + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(Vm + (j + e) * WP + 4 * cg);
#pragma unroll
            for (int c = 0; c < 4; ++c) intra[c] = fmaf(pr[e], vv[c], intra[c]);
          }
        }
#pragma unroll 2
        for (int x = 0; x < D; x += 4) {
          const f32x4_t qr = *reinterpret_cast<const f32x4_t*>(Qm + i * DP + x);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x4_t sr = *reinterpret_cast<const f32x4_t*>(Sm + (x + e) * WP + 4 * cg);
#pragma unroll
            for (int c = 0; c < 4; ++c) inter[c] = fmaf(qr[e], sr[c], inter[c]);
          }
        }
      }
      const float a_i = exp2f(-sl2 * (float)(i + 1));
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[m][c] = fmaf(a_i, inter[c], intra[c]);
    }
    if constexpr (EPI) {
      // W == D: the row's TC column groups are TC consecutive threads
#pragma unroll
      for (int m = 0; m < OR; ++m) {
        const int i = rg + RG * m;
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) ss = fmaf(ov[m][c], ov[m][c], ss);
        if (i < CS) ssq[i][cg] = ss;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < OR; ++m) {
        const int i = rg + RG * m;
        if (i >= n) continue;
        float tot = 0.f;
        for (int g = 0; g < TC; ++g) tot += ssq[i][g];
        const float rn = 1.f / sqrtf(tot / (float)D + p.eps);
        const size_t g0 = (size_t)tok(t0 + i) * D + c0 + 4 * cg;
        const f32x4_t gt = *reinterpret_cast<const f32x4_t*>((const float*)p.gate + head_off + g0);
        f32x4_t y;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          y[c] = ov[m][c] * rn * p.norm_w[(size_t)row.h * D + c0 + 4 * cg + c] *
                 (1.f / (1.f + expf(-gt[c])));
        *reinterpret_cast<f32x4_t*>(og + g0) = y;
      }
    } else {
#pragma unroll
      for (int m = 0; m < OR; ++m) {
        const int i = rg + RG * m;
        if (i < n) *reinterpret_cast<f32x4_t*>(og + (size_t)tok(t0 + i) * D + c0 + 4 * cg) = ov[m];
      }
    }
    __syncthreads();  // every thread is done reading Sm
    // ---- state slice: S = lambda^n S + K^T diag(b) V ----
    const float gdec = exp2f(-sl2 * (float)n);
#pragma unroll
    for (int m = 0; m < SR; ++m) {
      const int x = rg + RG * m;
      if (x >= D) continue;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int j = 0; j < n; ++j) {
        const float bk = bj[j] * Km[j * DP + x];
        const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(Vm + j * WP + 4 * cg);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(bk, vv[c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) sv[m][c] = fmaf(gdec, sv[m][c], acc[c]);
      *reinterpret_cast<f32x4_t*>(Sm + x * WP + 4 * cg) = sv[m];
    }
  }
  if (p.state_out) {
#pragma unroll
    for (int m = 0; m < SR; ++m) {
      const int x = rg + RG * m;
      if (x < D)
        *reinterpret_cast<f32x4_t*>(p.state_out + (size_t)row.st * D * D + (size_t)x * D + c0 +
                                    4 * cg) = sv[m];
    }
  }
}

// fp32 forward of short rows in the parallel form: the same causal sum,
//
//   o_i = sum_{j <= i} lambda^(i-j) (q_i . k_j) v_j + lambda^(i+1) q_i^T S0,
//   S_N = lambda^N S0 + sum_t lambda^(N-1-t) k_t v_t^T,
//
// evaluated without the chunk recursion ("Hybrid Linear Attention": the
// intra-block part of Lightning Attention is exactly this masked product).
// The chunked kernel walks a row's chunks in sequence, so a short row costs
// a few chunk latencies on a nearly idle GPU; here every block of QB query
// rows and every block of QB state rows is its own workgroup, and the
// longest dependency chain is one query block's pass over the keys in steps
// of KB.  At d <= 64 a workgroup is two halves of 256 threads that take the
// steps alternately, each with its own K, V and score buffers, and add their
// partial sums in a fixed order at the end (the chain is half as long, the
// result stays bitwise reproducible); at d = 128 the buffers of a second
// half do not fit the LDS beside S0, and one half takes every step.  Its
// work grows as N^2, so it serves rows of at most kQuadMaxN tokens.  Grid:
// rows x (ceil(N / QB) query blocks + D / QB state blocks when the state is
// written).
constexpr int kQuadQB = 16, kQuadKB = 64;
template <int D>
constexpr int quad_halves() { return D <= 64 ? 2 : 1; }
template <int D>
__global__ __launch_bounds__(256 * quad_halves<D>()) void fwd_f32_quad_kernel(FwdPass p, int nqb,
                                                                             int nblk) {
  constexpr int QB = kQuadQB, KB = kQuadKB, NH = quad_halves<D>();
  constexpr int DP = D + 4;       // padded rows of Q, K, V and S0
  constexpr int CG = D / 4;       // float4 column groups of a row
  constexpr int PAIRS = QB * CG;  // (row, column group) outputs of a block
  constexpr int NP = (PAIRS + 255) / 256;  // of them per thread of a half
  constexpr int TV = KB * CG / 256;        // float4 of a KB-row tile per thread
  static_assert(D % 16 == 0 && TV >= 1, "head dim");
  // per half: K, V (or, for state blocks, K columns as [KB][QB]), scores, b
  __shared__ __attribute__((aligned(16))) float Qs[QB * DP], Ks[NH][KB * DP], Vs[NH][KB * DP],
      Ps[NH][QB * (KB + 4)], bt[NH][KB], Ss[D * DP];
  const int hf = threadIdx.x / 256, tid = threadIdx.x % 256;  // half, thread in the half
  const int r_idx = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int N = p.N, h = r_idx % p.H;
  const float sl2 = p.slope[h] * kLog2e;
  const size_t head_off = (size_t)r_idx * N * D;
  const float* qg = (const float*)p.q + head_off;
  const float* kg = (const float*)p.k + head_off;
  const float* vg = (const float*)p.v + head_off;
  const float* S0 = p.state_in ? p.state_in + (size_t)r_idx * D * D : nullptr;
  // rows r0 .. r0 + KB - 1 of a token tensor (zero past N), TV float4 per
  // thread: fetched into registers one step ahead, then put into LDS
  f32x4_t kr[TV], vr[TV];
  auto fetch = [&](f32x4_t (&x)[TV], const float* src, int r0) {
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + 256 * u, r = e / CG, c4 = e % CG;
      x[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (r0 + r < N) x[u] = *reinterpret_cast<const f32x4_t*>(src + (size_t)(r0 + r) * D + 4 * c4);
    }
  };
  auto put = [&](float* dst, const f32x4_t (&x)[TV]) {
#pragma unroll
    for (int u = 0; u < TV; ++u) {
      const int e = tid + 256 * u;
      *reinterpret_cast<f32x4_t*>(dst + (e / CG) * DP + 4 * (e % CG)) = x[u];
    }
  };
  // the halves' partial sums meet in half 0 through half 1's K buffer
  float* part = Ks[NH - 1];
  f32x4_t acc[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (blk < nqb) {
    // ---- query rows i0 .. i0 + QB - 1 -------------------------------------
    const int i0 = QB * blk;
    const int kend = min(N, i0 + QB);  // keys 0 .. kend - 1 reach the block
    const int nsteps = (kend + KB - 1) / KB;
    if (hf < nsteps) {
      fetch(kr, kg, KB * hf);
      fetch(vr, vg, KB * hf);
    }
    for (int e = threadIdx.x; e < QB * CG; e += 256 * NH) {
      const int r = e / CG, c4 = e % CG;
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
      if (i0 + r < N) x = *reinterpret_cast<const f32x4_t*>(qg + (size_t)(i0 + r) * D + 4 * c4);
      *reinterpret_cast<f32x4_t*>(Qs + r * DP + 4 * c4) = x;
    }
    if (S0) {
      for (int e = threadIdx.x; e < D * CG; e += 256 * NH) {
        const int r = e / CG, c4 = e % CG;
        *reinterpret_cast<f32x4_t*>(Ss + r * DP + 4 * c4) =
            *reinterpret_cast<const f32x4_t*>(S0 + (size_t)r * D + 4 * c4);
      }
    }
    // score entries of this thread: query row i0 + si, keys sj + 16 m
    const int si = tid / 16, sj = tid % 16;
    float* Kh = Ks[hf];
    float* Vh = Vs[hf];
    float* Ph = Ps[hf];
    // every thread runs the same number of rounds (barriers); in round it,
    // half hf takes step NH it + hf when it exists
    for (int it = 0; it * NH < nsteps; ++it) {
      const int st = NH * it + hf;
      const bool mine = st < nsteps;
      const int j0 = KB * st;
      __syncthreads();  // the previous round is done with this half's buffers
      if (mine) {
        put(Kh, kr);
        put(Vh, vr);
        if (st + NH < nsteps) {  // this half's next step loads during this one
          fetch(kr, kg, j0 + KB * NH);
          fetch(vr, vg, j0 + KB * NH);
        }
      }
      __syncthreads();
      if (mine) {
        // masked, decayed scores P[si][sj + 16 m]
        float sc[KB / 16];
#pragma unroll
        for (int m = 0; m < KB / 16; ++m) sc[m] = 0.f;
#pragma unroll 4
        for (int f = 0; f < D; f += 4) {
          const f32x4_t qa = *reinterpret_cast<const f32x4_t*>(Qs + si * DP + f);
#pragma unroll
          for (int m = 0; m < KB / 16; ++m) {
            const f32x4_t kb = *reinterpret_cast<const f32x4_t*>(Kh + (sj + 16 * m) * DP + f);
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[m] = fmaf(qa[e], kb[e], sc[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < KB / 16; ++m) {
          const int i = i0 + si, j = j0 + sj + 16 * m;
          Ph[si * (KB + 4) + sj + 16 * m] = j <= i ? sc[m] * exp2f(-sl2 * (float)(i - j)) : 0.f;
        }
      }
      __syncthreads();
      if (mine) {
        // o[i][4 cg ..] += sum_j P[i][j] V[j][4 cg ..]
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          const int e = tid + 256 * u;
          if (e < PAIRS) {
            const int i = e / CG, cg = e % CG;
#pragma unroll 4
            for (int j = 0; j < KB; j += 4) {
              const f32x4_t pr = *reinterpret_cast<const f32x4_t*>(Ph + i * (KB + 4) + j);
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(Vh + (j + x) * DP + 4 * cg);
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[u][c] = fmaf(pr[x], vv[c], acc[u][c]);
              }
            }
          }
        }
      }
    }
    // + lambda^(i+1) q_i^T S0 (S0 in LDS since the first round), by the last
    // half; then the halves' sums are added in half 0 and stored
    if (S0 && hf == NH - 1) {
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int e = tid + 256 * u;
        if (e >= PAIRS) continue;
        const int i = e / CG, cg = e % CG;
        f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int f = 0; f < D; f += 4) {
          const f32x4_t qa = *reinterpret_cast<const f32x4_t*>(Qs + i * DP + f);
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            const f32x4_t srow = *reinterpret_cast<const f32x4_t*>(Ss + (f + y) * DP + 4 * cg);
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = fmaf(qa[y], srow[c], x[c]);
          }
        }
        const float a = exp2f(-sl2 * (float)(i0 + i + 1));
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[u][c] = fmaf(a, x[c], acc[u][c]);
      }
    }
    if constexpr (NH == 2) {
      __syncthreads();  // every half is done with its buffers
      if (hf == 1) {
#pragma unroll
        for (int u = 0; u < NP; ++u)
          *reinterpret_cast<f32x4_t*>(part + 4 * (tid + 256 * u)) = acc[u];
      }
      __syncthreads();
    }
    if (hf == 0) {
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int e = tid + 256 * u;
        if (e >= PAIRS) continue;
        const int i = e / CG, cg = e % CG;
        if (i0 + i >= N) continue;
        f32x4_t y = acc[u];
        if constexpr (NH == 2) {
          const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(part + 4 * e);
#pragma unroll
          for (int c = 0; c < 4; ++c) y[c] += o1[c];
        }
        *reinterpret_cast<f32x4_t*>((float*)p.o + head_off + (size_t)(i0 + i) * D + 4 * cg) = y;
      }
    }
  } else {
    // ---- state rows f0 .. f0 + QB - 1 of S_N ------------------------------
    const int f0 = QB * (blk - nqb);
    const int nsteps = (N + KB - 1) / KB;
    // K columns f0 .. f0 + QB - 1 of KB tokens: one float4 per thread
    static_assert(KB * (QB / 4) == 256, "one K float4 per thread");
    const int kr_r = tid / (QB / 4), kr_c = tid % (QB / 4);
    auto fetch_k = [&](int t0) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
      if (t0 + kr_r < N)
        x = *reinterpret_cast<const f32x4_t*>(kg + (size_t)(t0 + kr_r) * D + f0 + 4 * kr_c);
      return x;
    };
    f32x4_t kc = {0.f, 0.f, 0.f, 0.f};
    if (hf < nsteps) {
      kc = fetch_k(KB * hf);
      fetch(vr, vg, KB * hf);
    }
    if (S0 && hf == 0) {
      const float gN = exp2f(-sl2 * (float)N);
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int e = tid + 256 * u;
        if (e < PAIRS) {
          const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(S0 + (size_t)(f0 + e / CG) * D +
                                                               4 * (e % CG));
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[u][c] = gN * s0[c];
        }
      }
    }
    float* Kh = Ks[hf];
    float* Vh = Vs[hf];
    float* bh = bt[hf];
    for (int it = 0; it * NH < nsteps; ++it) {
      const int st = NH * it + hf;
      const bool mine = st < nsteps;
      const int t0 = KB * st;
      __syncthreads();  // the previous round is done with this half's buffers
      if (mine) {
        *reinterpret_cast<f32x4_t*>(Kh + kr_r * QB + 4 * kr_c) = kc;  // Kh as [KB][QB]
        put(Vh, vr);
        if (tid < KB) bh[tid] = t0 + tid < N ? exp2f(-sl2 * (float)(N - 1 - t0 - tid)) : 0.f;
        if (st + NH < nsteps) {
          kc = fetch_k(t0 + KB * NH);
          fetch(vr, vg, t0 + KB * NH);
        }
      }
      __syncthreads();
      if (mine) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
          const int e = tid + 256 * u;
          if (e < PAIRS) {
            const int fl = e / CG, cg = e % CG;
#pragma unroll 8
            for (int t = 0; t < KB; ++t) {
              const float w = bh[t] * Kh[t * QB + fl];
              const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(Vh + t * DP + 4 * cg);
#pragma unroll
              for (int c = 0; c < 4; ++c) acc[u][c] = fmaf(w, vv[c], acc[u][c]);
            }
          }
        }
      }
    }
    if constexpr (NH == 2) {
      __syncthreads();
      if (hf == 1) {
#pragma unroll
        for (int u = 0; u < NP; ++u)
          *reinterpret_cast<f32x4_t*>(part + 4 * (tid + 256 * u)) = acc[u];
      }
      __syncthreads();
    }
    if (hf == 0) {
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int e = tid + 256 * u;
        if (e >= PAIRS) continue;
        f32x4_t y = acc[u];
        if constexpr (NH == 2) {
          const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(part + 4 * e);
#pragma unroll
          for (int c = 0; c < 4; ++c) y[c] += s1[c];
        }
        *reinterpret_cast<f32x4_t*>(p.state_out + (size_t)r_idx * D * D +
                                    (size_t)(f0 + e / CG) * D + 4 * (e % CG)) = y;
      }
    }
  }
}

template <int D>
hipError_t launch_f32_quad(const FwdPass& p, hipStream_t s) {
  const int nqb = (p.N + kQuadQB - 1) / kQuadQB;
  const int nblk = nqb + (p.state_out ? D / kQuadQB : 0);
  const unsigned grid = (unsigned)(p.B * p.H * nblk);
  hipLaunchKernelGGL((fwd_f32_quad_kernel<D>), dim3(grid), dim3(256 * quad_halves<D>()), 0, s, p,
                     nqb, nblk);
  return hipGetLastError();
}

template <int D, int CS>
hipError_t launch_f32(const FwdPass& p, const SeqTable& t, hipStream_t s) {
  const unsigned rows = (unsigned)((t.nseq > 0 ? t.nseq : p.B) * p.H);
  constexpr int W = D < 16 ? D : 16;
  // the epilogue keeps whole rows (W = D): at d = 128, blocks of 32 rows fit
  // the LDS
  constexpr int CSE = D == 128 && CS > 32 ? 32 : CS;
  if (p.gate)
    hipLaunchKernelGGL((fwd_f32_kernel<D, CSE, D, true>), dim3(rows), dim3(256), 0, s, p, t);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, CS, W, false>), dim3(rows * (D / W)), dim3(256), 0, s,
                       p, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const ScanPass& p, const SeqTable& t, hipStream_t s) {
  const int per_head = p.D * p.D / 4;
  const unsigned grid = (unsigned)((t.nseq > 0 ? t.nseq : p.B) * p.H * ((per_head + 255) / 256));
  hipLaunchKernelGGL(scan_kernel, dim3(grid), dim3(256), 0, s, p, t);
  return hipGetLastError();
}

// Chunks are evaluated in blocks of min(C, 64) rows; the result does not
// depend on the blocking beyond rounding.
hipError_t launch_fwd_f32(const FwdPass& p, const SeqTable& t, hipStream_t s) {
  // Short forward rows of the uniform layout take the parallel form (its
  // output workgroups read every state row, so an in-place continuation,
  // state_out == state_in, keeps the chunked kernel, whose workgroups read
  // and write disjoint column slices).
  if (!p.reverse && !p.gate && t.nseq == 0 && p.N <= kQuadMaxN &&
      !(p.state_in && p.state_in == p.state_out)) {
    switch (p.D) {
      case 16: return launch_f32_quad<16>(p, s);
      case 32: return launch_f32_quad<32>(p, s);
      case 64: return launch_f32_quad<64>(p, s);
      case 128: return launch_f32_quad<128>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int cs = p.C;
  switch (p.D) {
    case 16: return cs >= 64 ? launch_f32<16, 64>(p, t, s) : cs >= 32 ? launch_f32<16, 32>(p, t, s) : launch_f32<16, 16>(p, t, s);
    case 32: return cs >= 64 ? launch_f32<32, 64>(p, t, s) : cs >= 32 ? launch_f32<32, 32>(p, t, s) : launch_f32<32, 16>(p, t, s);
    case 64: return cs >= 64 ? launch_f32<64, 64>(p, t, s) : cs >= 32 ? launch_f32<64, 32>(p, t, s) : launch_f32<64, 16>(p, t, s);
    case 128: return cs >= 64 ? launch_f32<128, 64>(p, t, s) : cs >= 32 ? launch_f32<128, 32>(p, t, s) : launch_f32<128, 16>(p, t, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
