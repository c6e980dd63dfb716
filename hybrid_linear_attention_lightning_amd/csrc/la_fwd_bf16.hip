// la_fwd_bf16.hip -- chunked Lightning Attention forward on bf16 MFMA (gfx950).
//
// Computes, per (b, h) and per segment of the sequence, the chunked form of
// o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t^T S_in:
// for a chunk of n <= C tokens (local rows i, j) with carried d x d state S,
//
//     O   = ((Q K^T) * M) V + diag(a) Q S,   M[i][j] = lambda^(i-j) (j <= i)
//     S  <- lambda^n S + K^T diag(b) V,       a_i = lambda^(i+1), b_j = lambda^(n-1-j)
//
// This is the intra-chunk / inter-chunk split of the recursion that the Ling &
// Ring 2.6 pages describe for their context-parallel kernels ("Context Parallel
// for Lightning Attention": the state recursion unfolded into matrix form).
//
// Design (MI355X):
//  * one workgroup of 4 waves owns a whole head (all d value columns) over one
//    segment of the sequence, so Q K^T is computed once per chunk and every
//    operand is read from HBM once; parallelism beyond B*H comes from segments,
//    whose start states the piece and scan kernels assemble (the "local
//    recursion + global correction" algebra of the same section);
//  * each wave owns D/64 tiles of 16 value columns of the fp32 state, kept in
//    registers for the whole segment;
//  * the three operands that are not inputs -- the masked scores P, the state
//    S and b*V -- are handed to the matrix cores as bf16 hi + lo pairs, so the
//    products carry ~16 significant bits (plain bf16 operands would lose as
//    much accuracy as the final rounding of the output);
//  * Q and K are staged row-major in LDS, K and V also transposed (feature
//    rows) in "fragment order" (frag_pos), so MFMA results feed back as MFMA
//    operands without a transpose; the masked scores of a chunk are exchanged
//    through LDS in the region of K and K^T, which are dead by then.
// The same kernel in STATE_ONLY mode computes piece states (K^T diag(b) V
// accumulated over a piece) for the segment pre-pass.
#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 256;

__host__ __device__ constexpr int frag_base(int qb) {
  // number of 32-key P^T fragments that query blocks 0..qb-1 use (qb/2+1 each)
  return qb + ((qb & 1) ? (qb >> 1) * (qb >> 1) : (qb >> 1) * ((qb >> 1) - 1));
}

template <int C, int D, bool STATE_ONLY>
struct Cfg {
  static constexpr int NQB = C / 16;   // 16-token query / key blocks per chunk
  static constexpr int KSC = C / 32;   // 32-token contraction steps
  static constexpr int KSD = D / 32;   // 32-feature contraction steps
  static constexpr int NT = D / 16;    // 16-feature tiles (key and value side)
  static constexpr int WT = NT / 4;    // value tiles owned by each wave
  static constexpr int QS = D + 8;     // row stride (elements) of Qs / Ks
  static constexpr int TS = C + 8;     // row stride (elements) of Kt / Vt
  static constexpr int NFRAG = frag_base(NQB);
  static constexpr int MAXT = NQB == 8 ? 9 : NQB == 4 ? 4 : 2;  // P^T tiles per wave
  static constexpr int QCH = STATE_ONLY ? 0 : (C * D / 8 + kThreads - 1) / kThreads;
  static constexpr int NB = C * D / 64;  // 8x8 blocks per tensor
  static constexpr int KVB = (2 * NB + kThreads - 1) / kThreads;
  static constexpr int Q_ELEMS = STATE_ONLY ? 0 : C * QS;
  static constexpr int K_ELEMS = STATE_ONLY ? 0 : C * QS;
  static constexpr int T_ELEMS = D * TS;
  static constexpr int PT_HALF = NFRAG * 64 * 8;  // one of P_hi / P_lo
  // the P^T exchange reuses the space of K and K^T when it fits there
  static constexpr bool PT_ALIAS = STATE_ONLY || 2 * PT_HALF <= K_ELEMS + T_ELEMS;
  static constexpr int LDS_ELEMS = Q_ELEMS + K_ELEMS + 2 * T_ELEMS + (PT_ALIAS ? 0 : 2 * PT_HALF);
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(D == 64 || D == 128, "head dim");
};

// (key block, query block) of the m-th P^T tile of a wave; balanced so that
// every wave does the same number of 16x16 tiles when C = 128.
template <int NQB>
__device__ __forceinline__ bool tile_of(int wave, int m, int& kb, int& qb) {
  if constexpr (NQB == 8) {
    const int first = 8 - wave;  // tiles of query block 7-wave
    if (m < first) {
      kb = m;
      qb = 7 - wave;
    } else {
      kb = m - first;
      qb = wave;
    }
    return true;
  } else {
    qb = wave;
    kb = m;
    return wave < NQB && m <= wave;
  }
}

template <int C, int D, bool STATE_ONLY>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdPass p, PiecePass pp) {
  using G = Cfg<C, D, STATE_ONLY>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[G::LDS_ELEMS];
  uint16_t* Qs = smem;
  uint16_t* Ks = Qs + G::Q_ELEMS;
  uint16_t* Kt = Ks + G::K_ELEMS;
  uint16_t* Vt = Kt + G::T_ELEMS;
  // P^T hi / lo fragments, written after K and K^T are dead
  uint16_t* Pth = G::PT_ALIAS ? Ks : Vt + G::T_ELEMS;
  uint16_t* Ptl = Pth + G::PT_HALF;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;

  // ---- work item -------------------------------------------------------
  int b, h, tau0, tau_end, N;
  bool reverse;
  const float* slope;
  const uint16_t *qg = nullptr, *kg, *vg;
  uint16_t* og = nullptr;
  const float* s_init = nullptr;
  float* s_final = nullptr;
  if constexpr (STATE_ONLY) {
    const int piece = blockIdx.x % pp.npiece;
    const int bh = blockIdx.x / pp.npiece;
    h = bh % pp.H;
    b = bh / pp.H;
    N = pp.N;
    reverse = pp.reverse;
    slope = pp.slope;
    tau0 = piece * pp.piece_len;
    tau_end = min(N, tau0 + pp.piece_len);
    // needed only if the nearest segment start at or after the piece end is
    // a real segment start and the decay over the gap is not negligible
    const int r_star = (tau_end + pp.seg_len - 1) / pp.seg_len;
    if (r_star > pp.nseg - 1) return;
    const float gap = (float)(r_star * pp.seg_len - tau_end);
    if (slope[h] * kLog2e * gap >= kSkipLog2) return;
    const size_t head_off = ((size_t)b * pp.H + h) * (size_t)N * D;
    kg = (const uint16_t*)pp.k + head_off;
    vg = (const uint16_t*)pp.v + head_off;
    s_final = pp.pieces + ((size_t)bh * pp.npiece + piece) * D * D;
  } else {
    const int seg = blockIdx.x % p.nseg;
    const int bh = blockIdx.x / p.nseg;
    h = bh % p.H;
    b = bh / p.H;
    N = p.N;
    reverse = p.reverse;
    slope = p.slope;
    tau0 = seg * p.seg_len;
    tau_end = min(N, tau0 + p.seg_len);
    const size_t head_off = ((size_t)b * p.H + h) * (size_t)N * D;
    qg = (const uint16_t*)p.q + head_off;
    kg = (const uint16_t*)p.k + head_off;
    vg = (const uint16_t*)p.v + head_off;
    og = (uint16_t*)p.o + head_off;
    if (seg == 0)
      s_init = p.state_in ? p.state_in + (size_t)bh * D * D : nullptr;
    else
      s_init = p.seg_states + ((size_t)bh * p.nseg + seg) * D * D;
    if (seg == p.nseg - 1 && p.state_out) s_final = p.state_out + (size_t)bh * D * D;
  }
  const float sl2 = slope[h] * kLog2e;  // lambda^e = exp2(-sl2 * e)

  // ---- per-lane decay tables --------------------------------------------
  // P^T tile element: key row j = 16kb + 4lg + r, query column i = 16qb + li.
  // Diagonal tiles use md (zero above the diagonal); off-diagonal tiles use
  // lambda^(16 (qb-kb-1)) * mo[r], both factors <= 1 so nothing overflows.
  float md[4], mo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = li - 4 * lg - r;
    md[r] = e >= 0 ? exp2f(-sl2 * (float)e) : 0.f;
    mo[r] = exp2f(-sl2 * (float)(16 + e));
  }
  float aq[G::NQB];  // a_i for this lane's query column in each query block
#pragma unroll
  for (int qb = 0; qb < G::NQB; ++qb) aq[qb] = exp2f(-sl2 * (float)(16 * qb + li + 1));
  // Full chunk: b for the e-th token of a V fragment of step ks (token
  // 32ks + xl(e)) is lambda^(32 (KSC-1-ks)) * bl[e] with bl[e] = lambda^(31 - xl(e)).
  float bl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int xl = e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4;
    bl[e] = exp2f(-sl2 * (float)(31 - xl));
  }

  // ---- fp32 state: this wave's WT value tiles x NT key tiles ------------
  // S[wt][t][r] = S[key 16t + 4lg + r][value 16(wave*WT + wt) + li]
  f32x4_t S[G::WT][G::NT];
#pragma unroll
  for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
    for (int t = 0; t < G::NT; ++t) {
      const int col = 16 * (wave * G::WT + wt) + li;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[wt][t][r] = s_init ? s_init[(size_t)(16 * t + 4 * lg + r) * D + col] : 0.f;
    }

  // ---- staging registers ------------------------------------------------
  u32x4_t qr[G::QCH > 0 ? G::QCH : 1];
  u32x4_t kvr[G::KVB][8];
  auto tok = [&](int tau) { return reverse ? (N - 1 - tau) : tau; };

  auto load_chunk = [&](int tc, int n) {
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int m = 0; m < G::QCH; ++m) {
        const int id = tid + kThreads * m;
        const int row = id / (D / 8), c8 = id % (D / 8);
        qr[m] = (id < C * D / 8 && row < n)
                    ? *reinterpret_cast<const u32x4_t*>(qg + (size_t)tok(tc + row) * D + 8 * c8)
                    : u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int m = 0; m < G::KVB; ++m) {
      const int blk = tid + kThreads * m;
      const bool isk = blk < G::NB;
      const int bid = isk ? blk : blk - G::NB;
      const int cg = bid % (D / 8), tg = bid / (D / 8);
      const int tb = tg >> 2, g = tg & 3;
      const uint16_t* src = isk ? kg : vg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int x = 32 * tb + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
        kvr[m][e] = (blk < 2 * G::NB && x < n)
                        ? *reinterpret_cast<const u32x4_t*>(src + (size_t)tok(tc + x) * D + 8 * cg)
                        : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto store_chunk = [&]() {
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int m = 0; m < G::QCH; ++m) {
        const int id = tid + kThreads * m;
        if (id < C * D / 8) {
          const int row = id / (D / 8), c8 = id % (D / 8);
          *reinterpret_cast<u32x4_t*>(Qs + row * G::QS + 8 * c8) = qr[m];
        }
      }
    }
#pragma unroll
    for (int m = 0; m < G::KVB; ++m) {
      const int blk = tid + kThreads * m;
      if (blk < 2 * G::NB) {
        const bool isk = blk < G::NB;
        const int bid = isk ? blk : blk - G::NB;
        const int cg = bid % (D / 8), tg = bid / (D / 8);
        const int tb = tg >> 2, g = tg & 3;
        if constexpr (!STATE_ONLY) {
          if (isk) {  // row-major K for Q K^T
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int x = 32 * tb + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
              *reinterpret_cast<u32x4_t*>(Ks + x * G::QS + 8 * cg) = kvr[m][e];
            }
          }
        }
        // transposed copy: feature row, 8 tokens in fragment order
        uint16_t* base = (isk ? Kt : Vt) + (8 * cg) * G::TS + 32 * tb + 8 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // feature pair (2c, 2c+1)
          u32x4_t lo, hi;
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            const uint32_t a = kvr[m][2 * mm][c], bb = kvr[m][2 * mm + 1][c];
            lo[mm] = (a & 0xFFFFu) | (bb << 16);
            hi[mm] = (a >> 16) | (bb & 0xFFFF0000u);
          }
          *reinterpret_cast<u32x4_t*>(base + (2 * c) * G::TS) = lo;
          *reinterpret_cast<u32x4_t*>(base + (2 * c + 1) * G::TS) = hi;
        }
      }
    }
  };

  if (tau0 < tau_end) load_chunk(tau0, min(C, tau_end - tau0));

  for (int tc = tau0; tc < tau_end; tc += C) {
    const int n = min(C, tau_end - tc);
    store_chunk();
    __syncthreads();  // chunk tc is in LDS
    if (tc + C < tau_end) load_chunk(tc + C, min(C, tau_end - tc - C));
    const float gdec = exp2f(-sl2 * (float)n);

    // S_{c-1} as hi/lo bf16 A-operands of S^T (value row w, 8 keys)
    u32x4_t sfh[G::WT][G::KSD], sfl[G::WT][G::KSD];
    // this wave's masked P^T tiles, hi/lo
    u32x2_t ph[G::MAXT], pl[G::MAXT];
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          u32x2_t h0, l0, h1, l1;
          split4(S[wt][2 * ks], h0, l0);
          split4(S[wt][2 * ks + 1], h1, l1);
          sfh[wt][ks] = u32x4_t{h0[0], h0[1], h1[0], h1[1]};
          sfl[wt][ks] = u32x4_t{l0[0], l0[1], l1[0], l1[1]};
        }

      // ---- masked scores P^T = (K Q^T) * M^T, kept in registers ----------
#pragma unroll
      for (int m = 0; m < G::MAXT; ++m) {
        int kb, qb;
        if (!tile_of<G::NQB>(wave, m, kb, qb)) continue;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          const u32x4_t kf = lds_read16(Ks + (16 * kb + li) * G::QS + 32 * ks + 8 * lg);
          const u32x4_t qf = lds_read16(Qs + (16 * qb + li) * G::QS + 32 * ks + 8 * lg);
          acc = mfma16(kf, qf, acc);
        }
        const int delta = qb - kb;
        if (delta == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= md[r];
        } else {
          const float f = exp2f(-sl2 * (float)(16 * (delta - 1)));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= f * mo[r];
        }
        split4(acc, ph[m], pl[m]);
      }
    }

    // ---- V fragments (row w of V^T, 8 tokens) for this wave's value tiles ----
    u32x4_t vfr[G::WT][G::KSC];
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int ks = 0; ks < G::KSC; ++ks)
        vfr[wt][ks] = lds_read16(Vt + (16 * (wave * G::WT + wt) + li) * G::TS + 32 * ks + 8 * lg);

    // ---- state update S <- lambda^n S + K^T diag(b) V (b*V as hi + lo) ----
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int t = 0; t < G::NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[wt][t][r] *= gdec;
#pragma unroll
    for (int ks = 0; ks < G::KSC; ++ks) {
      float bks[8];
      if (n == C) {
        const float f = exp2f(-sl2 * (float)(32 * (G::KSC - 1 - ks)));
#pragma unroll
        for (int e = 0; e < 8; ++e) bks[e] = f * bl[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = 32 * ks + (e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4);
          bks[e] = x < n ? exp2f(-sl2 * (float)(n - 1 - x)) : 0.f;
        }
      }
      u32x4_t vbh[G::WT], vbl[G::WT];
#pragma unroll
      for (int wt = 0; wt < G::WT; ++wt) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t w0 = vfr[wt][ks][2 * c], w1 = vfr[wt][ks][2 * c + 1];
          const f32x4_t x = {bf_lo(w0) * bks[4 * c], bf_hi(w0) * bks[4 * c + 1],
                             bf_lo(w1) * bks[4 * c + 2], bf_hi(w1) * bks[4 * c + 3]};
          u32x2_t hh, ll;
          split4(x, hh, ll);
          vbh[wt][2 * c] = hh[0];
          vbh[wt][2 * c + 1] = hh[1];
          vbl[wt][2 * c] = ll[0];
          vbl[wt][2 * c + 1] = ll[1];
        }
      }
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        const u32x4_t kf = lds_read16(Kt + (16 * t + li) * G::TS + 32 * ks + 8 * lg);
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) {
          S[wt][t] = mfma16(kf, vbh[wt], S[wt][t]);
          S[wt][t] = mfma16(kf, vbl[wt], S[wt][t]);
        }
      }
    }

    if constexpr (!STATE_ONLY) {
      __syncthreads();  // K and K^T are dead: their space takes the P^T fragments
#pragma unroll
      for (int m = 0; m < G::MAXT; ++m) {
        int kb, qb;
        if (!tile_of<G::NQB>(wave, m, kb, qb)) continue;
        const int off = ((frag_base(qb) + (kb >> 1)) * 64 + lane) * 8;
        const int half = (kb & 1) * 4;
        *reinterpret_cast<u32x2_t*>(Pth + off + half) = ph[m];
        *reinterpret_cast<u32x2_t*>(Ptl + off + half) = pl[m];
        if (kb == qb && !(qb & 1)) {  // even diagonal: the other half of the step is empty
          *reinterpret_cast<u32x2_t*>(Pth + off + 4) = u32x2_t{0, 0};
          *reinterpret_cast<u32x2_t*>(Ptl + off + 4) = u32x2_t{0, 0};
        }
      }
      __syncthreads();  // all P^T fragments written

      // ---- outputs: O^T = diag(a) (S^T Q^T) + V^T P^T, per query block ----
#pragma unroll
      for (int qb = 0; qb < G::NQB; ++qb) {
        // Q^T as B operand in the key order of the S fragments:
        // features {32ks + 4lg + r} and {32ks + 16 + 4lg + r}
        u32x4_t qf[G::KSD];
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          const uint16_t* row = Qs + (16 * qb + li) * G::QS + 32 * ks + 4 * lg;
          const u32x2_t a0 = lds_read8(row), a1 = lds_read8(row + 16);
          qf[ks] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        }
        u32x4_t pfh[G::KSC], pfl[G::KSC];
#pragma unroll
        for (int ks = 0; ks <= qb / 2; ++ks) {
          const int off = ((frag_base(qb) + ks) * 64 + lane) * 8;
          pfh[ks] = lds_read16(Pth + off);
          pfl[ks] = lds_read16(Ptl + off);
        }
        const int i = 16 * qb + li;
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < G::KSD; ++ks) {
            acc = mfma16(sfh[wt][ks], qf[ks], acc);
            acc = mfma16(sfl[wt][ks], qf[ks], acc);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= aq[qb];
#pragma unroll
          for (int ks = 0; ks <= qb / 2; ++ks) {
            acc = mfma16(vfr[wt][ks], pfh[ks], acc);
            acc = mfma16(vfr[wt][ks], pfl[ks], acc);
          }
          if (i < n) {
            uint16_t* dst = og + (size_t)tok(tc + i) * D + 16 * (wave * G::WT + wt) + 4 * lg;
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack2(acc[0], acc[1]), pack2(acc[2], acc[3])};
          }
        }
      }
    }
    __syncthreads();  // LDS free for the next chunk
  }

  if (s_final) {
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        const int col = 16 * (wave * G::WT + wt) + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) s_final[(size_t)(16 * t + 4 * lg + r) * D + col] = S[wt][t][r];
      }
  }
}

template <int C, int D>
hipError_t launch_fwd_cd(const FwdPass& p, hipStream_t s) {
  PiecePass none{};
  const unsigned grid = (unsigned)(p.B * p.H * p.nseg);
  hipLaunchKernelGGL((fwd_bf16_kernel<C, D, false>), dim3(grid), dim3(kThreads), 0, s, p, none);
  return hipGetLastError();
}

template <int C, int D>
hipError_t launch_pieces_cd(const PiecePass& pp, hipStream_t s) {
  FwdPass none{};
  const unsigned grid = (unsigned)(pp.B * pp.H * pp.npiece);
  hipLaunchKernelGGL((fwd_bf16_kernel<C, D, true>), dim3(grid), dim3(kThreads), 0, s, none, pp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdPass& p, hipStream_t s) {
  if (p.D == 128) {
    if (p.C == 128) return launch_fwd_cd<128, 128>(p, s);
    if (p.C == 64) return launch_fwd_cd<64, 128>(p, s);
    if (p.C == 32) return launch_fwd_cd<32, 128>(p, s);
  } else if (p.D == 64) {
    if (p.C == 128) return launch_fwd_cd<128, 64>(p, s);
    if (p.C == 64) return launch_fwd_cd<64, 64>(p, s);
    if (p.C == 32) return launch_fwd_cd<32, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pieces_bf16(const PiecePass& p, hipStream_t s) {
  if (p.D == 128) {
    if (p.C == 128) return launch_pieces_cd<128, 128>(p, s);
    if (p.C == 64) return launch_pieces_cd<64, 128>(p, s);
    if (p.C == 32) return launch_pieces_cd<32, 128>(p, s);
  } else if (p.D == 64) {
    if (p.C == 128) return launch_pieces_cd<128, 64>(p, s);
    if (p.C == 64) return launch_pieces_cd<64, 64>(p, s);
    if (p.C == 32) return launch_pieces_cd<32, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
