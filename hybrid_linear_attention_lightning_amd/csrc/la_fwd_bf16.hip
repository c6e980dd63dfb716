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
//  * one workgroup of d/16 waves owns a whole head (all d value columns) over one
//    segment of the sequence, so Q K^T is computed once per chunk and every
//    operand is read from HBM once; parallelism beyond B*H comes from segments,
//    whose start states the piece and scan kernels assemble (the "local
//    recursion + global correction" algebra of the same section);
//  * each wave owns one tile of 16 value columns of the fp32 state, kept in
//    registers for the whole segment; two waves per SIMD hide each other's
//    latencies;
//  * the three operands that are not inputs -- the masked scores P, the state
//    S and b*V -- are handed to the matrix cores as bf16 hi + lo pairs, so the
//    products carry ~16 significant bits (plain bf16 operands would lose as
//    much accuracy as the final rounding of the output);
//  * Q, K and V are staged row-major in LDS with an XOR swizzle of 16-byte
//    chunks that keeps every access pattern below free of bank conflicts and
//    depends only on the row modulo 16, so every LDS address is a per-lane
//    constant plus a compile-time offset; K^T and V^T fragments (contractions
//    over tokens) come straight from the row-major tiles through the
//    transposing LDS read of gfx950; K and V move global -> LDS without
//    registers; the masked scores of a chunk are exchanged between waves
//    through LDS in the exact register order of the MFMA B operand.
// The same kernel in STATE_ONLY mode computes piece states (K^T diag(b) V
// accumulated over a piece) for the segment pre-pass.
#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {


__host__ __device__ constexpr int frag_base(int qb) {
  // number of 32-key P^T fragments that query blocks 0..qb-1 use (qb/2+1 each)
  return qb + ((qb & 1) ? (qb >> 1) * (qb >> 1) : (qb >> 1) * ((qb >> 1) - 1));
}

template <int C, int D, bool STATE_ONLY>
struct Cfg {
  static constexpr int NW = D / 16;    // waves: one 16-column value tile each
  static constexpr int THREADS = 64 * NW;
  static constexpr int NQB = C / 16;   // 16-token query / key blocks per chunk
  static constexpr int KSC = C / 32;   // 32-token contraction steps
  static constexpr int KSD = D / 32;   // 32-feature contraction steps
  static constexpr int NT = D / 16;    // 16-feature tiles (key and value side)
  static constexpr int WT = NT / NW;   // value tiles owned by each wave (1)
  static constexpr int NFRAG = frag_base(NQB);
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR; // rows per wave-wide 16-byte-per-lane move
  static constexpr int QCH = C * CPR / THREADS;   // Q chunks per thread (>= 1)
  static constexpr int NTILE = NQB * (NQB + 1) / 2;       // causal 16x16 score tiles
  static constexpr int MAXT = (NTILE + NW - 1) / NW;      // score tiles per wave
  static constexpr int TILE = C * D;              // elements per tile
  static constexpr int PT_HALF = NFRAG * 64 * 8;  // one of P_hi / P_lo
  // STATE_ONLY: K, V double-buffered; otherwise K, V, Q and the P^T exchange
  static constexpr int LDS_ELEMS = STATE_ONLY ? 4 * TILE : 3 * TILE + 2 * PT_HALF;
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(QCH >= 1, "tile smaller than one chunk per thread");
  static_assert(WT == 1, "one value tile per wave");
  static_assert((RPI * NW) % 16 == 0 && (THREADS / CPR) % 16 == 0, "row mod 16 per lane");
};

// Swizzle of the 16-byte chunk index of row r of a [C][D] bf16 tile.  It
// depends on r mod 16 only, and makes the row-fragment reads (16 rows x 16 B),
// the permuted 8-byte Q reads, the transposing reads (4 rows x 32 B per lane
// group) and the 16-byte staging writes free of LDS bank conflicts (checked
// against a 64-bank model for every pattern the kernel issues).
template <int D>
__host__ __device__ constexpr int swz_of(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return ((r >> 1) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1) | (((r >> 3) & 1) << 2);
}

// (key block, query block) of causal score tile number t, tiles numbered
// along query blocks: t = qb (qb + 1) / 2 + kb, kb <= qb.  Wave w computes
// tiles w, w + NW, w + 2 NW, ...
__device__ __forceinline__ void tile_of(int t, int& kb, int& qb) {
  int q = 0;
  while ((q + 1) * (q + 2) / 2 <= t) ++q;
  qb = q;
  kb = t - q * (q + 1) / 2;
}

template <int C, int D, bool STATE_ONLY>
__global__ __launch_bounds__(D / 16 * 64) void fwd_bf16_kernel(FwdPass p, PiecePass pp) {
  using G = Cfg<C, D, STATE_ONLY>;
  constexpr int kThreads = G::THREADS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[G::LDS_ELEMS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;

  // ---- work item -------------------------------------------------------
  int bh, tau0, tau_end, N, H;
  bool reverse;
  const float* slope;
  const uint16_t *qg = nullptr, *kg, *vg;
  uint16_t* og = nullptr;
  const float* s_init = nullptr;
  float* s_final = nullptr;
  if constexpr (STATE_ONLY) {
    // Pieces are numbered by distance from the end of their segment first:
    // the pieces every head needs (those just before a segment start) take
    // the lowest workgroup ids, so they are dispatched first and spread over
    // all XCDs (consecutive ids go to different XCDs), and the workgroups
    // that exit at once come last.
    const int ppseg = pp.seg_len / pp.piece_len;
    const int groups = pp.B * pp.H * (pp.nseg - 1);
    const int rank = blockIdx.x / groups;  // 0 = last piece of its segment
    const int g = blockIdx.x - rank * groups;
    const int sidx = g % (pp.nseg - 1);
    const int piece = sidx * ppseg + (ppseg - 1 - rank);
    bh = g / (pp.nseg - 1);
    H = pp.H;
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
    if (slope[bh % H] * kLog2e * gap >= kSkipLog2) return;
    const size_t head_off = (size_t)bh * (size_t)N * D;
    kg = (const uint16_t*)pp.k + head_off;
    vg = (const uint16_t*)pp.v + head_off;
    s_final = pp.pieces + ((size_t)bh * pp.npiece + piece) * D * D;
  } else {
    const int seg = blockIdx.x % p.nseg;
    bh = blockIdx.x / p.nseg;
    H = p.H;
    N = p.N;
    reverse = p.reverse;
    slope = p.slope;
    tau0 = seg * p.seg_len;
    tau_end = min(N, tau0 + p.seg_len);
    const size_t head_off = (size_t)bh * (size_t)N * D;
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
  const float sl2 = slope[bh % H] * kLog2e;  // lambda^e = exp2(-sl2 * e)

  // ---- per-lane decay tables --------------------------------------------
  // P^T tile element: key row j = 16kb + 4lg + r, query column i = 16qb + li.
  // Diagonal tiles use md (zero above the diagonal); off-diagonal tiles use
  // lambda^(16 (qb-kb-1)) * mo[r], both factors <= 1 so nothing overflows.
  float md[4], mo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = li - 4 * lg - r;
    md[r] = e >= 0 ? fast_exp2(-sl2 * (float)e) : 0.f;
    mo[r] = fast_exp2(-sl2 * (float)(16 + e));
  }
  // Full chunk: b for token 32ks + 8lg + e of a fragment is
  // lambda^(32 (KSC-1-ks)) * bl[e] with bl[e] = lambda^(31 - 8lg - e).
  float bl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bl[e] = fast_exp2(-sl2 * (float)(31 - 8 * lg - e));

  // ---- per-lane LDS offsets (elements); loop indices add constants ------
  // row fragments: rows 16kb + li, features 32ks + 8lg .. +8  (+ 16kb*D)
  const int sA = swz_of<D>(li);
  int offA[G::KSD];
#pragma unroll
  for (int ks = 0; ks < G::KSD; ++ks) offA[ks] = li * D + 8 * ((4 * ks + lg) ^ sA);
  // permuted Q fragments: row 16qb + li, features 32ks + 16hh + 4lg .. +4  (+ 16qb*D)
  int offC[G::KSD][2];
#pragma unroll
  for (int ks = 0; ks < G::KSD; ++ks)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      offC[ks][hh] = li * D + 8 * ((4 * ks + (lg >> 1) + 2 * hh) ^ sA) + 4 * (lg & 1);
  // transposing reads: row 32ks + 8lg + (li>>2) + 4hh, column 16t + 4(li&3)  (+ 32ks*D)
  auto off_tr = [&](int hh, int t) {
    const int r = 8 * lg + (li >> 2) + 4 * hh;
    return r * D + 8 * ((2 * t + ((li & 3) >> 1)) ^ swz_of<D>(r & 15)) + 4 * (li & 1);
  };
  // column fragment (8 tokens 32ks + 8lg .., one feature column) from two
  // transposing reads at tile + o0 and tile + o1
  auto col_frag = [&](const uint16_t* tile, int o0, int o1) -> u32x4_t {
    const u32x2_t a = lds_read_tr8(tile + o0);
    const u32x2_t c = lds_read_tr8(tile + o1);
    return u32x4_t{a[0], a[1], c[0], c[1]};
  };

  // ---- fp32 state: this wave's WT value tiles x NT key tiles ------------
  // S[wt][t][r] = S[key 16t + 4lg + r][value 16(wave*WT + wt) + li]
  f32x4_t S[G::WT][G::NT];
  if (s_init) {
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int t = 0; t < G::NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[wt][t][r] = s_init[(size_t)(16 * t + 4 * lg + r) * D + 16 * (wave * G::WT + wt) + li];
  } else {
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int t = 0; t < G::NT; ++t) S[wt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging ------------------------------------------------------------
  // K and V go global -> LDS directly (no registers), each into a tile that
  // is dead by the time the load is issued; Q goes global -> registers one
  // chunk ahead -> swizzled LDS at the top of the next chunk.  Rows past the
  // end of the sequence read the last valid row: such K and V rows only ever
  // meet zero weights (causal mask, b = 0), and Q rows past the end produce
  // outputs that are not stored.
  const long rstep = reverse ? -(long)D : (long)D;  // elements between positions
  auto pos_ptr = [&](const uint16_t* base, int tau) {
    return base + (long)(reverse ? (N - 1 - tau) : tau) * D;
  };
  // Direct moves: wave instruction j covers rows RPI*j .. RPI*j + RPI-1 (the
  // wave's instructions are j = wave, wave+NW, ..., and RPI*NW is a multiple
  // of 16, so row mod 16 is fixed per lane); lane l lands in physical chunk
  // l % CPR of row RPI*j + l / CPR and fetches the logical chunk the swizzle
  // maps there.
  const int dm_row = lane / G::CPR;
  const int dm_col = 8 * ((lane % G::CPR) ^ swz_of<D>((G::RPI * wave + dm_row) & 15));
  auto load_direct = [&](const uint16_t* src, uint16_t* tile, int tc, int n) {
    const uint16_t* base = pos_ptr(src, tc) + dm_col;
#pragma unroll
    for (int j = wave; j < C / G::RPI; j += G::NW) {
      const int row = G::RPI * j + dm_row;
      __builtin_amdgcn_global_load_lds(
          base + (long)min(row, n - 1) * rstep,
          (__attribute__((address_space(3))) void*)(tile + G::RPI * j * D), 16, 0, 0);
    }
  };
  // Q: thread chunk m is row tid/CPR + (256/CPR) m, chunk tid % CPR
  const int qrow = tid / G::CPR;
  const int qoff = qrow * D + 8 * ((tid % G::CPR) ^ swz_of<D>(qrow & 15));
  u32x4_t qstg[G::QCH];
  auto load_q = [&](int tc, int n) {
    const uint16_t* base = pos_ptr(qg, tc) + 8 * (tid % G::CPR);
#pragma unroll
    for (int m = 0; m < G::QCH; ++m) {
      const int row = qrow + (kThreads / G::CPR) * m;
      qstg[m] = *reinterpret_cast<const u32x4_t*>(base + (long)min(row, n - 1) * rstep);
    }
  };

  // S <- lambda^n S + K^T diag(b) V for the chunk in (Kt, V fragments vfr)
  int offTK[G::NT][2];
#pragma unroll
  for (int t = 0; t < G::NT; ++t) {
    offTK[t][0] = off_tr(0, t);
    offTK[t][1] = off_tr(1, t);
  }
  auto state_update = [&](const uint16_t* Kt, const u32x4_t (&vfr)[G::WT][G::KSC], int n) {
    const float gdec = fast_exp2(-sl2 * (float)n);
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
        const float f = fast_exp2(-sl2 * (float)(32 * (G::KSC - 1 - ks)));
#pragma unroll
        for (int e = 0; e < 8; ++e) bks[e] = f * bl[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = 32 * ks + 8 * lg + e;
          bks[e] = x < n ? fast_exp2(-sl2 * (float)(n - 1 - x)) : 0.f;
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
      const uint16_t* Kk = Kt + 32 * ks * D;
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        const u32x4_t kf = col_frag(Kk, offTK[t][0], offTK[t][1]);
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) S[wt][t] = mfma16(kf, vbh[wt], S[wt][t]);
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) S[wt][t] = mfma16(kf, vbl[wt], S[wt][t]);
      }
    }
  };

  auto load_vfr = [&](const uint16_t* Vt, u32x4_t (&vfr)[G::WT][G::KSC]) {
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt) {
      const int o0 = off_tr(0, wave * G::WT + wt), o1 = off_tr(1, wave * G::WT + wt);
#pragma unroll
      for (int ks = 0; ks < G::KSC; ++ks) vfr[wt][ks] = col_frag(Vt + 32 * ks * D, o0, o1);
    }
  };

  if constexpr (STATE_ONLY) {
    // K and V double-buffered: chunk c+1 streams in while chunk c is used
    int buf = 0;
    if (tau0 < tau_end) {
      load_direct(kg, smem, tau0, min(C, tau_end - tau0));
      load_direct(vg, smem + G::TILE, tau0, min(C, tau_end - tau0));
    }
    for (int tc = tau0; tc < tau_end; tc += C) {
      const int n = min(C, tau_end - tc);
      uint16_t* Kc = smem + (2 * buf) * G::TILE;
      uint16_t* Vc = Kc + G::TILE;
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk tc have landed
      lds_barrier();
      if (tc + C < tau_end) {
        uint16_t* Kn = smem + (2 * (buf ^ 1)) * G::TILE;
        load_direct(kg, Kn, tc + C, min(C, tau_end - tc - C));
        load_direct(vg, Kn + G::TILE, tc + C, min(C, tau_end - tc - C));
      }
      u32x4_t vfr[G::WT][G::KSC];
      load_vfr(Vc, vfr);
      state_update(Kc, vfr, n);
      lds_barrier();  // chunk tc's tiles are free for chunk tc + 2C
      buf ^= 1;
    }
  } else {
    uint16_t* Ks = smem;
    uint16_t* Vs = Ks + G::TILE;
    uint16_t* Qs = Vs + G::TILE;
    uint16_t* Pth = Qs + G::TILE;
    uint16_t* Ptl = Pth + G::PT_HALF;
    if (tau0 < tau_end) {
      const int n0 = min(C, tau_end - tau0);
      load_direct(kg, Ks, tau0, n0);
      load_direct(vg, Vs, tau0, n0);
      load_q(tau0, n0);
    }
    for (int tc = tau0; tc < tau_end; tc += C) {
      const int n = min(C, tau_end - tc);
      const bool more = tc + C < tau_end;
      const int n_next = more ? min(C, tau_end - tc - C) : 0;
#pragma unroll
      for (int m = 0; m < G::QCH; ++m)
        *reinterpret_cast<u32x4_t*>(Qs + qoff + (kThreads / G::CPR) * m * D) = qstg[m];
      __builtin_amdgcn_s_waitcnt(0);  // this wave's K/V loads have landed
      lds_barrier();                  // chunk tc is in LDS
      if (more) load_q(tc + C, n_next);

      // ---- masked scores P^T = (K Q^T) * M^T -> LDS as hi/lo B fragments ----
      // Tile (kb, qb), lane (lg, li) holds keys 16kb + 4lg + r of query
      // 16qb + li; in the 32-key step kb/2 these are element 4(lg&1) + r of
      // consumer lane (2(kb&1) + (lg>>1), li).
#pragma unroll 1
      for (int t = wave; t < G::NTILE; t += G::NW) {
        int kb, qb;
        tile_of(t, kb, qb);
        const uint16_t* Kb = Ks + 16 * kb * D;
        const uint16_t* Qb = Qs + 16 * qb * D;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks)
          acc = mfma16(lds_read16(Kb + offA[ks]), lds_read16(Qb + offA[ks]), acc);
        const int delta = qb - kb;
        if (delta == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= md[r];
        } else {
          const float f = fast_exp2(-sl2 * (float)(16 * (delta - 1)));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= f * mo[r];
        }
        u32x2_t hi, lo;
        split4(acc, hi, lo);
        const int base = (frag_base(qb) + (kb >> 1)) * 64;
        const int off = (base + 16 * (2 * (kb & 1) + (lg >> 1)) + li) * 8 + 4 * (lg & 1);
        *reinterpret_cast<u32x2_t*>(Pth + off) = hi;
        *reinterpret_cast<u32x2_t*>(Ptl + off) = lo;
        if (kb == qb && !(qb & 1)) {  // even diagonal: keys 16..31 of the step are future
          *reinterpret_cast<u32x2_t*>(Pth + off + 256) = u32x2_t{0, 0};
          *reinterpret_cast<u32x2_t*>(Ptl + off + 256) = u32x2_t{0, 0};
        }
      }

      u32x4_t vfr[G::WT][G::KSC];
      load_vfr(Vs, vfr);

      // S_{c-1} as hi/lo bf16 A-operands of S^T (value row w, 8 keys)
      u32x4_t sfh[G::WT][G::KSD], sfl[G::WT][G::KSD];
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

      state_update(Ks, vfr, n);

      lds_barrier();  // P^T fragments written; K and V tiles are dead
      if (more) {
        load_direct(kg, Ks, tc + C, n_next);
        load_direct(vg, Vs, tc + C, n_next);
      }

      // ---- outputs: O^T = diag(a) (S^T Q^T) + V^T P^T, per query block ----
      uint16_t* orow = og + (long)(reverse ? (N - 1 - tc) : tc) * D + 16 * (wave * G::WT) + 4 * lg;
#pragma unroll 1
      for (int qb = 0; qb < G::NQB; ++qb) {
        // Q^T as B operand in the key order of the S fragments:
        // features {32ks + 4lg + r} and {32ks + 16 + 4lg + r}
        const uint16_t* Qb = Qs + 16 * qb * D;
        u32x4_t qf[G::KSD];
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          const u32x2_t a0 = lds_read8(Qb + offC[ks][0]);
          const u32x2_t a1 = lds_read8(Qb + offC[ks][1]);
          qf[ks] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        }
        const uint16_t* Pq = Pth + (frag_base(qb) * 64 + lane) * 8;
        u32x4_t pfh[G::KSC], pfl[G::KSC];
#pragma unroll
        for (int ks = 0; ks < G::KSC; ++ks) {
          if (ks <= qb / 2) {
            pfh[ks] = lds_read16(Pq + ks * 512);
            pfl[ks] = lds_read16(Pq + G::PT_HALF + ks * 512);
          }
        }
        const int i = 16 * qb + li;
        const float aq = fast_exp2(-sl2 * (float)(i + 1));
        f32x4_t acc[G::WT], acl[G::WT];
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) {
          acc[wt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          acl[wt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks)
#pragma unroll
          for (int wt = 0; wt < G::WT; ++wt) {
            acc[wt] = mfma16(sfh[wt][ks], qf[ks], acc[wt]);
            acl[wt] = mfma16(sfl[wt][ks], qf[ks], acl[wt]);
          }
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[wt][r] = (acc[wt][r] + acl[wt][r]) * aq;
#pragma unroll
        for (int ks = 0; ks < G::KSC; ++ks) {
          if (ks <= qb / 2) {
#pragma unroll
            for (int wt = 0; wt < G::WT; ++wt) {
              acc[wt] = mfma16(vfr[wt][ks], pfh[ks], acc[wt]);
              acc[wt] = mfma16(vfr[wt][ks], pfl[ks], acc[wt]);
            }
          }
        }
        if (i < n) {
          uint16_t* dst = orow + (long)i * rstep;
#pragma unroll
          for (int wt = 0; wt < G::WT; ++wt)
            *reinterpret_cast<u32x2_t*>(dst + 16 * wt) =
                u32x2_t{pack2(acc[wt][0], acc[wt][1]), pack2(acc[wt][2], acc[wt][3])};
        }
      }
      lds_barrier();  // Q and P^T tiles are free for the next chunk
    }
  }

  if (s_final) {
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int t = 0; t < G::NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_final[(size_t)(16 * t + 4 * lg + r) * D + 16 * (wave * G::WT + wt) + li] = S[wt][t][r];
  }
}

template <int C, int D>
hipError_t launch_fwd_cd(const FwdPass& p, hipStream_t s) {
  PiecePass none{};
  const unsigned grid = (unsigned)(p.B * p.H * p.nseg);
  hipLaunchKernelGGL((fwd_bf16_kernel<C, D, false>), dim3(grid), dim3(D / 16 * 64), 0, s, p, none);
  return hipGetLastError();
}

template <int C, int D>
hipError_t launch_pieces_cd(const PiecePass& pp, hipStream_t s) {
  FwdPass none{};
  const unsigned grid = (unsigned)(pp.B * pp.H * pp.npiece);
  hipLaunchKernelGGL((fwd_bf16_kernel<C, D, true>), dim3(grid), dim3(D / 16 * 64), 0, s, none, pp);
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
