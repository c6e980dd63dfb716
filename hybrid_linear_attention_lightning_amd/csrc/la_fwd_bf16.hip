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
//  * Q, K and V are staged row-major in LDS with an XOR swizzle of 16-byte
//    chunks that keeps every access pattern below free of bank conflicts;
//    K^T and V^T fragments (contractions over tokens) come straight from the
//    row-major tiles through the transposing LDS read of gfx950; the masked
//    scores of a chunk are exchanged between waves through LDS in the exact
//    register order of the MFMA B operand.
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
  static constexpr int NFRAG = frag_base(NQB);
  static constexpr int CH = C * D / 8;  // 16-byte chunks per tile
  static constexpr int QCH = (CH + kThreads - 1) / kThreads;  // per thread and tensor
  static constexpr int NTEN = STATE_ONLY ? 4 : 3;  // K,V double-buffered / K,V,Q
  static constexpr int TILE = C * D;                            // elements per tile
  static constexpr int PT_HALF = NFRAG * 64 * 8;                // one of P_hi / P_lo
  static constexpr int LDS_ELEMS = NTEN * TILE + (STATE_ONLY ? 0 : 2 * PT_HALF);
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(D == 64 || D == 128, "head dim");
};

// Element offset of (row, col) in a swizzled row-major [C][D] bf16 tile: the
// 16-byte chunk index is XORed with a function of the row chosen so that the
// row-fragment reads (16 rows x 16 B), the permuted 8-byte Q reads, the
// transposing reads (4 rows x 32 B per lane group) and the staging writes are
// all free of LDS bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  int s;
  if constexpr (D == 128)
    s = ((row & 3) << 2) | ((row >> 2) & 3);
  else
    s = (((row & 3) << 1) ^ (row >> 2)) & 7;
  return row * D + ((((col >> 3) ^ s) & (D / 8 - 1)) << 3) + (col & 7);
}

// (key block, query block) of the m-th P^T tile of a wave.  For C = 128 wave w
// takes query blocks 7-w and w (9 tiles each wave); otherwise query block w.
template <int NQB>
__device__ __forceinline__ bool tile_of(int wave, int m, int& kb, int& qb) {
  if constexpr (NQB == 8) {
    const int first = 8 - wave;
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
  constexpr int MAXT = G::NQB == 8 ? 9 : G::NQB == 4 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[G::LDS_ELEMS];
  uint16_t* Ks = smem;
  uint16_t* Vs = Ks + G::TILE;
  uint16_t* Qs = Vs + G::TILE;  // without STATE_ONLY (STATE_ONLY: second K,V buffer)
  uint16_t* Pth = Qs + G::TILE;
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
    md[r] = e >= 0 ? fast_exp2(-sl2 * (float)e) : 0.f;
    mo[r] = fast_exp2(-sl2 * (float)(16 + e));
  }
  // Full chunk: b for token 32ks + 8lg + e of a fragment is
  // lambda^(32 (KSC-1-ks)) * bl[e] with bl[e] = lambda^(31 - 8lg - e).
  float bl[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bl[e] = fast_exp2(-sl2 * (float)(31 - 8 * lg - e));

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

  // ---- staging ------------------------------------------------------------
  // K and V go global -> LDS directly (no registers), each into a tile that
  // is dead by the time the load is issued; Q goes global -> registers one
  // chunk ahead -> swizzled LDS at the top of the next chunk.  Rows past the
  // end of the sequence read the last valid row: such K and V rows only ever
  // meet zero weights (causal mask, b = 0), and Q rows past the end produce
  // outputs that are not stored.
  auto tok = [&](int tau) { return reverse ? (N - 1 - tau) : tau; };
  constexpr int RPI = 64 / (D / 8);  // rows per wave-wide 16-byte-per-lane load
  auto load_direct = [&](const uint16_t* src, uint16_t* tile, int tc, int n) {
#pragma unroll
    for (int j = wave; j < C / RPI; j += 4) {
      const int row = RPI * j + lane / (D / 8);
      // lane l lands in physical chunk l % (D/8) of its row: fetch the logical
      // chunk the swizzle maps there (XOR is its own inverse)
      const int c = swz<D>(row, 8 * (lane % (D / 8))) - row * D;
      const uint16_t* g = src + (size_t)tok(tc + min(row, n - 1)) * D + c;
      __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(tile + RPI * j * D),
                                       16, 0, 0);
    }
  };
  u32x4_t qstg[G::QCH];
  auto load_q = [&](int tc, int n) {
#pragma unroll
    for (int m = 0; m < G::QCH; ++m) {
      const int id = tid + kThreads * m;
      const int row = id / (D / 8), c8 = id % (D / 8);
      const size_t off = (size_t)tok(tc + min(row, n - 1)) * D + 8 * c8;
      if (id < G::CH) qstg[m] = *reinterpret_cast<const u32x4_t*>(qg + off);
    }
  };
  auto store_q = [&]() {
#pragma unroll
    for (int m = 0; m < G::QCH; ++m) {
      const int id = tid + kThreads * m;
      if (id < G::CH)
        *reinterpret_cast<u32x4_t*>(Qs + swz<D>(id / (D / 8), 8 * (id % (D / 8)))) = qstg[m];
    }
  };

  // operand fragment of a column of a row-major tile: 8 consecutive rows
  // k0..k0+7 (this lane group's 8) at column c0 + li, via two transposing reads
  auto col_frag = [&](const uint16_t* tile, int k0, int c0) -> u32x4_t {
    const int row = k0 + (li >> 2), col = c0 + 4 * (li & 3);
    const u32x2_t a = lds_read_tr8(tile + swz<D>(row, col));
    const u32x2_t c = lds_read_tr8(tile + swz<D>(row + 4, col));
    return u32x4_t{a[0], a[1], c[0], c[1]};
  };

  // S <- lambda^n S + K^T diag(b) V for the chunk in (Kt, Vt); vfr holds this
  // wave's V^T fragments (value rows, 8 tokens per lane group)
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
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        const u32x4_t kf = col_frag(Kt, 32 * ks + 8 * lg, 16 * t);
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) S[wt][t] = mfma16(kf, vbh[wt], S[wt][t]);
#pragma unroll
        for (int wt = 0; wt < G::WT; ++wt) S[wt][t] = mfma16(kf, vbl[wt], S[wt][t]);
      }
    }
  };

  auto load_vfr = [&](const uint16_t* Vt, u32x4_t (&vfr)[G::WT][G::KSC]) {
#pragma unroll
    for (int wt = 0; wt < G::WT; ++wt)
#pragma unroll
      for (int ks = 0; ks < G::KSC; ++ks)
        vfr[wt][ks] = col_frag(Vt, 32 * ks + 8 * lg, 16 * (wave * G::WT + wt));
  };

  if constexpr (STATE_ONLY) {
    // K and V double-buffered: chunk c+1 streams in while chunk c is used
    int buf = 0;
    if (tau0 < tau_end) {
      load_direct(kg, Ks, tau0, min(C, tau_end - tau0));
      load_direct(vg, Vs, tau0, min(C, tau_end - tau0));
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
      store_q();
      __builtin_amdgcn_s_waitcnt(0);  // this wave's K/V loads have landed
      lds_barrier();                  // chunk tc is in LDS
      if (more) load_q(tc + C, n_next);

      // ---- masked scores P^T = (K Q^T) * M^T -> LDS as hi/lo B fragments ----
      // Tile (kb, qb), lane (lg, li) holds keys 16kb + 4lg + r of query
      // 16qb + li; in the 32-key step kb/2 these are element 4(lg&1) + r of
      // consumer lane (2(kb&1) + (lg>>1), li).
#pragma unroll 1
      for (int m = 0; m < MAXT; ++m) {
        int kb, qb;
        if (!tile_of<G::NQB>(wave, m, kb, qb)) continue;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          const u32x4_t kf = lds_read16(Ks + swz<D>(16 * kb + li, 32 * ks + 8 * lg));
          const u32x4_t qf = lds_read16(Qs + swz<D>(16 * qb + li, 32 * ks + 8 * lg));
          acc = mfma16(kf, qf, acc);
        }
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
          const int offz = (base + 16 * (2 + (lg >> 1)) + li) * 8 + 4 * (lg & 1);
          *reinterpret_cast<u32x2_t*>(Pth + offz) = u32x2_t{0, 0};
          *reinterpret_cast<u32x2_t*>(Ptl + offz) = u32x2_t{0, 0};
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
#pragma unroll 1
      for (int qb = 0; qb < G::NQB; ++qb) {
        // Q^T as B operand in the key order of the S fragments:
        // features {32ks + 4lg + r} and {32ks + 16 + 4lg + r}
        u32x4_t qf[G::KSD];
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          const int row = 16 * qb + li;
          const u32x2_t a0 = lds_read8(Qs + swz<D>(row, 32 * ks + 4 * lg));
          const u32x2_t a1 = lds_read8(Qs + swz<D>(row, 32 * ks + 16 + 4 * lg));
          qf[ks] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        }
        u32x4_t pfh[G::KSC], pfl[G::KSC];
#pragma unroll
        for (int ks = 0; ks < G::KSC; ++ks) {
          if (ks <= qb / 2) {
            const int off = ((frag_base(qb) + ks) * 64 + lane) * 8;
            pfh[ks] = lds_read16(Pth + off);
            pfl[ks] = lds_read16(Ptl + off);
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
#pragma unroll
          for (int wt = 0; wt < G::WT; ++wt) {
            uint16_t* dst = og + (size_t)tok(tc + i) * D + 16 * (wave * G::WT + wt) + 4 * lg;
            *reinterpret_cast<u32x2_t*>(dst) =
                u32x2_t{pack2(acc[wt][0], acc[wt][1]), pack2(acc[wt][2], acc[wt][3])};
          }
        }
      }
      lds_barrier();  // Q and P^T tiles are free for the next chunk
    }
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
