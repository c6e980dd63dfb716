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
//  * one workgroup of d/32 waves owns a whole head over one segment of the
//    sequence, so Q K^T is computed once per chunk and every operand is read
//    from HBM once; parallelism beyond B*H comes from segments, whose start
//    states the piece and scan kernels assemble (the "local recursion +
//    global correction" algebra of the same section);
//  * wave w owns value columns 32w .. 32w+31: its slice of the fp32 state
//    lives in its registers for the whole segment and it computes every
//    output and state element of those columns.  Operands shared by all
//    columns (Q, K and the masked scores) are read from LDS once per wave, so
//    wider column slices mean less LDS traffic; at one wave per SIMD each
//    phase is unrolled so that a wave keeps loads, matrix-core and vector
//    work in flight together;
//  * the masked scores P^T = (K Q^T) * M^T are computed once per chunk -- wave
//    w takes the score tiles of query blocks w and NQB-1-w, reusing each K
//    fragment for both -- and exchanged through LDS in the register order of
//    the P V product's B operand;
//  * the three operands that are not inputs -- the masked scores P, the state
//    S and b*V -- are handed to the matrix cores as bf16 hi + lo pairs, so the
//    products carry ~16 significant bits (plain bf16 operands would lose as
//    much accuracy as the final rounding of the output);
//  * Q, K and V are staged row-major in LDS with an XOR swizzle of 16-byte
//    chunks (see swz_of) that depends only on the row modulo 16, so every
//    LDS address is a per-lane constant plus a compile-time offset; K^T and
//    V^T fragments (contractions over tokens) come straight from the
//    row-major tiles through the transposing LDS read of gfx950; Q, K and V
//    move global -> LDS without passing through registers.
// The same kernel in STATE_ONLY mode computes piece states (K^T diag(b) V
// accumulated over a piece) for the segment pre-pass, and with EPI applies
// the output epilogue (per-head RMSNorm, weight, sigmoid gate) before the
// outputs are stored.
#include <type_traits>

#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {

template <int C, int D, bool STATE_ONLY>
struct Cfg {
  static constexpr int NW = D / 32;    // waves: 32 value columns each
  static constexpr int THREADS = 64 * NW;
  static constexpr int CT = 2;         // 16-column value tiles per wave (the
                                       // output stores assume exactly two)
  static constexpr int NQB = C / 16;   // 16-token query / key blocks per chunk
  static constexpr int KSC = C / 32;   // 32-token contraction steps
  static constexpr int KSD = D / 32;   // 32-feature contraction steps
  static constexpr int NT = D / 16;    // 16-feature tiles of the state
  static constexpr int NPAIR = (NQB + 1) / 2;  // query-block pairs {p, NQB-1-p}
  static constexpr int NFRAG = frag_base(NQB);
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR; // rows per wave-wide 16-byte-per-lane move
  static constexpr int TILE = C * D;              // elements per tile
  static constexpr int PT_HALF = NFRAG * 64 * 8;  // one of P_hi / P_lo
  static_assert(C == 32 || C == 64 || C == 128, "chunk");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert((RPI * NW) % 16 == 0, "row mod 16 per lane");
  static_assert(C % (RPI * NW) == 0, "whole direct moves per wave");
  static_assert((STATE_ONLY ? 4 * TILE : 3 * TILE + 2 * PT_HALF) * 2 + 4 * NW * C <= 160 * 1024,
                "LDS");
};


// EPI: the output epilogue (per-head RMSNorm, per-channel weight, sigmoid
// gate) is applied to the fp32 outputs before they are rounded and stored.
template <int C, int D, bool STATE_ONLY, bool EPI>
__global__ __launch_bounds__(D / 32 * 64) void fwd_bf16_kernel(FwdPass p, PiecePass pp,
                                                                const SeqTable st) {
  static_assert(!(STATE_ONLY && EPI), "the epilogue belongs to the main pass");
  using G = Cfg<C, D, STATE_ONLY>;
  constexpr int CT = G::CT;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;

  // ---- work item -------------------------------------------------------
  // One (sequence, head) row and a token range [tau0, tau_end) of it; token
  // positions count from the row's first token (or from its last one when
  // the pass runs backwards in time).
  const bool packed = st.nseq > 0;
  Row row;
  int tau0, tau_end;
  bool reverse;
  const float* slope;
  const uint16_t *qg = nullptr, *kg, *vg, *gg = nullptr;
  uint16_t* og = nullptr;
  const float* s_init = nullptr;
  bool s_init_t = false;  // s_init holds S^T
  float* s_final = nullptr;
  if constexpr (STATE_ONLY) {
    // Pieces are numbered by distance from the end of their segment first:
    // the pieces every head needs (those just before a segment start) take
    // the lowest workgroup ids, so they are dispatched first and spread over
    // all XCDs (consecutive ids go to different XCDs), and the workgroups
    // that exit at once come last.  Packed batches: head fastest within a
    // rank, then segments in schedule order.
    const int ppseg = pp.seg_len / pp.piece_len;
    const int per_row = packed ? pp.G : pp.nseg - 1;  // segment groups per row / head
    const int groups = (packed ? pp.H : pp.B * pp.H) * per_row;
    const int rank = blockIdx.x / groups;  // 0 = last piece of its segment
    const int g = blockIdx.x - rank * groups;
    int seg;
    if (packed) {
      const int gs = g / pp.H, h = g - gs * pp.H;
      const int i = seq_of_segment(st, gs);
      row = packed_row(st, i, h, pp.H, pp.G, ppseg);
      seg = gs - st.g0[i];
    } else {
      row = uniform_row(g / per_row, pp.H, pp.N, pp.nseg, pp.npiece);
      seg = g % per_row;
    }
    const int piece = seg * ppseg + (ppseg - 1 - rank);
    reverse = pp.reverse;
    slope = pp.slope;
    tau0 = piece * pp.piece_len;
    tau_end = min(row.len, tau0 + pp.piece_len);
    // needed only if the nearest segment start at or after the piece end is
    // a real segment start and the decay over the gap is not negligible
    const int r_star = (tau_end + pp.seg_len - 1) / pp.seg_len;
    if (tau0 >= tau_end || r_star > row.nseg - 1) return;
    const float rate = slope[row.h] * kLog2e;  // log2 of the decay per token
    const float gap = (float)(r_star * pp.seg_len - tau_end);
    if (rate * gap >= kSkipLog2) return;
    // by the same rule, the piece's tokens whose decay to that segment start
    // is below 2^-kSkipLog2 are not accumulated: the pass starts at the
    // chunk that holds the earliest token above it
    if (rate * (float)(tau_end - tau0) > kSkipLog2) {
      const int keep = (int)(kSkipLog2 / rate) + 1;  // < tau_end - tau0 + gap here
      const int first = r_star * pp.seg_len - keep;  // earliest token kept
      if (first > tau0) tau0 += ((first - tau0) / C) * C;
    }
    const size_t head_off = row.tok * D;
    kg = (const uint16_t*)pp.k + head_off;
    vg = (const uint16_t*)pp.v + head_off;
    s_final = pp.pieces + ((size_t)row.piecebase + piece) * D * D;
  } else {
    int seg;
    if (packed) {
      // head fastest: consecutive workgroups (which go to different XCDs)
      // take the heads of one segment, so every XCD gets the same share of
      // each sequence; segments in schedule order, longest sequence first
      const int gs = blockIdx.x / p.H, h = blockIdx.x - gs * p.H;
      const int i = seq_of_segment(st, gs);
      row = packed_row(st, i, h, p.H, p.G, 0);
      seg = gs - st.g0[i];
    } else {
      row = uniform_row(blockIdx.x / p.nseg, p.H, p.N, p.nseg, 0);
      seg = blockIdx.x % p.nseg;
    }
    reverse = p.reverse;
    slope = p.slope;
    tau0 = seg * p.seg_len;
    tau_end = min(row.len, tau0 + p.seg_len);
    const size_t head_off = row.tok * D;
    qg = (const uint16_t*)p.q + head_off;
    kg = (const uint16_t*)p.k + head_off;
    vg = (const uint16_t*)p.v + head_off;
    og = (uint16_t*)p.o + head_off;
    if constexpr (EPI) gg = (const uint16_t*)p.gate + head_off;
    if (row.nseg > 1) {
      // segment 0 too: the scan kernel copied state_in into entry 0, so no
      // workgroup reads state_in while the last segment writes state_out
      s_init = p.seg_states + ((size_t)row.segbase + seg) * D * D;
      s_init_t = p.seg_states_transposed;
    } else {
      s_init = p.state_in ? p.state_in + (size_t)row.st * D * D : nullptr;
    }
    if (seg == row.nseg - 1 && p.state_out) s_final = p.state_out + (size_t)row.st * D * D;
  }
  const int N = row.len;  // reversed positions count back from the row's last token
  const float sl2 = slope[row.h] * kLog2e;  // lambda^e = exp2(-sl2 * e)
  // states from an earlier call: a workspace whose tag is not the expected
  // one starts the row from NaN, so every output of the pass is NaN
  bool poison = false;
  if constexpr (!STATE_ONLY) {
    if (p.tag) {
#pragma unroll
      for (int i = 0; i < kTagWords; ++i) poison |= p.tag[i] != p.tag_expect.w[i];
    }
  }
  const int col0 = 32 * wave;                // this wave's first value column

  // ---- fp32 state: S[t][ct][r] = S[feature feat(t, r)][value col0 + vcol(ct, li)]
  // Value columns of the wave's two 16-column tiles are interleaved by 4:
  // tile ct, row m is column 8(m>>2) + 4ct + (m&3), so that the 4 output
  // columns a lane holds in each tile are 8 adjacent columns in all.
  // Feature order: tiles 2m and 2m+1 hold, in lane group lg, the two halves
  // of the 8 consecutive features 32m + 8lg .. +7, so that the state, split
  // into bf16 operands, meets Q in the plain row-fragment order.
  auto feat = [&](int t, int r) { return 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + r; };
  auto vcol = [&](int ct, int m) { return 8 * (m >> 2) + 4 * ct + (m & 3); };
  f32x4_t S[G::NT][CT];
#pragma unroll
  for (int t = 0; t < G::NT; ++t)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[t][ct][r] = poison    ? __builtin_nanf("")
                      : !s_init  ? 0.f
                      : s_init_t ? s_init[(size_t)(col0 + vcol(ct, li)) * D + feat(t, r)]
                                 : s_init[(size_t)feat(t, r) * D + col0 + vcol(ct, li)];

  // ---- per-lane decay tables --------------------------------------------
  // P^T tile element: key row 16kb + 4lg + r, query column 16qb + li.
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
  // a of query 16qb + li is a_lane * lambda^(16 qb)
  const float a_lane = fast_exp2(-sl2 * (float)(li + 1));

  // ---- per-lane LDS offsets (elements); loop indices add constants ------
  // row fragments (16 B): rows 16x + li, features 32ks + 8lg .. +7
  const int sA = swz_of<D>(li);
  int offA[G::KSD];
#pragma unroll
  for (int ks = 0; ks < G::KSD; ++ks) offA[ks] = li * D + 8 * ((4 * ks + lg) ^ sA);
  // transposing reads: row 8lg + (li>>2) + 4hh (+32ks), 4 columns from
  // cols(li&3) on; lane i of the lane group then receives column
  // cols(i>>2) + (i&3) of those 4 rows.  Value tiles take the interleaved
  // value columns (cols(j) = col0 + vcol(ct, 4j)), K^T tiles the state's
  // feature order (cols(j) = feat(t, 0) of lane group j).
  auto off_tr = [&](int hh, int chunk16, int half) {
    const int r = 8 * lg + (li >> 2) + 4 * hh;
    return r * D + 8 * (chunk16 ^ swz_of<D>(r & 15)) + 4 * half;
  };
  int offT[G::NT][2], offV[CT][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int t = 0; t < G::NT; ++t) offT[t][hh] = off_tr(hh, 4 * (t >> 1) + (li & 3), t & 1);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      offV[ct][hh] = off_tr(hh, 4 * wave + (li & 3), ct);
  }
  // The per-lane offsets are re-issued in place at the top of every chunk
  // through an empty asm, so the compiler cannot hoist the dozens of
  // addresses derived from them out of the chunk loop, where they would stay
  // live and spill.
  auto refresh_offsets = [&]() {
#pragma unroll
    for (int ks = 0; ks < G::KSD; ++ks) {
      offA[ks] = opaque(offA[ks]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int t = 0; t < G::NT; ++t) offT[t][hh] = opaque(offT[t][hh]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) offV[ct][hh] = opaque(offV[ct][hh]);
    }
  };
  auto& lA = offA;
  auto& lT = offT;
  auto& lV = offV;

  // column fragment: 8 tokens 32ks + 8lg .. +7 of one column, from two
  // transposing reads
  auto col_frag = [&](const uint16_t* tile, int ks, const int (&o)[2]) -> u32x4_t {
    const u32x2_t a = lds_read_tr8(tile + 32 * ks * D + o[0]);
    const u32x2_t c = lds_read_tr8(tile + 32 * ks * D + o[1]);
    return u32x4_t{a[0], a[1], c[0], c[1]};
  };

  // ---- staging ------------------------------------------------------------
  // Rows past the end of the sequence read the last valid row: such K and V
  // rows only ever meet zero weights (causal mask, b = 0), and Q rows past
  // the end produce outputs that are not stored.
  //
  // Direct moves: the wave's instruction m covers rows RPI (wave + NW m) ..
  // +RPI-1 of the tile; lane l lands in physical chunk l % CPR of the row
  // RPI (wave + NW m) + l / CPR and fetches the logical chunk the swizzle maps
  // there (RPI NW is a multiple of 16, so row mod 16 is fixed per lane).
  // Global offsets count from the chunk's lowest-address token, so they are
  // non-negative in both directions.  The LDS destination goes to the
  // instruction as a plain address (through an empty asm), so the compiler
  // does not tie these writes to the tile variables and does not hold later
  // LDS reads of other tiles until they land; the kernel waits for them
  // itself (a vmcnt wait and a barrier before the tile is read).
  constexpr int DM_STEP = G::RPI * G::NW;  // rows between a lane's moves
  constexpr int DM_N = C / DM_STEP;        // moves per wave and tile
  const int dm_row0 = G::RPI * wave + lane / G::CPR;
  const int dm_col = 8 * ((lane % G::CPR) ^ swz_of<D>(dm_row0 & 15));
  // a full chunk's moves share one per-lane byte offset; move m adds
  // m * dm_step elements to the (wave-uniform) base
  const uint32_t dm_off_b = 2u * (uint32_t)((reverse ? (C - 1 - dm_row0) : dm_row0) * D + dm_col);
  const int dm_step = reverse ? -DM_STEP * D : DM_STEP * D;
  auto load_direct = [&](const uint16_t* src, uint16_t* tile, int tc, int n) {
    const uint16_t* base = src + (long)(reverse ? (N - tc - n) : tc) * D;
    const uint32_t lds0 = opaque_s((uint32_t)(uintptr_t)(tile + G::RPI * wave * D));
    constexpr uint32_t kMoveBytes = 2u * G::RPI * G::NW * D;  // LDS bytes between moves
    if (n == C) {
#pragma unroll
      for (int m = 0; m < DM_N; ++m)
        dma16(buffer_rsrc(base + (long)m * dm_step), dm_off_b, lds0 + kMoveBytes * m);
    } else {
      const auto rs = buffer_rsrc(base);
#pragma unroll
      for (int m = 0; m < DM_N; ++m) {
        const int rr = min(dm_row0 + DM_STEP * m, n - 1);
        dma16(rs, 2u * (uint32_t)((reverse ? (n - 1 - rr) : rr) * D + dm_col), lds0 + kMoveBytes * m);
      }
    }
  };

  // V^T fragments of this wave's value tiles, all token steps of the chunk
  auto load_vfr = [&](const uint16_t* Vt, u32x4_t (&vf)[G::KSC][CT]) {
#pragma unroll
    for (int ks = 0; ks < G::KSC; ++ks)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) vf[ks][ct] = col_frag(Vt, ks, lV[ct]);
  };

  // S <- lambda^n S + K^T diag(b) V for the chunk (K tile Kt, V fragments vf)
  // FULL (n == C) is a compile-time flag, so that a full chunk's update is
  // one branch-free block the scheduler can interleave across token steps.
  // b*V for token step ks as hi/lo B operands: unit u = (ct, c) covers 4 of
  // the 8 tokens of one value tile
  auto make_bv_unit = [&](const u32x4_t (&vf)[G::KSC][CT], int ks, const float (&bk)[8], int u,
                          u32x4_t (&bvh)[CT], u32x4_t (&bvl)[CT]) __attribute__((always_inline)) {
    const int ct = u >> 1, c = u & 1;
    const uint32_t w0 = vf[ks][ct][2 * c], w1 = vf[ks][ct][2 * c + 1];
    const f32x4_t x = {bf_lo(w0) * bk[4 * c], bf_hi(w0) * bk[4 * c + 1],
                       bf_lo(w1) * bk[4 * c + 2], bf_hi(w1) * bk[4 * c + 3]};
    u32x2_t h2, l2;
    split4(x, h2, l2);
    bvh[ct][2 * c] = h2[0];
    bvh[ct][2 * c + 1] = h2[1];
    bvl[ct][2 * c] = l2[0];
    bvl[ct][2 * c + 1] = l2[1];
  };
  // S <- lambda^n S + K^T diag(b) V for the chunk (K tile Kt, V fragments vf).
  // A full chunk's update is scheduled by hand: 32 groups (token step ks,
  // state tile t) of four products, each carrying a slice of the vector work
  // of the next step's b*V and the K^T reads three groups ahead, closed by a
  // scheduling fence.  A single wave then keeps the matrix cores and the
  // vector ALU busy together, which the compiler's own order does not.
  auto state_update_full = [&](const uint16_t* Kt, const u32x4_t (&vf)[G::KSC][CT]) __attribute__((always_inline)) {
    constexpr int NG = G::KSC * G::NT;  // groups
    constexpr int PF = 3;               // K^T prefetch distance (groups)
    const float gdec = fast_exp2(-sl2 * (float)C);
    float bk[8];
    auto set_bk = [&](int ks) {
      const float f = fast_exp2(-sl2 * (float)(32 * (G::KSC - 1 - ks)));
#pragma unroll
      for (int e = 0; e < 8; ++e) bk[e] = f * bl[e];
    };
    u32x4_t bvh[2][CT], bvl[2][CT];
    set_bk(0);
#pragma unroll
    for (int u = 0; u < 2 * CT; ++u) make_bv_unit(vf, 0, bk, u, bvh[0], bvl[0]);
    u32x4_t kt[PF + 1];
#pragma unroll
    for (int g = 0; g < PF; ++g) kt[g] = col_frag(Kt, g / G::NT, lT[g % G::NT]);
    if (G::KSC > 1) set_bk(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int ks = g / G::NT, t = g % G::NT;
      if (g + PF < NG) kt[(g + PF) % (PF + 1)] = col_frag(Kt, (g + PF) / G::NT, lT[(g + PF) % G::NT]);
      if (ks == 0) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[t][ct][r] *= gdec;
      }
      const u32x4_t& k = kt[g % (PF + 1)];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) S[t][ct] = mfma16(k, bvh[ks & 1][ct], S[t][ct]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) S[t][ct] = mfma16(k, bvl[ks & 1][ct], S[t][ct]);
      // vector work of step ks+1: its 2*CT b*V units spread evenly over the
      // step's NT groups, then the b factors of step ks+2
      if (ks + 1 < G::KSC) {
        constexpr int US = G::NT / (2 * CT);  // groups per unit
        static_assert(US >= 1 && G::NT % (2 * CT) == 0, "b*V units per step");
        if (t % US == US - 1)
          make_bv_unit(vf, ks + 1, bk, t / US, bvh[(ks + 1) & 1], bvl[(ks + 1) & 1]);
        if (t == G::NT - 1 && ks + 2 < G::KSC) set_bk(ks + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // compiler-scheduled order: partial chunks (the last of a sequence) and the
  // piece kernel
  auto state_update_partial = [&](const uint16_t* Kt, const u32x4_t (&vf)[G::KSC][CT], int n) __attribute__((always_inline)) {
    const float gdec = fast_exp2(-sl2 * (float)n);
#pragma unroll
    for (int t = 0; t < G::NT; ++t)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[t][ct][r] *= gdec;
#pragma unroll
    for (int ks = 0; ks < G::KSC; ++ks) {
      float bk[8];
      if (n == C) {
        const float f = fast_exp2(-sl2 * (float)(32 * (G::KSC - 1 - ks)));
#pragma unroll
        for (int e = 0; e < 8; ++e) bk[e] = f * bl[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = 32 * ks + 8 * opaque(lg) + e;
          bk[e] = x < n ? fast_exp2(-sl2 * (float)(n - 1 - x)) : 0.f;
        }
      }
      u32x4_t bvh[CT], bvl[CT];
#pragma unroll
      for (int u = 0; u < 2 * CT; ++u) make_bv_unit(vf, ks, bk, u, bvh, bvl);
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        const u32x4_t kt = col_frag(Kt, ks, lT[t]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) S[t][ct] = mfma16(kt, bvh[ct], S[t][ct]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) S[t][ct] = mfma16(kt, bvl[ct], S[t][ct]);
      }
    }
  };
  auto state_update = [&](const uint16_t* Kt, const u32x4_t (&vf)[G::KSC][CT], int n) __attribute__((always_inline)) {
    // The piece kernel keeps the compiler-scheduled loop: the hand
    // schedule's extra live fragments would halve its occupancy.
    if (!STATE_ONLY && n == C)
      state_update_full(Kt, vf);
    else
      state_update_partial(Kt, vf, n);
  };

  if constexpr (STATE_ONLY) {
    // K and V double-buffered: chunk c+1 streams in while chunk c is used.
    // Each buffer is its own variable and the loop is unrolled by two, so
    // every LDS read names its buffer statically.
    __shared__ __attribute__((aligned(16))) uint16_t K0[G::TILE], V0[G::TILE], K1[G::TILE],
        V1[G::TILE];
    auto chunk = [&](auto par, int tc) {
      constexpr int PAR = decltype(par)::value;
      refresh_offsets();
      const int n = min(C, tau_end - tc);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk tc have landed
      lds_barrier();                  // ... everyone's, and chunk tc - C is done
      if (tc + C < tau_end) {
        load_direct(kg, PAR ? K0 : K1, tc + C, min(C, tau_end - tc - C));
        load_direct(vg, PAR ? V0 : V1, tc + C, min(C, tau_end - tc - C));
      }
      u32x4_t vf[G::KSC][CT];
      load_vfr(PAR ? V1 : V0, vf);
      state_update(PAR ? K1 : K0, vf, n);
    };
    if (tau0 < tau_end) {
      load_direct(kg, K0, tau0, min(C, tau_end - tau0));
      load_direct(vg, V0, tau0, min(C, tau_end - tau0));
    }
    for (int tc = tau0; tc < tau_end; tc += 2 * C) {
      chunk(std::integral_constant<int, 0>{}, tc);
      if (tc + C < tau_end) chunk(std::integral_constant<int, 1>{}, tc + C);
    }
  } else {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[G::TILE], Vs[G::TILE], Qs[G::TILE],
        Pth[G::PT_HALF], Ptl[G::PT_HALF];
    // epilogue: per-wave partial sums of squares of each output row, the
    // norm weights of this lane's columns (col0 + 8lg + 4ct + r) and the eps
    __shared__ float ssq[EPI ? G::NW : 1][EPI ? C : 1];
    float wn[EPI ? CT : 1][4];
    float eps = 0.f;
    if constexpr (EPI) {
      eps = p.eps;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          wn[ct][r] = p.norm_w[(size_t)row.h * D + col0 + 8 * lg + 4 * ct + r];
    }
    // All three tiles move straight from HBM to LDS.  Per chunk: K and V
    // (issued during the previous chunk: V once its tile has been read into
    // registers, K after the score tiles) feed the state update, which gives
    // Q (issued last, once the previous outputs are done with its tile) time
    // to land before the score tiles need it.
    if (tau0 < tau_end) {
      const int n0 = min(C, tau_end - tau0);
      load_direct(kg, Ks, tau0, n0);
      load_direct(vg, Vs, tau0, n0);
      load_direct(qg, Qs, tau0, n0);
    }
    for (int tc = tau0; tc < tau_end; tc += C) {
      const int n = min(C, tau_end - tc);
      const bool more = tc + C < tau_end;
      const int n_next = more ? min(C, tau_end - tc - C) : 0;
      refresh_offsets();
      // Vector-memory operations complete in issue order: with at most
      // DM_N (Q's moves) outstanding, this wave's K and V moves and earlier
      // output stores are done.
      wait_vmcnt<DM_N>();
      lds_barrier();  // K and V of chunk tc are in LDS

      u32x4_t vf[G::KSC][CT];
      load_vfr(Vs, vf);

      // S_{c-1} as hi/lo bf16 A operands of S^T (value row li, features
      // 32ks + 8lg .. +7)
      u32x4_t sfh[CT][G::KSD], sfl[CT][G::KSD];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          u32x2_t h0, l0, h1, l1;
          split4(S[2 * ks][ct], h0, l0);
          split4(S[2 * ks + 1][ct], h1, l1);
          sfh[ct][ks] = u32x4_t{h0[0], h0[1], h1[0], h1[1]};
          sfl[ct][ks] = u32x4_t{l0[0], l0[1], l1[0], l1[1]};
        }

      state_update(Ks, vf, n);

      // epilogue: this lane's gate values (rows 16qb + li, columns col0 +
      // 8lg .. +7).  Issued after Q's moves and before the next chunk's V
      // and K (vector-memory operations complete in order), they land during
      // the score tiles without delaying either.
      constexpr int kGateLoads = EPI ? G::NQB : 0;
      u32x4_t gq[EPI ? G::NQB : 1];
      if constexpr (EPI) {
        const uint16_t* gb = gg + (long)tc * D + col0;
#pragma unroll
        for (int qb = 0; qb < G::NQB; ++qb) {
          const int rr = min(16 * qb + li, n - 1);
          gq[qb] = *reinterpret_cast<const u32x4_t*>(at_bytes(gb, 2u * (uint32_t)(rr * D + 8 * lg)));
        }
      }

      wait_vmcnt<kGateLoads>();  // Q's moves (issued before the gate loads) are done
      lds_barrier();  // Q of chunk tc is in LDS; every wave has read V
      // V's tile was read into registers at the top of the chunk: the next
      // chunk's V moves in from here on, a whole chunk ahead of its use
      if (more) load_direct(vg, Vs, tc + C, n_next);

      // ---- masked scores P^T = (K Q^T) * M^T -> LDS as hi/lo B fragments ----
      // Tile (kb, qb), lane (lg, li) holds keys 16kb + 4lg + r of query
      // 16qb + li; in the 32-key step kb/2 these are element 4(lg&1) + r of
      // consumer lane (2(kb&1) + (lg>>1), li).  Wave w takes the query-block
      // pairs {p, NQB-1-p}, p = w, w + NW, ...: NQB+1 tiles per pair, and each
      // K fragment serves both blocks of the pair.
      auto score_mfma = [&](const u32x4_t (&kf)[G::KSD], const u32x4_t (&qf)[G::KSD]) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) acc = mfma16(kf[ks], qf[ks], acc);
        return acc;
      };
      auto score_store = [&](f32x4_t acc, int kb, int qb) {
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
      };
      auto pair_tiles = [&](auto pr_c) {
        constexpr int qlo = decltype(pr_c)::value, qhi = G::NQB - 1 - qlo;
        u32x4_t qfl[G::KSD], qfh[G::KSD];
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          qfl[ks] = lds_read16(Qs + 16 * qlo * D + lA[ks]);
          qfh[ks] = lds_read16(Qs + 16 * qhi * D + lA[ks]);
        }
        // K fragments double-buffered: key block kb+1's reads are in flight
        // while block kb's tiles are computed
        u32x4_t kf[2][G::KSD];
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) kf[0][ks] = lds_read16(Ks + lA[ks]);
#pragma unroll
        for (int kb = 0; kb <= qhi; ++kb) {
          if (kb + 1 <= qhi) {
#pragma unroll
            for (int ks = 0; ks < G::KSD; ++ks)
              kf[(kb + 1) & 1][ks] = lds_read16(Ks + 16 * (kb + 1) * D + lA[ks]);
          }
          score_store(score_mfma(kf[kb & 1], qfh), kb, qhi);
          if (kb <= qlo && qlo != qhi) score_store(score_mfma(kf[kb & 1], qfl), kb, qlo);
        }
      };
      for (int pr = wave; pr < G::NPAIR; pr += G::NW) {
        if (pr == 0) pair_tiles(std::integral_constant<int, 0>{});
        if constexpr (G::NPAIR > 1) if (pr == 1) pair_tiles(std::integral_constant<int, 1>{});
        if constexpr (G::NPAIR > 2) if (pr == 2) pair_tiles(std::integral_constant<int, 2>{});
        if constexpr (G::NPAIR > 3) if (pr == 3) pair_tiles(std::integral_constant<int, 3>{});
      }

      lds_barrier();  // P^T fragments written; the K tile is dead
      if (more) load_direct(kg, Ks, tc + C, n_next);

      // ---- outputs: O^T = diag(a) (S^T Q^T) + V^T P^T, per query block ----
      // outputs are addressed from the chunk's lowest-address token: a
      // wave-uniform base per query block and one per-lane byte offset
      // (li passes through opaque)
      uint16_t* obase = og + (long)(reverse ? (N - tc - n) : tc) * D + col0;
      const int li_c = opaque(li);
      const uint32_t o_lane_b = 2u * (uint32_t)(8 * lg + (reverse ? (n - 1 - li_c) : li_c) * D);
      const int o_qb = reverse ? -16 * D : 16 * D;
      // epilogue: gated, weighted rows held until every wave's sums of squares
      // are in LDS
      f32x4_t z[EPI ? G::NQB : 1][CT];
      // finished rows of query block qb: stored, or (epilogue) gated and
      // weighted and their sums of squares handed to LDS
      auto tail = [&](int qb, const f32x4_t (&acc)[CT], bool store) __attribute__((always_inline)) {
        if constexpr (EPI) {
          float ss = 0.f;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              ss = fmaf(acc[ct][r], acc[ct][r], ss);
              const uint32_t gw = gq[qb][2 * ct + (r >> 1)];
              const float g = (r & 1) ? bf_hi(gw) : bf_lo(gw);
              const float sig = __builtin_amdgcn_rcpf(1.f + fast_exp2(-kLog2e * g));
              z[qb][ct][r] = acc[ct][r] * wn[ct][r] * sig;
            }
          // the row's 32 columns of this wave sit in the 4 lane groups
          ss = sum_lane_xor32(sum_lane_xor16(ss));
          if (lg == 0) ssq[wave][16 * qb + li] = ss;
        } else if (store) {
          // this lane's 8 adjacent columns of row 16qb + li: one 16-byte store
          *reinterpret_cast<u32x4_t*>(at_bytes(obase + qb * o_qb, o_lane_b)) =
              u32x4_t{pack2(acc[0][0], acc[0][1]), pack2(acc[0][2], acc[0][3]),
                      pack2(acc[1][0], acc[1][1]), pack2(acc[1][2], acc[1][3])};
        }
      };
      // Full chunk, software-pipelined over query blocks: block qb's Q^T
      // fragments were read during block qb-1; its own P^T fragments are
      // read first and land during its 16 inter-chunk products; the tail of
      // block qb-1 runs between block qb's products.
      auto outputs_full = [&]() __attribute__((always_inline)) {
        u32x4_t qf[2][G::KSD];
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) qf[0][ks] = lds_read16(Qs + lA[ks]);
        f32x4_t hold[CT];
#pragma unroll
        for (int qb = 0; qb < G::NQB; ++qb) {
          const int b = qb & 1;
          u32x4_t pfh[G::KSC], pfl[G::KSC];
#pragma unroll
          for (int ks = 0; ks <= qb / 2; ++ks) {
            pfh[ks] = lds_read16(Pth + (frag_base(qb) + ks) * 512 + 8 * lane);
            pfl[ks] = lds_read16(Ptl + (frag_base(qb) + ks) * 512 + 8 * lane);
          }
          if (qb + 1 < G::NQB) {
#pragma unroll
            for (int ks = 0; ks < G::KSD; ++ks)
              qf[b ^ 1][ks] = lds_read16(Qs + 16 * (qb + 1) * D + lA[ks]);
          }
          f32x4_t x[CT], a[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            x[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            a[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int ks = 0; ks < G::KSD; ++ks)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
              for (int ct = 0; ct < CT; ++ct)
                x[ct] = mfma16(hl ? sfl[ct][ks] : sfh[ct][ks], qf[b][ks], x[ct]);
#pragma unroll
          for (int ks = 0; ks <= qb / 2; ++ks)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
              for (int ct = 0; ct < CT; ++ct)
                a[ct] = mfma16(vf[ks][ct], hl ? pfl[ks] : pfh[ks], a[ct]);
          if (qb > 0) tail(qb - 1, hold, true);
          __builtin_amdgcn_sched_barrier(0);
          const float aq = a_lane * fast_exp2(-sl2 * (float)(16 * qb));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) hold[ct][r] = fmaf(aq, x[ct][r], a[ct][r]);
          __builtin_amdgcn_sched_barrier(0);
        }
        tail(G::NQB - 1, hold, true);
      };
      // partial chunk (the last of a sequence): straightforward order
      auto outputs = [&](auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
        for (int qb = 0; qb < G::NQB; ++qb) {
          // Q^T as B operand: row fragments, the S fragments' feature order
          u32x4_t qf[G::KSD];
#pragma unroll
          for (int ks = 0; ks < G::KSD; ++ks) qf[ks] = lds_read16(Qs + 16 * qb * D + lA[ks]);
          u32x4_t pfh[G::KSC], pfl[G::KSC];
#pragma unroll
          for (int ks = 0; ks <= qb / 2; ++ks) {
            pfh[ks] = lds_read16(Pth + (frag_base(qb) + ks) * 512 + 8 * lane);
            pfl[ks] = lds_read16(Ptl + (frag_base(qb) + ks) * 512 + 8 * lane);
          }
          const float aq = a_lane * fast_exp2(-sl2 * (float)(16 * qb));
          f32x4_t acc[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < G::KSD; ++ks) {
              x = mfma16(sfh[ct][ks], qf[ks], x);
              x = mfma16(sfl[ct][ks], qf[ks], x);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[ct][r] = x[r] * aq;
#pragma unroll
            for (int ks = 0; ks <= qb / 2; ++ks) {
              acc[ct] = mfma16(vf[ks][ct], pfh[ks], acc[ct]);
              acc[ct] = mfma16(vf[ks][ct], pfl[ks], acc[ct]);
            }
          }
          tail(qb, acc, FULL || 16 * qb + li_c < n);
        }
      };
      if (n == C)
        outputs_full();
      else
        outputs(std::false_type{});
      lds_barrier();  // Q and P^T tiles are free for the next chunk
      if constexpr (EPI) {
        // every wave's sums of squares are in: scale the held rows
#pragma unroll
        for (int qb = 0; qb < G::NQB; ++qb) {
          float tot = 0.f;
#pragma unroll
          for (int w = 0; w < G::NW; ++w) tot += ssq[w][16 * qb + li];
          const float rn = __builtin_amdgcn_rsqf(tot * (1.f / D) + eps);
          if (16 * qb + li_c < n) {
            *reinterpret_cast<u32x4_t*>(at_bytes(obase + qb * o_qb, o_lane_b)) =
                u32x4_t{pack2(z[qb][0][0] * rn, z[qb][0][1] * rn),
                        pack2(z[qb][0][2] * rn, z[qb][0][3] * rn),
                        pack2(z[qb][1][0] * rn, z[qb][1][1] * rn),
                        pack2(z[qb][1][2] * rn, z[qb][1][3] * rn)};
          }
        }
      }
      // after the epilogue's stores, so that the next chunk's wait for its K
      // and V (all but Q's moves) does not wait for Q
      if (more) load_direct(qg, Qs, tc + C, n_next);
    }
  }

  if (s_final) {
#pragma unroll
    for (int t = 0; t < G::NT; ++t)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_final[(size_t)feat(t, r) * D + col0 + vcol(ct, li)] = S[t][ct][r];
  }
}

template <int C, int D>
hipError_t launch_fwd_cd(const FwdPass& p, const SeqTable& t, hipStream_t s) {
  PiecePass none{};
  const unsigned grid = (unsigned)(t.nseq > 0 ? p.H * p.G : p.B * p.H * p.nseg);
  if (p.gate)
    hipLaunchKernelGGL((fwd_bf16_kernel<C, D, false, true>), dim3(grid), dim3(D / 32 * 64), 0, s,
                       p, none, t);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<C, D, false, false>), dim3(grid), dim3(D / 32 * 64), 0,
                       s, p, none, t);
  return hipGetLastError();
}

template <int C, int D>
hipError_t launch_pieces_cd(const PiecePass& pp, const SeqTable& t, hipStream_t s) {
  FwdPass none{};
  const unsigned grid = (unsigned)(t.nseq > 0 ? pp.H * pp.G * (pp.seg_len / pp.piece_len)
                                              : pp.B * pp.H * pp.npiece);
  hipLaunchKernelGGL((fwd_bf16_kernel<C, D, true, false>), dim3(grid), dim3(D / 32 * 64), 0, s,
                     none, pp, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdPass& p, const SeqTable& t, hipStream_t s) {
  if (p.D == 128) {
    if (p.C == 128) return launch_fwd_cd<128, 128>(p, t, s);
    if (p.C == 64) return launch_fwd_cd<64, 128>(p, t, s);
    if (p.C == 32) return launch_fwd_cd<32, 128>(p, t, s);
  } else if (p.D == 64) {
    if (p.C == 128) return launch_fwd_cd<128, 64>(p, t, s);
    if (p.C == 64) return launch_fwd_cd<64, 64>(p, t, s);
    if (p.C == 32) return launch_fwd_cd<32, 64>(p, t, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pieces_bf16(const PiecePass& p, const SeqTable& t, hipStream_t s) {
  // A piece state does not depend on the chunk length it is accumulated in,
  // and piece lengths are multiples of C.  Chunks of at most 64 tokens keep
  // the double-buffered K and V tiles at 64 KB (d = 128), so two workgroups
  // share a CU and hide each other's load latency.
  if (p.D == 128) {
    if (p.C >= 64) return launch_pieces_cd<64, 128>(p, t, s);
    if (p.C == 32) return launch_pieces_cd<32, 128>(p, t, s);
  } else if (p.D == 64) {
    if (p.C >= 64) return launch_pieces_cd<64, 64>(p, t, s);
    if (p.C == 32) return launch_pieces_cd<32, 64>(p, t, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
