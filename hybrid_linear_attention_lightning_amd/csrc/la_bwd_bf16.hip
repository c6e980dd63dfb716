// la_bwd_bf16.hip -- fused reverse pass of the Lightning Attention backward
// on bf16 MFMA (gfx950): dK and dV in one pass over time-reversed chunks.
//
// With L = sum_t o_t . dout_t and o from the forward (Ling & Ring 2.6 pages,
// "Hybrid Linear Attention" and "Long-Context Training: Context Parallel for
// Lightning Attention" sections), the key and value gradients are anti-causal
// sums,
//
//     dk_s = sum_{t>=s} lambda^(t-s) (v_s . dout_t) q_t
//     dv_s = sum_{t>=s} lambda^(t-s) (k_s . q_t) dout_t,
//
// i.e. two causal passes over the reversed sequence: pass A with
// (q, k, v) -> (V, dO, Q) gives dk, pass B with (K, Q, dO) gives dv.  Their
// carried states are transposes of each other: pass A carries
// G = sum lambda^.. dout_t q_t^T (d_o x d_q), pass B carries G^T.  This
// kernel runs both passes chunk by chunk with ONE state:
//  * wave w owns the d_q columns 32w .. 32w+31 of G (fp32, in registers) and
//    updates them exactly as the forward kernel updates its state (K^T -> dO
//    tile, V -> Q fragments);
//  * the outgoing G is split into bf16 hi + lo as pass A's A operands
//    (registers); after the dK outputs the same values go, transposed, into
//    an LDS tile G^T (rows d_q) that every wave reads back with the
//    transposing LDS read as pass B's A operands for its own d_o columns --
//    in two rounds of d/2 rows, so that the tile needs half the space;
//  * both passes' masked score tiles are computed once per chunk (waves
//    0..NW/2-1 take pass A's, the others pass B's) and exchanged through LDS;
//  * dK and dV are written per query block, dK first.
// So each chunk updates one state instead of two and reads Q and dO once.
// The LDS holds the dO and Q tiles, V and K double-buffered (the next
// chunk's move a whole chunk ahead), two score sets and half of G^T hi/lo:
// 152 KB at C = 64, d = 128, which is why the fused pass serves chunks of up
// to 64.
#include "la_common.h"
#include "la_internal.h"

namespace la {
namespace {

template <int C, int D>
struct BCfg {
  static constexpr int NW = D / 32;    // waves: 32 columns each
  static constexpr int THREADS = 64 * NW;
  static constexpr int CT = 2;         // 16-column tiles per wave
  static constexpr int NQB = C / 16;   // 16-token blocks per chunk
  static constexpr int KSC = C / 32;   // 32-token contraction steps
  static constexpr int KSD = D / 32;   // 32-feature contraction steps
  static constexpr int NT = D / 16;    // 16-feature tiles of the state
  static constexpr int NPAIR = (NQB + 1) / 2;
  static constexpr int NFRAG = frag_base(NQB);
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int TILE = C * D;
  static constexpr int PT_HALF = NFRAG * 64 * 8;
  static_assert(C == 32 || C == 64, "chunk");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(C % (RPI * NW) == 0, "whole direct moves per wave");
  static_assert((6 * TILE + 4 * PT_HALF + D * D) * 2 <= 160 * 1024, "LDS");
};

template <int C, int D>
__global__ __launch_bounds__(D / 32 * 64) void bwd_kv_bf16_kernel(BwdPass p, const SeqTable st) {
  using G = BCfg<C, D>;
  constexpr int CT = G::CT;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63, li = lane & 15, lg = lane >> 4;

  // ---- work item: one (sequence, head) row and one segment of it; the pass
  // runs backwards in time (pass position tau is token len-1-tau of the row)
  const bool packed = st.nseq > 0;
  Row row;
  int seg;
  if (packed) {
    const int gs = blockIdx.x / p.H, h = blockIdx.x - gs * p.H;
    const int i = seq_of_segment(st, gs);
    row = packed_row(st, i, h, p.H, p.G, 0);
    seg = gs - st.g0[i];
  } else {
    row = uniform_row(blockIdx.x / p.nseg, p.H, p.N, p.nseg, 0);
    seg = blockIdx.x % p.nseg;
  }
  const int tau0 = seg * p.seg_len;
  const int tau_end = min(row.len, tau0 + p.seg_len);
  const int N = row.len;
  const size_t head_off = row.tok * D;
  const uint16_t* qg = (const uint16_t*)p.q + head_off;
  const uint16_t* kg = (const uint16_t*)p.k + head_off;
  const uint16_t* vg = (const uint16_t*)p.v + head_off;
  const uint16_t* dog = (const uint16_t*)p.dout + head_off;
  uint16_t* dkg = (uint16_t*)p.dk + head_off;
  uint16_t* dvg = (uint16_t*)p.dv + head_off;
  const float* s_init = seg > 0 ? p.seg_states + ((size_t)row.segbase + seg) * D * D : nullptr;
  const float sl2 = p.slope[row.h] * kLog2e;
  const int col0 = 32 * wave;

  // ---- G (pass A's state): S[t][ct][r] = G[d_o feat(t, r)][d_q col0 + vcol(ct, li)]
  auto feat = [&](int t, int r) { return 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + r; };
  auto vcol = [&](int ct, int m) { return 8 * (m >> 2) + 4 * ct + (m & 3); };
  f32x4_t S[G::NT][CT];
#pragma unroll
  for (int t = 0; t < G::NT; ++t)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[t][ct][r] = s_init ? s_init[(size_t)feat(t, r) * D + col0 + vcol(ct, li)] : 0.f;

  // ---- per-lane decay tables (as in the forward kernel) ------------------
  float md[4], mo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = li - 4 * lg - r;
    md[r] = e >= 0 ? fast_exp2(-sl2 * (float)e) : 0.f;
    mo[r] = fast_exp2(-sl2 * (float)(16 + e));
  }
  const float a_lane = fast_exp2(-sl2 * (float)(li + 1));

  // ---- per-lane LDS offsets ----------------------------------------------
  const int sA = swz_of<D>(li);
  int lA[G::KSD];
#pragma unroll
  for (int ks = 0; ks < G::KSD; ++ks) lA[ks] = li * D + 8 * ((4 * ks + lg) ^ sA);
  auto off_tr = [&](int hh, int chunk16, int half) {
    const int r = 8 * lg + (li >> 2) + 4 * hh;
    return r * D + 8 * (chunk16 ^ swz_of<D>(r & 15)) + 4 * half;
  };
  int lT[G::NT][2], lV[CT][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int t = 0; t < G::NT; ++t) lT[t][hh] = off_tr(hh, 4 * (t >> 1) + (li & 3), t & 1);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) lV[ct][hh] = off_tr(hh, 4 * wave + (li & 3), ct);
  }
  auto col_frag = [&](const uint16_t* tile, int ks, const int (&o)[2]) -> u32x4_t {
    const u32x2_t a = lds_read_tr8(tile + 32 * ks * D + o[0]);
    const u32x2_t c = lds_read_tr8(tile + 32 * ks * D + o[1]);
    return u32x4_t{a[0], a[1], c[0], c[1]};
  };

  // V and K double-buffered (chunk parity); G^T exchanged in two halves of
  // D/2 rows (d_q) through Th / Tl
  __shared__ __attribute__((aligned(16))) uint16_t Ot[G::TILE], Qt[G::TILE], V0[G::TILE],
      V1[G::TILE], K0[G::TILE], K1[G::TILE], PAh[G::PT_HALF], PAl[G::PT_HALF],
      PBh[G::PT_HALF], PBl[G::PT_HALF], Th[D * D / 2], Tl[D * D / 2];

  // ---- direct global -> LDS moves (reversed rows), as in the forward ------
  constexpr int DM_STEP = G::RPI * G::NW;
  constexpr int DM_N = C / DM_STEP;
  const int dm_row0 = G::RPI * wave + lane / G::CPR;
  const int dm_col = 8 * ((lane % G::CPR) ^ swz_of<D>(dm_row0 & 15));
  const uint32_t dm_off_b = 2u * (uint32_t)((C - 1 - dm_row0) * D + dm_col);
  auto load_direct = [&](const uint16_t* src, uint16_t* tile, int tc, int n) {
    const uint16_t* base = src + (long)(N - tc - n) * D;
    const uint32_t lds0 = opaque_s((uint32_t)(uintptr_t)(tile + G::RPI * wave * D));
    constexpr uint32_t kMoveBytes = 2u * G::RPI * G::NW * D;
    if (n == C) {
#pragma unroll
      for (int m = 0; m < DM_N; ++m)
        dma16(buffer_rsrc(base - (long)m * DM_STEP * D), dm_off_b, lds0 + kMoveBytes * m);
    } else {
      const auto rs = buffer_rsrc(base);
#pragma unroll
      for (int m = 0; m < DM_N; ++m) {
        const int rr = min(dm_row0 + DM_STEP * m, n - 1);
        dma16(rs, 2u * (uint32_t)((n - 1 - rr) * D + dm_col), lds0 + kMoveBytes * m);
      }
    }
  };

  // ---- score tiles of one pass: P^T = (K Q^T) * M^T into (Ph, Pl) ---------
  auto score_tile = [&](const u32x4_t (&kf)[G::KSD], const u32x4_t (&qf)[G::KSD], int kb, int qb,
                        uint16_t* Ph, uint16_t* Pl) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < G::KSD; ++ks) acc = mfma16(kf[ks], qf[ks], acc);
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
    *reinterpret_cast<u32x2_t*>(Ph + off) = hi;
    *reinterpret_cast<u32x2_t*>(Pl + off) = lo;
    if (kb == qb && !(qb & 1)) {
      *reinterpret_cast<u32x2_t*>(Ph + off + 256) = u32x2_t{0, 0};
      *reinterpret_cast<u32x2_t*>(Pl + off + 256) = u32x2_t{0, 0};
    }
  };
  auto pair_tiles = [&](int qlo, const uint16_t* Ktile, const uint16_t* Qtile, uint16_t* Ph,
                        uint16_t* Pl) {
    const int qhi = G::NQB - 1 - qlo;
    u32x4_t qfl[G::KSD], qfh[G::KSD];
#pragma unroll
    for (int ks = 0; ks < G::KSD; ++ks) {
      qfl[ks] = lds_read16(Qtile + 16 * qlo * D + lA[ks]);
      qfh[ks] = lds_read16(Qtile + 16 * qhi * D + lA[ks]);
    }
    for (int kb = 0; kb <= qhi; ++kb) {
      u32x4_t kf[G::KSD];
#pragma unroll
      for (int ks = 0; ks < G::KSD; ++ks) kf[ks] = lds_read16(Ktile + 16 * kb * D + lA[ks]);
      score_tile(kf, qfh, kb, qhi, Ph, Pl);
      if (kb <= qlo && qlo != qhi) score_tile(kf, qfl, kb, qlo, Ph, Pl);
    }
  };

  // ---- outputs of one pass: O^T = diag(a) (A-operand state^T Q^T) + V^T P^T
  auto outputs = [&](const uint16_t* Qtile, const u32x4_t (&sh)[CT][G::KSD],
                     const u32x4_t (&sl)[CT][G::KSD], const u32x4_t (&vf)[G::KSC][CT],
                     const uint16_t* Ph, const uint16_t* Pl, uint16_t* og, int tc, int n) {
    uint16_t* obase = og + (long)(N - tc - n) * D + col0;
#pragma unroll
    for (int qb = 0; qb < G::NQB; ++qb) {
      u32x4_t qf[G::KSD];
#pragma unroll
      for (int ks = 0; ks < G::KSD; ++ks) qf[ks] = lds_read16(Qtile + 16 * qb * D + lA[ks]);
      u32x4_t pfh[G::KSC], pfl[G::KSC];
#pragma unroll
      for (int ks = 0; ks <= qb / 2; ++ks) {
        pfh[ks] = lds_read16(Ph + (frag_base(qb) + ks) * 512 + 8 * lane);
        pfl[ks] = lds_read16(Pl + (frag_base(qb) + ks) * 512 + 8 * lane);
      }
      const float aq = a_lane * fast_exp2(-sl2 * (float)(16 * qb));
      f32x4_t acc[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KSD; ++ks) {
          x = mfma16(sh[ct][ks], qf[ks], x);
          x = mfma16(sl[ct][ks], qf[ks], x);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ct][r] = x[r] * aq;
#pragma unroll
        for (int ks = 0; ks <= qb / 2; ++ks) {
          acc[ct] = mfma16(vf[ks][ct], pfh[ks], acc[ct]);
          acc[ct] = mfma16(vf[ks][ct], pfl[ks], acc[ct]);
        }
      }
      const int pos = 16 * qb + li;  // position in the chunk (pass order)
      if (pos < n)
        *reinterpret_cast<u32x4_t*>(obase + (8 * lg + (n - 1 - pos) * D)) =
            u32x4_t{pack2(acc[0][0], acc[0][1]), pack2(acc[0][2], acc[0][3]),
                    pack2(acc[1][0], acc[1][1]), pack2(acc[1][2], acc[1][3])};
    }
  };

  // One chunk; PAR (the chunk's parity) names this chunk's V and K buffers.
  // Per chunk: all four tiles have landed at the top (dO and Q were issued
  // after the previous chunk's scores, V and K a whole chunk ahead); the next
  // chunk's V and K are issued at once into the other buffers.
  auto chunk = [&](auto par_c, int tc) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    uint16_t* Vc = PAR ? V1 : V0;
    uint16_t* Kc = PAR ? K1 : K0;
    uint16_t* Vn = PAR ? V0 : V1;
    uint16_t* Kn = PAR ? K0 : K1;
    const int n = min(C, tau_end - tc);
    const bool more = tc + C < tau_end;
    const int n_next = more ? min(C, tau_end - tc - C) : 0;
#pragma unroll
    for (int ks = 0; ks < G::KSD; ++ks) lA[ks] = opaque(lA[ks]);
    // vector-memory operations complete in issue order: the tiles of this
    // chunk were issued before the previous chunk's 2 NQB output stores
    if (tc == tau0)
      wait_vmcnt<0>();
    else
      wait_vmcnt<2 * G::NQB>();
    lds_barrier();  // every wave's moves have landed; the previous chunk is done
    if (more) {
      load_direct(vg, Vn, tc + C, n_next);
      load_direct(kg, Kn, tc + C, n_next);
    }

    // Q^T (pass A's V) and dO^T (pass B's V) fragments of this wave's columns
    u32x4_t vfA[G::KSC][CT], vfB[G::KSC][CT];
#pragma unroll
    for (int ks = 0; ks < G::KSC; ++ks)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        vfA[ks][ct] = col_frag(Qt, ks, lV[ct]);
        vfB[ks][ct] = col_frag(Ot, ks, lV[ct]);
      }

    // outgoing G as hi/lo A operands of pass A (registers)
    u32x4_t sfh[CT][G::KSD], sfl[CT][G::KSD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int t = 0; t < G::NT; ++t) {
        u32x2_t h, l;
        split4(S[t][ct], h, l);
        sfh[ct][t >> 1][2 * (t & 1)] = h[0];
        sfh[ct][t >> 1][2 * (t & 1) + 1] = h[1];
        sfl[ct][t >> 1][2 * (t & 1)] = l[0];
        sfl[ct][t >> 1][2 * (t & 1) + 1] = l[1];
      }

    // G <- lambda^n G + dO^T diag(b) Q (K^T fragments from the dO tile)
    {
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
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = 32 * ks + 8 * lg + e;
          bk[e] = x < n ? fast_exp2(-sl2 * (float)(n - 1 - x)) : 0.f;
        }
        u32x4_t bvh[CT], bvl[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint32_t w0 = vfA[ks][ct][2 * c], w1 = vfA[ks][ct][2 * c + 1];
            const f32x4_t x = {bf_lo(w0) * bk[4 * c], bf_hi(w0) * bk[4 * c + 1],
                               bf_lo(w1) * bk[4 * c + 2], bf_hi(w1) * bk[4 * c + 3]};
            u32x2_t h2, l2;
            split4(x, h2, l2);
            bvh[ct][2 * c] = h2[0];
            bvh[ct][2 * c + 1] = h2[1];
            bvl[ct][2 * c] = l2[0];
            bvl[ct][2 * c + 1] = l2[1];
          }
#pragma unroll
        for (int t = 0; t < G::NT; ++t) {
          const u32x4_t kt = col_frag(Ot, ks, lT[t]);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) S[t][ct] = mfma16(kt, bvh[ct], S[t][ct]);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) S[t][ct] = mfma16(kt, bvl[ct], S[t][ct]);
        }
      }
    }

    // score tiles: the first half of the waves pass A's (dO V^T), the others
    // pass B's (Q K^T)
    {
      constexpr int HW = G::NW / 2;
      const bool passA = wave < HW;
      const int w = passA ? wave : wave - HW;
      for (int pr = w; pr < G::NPAIR; pr += HW) {
        if (passA)
          pair_tiles(pr, Ot, Vc, PAh, PAl);
        else
          pair_tiles(pr, Qt, Kc, PBh, PBl);
      }
    }

    lds_barrier();  // scores written; dO and Q tiles are dead
    if (more) {
      load_direct(dog, Ot, tc + C, n_next);
      load_direct(qg, Qt, tc + C, n_next);
    }

    // dK = pass A's output (its q is V), with G from registers
    outputs(Vc, sfh, sfl, vfA, PAh, PAl, dkg, tc, n);

    // G^T for pass B, through LDS in two rounds of D/2 rows (d_q): in round
    // rd the waves owning d_q rows rd D/2 .. write them (4 adjacent d_o per
    // write), then every wave reads the fragments of its own d_o columns
    u32x4_t gh[CT][G::KSD], gl[CT][G::KSD];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      if (col0 >= rd * (D / 2) && col0 < (rd + 1) * (D / 2)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int t = 0; t < G::NT; ++t) {
            const int j = col0 + vcol(ct, li) - rd * (D / 2);
            const int off = j * D + 8 * ((4 * (t >> 1) + lg) ^ swz_of<D>(j & 15)) + 4 * (t & 1);
            *reinterpret_cast<u32x2_t*>(Th + off) =
                u32x2_t{sfh[ct][t >> 1][2 * (t & 1)], sfh[ct][t >> 1][2 * (t & 1) + 1]};
            *reinterpret_cast<u32x2_t*>(Tl + off) =
                u32x2_t{sfl[ct][t >> 1][2 * (t & 1)], sfl[ct][t >> 1][2 * (t & 1) + 1]};
          }
      }
      lds_barrier();
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int ks = 0; ks < G::KSD / 2; ++ks) {
          gh[ct][rd * (G::KSD / 2) + ks] = col_frag(Th, ks, lV[ct]);
          gl[ct][rd * (G::KSD / 2) + ks] = col_frag(Tl, ks, lV[ct]);
        }
      if (rd == 0) lds_barrier();  // the half buffer is read before the second half rewrites it
    }
    // dV = pass B's output (its q is K), with G^T from the exchange
    outputs(Kc, gh, gl, vfB, PBh, PBl, dvg, tc, n);
  };

  if (tau0 < tau_end) {
    const int n0 = min(C, tau_end - tau0);
    load_direct(dog, Ot, tau0, n0);
    load_direct(qg, Qt, tau0, n0);
    load_direct(vg, V0, tau0, n0);
    load_direct(kg, K0, tau0, n0);
  }
  for (int tc = tau0; tc < tau_end; tc += 2 * C) {
    chunk(std::integral_constant<int, 0>{}, tc);
    if (tc + C < tau_end) chunk(std::integral_constant<int, 1>{}, tc + C);
  }
}

template <int C, int D>
hipError_t launch_cd(const BwdPass& p, const SeqTable& t, hipStream_t s) {
  const unsigned grid = (unsigned)(t.nseq > 0 ? p.H * p.G : p.B * p.H * p.nseg);
  hipLaunchKernelGGL((bwd_kv_bf16_kernel<C, D>), dim3(grid), dim3(D / 32 * 64), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_kv_bf16(const BwdPass& p, const SeqTable& t, hipStream_t s) {
  if (p.D == 128) {
    if (p.C == 64) return launch_cd<64, 128>(p, t, s);
    if (p.C == 32) return launch_cd<32, 128>(p, t, s);
  } else if (p.D == 64) {
    if (p.C == 64) return launch_cd<64, 64>(p, t, s);
    if (p.C == 32) return launch_cd<32, 64>(p, t, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
