// la_api.cpp -- the C ABI (include/lightning_la.h): argument validation,
// execution plan, launches on the caller's stream.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and needs no GPU.  No exception crosses the boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/lightning_la.h"
#include "la_internal.h"

// The scratch buffer of la_prefill_noalloc: segment start states, piece
// states and their tag live here instead of in a caller's workspace.  Every
// GPU the library runs on holds one until the process ends.  In host code
// the name `scratch` is a host-side stand-in, not a device address: kernels
// receive the address hipGetSymbolAddress returns for the current device.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Workgroups the bf16 prefill aims for: one per compute unit of an MI355X
// (256 CUs).  Fixed, so that la_workspace_bytes needs no device query.
constexpr int kTargetWorkgroups = 256;
// Upper bound on a piece of the segment pre-pass (tokens), and the number of
// pieces a segment is cut into at least: short segments get two pieces, so
// that the pre-pass has more workgroups of fewer chunks each (the 8K-token
// prefill: 36.6 us against 40.8 us for one piece per segment; four or more
// pieces were slower again).
constexpr int kMaxPieceLen = 1024;
constexpr int kMinPiecesPerSeg = 2;

// Workspace of a segmented plan: piece states, segment start states, then
// the tag that identifies them (la::WsTag).
struct Plan {
  int nseg = 1, seg_len = 0, piece_len = 0, npiece = 0;
  int G = 0;             // packed batches: segments per head
  bool prepass = false;  // some row has more than one segment
  size_t pieces_bytes = 0, seg_bytes = 0;
  size_t ws() const { return prepass ? pieces_bytes + seg_bytes + la::kTagBytes : 0; }
  size_t tag_off() const { return pieces_bytes + seg_bytes; }
  // The piece kernel runs one workgroup of 2 d threads per piece state: the
  // launch's 32-bit count of work-items bounds the number of pieces (a
  // segment of a prime number of chunks has one-chunk pieces, so the size
  // limits on B, H and N alone do not).
  bool pieces_fit(int d) const {
    if (!prepass) return true;
    const unsigned long long slots = pieces_bytes / ((size_t)d * d * sizeof(float));
    return slots * (2ull * d) < (1ull << 32);
  }
};

// The chunk length the kernels run: the bf16 kernels take chunks of 32, 64
// or 128 tokens, and a bf16 request for 16 runs in 32-token chunks (the chunk
// length changes only the rounding, never the result).
int run_chunk(la_dtype_t dt, int C) { return dt == LA_BF16 && C == 16 ? 32 : C; }

// The identity of the segment start states a pre-pass computes: sizes,
// direction, the k / v / slope / state_in pointers it reads and (packed
// batches) a hash of the sequence table.
la::WsTag make_tag(int B, int H, int N, int d, int C, bool reverse, const void* k,
                   const void* v, const float* slope, const float* state_in,
                   const la::SeqTable* t) {
  la::WsTag g{};
  auto lo = [](const void* x) { return (uint32_t)(uintptr_t)x; };
  auto hi = [](const void* x) { return (uint32_t)((uint64_t)(uintptr_t)x >> 32); };
  uint32_t h = 2166136261u;  // FNV-1a over nseq and cu
  if (t && t->nseq > 0) {
    auto mix = [&](uint32_t x) {
      for (int b = 0; b < 4; ++b) h = (h ^ ((x >> (8 * b)) & 0xffu)) * 16777619u;
    };
    mix((uint32_t)t->nseq);
    for (int s = 0; s <= t->nseq; ++s) mix((uint32_t)t->cu[s]);
  }
  const uint32_t w[la::kTagWords] = {0x4C415447u, (uint32_t)B, (uint32_t)H, (uint32_t)N,
                                      (uint32_t)d, (uint32_t)C, reverse ? 1u : 0u, lo(k), hi(k),
                                      lo(v), hi(v), lo(slope), hi(slope), lo(state_in),
                                      hi(state_in), h};
  for (int i = 0; i < la::kTagWords; ++i) g.w[i] = w[i];
  return g;
}

// The uniform layout's (empty) sequence table.
const la::SeqTable& uniform_table() {
  static const la::SeqTable t{};
  return t;
}

// Largest piece length (a multiple of C dividing seg_len, at most
// kMaxPieceLen tokens, and at most half the segment when it holds two or
// more chunks).
int piece_len_for(int seg_len, int C) {
  const int seg_chunks = seg_len / C;
  int pc = 1;
  for (int x = 1; x <= seg_chunks; ++x)
    if (seg_chunks % x == 0 && (long long)x * C <= kMaxPieceLen &&
        (x == 1 || seg_chunks / x >= kMinPiecesPerSeg))
      pc = x;
  return pc * C;
}

bool d_ok(la_dtype_t dt, int d) {
  if (dt == LA_BF16) return d == 64 || d == 128;
  return d == 16 || d == 32 || d == 64 || d == 128;
}
bool c_ok(int C) { return C == 16 || C == 32 || C == 64 || C == 128; }

Plan make_plan(la_dtype_t dt, int B, int H, int N, int d, int C) {
  Plan p;
  if (dt != LA_BF16) {
    p.seg_len = N;
    return p;
  }
  const long long heads = (long long)B * H;
  const int nchunks = (N + C - 1) / C;
  int nseg = 1;
  if (heads < kTargetWorkgroups) nseg = (int)((kTargetWorkgroups + heads - 1) / heads);
  if (nseg > nchunks) nseg = nchunks;
  const int seg_chunks = (nchunks + nseg - 1) / nseg;
  nseg = (nchunks + seg_chunks - 1) / seg_chunks;
  p.nseg = nseg;
  p.seg_len = seg_chunks * C;
  if (nseg > 1) {
    p.prepass = true;
    p.piece_len = piece_len_for(p.seg_len, C);
    p.npiece = (nseg - 1) * (p.seg_len / p.piece_len);
    const size_t dd = (size_t)d * d * sizeof(float);
    p.pieces_bytes = (size_t)heads * p.npiece * dd;
    p.seg_bytes = (size_t)heads * nseg * dd;
  }
  return p;
}

// The same segments with fewer, longer pieces, until the workspace fits in
// cap bytes (the piece length stays a multiple of C dividing the segment
// length); false if even one piece per segment does not fit.  The piece
// length changes only the rounding of the segment start states.
bool fit_plan(Plan* p, long long rows, int d, int C, size_t cap) {
  if (p->ws() <= cap) return true;
  const int seg_chunks = p->seg_len / C;
  const size_t dd = (size_t)d * d * sizeof(float);
  for (int pc = p->piece_len / C + 1; pc <= seg_chunks; ++pc) {
    if (seg_chunks % pc) continue;
    p->piece_len = pc * C;
    p->npiece = (p->nseg - 1) * (seg_chunks / pc);
    p->pieces_bytes = (size_t)rows * p->npiece * dd;
    if (p->ws() <= cap) return true;
  }
  return false;
}

// Packed batch (cu already validated): segments of seg_len tokens, chosen so
// that the H * sum_s ceil(n_s / seg_len) workgroups fill the GPU; every
// sequence has at least one segment.  Sequences are scheduled longest first
// (ties in sequence order).  Fills t.
Plan make_plan_packed(la_dtype_t dt, int H, int d, int C, int nseq, const int* cu,
                      la::SeqTable* t) {
  Plan p;
  t->nseq = nseq;
  t->T = cu[nseq];
  for (int s = 0; s <= nseq; ++s) t->cu[s] = cu[s];
  const long long T = cu[nseq];
  long long L = C;
  if (dt == LA_BF16) {
    const long long per_wg = ((long long)H * T + kTargetWorkgroups - 1) / kTargetWorkgroups;
    L = ((per_wg + C - 1) / C) * C;
    if (L < C) L = C;
  } else {
    L = T > 0 ? T : 1;  // the fp32 path runs every sequence whole
  }
  for (int i = 0; i < nseq; ++i) t->ord[i] = i;
  std::stable_sort(t->ord, t->ord + nseq,
                   [&](int a, int b) { return cu[a + 1] - cu[a] > cu[b + 1] - cu[b]; });
  int g = 0;
  bool multi = false;
  for (int i = 0; i < nseq; ++i) {
    const int s = t->ord[i];
    t->g0[i] = g;
    const long long n = cu[s + 1] - cu[s];
    const int ns = n > L ? (int)((n + L - 1) / L) : 1;
    multi = multi || ns > 1;
    g += ns;
  }
  t->g0[nseq] = g;
  p.G = g;
  p.seg_len = (int)L;
  p.nseg = 0;  // per sequence: g0[s+1] - g0[s]
  if (multi) {
    p.prepass = true;
    p.piece_len = piece_len_for(p.seg_len, C);
    const size_t dd = (size_t)d * d * sizeof(float);
    p.pieces_bytes = (size_t)H * g * (p.seg_len / p.piece_len) * dd;
    p.seg_bytes = (size_t)H * g * dd;
  }
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

la_status_t hip_status(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

// Device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

la_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return LA_OK;
}

// Shape checks shared by prefill and its backward.
la_status_t check_seq(la_dtype_t dt, int B, int H, int N, int d, int C) {
  if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_BAD_DTYPE;
  if (B < 1 || H < 1 || N < 1 || !d_ok(dt, d) || !c_ok(C)) return LA_ERR_BAD_SHAPE;
  // int indexing of token offsets inside the kernels (below 2^30), and a
  // launch's 32-bit count of work-items: at most 24 workgroups of 256
  // threads per row (the fp32 short-row kernel), so B H rows below 2^19
  if ((long long)B * H * N > (1LL << 31) / 2) return LA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 19)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

la::FwdPass make_fwd(const Plan& pl, int B, int H, int N, int d, int C, const void* q,
                     const void* k, const void* v, const float* slope, const float* state_in,
                     void* o, float* state_out, bool reverse, void* workspace) {
  // (packed batches: B = 1, N = T, and the sequence table travels beside)
  la::FwdPass fp{};
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.o = o;
  fp.slope = slope;
  fp.state_in = state_in;
  fp.state_out = state_out;
  fp.B = B;
  fp.H = H;
  fp.N = N;
  fp.D = d;
  fp.C = C;
  fp.reverse = reverse;
  fp.seg_len = pl.seg_len;
  fp.nseg = pl.nseg;
  fp.G = pl.G;
  if (pl.prepass) fp.seg_states = (const float*)((const char*)workspace + pl.pieces_bytes);
  return fp;
}

// A pass that reads segment start states an earlier call left in the
// workspace: it checks their tag first.
void expect_states(la::FwdPass* fp, const Plan& pl, void* workspace, const la::WsTag& tag) {
  if (!pl.prepass) return;
  fp->tag = (const uint32_t*)((const char*)workspace + pl.tag_off());
  fp->tag_expect = tag;
}

// Segment start states (piece kernel + scan); nothing when there is one segment.
la_status_t run_prepass(const Plan& pl, const la::SeqTable& t, int B, int H, int N, int d, int C,
                        const void* k, const void* v, const float* slope, const float* state_in,
                        bool reverse, void* workspace, hipStream_t s) {
  if (!pl.prepass) return LA_OK;
  float* pieces = (float*)workspace;
  float* seg_states = (float*)((char*)workspace + pl.pieces_bytes);
  la::PiecePass pp{};
  pp.k = k;
  pp.v = v;
  pp.slope = slope;
  pp.pieces = pieces;
  pp.B = B;
  pp.H = H;
  pp.N = N;
  pp.D = d;
  pp.C = C;
  pp.reverse = reverse;
  pp.piece_len = pl.piece_len;
  pp.npiece = pl.npiece;
  pp.seg_len = pl.seg_len;
  pp.nseg = pl.nseg;
  pp.G = pl.G;
  la_status_t st = hip_status(la::launch_pieces_bf16(pp, t, s));
  if (st != LA_OK) return st;
  la::ScanPass sp{};
  sp.pieces = pieces;
  sp.state_in = state_in;
  sp.seg_states = seg_states;
  sp.slope = slope;
  sp.B = B;
  sp.H = H;
  sp.N = N;
  sp.D = d;
  sp.piece_len = pl.piece_len;
  sp.npiece = pl.npiece;
  sp.seg_len = pl.seg_len;
  sp.nseg = pl.nseg;
  sp.G = pl.G;
  sp.tag = (uint32_t*)((char*)workspace + pl.tag_off());
  sp.tag_value = make_tag(B, H, N, d, C, reverse, k, v, slope, state_in, &t);
  return hip_status(la::launch_scan(sp, t, s));
}

la_status_t run_main(la_dtype_t dt, const la::FwdPass& fp, const la::SeqTable& t,
                     hipStream_t s) {
  if (dt == LA_F32) return hip_status(la::launch_fwd_f32(fp, t, s));
  return hip_status(la::launch_fwd_bf16(fp, t, s));
}

// One causal (or, with reverse, anti-causal) pass with its segment pre-pass.
la_status_t run_pass(la_dtype_t dt, const Plan& pl, const la::SeqTable& t, int B, int H, int N,
                     int d, int C, const void* q, const void* k, const void* v,
                     const float* slope, const float* state_in, void* o, float* state_out,
                     bool reverse, void* workspace, hipStream_t s) {
  la_status_t st =
      run_prepass(pl, t, B, H, N, d, C, k, v, slope, state_in, reverse, workspace, s);
  if (st != LA_OK) return st;
  return run_main(dt, make_fwd(pl, B, H, N, d, C, q, k, v, slope, state_in, o, state_out,
                               reverse, workspace),
                  t, s);
}

// The passes of the backward.  dq_t = S_t dout_t is the causal pass
// with (q, k, v) -> (dout, v, k).  dk_s = sum_{t>=s} lambda^(t-s) (v_s .
// dout_t) q_t is the anti-causal pass (v, dout, q) and dv_s = sum_{t>=s}
// lambda^(t-s) (k_s . q_t) dout_t the anti-causal pass (k, q, dout).  The
// states of the dv pass (sums of q dout^T) are the transposes of the dk
// pass's (sums of dout q^T), so the dv pass reads the dk pass's segment
// start states transposed instead of running its own pre-pass.
// With fwd_states, the workspace holds the forward's segment start states
// (sums of k v^T); the dq pass's are their transposes.
la_status_t run_bwd(la_dtype_t dt, const Plan& pl, const la::SeqTable& t, int B, int H, int N,
                    int d, int C, const void* q, const void* k, const void* v, const void* dout,
                    const float* slope, void* dq, void* dk, void* dv, void* workspace,
                    hipStream_t s, bool fwd_states = false) {
  la_status_t st;
  if (fwd_states) {
    la::FwdPass fp =
        make_fwd(pl, B, H, N, d, C, dout, v, k, slope, nullptr, dq, nullptr, false, workspace);
    fp.seg_states_transposed = true;
    // the forward's states: from (k, v) with no initial state
    expect_states(&fp, pl, workspace, make_tag(B, H, N, d, C, false, k, v, slope, nullptr, &t));
    st = run_main(dt, fp, t, s);
  } else {
    st = run_pass(dt, pl, t, B, H, N, d, C, dout, v, k, slope, nullptr, dq, nullptr, false,
                  workspace, s);
  }
  if (st != LA_OK) return st;
  if (dt == LA_BF16) {
    // bf16: dk and dv in one fused reverse pass with one state, after the
    // (v, dout, q) pass's segment pre-pass.  The fused pass holds four tiles,
    // two score sets and the transposed state in LDS, which fits chunks of up
    // to 64 tokens; with C = 128 it runs 64-token chunks inside the same
    // segments (segment lengths are multiples of C; the chunk length changes
    // only the rounding).
    st = run_prepass(pl, t, B, H, N, d, C, dout, q, slope, nullptr, true, workspace, s);
    if (st != LA_OK) return st;
    la::BwdPass bp{};
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.dout = dout;
    bp.dk = dk;
    bp.dv = dv;
    bp.slope = slope;
    bp.B = B;
    bp.H = H;
    bp.N = N;
    bp.D = d;
    bp.C = C < 64 ? C : 64;
    bp.seg_len = pl.seg_len;
    bp.nseg = pl.nseg;
    bp.G = pl.G;
    if (pl.prepass) bp.seg_states = (const float*)((const char*)workspace + pl.pieces_bytes);
    return hip_status(la::launch_bwd_kv_bf16(bp, t, s));
  }
  st = run_pass(dt, pl, t, B, H, N, d, C, v, dout, q, slope, nullptr, dk, nullptr, true,
                workspace, s);
  if (st != LA_OK) return st;
  la::FwdPass fp =
      make_fwd(pl, B, H, N, d, C, k, q, dout, slope, nullptr, dv, nullptr, true, workspace);
  fp.seg_states_transposed = true;
  return run_main(dt, fp, t, s);
}

// Checks of la_prefill / la_prefill_main (q and o may be null for the prepass).
la_status_t check_prefill(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                          const void* k, const void* v, const float* slope,
                          const float* state_in, const void* o, const float* state_out,
                          const void* workspace, size_t workspace_bytes, bool need_qo,
                          Plan* plan, bool own_workspace = false) {
  la_status_t st = check_seq(dt, B, H, N, d, C);
  if (st != LA_OK) return st;
  if (!k || !v || !slope || (need_qo && (!q || !o))) return LA_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state_in) ||
      !aligned16(state_out) || ((uintptr_t)slope & 3u))
    return LA_ERR_ALIGNMENT;
  const size_t esz = dt == LA_BF16 ? 2 : 4;
  const size_t tb = (size_t)B * H * N * d * esz;
  const size_t sb = (size_t)B * H * d * d * sizeof(float);
  if (o && (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb)))
    return LA_ERR_ALIAS;
  if (state_in && state_out && state_in != state_out && overlap(state_in, sb, state_out, sb))
    return LA_ERR_ALIAS;
  if (state_out && ((q && overlap(state_out, sb, q, tb)) || overlap(state_out, sb, k, tb) ||
                    overlap(state_out, sb, v, tb) || (o && overlap(state_out, sb, o, tb))))
    return LA_ERR_ALIAS;
  *plan = make_plan(dt, B, H, N, d, C);
  if (own_workspace) return LA_OK;  // the caller of check_prefill provides it
  if (!plan->pieces_fit(d)) return LA_ERR_UNSUPPORTED;
  if (plan->ws() > 0 && (!workspace || workspace_bytes < plan->ws())) return LA_ERR_WORKSPACE;
  if (plan->ws() > 0 && !aligned16(workspace)) return LA_ERR_ALIGNMENT;
  return LA_OK;
}

// Checks shared by the packed-batch calls; fills t and the plan.
la_status_t check_packed(la_dtype_t dt, int H, int d, int C, int nseq, const int* cu,
                         la::SeqTable* t, Plan* plan) {
  if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_BAD_DTYPE;
  if (H < 1 || nseq < 1 || !d_ok(dt, d) || !c_ok(C)) return LA_ERR_BAD_SHAPE;
  // at most kMaxSeqs * H rows of 8 fp32 column slices of 256 threads: the
  // launch's 32-bit count of work-items
  if (nseq > la::kMaxSeqs || H > 4096) return LA_ERR_UNSUPPORTED;
  if (!cu) return LA_ERR_NULL_POINTER;
  if (cu[0] != 0) return LA_ERR_BAD_SHAPE;
  for (int s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s]) return LA_ERR_BAD_SHAPE;
  if ((long long)H * cu[nseq] > (1LL << 31) / 2) return LA_ERR_UNSUPPORTED;
  *plan = make_plan_packed(dt, H, d, C, nseq, cu, t);
  if (!plan->pieces_fit(d)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

la_status_t check_workspace(const Plan& pl, const void* workspace, size_t workspace_bytes) {
  if (pl.ws() > 0 && (!workspace || workspace_bytes < pl.ws())) return LA_ERR_WORKSPACE;
  if (pl.ws() > 0 && !aligned16(workspace)) return LA_ERR_ALIGNMENT;
  return LA_OK;
}

// la_prefill_bwd, and with fwd_states la_prefill_bwd_reuse (the workspace
// holds the forward's segment start states; only the bf16 path has them)
la_status_t prefill_bwd(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                        const void* k, const void* v, const void* dout, const float* slope,
                        const float* state_in, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, void* stream, bool fwd_states) {
  C = run_chunk(dt, C);
  try {
    la_status_t st = check_seq(dt, B, H, N, d, C);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !dout || !slope || !dq || !dk || !dv) return LA_ERR_NULL_POINTER;
    if (state_in) return LA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)slope & 3u))
      return LA_ERR_ALIGNMENT;
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const size_t tb = (size_t)B * H * N * d * esz;
    const void* ins[4] = {q, k, v, dout};
    void* outs[3] = {dq, dk, dv};
    for (int a = 0; a < 3; ++a) {
      for (int b = 0; b < 4; ++b)
        if (overlap(outs[a], tb, ins[b], tb)) return LA_ERR_ALIAS;
      for (int b = a + 1; b < 3; ++b)
        if (overlap(outs[a], tb, outs[b], tb)) return LA_ERR_ALIAS;
    }
    const Plan pl = make_plan(dt, B, H, N, d, C);
    if (!pl.pieces_fit(d)) return LA_ERR_UNSUPPORTED;
    if (pl.ws() > 0 && (!workspace || workspace_bytes < pl.ws())) return LA_ERR_WORKSPACE;
    if (pl.ws() > 0 && !aligned16(workspace)) return LA_ERR_ALIGNMENT;
    return run_bwd(dt, pl, uniform_table(), B, H, N, d, C, q, k, v, dout, slope, dq, dk, dv,
                   workspace, (hipStream_t)stream, fwd_states && dt == LA_BF16);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

// la_prefill_bwd_varlen, and with fwd_states la_prefill_bwd_varlen_reuse
la_status_t prefill_bwd_varlen(la_dtype_t dt, int H, int d, int C, int nseq, const int* cu_seqlens,
                               const void* q, const void* k, const void* v, const void* dout,
                               const float* slope, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream,
                               bool fwd_states) {
  C = run_chunk(dt, C);
  try {
    la::SeqTable t;
    Plan pl;
    la_status_t st = check_packed(dt, H, d, C, nseq, cu_seqlens, &t, &pl);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !dout || !slope || !dq || !dk || !dv) return LA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)slope & 3u))
      return LA_ERR_ALIGNMENT;
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const size_t tb = (size_t)H * t.T * d * esz;
    const void* ins[4] = {q, k, v, dout};
    void* outs[3] = {dq, dk, dv};
    for (int a = 0; a < 3; ++a) {
      for (int b = 0; b < 4; ++b)
        if (overlap(outs[a], tb, ins[b], tb)) return LA_ERR_ALIAS;
      for (int b = a + 1; b < 3; ++b)
        if (overlap(outs[a], tb, outs[b], tb)) return LA_ERR_ALIAS;
    }
    st = check_workspace(pl, workspace, workspace_bytes);
    if (st != LA_OK) return st;
    // the three passes of la_prefill_bwd, each sequence reversed in place
    return run_bwd(dt, pl, t, 1, H, t.T, d, C, q, k, v, dout, slope, dq, dk, dv, workspace,
                   (hipStream_t)stream, fwd_states && dt == LA_BF16);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

}  // namespace

extern "C" {

la_status_t la_prefill(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                       const void* k, const void* v, const float* slope, const float* state_in,
                       void* o, float* state_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  C = run_chunk(dt, C);
  try {
    Plan pl;
    const la_status_t st = check_prefill(dt, B, H, N, d, C, q, k, v, slope, state_in, o,
                                         state_out, workspace, workspace_bytes, true, &pl);
    if (st != LA_OK) return st;
    return run_pass(dt, pl, uniform_table(), B, H, N, d, C, q, k, v, slope, state_in, o,
                    state_out, false, workspace, (hipStream_t)stream);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_prefill_noalloc(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                               const void* k, const void* v, const float* slope,
                               const float* state_in, void* o, float* state_out, void* stream) {
  C = run_chunk(dt, C);
  try {
    Plan pl;
    la_status_t st = check_prefill(dt, B, H, N, d, C, q, k, v, slope, state_in, o, state_out,
                                   nullptr, 0, true, &pl, true);
    if (st != LA_OK) return st;
    if (!fit_plan(&pl, (long long)B * H, d, C, kScratchBytes)) return LA_ERR_WORKSPACE;
    if (!pl.pieces_fit(d)) return LA_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (pl.ws() > 0) {
      st = scratch_address(&ws);
      if (st != LA_OK) return st;
    }
    return run_pass(dt, pl, uniform_table(), B, H, N, d, C, q, k, v, slope, state_in, o,
                    state_out, false, ws, (hipStream_t)stream);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_prefill_gated(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                             const void* k, const void* v, const float* slope,
                             const float* state_in, const void* gate, const float* norm_weight,
                             float eps, void* y, float* state_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  C = run_chunk(dt, C);
  try {
    Plan pl;
    const la_status_t st = check_prefill(dt, B, H, N, d, C, q, k, v, slope, state_in, y,
                                         state_out, workspace, workspace_bytes, true, &pl);
    if (st != LA_OK) return st;
    if (!gate || !norm_weight) return LA_ERR_NULL_POINTER;
    if (!aligned16(gate) || ((uintptr_t)norm_weight & 3u)) return LA_ERR_ALIGNMENT;
    if (!(eps >= 0.f) || eps > 3.0e38f) return LA_ERR_BAD_SHAPE;  // also rejects NaN
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const size_t tb = (size_t)B * H * N * d * esz;
    if (overlap(y, tb, gate, tb) || overlap(y, tb, norm_weight, (size_t)H * d * sizeof(float)))
      return LA_ERR_ALIAS;
    if (state_out && (overlap(state_out, (size_t)B * H * d * d * sizeof(float), gate, tb)))
      return LA_ERR_ALIAS;
    const hipStream_t s = (hipStream_t)stream;
    la_status_t r = run_prepass(pl, uniform_table(), B, H, N, d, C, k, v, slope, state_in, false,
                                workspace, s);
    if (r != LA_OK) return r;
    la::FwdPass fp = make_fwd(pl, B, H, N, d, C, q, k, v, slope, state_in, y, state_out, false,
                              workspace);
    fp.gate = gate;
    fp.norm_w = norm_weight;
    fp.eps = eps;
    return run_main(dt, fp, uniform_table(), s);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_prefill_prepass(la_dtype_t dt, int B, int H, int N, int d, int C, const void* k,
                               const void* v, const float* slope, const float* state_in,
                               void* workspace, size_t workspace_bytes, void* stream) {
  C = run_chunk(dt, C);
  try {
    Plan pl;
    const la_status_t st = check_prefill(dt, B, H, N, d, C, nullptr, k, v, slope, state_in,
                                         nullptr, nullptr, workspace, workspace_bytes, false, &pl);
    if (st != LA_OK) return st;
    return run_prepass(pl, uniform_table(), B, H, N, d, C, k, v, slope, state_in, false,
                       workspace, (hipStream_t)stream);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_prefill_main(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                            const void* k, const void* v, const float* slope,
                            const float* state_in, void* o, float* state_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  C = run_chunk(dt, C);
  try {
    Plan pl;
    const la_status_t st = check_prefill(dt, B, H, N, d, C, q, k, v, slope, state_in, o,
                                         state_out, workspace, workspace_bytes, true, &pl);
    if (st != LA_OK) return st;
    la::FwdPass fp =
        make_fwd(pl, B, H, N, d, C, q, k, v, slope, state_in, o, state_out, false, workspace);
    // the states of la_prefill_prepass with the same arguments
    expect_states(&fp, pl, workspace,
                  make_tag(B, H, N, d, C, false, k, v, slope, state_in, &uniform_table()));
    return run_main(dt, fp, uniform_table(), (hipStream_t)stream);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_decode_step(la_dtype_t dt, int B, int H, int d, const void* q, const void* k,
                           const void* v, const float* slope, float* state, void* o,
                           void* stream) {
  try {
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_BAD_DTYPE;
    if (B < 1 || H < 1 || !d_ok(dt, d)) return LA_ERR_BAD_SHAPE;
    // B H workgroups of at most 1024 threads: the launch's 32-bit count of work-items
    if ((long long)B * H > (1LL << 21)) return LA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !slope || !state || !o) return LA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) ||
        !aligned16(o) || ((uintptr_t)slope & 3u))
      return LA_ERR_ALIGNMENT;
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const size_t tb = (size_t)B * H * d * esz;
    const size_t sb = (size_t)B * H * d * d * sizeof(float);
    if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) ||
        overlap(o, tb, state, sb) || overlap(state, sb, q, tb) || overlap(state, sb, k, tb) ||
        overlap(state, sb, v, tb))
      return LA_ERR_ALIAS;
    return hip_status(la::launch_decode(dt == LA_BF16, B, H, d, q, k, v, slope, state, o,
                                        (hipStream_t)stream));
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_decode_tokens(la_dtype_t dt, int B, int H, int K, int d, const void* q,
                             const void* k, const void* v, const float* slope, float* state,
                             void* o, void* stream) {
  try {
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_BAD_DTYPE;
    if (B < 1 || H < 1 || K < 1 || !d_ok(dt, d)) return LA_ERR_BAD_SHAPE;
    if (K > 128) return LA_ERR_UNSUPPORTED;
    // the limits of la_prefill, whose kernels serve K > 16
    if ((long long)B * H * K > (1LL << 31) / 2) return LA_ERR_UNSUPPORTED;
    if ((long long)B * H > (1LL << 19)) return LA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !slope || !state || !o) return LA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) ||
        !aligned16(o) || ((uintptr_t)slope & 3u))
      return LA_ERR_ALIGNMENT;
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const size_t tb = (size_t)B * H * K * d * esz;
    const size_t sb = (size_t)B * H * d * d * sizeof(float);
    if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) ||
        overlap(o, tb, state, sb) || overlap(state, sb, q, tb) || overlap(state, sb, k, tb) ||
        overlap(state, sb, v, tb))
      return LA_ERR_ALIAS;
    // A few tokens: the recurrence on the streamed state (vector ALU).
    if (K <= la::kDecodeTokensMax)
      return hip_status(la::launch_decode_tokens(dt == LA_BF16, B, H, K, d, q, k, v, slope,
                                                 state, o, (hipStream_t)stream));
    // More: one chunk of the prefill (the smallest chunk length that holds
    // them), continued from and written back to the same state: one segment
    // per row, so no workspace.
    const int C = dt == LA_F32 ? 64 : (K <= 32 ? 32 : K <= 64 ? 64 : 128);
    Plan pl = make_plan(dt, B, H, K, d, C);
    if (pl.prepass) return LA_ERR_HIP;  // cannot happen: K <= C gives one segment
    return run_main(dt,
                    make_fwd(pl, B, H, K, d, C, q, k, v, slope, state, o, state, false, nullptr),
                    uniform_table(), (hipStream_t)stream);
  } catch (...) {
    return LA_ERR_HIP;
  }
}


la_status_t la_prefill_bwd(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                           const void* k, const void* v, const void* dout, const float* slope,
                           const float* state_in, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_bwd(dt, B, H, N, d, C, q, k, v, dout, slope, state_in, dq, dk, dv, workspace,
                     workspace_bytes, stream, false);
}

la_status_t la_prefill_bwd_reuse(la_dtype_t dt, int B, int H, int N, int d, int C, const void* q,
                                 const void* k, const void* v, const void* dout,
                                 const float* slope, const float* state_in, void* dq, void* dk,
                                 void* dv, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return prefill_bwd(dt, B, H, N, d, C, q, k, v, dout, slope, state_in, dq, dk, dv, workspace,
                     workspace_bytes, stream, true);
}

la_status_t la_prefill_varlen(la_dtype_t dt, int H, int d, int C, int nseq,
                              const int* cu_seqlens, const void* q, const void* k,
                              const void* v, const float* slope, const float* state_in, void* o,
                              float* state_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  C = run_chunk(dt, C);
  try {
    la::SeqTable t;
    Plan pl;
    la_status_t st = check_packed(dt, H, d, C, nseq, cu_seqlens, &t, &pl);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !o || !slope) return LA_ERR_NULL_POINTER;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state_in) ||
        !aligned16(state_out) || ((uintptr_t)slope & 3u))
      return LA_ERR_ALIGNMENT;
    const size_t esz = dt == LA_BF16 ? 2 : 4;
    const size_t tb = (size_t)H * t.T * d * esz;
    const size_t sb = (size_t)nseq * H * d * d * sizeof(float);
    if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb))
      return LA_ERR_ALIAS;
    if (state_in && state_out && state_in != state_out && overlap(state_in, sb, state_out, sb))
      return LA_ERR_ALIAS;
    if (state_out && (overlap(state_out, sb, q, tb) || overlap(state_out, sb, k, tb) ||
                      overlap(state_out, sb, v, tb) || overlap(state_out, sb, o, tb)))
      return LA_ERR_ALIAS;
    st = check_workspace(pl, workspace, workspace_bytes);
    if (st != LA_OK) return st;
    return run_pass(dt, pl, t, 1, H, t.T, d, C, q, k, v, slope, state_in, o, state_out, false,
                    workspace, (hipStream_t)stream);
  } catch (...) {
    return LA_ERR_HIP;
  }
}

la_status_t la_prefill_bwd_varlen(la_dtype_t dt, int H, int d, int C, int nseq,
                                  const int* cu_seqlens, const void* q, const void* k,
                                  const void* v, const void* dout, const float* slope, void* dq,
                                  void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return prefill_bwd_varlen(dt, H, d, C, nseq, cu_seqlens, q, k, v, dout, slope, dq, dk, dv,
                            workspace, workspace_bytes, stream, false);
}

la_status_t la_prefill_bwd_varlen_reuse(la_dtype_t dt, int H, int d, int C, int nseq,
                                        const int* cu_seqlens, const void* q, const void* k,
                                        const void* v, const void* dout, const float* slope,
                                        void* dq, void* dk, void* dv, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return prefill_bwd_varlen(dt, H, d, C, nseq, cu_seqlens, q, k, v, dout, slope, dq, dk, dv,
                            workspace, workspace_bytes, stream, true);
}

size_t la_workspace_bytes_varlen(int op, la_dtype_t dt, int H, int d, int C, int nseq,
                                 const int* cu_seqlens) {
  C = run_chunk(dt, C);
  if (op != 0 && op != 1) return (size_t)-1;
  la::SeqTable t;
  Plan pl;
  if (check_packed(dt, H, d, C, nseq, cu_seqlens, &t, &pl) != LA_OK) return (size_t)-1;
  return pl.ws();
}

size_t la_workspace_bytes(int op, la_dtype_t dt, int B, int H, int N, int d, int C) {
  C = run_chunk(dt, C);
  if (op != 0 && op != 1) return (size_t)-1;
  if (check_seq(dt, B, H, N, d, C) != LA_OK) return (size_t)-1;
  return make_plan(dt, B, H, N, d, C).ws();
}

la_status_t la_probe_stream_rmw(float* x, size_t n, float a, int load_policy, int store_policy,
                                void* stream) {
  try {
    if (!x) return LA_ERR_NULL_POINTER;
    if (load_policy != 0 && load_policy != la::kCpolNt) return LA_ERR_UNSUPPORTED;
    if (store_policy != 0 && store_policy != la::kCpolNt && store_policy != la::kCpolSc1)
      return LA_ERR_UNSUPPORTED;
    // one workgroup of 256 threads per 1024 float4: the launch's 32-bit count of
    // work-items holds at most 2^24 - 1 workgroups
    if (n == 0 || n % 4 != 0) return LA_ERR_BAD_SHAPE;
    if (n / 4 > (size_t)((1u << 24) - 1) * 1024) return LA_ERR_UNSUPPORTED;
    if (!aligned16(x)) return LA_ERR_ALIGNMENT;
    return hip_status(
        la::launch_stream_rmw(x, n, a, load_policy, store_policy, (hipStream_t)stream));
  } catch (...) {
    return LA_ERR_HIP;
  }
}

const char* la_status_string(la_status_t s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case LA_ERR_BAD_SHAPE: return "bad shape: B, H, N must be >= 1; d or C not supported";
    case LA_ERR_BAD_DTYPE: return "bad dtype: expected LA_F32 or LA_BF16";
    case LA_ERR_UNSUPPORTED: return "request not supported by this library version";
    case LA_ERR_WORKSPACE: return "workspace missing or smaller than la_workspace_bytes()";
    case LA_ERR_HIP: return "a HIP launch or runtime call failed";
    case LA_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case LA_ERR_ALIAS: return "an output overlaps an input it must not overlap";
  }
  return "unknown status";
}

int la_abi_version(void) { return LA_ABI_VERSION; }

}  // extern "C"
