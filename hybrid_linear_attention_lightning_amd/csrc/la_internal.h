// la_internal.h -- host-side interface between the C ABI (la_api.cpp) and the
// kernel launchers.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

// Packed (variable-length) batches.  nseq == 0: the uniform layout, token
// tensors [B][H][N][D] and states [B][H][D][D].  nseq > 0: token tensors
// [H][T][D] holding nseq sequences back to back, sequence s on tokens
// cu[s] .. cu[s+1]-1 of every head, states [nseq][H][D][D]; each sequence is
// its own recurrence from its own initial state.
// Work is scheduled longest sequence first: schedule position i holds
// sequence ord[i] (lengths non-increasing in i).  Segments (see FwdPass) are
// numbered per head in schedule order: position i owns segments
// g0[i] .. g0[i+1]-1, at least one even for an empty sequence.  The table
// travels to the kernels by value, as a kernel argument (3 KB).
constexpr int kMaxSeqs = 256;
struct SeqTable {
  int nseq;
  int T;
  int cu[kMaxSeqs + 1];
  int g0[kMaxSeqs + 1];
  int ord[kMaxSeqs];
};

// Identity of the segment start states a pre-pass leaves in a workspace:
// the sizes, direction and input pointers they were computed from.  The
// scan kernel writes it behind the states; a pass that reads states computed
// by an earlier call (la_prefill_main, the _reuse backward) compares it with
// the identity it expects and, on a mismatch, starts every row from NaN, so
// that a wrong workspace gives NaN outputs instead of plausible wrong ones.
constexpr int kTagWords = 16;
constexpr size_t kTagBytes = 256;  // tag area at the end of the workspace
struct WsTag {
  uint32_t w[kTagWords];
};

// One causal chunked pass o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s
// (+ lambda^(t+1) q_t^T S_in) over [B][H][N][D] token tensors.  With
// reverse = true the pass runs over the time-reversed sequence (token
// N-1-tau at position tau) and writes its output in the same reversed
// positions, which gives the anti-causal sums the backward needs.
struct FwdPass {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* slope;
  const float* state_in;   // [B][H][D][D] or nullptr (zero)
  float* state_out;        // [B][H][D][D] or nullptr
  int B, H, N, D, C;
  bool reverse;
  // Segment parallelism: the sequence is cut into nseg segments of seg_len
  // tokens (a multiple of C); when a row has two or more segments, segment r
  // starts from seg_states[b][h][r], where entry 0 is the scan kernel's copy
  // of state_in; a row of one segment reads state_in itself.  Packed
  // batches: G segments per head, seg_states[h][g].
  int seg_len;
  int nseg;
  int G;
  const float* seg_states;  // [B][H][nseg][D][D] / [H][G][D][D], or nullptr
  // The segment start states are stored transposed (S^T): a pass whose
  // states are the transposes of another pass's reuses that pass's pre-pass.
  bool seg_states_transposed;
  // States from an earlier call: check the workspace tag (tag != nullptr)
  // against tag_expect before using them.
  const uint32_t* tag;
  WsTag tag_expect;
  // Output epilogue (forward only), when gate != nullptr:
  // o = RMSNorm_head(o) * norm_w[h] * sigmoid(gate), gate laid out like o.
  const void* gate;
  const float* norm_w;  // [H][D]
  float eps;
};

// The fused reverse pass of the backward (dk and dv together, bf16, C <= 64):
// token tensors and segment plan as for FwdPass; seg_states holds the segment
// start states of the (v, dout, q) pass, i.e. sums of dout q^T.
struct BwdPass {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dk;
  void* dv;
  const float* slope;
  int B, H, N, D, C;
  int seg_len, nseg, G;
  const float* seg_states;
};

// Per-piece local states for the segment pre-pass:
// piece p of length piece_len ends at token e_p = min(N, (p+1) piece_len) - 1
// and holds sum_{t in piece} lambda^(e_p - t) k_t v_t^T.
struct PiecePass {
  const void* k;
  const void* v;
  const float* slope;
  float* pieces;  // [B][H][npiece][D][D]; packed: [H][G][seg_len/piece_len][D][D]
  int B, H, N, D, C;
  bool reverse;
  int piece_len, npiece;
  int seg_len, nseg;  // a piece is computed only if some segment start needs it
  int G;              // packed batches: segments per head
};

// Segment start states from the piece states (and state_in).  Entry r = 0 of
// each row that has two or more segments receives a copy of its state_in (or
// zeros), so that no workgroup of the main pass reads state_in while another
// writes state_out (in-place continuation).
struct ScanPass {
  const float* pieces;     // as PiecePass::pieces
  const float* state_in;   // [B][H][D][D] / [nseq][H][D][D] or nullptr
  float* seg_states;       // as FwdPass::seg_states
  uint32_t* tag;           // the workspace tag, written by workgroup 0
  WsTag tag_value;
  const float* slope;
  int B, H, N, D;
  int piece_len, npiece;
  int seg_len, nseg;
  int G;
};

// One (sequence, head) recurrence of a pass, and where its data lives.
struct Row {
  size_t tok;     // its first token row in the token tensors
  int len;        // tokens
  int h;          // head (slope index)
  int st;         // its d x d state in state_in / state_out
  int segbase;    // its first entry in seg_states
  int piecebase;  // its first entry in pieces
  int nseg;       // segments
};

// Row b*H + h of the uniform layout.
__host__ __device__ inline Row uniform_row(int bh, int H, int N, int nseg, int npiece) {
  return Row{(size_t)bh * (size_t)N, N, bh % H, bh, bh * nseg, bh * npiece, nseg};
}

// Row (sequence at schedule position i, head h) of a packed batch; ppseg =
// pieces per segment.
__host__ __device__ inline Row packed_row(const SeqTable& t, int i, int h, int H, int G,
                                          int ppseg) {
  const int s = t.ord[i], g = t.g0[i];
  return Row{(size_t)h * (size_t)t.T + (size_t)t.cu[s], t.cu[s + 1] - t.cu[s], h, s * H + h,
             h * G + g, (h * G + g) * ppseg, t.g0[i + 1] - g};
}

// The schedule position that owns segment g (0 <= g < g0[nseq]): the largest
// i with g0[i] <= g; g0 is strictly increasing.
__host__ __device__ inline int seq_of_segment(const SeqTable& t, int g) {
  int lo = 0, hi = t.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (t.g0[mid] <= g)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

hipError_t launch_fwd_bf16(const FwdPass& p, const SeqTable& t, hipStream_t s);
// fp32 forward; forward rows of at most kQuadMaxN tokens (uniform layout, no
// epilogue) are evaluated in the parallel form, longer ones chunk by chunk.
constexpr int kQuadMaxN = 256;
hipError_t launch_fwd_f32(const FwdPass& p, const SeqTable& t, hipStream_t s);
hipError_t launch_pieces_bf16(const PiecePass& p, const SeqTable& t, hipStream_t s);
hipError_t launch_scan(const ScanPass& p, const SeqTable& t, hipStream_t s);
hipError_t launch_bwd_kv_bf16(const BwdPass& p, const SeqTable& t, hipStream_t s);
hipError_t launch_decode(bool bf16, int B, int H, int D, const void* q, const void* k,
                         const void* v, const float* slope, float* state, void* o,
                         hipStream_t s);
// K <= kDecodeTokensMax tokens per (b, h) in one call, token tensors [B][H][K][D].
constexpr int kDecodeTokensMax = 16;
hipError_t launch_decode_tokens(bool bf16, int B, int H, int K, int D, const void* q,
                                const void* k, const void* v, const float* slope, float* state,
                                void* o, hipStream_t s);

// Measurement helper (la_probe.hip): x <- a x over n floats in place.  The
// load policy is 0 or kCpolNt, the store policy 0, kCpolNt or kCpolSc1
// (cache-policy bits of the buffer instructions).
constexpr int kCpolNt = 2, kCpolSc1 = 16;
hipError_t launch_stream_rmw(float* x, size_t n, float a, int load_policy, int store_policy,
                             hipStream_t s);

// Decay factors below this power of two are treated as exact zeros when a
// segment start state is assembled from piece states: lambda^dist < 2^-kSkipLog2
// means the piece contributes less than 2^-32 of its own magnitude, 2^8 below
// the fp32 resolution (2^-24) of a sum that also holds the undecayed last
// piece of the segment (pieces have equal lengths).
constexpr float kSkipLog2 = 32.0f;

}  // namespace la
