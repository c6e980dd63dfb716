// la_internal.h -- host-side interface between the C ABI (la_api.cpp) and the
// kernel launchers.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

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
  // tokens (a multiple of C); segment r > 0 starts from seg_states[b][h][r]
  // (entry r = 0 is unused and state_in is used instead).
  int seg_len;
  int nseg;
  const float* seg_states;  // [B][H][nseg][D][D] or nullptr when nseg == 1
};

// Per-piece local states for the segment pre-pass:
// piece p of length piece_len ends at token e_p = min(N, (p+1) piece_len) - 1
// and holds sum_{t in piece} lambda^(e_p - t) k_t v_t^T.
struct PiecePass {
  const void* k;
  const void* v;
  const float* slope;
  float* pieces;  // [B][H][npiece][D][D]
  int B, H, N, D, C;
  bool reverse;
  int piece_len, npiece;
  int seg_len, nseg;  // a piece is computed only if some segment start needs it
};

// Segment start states from the piece states (and state_in).
struct ScanPass {
  const float* pieces;     // [B][H][npiece][D][D]
  const float* state_in;   // [B][H][D][D] or nullptr
  float* seg_states;       // [B][H][nseg][D][D]
  const float* slope;
  int B, H, N, D;
  int piece_len, npiece;
  int seg_len, nseg;
};

hipError_t launch_fwd_bf16(const FwdPass& p, hipStream_t s);
hipError_t launch_fwd_f32(const FwdPass& p, hipStream_t s);
hipError_t launch_pieces_bf16(const PiecePass& p, hipStream_t s);
hipError_t launch_scan(const ScanPass& p, hipStream_t s);
hipError_t launch_decode(bool bf16, int B, int H, int D, const void* q, const void* k,
                         const void* v, const float* slope, float* state, void* o,
                         hipStream_t s);

// Decay factors below this power of two are treated as exact zeros when a
// segment start state is assembled from piece states: lambda^dist < 2^-kSkipLog2
// means the piece contributes less than 2^-64 of its own magnitude, 2^40 below
// the fp32 resolution of a sum that also holds the undecayed last piece of
// the segment (pieces have equal lengths).
constexpr float kSkipLog2 = 64.0f;

}  // namespace la
