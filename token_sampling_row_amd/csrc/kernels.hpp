// Plain structures shared by the C-ABI host layer and the gfx950 kernels, and
// the launch entry points the host layer calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "trace.hpp"

namespace tsr {

// One row's sampling parameters, laid out as the C ABI's tsr_params.
struct RowParams {
  double temperature;
  int32_t top_k;
  double top_p;
  double min_p;
  int32_t filter_mode;
};

// Sampling parameters after host-side validation.
struct KParams {
  float c;             // log2(e) / T
  float cR;            // c * (log-probability bins per unit of log2)
  double minp_off;     // T * ln(min_p): min-p keeps v >= M + minp_off
  double top_p;
  int top_k;           // 0 = off (the host maps k <= 0 and k >= V to 0)
  int flags;
  uint32_t key0, key1; // Philox key = seed (low word, high word)
  uint32_t step_lo, step_hi;
  const uint32_t* allowed;   // allowed-token bitmask rows (F_MASK), token i = bit i % 32 of word i / 32
  long long allowed_stride;  // words between mask rows
  const int32_t* hist;       // look-back window rows (F_REP): recent token ids
  long long hist_stride;     // ids between window rows
  int hist_len;              // ids per row (<= kHistMax)
  double rpen;               // repetition penalty r
  const RowParams* rowp;     // per-row parameters (F_ROWP), validated and derived per row
#if TSR_TRACE
  unsigned long long* trace; // phase stamps (tracing build only)
#endif
};
enum : int {
  F_GREEDY = 1,   // temperature 0
  F_K = 2,        // top-k active
  F_P = 4,        // top-p active
  F_M = 8,        // min-p active
  F_SEQ = 16,     // SEQUENTIAL filter mode
  F_Z = 32,       // the full weight sum is wanted (kept-mass diagnostic)
  F_MASK = 64,    // an allowed-token bitmask applies
  F_REP = 128,    // a repetition penalty applies
  F_ROWP = 256,   // each row has its own parameters (rowp)
};
constexpr int kHistMax = 64;   // longest look-back window
// Filters whose kept set may be far larger than any candidate buffer: no
// top-k, or one too large for the per-thread-maxima sketch (the sampling
// launch then takes the WIDE kernel instance).
inline bool wide_filters(const KParams& kp, int block) {
  if (kp.flags & F_GREEDY) return false;
  if (!(kp.flags & (F_K | F_P | F_M))) return false;
  return !(kp.flags & F_K) || kp.top_k > block / 4;
}

struct DiagPtrs {
  int32_t* status;
  int32_t* kept_count;
  float* threshold;
  double* kept_mass;
  float* probs;
  float* logprob;   // log p~ of the drawn token
};

// Per-handle workspace of the beam step: each beam row's best candidates,
// best first (score, token), kBeamMax per row, written by the row kernel and
// merged per group by the kernel that follows it in the stream.
constexpr int kBeamMax = 16;
struct BeamWs {
  double* score;
  int32_t* tok;
};

// What the wide verify path records of one target or draft row: the kept
// weight sum Z_S, the row maximum M, the kept set {v >= tau}, the status, and
// a token (greedy: the argmax; else the row's own draw where it is known).
struct RowRec {
  double zs;
  float M;
  float tau;
  int status;
  int tok;
};

// Per-handle workspace of the verify step: per (sequence, position) results,
// one arrival counter per sequence for the tree kernel (zero between calls;
// null where no tree verify runs); for rows wider
// than two register rows per workgroup, `recs` row records per sequence (its
// target rows from 0, its draft rows from recs / 2).
struct VerifyWs {
  int32_t* acc;
  int32_t* tok;
  int32_t* st_t;
  int32_t* st_d;
  uint32_t* counter;
  int kmax1;      // max_k + 1: stride of the per-position arrays
  RowRec* rec;    // null: the wide path is not available
  int recs;       // 2 * kmax1
  unsigned long long* part;   // per sequence 2 * kMaxSlices residual sums (double bits)
  int nseq;       // sequences of the call (set per launch)
};

constexpr int kMaxSlices = 16;   // residual slices per row on the wide verify path

int max_vocab_sample(int dtype);
int max_vocab_verify(int dtype);          // with the row records (wide rows)
int max_vocab_verify_narrow(int dtype);   // without them

// ragged: a row does not split into whole 16-byte chunks (vocab not a
// multiple of 4 / 8). Rows may start at any element boundary.
hipError_t launch_greedy(const void* logits, int dtype, int rows, int V, long long stride_bytes,
                         int ragged, int32_t* out, int32_t* status, hipStream_t s);
hipError_t launch_sample(const void* logits, int dtype, int rows, int V, long long stride_bytes,
                         int ragged, const KParams& kp, int32_t* out,
                         const DiagPtrs& dg, hipStream_t s);
hipError_t launch_verify(const void* tgt, const void* dft, int dtype, const int32_t* xs,
                         int rows, int K, int V, int ragged, const KParams& kp,
                         const VerifyWs& ws, int32_t* out_tokens, int32_t* out_acc,
                         int32_t* out_status, hipStream_t s);
hipError_t launch_tree(const void* tgt, const void* dft, int dtype, const int32_t* parent,
                       const int32_t* tokens, int rows, int N, int V, int ragged,
                       const KParams& kp, const VerifyWs& ws, int32_t* out_tokens,
                       int32_t* out_path, int32_t* out_acc, int32_t* out_status, hipStream_t s);
hipError_t launch_beam(const void* logits, int dtype, int groups, int beam, int V,
                       long long stride_bytes, int ragged, const double* scores, BeamWs ws,
                       int32_t* out_parent, int32_t* out_tok, double* out_score,
                       int32_t* out_status, hipStream_t s);
int max_vocab_beam(int dtype);
hipError_t launch_philox(const uint32_t* ctr, int n, uint32_t k0, uint32_t k1, uint32_t* out,
                         hipStream_t s);

}  // namespace tsr
