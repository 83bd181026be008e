// C-ABI host layer: argument validation, workspace, dispatch and error mapping.
// Nothing here computes on logits; every step of the path runs in kernels.hip.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "tsr.h"
#include "kernels.hpp"
#if TSR_TRACE
#include "tsr_trace.h"
#endif

struct tsr_ctx {
  int device;
  int max_rows;
  int max_vocab;
  int max_k;
  uint64_t seed;
  tsr::VerifyWs ws;
  tsr::BeamWs bws;
  void* ws_block;
#if TSR_TRACE
  unsigned long long* trace;   // phase stamps (tracing build)
#endif
};

namespace {

// Per-row parameters are read on the device with this layout.
static_assert(sizeof(tsr::RowParams) == sizeof(tsr_params), "tsr_params layout");
static_assert(offsetof(tsr::RowParams, temperature) == offsetof(tsr_params, temperature) &&
                  offsetof(tsr::RowParams, top_k) == offsetof(tsr_params, top_k) &&
                  offsetof(tsr::RowParams, top_p) == offsetof(tsr_params, top_p) &&
                  offsetof(tsr::RowParams, min_p) == offsetof(tsr_params, min_p) &&
                  offsetof(tsr::RowParams, filter_mode) == offsetof(tsr_params, filter_mode),
              "tsr_params layout");

constexpr double kTemperatureMin = 1e-30;
constexpr int kMaxDraft = 32;
constexpr int kMaxTreeNodes = 32;

// Runs f with the handle's device current and restores the caller's device.
template <class F>
int on_device(int device, F&& f) {
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return TSR_EDEVICE;
  if (prev != device && hipSetDevice(device) != hipSuccess) return TSR_EDEVICE;
  const int rc = f();
  if (prev != device) (void)hipSetDevice(prev);
  return rc;
}

int check_params(const tsr_params* p) {
  if (!p) return TSR_EINVAL;
  if (!isfinite(p->temperature) || !isfinite(p->top_p) || !isfinite(p->min_p))
    return TSR_EINVAL;
  if (p->temperature < 0.0) return TSR_EINVAL;
  if (p->temperature > 0.0 && p->temperature < kTemperatureMin) return TSR_EINVAL;
  if (p->top_p < 0.0) return TSR_EINVAL;
  if (p->filter_mode != TSR_JOINT && p->filter_mode != TSR_SEQUENTIAL) return TSR_EINVAL;
  return TSR_OK;
}

tsr::KParams make_kparams(uint64_t seed, const tsr_params* p, int vocab, uint64_t step,
                          bool want_z) {
  tsr::KParams kp{};
  const double T = p->temperature;
  if (T == 0.0) {
    kp.flags = tsr::F_GREEDY;
    kp.c = 1.0f;
  } else {
    kp.c = (float)(1.4426950408889634 / T);
    kp.cR = kp.c * 16.0f;
    if (p->top_k > 0 && p->top_k < vocab) {
      kp.top_k = p->top_k;
      kp.flags |= tsr::F_K;
    }
    if (p->top_p < 1.0) {
      kp.top_p = p->top_p;
      kp.flags |= tsr::F_P;
    }
    if (p->min_p > 0.0 && p->min_p < 1.0) {
      kp.minp_off = T * log(p->min_p);
      kp.flags |= tsr::F_M;
    }
    if (p->filter_mode == TSR_SEQUENTIAL) kp.flags |= tsr::F_SEQ;
    if (want_z) kp.flags |= tsr::F_Z;
  }
  kp.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  kp.key1 = (uint32_t)(seed >> 32);
  kp.step_lo = (uint32_t)(step & 0xFFFFFFFFu);
  kp.step_hi = (uint32_t)(step >> 32);
  return kp;
}

int esize(int dtype) { return dtype == TSR_F32 ? 4 : 2; }

bool elem_aligned(const void* p, int dtype) {
  return ((uintptr_t)p % (uintptr_t)esize(dtype)) == 0;
}

// Arguments every verify entry point checks (the handle's limits aside).
int check_verify(const void* target_logits, const void* draft_logits, int dtype,
                 const int32_t* draft_tokens, int rows, int K, int vocab,
                 const tsr_params* params, const int32_t* out_tokens,
                 const int32_t* out_accepted) {
  if (!target_logits || !draft_tokens || !out_tokens || !out_accepted) return TSR_EINVAL;
  if (dtype != TSR_F32 && dtype != TSR_BF16) return TSR_EINVAL;
  if (rows < 0 || vocab < 1 || K < 1 || K > kMaxDraft) return TSR_EINVAL;
  const int prc = check_params(params);
  if (prc != TSR_OK) return prc;
  if (params->temperature > 0.0 && !draft_logits) return TSR_EINVAL;
  if (!elem_aligned(target_logits, dtype) || (draft_logits && !elem_aligned(draft_logits, dtype)))
    return TSR_EINVAL;
  if (vocab > tsr::max_vocab_verify(dtype)) return TSR_EUNSUPPORTED;
  return TSR_OK;
}

// The verify launch once the arguments are checked (the device is current).
int launch_verify_checked(const void* target_logits, const void* draft_logits, int dtype,
                          const int32_t* draft_tokens, int rows, int K, int vocab,
                          const tsr::KParams& kp, const tsr::VerifyWs& ws, int32_t* out_tokens,
                          int32_t* out_accepted, int32_t* out_status, void* hip_stream) {
  // a row of a whole number of 16-byte chunks has no partial one (rows may
  // start at any element boundary)
  const int ragged = (vocab % (dtype == TSR_F32 ? 4 : 8)) != 0;
  const hipError_t e = tsr::launch_verify(target_logits, draft_logits, dtype, draft_tokens, rows,
                                          K, vocab, ragged, kp, ws, out_tokens,
                                          out_accepted, out_status, (hipStream_t)hip_stream);
  return e == hipSuccess ? TSR_OK : TSR_EDEVICE;
}

// spec_verify_noalloc's workspace: the per-(sequence, position) results (four
// int32 arrays of kStaticSlots), in `scratch` below: one copy per device,
// held until the process ends, shared by every call on that device. Every
// call writes each slot it reads, so nothing needs clearing.
constexpr int kStaticSlots = 1 << 16;   // sequences x (K + 1) positions
constexpr int kStaticSeqs = 1 << 14;    // sequences per call
constexpr size_t kStaticBytes = 4 * (size_t)kStaticSlots * sizeof(int32_t);
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

}  // namespace

// In host code `scratch` names a host-side stand-in, not device memory: only
// its address from hipGetSymbolAddress (static_workspace) reaches kernels.
static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

// The device address of `scratch` on `device` (the current device), looked up
// once per device and kept.
int static_workspace(int device, void** out) {
  if (device >= kMaxDevices) return TSR_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TSR_EDEVICE;
    g_static_ptr[device] = p;
  }
  *out = g_static_ptr[device];
  return TSR_OK;
}

}  // namespace

extern "C" {

const char* sampler_strerror(int code) {
  switch (code) {
    case TSR_OK: return "ok";
    case TSR_EINVAL: return "invalid argument";
    case TSR_ENOMEM: return "out of device memory";
    case TSR_EDEVICE: return "HIP runtime error";
    case TSR_EUNSUPPORTED: return "size not supported by this build";
    default: return "unknown error code";
  }
}

int sampler_init(tsr_handle* out, int device, int max_rows, int max_vocab, int max_k,
                 uint64_t seed) {
  if (!out) return TSR_EINVAL;
  *out = nullptr;
  if (max_rows < 1 || max_vocab < 1 || max_k < 0 || max_k > kMaxDraft) return TSR_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return TSR_EDEVICE;
  if (device < 0 || device >= ndev) return TSR_EINVAL;
  tsr_ctx* h = (tsr_ctx*)calloc(1, sizeof(tsr_ctx));
  if (!h) return TSR_ENOMEM;
  h->device = device;
  h->max_rows = max_rows;
  h->max_vocab = max_vocab;
  h->max_k = max_k;
  h->seed = seed;
  const int rc = on_device(device, [&]() -> int {
    const size_t slots = (size_t)max_rows * (size_t)(max_k + 1);
    const size_t vbytes = 4 * slots * sizeof(int32_t) + (size_t)max_rows * sizeof(uint32_t);
    const size_t bslots = (size_t)max_rows * tsr::kBeamMax;
    const size_t rbytes = (size_t)max_rows * 2 * (size_t)(max_k + 1) * sizeof(tsr::RowRec) +
                          (size_t)max_rows * 2 * tsr::kMaxSlices * sizeof(unsigned long long);
    const size_t bbytes = bslots * (sizeof(double) + sizeof(int32_t));
    const size_t bytes = ((vbytes + 7) & ~(size_t)7) + rbytes + bbytes;
    if (hipMalloc(&h->ws_block, bytes) != hipSuccess) return TSR_ENOMEM;
    if (hipMemset(h->ws_block, 0, bytes) != hipSuccess) return TSR_EDEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return TSR_EDEVICE;
    int32_t* base = (int32_t*)h->ws_block;
    h->ws.acc = base;
    h->ws.tok = base + slots;
    h->ws.st_t = base + 2 * slots;
    h->ws.st_d = base + 3 * slots;
    h->ws.counter = (uint32_t*)(base + 4 * slots);
    h->ws.kmax1 = max_k + 1;
    // wide verify: per sequence 2 (max_k + 1) row records
    h->ws.rec = (tsr::RowRec*)((char*)h->ws_block + ((vbytes + 7) & ~(size_t)7));
    h->ws.recs = 2 * (max_k + 1);
    h->ws.part = (unsigned long long*)(h->ws.rec + (size_t)max_rows * 2 * (max_k + 1));
    // beam step: per row kBeamMax (score, token)
    char* bb = (char*)h->ws_block + ((vbytes + 7) & ~(size_t)7) + rbytes;
    h->bws.score = (double*)bb;
    h->bws.tok = (int32_t*)(bb + bslots * sizeof(double));
#if TSR_TRACE
    if (hipMalloc(&h->trace, TSR_TRACE_WORDS * sizeof(uint64_t)) != hipSuccess) return TSR_ENOMEM;
    if (hipMemset(h->trace, 0, TSR_TRACE_WORDS * sizeof(uint64_t)) != hipSuccess) return TSR_EDEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return TSR_EDEVICE;
#endif
    return TSR_OK;
  });
  if (rc != TSR_OK) {
    if (h->ws_block) (void)hipFree(h->ws_block);
#if TSR_TRACE
    if (h->trace) (void)hipFree(h->trace);
#endif
    free(h);
    return rc;
  }
  *out = h;
  return TSR_OK;
}

int sampler_destroy(tsr_handle h) {
  if (!h) return TSR_OK;
  const int rc = on_device(h->device, [&]() -> int {
    if (hipDeviceSynchronize() != hipSuccess) return TSR_EDEVICE;
    if (h->ws_block && hipFree(h->ws_block) != hipSuccess) return TSR_EDEVICE;
#if TSR_TRACE
    if (h->trace && hipFree(h->trace) != hipSuccess) return TSR_EDEVICE;
#endif
    return TSR_OK;
  });
  free(h);
  return rc;
}

int greedy_argmax(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                  int64_t row_stride, int32_t* out_tokens, int32_t* out_status,
                  void* hip_stream) {
  if (!h || !logits || !out_tokens) return TSR_EINVAL;
  if (dtype != TSR_F32 && dtype != TSR_BF16) return TSR_EINVAL;
  if (rows < 0 || rows > h->max_rows || vocab < 1 || vocab > h->max_vocab) return TSR_EINVAL;
  if (row_stride < vocab || !elem_aligned(logits, dtype)) return TSR_EINVAL;
  if (vocab > tsr::max_vocab_sample(dtype)) return TSR_EUNSUPPORTED;
  if (rows == 0) return TSR_OK;
  const long long sb = (long long)row_stride * esize(dtype);
  const int ragged = (vocab % (dtype == TSR_F32 ? 4 : 8)) != 0;   // a partial last chunk
  return on_device(h->device, [&]() -> int {
    const hipError_t e = tsr::launch_greedy(logits, dtype, rows, vocab, sb, ragged,
                                            out_tokens, out_status, (hipStream_t)hip_stream);
    return e == hipSuccess ? TSR_OK : TSR_EDEVICE;
  });
}

int sample_rows_ex(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                   int64_t row_stride, const tsr_constraints* cons, const tsr_params* params,
                   uint64_t step, int32_t* out_tokens, float* out_logprob, const tsr_diag* diag,
                   void* hip_stream) {
  if (!h || !logits || !out_tokens) return TSR_EINVAL;
  if (dtype != TSR_F32 && dtype != TSR_BF16) return TSR_EINVAL;
  if (rows < 0 || rows > h->max_rows || vocab < 1 || vocab > h->max_vocab) return TSR_EINVAL;
  if (row_stride < vocab || !elem_aligned(logits, dtype)) return TSR_EINVAL;
  const tsr_constraints none{};
  const tsr_constraints& cs = cons ? *cons : none;
  if (cs.allowed) {
    const int64_t words = ((int64_t)vocab + 31) / 32;
    if (cs.allowed_stride < words || ((uintptr_t)cs.allowed % 4) != 0) return TSR_EINVAL;
  }
  if (!cs.history && cs.history_len > 0) return TSR_EINVAL;   // a window length without ids
  const bool rep_given = cs.history && cs.history_len > 0;
  if (rep_given) {
    if (cs.history_len > tsr::kHistMax || cs.history_stride < cs.history_len ||
        ((uintptr_t)cs.history % 4) != 0)
      return TSR_EINVAL;
    if (!isfinite(cs.repetition_penalty) || cs.repetition_penalty < 1.0) return TSR_EINVAL;
  } else if (cs.history_len < 0) {
    return TSR_EINVAL;
  }
  if (cs.row_params && ((uintptr_t)cs.row_params % alignof(tsr_params)) != 0) return TSR_EINVAL;
  const tsr_params unit{1.0, 0, 1.0, 0.0, TSR_JOINT};
  if (!params && cs.row_params) params = &unit;   // the rows carry their own
  const int prc = check_params(params);
  if (prc != TSR_OK) return prc;
  if (vocab > tsr::max_vocab_sample(dtype)) return TSR_EUNSUPPORTED;
  if (rows == 0) return TSR_OK;
  tsr::DiagPtrs dg{};
  if (diag) {
    dg.status = diag->status;
    dg.kept_count = diag->kept_count;
    dg.threshold = diag->threshold;
    dg.kept_mass = diag->kept_mass;
    dg.probs = diag->probs;
  }
  dg.logprob = out_logprob;
  tsr::KParams kp = make_kparams(h->seed, params, vocab, step, dg.kept_mass != nullptr);
#if TSR_TRACE
  kp.trace = h->trace;
#endif
  if (cs.row_params) {
    kp.rowp = reinterpret_cast<const tsr::RowParams*>(cs.row_params);
    kp.flags |= tsr::F_ROWP;
    if (dg.kept_mass) kp.flags |= tsr::F_Z;
  }
  if (cs.allowed) {
    kp.allowed = cs.allowed;
    kp.allowed_stride = (long long)cs.allowed_stride;
    kp.flags |= tsr::F_MASK;
  }
  if (rep_given && cs.repetition_penalty != 1.0) {
    kp.hist = cs.history;
    kp.hist_stride = (long long)cs.history_stride;
    kp.hist_len = cs.history_len;
    kp.rpen = cs.repetition_penalty;
    kp.flags |= tsr::F_REP;
  }
  const long long sb = (long long)row_stride * esize(dtype);
  const int ragged = (vocab % (dtype == TSR_F32 ? 4 : 8)) != 0;   // a partial last chunk
  return on_device(h->device, [&]() -> int {
    const hipError_t e = tsr::launch_sample(logits, dtype, rows, vocab, sb, ragged, kp,
                                            out_tokens, dg, (hipStream_t)hip_stream);
    return e == hipSuccess ? TSR_OK : TSR_EDEVICE;
  });
}

int sample_rows_masked(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                       int64_t row_stride, const uint32_t* allowed, int64_t allowed_stride,
                       const tsr_params* params, uint64_t step, int32_t* out_tokens,
                       float* out_logprob, const tsr_diag* diag, void* hip_stream) {
  tsr_constraints cs{};
  cs.allowed = allowed;
  cs.allowed_stride = allowed_stride;
  return sample_rows_ex(h, logits, dtype, rows, vocab, row_stride, &cs, params, step, out_tokens,
                        out_logprob, diag, hip_stream);
}

int sample_rows(tsr_handle h, const void* logits, int dtype, int rows, int vocab,
                int64_t row_stride, const tsr_params* params, uint64_t step,
                int32_t* out_tokens, const tsr_diag* diag, void* hip_stream) {
  return sample_rows_masked(h, logits, dtype, rows, vocab, row_stride, nullptr, 0, params, step,
                            out_tokens, nullptr, diag, hip_stream);
}

int spec_verify(tsr_handle h, const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, int rows, int K, int vocab,
                const tsr_params* params, uint64_t step, int32_t* out_tokens,
                int32_t* out_accepted, int32_t* out_status, void* hip_stream) {
  if (!h) return TSR_EINVAL;
  if (rows > h->max_rows || vocab > h->max_vocab || K > h->max_k) return TSR_EINVAL;
  const int rc = check_verify(target_logits, draft_logits, dtype, draft_tokens, rows, K, vocab,
                              params, out_tokens, out_accepted);
  if (rc != TSR_OK || rows == 0) return rc;
  tsr::KParams kp = make_kparams(h->seed, params, vocab, step, false);
#if TSR_TRACE
  kp.trace = h->trace;
#endif
  return on_device(h->device, [&]() -> int {
    return launch_verify_checked(target_logits, draft_logits, dtype, draft_tokens, rows, K, vocab,
                                 kp, h->ws, out_tokens, out_accepted, out_status, hip_stream);
  });
}

int spec_verify_noalloc(int device, uint64_t seed, const void* target_logits,
                        const void* draft_logits, int dtype, const int32_t* draft_tokens,
                        int rows, int K, int vocab, const tsr_params* params, uint64_t step,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_status,
                        void* hip_stream) {
  if (rows > kStaticSeqs || (int64_t)rows * (K + 1) > kStaticSlots) return TSR_EINVAL;
  const int rc = check_verify(target_logits, draft_logits, dtype, draft_tokens, rows, K, vocab,
                              params, out_tokens, out_accepted);
  if (rc != TSR_OK) return rc;
  if (vocab > tsr::max_vocab_verify_narrow(dtype)) return TSR_EUNSUPPORTED;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return TSR_EDEVICE;
  if (device < 0 || device >= ndev) return TSR_EINVAL;
  if (rows == 0) return TSR_OK;
  const tsr::KParams kp = make_kparams(seed, params, vocab, step, false);
  return on_device(device, [&]() -> int {
    void* base = nullptr;
    const int src = static_workspace(device, &base);
    if (src != TSR_OK) return src;
    int32_t* b = (int32_t*)base;
    tsr::VerifyWs ws;
    ws.acc = b;
    ws.tok = b + kStaticSlots;
    ws.st_t = b + 2 * kStaticSlots;
    ws.st_d = b + 3 * kStaticSlots;
    ws.counter = nullptr;   // the two-row verify keeps no arrival counters
    ws.kmax1 = K + 1;
    ws.rec = nullptr;   // the array holds no row records: register-pair rows only
    ws.recs = 0;
    ws.part = nullptr;
    return launch_verify_checked(target_logits, draft_logits, dtype, draft_tokens, rows, K, vocab,
                                 kp, ws, out_tokens, out_accepted, out_status, hip_stream);
  });
}

int tree_verify(tsr_handle h, const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* parent, const int32_t* tokens, int rows, int nodes, int vocab,
                const tsr_params* params, uint64_t step, int32_t* out_tokens, int32_t* out_path,
                int32_t* out_accepted, int32_t* out_status, void* hip_stream) {
  if (!h || !target_logits || !parent || !tokens || !out_tokens || !out_path || !out_accepted)
    return TSR_EINVAL;
  if (dtype != TSR_F32 && dtype != TSR_BF16) return TSR_EINVAL;
  if (rows < 0 || rows > h->max_rows || vocab < 1 || vocab > h->max_vocab) return TSR_EINVAL;
  if (nodes < 1 || nodes > kMaxTreeNodes || nodes > h->max_k + 1) return TSR_EINVAL;
  const int prc = check_params(params);
  if (prc != TSR_OK) return prc;
  if (params->temperature > 0.0 && !draft_logits) return TSR_EINVAL;
  if (!elem_aligned(target_logits, dtype) || (draft_logits && !elem_aligned(draft_logits, dtype)))
    return TSR_EINVAL;
  if (vocab > tsr::max_vocab_verify(dtype)) return TSR_EUNSUPPORTED;
  if (rows == 0) return TSR_OK;
  tsr::KParams kp = make_kparams(h->seed, params, vocab, step, false);
#if TSR_TRACE
  kp.trace = h->trace;
#endif
  // a row of a whole number of 16-byte chunks has no partial one (rows may
  // start at any element boundary)
  const int ragged = (vocab % (dtype == TSR_F32 ? 4 : 8)) != 0;
  return on_device(h->device, [&]() -> int {
    const hipError_t e = tsr::launch_tree(target_logits, draft_logits, dtype, parent, tokens, rows,
                                          nodes, vocab, ragged, kp, h->ws, out_tokens,
                                          out_path, out_accepted, out_status,
                                          (hipStream_t)hip_stream);
    return e == hipSuccess ? TSR_OK : TSR_EDEVICE;
  });
}

int beam_step(tsr_handle h, const void* logits, int dtype, int groups, int beam, int vocab,
              int64_t row_stride, const double* beam_scores, int32_t* out_parent,
              int32_t* out_token, double* out_score, int32_t* out_status, void* hip_stream) {
  if (!h || !logits || !beam_scores || !out_parent || !out_token || !out_score) return TSR_EINVAL;
  if (dtype != TSR_F32 && dtype != TSR_BF16) return TSR_EINVAL;
  if (beam < 1 || beam > tsr::kBeamMax || groups < 0) return TSR_EINVAL;
  if ((int64_t)groups * beam > h->max_rows || vocab < 1 || vocab > h->max_vocab) return TSR_EINVAL;
  if (row_stride < vocab || !elem_aligned(logits, dtype) || ((uintptr_t)beam_scores % 8) != 0)
    return TSR_EINVAL;
  if (vocab > tsr::max_vocab_beam(dtype)) return TSR_EUNSUPPORTED;
  const long long sb = (long long)row_stride * esize(dtype);
  if (groups == 0) return TSR_OK;
  const int ragged = (vocab % (dtype == TSR_F32 ? 4 : 8)) != 0;   // a partial last chunk
  return on_device(h->device, [&]() -> int {
    const hipError_t e = tsr::launch_beam(logits, dtype, groups, beam, vocab, sb, ragged,
                                          beam_scores, h->bws, out_parent, out_token, out_score,
                                          out_status, (hipStream_t)hip_stream);
    return e == hipSuccess ? TSR_OK : TSR_EDEVICE;
  });
}

int sampler_philox(tsr_handle h, const uint32_t* counters, int n, uint32_t* out_words,
                   void* hip_stream) {
  if (!h || !counters || !out_words || n < 0) return TSR_EINVAL;
  if (n == 0) return TSR_OK;
  return on_device(h->device, [&]() -> int {
    const hipError_t e = tsr::launch_philox(counters, n, (uint32_t)(h->seed & 0xFFFFFFFFu),
                                            (uint32_t)(h->seed >> 32), out_words,
                                            (hipStream_t)hip_stream);
    return e == hipSuccess ? TSR_OK : TSR_EDEVICE;
  });
}

#if TSR_TRACE
int sampler_trace_read(tsr_handle h, uint64_t* out, int64_t n) {
  if (!h || !out || n < 0 || n > TSR_TRACE_WORDS) return TSR_EINVAL;
  return on_device(h->device, [&]() -> int {
    if (hipDeviceSynchronize() != hipSuccess) return TSR_EDEVICE;
    if (n && hipMemcpy(out, h->trace, (size_t)n * sizeof(uint64_t), hipMemcpyDeviceToHost) !=
                 hipSuccess)
      return TSR_EDEVICE;
    return TSR_OK;
  });
}

int sampler_trace_clear(tsr_handle h) {
  if (!h) return TSR_EINVAL;
  return on_device(h->device, [&]() -> int {
    if (hipDeviceSynchronize() != hipSuccess) return TSR_EDEVICE;
    if (hipMemset(h->trace, 0, TSR_TRACE_WORDS * sizeof(uint64_t)) != hipSuccess)
      return TSR_EDEVICE;
    return hipDeviceSynchronize() == hipSuccess ? TSR_OK : TSR_EDEVICE;
  });
}
#endif

}  // extern "C"
