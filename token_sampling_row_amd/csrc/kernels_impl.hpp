// gfx950 kernel templates of the sampler: greedy argmax, sample_rows, the
// speculative verify step and the Philox test hook. One workgroup of kBlock
// threads per row. Rows up to 19 chunks per thread stay in VGPRs (row_regs);
// wider rows stream through the cache hierarchy (row_stream).
#pragma once

#include "row_regs.hpp"
#include "row_stream.hpp"

namespace tsr {

__device__ __forceinline__ Filters make_filters(const KParams& kp, float M) {
  Filters f;
  f.k_on = (kp.flags & F_K) != 0;
  f.p_on = (kp.flags & F_P) != 0;
  f.m_on = (kp.flags & F_M) != 0;
  f.seq = (kp.flags & F_SEQ) != 0;
  f.k = kp.top_k;
  f.top_p = kp.top_p;
  f.tau_m = f.m_on ? ceil_to_float((double)M + kp.minp_off) : kNegInf;
  return f;
}

// Row `row`'s own parameters (F_ROWP) in place of the call's: validated as
// the host validates a call's (false: the row is TSR_ROW_BADPARAM), then
// derived as the host derives them (temperature to c, the filters' switches).
__device__ __forceinline__ bool row_kparams(KParams& kp, int row, int V) {
  const RowParams q = kp.rowp[row];
  const double T = q.temperature;
  if (!isfinite(T) || !isfinite(q.top_p) || !isfinite(q.min_p)) return false;
  if (T < 0.0 || (T > 0.0 && T < 1e-30) || q.top_p < 0.0) return false;
  if (q.filter_mode != 0 && q.filter_mode != 1) return false;
  const int keep = kp.flags & (F_MASK | F_REP | F_ROWP);
  const bool want_z = (kp.flags & F_Z) != 0;
  kp.flags = keep;
  kp.top_k = 0;
  if (T == 0.0) {
    kp.flags |= F_GREEDY;
    kp.c = 1.0f;
    return true;
  }
  kp.c = (float)(1.4426950408889634 / T);
  kp.cR = kp.c * 16.0f;
  if (q.top_k > 0 && q.top_k < V) {
    kp.top_k = q.top_k;
    kp.flags |= F_K;
  }
  if (q.top_p < 1.0) {
    kp.top_p = q.top_p;
    kp.flags |= F_P;
  }
  if (q.min_p > 0.0 && q.min_p < 1.0) {
    kp.minp_off = T * log(q.min_p);
    kp.flags |= F_M;
  }
  if (q.filter_mode == 1) kp.flags |= F_SEQ;
  if (want_z) kp.flags |= F_Z;
  return true;
}
constexpr int kRowBadParam = 4;

// JOINT top-p measures mass against the row's full weight sum.
__device__ __forceinline__ bool joint_top_p(const KParams& kp) {
  const bool k_on = kp.flags & F_K, p_on = kp.flags & F_P, seq = kp.flags & F_SEQ;
  return p_on && !(seq && k_on);
}
// The streaming path also forms the full sum for the kept-mass diagnostic.
__device__ __forceinline__ bool wants_z(const KParams& kp) {
  return (kp.flags & F_Z) || joint_top_p(kp);
}

__device__ __forceinline__ double draw_uniform(const KParams& kp, uint32_t row, uint32_t pos,
                                               uint32_t domain, int word) {
  const uint4 w = philox4x32_10(make_uint4(row, pos | (domain << 16), kp.step_lo, kp.step_hi),
                                kp.key0, kp.key1);
  return (double)(word == 0 ? w.x : w.y) * 0x1p-32;
}

// wtok / zs: weight of the drawn token and of S (log p~ of the draw is their
// log ratio, eq. 39.2); greedy passes 1, 1 (a point mass) and bad rows NaN.
__device__ __forceinline__ void write_row(int row, int tok, int status, int kept, float tmin,
                                          double kmass, double wtok, double zs, int32_t* out,
                                          const DiagPtrs& dg) {
  if (threadIdx.x == 0) {
    out[row] = tok;
    if (dg.status) dg.status[row] = status;
    if (dg.kept_count) dg.kept_count[row] = kept;
    if (dg.threshold) dg.threshold[row] = tmin;
    if (dg.kept_mass) dg.kept_mass[row] = kmass;
    if (dg.logprob) dg.logprob[row] = log_ratio(wtok, zs);
  }
}
constexpr double kNaN = __builtin_nan("");

__device__ __forceinline__ void zero_probs(const DiagPtrs& dg, int row, int V) {
  if (dg.probs) {
    float* pr = dg.probs + (long long)row * V;
    for (int i = threadIdx.x; i < V; i += kBlock) pr[i] = 0.0f;
  }
}
// Diagnostics of a greedy row: p~ is the point mass at the drawn token (|S| 1,
// the threshold its logit M, kept mass 1).
__device__ __forceinline__ void greedy_row(int row, int tok, float M, int V, int32_t* out,
                                           const DiagPtrs& dg) {
  write_row(row, tok, 0, 1, M, 1.0, 1.0, 1.0, out, dg);
  if (dg.probs) {
    float* pr = dg.probs + (long long)row * V;
    for (int i = threadIdx.x; i < V; i += kBlock) pr[i] = i == tok ? 1.0f : 0.0f;
  }
}

// Kept set, draw and diagnostics of one row on the streaming path.
template <int DT>
__device__ __noinline__ void stream_finish(const StreamRow<DT> s, int row, float M, double Z,
                                           const KParams kp, const Filters f, double u,
                                           int32_t* out, const DiagPtrs dg) {
  const Cut cut = general_stream(s, M, Z, kp.c, kp.cR, f);
  double zs, wt;
  const int tok = walk_stream(s, cut.tau, M, kp.c, u, &zs, &wt);
  int kept = cut.kept;
  float tmin = cut.tau;
  if (dg.kept_count || dg.threshold) stream_kept_stats(s, cut.tau, &kept, &tmin);
  if (dg.kept_mass && !(Z > 0.0)) Z = stream_weight_sum(s, -kFltMax, M, kp.c);
  write_row(row, tok, 0, kept, tmin, Z > 0.0 ? zs / Z : 0.0, wt, zs, out, dg);
  if (dg.probs) stream_probs(s, cut.tau, M, kp.c, zs, dg.probs + (long long)row * s.V);
}

// Diagnostics of a row whose token the register path drew: they re-read the
// row (validation outputs, off the timed path). Not inlined, and nothing is
// live in the caller after it, so the hot path keeps no values for it.
template <int DT>
__device__ __noinline__ void diag_finish(const StreamRow<DT> s, int row, int tok, int kept,
                                         float tau, float M, float c, double zs, double wt,
                                         int32_t* out, const DiagPtrs dg) {
  float tmin = tau;
  if (dg.kept_count || dg.threshold) stream_kept_stats(s, tau, &kept, &tmin);
  const double Z = dg.kept_mass ? stream_weight_sum(s, -kFltMax, M, c) : 0.0;
  write_row(row, tok, 0, kept, tmin, Z > 0.0 ? zs / Z : 0.0, wt, zs, out, dg);
  if (dg.probs) stream_probs(s, tau, M, c, zs, dg.probs + (long long)row * s.V);
}

// A register-resident row seen through the StreamRow interface, so the
// general kept-set search can run on it without re-reading HBM.
template <int DT, int NC>
struct RegView {
  const RegRow<DT, NC>& r;
  static constexpr int nct = NC;
  __device__ __forceinline__ void elems(int j, float* v, float* m) const {
    r.elems(j, v);
    *m = r.cmax(j);
  }
  __device__ __forceinline__ int base(int j) const { return r.base(j); }
};

// JOINT top-k / top-p over a bf16 row held in registers, exactly, from one
// histogram pass without an exponential per element. Bins are 1/32 logit
// wide below the row max, bin b = (M - v) * 32, exact for bf16 rows with
// |M| <= 2^15 (the difference of two such values is exact in float). Where
// |v| >= 4 the bf16 grid spacing is at least 1/32, so such a bin holds one
// value, the largest bf16 value at or below M - b/32; its count gives its
// weight exactly. The other bins (|v| < 4 somewhere in the bin, or the last
// bin, past 32 logits below the max) sum fixed-point weights per element.
// Counts go to kVCopies copies by lane, so lanes that fall in the same bin
// mostly hit different words. The bin masses give Z, the boundary bin
// (find_boundary) and, when that bin holds one value, the cut; otherwise its
// elements are sorted and resolved exactly (resolve_sorted). ok = false when
// the boundary bin holds more than kCap elements (the caller then takes the
// general search). kept / zs are -1 when min-p cuts deeper.
template <int NC>
__device__ __forceinline__ Cut bf16_value_cut(const RegRow<1, NC>& r, float M, float c,
                                              const Filters& f, Lds& L, bool* ok) {
  constexpr int EPC = Fmt<1>::EPC;
  const int tid = threadIdx.x;
  for (int i = tid; i < kVCopies * kVStride; i += kBlock) L.vcnt[i] = 0u;
  for (int i = tid; i < kBins; i += kBlock) {
    L.hcnt[i] = 0u;
    L.hmass[i] = 0ull;
  }
  // bins b >= bneg lie wholly at or below -4, bins b <= bpos wholly above 4
  const int bneg = (int)ceilf((M + 4.0f) * (float)kVRes);
  const int bpos = (int)floorf((M - 4.0f) * (float)kVRes) - 1;
  auto pure = [&](int b) { return (b < kVBins - 1) & ((b >= bneg) | (b <= bpos)); };
  // (M - v) * kVRes as one fused rounding of 32 (M - v): the same value
  // wherever the difference is exact, i.e. in every bin but the last
  const float M32 = M * (float)kVRes;
  uint32_t* cnt = L.vcnt + (__lane_id() & (kVCopies - 1)) * kVStride;
  __syncthreads();
  // counts, branch-free: -inf lands in the last bin with the clamp and is
  // taken out of it again below (counted where a chunk reaches that bin). The
  // elements of bins without a single value are weighed too, behind one test
  // per chunk row from the chunk's lowest and highest bin (every bin in
  // [bneg, kVBins - 2], or every bin at or below bpos, means none is there; a
  // chunk holding -inf reaches the last bin and so takes the per-element test)
  uint32_t ninf = 0u;
  auto count = [&](int j) {
    float v[EPC];
    r.elems(j, v);
    int b[EPC];
    int lo = kVBins, hi = 0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      b[e] = (int)fminf(fmaf(v[e], -(float)kVRes, M32), (float)(kVBins - 1));
      lo = min(lo, b[e]);
      hi = max(hi, b[e]);
      atomicAdd(&cnt[b[e]], 1u);
    }
    const bool imp = !((hi <= kVBins - 2) & ((lo >= bneg) | (hi <= bpos)));
    if (__any(imp)) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const bool fin = v[e] > kNegInf;
        ninf += fin ? 0u : 1u;
        if (fin & !pure(b[e])) atomicAdd(&L.hmass[hslot(b[e])], to_fixed(weight(v[e], M, c)));
      }
    }
  };
  // chunk rows past the 32nd at fixed register indices
  constexpr int kDyn = NC > 32 ? 32 : NC;
#pragma unroll 1
  for (int j = 0; j < kDyn; ++j) count(j);
  static_for<kDyn, NC>([&](auto jc) { count(decltype(jc)::value); });
  if (ninf) atomicSub(&cnt[kVBins - 1], ninf);
  __syncthreads();
  // the bin totals and the boundary in one block pass: thread t owns bins 2t
  // and 2t + 1, and a block scan of (count, fixed-point mass) in bin order
  // gives Z exactly and each bin what lies above it; the boundary rule is
  // find_boundary's (nothing above the bins, the row max among them)
  static_assert(kVBins == 2 * kBlock, "two bins per thread");
  const int lane = __lane_id(), wid = tid / kWave;
  uint32_t nb[2];
  unsigned long long mb[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = 2 * tid + q;
    uint32_t n = 0u;
#pragma unroll
    for (int k = 0; k < kVCopies; ++k) n += L.vcnt[k * kVStride + b];
    L.hcnt[hslot(b)] = n;
    unsigned long long mm = L.hmass[hslot(b)];
    if (n && pure(b)) {
      // the bin's one value: M - b/32 (exact) rounded down to the bf16 grid
      const uint32_t x = __float_as_uint(M - (float)b * (1.0f / kVRes));
      const uint32_t xv = (x & 0xFFFFu) == 0u ? x
                          : ((x >> 31) ? (x & 0xFFFF0000u) + 0x10000u : (x & 0xFFFF0000u));
      const double m = (double)n * (double)weight(__uint_as_float(xv), M, c);
      mm = (unsigned long long)(m * kFix + 0.5);
      L.hmass[hslot(b)] = mm;
    }
    nb[q] = n;
    mb[q] = mm;
  }
  const int tc = (int)(nb[0] + nb[1]);
  const unsigned long long tm = mb[0] + mb[1];
  const int ic = wave_incl_scan(tc);
  const unsigned long long im = wave_incl_scan(tm);
  if (lane == kWave - 1) {
    L.bs.i[wid] = ic;
    L.bs.q[wid] = im;
  }
  __syncthreads();
  int cbefore = 0, call = 0;
  unsigned long long mbefore = 0ull, mall = 0ull;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int tcw = L.bs.i[w];
    const unsigned long long tmw = L.bs.q[w];
    cbefore += w < wid ? tcw : 0;
    mbefore += w < wid ? tmw : 0ull;
    call += tcw;
    mall += tmw;
  }
  const double Z = (double)mall * kInvFix;
  const double thr = f.p_on ? f.top_p * Z : 0.0;
  const int ex_c = cbefore + ic - tc;
  const unsigned long long ex_m = mbefore + im - tm;
  int first = kBins, dk = kBins, dp = -1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = 2 * tid + q;
    const int rc = ex_c + (q ? (int)nb[0] : 0);
    const unsigned long long rm = ex_m + (q ? mb[0] : 0ull);
    if (nb[q]) {
      first = min(first, b);
      if (f.k_on && dk == kBins && rc + (int)nb[q] >= f.k) dk = b;
      if (f.p_on && (double)rm * kInvFix < thr) dp = b;
    }
  }
  first = wave_min(first);
  dk = wave_min(dk);
  dp = wave_max(dp);
  if (lane == 0) {
    L.bs.u[wid] = (uint32_t)first;
    L.bs.f[wid] = (float)dk;
    L.bs.d[wid] = (double)dp;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    first = min(first, (int)L.bs.u[w]);
    dk = min(dk, (int)L.bs.f[w]);
    dp = max(dp, (int)L.bs.d[w]);
  }
  if (f.p_on) dp = max(dp, first);
  int d = kBins;
  if (f.k_on) d = min(d, dk);
  if (f.p_on) d = min(d, dp < 0 ? kBins : dp);
  int add_c = call;
  double add_m = (double)mall * kInvFix;
  if (d < kBins) {   // what lies above bin d, from its owner's prefix
    if (tid == (d >> 1)) {
      L.si[5] = ex_c + ((d & 1) ? (int)nb[0] : 0);
      L.sd[5] = (double)(ex_m + ((d & 1) ? mb[0] : 0ull)) * kInvFix;
    }
    __syncthreads();
    add_c = L.si[5];
    add_m = L.sd[5];
  }
  __syncthreads();
  *ok = true;
  Cut cut;
  const float floor_m = f.tau_m > kNegInf ? f.tau_m : -kFltMax;
  if (d == kBins) {   // no cut inside the bins
    cut.tau = floor_m;
    cut.kept = -1;
    cut.zs = -1.0;
    return cut;
  }
  if (pure(d)) {      // the boundary bin is one value group, kept whole
    const uint32_t x = __float_as_uint(M - (float)d * (1.0f / kVRes));
    const uint32_t xv = (x & 0xFFFFu) == 0u ? x
                        : ((x >> 31) ? (x & 0xFFFF0000u) + 0x10000u : (x & 0xFFFF0000u));
    const float vd = __uint_as_float(xv);
    cut.tau = fmaxf(vd, floor_m);
    const bool exact = !(floor_m > vd);
    cut.kept = exact ? add_c + (int)L.hcnt[hslot(d)] : -1;
    cut.zs = exact ? add_m + (double)L.hmass[hslot(d)] * kInvFix : -1.0;
    __syncthreads();
    return cut;
  }
  // several values in the boundary bin: its elements, sorted, decide
  const int nd = (int)L.hcnt[hslot(d)];
  __syncthreads();
  if (nd > kCap) {
    *ok = false;
    return cut;
  }
  if (tid == 0) L.si[6] = 0;
  __syncthreads();
#pragma unroll 1
  for (int j = 0; j < NC; ++j) {
    float v[EPC];
    r.elems(j, v);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if (v[e] > kNegInf) {
        const int b = (int)fminf(fmaf(v[e], -(float)kVRes, M32), (float)(kVBins - 1));
        const bool hit = b == d;
        const unsigned long long m = __ballot(hit);
        if (m) {   // one counter update per wavefront
          const int first = __builtin_ctzll(m);
          int at = 0;
          if (__lane_id() == first) at = atomicAdd(&L.si[6], __popcll(m));
          at = __builtin_amdgcn_readlane(at, first);
          if (hit)
            L.key[at + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] =
                cand_key(v[e], r.base(j) + e);
        }
      }
    }
  }
  __syncthreads();
  sort_keys_desc(L, nd);
  const Resolved res = resolve_sorted(L, nd, add_c, add_m, M, c, f, thr, false);
  if (res.n_in > 0) {
    cut.tau = fmaxf(res.tau, floor_m);
    const bool exact = !(floor_m > res.tau);
    cut.kept = exact ? add_c + res.n_in : -1;
    cut.zs = exact ? res.zs : -1.0;
  } else {            // nothing of the bin stays: S is what lies above it
    cut.tau = fmaxf(next_up(key2f(key_hi(L.key[0]))), floor_m);
    cut.kept = -1;
    cut.zs = -1.0;
  }
  __syncthreads();
  return cut;
}

// The kept set of a register-resident row whose candidates did not fit the
// LDS buffer: the histogram search of the streaming path, over the registers
// (for JOINT bf16 rows, the exact value histogram above first).
template <int DT, int NC>
__device__ __forceinline__ Cut reg_general(const RegRow<DT, NC>& r, float M, float c, float cR,
                                           const Filters& f, Lds& L) {
  if (!f.k_on && !f.p_on) {   // min-p alone: its cut is the kept set
    Cut cut;
    cut.tau = f.tau_m > kNegInf ? f.tau_m : -kFltMax;
    cut.kept = -1;
    cut.zs = -1.0;
    return cut;
  }
  if constexpr (DT == 1) {
    if (!(f.seq && f.k_on && f.p_on) && fabsf(M) <= 32768.0f) {
      bool ok;
      const Cut cut = bf16_value_cut(r, M, c, f, L, &ok);
      if (ok) return cut;
    }
  }
  const RegView<DT, NC> s{r};
  if (f.seq && f.k_on && f.p_on) {
    // SEQUENTIAL: top-k alone first; its kept mass is top-p's reference
    Filters fk = f;
    fk.p_on = false;
    fk.m_on = false;
    fk.tau_m = kNegInf;
    const Cut ck = general_search<DT>(s, M, c, cR, fk, 0.0);
    const double zk = ck.zs >= 0.0 ? ck.zs : reg_kept_mass(r, ck.tau, M, c, L);
    return general_search<DT>(s, M, c, cR, f, f.top_p * zk);
  }
  const double Z = f.p_on ? reg_weight_sum(r, M, c, L) : 0.0;
  return general_search<DT>(s, M, c, cR, f, f.p_on ? f.top_p * Z : 0.0);
}

// ---------------------------------------------------------------- greedy

template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void greedy_kernel(const unsigned char* logits,
                                                        long long stride_bytes, int V,
                                                        int ragged, int32_t* out,
                                                        int32_t* status) {
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  const int row = blockIdx.x;
  RegRow<DT, NC> r;
  r.load(logits + (long long)row * stride_bytes, V, ragged != 0);
  const RowStats st = reg_stats(r, false, 1.0f, L);
  int tok = -1;
  if (st.status == 0) tok = reg_argmax(r, st.M, L);
  if (threadIdx.x == 0) {
    out[row] = tok;
    if (status) status[row] = st.status;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void greedy_kernel_stream(const unsigned char* logits,
                                                               long long stride_bytes, int V,
                                                               int32_t* out, int32_t* status) {
  TSR_TRACE_INIT(nullptr);
  const int row = blockIdx.x;
  const StreamRow<DT> s(logits + (long long)row * stride_bytes, V);
  const StreamStats st = stream_stats(s, false, 1.0f);
  int tok = -1;
  if (st.status == 0) tok = stream_argmax(s, st.M);
  if (threadIdx.x == 0) {
    out[row] = tok;
    if (status) status[row] = st.status;
  }
}

// ---------------------------------------------------------------- sample_rows

// The streaming view of row `row` (for the streaming finish and the
// diagnostics), with the allowed-token mask (EXT 1) and the repetition
// penalty (EXT 1 or 2, when asked for).
template <int DT, int EXT>
__device__ __forceinline__ StreamRow<DT> row_stream_view(const unsigned char* p, int V,
                                                         const KParams& kp, int row) {
  return StreamRow<DT>(p, V,
                       EXT == 1 ? kp.allowed + (long long)row * kp.allowed_stride : nullptr,
                       ((EXT == 1 || EXT == 2) && (kp.flags & F_REP)) ? kp.hist_len : 0,
                       kp.rpen);
}

// WIDE (bf16): rows whose kept set the candidate bound cannot narrow are
// finished over the registers (reg_general, then the walk) instead of by the
// streaming path. A separate instance, chosen on the host for filters without
// a small top-k, so the common instance keeps its registers and code size.
// EXT 1: an allowed-token bitmask applies (constrained decoding), its words
// read into registers ahead of the row and applied in pass A, and a
// repetition penalty may (F_REP); EXT 2: a repetition penalty applies.
// The bf16 instances of EXT 1-2 are WIDE.
template <int DT, int NC, bool WIDE, int EXT>
__global__ __launch_bounds__(kBlock) void sample_kernel(const unsigned char* logits,
                                                        long long stride_bytes, int V,
                                                        int ragged, KParams kp0,
                                                        int32_t* out, DiagPtrs dg) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  const int row = blockIdx.x;
  const unsigned char* p = logits + (long long)row * stride_bytes;
  constexpr bool MASK = EXT == 1, REP = EXT == 1 || EXT == 2;
  KParams kp = kp0;
#if TSR_TRACE
  TSR_TRACE_INIT(kp0.trace);
  TSR_STAMP(kStEntry);
#endif
  if ((kp.flags & F_ROWP) && !row_kparams(kp, row, V)) {
    write_row(row, -1, kRowBadParam, 0, kNegInf, 0.0, kNaN, kNaN, out, dg);
    zero_probs(dg, row, V);
    return;
  }
  RegRow<DT, NC> r;
  RowExtras x;
  if (REP && (kp.flags & F_REP)) {   // the window ids, read by wave 0 before the row
    x.hn = kp.hist_len;
    x.r = kp.rpen;
    x.row = p;
    if ((int)threadIdx.x < x.hn) x.hv = kp.hist[(long long)row * kp.hist_stride + threadIdx.x];
  }
  MaskRegs<DT, NC> mk;
  if constexpr (MASK) mk.load(kp.allowed + (long long)row * kp.allowed_stride, V);
  r.load(p, V, ragged != 0);
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const double u = draw_uniform(kp, (uint32_t)row, 0u, 0u, 0);
  asm volatile("" ::"s"(u));   // the draw's uniform while the loads fly
  TSR_STAMP(kStIssued);
  const RowStats st = reg_stats<MASK, REP>(r, !greedy && joint_top_p(kp), kp.c, L, V, x, &mk);
  if (st.status != 0) {
    write_row(row, -1, st.status, 0, kNegInf, 0.0, kNaN, kNaN, out, dg);
    zero_probs(dg, row, V);
    return;
  }
  if (greedy) {
    greedy_row(row, reg_argmax(r, st.M, L), st.M, V, out, dg);
    return;
  }
  const float M = st.M, c = kp.c;
  const Filters f = make_filters(kp, M);
  TSR_STAMP(kStCutStart);
  float tau = -kFltMax;     // no filter: every finite logit
  int kept = -1, tok;
  double zs, wt;
  if (f.k_on || f.p_on || f.m_on) {
    // the cut and the draw; the registers are dead afterwards. Without min-p
    // or a small top-k the WIDE instance goes straight to its register search
    // (no candidate bound can narrow a wide kept set).
    const bool narrow =
        f.m_on || ((EXT != 0 || (kp.flags & F_ROWP)) && f.k_on && f.k <= kBlock / 4);
    FastOut fo{0, 0, -1, kPosInf, 0, 0.0, 0.0};
    if (!(WIDE && DT == 1) || narrow)
      fo = fast_cut<MASK>(r, V, M, st.tmin, st.zlo, c, f, u, L, st.nallow);
    if (fo.ok) {
      tau = fo.tau;
      kept = fo.kept;
      zs = fo.zs;
      wt = fo.wtok;
      tok = fo.token;
    } else if constexpr (DT == 1 && WIDE) {
      // too many candidates for the LDS buffer: the search over the registers
      // (the exact value histogram of bf16 rows), then the walk
      const Cut cut = reg_general(r, M, c, kp.cR, f, L);
      TSR_STAMP(kStGeneral);
      tau = cut.tau;
      kept = cut.kept;
      tok = walk_regs<NC, EPC>(KeptWeights<DT, NC>{r, tau, M, c}, u, L, &zs, &wt);
      TSR_STAMP(kStWalk);
    } else {
      // the streaming path finishes this row
      stream_finish(row_stream_view<DT, EXT>(p, V, kp, row), row, M, -1.0, kp, f, u, out, dg);
      return;
    }
  } else {
    tok = walk_regs<NC, EPC>(KeptWeights<DT, NC>{r, tau, M, c}, u, L, &zs, &wt);
    TSR_STAMP(kStWalk);
  }
  if (dg.kept_count || dg.threshold || dg.kept_mass || dg.probs) {
    diag_finish(row_stream_view<DT, EXT>(p, V, kp, row), row, tok, kept, tau, M, c, zs, wt, out,
                dg);
    return;
  }
  write_row(row, tok, 0, kept, tau, 0.0, wt, zs, out, dg);
  TSR_STAMP(kStEnd);
  TSR_TRACE_FLUSH();
}

// Rows wider than the register file: every pass streams the row.
template <int DT>
__global__ __launch_bounds__(kBlock) void sample_kernel_stream(const unsigned char* logits,
                                                               long long stride_bytes, int V,
                                                               KParams kp0, int32_t* out,
                                                               DiagPtrs dg) {
  const int row = blockIdx.x;
  const unsigned char* p = logits + (long long)row * stride_bytes;
  KParams kp = kp0;
  TSR_TRACE_INIT(nullptr);
  if ((kp.flags & F_ROWP) && !row_kparams(kp, row, V)) {
    write_row(row, -1, kRowBadParam, 0, kNegInf, 0.0, kNaN, kNaN, out, dg);
    zero_probs(dg, row, V);
    return;
  }
  int hn = 0;
  if (kp.flags & F_REP) {   // publish the look-back window before any read
    hn = kp.hist_len;
    if (threadIdx.x < kWave)
      hist_publish<DT>((int)threadIdx.x < hn ? kp.hist[(long long)row * kp.hist_stride + threadIdx.x]
                                             : -1,
                       hn, V, tsr_lds);
    __syncthreads();
  }
  const StreamRow<DT> s(p, V,
                        (kp.flags & F_MASK) ? kp.allowed + (long long)row * kp.allowed_stride
                                            : nullptr,
                        hn, kp.rpen);
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const StreamStats st = stream_stats(s, !greedy && wants_z(kp), kp.c);
  if (st.status != 0) {
    write_row(row, -1, st.status, 0, kNegInf, 0.0, kNaN, kNaN, out, dg);
    zero_probs(dg, row, V);
    return;
  }
  if (greedy) {
    greedy_row(row, stream_argmax(s, st.M), st.M, V, out, dg);
    return;
  }
  const Filters f = make_filters(kp, st.M);
  const double u = draw_uniform(kp, (uint32_t)row, 0u, 0u, 0);
  stream_finish(s, row, st.M, st.z, kp, f, u, out, dg);
}

// ---------------------------------------------------------------- beam step

// The k (<= kBeamMax) largest finite logits of a register-resident row, lowest
// id first among equals, as order keys fkey(v) << 32 | ~id in L.key[0, n),
// descending; returns n = min(k, finite elements). The top-k sketch bounds the
// candidates; up to one wavefront's worth are sorted in registers, up to kCap
// in LDS; beyond that (a tie group of thousands at the boundary) k rounds of a
// block-wide maximum below the previous key.
template <int DT, int NC>
__device__ __forceinline__ int reg_top_keys(const RegRow<DT, NC>& r, float M, float tmin, int k,
                                         Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int tid = threadIdx.x, lane = __lane_id(), wid = tid / kWave;
  float Lb = topk_sketch(r, M, tmin, k, L);
  if (!(Lb > -kFltMax)) Lb = -kFltMax;   // fewer than k maxima: every finite element
  __syncthreads();
  wave_compact(r, Lb, L);
  __syncthreads();
  const int total = wave_regions_total(L);
  if (total <= kWaveCap) {
    if (tid < kWave) {
      int n = 0, sq = 0, so = 0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        const int cq = L.wcnt[q];
        if (lane >= n && lane < n + cq) {
          sq = q;
          so = lane - n;
        }
        n += cq;
      }
      unsigned long long key = 0ull;
      if (lane < n) key = cand_key(__uint_as_float(L.wc[sq].val[so]), (int)L.wc[sq].idx[so]);
      key = wave_sort_desc<kWave>(key);
      if (lane < k) L.key[lane] = key;
    }
    __syncthreads();
    return total < k ? total : k;
  }
  // one thread's candidates >= Lb, counted, then compacted in thread order
  const unsigned long long cmask = wave_chunk_mask<NC>([&](int j) { return r.cmax(j) >= Lb; });
  int cnt = 0;
  for (unsigned long long m = cmask; m;) {
    const int j = pop_low(m);
    float v[EPC];
    r.elems(j, v);
#pragma unroll
    for (int e = 0; e < EPC; ++e) cnt += (v[e] >= Lb) ? 1 : 0;
  }
  int all;
  int off = block_excl_scan<kBlock>(cnt, &all, L.bs);
  if (all <= kCap) {
    for (unsigned long long m = __any(cnt != 0) ? cmask : 0ull; m;) {
      const int j = pop_low(m);
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (v[e] >= Lb) L.key[off++] = cand_key(v[e], r.base(j) + e);
    }
    __syncthreads();
    sort_keys_desc(L, all);
    return all < k ? all : k;
  }
  unsigned long long prev = ~0ull;
  int n = 0;
  for (; n < k; ++n) {
    unsigned long long best = 0ull;
    for (unsigned long long m = cmask; m;) {
      const int j = pop_low(m);
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const unsigned long long key = cand_key(v[e], r.base(j) + e);
        if (v[e] >= Lb && key < prev && key > best) best = key;
      }
    }
    best = wave_reduce(best, [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
    __syncthreads();
    if (lane == 0) L.hmass[wid] = best;   // (histogram masses: free here)
    __syncthreads();
    best = 0ull;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) best = L.hmass[q] > best ? L.hmass[q] : best;
    if (best == 0ull) break;
    __syncthreads();
    if (tid == 0) L.key[n] = best;
    prev = best;
  }
  __syncthreads();
  return n;
}

// One beam-search step [P2 39.1, eq. 39.1 and Listing 39.1]: workgroup row =
// g * beam + b holds beam b of group g. It writes its best candidates
// (score s_b + log p_b(i), token), best first, to the workspace; a
// one-wavefront kernel per group that follows in the stream (launch_beam)
// merges the beams' sorted lists (equal scores: lower b first) and writes the
// group's output.
template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void beam_kernel(const unsigned char* logits,
                                                      long long stride_bytes, int V,
                                                      int ragged, int beam, const double* scores,
                                                      BeamWs ws) {
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const unsigned char* p = logits + (long long)row * stride_bytes;
  RegRow<DT, NC> r;
  r.load(p, V, ragged != 0);
  const double sb = scores[row];
  // the row's weight sum Z is formed as the chunks land (log p = v - M - ln Z)
  const RowStats st = reg_stats<false, false, true>(r, true, kLog2e, L);
  const bool bad = st.status == 1 || sb != sb || sb == (double)kPosInf;
  int n = 0;
  double lnz = 0.0;
  if (!bad && st.status == 0 && sb > (double)kNegInf) {
    lnz = log(st.zlo);
    n = reg_top_keys(r, st.M, st.tmin, beam, L);
  }
  if (tid == 0) {
    // the row's list for the group merge that follows in the stream (a bad
    // row marks its first score NaN, which no other row's list holds)
    for (int q = 0; q < beam; ++q) {
      double sc = (double)kNegInf;
      int tk = -1;
      if (q < n) {
        const unsigned long long key = L.key[q];
        sc = sb + ((double)key2f(key_hi(key)) - (double)st.M) - lnz;
        tk = (int)~(uint32_t)key;
      }
      if (bad && q == 0) sc = __builtin_nan("");
      const long long slot = (long long)row * kBeamMax + q;
      ws.score[slot] = sc;
      ws.tok[slot] = tk;
    }
  }
}

// ---------------------------------------------------------------- verify

// Residual weights max(0, p~ - q~) of one verify position (eq. 39.4), both
// rows resident in this workgroup with the same element layout.
// The residual's per-element weight max(0, p~ - q~), with p~ = w_p / Z_p over
// {a >= tp} and q~ likewise: in float, like the weights themselves (their
// exponentials are float; double steps after them add no accuracy).
__device__ __forceinline__ float residual_weight(float a, float b, float tp, float Mp, float tq,
                                                 float Mq, float c, float izp, float izq) {
  const float pe = a >= tp ? weight(a, Mp, c) * izp : 0.0f;
  const float qe = b >= tq ? weight(b, Mq, c) * izq : 0.0f;
  return fmaxf(pe - qe, 0.0f);
}

template <int DT, int NC>
struct ResidualWeights {
  const RegRow<DT, NC>& rp;
  const RegRow<DT, NC>& rq;
  float tp, Mp, tq, Mq, c;
  float izp, izq;   // 1 / Z_p, 1 / Z_q
  __device__ __forceinline__ void operator()(int j, float* w) const {
    constexpr int EPC = Fmt<DT>::EPC;
    if (tp == -kFltMax && tq == -kFltMax) {   // both rows keep every element
      float a[EPC], b[EPC];
      rp.elems(j, a);
      rq.elems(j, b);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        w[e] = fmaxf(weight(a[e], Mp, c) * izp - weight(b[e], Mq, c) * izq, 0.0f);
      return;
    }
    if (rp.cmax(j) >= tp) {
      float a[EPC], b[EPC];
      rp.elems(j, a);
      rq.elems(j, b);
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = residual_weight(a[e], b[e], tp, Mp, tq, Mq, c, izp, izq);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = 0.0f;
    }
  }
};

// Tree verify: the target distribution left at a node after k rejected
// candidates, p_{k+1} = max(0, p_k - q~) normalised (p_1 = p~; a step whose
// residual sum is zero leaves p unchanged: zinv 0), per element; L.tz[s]
// holds 1 / Z of step s. LAST: the unnormalised residual of one more step
// (for its sum). The weights are relative (the walk normalises).
template <int DT, int NC, bool LAST>
struct TreeWeights {
  const RegRow<DT, NC>& rp;
  const RegRow<DT, NC>& rq;
  float tp, Mp, tq, Mq, c;
  double inv_zp, inv_zq;
  int k;
  const Lds& L;
  __device__ __forceinline__ double pk(double pe, double qe) const {
    for (int s2 = 0; s2 < k; ++s2) {
      const double zi = L.tz[s2];
      if (zi > 0.0) pe = fmax(0.0, pe - qe) * zi;
    }
    return pe;
  }
  __device__ __forceinline__ void operator()(int j, float* w) const {
    constexpr int EPC = Fmt<DT>::EPC;
    if (rp.cmax(j) >= tp) {
      float a[EPC], b[EPC];
      rp.elems(j, a);
      rq.elems(j, b);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const double pe = a[e] >= tp ? (double)weight(a[e], Mp, c) * inv_zp : 0.0;
        const double qe = b[e] >= tq ? (double)weight(b[e], Mq, c) * inv_zq : 0.0;
        double x = pk(pe, qe);
        if (LAST) x = fmax(0.0, x - qe);
        w[e] = (float)x;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = 0.0f;
    }
  }
};

// Block-wide sum of a per-element weight functor over the register row.
template <int NC, int EPC, class CW>
__device__ __forceinline__ double reg_functor_sum(const CW& cw, Lds& L) {
  double acc = 0.0;
#pragma nounroll
  for (int j = 0; j < NC; ++j) {
    float w[EPC];
    cw(j, w);
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) t += w[e];
    acc += (double)t;
  }
  return block_sum<kBlock>(acc, L.bs);
}

struct RowCut {
  int status;
  float M;
  float tau;
  double zs;     // weight sum over S
};

// Status, row max and kept set of a resident row, with the exact kept weight.
// need_zs false: a row that only draws from its own p~ (the walk forms the
// sum), so Z_S is left out where it would take a pass of its own (zs -1).
template <int DT, int NC>
__device__ __forceinline__ RowCut verify_row_cut(RegRow<DT, NC>& r, int V, const KParams& kp,
                                                 Lds& L, bool need_zs = true) {
  const RowStats st = reg_stats(r, joint_top_p(kp), kp.c, L);
  RowCut rc{st.status, st.M, kPosInf, 0.0};
  if (st.status != 0) return rc;
  const Filters f = make_filters(kp, st.M);
  if (!f.k_on && !f.p_on && !f.m_on) {
    rc.tau = -kFltMax;
    rc.zs = need_zs ? reg_kept_mass(r, rc.tau, st.M, kp.c, L) : -1.0;
    return rc;
  }
  const FastOut fo = fast_cut(r, V, st.M, st.tmin, st.zlo, kp.c, f, 0.0, L);
  if (fo.ok) {
    rc.tau = fo.tau;
    rc.zs = fo.zs;
    return rc;
  }
  const Cut cut = reg_general(r, st.M, kp.c, kp.cR, f, L);
  rc.tau = cut.tau;
  rc.zs = need_zs ? reg_kept_mass(r, rc.tau, st.M, kp.c, L) : -1.0;
  return rc;
}

template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void verify_kernel(const unsigned char* tgt,
                                                        const unsigned char* dft,
                                                        const int32_t* xs, int K, int V,
                                                        int ragged, KParams kp,
                                                        VerifyWs ws) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  // the draft positions (two rows each) first, then every sequence's bonus
  // position (the target row only): when the grid exceeds the device, the
  // lighter workgroups are the ones that wait
  const int nseq = (int)gridDim.x / (K + 1);
  const int blk = (int)blockIdx.x;
  const int b = blk < nseq * K ? blk / K : blk - nseq * K;
  const int j = blk < nseq * K ? blk - b * K : K;
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const unsigned char* tp = tgt + ((long long)b * (K + 1) + j) * rowbytes;
  const unsigned char* dp = dft + ((long long)b * K + (j < K ? j : 0)) * rowbytes;
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const bool with_draft = !greedy && j < K;
  RegRow<DT, NC> rp, rq;
  rp.load(tp, V, ragged != 0);
  if (with_draft) rq.load(dp, V, ragged != 0);
  asm volatile("" ::: "memory");   // both rows' loads in flight before any use
  int st_t = 0, st_d = 0, acc = 0, tok = -1;
  const int x = j < K ? xs[(long long)b * K + j] : 0;
  const bool x_ok = x >= 0 && x < V;
  if (greedy) {
    const RowStats s = reg_stats(rp, false, 1.0f, L);
    st_t = s.status;
    if (st_t == 0) {
      tok = reg_argmax(rp, s.M, L);
      acc = (j < K && x == tok) ? 1 : 0;
    }
  } else {
    // the bonus row (j = K) only draws from p~: no separate kept-mass pass
    const RowCut cp = verify_row_cut(rp, V, kp, L, j < K);
    st_t = cp.status;
    const double u0 = draw_uniform(kp, (uint32_t)b, (uint32_t)j, 1u, 0);
    const double u1 = draw_uniform(kp, (uint32_t)b, (uint32_t)j, 1u, 1);
    if (j == K) {
      if (st_t == 0) {
        double zs;
        tok = walk_regs<NC, EPC>(KeptWeights<DT, NC>{rp, cp.tau, cp.M, kp.c}, u0, L, &zs);
      }
    } else {
      const RowCut cq = verify_row_cut(rq, V, kp, L);
      st_d = cq.status;
      if (st_t == 0 && st_d == 0 && x_ok) {
        const float lp = load_elem<DT>(tp, x), lq = load_elem<DT>(dp, x);
        const double pt = lp >= cp.tau ? (double)weight(lp, cp.M, kp.c) / cp.zs : 0.0;
        const double qt = lq >= cq.tau ? (double)weight(lq, cq.M, kp.c) / cq.zs : 0.0;
        const double a = fmin(1.0, pt / fmax(qt, 1e-300));
        acc = u0 < a ? 1 : 0;
        if (!acc) {
          double zr;
          tok = walk_regs<NC, EPC>(ResidualWeights<DT, NC>{rp, rq, cp.tau, cp.M, cq.tau, cq.M,
                                                           kp.c, (float)(1.0 / cp.zs),
                                                           (float)(1.0 / cq.zs)},
                                   u1, L, &zr);
          if (!(zr > 0.0)) {
            double zs;
            tok = walk_regs<NC, EPC>(KeptWeights<DT, NC>{rp, cp.tau, cp.M, kp.c}, u1, L, &zs);
          }
        }
      }
    }
  }
  if (threadIdx.x == 0) {   // the position's results, for the finish kernel
    const int slot = b * ws.kmax1 + j;
    ws.acc[slot] = acc;
    ws.tok[slot] = tok;
    ws.st_t[slot] = st_t;
    ws.st_d[slot] = st_d;
  }
}

// Tree (multi-candidate) verify [P3 "Extensions and Variants"; P2 39.4]: one
// workgroup per (sequence b, node v). Node v's children (nodes whose parent
// is v, in node order) are its candidates, tested in order against the
// target distribution the earlier rejections left (p_1 = p~_v, then
// max(0, p_c - q~_v) normalised); the first kept child, or else a draw from
// the final p (w1 of the node's counter), is the node's result. The
// sequence's last workgroup follows kept children from the root and writes
// the emitted tokens and the accepted path. The tree (parent ids, tokens) is
// read by every workgroup; N <= 32.
template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void tree_kernel(const unsigned char* tgt,
                                                      const unsigned char* dft,
                                                      const int32_t* parent, const int32_t* tokens,
                                                      int N, int V, int ragged, KParams kp,
                                                      VerifyWs ws, int32_t* out_tokens,
                                                      int32_t* out_path, int32_t* out_acc,
                                                      int32_t* out_status) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  // node-major order: earlier nodes (the ones likely to have children, two
  // rows to read) are dispatched before the later ones (leaves, one row)
  const int nseq = (int)gridDim.x / N;
  const int v = (int)blockIdx.x / nseq;
  const int b = (int)blockIdx.x - v * nseq;
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const unsigned char* tp = tgt + ((long long)b * N + v) * rowbytes;
  const unsigned char* dp = dft + ((long long)b * N + v) * rowbytes;
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  // the tree, one node per lane (every wavefront reads it)
  const int lane = __lane_id();
  const bool ln = lane < N;
  const int pa = ln ? parent[(long long)b * N + lane] : 0;
  const int tk = ln ? tokens[(long long)b * N + lane] : 0;
  const bool bad_tree =
      __ballot(ln && (lane == 0 ? pa != -1 : (pa < 0 || pa >= lane))) != 0ull;
  const bool bad_tok = __ballot(ln && lane > 0 && (tk < 0 || tk >= V)) != 0ull;
  const unsigned long long chm = __ballot(ln && lane > 0 && pa == v);
  const bool with_draft = !greedy && chm != 0ull;
  RegRow<DT, NC> rp, rq;
  rp.load(tp, V, ragged != 0);
  if (with_draft) rq.load(dp, V, ragged != 0);
  asm volatile("" ::: "memory");
  int st_t = 0, st_d = 0, kept = -1, tok = -1;
  if (greedy) {
    const RowStats st = reg_stats(rp, false, 1.0f, L);
    st_t = st.status;
    if (st_t == 0) {
      tok = reg_argmax(rp, st.M, L);
      const unsigned long long hit = chm & __ballot(tk == tok);
      kept = hit ? __ffsll((long long)hit) - 1 : -1;
    }
  } else {
    // a node without children only draws from p~: no separate kept-mass pass
    const RowCut cp = verify_row_cut(rp, V, kp, L, with_draft);
    st_t = cp.status;
    RowCut cq{0, 0.0f, kPosInf, 1.0};
    if (with_draft) {
      cq = verify_row_cut(rq, V, kp, L);
      st_d = cq.status;
    }
    if (st_t == 0 && st_d == 0 && !bad_tree && !bad_tok) {
      const double izp = 1.0 / cp.zs, izq = with_draft ? 1.0 / cq.zs : 0.0;
      int k = 0;
      for (unsigned long long m = chm; m; m &= m - 1ull, ++k) {
        const int child = __ffsll((long long)m) - 1;
        const int x = readlane_u32((uint32_t)tk, child);
        const float lp = load_elem<DT>(tp, x), lq = load_elem<DT>(dp, x);
        const double pe = lp >= cp.tau ? (double)weight(lp, cp.M, kp.c) * izp : 0.0;
        const double qe = lq >= cq.tau ? (double)weight(lq, cq.M, kp.c) * izq : 0.0;
        const TreeWeights<DT, NC, false> tw{rp, rq, cp.tau, cp.M, cq.tau, cq.M, kp.c, izp, izq, k, L};
        const double pc = tw.pk(pe, qe);
        const double a = fmin(1.0, pc / fmax(qe, 1e-300));
        if (draw_uniform(kp, (uint32_t)b, (uint32_t)(v * 32 + k), 2u, 0) < a) {
          kept = child;
          break;
        }
        // rejected: the next residual's normaliser
        const double z = reg_functor_sum<NC, EPC>(
            TreeWeights<DT, NC, true>{rp, rq, cp.tau, cp.M, cq.tau, cq.M, kp.c, izp, izq, k, L}, L);
        if (threadIdx.x == 0) L.tz[k] = z > 0.0 ? 1.0 / z : 0.0;
        __syncthreads();
      }
      if (kept < 0) {
        const double u1 = draw_uniform(kp, (uint32_t)b, (uint32_t)(v * 32), 2u, 1);
        double zt;
        if (k == 0)
          tok = walk_regs<NC, EPC>(KeptWeights<DT, NC>{rp, cp.tau, cp.M, kp.c}, u1, L, &zt);
        else
          tok = walk_regs<NC, EPC>(
              TreeWeights<DT, NC, false>{rp, rq, cp.tau, cp.M, cq.tau, cq.M, kp.c, izp, izq, k, L},
              u1, L, &zt);
      }
    }
  }
  if (threadIdx.x == 0) {
    const int slot = b * ws.kmax1 + v;
    __hip_atomic_store(&ws.acc[slot], kept, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ws.tok[slot], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ws.st_t[slot], st_t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ws.st_d[slot], st_d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t prev = __hip_atomic_fetch_add(&ws.counter[b], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    L.si[0] = prev == (uint32_t)(N - 1);
  }
  __syncthreads();
  if (!L.si[0] || threadIdx.x >= kWave) return;
  // the sequence's last workgroup, wave 0 (lane n: node n)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int s0 = b * ws.kmax1;
  const int nt = ln ? __hip_atomic_load(&ws.st_t[s0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  const int nd = ln ? __hip_atomic_load(&ws.st_d[s0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  const int nk = ln ? __hip_atomic_load(&ws.acc[s0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -1;
  const int ntok = ln ? __hip_atomic_load(&ws.tok[s0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -1;
  const unsigned long long bt = __ballot(nt != 0), bd = __ballot(nd != 0);
  const int status = bad_tree ? 5
                     : bt ? readlane_u32((uint32_t)nt, __ffsll((long long)bt) - 1)
                     : bd ? readlane_u32((uint32_t)nd, __ffsll((long long)bd) - 1)
                     : (bad_tok ? 3 : 0);
  int32_t* ot = out_tokens + (long long)b * N;
  int32_t* op = out_path + (long long)b * N;
  // follow the kept children from the root (every lane in step); lane q
  // keeps the q-th step's node and token
  int n = 0, my_node = -1, my_tok = -1;
  if (!status) {
    int node = 0;
    for (int guard = 0; guard < N; ++guard) {
      const int ch = (int)readlane_u32((uint32_t)nk, node);
      if (ch < 0) break;
      const int t = (int)readlane_u32((uint32_t)tk, ch);
      my_node = lane == n ? ch : my_node;
      my_tok = lane == n ? t : my_tok;
      ++n;
      node = ch;
    }
    const int last = (int)readlane_u32((uint32_t)ntok, node);
    my_tok = lane == n ? last : my_tok;
  }
  if (ln) {
    ot[lane] = my_tok;
    op[lane] = my_node;
  }
  if (lane == 0) {
    out_acc[b] = n;
    if (out_status) out_status[b] = status;
    __hip_atomic_store(&ws.counter[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

static __global__ void philox_kernel(const uint32_t* ctr, int n, uint32_t k0, uint32_t k1,
                                     uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const uint4 c = make_uint4(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]);
    const uint4 w = philox4x32_10(c, k0, k1);
    out[4 * i] = w.x;
    out[4 * i + 1] = w.y;
    out[4 * i + 2] = w.z;
    out[4 * i + 3] = w.w;
  }
}

}  // namespace tsr
