// The register-resident fast path: one workgroup holds its row in VGPRs
// (thread t owns 16-byte chunks j*kBlock + t, j < NC), reads HBM once and
// resolves the kept set from a few candidates staged in LDS.
//
// Candidate bound Lb <= tau: min-p gives a logit threshold directly; top-k
// uses a sketch, the k-th largest of the per-thread (or per-chunk) maxima,
// which can only be at or below the k-th largest logit. The logits >= Lb are
// the candidates; at most kWaveCap of them are resolved and drawn by one
// wavefront with no barriers, up to kCap by the whole workgroup.
#pragma once

#include "row_common.hpp"

namespace tsr {

template <int DT, int NC>
struct RegRow {
  static constexpr int EPC = Fmt<DT>::EPC;
  uint4 raw[NC];
  float cm[NC];   // chunk maxima; -inf past the end of the row
  float tmax;     // this thread's maximum

  int nwhole;     // whole 16-byte chunks in the row (chunk ids at or past it are not)
  uint4 tail;     // the partial chunk, read element-wise, when the row is ragged

  // Whole chunks of a 16-byte aligned row are 128-bit buffer loads off one
  // resource, all issued back to back with no per-load address registers.
  // Chunks at or past `nwhole` come back as zeros from the range check and are
  // replaced in pass A of reg_stats (by -inf, or by `tail` for the partial
  // chunk of a ragged row), so no wait is forced here. UNALIGNED rows are read
  // element-wise.
  template <bool UNALIGNED = false>
  __device__ __forceinline__ void load(const unsigned char* p, int V, bool ragged) {
    if constexpr (UNALIGNED) {
      nwhole = 0x7FFFFFFF;
      tail = neg_inf_chunk<DT>();
#pragma unroll
      for (int j = 0; j < NC; ++j)
        raw[j] = load_chunk_slow<DT>(p, (long long)j * kBlock + threadIdx.x, V);
    } else {
      nwhole = V / EPC;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(p), (short)0, nwhole * 16, 0x00020000);
      const int voff = (int)threadIdx.x * 16;
#pragma unroll
      for (int j = 0; j < NC; ++j)
        raw[j] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * kBlock * 16, 0));
      tail = neg_inf_chunk<DT>();
      if (ragged && nwhole * EPC < V && (nwhole % kBlock) == (int)threadIdx.x)
        tail = load_chunk_slow<DT>(p, nwhole, V);
    }
  }
  // Pass-A fix-up of chunk j (see load).
  __device__ __forceinline__ uint4 settle(int j, uint4 t) const {
    const int cid = j * kBlock + (int)threadIdx.x;
    if (cid >= nwhole) t = cid == nwhole ? tail : neg_inf_chunk<DT>();
    return t;
  }
  __device__ __forceinline__ int base(int j) const {
    return (j * kBlock + (int)threadIdx.x) * EPC;
  }
  // Packed chunk j. The empty asm makes each pass unpack afresh from the
  // packed registers instead of keeping unpacked copies alive between passes.
  __device__ __forceinline__ uint4 packed(int j) const {
    uint4 t = raw[j];
    asm volatile("" : "+v"(t.x), "+v"(t.y), "+v"(t.z), "+v"(t.w));
    return t;
  }
  __device__ __forceinline__ void elems(int j, float* v) const { unpack<DT>(packed(j), v); }
};

// NaN detector on packed data: the running maximum of the magnitude bits of
// every element. A NaN has magnitude bits above those of infinity.
template <int DT> struct NanAcc;
template <> struct NanAcc<0> {
  uint32_t a = 0u;
  __device__ __forceinline__ void add(uint4 t) {
    a = max(a, max(max(t.x & 0x7FFFFFFFu, t.y & 0x7FFFFFFFu),
                   max(t.z & 0x7FFFFFFFu, t.w & 0x7FFFFFFFu)));
  }
  __device__ __forceinline__ bool nan() const { return a > 0x7F800000u; }
};
template <> struct NanAcc<1> {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 a = {0, 0};
  __device__ __forceinline__ static us2 mag(uint32_t w) {
    return __builtin_bit_cast(us2, w & 0x7FFF7FFFu);
  }
  __device__ __forceinline__ void add(uint4 t) {
    a = __builtin_elementwise_max(
        a, __builtin_elementwise_max(__builtin_elementwise_max(mag(t.x), mag(t.y)),
                                     __builtin_elementwise_max(mag(t.z), mag(t.w))));
  }
  __device__ __forceinline__ bool nan() const { return a.x > 0x7F80u || a.y > 0x7F80u; }
};

struct RowStats {
  int status;     // TSR_ROW_*
  float M;        // row max
  float smin;     // smallest finite chunk maximum
  double z;       // sum of weights over the row (when asked for)
};

// Row statistics in two passes over the registers. Pass A runs as the loads
// land: NaN/+inf detection, chunk maxima, thread max. Pass B (only when the
// weight sum is wanted) sums 2^((v - m_t) c) against the thread's own max m_t:
// no running rescale, so every chunk is independent work. One barrier round
// combines the waves.
template <int DT, int NC>
__device__ __forceinline__ RowStats reg_stats(RegRow<DT, NC>& r, bool need_z, float c, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  float tmax = kNegInf, smin = kPosInf;
  NanAcc<DT> nan;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const uint4 t = r.settle(j, r.packed(j));
    r.raw[j] = t;
    nan.add(t);
    float v[EPC];
    unpack<DT>(t, v);
    float m = fmaxf(v[0], v[1]);
#pragma unroll
    for (int e = 2; e < EPC; ++e) m = fmaxf(m, v[e]);
    r.cm[j] = m;
    tmax = fmaxf(tmax, m);
    smin = m > kNegInf ? fminf(smin, m) : smin;
    sched_fence();
  }
  r.tmax = tmax;
  double zt = 0.0;
  if (need_z && tmax > kNegInf && tmax < kPosInf) {
    double acc[2] = {0.0, 0.0};
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float v[EPC];
      r.elems(j, v);
      float s[EPC / 2];
#pragma unroll
      for (int e = 0; e < EPC / 2; ++e)
        s[e] = weight(v[2 * e], tmax, c) + weight(v[2 * e + 1], tmax, c);
      float t = s[0];
#pragma unroll
      for (int e = 1; e < EPC / 2; ++e) t += s[e];
      acc[j & 1] += (double)t;
      sched_fence();
    }
    zt = acc[0] + acc[1];
  }
  // wave level
  const float wm = wave_max(tmax);
  const float ws = wave_min(smin);
  const int wb = __any(nan.nan()) ? 1 : 0;
  double wz = 0.0;
  if (need_z)   // relative to the wave max
    wz = wave_sum(tmax > kNegInf && tmax < kPosInf ? zt * (double)weight(tmax, wm, c) : 0.0);
  const int wid = threadIdx.x / kWave;
  __syncthreads();
  if (__lane_id() == 0) L.ws[wid] = WaveStats{wm, ws, wz, wb};
  __syncthreads();
  RowStats st;
  float M = kNegInf, sm = kPosInf;
  int bad = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    M = fmaxf(M, L.ws[w].m);
    sm = fminf(sm, L.ws[w].smin);
    bad |= L.ws[w].bad;
  }
  double Z = -1.0;
  if (need_z) {
    Z = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (L.ws[w].m > kNegInf && M > kNegInf) Z += L.ws[w].z * (double)weight(L.ws[w].m, M, c);
  }
  st.M = M;
  st.smin = sm;
  st.z = Z;
  st.status = (bad || M == kPosInf) ? 1 : (M > kNegInf ? 0 : 2);
  return st;
}

// Lowest index among the maximal logits.
template <int DT, int NC>
__device__ __forceinline__ int reg_argmax(const RegRow<DT, NC>& r, float M, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  int best = 0x7FFFFFFF;
  if (r.tmax == M) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (r.cm[j] == M) {
        float v[EPC];
        r.elems(j, v);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (v[e] == M) best = min(best, r.base(j) + e);
      }
    }
  }
  return block_min<kBlock>(best, L.bs);
}

// ---------------------------------------------------------------- the walk
// Inverse-CDF draw in ascending token id over per-element weights: the first
// element whose running total exceeds u * (total weight). cw(j, w) fills the
// EPC weights of chunk j (j is a compile-time constant after unrolling).
// Returns the element index; *total_out gets the total weight.
template <int NC, int EPC, class CW>
__device__ __forceinline__ int walk_regs(CW&& cw, double u, Lds& L, double* total_out) {
  static_assert(NC <= kWalkBatch, "walk scratch too small");
  const int tid = threadIdx.x, lane = __lane_id(), wid = tid / kWave;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    float w[EPC];
    cw(j, w);
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) s += (double)w[e];
    if (__any(s > 0.0)) s = wave_sum(s);   // skip the shuffles for empty wave chunks
    if (lane == 0) L.jsum[wid * kWalkBatch + j] = s;
  }
  __syncthreads();
  if (tid < kWave) {
    // lane j < NC totals chunk row j over the waves; a scan over lanes gives
    // the running total in id order
    double sj = 0.0;
    if (lane < NC)
      for (int w = 0; w < kWaves; ++w) sj += L.jsum[w * kWalkBatch + lane];
    const double incl = wave_incl_scan(sj);
    const double tot = readlane_t(incl, 63);
    const double target = u * tot;
    const double excl = incl - sj;
    const unsigned long long hit = __ballot(sj > 0.0 && target < incl);
    const unsigned long long nz = __ballot(sj > 0.0);
    const int last = nz ? 63 - __clzll((long long)nz) : 0;
    const int jstar = hit ? __ffsll((long long)hit) - 1 : last;
    const double r1 = hit ? target - readlane_t(excl, jstar) : kPosInf;
    if (lane == 0) {
      L.si[2] = jstar;
      L.sd[2] = r1;
      L.sd[3] = tot;
    }
  }
  __syncthreads();
  const int jstar = L.si[2];
  const double r1 = L.sd[2];
  *total_out = L.sd[3];
  float wj[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) wj[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
    if (j == jstar) cw(j, wj);
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < EPC; ++e) mine += (double)wj[e];
  double tot2;
  const double ex = block_excl_scan<kBlock>(mine, &tot2, L.bs);
  const bool own = mine > 0.0 && ex <= r1 && r1 < ex + mine;
  int owner = block_min<kBlock>(own ? tid : 0x7FFFFFFF, L.bs);
  bool fallback = false;
  if (owner == 0x7FFFFFFF) {  // rounding put the target past the end: last kept
    owner = block_max<kBlock>(mine > 0.0 ? tid : -1, L.bs);
    fallback = true;
  }
  if (tid == owner) {
    double run = ex;
    int pick = -1, lastpos = -1;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if (wj[e] > 0.0f) {
        run += (double)wj[e];
        lastpos = e;
        if (pick < 0 && !fallback && r1 < run) pick = e;
      }
    }
    if (pick < 0) pick = lastpos;
    L.si[3] = (jstar * kBlock + tid) * EPC + pick;
  }
  __syncthreads();
  const int tok = L.si[3];
  __syncthreads();
  return tok;
}

// Weights of S = {v >= tau}; chunks whose maximum is below tau contribute
// zeros without any exponential.
template <int DT, int NC>
struct KeptWeights {
  const RegRow<DT, NC>& r;
  float tau, M, c;
  __device__ __forceinline__ void operator()(int j, float* w) const {
    constexpr int EPC = Fmt<DT>::EPC;
    if (r.cm[j] >= tau) {
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = v[e] >= tau ? weight(v[e], M, c) : 0.0f;
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = 0.0f;
    }
  }
};

// |S| and the smallest kept value, for S = {v >= tau}.
template <int DT, int NC>
__device__ __forceinline__ void reg_kept_stats(const RegRow<DT, NC>& r, float tau, Lds& L,
                                               int* count, float* vmin) {
  constexpr int EPC = Fmt<DT>::EPC;
  int n = 0;
  float mn = kPosInf;
  if (r.tmax >= tau) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (r.cm[j] >= tau) {
        float v[EPC];
        r.elems(j, v);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (v[e] >= tau) {
            ++n;
            mn = fminf(mn, v[e]);
          }
      }
  }
  *count = block_sum<kBlock>(n, L.bs);
  *vmin = block_min<kBlock>(mn, L.bs);
}

template <int DT, int NC>
__device__ __forceinline__ double reg_kept_mass(const RegRow<DT, NC>& r, float tau, float M,
                                                float c, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < NC; ++j)
    if (r.cm[j] >= tau) {
      float v[EPC];
      r.elems(j, v);
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) t += v[e] >= tau ? weight(v[e], M, c) : 0.0f;
      s += (double)t;
    }
  return block_sum<kBlock>(s, L.bs);
}

// ---------------------------------------------------------------- fast cut
struct FastOut {
  int ok;         // 0: the candidates did not fit; use the general path
  int drawn;      // 1: token already drawn (kept set small enough for one wave)
  int token;
  float tau;
  int kept;
  double zs;      // sum of weights over S
};

// Candidate bound, candidate compaction and exact resolution (see the file
// comment). Z is the row's weight sum (needed for JOINT top-p), u the uniform.
template <int DT, int NC>
__device__ __forceinline__ FastOut fast_cut(const RegRow<DT, NC>& r, int V, float M, float smin,
                                            double Z, float c, const Filters& f, double u,
                                            Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int tid = threadIdx.x;
  FastOut out{0, 0, -1, kPosInf, 0, 0.0};
  // In SEQUENTIAL mode top-p measures against the whole top-k set, so min-p
  // may not narrow the candidates there.
  const bool seq_kp = f.seq && f.k_on && f.p_on;
  float Lb = seq_kp ? kNegInf : f.tau_m;
  if (V <= kCap) {
    Lb = fmaxf(Lb, -kFltMax);           // the whole (finite) row fits
  } else if (f.k_on) {
    const float lo = fmaxf(Lb, smin);
    // sketch values: per-thread maxima when k is small, else chunk maxima
    const bool by_thread = f.k <= kBlock / 4;
    int ns = 0;
    if (by_thread) {
      ns = r.tmax >= lo ? 1 : 0;
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j) ns += (r.cm[j] >= lo) ? 1 : 0;
    }
    ns = block_sum<kBlock>(ns, L.bs);
    if (ns >= f.k) {
      const float span = M - lo;
      const float scale = (span > 0.0f && span <= kFltMax) ? fminf((float)kBins / span, 1e30f)
                                                           : 0.0f;
      auto sbin = [&](float x) -> int {
        const float t = (M - x) * scale;
        return t < (float)(kBins - 1) ? (int)t : kBins - 1;
      };
      for (int i = tid; i < kBins; i += kBlock) L.hcnt[i] = 0u;
      if (tid == 0) {
        L.si[6] = kBins - 1;
        L.su[0] = 0xFFFFFFFFu;
      }
      __syncthreads();
      if (by_thread) {
        if (r.tmax >= lo) atomicAdd(&L.hcnt[sbin(r.tmax)], 1u);
      } else {
#pragma unroll
        for (int j = 0; j < NC; ++j)
          if (r.cm[j] >= lo) atomicAdd(&L.hcnt[sbin(r.cm[j])], 1u);
      }
      __syncthreads();
      if (tid < kWave) {
        constexpr int PER = kBins / kWave;
        int lc = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) lc += (int)L.hcnt[tid * PER + i];
        const int ic = wave_incl_scan(lc);
        int run = ic - lc;
        int found = kBins;
        if (run < f.k && ic >= f.k) {
          for (int i = 0; i < PER; ++i) {
            run += (int)L.hcnt[tid * PER + i];
            if (run >= f.k) { found = tid * PER + i; break; }
          }
        }
        found = wave_min(found);
        if (tid == 0 && found < kBins) L.si[6] = found;
      }
      __syncthreads();
      const int bk = L.si[6];
      if (by_thread) {
        if (r.tmax >= lo && sbin(r.tmax) == bk) atomicMin(&L.su[0], fkey(r.tmax));
      } else {
#pragma unroll
        for (int j = 0; j < NC; ++j)
          if (r.cm[j] >= lo && sbin(r.cm[j]) == bk) atomicMin(&L.su[0], fkey(r.cm[j]));
      }
      __syncthreads();
      const uint32_t kb = L.su[0];
      if (kb != 0xFFFFFFFFu) Lb = fmaxf(Lb, key2f(kb));
    }
  }
  if (!(Lb > kNegInf)) return out;
  // count and compact the candidates (logits >= Lb) into LDS
  int cnt = 0;
  if (r.tmax >= Lb) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (r.cm[j] >= Lb) {
        float v[EPC];
        r.elems(j, v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) cnt += (v[e] >= Lb) ? 1 : 0;
      }
  }
  int total;
  int off = block_excl_scan<kBlock>(cnt, &total, L.bs);
  if (total > kCap) return out;
  if (cnt) {
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (r.cm[j] >= Lb) {
        float v[EPC];
        r.elems(j, v);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (v[e] >= Lb && off < kCap) L.key[off++] = cand_key(v[e], r.base(j) + e);
      }
  }
  __syncthreads();
  const double thr = f.p_on ? f.top_p * Z : 0.0;
  out.ok = 1;
  if (total <= kWaveCap) {
    if (tid < kWave) wave_resolve_draw(L, total, M, c, f, thr, u);
    __syncthreads();
    out.drawn = 1;
    out.token = L.si[0];
    out.kept = L.si[1];
    out.tau = L.sf[0];
    out.zs = L.sd[1];
    __syncthreads();
    return out;
  }
  sort_keys_desc(L, total);
  const Resolved res = resolve_sorted(L, total, 0, 0.0, M, c, f, thr, f.seq);
  out.tau = res.tau;
  out.kept = res.n_in;
  out.zs = res.zs;
  return out;
}

}  // namespace tsr
