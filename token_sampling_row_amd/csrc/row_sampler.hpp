// One workgroup resolves one row of logits: row statistics, the kept set S of
// the filter chain, and draws by inverse CDF in token-id order.
//
// The row lives in VGPRs for the whole call: thread t holds 16-byte chunks
// j*BLOCK + t (j < NC), so each wavefront load is 1 KiB contiguous and HBM is
// read exactly once. Every later step runs on registers and LDS.
//
// The kept set is always S = {v >= tau} (tie groups are kept or dropped
// whole). tau is found without sorting the row:
//  * fast path: a lower bound Lb <= tau from min-p (a logit threshold) and from
//    top-k (the k-th largest chunk maximum is at most the k-th largest logit);
//    the few logits >= Lb go to LDS, are sorted there and resolved exactly;
//  * general path (top-p over a wide nucleus, or too many candidates):
//    histograms of (count, mass) by log-probability bin, then by exact key
//    digits inside the boundary bin, until the boundary region fits in LDS.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace tsr {

constexpr int kCap = 2048;    // candidates resolved exactly in LDS
constexpr int kBins = 1024;   // bins of every histogram level
constexpr int kLogRes = 16;   // log-probability bins per unit of log2(p / p_max)
constexpr int kMaxNC = 20;    // chunks per thread the walk scratch is sized for

struct Lds {
  unsigned long long key[kCap];     // candidate sort keys: fkey(v) << 32 | ~index
  double pref[kCap + 1];            // exclusive prefix of candidate weights
  uint32_t hcnt[kBins];             // histogram counts
  unsigned long long hmass[kBins];  // histogram masses, fixed point 2^-40
  double jsum[16 * kMaxNC];         // walk: per (wave, chunk row) sums
  BlockScratch bs;
  int si[8];
  uint32_t su[8];
  double sd[8];
};

constexpr double kFix = 1099511627776.0;      // 2^40
constexpr double kInvFix = 1.0 / 1099511627776.0;

__device__ __forceinline__ unsigned long long to_fixed(float w) {
  return (unsigned long long)((double)w * kFix + 0.5);
}

__device__ __forceinline__ float next_up(float f) {
  if (!(f < kPosInf)) return f;
  if (f == 0.0f) return __uint_as_float(1u);
  const uint32_t b = __float_as_uint(f);
  return __uint_as_float(f > 0.0f ? b + 1u : b - 1u);
}
// Smallest float >= th.
__device__ __forceinline__ float ceil_to_float(double th) {
  float f = (float)th;
  if ((double)f < th) f = next_up(f);
  return f;
}

// Row data resident in VGPRs.
template <int DT, int NC, int BLOCK>
struct Row {
  static constexpr int EPC = Fmt<DT>::EPC;
  uint4 raw[NC];
  float cm[NC];   // chunk maxima; -inf past the end of the row
  float tmax;     // this thread's maximum

  // Whole chunks of a 16-byte aligned row are plain 128-bit loads, all issued
  // back to back; chunks past the end read a -inf chunk. `ragged` rows (vocab
  // not a multiple of the chunk, or an unaligned row) patch the partial chunk
  // from element loads, or load everything element-wise when unaligned.
  __device__ __forceinline__ void load(const unsigned char* p, int V, bool aligned,
                                       bool ragged) {
    constexpr int ESZ = Fmt<DT>::ESZ;
    if (!ragged || aligned) {
      const uint4* neg = &g_neg_inf_chunk[DT];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const long long c = (long long)j * BLOCK + threadIdx.x;
        const bool whole = (c + 1) * EPC <= V;
        raw[j] = *(whole ? reinterpret_cast<const uint4*>(p + c * EPC * ESZ) : neg);
      }
      if (ragged) {
        const long long cl = V / EPC;  // the partial chunk, if V % EPC != 0
        if (cl * EPC < V && (int)(cl % BLOCK) == (int)threadIdx.x) {
          const uint4 patch = load_chunk_slow<DT>(p, cl, V);
          const int jl = (int)(cl / BLOCK);
#pragma unroll
          for (int j = 0; j < NC; ++j)
            if (j == jl) raw[j] = patch;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NC; ++j)
        raw[j] = load_chunk_slow<DT>(p, (long long)j * BLOCK + threadIdx.x, V);
    }
  }
  __device__ __forceinline__ int base(int j) const {
    return (j * BLOCK + (int)threadIdx.x) * EPC;
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

struct RowStats {
  int status;     // TSR_ROW_*
  float M;        // row max
  float smin;     // smallest finite chunk maximum
  double z;       // sum of weights over the row (only if asked for)
};

// Pass over the registers: chunk maxima, max, NaN/+inf flag, and (optionally)
// the weight sum with a running per-thread reference max, rescaled on the fly.
// NaN detector on packed data: the running maximum of the magnitude bits of
// every element. A NaN has magnitude bits above those of infinity.
template <int DT> struct NanAcc;
template <> struct NanAcc<0> {
  uint32_t a = 0u;
  __device__ __forceinline__ void add(uint4 t) {
    a = max(a, max(max(t.x & 0x7FFFFFFFu, t.y & 0x7FFFFFFFu), max(t.z & 0x7FFFFFFFu, t.w & 0x7FFFFFFFu)));
  }
  __device__ __forceinline__ bool nan() const { return a > 0x7F800000u; }
};
template <> struct NanAcc<1> {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  us2 a = {0, 0};
  __device__ __forceinline__ static us2 mag(uint32_t w) {
    const uint32_t m = w & 0x7FFF7FFFu;
    return __builtin_bit_cast(us2, m);
  }
  __device__ __forceinline__ void add(uint4 t) {
    a = __builtin_elementwise_max(a, __builtin_elementwise_max(
            __builtin_elementwise_max(mag(t.x), mag(t.y)),
            __builtin_elementwise_max(mag(t.z), mag(t.w))));
  }
  __device__ __forceinline__ bool nan() const { return a.x > 0x7F80u || a.y > 0x7F80u; }
};

// Pass over the registers: chunk maxima, max, NaN/+inf flag, and (optionally)
// the weight sum with a running per-thread reference max, rescaled on the fly.
template <int DT, int NC, int BLOCK>
__device__ __forceinline__ RowStats row_stats(Row<DT, NC, BLOCK>& r, bool need_z, float c,
                                              Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  float tmax = kNegInf, smin = kPosInf, mt = kNegInf;
  double zt = 0.0;
  NanAcc<DT> nan;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const uint4 t = r.packed(j);
    nan.add(t);
    float v[EPC];
    unpack<DT>(t, v);
    float m = v[0];
#pragma unroll
    for (int e = 1; e < EPC; ++e) m = fmaxf(m, v[e]);
    r.cm[j] = m;
    tmax = fmaxf(tmax, m);
    if (m > kNegInf) smin = fminf(smin, m);
    if (need_z && m > kNegInf) {
      if (m > mt) {
        zt = (mt > kNegInf) ? zt * (double)weight(mt, m, c) : 0.0;
        mt = m;
      }
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) s += weight(v[e], mt, c);
      zt += (double)s;
    }
  }
  r.tmax = tmax;
  RowStats st;
  st.M = block_max<BLOCK>(tmax, L.bs);
  const int anybad = block_max<BLOCK>(nan.nan() ? 1 : 0, L.bs);
  st.smin = block_min<BLOCK>(smin, L.bs);
  st.z = -1.0;
  if (need_z) {
    const double mine =
        (mt > kNegInf && st.M > kNegInf) ? zt * (double)weight(mt, st.M, c) : 0.0;
    st.z = block_sum<BLOCK>(mine, L.bs);
  }
  st.status = (anybad || st.M == kPosInf) ? 1 : (st.M > kNegInf ? 0 : 2);
  return st;
}

// Lowest index among the maximal logits.
template <int DT, int NC, int BLOCK>
__device__ __forceinline__ int row_argmax(const Row<DT, NC, BLOCK>& r, float M, Lds& L) {
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
  return block_min<BLOCK>(best, L.bs);
}

// ---------------------------------------------------------------- LDS sort
// Bitonic sort of key[0, n) into descending order (n <= kCap).
template <int BLOCK>
__device__ __forceinline__ void sort_keys_desc(Lds& L, int n) {
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  for (int i = n + (int)threadIdx.x; i < n2; i += BLOCK) L.key[i] = 0ull;
  __syncthreads();
  for (int k2 = 2; k2 <= n2; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += BLOCK) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = L.key[i], b = L.key[ixj];
          const bool desc = (i & k2) == 0;
          if (desc ? (a < b) : (a > b)) {
            L.key[i] = b;
            L.key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ uint32_t key_hi(unsigned long long k) { return (uint32_t)(k >> 32); }

// First sorted position holding the same value as position m.
__device__ __forceinline__ int group_first(const Lds& L, int m) {
  const uint32_t k = key_hi(L.key[m]);
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (key_hi(L.key[mid]) > k) lo = mid + 1; else hi = mid;
  }
  return lo;
}

struct Resolved {
  float tau;      // smallest kept value (valid iff n_in > 0)
  int n_in;       // kept candidates
  double zs;      // mass_above + kept candidate mass
};

// Exact resolution over the candidates key[0, n) (sorted descending), which
// hold every logit of the boundary region; cnt_above / mass_above count the
// logits above the region (all kept by construction).
//  top-k: keep a group iff cnt_above + (candidates strictly above) < k.
//  top-p: keep iff mass_above + (candidate mass strictly above) < thr, or the
//         group is the row max. With seq_k, thr = top_p * (mass kept by top-k).
template <int BLOCK>
__device__ __forceinline__ Resolved resolve_sorted(Lds& L, int n, int cnt_above, double mass_above, float M,
                                   float c, bool k_on, int k, bool p_on, double thr,
                                   bool seq_k, double top_p, float tau_m) {
  static_assert(2 * BLOCK >= kCap, "two candidates per thread must cover the LDS");
  // weights and their exclusive prefix in sorted order (two positions per thread)
  const int p0 = 2 * (int)threadIdx.x, p1 = p0 + 1;
  const double w0 = p0 < n ? (double)weight(key2f(key_hi(L.key[p0])), M, c) : 0.0;
  const double w1 = p1 < n ? (double)weight(key2f(key_hi(L.key[p1])), M, c) : 0.0;
  double tot;
  const double ex = block_excl_scan<BLOCK>(w0 + w1, &tot, L.bs);
  if (p0 < n) L.pref[p0] = ex;
  if (p1 < n) L.pref[p1] = ex + w0;
  if (threadIdx.x == 0) L.pref[n] = tot;
  __syncthreads();

  const uint32_t kM = fkey(M);
  int f0 = 0, f1 = 0;
  if (p0 < n) f0 = group_first(L, p0);
  if (p1 < n) f1 = group_first(L, p1);
  double thr_eff = thr;
  if (k_on && seq_k) {
    const int nk = block_sum<BLOCK>((p0 < n && cnt_above + f0 < k ? 1 : 0) +
                                    (p1 < n && cnt_above + f1 < k ? 1 : 0), L.bs);
    thr_eff = top_p * (mass_above + L.pref[nk]);
  }
  const uint32_t kmin = fkey(tau_m);
  auto kept = [&](int m, int f) -> int {
    if (m >= n) return 0;
    if (key_hi(L.key[m]) < kmin) return 0;
    if (k_on && !(cnt_above + f < k)) return 0;
    if (p_on && !(mass_above + L.pref[f] < thr_eff) && key_hi(L.key[m]) != kM) return 0;
    return 1;
  };
  const int n_in = block_sum<BLOCK>(kept(p0, f0) + kept(p1, f1), L.bs);
  Resolved res;
  res.n_in = n_in;
  res.tau = n_in > 0 ? key2f(key_hi(L.key[n_in - 1])) : kPosInf;
  res.zs = mass_above + L.pref[n_in];
  __syncthreads();
  return res;
}

// Boundary search over one histogram level (run by every thread; wave 0 does
// the work). Bins are in descending value order. Returns the boundary bin d*
// = min(top-k bin, top-p bin) or kBins if no filter cuts inside this region;
// *add_cnt / *add_mass get the totals of the bins before d*.
__device__ __forceinline__ int find_boundary(Lds& L, int cnt_above, double mass_above, bool k_on, int k,
                             bool p_on, double thr, bool has_max, int* add_cnt,
                             double* add_mass) {
  constexpr int PER = kBins / kWave;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int lc = 0;
    unsigned long long lm = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      lc += (int)L.hcnt[lane * PER + i];
      lm += L.hmass[lane * PER + i];
    }
    const int ic = wave_incl_scan(lc);
    const unsigned long long im = wave_incl_scan(lm);
    int run_c = ic - lc;
    unsigned long long run_m = im - lm;
    int dk = kBins, dp = -1, first = kBins;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = lane * PER + i;
      const int cb = (int)L.hcnt[b];
      if (cb > 0 && first == kBins) first = b;
      if (k_on && dk == kBins && cb > 0 && cnt_above + run_c + cb >= k) dk = b;
      if (p_on && cb > 0 && mass_above + (double)run_m * kInvFix < thr) dp = b;
      run_c += cb;
      run_m += L.hmass[b];
    }
    dk = wave_min(dk);
    dp = wave_max(dp);
    first = wave_min(first);
    if (p_on && has_max) dp = max(dp, first);
    int d = kBins;
    if (k_on) d = min(d, dk);
    if (p_on) d = min(d, dp < 0 ? kBins : dp);
    // totals of the bins before d
    int bc = 0;
    unsigned long long bm = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = lane * PER + i;
      if (b < d) {
        bc += (int)L.hcnt[b];
        bm += L.hmass[b];
      }
    }
    bc = wave_sum(bc);
    bm = wave_sum(bm);
    if (lane == 0) {
      L.si[4] = d;
      L.si[5] = bc;
      L.sd[4] = (double)bm * kInvFix;
    }
  }
  __syncthreads();
  const int d = L.si[4];
  *add_cnt = L.si[5];
  *add_mass = L.sd[4];
  __syncthreads();
  return d;
}

struct Cut {
  int status;
  float M;
  float tau;      // S = {v >= tau}
  int kept;       // |S|, or -1 if not counted yet
  double zs;      // sum of weights over S
  double z;       // sum of weights over the row, or -1
};

// The general path: log-probability bins, then exact key digits, then LDS.
template <int DT, int NC, int BLOCK>
__device__ __forceinline__ void general_cut(const Row<DT, NC, BLOCK>& r, float M, float c, float cR,
                            float tau_m, bool k_on, int k, bool p_on, double thr, Lds& L,
                            float* tau_out, int* kept_out, double* zs_out) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int tid = threadIdx.x;
  // level 1: bins of log2(p / p_max) over finite logits >= tau_m
  for (int i = tid; i < kBins; i += BLOCK) {
    L.hcnt[i] = 0u;
    L.hmass[i] = 0ull;
  }
  __syncthreads();
  auto lbin = [&](float v) -> int {
    const float t = (M - v) * cR;
    return t < (float)(kBins - 1) ? (int)t : kBins - 1;
  };
  if (r.tmax >= tau_m) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (r.cm[j] >= tau_m && r.cm[j] > kNegInf) {
        float v[EPC];
        r.elems(j, v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          if (v[e] >= tau_m && v[e] > kNegInf) {
            const int b = lbin(v[e]);
            atomicAdd(&L.hcnt[b], 1u);
            atomicAdd(&L.hmass[b], to_fixed(weight(v[e], M, c)));
          }
        }
      }
    }
  }
  __syncthreads();
  int cnt_above = 0, add_c = 0;
  double mass_above = 0.0, add_m = 0.0;
  int d = find_boundary(L, 0, 0.0, k_on, k, p_on, thr, true, &add_c, &add_m);
  if (d == kBins) {
    // no cut inside: S = every finite logit >= tau_m
    *tau_out = tau_m > kNegInf ? tau_m : -kFltMax;
    *kept_out = -1;
    *zs_out = -1.0;
    return;
  }
  cnt_above = add_c;
  mass_above = add_m;
  int ncur = (int)L.hcnt[d];
  __syncthreads();
  // region: level-1 bin d, then key ranges [klo, khi] within it
  bool by_key = false;
  uint32_t klo = 0u, khi = 0xFFFFFFFFu;
  auto in_region = [&](float v) -> bool {
    if (!(v >= tau_m) || !(v > kNegInf)) return false;
    if (by_key) {
      const uint32_t kk = fkey(v);
      return kk >= klo && kk <= khi;
    }
    return lbin(v) == d;
  };
  bool contains_max = (d == 0);
  for (int level = 0; level < 4 && ncur > kCap; ++level) {
    // key range of the region
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (in_region(v[e])) {
          const uint32_t kk = fkey(v[e]);
          mn = min(mn, kk);
          mx = max(mx, kk);
        }
    }
    mn = block_min_u32<BLOCK>(mn, L.bs);
    mx = block_max_u32<BLOCK>(mx, L.bs);
    by_key = true;
    klo = mn;
    khi = mx;
    if (mn == mx) break;  // a single tie group: resolved below as one candidate group
    const uint32_t span = mx - mn;
    const int bits = 32 - __clz(span);
    const int shift = bits > 10 ? bits - 10 : 0;
    for (int i = tid; i < kBins; i += BLOCK) {
      L.hcnt[i] = 0u;
      L.hmass[i] = 0ull;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (in_region(v[e])) {
          const int b = (kBins - 1) - (int)((fkey(v[e]) - klo) >> shift);
          atomicAdd(&L.hcnt[b], 1u);
          atomicAdd(&L.hmass[b], to_fixed(weight(v[e], M, c)));
        }
    }
    __syncthreads();
    const bool has_max = contains_max && (khi == fkey(M));
    const int d2 = find_boundary(L, cnt_above, mass_above, k_on, k, p_on, thr, has_max,
                                 &add_c, &add_m);
    // the region was chosen to hold the cut, so some bin must cut here
    const int dd = d2 == kBins ? kBins - 1 : d2;
    ncur = (int)L.hcnt[dd];
    cnt_above += add_c;
    mass_above += add_m;
    const uint32_t lo2 = klo + ((uint32_t)((kBins - 1) - dd) << shift);
    const uint32_t hi2 = min(khi, lo2 + ((shift >= 32) ? 0xFFFFFFFFu : ((1u << shift) - 1u)));
    contains_max = has_max && hi2 == khi;
    klo = lo2;
    khi = hi2;
    __syncthreads();
  }
  if (by_key && klo == khi && ncur > kCap) {
    // one tie group larger than the LDS: decide it as a whole
    const float v = key2f(klo);
    const double w = (double)weight(v, M, c);
    bool keep = true;
    if (k_on && !(cnt_above < k)) keep = false;
    if (p_on && !(mass_above < thr) && fkey(v) != fkey(M)) keep = false;
    *tau_out = keep ? v : next_up(v);
    *kept_out = cnt_above + (keep ? ncur : 0);
    *zs_out = mass_above + (keep ? (double)ncur * w : 0.0);
    return;
  }
  // compact the region into LDS
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    float v[EPC];
    r.elems(j, v);
#pragma unroll
    for (int e = 0; e < EPC; ++e) cnt += in_region(v[e]) ? 1 : 0;
  }
  int total;
  int off = block_excl_scan<BLOCK>(cnt, &total, L.bs);
  if (cnt) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (in_region(v[e]) && off < kCap)
          L.key[off++] = ((unsigned long long)fkey(v[e]) << 32) |
                         (unsigned long long)(uint32_t)~(uint32_t)(r.base(j) + e);
    }
  }
  __syncthreads();
  total = min(total, kCap);
  sort_keys_desc<BLOCK>(L, total);
  const Resolved res = resolve_sorted<BLOCK>(L, total, cnt_above, mass_above, M, c, k_on, k,
                                             p_on, thr, false, 0.0, tau_m);
  if (res.n_in > 0) {
    *tau_out = res.tau;
    *kept_out = cnt_above + res.n_in;
    *zs_out = res.zs;
  } else {
    // nothing of the region stays: S is exactly what lies above it
    *tau_out = key2f(khi) < kPosInf && by_key ? next_up(key2f(khi)) : tau_m;
    *kept_out = cnt_above;
    *zs_out = mass_above;
  }
}

// The kept set of one row for temperature > 0.
template <int DT, int NC, int BLOCK>
__device__ __forceinline__ Cut row_cut(Row<DT, NC, BLOCK>& r, const KParams& kp, int V, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  const bool k_on = (kp.flags & F_K) != 0;
  const bool p_on = (kp.flags & F_P) != 0;
  const bool m_on = (kp.flags & F_M) != 0;
  const bool seq = (kp.flags & F_SEQ) != 0;
  const int k = kp.top_k;
  const bool need_z = (kp.flags & F_Z) || (p_on && !(seq && k_on));
  const RowStats st = row_stats(r, need_z, kp.c, L);
  Cut cut;
  cut.status = st.status;
  cut.M = st.M;
  cut.z = st.z;
  cut.tau = kPosInf;
  cut.kept = 0;
  cut.zs = 0.0;
  if (st.status != 0) return cut;
  const float M = st.M;
  const float c = kp.c;
  const int tid = threadIdx.x;
  const float tau_m = m_on ? ceil_to_float((double)M + kp.minp_off) : kNegInf;

  // ---- fast path: a lower bound Lb <= tau with few logits above it. In
  // SEQUENTIAL mode top-p measures against the whole top-k set, so min-p may
  // not narrow the candidates there.
  const bool seq_kp = seq && k_on && p_on;
  float Lb = seq_kp ? kNegInf : tau_m;
  if (k_on) {
    const float lo = fmaxf(Lb, st.smin);
    int ns = 0;
#pragma unroll
    for (int j = 0; j < NC; ++j) ns += (r.cm[j] >= lo) ? 1 : 0;
    ns = block_sum<BLOCK>(ns, L.bs);
    if (ns >= k) {
      const float span = M - lo;
      const float scale = (span > 0.0f && span <= kFltMax) ? fminf((float)kBins / span, 1e30f)
                                                           : 0.0f;
      auto sbin = [&](float x) -> int {
        const float t = (M - x) * scale;
        return t < (float)(kBins - 1) ? (int)t : kBins - 1;
      };
      for (int i = tid; i < kBins; i += BLOCK) L.hcnt[i] = 0u;
      if (tid == 0) {
        L.si[0] = kBins - 1;
        L.su[0] = 0xFFFFFFFFu;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NC; ++j)
        if (r.cm[j] >= lo) atomicAdd(&L.hcnt[sbin(r.cm[j])], 1u);
      __syncthreads();
      if (tid < kWave) {
        constexpr int PER = kBins / kWave;
        int lc = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) lc += (int)L.hcnt[tid * PER + i];
        const int ic = wave_incl_scan(lc);
        int run = ic - lc;
        int found = kBins;
        if (run < k && ic >= k) {
          for (int i = 0; i < PER; ++i) {
            run += (int)L.hcnt[tid * PER + i];
            if (run >= k) { found = tid * PER + i; break; }
          }
        }
        found = wave_min(found);
        if (tid == 0 && found < kBins) L.si[0] = found;
      }
      __syncthreads();
      const int bk = L.si[0];
#pragma unroll
      for (int j = 0; j < NC; ++j)
        if (r.cm[j] >= lo && sbin(r.cm[j]) == bk) atomicMin(&L.su[0], fkey(r.cm[j]));
      __syncthreads();
      Lb = fmaxf(Lb, key2f(L.su[0]));
      __syncthreads();
    }
  }
  bool fast = Lb > kNegInf;
  int total = 0;
  if (fast) {
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
    int off = block_excl_scan<BLOCK>(cnt, &total, L.bs);
    if (total <= kCap) {
      if (cnt) {
#pragma unroll
        for (int j = 0; j < NC; ++j)
          if (r.cm[j] >= Lb) {
            float v[EPC];
            r.elems(j, v);
#pragma unroll
            for (int e = 0; e < EPC; ++e)
              if (v[e] >= Lb)
                if (off < kCap)
                  L.key[off++] = ((unsigned long long)fkey(v[e]) << 32) |
                                 (unsigned long long)(uint32_t)~(uint32_t)(r.base(j) + e);
          }
      }
      __syncthreads();
    } else {
      fast = false;
    }
  }
  if (fast) {
    sort_keys_desc<BLOCK>(L, total);
    const double thr = p_on ? kp.top_p * st.z : 0.0;
    const Resolved res = resolve_sorted<BLOCK>(L, total, 0, 0.0, M, c, k_on, k, p_on, thr,
                                               seq, kp.top_p, tau_m);
    cut.tau = res.tau;
    cut.kept = res.n_in;
    cut.zs = res.zs;
    return cut;
  }

  // ---- general path
  if (!k_on && !p_on) {
    cut.tau = m_on ? tau_m : -kFltMax;
    cut.kept = -1;
    cut.zs = -1.0;
    return cut;
  }
  double Z = st.z;
  if (Z < 0.0) {
    double zt = 0.0;
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (r.cm[j] > kNegInf) {
        float v[EPC];
        r.elems(j, v);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s += weight(v[e], M, c);
        zt += (double)s;
      }
    Z = block_sum<BLOCK>(zt, L.bs);
    cut.z = Z;
  }
  float tau;
  int kept;
  double zs;
  if (seq && k_on && p_on) {
    // SEQUENTIAL: top-k alone first (its kept mass is top-p's reference)
    float tk;
    int kk;
    double zk;
    general_cut(r, M, c, kp.cR, kNegInf, true, k, false, 0.0, L, &tk, &kk, &zk);
    if (zk < 0.0) zk = Z;
    general_cut(r, M, c, kp.cR, tau_m, true, k, true, kp.top_p * zk, L, &tau, &kept, &zs);
  } else {
    general_cut(r, M, c, kp.cR, tau_m, k_on, k, p_on, kp.top_p * Z, L, &tau, &kept, &zs);
  }
  cut.tau = tau;
  cut.kept = kept;
  cut.zs = zs;
  return cut;
}

// ---------------------------------------------------------------- the walk
// Inverse-CDF draw in ascending token id over per-element weights:
// the first element whose running total exceeds u * (total weight).
// cw(j, w) fills the EPC weights of chunk j (j is a compile-time constant
// after unrolling). Returns the element index; *total_out gets the total.
template <int NC, int EPC, int BLOCK, class CW>
__device__ __forceinline__ int walk_draw(CW&& cw, double u, Lds& L, double* total_out) {
  static_assert(NC <= kMaxNC, "walk scratch too small");
  constexpr int W = BLOCK / kWave;
  const int tid = threadIdx.x, lane = __lane_id(), wid = tid / kWave;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    float w[EPC];
    cw(j, w);
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) s += (double)w[e];
    s = wave_sum(s);
    if (lane == 0) L.jsum[wid * NC + j] = s;
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    double sj[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      double s = 0.0;
      for (int w = 0; w < W; ++w) s += L.jsum[w * NC + j];
      sj[j] = s;
      tot += s;
    }
    const double target = u * tot;
    int jstar = -1;
    double r1 = 0.0, run = 0.0;
    int jlast = 0;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (sj[j] > 0.0) {
        if (jstar < 0 && target < run + sj[j]) {
          jstar = j;
          r1 = target - run;
        }
        jlast = j;
      }
      run += sj[j];
    }
    if (jstar < 0) {  // rounding put the target past the end: take the last kept
      jstar = jlast;
      r1 = kPosInf;
    }
    L.si[0] = jstar;
    L.sd[0] = r1;
    L.sd[1] = tot;
  }
  __syncthreads();
  const int jstar = L.si[0];
  const double r1 = L.sd[0];
  *total_out = L.sd[1];
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
  const double ex = block_excl_scan<BLOCK>(mine, &tot2, L.bs);
  const bool own = mine > 0.0 && ex <= r1 && r1 < ex + mine;
  int owner = block_min<BLOCK>(own ? tid : 0x7FFFFFFF, L.bs);
  bool fallback = false;
  if (owner == 0x7FFFFFFF) {
    owner = block_max<BLOCK>(mine > 0.0 ? tid : -1, L.bs);
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
    L.si[1] = (jstar * BLOCK + tid) * EPC + pick;
  }
  __syncthreads();
  const int tok = L.si[1];
  __syncthreads();
  return tok;
}

}  // namespace tsr
