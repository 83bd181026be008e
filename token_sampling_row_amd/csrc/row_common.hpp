// Shared pieces of the per-row sampler: LDS layout, constants, the kept-set
// resolution over sorted candidates, histogram boundary search, wave sorts.
//
// The kept set of a row is always S = {v >= tau}: every filter keeps whole
// tie groups of logits (ranking by logit value, which temperature preserves),
// so one threshold describes the intersection of top-k, top-p and min-p.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace tsr {

constexpr int kBlock = 512;   // threads per row (8 wavefronts, 256 VGPRs each)
constexpr int kCap = 2048;    // candidates resolved exactly in LDS
constexpr int kWaveCap = 64;  // candidates resolved by one wavefront without barriers
constexpr int kBins = 1024;   // bins of every histogram level
constexpr int kLogRes = 16;   // log-probability bins per unit of log2(p / p_max)
constexpr int kWalkBatch = 40;  // chunk rows per step of the inverse-CDF walk
constexpr int kWaves = kBlock / kWave;

struct WaveStats {
  float m;       // wave max
  float smin;    // smallest finite chunk maximum in the wave
  double z;      // weight sum relative to m
  int bad;       // NaN or +inf seen
};

struct Lds {
  unsigned long long key[kCap];     // candidate sort keys: fkey(v) << 32 | ~index
  double pref[kCap + 1];            // exclusive prefix of candidate weights
  uint32_t hcnt[kBins];             // histogram counts
  unsigned long long hmass[kBins];  // histogram masses, fixed point 2^-40
  double jsum[kWaves * kWalkBatch]; // walk: per (wave, chunk row) sums
  WaveStats ws[kWaves];
  BlockScratch bs;
  int si[8];
  uint32_t su[8];
  float sf[8];
  double sd[8];
};

// One LDS instance per translation unit; every kernel of the unit uses it, as
// do the non-inlined functions of the streaming path.
static __shared__ Lds tsr_lds;

constexpr double kFix = 1099511627776.0;  // 2^40
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

__device__ __forceinline__ uint32_t key_hi(unsigned long long k) { return (uint32_t)(k >> 32); }
__device__ __forceinline__ unsigned long long cand_key(float v, int index) {
  return ((unsigned long long)fkey(v) << 32) | (unsigned long long)(uint32_t)~(uint32_t)index;
}

// Filters after validation, per row.
struct Filters {
  bool k_on, p_on, m_on, seq;
  int k;
  double top_p;
  float tau_m;    // min-p keeps v >= tau_m (-inf when off)
};

struct Cut {
  float tau;      // S = {v >= tau}
  int kept;       // |S|, or -1 when not counted
  double zs;      // sum over S of weights, or -1 when not summed
};

// Combine two (max, weight sum relative to that max) pairs.
__device__ __forceinline__ void mz_combine(float& m, double& z, float m2, double z2, float c) {
  const float mx = fmaxf(m, m2);
  double r = 0.0;
  if (m > kNegInf) r += z * (double)weight(m, mx, c);
  if (m2 > kNegInf) r += z2 * (double)weight(m2, mx, c);
  m = mx;
  z = r;
}

// ---------------------------------------------------------------- LDS sort
// Bitonic sort of key[0, n) into descending order (n <= kCap).
__device__ __forceinline__ void sort_keys_desc(Lds& L, int n) {
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  for (int i = n + (int)threadIdx.x; i < n2; i += kBlock) L.key[i] = 0ull;
  __syncthreads();
  for (int k2 = 2; k2 <= n2; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += kBlock) {
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
//  min-p: keep iff v >= tau_m.
__device__ __forceinline__ Resolved resolve_sorted(Lds& L, int n, int cnt_above,
                                                   double mass_above, float M, float c,
                                                   const Filters& f, double thr, bool seq_k) {
  constexpr int P = kCap / kBlock;   // consecutive sorted positions per thread
  const int m0 = (int)threadIdx.x * P;
  double w[P];
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    w[i] = m0 + i < n ? (double)weight(key2f(key_hi(L.key[m0 + i])), M, c) : 0.0;
    local += w[i];
  }
  double tot;
  const double ex = block_excl_scan<kBlock>(local, &tot, L.bs);
  double run = ex;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    if (m0 + i < n) L.pref[m0 + i] = run;
    run += w[i];
  }
  if (threadIdx.x == 0) L.pref[n] = tot;
  __syncthreads();

  const uint32_t kM = fkey(M);
  const uint32_t kmin = fkey(f.tau_m);
  int g[P];
#pragma unroll
  for (int i = 0; i < P; ++i) g[i] = m0 + i < n ? group_first(L, m0 + i) : 0;
  double thr_eff = thr;
  if (f.k_on && seq_k) {
    int nk = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) nk += (m0 + i < n && cnt_above + g[i] < f.k) ? 1 : 0;
    nk = block_sum<kBlock>(nk, L.bs);
    thr_eff = f.top_p * (mass_above + L.pref[nk]);
  }
  int nkept = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int m = m0 + i;
    bool keep = m < n && key_hi(L.key[m]) >= kmin;
    if (keep && f.k_on && !(cnt_above + g[i] < f.k)) keep = false;
    if (keep && f.p_on && !(mass_above + L.pref[g[i]] < thr_eff) && key_hi(L.key[m]) != kM)
      keep = false;
    nkept += keep ? 1 : 0;
  }
  const int n_in = block_sum<kBlock>(nkept, L.bs);
  Resolved res;
  res.n_in = n_in;
  res.tau = n_in > 0 ? key2f(key_hi(L.key[n_in - 1])) : kPosInf;
  res.zs = mass_above + L.pref[n_in];
  __syncthreads();
  return res;
}

// Boundary search over one histogram level (every thread calls; wave 0 does
// the work). Bins are in descending value order. Returns the boundary bin
// d* = min(top-k bin, top-p bin), or kBins if no filter cuts inside the
// region; *add_cnt / *add_mass get the totals of the bins before d*.
__device__ __forceinline__ int find_boundary(Lds& L, int cnt_above, double mass_above,
                                             const Filters& f, double thr, bool has_max,
                                             int* add_cnt, double* add_mass) {
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
      if (f.k_on && dk == kBins && cb > 0 && cnt_above + run_c + cb >= f.k) dk = b;
      if (f.p_on && cb > 0 && mass_above + (double)run_m * kInvFix < thr) dp = b;
      run_c += cb;
      run_m += L.hmass[b];
    }
    dk = wave_min(dk);
    dp = wave_max(dp);
    first = wave_min(first);
    if (f.p_on && has_max) dp = max(dp, first);
    int d = kBins;
    if (f.k_on) d = min(d, dk);
    if (f.p_on) d = min(d, dp < 0 ? kBins : dp);
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

// Wave 0 resolves up to kWaveCap unsorted candidates key[0, n) (every logit
// >= the candidate bound, which is <= tau) and draws from S in token-id order.
// Each lane holds one candidate and learns, by reading every other lane
// (v_readlane, no LDS), how many candidates are strictly larger and their
// mass; the draw sums, per kept lane, the kept mass at or below its id.
// Results: L.si[0] token, L.si[1] |S|, L.sf[0] tau, L.sd[1] sum of weights
// over S. Called by wave 0 only; no barriers inside.
__device__ __forceinline__ void wave_resolve_draw(Lds& L, int n, float M, float c,
                                                  const Filters& f, double thr_joint,
                                                  double u) {
  const int lane = __lane_id();
  const bool valid = lane < n;
  const unsigned long long key = valid ? L.key[lane] : 0ull;
  const uint32_t kh = key_hi(key);
  const float v = key2f(kh);
  const uint32_t idx = ~(uint32_t)key;
  const double w = valid ? (double)weight(v, M, c) : 0.0;
  int cnt_gt = 0;
  double mass_gt = 0.0;
  for (int j = 0; j < n; ++j) {
    const uint32_t kj = readlane_u32(kh, j);
    const double wj = readlane_t(w, j);
    if (kj > kh) {
      ++cnt_gt;
      mass_gt += wj;
    }
  }
  const bool keep_k = !f.k_on || cnt_gt < f.k;
  double thr = thr_joint;
  if (f.seq && f.k_on && f.p_on) thr = f.top_p * wave_sum(valid && keep_k ? w : 0.0);
  const bool keep = valid && v >= f.tau_m && keep_k &&
                    (!f.p_on || mass_gt < thr || kh == fkey(M));
  const unsigned long long km = __ballot(keep);
  const int n_in = __popcll(km);
  const float tau = key2f(wave_min_u32(keep ? kh : 0xFFFFFFFFu));
  // draw: running kept mass in ascending token id
  double C = 0.0;
  for (int j = 0; j < n; ++j) {
    if ((km >> j) & 1ull) {
      const uint32_t ij = readlane_u32(idx, j);
      const double wj = readlane_t(w, j);
      if (ij <= idx) C += wj;
    }
  }
  const double total =
      wave_reduce(keep ? C : 0.0, [](double a, double b) { return a > b ? a : b; });
  const double target = u * total;
  const bool hit = keep && C > target;
  const int token = __ballot(hit) ? (int)wave_min_u32(hit ? idx : 0xFFFFFFFFu)
                                  : (int)wave_max_u32(keep ? idx : 0u);
  if (lane == 0) {
    L.si[0] = token;
    L.si[1] = n_in;
    L.sf[0] = tau;
    L.sd[0] = total;
    L.sd[1] = total;
  }
}

}  // namespace tsr
