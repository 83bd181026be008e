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
constexpr int kWalkLds = 16;    // up to this many chunk rows per thread the walk's per-thread sums share the LDS union
constexpr int kWaves = kBlock / kWave;
constexpr int kVRes = 32;        // bf16 value histogram: bins per logit below the max
constexpr int kVBins = 1024;     //   bins (32 logits)
constexpr int kVCopies = 4;      //   count copies (lane & 3): fewer lanes per address
constexpr int kVStride = kVBins + 1;   // copies one bank apart

struct WaveStats {
  float m;       // wave max
  float smin;    // smallest finite chunk maximum in the wave
  double z;      // weight sum relative to m
  int bad;       // NaN or +inf seen
  int na;        // allowed elements (masked rows)
};

struct Lds {
  union {
    struct {
      unsigned long long key[kCap];   // candidate sort keys: fkey(v) << 32 | ~index
      double pref[kCap + 1];          // exclusive prefix of candidate weights
    };
    uint32_t vcnt[kVCopies * kVStride];   // bf16 value histogram: per-copy counts
    unsigned long long own[kBlock];       // per thread: window entries in its chunks (after pass A)
    double jrow[kWalkBatch][kWaves * 4];  // walk: per (chunk row, 16-lane row) sums
    float wsum[kWalkLds][kBlock];         // walk: per (chunk row, thread) sums (wider rows: walk_sums)
  };
  uint32_t hcnt[kBins];             // histogram counts
  unsigned long long hmass[kBins];  // histogram masses, fixed point 2^-40
  double jsum[kWaves * kWalkBatch]; // walk: per (wave, chunk row) sums
  struct WaveCands {                // candidates found by one wavefront
    uint32_t val[kWaveCap];         // value bits (float32)
    uint32_t idx[kWaveCap];         // token ids
  } wc[kWaves];
  int wcnt[kWaves];                 // candidates found by each wavefront
  int hist[kHistMax];               // the look-back window (-1: not a token of the row)
  float hval[kHistMax];             // its penalised logits (register path)
  double tz[32];                    // tree verify: 1 / Z of each residual step
  uint32_t hbits[kWave];            // chunks holding a window token, hashed (chunk mod 2048)
  WaveStats ws[kWaves];
  BlockScratch bs;
  int si[8];
  uint32_t su[8];
  float sf[8];
  double sd[8];
#if TSR_TRACE
  TraceLds trace;                   // the phase stamps (tracing build)
#endif
};

// Histogram bin b lives at slot (b % 16) * 64 + b / 16: the 16 consecutive
// bins one lane scans are 64 words apart, so the reads of a wavefront at one
// step fall in distinct banks (bins b and b + 1 side by side would put a whole
// wavefront on two banks).
static_assert(kBins == 1024, "hslot assumes 1024 bins");
__device__ __forceinline__ int hslot(int b) { return ((b & 15) << 6) | (b >> 4); }

// Allowed-token mask of one 16-byte chunk c: its EPC bits (token i is bit
// i % 32 of word i / 32), from a word array (global or LDS).
template <int DT>
__device__ __forceinline__ uint32_t chunk_mask_bits(const uint32_t* words, long long c) {
  if constexpr (DT == 0) return (words[c >> 3] >> ((uint32_t)(c & 7) * 4u)) & 0xFu;
  else return (words[c >> 2] >> ((uint32_t)(c & 3) * 8u)) & 0xFFu;
}
// A chunk with its disallowed elements replaced by -inf (constrained decoding:
// the mask applies before any other step).
template <int DT>
__device__ __forceinline__ uint4 apply_mask(uint4 t, uint32_t bits) {
  uint32_t x[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t keep;
    uint32_t ninf;
    if constexpr (DT == 0) {
      keep = 0u - ((bits >> i) & 1u);
      ninf = 0xFF800000u;
    } else {
      keep = ((0u - ((bits >> (2 * i)) & 1u)) & 0x0000FFFFu) |
             ((0u - ((bits >> (2 * i + 1)) & 1u)) & 0xFFFF0000u);
      ninf = 0xFF80FF80u;
    }
    x[i] = (x[i] & keep) | (ninf & ~keep);
  }
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Repetition penalty of one logit (the CTRL rule): z / r above zero, z * r
// otherwise, in double, rounded to the row's element type (bf16: nearest
// even from the float32).
template <int DT>
__device__ __forceinline__ float penalize(float z, double r) {
  float f = (float)(z > 0.0f ? (double)z / r : (double)z * r);
  if constexpr (DT == 1) {
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7F800000u) != 0x7F800000u)
      f = __uint_as_float((b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u);
  }
  return f;
}
// Element i of a row (exact float value).
template <int DT>
__device__ __forceinline__ float load_elem(const unsigned char* p, int i) {
  if constexpr (DT == 0)
    return reinterpret_cast<const float*>(p)[i];
  else
    return __uint_as_float((uint32_t)reinterpret_cast<const unsigned short*>(p)[i] << 16);
}
// A chunk with element e replaced by the value v, unless that element is
// -inf (a masked-out token: it stays out; an allowed -inf penalises to -inf).
template <int DT>
__device__ __forceinline__ uint4 replace_elem(uint4 t, int e, float v) {
  constexpr int EPC = Fmt<DT>::EPC;
  float w[EPC];
  unpack<DT>(t, w);
#pragma unroll
  for (int q = 0; q < EPC; ++q)
    if (q == e && w[q] != kNegInf) w[q] = v;
  uint32_t x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == 0)
      x[i] = __float_as_uint(w[i]);
    else
      x[i] = (__float_as_uint(w[2 * i]) >> 16) | (__float_as_uint(w[2 * i + 1]) & 0xFFFF0000u);
  }
  return make_uint4(x[0], x[1], x[2], x[3]);
}
// A chunk with the elements flagged in `hit` (bit e: element e) penalised.
template <int DT>
__device__ __forceinline__ uint4 penalize_chunk(uint4 t, uint32_t hit, double r) {
  constexpr int EPC = Fmt<DT>::EPC;
  float v[EPC];
  unpack<DT>(t, v);
#pragma unroll
  for (int e = 0; e < EPC; ++e)
    if ((hit >> e) & 1u) v[e] = penalize<DT>(v[e], r);
  uint32_t x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == 0)
      x[i] = __float_as_uint(v[i]);
    else
      x[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
  }
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// One LDS instance per translation unit; every kernel of the unit uses it, as
// do the non-inlined functions of the streaming path.
static __shared__ Lds tsr_lds;

// Phase stamps (tracing build; empty statements otherwise): a kernel that
// stamps begins the record at entry (null buffer: none kept) and flushes it
// when its row is done.
#if TSR_TRACE
#define TSR_STAMP(slot) ::tsr::trace_stamp(::tsr::tsr_lds.trace, (slot))
#define TSR_TRACE_INIT(ptr) ::tsr::trace_begin(::tsr::tsr_lds.trace, (ptr))
#define TSR_TRACE_FLUSH() ::tsr::trace_flush(::tsr::tsr_lds.trace)
#else
#define TSR_STAMP(slot) ((void)0)
#define TSR_TRACE_INIT(ptr) ((void)0)
#define TSR_TRACE_FLUSH() ((void)0)
#endif

// The look-back window of the repetition penalty, published by wave 0 (all
// lanes, lane h holding id hv of the window's first n): L.hist[h] = the id if
// it is a token of the row, else -1; L.own[t] gets bit h when thread t's
// chunks hold it (chunk id / EPC mod kBlock); L.hbits flags its chunk, hashed
// to 2048 bits, for the streaming reads. Repeated ids stay in the list (their
// users apply each distinct id once). A barrier must follow.
template <int DT>
__device__ __forceinline__ void hist_publish(int hv, int n, int V, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int lane = __lane_id();
  const bool in = lane < n && hv >= 0 && hv < V;
#pragma unroll
  for (int k = 0; k < kBlock / kWave; ++k) L.own[k * kWave + lane] = 0ull;
  L.hbits[lane] = 0u;
  if (lane < n) L.hist[lane] = in ? hv : -1;
  if (in) {   // (a wavefront's LDS operations complete in order: after the clears)
    const int c = hv / EPC;
    atomicOr(&L.own[c % kBlock], 1ull << lane);
    atomicOr(&L.hbits[(c >> 5) & (kWave - 1)], 1u << (c & 31));
  }
}


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

// Inverse-CDF draw over the kept candidates key[0, n) (the first n_in of the
// value-sorted candidates): re-keyed by token id, sorted ascending by id, an
// exclusive scan of their weights, and the first id whose running total
// exceeds u * Z_S (else the last id with weight). Every thread calls.
__device__ __forceinline__ int draw_sorted(Lds& L, int n, float M, float c, double u,
                                           double* wtok) {
  constexpr int P = kCap / kBlock;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const unsigned long long k = L.key[i];
    L.key[i] = ((unsigned long long)(uint32_t)k << 32) | (k >> 32);
  }
  __syncthreads();
  sort_keys_desc(L, n);
  const int m0 = (int)threadIdx.x * P;
  float w[P];
  double local = 0.0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    w[i] = m0 + i < n ? weight(key2f((uint32_t)L.key[m0 + i]), M, c) : 0.0f;
    local += (double)w[i];
  }
  double tot;
  const double ex = block_excl_scan<kBlock>(local, &tot, L.bs);
  const double target = u * tot;
  int hit = 0x7FFFFFFF, lastw = -1;
  double run = ex;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    run += (double)w[i];
    if (w[i] > 0.0f) {
      lastw = m0 + i;
      if (hit == 0x7FFFFFFF && target < run) hit = m0 + i;
    }
  }
  int pos = block_min<kBlock>(hit, L.bs);
  if (pos == 0x7FFFFFFF) pos = block_max<kBlock>(lastw, L.bs);
  const int token = (int)~key_hi(L.key[pos]);
  *wtok = (double)weight(key2f((uint32_t)L.key[pos]), M, c);
  __syncthreads();
  return token;
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
      lc += (int)L.hcnt[hslot(lane * PER + i)];
      lm += L.hmass[hslot(lane * PER + i)];
    }
    const int ic = wave_incl_scan(lc);
    const unsigned long long im = wave_incl_scan(lm);
    int run_c = ic - lc;
    unsigned long long run_m = im - lm;
    int dk = kBins, dp = -1, first = kBins;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = lane * PER + i;
      const int cb = (int)L.hcnt[hslot(b)];
      if (cb > 0 && first == kBins) first = b;
      if (f.k_on && dk == kBins && cb > 0 && cnt_above + run_c + cb >= f.k) dk = b;
      if (f.p_on && cb > 0 && mass_above + (double)run_m * kInvFix < thr) dp = b;
      run_c += cb;
      run_m += L.hmass[hslot(b)];
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
        bc += (int)L.hcnt[hslot(b)];
        bm += L.hmass[hslot(b)];
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

// Wave 0 resolves the candidates of the per-wavefront regions (at most
// kWaveCap in all; every logit >= the candidate bound, which is <= tau) and
// draws from S in token-id order.
//  - Value order, needed only when top-k can cut (more candidates than k) or
//    top-p may drop a group: the candidates are sorted by (value, lowest id
//    first); the first position of a lane's tie group is the number of logits
//    strictly above it, and an exclusive scan of the weights at that position
//    is their mass. Every filter keeps a prefix of this order. Top-p keeps
//    every group for certain when the mass above the lowest group is already
//    below the threshold.
//  - JOINT top-p compares against top_p * Z. With only a lower bound of Z
//    (z_exact false) a group that the bound would drop might be kept by the
//    exact Z: then nothing is decided, L.si[7] is set and the caller calls
//    again with the exact Z.
//  - The draw: the kept candidates sorted by token id, an inclusive scan of
//    their weights C, and the first id with u * Z_S < C.
// At most 16 candidates are sorted inside the first 16 lanes (DPP only).
// Results: L.si[0] token, L.si[1] |S|, L.sf[0] tau, L.sd[1] Z_S (sum of
// weights over S), L.si[7] 0 or 1 (see above). Wave 0 only, all lanes active.
template <int W>
__device__ __forceinline__ void wave_resolve_draw_w(Lds& L, unsigned long long key, int n, float M,
                                                    float c, const Filters& f, double zref,
                                                    bool z_exact, bool all_in, double u) {
  const int lane = __lane_id();
  if (all_in) {   // the candidates are every finite element: their sum is Z
    zref = sum_w<W>(lane < n ? (double)weight(key2f(key_hi(key)), M, c) : 0.0);
    z_exact = true;
  }
  const uint32_t kM = fkey(M);
  const bool seq_kp = f.seq && f.k_on && f.p_on;
  const bool k_cuts = f.k_on && n > f.k;
  int n_in;
  float tau;
  // token-id order for the draw: (~id) << 32 | value key, descending; sorted
  // alongside the value order (two independent chains the scheduler can
  // interleave) and masked by S = {v >= tau} afterwards
  const unsigned long long idkey =
      lane < n ? (((unsigned long long)(uint32_t)key << 32) | key_hi(key)) : 0ull;
  unsigned long long ids;
  bool sorted = k_cuts;
  if (!k_cuts && f.p_on) {
    // top-p is certain to keep every group when the mass above the lowest
    // group is below its threshold (top-k keeps all n candidates here)
    const bool valid = lane < n;
    const uint32_t kh = key_hi(key);
    const double w = valid ? (double)weight(key2f(kh), M, c) : 0.0;
    const double wall = sum_w<W>(w);
    const uint32_t kmin = min_u32_w<W>(valid ? kh : 0xFFFFFFFFu);
    const double above = wall - sum_w<W>(valid && kh == kmin ? w : 0.0);
    const double thr = f.top_p * (seq_kp ? wall : (z_exact ? zref : zref * (1.0 - 1e-4)));
    sorted = !(above < thr) && kmin != kM;
  }
  if (sorted) {
    // the value order alone decides the cut (equal values form one group),
    // so the value keys sort without their ids
    ids = wave_sort_desc<W>(idkey);
    const uint32_t kh = wave_sort_desc<W>(key_hi(key));
    const bool valid = lane < n;
    const float v = key2f(kh);
    const double w = valid ? (double)weight(v, M, c) : 0.0;
    const uint32_t prev = dpp_u32<kDppWaveShr1>(kh);
    const bool start = valid && (lane == 0 || prev != kh);
    const int cnt_gt = incl_max_scan_w<W>(start ? lane : 0);
    const double incl = incl_scan_w<W>(w);
    const double mass_gt = incl_max_scan_w<W>(start ? incl - w : 0.0);
    const bool keep_k = !f.k_on || cnt_gt < f.k;
    const bool keep_m = v >= f.tau_m;
    bool keep_p = true;
    if (f.p_on) {
      double thr;
      if (seq_kp)
        thr = f.top_p * sum_w<W>(valid && keep_k ? w : 0.0);
      else
        thr = f.top_p * (z_exact ? zref : zref * (1.0 - 1e-4));
      keep_p = mass_gt < thr || kh == kM;
      if (!seq_kp && !z_exact && __any(valid && keep_k && keep_m && !keep_p)) {
        if (lane == 0) L.si[7] = 1;
        return;
      }
    }
    // every filter keeps a prefix of whole groups: S = {v >= tau}
    const bool keep = valid && keep_k && keep_m && keep_p;
    n_in = __popcll(__ballot(keep));
    tau = key2f(readlane_u32(kh, n_in - 1));
  } else {
    ids = wave_sort_desc<W>(idkey);
    const uint32_t kh = key_hi(key);
    const bool keep = lane < n && key2f(kh) >= f.tau_m;
    n_in = __popcll(__ballot(keep));
    tau = key2f(min_u32_w<W>(keep ? kh : 0xFFFFFFFFu));
  }
  const float vi = key2f((uint32_t)ids);
  const bool in = lane < n && vi >= tau;
  const uint32_t idx = ~key_hi(ids);
  const double w = in ? (double)weight(vi, M, c) : 0.0;
  const double C = incl_scan_w<W>(w);
  const double total = readlane_t(C, W - 1);
  const double target = u * total;
  const unsigned long long hit = __ballot(in && C > target);
  int pos;
  if (hit) {
    pos = __ffsll((long long)hit) - 1;
  } else {  // rounding put the target past the end: the last kept id with weight
    const unsigned long long pw = __ballot(in && w > 0.0);
    pos = 63 - __clzll((long long)pw);
  }
  const int token = (int)readlane_u32(idx, pos);
  const double wt = readlane_t(w, pos);
  if (lane == 0) {
    L.si[0] = token;
    L.si[1] = n_in;
    L.si[7] = 0;
    L.sf[0] = tau;
    L.sd[1] = total;
    L.sd[2] = wt;
  }
}

__device__ __forceinline__ void wave_resolve_draw(Lds& L, float M, float c, const Filters& f,
                                                  double zref, bool z_exact, bool all_in,
                                                  double u) {
  const int lane = __lane_id();
  // all counts first (independent LDS reads), then one read per lane
  int cq[kWaves];
#pragma unroll
  for (int q = 0; q < kWaves; ++q) cq[q] = L.wcnt[q];
  int n = 0, sq = 0, so = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    if (lane >= n && lane < n + cq[q]) {
      sq = q;
      so = lane - n;
    }
    n += cq[q];
  }
  unsigned long long key = 0ull;
  if (lane < n) key = cand_key(__uint_as_float(L.wc[sq].val[so]), (int)L.wc[sq].idx[so]);
  if (n <= 16)
    wave_resolve_draw_w<16>(L, key, n, M, c, f, zref, z_exact, all_in, u);
  else
    wave_resolve_draw_w<64>(L, key, n, M, c, f, zref, z_exact, all_in, u);
}

}  // namespace tsr
