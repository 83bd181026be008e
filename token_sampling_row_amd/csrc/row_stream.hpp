// The streaming general path: rows wider than the register file, and kept
// sets the candidate bound cannot narrow (top-p over a wide nucleus, min-p or
// top-k over thousands of logits). Each pass re-reads the row through the
// cache hierarchy; the functions are not inlined so the register-resident
// kernels pay nothing for them.
//
// Kept-set search: a histogram of (count, mass) over log-probability bins of
// the logits >= the min-p threshold finds the bin where top-k or top-p cuts;
// histograms over exact key digits narrow that bin until what is left fits
// in LDS, where it is sorted and resolved exactly (resolve_sorted).
#pragma once

#include "row_common.hpp"

namespace tsr {

template <int DT>
struct StreamRow {
  static constexpr int EPC = Fmt<DT>::EPC;
  const unsigned char* p;
  int V;
  int nct;        // chunks per thread
  const uint32_t* mask;   // the row's allowed-token words, or null
  int hn;                 // look-back window entries published in LDS (0: no penalty)
  double rpen;            // repetition penalty

  __device__ __forceinline__ StreamRow(const unsigned char* p_, int V_,
                                       const uint32_t* mask_ = nullptr, int hn_ = 0,
                                       double rpen_ = 1.0)
      : p(p_), V(V_), mask(mask_), hn(hn_), rpen(rpen_) {
    const long long chunks = ((long long)V + EPC - 1) / EPC;
    nct = (int)((chunks + kBlock - 1) / kBlock);
  }
  __device__ __forceinline__ long long chunk_id(int j) const {
    return (long long)j * kBlock + threadIdx.x;
  }
  __device__ __forceinline__ int base(int j) const { return (int)(chunk_id(j) * EPC); }
  __device__ __forceinline__ uint4 chunk(int j) const {
    const long long c = chunk_id(j);
    if (c * EPC >= V) return neg_inf_chunk<DT>();
    // a whole chunk is one 16-byte load at whatever alignment the row has
    // (the unaligned access mode); the partial one is read element-wise
    uint4 t;
    if ((c + 1) * EPC <= V)
      __builtin_memcpy(&t, p + c * EPC * Fmt<DT>::ESZ, sizeof(t));
    else
      t = load_chunk_slow<DT>(p, c, V);
    uint4 m = mask ? apply_mask<DT>(t, chunk_mask_bits<DT>(mask, c)) : t;
    if (hn > 0) {   // window tokens in this chunk (the hashed flag first)
      const Lds& L = tsr_lds;
      if ((L.hbits[(c >> 5) & (kWave - 1)] >> (c & 31)) & 1u) {
        uint32_t hit = 0u;
        for (int h = 0; h < hn; ++h) {
          const long long d = (long long)L.hist[h] - c * EPC;
          hit |= (d >= 0 && d < EPC) ? 1u << (uint32_t)d : 0u;
        }
        if (hit) m = penalize_chunk<DT>(m, hit, rpen);
      }
    }
    return m;
  }
  __device__ __forceinline__ void elems(int j, float* v, float* m) const {
    unpack<DT>(chunk(j), v);
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < EPC; ++e) mx = fmaxf(mx, v[e]);
    *m = mx;
  }
};

struct StreamStats {
  int status;
  float M;
  float smin;
  double z;
};

template <int DT>
__device__ __noinline__ StreamStats stream_stats(const StreamRow<DT> s, bool need_z, float c) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  float tmax = kNegInf, smin = kPosInf, mt = kNegInf;
  double zt = 0.0;
  bool bad = false;
  for (int j = 0; j < s.nct; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
#pragma unroll
    for (int e = 0; e < EPC; ++e) bad |= !(v[e] <= kFltMax);
    tmax = fmaxf(tmax, m);
    if (m > kNegInf) smin = fminf(smin, m);
    if (need_z && m > kNegInf) {
      if (m > mt) {
        zt = (mt > kNegInf) ? zt * (double)weight(mt, m, c) : 0.0;
        mt = m;
      }
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) t += weight(v[e], mt, c);
      zt += (double)t;
    }
  }
  StreamStats st;
  st.M = block_max<kBlock>(tmax, L.bs);
  const int anybad = block_max<kBlock>(bad ? 1 : 0, L.bs);
  st.smin = block_min<kBlock>(smin, L.bs);
  st.z = -1.0;
  if (need_z) {
    const double mine = (mt > kNegInf && st.M > kNegInf) ? zt * (double)weight(mt, st.M, c) : 0.0;
    st.z = block_sum<kBlock>(mine, L.bs);
  }
  st.status = (anybad || st.M == kPosInf) ? 1 : (st.M > kNegInf ? 0 : 2);
  return st;
}

template <int DT>
__device__ __noinline__ int stream_argmax(const StreamRow<DT> s, float M) {
  constexpr int EPC = Fmt<DT>::EPC;
  int best = 0x7FFFFFFF;
  for (int j = 0; j < s.nct && best == 0x7FFFFFFF; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
    if (m == M) {
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (v[e] == M) best = min(best, s.base(j) + e);
    }
  }
  return block_min<kBlock>(best, tsr_lds.bs);
}

template <int DT>
__device__ __noinline__ double stream_weight_sum(const StreamRow<DT> s, float tau, float M,
                                                 float c) {
  constexpr int EPC = Fmt<DT>::EPC;
  double z = 0.0;
  for (int j = 0; j < s.nct; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
    if (m >= tau) {
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) t += v[e] >= tau ? weight(v[e], M, c) : 0.0f;
      z += (double)t;
    }
  }
  return block_sum<kBlock>(z, tsr_lds.bs);
}

// One kept-set search (see the file comment) for the filters f with top-p
// threshold thr (in weight units). Returns tau; kept / zs are filled when the
// search resolved them (else -1). Row is a StreamRow, or a view of a row held
// in registers with the same interface (nct, elems(j, v, &max), base(j)).
template <int DT, class Row>
__device__ __forceinline__ Cut general_search(const Row& s, float M, float c, float cR,
                                              const Filters& f, double thr) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  const int tid = threadIdx.x;
  const float tau_m = f.tau_m;
  for (int i = tid; i < kBins; i += kBlock) {
    L.hcnt[i] = 0u;
    L.hmass[i] = 0ull;
  }
  __syncthreads();
  auto lbin = [&](float v) -> int {
    const float t = (M - v) * cR;
    return t < (float)(kBins - 1) ? (int)t : kBins - 1;
  };
#pragma unroll 1
  for (int j = 0; j < s.nct; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
    if (m >= tau_m && m > kNegInf) {
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (v[e] >= tau_m && v[e] > kNegInf) {
          const int b = lbin(v[e]);
          atomicAdd(&L.hcnt[hslot(b)], 1u);
          atomicAdd(&L.hmass[hslot(b)], to_fixed(weight(v[e], M, c)));
        }
    }
  }
  __syncthreads();
  int add_c = 0;
  double add_m = 0.0;
  const int d = find_boundary(L, 0, 0.0, f, thr, true, &add_c, &add_m);
  Cut cut;
  if (d == kBins) {  // no cut inside: S = every finite logit >= tau_m
    cut.tau = tau_m > kNegInf ? tau_m : -kFltMax;
    cut.kept = -1;
    cut.zs = -1.0;
    return cut;
  }
  int cnt_above = add_c;
  double mass_above = add_m;
  int ncur = (int)L.hcnt[hslot(d)];
  __syncthreads();
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
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  #pragma unroll 1
  for (int j = 0; j < s.nct; ++j) {
      float v[EPC], m;
      s.elems(j, v, &m);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (in_region(v[e])) {
          const uint32_t kk = fkey(v[e]);
          mn = min(mn, kk);
          mx = max(mx, kk);
        }
    }
    mn = block_min_u32<kBlock>(mn, L.bs);
    mx = block_max_u32<kBlock>(mx, L.bs);
    by_key = true;
    klo = mn;
    khi = mx;
    if (mn == mx) break;  // a single tie group, decided whole below
    const uint32_t span = mx - mn;
    const int bits = 32 - __clz(span);
    const int shift = bits > 10 ? bits - 10 : 0;
    for (int i = tid; i < kBins; i += kBlock) {
      L.hcnt[i] = 0u;
      L.hmass[i] = 0ull;
    }
    __syncthreads();
  #pragma unroll 1
  for (int j = 0; j < s.nct; ++j) {
      float v[EPC], m;
      s.elems(j, v, &m);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (in_region(v[e])) {
          const int b = (kBins - 1) - (int)((fkey(v[e]) - klo) >> shift);
          atomicAdd(&L.hcnt[hslot(b)], 1u);
          atomicAdd(&L.hmass[hslot(b)], to_fixed(weight(v[e], M, c)));
        }
    }
    __syncthreads();
    const bool has_max = contains_max && (khi == fkey(M));
    const int d2 = find_boundary(L, cnt_above, mass_above, f, thr, has_max, &add_c, &add_m);
    const int dd = d2 == kBins ? kBins - 1 : d2;
    ncur = (int)L.hcnt[hslot(dd)];
    cnt_above += add_c;
    mass_above += add_m;
    const uint32_t lo2 = klo + ((uint32_t)((kBins - 1) - dd) << shift);
    const uint32_t hi2 = min(khi, lo2 + ((1u << shift) - 1u));
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
    if (f.k_on && !(cnt_above < f.k)) keep = false;
    if (f.p_on && !(mass_above < thr) && fkey(v) != fkey(M)) keep = false;
    cut.tau = keep ? v : next_up(v);
    cut.kept = cnt_above + (keep ? ncur : 0);
    cut.zs = mass_above + (keep ? (double)ncur * w : 0.0);
    return cut;
  }
  int cnt = 0;
#pragma unroll 1
  for (int j = 0; j < s.nct; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
#pragma unroll
    for (int e = 0; e < EPC; ++e) cnt += in_region(v[e]) ? 1 : 0;
  }
  int total;
  int off = block_excl_scan<kBlock>(cnt, &total, L.bs);
  if (cnt) {
  #pragma unroll 1
  for (int j = 0; j < s.nct; ++j) {
      float v[EPC], m;
      s.elems(j, v, &m);
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (in_region(v[e]) && off < kCap) L.key[off++] = cand_key(v[e], s.base(j) + e);
    }
  }
  __syncthreads();
  total = min(total, kCap);
  sort_keys_desc(L, total);
  const Resolved res = resolve_sorted(L, total, cnt_above, mass_above, M, c, f, thr, false);
  if (res.n_in > 0) {
    cut.tau = res.tau;
    cut.kept = cnt_above + res.n_in;
    cut.zs = res.zs;
  } else {
    // nothing of the region stays: S is exactly what lies above it
    cut.tau = by_key ? next_up(key2f(khi)) : tau_m;
    cut.kept = cnt_above;
    cut.zs = mass_above;
  }
  return cut;
}

// The kept set when the candidate bound failed: Z is the row's weight sum or
// -1 (then summed here).
template <int DT>
__device__ __noinline__ Cut general_stream(const StreamRow<DT> s, float M, double Z, float c,
                                           float cR, const Filters f) {
  if (!f.k_on && !f.p_on) {
    Cut cut;
    cut.tau = f.tau_m > kNegInf ? f.tau_m : -kFltMax;
    cut.kept = -1;
    cut.zs = -1.0;
    return cut;
  }
  if (Z < 0.0 && f.p_on && !(f.seq && f.k_on)) Z = stream_weight_sum(s, -kFltMax, M, c);
  if (f.seq && f.k_on && f.p_on) {
    // SEQUENTIAL: top-k alone first; its kept mass is top-p's reference
    Filters fk = f;
    fk.p_on = false;
    fk.m_on = false;
    fk.tau_m = kNegInf;
    const Cut ck = general_search<DT>(s, M, c, cR, fk, 0.0);
    double zk = ck.zs;
    if (zk < 0.0) zk = stream_weight_sum(s, ck.tau, M, c);
    return general_search<DT>(s, M, c, cR, f, f.top_p * zk);
  }
  return general_search<DT>(s, M, c, cR, f, f.p_on ? f.top_p * Z : 0.0);
}

// Inverse-CDF draw over S = {v >= tau} in ascending token id, streaming the
// row in batches of kWalkBatch chunk rows. Returns the token; *total_out the
// weight sum over S.
template <int DT>
__device__ __noinline__ int walk_stream(const StreamRow<DT> s, float tau, float M, float c,
                                        double u, double* total_out, double* wtok) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  const int tid = threadIdx.x, lane = __lane_id(), wid = tid / kWave;
  const double Z = stream_weight_sum(s, tau, M, c);
  *total_out = Z;
  const double target = u * Z;
  double before = 0.0;      // weight of the batches already passed
  int jstar = -1, last_nz = -1;
  double r1 = 0.0;
  for (int j0 = 0; j0 < s.nct && jstar < 0; j0 += kWalkBatch) {
    const int nb = min(kWalkBatch, s.nct - j0);
    for (int jj = 0; jj < nb; ++jj) {
      float v[EPC], m;
      s.elems(j0 + jj, v, &m);
      float t = 0.0f;
      if (m >= tau) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) t += v[e] >= tau ? weight(v[e], M, c) : 0.0f;
      }
      double sd = (double)t;
      if (__any(sd > 0.0)) sd = wave_sum(sd);
      if (lane == 0) L.jsum[wid * kWalkBatch + jj] = sd;
    }
    __syncthreads();
    if (tid < kWave) {
      double sj = 0.0;
      if (lane < nb)
        for (int w = 0; w < kWaves; ++w) sj += L.jsum[w * kWalkBatch + lane];
      const double incl = wave_incl_scan(sj) + before;
      const double excl = incl - sj;
      const unsigned long long hit = __ballot(sj > 0.0 && target < incl);
      const unsigned long long nz = __ballot(sj > 0.0);
      const int hl = hit ? __ffsll((long long)hit) - 1 : 0;
      const double e_at = readlane_t(excl, hl);
      const double batch_end = readlane_t(incl, 63);
      if (lane == 0) {
        L.si[2] = hit ? j0 + hl : -1;
        L.sd[2] = target - e_at;
        L.sd[3] = batch_end;
        L.si[5] = nz ? j0 + 63 - __clzll((long long)nz) : -1;
      }
    }
    __syncthreads();
    jstar = L.si[2];
    r1 = L.sd[2];
    if (L.si[5] >= 0) last_nz = L.si[5];
    before = L.sd[3];
    __syncthreads();
  }
  bool fallback = false;
  if (jstar < 0) {  // rounding put the target past the end: the last kept token
    jstar = max(last_nz, 0);
    fallback = true;
  }
  float v[EPC], m;
  s.elems(jstar, v, &m);
  float wj[EPC];
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    wj[e] = v[e] >= tau ? weight(v[e], M, c) : 0.0f;
    mine += (double)wj[e];
  }
  double tot2;
  const double ex = block_excl_scan<kBlock>(mine, &tot2, L.bs);
  const bool own = !fallback && mine > 0.0 && ex <= r1 && r1 < ex + mine;
  int owner = block_min<kBlock>(own ? tid : 0x7FFFFFFF, L.bs);
  if (owner == 0x7FFFFFFF) {
    owner = block_max<kBlock>(mine > 0.0 ? tid : -1, L.bs);
    fallback = true;
  }
  if (tid == owner) {
    double run = ex;
    int pick = -1, lastpos = -1;
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      if (wj[e] > 0.0f) {
        run += (double)wj[e];
        lastpos = e;
        if (pick < 0 && !fallback && r1 < run) pick = e;
      }
    if (pick < 0) pick = lastpos;
    L.si[3] = s.base(jstar) + pick;
    double wp = 0.0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) wp = e == pick ? (double)wj[e] : wp;
    L.sd[4] = wp;
  }
  __syncthreads();
  const int tok = L.si[3];
  *wtok = L.sd[4];
  __syncthreads();
  return tok;
}

// |S| and the smallest kept value for S = {v >= tau}.
template <int DT>
__device__ __noinline__ void stream_kept_stats(const StreamRow<DT> s, float tau, int* count,
                                               float* vmin) {
  constexpr int EPC = Fmt<DT>::EPC;
  int n = 0;
  float mn = kPosInf;
  for (int j = 0; j < s.nct; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
    if (m >= tau) {
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (v[e] >= tau) {
          ++n;
          mn = fminf(mn, v[e]);
        }
    }
  }
  *count = block_sum<kBlock>(n, tsr_lds.bs);
  *vmin = block_min<kBlock>(mn, tsr_lds.bs);
}

// Dense p~ (eq. 39.2) for the validation output.
template <int DT>
__device__ __noinline__ void stream_probs(const StreamRow<DT> s, float tau, float M, float c,
                                          double zs, float* out) {
  constexpr int EPC = Fmt<DT>::EPC;
  const double inv = 1.0 / zs;
  for (int j = 0; j < s.nct; ++j) {
    float v[EPC], m;
    s.elems(j, v, &m);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int i = s.base(j) + e;
      if (i < s.V) out[i] = v[e] >= tau ? (float)((double)weight(v[e], M, c) * inv) : 0.0f;
    }
  }
}

}  // namespace tsr
