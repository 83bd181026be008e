// The register-resident fast path: one workgroup holds its row in VGPRs
// (thread t owns 16-byte chunks j*kBlock + t, j < NC), reads HBM once and
// resolves the kept set from a few candidates staged in LDS.
//
// Candidate bound Lb <= tau: min-p gives a logit threshold directly; top-k
// uses a sketch, the k-th largest of the per-thread (or per-chunk) maxima,
// which can only be at or below the k-th largest logit. The logits >= Lb are
// the candidates; at most kWaveCap of them are resolved and drawn by one
// wavefront with no barriers, up to kCap by the whole workgroup.
//
// Code size matters as much as instruction count here: a launch runs each
// phase once per workgroup, so code the instruction cache does not hold is
// fetched from memory at every launch. Only the pass that reduces chunks as
// their loads land is unrolled (its waits count loads); every later pass
// loops over chunk rows, reading chunk j of the register-resident row with a
// wavefront-uniform j (s_set_gpr_idx indexing of a register vector).
#pragma once

#include "row_common.hpp"

#ifndef TSR_ROW_NO_CMAX
#define TSR_ROW_NO_CMAX 0
#endif

namespace tsr {

// Cache policy of the row loads: non-temporal, so the streamed logits are the
// first lines the caches give up and the kernel's own code stays in L2 from
// one launch to the next (each dispatch starts with a cold instruction cache).
constexpr int kLoadNonTemporal = 2;

template <int N> struct VecU { typedef uint32_t type __attribute__((ext_vector_type(N))); };
template <int N> struct VecF { typedef float type __attribute__((ext_vector_type(N))); };

// Register vectors hold at most 32 dwords: a row of NC chunk rows per thread
// lives in a power-of-two bank A and, when NC is not a power of two, a bank B
// with the rest.
constexpr int bank_a(int nc) {
  return nc >= 32 ? 32 : nc >= 16 ? 16 : nc >= 8 ? 8 : nc >= 4 ? 4 : nc >= 2 ? 2 : 1;
}

template <int DT, int NC>
struct RegRow {
  static constexpr int EPC = Fmt<DT>::EPC;
  static constexpr int NA = bank_a(NC);
  static constexpr int NB = NC - NA;
  static constexpr int NBS = NB > 0 ? NB : 1;
  static_assert(NB <= 32, "chunk rows per thread");
  typename VecU<NA>::type ax, ay, az, aw;   // the chunks, one vector per dword
  typename VecU<NBS>::type bx, by, bz, bw;
  // Chunk maxima (-inf past the end of the row), kept in registers up to 32
  // chunk rows; wider rows recompute them (their registers are needed more),
  // as do the units that hold two rows (TSR_ROW_NO_CMAX defined to 1 before
  // this header: the verify step).
  static constexpr bool kKeepCmax = NC <= 32 && !TSR_ROW_NO_CMAX;
  typename VecF<kKeepCmax ? NA : 1>::type ca;
  typename VecF<kKeepCmax ? NBS : 1>::type cb;
  float tmax;     // this thread's maximum

  int nwhole;     // whole 16-byte chunks in the row (chunk ids at or past it are not)
  int jfull;      // chunk rows j < jfull are whole for every thread
  uint4 tail;     // the partial chunk, read element-wise, when the row is ragged

  // Chunk row j: a compile-time j in unrolled code, else wavefront-uniform.
  __device__ __forceinline__ uint4 get(int j) const {
    if (NB == 0 || j < NA) return make_uint4(ax[j], ay[j], az[j], aw[j]);
    const int i = j - NA;
    return make_uint4(bx[i], by[i], bz[i], bw[i]);
  }
  __device__ __forceinline__ void put(int j, uint4 t) {
    if (NB == 0 || j < NA) {
      ax[j] = t.x; ay[j] = t.y; az[j] = t.z; aw[j] = t.w;
    } else {
      const int i = j - NA;
      bx[i] = t.x; by[i] = t.y; bz[i] = t.z; bw[i] = t.w;
    }
  }
  __device__ __forceinline__ float cmax(int j) const;
  __device__ __forceinline__ void put_cmax(int j, float m) {
    if constexpr (kKeepCmax) {
      if (NB == 0 || j < NA) ca[j] = m; else cb[j - NA] = m;
    }
  }

  // Whole chunks of a row are 128-bit buffer loads off one resource whose
  // size is the row's whole chunks, all issued back to back. The full byte
  // offset of each load goes in its VGPR offset, the part the hardware checks
  // against the resource size (the scalar offset is not checked), so chunks
  // at or past `nwhole` are never read: they come back as zeros and are
  // replaced in pass A of reg_stats (by -inf, or by `tail` for the partial
  // chunk of a ragged row), and no wait is forced here. A row need not start
  // on a 16-byte boundary (an odd row stride): the HSA runtime runs the GPU in
  // unaligned access mode, which the compiler assumes for every global access
  // too, and a 128-bit load at any byte address returns those 16 bytes.
  __device__ __forceinline__ void load(const unsigned char* p, int V, bool ragged) {
    nwhole = V / EPC;
    jfull = nwhole / kBlock;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(p), (short)0, nwhole * 16, 0x00020000);
    const int voff = (int)threadIdx.x * 16;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      put(j, __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, voff + j * kBlock * 16, 0, kLoadNonTemporal)));
      sched_fence();   // issue in chunk order: pass A waits for them in that order
    }
    tail = neg_inf_chunk<DT>();
    if (ragged && nwhole * EPC < V && (nwhole % kBlock) == (int)threadIdx.x)
      tail = load_chunk_slow<DT>(p, nwhole, V);
  }
  // Pass-A fix-up of chunk j (see load): only chunk rows at or past jfull
  // (a uniform test) can hold chunks past the end; the fix is branch-free.
  __device__ __forceinline__ uint4 settle(int j, uint4 t) const {
    if (j >= jfull) {
      const int cid = j * kBlock + (int)threadIdx.x;
      const uint4 ni = neg_inf_chunk<DT>();
      const bool past = cid >= nwhole, at = cid == nwhole;
      t.x = past ? (at ? tail.x : ni.x) : t.x;
      t.y = past ? (at ? tail.y : ni.y) : t.y;
      t.z = past ? (at ? tail.z : ni.z) : t.z;
      t.w = past ? (at ? tail.w : ni.w) : t.w;
    }
    return t;
  }
  __device__ __forceinline__ int base(int j) const {
    return (j * kBlock + (int)threadIdx.x) * EPC;
  }
  __device__ __forceinline__ void elems(int j, float* v) const { unpack<DT>(get(j), v); }
};

// Constrained decoding: the allowed-token mask words of a register row, in
// registers. Every chunk row j of a G-lane group (G = 32 / EPC chunks per
// word) reads one mask word, so lane t of the group loads the word of chunk
// row q*G + (t mod G) for q < NQ, and chunk row j's word reaches the group's
// lanes from lane j mod G (DPP quad permute for bf16, a swizzle for fp32).
// Ordinary loads issued before the row's: their waits are the compiler's, no
// LDS and no barrier. Words past the mask read as 0 (disallowed).
template <int DT, int NC>
struct MaskRegs {
  static constexpr int G = 32 / Fmt<DT>::EPC;
  static constexpr int NQ = (NC + G - 1) / G;
  uint32_t w[NQ];
  __device__ __forceinline__ void load(const uint32_t* m, int V) {
    const int words = (V + 31) >> 5;
    const int t = (int)threadIdx.x;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int jr = q * G + t % G;
      const int wi = jr * (kBlock / G) + t / G;
      const uint32_t x = m[wi < words ? wi : words - 1];
      w[q] = (jr < NC && wi < words) ? x : 0u;
    }
    sched_fence();   // issued before the row's loads, so they land first
  }
  template <int J>
  __device__ __forceinline__ uint32_t get() const {
    constexpr int R = J % G;
    const int x = (int)w[J / G];
    if constexpr (G == 4) {
      return (uint32_t)__builtin_amdgcn_update_dpp(0, x, R | (R << 2) | (R << 4) | (R << 6), 0xF,
                                                   0xF, false);
    } else {
      static_assert(G == 8, "fp32 or bf16");
      return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x18 | (R << 5));
    }
  }
};

// Bit j set iff pred(j) holds in some lane (pred is evaluated by every lane;
// call with the whole wavefront active). Each lane sets its own bits (vector
// instructions only, no scalar test per chunk row), then one OR across the
// wavefront.
template <int NC, class Pred>
__device__ __forceinline__ unsigned long long wave_chunk_mask(Pred pred) {
  static_assert(NC <= 64, "one bit per chunk row");
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (j < 32) lo |= pred(j) ? (1u << (j & 31)) : 0u;
    else hi |= pred(j) ? (1u << (j & 31)) : 0u;
  }
  auto bor = [](uint32_t a, uint32_t b) { return a | b; };
  lo = wave_reduce(lo, bor);
  if constexpr (NC > 32) hi = wave_reduce(hi, bor);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ int pop_low(unsigned long long& m) {
  const int j = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
  m &= m - 1ull;
  return j;
}

// Largest element of a chunk (both halves of a bf16 word widened exactly);
// NaN if the chunk holds one.
template <int DT>
__device__ __forceinline__ float chunk_max(uint4 t) {
  float v[Fmt<DT>::EPC];
  unpack<DT>(t, v);
  if constexpr (DT == 0) {
    return fmax3n(fmax3n(v[0], v[1], v[2]), v[3], v[3]);
  } else {
    float m = fmax3n(v[0], v[1], v[2]);
    m = fmax3n(m, v[3], v[4]);
    m = fmax3n(m, v[5], v[6]);
    return fmaxn(m, v[7]);
  }
}

template <int DT, int NC>
__device__ __forceinline__ float RegRow<DT, NC>::cmax(int j) const {
  if constexpr (kKeepCmax) return (NB == 0 || j < NA) ? ca[j] : cb[j - NA];
  else return chunk_max<DT>(get(j));
}

// The per-row look-back window of the repetition penalty (hn ids, lane h of
// wave 0 holding id hv; r the penalty), chosen at run time.
struct RowExtras {
  int hn = 0;
  int hv = -1;
  double r = 1.0;
  const unsigned char* row = nullptr;   // the row's logits (window values are read back)
};

struct RowStats {
  int status;     // TSR_ROW_*
  float M;        // row max
  float tmin;     // smallest finite per-thread maximum
  double zlo;     // a lower bound of the row's weight sum (when asked for)
  int nallow;     // at least the number of allowed elements (huge without a mask)
};

// Row statistics in one pass over the registers as the loads land: NaN/+inf
// detection, chunk maxima, thread max. The empty asm at the end of each chunk
// pins the running maximum in program order, so chunk j is reduced as soon as
// its load has arrived instead of after the whole row.
// need_zlo: also sum the weights of the per-thread maxima (one exponential
// per thread). That is a lower bound of the row's
// weight sum Z, enough to settle JOINT top-p whenever the nucleus is not
// close to the cut.
// MASK: apply the allowed-token mask (mk, loaded before the row) to each
// chunk first, and count the allowed tokens (a row with few of them is
// resolved over all its finite elements). Then, when x holds a look-back
// window, the repetition penalty: wave 0 reads the window tokens' logits back
// and publishes their penalised values, and the thread that holds a window
// token puts its new value in place and refreshes its maxima (REP instances).
// Pass A over the registers as the loads land (see reg_stats); MASKED: the
// allowed-token mask words (mk) are applied to each chunk first and the
// allowed ids counted in *nallow. Returns the
// thread's maximum.
// ONLINE: also the thread's weight sum relative to its own maximum, formed as
// the chunks land (the running sum is rescaled whenever the running maximum
// grows), in *z; c = log2(e) / T.
template <int J, int NC, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < NC) {
    f(std::integral_constant<int, J>{});
    static_for<J + 1, NC>(f);
  }
}

template <bool MASKED, bool ONLINE = false, int DT, int NC>
__device__ __forceinline__ float reg_pass_a(RegRow<DT, NC>& r, const Lds& L, float c = 0.0f,
                                            double* z = nullptr,
                                            const MaskRegs<DT, NC>* mk = nullptr,
                                            int* nallow = nullptr) {
  float tmax = kNegInf;
  double zr = 0.0;
  int na = 0;
  // thread t's chunk j takes bits tsh.. of its chunk row's mask word
  const uint32_t tsh = ((uint32_t)threadIdx.x % (32 / Fmt<DT>::EPC)) * Fmt<DT>::EPC;
  static_for<0, NC>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    uint32_t mwc = 0u;
    if constexpr (MASKED) mwc = mk->template get<j>();
    uint4 t = r.get(j);
    asm volatile("" : "+v"(t.x), "+v"(t.y), "+v"(t.z), "+v"(t.w));
    t = r.settle(j, t);
    if constexpr (MASKED) {
      // element-wise masking only where some lane's chunk is partly allowed;
      // wholly allowed or wholly disallowed chunks (the common case of a
      // grammar's small or near-complete sets) take one select per dword
      constexpr uint32_t kAll = (1u << Fmt<DT>::EPC) - 1u;
      const uint32_t bits = (mwc >> tsh) & kAll;
      na += __builtin_popcount(bits);
      if (__any(bits != 0u && bits != kAll)) {
        t = apply_mask<DT>(t, bits);
      } else {
        const uint4 ni = neg_inf_chunk<DT>();
        t.x = bits ? t.x : ni.x;
        t.y = bits ? t.y : ni.y;
        t.z = bits ? t.z : ni.z;
        t.w = bits ? t.w : ni.w;
      }
    }
    r.put(j, t);
    const float m = chunk_max<DT>(t);
    r.put_cmax(j, m);
    if constexpr (ONLINE) {
      const float mn = fmaxn(tmax, m);
      if (mn > kNegInf) {
        zr = tmax > kNegInf ? zr * (double)weight(tmax, mn, c) : 0.0;
        float v[Fmt<DT>::EPC];
        unpack<DT>(t, v);
        float sw = 0.0f;
#pragma unroll
        for (int e = 0; e < Fmt<DT>::EPC; ++e) sw += weight(v[e], mn, c);
        zr += (double)sw;
      }
    }
    tmax = fmaxn(tmax, m);
    asm volatile("" : "+v"(tmax));
  });
  if constexpr (ONLINE) *z = zr;
  if constexpr (MASKED) *nallow = na;
  return tmax;
}

// ZEXACT: need_zlo's sum is the exact Z (every element's weight, formed in
// pass A) instead of a lower bound.
template <bool MASK = false, bool REP = false, bool ZEXACT = false, int DT, int NC>
__device__ __forceinline__ RowStats reg_stats(RegRow<DT, NC>& r, bool need_zlo, float c, Lds& L,
                                              int V = 0, const RowExtras& x = RowExtras{},
                                              const MaskRegs<DT, NC>* mk = nullptr) {
  // allowed ids, counted by chunk in pass A (bits of ids past V in the last
  // chunk may be set: an over-count)
  int nallow = 0x7FFFFFFF;
  double zown = 0.0;
  float tmax = reg_pass_a<MASK, ZEXACT>(r, L, c, &zown, mk, &nallow);
  TSR_STAMP(kStPassA);
  if (REP && x.hn > 0) {
    if (threadIdx.x < kWave) {
      // wave 0: each window token's logit, read back from the row (one per
      // lane, in parallel) and penalised once here
      const bool in = (int)threadIdx.x < x.hn && x.hv >= 0 && x.hv < V;
      if (in) L.hval[threadIdx.x] = penalize<DT>(load_elem<DT>(x.row, x.hv), x.r);
      hist_publish<DT>(x.hv, x.hn, V, L);
    }
    __syncthreads();
    unsigned long long om = L.own[threadIdx.x];
    if (om) {   // this thread's chunks hold window tokens: put their penalised
                // values in place (a repeated id writes the same value again);
                // a masked-out token stays -inf
      while (om) {
        const int h = __builtin_ctzll(om);
        om &= om - 1ull;
        const int id = L.hist[h];
        const int cid = id / Fmt<DT>::EPC;
        const int j = cid / kBlock;
        const uint4 t = replace_elem<DT>(r.get(j), id - cid * Fmt<DT>::EPC, L.hval[h]);
        r.put(j, t);
        r.put_cmax(j, chunk_max<DT>(t));
      }
      float m = kNegInf;
#pragma unroll
      for (int j = 0; j < NC; ++j) m = fmaxn(m, r.cmax(j));
      tmax = m;
    }
  }
  r.tmax = tmax;
  // the thread max's own weight, relative to itself
  static_assert(!(ZEXACT && REP), "the exact sum is formed before the penalty");
  const double zt = (need_zlo && tmax > kNegInf && tmax < kPosInf) ? (ZEXACT ? zown : 1.0) : 0.0;
  // wave level
  const float wm = wave_maxn(tmax);
  const float wt = wave_min(tmax > kNegInf ? tmax : kPosInf);
  const int wb = 0;
  double wz = 0.0;
  int wna = 0;
  if constexpr (MASK) wna = wave_sum(nallow);
  if (need_zlo)   // relative to the wave max
    wz = wave_sum(tmax > kNegInf && tmax < kPosInf ? zt * (double)weight(tmax, wm, c) : 0.0);
  const int wid = threadIdx.x / kWave;
  __syncthreads();
  if (__lane_id() == 0) L.ws[wid] = WaveStats{wm, wt, wz, wb, wna};
  __syncthreads();
  TSR_STAMP(kStStats);
  RowStats st;
  float M = kNegInf, tmin = kPosInf;
  int anybad = 0, na = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    M = fmaxn(M, L.ws[w].m);
    tmin = fminf(tmin, L.ws[w].smin);
    anybad |= L.ws[w].bad;
    na += L.ws[w].na;
  }
  st.nallow = MASK ? na : 0x7FFFFFFF;
  double Z = 0.0;
  if (need_zlo) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (L.ws[w].m > kNegInf && M > kNegInf && M < kPosInf)
        Z += L.ws[w].z * (double)weight(L.ws[w].m, M, c);
  }
  st.M = M;
  st.tmin = tmin;
  st.zlo = Z;
  // NaN or +inf anywhere in the row shows in its (NaN-propagating) maximum
  st.status = (anybad || M != M || M == kPosInf) ? 1 : (M > kNegInf ? 0 : 2);
  TSR_STAMP(kStStatsDone);
  return st;
}

// The row's weight sum Z = sum of 2^((v - M) c) over every element.
template <int DT, int NC>
__device__ __forceinline__ double reg_weight_sum(const RegRow<DT, NC>& r, float M, float c,
                                                 Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  double acc = 0.0;
#pragma nounroll
  for (int j = 0; j < NC; ++j) {
    float v[EPC];
    r.elems(j, v);
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) t += weight(v[e], M, c);
    acc += (double)t;
  }
  return block_sum<kBlock>(acc, L.bs);
}

// Lowest index among the maximal logits.
template <int DT, int NC>
__device__ __forceinline__ int reg_argmax(const RegRow<DT, NC>& r, float M, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  int best = 0x7FFFFFFF;
  if (__any(r.tmax == M)) {
    unsigned long long m = wave_chunk_mask<NC>([&](int j) { return r.cmax(j) == M; });
    while (m) {
      const int j = pop_low(m);
      if (r.cmax(j) == M) {
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
// The per-(chunk row, thread) weight sums of the walk: inside the LDS union
// up to kWalkLds chunk rows per thread, in an array of their own (one
// workgroup per CU holds it) for the wider rows.
template <int NC>
__device__ __forceinline__ float (*walk_sums(Lds& L))[kBlock] {
  if constexpr (NC <= kWalkLds) {
    return L.wsum;
  } else {
    __shared__ float wide[NC][kBlock];
    return wide;
  }
}

// Inverse-CDF draw in ascending token id over per-element weights: the first
// element whose running total exceeds u * (total weight). cw(j, w) fills the
// EPC weights of chunk row j (j is wavefront-uniform). Returns the element
// index (-1: no weight); *total_out gets the total weight, *wtok (if given)
// the drawn element's weight.
// Every thread's chunk sum goes to LDS (no lane exchange per chunk row); each
// chunk row's total is then added over its 512 threads (eight per lane in
// order, then a wavefront sum), wavefront 0 finds the chunk row and, from the
// same LDS sums, the thread where the target falls, and that thread alone
// walks its chunk.
template <int NC, int EPC, class CW>
__device__ __forceinline__ int walk_regs(CW&& cw, double u, Lds& L, double* total_out,
                                         double* wtok = nullptr) {
  static_assert(NC <= kWave, "one lane per chunk row in the search");
  const int tid = threadIdx.x, lane = __lane_id(), wid = tid / kWave;
  float (*wsum)[kBlock] = walk_sums<NC>(L);
  auto weigh = [&](int j) {
    float w[EPC];
    cw(j, w);
    float sf = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) sf += w[e];
    wsum[j][tid] = sf;
  };
  // chunk rows past the 32nd at fixed register indices (a run-time index
  // there takes a select chain per chunk)
  constexpr int kDyn = NC > 32 ? 32 : NC;
#pragma unroll 2
  for (int j = 0; j < kDyn; ++j) weigh(j);
  static_for<kDyn, NC>([&](auto jc) { weigh(decltype(jc)::value); });
  __syncthreads();
  // chunk row totals: wavefront w adds rows w, w + 8, ... (8 sums per lane),
  // its rows' chains side by side up to 32 chunk rows (in the 38-chunk-row
  // instances that costs registers the walk needs: one row at a time there)
  if constexpr (NC > 32) {
    for (int j = wid; j < NC; j += kWaves) {
      double s = 0.0;
#pragma unroll
      for (int q = 0; q < kBlock / kWave; ++q) s += (double)wsum[j][lane * (kBlock / kWave) + q];
      s = wave_sum(s);
      if (lane == 0) L.jsum[j] = s;
    }
  } else {
    constexpr int kPer = (NC + kWaves - 1) / kWaves;
    double s[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = wid + i * kWaves;
      s[i] = 0.0;
      if (j < NC) {
#pragma unroll
        for (int q = 0; q < kBlock / kWave; ++q)
          s[i] += (double)wsum[j][lane * (kBlock / kWave) + q];
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) s[i] = wave_sum(s[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (wid + i * kWaves < NC) L.jsum[wid + i * kWaves] = s[i];
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const double sj = lane < NC ? L.jsum[lane] : 0.0;
    const double incl = wave_incl_scan(sj);
    const double tot = readlane_t(incl, 63);
    const double target = u * tot;
    const unsigned long long hit = __ballot(sj > 0.0 && target < incl);
    const unsigned long long nz = __ballot(sj > 0.0);
    const int last = nz ? 63 - __clzll((long long)nz) : 0;
    const int jstar = hit ? __ffsll((long long)hit) - 1 : last;
    const double r1 = hit ? target - readlane_t(incl - sj, jstar) : kPosInf;
    // the thread of row jstar where r1 falls (lane l holds threads 8l..8l+7)
    double ts[kBlock / kWave];
    double ls = 0.0;
#pragma unroll
    for (int q = 0; q < kBlock / kWave; ++q) {
      ts[q] = (double)wsum[jstar][lane * (kBlock / kWave) + q];
      ls += ts[q];
    }
    const double li = wave_incl_scan(ls);
    const double lx = li - ls;
    const bool mine = ls > 0.0 && lx <= r1 && r1 < li;
    const unsigned long long hl = __ballot(mine);
    int owner = -1;
    double r2 = 0.0;
    if (hl) {
      const int l0 = __ffsll((long long)hl) - 1;
      if (lane == l0) {
        double run = lx;
        for (int q = 0; q < kBlock / kWave; ++q) {
          if (ts[q] > 0.0 && r1 < run + ts[q]) {
            owner = lane * (kBlock / kWave) + q;
            r2 = r1 - run;
            break;
          }
          run += ts[q];
        }
        if (owner < 0) {   // rounding inside the lane: its last thread with weight
          for (int q = kBlock / kWave - 1; q >= 0; --q)
            if (ts[q] > 0.0) {
              owner = lane * (kBlock / kWave) + q;
              break;
            }
          r2 = kPosInf;
        }
      }
      owner = (int)readlane_u32((uint32_t)owner, l0);
      r2 = readlane_t(r2, l0);
    } else {
      // the target past the row's end (rounding): its last thread with weight
      const unsigned long long nzl = __ballot(ls > 0.0);
      const int l1 = nzl ? 63 - __clzll((long long)nzl) : 0;
      int o = -1;
      for (int q = kBlock / kWave - 1; q >= 0; --q)
        if (o < 0 && ts[q] > 0.0) o = lane * (kBlock / kWave) + q;
      owner = (int)readlane_u32((uint32_t)o, l1);
      r2 = kPosInf;
    }
    if (lane == 0) {
      L.si[2] = jstar;
      L.si[3] = owner;
      L.sd[2] = r2;
      L.sd[3] = tot;
    }
  }
  __syncthreads();
  const int jstar = __builtin_amdgcn_readfirstlane(L.si[2]);
  const int owner = __builtin_amdgcn_readfirstlane(L.si[3]);
  *total_out = L.sd[3];
  if (tid == owner) {
    const double r2 = L.sd[2];
    float wj[EPC];
    cw(jstar, wj);
    double run = 0.0;
    int pick = -1, lastpos = -1;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if (wj[e] > 0.0f) {
        run += (double)wj[e];
        lastpos = e;
        if (pick < 0 && r2 < run) pick = e;
      }
    }
    if (pick < 0) pick = lastpos;
    L.si[4] = (jstar * kBlock + tid) * EPC + pick;
    double wp = 0.0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) wp = e == pick ? (double)wj[e] : wp;
    L.sd[4] = wp;
  }
  __syncthreads();
  const int tok = owner >= 0 ? L.si[4] : -1;
  if (wtok) *wtok = L.sd[4];
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
    float v[EPC];
    r.elems(j, v);
    if (tau == -kFltMax) {   // every element (-inf weighs 0): no test at all
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = weight(v[e], M, c);
      return;
    }
    // a chunk wholly below tau is skipped on its maximum (kept in registers,
    // else recomputed); the widest rows keep none and only reach here with
    // wide kept sets, so they weigh every element instead
    constexpr bool kReg = RegRow<DT, NC>::kKeepCmax, kNone = !kReg && NC > 16;
    float mx = v[0];
    if constexpr (!kReg && !kNone) {
#pragma unroll
      for (int e = 1; e < EPC; ++e) mx = fmaxf(mx, v[e]);
    }
    if (kNone || (kReg ? r.cmax(j) : mx) >= tau) {
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
  if (__any(r.tmax >= tau)) {
    unsigned long long m = wave_chunk_mask<NC>([&](int j) { return r.cmax(j) >= tau; });
    while (m) {
      const int j = pop_low(m);
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
  if (tau == -kFltMax) {
    // every finite element: no chunk to skip, so the chunk rows go in
    // program order, a few at a time (independent exponentials)
#pragma unroll 4
    for (int j = 0; j < NC; ++j) {
      float v[EPC];
      r.elems(j, v);
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) t += weight(v[e], M, c);   // -inf weighs 0
      s += (double)t;
    }
    return block_sum<kBlock>(s, L.bs);
  }
  unsigned long long m = wave_chunk_mask<NC>([&](int j) { return r.cmax(j) >= tau; });
  while (m) {
    const int j = pop_low(m);
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
  double wtok;    // weight of the drawn token
};

// Single-pass compaction of the logits >= Lb into the wavefront's own LDS
// region, in ballot order. Chunks no lane of the wavefront can contribute to
// are skipped on their maxima; a wavefront stops once it has more than
// kWaveCap (then the caller takes another route), and does not start when more
// than kWaveCap/4 of its threads hold a candidate: the row then has too many
// for one wavefront unless its candidates are concentrated in this wavefront,
// and the caller's other routes give the same result.
template <int DT, int NC>
__device__ __forceinline__ void wave_compact(const RegRow<DT, NC>& r, float Lb, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int wid = threadIdx.x / kWave;
  int base = 0;
  const int holders = __popcll(__ballot(r.tmax >= Lb));
  if (holders > kWaveCap / 4) {
    base = kWaveCap + 1;
  } else if (holders) {
    unsigned long long m = wave_chunk_mask<NC>([&](int j) { return r.cmax(j) >= Lb; });
    TSR_STAMP(kStMask);
    while (m && base <= kWaveCap) {
      const int j = pop_low(m);
      float v[EPC];
      r.elems(j, v);
      bool hit[EPC];
      int nh = 0;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        hit[e] = v[e] >= Lb;
        nh += hit[e] ? 1 : 0;
      }
      const int ib = r.base(j);
      if (!__any(nh > 1)) {
        // at most one hit per lane (the usual case): the hit by selects, its
        // slot from the ballot of the lanes that hold one; no branch per element
        float hv = v[0];
        int he = 0;
#pragma unroll
        for (int e = 1; e < EPC; ++e) {
          hv = hit[e] ? v[e] : hv;
          he = hit[e] ? e : he;
        }
        const unsigned long long hm = __ballot(nh > 0);
        const int slot = base + (int)__builtin_amdgcn_mbcnt_hi(
                                    (uint32_t)(hm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)hm, 0u));
        if (nh > 0 && slot < kWaveCap) {
          L.wc[wid].val[slot] = __float_as_uint(hv);
          L.wc[wid].idx[slot] = (uint32_t)(ib + he);
        }
        base += __popcll(hm);
        continue;
      }
      // several hits in some lane: per element, the append only for the
      // elements some lane holds
      unsigned long long b[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) b[e] = __ballot(hit[e]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (b[e]) {
          const int nb = base + __popcll(b[e]);
          if (nb <= kWaveCap && hit[e]) {
            const int slot = base + (int)__builtin_amdgcn_mbcnt_hi(
                                        (uint32_t)(b[e] >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)b[e], 0u));
            L.wc[wid].val[slot] = __float_as_uint(v[e]);
            L.wc[wid].idx[slot] = (uint32_t)(ib + e);
          }
          base = nb;
        }
      }
    }
  }
  if (__lane_id() == 0) L.wcnt[wid] = base;
  TSR_STAMP(kStCompactEnd);
}

// Candidates the per-wavefront regions hold in all (after a barrier).
__device__ __forceinline__ int wave_regions_total(const Lds& L) {
  int t = 0;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) t += L.wcnt[q];
  return t;
}

// Top-k candidate bound: for k up to the wavefronts of a workgroup, the k-th
// largest wavefront maximum; else the k-th largest of the per-thread maxima
// (k <= kBlock/4) or of the chunk maxima; each is at most the k-th largest
// logit.
// Found on a linear histogram of [lo, M]: the bound is the lower edge of the
// bin that reaches k (two bin widths down, then checked to fall in a lower
// bin, so it is at most every value of that bin), else, where rounding
// defeats that check, the smallest value in the bin. Returns -inf when fewer
// than k values are >= lo. cleared: the histogram counts are already zero
// (and a barrier has passed since).
template <int DT, int NC>
__device__ __forceinline__ float topk_sketch(const RegRow<DT, NC>& r, float M, float lo,
                                             int k, Lds& L, bool cleared = false) {
  const int tid = threadIdx.x;
  const bool by_thread = k <= kBlock / 4;
  if (k <= kWaves) {
    // the k-th largest of the wavefront maxima (row statistics, in LDS since
    // their barrier): k elements of the row are at least that large, so it
    // bounds the k-th largest logit too, with no pass of its own
    float mw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mw[w] = L.ws[w].m;
    float kth = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      int above = 0;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) above += (mw[v] > mw[w] || (mw[v] == mw[w] && v < w)) ? 1 : 0;
      kth = above == k - 1 ? mw[w] : kth;
    }
    if (kth >= lo) return kth;
  }
  const float span = M - lo;
  const float scale = (span > 0.0f && span <= kFltMax) ? fminf((float)kBins / span, 1e30f) : 0.0f;
  auto sbin = [&](float x) -> int {
    const float t = (M - x) * scale;
    return t < (float)(kBins - 1) ? (int)t : kBins - 1;
  };
  if (!cleared) {
    for (int i = tid; i < kBins; i += kBlock) L.hcnt[i] = 0u;
    __syncthreads();
  }
  if (by_thread) {
    if (r.tmax >= lo) atomicAdd(&L.hcnt[hslot(sbin(r.tmax))], 1u);
  } else {
#pragma nounroll
    for (int j = 0; j < NC; ++j) {
      const float x = r.cmax(j);
      if (x >= lo) atomicAdd(&L.hcnt[hslot(sbin(x))], 1u);
    }
  }
  __syncthreads();
  if (tid < kWave) {
    constexpr int PER = kBins / kWave;
    int hc[PER];
    int lc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      hc[i] = (int)L.hcnt[hslot(tid * PER + i)];
      lc += hc[i];
    }
    const int ic = wave_incl_scan(lc);
    int run = ic - lc;
    int found = kBins;
    if (run < k && ic >= k) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        run += hc[i];
        if (found == kBins && run >= k) found = tid * PER + i;
      }
    }
    found = wave_min(found);
    // the bin's lower edge, where it provably lies below every value of the
    // bin (sbin is monotone: a value of a lower bin is below the whole bin)
    float edge = kNegInf;
    if (found < kBins) {
      edge = fmaxf(M - (float)(found + 2) / scale, lo);
      if (!(edge == lo || sbin(edge) > found)) edge = __builtin_nanf("");
    }
    if (tid == 0) {
      L.si[6] = found;
      L.sf[6] = edge;
      L.su[0] = 0xFFFFFFFFu;
    }
  }
  __syncthreads();
  const int bk = L.si[6];
  const float edge = L.sf[6];
  if (bk >= kBins) return kNegInf;
  if (edge == edge) return edge;
  if (by_thread) {
    if (r.tmax >= lo && sbin(r.tmax) == bk) atomicMin(&L.su[0], fkey(r.tmax));
  } else {
#pragma nounroll
    for (int j = 0; j < NC; ++j) {
      const float x = r.cmax(j);
      if (x >= lo && sbin(x) == bk) atomicMin(&L.su[0], fkey(x));
    }
  }
  __syncthreads();
  const uint32_t kb = L.su[0];
  return kb != 0xFFFFFFFFu ? key2f(kb) : kNegInf;
}

// Candidate bound, compaction and exact resolution (see the file comment).
// zlo is a lower bound of the row's weight sum (JOINT top-p); the exact sum is
// formed here only when the bound cannot settle the cut. u is the uniform.
// MASK: nallow bounds the row's allowed tokens from above.
template <bool MASK = false, int DT, int NC>
__device__ __forceinline__ FastOut fast_cut(const RegRow<DT, NC>& r, int V, float M, float tmin,
                                            double zlo, float c, const Filters& f, double u,
                                            Lds& L, int nallow = 0) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int tid = threadIdx.x;
  FastOut out{0, 0, -1, kPosInf, 0, 0.0, 0.0};
  // In SEQUENTIAL mode top-p measures against the whole top-k set, so min-p
  // may not narrow the candidates there.
  const bool seq_kp = f.seq && f.k_on && f.p_on;
  const bool joint_p = f.p_on && !seq_kp;
  float Lb = seq_kp ? kNegInf : f.tau_m;
  // the whole (finite, allowed) row fits one wavefront: every finite element
  // is a candidate and their sum is Z
  bool all_in = MASK && nallow <= kWaveCap;
  if (all_in || V <= kWaveCap) Lb = -kFltMax;
  bool fits = false, cleared = false;
  if (Lb > kNegInf) {
    // the sketch's histogram counts are cleared under the compaction's barrier
    if (f.k_on)
      for (int i = tid; i < kBins; i += kBlock) L.hcnt[i] = 0u;
    cleared = f.k_on;
    wave_compact(r, Lb, L);
    __syncthreads();
    TSR_STAMP(kStCompact1);
    fits = wave_regions_total(L) <= kWaveCap;
  }
  if (!fits && f.k_on && V > kWaveCap) {
    __syncthreads();
    const float kb = topk_sketch(r, M, fmaxf(Lb, tmin), f.k, L, cleared);
    TSR_STAMP(kStSketch);
    if (kb > Lb) {
      Lb = kb;
      all_in = false;
      wave_compact(r, Lb, L);
      __syncthreads();
      TSR_STAMP(kStCompact2);
      fits = wave_regions_total(L) <= kWaveCap;
    }
  }
  if (!(Lb > kNegInf)) return out;
  out.ok = 1;
  if (fits) {
    double zref = zlo;
    bool zx = !joint_p;
#pragma nounroll
    for (;;) {
      if (tid < kWave) wave_resolve_draw(L, M, c, f, zref, zx, all_in, u);
      __syncthreads();
      if (!L.si[7]) break;
      zref = reg_weight_sum(r, M, c, L);
      zx = true;
    }
    TSR_STAMP(kStResolve);
    out.drawn = 1;
    out.token = L.si[0];
    out.kept = L.si[1];
    out.tau = L.sf[0];
    out.zs = L.sd[1];
    out.wtok = L.sd[2];
    __syncthreads();
    return out;
  }
  // more than one wavefront's worth: count, compact in thread order, sort
  int cnt = 0;
  const unsigned long long cmask = wave_chunk_mask<NC>([&](int j) { return r.cmax(j) >= Lb; });
  unsigned long long m = cmask;
  while (m) {
    const int j = pop_low(m);
    float v[EPC];
    r.elems(j, v);
#pragma unroll
    for (int e = 0; e < EPC; ++e) cnt += (v[e] >= Lb) ? 1 : 0;
  }
  int total;
  int off = block_excl_scan<kBlock>(cnt, &total, L.bs);
  if (total > kCap) {
    out.ok = 0;
    return out;
  }
  m = __any(cnt != 0) ? cmask : 0ull;
  while (m) {
    const int j = pop_low(m);
    float v[EPC];
    r.elems(j, v);
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      if (v[e] >= Lb && off < kCap) L.key[off++] = cand_key(v[e], r.base(j) + e);
  }
  const double Z = joint_p ? reg_weight_sum(r, M, c, L) : 0.0;
  __syncthreads();
  sort_keys_desc(L, total);
  const Resolved res = resolve_sorted(L, total, 0, 0.0, M, c, f, f.p_on ? f.top_p * Z : 0.0,
                                      f.seq);
  out.tau = res.tau;
  out.kept = res.n_in;
  out.zs = res.zs;
  out.token = draw_sorted(L, res.n_in, M, c, u, &out.wtok);
  out.drawn = 1;
  return out;
}

}  // namespace tsr
