// Device primitives for the gfx950 sampler: element formats, order keys,
// Philox4x32-10, and wavefront/workgroup reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tsr {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();
constexpr float kFltMax = 3.402823466e+38f;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ formats
// One 16-byte chunk holds 4 float32 or 8 bfloat16 logits.
template <int DT> struct Fmt;
template <> struct Fmt<0> { static constexpr int EPC = 4; static constexpr int ESZ = 4; };
template <> struct Fmt<1> { static constexpr int EPC = 8; static constexpr int ESZ = 2; };

template <int DT>
__device__ __forceinline__ void unpack(const uint4 r, float* v) {
  if constexpr (DT == 0) {
    v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
    v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
  } else {
    // bf16 -> f32 is exact: the bf16 bits are the top half of the f32 bits.
    v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xFFFF0000u);
    v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xFFFF0000u);
    v[4] = __uint_as_float(r.z << 16); v[5] = __uint_as_float(r.z & 0xFFFF0000u);
    v[6] = __uint_as_float(r.w << 16); v[7] = __uint_as_float(r.w & 0xFFFF0000u);
  }
}

// Element-wise load of chunk c of a row (elements [c*EPC, c*EPC+EPC));
// elements at or past V read as -inf. Branch-free: an element past the end
// re-reads element V-1 and is replaced by -inf. Used for the ragged tail of a
// row.
template <int DT>
__device__ __forceinline__ uint4 load_chunk_slow(const unsigned char* row, long long c, int V) {
  constexpr int EPC = Fmt<DT>::EPC;
  const long long e0 = c * EPC;
  const long long last = (long long)V - 1;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (DT == 0) {
      const long long i = e0 + q;
      const uint32_t x = *reinterpret_cast<const uint32_t*>(row + (i < V ? i : last) * 4);
      w[q] = i < V ? x : 0xFF800000u;
    } else {
      const long long i0 = e0 + 2 * q, i1 = i0 + 1;
      const uint32_t lo = *reinterpret_cast<const uint16_t*>(row + (i0 < V ? i0 : last) * 2);
      const uint32_t hi = *reinterpret_cast<const uint16_t*>(row + (i1 < V ? i1 : last) * 2);
      w[q] = (i0 < V ? lo : 0xFF80u) | ((i1 < V ? hi : 0xFF80u) << 16);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DT>
__device__ __forceinline__ uint4 neg_inf_chunk() {
  return DT == 0 ? make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u)
                 : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
}

// A chunk of -inf in global memory: chunks past the end of a row load from
// here, so every chunk of a row is one unconditional 128-bit load.
static __device__ uint4 g_neg_inf_chunk[2] = {
    {0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u},
    {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}};

template <int DT>
__device__ __forceinline__ float load_elem(const unsigned char* row, long long i) {
  if constexpr (DT == 0) return *reinterpret_cast<const float*>(row + i * 4);
  return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(row + i * 2)) << 16);
}

// Keeps the scheduler from interleaving consecutive chunk iterations of an
// unrolled loop over register-resident data; bounded register pressure
// matters more here than instruction-level overlap across chunks.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ------------------------------------------------------------ order keys
// Monotone map float -> uint32 (-0 and +0 share a key; larger float, larger key).
__device__ __forceinline__ uint32_t fkey(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Relative weight of a logit against the row max M: e = 2^((v - M) * c) with
// c = log2(e) / T, i.e. exp((v - M) / T) = p_v / p_max. Every mass in the
// library is a sum of this one expression, so sums formed in different places
// see identical terms.
__device__ __forceinline__ float weight(float v, float M, float c) {
  return __builtin_amdgcn_exp2f((v - M) * c);
}

// ln(a / b) for positive a and b (NaN in, NaN out): the binary exponents
// exactly, the mantissas in [0.5, 1) by the hardware log2 (about 1e-7
// absolute), instead of two double-precision logarithms.
__device__ __forceinline__ float log_ratio(double a, double b) {
  int ea, eb;
  const double ma = frexp(a, &ea), mb = frexp(b, &eb);
  const double l2 = (double)(__builtin_amdgcn_logf((float)ma) - __builtin_amdgcn_logf((float)mb)) +
                    (double)(ea - eb);
  return (float)(l2 * 0.6931471805599453);
}

// ------------------------------------------------------------ Philox4x32-10
// Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten
// rounds of two 32x32->64 products, each high word xored with the other
// counter words and the key, the key advanced by Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo_a = 0xD2511F53u * x.x, hi_a = __umulhi(0xD2511F53u, x.x);
    const uint32_t lo_b = 0xCD9E8D57u * x.z, hi_b = __umulhi(0xCD9E8D57u, x.z);
    x = make_uint4(hi_b ^ x.y ^ k0, lo_b, hi_a ^ x.w ^ k1, lo_a);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return x;
}

// ------------------------------------------------------------ wave ops
// Reductions and scans over the 64 lanes of a wavefront with DPP lane moves
// (a modifier on an ordinary VALU instruction) inside each 16-lane row, and
// v_readlane across rows: no LDS round trips. Every lane gets the same result,
// combined in the same order, so float sums are deterministic.
enum : int {
  kDppXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppQuadMirror = 0x1B,  // quad_perm [3,2,1,0]
  kDppRor4 = 0x124, kDppRor8 = 0x128, kDppRor12 = 0x12C,  // rotate inside a row
  kDppHalfMirror = 0x141,
  kDppMirror = 0x140,
  kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118,
  kDppBcast15 = 0x142, kDppBcast31 = 0x143,
  kDppWaveShr1 = 0x138,  // whole-wave shift by one lane (lane 0 reads zero)
};

template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWMASK, 0xF, false);
}
// A DPP permutation in which every lane reads a valid lane (quad_perm, row
// mirrors, row rotations): no "old" value is needed, so none is materialised.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_perm_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f32(float x) {
  return __uint_as_float(dpp_u32<CTRL, ROWMASK>(__float_as_uint(x)));
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const uint32_t lo = dpp_u32<CTRL, ROWMASK>((uint32_t)x);
  const uint32_t hi = dpp_u32<CTRL, ROWMASK>((uint32_t)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ double dpp_f64(double x) {
  return __longlong_as_double((long long)dpp_u64<CTRL, ROWMASK>((unsigned long long)__double_as_longlong(x)));
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}
__device__ __forceinline__ float readlane_f32(float x, int l) {
  return __uint_as_float(readlane_u32(__float_as_uint(x), l));
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int l) {
  return ((unsigned long long)readlane_u32((uint32_t)(x >> 32), l) << 32) |
         readlane_u32((uint32_t)x, l);
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  return __longlong_as_double((long long)readlane_u64((unsigned long long)__double_as_longlong(x), l));
}

// Lane moves for 32- and 64-bit values.
template <int CTRL, int ROWMASK = 0xF, class T>
__device__ __forceinline__ T dpp_t(T x) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp_u32<CTRL, ROWMASK>(__builtin_bit_cast(uint32_t, x)));
  } else {
    return __builtin_bit_cast(T, dpp_u64<CTRL, ROWMASK>(__builtin_bit_cast(unsigned long long, x)));
  }
}
template <int CTRL, class T>
__device__ __forceinline__ T dpp_perm_t(T x) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp_perm_u32<CTRL>(__builtin_bit_cast(uint32_t, x)));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const uint32_t lo = dpp_perm_u32<CTRL>((uint32_t)u), hi = dpp_perm_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, ((unsigned long long)hi << 32) | lo);
  }
}
template <class T>
__device__ __forceinline__ T readlane_t(T x, int l) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, readlane_u32(__builtin_bit_cast(uint32_t, x), l));
  } else {
    return __builtin_bit_cast(T, readlane_u64(__builtin_bit_cast(unsigned long long, x), l));
  }
}

// Butterfly inside each 16-lane row, then the four row results in fixed order.
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  x = op(x, dpp_perm_t<kDppXor1>(x));
  x = op(x, dpp_perm_t<kDppXor2>(x));
  x = op(x, dpp_perm_t<kDppHalfMirror>(x));
  x = op(x, dpp_perm_t<kDppMirror>(x));
  return op(op(readlane_t(x, 0), readlane_t(x, 16)), op(readlane_t(x, 32), readlane_t(x, 48)));
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float x) {
  return wave_reduce(x, [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ int wave_sum(int x) {
  return wave_reduce(x, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ int wave_min(int x) {
  return wave_reduce(x, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ int wave_max(int x) {
  return wave_reduce(x, [](int a, int b) { return max(a, b); });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return min(a, b); });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return max(a, b); });
}
__device__ __forceinline__ double wave_sum(double x) {
  return wave_reduce(x, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ unsigned long long wave_sum(unsigned long long x) {
  return wave_reduce(x, [](unsigned long long a, unsigned long long b) { return a + b; });
}

// Inclusive scans: shifts by 1, 2, 4, 8 inside rows, then the totals of
// earlier rows broadcast in (row_bcast:15 into rows 1 and 3, row_bcast:31
// into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += (int)dpp_u32<kDppShr1>((uint32_t)x);
  x += (int)dpp_u32<kDppShr2>((uint32_t)x);
  x += (int)dpp_u32<kDppShr4>((uint32_t)x);
  x += (int)dpp_u32<kDppShr8>((uint32_t)x);
  x += (int)dpp_u32<kDppBcast15, 0xA>((uint32_t)x);
  x += (int)dpp_u32<kDppBcast31, 0xC>((uint32_t)x);
  return x;
}
__device__ __forceinline__ double wave_incl_scan(double x) {
  x += dpp_f64<kDppShr1>(x);
  x += dpp_f64<kDppShr2>(x);
  x += dpp_f64<kDppShr4>(x);
  x += dpp_f64<kDppShr8>(x);
  x += dpp_f64<kDppBcast15, 0xA>(x);
  x += dpp_f64<kDppBcast31, 0xC>(x);
  return x;
}
__device__ __forceinline__ unsigned long long wave_incl_scan(unsigned long long x) {
  x += dpp_u64<kDppShr1>(x);
  x += dpp_u64<kDppShr2>(x);
  x += dpp_u64<kDppShr4>(x);
  x += dpp_u64<kDppShr8>(x);
  x += dpp_u64<kDppBcast15, 0xA>(x);
  x += dpp_u64<kDppBcast31, 0xC>(x);
  return x;
}

// Inclusive max-scans (values must be >= 0: lanes outside a DPP source row
// read 0).
__device__ __forceinline__ int wave_incl_max_scan(int x) {
  x = max(x, (int)dpp_u32<kDppShr1>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppShr2>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppShr4>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppShr8>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppBcast15, 0xA>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppBcast31, 0xC>((uint32_t)x));
  return x;
}
__device__ __forceinline__ double wave_incl_max_scan(double x) {
  x = fmax(x, dpp_f64<kDppShr1>(x));
  x = fmax(x, dpp_f64<kDppShr2>(x));
  x = fmax(x, dpp_f64<kDppShr4>(x));
  x = fmax(x, dpp_f64<kDppShr8>(x));
  x = fmax(x, dpp_f64<kDppBcast15, 0xA>(x));
  x = fmax(x, dpp_f64<kDppBcast31, 0xC>(x));
  return x;
}

// The same over the first W lanes only (W = 16: one DPP row, whatever the
// other rows hold; W = 64: the whole wavefront). Where the other rows hold
// the operation's identity the results equal the whole-wavefront ones.
template <int W, class T, class Op>
__device__ __forceinline__ T reduce_w(T x, Op op) {
  static_assert(W == 16 || W == 64, "width");
  if constexpr (W == 64) {
    return wave_reduce(x, op);
  } else {
    x = op(x, dpp_perm_t<kDppXor1>(x));
    x = op(x, dpp_perm_t<kDppXor2>(x));
    x = op(x, dpp_perm_t<kDppHalfMirror>(x));
    x = op(x, dpp_perm_t<kDppMirror>(x));
    return readlane_t(x, 0);
  }
}
template <int W>
__device__ __forceinline__ double sum_w(double x) {
  return reduce_w<W>(x, [](double a, double b) { return a + b; });
}
template <int W>
__device__ __forceinline__ uint32_t min_u32_w(uint32_t x) {
  return reduce_w<W>(x, [](uint32_t a, uint32_t b) { return min(a, b); });
}
template <int W>
__device__ __forceinline__ double incl_scan_w(double x) {
  if constexpr (W == 64) return wave_incl_scan(x);
  x += dpp_f64<kDppShr1>(x);
  x += dpp_f64<kDppShr2>(x);
  x += dpp_f64<kDppShr4>(x);
  x += dpp_f64<kDppShr8>(x);
  return x;
}
template <int W>
__device__ __forceinline__ int incl_max_scan_w(int x) {
  if constexpr (W == 64) return wave_incl_max_scan(x);
  x = max(x, (int)dpp_u32<kDppShr1>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppShr2>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppShr4>((uint32_t)x));
  x = max(x, (int)dpp_u32<kDppShr8>((uint32_t)x));
  return x;
}
template <int W>
__device__ __forceinline__ double incl_max_scan_w(double x) {
  if constexpr (W == 64) return wave_incl_max_scan(x);
  x = fmax(x, dpp_f64<kDppShr1>(x));
  x = fmax(x, dpp_f64<kDppShr2>(x));
  x = fmax(x, dpp_f64<kDppShr4>(x));
  x = fmax(x, dpp_f64<kDppShr8>(x));
  return x;
}

// ------------------------------------------------------------ wave sort
// Value of lane (i ^ D) for D in {1, 2, 4, 8, 16, 32}: DPP inside 16-lane rows,
// ds_swizzle across the two rows of a 32-lane half, ds_bpermute across halves.
template <int D>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  if constexpr (D == 1) {
    return dpp_perm_u32<kDppXor1>(x);
  } else if constexpr (D == 2) {
    return dpp_perm_u32<kDppXor2>(x);
  } else if constexpr (D == 4) {
    const uint32_t dn = dpp_perm_u32<kDppRor4>(x), up = dpp_perm_u32<kDppRor12>(x);
    return (__lane_id() & 4) ? dn : up;
  } else if constexpr (D == 8) {
    return dpp_perm_u32<kDppRor8>(x);
  } else if constexpr (D == 16) {
    // v_permlane16_swap: result 0 holds rows 0, 0, 2, 2 and result 1 rows
    // 1, 1, 3, 3 (16-lane rows), so each lane takes the other row of its pair
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(D == 32, "lane distance");
    // v_permlane32_swap: result 0 holds the low half twice, result 1 the high
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}
// Value of lane (i ^ (S - 1)): the mirror image inside aligned blocks of S lanes.
template <int S>
__device__ __forceinline__ uint32_t lane_mirror(uint32_t x) {
  if constexpr (S == 2) {
    return dpp_perm_u32<kDppXor1>(x);
  } else if constexpr (S == 4) {
    return dpp_perm_u32<kDppQuadMirror>(x);
  } else if constexpr (S == 8) {
    return dpp_perm_u32<kDppHalfMirror>(x);
  } else if constexpr (S == 16) {
    return dpp_perm_u32<kDppMirror>(x);
  } else if constexpr (S == 32) {
    return lane_xor<16>(dpp_perm_u32<kDppMirror>(x));                   // i ^ 15 ^ 16
  } else {
    static_assert(S == 64, "block size");
    return lane_xor<32>(lane_xor<16>(dpp_perm_u32<kDppMirror>(x)));     // i ^ 15 ^ 16 ^ 32
  }
}
// One comparator layer: each lane meets its partner (mirror inside blocks of
// S lanes when MIRROR, else lane ^ S) and the lower lane of the pair keeps the
// larger key.
template <int S, bool MIRROR>
__device__ __forceinline__ unsigned long long cx_layer(unsigned long long x) {
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  uint32_t plo, phi;
  bool low;
  if constexpr (MIRROR) {
    plo = lane_mirror<S>(lo);
    phi = lane_mirror<S>(hi);
    low = (__lane_id() & (S / 2)) == 0;
  } else {
    plo = lane_xor<S>(lo);
    phi = lane_xor<S>(hi);
    low = (__lane_id() & S) == 0;
  }
  const unsigned long long y = ((unsigned long long)phi << 32) | plo;
  return ((x > y) != low) ? y : x;
}
template <int S, bool MIRROR>
__device__ __forceinline__ uint32_t cx_layer(uint32_t x) {
  uint32_t p;
  bool low;
  if constexpr (MIRROR) {
    p = lane_mirror<S>(x);
    low = (__lane_id() & (S / 2)) == 0;
  } else {
    p = lane_xor<S>(x);
    low = (__lane_id() & S) == 0;
  }
  return ((x > p) != low) ? p : x;
}
// Sorts one 32- or 64-bit key per lane into descending lane order inside each aligned
// block of W lanes (W = 16: DPP only; W = 64: the whole wavefront), with the
// bitonic network in its mirror form: every comparator keeps the larger key
// in the lower lane. All 64 lanes must be active.
template <int W, class T>
__device__ __forceinline__ T wave_sort_desc(T x) {
  static_assert(W == 16 || W == 64, "sort width");
  static_assert(sizeof(T) == 8 || sizeof(T) == 4, "32- or 64-bit keys");
  x = cx_layer<2, true>(x);
  x = cx_layer<4, true>(x);
  x = cx_layer<1, false>(x);
  x = cx_layer<8, true>(x);
  x = cx_layer<2, false>(x);
  x = cx_layer<1, false>(x);
  x = cx_layer<16, true>(x);
  x = cx_layer<4, false>(x);
  x = cx_layer<2, false>(x);
  x = cx_layer<1, false>(x);
  if constexpr (W == 64) {
    x = cx_layer<32, true>(x);
    x = cx_layer<8, false>(x);
    x = cx_layer<4, false>(x);
    x = cx_layer<2, false>(x);
    x = cx_layer<1, false>(x);
    x = cx_layer<64, true>(x);
    x = cx_layer<16, false>(x);
    x = cx_layer<8, false>(x);
    x = cx_layer<4, false>(x);
    x = cx_layer<2, false>(x);
    x = cx_layer<1, false>(x);
  }
  return x;
}

// NaN-propagating maxima (IEEE 754-2019 maximum; v_maximum3_f32 on gfx950):
// a NaN anywhere in a row reaches the row maximum, which is how NaN rows are
// detected, with no per-element test.
__device__ __forceinline__ float fmaxn(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmax3n(float a, float b, float c) { return fmaxn(fmaxn(a, b), c); }
__device__ __forceinline__ float wave_maxn(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxn(a, b); });
}

// ------------------------------------------------------------ block ops
// Scratch for block reductions: one slot per wave (at most 16 waves).
struct BlockScratch {
  float f[16];
  int i[16];
  uint32_t u[16];
  double d[16];
  unsigned long long q[16];
};

template <int BLOCK>
__device__ __forceinline__ float block_max(float v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_max(v);
  __syncthreads();
  if (__lane_id() == 0) s.f[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = s.f[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = fmaxf(r, s.f[w]);
  return r;
}
template <int BLOCK>
__device__ __forceinline__ float block_min(float v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_min(v);
  __syncthreads();
  if (__lane_id() == 0) s.f[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = s.f[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = fminf(r, s.f[w]);
  return r;
}
template <int BLOCK>
__device__ __forceinline__ int block_sum(int v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (__lane_id() == 0) s.i[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) r += s.i[w];
  return r;
}
template <int BLOCK>
__device__ __forceinline__ int block_min(int v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_min(v);
  __syncthreads();
  if (__lane_id() == 0) s.i[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = s.i[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = min(r, s.i[w]);
  return r;
}
template <int BLOCK>
__device__ __forceinline__ int block_max(int v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_max(v);
  __syncthreads();
  if (__lane_id() == 0) s.i[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = s.i[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = max(r, s.i[w]);
  return r;
}
template <int BLOCK>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_min_u32(v);
  __syncthreads();
  if (__lane_id() == 0) s.u[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = s.u[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = min(r, s.u[w]);
  return r;
}
template <int BLOCK>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_max_u32(v);
  __syncthreads();
  if (__lane_id() == 0) s.u[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = s.u[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = max(r, s.u[w]);
  return r;
}
// Sum in a fixed order (lanes by butterfly, then waves 0..W-1): deterministic.
template <int BLOCK>
__device__ __forceinline__ double block_sum(double v, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (__lane_id() == 0) s.d[threadIdx.x / kWave] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int w = 0; w < W; ++w) r += s.d[w];
  return r;
}
// Exclusive scan across the block in thread order; *total gets the sum.
template <int BLOCK>
__device__ __forceinline__ int block_excl_scan(int v, int* total, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  const int inc = wave_incl_scan(v);
  __syncthreads();
  if (__lane_id() == kWave - 1) s.i[threadIdx.x / kWave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  const int wid = threadIdx.x / kWave;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int t = s.i[w];
    if (w < wid) before += t;
    all += t;
  }
  *total = all;
  return before + inc - v;
}
template <int BLOCK>
__device__ __forceinline__ double block_excl_scan(double v, double* total, BlockScratch& s) {
  constexpr int W = BLOCK / kWave;
  const double inc = wave_incl_scan(v);
  __syncthreads();
  if (__lane_id() == kWave - 1) s.d[threadIdx.x / kWave] = inc;
  __syncthreads();
  double before = 0.0, all = 0.0;
  const int wid = threadIdx.x / kWave;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const double t = s.d[w];
    if (w < wid) before += t;
    all += t;
  }
  *total = all;
  // exclusive prefix = (earlier waves) + (earlier lanes of this wave)
  return before + dpp_t<kDppWaveShr1>(inc);
}

}  // namespace tsr
