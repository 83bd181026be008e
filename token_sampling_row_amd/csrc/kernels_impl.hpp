// gfx950 kernel templates of the sampler: greedy argmax, sample_rows, the speculative
// verify step, and the Philox test hook. One workgroup of 1024 threads (16
// wavefronts) per row; the row is held in VGPRs (see row_sampler.hpp).
#pragma once

#include "kernels.hpp"
#include "row_sampler.hpp"

namespace tsr {

constexpr int kBlock = 1024;

template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void greedy_kernel(const unsigned char* logits,
                                                        long long stride_bytes, int V,
                                                        int aligned, int ragged,
                                                        int32_t* out, int32_t* status) {
  __shared__ Lds L;
  const int row = blockIdx.x;
  Row<DT, NC, kBlock> r;
  r.load(logits + (long long)row * stride_bytes, V, aligned != 0, ragged != 0);
  const RowStats st = row_stats(r, false, 1.0f, L);
  int tok = -1;
  if (st.status == 0) tok = row_argmax(r, st.M, L);
  if (threadIdx.x == 0) {
    out[row] = tok;
    if (status) status[row] = st.status;
  }
}

// Weights of the kept set S = {v >= tau} for the walk; chunks whose maximum is
// below tau contribute zeros without any exponential.
template <int DT, int NC>
struct KeptWeights {
  const Row<DT, NC, kBlock>& r;
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

// Count and smallest value of S = {v >= tau} (used when a cut left them open).
template <int DT, int NC>
__device__ __forceinline__ void kept_stats(const Row<DT, NC, kBlock>& r, float tau, Lds& L, int* count,
                           float* vmin) {
  constexpr int EPC = Fmt<DT>::EPC;
  int n = 0;
  float mn = kPosInf;
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
  *count = block_sum<kBlock>(n, L.bs);
  *vmin = block_min<kBlock>(mn, L.bs);
}

template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void sample_kernel(const unsigned char* logits,
                                                        long long stride_bytes, int V,
                                                        int aligned, int ragged, KParams kp,
                                                        int32_t* out, DiagPtrs dg) {
  constexpr int EPC = Fmt<DT>::EPC;
  __shared__ Lds L;
  const int row = blockIdx.x;
  Row<DT, NC, kBlock> r;
  r.load(logits + (long long)row * stride_bytes, V, aligned != 0, ragged != 0);
  if (kp.flags & F_GREEDY) {
    const RowStats st = row_stats(r, false, 1.0f, L);
    int tok = -1;
    if (st.status == 0) tok = row_argmax(r, st.M, L);
    if (threadIdx.x == 0) {
      out[row] = tok;
      if (dg.status) dg.status[row] = st.status;
      if (dg.kept_count) dg.kept_count[row] = 0;
      if (dg.threshold) dg.threshold[row] = kNegInf;
      if (dg.kept_mass) dg.kept_mass[row] = 0.0;
    }
    return;
  }
  const Cut cut = row_cut(r, kp, V, L);
  if (cut.status != 0) {
    if (threadIdx.x == 0) {
      out[row] = -1;
      if (dg.status) dg.status[row] = cut.status;
      if (dg.kept_count) dg.kept_count[row] = 0;
      if (dg.threshold) dg.threshold[row] = kNegInf;
      if (dg.kept_mass) dg.kept_mass[row] = 0.0;
    }
    if (dg.probs) {
      float* pr = dg.probs + (long long)row * V;
      for (int i = threadIdx.x; i < V; i += kBlock) pr[i] = 0.0f;
    }
    return;
  }
  const uint4 w = philox4x32_10(make_uint4((uint32_t)row, 0u, kp.step_lo, kp.step_hi),
                                kp.key0, kp.key1);
  const double u = (double)w.x * 0x1p-32;
  double zs;
  const int tok = walk_draw<NC, EPC, kBlock>(KeptWeights<DT, NC>{r, cut.tau, cut.M, kp.c}, u,
                                             L, &zs);
  int kept = cut.kept;
  float tmin = cut.tau;
  if (dg.kept_count || dg.threshold) kept_stats(r, cut.tau, L, &kept, &tmin);
  if (threadIdx.x == 0) {
    out[row] = tok;
    if (dg.status) dg.status[row] = 0;
    if (dg.kept_count) dg.kept_count[row] = kept;
    if (dg.threshold) dg.threshold[row] = tmin;
    if (dg.kept_mass) dg.kept_mass[row] = cut.z > 0.0 ? zs / cut.z : 0.0;
  }
  if (dg.probs) {
    float* pr = dg.probs + (long long)row * V;
    const double inv = 1.0 / zs;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float v[EPC];
      r.elems(j, v);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int i = r.base(j) + e;
        if (i < V)
          pr[i] = v[e] >= cut.tau ? (float)((double)weight(v[e], cut.M, kp.c) * inv) : 0.0f;
      }
    }
  }
}

// Residual weights max(0, p~ - q~) of one verify position (eq. 39.4), both
// rows resident in this workgroup with the same element layout.
template <int DT, int NC>
struct ResidualWeights {
  const Row<DT, NC, kBlock>& rp;
  const Row<DT, NC, kBlock>& rq;
  float tp, Mp, tq, Mq, c;
  double inv_zp, inv_zq;
  __device__ __forceinline__ void operator()(int j, float* w) const {
    constexpr int EPC = Fmt<DT>::EPC;
    if (rp.cm[j] >= tp) {
      float a[EPC], b[EPC];
      rp.elems(j, a);
      rq.elems(j, b);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const double pe = a[e] >= tp ? (double)weight(a[e], Mp, c) * inv_zp : 0.0;
        const double qe = b[e] >= tq ? (double)weight(b[e], Mq, c) * inv_zq : 0.0;
        const double d = pe - qe;
        w[e] = d > 0.0 ? (float)d : 0.0f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) w[e] = 0.0f;
    }
  }
};

template <int DT, int NC>
__device__ __forceinline__ double kept_mass(const Row<DT, NC, kBlock>& r, float tau, float M, float c, Lds& L) {
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

template <int DT, int NC>
__global__ __launch_bounds__(kBlock) void verify_kernel(const unsigned char* tgt,
                                                        const unsigned char* dft,
                                                        const int32_t* xs, int K, int V,
                                                        int aligned, int ragged, KParams kp,
                                                        VerifyWs ws,
                                                        int32_t* out_tokens,
                                                        int32_t* out_acc,
                                                        int32_t* out_status) {
  constexpr int EPC = Fmt<DT>::EPC;
  __shared__ Lds L;
  const int b = blockIdx.x / (K + 1);
  const int j = blockIdx.x - b * (K + 1);
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const unsigned char* tp = tgt + ((long long)b * (K + 1) + j) * rowbytes;
  const unsigned char* dp = dft + ((long long)b * K + (j < K ? j : 0)) * rowbytes;
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const bool with_draft = !greedy && j < K;
  Row<DT, NC, kBlock> rp, rq;
  rp.load(tp, V, aligned != 0, ragged != 0);
  if (with_draft) rq.load(dp, V, aligned != 0, ragged != 0);
  int st_t = 0, st_d = 0, acc = 0, tok = -1;
  const int x = j < K ? xs[(long long)b * K + j] : 0;
  const bool x_ok = x >= 0 && x < V;
  if (greedy) {
    const RowStats s = row_stats(rp, false, 1.0f, L);
    st_t = s.status;
    if (st_t == 0) {
      tok = row_argmax(rp, s.M, L);
      acc = (j < K && x == tok) ? 1 : 0;
    }
  } else {
    const Cut cp = row_cut(rp, kp, V, L);
    st_t = cp.status;
    const uint4 w = philox4x32_10(make_uint4((uint32_t)b, (uint32_t)j | (1u << 16), kp.step_lo,
                                             kp.step_hi), kp.key0, kp.key1);
    const double u0 = (double)w.x * 0x1p-32;
    const double u1 = (double)w.y * 0x1p-32;
    if (j == K) {
      if (st_t == 0) {
        double zs;
        tok = walk_draw<NC, EPC, kBlock>(KeptWeights<DT, NC>{rp, cp.tau, cp.M, kp.c}, u0, L, &zs);
      }
    } else {
      const Cut cq = row_cut(rq, kp, V, L);
      st_d = cq.status;
      if (st_t == 0 && st_d == 0 && x_ok) {
        const double zp = cp.zs > 0.0 ? cp.zs : kept_mass(rp, cp.tau, cp.M, kp.c, L);
        const double zq = cq.zs > 0.0 ? cq.zs : kept_mass(rq, cq.tau, cq.M, kp.c, L);
        const float lp = load_elem<DT>(tp, x), lq = load_elem<DT>(dp, x);
        const double pt = lp >= cp.tau ? (double)weight(lp, cp.M, kp.c) / zp : 0.0;
        const double qt = lq >= cq.tau ? (double)weight(lq, cq.M, kp.c) / zq : 0.0;
        const double a = fmin(1.0, pt / fmax(qt, 1e-300));
        acc = u0 < a ? 1 : 0;
        if (!acc) {
          double zr;
          tok = walk_draw<NC, EPC, kBlock>(
              ResidualWeights<DT, NC>{rp, rq, cp.tau, cp.M, cq.tau, cq.M, kp.c, 1.0 / zp, 1.0 / zq},
              u1, L, &zr);
          if (!(zr > 0.0)) {
            double zs;
            tok = walk_draw<NC, EPC, kBlock>(KeptWeights<DT, NC>{rp, cp.tau, cp.M, kp.c}, u1, L,
                                             &zs);
          }
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    const int slot = b * ws.kmax1 + j;
    __hip_atomic_store(&ws.acc[slot], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ws.tok[slot], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ws.st_t[slot], st_t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ws.st_d[slot], st_d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t prev = __hip_atomic_fetch_add(&ws.counter[b], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (uint32_t)K) {
      // last of the K+1 workgroups of this sequence: assemble its output
      const int s0 = b * ws.kmax1;
      int status = 0;
      for (int q = 0; q <= K && !status; ++q)
        status = __hip_atomic_load(&ws.st_t[s0 + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int q = 0; q < K && !status; ++q)
        status = __hip_atomic_load(&ws.st_d[s0 + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int q = 0; q < K && !status; ++q) {
        const int xq = xs[(long long)b * K + q];
        if (xq < 0 || xq >= V) status = 3;
      }
      int32_t* o = out_tokens + (long long)b * (K + 1);
      int n = 0;
      if (status) {
        for (int q = 0; q <= K; ++q) o[q] = -1;
      } else {
        while (n < K &&
               __hip_atomic_load(&ws.acc[s0 + n], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          o[n] = xs[(long long)b * K + n];
          ++n;
        }
        o[n] = __hip_atomic_load(&ws.tok[s0 + n], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int q = n + 1; q <= K; ++q) o[q] = -1;
      }
      out_acc[b] = n;
      if (out_status) out_status[b] = status;
      __hip_atomic_store(&ws.counter[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
