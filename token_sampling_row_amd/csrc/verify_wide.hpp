// Speculative verify (spec_verify, tree_verify) for rows wider than two
// register rows per workgroup: 16 < chunks per thread <= 38 (up to 155,648
// bf16 or 77,824 float32 logits per row).
//
// The row kernel takes one target or draft row per workgroup, held in VGPRs,
// and records its status, maximum M, kept set {v >= tau} and kept weight sum
// Z_S, the quantities every later step needs (for greedy verify, the row's
// argmax); a tree node without children, whose draw from its own p~ is
// already known to be needed, draws it there. spec_verify's bonus rows come
// last in the grid and record tau alone. A kept set the candidate bound
// cannot narrow is found on the streaming path, as the sampler does.
//
// spec_verify then takes two more launches. The finish kernel runs one
// workgroup per (sequence, slice of kSliceRows chunk rows): each derives the
// acceptance tests (eq. 39.3) and the first rejection n from the records, and
// sums the residual max(0, p~ - q~) of position n over its slice (every draft
// kept: p~ of the bonus row). The draw kernel (one workgroup per sequence)
// adds the slices' sums in order and draws from the residual (eq. 39.4), or
// the bonus token from p~, inside the slice where the target falls. The
// launch boundaries order the steps: no workgroup waits on another and no
// cross-workgroup fence is needed.
//
// tree_verify's finish takes one workgroup per sequence: it follows the kept
// children from the root and, at a node whose candidates are rejected,
// streams the node's two rows (one pass per rejected candidate for the next
// residual's normaliser, then the draw).
#pragma once

#include "kernels_impl.hpp"

namespace tsr {

// ---------------------------------------------------------------- helpers

// A wave-uniform lane's record.
__device__ __forceinline__ RowRec readlane_rec(const RowRec& r, int l) {
  RowRec o;
  o.zs = readlane_t(r.zs, l);
  o.M = readlane_f32(r.M, l);
  o.tau = readlane_f32(r.tau, l);
  o.status = (int)readlane_u32((uint32_t)r.status, l);
  o.tok = (int)readlane_u32((uint32_t)r.tok, l);
  return o;
}

// A row's quantities as recorded: p~_i = w_i / zs for v_i >= tau, where
// w_i = 2^((v_i - M) c).
__device__ __forceinline__ double rec_p(const RowRec& r, float v, float c) {
  return v >= r.tau ? (double)weight(v, r.M, c) / r.zs : 0.0;
}
// The same through a precomputed 1 / zs (the residual's per-element form).
__device__ __forceinline__ double rec_pi(const RowRec& r, float v, float c, double izs) {
  return v >= r.tau ? (double)weight(v, r.M, c) * izs : 0.0;
}

constexpr int kStreamBatch = 4;   // chunk rows of both rows in flight per thread

// Batched stream of two rows (target p, draft q) of the same layout: calls
// f(jrow, a[EPC], b[EPC]) for every chunk row j0 <= jrow < j1 (< nct) of this
// thread, B chunk rows' loads issued before the first is used.
template <int DT, int B, class F>
__device__ __forceinline__ void stream2(const StreamRow<DT>& sp, const StreamRow<DT>& sq, int j0,
                                        int j1, F&& f) {
  constexpr int EPC = Fmt<DT>::EPC;
#pragma unroll 1
  for (int jb = j0; jb < j1; jb += B) {
    uint4 ta[B], tb[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const bool in = jb + q < j1;
      ta[q] = in ? sp.chunk(jb + q) : neg_inf_chunk<DT>();
      tb[q] = in ? sq.chunk(jb + q) : neg_inf_chunk<DT>();
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      float a[EPC], b[EPC];
      unpack<DT>(ta[q], a);
      unpack<DT>(tb[q], b);
      f(jb + q, a, b);
    }
  }
}

// Inverse-CDF draw in ascending token id over per-element weights of two
// streamed rows, w(a, b) >= 0, restricted to chunk rows [j0, j1) (a float per
// element; a chunk's EPC weights added in float, everything past that in
// double, in a fixed order). The target is u times the range's total
// (ABS false) or u itself (ABS true); the draw is the first element whose
// running total exceeds it, else the last element with weight. Needs
// j1 - j0 <= kWalkBatch. Returns the element (-1: no weight in the range);
// *total_out the range's total weight.
template <int DT, bool ABS, class W>
__device__ __forceinline__ int walk_stream2(const StreamRow<DT>& sp, const StreamRow<DT>& sq,
                                            int j0, int j1, W&& wfn, double u, Lds& L,
                                            double* total_out) {
  constexpr int EPC = Fmt<DT>::EPC;
  const int tid = threadIdx.x, lane = __lane_id(), wid = tid / kWave;
  const int nj = j1 - j0;
  // per chunk row, each 16-lane row's total, in LDS (added in fixed order below)
  stream2<DT, kStreamBatch>(sp, sq, j0, j1, [&](int j, const float* a, const float* b) {
    float sf = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) sf += wfn(a[e], b[e]);
    double s = (double)sf;
    if (__any(s > 0.0)) {
      s += dpp_perm_t<kDppXor1>(s);
      s += dpp_perm_t<kDppXor2>(s);
      s += dpp_perm_t<kDppHalfMirror>(s);
      s += dpp_perm_t<kDppMirror>(s);
    }
    if ((lane & 15) == 0) L.jrow[j - j0][wid * 4 + (lane >> 4)] = s;
  });
  __syncthreads();
  if (tid < kWave) {
    double sj = 0.0;
    if (lane < nj)
#pragma unroll
      for (int q = 0; q < kWaves * 4; ++q) sj += L.jrow[lane][q];
    const double incl = wave_incl_scan(sj);
    const double tot = readlane_t(incl, 63);
    const double target = ABS ? u : u * tot;
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
  const int jstar = j0 + __builtin_amdgcn_readfirstlane(L.si[2]);
  const double r1 = L.sd[2];
  *total_out = L.sd[3];
  float a[EPC], b[EPC], wj[EPC];
  unpack<DT>(sp.chunk(jstar), a);
  unpack<DT>(sq.chunk(jstar), b);
  float minef = 0.0f;   // the same float sum as above
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    wj[e] = wfn(a[e], b[e]);
    minef += wj[e];
  }
  const double mine = (double)minef;
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
    L.si[3] = sp.base(jstar) + pick;
  }
  __syncthreads();
  const int tok = owner >= 0 ? L.si[3] : -1;   // -1: no weight at all
  __syncthreads();
  return tok;
}

// Block-wide sum of w(a, b) over two streamed rows (the same float-then-double
// order as walk_stream2).
template <int DT, class W>
__device__ __forceinline__ double sum_stream2(const StreamRow<DT>& sp, const StreamRow<DT>& sq,
                                              W&& wfn, Lds& L) {
  constexpr int EPC = Fmt<DT>::EPC;
  double acc = 0.0;
  stream2<DT, kStreamBatch>(sp, sq, 0, sp.nct, [&](int, const float* a, const float* b) {
    float sf = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) sf += wfn(a[e], b[e]);
    acc += (double)sf;
  });
  return block_sum<kBlock>(acc, L.bs);
}

// ---------------------------------------------------------------- row kernel

// The rest of a row whose kept set the candidate bound could not narrow, on
// the streaming path (not inlined: the register row is dead by then, so the
// row kernel keeps no registers for it): tau, Z_S and, for a row that draws,
// the token; the record is written to out.
template <int DT>
__device__ __noinline__ void stream_row_rest(const StreamRow<DT> s, float M, const KParams kp,
                                             const Filters f, bool draws, double u, RowRec* out) {
  const Cut cut = general_stream(s, M, -1.0, kp.c, kp.cR, f);
  RowRec rec{0.0, M, cut.tau, 0, -1};
  if (draws) {
    double wt;
    rec.tok = walk_stream(s, cut.tau, M, kp.c, u, &rec.zs, &wt);
  } else {
    rec.zs = cut.zs >= 0.0 ? cut.zs : stream_weight_sum(s, cut.tau, M, kp.c);
  }
  if (threadIdx.x == 0) *out = rec;
}

// One row per workgroup: status, M, tau and Z_S (greedy: status, M and the
// argmax in tok), and where known the row's own draw in tok. TREE: the rows
// of sequence b are its N target rows then its N draft rows (a draft row of a
// node without children, and every draft row at temperature 0, is skipped);
// else its K + 1 target rows then its K draft rows.
template <int DT, int NC, bool TREE>
__global__ __launch_bounds__(kBlock) void verify_rows_kernel(const unsigned char* tgt,
                                                             const unsigned char* dft,
                                                             const int32_t* parent, int K, int V,
                                                             int ragged, KParams kp,
                                                             VerifyWs ws) {
  constexpr int EPC = Fmt<DT>::EPC;
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const int T = TREE ? K : K + 1;            // target rows per sequence (K = N for trees)
  const int D = greedy ? 0 : (TREE ? K : K); // draft rows
  const int R = T + D;
  int b, s;
  if constexpr (TREE) {
    b = (int)blockIdx.x / R;
    s = (int)blockIdx.x - b * R;
  } else {
    // spec_verify: every sequence's K draft positions first, the bonus rows
    // (target row K, the lightest: no kept mass, no draw) last
    const int nseq = (int)gridDim.x / R;
    const int blk = (int)blockIdx.x, nb = nseq * (R - 1);
    if (blk < nb) {
      b = blk / (R - 1);
      const int q = blk - b * (R - 1);
      s = q < K ? q : q + 1;    // targets 0..K-1, then the drafts
    } else {
      b = blk - nb;
      s = K;
    }
  }
  const bool is_t = s < T;
  const int j = is_t ? s : s - T;
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const unsigned char* p = is_t ? tgt + ((long long)b * T + j) * rowbytes
                                : dft + ((long long)b * (TREE ? K : K) + j) * rowbytes;
  bool leaf = false;
  if constexpr (TREE) {
    const int lane = __lane_id();
    const int pa = lane < K ? parent[(long long)b * K + lane] : -2;
    leaf = __ballot(lane < K && lane > 0 && pa == j) == 0ull;
    if (!is_t && leaf) return;      // a node without children: its draft row is not needed
  }
  RowRec* const slot = ws.rec + (long long)b * ws.recs + (is_t ? j : ws.recs / 2 + j);
  RegRow<DT, NC> r;
  r.load(p, V, ragged != 0);
  RowRec rec{0.0, 0.0f, kPosInf, 0, -1};
  const RowStats st = reg_stats(r, !greedy && joint_top_p(kp), kp.c, L);
  rec.status = st.status;
  rec.M = st.M;
  if (greedy) {
    if (st.status == 0) rec.tok = reg_argmax(r, st.M, L);
  } else {
    if (st.status == 0) {
      // a tree node without children draws from its p~ with w1 of (row,
      // node * 32); the other rows need tau and Z_S only, and spec_verify's
      // bonus row tau alone (its draw, when every draft is kept, is the
      // draw kernel's)
      const bool draws = TREE && is_t && leaf;
      const bool need_zs = !(!TREE && j == K);
      const double u = draws ? draw_uniform(kp, (uint32_t)b, (uint32_t)(j * 32), 2u, 1) : 0.0;
      const Filters f = make_filters(kp, st.M);
      const bool filt = f.k_on || f.p_on || f.m_on;
      rec.tau = -kFltMax;   // no filter: every finite logit
      if (filt) {
        // the cut, and for a row that draws, the draw (the register row is
        // dead afterwards)
        const FastOut fo = fast_cut(r, V, st.M, st.tmin, st.zlo, kp.c, f, u, L);
        if (!fo.ok) {
          stream_row_rest<DT>(StreamRow<DT>(p, V), st.M, kp, f, draws, u, slot);
          return;
        }
        rec.tau = fo.tau;
        rec.zs = fo.zs;
        if (draws) rec.tok = fo.token;
      } else if (draws) {
        rec.tok = walk_regs<NC, EPC>(KeptWeights<DT, NC>{r, rec.tau, st.M, kp.c}, u, L, &rec.zs);
      } else if (need_zs) {
        rec.zs = reg_kept_mass(r, rec.tau, st.M, kp.c, L);
      }
    }
  }
  if (threadIdx.x == 0) *slot = rec;
}

// ---------------------------------------------------------------- finish: spec

// Chunk rows per slice of the residual (one batch of loads).
constexpr int kSliceRows = kStreamBatch;
static_assert((38 + kSliceRows - 1) / kSliceRows <= kMaxSlices, "residual slices per row");
// Per sequence, slot of ws.part that holds the rejecting position (or -1).
constexpr int kPartPos = 2 * kMaxSlices - 1;

// One workgroup per (sequence b, slice s of the rows): every workgroup
// derives the sequence's outcome from the records (the acceptance tests of
// eq. 39.3 at each position, the first rejection n) and slice 0 writes the
// outputs. With a rejection at temperature > 0, slice s also sums the
// residual max(0, p~ - q~) of position n (and p~ itself, for a residual
// without mass) over its chunk rows into ws.part; the draw at n is left to
// verify_draw_kernel (the next launch, which sees every slice's sums).
template <int DT>
__global__ __launch_bounds__(kBlock) void verify_finish_kernel(
    const unsigned char* tgt, const unsigned char* dft, const int32_t* xs, int K, int V,
    KParams kp, VerifyWs ws, int32_t* out_tokens, int32_t* out_acc,
    int32_t* out_status) {
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  const int S = (int)gridDim.x / ws.nseq;
  const int b = (int)blockIdx.x / S, sl = (int)blockIdx.x - b * S;
  const int tid = threadIdx.x, lane = __lane_id();
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const RowRec* rt = ws.rec + (long long)b * ws.recs;
  const RowRec* rd = rt + ws.recs / 2;
  if (tid < kWave) {
    // lane q: position q (target row q, draft row q, draft token x_q)
    const bool inq = lane <= K, dq = lane < K;
    const RowRec t = inq ? rt[lane] : RowRec{1.0, 0.0f, kPosInf, 0, -1};
    const RowRec d = (dq && !greedy) ? rd[lane] : RowRec{1.0, 0.0f, kPosInf, 0, -1};
    const int x = dq ? xs[(long long)b * K + lane] : 0;
    const bool x_ok = x >= 0 && x < V;
    const unsigned long long bt = __ballot(inq && t.status != 0), bd = __ballot(dq && d.status != 0);
    const unsigned long long bx = __ballot(dq && !x_ok);
    const int status = bt ? readlane_u32((uint32_t)t.status, __ffsll((long long)bt) - 1)
                       : bd ? readlane_u32((uint32_t)d.status, __ffsll((long long)bd) - 1)
                            : (bx ? 3 : 0);
    bool acc = true;
    if (!status && dq) {
      if (greedy) {
        acc = x == t.tok;
      } else {
        const float lp = load_elem<DT>(tgt + ((long long)b * (K + 1) + lane) * rowbytes, x);
        const float lq = load_elem<DT>(dft + ((long long)b * K + lane) * rowbytes, x);
        const double pt = rec_p(t, lp, kp.c), qt = rec_p(d, lq, kp.c);
        const double a = fmin(1.0, pt / fmax(qt, 1e-300));
        acc = draw_uniform(kp, (uint32_t)b, (uint32_t)lane, 1u, 0) < a;
      }
    }
    const unsigned long long rej = __ballot(dq && !acc);
    const int n = status ? 0 : (rej ? __ffsll((long long)rej) - 1 : K);
    // greedy, or every draft kept: the emitted token is already known
    const int known = (greedy || n == K) ? readlane_u32((uint32_t)t.tok, n) : -1;
    const RowRec tn = readlane_rec(t, n), dn = readlane_rec(d, n);
    if (lane == 0) {
      L.si[0] = status;
      L.si[1] = n;
      L.si[4] = known;
      L.sf[0] = tn.M;
      L.sf[1] = tn.tau;
      L.sd[0] = tn.zs;
      L.sf[2] = dn.M;
      L.sf[3] = dn.tau;
      L.sd[1] = dn.zs;
    }
  }
  __syncthreads();
  const int status = L.si[0], n = L.si[1], tok = L.si[4];
  // a draw left to the draw kernel: the residual at the first rejection, or,
  // every draft kept, the bonus draw from p~ of target row K
  const bool pending = !status && !greedy;
  const bool bonus = n == K;
  unsigned long long* part = ws.part + (long long)b * (2 * kMaxSlices);
  if (sl == 0) {
    // every output but the pending draw's token
    if (tid <= K) {
      const int x = tid < K ? xs[(long long)b * K + tid] : 0;
      if (!(pending && tid == n))
        out_tokens[(long long)b * (K + 1) + tid] =
            status ? -1 : (tid < n ? x : (tid == n ? tok : -1));
    }
    if (tid == 0) {
      out_acc[b] = status ? 0 : n;
      if (out_status) out_status[b] = status;
      part[kPartPos] = pending ? (unsigned long long)n : ~0ull;
    }
  }
  if (!pending) return;
  const RowRec tn{L.sd[0], L.sf[0], L.sf[1], 0, -1}, dn{L.sd[1], L.sf[2], L.sf[3], 0, -1};
  const StreamRow<DT> sp(tgt + ((long long)b * (K + 1) + n) * rowbytes, V);
  const float c = kp.c;
  const int j0 = sl * kSliceRows, j1 = min(j0 + kSliceRows, sp.nct);
  double pr = 0.0, pp = 0.0;
  if (bonus) {
    // p~'s weight of the bonus row only (there is no draft row K)
    stream2<DT, kSliceRows>(sp, sp, j0, j1, [&](int, const float* a, const float*) {
      float fp = 0.0f;
#pragma unroll
      for (int e = 0; e < Fmt<DT>::EPC; ++e) fp += a[e] >= tn.tau ? weight(a[e], tn.M, c) : 0.0f;
      pp += (double)fp;
    });
  } else {
    // this slice's two sums: the residual's and p~'s (unnormalised) weight
    const StreamRow<DT> sq(dft + ((long long)b * K + n) * rowbytes, V);
    const float izp = (float)(1.0 / tn.zs), izq = (float)(1.0 / dn.zs);
    stream2<DT, kSliceRows>(sp, sq, j0, j1, [&](int, const float* a, const float* q) {
      float fr = 0.0f, fp = 0.0f;
#pragma unroll
      for (int e = 0; e < Fmt<DT>::EPC; ++e) {
        fr += residual_weight(a[e], q[e], tn.tau, tn.M, dn.tau, dn.M, c, izp, izq);
        fp += a[e] >= tn.tau ? weight(a[e], tn.M, c) : 0.0f;
      }
      pr += (double)fr;
      pp += (double)fp;
    });
  }
  pr = block_sum<kBlock>(pr, L.bs);
  pp = block_sum<kBlock>(pp, L.bs);
  if (tid == 0) {
    part[2 * sl] = (unsigned long long)__double_as_longlong(pr);
    part[2 * sl + 1] = (unsigned long long)__double_as_longlong(pp);
  }
}

// One workgroup per sequence with a draw pending (ws.part holds its position
// n and, per slice, the residual's and p~'s sums): the slice where u * Z_r
// falls (u from w1 of position n; p~ itself when Z_r = 0), and the draw inside
// it, the token emitted at n (eq. 39.4); n = K (every draft kept): the bonus
// draw from p~ of target row K with w0 of position K.
template <int DT>
__global__ __launch_bounds__(kBlock) void verify_draw_kernel(
    const unsigned char* tgt, const unsigned char* dft, int K, int V, KParams kp,
    VerifyWs ws, int32_t* out_tokens) {
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  const int b = blockIdx.x, tid = threadIdx.x, lane = __lane_id();
  const unsigned long long* part = ws.part + (long long)b * (2 * kMaxSlices);
  const unsigned long long pos = part[kPartPos];
  if (pos == ~0ull) return;
  const int n = (int)pos;
  const bool bonus = n == K;   // every draft kept: p~ of target row K, w0 of position K
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const RowRec tn = ws.rec[(long long)b * ws.recs + n];
  const RowRec dn = bonus ? tn : ws.rec[(long long)b * ws.recs + ws.recs / 2 + n];
  const StreamRow<DT> sp(tgt + ((long long)b * (K + 1) + n) * rowbytes, V);
  const StreamRow<DT> sq = bonus ? sp
                                 : StreamRow<DT>(dft + ((long long)b * K + n) * rowbytes, V);
  const int S = (sp.nct + kSliceRows - 1) / kSliceRows;
  if (tid < kWave) {
    const bool in = lane < S;
    const double r = in ? __longlong_as_double((long long)part[2 * lane]) : 0.0;
    const double q = in ? __longlong_as_double((long long)part[2 * lane + 1]) : 0.0;
    const double ri = wave_incl_scan(r), qi = wave_incl_scan(q);
    const double zr = readlane_t(ri, 63), zq = readlane_t(qi, 63);
    // no residual mass (p~ = q~): the draw is from p~ itself
    const bool use_r = zr > 0.0;
    const double w = use_r ? r : q, wi = use_r ? ri : qi;
    const double uu = bonus ? draw_uniform(kp, (uint32_t)b, (uint32_t)K, 1u, 0)
                            : draw_uniform(kp, (uint32_t)b, (uint32_t)n, 1u, 1);
    const double target = uu * (use_r ? zr : zq);
    const unsigned long long hit = __ballot(w > 0.0 && target < wi);
    const unsigned long long nz = __ballot(w > 0.0);
    const int last = nz ? 63 - __clzll((long long)nz) : 0;
    const int ss = hit ? __ffsll((long long)hit) - 1 : last;
    const double r1 = hit ? target - readlane_t(wi - w, ss) : kPosInf;
    if (lane == 0) {
      L.si[6] = ss;
      L.si[7] = use_r;
      L.sd[4] = r1;
    }
  }
  __syncthreads();
  const int ss = L.si[6];
  const int k0 = ss * kSliceRows, k1 = min(k0 + kSliceRows, sp.nct);
  const double r1 = L.sd[4];
  const float c = kp.c;
  const float izp = (float)(1.0 / tn.zs), izq = (float)(1.0 / dn.zs);
  double zt;
  int tok;
  if (L.si[7])
    tok = walk_stream2<DT, true>(sp, sq, k0, k1, [&](float a, float q) -> float {
      return residual_weight(a, q, tn.tau, tn.M, dn.tau, dn.M, c, izp, izq);
    }, r1, L, &zt);
  else
    tok = walk_stream2<DT, true>(sp, sq, k0, k1, [&](float a, float) -> float {
      return a >= tn.tau ? weight(a, tn.M, c) : 0.0f;
    }, r1, L, &zt);
  if (tid == 0) out_tokens[(long long)b * (K + 1) + n] = tok;
}

// ---------------------------------------------------------------- finish: tree

template <int DT>
__global__ __launch_bounds__(kBlock) void tree_finish_kernel(
    const unsigned char* tgt, const unsigned char* dft, const int32_t* parent,
    const int32_t* tokens, int N, int V, KParams kp, VerifyWs ws,
    int32_t* out_tokens, int32_t* out_path, int32_t* out_acc, int32_t* out_status) {
  Lds& L = tsr_lds;
  TSR_TRACE_INIT(nullptr);
  const int b = blockIdx.x, tid = threadIdx.x, lane = __lane_id();
  const bool greedy = (kp.flags & F_GREEDY) != 0;
  const long long rowbytes = (long long)V * Fmt<DT>::ESZ;
  const RowRec* rt = ws.rec + (long long)b * ws.recs;
  const RowRec* rd = rt + ws.recs / 2;
  const float c = kp.c;
  // the tree, one node per lane (every wavefront reads it)
  const bool ln = lane < N;
  const int pa = ln ? parent[(long long)b * N + lane] : 0;
  const int tk = ln ? tokens[(long long)b * N + lane] : 0;
  const bool bad_tree = __ballot(ln && (lane == 0 ? pa != -1 : (pa < 0 || pa >= lane))) != 0ull;
  const bool bad_tok = __ballot(ln && lane > 0 && (tk < 0 || tk >= V)) != 0ull;
  int status = 0;
  if (bad_tree) {
    status = 5;
  } else {
    const int st_t = ln ? rt[lane].status : 0;
    // a draft row counts only for a node with children (bit v: node v has some)
    unsigned long long kids = 0ull;
#pragma unroll 1
    for (int v = 0; v < N; ++v) kids |= (__ballot(ln && lane > 0 && pa == v) != 0ull) ? 1ull << v : 0ull;
    const bool hc = ln && ((kids >> lane) & 1ull);
    const int st_d = (!greedy && hc) ? rd[lane].status : 0;
    const unsigned long long bt = __ballot(st_t != 0), bd = __ballot(st_d != 0);
    status = bt ? readlane_u32((uint32_t)st_t, __ffsll((long long)bt) - 1)
             : bd ? readlane_u32((uint32_t)st_d, __ffsll((long long)bd) - 1)
                  : (bad_tok ? 3 : 0);
  }
  // follow the kept children from the root; lane q keeps the q-th step's node
  // and token (every lane in step; wave-uniform decisions)
  int n = 0, my_node = -1, my_tok = -1;
  if (!status) {
    int v = 0;
    for (int guard = 0; guard < N; ++guard) {
      const unsigned long long chm = __ballot(ln && lane > 0 && pa == v);
      const RowRec t = rt[v];
      int kept = -1, tok = -1;
      if (greedy) {
        const unsigned long long hit = chm & __ballot(tk == t.tok);
        kept = hit ? __ffsll((long long)hit) - 1 : -1;
        tok = t.tok;
      } else if (!chm) {
        tok = t.tok;               // a leaf: drawn by the row kernel
      } else {
        const RowRec d = rd[v];
        const unsigned char* tp = tgt + ((long long)b * N + v) * rowbytes;
        const unsigned char* dp = dft + ((long long)b * N + v) * rowbytes;
        const StreamRow<DT> sp(tp, V), sq(dp, V);
        const double izp = 1.0 / t.zs, izq = 1.0 / d.zs;
        // p_1 = p~_v; after k rejections p_{k+1} = max(0, p_k - q~) / Z_k (L.tz)
        int k = 0;
        auto pk = [&](double pe, double qe) -> double {
          for (int s2 = 0; s2 < k; ++s2) {
            const double zi = L.tz[s2];
            if (zi > 0.0) pe = fmax(0.0, pe - qe) * zi;
          }
          return pe;
        };
        for (unsigned long long m = chm; m; m &= m - 1ull, ++k) {
          const int child = __ffsll((long long)m) - 1;
          const int x = readlane_u32((uint32_t)tk, child);
          const double pe = rec_pi(t, load_elem<DT>(tp, x), c, izp);
          const double qe = rec_pi(d, load_elem<DT>(dp, x), c, izq);
          const double a = fmin(1.0, pk(pe, qe) / fmax(qe, 1e-300));
          if (draw_uniform(kp, (uint32_t)b, (uint32_t)(v * 32 + k), 2u, 0) < a) {
            kept = child;
            break;
          }
          // rejected: the next residual's normaliser, one streamed pass
          __syncthreads();
          const double z = sum_stream2<DT>(sp, sq, [&](float av, float qv) -> float {
            const double qe2 = rec_pi(d, qv, c, izq);
            return (float)fmax(0.0, pk(rec_pi(t, av, c, izp), qe2) - qe2);
          }, L);
          if (tid == 0) L.tz[k] = z > 0.0 ? 1.0 / z : 0.0;
          __syncthreads();
        }
        if (kept < 0) {
          const double u1 = draw_uniform(kp, (uint32_t)b, (uint32_t)(v * 32), 2u, 1);
          double zt;
          tok = walk_stream2<DT, false>(sp, sq, 0, sp.nct, [&](float av, float qv) -> float {
            return (float)pk(rec_pi(t, av, c, izp), rec_pi(d, qv, c, izq));
          }, u1, L, &zt);
        }
      }
      if (kept < 0) {
        my_tok = lane == n ? tok : my_tok;
        break;
      }
      my_node = lane == n ? kept : my_node;
      my_tok = lane == n ? readlane_u32((uint32_t)tk, kept) : my_tok;
      ++n;
      v = kept;
    }
  }
  if (tid < N) {
    out_tokens[(long long)b * N + tid] = status ? -1 : my_tok;
    out_path[(long long)b * N + tid] = status ? -1 : my_node;
  }
  if (tid == 0) {
    out_acc[b] = status ? 0 : n;
    if (out_status) out_status[b] = status;
  }
}

}  // namespace tsr
