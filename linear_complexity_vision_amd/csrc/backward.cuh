// Bi-WKV backward: gradients of Eq. (5) with respect to k, v, w and u.
#pragma once

#include "common.cuh"

namespace {

// ---------------------------------------------------------------------------------------------
// The Vision-RWKV article states that the backward pass of Bi-WKV is again an O(TC) recurrence
// but does not print it; the gradients below follow from Eq. (5). Per (batch, channel) row, with
// the weights p_ti of Eq. (5) (token t attending to token i), the upstream gradient g = dL/dy,
// the denominator D_t of Eq. (5), q_t = g_t / D_t and r_t = q_t y_t:
//   dv_i = e^{k_i} (Qpre_i + Qsuf_i + e^u q_i)
//   dk_i = v_i dv_i - e^{k_i} (Rpre_i + Rsuf_i + e^u r_i)
//   du   = sum_t e^{u + k_t} (q_t v_t - r_t)
//   dw   = -(lam / T) sum_j (b_j Qpre_j - d_j Rpre_j + a_j Qsuf_j - c_j Rsuf_j)
// where lam = e^{-w/T}, Qpre_i = sum_{t<i} lam^{i-1-t} q_t, Qsuf_i = sum_{t>i} lam^{t-i-1} q_t (R
// alike), and a, b, c, d are the four states of Eq. (6) at token j. dw counts |t-i|-1 as the
// number of tokens strictly between t and i and splits lam^{|t-i|-1} at each of them, so every
// sum above is an ordinary decayed prefix or suffix sum.
//
// Work split: a thread owns one chunk of BK tokens of one (batch, channel) row; 64 consecutive
// channels form a wavefront, so every token step of a wavefront moves whole lines.
//
// Position-free sums: a prefix sum anchored at token p, sum_{t<=p} 2^{x_t - (p-t) D} y_t (D =
// w log2(e) / T, x_t the term's own base-2 exponent), is 2^{-p D} sum_{t<=p} 2^{x_t + t D} y_t, and a
// suffix sum anchored at p is 2^{p D} sum_{t>=p} 2^{x_t - t D} y_t. Every term therefore gets its
// exponent x_t + t D (prefix) or x_t - t D (suffix) once, with t D formed exactly from the integer
// t; chunk sums and carries are plain sums, and the anchor enters once, where a sum is used. No
// exponent is moved step by step, so rounding does not accumulate along a row. Every sum is an
// aggregate (m, F, G) = (F, G) * 2^m with a running maximum (agg_add), so any k, w, u and g stay
// finite. Five passes over the row's chunks:
//   1. per chunk, the prefix- and suffix-form sums of (e^k v, e^k);
//   2. carries of those sums into every chunk (two-level scan per row, one workgroup per
//      batch item and 64-channel tile);
//   3. per chunk, y, D, q, r, the chunk's sums of (q, r) and the du terms;
//   4. carries of the (q, r) sums;
//   5. per chunk, the four states and the (q, r) prefix and suffix sums at each token: dk, dv and
//      the dw terms.
// Passes 3 and 5 fold the dw and du terms of a workgroup's chunks in LDS, in a fixed order; a last
// kernel folds those, in a fixed order, into dw and du.
// Scratch: four [6][rows * n_chunks][C] float arrays of sums and carries, two
// [rows * ceil(n_chunks / 4)][C] arrays of per-workgroup dw / du terms.

constexpr int BK = 8;             // tokens per thread chunk
constexpr int kBwdWaves = 4;      // chunks (wavefronts) per workgroup of the per-chunk passes
constexpr int kCarryGroups = 16;  // chunk groups per row in the carry scan
constexpr int kReduceGroups = 16;  // row segments per channel in the dw / du fold

// Scratch arrays are planar: quantity q of chunk j of batch item b, channel c at
// q * plane + (b * n_chunks + j) * C + c.
struct BwdScratch {
  float* a1;   // [6] chunk sums of (e^k v, e^k): forward (anchored at the chunk's last slot), backward
  float* x1;   // [6] carries: forward (anchored just before the chunk), backward (just after it)
  float* a2;   // [6] chunk sums of (q, r)
  float* x2;   // [6] carries of (q, r)
  float* pw;   // dw terms per workgroup (before the factor -lam / T), [rows * n_wg][C]
  float* pu;   // du terms per workgroup, [rows * n_wg][C]
  long long plane;  // rows * n_chunks * C
};

struct BwdParams {
  const void* k;
  const void* v;
  const float* w;
  const float* u;
  const float* g;
  float* dk;
  float* dv;
  float* dw;
  float* du;
  long long T;
  int B, C, n_chunks;
  int n_wg;  // workgroups per row of the per-chunk passes (ceil(n_chunks / kBwdWaves))
  BwdScratch s;
};

__device__ __forceinline__ void agg_put(float* base, long long plane, long long idx, int q0, Agg a) {
  base[(q0 + 0) * plane + idx] = a.m;
  base[(q0 + 1) * plane + idx] = a.F;
  base[(q0 + 2) * plane + idx] = a.G;
}
__device__ __forceinline__ Agg agg_get(const float* base, long long plane, long long idx, int q0) {
  return Agg{base[(q0 + 0) * plane + idx], base[(q0 + 1) * plane + idx], base[(q0 + 2) * plane + idx]};
}

// Per-channel decay in base 2 and bonus, as the forward kernels form them.
__device__ __forceinline__ float bwd_decay(const BwdParams& p, int c) {
  return (p.w[c] / static_cast<float>(p.T)) * kLog2e;
}

template <int DT>
__device__ __forceinline__ float bwd_load(const void* base, long long i) {
  if constexpr (DT == BIWKV_F32) {
    return reinterpret_cast<const float*>(base)[i];
  } else {
    const unsigned short h = reinterpret_cast<const unsigned short*>(base)[i];
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  }
}

// The thread's chunk: batch item b, channel c, chunk j, tokens [t0, t0 + n).
struct BwdLane {
  int b, c, j, n;
  long long t0;
  bool on;
};

__device__ __forceinline__ BwdLane bwd_lane(const BwdParams& p) {
  BwdLane l;
  l.c = blockIdx.x * 64 + (threadIdx.x & 63);
  l.j = blockIdx.y * kBwdWaves + (threadIdx.x >> 6);
  l.b = blockIdx.z;
  l.t0 = static_cast<long long>(l.j) * BK;
  const long long rem = p.T - l.t0;
  l.n = rem <= 0 ? 0 : (rem < BK ? static_cast<int>(rem) : BK);
  l.on = l.c < p.C && l.j < p.n_chunks;
  return l;
}

// Folds one value per thread over the workgroup's wavefronts (its chunks, in order) and writes the
// channel's sum to dst[(b * n_wg + workgroup) * C + c]. Every thread of the workgroup calls it.
__device__ __forceinline__ void bwd_fold_terms(const BwdParams& p, const BwdLane& l, float x, float* dst) {
  __shared__ float part[kBwdWaves][64];
  const int cl = threadIdx.x & 63, wv = threadIdx.x >> 6;
  part[wv][cl] = x;
  __syncthreads();
  if (wv == 0 && l.c < p.C) {
    float sum = part[0][cl];
#pragma unroll
    for (int i = 1; i < kBwdWaves; ++i) sum += part[i][cl];
    dst[(static_cast<long long>(l.b) * p.n_wg + blockIdx.y) * p.C + l.c] = sum;
  }
}

// Pass 1: chunk sums of (e^k v, e^k), prefix form and suffix form.
template <int DT>
__global__ void __launch_bounds__(64 * kBwdWaves) bwd_chunk_sums_kernel(BwdParams p) {
  const BwdLane l = bwd_lane(p);
  if (!l.on) return;
  const float D = bwd_decay(p, l.c);
  const long long row0 = static_cast<long long>(l.b) * p.T * p.C + l.c;
  Agg f = agg_empty(), bk = agg_empty();
#pragma unroll
  for (int i = 0; i < BK; ++i) {
    if (i < l.n) {
      const long long e = row0 + (l.t0 + i) * p.C;
      const float kl = bwd_load<DT>(p.k, e) * kLog2e, v = bwd_load<DT>(p.v, e);
      const float tD = static_cast<float>(l.t0 + i) * D;
      f = agg_add(f, Agg{kl + tD, v, 1.f});
      bk = agg_add(bk, Agg{kl - tD, v, 1.f});
    }
  }
  const long long idx = (static_cast<long long>(l.b) * p.n_chunks + l.j) * p.C + l.c;
  agg_put(p.s.a1, p.s.plane, idx, 0, f);
  agg_put(p.s.a1, p.s.plane, idx, 3, bk);
}

// Passes 2 and 4: carries of position-free chunk sums into every chunk of a row: forward, the sum
// of the prefix-form sums of the earlier chunks; backward, of the suffix-form sums of the later
// ones. One workgroup per (batch item, 64-channel tile): thread (c, grp) folds a contiguous group
// of chunks, one thread per channel folds the group sums, and each thread hands the carries to its
// group's chunks. Fixed order, so the result is reproducible.
__global__ void __launch_bounds__(64 * kCarryGroups)
    bwd_carry_kernel(BwdParams p, const float* __restrict__ sums, float* __restrict__ carries) {
  __shared__ float gs[kCarryGroups][6][64];  // group sums
  __shared__ float gc[kCarryGroups][6][64];  // group carries
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  const int b = blockIdx.y;
  const bool on = c < p.C;
  const int nch = p.n_chunks;
  const int per = (nch + kCarryGroups - 1) / kCarryGroups;
  const int j0 = grp * per, j1 = j0 + per < nch ? j0 + per : nch;
  const long long base = static_cast<long long>(b) * nch * p.C + c;
  const long long plane = p.s.plane;
  Agg f = agg_empty(), bk = agg_empty();
  if (on) {
#pragma unroll 4
    for (int j = j0; j < j1; ++j) f = agg_add(f, agg_get(sums, plane, base + static_cast<long long>(j) * p.C, 0));
#pragma unroll 4
    for (int j = j1 - 1; j >= j0; --j)
      bk = agg_add(agg_get(sums, plane, base + static_cast<long long>(j) * p.C, 3), bk);
  }
  gs[grp][0][cl] = f.m;
  gs[grp][1][cl] = f.F;
  gs[grp][2][cl] = f.G;
  gs[grp][3][cl] = bk.m;
  gs[grp][4][cl] = bk.F;
  gs[grp][5][cl] = bk.G;
  __syncthreads();
  if (grp == 0) {
    Agg x = agg_empty();
    for (int k = 0; k < kCarryGroups; ++k) {
      gc[k][0][cl] = x.m;
      gc[k][1][cl] = x.F;
      gc[k][2][cl] = x.G;
      x = agg_add(x, Agg{gs[k][0][cl], gs[k][1][cl], gs[k][2][cl]});
    }
    Agg y = agg_empty();
    for (int k = kCarryGroups - 1; k >= 0; --k) {
      gc[k][3][cl] = y.m;
      gc[k][4][cl] = y.F;
      gc[k][5][cl] = y.G;
      y = agg_add(Agg{gs[k][3][cl], gs[k][4][cl], gs[k][5][cl]}, y);
    }
  }
  __syncthreads();
  if (!on) return;
  Agg x{gc[grp][0][cl], gc[grp][1][cl], gc[grp][2][cl]};
#pragma unroll 4
  for (int j = j0; j < j1; ++j) {
    const long long at = base + static_cast<long long>(j) * p.C;
    agg_put(carries, plane, at, 0, x);
    x = agg_add(x, agg_get(sums, plane, at, 0));
  }
  Agg y{gc[grp][3][cl], gc[grp][4][cl], gc[grp][5][cl]};
#pragma unroll 4
  for (int j = j1 - 1; j >= j0; --j) {
    const long long at = base + static_cast<long long>(j) * p.C;
    agg_put(carries, plane, at, 3, y);
    y = agg_add(agg_get(sums, plane, at, 3), y);
  }
}

// Re-anchors a position-free prefix-form sum at token p (2^{-p D}) or a suffix-form one.
__device__ __forceinline__ Agg at_prefix(Agg a, long long p, float D) {
  a.m -= static_cast<float>(p) * D;
  return a;
}
__device__ __forceinline__ Agg at_suffix(Agg a, long long p, float D) {
  a.m += static_cast<float>(p) * D;
  return a;
}

// The chunk's tokens and, per token, the position-free sums of (e^k v, e^k) over the earlier
// tokens (pre) and the later ones (suf), and y, log2 D and g of each token. Shared by passes 3
// and 5.
template <int DT>
struct BwdChunk {
  float kl[BK], v[BK], g[BK];  // k log2(e), v, g (padded slots: k = -inf)
  Agg pre[BK];                 // prefix form, tokens before i
  Agg suf[BK];                 // suffix form, tokens after i
  float y[BK], lD[BK];         // output and log2 of Eq. (5)'s denominator (0 in padded slots)

  __device__ __forceinline__ void run(const BwdParams& p, const BwdLane& l, float D, float U) {
    const long long row0 = static_cast<long long>(l.b) * p.T * p.C + l.c;
#pragma unroll
    for (int i = 0; i < BK; ++i) {
      if (i < l.n) {
        const long long e = row0 + (l.t0 + i) * p.C;
        kl[i] = bwd_load<DT>(p.k, e) * kLog2e;
        v[i] = bwd_load<DT>(p.v, e);
        g[i] = p.g[e];
      } else {
        kl[i] = kNegInf;
        v[i] = 0.f;
        g[i] = 0.f;
      }
    }
    const long long idx = (static_cast<long long>(l.b) * p.n_chunks + l.j) * p.C + l.c;
    Agg x = agg_get(p.s.x1, p.s.plane, idx, 0), yb = agg_get(p.s.x1, p.s.plane, idx, 3);
#pragma unroll
    for (int i = 0; i < BK; ++i) {
      pre[i] = x;
      x = agg_add(x, Agg{kl[i] + static_cast<float>(l.t0 + i) * D, v[i], 1.f});
    }
#pragma unroll
    for (int i = BK - 1; i >= 0; --i) {
      suf[i] = yb;
      yb = agg_add(Agg{kl[i] - static_cast<float>(l.t0 + i) * D, v[i], 1.f}, yb);
    }
#pragma unroll
    for (int i = 0; i < BK; ++i) {
      const long long t = l.t0 + i;
      // Eq. (7): (a + b + e^{u+k} v) / (c + d + e^{u+k}), a, c anchored at t - 1, b, d at t + 1
      const Agg tot = agg_add(agg_add(at_prefix(pre[i], t - 1, D), at_suffix(suf[i], t + 1, D)),
                              Agg{kl[i] + U, v[i], 1.f});
      const bool ok = i < l.n && tot.G > 0.f;
      y[i] = ok ? tot.F / tot.G : 0.f;
      lD[i] = ok ? tot.m + fast_log2(tot.G) : 0.f;
    }
  }
  // (q, r) = (g, g y) 2^{-log2 D} of token i, position-free in prefix or suffix form
  __device__ __forceinline__ Agg qr_prefix(int i, long long t, float D) const {
    return i < BK && kl[i] != kNegInf ? Agg{-lD[i] + static_cast<float>(t) * D, g[i], g[i] * y[i]} : agg_empty();
  }
  __device__ __forceinline__ Agg qr_suffix(int i, long long t, float D) const {
    return i < BK && kl[i] != kNegInf ? Agg{-lD[i] - static_cast<float>(t) * D, g[i], g[i] * y[i]} : agg_empty();
  }
};

// Pass 3: position-free chunk sums of (q, r) and the du terms.
template <int DT>
__device__ __forceinline__ float bwd_sweep1(const BwdParams& p, const BwdLane& l) {
  const float D = bwd_decay(p, l.c), U = p.u[l.c] * kLog2e;
  BwdChunk<DT> ch;
  ch.run(p, l, D, U);
  Agg f = agg_empty(), bk = agg_empty();
  float du = 0.f;
#pragma unroll
  for (int i = 0; i < BK; ++i) {
    if (i < l.n) {
      const long long t = l.t0 + i;
      f = agg_add(f, ch.qr_prefix(i, t, D));
      bk = agg_add(bk, ch.qr_suffix(i, t, D));
      // e^{u+k} (q v - r) = p_tt g (v - y)
      du = fmaf(fast_exp2(U + ch.kl[i] - ch.lD[i]) * ch.g[i], ch.v[i] - ch.y[i], du);
    }
  }
  const long long idx = (static_cast<long long>(l.b) * p.n_chunks + l.j) * p.C + l.c;
  agg_put(p.s.a2, p.s.plane, idx, 0, f);
  agg_put(p.s.a2, p.s.plane, idx, 3, bk);
  return du;
}

template <int DT>
__global__ void __launch_bounds__(64 * kBwdWaves) bwd_sweep1_kernel(BwdParams p) {
  const BwdLane l = bwd_lane(p);
  const float du = l.on ? bwd_sweep1<DT>(p, l) : 0.f;
  bwd_fold_terms(p, l, du, p.s.pu);
}

// Pass 5: dk, dv and the dw terms.
template <int DT>
__device__ __forceinline__ float bwd_sweep2(const BwdParams& p, const BwdLane& l) {
  const float D = bwd_decay(p, l.c), U = p.u[l.c] * kLog2e;
  BwdChunk<DT> ch;
  ch.run(p, l, D, U);
  const long long idx = (static_cast<long long>(l.b) * p.n_chunks + l.j) * p.C + l.c;
  // position-free (q, r) sums over the later tokens of each slot, then over the earlier ones
  Agg qs[BK];
  Agg ys = agg_get(p.s.x2, p.s.plane, idx, 3);
#pragma unroll
  for (int i = BK - 1; i >= 0; --i) {
    qs[i] = ys;
    if (i < l.n) ys = agg_add(ch.qr_suffix(i, l.t0 + i, D), ys);
  }
  Agg xq = agg_get(p.s.x2, p.s.plane, idx, 0);
  float dw = 0.f;
  const long long row0 = static_cast<long long>(l.b) * p.T * p.C + l.c;
#pragma unroll
  for (int i = 0; i < BK; ++i) {
    if (i < l.n) {
      const long long t = l.t0 + i;
      // Qpre (anchored at t - 1) + Qsuf (at t + 1) + e^u q, and the same for r; times e^{k_t}
      const Agg self{U - ch.lD[i], ch.g[i], ch.g[i] * ch.y[i]};
      const Agg s = agg_add(agg_add(at_prefix(xq, t - 1, D), at_suffix(qs[i], t + 1, D)), self);
      const float sc = s.m == kNegInf ? 0.f : fast_exp2(s.m + ch.kl[i]);
      const float dv = s.F * sc;
      const float dk = fmaf(ch.v[i], dv, -s.G * sc);
      const long long e = row0 + t * p.C;
      p.dv[e] = dv;
      p.dk[e] = dk;
      // b Qpre - d Rpre + a Qsuf - c Rsuf at token t: the anchors t + 1 and t - 1 leave 2^{2D}
      const Agg& bd = ch.suf[i];
      const Agg& ac = ch.pre[i];
      if (bd.m != kNegInf && xq.m != kNegInf)
        dw += (bd.F * xq.F - bd.G * xq.G) * fast_exp2(bd.m + xq.m + 2.f * D);
      if (ac.m != kNegInf && qs[i].m != kNegInf)
        dw += (ac.F * qs[i].F - ac.G * qs[i].G) * fast_exp2(ac.m + qs[i].m + 2.f * D);
      xq = agg_add(xq, ch.qr_prefix(i, t, D));
    }
  }
  return dw;
}

template <int DT>
__global__ void __launch_bounds__(64 * kBwdWaves) bwd_sweep2_kernel(BwdParams p) {
  const BwdLane l = bwd_lane(p);
  const float dw = l.on ? bwd_sweep2<DT>(p, l) : 0.f;
  bwd_fold_terms(p, l, dw, p.s.pw);
}

// dw = du = 0 for an empty sequence (nothing to sum).
__global__ void bwd_zero_kernel(float* dw, float* du, int C) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c < C) dw[c] = du[c] = 0.f;
}

// dw and du: fold the per-workgroup terms in batch and workgroup order. Thread (c, grp) of a
// workgroup of 64 channels sums a contiguous segment of the rows; the segments are then added in
// order.
__global__ void __launch_bounds__(64 * kReduceGroups) bwd_reduce_kernel(BwdParams p) {
  __shared__ float pw[kReduceGroups][64], pu[kReduceGroups][64];
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  const long long n = static_cast<long long>(p.B) * p.n_wg;
  const long long per = (n + kReduceGroups - 1) / kReduceGroups;
  const long long r0 = grp * per, r1 = r0 + per < n ? r0 + per : n;
  float sw = 0.f, su = 0.f;
  if (c < p.C) {
#pragma unroll 8
    for (long long r = r0; r < r1; ++r) {
      sw += p.s.pw[r * p.C + c];
      su += p.s.pu[r * p.C + c];
    }
  }
  pw[grp][cl] = sw;
  pu[grp][cl] = su;
  __syncthreads();
  if (grp != 0 || c >= p.C) return;
  sw = 0.f;
  su = 0.f;
  for (int i = 0; i < kReduceGroups; ++i) {
    sw += pw[i][cl];
    su += pu[i][cl];
  }
  const float D = bwd_decay(p, c);
  p.dw[c] = -(fast_exp2(-D) / static_cast<float>(p.T)) * sw;
  p.du[c] = su;
}

}  // namespace
