// Bi-WKV backward: gradients of Eq. (5) with respect to k, v, w and u.
#pragma once

#include "common.h"

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
// The kernels that compute them are in bwd_tile.h; this file holds what the last step of every
// backward call shares: the fold of the per-chunk dw and du terms.

constexpr int kReduceGroups = 16;  // row segments per channel in the dw / du fold

// Per-chunk terms of dw and du: row r (batch item and chunk, in that order), channel c at
// r * C + c.
struct BwdScratch {
  float* pw;  // dw terms (before the factor -lam / T)
  float* pu;  // du terms
};

struct BwdParams {
  const float* w;
  float* dw;
  float* du;
  long long T;
  int B, C, n_chunks;
  int n_wg;  // term rows per batch item
  BwdScratch s;
};

// Per-channel decay in base 2, as the forward kernels form it.
__device__ __forceinline__ float bwd_decay(const BwdParams& p, int c) {
  return (p.w[c] / static_cast<float>(p.T)) * kLog2e;
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
