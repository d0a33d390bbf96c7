// Q-Shift gather kernel and scratch initialisation kernels.
#pragma once

#include "common.cuh"

namespace {

// ---------------------------------------------------------------------------------------------
// Q-Shift gather kernel: out[b, n, c] = X-dagger; bit copies only. With bidir set, the shift along
// a sparse token sequence (the host passes a 1 x N grid): the down and up groups then move along
// the sequence too, like the right and left groups.
// ---------------------------------------------------------------------------------------------

template <int V>
struct Bits;
template <>
struct Bits<4> {
  using t = uint4;
};
template <>
struct Bits<1> {
  using t = uint32_t;
};

template <int V>
__global__ void __launch_bounds__(256)
    qshift_kernel(const uint32_t* __restrict__ x, uint32_t* __restrict__ out, long long rows,
                  int H, int W, int C, int s, int g1, int g2, int g3, int g4, int bidir) {
  using vec_t = typename Bits<V>::t;
  const int CV = C / V;
  const long long n = rows * CV;
  const long long HW = static_cast<long long>(H) * W;
  for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long r = i / CV;
    const int c = static_cast<int>(i - r * CV) * V;
    const long long t = r % HW;
    const int h = static_cast<int>(t / W);
    const int w = static_cast<int>(t - static_cast<long long>(h) * W);
    // the vertical groups' coordinate, extent and token step
    const int hv = bidir ? w : h, Hv = bidir ? W : H;
    const long long step = bidir ? 1 : W;
    long long src = r;
    bool ok = true;
    if (c < g1) {
      ok = w >= s;
      src = r - s;
    } else if (c < g2) {
      ok = w < W - s;
      src = r + s;
    } else if (c < g3) {
      ok = hv >= s;
      src = r - s * step;
    } else if (c < g4) {
      ok = hv < Hv - s;
      src = r + s * step;
    }
    vec_t val{};
    if (ok) val = *reinterpret_cast<const vec_t*>(x + src * C + c);
    *reinterpret_cast<vec_t*>(out + r * C + c) = val;
  }
}

// V consecutive floats (V = 4: one 16-byte access) between memory and a register array.
template <int V>
__device__ __forceinline__ void load_floats(float* d, const float* p) {
  if constexpr (V == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    d[0] = q.x;
    d[1] = q.y;
    d[2] = q.z;
    d[3] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) d[e] = p[e];
  }
}
template <int V>
__device__ __forceinline__ void store_floats(float* p, const float* d) {
  if constexpr (V == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(d[0], d[1], d[2], d[3]);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) p[e] = d[e];
  }
}

// ---------------------------------------------------------------------------------------------
// Q-Shift mixing, Eq. (9) as printed: out[j, b, n, c] = x[b, n, c] + (1 - mu[j, c]) * X-dagger[b,
// n, c] for j < n_mix. One pass reads x and its shifted source once and writes every mix (the
// inputs of the R, K, V projections), V consecutive channels per thread.
// ---------------------------------------------------------------------------------------------
template <int V>
__global__ void __launch_bounds__(256)
    qshift_mix_kernel(const float* __restrict__ x, const float* __restrict__ mu,
                      float* __restrict__ out, long long rows, int H, int W, int C, int n_mix,
                      int s, int g1, int g2, int g3, int g4) {
  const int CV = C / V;
  const long long n = rows * CV;
  const long long HW = static_cast<long long>(H) * W;
  const long long plane = rows * C;  // elements of one mix
  for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const long long r = i / CV;
    const int c = static_cast<int>(i - r * CV) * V;
    const long long t = r % HW;
    const int h = static_cast<int>(t / W);
    const int w = static_cast<int>(t - static_cast<long long>(h) * W);
    long long src = r;
    bool ok = true;
    if (c < g1) {  // right
      ok = w >= s;
      src = r - s;
    } else if (c < g2) {  // left
      ok = w < W - s;
      src = r + s;
    } else if (c < g3) {  // down
      ok = h >= s;
      src = r - static_cast<long long>(s) * W;
    } else if (c < g4) {  // up
      ok = h < H - s;
      src = r + static_cast<long long>(s) * W;
    }
    float xv[V], xd[V], m[V], o[V];
    load_floats<V>(xv, x + r * C + c);
    if (ok)
      load_floats<V>(xd, x + src * C + c);
    else
#pragma unroll
      for (int e = 0; e < V; ++e) xd[e] = 0.f;
    for (int j = 0; j < n_mix; ++j) {
      load_floats<V>(m, mu + static_cast<long long>(j) * C + c);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = xv[e] + (1.f - m[e]) * xd[e];
      store_floats<V>(out + j * plane + r * C + c, o);
    }
  }
}

// Zero fill for freshly allocated scratch (a kernel, not a memset, so it is safe to replay).
__global__ void fill_u64_kernel(unsigned long long* p, long long n) {
  for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x)
    p[i] = 0ull;
}

__global__ void init_counters_kernel(Counters* c) {
  c->ticket = 0u;
  c->done = 0u;
  c->epoch = 1u;
  c->fault = 0u;
}

}  // namespace
