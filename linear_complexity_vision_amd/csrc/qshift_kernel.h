// Q-Shift gather kernel and scratch initialisation kernels.
#pragma once

#include "common.h"

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
  using t = uint32_t __attribute__((ext_vector_type(4)));  // a native vector (one 16-byte access)
};
template <>
struct Bits<1> {
  using t = uint32_t;
};

// Unsigned division of 0 <= n < 2^31 by a divisor fixed for the launch: a high multiply, an add
// and a shift (Granlund and Montgomery, "Division by invariant integers using multiplication",
// 1994: m = floor(2^32 (2^l - d) / d) + 1 with l = ceil(log2 d), q = (mulhi(m, n) + n) >> l).
struct FastDiv {
  uint32_t d, m, l;
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t t = __umulhi(n, m);
    return static_cast<uint32_t>((static_cast<unsigned long long>(t) + n) >> l);
  }
};
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned long long m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, static_cast<uint32_t>(m), l};
}

// Index of item i (V channels of one token): row r, first channel c, and the token's (h, w).
// Below 2^31 items the divisions are multiply-shifts; beyond, plain 64-bit arithmetic.
struct QsIndex {
  long long r;
  int c, h, w;
};
template <bool BIG>
__device__ __forceinline__ QsIndex qs_index(long long i, FastDiv cv, FastDiv hw, FastDiv wd, int V) {
  QsIndex q;
  if constexpr (BIG) {
    q.r = i / cv.d;
    q.c = static_cast<int>(i - q.r * cv.d) * V;
    const long long t = q.r % hw.d;
    q.h = static_cast<int>(t / wd.d);
    q.w = static_cast<int>(t - static_cast<long long>(q.h) * wd.d);
  } else {
    const uint32_t iu = static_cast<uint32_t>(i);
    const uint32_t r = cv.div(iu);
    q.r = r;
    q.c = static_cast<int>(iu - r * cv.d) * V;
    const uint32_t t = r - hw.div(r) * hw.d;
    const uint32_t h = wd.div(t);
    q.h = static_cast<int>(h);
    q.w = static_cast<int>(t - h * wd.d);
  }
  return q;
}

// Every byte is read or written once: non-temporal loads and stores.
template <class T>
__device__ __forceinline__ T nt_load(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <class T>
__device__ __forceinline__ void nt_store(T v, T* p) {
  __builtin_nontemporal_store(v, p);
}

template <int V, bool BIG>
__global__ void __launch_bounds__(256)
    qshift_kernel(const uint32_t* __restrict__ x, uint32_t* __restrict__ out, long long rows,
                  FastDiv cv, FastDiv hw, FastDiv wd, int H, int W, int C, int s, int g1, int g2,
                  int g3, int g4, int bidir) {
  using vec_t = typename Bits<V>::t;
  const long long n = rows * cv.d;
  for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const QsIndex q = qs_index<BIG>(i, cv, hw, wd, V);
    const long long r = q.r;
    const int c = q.c, h = q.h, w = q.w;
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
    if (ok) val = nt_load(reinterpret_cast<const vec_t*>(x + src * C + c));
    nt_store(val, reinterpret_cast<vec_t*>(out + r * C + c));
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
    using f4 = float __attribute__((ext_vector_type(4)));
    nt_store(f4{d[0], d[1], d[2], d[3]}, reinterpret_cast<f4*>(p));
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) nt_store(d[e], p + e);
  }
}

// ---------------------------------------------------------------------------------------------
// Q-Shift mixing, Eq. (9) as printed: out[j, b, n, c] = x[b, n, c] + (1 - mu[j, c]) * X-dagger[b,
// n, c] for j < n_mix. One pass reads x and its shifted source once and writes every mix (the
// inputs of the R, K, V projections), V consecutive channels per thread.
// ---------------------------------------------------------------------------------------------
template <int V, bool BIG>
__global__ void __launch_bounds__(256)
    qshift_mix_kernel(const float* __restrict__ x, const float* __restrict__ mu,
                      float* __restrict__ out, long long rows, FastDiv cv, FastDiv hw, FastDiv wd,
                      int H, int W, int C, int n_mix, int s, int g1, int g2, int g3, int g4) {
  const long long n = rows * cv.d;
  const long long plane = rows * C;  // elements of one mix
  for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const QsIndex q = qs_index<BIG>(i, cv, hw, wd, V);
    const long long r = q.r;
    const int c = q.c, h = q.h, w = q.w;
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
  c->done = 0u;
  c->epoch = 1u;
  c->fault = 0u;
  c->pad = 0u;
}

}  // namespace
