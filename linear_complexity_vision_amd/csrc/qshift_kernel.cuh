// Q-Shift gather kernel and scratch initialisation kernels.
#pragma once

#include "common.cuh"

namespace {

// ---------------------------------------------------------------------------------------------
// Q-Shift gather kernel: out[b, n, c] = X-dagger; bit copies only.
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
                  int H, int W, int C, int s, int g1, int g2, int g3, int g4) {
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
    long long src = r;
    bool ok = true;
    if (c < g1) {
      ok = w >= s;
      src = r - s;
    } else if (c < g2) {
      ok = w < W - s;
      src = r + s;
    } else if (c < g3) {
      ok = h >= s;
      src = r - static_cast<long long>(s) * W;
    } else if (c < g4) {
      ok = h < H - s;
      src = r + static_cast<long long>(s) * W;
    }
    vec_t val{};
    if (ok) val = *reinterpret_cast<const vec_t*>(x + src * C + c);
    *reinterpret_cast<vec_t*>(out + r * C + c) = val;
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
