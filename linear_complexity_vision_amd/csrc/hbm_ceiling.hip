// hbm_ceiling — streaming kernels that move exactly the bytes of a Bi-WKV forward call and do
// nothing else, for measuring what HBM delivers to such a byte mix on this device.
//
// A Bi-WKV forward call (Eq. (5) of "OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV Backbone",
// section "Linear Complexity Bidirectional Attention") reads k and v once (bf16 or fp32) and
// writes one fp32 output per element. The kernels here read the same two arrays and write the
// same output with out = k + v, so their duration is a measured ceiling for any kernel with that
// byte mix: the fraction of it that the Bi-WKV kernel reaches says how much of the gap to the
// published peak is the memory system's and how much the kernel's.
//
// Modes: 0 = read k, v and write out (the forward's mix); 1 = read k and v only; 2 = write out
// only. Each thread moves 16-byte pieces (8 bf16 or 4 fp32 elements of k and of v), or 8-byte
// pieces with policy bit 2 (4 bf16 elements and one 16-byte store, or 2 fp32 elements), U pieces
// per loop trip with every load issued before the first store, in a grid-stride loop over
// `blocks` workgroups. Cache policy: bit 0 non-temporal loads, bit 1 non-temporal stores.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "hbm_ceiling.h"

namespace {

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using f32x4 = float __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}
template <bool NT>
__device__ __forceinline__ void st(f32x4 v, f32x4* p) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One piece: 16 bytes of k and of v. bf16 pieces hold 8 elements (32 bytes of output), fp32
// pieces 4 (16 bytes).
template <int DT, int U, bool NTL, bool NTS, int MODE>
__global__ void __launch_bounds__(256) stream_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                     f32x4* __restrict__ out, long long pieces) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  long long i0 = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i0 < pieces; i0 += stride * U) {
    u32x4 a[U], b[U];
    if constexpr (MODE != 2) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const long long i = i0 + j * stride;
        if (i < pieces) {
          a[j] = ld<NTL>(k + i);
          b[j] = ld<NTL>(v + i);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long long i = i0 + j * stride;
      if (i >= pieces) break;
      if constexpr (MODE == 1) {
        acc ^= a[j].x ^ a[j].y ^ a[j].z ^ a[j].w ^ b[j].x ^ b[j].y ^ b[j].z ^ b[j].w;
      } else if constexpr (MODE == 2) {
        const float f = static_cast<float>(i);
        if constexpr (DT == HBM_BF16) {
          st<NTS>(f32x4{f, f, f, f}, out + 2 * i);
          st<NTS>(f32x4{f, f, f, f}, out + 2 * i + 1);
        } else {
          st<NTS>(f32x4{f, f, f, f}, out + i);
        }
      } else if constexpr (DT == HBM_BF16) {
        const u32x4 p = a[j], q = b[j];
        st<NTS>(f32x4{bf_lo(p.x) + bf_lo(q.x), bf_hi(p.x) + bf_hi(q.x), bf_lo(p.y) + bf_lo(q.y),
                      bf_hi(p.y) + bf_hi(q.y)},
                out + 2 * i);
        st<NTS>(f32x4{bf_lo(p.z) + bf_lo(q.z), bf_hi(p.z) + bf_hi(q.z), bf_lo(p.w) + bf_lo(q.w),
                      bf_hi(p.w) + bf_hi(q.w)},
                out + 2 * i + 1);
      } else {
        const u32x4 p = a[j], q = b[j];
        st<NTS>(f32x4{__uint_as_float(p.x) + __uint_as_float(q.x), __uint_as_float(p.y) + __uint_as_float(q.y),
                      __uint_as_float(p.z) + __uint_as_float(q.z), __uint_as_float(p.w) + __uint_as_float(q.w)},
                out + i);
      }
    }
  }
  if constexpr (MODE == 1) {
    // keeps the loads alive; the xor of random data is this value with probability 2^-32, and
    // then one 16-byte word of out is written
    if (acc == 0x9e3779b9u) out[0] = f32x4{1.f, 1.f, 1.f, 1.f};
  }
}

// 8-byte pieces: 4 bf16 elements (one 16-byte store) or 2 fp32 elements (one 8-byte store)
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
using f32x2 = float __attribute__((ext_vector_type(2)));
template <int DT, int U, bool NTL, bool NTS, int MODE>
__global__ void __launch_bounds__(256) stream_kernel_narrow(const u32x2* __restrict__ k, const u32x2* __restrict__ v,
                                                            float* __restrict__ out, long long pieces) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  long long i0 = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i0 < pieces; i0 += stride * U) {
    u32x2 a[U], b[U];
    if constexpr (MODE != 2) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const long long i = i0 + j * stride;
        if (i < pieces) {
          a[j] = NTL ? __builtin_nontemporal_load(k + i) : k[i];
          b[j] = NTL ? __builtin_nontemporal_load(v + i) : v[i];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long long i = i0 + j * stride;
      if (i >= pieces) break;
      if constexpr (MODE == 1) {
        acc ^= a[j].x ^ a[j].y ^ b[j].x ^ b[j].y;
      } else if constexpr (DT == HBM_BF16) {
        f32x4 o;
        if constexpr (MODE == 2) {
          const float f = static_cast<float>(i);
          o = f32x4{f, f, f, f};
        } else {
          o = f32x4{bf_lo(a[j].x) + bf_lo(b[j].x), bf_hi(a[j].x) + bf_hi(b[j].x), bf_lo(a[j].y) + bf_lo(b[j].y),
                    bf_hi(a[j].y) + bf_hi(b[j].y)};
        }
        st<NTS>(o, reinterpret_cast<f32x4*>(out) + i);
      } else {
        f32x2 o;
        if constexpr (MODE == 2) {
          const float f = static_cast<float>(i);
          o = f32x2{f, f};
        } else {
          o = f32x2{__uint_as_float(a[j].x) + __uint_as_float(b[j].x), __uint_as_float(a[j].y) + __uint_as_float(b[j].y)};
        }
        f32x2* q = reinterpret_cast<f32x2*>(out) + i;
        if constexpr (NTS)
          __builtin_nontemporal_store(o, q);
        else
          *q = o;
      }
    }
  }
  if constexpr (MODE == 1) {
    if (acc == 0x9e3779b9u) out[0] = 1.f;  // keeps the loads alive (see stream_kernel)
  }
}

template <int DT, int U, bool NTL, bool NTS>
void launch_mode(int mode, dim3 grid, hipStream_t st, const u32x4* k, const u32x4* v, f32x4* out,
                 long long pieces) {
  if (mode == 0)
    hipLaunchKernelGGL((stream_kernel<DT, U, NTL, NTS, 0>), grid, dim3(256), 0, st, k, v, out, pieces);
  else if (mode == 1)
    hipLaunchKernelGGL((stream_kernel<DT, U, NTL, NTS, 1>), grid, dim3(256), 0, st, k, v, out, pieces);
  else
    hipLaunchKernelGGL((stream_kernel<DT, U, NTL, NTS, 2>), grid, dim3(256), 0, st, k, v, out, pieces);
}

template <int DT, int U, bool NTL, bool NTS>
void launch_mode_narrow(int mode, dim3 grid, hipStream_t st, const u32x2* k, const u32x2* v, float* out,
                        long long pieces) {
  if (mode == 0)
    hipLaunchKernelGGL((stream_kernel_narrow<DT, U, NTL, NTS, 0>), grid, dim3(256), 0, st, k, v, out, pieces);
  else if (mode == 1)
    hipLaunchKernelGGL((stream_kernel_narrow<DT, U, NTL, NTS, 1>), grid, dim3(256), 0, st, k, v, out, pieces);
  else
    hipLaunchKernelGGL((stream_kernel_narrow<DT, U, NTL, NTS, 2>), grid, dim3(256), 0, st, k, v, out, pieces);
}
template <int DT, int U>
void launch_policy(int mode, int policy, dim3 grid, hipStream_t st, const u32x4* k, const u32x4* v, f32x4* out,
                   long long pieces) {
  if (policy & 4) {
    const auto* k2 = reinterpret_cast<const u32x2*>(k);
    const auto* v2 = reinterpret_cast<const u32x2*>(v);
    auto* o = reinterpret_cast<float*>(out);
    switch (policy & 3) {
      case 0: launch_mode_narrow<DT, U, false, false>(mode, grid, st, k2, v2, o, pieces); break;
      case 1: launch_mode_narrow<DT, U, true, false>(mode, grid, st, k2, v2, o, pieces); break;
      case 2: launch_mode_narrow<DT, U, false, true>(mode, grid, st, k2, v2, o, pieces); break;
      default: launch_mode_narrow<DT, U, true, true>(mode, grid, st, k2, v2, o, pieces); break;
    }
    return;
  }
  switch (policy) {
    case 0: launch_mode<DT, U, false, false>(mode, grid, st, k, v, out, pieces); break;
    case 1: launch_mode<DT, U, true, false>(mode, grid, st, k, v, out, pieces); break;
    case 2: launch_mode<DT, U, false, true>(mode, grid, st, k, v, out, pieces); break;
    default: launch_mode<DT, U, true, true>(mode, grid, st, k, v, out, pieces); break;
  }
}

template <int DT>
void launch_unroll(int mode, int unroll, int policy, dim3 grid, hipStream_t st, const u32x4* k, const u32x4* v,
                   f32x4* out, long long pieces) {
  switch (unroll) {
    case 1: launch_policy<DT, 1>(mode, policy, grid, st, k, v, out, pieces); break;
    case 2: launch_policy<DT, 2>(mode, policy, grid, st, k, v, out, pieces); break;
    case 4: launch_policy<DT, 4>(mode, policy, grid, st, k, v, out, pieces); break;
    default: launch_policy<DT, 8>(mode, policy, grid, st, k, v, out, pieces); break;
  }
}

}  // namespace

extern "C" {

int hbm_stream(const void* k, const void* v, float* out, int64_t n, int dtype, int mode, int blocks,
               int unroll, int policy, void* stream) {
  if (n < 0 || blocks < 0) return HBM_ERR_ARG;
  if (dtype != HBM_F32 && dtype != HBM_BF16) return HBM_ERR_ARG;
  if (mode < 0 || mode > 2 || policy < 0 || policy > 7) return HBM_ERR_ARG;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return HBM_ERR_ARG;
  const int per_piece = (dtype == HBM_BF16 ? 8 : 4) / ((policy & 4) ? 2 : 1);
  if (n % per_piece != 0) return HBM_ERR_ARG;
  if (n == 0) return HBM_OK;
  if (!k || !v || !out) return HBM_ERR_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                        reinterpret_cast<uintptr_t>(out);
  if (mis % 16 != 0) return HBM_ERR_ARG;
  const long long pieces = n / per_piece;
  long long grid = blocks;
  const long long cover = (pieces + 255) / 256;  // one piece per thread
  if (grid == 0 || grid > cover) grid = cover;
  if (grid > 0x7fffffffll) return HBM_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const auto* kp = static_cast<const u32x4*>(k);
  const auto* vp = static_cast<const u32x4*>(v);
  auto* op = reinterpret_cast<f32x4*>(out);
  const dim3 g(static_cast<unsigned>(grid));
  if (dtype == HBM_BF16)
    launch_unroll<HBM_BF16>(mode, unroll, policy, g, st, kp, vp, op, pieces);
  else
    launch_unroll<HBM_F32>(mode, unroll, policy, g, st, kp, vp, op, pieces);
  return hipGetLastError() == hipSuccess ? HBM_OK : HBM_ERR_HIP;
}

}  // extern "C"
