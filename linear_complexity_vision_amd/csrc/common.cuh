// Constants, parameter blocks and device helpers shared by the libbiwkv kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "biwkv.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr unsigned kSpinLimit = 1u << 20;  // bounded wait per channel look-back (~1 s)
constexpr unsigned kFaultSpin = 1u;        // fault bit: a bounded wait ran out
constexpr unsigned kFaultTicket = 2u;      // fault bit: a ticket beyond the grid (stale counter)
// Largest decay/growth range (in powers of two) across one wavefront's tokens for which a single
// exponent reference per wavefront keeps every significant term a normal fp32 number. Beyond it
// (|w|/T above ~3 for 16 tokens per wavefront) the wavefront uses per-token references.
constexpr float kFastRange = 64.f;
// Bonus (u log2 e) above which the self weight is formed per token in the wide path.
constexpr float kBonusRange = 60.f;

// Per-(device, stream) counter block. epoch starts at 1 so that zeroed slot words never match.
struct Counters {
  unsigned int ticket;  // next chunk ticket of the running launch
  unsigned int done;    // workgroups finished in the running launch
  unsigned int epoch;   // launch generation, part of every published word's tag
  unsigned int fault;   // sticky fault bits for the host diagnostic
};

struct BiwkvParams {
  const void* k;
  const void* v;
  const void* r;         // gate input (gated entry only)
  const float* w;
  const float* u;
  float* out;
  long long T;           // tokens per sequence
  int C;                 // channels
  int n_tiles;           // channel tiles per batch item
  int n_chunks;          // chunks per (batch, tile) row
  unsigned int total;    // number of workgroups = B * n_tiles * n_chunks
  int H, W, shift;       // Q-Shift grid (fused entry only)
  int g1, g2, g3, g4;    // Q-Shift channel-group bounds (fused entry only)
  int bidir;             // fused entry: shift along the token sequence (W = 1), not the grid
  int group;                  // chunks per exchange group
  int n_groups;               // groups per row
  unsigned long long* agg;    // chunk sums: [row][chunk][dir][tile channel][2 tagged words]
  unsigned long long* gagg;   // group sums: [row][group][dir][tile channel][2 tagged words]
  Counters* ctr;
};

// ---------------------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Storage formats of k and v. raw_t is what one lane loads for its V channels of one token.
template <int DT, int V>
struct KV;

template <>
struct KV<BIWKV_F32, 2> {
  using raw_t = float2;
  static __device__ __forceinline__ raw_t load(const void* base, long long idx) {
    return *reinterpret_cast<const float2*>(static_cast<const float*>(base) + idx);
  }
  static __device__ __forceinline__ raw_t zero() { return make_float2(0.f, 0.f); }
  static __device__ __forceinline__ void unpack(raw_t r, float (&f)[2]) {
    f[0] = r.x;
    f[1] = r.y;
  }
};

template <>
struct KV<BIWKV_F32, 1> {
  using raw_t = float;
  static __device__ __forceinline__ raw_t load(const void* base, long long idx) {
    return static_cast<const float*>(base)[idx];
  }
  static __device__ __forceinline__ raw_t zero() { return 0.f; }
  static __device__ __forceinline__ void unpack(raw_t r, float (&f)[1]) { f[0] = r; }
};

template <>
struct KV<BIWKV_BF16, 2> {
  using raw_t = uint32_t;  // two bf16 values, lower channel in the low half
  static __device__ __forceinline__ raw_t load(const void* base, long long idx) {
    return *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + idx);
  }
  static __device__ __forceinline__ raw_t zero() { return 0u; }
  static __device__ __forceinline__ void unpack(raw_t r, float (&f)[2]) {
    f[0] = __uint_as_float(r << 16);
    f[1] = __uint_as_float(r & 0xffff0000u);
  }
};

template <>
struct KV<BIWKV_BF16, 1> {
  using raw_t = uint32_t;  // one bf16 value in the low half
  static __device__ __forceinline__ raw_t load(const void* base, long long idx) {
    return static_cast<const uint16_t*>(base)[idx];
  }
  static __device__ __forceinline__ raw_t zero() { return 0u; }
  static __device__ __forceinline__ void unpack(raw_t r, float (&f)[1]) {
    f[0] = __uint_as_float(r << 16);
  }
};

template <int V>
__device__ __forceinline__ void store_out(float* out, long long idx, const float (&y)[V]);

template <>
__device__ __forceinline__ void store_out<2>(float* out, long long idx, const float (&y)[2]) {
  *reinterpret_cast<float2*>(out + idx) = make_float2(y[0], y[1]);
}

template <>
__device__ __forceinline__ void store_out<1>(float* out, long long idx, const float (&y)[1]) {
  out[idx] = y[0];
}

// Per-lane (alpha, beta) record of one token: alpha_j then beta_j for the lane's V channels.
template <int V>
struct AlphaBeta;
template <>
struct AlphaBeta<2> {
  using type = float4;
  static __device__ __forceinline__ type make(const float (&a)[2], const float (&b)[2]) {
    return make_float4(a[0], a[1], b[0], b[1]);
  }
  static __device__ __forceinline__ void split(type r, float (&a)[2], float (&b)[2]) {
    a[0] = r.x;
    a[1] = r.y;
    b[0] = r.z;
    b[1] = r.w;
  }
};
template <>
struct AlphaBeta<1> {
  using type = float2;
  static __device__ __forceinline__ type make(const float (&a)[1], const float (&b)[1]) {
    return make_float2(a[0], b[0]);
  }
  static __device__ __forceinline__ void split(type r, float (&a)[1], float (&b)[1]) {
    a[0] = r.x;
    b[0] = r.y;
  }
};

// Q-Shift source of one channel (listing order: groups shift right, left, down, up; the rest is
// copied): the source token is t + off, valid when the column of t lies in [wmin, wmax) and t lies
// in [tmin, tmax); invalid sources read as zero.
struct QShiftLane {
  long long off, tmin, tmax;
  int wmin, wmax;
  __device__ __forceinline__ void init(int ch, int H, int W, long long T, int s, int g1, int g2,
                                       int g3, int g4) {
    off = 0;
    tmin = 0;
    tmax = T;
    wmin = 0;
    wmax = W;
    if (ch < g1) {  // right: out[h, w] = x[h, w - s]
      off = -s;
      wmin = s;
    } else if (ch < g2) {  // left: out[h, w] = x[h, w + s]
      off = s;
      wmax = W - s;
    } else if (ch < g3) {  // down: out[h, w] = x[h - s, w]
      off = -static_cast<long long>(s) * W;
      tmin = static_cast<long long>(s) * W;
    } else if (ch < g4) {  // up: out[h, w] = x[h + s, w]
      off = static_cast<long long>(s) * W;
      tmax = static_cast<long long>(H - s) * W;
    }
  }
  __device__ __forceinline__ bool valid(long long t, int col) const {
    return col >= wmin && col < wmax && t >= tmin && t < tmax;
  }
};

// A decayed partial sum of Eq. (6): value F * 2^m (numerator) and G * 2^m (denominator).
// m == -inf is the empty aggregate (F == G == 0).
struct Agg {
  float m, F, G;
};

__device__ __forceinline__ Agg agg_empty() { return Agg{kNegInf, 0.f, 0.f}; }

// Sum of two aggregates with the same anchor token, rescaled to the larger exponent.
__device__ __forceinline__ Agg agg_add(Agg a, Agg b) {
  if (a.m == kNegInf) return b;
  if (b.m == kNegInf) return a;
  const float m = fmaxf(a.m, b.m);
  const float sa = fast_exp2(a.m - m), sb = fast_exp2(b.m - m);
  return Agg{m, a.F * sa + b.F * sb, a.G * sa + b.G * sb};
}

// Moving the anchor n tokens further away multiplies every term by e^{-n w / T}: in base 2 the
// exponent drops by n * D with D = w * log2(e) / T.
__device__ __forceinline__ Agg agg_shift(Agg a, float steps, float D) {
  a.m -= steps * D;
  return a;
}

// Sums that cross workgroups are stored as two 64-bit words, (l, mu) each tagged with the launch
// epoch in the upper half: l = m + log2(G) is the log-weight and mu = F / G the weighted mean of v.
// A reader accepts a slot only when both tags carry the current epoch, so no fence is needed.
__device__ __forceinline__ void slot_store(unsigned long long* slot, Agg a, unsigned epoch) {
  float l = kNegInf, mu = 0.f;
  if (a.m != kNegInf && a.G > 0.f) {
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  const unsigned long long tag = static_cast<unsigned long long>(epoch) << 32;
  __hip_atomic_store(slot, tag | __float_as_uint(l), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 1, tag | __float_as_uint(mu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void slot_load(const unsigned long long* slot, unsigned long long* w) {
  w[0] = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  w[1] = __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool slot_ready(const unsigned long long* w, unsigned epoch) {
  return static_cast<unsigned>(w[0] >> 32) == epoch && static_cast<unsigned>(w[1] >> 32) == epoch;
}

__device__ __forceinline__ Agg slot_value(const unsigned long long* w) {
  const float l = __uint_as_float(static_cast<unsigned>(w[0]));
  if (l == kNegInf) return agg_empty();
  return Agg{l, __uint_as_float(static_cast<unsigned>(w[1])), 1.f};
}

enum : int { kFwd = 0, kBwd = 1 };

// Slots one thread reads per exchange pass (the host keeps every pass within this bound), and how
// many of them are in flight at once.
constexpr int kMaxSlotsPerThread = 8;
constexpr int kSlotBatch = 4;

}  // namespace
