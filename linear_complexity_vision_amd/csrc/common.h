// Constants, parameter blocks and device helpers shared by the libbiwkv kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "biwkv.h"

// Types shared by the translation units of the library (they appear in its internal
// interfaces, so they have external linkage).

// Counter block of the single-pass exchange (per (device, stream), or the allocation-free
// entry's static one). Slots are tagged with epoch + 1, so an all-zero block is a valid start.
struct Counters {
  unsigned int done;   // workgroups finished in the running launch
  unsigned int epoch;  // launch generation, part of every published word's tag
  unsigned int fault;  // sticky bits for the host diagnostic (kFaultSpin)
  unsigned int pad;
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
  int H, W, shift;       // Q-Shift grid (fused entry only)
  int g1, g2, g3, g4;    // Q-Shift channel-group bounds (fused entry only)
  int bidir;             // fused entry: shift along the token sequence (W = 1), not the grid
};

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
// Polls of a peer chunk's slot before a waiting workgroup recomputes that chunk's sums itself
// (each poll is a round trip to memory, about a microsecond under load): far above what an
// exchange between resident workgroups takes, far below a stall.
constexpr unsigned kSpinDefault = 1u << 12;
constexpr unsigned kFaultSpin = 1u;  // fault-word bit: a wait ran out and a peer's sums were recomputed
// Largest decay/growth range (in powers of two) across one wavefront's tokens for which a single
// exponent reference per wavefront keeps every significant term a normal fp32 number. Beyond it
// (|w|/T above ~3 for 16 tokens per wavefront) the wavefront uses per-token references.
constexpr float kFastRange = 64.f;
// Bonus (u log2 e) above which the self weight is formed per token in the wide path.
constexpr float kBonusRange = 60.f;

// ---------------------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

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

// The same (l, mu) pair without tags, for the chunk totals of a two-pass launch (written by one
// kernel, read by the next).
__device__ __forceinline__ float2 slot_pack(Agg a) {
  float l = kNegInf, mu = 0.f;
  if (a.m != kNegInf && a.G > 0.f) {
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  return make_float2(l, mu);
}

__device__ __forceinline__ Agg slot_unpack(float2 s) {
  return Agg{fmaxf(s.x, -1e30f), s.y, s.x == kNegInf ? 0.f : 1.f};
}

enum : int { kFwd = 0, kBwd = 1 };

}  // namespace
