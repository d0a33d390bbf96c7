// Constants, parameter blocks and device helpers shared by the libbiwkv kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

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
// Decay over a whole row (|w| log2 e, base 2) above which a row takes the wide form: its sums'
// exponents can then reach magnitudes where one fp32 exponent no longer resolves 1e-5, so the
// wide form carries token counts separately (Sum). Below it one exponent is exact enough.
constexpr float kExactRange = 128.f;

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

// The scans and the exchange use a finite exponent for an empty sum (F = G = 0), far below any
// real one: 2^(empty - m) is then exactly 0 against a real exponent and 1 against another empty
// one, so adding sums needs no branch.
constexpr float kEmptyM = -1e30f;

// A decayed partial sum of Eq. (6) at some anchor token: numerator F and denominator G, scaled by
// 2^e with e = q D + m. D = w log2(e) / T is the channel's decay per token (base 2), q a whole
// number of tokens (held exactly in fp32) and m the rest (a key's k log2 e plus the sum's own
// scale). Moving the anchor n tokens further from the terms multiplies each by e^{-n w / T}, which
// only lowers q by n: token distances are never rounded into the exponent. Two sums are compared
// through (q1 - q2) D + (m1 - m2), an exact distance times D, so their relative weight stays
// accurate even when both exponents are huge (|w| = 1e4 puts about 14,000 binary orders of
// magnitude across a row, where one fp32 exponent would only resolve 2^-10).
struct Sum {
  float q, m, F, G;
};

__device__ __forceinline__ Sum sum_empty() { return Sum{0.f, kEmptyM, 0.f, 0.f}; }

// Exponent of (qa, ma) minus exponent of (qb, mb).
__device__ __forceinline__ float sum_rel(float qa, float ma, float qb, float mb, float D) {
  return fmaf(qa - qb, D, ma - mb);
}

// The sum of two sums at the same anchor, kept at the larger exponent.
__device__ __forceinline__ Sum sum_add(Sum a, Sum b, float D) {
  const float d = sum_rel(a.q, a.m, b.q, b.m, D);
  const bool big = d >= 0.f;  // a has the larger exponent
  const float s = fast_exp2(-fabsf(d));
  Sum r;
  r.q = big ? a.q : b.q;
  r.m = big ? a.m : b.m;
  r.F = big ? fmaf(b.F, s, a.F) : fmaf(a.F, s, b.F);
  r.G = big ? fmaf(b.G, s, a.G) : fmaf(a.G, s, b.G);
  return r;
}

// The anchor moved n tokens further from the terms (n < 0: closer).
__device__ __forceinline__ Sum sum_shift(Sum a, float n) {
  a.q -= n;
  return a;
}

// The single-exponent sums of the fast form: (m, F, G) meaning F 2^m and G 2^m. The fast form
// only takes rows whose exponents stay small (|w| log2 e <= kExactRange), where one fp32
// exponent is exact enough.
__device__ __forceinline__ Agg agg_none() { return Agg{kEmptyM, 0.f, 0.f}; }

// Sums that cross workgroups are stored as tagged 64-bit words, each with the launch epoch in its
// upper half: a fast-form row publishes (l, mu), a wide-form row (q, l, mu); l = m + log2(G) is
// the log-weight and mu = F / G the weighted mean of v. A reader accepts a slot only when every
// tag carries the current epoch, so no fence is needed. Every chunk of a row takes the same form,
// so a row's slots all have one format; slots are kSlotWords words apart.
constexpr int kSlotWords = 3;
template <class A>
constexpr int kSlotUsed = std::is_same<A, Sum>::value ? 3 : 2;

__device__ __forceinline__ void slot_store(unsigned long long* slot, Agg a, unsigned epoch) {
  float l = kNegInf, mu = 0.f;
  if (a.m > kEmptyM && a.G > 0.f) {
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  const unsigned long long tag = static_cast<unsigned long long>(epoch) << 32;
  __hip_atomic_store(slot, tag | __float_as_uint(l), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 1, tag | __float_as_uint(mu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void slot_store(unsigned long long* slot, Sum a, unsigned epoch) {
  float q = 0.f, l = kNegInf, mu = 0.f;
  if (a.m > kEmptyM && a.G > 0.f) {
    q = a.q;
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  const unsigned long long tag = static_cast<unsigned long long>(epoch) << 32;
  __hip_atomic_store(slot, tag | __float_as_uint(l), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 1, tag | __float_as_uint(mu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 2, tag | __float_as_uint(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class A>
__device__ __forceinline__ void slot_load(const unsigned long long* slot, unsigned long long* w) {
#pragma unroll
  for (int i = 0; i < kSlotUsed<A>; ++i) w[i] = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same words through the L2 of the workgroup's own XCD, for rows whose chunks all run on one
// XCD (the L2 is shared by that XCD's CUs only): plain stores, which reach the L2 as every store
// does, and non-temporal loads, which the CU's own L1 does not keep, so every poll is served by
// that L2. Measured on MI355X with one writer and one poller per XCD, an idle device shows the
// word 200-480 ns after the store this way, against 480-720 ns for device-scope atomics (loads
// carrying only sc0 keep hitting the poller's stale L1 line and never see it). `rs` spans the
// slot array and `off` is the slot's byte offset in it. A reader on another XCD would at worst
// see older tags, never a wrong value: it would wait and then recompute.
typedef unsigned int slot_u2 __attribute__((ext_vector_type(2)));
constexpr int kSlotL2Load = 2;   // nt
constexpr int kSlotL2Store = 0;  // default

__device__ __forceinline__ void slot_word_l2(__amdgpu_buffer_rsrc_t rs, uint32_t off, unsigned long long w) {
  slot_u2 x;
  x.x = static_cast<unsigned>(w);
  x.y = static_cast<unsigned>(w >> 32);
  __builtin_amdgcn_raw_buffer_store_b64(x, rs, off, 0, kSlotL2Store);
}

__device__ __forceinline__ void slot_store_l2(__amdgpu_buffer_rsrc_t rs, uint32_t off, Agg a, unsigned epoch) {
  float l = kNegInf, mu = 0.f;
  if (a.m > kEmptyM && a.G > 0.f) {
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  const unsigned long long tag = static_cast<unsigned long long>(epoch) << 32;
  slot_word_l2(rs, off, tag | __float_as_uint(l));
  slot_word_l2(rs, off + 8u, tag | __float_as_uint(mu));
}

__device__ __forceinline__ void slot_store_l2(__amdgpu_buffer_rsrc_t rs, uint32_t off, Sum a, unsigned epoch) {
  float q = 0.f, l = kNegInf, mu = 0.f;
  if (a.m > kEmptyM && a.G > 0.f) {
    q = a.q;
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  const unsigned long long tag = static_cast<unsigned long long>(epoch) << 32;
  slot_word_l2(rs, off, tag | __float_as_uint(l));
  slot_word_l2(rs, off + 8u, tag | __float_as_uint(mu));
  slot_word_l2(rs, off + 16u, tag | __float_as_uint(q));
}

template <class A>
__device__ __forceinline__ void slot_load_l2(__amdgpu_buffer_rsrc_t rs, uint32_t off, unsigned long long* w) {
#pragma unroll
  for (int i = 0; i < kSlotUsed<A>; ++i) {
    const slot_u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8u * i, 0, kSlotL2Load);
    w[i] = static_cast<unsigned long long>(x.x) | (static_cast<unsigned long long>(x.y) << 32);
  }
}

template <class A>
__device__ __forceinline__ bool slot_ready(const unsigned long long* w, unsigned epoch) {
  bool ok = true;
#pragma unroll
  for (int i = 0; i < kSlotUsed<A>; ++i) ok = ok && static_cast<unsigned>(w[i] >> 32) == epoch;
  return ok;
}

template <class A>
__device__ __forceinline__ A slot_value(const unsigned long long* w);
template <>
__device__ __forceinline__ Agg slot_value<Agg>(const unsigned long long* w) {
  const float l = __uint_as_float(static_cast<unsigned>(w[0]));
  if (!(l > kEmptyM)) return agg_none();
  return Agg{l, __uint_as_float(static_cast<unsigned>(w[1])), 1.f};
}
template <>
__device__ __forceinline__ Sum slot_value<Sum>(const unsigned long long* w) {
  const float l = __uint_as_float(static_cast<unsigned>(w[0]));
  if (!(l > kEmptyM)) return sum_empty();
  return Sum{__uint_as_float(static_cast<unsigned>(w[2])), l, __uint_as_float(static_cast<unsigned>(w[1])), 1.f};
}

// The same pairs without tags, for the chunk totals and carries of a two-pass launch (written by
// one kernel, read by the next), as (q, l, mu, -): a fast-form sum has q = 0.
__device__ __forceinline__ float4 slot_pack(Sum a) {
  float q = 0.f, l = kNegInf, mu = 0.f;
  if (a.m > kEmptyM && a.G > 0.f) {
    q = a.q;
    l = a.m + fast_log2(a.G);
    mu = a.F * fast_rcp(a.G);
  }
  return make_float4(q, l, mu, 0.f);
}
__device__ __forceinline__ float4 slot_pack(Agg a) { return slot_pack(Sum{0.f, a.m, a.F, a.G}); }

__device__ __forceinline__ Sum slot_unpack(float4 s) {
  if (!(s.y > kEmptyM)) return sum_empty();
  return Sum{s.x, s.y, s.z, 1.f};
}

enum : int { kFwd = 0, kBwd = 1 };

}  // namespace
