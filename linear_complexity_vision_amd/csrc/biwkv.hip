// libbiwkv — Bi-WKV and Q-Shift for AMD Instinct MI355X (gfx950, CDNA4), hand-written HIP.
//
// What is computed (cited by page title and equation):
//   * Bi-WKV: "OpenGVLab&港中文&复旦&南大&清华提出Vision-RWKV Backbone" (Vision-RWKV article),
//     section "Linear Complexity Bidirectional Attention", Eq. (5); evaluated through the
//     four-state RNN form of Eq. (6)-(7) (a, c forward; b, d backward; output of Eq. (7)).
//   * Q-Shift: the q_shift function of "LinXin's Blog" Vision-RWKV notes.
//
// How (MI355X-first design; see include/biwkv.h for the ABI):
//   * Layout [B, T, C]; lanes map to consecutive channels, so every load of k, v and every store
//     of out is one contiguous segment per wavefront. Each lane owns V channels of one tile of
//     64*V channels; each wavefront owns LW consecutive tokens; a workgroup of NW wavefronts owns
//     a chunk of LW*NW tokens of one (batch, tile) row.
//   * One pass over HBM. A wavefront keeps its tokens in registers from load to store. Per chunk
//     it forms the Eq. (6) partial sums of its tokens (the aggregate of a decayed sum is a
//     triple (m, F, G) meaning F*2^m, G*2^m; appending n tokens shifts m by -n*w*log2(e)/T,
//     so e^{-w/T} powers are never formed by repeated multiplication across chunks).
//   * Chunks of a row are combined by a decoupled look-back in both directions: every chunk
//     publishes its aggregate as soon as it has read its data, then walks towards the row start
//     (forward states a, c) and towards the row end (backward states b, d) until it meets an
//     inclusive prefix/suffix. Chunk identities come from a ticket counter, so a chunk only waits
//     for chunks that hold tickets or will get them while it waits (the host limits the chunks
//     per row to what can be resident), and every wait is bounded.
//   * Exponents are kept relative to a running maximum (base 2), so any sign of w and large k
//     or u never overflow fp32.
//   * Q-Shift for the fused entry is an index remap applied to the k/v loads (zero-filled
//     sources load as 0); no shifted copy is materialised.
//   * No MFMA: the path has no dense contraction. No packed-FP32 instructions are emitted
//     (the library is built with that target feature disabled).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

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
  unsigned long long* slots;  // published aggregates: [row][chunk][dir][tile channel][2 words]
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

// Published form: (l, mu) with l = m + log2(G) the log-weight and mu = F / G the weighted mean.
__device__ __forceinline__ Agg agg_from_pub(float l, float mu) {
  if (l == kNegInf) return agg_empty();
  return Agg{l, mu, 1.f};
}

__device__ __forceinline__ unsigned long long pack_word(float x, unsigned tag) {
  return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(x);
}

// Canonical (published) form of an aggregate: l = m + log2(G), mu = F / G, stored as (l, mu, 1).
// Every value that crosses chunks is folded and stored in this form, so a reader that rebuilds a
// carry from published aggregates gets exactly the value the publisher computed.
__device__ __forceinline__ Agg agg_canon(Agg a) {
  if (a.m == kNegInf || !(a.G > 0.f)) return agg_empty();
  return Agg{a.m + fast_log2(a.G), a.F * fast_rcp(a.G), 1.f};
}

// Stores a canonical aggregate (two tagged 64-bit words; readers accept only matching tags).
__device__ __forceinline__ void publish(unsigned long long* slot, Agg c, unsigned tag) {
  __hip_atomic_store(slot, pack_word(c.m, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + 1, pack_word(c.F, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads one published slot. Returns 0 if not yet published in this launch, 1 for an aggregate,
// 2 for an inclusive prefix/suffix.
__device__ __forceinline__ int read_slot(const unsigned long long* slot, unsigned epoch, Agg* out) {
  const unsigned long long w0 =
      __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long w1 =
      __hip_atomic_load(slot + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned t0 = static_cast<unsigned>(w0 >> 32), t1 = static_cast<unsigned>(w1 >> 32);
  if (t0 != t1 || (t0 >> 1) != epoch) return 0;
  *out = agg_from_pub(__uint_as_float(static_cast<unsigned>(w0)),
                      __uint_as_float(static_cast<unsigned>(w1)));
  return (t0 & 1u) ? 2 : 1;
}

enum : int { kFwd = 0, kBwd = 1 };
enum : unsigned { kKindAgg = 0, kKindInc = 1 };

// ---------------------------------------------------------------------------------------------
// Bi-WKV chunk-scan kernel (one pass, both directions, decoupled look-back across chunks)
// ---------------------------------------------------------------------------------------------

template <int DT, int V, int LW, int NW, bool FUSED>
__global__ void __launch_bounds__(NW * 64)
    biwkv_chunk_scan_kernel(BiwkvParams p) {
  using S = KV<DT, V>;
  using raw_t = typename S::raw_t;
  constexpr int TILE = 64 * V;
  constexpr int LWG = LW * NW;

  __shared__ unsigned sh_ticket, sh_epoch;
  __shared__ float lds_agg[NW][6][TILE];  // per wavefront: m, F, G (forward), mb, Fb, Gb (backward)
  __shared__ float lds_pre[NW][3][TILE];  // exclusive forward aggregate inside the chunk
  __shared__ float lds_suf[NW][3][TILE];  // exclusive backward aggregate inside the chunk
  __shared__ float lds_x[3][TILE];        // forward carry into the chunk (tokens before it)
  __shared__ float lds_y[3][TILE];        // backward carry into the chunk (tokens after it)

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (threadIdx.x == 0) {
    sh_ticket = __hip_atomic_fetch_add(&p.ctr->ticket, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    sh_epoch = __hip_atomic_load(&p.ctr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const unsigned epoch = sh_epoch;
  // A ticket beyond the grid can only come from a counter left non-zero by an earlier launch;
  // such a workgroup touches no data (its row would be out of range) and only retires.
  const bool valid_ticket = sh_ticket < p.total;
  if (!valid_ticket && threadIdx.x == 0)
    __hip_atomic_fetch_or(&p.ctr->fault, kFaultTicket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned ticket = valid_ticket ? sh_ticket : 0u;

  // Tickets enumerate rows in order and, inside a row, chunks in order.
  const int chunk = static_cast<int>(ticket % static_cast<unsigned>(p.n_chunks));
  const int row = static_cast<int>(ticket / static_cast<unsigned>(p.n_chunks));
  const int tile = row % p.n_tiles;
  const long long b = row / p.n_tiles;
  const long long T = p.T;
  const int C = p.C;
  const int c0 = tile * TILE + lane * V;  // first channel of this lane
  const bool lane_on = valid_ticket && c0 < C;  // the host guarantees V | C when V > 1

  const long long s_chunk = static_cast<long long>(chunk) * LWG;
  const int n_chunk_tok = static_cast<int>(T - s_chunk < LWG ? T - s_chunk : LWG);
  const long long s_w = s_chunk + static_cast<long long>(wave) * LW;
  const long long rem = T - s_w;
  const int n_w = (rem <= 0 || !valid_ticket) ? 0 : (rem < LW ? static_cast<int>(rem) : LW);

  // Per-channel constants in base 2: D = w log2(e) / T, lam = 2^{-D} (one decay step),
  // U = u log2(e), grow = max(0, -D) (largest per-step growth).
  float D[V], lam[V], U[V], grow[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const float wc = lane_on ? p.w[c0 + j] : 0.f;
    const float uc = lane_on ? p.u[c0 + j] : 0.f;
    D[j] = (wc / static_cast<float>(T)) * kLog2e;
    lam[j] = fast_exp2(-D[j]);
    U[j] = uc * kLog2e;
    grow[j] = fmaxf(-D[j], 0.f);
  }

  // ---- load this wavefront's tokens (coalesced along C) ----
  raw_t kr[LW], vr[LW];
  int hh = 0, ww = 0;
  int grp = 4;  // Q-Shift channel group of this lane (4 = copied)
  if constexpr (FUSED) {
    hh = static_cast<int>(s_w / p.W);
    ww = static_cast<int>(s_w % p.W);
    grp = c0 < p.g1 ? 0 : c0 < p.g2 ? 1 : c0 < p.g3 ? 2 : c0 < p.g4 ? 3 : 4;
  }
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const long long t = s_w + i;
    bool ok = lane_on && i < n_w;
    long long src = t;
    if constexpr (FUSED) {
      const int s = p.shift;
      switch (grp) {
        case 0: ok = ok && ww >= s; src = t - s; break;                                   // right
        case 1: ok = ok && ww < p.W - s; src = t + s; break;                              // left
        case 2: ok = ok && hh >= s; src = t - static_cast<long long>(s) * p.W; break;     // down
        case 3: ok = ok && hh < p.H - s; src = t + static_cast<long long>(s) * p.W; break; // up
        default: break;                                                                   // copy
      }
      if (++ww == p.W) {
        ww = 0;
        ++hh;
      }
    }
    const long long idx = (b * T + src) * C + c0;
    kr[i] = ok ? S::load(p.k, idx) : S::zero();
    vr[i] = ok ? S::load(p.v, idx) : S::zero();
  }

  // ---- phase A: the wavefront's own aggregates (forward anchored at its last token,
  //      backward anchored at its first token), stabilised by the largest exponent ----
  // wide: some lane's decay range over the wavefront exceeds what one reference can hold.
  bool wide_lane = false;
#pragma unroll
  for (int j = 0; j < V; ++j)
    wide_lane = wide_lane || fabsf(D[j]) * static_cast<float>(LW - 1) > kFastRange;
  const bool wide = __ballot(wide_lane) != 0ull;

  float kmax[V];
#pragma unroll
  for (int j = 0; j < V; ++j) kmax[j] = kNegInf;
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    if (i < n_w) {
      float kf[V];
      S::unpack(kr[i], kf);
#pragma unroll
      for (int j = 0; j < V; ++j) kmax[j] = fmaxf(kmax[j], kf[j] * kLog2e);
    }
  }
  Agg af[V], ab[V];  // forward (anchored at the last token) and backward (at the first token)
  float pr[LW][V];   // fast path: e^{k_i} relative to 2^{mw}, every weight of the wavefront <= 1
  if (!wide) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float mw = n_w > 0 ? kmax[j] + grow[j] * static_cast<float>(n_w - 1) : kNegInf;
      af[j] = Agg{mw, 0.f, 0.f};
      ab[j] = Agg{mw, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      if (i < n_w) {
        float kf[V], vf[V];
        S::unpack(kr[i], kf);
        S::unpack(vr[i], vf);
#pragma unroll
        for (int j = 0; j < V; ++j) {
          pr[i][j] = fast_exp2(fmaf(kf[j], kLog2e, -af[j].m));
          af[j].F = fmaf(af[j].F, lam[j], pr[i][j] * vf[j]);
          af[j].G = fmaf(af[j].G, lam[j], pr[i][j]);
        }
      }
    }
#pragma unroll
    for (int i = LW - 1; i >= 0; --i) {
      if (i < n_w) {
        float vf[V];
        S::unpack(vr[i], vf);
#pragma unroll
        for (int j = 0; j < V; ++j) {
          ab[j].F = fmaf(ab[j].F, lam[j], pr[i][j] * vf[j]);
          ab[j].G = fmaf(ab[j].G, lam[j], pr[i][j]);
        }
      }
    }
  } else {
    // Wide range: one decay step at a time, each sum kept against its own running maximum.
#pragma unroll
    for (int j = 0; j < V; ++j) af[j] = ab[j] = agg_empty();
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      if (i < n_w) {
        float kf[V], vf[V];
        S::unpack(kr[i], kf);
        S::unpack(vr[i], vf);
#pragma unroll
        for (int j = 0; j < V; ++j)
          af[j] = agg_add(agg_shift(af[j], 1.f, D[j]), Agg{kf[j] * kLog2e, vf[j], 1.f});
      }
    }
#pragma unroll
    for (int i = LW - 1; i >= 0; --i) {
      if (i < n_w) {
        float kf[V], vf[V];
        S::unpack(kr[i], kf);
        S::unpack(vr[i], vf);
#pragma unroll
        for (int j = 0; j < V; ++j)
          ab[j] = agg_add(agg_shift(ab[j], 1.f, D[j]), Agg{kf[j] * kLog2e, vf[j], 1.f});
      }
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int ch = lane * V + j;
    lds_agg[wave][0][ch] = af[j].m;
    lds_agg[wave][1][ch] = af[j].F;
    lds_agg[wave][2][ch] = af[j].G;
    lds_agg[wave][3][ch] = ab[j].m;
    lds_agg[wave][4][ch] = ab[j].F;
    lds_agg[wave][5][ch] = ab[j].G;
  }
  __syncthreads();

  // ---- phase B: chunk aggregates, publication and look-back (one wavefront per direction) ----
  const int fwd_wave = 0;
  const int bwd_wave = NW > 1 ? 1 : 0;
  const long long row_slots = static_cast<long long>(row) * p.n_chunks;
  auto slot_of = [&](int ck, int dir, int j) -> unsigned long long* {
    return p.slots + (((row_slots + ck) * 2 + dir) * TILE + lane * V + j) * 2;
  };

  if (wave == fwd_wave) {
    Agg acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = agg_empty();
    for (int wv = 0; wv < NW; ++wv) {
      const long long rem_w = T - (s_chunk + static_cast<long long>(wv) * LW);
      const int n = rem_w <= 0 ? 0 : (rem_w < LW ? static_cast<int>(rem_w) : LW);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int ch = lane * V + j;
        lds_pre[wv][0][ch] = acc[j].m;
        lds_pre[wv][1][ch] = acc[j].F;
        lds_pre[wv][2][ch] = acc[j].G;
        const Agg a{lds_agg[wv][0][ch], lds_agg[wv][1][ch], lds_agg[wv][2][ch]};
        acc[j] = agg_add(agg_shift(acc[j], static_cast<float>(n), D[j]), a);
      }
    }
    Agg x[V];
#pragma unroll
    for (int j = 0; j < V; ++j) x[j] = agg_empty();
    if (lane_on && p.n_chunks > 1) {
      const int last = p.n_chunks - 1;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const Agg self = agg_canon(acc[j]);
        if (chunk == 0) {
          publish(slot_of(0, kFwd, j), self, epoch * 2u + kKindInc);
          continue;
        }
        if (chunk < last) publish(slot_of(chunk, kFwd, j), self, epoch * 2u + kKindAgg);
        // Walk towards the row start until an inclusive prefix is published (chunk 0 always
        // publishes one), then fold the aggregates after it left to right.
        int ck = chunk - 1;
        unsigned spins = 0;
        bool lost = false;
        Agg a;
        for (;;) {
          const int kind = read_slot(slot_of(ck, kFwd, j), epoch, &a);
          if (kind == 2) break;
          if (kind == 1) {
            --ck;
            continue;
          }
          if (++spins > kSpinLimit) {
            lost = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        Agg xc = a;
        for (int q = ck + 1; q < chunk && !lost;) {
          // A slot seen as an aggregate may be caught while it is re-tagged as inclusive (its
          // two words briefly disagree): read it again.
          const int kind = read_slot(slot_of(q, kFwd, j), epoch, &a);
          if (kind == 0) {
            if (++spins > kSpinLimit) lost = true;
            continue;
          }
          xc = kind == 2 ? a  // already the canonical fold up to q
                         : agg_canon(agg_add(agg_shift(xc, static_cast<float>(LWG), D[j]), a));
          ++q;
        }
        if (lost) {
          __hip_atomic_fetch_or(&p.ctr->fault, kFaultSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          xc = agg_empty();
        }
        x[j] = xc;
        if (chunk < last) {
          const Agg inc = agg_canon(agg_add(agg_shift(xc, static_cast<float>(n_chunk_tok), D[j]), self));
          publish(slot_of(chunk, kFwd, j), inc, epoch * 2u + kKindInc);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      lds_x[0][ch] = x[j].m;
      lds_x[1][ch] = x[j].F;
      lds_x[2][ch] = x[j].G;
    }
  }

  if (wave == bwd_wave) {
    Agg acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = agg_empty();
    for (int wv = NW - 1; wv >= 0; --wv) {
      const long long rem_w = T - (s_chunk + static_cast<long long>(wv) * LW);
      const int n = rem_w <= 0 ? 0 : (rem_w < LW ? static_cast<int>(rem_w) : LW);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int ch = lane * V + j;
        lds_suf[wv][0][ch] = acc[j].m;
        lds_suf[wv][1][ch] = acc[j].F;
        lds_suf[wv][2][ch] = acc[j].G;
        const Agg a{lds_agg[wv][3][ch], lds_agg[wv][4][ch], lds_agg[wv][5][ch]};
        acc[j] = agg_add(a, agg_shift(acc[j], static_cast<float>(n), D[j]));
      }
    }
    Agg y[V];
#pragma unroll
    for (int j = 0; j < V; ++j) y[j] = agg_empty();
    if (lane_on && p.n_chunks > 1) {
      const int last = p.n_chunks - 1;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const Agg self = agg_canon(acc[j]);
        if (chunk == last) {
          publish(slot_of(last, kBwd, j), self, epoch * 2u + kKindInc);
          continue;
        }
        if (chunk > 0) publish(slot_of(chunk, kBwd, j), self, epoch * 2u + kKindAgg);
        // Walk towards the row end until an inclusive suffix is published (the last chunk always
        // publishes one), then fold the aggregates before it right to left.
        int ck = chunk + 1;
        unsigned spins = 0;
        bool lost = false;
        Agg a;
        for (;;) {
          const int kind = read_slot(slot_of(ck, kBwd, j), epoch, &a);
          if (kind == 2) break;
          if (kind == 1) {
            ++ck;
            continue;
          }
          if (++spins > kSpinLimit) {
            lost = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        Agg yc = a;
        for (int q = ck - 1; q > chunk && !lost;) {
          const int kind = read_slot(slot_of(q, kBwd, j), epoch, &a);
          if (kind == 0) {  // caught while being re-tagged: read again
            if (++spins > kSpinLimit) lost = true;
            continue;
          }
          yc = kind == 2 ? a  // already the canonical fold from q
                         : agg_canon(agg_add(a, agg_shift(yc, static_cast<float>(LWG), D[j])));
          --q;
        }
        if (lost) {
          __hip_atomic_fetch_or(&p.ctr->fault, kFaultSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          yc = agg_empty();
        }
        y[j] = yc;
        if (chunk > 0) {
          const Agg inc = agg_canon(agg_add(self, agg_shift(yc, static_cast<float>(n_chunk_tok), D[j])));
          publish(slot_of(chunk, kBwd, j), inc, epoch * 2u + kKindInc);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      lds_y[0][ch] = y[j].m;
      lds_y[1][ch] = y[j].F;
      lds_y[2][ch] = y[j].G;
    }
  }
  __syncthreads();

  // ---- phase C: each wavefront sweeps its tokens forward (a, c) then backward (b, d) and
  //      writes Eq. (7) ----
  if (n_w > 0) {
    Agg xw[V], yw[V];
    const float before = static_cast<float>(wave * LW);  // tokens between chunk start and s_w
    const float after = static_cast<float>(n_chunk_tok - wave * LW - n_w);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      const Agg X{lds_x[0][ch], lds_x[1][ch], lds_x[2][ch]};
      const Agg P{lds_pre[wave][0][ch], lds_pre[wave][1][ch], lds_pre[wave][2][ch]};
      const Agg Y{lds_y[0][ch], lds_y[1][ch], lds_y[2][ch]};
      const Agg Q{lds_suf[wave][0][ch], lds_suf[wave][1][ch], lds_suf[wave][2][ch]};
      xw[j] = agg_add(agg_shift(X, before, D[j]), P);  // a, c just before the first token
      yw[j] = agg_add(Q, agg_shift(Y, after, D[j]));   // b, d just after the last token
    }
    float al[LW][V], be[LW][V];
    if (!wide) {
      float M[V], A[V], Cs[V], Bs[V], Ds[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        // Every scaled term below is <= 1: local weights and carries all sit under M.
        M[j] = fmaxf(fmaxf(kmax[j], xw[j].m), yw[j].m) + grow[j] * static_cast<float>(n_w - 1);
        const float sx = fast_exp2(xw[j].m - M[j]);
        const float sy = fast_exp2(yw[j].m - M[j]);
        A[j] = xw[j].F * sx;
        Cs[j] = xw[j].G * sx;
        Bs[j] = yw[j].F * sy;
        Ds[j] = yw[j].G * sy;
      }
      // forward sweep: keep alpha = a - c v and beta = c + e^{u+k} for each token
#pragma unroll
      for (int i = 0; i < LW; ++i) {
        if (i < n_w) {
          float kf[V], vf[V];
          S::unpack(kr[i], kf);
          S::unpack(vr[i], vf);
#pragma unroll
          for (int j = 0; j < V; ++j) {
            const float x = fmaf(kf[j], kLog2e, -M[j]);
            const float pi = fast_exp2(x);
            const float e = fmaxf(fast_exp2(x + U[j]), 1.17549435e-38f);
            al[i][j] = fmaf(-Cs[j], vf[j], A[j]);
            be[i][j] = Cs[j] + e;
            A[j] = fmaf(A[j], lam[j], pi * vf[j]);
            Cs[j] = fmaf(Cs[j], lam[j], pi);
          }
        }
      }
      // backward sweep: y = v + (a + b - (c + d) v) / (c + d + e^{u+k})
#pragma unroll
      for (int i = LW - 1; i >= 0; --i) {
        if (i < n_w) {
          float kf[V], vf[V], y[V];
          S::unpack(kr[i], kf);
          S::unpack(vr[i], vf);
#pragma unroll
          for (int j = 0; j < V; ++j) {
            const float num = fmaf(-Ds[j], vf[j], al[i][j] + Bs[j]);
            const float den = be[i][j] + Ds[j];
            y[j] = fmaf(num, fast_rcp(den), vf[j]);
            const float pi = fast_exp2(fmaf(kf[j], kLog2e, -M[j]));
            Bs[j] = fmaf(Bs[j], lam[j], pi * vf[j]);
            Ds[j] = fmaf(Ds[j], lam[j], pi);
          }
          if (lane_on) store_out<V>(p.out, (b * T + s_w + i) * C + c0, y);
        }
      }
    } else {
      // Wide range: the forward state of each token is kept with its own exponent (in pr), the
      // backward state is stepped token by token, and Eq. (7) is formed against the largest of
      // the three exponents (forward, backward, self).
#pragma unroll
      for (int i = 0; i < LW; ++i) {
        if (i < n_w) {
          float kf[V], vf[V];
          S::unpack(kr[i], kf);
          S::unpack(vr[i], vf);
#pragma unroll
          for (int j = 0; j < V; ++j) {
            pr[i][j] = xw[j].m;
            al[i][j] = fmaf(-xw[j].G, vf[j], xw[j].F);
            be[i][j] = xw[j].G;
            xw[j] = agg_add(agg_shift(xw[j], 1.f, D[j]), Agg{kf[j] * kLog2e, vf[j], 1.f});
          }
        }
      }
#pragma unroll
      for (int i = LW - 1; i >= 0; --i) {
        if (i < n_w) {
          float kf[V], vf[V], y[V];
          S::unpack(kr[i], kf);
          S::unpack(vr[i], vf);
#pragma unroll
          for (int j = 0; j < V; ++j) {
            const float ks = fmaf(kf[j], kLog2e, U[j]);
            const float Mt = fmaxf(fmaxf(pr[i][j], yw[j].m), ks);
            const float sa = fast_exp2(pr[i][j] - Mt), sb = fast_exp2(yw[j].m - Mt);
            const float e = fast_exp2(ks - Mt);
            const float num = al[i][j] * sa + fmaf(-yw[j].G, vf[j], yw[j].F) * sb;
            const float den = be[i][j] * sa + yw[j].G * sb + e;
            y[j] = fmaf(num, fast_rcp(den), vf[j]);
            yw[j] = agg_add(agg_shift(yw[j], 1.f, D[j]), Agg{kf[j] * kLog2e, vf[j], 1.f});
          }
          if (lane_on) store_out<V>(p.out, (b * T + s_w + i) * C + c0, y);
        }
      }
    }
  }

  // ---- retire: the last workgroup of the launch resets the counters for the next launch ----
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned fin =
        __hip_atomic_fetch_add(&p.ctr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (fin + 1u == p.total) {
      __hip_atomic_store(&p.ctr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.ctr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&p.ctr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

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

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------

thread_local int t_last_hip_error = 0;

int hip_fail(hipError_t e) {
  t_last_hip_error = static_cast<int>(e);
  return BIWKV_ERR_HIP;
}

struct StreamScratch {
  Counters* ctr = nullptr;
  unsigned long long* slots = nullptr;
  long long slot_words = 0;
  std::vector<void*> retired;  // outgrown slot buffers; pending launches may still use them
};

std::mutex g_mu;
std::map<std::pair<int, void*>, StreamScratch*> g_scratch;
std::map<std::pair<int, const void*>, int> g_capacity;  // (device, kernel) -> resident workgroups

int current_device(int* dev) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return BIWKV_ERR_NO_DEVICE;
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// Scratch of (device, stream) with at least `words` slot words. Caller holds g_mu.
int get_scratch(int dev, void* stream, long long words, StreamScratch** out) {
  auto key = std::make_pair(dev, stream);
  StreamScratch*& sc = g_scratch[key];
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!sc) {
    StreamScratch* fresh = new StreamScratch();
    hipError_t e = hipMalloc(&fresh->ctr, 256);
    if (e != hipSuccess) {
      delete fresh;
      g_scratch.erase(key);
      return hip_fail(e);
    }
    hipLaunchKernelGGL(init_counters_kernel, dim3(1), dim3(1), 0, st, fresh->ctr);
    e = hipGetLastError();
    if (e != hipSuccess) {
      (void)hipFree(fresh->ctr);
      delete fresh;
      g_scratch.erase(key);
      return hip_fail(e);
    }
    sc = fresh;
  }
  if (sc->slot_words < words) {
    long long want = sc->slot_words ? sc->slot_words : (1ll << 16);
    while (want < words) want *= 2;
    unsigned long long* buf = nullptr;
    hipError_t e = hipMalloc(&buf, static_cast<size_t>(want) * sizeof(unsigned long long));
    if (e != hipSuccess) return hip_fail(e);
    long long blocks = (want + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, buf,
                       want);
    e = hipGetLastError();
    if (e != hipSuccess) {
      (void)hipFree(buf);
      return hip_fail(e);
    }
    if (sc->slots) sc->retired.push_back(sc->slots);
    sc->slots = buf;
    sc->slot_words = want;
  }
  *out = sc;
  return BIWKV_OK;
}

int resident_capacity(int dev, const void* kernel, int block, int* cap) {
  auto key = std::make_pair(dev, kernel);
  auto it = g_capacity.find(key);
  if (it != g_capacity.end()) {
    *cap = it->second;
    return BIWKV_OK;
  }
  int per_cu = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0);
  if (e != hipSuccess) return hip_fail(e);
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e);
  *cap = per_cu * cus;
  g_capacity[key] = *cap;
  return BIWKV_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!na || !nb) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Q-Shift group bounds exactly as the listing computes them: int(C * gamma * j) in double.
void group_bounds(int64_t C, double gamma, int64_t g[4]) {
  for (int j = 1; j <= 4; ++j) g[j - 1] = static_cast<int64_t>(static_cast<double>(C) * gamma * j);
}

int check_qshift_params(int64_t H, int64_t W, int shift, double gamma) {
  if (!(gamma >= 0.0 && gamma <= 0.25)) return BIWKV_ERR_PARAM;
  if (shift < 0 || shift > H || shift > W) return BIWKV_ERR_PARAM;
  return BIWKV_OK;
}

constexpr int64_t kMaxDim = (1ll << 31) - 1;

int check_bitc_shape(int64_t B, int64_t T, int64_t C) {
  if (B < 0 || T < 0 || C < 0) return BIWKV_ERR_SHAPE;
  if (B > kMaxDim || T > kMaxDim || C > kMaxDim) return BIWKV_ERR_SHAPE;
  if (B && T && C) {
    const long double n = static_cast<long double>(B) * T * C * 4.0L;
    if (n > 9.0e18L) return BIWKV_ERR_SHAPE;
  }
  return BIWKV_OK;
}

// Tile shapes: LW tokens per wavefront, NW wavefronts per workgroup.
constexpr int kLW = 16;
constexpr int kNW = 8;

template <int DT, int V, bool FUSED>
int launch_biwkv(BiwkvParams prm, int64_t B, int dev, void* stream) {
  constexpr int TILE = 64 * V;
  constexpr int LWG = kLW * kNW;
  const void* kfn = reinterpret_cast<const void*>(&biwkv_chunk_scan_kernel<DT, V, kLW, kNW, FUSED>);
  const int64_t n_tiles = (prm.C + TILE - 1) / TILE;
  const int64_t n_chunks = (prm.T + LWG - 1) / LWG;
  const int64_t total = B * n_tiles * n_chunks;
  if (total > 0x7FFFFFFFll) return BIWKV_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(g_mu);
  int cap = 0;
  int rc = resident_capacity(dev, kfn, kNW * 64, &cap);
  if (rc) return rc;
  if (n_chunks > cap) return BIWKV_ERR_UNSUPPORTED;
  StreamScratch* sc = nullptr;
  const long long words = B * n_tiles * n_chunks * 2 * TILE * 2;
  rc = get_scratch(dev, stream, words, &sc);
  if (rc) return rc;
  prm.n_tiles = static_cast<int>(n_tiles);
  prm.n_chunks = static_cast<int>(n_chunks);
  prm.total = static_cast<unsigned>(total);
  prm.slots = sc->slots;
  prm.ctr = sc->ctr;
  hipLaunchKernelGGL((biwkv_chunk_scan_kernel<DT, V, kLW, kNW, FUSED>),
                     dim3(static_cast<unsigned>(total)), dim3(kNW * 64), 0,
                     static_cast<hipStream_t>(stream), prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

template <bool FUSED>
int dispatch_biwkv(BiwkvParams prm, int64_t B, int dtype, bool vec2, int dev, void* stream) {
  if (dtype == BIWKV_F32)
    return vec2 ? launch_biwkv<BIWKV_F32, 2, FUSED>(prm, B, dev, stream)
                : launch_biwkv<BIWKV_F32, 1, FUSED>(prm, B, dev, stream);
  return vec2 ? launch_biwkv<BIWKV_BF16, 2, FUSED>(prm, B, dev, stream)
              : launch_biwkv<BIWKV_BF16, 1, FUSED>(prm, B, dev, stream);
}

int validate_biwkv(const void* k, const void* v, const float* w, const float* u, const float* out,
                   int64_t B, int64_t T, int64_t C, int dtype) {
  int rc = check_bitc_shape(B, T, C);
  if (rc) return rc;
  if (dtype != BIWKV_F32 && dtype != BIWKV_BF16) return BIWKV_ERR_DTYPE;
  const bool nonempty = B && T && C;
  if (nonempty && (!k || !v || !out)) return BIWKV_ERR_NULL;
  if (C && (!w || !u)) return BIWKV_ERR_NULL;
  if (!nonempty) return BIWKV_OK;
  const size_t es = dtype == BIWKV_F32 ? 4 : 2;
  if (!aligned(k, es) || !aligned(v, es) || !aligned(out, 4) || !aligned(w, 4) || !aligned(u, 4))
    return BIWKV_ERR_ALIGN;
  const size_t n = static_cast<size_t>(B) * T * C;
  if (ranges_overlap(out, n * 4, k, n * es) || ranges_overlap(out, n * 4, v, n * es) ||
      ranges_overlap(out, n * 4, w, C * 4) || ranges_overlap(out, n * 4, u, C * 4))
    return BIWKV_ERR_ALIAS;
  return BIWKV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------------------------

extern "C" {

int biwkv_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                  int64_t B, int64_t T, int64_t C, int dtype, void* stream) {
  int rc = validate_biwkv(k, v, w, u, out, B, T, C, dtype);
  if (rc || !(B && T && C)) return rc;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  const size_t es = dtype == BIWKV_F32 ? 4 : 2;
  const bool vec2 = (C % 2 == 0) && aligned(k, 2 * es) && aligned(v, 2 * es) && aligned(out, 8);
  BiwkvParams prm{};
  prm.k = k;
  prm.v = v;
  prm.w = w;
  prm.u = u;
  prm.out = out;
  prm.T = T;
  prm.C = static_cast<int>(C);
  return dispatch_biwkv<false>(prm, B, dtype, vec2, dev, stream);
}

int biwkv_qshift_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                         int64_t B, int64_t H, int64_t W, int64_t C, int shift, double gamma,
                         int dtype, void* stream) {
  if (H < 0 || W < 0 || H > kMaxDim || W > kMaxDim) return BIWKV_ERR_SHAPE;
  const int64_t T = H * W;
  int rc = validate_biwkv(k, v, w, u, out, B, T, C, dtype);
  if (rc) return rc;
  rc = check_qshift_params(H, W, shift, gamma);
  if (rc || !(B && T && C)) return rc;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  int64_t g[4];
  group_bounds(C, gamma, g);
  const size_t es = dtype == BIWKV_F32 ? 4 : 2;
  const bool groups_even = (g[0] % 2 == 0) && (g[1] % 2 == 0) && (g[2] % 2 == 0) && (g[3] % 2 == 0);
  const bool vec2 = (C % 2 == 0) && groups_even && aligned(k, 2 * es) && aligned(v, 2 * es) &&
                    aligned(out, 8);
  BiwkvParams prm{};
  prm.k = k;
  prm.v = v;
  prm.w = w;
  prm.u = u;
  prm.out = out;
  prm.T = T;
  prm.C = static_cast<int>(C);
  prm.H = static_cast<int>(H);
  prm.W = static_cast<int>(W);
  prm.shift = shift;
  prm.g1 = static_cast<int>(g[0]);
  prm.g2 = static_cast<int>(g[1]);
  prm.g3 = static_cast<int>(g[2]);
  prm.g4 = static_cast<int>(g[3]);
  return dispatch_biwkv<true>(prm, B, dtype, vec2, dev, stream);
}

int qshift(const float* x, float* out, int64_t B, int64_t H, int64_t W, int64_t C, int shift,
           double gamma, void* stream) {
  if (H < 0 || W < 0 || H > kMaxDim || W > kMaxDim) return BIWKV_ERR_SHAPE;
  int rc = check_bitc_shape(B, H * W, C);
  if (rc) return rc;
  const bool nonempty = B && H && W && C;
  if (nonempty && (!x || !out)) return BIWKV_ERR_NULL;
  rc = check_qshift_params(H, W, shift, gamma);
  if (rc || !nonempty) return rc;
  if (!aligned(x, 4) || !aligned(out, 4)) return BIWKV_ERR_ALIGN;
  const size_t n = static_cast<size_t>(B) * H * W * C;
  if (ranges_overlap(out, n * 4, x, n * 4)) return BIWKV_ERR_ALIAS;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  int64_t g[4];
  group_bounds(C, gamma, g);
  const bool vec4 = (C % 4 == 0) && (g[0] % 4 == 0) && (g[1] % 4 == 0) && (g[2] % 4 == 0) &&
                    (g[3] % 4 == 0) && aligned(x, 16) && aligned(out, 16);
  const long long rows = B * H * W;
  const long long items = rows * (vec4 ? C / 4 : C);
  long long blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t* xi = reinterpret_cast<const uint32_t*>(x);
  uint32_t* oi = reinterpret_cast<uint32_t*>(out);
  if (vec4)
    hipLaunchKernelGGL(qshift_kernel<4>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, xi,
                       oi, rows, static_cast<int>(H), static_cast<int>(W), static_cast<int>(C),
                       shift, static_cast<int>(g[0]), static_cast<int>(g[1]),
                       static_cast<int>(g[2]), static_cast<int>(g[3]));
  else
    hipLaunchKernelGGL(qshift_kernel<1>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, xi,
                       oi, rows, static_cast<int>(H), static_cast<int>(W), static_cast<int>(C),
                       shift, static_cast<int>(g[0]), static_cast<int>(g[1]),
                       static_cast<int>(g[2]), static_cast<int>(g[3]));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

const char* biwkv_status_string(int status) {
  switch (status) {
    case BIWKV_OK: return "ok";
    case BIWKV_ERR_NULL: return "a required pointer is NULL";
    case BIWKV_ERR_SHAPE: return "invalid shape (negative, too large, or T != H*W)";
    case BIWKV_ERR_DTYPE: return "unknown dtype (expected BIWKV_F32 or BIWKV_BF16)";
    case BIWKV_ERR_PARAM: return "invalid Q-Shift parameter (gamma outside [0, 1/4], or shift < 0 or > min(H, W))";
    case BIWKV_ERR_ALIAS: return "output overlaps an input";
    case BIWKV_ERR_ALIGN: return "pointer not aligned to its element size";
    case BIWKV_ERR_NO_DEVICE: return "no usable HIP device";
    case BIWKV_ERR_HIP: return "HIP runtime error (see biwkv_last_hip_error)";
    case BIWKV_ERR_UNSUPPORTED: return "sequence needs more chunks than can be resident at once";
    default: return "unknown status";
  }
}

int biwkv_last_hip_error(void) { return t_last_hip_error; }

int biwkv_stream_fault_flags(void* stream, uint32_t* flags) {
  if (!flags) return BIWKV_ERR_NULL;
  *flags = 0;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_scratch.find(std::make_pair(dev, stream));
  if (it == g_scratch.end() || !it->second) return BIWKV_OK;
  Counters c{};
  e = hipMemcpy(&c, it->second->ctr, sizeof(Counters), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  *flags = c.fault;
  if (c.fault) {
    const unsigned zero = 0;
    e = hipMemcpy(reinterpret_cast<char*>(it->second->ctr) + offsetof(Counters, fault), &zero,
                  sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
  }
  return BIWKV_OK;
}

int biwkv_version(void) { return 100; }

}  // extern "C"
