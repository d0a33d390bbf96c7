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

// ---------------------------------------------------------------------------------------------
// Bi-WKV chunk-scan kernel: one pass over HBM, both directions, per-row exchange of chunk sums
// ---------------------------------------------------------------------------------------------
//
// Scratch words (per launch): agg[row][chunk][dir][tile channel] and carry[...] as packed (l, mu),
// and one arrival counter per row. A chunk stores its aggregates, releases, and counts itself in;
// the chunk that arrives last in a row (it knows every aggregate of the row is published) acquires,
// scans the row in a fixed order, stores every chunk's exclusive carries, releases, and flags the
// row. The others wait for the flag, acquire, and read their two carries. The fixed scan order
// makes results bitwise reproducible; the waits only depend on chunks that hold tickets.

template <int DT, int V, int LW, int NW, bool FUSED>
__global__ void __launch_bounds__(NW * 64)
    biwkv_chunk_scan_kernel(BiwkvParams p) {
  using S = KV<DT, V>;
  using raw_t = typename S::raw_t;
  constexpr int TILE = 64 * V;
  constexpr int LWG = LW * NW;
  constexpr int HALF = LW / 2;
  constexpr int KQ = NW * 64 / TILE;  // threads per channel in the exchange passes
  static_assert(LW % 2 == 0, "LW must be even");
  static_assert(KQ * TILE == NW * 64, "channels must divide the workgroup");
  static_assert(KQ * 6 * TILE + 6 * TILE <= NW * 12 * TILE, "exchange scratch must fit the LDS block");
  constexpr int kPhaseFloats = NW * 12 * TILE;       // phase A/B sums
  constexpr int kSweepFloats = NW * HALF * TILE * 2;  // phase C: (alpha, beta) per token
  __shared__ float lds[kPhaseFloats > kSweepFloats ? kPhaseFloats : kSweepFloats];
  __shared__ float lds_own[2][3][TILE];  // this chunk's own forward / backward sums
  __shared__ unsigned sh_ticket, sh_flag, sh_epoch;
  float (*lds_agg)[6][TILE] = reinterpret_cast<float (*)[6][TILE]>(lds);
  float (*lds_pre)[3][TILE] = reinterpret_cast<float (*)[3][TILE]>(lds + NW * 6 * TILE);
  float (*lds_suf)[3][TILE] = reinterpret_cast<float (*)[3][TILE]>(lds + NW * 9 * TILE);
  // once every wavefront has taken its in-chunk sums, the block holds the exchange partials
  // and the final carries
  float (*lds_comb)[2][3][TILE] = reinterpret_cast<float (*)[2][3][TILE]>(lds);
  float (*lds_xy)[3][TILE] = reinterpret_cast<float (*)[3][TILE]>(lds + KQ * 6 * TILE);
  // phase C: per wavefront and token of the current half, (alpha, beta) of each channel
  using ab_t = typename AlphaBeta<V>::type;
  ab_t (*lds_ab)[HALF][64] = reinterpret_cast<ab_t (*)[HALF][64]>(lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (tid == 0) {
    sh_ticket = __hip_atomic_fetch_add(&p.ctr->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_epoch = __hip_atomic_load(&p.ctr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const unsigned epoch = sh_epoch;
  // A ticket beyond the grid can only come from a counter left non-zero by an earlier launch;
  // such a workgroup touches no data and only retires.
  const bool valid_ticket = sh_ticket < p.total;
  if (!valid_ticket && tid == 0)
    __hip_atomic_fetch_or(&p.ctr->fault, kFaultTicket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned ticket = valid_ticket ? sh_ticket : 0u;

  // Tickets enumerate rows in order and, inside a row, chunks in order.
  const int n = p.n_chunks;
  const int chunk = static_cast<int>(ticket % static_cast<unsigned>(n));
  const int row = static_cast<int>(ticket / static_cast<unsigned>(n));
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
  // U = u log2(e), grow = max(0, -D) (largest per-step growth), eU = 2^U (bounded).
  float D[V], lam[V], U[V], grow[V], eU[V];
  bool wide_lane = false;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const float wc = lane_on ? p.w[c0 + j] : 0.f;
    const float uc = lane_on ? p.u[c0 + j] : 0.f;
    D[j] = (wc / static_cast<float>(T)) * kLog2e;
    lam[j] = fast_exp2(-D[j]);
    U[j] = uc * kLog2e;
    grow[j] = fmaxf(-D[j], 0.f);
    eU[j] = fminf(fast_exp2(U[j]), 3.40282347e+38f);
    wide_lane = wide_lane || fabsf(D[j]) * static_cast<float>(LW - 1) > kFastRange || U[j] > kBonusRange;
  }
  // wide: some lane's decay range over the wavefront, or its bonus, exceeds what one exponent
  // reference per wavefront can hold; the wavefront then keeps one reference per token.
  const bool wide = __ballot(wide_lane) != 0ull;

  // ---- load this wavefront's tokens (coalesced along C) ----
  raw_t kr[LW], vr[LW];
  QShiftLane qs;
  int col = 0;
  if constexpr (FUSED) {
    qs.init(c0, p.H, p.W, T, p.shift, p.g1, p.g2, p.g3, p.g4);  // V channels share a group
    col = static_cast<int>(s_w % p.W);
  }
  const long long base = b * T * C + c0 + (FUSED ? qs.off * C : 0);
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const long long t = s_w + i;
    bool ok = lane_on && i < n_w;
    if constexpr (FUSED) {
      ok = ok && qs.valid(t, col);
      col = col + 1 == p.W ? 0 : col + 1;
    }
    const long long idx = base + t * C;
    kr[i] = ok ? S::load(p.k, idx) : S::zero();
    vr[i] = ok ? S::load(p.v, idx) : S::zero();
  }

  // ---- phase A: the wavefront's own sums: forward (anchored at its last token), backward
  //      (anchored at its first token) and backward over its second half (anchored at token HALF) --
  float kmax[V];
#pragma unroll
  for (int j = 0; j < V; ++j) kmax[j] = kNegInf;
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    if (i < n_w) {
      float kf[V];
      S::unpack(kr[i], kf);
#pragma unroll
      for (int j = 0; j < V; ++j) kmax[j] = fmaxf(kmax[j], kf[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) kmax[j] *= kLog2e;
  Agg af[V], ab[V], ab1[V];
  if (!wide) {
    // every weight of the wavefront is <= 1 against mw; p_i is formed once here and once in
    // phase C (against the final reference), so k and v are the only per-token state kept
    float pa[LW][V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float mw = n_w > 0 ? kmax[j] + grow[j] * static_cast<float>(n_w - 1) : kNegInf;
      af[j] = Agg{mw, 0.f, 0.f};
      ab[j] = Agg{mw, 0.f, 0.f};
      ab1[j] = Agg{mw, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      if (i < n_w) {
        float kf[V], vf[V];
        S::unpack(kr[i], kf);
        S::unpack(vr[i], vf);
#pragma unroll
        for (int j = 0; j < V; ++j) {
          pa[i][j] = fast_exp2(fmaf(kf[j], kLog2e, -af[j].m));
          af[j].F = fmaf(af[j].F, lam[j], pa[i][j] * vf[j]);
          af[j].G = fmaf(af[j].G, lam[j], pa[i][j]);
        }
      }
    }
#pragma unroll
    for (int i = LW - 1; i >= 0; --i) {
      if (i == HALF - 1) {
#pragma unroll
        for (int j = 0; j < V; ++j) ab1[j] = ab[j];
      }
      if (i < n_w) {
        float vf[V];
        S::unpack(vr[i], vf);
#pragma unroll
        for (int j = 0; j < V; ++j) {
          ab[j].F = fmaf(ab[j].F, lam[j], pa[i][j] * vf[j]);
          ab[j].G = fmaf(ab[j].G, lam[j], pa[i][j]);
        }
      }
    }
  } else {
    // Wide range: one decay step at a time, each sum kept against its own running maximum.
#pragma unroll
    for (int j = 0; j < V; ++j) af[j] = ab[j] = ab1[j] = agg_empty();
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
      if (i == HALF - 1) {
#pragma unroll
        for (int j = 0; j < V; ++j) ab1[j] = ab[j];
      }
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

  // ---- phase B: chunk sums (one wavefront per direction), publication, exchange ----
  const bool exchange = n > 1 && valid_ticket;
  const int fwd_wave = 0;
  const int bwd_wave = NW > 1 ? 1 : 0;
  const int G = p.group;
  const int grp_id = chunk / G;
  const int g_first = grp_id * G;
  const int g_end = g_first + G < n ? g_first + G : n;  // one past the group's last chunk
  const long long row_chunks = static_cast<long long>(row) * n;
  const long long row_groups = static_cast<long long>(row) * p.n_groups;
  auto agg_slot = [&](int ck, int dir, int ch) -> unsigned long long* {
    return p.agg + (((row_chunks + ck) * 2 + dir) * TILE + ch) * 2;
  };
  auto gagg_slot = [&](int gi, int dir, int ch) -> unsigned long long* {
    return p.gagg + (((row_groups + gi) * 2 + dir) * TILE + ch) * 2;
  };
  // token anchors: a forward sum is anchored at its last token, a backward sum at its first
  auto chunk_last = [&](long long ck) -> long long {
    const long long e = (ck + 1) * LWG;
    return (e < T ? e : T) - 1;
  };

  Agg own[V];
  if (wave == fwd_wave) {
#pragma unroll
    for (int j = 0; j < V; ++j) own[j] = agg_empty();
    for (int wv = 0; wv < NW; ++wv) {
      const long long rem_w = T - (s_chunk + static_cast<long long>(wv) * LW);
      const int nn = rem_w <= 0 ? 0 : (rem_w < LW ? static_cast<int>(rem_w) : LW);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int ch = lane * V + j;
        lds_pre[wv][0][ch] = own[j].m;
        lds_pre[wv][1][ch] = own[j].F;
        lds_pre[wv][2][ch] = own[j].G;
        const Agg a{lds_agg[wv][0][ch], lds_agg[wv][1][ch], lds_agg[wv][2][ch]};
        own[j] = agg_add(agg_shift(own[j], static_cast<float>(nn), D[j]), a);
      }
    }
    if (exchange) {
#pragma unroll
      for (int j = 0; j < V; ++j) slot_store(agg_slot(chunk, kFwd, lane * V + j), own[j], epoch);
    }
  }
  if (wave == bwd_wave) {
    Agg acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = agg_empty();
    for (int wv = NW - 1; wv >= 0; --wv) {
      const long long rem_w = T - (s_chunk + static_cast<long long>(wv) * LW);
      const int nn = rem_w <= 0 ? 0 : (rem_w < LW ? static_cast<int>(rem_w) : LW);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int ch = lane * V + j;
        lds_suf[wv][0][ch] = acc[j].m;
        lds_suf[wv][1][ch] = acc[j].F;
        lds_suf[wv][2][ch] = acc[j].G;
        const Agg a{lds_agg[wv][3][ch], lds_agg[wv][4][ch], lds_agg[wv][5][ch]};
        acc[j] = agg_add(a, agg_shift(acc[j], static_cast<float>(nn), D[j]));
      }
    }
    if (exchange) {
#pragma unroll
      for (int j = 0; j < V; ++j) slot_store(agg_slot(chunk, kBwd, lane * V + j), acc[j], epoch);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      lds_own[kBwd][0][ch] = acc[j].m;
      lds_own[kBwd][1][ch] = acc[j].F;
      lds_own[kBwd][2][ch] = acc[j].G;
    }
  }
  if (wave == fwd_wave) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      lds_own[kFwd][0][ch] = own[j].m;
      lds_own[kFwd][1][ch] = own[j].F;
      lds_own[kFwd][2][ch] = own[j].G;
    }
  }
  __syncthreads();

  // This wavefront's exclusive sums inside the chunk move to registers: LDS is reused below.
  Agg P[V], Q[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int ch = lane * V + j;
    P[j] = Agg{lds_pre[wave][0][ch], lds_pre[wave][1][ch], lds_pre[wave][2][ch]};
    Q[j] = Agg{lds_suf[wave][0][ch], lds_suf[wave][1][ch], lds_suf[wave][2][ch]};
  }
  __syncthreads();

  // Exchange passes: thread (xc, xk) folds every KQ-th slot of a fixed list for channel xc; the KQ
  // partials of a channel are then added in xk order, so the result is the same in every run.
  const int xc = tid % TILE;
  const int xk = tid / TILE;
  const int xcg = tile * TILE + xc;  // global channel of this thread in the exchange passes
  const float xD = (valid_ticket && xcg < C) ? (p.w[xcg] / static_cast<float>(T)) * kLog2e : 0.f;
  bool timed_out = false;
  // Reads the slots of entries xk, xk + KQ, ... in batches (the loads of a batch are all issued
  // before any is waited on) and folds them, in entry order, into a forward and a backward
  // partial.
  auto exchange_pass = [&](int count, auto&& entry, Agg* pf, Agg* pb) {
    *pf = agg_empty();
    *pb = agg_empty();
    for (int q0 = 0; xk + q0 * KQ < count; q0 += kSlotBatch) {
      unsigned long long wbuf[kSlotBatch][2];
#pragma unroll
      for (int q = 0; q < kSlotBatch; ++q) {
        const int e = xk + (q0 + q) * KQ;
        if (e < count) {
          int dir;
          float dist;
          slot_load(entry(e, &dir, &dist), wbuf[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < kSlotBatch; ++q) {
        const int e = xk + (q0 + q) * KQ;
        if (e < count) {
          unsigned spins = 0;
          while (!slot_ready(wbuf[q], epoch) && !timed_out) {
            if (++spins > kSpinLimit) {
              timed_out = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            int dir;
            float dist;
            slot_load(entry(e, &dir, &dist), wbuf[q]);
          }
          int dir;
          float dist;
          entry(e, &dir, &dist);
          const Agg a = agg_shift(slot_value(wbuf[q]), dist, xD);
          if (dir == kFwd)
            *pf = agg_add(*pf, a);
          else
            *pb = agg_add(*pb, a);
        }
      }
    }
  };
  auto store_partials = [&](Agg pf, Agg pb) {
    lds_comb[xk][kFwd][0][xc] = pf.m;
    lds_comb[xk][kFwd][1][xc] = pf.F;
    lds_comb[xk][kFwd][2][xc] = pf.G;
    lds_comb[xk][kBwd][0][xc] = pb.m;
    lds_comb[xk][kBwd][1][xc] = pb.F;
    lds_comb[xk][kBwd][2][xc] = pb.G;
  };
  auto combine = [&](int dir, int ch) -> Agg {
    Agg r = agg_empty();
#pragma unroll
    for (int k = 0; k < KQ; ++k)
      r = agg_add(r, Agg{lds_comb[k][dir][0][ch], lds_comb[k][dir][1][ch], lds_comb[k][dir][2][ch]});
    return r;
  };

  // Pass G: the last chunk of a group publishes the group's sums (forward anchored at the
  // group's last token, backward at its first token).
  if (exchange && chunk == g_end - 1) {
    const int mates = g_end - g_first - 1;
    const long long g_last_tok = chunk_last(chunk);
    const long long g_first_tok = static_cast<long long>(g_first) * LWG;
    auto entry = [&](int e, int* dir, float* dist) -> const unsigned long long* {
      if (e < mates) {  // forward sums of the earlier members
        const int ck = g_first + e;
        *dir = kFwd;
        *dist = static_cast<float>(g_last_tok - chunk_last(ck));
        return agg_slot(ck, kFwd, xc);
      }
      const int ck = g_first + (e - mates);  // backward sums of the earlier members
      *dir = kBwd;
      *dist = static_cast<float>(static_cast<long long>(ck) * LWG - g_first_tok);
      return agg_slot(ck, kBwd, xc);
    };
    Agg pf, pb;
    exchange_pass(2 * mates, entry, &pf, &pb);
    store_partials(pf, pb);
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int ch = lane * V + j;
        const Agg of{lds_own[kFwd][0][ch], lds_own[kFwd][1][ch], lds_own[kFwd][2][ch]};
        const Agg ob{lds_own[kBwd][0][ch], lds_own[kBwd][1][ch], lds_own[kBwd][2][ch]};
        const Agg tf = agg_add(combine(kFwd, ch), of);
        const Agg tb = agg_add(combine(kBwd, ch), agg_shift(ob, static_cast<float>(s_chunk - g_first_tok), D[j]));
        slot_store(gagg_slot(grp_id, kFwd, ch), tf, epoch);
        slot_store(gagg_slot(grp_id, kBwd, ch), tb, epoch);
      }
    }
    __syncthreads();
  }

  // Pass R: this chunk's carries from the group sums of the other groups and the chunk sums of
  // its own group. Entry order: forward group sums, forward member sums, backward member sums,
  // backward group sums.
  if (exchange) {
    const long long tgt_f = s_chunk - 1;             // forward carry anchor
    const long long tgt_b = s_chunk + n_chunk_tok;   // backward carry anchor
    const int nfg = grp_id;                          // earlier groups
    const int nfm = chunk - g_first;                 // earlier members
    const int nbm = g_end - 1 - chunk;               // later members
    const int nbg = p.n_groups - 1 - grp_id;         // later groups
    auto entry = [&](int e, int* dir, float* dist) -> const unsigned long long* {
      if (e < nfg) {
        *dir = kFwd;
        *dist = static_cast<float>(tgt_f - chunk_last(static_cast<long long>(e + 1) * G - 1));
        return gagg_slot(e, kFwd, xc);
      }
      e -= nfg;
      if (e < nfm) {
        const int ck = g_first + e;
        *dir = kFwd;
        *dist = static_cast<float>(tgt_f - chunk_last(ck));
        return agg_slot(ck, kFwd, xc);
      }
      e -= nfm;
      if (e < nbm) {
        const int ck = chunk + 1 + e;
        *dir = kBwd;
        *dist = static_cast<float>(static_cast<long long>(ck) * LWG - tgt_b);
        return agg_slot(ck, kBwd, xc);
      }
      e -= nbm;
      const int gi = grp_id + 1 + e;
      *dir = kBwd;
      *dist = static_cast<float>(static_cast<long long>(gi) * G * LWG - tgt_b);
      return gagg_slot(gi, kBwd, xc);
    };
    Agg pf, pb;
    exchange_pass(nfg + nfm + nbm + nbg, entry, &pf, &pb);
    store_partials(pf, pb);
  }
  if (timed_out)
    __hip_atomic_fetch_or(&p.ctr->fault, kFaultSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      const Agg x = exchange ? combine(kFwd, ch) : agg_empty();
      const Agg y = exchange ? combine(kBwd, ch) : agg_empty();
      lds_xy[0][0][ch] = x.m;
      lds_xy[0][1][ch] = x.F;
      lds_xy[0][2][ch] = x.G;
      lds_xy[1][0][ch] = y.m;
      lds_xy[1][1][ch] = y.F;
      lds_xy[1][2][ch] = y.G;
    }
  }
  __syncthreads();

  // ---- phase C: each wavefront sweeps each half of its tokens forward (a, c) then backward
  //      (b, d) and writes Eq. (7) ----
  Agg xw[V], yw[V];
  if (n_w > 0) {
    const float before = static_cast<float>(wave * LW);  // tokens between chunk start and s_w
    const float after = static_cast<float>(n_chunk_tok - wave * LW - n_w);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int ch = lane * V + j;
      const Agg X{lds_xy[0][0][ch], lds_xy[0][1][ch], lds_xy[0][2][ch]};
      const Agg Y{lds_xy[1][0][ch], lds_xy[1][1][ch], lds_xy[1][2][ch]};
      xw[j] = agg_add(agg_shift(X, before, D[j]), P[j]);  // a, c just before the first token
      yw[j] = agg_add(Q[j], agg_shift(Y, after, D[j]));   // b, d just after the last token
    }
  }
  __syncthreads();  // the carries are read: the LDS block now holds per-token (alpha, beta)
  if (n_w > 0) {
    using AB = AlphaBeta<V>;
    const int n1 = n_w > HALF ? n_w - HALF : 0;  // tokens in the second half
    if (!wide) {
      float M[V], A[V], Cs[V], Bs[V], Ds[V];
      float ph[HALF][V];  // p of each token of the current half, against M
#pragma unroll
      for (int j = 0; j < V; ++j) {
        // Every scaled term below is <= 1: local weights and carries all sit under M.
        const float top = fmaxf(fmaxf(kmax[j], xw[j].m), yw[j].m);
        M[j] = top + grow[j] * static_cast<float>(n_w - 1);
        const float sig = fast_exp2(kmax[j] - top);  // 2^{mw - M}
        const float sx = fast_exp2(xw[j].m - M[j]);
        A[j] = xw[j].F * sx;
        Cs[j] = xw[j].G * sx;
        // backward state entering the first half: the carry after the second half, plus the
        // second half's own sum (both under M)
        const float sy = fast_exp2(yw[j].m - M[j]);
        const float l1 = fast_exp2(-static_cast<float>(n1) * D[j]);
        Bs[j] = fmaf(yw[j].F * sy, l1, sig * ab1[j].F);
        Ds[j] = fmaf(yw[j].G * sy, l1, sig * ab1[j].G);
        yw[j].F *= sy;
        yw[j].G *= sy;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i0 = h * HALF;
        if (i0 < n_w) {
#pragma unroll
          for (int i = 0; i < HALF; ++i) {
            if (i0 + i < n_w) {
              float kf[V], vf[V];
              S::unpack(kr[i0 + i], kf);
              S::unpack(vr[i0 + i], vf);
              float al[V], be[V];
#pragma unroll
              for (int j = 0; j < V; ++j) {
                const float pi = fast_exp2(fmaf(kf[j], kLog2e, -M[j]));
                ph[i][j] = pi;
                const float e = fmaxf(pi * eU[j], 1.17549435e-38f);
                al[j] = fmaf(-Cs[j], vf[j], A[j]);
                be[j] = Cs[j] + e;
                A[j] = fmaf(A[j], lam[j], pi * vf[j]);
                Cs[j] = fmaf(Cs[j], lam[j], pi);
              }
              lds_ab[wave][i][lane] = AB::make(al, be);
            }
          }
          if (h == 1) {
#pragma unroll
            for (int j = 0; j < V; ++j) {
              Bs[j] = yw[j].F;
              Ds[j] = yw[j].G;
            }
          }
#pragma unroll
          for (int i = HALF - 1; i >= 0; --i) {
            if (i0 + i < n_w) {
              float vf[V], y[V], al[V], be[V];
              S::unpack(vr[i0 + i], vf);
              AB::split(lds_ab[wave][i][lane], al, be);
#pragma unroll
              for (int j = 0; j < V; ++j) {
                const float num = fmaf(-Ds[j], vf[j], al[j] + Bs[j]);
                const float den = be[j] + Ds[j];
                y[j] = fmaf(num, fast_rcp(den), vf[j]);
                const float pi = ph[i][j];
                Bs[j] = fmaf(Bs[j], lam[j], pi * vf[j]);
                Ds[j] = fmaf(Ds[j], lam[j], pi);
              }
              if (lane_on) store_out<V>(p.out, (b * T + s_w + i0 + i) * C + c0, y);
            }
          }
        }
      }
    } else {
      // Wide range: the forward state of each token is kept as (log-weight of c, a/c) in (be, al),
      // the backward state is stepped token by token, and Eq. (7) is formed against the largest
      // of the three exponents (forward, backward, self).
      Agg xs[V], ys[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        xs[j] = xw[j];
        ys[j] = agg_add(ab1[j], agg_shift(yw[j], static_cast<float>(n1), D[j]));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i0 = h * HALF;
        if (i0 < n_w) {
#pragma unroll
          for (int i = 0; i < HALF; ++i) {
            if (i0 + i < n_w) {
              float vf[V];
              S::unpack(vr[i0 + i], vf);
              float kf[V], al[V], be[V];
              S::unpack(kr[i0 + i], kf);
#pragma unroll
              for (int j = 0; j < V; ++j) {
                const bool any = xs[j].m != kNegInf && xs[j].G > 0.f;
                be[j] = any ? xs[j].m + fast_log2(xs[j].G) : kNegInf;
                al[j] = any ? xs[j].F * fast_rcp(xs[j].G) - vf[j] : 0.f;
                xs[j] = agg_add(agg_shift(xs[j], 1.f, D[j]), Agg{kf[j] * kLog2e, vf[j], 1.f});
              }
              lds_ab[wave][i][lane] = AB::make(al, be);
            }
          }
          if (h == 1) {
#pragma unroll
            for (int j = 0; j < V; ++j) ys[j] = yw[j];
          }
#pragma unroll
          for (int i = HALF - 1; i >= 0; --i) {
            if (i0 + i < n_w) {
              float kf[V], vf[V], y[V], al[V], be[V];
              S::unpack(kr[i0 + i], kf);
              S::unpack(vr[i0 + i], vf);
              AB::split(lds_ab[wave][i][lane], al, be);
#pragma unroll
              for (int j = 0; j < V; ++j) {
                const float kl = kf[j] * kLog2e;
                const float ks = kl + U[j];
                const float Mt = fmaxf(fmaxf(be[j], ys[j].m), ks);
                const float sa = fast_exp2(be[j] - Mt), sb = fast_exp2(ys[j].m - Mt);
                const float e = fast_exp2(ks - Mt);
                const float num = al[j] * sa + fmaf(-ys[j].G, vf[j], ys[j].F) * sb;
                const float den = sa + ys[j].G * sb + e;
                y[j] = fmaf(num, fast_rcp(den), vf[j]);
                ys[j] = agg_add(agg_shift(ys[j], 1.f, D[j]), Agg{kl, vf[j], 1.f});
              }
              if (lane_on) store_out<V>(p.out, (b * T + s_w + i0 + i) * C + c0, y);
            }
          }
        }
      }
    }
  }

  // ---- retire: the last workgroup of the launch resets the counters for the next launch ----
  __syncthreads();
  if (tid == 0) {
    const unsigned fin =
        __hip_atomic_fetch_add(&p.ctr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_flag = fin + 1u == p.total;
  }
  __syncthreads();
  if (sh_flag && tid == 0) {
    __hip_atomic_store(&p.ctr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p.ctr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&p.ctr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------------------------
// Bi-WKV whole-row kernel: one workgroup owns every token of a (batch, channel tile) row
// ---------------------------------------------------------------------------------------------
//
// Used when a row fits in one workgroup's registers (T * TILE elements, 64 tokens per lane at
// most). Lane (c, g) holds channel c of the tile and token group g (L consecutive tokens); the
// GROUPS = 1024 / TILE groups of a channel are combined by a Hillis-Steele scan in LDS, so no
// data leaves the workgroup between load and store. Each lane then sweeps its tokens in
// sub-blocks of 8: forward states (a, c) left to right, keeping (alpha, beta) = (a - c v, c +
// e^{u+k}) per token in LDS, then backward states (b, d) right to left, writing Eq. (7).

// Per-lane token storage of the whole-row kernel: bf16 k and v packed in one 32-bit register per
// token (k in the low half, v in the high half); fp32 k and v in two registers.
template <int DT, int L>
struct RowKV;

template <int L>
struct RowKV<BIWKV_BF16, L> {
  uint32_t r[L];
  __device__ __forceinline__ void load(const void* k, const void* v, long long idx, bool ok, int i) {
    uint32_t kb = 0u, vb = 0u;
    if (ok) {
      kb = static_cast<const uint16_t*>(k)[idx];
      vb = static_cast<const uint16_t*>(v)[idx];
    }
    r[i] = kb | (vb << 16);
  }
  __device__ __forceinline__ float k(int i) const { return __uint_as_float(r[i] << 16); }
  __device__ __forceinline__ float v(int i) const { return __uint_as_float(r[i] & 0xffff0000u); }
};

template <int L>
struct RowKV<BIWKV_F32, L> {
  float kk[L], vv[L];
  // idx must be in bounds even when !ok (the value is then replaced by zero)
  __device__ __forceinline__ void load(const void* k, const void* v, long long idx, bool ok, int i) {
    const float kx = static_cast<const float*>(k)[idx];
    const float vx = static_cast<const float*>(v)[idx];
    kk[i] = ok ? kx : 0.f;
    vv[i] = ok ? vx : 0.f;
  }
  __device__ __forceinline__ float k(int i) const { return kk[i]; }
  __device__ __forceinline__ float v(int i) const { return vv[i]; }
};

struct RowParams {
  const void* k;
  const void* v;
  const float* w;
  const float* u;
  float* out;
  long long T;
  int C;
  int n_rows;   // B * tiles
  int n_tiles;  // channel tiles per batch item
  int share;    // rows sharing one 128-byte line of k (mapped to one XCD), 1 = identity
  int H, W, shift, g1, g2, g3, g4;  // Q-Shift (fused entry only)
};

template <int DT, int TILE, int L, bool FUSED>
__global__ void __launch_bounds__(1024)
    biwkv_row_kernel(RowParams p) {
  constexpr int NT = 1024;
  constexpr int GROUPS = NT / TILE;
  constexpr int SB = 8;            // tokens per sub-block of the sweeps
  constexpr int NSB = L / SB;
  static_assert(L % SB == 0 && NT % TILE == 0, "bad row-kernel shape");
  constexpr int kScanFloats = 2 * 6 * NT;  // double-buffered (m, F, G) forward + backward
  constexpr int kSweepFloats = SB * NT * 2;
  __shared__ float lds[kScanFloats > kSweepFloats ? kScanFloats : kSweepFloats];
  float (*scan)[6][NT] = reinterpret_cast<float (*)[6][NT]>(lds);
  float2 (*lds_ab)[NT] = reinterpret_cast<float2 (*)[NT]>(lds);

  const int tid = threadIdx.x;
  const int c = tid % TILE;
  const int g = tid / TILE;
  // Rows whose tiles share a cache line of k run on one XCD (workgroup i runs on XCD i % 8), so
  // the line is fetched into that XCD's L2 once.
  int row = blockIdx.x;
  if (p.share > 1) {
    const int sh = p.share;
    row = ((row / (8 * sh)) * 8 + row % 8) * sh + (row / 8) % sh;
  }
  const int tile = row % p.n_tiles;
  const long long b = row / p.n_tiles;
  const long long T = p.T;
  const int C = p.C;
  const int ch = tile * TILE + c;
  const bool lane_on = ch < C;
  const long long s_g = static_cast<long long>(g) * L;
  const long long rem = T - s_g;
  const int n_g = rem <= 0 ? 0 : (rem < L ? static_cast<int>(rem) : L);

  const float wc = lane_on ? p.w[ch] : 0.f;
  const float uc = lane_on ? p.u[ch] : 0.f;
  const float D = (wc / static_cast<float>(T)) * kLog2e;
  const float lam = fast_exp2(-D);
  const float U = uc * kLog2e;
  const float grow = fmaxf(-D, 0.f);
  const float eU = fast_exp2(U);
  const bool wide_lane = fabsf(D) * static_cast<float>(L - 1) > kFastRange || U > kBonusRange ||
                         U < -kBonusRange;
  const bool wide = __ballot(wide_lane) != 0ull;

  // ---- load the lane's tokens ----
  RowKV<DT, L> kv;
  QShiftLane qs;
  int col = 0;
  if constexpr (FUSED) {
    qs.init(ch, p.H, p.W, T, p.shift, p.g1, p.g2, p.g3, p.g4);
    col = static_cast<int>(s_g % p.W);
  }
  // Loads are unconditional from an in-bounds address (the token itself when its shifted source
  // is outside the grid, element 0 for masked lanes) and masked values become zero: no
  // divergent branches around the loads.
  const long long row_base = b * T * C + (lane_on ? ch : 0);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool in_row = lane_on && i < n_g;
    const long long t = in_row ? s_g + i : 0;
    bool ok = in_row;
    long long src = t;
    if constexpr (FUSED) {
      const bool shifted = in_row && qs.valid(t, col);  // masked tokens keep t = 0, unshifted
      ok = shifted;
      src = shifted ? t + qs.off : t;
      col = col + 1 == p.W ? 0 : col + 1;
    }
    kv.load(p.k, p.v, (in_row ? row_base : 0) + src * C, ok, i);
  }

  // ---- phase A: lane sums (forward anchored at its last token, backward at its first) and, per
  //      sub-block, the backward sum of everything after it inside the lane ----
  float kmax = kNegInf;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (i < n_g) {
      kmax = fmaxf(kmax, kv.k(i));
    }
  }
  kmax *= kLog2e;
  Agg af, ab;
  Agg cap[NSB];  // cap[q]: backward sum of tokens >= (q + 1) * SB, anchored at (q + 1) * SB
  if (!wide) {
    const float mw = n_g > 0 ? kmax + grow * static_cast<float>(n_g - 1) : kNegInf;
    af = Agg{mw, 0.f, 0.f};
    float bF[NSB], bG[NSB];  // backward sum of each sub-block, anchored at its first token
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      bF[q] = bG[q] = 0.f;
      float r = 1.f;  // lam^{i - q SB}
#pragma unroll
      for (int i = q * SB; i < (q + 1) * SB; ++i) {
        if (i < n_g) {
          const float kf = kv.k(i), vf = kv.v(i);
          const float pi = fast_exp2(fmaf(kf, kLog2e, -mw));
          af.F = fmaf(af.F, lam, pi * vf);
          af.G = fmaf(af.G, lam, pi);
          const float pr = pi * r;
          bF[q] = fmaf(pr, vf, bF[q]);
          bG[q] += pr;
          r *= lam;
        }
      }
    }
    const float lsb = fast_exp2(-static_cast<float>(SB) * D);  // lam^SB
    float cF = 0.f, cG = 0.f;
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      cap[q] = Agg{mw, cF, cG};
      cF = fmaf(cF, lsb, bF[q]);
      cG = fmaf(cG, lsb, bG[q]);
    }
    ab = Agg{mw, cF, cG};
  } else {
    // Wide range: one decay step at a time, each sum against its own running maximum.
    af = agg_empty();
    Agg bs[NSB];
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      bs[q] = agg_empty();
#pragma unroll
      for (int i = (q + 1) * SB - 1; i >= q * SB; --i) {
        if (i < n_g) {
          bs[q] = agg_add(agg_shift(bs[q], 1.f, D), Agg{kv.k(i) * kLog2e, kv.v(i), 1.f});
        }
      }
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < n_g) {
        af = agg_add(agg_shift(af, 1.f, D), Agg{kv.k(i) * kLog2e, kv.v(i), 1.f});
      }
    }
    Agg cs = agg_empty();
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      cap[q] = cs;
      cs = agg_add(bs[q], agg_shift(cs, static_cast<float>(SB), D));
    }
    ab = cs;
  }

  // ---- inclusive scans over the groups of each channel (Hillis-Steele, fixed order) ----
  int cur = 0;
  scan[0][0][tid] = af.m;
  scan[0][1][tid] = af.F;
  scan[0][2][tid] = af.G;
  scan[0][3][tid] = ab.m;
  scan[0][4][tid] = ab.F;
  scan[0][5][tid] = ab.G;
  __syncthreads();
  auto last_tok = [&](int gi) -> long long {  // last token of group gi (clipped to the row)
    const long long e = static_cast<long long>(gi + 1) * L;
    return (e < T ? e : T) - 1;
  };
#pragma unroll
  for (int d = 1; d < GROUPS; d *= 2) {
    Agg f{scan[cur][0][tid], scan[cur][1][tid], scan[cur][2][tid]};
    Agg bk{scan[cur][3][tid], scan[cur][4][tid], scan[cur][5][tid]};
    if (g >= d) {
      const int o = tid - d * TILE;
      const Agg pf{scan[cur][0][o], scan[cur][1][o], scan[cur][2][o]};
      f = agg_add(agg_shift(pf, static_cast<float>(last_tok(g) - last_tok(g - d)), D), f);
    }
    if (g + d < GROUPS) {
      const int o = tid + d * TILE;
      const Agg pb{scan[cur][3][o], scan[cur][4][o], scan[cur][5][o]};
      bk = agg_add(bk, agg_shift(pb, static_cast<float>(d * L), D));
    }
    cur ^= 1;
    scan[cur][0][tid] = f.m;
    scan[cur][1][tid] = f.F;
    scan[cur][2][tid] = f.G;
    scan[cur][3][tid] = bk.m;
    scan[cur][4][tid] = bk.F;
    scan[cur][5][tid] = bk.G;
    __syncthreads();
  }
  // exclusive carries: forward sum of the earlier groups (anchored just before this lane's first
  // token), backward sum of the later groups (anchored just after its last token)
  Agg X = agg_empty(), Y = agg_empty();
  if (g > 0) {
    const int o = tid - TILE;
    X = Agg{scan[cur][0][o], scan[cur][1][o], scan[cur][2][o]};
  }
  if (g + 1 < GROUPS) {
    const int o = tid + TILE;
    Y = Agg{scan[cur][3][o], scan[cur][4][o], scan[cur][5][o]};
  }
  __syncthreads();  // the scan buffer becomes the (alpha, beta) buffer

  // ---- phase C: sweep each sub-block forward, then backward, writing Eq. (7) ----
  if (n_g > 0) {
    float* outp = p.out + b * T * C + ch;
    if (!wide) {
      // every scaled term is <= 1 against M
      const float top = fmaxf(fmaxf(kmax, X.m), Y.m);
      const float M = top + grow * static_cast<float>(n_g - 1);
      const float sig = fast_exp2(kmax - top);  // 2^{mw - M}
      const float sx = fast_exp2(X.m - M), sy = fast_exp2(Y.m - M);
      float A = X.F * sx, Cs = X.G * sx;
      const float YF = Y.F * sy, YG = Y.G * sy;
#pragma unroll
      for (int q = 0; q < NSB; ++q) {
        if (q * SB < n_g) {
          float ph[SB];
#pragma unroll
          for (int i = 0; i < SB; ++i) {
            const int t = q * SB + i;
            if (t < n_g) {
              const float kf = kv.k(t), vf = kv.v(t);
              const float pi = fast_exp2(fmaf(kf, kLog2e, -M));
              ph[i] = pi;
              const float al = fmaf(-Cs, vf, A);
              const float be = fmaf(pi, eU, Cs);
              lds_ab[i][tid] = make_float2(al, be);
              A = fmaf(A, lam, pi * vf);
              Cs = fmaf(Cs, lam, pi);
            }
          }
          // backward state entering this sub-block from the right: the later sub-blocks of the
          // lane plus the later groups
          const int end = (q + 1) * SB < n_g ? (q + 1) * SB : n_g;
          const float lr = fast_exp2(-static_cast<float>(n_g - end) * D);
          float Bs = fmaf(YF, lr, sig * cap[q].F);
          float Ds = fmaf(YG, lr, sig * cap[q].G);
#pragma unroll
          for (int i = SB - 1; i >= 0; --i) {
            const int t = q * SB + i;
            if (t < n_g) {
              const float vf = kv.v(t);
              const float2 ab2 = lds_ab[i][tid];
              const float num = fmaf(-Ds, vf, ab2.x + Bs);
              const float den = fmaxf(ab2.y + Ds, 1.17549435e-38f);
              const float y = fmaf(num, fast_rcp(den), vf);
              if (lane_on) outp[(s_g + t) * C] = y;
              Bs = fmaf(Bs, lam, ph[i] * vf);
              Ds = fmaf(Ds, lam, ph[i]);
            }
          }
        }
      }
    } else {
      Agg xs = X;
#pragma unroll
      for (int q = 0; q < NSB; ++q) {
        if (q * SB < n_g) {
#pragma unroll
          for (int i = 0; i < SB; ++i) {
            const int t = q * SB + i;
            if (t < n_g) {
              const float kf = kv.k(t), vf = kv.v(t);
              const bool any = xs.m != kNegInf && xs.G > 0.f;
              const float be = any ? xs.m + fast_log2(xs.G) : kNegInf;
              const float al = any ? xs.F * fast_rcp(xs.G) - vf : 0.f;
              lds_ab[i][tid] = make_float2(al, be);
              xs = agg_add(agg_shift(xs, 1.f, D), Agg{kf * kLog2e, vf, 1.f});
            }
          }
          const int end = (q + 1) * SB < n_g ? (q + 1) * SB : n_g;
          Agg ys = agg_add(cap[q], agg_shift(Y, static_cast<float>(n_g - end), D));
#pragma unroll
          for (int i = SB - 1; i >= 0; --i) {
            const int t = q * SB + i;
            if (t < n_g) {
              const float kf = kv.k(t), vf = kv.v(t);
              const float2 ab2 = lds_ab[i][tid];
              const float kl = kf * kLog2e;
              const float ks = kl + U;
              const float Mt = fmaxf(fmaxf(ab2.y, ys.m), ks);
              const float sa = fast_exp2(ab2.y - Mt), sb = fast_exp2(ys.m - Mt);
              const float e = fast_exp2(ks - Mt);
              const float num = ab2.x * sa + fmaf(-ys.G, vf, ys.F) * sb;
              const float den = sa + ys.G * sb + e;
              const float y = fmaf(num, fast_rcp(den), vf);
              if (lane_on) outp[(s_g + t) * C] = y;
              ys = agg_add(agg_shift(ys, 1.f, D), Agg{kl, vf, 1.f});
            }
          }
        }
      }
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
  std::vector<void*> retired;  // outgrown buffers; pending launches may still use them
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

template <typename Tp>
int grow_zeroed(Tp** buf, long long* cap, long long need, long long min_cap, hipStream_t st,
                std::vector<void*>* retired) {
  if (*cap >= need) return BIWKV_OK;
  long long want = *cap ? *cap : min_cap;
  while (want < need) want *= 2;
  const long long words = (want * static_cast<long long>(sizeof(Tp)) + 7) / 8;
  unsigned long long* fresh = nullptr;
  hipError_t e = hipMalloc(&fresh, static_cast<size_t>(words) * 8);
  if (e != hipSuccess) return hip_fail(e);
  long long blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, fresh, words);
  e = hipGetLastError();
  if (e != hipSuccess) {
    (void)hipFree(fresh);
    return hip_fail(e);
  }
  if (*buf) retired->push_back(*buf);
  *buf = reinterpret_cast<Tp*>(fresh);
  *cap = want;
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
  int rc = grow_zeroed(&sc->slots, &sc->slot_words, words, 1ll << 16, st, &sc->retired);
  if (rc) return rc;
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
  // Exchange groups: about sqrt(n) chunks each, so a chunk reads at most (groups - 1) group sums
  // and (group - 1) member sums; both passes must fit the per-thread slot budget.
  constexpr int KQ = kNW * 64 / TILE;
  int64_t group = 1;
  while (group * group < n_chunks) ++group;
  const int64_t n_groups = (n_chunks + group - 1) / group;
  const int64_t budget = static_cast<int64_t>(KQ) * kMaxSlotsPerThread;
  if ((n_groups - 1) + (group - 1) > budget || 2 * (group - 1) > budget) return BIWKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  int cap = 0;
  int rc = resident_capacity(dev, kfn, kNW * 64, &cap);
  if (rc) return rc;
  if (n_chunks > cap) return BIWKV_ERR_UNSUPPORTED;
  StreamScratch* sc = nullptr;
  const long long agg_words = total * 2 * TILE * 2;
  const long long gagg_words = B * n_tiles * n_groups * 2 * TILE * 2;
  rc = get_scratch(dev, stream, agg_words + gagg_words, &sc);
  if (rc) return rc;
  prm.n_tiles = static_cast<int>(n_tiles);
  prm.n_chunks = static_cast<int>(n_chunks);
  prm.total = static_cast<unsigned>(total);
  prm.group = static_cast<int>(group);
  prm.n_groups = static_cast<int>(n_groups);
  prm.agg = sc->slots;
  prm.gagg = sc->slots + agg_words;
  prm.ctr = sc->ctr;
  hipLaunchKernelGGL((biwkv_chunk_scan_kernel<DT, V, kLW, kNW, FUSED>),
                     dim3(static_cast<unsigned>(total)), dim3(kNW * 64), 0,
                     static_cast<hipStream_t>(stream), prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

template <int DT, int TILE, int L, bool FUSED>
int launch_row(const BiwkvParams& bp, int64_t B, void* stream) {
  RowParams rp{};
  rp.k = bp.k;
  rp.v = bp.v;
  rp.w = bp.w;
  rp.u = bp.u;
  rp.out = bp.out;
  rp.T = bp.T;
  rp.C = bp.C;
  rp.H = bp.H;
  rp.W = bp.W;
  rp.shift = bp.shift;
  rp.g1 = bp.g1;
  rp.g2 = bp.g2;
  rp.g3 = bp.g3;
  rp.g4 = bp.g4;
  const int64_t n_tiles = (bp.C + TILE - 1) / TILE;
  const int64_t n_rows = B * n_tiles;
  if (n_rows > 0x7FFFFFFFll) return BIWKV_ERR_SHAPE;
  const int elem = DT == BIWKV_F32 ? 4 : 2;
  int share = 128 / (TILE * elem);
  if (share < 1 || n_rows % (8 * share) != 0) share = 1;
  rp.n_rows = static_cast<int>(n_rows);
  rp.n_tiles = static_cast<int>(n_tiles);
  rp.share = share;
  hipLaunchKernelGGL((biwkv_row_kernel<DT, TILE, L, FUSED>), dim3(static_cast<unsigned>(n_rows)),
                     dim3(1024), 0, static_cast<hipStream_t>(stream), rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// Whole-row kernel when the sequence fits one workgroup (64 tokens per lane for bf16 k/v, 32 for
// fp32), else the chunked kernel with the cross-workgroup exchange. Returns 1 if not handled.
template <int DT, bool FUSED>
int try_row(const BiwkvParams& bp, int64_t B, void* stream) {
  const long long T = bp.T;
  if (T <= 256) return launch_row<DT, 64, 16, FUSED>(bp, B, stream);
  if (T <= 512) return launch_row<DT, 64, 32, FUSED>(bp, B, stream);
  if constexpr (DT == BIWKV_BF16) {
    if (T <= 1024) return launch_row<DT, 64, 64, FUSED>(bp, B, stream);
    if (T <= 2048) return launch_row<DT, 16, 32, FUSED>(bp, B, stream);
    if (T <= 4096) return launch_row<DT, 16, 64, FUSED>(bp, B, stream);
  } else {
    if (T <= 1024) return launch_row<DT, 16, 16, FUSED>(bp, B, stream);
    if (T <= 2048) return launch_row<DT, 16, 32, FUSED>(bp, B, stream);
  }
  return 1;
}

template <bool FUSED>
int dispatch_biwkv(BiwkvParams prm, int64_t B, int dtype, bool vec2, int dev, void* stream) {
  const int rrc = dtype == BIWKV_F32 ? try_row<BIWKV_F32, FUSED>(prm, B, stream)
                                     : try_row<BIWKV_BF16, FUSED>(prm, B, stream);
  if (rrc != 1) return rrc;
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
