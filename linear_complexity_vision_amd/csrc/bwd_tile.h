// Bi-WKV backward in one launch: the gradients of Eq. (5) (see backward.h for the formulas) with
// the tile kernel's work split.
#pragma once

#include "backward.h"
#include "row_kernel.h"

namespace {

// ---------------------------------------------------------------------------------------------
// A workgroup of NT threads owns one chunk (GROUPS * L tokens) of a (batch, 64-channel tile) row;
// lane (c, g) holds channel c at L consecutive tokens, and keeps k, v and the upstream gradient g
// of those tokens in registers from load to store, with the output y and log2 of Eq. (5)'s
// denominator once they are known. Two rounds of the same three steps:
//   1. lane sums of (e^k v, e^k) in prefix and suffix form, scanned over the workgroup's groups
//      and exchanged with the other chunks of the row; a sweep over the lane's tokens gives y and
//      log2 D at every token;
//   2. lane sums of (q, r) = (g, g y) / D, scanned and exchanged the same way; a sweep gives dv,
//      dk and the dw terms at every token (the four states of the first round are formed again
//      on the way), and the du terms.
// A row of one chunk runs in one launch. A longer row runs in three launches of the same kernel,
// each reading the chunk sums the one before wrote, so no workgroup waits for another:
//   stage 1 writes every chunk's round-1 sums;
//   stage 2 folds the other chunks' round-1 sums into its carries, sweeps round 1, and writes
//     every chunk's round-2 sums;
//   stage 3 does both rounds with the carries of both, and writes dk, dv and the dw, du terms.
// The dw and du terms of a workgroup are folded per channel in LDS, in a fixed order; a last
// kernel folds those of the row's chunks.
//
// Position-free sums. A prefix sum anchored at token p is 2^{-pD} sum_{t<=p} 2^{x_t + tD} y_t and a
// suffix sum 2^{pD} sum_{t>=p} 2^{x_t - tD} y_t (D = w log2(e) / T), so a term's exponent is fixed
// once and sums over any set of tokens are plain sums: the scans and the exchange move no
// exponent. A sum is an aggregate (m, F, G) = (F, G) 2^m. In the round-1 sweep the running sums
// of (e^k v, e^k) take each term at their running maximum (two exp2 per term), so their exponent
// is that of their largest term and the denominator of y is always formed against a term it
// contains. In the round-2 sweep a running sum keeps one exponent per sub-block of SB tokens (the
// larger of its own and the sub-block's largest term) and each term costs one exp2. The products
// b Qpre, d Rpre, a Qsuf, c Rsuf of dw pair a prefix with a suffix sum at the same token, so
// their position factors cancel and leave 2^{2D}.
//
// Precision: lane and sub-block sums form their terms against the largest of them, so a term
// more than 2^-126 below it is lost; exponents inside a sub-block differ by the keys' spread plus
// (SB - 1) |D|. The round-2 factors e^{k_i} 2^{exponent of a running sum} are at most
// 2^{2 (SB - 1) |D|} (a weight p_ti <= 1 times the sub-block's spread of positions), finite for
// |w| / T below about 20 (every workload has |w| / T < 0.05).
// ---------------------------------------------------------------------------------------------

constexpr int kBtTile = 64;  // channels per tile (one wavefront)
constexpr int kBtSB = 4;     // tokens per sub-block of the sweeps
constexpr int kBwdLane = 8;  // tokens per lane of the tile kernel (its fast / wide vote)
// Cache policy of the k, v, g loads: the default one, unlike the forward's streaming loads. The
// stages read the same k, v (and g) one after the other, and 134 MB of them at B=4, T=4096,
// C=1024 fit the 256 MB memory-side cache, so later stages hit it (173 against 193 us there).
constexpr int kBtLoadPolicy = 0;

struct BwdTileParams {
  const void* k;
  const void* v;
  const float* w;
  const float* u;
  const float* g;
  float* dk;
  float* dv;
  float* pw;  // dw terms per (batch item, chunk, channel), before the factor -lam / T
  float* pu;  // du terms per (batch item, chunk, channel)
  float* sums1;   // round-1 chunk sums: [row][chunk][dir][64][3] floats (m, F, G)
  float* sums2;   // round-2 chunk sums, same layout
  float* carry1;  // round-1 carries of every chunk (earlier chunks, later chunks), same layout
  float* carry2;  // round-2 carries, same layout
  long long T;
  int C;
  int n_tiles;   // channel tiles per batch item
  int n_chunks;  // chunks per row
  // single launch (bwd_one_kernel): the exchange between the chunks of a row
  Counters* ctr;              // epoch block (n_chunks > 1)
  unsigned long long* slots;  // [round][row][chunk][dir][64] tagged (m, F, G) words
  unsigned* row_fail;         // per row: the launch's tag when a wait of that row ran out
  unsigned total;             // workgroups of the launch
  unsigned spin_limit;        // polls of a peer's slot before the row is handed to the fallback
  // single launch: rows [0, xcd_rows) run every chunk on one XCD and exchange through its L2
  // (blocks go to the n_xcd XCDs round robin); 0 keeps the plain order
  int xcd_rows, n_xcd;
};

// Makes register values opaque to the compiler (no instruction), so that values derived from them
// in one phase are formed again in the next instead of being kept live in between.
template <int N>
__device__ __forceinline__ void bt_fence(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}
__device__ __forceinline__ void bt_fence(float& x) { asm volatile("" : "+v"(x)); }

// Per-lane token storage: bf16 k and v packed in one register (k low, v high), fp32 in two; empty
// slots (past the row, or a masked channel) hold k = -inf, v = 0.
template <int DT, int L>
struct BtKV;
template <int L>
struct BtKV<BIWKV_BF16, L> {
  uint32_t r[L];
  __device__ __forceinline__ float k(int i) const { return __uint_as_float(r[i] << 16); }
  __device__ __forceinline__ float v(int i) const { return __uint_as_float(r[i] & 0xffff0000u); }
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int i = 0; i < L; ++i) asm volatile("" : "+v"(r[i]));
  }
  template <int POL>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t km, __amdgpu_buffer_rsrc_t vm, uint32_t off, int i) {
    const uint32_t kx = __builtin_amdgcn_raw_buffer_load_b16(km, off, 0, POL);
    const uint32_t vx = __builtin_amdgcn_raw_buffer_load_b16(vm, off, 0, POL);
    r[i] = kx | (vx << 16);
  }
  __device__ __forceinline__ void empty(int i) { r[i] = (r[i] & 0xffff0000u) | 0xff80u; }  // k = -inf
};
template <int L>
struct BtKV<BIWKV_F32, L> {
  float kk[L], vv[L];
  __device__ __forceinline__ float k(int i) const { return kk[i]; }
  __device__ __forceinline__ float v(int i) const { return vv[i]; }
  __device__ __forceinline__ void fence() {
    bt_fence(kk);
    bt_fence(vv);
  }
  template <int POL>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t km, __amdgpu_buffer_rsrc_t vm, uint32_t off, int i) {
    kk[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(km, off, 0, POL));
    vv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vm, off, 0, POL));
  }
  __device__ __forceinline__ void empty(int i) { kk[i] = kNegInf; }
};

// The larger of an aggregate's exponent and mx, and the aggregate rescaled to it.
__device__ __forceinline__ Agg bt_rebase(Agg a, float mx) {
  const float r = fmaxf(a.m, mx);
  const float s = fast_exp2(a.m - r);
  return Agg{r, a.F * s, a.G * s};
}

// An aggregate of SB terms 2^{x_i} (F_i, G_i) against their largest exponent (empty: kEmptyM).
template <int SB>
__device__ __forceinline__ Agg bt_block(const float (&x)[SB], const float (&F)[SB], const float (&G)[SB]) {
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < SB; ++i) mx = fmaxf(mx, x[i]);
  const float ref = mx == kNegInf ? 0.f : mx;
  Agg a{mx == kNegInf ? kEmptyM : mx, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SB; ++i) {
    const float e = fast_exp2(x[i] - ref);
    a.F = fmaf(e, F[i], a.F);
    a.G = fmaf(e, G[i], a.G);
  }
  return a;
}

template <int NT>
constexpr int kBtRedFloats = 6 * (NT / kBtTile) * (kBtTile + 1);

// LDS of the backward tile kernel.
template <int NT>
struct BtShared {
  float sw[4][kBtSB][NT];          // sweep records of one sub-block (wide form)
  float red[kBtRedFloats<NT>];     // lane sums (group-major)
  float xy[kBtRedFloats<NT>];      // carries
  float dch[kBtTile];              // D of each channel of the tile
  float fold[2][NT / kBtTile][kBtTile];  // dw and du terms of each lane
};

// Lane constants: lane (c, g) of the workgroup for chunk `chunk` of row `row` holds channel ch of
// batch item bi at the tokens [s_g, s_g + L).
struct BtLane {
  int row, chunk, bi, ch, c, g;
  bool on;
  long long s_g;  // first token
  float D, U;           // w log2(e) / T and u log2(e) of the channel (0 when masked)
};

template <int L, int NT>
__device__ __forceinline__ BtLane bt_lane_index(const BwdTileParams& p, unsigned unit) {
  constexpr int CT = (NT / kBtTile) * L;
  BtLane ln;
  const int tid = threadIdx.x;
  ln.c = tid % kBtTile;
  ln.g = tid / kBtTile;
  const unsigned nc = static_cast<unsigned>(p.n_chunks);
  if (unit < static_cast<unsigned>(p.xcd_rows) * nc) {
    // block `unit` runs on XCD unit % n_xcd: XCD x takes rows x, x + n_xcd, ... whole, in order
    const unsigned nx = static_cast<unsigned>(p.n_xcd);
    const unsigned s = __builtin_amdgcn_readfirstlane(unit / nx);
    const unsigned x = unit - s * nx;
    const unsigned rg = __builtin_amdgcn_readfirstlane(s / nc);
    ln.row = static_cast<int>(rg * nx + x);
    ln.chunk = static_cast<int>(s - rg * nc);
  } else {
    ln.row = __builtin_amdgcn_readfirstlane(unit / nc);
    ln.chunk = static_cast<int>(unit) - ln.row * p.n_chunks;
  }
  ln.bi = __builtin_amdgcn_readfirstlane(ln.row / p.n_tiles);
  const int tile = ln.row - ln.bi * p.n_tiles;
  ln.ch = tile * kBtTile + ln.c;
  ln.on = ln.ch < p.C;
  ln.s_g = static_cast<long long>(ln.chunk) * CT + static_cast<long long>(ln.g) * L;
  return ln;
}

// The lane's D and U from its w and u (a masked lane passes 0: D = U = 0).
__device__ __forceinline__ void bt_lane_params(BtLane& ln, long long T, float wc, float uc) {
  ln.D = (wc / static_cast<float>(T)) * kLog2e;
  ln.U = uc * kLog2e;
}

template <int L, int NT>
__device__ __forceinline__ BtLane bt_lane(const BwdTileParams& p, unsigned unit) {
  BtLane ln = bt_lane_index<L, NT>(p, unit);
  bt_lane_params(ln, p.T, ln.on ? p.w[ln.ch] : 0.f, ln.on ? p.u[ln.ch] : 0.f);
  return ln;
}

// Loads N consecutive tokens of a wavefront, starting at t0 (the same for every lane), of batch
// item bi: k and v, and g when gg is given. Each token goes through a buffer resource over the
// rest of the batch item (a uniform base, so scalar registers) and the lane's channel offset, so
// one vector register addresses every token; tokens past the row read 0 and are then marked empty
// (k = -inf), masked channels read 0. The host keeps a batch item below 2^31 bytes.
template <int DT, int N, int POL = kBtLoadPolicy>
__device__ __forceinline__ void bt_load(const BwdTileParams& p, int bi, long long t0, int ch, bool on,
                                        BtKV<DT, N>& kv, float* gg) {
  constexpr int ES = DT == BIWKV_F32 ? 4 : 2;
  const long long plane = p.T * p.C;  // elements of one batch item
  const char* kb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.k) + static_cast<unsigned long long>(bi) * plane * ES));
  const char* vb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.v) + static_cast<unsigned long long>(bi) * plane * ES));
  const char* gb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.g) + static_cast<unsigned long long>(bi) * plane * 4));
  const int t0u = __builtin_amdgcn_readfirstlane(static_cast<int>(t0));
  const int rb = p.C * ES, rg = p.C * 4;                     // bytes per token
  const int avail = static_cast<int>(plane * ES), availg = static_cast<int>(plane * 4);
  const uint32_t off = on ? static_cast<uint32_t>(ch) * ES : kOutOfRange;
  const uint32_t offg = on ? static_cast<uint32_t>(ch) * 4 : kOutOfRange;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int a = (t0u + i) * rb;  // below 2^31: T < 2^31 / (4 C) and the row's padding
    const int left = avail - a;
    const uint32_t n = static_cast<uint32_t>(left > 0 ? left : 0);
    kv.template load<POL>(make_rsrc(kb + a, n), make_rsrc(vb + a, n), off, i);
    if (gg) {
      const int ag = (t0u + i) * rg;
      const int lg = availg - ag;
      gg[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          make_rsrc(gb + ag, static_cast<uint32_t>(lg > 0 ? lg : 0)), offg, 0, POL));
    }
  }
  if (t0u + N > p.T) {  // uniform: only wavefronts at the end of a row
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (t0u + i >= p.T) kv.empty(i);
  }
}

// bf16 k and v of N consecutive tokens from t0, as channel pairs (C even, 4-byte aligned k and v):
// lanes 2j and 2j + 1 read channels (2j, 2j + 1) as one 32-bit word, at even and odd tokens, as
// the forward tile kernel does (RowKVPair: prepare(q) then gives each lane its own channel). Half
// the load instructions of 16-bit loads, and each lands in its final register. Tokens past the
// row are marked empty.
template <int N, int POL = kBtLoadPolicy>
__device__ __forceinline__ void bt_load_pairs(const BwdTileParams& p, int bi, long long t0, int ch, bool on,
                                              RowKVPair<N>& kv, float* gg) {
  const long long plane = p.T * p.C;
  const char* kb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.k) + static_cast<unsigned long long>(bi) * plane * 2));
  const char* vb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.v) + static_cast<unsigned long long>(bi) * plane * 2));
  const int t0u = __builtin_amdgcn_readfirstlane(static_cast<int>(t0));
  const int rb = p.C * 2;                     // bytes per token
  const int avail = static_cast<int>(plane * 2);
  const int odd = ch & 1;                     // tiles start at even channels
  const uint32_t off = on ? static_cast<uint32_t>(odd * rb + (ch - odd) * 2) : kOutOfRange;
#pragma unroll
  for (int m = 0; m < N / 2; ++m) {
    const int a = (t0u + 2 * m) * rb;  // below 2^31 (host check)
    const int left = avail - a;
    const uint32_t n = static_cast<uint32_t>(left > 0 ? left : 0);
    kv.kk[m] = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(kb + a, n), off, 0, POL);
    kv.vv[m] = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(vb + a, n), off, 0, POL);
  }
  if (gg) {  // the upstream gradient: fp32, each lane its own channel
    const char* gb = reinterpret_cast<const char*>(
        uniform_u64(reinterpret_cast<unsigned long long>(p.g) + static_cast<unsigned long long>(bi) * plane * 4));
    const int rg = p.C * 4, availg = static_cast<int>(plane * 4);
    const uint32_t offg = on ? static_cast<uint32_t>(ch) * 4 : kOutOfRange;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ag = (t0u + i) * rg;
      const int lg = availg - ag;
      gg[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          make_rsrc(gb + ag, static_cast<uint32_t>(lg > 0 ? lg : 0)), offg, 0, POL));
    }
  }
  if (t0u + N > p.T) kv.pad(static_cast<int>(p.T - t0u), odd);  // only wavefronts at a row's end
}

// Stores dv and dk of token t (the same for every lane of the wavefront) of batch item bi through
// a buffer resource over the rest of the batch item and the lane's channel offset: tokens past
// the row and masked channels fall out of range and the hardware drops them, so no lane branches.
__device__ __forceinline__ void bt_store(const BwdTileParams& p, int bi, long long t, int ch, bool on, float dv,
                                         float dk) {
  const long long plane = p.T * p.C;
  const unsigned long long item = static_cast<unsigned long long>(bi) * plane * 4;
  const int tu = __builtin_amdgcn_readfirstlane(static_cast<int>(t));
  const int a = tu * p.C * 4;  // below 2^31 (host check)
  const int left = static_cast<int>(plane * 4) - a;
  const uint32_t n = static_cast<uint32_t>(left > 0 ? left : 0);
  const uint32_t off = on ? static_cast<uint32_t>(ch) * 4 : kOutOfRange;
  const char* dvb = reinterpret_cast<const char*>(uniform_u64(reinterpret_cast<unsigned long long>(p.dv) + item));
  const char* dkb = reinterpret_cast<const char*>(uniform_u64(reinterpret_cast<unsigned long long>(p.dk) + item));
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dv), make_rsrc(dvb + a, n), off, 0, kStream);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dk), make_rsrc(dkb + a, n), off, 0, kStream);
}

enum : int { kBtLocal = 0, kBtProduce = 1, kBtConsume = 2 };

// Carries of the lanes from their sums. In: the lane's forward sum f and backward sum b. Out: X,
// the sum over every token of the row before the lane, and Y, over every token after it.
// Position-free sums (ANCHORED false) are plain sums in a fixed order; anchored sums (f at the
// lane's last slot, b at its first token; X anchored just before the lane, Y just after it) move
// by n tokens with exponent shifts of n D. The lane sums go to LDS; the first wavefront, one lane
// per channel, scans the channel's GROUPS groups in order (work-efficient: the other wavefronts
// wait at the barrier while the CU's other workgroup uses the vector unit), and the carries come
// back through LDS. MODE:
//   kBtLocal: the row is one chunk, the scan starts empty;
//   kBtProduce: the chunk's sums (forward at its last slot, backward at its first token) go to
//     sums for a later launch, and X, Y are not formed;
//   kBtConsume: the scan starts from the chunk's carries (the sums of the row's earlier and later
//     chunks, formed by bwd_carry_kernel from the sums an earlier launch wrote).
template <int NT, int L, bool ANCHORED, int MODE>
__device__ __forceinline__ void bt_carries(Agg f, Agg b, Agg& X, Agg& Y, BtShared<NT>* sh, float* sums,
                                           const BwdTileParams& p, const BtLane& ln) {
  constexpr int GROUPS = NT / kBtTile;
  constexpr int PAD = kBtTile + 1;
  constexpr int RS = GROUPS * PAD;
  float* red = sh->red;
  float* xy = sh->xy;
  const int wi = ln.g * PAD + ln.c;
  red[0 * RS + wi] = f.m;
  red[1 * RS + wi] = f.F;
  red[2 * RS + wi] = f.G;
  red[3 * RS + wi] = b.m;
  red[4 * RS + wi] = b.F;
  red[5 * RS + wi] = b.G;
  __syncthreads();
  if (ln.g == 0) {  // the first wavefront: lane c scans channel c
    const int c = ln.c;
    const float Dt = ANCHORED ? ln.D : 0.f;
    const float step = static_cast<float>(L);
    const int nch = p.n_chunks, chunk = ln.chunk;
    float* rs = sums + static_cast<size_t>(ln.row) * nch * 2 * kBtTile * 3;
    auto slot = [&](int ck, int dir) { return rs + (static_cast<size_t>(ck * 2 + dir) * kBtTile + c) * 3; };
    Agg x = row_empty(), y = row_empty();
    if constexpr (MODE == kBtConsume) {
      const float* cf = slot(chunk, kFwd);
      const float* cb = slot(chunk, kBwd);
      x = Agg{cf[0], cf[1], cf[2]};  // anchored just before the chunk: before group 0
      y = Agg{cb[0], cb[1], cb[2]};  // just after the chunk: after the last group
    }
#pragma unroll
    for (int gi = 0; gi < GROUPS; ++gi) {
      const int o = gi * PAD + c;
      if constexpr (MODE != kBtProduce) {
        xy[0 * RS + o] = x.m;
        xy[1 * RS + o] = x.F;
        xy[2 * RS + o] = x.G;
      }
      // from just before group gi to its last slot, where its own sum is anchored
      x = agg_add_f(agg_shift(x, step, Dt), Agg{red[0 * RS + o], red[1 * RS + o], red[2 * RS + o]});
    }
#pragma unroll
    for (int gi = GROUPS - 1; gi >= 0; --gi) {
      const int o = gi * PAD + c;
      if constexpr (MODE != kBtProduce) {
        xy[3 * RS + o] = y.m;
        xy[4 * RS + o] = y.F;
        xy[5 * RS + o] = y.G;
      }
      y = agg_add_f(Agg{red[3 * RS + o], red[4 * RS + o], red[5 * RS + o]}, agg_shift(y, step, Dt));
    }
    if constexpr (MODE == kBtProduce) {  // the chunk's own sums
      float* o = slot(chunk, kFwd);
      o[0] = x.m;
      o[1] = x.F;
      o[2] = x.G;
      o = slot(chunk, kBwd);
      o[0] = y.m;
      o[1] = y.F;
      o[2] = y.G;
    }
  }
  if constexpr (MODE != kBtProduce) {
    __syncthreads();
    X = Agg{xy[0 * RS + wi], xy[1 * RS + wi], xy[2 * RS + wi]};
    Y = Agg{xy[3 * RS + wi], xy[4 * RS + wi], xy[5 * RS + wi]};
  }
}

// ---------------------------------------------------------------------------------------------
// Single launch: the chunks of a row exchange their sums through slots, one round at a time.
// A chunk's sum is published as three tagged 64-bit words (m, F, G), each carrying the launch's
// tag in its upper half, so a reader accepts a slot without a fence once every tag matches. (The
// round-2 sums are signed, so the forward's (log-weight, mean) pair does not apply.)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void bt_slot_put(unsigned long long* s, Agg a, unsigned tag) {
  const unsigned long long t = static_cast<unsigned long long>(tag) << 32;
  __hip_atomic_store(s, t | __float_as_uint(a.m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(s + 1, t | __float_as_uint(a.F), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(s + 2, t | __float_as_uint(a.G), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void bt_slot_get(const unsigned long long* s, unsigned long long (&w)[3]) {
#pragma unroll
  for (int i = 0; i < 3; ++i) w[i] = __hip_atomic_load(s + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool bt_slot_ready(const unsigned long long (&w)[3], unsigned tag) {
  return static_cast<unsigned>(w[0] >> 32) == tag && static_cast<unsigned>(w[1] >> 32) == tag &&
         static_cast<unsigned>(w[2] >> 32) == tag;
}
// The same words through the L2 of the workgroup's own XCD, for rows whose chunks all run on one
// XCD: plain stores and non-temporal loads, which the CU's L1 does not keep (as the forward tile
// kernel's slot_store_l2 / slot_load_l2). `rs` spans the slot array, `off` is the byte offset.
__device__ __forceinline__ void bt_slot_put_l2(__amdgpu_buffer_rsrc_t rs, uint32_t off, Agg a, unsigned tag) {
  const unsigned long long t = static_cast<unsigned long long>(tag) << 32;
  slot_word_l2(rs, off, t | __float_as_uint(a.m));
  slot_word_l2(rs, off + 8u, t | __float_as_uint(a.F));
  slot_word_l2(rs, off + 16u, t | __float_as_uint(a.G));
}
__device__ __forceinline__ void bt_slot_get_l2(__amdgpu_buffer_rsrc_t rs, uint32_t off, unsigned long long (&w)[3]) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const slot_u2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8u * i, 0, kSlotL2Load);
    w[i] = static_cast<unsigned long long>(x.x) | (static_cast<unsigned long long>(x.y) << 32);
  }
}
__device__ __forceinline__ Agg bt_slot_value(const unsigned long long (&w)[3]) {
  return Agg{__uint_as_float(static_cast<unsigned>(w[0])), __uint_as_float(static_cast<unsigned>(w[1])),
             __uint_as_float(static_cast<unsigned>(w[2]))};
}

// Counts a workgroup out of a single launch once none of its wavefronts reads a slot again; the
// last one resets the count and moves the epoch on for the next launch on the stream (whose tags
// then differ from every slot written so far).
__device__ __forceinline__ unsigned bt_retire_begin(const BwdTileParams& p) {
  return __hip_atomic_fetch_add(&p.ctr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void bt_retire_end(const BwdTileParams& p, unsigned fin) {
  if (fin != kNotRetiring && fin + 1u == p.total) {
    __hip_atomic_store(&p.ctr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&p.ctr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Carries of the lanes from their sums in a single launch (round rnd of the row's exchange). In
// and out as bt_carries. The first wavefront scans each channel's groups from empty (the lanes'
// carries inside the chunk) and publishes the chunk's sums (forward at its last slot, backward at
// its first token); then every wavefront takes a share of the row's other chunks (wavefront g
// folds entries g, g + GROUPS, ... in order: the forward sums of the earlier chunks, then the
// backward sums of the later ones), the shares are folded in wavefront order, and each lane's
// carry is the chunk's carry moved to the lane plus its carry inside the chunk. The result does
// not depend on arrival order. Returns true (for the whole workgroup) when a wait ran out; X and Y
// are then not formed.
template <int NT, int L, bool ANCHORED>
__device__ __forceinline__ bool bt_exchange(Agg f, Agg b, Agg& X, Agg& Y, BtShared<NT>* sh, const BwdTileParams& p,
                            const BtLane& ln, int rnd, const unsigned* sh_tag) {
  constexpr int GROUPS = NT / kBtTile;
  constexpr int PAD = kBtTile + 1;
  constexpr int RS = GROUPS * PAD;
  constexpr int CT = GROUPS * L;
  float* red = sh->red;
  float* xy = sh->xy;
  float* part = &sh->sw[0][0][0];  // [GROUPS][6][64]: the wavefronts' shares (the sweep records
                                   // of the wide form are not live here)
  const int wi = ln.g * PAD + ln.c;
  red[0 * RS + wi] = f.m;
  red[1 * RS + wi] = f.F;
  red[2 * RS + wi] = f.G;
  red[3 * RS + wi] = b.m;
  red[4 * RS + wi] = b.F;
  red[5 * RS + wi] = b.G;
  __syncthreads();
  const unsigned tag = __builtin_amdgcn_readfirstlane(*sh_tag);  // written before the first barrier
  const int c = ln.c;
  const float Dt = ANCHORED ? ln.D : 0.f;  // lane (c, g) holds channel c of the tile
  const float step = static_cast<float>(L);
  const int nch = p.n_chunks, chunk = ln.chunk;
  unsigned long long* rs =
      p.slots + ((static_cast<size_t>(rnd) * p.total + static_cast<size_t>(ln.row) * nch) * 2 * kBtTile) * 3;
  auto slot = [&](int ck, int dir) { return rs + (static_cast<size_t>(ck * 2 + dir) * kBtTile + c) * 3; };
  // rows whose chunks all run on one XCD exchange through its L2 (byte offsets into the slot
  // array, which the host keeps below 4 GiB for them)
  const bool local = ln.row < p.xcd_rows;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.slots, 0xFFFFFFFFu);
  auto soff = [&](const unsigned long long* sp) { return static_cast<uint32_t>((sp - p.slots) * 8); };
  auto put = [&](unsigned long long* sp, Agg a) {
    if (local)
      bt_slot_put_l2(srs, soff(sp), a, tag);
    else
      bt_slot_put(sp, a, tag);
  };
  auto get = [&](const unsigned long long* sp, unsigned long long (&w)[3]) {
    if (local)
      bt_slot_get_l2(srs, soff(sp), w);
    else
      bt_slot_get(sp, w);
  };
  if (ln.g == 0) {
    Agg x = row_empty(), y = row_empty();
#pragma unroll
    for (int gi = 0; gi < GROUPS; ++gi) {
      const int o = gi * PAD + c;
      xy[0 * RS + o] = x.m;
      xy[1 * RS + o] = x.F;
      xy[2 * RS + o] = x.G;
      x = agg_add_f(agg_shift(x, step, Dt), Agg{red[0 * RS + o], red[1 * RS + o], red[2 * RS + o]});
    }
#pragma unroll
    for (int gi = GROUPS - 1; gi >= 0; --gi) {
      const int o = gi * PAD + c;
      xy[3 * RS + o] = y.m;
      xy[4 * RS + o] = y.F;
      xy[5 * RS + o] = y.G;
      y = agg_add_f(Agg{red[3 * RS + o], red[4 * RS + o], red[5 * RS + o]}, agg_shift(y, step, Dt));
    }
    if (nch > 1) {
      put(slot(chunk, kFwd), x);
      put(slot(chunk, kBwd), y);
    }
  }
  // this wavefront's share of the other chunks' sums, moved to the chunk's carry anchors (just
  // before its first token, just after its last slot)
  Agg pf = row_empty(), pb = row_empty();
  bool timed_out = false;
  const int nf = chunk, ne = nch - 1;
  // A lane polls up to EB entries together: every poll round reissues the loads of the entries
  // not yet seen, so a batch costs one round trip after its last peer publishes.
  constexpr int EB = 2;
  for (int e0 = ln.g; e0 < ne; e0 += EB * GROUPS) {
    unsigned long long w[EB][3];
    bool ok[EB];
    auto entry = [&](int j) {
      const int e = e0 + j * GROUPS;
      return slot(e < nf ? e : e + 1, e < nf ? kFwd : kBwd);
    };
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      ok[j] = e0 + j * GROUPS >= ne;  // no entry: nothing to wait for
      if (!ok[j] && p.spin_limit != 0) get(entry(j), w[j]);
    }
    bool all = true;
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      ok[j] = ok[j] || (p.spin_limit != 0 && bt_slot_ready(w[j], tag));
      all = all && ok[j];
    }
    for (unsigned spins = 1; !all && spins < p.spin_limit; ++spins) {
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int j = 0; j < EB; ++j)
        if (!ok[j]) get(entry(j), w[j]);
      all = true;
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        ok[j] = ok[j] || bt_slot_ready(w[j], tag);
        all = all && ok[j];
      }
    }
    if (!all) timed_out = true;
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int e = e0 + j * GROUPS;
      if (e >= ne || !ok[j]) continue;
      const bool fwd = e < nf;
      const int ck = fwd ? e : e + 1;
      const float dist = static_cast<float>(fwd ? (chunk - 1 - ck) : (ck - chunk - 1)) * CT;
      const Agg a = agg_shift(bt_slot_value(w[j]), dist, Dt);
      if (fwd)
        pf = agg_add_f(pf, a);
      else
        pb = agg_add_f(pb, a);
    }
  }
  {
    float* q = part + ln.g * 6 * kBtTile + c;
    q[0 * kBtTile] = pf.m;
    q[1 * kBtTile] = pf.F;
    q[2 * kBtTile] = pf.G;
    q[3 * kBtTile] = pb.m;
    q[4 * kBtTile] = pb.F;
    q[5 * kBtTile] = pb.G;
  }
  if (block_any(timed_out)) return true;
  if (ln.g == 0) {
    Agg cf = row_empty(), cb = row_empty();
#pragma unroll
    for (int gi = 0; gi < GROUPS; ++gi) {
      const float* q = part + gi * 6 * kBtTile + c;
      cf = agg_add_f(cf, Agg{q[0 * kBtTile], q[1 * kBtTile], q[2 * kBtTile]});
      cb = agg_add_f(cb, Agg{q[3 * kBtTile], q[4 * kBtTile], q[5 * kBtTile]});
    }
#pragma unroll
    for (int gi = 0; gi < GROUPS; ++gi) {
      const int o = gi * PAD + c;
      const Agg x = agg_add_f(agg_shift(cf, static_cast<float>(gi) * step, Dt),
                              Agg{xy[0 * RS + o], xy[1 * RS + o], xy[2 * RS + o]});
      const Agg y = agg_add_f(Agg{xy[3 * RS + o], xy[4 * RS + o], xy[5 * RS + o]},
                              agg_shift(cb, static_cast<float>(GROUPS - 1 - gi) * step, Dt));
      xy[0 * RS + o] = x.m;
      xy[1 * RS + o] = x.F;
      xy[2 * RS + o] = x.G;
      xy[3 * RS + o] = y.m;
      xy[4 * RS + o] = y.F;
      xy[5 * RS + o] = y.G;
    }
  }
  __syncthreads();
  X = Agg{xy[0 * RS + wi], xy[1 * RS + wi], xy[2 * RS + wi]};
  Y = Agg{xy[3 * RS + wi], xy[4 * RS + wi], xy[5 * RS + wi]};
  return false;
}

// ---------------------------------------------------------------------------------------------
// Wide form (any w, u): position-free sums, running maxima. Returns the lane's (dw, du) terms.
// Out of line: it needs more registers than the fast form, and keeping it apart gives it its own
// allocation. It reads the parameters through the kernel's argument pointer.
// ---------------------------------------------------------------------------------------------
template <int DT, int L, int NT, int STAGE>
__device__ __noinline__ float4 bt_body_wide(const BwdTileParams* args, BtShared<NT>* sh, const unsigned* sh_tag,
                                            unsigned unit) {
  constexpr int SB = kBtSB;
  constexpr int NSB = L / SB;
  constexpr int MODE = STAGE == 0 ? kBtLocal : kBtConsume;  // when a round's carries are formed
  const float4 failed = make_float4(0.f, 0.f, 1.f, 0.f);  // STAGE 4: a wait ran out
  const BwdTileParams p = *args;
  const BtLane lnv = bt_lane<L, NT>(p, unit);
  const int tid = threadIdx.x;
  const bool on = lnv.on;
  const long long s_g = lnv.s_g;
  const float D = lnv.D, U = lnv.U;
  auto& sw = sh->sw;
  BtKV<DT, L> kv;
  float gg[L];
  // a single launch reads k, v and g once: streaming loads
  bt_load<DT, L, STAGE == 4 ? kStream : kBtLoadPolicy>(p, lnv.bi, lnv.s_g, lnv.ch, lnv.on, kv, gg);
  // token position times D, exact for t < 2^24
  float Dp = D;  // the copy positions are formed from, made opaque between phases
  auto tD = [&](int i) { return static_cast<float>(s_g + i) * Dp; };
  auto kl = [&](int i) { return kv.k(i) * kLog2e; };  // -inf in empty slots

  // ---- round 1: lane sums of (e^k v, e^k), prefix form and (per sub-block) suffix form ----
  Agg lane_f = row_empty();
  Agg cap1[NSB];  // suffix-form sum of the lane's sub-blocks after q
  {
    Agg sbs[NSB];
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float xp[SB], xs[SB], vv[SB], one[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        xp[i] = kl(j) + tD(j);
        xs[i] = kl(j) - tD(j);
        vv[i] = kv.v(j);
        one[i] = 1.f;
      }
      lane_f = agg_add_f(lane_f, bt_block<SB>(xp, vv, one));
      sbs[q] = bt_block<SB>(xs, vv, one);
      __builtin_amdgcn_sched_barrier(0);  // one sub-block at a time (bounded live values)
    }
    Agg run = row_empty();
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      cap1[q] = run;
      run = agg_add_f(sbs[q], run);
    }
    Agg Xc, Yc;
    if constexpr (STAGE == 1) {
      bt_carries<NT, L, false, kBtProduce>(lane_f, run, Xc, Yc, sh, p.sums1, p, lnv);
      return make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (STAGE == 4) {
      if (bt_exchange<NT, L, false>(lane_f, run, Xc, Yc, sh, p, lnv, 0, sh_tag)) return failed;
    } else {
      bt_carries<NT, L, false, MODE>(lane_f, run, Xc, Yc, sh, p.carry1, p, lnv);
    }
    lane_f = Xc;
    // from here cap1[q] is the suffix-form sum of every token after sub-block q
#pragma unroll
    for (int q = 0; q < NSB; ++q) cap1[q] = agg_add_f(Yc, cap1[q]);
  }
  const Agg X1 = lane_f;  // prefix-form sum of every token before the lane
  // values derived from the stored tokens are formed again in each phase, not kept live
  auto fence_all = [&]() {
    kv.fence();
    bt_fence(gg);
    bt_fence(Dp);
  };
  fence_all();

  // ---- round 1 sweep: y and log2 D at every token ----
  float y[L], nl[L];  // output and -log2 of the denominator (-inf in empty slots)
  {
    Agg A = X1;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        sw[0][i][tid] = A.m;
        sw[1][i][tid] = A.F;
        sw[2][i][tid] = A.G;
        A = agg_add_f(A, Agg{kl(j) + tD(j), kv.v(j), 1.f});
      }
      Agg Bs = cap1[q];
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int j = q * SB + i;
        const float t = static_cast<float>(s_g + j);
        const float am = sw[0][i][tid], aF = sw[1][i][tid], aG = sw[2][i][tid];
        // Eq. (7): (a + b + e^{u+k} v) / (c + d + e^{u+k}); a, c anchored at t - 1, b, d at t + 1
        const float xa = am - (t - 1.f) * D, xb = Bs.m + (t + 1.f) * D, xe = kl(j) + U;
        const float M = fmaxf(fmaxf(xa, xb), xe);
        const float sa = fast_exp2(xa - M), sb = fast_exp2(xb - M), se = fast_exp2(xe - M);
        const float vj = kv.v(j);
        const float num = fmaf(aF, sa, fmaf(Bs.F, sb, se * vj));
        const float den = fmaf(aG, sa, fmaf(Bs.G, sb, se));  // >= 1: M is a term's exponent
        const bool live = xe != kNegInf;
        y[j] = live ? num * fast_rcp(den) : 0.f;
        nl[j] = live ? -(M + fast_log2(den)) : kNegInf;
        Bs = agg_add_f(Bs, Agg{kl(j) - tD(j), vj, 1.f});
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  fence_all();
  bt_fence(y);
  bt_fence(nl);

  // ---- round 2: lane sums of (q, r) = (g, g y) 2^{-log2 D}; du terms ----
  Agg X2;
  Agg cap2[NSB];
  float du = 0.f;
  {
    Agg lane2 = row_empty();
    Agg sbs[NSB];
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float xp[SB], xs[SB], qq[SB], rr[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        xp[i] = nl[j] + tD(j);
        xs[i] = nl[j] - tD(j);
        qq[i] = gg[j];
        rr[i] = gg[j] * y[j];
        // e^{u+k} (q v - r) = p_tt g (v - y)
        du = fmaf(fast_exp2(U + kl(j) + nl[j]) * gg[j], kv.v(j) - y[j], du);
      }
      lane2 = agg_add_f(lane2, bt_block<SB>(xp, qq, rr));
      sbs[q] = bt_block<SB>(xs, qq, rr);
      __builtin_amdgcn_sched_barrier(0);
    }
    Agg run = row_empty();
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      cap2[q] = run;
      run = agg_add_f(sbs[q], run);
    }
    Agg Y2;
    if constexpr (STAGE == 2) {
      bt_carries<NT, L, false, kBtProduce>(lane2, run, X2, Y2, sh, p.sums2, p, lnv);
      return make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (STAGE == 4) {
      if (bt_exchange<NT, L, false>(lane2, run, X2, Y2, sh, p, lnv, 1, sh_tag)) return failed;
    } else {
      bt_carries<NT, L, false, MODE>(lane2, run, X2, Y2, sh, p.carry2, p, lnv);
    }
#pragma unroll
    for (int q = 0; q < NSB; ++q) cap2[q] = agg_add_f(Y2, cap2[q]);
  }

  fence_all();
  bt_fence(y);
  bt_fence(nl);

  // ---- round 2 sweep: dv, dk and the dw terms ----
  float dw1 = 0.f, dw2 = 0.f;  // sum b Qpre - d Rpre (against 2^e1), sum a Qsuf - c Rsuf (2^e2)
  float e1 = kEmptyM, e2 = kEmptyM;
  {
    Agg A = X1, QA = X2;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float mx = kNegInf, mq = kNegInf;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        mx = fmaxf(mx, kl(q * SB + i) + tD(q * SB + i));
        mq = fmaxf(mq, nl[q * SB + i] + tD(q * SB + i));
      }
      // one exponent per running sum for the whole sub-block
      A = bt_rebase(A, mx);
      QA = bt_rebase(QA, mq);
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        sw[0][i][tid] = A.F;
        sw[1][i][tid] = A.G;
        sw[2][i][tid] = QA.F;
        sw[3][i][tid] = QA.G;
        const float e = fast_exp2(kl(j) + tD(j) - A.m);
        A.F = fmaf(e, kv.v(j), A.F);
        A.G += e;
        const float eq = fast_exp2(nl[j] + tD(j) - QA.m);
        QA.F = fmaf(eq, gg[j], QA.F);
        QA.G = fmaf(eq, gg[j] * y[j], QA.G);
      }
      float ms = kNegInf, mqs = kNegInf;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        ms = fmaxf(ms, kl(q * SB + i) - tD(q * SB + i));
        mqs = fmaxf(mqs, nl[q * SB + i] - tD(q * SB + i));
      }
      Agg Bs = bt_rebase(cap1[q], ms), QB = bt_rebase(cap2[q], mqs);
      float s1 = 0.f, s2 = 0.f;  // against 2^{Bs.m + QA.m} and 2^{A.m + QB.m}
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int j = q * SB + i;
        const long long tt = s_g + j;
        const float t = static_cast<float>(tt);
        const float aF = sw[0][i][tid], aG = sw[1][i][tid];
        const float qF = sw[2][i][tid], qG = sw[3][i][tid];
        // b Qpre - d Rpre and a Qsuf - c Rsuf at this token (their position factors cancel)
        s1 = fmaf(Bs.F, qF, fmaf(-Bs.G, qG, s1));
        s2 = fmaf(aF, QB.F, fmaf(-aG, QB.G, s2));
        // e^{k} (Qpre + Qsuf + e^u q) and the same over r
        const float k2 = kl(j);
        const float c1 = qF != 0.f || qG != 0.f ? fast_exp2(QA.m - (t - 1.f) * D + k2) : 0.f;
        const float c2 = QB.F != 0.f || QB.G != 0.f ? fast_exp2(QB.m + (t + 1.f) * D + k2) : 0.f;
        const float c3 = fast_exp2(U + nl[j] + k2);
        const float dvj = fmaf(qF, c1, fmaf(QB.F, c2, gg[j] * c3));
        const float rj = fmaf(qG, c1, fmaf(QB.G, c2, gg[j] * y[j] * c3));
        const float dkj = fmaf(kv.v(j), dvj, -rj);
        bt_store(p, lnv.bi, tt, lnv.ch, on, dvj, dkj);
        const float e = fast_exp2(k2 - tD(j) - Bs.m);
        Bs.F = fmaf(e, kv.v(j), Bs.F);
        Bs.G += e;
        const float eq = fast_exp2(nl[j] - tD(j) - QB.m);
        QB.F = fmaf(eq, gg[j], QB.F);
        QB.G = fmaf(eq, gg[j] * y[j], QB.G);
      }
      // fold the sub-block's dw sums into the lane's, at the larger exponent
      const float f1 = Bs.m + QA.m, f2 = A.m + QB.m;
      const float m1 = fmaxf(e1, f1), m2 = fmaxf(e2, f2);
      dw1 = fmaf(dw1, fast_exp2(e1 - m1), s1 * fast_exp2(f1 - m1));
      dw2 = fmaf(dw2, fast_exp2(e2 - m2), s2 * fast_exp2(f2 - m2));
      e1 = m1;
      e2 = m2;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the lane's dw terms: (sum1 2^{e1} + sum2 2^{e2}) 2^{2D}
  float dw = 0.f;
  if (e1 > kEmptyM) dw += dw1 * fast_exp2(e1 + 2.f * D);
  if (e2 > kEmptyM) dw += dw2 * fast_exp2(e2 + 2.f * D);

  return make_float4(dw, du, 0.f, 0.f);
}

// ---------------------------------------------------------------------------------------------
// Fast form: the lane's terms are formed against one reference per lane and the states of Eq. (6)
// move one token with a multiply by lam = 2^{-D}, as in the forward tile kernel's fast form.
// Round 1 keys k, values (v, 1); round 2 keys -log2 D_t, values (g, g y). Lane sums are anchored
// (forward at the lane's last slot, backward at its first token) and the scan and exchange move
// them with exponent shifts. Valid while the growth across a lane, |D| (L - 1), stays within
// kBtFastRange: every state is then at least 2^{-2 span} of its largest term, so the products of
// a round-1 and a round-2 state in dw stay normal numbers; and while |u| log2(e) <= kBonusRange.
// ---------------------------------------------------------------------------------------------
constexpr float kBtFastRange = 24.f;

// Whether a channel needs the wide form. Every kernel of a backward call takes the same vote over
// the 64 channels of a tile, so all stages of a row use the same form.
template <int L>
__device__ __forceinline__ bool bt_wide_lane(float D, float U) {
  return fabsf(D) * static_cast<float>(L - 1) > kBtFastRange || fabsf(U) > kBonusRange;
}

template <int DT, int L, int NT, int STAGE, bool PAIR>
__device__ __forceinline__ float2 bt_body_fast(const BwdTileParams& p, const BtLane& ln, BtShared<NT>* sh) {
  constexpr int SB = kBtSB;
  constexpr int NSB = L / SB;
  constexpr int MODE = STAGE == 0 ? kBtLocal : kBtConsume;  // when a round's carries are formed
  const float D = ln.D, U = ln.U;
  const float lam = fast_exp2(-D);
  const float span = fmaxf(-D, 0.f) * static_cast<float>(L - 1);  // largest growth inside a lane
  const float eU = fast_exp2(U);
  std::conditional_t<PAIR, RowKVPair<L>, BtKV<DT, L>> kv;
  float gg[L];
  if constexpr (PAIR) {
    bt_load_pairs<L>(p, ln.bi, ln.s_g, ln.ch, ln.on, kv, gg);
#pragma unroll
    for (int q = 0; q < L / 8; ++q) kv.prepare(q);
  } else {
    bt_load<DT, L>(p, ln.bi, ln.s_g, ln.ch, ln.on, kv, gg);
  }
  auto kl = [&](int i) { return kv.k(i) * kLog2e; };  // -inf in empty slots

  // ---- round 1 lane sums (against 2^{kmax + span}) and the caps: backward sums of the lane's
  //      sub-blocks after q, anchored at the first token after sub-block q ----
  float kmax = kNegInf;
#pragma unroll
  for (int i = 0; i < L; ++i) kmax = fmaxf(kmax, kl(i));
  float capF[NSB], capG[NSB];
  Agg X, Y;
  {
    const float ref = kmax == kNegInf ? 0.f : kmax + span;
    float pp[L];
#pragma unroll
    for (int i = 0; i < L; ++i) pp[i] = fast_exp2(kl(i) - ref);
    float fF = 0.f, fG = 0.f, cF = 0.f, cG = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      fF = fmaf(fF, lam, pp[i] * kv.v(i));
      fG = fmaf(fG, lam, pp[i]);
    }
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      capF[q] = cF;
      capG[q] = cG;
#pragma unroll
      for (int i = (q + 1) * SB - 1; i >= q * SB; --i) {
        cF = fmaf(cF, lam, pp[i] * kv.v(i));
        cG = fmaf(cG, lam, pp[i]);
      }
    }
    const float m = kmax == kNegInf ? kEmptyM : ref;
    if constexpr (STAGE == 1) {
      bt_carries<NT, L, true, kBtProduce>(Agg{m, fF, fG}, Agg{m, cF, cG}, X, Y, sh, p.sums1, p, ln);
      return make_float2(0.f, 0.f);
    }
    bt_carries<NT, L, true, MODE>(Agg{m, fF, fG}, Agg{m, cF, cG}, X, Y, sh, p.carry1, p, ln);
  }
  kv.fence();
  bt_fence(gg);

  // ---- round 1 sweep: y and the reciprocal of the denominator at every token, against 2^M
  //      (D_t = den_t 2^M); the self weight p_tt = e / den gives the du terms ----
  const float top = fmaxf(fmaxf(kmax, X.m), Y.m);
  const float M = top + span;
  const float sig = fast_exp2(kmax - top);  // the caps' scale against 2^M
  const float sx = fast_exp2(X.m - M), sy = fast_exp2(Y.m - M);
  const float YF = Y.F * sy, YG = Y.G * sy;
  float y[L], rd[L];  // output and 1 / den (0 in empty slots)
  float du = 0.f;
  {
    float A = X.F * sx, Cs = X.G * sx;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float ph[SB], ra[SB], rc[SB];  // terms, and the forward states before each token
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        ph[i] = fast_exp2(kl(j) - M);
        ra[i] = A;
        rc[i] = Cs;
        A = fmaf(A, lam, ph[i] * kv.v(j));
        Cs = fmaf(Cs, lam, ph[i]);
      }
      // backward states entering from the right: the lane's later sub-blocks and later tokens
      const float lr = fast_exp2(-static_cast<float>(L - (q + 1) * SB) * D);
      float Bs = fmaf(YF, lr, sig * capF[q]), Ds = fmaf(YG, lr, sig * capG[q]);
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int j = q * SB + i;
        const float vj = kv.v(j);
        const float e = ph[i] * eU;
        const float num = ra[i] + fmaf(e, vj, Bs);
        const float den = rc[i] + Ds + e;
        const bool live = kv.k(j) != kNegInf;
        const float r = fast_rcp(den);
        y[j] = live ? num * r : 0.f;
        rd[j] = live ? r : 0.f;
        // e^{u+k} (q v - r) = p_tt g (v - y), with p_tt = e / den
        if constexpr (STAGE == 0 || STAGE == 3) du = fmaf(e * rd[j] * gg[j], vj - y[j], du);
        Bs = fmaf(Bs, lam, ph[i] * vj);
        Ds = fmaf(Ds, lam, ph[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  kv.fence();
  bt_fence(gg);
  bt_fence(y);
  bt_fence(rd);

  // ---- round 2 lane sums of (q, r) = (g, g y) / D and caps. With log2 D_t = M - log2 rd_t the
  //      lane's reference is qmax + span, qmax = -M + log2(max rd), and a term against it is
  //      g (rd / max rd) 2^{-span}: no exponential per token ----
  float rmax = 0.f;
#pragma unroll
  for (int i = 0; i < L; ++i) rmax = fmaxf(rmax, rd[i]);
  const float qmax = rmax > 0.f ? fast_log2(rmax) - M : kNegInf;
  float capQ[NSB], capR[NSB];
  Agg X2, Y2;
  {
    const float ref = qmax == kNegInf ? 0.f : qmax + span;
    const float qs = rmax > 0.f ? fast_rcp(rmax) * fast_exp2(-span) : 0.f;
    float qq[L];
#pragma unroll
    for (int i = 0; i < L; ++i) qq[i] = rd[i] * qs * gg[i];
    float fQ = 0.f, fR = 0.f, cQ = 0.f, cR = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      fQ = fmaf(fQ, lam, qq[i]);
      fR = fmaf(fR, lam, qq[i] * y[i]);
    }
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      capQ[q] = cQ;
      capR[q] = cR;
#pragma unroll
      for (int i = (q + 1) * SB - 1; i >= q * SB; --i) {
        cQ = fmaf(cQ, lam, qq[i]);
        cR = fmaf(cR, lam, qq[i] * y[i]);
      }
    }
    const float m = qmax == kNegInf ? kEmptyM : ref;
    if constexpr (STAGE == 2) {
      bt_carries<NT, L, true, kBtProduce>(Agg{m, fQ, fR}, Agg{m, cQ, cR}, X2, Y2, sh, p.sums2, p, ln);
      return make_float2(0.f, 0.f);
    }
    bt_carries<NT, L, true, MODE>(Agg{m, fQ, fR}, Agg{m, cQ, cR}, X2, Y2, sh, p.carry2, p, ln);
  }
  kv.fence();
  bt_fence(gg);
  bt_fence(y);
  bt_fence(rd);

  // ---- round 2 sweep: dv, dk and the dw terms, against 2^M (round 1) and 2^Mq (round 2) ----
  const float topq = fmaxf(fmaxf(qmax, X2.m), Y2.m);
  const float Mq = topq + span;
  const float sigq = fast_exp2(qmax - topq);
  const float sqx = fast_exp2(X2.m - Mq), sqy = fast_exp2(Y2.m - Mq);
  const float S3 = fast_exp2(-M - Mq);  // q_t against 2^Mq is g_t rd_t 2^{-M - Mq}
  const float YQ = Y2.F * sqy, YR = Y2.G * sqy;
  float dwacc = 0.f;  // sum over tokens of b Qpre - d Rpre + a Qsuf - c Rsuf, against 2^{M + Mq}
  {
    float A = X.F * sx, Cs = X.G * sx, QA = X2.F * sqx, QR = X2.G * sqx;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float ph[SB], qh[SB], ra[SB], rc[SB], rqa[SB], rqr[SB];  // forward states before each token
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        ph[i] = fast_exp2(kl(j) - M);
        qh[i] = rd[j] * S3 * gg[j];
        ra[i] = A;
        rc[i] = Cs;
        rqa[i] = QA;
        rqr[i] = QR;
        A = fmaf(A, lam, ph[i] * kv.v(j));
        Cs = fmaf(Cs, lam, ph[i]);
        QA = fmaf(QA, lam, qh[i]);
        QR = fmaf(QR, lam, qh[i] * y[j]);
      }
      const float lr = fast_exp2(-static_cast<float>(L - (q + 1) * SB) * D);
      float Bs = fmaf(YF, lr, sig * capF[q]), Ds = fmaf(YG, lr, sig * capG[q]);
      float QB = fmaf(YQ, lr, sigq * capQ[q]), QRB = fmaf(YR, lr, sigq * capR[q]);
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int j = q * SB + i;
        const long long tt = ln.s_g + j;
        const float a = ra[i], c = rc[i], qa = rqa[i], qr = rqr[i];
        dwacc = fmaf(Bs, qa, fmaf(-Ds, qr, fmaf(a, QB, fmaf(-c, QRB, dwacc))));
        // e^{k} (Qpre + Qsuf + e^u q) and the same over r
        const float vj = kv.v(j);
        const float K = fast_exp2(kl(j) + Mq);
        const float self = qh[i] * eU;
        const float dvj = K * (qa + QB + self);
        const float rj = K * (qr + QRB + self * y[j]);
        bt_store(p, ln.bi, tt, ln.ch, ln.on, dvj, fmaf(vj, dvj, -rj));
        Bs = fmaf(Bs, lam, ph[i] * vj);
        Ds = fmaf(Ds, lam, ph[i]);
        QB = fmaf(QB, lam, qh[i]);
        QRB = fmaf(QRB, lam, qh[i] * y[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // a lane with no token (the end of a row) has no dw terms; its anchored carries may have moved
  // through many empty slots of growth, so 2^{M + Mq} is not formed for it
  const float dw = kmax != kNegInf && dwacc != 0.f ? dwacc * fast_exp2(M + Mq) : 0.f;
  return make_float2(dw, du);
}

// The upstream gradient of N consecutive tokens from t0 (the same for every lane) of batch item
// bi, channel ch; tokens past the row and masked channels read 0.
template <int N, int POL>
__device__ __forceinline__ void bt_load_g(const BwdTileParams& p, int bi, long long t0, int ch, bool on,
                                          float (&gg)[N]) {
  const long long plane = p.T * p.C;
  const char* gb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.g) + static_cast<unsigned long long>(bi) * plane * 4));
  const int t0u = __builtin_amdgcn_readfirstlane(static_cast<int>(t0));
  const int rg = p.C * 4, availg = static_cast<int>(plane * 4);
  const uint32_t offg = on ? static_cast<uint32_t>(ch) * 4 : kOutOfRange;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int ag = (t0u + i) * rg;  // below 2^31 (host check)
    const int lg = availg - ag;
    gg[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(gb + ag, static_cast<uint32_t>(lg > 0 ? lg : 0)), offg, 0, POL));
  }
}

// ---------------------------------------------------------------------------------------------
// Single launch, fast form. The lane keeps its tokens' k and v in registers, and from round 1 on
// g / D at each token. Round 1 (lane sums, exchange, sweep) gives y and 1 / D at each
// sub-block's tokens, which turn at once into that sub-block's round-2 terms (q, r) = (g, g y) / D;
// the round-2 lane sums are formed like the forward tile kernel's (each sub-block against its own
// largest term, the running sum rescaled when a larger one arrives). After the round-2 exchange
// the round-2 sweep forms the round-1 sweep of each sub-block again (the same arithmetic on the
// same values, for y and the states of dw) and writes dv, dk and the dw terms. Returns (dw terms,
// du terms, failed, -); failed when a wait of either exchange ran out.
// ---------------------------------------------------------------------------------------------
template <int DT, int L, bool PAIR>
using BtOneKV = std::conditional_t<PAIR, RowKVPair<L>, BtKV<DT, L>>;

// Issues the loads of the chunk's k and v for bt_body_one (nothing waits here).
template <int DT, int L, bool PAIR>
__device__ __forceinline__ void bt_one_load(const BwdTileParams& p, const BtLane& ln, BtOneKV<DT, L, PAIR>& kv) {
  if constexpr (PAIR)
    bt_load_pairs<L, kStream>(p, ln.bi, ln.s_g, ln.ch, ln.on, kv, nullptr);
  else
    bt_load<DT, L, kStream>(p, ln.bi, ln.s_g, ln.ch, ln.on, kv, nullptr);
}

template <int DT, int L, int NT, bool PAIR>
__device__ __forceinline__ float4 bt_body_one(const BwdTileParams& p, const BtLane& ln, BtOneKV<DT, L, PAIR>& kv,
                                              BtShared<NT>* sh, const unsigned* sh_tag, unsigned& fin) {
  constexpr int SB = kBtSB;
  constexpr int NSB = L / SB;
  const float4 failed = make_float4(0.f, 0.f, 1.f, 0.f);
  const float D = ln.D, U = ln.U;
  const float lam = fast_exp2(-D);
  const float lsb = fast_exp2(-static_cast<float>(SB) * D);  // lam^SB
  const float span = fmaxf(-D, 0.f) * static_cast<float>(L - 1);  // largest growth inside a lane
  const float eU = fast_exp2(U);
  if constexpr (PAIR) {
#pragma unroll
    for (int q = 0; q < L / 8; ++q) kv.prepare(q);
  }
  auto kl = [&](int i) { return kv.k(i) * kLog2e; };  // -inf in empty slots

  // ---- round 1 lane sums (against 2^{kmax + span}) and the caps, as in bt_body_fast ----
  float kmax = kNegInf;
#pragma unroll
  for (int i = 0; i < L; ++i) kmax = fmaxf(kmax, kl(i));
  float capF[NSB], capG[NSB];
  Agg X, Y;
  // g streams in one sub-block ahead of the round-1 sweep (the first during the exchange); loading
  // all of a lane's g with its k and v measured slower (120 against 110 us at B=4, T=4096,
  // C=1024)
  float gq[SB];
  {
    const float ref = kmax == kNegInf ? 0.f : kmax + span;
    float pp[L];
#pragma unroll
    for (int i = 0; i < L; ++i) pp[i] = fast_exp2(kl(i) - ref);
    float fF = 0.f, fG = 0.f, cF = 0.f, cG = 0.f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      fF = fmaf(fF, lam, pp[i] * kv.v(i));
      fG = fmaf(fG, lam, pp[i]);
    }
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      capF[q] = cF;
      capG[q] = cG;
#pragma unroll
      for (int i = (q + 1) * SB - 1; i >= q * SB; --i) {
        cF = fmaf(cF, lam, pp[i] * kv.v(i));
        cG = fmaf(cG, lam, pp[i]);
      }
    }
    const float m = kmax == kNegInf ? kEmptyM : ref;
    bt_load_g<SB, kStream>(p, ln.bi, ln.s_g, ln.ch, ln.on, gq);
    if (bt_exchange<NT, L, true>(Agg{m, fF, fG}, Agg{m, cF, cG}, X, Y, sh, p, ln, 0, sh_tag)) return failed;
  }
  kv.fence();

  // ---- the round-1 sweep of one sub-block: y and 1 / D at its tokens, against 2^M; also the
  //      terms, the forward states before each token and the backward states after it ----
  const float top = fmaxf(fmaxf(kmax, X.m), Y.m);
  const float M = top + span;
  const float sig = fast_exp2(kmax - top);  // the caps' scale against 2^M
  const float sx = fast_exp2(X.m - M), sy = fast_exp2(Y.m - M);
  const float YF = Y.F * sy, YG = Y.G * sy;
  auto sweep1 = [&](int q, float& A, float& Cs, float (&ph)[SB], float (&ra)[SB], float (&rc)[SB],
                    float (&yv)[SB], float (&rdv)[SB], float (&bs)[SB], float (&ds)[SB]) {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int j = q * SB + i;
      ph[i] = fast_exp2(kl(j) - M);
      ra[i] = A;
      rc[i] = Cs;
      A = fmaf(A, lam, ph[i] * kv.v(j));
      Cs = fmaf(Cs, lam, ph[i]);
    }
    // backward states entering from the right: the lane's later sub-blocks and later tokens
    const float lr = fast_exp2(-static_cast<float>(L - (q + 1) * SB) * D);
    float Bs = fmaf(YF, lr, sig * capF[q]), Ds = fmaf(YG, lr, sig * capG[q]);
#pragma unroll
    for (int i = SB - 1; i >= 0; --i) {
      const int j = q * SB + i;
      const float vj = kv.v(j);
      const float e = ph[i] * eU;
      const float num = ra[i] + fmaf(e, vj, Bs);
      const float den = rc[i] + Ds + e;
      const bool live = kv.k(j) != kNegInf;
      const float r = fast_rcp(den);
      yv[i] = live ? num * r : 0.f;
      rdv[i] = live ? r : 0.f;
      bs[i] = Bs;
      ds[i] = Ds;
      Bs = fmaf(Bs, lam, ph[i] * vj);
      Ds = fmaf(Ds, lam, ph[i]);
    }
  };

  // ---- round 1 sweep with the round-2 lane sums of (q, r) and the du terms. A sub-block's terms
  //      are g (rd / rmax) 2^{-span} against 2^{mq + span}, mq = log2(rmax) - M (rmax: its
  //      largest 1 / D) ----
  const float e_span = fast_exp2(-span);
  float du = 0.f;
  float mrun = kNegInf;  // (fQ, fR) are against 2^{mrun + span}
  float fQ = 0.f, fR = 0.f;
  float bQ[NSB], bR[NSB], bm[NSB];  // each sub-block's backward sums, anchored at its first token
  float gr[L];                      // g / D at each token, against 2^{-M}
  {
    float A = X.F * sx, Cs = X.G * sx;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float gn[SB];
      if (q + 1 < NSB) bt_load_g<SB, kStream>(p, ln.bi, ln.s_g + (q + 1) * SB, ln.ch, ln.on, gn);
      float ph[SB], ra[SB], rc[SB], yv[SB], rdv[SB], bs[SB], ds[SB];
      sweep1(q, A, Cs, ph, ra, rc, yv, rdv, bs, ds);
      float rmx = 0.f;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int j = q * SB + i;
        // e^{u+k} (q v - r) = p_tt g (v - y), with p_tt = e / den
        du = fmaf(ph[i] * eU * rdv[i] * gq[i], kv.v(j) - yv[i], du);
        rmx = fmaxf(rmx, rdv[i]);
        gr[j] = rdv[i] * gq[i];
      }
      const float mq = rmx > 0.f ? fast_log2(rmx) - M : kNegInf;
      const float qs = rmx > 0.f ? fast_rcp(rmx) * e_span : 0.f;
      float qq[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) qq[i] = gr[q * SB + i] * qs;
      float sQ = 0.f, sR = 0.f;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        sQ = fmaf(sQ, lam, qq[i]);
        sR = fmaf(sR, lam, qq[i] * yv[i]);
      }
      float cQ = 0.f, cR = 0.f;
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        cQ = fmaf(cQ, lam, qq[i]);
        cR = fmaf(cR, lam, qq[i] * yv[i]);
      }
      bQ[q] = cQ;
      bR[q] = cR;
      bm[q] = mq;
      // move the running sums SB tokens on and add this sub-block at the larger exponent
      const float mn = fmaxf(mrun, mq);
      const float mr = mn == kNegInf ? 0.f : mn;
      const float sr = fast_exp2(mrun - mr) * lsb, sq = fast_exp2(mq - mr);
      fQ = fmaf(fQ, sr, sQ * sq);
      fR = fmaf(fR, sr, sR * sq);
      mrun = mn;
      if (q + 1 < NSB) {
#pragma unroll
        for (int i = 0; i < SB; ++i) gq[i] = gn[i];
      }
      __builtin_amdgcn_sched_barrier(0);  // one sub-block at a time (bounded live values)
    }
  }
  const float qmax = mrun;  // -inf when the lane holds no token
  float capQ[NSB], capR[NSB];
  Agg X2, Y2;
  {
    const float mr = mrun == kNegInf ? 0.f : mrun;
    float cQ = 0.f, cR = 0.f;
#pragma unroll
    for (int q = NSB - 1; q >= 0; --q) {
      capQ[q] = cQ;
      capR[q] = cR;
      const float sq = fast_exp2(bm[q] - mr);
      cQ = fmaf(cQ, lsb, bQ[q] * sq);
      cR = fmaf(cR, lsb, bR[q] * sq);
    }
    const float m = qmax == kNegInf ? kEmptyM : qmax + span;
    if (bt_exchange<NT, L, true>(Agg{m, fQ, fR}, Agg{m, cQ, cR}, X2, Y2, sh, p, ln, 1, sh_tag)) return failed;
  }
  // every wavefront is past its last read of a slot
  if (threadIdx.x == 0 && p.n_chunks > 1) fin = bt_retire_begin(p);
  kv.fence();
  bt_fence(gr);

  // ---- round 2 sweep: dv, dk and the dw terms, against 2^M (round 1) and 2^Mq (round 2) ----
  const float topq = fmaxf(fmaxf(qmax, X2.m), Y2.m);
  const float Mq = topq + span;
  const float sigq = fast_exp2(qmax - topq);
  const float sqx = fast_exp2(X2.m - Mq), sqy = fast_exp2(Y2.m - Mq);
  const float S3 = fast_exp2(-M - Mq);  // q_t against 2^Mq is g_t rd_t 2^{-M - Mq}
  const float YQ = Y2.F * sqy, YR = Y2.G * sqy;
  float dwacc = 0.f;  // sum over tokens of b Qpre - d Rpre + a Qsuf - c Rsuf, against 2^{M + Mq}
  {
    float A = X.F * sx, Cs = X.G * sx, QA = X2.F * sqx, QR = X2.G * sqx;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float ph[SB], ra[SB], rc[SB], yv[SB], rdv[SB], bs[SB], ds[SB];
      sweep1(q, A, Cs, ph, ra, rc, yv, rdv, bs, ds);
      float qh[SB], rqa[SB], rqr[SB];  // q against 2^Mq, and the round-2 forward states
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        qh[i] = gr[q * SB + i] * S3;
        rqa[i] = QA;
        rqr[i] = QR;
        QA = fmaf(QA, lam, qh[i]);
        QR = fmaf(QR, lam, qh[i] * yv[i]);
      }
      const float lr = fast_exp2(-static_cast<float>(L - (q + 1) * SB) * D);
      float QB = fmaf(YQ, lr, sigq * capQ[q]), QRB = fmaf(YR, lr, sigq * capR[q]);
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int j = q * SB + i;
        const long long tt = ln.s_g + j;
        dwacc = fmaf(bs[i], rqa[i], fmaf(-ds[i], rqr[i], fmaf(ra[i], QB, fmaf(-rc[i], QRB, dwacc))));
        // e^{k} (Qpre + Qsuf + e^u q) and the same over r
        const float vj = kv.v(j);
        const float K = fast_exp2(kl(j) + Mq);
        const float self = qh[i] * eU;
        const float dvj = K * (rqa[i] + QB + self);
        const float rj = K * (rqr[i] + QRB + self * yv[i]);
        bt_store(p, ln.bi, tt, ln.ch, ln.on, dvj, fmaf(vj, dvj, -rj));
        QB = fmaf(QB, lam, qh[i]);
        QRB = fmaf(QRB, lam, qh[i] * yv[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // a lane with no token (the end of a row) has no dw terms (see bt_body_fast)
  const float dw = kmax != kNegInf && dwacc != 0.f ? dwacc * fast_exp2(M + Mq) : 0.f;
  return make_float4(dw, du, 0.f, 0.f);
}

// ---------------------------------------------------------------------------------------------
// Stage 1 of a multi-chunk row: the round-1 sums of every chunk. A lane holds one channel of one
// chunk (64 tokens, like a lane of the forward tile kernel), so the chunk's sums are the lane's
// and no scan is needed. The form matches what stages 2 and 3 read: anchored sums (forward at the
// chunk's last slot, backward at its first token) formed per 8-token sub-block against the
// sub-block's own reference and combined with exponent shifts, or position-free sums (wide form).
// The tile's channels vote on the form exactly as the tile kernel's workgroups do.
// ---------------------------------------------------------------------------------------------
// (bf16 channel pairs: 64 tokens of k and v per lane in 64 registers, four waves per SIMD. The
// 16-bit and fp32 loads need more registers while in flight: two waves per SIMD. The wide form
// lives out of line.)
// Wide form of a chunk's sums: position-free, against running maxima. Rare, so out of line with
// its own register allocation; it loads the chunk itself.
template <int DT, int CT>
__device__ __noinline__ void bwd_chunk_sums_wide(const BwdTileParams* args, int bi, long long t0, int ch,
                                                 bool on, float D, float* o) {
  constexpr int SUB = kBwdLane;
  constexpr int NSUB = CT / SUB;
  const BwdTileParams& p = *args;
  BtKV<DT, CT> kv;
  bt_load<DT, CT>(p, bi, t0, ch, on, kv, nullptr);
  Agg fw = row_empty(), bw = row_empty();
#pragma unroll
  for (int q = 0; q < NSUB; ++q) {
    float xp[SUB], xs[SUB], vv[SUB], one[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      const int j = q * SUB + i;
      const float kl = kv.k(j) * kLog2e, tD = static_cast<float>(t0 + j) * D;
      xp[i] = kl + tD;
      xs[i] = kl - tD;
      vv[i] = kv.v(j);
      one[i] = 1.f;
    }
    fw = agg_add_f(fw, bt_block<SUB>(xp, vv, one));
    bw = agg_add_f(bw, bt_block<SUB>(xs, vv, one));
    __builtin_amdgcn_sched_barrier(0);
  }
  o[0] = fw.m;
  o[1] = fw.F;
  o[2] = fw.G;
  o += kBtTile * 3;
  o[0] = bw.m;
  o[1] = bw.F;
  o[2] = bw.G;
}

template <int DT, int CT, int NT, bool PAIR>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(PAIR ? 4 : 2)))
    bwd_chunk_sums_kernel(BwdTileParams p) {
  static_assert(!PAIR || DT == BIWKV_BF16, "pairs are bf16 channel pairs");
  constexpr int SUB = kBwdLane;  // tokens per sub-block: the tile kernel's lane length
  constexpr int NSUB = CT / SUB;
  const int tid = threadIdx.x;
  const int c = tid % kBtTile;
  // workgroup x: row x / per_row, chunks (x % per_row) * NT / 64 onwards (one wavefront each)
  const int per_row = (p.n_chunks + NT / kBtTile - 1) / (NT / kBtTile);
  const int row = static_cast<int>(blockIdx.x) / per_row;
  const int chunk = (static_cast<int>(blockIdx.x) - row * per_row) * (NT / kBtTile) + tid / kBtTile;
  const int bi = row / p.n_tiles;
  const int tile = row - bi * p.n_tiles;
  const int ch = tile * kBtTile + c;
  const bool on = ch < p.C && chunk < p.n_chunks;
  const long long T = p.T;
  const float D = on ? (p.w[ch] / static_cast<float>(T)) * kLog2e : 0.f;
  const float U = on ? p.u[ch] * kLog2e : 0.f;
  // the tile kernel's vote (a wavefront holds the tile's 64 channels)
  const bool wide =
      __ballot(bt_wide_lane<kBwdLane>(D, U)) != 0ull;
  if (chunk >= p.n_chunks) return;  // (after the vote: every lane of the wavefront took part)
  const long long t0 = static_cast<long long>(chunk) * CT;
  float* o = p.sums1 + ((static_cast<size_t>(row) * p.n_chunks + chunk) * 2 * kBtTile + c) * 3;
  if (wide) {
    // the kernel's only argument is p, at the start of the argument segment
    const auto* args = (const BwdTileParams*)(__builtin_amdgcn_kernarg_segment_ptr());
    bwd_chunk_sums_wide<DT, CT>(args, bi, t0, ch, on, D, o);
    return;
  }
  std::conditional_t<PAIR, RowKVPair<CT>, BtKV<DT, CT>> kv;
  if constexpr (PAIR)
    bt_load_pairs<CT>(p, bi, t0, ch, on, kv, nullptr);
  else
    bt_load<DT, CT>(p, bi, t0, ch, on, kv, nullptr);
  Agg fw = row_empty(), bw = row_empty();
  {
    const float lam = fast_exp2(-D);
    const float span = fmaxf(-D, 0.f) * static_cast<float>(SUB - 1);
#pragma unroll
    for (int q = 0; q < NSUB; ++q) {
      if constexpr (PAIR) kv.prepare(q);  // waits only for this sub-block's words
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < SUB; ++i) mx = fmaxf(mx, kv.k(q * SUB + i) * kLog2e);
      const float ref = mx == kNegInf ? 0.f : mx + span;
      float fF = 0.f, fG = 0.f, bF = 0.f, bG = 0.f;
      float pp[SUB];
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        pp[i] = fast_exp2(kv.k(q * SUB + i) * kLog2e - ref);
        fF = fmaf(fF, lam, pp[i] * kv.v(q * SUB + i));
        fG = fmaf(fG, lam, pp[i]);
      }
#pragma unroll
      for (int i = SUB - 1; i >= 0; --i) {
        bF = fmaf(bF, lam, pp[i] * kv.v(q * SUB + i));
        bG = fmaf(bG, lam, pp[i]);
      }
      const float m = mx == kNegInf ? kEmptyM : ref;
      // forward: from the sub-block's last token to the chunk's last slot; backward: from its
      // first token to the chunk's first token
      fw = agg_add_f(agg_shift(fw, static_cast<float>(SUB), D), Agg{m, fF, fG});
      bw = agg_add_f(bw, agg_shift(Agg{m, bF, bG}, static_cast<float>(q * SUB), D));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  o[0] = fw.m;
  o[1] = fw.F;
  o[2] = fw.G;
  o += kBtTile * 3;
  o[0] = bw.m;
  o[1] = bw.F;
  o[2] = bw.G;
}

// ---------------------------------------------------------------------------------------------
// Carries of every chunk of a row from the chunk sums: forward, the sum over the earlier chunks
// anchored just before the chunk; backward, over the later chunks anchored just after it (moved
// CT tokens per chunk; position-free sums of the wide form are plain sums). Thread (c, grp) of a
// workgroup of 64 channels x kCarryGroups groups folds a contiguous range of the row's chunks;
// one thread per channel folds the group sums; each thread then writes its chunks' carries. Fixed
// order, so the result is reproducible. The tile's channels vote on the form as the tile kernel's
// workgroups do (a wavefront holds the tile's 64 channels).
// ---------------------------------------------------------------------------------------------
constexpr int kCarryGroups = 16;

// The carries of one row (`row`) by a workgroup of 64 x GR threads (thread (c, grp)), with LDS for
// the group sums gs and group carries gc. VL: the tile kernel's lane length, whose vote decides
// the form.
template <int CT, int GR, int VL>
__device__ __forceinline__ void bt_row_carries(const BwdTileParams& p, const float* __restrict__ sums,
                                               float* __restrict__ carry, int row, float (*gs)[6][kBtTile],
                                               float (*gc)[6][kBtTile]) {
  const int c = threadIdx.x % kBtTile, grp = threadIdx.x / kBtTile;
  const int bi = row / p.n_tiles;
  const int ch = (row - bi * p.n_tiles) * kBtTile + c;
  const bool on = ch < p.C;
  const float Dc = on ? (p.w[ch] / static_cast<float>(p.T)) * kLog2e : 0.f;
  const float Uc = on ? p.u[ch] * kLog2e : 0.f;
  const bool wide = __ballot(bt_wide_lane<VL>(Dc, Uc)) != 0ull;
  const float D = wide ? 0.f : Dc;  // exponent shift per token (none for position-free sums)
  const float step = static_cast<float>(CT);
  const int nch = p.n_chunks;
  const int per = (nch + GR - 1) / GR;
  const int j0 = grp * per, j1 = j0 + per < nch ? j0 + per : nch;
  const size_t base = static_cast<size_t>(row) * nch * 2 * kBtTile * 3 + static_cast<size_t>(c) * 3;
  auto at = [&](int j, int dir) { return base + static_cast<size_t>(j * 2 + dir) * kBtTile * 3; };
  auto get = [&](const float* a, size_t i) { return Agg{a[i], a[i + 1], a[i + 2]}; };
  // group sums: forward anchored at the group's last chunk's last slot, backward at its first
  // chunk's first token
  Agg f = row_empty(), b = row_empty();
#pragma unroll 4
  for (int j = j0; j < j1; ++j) f = agg_add_f(agg_shift(f, step, D), get(sums, at(j, kFwd)));
#pragma unroll 4
  for (int j = j1 - 1; j >= j0; --j) b = agg_add_f(get(sums, at(j, kBwd)), agg_shift(b, step, D));
  gs[grp][0][c] = f.m;
  gs[grp][1][c] = f.F;
  gs[grp][2][c] = f.G;
  gs[grp][3][c] = b.m;
  gs[grp][4][c] = b.F;
  gs[grp][5][c] = b.G;
  __syncthreads();
  if (grp == 0) {
    Agg x = row_empty();
    for (int k = 0; k < GR; ++k) {
      const int a0 = k * per, a1 = a0 + per < nch ? a0 + per : nch;
      const int len = a1 > a0 ? a1 - a0 : 0;
      gc[k][0][c] = x.m;
      gc[k][1][c] = x.F;
      gc[k][2][c] = x.G;
      x = agg_add_f(agg_shift(x, step * len, D), Agg{gs[k][0][c], gs[k][1][c], gs[k][2][c]});
    }
    Agg y = row_empty();
    for (int k = GR - 1; k >= 0; --k) {
      const int a0 = k * per, a1 = a0 + per < nch ? a0 + per : nch;
      const int len = a1 > a0 ? a1 - a0 : 0;
      gc[k][3][c] = y.m;
      gc[k][4][c] = y.F;
      gc[k][5][c] = y.G;
      y = agg_add_f(Agg{gs[k][3][c], gs[k][4][c], gs[k][5][c]}, agg_shift(y, step * len, D));
    }
  }
  __syncthreads();
  Agg x{gc[grp][0][c], gc[grp][1][c], gc[grp][2][c]};
#pragma unroll 4
  for (int j = j0; j < j1; ++j) {
    const size_t o = at(j, kFwd);
    carry[o] = x.m;
    carry[o + 1] = x.F;
    carry[o + 2] = x.G;
    x = agg_add_f(agg_shift(x, step, D), get(sums, o));
  }
  Agg y{gc[grp][3][c], gc[grp][4][c], gc[grp][5][c]};
#pragma unroll 4
  for (int j = j1 - 1; j >= j0; --j) {
    const size_t o = at(j, kBwd);
    carry[o] = y.m;
    carry[o + 1] = y.F;
    carry[o + 2] = y.G;
    y = agg_add_f(get(sums, o), agg_shift(y, step, D));
  }
}

template <int CT>
__global__ void __launch_bounds__(64 * kCarryGroups)
    bwd_carry_kernel(BwdTileParams p, const float* __restrict__ sums, float* __restrict__ carry) {
  __shared__ float gs[kCarryGroups][6][kBtTile];  // group sums
  __shared__ float gc[kCarryGroups][6][kBtTile];  // group carries
  bt_row_carries<CT, kCarryGroups, kBwdLane>(p, sums, carry, blockIdx.x, gs, gc);
}

// One workgroup's share of a backward launch: the chunk `unit` (row-major over (row, chunk)) in
// STAGE 0 (a row of one chunk, the whole backward) or STAGE 1, 2, 3 (the three launches of a
// longer row, see the top of this file), with the dw and du terms of STAGE 0 and 3 folded per
// channel over the groups, in order, and written to pw, pu.
// PAIR: bf16 k and v as 32-bit channel pairs (bt_load_pairs).
template <int DT, int L, int NT, int STAGE, bool PAIR>
__device__ __forceinline__ void bt_stage(const BwdTileParams& p, unsigned unit, BtShared<NT>& sh) {
  static_assert(!PAIR || (DT == BIWKV_BF16 && L % 8 == 0), "pairs are bf16 channel pairs");
  static_assert(L % kBtSB == 0 && NT % kBtTile == 0 && NT <= 1024, "bad backward tile shape");
  static_assert(((NT / kBtTile) & (NT / kBtTile - 1)) == 0, "a channel's groups share a wavefront");
  const BtLane ln = bt_lane<L, NT>(p, unit);
  if (ln.g == 0) sh.dch[ln.c] = ln.D;  // read by the scans, after their first barrier
  // The whole workgroup takes the wide form when any of its channels needs it; every wavefront
  // holds all 64 channels, so a wavefront vote is the workgroup's vote (and every chunk of the
  // row, in every stage, votes the same way).
  const bool wide_lane = bt_wide_lane<L>(ln.D, ln.U);
  float2 r;
  if (__ballot(wide_lane) != 0ull) {
    const auto* args = (const BwdTileParams*)(__builtin_amdgcn_kernarg_segment_ptr());
    const float4 rw = bt_body_wide<DT, L, NT, STAGE>(args, &sh, nullptr, unit);
    r = make_float2(rw.x, rw.y);
  } else {
    r = bt_body_fast<DT, L, NT, STAGE, PAIR>(p, ln, &sh);
  }
  if constexpr (STAGE == 0 || STAGE == 3) {
    // ---- per-channel fold of the lanes' dw and du terms over the groups, in order ----
    sh.fold[0][ln.g][ln.c] = r.x;
    sh.fold[1][ln.g][ln.c] = r.y;
    __syncthreads();
    if (ln.g == 0 && ln.on) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int i = 0; i < NT / kBtTile; ++i) {
        a += sh.fold[0][i][ln.c];
        b += sh.fold[1][i][ln.c];
      }
      const long long at = (static_cast<long long>(ln.bi) * p.n_chunks + ln.chunk) * p.C + ln.ch;
      p.pw[at] = a;
      p.pu[at] = b;
    }
  }
}

template <int DT, int L, int NT, int WPE, int STAGE, bool PAIR>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE)))
    bwd_tile_kernel(BwdTileParams p) {
  __shared__ BtShared<NT> sh;
  bt_stage<DT, L, NT, STAGE, PAIR>(p, blockIdx.x, sh);
}

// ---------------------------------------------------------------------------------------------
// The backward in one launch (rows of several chunks whose chunks are resident together; blocks
// start in order, so a row's chunks only wait for slots that earlier rows free): both rounds'
// chunk sums go through the slot exchange (bt_exchange). A workgroup whose wait runs out stores
// nothing and marks its row in row_fail with the launch's tag; bwd_one_reduce_kernel then computes
// that row again on its own, so no result depends on the chunks being resident together.
// ---------------------------------------------------------------------------------------------
template <int DT, int L, int NT, bool PAIR>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4)))
    bwd_one_kernel(BwdTileParams p) {
  static_assert(!PAIR || (DT == BIWKV_BF16 && L % 8 == 0), "pairs are bf16 channel pairs");
  static_assert(L % kBtSB == 0 && NT % kBtTile == 0 && NT <= 1024, "bad backward tile shape");
  static_assert(((NT / kBtTile) & (NT / kBtTile - 1)) == 0, "a channel's groups share a wavefront");
  __shared__ BtShared<NT> sh;
  __shared__ unsigned sh_tag;
  const int tid = threadIdx.x;
  BtLane ln = bt_lane_index<L, NT>(p, blockIdx.x);
  // Every vector load is issued before anything waits: w and u (range-checked: a masked lane reads
  // 0), then the chunk's k and v in the fast form's layout; the form is chosen once w and u have
  // arrived, and the wide form loads the chunk again itself.
  const uint32_t coff = ln.on ? static_cast<uint32_t>(ln.ch) * 4u : kOutOfRange;
  const uint32_t cbytes = static_cast<uint32_t>(p.C) * 4u;
  const uint32_t wbits = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.w, cbytes), coff, 0, 0);
  const uint32_t ubits = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.u, cbytes), coff, 0, 0);
  BtOneKV<DT, L, PAIR> kv;
  bt_one_load<DT, L, PAIR>(p, ln, kv);
  // slots are tagged with the launch's epoch + 1 (never 0, so zeroed slots never match); the tag
  // is read after the exchange's first barrier. The epoch comes through the scalar cache, which
  // holds no stale copy (caches are invalidated when a launch starts, and the counter only moves
  // once every workgroup of the launch has read it); the load waits on the scalar counter only.
  unsigned ep = 0u;
  if (p.n_chunks > 1) {
    const unsigned long long ea = uniform_u64(reinterpret_cast<unsigned long long>(&p.ctr->epoch));
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(ep) : "s"(ea) : "memory");
  }
  if (tid == 0) sh_tag = p.n_chunks > 1 ? ep + 1u : 1u;
  bt_lane_params(ln, p.T, __uint_as_float(wbits), __uint_as_float(ubits));
  if (ln.g == 0) sh.dch[ln.c] = ln.D;
  const bool wide_lane = bt_wide_lane<L>(ln.D, ln.U);
  unsigned fin = kNotRetiring;
  float4 r;
  if (__ballot(wide_lane) != 0ull) {
    const auto* args = (const BwdTileParams*)(__builtin_amdgcn_kernarg_segment_ptr());
    r = bt_body_wide<DT, L, NT, 4>(args, &sh, &sh_tag, blockIdx.x);
  } else {
    r = bt_body_one<DT, L, NT, PAIR>(p, ln, kv, &sh, &sh_tag, fin);
  }
  if (r.z != 0.f) {  // uniform: a wait ran out
    if (tid == 0) {
      p.row_fail[ln.row] = sh_tag;
      __hip_atomic_fetch_or(&p.ctr->fault, kFaultSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    sh.fold[0][ln.g][ln.c] = r.x;
    sh.fold[1][ln.g][ln.c] = r.y;
    __syncthreads();
    if (ln.g == 0 && ln.on) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int i = 0; i < NT / kBtTile; ++i) {
        a += sh.fold[0][i][ln.c];
        b += sh.fold[1][i][ln.c];
      }
      const long long at = (static_cast<long long>(ln.bi) * p.n_chunks + ln.chunk) * p.C + ln.ch;
      p.pw[at] = a;
      p.pu[at] = b;
    }
  }
  if (p.n_chunks > 1 && tid == 0) {
    if (fin == kNotRetiring) fin = bt_retire_begin(p);
    bt_retire_end(p, fin);
  }
}

// A row of the last bwd_one_kernel launch whose waits ran out, computed again by one workgroup
// alone: the three stages of the multi-launch form over the row's chunks in order (chunk sums,
// carries, round 1 and the round-2 sums, carries, both rounds), so it needs no other workgroup.
// Inlined into the kernel that calls it: bt_stage's wide form reads the parameters through the
// kernel's argument segment pointer, which only a kernel body has (an out-of-line function sees a
// null pointer there).
template <int DT, int L, int NT, bool PAIR>
__device__ __forceinline__ void bt_row_fallback(const BwdTileParams& p, int row, BtShared<NT>& sh) {
  constexpr int CT = (NT / kBtTile) * L;
  constexpr int GR = NT / kBtTile;
  static_assert(sizeof(sh.sw) >= 2 * GR * 6 * kBtTile * sizeof(float), "carry scratch");
  float(*gs)[6][kBtTile] = reinterpret_cast<float(*)[6][kBtTile]>(&sh.sw[0][0][0]);
  float(*gc)[6][kBtTile] = gs + GR;
  const unsigned u0 = static_cast<unsigned>(row) * static_cast<unsigned>(p.n_chunks);
  for (int ck = 0; ck < p.n_chunks; ++ck) {
    bt_stage<DT, L, NT, 1, PAIR>(p, u0 + ck, sh);
    __syncthreads();
  }
  bt_row_carries<CT, GR, L>(p, p.sums1, p.carry1, row, gs, gc);
  __syncthreads();
  for (int ck = 0; ck < p.n_chunks; ++ck) {
    bt_stage<DT, L, NT, 2, PAIR>(p, u0 + ck, sh);
    __syncthreads();
  }
  bt_row_carries<CT, GR, L>(p, p.sums2, p.carry2, row, gs, gc);
  __syncthreads();
  for (int ck = 0; ck < p.n_chunks; ++ck) {
    bt_stage<DT, L, NT, 3, PAIR>(p, u0 + ck, sh);
    __syncthreads();
  }
}

// The last kernel of a single-launch call, one workgroup per 64-channel tile: first the rows of
// that tile whose waits ran out in the bwd_one_kernel launch before it (row_fail holds that
// launch's tag, which is the epoch now), each computed again by bt_row_fallback; then dw and du of
// the tile's channels, the per-chunk terms folded in batch and chunk order (thread (c, grp) sums
// a contiguous segment of them, the segments are added in order). p addresses chunks in plain row
// order (xcd_rows = 0).
template <int DT, int L, int NT, bool PAIR>
__global__ void __launch_bounds__(NT) bwd_one_reduce_kernel(BwdTileParams p, BwdParams rp) {
  constexpr int GR = NT / kBtTile;
  constexpr int kHeld = 32;  // partial sums of a lane held in registers (more are read in a loop)
  __shared__ BtShared<NT> sh;
  const int tile = blockIdx.x;
  const int c = threadIdx.x % kBtTile, grp = threadIdx.x / kBtTile;
  const int ch = tile * kBtTile + c;
  const int chc = ch < rp.C ? ch : rp.C - 1;  // a masked lane reads a valid term and ignores it
  const long long n = static_cast<long long>(rp.B) * rp.n_wg;
  const long long per = (n + GR - 1) / GR;
  const long long r0 = grp * per, r1 = r0 + per < n ? r0 + per : n;
  // This lane's dw and du terms, the row flags of the first 64 batch items and the launch's tag
  // are all requested before anything waits (one round trip): the terms are read unconditionally
  // at clamped rows, the tag through the scalar cache (its wait is on the scalar counter only).
  // The terms are read non-temporally, so the CU's L1 keeps no copy that a second read could find
  // stale after this workgroup computed a row again below.
  float hw[kHeld], hu[kHeld];
  const bool held = per <= kHeld;
  if (held) {
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
      const long long r = r0 + i < n ? r0 + i : n - 1;
      hw[i] = __builtin_nontemporal_load(rp.s.pw + r * rp.C + chc);
      hu[i] = __builtin_nontemporal_load(rp.s.pu + r * rp.C + chc);
    }
  }
  const bool many = p.n_chunks > 1;
  const int lane = static_cast<int>(threadIdx.x % 64);
  const int b0c = lane < rp.B ? lane : rp.B - 1;
  const unsigned flag0 = many ? p.row_fail[b0c * p.n_tiles + tile] : 0u;
  unsigned tag = 0u;
  if (many) {
    const unsigned long long ea = uniform_u64(reinterpret_cast<unsigned long long>(&p.ctr->epoch));
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(tag) : "s"(ea) : "memory");
  }
  // the terms in a fixed order (the same additions whether held or read in the loop)
  auto fold = [&](float& sw, float& su, bool use_held) {
    sw = 0.f;
    su = 0.f;
    if (use_held) {
#pragma unroll
      for (int i = 0; i < kHeld; ++i) {
        if (r0 + i < r1) {
          sw += hw[i];
          su += hu[i];
        }
      }
    } else {
#pragma unroll 8
      for (long long r = r0; r < r1; ++r) {
        sw += __builtin_nontemporal_load(rp.s.pw + r * rp.C + chc);
        su += __builtin_nontemporal_load(rp.s.pu + r * rp.C + chc);
      }
    }
  };
  // Rows whose waits ran out in the bwd_one_kernel launch before this one (row_fail holds that
  // launch's tag, which is the epoch now). Lane j of every wavefront holds the flag of batch item
  // b0 + j; the vote is the same in every wavefront, so the fallback's barriers are met by all.
  // The held terms are only used when no row was computed again, so they are not live across the
  // (out-of-line) fallback.
  auto hits = [&](int b0) {
    const int bi = b0 + lane;
    const unsigned f = b0 == 0 ? flag0 : (bi < rp.B ? p.row_fail[bi * p.n_tiles + tile] : 0u);
    return __ballot(bi < rp.B && f == tag);
  };
  bool any = false;
  if (many)
    for (int b0 = 0; b0 < rp.B; b0 += 64) any = any || hits(b0) != 0ull;
  float sw, su;
  if (!any) {
    fold(sw, su, held);
  } else {
    for (int b0 = 0; b0 < rp.B; b0 += 64) {
      unsigned long long m = hits(b0);
      while (m != 0ull) {
        const int j = __builtin_ctzll(m);
        m &= m - 1ull;
        bt_row_fallback<DT, L, NT, PAIR>(p, (b0 + j) * p.n_tiles + tile, sh);
      }
    }
    __syncthreads();  // the rows' terms, written by this workgroup, are visible to it
    fold(sw, su, false);
  }
  sh.fold[0][grp][c] = sw;
  sh.fold[1][grp][c] = su;
  __syncthreads();
  if (grp != 0 || ch >= rp.C) return;
  sw = 0.f;
  su = 0.f;
  for (int i = 0; i < GR; ++i) {
    sw += sh.fold[0][i][c];
    su += sh.fold[1][i][c];
  }
  const float D = bwd_decay(rp, ch);
  rp.dw[ch] = -(fast_exp2(-D) / static_cast<float>(rp.T)) * sw;
  rp.du[ch] = su;
}

}  // namespace
