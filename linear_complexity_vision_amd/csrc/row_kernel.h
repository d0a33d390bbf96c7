// Bi-WKV tile kernel: a (batch, channel tile) row held by one workgroup, or by a few workgroups
// (chunks of the row) that exchange their sums.
#pragma once

#include <type_traits>

#include "common.h"

namespace {

// ---------------------------------------------------------------------------------------------
// Bi-WKV tile kernel: a workgroup of NT threads owns one chunk (GROUPS * L tokens) of a (batch,
// channel tile) row; a tile is 64 channels (one 128-byte line of bf16 k, two of fp32), so every
// load and store of a wavefront moves whole lines.
// ---------------------------------------------------------------------------------------------
//
// Lane (c, g) holds channel c of the tile and token group g (L consecutive tokens) in registers
// from load to store. The GROUPS = NT / TILE group sums of a channel are combined by scans on
// lane shuffles: the sums go through LDS into a transposed layout in which one channel's groups
// are consecutive lanes of one wavefront. A row of several chunks is combined in one of two ways:
//
//  * single pass (every workgroup of the launch fits on the device at once): each workgroup
//    publishes its chunk's forward and backward sums (epoch-tagged slots, see slot_store) and
//    folds the sums of the other chunks of its row, in a fixed order, into its carries. Every
//    wait is bounded; a workgroup that does not see a peer's sums in time recomputes them from
//    that chunk's k and v in HBM (the sums are plain decayed sums of Eq. (6)), so the result
//    never depends on the peers being resident.
//  * two passes: a sums launch writes every chunk's totals, and an output launch folds them into
//    its carries; nothing waits.
//
// Each lane then sweeps its tokens in sub-blocks of 8: forward states (a, c) left to right, then
// backward states (b, d) right to left, writing Eq. (7).
//
// Every lane holds exactly L token slots. Slots past the end of the row hold k = -inf, i.e. a
// weight of exactly 0, so the sweeps need no per-token bounds: a lane's forward sum is anchored
// at its last slot, and such slots are only ever followed by more empty slots. Loads and stores
// go through range-checked buffer resources that start at the chunk, so slots past the row read 0
// and their stores are dropped by the hardware, and the 32-bit offsets only span one chunk.

// Per-lane token storage: bf16 k and v packed in one 32-bit register per token (k in the low
// half, v in the high half); fp32 k and v in two registers. fence() makes the stored words
// opaque to the compiler (no instruction), so values unpacked in one phase are not kept live
// into the next one: unpacking again is cheaper than the registers. pad(n, odd) sets k = -inf in
// slots n and later (on the words as loaded); prepare(q) makes sub-block q readable through
// k() and v() (a no-op unless words are shared between lanes).
template <int DT, int L>
struct RowKV;

template <int L>
struct RowKV<BIWKV_BF16, L> {
  uint32_t r[L];
  __device__ __forceinline__ float k(int i) const { return __uint_as_float(r[i] << 16); }
  __device__ __forceinline__ float v(int i) const { return __uint_as_float(r[i] & 0xffff0000u); }
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int i = 0; i < L; ++i) asm volatile("" : "+v"(r[i]));
  }
  __device__ __forceinline__ void pad(int n, int) {
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (i >= n) r[i] = (r[i] & 0xffff0000u) | 0xff80u;
  }
  __device__ __forceinline__ void prepare(int) {}
};

template <int L>
struct RowKV<BIWKV_F32, L> {
  float kk[L], vv[L];
  __device__ __forceinline__ float k(int i) const { return kk[i]; }
  __device__ __forceinline__ float v(int i) const { return vv[i]; }
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int i = 0; i < L; ++i) asm volatile("" : "+v"(kk[i]), "+v"(vv[i]));
  }
  __device__ __forceinline__ void pad(int n, int) {
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (i >= n) kk[i] = kNegInf;
  }
  __device__ __forceinline__ void prepare(int) {}
};

// bf16 with channel pairs: lanes 2j and 2j+1 load channels (2j, 2j+1) as one 32-bit word, the
// even lane at even tokens and the odd lane at odd tokens, so 32-bit loads land in the final
// registers. prepare() swaps 16-bit halves with the neighbour lane, after which a lane keeps its
// own channel at two consecutive tokens in each register (k[2m] | k[2m+1] << 16, likewise v).
template <int L>
struct RowKVPair {
  static_assert(L % 2 == 0, "paired storage needs an even token count");
  uint32_t kk[L / 2], vv[L / 2];
  __device__ __forceinline__ float k(int i) const {
    return __uint_as_float((i & 1) ? (kk[i >> 1] & 0xffff0000u) : (kk[i >> 1] << 16));
  }
  __device__ __forceinline__ float v(int i) const {
    return __uint_as_float((i & 1) ? (vv[i >> 1] & 0xffff0000u) : (vv[i >> 1] << 16));
  }
  __device__ __forceinline__ void fence() {
#pragma unroll
    for (int m = 0; m < L / 2; ++m) asm volatile("" : "+v"(kk[m]), "+v"(vv[m]));
  }
  __device__ __forceinline__ void pad(int n, int odd) {
#pragma unroll
    for (int m = 0; m < L / 2; ++m)
      if (2 * m + odd >= n) kk[m] = 0xff80ff80u;  // this lane loaded token 2m + odd
  }
  // sub-block q covers words [q * 4, q * 4 + 4) (8 tokens)
  __device__ __forceinline__ void prepare(int q) {
    // even lane: (own low, neighbour low); odd lane: (neighbour high, own high)
    const uint32_t sel = (threadIdx.x & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int m = q * 4; m < q * 4 + 4; ++m) {
      const uint32_t nk = __builtin_amdgcn_mov_dpp(kk[m], 0xB1, 0xf, 0xf, false);
      const uint32_t nv = __builtin_amdgcn_mov_dpp(vv[m], 0xB1, 0xf, 0xf, false);
      kk[m] = __builtin_amdgcn_perm(nk, kk[m], sel);
      vv[m] = __builtin_amdgcn_perm(nv, vv[m], sel);
    }
  }
};

// Raw buffer resource over n_bytes at base (both uniform over the wavefront; they are read from
// the first lane so that the resource lives in scalar registers). The range check covers the
// whole offset (it is all passed in the vector offset): an offset at or past n_bytes reads 0
// and drops a store.
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long a) {
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t n_bytes) {
  void* ub = reinterpret_cast<void*>(uniform_u64(reinterpret_cast<unsigned long long>(base)));
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0),
                                           static_cast<int>(__builtin_amdgcn_readfirstlane(n_bytes)),
                                           0x00020000);
}
// Cache policy of the k, v loads and the out stores: non-temporal (each byte is touched once, so
// nothing is worth keeping in L2 or the memory-side cache; it measures about 1.6x faster than the
// default policy for these access patterns on MI355X).
constexpr int kStream = 2;
// Byte offset of a skipped access: past every resource (the host keeps a batch item's k, v and
// out below 2^31 bytes), and adding up to 2^31 - 1 more does not wrap.
constexpr uint32_t kOutOfRange = 0x80000000u;

// How a launch combines the chunks of a row (one chunk per row needs neither).
enum : int {
  kSinglePass = 0,  // slot exchange between resident workgroups, recompute on a timed-out wait
  kSumsPass = 1,    // two passes, first: write every chunk's totals to RowParams::sums
  kOutPass = 2,     // two passes, second (after row_carry_kernel): the chunk's carries, then the
                    // outputs
};

struct RowParams {
  const void* k;
  const void* v;
  const void* r;  // gate input of Eq. (2), [B, T, C] like k (gated entry only)
  const float* w;
  const float* u;
  float* out;
  long long T;
  int C;
  int n_tiles;   // channel tiles per batch item
  int n_chunks;  // workgroups per row
  unsigned total;                // workgroups of the launch
  unsigned spin_limit;           // single pass: polls of a peer's slot before recomputing its sums
                                 // (0: recompute every peer without polling)
  Counters* ctr;                 // single pass: epoch block (n_chunks > 1)
  unsigned long long* slots;     // single pass: [row][chunk][dir][TILE] (q, l, mu) tagged slot words
  float4* sums;                  // two passes: [row][chunk][dir][TILE] (q, l, mu) chunk totals
  float4* carries;               // two passes: [row][chunk][dir][TILE] (q, l, mu) exclusive carries
  int H, W, shift, g1, g2, g3, g4;  // Q-Shift (fused entry only)
  int bidir;  // fused: the bidirectional shift along a sparse token sequence (the host sets W = 1)
  // single pass: rows [0, xcd_rows) run every chunk on one XCD and exchange through its L2
  // (blocks go to the n_xcd XCDs round robin); 0 keeps the plain order
  int xcd_rows, n_xcd;
};

// Counts a workgroup out of a single-pass launch once none of its wavefronts reads the epoch or a
// slot again; the last one resets the count and moves the epoch on for the next launch on the
// stream. The count is issued before the sweeps and its result looked at after them
// (row_retire_end), so its round trip hides behind the sweeps instead of delaying the calling
// wavefront's.
__device__ __forceinline__ unsigned row_retire_begin(const RowParams& p) {
  return __hip_atomic_fetch_add(&p.ctr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr unsigned kNotRetiring = ~0u;
__device__ __forceinline__ void row_retire_end(const RowParams& p, unsigned fin) {
  if (fin != kNotRetiring && fin + 1u == p.total) {
    __hip_atomic_store(&p.ctr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&p.ctr->epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Whether any thread of the workgroup has pred set (a barrier). The result is read from the first
// lane so that the compiler sees a uniform value and branches on it without linearising both
// sides.
__device__ __forceinline__ bool block_any(bool pred) {
  return __builtin_amdgcn_readfirstlane(__syncthreads_or(pred) ? 1 : 0) != 0;
}

// Per-lane constants: lane (c, g) of the workgroup for chunk `chunk` of row `row` holds channel
// ch = tile * TILE + c at the tokens [s_g, s_g + n_g) of batch item b (n_g < L only at the end
// of a row).
struct RowLane {
  long long b, s_g;
  int row, chunk, c, g, ch, n_g;
  bool on;
  float D, lam, U, grow, eU;
};

template <int TILE, int L, int NT>
__device__ __forceinline__ RowLane row_lane_index(const RowParams& p, unsigned unit) {
  constexpr int CT = (NT / TILE) * L;  // tokens per chunk
  RowLane ln;
  const int tid = threadIdx.x;
  ln.c = tid % TILE;
  ln.g = tid / TILE;
  // integer division runs on the vector unit: read the (uniform) results back into scalars
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
  const int bi = __builtin_amdgcn_readfirstlane(ln.row / p.n_tiles);
  const int tile = ln.row - bi * p.n_tiles;
  ln.b = bi;
  ln.ch = tile * TILE + ln.c;
  ln.on = ln.ch < p.C;
  ln.s_g = static_cast<long long>(ln.chunk) * CT + static_cast<long long>(ln.g) * L;
  const long long rem = p.T - ln.s_g;
  ln.n_g = rem <= 0 ? 0 : (rem < L ? static_cast<int>(rem) : L);
  return ln;
}

// The lane's per-channel constants from its w and u (0 for a masked lane).
__device__ __forceinline__ void row_lane_params(RowLane& ln, long long T, float wc, float uc) {
  ln.D = (wc / static_cast<float>(T)) * kLog2e;
  ln.lam = fast_exp2(-ln.D);
  ln.U = uc * kLog2e;
  ln.grow = fmaxf(-ln.D, 0.f);
  ln.eU = fast_exp2(ln.U);
}

template <int TILE, int L, int NT>
__device__ __forceinline__ RowLane row_lane(const RowParams& p, unsigned unit) {
  RowLane ln = row_lane_index<TILE, L, NT>(p, unit);
  row_lane_params(ln, p.T, ln.on ? p.w[ln.ch] : 0.f, ln.on ? p.u[ln.ch] : 0.f);
  return ln;
}

// Loads word m of the lane's k and v (one token, or a channel pair at one token) at byte offset off
// of the resources km and vm, with cache policy POL.
template <int DT, bool PAIR, int POL, class Store>
__device__ __forceinline__ void row_load_word(Store& kv, int m, __amdgpu_buffer_rsrc_t km,
                                              __amdgpu_buffer_rsrc_t vm, uint32_t off) {
  if constexpr (PAIR) {
    kv.kk[m] = __builtin_amdgcn_raw_buffer_load_b32(km, off, 0, POL);
    kv.vv[m] = __builtin_amdgcn_raw_buffer_load_b32(vm, off, 0, POL);
  } else if constexpr (DT == BIWKV_F32) {
    kv.kk[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(km, off, 0, POL));
    kv.vv[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vm, off, 0, POL));
  } else {
    const uint32_t kx = __builtin_amdgcn_raw_buffer_load_b16(km, off, 0, POL);
    const uint32_t vx = __builtin_amdgcn_raw_buffer_load_b16(vm, off, 0, POL);
    kv.r[m] = kx | (vx << 16);
  }
}

// Bytes of a resource that starts `start` bytes into an array of `size` bytes: what is left of the
// array, clamped to what a 32-bit range check can express (an offset inside one chunk never
// reaches the clamp, so the check still drops exactly the accesses past the array).
__device__ __forceinline__ uint32_t row_span(long long size, long long start) {
  const long long left = size - start;
  return static_cast<uint32_t>(left <= 0 ? 0 : (left < 0x7fffffffll ? left : 0x7fffffffll));
}

// Issues every load of the lane's k and v (Q-Shift applied when FUSED: padded sources read 0) and
// marks the slots past the row empty. Nothing waits here: phase A consumes the words in load
// order as they arrive. Every resource starts at (or, fused, s W tokens before) the chunk, so the
// 32-bit offsets span one chunk whatever the size of a batch item.
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, int POL, class Store>
__device__ __forceinline__ void row_load(const RowParams& p, const RowLane& ln, Store& kv) {
  const long long T = p.T;
  const int C = p.C;
  const long long plane = T * C;  // elements of one batch item
  constexpr int ES = DT == BIWKV_F32 ? 4 : 2;
  const long long item = plane * ES;  // bytes of one batch item
  const char* kb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.k) + ln.b * item));
  const char* vb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.v) + ln.b * item));
  const uint32_t row_bytes = static_cast<uint32_t>(C) * ES;
  // PAIR: lane 2j + odd reads channels (2j, 2j + 1) at tokens 2m + odd
  constexpr int STEP = PAIR ? 2 : 1;
  constexpr int NW = L / STEP;  // words per lane and array
  const int odd = PAIR ? (ln.c & 1) : 0;
  const uint32_t lane_byte = static_cast<uint32_t>(ln.ch - odd) * ES;
  constexpr int CT = (NT / TILE) * L;
  if constexpr (!FUSED) {
    // One resource per array from the chunk's start to the end of the batch item; word m adds its
    // token offset to the lane's vector offset (one add, no scalar work per word: sixteen
    // wavefronts of a CU share one scalar unit). Tokens past the row fall past the resource and
    // read 0, and so does every slot of a masked lane.
    const long long c0 = static_cast<long long>(ln.chunk) * CT * row_bytes;  // chunk start
    // offsets below 2^31 (the host checks CT * C * 4)
    const uint32_t lane_off =
        ln.on ? static_cast<uint32_t>(ln.g * L + odd) * row_bytes + lane_byte : kOutOfRange;
    const uint32_t n = row_span(item, c0);
    const __amdgpu_buffer_rsrc_t km = make_rsrc(kb + c0, n);
    const __amdgpu_buffer_rsrc_t vm = make_rsrc(vb + c0, n);
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      row_load_word<DT, PAIR, POL>(kv, m, km, vm, lane_off + static_cast<uint32_t>(m * STEP) * row_bytes);
      __builtin_amdgcn_sched_barrier(0);  // each word's offset formed just before its loads
    }
  } else {
    // Q-Shift: the lane reads its own channel at token t + delta, where delta is fixed by the
    // channel's quarter (right: -s, left: +s, down: -s W, up: +s W, rest: 0). The resources start
    // SH = s W tokens before the chunk, so every lane offset is non-negative; word m adds its token
    // offset, and sources past the end of the batch item fall past the resource and read 0. The
    // other zero-filled sources (a column outside the quarter's band, or a row above the grid for
    // "down") are cleared words of a per-lane mask, set once. The bidirectional shift of a sparse
    // sequence (W = 1) moves the right and down groups by -s and the left and up groups by +s, with
    // no column bands: only the first s tokens of the -s groups are cleared.
    const int Wd = p.W, sh = p.shift, SH = p.shift * p.W;
    int delta = 0, lo = 0, hi = Wd;  // valid columns [lo, hi)
    bool down = false;
    if (p.bidir) {
      if (ln.ch < p.g4) {
        down = ln.ch < p.g1 || (ln.ch >= p.g2 && ln.ch < p.g3);
        delta = down ? -sh : sh;
      }
    } else if (ln.ch < p.g1) {
      delta = -sh;
      lo = sh;
    } else if (ln.ch < p.g2) {
      delta = sh;
      hi = Wd - sh;
    } else if (ln.ch < p.g3) {
      delta = -SH;
      down = true;
    } else if (ln.ch < p.g4) {
      delta = SH;
    }
    const int t0 = ln.chunk * CT + ln.g * L + odd;  // token of word 0 (T < 2^31)
    // bit m: word m (token t0 + STEP m) reads a source inside the grid
    using Mask = std::conditional_t<(NW > 32), unsigned long long, uint32_t>;
    constexpr int MB = 8 * sizeof(Mask);
    auto below = [](int n) { return n >= MB ? ~Mask(0) : (Mask(1) << n) - Mask(1); };  // bits [0, n)
    Mask valid = ln.on ? below(NW) : Mask(0);
    // clears the words whose token lies in [a, b)
    auto clear = [&](int a, int b) {
      int ma = (a - t0 + STEP - 1) >> (STEP - 1), mb = (b - t0 + STEP - 1) >> (STEP - 1);
      ma = ma < 0 ? 0 : (ma > NW ? NW : ma);
      mb = mb < 0 ? 0 : (mb > NW ? NW : mb);
      valid &= ~(below(mb) & ~below(ma));
    };
    if (lo > 0 || hi < Wd) {
      const int t_last = t0 + STEP * (NW - 1);
      for (int r = t0 / Wd; r * Wd <= t_last; ++r) {
        clear(r * Wd, r * Wd + lo);
        clear(r * Wd + hi, r * Wd + Wd);
      }
    }
    if (down) clear(t0, SH);
    // offsets below 2^31 (the host checks (CT + 2 s W) * C * 4)
    const uint32_t lane_off = static_cast<uint32_t>(ln.g * L + odd + delta + SH) * row_bytes + lane_byte;
    const long long c0 = (static_cast<long long>(ln.chunk) * CT - SH) * row_bytes;  // may be negative
    const uint32_t n = row_span(item, c0);
    const __amdgpu_buffer_rsrc_t km = make_rsrc(kb + c0, n);
    const __amdgpu_buffer_rsrc_t vm = make_rsrc(vb + c0, n);
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      // all ones when word m is valid (bit m of the mask, sign-extended)
      const uint32_t keep =
          static_cast<uint32_t>(static_cast<std::make_signed_t<Mask>>(valid << (MB - 1 - m)) >> (MB - 1));
      const uint32_t off = ((lane_off + static_cast<uint32_t>(m * STEP) * row_bytes) & keep) | (kOutOfRange & ~keep);
      row_load_word<DT, PAIR, POL>(kv, m, km, vm, off);
      __builtin_amdgcn_sched_barrier(0);  // each word's offset formed just before its loads
    }
  }
  // all loads in flight before anything consumes them
  __builtin_amdgcn_sched_barrier(0);
  if (__ballot(ln.n_g < L) != 0ull) kv.pad(ln.n_g, odd);  // only waves at the end of a row
}

// One chunk whose loads are issued: lane sums (phase A), scan over the groups and exchange with
// the other chunks, sweeps (phase C). WIDE selects the per-token running-maximum arithmetic; the fast form scales
// the terms of a sub-block against one exponent, which keeps every significant term a normal
// fp32 number while the decay or growth across a lane stays within kFastRange.
// LDS of the tile kernel: the wide form's per-token sweep buffer (8 tokens x NT lanes of float2),
// which first holds the lane sums, then the carries and the per-channel D outside it.
template <int NT>
constexpr int kRowSweepFloats = 8 * NT * 3;
// Row pitch of the group-major lane-sum and carry buffers. Lane (tg, tc) of the transposed layout
// reads word tg * pitch + tc with tg = lane % GROUPS: a pitch of TILE + 64 / GROUPS puts the 64
// lanes of a wavefront on 64 different banks (a pitch of TILE + 1 put up to 8 on one).
template <int TILE, int NT>
constexpr int kRowPad = TILE + (NT / TILE < 64 ? 64 / (NT / TILE) : 1);
template <int TILE, int NT>
constexpr int kRowLdsFloats = kRowSweepFloats<NT> + 8 * (NT / TILE) * kRowPad<TILE, NT> + TILE;

// Single-exponent sums with a finite empty exponent (kEmptyM), so that adding them needs no
// branch: the fast form's addition, also used by the backward's scans.
__device__ __forceinline__ Agg row_empty() { return Agg{kEmptyM, 0.f, 0.f}; }
__device__ __forceinline__ Agg agg_add_f(Agg a, Agg b) {
  const float m = fmaxf(a.m, b.m);
  const float sa = fast_exp2(a.m - m), sb = fast_exp2(b.m - m);
  return Agg{m, fmaf(a.F, sa, b.F * sb), fmaf(a.G, sa, b.G * sb)};
}

// One DPP move of a float across the lanes of a row (CTRL: the DPP control word).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// The tile kernel works on single-exponent sums (Agg) in the fast form and on sums with exact
// token counts (Sum) in the wide form; these overloads let the scans and the exchange serve both.
template <class A>
__device__ __forceinline__ A acc_empty();
template <>
__device__ __forceinline__ Agg acc_empty<Agg>() { return agg_none(); }
template <>
__device__ __forceinline__ Sum acc_empty<Sum>() { return sum_empty(); }
__device__ __forceinline__ Agg acc_add(Agg a, Agg b, float) { return agg_add_f(a, b); }
__device__ __forceinline__ Sum acc_add(Sum a, Sum b, float D) { return sum_add(a, b, D); }
__device__ __forceinline__ Agg acc_shift(Agg a, float n, float D) { return agg_shift(a, n, D); }
__device__ __forceinline__ Sum acc_shift(Sum a, float n, float) { return sum_shift(a, n); }
// A two-pass total or carry as the kernel's sum type (a fast-form row's exponents are small, so
// q D + l is exact enough there).
template <class A>
__device__ __forceinline__ A acc_unpack(float4 s, float D);
template <>
__device__ __forceinline__ Sum acc_unpack<Sum>(float4 s, float) { return slot_unpack(s); }
template <>
__device__ __forceinline__ Agg acc_unpack<Agg>(float4 s, float D) {
  if (!(s.y > kEmptyM)) return agg_none();
  return Agg{fmaf(s.x, D, s.y), s.z, 1.f};
}
// Sums in LDS: quantity j of lane i at base[j * RS + i] (3 quantities for Agg, 4 for Sum).
__device__ __forceinline__ void acc_put(float* base, int RS, int i, const Agg& a) {
  base[0 * RS + i] = a.m;
  base[1 * RS + i] = a.F;
  base[2 * RS + i] = a.G;
}
__device__ __forceinline__ void acc_put(float* base, int RS, int i, const Sum& a) {
  base[0 * RS + i] = a.m;
  base[1 * RS + i] = a.F;
  base[2 * RS + i] = a.G;
  base[3 * RS + i] = a.q;
}
template <class A>
__device__ __forceinline__ A acc_get(const float* base, int RS, int i);
template <>
__device__ __forceinline__ Agg acc_get<Agg>(const float* base, int RS, int i) {
  return Agg{base[0 * RS + i], base[1 * RS + i], base[2 * RS + i]};
}
template <>
__device__ __forceinline__ Sum acc_get<Sum>(const float* base, int RS, int i) {
  return Sum{base[3 * RS + i], base[0 * RS + i], base[1 * RS + i], base[2 * RS + i]};
}

// Sums moved between the W consecutive lanes that hold one channel's groups (W is a power of two
// up to 64). from_below<W, d> gives a lane the value of the lane d below it and from_above<W, d>
// that of the lane d above; the callers only use results from inside the segment. Segments of up
// to 16 lanes lie inside one DPP row, so these are row shifts (plain VALU moves); wider segments go
// through the LDS crossbar (ds_bpermute).
template <int W, int d>
__device__ __forceinline__ float lane_from_below(float x) {
  if constexpr (W <= 16)
    return dpp_move<0x110 + d>(x);  // row_shr
  else
    return __shfl_up(x, d, W);
}
template <int W, int d>
__device__ __forceinline__ float lane_from_above(float x) {
  if constexpr (W <= 16)
    return dpp_move<0x100 + d>(x);  // row_shl
  else
    return __shfl_down(x, d, W);
}
template <int W, int d>
__device__ __forceinline__ Agg acc_from_below(Agg a) {
  return Agg{lane_from_below<W, d>(a.m), lane_from_below<W, d>(a.F), lane_from_below<W, d>(a.G)};
}
template <int W, int d>
__device__ __forceinline__ Sum acc_from_below(Sum a) {
  return Sum{lane_from_below<W, d>(a.q), lane_from_below<W, d>(a.m), lane_from_below<W, d>(a.F),
             lane_from_below<W, d>(a.G)};
}
template <int W, int d>
__device__ __forceinline__ Agg acc_from_above(Agg a) {
  return Agg{lane_from_above<W, d>(a.m), lane_from_above<W, d>(a.F), lane_from_above<W, d>(a.G)};
}
template <int W, int d>
__device__ __forceinline__ Sum acc_from_above(Sum a) {
  return Sum{lane_from_above<W, d>(a.q), lane_from_above<W, d>(a.m), lane_from_above<W, d>(a.F),
             lane_from_above<W, d>(a.G)};
}
template <int W>
__device__ __forceinline__ Agg acc_from_first(Agg a) {
  return Agg{__shfl(a.m, 0, W), __shfl(a.F, 0, W), __shfl(a.G, 0, W)};
}
template <int W>
__device__ __forceinline__ Sum acc_from_first(Sum a) {
  return Sum{__shfl(a.q, 0, W), __shfl(a.m, 0, W), __shfl(a.F, 0, W), __shfl(a.G, 0, W)};
}

// Inclusive scans over the W groups of a channel (lane tg holds group tg; groups are L slots
// apart): forward over groups 0..tg, anchored at tg's last slot, and (BWD) backward over
// tg..W-1, anchored at tg's first token. Hillis-Steele, fixed order.
template <int W, int L, bool BWD, int d = 1, class A>
__device__ __forceinline__ void group_scan(A& f, A& bk, int tg, float D) {
  if constexpr (d < W) {
    const A pf = acc_from_below<W, d>(f);
    if (tg >= d) f = acc_add(acc_shift(pf, static_cast<float>(d * L), D), f, D);
    if constexpr (BWD) {
      const A pb = acc_from_above<W, d>(bk);
      if (tg + d < W) bk = acc_add(bk, acc_shift(pb, static_cast<float>(d * L), D), D);
    }
    group_scan<W, L, BWD, 2 * d>(f, bk, tg, D);
  }
}

// Folds the W lanes' sums (a, and b when BWD) into the segment's first lane in a fixed tree.
template <int W, bool BWD, int s = 1, class A>
__device__ __forceinline__ void group_fold(A& a, A& b, int tg, float D) {
  if constexpr (s < W) {
    const A oa = acc_from_above<W, s>(a);
    if ((tg & (2 * s - 1)) == 0) a = acc_add(a, oa, D);
    if constexpr (BWD) {
      const A ob = acc_from_above<W, s>(b);
      if ((tg & (2 * s - 1)) == 0) b = acc_add(b, ob, D);
    }
    group_fold<W, BWD, 2 * s>(a, b, tg, D);
  }
}

// One token of channel ch of batch item b as the chunk's sums see it (Q-Shift applied when FUSED;
// a zero-filled source is k = 0, v = 0), by plain loads. Used only to recompute a peer chunk's sums.
template <int DT, bool FUSED>
__device__ __forceinline__ void row_token(const RowParams& p, long long b, int ch, long long t, float& kf,
                                          float& vf) {
  long long src = t;
  bool ok = true;
  if constexpr (FUSED) {
    const long long s = p.shift, W = p.W;
    if (p.bidir) {
      if (ch < p.g4) {
        const bool back = ch < p.g1 || (ch >= p.g2 && ch < p.g3);
        src = back ? t - s : t + s;
        ok = src >= 0 && src < p.T;
      }
    } else {
      const long long col = t % W;
      if (ch < p.g1) {
        ok = col >= s;
        src = t - s;
      } else if (ch < p.g2) {
        ok = col < W - s;
        src = t + s;
      } else if (ch < p.g3) {
        ok = t >= s * W;
        src = t - s * W;
      } else if (ch < p.g4) {
        ok = t < static_cast<long long>(p.H - s) * W;
        src = t + s * W;
      }
    }
  }
  if (!ok) {
    kf = 0.f;
    vf = 0.f;
    return;
  }
  const long long idx = (b * p.T + src) * p.C + ch;
  if constexpr (DT == BIWKV_F32) {
    kf = static_cast<const float*>(p.k)[idx];
    vf = static_cast<const float*>(p.v)[idx];
  } else {
    kf = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p.k)[idx]) << 16);
    vf = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p.v)[idx]) << 16);
  }
}

// The sums of chunk ck of batch item b, channel ch, recomputed from k and v: forward anchored at
// the chunk's last slot, or backward anchored at its first token. This is what the chunk
// publishes, so a workgroup whose wait for a peer runs out takes it from here instead; a masked
// channel gives the empty sum. Each token enters with its exact distance to the anchor, and the
// terms are summed against their running maximum, so any w, u and k stay finite and accurate.
template <int DT, int CT, bool FUSED>
__device__ __noinline__ Sum row_recompute(const RowParams* args, long long b, int ch, int ck, bool fwd, float D) {
  const RowParams& p = *args;
  if (ch >= p.C) return sum_empty();
  const long long s = static_cast<long long>(ck) * CT;
  const long long e = s + CT < p.T ? s + CT : p.T;  // exclusive
  const long long anchor = fwd ? s + CT - 1 : s;
  Sum a = sum_empty();
#pragma unroll 8
  for (long long t = s; t < e; ++t) {
    float kf, vf;
    row_token<DT, FUSED>(p, b, ch, t, kf, vf);
    const float n = static_cast<float>(fwd ? anchor - t : t - anchor);  // distance to the anchor
    a = sum_add(a, Sum{-n, kf * kLog2e, vf, 1.f}, D);
  }
  return a;
}

// Gate inputs r of Eq. (2) for the SB tokens of a lane's sub-block q (raw bits: an fp32 value, or
// a bf16 value in the low half), through per-token resources like the unfused k, v loads.
template <int DT, int TILE, int L, int NT, int SB>
struct RowGate {
  const char* base;   // the chunk's first token of r in the lane's batch item
  long long left;     // bytes from there to the end of the batch item
  uint32_t lane_off;  // this lane's offset from the chunk start (out of range when masked)
  int row_bytes;
  __device__ __forceinline__ void init(const RowParams& p, const RowLane& ln) {
    constexpr int ES = DT == BIWKV_F32 ? 4 : 2;
    constexpr int CT = (NT / TILE) * L;
    const long long item = p.T * p.C * ES;
    row_bytes = p.C * ES;
    const long long c0 = static_cast<long long>(ln.chunk) * CT * row_bytes;
    base = reinterpret_cast<const char*>(
        uniform_u64(reinterpret_cast<unsigned long long>(p.r) + ln.b * item + c0));
    left = item - c0;
    lane_off = ln.on ? static_cast<uint32_t>(ln.g * L) * row_bytes + static_cast<uint32_t>(ln.ch) * ES
                     : kOutOfRange;
  }
  __device__ __forceinline__ void load(int q, uint32_t (&dst)[SB]) const {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const long long adv = static_cast<long long>(q * SB + i) * row_bytes;
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(base + adv, row_span(left, adv));
      if constexpr (DT == BIWKV_F32)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b32(rr, lane_off, 0, kStream);
      else
        dst[i] = __builtin_amdgcn_raw_buffer_load_b16(rr, lane_off, 0, kStream);
    }
  }
  __device__ __forceinline__ static float value(uint32_t bits) {
    return __uint_as_float(DT == BIWKV_F32 ? bits : (bits << 16));
  }
};

template <int DT, int TILE, int L, bool PAIR>
using RowStore = std::conditional_t<PAIR, RowKVPair<L>, RowKV<DT, L>>;

// CAUSAL: the causal attention (Eq. (7) without the backward states b, d): only forward sums
// are formed, scanned and exchanged, and the output comes out of the forward sweep. MODE: how the
// chunks of a row are combined (kSinglePass, kSumsPass, kOutPass). Returns false only in the fast
// form of a single pass whose wait for a peer ran out: nothing is stored then, and the caller
// runs the chunk again through the wide form, which recomputes the missing sums (its own slot is
// already published: `published`).
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool WIDE, bool CAUSAL, bool GATED, int MODE>
__device__ __forceinline__ bool row_body(const RowParams& p, const RowParams* args, const RowLane& ln,
                                         RowStore<DT, TILE, L, PAIR>& kv, float* lds,
                                         unsigned epoch_raw, bool published, unsigned& fin) {
  constexpr int GROUPS = NT / TILE;
  constexpr int CT = GROUPS * L;  // tokens per chunk
  constexpr int SB = 8;  // tokens per sub-block of the sweeps
  // the fast form's sums keep one exponent; the wide form's keep exact token counts
  using A = std::conditional_t<WIDE, Sum, Agg>;
  constexpr int NSB = L / SB;
  static_assert(L % SB == 0, "bad row-kernel shape");
  static_assert((GROUPS & (GROUPS - 1)) == 0 && GROUPS <= 64, "a channel's groups share a wavefront");
  // wide-form sweep records, per token of a sub-block: the prefix mean, and the prefix weight's
  // exponent as (token count, rest)
  float (*lds_al)[NT] = reinterpret_cast<float (*)[NT]>(lds);
  float (*lds_pq)[NT] = reinterpret_cast<float (*)[NT]>(lds + SB * NT);
  float (*lds_pm)[NT] = reinterpret_cast<float (*)[NT]>(lds + 2 * SB * NT);
  const int tid = threadIdx.x;
  const int g = ln.g;
  const long long T = p.T;
  const int C = p.C;
  const float D = ln.D, lam = ln.lam, grow = ln.grow;
  const float span = grow * static_cast<float>(L - 1);  // largest growth inside one lane

  // ---- phase A: lane sums (forward anchored at its last slot, backward at its first) and, per
  //      sub-block, the backward sum of everything after it inside the lane ----
  A af, ab;
  float kmax = kNegInf;
  float capF[WIDE ? 1 : NSB], capG[WIDE ? 1 : NSB];  // fast form: anchored at (q + 1) * SB
  Sum cap[WIDE ? NSB : 1];                           // wide form
  if constexpr (!WIDE) {
    // Each sub-block's terms are formed against its own largest key mq (k log2 e), as
    // 2^{k log2 e - mq - span} <= 1, and the running forward sum is rescaled when a larger key
    // arrives: any keys are safe, and a sub-block is processed as soon as its words arrive.
    const float lsb = fast_exp2(-static_cast<float>(SB) * D);  // lam^SB
    float mrun = kNegInf;  // the forward sums (fF, fG) are against 2^{mrun + span}
    float fF = 0.f, fG = 0.f;
    float bF[NSB], bG[NSB], bm[NSB];  // backward sum of each sub-block, anchored at its first
                                      // token, against 2^{bm + span}
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      kv.prepare(q);  // waits only for this sub-block's words
      float mq = kNegInf;
#pragma unroll
      for (int i = 0; i < SB; ++i) mq = fmaxf(mq, kv.k(q * SB + i));
      mq *= kLog2e;
      const float ref = mq == kNegInf ? 0.f : mq + span;  // an empty sub-block has only 0 terms
      float pp[SB], pv[SB];
      float qF = 0.f, qG = 0.f;
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int t = q * SB + i;
        pp[i] = fast_exp2(fmaf(kv.k(t), kLog2e, -ref));
        pv[i] = pp[i] * kv.v(t);
        qF = fmaf(qF, lam, pv[i]);
        qG = fmaf(qG, lam, pp[i]);
      }
      if constexpr (!CAUSAL) {
        bF[q] = pv[SB - 1];
        bG[q] = pp[SB - 1];
#pragma unroll
        for (int i = SB - 2; i >= 0; --i) {
          bF[q] = fmaf(bF[q], lam, pv[i]);
          bG[q] = fmaf(bG[q], lam, pp[i]);
        }
        bm[q] = mq;
      }
      // move the running sums SB tokens on and add this sub-block at the larger exponent
      const float mn = fmaxf(mrun, mq);
      const float mr = mn == kNegInf ? 0.f : mn;
      const float sr = fast_exp2(mrun - mr) * lsb, sq = fast_exp2(mq - mr);
      fF = fmaf(fF, sr, qF * sq);
      fG = fmaf(fG, sr, qG * sq);
      mrun = mn;
      __builtin_amdgcn_sched_barrier(0);  // one sub-block at a time (bounded live values)
    }
    kmax = mrun;  // largest key of the lane (-inf when it holds no token)
    const float mr = mrun == kNegInf ? 0.f : mrun;
    float cF = 0.f, cG = 0.f;
    if constexpr (!CAUSAL) {
#pragma unroll
      for (int q = NSB - 1; q >= 0; --q) {
        capF[q] = cF;
        capG[q] = cG;
        const float sq = fast_exp2(bm[q] - mr);
        cF = fmaf(cF, lsb, bF[q] * sq);
        cG = fmaf(cG, lsb, bG[q] * sq);
      }
    }
    // the lane sums and the caps are against 2^{kmax + span}
    const float m_agg = kmax == kNegInf ? kEmptyM : kmax + span;
    af = Agg{m_agg, fF, fG};
    ab = CAUSAL ? agg_none() : Agg{m_agg, cF, cG};
  } else {
#pragma unroll
    for (int q = 0; q < NSB; ++q) kv.prepare(q);
    // Wide range: one token at a time, each sum against its own running maximum; moving a sum
    // one token on only changes its token count (an empty slot, k = -inf, adds nothing).
    af = sum_empty();
#pragma unroll
    for (int i = 0; i < L; ++i) af = sum_add(sum_shift(af, 1.f), Sum{0.f, kv.k(i) * kLog2e, kv.v(i), 1.f}, D);
    ab = sum_empty();
    if constexpr (!CAUSAL) {
      Sum bs[NSB];
#pragma unroll
      for (int q = 0; q < NSB; ++q) {
        bs[q] = sum_empty();
#pragma unroll
        for (int i = (q + 1) * SB - 1; i >= q * SB; --i)
          bs[q] = sum_add(sum_shift(bs[q], 1.f), Sum{0.f, kv.k(i) * kLog2e, kv.v(i), 1.f}, D);
      }
#pragma unroll
      for (int q = NSB - 1; q >= 0; --q) {
        cap[q] = ab;
        ab = sum_add(bs[q], sum_shift(ab, static_cast<float>(SB)), D);
      }
    }
  }
  kv.fence();
  // GATED: the gate inputs of sub-block 0 load during the scan and the exchange
  RowGate<DT, TILE, L, NT, SB> gate;
  uint32_t r_next[GATED ? SB : 1];
  if constexpr (GATED && MODE != kSumsPass) {
    gate.init(p, ln);
    gate.load(0, r_next);
  }

  // ---- scans over the groups of each channel. The lane sums go to LDS group-major; lane
  //      (tg, tc) = (tid % GROUPS, tid / GROUPS) then takes group tg of channel tc, so the groups
  //      of a channel are GROUPS consecutive lanes of one wavefront and the scans (and the
  //      exchange) run on lane shuffles without barriers. Carries go back the same way. ----
  constexpr int PAD = kRowPad<TILE, NT>;  // row pitch of the group-major buffers
  constexpr int RS = GROUPS * PAD;      // floats per quantity
  float* red = lds;                     // [8][RS] lane sums (inside the sweep buffer)
  float* xy = lds + kRowSweepFloats<NT>;  // [8][RS] carries (outside it: read during the sweeps)
  float* dch = xy + 8 * RS;             // [TILE] D of each channel
  const int wi = g * PAD + ln.c;
  acc_put(red, RS, wi, af);
  acc_put(red + 4 * RS, RS, wi, ab);
  if (g == 0) dch[ln.c] = D;
  __syncthreads();
  const int tg = tid % GROUPS, tc = tid / GROUPS;
  const int ti = tg * PAD + tc;
  const float Dt = dch[tc];
  A f = acc_get<A>(red, RS, ti);
  A bk = acc_get<A>(red + 4 * RS, RS, ti);
  group_scan<GROUPS, L, !CAUSAL>(f, bk, tg, Dt);
  // exclusive carries: forward sum of the earlier groups (anchored just before the group's first
  // token), backward sum of the later groups (anchored just after its last slot)
  A X = acc_from_below<GROUPS, 1>(f), Y = acc_from_above<GROUPS, 1>(bk);
  if (tg == 0) X = acc_empty<A>();
  if (CAUSAL || tg == GROUPS - 1) Y = acc_empty<A>();
  bool timed_out = false;  // fast single pass: a peer's sums did not arrive in time
  if (p.n_chunks > 1) {
    // ---- the other chunks of the row ----
    const int nch = p.n_chunks, chunk = ln.chunk;
    const size_t row_base = static_cast<size_t>(ln.row) * nch * 2 * TILE;
    if constexpr (MODE == kSumsPass) {
      // the chunk's totals: forward (inclusive at the last group, anchored at the chunk's last
      // slot) and backward (inclusive at group 0, anchored at the chunk's first token)
      if (tg == GROUPS - 1) p.sums[row_base + (chunk * 2 + kFwd) * TILE + tc] = slot_pack(f);
      if (!CAUSAL && tg == 0) p.sums[row_base + (chunk * 2 + kBwd) * TILE + tc] = slot_pack(bk);
      return true;
    }
    if constexpr (MODE == kOutPass) {
      // the chunk's exclusive carries (row_carry_kernel): forward anchored just before the
      // chunk's first token, backward just after its last slot
      A pf = acc_empty<A>(), pb = acc_empty<A>();
      if (tg == 0) {
        pf = acc_unpack<A>(p.carries[row_base + (chunk * 2 + kFwd) * TILE + tc], Dt);
        if (!CAUSAL) pb = acc_unpack<A>(p.carries[row_base + (chunk * 2 + kBwd) * TILE + tc], Dt);
      }
      pf = acc_from_first<GROUPS>(pf);
      X = acc_add(acc_shift(pf, static_cast<float>(tg * L), Dt), X, Dt);
      if constexpr (!CAUSAL) {
        pb = acc_from_first<GROUPS>(pb);
        Y = acc_add(Y, acc_shift(pb, static_cast<float>((GROUPS - 1 - tg) * L), Dt), Dt);
      }
    } else {
    unsigned epoch = 0;
    unsigned long long* rs = p.slots + row_base * kSlotWords;
    auto slot = [&](int ck, int dir) { return rs + (static_cast<size_t>(ck * 2 + dir) * TILE + tc) * kSlotWords; };
    // rows whose chunks all run on one XCD exchange through its L2 (byte offsets into the slot
    // array, which a single pass keeps far below 4 GiB)
    const bool local = ln.row < p.xcd_rows;
    const long long slot_bytes = static_cast<long long>(p.total) * 2 * TILE * kSlotWords * 8;
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(p.slots, static_cast<uint32_t>(slot_bytes < 0xFFFFFFFFll ? slot_bytes : 0xFFFFFFFFll));
    auto soff = [&](const unsigned long long* sp) { return static_cast<uint32_t>((sp - p.slots) * 8); };
    auto put = [&](unsigned long long* sp, const A& a) {
      if (local)
        slot_store_l2(srs, soff(sp), a, epoch);
      else
        slot_store(sp, a, epoch);
    };
    auto get = [&](const unsigned long long* sp, unsigned long long* w) {
      if (local)
        slot_load_l2<A>(srs, soff(sp), w);
      else
        slot_load<A>(sp, w);
    };
    if constexpr (MODE == kSinglePass) {
      // the slots' tag: the launch's epoch + 1 (never 0, so zeroed slots never match, whatever the
      // counter block started at)
      epoch = __builtin_amdgcn_readfirstlane(epoch_raw) + 1u;
      // the chunk's own sums, anchored as the totals above
      if (!published) {
        if (tg == GROUPS - 1) put(slot(chunk, kFwd), f);
        if (!CAUSAL && tg == 0) put(slot(chunk, kBwd), bk);
      }
    }
    // Entries: forward sums of chunks 0 .. chunk-1, then backward sums of chunks chunk+1 ..
    // nch-1. Lane tg folds entries tg, tg + GROUPS, ... in order; the lanes' partials are then
    // folded in a fixed tree, so the result does not depend on arrival order.
    const int nf = chunk, ne = CAUSAL ? chunk : nch - 1;
    A pf = acc_empty<A>(), pb = acc_empty<A>();
    bool recomputed = false;
    // a poll limit of 0 recomputes every peer's sums without polling
    const bool poll = p.spin_limit != 0;
    // A lane issues the loads of up to EB entries before it waits for any of them, so a lane
    // with several entries pays one round trip, not one per entry.
    constexpr int EB = GROUPS >= 8 ? 1 : 8 / GROUPS;
    for (int e0 = tg; e0 < ne; e0 += EB * GROUPS) {
      unsigned long long wv[EB][kSlotUsed<A>];
      if (poll) {
#pragma unroll
        for (int j = 0; j < EB; ++j) {
          const int e = e0 + j * GROUPS;
          if (e < ne) get(slot(e < nf ? e : e + 1, e < nf ? kFwd : kBwd), wv[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        const int e = e0 + j * GROUPS;
        if (e >= ne) break;
        const bool fwd = e < nf;
        const int ck = fwd ? e : e + 1;
        // distance from the entry's anchor to this chunk's carry anchor (chunks before this one
        // are full, so slot positions are token positions)
        const float dist = static_cast<float>(fwd ? (chunk - 1 - ck) : (ck - chunk - 1)) * CT;
        A a;
        {
          const unsigned long long* sp = slot(ck, fwd ? kFwd : kBwd);
          bool ready = false;
          if (poll) {
            ready = slot_ready<A>(wv[j], epoch);
            if (!ready && GATED) {
              // one poll at a time: the gated kernel holds its first gate inputs in flight here,
              // and a second poll's registers cost it spills and waits
              for (unsigned spins = 0; spins < p.spin_limit && !ready; ++spins) {
                __builtin_amdgcn_s_sleep(2);
                get(sp, wv[j]);
                ready = slot_ready<A>(wv[j], epoch);
              }
            } else if (!ready) {
              // Two polls in flight, issued a short sleep apart: a slot published just after one
              // poll was served is seen by the next one instead of a full round trip later.
              unsigned long long w2[kSlotUsed<A>];
              get(sp, w2);
              for (unsigned spins = 0; spins < p.spin_limit; spins += 2) {
                __builtin_amdgcn_s_sleep(2);
                get(sp, wv[j]);
                if (slot_ready<A>(w2, epoch)) {  // the older poll
#pragma unroll
                  for (int x = 0; x < kSlotUsed<A>; ++x) wv[j][x] = w2[x];
                  ready = true;
                  break;
                }
                __builtin_amdgcn_s_sleep(2);
                get(sp, w2);
                if (slot_ready<A>(wv[j], epoch)) {
                  ready = true;
                  break;
                }
              }
            }
          }
          if (ready) {
            a = slot_value<A>(wv[j]);
          } else if constexpr (WIDE) {
            // the peer has not published in time (it may not be resident): its sums from k, v
            a = row_recompute<DT, CT, FUSED>(args, ln.b, ln.ch - ln.c + tc, ck, fwd, Dt);
            recomputed = true;
          } else {
            timed_out = true;
            a = acc_empty<A>();
          }
        }
        a = acc_shift(a, dist, Dt);
        if (fwd)
          pf = acc_add(pf, a, Dt);
        else
          pb = acc_add(pb, a, Dt);
      }
    }
    if constexpr (MODE == kSinglePass && WIDE) {
      if (recomputed)
        __hip_atomic_fetch_or(&p.ctr->fault, kFaultSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    group_fold<GROUPS, !CAUSAL>(pf, pb, tg, Dt);
    // pf (from the first lane of the channel) is anchored just before the chunk, pb just after it
    pf = acc_from_first<GROUPS>(pf);
    X = acc_add(acc_shift(pf, static_cast<float>(tg * L), Dt), X, Dt);
    if constexpr (!CAUSAL) {
      pb = acc_from_first<GROUPS>(pb);
      Y = acc_add(Y, acc_shift(pb, static_cast<float>((GROUPS - 1 - tg) * L), Dt), Dt);
    }
    }
  }
  acc_put(xy, RS, ti, X);
  acc_put(xy + 4 * RS, RS, ti, Y);
  // past this barrier the sum buffer becomes the (alpha, beta) buffer; the fast form of a single
  // pass gives up there as a workgroup if any wait ran out (the wide form recomputes what is
  // missing), having stored nothing
  if constexpr (MODE == kSinglePass && !WIDE) {
    if (block_any(timed_out)) return false;
  } else {
    __syncthreads();
  }
  X = acc_get<A>(xy, RS, wi);
  Y = acc_get<A>(xy + 4 * RS, RS, wi);
  // every wavefront is past its last read of the epoch and of the slots
  if (MODE == kSinglePass && p.n_chunks > 1 && tid == 0) fin = row_retire_begin(p);
  kv.fence();

  // ---- phase C: sweep each sub-block forward, then backward, writing Eq. (7) ----
  if (ln.n_g <= 0) return true;  // no barrier follows
  const long long plane = T * C;
  const long long o0 = static_cast<long long>(ln.chunk) * CT * C;  // the chunk's first output
  const __amdgpu_buffer_rsrc_t orr = make_rsrc(p.out + ln.b * plane + o0, row_span((plane - o0) * 4, 0));
  const uint32_t row_bytes = static_cast<uint32_t>(C) * 4u;
  // slots past the row (and masked lanes) store out of range; offsets span one chunk
  const uint32_t out0 =
      ln.on ? static_cast<uint32_t>(g * L) * row_bytes + static_cast<uint32_t>(ln.ch) * 4u : kOutOfRange;
  if constexpr (!WIDE) {
    // every scaled term is <= 1 against M
    const float top = fmaxf(fmaxf(kmax, X.m), Y.m);
    const float M = top + span;
    const float sig = fast_exp2(kmax - top);  // 2^{kmax + span - M}: the caps' scale against M
    const float sx = fast_exp2(X.m - M), sy = fast_exp2(Y.m - M);
    const float eU = ln.eU;
    if constexpr (CAUSAL) {
      // Eq. (7) with b = d = 0, straight out of the forward sweep. Only earlier tokens count
      // here, so one lane-wide reference would let a row's first tokens, with keys far below a
      // later one, underflow to 0 / 0. The prefix's numerator and denominator are kept instead
      // against a running reference 2^{r}: they start as (prefix mean, 1) with r the log2 of the
      // prefix weight at the lane's start, and r rises to each larger key as it arrives. The
      // largest term the prefix ever held is 1 and it decays by at most kFastRange binary orders
      // across the lane, so the denominator stays a normal number.
      const bool any = X.m > kEmptyM && X.G > 0.f;
      float r = any ? X.m + fast_log2(X.G) : kEmptyM;
      float A = any ? X.F * fast_rcp(X.G) : 0.f, Cs = any ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const float kf = kv.k(t), vf = kv.v(t);
        const float kl = kf * kLog2e;
        const float nr = fmaxf(r, kl);
        const float sc = fast_exp2(r - nr);
        A *= sc;
        Cs *= sc;
        r = nr;
        const float pi = fast_exp2(kl - r);
        const float pu = pi * eU;
        const float y = fmaf(pu, vf, A) * fast_rcp(pu + Cs);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        A = fmaf(A, lam, pi * vf);
        Cs = fmaf(Cs, lam, pi);
      }
      return true;
    }
    float A = X.F * sx, Cs = X.G * sx;
    const float YF = Y.F * sy, YG = Y.G * sy;
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
      float ph[SB], pv[SB];  // the sub-block's terms and terms times v, kept for the backward sweep
      float s1[SB], s2[SB];  // numerator and denominator so far, per token
      uint32_t r_cur[GATED ? SB : 1];
      if constexpr (GATED) {  // this sub-block's gate inputs; the next one's start loading
#pragma unroll
        for (int i = 0; i < SB; ++i) r_cur[i] = r_next[i];
        if (q + 1 < NSB) gate.load(q + 1, r_next);
      }
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int t = q * SB + i;
        const float kf = kv.k(t), vf = kv.v(t);
        const float pi = fast_exp2(fmaf(kf, kLog2e, -M));
        ph[i] = pi;
        pv[i] = pi * vf;
        // numerator and denominator of Eq. (5) over the earlier tokens and the token itself (the
        // bonus term); the backward sweep adds the later tokens
        s1[i] = fmaf(pv[i], eU, A);
        s2[i] = fmaf(pi, eU, Cs);
        A = fmaf(A, lam, pv[i]);
        Cs = fmaf(Cs, lam, pi);
      }
      // backward state entering this sub-block from the right: the later sub-blocks of the lane
      // plus the later groups
      const float lr = fast_exp2(-static_cast<float>(L - (q + 1) * SB) * D);
      float Bs = fmaf(YF, lr, sig * capF[q]);
      float Ds = fmaf(YG, lr, sig * capG[q]);
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int t = q * SB + i;
        const float num = s1[i] + Bs;
        const float den = s2[i] + Ds;  // >= the lane's largest term, a normal number
        float y;
        if constexpr (GATED) {
          // sigma(r) y = num / (den (1 + e^{-r})): one reciprocal for both divisions
          const float er = fast_exp2(-kLog2e * gate.value(r_cur[i]));
          y = num * fast_rcp(den * (1.f + er));
        } else {
          y = num * fast_rcp(den);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        Bs = fmaf(Bs, lam, pv[i]);
        Ds = fmaf(Ds, lam, ph[i]);
      }
    }
  } else {
    const float U = ln.U;
    Sum xs = X;
    if constexpr (CAUSAL) {
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const float kf = kv.k(t), vf = kv.v(t);
        const bool any = xs.m > kEmptyM && xs.G > 0.f;
        const float kl = kf * kLog2e;
        const float ks = kl + U;
        // log2 of the prefix weight over the token's own (bonus) weight
        const float dp = any ? sum_rel(xs.q, xs.m + fast_log2(xs.G), 0.f, ks, D) : kNegInf;
        const float mp = any ? xs.F * fast_rcp(xs.G) : 0.f;  // prefix mean
        const float sa = fast_exp2(fminf(dp, 0.f)), e = fast_exp2(fminf(-dp, 0.f));
        // the weighted mean itself (not v plus a correction), so the rounding error scales with
        // the magnitudes the mean is formed from, not with |v| of a token of negligible weight
        const float y = fmaf(mp, sa, e * vf) * fast_rcp(sa + e);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        xs = sum_add(sum_shift(xs, 1.f), Sum{0.f, kl, vf, 1.f}, D);
      }
      return true;
    }
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int t = q * SB + i;
        const float kf = kv.k(t), vf = kv.v(t);
        const bool any = xs.m > kEmptyM && xs.G > 0.f;
        lds_al[i][tid] = any ? xs.F * fast_rcp(xs.G) : 0.f;  // prefix mean
        lds_pq[i][tid] = xs.q;
        lds_pm[i][tid] = any ? xs.m + fast_log2(xs.G) : kEmptyM;  // log2 of the prefix weight
        xs = sum_add(sum_shift(xs, 1.f), Sum{0.f, kf * kLog2e, vf, 1.f}, D);
      }
      Sum ys = sum_add(cap[q], sum_shift(Y, static_cast<float>(L - (q + 1) * SB)), D);
      uint32_t r_cur[GATED ? SB : 1];
      if constexpr (GATED) {
        if (q == 0) {
#pragma unroll
          for (int i = 0; i < SB; ++i) r_cur[i] = r_next[i];
        } else {
          gate.load(q, r_cur);
        }
      }
#pragma unroll
      for (int i = SB - 1; i >= 0; --i) {
        const int t = q * SB + i;
        const float kf = kv.k(t), vf = kv.v(t);
        const float al = lds_al[i][tid], pq = lds_pq[i][tid], pm = lds_pm[i][tid];
        const float kl = kf * kLog2e;
        const float ks = kl + U;
        // The prefix, suffix and own (bonus) weights against the largest of them. Each pair is
        // compared through its exact difference of token counts, so two far contributions of
        // nearly equal weight (the two ends of a row with strong growth) keep their ratio.
        float rq = 0.f, rm = ks;  // the largest so far
        if (sum_rel(pq, pm, rq, rm, D) > 0.f) {
          rq = pq;
          rm = pm;
        }
        if (sum_rel(ys.q, ys.m, rq, rm, D) > 0.f) {
          rq = ys.q;
          rm = ys.m;
        }
        const float sa = fast_exp2(sum_rel(pq, pm, rq, rm, D)), sb = fast_exp2(sum_rel(ys.q, ys.m, rq, rm, D));
        const float e = fast_exp2(sum_rel(0.f, ks, rq, rm, D));
        // the weighted mean itself: its rounding error scales with the magnitudes it is formed
        // from (den >= 1: one of the three weights is the largest, 1)
        const float num = fmaf(al, sa, fmaf(ys.F, sb, e * vf));
        const float den = sa + ys.G * sb + e;
        float y;
        if constexpr (GATED) {
          const float er = fast_exp2(-kLog2e * gate.value(r_cur[i]));
          y = num * fast_rcp(den * (1.f + er));
        } else {
          y = num * fast_rcp(den);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        ys = sum_add(sum_shift(ys, 1.f), Sum{0.f, kl, vf, 1.f}, D);
      }
    }
  }
  return true;
}

// ---------------------------------------------------------------------------------------------
// Carries of the two-pass form: for every chunk j of a row and channel, the sum of the forward
// totals of chunks 0 .. j-1 (anchored just before chunk j's first token, token j CT - 1) and of
// the backward totals of chunks j+1 .. n-1 (anchored just after its last slot, token (j+1) CT).
// One wavefront per (row, channel): lane s holds segment s of `per` consecutive chunks (64
// segments), forms the segment's sums, and the lanes scan them with shuffles; each lane then
// writes its chunks' carries. Moving a sum between anchors changes only its token count, and the
// order of the additions is fixed, so the carries are bitwise reproducible.
// ---------------------------------------------------------------------------------------------
constexpr int kCarryChans = 16;  // wavefronts (channels) per workgroup

struct CarryParams {
  const float4* sums;
  float4* carries;
  const float* w;
  long long T;
  int C, n_tiles, n_chunks, CT, causal;
};

// Chunks of a lane's segment held in registers (rows of up to 64 * 8 chunks); beyond that the
// totals are read from memory as they are needed.
constexpr int kCarryRegs = 8;

__device__ __forceinline__ Sum sum_shfl_up(Sum a, int d) {
  return Sum{__shfl_up(a.q, d), __shfl_up(a.m, d), __shfl_up(a.F, d), __shfl_up(a.G, d)};
}
__device__ __forceinline__ Sum sum_shfl_down(Sum a, int d) {
  return Sum{__shfl_down(a.q, d), __shfl_down(a.m, d), __shfl_down(a.F, d), __shfl_down(a.G, d)};
}

template <int TILE>
__global__ void __launch_bounds__(64 * kCarryChans) row_carry_kernel(CarryParams p) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int SLICES = TILE / kCarryChans;
  const int row = blockIdx.x / SLICES, slice = blockIdx.x - row * SLICES;
  const int tc = slice * kCarryChans + wv;
  const int ch = (row % p.n_tiles) * TILE + tc;
  const int n = p.n_chunks;
  const int per = (n + 63) / 64;
  const int c0 = lane * per < n ? lane * per : n, c1 = c0 + per < n ? c0 + per : n;
  const float seg = static_cast<float>(per) * static_cast<float>(p.CT);  // tokens per segment
  const float ct = static_cast<float>(p.CT);
  const size_t base = static_cast<size_t>(row) * n * 2 * TILE + tc;
  auto at = [&](int j, int dir) { return base + static_cast<size_t>(j * 2 + dir) * TILE; };
  const float4* __restrict__ sums = p.sums;
  float4* __restrict__ carries = p.carries;
  // every load of the lane is issued before any result is used (one round trip)
  const bool inreg = per <= kCarryRegs;
  float4 tf[kCarryRegs], tb[kCarryRegs];
  if (inreg) {
#pragma unroll
    for (int i = 0; i < kCarryRegs; ++i) {
      if (c0 + i < c1) {
        tf[i] = sums[at(c0 + i, kFwd)];
        tb[i] = p.causal ? make_float4(0.f, kNegInf, 0.f, 0.f) : sums[at(c0 + i, kBwd)];
      }
    }
  }
  const float D = ch < p.C ? (p.w[ch] / static_cast<float>(p.T)) * kLog2e : 0.f;
  // segment sums: forward anchored at the segment's last slot, (lane + 1) per CT - 1, and
  // backward at its first token, lane per CT (a short or empty last segment keeps those anchors)
  Sum f = sum_empty(), b = sum_empty();
  const int cf = lane * per + per - 1;  // chunk whose last slot is the forward anchor
  if (inreg) {
#pragma unroll
    for (int i = 0; i < kCarryRegs; ++i) {
      const int j = c0 + i;
      if (j < c1) {
        f = sum_add(f, sum_shift(slot_unpack(tf[i]), static_cast<float>(cf - j) * ct), D);
        b = sum_add(b, sum_shift(slot_unpack(tb[i]), static_cast<float>(i) * ct), D);
      }
    }
  } else {
    for (int j = c0; j < c1; ++j) {
      f = sum_add(f, sum_shift(slot_unpack(sums[at(j, kFwd)]), static_cast<float>(cf - j) * ct), D);
      if (!p.causal) b = sum_add(b, sum_shift(slot_unpack(sums[at(j, kBwd)]), static_cast<float>(j - c0) * ct), D);
    }
  }
  // inclusive scans over the segments: forward over lanes 0 .. lane, backward over lane .. 63
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const Sum pf = sum_shfl_up(f, d);
    if (lane >= d) f = sum_add(sum_shift(pf, static_cast<float>(d) * seg), f, D);
    const Sum pb = sum_shfl_down(b, d);
    if (lane + d < 64) b = sum_add(b, sum_shift(pb, static_cast<float>(d) * seg), D);
  }
  // entering sums: the earlier segments' forward sum, anchored at c0 CT - 1, and the later
  // segments' backward sum, anchored at (lane + 1) per CT
  Sum X = sum_shfl_up(f, 1), Y = sum_shfl_down(b, 1);
  if (lane == 0) X = sum_empty();
  if (p.causal || lane == 63) Y = sum_empty();
  const int ce = lane * per + per;  // first chunk after the segment (the backward anchor's chunk)
  // each chunk's carries: the entering sum plus the segment's chunks on the near side, moved to
  // the chunk's own anchor
  if (inreg) {
    Sum x = X;
#pragma unroll
    for (int i = 0; i < kCarryRegs; ++i) {
      if (c0 + i < c1) {
        carries[at(c0 + i, kFwd)] = slot_pack(sum_shift(x, static_cast<float>(i) * ct));
        x = sum_add(x, sum_shift(slot_unpack(tf[i]), -static_cast<float>(i + 1) * ct), D);
      }
    }
    if (!p.causal) {
      Sum y = Y;
#pragma unroll
      for (int i = kCarryRegs - 1; i >= 0; --i) {
        const int j = c0 + i;
        if (j < c1) {
          carries[at(j, kBwd)] = slot_pack(sum_shift(y, static_cast<float>(ce - 1 - j) * ct));
          y = sum_add(y, sum_shift(slot_unpack(tb[i]), -static_cast<float>(ce - j) * ct), D);
        }
      }
    }
  } else {
    for (int j = c0; j < c1; ++j) {
      carries[at(j, kFwd)] = slot_pack(sum_shift(X, static_cast<float>(j - c0) * ct));
      X = sum_add(X, sum_shift(slot_unpack(sums[at(j, kFwd)]), -static_cast<float>(j + 1 - c0) * ct), D);
    }
    if (!p.causal) {
      for (int j = c1 - 1; j >= c0; --j) {
        carries[at(j, kBwd)] = slot_pack(sum_shift(Y, static_cast<float>(ce - 1 - j) * ct));
        Y = sum_add(Y, sum_shift(slot_unpack(sums[at(j, kBwd)]), -static_cast<float>(ce - j) * ct), D);
      }
    }
  }
}

// The epoch counter of a single pass, read through the scalar cache (the load waits in its own
// asm block, on the scalar counter only, so vector loads issued before it stay in flight). The
// cache holds no stale copy: caches are invalidated when a launch starts, and no workgroup moves
// the counter before every workgroup of the launch has read it.
template <int MODE>
__device__ __forceinline__ unsigned row_epoch(const RowParams& p) {
  unsigned e = 0u;
  if (MODE == kSinglePass && p.n_chunks > 1) {
    const unsigned long long ep = uniform_u64(reinterpret_cast<unsigned long long>(&p.ctr->epoch));
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(e) : "s"(ep) : "memory");
  }
  return e;
}

// The wide form is rare (extreme w or u) and needs more registers than the fast form: keeping it
// out of line gives it its own register allocation, so its spills never touch the fast form. It
// reads the parameters from the kernel's argument segment (a pointer, so the kernel keeps them in
// scalar registers instead of building a private copy). It also takes over a fast-form chunk of a
// single pass whose wait ran out (`published`: that chunk's slot is already out).
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED, int MODE, int POL>
__device__ __noinline__ void row_body_wide(const RowParams* args, float* lds, unsigned unit, bool published) {
  const RowParams p = *args;
  const unsigned ep = row_epoch<MODE>(p);
  const RowLane ln = row_lane<TILE, L, NT>(p, unit);
  RowStore<DT, TILE, L, PAIR> kv;
  row_load<DT, TILE, L, NT, FUSED, PAIR, POL>(p, ln, kv);
  unsigned fin = kNotRetiring;
  row_body<DT, TILE, L, NT, FUSED, PAIR, true, CAUSAL, GATED, MODE>(p, args, ln, kv, lds, ep, published, fin);
  row_retire_end(p, fin);
}

// Cache policy of a launch's k, v loads: the sums pass of two keeps the default policy, so the
// output pass finds the chunks it reads again in the memory-side cache; every other launch
// touches them once.
template <int MODE>
constexpr int kRowLoadPolicy = MODE == kSumsPass ? 0 : kStream;

template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED, int MODE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4)))
    biwkv_row_kernel(RowParams p) {
  static_assert(!PAIR || (DT == BIWKV_BF16 && TILE % 2 == 0), "pairs are bf16 channel pairs");
  static_assert(!(GATED && (CAUSAL || FUSED)), "the gate is built for the bidirectional entry");
  static_assert(!(GATED && MODE == kSumsPass), "the sums pass has no outputs to gate");
  static_assert(64 % TILE == 0 || TILE % 64 == 0, "bad row-kernel tile");
  static_assert(TILE <= 64, "a wavefront must hold every channel of the tile");
  static_assert(NT % 256 == 0 && NT <= 1024 && NT >= 2 * TILE, "bad row-kernel workgroup size");
  constexpr int POL = kRowLoadPolicy<MODE>;
  __shared__ float lds[kRowLdsFloats<TILE, NT>];
  const unsigned unit = blockIdx.x;
  // the kernel's only argument is p, at the start of the argument segment (the argument segment
  // pointer exists only here, in the kernel: out-of-line functions get it passed down)
  const auto* args = (const RowParams*)(__builtin_amdgcn_kernarg_segment_ptr());
  RowLane ln = row_lane_index<TILE, L, NT>(p, unit);
  RowStore<DT, TILE, L, PAIR> kv;
  unsigned ep = 0;
  // Single passes over 32-bit words issue every vector load before anything waits: w and u
  // (range-checked: a masked lane reads 0), then the chunk's k and v in the fast form's layout;
  // the form is chosen once w and u have arrived, and the wide form loads the chunk again itself.
  // Elsewhere (16-bit loads, two passes) the early loads cost the fast form registers: the form is
  // chosen first.
  constexpr bool kEarly = MODE == kSinglePass && (PAIR || DT == BIWKV_F32);
  if constexpr (kEarly) {
    const uint32_t coff = ln.on ? static_cast<uint32_t>(ln.ch) * 4u : kOutOfRange;
    const uint32_t cbytes = static_cast<uint32_t>(p.C) * 4u;
    const uint32_t wbits = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.w, cbytes), coff, 0, 0);
    const uint32_t ubits = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.u, cbytes), coff, 0, 0);
    row_load<DT, TILE, L, NT, FUSED, PAIR, POL>(p, ln, kv);
    ep = row_epoch<MODE>(p);
    row_lane_params(ln, p.T, __uint_as_float(wbits), __uint_as_float(ubits));
  } else {
    ep = row_epoch<MODE>(p);
    row_lane_params(ln, p.T, ln.on ? p.w[ln.ch] : 0.f, ln.on ? p.u[ln.ch] : 0.f);
  }
  // The whole workgroup takes the wide form when any of its channels needs it: decay or growth
  // across one lane beyond kFastRange, a bonus beyond kBonusRange, or decay across the row beyond
  // kExactRange (the sums' exponents then need exact token counts). Every wavefront holds all TILE
  // channels, so a wavefront vote is the workgroup's vote, and every chunk of a row votes alike.
  const bool wide_lane = fabsf(ln.D) * static_cast<float>(L - 1) > kFastRange || ln.U > kBonusRange ||
                         ln.U < -kBonusRange || fabsf(ln.D) * static_cast<float>(p.T) > kExactRange;
  const bool fast = __ballot(wide_lane) == 0ull;
  if constexpr (kEarly) {
    // one call site of the wide form: from the start, or for a fast chunk whose wait ran out (its
    // slot already published)
    unsigned fin = kNotRetiring;
    if (fast && row_body<DT, TILE, L, NT, FUSED, PAIR, false, CAUSAL, GATED, MODE>(p, args, ln, kv, lds, ep, false, fin)) {
      row_retire_end(p, fin);
      return;
    }
    row_body_wide<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED, MODE, POL>(args, lds, unit, fast);
  } else {
    if (!fast) {
      row_body_wide<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED, MODE, POL>(args, lds, unit, false);
    } else {
      row_load<DT, TILE, L, NT, FUSED, PAIR, POL>(p, ln, kv);
      unsigned fin = kNotRetiring;
      if (!row_body<DT, TILE, L, NT, FUSED, PAIR, false, CAUSAL, GATED, MODE>(p, args, ln, kv, lds, ep, false, fin))
        row_body_wide<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED, MODE, POL>(args, lds, unit, true);
      row_retire_end(p, fin);
    }
  }
}

}  // namespace
