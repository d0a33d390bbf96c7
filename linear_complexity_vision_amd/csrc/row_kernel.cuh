// Bi-WKV tile kernel: a (batch, channel tile) row held by one workgroup, or by a few workgroups
// (chunks of the row) that exchange their sums.
#pragma once

#include <type_traits>

#include "common.cuh"

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
// are consecutive lanes of one wavefront. When a row has several chunks, each workgroup
// publishes its chunk's forward and backward sums (epoch-tagged slots, see slot_store) and folds
// the sums of the other chunks of its row, in a fixed order, into its carries. When the whole
// grid fits on the device the chunks follow the grid order; otherwise workgroups take tickets in
// launch order and the chunks of a row hold consecutive tickets, so a workgroup only waits for
// workgroups that have started or will start once earlier rows finish. Each lane then sweeps its
// tokens in sub-blocks of 8: forward states (a, c) left to right, keeping (alpha, beta) = (a - c
// v, c + e^{u+k}) per token in LDS, then backward states (b, d) right to left, writing Eq. (7).
//
// Every lane holds exactly L token slots. Slots past the end of the row hold k = -inf, i.e. a
// weight of exactly 0, so the sweeps need no per-token bounds: a lane's forward sum is anchored
// at its last slot, and such slots are only ever followed by more empty slots. Loads and stores
// go through range-checked buffer resources over one batch item, so slots past the row read 0
// and their stores are dropped by the hardware.

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
  int ordered;                   // 1: workgroups take tickets (more than fit on the device)
  Counters* ctr;                 // ticket / epoch block (n_chunks > 1)
  unsigned long long* slots;     // [row][chunk][dir][TILE] (l, mu) slot pairs (n_chunks > 1)
  int H, W, shift, g1, g2, g3, g4;  // Q-Shift (fused entry only)
  int bidir;  // fused: the bidirectional shift along a sparse token sequence (the host sets W = 1)
};

// Counts a workgroup out of a chunked launch once none of its wavefronts reads the epoch or a slot
// again; the last one resets the counters for the next launch on the stream. Nothing else waits
// for it, so only the calling wavefront sees the round trip.
__device__ __forceinline__ void row_retire(const RowParams& p) {
  const unsigned fin = __hip_atomic_fetch_add(&p.ctr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (fin + 1u == p.total) {
    __hip_atomic_store(&p.ctr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
__device__ __forceinline__ RowLane row_lane(const RowParams& p, unsigned unit) {
  constexpr int CT = (NT / TILE) * L;  // tokens per chunk
  RowLane ln;
  const int tid = threadIdx.x;
  ln.c = tid % TILE;
  ln.g = tid / TILE;
  // integer division runs on the vector unit: read the (uniform) results back into scalars
  ln.row = __builtin_amdgcn_readfirstlane(unit / static_cast<unsigned>(p.n_chunks));
  ln.chunk = static_cast<int>(unit) - ln.row * p.n_chunks;
  const int bi = __builtin_amdgcn_readfirstlane(ln.row / p.n_tiles);
  const int tile = ln.row - bi * p.n_tiles;
  ln.b = bi;
  ln.ch = tile * TILE + ln.c;
  ln.on = ln.ch < p.C;
  ln.s_g = static_cast<long long>(ln.chunk) * CT + static_cast<long long>(ln.g) * L;
  const long long rem = p.T - ln.s_g;
  ln.n_g = rem <= 0 ? 0 : (rem < L ? static_cast<int>(rem) : L);
  const float wc = ln.on ? p.w[ln.ch] : 0.f;
  const float uc = ln.on ? p.u[ln.ch] : 0.f;
  ln.D = (wc / static_cast<float>(p.T)) * kLog2e;
  ln.lam = fast_exp2(-ln.D);
  ln.U = uc * kLog2e;
  ln.grow = fmaxf(-ln.D, 0.f);
  ln.eU = fast_exp2(ln.U);
  return ln;
}

// Loads word m of the lane's k and v (one token, or a channel pair at one token) at byte offset off
// of the resources km and vm.
template <int DT, bool PAIR, class Store>
__device__ __forceinline__ void row_load_word(Store& kv, int m, __amdgpu_buffer_rsrc_t km,
                                              __amdgpu_buffer_rsrc_t vm, uint32_t off) {
  if constexpr (PAIR) {
    kv.kk[m] = __builtin_amdgcn_raw_buffer_load_b32(km, off, 0, kStream);
    kv.vv[m] = __builtin_amdgcn_raw_buffer_load_b32(vm, off, 0, kStream);
  } else if constexpr (DT == BIWKV_F32) {
    kv.kk[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(km, off, 0, kStream));
    kv.vv[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vm, off, 0, kStream));
  } else {
    const uint32_t kx = __builtin_amdgcn_raw_buffer_load_b16(km, off, 0, kStream);
    const uint32_t vx = __builtin_amdgcn_raw_buffer_load_b16(vm, off, 0, kStream);
    kv.r[m] = kx | (vx << 16);
  }
}

// Issues every load of the lane's k and v (Q-Shift applied when FUSED: padded sources read 0) and
// marks the slots past the row empty. Nothing waits here: phase A consumes the words in load
// order as they arrive.
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, class Store>
__device__ __forceinline__ void row_load(const RowParams& p, const RowLane& ln, Store& kv) {
  const long long T = p.T;
  const int C = p.C;
  const long long plane = T * C;  // elements of one batch item
  constexpr int ES = DT == BIWKV_F32 ? 4 : 2;
  const char* kb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.k) + ln.b * plane * ES));
  const char* vb = reinterpret_cast<const char*>(
      uniform_u64(reinterpret_cast<unsigned long long>(p.v) + ln.b * plane * ES));
  const uint32_t row_bytes = static_cast<uint32_t>(C) * ES;
  // PAIR: lane 2j + odd reads channels (2j, 2j + 1) at tokens 2m + odd
  constexpr int STEP = PAIR ? 2 : 1;
  constexpr int NW = L / STEP;  // words per lane and array
  const int odd = PAIR ? (ln.c & 1) : 0;
  const uint32_t lane_byte = static_cast<uint32_t>(ln.ch - odd) * ES;
  constexpr int CT = (NT / TILE) * L;
  if constexpr (!FUSED) {
    // The token offset of word m is uniform, so it moves the resource base (scalar work) and the
    // lane keeps one vector offset. Tokens past the row fall past the shortened resource and
    // read 0, and so does every slot of a masked lane.
    // byte counts below 2^31 (the host checks (T + CT) * C * 4), so 32-bit scalar arithmetic
    const int c0 = ln.chunk * CT * static_cast<int>(row_bytes);  // chunk start
    const int avail = static_cast<int>(plane * ES) - c0;       // bytes from there to the end
    const uint32_t lane_off =
        ln.on ? static_cast<uint32_t>(ln.g * L + odd) * row_bytes + lane_byte : kOutOfRange;
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const int adv = m * STEP * static_cast<int>(row_bytes);
      const int left = avail - adv;
      const uint32_t n = static_cast<uint32_t>(left > 0 ? left : 0);
      const __amdgpu_buffer_rsrc_t km = make_rsrc(kb + c0 + adv, n);
      const __amdgpu_buffer_rsrc_t vm = make_rsrc(vb + c0 + adv, n);
      row_load_word<DT, PAIR>(kv, m, km, vm, lane_off);
    }
  } else {
    // Q-Shift: the lane reads its own channel at token t + delta, where delta is fixed by the
    // channel's quarter (right: -s, left: +s, down: -s W, up: +s W, rest: 0). Word m's resource
    // starts SH = s W tokens before the word's token, so every lane offset is non-negative and
    // constant; sources past the end of the batch item fall past the resource and read 0. The
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
    const int t0 = ln.chunk * CT + ln.g * L + odd;  // token of word 0 (T < 2^31 / (4 C))
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
    const uint32_t lane_off = static_cast<uint32_t>(ln.g * L + odd + delta + SH) * row_bytes + lane_byte;
    // byte counts below 2^31 (the host checks (T + CT + 2 s W) * C * 4), so 32-bit arithmetic
    const int c0 = (ln.chunk * CT - SH) * static_cast<int>(row_bytes);  // may be negative
    const int avail = static_cast<int>(plane * ES) - c0;
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const int adv = m * STEP * static_cast<int>(row_bytes);
      const int left = avail - adv;
      const uint32_t n = static_cast<uint32_t>(left > 0 ? left : 0);
      const __amdgpu_buffer_rsrc_t km = make_rsrc(kb + c0 + adv, n);
      const __amdgpu_buffer_rsrc_t vm = make_rsrc(vb + c0 + adv, n);
      // all ones when word m is valid (bit m of the mask, sign-extended)
      const uint32_t keep =
          static_cast<uint32_t>(static_cast<std::make_signed_t<Mask>>(valid << (MB - 1 - m)) >> (MB - 1));
      const uint32_t off = (lane_off & keep) | (kOutOfRange & ~keep);
      row_load_word<DT, PAIR>(kv, m, km, vm, off);
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
constexpr int kRowSweepFloats = 8 * NT * 2;
// Row pitch of the group-major lane-sum and carry buffers. Lane (tg, tc) of the transposed layout
// reads word tg * pitch + tc with tg = lane % GROUPS: a pitch of TILE + 64 / GROUPS puts the 64
// lanes of a wavefront on 64 different banks (a pitch of TILE + 1 put up to 8 on one).
template <int TILE, int NT>
constexpr int kRowPad = TILE + (NT / TILE < 64 ? 64 / (NT / TILE) : 1);
template <int TILE, int NT>
constexpr int kRowLdsFloats = kRowSweepFloats<NT> + 6 * (NT / TILE) * kRowPad<TILE, NT> + TILE;

// The scans and the exchange use a finite exponent for an empty aggregate (F = G = 0), far below
// any real one: 2^(empty - m) is then exactly 0 against a real exponent and 1 against another
// empty one, so adding aggregates needs no branch.
constexpr float kEmptyM = -1e30f;
__device__ __forceinline__ Agg row_empty() { return Agg{kEmptyM, 0.f, 0.f}; }
__device__ __forceinline__ Agg agg_add_f(Agg a, Agg b) {
  const float m = fmaxf(a.m, b.m);
  const float sa = fast_exp2(a.m - m), sb = fast_exp2(b.m - m);
  return Agg{m, fmaf(a.F, sa, b.F * sb), fmaf(a.G, sa, b.G * sb)};
}

// Aggregates moved between the W consecutive lanes that hold one channel's groups (W is a power
// of two up to 64). from_below<W, d> gives a lane the value of the lane d below it and
// from_above<W, d> that of the lane d above; the callers only use results from inside the
// segment. Segments of up to 16 lanes lie inside one DPP row, so these are row shifts (plain
// VALU moves); wider segments go through the LDS crossbar (ds_bpermute).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int W, int d>
__device__ __forceinline__ Agg agg_from_below(Agg a) {
  if constexpr (W <= 16)
    return Agg{dpp_move<0x110 + d>(a.m), dpp_move<0x110 + d>(a.F), dpp_move<0x110 + d>(a.G)};  // row_shr
  else
    return Agg{__shfl_up(a.m, d, W), __shfl_up(a.F, d, W), __shfl_up(a.G, d, W)};
}
template <int W, int d>
__device__ __forceinline__ Agg agg_from_above(Agg a) {
  if constexpr (W <= 16)
    return Agg{dpp_move<0x100 + d>(a.m), dpp_move<0x100 + d>(a.F), dpp_move<0x100 + d>(a.G)};  // row_shl
  else
    return Agg{__shfl_down(a.m, d, W), __shfl_down(a.F, d, W), __shfl_down(a.G, d, W)};
}
template <int W>
__device__ __forceinline__ Agg agg_from_first(Agg a) {
  return Agg{__shfl(a.m, 0, W), __shfl(a.F, 0, W), __shfl(a.G, 0, W)};
}

// Inclusive scans over the W groups of a channel (lane tg holds group tg; groups are L slots
// apart): forward over groups 0..tg, anchored at tg's last slot, and (BWD) backward over
// tg..W-1, anchored at tg's first token. Hillis-Steele, fixed order.
template <int W, int L, bool BWD, int d = 1>
__device__ __forceinline__ void group_scan(Agg& f, Agg& bk, int tg, float D) {
  if constexpr (d < W) {
    const Agg pf = agg_from_below<W, d>(f);
    if (tg >= d) f = agg_add_f(agg_shift(pf, static_cast<float>(d * L), D), f);
    if constexpr (BWD) {
      const Agg pb = agg_from_above<W, d>(bk);
      if (tg + d < W) bk = agg_add_f(bk, agg_shift(pb, static_cast<float>(d * L), D));
    }
    group_scan<W, L, BWD, 2 * d>(f, bk, tg, D);
  }
}

// Folds the W lanes' sums (a, and b when BWD) into the segment's first lane in a fixed tree.
template <int W, bool BWD, int s = 1>
__device__ __forceinline__ void group_fold(Agg& a, Agg& b, int tg) {
  if constexpr (s < W) {
    const Agg oa = agg_from_above<W, s>(a);
    if ((tg & (2 * s - 1)) == 0) a = agg_add_f(a, oa);
    if constexpr (BWD) {
      const Agg ob = agg_from_above<W, s>(b);
      if ((tg & (2 * s - 1)) == 0) b = agg_add_f(b, ob);
    }
    group_fold<W, BWD, 2 * s>(a, b, tg);
  }
}

// Gate inputs r of Eq. (2) for the SB tokens of a lane's sub-block q (raw bits: an fp32 value, or
// a bf16 value in the low half), through per-token resources like the unfused k, v loads.
template <int DT, int TILE, int L, int NT, int SB>
struct RowGate {
  const char* base;   // the batch item's r
  int c0, avail;      // chunk start (bytes) and bytes from there to the item's end
  uint32_t lane_off;  // this lane's offset from the chunk start (out of range when masked)
  int row_bytes;
  __device__ __forceinline__ void init(const RowParams& p, const RowLane& ln) {
    constexpr int ES = DT == BIWKV_F32 ? 4 : 2;
    constexpr int CT = (NT / TILE) * L;
    const long long plane = p.T * p.C;
    base = reinterpret_cast<const char*>(
        uniform_u64(reinterpret_cast<unsigned long long>(p.r) + ln.b * plane * ES));
    row_bytes = p.C * ES;
    c0 = ln.chunk * CT * row_bytes;
    avail = static_cast<int>(plane * ES) - c0;
    lane_off = ln.on ? static_cast<uint32_t>(ln.g * L) * row_bytes + static_cast<uint32_t>(ln.ch) * ES
                     : kOutOfRange;
  }
  __device__ __forceinline__ void load(int q, uint32_t (&dst)[SB]) const {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int adv = (q * SB + i) * row_bytes;
      const int left = avail - adv;
      const __amdgpu_buffer_rsrc_t rr =
          make_rsrc(base + c0 + adv, static_cast<uint32_t>(left > 0 ? left : 0));
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
// are formed, scanned and exchanged, and the output comes out of the forward sweep.
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool WIDE, bool CAUSAL, bool GATED>
__device__ __forceinline__ void row_body(const RowParams& p, const RowLane& ln,
                                         RowStore<DT, TILE, L, PAIR>& kv, float* lds,
                                         const unsigned* sh_epoch) {
  constexpr int GROUPS = NT / TILE;
  constexpr int CT = GROUPS * L;  // tokens per chunk
  constexpr int SB = 8;  // tokens per sub-block of the sweeps
  constexpr int NSB = L / SB;
  static_assert(L % SB == 0, "bad row-kernel shape");
  static_assert((GROUPS & (GROUPS - 1)) == 0 && GROUPS <= 64, "a channel's groups share a wavefront");
  float2 (*lds_ab)[NT] = reinterpret_cast<float2 (*)[NT]>(lds);
  const int tid = threadIdx.x;
  const int g = ln.g;
  const long long T = p.T;
  const int C = p.C;
  const float D = ln.D, lam = ln.lam, grow = ln.grow;
  const float span = grow * static_cast<float>(L - 1);  // largest growth inside one lane

  // ---- phase A: lane sums (forward anchored at its last slot, backward at its first) and, per
  //      sub-block, the backward sum of everything after it inside the lane ----
  Agg af, ab;
  float kmax = kNegInf;
  float capF[WIDE ? 1 : NSB], capG[WIDE ? 1 : NSB];  // fast form: anchored at (q + 1) * SB
  Agg cap[WIDE ? NSB : 1];                           // wide form
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
    ab = CAUSAL ? row_empty() : Agg{m_agg, cF, cG};
  } else {
#pragma unroll
    for (int q = 0; q < NSB; ++q) kv.prepare(q);
    // Wide range: one decay step at a time, each sum against its own running maximum (an empty
    // slot, k = -inf, adds nothing).
    af = agg_empty();
#pragma unroll
    for (int i = 0; i < L; ++i)
      af = agg_add(agg_shift(af, 1.f, D), Agg{kv.k(i) * kLog2e, kv.v(i), 1.f});
    ab = agg_empty();
    if constexpr (!CAUSAL) {
      Agg bs[NSB];
#pragma unroll
      for (int q = 0; q < NSB; ++q) {
        bs[q] = agg_empty();
#pragma unroll
        for (int i = (q + 1) * SB - 1; i >= q * SB; --i)
          bs[q] = agg_add(agg_shift(bs[q], 1.f, D), Agg{kv.k(i) * kLog2e, kv.v(i), 1.f});
      }
#pragma unroll
      for (int q = NSB - 1; q >= 0; --q) {
        cap[q] = ab;
        ab = agg_add(bs[q], agg_shift(ab, static_cast<float>(SB), D));
      }
    }
  }
  kv.fence();
  // GATED: the gate inputs of sub-block 0 load during the scan and the exchange
  RowGate<DT, TILE, L, NT, SB> gate;
  uint32_t r_next[GATED ? SB : 1];
  if constexpr (GATED) {
    gate.init(p, ln);
    gate.load(0, r_next);
  }

  // ---- scans over the groups of each channel. The lane sums go to LDS group-major; lane
  //      (tg, tc) = (tid % GROUPS, tid / GROUPS) then takes group tg of channel tc, so the groups
  //      of a channel are GROUPS consecutive lanes of one wavefront and the scans (and the
  //      exchange) run on lane shuffles without barriers. Carries go back the same way. ----
  constexpr int PAD = kRowPad<TILE, NT>;  // row pitch of the group-major buffers
  constexpr int RS = GROUPS * PAD;      // floats per quantity
  float* red = lds;                     // [6][RS] lane sums (inside the sweep buffer)
  float* xy = lds + kRowSweepFloats<NT>;  // [6][RS] carries (outside it: read during the sweeps)
  float* dch = xy + 6 * RS;             // [TILE] D of each channel
  const int wi = g * PAD + ln.c;
  if constexpr (WIDE) {  // the wide sums mark an empty aggregate with -inf
    af.m = fmaxf(af.m, kEmptyM);
    ab.m = fmaxf(ab.m, kEmptyM);
  }
  red[0 * RS + wi] = af.m;
  red[1 * RS + wi] = af.F;
  red[2 * RS + wi] = af.G;
  red[3 * RS + wi] = ab.m;
  red[4 * RS + wi] = ab.F;
  red[5 * RS + wi] = ab.G;
  if (g == 0) dch[ln.c] = D;
  __syncthreads();
  const int tg = tid % GROUPS, tc = tid / GROUPS;
  const int ti = tg * PAD + tc;
  const float Dt = dch[tc];
  Agg f{red[0 * RS + ti], red[1 * RS + ti], red[2 * RS + ti]};
  Agg bk{red[3 * RS + ti], red[4 * RS + ti], red[5 * RS + ti]};
  group_scan<GROUPS, L, !CAUSAL>(f, bk, tg, Dt);
  // exclusive carries: forward sum of the earlier groups (anchored just before the group's first
  // token), backward sum of the later groups (anchored just after its last slot)
  Agg X = agg_from_below<GROUPS, 1>(f), Y = agg_from_above<GROUPS, 1>(bk);
  if (tg == 0) X = row_empty();
  if (CAUSAL || tg == GROUPS - 1) Y = row_empty();
  if (p.n_chunks > 1) {
    // ---- exchange with the other chunks of the row ----
    const int nch = p.n_chunks, chunk = ln.chunk;
    const unsigned epoch = __builtin_amdgcn_readfirstlane(*sh_epoch);  // set before the barrier
    unsigned long long* rs = p.slots + static_cast<size_t>(ln.row) * nch * 2 * TILE * 2;
    auto slot = [&](int ck, int dir) { return rs + (static_cast<size_t>(ck * 2 + dir) * TILE + tc) * 2; };
    // the chunk's own sums: forward (inclusive at the last group, anchored at the chunk's last
    // slot) and backward (inclusive at group 0, anchored at the chunk's first token)
    if (tg == GROUPS - 1) slot_store(slot(chunk, kFwd), f, epoch);
    if (!CAUSAL && tg == 0) slot_store(slot(chunk, kBwd), bk, epoch);
    // Entries: forward sums of chunks 0 .. chunk-1, then backward sums of chunks chunk+1 ..
    // nch-1. Lane tg folds entries tg, tg + GROUPS, ... in order; the lanes' partials are then
    // folded in a fixed tree, so the result does not depend on arrival order.
    const int nf = chunk, ne = CAUSAL ? chunk : nch - 1;
    Agg pf = row_empty(), pb = row_empty();
    bool timed_out = false;
    // A lane issues the loads of up to EB entries before it waits for any of them, so a lane
    // with several entries pays one round trip, not one per entry.
    constexpr int EB = GROUPS >= 8 ? 1 : 8 / GROUPS;
    for (int e0 = tg; e0 < ne; e0 += EB * GROUPS) {
      unsigned long long wv[EB][2];
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        const int e = e0 + j * GROUPS;
        if (e < ne) slot_load(slot(e < nf ? e : e + 1, e < nf ? kFwd : kBwd), wv[j]);
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
        const unsigned long long* sp = slot(ck, fwd ? kFwd : kBwd);
        if (GATED) {
          // one poll at a time: the gated kernel holds its first gate inputs in flight here,
          // and a second poll's registers cost it spills and waits
          for (unsigned spins = 0; !slot_ready(wv[j], epoch); ++spins) {
            if (spins > kSpinLimit) {
              timed_out = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            slot_load(sp, wv[j]);
          }
        } else if (!slot_ready(wv[j], epoch)) {
          // Two polls in flight, issued a short sleep apart: a slot published just after one
          // poll was served is seen by the next one instead of a full round trip later.
          unsigned long long w2[2];
          slot_load(sp, w2);
          for (unsigned spins = 0;; spins += 2) {
            __builtin_amdgcn_s_sleep(2);
            slot_load(sp, wv[j]);
            if (slot_ready(w2, epoch)) {  // the older poll
              wv[j][0] = w2[0];
              wv[j][1] = w2[1];
              break;
            }
            if (spins > kSpinLimit) {
              timed_out = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            slot_load(sp, w2);
            if (slot_ready(wv[j], epoch)) break;
          }
        }
        Agg a = slot_value(wv[j]);
        a.m = fmaxf(a.m, kEmptyM);
        a = agg_shift(a, dist, Dt);
        if (fwd)
          pf = agg_add_f(pf, a);
        else
          pb = agg_add_f(pb, a);
      }
    }
    if (timed_out)
      __hip_atomic_fetch_or(&p.ctr->fault, kFaultSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    group_fold<GROUPS, !CAUSAL>(pf, pb, tg);
    // pf (from the first lane of the channel) is anchored just before the chunk, pb just after it
    pf = agg_from_first<GROUPS>(pf);
    X = agg_add_f(agg_shift(pf, static_cast<float>(tg * L), Dt), X);
    if constexpr (!CAUSAL) {
      pb = agg_from_first<GROUPS>(pb);
      Y = agg_add_f(Y, agg_shift(pb, static_cast<float>((GROUPS - 1 - tg) * L), Dt));
    }
  }
  xy[0 * RS + ti] = X.m;
  xy[1 * RS + ti] = X.F;
  xy[2 * RS + ti] = X.G;
  xy[3 * RS + ti] = Y.m;
  xy[4 * RS + ti] = Y.F;
  xy[5 * RS + ti] = Y.G;
  __syncthreads();  // past it, the sum buffer becomes the (alpha, beta) buffer
  X = Agg{xy[0 * RS + wi], xy[1 * RS + wi], xy[2 * RS + wi]};
  Y = Agg{xy[3 * RS + wi], xy[4 * RS + wi], xy[5 * RS + wi]};
  // every wavefront is past its last read of the epoch and of the slots
  if (p.n_chunks > 1 && tid == 0) row_retire(p);
  kv.fence();

  // ---- phase C: sweep each sub-block forward, then backward, writing Eq. (7) ----
  if (ln.n_g <= 0) return;  // no barrier follows
  const long long plane = T * C;
  const __amdgpu_buffer_rsrc_t orr =
      make_rsrc(p.out + ln.b * plane, static_cast<uint32_t>(plane * 4));
  const uint32_t row_bytes = static_cast<uint32_t>(C) * 4u;
  // slots past the row (and masked lanes) store out of range
  const uint32_t out0 =
      ln.on ? static_cast<uint32_t>(ln.s_g) * row_bytes + static_cast<uint32_t>(ln.ch) * 4u
            : kOutOfRange;
  if constexpr (!WIDE) {
    // every scaled term is <= 1 against M
    const float top = fmaxf(fmaxf(kmax, X.m), Y.m);
    const float M = top + span;
    const float sig = fast_exp2(kmax - top);  // 2^{kmax + span - M}: the caps' scale against M
    const float sx = fast_exp2(X.m - M), sy = fast_exp2(Y.m - M);
    const float eU = ln.eU;
    float A = X.F * sx, Cs = X.G * sx;
    const float YF = Y.F * sy, YG = Y.G * sy;
    if constexpr (CAUSAL) {  // Eq. (7) with b = d = 0, straight out of the forward sweep
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const float kf = kv.k(t), vf = kv.v(t);
        const float pi = fast_exp2(fmaf(kf, kLog2e, -M));
        const float al = fmaf(-Cs, vf, A);
        const float be = fmaf(pi, eU, Cs);  // >= the token's own term, a normal number
        const float y = fmaf(al, fast_rcp(be), vf);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        A = fmaf(A, lam, pi * vf);
        Cs = fmaf(Cs, lam, pi);
      }
      return;
    }
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
    Agg xs = X;
    if constexpr (CAUSAL) {
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const float kf = kv.k(t), vf = kv.v(t);
        const bool any = xs.m != kNegInf && xs.G > 0.f;
        const float be = any ? xs.m + fast_log2(xs.G) : kNegInf;  // log2 of the prefix weight
        const float al = any ? xs.F * fast_rcp(xs.G) - vf : 0.f;  // prefix mean minus v
        const float kl = kf * kLog2e;
        const float ks = kl + U;
        const float Mt = fmaxf(be, ks);
        const float sa = fast_exp2(be - Mt), e = fast_exp2(ks - Mt);
        const float y = fmaf(al * sa, fast_rcp(sa + e), vf);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        xs = agg_add(agg_shift(xs, 1.f, D), Agg{kl, vf, 1.f});
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < NSB; ++q) {
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int t = q * SB + i;
        const float kf = kv.k(t), vf = kv.v(t);
        const bool any = xs.m != kNegInf && xs.G > 0.f;
        const float be = any ? xs.m + fast_log2(xs.G) : kNegInf;
        const float al = any ? xs.F * fast_rcp(xs.G) - vf : 0.f;
        lds_ab[i][tid] = make_float2(al, be);
        xs = agg_add(agg_shift(xs, 1.f, D), Agg{kf * kLog2e, vf, 1.f});
      }
      Agg ys = agg_add(cap[q], agg_shift(Y, static_cast<float>(L - (q + 1) * SB), D));
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
        const float2 ab2 = lds_ab[i][tid];
        const float kl = kf * kLog2e;
        const float ks = kl + U;
        const float Mt = fmaxf(fmaxf(ab2.y, ys.m), ks);
        const float sa = fast_exp2(ab2.y - Mt), sb = fast_exp2(ys.m - Mt);
        const float e = fast_exp2(ks - Mt);
        const float num = ab2.x * sa + fmaf(-ys.G, vf, ys.F) * sb;
        const float den = sa + ys.G * sb + e;
        float y;
        if constexpr (GATED) {
          const float er = fast_exp2(-kLog2e * gate.value(r_cur[i]));
          y = fmaf(vf, den, num) * fast_rcp(den * (1.f + er));
        } else {
          y = fmaf(num, fast_rcp(den), vf);
        }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), orr, out0 + t * row_bytes, 0,
                                              kStream);
        ys = agg_add(agg_shift(ys, 1.f, D), Agg{kl, vf, 1.f});
      }
    }
  }
}

// The wide form is rare (extreme w or u) and needs more registers than the fast form: keeping it
// out of line gives it its own register allocation, so its spills never touch the fast form. It
// reads the parameters from the kernel's argument segment (a pointer, so the kernel keeps them in
// scalar registers instead of building a private copy).
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
__device__ __noinline__ void row_body_wide(const RowParams* args, float* lds, unsigned unit,
                                           const unsigned* sh_epoch) {
  const RowParams p = *args;
  const RowLane ln = row_lane<TILE, L, NT>(p, unit);
  RowStore<DT, TILE, L, PAIR> kv;
  row_load<DT, TILE, L, NT, FUSED, PAIR>(p, ln, kv);
  row_body<DT, TILE, L, NT, FUSED, PAIR, true, CAUSAL, GATED>(p, ln, kv, lds, sh_epoch);
}

template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4)))
    biwkv_row_kernel(RowParams p) {
  static_assert(!PAIR || (DT == BIWKV_BF16 && TILE % 2 == 0), "pairs are bf16 channel pairs");
  static_assert(!(GATED && (CAUSAL || FUSED)), "the gate is built for the bidirectional entry");
  static_assert(64 % TILE == 0 || TILE % 64 == 0, "bad row-kernel tile");
  static_assert(TILE <= 64, "a wavefront must hold every channel of the tile");
  static_assert(NT % 256 == 0 && NT <= 1024 && NT >= 2 * TILE, "bad row-kernel workgroup size");
  __shared__ float lds[kRowLdsFloats<TILE, NT>];
  __shared__ unsigned sh_ticket, sh_epoch;
  const int tid = threadIdx.x;
  const bool chunked = p.n_chunks > 1;
  unsigned unit = blockIdx.x;
  bool valid = true;
  if (chunked && !p.ordered) {
    // Every workgroup of the launch fits on the device at once: chunks follow the grid order,
    // and the launch epoch is only needed once the scan (and its barriers) is done.
    if (tid == 0)
      sh_epoch = __hip_atomic_load(&p.ctr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (chunked) {
    if (tid == 0) {
      sh_ticket = __hip_atomic_fetch_add(&p.ctr->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh_epoch = __hip_atomic_load(&p.ctr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // A ticket beyond the grid can only come from a counter left non-zero by an earlier launch;
    // such a workgroup touches no data and only retires.
    valid = __builtin_amdgcn_readfirstlane(sh_ticket) < p.total;
    if (!valid && tid == 0)
      __hip_atomic_fetch_or(&p.ctr->fault, kFaultTicket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // uniform values: keep them in scalar registers (buffer resources are built from them)
    unit = __builtin_amdgcn_readfirstlane(sh_ticket);
  }
  if (valid) {  // uniform over the workgroup
    const RowLane ln = row_lane<TILE, L, NT>(p, unit);
    // The whole workgroup takes the wide form when any of its channels needs it. Every
    // wavefront holds all TILE channels, so a wavefront vote is the workgroup's vote.
    const bool wide_lane = fabsf(ln.D) * static_cast<float>(L - 1) > kFastRange ||
                           ln.U > kBonusRange || ln.U < -kBonusRange;
    if (__ballot(wide_lane) != 0ull) {
      // the kernel's only argument is p, at the start of the argument segment
      const auto* args = (const RowParams*)(__builtin_amdgcn_kernarg_segment_ptr());
      row_body_wide<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED>(args, lds, unit, &sh_epoch);
    } else {
      RowStore<DT, TILE, L, PAIR> kv;
      row_load<DT, TILE, L, NT, FUSED, PAIR>(p, ln, kv);
      row_body<DT, TILE, L, NT, FUSED, PAIR, false, CAUSAL, GATED>(p, ln, kv, lds, &sh_epoch);
    }
  }
  if (!valid && tid == 0) row_retire(p);  // (a valid workgroup retires after its exchange)
}

}  // namespace
