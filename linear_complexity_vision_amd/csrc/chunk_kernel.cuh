// Bi-WKV chunk-scan kernel (rows longer than one workgroup holds).
#pragma once

#include "common.cuh"

namespace {

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

}  // namespace
