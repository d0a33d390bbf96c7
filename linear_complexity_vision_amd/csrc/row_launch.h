// Launches of the Bi-WKV tile kernel (included by the forward translation units).
#pragma once

#include "host.h"
#include "row_kernel.h"

namespace biwkv_host {

// The shape of the two-pass form: short chunks (4 groups of 32 tokens, 128 tokens per 256-thread
// workgroup), so that several workgroups share a CU and one's loads overlap another's arithmetic;
// nothing waits, and the carry kernel makes each chunk's cost independent of the row length.
constexpr int kTwoL = 32;
constexpr int kTwoNT = 256;

// Parameters of a tile-kernel launch with chunks of CT tokens. Returns the number of workgroups
// in *total, or an error.
template <int TILE, int CT, bool FUSED>
int row_params(const BiwkvParams& bp, int64_t B, RowParams* rp, long long* total) {
  const long long T = bp.T;
  // byte offsets inside one chunk of out (and so of k, v) must stay below 2^31 (the fused loads
  // also start each word's resource s W tokens early and reach s W tokens late)
  const long long reach = FUSED ? 2ll * bp.shift * bp.W : 0;
  if ((CT + reach) * static_cast<long long>(bp.C) * 4 >= (1ll << 31)) return BIWKV_ERR_UNSUPPORTED;
  const int64_t n_tiles = (bp.C + TILE - 1) / TILE;
  const int64_t n_chunks = (T + CT - 1) / CT;
  *total = B * n_tiles * n_chunks;
  if (*total > 0x7FFFFFFFll) return BIWKV_ERR_SHAPE;
  *rp = RowParams{};
  rp->k = bp.k;
  rp->v = bp.v;
  rp->r = bp.r;
  rp->w = bp.w;
  rp->u = bp.u;
  rp->out = bp.out;
  rp->T = T;
  rp->C = bp.C;
  rp->H = bp.H;
  rp->W = bp.W;
  rp->shift = bp.shift;
  rp->g1 = bp.g1;
  rp->g2 = bp.g2;
  rp->g3 = bp.g3;
  rp->g4 = bp.g4;
  rp->bidir = bp.bidir;
  rp->n_tiles = static_cast<int>(n_tiles);
  rp->n_chunks = static_cast<int>(n_chunks);
  rp->total = static_cast<unsigned>(*total);
  rp->spin_limit = g_spin_limit.load();
  return BIWKV_OK;
}

// Two passes: every chunk's totals, each chunk's carries (row_carry_kernel), then the outputs.
// Caller holds g_mu.
template <int DT, int TILE, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
int launch_two_pass(const BiwkvParams& bp, int64_t B, int dev, void* stream, const FixedScratch* fixed) {
  constexpr int L = kTwoL, NT = kTwoNT, CT = (NT / TILE) * L;
  RowParams rp;
  long long total = 0;
  int rc = row_params<TILE, CT, FUSED>(bp, B, &rp, &total);
  if (rc) return rc;
  // totals and carries: one (q, l, mu, -) float4 each per (chunk, direction, channel)
  const long long words = total * 2 * TILE * 4;
  unsigned long long* buf = nullptr;
  if (fixed) {
    if (words > fixed->n_words) return BIWKV_ERR_SCRATCH;
    buf = fixed->words;
  } else {
    StreamScratch* sc = nullptr;
    rc = get_scratch(dev, stream, words, &sc);
    if (rc) return rc;
    buf = sc->slots;
  }
  rp.sums = reinterpret_cast<float4*>(buf);
  rp.carries = rp.sums + total * 2 * TILE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(total)), block(NT);
  hipLaunchKernelGGL((biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, false, kSumsPass>), grid, block, 0, st,
                     rp);
  CarryParams cp{};
  cp.sums = rp.sums;
  cp.carries = rp.carries;
  cp.w = bp.w;
  cp.T = bp.T;
  cp.C = bp.C;
  cp.n_tiles = rp.n_tiles;
  cp.n_chunks = rp.n_chunks;
  cp.CT = CT;
  cp.causal = CAUSAL ? 1 : 0;
  const long long rows = total / rp.n_chunks;
  hipLaunchKernelGGL((row_carry_kernel<TILE>), dim3(static_cast<unsigned>(rows * (TILE / kCarryChans))),
                     dim3(64 * kCarryChans), 0, st, cp);
  hipLaunchKernelGGL((biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED, kOutPass>), grid, block, 0, st,
                     rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// One launch of the tile kernel (chunks of (NT / TILE) * L tokens) when all of its workgroups fit
// on the device at once; otherwise (or when BIWKV_OPT_TWO_PASS asks for it) the two-pass form.
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
int launch_row(const BiwkvParams& bp, int64_t B, int dev, void* stream, const FixedScratch* fixed) {
  constexpr int CT = (NT / TILE) * L;
  RowParams rp;
  long long total = 0;
  int rc = row_params<TILE, CT, FUSED>(bp, B, &rp, &total);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(total)), block(NT);
  const void* kfn =
      reinterpret_cast<const void*>(&biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED, kSinglePass>);
  std::lock_guard<std::mutex> lock(g_mu);
  int cap = 0;
  rc = resident_capacity(dev, kfn, NT, &cap);
  if (rc) return rc;
  // One launch needs every chunk of a row resident at once, not the whole grid: a chunk waits only
  // on the chunks of its own row, and blocks start in order, so a later row's chunks only wait for
  // slots that earlier rows free. Beyond one round, the chunks of a row that has started but not
  // yet got all its slots hold theirs idle; limiting a row to a quarter of the resident slots
  // bounds that loss, and longer rows take the two-pass form. BIWKV_OPT_TWO_PASS = 2 takes one
  // launch whenever a row fits at all.
  const int opt = g_two_pass.load();
  const bool one_launch = rp.n_chunks == 1 || total <= cap ||
                          (opt == 2 ? rp.n_chunks <= cap : rp.n_chunks <= cap / 4);
  if (opt == 1 || !one_launch)
    return launch_two_pass<DT, TILE, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
  if (rp.n_chunks > 1) {
    // single pass: three tagged 64-bit words per (chunk, direction, channel)
    const long long words = total * 2 * TILE * kSlotWords;
    if (g_xcd_local.load()) {
      int nx = 1;
      rc = device_xcds(dev, &nx);
      if (rc) return rc;
      const long long rows = total / rp.n_chunks;
      // a row kept on one XCD needs all its chunks resident there, on 1 / nx of the device
      if (nx > 1 && rp.n_chunks <= cap / nx) {
        rp.n_xcd = nx;
        rp.xcd_rows = static_cast<int>(rows / nx * nx);
      }
    }
    if (fixed) {
      if (words > fixed->n_words) return BIWKV_ERR_SCRATCH;
      rp.ctr = fixed->ctr;
      rp.slots = fixed->words;
    } else {
      StreamScratch* sc = nullptr;
      rc = get_scratch(dev, stream, words, &sc);
      if (rc) return rc;
      rp.ctr = sc->ctr;
      rp.slots = sc->slots;
    }
  }
  hipLaunchKernelGGL((biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED, kSinglePass>), grid, block, 0,
                     st, rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// Tile shapes: 64 channels per tile (one 128-byte line of bf16 k, two of fp32), 64 registers of
// k and v per lane, and chunks no longer than the sequence needs.
//  - Rows that one round of 1024-thread workgroups covers (at most one per CU) take one chunk of
//    up to 1024 tokens per row in 1024 threads (16 wavefronts per CU).
//  - More rows, and rows longer than 1024 tokens, take 512-thread workgroups, two per CU: the one
//    a CU received first gets its data first and computes and writes while the other one still
//    reads, so reads and writes overlap instead of alternating round by round. bf16 rows up to
//    896 tokens split into chunks of 448 (7 sub-blocks per lane); longer ones into 512. fp32 rows
//    up to 256 tokens take 32-channel tiles in 256 threads instead, four workgroups per CU (384
//    rows of 196 tokens: 14.6 against 16.3 us), with the same per-channel arithmetic.
//  - fp32 rows longer than 256 tokens keep 1024 threads: at 32 tokens per lane their 512-thread
//    chunks are short and the exchange between them dominates (config B1 T16384 C768: 44 against
//    42 us).
template <int DT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
int try_row_shape(const BiwkvParams& bp, int64_t B, int dev, void* stream, const FixedScratch* fixed) {
  const long long T = bp.T;
  int cus = 0;
  const int rc = device_cus(dev, &cus);
  if (rc) return rc;
  const bool one_round = B * ((bp.C + 63) / 64) <= cus;  // rows
  if constexpr (DT == BIWKV_BF16) {
    if (T <= 256) {
      if (one_round) return launch_row<DT, 64, 16, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
      return launch_row<DT, 64, 32, 512, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
    }
    if (T <= 512) {
      if (one_round) return launch_row<DT, 64, 32, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
      return launch_row<DT, 64, 64, 512, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
    }
    if (T <= 1024 && one_round)
      return launch_row<DT, 64, 64, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
    if (T <= 896) return launch_row<DT, 64, 56, 512, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
    return launch_row<DT, 64, 64, 512, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
  } else {
    if (T <= 256) {
      if (one_round) return launch_row<DT, 64, 16, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
      // 32-channel tiles (one 128-byte fp32 line per token) in 256 threads: twice the workgroups,
      // four per CU, so the rows spread evenly over the CUs
      return launch_row<DT, 32, 32, 256, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
    }
    return launch_row<DT, 64, 32, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream, fixed);
  }
}

// The tile kernel for one storage type and entry (kind), at the shape T calls for.
template <int DT, bool PAIR>
int forward_kind(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream, const FixedScratch* fixed) {
  switch (kind) {
    case kFused: return try_row_shape<DT, true, PAIR, false, false>(bp, B, dev, stream, fixed);
    case kCausal: return try_row_shape<DT, false, PAIR, true, false>(bp, B, dev, stream, fixed);
    case kGated: return try_row_shape<DT, false, PAIR, false, true>(bp, B, dev, stream, fixed);
    default: return try_row_shape<DT, false, PAIR, false, false>(bp, B, dev, stream, fixed);
  }
}

}  // namespace biwkv_host
