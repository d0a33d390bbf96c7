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
#include <type_traits>
#include <utility>
#include <vector>

#include "biwkv.h"

#include "backward.cuh"
#include "bwd_tile.cuh"
#include "chunk_kernel.cuh"
#include "common.cuh"
#include "qshift_kernel.cuh"
#include "row_kernel.cuh"

namespace {

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
  float* bwd = nullptr;  // backward pass sums, carries and per-chunk terms
  long long bwd_floats = 0;
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

// The sequence shift of N tokens: the same gamma range, 0 <= shift <= N.
int check_bidir_params(int64_t N, int shift, double gamma) {
  if (!(gamma >= 0.0 && gamma <= 0.25)) return BIWKV_ERR_PARAM;
  if (shift < 0 || shift > N) return BIWKV_ERR_PARAM;
  return BIWKV_OK;
}

constexpr int64_t kMaxDim = (1ll << 31) - 1;
constexpr int kMaxMix = 8;  // mixing vectors per qshift_mix call

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

// Tile kernel launch: rows of TILE channels, chunks of (NT / TILE) * L tokens. Returns 1 when
// the shape is outside what the kernel addresses (the caller then uses the chunk-scan kernel).
template <int DT, int TILE, int L, int NT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
int launch_row(const BiwkvParams& bp, int64_t B, int dev, void* stream) {
  constexpr int CT = (NT / TILE) * L;
  const long long T = bp.T;
  // byte offsets into one batch item of out (and so of k, v), including the empty slots past
  // the row end, must stay below 2^31
  // (the fused loads also start each word's resource s W tokens early and reach s W tokens late)
  const long long reach = FUSED ? 2ll * bp.shift * bp.W : 0;
  if ((T + CT + reach) * static_cast<long long>(bp.C) * 4 >= (1ll << 31)) return 1;
  const int64_t n_tiles = (bp.C + TILE - 1) / TILE;
  const int64_t n_chunks = (T + CT - 1) / CT;
  const int64_t total = B * n_tiles * n_chunks;
  if (total > 0x7FFFFFFFll) return BIWKV_ERR_SHAPE;
  RowParams rp{};
  rp.k = bp.k;
  rp.v = bp.v;
  rp.r = bp.r;
  rp.w = bp.w;
  rp.u = bp.u;
  rp.out = bp.out;
  rp.T = T;
  rp.C = bp.C;
  rp.H = bp.H;
  rp.W = bp.W;
  rp.shift = bp.shift;
  rp.g1 = bp.g1;
  rp.g2 = bp.g2;
  rp.g3 = bp.g3;
  rp.g4 = bp.g4;
  rp.bidir = bp.bidir;
  rp.n_tiles = static_cast<int>(n_tiles);
  rp.n_chunks = static_cast<int>(n_chunks);
  rp.total = static_cast<unsigned>(total);
  if (n_chunks > 1) {
    // The chunks of a row wait for each other: they must all fit on the device at once.
    const void* kfn = reinterpret_cast<const void*>(&biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED>);
    std::lock_guard<std::mutex> lock(g_mu);
    int cap = 0;
    int rc = resident_capacity(dev, kfn, NT, &cap);
    if (rc) return rc;
    if (n_chunks > cap) return 1;
    rp.ordered = total > cap ? 1 : 0;
    StreamScratch* sc = nullptr;
    rc = get_scratch(dev, stream, total * 2 * TILE * 2, &sc);
    if (rc) return rc;
    rp.ctr = sc->ctr;
    rp.slots = sc->slots;
    hipLaunchKernelGGL((biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED>),
                       dim3(static_cast<unsigned>(total)), dim3(NT), 0,
                       static_cast<hipStream_t>(stream), rp);
  } else {
    hipLaunchKernelGGL((biwkv_row_kernel<DT, TILE, L, NT, FUSED, PAIR, CAUSAL, GATED>),
                       dim3(static_cast<unsigned>(total)), dim3(NT), 0,
                       static_cast<hipStream_t>(stream), rp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// Tile shapes: 64 channels per tile (one 128-byte line of bf16 k, two of fp32), 64 registers of
// k and v per lane, and chunks no longer than the sequence needs. Rows longer than one chunk of
// 1024 tokens use 512-thread workgroups (two per CU): the workgroup a CU received first gets its
// data first and computes and writes while the other one still reads, so reads and writes
// overlap. fp32 rows keep 1024 threads: at 32 tokens per lane their 512-thread chunks are short
// and the exchange between them dominates.
template <int DT, bool FUSED, bool PAIR, bool CAUSAL, bool GATED>
int try_row_shape(const BiwkvParams& bp, int64_t B, int dev, void* stream) {
  const long long T = bp.T;
  if constexpr (DT == BIWKV_BF16) {
    if (T <= 256) return launch_row<DT, 64, 16, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream);
    if (T <= 512) return launch_row<DT, 64, 32, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream);
    if (T <= 1024) return launch_row<DT, 64, 64, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream);
    return launch_row<DT, 64, 64, 512, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream);
  } else {
    if (T <= 256) return launch_row<DT, 64, 16, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream);
    return launch_row<DT, 64, 32, 1024, FUSED, PAIR, CAUSAL, GATED>(bp, B, dev, stream);
  }
}

// bf16 rows read channel pairs as 32-bit words when every pair is whole: C even, 4-byte aligned
// k and v, and Q-Shift group boundaries on even channels.
bool pairs_ok(const BiwkvParams& bp, bool fused) {
  if (bp.C % 2 != 0 || !aligned(bp.k, 4) || !aligned(bp.v, 4)) return false;
  if (fused && ((bp.g1 | bp.g2 | bp.g3 | bp.g4) & 1)) return false;
  return true;
}

template <int DT, bool FUSED, bool CAUSAL = false, bool GATED = false>
int try_row(const BiwkvParams& bp, int64_t B, int dev, void* stream) {
  if constexpr (DT == BIWKV_BF16) {
    if (pairs_ok(bp, FUSED)) return try_row_shape<DT, FUSED, true, CAUSAL, GATED>(bp, B, dev, stream);
  }
  return try_row_shape<DT, FUSED, false, CAUSAL, GATED>(bp, B, dev, stream);
}

template <bool FUSED>
int dispatch_biwkv(BiwkvParams prm, int64_t B, int dtype, bool vec2, int dev, void* stream) {
  const int rrc = dtype == BIWKV_F32 ? try_row<BIWKV_F32, FUSED>(prm, B, dev, stream)
                                     : try_row<BIWKV_BF16, FUSED>(prm, B, dev, stream);
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

// The gather behind qshift and qshift_bidir (parameters already checked, nothing empty). bidir:
// the sequence shift, given as a 1 x N grid.
int launch_qshift(const float* x, float* out, int64_t B, int64_t H, int64_t W, int64_t C, int shift,
                  double gamma, int bidir, void* stream) {
  if (!aligned(x, 4) || !aligned(out, 4)) return BIWKV_ERR_ALIGN;
  const size_t n = static_cast<size_t>(B) * H * W * C;
  if (ranges_overlap(out, n * 4, x, n * 4)) return BIWKV_ERR_ALIAS;
  int dev = 0;
  int rc = current_device(&dev);
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
  // index divisors of the launch (channel groups per row, tokens per image, columns)
  const FastDiv cv = make_fastdiv(static_cast<uint32_t>(vec4 ? C / 4 : C));
  const FastDiv hw = make_fastdiv(static_cast<uint32_t>(H * W)), wd = make_fastdiv(static_cast<uint32_t>(W));
  const bool big = items >= (1ll << 31);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int Hi = static_cast<int>(H), Wi = static_cast<int>(W), Ci = static_cast<int>(C);
  const int g0 = static_cast<int>(g[0]), g1 = static_cast<int>(g[1]), g2 = static_cast<int>(g[2]),
            g3 = static_cast<int>(g[3]);
  if (vec4 && !big)
    hipLaunchKernelGGL((qshift_kernel<4, false>), grid, block, 0, st, xi, oi, rows, cv, hw, wd, Hi, Wi, Ci,
                       shift, g0, g1, g2, g3, bidir);
  else if (vec4)
    hipLaunchKernelGGL((qshift_kernel<4, true>), grid, block, 0, st, xi, oi, rows, cv, hw, wd, Hi, Wi, Ci,
                       shift, g0, g1, g2, g3, bidir);
  else if (!big)
    hipLaunchKernelGGL((qshift_kernel<1, false>), grid, block, 0, st, xi, oi, rows, cv, hw, wd, Hi, Wi, Ci,
                       shift, g0, g1, g2, g3, bidir);
  else
    hipLaunchKernelGGL((qshift_kernel<1, true>), grid, block, 0, st, xi, oi, rows, cv, hw, wd, Hi, Wi, Ci,
                       shift, g0, g1, g2, g3, bidir);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// The fused entries' common part: Bi-WKV of the shifted k and v (grid Q-Shift, or with bidir the
// sequence shift, passed as H = N, W = 1). Parameters already checked, nothing empty.
int fused_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                  int64_t B, int64_t H, int64_t W, int64_t C, int shift, double gamma, int dtype,
                  int bidir, void* stream) {
  int dev = 0;
  int rc = current_device(&dev);
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
  prm.T = H * W;
  prm.C = static_cast<int>(C);
  prm.H = static_cast<int>(H);
  prm.W = static_cast<int>(W);
  prm.shift = shift;
  prm.g1 = static_cast<int>(g[0]);
  prm.g2 = static_cast<int>(g[1]);
  prm.g3 = static_cast<int>(g[2]);
  prm.g4 = static_cast<int>(g[3]);
  prm.bidir = bidir;
  if (!bidir) return dispatch_biwkv<true>(prm, B, dtype, vec2, dev, stream);
  // the sequence shift exists in the tile kernel only: a shape it does not address has no fallback
  rc = dtype == BIWKV_F32 ? try_row<BIWKV_F32, true>(prm, B, dev, stream)
                          : try_row<BIWKV_BF16, true>(prm, B, dev, stream);
  return rc == 1 ? BIWKV_ERR_UNSUPPORTED : rc;
}

// Backward tile shape: 8 tokens per lane, 512 threads (two workgroups per CU, so one's loads
// overlap the other's arithmetic), 64-token chunks.
constexpr int kBwdL = 8;
constexpr int kBwdNT = 512;

// The backward: bwd_tile_kernel in one launch (a row of one chunk) or three (stages 1, 2, 3),
// then the dw / du fold. Arguments already checked, nothing empty.
template <int DT, int L, int NT, int WPE, bool PAIR>
int launch_bwd_tile(const void* k, const void* v, const float* w, const float* u, const float* g,
                    float* dk, float* dv, float* dw, float* du, int64_t B, int64_t T, int64_t C, int dev,
                    void* stream) {
  constexpr int CT = (NT / kBtTile) * L;
  const int64_t n_tiles = (C + kBtTile - 1) / kBtTile;
  const int64_t n_chunks = (T + CT - 1) / CT;
  const int64_t total = B * n_tiles * n_chunks;
  if (total > 0x7FFFFFFFll) return BIWKV_ERR_SHAPE;
  // the loads address a batch item (fp32 g, and the row's padding) with 32-bit byte offsets
  if ((T + CT) * C * 4 >= (1ll << 31)) return BIWKV_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  BwdTileParams tp{};
  {
    std::lock_guard<std::mutex> lock(g_mu);
    StreamScratch* sc = nullptr;
    int rc = get_scratch(dev, stream, 0, &sc);
    if (rc) return rc;
    const long long terms = B * n_chunks * C;                         // dw, du terms
    const long long sums = n_chunks > 1 ? total * 2 * kBtTile * 3 : 0;  // chunk sums per round
    rc = grow_zeroed(&sc->bwd, &sc->bwd_floats, 2 * terms + 4 * sums, 1ll << 20, st, &sc->retired);
    if (rc) return rc;
    tp.pw = sc->bwd;
    tp.pu = sc->bwd + terms;
    tp.sums1 = sc->bwd + 2 * terms;
    tp.sums2 = tp.sums1 + sums;
    tp.carry1 = tp.sums2 + sums;
    tp.carry2 = tp.carry1 + sums;
  }
  tp.k = k;
  tp.v = v;
  tp.w = w;
  tp.u = u;
  tp.g = g;
  tp.dk = dk;
  tp.dv = dv;
  tp.T = T;
  tp.C = static_cast<int>(C);
  tp.n_tiles = static_cast<int>(n_tiles);
  tp.n_chunks = static_cast<int>(n_chunks);
  const dim3 grid(static_cast<unsigned>(total)), block(NT);
  if (n_chunks == 1) {
    hipLaunchKernelGGL((bwd_tile_kernel<DT, L, NT, WPE, 0, PAIR>), grid, block, 0, st, tp);
  } else {
    // stage 1: one lane per (channel, chunk); 8 chunks of a row per workgroup
    constexpr int SNT = 512;
    const dim3 sgrid(static_cast<unsigned>((n_chunks + SNT / kBtTile - 1) / (SNT / kBtTile) * B * n_tiles));
    hipLaunchKernelGGL((bwd_chunk_sums_kernel<DT, CT, SNT, PAIR>), sgrid, dim3(SNT), 0, st, tp);
    const dim3 rows(static_cast<unsigned>(B * n_tiles)), cblock(64 * kCarryGroups);
    hipLaunchKernelGGL((bwd_carry_kernel<CT>), rows, cblock, 0, st, tp, tp.sums1, tp.carry1);
    hipLaunchKernelGGL((bwd_tile_kernel<DT, L, NT, WPE, 2, PAIR>), grid, block, 0, st, tp);
    hipLaunchKernelGGL((bwd_carry_kernel<CT>), rows, cblock, 0, st, tp, tp.sums2, tp.carry2);
    hipLaunchKernelGGL((bwd_tile_kernel<DT, L, NT, WPE, 3, PAIR>), grid, block, 0, st, tp);
  }
  BwdParams rp{};
  rp.w = w;
  rp.dw = dw;
  rp.du = du;
  rp.T = T;
  rp.B = static_cast<int>(B);
  rp.C = static_cast<int>(C);
  rp.n_chunks = static_cast<int>(n_chunks);
  rp.n_wg = static_cast<int>(n_chunks);
  rp.s.pw = tp.pw;
  rp.s.pu = tp.pu;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>((C + 63) / 64)), dim3(64 * kReduceGroups), 0,
                     st, rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
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

int biwkv_gated_forward(const void* k, const void* v, const void* r, const float* w, const float* u,
                        float* out, int64_t B, int64_t T, int64_t C, int dtype, void* stream) {
  int rc = validate_biwkv(k, v, w, u, out, B, T, C, dtype);
  if (rc || !(B && T && C)) return rc;
  if (!r) return BIWKV_ERR_NULL;
  const size_t es = dtype == BIWKV_F32 ? 4 : 2;
  if (!aligned(r, es)) return BIWKV_ERR_ALIGN;
  const size_t n = static_cast<size_t>(B) * T * C;
  if (ranges_overlap(out, n * 4, r, n * es)) return BIWKV_ERR_ALIAS;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  BiwkvParams prm{};
  prm.k = k;
  prm.v = v;
  prm.r = r;
  prm.w = w;
  prm.u = u;
  prm.out = out;
  prm.T = T;
  prm.C = static_cast<int>(C);
  // tile kernel only: a shape it does not address has no fallback
  rc = dtype == BIWKV_F32 ? try_row<BIWKV_F32, false, false, true>(prm, B, dev, stream)
                          : try_row<BIWKV_BF16, false, false, true>(prm, B, dev, stream);
  return rc == 1 ? BIWKV_ERR_UNSUPPORTED : rc;
}

int biwkv_backward(const void* k, const void* v, const float* w, const float* u, const float* g,
                   float* dk, float* dv, float* dw, float* du, int64_t B, int64_t T, int64_t C,
                   int dtype, void* stream) {
  int rc = check_bitc_shape(B, T, C);
  if (rc) return rc;
  if (dtype != BIWKV_F32 && dtype != BIWKV_BF16) return BIWKV_ERR_DTYPE;
  const bool nonempty = B && T && C;
  if (nonempty && (!k || !v || !g || !dk || !dv)) return BIWKV_ERR_NULL;
  if (C && (!w || !u || !dw || !du)) return BIWKV_ERR_NULL;
  if (!C) return BIWKV_OK;
  const size_t es = dtype == BIWKV_F32 ? 4 : 2;
  const size_t n = static_cast<size_t>(B) * T * C;
  if ((nonempty && (!aligned(k, es) || !aligned(v, es) || !aligned(g, 4) || !aligned(dk, 4) ||
                    !aligned(dv, 4))) ||
      !aligned(w, 4) || !aligned(u, 4) || !aligned(dw, 4) || !aligned(du, 4))
    return BIWKV_ERR_ALIGN;
  // outputs overlap neither each other nor any input
  const void* outs[4] = {dk, dv, dw, du};
  const size_t out_n[4] = {nonempty ? n * 4 : 0, nonempty ? n * 4 : 0, static_cast<size_t>(C) * 4,
                           static_cast<size_t>(C) * 4};
  const void* ins[5] = {k, v, g, w, u};
  const size_t in_n[5] = {nonempty ? n * es : 0, nonempty ? n * es : 0, nonempty ? n * 4 : 0,
                          static_cast<size_t>(C) * 4, static_cast<size_t>(C) * 4};
  for (int a = 0; a < 4; ++a) {
    for (int b2 = 0; b2 < 5; ++b2)
      if (ranges_overlap(outs[a], out_n[a], ins[b2], in_n[b2])) return BIWKV_ERR_ALIAS;
    for (int b2 = a + 1; b2 < 4; ++b2)
      if (ranges_overlap(outs[a], out_n[a], outs[b2], out_n[b2])) return BIWKV_ERR_ALIAS;
  }
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned cb = static_cast<unsigned>((C + 255) / 256);
  if (!nonempty) {
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(cb), dim3(256), 0, st, dw, du, static_cast<int>(C));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? BIWKV_OK : hip_fail(e);
  }
  // token positions times D must be exact in fp32
  if (T >= (1ll << 24)) return BIWKV_ERR_UNSUPPORTED;
  if (dtype == BIWKV_F32)
    return launch_bwd_tile<BIWKV_F32, kBwdL, kBwdNT, 4, false>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
  // bf16 k and v load as 32-bit channel pairs when every pair is whole and aligned
  if (C % 2 == 0 && aligned(k, 4) && aligned(v, 4))
    return launch_bwd_tile<BIWKV_BF16, kBwdL, kBwdNT, 4, true>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
  return launch_bwd_tile<BIWKV_BF16, kBwdL, kBwdNT, 4, false>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
}

int biwkv_causal_forward(const void* k, const void* v, const float* w, const float* u, float* out,
                         int64_t B, int64_t T, int64_t C, int dtype, void* stream) {
  int rc = validate_biwkv(k, v, w, u, out, B, T, C, dtype);
  if (rc || !(B && T && C)) return rc;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  BiwkvParams prm{};
  prm.k = k;
  prm.v = v;
  prm.w = w;
  prm.u = u;
  prm.out = out;
  prm.T = T;
  prm.C = static_cast<int>(C);
  // tile kernel only: a shape it does not address has no fallback
  rc = dtype == BIWKV_F32 ? try_row<BIWKV_F32, false, true>(prm, B, dev, stream)
                          : try_row<BIWKV_BF16, false, true>(prm, B, dev, stream);
  return rc == 1 ? BIWKV_ERR_UNSUPPORTED : rc;
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
  return fused_forward(k, v, w, u, out, B, H, W, C, shift, gamma, dtype, 0, stream);
}

int biwkv_qshift_bidir_forward(const void* k, const void* v, const float* w, const float* u,
                               float* out, int64_t B, int64_t N, int64_t C, int shift, double gamma,
                               int dtype, void* stream) {
  int rc = validate_biwkv(k, v, w, u, out, B, N, C, dtype);
  if (rc) return rc;
  rc = check_bidir_params(N, shift, gamma);
  if (rc || !(B && N && C)) return rc;
  return fused_forward(k, v, w, u, out, B, N, 1, C, shift, gamma, dtype, 1, stream);
}

int qshift_mix(const float* x, const float* mu, float* out, int64_t B, int64_t H, int64_t W,
               int64_t C, int n_mix, int shift, double gamma, void* stream) {
  if (H < 0 || W < 0 || H > kMaxDim || W > kMaxDim) return BIWKV_ERR_SHAPE;
  if (n_mix < 0 || n_mix > kMaxMix) return BIWKV_ERR_SHAPE;
  int rc = check_bitc_shape(B, H * W, C);
  if (rc) return rc;
  const bool nonempty = B && H && W && C && n_mix;
  if (nonempty && (!x || !mu || !out)) return BIWKV_ERR_NULL;
  rc = check_qshift_params(H, W, shift, gamma);
  if (rc || !nonempty) return rc;
  if (!aligned(x, 4) || !aligned(mu, 4) || !aligned(out, 4)) return BIWKV_ERR_ALIGN;
  const size_t n = static_cast<size_t>(B) * H * W * C;
  const size_t out_bytes = n * 4 * static_cast<size_t>(n_mix);
  if (ranges_overlap(out, out_bytes, x, n * 4) || ranges_overlap(out, out_bytes, mu, C * 4 * n_mix))
    return BIWKV_ERR_ALIAS;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  int64_t g[4];
  group_bounds(C, gamma, g);
  const bool vec4 = (C % 4 == 0) && (g[0] % 4 == 0) && (g[1] % 4 == 0) && (g[2] % 4 == 0) &&
                    (g[3] % 4 == 0) && aligned(x, 16) && aligned(mu, 16) && aligned(out, 16);
  const long long rows = B * H * W;
  const long long items = rows * (vec4 ? C / 4 : C);
  long long blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const FastDiv cv = make_fastdiv(static_cast<uint32_t>(vec4 ? C / 4 : C));
  const FastDiv hw = make_fastdiv(static_cast<uint32_t>(H * W)), wd = make_fastdiv(static_cast<uint32_t>(W));
  const bool big = items >= (1ll << 31);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int Hi = static_cast<int>(H), Wi = static_cast<int>(W), Ci = static_cast<int>(C);
  const int g0 = static_cast<int>(g[0]), g1 = static_cast<int>(g[1]), g2 = static_cast<int>(g[2]),
            g3 = static_cast<int>(g[3]);
  if (vec4 && !big)
    hipLaunchKernelGGL((qshift_mix_kernel<4, false>), grid, block, 0, st, x, mu, out, rows, cv, hw, wd, Hi,
                       Wi, Ci, n_mix, shift, g0, g1, g2, g3);
  else if (vec4)
    hipLaunchKernelGGL((qshift_mix_kernel<4, true>), grid, block, 0, st, x, mu, out, rows, cv, hw, wd, Hi,
                       Wi, Ci, n_mix, shift, g0, g1, g2, g3);
  else if (!big)
    hipLaunchKernelGGL((qshift_mix_kernel<1, false>), grid, block, 0, st, x, mu, out, rows, cv, hw, wd, Hi,
                       Wi, Ci, n_mix, shift, g0, g1, g2, g3);
  else
    hipLaunchKernelGGL((qshift_mix_kernel<1, true>), grid, block, 0, st, x, mu, out, rows, cv, hw, wd, Hi,
                       Wi, Ci, n_mix, shift, g0, g1, g2, g3);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
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
  return launch_qshift(x, out, B, H, W, C, shift, gamma, 0, stream);
}

int qshift_bidir(const float* x, float* out, int64_t B, int64_t N, int64_t C, int shift, double gamma,
                 void* stream) {
  int rc = check_bitc_shape(B, N, C);
  if (rc) return rc;
  const bool nonempty = B && N && C;
  if (nonempty && (!x || !out)) return BIWKV_ERR_NULL;
  rc = check_bidir_params(N, shift, gamma);
  if (rc || !nonempty) return rc;
  return launch_qshift(x, out, B, 1, N, C, shift, gamma, 1, stream);
}

const char* biwkv_status_string(int status) {
  switch (status) {
    case BIWKV_OK: return "ok";
    case BIWKV_ERR_NULL: return "a required pointer is NULL";
    case BIWKV_ERR_SHAPE: return "invalid shape (negative, too large, or T != H*W)";
    case BIWKV_ERR_DTYPE: return "unknown dtype (expected BIWKV_F32 or BIWKV_BF16)";
    case BIWKV_ERR_PARAM: return "invalid shift parameter (gamma outside [0, 1/4], or shift < 0 or beyond the grid (min(H, W)) or the sequence (N))";
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
    // Clear the fault word, and the ticket and arrival counts that an interrupted launch may
    // have left behind (the stream is idle here); the epoch keeps counting.
    Counters fresh = c;
    fresh.ticket = 0;
    fresh.done = 0;
    fresh.fault = 0;
    e = hipMemcpy(it->second->ctr, &fresh, sizeof(Counters), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
  }
  return BIWKV_OK;
}

int biwkv_version(void) { return 100; }

}  // extern "C"
