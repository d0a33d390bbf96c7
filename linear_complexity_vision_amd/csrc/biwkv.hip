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
//   * The chunks of a row are combined through their decayed sums: in one launch, by an exchange
//     of epoch-tagged slots between resident workgroups (a wait that runs out recomputes the
//     peer's sums from k and v, so no result depends on residency), or in two launches when the
//     workgroups cannot all be resident (every chunk's totals, then the outputs).
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

#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "biwkv.h"

#include "common.h"
#include "host.h"
#include "qshift_kernel.h"

namespace biwkv_host {

namespace {

thread_local int t_last_hip_error = 0;

std::map<std::pair<int, void*>, StreamScratch*> g_scratch;
std::map<std::pair<int, const void*>, int> g_capacity;  // (device, kernel) -> resident workgroups
std::map<int, int> g_xcds;                                // device -> XCDs
std::map<int, int> g_cus;                                 // device -> compute units

// Grows a zero-filled scratch buffer in stream order: the new buffer is allocated and cleared on
// `st`, and the outgrown one is freed on `st` behind every launch already queued that uses it.
template <typename Tp>
int grow_zeroed(Tp** buf, long long* cap, long long need, long long min_cap, hipStream_t st) {
  if (*cap >= need) return BIWKV_OK;
  long long want = *cap ? *cap : min_cap;
  while (want < need) want *= 2;
  const long long words = (want * static_cast<long long>(sizeof(Tp)) + 7) / 8;
  void* fresh = nullptr;
  hipError_t e = hipMallocAsync(&fresh, static_cast<size_t>(words) * 8, st);
  if (e != hipSuccess) return hip_fail(e);
  long long blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<unsigned long long*>(fresh), words);
  e = hipGetLastError();
  if (e != hipSuccess) {
    (void)hipFreeAsync(fresh, st);
    return hip_fail(e);
  }
  if (*buf) {
    e = hipFreeAsync(*buf, st);
    if (e != hipSuccess) {
      (void)hipFreeAsync(fresh, st);
      return hip_fail(e);
    }
  }
  *buf = static_cast<Tp*>(fresh);
  *cap = want;
  return BIWKV_OK;
}

// The stream's scratch record, created (with its counter block) on first use. Caller holds g_mu.
int stream_scratch(int dev, void* stream, StreamScratch** out) {
  auto key = std::make_pair(dev, stream);
  StreamScratch*& sc = g_scratch[key];
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!sc) {
    StreamScratch* fresh = new StreamScratch();
    hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&fresh->ctr), 256, st);
    if (e != hipSuccess) {
      delete fresh;
      g_scratch.erase(key);
      return hip_fail(e);
    }
    hipLaunchKernelGGL(init_counters_kernel, dim3(1), dim3(1), 0, st, fresh->ctr);
    e = hipGetLastError();
    if (e != hipSuccess) {
      (void)hipFreeAsync(fresh->ctr, st);
      delete fresh;
      g_scratch.erase(key);
      return hip_fail(e);
    }
    sc = fresh;
  }
  *out = sc;
  return BIWKV_OK;
}

}  // namespace

std::mutex g_mu;
std::atomic<unsigned> g_spin_limit{kSpinDefault};
std::atomic<int> g_two_pass{0};
std::atomic<int> g_wide_index{0};
std::atomic<int> g_xcd_local{1};

int hip_fail(hipError_t e) {
  t_last_hip_error = static_cast<int>(e);
  return BIWKV_ERR_HIP;
}

int current_device(int* dev) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return BIWKV_ERR_NO_DEVICE;
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

int get_scratch(int dev, void* stream, long long words, StreamScratch** out) {
  StreamScratch* sc = nullptr;
  int rc = stream_scratch(dev, stream, &sc);
  if (rc) return rc;
  rc = grow_zeroed(&sc->slots, &sc->slot_words, words, 1ll << 16, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  *out = sc;
  return BIWKV_OK;
}

int get_bwd_scratch(int dev, void* stream, long long floats, float** out) {
  StreamScratch* sc = nullptr;
  int rc = stream_scratch(dev, stream, &sc);
  if (rc) return rc;
  rc = grow_zeroed(&sc->bwd, &sc->bwd_floats, floats, 1ll << 20, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  *out = sc->bwd;
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

int device_cus(int dev, int* n) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) {
    *n = it->second;
    return BIWKV_OK;
  }
  int x = 0;
  const hipError_t e = hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e);
  *n = x > 0 ? x : 1;
  g_cus[dev] = *n;
  return BIWKV_OK;
}

int device_xcds(int dev, int* n) {
  auto it = g_xcds.find(dev);
  if (it != g_xcds.end()) {
    *n = it->second;
    return BIWKV_OK;
  }
  int x = 0;
  const hipError_t e = hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev);
  if (e != hipSuccess) return hip_fail(e);
  *n = x > 0 ? x : 1;
  g_xcds[dev] = *n;
  return BIWKV_OK;
}

}  // namespace biwkv_host

using namespace biwkv_host;

namespace {

// The allocation-free entry's scratch: one counter block (256 bytes) and the chunk sums of one
// launch, as a file-scope device array. Each device holds its own copy at its own address, found
// with hipGetSymbolAddress once per device; host code uses only that address (the array's name
// here is a host-side stand-in, not a device address). All calls on a device share it.
constexpr size_t kStaticCounterBytes = 256;
constexpr size_t kStaticScratchBytes = kStaticCounterBytes + (8u << 20);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::map<int, void*> g_static_scratch;  // device -> address of its scratch (guarded by g_mu)

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!na || !nb) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}


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

// Tile kernel launch: rows of TILE channels, chunks of (NT / TILE) * L tokens. A row of several
// chunks runs in one launch when every workgroup fits on the device at once (and two passes are
// not asked for), otherwise in two.
// bf16 rows read channel pairs as 32-bit words when every pair is whole: C even, 4-byte aligned
// k and v, and Q-Shift group boundaries on even channels.
bool pairs_ok(const BiwkvParams& bp, bool fused) {
  if (bp.C % 2 != 0 || !aligned(bp.k, 4) || !aligned(bp.v, 4)) return false;
  if (fused && ((bp.g1 | bp.g2 | bp.g3 | bp.g4) & 1)) return false;
  return true;
}

// The tile kernel for a storage type and entry (parameters already checked, nothing empty).
int forward_dispatch(const BiwkvParams& bp, int64_t B, int dtype, int kind, int dev, void* stream,
                     const FixedScratch* fixed = nullptr) {
  if (dtype == BIWKV_F32) return forward_f32(bp, B, kind, dev, stream, fixed);
  if (pairs_ok(bp, kind == kFused)) return forward_bf16_pair(bp, B, kind, dev, stream, fixed);
  return forward_bf16(bp, B, kind, dev, stream, fixed);
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
  const bool big = items >= (1ll << 31) || g_wide_index.load() != 0;
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
  return forward_dispatch(prm, B, dtype, kFused, dev, stream);
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
  BiwkvParams prm{};
  prm.k = k;
  prm.v = v;
  prm.w = w;
  prm.u = u;
  prm.out = out;
  prm.T = T;
  prm.C = static_cast<int>(C);
  return forward_dispatch(prm, B, dtype, kPlain, dev, stream);
}

int biwkv_forward_noalloc(const void* k, const void* v, const float* w, const float* u, float* out,
                          int64_t B, int64_t T, int64_t C, int dtype, void* stream) {
  int rc = validate_biwkv(k, v, w, u, out, B, T, C, dtype);
  if (rc || !(B && T && C)) return rc;
  int dev = 0;
  rc = current_device(&dev);
  if (rc) return rc;
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_static_scratch.find(dev);
    if (it != g_static_scratch.end()) {
      base = it->second;
    } else {
      hipError_t e = hipGetSymbolAddress(&base, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      g_static_scratch[dev] = base;
    }
  }
  FixedScratch fixed{};
  fixed.ctr = static_cast<Counters*>(base);
  fixed.words = reinterpret_cast<unsigned long long*>(static_cast<char*>(base) + kStaticCounterBytes);
  fixed.n_words = static_cast<long long>((kStaticScratchBytes - kStaticCounterBytes) / 8);
  BiwkvParams prm{};
  prm.k = k;
  prm.v = v;
  prm.w = w;
  prm.u = u;
  prm.out = out;
  prm.T = T;
  prm.C = static_cast<int>(C);
  return forward_dispatch(prm, B, dtype, kPlain, dev, stream, &fixed);
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
  return forward_dispatch(prm, B, dtype, kGated, dev, stream);
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
  if (!nonempty) return backward_empty(dw, du, C, stream);
  // token positions times D must be exact in fp32
  if (T >= (1ll << 24)) return BIWKV_ERR_UNSUPPORTED;
  return backward(k, v, w, u, g, dk, dv, dw, du, B, T, C, dtype, dev, stream);
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
  return forward_dispatch(prm, B, dtype, kCausal, dev, stream);
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
  const bool big = items >= (1ll << 31) || g_wide_index.load() != 0;
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
    case BIWKV_ERR_PARAM: return "invalid parameter (gamma outside [0, 1/4], shift < 0 or beyond the grid (min(H, W)) or the sequence (N), or an unknown option or option value)";
    case BIWKV_ERR_ALIAS: return "output overlaps an input";
    case BIWKV_ERR_ALIGN: return "pointer not aligned to its element size";
    case BIWKV_ERR_NO_DEVICE: return "no usable HIP device";
    case BIWKV_ERR_HIP: return "HIP runtime error (see biwkv_last_hip_error)";
    case BIWKV_ERR_SCRATCH: return "problem needs more scratch than the allocation-free entry's static buffer holds (8 MiB of chunk sums)";
    case BIWKV_ERR_UNSUPPORTED: return "shape outside what the kernels address (see the entry point's limits)";
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
    // Clear the fault word (the stream is idle here); the epoch keeps counting.
    Counters fresh = c;
    fresh.fault = 0;
    e = hipMemcpy(it->second->ctr, &fresh, sizeof(Counters), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
  }
  return BIWKV_OK;
}

int biwkv_release_scratch(void* stream) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_scratch.find(std::make_pair(dev, stream));
  if (it == g_scratch.end()) return BIWKV_OK;
  StreamScratch* sc = it->second;
  g_scratch.erase(it);
  if (!sc) return BIWKV_OK;
  // stream-ordered frees: they take effect once the launches already queued on the stream are done
  hipError_t e = hipSuccess;
  for (void* p : {static_cast<void*>(sc->ctr), static_cast<void*>(sc->slots), static_cast<void*>(sc->bwd)}) {
    if (!p) continue;
    const hipError_t ei = hipFreeAsync(p, st);
    if (e == hipSuccess) e = ei;
  }
  delete sc;
  return e == hipSuccess ? BIWKV_OK : hip_fail(e);
}

int biwkv_set_option(int option, int64_t value, int64_t* previous) {
  switch (option) {
    case BIWKV_OPT_SPIN_LIMIT: {
      if (value < 0 || value > 0xffffffffll) return BIWKV_ERR_PARAM;
      const unsigned old = g_spin_limit.exchange(static_cast<unsigned>(value));
      if (previous) *previous = old;
      return BIWKV_OK;
    }
    case BIWKV_OPT_TWO_PASS:
    case BIWKV_OPT_WIDE_INDEX:
    case BIWKV_OPT_XCD_LOCAL: {
      if (value != 0 && value != 1 && !(option == BIWKV_OPT_TWO_PASS && value == 2)) return BIWKV_ERR_PARAM;
      std::atomic<int>& opt = option == BIWKV_OPT_TWO_PASS    ? g_two_pass
                              : option == BIWKV_OPT_WIDE_INDEX ? g_wide_index
                                                               : g_xcd_local;
      const int old = opt.exchange(static_cast<int>(value));
      if (previous) *previous = old;
      return BIWKV_OK;
    }
    default:
      return BIWKV_ERR_PARAM;
  }
}

int biwkv_version(void) { return 20000; }

}  // extern "C"
