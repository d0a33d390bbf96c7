// libbiwkv translation unit: the Bi-WKV backward launches.
#include "backward.h"
#include "bwd_tile.h"
#include "host.h"

namespace biwkv_host {

namespace {

// Backward tile shape of the multi-launch form: 8 tokens per lane, 512 threads (two workgroups
// per CU, so one's loads overlap the other's arithmetic), 64-token chunks.
constexpr int kBwdL = 8;
constexpr int kBwdNT = 512;
// The single launch: 16 tokens per lane (k and v in registers, nothing else per token), 512
// threads, 128-token chunks.
constexpr int kOneL = 16;
constexpr int kOneNT = 512;
constexpr int kNotTaken = -1000;  // launch_bwd_one: the shape takes the multi-launch form

// The dw / du fold of every backward call.
int launch_reduce(const float* w, float* dw, float* du, int64_t B, int64_t T, int64_t C, int64_t n_chunks,
                  float* pw, float* pu, hipStream_t st) {
  BwdParams rp{};
  rp.w = w;
  rp.dw = dw;
  rp.du = du;
  rp.T = T;
  rp.B = static_cast<int>(B);
  rp.C = static_cast<int>(C);
  rp.n_chunks = static_cast<int>(n_chunks);
  rp.n_wg = static_cast<int>(n_chunks);
  rp.s.pw = pw;
  rp.s.pu = pu;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>((C + 63) / 64)), dim3(64 * kReduceGroups), 0,
                     st, rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

// The backward in one launch (bwd_one_kernel), then bwd_one_reduce_kernel: the rows whose waits
// ran out again, and the dw / du fold. kNotTaken when a row's chunks could not all be resident at once (the
// multi-launch form then serves the call), or when BIWKV_OPT_TWO_PASS asks for that form.
template <int DT, bool PAIR>
int launch_bwd_one(const void* k, const void* v, const float* w, const float* u, const float* g, float* dk,
                   float* dv, float* dw, float* du, int64_t B, int64_t T, int64_t C, int dev, void* stream) {
  constexpr int L = kOneL, NT = kOneNT, CT = (NT / kBtTile) * L;
  if (g_two_pass.load() == 1) return kNotTaken;
  const int64_t n_tiles = (C + kBtTile - 1) / kBtTile;
  const int64_t n_chunks = (T + CT - 1) / CT;
  const int64_t rows = B * n_tiles;
  const int64_t total = rows * n_chunks;
  if (total > 0x7FFFFFFFll) return kNotTaken;
  // 32-bit byte offsets inside a batch item of g (and the row's padding)
  if ((T + CT) * C * 4 >= (1ll << 31)) return kNotTaken;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* kfn = reinterpret_cast<const void*>(&bwd_one_kernel<DT, L, NT, PAIR>);
  std::lock_guard<std::mutex> lock(g_mu);
  int cap = 0;
  int rc = resident_capacity(dev, kfn, NT, &cap);
  if (rc) return rc;
  // a row's chunks wait only for each other; at most a quarter of the resident workgroups per row
  // (the rule of the forward tile kernel's single pass)
  if (n_chunks > 1 && n_chunks > cap / 4) return kNotTaken;
  BwdTileParams tp{};
  const long long terms = B * n_chunks * C;                          // dw, du terms
  const long long sums = n_chunks > 1 ? total * 2 * kBtTile * 3 : 0;  // fallback: chunk sums per round
  const long long flags = n_chunks > 1 ? rows : 0;
  float* scr = nullptr;
  rc = get_bwd_scratch(dev, stream, 2 * terms + 4 * sums + flags, &scr);
  if (rc) return rc;
  tp.pw = scr;
  tp.pu = scr + terms;
  tp.sums1 = scr + 2 * terms;
  tp.sums2 = tp.sums1 + sums;
  tp.carry1 = tp.sums2 + sums;
  tp.carry2 = tp.carry1 + sums;
  tp.row_fail = reinterpret_cast<unsigned*>(tp.carry2 + sums);
  if (n_chunks > 1) {
    // two rounds of three tagged words per (chunk, direction, channel)
    const long long words = 2 * total * 2 * kBtTile * 3;
    StreamScratch* sc = nullptr;
    rc = get_scratch(dev, stream, words, &sc);
    if (rc) return rc;
    tp.ctr = sc->ctr;
    tp.slots = sc->slots;
    // a row kept on one XCD needs all its chunks resident there, on 1 / nx of the device; its slots
    // are addressed with 32-bit byte offsets
    if (g_xcd_local.load() && words * 8 < 0xFFFFFFFFll) {
      int nx = 1;
      rc = device_xcds(dev, &nx);
      if (rc) return rc;
      if (nx > 1 && n_chunks <= cap / nx) {
        tp.n_xcd = nx;
        tp.xcd_rows = static_cast<int>(rows / nx * nx);
      }
    }
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
  tp.total = static_cast<unsigned>(total);
  tp.spin_limit = g_spin_limit.load();
  hipLaunchKernelGGL((bwd_one_kernel<DT, L, NT, PAIR>), dim3(static_cast<unsigned>(total)), dim3(NT), 0, st, tp);
  // rows whose waits ran out again (in plain row order), then dw and du
  BwdTileParams fp = tp;
  fp.xcd_rows = 0;
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
  hipLaunchKernelGGL((bwd_one_reduce_kernel<DT, L, NT, PAIR>), dim3(static_cast<unsigned>(n_tiles)), dim3(NT), 0, st,
                     fp, rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return BIWKV_OK;
}

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
  // The launches of one call share the stream's scratch: the lock is held until the last one is
  // queued, so calls from several host threads on one stream cannot interleave their stages.
  std::lock_guard<std::mutex> lock(g_mu);
  const long long terms = B * n_chunks * C;                         // dw, du terms
  const long long sums = n_chunks > 1 ? total * 2 * kBtTile * 3 : 0;  // chunk sums per round
  float* scr = nullptr;
  int rc = get_bwd_scratch(dev, stream, 2 * terms + 4 * sums, &scr);
  if (rc) return rc;
  tp.pw = scr;
  tp.pu = scr + terms;
  tp.sums1 = scr + 2 * terms;
  tp.sums2 = tp.sums1 + sums;
  tp.carry1 = tp.sums2 + sums;
  tp.carry2 = tp.carry1 + sums;
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return launch_reduce(w, dw, du, B, T, C, n_chunks, tp.pw, tp.pu, st);
}

}  // namespace

int backward_empty(float* dw, float* du, int64_t C, void* stream) {
  const unsigned cb = static_cast<unsigned>((C + 255) / 256);
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(cb), dim3(256), 0, static_cast<hipStream_t>(stream), dw, du,
                     static_cast<int>(C));
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? BIWKV_OK : hip_fail(e);
}

int backward(const void* k, const void* v, const float* w, const float* u, const float* g, float* dk, float* dv,
             float* dw, float* du, int64_t B, int64_t T, int64_t C, int dtype, int dev, void* stream) {
  // rows longer than one 64-token chunk: one launch when the row's chunks fit on the device
  if (T > static_cast<int64_t>(kBwdL) * (kBwdNT / kBtTile)) {
    int rc = kNotTaken;
    if (dtype == BIWKV_F32)
      rc = launch_bwd_one<BIWKV_F32, false>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
    else if (C % 2 == 0 && aligned(k, 4) && aligned(v, 4))
      rc = launch_bwd_one<BIWKV_BF16, true>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
    else
      rc = launch_bwd_one<BIWKV_BF16, false>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
    if (rc != kNotTaken) return rc;
  }
  if (dtype == BIWKV_F32)
    return launch_bwd_tile<BIWKV_F32, kBwdL, kBwdNT, 4, false>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
  // bf16 k and v load as 32-bit channel pairs when every pair is whole and aligned
  if (C % 2 == 0 && aligned(k, 4) && aligned(v, 4))
    return launch_bwd_tile<BIWKV_BF16, kBwdL, kBwdNT, 4, true>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
  return launch_bwd_tile<BIWKV_BF16, kBwdL, kBwdNT, 4, false>(k, v, w, u, g, dk, dv, dw, du, B, T, C, dev, stream);
}

}  // namespace biwkv_host
