// Host-side state and helpers shared by the translation units of libbiwkv: the per-stream
// scratch, the options, residency queries, and the launch entry points of each unit.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "biwkv.h"
#include "common.h"

namespace biwkv_host {

// BIWKV_ERR_HIP, remembering the raw error for biwkv_last_hip_error.
int hip_fail(hipError_t e);

// The current device (BIWKV_ERR_NO_DEVICE when there is none).
int current_device(int* dev);

// Library-owned scratch of one (device, stream), allocated and grown in stream order.
struct StreamScratch {
  Counters* ctr = nullptr;
  unsigned long long* slots = nullptr;  // single-pass slots, or two-pass chunk totals and carries
  long long slot_words = 0;
  float* bwd = nullptr;  // backward pass sums, carries and per-chunk terms
  long long bwd_floats = 0;
};

// Guards the scratch map and the residency cache; a caller holds it from the scratch lookup until
// its last launch that uses the scratch is queued.
extern std::mutex g_mu;

// Scratch of (device, stream) with at least `words` 64-bit slot words. Caller holds g_mu.
int get_scratch(int dev, void* stream, long long words, StreamScratch** out);

// The stream's backward scratch grown to at least `floats` floats. Caller holds g_mu.
int get_bwd_scratch(int dev, void* stream, long long floats, float** out);

// Workgroups of `kernel` (with `block` threads) that fit on device `dev` at once. Caller holds g_mu.
int resident_capacity(int dev, const void* kernel, int block, int* cap);

// XCDs of device `dev` (workgroups are handed to them round robin). Caller holds g_mu.
int device_xcds(int dev, int* n);

// Compute units of device `dev`. Takes g_mu itself.
int device_cus(int dev, int* n);

// Options (biwkv_set_option).
extern std::atomic<unsigned> g_spin_limit;
extern std::atomic<int> g_two_pass;
extern std::atomic<int> g_wide_index;
extern std::atomic<int> g_xcd_local;

// Scratch that the caller provides instead of the per-stream buffers: a counter block followed by
// `n_words` 64-bit words (the allocation-free entry's static array).
struct FixedScratch {
  Counters* ctr;
  unsigned long long* words;
  long long n_words;
};

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Which tile-kernel entry a forward launch serves.
enum : int { kPlain = 0, kFused = 1, kCausal = 2, kGated = 3 };

// Forward launches of the tile kernel, one translation unit each (parameters already checked,
// nothing empty). fixed: NULL for the per-stream scratch.
int forward_f32(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream, const FixedScratch* fixed);
int forward_bf16(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream, const FixedScratch* fixed);
int forward_bf16_pair(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream,
                      const FixedScratch* fixed);

// dw = du = 0 for a backward call with B * T == 0 (and C > 0).
int backward_empty(float* dw, float* du, int64_t C, void* stream);

// The backward launches (arguments already checked, B * T * C > 0).
int backward(const void* k, const void* v, const float* w, const float* u, const float* g, float* dk, float* dv,
             float* dw, float* du, int64_t B, int64_t T, int64_t C, int dtype, int dev, void* stream);

}  // namespace biwkv_host
