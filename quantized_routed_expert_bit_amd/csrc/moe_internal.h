// Private interface between the C ABI (moe_host.cpp) and the kernels
// (moe_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace qreb {

// Storage format constants (record format in include/moe.h).
constexpr int kGroup = 64;
constexpr int kTileRows = 64;
constexpr int kQ4TileBytes = 2304;     // 2048 code bytes + 64 (scale, bias) fp16 pairs
constexpr int kQ4CodeBytes = 2048;
constexpr int kQ8TileBytes = 4352;     // 4096 code bytes + 256
constexpr int kQ8CodeBytes = 4096;
constexpr int kHeaderBytes = 256;
constexpr uint32_t kMagic = 0x58455251u;
constexpr uint32_t kVersion = 1;

// Router launch geometry: four waves, eight 64-column groups per workgroup
// (two per wave), up to kRouterTokMax tokens per workgroup.
constexpr int kRouterWaves = 4;
constexpr int kRouterGPW = 8;
constexpr int kRouterTokMax = 16;
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;
constexpr int kMaxDevices = 64;
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

// Streaming (GEMV) expert path: up to kGemvTok tokens per pass over the weights.
constexpr int kGemvTok = 16;
constexpr int kGemvTokV2 = 4;   // token rows per streaming pass (register accumulators)
constexpr int kGemvWaves = 4;   // waves per streaming workgroup (they split the K groups)
constexpr int kGemvThreads = 64 * kGemvWaves;

// Matrix-core (MFMA) expert path: rows (tokens) per wide tile, per narrow tile.
constexpr int kMfmaBM = 128;
constexpr int kNarrowBM = 32;
constexpr int kMfmaWaves = 4;
// Wide matrix-core launches: one workgroup per (128-row tile, column block)
// unit; a block is kWideColsUp gate/up columns or kWideColsDn down columns.
constexpr int kWideWaves = 4;
constexpr int kWideColsUp = kWideWaves * 32;
constexpr int kWideColsDn = kWideWaves * 64;
// Entries per XCD of a wide unit list for nt row tiles, nts of them the
// shared expert's, with ncr (routed) and ncs (shared) column blocks: tiles are
// dealt to the 8 XCDs in rounds, so an XCD gets at most ceil(n / 8) of n.
inline int wide_cap(int nt, int nts, int ncr, int ncs) { return (nt + 7) / 8 * ncr + (nts + 7) / 8 * ncs; }

// misc[] slots (int32) in the workspace
enum MiscSlot {
  kNGemv = 1,       // items on the streaming path
  kNMfma = 2,       // items on the matrix-core path
  kNTiles = 3,      // matrix-core row tiles
  kPredValid = 4,   // predicted slots a lookahead left for the next forward (0: none)
  kNNarrow = 5,     // matrix-core narrow (32-row) tiles
  kUnitsUp = 8,     // [8] wide gate/up units listed for each XCD
  kUnitsDn = 16,    // [8] wide down units listed for each XCD
  kMiscInts = 64,
};

// Expert-cache state in the workspace (byte offsets inside its region; every
// array is sized for kMaxExperts, which bounds both E and the slot count).
constexpr int kCacheStats = 16;
constexpr size_t kCacheSlotOf = 0;                                  // int [E]: slot or -1
constexpr size_t kCacheOwner = kCacheSlotOf + 4 * kMaxExperts;      // int [S]: expert or -1
constexpr size_t kCacheFreq = kCacheOwner + 4 * kMaxExperts;        // u32 [E]
constexpr size_t kCacheStamp = kCacheFreq + 4 * kMaxExperts;        // u32 [S]
constexpr size_t kCachePf = kCacheStamp + 4 * kMaxExperts;          // u32 [S]
constexpr size_t kCacheCopyD = kCachePf + 4 * kMaxExperts;          // int [2 E] demand copies
constexpr size_t kCacheCopyP = kCacheCopyD + 8 * kMaxExperts;       // int [2 E] prefetch copies
constexpr size_t kCacheNCopyD = kCacheCopyP + 8 * kMaxExperts;
constexpr size_t kCacheNCopyP = kCacheNCopyD + 4;
constexpr size_t kCacheClock = kCacheNCopyP + 4;
constexpr size_t kCacheStatsOff = kCacheClock + 8;                  // u64 [kCacheStats]
constexpr size_t kCacheBytes = kCacheStatsOff + 8 * kCacheStats;

struct WsLayout {
  size_t part, x16, xs, ids, p, offs, misc,
      slots, items, mitems, ntiles, wunits_up, wunits_dn, pred, hbuf, hs, yslot, xn, cache, total;
  int cap_up, cap_dn;   // entries per XCD of the wide unit lists
};

// All sizes derived from the config; identical on every call.
WsLayout ws_layout(const moe_config& c);
int router_ksplit(int hidden);            // k-splits of the router reduction
int router_tok_block(int n_tokens, int e_pad);   // tokens per router workgroup

struct LayerDev {
  // weights
  const uint8_t* router;
  const float* router_bias;
  const uint8_t* bank;      // the records the kernels read: the bank, or the cache's slots
  uint64_t stride;
  const uint8_t* shared;
  const int* slot_of;       // with an expert cache: expert -> slot (in the workspace), else NULL
  // expert cache: where missing records are copied from, slot count, bytes per copy
  const uint8_t* cache_src;
  uint64_t cache_src_stride;
  int cache_slots;
  uint64_t rec_bytes;
  // shape
  int H, E, Epad, k, I, Is, has_shared, rmsnorm, max_tokens;
  int mfma_min_rows;   // rows at which an expert leaves the streaming path
  int wide_min_rows;   // rows at which it uses 128-row instead of 32-row tiles
  int narrow_cs_min_wgs;   // 32-row tiles split columns, not K, from this many workgroups
  int n_cu;            // compute units of the device
  // workspace
  uint8_t* ws;
  WsLayout L;
};

// Router (+ top-k + bucketing).  mode: 0 forward, 1 logits only, 2 lookahead
// prediction into the context's own pred[] buffer.
hipError_t launch_router(const LayerDev& d, const void* x, int x_f32, int T, int mode,
                         float* logits_out, int32_t* ids_out, float* p_out,
                         hipStream_t s);
// The streaming launches also run the narrow (32-row) matrix-core tiles.
hipError_t launch_gemv_up(const LayerDev& d, int T, hipStream_t s);
hipError_t launch_gemv_down(const LayerDev& d, int T, hipStream_t s);
bool mfma_needed(const LayerDev& d, int T);
hipError_t launch_mfma_up(const LayerDev& d, int T, hipStream_t s);
hipError_t launch_mfma_down(const LayerDev& d, int T, hipStream_t s);
hipError_t launch_combine(const LayerDev& d, int T, const float* p, const float* residual, float* y,
                          hipStream_t s);
hipError_t launch_ws_init(const LayerDev& d, hipStream_t s);
hipError_t launch_rmsnorm(const LayerDev& d, const void* x, int x_f32, int T, hipStream_t s);
hipError_t launch_debug_dequant(const void* tiles, int bits, int rows, int cols, float* out,
                                hipStream_t s);
// Expert cache: plan (mode 0 demand from the bucketing, 1 prefetch from the
// npred predicted ids), fill (at most max_copies records), reset.
// mode 0: this forward's experts; 1: prefetch of the first `top` (0: all k)
// predicted experts of each token
hipError_t launch_cache_plan(const LayerDev& d, int mode, int npred, int top, hipStream_t s);
hipError_t launch_cache_fill(const LayerDev& d, int mode, int max_copies, hipStream_t s);
hipError_t launch_cache_reset(const LayerDev& d, hipStream_t s);
// CRC-32 (zlib's) of n byte ranges base + r * stride + off, len bytes each
// (base 16-byte aligned, stride and off multiples of 16), into host_out[r];
// dev_tmp holds tmp_words partial results.  Synchronizes the stream.
hipError_t crc32_ranges(const uint8_t* base, uint64_t stride, uint64_t off, uint64_t len, int n,
                        uint32_t* dev_tmp, size_t tmp_words, uint32_t* host_out, hipStream_t s);
// 3-bit residual-VQ products (moe_rvq.hip): workspace bytes, and the
// tables -> lookups -> slice reduction sequence.
size_t rvq_workspace(int T, int K, int R, int n_mats);
hipError_t launch_rvq_gemv(const void* x, int x_f32, int T, int K, const uint8_t* mats,
                           uint64_t mat_stride, int n_mats, int R, const uint16_t* cb, float* y,
                           uint8_t* ws, hipStream_t s);
// Device address of the library's static scratch array (kNoallocScratchBytes)
// on `device`, which must be the current device; looked up once per device.
hipError_t noalloc_scratch(int device, uint8_t** out);

}  // namespace qreb
