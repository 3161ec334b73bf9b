// 3-bit residual-VQ matrices (gfx950): the expert codec of the WASTE page
// ("Kimi K3'ü 29 GB RAM'de ...", section "Quantization ve doğruluk").  Every
// run of 8 consecutive weights of a row is the sum of one entry from each of
// three 256-entry codebooks of 8-vectors: three 8-bit indices per 8 weights,
// 3.00 bits per weight.  The product never rebuilds the matrix: per input row
// x_t, partial inner-product tables
//     tab_t[j][s][c] = <C_s[c], x_t[8j .. 8j+7]>
// are built in LDS by every workgroup for the 64 columns it is working on,
// and a row's output is the sum over its runs j of three table lookups,
// tab_t[j][0][i0] + tab_t[j][1][i1] + tab_t[j][2][i2] (rvq_gemv_kernel):
// three lookups and two additions per run of 8 weights, as the page counts
// them.  Tables are fp32 and every sum
// fp32; the K groups' partial sums are added in group order
// (rvq_reduce_kernel).
//
// Layout (normative text in include/moe.h): a matrix of R rows by K columns
// (multiples of 64) is (R/64) * (K/64) tiles of 1536 bytes in row-block-major
// order; byte s*512 + r*8 + j of a tile is the stage-s index of row r's run j.
// One wave64 load of 8 bytes per lane reads one stage's indices of 64 rows'
// 8 runs (512 contiguous bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "moe_internal.h"

namespace qreb {

constexpr int kRvqTileBytes = 1536;
constexpr int kRvqThreads = 1024;
constexpr int kRvqRowsPerThread = 4;
constexpr int kRvqRows = kRvqThreads * kRvqRowsPerThread;   // rows per workgroup
constexpr int kRvqTokMax = 4;      // tokens per pass (one tile's tables: 24 KiB per token)
// 64-column tiles per K group of a workgroup: chosen per shape in this range
constexpr int kRvqTilesMin = 4;
constexpr int kRvqTilesMax = 8;

__device__ __forceinline__ float rvq_f16(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// The TP tokens' table values of one entry, read as one 4-, 8- or 16-byte LDS load.
template <int TP> struct RvqVec;
template <> struct RvqVec<1> {
  using type = float;
  __device__ static float at(float v, int) { return v; }
};
template <> struct RvqVec<2> {
  using type = float2;
  __device__ static float at(float2 v, int i) { return i ? v.y : v.x; }
};
template <> struct RvqVec<4> {
  using type = float4;
  __device__ static float at(float4 v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
};

// Workgroup = (K group kg of up to tpg tiles, matrix m, block
// rb of kRvqRows rows), for the TP tokens t0 .. t0+TP-1 (TP = 1, 2 or 4).
// Per tile the workgroup builds the tile's tables in LDS, laid out
// [run j][stage s][entry c][token], so that the TP tokens' values of one
// entry are adjacent: thread tid owns codebook entry c = tid % 256 of all
// three stages (in registers) and the runs tid / 256 and tid / 256 + 4 of
// the tile.  Each thread then adds, for its kRvqRowsPerThread rows, three
// lookups per run, each one 4-, 8- or 16-byte LDS read serving every token
// of the pass, with the row's indices loaded once per tile; after the
// group's last tile it writes the partial outputs part[kg][m][t][r].  Work
// items are numbered K-group major and dealt to the eight XCDs in contiguous
// ranges (workgroup b runs on XCD b mod 8).
template <int TP>
__global__ __launch_bounds__(kRvqThreads) void rvq_gemv_kernel(
    const uint8_t* __restrict__ mats, uint64_t mat_stride, int R, int K, int T, int t0,
    const void* __restrict__ x, int x_f32, const uint16_t* __restrict__ cb,
    float* __restrict__ part, int n_rb, int n_mats, int n_work, int per_xcd, int tpg) {
  extern __shared__ float4 lt4[];   // [8 runs][3][256][TP] tables, then [TP][group columns] x
  float* lt = reinterpret_cast<float*>(lt4);
  const int w = (int)(blockIdx.x & 7u) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= n_work) return;
  const int kg = w / (n_mats * n_rb), mr = w % (n_mats * n_rb);
  const int m = mr / n_rb, rb = mr % n_rb;
  const int tid = threadIdx.x;
  const int G = K / 64;
  const int g0 = kg * tpg, g1 = min(G, g0 + tpg);
  const int ncol = (g1 - g0) * 64;
  float* xs = lt + TP * 8 * 768;   // [TP][ncol]
  for (int i = tid; i < TP * ncol; i += kRvqThreads) {
    // a pass of 4 may carry 3 tokens (a fourth pass slot of zeros, not written)
    if (t0 + i / ncol >= T) {
      xs[i] = 0.f;
      continue;
    }
    const size_t src = (size_t)(t0 + i / ncol) * K + (size_t)g0 * 64 + i % ncol;
    xs[i] = x_f32 ? static_cast<const float*>(x)[src]
                  : __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(x)[src] << 16);
  }
  // codebook entry c of the three stages
  const int c = tid & 255, jq = tid >> 8;
  float e[3][8];
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const uint4 v = *reinterpret_cast<const uint4*>(cb + ((size_t)st * 256 + c) * 8);
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      e[st][2 * d] = rvq_f16((uint16_t)(wd[d] & 0xffffu));
      e[st][2 * d + 1] = rvq_f16((uint16_t)(wd[d] >> 16));
    }
  }
  // the thread's rows' index bytes in tile g0 (rows past R read row 0's and
  // are not written); the next tile of a row is kRvqTileBytes further
  const uint8_t* src[kRvqRowsPerThread];
#pragma unroll
  for (int q = 0; q < kRvqRowsPerThread; ++q) {
    int r = rb * kRvqRows + q * kRvqThreads + tid;
    r = r < R ? r : 0;
    src[q] = mats + (size_t)m * mat_stride + ((size_t)(r >> 6) * G + g0) * kRvqTileBytes + (r & 63) * 8;
  }
  float acc[kRvqRowsPerThread][TP];
#pragma unroll
  for (int q = 0; q < kRvqRowsPerThread; ++q)
#pragma unroll
    for (int tt = 0; tt < TP; ++tt) acc[q][tt] = 0.f;
  for (int g = g0; g < g1; ++g) {
    uint64_t ix[kRvqRowsPerThread][3];
#pragma unroll
    for (int q = 0; q < kRvqRowsPerThread; ++q) {
#pragma unroll
      for (int st = 0; st < 3; ++st)
        ix[q][st] = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(src[q] + st * 512));
      src[q] += kRvqTileBytes;
    }
    // x staged (first tile) or the previous tile's lookups done
    __syncthreads();
    // tab[tt][j][st][c] = <C_st[c], x_tt[8j .. 8j+7]> for this tile's runs j
#pragma unroll
    for (int tt = 0; tt < TP; ++tt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = jq + 4 * h;
        const float* xr = xs + tt * ncol + (g - g0) * 64 + j * 8;
        const float4 xa = *reinterpret_cast<const float4*>(xr);
        const float4 xb = *reinterpret_cast<const float4*>(xr + 4);
        const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int st = 0; st < 3; ++st) {
          float d = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) d = fmaf(e[st][k], xv[k], d);
          lt[(((j * 3 + st) * 256) + c) * TP + tt] = d;
        }
      }
    }
    __syncthreads();
    // row by row: one row's 24 table offsets serve every token; the TP
    // tokens' values of an entry are adjacent, so each lookup is one LDS read
    using VT = typename RvqVec<TP>::type;
    const VT* tv = reinterpret_cast<const VT*>(lt);
#pragma unroll
    for (int q = 0; q < kRvqRowsPerThread; ++q) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const VT* row = tv + jj * 768;
        const uint32_t a = (uint32_t)(ix[q][0] >> (8 * jj)) & 0xffu;
        const uint32_t b = (uint32_t)(ix[q][1] >> (8 * jj)) & 0xffu;
        const uint32_t cc = (uint32_t)(ix[q][2] >> (8 * jj)) & 0xffu;
        const VT va = row[a], vb = row[256 + b], vc = row[512 + cc];
#pragma unroll
        for (int tt = 0; tt < TP; ++tt)
          acc[q][tt] += (RvqVec<TP>::at(va, tt) + RvqVec<TP>::at(vb, tt)) + RvqVec<TP>::at(vc, tt);
      }
      // keeps the scheduler from hoisting every row's lookups at once
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int tt = 0; tt < TP; ++tt) {
#pragma unroll
    for (int q = 0; q < kRvqRowsPerThread; ++q) {
      const int r = rb * kRvqRows + q * kRvqThreads + tid;
      if (r < R && t0 + tt < T) part[(((size_t)kg * n_mats + m) * T + t0 + tt) * R + r] = acc[q][tt];
    }
  }
}

// y[m][t][r] = sum over the K groups of part[kg][m][t][r], in group order;
// one output per thread, eight groups' loads in flight at a time.
__global__ __launch_bounds__(256) void rvq_reduce_kernel(const float* __restrict__ part, int KG,
                                                         size_t n, float* __restrict__ y) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  int kg = 0;
  for (; kg + 8 <= KG; kg += 8) {
    float p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = part[(size_t)(kg + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += p[u];
  }
  for (; kg < KG; ++kg) v += part[(size_t)kg * n + i];
  y[i] = v;
}

static size_t rvq_al(size_t v) { return (v + 255) & ~size_t(255); }

static int rvq_groups(int K, int tpg) {
  const int G = K / 64;
  return (G + tpg - 1) / tpg;
}

// Tiles per K group: the workgroups (one per CU at a time: 16 waves of 84 or
// more registers) run in ceil(work / CUs) rounds of a time proportional to
// the group's tiles, so the size with the fewest rounds x tiles is taken, the
// larger on a tie (fewer partial sums to add).  16 matrices of 4096 x 7168 on
// 256 CUs: 7 tiles, one round of 256 workgroups (one token 58 -> 48 us against
// 4 tiles, 448 workgroups in two rounds).
static int rvq_tiles_per_group(int K, int n_mats, int n_rb, int n_cu) {
  int best = kRvqTilesMin;
  long best_cost = -1;
  for (int tpg = kRvqTilesMin; tpg <= kRvqTilesMax; ++tpg) {
    const long work = (long)rvq_groups(K, tpg) * n_mats * n_rb;
    const long cost = (work + n_cu - 1) / n_cu * tpg;
    if (best_cost < 0 || cost <= best_cost) {
      best = tpg;
      best_cost = cost;
    }
  }
  return best;
}

size_t rvq_workspace(int T, int K, int R, int n_mats) {
  // launch limits: at most 2^20 workgroups and 2^31 outputs; partial sums
  // for the most K groups (the smallest group size)
  const uint64_t n_rb = ((uint64_t)R + kRvqRows - 1) / kRvqRows;
  if ((uint64_t)rvq_groups(K, kRvqTilesMin) * (uint64_t)n_mats * n_rb > (1u << 20) ||
      (uint64_t)n_mats * (uint64_t)T * (uint64_t)R > (1ull << 31))
    return 0;
  return rvq_al((size_t)rvq_groups(K, kRvqTilesMin) * n_mats * T * R * 4);
}

hipError_t launch_rvq_gemv(const void* x, int x_f32, int T, int K, const uint8_t* mats,
                           uint64_t mat_stride, int n_mats, int R, const uint16_t* cb, float* y,
                           uint8_t* ws, hipStream_t s) {
  // the LDS limit of the 2- and 4-token kernels and the CU count, once per
  // device
  hipError_t e;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static int n_cus[kMaxDevices] = {};
  int n_cu;
  {
    static std::mutex mu;
    static bool lds_set[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!lds_set[dev]) {
      int v = 0;
      e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      if (v < 1) return hipErrorInvalidDevice;
      n_cus[dev] = v;
      const void* fns[3] = {reinterpret_cast<const void*>(rvq_gemv_kernel<1>),
                            reinterpret_cast<const void*>(rvq_gemv_kernel<2>),
                            reinterpret_cast<const void*>(rvq_gemv_kernel<4>)};
      for (int i = 0; i < 3; ++i) {
        e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                (1 << i) * (8 * 768 + kRvqTilesMax * 64) * 4);
        if (e != hipSuccess) return e;
      }
      lds_set[dev] = true;
    }
    n_cu = n_cus[dev];
  }
  float* part = reinterpret_cast<float*>(ws);
  const int n_rb = (R + kRvqRows - 1) / kRvqRows;
  const int tpg = rvq_tiles_per_group(K, n_mats, n_rb, n_cu);
  const int KG = rvq_groups(K, tpg);
  const int n_work = KG * n_mats * n_rb, per_xcd = (n_work + 7) / 8;
  const int ncol = (K / 64 < tpg ? K / 64 : tpg) * 64;
  // passes of 4, 2 or 1 tokens; each holds TP x (24 KiB of tables + the
  // group's x) in LDS
  for (int t0 = 0; t0 < T;) {
    // passes of 4 tokens (3 remaining run as a pass of 4: one 4-token pass
    // costs less than passes of 2 and 1), then 2, then 1
    const int tp = T - t0 >= 3 ? 4 : T - t0 >= 2 ? 2 : 1;
    const size_t lds = (size_t)tp * (8 * 768 + ncol) * 4;
    const dim3 grid(per_xcd * 8), block(kRvqThreads);
    if (tp == 1)
      hipLaunchKernelGGL(rvq_gemv_kernel<1>, grid, block, lds, s, mats, mat_stride, R, K, T, t0, x,
                         x_f32, cb, part, n_rb, n_mats, n_work, per_xcd, tpg);
    else if (tp == 2)
      hipLaunchKernelGGL(rvq_gemv_kernel<2>, grid, block, lds, s, mats, mat_stride, R, K, T, t0, x,
                         x_f32, cb, part, n_rb, n_mats, n_work, per_xcd, tpg);
    else
      hipLaunchKernelGGL(rvq_gemv_kernel<4>, grid, block, lds, s, mats, mat_stride, R, K, T, t0, x,
                         x_f32, cb, part, n_rb, n_mats, n_work, per_xcd, tpg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    t0 += tp;   // (may pass T: the last pass of 4 carried 3 tokens)
  }
  const size_t n = (size_t)n_mats * T * R;
  hipLaunchKernelGGL(rvq_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, KG, n, y);
  return hipGetLastError();
}

}  // namespace qreb
