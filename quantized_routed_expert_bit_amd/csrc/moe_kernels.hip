// HIP kernels (gfx950) of the routed-expert MoE layer.
//
// Layer definition and sources: include/moe.h.  Summary of the kernels:
//   router_kernel   8-bit router GEMV -> fp32 partial logits per k-split; the
//                   last workgroup of each token block sums them, adds the
//                   logit bias and selects top-k with wave64 shuffles, then the
//                   last token block buckets the (token, rank) slots by expert
//                   and writes the work lists (one launch, no spinning).
//   gemv_up_kernel  streaming expert path, gate and up: one lane per weight
//                   row, 16-byte coalesced tile loads, nibbles unpacked in
//                   registers, x read through the scalar cache; writes
//                   h = SiLU(g) * u in fp16 and its per-64 group sums.
//   gemv_down_kernel  the same for the down matrix; writes one fp32 row per
//                   (token, expert) slot.
//   combine_kernel  y[t] = sum_j p[t,j] y_slot[t,j] + y_shared[t] in fixed order.
//
// Dot products use v_dot2_f32_f16 on codes lifted to fp16 with the exponent
// trick: (q | 0x6400) is the fp16 value 1024 + q exactly (q < 1024), so
//     sum_k x_k (s q_k + b) = s * sum_k x_k (1024 + q_k) + (b - 1024 s) * sum_k x_k
// with fp32 accumulation; the group sums sum_k x_k come from the same fp16
// values that enter the dot products.
#include "moe_internal.h"

#include <math.h>

namespace qreb {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}
__device__ __forceinline__ float f16f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f16bits(_Float16 v) { return __builtin_bit_cast(uint16_t, v); }
__device__ __forceinline__ float bf16f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Pointers into memory no kernel writes during the launch that reads it; with
// a wave-uniform address a load through this address space is a scalar load.
typedef const __attribute__((address_space(4))) uint32_t* cu32p;
typedef const __attribute__((address_space(4))) float* cf32p;
__device__ __forceinline__ cu32p as_const(const uint32_t* p) { return (cu32p)(uintptr_t)p; }
__device__ __forceinline__ cf32p as_const(const float* p) { return (cf32p)(uintptr_t)p; }

// Code lifting.  gfx9 VOP3 cannot encode a literal, so the mask goes in an
// SGPR and the exponent pattern 0x6400 0x6400 in a VGPR: one v_and_or_b32 per
// fp16 pair (plus one shift for all but the first pair of a dword).
struct Lift {
  uint32_t magic;
  __device__ __forceinline__ Lift() { asm("v_mov_b32 %0, 0x64006400" : "=v"(magic)); }
  // 4-bit: dword holds columns 8d..8d+7 (nibble i = column 8d+i); pair p is
  // the fp16 pair (1024 + q[8d+p], 1024 + q[8d+p+4]).
  __device__ __forceinline__ uint32_t q4(uint32_t w, int p) const {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w >> (4 * p)), "s"(0x000F000Fu), "v"(magic));
    return r;
  }
  // 8-bit: dword holds columns 4d..4d+3; pair p = (1024 + q[4d+p], 1024 + q[4d+p+2]).
  __device__ __forceinline__ uint32_t q8(uint32_t w, int p) const {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w >> (8 * p)), "s"(0x00FF00FFu), "v"(magic));
    return r;
  }
};
// Position of column c (within a 64-column group) in the paired fp16 order the
// 4-bit and 8-bit dot products consume.
__device__ __forceinline__ int pair_pos4(int c) { return (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1); }
__device__ __forceinline__ int pair_pos8(int c) { return (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1); }

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

// Unpack one 16-byte 4-bit piece (32 columns) into 16 fp16 pairs.
__device__ __forceinline__ void unpack16_q4(const Lift& L, uint4 c, uint32_t* w) {
  const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) w[i * 4 + p] = L.q4(d[i], p);
}

// Deterministic wave64 sum: every lane ends with the value lane 0 computes.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return __shfl(v, 0);
}

// Exclusive scan of n ints held in LDS (n <= 256 * 8), by a 256-thread block.
// Returns the total.  All threads must call it.
__device__ int block_excl_scan(int* data, int n, int* scratch256) {
  const int tid = threadIdx.x;
  const int per = (n + 255) / 256;
  const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += data[i];
  scratch256[tid] = s;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int v = tid >= off ? scratch256[tid - off] : 0;
    __syncthreads();
    scratch256[tid] += v;
    __syncthreads();
  }
  int run = scratch256[tid] - s;  // exclusive prefix of this thread's chunk
  const int total = scratch256[255];
  for (int i = b0; i < b1; ++i) {
    int v = data[i];
    data[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// ------------------------------------------------------------------ router --

struct RouterArgs {
  const uint8_t* router;
  const float* bias;
  const void* x;
  int x_f32, T, H, G, E, Epad, k, KS, TBR, n_tb, n_rb, mode, write_x;
  float* part;
  uint16_t* x16;
  uint16_t* x16lo;
  float* xs;
  int* cnt_tb;
  int* misc;
  int* counts;
  int* rank;
  int* ids_ws;
  float* p_ws;
  int32_t* ids_out;
  float* p_out;
  float* logits_out;
  int* pred;
  int* offs;
  int* slots;
  int4* items;
  int4* mitems;
  int2* mtiles;
  int mfma_min_rows, has_shared;
};

// Runs in the single workgroup that finishes last: counts -> offsets -> slot
// lists grouped by expert -> work lists.  Resets every counter it consumed.
__device__ void bucket_final(const RouterArgs& a) {
  __shared__ int s_cnt[kMaxExperts + 2];
  __shared__ int s_off[kMaxExperts + 2];
  __shared__ int s_flag[kMaxExperts + 2];
  __shared__ unsigned char s_pred[kMaxExperts];
  __shared__ int s_scan[256];
  __shared__ int s_tot[4];
  const int tid = threadIdx.x;
  const int E = a.E, Tk = a.T * a.k;
  const int R = a.mfma_min_rows;
  for (int e = tid; e < E; e += 256) {
    int c = atomicExch(&a.counts[e], 0);
    s_cnt[e] = c;
    s_off[e] = c;
    s_pred[e] = 0;
  }
  const int pv = a.misc[kPredValid];
  __syncthreads();
  block_excl_scan(s_off, E, s_scan);
  for (int e = tid; e < E; e += 256) a.offs[e] = s_off[e];
  if (tid == 0) a.offs[E] = Tk;
  for (int s = tid; s < Tk; s += 256) {
    const int e = a.ids_ws[s];
    a.slots[s_off[e] + a.rank[s]] = s;
  }
  if (a.has_shared)
    for (int t = tid; t < a.T; t += 256) a.slots[Tk + t] = Tk + t;
  for (int s = tid; s < pv; s += 256) {
    const int e = a.pred[s];
    if (e >= 0 && e < E) s_pred[e] = 1;
  }
  __syncthreads();
  // Work lists: streaming (0 < rows < R) and matrix-core (rows >= R).  With a
  // lookahead prediction, predicted experts come first; order never changes a
  // result, only when an expert's weights are streamed.
  for (int path = 0; path < 2; ++path) {
    int base = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int e = tid; e < E; e += 256) {
        const int c = s_cnt[e];
        const bool on = path == 0 ? (c > 0 && c < R) : (c >= R);
        const bool first = pv ? s_pred[e] != 0 : true;
        s_flag[e] = on && (pass == 0 ? first : !first) ? 1 : 0;
      }
      __syncthreads();
      // flags -> positions (scan keeps the flag in s_scan-derived order)
      for (int e = tid; e < E; e += 256) s_off[e] = s_flag[e];
      __syncthreads();
      const int n = block_excl_scan(s_off, E, s_scan);
      for (int e = tid; e < E; e += 256)
        if (s_flag[e]) {
          int4 it;
          it.x = e;
          it.y = s_cnt[e];
          it.z = 0;  // list offset filled below
          it.w = 0;
          (path == 0 ? a.items : a.mitems)[base + s_off[e]] = it;
        }
      base += n;
      __syncthreads();
      if (!pv) break;
    }
    if (tid == 0) s_tot[path] = base;
    __syncthreads();
  }
  // list offsets (exclusive scan of counts, recomputed) for each item
  for (int e = tid; e < E; e += 256) s_off[e] = s_cnt[e];
  __syncthreads();
  block_excl_scan(s_off, E, s_scan);
  int n_gemv = s_tot[0], n_mfma = s_tot[1];
  for (int i = tid; i < n_gemv; i += 256) a.items[i].z = s_off[a.items[i].x];
  for (int i = tid; i < n_mfma; i += 256) a.mitems[i].z = s_off[a.mitems[i].x];
  __syncthreads();
  if (tid == 0 && a.has_shared) {
    int4 it;
    it.x = E;
    it.y = a.T;
    it.z = Tk;
    it.w = 0;
    if (a.T >= R) a.mitems[n_mfma++] = it;
    else a.items[n_gemv++] = it;
  }
  __syncthreads();
  if (tid == 0) s_tot[2] = n_mfma;
  __syncthreads();
  n_mfma = s_tot[2];
  // matrix-core row tiles: (item, first row)
  for (int i = tid; i < n_mfma; i += 256) s_flag[i] = (a.mitems[i].y + kMfmaBM - 1) / kMfmaBM;
  __syncthreads();
  for (int i = tid; i < n_mfma; i += 256) s_off[i] = s_flag[i];
  __syncthreads();
  const int n_tiles = block_excl_scan(s_off, n_mfma, s_scan);
  for (int i = tid; i < n_mfma; i += 256)
    for (int j = 0; j < s_flag[i]; ++j) a.mtiles[s_off[i] + j] = make_int2(i, j * kMfmaBM);
  if (tid == 0) {
    a.misc[kNGemv] = n_gemv;
    a.misc[kNMfma] = n_mfma;
    a.misc[kNTiles] = n_tiles;
    a.misc[kPredValid] = 0;
    a.misc[kCntAll] = 0;
  }
}

__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  __shared__ uint16_t xr[kRouterTokMax][kRouterWaves][64];
  __shared__ uint16_t xrl[kRouterTokMax][kRouterWaves][64];
  __shared__ float xsum[kRouterTokMax][kRouterWaves];
  __shared__ float red[kRouterWaves][kRouterTokMax][64];
  __shared__ int flag;

  const int rb = blockIdx.x, ks = blockIdx.y, tb = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = tb * a.TBR;
  const int nt = min(a.TBR, a.T - t0);
  const int g0 = ks * kRouterWaves;
  const int ng = min(kRouterWaves, a.G - g0);
  const bool wx = a.write_x && rb == 0;

  // 1. x -> fp16 hi (+ lo for fp32 input) in the 8-bit pair order; the rb == 0
  //    workgroups also publish it in the 4-bit pair order for the experts.
  for (int i = tid; i < nt * ng * 64; i += 256) {
    const int t = i / (ng * 64), r = i - t * (ng * 64), gl = r >> 6, c = r & 63;
    const size_t src = (size_t)(t0 + t) * a.H + (size_t)(g0 + gl) * 64 + c;
    const float v = a.x_f32 ? static_cast<const float*>(a.x)[src]
                            : bf16f(static_cast<const uint16_t*>(a.x)[src]);
    const _Float16 hi = (_Float16)v;
    const _Float16 lo = (_Float16)(v - (float)hi);
    xr[t][gl][pair_pos8(c)] = f16bits(hi);
    xrl[t][gl][pair_pos8(c)] = f16bits(lo);
    if (wx) {
      const size_t dst = (size_t)(t0 + t) * a.H + (size_t)(g0 + gl) * 64 + pair_pos4(c);
      a.x16[dst] = f16bits(hi);
      if (a.x_f32) a.x16lo[dst] = f16bits(lo);
    }
  }
  __syncthreads();
  if (tid < nt * ng) {
    const int t = tid / ng, gl = tid - t * ng;
    float s = 0.f;
    for (int c = 0; c < 64; ++c) s += f16f(xr[t][gl][c]) + f16f(xrl[t][gl][c]);
    xsum[t][gl] = s;
    if (wx) a.xs[(size_t)(t0 + t) * a.G + g0 + gl] = s;
  }
  __syncthreads();

  // 2. one wave per group: lane = expert row
  if (wave < ng) {
    const uint8_t* tile = a.router + ((size_t)rb * a.G + g0 + wave) * kQ8TileBytes;
    const Lift L;
    uint32_t w[32];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint4 c = ld16(tile + cc * 1024 + lane * 16);
      const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int dw = 0; dw < 4; ++dw)
#pragma unroll
        for (int p = 0; p < 2; ++p) w[(cc * 4 + dw) * 2 + p] = L.q8(d[dw], p);
    }
    const uint32_t sb = ld4(tile + kQ8CodeBytes + lane * 4);
    const float s = f16f(sb & 0xffffu), b = f16f(sb >> 16);
    const float cf = fmaf(-1024.f, s, b);
    for (int t = 0; t < nt; ++t) {
      const uint32_t* xp = reinterpret_cast<const uint32_t*>(&xr[t][wave][0]);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) d = dot2(w[i], xp[i], d);
      if (a.x_f32) {
        const uint32_t* xq = reinterpret_cast<const uint32_t*>(&xrl[t][wave][0]);
#pragma unroll
        for (int i = 0; i < 32; ++i) d = dot2(w[i], xq[i], d);
      }
      red[wave][t][lane] = fmaf(s, d, cf * xsum[t][wave]);
    }
  }
  __syncthreads();
  for (int i = tid; i < nt * 64; i += 256) {
    const int t = i >> 6, l = i & 63;
    float v = 0.f;
    for (int w = 0; w < ng; ++w) v += red[w][t][l];
    a.part[((size_t)ks * a.T + t0 + t) * a.Epad + rb * 64 + l] = v;
  }

  // 3. last workgroup of this token block: top-k
  __threadfence();
  __syncthreads();
  if (tid == 0) flag = (atomicAdd(&a.cnt_tb[tb], 1) == a.n_rb * a.KS - 1);
  __syncthreads();
  if (!flag) return;
  __threadfence();
  if (tid == 0) a.cnt_tb[tb] = 0;

  const int NE = a.Epad >> 6;
  for (int t = wave; t < nt; t += kRouterWaves) {
    const int tok = t0 + t;
    float v[kMaxExperts / 64];
#pragma unroll
    for (int i = 0; i < kMaxExperts / 64; ++i) {
      v[i] = -INFINITY;
      const int e = lane + 64 * i;
      if (i < NE && e < a.E) {
        float s = 0.f;
        for (int k2 = 0; k2 < a.KS; ++k2) s += a.part[((size_t)k2 * a.T + tok) * a.Epad + e];
        if (a.bias) s += a.bias[e];
        v[i] = s == s ? s : -INFINITY;   // a NaN logit (out of contract) ranks last
        if (a.mode == 1) a.logits_out[(size_t)tok * a.E + e] = s;
      }
    }
    if (a.mode == 1) continue;
    uint32_t taken = 0;
    float myv = 0.f;
    int myi = 0;
    for (int j = 0; j < a.k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxExperts / 64; ++i) {
        const int e = lane + 64 * i;
        if (i < NE && e < a.E && !((taken >> i) & 1u) && (bi == 0x7fffffff || v[i] > bv)) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == j) {
        myv = bv;
        myi = bi;
      }
    }
    const float mx = __shfl(myv, 0);
    const float z = lane < a.k ? expf(myv - mx) : 0.f;
    float sum = 0.f;
    for (int j = 0; j < a.k; ++j) sum += __shfl(z, j);
    myi = myi < a.E ? myi : 0;        // always an expert index, whatever the inputs
    if (lane < a.k) {
      const size_t o = (size_t)tok * a.k + lane;
      if (a.mode == 0) {
        const float p = z / sum;
        a.ids_ws[o] = myi;
        a.p_ws[o] = p;
        if (a.ids_out) a.ids_out[o] = myi;
        if (a.p_out) a.p_out[o] = p;
        a.rank[o] = atomicAdd(&a.counts[myi], 1);
      } else {
        a.pred[o] = myi;
      }
    }
  }
  if (a.mode == 1) return;

  // 4. last token block: bucketing (forward) or publish the prediction
  __threadfence();
  __syncthreads();
  if (tid == 0) flag = (atomicAdd(&a.misc[kCntAll], 1) == a.n_tb - 1);
  __syncthreads();
  if (!flag) return;
  __threadfence();
  if (a.mode == 2) {
    if (tid == 0) {
      a.misc[kPredValid] = a.T * a.k;   // number of predicted slots
      a.misc[kCntAll] = 0;
    }
    return;
  }
  bucket_final(a);
}

// --------------------------------------------------------- streaming path --

__device__ __forceinline__ size_t h_off(int slot, int Tk, int I, int Is) {
  return slot < Tk ? (size_t)slot * I : (size_t)Tk * I + (size_t)(slot - Tk) * Is;
}
__device__ __forceinline__ size_t hs_off(int slot, int Tk, int I, int Is) {
  return slot < Tk ? (size_t)slot * (I >> 6) : (size_t)Tk * (I >> 6) + (size_t)(slot - Tk) * (Is >> 6);
}

__global__ __launch_bounds__(256) void gemv_up_kernel(
    const uint8_t* __restrict__ bank, uint64_t stride, const uint8_t* __restrict__ shared,
    int H, int E, int k, int I, int Is, int T, int x_f32, const uint32_t* __restrict__ x16,
    const uint32_t* __restrict__ x16lo, const float* __restrict__ xs,
    const int4* __restrict__ items, const int* __restrict__ misc, const int* __restrict__ slots,
    uint16_t* __restrict__ hbuf, float* __restrict__ hs) {
  __shared__ int s_tok[kGemvTok];
  __shared__ int s_slot[kGemvTok];
  __shared__ float red[kGemvWaves][2][kGemvTok][64];
  const int item_i = blockIdx.y;
  if (item_i >= misc[kNGemv]) return;
  const int4 it = items[item_i];
  const int e = it.x, m = it.y, loff = it.z;
  const bool sh = e == E;
  const int inter = sh ? Is : I;
  const int rb = blockIdx.x;
  if (rb * 64 >= inter) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H >> 6, Tk = T * k;
  const size_t sec = (size_t)(inter >> 6) * G * kQ4TileBytes;
  const uint8_t* rec = sh ? shared : bank + (size_t)e * stride;
  const uint8_t* gate = rec + kHeaderBytes + (size_t)rb * G * kQ4TileBytes;
  const uint8_t* up = gate + sec;
  const int gbeg = (G * wave) / kGemvWaves, gend = (G * (wave + 1)) / kGemvWaves;
  const int hw = H >> 1;  // dwords per x16 row
  const Lift L;

  for (int p0 = 0; p0 < m; p0 += kGemvTok) {
    const int nt = min(kGemvTok, m - p0);
    if (tid < nt) {
      const int slot = slots[loff + p0 + tid];
      s_slot[tid] = slot;
      s_tok[tid] = slot < Tk ? slot / k : slot - Tk;
    }
    __syncthreads();
    float ag[kGemvTok], au[kGemvTok];
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t) ag[t] = au[t] = 0.f;
    for (int g = gbeg; g < gend; ++g) {
      const uint8_t* tg = gate + (size_t)g * kQ4TileBytes;
      const uint8_t* tu = up + (size_t)g * kQ4TileBytes;
      const uint4 cg0 = ld16(tg + lane * 16), cg1 = ld16(tg + 1024 + lane * 16);
      const uint4 cu0 = ld16(tu + lane * 16), cu1 = ld16(tu + 1024 + lane * 16);
      const uint32_t sbg = ld4(tg + kQ4CodeBytes + lane * 4);
      const uint32_t sbu = ld4(tu + kQ4CodeBytes + lane * 4);
      uint32_t wg[32], wu[32];
      unpack16_q4(L, cg0, wg);
      unpack16_q4(L, cg1, wg + 16);
      unpack16_q4(L, cu0, wu);
      unpack16_q4(L, cu1, wu + 16);
      const float sg = f16f(sbg & 0xffffu), cg = fmaf(-1024.f, sg, f16f(sbg >> 16));
      const float su = f16f(sbu & 0xffffu), cu = fmaf(-1024.f, su, f16f(sbu >> 16));
#pragma unroll
      for (int t = 0; t < kGemvTok; ++t) {
        if (t < nt) {
          const int tok = __builtin_amdgcn_readfirstlane(s_tok[t]);
          const cu32p xp = as_const(x16 + (size_t)tok * hw + g * 32);
          float dg = 0.f, du = 0.f;
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const uint32_t xv = xp[i];
            dg = dot2(wg[i], xv, dg);
            du = dot2(wu[i], xv, du);
          }
          if (x_f32) {
            const cu32p xq = as_const(x16lo + (size_t)tok * hw + g * 32);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              const uint32_t xv = xq[i];
              dg = dot2(wg[i], xv, dg);
              du = dot2(wu[i], xv, du);
            }
          }
          const float xsv = as_const(xs)[(size_t)tok * G + g];
          ag[t] += fmaf(sg, dg, cg * xsv);
          au[t] += fmaf(su, du, cu * xsv);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t)
      if (t < nt) {
        red[wave][0][t][lane] = ag[t];
        red[wave][1][t][lane] = au[t];
      }
    __syncthreads();
    for (int t = wave; t < nt; t += kGemvWaves) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) {
        gs += red[w][0][t][lane];
        us += red[w][1][t][lane];
      }
      const float hv = gs / (1.f + expf(-gs)) * us;
      const _Float16 h16 = (_Float16)hv;
      const int slot = s_slot[t];
      const int col = rb * 64 + lane;
      hbuf[h_off(slot, Tk, I, Is) + pair_pos4(col)] = f16bits(h16);
      const float hsum = wave_sum((float)h16);
      if (lane == 0) hs[hs_off(slot, Tk, I, Is) + rb] = hsum;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void gemv_down_kernel(
    const uint8_t* __restrict__ bank, uint64_t stride, const uint8_t* __restrict__ shared,
    int H, int E, int k, int I, int Is, int T, const int4* __restrict__ items,
    const int* __restrict__ misc, const int* __restrict__ slots,
    const uint32_t* __restrict__ hbuf32, const float* __restrict__ hs,
    float* __restrict__ yslot) {
  __shared__ int s_slot[kGemvTok];
  __shared__ float red[kGemvWaves][kGemvTok][64];
  const int item_i = blockIdx.y;
  if (item_i >= misc[kNGemv]) return;
  const int4 it = items[item_i];
  const int e = it.x, m = it.y, loff = it.z;
  const bool sh = e == E;
  const int inter = sh ? Is : I;
  const int rb = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H >> 6, G2 = inter >> 6, Tk = T * k;
  const size_t sec = (size_t)G2 * G * kQ4TileBytes;
  const uint8_t* rec = sh ? shared : bank + (size_t)e * stride;
  const uint8_t* down = rec + kHeaderBytes + 2 * sec + (size_t)rb * G2 * kQ4TileBytes;
  const int gbeg = (G2 * wave) / kGemvWaves, gend = (G2 * (wave + 1)) / kGemvWaves;
  const Lift L;

  for (int p0 = 0; p0 < m; p0 += kGemvTok) {
    const int nt = min(kGemvTok, m - p0);
    if (tid < nt) s_slot[tid] = slots[loff + p0 + tid];
    __syncthreads();
    float acc[kGemvTok];
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t) acc[t] = 0.f;
    for (int g = gbeg; g < gend; ++g) {
      const uint8_t* td = down + (size_t)g * kQ4TileBytes;
      const uint4 c0 = ld16(td + lane * 16), c1 = ld16(td + 1024 + lane * 16);
      const uint32_t sb = ld4(td + kQ4CodeBytes + lane * 4);
      uint32_t w[32];
      unpack16_q4(L, c0, w);
      unpack16_q4(L, c1, w + 16);
      const float s = f16f(sb & 0xffffu), c = fmaf(-1024.f, s, f16f(sb >> 16));
#pragma unroll
      for (int t = 0; t < kGemvTok; ++t) {
        if (t < nt) {
          const int slot = __builtin_amdgcn_readfirstlane(s_slot[t]);
          const cu32p hp = as_const(hbuf32 + (h_off(slot, Tk, I, Is) >> 1) + g * 32);
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < 32; ++i) d = dot2(w[i], hp[i], d);
          acc[t] += fmaf(s, d, c * as_const(hs)[hs_off(slot, Tk, I, Is) + g]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t)
      if (t < nt) red[wave][t][lane] = acc[t];
    __syncthreads();
    for (int t = wave; t < nt; t += kGemvWaves) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) v += red[w][t][lane];
      yslot[(size_t)s_slot[t] * H + rb * 64 + lane] = v;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- combine ----

__global__ __launch_bounds__(256) void combine_kernel(int H, int k, int T, int has_shared,
                                                      const float* __restrict__ p,
                                                      const float* __restrict__ yslot,
                                                      float* __restrict__ y) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H) return;
  const int Tk = T * k;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) acc = fmaf(p[t * k + j], yslot[(size_t)(t * k + j) * H + c], acc);
  if (has_shared) acc += yslot[(size_t)(Tk + t) * H + c];
  y[(size_t)t * H + c] = acc;
}

// ---------------------------------------------------------------- misc ----

__global__ void fill_i32_kernel(int* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// One thread per (row, dword of codes): decodes with the same unpacking the
// kernels use and writes s * q + b in fp32.
__global__ void debug_dequant_kernel(const uint8_t* __restrict__ tiles, int bits, int rows,
                                     int cols, float* __restrict__ out) {
  const int G = cols >> 6;
  const int per_row = cols / (bits == 4 ? 8 : 4);  // dwords per row
  const long n = (long)rows * per_row;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int r = (int)(i / per_row), dwi = (int)(i - (long)r * per_row);
  const int rb = r >> 6, rr = r & 63;
  const Lift L;
  if (bits == 4) {
    const int g = dwi >> 3, within = dwi & 7, h = within >> 2, d = within & 3;
    const uint8_t* tile = tiles + ((size_t)rb * G + g) * kQ4TileBytes;
    const uint32_t w = ld4(tile + h * 1024 + rr * 16 + d * 4);
    const uint32_t sb = ld4(tile + kQ4CodeBytes + rr * 4);
    const float s = f16f(sb & 0xffffu), b = f16f(sb >> 16);
    const int c0 = g * 64 + h * 32 + d * 8;
    for (int p = 0; p < 4; ++p) {
      const uint32_t pr = L.q4(w, p);
      out[(size_t)r * cols + c0 + p] = fmaf(s, f16f(pr & 0xffffu) - 1024.f, b);
      out[(size_t)r * cols + c0 + p + 4] = fmaf(s, f16f(pr >> 16) - 1024.f, b);
    }
  } else {
    const int g = dwi >> 4, within = dwi & 15, c4 = within >> 2, d = within & 3;
    const uint8_t* tile = tiles + ((size_t)rb * G + g) * kQ8TileBytes;
    const uint32_t w = ld4(tile + c4 * 1024 + rr * 16 + d * 4);
    const uint32_t sb = ld4(tile + kQ8CodeBytes + rr * 4);
    const float s = f16f(sb & 0xffffu), b = f16f(sb >> 16);
    const int c0 = g * 64 + c4 * 16 + d * 4;
    for (int p = 0; p < 2; ++p) {
      const uint32_t pr = L.q8(w, p);
      out[(size_t)r * cols + c0 + p] = fmaf(s, f16f(pr & 0xffffu) - 1024.f, b);
      out[(size_t)r * cols + c0 + p + 2] = fmaf(s, f16f(pr >> 16) - 1024.f, b);
    }
  }
}

// ------------------------------------------------------------- launches ----

static inline uint8_t* wsp(const LayerDev& d, size_t off) { return d.ws + off; }

hipError_t launch_router(const LayerDev& d, const void* x, int x_f32, int T, int mode,
                         float* logits_out, int32_t* ids_out, float* p_out, hipStream_t s) {
  RouterArgs a{};
  a.router = d.router;
  a.bias = d.router_bias;
  a.x = x;
  a.x_f32 = x_f32;
  a.T = T;
  a.H = d.H;
  a.G = d.H / kGroup;
  a.E = d.E;
  a.Epad = d.Epad;
  a.k = d.k;
  a.KS = router_ksplit(d.H);
  a.TBR = router_tok_block(T);
  a.n_tb = (T + a.TBR - 1) / a.TBR;
  a.n_rb = d.Epad / kTileRows;
  a.mode = mode;
  a.write_x = mode == 0;
  a.part = reinterpret_cast<float*>(wsp(d, d.L.part));
  a.x16 = reinterpret_cast<uint16_t*>(wsp(d, d.L.x16));
  a.x16lo = reinterpret_cast<uint16_t*>(wsp(d, d.L.x16lo));
  a.xs = reinterpret_cast<float*>(wsp(d, d.L.xs));
  a.cnt_tb = reinterpret_cast<int*>(wsp(d, d.L.cnt_tb));
  a.misc = reinterpret_cast<int*>(wsp(d, d.L.misc));
  a.counts = reinterpret_cast<int*>(wsp(d, d.L.counts));
  a.rank = reinterpret_cast<int*>(wsp(d, d.L.rank));
  a.ids_ws = reinterpret_cast<int*>(wsp(d, d.L.ids));
  a.p_ws = reinterpret_cast<float*>(wsp(d, d.L.p));
  a.ids_out = ids_out;
  a.p_out = p_out;
  a.logits_out = logits_out;
  a.pred = reinterpret_cast<int*>(wsp(d, d.L.pred));
  a.offs = reinterpret_cast<int*>(wsp(d, d.L.offs));
  a.slots = reinterpret_cast<int*>(wsp(d, d.L.slots));
  a.items = reinterpret_cast<int4*>(wsp(d, d.L.items));
  a.mitems = reinterpret_cast<int4*>(wsp(d, d.L.mitems));
  a.mtiles = reinterpret_cast<int2*>(wsp(d, d.L.mtiles));
  a.mfma_min_rows = d.mfma_min_rows;
  a.has_shared = d.has_shared;
  dim3 grid(a.n_rb, a.KS, a.n_tb);
  hipLaunchKernelGGL(router_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_experts(const LayerDev& d, int x_f32, int T, hipStream_t s) {
  const int Tk = T * d.k;
  const int ni = (Tk < d.E ? Tk : d.E) + (d.has_shared ? 1 : 0);
  const int imax = d.Is > d.I ? d.Is : d.I;
  const uint32_t* x16 = reinterpret_cast<const uint32_t*>(wsp(d, d.L.x16));
  const uint32_t* x16lo = reinterpret_cast<const uint32_t*>(wsp(d, d.L.x16lo));
  const float* xs = reinterpret_cast<const float*>(wsp(d, d.L.xs));
  const int4* items = reinterpret_cast<const int4*>(wsp(d, d.L.items));
  const int* misc = reinterpret_cast<const int*>(wsp(d, d.L.misc));
  const int* slots = reinterpret_cast<const int*>(wsp(d, d.L.slots));
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(wsp(d, d.L.hbuf));
  float* hs = reinterpret_cast<float*>(wsp(d, d.L.hs));
  float* yslot = reinterpret_cast<float*>(wsp(d, d.L.yslot));
  hipLaunchKernelGGL(gemv_up_kernel, dim3(imax / 64, ni), dim3(256), 0, s, d.bank, d.stride,
                     d.shared, d.H, d.E, d.k, d.I, d.Is, T, x_f32, x16, x16lo, xs, items, misc,
                     slots, hbuf, hs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(gemv_down_kernel, dim3(d.H / 64, ni), dim3(256), 0, s, d.bank, d.stride,
                     d.shared, d.H, d.E, d.k, d.I, d.Is, T, items, misc, slots,
                     reinterpret_cast<const uint32_t*>(hbuf), hs, yslot);
  return hipGetLastError();
}

hipError_t launch_combine(const LayerDev& d, int T, const float* p, float* y, hipStream_t s) {
  const float* yslot = reinterpret_cast<const float*>(wsp(d, d.L.yslot));
  hipLaunchKernelGGL(combine_kernel, dim3((d.H + 255) / 256, T), dim3(256), 0, s, d.H, d.k, T,
                     d.has_shared, p, yslot, y);
  return hipGetLastError();
}

hipError_t launch_ws_init(const LayerDev& d, hipStream_t s) {
  // counts [E], cnt_tb [..], misc [kMiscInts] must start at zero; they are
  // contiguous ints in the layout (counts .. misc end).
  int* base = reinterpret_cast<int*>(wsp(d, d.L.counts));
  const size_t n = (d.L.misc + kMiscInts * sizeof(int) - d.L.counts) / sizeof(int);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, base,
                     (int)n, 0);
  return hipGetLastError();
}

hipError_t launch_debug_dequant(const void* tiles, int bits, int rows, int cols, float* out,
                                hipStream_t s) {
  const long n = (long)rows * (cols / (bits == 4 ? 8 : 4));
  hipLaunchKernelGGL(debug_dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(tiles), bits, rows, cols, out);
  return hipGetLastError();
}

}  // namespace qreb
