// arfuse — fused all-reduce epilogue + residual add + RMSNorm (+ FP4) for
// gfx950 (MI355X). Kernels and the C ABI declared in include/arfuse.h.
//
// Design (one launch per call, HBM-bound, no matrix cores: the path is not a
// contraction):
//  * One workgroup per token row. Thread `lane` owns the 16-byte vectors
//    v = k * blockDim + lane (k < VPT) of the row, i.e. 8 consecutive bf16
//    elements per vector; consecutive lanes touch consecutive 16 bytes, so
//    every wave load is one fully coalesced 1 KiB transaction per partial.
//  * Every load of the row (N partials, residual, gamma) is issued before any
//    arithmetic, so a thread keeps N+2 independent 16-byte loads in flight.
//  * h stays in VGPRs between the sum and the normalize: no intermediate HBM
//    round trip (Deep Dive: AllReduce and AllReduce Fusion in TensorRT-LLM,
//    §6.1 and §6.4).
//  * The row's sum of squares is reduced across the wave with XOR shuffles,
//    then across waves through one LDS slot per wave, summed in wave order by
//    every thread (a fixed tree: deterministic, no atomics).
//  * Ragged rows (d/8 not a multiple of the block) clamp the vector index of
//    idle lanes to the last vector, so all loads stay unconditional and in
//    bounds; clamped lanes store nothing and add nothing.
//
// Arithmetic contract:
//  * rank sum and residual add: fp32 IEEE adds in rank order, residual last
//    (built with -ffp-contract=off); residual_out is bf16 round-to-nearest-
//    even of that h.
//  * the norm runs in fp64: sum of h^2, mean, 1/sqrt(mean + eps) and
//    y = (h * inv) * gamma, rounded once to fp32 (y32). MI355X executes fp64
//    FMAs at the fp32 (non-packed) rate and this kernel is HBM-bound, so the
//    extra precision costs no time and keeps y32 within an ulp of an fp64
//    reference.
//  * FP4 quantizes y32: s = E4M3(fl32(blockmax / 6)) (IEEE division), then
//    |y| / s rounded to the E2M1 grid with ties to the even code, decided by
//    exact comparisons with s * threshold (see e2m1_rne).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "arfuse.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBlock = 1024;
constexpr int kWave = 64;

struct RowArgs {
  const u32x4* part[ARFUSE_MAX_PARTIALS];  // plain: 16 B = 8 bf16; LL: 16 B words
  const u32x4* residual;
  const f32x4* gamma;
  u32x4* out;
  u32x4* residual_out;
  uint32_t* codes;   // 8 E2M1 codes per dword
  uint8_t* scales;
  arfuse_ll_status* status;
  int64_t d8;        // 16-byte bf16 vectors per row (d / 8)
  uint64_t ll_flag;
  float eps;
  uint32_t max_polls;
};

// ------------------------------------------------------------ bf16 helpers

__device__ __forceinline__ void widen8(u32x4 r, float f[8]) {
  f[0] = __uint_as_float(r.x << 16);
  f[1] = __uint_as_float(r.x & 0xFFFF0000u);
  f[2] = __uint_as_float(r.y << 16);
  f[3] = __uint_as_float(r.y & 0xFFFF0000u);
  f[4] = __uint_as_float(r.z << 16);
  f[5] = __uint_as_float(r.z & 0xFFFF0000u);
  f[6] = __uint_as_float(r.w << 16);
  f[7] = __uint_as_float(r.w & 0xFFFF0000u);
}

// Two fp32 -> two bf16, round to nearest even: gfx950's packed conversion
// (v_cvt_pk_bf16_f32), one instruction per pair. Its rounding is checked
// against the oracle on every tie and near-tie pattern of every 16-bit prefix
// through arfuse_round_bf16.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ u32x4 narrow8(const float f[8]) {
  return u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
               pack_bf16(f[6], f[7])};
}

// ------------------------------------------------------------- FP4 helpers

// E4M3 (OCP, bias 7, max 448) code of x >= 0, nearest with ties to even.
// Below 2^-6 the format is fixed point with step 2^-9: x * 512 is exact and
// rintf rounds half to even, giving codes 0..8 (8 is 2^-6, the first normal
// code). Otherwise keep 3 mantissa bits of the fp32 pattern with the same
// carry trick as bf16 (bit 20 is the lowest kept bit); the fp32 exponent
// minus 120 is the E4M3 exponent field. Above 448 saturate.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sub = (uint32_t)rintf(x * 512.0f);
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t c = min((u >> 20) - (120u << 3), 0x7Eu);
  return x < 0.015625f ? sub : c;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  if (c < 8u) return (float)c * 0.001953125f;  // c * 2^-9, exact
  return __uint_as_float((c + (120u << 3)) << 20);
}

// E2M1 magnitude code (0, .5, 1, 1.5, 2, 3, 4, 6 -> 0..7) of q = |y| / s,
// rounded to nearest with ties to the even code: ties at .25, 1.25, 2.5 and 5
// round down, those at .75, 1.75 and 3.5 round up, above 6 saturates.
// Instead of forming the quotient, |y| is compared with the products s*T,
// which are exact in fp32 (s has 4 significant bits, T at most 3). This takes
// the same decision as rounding the correctly rounded fp32 quotient for every
// finite |y|: the quotient's rounding can only matter within a couple of ulps
// of s*T, and an exhaustive sweep there (every scale, every threshold) finds
// no difference.
struct E2M1Thresholds {
  float t[7];
};

__device__ __forceinline__ E2M1Thresholds e2m1_thresholds(float s) {
  // s == 0: every magnitude is 0, which +inf thresholds give for finite |y|
  const float ss = (s != 0.0f) ? s : __builtin_inff();
  return E2M1Thresholds{{ss * 0.25f, ss * 0.75f, ss * 1.25f, ss * 1.75f, ss * 2.5f, ss * 3.5f,
                         ss * 5.0f}};
}

// The magnitude is the number of thresholds |y| passes (strictly for the
// ties that round down, t[0], t[2], t[4], t[6]); the thresholds ascend, so
// three comparisons find it: t[3] splits {0..3} from {4..7}, then t[1] or
// t[5], then one of the strict ones.
__device__ __forceinline__ uint32_t e2m1_rne(float a, const E2M1Thresholds& th) {
  const bool b2 = a >= th.t[3];
  const bool b1 = a >= (b2 ? th.t[5] : th.t[1]);
  const float tl = b2 ? (b1 ? th.t[6] : th.t[4]) : (b1 ? th.t[2] : th.t[0]);
  return (b2 ? 4u : 0u) + (b1 ? 2u : 0u) + (a > tl ? 1u : 0u);
}

// FP4 of the 8 values a lane holds. Lanes (2m, 2m+1) hold one 16-element
// block, so the block max is one XOR-1 shuffle away. Every lane of the wave
// must call this (the shuffle is a wave-wide operation).
__device__ __forceinline__ void fp4_pair(const float y[8], uint32_t& codes8, uint32_t& scale) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(y[e]));
  am = fmaxf(am, __shfl_xor(am, 1));
  const uint32_t sc = e4m3_rne(am / 6.0f);
  const E2M1Thresholds th = e2m1_thresholds(e4m3_value(sc));
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t mag = e2m1_rne(fabsf(y[e]), th);
    c |= (((__float_as_uint(y[e]) >> 31) << 3) | mag) << (4 * e);
  }
  codes8 = c;
  scale = sc;
}

// ------------------------------------------------------------- LL helpers

__device__ __forceinline__ bool ll_ok(u32x4 w, uint64_t flag) {
  return (w.z == (uint32_t)flag) & (w.w == (uint32_t)(flag >> 32));
}

// A word whose flag does not match is re-read with cache-bypassing (volatile)
// loads, a short sleep apart, at most max_polls times. Returns the last word
// read; *bad counts a word that never matched.
__device__ __forceinline__ u32x4 ll_repoll(const u32x4* p, u32x4 w, uint64_t flag,
                                                     uint32_t max_polls, uint32_t* bad) {
  for (uint32_t i = 0; i < max_polls; ++i) {
    __builtin_amdgcn_s_sleep(2);
    w = *(const volatile u32x4*)p;
    if (ll_ok(w, flag)) return w;
  }
  *bad += 1;
  return w;
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ void store16(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// DPP lane move of a double (two 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}

// Sum of a double over each row of 16 lanes, in every lane of the row: quad
// swaps (lane ^ 1, lane ^ 2), then the mirror inside each half row (quad 0
// with quad 1), then the mirror inside the row (half 0 with half 1). The
// additions are commutative pairs, so every lane of a row gets the same bits.
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ double lane_f64(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}

// Sum over the wave's 64 lanes (same value in every lane): the four row sums
// added in row order. A fixed tree: the result does not depend on timing.
__device__ __forceinline__ double wave_sum(double v) {
  v = row16_sum(v);
  return ((lane_f64(v, 0) + lane_f64(v, 16)) + lane_f64(v, 32)) + lane_f64(v, 48);
}

// ------------------------------------------------------------- row kernel

// Lane geometry. A thread handles 8 elements of its row per chunk k < VPT, as
// two groups of 4 (j = 0, 1); group_elem() is the row offset of a group's
// first element.
//  plain: the 8 elements are the contiguous 16-byte vector v = k*nthr + lane.
//  LL: each 16-byte word carries 4 elements, so the wave's 128 words of a
//      chunk are loaded as two fully contiguous 1 KiB instructions: lane i
//      takes words i and 64 + i of the wave's tile, i.e. groups at tile
//      offsets 4i and 256 + 4i.
template <bool LL>
__device__ __forceinline__ int64_t group_elem(int k, int j, int lane, int nthr) {
  if constexpr (LL)
    return 8 * ((int64_t)k * nthr + (lane & ~(kWave - 1))) + 256 * j + 4 * (lane & (kWave - 1));
  else
    return 8 * ((int64_t)k * nthr + lane) + 4 * j;
}

template <bool NT>
__device__ __forceinline__ u32x2 load8(const u32x2* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ void store8(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }

// FP4 of a 4-element group in the LL geometry: lanes 4m..4m+3 hold one
// 16-element block (two XOR shuffles give its max); 4 codes = 16 bits.
__device__ __forceinline__ void fp4_quad(const float* y, uint32_t& codes4, uint32_t& scale) {
  float am = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  const uint32_t sc = e4m3_rne(am / 6.0f);
  const E2M1Thresholds th = e2m1_thresholds(e4m3_value(sc));
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c |= (((__float_as_uint(y[e]) >> 31) << 3) | e2m1_rne(fabsf(y[e]), th)) << (4 * e);
  codes4 = c;
  scale = sc;
}

// Typed access at a byte offset from a base pointer. Row base pointers are
// uniform across the workgroup (scalar registers) and lane offsets fit in 32
// bits (rows are at most 65536 elements), so every load and store takes the
// scalar-base + 32-bit vector-offset form and a lane keeps one offset register
// for all N + 1 input streams instead of a 64-bit address per stream; that
// leaves room to keep all of a row's loads in flight at once.
template <typename T>
__device__ __forceinline__ const T* at(const char* base, uint32_t off) {
  return reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ __forceinline__ T* at_w(char* base, uint32_t off) {
  return reinterpret_cast<T*>(base + off);
}

template <int N, int VPT, bool LL, bool OUT, bool FP4>
__global__ __launch_bounds__(kMaxBlock) void row_kernel(RowArgs a) {
  const int lane = threadIdx.x;
  const int nthr = blockDim.x;
  const uint32_t d = (uint32_t)(a.d8 * 8);
  const int64_t rb = (int64_t)blockIdx.x * d;  // first element of the row

  // row bases: partials (bf16, or LL words of 4 bytes per element), residual,
  // outputs (bf16), FP4 codes (half a byte per element), scales (1/16)
  const char* prow[N];
#pragma unroll
  for (int i = 0; i < N; ++i) prow[i] = (const char*)a.part[i] + rb * (LL ? 4 : 2);
  const char* rrow = (const char*)a.residual + rb * 2;
  const char* grow = (const char*)a.gamma;
  char* orow = (char*)a.residual_out + rb * 2;
  char* yrow = (char*)a.out + rb * 2;
  char* crow = (char*)a.codes + rb / 2;
  char* srow = (char*)a.scales + rb / 16;

  // group offsets (elements), clamped into the row for idle lanes so every
  // load stays in bounds; idle lanes store nothing and add nothing
  uint32_t eo[VPT][2];
  bool ok[VPT][2];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if constexpr (LL) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t e = (uint32_t)group_elem<LL>(k, j, lane, nthr);
        ok[k][j] = e < d;
        eo[k][j] = ok[k][j] ? e : d - 4;
      }
    } else {  // the two groups of a plain vector share one validity
      const uint32_t e = (uint32_t)group_elem<LL>(k, 0, lane, nthr);
      ok[k][0] = ok[k][1] = e < d;
      eo[k][0] = ok[k][0] ? e : d - 8;
      eo[k][1] = eo[k][0] + 4;
    }
  }

  // ---- issue every load of the row
  u32x4 raw[VPT][N][LL ? 2 : 1];
  u32x4 rres[VPT];
  f32x4 g[VPT][2];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (LL) {
        raw[k][i][0] = load16<true>(at<u32x4>(prow[i], eo[k][0] * 4));
        raw[k][i][1] = load16<true>(at<u32x4>(prow[i], eo[k][1] * 4));
      } else {
        raw[k][i][0] = load16<true>(at<u32x4>(prow[i], eo[k][0] * 2));
      }
    }
    if constexpr (LL) {
      const u32x2 r0 = load8<true>(at<u32x2>(rrow, eo[k][0] * 2));
      const u32x2 r1 = load8<true>(at<u32x2>(rrow, eo[k][1] * 2));
      rres[k] = u32x4{r0.x, r0.y, r1.x, r1.y};
    } else {
      rres[k] = load16<true>(at<u32x4>(rrow, eo[k][0] * 2));
    }
    g[k][0] = *at<f32x4>(grow, eo[k][0] * 4);
    g[k][1] = *at<f32x4>(grow, eo[k][1] * 4);
  }
  // keep the scheduler from interleaving arithmetic into the load block: all
  // N + 3 loads of the row are in flight before the first use
  __builtin_amdgcn_sched_barrier(0);

  // ---- LL: check every flag with plain compares; only a lane holding a
  // mismatched word takes the (bounded) re-poll path. Then unpack the payload.
  uint32_t bad = 0;
  u32x4 pv[VPT][N];
  if constexpr (LL) {
    bool all_ok = true;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) all_ok &= !ok[k][j] || ll_ok(raw[k][i][j], a.ll_flag);
    if (__builtin_expect(!all_ok, 0)) {
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (ok[k][j] && !ll_ok(raw[k][i][j], a.ll_flag))
              raw[k][i][j] = ll_repoll(at<u32x4>(prow[i], eo[k][j] * 4), raw[k][i][j], a.ll_flag,
                                       a.max_polls, &bad);
    }
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (LL)
        pv[k][i] = u32x4{raw[k][i][0].x, raw[k][i][0].y, raw[k][i][1].x, raw[k][i][1].y};
      else
        pv[k][i] = raw[k][i][0];
    }
  }

  // ---- rank-ordered fp32 sum, residual last, residual_out, sum of squares
  float h[VPT][8];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float acc[8], f[8];
    widen8(pv[k][0], acc);
#pragma unroll
    for (int i = 1; i < N; ++i) {
      widen8(pv[k][i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + f[e];
    }
    widen8(rres[k], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) h[k][e] = acc[e] + f[e];
    const u32x4 hb = narrow8(h[k]);
    if constexpr (LL) {
      if (ok[k][0]) store8(at_w<u32x2>(orow, eo[k][0] * 2), u32x2{hb.x, hb.y});
      if (ok[k][1]) store8(at_w<u32x2>(orow, eo[k][1] * 2), u32x2{hb.z, hb.w});
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ok[k][e / 4]) ss += (double)h[k][e] * (double)h[k][e];
    } else if (ok[k][0]) {
      store16(at_w<u32x4>(orow, eo[k][0] * 2), hb);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (double)h[k][e] * (double)h[k][e];
    }
  }

  if constexpr (LL) {
    if (bad && a.status) {
      atomicAdd((unsigned long long*)&a.status->bad_words, (unsigned long long)bad);
      atomicOr(&a.status->code, (uint32_t)ARFUSE_ERR_FLAG_TIMEOUT);
    }
  }

  // ---- row reduction: DPP tree inside each wave, one LDS slot per wave, then
  // every wave sums the (at most 16) slots with the same 16-lane tree
  __shared__ double red[kMaxBlock / kWave];
  ss = wave_sum(ss);
  if ((lane & (kWave - 1)) == 0) red[lane / kWave] = ss;
  __syncthreads();
  const int nw = nthr / kWave;
  const int wl = lane & (kWave - 1);
  const double tot = lane_f64(row16_sum(wl < nw ? red[wl] : 0.0), 0);
  const double inv = 1.0 / sqrt(tot / (double)d + (double)a.eps);

  // ---- normalize, scale by gamma, store bf16 and/or FP4
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float y[8];
    const float gg[8] = {g[k][0].x, g[k][0].y, g[k][0].z, g[k][0].w,
                         g[k][1].x, g[k][1].y, g[k][1].z, g[k][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)(((double)h[k][e] * inv) * (double)gg[e]);
    if constexpr (OUT) {
      const u32x4 yb = narrow8(y);
      if constexpr (LL) {
        if (ok[k][0]) store8(at_w<u32x2>(yrow, eo[k][0] * 2), u32x2{yb.x, yb.y});
        if (ok[k][1]) store8(at_w<u32x2>(yrow, eo[k][1] * 2), u32x2{yb.z, yb.w});
      } else if (ok[k][0]) {
        store16(at_w<u32x4>(yrow, eo[k][0] * 2), yb);
      }
    }
    if constexpr (FP4) {
      if constexpr (LL) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t c4, sc;
          fp4_quad(y + 4 * j, c4, sc);
          if (ok[k][j]) {
            *at_w<uint16_t>(crow, eo[k][j] / 2) = (uint16_t)c4;
            if ((lane & 3) == 0) *at_w<uint8_t>(srow, eo[k][j] / 16) = (uint8_t)sc;
          }
        }
      } else {
        uint32_t c8, sc;
        fp4_pair(y, c8, sc);
        if (ok[k][0]) {
          __builtin_nontemporal_store(c8, at_w<uint32_t>(crow, eo[k][0] / 2));
          if ((eo[k][0] & 15) == 0) *at_w<uint8_t>(srow, eo[k][0] / 16) = (uint8_t)sc;
        }
      }
    }
  }
}

// Same argument block and launch shape as row_kernel, no work: the floor.
__global__ __launch_bounds__(kMaxBlock) void floor_kernel(RowArgs) {}

// FP4 of fp32 y [t][d]: thread i owns global 16-byte-bf16-vector index i
// (8 fp32 values); rows hold an even number of such vectors, so the pair
// (2m, 2m+1) never straddles a row. Idle lanes clamp like row_kernel.
__global__ __launch_bounds__(256) void quant_kernel(const f32x4* y, int64_t nvec, uint32_t* codes,
                                                    uint8_t* scales) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = v < nvec;
  const int64_t vc = valid ? v : nvec - 1;
  const f32x4 a = y[2 * vc], b = y[2 * vc + 1];
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t c8, sc;
  fp4_pair(f, c8, sc);
  if (valid) {
    codes[v] = c8;
    if ((v & 1) == 0) scales[v >> 1] = (uint8_t)sc;
  }
}

// The bf16 rounding of the fused kernel applied to an fp32 array (test entry).
__global__ __launch_bounds__(256) void round_bf16_kernel(const f32x2* x, int64_t npairs,
                                                         uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < npairs) out[i] = pack_bf16(x[i].x, x[i].y);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) store16(dst + i, load16<true>(src + i));
}

// ------------------------------------------------------------ dispatch

typedef void (*RowFn)(RowArgs);

template <int N, int VPT, bool LL>
RowFn by_epi(int epi) {
  switch (epi) {
    case ARFUSE_EPI_BF16: return row_kernel<N, VPT, LL, true, false>;
    case ARFUSE_EPI_FP4: return row_kernel<N, VPT, LL, false, true>;
    case ARFUSE_EPI_BF16 | ARFUSE_EPI_FP4: return row_kernel<N, VPT, LL, true, true>;
  }
  return nullptr;
}

template <int N, int VPT>
RowFn by_layout(bool ll, int epi) {
  return ll ? by_epi<N, VPT, true>(epi) : by_epi<N, VPT, false>(epi);
}

template <int N>
RowFn by_vpt(int vpt, bool ll, int epi) {
  switch (vpt) {
    case 1: return by_layout<N, 1>(ll, epi);
    case 2: return by_layout<N, 2>(ll, epi);
    case 4: return by_layout<N, 4>(ll, epi);
    case 8: return by_layout<N, 8>(ll, epi);
  }
  return nullptr;
}

RowFn select_row_kernel(int n, int vpt, bool ll, int epi) {
  switch (n) {
    case 1: return by_vpt<1>(vpt, ll, epi);
    case 2: return by_vpt<2>(vpt, ll, epi);
    case 3: return by_vpt<3>(vpt, ll, epi);
    case 4: return by_vpt<4>(vpt, ll, epi);
    case 5: return by_vpt<5>(vpt, ll, epi);
    case 6: return by_vpt<6>(vpt, ll, epi);
    case 7: return by_vpt<7>(vpt, ll, epi);
    case 8: return by_vpt<8>(vpt, ll, epi);
  }
  return nullptr;
}

// ------------------------------------------------------------ host checks

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ARFUSE_ERR_LAUNCH carries the runtime's hipError_t in bits 8 and up.
int launch_status(hipError_t e) {
  return e == hipSuccess ? ARFUSE_OK : (ARFUSE_ERR_LAUNCH | ((int)e << 8));
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, int64_t bytes) {
  return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
}

// Launch shape: the smallest VPT in {1, 2, 4, 8} whose 1024-thread block
// covers the row, block rounded up to whole waves; or the caller's override.
int choose_launch(int64_t d8, const arfuse_opts* o, int* block, int* vpt) {
  int v = o ? o->vpt : 0;
  int b = o ? o->block_threads : 0;
  if (v != 0 && v != 1 && v != 2 && v != 4 && v != 8) return ARFUSE_ERR_INVALID_ARG;
  if (b != 0 && (b < kWave || b > kMaxBlock || b % kWave)) return ARFUSE_ERR_INVALID_ARG;
  if (v == 0) {
    if (b != 0) {
      for (v = 1; v <= 8 && (int64_t)v * b < d8; v *= 2) {
      }
      if (v > 8) return ARFUSE_ERR_UNSUPPORTED;
    } else {
      for (v = 1; v <= 8 && (int64_t)v * kMaxBlock < d8; v *= 2) {
      }
      if (v > 8) return ARFUSE_ERR_UNSUPPORTED;
    }
  }
  if (b == 0) {
    int64_t need = (d8 + v - 1) / v;
    b = (int)(((need + kWave - 1) / kWave) * kWave);
    if (b < kWave) b = kWave;
  }
  if ((int64_t)v * b < d8) return ARFUSE_ERR_UNSUPPORTED;
  *block = b;
  *vpt = v;
  return ARFUSE_OK;
}

int check_shape(int n, int64_t t, int64_t d, int epi) {
  if (n < 1 || n > ARFUSE_MAX_PARTIALS) return ARFUSE_ERR_INVALID_ARG;
  if (t < 0 || d <= 0 || d % 16) return ARFUSE_ERR_INVALID_ARG;
  if (epi < 1 || epi > 3) return ARFUSE_ERR_INVALID_ARG;
  if (d > ARFUSE_MAX_D) return ARFUSE_ERR_UNSUPPORTED;
  if (t > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;  // one workgroup per row
  return ARFUSE_OK;
}

int rmsnorm_impl(const void* const* partials, int n, const void* residual, const float* gamma,
                 float eps, void* out, void* residual_out, uint8_t* fp4_out, uint8_t* fp4_scales,
                 int64_t t, int64_t d, void* stream, const arfuse_opts* opts) {
  const int layout = opts ? opts->layout : ARFUSE_LAYOUT_PLAIN;
  if (layout != ARFUSE_LAYOUT_PLAIN && layout != ARFUSE_LAYOUT_LL) return ARFUSE_ERR_INVALID_ARG;
  const bool ll = layout == ARFUSE_LAYOUT_LL;
  const int epi = (out ? ARFUSE_EPI_BF16 : 0) | (fp4_out ? ARFUSE_EPI_FP4 : 0);
  int rc = check_shape(n, t, d, epi ? epi : 1);
  if (rc) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ARFUSE_ERR_INVALID_ARG;
  int block = 0, vpt = 0;
  rc = choose_launch(d / 8, opts, &block, &vpt);
  if (rc) return rc;
  if (t == 0) return ARFUSE_OK;  // no-op: buffers are never touched, may be NULL
  if (!partials) return ARFUSE_ERR_INVALID_ARG;
  if (!epi) return ARFUSE_ERR_INVALID_ARG;  // nothing to write
  if ((fp4_out == nullptr) != (fp4_scales == nullptr)) return ARFUSE_ERR_INVALID_ARG;
  if (!residual || !gamma || !residual_out) return ARFUSE_ERR_INVALID_ARG;
  if (!aligned16(residual) || !aligned16(gamma) || !aligned16(residual_out) ||
      (out && !aligned16(out)) || (fp4_out && !aligned16(fp4_out)))
    return ARFUSE_ERR_INVALID_ARG;
  const int64_t plane = t * d * 2;                // one bf16 [t][d]
  const int64_t pbytes = ll ? 2 * plane : plane;  // one partial
  Range in[ARFUSE_MAX_PARTIALS + 2];
  int nin = 0;
  for (int i = 0; i < n; ++i) {
    if (!partials[i] || !aligned16(partials[i])) return ARFUSE_ERR_INVALID_ARG;
    in[nin++] = range_of(partials[i], pbytes);
  }
  in[nin++] = range_of(gamma, d * 4);
  const Range rres = range_of(residual, plane);
  Range outs[4];
  int nout = 0;
  outs[nout++] = range_of(residual_out, plane);
  if (out) outs[nout++] = range_of(out, plane);
  if (fp4_out) {
    outs[nout++] = range_of(fp4_out, t * d / 2);
    outs[nout++] = range_of(fp4_scales, t * d / 16);
  }
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], in[i])) return ARFUSE_ERR_INVALID_ARG;
    for (int p = o + 1; p < nout; ++p)
      if (overlap(outs[o], outs[p])) return ARFUSE_ERR_INVALID_ARG;
    // residual_out may be residual itself (in place), nothing else may overlap it
    if (o == 0) {
      if (outs[0].lo != rres.lo && overlap(outs[0], rres)) return ARFUSE_ERR_INVALID_ARG;
    } else if (overlap(outs[o], rres)) {
      return ARFUSE_ERR_INVALID_ARG;
    }
  }

  RowArgs a = {};
  for (int i = 0; i < n; ++i) a.part[i] = (const u32x4*)partials[i];
  a.residual = (const u32x4*)residual;
  a.gamma = (const f32x4*)gamma;
  a.out = (u32x4*)out;
  a.residual_out = (u32x4*)residual_out;
  a.codes = (uint32_t*)fp4_out;
  a.scales = fp4_scales;
  a.status = opts ? opts->status : nullptr;
  a.d8 = d / 8;
  a.ll_flag = opts ? opts->ll_flag : 0;
  a.eps = eps;
  a.max_polls = opts ? opts->max_polls : 0;

  const void* fn = (const void*)select_row_kernel(n, vpt, ll, epi);
  if (!fn) return ARFUSE_ERR_UNSUPPORTED;
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)t), dim3((unsigned)block), args, 0,
                                 (hipStream_t)stream);
  return launch_status(e);
}

}  // namespace

extern "C" {

int arfuse_rmsnorm(const void* const* partials, int n_partials, const void* residual,
                   const float* gamma, float eps, void* out, void* residual_out, uint8_t* fp4_out,
                   uint8_t* fp4_scales, int64_t t, int64_t d, void* stream) {
  return rmsnorm_impl(partials, n_partials, residual, gamma, eps, out, residual_out, fp4_out,
                      fp4_scales, t, d, stream, nullptr);
}

int arfuse_rmsnorm_ex(const void* const* partials, int n_partials, const void* residual,
                      const float* gamma, float eps, void* out, void* residual_out,
                      uint8_t* fp4_out, uint8_t* fp4_scales, int64_t t, int64_t d, void* stream,
                      const arfuse_opts* opts) {
  return rmsnorm_impl(partials, n_partials, residual, gamma, eps, out, residual_out, fp4_out,
                      fp4_scales, t, d, stream, opts);
}

int arfuse_quantize_fp4(const float* y, int64_t t, int64_t d, uint8_t* codes, uint8_t* scales,
                        void* stream) {
  if (t < 0 || d <= 0 || d % 16) return ARFUSE_ERR_INVALID_ARG;
  if (t == 0) return ARFUSE_OK;
  if (!y || !codes || !scales) return ARFUSE_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(codes)) return ARFUSE_ERR_INVALID_ARG;
  const Range ry = range_of(y, t * d * 4), rc = range_of(codes, t * d / 2),
              rs = range_of(scales, t * d / 16);
  if (overlap(ry, rc) || overlap(ry, rs) || overlap(rc, rs)) return ARFUSE_ERR_INVALID_ARG;
  const int64_t nvec = t * (d / 8);
  const int64_t grid = (nvec + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  const f32x4* yy = (const f32x4*)y;
  uint32_t* cc = (uint32_t*)codes;
  int64_t nv = nvec;
  void* args[] = {&yy, &nv, &cc, &scales};
  hipError_t e = hipLaunchKernel((const void*)quant_kernel, dim3((unsigned)grid), dim3(256), args,
                                 0, (hipStream_t)stream);
  return launch_status(e);
}

int arfuse_query_launch(int n_partials, int64_t t, int64_t d, int epilogue,
                        const arfuse_opts* opts, arfuse_launch_info* info) {
  if (!info) return ARFUSE_ERR_INVALID_ARG;
  int rc = check_shape(n_partials, t, d, epilogue);
  if (rc) return rc;
  if (opts && opts->layout != ARFUSE_LAYOUT_PLAIN && opts->layout != ARFUSE_LAYOUT_LL)
    return ARFUSE_ERR_INVALID_ARG;
  int block = 0, vpt = 0;
  rc = choose_launch(d / 8, opts, &block, &vpt);
  if (rc) return rc;
  info->grid = t;
  info->block = block;
  info->vpt = vpt;
  return ARFUSE_OK;
}

int arfuse_launch_floor(int n_partials, int64_t t, int64_t d, int epilogue,
                        const arfuse_opts* opts, void* stream) {
  int rc = check_shape(n_partials, t, d, epilogue);
  if (rc) return rc;
  int block = 0, vpt = 0;
  rc = choose_launch(d / 8, opts, &block, &vpt);
  if (rc) return rc;
  if (t == 0) return ARFUSE_OK;
  RowArgs a = {};
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel((const void*)floor_kernel, dim3((unsigned)t), dim3((unsigned)block),
                                 args, 0, (hipStream_t)stream);
  return launch_status(e);
}

int arfuse_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes < 0 || bytes % 16 || !aligned16(dst) || !aligned16(src))
    return ARFUSE_ERR_INVALID_ARG;
  if (bytes > 0 && overlap(range_of(dst, bytes), range_of(src, bytes))) return ARFUSE_ERR_INVALID_ARG;
  if (bytes == 0) return ARFUSE_OK;
  const int64_t n = bytes / 16;
  const int64_t grid = (n + 255) / 256;  // one 16-byte vector per thread
  if (grid > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  const u32x4* s = (const u32x4*)src;
  u32x4* dd = (u32x4*)dst;
  int64_t nn = n;
  void* args[] = {&s, &dd, &nn};
  hipError_t e = hipLaunchKernel((const void*)copy_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                                 (hipStream_t)stream);
  return launch_status(e);
}

int arfuse_round_bf16(const float* x, int64_t n, uint16_t* out, void* stream) {
  if (n < 0 || n % 2) return ARFUSE_ERR_INVALID_ARG;
  if (n == 0) return ARFUSE_OK;
  if (!x || !out || ((uintptr_t)x & 7u) || ((uintptr_t)out & 3u)) return ARFUSE_ERR_INVALID_ARG;
  if (overlap(range_of(x, n * 4), range_of(out, n * 2))) return ARFUSE_ERR_INVALID_ARG;
  const int64_t npairs = n / 2;
  const int64_t grid = (npairs + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  const f32x2* xx = (const f32x2*)x;
  uint32_t* oo = (uint32_t*)out;
  int64_t np = npairs;
  void* args[] = {&xx, &np, &oo};
  hipError_t e = hipLaunchKernel((const void*)round_bf16_kernel, dim3((unsigned)grid), dim3(256),
                                 args, 0, (hipStream_t)stream);
  return launch_status(e);
}

const char* arfuse_status_string(int status) {
  if ((status & 0xFF) == ARFUSE_ERR_LAUNCH) return "kernel launch failed";
  switch (status) {
    case ARFUSE_OK: return "ok";
    case ARFUSE_ERR_INVALID_ARG: return "invalid argument";
    case ARFUSE_ERR_UNSUPPORTED: return "unsupported shape or launch";
    case ARFUSE_ERR_LAUNCH: return "kernel launch failed";
    case ARFUSE_ERR_FLAG_TIMEOUT: return "LL flag did not match after the bounded poll";
  }
  return "unknown status";
}

int arfuse_version(void) { return ARFUSE_VERSION; }

}  // extern "C"
