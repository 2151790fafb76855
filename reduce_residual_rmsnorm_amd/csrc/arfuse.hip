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
//  * FP4 quantizes y32: s = E4M3(fl32(blockmax / 6)), q = fl32(|y| / s) with
//    IEEE division, q rounded to the E2M1 grid with ties to the even code.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "arfuse.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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

// Round to nearest even for finite x: adding 0x7FFF plus the lowest kept bit
// carries into the kept half exactly when the dropped half is above one half
// of a bf16 ulp, or equal to it with an odd kept half.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4 narrow8(const float f[8]) {
  u32x4 r;
  r.x = bf16_rne(f[0]) | (bf16_rne(f[1]) << 16);
  r.y = bf16_rne(f[2]) | (bf16_rne(f[3]) << 16);
  r.z = bf16_rne(f[4]) | (bf16_rne(f[5]) << 16);
  r.w = bf16_rne(f[6]) | (bf16_rne(f[7]) << 16);
  return r;
}

// ------------------------------------------------------------- FP4 helpers

// E4M3 (OCP, bias 7, max 448) code of x >= 0, nearest with ties to even.
// Below 2^-6 the format is fixed point with step 2^-9: x * 512 is exact and
// rintf rounds half to even, giving codes 0..8 (8 is 2^-6, the first normal
// code). Otherwise keep 3 mantissa bits of the fp32 pattern with the same
// carry trick as bf16 (bit 20 is the lowest kept bit); the fp32 exponent
// minus 120 is the E4M3 exponent field. Above 448 saturate.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  if (x < 0.015625f) return (uint32_t)rintf(x * 512.0f);
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  uint32_t c = (u >> 20) - (120u << 3);
  return c > 0x7Eu ? 0x7Eu : c;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  if (c < 8u) return (float)c * 0.001953125f;  // c * 2^-9, exact
  return __uint_as_float((c + (120u << 3)) << 20);
}

// E2M1 magnitude code of q >= 0 (0, .5, 1, 1.5, 2, 3, 4, 6): a tie goes to
// the even code, so ties at .25, 1.25, 2.5 and 5 round down and those at .75,
// 1.75 and 3.5 round up; above 6 saturates.
__device__ __forceinline__ uint32_t e2m1_rne(float q) {
  return (uint32_t)(q > 0.25f) + (uint32_t)(q >= 0.75f) + (uint32_t)(q > 1.25f) +
         (uint32_t)(q >= 1.75f) + (uint32_t)(q > 2.5f) + (uint32_t)(q >= 3.5f) +
         (uint32_t)(q > 5.0f);
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
  const float s = e4m3_value(sc);
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t mag = (s != 0.0f) ? e2m1_rne(fabsf(y[e]) / s) : 0u;
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
__device__ __attribute__((noinline)) u32x4 ll_repoll(const u32x4* p, u32x4 w, uint64_t flag,
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

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// ------------------------------------------------------------- row kernel

template <int N, int VPT, bool LL, bool OUT, bool FP4>
__global__ __launch_bounds__(kMaxBlock) void row_kernel(RowArgs a) {
  const int lane = threadIdx.x;
  const int nthr = blockDim.x;
  const int64_t d8 = a.d8;
  const int64_t row = blockIdx.x;
  const int64_t base = row * d8;

  bool valid[VPT];
  int64_t vi[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int64_t v = (int64_t)k * nthr + lane;
    valid[k] = v < d8;
    vi[k] = valid[k] ? v : d8 - 1;
  }

  // ---- issue every load of the row
  constexpr int W = LL ? 2 : 1;  // 16-byte words per 8 elements
  u32x4 raw[VPT][N][W];
  u32x4 rres[VPT];
  f32x4 g[VPT][2];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int w = 0; w < W; ++w) raw[k][i][w] = load16<true>(a.part[i] + (base + vi[k]) * W + w);
    }
    rres[k] = load16<true>(a.residual + base + vi[k]);
    g[k][0] = a.gamma[2 * vi[k]];
    g[k][1] = a.gamma[2 * vi[k] + 1];
  }

  // ---- LL: check flags, re-poll the mismatches, unpack the payload
  uint32_t bad = 0;
  u32x4 pv[VPT][N];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (LL) {
        u32x4 w0 = raw[k][i][0], w1 = raw[k][i][1];
        if (valid[k]) {
          const u32x4* p = a.part[i] + (base + vi[k]) * 2;
          if (__builtin_expect(!ll_ok(w0, a.ll_flag), 0)) w0 = ll_repoll(p, w0, a.ll_flag, a.max_polls, &bad);
          if (__builtin_expect(!ll_ok(w1, a.ll_flag), 0)) w1 = ll_repoll(p + 1, w1, a.ll_flag, a.max_polls, &bad);
        }
        pv[k][i] = u32x4{w0.x, w0.y, w1.x, w1.y};
      } else {
        pv[k][i] = raw[k][i][0];
      }
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
    if (valid[k]) {
      store16(a.residual_out + base + vi[k], narrow8(h[k]));
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

  // ---- row reduction: wave XOR tree, then one LDS slot per wave
  __shared__ double red[kMaxBlock / kWave];
  ss = wave_sum(ss);
  if ((lane & (kWave - 1)) == 0) red[lane / kWave] = ss;
  __syncthreads();
  double tot = 0.0;
  const int nw = nthr / kWave;
  for (int w = 0; w < nw; ++w) tot += red[w];
  const double inv = 1.0 / sqrt(tot / (double)(d8 * 8) + (double)a.eps);

  // ---- normalize, scale by gamma, store bf16 and/or FP4
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float y[8];
    const float gg[8] = {g[k][0].x, g[k][0].y, g[k][0].z, g[k][0].w,
                         g[k][1].x, g[k][1].y, g[k][1].z, g[k][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)(((double)h[k][e] * inv) * (double)gg[e]);
    if constexpr (OUT) {
      if (valid[k]) store16(a.out + base + vi[k], narrow8(y));
    }
    if constexpr (FP4) {
      uint32_t c8, sc;
      fp4_pair(y, c8, sc);
      if (valid[k]) {
        __builtin_nontemporal_store(c8, a.codes + base + vi[k]);
        if ((vi[k] & 1) == 0) a.scales[(base + vi[k]) >> 1] = (uint8_t)sc;
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

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    store16(dst + i, load16<true>(src + i));
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
  int64_t grid = (n + 255) / 256;
  if (grid > 256 * 32) grid = 256 * 32;  // 32 workgroups per CU, grid-stride beyond
  const u32x4* s = (const u32x4*)src;
  u32x4* dd = (u32x4*)dst;
  int64_t nn = n;
  void* args[] = {&s, &dd, &nn};
  hipError_t e = hipLaunchKernel((const void*)copy_kernel, dim3((unsigned)grid), dim3(256), args, 0,
                                 (hipStream_t)stream);
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
