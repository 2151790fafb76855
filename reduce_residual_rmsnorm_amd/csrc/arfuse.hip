// arfuse — fused all-reduce epilogue + residual add + RMSNorm (+ FP4) for
// gfx950 (MI355X). The C ABI declared in include/arfuse.h and its auxiliary
// kernels; the device helpers and the row kernel are in arfuse_device.hpp.
//
// Design (one launch per call, HBM-bound, no matrix cores: the path is not a
// contraction):
//  * One workgroup per token row (or per slice of a split row). Thread `lane`
//    owns the 16-byte vectors v = k * blockDim + lane (k < VPT) of the row,
//    i.e. 8 consecutive bf16 elements per vector; consecutive lanes touch
//    consecutive 16 bytes, so every wave load is one fully coalesced 1 KiB
//    transaction per partial.
//  * While the row fits the registers at once, every partial and residual
//    load is issued before any arithmetic (gamma follows the rank sum, out of
//    the partials' fetch); wider rows run as a pipeline of chunks with loads
//    one or two chunks ahead.
//  * h stays in VGPRs between the sum and the normalize: no intermediate HBM
//    round trip (Deep Dive: AllReduce and AllReduce Fusion in TensorRT-LLM,
//    §6.1 and §6.4). residual_out is stored next to y, after the row's reads.
//  * The row's sum of squares is reduced across the wave with DPP moves, then
//    across waves through one LDS slot per wave, summed by the same 16-lane
//    tree in every wave (a fixed tree: deterministic, no atomics).
//  * Calls whose rows take several rounds of workgroups (prefill) run
//    instances whose output stores write through to memory; decode-sized
//    calls keep non-temporal stores (see out_store).
//  * Ragged rows (d/8 not a multiple of the block) clamp the vector index of
//    idle lanes to the last vector, so all loads stay unconditional and in
//    bounds; clamped lanes store nothing and add nothing.
//
// Arithmetic contract:
//  * rank sum and residual add: fp32 IEEE adds in rank order, residual last
//    (built with -ffp-contract=off); residual_out is bf16 round-to-nearest-
//    even of that h.
//  * the norm: sum of h^2 in fp64 (exact squares by FMA), inverse RMS
//    1/sqrt(mean + eps) in fp64, rounded once to fp32; y = (h * inv) * gamma
//    by two fp32 multiplies.
//  * FP4 quantizes y: s = E4M3(fl32(blockmax / 6)) (the quotient exactly as
//    IEEE division gives it, then gfx950's E4M3 conversion), then |y| / s
//    rounded to the E2M1 grid with ties to the even code: gfx950's FP4
//    conversion inside a reciprocal envelope, with exact comparisons against
//    s * threshold where the envelope leaves a decision open (see
//    e2m1_envelope and e2m1_two).

#include <cstring>
#include <mutex>

#include "arfuse_device.hpp"

namespace arfuse_detail {
namespace {

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

// FP4 of fp32 y [t][d] in the lane geometry of the LL layout: thread i owns
// the 4-element group i, so lanes 4m..4m+3 hold one 16-element block, as a
// wave of an LL row does (fp4_quad, the same 16-bit code store and scale
// store). d % 16 == 0, so the groups of a block never straddle a row and the
// 4 lanes of a block are all valid or all idle; idle lanes clamp to the last
// block.
__global__ __launch_bounds__(256) void quant_ll_kernel(const f32x4* y, int64_t ngroups,
                                                       uint16_t* codes, uint8_t* scales) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = v < ngroups;
  const int64_t vc = valid ? v : ngroups - 4 + (v & 3);
  const f32x4 a = y[vc];
  const float f[4] = {a.x, a.y, a.z, a.w};
  uint32_t c4, sc;
  fp4_quad(f, c4, sc);
  if (valid) {
    codes[v] = (uint16_t)c4;
    if ((v & 3) == 0) scales[v >> 2] = (uint8_t)sc;
  }
}

// The fused call's byte mix without its arithmetic: one workgroup per row,
// the row kernel's lane geometry and vectors per thread, non-temporal loads;
// the streaming instances' write-through stores where the fused call takes
// them (several rounds of workgroups), else non-temporal stores. Row r of
// every output plane receives the XOR of row r of the input planes. Every
// load of the row is issued before the first use, as in a row-kernel
// instance that holds its whole row. (With the default-policy stores and
// residual loads of the fused call's one-round instances, this kernel, which
// stores each vector as soon as its own loads land, is slower: t=512 N=8
// 18.7 us against 16.4; the fused call's rows store only after their row's
// reduction.)
constexpr int kMixMaxIn = ARFUSE_MAX_PARTIALS + 1;
constexpr int kMixMaxOut = 3;
struct MixArgs {
  const u32x4* in[kMixMaxIn];
  u32x4* out[kMixMaxOut];
  int64_t d8;
  int32_t n_in, n_out;
};

template <int VPT, bool STREAM>
__global__ __launch_bounds__(kMaxBlock) void mix_kernel(MixArgs a) {
  const int lane = threadIdx.x;
  const int nthr = blockDim.x;
  const uint32_t d8 = (uint32_t)a.d8;
  const int64_t rb = (int64_t)blockIdx.x * d8 * 16;  // row base, bytes
  uint32_t off[VPT];
  bool ok[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const uint32_t v = (uint32_t)(k * nthr + lane);
    ok[k] = v < d8;
    off[k] = (ok[k] ? v : d8 - 1) * 16u;
  }
  u32x4 raw[VPT][kMixMaxIn];
#pragma unroll
  for (int k = 0; k < VPT; ++k)
#pragma unroll
    for (int i = 0; i < kMixMaxIn; ++i)
      if (i < a.n_in) raw[k][i] = load16<true>(at<u32x4>((const char*)a.in[i] + rb, off[k]));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    u32x4 x = raw[k][0];
#pragma unroll
    for (int i = 1; i < kMixMaxIn; ++i)
      if (i < a.n_in) x ^= raw[k][i];
    if (ok[k]) {
#pragma unroll
      for (int o = 0; o < kMixMaxOut; ++o)
        if (o < a.n_out)
          out_store<STREAM ? kStoreThrough : kStoreNT>((char*)a.out[o] + rb, off[k], x);
    }
  }
}

// The bf16 rounding of the fused kernel applied to an fp32 array (test entry).
__global__ __launch_bounds__(256) void round_bf16_kernel(const f32x2* x, int64_t npairs,
                                                         uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < npairs) out[i] = pack_bf16(x[i].x, x[i].y);
}

// The FP8 conversion of the fused kernel (inv_scale 1) applied to an fp32
// array (test entry).
__global__ __launch_bounds__(256) void round_fp8_kernel(const f32x4* x, int64_t nquads,
                                                        uint32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nquads) {
    const f32x4 v = x[i];
    const float y[4] = {v.x, v.y, v.z, v.w};
    out[i] = fp8_quad(y, 1.0f);
  }
}

// gfx950's FP4 conversion (scale 1) of fp32 pairs, as the fused kernel's
// fast FP4 path uses it: byte i holds x[2i] (low nibble) and x[2i + 1].
__global__ __launch_bounds__(256) void round_fp4_kernel(const f32x2* x, int64_t npairs,
                                                        uint8_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < npairs) {
    const f32x2 v = x[i];
    out[i] = (uint8_t)cvt_fp4x2<0>(0u, v.x, v.y);
  }
}

// Streaming copy, 16 bytes per thread: non-temporal loads and the
// write-through stores of the prefill instances (1 GiB: 6.52 TB/s with
// non-temporal stores, 6.64 with these).
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x;
  const int64_t i = b + threadIdx.x;
  if (i < n) out_store<kStoreThrough>((char*)(dst + b), threadIdx.x * 16u, load16<true>(src + i));
}

// ------------------------------------------------------------ dispatch

RowFn select_row_kernel(int n, int vpt, int layout, int epi, int kind) {
  switch (n) {
    case 1: return select_row_kernel_n1(vpt, layout, epi, kind);
    case 2: return select_row_kernel_n2(vpt, layout, epi, kind);
    case 3: return select_row_kernel_n3(vpt, layout, epi, kind);
    case 4: return select_row_kernel_n4(vpt, layout, epi, kind);
    case 5: return select_row_kernel_n5(vpt, layout, epi, kind);
    case 6: return select_row_kernel_n6(vpt, layout, epi, kind);
    case 7: return select_row_kernel_n7(vpt, layout, epi, kind);
    case 8: return select_row_kernel_n8(vpt, layout, epi, kind);
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

// Sentinel layout with a reset set: up to this many rows, the rows leave the
// reset to extra blocks of the same launch (the rows occupy at most half of
// the 256 CUs, so the reset stores run on CUs that would otherwise idle);
// above it every row block refills its own row.
constexpr int64_t kSpreadResetRows = 128;

// Rows times vectors per thread at and above which a call runs the
// streaming-store instances (kRowStream; see out_store): several rounds of
// workgroups, prefill. N=8 against the whole-row instances: faster at
// t*VPT = 1536 (t=1536 d=8192: 46.4 against 48.7 us), 2048 (t=2048 d=8192:
// 60.5 against 66.7; t=1024 d=16384: 62.0 against 69.3) and above; slower
// at 1024 (t=1024 d=8192: 32.2 against 30.45; t=512 d=16384: 32.9 against
// 31.9) and below, and at decode. LL rows have no streaming instances
// (their words are decode-sized by design).
constexpr int64_t kStreamStoreChunks = 1536;

int row_kind(int64_t t, int lg, int vpt, int layout) {
  if (lg != 0) return kRowSplit;
  if (layout != ARFUSE_LAYOUT_LL && t * vpt >= kStreamStoreChunks) return kRowStream;
  return kRowWhole;
}

// Extra reset blocks of a call: N planes of t * d / 8 vectors, one vector per
// thread. 0 when the rows do the reset themselves or there is none.
int64_t reset_blocks(int n, int64_t t, int64_t d, int block, bool reset) {
  if (!reset || t > kSpreadResetRows) return 0;
  const int64_t plane_vecs = t * d / 8;
  return (int64_t)n * ((plane_vecs + block - 1) / block);
}

// Split rows are compiled for one or two vectors per thread: a slice covers at
// most 2 * kMaxBlock vectors (16,384 elements).
constexpr int kMaxSplitVpt = 2;

// The launch of a call whose rows are split 1 << lg ways.
int row_launch(int64_t d, int lg, const arfuse_opts* o, int* block, int* vpt) {
  const int rc = choose_launch((d / 8) >> lg, o, block, vpt);
  if (rc) return rc;
  if (lg != 0 && *vpt > kMaxSplitVpt) return ARFUSE_ERR_UNSUPPORTED;
  return ARFUSE_OK;
}

// Work per SIMD of a workgroup covering `vecs` 16-byte vectors per partial at
// the default launch: vectors per thread times waves per SIMD.
int64_t work_per_simd(int64_t vecs) {
  int64_t v = 1;
  while (v * kMaxBlock < vecs) v *= 2;
  const int64_t block = (vecs + v - 1) / v;
  return v * ((block + 4 * kWave - 1) / (4 * kWave));
}

// ARFUSE_SPLIT_AUTO: the smallest split whose slices need at most 256 threads
// (one wave per SIMD at one vector per thread) and read at most 16 KiB of
// partials per workgroup, within the split limits; kept only where it removes
// at least three waves' work per SIMD or the unsplit workgroup would read
// 128 KiB or more. Measured on MI355X decode chains: the exchange costs about
// 0.75 us, and a CU fetching data the caches do not hold reads a few tens of
// GB/s, so a row's bytes are best spread thin once they are many.
// The all-reduce alone (no norm) needs no exchange, so it splits whenever
// the row reads 32 KiB or more.
int auto_split_log2(int n, int64_t t, int64_t d, bool ll, bool norm) {
  const int64_t d8 = d / 8;
  const int64_t vec_bytes = (ll ? 32 : 16) * (int64_t)n;
  int lg = 0;
  while (lg < 3 && ((d8 >> lg) > 256 || (d8 >> lg) * vec_bytes > 16384)) ++lg;
  while (lg > 0 && ((t << lg) > ARFUSE_MAX_SPLIT_BLOCKS || d % (16LL << lg))) --lg;
  if (lg == 0 || (d8 >> lg) > kMaxSplitVpt * kMaxBlock) return 0;
  if (!norm) return d8 * vec_bytes >= 32768 ? lg : 0;
  if (work_per_simd(d8) - work_per_simd(d8 >> lg) < 3 && d8 * vec_bytes < 131072) return 0;
  return lg;
}

// Split rows launch their slices at row positions 0..prows-1, prows being t
// rounded up to a multiple of 8, so that every slice of a row can take the
// same b mod 8 (its XCD; the kernel maps workgroup b to its row and slice
// with shifts and masks); rows past t are padding. With
// t * split <= ARFUSE_MAX_SPLIT_BLOCKS and split <= 8, the padded launch
// prows * split fits the same cap (256 / split is a multiple of 8).
int64_t split_rows(int64_t t, int lg) { return lg ? (t + 7) / 8 * 8 : t; }

// Bytes of a split call's exchange slots: two regions of one 128-byte line
// per row position (at most 128 positions: 32 KiB).
int64_t split_ws_bytes(int64_t t, int lg) { return lg ? split_rows(t, lg) * 256 : 0; }

// Split rows: the validated number of workgroups per row, as its log2 (0 when
// a row is one workgroup). Every workgroup of a split row must be resident at
// once, hence the cap on t * split.
int split_log2(const arfuse_opts* o, int n, int64_t t, int64_t d, int epi, int* lg) {
  const uint32_t s = o ? o->split : 0u;
  *lg = 0;
  if (s == ARFUSE_SPLIT_AUTO) {
    *lg = auto_split_log2(n, t, d, o->layout == ARFUSE_LAYOUT_LL, epi != 0);
    return ARFUSE_OK;
  }
  if (s <= 1) return ARFUSE_OK;
  if (s != 2 && s != 4 && s != 8) return ARFUSE_ERR_INVALID_ARG;
  if (d % (16 * (int64_t)s)) return ARFUSE_ERR_INVALID_ARG;
  if (t * (int64_t)s > ARFUSE_MAX_SPLIT_BLOCKS) return ARFUSE_ERR_UNSUPPORTED;
  *lg = s == 2 ? 1 : s == 4 ? 2 : 3;
  return ARFUSE_OK;
}

int check_shape(int n, int64_t t, int64_t d, int epi) {
  if (n < 1 || n > ARFUSE_MAX_PARTIALS) return ARFUSE_ERR_INVALID_ARG;
  if (t < 0 || d <= 0 || d % 16) return ARFUSE_ERR_INVALID_ARG;
  if (epi < 0 || epi > 7) return ARFUSE_ERR_INVALID_ARG;
  if ((epi & ARFUSE_EPI_FP4) && (epi & ARFUSE_EPI_FP8)) return ARFUSE_ERR_UNSUPPORTED;
  if (d > ARFUSE_MAX_D) return ARFUSE_ERR_UNSUPPORTED;
  if (t > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;  // one workgroup per row
  return ARFUSE_OK;
}

int rmsnorm_impl(const void* const* partials, int n, const void* residual, const float* gamma,
                 float eps, void* out, void* residual_out, uint8_t* fp4_out, uint8_t* fp4_scales,
                 int64_t t, int64_t d, void* stream, const arfuse_opts* opts) {
  const int layout = opts ? opts->layout : ARFUSE_LAYOUT_PLAIN;
  if (layout != ARFUSE_LAYOUT_PLAIN && layout != ARFUSE_LAYOUT_LL &&
      layout != ARFUSE_LAYOUT_SENTINEL)
    return ARFUSE_ERR_INVALID_ARG;
  if (opts && opts->reserved2 != 0) return ARFUSE_ERR_INVALID_ARG;
  if (opts && opts->max_polls > ARFUSE_MAX_POLLS) return ARFUSE_ERR_INVALID_ARG;
  const bool ll = layout == ARFUSE_LAYOUT_LL;
  const bool sentinel = layout == ARFUSE_LAYOUT_SENTINEL;
  uint8_t* fp8_out = opts ? opts->fp8_out : nullptr;
  void* const* reset = opts ? opts->reset : nullptr;
  const uint32_t spat = (opts && opts->sentinel) ? opts->sentinel : ARFUSE_SENTINEL_DEFAULT;
  if (spat > 0xFFFFu) return ARFUSE_ERR_INVALID_ARG;
  if (reset && !sentinel) return ARFUSE_ERR_INVALID_ARG;
  if (fp8_out && !isfinite(opts->fp8_inv_scale)) return ARFUSE_ERR_INVALID_ARG;
  const int epi = (out ? ARFUSE_EPI_BF16 : 0) | (fp4_out ? ARFUSE_EPI_FP4 : 0) |
                  (fp8_out ? ARFUSE_EPI_FP8 : 0);
  int rc = check_shape(n, t, d, epi);
  if (rc) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ARFUSE_ERR_INVALID_ARG;
  int lg = 0;
  rc = split_log2(opts, n, t, d, epi, &lg);
  if (rc) return rc;
  int block = 0, vpt = 0;
  rc = row_launch(d, lg, opts, &block, &vpt);
  if (rc) return rc;
  if (t == 0) return ARFUSE_OK;  // no-op: buffers are never touched, may be NULL
  // the split exchange (sums of squares) needs the workspace; the all-reduce
  // alone has no norm and splits without one
  void* workspace = (opts && lg != 0 && epi != 0) ? opts->workspace : nullptr;
  if (lg != 0 && epi != 0 && (!workspace || !aligned16(workspace))) return ARFUSE_ERR_INVALID_ARG;
  if (!partials) return ARFUSE_ERR_INVALID_ARG;
  if ((fp4_out == nullptr) != (fp4_scales == nullptr)) return ARFUSE_ERR_INVALID_ARG;
  if (epi != 0 && !gamma) return ARFUSE_ERR_INVALID_ARG;  // norm outputs need gamma
  if (epi == 0 && !residual_out) return ARFUSE_ERR_INVALID_ARG;  // nothing to write
  if ((residual && !aligned16(residual)) || (gamma && !aligned16(gamma)) ||
      (residual_out && !aligned16(residual_out)) || (out && !aligned16(out)) ||
      (fp4_out && !aligned16(fp4_out)) || (fp8_out && !aligned16(fp8_out)))
    return ARFUSE_ERR_INVALID_ARG;
  const int64_t plane = t * d * 2;                // one bf16 [t][d]
  const int64_t pbytes = ll ? 2 * plane : plane;  // one partial
  Range in[ARFUSE_MAX_PARTIALS + 2];
  int nin = 0;
  for (int i = 0; i < n; ++i) {
    if (!partials[i] || !aligned16(partials[i])) return ARFUSE_ERR_INVALID_ARG;
    in[nin++] = range_of(partials[i], pbytes);
  }
  if (gamma && epi != 0) in[nin++] = range_of(gamma, d * 4);
  Range outs[7 + ARFUSE_MAX_PARTIALS];
  int nout = 0;
  const bool rout_first = residual_out != nullptr;
  if (residual_out) outs[nout++] = range_of(residual_out, plane);
  if (out) outs[nout++] = range_of(out, plane);
  if (fp4_out) {
    outs[nout++] = range_of(fp4_out, t * d / 2);
    outs[nout++] = range_of(fp4_scales, t * d / 16);
  }
  if (fp8_out) outs[nout++] = range_of(fp8_out, t * d);
  const int64_t prows = split_rows(t, lg);
  if ((prows << lg) > ARFUSE_MAX_SPLIT_BLOCKS && lg) return ARFUSE_ERR_UNSUPPORTED;
  if (workspace) outs[nout++] = range_of(workspace, split_ws_bytes(t, lg));
  arfuse_ll_status* status = opts ? opts->status : nullptr;
  if (status) {  // written by device atomics: 8-byte aligned, shared with nothing
    if ((uintptr_t)status & 7u) return ARFUSE_ERR_INVALID_ARG;
    outs[nout++] = range_of(status, (int64_t)sizeof(arfuse_ll_status));
  }
  if (reset) {
    for (int i = 0; i < n; ++i) {
      if (!reset[i] || !aligned16(reset[i])) return ARFUSE_ERR_INVALID_ARG;
      outs[nout++] = range_of(reset[i], plane);
    }
  }
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o], in[i])) return ARFUSE_ERR_INVALID_ARG;
    for (int p = o + 1; p < nout; ++p)
      if (overlap(outs[o], outs[p])) return ARFUSE_ERR_INVALID_ARG;
    if (residual) {
      // residual_out may be residual itself (in place), nothing else may overlap it
      const Range rres = range_of(residual, plane);
      if (o == 0 && rout_first) {
        if (outs[0].lo != rres.lo && overlap(outs[0], rres)) return ARFUSE_ERR_INVALID_ARG;
      } else if (overlap(outs[o], rres)) {
        return ARFUSE_ERR_INVALID_ARG;
      }
    }
  }

  // A call that can wait (the arrival checks of the LL and sentinel layouts,
  // a split row's exchange of its sum of squares) gives up after a bounded
  // wait and then leaves rows unspecified; the status word is the only place
  // that says so, so such a call must have one.
  const bool waits = ll || sentinel || (lg != 0 && epi != 0);
  if (waits && !status) return ARFUSE_ERR_INVALID_ARG;

  RowArgs a = {};
  for (int i = 0; i < n; ++i) a.part[i] = (const u32x4*)partials[i];
  if (reset)
    for (int i = 0; i < n; ++i) a.reset[i] = (u32x4*)reset[i];
  a.residual = (const u32x4*)residual;
  a.gamma = (const f32x4*)gamma;
  a.out = (u32x4*)out;
  a.residual_out = (u32x4*)residual_out;
  a.codes = (uint32_t*)fp4_out;
  a.scales = fp4_scales;
  a.fp8 = fp8_out;
  a.status = opts ? opts->status : nullptr;
  a.d8 = d / 8;
  a.ll_flag = opts ? opts->ll_flag : 0;
  a.eps = eps;
  a.inv_d = 1.0 / (double)d;
  a.fp8_inv_scale = fp8_out ? opts->fp8_inv_scale : 1.0f;
  a.max_polls = opts ? opts->max_polls : 0;
  a.sentinel2 = spat | (spat << 16);
  const int64_t extra = reset_blocks(n, t, d, block, reset != nullptr);
  a.flags = (residual ? kHasResidual : 0u) | (residual_out ? kHasResidualOut : 0u) |
            ((reset && extra == 0) ? kReset : 0u);
  a.rows = (uint32_t)t;
  a.split_log2 = (uint32_t)lg;
  a.ds8 = (uint32_t)((d / 8) >> lg);
  a.ws = (u32x4*)workspace;
  a.prows = (uint32_t)prows;
  a.plane_vecs = (uint32_t)(t * d / 8);  // only read by reset blocks: t <= 128
  a.reset_bpp = (uint32_t)((t * d / 8 + block - 1) / block);

  const void* fn = (const void*)select_row_kernel(n, vpt, layout, epi, row_kind(t, lg, vpt, layout));
  if (!fn) return ARFUSE_ERR_UNSUPPORTED;
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)((prows << lg) + extra)), dim3((unsigned)block), args, 0,
                                 (hipStream_t)stream);
  return launch_status(e);
}

// ------------------------------------------------------------ allocation-free calls

// The exchange slots of arfuse_rmsnorm_noalloc: the largest split call's
// (128 row positions, two 128-byte lines each), 32 KiB. Each GPU the library
// runs on holds its own copy from the library's load until the process ends.
// Host code never uses this name as an address (on the host it names a
// stand-in, not device memory): the device address is looked up per device
// with hipGetSymbolAddress (scratch_on).
constexpr int64_t kScratchBytes = ARFUSE_NOALLOC_BYTES;
static __device__ __align__(256) u32x4 scratch[kScratchBytes / 16];

// Device address of `scratch` per device, found once (with that device
// current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream). Allocates nothing.
int scratch_on(hipStream_t stream, void** addr) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return launch_status(e);
  if (dev < 0 || dev >= kMaxDevices) return ARFUSE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return launch_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return launch_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return launch_status(e);
    if (!p) return ARFUSE_ERR_LAUNCH;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return ARFUSE_OK;
}

}  // namespace
}  // namespace arfuse_detail

using namespace arfuse_detail;

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

int arfuse_rmsnorm_noalloc(const void* const* partials, int n_partials, const void* residual,
                           const float* gamma, float eps, void* out, void* residual_out,
                           uint8_t* fp4_out, uint8_t* fp4_scales, int64_t t, int64_t d,
                           void* stream, const arfuse_opts* opts) {
  // the library's static slots stand in for the caller's workspace
  if (opts && opts->workspace) return ARFUSE_ERR_INVALID_ARG;
  void* slots = nullptr;
  const int rc = scratch_on((hipStream_t)stream, &slots);
  if (rc) return rc;
  arfuse_opts o;
  if (opts)
    o = *opts;
  else
    memset(&o, 0, sizeof o);
  o.workspace = slots;
  // every split the library launches fits the slots: a split row has at
  // least 2 workgroups and t * split <= ARFUSE_MAX_SPLIT_BLOCKS, so at most
  // ARFUSE_MAX_SPLIT_BLOCKS / 2 row positions of 256 bytes
  static_assert(kScratchBytes >= ARFUSE_MAX_SPLIT_BLOCKS / 2 * 256, "scratch smaller than a split call");
  return rmsnorm_impl(partials, n_partials, residual, gamma, eps, out, residual_out, fp4_out,
                      fp4_scales, t, d, stream, &o);
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

int arfuse_quantize_fp4_ll(const float* y, int64_t t, int64_t d, uint8_t* codes, uint8_t* scales,
                           void* stream) {
  if (t < 0 || d <= 0 || d % 16) return ARFUSE_ERR_INVALID_ARG;
  if (t == 0) return ARFUSE_OK;
  if (!y || !codes || !scales) return ARFUSE_ERR_INVALID_ARG;
  if (!aligned16(y) || ((uintptr_t)codes & 1u)) return ARFUSE_ERR_INVALID_ARG;
  const Range ry = range_of(y, t * d * 4), rc = range_of(codes, t * d / 2),
              rs = range_of(scales, t * d / 16);
  if (overlap(ry, rc) || overlap(ry, rs) || overlap(rc, rs)) return ARFUSE_ERR_INVALID_ARG;
  const int64_t ngroups = t * (d / 4);
  const int64_t grid = (ngroups + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  const f32x4* yy = (const f32x4*)y;
  uint16_t* cc = (uint16_t*)codes;
  int64_t ng = ngroups;
  void* args[] = {&yy, &ng, &cc, &scales};
  hipError_t e = hipLaunchKernel((const void*)quant_ll_kernel, dim3((unsigned)grid), dim3(256),
                                 args, 0, (hipStream_t)stream);
  return launch_status(e);
}

int arfuse_stream_mix(const void* const* in, int n_in, void* const* out, int n_out, int64_t t,
                      int64_t d, void* stream) {
  if (n_in < 1 || n_in > kMixMaxIn || n_out < 1 || n_out > kMixMaxOut) return ARFUSE_ERR_INVALID_ARG;
  if (t < 0 || d <= 0 || d % 16) return ARFUSE_ERR_INVALID_ARG;
  if (d > ARFUSE_MAX_D || t > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  int block = 0, vpt = 0;
  int rc = choose_launch(d / 8, nullptr, &block, &vpt);
  if (rc) return rc;
  if (t == 0) return ARFUSE_OK;
  if (!in || !out) return ARFUSE_ERR_INVALID_ARG;
  const int64_t plane = t * d * 2;
  MixArgs a = {};
  for (int i = 0; i < n_in; ++i) {
    if (!in[i] || !aligned16(in[i])) return ARFUSE_ERR_INVALID_ARG;
    a.in[i] = (const u32x4*)in[i];
  }
  for (int o = 0; o < n_out; ++o) {
    if (!out[o] || !aligned16(out[o])) return ARFUSE_ERR_INVALID_ARG;
    for (int i = 0; i < n_in; ++i)
      if (overlap(range_of(out[o], plane), range_of(in[i], plane))) return ARFUSE_ERR_INVALID_ARG;
    for (int p = 0; p < o; ++p)
      if (overlap(range_of(out[o], plane), range_of(out[p], plane))) return ARFUSE_ERR_INVALID_ARG;
    a.out[o] = (u32x4*)out[o];
  }
  a.d8 = d / 8;
  a.n_in = n_in;
  a.n_out = n_out;
  const bool stream_stores = row_kind(t, 0, vpt, ARFUSE_LAYOUT_PLAIN) == kRowStream;
  const void* fn = nullptr;
  switch (vpt) {
    case 1: fn = stream_stores ? (const void*)mix_kernel<1, true> : (const void*)mix_kernel<1, false>; break;
    case 2: fn = stream_stores ? (const void*)mix_kernel<2, true> : (const void*)mix_kernel<2, false>; break;
    case 4: fn = stream_stores ? (const void*)mix_kernel<4, true> : (const void*)mix_kernel<4, false>; break;
    case 8: fn = stream_stores ? (const void*)mix_kernel<8, true> : (const void*)mix_kernel<8, false>; break;
  }
  if (!fn) return ARFUSE_ERR_UNSUPPORTED;
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)t), dim3((unsigned)block), args, 0,
                                 (hipStream_t)stream);
  return launch_status(e);
}

int arfuse_query_launch(int n_partials, int64_t t, int64_t d, int epilogue,
                        const arfuse_opts* opts, arfuse_launch_info* info) {
  if (!info) return ARFUSE_ERR_INVALID_ARG;
  int rc = check_shape(n_partials, t, d, epilogue);
  if (rc) return rc;
  if (opts && opts->layout != ARFUSE_LAYOUT_PLAIN && opts->layout != ARFUSE_LAYOUT_LL &&
      opts->layout != ARFUSE_LAYOUT_SENTINEL)
    return ARFUSE_ERR_INVALID_ARG;
  int lg = 0;
  rc = split_log2(opts, n_partials, t, d, epilogue, &lg);
  if (rc) return rc;
  int block = 0, vpt = 0;
  rc = row_launch(d, lg, opts, &block, &vpt);
  if (rc) return rc;
  const bool reset = opts && opts->layout == ARFUSE_LAYOUT_SENTINEL && opts->reset;
  info->grid = (split_rows(t, lg) << lg) + reset_blocks(n_partials, t, d, block, reset);
  info->block = block;
  info->vpt = vpt;
  info->split = 1 << lg;
  info->stream_stores = row_kind(t, lg, vpt, opts ? opts->layout : ARFUSE_LAYOUT_PLAIN) == kRowStream;
  info->workspace_bytes = split_ws_bytes(t, lg);
  return ARFUSE_OK;
}

int arfuse_launch_floor(int n_partials, int64_t t, int64_t d, int epilogue,
                        const arfuse_opts* opts, void* stream) {
  int rc = check_shape(n_partials, t, d, epilogue);
  if (rc) return rc;
  int lg = 0;
  rc = split_log2(opts, n_partials, t, d, epilogue, &lg);
  if (rc) return rc;
  int block = 0, vpt = 0;
  rc = row_launch(d, lg, opts, &block, &vpt);
  if (rc) return rc;
  if (t == 0) return ARFUSE_OK;
  const bool reset = opts && opts->layout == ARFUSE_LAYOUT_SENTINEL && opts->reset;
  const int64_t grid = (split_rows(t, lg) << lg) + reset_blocks(n_partials, t, d, block, reset);
  RowArgs a = {};
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel((const void*)floor_kernel, dim3((unsigned)grid), dim3((unsigned)block),
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

int arfuse_round_fp8(const float* x, int64_t n, uint8_t* out, void* stream) {
  if (n < 0 || n % 4) return ARFUSE_ERR_INVALID_ARG;
  if (n == 0) return ARFUSE_OK;
  if (!x || !out || !aligned16(x) || ((uintptr_t)out & 3u)) return ARFUSE_ERR_INVALID_ARG;
  if (overlap(range_of(x, n * 4), range_of(out, n))) return ARFUSE_ERR_INVALID_ARG;
  const int64_t nquads = n / 4;
  const int64_t grid = (nquads + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  const f32x4* xx = (const f32x4*)x;
  uint32_t* oo = (uint32_t*)out;
  int64_t nq = nquads;
  void* args[] = {&xx, &nq, &oo};
  hipError_t e = hipLaunchKernel((const void*)round_fp8_kernel, dim3((unsigned)grid), dim3(256),
                                 args, 0, (hipStream_t)stream);
  return launch_status(e);
}

int arfuse_round_fp4(const float* x, int64_t n, uint8_t* out, void* stream) {
  if (n < 0 || n % 2) return ARFUSE_ERR_INVALID_ARG;
  if (n == 0) return ARFUSE_OK;
  if (!x || !out || ((uintptr_t)x & 7u)) return ARFUSE_ERR_INVALID_ARG;
  if (overlap(range_of(x, n * 4), range_of(out, n / 2))) return ARFUSE_ERR_INVALID_ARG;
  const int64_t npairs = n / 2;
  const int64_t grid = (npairs + 255) / 256;
  if (grid > 0x7FFFFFFFLL) return ARFUSE_ERR_UNSUPPORTED;
  const f32x2* xx = (const f32x2*)x;
  int64_t np = npairs;
  void* args[] = {&xx, &np, &out};
  hipError_t e = hipLaunchKernel((const void*)round_fp4_kernel, dim3((unsigned)grid), dim3(256),
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
