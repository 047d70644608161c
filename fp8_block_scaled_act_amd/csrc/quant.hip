// Dynamic FP8 (e4m3) quantization kernels for gfx950 and their C entry points.
//
//  * fp8_act_quant_block: one fp32 scale per 1x128 block (DeepSeek-V3
//    act_quant, "How to Profile DeepSeek-V3 Inference Kernels Using Triton
//    Autotuning", section "Benchmarking the Activation Quantization Kernel").
//  * fp8_amax_quant_tensor: one scale from the exact amax over the tensor,
//    with a grid that grows with the input and no single-address atomic
//    (TensorRT-LLM PR "Size the per-tensor FP8 dynamic-quant amax grid to the
//    input", sections "Description" and "Correctness").
//  * fp8_weight_quant_block: one scale per 128x128 weight block.
//
// Rule for a group: amax = max|x|, s = fl32(amax/448), q = e4m3(clamp(x/s)).
// All three are HBM-bound streams: 16-byte loads, reductions in registers via
// DPP, no LDS on the block path.
#include "device_common.h"
#include "host_common.h"

namespace fp8bs {
namespace {

constexpr int kThreads = 256;

// A load that marks its cache lines as streamed (read once), for inputs that
// no later pass of the same call reads again.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// 1x128 blocks. Eight lanes own one block: lane `sub` holds elements
// [8*sub, 8*sub+8) and [64+8*sub, 64+8*sub+8), so each 16-byte load
// instruction of a wave reads eight whole 128-byte halves of blocks. The
// block amax is a 3-step DPP max inside the 8-lane group.
// ---------------------------------------------------------------------------

// Power-of-two scale (the ue8m0 variants): the smallest 2^e >= amax/448 with
// e >= -127, read off amax's bits (amax > 0). With amax = m * 2^E, m in [1, 2)
// and 448 = 1.75 * 2^8: e = E - 8 if m <= 1.75, else E - 7; subnormal amax
// (below 2^-126) gives e < -127, so -127. Also r = 2^-e (e <= 120 for bf16
// inputs, so r is a normal float): x / s is then the exact product x * r,
// rounded only where it leaves the normal range, like the division.
__device__ __forceinline__ void pow2_scale(float amax, float& s, float& r) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = static_cast<int>((b >> 23) & 0xFFu);
  int e = ef == 0 ? -127 : ef - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  e = e < -127 ? -127 : e;
  s = e >= -126 ? __uint_as_float(static_cast<uint32_t>(e + 127) << 23) : __uint_as_float(0x00400000u);
  r = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

__device__ __forceinline__ uint2 quant8_pow2(const uint4 v, float r) {
  float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] *= r;
  return make_uint2(pack4_e4m3(f[0], f[1], f[2], f[3]), pack4_e4m3(f[4], f[5], f[6], f[7]));
}

// P2: power-of-two scales (ue8m0) instead of amax/448
template <bool P2>
__global__ __launch_bounds__(kThreads) void act_quant_block_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, float* __restrict__ scale,
    int64_t nblocks) {
  const int64_t blk = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 3;
  const int sub = threadIdx.x & 7;
  if (blk >= nblocks) return;  // whole 8-lane groups leave together

  // streamed loads: x is read once (rotated inputs, alternating runs: prefill
  // 17.4-18.0 -> 16.2 us, large-M 19.3 -> 18.1-18.2 us; the same loads in the
  // float32-input kernel, and in the block kernel of the one-call block and
  // per-tensor quant, whose second pass re-reads x, were slower)
  const uint4 v0 = load_nt(x + blk * 16 + sub);
  const uint4 v1 = load_nt(x + blk * 16 + 8 + sub);

  float s;
  uint2 o0, o1;
  if constexpr (P2) {
    float m = 0.0f;
    m = absmax2(v0.x, m); m = absmax2(v0.y, m); m = absmax2(v0.z, m); m = absmax2(v0.w, m);
    m = absmax2(v1.x, m); m = absmax2(v1.y, m); m = absmax2(v1.z, m); m = absmax2(v1.w, m);
    const float amax = group8_max(m);
    float r;
    pow2_scale(amax, s, r);
    o0 = quant8_pow2(v0, r);
    o1 = quant8_pow2(v1, r);
    if (amax == 0.0f) {  // all-zero block: scale 0, codes 0x00
      s = 0.0f;
      o0 = make_uint2(0u, 0u);
      o1 = make_uint2(0u, 0u);
    }
  } else {
    s = quant_block_bf16(v0, v1, o0, o1);
  }
  q[blk * 16 + sub] = o0;
  q[blk * 16 + 8 + sub] = o1;
  if (sub == 0) scale[blk] = s;
}

// float32 input: eight lanes per 1x128 block (512 bytes), lane `sub` holding
// the float4 chunks sub, sub+8, sub+16 and sub+24, so each 16-byte load of a
// wave reads eight whole 128-byte quarters of blocks. The quotient is the
// IEEE division: the reciprocal-based form used for bf16 inputs is proven
// exact only for 8-bit significands.
__global__ __launch_bounds__(kThreads) void act_quant_block_f32_kernel(
    const float4* __restrict__ x, uint32_t* __restrict__ q, float* __restrict__ scale, int64_t nblocks) {
  const int64_t blk = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 3;
  const int sub = threadIdx.x & 7;
  if (blk >= nblocks) return;  // whole 8-lane groups leave together
  float4 v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = x[blk * 32 + sub + 8 * c];
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    m = fmaxf(fmaxf(fmaxf(m, fabsf(v[c].x)), fmaxf(fabsf(v[c].y), fabsf(v[c].z))), fabsf(v[c].w));
  const float amax = group8_max(m);
  const float s = div_ieee(amax, kE4m3Max);
  const bool zero = amax == 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t o = pack4_e4m3(div_ieee(v[c].x, s), div_ieee(v[c].y, s), div_ieee(v[c].z, s), div_ieee(v[c].w, s));
    q[blk * 32 + sub + 8 * c] = zero ? 0u : o;
  }
  if (sub == 0) scale[blk] = s;
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: one workgroup per block. Thread t covers row t/2,
// columns [64*(t%2), 64*(t%2)+64) as 8 uint4.
// ---------------------------------------------------------------------------
template <bool P2>
__global__ __launch_bounds__(kThreads) void weight_quant_block_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ q, float* __restrict__ scale,
    int64_t K) {
  __shared__ float wave_max_lds[kThreads / 64];
  const int64_t kb = K / 128;
  const int64_t bn = blockIdx.y, bk = blockIdx.x;
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t base = (bn * 128 + row) * K + bk * 128 + half * 64;
  const uint4* src = reinterpret_cast<const uint4*>(w + base);
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = src[i];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = absmax2(v[i].x, m); m = absmax2(v[i].y, m);
    m = absmax2(v[i].z, m); m = absmax2(v[i].w, m);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wave_max_lds[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wave_max_lds[0], wave_max_lds[1]),
                           fmaxf(wave_max_lds[2], wave_max_lds[3]));
  float s;
  uint2 o[8];
  if constexpr (P2) {
    float r;
    pow2_scale(amax, s, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = quant8_pow2(v[i], r);
  } else {
    s = div_ieee(amax, kE4m3Max);
    if (s >= kFastScaleMin) {  // uniform across the workgroup
      const float r = div_ieee(1.0f, s);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = quant8<true>(v[i], s, r);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = quant8<false>(v[i], s, 0.0f);
    }
  }
  if (amax == 0.0f) {
    s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_uint2(0u, 0u);
  }
  uint4* dst = reinterpret_cast<uint4*>(q + base);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dst[i] = make_uint4(o[2 * i].x, o[2 * i].y, o[2 * i + 1].x, o[2 * i + 1].y);
  if (threadIdx.x == 0) scale[bn * kb + bk] = s;
}

// ---------------------------------------------------------------------------
// Per-tensor quantization.
//
// Small inputs (numel <= kSmallNumel): one workgroup of 1024 threads reads
// the tensor for the amax, reduces in LDS, then quantizes (the second read
// hits L2). Mid-size inputs (numel <= kMidNumel): one launch too, with
// several workgroups that each read the whole tensor for the amax (from L2
// after the first reader on each XCD) and then quantize their own share;
// the amax is exact and order-free, so every workgroup finds the same one
// and no partial maxima cross workgroups (graph-replayed, against the two
// launches below: 32768 elements 3.9 against 4.9 us, 65536 elements 4.3
// against 5.0 us; at 98304 elements the workgroup's read of the whole tensor
// makes it slower, 5.4 against 4.9 us). Large inputs: stage 1 writes one
// partial max per workgroup to the workspace (grid sized to numel, capped),
// stage 2 has every workgroup reduce those partials itself before quantizing
// its share; workgroup 0 writes the scale. No atomics, deterministic. Stage
// 2 writes the codes with non-temporal stores, which keep them from pushing
// the input out of the last-level cache before stage 2 has read it
// (measured: 141 -> 116 us on a 256 MiB tensor, larger than that cache).
// ---------------------------------------------------------------------------
constexpr int64_t kSmallNumel = 1 << 14;
constexpr int64_t kMidNumel = 1 << 16;
constexpr int kMaxPartials = 1024;
constexpr int kSmallThreads = 1024;
// uint4 per thread in flight in a mid-size workgroup's read of the whole
// tensor, and uint4 (8 elements) per workgroup in its share of the codes
constexpr int kMidVec = 8;
constexpr int kMidShare = 1024;
// uint4 (8 bf16) per thread per iteration of the amax pass: 4 with up to
// four workgroups per CU, 8 with one workgroup per CU for inputs whose
// 4-deep grid would exceed four workgroups per CU (256 MiB: 47.3 -> 40.8 us
// for the amax stage alone, 110.4 -> 103.7 us for the quantization; 16 Mi
// elements: 10.1 -> 9.3 / 19.2 -> 17.2 us; below that, fewer and deeper
// workgroups were slower: 4.2 -> 4.8 us at 131072 elements)
constexpr int kVecPerThread = 4;
constexpr int kVecDeep = 8;
// uint4 per thread per iteration of the apply pass (the codes' stores follow
// each iteration's loads; amax and apply passes over 256 MiB: 113.4 us with
// 2 in flight, 114.9 with 4)
constexpr int kApplyVec = 2;

__device__ __forceinline__ float tail_absmax(const uint16_t* x, int64_t begin, int64_t end, float m) {
  for (int64_t i = begin; i < end; ++i)
    m = fmaxf(m, fabsf(__uint_as_float(static_cast<uint32_t>(x[i]) << 16)));
  return m;
}

template <bool kFast>
__device__ __forceinline__ void tail_quant(const uint16_t* x, uint8_t* q, int64_t begin,
                                           int64_t end, float s, float r, bool zero) {
  for (int64_t i = begin; i < end; ++i) {
    const float f = __uint_as_float(static_cast<uint32_t>(x[i]) << 16);
    const float y = kFast ? div_by_scale(f, s, r) : div_ieee(f, s);
    const uint32_t c = pack4_e4m3(y, 0.0f, 0.0f, 0.0f) & 0xFFu;
    q[i] = zero ? 0 : static_cast<uint8_t>(c);
  }
}

template <int kBlock>
__device__ __forceinline__ float block_max(float m, float* lds) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) r = fmaxf(r, lds[i]);
  return r;
}

template <bool kFast>
__device__ __forceinline__ void quant_range(const uint4* xv, uint2* qv, int64_t nvec,
                                            int64_t first, int64_t stride, float s, float r,
                                            bool zero) {
  for (int64_t i = first; i < nvec; i += stride) {
    uint2 o = quant8<kFast>(xv[i], s, r);
    if (zero) o = make_uint2(0u, 0u);
    qv[i] = o;
  }
}

typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(uint2 v, uint2* p) {
  const u32x2_nt w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_nt*>(p));
}

// the same with kApplyVec vectors per thread in flight, the codes
// stored non-temporally, and the tensor walked from its end: the first pass
// walked it from the start, so the last-level cache holds its most recently
// read part, which this pass then reads first (when the input is larger
// than that cache, a walk in the same order would find every line evicted)
// pre: the thread's first kApplyVec vectors (i = first + j*stride),
// loaded by the caller (each index clamped to the tensor, so the loads are
// unconditional); those past the end are not stored
template <bool kFast>
__device__ __forceinline__ void quant_range_nt(const uint4* xv, uint2* qv, int64_t nvec,
                                                int64_t first, int64_t stride, float s, float r,
                                                bool zero, const uint4 (&pre)[kApplyVec]) {
#pragma unroll
  for (int j = 0; j < kApplyVec; ++j) {
    const int64_t i = first + j * stride;
    if (i < nvec) {
      uint2 o = quant8<kFast>(pre[j], s, r);
      if (zero) o = make_uint2(0u, 0u);
      store_nt(o, qv + nvec - 1 - i);
    }
  }
  int64_t i = first + kApplyVec * stride;
  for (; i + (kApplyVec - 1) * stride < nvec; i += kApplyVec * stride) {
    uint4 v[kApplyVec];
#pragma unroll
    for (int j = 0; j < kApplyVec; ++j) v[j] = xv[nvec - 1 - (i + j * stride)];
#pragma unroll
    for (int j = 0; j < kApplyVec; ++j) {
      uint2 o = quant8<kFast>(v[j], s, r);
      if (zero) o = make_uint2(0u, 0u);
      store_nt(o, qv + nvec - 1 - (i + j * stride));
    }
  }
  for (; i < nvec; i += stride) {
    uint2 o = quant8<kFast>(xv[nvec - 1 - i], s, r);
    if (zero) o = make_uint2(0u, 0u);
    store_nt(o, qv + nvec - 1 - i);
  }
}

__global__ __launch_bounds__(kSmallThreads) void tensor_quant_small_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale,
    int64_t numel) {
  __shared__ float lds[kSmallThreads / 64];
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nvec = numel >> 3;
  float m = 0.0f;
  // at most kSmallNumel / 8 / kSmallThreads = 2 vectors per thread: both in flight
  static_assert(kSmallNumel / 8 <= 2 * kSmallThreads, "small path: two vectors per thread");
  const int64_t i0 = threadIdx.x, i1 = threadIdx.x + kSmallThreads;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  const uint4 v0 = i0 < nvec ? xv[i0] : z;
  const uint4 v1 = i1 < nvec ? xv[i1] : z;
  m = absmax2(v0.x, m); m = absmax2(v0.y, m); m = absmax2(v0.z, m); m = absmax2(v0.w, m);
  m = absmax2(v1.x, m); m = absmax2(v1.y, m); m = absmax2(v1.z, m); m = absmax2(v1.w, m);
  if (threadIdx.x == 0) m = tail_absmax(x, nvec << 3, numel, m);
  const float amax = block_max<kSmallThreads>(m, lds);
  const float s = div_ieee(amax, kE4m3Max);
  const bool zero = amax == 0.0f;
  uint2* qv = reinterpret_cast<uint2*>(q);
  if (s >= kFastScaleMin) {
    const float r = div_ieee(1.0f, s);
    quant_range<true>(xv, qv, nvec, threadIdx.x, kSmallThreads, s, r, zero);
    if (threadIdx.x == 0) tail_quant<true>(x, q, nvec << 3, numel, s, r, zero);
  } else {
    quant_range<false>(xv, qv, nvec, threadIdx.x, kSmallThreads, s, 0.0f, zero);
    if (threadIdx.x == 0) tail_quant<false>(x, q, nvec << 3, numel, s, 0.0f, zero);
  }
  if (threadIdx.x == 0) scale[0] = s;
}

// The exact absolute maximum over the whole tensor, by one workgroup of
// kSmallThreads threads with kVec vectors per thread in flight; every thread
// gets the result.
template <int kVec>
__device__ __forceinline__ float workgroup_absmax(const uint16_t* x, int64_t numel, float* lds) {
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nvec = numel >> 3;
  float m = 0.0f;
  int64_t i = threadIdx.x;
  for (; i + (kVec - 1) * kSmallThreads < nvec; i += kVec * kSmallThreads) {
    uint4 v[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) v[j] = xv[i + j * kSmallThreads];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      m = absmax2(v[j].x, m); m = absmax2(v[j].y, m);
      m = absmax2(v[j].z, m); m = absmax2(v[j].w, m);
    }
  }
  for (; i < nvec; i += kSmallThreads) {
    const uint4 v = xv[i];
    m = absmax2(v.x, m); m = absmax2(v.y, m); m = absmax2(v.z, m); m = absmax2(v.w, m);
  }
  if (threadIdx.x == 0) m = tail_absmax(x, nvec << 3, numel, m);
  return block_max<kSmallThreads>(m, lds);
}

// Mid-size inputs: workgroup b quantizes vectors [b*share, (b+1)*share) after
// its own read of the whole tensor for the amax; workgroup 0 also does the
// elements past the last whole vector and writes the scale.
__global__ __launch_bounds__(kSmallThreads) void tensor_quant_mid_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale, int64_t numel,
    int64_t share) {
  __shared__ float lds[kSmallThreads / 64];
  const float amax = workgroup_absmax<kMidVec>(x, numel, lds);
  const float s = div_ieee(amax, kE4m3Max);
  const bool zero = amax == 0.0f;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  const int64_t nvec = numel >> 3;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * share;
  const int64_t hi = min(lo + share, nvec);
  const bool head = blockIdx.x == 0 && threadIdx.x == 0;
  if (s >= kFastScaleMin) {
    const float r = div_ieee(1.0f, s);
    quant_range<true>(xv, qv, hi, lo + threadIdx.x, kSmallThreads, s, r, zero);
    if (head) tail_quant<true>(x, q, nvec << 3, numel, s, r, zero);
  } else {
    quant_range<false>(xv, qv, hi, lo + threadIdx.x, kSmallThreads, s, 0.0f, zero);
    if (head) tail_quant<false>(x, q, nvec << 3, numel, s, 0.0f, zero);
  }
  if (head) scale[0] = s;
}

// kStream: streamed loads, for the amax stage alone (45.4 against 47.8 us
// over 256 MiB); the quantization's first pass does not stream, because its
// second pass re-reads the tensor and finds part of it in the last-level
// cache only if the first pass left it there.
template <bool kStream, int kVec>
__global__ __launch_bounds__(kThreads) void tensor_amax_partial_kernel(
    const uint16_t* __restrict__ x, float* __restrict__ partial, int64_t numel) {
  __shared__ float lds[kThreads / 64];
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nvec = numel >> 3;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  float m = 0.0f;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kVec - 1) * stride < nvec; i += kVec * stride) {
    uint4 v[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) v[j] = kStream ? load_nt(xv + i + j * stride) : xv[i + j * stride];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      m = absmax2(v[j].x, m); m = absmax2(v[j].y, m);
      m = absmax2(v[j].z, m); m = absmax2(v[j].w, m);
    }
  }
  for (; i < nvec; i += stride) {
    const uint4 v = xv[i];
    m = absmax2(v.x, m); m = absmax2(v.y, m); m = absmax2(v.z, m); m = absmax2(v.w, m);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) m = tail_absmax(x, nvec << 3, numel, m);
  m = block_max<kThreads>(m, lds);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void tensor_apply_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale,
    const float* __restrict__ partial, int npartial, int64_t numel) {
  __shared__ float lds[kThreads / 64];
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  const int64_t nvec = numel >> 3;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  // The first iteration's vectors go out before the partial maxima are read,
  // so that their latency overlaps the reduction of the partials (which the
  // quantization needs first). Unconditional loads at clamped indices: a
  // conditional one would be sunk by the compiler to its use, after the
  // partials.
  uint4 pre[kApplyVec];
#pragma unroll
  for (int j = 0; j < kApplyVec; ++j) {
    const int64_t idx = nvec - 1 - (first + j * stride);
    pre[j] = xv[idx > 0 ? idx : 0];
  }
  __builtin_amdgcn_sched_barrier(0);
  float m = 0.0f;
  for (int i = threadIdx.x; i < npartial; i += kThreads) m = fmaxf(m, partial[i]);
  const float amax = block_max<kThreads>(m, lds);
  const float s = div_ieee(amax, kE4m3Max);
  const bool zero = amax == 0.0f;
  const bool head = blockIdx.x == 0 && threadIdx.x == 0;
  if (s >= kFastScaleMin) {
    const float r = div_ieee(1.0f, s);
    quant_range_nt<true>(xv, qv, nvec, first, stride, s, r, zero, pre);
    if (head) tail_quant<true>(x, q, nvec << 3, numel, s, r, zero);
  } else {
    quant_range_nt<false>(xv, qv, nvec, first, stride, s, 0.0f, zero, pre);
    if (head) tail_quant<false>(x, q, nvec << 3, numel, s, 0.0f, zero);
  }
  if (head) scale[0] = s;
}

// Quantization with a given scale (fp8_static_quant_tensor): s read from
// device memory, a zero scale giving 0x00 codes, the quotient by IEEE
// division (the three-operation form is proven only for scales of the form
// fl32(amax / 448) with a bf16 amax). One-shot grid sized to numel:
// workgroup b takes the 512 vectors from 512 b, thread t the vectors
// 512 b + t and 512 b + 256 + t, both loads issued before either store;
// workgroup 0's thread 0 also does the elements past the last whole vector.
// Measured against a grid-stride loop (four to eight workgroups per CU, two
// vectors in flight per thread): 256 MiB of x 78.6 -> 70.1 us, 64 MiB
// 20.1 -> 18.1 us, 4 MiB 3.5 -> 3.3 us; four vectors per thread or one were
// no faster. kNt: non-temporal code stores, for inputs of at least 256 MiB
// (67.7 against 70.1 us there; 18.8 against 18.1 us at 64 MiB, where the
// codes still fit the last-level cache beside x and a GEMM reads them next).
template <bool kNt>
__global__ __launch_bounds__(kThreads) void tensor_static_quant_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, const float* __restrict__ scale, int64_t numel) {
  const float s = scale[0];
  const bool zero = s == 0.0f;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  const int64_t nvec = numel >> 3;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * (2 * kThreads) + threadIdx.x;
  const int64_t i1 = i0 + kThreads;
  auto put = [&](uint2 o, int64_t i) {
    if (zero) o = make_uint2(0u, 0u);
    if constexpr (kNt)
      store_nt(o, qv + i);
    else
      qv[i] = o;
  };
  if (i1 < nvec) {
    const uint4 v0 = xv[i0];
    const uint4 v1 = xv[i1];
    put(quant8<false>(v0, s, 0.0f), i0);
    put(quant8<false>(v1, s, 0.0f), i1);
  } else if (i0 < nvec) {
    put(quant8<false>(xv[i0], s, 0.0f), i0);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) tail_quant<false>(x, q, nvec << 3, numel, s, 0.0f, zero);
}
// inputs from this many elements (256 MiB of bf16) store their codes non-temporally
constexpr int64_t kStaticNtNumel = int64_t{1} << 27;

// The amax stage alone (fp8_amax_tensor): the exact amax and the scale.
// Large inputs: tensor_amax_partial_kernel, then one workgroup reduces the
// partial maxima; small and mid-size inputs: one 1024-thread workgroup reads
// everything (65536 elements: 3.5 against 4.2 us for the two launches).
__global__ __launch_bounds__(kThreads) void tensor_amax_final_kernel(const float* __restrict__ partial,
                                                                     int npartial, float* __restrict__ amax_out,
                                                                     float* __restrict__ scale) {
  __shared__ float lds[kThreads / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < npartial; i += kThreads) m = fmaxf(m, partial[i]);
  const float amax = block_max<kThreads>(m, lds);
  if (threadIdx.x == 0) {
    amax_out[0] = amax;
    scale[0] = div_ieee(amax, kE4m3Max);
  }
}

__global__ __launch_bounds__(kSmallThreads) void tensor_amax_small_kernel(const uint16_t* __restrict__ x,
                                                                          int64_t numel, float* __restrict__ amax_out,
                                                                          float* __restrict__ scale) {
  __shared__ float lds[kSmallThreads / 64];
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t nvec = numel >> 3;
  const int64_t i0 = threadIdx.x, i1 = threadIdx.x + kSmallThreads;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  const uint4 v0 = i0 < nvec ? xv[i0] : z;
  const uint4 v1 = i1 < nvec ? xv[i1] : z;
  float m = 0.0f;
  m = absmax2(v0.x, m); m = absmax2(v0.y, m); m = absmax2(v0.z, m); m = absmax2(v0.w, m);
  m = absmax2(v1.x, m); m = absmax2(v1.y, m); m = absmax2(v1.z, m); m = absmax2(v1.w, m);
  if (threadIdx.x == 0) m = tail_absmax(x, nvec << 3, numel, m);
  const float amax = block_max<kSmallThreads>(m, lds);
  if (threadIdx.x == 0) {
    amax_out[0] = amax;
    scale[0] = div_ieee(amax, kE4m3Max);
  }
}

// the amax stage alone for mid-size inputs: one workgroup, eight loads per
// thread in flight
__global__ __launch_bounds__(kSmallThreads) void tensor_amax_mid_kernel(const uint16_t* __restrict__ x,
                                                                        int64_t numel, float* __restrict__ amax_out,
                                                                        float* __restrict__ scale) {
  __shared__ float lds[kSmallThreads / 64];
  const float amax = workgroup_absmax<kMidVec>(x, numel, lds);
  if (threadIdx.x == 0) {
    amax_out[0] = amax;
    scale[0] = div_ieee(amax, kE4m3Max);
  }
}

// ---------------------------------------------------------------------------
// Block and per-tensor quantization of the same X (both quantize the
// activation of the large-M workload): the block kernel above, with
// 1024-thread workgroups that also write the max of their 128 block maxima,
// is the per-tensor amax's first pass, so X is read twice rather than three
// times; the second pass is tensor_apply_kernel over those partials.
// ---------------------------------------------------------------------------
constexpr int kBTThreads = 1024;

__global__ __launch_bounds__(kBTThreads) void act_quant_block_partial_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ partial, int64_t nblocks) {
  __shared__ float lds[kBTThreads / 64];
  const int64_t blk = (static_cast<int64_t>(blockIdx.x) * kBTThreads + threadIdx.x) >> 3;
  const int sub = threadIdx.x & 7;
  float amax = 0.0f;
  if (blk < nblocks) {   // whole 8-lane groups
    const uint4 v0 = x[blk * 16 + sub];
    const uint4 v1 = x[blk * 16 + 8 + sub];
    uint2 o0, o1;
    const float s = quant_block_bf16(v0, v1, o0, o1, amax);
    q[blk * 16 + sub] = o0;
    q[blk * 16 + 8 + sub] = o1;
    if (sub == 0) scale[blk] = s;
  }
  amax = block_max<kBTThreads>(amax, lds);
  if (threadIdx.x == 0) partial[blockIdx.x] = amax;
}

int64_t block_tensor_partials(int64_t M, int64_t K) {
  return (M * (K / 128) * 8 + kBTThreads - 1) / kBTThreads;
}

// Grid of the amax pass (= its number of partial maxima, at most
// kMaxPartials) and whether it runs the deep form (kVecDeep vectors per
// thread, one workgroup per CU)
struct TensorGrid {
  int g;
  bool deep;
};
TensorGrid tensor_grid(int64_t numel, int num_cus) {
  const int64_t nvec = (numel >> 3) + 1;
  const int64_t per_wg = static_cast<int64_t>(kThreads) * kVecPerThread;
  const int64_t g = (nvec + per_wg - 1) / per_wg;
  if (g > 4LL * num_cus) return {static_cast<int>(std::min<int64_t>(kMaxPartials, num_cus)), true};
  return {static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kMaxPartials, g))), false};
}
// Grid of the apply pass: up to 8 workgroups per CU, 4 once each thread
// would take more than 8 vectors at 8 (256 MiB: 105.7 -> 99.6 us for the
// quantization; 16 Mi elements: 17.3 against 17.7 us with 8)
int64_t apply_grid(int64_t numel, int num_cus) {
  const int64_t nvec = (numel >> 3) + 1;
  const int64_t ga = (nvec + kThreads * kApplyVec - 1) / (kThreads * kApplyVec);
  const int64_t per_cu = nvec > 8LL * num_cus * kThreads * 8 ? 4 : 8;
  return std::min<int64_t>(ga, per_cu * num_cus);
}
template <bool kStream>
void launch_amax_partial(const TensorGrid& tg, const uint16_t* x, float* partial, int64_t numel, hipStream_t st) {
  if (tg.deep)
    hipLaunchKernelGGL((tensor_amax_partial_kernel<kStream, kVecDeep>), dim3(tg.g), dim3(kThreads), 0, st, x,
                       partial, numel);
  else
    hipLaunchKernelGGL((tensor_amax_partial_kernel<kStream, kVecPerThread>), dim3(tg.g), dim3(kThreads), 0, st, x,
                       partial, numel);
}

// ---------------------------------------------------------------------------
// test hook: elementwise fp32 -> e4m3 with the library's conversion
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void debug_encode_kernel(const float4* __restrict__ in,
                                                                uint32_t* __restrict__ out,
                                                                int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n4) return;
  const float4 v = in[i];
  out[i] = pack4_e4m3(v.x, v.y, v.z, v.w);
}

__global__ void debug_encode_tail_kernel(const float* __restrict__ in, uint8_t* __restrict__ out,
                                         int64_t begin, int64_t n) {
  const int64_t i = begin + threadIdx.x;
  if (i < n) out[i] = static_cast<uint8_t>(pack4_e4m3(in[i], 0.0f, 0.0f, 0.0f) & 0xFFu);
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" {

const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "FP8BS_OK";
    case FP8BS_ERR_NULL: return "FP8BS_ERR_NULL: a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "FP8BS_ERR_SHAPE: size out of range or not a multiple of 128";
    case FP8BS_ERR_ALIGN: return "FP8BS_ERR_ALIGN: pointer not aligned as documented";
    case FP8BS_ERR_WORKSPACE: return "FP8BS_ERR_WORKSPACE: workspace missing or too small";
    case FP8BS_ERR_DEVICE: return "FP8BS_ERR_DEVICE: no HIP device or device is not gfx950";
    case FP8BS_ERR_LAUNCH: return "FP8BS_ERR_LAUNCH: kernel launch failed";
    case FP8BS_ERR_INTERNAL: return "FP8BS_ERR_INTERNAL: a HIP runtime query needed for set-up failed";
    default: return "FP8BS_ERR_UNKNOWN";
  }
}

}  // extern "C"

namespace fp8bs {
namespace {
template <bool P2>
int act_quant_block(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, float* scale, void* stream) {
  if (!x_bf16 || !q_e4m3 || !scale) return FP8BS_ERR_NULL;
  if (M < 1 || K < 128 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (M > (INT64_MAX / K)) return FP8BS_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scale, 4)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  const int64_t nblocks = M * (K / 128);
  const int64_t grid = (nblocks * 8 + kThreads - 1) / kThreads;
  if (grid > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL((act_quant_block_kernel<P2>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     as_stream(stream), static_cast<const uint4*>(x_bf16), static_cast<uint2*>(q_e4m3),
                     scale, nblocks);
  return launch_status();
}

template <bool P2>
int weight_quant_block(const void* w_bf16, int64_t N, int64_t K, void* q_e4m3, float* scale, void* stream) {
  if (!w_bf16 || !q_e4m3 || !scale) return FP8BS_ERR_NULL;
  if (N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (N / 128 > 65535 || K / 128 > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scale, 4)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  (void)hipGetLastError();
  hipLaunchKernelGGL((weight_quant_block_kernel<P2>),
                     dim3(static_cast<unsigned>(K / 128), static_cast<unsigned>(N / 128)),
                     dim3(kThreads), 0, as_stream(stream), static_cast<const uint16_t*>(w_bf16),
                     static_cast<uint8_t*>(q_e4m3), scale, K);
  return launch_status();
}
}  // namespace
}  // namespace fp8bs

extern "C" {

int fp8_act_quant_block(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, float* scale,
                        void* stream) {
  return act_quant_block<false>(x_bf16, M, K, q_e4m3, scale, stream);
}

int fp8_act_quant_block_ue8m0(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, float* scale,
                              void* stream) {
  return act_quant_block<true>(x_bf16, M, K, q_e4m3, scale, stream);
}

int fp8_act_quant_block_f32(const float* x_f32, int64_t M, int64_t K, void* q_e4m3, float* scale,
                            void* stream) {
  if (!x_f32 || !q_e4m3 || !scale) return FP8BS_ERR_NULL;
  if (M < 1 || K < 128 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (M > (INT64_MAX / K)) return FP8BS_ERR_SHAPE;
  if (!aligned(x_f32, 16) || !aligned(q_e4m3, 16) || !aligned(scale, 4)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  const int64_t nblocks = M * (K / 128);
  const int64_t grid = (nblocks * 8 + kThreads - 1) / kThreads;
  if (grid > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(act_quant_block_f32_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     as_stream(stream), reinterpret_cast<const float4*>(x_f32), static_cast<uint32_t*>(q_e4m3),
                     scale, nblocks);
  return launch_status();
}

int fp8_weight_quant_block(const void* w_bf16, int64_t N, int64_t K, void* q_e4m3, float* scale,
                           void* stream) {
  return weight_quant_block<false>(w_bf16, N, K, q_e4m3, scale, stream);
}

int fp8_weight_quant_block_ue8m0(const void* w_bf16, int64_t N, int64_t K, void* q_e4m3, float* scale,
                                 void* stream) {
  return weight_quant_block<true>(w_bf16, N, K, q_e4m3, scale, stream);
}

size_t fp8_amax_quant_tensor_workspace_bytes(int64_t numel) {
  return numel > kMidNumel ? kMaxPartials * sizeof(float) : 0;
}

}  // extern "C"

namespace fp8bs {
namespace {
// The two launches of the per-tensor quantization (one for small and
// mid-size inputs);
// `partial` holds at least fp8_amax_quant_tensor_workspace_bytes(numel)
// bytes. Arguments are checked by the callers.
int amax_quant_tensor_launch(const void* x_bf16, int64_t numel, void* q_e4m3, float* scale, float* partial,
                             const DeviceInfo& dev, void* stream) {
  hipStream_t st = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_e4m3);
  (void)hipGetLastError();
  if (numel <= kSmallNumel) {
    hipLaunchKernelGGL(tensor_quant_small_kernel, dim3(1), dim3(kSmallThreads), 0, st, x, q, scale,
                       numel);
    return launch_status();
  }
  if (numel <= kMidNumel) {
    const int64_t nvec = numel >> 3;
    const int64_t g = std::min<int64_t>(dev.num_cus, (nvec + kMidShare - 1) / kMidShare);
    hipLaunchKernelGGL(tensor_quant_mid_kernel, dim3(static_cast<unsigned>(g)), dim3(kSmallThreads), 0, st, x, q,
                       scale, numel, (nvec + g - 1) / g);
    return launch_status();
  }
  const TensorGrid tg = tensor_grid(numel, dev.num_cus);
  const int g = tg.g;
  launch_amax_partial<false>(tg, x, partial, numel, st);
  if (hipGetLastError() != hipSuccess) return FP8BS_ERR_LAUNCH;
  const int64_t ga = apply_grid(numel, dev.num_cus);
  hipLaunchKernelGGL(tensor_apply_kernel, dim3(static_cast<unsigned>(ga)), dim3(kThreads), 0, st, x,
                     q, scale, partial, g, numel);
  return launch_status();
}

int amax_quant_tensor_check(const void* x_bf16, int64_t numel, void* q_e4m3, float* scale) {
  if (!x_bf16 || !q_e4m3 || !scale) return FP8BS_ERR_NULL;
  if (numel < 1) return FP8BS_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scale, 4)) return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}

// Scratch of the allocation-free per-tensor quantization: the partial maxima
// of its first pass, in a device array of the library's own (zero-filled
// when the code object loads, and only ever written before it is read, so
// nothing needs clearing). Host code never uses the array's name, which on
// the host is a stand-in and not a device address: it uses the address that
// hipGetSymbolAddress returns for the current device, looked up on the first
// call on each device and kept per device.
constexpr size_t kScratchBytes = kMaxPartials * sizeof(float);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

void* scratch_address(int* status) {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> addr[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    *status = FP8BS_ERR_DEVICE;
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      *status = FP8BS_ERR_INTERNAL;
      return nullptr;
    }
    addr[dev].store(p, std::memory_order_release);   // the same value from every thread
  }
  *status = FP8BS_OK;
  return p;
}
}  // namespace
}  // namespace fp8bs

extern "C" {

int fp8_amax_quant_tensor(const void* x_bf16, int64_t numel, void* q_e4m3, float* scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = amax_quant_tensor_check(x_bf16, numel, q_e4m3, scale);
  if (rc != FP8BS_OK) return rc;
  const size_t need = fp8_amax_quant_tensor_workspace_bytes(numel);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
  }
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  return amax_quant_tensor_launch(x_bf16, numel, q_e4m3, scale, static_cast<float*>(workspace), dev, stream);
}

int fp8_static_quant_tensor(const void* x_bf16, int64_t numel, const float* scale, void* q_e4m3,
                            void* stream) {
  if (!x_bf16 || !scale || !q_e4m3) return FP8BS_ERR_NULL;
  if (numel < 1 || numel >= (int64_t{1} << 42)) return FP8BS_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scale, 4)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  const int64_t g = std::max<int64_t>(1, ((numel >> 3) + 2 * kThreads - 1) / (2 * kThreads));
  if (g > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  (void)hipGetLastError();
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  uint8_t* q = static_cast<uint8_t*>(q_e4m3);
  if (numel >= kStaticNtNumel)
    hipLaunchKernelGGL(tensor_static_quant_kernel<true>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                       as_stream(stream), x, q, scale, numel);
  else
    hipLaunchKernelGGL(tensor_static_quant_kernel<false>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                       as_stream(stream), x, q, scale, numel);
  return launch_status();
}

int fp8_amax_tensor(const void* x_bf16, int64_t numel, float* amax, float* scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!x_bf16 || !amax || !scale) return FP8BS_ERR_NULL;
  if (numel < 1) return FP8BS_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(amax, 4) || !aligned(scale, 4)) return FP8BS_ERR_ALIGN;
  const size_t need = fp8_amax_quant_tensor_workspace_bytes(numel);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
  }
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  hipStream_t st = as_stream(stream);
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  (void)hipGetLastError();
  if (numel <= kSmallNumel) {
    hipLaunchKernelGGL(tensor_amax_small_kernel, dim3(1), dim3(kSmallThreads), 0, st, x, numel, amax, scale);
    return launch_status();
  }
  if (numel <= kMidNumel) {
    hipLaunchKernelGGL(tensor_amax_mid_kernel, dim3(1), dim3(kSmallThreads), 0, st, x, numel, amax, scale);
    return launch_status();
  }
  float* partial = static_cast<float*>(workspace);
  const TensorGrid tg = tensor_grid(numel, dev.num_cus);
  const int g = tg.g;
  launch_amax_partial<true>(tg, x, partial, numel, st);
  if (hipGetLastError() != hipSuccess) return FP8BS_ERR_LAUNCH;
  hipLaunchKernelGGL(tensor_amax_final_kernel, dim3(1), dim3(kThreads), 0, st, partial, g, amax, scale);
  return launch_status();
}

int fp8_amax_quant_tensor_noalloc(const void* x_bf16, int64_t numel, void* q_e4m3, float* scale, void* stream) {
  const int rc = amax_quant_tensor_check(x_bf16, numel, q_e4m3, scale);
  if (rc != FP8BS_OK) return rc;
  // the first pass writes at most kMaxPartials partial maxima, whatever numel
  if (fp8_amax_quant_tensor_workspace_bytes(numel) > kScratchBytes) return FP8BS_ERR_WORKSPACE;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  int st = FP8BS_OK;
  void* partial = scratch_address(&st);
  if (st != FP8BS_OK) return st;
  return amax_quant_tensor_launch(x_bf16, numel, q_e4m3, scale, static_cast<float*>(partial), dev, stream);
}

size_t fp8_act_quant_block_tensor_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 128 || K % 128 != 0 || M > (INT64_MAX / K)) return 0;
  return static_cast<size_t>((block_tensor_partials(M, K) * 4 + 255) / 256 * 256);
}

int fp8_act_quant_block_tensor(const void* x_bf16, int64_t M, int64_t K, void* qb_e4m3, float* block_scale,
                               void* qt_e4m3, float* tensor_scale, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!x_bf16 || !qb_e4m3 || !block_scale || !qt_e4m3 || !tensor_scale) return FP8BS_ERR_NULL;
  if (M < 1 || K < 128 || K % 128 != 0 || M > (INT64_MAX / K)) return FP8BS_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(qb_e4m3, 16) || !aligned(block_scale, 4) || !aligned(qt_e4m3, 16) ||
      !aligned(tensor_scale, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t np = block_tensor_partials(M, K);
  if (np > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  const size_t need = fp8_act_quant_block_tensor_workspace_bytes(M, K);
  if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  hipStream_t st = as_stream(stream);
  float* partial = static_cast<float*>(workspace);
  (void)hipGetLastError();
  hipLaunchKernelGGL(act_quant_block_partial_kernel, dim3(static_cast<unsigned>(np)), dim3(kBTThreads), 0, st,
                     static_cast<const uint4*>(x_bf16), static_cast<uint2*>(qb_e4m3), block_scale, partial,
                     M * (K / 128));
  if (hipGetLastError() != hipSuccess) return FP8BS_ERR_LAUNCH;
  const int64_t numel = M * K;
  const int64_t ga = apply_grid(numel, dev.num_cus);
  hipLaunchKernelGGL(tensor_apply_kernel, dim3(static_cast<unsigned>(ga)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x_bf16), static_cast<uint8_t*>(qt_e4m3), tensor_scale, partial,
                     static_cast<int>(np), numel);
  return launch_status();
}

int fp8bs_debug_encode_e4m3(const float* in, void* out, int64_t n, void* stream) {
  if (!in || !out) return FP8BS_ERR_NULL;
  if (n < 1) return FP8BS_ERR_SHAPE;
  if (!aligned(in, 16) || !aligned(out, 16)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  const int64_t n4 = n / 4;
  (void)hipGetLastError();
  if (n4 > 0) {
    const int64_t grid = (n4 + kThreads - 1) / kThreads;
    if (grid > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
    hipLaunchKernelGGL(debug_encode_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       as_stream(stream), reinterpret_cast<const float4*>(in),
                       static_cast<uint32_t*>(out), n4);
  }
  if (n % 4) {
    hipLaunchKernelGGL(debug_encode_tail_kernel, dim3(1), dim3(4), 0, as_stream(stream), in,
                       static_cast<uint8_t*>(out), n4 * 4, n);
  }
  return launch_status();
}

}  // extern "C"
