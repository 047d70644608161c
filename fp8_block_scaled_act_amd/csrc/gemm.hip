// Block-scaled FP8 GEMM for gfx950: C[M,N] (bf16) = A[M,K] . W[N,K]^T with
// one fp32 scale per 1x128 block of A and per 128x128 block of W.
//
// What is computed ("How to Profile DeepSeek-V3 Inference Kernels Using
// Triton Autotuning", sections "Understanding the Autotuned Kernels in
// DeepSeek-V3" and "Autotune Configuration Structure": FP8 matmul with
// per-block scaling, K in steps of 128): for each K block b,
//     acc[m,n] += (sum_{k in b} A[m,k] W[n,k]) * (a_scale[m,b] * w_scale[n/128,b])
// and C = bf16_rne(acc).
//
// Mapping onto CDNA4: one K block of 128 is exactly the K of one
// v_mfma_f32_16x16x128_f8f6f4, so each MFMA yields the fresh per-block
// partial P_b of a 16x16 output tile (accumulator input 0) and the scale is
// applied once per K block with one FMA per output in fp32 registers. W is
// the MFMA's first operand (16 output rows n) and A the second (16 output
// columns m): every lane then holds 4 outputs of one activation row m that
// share a single combined scale a_scale[m,b] * w_scale[n/128,b].
#include "device_common.h"
#include "host_common.h"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 128;     // output rows n per workgroup (= one weight scale block)
constexpr int kBM = 128;     // output columns m per workgroup
constexpr int kBK = 128;     // K block
constexpr int kThreads = 256;
constexpr int kTileBytes = kBN * kBK;  // 16 KiB per operand tile

__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format 0 = e4m3 for both operands; scale operands 0 select the unscaled MFMA
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// LDS tile: 128 rows of 128 bytes as 8 chunks of 16 bytes; chunk c of row r
// sits at position c ^ (r & 7) so that 16 lanes reading one chunk column of
// 16 consecutive rows spread over the banks.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f2 v = {lo, hi};
  const bf2 r = __builtin_convertvector(v, bf2);
  return __builtin_bit_cast(uint32_t, r);
}

__global__ __launch_bounds__(kThreads) void gemm_blockscaled_v1_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* __restrict__ C, int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1;          // wave's 64-row slice of n
  const int wm = wave >> 1;         // wave's 64-column slice of m
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t KB = K / kBK;
  const int64_t nblk = n0 / 128;

  // global -> register staging: 1024 chunks of 16 B per operand tile, 4 per thread
  // chunk id = tid + 256*i: row = id >> 3, c = id & 7
  uint4 rw[4], ra[4];
  auto load_tiles = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, c = id & 7;
      rw[i] = *reinterpret_cast<const uint4*>(W + (n0 + row) * K + kb * kBK + c * 16);
      const int64_t m = m0 + row;
      ra[i] = m < M ? *reinterpret_cast<const uint4*>(A + m * K + kb * kBK + c * 16)
                    : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int lrow = lane & 15;   // row within a 16-row fragment
  const int lgrp = lane >> 4;   // 32-byte K slice of the fragment
  int64_t mcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mcol[j] = m0 + wm * 64 + j * 16 + lrow;

  load_tiles(0);
  for (int64_t kb = 0; kb < KB; ++kb) {
    __syncthreads();  // previous iteration done reading LDS
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kThreads * i;
      const int row = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(lds_w + lds_off(row, c)) = rw[i];
      *reinterpret_cast<uint4*>(lds_a + lds_off(row, c)) = ra[i];
    }
    __syncthreads();
    if (kb + 1 < KB) load_tiles(kb + 1);

    // combined scales for this lane's four activation rows
    const float swb = sw[nblk * KB + kb];
    float cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cs[j] = (mcol[j] < M ? sa[mcol[j] * KB + kb] : 0.0f) * swb;

    v8i fw[4], fa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wn * 64 + i * 16 + lrow;
      const uint4 lo = *reinterpret_cast<const uint4*>(lds_w + lds_off(row, 2 * lgrp));
      const uint4 hi = *reinterpret_cast<const uint4*>(lds_w + lds_off(row, 2 * lgrp + 1));
      fw[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wm * 64 + j * 16 + lrow;
      const uint4 lo = *reinterpret_cast<const uint4*>(lds_a + lds_off(row, 2 * lgrp));
      const uint4 hi = *reinterpret_cast<const uint4*>(lds_a + lds_off(row, 2 * lgrp + 1));
      fa[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f p = mfma_16x16x128_fp8(fw[i], fa[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(p[r], cs[j], acc[i][j][r]);
      }
  }

  // epilogue: lane holds D[n = 16i + 4*lgrp + r][m = 16j + lrow] -> C[m][n..n+3]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = mcol[j];
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + wn * 64 + i * 16 + lgrp * 4;
      uint2 o;
      o.x = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
      o.y = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
      *reinterpret_cast<uint2*>(C + m * N + n) = o;
    }
  }
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" {

size_t fp8_gemm_blockscaled_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)M; (void)N; (void)K;
  return 0;
}

int fp8_gemm_blockscaled(const void* a_e4m3, const float* a_scale, const void* w_e4m3,
                         const float* w_scale, void* c_bf16, int64_t M, int64_t N, int64_t K,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!a_e4m3 || !a_scale || !w_e4m3 || !w_scale || !c_bf16) return FP8BS_ERR_NULL;
  if (M < 1 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (M > (INT64_MAX / K) || M > (INT64_MAX / N) || N > (INT64_MAX / K)) return FP8BS_ERR_SHAPE;
  if ((M + kBM - 1) / kBM > 65535 || N / kBN > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (!aligned(a_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(c_bf16, 16) ||
      !aligned(a_scale, 4) || !aligned(w_scale, 4))
    return FP8BS_ERR_ALIGN;
  const size_t need = fp8_gemm_blockscaled_workspace_bytes(M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FP8BS_ERR_WORKSPACE;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(N / kBN), static_cast<unsigned>((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(gemm_blockscaled_v1_kernel, grid, dim3(kThreads), 0, as_stream(stream),
                     static_cast<const uint8_t*>(a_e4m3), a_scale,
                     static_cast<const uint8_t*>(w_e4m3), w_scale, static_cast<uint16_t*>(c_bf16),
                     M, N, K);
  return launch_status();
}

}  // extern "C"
