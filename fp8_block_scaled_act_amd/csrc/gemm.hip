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

constexpr int kBK = 128;     // K block

__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format 0 = e4m3 for both operands; scale operands 0 select the unscaled MFMA
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f2 v = {lo, hi};
  const bf2 r = __builtin_convertvector(v, bf2);
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// Main kernel. Workgroup tile 256 (n) x 128 (m), four waves in a 2 x 2 grid,
// each wave 128 (n) x 64 (m) = 8 x 4 MFMA tiles of 16 x 16. Per K block a
// wave issues 32 MFMAs and 128 scale FMAs per lane.
//
// Operand tiles and the K block's activation scales go from global memory
// straight into LDS (global_load_lds, no VGPR staging) in a three-stage ring.
// A 128-byte tile row holds 8 chunks of 16 bytes; chunk c of row r is stored
// at position c ^ ((r >> 1) & 7), so the 16 lanes that read one chunk column
// of 16 consecutive rows touch all 64 banks once. The 128 activation scales
// of a stage are stored so that each lane's four (rows 16j + lane%16) are
// adjacent. The weight scale is one scalar load per wave and K block.
//
// The MFMAs of MFMA row-tile i are issued before the scale FMAs of row-tile
// i-1, whose results are complete by then, so the matrix core and the VALU
// work side by side.
// ---------------------------------------------------------------------------
constexpr int kPBN = 256;
constexpr int kPBM = 128;
constexpr int kPStages = 3;
constexpr int kPThreads = 256;
constexpr int kPWBytes = kPBN * kBK;                           // 32 KiB
constexpr int kPABytes = kPBM * kBK;                           // 16 KiB
constexpr int kPSBytes = kPBM * 4;                             // 512 B of scales
constexpr int kPStageBytes = kPWBytes + kPABytes + kPSBytes;
constexpr int kPWLoads = kPWBytes / 1024 / 4;                  // per wave: 8
constexpr int kPALoads = kPABytes / 1024 / 4;                  // per wave: 4
constexpr int kGroupM = 8;                                     // m tiles walked per n tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int c0) {
  const int x = swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 128 + ((c0 ^ x) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + row * 128 + (((c0 + 1) ^ x) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// waits until at most `n` vector-memory loads of this wave are outstanding
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}

struct PrefillArgs {
  const uint8_t* A;
  const float* sa;
  const uint8_t* W;
  const float* sw;
  uint16_t* C;
  int64_t M, N, K;
  int tiles_m, tiles_n;
};

// Global -> LDS copies (global_load_lds): each lane copies 16 (or 4) bytes
// from its own address to LDS at lds_base + 16 * lane (or 4 * lane);
// lds_base is wave-uniform. Issued from inline assembly so that the
// compiler's wait insertion does not treat every later LDS read as
// dependent on every copy in flight (it cannot tell the ring stages apart and
// would wait for all of them); the kernel waits on vmcnt and barriers itself.
// The instruction writes no VGPR, so no register is left in flight.
__device__ __forceinline__ void copy16_to_lds(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base)
               : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef const __attribute__((address_space(3))) uint8_t* lds_u8_ptr;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8_ptr)p));
}

__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_blockscaled_prefill_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* __restrict__ C, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kPStages * kPStageBytes];

  // XCD-aware tile order: the 8 XCDs take workgroups round-robin, so give
  // each XCD one contiguous range of tiles, walked kGroupM m tiles per n tile
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  const int group = t / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (t % (kGroupM * tiles_n)) % gsize;
  const int tn = (t % (kGroupM * tiles_n)) / gsize;
  const int64_t n0 = static_cast<int64_t>(tn) * kPBN;
  const int64_t m0 = static_cast<int64_t>(tm) * kPBM;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1;
  const int wm = wave >> 1;
  const int KB = static_cast<int>(K / kBK);

  // --- per-lane global sources of the direct-to-LDS loads (rows clamped to
  //     the matrix: rows past M or N load valid memory and are never stored)
  const int lrow8 = lane >> 3;          // row within a 1 KiB slot
  const int lpos = lane & 7;            // physical chunk position
  const uint8_t* wsrc[kPWLoads];
#pragma unroll
  for (int i = 0; i < kPWLoads; ++i) {
    const int row = (wave * kPWLoads + i) * 8 + lrow8;
    const int64_t gr = min<int64_t>(n0 + row, N - 1);
    wsrc[i] = W + gr * K + ((lpos ^ swz(row)) << 4);
  }
  const uint8_t* asrc[kPALoads];
#pragma unroll
  for (int i = 0; i < kPALoads; ++i) {
    const int row = (wave * kPALoads + i) * 8 + lrow8;
    const int64_t gr = min<int64_t>(m0 + row, M - 1);
    asrc[i] = A + gr * K + ((lpos ^ swz(row)) << 4);
  }
  // waves 0 and 1 fetch the scales of m rows [64*wave, 64*wave + 64): lane L
  // takes row 16*(L%4) + L/4, which lands at LDS float L of that half
  const bool loads_scales = wave < 2;
  const float* ssrc = sa + min<int64_t>(m0 + wave * 64 + 16 * (lane & 3) + (lane >> 2), M - 1) * KB;

  // wave-uniform: the weight-scale row address stays in scalar registers
  const int64_t nb = min<int64_t>((n0 + wn * 128) / 128, N / 128 - 1);
  const float* swrow = sw + nb * KB;

  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int kb) {
    const uint32_t st = lds0 + (kb % kPStages) * kPStageBytes;
#pragma unroll
    for (int i = 0; i < kPWLoads; ++i)
      copy16_to_lds(wsrc[i] + static_cast<int64_t>(kb) * kBK, st + (wave * kPWLoads + i) * 1024);
#pragma unroll
    for (int i = 0; i < kPALoads; ++i)
      copy16_to_lds(asrc[i] + static_cast<int64_t>(kb) * kBK,
                    st + kPWBytes + (wave * kPALoads + i) * 1024);
    if (loads_scales) copy4_to_lds(ssrc + kb, st + kPWBytes + kPABytes + wave * 256);
  };

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int c0 = 2 * (lane >> 4);
  const int arow = wm * 64 + (lane & 15);
  const int wrow = wn * 128 + (lane & 15);
  issue(0);
  if (KB > 1) issue(1);
  for (int kb = 0; kb < KB; ++kb) {
    // this wave's copies of block kb (issued two iterations back) are done
    // once at most the next block's group is outstanding
    if (kb + 1 < KB) {
      if (loads_scales) wait_vmcnt<kPWLoads + kPALoads + 1>();
      else wait_vmcnt<kPWLoads + kPALoads>();
    } else {
      wait_vmcnt<0>();
    }
    // Plain barrier, no memory fence: every wave's part of block kb is in
    // LDS, and every wave's LDS reads of block kb-1 are complete (they fed
    // MFMAs already issued), so stage (kb+2)%3 may be refilled.
    __builtin_amdgcn_s_barrier();
    if (kb + 2 < KB) issue(kb + 2);

    const uint8_t* st = lds + (kb % kPStages) * kPStageBytes;
    const uint8_t* sA = st + kPWBytes;
    const float4 sav = *reinterpret_cast<const float4*>(st + kPWBytes + kPABytes + wm * 256 + (lane & 15) * 16);
    const float swb = swrow[kb];
    const float cs[4] = {sav.x * swb, sav.y * swb, sav.z * swb, sav.w * swb};

    v8i af[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) af[j] = lds_frag(sA, arow + j * 16, c0);
    v4f pp[4], pc[4];
    {
      const v8i wf = lds_frag(st, wrow, c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) pp[j] = mfma_16x16x128_fp8(wf, af[j]);
    }
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      const v8i wf = lds_frag(st, wrow + i * 16, c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) pc[j] = mfma_16x16x128_fp8(wf, af[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = __builtin_fmaf(pp[j][r], cs[j], acc[i - 1][j][r]);
#pragma unroll
      for (int j = 0; j < 4; ++j) pp[j] = pc[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[7][j][r] = __builtin_fmaf(pp[j][r], cs[j], acc[7][j][r]);
  }

  // epilogue: lane holds D[n = 16i + 4*(lane/16) + r][m = 16j + lane%16]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + wm * 64 + j * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = n0 + wn * 128 + i * 16 + (lane >> 4) * 4;
      if (n >= N) continue;
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
  if ((M + 127) / 128 * ((N + 255) / 256) > 0x7FFFFFF0LL || K / 128 > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (!aligned(a_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(c_bf16, 16) ||
      !aligned(a_scale, 4) || !aligned(w_scale, 4))
    return FP8BS_ERR_ALIGN;
  const size_t need = fp8_gemm_blockscaled_workspace_bytes(M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FP8BS_ERR_WORKSPACE;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  (void)hipGetLastError();
  const int64_t tiles_m = (M + kPBM - 1) / kPBM;
  const int64_t tiles_n = (N + kPBN - 1) / kPBN;
  const int64_t grid = (tiles_m * tiles_n + 7) / 8 * 8;
  hipLaunchKernelGGL(gemm_blockscaled_prefill_kernel, dim3(static_cast<unsigned>(grid)),
                     dim3(kPThreads), 0, as_stream(stream), static_cast<const uint8_t*>(a_e4m3),
                     a_scale, static_cast<const uint8_t*>(w_e4m3), w_scale,
                     static_cast<uint16_t*>(c_bf16), M, N, K, static_cast<int>(tiles_m),
                     static_cast<int>(tiles_n));
  return launch_status();
}

}  // extern "C"
