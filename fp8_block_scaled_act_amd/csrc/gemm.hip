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
// applied once per K block with one FMA per output in fp32 registers (the
// fp32 promotion interval of the DeepSeek-V3 design: the matrix cores' own
// sum of 128 products is block floating point, see the comparison rule of
// the tests). W is the MFMA's first operand (16 output rows n) and A the
// second (16 output columns m): every lane then holds 4 outputs of one
// activation row m that share a single combined scale.
#include <type_traits>

#include "device_common.h"
#include "host_common.h"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;     // K block
// m tiles walked per n tile (tile order): 4 for the 256 x 256 tiles, whose
// C stores are non-temporal, else 8. Large-M (16384 x 7168 x 2048), one GPU,
// alternating runs: 8 m tiles with cached C stores 227-234 us, 4 with cached
// stores 229 us, 8 with non-temporal stores 230 us, 4 with non-temporal
// stores 222-228 us (2 and 16: 224-226 and 227-230 us); prefill unchanged.
// The L2 fills per launch stay the same (about 181 MiB), so the gain is not
// in the L2; the C stores that skip the caches leave the last-level cache to
// the operands.
template <int BN>
constexpr int group_m() { return BN == 256 ? 4 : 8; }

__device__ __forceinline__ v4f mfma_16x16x128_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format 0 = e4m3 for both operands; scale operands 0 select the unscaled MFMA
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// The matrix cores' own block scaling: D = (A * 2^(sa-127)) . (B * 2^(sb-127)) + C,
// the scale bytes (e8m0) per lane, each applying to that lane's row or column
// and 32-element K slice. Used when the block scales are powers of two.
__device__ __forceinline__ v4f mfma_16x16x128_fp8_scaled(const v8i& a, const v8i& b, const v4f& c, int sa,
                                                        int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// e8m0 byte of a power-of-two float scale: its biased exponent (2^-127, a
// subnormal, and 0.0 both give 0, i.e. 2^-127; a zero scale only ever
// multiplies all-zero codes)
__device__ __forceinline__ int e8m0_byte(float s) {
  return static_cast<int>((__float_as_uint(s) >> 23) & 0xFFu);
}

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f2 v = {lo, hi};
  const bf2 r = __builtin_convertvector(v, bf2);
  return __builtin_bit_cast(uint32_t, r);
}

// Buffer resource (V#) of a raw byte buffer: base address, size in bytes
// (num_records, stride 0), 32-bit data format. Loads at offsets at or past
// the size return zeros instead of touching memory. All four words are
// wave-uniform and live in scalar registers.
typedef int v4i_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i_rsrc make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i_rsrc r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}
// Buffer -> LDS copies (buffer_load ... lds): each lane copies 16 (or 4)
// bytes at its byte offset `voff` into the buffer to LDS at
// lds_base + 16 * lane (or 4 * lane); lds_base is wave-uniform. Issued from
// inline assembly so that the compiler's wait insertion does not treat every
// later LDS read as dependent on every copy in flight (it cannot tell the
// ring stages apart and would wait for all of them); the kernel waits on
// vmcnt and barriers itself. The instruction writes no VGPR, so no register
// is left in flight. The offset is the only per-lane operand, and the range
// check replaces any clamping of rows past the end of a matrix.
__device__ __forceinline__ void copy16_buf_to_lds(uint32_t voff, v4i_rsrc rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds_base)
               : "memory", "m0");
}
// The same with the non-temporal hint, for data that no other workgroup
// reads again from the caches (streamed weight rows)
__device__ __forceinline__ void copy16_buf_to_lds_nt(uint32_t voff, v4i_rsrc rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
               "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_buf_to_lds(uint32_t voff, v4i_rsrc rsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(lds_base)
               : "memory", "m0");
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef const __attribute__((address_space(3))) uint8_t* lds_u8_ptr;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8_ptr)p));
}

// waits until at most `n` vector-memory loads of this wave are outstanding
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}

// LDS tile rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is
// stored at position c ^ g(r), g(r) = r2 | r1 << 1 | r3 << 2 (bits of r).
// A fragment read has lanes 0-15 on chunk c and lanes 16-31 on chunk c+2 of
// rows 0-15 (and so on): g keeps every group of 32 lanes on distinct 4-byte
// banks of the 128-bank LDS (measured: the plain (r >> 1) & 7 order left a
// two-way conflict on every read), and every group of 16 on distinct banks
// of a 64-bank view as well.
__device__ __forceinline__ int swz(int row) {
  return ((row >> 2) & 1) | (row & 2) | (((row >> 3) & 1) << 2);
}

// Position swizzle of the activation-scale chunks (8 floats per row): rows
// r and r+4, r+8, r+12 get distinct XOR masks, so 16 consecutive rows read
// at one block position hit distinct banks of a 32-, 64- or 128-bank view.
// Only bits 0-3 of r matter; the copy's rows 8g + l/8 and the read's rows
// 16j + l%16 agree on them.
__device__ __forceinline__ int sfold(int r) {
  return (r & 7) ^ (((r >> 3) & 1) << 1);
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int c0) {
  const int x = swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 128 + ((c0 ^ x) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + row * 128 + (((c0 + 1) ^ x) << 4));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// ---------------------------------------------------------------------------
// Tiled kernel. Workgroup tile BN (n) x BM (m) of WN x WM waves, each wave
// TN x TM = (BN/WN) x (BM/WM) = NI x NJ MFMA tiles of 16 x 16. Per K block a
// wave issues NI*NJ MFMAs and 4*NI*NJ scale FMAs per lane.
//
// Operand tiles go from global memory straight into LDS (buffer loads with
// the LDS bit) in two stages, block kb in stage kb % 2. The copies of block
// kb+1's W tile go into the W half of the stage block kb-1 left, spread over
// the first two MFMA rows of block kb. A wave reads its A fragments at the
// start of a block and holds them in registers for the whole block, so after
// a barrier in the middle of block kb (every wave past its first MFMA rows)
// the A half of block kb's own stage is free: block kb+2's A tile is copied
// into it there. The A copies get about a block and a half to land and the W
// copies about one, and the per-CU copy path, which moves about 48 bytes a
// clock for these copies (a probe on this chip: one 64 KiB tile pair takes
// 1370 clocks against the 2048 MFMA clocks of a 256 x 256 block), is kept
// busy over more of the block than with both tiles copied one block ahead
// (prefill and large-M GEMMs 4% faster). The activation scales go to LDS
// in chunks of 8 K blocks (double-buffered, copied with the first block of
// each chunk): a's scales are row-major [M, K/128], so fetching a block's
// BM scales alone would touch BM separate cache lines per K block. The
// weight scale is one scalar load per wave and K block (a wave's TN rows sit
// in one 128-row weight block).
//
// The MFMAs of MFMA row i are issued before the scale FMAs of row i-1, whose
// results are complete by then, so the matrix core and the VALU overlap. The
// last MFMA row of a block is issued after the next block's barrier, while
// that block's first fragment reads are in flight.
// ---------------------------------------------------------------------------
template <int BN, int BM, int WN, int WM, int STAGES>
struct TileCfg {
  static constexpr int kWaves = WN * WM;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TN = BN / WN;
  static constexpr int TM = BM / WM;
  static constexpr int NI = TN / 16;
  static constexpr int NJ = TM / 16;
  static constexpr int kWBytes = BN * kBK;
  static constexpr int kABytes = BM * kBK;
  static constexpr int kStageBytes = kWBytes + kABytes;
  static constexpr int kWLoads = kWBytes / 1024 / kWaves;   // 1 KiB copies per wave
  static constexpr int kALoads = kABytes / 1024 / kWaves;
  // activation scales: chunks of kSChunk K blocks (BM rows x kSChunk floats),
  // copied 4 bytes a lane, kSCopies copies per wave per chunk
  static constexpr int kSChunk = 8;
  static constexpr int kSChunkBytes = BM * kSChunk * 4;
  static constexpr int kSCopies = kSChunkBytes / 256 / kWaves;
  static_assert(kWLoads * 1024 * kWaves == kWBytes && kALoads * 1024 * kWaves == kABytes, "loads");
  static_assert(kSCopies * 256 * kWaves == kSChunkBytes, "scale copies");
  static_assert(TN <= 128 && 128 % TN == 0, "a wave's rows must sit in one weight block");
  static_assert(STAGES == 2, "the copy schedule assumes two stages");
  static_assert(STAGES * kStageBytes + 2 * kSChunkBytes <= 160 * 1024, "LDS");
};

// MODE 0: fp32 block scales, one scale FMA per output and K block.
// MODE 1: power-of-two block scales, applied by the matrix cores (no scale
//         FMAs; the fp32 accumulator is the MFMA's own, chained over K).
// MODE 2: one scale per tensor (sa[0], sw[0]): products accumulated by the
//         matrix cores unscaled, the scale product applied in the epilogue.
// PART: split K (blockIdx.y = split, kb_per K blocks each) and store the
// fp32 partial sums [split][M][N] to `part` instead of C; a second kernel adds
// them in split order.
template <int BN, int BM, int WN, int WM, int STAGES, int WAVES_PER_EU, int MODE, bool PART = false>
__global__ __launch_bounds__(64 * WN * WM) __attribute__((amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void gemm_blockscaled_tiled_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* __restrict__ C, int64_t M, int64_t N, int64_t K,
    int tiles_m, int tiles_n, float* __restrict__ part = nullptr, int kb_per = 0) {
  using T = TileCfg<BN, BM, WN, WM, STAGES>;
  constexpr int NI = T::NI, NJ = T::NJ;
  constexpr bool HW = MODE >= 1;
  constexpr bool TS = MODE == 2;
  // the operand ring, then (block scales only) two buffers of activation-scale chunks
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * T::kStageBytes + (TS ? 0 : 2 * T::kSChunkBytes)];

  // XCD-aware tile order: the 8 XCDs take workgroups round-robin, so give
  // each XCD one contiguous range of tiles, walked kGroupM m tiles per n tile
  constexpr int kGroupM = group_m<BN>();
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = (ntiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  const int group = t / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (t % (kGroupM * tiles_n)) % gsize;
  const int tn = (t % (kGroupM * tiles_n)) / gsize;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % WN;
  const int wm = wave / WN;
  const int KB = static_cast<int>(K / kBK);
  // this workgroup's K blocks: [kb0, kb_end) (all of K unless PART)
  const int sp = PART ? static_cast<int>(blockIdx.y) : 0;
  const int kb0 = PART ? sp * kb_per : 0;
  const int kb_end = PART ? min(KB, kb0 + kb_per) : KB;

  // --- copy sources: per-lane 32-bit byte offsets into buffers that start
  //     at the tile's first row and end at the matrix's last row (rows past
  //     M or N read as zeros; their outputs are never stored)
  const int lrow8 = lane >> 3;          // row within a 1 KiB slot
  const int lpos = lane & 7;            // physical chunk position
  uint32_t woff[T::kWLoads];
#pragma unroll
  for (int i = 0; i < T::kWLoads; ++i) {
    const int row = (wave * T::kWLoads + i) * 8 + lrow8;
    woff[i] = static_cast<uint32_t>(row * K + ((lpos ^ swz(row)) << 4));
  }
  uint32_t aoff[T::kALoads];
#pragma unroll
  for (int i = 0; i < T::kALoads; ++i) {
    const int row = (wave * T::kALoads + i) * 8 + lrow8;
    aoff[i] = static_cast<uint32_t>(row * K + ((lpos ^ swz(row)) << 4));
  }
  const int64_t wrows = min<int64_t>(BN, N - n0), arows = min<int64_t>(BM, M - m0);
  const uint8_t* wtile = W + n0 * K;
  const uint8_t* atile = A + m0 * K;
  const float* stile = sa + m0 * KB;
  // Activation scales of chunk c (K blocks 8c .. 8c+7): copy q of this wave
  // has lane l fetch row r = 8*(wave*kSCopies + q) + l/8, block
  // 8c + ((l%8) ^ sfold(r)). Eight lanes share one row's 32 contiguous bytes,
  // so a copy touches 8 rows' lines (a copy per K block would touch one line
  // per row). In LDS a chunk holds 8 floats a row, block x of row r at
  // position x ^ sfold(r): the 16 rows a K block's scale read covers then
  // fall on distinct banks (the unswizzled stride of 8 floats conflicted).
  // Blocks past K/128 in the last chunk read the next row's scales or zeros
  // (past the buffer) and are never used.
  // (kSCopies is even, so copy q's rows have bit 3 equal to q's parity)
  static_assert(T::kSCopies % 2 == 0, "scale copies per wave");
  // The two per-lane offsets are recomputed at each chunk (every eighth
  // block) from a lane id the compiler cannot hoist: kept live across the K
  // loop they pushed the power-of-two kernel over its registers, and the
  // spill's reload waited for every copy in flight.
  auto scale_offsets = [&](uint32_t* so) {
    int ln = static_cast<int>(threadIdx.x & 63);
    asm volatile("" : "+v"(ln));
    const uint32_t srow = static_cast<uint32_t>((wave * T::kSCopies * 8 + (ln >> 3)) * KB * 4);
    so[0] = srow + static_cast<uint32_t>(((ln & 7) ^ sfold(ln >> 3)) * 4);
    so[1] = srow + static_cast<uint32_t>(((ln & 7) ^ sfold(8 + (ln >> 3))) * 4);
  };
  // wave-uniform: the weight-scale row address stays in scalar registers
  const int64_t nb = min<int64_t>((n0 + wn * T::TN) / 128, N / 128 - 1);
  const float* swrow = sw + nb * KB;

  const uint32_t lds0 = lds_addr(lds);
  // Copy p of this wave's part of block kb (p < kPer: W copies, then A
  // copies; the copies of a scale chunk go with p == 0 of the chunk's first
  // block). Inside the K loop the copies of the block being prefetched are
  // spread over the first MFMA rows. Each buffer starts at column 128*kb of
  // the tile's first row.
  auto issue_part = [&](int kb, int p) {
    const uint32_t st = lds0 + (kb % STAGES) * T::kStageBytes;
    const uint32_t cb = static_cast<uint32_t>(kb) * kBK;
    if (p < T::kWLoads) {
      copy16_buf_to_lds(woff[p], make_rsrc(wtile + cb, static_cast<uint32_t>(wrows * K) - cb),
                        st + (wave * T::kWLoads + p) * 1024);
    } else {
      const int q = p - T::kWLoads;
      copy16_buf_to_lds(aoff[q], make_rsrc(atile + cb, static_cast<uint32_t>(arows * K) - cb),
                        st + T::kWBytes + (wave * T::kALoads + q) * 1024);
    }
    if constexpr (!TS) {
      if (p == 0 && ((kb & (T::kSChunk - 1)) == 0 || (PART && kb == kb0))) {
        const int c = kb / T::kSChunk;
        const v4i_rsrc sr = make_rsrc(stile + c * T::kSChunk, static_cast<uint32_t>(arows * KB * 4 - c * T::kSChunk * 4));
        const uint32_t sd = lds0 + STAGES * T::kStageBytes + (c & 1) * T::kSChunkBytes + wave * T::kSCopies * 256;
        uint32_t soff[2];
        scale_offsets(soff);
#pragma unroll
        for (int q = 0; q < T::kSCopies; ++q)
          copy4_buf_to_lds(soff[q & 1] + static_cast<uint32_t>(q * 8 * KB * 4), sr, sd + q * 256);
      }
    }
  };
  auto issue = [&](int kb) {
#pragma unroll
    for (int p = 0; p < T::kWLoads + T::kALoads; ++p) issue_part(kb, p);
  };

  v4f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int c0 = 2 * (lane >> 4);
  const int arow = wm * T::TM + (lane & 15);
  const int wrow = wn * T::TN + (lane & 15);
  // prologue: block 0's tiles and block 1's A tile (block 1's W tile is
  // copied during block 0)
  issue(kb0);
  if (kb0 + 1 < kb_end) {
#pragma unroll
    for (int q = 0; q < T::kALoads; ++q) issue_part(kb0 + 1, T::kWLoads + q);
  }
  constexpr int kPer = T::kWLoads + T::kALoads;   // operand copies per block (scale chunks aside)
  // The weight scale of block kb+1 is loaded (scalar load) after the last
  // fragment read of block kb and waited for right after the next barrier,
  // before the first fragment read: scalar loads complete out of order, so
  // while one is in flight every wait for an LDS read is a full wait.
  float swb = TS ? 1.0f : swrow[kb0];
  // Software pipeline across blocks. The MFMAs of the last W row of block
  // kb-1 are issued after the barrier that opens block kb, interleaved with
  // the reads of block kb's A fragments (each read refills the registers the
  // MFMA before it has consumed), so the matrix unit has work while those
  // first reads are in flight. The scale FMAs of every MFMA row run after the
  // next row's MFMAs. Before the first block all of this state is zero, which
  // makes the extra MFMAs and FMAs of the first prologue exact no-ops.
  v8i af[NJ];
  v8i wlast;
  v4f pp[NJ];
  float csl[NJ];
  int sal[NJ];          // HW: e8m0 activation scales of the last row's block
  int swl = 127;        // HW: e8m0 weight scale of the last row's block
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    af[j] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    pp[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    csl[j] = 0.0f;
    sal[j] = 127;
  }
  wlast = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  // copies issued during a block: kPerRow per MFMA row, W tile of the next
  // block first, then (after the mid-block barrier) the A tile of the block
  // after it; rows 0 .. NI-2 can issue (the last row runs after the next
  // block's barrier)
  constexpr int kPerRow = kPer / 2 <= NI - 1 ? 2 : 4;
  static_assert(T::kWLoads % kPerRow == 0 && T::kALoads % kPerRow == 0, "a row issues copies of one tile");
  static_assert(kPer / kPerRow <= NI - 1, "every copy must be issued");
  constexpr int kARow = T::kWLoads / kPerRow;   // first row that copies A, after the barrier
  // copies of MFMA row i of block kb (PF blocks only, uniform over the
  // workgroup): W copies of block kb+1, then the barrier and the A copies of
  // block kb+2. In the last prefetching block kb+2 is past the end: those
  // copies read rows below the tile's last (or zeros past the matrix) into a
  // stage half no block reads again.
  auto issue_row = [&](int kb, int i) {
    if (i == kARow) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = i * kPerRow; p < (i + 1) * kPerRow; ++p) {
      if (p < T::kWLoads) issue_part(kb + 1, p);
      else if (p < kPer) issue_part(kb + 2, p);
    }
  };

  // One K block. PF: the block STAGES-1 ahead is copied in during this one
  // (all but the last STAGES-1 blocks); the two loops keep that decision out
  // of the loop body.
  auto step = [&](int kb, auto pf) {
    constexpr bool PF = decltype(pf)::value;
    // this wave's copies of block kb (and of the scale chunk that starts at
    // kb) are done once at most the copies of the blocks issued after it
    // remain: STAGES-2 groups of at least kPer copies while blocks are being
    // prefetched, fewer in the last iterations (loads complete in order)
    if (kb + 1 < kb_end)
      wait_vmcnt<T::kALoads>();   // block kb+1's A copies, issued last, may be in flight
    else
      wait_vmcnt<0>();
    // The last W fragment of block kb-1 (wlast) was read but not yet used:
    // wait for every LDS read (and the scalar load of the weight scale) so
    // that no read of block kb-1's stage is in flight past the barrier.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    // Plain barrier, no memory fence: every wave's part of block kb is in
    // LDS, and every wave's LDS reads of block kb-1 have returned, so that
    // stage may be refilled.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::"s"(swb));
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* st = lds + (kb % STAGES) * T::kStageBytes;
    const uint8_t* sA = st + T::kWBytes;
    float sav[NJ];
    if constexpr (TS) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) sav[j] = 1.0f;
    } else {
      // rows wm*TM + 16j + lane%16 of the chunk holding block kb (the
      // position swizzle depends on the row mod 16 only)
      const float* sv = reinterpret_cast<const float*>(lds + STAGES * T::kStageBytes +
                                                       ((kb / T::kSChunk) & 1) * T::kSChunkBytes) +
                        (wm * T::TM + (lane & 15)) * T::kSChunk + ((kb & (T::kSChunk - 1)) ^ sfold(lane & 15));
#pragma unroll
      for (int j = 0; j < NJ; ++j) sav[j] = sv[j * 16 * T::kSChunk];
    }
    v8i wcur = lds_frag(st, wrow, c0);
    if constexpr (HW) {
      // last row of block kb-1 (its scales in swl, sal); each A fragment is
      // refilled right after its MFMA
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[NI - 1][j] = mfma_16x16x128_fp8_scaled(wlast, af[j], acc[NI - 1][j], swl, sal[j]);
        af[j] = lds_frag(sA, arow + j * 16, c0);
      }
      v8i wnext = lds_frag(st, wrow + 16, c0);
      const int swb8 = TS ? 127 : e8m0_byte(swb);
      int sab[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) sab[j] = TS ? 127 : e8m0_byte(sav[j]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[0][j] = mfma_16x16x128_fp8_scaled(wcur, af[j], acc[0][j], swb8, sab[j]);
      if constexpr (PF) {
        issue_row(kb, 0);
      }
#pragma unroll
      for (int i = 1; i < NI - 1; ++i) {
        wcur = wnext;
        wnext = lds_frag(st, wrow + (i + 1) * 16, c0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_16x16x128_fp8_scaled(wcur, af[j], acc[i][j], swb8, sab[j]);
        if constexpr (PF) {
          issue_row(kb, i);
        }
      }
      wlast = wnext;
      swl = swb8;
#pragma unroll
      for (int j = 0; j < NJ; ++j) sal[j] = sab[j];
    } else {
    // last row of block kb-1; each A fragment is refilled right after its MFMA
    v4f pc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      pc[j] = mfma_16x16x128_fp8(wlast, af[j]);
      af[j] = lds_frag(sA, arow + j * 16, c0);
    }
    v8i wnext = lds_frag(st, wrow + 16, c0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[NI - 2][j][r] = __builtin_fmaf(pp[j][r], csl[j], acc[NI - 2][j][r]);
    // row 0 of block kb
#pragma unroll
    for (int j = 0; j < NJ; ++j) pp[j] = mfma_16x16x128_fp8(wcur, af[j]);
    if constexpr (PF) {
      issue_row(kb, 0);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[NI - 1][j][r] = __builtin_fmaf(pc[j][r], csl[j], acc[NI - 1][j][r]);
    float cs[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) cs[j] = sav[j] * swb;
    // rows 1..NI-2; W fragments double-buffered: the fragment of row i+1 is
    // read before the MFMAs of row i, so its LDS latency hides behind them
#pragma unroll
    for (int i = 1; i < NI - 1; ++i) {
      wcur = wnext;
      wnext = lds_frag(st, wrow + (i + 1) * 16, c0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) pc[j] = mfma_16x16x128_fp8(wcur, af[j]);
      if constexpr (PF) {
        issue_row(kb, i);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i - 1][j][r] = __builtin_fmaf(pp[j][r], cs[j], acc[i - 1][j][r]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) pp[j] = pc[j];
    }
    // pp holds row NI-2; the last row's fragment waits in wlast
    wlast = wnext;
#pragma unroll
    for (int j = 0; j < NJ; ++j) csl[j] = cs[j];
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!TS) swb = swrow[min(kb + 1, kb_end - 1)];
  };
  const int kb_pf = max(kb_end - (STAGES - 1), kb0);
  for (int kb = kb0; kb < kb_pf; ++kb) step(kb, std::true_type{});
  for (int kb = kb_pf; kb < kb_end; ++kb) step(kb, std::false_type{});
  if constexpr (HW) {
    // last row of the last block
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[NI - 1][j] = mfma_16x16x128_fp8_scaled(wlast, af[j], acc[NI - 1][j], swl, sal[j]);
  } else {
    // last row of the last block
    v4f pc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) pc[j] = mfma_16x16x128_fp8(wlast, af[j]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[NI - 2][j][r] = __builtin_fmaf(pp[j][r], csl[j], acc[NI - 2][j][r]);
        acc[NI - 1][j][r] = __builtin_fmaf(pc[j][r], csl[j], acc[NI - 1][j][r]);
      }
  }

  // Epilogue through LDS, so that every global store writes whole rows of C.
  // Lane holds D[n = 16i + 4*(lane/16) + r][m = 16j + lane%16] of the wave's
  // sub-tile; the bf16 tile is staged row-major (m rows of BN values) in the
  // ring, 16-byte chunk c of row m stored at chunk c ^ (m & 15), which keeps
  // the 8-byte writes of a half-wave (16 rows, one chunk pair) and the
  // 16-byte row reads free of bank conflicts.
  static_assert(BM * BN * 2 <= STAGES * T::kStageBytes, "C tile must fit the LDS ring");
  constexpr int kRowBytes = BN * 2;
  constexpr int kChunks = BN / 8;
  if constexpr (TS) {
    // the tensor scales' product, once per output (then the bf16 rounding)
    const float st = sa[0] * sw[0];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] *= st;
  }
  if constexpr (PART) {
    // The last MFMA row above must run with every lane active: the stores
    // below are conditional, and the compiler would otherwise sink those
    // MFMAs into them, where a scale moved into a VGPR under the partial
    // EXEC mask leaves stale bytes in the inactive lanes (the matrix cores
    // read every lane's operands). The empty asm pins the results here.
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[i][j]));
    // the fp32 partial sums of this K split, 16 bytes a lane (four n of one
    // m), stored non-temporally: the reduce kernel reads them once
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t m = m0 + wm * T::TM + j * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t n = n0 + wn * T::TN + i * 16 + (lane >> 4) * 4;
        if (m < M && n < N) {
          float* q = part + (static_cast<int64_t>(sp) * M + m) * N + n;
          __builtin_nontemporal_store(acc[i][j][0], q);
          __builtin_nontemporal_store(acc[i][j][1], q + 1);
          __builtin_nontemporal_store(acc[i][j][2], q + 2);
          __builtin_nontemporal_store(acc[i][j][3], q + 3);
        }
      }
    }
    return;
  }
  __syncthreads();   // every wave is done reading the last stage
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ml = wm * T::TM + j * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int nl = wn * T::TN + i * 16 + (lane >> 4) * 4;
      const int off = ml * kRowBytes + (((nl >> 3) ^ (ml & 15)) << 4) + ((nl & 4) << 1);
      uint2 o;
      o.x = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
      o.y = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
      *reinterpret_cast<uint2*>(lds + off) = o;
    }
  }
  __syncthreads();
  static_assert(BM * kChunks % T::kThreads == 0, "row chunks per thread");
#pragma unroll
  for (int k = 0; k < BM * kChunks / T::kThreads; ++k) {
    const int idx = k * T::kThreads + static_cast<int>(threadIdx.x);
    const int ml = idx / kChunks, c = idx % kChunks;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + ml * kRowBytes + ((c ^ (ml & 15)) << 4));
    const int64_t m = m0 + ml, n = n0 + c * 8;
    if (m < M && n < N) {
      if constexpr (BN == 256) {
        // non-temporal: C is written once and not read back here
        const v4i w4 = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
        __builtin_nontemporal_store(w4, reinterpret_cast<v4i*>(C + m * N + n));
      } else {
        *reinterpret_cast<uint4*>(C + m * N + n) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernels. At decode shapes the GEMM is bound by streaming W from HBM.
//
// Small M (M <= 8): a workgroup takes R W rows over the whole of K, sixteen
// waves; the waves split K into steps of P K blocks (P = 16 / R), wave w
// taking steps w, w+16, w+32, ... and keeping kDecDepth of them in flight,
// W fragments and A fragments loaded straight from global memory into
// registers (A is small and stays in L2). Each step is one MFMA plus the
// scale FMAs. The sixteen waves' partial sums are added through LDS in a
// fixed order, so the result is deterministic and no second kernel or
// workspace is needed. Every workgroup reads all of A (through L2), which
// costs little while A is at most 8 rows. (Staging A in LDS before the K
// loop, as the fused kernel below does with the quantized X, measured
// slower here: 5.8 against 5.4 us at M = 1 with packed blocks; past M = 8
// the kernel that streams A through LDS in chunks takes over.)
//
// Packed K blocks (P > 1, for M <= R): a 16x16 MFMA tile has 16 W rows, but
// with R = 16 / P W rows per workgroup the grid has P times as many
// workgroups, so that every CU streams W (N = 2048: 128 workgroups of 16
// rows leave half of the 256 CUs idle; 256 workgroups of 8 rows read the
// 14.7 MB of W in 4.2 instead of 5.1 us in a read-only probe). The MFMA's
// 16 rows (and 16 activation columns) are then P groups of R: group g
// carries K block P*s + g of the same R W rows and of activation rows
// 0..R-1, and the diagonal blocks of its 16x16 result (W group g against
// activation group g) are the partial sums of those blocks; the
// off-diagonal blocks are discarded. Lane l supplies row (l%16)%R of group
// (l%16)/R; its four outputs lie in one group, and they are kept when that
// group is its own column's.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 16;
// K blocks packed into one MFMA (rows per workgroup 16 / P must hold the M
// activation rows): the streaming kernel takes M <= 8 with two
constexpr int kDecPackMaxM = 8;
constexpr int kDecStreamMaxM = kDecPackMaxM;

// Sum over each row of 16 lanes by DPP lane swaps: pairs i^1 and i^2 (quad
// permutations), then the mirror images within 8 and within 16 lanes. Each
// step adds a lane's value to its partner's, so every lane of a row ends
// with the same bits. All lanes of the wave must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);   // row_half_mirror
  v += dpp_f32<0x140>(v);   // row_mirror
  return v;
}

// Final sums and bf16 stores of a small-M decode workgroup, called by every
// thread after a barrier. red holds the waves' float4 results, lane l of
// wave w at red[w * 64 + l]; lane l holds D[n = 4*(l/16) + r][m = l%16] of
// its wave's MFMA tile. Output group o = (quad q = o / M, activation row
// m = o % M) is W rows n0 + 4q .. +3 against activation row m; in K-block
// group g it sits in lane 16q + m + 5*g*R (W rows and activation columns
// both shifted by g*R). A row of 16 threads takes one output group: thread
// i adds the P group terms of wave i in group order, then the row adds the
// waves by lane swaps. The order is fixed, so the result is deterministic.
template <int P, int R = 16 / P>
__device__ __forceinline__ void decode_store(const float4* red, int M, int64_t n0, int64_t N, uint16_t* C) {
  static_assert(kDecWaves <= 16, "one wave per thread of a 16-thread row");
  const int nout = (R / 4) * M;
  const int i = threadIdx.x & 15;
  for (int ob = 0; ob < nout; ob += 4 * kDecWaves) {
    const int o = ob + static_cast<int>(threadIdx.x >> 4);
    const int q = o / M, m = o - q * M;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (o < nout && i < kDecWaves) {
      const int l0 = 16 * q + m;
      v = red[i * 64 + l0];
#pragma unroll
      for (int g = 1; g < P; ++g) {
        const float4 u = red[i * 64 + l0 + 5 * g * R];
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
      }
    }
    v.x = row16_sum(v.x);
    v.y = row16_sum(v.y);
    v.z = row16_sum(v.z);
    v.w = row16_sum(v.w);
    if (o < nout && i == 0) {
      uint2 out;
      out.x = bf16x2_rne(v.x, v.y);
      out.y = bf16x2_rne(v.z, v.w);
      *reinterpret_cast<uint2*>(C + m * N + n0 + 4 * q) = out;
    }
  }
}

// P: K blocks packed per MFMA (M <= 16 / P); kDecDepth: steps in flight per
// wave; TS: one scale per tensor (sa[0] * sw[0] for every block)
template <int P, int kDecDepth, bool TS>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(kDecWaves / 4, kDecWaves / 4)))
void gemm_blockscaled_decode_stream_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* __restrict__ C, int M, int64_t N, int64_t K) {
  constexpr int R = 16 / P;
  __shared__ float4 red[kDecWaves * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * R;
  const int KB = static_cast<int>(K / kBK);

  // lane l supplies W row n0 + rsub and A row rsub (rows past M read row
  // M-1: valid memory, results never stored) of K block P*s + grp of step s,
  // bytes 32*(l/16) ..+32 of the block
  const int rsub = (lane & 15) % R;
  const int grp = (lane & 15) / R;
  const int koff = 32 * (lane >> 4);
  const uint8_t* wp = W + (n0 + rsub) * K + koff;
  const int64_t am = min<int64_t>(rsub, M - 1);
  const uint8_t* ap = A + am * K + koff;
  const float* sp = sa + am * KB;
  const float* swrow = sw + (n0 / 128) * KB;

  // this wave's steps: s = wave + kDecWaves * t, t = 0 .. nt-1; a lane
  // whose block is past K (last step, KB not a multiple of P) loads
  // nothing and contributes zeros
  const int S = (KB + P - 1) / P;
  const int nt = S > wave ? (S - wave + kDecWaves - 1) / kDecWaves : 0;
  uint4 wq[kDecDepth][2];
  uint4 aq[kDecDepth][2];
  float sq[kDecDepth];
  auto load = [&](int d, int t) {
    const int64_t kb = static_cast<int64_t>(wave + kDecWaves * t) * P + grp;
    if (P == 1 || kb < KB) {
      wq[d][0] = *reinterpret_cast<const uint4*>(wp + kb * kBK);
      wq[d][1] = *reinterpret_cast<const uint4*>(wp + kb * kBK + 16);
      aq[d][0] = *reinterpret_cast<const uint4*>(ap + kb * kBK);
      aq[d][1] = *reinterpret_cast<const uint4*>(ap + kb * kBK + 16);
      if constexpr (!TS) sq[d] = sp[kb];
    } else {
      wq[d][0] = wq[d][1] = make_uint4(0, 0, 0, 0);
      aq[d][0] = aq[d][1] = make_uint4(0, 0, 0, 0);
      if constexpr (!TS) sq[d] = 0.0f;
    }
  };
  const float cst = TS ? sa[0] * sw[0] : 0.0f;
#pragma unroll
  for (int d = 0; d < kDecDepth; ++d)
    if (d < nt) load(d, d);

  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0 = 0; t0 < nt; t0 += kDecDepth) {
#pragma unroll
    for (int d = 0; d < kDecDepth; ++d) {
      const int t = t0 + d;
      if (t < nt) {
        const v8i wf = v8i{(int)wq[d][0].x, (int)wq[d][0].y, (int)wq[d][0].z, (int)wq[d][0].w,
                           (int)wq[d][1].x, (int)wq[d][1].y, (int)wq[d][1].z, (int)wq[d][1].w};
        const v8i af = v8i{(int)aq[d][0].x, (int)aq[d][0].y, (int)aq[d][0].z, (int)aq[d][0].w,
                           (int)aq[d][1].x, (int)aq[d][1].y, (int)aq[d][1].z, (int)aq[d][1].w};
        const int kb = (wave + kDecWaves * t) * P + grp;
        const float swb = TS ? 1.0f : (P == 1 || kb < KB ? swrow[kb] : 0.0f);
        const float cs = TS ? cst : sq[d] * swb;
        if (t + kDecDepth < nt) load(d, t + kDecDepth);
        const v4f p = mfma_16x16x128_fp8(wf, af);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], cs, acc[r]);
      }
    }
  }

  red[wave * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  decode_store<P, R>(red, M, n0, N, C);
}

template <bool TS>
int launch_decode_stream(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* c,
                         int64_t M, int64_t N, int64_t K, hipStream_t st) {
  hipLaunchKernelGGL((gemm_blockscaled_decode_stream_kernel<2, 4, TS>), dim3(static_cast<unsigned>(N / 8)),
                     dim3(64 * kDecWaves), 0, st, a, sa, w, sw, c, static_cast<int>(M), N, K);
  return FP8BS_OK;
}

// ---------------------------------------------------------------------------
// Small-M decode GEMM with the block act-quant fused in (M <= kFusedMaxM):
// C = A_q . W^T with (A_q, sa) the 1x128 block quantization of the bf16
// activations X, in one launch; the quantized activations never go to
// global memory.
//
// Same workgroup shape, K order and packing as the streaming kernel above:
// R W rows per workgroup over the whole of K, wave w taking steps w, w+16,
// ... of P K blocks each. Each workgroup quantizes all of X into LDS (codes
// and scales) while its waves' first W loads are in flight, with the
// act-quant kernel's rule and lane mapping (eight lanes per 1x128 block, the
// same helper), and runs the K loop with A fragments and scales read from
// LDS (the order of the loads is explained below). The arithmetic after that is the
// streaming kernel's, operation for operation, so the results are those of
// the two-launch path (act-quant, then the GEMM) bit for bit. Every
// workgroup quantizes all of X: that redundant work grows with M, so the
// fused form serves the smallest M only.
//
// LDS: the wave partial sums (16 KiB), the scales [M][K/128], then the codes
// of K block kb at kb*128*M: half h (16 bytes) of quarter q (32 bytes) of
// row m at ((h*4 + q)*M + m)*16, so that a fragment read (lanes 16q..16q+15
// on rows 0..15, one half) is one contiguous run of 16-byte chunks.
// ---------------------------------------------------------------------------
constexpr int kFusedLdsBytes = 160 * 1024;
constexpr int kFusedRedBytes = kDecWaves * 64 * 16;
// largest M for the one-kernel act-quant + GEMM (N = 2048, K = 7168: one
// kernel 5.6 / 6.2 / 8.5 us at M = 1 / 4 / 8 against 7.2 / 7.7 / 9.2 us
// for the two launches)
constexpr int64_t kFusedMaxM = 8;

__host__ __device__ inline int64_t fused_scale_bytes(int64_t M, int64_t K) { return (M * (K / kBK) * 4 + 15) / 16 * 16; }
inline bool fused_fits(int64_t M, int64_t K) {
  return M <= kFusedMaxM && kFusedRedBytes + fused_scale_bytes(M, K) + M * K <= kFusedLdsBytes;
}

// X: bf16 [M, K]; P: K blocks packed per MFMA (M <= 16 / P)
template <int kDepth, int P>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(kDecWaves / 4, kDecWaves / 4)))
void act_quant_gemm_decode_kernel(const uint16_t* __restrict__ X, const uint8_t* __restrict__ W,
                                  const float* __restrict__ sw, uint16_t* __restrict__ C, int M, int64_t N,
                                  int64_t K) {
  constexpr int R = 16 / P;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFusedLdsBytes];
  float4* red = reinterpret_cast<float4*>(lds);
  const int KB = static_cast<int>(K / kBK);
  float* ssa = reinterpret_cast<float*>(lds + kFusedRedBytes);
  uint8_t* scode = lds + kFusedRedBytes + fused_scale_bytes(M, K);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * R;

  // lane l: W row n0 + rsub, K block P*s + grp of step s (as in the
  // streaming kernel; a block past K contributes zeros)
  const int rsub = (lane & 15) % R;
  const int grp = (lane & 15) / R;
  const uint8_t* wp = W + (n0 + rsub) * K + 32 * (lane >> 4);
  const float* swrow = sw + (n0 / 128) * KB;
  const int S = (KB + P - 1) / P;
  const int nt = S > wave ? (S - wave + kDecWaves - 1) / kDecWaves : 0;

  // X is quantized into LDS (row-major M x K, block b = m*KB + kb at
  // element 128*b), kPass blocks a thread per pass. The first pass's X loads
  // are issued before the first W loads: loads complete in order, so X (in
  // L2) issued after W (from HBM) could not be quantized before all of
  // those W loads had landed.
  constexpr int kPass = 4;
  constexpr int kBlocksPerPass = 64 * kDecWaves / 8;
  const int nblk = M * KB;
  const int sub = threadIdx.x & 7;
  const int bfirst = static_cast<int>(threadIdx.x >> 3);
  uint4 v[kPass][2];
  auto xload = [&](int b0) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int b = b0 + u * kBlocksPerPass;
      if (b < nblk) {
        const uint4* xb = reinterpret_cast<const uint4*>(X + static_cast<int64_t>(b) * kBK);
        v[u][0] = xb[sub];
        v[u][1] = xb[8 + sub];
      }
    }
  };
  auto xquant = [&](int b0) {
#pragma unroll
    for (int u = 0; u < kPass; ++u) {
      const int b = b0 + u * kBlocksPerPass;
      if (b < nblk) {
        uint2 o0, o1;
        const float sb = quant_block_bf16(v[u][0], v[u][1], o0, o1);
        const int m = b / KB, kb = b % KB;
        // codes of elements 8*sub.. (quarter sub/4) and 64 + 8*sub..
        // (quarter 2 + sub/4); both at byte 8*(sub%4) of their quarter
        const int h = (sub & 3) >> 1;
        uint8_t* cb = scode + static_cast<int64_t>(kb) * kBK * M + (sub & 1) * 8;
        *reinterpret_cast<uint2*>(cb + ((h * 4 + (sub >> 2)) * M + m) * 16) = o0;
        *reinterpret_cast<uint2*>(cb + ((h * 4 + 2 + (sub >> 2)) * M + m) * 16) = o1;
        if (sub == 0) ssa[b] = sb;
      }
    }
  };
  xload(bfirst);

  // W: the first kDepth steps of every wave are loaded unconditionally, so
  // that the number of loads after X's is fixed and the wait for X does not
  // include them. A block past K (or a step past the wave's last) reads
  // the last block instead; the K loop zeroes or skips it.
  uint4 wq[kDepth][2];
  auto loadw = [&](int d, int t) {
    const int64_t kb = min<int64_t>(static_cast<int64_t>(wave + kDecWaves * t) * P + grp, KB - 1);
    wq[d][0] = *reinterpret_cast<const uint4*>(wp + kb * kBK);
    wq[d][1] = *reinterpret_cast<const uint4*>(wp + kb * kBK + 16);
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) loadw(d, d);

  xquant(bfirst);
  for (int b0 = bfirst + kPass * kBlocksPerPass; b0 < nblk; b0 += kPass * kBlocksPerPass) {
    xload(b0);
    xquant(b0);
  }
  __syncthreads();

  // lane l: A row min(rsub, M-1) (rows past M repeat row M-1; their outputs
  // are never stored), quarter l/16 of each K block
  const int ar = min(rsub, M - 1);
  const uint8_t* ap = scode + ((lane >> 4) * M + ar) * 16;
  const float* sp = ssa + ar * KB;
  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int t0 = 0; t0 < nt; t0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int t = t0 + d;
      if (t < nt) {
        const int kb = (wave + kDecWaves * t) * P + grp;
        const bool in = P == 1 || kb < KB;
        v8i wf = v8i{(int)wq[d][0].x, (int)wq[d][0].y, (int)wq[d][0].z, (int)wq[d][0].w,
                     (int)wq[d][1].x, (int)wq[d][1].y, (int)wq[d][1].z, (int)wq[d][1].w};
        if (!in) wf = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        const uint8_t* ak = ap + static_cast<int64_t>(kb) * kBK * M;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
        if (in) {
          lo = *reinterpret_cast<const uint4*>(ak);
          hi = *reinterpret_cast<const uint4*>(ak + 4 * M * 16);
        }
        const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const float cs = in ? sp[kb] * swrow[kb] : 0.0f;
        if (t + kDepth < nt) loadw(d, t + kDepth);
        const v4f p = mfma_16x16x128_fp8(wf, af);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], cs, acc[r]);
      }
    }
  }

  red[wave * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  decode_store<P>(red, M, n0, N, C);
}

int launch_act_quant_gemm_decode(const void* x, const uint8_t* w, const float* sw, uint16_t* c, int64_t M,
                                 int64_t N, int64_t K, hipStream_t st) {
  static_assert(kFusedMaxM <= kDecPackMaxM, "the fused form packs two K blocks per MFMA");
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  // the W loads of a wave's first kDepth steps are issued up front, whether
  // or not the wave has that many: two when no wave has more (K <= 8192)
  const int64_t steps = (K / kBK + 1) / 2;
  if (steps <= 2 * kDecWaves)
    hipLaunchKernelGGL((act_quant_gemm_decode_kernel<2, 2>), dim3(static_cast<unsigned>(N / 8)),
                       dim3(64 * kDecWaves), 0, st, xb, w, sw, c, static_cast<int>(M), N, K);
  else
    hipLaunchKernelGGL((act_quant_gemm_decode_kernel<4, 2>), dim3(static_cast<unsigned>(N / 8)),
                       dim3(64 * kDecWaves), 0, st, xb, w, sw, c, static_cast<int>(M), N, K);
  return FP8BS_OK;
}

// ---------------------------------------------------------------------------
// Larger decode M with wide W (32 < M <= 64, N > 2048): the work is cut
// into many pieces of W so that A is shared: workgroup (n tile of 64 rows, K
// split) has four waves, wave w owning W rows 16w..16w+15 of the tile. Each wave
// loads its W fragments straight from global memory into registers
// (kDepth K blocks in flight), the K split's slice of A (at most 64 rows)
// and its activation scales are staged once in LDS and shared, and each K
// block is one MFMA per 16 activation rows plus the scale FMAs (reading the
// scales from global memory in the K loop cost 2 us per call at M = 64 on
// the decode shape: 15.9 against 13.9 us). With more than one K split the fp32
// partial sums go to the workspace and a second kernel adds them in split
// order (deterministic) and rounds to bf16.
// ---------------------------------------------------------------------------
constexpr int kDecRows = 64;        // W rows per workgroup
constexpr int kDecDepth = 4;        // K blocks of W in flight per wave
constexpr int kDecMaxKb = 16;       // K blocks per split (A slice in LDS)
constexpr int kDecMaxM = 64;
constexpr int kDecMaxSplits = 32;   // the reduction keeps one float4 per split in flight

// MT: 16-row groups of A (M <= 16*MT); KBMAX: K blocks per split (LDS size)
template <int MT, int KBMAX, bool TS>
__global__ __launch_bounds__(256) void gemm_blockscaled_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* __restrict__ C, float* __restrict__ ws, int M, int64_t N,
    int64_t K, int kb_per, int splits) {
  // the A slice, then a 16-byte slot that takes the stores of chunks past
  // the slice's end
  __shared__ __attribute__((aligned(1024))) uint8_t lds[KBMAX * MT * 16 * 128 + 16];
  __shared__ float ssa[MT * 16 * KBMAX];     // the split's activation scales, [row][k]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kDecRows;
  const int sp = blockIdx.y;
  const int KB = static_cast<int>(K / kBK);
  const int kb0 = sp * kb_per;
  const int nkb = min(KB - kb0, kb_per);
  if (nkb <= 0) return;

  const int64_t nrow = n0 + wave * 16 + (lane & 15);          // this lane's W row
  const uint8_t* wp = W + min<int64_t>(nrow, N - 1) * K + static_cast<int64_t>(kb0) * kBK + 32 * (lane >> 4);
  const float* swrow = sw + ((n0 + wave * 16) / 128) * KB + kb0;
  // Stage A rows [0, 16*MT) x K blocks [kb0, kb0 + nkb) in LDS (rows >= M
  // read row M-1: valid memory, results never stored), swizzled as in the
  // tiled kernel, and the split's activation scales, so that the K loop
  // waits on no global load but W's. The first pass of those loads (all of
  // them while nkb * 16*MT * 8 <= kAPass * 256) is issued before the W
  // loads: loads complete in order, so A (in L2) issued after W (from HBM)
  // could not be stored before all of W had landed.
  constexpr int MP = 16 * MT;
  constexpr int kAPass = 8;
  const int nchunk = nkb * MP * 8;
  // chunk id: K block id / (8*MP), row (id / 8) % MP, 16-byte chunk id % 8;
  // a load past the last chunk reads the last one again (unconditional
  // loads leave the compiler no reason to wait for them early)
  auto asrc = [&](int id) {
    id = min(id, nchunk - 1);
    const int64_t gr = min((id / 8) % MP, M - 1);
    return reinterpret_cast<const uint4*>(A + gr * K + static_cast<int64_t>(kb0 + id / (MP * 8)) * kBK + (id % 8) * 16);
  };
  auto adst = [&](int id) {
    const int row = (id / 8) % MP;
    return reinterpret_cast<uint4*>(id < nchunk ? lds + ((id / (MP * 8)) * MP + row) * 128 + (((id % 8) ^ swz(row)) << 4)
                                                : lds + KBMAX * MT * 16 * 128);
  };
  const int id0 = static_cast<int>(threadIdx.x);
  // (eight named registers rather than an array, which the compiler would
  // keep in scratch memory)
#define FP8BS_ALOAD(u) const uint4 av##u = *asrc(id0 + (u) * 256);
  FP8BS_ALOAD(0) FP8BS_ALOAD(1) FP8BS_ALOAD(2) FP8BS_ALOAD(3)
  FP8BS_ALOAD(4) FP8BS_ALOAD(5) FP8BS_ALOAD(6) FP8BS_ALOAD(7)
#undef FP8BS_ALOAD
  static_assert(kAPass == 8, "one named register per chunk of the first pass");
  // the first pass of the scales: MP * nkb <= 16 * MT * KBMAX values
  constexpr int kSPass = (MT * 16 * KBMAX + 255) / 256;
  float sv[kSPass];
  if constexpr (!TS) {
#pragma unroll
    for (int u = 0; u < kSPass; ++u) {
      const int id = min(static_cast<int>(threadIdx.x) + u * 256, MP * nkb - 1);
      const int row = id / nkb, k = id - row * nkb;
      sv[u] = sa[static_cast<int64_t>(min(row, M - 1)) * KB + kb0 + k];
    }
  }

  // W fragments: the first kDecDepth blocks, loaded unconditionally (a block
  // past the split's last reads its last block and is never used), so that
  // the number of loads after A's is fixed; the scheduling barriers keep
  // the compiler from moving A's loads behind them
  __builtin_amdgcn_sched_barrier(0);
  uint4 wq[kDecDepth][2];
#pragma unroll
  for (int d = 0; d < kDecDepth; ++d) {
    const int kk = min(d, nkb - 1);
    wq[d][0] = *reinterpret_cast<const uint4*>(wp + kk * kBK);
    wq[d][1] = *reinterpret_cast<const uint4*>(wp + kk * kBK + 16);
  }

  __builtin_amdgcn_sched_barrier(0);
#define FP8BS_ASTORE(u) *adst(id0 + (u) * 256) = av##u;
  FP8BS_ASTORE(0) FP8BS_ASTORE(1) FP8BS_ASTORE(2) FP8BS_ASTORE(3)
  FP8BS_ASTORE(4) FP8BS_ASTORE(5) FP8BS_ASTORE(6) FP8BS_ASTORE(7)
#undef FP8BS_ASTORE
  if constexpr (!TS) {
#pragma unroll
    for (int u = 0; u < kSPass; ++u) {
      const int id = static_cast<int>(threadIdx.x) + u * 256;
      if (id < MP * nkb) {
        const int row = id / nkb, k = id - row * nkb;
        ssa[row * KBMAX + k] = sv[u];
      }
    }
  }
  for (int id = id0 + kAPass * 256; id < nchunk; id += 256) *adst(id) = *asrc(id);

  __syncthreads();

  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const int c0 = 2 * (lane >> 4);
  for (int kk = 0; kk < nkb; kk += kDecDepth) {
#pragma unroll
    for (int d = 0; d < kDecDepth; ++d) {
      const int k = kk + d;
      if (k < nkb) {
        const v8i wf = v8i{(int)wq[d][0].x, (int)wq[d][0].y, (int)wq[d][0].z, (int)wq[d][0].w,
                           (int)wq[d][1].x, (int)wq[d][1].y, (int)wq[d][1].z, (int)wq[d][1].w};
        if (k + kDecDepth < nkb) {
          wq[d][0] = *reinterpret_cast<const uint4*>(wp + (k + kDecDepth) * kBK);
          wq[d][1] = *reinterpret_cast<const uint4*>(wp + (k + kDecDepth) * kBK + 16);
        }
        const float swb = TS ? 1.0f : swrow[k];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const v8i af = lds_frag(lds + k * MP * 128, j * 16 + (lane & 15), c0);
          const v4f p = mfma_16x16x128_fp8(wf, af);
          const float cs = TS ? sa[0] * sw[0] : ssa[(j * 16 + (lane & 15)) * KBMAX + k] * swb;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(p[r], cs, acc[j][r]);
        }
      }
    }
  }

  // lane holds D[n = 16*wave + 4*(lane/16) + r][m = 16j + lane%16]
  const int64_t n = n0 + wave * 16 + (lane >> 4) * 4;
  if (n >= N) return;
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = j * 16 + (lane & 15);
    if (m >= M) continue;
    if (splits == 1) {
      uint2 o;
      o.x = bf16x2_rne(acc[j][0], acc[j][1]);
      o.y = bf16x2_rne(acc[j][2], acc[j][3]);
      *reinterpret_cast<uint2*>(C + m * N + n) = o;
    } else {
      // non-temporal: the partials are read once, by the reduce kernel (M = 64
      // on the decode shape: 14.0 -> 13.0 us per call)
      float* q = ws + (static_cast<int64_t>(sp) * M + m) * N + n;
      __builtin_nontemporal_store(acc[j][0], q);
      __builtin_nontemporal_store(acc[j][1], q + 1);
      __builtin_nontemporal_store(acc[j][2], q + 2);
      __builtin_nontemporal_store(acc[j][3], q + 3);
    }
  }
}

// C[m, n..n+3] = bf16(sum over splits s = 0, 1, ... of ws[s][m][n..n+3])
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float* __restrict__ ws,
                                                                  uint16_t* __restrict__ C,
                                                                  int64_t mn4, int splits) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= mn4) return;
  const float4* p = reinterpret_cast<const float4*>(ws) + i;
  // all loads in flight, then added in split order; the loads are streamed
  // (each partial is read once: N = 2048, K = 7168, M = 128 split-K GEMM and
  // reduce 16.5 -> 14.9 us, M = 256 / 512 unchanged)
  float4 v[kDecMaxSplits];
#pragma unroll
  for (int k = 0; k < kDecMaxSplits; ++k)
    if (k < splits) {
      const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p + k * mn4));
      v[k] = make_float4(t[0], t[1], t[2], t[3]);
    }
  float4 s = v[0];
#pragma unroll
  for (int k = 1; k < kDecMaxSplits; ++k)
    if (k < splits) { s.x += v[k].x; s.y += v[k].y; s.z += v[k].z; s.w += v[k].w; }
  uint2 o;
  o.x = bf16x2_rne(s.x, s.y);
  o.y = bf16x2_rne(s.z, s.w);
  reinterpret_cast<uint2*>(C)[i] = o;
}

struct DecodePlan {
  int kb_per;
  int splits;
};

// K split for the decode kernel: enough workgroups to keep ~512 in flight,
// at most kDecMaxKb K blocks per split
// (a W of at most kDecSmallW bytes is not worth spreading: one split unless K
// needs more, so no workspace and no second kernel)
constexpr int64_t kDecSmallW = int64_t{1} << 21;
inline DecodePlan decode_plan(int64_t N, int64_t K) {
  const int64_t KB = K / kBK;
  const int64_t ntiles = (N + kDecRows - 1) / kDecRows;
  int64_t want = N * K <= kDecSmallW ? 1 : (512 + ntiles - 1) / ntiles;
  want = std::max<int64_t>(want, (KB + kDecMaxKb - 1) / kDecMaxKb);
  want = std::min<int64_t>(want, KB);
  int kb_per = static_cast<int>((KB + want - 1) / want);
  kb_per = std::max(1, std::min(kb_per, kDecMaxKb));
  // at most kDecMaxSplits splits (raises K blocks per split; K beyond
  // kDecMaxSplits * kDecMaxKb blocks is rejected by the entry point)
  kb_per = std::max<int>(kb_per, static_cast<int>((KB + kDecMaxSplits - 1) / kDecMaxSplits));
  const int splits = static_cast<int>((KB + kb_per - 1) / kb_per);
  return {kb_per, splits};
}

inline bool use_decode(int64_t M) { return M <= kDecMaxM; }
// The chunked full-K kernel (below) serves 8 < M <= kFullMaxM for every N,
// and kFullMaxM < M <= 64 while N <= kFull2dMaxN (N / 8 workgroups: one per
// CU on 256 CUs); the split-K kernel and its reduce serve the rest of
// 32 < M <= 64.
constexpr int kFullMaxM = 32;
constexpr int64_t kFull2dMaxN = 2048;
inline bool use_split_k(int64_t M, int64_t N) { return use_decode(M) && M > kFullMaxM && N > kFull2dMaxN; }

size_t decode_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const DecodePlan p = decode_plan(N, K);
  return p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
}

template <bool TS>
int launch_decode(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* c,
                  float* ws, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const DecodePlan p = decode_plan(N, K);
  const dim3 grid(static_cast<unsigned>((N + kDecRows - 1) / kDecRows), static_cast<unsigned>(p.splits));
  const int m = static_cast<int>(M);
  const int mt = (m + 15) / 16;
#define FP8BS_DEC(MT, KBM)                                                                      \
  hipLaunchKernelGGL((gemm_blockscaled_decode_kernel<MT, KBM, TS>), grid, dim3(256), 0, st, a, sa, w, \
                     sw, c, ws, m, N, K, p.kb_per, p.splits)
#define FP8BS_DEC_KB(MT)                      \
  if (p.kb_per <= 4) FP8BS_DEC(MT, 4);        \
  else if (p.kb_per <= 8) FP8BS_DEC(MT, 8);   \
  else FP8BS_DEC(MT, 16);
  // M > 32 here (smaller M takes the kernels above)
  if (mt <= 3) {
    FP8BS_DEC_KB(3)
  } else {
    FP8BS_DEC_KB(4)
  }
#undef FP8BS_DEC_KB
#undef FP8BS_DEC
  if (p.splits > 1) {
    if (hipGetLastError() != hipSuccess) return FP8BS_ERR_LAUNCH;
    const int64_t mn4 = M * N / 4;
    hipLaunchKernelGGL(gemm_splitk_reduce_kernel, dim3(static_cast<unsigned>((mn4 + 255) / 256)), dim3(256), 0, st,
                       ws, c, mn4, p.splits);
  }
  return FP8BS_OK;
}

// ---------------------------------------------------------------------------
// Decode with A staged through LDS (8 < M <= 32, and 32 < M <= 64 when
// N <= kFull2dMaxN). The output is tiled in two dimensions: a workgroup
// takes NR W rows over the whole of K against one group of MP = 16 MT
// activation rows (blockIdx.y), with sixteen waves. A, W and both scales
// reach it through the per-CU copy path in that path's efficient form: 1 KiB
// copies (eight rows of 128 bytes, buffer loads with the LDS bit) of chunks
// of CB K blocks, two chunks in flight (three with 16 x 16 tiles). Fragment
// loads straight into registers touch sixteen half-used 128-byte lines per
// instruction and left the streaming kernel bound by A's loads once M passed
// 8. Wave w takes the K blocks kb = w (mod 16): per block, one MFMA per 16
// activation rows, then the scale FMAs. The sixteen waves' partial sums are
// added through LDS in wave order: deterministic, one launch, no workspace.
// Every global load of the kernel is one of these copies, so the kernel
// alone counts them when it waits.
//
// Every CU reads its W rows and its group's activation rows over all of K,
// so the shape of the tile sets the bytes per CU: 8 W rows (the MFMA's rows
// 8..15 repeat rows 0..7, and those outputs are dropped) against all M <= 16
// rows; 16 W rows against two groups of 16 rows for 16 < M <= 32 (32 rows
// per CU instead of 8 + 32); 16 W rows against two groups of 32 rows for
// 32 < M <= 64 (48 rows per CU instead of 8 + 64). The grid is N / 8 in
// every case; the two groups' workgroups of one W tile have ids 2048 / 16 =
// 128 apart, a multiple of 8, so they run on one XCD and the second read of
// their W rows comes from its L2. Decode shape (N = 2048, K = 7168,
// graph-replayed, rotated inputs): M = 12 / 16 / 24 / 32 in 7.0 / 7.2 /
// 8.2 / 8.2 us, and M = 33 / 48 / 64 in 9.8 / 9.9 / 10.1 us in one launch
// (the split-K kernel and its reduce: 10.6 / 11.0 / 11.9 us). Past
// N = 2048 the grid no longer fits one round of the CUs, and the split-K
// kernel is faster (M = 64, N = 4096: 17.7 against 18.9 us).
// ---------------------------------------------------------------------------
constexpr int kFullWaves = 16;
// MT: 16-row tiles of A per workgroup (MP = 16 MT rows, one M group);
// NR: W rows per workgroup (8: the MFMA's rows 8..15 repeat rows 0..7; 16)
template <int MT, int NR>
struct FullCfg {
  static constexpr int MP = 16 * MT;                    // A rows staged per M group
  static_assert(MT == 1 || MT == 2, "one or two 16-row tiles");
  static_assert(NR == 8 || NR == 16, "8 or 16 W rows");
  static constexpr int CB = MT == 1 && NR == 8 ? 16 : 8;   // K blocks per chunk
  // chunk buffers: three (two chunks in flight), four where they fit (16 W
  // rows against 16 activation rows: 8.0 against 8.2 us at M = 24; chunks of
  // 4 K blocks with five or six buffers were 15-30% slower everywhere)
  static constexpr int NBUF = MT == 1 && NR == 16 ? 4 : 3;
  static constexpr int kAChunk = MP * CB * 128;         // A bytes per chunk
  static constexpr int kWChunk = NR * CB * 128;         // W bytes per chunk
  static constexpr int kSChunk = (MP * CB * 4 + 1023) / 1024 * 1024;   // activation scales per chunk (padded to 1 KiB)
  static constexpr int kChunk = kAChunk + kWChunk + kSChunk + 256;   // + the weight scales
  static constexpr int kSCopies4 = MP * CB * 4 / 256;        // 256-byte scale copies per chunk
  static constexpr int kSRows16 = 256 / CB;                   // rows one 1 KiB scale copy covers
  static_assert(CB <= kFullWaves && MP * CB * 4 % 256 == 0 && kSCopies4 <= kFullWaves && MP <= kSRows16, "copies");
  static_assert(kFullWaves * MT * 64 * 16 <= NBUF * kChunk, "the waves' partial sums fit the chunk buffers");
  static_assert(NBUF * kChunk <= 160 * 1024, "LDS");
};

// SC16: the activation scales go in one 1 KiB copy per chunk (rows of K/128
// floats 16-byte aligned: K/128 a multiple of 4), else in 256-byte copies
template <int MT, int NR, bool TS, bool SC16>
__global__ __launch_bounds__(64 * kFullWaves) void gemm_blockscaled_decode_full_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, uint16_t* __restrict__ C, int M, int64_t N, int64_t K) {
  using F = FullCfg<MT, NR>;
  constexpr int MP = F::MP, CB = F::CB;
  // NBUF chunk buffers, each [A: CB blocks x MP rows x 128][W: CB blocks x NR
  // rows x 128][activation scales: MP x CB, padded to 1 KiB][weight scales: CB]
  __shared__ __attribute__((aligned(1024))) uint8_t lds[F::NBUF * F::kChunk];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * NR;
  const int m0 = static_cast<int>(blockIdx.y) * MP;      // first A row of this M group
  const int Mg = min(M - m0, MP);                         // its rows
  const int KB = static_cast<int>(K / kBK);
  const int nchunks = (KB + CB - 1) / CB;
  const uint32_t lds0 = lds_addr(lds);

  // Copies of chunk c: kTot copies, copy k issued by wave k % 16 (no copy is
  // issued twice: each copy instruction costs the copy path about the same
  // whatever its size, and repeating the small scale copies in every wave
  // cost 2-3 us per call at M = 64):
  // - A copy k < kACopies covers K block k / (MP/8) of the chunk and the
  //   group's rows 8 (k % (MP/8)) .. +7; lane l fetches row r = 8 (k % (MP/8))
  //   + l/8, the 16-byte piece that the row swizzle puts at LDS position
  //   l % 8. Rows at or past the group's last read zeros (range-checked
  //   buffer).
  // - W copies: NR/8 per K block of the chunk, eight of the workgroup's rows
  //   each, laid out like A.
  // - activation-scale copies: the chunk's [row][CB] floats, in one 1 KiB
  //   copy (4 floats a lane) when the rows are 16-byte aligned, else in
  //   256-byte copies of 64 floats.
  // - weight-scale copy: the chunk's CB weight scales (the workgroup's NR
  //   rows sit in one 128-row block; lanes past CB fetch floats never used).
  // Blocks past K/128 in the last chunk read the next row or zeros and are
  // never used.
  constexpr int kACopies = MP * CB / 8;
  constexpr int kWCopies = NR * CB / 8;
  constexpr int kSCopies = SC16 ? 1 : F::kSCopies4;
  constexpr int kTot = kACopies + kWCopies + (TS ? 0 : kSCopies + 1);
  const v4i_rsrc ar = make_rsrc(A + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(Mg * K));
  const v4i_rsrc wr = make_rsrc(W + n0 * K, static_cast<uint32_t>(NR * K));
  const v4i_rsrc sr = make_rsrc(sa + static_cast<int64_t>(m0) * KB, static_cast<uint32_t>(Mg * KB * 4));
  const v4i_rsrc swr = make_rsrc(sw + (n0 / 128) * KB, static_cast<uint32_t>(KB * 4));
  auto issue_chunk = [&](int c) {
    const uint32_t base = lds0 + (c % F::NBUF) * F::kChunk;
    for (int k = wave; k < kTot; k += kFullWaves) {
      if (k < kACopies) {
        const int cb = k / (MP / 8);
        const int r = 8 * (k % (MP / 8)) + (lane >> 3);
        const uint32_t off = static_cast<uint32_t>(r * K) + static_cast<uint32_t>(c * CB + cb) * kBK +
                             static_cast<uint32_t>(((lane & 7) ^ swz(r)) << 4);
        copy16_buf_to_lds(off, ar, base + k * 1024);
      } else if (k < kACopies + kWCopies) {
        const int idx = k - kACopies;
        const int cb = idx / (NR / 8);
        const int r = 8 * (idx % (NR / 8)) + (lane >> 3);
        const uint32_t off = static_cast<uint32_t>(r * K) + static_cast<uint32_t>(c * CB + cb) * kBK +
                             static_cast<uint32_t>(((lane & 7) ^ swz(r)) << 4);
        // non-temporal: W rows are streamed, A rows are read by every
        // workgroup of the group (N = 2048, K = 7168, alternating runs:
        // M = 16 / 32 / 64 from 7.3 / 8.1-8.2 / 10.0-10.1 to 7.0-7.1 / 7.9-8.0 /
        // 9.8-9.9 us; the sc0 or sc1 bits besides nt made no difference, sc1
        // alone none at all)
        copy16_buf_to_lds_nt(off, wr, base + F::kAChunk + idx * 1024);
      } else if (k < kACopies + kWCopies + kSCopies) {
        if constexpr (SC16) {
          const int r = (4 * lane) / CB, x = (4 * lane) % CB;
          copy16_buf_to_lds(static_cast<uint32_t>((r * KB + c * CB + x) * 4), sr, base + F::kAChunk + F::kWChunk);
        } else {
          const int s = k - kACopies - kWCopies;
          const int e = s * 64 + lane;
          const int r = e / CB, x = e % CB;
          copy4_buf_to_lds(static_cast<uint32_t>((r * KB + c * CB + x) * 4), sr,
                           base + F::kAChunk + F::kWChunk + s * 256);
        }
      } else {
        copy4_buf_to_lds(static_cast<uint32_t>((c * CB + lane) * 4), swr,
                         base + F::kAChunk + F::kWChunk + F::kSChunk);
      }
    }
  };
  // this wave's copies per chunk: the first kTot % 16 waves issue one more
  constexpr int kFew = kTot / kFullWaves, kExtra = kTot % kFullWaves;
  auto wait_chunks = [&](auto n) {   // all but this wave's copies of the last n chunks issued are done
    constexpr int kN = decltype(n)::value;
    if (wave < kExtra)
      wait_vmcnt<kN * (kFew + 1)>();
    else
      wait_vmcnt<kN * kFew>();
  };

  const float tscale = TS ? sa[0] * sw[0] : 0.0f;

  // chunks 0 .. NBUF-2 now; chunk c + NBUF - 1 right after the barrier that
  // opens chunk c (every wave is then done with chunk c-1, whose buffer it
  // refills), so NBUF - 1 chunks stay in flight behind the one computed
  for (int c = 0; c < F::NBUF - 1; ++c)
    if (c < nchunks) issue_chunk(c);

  v4f acc[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const int c0 = 2 * (lane >> 4);
  for (int c = 0; c < nchunks; ++c) {
    // chunk c's copies are done once at most those of the chunks issued
    // after it remain: min(NBUF - 2, nchunks - 1 - c) chunks
    const int after = min(F::NBUF - 2, nchunks - 1 - c);
    if (after >= 2)
      wait_chunks(std::integral_constant<int, 2>{});
    else if (after == 1)
      wait_chunks(std::integral_constant<int, 1>{});
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of chunk c-1 are back
    __builtin_amdgcn_s_barrier();
    if (c + F::NBUF - 1 < nchunks) issue_chunk(c + F::NBUF - 1);
    const uint8_t* chunk = lds + (c % F::NBUF) * F::kChunk;
    const float* ss = reinterpret_cast<const float*>(chunk + F::kAChunk + F::kWChunk);
    const float* sws = ss + F::kSChunk / 4;   // the weight scales follow the padded activation scales
    for (int x = (wave - c * CB) & 15; x < CB; x += 16) {
      const int kb = c * CB + x;
      if (kb >= KB) break;
      const float swb = TS ? 1.0f : sws[x];
      const v8i wf = lds_frag(chunk + F::kAChunk + x * NR * 128, lane & (NR - 1), c0);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const v8i af = lds_frag(chunk + x * MP * 128, j * 16 + (lane & 15), c0);
        const v4f p = mfma_16x16x128_fp8(wf, af);
        const float cs = TS ? tscale : ss[(j * 16 + (lane & 15)) * CB + x] * swb;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = __builtin_fmaf(p[r], cs, acc[j][r]);
      }
    }
  }
  // every wave is done with the chunk buffers (and no copy is in flight: the
  // last chunk waited for all of them)
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();

  // the waves' partial sums, [wave][j][lane] float4, over the chunk buffers
  float4* red = reinterpret_cast<float4*>(lds);
#pragma unroll
  for (int j = 0; j < MT; ++j)
    red[(wave * MT + j) * 64 + lane] = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
  __syncthreads();
  // thread t < (NR/4) Mg: activation row m = t / (NR/4) of the group, W rows
  // n0 + 4 q .. +3 (q = t % (NR/4)), which lane 16 q + m%16 of tile m/16
  // holds in every wave; added in wave order
  constexpr int Q = NR / 4;
  const int t = static_cast<int>(threadIdx.x);
  if (t < Q * Mg) {
    const int m = t / Q, q = t % Q;
    const int l = 16 * q + (m & 15), j = m >> 4;
    float4 s = red[j * 64 + l];
    for (int w = 1; w < kFullWaves; ++w) {
      const float4 u = red[(w * MT + j) * 64 + l];
      s.x += u.x; s.y += u.y; s.z += u.z; s.w += u.w;
    }
    uint2 o;
    o.x = bf16x2_rne(s.x, s.y);
    o.y = bf16x2_rne(s.z, s.w);
    *reinterpret_cast<uint2*>(C + static_cast<int64_t>(m0 + m) * N + n0 + 4 * q) = o;
  }
}

template <bool TS>
int launch_decode_full(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* c,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int m = static_cast<int>(M);
  const bool sc16 = TS || (K / kBK) % 4 == 0;
#define FP8BS_FULL(MT, NR, MG)                                                                              \
  do {                                                                                                      \
    const dim3 grid(static_cast<unsigned>(N / NR), MG);                                                     \
    if (sc16)                                                                                               \
      hipLaunchKernelGGL((gemm_blockscaled_decode_full_kernel<MT, NR, TS, true>), grid, dim3(64 * kFullWaves), \
                         0, st, a, sa, w, sw, c, m, N, K);                                                  \
    else                                                                                                    \
      hipLaunchKernelGGL((gemm_blockscaled_decode_full_kernel<MT, NR, TS, false>), grid, dim3(64 * kFullWaves), \
                         0, st, a, sa, w, sw, c, m, N, K);                                                  \
  } while (0)
  // N / 8 workgroups in each case
  if (m <= 16) {
    FP8BS_FULL(1, 8, 1);
  } else if (m <= 32) {
    FP8BS_FULL(1, 16, 2);
  } else {
    FP8BS_FULL(2, 16, 2);
  }
#undef FP8BS_FULL
  return FP8BS_OK;
}

// Test hook: the matrix cores' dot product of one K block, as every GEMM
// kernel here computes it (mfma_16x16x128_fp8, accumulator input 0). Tile t
// holds 16 W rows and 16 A rows of 128 codes; the wave's lanes load them in
// the fragment layout of the GEMM kernels and store the fp32 16x16 result
// D[t][n][m] = sum_k W[t][n][k] * A[t][m][k].
__global__ __launch_bounds__(64) void debug_mfma_block_kernel(const uint8_t* __restrict__ A,
                                                               const uint8_t* __restrict__ W,
                                                               float* __restrict__ D, int64_t tiles) {
  const int64_t t = blockIdx.x;
  if (t >= tiles) return;
  const int lane = threadIdx.x;
  const int64_t off = t * 2048 + (lane & 15) * 128 + 32 * (lane >> 4);
  const uint4 a0 = *reinterpret_cast<const uint4*>(A + off);
  const uint4 a1 = *reinterpret_cast<const uint4*>(A + off + 16);
  const uint4 w0 = *reinterpret_cast<const uint4*>(W + off);
  const uint4 w1 = *reinterpret_cast<const uint4*>(W + off + 16);
  const v8i af = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i wf = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
  const v4f d = mfma_16x16x128_fp8(wf, af);
  // lane holds D[n = 4 * (lane / 16) + r][m = lane % 16]
  float* o = D + t * 256 + (lane & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r) o[(4 * (lane >> 4) + r) * 16] = d[r];
}

template <int BN, int BM, int WN, int WM, int STAGES, int WPE, int MODE>
int launch_tiled(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* c,
                 int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t grid = (tiles_m * tiles_n + 7) / 8 * 8;
  if (grid > 0x7FFFFFF0LL) return FP8BS_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_blockscaled_tiled_kernel<BN, BM, WN, WM, STAGES, WPE, MODE>),
                     dim3(static_cast<unsigned>(grid)), dim3(64 * WN * WM), 0, st, a, sa, w, sw, c,
                     M, N, K, static_cast<int>(tiles_m), static_cast<int>(tiles_n));
  return FP8BS_OK;
}

// Split K for the tiled kernel. Past the decode kernels (M > 64), an output
// with fewer 128 x 128 tiles than CUs leaves most of the chip idle while each
// workgroup walks all of K (N = 2048, K = 7168: M = 96 to 1024 all took about
// 48 us, against 10 us at M = 64). K is then split so that about one
// 128 x 128 workgroup per CU runs (at most kDecMaxSplits splits); each split
// stores fp32 partial sums and gemm_splitk_reduce_kernel adds them in split
// order (deterministic) and rounds to bf16. N = 2048, K = 7168: M = 96 / 128
// / 256 / 512 / 1024 in 16.3 / 16.6 / 19.5 / 26.9 / 38.1 us against 49.6 /
// 50.7 / 47.5 / 48.9 / 48.8 us; K = 2048: M = 130, N = 384 in 9.2 against
// 14.4 us, M = 300, N = 1024 in 12.0 against 14.2 us. A short K gains less
// than the partials and the reduce launch cost once the tiles are many or K
// is shorter still (M = 128, N = 7168, K = 2048: 17.2 against 17.0 us; M = 96,
// N = 256, K = 1024 with one scale per tensor: 9.5 against 7.0 us), so K is
// split from 32 blocks, or from 16 blocks with at most 32 tiles. A target of
// two workgroups per CU was slower (M = 128: 22.7 us).
constexpr int64_t kSplitCUs = 256;      // MI355X's CUs: the plan (and the workspace size) is per shape
struct TiledSplit {
  int splits;
  int kb_per;
};
inline TiledSplit tiled_split_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t KB = K / kBK;
  const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (use_decode(M) || tiles256 >= kSplitCUs || tiles128 >= kSplitCUs || KB < 16 || (KB < 32 && tiles128 > 32))
    return {1, static_cast<int>(KB)};
  int64_t want = (kSplitCUs + tiles128 - 1) / tiles128;
  want = std::min<int64_t>(std::min<int64_t>(want, KB), kDecMaxSplits);
  const int kb_per = static_cast<int>((KB + want - 1) / want);
  return {static_cast<int>((KB + kb_per - 1) / kb_per), kb_per};
}

template <int MODE>
int launch_tiled_split(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* c,
                       float* ws, int64_t M, int64_t N, int64_t K, const TiledSplit& p, hipStream_t st) {
  const int64_t tiles_m = (M + 127) / 128;
  const int64_t tiles_n = (N + 127) / 128;
  const int64_t grid = (tiles_m * tiles_n + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_blockscaled_tiled_kernel<128, 128, 2, 2, 2, 2, MODE, true>),
                     dim3(static_cast<unsigned>(grid), static_cast<unsigned>(p.splits)), dim3(256), 0, st, a, sa,
                     w, sw, c, M, N, K, static_cast<int>(tiles_m), static_cast<int>(tiles_n), ws, p.kb_per);
  if (hipGetLastError() != hipSuccess) return FP8BS_ERR_LAUNCH;
  const int64_t mn4 = M * N / 4;
  hipLaunchKernelGGL(gemm_splitk_reduce_kernel, dim3(static_cast<unsigned>((mn4 + 255) / 256)), dim3(256), 0, st,
                     ws, c, mn4, p.splits);
  return FP8BS_OK;
}

// Sizes every GEMM entry point accepts: K and N multiples of 128, products
// that fit int64, K at most 2^22, and for the split-K decode kernel at most
// kDecMaxSplits * kDecMaxKb K blocks.
inline bool gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return false;
  if (M > (INT64_MAX / K) || M > (INT64_MAX / N) || N > (INT64_MAX / K)) return false;
  if (K > (int64_t{1} << 22) || (M + 127) / 128 > 0x7FFFFFFF) return false;
  if (use_split_k(M, N) && K / 128 > static_cast<int64_t>(kDecMaxSplits) * kDecMaxKb)
    return false;
  return true;
}

}  // namespace
}  // namespace fp8bs

using namespace fp8bs;

extern "C" {

size_t fp8_gemm_blockscaled_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!gemm_shape_ok(M, N, K)) return 0;
  if (use_split_k(M, N)) return decode_workspace_bytes(M, N, K);
  const TiledSplit p = tiled_split_plan(M, N, K);
  return p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
}

}  // extern "C"

namespace fp8bs {
namespace {
template <int MODE>
int gemm_blockscaled(const void* a_e4m3, const float* a_scale, const void* w_e4m3, const float* w_scale,
                     void* c_bf16, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!a_e4m3 || !a_scale || !w_e4m3 || !w_scale || !c_bf16) return FP8BS_ERR_NULL;
  if (!gemm_shape_ok(M, N, K)) return FP8BS_ERR_SHAPE;
  if (!aligned(a_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(c_bf16, 16) ||
      !aligned(a_scale, 4) || !aligned(w_scale, 4))
    return FP8BS_ERR_ALIGN;
  const size_t need = fp8_gemm_blockscaled_workspace_bytes(M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FP8BS_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return FP8BS_ERR_ALIGN;   // the reduce reads float4
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  const uint8_t* a = static_cast<const uint8_t*>(a_e4m3);
  const uint8_t* w = static_cast<const uint8_t*>(w_e4m3);
  uint16_t* c = static_cast<uint16_t*>(c_bf16);
  hipStream_t st = as_stream(stream);
  (void)hipGetLastError();
  int rc;
  // decode shapes are bound by streaming W: the FMA kernels serve both scale
  // formats (with power-of-two scales the scale product is exact there too)
  if (use_decode(M)) {
    if (M <= kDecStreamMaxM)
      rc = launch_decode_stream<MODE == 2>(a, a_scale, w, w_scale, c, M, N, K, st);
    else if (!use_split_k(M, N))
      rc = launch_decode_full<MODE == 2>(a, a_scale, w, w_scale, c, M, N, K, st);
    else
      rc = launch_decode<MODE == 2>(a, a_scale, w, w_scale, c, static_cast<float*>(workspace), M, N, K, st);
    if (rc != FP8BS_OK) return rc;
    return launch_status();
  }
  // 256 x 256 tiles (eight waves, two per SIMD) when they fill the chip,
  // else 128 x 128 tiles (two workgroups per CU)
  // (K split when even the 128 x 128 tiles are fewer than the CUs)
  const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
  const TiledSplit sp = tiled_split_plan(M, N, K);
  if (tiles256 >= dev.num_cus)
    rc = launch_tiled<256, 256, 2, 4, 2, 2, MODE>(a, a_scale, w, w_scale, c, M, N, K, st);
  else if (sp.splits > 1)
    rc = launch_tiled_split<MODE>(a, a_scale, w, w_scale, c, static_cast<float*>(workspace), M, N, K, sp, st);
  else
    rc = launch_tiled<128, 128, 2, 2, 2, 2, MODE>(a, a_scale, w, w_scale, c, M, N, K, st);
  if (rc != FP8BS_OK) return rc;
  return launch_status();
}

}  // namespace
}  // namespace fp8bs

extern "C" {

int fp8_gemm_blockscaled(const void* a_e4m3, const float* a_scale, const void* w_e4m3,
                         const float* w_scale, void* c_bf16, int64_t M, int64_t N, int64_t K,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_blockscaled<0>(a_e4m3, a_scale, w_e4m3, w_scale, c_bf16, M, N, K, workspace,
                             workspace_bytes, stream);
}

int fp8_gemm_blockscaled_ue8m0(const void* a_e4m3, const float* a_scale, const void* w_e4m3,
                               const float* w_scale, void* c_bf16, int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_blockscaled<1>(a_e4m3, a_scale, w_e4m3, w_scale, c_bf16, M, N, K, workspace,
                             workspace_bytes, stream);
}

int fp8_gemm_tensorscaled(const void* a_e4m3, const float* a_scale, const void* w_e4m3,
                          const float* w_scale, void* c_bf16, int64_t M, int64_t N, int64_t K,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_blockscaled<2>(a_e4m3, a_scale, w_e4m3, w_scale, c_bf16, M, N, K, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"

namespace fp8bs {
namespace {
inline int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }
// the two-launch form runs the GEMM's own checks, so the call accepts what
// the GEMM accepts (the one-kernel form has no further limit)
inline bool act_gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
  return gemm_shape_ok(M, N, K);
}
}  // namespace
}  // namespace fp8bs

extern "C" {

size_t fp8_act_quant_gemm_blockscaled_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!act_gemm_shape_ok(M, N, K) || fused_fits(M, K)) return 0;
  return static_cast<size_t>(round256(M * K) + round256(M * (K / kBK) * 4)) +
         fp8_gemm_blockscaled_workspace_bytes(M, N, K);
}

int fp8_act_quant_gemm_blockscaled(const void* x_bf16, const void* w_e4m3, const float* w_scale, void* c_bf16,
                                   int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!x_bf16 || !w_e4m3 || !w_scale || !c_bf16) return FP8BS_ERR_NULL;
  if (!act_gemm_shape_ok(M, N, K)) return FP8BS_ERR_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(w_e4m3, 16) || !aligned(c_bf16, 16) || !aligned(w_scale, 4))
    return FP8BS_ERR_ALIGN;
  if (fused_fits(M, K)) {
    const DeviceInfo dev = current_device();
    if (dev.status != FP8BS_OK) return dev.status;
    (void)hipGetLastError();
    launch_act_quant_gemm_decode(x_bf16, static_cast<const uint8_t*>(w_e4m3), w_scale,
                                 static_cast<uint16_t*>(c_bf16), M, N, K, as_stream(stream));
    return launch_status();
  }
  // two launches through the workspace: block act-quant, then the GEMM
  const size_t need = fp8_act_quant_gemm_blockscaled_workspace_bytes(M, N, K);
  if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FP8BS_ERR_ALIGN;
  uint8_t* q = static_cast<uint8_t*>(workspace);
  float* sa = reinterpret_cast<float*>(q + round256(M * K));
  uint8_t* gws = q + round256(M * K) + round256(M * (K / kBK) * 4);
  const size_t gws_bytes = need - static_cast<size_t>(gws - q);
  int rc = fp8_act_quant_block(x_bf16, M, K, q, sa, stream);
  if (rc != FP8BS_OK) return rc;
  return fp8_gemm_blockscaled(q, sa, w_e4m3, w_scale, c_bf16, M, N, K, gws_bytes ? gws : nullptr, gws_bytes,
                              stream);
}

}  // extern "C"

extern "C" {

int fp8bs_debug_mfma_block(const void* a_e4m3, const void* w_e4m3, float* d, int64_t tiles, void* stream) {
  if (!a_e4m3 || !w_e4m3 || !d) return FP8BS_ERR_NULL;
  if (tiles < 1 || tiles > 0x7FFFFFFF) return FP8BS_ERR_SHAPE;
  if (!aligned(a_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(d, 4)) return FP8BS_ERR_ALIGN;
  const DeviceInfo dev = current_device();
  if (dev.status != FP8BS_OK) return dev.status;
  (void)hipGetLastError();
  hipLaunchKernelGGL(debug_mfma_block_kernel, dim3(static_cast<unsigned>(tiles)), dim3(64), 0, as_stream(stream),
                     static_cast<const uint8_t*>(a_e4m3), static_cast<const uint8_t*>(w_e4m3), d, tiles);
  return launch_status();
}

}  // extern "C"
