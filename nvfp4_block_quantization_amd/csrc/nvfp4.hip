// nvfp4.hip -- gfx950 kernels and the C ABI (include/nvfp4.h) of libnvfp4.so.
//
// Kernels:
//   amax_partial / amax_finish  per-tensor amax: grid-stride 16-byte loads, one
//                               partial per workgroup, a one-workgroup finish
//                               (no atomics, so the result is order-free).
//   quant_row                   1x16 row blocks, row-wise copy only: a flat
//                               stream of 16-element blocks, one block per lane,
//                               optional Hadamard transform and stochastic
//                               rounding, Four Over Six in registers.
//   quant_strip                 256x64 strips for the column-wise copy and
//                               16x16 tiles: row blocks from registers, each
//                               64x64 sub-tile (and its random words) staged in
//                               LDS and read back by columns; the column copy
//                               leaves as whole 128-byte lines.
//   dequant_rows                codes + scales (+ S_t) -> fp32, row by row.
//   MXFP4                       the row and strip kernels instantiated for
//                               32-element blocks with E8M0 scales (no tensor
//                               scale); dequant_rows reads their E8M0 scales.
//   err_stats                   round-to-nearest quantization binned by scaled
//                               value: counts and squared errors, with an
//                               exact-scale reference.
// The FP4 GEMMs that consume the quantized copies are in gemm.hip.
#include "nvfp4_device.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <math.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "nvfp4.h"

namespace nvfp4 {

constexpr int kBF16 = NVFP4_IN_BF16;
constexpr int kF32 = NVFP4_IN_F32;
constexpr int kThreads = 256;

// ---------------------------------------------------------------- params ---

struct QuantParams {
  const float* amax;
  float cap6;        // fl(6 * scale_cap), exact for 448 and 256
  uint32_t rht_mask;
  uint32_t k0, k1;   // Philox key (stochastic rounding)
  int64_t row_offset;  // global row of row 0 (tile kernel)
  int64_t idx_base;    // row_offset * cols: element index of the first element (row kernel)
  int idx_below_2_34;  // every element index of the launch is below 2^34: Philox counters have high word 0
  int emit_row, emit_col;
  uint8_t* codes_row;
  uint8_t* scales_row;
  uint8_t* codes_col;
  uint8_t* scales_col;
  float* tensor_scale;
};

struct TensorScale {
  float st;
  Divisor den6, den4;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming load of input read exactly once.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// S_t = fl(amax / fl(6 * cap)); the candidates divide the block max by
// fl(6 * S_t) and fl(4 * S_t).
__device__ __forceinline__ TensorScale tensor_scale(const float* amax, float cap6) {
  TensorScale t;
  t.st = __fdiv_rn(*amax, cap6);
  t.den6 = make_divisor(6.0f * t.st);
  t.den4 = make_divisor(4.0f * t.st);
  return t;
}

// Load 16 consecutive input elements (16-byte aligned) as binary32.
template <int DT>
__device__ __forceinline__ void load16(const void* __restrict__ x, int64_t elem0, float* y) {
  if constexpr (DT == kBF16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + elem0);
    const uint4 a = p[0], b = p[1];
    unpack_bf16x8(a, y);
    unpack_bf16x8(b, y + 8);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + elem0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = p[j];
      y[4 * j] = v.x;
      y[4 * j + 1] = v.y;
      y[4 * j + 2] = v.z;
      y[4 * j + 3] = v.w;
    }
  }
}

// ------------------------------------------------------------------ amax ---

__device__ __forceinline__ float block_max256(float m, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int DT>
__device__ __forceinline__ float vec_absmax(uint4 q) {
  if constexpr (DT == kBF16) {
    // |bf16| as the high half of a binary32 with the sign bit cleared
    const float a = fmaxf(__uint_as_float((q.x << 16) & 0x7FFFFFFFu), __uint_as_float(q.x & 0x7FFF0000u));
    const float b = fmaxf(__uint_as_float((q.y << 16) & 0x7FFFFFFFu), __uint_as_float(q.y & 0x7FFF0000u));
    const float c = fmaxf(__uint_as_float((q.z << 16) & 0x7FFFFFFFu), __uint_as_float(q.z & 0x7FFF0000u));
    const float d = fmaxf(__uint_as_float((q.w << 16) & 0x7FFFFFFFu), __uint_as_float(q.w & 0x7FFF0000u));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
  } else {
    return fmaxf(fmaxf(fabsf(__uint_as_float(q.x)), fabsf(__uint_as_float(q.y))),
                 fmaxf(fabsf(__uint_as_float(q.z)), fabsf(__uint_as_float(q.w))));
  }
}

// Without the transform: n elements as 16-byte vectors; each workgroup walks
// contiguous chunks of kThreads * kAmaxDepth vectors with kAmaxDepth loads in
// flight per thread.  With it: n / 16
// blocks of 16, each transformed in registers.
constexpr int kAmaxDepth = 8;

template <int DT, bool RHT>
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const void* __restrict__ x, int64_t n,
                                                                uint32_t mask, float* __restrict__ partials) {
  __shared__ float red[4];
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * kThreads;
  float m = 0.0f;
  if constexpr (!RHT) {
    constexpr int VEC = DT == kBF16 ? 8 : 4;
    const int64_t nv = n / VEC;
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    // workgroup-contiguous chunks: each load instruction of a workgroup covers 4 KB
    const int64_t chunk = (int64_t)kThreads * kAmaxDepth;
    const int64_t nchunk = nv / chunk;
    for (int64_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
      const uint4* base = xv + c * chunk + threadIdx.x;
      uint4 q[kAmaxDepth];
#pragma unroll
      for (int u = 0; u < kAmaxDepth; ++u) q[u] = load_stream(base + u * kThreads);
#pragma unroll
      for (int u = 0; u < kAmaxDepth; ++u) m = fmaxf(m, vec_absmax<DT>(q[u]));
    }
    for (int64_t v = nchunk * chunk + tid; v < nv; v += nth) m = fmaxf(m, vec_absmax<DT>(xv[v]));
    for (int64_t e = nv * VEC + tid; e < n; e += nth) {
      float f;
      if constexpr (DT == kBF16) f = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[e] << 16);
      else f = reinterpret_cast<const float*>(x)[e];
      m = fmaxf(m, fabsf(f));
    }
  } else {
    const int64_t nb = n / 16;
    for (int64_t b = tid; b < nb; b += nth) {
      float y[16];
      load16<DT>(x, 16 * b, y);
      rht16(y, mask);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(y[i]));
    }
  }
  m = block_max256(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void amax_finish_kernel(const float* __restrict__ partials, int n,
                                                               float* __restrict__ amax) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, partials[i]);
  m = block_max256(m, red);
  if (threadIdx.x == 0) amax[0] = m;
}

// Each workgroup: S_t, its (d, 1/d) table for the 127 E4M3 codes, and (block 0)
// the tensor-scale output.
__device__ __forceinline__ TensorScale workgroup_setup(const QuantParams& p, f32x2* tab) {
  const TensorScale ts = tensor_scale(p.amax, p.cap6);
  fill_scale_table(tab, ts.st);
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.tensor_scale) p.tensor_scale[0] = ts.st;
  __syncthreads();
  return ts;
}

// A raw buffer resource over `bytes` bytes at `base`: accesses at offsets past
// the range are dropped by the hardware (stores) or return zero (loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------- row-wise, 1x16 ---

// The row copy of 1x16 blocks needs no neighbour: the tensor is a flat stream
// of 16-element blocks.  One block per lane; a chunk is U blocks per lane with
// each wave instruction loading 64 consecutive blocks.  Persistent workgroups
// walk the chunks and prefetch the next chunk's input while quantizing the
// current one (ping-pong register buffers); a grid of one workgroup per chunk
// runs the same kernel once through.  Loads and stores go through
// buffer resources that end where the chunk's blocks end, so no lane branches
// around a memory access and every wait for a prefetched chunk is exact.
template <int DT>
struct RawBlock {
  uint4 v[DT == kBF16 ? 2 : 4];
};

template <int DT>
__device__ __forceinline__ void unpack_raw(const RawBlock<DT>& r, float* y) {
  if constexpr (DT == kBF16) {
    unpack_bf16x8(r.v[0], y);
    unpack_bf16x8(r.v[1], y + 8);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y[4 * j] = __uint_as_float(r.v[j].x);
      y[4 * j + 1] = __uint_as_float(r.v[j].y);
      y[4 * j + 2] = __uint_as_float(r.v[j].z);
      y[4 * j + 3] = __uint_as_float(r.v[j].w);
    }
  }
}

template <int DT, bool RHT, bool SR, int RULE, int U, bool MX>
struct RowChunk {
  RawBlock<DT> raw[U];
  static constexpr uint32_t kBlockBytes = DT == kBF16 ? 32u : 64u;
  static constexpr int64_t kPer = (int64_t)kThreads * U;  // blocks per chunk

  // Blocks of chunk c that exist (0 .. kPer).
  __device__ __forceinline__ static int64_t valid_blocks(int64_t c, int64_t nblocks) {
    const int64_t left = nblocks - c * kPer;
    return left <= 0 ? 0 : (left < kPer ? left : kPer);
  }
  // This lane's u-th block, counted from the chunk's first block.
  __device__ __forceinline__ static uint32_t local(int u) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (uint32_t)(wave * (64 * U) + 64 * u + lane);
  }
  // Every lane issues the same loads whether or not its block exists: the
  // buffer resource covers the chunk's existing blocks and returns zeros past
  // them, so the waits for a prefetched chunk count its loads exactly.
  __device__ __forceinline__ void load(const void* __restrict__ x, int64_t c, int64_t nblocks) {
    const int64_t nv = valid_blocks(c, nblocks);
    const char* base = reinterpret_cast<const char*>(x) + (nv > 0 ? c * kPer * kBlockBytes : 0);
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(const_cast<char*>(base), (uint32_t)(nv * kBlockBytes));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = local(u) * kBlockBytes;
#pragma unroll
      for (int j = 0; j < (int)(kBlockBytes / 16); ++j) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * j, 0, 0);
        raw[u].v[j] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  __device__ __forceinline__ void process(int64_t c, int64_t nblocks, const QuantParams& p, const f32x2* tab,
                                          const TensorScale& ts, const PhiloxKey& key) const {
    constexpr uint32_t kDrop = 0xFFFFFFF0u;
    const int64_t nv = valid_blocks(c, nblocks);
    const int64_t b0 = nv > 0 ? c * kPer : 0;
    // stores past the chunk's existing blocks are dropped by the hardware
    const __amdgpu_buffer_rsrc_t rc = raw_rsrc(p.codes_row + 8 * b0, (uint32_t)(8 * nv));
    const __amdgpu_buffer_rsrc_t rsc =
        raw_rsrc(p.scales_row + (MX ? b0 / 2 : b0), (uint32_t)(MX ? nv / 2 : nv));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t lb = local(u);
      const int64_t b = b0 + lb;  // the block's index (its words' counter); past the end only for dropped stores
      float y[16];
      unpack_raw<DT>(raw[u], y);
      if constexpr (RHT) rht16(y, p.rht_mask);
      uint32_t w[16];
      if constexpr (SR) {
        const uint64_t idx0 = (uint64_t)p.idx_base + (uint64_t)(16 * b);
        if (p.idx_below_2_34) {  // uniform
          sr_words16_hi_uniform((uint32_t)(idx0 >> 2), 0u, key, w);
        } else {
          sr_words16(idx0, key, w);
        }
      }
      if constexpr (MX) {
        // a 32-element block is the 16-element halves of lanes 2k and 2k + 1
        float m = absmax16(y);
        m = fmaxf(m, dpp<kDppXor1>(m));
        const uint32_t code = mx_scale_code(m);
        const BlockCodes cc = mx_round16<SR>(y, code, w);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{cc.lo, cc.hi}, rc, 8u * lb, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, rsc, (lb & 1) == 0 ? (lb >> 1) : kDrop, 0, 0);
      } else {
        // 4/6 decided from the error estimates where they suffice, as in the
        // strip kernel: 5 more VGPRs (a wave less per SIMD), yet 2-3% faster on
        // the 1x16 activation shape and as fast on the gradient shape
        const BlockResult r = quant_block16<SR, RULE, true>(y, w, tab, ts.den6, ts.den4);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{r.codes.lo, r.codes.hi}, rc, 8u * lb, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)r.sb, rsc, lb, 0, 0);
      }
    }
  }
};

template <int DT, bool RHT, bool SR, int RULE, int U, bool MX>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(const void* __restrict__ x, int64_t nblocks,
                                                             QuantParams p) {
  __shared__ f32x2 tab[128];
  TensorScale ts{};
  if constexpr (!MX) ts = workgroup_setup(p, tab);
  const int64_t per_chunk = (int64_t)kThreads * U;
  const int64_t nchunks = (nblocks + per_chunk - 1) / per_chunk;
  const int64_t G = gridDim.x;
  const PhiloxKey key = philox_key(p.k0, p.k1);
  RowChunk<DT, RHT, SR, RULE, U, MX> A, B;
  int64_t c = blockIdx.x;
  A.load(x, c, nblocks);
  if (G >= nchunks) {  // one chunk per workgroup
    A.process(c, nblocks, p, tab, ts, key);
    return;
  }
  // Branch-free trips: chunks past the end load zeros and store nothing; the
  // loop leaves (uniformly) rather than quantize a chunk that does not exist.
  for (; c < nchunks; c += 2 * G) {
    B.load(x, c + G, nblocks);
    A.process(c, nblocks, p, tab, ts, key);
    if (c + G >= nchunks) break;
    A.load(x, c + 2 * G, nblocks);
    B.process(c + G, nblocks, p, tab, ts, key);
  }
}

// ------------------------------------------ strips: column copy and 2D ---

// A workgroup owns a strip of 256 rows x 64 columns and walks it as four
// 64x64 sub-tiles.  In a sub-tile, lanes 16g..16g+15 (one DPP row) own the
// 16x16 block g: one block row per lane in the row pass, one block column per
// lane in the column pass; every LDS exchange of a sub-tile stays inside one
// wave (wave w owns rows 16w .. 16w + 15 in both passes), so waves run free of
// each other until the strip's end (16x16 tiles need no column pass: their
// column copy's codes are the row copy's, transposed across the DPP row).  The
// row copy is stored straight from registers.  The column copy of a 256-row
// strip is one full 128-byte line per column of the output (256 rows x 4
// bits), so its codes and scales are collected in LDS and written at the end
// with 16-byte stores, 8 whole lines per wave instruction.  The input is read
// once, with streaming (non-temporal) loads that do not displace the partly
// written output lines from the L2.
constexpr int kStripRows = 256;

// Wave-private LDS exchange: wait until this wave's LDS accesses have completed
// and keep the compiler from moving memory operations across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_wave_barrier();
}
constexpr int64_t kStripMaxCols = 1ll << 24;  // column copies and 16x16 tiles: at most 2^24 columns

__device__ __forceinline__ uint32_t xcd_order(uint32_t bid, uint32_t nb) {
  const uint32_t q = nb >> 3, rem = nb & 7;
  const uint32_t xcd = bid & 7, slot = bid >> 3;
  return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

// Strips are enumerated in blocks of 4 strip-rows x 32 strip-columns (1024
// rows x 2048 columns; strip-rows fastest inside a block, blocks row by row) and
// each XCD takes one contiguous range of that order (xcd_order).  The strips
// whose row copies share a 128-byte line (4 side by side) and those whose
// column-copy scales share one (NVFP4 1D: 8 above one another, as 2 lines of 4)
// are then on one XCD at the same time and their pieces meet in its L2, while
// each row is still read in 2 KB runs.  (Measured against column-fastest order:
// HBM writes fall from 1.06-1.19x to 1.00-1.02x the algorithmic bytes.)
constexpr uint32_t kBlockY = 4, kBlockX = 32;

__device__ __forceinline__ void strip_coords(uint32_t s, uint32_t strips_y, uint32_t strips_x, uint32_t& sy,
                                             uint32_t& sx) {
  const uint32_t full = kBlockY * strips_x;  // strips in one full block-row
  const uint32_t brow = s / full;
  const uint32_t by = min(kBlockY, strips_y - kBlockY * brow);
  const uint32_t t = s - brow * full;
  const uint32_t bcol = t / (by * kBlockX), l = t - bcol * (by * kBlockX);
  sy = kBlockY * brow + l % by;
  sx = kBlockX * bcol + l / by;
}

// Block formats of the strip kernel.
enum StripFormat : int {
  kFmt1D = 0,  // NVFP4 1x16 row blocks and 16x1 column blocks
  kFmt2D = 1,  // NVFP4 16x16 tiles, one scale shared by both copies
  kFmtMX = 2   // MXFP4 1x32 row blocks and 32x1 column blocks
};

template <int DT, int FMT, bool SR, int RULE>
__global__ __launch_bounds__(kThreads) void quant_strip_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                               uint32_t strips_x, QuantParams p) {
  constexpr bool TWO_D = FMT == kFmt2D;
  constexpr bool MX = FMT == kFmtMX;
  // The staged sub-tile keeps the input's own width: bf16 inputs are staged as
  // bf16 (a 9 KB array instead of 17 KB, so four workgroups fit in a CU's LDS)
  // and widened again when read; binary32 inputs are staged as binary32.
  constexpr bool HALF = DT == kBF16;
  constexpr int VP = HALF ? 36 : 68;  // LDS pitch (dwords) of the staged sub-tile: 64 values + 16 bytes of padding
  // LDS pitch (dwords) of the staged random words, odd: the row pass stores word
  // k of lanes (row 16 bi + i, columns 16 bj ..) at row * WP + 16 bj + k, which
  // an odd pitch spreads over 64 distinct banks (a pitch of 68 put four lanes
  // on each bank); the column pass reads 64 consecutive words of a row
  constexpr int WP = SR ? 65 : 1;
  constexpr int CP = kStripRows / 8 + 4;  // LDS pitch (dwords) of the column-copy codes: the strip's bytes + 16
  constexpr int TR = kStripRows / 16;     // 16-row blocks (and 2D tile rows) per strip
  // column-copy scale bytes per column of the strip: 16 (NVFP4 1D), 8 (MXFP4); 2D: 16 per tile column
  constexpr int SPC = MX ? kStripRows / 32 : kStripRows / 16;
  // 16-byte accesses (staging, line collection, write-out) need 16-byte alignment
  __shared__ f32x2 tab[128];
  // (16x16 tiles need no staging: their column copy is the row copy transposed)
  __shared__ __attribute__((aligned(16))) uint32_t lds_v[TWO_D ? 1 : 64 * VP];
  __shared__ __attribute__((aligned(16))) uint32_t lds_w[SR && !TWO_D ? 64 * WP : 1];
  __shared__ __attribute__((aligned(16))) uint32_t col_codes[64 * CP];
  __shared__ __attribute__((aligned(16))) uint32_t col_scales[TWO_D ? TR : 64 * SPC / 4];
  __shared__ float lds_m[MX ? 4 * 64 : 1];  // MXFP4: column maxima of each wave's 16 rows

  uint32_t sy, sx;
  strip_coords(xcd_order(blockIdx.x, gridDim.x), (uint32_t)((rows + kStripRows - 1) / kStripRows), strips_x, sy, sx);
  const int t = threadIdx.x, g = t >> 4, i = t & 15;
  const int bi = g >> 2, bj = g & 3;
  const PhiloxKey key = philox_key(p.k0, p.k1);
  const int64_t sr0 = (int64_t)sy * kStripRows;           // first row of the strip
  const int64_t c0 = (int64_t)sx * 64 + 16 * bj;          // first column of this lane's blocks
  const int64_t rows_left = rows - sr0;
  const int nsub = (int)((rows_left < kStripRows ? rows_left : kStripRows) + 63) / 64;
  const bool col_ok = c0 < cols;

  // Element index of this lane's first element in sub-tile q: E(q) + L, with
  // E(q) = sr0 * cols + 64 sx + 64 q cols the same for the whole workgroup and
  // L = (16 bi + i) cols + 16 bj the lane's offset inside the sub-tile.  Input,
  // output and random-stream addresses are a uniform base plus a 32-bit lane
  // offset (cols <= 2^24, checked on the host, keeps L times the element size
  // below 2^32).
  const int64_t e_step = 64 * cols;
  const uint32_t L = (uint32_t)(16 * bi + i) * (uint32_t)cols + 16u * (uint32_t)bj;
  const uint32_t lmax = 63u * (uint32_t)cols + 48u;  // the largest L in the workgroup
  constexpr uint32_t ES = DT == kBF16 ? 2u : 4u;     // input bytes per element
  auto lane_valid = [&](int q) { return col_ok && sr0 + 64 * q + 16 * bi < rows; };  // whole 16x16 blocks
  // Input of sub-tile q for this lane (lanes of blocks outside the tensor read
  // the sub-tile's first elements, which exist, and store nothing).
  auto load_sub = [&](int q, int64_t eq, RawBlock<DT>& raw) {
    const uint32_t off = lane_valid(q) ? L * ES : 0u;
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + eq * ES + off);
#pragma unroll
    for (int j = 0; j < (DT == kBF16 ? 2 : 4); ++j) raw.v[j] = load_stream(src + j);
  };
  const int64_t e_first = sr0 * cols + (int64_t)sx * 64;
  RawBlock<DT> buf0, buf1;
  load_sub(0, e_first, buf0);
  TensorScale ts{};
  if constexpr (!MX) ts = workgroup_setup(p, tab);

  // One 64x64 sub-tile whose uniform element base is eq; prefetches sub-tile
  // q + AHEAD into `nxt` (PF: 1 = always, 0 = never, -1 = when q + 1 < nsub).
  auto sub_tile = [&](auto PF, auto AHEAD, int q, int64_t eq, const RawBlock<DT>& raw, RawBlock<DT>& nxt) {
    constexpr int ahead = decltype(AHEAD)::value;
    const int64_t r0 = sr0 + 64 * q + 16 * bi;  // first row of this lane's 16x16 block
    const bool valid = lane_valid(q);
    if constexpr (decltype(PF)::value == 1) {
      load_sub(q + ahead, eq + ahead * e_step, nxt);
    } else if constexpr (decltype(PF)::value == -1) {
      if (q + 1 < nsub) load_sub(q + 1, eq + e_step, nxt);
    }

    // ---- row pass: lane i holds row r0 + i, columns c0 .. c0 + 15 (element index eq + L ..)
    float y[16];
    uint32_t w[16];
    unpack_raw<DT>(raw, y);
    if constexpr (SR) {
      // Philox counters (idx / 4): a uniform part and the lane's L / 4; when no
      // lane's low counter word wraps (always, short of 2^34-element strides),
      // the high word is uniform and the low word a 32-bit add
      const uint64_t qu = (uint64_t)(eq + p.idx_base) >> 2;
      if ((uint64_t)(uint32_t)qu + (lmax >> 2) + 3u < (1ull << 32)) {
        sr_words16_hi_uniform((uint32_t)qu + (L >> 2), (uint32_t)(qu >> 32), key, w);
      } else {
        sr_words16((uint64_t)(eq + p.idx_base) + L, key, w);
      }
    }
    BlockResult res;
    if constexpr (MX) {
      // the 32-column block of columns c0 .. is shared with lane t ^ 16 (bj ^ 1)
      float m = absmax16(y);
      m = fmaxf(m, swizzle_xor16(m));
      res.sb = mx_scale_code(m);
      res.codes = mx_round16<SR>(y, res.sb, w);
    } else if constexpr (TWO_D) {
      res = quant_tile_row16<SR, RULE, true>(y, w, tab, ts.den6, ts.den4);
    } else {
      res = quant_block16<SR, RULE, true>(y, w, tab, ts.den6, ts.den4);
    }

    {
      // Row copy through buffer stores: a lane that stores nothing gets an offset
      // beyond the resource's range, which the hardware drops, so every lane (and
      // every path) issues the same stores and the waits for the prefetched
      // sub-tile count them exactly.  Resources cover this sub-tile's 64 rows.
      constexpr uint32_t kDrop = 0xFFFFFFF0u;
      const bool er = p.emit_row != 0;
      const int64_t srow = (sr0 + 64 * q) / 16;  // first 16-row block row of the sub-tile
      const __amdgpu_buffer_rsrc_t rc = raw_rsrc(er ? p.codes_row + (eq >> 1) : nullptr,
                                                 er ? (uint32_t)(64 * (cols / 2)) : 0u);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{res.codes.lo, res.codes.hi}, rc, valid ? (L >> 1) : kDrop, 0, 0);
      if constexpr (MX) {
        const __amdgpu_buffer_rsrc_t rs = raw_rsrc(er ? p.scales_row + (eq >> 5) : nullptr,
                                                   er ? (uint32_t)(64 * (cols / 32)) : 0u);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)res.sb, rs, (valid && (bj & 1) == 0) ? (L >> 5) : kDrop, 0, 0);
      } else if constexpr (TWO_D) {
        const __amdgpu_buffer_rsrc_t rs = raw_rsrc(er ? p.scales_row + srow * (cols / 16) + (int64_t)sx * 4 : nullptr,
                                                   er ? (uint32_t)(4 * (cols / 16)) : 0u);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)res.sb, rs,
                                             (valid && i == 0) ? (uint32_t)(bi * (cols / 16) + bj) : kDrop, 0, 0);
      } else {
        const __amdgpu_buffer_rsrc_t rs = raw_rsrc(er ? p.scales_row + (eq >> 4) : nullptr,
                                                   er ? (uint32_t)(64 * (cols / 16)) : 0u);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)res.sb, rs, valid ? (L >> 4) : kDrop, 0, 0);
      }
    }
    if (!p.emit_col) return;  // uniform across the workgroup

    // ---- 16x16 tiles: the column copy shares the tile's scale, reciprocal,
    // 4/6 choice and every element's word, so its codes are the row copy's,
    // transposed inside the tile (in registers, across the lanes of the DPP row)
    if constexpr (TWO_D) {
      const BlockCodes cc = transpose_tile16(res.codes, i);
      const int col = 16 * bj + i;
      *reinterpret_cast<uint2*>(col_codes + col * CP + 8 * q + 2 * bi) = make_uint2(cc.lo, cc.hi);
      if (i == 0) reinterpret_cast<uint8_t*>(col_scales)[bj * TR + 4 * q + bi] = (uint8_t)res.sb;
      return;
    }

    // ---- stage the sub-tile (and its random words) in LDS
    {
      const int row = 16 * bi + i;
      if constexpr (HALF) {
        uint4* dv = reinterpret_cast<uint4*>(lds_v + row * VP + 8 * bj);
        dv[0] = raw.v[0];
        dv[1] = raw.v[1];
      } else {
        float4* dv = reinterpret_cast<float4*>(lds_v + row * VP + 16 * bj);
#pragma unroll
        for (int j = 0; j < 4; ++j) dv[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
      }
      if constexpr (SR) {
        // 4-byte words, which the compiler pairs into two-address stores
        // (ds_write2_b32 takes its two words from any two registers; 16-byte
        // stores would first gather the scattered Philox results with moves)
        typedef __attribute__((address_space(3))) uint32_t lds_word;
        lds_word* dw = (lds_word*)(lds_w + row * WP + 16 * bj);
#pragma unroll
        for (int k = 0; k < 16; ++k) dw[k] = w[k];
      }
    }
    if constexpr (MX) {
      __syncthreads();
    } else {
      wave_lds_sync();  // the staged band is this wave's own
    }

    // ---- column pass: lane i holds column 16 * bj + i, rows r0 .. r0 + 15
    const int col = 16 * bj + i;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = 16 * bi + k;
      if constexpr (HALF) {
        y[k] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(lds_v)[row * 2 * VP + col] << 16);
      } else {
        y[k] = __uint_as_float(lds_v[row * VP + col]);
      }
      if constexpr (SR) w[k] = lds_w[row * WP + col];
    }
    float mcol = 0.0f;
    if constexpr (MX) {
      // a 32-row block spans waves 2h and 2h + 1: swap the column maxima through LDS
      mcol = absmax16(y);
      lds_m[bi * 64 + col] = mcol;
    }
    if constexpr (MX) {
      __syncthreads();  // the next sub-tile overwrites the staging area
    } else {
      wave_lds_sync();
    }
    BlockCodes cc;
    uint32_t sbc;
    if constexpr (MX) {
      sbc = mx_scale_code(fmaxf(mcol, lds_m[(bi ^ 1) * 64 + col]));
      cc = mx_round16<SR>(y, sbc, w);
    } else {
      const BlockResult rc = quant_block16<SR, RULE, true>(y, w, tab, ts.den6, ts.den4);
      cc = rc.codes;
      sbc = rc.sb;
    }
    // collect: column `col`, bytes 32q + 8bi .. of its 128-byte line; scale byte 4q + bi (MXFP4: 2q + bi/2)
    *reinterpret_cast<uint2*>(col_codes + col * CP + 8 * q + 2 * bi) = make_uint2(cc.lo, cc.hi);
    uint8_t* csb = reinterpret_cast<uint8_t*>(col_scales);
    if constexpr (MX) {
      if ((bi & 1) == 0) csb[col * SPC + 2 * q + (bi >> 1)] = (uint8_t)sbc;
    } else {
      csb[col * SPC + 4 * q + bi] = (uint8_t)sbc;
    }
  };

  using PF_ALWAYS = std::integral_constant<int, 1>;
  using PF_NEVER = std::integral_constant<int, 0>;
  using PF_IF = std::integral_constant<int, -1>;
  using NEXT = std::integral_constant<int, 1>;
  using SECOND = std::integral_constant<int, 2>;
  if (nsub == 4) {
    // a full strip: straight-line code, so that every wait for a prefetched
    // sub-tile counts exactly the memory operations issued after it
    if constexpr (!TWO_D) {
      // 1x16 and MXFP4 blocks: two sub-tiles in flight (measured 2% faster on
      // the 65536x8192 activation; the 16x16 tiles run better with one)
      RawBlock<DT> buf2;
      load_sub(1, e_first + e_step, buf1);
      sub_tile(PF_ALWAYS{}, SECOND{}, 0, e_first, buf0, buf2);
      sub_tile(PF_ALWAYS{}, SECOND{}, 1, e_first + e_step, buf1, buf0);
      sub_tile(PF_NEVER{}, SECOND{}, 2, e_first + 2 * e_step, buf2, buf1);
      sub_tile(PF_NEVER{}, SECOND{}, 3, e_first + 3 * e_step, buf0, buf1);
    } else {
      sub_tile(PF_ALWAYS{}, NEXT{}, 0, e_first, buf0, buf1);
      sub_tile(PF_ALWAYS{}, NEXT{}, 1, e_first + e_step, buf1, buf0);
      sub_tile(PF_ALWAYS{}, NEXT{}, 2, e_first + 2 * e_step, buf0, buf1);
      sub_tile(PF_NEVER{}, NEXT{}, 3, e_first + 3 * e_step, buf1, buf0);
    }
  } else {
    // Two sub-tiles per trip so that the prefetch buffers alternate without copies.
    int64_t eq = e_first;
    for (int q = 0; q < nsub; q += 2) {  // uniform trip count
      sub_tile(PF_IF{}, NEXT{}, q, eq, buf0, buf1);
      if (q + 1 < nsub) sub_tile(PF_IF{}, NEXT{}, q + 1, eq + e_step, buf1, buf0);
      eq += 2 * e_step;
    }
  }
  if (!p.emit_col) return;
  __syncthreads();

  // ---- write the strip's column copy: per column, rows_valid / 2 code bytes
  // and rows_valid / 16 (MXFP4: / 32) scale bytes, contiguous in the output
  const int rows_valid = (int)(rows_left < kStripRows ? rows_left : kStripRows);  // a multiple of 16
  const int cbytes = rows_valid / 2;
  const bool wide = ((rows / 2) & 15) == 0;  // every column's line starts 16-byte aligned
  constexpr int PARTS = kStripRows / 32;  // 16-byte parts of a column's codes
#pragma unroll
  for (int j = 0; j < 64 * PARTS / kThreads; ++j) {
    const int k = t + kThreads * j;
    const int colk = k / PARTS, part = k % PARTS;
    const int64_t c = (int64_t)sx * 64 + colk;
    if (c >= cols || 16 * part >= cbytes) continue;
    uint8_t* dst = p.codes_col + c * (rows / 2) + sr0 / 2 + 16 * part;
    const uint4 v = *reinterpret_cast<const uint4*>(col_codes + colk * CP + 4 * part);
    if (wide && 16 * part + 16 <= cbytes) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
      if (16 * part + 16 <= cbytes) *reinterpret_cast<uint2*>(dst + 8) = make_uint2(v.z, v.w);
    }
  }
  const uint8_t* cs = reinterpret_cast<const uint8_t*>(col_scales);
  if constexpr (TWO_D) {
    const int sbytes = rows_valid / 16;  // scale bytes per tile column
    for (int k = t; k < 4 * TR; k += kThreads) {
      const int tc = k / TR, j = k % TR;
      const int64_t ctile = (int64_t)sx * 4 + tc;
      if (ctile * 16 < cols && j < sbytes) p.scales_col[ctile * (rows / 16) + sr0 / 16 + j] = cs[tc * TR + j];
    }
  } else {
    constexpr int BR = MX ? 32 : 16;  // rows per column block
    const int sbytes = rows_valid / BR;
    // a full strip's SPC scale bytes of a column are contiguous in the output:
    // one SPC-byte store per column when that run is aligned, bytes otherwise
    const bool whole = sbytes == SPC && ((rows / BR) % SPC) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.scales_col) % SPC) == 0;
    if (whole) {
      if (t < 64) {
        const int64_t c = (int64_t)sx * 64 + t;
        uint8_t* dst = p.scales_col + c * (rows / BR) + sr0 / BR;
        if (c < cols) {
          if constexpr (SPC >= 16) {
#pragma unroll
            for (int u = 0; u < SPC / 16; ++u)
              reinterpret_cast<uint4*>(dst)[u] = reinterpret_cast<const uint4*>(cs + t * SPC)[u];
          } else {
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(cs + t * SPC);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 64 * SPC / kThreads; ++j) {
        const int k = t + kThreads * j;  // 64 columns x SPC bytes
        const int colk = k / SPC, b = k % SPC;
        const int64_t c = (int64_t)sx * 64 + colk;
        if (c < cols && b < sbytes) p.scales_col[c * (rows / BR) + sr0 / BR + b] = cs[colk * SPC + b];
      }
    }
  }
}

// Only the tensor scale (empty tensors).
__global__ void tensor_scale_kernel(const float* __restrict__ amax, float cap6, float* __restrict__ out) {
  if (threadIdx.x == 0) out[0] = __fdiv_rn(amax[0], cap6);
}

// -------------------------------------------------------- error analysis ---

// Per 16x16 region (16 lanes of a DPP row, one region row per lane): the
// round-to-nearest quantization exactly as the quantize kernels compute it
// (1x16 row blocks, optionally transformed, or one 16x16 tile), then per
// element its scaled value z = fl(y * e) picks a bin, and the bin accumulates
// the element count, eps^2 with eps = fl(y - fl(v * d)), and eps*^2 for the
// reference that maps the block max exactly onto the chosen T (binary64):
// v* = nearest-even E2M1 of T|y| / m, taken by comparing T|y| with the
// midpoints times m (exact products), xh* = fl64(v* * m / T).
constexpr int kMaxBins = 64;
// The workgroup's histogram is kept in 16 copies, lane i of every DPP row
// adding into copy i: lanes of one wave that hit the same bin then collide in
// groups of at most four instead of sixty-four (LDS atomics to one address
// serialize).  The copies are summed when the workgroup ends.
constexpr int kHistCopies = 16;

// The E2M1 grid values times m / T (binary64), as seven scalars passed by
// value so that the compiler keeps them in registers: a select between
// elements of an array (or of a struct behind a reference) becomes a load of
// the selected element from scratch memory.
struct ScaledGrid {
  double x1, x2, x3, x4, x5, x6, x7;
};

// Midpoints of the E2M1 grid (times m), ties to the even grid index: the first
// test that holds, in increasing order, picks the value (x7 when none does, as
// for a NaN).  Written as selects from the top down, so that no lane branches.
__device__ __forceinline__ double exact_scale_value(double ty, double m, ScaledGrid g) {
  double v = g.x7;
  v = ty <= 5.0 * m ? g.x6 : v;
  v = ty < 3.5 * m ? g.x5 : v;
  v = ty <= 2.5 * m ? g.x4 : v;
  v = ty < 1.75 * m ? g.x3 : v;
  v = ty <= 1.25 * m ? g.x2 : v;
  v = ty < 0.75 * m ? g.x1 : v;
  v = ty <= 0.25 * m ? 0.0 : v;
  return v;
}

template <int DT, bool RHT, bool TWO_D, int RULE>
__global__ __launch_bounds__(kThreads) void err_stats_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                             QuantParams p, float inv_w, int nbins,
                                                             double* __restrict__ stats) {
  __shared__ f32x2 tab[128];
  __shared__ double hist[3 * kMaxBins * kHistCopies];  // [quantity, bin][copy]
  for (int k = threadIdx.x; k < 3 * nbins * kHistCopies; k += kThreads) hist[k] = 0.0;
  const TensorScale ts = workgroup_setup(p, tab);  // ends with a barrier
  const int g = threadIdx.x >> 4, i = threadIdx.x & 15;
  double* const mine = hist + i;  // this lane's copy (stride kHistCopies)
  const int64_t rcols = cols / 16, nreg = (rows / 16) * rcols;
  for (int64_t reg0 = (int64_t)blockIdx.x * 16; reg0 < nreg; reg0 += (int64_t)gridDim.x * 16) {
    const int64_t reg = reg0 + g;
    const bool active = reg < nreg;  // whole 16-lane groups
    const int64_t rr = active ? reg / rcols : 0, cc = active ? reg - rr * rcols : 0;
    float y[16];
    load16<DT>(x, (rr * 16 + i) * cols + cc * 16, y);
    if constexpr (RHT) rht16(y, p.rht_mask);
    BlockResult res;
    float m = absmax16(y);
    if constexpr (TWO_D) {
      res = quant_tile_row16<false, RULE>(y, nullptr, tab, ts.den6, ts.den4);
      m = row16_max(m);
    } else {
      res = quant_block16<false, RULE>(y, nullptr, tab, ts.den6, ts.den4);
    }
    const float d = tab[res.sb].x;
    f32x2 v[8];
    v[0] = fp4_pair_values<0>(res.codes.lo);
    v[1] = fp4_pair_values<1>(res.codes.lo);
    v[2] = fp4_pair_values<2>(res.codes.lo);
    v[3] = fp4_pair_values<3>(res.codes.lo);
    v[4] = fp4_pair_values<0>(res.codes.hi);
    v[5] = fp4_pair_values<1>(res.codes.hi);
    v[6] = fp4_pair_values<2>(res.codes.hi);
    v[7] = fp4_pair_values<3>(res.codes.hi);
    const double T = res.four ? 4.0 : 6.0, md = (double)m;
    const ScaledGrid xs{(0.5 * md) / T, md / T, (1.5 * md) / T, (2.0 * md) / T,
                        (3.0 * md) / T, (4.0 * md) / T, (6.0 * md) / T};
    if (!active) continue;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float z = y[k] * res.e;
      int b = (int)(fabsf(z) * inv_w);  // exact: inv_w is a power of two
      b = b < nbins - 1 ? b : nbins - 1;
      const float vk = (k & 1) ? v[k >> 1].y : v[k >> 1].x;
      const float eps = y[k] - vk * d;
      const double yd = (double)y[k];
      const double xh = m != 0.0f ? exact_scale_value(T * fabs(yd), md, xs) : 0.0;
      const double es = yd - copysign(xh, yd);
      atomicAdd(&mine[kHistCopies * b], 1.0);
      atomicAdd(&mine[kHistCopies * (nbins + b)], (double)eps * (double)eps);
      atomicAdd(&mine[kHistCopies * (2 * nbins + b)], es * es);
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < 3 * nbins; k += kThreads) {
    double sum = 0.0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) sum += hist[kHistCopies * k + c];
    atomicAdd(&stats[k], sum);
  }
}

__global__ void zero_f64_kernel(double* __restrict__ p, int n) {
  for (int k = threadIdx.x; k < n; k += blockDim.x) p[k] = 0.0;
}

// ------------------------------------------------------------ dequantize ---

// Dequantize, row by row: each workgroup takes whole rows; per row, lane g
// turns 4 codes (2 bytes) into one 16-byte float4, so every wave store
// instruction writes 1 KB of contiguous output.
enum DequantFormat : int { kDqNv1D = 0, kDqNv2D = 1, kDqMx = 2 };

template <int FMT>
__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                const float* __restrict__ tsp, int64_t rows,
                                                                int64_t cols, float* __restrict__ out) {
  constexpr int BLK = FMT == kDqMx ? 32 : 16;  // elements per scale
  const float st = FMT == kDqMx ? 1.0f : tsp[0];
  const int64_t g4 = cols / 4;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* crow = reinterpret_cast<const uint16_t*>(codes + r * (cols / 2));
    const uint8_t* srow = scales + (FMT == kDqNv2D ? r / 16 : r) * (cols / BLK);
    float4* orow = reinterpret_cast<float4*>(out + r * cols);
#pragma unroll 4
    for (int64_t g = threadIdx.x; g < g4; g += kThreads) {
      const uint32_t c4 = crow[g];
      const uint32_t sb = srow[(4 * g) / BLK];
      float d;
      if constexpr (FMT == kDqMx) {  // 2^(sb - 127); E8M0 code 255 is NaN
        d = sb == 0u ? __uint_as_float(0x00400000u) : (sb == 255u ? __uint_as_float(0x7FC00000u) : __uint_as_float(sb << 23));
      } else {
        d = e4m3_decode(sb) * st;
      }
      const f32x2 v0 = fp4_pair_values<0>(c4), v1 = fp4_pair_values<1>(c4);
      orow[g] = make_float4(v0.x * d, v0.y * d, v1.x * d, v1.y * d);
    }
  }
}


// ------------------------------------------------------------- dispatch ---

template <typename F>
static void with_bool(bool b, F&& f) {
  if (b) f(std::true_type{});
  else f(std::false_type{});
}
template <typename F>
static void with_dtype(int dt, F&& f) {
  if (dt == kBF16) f(std::integral_constant<int, kBF16>{});
  else f(std::integral_constant<int, kF32>{});
}
template <typename F>
static void with_rule(int rule, F&& f) {
  switch (rule) {
    case kRuleNone: f(std::integral_constant<int, kRuleNone>{}); break;
    case kRuleMse: f(std::integral_constant<int, kRuleMse>{}); break;
    case kRuleMae: f(std::integral_constant<int, kRuleMae>{}); break;
    default: f(std::integral_constant<int, kRuleMaxErr>{}); break;
  }
}

constexpr int kRowU = 1;
constexpr int64_t kDequantMaxGrid = 4096;  // workgroups of the row-wise dequantize (grid-stride over rows)
constexpr int kAmaxMaxParts = 1024;

// Resident workgroups of a kernel on the current device (persistent grids).
template <typename K>
static int64_t resident_grid(K kernel, size_t dyn_lds = 0) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), kThreads,
                                                    dyn_lds) != hipSuccess ||
      per_cu <= 0)
    per_cu = 4;
  return (int64_t)cus * per_cu;
}

}  // namespace nvfp4

using namespace nvfp4;

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- the amax pass without a caller workspace ---------------------------------
// For callers that cannot allocate device memory (graph capture, serving loops):
// the pass's per-workgroup partial maxima go to this file-scope array instead of
// a workspace.  Each GPU the library runs on holds its own copy (4 KB) until the
// process ends.  In host code `scratch` only names the symbol: its device
// address, different on every GPU, comes from hipGetSymbolAddress with that GPU
// current, once per device, and only that address is passed to kernels.  Every
// call on one GPU uses the same array, so calls that overlap on one GPU (on
// different streams, or from different threads) race; the partial kernel
// overwrites every entry the finish kernel reads, so nothing needs clearing.
constexpr int kScratchFloats = kAmaxMaxParts;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static float* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the GPU that runs `s` (the current device
// for the null stream).
static nvfp4_status scratch_for_stream(hipStream_t s, float** out) {
  int dev = 0;
  if (s) {
    if (hipStreamGetDevice(s, &dev) != hipSuccess) return NVFP4_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return NVFP4_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return NVFP4_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return NVFP4_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return NVFP4_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

// The value a C caller passed for an enum-typed parameter, read from its bytes:
// a value outside the enumerators is legal in C but may not be loaded as the
// C++ enum type, and validation must see it to reject it.
template <typename E>
static int enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

// Shapes whose element count (and byte count of a binary32 copy) fits in int64.
constexpr int64_t kMaxElements = 1ll << 60;
static bool dims_ok(int64_t rows, int64_t cols) {
  return rows >= 0 && cols >= 0 && (cols == 0 || rows <= kMaxElements / cols);
}

// Element indices (row_offset + r) * cols + c of the random stream stay below 2^62.
static bool row_offset_ok(int64_t row_offset, int64_t rows, int64_t cols) {
  return row_offset >= 0 && (cols == 0 || row_offset <= (1ll << 62) / cols - rows);
}

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(nvfp4_status s) {
  switch (enum_bits(s)) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (dims must be >= 0 and multiples of 16 where blocks need it)";
    case NVFP4_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case NVFP4_ERR_DTYPE: return "unknown input dtype";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported option or option combination";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

uint16_t nvfp4_rht_signs_from_seed(uint64_t seed) {
  // host evaluation of Philox-4x32-10 at counter (0, 0, 0, 1)
  uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 1, k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return (uint16_t)(c0 & 0xFFFFu);
}

static int amax_parts(int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  int64_t parts = (n + (int64_t)kThreads * 32 - 1) / ((int64_t)kThreads * 32);
  if (parts < 1) parts = 1;
  if (parts > kAmaxMaxParts) parts = kAmaxMaxParts;
  return (int)parts;
}

size_t nvfp4_amax_workspace_bytes(int64_t rows, int64_t cols) {
  if (!dims_ok(rows, cols)) return 0;
  return sizeof(float) * (size_t)amax_parts(rows, cols);
}

// Argument checks shared by both amax entry points.
static nvfp4_status amax_args(const void* x, int dtype, int64_t rows, int64_t cols, bool rht, const float* amax_dev) {
  if (!dims_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (dtype != NVFP4_IN_BF16 && dtype != NVFP4_IN_F32) return NVFP4_ERR_DTYPE;
  if (rht && cols % 16) return NVFP4_ERR_SHAPE;
  if (!amax_dev) return NVFP4_ERR_NULL;
  const int64_t n = rows * cols;
  if (n > 0 && !x) return NVFP4_ERR_NULL;
  if (n > 0 && !aligned16(x)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// The two amax kernels: partial maxima of `parts` workgroups into `partials`,
// then their maximum into amax_dev.
static nvfp4_status launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, bool rht, uint32_t mask,
                                float* amax_dev, float* partials, int parts, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n > 0) {
    with_dtype(dtype, [&](auto DT) {
      with_bool(rht, [&](auto RHT) {
        hipLaunchKernelGGL((amax_partial_kernel<DT(), RHT()>), dim3(parts), dim3(kThreads), 0, s, x, n, mask,
                           partials);
      });
    });
    hipLaunchKernelGGL(amax_finish_kernel, dim3(1), dim3(kThreads), 0, s, partials, parts, amax_dev);
  } else {
    hipLaunchKernelGGL(amax_finish_kernel, dim3(1), dim3(kThreads), 0, s, partials, 0, amax_dev);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype dtype_arg, int64_t rows, int64_t cols, const nvfp4_config* cfg,
                        float* amax_dev, void* workspace, size_t workspace_bytes, void* stream) {
  const int dtype = enum_bits(dtype_arg);
  const bool rht = cfg && cfg->rht;
  const nvfp4_status st = amax_args(x, dtype, rows, cols, rht, amax_dev);
  if (st != NVFP4_OK) return st;
  const int parts = amax_parts(rows, cols);
  if (!workspace || workspace_bytes < sizeof(float) * (size_t)parts) return NVFP4_ERR_WORKSPACE;
  return launch_amax(x, dtype, rows, cols, rht, rht ? cfg->rht_sign_mask : 0u, amax_dev,
                     reinterpret_cast<float*>(workspace), parts, reinterpret_cast<hipStream_t>(stream));
}

nvfp4_status nvfp4_amax_noalloc(const void* x, nvfp4_dtype dtype_arg, int64_t rows, int64_t cols,
                                const nvfp4_config* cfg, float* amax_dev, void* stream) {
  const int dtype = enum_bits(dtype_arg);
  const bool rht = cfg && cfg->rht;
  const nvfp4_status st = amax_args(x, dtype, rows, cols, rht, amax_dev);
  if (st != NVFP4_OK) return st;
  const int parts = amax_parts(rows, cols);
  if (parts > kScratchFloats) return NVFP4_ERR_WORKSPACE;  // never for the capped partial count
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* partials = nullptr;
  const nvfp4_status sp = scratch_for_stream(s, &partials);
  if (sp != NVFP4_OK) return sp;
  return launch_amax(x, dtype, rows, cols, rht, rht ? cfg->rht_sign_mask : 0u, amax_dev, partials, parts, s);
}

nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype dtype_arg, int64_t rows, int64_t cols, const nvfp4_config* cfg,
                            const float* amax_dev, const nvfp4_outputs* out, void* stream) {
  if (!cfg || !out || !amax_dev) return NVFP4_ERR_NULL;
  const int dtype = enum_bits(dtype_arg);
  if (dtype != NVFP4_IN_BF16 && dtype != NVFP4_IN_F32) return NVFP4_ERR_DTYPE;
  if (cfg->block != NVFP4_BLOCK_1D && cfg->block != NVFP4_BLOCK_2D) return NVFP4_ERR_UNSUPPORTED;
  if (cfg->rule < NVFP4_RULE_NONE || cfg->rule > NVFP4_RULE_MAXERR) return NVFP4_ERR_UNSUPPORTED;
  if (cfg->scale_cap != 448.0f && cfg->scale_cap != 256.0f) return NVFP4_ERR_UNSUPPORTED;
  const bool two_d = cfg->block == NVFP4_BLOCK_2D;
  const bool erow = cfg->emit_rowwise != 0, ecol = cfg->emit_colwise != 0;
  if (!erow && !ecol) return NVFP4_ERR_UNSUPPORTED;
  if (cfg->rht && (two_d || ecol)) return NVFP4_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (cols % 16) return NVFP4_ERR_SHAPE;
  if (!row_offset_ok(cfg->row_offset, rows, cols)) return NVFP4_ERR_SHAPE;
  if ((two_d || ecol) && rows % 16) return NVFP4_ERR_SHAPE;
  if ((two_d || ecol) && cols > kStripMaxCols) return NVFP4_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n > 0) {
    if (!x) return NVFP4_ERR_NULL;
    if (erow && (!out->codes_row || !out->scales_row)) return NVFP4_ERR_NULL;
    if (ecol && (!out->codes_col || !out->scales_col)) return NVFP4_ERR_NULL;
    if (!aligned16(x)) return NVFP4_ERR_ALIGN;
    if (erow && !aligned16(out->codes_row)) return NVFP4_ERR_ALIGN;
    if (ecol && !aligned16(out->codes_col)) return NVFP4_ERR_ALIGN;
  }

  QuantParams p;
  p.amax = amax_dev;
  p.cap6 = 6.0f * cfg->scale_cap;
  p.rht_mask = cfg->rht ? (uint32_t)cfg->rht_sign_mask : 0u;
  p.k0 = (uint32_t)cfg->sr_seed;
  p.k1 = (uint32_t)(cfg->sr_seed >> 32);
  p.row_offset = cfg->row_offset;
  p.idx_base = cfg->row_offset * cols;
  p.idx_below_2_34 = p.idx_base + rows * cols <= (1ll << 34);
  p.emit_row = erow;
  p.emit_col = ecol;
  p.codes_row = out->codes_row;
  p.scales_row = out->scales_row;
  p.codes_col = out->codes_col;
  p.scales_col = out->scales_col;
  p.tensor_scale = out->tensor_scale;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  if (n == 0) {
    if (p.tensor_scale) hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(64), 0, s, amax_dev, p.cap6, p.tensor_scale);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
  }

  if (!two_d && !ecol) {
    const int64_t nblocks = n / 16;
    const int64_t per_wg = (int64_t)kThreads * kRowU;
    const int64_t nchunks = (nblocks + per_wg - 1) / per_wg;
    with_dtype(dtype, [&](auto DT) {
      with_bool(cfg->rht != 0, [&](auto RHT) {
        with_bool(cfg->sr != 0, [&](auto SR) {
          with_rule(cfg->rule, [&](auto RULE) {
            auto k = quant_row_kernel<DT(), RHT(), SR(), RULE(), kRowU, false>;
            // With stochastic rounding a chunk's arithmetic (a Philox word per
            // element) is long enough for the other resident waves to hide a new
            // workgroup's first load, and one workgroup per chunk lets the
            // dispatcher balance the chunks over the CUs (a persistent grid gives
            // some workgroups one chunk more than others).  Lighter chunks keep
            // the persistent grid, whose prefetch hides the load latency.
            // (the grid size is a 32-bit count: beyond 2^30 chunks, persistent)
            int64_t grid = SR() && nchunks <= (1ll << 30) ? nchunks : resident_grid(k);
            if (grid > nchunks) grid = nchunks;
            hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, p);
          });
        });
      });
    });
  } else {
    const int64_t strips_x = (cols + 63) / 64, strips_y = (rows + kStripRows - 1) / kStripRows;
    const int64_t nstrips = strips_x * strips_y;
    if (nstrips > (1ll << 24)) return NVFP4_ERR_SHAPE;  // the dispatch counts work-items in 32 bits
    with_dtype(dtype, [&](auto DT) {
      with_bool(two_d, [&](auto TWO_D) {
        with_bool(cfg->sr != 0, [&](auto SR) {
          with_rule(cfg->rule, [&](auto RULE) {
            constexpr int FMT = TWO_D() ? kFmt2D : kFmt1D;
            hipLaunchKernelGGL((quant_strip_kernel<DT(), FMT, SR(), RULE()>), dim3((unsigned)nstrips),
                               dim3(kThreads), 0, s, x, rows, cols, (uint32_t)strips_x, p);
          });
        });
      });
    });
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t rows,
                              int64_t cols, nvfp4_block block_arg, float* out, void* stream) {
  const int block = enum_bits(block_arg);
  if (block != NVFP4_BLOCK_1D && block != NVFP4_BLOCK_2D) return NVFP4_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols) || cols % 16) return NVFP4_ERR_SHAPE;
  if (block == NVFP4_BLOCK_2D && rows % 16) return NVFP4_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n == 0) return NVFP4_OK;
  if (!codes || !scales || !tensor_scale || !out) return NVFP4_ERR_NULL;
  if (!aligned16(codes) || !aligned16(out)) return NVFP4_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)(rows < kDequantMaxGrid ? rows : kDequantMaxGrid);
  if (block == NVFP4_BLOCK_2D)
    hipLaunchKernelGGL(dequant_rows_kernel<kDqNv2D>, dim3(grid), dim3(kThreads), 0, s, codes, scales, tensor_scale,
                       rows, cols, out);
  else
    hipLaunchKernelGGL(dequant_rows_kernel<kDqNv1D>, dim3(grid), dim3(kThreads), 0, s, codes, scales, tensor_scale,
                       rows, cols, out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_mxfp4_quantize(const void* x, nvfp4_dtype dtype_arg, int64_t rows, int64_t cols,
                                  const nvfp4_mx_config* cfg, const nvfp4_mx_outputs* out, void* stream) {
  if (!cfg || !out) return NVFP4_ERR_NULL;
  const int dtype = enum_bits(dtype_arg);
  if (dtype != NVFP4_IN_BF16 && dtype != NVFP4_IN_F32) return NVFP4_ERR_DTYPE;
  const bool erow = cfg->emit_rowwise != 0, ecol = cfg->emit_colwise != 0;
  if (!erow && !ecol) return NVFP4_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols) || cols % 32) return NVFP4_ERR_SHAPE;
  if (!row_offset_ok(cfg->row_offset, rows, cols)) return NVFP4_ERR_SHAPE;
  if (ecol && rows % 32) return NVFP4_ERR_SHAPE;
  if (ecol && cols > kStripMaxCols) return NVFP4_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n == 0) return NVFP4_OK;
  if (!x) return NVFP4_ERR_NULL;
  if (erow && (!out->codes_row || !out->scales_row)) return NVFP4_ERR_NULL;
  if (ecol && (!out->codes_col || !out->scales_col)) return NVFP4_ERR_NULL;
  if (!aligned16(x)) return NVFP4_ERR_ALIGN;
  if (erow && !aligned16(out->codes_row)) return NVFP4_ERR_ALIGN;
  if (ecol && !aligned16(out->codes_col)) return NVFP4_ERR_ALIGN;

  QuantParams p{};
  p.k0 = (uint32_t)cfg->sr_seed;
  p.k1 = (uint32_t)(cfg->sr_seed >> 32);
  p.row_offset = cfg->row_offset;
  p.idx_base = cfg->row_offset * cols;
  p.idx_below_2_34 = p.idx_base + rows * cols <= (1ll << 34);
  p.emit_row = erow;
  p.emit_col = ecol;
  p.codes_row = out->codes_row;
  p.scales_row = out->scales_row;
  p.codes_col = out->codes_col;
  p.scales_col = out->scales_col;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!ecol) {
    const int64_t nblocks = n / 16;
    const int64_t per_wg = (int64_t)kThreads * kRowU;
    const int64_t nchunks = (nblocks + per_wg - 1) / per_wg;
    with_dtype(dtype, [&](auto DT) {
      with_bool(cfg->sr != 0, [&](auto SR) {
        auto k = quant_row_kernel<DT(), false, SR(), kRuleNone, kRowU, true>;
        int64_t grid = resident_grid(k);
        if (grid > nchunks) grid = nchunks;
        hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), 0, s, x, nblocks, p);
      });
    });
  } else {
    const int64_t strips_x = (cols + 63) / 64, strips_y = (rows + kStripRows - 1) / kStripRows;
    const int64_t nstrips = strips_x * strips_y;
    if (nstrips > (1ll << 24)) return NVFP4_ERR_SHAPE;
    with_dtype(dtype, [&](auto DT) {
      with_bool(cfg->sr != 0, [&](auto SR) {
        hipLaunchKernelGGL((quant_strip_kernel<DT(), kFmtMX, SR(), kRuleNone>), dim3((unsigned)nstrips),
                           dim3(kThreads), 0, s, x, rows, cols, (uint32_t)strips_x, p);
      });
    });
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                    float* out, void* stream) {
  if (!dims_ok(rows, cols) || cols % 32) return NVFP4_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n == 0) return NVFP4_OK;
  if (!codes || !scales || !out) return NVFP4_ERR_NULL;
  if (!aligned16(codes) || !aligned16(out)) return NVFP4_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)(rows < kDequantMaxGrid ? rows : kDequantMaxGrid);
  hipLaunchKernelGGL(dequant_rows_kernel<kDqMx>, dim3(grid), dim3(kThreads), 0, s, codes, scales, nullptr, rows,
                     cols, out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_error_stats(const void* x, nvfp4_dtype dtype_arg, int64_t rows, int64_t cols, const nvfp4_config* cfg,
                               const float* amax_dev, float bin_width, int32_t nbins, double* stats_dev,
                               void* stream) {
  if (!cfg || !amax_dev || !stats_dev) return NVFP4_ERR_NULL;
  const int dtype = enum_bits(dtype_arg);
  if (dtype != NVFP4_IN_BF16 && dtype != NVFP4_IN_F32) return NVFP4_ERR_DTYPE;
  if (cfg->block != NVFP4_BLOCK_1D && cfg->block != NVFP4_BLOCK_2D) return NVFP4_ERR_UNSUPPORTED;
  if (cfg->rule < NVFP4_RULE_NONE || cfg->rule > NVFP4_RULE_MAXERR) return NVFP4_ERR_UNSUPPORTED;
  if (cfg->scale_cap != 448.0f && cfg->scale_cap != 256.0f) return NVFP4_ERR_UNSUPPORTED;
  const bool two_d = cfg->block == NVFP4_BLOCK_2D;
  if (cfg->sr || (cfg->rht && two_d)) return NVFP4_ERR_UNSUPPORTED;
  if (nbins < 1 || nbins > kMaxBins) return NVFP4_ERR_UNSUPPORTED;
  int ex = 0;
  if (!(bin_width > 0.0f) || frexpf(bin_width, &ex) != 0.5f || ex < -100 || ex > 100) return NVFP4_ERR_UNSUPPORTED;
  if (!dims_ok(rows, cols) || rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
  const int64_t n = rows * cols;
  if (n > 0 && !x) return NVFP4_ERR_NULL;
  if (n > 0 && !aligned16(x)) return NVFP4_ERR_ALIGN;
  QuantParams p{};
  p.amax = amax_dev;
  p.cap6 = 6.0f * cfg->scale_cap;
  p.rht_mask = cfg->rht ? (uint32_t)cfg->rht_sign_mask : 0u;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_f64_kernel, dim3(1), dim3(kThreads), 0, s, stats_dev, 3 * nbins);
  const int64_t nreg = (rows / 16) * (cols / 16);
  if (nreg > 0) {
    const float inv_w = 1.0f / bin_width;  // exact: a power of two
    const int64_t groups = (nreg + 15) / 16;
    with_dtype(dtype, [&](auto DT) {
      with_bool(cfg->rht != 0, [&](auto RHT) {
        with_bool(two_d, [&](auto TWO_D) {
          with_rule(cfg->rule, [&](auto RULE) {
            if constexpr (!(RHT() && TWO_D())) {
              auto k = err_stats_kernel<DT(), RHT(), TWO_D(), RULE()>;
              int64_t grid = resident_grid(k);
              if (grid > groups) grid = groups;
              hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), 0, s, x, rows, cols, p, inv_w, nbins,
                                 stats_dev);
            }
          });
        });
      });
    });
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
