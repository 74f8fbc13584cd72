// gemm.hip -- the consumer of the quantized copies: C = A B^T on FP4 operands
// with gfx950 matrix cores.
//
// Both operands are row copies with K contiguous ("NT"): A codes [M][K/2],
// B codes [N][K/2], two E2M1 codes per byte (even element in the low nibble).
//
//   MXFP4 x MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4.
//     The instruction applies one E8M0 scale per lane, i.e. per row and 32
//     consecutive K values, which is exactly the MXFP4 block.
//   NVFP4 x NVFP4: the instruction's scale is a power of two per 32 values, so
//     it cannot carry 16-element E4M3 scales.  Every element v * dec(sb) is
//     exact in fp16 (at most 6 significant bits, magnitudes 2^-10 .. 2688), so
//     the operands are expanded in registers to fp16 and multiplied with
//     v_mfma_f32_32x32x16_f16; the two tensor scales multiply the fp32 result.
//
// Lane layout of the 32x32 instructions (established on the device): lane l
// supplies row l % 32 of A (and of B) for K values [32 (l / 32), +32) of a
// 64-wide FP4 step, or [8 (l / 32), +8) of a 16-wide fp16 step; result register
// r of lane l is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  Any consistent
// assignment of K values to the two lane halves gives the same sum, so each
// half here walks its own contiguous K range and loads whole 16-byte pieces.
//
// Tiling: a workgroup of 4 waves owns a 128x128 tile of C, each wave a 64x64
// quarter (2x2 instruction tiles); operand fragments come straight from
// global memory (each 16-byte piece feeds two instructions of the wave and the
// neighbouring waves hit it in L2), with the next K step's fragments loaded
// while the current step's instructions run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace fp4gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTile = 128;  // workgroup tile of C (M and N)

// Dispatch order: consecutive workgroups go round-robin over the 8 XCDs; give
// each XCD one contiguous range of tiles (N fastest), so the tiles that share
// A rows run on the same XCD and meet in its L2.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t nb) {
  const uint32_t q = nb >> 3, rem = nb & 7;
  const uint32_t xcd = bid & 7, slot = bid >> 3;
  return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

__device__ __forceinline__ void store_tile(float* __restrict__ C, int64_t M, int64_t N, int64_t r0, int64_t c0,
                                           const v16f& acc, int l, float scale_unused) {
  const int64_t col = c0 + (l & 31);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = r0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    if (row < M) C[row * N + col] = acc[r];
  }
}

// ------------------------------------------------------------------ MXFP4 ---

struct MxFrag {
  uint4 q[4];   // 4 x 32 FP4 values: K [kb + 32 c, +32) for c = 0..3
  uint32_t s;   // their 4 E8M0 scales, byte c for chunk c
};

__device__ __forceinline__ void mx_load(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                        int64_t row, int64_t K, int64_t kb, MxFrag& f) {
  const uint8_t* p = codes + row * (K / 2) + kb / 2;
  const uint8_t* ps = scales + row * (K / 32) + kb / 32;
  if (kb + 128 <= K) {
#pragma unroll
    for (int c = 0; c < 4; ++c) f.q[c] = reinterpret_cast<const uint4*>(p)[c];
    f.s = *reinterpret_cast<const uint32_t*>(ps);  // kb is a multiple of 128: 4-byte aligned
  } else {  // K tail: missing 32-value chunks are zero (scale 2^0)
    f.s = 0x7F7F7F7Fu;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (kb + 32 * c < K) {
        f.q[c] = reinterpret_cast<const uint4*>(p)[c];
        f.s = (f.s & ~(0xFFu << (8 * c))) | ((uint32_t)ps[c] << (8 * c));
      } else {
        f.q[c] = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <int C>
__device__ __forceinline__ v16f mx_mfma(const MxFrag& a, const MxFrag& b, v16f acc) {
  const v8i va = {(int)a.q[C].x, (int)a.q[C].y, (int)a.q[C].z, (int)a.q[C].w, 0, 0, 0, 0};
  const v8i vb = {(int)b.q[C].x, (int)b.q[C].y, (int)b.q[C].z, (int)b.q[C].w, 0, 0, 0, 0};
  // formats 4/4: E2M1 x E2M1; scale byte C of each lane's scale word
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, C, (int)a.s, C, (int)b.s);
}

__global__ __launch_bounds__(kThreads) void mx_gemm_kernel(const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ As,
                                                           const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ Bs, int64_t M, int64_t N,
                                                           int64_t K, float* __restrict__ C, uint32_t tiles_n) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5;
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const uint32_t tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * kTile + 64 * (wave >> 1), n0 = (int64_t)tn * kTile + 64 * (wave & 1);
  int64_t ra[2], rb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = m0 + 32 * i + (l & 31), s = n0 + 32 * i + (l & 31);
    ra[i] = r < M ? r : M - 1;  // rows past the edge load a valid row; their results are not stored
    rb[i] = s < N ? s : N - 1;
  }
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  MxFrag fa[2][2], fb[2][2];  // [buffer][tile]
  auto load = [&](int buf, int64_t k0) {
    const int64_t kb = k0 + 128 * h;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      mx_load(A, As, ra[i], K, kb, fa[buf][i]);
      mx_load(B, Bs, rb[i], K, kb, fb[buf][i]);
    }
  };
  auto step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mx_mfma<0>(fa[buf][i], fb[buf][j], acc[i][j]);
        acc[i][j] = mx_mfma<1>(fa[buf][i], fb[buf][j], acc[i][j]);
        acc[i][j] = mx_mfma<2>(fa[buf][i], fb[buf][j], acc[i][j]);
        acc[i][j] = mx_mfma<3>(fa[buf][i], fb[buf][j], acc[i][j]);
      }
  };
  load(0, 0);
  for (int64_t k0 = 0; k0 < K; k0 += 512) {
    if (k0 + 256 < K) load(1, k0 + 256);
    step(0);
    if (k0 + 256 >= K) break;
    if (k0 + 512 < K) load(0, k0 + 512);
    step(1);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) store_tile(C, M, N, m0 + 32 * i, n0 + 32 * j, acc[i][j], l, 1.0f);
}

// ------------------------------------------------------------------ NVFP4 ---

struct NvFrag {
  uint4 q[2];  // 64 FP4 values: K [kb, kb + 64)
  uint32_t s;  // E4M3 scales of the four 16-value blocks
};

__device__ __forceinline__ void nv_load(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                        int64_t row, int64_t srow, int64_t K, int64_t kb, NvFrag& f) {
  const uint8_t* p = codes + row * (K / 2) + kb / 2;
  const uint8_t* ps = scales + srow * (K / 16) + kb / 16;
  if (kb + 64 <= K) {
    f.q[0] = reinterpret_cast<const uint4*>(p)[0];
    f.q[1] = reinterpret_cast<const uint4*>(p)[1];
    f.s = *reinterpret_cast<const uint32_t*>(ps);  // kb is a multiple of 64: 4-byte aligned
  } else {  // K tail in 16-value blocks: missing blocks are zero
    uint32_t w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w[c] = kb + 8 * c < K ? reinterpret_cast<const uint32_t*>(p)[c] : 0u;
    f.q[0] = make_uint4(w[0], w[1], w[2], w[3]);
    f.q[1] = make_uint4(w[4], w[5], w[6], w[7]);
    f.s = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (kb + 16 * c < K) f.s |= (uint32_t)ps[c] << (8 * c);
  }
}

// fp16 operand for K values [kb + 8 c, +8): codes word c, scale of block c / 2.
template <int C>
__device__ __forceinline__ v8h nv_half8(const NvFrag& f, const h2 sc2[4]) {
  const uint32_t w = C < 4 ? (C == 0 ? f.q[0].x : C == 1 ? f.q[0].y : C == 2 ? f.q[0].z : f.q[0].w)
                           : (C == 4 ? f.q[1].x : C == 5 ? f.q[1].y : C == 6 ? f.q[1].z : f.q[1].w);
  const h2 s = sc2[C >> 1];
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// The four E4M3 block scales as fp16 pairs (exact: E4M3 lies inside fp16).
__device__ __forceinline__ void nv_scales(uint32_t s, h2 out[4]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(s, false);  // bytes 0, 1
  const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(s, true);   // bytes 2, 3
  const _Float16 v0 = (_Float16)lo.x, v1 = (_Float16)lo.y, v2 = (_Float16)hi.x, v3 = (_Float16)hi.y;
  out[0] = h2{v0, v0};
  out[1] = h2{v1, v1};
  out[2] = h2{v2, v2};
  out[3] = h2{v3, v3};
}

template <int C>
__device__ __forceinline__ v16f nv_mfma(const NvFrag& a, const h2 sa[4], const NvFrag& b, const h2 sb[4], v16f acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(nv_half8<C>(a, sa), nv_half8<C>(b, sb), acc, 0, 0, 0);
}

template <bool A2D, bool B2D>
__global__ __launch_bounds__(kThreads) void nv_gemm_kernel(const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ As,
                                                           const float* __restrict__ ats,
                                                           const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ Bs,
                                                           const float* __restrict__ bts, int64_t M, int64_t N,
                                                           int64_t K, float* __restrict__ C, uint32_t tiles_n) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5;
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const uint32_t tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * kTile + 64 * (wave >> 1), n0 = (int64_t)tn * kTile + 64 * (wave & 1);
  int64_t ra[2], rb[2], sa_row[2], sb_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t r = m0 + 32 * i + (l & 31), s = n0 + 32 * i + (l & 31);
    ra[i] = r < M ? r : M - 1;
    rb[i] = s < N ? s : N - 1;
    sa_row[i] = A2D ? ra[i] / 16 : ra[i];
    sb_row[i] = B2D ? rb[i] / 16 : rb[i];
  }
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  NvFrag fa[2][2], fb[2][2];
  auto load = [&](int buf, int64_t k0) {
    const int64_t kb = k0 + 64 * h;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      nv_load(A, As, ra[i], sa_row[i], K, kb, fa[buf][i]);
      nv_load(B, Bs, rb[i], sb_row[i], K, kb, fb[buf][i]);
    }
  };
  auto step = [&](int buf) {
    h2 sca[2][4], scb[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      nv_scales(fa[buf][i].s, sca[i]);
      nv_scales(fb[buf][i].s, scb[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = nv_mfma<0>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<1>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<2>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<3>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<4>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<5>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<6>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
        acc[i][j] = nv_mfma<7>(fa[buf][i], sca[i], fb[buf][j], scb[j], acc[i][j]);
      }
  };
  load(0, 0);
  for (int64_t k0 = 0; k0 < K; k0 += 256) {
    if (k0 + 128 < K) load(1, k0 + 128);
    step(0);
    if (k0 + 128 >= K) break;
    if (k0 + 256 < K) load(0, k0 + 256);
    step(1);
  }
  // the two tensor scales, applied once: fl32(acc * S_tA * S_tB) with the product taken in binary64
  const double ts = (double)ats[0] * (double)bts[0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v16f t;
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = (float)((double)acc[i][j][r] * ts);
      store_tile(C, M, N, m0 + 32 * i, n0 + 32 * j, t, l, 1.0f);
    }
}

}  // namespace fp4gemm

using namespace fp4gemm;

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

extern "C" {

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                        nvfp4_block a_block, const uint8_t* b_codes, const uint8_t* b_scales,
                        const float* b_tensor_scale, nvfp4_block b_block, int64_t M, int64_t N, int64_t K, float* c,
                        void* stream) {
  if ((a_block != NVFP4_BLOCK_1D && a_block != NVFP4_BLOCK_2D) ||
      (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D))
    return NVFP4_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || K % 64) return NVFP4_ERR_SHAPE;
  if ((a_block == NVFP4_BLOCK_2D && M % 16) || (b_block == NVFP4_BLOCK_2D && N % 16)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c) return NVFP4_ERR_NULL;
  if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales || !a_tensor_scale || !b_tensor_scale))
    return NVFP4_ERR_NULL;
  if (!al16(a_codes) || !al16(b_codes) || !al4(a_scales) || !al4(b_scales) || !al4(c)) return NVFP4_ERR_ALIGN;
  const int64_t tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  if (tiles_m * tiles_n > (1ll << 24)) return NVFP4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (K == 0) {
    hipMemsetAsync(c, 0, sizeof(float) * (size_t)(M * N), s);
  } else if (a_block == NVFP4_BLOCK_2D) {
    if (b_block == NVFP4_BLOCK_2D)
      hipLaunchKernelGGL((nv_gemm_kernel<true, true>), grid, dim3(kThreads), 0, s, a_codes, a_scales, a_tensor_scale,
                         b_codes, b_scales, b_tensor_scale, M, N, K, c, (uint32_t)tiles_n);
    else
      hipLaunchKernelGGL((nv_gemm_kernel<true, false>), grid, dim3(kThreads), 0, s, a_codes, a_scales, a_tensor_scale,
                         b_codes, b_scales, b_tensor_scale, M, N, K, c, (uint32_t)tiles_n);
  } else {
    if (b_block == NVFP4_BLOCK_2D)
      hipLaunchKernelGGL((nv_gemm_kernel<false, true>), grid, dim3(kThreads), 0, s, a_codes, a_scales, a_tensor_scale,
                         b_codes, b_scales, b_tensor_scale, M, N, K, c, (uint32_t)tiles_n);
    else
      hipLaunchKernelGGL((nv_gemm_kernel<false, false>), grid, dim3(kThreads), 0, s, a_codes, a_scales,
                         a_tensor_scale, b_codes, b_scales, b_tensor_scale, M, N, K, c, (uint32_t)tiles_n);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* c, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 128) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c) return NVFP4_ERR_NULL;
  if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return NVFP4_ERR_NULL;
  if (!al16(a_codes) || !al16(b_codes) || !al4(a_scales) || !al4(b_scales) || !al4(c)) return NVFP4_ERR_ALIGN;
  const int64_t tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  if (tiles_m * tiles_n > (1ll << 24)) return NVFP4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) {
    hipMemsetAsync(c, 0, sizeof(float) * (size_t)(M * N), s);
  } else {
    hipLaunchKernelGGL(mx_gemm_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kThreads), 0, s, a_codes, a_scales,
                       b_codes, b_scales, M, N, K, c, (uint32_t)tiles_n);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
