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
// Tiling (both formats): a workgroup of 4 waves owns a 256x256 tile of C, each
// wave a 128x128 quarter (4x4 instruction tiles, 256 fp32 accumulators per lane);
// 128-value K steps are staged in a ring of four LDS stages, filled by direct
// global-to-LDS loads three steps ahead of the step being computed.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "nvfp4.h"

namespace fp4gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

constexpr int kThreads = 256;

// Dispatch order: consecutive workgroups go round-robin over the 8 XCDs; give
// each XCD one contiguous range of tile numbers (grouped_tile below turns them
// into tiles), so the tiles that share operands run on the same XCD and meet in
// its L2.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t nb) {
  const uint32_t q = nb >> 3, rem = nb & 7;
  const uint32_t xcd = bid & 7, slot = bid >> 3;
  return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

__device__ __forceinline__ void store_tile(float* __restrict__ C, int64_t M, int64_t N, int64_t r0, int64_t c0,
                                           const v16f& acc, int l) {
  const int64_t col = c0 + (l & 31);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = r0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    if (row < M) C[row * N + col] = acc[r];
  }
}

// ------------------------------------------------------------------ MXFP4 ---

// Per 128-value K step the workgroup's 256 A rows and 256 B rows (64 bytes
// each) and their scale words are staged in LDS; every 16-byte operand piece
// read from LDS feeds four instructions.  LDS pieces are XOR-swizzled by row so
// that the 16 lanes of a read phase hit distinct banks.
constexpr int kBig = 256;  // workgroup tile (M and N)
constexpr int kStepK = 128;

struct MxStage {
  u32x4 a[kBig * 4];  // 256 rows x 4 pieces of 16 bytes (32 FP4 values each)
  u32x4 b[kBig * 4];
  uint32_t sa[kBig];  // 4 E8M0 scales per row (the step's four 32-value blocks)
  uint32_t sb[kBig];
};

__device__ __forceinline__ int piece_slot(int row, int part) { return row * 4 + (part ^ ((row >> 2) & 3)); }

// Grouped raster: 8 tile columns per group, rows outer, so that the 32
// workgroups one XCD runs at a time cover 4 tile rows x 8 tile columns and
// share their A and B slices in its L2 (measured 6% faster on 8192x20480x5120
// than groups of 4 tile rows).
__device__ __forceinline__ void grouped_tile(uint32_t L, uint32_t tiles_m, uint32_t tiles_n, uint32_t& tm,
                                             uint32_t& tn) {
  constexpr uint32_t G = 8;
  const uint32_t group = L / (G * tiles_m), first = group * G;
  const uint32_t gsize = tiles_n - first < G ? tiles_n - first : G;
  const uint32_t in = L - group * G * tiles_m;
  tn = first + in % gsize;
  tm = in / gsize;
}

template <int C>
__device__ __forceinline__ v16f mx_mfma_s(u32x4 a, u32x4 b, uint32_t sa, uint32_t sb, v16f acc) {
  const v8i va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, 2 * C, (int)sa, 2 * C, (int)sb);
}

// Operand pieces of one 64-value chunk (CH = 0, 1) of a K step, from LDS.
template <int CH>
__device__ __forceinline__ void mx_read(const MxStage& s, int wr, int wc, int l, int h, u32x4 (&fa)[4],
                                        u32x4 (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[i] = s.a[piece_slot(wr + 32 * i + (l & 31), 2 * CH + h)];
    fb[i] = s.b[piece_slot(wc + 32 * i + (l & 31), 2 * CH + h)];
  }
}

// The 16 instructions of one chunk: every A piece meets every B piece.
template <int CH>
__device__ __forceinline__ void mx_mma(const u32x4 (&fa)[4], const u32x4 (&fb)[4], const uint32_t (&sa)[4],
                                       const uint32_t (&sb)[4], v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mx_mfma_s<CH>(fa[i], fb[j], sa[i], sb[j], acc[i][j]);
}

__device__ __forceinline__ void mx_read_scales(const MxStage& s, int wr, int wc, int l, int h, uint32_t (&sa)[4],
                                               uint32_t (&sb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = s.sa[wr + 32 * i + (l & 31)] >> (8 * h);  // lane half h: blocks 2c + h -> byte 2c
    sb[i] = s.sb[wc + 32 * i + (l & 31)] >> (8 * h);
  }
}

// The operands travel from memory straight into a ring of four LDS stages
// (global_load_lds, no staging registers), three K steps ahead of the step
// being computed.  The barrier that publishes a stage waits only for that
// stage's loads (vmcnt counts the two younger steps' loads as still pending).
constexpr int kRing = 4;

// s_waitcnt immediate: vector-memory count <= N, LDS/scalar count 0 (gfx9 encoding)
#define MX_WAIT_VM_LGKM0(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (0 << 8) | (((N) >> 4) << 14))

__global__ __launch_bounds__(kThreads) void mx_gemm_dma_kernel(const uint8_t* __restrict__ A,
                                                               const uint8_t* __restrict__ As,
                                                               const uint8_t* __restrict__ B,
                                                               const uint8_t* __restrict__ Bs, int64_t M, int64_t N,
                                                               int64_t K, float* __restrict__ C, uint32_t tiles_m,
                                                               uint32_t tiles_n) {
  __shared__ MxStage st[kRing];
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, h = l >> 5;
  uint32_t tm, tn;
  grouped_tile(xcd_tile(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int64_t am0 = (int64_t)tm * kBig, bn0 = (int64_t)tn * kBig;
  const int64_t kbytes = K / 2;

  // Load j of thread t fills LDS slot p = t + 256 j, i.e. row p / 4 = t / 4 + 64 j and
  // stored part t % 4, which holds the operand piece part (t % 4) ^ swizzle(row).
  int64_t offa[4], offb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (t >> 2) + 64 * j;
    const int part = (t & 3) ^ ((row >> 2) & 3);
    const int64_t ar = am0 + row, br = bn0 + row;
    offa[j] = (ar < M ? ar : M - 1) * kbytes + 16 * part;  // rows past the edge load a valid row
    offb[j] = (br < N ? br : N - 1) * kbytes + 16 * part;
  }
  const int64_t sar = am0 + t < M ? am0 + t : M - 1, sbr = bn0 + t < N ? bn0 + t : N - 1;
  const uint8_t* gsa = As + sar * (K / 32);
  const uint8_t* gsb = Bs + sbr * (K / 32);
  const int wbase = 64 * wave;  // first slot (and scale row) this wave's loads fill

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wr = 128 * (wave >> 1), wc = 128 * (wave & 1);  // this wave's quarter of the tile
  const int64_t nsteps = K / kStepK, last = nsteps - 1;
  // 10 loads per step and thread (q = 0 .. 9: A and B pieces j = q / 2
  // alternately, then the two scale words); past the last step they re-read it
  auto issue_one = [&](int64_t step, int q) {
    const int64_t st_ = step < last ? step : last;
    MxStage& d = st[step & (kRing - 1)];
    const int64_t kb = st_ * (kStepK / 2);
    if (q < 8) {
      const int j = q >> 1;
      if ((q & 1) == 0) {
        __builtin_amdgcn_global_load_lds(A + offa[j] + kb, &d.a[256 * j + wbase], 16, 0, 0);
      } else {
        __builtin_amdgcn_global_load_lds(B + offb[j] + kb, &d.b[256 * j + wbase], 16, 0, 0);
      }
    } else if (q == 8) {
      __builtin_amdgcn_global_load_lds(gsa + st_ * (kStepK / 32), &d.sa[wbase], 4, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(gsb + st_ * (kStepK / 32), &d.sb[wbase], 4, 0, 0);
    }
  };
  auto issue = [&](int64_t step) {
#pragma unroll
    for (int q = 0; q < 10; ++q) issue_one(step, q);
  };
  issue(0);
  issue(1);
  issue(2);
  MX_WAIT_VM_LGKM0(20);  // step 0 landed (steps 1 and 2 may be pending)
  __builtin_amdgcn_s_barrier();

  u32x4 f0a[4], f0b[4], f1a[4], f1b[4];
  uint32_t sa[4], sb[4], nsa[4], nsb[4];
  mx_read<0>(st[0], wr, wc, l, h, f0a, f0b);
  mx_read_scales(st[0], wr, wc, l, h, sa, sb);
  for (int64_t s = 0; s < nsteps; ++s) {
    const MxStage& cur = st[s & (kRing - 1)];
    const MxStage& nxt = st[(s + 1) & (kRing - 1)];
    mx_read<1>(cur, wr, wc, l, h, f1a, f1b);
    __builtin_amdgcn_sched_barrier(0);
    // the chunk-0 products, with the loads of step s + 3 (into stage (s + 3) % 4 =
    // (s - 1) % 4, read by every wave before the last barrier) issued between them
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mx_mfma_s<0>(f0a[i], f0b[j], sa[i], sb[j], acc[i][j]);
        if (4 * i + j < 10) issue_one(s + 3, 4 * i + j);
        __builtin_amdgcn_sched_barrier(0);
      }
    MX_WAIT_VM_LGKM0(20);  // this thread's loads of step s + 1 have landed; steps s + 2, s + 3 pending
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    mx_read<0>(nxt, wr, wc, l, h, f0a, f0b);
    mx_read_scales(nxt, wr, wc, l, h, nsa, nsb);
    __builtin_amdgcn_sched_barrier(0);
    mx_mma<1>(f1a, f1b, sa, sb, acc);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = nsa[i];
      sb[i] = nsb[i];
    }
  }
  MX_WAIT_VM_LGKM0(0);  // no load may still be writing LDS when the workgroup ends
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) store_tile(C, M, N, am0 + wr + 32 * i, bn0 + wc + 32 * j, acc[i][j], l);
}
#undef MX_WAIT_VM_LGKM0

// ------------------------------------------------------------------ NVFP4 ---

// Same workgroup tiling and LDS ring as MXFP4.  Per 128-value K step a row
// brings 64 code bytes (four 16-byte pieces) and eight E4M3 scales (two scale
// words); each 16-value block becomes fp16 operands in registers: the code
// converts exactly to fp16, times its block scale (exact: at most 6 significant
// bits), and the fp16 instruction 32x32x16 takes 8 values per lane.  Lane half
// h walks K values [64 h, 64 h + 64) of the step: pieces 2h and 2h + 1.
struct NvStage {
  u32x4 a[kBig * 4];
  u32x4 b[kBig * 4];
  uint32_t sa[2][kBig];  // scale words: [0] blocks 0-3 of the step, [1] blocks 4-7
  uint32_t sb[2][kBig];
};

// The four E4M3 scales of a word as fp16 pairs (exact: E4M3 lies inside fp16).
__device__ __forceinline__ void nv_scales(uint32_t s, h2 (&out)[4]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(s, false);  // bytes 0, 1
  const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(s, true);   // bytes 2, 3
  const _Float16 v0 = (_Float16)lo.x, v1 = (_Float16)lo.y, v2 = (_Float16)hi.x, v3 = (_Float16)hi.y;
  out[0] = h2{v0, v0};
  out[1] = h2{v1, v1};
  out[2] = h2{v2, v2};
  out[3] = h2{v3, v3};
}

// 8 codes (one word) times their block scale, as an fp16 operand.
__device__ __forceinline__ v8h nv_half8(uint32_t w, h2 s) {
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ uint32_t word_of(const u32x4 (&q)[2], int c) {
  const u32x4 v = q[c >> 2];
  const int k = c & 3;
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

template <bool A2D, bool B2D>
__global__ __launch_bounds__(kThreads) void nv_gemm_kernel(const uint8_t* __restrict__ A,
                                                           const uint8_t* __restrict__ As,
                                                           const float* __restrict__ ats,
                                                           const uint8_t* __restrict__ B,
                                                           const uint8_t* __restrict__ Bs,
                                                           const float* __restrict__ bts, int64_t M, int64_t N,
                                                           int64_t K, float* __restrict__ C, uint32_t tiles_m,
                                                           uint32_t tiles_n) {
  __shared__ NvStage st[kRing];
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, h = l >> 5;
  uint32_t tm, tn;
  grouped_tile(xcd_tile(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int64_t am0 = (int64_t)tm * kBig, bn0 = (int64_t)tn * kBig;
  const int64_t kbytes = K / 2;

  int64_t offa[4], offb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (t >> 2) + 64 * j;
    const int part = (t & 3) ^ ((row >> 2) & 3);
    const int64_t ar = am0 + row, br = bn0 + row;
    offa[j] = (ar < M ? ar : M - 1) * kbytes + 16 * part;
    offb[j] = (br < N ? br : N - 1) * kbytes + 16 * part;
  }
  int64_t sar = am0 + t < M ? am0 + t : M - 1, sbr = bn0 + t < N ? bn0 + t : N - 1;
  if (A2D) sar /= 16;
  if (B2D) sbr /= 16;
  const uint8_t* gsa = As + sar * (K / 16);
  const uint8_t* gsb = Bs + sbr * (K / 16);
  const int wbase = 64 * wave;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wr = 128 * (wave >> 1), wc = 128 * (wave & 1);
  const int64_t nsteps = K / kStepK, last = nsteps - 1;
  auto issue = [&](int64_t step) {  // 12 loads per step and thread
    const int64_t st_ = step < last ? step : last;
    NvStage& d = st[step & (kRing - 1)];
    const int64_t kb = st_ * (kStepK / 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_global_load_lds(A + offa[j] + kb, &d.a[256 * j + wbase], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(B + offb[j] + kb, &d.b[256 * j + wbase], 16, 0, 0);
    }
    const int64_t ks = st_ * (kStepK / 16);  // 8 scale bytes per row and step
    __builtin_amdgcn_global_load_lds(gsa + ks, &d.sa[0][wbase], 4, 0, 0);
    __builtin_amdgcn_global_load_lds(gsa + ks + 4, &d.sa[1][wbase], 4, 0, 0);
    __builtin_amdgcn_global_load_lds(gsb + ks, &d.sb[0][wbase], 4, 0, 0);
    __builtin_amdgcn_global_load_lds(gsb + ks + 4, &d.sb[1][wbase], 4, 0, 0);
  };
#define NV_WAIT_VM_LGKM0(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (0 << 8) | (((N) >> 4) << 14))
  issue(0);
  issue(1);
  issue(2);
  NV_WAIT_VM_LGKM0(24);
  __builtin_amdgcn_s_barrier();

  // this lane's code pieces (2 per tile) and scale words of the current step
  u32x4 qa[4][2], qb[4][2];
  uint32_t wsa[4], wsb[4];
  auto read_step = [&](const NvStage& s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wr + 32 * i + (l & 31), rb = wc + 32 * i + (l & 31);
      qa[i][0] = s.a[piece_slot(ra, 2 * h)];
      qa[i][1] = s.a[piece_slot(ra, 2 * h + 1)];
      qb[i][0] = s.b[piece_slot(rb, 2 * h)];
      qb[i][1] = s.b[piece_slot(rb, 2 * h + 1)];
      wsa[i] = s.sa[h][ra];
      wsb[i] = s.sb[h][rb];
    }
  };
  read_step(st[0]);
  for (int64_t s = 0; s < nsteps; ++s) {
    issue(s + 3);
    h2 sca[4][4], scb[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nv_scales(wsa[i], sca[i]);
      nv_scales(wsb[i], scb[i]);
    }
    // chunk c + 1's operands are expanded while chunk c's 16 products run: two
    // operand sets alternate, and each product is followed by four of the
    // expansion's 64 instructions
    v8h fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[0][i] = nv_half8(word_of(qa[i], 0), sca[i][0]);
      fb[0][i] = nv_half8(word_of(qb[i], 0), scb[i][0]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {  // 16-value chunk c: word c of the lane's 8, block c / 2
      const int cur = c & 1;
      if (c < 7) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[cur ^ 1][i] = nv_half8(word_of(qa[i], c + 1), sca[i][(c + 1) >> 1]);
          fb[cur ^ 1][i] = nv_half8(word_of(qb[i], c + 1), scb[i][(c + 1) >> 1]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
      if (c < 7) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    NV_WAIT_VM_LGKM0(24);  // this thread's loads of step s + 1 have landed; steps s + 2, s + 3 pending
    __builtin_amdgcn_s_barrier();
    if (s + 1 < nsteps) read_step(st[(s + 1) & (kRing - 1)]);
  }
  NV_WAIT_VM_LGKM0(0);
#undef NV_WAIT_VM_LGKM0
  // the two tensor scales, applied once: fl32(acc * S_tA * S_tB) with the product taken in binary64
  const double ts = (double)ats[0] * (double)bts[0];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v16f o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = (float)((double)acc[i][j][r] * ts);
      store_tile(C, M, N, am0 + wr + 32 * i, bn0 + wc + 32 * j, o, l);
    }
}

// C = 0 for K == 0 (a kernel rather than a memset, so that the call can sit in
// a captured graph).
__global__ void zero_c_kernel(float* __restrict__ c, int64_t n) {
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x)
    c[k] = 0.0f;
}

__host__ void zero_c(float* c, int64_t n, hipStream_t s) {
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(zero_c_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(kThreads), 0, s, c, n);
}

}  // namespace fp4gemm

using namespace fp4gemm;

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Each GEMM dimension at most 2^31, so that M * N and the tile counts fit in int64.
constexpr int64_t kMaxDim = 1ll << 31;

extern "C" {

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                        nvfp4_block a_block_arg, const uint8_t* b_codes, const uint8_t* b_scales,
                        const float* b_tensor_scale, nvfp4_block b_block_arg, int64_t M, int64_t N, int64_t K,
                        float* c, void* stream) {
  // read from the enum's bytes: a C caller may pass any int, which validation must reject
  int a_block, b_block;
  memcpy(&a_block, &a_block_arg, sizeof a_block);
  memcpy(&b_block, &b_block_arg, sizeof b_block);
  if ((a_block != NVFP4_BLOCK_1D && a_block != NVFP4_BLOCK_2D) ||
      (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D))
    return NVFP4_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || K % 128) return NVFP4_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return NVFP4_ERR_SHAPE;
  if ((a_block == NVFP4_BLOCK_2D && M % 16) || (b_block == NVFP4_BLOCK_2D && N % 16)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c) return NVFP4_ERR_NULL;
  if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales || !a_tensor_scale || !b_tensor_scale))
    return NVFP4_ERR_NULL;
  if (!al16(a_codes) || !al16(b_codes) || !al4(a_scales) || !al4(b_scales) || !al4(c)) return NVFP4_ERR_ALIGN;
  const int64_t tiles_m = (M + kBig - 1) / kBig, tiles_n = (N + kBig - 1) / kBig;
  if (tiles_m * tiles_n > (1ll << 24)) return NVFP4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const uint32_t tm = (uint32_t)tiles_m, tn = (uint32_t)tiles_n;
  if (K == 0) {
    zero_c(c, M * N, s);
  } else if (a_block == NVFP4_BLOCK_2D) {
    if (b_block == NVFP4_BLOCK_2D)
      hipLaunchKernelGGL((nv_gemm_kernel<true, true>), grid, dim3(kThreads), 0, s, a_codes, a_scales, a_tensor_scale,
                         b_codes, b_scales, b_tensor_scale, M, N, K, c, tm, tn);
    else
      hipLaunchKernelGGL((nv_gemm_kernel<true, false>), grid, dim3(kThreads), 0, s, a_codes, a_scales, a_tensor_scale,
                         b_codes, b_scales, b_tensor_scale, M, N, K, c, tm, tn);
  } else {
    if (b_block == NVFP4_BLOCK_2D)
      hipLaunchKernelGGL((nv_gemm_kernel<false, true>), grid, dim3(kThreads), 0, s, a_codes, a_scales, a_tensor_scale,
                         b_codes, b_scales, b_tensor_scale, M, N, K, c, tm, tn);
    else
      hipLaunchKernelGGL((nv_gemm_kernel<false, false>), grid, dim3(kThreads), 0, s, a_codes, a_scales,
                         a_tensor_scale, b_codes, b_scales, b_tensor_scale, M, N, K, c, tm, tn);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* c, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 128) return NVFP4_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c) return NVFP4_ERR_NULL;
  if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return NVFP4_ERR_NULL;
  if (!al16(a_codes) || !al16(b_codes) || !al4(a_scales) || !al4(b_scales) || !al4(c)) return NVFP4_ERR_ALIGN;
  const int64_t bm = (M + kBig - 1) / kBig, bn = (N + kBig - 1) / kBig;
  if (bm * bn > (1ll << 24)) return NVFP4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (K == 0) {
    zero_c(c, M * N, s);
  } else {
    hipLaunchKernelGGL(mx_gemm_dma_kernel, dim3((unsigned)(bm * bn)), dim3(kThreads), 0, s, a_codes, a_scales,
                       b_codes, b_scales, M, N, K, c, (uint32_t)bm, (uint32_t)bn);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
