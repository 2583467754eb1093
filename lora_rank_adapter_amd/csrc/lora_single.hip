// Single-adapter LoRA forward and backward on gfx950.
//
// Definitions (API page "nemo_automodel.components._peft.lora_kernel"):
//   forward  (lora_forward_kernel):   res += s * (x @ A) @ B
//   backward (lora_da_dx_kernel):     DYB = dY @ B^T, dX = s * DYB @ A^T,
//                                     dA = s * X^T @ DYB (token reduction)
//            (lora_db_kernel):        AXT = A^T-frame product X @ A,
//                                     dB = s * (X @ A)^T @ dY
// (A is K x r and B is r x L in the forward frame.)
//
// Kernels:
//   fused_kernel  one workgroup owns 16*BMB tokens: it contracts the streamed
//                 operand Z (X or dY) with the first weight W1 over all of Z's
//                 features (the four waves split the feature axis; bf16 rows
//                 of Z and W1 are loaded row-linearly into a per-wave LDS tile
//                 and read back as MFMA fragments; partial sums are reduced
//                 through LDS in a fixed order), so the rank-r intermediate H
//                 exists only in registers/LDS; then every wave holds s*H as
//                 bf16 hi+lo MFMA operands and the waves walk the output
//                 columns together, multiplying by the second weight W2 and
//                 adding into (or overwriting) the output, whose row segments
//                 are read and written row-linearly through a per-wave LDS
//                 tile. Optionally it also writes s*H (transposed, hi/lo
//                 planes) for the weight-gradient kernels. Streamed tensors
//                 are loaded and stored with the non-temporal cache policy.
//   shrink_kernel the same shrink alone, writing s*H as gradient planes and/or
//                 MFMA fragments for the column-band expand below.
//   expand_band_kernel  column-band expand (the split schedule): a workgroup
//                 owns a 256-column band, keeps its W2 fragments in
//                 registers and walks token tiles, writing whole 1 KB row
//                 segments.
//   tn_kernel     weight-gradient partial sums over a chunk of tokens:
//                 part[p][n][j] = sum_m Z[m][n] * G[j][m]. Z tiles are staged
//                 in LDS (XOR-swizzled rows) and read transposed.
//   reduce_kernel fixed-order sum of the partials into the strided output.
//   pack_kernel   lays a small weight out in the orientation a kernel needs.

#include <atomic>
#include <mutex>
#include <vector>

#include "lora_device.hpp"
#include "lora_host.hpp"

namespace lora {

__device__ __forceinline__ int64_t round_up_dev(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// ---------------------------------------------------------------------------
// small utility kernels
// ---------------------------------------------------------------------------

// One weight re-layout: dst[i*ld + j] = src[i*s_i + j*s_j] for i < rows,
// j < cols, and 0 in the padding up to dst_rows x dst_cols.
struct PackJob {
  const void* src;
  int64_t s_i, s_j, rows, cols;
  void* dst;
  int64_t dst_rows, dst_cols, ld;
  int64_t tiles_j, tiles;  // 32 x 32 tiles of dst: per tile row, total
};
struct PackArgs {
  PackJob job[2];
};

// Up to two re-layouts in one launch (workgroups [0, job[0].tiles) take the
// first). Each workgroup moves one 32 x 32 tile through LDS: it reads along
// whichever source index is unit-stride and writes dst rows contiguously, so
// a transposing pack stays coalesced on both sides.
template <class E>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  __shared__ E tile[32][33];
  int64_t b = blockIdx.x;
  const int sel = b < a.job[0].tiles ? 0 : 1;
  if (sel) b -= a.job[0].tiles;
  const PackJob jb = sel ? a.job[1] : a.job[0];
  const E* __restrict__ src = static_cast<const E*>(jb.src);
  E* __restrict__ dst = static_cast<E*>(jb.dst);
  const int64_t ti = b / jb.tiles_j;
  const int64_t tj = b - ti * jb.tiles_j;
  const int tx = threadIdx.x & 31;
  const int ty = threadIdx.x >> 5;
  const bool along_i = jb.s_i == 1 && jb.s_j != 1;
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int li = along_i ? tx : ty + k;
    const int lj = along_i ? ty + k : tx;
    const int64_t i = ti * 32 + li;
    const int64_t j = tj * 32 + lj;
    tile[li][lj] = (i < jb.rows && j < jb.cols) ? src[i * jb.s_i + j * jb.s_j] : E(0);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int64_t i = ti * 32 + ty + k;
    const int64_t j = tj * 32 + tx;
    if (i < jb.dst_rows && j < jb.dst_cols) dst[i * jb.ld + j] = tile[ty + k][tx];
  }
}

// E: float (float32 zero) or uint16_t (bfloat16 zero: all bits clear)
template <class E>
__global__ __launch_bounds__(256) void fill_zero_kernel(E* __restrict__ out, int64_t rows, int64_t cols, int64_t s_r,
                                                        int64_t s_c) {
  const int64_t total = rows * cols;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / cols;
    out[i * s_r + (idx - i * cols) * s_c] = E(0);
  }
}

// out(n, j) = sum over p = 0..P-1 (in that order) of part[p][n][j], j < r.
// A thread takes V adjacent j of one n (V = 4: 16-byte loads; rp is a
// multiple of 16 and the partials are 256-byte aligned). Loads are issued 16
// partials at a time; the adds keep the p order, so both widths give the
// same bits. OT: float, or uint16_t for a bfloat16 output (the float32 sum
// rounded once, to nearest even).
template <int V, class OT>
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int P, int64_t N, int rp, int r,
                                                     OT* __restrict__ out, int64_t os_n, int64_t os_j) {
  typedef float vec_t __attribute__((ext_vector_type(V)));
  const int per_n = rp / V;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= N * per_n) return;
  const int64_t n = idx / per_n;
  const int j = static_cast<int>(idx - n * per_n) * V;
  if (j >= r) return;  // rank padding
  const vec_t* src = reinterpret_cast<const vec_t*>(part + n * rp + j);
  const int64_t step = N * rp / V;
  // the partials are added in chunk order p = 0, 1, ..., P-1; each group of
  // 16 loads is issued before any of it is added (predicated past P), so the
  // loads of a group are in flight together rather than one per add
  // (16384 x 14336 dB, 9 chunks: 13.6 -> 8 us)
  vec_t s = vec_t(0.f);
  for (int pp = 0; pp < P; pp += 16) {
    vec_t v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = (pp + e < P) ? src[(pp + e) * step] : vec_t(0.f);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (pp + e < P) s = (pp + e == 0) ? v[e] : s + v[e];
  }
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if (j + e < r) {
      if constexpr (sizeof(OT) == 2)
        out[n * os_n + (j + e) * os_j] = static_cast<uint16_t>(bf16_bits(s[e]));
      else
        out[n * os_n + (j + e) * os_j] = s[e];
    }
  }
}

// ---------------------------------------------------------------------------
// fused shrink -> expand
// ---------------------------------------------------------------------------

struct FusedArgs {
  // shrink: stream Z (M x Kin) against W1 (r rows of Kin values)
  const void* z;
  int64_t ldz;
  const void* w1;
  int64_t ldw1;
  // expand: W2 (Nout rows of r values) into the output (M x Nout, float32
  // or, for the forward, bfloat16)
  const void* w2;
  int64_t ldw2;
  void* out;
  int64_t ldo;
  // s*H written for other kernels: transposed hi/lo planes for the gradient
  // kernels (rp rows of ldg tokens) and MFMA operand fragments for the
  // column-split expand (16-token block b, rank block q, lane l at
  // frag[(b * RB + q) * 64 + l])
  void* g;
  int64_t ldg;
  uint4* frag;
  int64_t M, Kin, Nout;
  int r, rp;
  float scale;
  int64_t tiles;  // token tiles present
};

// ---- shrink of one token tile --------------------------------------------
// H^T (rank x tokens) = W1 * Z^T over the whole feature axis for the tile's
// 16*BMB tokens. Wave w takes the w-th contiguous range of contraction chunks;
// U chunks per pipeline stage, two stages in flight; the NW partial sums are
// reduced through LDS in a fixed order. On return every wave holds s*H (acc) and its
// MFMA operand form (hf). Rows past M (Z) or past r (W1) lie outside their
// buffer descriptors and read as zero.
// LDS of shrink_tile: the NW partial sums (after the feature loop) share
// their memory with the per-wave row-linear staging tiles (during it; bf16
// only: the wave's 16*BMB stream rows and 16*RB weight rows of one stage,
// rows padded by 16 bytes so that the 16 rows one fragment read touches fall
// in distinct banks).
// WT: W1 is stored feature-major (Kin rows of ldw1 elements, the r ranks of
// a feature contiguous, as lora_B's L x r weight is for the dY shrink). The
// stage then holds its 32*U feature rows of rp ranks each (rows padded by 16
// bytes) after the stream rows, and the weight fragments are read from them
// with transposed LDS reads.
template <class Tag, int NW, int RB, int BMB, int U, bool WT = false>
struct ShrinkStage {
  static constexpr int ES = sizeof(typename Tag::elem);
  static constexpr bool LIN = ES == 2;
  static_assert(!WT || LIN, "feature-major weights are read as bf16 only");
  static constexpr int SROW = U * 4 * Tag::VEC * ES;  // bytes of a row per stage
  static constexpr int PITCH = SROW + 16;
  static constexpr int WOFF = 16 * BMB * PITCH;       // first weight byte of a wave's tile
  static constexpr int WPITCH = 32 * RB + 16;         // WT: bytes per staged feature row
  // per wave: stream rows, then weight rows
  static constexpr int BYTES = !LIN ? 0 : WT ? WOFF + 32 * U * WPITCH : 16 * (BMB + RB) * PITCH;
  static constexpr int RED = NW * BMB * RB * 64 * 16;
  static constexpr int TOTAL = (NW * BYTES > RED) ? NW * BYTES : RED;
};

template <class Tag, int NW, int RB, int BMB, int U, bool WT>
__device__ __forceinline__ void shrink_tile(const FusedArgs& p, int64_t m0, f32x4_t (*red)[BMB * RB][64],
                                            f32x4_t (&acc)[BMB][RB], uint4 (&hf)[BMB][RB], char* stage) {
  using E = typename Tag::elem;
  constexpr int VEC = Tag::VEC;
  constexpr int ES = sizeof(E);
  constexpr int CH = 4 * VEC;  // contraction values per MFMA step (4 lane groups)
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  // bf16 streams are loaded row-linearly (each instruction covers whole row
  // segments of the stage: SROW bytes of 64/LPR rows) into this wave's LDS
  // tile and read back in MFMA operand order; in MFMA order every instruction
  // would touch 16 rows x 64 bytes, half of each 128-byte line.
  using SS = ShrinkStage<Tag, NW, RB, BMB, U, WT>;
  constexpr bool LIN = SS::LIN;
  constexpr int LPR = SS::SROW / 16;                 // lanes per row
  constexpr int RPI = LIN ? 64 / LPR : 16;           // rows per row-linear load
  constexpr int ZN = LIN ? 16 * BMB / RPI : BMB;     // stream vectors per lane and step group
  constexpr int WN = LIN ? 16 * RB / RPI : RB;       // weight vectors per lane and step group
  static_assert(!LIN || (64 % LPR == 0 && (16 * BMB) % RPI == 0 && ZN * RPI == 16 * BMB && WN * RPI == 16 * RB),
                "stage shape");

  const rsrc_t rz = make_rsrc(static_cast<const E*>(p.z) + m0 * p.ldz, (p.M - m0) * p.ldz * ES);
  const rsrc_t rw1 = make_rsrc(p.w1, (WT ? p.Kin : (int64_t)p.r) * p.ldw1 * ES);
  uint32_t zoff[BMB];
#pragma unroll
  for (int b = 0; b < BMB; ++b) zoff[b] = static_cast<uint32_t>(((16 * b + col) * p.ldz + grp * VEC) * ES);
  // row-linear form: lane -> row i*RPI + lane/LPR, 16-byte piece lane%LPR of
  // the stage's row segment (step piece/4, lane group piece%4)
  const int lpiece = lane % LPR;
  const int lstep = lpiece >> 2;
  const int lgrp = lpiece & 3;
  uint32_t lrow[LIN ? ZN : 1];
  if constexpr (LIN) {
#pragma unroll
    for (int i = 0; i < ZN; ++i)
      lrow[i] = static_cast<uint32_t>(((i * RPI + lane / LPR) * p.ldz + lgrp * VEC) * ES);
  }
  uint32_t woff[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q) woff[q] = static_cast<uint32_t>(((int64_t)(16 * q + col) * p.ldw1 + grp * VEC) * ES);
  // weight rows past r lie outside rw1 and read as zero
  uint32_t lwrow[LIN ? WN : 1];
  // WT: vector i of a lane is 16-byte piece wpc[i] (8 ranks) of the stage's
  // feature row wl[i] (WN = U * RB vectors cover the 32*U rows of 2*RB
  // pieces); pieces at ranks >= r read as zero (r is a multiple of 8)
  int wl[WT ? WN : 1], wpc[WT ? WN : 1];
  static_assert(!WT || WN == U * RB, "feature-major weight vectors per stage");
  if constexpr (WT) {
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int v = i * 64 + lane;
      wl[i] = v / (2 * RB);
      wpc[i] = v % (2 * RB);
      lwrow[i] = (wpc[i] * 8 < p.r) ? static_cast<uint32_t>(((int64_t)wl[i] * p.ldw1 + wpc[i] * 8) * ES) : kOOB;
    }
  } else if constexpr (LIN) {
#pragma unroll
    for (int i = 0; i < WN; ++i)
      lwrow[i] = static_cast<uint32_t>(((int64_t)(i * RPI + lane / LPR) * p.ldw1 + lgrp * VEC) * ES);
  }

#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[b][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Each wave reduces one contiguous range of CH-wide chunks: its loads walk
  // along the rows, which keeps the DRAM pages they open few.
  const int64_t nch = (p.Kin + CH - 1) / CH;
  const int64_t per = (nch + NW - 1) / NW;
  const int64_t cbeg = (int64_t)wave * per;
  const int64_t cend = (cbeg + per < nch) ? cbeg + per : nch;
  constexpr int64_t cstep = U;
  // LIN: zf[0] holds the stage's ZN row-linear stream vectors and wf[0] its
  // WN row-linear weight vectors; else [u][b] and [u][q] MFMA fragments
  auto load1 = [&](uint4 (&zf)[U][ZN], uint4 (&wf)[U][WN], int64_t c) {
    if constexpr (LIN) {
      const int64_t cc = c + lstep;
      const bool kok = cc < cend && cc * CH + lgrp * VEC < p.Kin;
      const uint32_t kb = static_cast<uint32_t>(cc * CH * ES);
#pragma unroll
      for (int i = 0; i < ZN; ++i) zf[0][i] = sload16(rz, kok ? lrow[i] + kb : kOOB);
      if constexpr (WT) {
        // the stage's feature rows c*CH .. c*CH + 32*U - 1
        const uint32_t fb = static_cast<uint32_t>(c * CH * p.ldw1 * ES);
#pragma unroll
        for (int i = 0; i < WN; ++i) {
          const bool ok = c + wl[i] / CH < cend && c * CH + wl[i] < p.Kin && lwrow[i] != kOOB;
          wf[0][i] = bload16(rw1, ok ? lwrow[i] + fb : kOOB);
        }
      } else {
#pragma unroll
        for (int i = 0; i < WN; ++i) wf[0][i] = bload16(rw1, kok ? lwrow[i] + kb : kOOB);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t cc = c + u;
        const bool kok = cc < cend && cc * CH + grp * VEC < p.Kin;
        const uint32_t kb = static_cast<uint32_t>(cc * CH * ES);
#pragma unroll
        for (int b = 0; b < BMB; ++b) zf[u][b] = sload16(rz, kok ? zoff[b] + kb : kOOB);
#pragma unroll
        for (int q = 0; q < RB; ++q) wf[u][q] = bload16(rw1, kok ? woff[q] + kb : kOOB);
      }
    }
  };
  auto mma1 = [&](const uint4 (&zf)[U][ZN], const uint4 (&wf)[U][WN]) {
    if constexpr (LIN) {
      // the stage's rows into this wave's tile (stream rows, then weight
      // rows), then fragments in operand order
#pragma unroll
      for (int i = 0; i < ZN; ++i)
        *reinterpret_cast<uint4*>(stage + (i * RPI + lane / LPR) * SS::PITCH + lpiece * 16) = zf[0][i];
      uint4 w[U][RB];
      if constexpr (WT) {
#pragma unroll
        for (int i = 0; i < WN; ++i)
          *reinterpret_cast<uint4*>(stage + SS::WOFF + wl[i] * SS::WPITCH + wpc[i] * 16) = wf[0][i];
        // fragment (u, q): lane (col, grp) needs W1[16q + col][32u + 8grp + 0..7],
        // i.e. rank 16q + col of feature rows 32u + 8grp + 0..7. A transposed
        // read hands lane i of each 16-lane group element i%4 of the 8-byte
        // pieces addressed by lanes 4e + i/4 (e < 4): lane c addresses feature
        // row 32u + 8grp + 4h + c/4, ranks 16q + 4(c%4) .. +3.
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            uint2 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
              half[h] = lds_read_tr16(stage, SS::WOFF + (32 * u + 8 * grp + 4 * h + (col >> 2)) * SS::WPITCH +
                                                 (16 * q + 4 * (col & 3)) * 2);
            w[u][q] = make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
          }
      } else {
#pragma unroll
        for (int i = 0; i < WN; ++i)
          *reinterpret_cast<uint4*>(stage + (16 * BMB + i * RPI + lane / LPR) * SS::PITCH + lpiece * 16) = wf[0][i];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < RB; ++q)
            w[u][q] = *reinterpret_cast<const uint4*>(stage + (16 * (BMB + q) + col) * SS::PITCH + (u * 4 + grp) * 16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < BMB; ++b) {
          const uint4 z = *reinterpret_cast<const uint4*>(stage + (16 * b + col) * SS::PITCH + (u * 4 + grp) * 16);
#pragma unroll
          for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[b][q], w[u][q], z);
        }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < BMB; ++b)
#pragma unroll
          for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[b][q], wf[u][q], zf[u][b]);
    }
  };
  {
    // Two register stages of U chunks: the loads of the next stage are in
    // flight while the current one is multiplied. The loop body has no exit in
    // the middle: with an odd stage count the last pass multiplies a stage
    // of zeros (every load past this wave's range reads 0).
    uint4 zA[U][ZN], wA[U][WN], zB[U][ZN], wB[U][WN];
    if (cbeg < cend) {
      load1(zA, wA, cbeg);
      for (int64_t c = cbeg; c < cend; c += 2 * cstep) {
        load1(zB, wB, c + cstep);
        sched_fence();
        mma1(zA, wA);
        sched_fence();
        load1(zA, wA, c + 2 * cstep);
        sched_fence();
        mma1(zB, wB);
        sched_fence();
      }
    }
  }
  // the staging tiles share their memory with the partial sums
  if constexpr (LIN) __syncthreads();

#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) red[wave][b * RB + q][lane] = acc[b][q];
  __syncthreads();
#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int i = b * RB + q;
      f32x4_t sum = red[0][i][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][i][lane];
      sum *= p.scale;
      acc[b][q] = sum;
      hf[b][q] = split_frag<Tag>(sum);
    }
}

// s*H of the tile as transposed planes (rank-major, token-contiguous; bf16:
// hi plane then lo plane; f32: one plane) for every token row below ldg (rows
// past M hold zeros). Called by one wave.
template <class Tag, int RB, int BMB>
__device__ __forceinline__ void emit_planes(const FusedArgs& p, int64_t m0, const f32x4_t (&acc)[BMB][RB],
                                            const uint4 (&hf)[BMB][RB]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    const int64_t m = m0 + 16 * b + col;
    if (m < p.ldg) {
#pragma unroll
      for (int q = 0; q < RB; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t j = 16 * q + 4 * grp + i;
          if constexpr (sizeof(typename Tag::elem) == 2) {
            uint16_t* gh = static_cast<uint16_t*>(p.g);
            const uint32_t hw = (i < 2 ? hf[b][q].x : hf[b][q].y) >> (16 * (i & 1));
            const uint32_t lw = (i < 2 ? hf[b][q].z : hf[b][q].w) >> (16 * (i & 1));
            gh[j * p.ldg + m] = static_cast<uint16_t>(hw & 0xFFFFu);
            gh[((int64_t)p.rp + j) * p.ldg + m] = static_cast<uint16_t>(lw & 0xFFFFu);
          } else {
            static_cast<float*>(p.g)[j * p.ldg + m] = acc[b][q][i];
          }
        }
    }
  }
}

// What an expand does with its output: overwrite it in float32 (dX), add
// into float32 (Y, an accumulated dX), or add into bfloat16 (Y), the float32
// sum rounded once.
struct OutSet {
  using T = float;
  static constexpr bool ACCUM = false;
};
struct OutAdd {
  using T = float;
  static constexpr bool ACCUM = true;
};
struct OutAddBF16 {
  using T = uint16_t;
  static constexpr bool ACCUM = true;
};
struct OutSetBF16 {  // bfloat16 dX, overwritten (the float32 product rounded once)
  using T = uint16_t;
  static constexpr bool ACCUM = false;
};

// ---- expand of one token tile over all output columns ----------------------
// out^T tile (16 columns x 16 tokens) (+)= W2 * (s*H)^T for every 16-column
// block; wave w takes NBU consecutive blocks per stage (the NW waves cover
// NW*NBU adjacent blocks together), two stages in flight, and the stage walk
// starts at stage `rot` (mod the stage count) so that tiles in flight at the
// same time do not walk the same column offsets in lockstep.
//
// The output is read and written one row segment at a time: each stage's
// MFMA products (16 columns x 16 tokens per tile, in MFMA layout) go to an
// LDS tile, and lanes then take 16-byte pieces of whole rows, add the output
// row-linearly (when the expand accumulates) and store it. How long those row segments are decides
// how fast the output streams: 2 rows x 512 bytes per instruction stream at
// the speed of a plain elementwise add over the same tensor, 8 rows x 128
// bytes up to 40% slower (measured on a 16384 x 4096 float32 output). So:
//  - SH = false (a wave's own columns span >= 256 bytes): each wave's LDS tile
//    is private (LDS instructions of one wave complete in order, no barrier)
//    and the wave writes its own columns of all 16*BMB rows;
//  - SH = true (128 bytes: rank >= 64 leaves room for two column blocks per
//    wave; 16384 x 4096, rank 64: 152 -> 133 us; with 256-byte segments the
//    barrier costs more than it gains, 62 -> 66 us for the 8192 x 4096 dX):
//    the NW waves write their products into one LDS tile of the stage's
//    NW*16*NBU columns, wait at a barrier, and wave w then reads, adds and
//    writes rows [w*16*BMB/NW, (w+1)*16*BMB/NW) over all of them. Two tiles
//    alternate between stages, so one barrier per stage suffices: a wave
//    writes tile k%2 only after every wave has passed the barrier of stage
//    k-1, i.e. finished reading tile (k-2)%2.
// Output rows past M lie outside the output descriptor (loads read 0, stores
// are dropped); columns past the output use kOOB.
template <int NW, int BMB, int NBU>
struct ExpandRows {
  static constexpr int CW = 16 * NBU;                  // columns of a wave per stage
  static constexpr bool SH = CW <= 32 && NW * CW <= 256 && (16 * BMB) % NW == 0;
  static constexpr int TW = SH ? NW * CW : CW;         // columns of an LDS tile
  static constexpr int LDW = TW + 4;                   // LDS row pitch (floats)
  static constexpr int LPR = TW / 4;                   // lanes per row (16 bytes each)
  static constexpr int RPI = 64 / LPR;                 // rows per instruction
  static constexpr int ROWS = SH ? 16 * BMB / NW : 16 * BMB;  // rows a wave writes
  static constexpr int NI = ROWS / RPI;                // row instructions per stage
  static constexpr int TILE = 16 * BMB * LDW;          // floats per LDS tile
  // floats of LDS: SH, two shared tiles; else one private tile per wave
  static constexpr int FLOATS = SH ? 2 * TILE : NW * TILE;
  static_assert(64 % LPR == 0 && ROWS % RPI == 0 && NI >= 1, "stage shape");
};

// WT: W2 is stored rank-major (r rows of ldw2 elements, output columns
// contiguous, as lora_A's r x K weight is for dX). Each stage's rank rows
// over the wave's 16*NBU columns are then loaded row-linearly, written to
// the wave's own LDS tile `wlds` (WRows<NBU>::BYTES per rank block) and read
// back as fragments with transposed reads; a wave's LDS instructions complete
// in order, so the tile needs no barrier.
template <int NBU>
struct WRows {
  static constexpr int PITCH = 32 * NBU + 16;  // bytes per staged rank row
  static constexpr int VPR = 2 * NBU;          // 16-byte vectors per rank row
  static constexpr int BYTES = 16 * PITCH;     // one rank block (16 rows)
};

template <class Tag, int NW, int RB, int BMB, int NBU, class OM, bool WT>
__device__ __forceinline__ void expand_tile_rows(const FusedArgs& p, int64_t m0, int64_t rot,
                                                 const uint4 (&hf)[BMB][RB], float* lds, char* wlds) {
  using E = typename Tag::elem;
  constexpr int ES = sizeof(E);
  using WF = WFrag<Tag>;
  using wf_t = typename WF::type;
  using X = ExpandRows<NW, BMB, NBU>;
  constexpr int LDW = X::LDW;
  constexpr int RPI = X::RPI;
  constexpr int NI = X::NI;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int lr = lane / X::LPR;       // row within an instruction
  const int lc = (lane % X::LPR) * 4; // column within the tile
  // where this wave's products go in a tile, and the first row it writes out
  const int pcol = X::SH ? wave * X::CW : 0;
  const int row0 = X::SH ? wave * X::ROWS : 0;
  float* tile0 = X::SH ? lds : lds + wave * X::TILE;
  float* tile1 = X::SH ? lds + X::TILE : tile0;
  const rsrc_t rw2 = make_rsrc(p.w2, (WT ? (int64_t)p.r : p.Nout) * p.ldw2 * ES);
  // WT: raw vector i of a lane is piece wpc[i] (8 columns) of rank row wj[i]
  // of the stage's 16*NBU columns
  using WR = WRows<NBU>;
  constexpr int NV = WT ? 16 * RB * WR::VPR / 64 : 1;
  static_assert(!WT || (16 * RB * WR::VPR) % 64 == 0, "rank rows per stage");
  int wj[NV], wpc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    wj[i] = (i * 64 + lane) / WR::VPR;
    wpc[i] = (i * 64 + lane) % WR::VPR;
  }
  using O = Out<typename OM::T>;
  const rsrc_t ro = make_rsrc(static_cast<char*>(p.out) + m0 * p.ldo * O::ES, (p.M - m0) * p.ldo * O::ES);
  const int64_t nb_end = (p.Nout + 15) / 16;
  constexpr int gstep = NW * NBU;
  // stage bookkeeping in scalar registers (a 64-bit division would leave it
  // in vector registers and turn the selects below into branches)
  const int nst = uniform_int((nb_end + gstep - 1) / gstep);
  const int r0 = nst > 0 ? uniform_int(rot % nst) : 0;
  // first column block of stage k (of the whole workgroup); nb_end past the end
  auto stage_nb = [&](int k) -> int64_t {
    const int kk = k + r0;
    const int v = (kk - (kk >= nst ? nst : 0)) * gstep;
    return k < nst ? v : nb_end;
  };
  // first column block of the tile this lane writes out, for stage block nb0
  auto tile_nb = [&](int64_t nb0) -> int64_t { return X::SH ? nb0 : nb0 + wave * NBU; };
  // output offset of this lane's piece in row instruction i of the stage at nb0
  auto ooff = [&](int i, int64_t nb0) -> uint32_t {
    const int64_t n = tile_nb(nb0) * 16 + lc;
    const int row = row0 + RPI * i + lr;
    return (nb0 < nb_end && n < p.Nout) ? static_cast<uint32_t>(((int64_t)row * p.ldo + n) * O::ES) : kOOB;
  };
  auto load2 = [&](wf_t (&wv)[NBU][RB], uint4 (&rv)[NV], f32x4_t (&cv)[NI], int64_t nb0) {
    if constexpr (WT) {
      const int64_t n0w = (nb0 + wave * NBU) * 16;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int64_t n = n0w + wpc[i] * 8;
        const bool ok = nb0 < nb_end && wj[i] < p.r && n < p.Nout;
        rv[i] = bload16(rw2, ok ? static_cast<uint32_t>(((int64_t)wj[i] * p.ldw2 + n) * ES) : kOOB);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NBU; ++u) {
        const int64_t nb = nb0 + wave * NBU + u;
        const int64_t nrow = (nb0 < nb_end && nb * 16 + col < p.Nout) ? nb * 16 + col : p.Nout;  // p.Nout: outside rw2
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          const int j0 = 16 * q + 4 * grp;
          wv[u][q] = WF::bload(rw2, static_cast<uint32_t>((nrow * p.ldw2 + j0) * ES), j0, p.r);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (OM::ACCUM)
        cv[i] = O::load4(ro, ooff(i, nb0));
      else
        cv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto comp2 = [&](wf_t (&wv)[NBU][RB], const uint4 (&rv)[NV], f32x4_t (&cv)[NI], int64_t nb0, float* tile) {
    if constexpr (WT) {
      // fragment (u, q): lane (col, grp) needs W2[n][16q + 4grp + 0..3] for
      // column n = 16u + col of the wave's stage columns, i.e. column n of
      // rank rows 16q + 4grp + 0..3: lane c of a 16-lane group addresses rank
      // row 16q + 4grp + c/4, columns 16u + 4(c%4) .. +3 (the transposed read
      // hands lane i element i%4 of the pieces of lanes 4e + i/4, e < 4)
#pragma unroll
      for (int i = 0; i < NV; ++i)
        *reinterpret_cast<uint4*>(wlds + wj[i] * WR::PITCH + wpc[i] * 16) = rv[i];
#pragma unroll
      for (int u = 0; u < NBU; ++u)
#pragma unroll
        for (int q = 0; q < RB; ++q)
          wv[u][q] = lds_read_tr16(wlds, (16 * q + 4 * grp + (col >> 2)) * WR::PITCH + (16 * u + 4 * (col & 3)) * 2);
    }
#pragma unroll
    for (int u = 0; u < NBU; ++u) {
#pragma unroll
      for (int b = 0; b < BMB; ++b) {
        f32x4_t pr = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < RB; ++q) mma_rank16<Tag>(pr, WF::operand(wv[u][q]), hf[b][q]);
        // lane holds columns 16u + 4grp .. +3 (of this wave's blocks) of token 16b + col
        *reinterpret_cast<f32x4_t*>(tile + (16 * b + col) * LDW + pcol + 16 * u + 4 * grp) = pr;
      }
    }
    if constexpr (X::SH) __syncthreads();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const f32x4_t pr = *reinterpret_cast<const f32x4_t*>(tile + (row0 + RPI * i + lr) * LDW + lc);
      O::store4(ro, ooff(i, nb0), cv[i] + pr);
    }
  };
  // two stages in flight; stages past the end read zeros and store nothing
  // (WT: the raw rank rows are in flight, the fragments are formed in comp2)
  wf_t wvA[NBU][RB], wvB[NBU][RB];
  uint4 rvA[NV], rvB[NV];
  f32x4_t cvA[NI], cvB[NI];
  if (nst > 0) {
    load2(wvA, rvA, cvA, stage_nb(0));
    for (int k = 0; k < nst; k += 2) {
      load2(wvB, rvB, cvB, stage_nb(k + 1));
      sched_fence();
      comp2(wvA, rvA, cvA, stage_nb(k), tile0);
      sched_fence();
      load2(wvA, rvA, cvA, stage_nb(k + 2));
      sched_fence();
      comp2(wvB, rvB, cvB, stage_nb(k + 1), tile1);
      sched_fence();
    }
  }
}

// Fused shrink -> expand: one workgroup per token tile, the rank intermediate
// never leaves registers and LDS (optionally also written as planes for the
// gradient kernels).
// The expand's LDS tiles reuse the shrink's LDS (staging tiles
// and partial sums) once every wave has read its reduced sums.
// WT: both weights in the transposed storage (W1 feature-major, W2
// rank-major); the expand's per-wave weight tiles follow its output tiles.
template <class Tag, int NW, int RB, int BMB, int U, int NBU, class OM, bool EMIT_G, bool WT>
__global__ __launch_bounds__(64 * NW) void fused_kernel(FusedArgs p) {
  using SS = ShrinkStage<Tag, NW, RB, BMB, U, WT>;
  constexpr int XB = ExpandRows<NW, BMB, NBU>::FLOATS * 4;
  constexpr int XW = WT ? NW * RB * WRows<NBU>::BYTES : 0;
  constexpr int LDS = SS::TOTAL > XB + XW ? SS::TOTAL : XB + XW;
  __shared__ __attribute__((aligned(16))) char shr[LDS];
  auto red = reinterpret_cast<f32x4_t(*)[BMB * RB][64]>(shr);
  const int64_t tile = blockIdx.x;
  const int64_t m0 = tile * (16 * BMB);
  f32x4_t acc[BMB][RB];
  uint4 hf[BMB][RB];
  shrink_tile<Tag, NW, RB, BMB, U, WT>(p, m0, red, acc, hf, shr + wave_id() * SS::BYTES);
  if constexpr (EMIT_G) {
    if (wave_id() == 0) emit_planes<Tag, RB, BMB>(p, m0, acc, hf);
  }
  __syncthreads();  // every wave has read the partial sums
  expand_tile_rows<Tag, NW, RB, BMB, NBU, OM, WT>(p, m0, tile, hf, reinterpret_cast<float*>(shr),
                                                  shr + XB + wave_id() * RB * WRows<NBU>::BYTES);
}

// Shrink only: s*H of each token tile, written as gradient-kernel planes
// (EMIT_G) and/or expand fragments (EMIT_F).
template <class Tag, int NW, int RB, int BMB, int U, bool EMIT_G, bool EMIT_F, bool WT>
__global__ __launch_bounds__(64 * NW) void shrink_kernel(FusedArgs p) {
  using SS = ShrinkStage<Tag, NW, RB, BMB, U, WT>;
  __shared__ __attribute__((aligned(16))) char shr[SS::TOTAL];
  auto red = reinterpret_cast<f32x4_t(*)[BMB * RB][64]>(shr);
  const int64_t m0 = (int64_t)blockIdx.x * (16 * BMB);
  f32x4_t acc[BMB][RB];
  uint4 hf[BMB][RB];
  shrink_tile<Tag, NW, RB, BMB, U, WT>(p, m0, red, acc, hf, shr + wave_id() * SS::BYTES);
  const int wave = wave_id();
  if constexpr (EMIT_G) {
    if (wave == 0) emit_planes<Tag, RB, BMB>(p, m0, acc, hf);
  }
  if constexpr (EMIT_F) {
    if (wave == NW - 1) {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int b = 0; b < BMB; ++b)
#pragma unroll
        for (int q = 0; q < RB; ++q) p.frag[((m0 / 16 + b) * RB + q) * 64 + lane] = hf[b][q];
    }
  }
}

// Column-band expand (the split schedule's second kernel). Workgroup (c, g)
// owns the output columns [c*BW, (c+1)*BW), BW = NW*NBW*16 = 256, and walks
// the token tiles g, g+G, g+2G, ... (G = gridDim.y) of 16*BMB tokens each.
// Workgroup ids run over the bands first, so the workgroups resident at any
// time cover the same few token tiles: the chip streams a narrow window of
// output rows, which keeps a large output (thousands of rows of tens of KB)
// streaming at the speed of a plain elementwise pass, where one workgroup per
// token tile walking whole rows (all rows in flight at once) loses 10-20%.
// Wave w keeps the W2 fragments of its NBW column blocks in registers for the
// whole walk. Per tile: the s*H fragments (the same for every wave), the MFMA
// products into a shared LDS tile, a barrier, then wave w reads, adds
// (when accumulating) and writes rows [w*R, (w+1)*R), R = 16*BMB/NW, of the tile over the
// band, one whole 1 KB row segment per instruction. The next tile's
// fragments and output rows load while the current one is computed; two LDS
// tiles alternate, so one barrier per tile suffices (a wave writes tile k%2
// only after every wave has passed the barrier of tile k-1, i.e. finished
// reading tile (k-2)%2). Tiles past the last read zeros and store nothing
// (empty output descriptor).
// WT: W2 stored rank-major (r rows of ldw2 elements); each wave stages the
// rank rows of its 16*NBW columns one rank block at a time in its own LDS
// tile and reads its fragments back with transposed reads, before the walk.
template <int NW, int BMB, int NBW>
struct BandShape {
  static constexpr int BW = NW * NBW * 16;     // band columns
  static constexpr int LDW = BW + 4;           // LDS row pitch (floats)
  static constexpr int TILE = 16 * BMB * LDW;  // floats per LDS tile
  static constexpr int LDS_BYTES = 2 * TILE * 4;
};

// Band `band`, token group `group` of `ngroups` (the workgroup's coordinates).
template <class Tag, int NW, int RB, int BMB, int NBW, class OM, bool WT>
__device__ __forceinline__ void expand_band_body(const FusedArgs& p, int64_t band, int64_t group, int64_t ngroups,
                                                 float* lds) {
  using E = typename Tag::elem;
  using O = Out<typename OM::T>;
  constexpr int ES = sizeof(E);
  using WF = WFrag<Tag>;
  using wf_t = typename WF::type;
  using BS = BandShape<NW, BMB, NBW>;
  constexpr int BW = BS::BW;
  constexpr int LDW = BS::LDW;
  constexpr int LPR = BW / 4;           // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;         // rows per instruction
  constexpr int R = 16 * BMB / NW;      // rows a wave writes per tile
  constexpr int NI = R / RPI;           // row instructions per tile
  static_assert(LPR <= 64 && 64 % LPR == 0 && R % RPI == 0 && NI >= 1, "band shape");
  constexpr int TILE = BS::TILE;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int lr = lane / LPR;
  const int lc = (lane % LPR) * 4;
  const int64_t c0 = band * BW;  // first column of the band
  const int64_t nb0 = c0 / 16 + wave * NBW;     // first column block of this wave

  // this wave's W2 fragments (rows past Nout and ranks past r read as zero)
  wf_t w[NBW][RB];
  if constexpr (WT) {
    using WR = WRows<NBW>;
    constexpr int NV = 16 * WR::VPR / 64;  // vectors per lane and rank block
    static_assert(NV >= 1 && (16 * WR::VPR) % 64 == 0 && NW * WR::BYTES <= 2 * TILE * 4, "band weight tile");
    char* wl = reinterpret_cast<char*>(lds) + wave * WR::BYTES;
    const rsrc_t rw2 = make_rsrc(p.w2, (int64_t)p.r * p.ldw2 * ES);
    uint4 rv[RB][NV];
#pragma unroll
    for (int q = 0; q < RB; ++q)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int v = i * 64 + lane;
        const int j = 16 * q + v / WR::VPR;
        const int64_t n = nb0 * 16 + (v % WR::VPR) * 8;
        rv[q][i] = bload16(rw2, (j < p.r && n < p.Nout) ? static_cast<uint32_t>(((int64_t)j * p.ldw2 + n) * ES) : kOOB);
      }
    // rank block q: rows 16q .. 16q+15 into the wave's tile, then fragment u
    // (lane (col, grp): column 16u + col of rank rows 16q + 4grp + 0..3) by a
    // transposed read (lane c addresses row 4grp + c/4, columns 16u + 4(c%4)).
    // The next block's writes follow this block's reads in the wave's LDS
    // order.
#pragma unroll
    for (int q = 0; q < RB; ++q) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int v = i * 64 + lane;
        *reinterpret_cast<uint4*>(wl + (v / WR::VPR) * WR::PITCH + (v % WR::VPR) * 16) = rv[q][i];
      }
#pragma unroll
      for (int u = 0; u < NBW; ++u)
        w[u][q] = lds_read_tr16(wl, (4 * grp + (col >> 2)) * WR::PITCH + (16 * u + 4 * (col & 3)) * 2);
    }
    __syncthreads();  // the tiles below reuse this LDS
  } else {
    const rsrc_t rw2 = make_rsrc(p.w2, p.Nout * p.ldw2 * ES);
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
      const int64_t n = (nb0 + u) * 16 + col;
      const int64_t nrow = n < p.Nout ? n : p.Nout;  // p.Nout: outside rw2
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int j0 = 16 * q + 4 * grp;
        w[u][q] = WF::bload(rw2, static_cast<uint32_t>((nrow * p.ldw2 + j0) * ES), j0, p.r);
      }
    }
  }
  const int64_t gstride = ngroups;
  const int64_t ncol = c0 + lc;  // this lane's output column in the row-linear pass
  auto load_tile = [&](uint4 (&hf)[BMB][RB], f32x4_t (&cv)[NI], int64_t t) {
    const bool tok = t < p.tiles;
    const int64_t m0 = tok ? t * (16 * BMB) : 0;
#pragma unroll
    for (int b = 0; b < BMB; ++b)
#pragma unroll
      for (int q = 0; q < RB; ++q) hf[b][q] = tok ? p.frag[((m0 / 16 + b) * RB + q) * 64 + lane] : zero4();
    if constexpr (OM::ACCUM) {
      const rsrc_t ro = make_rsrc(static_cast<char*>(p.out) + m0 * p.ldo * O::ES, tok ? (p.M - m0) * p.ldo * O::ES : 0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = wave * R + RPI * i + lr;
        cv[i] = O::load4(ro, ncol < p.Nout ? static_cast<uint32_t>((row * p.ldo + ncol) * O::ES) : kOOB);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) cv[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto comp_tile = [&](const uint4 (&hf)[BMB][RB], const f32x4_t (&cv)[NI], int64_t t, float* tile) {
#pragma unroll
    for (int u = 0; u < NBW; ++u)
#pragma unroll
      for (int b = 0; b < BMB; ++b) {
        f32x4_t pr = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < RB; ++q) mma_rank16<Tag>(pr, WF::operand(w[u][q]), hf[b][q]);
        // lane holds columns 16u + 4grp .. +3 of this wave's blocks, token 16b + col
        *reinterpret_cast<f32x4_t*>(tile + (16 * b + col) * LDW + 16 * (wave * NBW + u) + 4 * grp) = pr;
      }
    __syncthreads();
    const int64_t m0 = t * (16 * BMB);
    const rsrc_t ro = make_rsrc(static_cast<char*>(p.out) + m0 * p.ldo * O::ES, t < p.tiles ? (p.M - m0) * p.ldo * O::ES : 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = wave * R + RPI * i + lr;
      const f32x4_t pr = *reinterpret_cast<const f32x4_t*>(tile + row * LDW + lc);
      O::store4(ro, ncol < p.Nout ? static_cast<uint32_t>((row * p.ldo + ncol) * O::ES) : kOOB, cv[i] + pr);
    }
  };
  uint4 hfA[BMB][RB], hfB[BMB][RB];
  f32x4_t cvA[NI], cvB[NI];
  if (group < p.tiles) {
    load_tile(hfA, cvA, group);
    for (int64_t t = group; t < p.tiles; t += 2 * gstride) {
      load_tile(hfB, cvB, t + gstride);
      sched_fence();
      comp_tile(hfA, cvA, t, lds);
      sched_fence();
      load_tile(hfA, cvA, t + 2 * gstride);
      sched_fence();
      comp_tile(hfB, cvB, t + gstride, lds + TILE);
      sched_fence();
    }
  }
}

template <class Tag, int NW, int RB, int BMB, int NBW, class OM, bool WT>
__global__ __launch_bounds__(64 * NW) void expand_band_kernel(FusedArgs p) {
  __shared__ __attribute__((aligned(16))) float lds[BandShape<NW, BMB, NBW>::TILE * 2];
  expand_band_body<Tag, NW, RB, BMB, NBW, OM, WT>(p, blockIdx.x, blockIdx.y, gridDim.y, lds);
}

// ---------------------------------------------------------------------------
// weight-gradient partial sums over token chunks
// ---------------------------------------------------------------------------

struct TnArgs {
  const void* z;   // M x N stream (row-major, 16-byte rows)
  int64_t ldz;
  const void* g;   // G^T: rp rows x ldg tokens (bf16: hi plane then lo plane)
  int64_t ldg;
  float* part;     // P x N x rp
  int64_t M, N;
  int rp;
  int64_t chunk;   // tokens per chunk, a multiple of 64
  int nblk, nchunk;  // column blocks (of kTnCols) and token chunks
  int per;           // work items per XCD run: ceil(nblk * nchunk / 8)
};

template <class Tag, int RB, int NW = 4>
struct TnShape {
  static constexpr int ES = sizeof(typename Tag::elem);
  static constexpr int NS = 64 * NW;                  // columns per workgroup (64 per wave)
  static constexpr int TS = (ES == 2) ? 64 : 32;      // tokens per stage
  static constexpr int GPL = (ES == 2) ? 2 : 1;       // G planes (bf16 hi/lo)
  // LDS row pitch of G, padded by 16 bytes: the 16 rows one fragment read
  // touches then fall in distinct banks (unpadded, 128-byte rows put them on
  // two bank groups; 16384 x 14336, rank 64: lora_bwd_db 164 -> 156 us)
  static constexpr int GPITCH = TS * ES + 16;
  static constexpr int ZT_BYTES = TS * NS * ES;       // the staged Z tile
  static constexpr int GS_BYTES = GPL * 16 * RB * GPITCH;
};

// The k-th work item of XCD `xcd` (the mapping below), with the Z tile and G
// rows staged in `zt` and `gs`.
template <class Tag, int RB, int NW = 4>
__device__ __forceinline__ void tn_body(const TnArgs& p, int xcd, int k, char* zt, char* gs) {
  using E = typename Tag::elem;
  using TSh = TnShape<Tag, RB, NW>;
  constexpr int VEC = Tag::VEC;
  constexpr int ES = sizeof(E);
  constexpr int NT = 64 * NW;         // threads
  constexpr int NSB = 4;              // 16-column blocks per wave
  constexpr int NS = TSh::NS;         // columns per workgroup
  static_assert(NS == 16 * NSB * NW, "tn columns");
  constexpr int TS = TSh::TS;         // tokens per stage (bf16: two 32-token MFMA steps)
  constexpr int ROWB = NS * ES;       // LDS bytes per staged Z row
  constexpr int VPR = NS / VEC;       // 128-bit vectors per Z row
  constexpr int ZV = TS * VPR / NT;   // Z vectors per thread per stage
  static_assert(ZV * NT == TS * VPR, "Z stage");
  constexpr int GPL = TSh::GPL;
  constexpr int GPITCH = TSh::GPITCH;
  constexpr int GVR = TS / VEC;           // vectors per G row
  constexpr int GTOT = GPL * 16 * RB * GVR;
  constexpr int GV = (GTOT + NT - 1) / NT;
  // rows 8 (bf16) or 4 (f32) apart are read together by the four lane groups:
  // XOR their 32/64-byte column windows apart to avoid LDS bank conflicts.
  constexpr int SWZ_SHIFT = (ES == 2) ? 3 : 2;
  constexpr int SWZ_UNIT = (ES == 2) ? 32 : 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  // Work items (token chunk c, column block b) in chunk-major order are cut
  // into 8 runs of `per` consecutive items, run x on XCD x (workgroup ids are
  // dealt round-robin to the XCDs: the k-th workgroup of XCD x takes item
  // x * per + k). With a multiple of 8 chunks every chunk's column blocks
  // share one XCD, so the chunk's G rows, which all of them read, stay in
  // that XCD's L2 (16384 x 14336, rank 64: lora_bwd_db 158 -> 144 us); with
  // fewer chunks each XCD still gets its share of the columns. Items past the
  // last exit.
  const int item = xcd * p.per + k;
  if (item >= p.nblk * p.nchunk) return;
  const int chunk_id = item / p.nblk;
  const int64_t n_base = (int64_t)(item - chunk_id * p.nblk) * NS;
  const int64_t m_begin = (int64_t)chunk_id * p.chunk;
  const int64_t m_end = (m_begin + p.chunk < p.M) ? (m_begin + p.chunk) : p.M;
  const E* z = static_cast<const E*>(p.z);
  const E* g = static_cast<const E*>(p.g);

  f32x4_t acc[NSB][RB];
#pragma unroll
  for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[nb][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // stages of loads in flight: one (two or three measured slower: the
  // registers then allow one wave per SIMD; 16384 x 14336, rank 64:
  // lora_bwd_db 169 -> 185 / 199 us)
  constexpr int DEPTH = 1;
  uint4 zr[DEPTH][ZV];
  uint4 gr[DEPTH][GV];

  // Z rows past the chunk end and G columns past M read 0 (the G buffer holds
  // zeros for tokens in [M, ldg)); Z columns past N use kOOB.
  const rsrc_t rz = make_rsrc(z + m_begin * p.ldz, (m_end - m_begin) * p.ldz * ES);
  const rsrc_t rg = make_rsrc(g, (int64_t)GPL * p.rp * p.ldg * ES);
  auto load_stage = [&](int d, int64_t m0) {
#pragma unroll
    for (int i = 0; i < ZV; ++i) {
      const int v = tid + NT * i;
      const int row = v / VPR;
      const int vc = v - row * VPR;
      const int64_t n = n_base + (int64_t)vc * VEC;
      zr[d][i] = sload16(rz, n < p.N ? static_cast<uint32_t>(((m0 - m_begin + row) * p.ldz + n) * ES) : kOOB);
    }
#pragma unroll
    for (int i = 0; i < GV; ++i) {
      const int v = tid + NT * i;
      const int grow = v / GVR;  // plane * 16*RB + j
      const int vc = v - grow * GVR;
      gr[d][i] = bload16(rg, v < GTOT ? static_cast<uint32_t>(((int64_t)grow * p.ldg + m0 + vc * VEC) * ES) : kOOB);
    }
  };

  // LDS byte offset of Z(row, column byte cb). bf16: the 32-byte (16-column)
  // block index is XORed with a 4-bit row code so that the 16 rows one
  // transposed read touches (rows 8g + j, g, j < 4) land in 16 different
  // blocks; f32: 64-byte windows XORed with rows 4 apart.
  auto zoff = [&](int row, int cb) -> int {
    if constexpr (ES == 2) {
      const int code = (row & 3) | (((row >> 3) & 3) << 2);
      return row * ROWB + ((((cb >> 5) ^ code) << 5) | (cb & 31));
    } else {
      return row * ROWB + (cb ^ (((row >> SWZ_SHIFT) & 3) * SWZ_UNIT));
    }
  };

  auto store_stage = [&](int d) {
#pragma unroll
    for (int i = 0; i < ZV; ++i) {
      const int v = tid + NT * i;
      const int row = v / VPR;
      const int vc = v - row * VPR;
      *reinterpret_cast<uint4*>(zt + zoff(row, vc * 16)) = zr[d][i];
    }
#pragma unroll
    for (int i = 0; i < GV; ++i) {
      const int v = tid + NT * i;
      if (v < GTOT) *reinterpret_cast<uint4*>(gs + (v / GVR) * GPITCH + (v % GVR) * 16) = gr[d][i];
    }
  };

  // f32 operand element (bf16 operands use transposed reads instead)
  auto zval = [&](int m, int nl) -> uint32_t { return *reinterpret_cast<const uint32_t*>(zt + zoff(m, nl * ES)); };

  auto compute = [&]() {
    if constexpr (ES == 2) {
#pragma unroll
      for (int u = 0; u < TS / 32; ++u) {
        uint4 ghi[RB], glo[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          ghi[q] = *reinterpret_cast<const uint4*>(gs + (16 * q + col) * GPITCH + u * 64 + grp * 16);
          glo[q] = *reinterpret_cast<const uint4*>(gs + (16 * RB + 16 * q + col) * GPITCH + u * 64 + grp * 16);
        }
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb) {
          // Z^T fragment: lane (col, grp) needs Z[32u + 8grp + 0..7][n0 + col]. A
          // transposed read hands lane i of each 16-lane group element i%4 of
          // the 8-byte pieces addressed by lanes 4e + i/4 (e < 4): lane c
          // addresses row 32u + 8grp + 4h + c/4, columns n0 + 4(c%4) .. +3.
          const int n0 = (wave * NSB + nb) * 16;
          uint2 half[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 32 * u + 8 * grp + 4 * h + (col >> 2);
            const int off = zoff(row, (n0 + 4 * (col & 3)) * 2);
            half[h] = lds_read_tr16(zt, off);
          }
          const uint4 zf = make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            mma_vec<Tag>(acc[nb][q], zf, ghi[q]);
            mma_vec<Tag>(acc[nb][q], zf, glo[q]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint4 gf[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q)
          gf[q] = *reinterpret_cast<const uint4*>(gs + (16 * q + col) * GPITCH + (u * 16 + 4 * grp) * 4);
#pragma unroll
        for (int nb = 0; nb < NSB; ++nb) {
          const int nl = (wave * NSB + nb) * 16 + col;
          const uint4 zf = make_uint4(zval(16 * u + 4 * grp + 0, nl), zval(16 * u + 4 * grp + 1, nl),
                                      zval(16 * u + 4 * grp + 2, nl), zval(16 * u + 4 * grp + 3, nl));
#pragma unroll
          for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[nb][q], zf, gf[q]);
        }
      }
    }
  };

  // DEPTH stages of loads in flight: stage s + DEPTH loads while stage s is
  // multiplied. Stages past the chunk read zeros (Z rows past the chunk end)
  // and add nothing, so the loop body needs no exit in the middle.
  const int64_t nstage = (m_end - m_begin + TS - 1) / TS;
  if (nstage > 0) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_stage(d, m_begin + d * TS);
    for (int64_t s = 0; s < nstage; s += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        __syncthreads();
        store_stage(d);
        __syncthreads();
        load_stage(d, m_begin + (s + d + DEPTH) * TS);
        sched_fence();
        compute();
        sched_fence();
      }
    }
  }

  float* part = p.part + (int64_t)chunk_id * p.N * p.rp;
#pragma unroll
  for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n_base + (wave * NSB + nb) * 16 + 4 * grp + i;
      if (n < p.N) {
#pragma unroll
        for (int q = 0; q < RB; ++q) part[n * p.rp + 16 * q + col] = acc[nb][q][i];
      }
    }
}

template <class Tag, int RB, int NW>
__global__ __launch_bounds__(64 * NW) void tn_kernel(TnArgs p) {
  using TSh = TnShape<Tag, RB, NW>;
  __shared__ __attribute__((aligned(16))) char zt[TSh::ZT_BYTES];
  __shared__ __attribute__((aligned(16))) char gs[TSh::GS_BYTES];
  tn_body<Tag, RB, NW>(p, static_cast<int>(blockIdx.x & 7), static_cast<int>(blockIdx.x >> 3), zt, gs);
}

// Where the workgroups of band_tn_kernel go: the first `tn_groups` groups of
// 8 consecutive ids (one per XCD) are weight-gradient groups, the rest
// column-band expand items.
struct BandTnMap {
  int64_t tn_groups;
  int64_t band_items, bands, band_groups;  // items = bands x token groups
};

// dX's column-band expand and dA's weight-gradient partials in one launch.
// Both read only what the shrink before them wrote (fragments and planes of
// s*dYB) and the call's inputs, so they may run side by side: the expand
// writes dX while the partial sums stream X, instead of a write-only pass
// and then a read-only one, each with its own tail. The weight-gradient
// workgroups (the longer ones) take the first ids, so they start first and
// the band items fill the CUs as they finish (16384 x 4096 x 14336, rank 64:
// lora_bwd_dx_da 181 us as two launches, 188 us with the two kinds
// interleaved evenly, 173 us this way). Group g < T of 8 workgroups takes,
// on XCD x, the weight-gradient item of XCD x's g-th workgroup in tn_kernel
// (ids are dealt round-robin to the XCDs, so a group of 8 consecutive ids
// covers each XCD once).
template <class Tag, int RB, int BMB, class OM, bool WT>
__global__ __launch_bounds__(256) void band_tn_kernel(FusedArgs a, TnArgs t, BandTnMap m) {
  using TSh = TnShape<Tag, RB>;
  constexpr int TN_LDS = TSh::ZT_BYTES + TSh::GS_BYTES;
  constexpr int BAND_LDS = BandShape<4, BMB, 4>::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char shr[TN_LDS > BAND_LDS ? TN_LDS : BAND_LDS];
  const int64_t g = blockIdx.x >> 3;
  const int x = static_cast<int>(blockIdx.x & 7);
  if (g < m.tn_groups) {
    tn_body<Tag, RB>(t, x, static_cast<int>(g), shr, shr + TSh::ZT_BYTES);
    return;
  }
  const int64_t i = (g - m.tn_groups) * 8 + x;
  if (i >= m.band_items) return;
  expand_band_body<Tag, 4, RB, BMB, 4, OM, WT>(a, i % m.bands, i / m.bands, m.band_groups,
                                               reinterpret_cast<float*>(shr));
}

// ---------------------------------------------------------------------------
// host-side schedule plan and launch helpers
// ---------------------------------------------------------------------------

constexpr int kTnCols = 256;  // columns per 4-wave tn_kernel workgroup (64 per wave)

// Stage sizes: U contraction chunks (shrink) and NBU column blocks (expand)
// per pipeline stage. A bf16 expand stage holds RB weight fragments
// (2 VGPRs) and BMB output tiles (4 VGPRs) per column block; keep a stage
// near 48 VGPRs. A shrink stage holds U*(BMB+RB) 16-byte vectors.
constexpr int pow2_floor(int v) { return v >= 8 ? 8 : v >= 4 ? 4 : v >= 2 ? 2 : 1; }
// At rank > 32 the register rule alone leaves one 32-feature step per
// stage, and the shrink loops are latency-bound with about one wave per SIMD
// (16384 x 14336 dY shrink: 3.6 resident waves per CU, 156 us); two steps
// per stage there measured 156 -> 95 us for that shrink and 441 -> 421 us
// for the forward at 16384 x 4096 x 14336, rank 64 (four steps: no further
// gain).
template <int RB, int BMB>
struct FusedShape {
  static constexpr int U0 = (8 / (BMB + RB)) > 0 ? pow2_floor(8 / (BMB + RB)) : 1;
  static constexpr int U = (RB >= 4 && U0 < 2) ? 2 : U0;
  // (four column blocks per stage at rank 64 measured no faster: 416 against
  // 417 us, with one wave per SIMD)
  static constexpr int NBU = pow2_floor(48 / (2 * RB + 4 * BMB));
};

// ---------------------------------------------------------------------------
// Schedule plan. Every choice follows from the shapes alone (no run-time
// tuning, no environment); each branch is reached by shape in the parity
// tests. Measured on the MI355X (rocprofv3 kernel traces):
//
//  - contraction <= 8192 features: fused_kernel (one launch, the rank
//    intermediate stays on chip), 4 waves. Token blocks (16 tokens each) per
//    tile: forward 4 or 2 while rb*bmb <= 8 and the grid keeps >= 512
//    workgroups, else 1; dX (no output loads) 2 at rank <= 16 while >= 256
//    workgroups, else 1 (8192 x 4096, rank 16: 63.6 against 67.0 us).
//  - contraction > 8192 features (the dX of an MLP-up layer contracts over
//    its 14336 outputs), or a forward output of 256 MB (the Infinity
//    Cache) or more: shrink_kernel writes s*H as MFMA fragments, then
//    expand_band_kernel updates the output band by band. In the fused kernel
//    every workgroup owns whole output rows, so all rows stream at once; at
//    16384 x 14336 (940 MB) that pattern tops out near 5.2 TB/s even as a
//    plain add, while the band order streams at 5.8 TB/s (forward 410 ->
//    352 us); at 8192 x 4096 (134 MB) the fused kernel stays faster (58.5
//    against 62.1 us).
//  - dX: the split schedule from a 128 MB output on, its band expand and
//    dA's weight-gradient partials in one launch (band_tn_kernel): 16384 x
//    4096 x 4096, rank 64 (268 MB): 170 -> 115 us for lora_bwd_dx_da; at
//    8192 x 4096 x 4096, rank 16 (134 MB) 60.2 against 60.4 us fused.
//  - shrink tiles: 16*bmb tokens with bmb 4 or 2 while rb*bmb <= 16 and
//    >= 256 workgroups; 1 at rank <= 16 (twice the workgroups measure faster
//    there: 34.8 against 36.7 us for the X*A shrink at 8192 x 4096, rank 16);
//    8 waves while the cross-wave partial-sum buffer stays <= 32 KB, else 4.
//  - column-band expand: 32-token tiles (16 at rank > 64, where the
//    fragments of two token blocks would not fit the registers), about four
//    tiles per workgroup.
//  - weight-gradient token chunks: about 512 workgroups in all, at most one
//    chunk per 64 tokens (P = 32 at 8192 x 4096 measured best for a launch
//    of its own: 16 chunks 16.5, 64 chunks 16.7 us against 15.1 us); about
//    256 beside dX's band expand; dB over wide outputs: 8-wave, 512-column
//    workgroups in one round (tn_plan).
// ---------------------------------------------------------------------------

constexpr int64_t kFusedMaxContraction = 8192;
constexpr int64_t kFusedMaxOutputBytes = int64_t(256) << 20;    // forward: below the Infinity Cache's size
constexpr int64_t kFusedMaxDxOutputBytes = int64_t(128) << 20;  // dX: below half of it

struct SinglePlan {
  bool fused;        // fused_kernel, else shrink_kernel + expand_band_kernel
  int bmb;           // token blocks per fused tile, or per expand_band tile
  int bmb_shrink;    // token blocks per shrink_kernel tile (its waves: launch_shrink)
};

static int bmb_expand(int64_t M, int rb) {
  for (int c : {4, 2}) {
    if (c * rb <= 8 && ceil_div(M, 16 * c) >= 512) return c;
  }
  return 1;
}

static int bmb_shrink(int64_t M, int rb) {
  if (rb == 1) return 1;
  for (int c : {4, 2}) {
    if (c * rb <= 16 && ceil_div(M, 16 * c) >= 256) return c;
  }
  return 1;
}

// dX/dA's shrink of dY: at rank 16 or less, 32-token tiles (one workgroup per
// CU at 8192 tokens) halve the weight rows each CU re-reads per dY row:
// lora_bwd_dx_da at rank 16 57.0 -> 56.3 us at 8192 x 4096 x 4096, 104.5 ->
// 101.0 at 16384 x 4096 x 4096, 166.8 -> 154.2 at 16384 x 4096 x 14336; the
// X*A shrinks of the forward and of dB measured 0.6-1.1 us slower with them.
static int bmb_shrink_dy(int64_t M, int rb) {
  if (rb == 1) return ceil_div(M, 32) >= 256 ? 2 : 1;
  return bmb_shrink(M, rb);
}

// forward (expand accumulates into its output) or dX (no output loads);
// kin = contraction of the shrink, nout = width of the expand, oes = bytes
// per output element.
static SinglePlan plan_single(bool forward, int64_t M, int64_t kin, int64_t nout, int rb, int64_t oes) {
  SinglePlan p{};
  p.fused = kin <= kFusedMaxContraction && M * nout * oes < (forward ? kFusedMaxOutputBytes : kFusedMaxDxOutputBytes);
  p.bmb_shrink = forward ? bmb_shrink(M, rb) : bmb_shrink_dy(M, rb);
  if (p.fused)
    p.bmb = forward ? bmb_expand(M, rb) : ((rb == 1 && ceil_div(M, 32) >= 256) ? 2 : 1);
  else
    p.bmb = rb <= 4 ? 2 : 1;
  return p;
}

// Token groups of the column-band expand: about four token tiles per
// workgroup (measured on a 16384 x 14336 float32 output: 32-token tiles and
// 1 KB bands stream at 5.8 TB/s with 64-128 groups, 4.9 TB/s with 16).
static int64_t band_groups(int64_t tiles) {
  const int64_t g = ceil_div(tiles, 4);
  return g < 1 ? 1 : g;
}

// Token chunks of the weight-gradient kernels: about `wgs` workgroups in all,
// a multiple of 8 chunks from 8 on (one XCD per chunk, the same number per
// XCD), at most one chunk per 64 tokens.
static int64_t tn_chunks_for(int64_t M, int64_t N, int64_t wgs, int64_t cols) {
  const int64_t slices = ceil_div(N, cols);
  int64_t P = ceil_div(wgs, slices);
  P = P < 8 ? P : (P + 4) / 8 * 8;
  const int64_t cap = ceil_div(M, 64);
  if (P > cap) P = cap;
  return P < 1 ? 1 : P;
}

// Weight-gradient plan: waves per workgroup (64 columns each), the chunk
// count the partials are sized for, tokens per chunk. dB over wide outputs
// (wide_ok, N >= kTnWideMin) takes 8-wave, 512-column workgroups: one stage
// of loads in flight per thread (more costs occupancy), so a wider workgroup
// keeps twice the bytes in flight, and each G row it stages serves twice the
// columns. Only one such workgroup fits a CU's LDS, so the grid is one round:
// as many token chunks as keep the workgroups within the 256 CUs
// (lora_bwd_db, rank 64, L = 14336: 16384 tokens 142.6 -> 138.8 us with 8
// chunks (224 workgroups), 134 us with 9 (252; a chunk's column blocks then
// no longer all share one XCD); 8192 tokens 83.7 -> 80.9 us; 448
// workgroups, 1.75 rounds: 152.6 and 96.2 us).
// dA's partial sums beside dX's band expand (band_tn_kernel) take about 256
// workgroups: the band items fill the rest of the chip, and half as many
// chunks halve the partials to write and add (lora_bwd_dx_da 172.0 -> 168.5
// us at 16384 x 4096 x 14336, 59.6 -> 57.7 us at 8192 x 4096 x 4096, 114.0
// -> 108.9 us at 8192 x 4096 x 14336; 128 workgroups: 179.7, 61.4, 112.5 us).
// The workspace holds the partials of the 512-workgroup plan, the most.
constexpr int64_t kTnWideMin = 8192;
constexpr int64_t kTnBandWgs = 256;
struct TnPlan {
  int nw;
  int64_t P, chunk;
};
static TnPlan tn_plan(int64_t M, int64_t N, bool wide_ok, bool beside_band = false) {
  TnPlan t;
  t.nw = (wide_ok && N >= kTnWideMin) ? 8 : 4;
  if (t.nw == 8) {
    int64_t P = 256 / ceil_div(N, (int64_t)512);
    const int64_t cap = ceil_div(M, 64);
    if (P > cap) P = cap;
    t.P = P < 1 ? 1 : P;
  } else {
    t.P = tn_chunks_for(M, N, beside_band ? kTnBandWgs : 512, 64 * t.nw);
  }
  t.chunk = round_up(ceil_div(M, t.P), 64);
  return t;
}

// ---------------------------------------------------------------------------
// kernel dispatch
// ---------------------------------------------------------------------------

template <class Tag, int NW, int RB, int BMB, class OM, bool EMIT_G, bool WT>
struct FusedLaunch {
  static void run(FusedArgs a, hipStream_t st) {
    using S = FusedShape<RB, BMB>;
    // kernels that write planes cover every token row below ldg (zeros past M)
    const int64_t rows = (EMIT_G && a.ldg > a.M) ? a.ldg : a.M;
    a.tiles = ceil_div(rows, 16 * BMB);
    launch((fused_kernel<Tag, NW, RB, BMB, S::U, S::NBU, OM, EMIT_G, WT>), dim3((unsigned)a.tiles), dim3(64 * NW),
           0, st, a);
  }
};

template <class Tag, int NW, int RB, int BMB, bool EMIT_G, bool EMIT_F, bool WT>
struct ShrinkLaunch {
  static void run(FusedArgs a, hipStream_t st) {
    using S = FusedShape<RB, BMB>;
    const int64_t rows = (EMIT_G && a.ldg > a.M) ? a.ldg : a.M;
    a.tiles = ceil_div(rows, 16 * BMB);
    launch((shrink_kernel<Tag, NW, RB, BMB, S::U, EMIT_G, EMIT_F, WT>), dim3((unsigned)a.tiles), dim3(64 * NW), 0,
           st, a);
  }
};

template <class Tag, int RB, int BMB, class OM, bool WT>
struct ExpandBandLaunch {
  static void run(FusedArgs a, hipStream_t st) {
    constexpr int NW = 4, NBW = 4;  // 256-column bands
    a.tiles = ceil_div(a.M, 16 * BMB);
    const int64_t bands = ceil_div(a.Nout, (int64_t)NW * NBW * 16);
    launch((expand_band_kernel<Tag, NW, RB, BMB, NBW, OM, WT>),
           dim3(static_cast<unsigned>(bands), static_cast<unsigned>(band_groups(a.tiles))), dim3(64 * NW), 0, st, a);
  }
};

// (rank blocks, token blocks) with rb * bmb <= 8
template <template <int, int> class L, class... A>
static void dispatch8(int rb, int bmb, A&&... args) {
  switch (rb * 10 + bmb) {
    case 11: L<1, 1>::run(args...); break;
    case 12: L<1, 2>::run(args...); break;
    case 14: L<1, 4>::run(args...); break;
    case 21: L<2, 1>::run(args...); break;
    case 22: L<2, 2>::run(args...); break;
    case 24: L<2, 4>::run(args...); break;
    case 41: L<4, 1>::run(args...); break;
    case 42: L<4, 2>::run(args...); break;
    default: L<8, 1>::run(args...); break;  // rb 8 (bmb 1 only)
  }
}

// The (rank blocks, token blocks) pairs plan_single gives dX: fused
// kernel (16-token tiles, 32 at one rank block) and column-band expand
// (32-token tiles, 16 at eight rank blocks); only these are instantiated.
template <template <int, int> class L, class... A>
static void dispatch_dx_fused(int rb, int bmb, A&&... args) {
  switch (rb * 10 + bmb) {
    case 11: L<1, 1>::run(args...); break;
    case 12: L<1, 2>::run(args...); break;
    case 21: L<2, 1>::run(args...); break;
    case 41: L<4, 1>::run(args...); break;
    default: L<8, 1>::run(args...); break;  // rb 8
  }
}
template <template <int, int> class L, class... A>
static void dispatch_dx_band(int rb, A&&... args) {
  switch (rb) {
    case 1: L<1, 2>::run(args...); break;
    case 2: L<2, 2>::run(args...); break;
    case 4: L<4, 2>::run(args...); break;
    default: L<8, 1>::run(args...); break;
  }
}

template <class Tag, class OM, bool EMIT_G, bool WT>
struct FusedNW {
  template <int RB, int BMB>
  using L = FusedLaunch<Tag, 4, RB, BMB, OM, EMIT_G, WT>;
};
template <class Tag, class OM, bool WT>
struct ExpandBandRB {
  template <int RB, int BMB>
  using L = ExpandBandLaunch<Tag, RB, BMB, OM, WT>;
};

template <class Tag, bool EMIT_G, bool EMIT_F, bool WT = false>
static void launch_shrink(const FusedArgs& a, int rb, int bmb, hipStream_t st) {
  // the pairs bmb_shrink() and bmb_shrink_dy() return; 8 waves while the cross-wave partial-sum
  // buffer (NW * rb * bmb KB) stays <= 32 KB, else 4
  switch (rb * 10 + bmb) {
    case 11: ShrinkLaunch<Tag, 8, 1, 1, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 12: ShrinkLaunch<Tag, 8, 1, 2, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 21: ShrinkLaunch<Tag, 8, 2, 1, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 22: ShrinkLaunch<Tag, 8, 2, 2, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 24: ShrinkLaunch<Tag, 4, 2, 4, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 41: ShrinkLaunch<Tag, 8, 4, 1, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 42: ShrinkLaunch<Tag, 4, 4, 2, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 44: ShrinkLaunch<Tag, 4, 4, 4, EMIT_G, EMIT_F, WT>::run(a, st); break;
    case 81: ShrinkLaunch<Tag, 4, 8, 1, EMIT_G, EMIT_F, WT>::run(a, st); break;
    default: ShrinkLaunch<Tag, 4, 8, 2, EMIT_G, EMIT_F, WT>::run(a, st); break;  // rb 8, bmb 2
  }
}

// tn_kernel's work items: column blocks x token chunks, `per` per XCD
static void tn_grid(TnArgs& a, int cols) {
  a.nblk = static_cast<int>(ceil_div(a.N, (int64_t)cols));
  a.nchunk = static_cast<int>(ceil_div(a.M, a.chunk));
  a.per = static_cast<int>(ceil_div((int64_t)a.nblk * a.nchunk, 8));
}

// Shrink Z against W1 and expand into the output as the plan says; with
// EMIT_G also writes the planes for the gradient kernels; WT: weights in the
// transposed storage (dX from nn.Linear-layout bf16 weights).
template <class Tag, class OM, bool EMIT_G, bool WT = false>
static void run_shrink_expand(FusedArgs a, const SinglePlan& pl, int rb, hipStream_t st) {
  if (pl.fused) {
    dispatch8<FusedNW<Tag, OM, EMIT_G, WT>::template L>(rb, pl.bmb, a, st);
    return;
  }
  launch_shrink<Tag, EMIT_G, true, WT>(a, rb, pl.bmb_shrink, st);
  dispatch8<ExpandBandRB<Tag, OM, WT>::template L>(rb, pl.bmb, a, st);
}

template <class Tag, class OM, bool WT>
struct BandTnRB {
  template <int RB, int BMB>
  struct L {
    static void run(FusedArgs a, TnArgs t, hipStream_t st) {
      a.tiles = ceil_div(a.M, 16 * BMB);
      tn_grid(t, kTnCols);
      BandTnMap m{};
      m.bands = ceil_div(a.Nout, (int64_t)256);
      m.band_groups = band_groups(a.tiles);
      m.band_items = m.bands * m.band_groups;
      m.tn_groups = t.per;
      const int64_t groups = m.tn_groups + ceil_div(m.band_items, (int64_t)8);
      launch((band_tn_kernel<Tag, RB, BMB, OM, WT>), dim3(static_cast<unsigned>(8 * groups)), dim3(256), 0, st, a, t,
             m);
    }
  };
};

template <class Tag>
static void launch_tn(TnArgs a, int rb, int nw, hipStream_t st) {
  tn_grid(a, 64 * nw);
  const dim3 grid(static_cast<unsigned>(8 * a.per));
  const dim3 block(static_cast<unsigned>(64 * nw));
  switch (rb * 10 + nw) {
    case 14: launch((tn_kernel<Tag, 1, 4>), grid, block, 0, st, a); break;
    case 24: launch((tn_kernel<Tag, 2, 4>), grid, block, 0, st, a); break;
    case 44: launch((tn_kernel<Tag, 4, 4>), grid, block, 0, st, a); break;
    case 84: launch((tn_kernel<Tag, 8, 4>), grid, block, 0, st, a); break;
    case 18: launch((tn_kernel<Tag, 1, 8>), grid, block, 0, st, a); break;
    case 28: launch((tn_kernel<Tag, 2, 8>), grid, block, 0, st, a); break;
    case 48: launch((tn_kernel<Tag, 4, 8>), grid, block, 0, st, a); break;
    default: launch((tn_kernel<Tag, 8, 8>), grid, block, 0, st, a); break;
  }
}

// The dX/dA call's kernels after the weights are in place: the fused
// shrink-expand (writing the planes of s*dYB) and then the weight-gradient
// partials; or, on the split schedule, the shrink and then dX's band expand
// and dA's partials in one launch.
template <class Tag, class OM, bool WT>
static void run_dx_da(FusedArgs a, TnArgs t, const SinglePlan& pl, int rb, hipStream_t st) {
  if (pl.fused) {
    dispatch_dx_fused<FusedNW<Tag, OM, true, WT>::template L>(rb, pl.bmb, a, st);
    launch_tn<Tag>(t, rb, 4, st);
    return;
  }
  launch_shrink<Tag, true, true, WT>(a, rb, pl.bmb_shrink, st);
  dispatch_dx_band<BandTnRB<Tag, OM, WT>::template L>(rb, a, t, st);
}



static PackJob pack_job(const void* src, int64_t s_i, int64_t s_j, int64_t rows, int64_t cols, void* dst,
                        int64_t dst_rows, int64_t dst_cols, int64_t ld) {
  PackJob j{src, s_i, s_j, rows, cols, dst, dst_rows, dst_cols, ld, ceil_div(dst_cols, 32), 0};
  j.tiles = ceil_div(dst_rows, 32) * j.tiles_j;
  return j;
}

// Launches the re-layouts (one or two) as a single kernel.
static void launch_pack(int32_t dtype, const PackJob& j0, const PackJob* j1, hipStream_t st) {
  PackArgs a{};
  a.job[0] = j0;
  if (j1) a.job[1] = *j1;
  const int64_t blocks = a.job[0].tiles + a.job[1].tiles;
  if (blocks <= 0) return;
  if (dtype == LORA_BF16)
    launch(pack_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
  else
    launch(pack_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
}

static void launch_fill_zero(const lora_mat* m, hipStream_t st) {
  const int64_t total = m->rows * m->cols;
  if (total <= 0) return;
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 8192) blocks = 8192;
  if (m->dtype == LORA_BF16)
    launch(fill_zero_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
           static_cast<uint16_t*>(m->ptr), m->rows, m->cols, m->stride_row, m->stride_col);
  else
    launch(fill_zero_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, static_cast<float*>(m->ptr),
           m->rows, m->cols, m->stride_row, m->stride_col);
}

template <class OT>
static void launch_reduce_t(const float* part, int P, int64_t N, int rp, int r, OT* out, int64_t os_n, int64_t os_j,
                            hipStream_t st) {
  // 16-byte loads while that keeps >= 256 workgroups (the 16384 x 14336 dB
  // call: 146 -> 140 us); fewer, longer threads measured slower at 8192 x
  // 4096, rank 16 (64 workgroups: +1.5 us per call)
  const int64_t wide = N * (rp / 4);
  if (wide >= 256 * 256)
    launch(reduce_kernel<4, OT>, dim3(static_cast<unsigned>(ceil_div(wide, 256))), dim3(256), 0, st, part, P, N, rp,
           r, out, os_n, os_j);
  else
    launch(reduce_kernel<1, OT>, dim3(static_cast<unsigned>(ceil_div(N * rp, 256))), dim3(256), 0, st, part, P, N,
           rp, r, out, os_n, os_j);
}

// The fixed-order sum of the P partials into out (float32 or bfloat16).
static void launch_reduce(const float* part, int P, int64_t N, int rp, int r, const lora_mat* out, int64_t os_n,
                          int64_t os_j, hipStream_t st) {
  if (N * r <= 0) return;
  if (out->dtype == LORA_BF16)
    launch_reduce_t(part, P, N, rp, r, static_cast<uint16_t*>(out->ptr), os_n, os_j, st);
  else
    launch_reduce_t(part, P, N, rp, r, static_cast<float*>(out->ptr), os_n, os_j, st);
}

// Buffer descriptors address with 32-bit byte offsets: every range one
// descriptor spans must stay below 2^31 bytes.
static bool fits32(int64_t bytes) { return bytes >= 0 && bytes <= kMaxBufferBytes; }

// Offsets the shrink/expand kernels form: one 64-token tile of the stream
// and of the output, and the whole of each weight.
static bool fused_fits(int64_t ldz, size_t es, int64_t r, int64_t ldw1, int64_t nout, int64_t ldw2, int64_t ldo,
                       size_t oes = 4) {
  const int64_t rp = padded_rank(static_cast<int>(r));
  return fits32(64 * ldz * (int64_t)es) && fits32(rp * ldw1 * (int64_t)es) && fits32((nout + 16) * ldw2 * (int64_t)es) &&
         fits32(64 * ldo * (int64_t)oes);
}

// Workspace pieces of each operation (the same function sizes and carves).
struct SingleLayout {
  size_t w1 = 0, w2 = 0, g = 0, part = 0, frag = 0;
  int64_t ldg = 0, P = 0;
  size_t total() const {
    return static_cast<size_t>(round_up(w1, 256) + round_up(w2, 256) + round_up(g, 256) + round_up(part, 256) +
                               round_up(frag, 256));
  }
};

static SingleLayout layout_for(int op, int64_t M, int64_t K, int64_t L, int r, int32_t dtype) {
  SingleLayout s;
  const size_t es = elem_size(dtype);
  const int64_t rp = padded_rank(r);
  // MFMA fragments of s*H: one 1 KB record per 16-token block and rank block,
  // for token rows rounded up to a 64-token tile
  const size_t frag = static_cast<size_t>(round_up(M > 0 ? M : 1, 64) / 16 * (rp / 16)) * 1024;
  if (op == LORA_OP_FWD) {
    s.w1 = static_cast<size_t>(rp * K) * es;  // A as r x K
    s.w2 = static_cast<size_t>(L * rp) * es;  // B as L x r
    s.frag = frag;
  } else if (op == LORA_OP_BWD_DX_DA) {
    s.w1 = static_cast<size_t>(rp * L) * es;  // B as r x L
    s.w2 = static_cast<size_t>(K * rp) * es;  // A as K x r
    s.ldg = round_up(M > 0 ? M : 1, 64);
    s.g = static_cast<size_t>(4 * rp * s.ldg);
    s.P = tn_plan(M, K, false).P;
    s.part = static_cast<size_t>(s.P * K * rp) * 4;
    s.frag = frag;
  } else {
    s.w1 = static_cast<size_t>(rp * K) * es;  // A as r x K
    s.ldg = round_up(M > 0 ? M : 1, 64);
    s.g = static_cast<size_t>(4 * rp * s.ldg);
    s.P = tn_plan(M, L, true).P;
    s.part = static_cast<size_t>(s.P * L * rp) * 4;
  }
  return s;
}

// ---------------------------------------------------------------------------
// kernel timing (measurement tools)
// ---------------------------------------------------------------------------

namespace {
struct EventPair {
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
std::atomic<bool> g_timing_on{false};
std::vector<EventPair> g_timing_events;  // reused across recording sessions
size_t g_timing_used = 0;                // pairs handed out since lora_timing_begin
}  // namespace

bool timing_take(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_timing_on.load(std::memory_order_relaxed)) return false;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (!g_timing_on.load(std::memory_order_relaxed)) return false;
  if (g_timing_used == g_timing_events.size()) {
    EventPair e{};
    if (hipEventCreate(&e.start) != hipSuccess) return false;
    if (hipEventCreate(&e.stop) != hipSuccess) {
      (void)hipEventDestroy(e.start);
      return false;
    }
    g_timing_events.push_back(e);
  }
  *start = g_timing_events[g_timing_used].start;
  *stop = g_timing_events[g_timing_used].stop;
  ++g_timing_used;
  return true;
}

}  // namespace lora

using namespace lora;

extern "C" int lora_abi_version(void) { return LORA_ABI_VERSION; }

extern "C" int lora_timing_begin(void) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  g_timing_used = 0;
  g_timing_on.store(true);
  return LORA_OK;
}

extern "C" int lora_timing_reserve(int64_t pairs) {
  if (pairs < 0) return LORA_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  while (static_cast<int64_t>(g_timing_events.size()) < pairs) {
    EventPair e{};
    if (hipEventCreate(&e.start) != hipSuccess) return LORA_ERR_LAUNCH;
    if (hipEventCreate(&e.stop) != hipSuccess) {
      (void)hipEventDestroy(e.start);
      return LORA_ERR_LAUNCH;
    }
    g_timing_events.push_back(e);
  }
  return LORA_OK;
}

extern "C" int lora_timing_pause(void) {
  g_timing_on.store(false);
  return LORA_OK;
}

extern "C" int lora_timing_resume(void) {
  g_timing_on.store(true);
  return LORA_OK;
}

extern "C" int lora_timing_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return LORA_ERR_NULL;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  double sum = 0.0;
  for (size_t i = 0; i < g_timing_used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timing_events[i].stop) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timing_events[i].start, g_timing_events[i].stop) != hipSuccess)
      return LORA_ERR_LAUNCH;
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int64_t>(g_timing_used);
  return LORA_OK;
}

extern "C" const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL: return "a required pointer is NULL";
    case LORA_ERR_SHAPE: return "operand shapes disagree or a size is unsupported";
    case LORA_ERR_DTYPE: return "unsupported or mixed dtype";
    case LORA_ERR_STRIDE: return "unsupported stride or alignment of a streamed operand";
    case LORA_ERR_RANK: return "rank outside [1, 128]";
    case LORA_ERR_WORKSPACE: return "workspace missing or too small";
    case LORA_ERR_LAUNCH: return "HIP kernel launch failed";
    case LORA_ERR_LIMIT: return "a size exceeds a library limit";
    default: return "unknown status";
  }
}

extern "C" size_t lora_workspace_bytes(int op, int64_t M, int64_t K, int64_t L, int32_t r, int32_t dtype) {
  if (op < LORA_OP_FWD || op > LORA_OP_BWD_DB) return 0;
  if (M < 0 || K < 0 || L < 0 || r < 1 || r > 128 || !float_dtype_ok(dtype)) return 0;
  // sizes whose x (M x K) or output (M x L) could not exist: every operand
  // fits in kMaxOperand bytes
  int64_t mk = 0, ml = 0;
  if (K > kMaxOperand || L > kMaxOperand || M > kMaxOperand || __builtin_mul_overflow(M, K, &mk) ||
      __builtin_mul_overflow(M, L, &ml) || mk > kMaxOperand || ml > kMaxOperand)
    return 0;
  return layout_for(op, M, K, L, r, dtype).total();
}

extern "C" int lora_fwd(const lora_mat* x, const lora_mat* lora_A, const lora_mat* lora_B, const lora_mat* res,
                        float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !lora_A || !lora_B || !res) return LORA_ERR_NULL;
  if (!valid_dims(x) || !valid_dims(lora_A) || !valid_dims(lora_B) || !valid_dims(res)) return LORA_ERR_SHAPE;
  const int64_t M = x->rows, K = x->cols, r = lora_A->cols, L = lora_B->cols;
  if (lora_A->rows != K || lora_B->rows != r || res->rows != M || res->cols != L) return LORA_ERR_SHAPE;
  // float32 output for any inputs; bfloat16 output (updated in place, one
  // rounding) for bfloat16 inputs
  if (!float_dtype_ok(x->dtype) || lora_A->dtype != x->dtype || lora_B->dtype != x->dtype ||
      !(res->dtype == LORA_F32 || (res->dtype == LORA_BF16 && x->dtype == LORA_BF16)))
    return LORA_ERR_DTYPE;
  if (r < 1 || r > 128) return LORA_ERR_RANK;
  if ((M * K > 0 && !x->ptr) || (K * r > 0 && !lora_A->ptr) || (r * L > 0 && !lora_B->ptr) ||
      (M * L > 0 && !res->ptr))
    return LORA_ERR_NULL;
  const int vec = vec_elems(x->dtype);
  if (K % vec != 0 || L % 4 != 0) return LORA_ERR_SHAPE;
  if (M * K > 0 && check_rowmajor_stream(x) != LORA_OK) return LORA_ERR_STRIDE;
  if (M * L > 0 && check_rowmajor_stream(res) != LORA_OK) return LORA_ERR_STRIDE;
  if (M == 0 || L == 0 || K == 0) return LORA_OK;

  const size_t es = elem_size(x->dtype);
  const int rb = rank_blocks(static_cast<int>(r));
  const int64_t rp = 16 * rb;
  // A is read in place when it is a view of an r x K row-major weight.
  const bool a_direct = lora_A->stride_row == 1 && lora_A->stride_col >= K &&
                        (lora_A->stride_col * (int64_t)es) % 16 == 0 && aligned(lora_A->ptr, 16);
  // B is read in place when it is a view of an L x r weight with r contiguous,
  // r a multiple of 4 and 4-element aligned rows (the kernel reads rank columns
  // in groups of 4).
  const bool b_direct = lora_B->stride_row == 1 && r % 4 == 0 && lora_B->stride_col >= r &&
                        lora_B->stride_col % 4 == 0 && aligned(lora_B->ptr, 4 * es);
  const SingleLayout lay = layout_for(LORA_OP_FWD, M, K, L, static_cast<int>(r), x->dtype);
  // Weights read in place and the fused schedule use no workspace: the
  // caller may then pass none.
  const size_t oes = elem_size(res->dtype);
  const SinglePlan plan = plan_single(true, M, K, L, rb, static_cast<int64_t>(oes));
  const bool needs_ws = !a_direct || !b_direct || !plan.fused;
  if (needs_ws && (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total()))
    return LORA_ERR_WORKSPACE;
  Carver cv(needs_ws ? workspace : nullptr);
  void* w1p = cv.take(lay.w1);
  void* w2p = cv.take(lay.w2);
  uint4* frag = static_cast<uint4*>(cv.take(lay.frag));
  if (!fused_fits(x->stride_row, es, r, a_direct ? lora_A->stride_col : K, L, b_direct ? lora_B->stride_col : rp,
                  res->stride_row, oes))
    return LORA_ERR_LIMIT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  FusedArgs a{};
  a.z = x->ptr;
  a.ldz = x->stride_row;
  PackJob jobs[2];
  int njobs = 0;
  if (a_direct) {
    a.w1 = lora_A->ptr;
    a.ldw1 = lora_A->stride_col;
  } else {
    jobs[njobs++] = pack_job(lora_A->ptr, lora_A->stride_col, lora_A->stride_row, r, K, w1p, rp, K, K);
    a.w1 = w1p;
    a.ldw1 = K;
  }
  if (b_direct) {
    a.w2 = lora_B->ptr;
    a.ldw2 = lora_B->stride_col;
  } else {
    jobs[njobs++] = pack_job(lora_B->ptr, lora_B->stride_col, lora_B->stride_row, L, r, w2p, L, rp, rp);
    a.w2 = w2p;
    a.ldw2 = rp;
  }
  if (njobs > 0) launch_pack(x->dtype, jobs[0], njobs > 1 ? &jobs[1] : nullptr, st);
  a.out = res->ptr;
  a.ldo = res->stride_row;
  a.M = M;
  a.Kin = K;
  a.Nout = L;
  a.r = static_cast<int>(r);
  a.rp = static_cast<int>(rp);
  a.scale = scale;
  a.frag = frag;
  if (res->dtype == LORA_BF16)
    run_shrink_expand<BF16, OutAddBF16, false>(a, plan, rb, st);
  else if (x->dtype == LORA_BF16)
    run_shrink_expand<BF16, OutAdd, false>(a, plan, rb, st);
  else
    run_shrink_expand<F32, OutAdd, false>(a, plan, rb, st);
  return launch_status();
}

// dX overwritten (accumulate = false) or added to (true); dA always overwritten.
static int bwd_dx_da(const lora_mat* xt, const lora_mat* dy, const lora_mat* lora_B, const lora_mat* lora_A,
                     float scale, const lora_mat* dx, const lora_mat* dA, void* workspace, size_t workspace_bytes,
                     void* stream, bool accumulate) {
  if (!xt || !dy || !lora_B || !lora_A || !dx || !dA) return LORA_ERR_NULL;
  if (!valid_dims(xt) || !valid_dims(dy) || !valid_dims(lora_B) || !valid_dims(lora_A) || !valid_dims(dx) ||
      !valid_dims(dA))
    return LORA_ERR_SHAPE;
  const int64_t K = xt->rows, M = xt->cols, L = dy->cols, r = lora_B->cols;
  if (dy->rows != M || lora_B->rows != L || lora_A->rows != r || lora_A->cols != K || dx->rows != M ||
      dx->cols != K || dA->rows != K || dA->cols != r)
    return LORA_ERR_SHAPE;
  // outputs in float32, or in bfloat16 with bfloat16 inputs
  auto out_ok = [&](int32_t d) { return d == LORA_F32 || (d == LORA_BF16 && xt->dtype == LORA_BF16); };
  if (!float_dtype_ok(xt->dtype) || dy->dtype != xt->dtype || lora_B->dtype != xt->dtype ||
      lora_A->dtype != xt->dtype || !out_ok(dx->dtype) || !out_ok(dA->dtype))
    return LORA_ERR_DTYPE;
  if (r < 1 || r > 128) return LORA_ERR_RANK;
  if ((K * M > 0 && !xt->ptr) || (M * L > 0 && !dy->ptr) || (L * r > 0 && !lora_B->ptr) ||
      (r * K > 0 && !lora_A->ptr) || (M * K > 0 && !dx->ptr) || (K * r > 0 && !dA->ptr))
    return LORA_ERR_NULL;
  const int vec = vec_elems(xt->dtype);
  if (K % vec != 0 || L % vec != 0) return LORA_ERR_SHAPE;
  if (K * M > 0 && check_colmajor_stream(xt) != LORA_OK) return LORA_ERR_STRIDE;
  if (M * L > 0 && check_rowmajor_stream(dy) != LORA_OK) return LORA_ERR_STRIDE;
  if (M * K > 0 && check_rowmajor_stream(dx) != LORA_OK) return LORA_ERR_STRIDE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (K == 0) return LORA_OK;
  if (M == 0 || L == 0) {
    if (!accumulate) launch_fill_zero(dx, st);
    launch_fill_zero(dA, st);
    return launch_status();
  }
  const SingleLayout lay = layout_for(LORA_OP_BWD_DX_DA, M, K, L, static_cast<int>(r), xt->dtype);
  if (!workspace || !aligned(workspace, 256)) return LORA_ERR_WORKSPACE;
  if (workspace_bytes < lay.total()) return LORA_ERR_WORKSPACE;
  Carver cv(workspace);
  void* w1p = cv.take(lay.w1);
  void* w2p = cv.take(lay.w2);
  void* gbuf = cv.take(lay.g);
  float* part = static_cast<float*>(cv.take(lay.part));
  uint4* frag = static_cast<uint4*>(cv.take(lay.frag));

  const int rb = rank_blocks(static_cast<int>(r));
  const int64_t rp = 16 * rb;
  const size_t es = elem_size(xt->dtype);
  const size_t oes = elem_size(dx->dtype);
  const SinglePlan plan = plan_single(false, M, L, K, rb, static_cast<int64_t>(oes));
  const int64_t chunk = tn_plan(M, K, false, !plan.fused).chunk;
  if (!fused_fits(dy->stride_row, es, r, L, K, rp, dx->stride_row, oes) ||
      !fits32(chunk * xt->stride_col * (int64_t)es) || !fits32((int64_t)lay.g))
    return LORA_ERR_LIMIT;
  // The kernels take W1 = B^T (r rows over the L outputs) and W2 = A^T (K rows
  // over the r ranks). bf16 weights in the nn.Linear layouts (lora_B L x r and
  // lora_A r x K, rows contiguous, 16-byte aligned rows, r a multiple of 8)
  // are read in place in that transposed storage; any other layout is first
  // packed into the workspace.
  const bool in_place = xt->dtype == LORA_BF16 && r % 8 == 0 && lora_B->stride_col == 1 &&
                        lora_B->stride_row >= r && lora_B->stride_row % 8 == 0 && aligned(lora_B->ptr, 16) &&
                        lora_A->stride_col == 1 && lora_A->stride_row >= K && lora_A->stride_row % 8 == 0 &&
                        aligned(lora_A->ptr, 16) && fits32(L * lora_B->stride_row * (int64_t)es) &&
                        fits32(r * lora_A->stride_row * (int64_t)es);
  FusedArgs a{};
  if (in_place) {
    a.w1 = lora_B->ptr;
    a.ldw1 = lora_B->stride_row;
    a.w2 = lora_A->ptr;
    a.ldw2 = lora_A->stride_row;
  } else {
    const PackJob jb = pack_job(lora_B->ptr, lora_B->stride_col, lora_B->stride_row, r, L, w1p, rp, L, L);
    const PackJob ja = pack_job(lora_A->ptr, lora_A->stride_col, lora_A->stride_row, K, r, w2p, K, rp, rp);
    launch_pack(xt->dtype, jb, &ja, st);
    a.w1 = w1p;
    a.ldw1 = L;
    a.w2 = w2p;
    a.ldw2 = rp;
  }
  a.z = dy->ptr;
  a.ldz = dy->stride_row;
  a.out = dx->ptr;
  a.ldo = dx->stride_row;
  a.g = gbuf;
  a.ldg = lay.ldg;
  a.M = M;
  a.Kin = L;
  a.Nout = K;
  a.r = static_cast<int>(r);
  a.rp = static_cast<int>(rp);
  a.scale = scale;
  a.frag = frag;
  TnArgs t{};
  t.z = xt->ptr;
  t.ldz = xt->stride_col;
  t.g = gbuf;
  t.ldg = lay.ldg;
  t.part = part;
  t.M = M;
  t.N = K;
  t.rp = static_cast<int>(rp);
  t.chunk = chunk;
  const int P = static_cast<int>(ceil_div(M, t.chunk));
  if (dx->dtype == LORA_BF16) {
    if (in_place) {
      if (accumulate)
        run_dx_da<BF16, OutAddBF16, true>(a, t, plan, rb, st);
      else
        run_dx_da<BF16, OutSetBF16, true>(a, t, plan, rb, st);
    } else {
      if (accumulate)
        run_dx_da<BF16, OutAddBF16, false>(a, t, plan, rb, st);
      else
        run_dx_da<BF16, OutSetBF16, false>(a, t, plan, rb, st);
    }
  } else if (xt->dtype == LORA_BF16) {
    if (in_place) {
      if (accumulate)
        run_dx_da<BF16, OutAdd, true>(a, t, plan, rb, st);
      else
        run_dx_da<BF16, OutSet, true>(a, t, plan, rb, st);
    } else {
      if (accumulate)
        run_dx_da<BF16, OutAdd, false>(a, t, plan, rb, st);
      else
        run_dx_da<BF16, OutSet, false>(a, t, plan, rb, st);
    }
  } else {
    if (accumulate)
      run_dx_da<F32, OutAdd, false>(a, t, plan, rb, st);
    else
      run_dx_da<F32, OutSet, false>(a, t, plan, rb, st);
  }
  launch_reduce(part, P, K, static_cast<int>(rp), static_cast<int>(r), dA, dA->stride_row,
                dA->stride_col, st);
  return launch_status();
}

extern "C" int lora_bwd_dx_da(const lora_mat* xt, const lora_mat* dy, const lora_mat* lora_B, const lora_mat* lora_A,
                              float scale, const lora_mat* dx, const lora_mat* dA, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return bwd_dx_da(xt, dy, lora_B, lora_A, scale, dx, dA, workspace, workspace_bytes, stream, false);
}

extern "C" int lora_bwd_dx_da_accumulate(const lora_mat* xt, const lora_mat* dy, const lora_mat* lora_B,
                                         const lora_mat* lora_A, float scale, const lora_mat* dx, const lora_mat* dA,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_dx_da(xt, dy, lora_B, lora_A, scale, dx, dA, workspace, workspace_bytes, stream, true);
}

extern "C" int lora_bwd_db(const lora_mat* lora_A, const lora_mat* xt, const lora_mat* dy, float scale,
                           const lora_mat* dB, void* workspace, size_t workspace_bytes, void* stream) {
  if (!lora_A || !xt || !dy || !dB) return LORA_ERR_NULL;
  if (!valid_dims(lora_A) || !valid_dims(xt) || !valid_dims(dy) || !valid_dims(dB)) return LORA_ERR_SHAPE;
  const int64_t r = lora_A->rows, K = lora_A->cols, M = xt->cols, L = dy->cols;
  if (xt->rows != K || dy->rows != M || dB->rows != r || dB->cols != L) return LORA_ERR_SHAPE;
  // dB in float32, or in bfloat16 with bfloat16 inputs
  if (!float_dtype_ok(lora_A->dtype) || xt->dtype != lora_A->dtype || dy->dtype != lora_A->dtype ||
      !(dB->dtype == LORA_F32 || (dB->dtype == LORA_BF16 && xt->dtype == LORA_BF16)))
    return LORA_ERR_DTYPE;
  if (r < 1 || r > 128) return LORA_ERR_RANK;
  if ((r * K > 0 && !lora_A->ptr) || (K * M > 0 && !xt->ptr) || (M * L > 0 && !dy->ptr) || (r * L > 0 && !dB->ptr))
    return LORA_ERR_NULL;
  const int vec = vec_elems(xt->dtype);
  if (K % vec != 0 || L % vec != 0) return LORA_ERR_SHAPE;
  if (K * M > 0 && check_colmajor_stream(xt) != LORA_OK) return LORA_ERR_STRIDE;
  if (M * L > 0 && check_rowmajor_stream(dy) != LORA_OK) return LORA_ERR_STRIDE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (L == 0) return LORA_OK;
  if (M == 0 || K == 0) {
    launch_fill_zero(dB, st);
    return launch_status();
  }
  const SingleLayout lay = layout_for(LORA_OP_BWD_DB, M, K, L, static_cast<int>(r), xt->dtype);
  if (!workspace || !aligned(workspace, 256)) return LORA_ERR_WORKSPACE;
  if (workspace_bytes < lay.total()) return LORA_ERR_WORKSPACE;
  Carver cv(workspace);
  void* w1p = cv.take(lay.w1);
  cv.take(lay.w2);
  void* gbuf = cv.take(lay.g);
  float* part = static_cast<float*>(cv.take(lay.part));

  const size_t es = elem_size(xt->dtype);
  const int rb = rank_blocks(static_cast<int>(r));
  const int64_t rp = 16 * rb;
  FusedArgs a{};
  const bool a_direct = lora_A->stride_col == 1 && lora_A->stride_row >= K &&
                        (lora_A->stride_row * (int64_t)es) % 16 == 0 && aligned(lora_A->ptr, 16);
  const TnPlan tp = tn_plan(M, L, true);
  const int64_t chunk = tp.chunk;
  if (!fused_fits(xt->stride_col, es, r, a_direct ? lora_A->stride_row : K, 0, 0, 0) ||
      !fits32(chunk * dy->stride_row * (int64_t)es) || !fits32((int64_t)lay.g))
    return LORA_ERR_LIMIT;
  if (a_direct) {
    a.w1 = lora_A->ptr;
    a.ldw1 = lora_A->stride_row;
  } else {
    launch_pack(xt->dtype, pack_job(lora_A->ptr, lora_A->stride_row, lora_A->stride_col, r, K, w1p, rp, K, K), nullptr,
                st);
    a.w1 = w1p;
    a.ldw1 = K;
  }
  a.z = xt->ptr;
  a.ldz = xt->stride_col;
  a.g = gbuf;
  a.ldg = lay.ldg;
  a.M = M;
  a.Kin = K;
  a.Nout = 0;
  a.r = static_cast<int>(r);
  a.rp = static_cast<int>(rp);
  a.scale = scale;
  const int bmb = bmb_shrink(M, rb);
  TnArgs t{};
  t.z = dy->ptr;
  t.ldz = dy->stride_row;
  t.g = gbuf;
  t.ldg = lay.ldg;
  t.part = part;
  t.M = M;
  t.N = L;
  t.rp = static_cast<int>(rp);
  t.chunk = chunk;
  const int P = static_cast<int>(ceil_div(M, t.chunk));
  if (xt->dtype == LORA_BF16) {
    launch_shrink<BF16, true, false>(a, rb, bmb, st);
    launch_tn<BF16>(t, rb, tp.nw, st);
  } else {
    launch_shrink<F32, true, false>(a, rb, bmb, st);
    launch_tn<F32>(t, rb, tp.nw, st);
  }
  // dB is r x L: partial row n = l, column j.
  launch_reduce(part, P, L, static_cast<int>(rp), static_cast<int>(r), dB, dB->stride_col,
                dB->stride_row, st);
  return launch_status();
}
