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
//                 features (the four waves split the feature axis, MFMA
//                 partial sums are reduced through LDS in a fixed order), so
//                 the rank-r intermediate H exists only in registers/LDS; then
//                 every wave holds s*H as bf16 hi+lo MFMA operands and the
//                 waves walk the output columns together, multiplying by the
//                 second weight W2 and adding into (or overwriting) the
//                 output with 128-bit accesses. Optionally it also writes s*H
//                 (transposed, hi/lo planes) for the weight-gradient kernels.
//   tn_kernel     weight-gradient partial sums over a chunk of tokens:
//                 part[p][n][j] = sum_m Z[m][n] * G[j][m]. Z tiles are staged
//                 in LDS (XOR-swizzled rows) and read transposed.
//   reduce_kernel fixed-order sum of the partials into the strided output.
//   pack_kernel   lays a small weight out in the orientation a kernel needs.

#include "lora_device.hpp"
#include "lora_host.hpp"

namespace lora {

// ---------------------------------------------------------------------------
// small utility kernels
// ---------------------------------------------------------------------------

template <class E>
__global__ __launch_bounds__(256) void pack_kernel(const E* __restrict__ src, int64_t s_i, int64_t s_j, int64_t rows,
                                                   int64_t cols, E* __restrict__ dst, int64_t dst_rows,
                                                   int64_t dst_cols, int64_t ld) {
  const int64_t total = dst_rows * dst_cols;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / dst_cols;
    const int64_t j = idx - i * dst_cols;
    dst[i * ld + j] = (i < rows && j < cols) ? src[i * s_i + j * s_j] : E(0);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ out, int64_t rows, int64_t cols,
                                                        int64_t s_r, int64_t s_c) {
  const int64_t total = rows * cols;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t i = idx / cols;
    out[i * s_r + (idx - i * cols) * s_c] = 0.0f;
  }
}

// out(n, j) = sum over p = 0..P-1 (in that order) of part[p][n][j], j < r.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, int P, int64_t N, int rp, int r,
                                                     float* __restrict__ out, int64_t os_n, int64_t os_j) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= N * r) return;
  const int64_t n = idx / r;
  const int j = static_cast<int>(idx - n * r);
  const float* src = part + n * rp + j;
  const int64_t step = N * rp;
  float s = src[0];
  for (int pp = 1; pp < P; ++pp) s += src[pp * step];
  out[n * os_n + j * os_j] = s;
}

// ---------------------------------------------------------------------------
// fused shrink -> expand
// ---------------------------------------------------------------------------

struct FusedArgs {
  const void* z;   // M x Kin stream (row-major, 16-byte rows)
  int64_t ldz;
  const void* w1;  // rows j < r of Kin contiguous values
  int64_t ldw1;
  const void* w2;  // rows n < Nout of r contiguous values
  int64_t ldw2;
  float* out;      // M x Nout float32
  int64_t ldo;
  void* g;         // emitted s*H transposed: rp rows of ldg tokens
  int64_t ldg;
  int64_t M, Kin, Nout;
  int r, rp;
  float scale;
};

template <class Tag, int RB, int BMB, int NBU, bool EXPAND, bool ACCUM, bool EMIT>
__global__ __launch_bounds__(256) void fused_kernel(FusedArgs p) {
  using E = typename Tag::elem;
  constexpr int VEC = Tag::VEC;
  constexpr int CH = 4 * VEC;  // contraction values per MFMA step (4 lane groups)
  constexpr int U = (8 / (BMB + RB)) > 0 ? (8 / (BMB + RB)) : 1;
  __shared__ f32x4_t red[4][BMB * RB][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * (16 * BMB);

  // ---- phase 1: H^T (rank x tokens) = W1 * Z^T, waves split the feature axis
  f32x4_t acc[BMB][RB];
#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[b][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const E* zrow[BMB];
  bool zok[BMB];
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    const int64_t m = m0 + 16 * b + col;
    zok[b] = m < p.M;
    zrow[b] = static_cast<const E*>(p.z) + (zok[b] ? m : 0) * p.ldz + grp * VEC;
  }
  const E* wrow[RB];
  bool wok[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q) {
    const int j = 16 * q + col;
    wok[q] = j < p.r;
    wrow[q] = static_cast<const E*>(p.w1) + (int64_t)(wok[q] ? j : 0) * p.ldw1 + grp * VEC;
  }

  const int64_t nch = (p.Kin + CH - 1) / CH;
  for (int64_t c = wave; c < nch; c += 4 * U) {
    uint4 zf[U][BMB];
    uint4 wf[U][RB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cc = c + 4 * u;
      const bool kok = cc < nch && cc * CH + grp * VEC < p.Kin;
#pragma unroll
      for (int b = 0; b < BMB; ++b) zf[u][b] = (kok && zok[b]) ? ld16(zrow[b] + cc * CH) : zero4();
#pragma unroll
      for (int q = 0; q < RB; ++q) wf[u][q] = (kok && wok[q]) ? ld16(wrow[q] + cc * CH) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < BMB; ++b)
#pragma unroll
        for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[b][q], wf[u][q], zf[u][b]);
  }

  // fixed-order reduction of the four waves' partial sums
#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) red[wave][b * RB + q][lane] = acc[b][q];
  __syncthreads();
  uint4 hf[BMB][RB];
#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int i = b * RB + q;
      f32x4_t s = red[0][i][lane];
      s += red[1][i][lane];
      s += red[2][i][lane];
      s += red[3][i][lane];
      s *= p.scale;
      acc[b][q] = s;
      hf[b][q] = split_frag<Tag>(s);
    }

  // ---- optional: write s*H transposed (rank-major, token-contiguous)
  if constexpr (EMIT) {
    if (wave == 0) {
#pragma unroll
      for (int b = 0; b < BMB; ++b) {
        const int64_t m = m0 + 16 * b + col;
        if (m < p.M) {
#pragma unroll
          for (int q = 0; q < RB; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int64_t j = 16 * q + 4 * grp + i;
              if constexpr (sizeof(E) == 2) {
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
  }

  // ---- phase 2: out^T tile (16 columns x 16 tokens) (+)= W2 * (s*H)^T
  if constexpr (EXPAND) {
    const E* w2 = static_cast<const E*>(p.w2);
    const int64_t nnb = (p.Nout + 15) / 16;
    for (int64_t nb0 = (int64_t)wave * NBU; nb0 < nnb; nb0 += 4 * NBU) {
      uint4 wv[NBU][RB];
      f32x4_t cv[NBU][BMB];
#pragma unroll
      for (int u = 0; u < NBU; ++u) {
        const int64_t nb = nb0 + u;
        const int64_t nrow = nb * 16 + col;
        const bool nok = nb < nnb && nrow < p.Nout;
        const E* wr = w2 + (nok ? nrow : 0) * p.ldw2;
#pragma unroll
        for (int q = 0; q < RB; ++q) wv[u][q] = nok ? load_wvec4<Tag>(wr, 16 * q + 4 * grp, p.r) : zero4();
        const int64_t ncol = nb * 16 + 4 * grp;
#pragma unroll
        for (int b = 0; b < BMB; ++b) {
          const int64_t m = m0 + 16 * b + col;
          const bool ok = nb < nnb && ncol < p.Nout && m < p.M;
          if (ACCUM && ok)
            cv[u][b] = ld16f(p.out + m * p.ldo + ncol);
          else
            cv[u][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < NBU; ++u) {
        const int64_t nb = nb0 + u;
        const int64_t ncol = nb * 16 + 4 * grp;
#pragma unroll
        for (int b = 0; b < BMB; ++b) {
#pragma unroll
          for (int q = 0; q < RB; ++q) mma_rank16<Tag>(cv[u][b], wv[u][q], hf[b][q]);
          const int64_t m = m0 + 16 * b + col;
          if (nb < nnb && ncol < p.Nout && m < p.M) st16f(p.out + m * p.ldo + ncol, cv[u][b]);
        }
      }
    }
  }
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
  int64_t chunk;   // tokens per chunk, a multiple of 32
};

template <class Tag, int RB>
__global__ __launch_bounds__(256) void tn_kernel(TnArgs p) {
  using E = typename Tag::elem;
  constexpr int VEC = Tag::VEC;
  constexpr int ES = sizeof(E);
  constexpr int NSB = 4;              // 16-column blocks per wave
  constexpr int NS = 64 * NSB;        // columns per workgroup
  constexpr int TS = 32;              // tokens per stage
  constexpr int ROWB = NS * ES;       // LDS bytes per staged Z row
  constexpr int VPR = NS / VEC;       // 128-bit vectors per Z row
  constexpr int ZV = TS * VPR / 256;  // Z vectors per thread per stage
  constexpr int GPL = (ES == 2) ? 2 : 1;  // G planes (bf16 hi/lo)
  constexpr int GROWB = TS * ES;          // LDS bytes per G row and plane
  constexpr int GVR = TS / VEC;           // vectors per G row
  constexpr int GTOT = GPL * 16 * RB * GVR;
  constexpr int GV = (GTOT + 255) / 256;
  // rows 8 (bf16) or 4 (f32) apart are read together by the four lane groups:
  // XOR their 32/64-byte column windows apart to avoid LDS bank conflicts.
  constexpr int SWZ_SHIFT = (ES == 2) ? 3 : 2;
  constexpr int SWZ_UNIT = (ES == 2) ? 32 : 64;

  __shared__ __attribute__((aligned(16))) char zt[TS * ROWB];
  __shared__ __attribute__((aligned(16))) char gs[GPL * 16 * RB * GROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t n_base = (int64_t)blockIdx.x * NS;
  const int64_t m_begin = (int64_t)blockIdx.y * p.chunk;
  const int64_t m_end = (m_begin + p.chunk < p.M) ? (m_begin + p.chunk) : p.M;
  const E* z = static_cast<const E*>(p.z);
  const E* g = static_cast<const E*>(p.g);

  f32x4_t acc[NSB][RB];
#pragma unroll
  for (int nb = 0; nb < NSB; ++nb)
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[nb][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 zr[ZV];
  uint4 gr[GV];

  auto load_stage = [&](int64_t m0) {
#pragma unroll
    for (int i = 0; i < ZV; ++i) {
      const int v = tid + 256 * i;
      const int row = v / VPR;
      const int vc = v - row * VPR;
      const int64_t m = m0 + row;
      const int64_t n = n_base + (int64_t)vc * VEC;
      zr[i] = (m < m_end && n < p.N) ? ld16(z + m * p.ldz + n) : zero4();
    }
#pragma unroll
    for (int i = 0; i < GV; ++i) {
      const int v = tid + 256 * i;
      uint4 val = zero4();
      if (v < GTOT) {
        const int grow = v / GVR;  // plane * 16*RB + j
        const int vc = v - grow * GVR;
        const int64_t m = m0 + (int64_t)vc * VEC;
        const E* src = g + (int64_t)grow * p.ldg + m;
        if (m + VEC <= m_end) {
          val = ld16(src);
        } else if (m < m_end) {
          union {
            E e[VEC];
            uint4 v;
          } tmp;
#pragma unroll
          for (int e = 0; e < VEC; ++e) tmp.e[e] = (m + e < m_end) ? src[e] : E(0);
          val = tmp.v;
        }
      }
      gr[i] = val;
    }
  };

  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < ZV; ++i) {
      const int v = tid + 256 * i;
      const int row = v / VPR;
      const int vc = v - row * VPR;
      const int off = row * ROWB + ((vc * 16) ^ (((row >> SWZ_SHIFT) & 3) * SWZ_UNIT));
      *reinterpret_cast<uint4*>(zt + off) = zr[i];
    }
#pragma unroll
    for (int i = 0; i < GV; ++i) {
      const int v = tid + 256 * i;
      if (v < GTOT) *reinterpret_cast<uint4*>(gs + v * 16) = gr[i];
    }
  };

  auto zval = [&](int m, int nl) -> uint32_t {
    const int off = m * ROWB + ((nl * ES) ^ (((m >> SWZ_SHIFT) & 3) * SWZ_UNIT));
    if constexpr (ES == 2)
      return *reinterpret_cast<const uint16_t*>(zt + off);
    else
      return *reinterpret_cast<const uint32_t*>(zt + off);
  };

  const int64_t nstage = (m_end - m_begin + TS - 1) / TS;
  if (nstage > 0) load_stage(m_begin);
  for (int64_t s = 0; s < nstage; ++s) {
    __syncthreads();
    store_stage();
    __syncthreads();
    if (s + 1 < nstage) load_stage(m_begin + (s + 1) * TS);

    if constexpr (ES == 2) {
      uint4 ghi[RB], glo[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        ghi[q] = *reinterpret_cast<const uint4*>(gs + (16 * q + col) * GROWB + grp * 16);
        glo[q] = *reinterpret_cast<const uint4*>(gs + (16 * RB + 16 * q + col) * GROWB + grp * 16);
      }
#pragma unroll
      for (int nb = 0; nb < NSB; ++nb) {
        const int nl = (wave * NSB + nb) * 16 + col;
        uint32_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = zval(8 * grp + e, nl);
        const uint4 zf = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          mma_vec<Tag>(acc[nb][q], zf, ghi[q]);
          mma_vec<Tag>(acc[nb][q], zf, glo[q]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint4 gf[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q)
          gf[q] = *reinterpret_cast<const uint4*>(gs + (16 * q + col) * GROWB + (u * 16 + 4 * grp) * 4);
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
  }

  float* part = p.part + (int64_t)blockIdx.y * p.N * p.rp;
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

// ---------------------------------------------------------------------------
// host-side launch helpers
// ---------------------------------------------------------------------------

constexpr int kTnCols = 256;  // columns per tn_kernel workgroup

// Fused-kernel token tile: the largest of 4/2/1 token blocks that still gives
// >= 512 workgroups (two per CU), with at most 16 (block x rank-block) tiles.
static int pick_bmb(int64_t M, int rb) {
  int bmb = env_int("LORA_FUSED_BMB", 0);
  if (bmb == 1 || bmb == 2 || bmb == 4) {
    if (bmb * rb <= 16) return bmb;
  }
  for (int c : {4, 2}) {
    if (c * rb <= 16 && ceil_div(M, 16 * c) >= 512) return c;
  }
  return 1;
}

static int64_t tn_chunks_max(int64_t M, int64_t N) {
  const int64_t slices = ceil_div(N, kTnCols);
  int64_t P = ceil_div(512, slices);
  const int64_t cap = ceil_div(M, 32);
  if (P > cap) P = cap;
  return P < 1 ? 1 : P;
}

static int64_t tn_chunk_tokens(int64_t M, int64_t N) {
  int64_t P = tn_chunks_max(M, N);
  const int64_t over = env_int("LORA_TN_CHUNKS", 0);
  if (over >= 1 && over < P) P = over;
  return round_up(ceil_div(M, P), 32);
}

template <class Tag, int RB, int BMB, bool EXPAND, bool ACCUM, bool EMIT>
static void launch_fused_t(const FusedArgs& a, hipStream_t st) {
  constexpr int NBU0 = 8 / BMB;
  constexpr int NBU1 = 16 / RB;
  constexpr int NBU = (NBU0 < NBU1 ? NBU0 : NBU1) > 0 ? (NBU0 < NBU1 ? NBU0 : NBU1) : 1;
  const dim3 grid(static_cast<unsigned>(ceil_div(a.M, 16 * BMB)));
  hipLaunchKernelGGL((fused_kernel<Tag, RB, BMB, NBU, EXPAND, ACCUM, EMIT>), grid, dim3(256), 0, st, a);
}

template <class Tag, bool EXPAND, bool ACCUM, bool EMIT>
static void launch_fused(const FusedArgs& a, int rb, int bmb, hipStream_t st) {
  switch (rb * 10 + bmb) {
    case 11: launch_fused_t<Tag, 1, 1, EXPAND, ACCUM, EMIT>(a, st); break;
    case 12: launch_fused_t<Tag, 1, 2, EXPAND, ACCUM, EMIT>(a, st); break;
    case 14: launch_fused_t<Tag, 1, 4, EXPAND, ACCUM, EMIT>(a, st); break;
    case 21: launch_fused_t<Tag, 2, 1, EXPAND, ACCUM, EMIT>(a, st); break;
    case 22: launch_fused_t<Tag, 2, 2, EXPAND, ACCUM, EMIT>(a, st); break;
    case 24: launch_fused_t<Tag, 2, 4, EXPAND, ACCUM, EMIT>(a, st); break;
    case 41: launch_fused_t<Tag, 4, 1, EXPAND, ACCUM, EMIT>(a, st); break;
    case 42: launch_fused_t<Tag, 4, 2, EXPAND, ACCUM, EMIT>(a, st); break;
    case 44: launch_fused_t<Tag, 4, 4, EXPAND, ACCUM, EMIT>(a, st); break;
    case 81: launch_fused_t<Tag, 8, 1, EXPAND, ACCUM, EMIT>(a, st); break;
    default: launch_fused_t<Tag, 8, 2, EXPAND, ACCUM, EMIT>(a, st); break;
  }
}

template <class Tag>
static void launch_tn(const TnArgs& a, int rb, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(ceil_div(a.N, kTnCols)), static_cast<unsigned>(ceil_div(a.M, a.chunk)));
  switch (rb) {
    case 1: hipLaunchKernelGGL((tn_kernel<Tag, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((tn_kernel<Tag, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((tn_kernel<Tag, 4>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((tn_kernel<Tag, 8>), grid, dim3(256), 0, st, a); break;
  }
}

static void launch_pack(int32_t dtype, const void* src, int64_t s_i, int64_t s_j, int64_t rows, int64_t cols,
                        void* dst, int64_t dst_rows, int64_t dst_cols, int64_t ld, hipStream_t st) {
  const int64_t total = dst_rows * dst_cols;
  if (total <= 0) return;
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 8192) blocks = 8192;
  if (dtype == LORA_BF16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(src), s_i, s_j, rows, cols, static_cast<uint16_t*>(dst), dst_rows,
                       dst_cols, ld);
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                       static_cast<const float*>(src), s_i, s_j, rows, cols, static_cast<float*>(dst), dst_rows,
                       dst_cols, ld);
}

static void launch_fill_zero(const lora_mat* m, hipStream_t st) {
  const int64_t total = m->rows * m->cols;
  if (total <= 0) return;
  int64_t blocks = ceil_div(total, 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<float*>(m->ptr), m->rows, m->cols, m->stride_row, m->stride_col);
}

static void launch_reduce(const float* part, int P, int64_t N, int rp, int r, float* out, int64_t os_n, int64_t os_j,
                          hipStream_t st) {
  const int64_t total = N * r;
  if (total <= 0) return;
  hipLaunchKernelGGL(reduce_kernel, dim3(static_cast<unsigned>(ceil_div(total, 256))), dim3(256), 0, st, part, P, N,
                     rp, r, out, os_n, os_j);
}

// Workspace pieces of each operation (the same function sizes and carves).
struct SingleLayout {
  size_t w1 = 0, w2 = 0, g = 0, part = 0;
  int64_t ldg = 0, chunk = 0, P = 0;
  size_t total() const {
    return static_cast<size_t>(round_up(w1, 256) + round_up(w2, 256) + round_up(g, 256) + round_up(part, 256));
  }
};

static SingleLayout layout_for(int op, int64_t M, int64_t K, int64_t L, int r, int32_t dtype) {
  SingleLayout s;
  const size_t es = elem_size(dtype);
  const int64_t rp = padded_rank(r);
  if (op == LORA_OP_FWD) {
    s.w1 = static_cast<size_t>(rp * K) * es;  // A as r x K
    s.w2 = static_cast<size_t>(L * rp) * es;  // B as L x r
  } else if (op == LORA_OP_BWD_DX_DA) {
    s.w1 = static_cast<size_t>(rp * L) * es;  // B as r x L
    s.w2 = static_cast<size_t>(K * rp) * es;  // A as K x r
    s.ldg = round_up(M > 0 ? M : 1, 32);
    s.g = static_cast<size_t>(4 * rp * s.ldg);
    s.P = tn_chunks_max(M, K);
    s.part = static_cast<size_t>(s.P * K * rp) * 4;
  } else {
    s.w1 = static_cast<size_t>(rp * K) * es;  // A as r x K
    s.ldg = round_up(M > 0 ? M : 1, 32);
    s.g = static_cast<size_t>(4 * rp * s.ldg);
    s.P = tn_chunks_max(M, L);
    s.part = static_cast<size_t>(s.P * L * rp) * 4;
  }
  return s;
}

}  // namespace lora

using namespace lora;

extern "C" int lora_abi_version(void) { return LORA_ABI_VERSION; }

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
  return layout_for(op, M, K, L, r, dtype).total();
}

extern "C" int lora_fwd(const lora_mat* x, const lora_mat* lora_A, const lora_mat* lora_B, const lora_mat* res,
                        float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !lora_A || !lora_B || !res) return LORA_ERR_NULL;
  if (!valid_dims(x) || !valid_dims(lora_A) || !valid_dims(lora_B) || !valid_dims(res)) return LORA_ERR_SHAPE;
  const int64_t M = x->rows, K = x->cols, r = lora_A->cols, L = lora_B->cols;
  if (lora_A->rows != K || lora_B->rows != r || res->rows != M || res->cols != L) return LORA_ERR_SHAPE;
  if (!float_dtype_ok(x->dtype) || lora_A->dtype != x->dtype || lora_B->dtype != x->dtype || res->dtype != LORA_F32)
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
  // B is read in place when it is a view of an L x r weight with r contiguous.
  const bool b_direct = lora_B->stride_row == 1 && lora_B->stride_col % 4 == 0 && aligned(lora_B->ptr, 4 * es);
  const SingleLayout lay = layout_for(LORA_OP_FWD, M, K, L, static_cast<int>(r), x->dtype);
  Carver cv(workspace);
  void* w1p = cv.take(lay.w1);
  void* w2p = cv.take(lay.w2);
  if (!a_direct || !b_direct) {
    if (!workspace) return LORA_ERR_WORKSPACE;
    if (workspace_bytes < cv.used) return LORA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return LORA_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  FusedArgs a{};
  a.z = x->ptr;
  a.ldz = x->stride_row;
  if (a_direct) {
    a.w1 = lora_A->ptr;
    a.ldw1 = lora_A->stride_col;
  } else {
    launch_pack(x->dtype, lora_A->ptr, lora_A->stride_col, lora_A->stride_row, r, K, w1p, rp, K, K, st);
    a.w1 = w1p;
    a.ldw1 = K;
  }
  if (b_direct) {
    a.w2 = lora_B->ptr;
    a.ldw2 = lora_B->stride_col;
  } else {
    launch_pack(x->dtype, lora_B->ptr, lora_B->stride_col, lora_B->stride_row, L, r, w2p, L, rp, rp, st);
    a.w2 = w2p;
    a.ldw2 = rp;
  }
  a.out = static_cast<float*>(res->ptr);
  a.ldo = res->stride_row;
  a.M = M;
  a.Kin = K;
  a.Nout = L;
  a.r = static_cast<int>(r);
  a.rp = static_cast<int>(rp);
  a.scale = scale;
  const int bmb = pick_bmb(M, rb);
  if (x->dtype == LORA_BF16)
    launch_fused<BF16, true, true, false>(a, rb, bmb, st);
  else
    launch_fused<F32, true, true, false>(a, rb, bmb, st);
  return launch_status();
}

extern "C" int lora_bwd_dx_da(const lora_mat* xt, const lora_mat* dy, const lora_mat* lora_B, const lora_mat* lora_A,
                              float scale, const lora_mat* dx, const lora_mat* dA, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!xt || !dy || !lora_B || !lora_A || !dx || !dA) return LORA_ERR_NULL;
  if (!valid_dims(xt) || !valid_dims(dy) || !valid_dims(lora_B) || !valid_dims(lora_A) || !valid_dims(dx) ||
      !valid_dims(dA))
    return LORA_ERR_SHAPE;
  const int64_t K = xt->rows, M = xt->cols, L = dy->cols, r = lora_B->cols;
  if (dy->rows != M || lora_B->rows != L || lora_A->rows != r || lora_A->cols != K || dx->rows != M ||
      dx->cols != K || dA->rows != K || dA->cols != r)
    return LORA_ERR_SHAPE;
  if (!float_dtype_ok(xt->dtype) || dy->dtype != xt->dtype || lora_B->dtype != xt->dtype ||
      lora_A->dtype != xt->dtype || dx->dtype != LORA_F32 || dA->dtype != LORA_F32)
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
    launch_fill_zero(dx, st);
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

  const int rb = rank_blocks(static_cast<int>(r));
  const int64_t rp = 16 * rb;
  // W1 = B^T (r x L, L contiguous); W2 = A^T (K x r, r contiguous).
  launch_pack(xt->dtype, lora_B->ptr, lora_B->stride_col, lora_B->stride_row, r, L, w1p, rp, L, L, st);
  launch_pack(xt->dtype, lora_A->ptr, lora_A->stride_col, lora_A->stride_row, K, r, w2p, K, rp, rp, st);

  FusedArgs a{};
  a.z = dy->ptr;
  a.ldz = dy->stride_row;
  a.w1 = w1p;
  a.ldw1 = L;
  a.w2 = w2p;
  a.ldw2 = rp;
  a.out = static_cast<float*>(dx->ptr);
  a.ldo = dx->stride_row;
  a.g = gbuf;
  a.ldg = lay.ldg;
  a.M = M;
  a.Kin = L;
  a.Nout = K;
  a.r = static_cast<int>(r);
  a.rp = static_cast<int>(rp);
  a.scale = scale;
  const int bmb = pick_bmb(M, rb);
  TnArgs t{};
  t.z = xt->ptr;
  t.ldz = xt->stride_col;
  t.g = gbuf;
  t.ldg = lay.ldg;
  t.part = part;
  t.M = M;
  t.N = K;
  t.rp = static_cast<int>(rp);
  t.chunk = tn_chunk_tokens(M, K);
  const int P = static_cast<int>(ceil_div(M, t.chunk));
  if (xt->dtype == LORA_BF16) {
    launch_fused<BF16, true, false, true>(a, rb, bmb, st);
    launch_tn<BF16>(t, rb, st);
  } else {
    launch_fused<F32, true, false, true>(a, rb, bmb, st);
    launch_tn<F32>(t, rb, st);
  }
  launch_reduce(part, P, K, static_cast<int>(rp), static_cast<int>(r), static_cast<float*>(dA->ptr), dA->stride_row,
                dA->stride_col, st);
  return launch_status();
}

extern "C" int lora_bwd_db(const lora_mat* lora_A, const lora_mat* xt, const lora_mat* dy, float scale,
                           const lora_mat* dB, void* workspace, size_t workspace_bytes, void* stream) {
  if (!lora_A || !xt || !dy || !dB) return LORA_ERR_NULL;
  if (!valid_dims(lora_A) || !valid_dims(xt) || !valid_dims(dy) || !valid_dims(dB)) return LORA_ERR_SHAPE;
  const int64_t r = lora_A->rows, K = lora_A->cols, M = xt->cols, L = dy->cols;
  if (xt->rows != K || dy->rows != M || dB->rows != r || dB->cols != L) return LORA_ERR_SHAPE;
  if (!float_dtype_ok(lora_A->dtype) || xt->dtype != lora_A->dtype || dy->dtype != lora_A->dtype ||
      dB->dtype != LORA_F32)
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
  if (a_direct) {
    a.w1 = lora_A->ptr;
    a.ldw1 = lora_A->stride_row;
  } else {
    launch_pack(xt->dtype, lora_A->ptr, lora_A->stride_row, lora_A->stride_col, r, K, w1p, rp, K, K, st);
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
  const int bmb = pick_bmb(M, rb);
  TnArgs t{};
  t.z = dy->ptr;
  t.ldz = dy->stride_row;
  t.g = gbuf;
  t.ldg = lay.ldg;
  t.part = part;
  t.M = M;
  t.N = L;
  t.rp = static_cast<int>(rp);
  t.chunk = tn_chunk_tokens(M, L);
  const int P = static_cast<int>(ceil_div(M, t.chunk));
  if (xt->dtype == LORA_BF16) {
    launch_fused<BF16, false, false, true>(a, rb, bmb, st);
    launch_tn<BF16>(t, rb, st);
  } else {
    launch_fused<F32, false, false, true>(a, rb, bmb, st);
    launch_tn<F32>(t, rb, st);
  }
  // dB is r x L: partial row n = l, column j.
  launch_reduce(part, P, L, static_cast<int>(rp), static_cast<int>(r), static_cast<float*>(dB->ptr), dB->stride_col,
                dB->stride_row, st);
  return launch_status();
}
