// Slot-addressed multi-adapter LoRA ops on gfx950 (API page
// "mstar.engine.resources.lora.ops", class LoraOpsBackend):
//   shrink:        h[t] = x[t] @ a[slot(t)]^T          (per output slice)
//   expand_fused:  y[t, slice i] += sc[slot(t)] * h[t, slice i] @ b[slot(t), slice i]^T
//   gather_shrink: h[t] = a[slot(t)][:, ids[t]]        (one column of the slot's adapter)
// plus the token-to-slot grouping that every op reads. The page's ops never
// wait on the host and never size anything from device data: grids are sized
// from host-known bounds (T, S, slice widths) and each workgroup finds its
// work on the device, exiting early when there is none.
//
// Work decomposition: the active tokens of a slot, in grouped order, are cut
// into tiles of TB tokens; tile k of the batch is found from counts[] with a
// wave-level scan (the row-split shrink and the pipelined shrink below 512
// tokens scan counts[] and ranks[] for live units instead, and deal them to
// the XCDs in equal runs). Every tile touches one slot's adapter only, so its
// rows are shared by all tokens of the tile.
//
// Kernels:
//   group_kernel               stable counting sort (one 1024-thread workgroup)
//   group_small_kernel         the same for up to 1024 tokens, one per thread
//   group_chunk_kernel         the same with one workgroup per 1024-token chunk
//   slot_shrink_kernel         shrink, one workgroup per (tile, slice, rank chunk)
//   slot_shrink_pipe_kernel    the same with contiguous per-wave feature ranges,
//                              descriptor loads and two register stages
//   slot_shrink_rows_kernel    shrink for many tokens: a 128-token tile x up to
//                              128 adapter rows per 8-wave workgroup, x staged
//                              once in LDS, one 16-row rank block per wave
//   slot_expand_band_kernel    expand for 512 tokens or more: a token piece x
//                              256-column band per workgroup, weights in
//                              registers, h fragments shared through LDS,
//                              1 KB row segments of y
//   slot_expand_stream_kernel  expand for fewer tokens: tile x column chunk,
//                              weights from L2, two stages of outputs in flight
//   slot_expand_kernel         expand for any layout (unaligned rows, y or b
//                              beyond 2 GiB)
//   slot_apply_kernel          apply_linear in one launch (h kept on chip)
// Every expand forms the update of an output element as an MFMA chain over
// its rank blocks starting from zero and then adds it to y, so all of them
// (and both forms of apply_linear) give the same bits.
//   gather_kernel              exact column gather, one wave per token

#include <mutex>
#include <type_traits>

#include "lora_device.hpp"
#include "lora_host.hpp"

namespace lora {

constexpr int kMaxSlots = 1024;
constexpr int kMaxSlices = 16;

// Device-resident rank intermediate of lora_apply_linear_noalloc: every GPU
// the library runs on holds its own copy (allocated with the code object when
// it loads on that device, kept until the process ends). Host code never uses
// the array's name as an address: its device address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
constexpr int64_t kScratchBytes = int64_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

__device__ __forceinline__ int clamp_rank(int v, int r_max) { return v < 0 ? 0 : (v > r_max ? r_max : v); }

// ---------------------------------------------------------------------------
// grouping: stable counting sort of the active tokens by slot (one workgroup)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void group_kernel(const int32_t* __restrict__ token_slot, int T, int S,
                                                     const int32_t* __restrict__ ranks, int r_max,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_tokens) {
  __shared__ int rho[kMaxSlots];
  __shared__ int cnt[kMaxSlots + 1];
  __shared__ int base[kMaxSlots + 1];
  __shared__ int wcnt[16][kMaxSlots + 1];  // per-wave count of each key in the current chunk
  __shared__ int wsum[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid < S) rho[tid] = clamp_rank(ranks[tid], r_max);
  for (int i = tid; i <= S; i += 1024) {
    cnt[i] = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) wcnt[w][i] = 0;
  }
  __syncthreads();

  // histogram (integer LDS atomics: the counts do not depend on their order)
  for (int t = tid; t < T; t += 1024) {
    const int s = token_slot[t];
    if (s >= 0 && s < S && rho[s] > 0) atomicAdd(&cnt[s], 1);
  }
  __syncthreads();

  // exclusive scan of the counts (S <= 1024: one value per thread)
  const int c = (tid < S) ? cnt[tid] : 0;
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int excl = before + incl - c;
  if (tid < S) {
    counts[tid] = c;
    offsets[tid] = excl;
    base[tid] = excl;
  }
  if (tid == S - 1) offsets[S] = excl + c;
  if (S == 0 && tid == 0) offsets[0] = 0;
  __syncthreads();

  // stable scatter in chunks of 1024 tokens, token order preserved within a slot
  int nbits = 0;
  while ((1 << nbits) <= S) ++nbits;  // keys 0..S (S = inactive)
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int t = t0 + tid;
    int key = S;
    if (t < T) {
      const int s = token_slot[t];
      if (s >= 0 && s < S && rho[s] > 0) key = s;
    }
    uint64_t peers = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (key >> bit) & 1;
      const uint64_t bal = __ballot(on);
      peers &= on ? bal : ~bal;
    }
    const int rank_in_wave = __popcll(peers & lt_mask);
    const bool leader = (peers & lt_mask) == 0;
    if (leader) wcnt[wave][key] = __popcll(peers);
    __syncthreads();
    if (key < S) {
      int pos = base[key] + rank_in_wave;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][key];
      sorted_tokens[pos] = t;
    }
    __syncthreads();
    if (tid < S) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) add += wcnt[w][tid];
      base[tid] += add;
    }
    __syncthreads();
    if (leader) wcnt[wave][key] = 0;
    __syncthreads();
  }
}

// Key of token t: its slot if active, else S (inactive).
__device__ __forceinline__ int group_key(const int32_t* __restrict__ token_slot, const int* rho, int t, int T, int S) {
  int key = S;
  if (t < T) {
    const int s = token_slot[t];
    if (s >= 0 && s < S && rho[s] > 0) key = s;
  }
  return key;
}

// Lanes of the wave that hold the same key as this lane (bit l = lane l),
// from one ballot per key bit; a single ballot when the whole wave holds one
// key (the usual case for tokens of one request). Needs all 64 lanes active.
__device__ __forceinline__ uint64_t key_peers(int key, int nbits) {
  const int k0 = __builtin_amdgcn_readfirstlane(key);
  if (__ballot(key == k0) == ~0ull) return ~0ull;
  uint64_t peers = ~0ull;
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = (key >> bit) & 1;
    const uint64_t bal = __ballot(on);
    peers &= on ? bal : ~bal;
  }
  return peers;
}

// The same stable counting sort with one workgroup per chunk of 1024 tokens
// (for T up to kGroupChunkMaxT). Every workgroup counts all T tokens itself:
// the total per slot gives the offsets (workgroup 0 writes counts and
// offsets), the count over the chunks before its own gives where its tokens
// of each slot start. It then places its chunk's tokens as group_kernel does.
// Counting uses one LDS atomic per distinct key of each wave.
constexpr int kGroupKeys = 32;  // token chunks (of 1024) the chunked grouping holds in registers
constexpr int kGroupChunkMaxT = 1024 * kGroupKeys;
__global__ __launch_bounds__(1024) void group_chunk_kernel(const int32_t* __restrict__ token_slot, int T, int S,
                                                           const int32_t* __restrict__ ranks, int r_max,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_tokens) {
  __shared__ int rho[kMaxSlots];
  __shared__ int cnt[kMaxSlots + 1];   // all tokens
  __shared__ int pre[kMaxSlots + 1];   // tokens of the chunks before this one
  __shared__ int base[kMaxSlots + 1];
  __shared__ int wcnt[16][kMaxSlots + 1];
  __shared__ int wsum[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c0 = static_cast<int>(blockIdx.x) * 1024;
  if (tid < S) rho[tid] = clamp_rank(ranks[tid], r_max);
  for (int i = tid; i <= S; i += 1024) {
    cnt[i] = 0;
    pre[i] = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) wcnt[w][i] = 0;
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) <= S) ++nbits;  // keys 0..S (S = inactive)
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // Histograms in per-wave rows of wcnt (the lane that leads a key in its
  // wave adds the key's count: no two lanes write one entry, no atomics).
  // All kGroupKeys token chunks are loaded into registers at once; chunk j
  // takes part while j*1024 < T (uniform, so every lane joins the ballots).
  int keys[kGroupKeys];
#pragma unroll
  for (int j = 0; j < kGroupKeys; ++j) {
    const int t = j * 1024 + tid;
    keys[j] = (t < T) ? token_slot[t] : -1;
  }
  const int nchunk = (T + 1023) / 1024;
  auto count_range = [&](int ja, int jb) {
#pragma unroll
    for (int j = 0; j < kGroupKeys; ++j) {
      if (j >= ja && j < jb) {
        const int sj = keys[j];
        const int k = (sj >= 0 && sj < S && rho[sj] > 0) ? sj : S;
        const uint64_t peers = key_peers(k, nbits);
        if ((peers & lt_mask) == 0 && k < S) wcnt[wave][k] += __popcll(peers);
      }
    }
  };
  auto sum_rows = [&](int* out) {
    for (int i = tid; i < S; i += 1024) {
      int v = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) v += wcnt[w][i];
      out[i] = v;
    }
  };
  const int bx = static_cast<int>(blockIdx.x);
  count_range(0, bx);  // the chunks before this one
  __syncthreads();
  sum_rows(pre);
  __syncthreads();
  count_range(bx, nchunk);  // the rest: the rows now hold every token
  __syncthreads();
  sum_rows(cnt);
  __syncthreads();
  for (int i = tid; i <= S; i += 1024) {
#pragma unroll
    for (int w = 0; w < 16; ++w) wcnt[w][i] = 0;
  }
  __syncthreads();

  // exclusive scan of the totals (S <= 1024: one value per thread)
  const int c = (tid < S) ? cnt[tid] : 0;
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int excl = before + incl - c;
  if (tid < S) base[tid] = excl + pre[tid];
  if (blockIdx.x == 0) {
    if (tid < S) {
      counts[tid] = c;
      offsets[tid] = excl;
    }
    if (tid == S - 1) offsets[S] = excl + c;
    if (S == 0 && tid == 0) offsets[0] = 0;
  }
  __syncthreads();

  // stable placement of this chunk's tokens
  const int t = c0 + tid;
  const int key = group_key(token_slot, rho, t, T, S);
  const uint64_t peers = key_peers(key, nbits);
  const int rank_in_wave = __popcll(peers & lt_mask);
  if ((peers & lt_mask) == 0) wcnt[wave][key] = __popcll(peers);
  __syncthreads();
  if (key < S) {
    int pos = base[key] + rank_in_wave;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][key];
    sorted_tokens[pos] = t;
  }
}

// The same stable counting sort for T <= 1024 (a decode batch): one token
// per thread of one workgroup. The tokens' slots and the ranks are loaded
// together; one ballot pass gives each wave's count of every key and each
// token's rank among the lanes of its wave with the same key before it; the
// per-key totals are scanned (one key per thread); a token then lands at its
// slot's offset plus the same-key tokens of earlier waves plus its rank in
// its wave. Four barriers and one round of global loads, where the chunked
// kernel's multi-chunk bookkeeping takes eight and three (GPU time per call:
// 256 tokens 6.7 -> 3.1 us, 1024 tokens 7.3 -> 3.6 us).
constexpr int kGroupSmallMaxT = 1024;
__global__ __launch_bounds__(1024) void group_small_kernel(const int32_t* __restrict__ token_slot, int T, int S,
                                                           const int32_t* __restrict__ ranks, int r_max,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_tokens) {
  __shared__ int rho[kMaxSlots];
  __shared__ int base[kMaxSlots + 1];
  __shared__ int wcnt[16][kMaxSlots + 1];  // per-wave count of each key
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slot = tid < T ? token_slot[tid] : -1;
  const int rk = tid < S ? ranks[tid] : 0;
  if (tid < S) rho[tid] = clamp_rank(rk, r_max);
  for (int i = tid; i <= S; i += 1024) {
#pragma unroll
    for (int w = 0; w < 16; ++w) wcnt[w][i] = 0;
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) <= S) ++nbits;  // keys 0..S (S = inactive)
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int key = (slot >= 0 && slot < S && rho[slot] > 0) ? slot : S;
  const uint64_t peers = key_peers(key, nbits);
  const int rank_in_wave = __popcll(peers & lt_mask);
  if ((peers & lt_mask) == 0) wcnt[wave][key] = __popcll(peers);
  __syncthreads();
  // per-key totals and their exclusive scan (S <= 1024: one key per thread)
  int c = 0;
  if (tid < S) {
#pragma unroll
    for (int w = 0; w < 16; ++w) c += wcnt[w][tid];
  }
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int excl = before + incl - c;
  if (tid < S) {
    counts[tid] = c;
    offsets[tid] = excl;
    base[tid] = excl;
  }
  if (tid == S - 1) offsets[S] = excl + c;
  if (S == 0 && tid == 0) offsets[0] = 0;
  __syncthreads();
  if (key < S) {
    int pos = base[key] + rank_in_wave;
    for (int w = 0; w < wave; ++w) pos += wcnt[w][key];
    sorted_tokens[pos] = tid;
  }
}

// ---------------------------------------------------------------------------
// tile lookup: tile `ti` of the batch -> (slot, first grouped index, length)
// ---------------------------------------------------------------------------

struct Tile {
  int slot;  // -1: no such tile
  int start;
  int len;
};

// Called by one full wave; every lane returns the same tile.
__device__ Tile find_tile(int ti, int tb, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
                          int S) {
  const int lane = threadIdx.x & 63;
  int running = 0;
  Tile out{-1, 0, 0};
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    const int c = (s < S) ? counts[s] : 0;
    const int nt = c > 0 ? (c - 1) / tb + 1 : 0;  // no overflow for counts near 2^31
    int incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = running + incl - nt;
    const bool mine = ti >= excl && ti < excl + nt;
    const uint64_t who = __ballot(mine);
    if (who) {
      const int src = __ffsll(static_cast<long long>(who)) - 1;
      const int k = ti - __shfl(excl, src, 64);
      const int cs = __shfl(c, src, 64);
      out.slot = s0 + src;
      out.start = __shfl(s < S ? offsets[s] : 0, src, 64) + k * tb;
      out.len = (cs - k * tb) < tb ? (cs - k * tb) : tb;
      return out;
    }
    running += __shfl(incl, 63, 64);
    if (running > ti) break;
  }
  return out;
}

// ---------------------------------------------------------------------------
// shrink: h[t, i, j] = sum_k x[t, k] * a[s, i*r_max + j, k], j < rank(s)
// ---------------------------------------------------------------------------

struct ShrinkArgs {
  const void* x;
  int64_t ldx;
  const void* a;
  int64_t as0, as1;  // slot and row strides (elements); k is contiguous
  float* h;
  int64_t hs0, hs1;  // token and slice strides; j contiguous
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted;
  const int32_t* ranks;
  int64_t K;
  int S, r_max, n_slices, row_chunks;
  int row_groups;   // row-split kernel: workgroups per token tile (NW * PPW rank-block pairs each)
  int64_t x_bytes;  // bytes of x a descriptor may span (GEMM kernel)
  bool h_vec;  // h rows 16-byte aligned (strides multiples of 4)
};

// Pipelined-shrink units: a slot with c grouped tokens and clamped rank rho
// has ceil(c / tb) tiles x n_slices slices x ceil(rho / rows) rank chunks;
// units run in slot order, then tile, slice, chunk. Wave-level: the unit
// count in *total, and the u-th unit (u < 0: count only).
struct PipeUnit {
  int slot;  // -1: no such unit
  int start, len, slice, chunk;
};

__device__ PipeUnit find_pipe_unit(int u, int tb, int rows, const ShrinkArgs& p, int* total) {
  const int lane = threadIdx.x & 63;
  int running = 0;
  PipeUnit out{-1, 0, 0, 0, 0};
  for (int s0 = 0; s0 < p.S; s0 += 64) {
    const int s = s0 + lane;
    const int c = (s < p.S) ? p.counts[s] : 0;
    const int rho = (s < p.S) ? clamp_rank(p.ranks[s], p.r_max) : 0;
    const int nch = (rho + rows - 1) / rows;
    const int nt = (c > 0 && rho > 0) ? ((c - 1) / tb + 1) * p.n_slices * nch : 0;
    int incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = running + incl - nt;
    const uint64_t who = __ballot(u >= excl && u < excl + nt);
    if (who) {
      const int src = __ffsll(static_cast<long long>(who)) - 1;
      const int local = u - __shfl(excl, src, 64);
      const int nchs = __shfl(nch, src, 64);
      const int cs = __shfl(c, src, 64);
      const int per_tile = p.n_slices * nchs;
      const int k = local / per_tile;
      const int rem = local - k * per_tile;
      out.slot = s0 + src;
      out.start = __shfl(s < p.S ? p.offsets[s] : 0, src, 64) + k * tb;
      out.len = (cs - k * tb) < tb ? (cs - k * tb) : tb;
      out.slice = rem / nchs;
      out.chunk = rem - out.slice * nchs;
    }
    running += __shfl(incl, 63, 64);
  }
  *total = running;
  return out;
}

// Row-split units: a slot with c grouped tokens and clamped rank rho has
// ceil(c / tb) token tiles of ceil(n_slices * ceil(rho / 16) / gp) row groups
// each; units run in slot order, then tile, then row group.
__device__ __forceinline__ int rows_units_of(int c, int rho, int tb, int gp, int n_slices) {
  if (c <= 0 || rho <= 0) return 0;
  return ((c - 1) / tb + 1) * ((n_slices * ((rho + 15) >> 4) + gp - 1) / gp);
}

struct RowsUnit {
  int slot;  // -1: no such unit
  int start, len, rg, nu;
};

// Wave-level: the unit count, and the u-th unit (u < 0: count only).
__device__ RowsUnit find_rows_unit(int u, int tb, int gp, const ShrinkArgs& p, int* total) {
  const int lane = threadIdx.x & 63;
  int running = 0;
  RowsUnit out{-1, 0, 0, 0, 0};
  for (int s0 = 0; s0 < p.S; s0 += 64) {
    const int s = s0 + lane;
    const int c = (s < p.S) ? p.counts[s] : 0;
    const int rho = (s < p.S) ? clamp_rank(p.ranks[s], p.r_max) : 0;
    const int nu = (c > 0 && rho > 0) ? (p.n_slices * ((rho + 15) >> 4) + gp - 1) / gp : 0;
    const int nt = rows_units_of(c, rho, tb, gp, p.n_slices);
    int incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = running + incl - nt;
    const bool mine = u >= excl && u < excl + nt;
    const uint64_t who = __ballot(mine);
    if (who) {
      const int src = __ffsll(static_cast<long long>(who)) - 1;
      const int local = u - __shfl(excl, src, 64);
      const int nus = __shfl(nu, src, 64);
      const int cs = __shfl(c, src, 64);
      const int k = local / nus;
      out.slot = s0 + src;
      out.start = __shfl(s < p.S ? p.offsets[s] : 0, src, 64) + k * tb;
      out.len = (cs - k * tb) < tb ? (cs - k * tb) : tb;
      out.rg = local - k * nus;
      out.nu = nus;
    }
    running += __shfl(incl, 63, 64);
  }
  *total = running;
  return out;
}


template <class Tag, int BMB, int RB>
__global__ __launch_bounds__(256) void slot_shrink_kernel(ShrinkArgs p) {
  using E = typename Tag::elem;
  constexpr int VEC = Tag::VEC;
  constexpr int CH = 4 * VEC;
  constexpr int TB = 16 * BMB;
  constexpr int U = (8 / (BMB + RB)) > 0 ? (8 / (BMB + RB)) : 1;
  __shared__ f32x4_t red[4][BMB * RB][64];
  __shared__ Tile sh_tile;
  __shared__ int sh_tok[TB];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int per_tile = p.n_slices * p.row_chunks;
  const int ti = blockIdx.x / per_tile;
  const int rem = blockIdx.x - ti * per_tile;
  const int slice = rem / p.row_chunks;
  const int j0 = (rem - slice * p.row_chunks) * 16 * RB;

  if (wave == 0) {
    const Tile tl = find_tile(ti, TB, p.counts, p.offsets, p.S);
    if (lane == 0) sh_tile = tl;
  }
  __syncthreads();
  const Tile tl = sh_tile;
  if (tl.slot < 0) return;
  const int rho = clamp_rank(p.ranks[tl.slot], p.r_max);
  if (j0 >= rho) return;
  if (threadIdx.x < TB) sh_tok[threadIdx.x] = (static_cast<int>(threadIdx.x) < tl.len) ? p.sorted[tl.start + threadIdx.x] : 0;
  __syncthreads();

  f32x4_t acc[BMB][RB];
#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[b][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const E* xrow[BMB];
  bool xok[BMB];
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    xok[b] = 16 * b + col < tl.len;
    xrow[b] = static_cast<const E*>(p.x) + (int64_t)sh_tok[16 * b + col] * p.ldx + grp * VEC;
  }
  const E* arow[RB];
  bool aok[RB];
  const E* a_slot = static_cast<const E*>(p.a) + (int64_t)tl.slot * p.as0;
#pragma unroll
  for (int q = 0; q < RB; ++q) {
    const int j = j0 + 16 * q + col;
    aok[q] = j < rho;
    arow[q] = a_slot + (int64_t)(slice * p.r_max + (aok[q] ? j : 0)) * p.as1 + grp * VEC;
  }
  bool bany[BMB];
#pragma unroll
  for (int b = 0; b < BMB; ++b) bany[b] = 16 * b < tl.len;

  const int64_t nch = (p.K + CH - 1) / CH;
  for (int64_t c = wave; c < nch; c += 4 * U) {
    uint4 xf[U][BMB];
    uint4 af[U][RB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cc = c + 4 * u;
      const bool kok = cc < nch && cc * CH + grp * VEC < p.K;
#pragma unroll
      for (int b = 0; b < BMB; ++b) xf[u][b] = (kok && xok[b]) ? ld16(xrow[b] + cc * CH) : zero4();
#pragma unroll
      for (int q = 0; q < RB; ++q) af[u][q] = (kok && aok[q]) ? ld16(arow[q] + cc * CH) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < BMB; ++b)
        if (bany[b]) {
#pragma unroll
          for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[b][q], af[u][q], xf[u][b]);
        }
  }

#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) red[wave][b * RB + q][lane] = acc[b][q];
  __syncthreads();
  // wave w stores token blocks w, w+4, ...
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    if ((b & 3) != wave) continue;
    if (16 * b + col >= tl.len) continue;
    float* hrow = p.h + (int64_t)sh_tok[16 * b + col] * p.hs0 + (int64_t)slice * p.hs1;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int i = b * RB + q;
      f32x4_t s = red[0][i][lane];
      s += red[1][i][lane];
      s += red[2][i][lane];
      s += red[3][i][lane];
      const int j = j0 + 16 * q + 4 * grp;
      if (p.h_vec && j + 4 <= rho) {
        st16f(hrow + j, s);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < rho) hrow[j + e] = s[e];
      }
    }
  }
}

// Per-wave feature loop of the pipelined shrink. The calling wave contracts
// the feature chunks [cbeg, cend) (CH = 4*VEC features each) of a tile's x
// rows (token block b < BMB: tokens tok[16b + lane%16], those at or past
// `len` masked) with the adapter rows j0 + 16q + (lane%16) (q < RB; rows at
// or past rho masked) of one slice of one slot. acc[b][q] gets the chunks
// added in increasing order; lane (col, grp) holds rows 4*grp..4*grp+3 of
// rank block q for token col, i.e. h[token][j0 + 16q + 4grp + i].
// bf16: each stage's x rows and adapter rows are loaded row-linearly (whole
// row segments per instruction) into the wave's LDS tile `stage` (rows padded
// by 16 bytes, SBYTES bytes) and read back as conflict-free fragments; f32:
// the fragments are loaded directly. Loads go through buffer descriptors
// (masked lanes use kOOB, no branches), and U chunks of the next stage are in
// flight while the current one is multiplied. Needs x and the slot's adapter
// rows within 2 GiB descriptors (the host checks).
template <class Tag, int BMB, int RB, int U>
struct PipeShrink {
  using E = typename Tag::elem;
  static constexpr int VEC = Tag::VEC;
  static constexpr int ES = sizeof(E);
  static constexpr int CH = 4 * VEC;  // features per MFMA step
  static constexpr bool LIN = ES == 2;
  static constexpr int SROW = U * CH * ES;
  static constexpr int PITCH = SROW + 16;
  static constexpr int LPR = SROW / 16;
  static constexpr int RPI = LIN ? 64 / LPR : 16;
  static constexpr int ZN = LIN ? 16 * BMB / RPI : BMB;
  static constexpr int WN = LIN ? 16 * RB / RPI : RB;
  static constexpr int SBYTES = LIN ? 16 * (BMB + RB) * PITCH : 0;

  static __device__ __forceinline__ void run(f32x4_t (&acc)[BMB][RB], const ShrinkArgs& p, const int* tok, int len,
                                             int slot, int slice, int j0, int rho, int cbeg, int cend, char* stage) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
    const rsrc_t ra = make_rsrc(static_cast<const E*>(p.a) + (int64_t)slot * p.as0,
                                (int64_t)p.n_slices * p.r_max * p.as1 * ES);
    uint32_t xoff[BMB];
    bool bany[BMB];
#pragma unroll
    for (int b = 0; b < BMB; ++b) {
      const bool ok = 16 * b + col < len;
      xoff[b] = ok ? static_cast<uint32_t>(((int64_t)tok[16 * b + col] * p.ldx + grp * VEC) * ES) : kOOB;
      bany[b] = 16 * b < len;
    }
    uint32_t aoff[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int j = j0 + 16 * q + col;
      aoff[q] = j < rho ? static_cast<uint32_t>(((int64_t)(slice * p.r_max + j) * p.as1 + grp * VEC) * ES) : kOOB;
    }

    const int lpiece = lane % LPR;
    const int lstep = lpiece >> 2;
    const int lgrp = lpiece & 3;
    uint32_t lx[LIN ? ZN : 1], la[LIN ? WN : 1];
    if constexpr (LIN) {
#pragma unroll
      for (int i = 0; i < ZN; ++i) {
        const int row = i * RPI + lane / LPR;
        lx[i] = row < len ? static_cast<uint32_t>(((int64_t)tok[row] * p.ldx + lgrp * VEC) * ES) : kOOB;
      }
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        const int j = j0 + i * RPI + lane / LPR;
        la[i] = j < rho ? static_cast<uint32_t>(((int64_t)(slice * p.r_max + j) * p.as1 + lgrp * VEC) * ES) : kOOB;
      }
    }

    const int K = static_cast<int>(p.K);
    // LIN: xf[0] holds the stage's ZN row-linear x vectors, af[0] its WN
    // adapter vectors; else [u][b] and [u][q] MFMA fragments
    auto load = [&](uint4 (&xf)[U][ZN], uint4 (&af)[U][WN], int c) {
      if constexpr (LIN) {
        const int cc = c + lstep;
        const bool kok = cc < cend && cc * CH + lgrp * VEC < K;
        const uint32_t kb = static_cast<uint32_t>(cc) * static_cast<uint32_t>(CH * ES);
#pragma unroll
        for (int i = 0; i < ZN; ++i) xf[0][i] = sload16(rx, (kok && lx[i] != kOOB) ? lx[i] + kb : kOOB);
#pragma unroll
        for (int i = 0; i < WN; ++i) af[0][i] = bload16(ra, (kok && la[i] != kOOB) ? la[i] + kb : kOOB);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int cc = c + u;
          const bool kok = cc < cend && cc * CH + grp * VEC < K;
          const uint32_t kb = static_cast<uint32_t>(cc) * static_cast<uint32_t>(CH * ES);  // < x row bytes when kok
#pragma unroll
          for (int b = 0; b < BMB; ++b) xf[u][b] = sload16(rx, (kok && xoff[b] != kOOB) ? xoff[b] + kb : kOOB);
#pragma unroll
          for (int q = 0; q < RB; ++q) af[u][q] = bload16(ra, (kok && aoff[q] != kOOB) ? aoff[q] + kb : kOOB);
        }
      }
    };
    auto mma = [&](const uint4 (&xf)[U][ZN], const uint4 (&af)[U][WN]) {
      if constexpr (LIN) {
#pragma unroll
        for (int i = 0; i < ZN; ++i)
          *reinterpret_cast<uint4*>(stage + (i * RPI + lane / LPR) * PITCH + lpiece * 16) = xf[0][i];
#pragma unroll
        for (int i = 0; i < WN; ++i)
          *reinterpret_cast<uint4*>(stage + (16 * BMB + i * RPI + lane / LPR) * PITCH + lpiece * 16) = af[0][i];
        uint4 w[U][RB];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < RB; ++q)
            w[u][q] = *reinterpret_cast<const uint4*>(stage + (16 * (BMB + q) + col) * PITCH + (u * 4 + grp) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int b = 0; b < BMB; ++b)
            if (bany[b]) {
              const uint4 z = *reinterpret_cast<const uint4*>(stage + (16 * b + col) * PITCH + (u * 4 + grp) * 16);
#pragma unroll
              for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[b][q], w[u][q], z);
            }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int b = 0; b < BMB; ++b)
            if (bany[b]) {
#pragma unroll
              for (int q = 0; q < RB; ++q) mma_vec<Tag>(acc[b][q], af[u][q], xf[u][b]);
            }
      }
    };
    // two register stages; the loop body has no exit in the middle (an odd
    // stage count ends with a stage of zeros)
    uint4 xA[U][ZN], aA[U][WN], xB[U][ZN], aB[U][WN];
    if (cbeg < cend) {
      load(xA, aA, cbeg);
      for (int c = cbeg; c < cend; c += 2 * U) {
        load(xB, aB, c + U);
        sched_fence();
        mma(xA, aA);
        sched_fence();
        load(xA, aA, c + 2 * U);
        sched_fence();
        mma(xB, aB);
        sched_fence();
      }
    }
  }
};

constexpr int kShrinkGroup = 4;  // token tiles per XCD group (pipelined shrink)

// Pipelined form of slot_shrink_kernel (same grid and reduction): every wave
// contracts one contiguous quarter of the feature axis with PipeShrink.
template <class Tag, int BMB, int RB, int U, bool DENSE>
__global__ __launch_bounds__(256) void slot_shrink_pipe_kernel(ShrinkArgs p) {
  using PS = PipeShrink<Tag, BMB, RB, U>;
  constexpr int TB = 16 * BMB;
  constexpr int RBYTES = 4 * BMB * RB * 64 * 16;
  // the staging tiles share their memory with the partial sums
  __shared__ __attribute__((aligned(16))) char shr[4 * PS::SBYTES > RBYTES ? 4 * PS::SBYTES : RBYTES];
  auto red = reinterpret_cast<f32x4_t(*)[BMB * RB][64]>(shr);
  __shared__ Tile sh_tile;
  __shared__ int sh_tok[TB];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  // Workgroup ids go round-robin over the 8 XCDs (id mod 8).
  // DENSE: only live (tile, slice, rank chunk) units, counted on the device,
  // dealt to the XCDs in 8 equal runs of consecutive units (a slot's units
  // share one L2); ids past the runs exit. For batches below 512 tokens,
  // where many slots hold one short tile and rank blocks past a slot's rank
  // would idle: 32 slots at 64 / 256 tokens 10.8 -> 8.2 / 12.6 -> 9.2 us;
  // with four rank blocks per workgroup (512 tokens and more) no gain and up
  // to 5% slower (the count is one more pass over the slots).
  // Else groups of kShrinkGroup consecutive token tiles (mostly tiles of one
  // slot) go to one XCD, and within a group the workgroups of one (slice,
  // rank chunk) follow each other: the adapter rows are re-read by the
  // group's tiles and each tile's x rows by its slice and rank-chunk
  // workgroups while they are in that XCD's L2. The grid is padded to a
  // multiple of 8 groups; tile numbers past the last tile find no slot and
  // exit.
  Tile tl;
  int slice, j0, rho;
  if constexpr (DENSE) {
    __shared__ PipeUnit sh_unit;
    if (wave == 0) {
      int total = 0;
      find_pipe_unit(-1, TB, 16 * RB, p, &total);
      const int per = (total + 7) >> 3;
      const int kk = static_cast<int>(blockIdx.x >> 3);
      const int u = static_cast<int>(blockIdx.x & 7) * per + kk;
      PipeUnit un{-1, 0, 0, 0, 0};
      if (kk < per && u < total) un = find_pipe_unit(u, TB, 16 * RB, p, &total);
      if (lane == 0) sh_unit = un;
    }
    __syncthreads();
    const PipeUnit un = sh_unit;
    if (un.slot < 0) return;
    tl = Tile{un.slot, un.start, un.len};
    slice = un.slice;
    j0 = un.chunk * 16 * RB;
    rho = clamp_rank(p.ranks[tl.slot], p.r_max);
  } else {
    const int per_tile = p.n_slices * p.row_chunks;
    const int kx = static_cast<int>(blockIdx.x >> 3);
    const int gw = kShrinkGroup * per_tile;  // workgroups per group
    const int r2 = kx % gw;
    const int ti = ((kx / gw) * 8 + static_cast<int>(blockIdx.x & 7)) * kShrinkGroup + r2 % kShrinkGroup;
    const int rem = r2 / kShrinkGroup;
    slice = rem / p.row_chunks;
    j0 = (rem - slice * p.row_chunks) * 16 * RB;
    if (wave == 0) {
      const Tile t = find_tile(ti, TB, p.counts, p.offsets, p.S);
      if (lane == 0) sh_tile = t;
    }
    __syncthreads();
    tl = sh_tile;
    if (tl.slot < 0) return;
    rho = clamp_rank(p.ranks[tl.slot], p.r_max);
    if (j0 >= rho) return;
  }
  if (threadIdx.x < TB) sh_tok[threadIdx.x] = (static_cast<int>(threadIdx.x) < tl.len) ? p.sorted[tl.start + threadIdx.x] : 0;
  __syncthreads();

  f32x4_t acc[BMB][RB];
#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) acc[b][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nch = static_cast<int>((p.K + PS::CH - 1) / PS::CH);
  const int per = (nch + 3) / 4;
  const int cbeg = wave * per;
  const int cend = (cbeg + per < nch) ? cbeg + per : nch;
  PS::run(acc, p, sh_tok, tl.len, tl.slot, slice, j0, rho, cbeg, cend, shr + wave * PS::SBYTES);
  if constexpr (PS::LIN) __syncthreads();

#pragma unroll
  for (int b = 0; b < BMB; ++b)
#pragma unroll
    for (int q = 0; q < RB; ++q) red[wave][b * RB + q][lane] = acc[b][q];
  __syncthreads();
  // wave w stores token blocks w, w+4, ...
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    if ((b & 3) != wave) continue;
    if (16 * b + col >= tl.len) continue;
    float* hrow = p.h + (int64_t)sh_tok[16 * b + col] * p.hs0 + (int64_t)slice * p.hs1;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int i = b * RB + q;
      f32x4_t sum = red[0][i][lane];
      sum += red[1][i][lane];
      sum += red[2][i][lane];
      sum += red[3][i][lane];
      const int j = j0 + 16 * q + 4 * grp;
      if (p.h_vec && j + 4 <= rho) {
        st16f(hrow + j, sum);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < rho) hrow[j + e] = sum[e];
      }
    }
  }
}

// Row-split shrink for bf16 inputs (x and one slot's a within 2 GiB
// descriptors). A workgroup of NW waves owns a tile of up to 128 grouped
// tokens of one slot against up to NW*PPW (slice, 16-row rank block) pairs of
// its slices (a slot with more pairs gets further row-group workgroups, the
// pairs split evenly over them). Wave w takes pairs w, w+NW, ... of its row
// group over the whole feature axis, so no partial sums are exchanged between
// waves. One workgroup streams only so fast (a lone 4-wave one about 28 GB/s)
// and the time follows the workgroup that moves the most bytes, so 8 waves of
// one pair each serve a tile: up to 8 pairs per workgroup.
// The tile's x rows are fetched once per stage of 32*U features by the whole
// workgroup, row-linearly (each load instruction covers whole row segments),
// into a double-buffered LDS tile with padded rows (every fragment read is
// conflict-free), while each wave streams
// its own pairs' adapter rows from global memory in two register stages. Each
// x fragment feeds NP MFMAs and each adapter fragment eight. Compared with one
// workgroup per (tile, slice, rank chunk), a tile's x rows reach the CU once
// per row group instead of once per slice and rank chunk, and each adapter
// row is shared by 128 tokens instead of 64.
// Only live (tile, row group) units get a workgroup's work, dealt to the
// XCDs in equal runs of consecutive units (see the kernel), so adapter and x
// rows are re-read from one XCD's L2.

template <int TT, int U, int NP, int NW>
__device__ __forceinline__ void shrink_rows_body(const ShrinkArgs& p, const Tile& tl, int rho, rsrc_t rx, rsrc_t ra,
                                                 const uint32_t (&xoff)[TT * U / NW], const bool (&bany)[TT],
                                                 const int (&psl)[4], const int (&pj)[4],
                                                 const int* tok, char* lds, char* alds) {
  constexpr int XV = TT * U / NW;    // x vectors per thread per stage
  constexpr int NA = NP * U;         // adapter vectors per lane and stage (row-linear)
  constexpr int ARPI = 64 / (4 * U);  // adapter rows per load instruction
  constexpr int LPR = 4 * U;         // 16-byte pieces of a row per stage
  constexpr int PITCH = 64 * U + 16;  // LDS row pitch: the 16 rows of a fragment read fall in distinct banks
  constexpr int BUFB = 16 * TT * PITCH;  // bytes per LDS buffer
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int K = static_cast<int>(p.K);
  const int nstage = (K + 32 * U - 1) / (32 * U);
  f32x4_t acc[TT][NP];
#pragma unroll
  for (int b = 0; b < TT; ++b)
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[b][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // entry v = tid + 64*NW*i of a stage: token row v / 4U, 16-byte piece v % 4U
  // of the row's stage segment (features 32*u + 8*g with u = piece / 4,
  // g = piece % 4): each load instruction covers whole row segments; the
  // piece goes to LDS at row * PITCH + piece * 16
  auto load_x = [&](uint4 (&xs)[XV], int st) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int v = tid + 64 * NW * i;
      const int u = (v % LPR) >> 2;
      const int g = v & 3;
      const bool kok = st < nstage && (st * U + u) * 32 + g * 8 < K;
      xs[i] = sload16(rx, (kok && xoff[i] != kOOB) ? xoff[i] + static_cast<uint32_t>(st * U) * 64u : kOOB);
    }
  };
  auto store_x = [&](const uint4 (&xs)[XV], int buf) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int v = tid + 64 * NW * i;
      *reinterpret_cast<uint4*>(lds + buf * BUFB + (v / LPR) * PITCH + (v % LPR) * 16) = xs[i];
    }
  };
  // This wave's adapter rows (16 per pair) are loaded row-linearly too: load
  // i covers rows i*ARPI .. +ARPI-1 (pair i*ARPI/16), lane -> row lane / 4U,
  // 16-byte piece lane % 4U; the pieces go to the wave's LDS tile and the
  // fragments are read back from it.
  const int apiece = lane % LPR;
  const int astep = apiece >> 2;
  const int agrp = apiece & 3;
  uint32_t aro[NA > 0 ? NA : 1];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = i * ARPI + lane / LPR;  // row of the wave's tile
    const int pr = (i * ARPI) / 16;         // its pair (compile-time per i)
    const int j = pj[pr] + (row & 15);
    aro[i] = j < rho ? static_cast<uint32_t>(((int64_t)(psl[pr] * p.r_max + j) * p.as1 + agrp * 8) * 2) : kOOB;
  }
  auto load_a = [&](uint4 (&al)[NA > 0 ? NA : 1], int st) {
    const int cc = st * U + astep;
    const bool kok = st < nstage && cc * 32 + agrp * 8 < K;
    const uint32_t kb = static_cast<uint32_t>(cc) * 64u;
#pragma unroll
    for (int i = 0; i < NA; ++i) al[i] = bload16(ra, (kok && aro[i] != kOOB) ? aro[i] + kb : kOOB);
  };
  auto mma = [&](const uint4 (&al)[NA > 0 ? NA : 1], int buf) {
    if constexpr (NP > 0) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        *reinterpret_cast<uint4*>(alds + (i * ARPI + lane / LPR) * PITCH + apiece * 16) = al[i];
      uint4 af[U][NP];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < NP; ++i)
          af[u][i] = *reinterpret_cast<const uint4*>(alds + (16 * i + col) * PITCH + (u * 4 + grp) * 16);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < TT; ++b)
          if (bany[b]) {
            const uint4 xf =
                *reinterpret_cast<const uint4*>(lds + buf * BUFB + (16 * b + col) * PITCH + (u * 4 + grp) * 16);
#pragma unroll
            for (int i = 0; i < NP; ++i) mma_vec<BF16>(acc[b][i], af[u][i], xf);
          }
    }
  };
  // Stage s: x in LDS buffer s & 1, adapter fragments in register set s & 1.
  // Stage s+1's x is stored after stage s is multiplied (its buffer was last
  // read before the previous barrier) and stage s+2's loads are issued then.
  // Stages past the end load zeros and add nothing, so the loop body needs no
  // exit in the middle.
  uint4 xs[XV];
  uint4 aA[NA > 0 ? NA : 1], aB[NA > 0 ? NA : 1];
  load_x(xs, 0);
  load_a(aA, 0);
  store_x(xs, 0);
  load_x(xs, 1);
  load_a(aB, 1);
  __syncthreads();
  for (int st = 0; st < nstage; st += 2) {
    mma(aA, 0);
    sched_fence();
    load_a(aA, st + 2);
    store_x(xs, 1);
    load_x(xs, st + 2);
    __syncthreads();
    mma(aB, 1);
    sched_fence();
    load_a(aB, st + 3);
    store_x(xs, 0);
    load_x(xs, st + 3);
    __syncthreads();
  }
  // lane holds rank rows pj + 4grp .. +3 of token 16b + col for each pair
#pragma unroll
  for (int b = 0; b < TT; ++b) {
    if (16 * b + col >= tl.len) continue;
    const int64_t t = tok[16 * b + col];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float* hrow = p.h + t * p.hs0 + (int64_t)psl[i] * p.hs1;
      const int j = pj[i] + 4 * grp;
      if (p.h_vec && j + 4 <= rho) {
        st16f(hrow + j, acc[b][i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < rho) hrow[j + e] = acc[b][i][e];
      }
    }
  }
}

template <int TT, int U, int PPW, int NW>
__global__ __launch_bounds__(64 * NW) void slot_shrink_rows_kernel(ShrinkArgs p) {
  static_assert((TT * U) % NW == 0 && (U & (U - 1)) == 0 && PPW >= 1 && PPW <= 4 && 64 * NW >= 16 * TT,
                "stage shape");
  constexpr int TB = 16 * TT;
  constexpr int XV = TT * U / NW;
  constexpr int GP = NW * PPW;  // (slice, rank block) pairs per workgroup
  // x stages; per wave: PPW pairs x 16 rows. At least 80 KB in all, so one
  // workgroup runs per CU and the dispatcher spreads the units over the CUs
  // instead of pairing some (prefill at r_max 128 / 64 / 32: 140 / 125 / 125
  // -> 138 / 125 / 123 us).
  constexpr int XBYTES = 2 * 16 * TT * (64 * U + 16);
  constexpr int ABYTES = 16 * PPW * (64 * U + 16);
  constexpr int kMinLds = 80 * 1024;
  constexpr int APAD = (XBYTES + NW * ABYTES >= kMinLds) ? 0 : (kMinLds - XBYTES - NW * ABYTES + 16 * NW - 1) / (16 * NW) * 16;
  __shared__ __attribute__((aligned(16))) char lds[XBYTES];
  __shared__ __attribute__((aligned(16))) char alds[NW][ABYTES + APAD];
  __shared__ int sh_tok[TB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  // Workgroup ids go round-robin over the 8 XCDs (id mod 8). The live units
  // are cut into 8 runs of `per` consecutive units, run x on XCD x, so every
  // XCD gets the same number and a tile's row groups and a slot's tiles
  // share one L2; ids past the runs exit.
  __shared__ RowsUnit sh_unit;
  if (wave == 0) {
    int total = 0;
    find_rows_unit(-1, TB, GP, p, &total);
    const int per = (total + 7) >> 3;
    const int k = static_cast<int>(blockIdx.x >> 3);
    const int u = static_cast<int>(blockIdx.x & 7) * per + k;
    RowsUnit un{-1, 0, 0, 0, 0};
    if (k < per && u < total) un = find_rows_unit(u, TB, GP, p, &total);
    if (lane == 0) sh_unit = un;
  }
  __syncthreads();
  const RowsUnit un = sh_unit;
  if (un.slot < 0) return;
  const Tile tl{un.slot, un.start, un.len};
  const int rg = un.rg;
  const int rho = clamp_rank(p.ranks[tl.slot], p.r_max);
  const int nq = (rho + 15) >> 4;
  const int npairs = p.n_slices * nq;
  // the slot's pairs split evenly over its row groups (a workgroup's time
  // follows its bytes: 24 pairs as 12 + 12 rather than 16 + 8, prefill at
  // r_max 128 187 -> 164 us, the same bits)
  const int nu = un.nu;
  const int pbeg = rg * npairs / nu;
  const int pend = (rg + 1) * npairs / nu;
  if (tid < TB) sh_tok[tid] = (tid < tl.len) ? p.sorted[tl.start + tid] : 0;
  __syncthreads();
  // this wave's pairs: pbeg + wave + NW*i for i < npw (waves without pairs still
  // load their share of x and take part in every barrier)
  const int avail = pend - pbeg - wave;
  const int npw = uniform_int(avail <= 0 ? 0 : (((avail + NW - 1) / NW) < PPW ? ((avail + NW - 1) / NW) : PPW));

  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
  const rsrc_t ra = make_rsrc(static_cast<const uint16_t*>(p.a) + (int64_t)tl.slot * p.as0,
                              (int64_t)p.n_slices * p.r_max * p.as1 * 2);
  uint32_t xoff[XV];
#pragma unroll
  for (int i = 0; i < XV; ++i) {
    const int v = tid + 64 * NW * i;
    const int row = v / (4 * U);
    const int u = (v % (4 * U)) >> 2;
    const int g = v & 3;
    xoff[i] = row < tl.len ? static_cast<uint32_t>(((int64_t)sh_tok[row] * p.ldx + u * 32 + g * 8) * 2) : kOOB;
  }
  bool bany[TT];
#pragma unroll
  for (int b = 0; b < TT; ++b) bany[b] = 16 * b < tl.len;
  // this wave's pairs: slice and first rank row (rows at or past rho read 0)
  int psl[4], pj[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pg = pbeg + wave + NW * i;
    const int sl = pg / nq;
    psl[i] = sl;
    pj[i] = 16 * (pg - sl * nq);
  }
  switch (npw) {
    case 0: shrink_rows_body<TT, U, 0, NW>(p, tl, rho, rx, ra, xoff, bany, psl, pj, sh_tok, lds, alds[wave]); break;
    case 1: shrink_rows_body<TT, U, 1, NW>(p, tl, rho, rx, ra, xoff, bany, psl, pj, sh_tok, lds, alds[wave]); break;
    case 2:
      if constexpr (PPW >= 2) shrink_rows_body<TT, U, 2, NW>(p, tl, rho, rx, ra, xoff, bany, psl, pj, sh_tok, lds, alds[wave]);
      break;
    case 3:
      if constexpr (PPW >= 3) shrink_rows_body<TT, U, 3, NW>(p, tl, rho, rx, ra, xoff, bany, psl, pj, sh_tok, lds, alds[wave]);
      break;
    default:
      if constexpr (PPW >= 4) shrink_rows_body<TT, U, 4, NW>(p, tl, rho, rx, ra, xoff, bany, psl, pj, sh_tok, lds, alds[wave]);
      break;
  }
}

// ---------------------------------------------------------------------------
// expand_fused: y[t, off_i + c] += sc[s] * sum_{j < rank} h[t, i, j] * b[s, off_i + c, j]
// ---------------------------------------------------------------------------

struct ExpandArgs {
  const float* h;
  int64_t hs0, hs1;
  const void* b;
  int64_t bs0, bs1;  // slot and row strides; j contiguous
  void* y;  // float32, or bfloat16 (weights in bfloat16): updated in place
  int64_t ldy;
  const float* scalings;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted;
  const int32_t* ranks;
  int S, r_max, n_slices, total_chunks;
  int64_t chunk_cols;  // columns per chunk (streaming kernel)
  int64_t y_bytes;     // bytes of y a descriptor may span (streaming and band kernels)
  int64_t h_bytes;     // bytes of h a descriptor may span (band kernel)
  int n_work;          // band kernel: pieces x total_chunks work items
  bool h_vec;  // h rows 16-byte aligned
  bool b_vec;  // b rows aligned for 4-element loads
  int64_t slice_off[kMaxSlices];
  int64_t slice_w[kMaxSlices];
  int chunk_begin[kMaxSlices + 1];
};

constexpr int kExpandNBU = 4;                  // 16-column blocks per wave
constexpr int kExpandCols = 64 * kExpandNBU;   // columns per workgroup

template <class Tag, class YT, int BMB, int RBM>
__global__ __launch_bounds__(256) void slot_expand_kernel(ExpandArgs p) {
  using E = typename Tag::elem;
  using O = Out<YT>;
  YT* const yp = static_cast<YT*>(p.y);
  constexpr int TB = 16 * BMB;
  constexpr int NBU = kExpandNBU;
  __shared__ Tile sh_tile;
  __shared__ int sh_tok[TB];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int ti = blockIdx.x / p.total_chunks;
  const int ch = blockIdx.x - ti * p.total_chunks;
  int slice = 0;
  while (slice + 1 < p.n_slices && ch >= p.chunk_begin[slice + 1]) ++slice;
  const int64_t c0 = (int64_t)(ch - p.chunk_begin[slice]) * kExpandCols;
  const int64_t width = p.slice_w[slice];
  const int64_t off = p.slice_off[slice];

  if (wave == 0) {
    const Tile tl = find_tile(ti, TB, p.counts, p.offsets, p.S);
    if (lane == 0) sh_tile = tl;
  }
  __syncthreads();
  const Tile tl = sh_tile;
  if (tl.slot < 0) return;
  const int rho = clamp_rank(p.ranks[tl.slot], p.r_max);
  if (threadIdx.x < TB) sh_tok[threadIdx.x] = (static_cast<int>(threadIdx.x) < tl.len) ? p.sorted[tl.start + threadIdx.x] : 0;
  __syncthreads();
  const float sc = p.scalings[tl.slot];
  const int nq = (rho + 15) / 16;

  // (sc * h)^T operand fragments of the tile's tokens; columns >= rank read as 0
  uint4 hf[BMB][RBM];
  bool tok_ok[BMB];
  const float* hrow[BMB];
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    tok_ok[b] = 16 * b + col < tl.len;
    hrow[b] = p.h + (int64_t)sh_tok[16 * b + col] * p.hs0 + (int64_t)slice * p.hs1;
#pragma unroll
    for (int q = 0; q < RBM; ++q) {
      f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int j = 16 * q + 4 * grp;
      if (tok_ok[b] && q < nq) {
        if (p.h_vec && j + 4 <= rho) {
          v = ld16f(hrow[b] + j);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < rho) v[e] = hrow[b][j + e];
        }
      }
      v *= sc;
      hf[b][q] = split_frag<Tag>(v);
    }
  }

  const E* b_slot = static_cast<const E*>(p.b) + (int64_t)tl.slot * p.bs0;
  // wave w: 16-column blocks w*NBU .. w*NBU+NBU-1 of this chunk
  uint4 wv[NBU][RBM];
  f32x4_t cv[NBU][BMB];
#pragma unroll
  for (int u = 0; u < NBU; ++u) {
    const int64_t cb = c0 + (int64_t)(wave * NBU + u) * 16;
    const int64_t nrow = cb + col;
    const bool nok = nrow < width;
    const E* wr = b_slot + (off + (nok ? nrow : 0)) * p.bs1;
#pragma unroll
    for (int q = 0; q < RBM; ++q) wv[u][q] = (nok && q < nq) ? load_wvec4<Tag>(wr, 16 * q + 4 * grp, rho, p.b_vec) : zero4();
    const int64_t ncol = cb + 4 * grp;
#pragma unroll
    for (int b = 0; b < BMB; ++b) {
      const bool ok = tok_ok[b] && ncol < width;
      cv[u][b] = ok ? O::ld4(yp + (int64_t)sh_tok[16 * b + col] * p.ldy + off + ncol) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int u = 0; u < NBU; ++u) {
    const int64_t cb = c0 + (int64_t)(wave * NBU + u) * 16;
    const int64_t ncol = cb + 4 * grp;
#pragma unroll
    for (int b = 0; b < BMB; ++b) {
      if (16 * b >= tl.len) continue;
      f32x4_t pr = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < RBM; ++q)
        if (q < nq) mma_rank16<Tag>(pr, wv[u][q], hf[b][q]);
      if (tok_ok[b] && ncol < width) O::st4(yp + (int64_t)sh_tok[16 * b + col] * p.ldy + off + ncol, cv[u][b] + pr);
    }
  }
}

// Column walk of the streaming expand. The workgroup's NW waves update the
// output columns [cb, ce) of one slice for a tile's tokens, 16*NBU columns per
// wave per stage, with the next stage's weight and output loads in flight
// while the current stage is multiplied. hf[b][q]: (sc*h)^T operand fragments
// of token block b (rank block q < NQ, ranks >= rho zero); yrow[b]: byte
// offset in y (elements of type YT) of this lane's token row at the slice
// start (used only when tok_ok[b]); rb: descriptor over the slot's weight rows
// of the slice (ldb elements apart). Masked lanes (tokens past the tile,
// columns past ce) use kOOB, so the loop has no branch around its memory
// operations.
template <class Tag, class YT, int BMB, int RBM, int NQ, int NBU, int NW>
__device__ __forceinline__ void expand_stream_walk(const uint4 (&hf)[BMB][RBM], const uint32_t (&yrow)[BMB],
                                                   const bool (&tok_ok)[BMB], rsrc_t ry, rsrc_t rb, int ldb, int cb,
                                                   int ce, int rho) {
  using E = typename Tag::elem;
  constexpr int ES = sizeof(E);
  using WF = WFrag<Tag>;
  using wf_t = typename WF::type;
  using O = Out<YT>;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  constexpr int kStage = NW * NBU * 16;
  const int nst = (ce - cb + kStage - 1) / kStage;
  auto yoff = [&](int b, int n) -> uint32_t {
    return (tok_ok[b] && n < ce) ? yrow[b] + static_cast<uint32_t>(n) * static_cast<uint32_t>(O::ES) : kOOB;
  };
  auto load2 = [&](wf_t (&wv)[NBU][NQ], f32x4_t (&cv)[NBU][BMB], int k) {
#pragma unroll
    for (int u = 0; u < NBU; ++u) {
      const int nb = cb + k * kStage + (wave * NBU + u) * 16;
      const int nrow = nb + col;
      const bool rok = k < nst && nrow < ce;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int j0 = 16 * q + 4 * grp;
        wv[u][q] = WF::bload(rb, rok ? static_cast<uint32_t>((nrow * ldb + j0) * ES) : kOOB, j0, rho);
      }
#pragma unroll
      for (int b = 0; b < BMB; ++b)
        cv[u][b] = O::load4(ry, k < nst ? yoff(b, nb + 4 * grp) : kOOB);
    }
  };
  auto comp2 = [&](const wf_t (&wv)[NBU][NQ], f32x4_t (&cv)[NBU][BMB], int k) {
#pragma unroll
    for (int u = 0; u < NBU; ++u) {
      const int nb = cb + k * kStage + (wave * NBU + u) * 16;
#pragma unroll
      for (int b = 0; b < BMB; ++b) {
        f32x4_t pr = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NQ; ++q) mma_rank16<Tag>(pr, WF::operand(wv[u][q]), hf[b][q]);
        O::store4(ry, yoff(b, nb + 4 * grp), cv[u][b] + pr);
      }
    }
  };
  wf_t wvA[NBU][NQ], wvB[NBU][NQ];
  f32x4_t cvA[NBU][BMB], cvB[NBU][BMB];
  // two stages in flight; a stage past the last loads nothing and its
  // columns (>= ce) store nothing, so the loop body has no exit in the middle
  if (nst > 0) {
    load2(wvA, cvA, 0);
    for (int k = 0; k < nst; k += 2) {
      load2(wvB, cvB, k + 1);
      sched_fence();
      comp2(wvA, cvA, k);
      sched_fence();
      load2(wvA, cvA, k + 2);
      sched_fence();
      comp2(wvB, cvB, k + 1);
      sched_fence();
    }
  }
}

// expand_stream_walk for the slot's rank-block count nq (a wave-uniform
// value), so each tile runs exactly the MFMAs its rank needs.
template <class Tag, class YT, int BMB, int RBM, int NBU, int NW>
__device__ __forceinline__ void expand_stream_cols(int nq, const uint4 (&hf)[BMB][RBM], const uint32_t (&yrow)[BMB],
                                                   const bool (&tok_ok)[BMB], rsrc_t ry, rsrc_t rb, int ldb, int cb,
                                                   int ce, int rho) {
#define LORA_WALK(NQ) expand_stream_walk<Tag, YT, BMB, RBM, NQ, NBU, NW>(hf, yrow, tok_ok, ry, rb, ldb, cb, ce, rho)
  switch (nq) {
    case 0: break;
    case 1: LORA_WALK(1); break;
    case 2: if constexpr (RBM >= 2) LORA_WALK(2); break;
    case 3: if constexpr (RBM >= 4) LORA_WALK(3); break;
    case 4: if constexpr (RBM >= 4) LORA_WALK(4); break;
    case 5: if constexpr (RBM >= 8) LORA_WALK(5); break;
    case 6: if constexpr (RBM >= 8) LORA_WALK(6); break;
    case 7: if constexpr (RBM >= 8) LORA_WALK(7); break;
    default: if constexpr (RBM >= 8) LORA_WALK(8); break;
  }
#undef LORA_WALK
}

// Streaming form of expand_fused (bf16/f32 b rows 4-element aligned, h rows
// 16-byte aligned, y below 2 GiB). A workgroup owns one tile (16*BMB tokens
// of one slot) and a chunk of one output slice (chunk_cols columns, walked
// 64*NBU columns per stage by the 4 waves, next stage's loads in flight while
// the current one is multiplied). Consecutive workgroups take the chunks of
// one tile, so the rows being updated at any time are few. Loads and stores
// go through buffer descriptors: masked lanes (tokens past the tile, columns
// past the slice) use an out-of-range offset.
template <class Tag, class YT, int BMB, int RBM, int NBU>
__global__ __launch_bounds__(256) void slot_expand_stream_kernel(ExpandArgs p) {
  using E = typename Tag::elem;
  constexpr int ES = sizeof(E);
  constexpr int64_t YES = sizeof(YT);
  constexpr int TB = 16 * BMB;
  __shared__ Tile sh_tile;
  __shared__ int sh_tok[TB];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int ti = blockIdx.x / p.total_chunks;
  const int ch = blockIdx.x - ti * p.total_chunks;
  int slice = 0;
  while (slice + 1 < p.n_slices && ch >= p.chunk_begin[slice + 1]) ++slice;
  const int64_t width = p.slice_w[slice];
  const int64_t off = p.slice_off[slice];
  const int64_t c_begin = (int64_t)(ch - p.chunk_begin[slice]) * p.chunk_cols;
  const int64_t c_end = (c_begin + p.chunk_cols < width) ? c_begin + p.chunk_cols : width;

  if (wave == 0) {
    const Tile tl = find_tile(ti, TB, p.counts, p.offsets, p.S);
    if (lane == 0) sh_tile = tl;
  }
  __syncthreads();
  const Tile tl = sh_tile;
  if (tl.slot < 0) return;
  const int rho = clamp_rank(p.ranks[tl.slot], p.r_max);
  if (threadIdx.x < TB) sh_tok[threadIdx.x] = (static_cast<int>(threadIdx.x) < tl.len) ? p.sorted[tl.start + threadIdx.x] : 0;
  __syncthreads();
  const float sc = p.scalings[tl.slot];
  const int nq = (rho + 15) / 16;

  // (sc * h)^T operand fragments of the tile's tokens; ranks >= rho read as 0
  uint4 hf[BMB][RBM];
  uint32_t yrow[BMB];
  bool tok_ok[BMB];
#pragma unroll
  for (int b = 0; b < BMB; ++b) {
    tok_ok[b] = 16 * b + col < tl.len;
    const int t = sh_tok[16 * b + col];
    yrow[b] = static_cast<uint32_t>(((int64_t)t * p.ldy + off) * YES);
    const float* hrow = p.h + (int64_t)t * p.hs0 + (int64_t)slice * p.hs1;
#pragma unroll
    for (int q = 0; q < RBM; ++q) {
      f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int j = 16 * q + 4 * grp;
      if (tok_ok[b] && j < rho) {
        if (j + 4 <= rho) {
          v = ld16f(hrow + j);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < rho) v[e] = hrow[j + e];
        }
      }
      v *= sc;
      hf[b][q] = split_frag<Tag>(v);
    }
  }

  const rsrc_t ry = make_rsrc(p.y, p.y_bytes);
  const rsrc_t rb = make_rsrc(static_cast<const E*>(p.b) + (int64_t)tl.slot * p.bs0 + off * p.bs1,
                              width * p.bs1 * ES);
  // column indices fit 32 bits (the host checks the descriptors' spans)
  expand_stream_cols<Tag, YT, BMB, RBM, NBU, 4>(nq, hf, yrow, tok_ok, ry, rb, static_cast<int>(p.bs1),
                                            static_cast<int>(c_begin), static_cast<int>(c_end), rho);
}

// One-launch apply_linear for small batches: the rank intermediate never
// leaves the chip. A workgroup owns a tile of up to 16 grouped tokens of one
// slot and a chunk of chunk_cols columns of one output slice. Its NW waves
// first contract the slice's adapter rows (the slot's whole rank) with the
// tile's x rows, each wave over one contiguous range of the feature axis
// (PipeShrink); the partial sums meet in LDS, and every wave adds them up in
// wave order, scales them by the slot's scaling and keeps them as (sc*h)^T
// operand fragments. The waves then walk the chunk's columns as the streaming
// expand does. Every chunk of a tile recomputes its slice's h; the x and
// adapter rows it re-reads come from L2, because the work items of one tile
// go to one XCD (workgroup ids are dealt round-robin to the 8 XCDs; item
// (tile, chunk) has id 8 * (chunk + total_chunks * (tile / 8)) + tile % 8).
// With NW = 4 the feature ranges and the summation order are those of the
// pipelined shrink, so y gets the bits of the two-launch path. Needs the
// descriptors of both the pipelined shrink and the streaming expand.
template <class Tag, class YT, int RBM, int NW, int U, int NBU>
__global__ __launch_bounds__(64 * NW) void slot_apply_kernel(ShrinkArgs ps, ExpandArgs pe) {
  using E = typename Tag::elem;
  constexpr int ES = sizeof(E);
  constexpr int64_t YES = sizeof(YT);
  using PS = PipeShrink<Tag, 1, RBM, U>;
  constexpr int RBYTES = NW * RBM * 64 * 16;
  // the staging tiles share their memory with the partial sums
  __shared__ __attribute__((aligned(16))) char shr[NW * PS::SBYTES > RBYTES ? NW * PS::SBYTES : RBYTES];
  auto red = reinterpret_cast<f32x4_t(*)[RBM][64]>(shr);
  __shared__ Tile sh_tile;
  __shared__ int sh_tok[16];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int tc = pe.total_chunks;
  const int kx = static_cast<int>(blockIdx.x >> 3);
  const int ti = (kx / tc) * 8 + static_cast<int>(blockIdx.x & 7);
  const int ch = kx - (kx / tc) * tc;
  int slice = 0;
  while (slice + 1 < pe.n_slices && ch >= pe.chunk_begin[slice + 1]) ++slice;
  const int64_t width = pe.slice_w[slice];
  const int64_t off = pe.slice_off[slice];
  const int64_t c_begin = (int64_t)(ch - pe.chunk_begin[slice]) * pe.chunk_cols;
  const int64_t c_end = (c_begin + pe.chunk_cols < width) ? c_begin + pe.chunk_cols : width;

  if (wave == 0) {
    const Tile tl = find_tile(ti, 16, ps.counts, ps.offsets, ps.S);
    if (lane == 0) sh_tile = tl;
  }
  __syncthreads();
  const Tile tl = sh_tile;
  if (tl.slot < 0) return;
  const int rho = clamp_rank(ps.ranks[tl.slot], ps.r_max);
  if (rho == 0) return;  // the slot adds nothing
  if (threadIdx.x < 16) sh_tok[threadIdx.x] = (static_cast<int>(threadIdx.x) < tl.len) ? ps.sorted[tl.start + threadIdx.x] : 0;
  __syncthreads();

  // shrink: rows >= rho and tokens past the tile load as zero, so every
  // partial sum past the slot's rank or the tile is +0
  f32x4_t acc[1][RBM];
#pragma unroll
  for (int q = 0; q < RBM; ++q) acc[0][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nch = static_cast<int>((ps.K + PS::CH - 1) / PS::CH);
  const int per = (nch + NW - 1) / NW;
  const int cbeg = wave * per;
  const int cend = (cbeg + per < nch) ? cbeg + per : nch;
  PS::run(acc, ps, sh_tok, tl.len, tl.slot, slice, 0, rho, cbeg, cend, shr + wave * PS::SBYTES);
  if constexpr (PS::LIN) __syncthreads();
#pragma unroll
  for (int q = 0; q < RBM; ++q) red[wave][q][lane] = acc[0][q];
  __syncthreads();

  // lane (col, grp) now finds h[token col][16q + 4grp + i] in red[.][q][lane]:
  // exactly the operand fragment the expand needs
  const float sc = pe.scalings[tl.slot];
  uint4 hf[1][RBM];
#pragma unroll
  for (int q = 0; q < RBM; ++q) {
    f32x4_t v = red[0][q][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w][q][lane];
    v *= sc;
    hf[0][q] = split_frag<Tag>(v);
  }
  const bool tok_ok[1] = {col < tl.len};
  const uint32_t yrow[1] = {static_cast<uint32_t>(((int64_t)sh_tok[col] * pe.ldy + off) * YES)};
  const rsrc_t ry = make_rsrc(pe.y, pe.y_bytes);
  const rsrc_t rb = make_rsrc(static_cast<const E*>(pe.b) + (int64_t)tl.slot * pe.bs0 + off * pe.bs1,
                              width * pe.bs1 * ES);
  expand_stream_cols<Tag, YT, 1, RBM, NBU, NW>((rho + 15) / 16, hf, yrow, tok_ok, ry, rb, static_cast<int>(pe.bs1),
                                           static_cast<int>(c_begin), static_cast<int>(c_end), rho);
}

// Column-band form of expand_fused (many tokens). A workgroup owns a piece
// of one slot's grouped tokens (at most kBandTokens) and a band of
// kBandCols = 256 columns of one output slice; wave w keeps the weight
// fragments of the band's columns [64w, 64w + 64) in registers. Per 16-token
// tile: the tile's (sc * h)^T operand fragments are built once per workgroup
// (wave w loads and converts rank blocks w, w + 4, ... one tile ahead) and
// shared through LDS; every wave multiplies them with its weight fragments
// into a shared LDS output tile; after one barrier wave w reads, adds and
// writes rows [4w, 4w + 4) of the tile over the band, one whole row segment
// (1 KB in float32) per instruction. Fragment and output tiles are double
// buffered, so one barrier per tile orders every LDS access: a buffer is
// written for tile k + 2 only after every wave has passed the barrier of
// tile k + 1, i.e. finished with tile k. Tiles past the piece load nothing
// and store nothing (masked offsets), and every wave runs the same number of
// barriers. Work items (piece, band) go to the XCDs in groups of kBandGroup
// consecutive items (mostly bands of one piece, which read the same h rows
// and weights), so those are re-read from one XCD's L2.
constexpr int kBandCols = 256;
// consecutive work items per XCD group (prefill, r_max 128 / 64: groups of
// 2, 4, 8 -> 267.2 / 258.9, 267.4 / 262.6, 272.3 / 265.5 us)
constexpr int kBandGroup = 2;

template <class Tag, class YT, int RBM>
__global__ __launch_bounds__(256) void slot_expand_band_kernel(ExpandArgs p) {
  constexpr int kBandTokens = RBM >= 8 ? 256 : 64;
  using E = typename Tag::elem;
  constexpr int ES = sizeof(E);
  constexpr int64_t YES = sizeof(YT);
  using WF = WFrag<Tag>;
  using wf_t = typename WF::type;
  using O = Out<YT>;
  constexpr int NW = 4;
  constexpr int NBW = kBandCols / (16 * NW);  // column blocks per wave
  constexpr int LDW = kBandCols + 4;          // LDS row pitch (floats)
  constexpr int R = 16 / NW;                  // rows a wave writes per tile
  constexpr int TILE = 16 * LDW;
  constexpr int QW = (RBM + NW - 1) / NW;     // rank blocks a wave converts per tile
  static_assert(kBandCols == 64 * 4, "one 16-byte piece per lane and row");
  __shared__ __attribute__((aligned(16))) float lds[2 * TILE];
  __shared__ uint4 hfs[2][RBM][64];           // fragment tiles
  __shared__ Tile sh_tile;
  __shared__ int sh_tok[kBandTokens];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int col = lane & 15;
  const int grp = lane >> 4;
  constexpr int G = kBandGroup;
  const int kx = static_cast<int>(blockIdx.x >> 3);
  const int item = ((kx / G) * 8 + static_cast<int>(blockIdx.x & 7)) * G + kx % G;
  if (item >= p.n_work) return;
  const int pi = item / p.total_chunks;
  const int ch = item - pi * p.total_chunks;
  int slice = 0;
  while (slice + 1 < p.n_slices && ch >= p.chunk_begin[slice + 1]) ++slice;
  const int64_t width = p.slice_w[slice];
  const int64_t off = p.slice_off[slice];
  const int c0 = (ch - p.chunk_begin[slice]) * kBandCols;

  if (wave == 0) {
    const Tile tl = find_tile(pi, kBandTokens, p.counts, p.offsets, p.S);
    if (lane == 0) sh_tile = tl;
  }
  __syncthreads();
  const Tile tl = sh_tile;
  if (tl.slot < 0) return;
  const int rho = clamp_rank(p.ranks[tl.slot], p.r_max);
  const int nq = (rho + 15) / 16;
  if (nq == 0) return;
  for (int i = threadIdx.x; i < kBandTokens; i += 256) sh_tok[i] = (i < tl.len) ? p.sorted[tl.start + i] : 0;
  __syncthreads();

  const float sc = p.scalings[tl.slot];
  const rsrc_t rb = make_rsrc(static_cast<const E*>(p.b) + (int64_t)tl.slot * p.bs0 + off * p.bs1,
                              width * p.bs1 * ES);
  const int ldb = static_cast<int>(p.bs1);
  const rsrc_t ry = make_rsrc(p.y, p.y_bytes);
  const rsrc_t rh = make_rsrc(p.h, p.h_bytes);
  const int ntiles = (tl.len + 15) / 16;
  const int lc = lane * 4;  // this lane's column of the band in the row-linear pass
  const bool col_ok = c0 + lc < width;

  auto walk = [&](auto nq_tag) {
    constexpr int NQ = decltype(nq_tag)::value;
    wf_t w[NBW][NQ];
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
      const int n = c0 + (wave * NBW + u) * 16 + col;
      const bool ok = n < width;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int j0 = 16 * q + 4 * grp;
        w[u][q] = WF::bload(rb, ok ? static_cast<uint32_t>((n * ldb + j0) * ES) : kOOB, j0, rho);
      }
    }
    struct Tl {
      f32x4_t hv[QW];  // this wave's rank blocks q = wave + NW*i of the tile's h
      f32x4_t cv[R];   // this wave's output rows (row-linear pieces)
      uint32_t yo[R];  // their offsets (kOOB when masked)
    };
    auto load_tile = [&](Tl& T, int t) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int tix = 16 * t + wave * R + i;
        const bool ok = t < ntiles && tix < tl.len && col_ok;
        const int tok = sh_tok[ok ? tix : 0];
        T.yo[i] = ok ? static_cast<uint32_t>(((int64_t)tok * p.ldy + off + c0 + lc) * YES) : kOOB;
        T.cv[i] = O::load4(ry, T.yo[i]);
      }
      const int tix = 16 * t + col;
      const bool tok_ok = t < ntiles && tix < tl.len;
      const int tok = sh_tok[tok_ok ? tix : 0];
      const uint32_t hbase = static_cast<uint32_t>(((int64_t)tok * p.hs0 + (int64_t)slice * p.hs1) * 4);
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const int q = wave + NW * i;
        const int j = 16 * q + 4 * grp;
        T.hv[i] = __builtin_bit_cast(f32x4_t, bload16(rh, (q < NQ && tok_ok && j < rho) ? hbase + j * 4 : kOOB));
      }
    };
    // this wave's rank blocks of the tile's h -> operand fragments in LDS
    auto put_frags = [&](const Tl& T, int buf) {
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const int q = wave + NW * i;
        if (q < NQ) {
          const int j = 16 * q + 4 * grp;
          f32x4_t v = T.hv[i];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (j + e < rho) ? v[e] : 0.f;  // padding may hold NaN
          v *= sc;
          hfs[buf][q][lane] = split_frag<Tag>(v);
        }
      }
    };
    auto comp_tile = [&](const Tl& T, int buf, const Tl& Tn) {
      uint4 hf[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) hf[q] = hfs[buf][q][lane];
      float* tile = lds + buf * TILE;
#pragma unroll
      for (int u = 0; u < NBW; ++u) {
        f32x4_t pr = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NQ; ++q) mma_rank16<Tag>(pr, WF::operand(w[u][q]), hf[q]);
        // lane holds columns 16u + 4grp .. +3 (of this wave's 64) of token col
        *reinterpret_cast<f32x4_t*>(tile + col * LDW + (wave * NBW + u) * 16 + 4 * grp) = pr;
      }
      put_frags(Tn, buf ^ 1);  // the next tile's fragments
      __syncthreads();
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const f32x4_t pr = *reinterpret_cast<const f32x4_t*>(tile + (wave * R + i) * LDW + lc);
        O::store4(ry, T.yo[i], T.cv[i] + pr);
      }
    };
    Tl A, B;
    load_tile(A, 0);
    put_frags(A, 0);
    load_tile(B, 1);
    __syncthreads();  // tile 0's fragments
    for (int t = 0; t < ntiles; t += 2) {
      comp_tile(A, 0, B);
      sched_fence();
      load_tile(A, t + 2);
      sched_fence();
      comp_tile(B, 1, A);
      sched_fence();
      load_tile(B, t + 3);
      sched_fence();
    }
  };
  switch (nq) {
    case 1: walk(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (RBM >= 2) walk(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (RBM >= 4) walk(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (RBM >= 4) walk(std::integral_constant<int, 4>{}); break;
    case 5: if constexpr (RBM >= 8) walk(std::integral_constant<int, 5>{}); break;
    case 6: if constexpr (RBM >= 8) walk(std::integral_constant<int, 6>{}); break;
    case 7: if constexpr (RBM >= 8) walk(std::integral_constant<int, 7>{}); break;
    default: if constexpr (RBM >= 8) walk(std::integral_constant<int, 8>{}); break;
  }
}

// ---------------------------------------------------------------------------
// gather_shrink: h[t, 0, j] = a[s, j, ids[t]] (exact), +0.0 for ids outside [0, V)
// ---------------------------------------------------------------------------

template <class E>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ ids, const E* __restrict__ a,
                                                     int64_t as0, int64_t as1, int64_t as2, int64_t V,
                                                     const int32_t* __restrict__ token_slot,
                                                     const int32_t* __restrict__ ranks, int T, int S, int r_max,
                                                     float* __restrict__ h, int64_t hs0) {
  const int t = blockIdx.x * 4 + wave_id();
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const int s = token_slot[t];
  if (s < 0 || s >= S) return;
  const int rho = clamp_rank(ranks[s], r_max);
  if (rho == 0) return;
  const int64_t id = ids[t];
  const bool valid = id >= 0 && id < V;
  const E* src = a + (int64_t)s * as0 + (valid ? id : 0) * as2;
  float* dst = h + (int64_t)t * hs0;
  for (int j = lane; j < rho; j += 64) {
    float v = 0.0f;
    if (valid) {
      if constexpr (sizeof(E) == 2)
        v = __uint_as_float(static_cast<uint32_t>(src[j * as1]) << 16);
      else
        v = src[j * as1];
    }
    dst[j] = v;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int check_addressing(const lora_addressing* addr, const int32_t* ranks) {
  if (!addr) return LORA_ERR_NULL;
  if (addr->T < 0 || addr->S < 0) return LORA_ERR_SHAPE;
  if (addr->S > kMaxSlots) return LORA_ERR_LIMIT;
  if (addr->T > 0 && (!addr->token_slot || !addr->sorted_tokens)) return LORA_ERR_NULL;
  if (!addr->counts && addr->S > 0) return LORA_ERR_NULL;
  if (!addr->offsets) return LORA_ERR_NULL;
  if (addr->S > 0 && !ranks) return LORA_ERR_NULL;
  return LORA_OK;
}

static int tile_bmb(int T) { return T >= 1024 ? 4 : 1; }

// Token tiles of the per-tile shrinks (16 tokens: bmb 1, or 64: bmb 4). A
// workgroup streams its tile's x rows and its rank block's adapter rows over
// the whole feature axis, and a CU streams only so fast, so the time follows
// the busiest CU: rounds of 256 workgroups times rows per workgroup, with the
// tokens taken as spread evenly over the S slots. Ties go to 16-token tiles.
// Measured (bf16, K 4096, slices 4096 + 1024 + 1024, ranks 0-64, four rank
// blocks per workgroup, us for 16- / 64-token tiles): 16 slots at 512 / 768 /
// 1024 tokens 14.8 / 22.5, 15.6 / 24.5, -; 32 slots at 1024 / 1152 / 1536
// tokens 16.5 / 23.0, 26.3 / 23.1, 26.8 / 25.1; 64 slots at 2048 / 3072 29.8 /
// 24.9, 36.8 / 29.3; 128 slots at 1024 / 2048 / 4096 / 5120 / 6144 30.4 /
// 36.0, 32.4 / 37.5, 42.1 / 42.1, 48.2 / 44.9, 55.4 / 46.0 (4608 tokens, the
// one miss: 42.3 / 43.2).
static int shrink_tile_bmb(int64_t T, int64_t S, int n_slices, int64_t row_chunks, int64_t a_rows) {
  if (T < 1024 || S < 1) return 1;
  auto cost = [&](int64_t bmb) {
    const int64_t wgs = S * ceil_div(T, 16 * bmb * S) * n_slices * row_chunks;
    return ceil_div(wgs, 256) * (16 * bmb + a_rows);
  };
  return cost(4) < cost(1) ? 4 : 1;
}

// 64-token tiles (bmb 4) come only with four rank blocks (rb 4): both are
// taken from 1024 tokens, rb 4 from 512. The grid covers every unit the
// kernels find on the device: the slots' tiles number at most
// ceil(T / tile) + S (each slot's last tile may be partial), and row_chunks
// covers the largest clamped rank.
template <class Tag>
static void launch_shrink(const ShrinkArgs& a, int bmb, int rb, int64_t tiles, bool pipe, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(tiles * a.n_slices * a.row_chunks));
  if (pipe) {
    const dim3 pgrid(static_cast<unsigned>(round_up(tiles, 8 * kShrinkGroup) * a.n_slices * a.row_chunks));
    if (bmb == 4)
      launch((slot_shrink_pipe_kernel<Tag, 4, 4, 2, false>), pgrid, dim3(256), 0, st, a);
    else if (rb == 4)
      launch((slot_shrink_pipe_kernel<Tag, 1, 4, 2, false>), pgrid, dim3(256), 0, st, a);
    else
      launch((slot_shrink_pipe_kernel<Tag, 1, 1, 4, true>), pgrid, dim3(256), 0, st, a);
    return;
  }
  if (bmb == 4)
    launch((slot_shrink_kernel<Tag, 4, 4>), grid, dim3(256), 0, st, a);
  else if (rb == 4)
    launch((slot_shrink_kernel<Tag, 1, 4>), grid, dim3(256), 0, st, a);
  else
    launch((slot_shrink_kernel<Tag, 1, 1>), grid, dim3(256), 0, st, a);
}

template <class Tag, class YT, int BMB>
static void launch_expand_b(const ExpandArgs& a, int rbm, dim3 grid, hipStream_t st) {
  switch (rbm) {
    case 1: launch((slot_expand_kernel<Tag, YT, BMB, 1>), grid, dim3(256), 0, st, a); break;
    case 2: launch((slot_expand_kernel<Tag, YT, BMB, 2>), grid, dim3(256), 0, st, a); break;
    case 4: launch((slot_expand_kernel<Tag, YT, BMB, 4>), grid, dim3(256), 0, st, a); break;
    default: launch((slot_expand_kernel<Tag, YT, BMB, 8>), grid, dim3(256), 0, st, a); break;
  }
}

// Streaming expand: (BMB, NBU) per rank-block count, chosen to keep the
// weight and output fragments of two stages within the register budget.
template <class Tag, class YT, int BMB>
static void launch_expand_stream(ExpandArgs a, int rbm, int64_t tiles, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(tiles * a.total_chunks));
  switch (rbm) {
    case 1: launch((slot_expand_stream_kernel<Tag, YT, BMB, 1, 4>), grid, dim3(256), 0, st, a); break;
    case 2: launch((slot_expand_stream_kernel<Tag, YT, BMB, 2, 4>), grid, dim3(256), 0, st, a); break;
    case 4: launch((slot_expand_stream_kernel<Tag, YT, BMB, 4, 2>), grid, dim3(256), 0, st, a); break;
    default: launch((slot_expand_stream_kernel<Tag, YT, BMB, 8, 2>), grid, dim3(256), 0, st, a); break;
  }
}

// Column-band expand: pieces of 256 tokens for slots with more than 64 rank
// columns (the workgroup's weight fragments span 8 rank blocks), 64 tokens
// otherwise (kernel-side: kBandTokens).
static int64_t band_piece_tokens(int rbm) { return rbm >= 8 ? 256 : 64; }

template <class Tag, class YT>
static void launch_expand_band(ExpandArgs a, int rbm, int64_t pieces, hipStream_t st) {
  a.n_work = static_cast<int>(pieces * a.total_chunks);
  const dim3 grid(static_cast<unsigned>(round_up(a.n_work, 8 * kBandGroup)));
  switch (rbm) {
    case 1: launch((slot_expand_band_kernel<Tag, YT, 1>), grid, dim3(256), 0, st, a); break;
    case 2: launch((slot_expand_band_kernel<Tag, YT, 2>), grid, dim3(256), 0, st, a); break;
    case 4: launch((slot_expand_band_kernel<Tag, YT, 4>), grid, dim3(256), 0, st, a); break;
    default: launch((slot_expand_band_kernel<Tag, YT, 8>), grid, dim3(256), 0, st, a); break;
  }
}

template <class Tag, class YT>
static void launch_expand(const ExpandArgs& a, int bmb, int rbm, int64_t tiles, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(tiles * a.total_chunks));
  if (bmb == 4)
    launch_expand_b<Tag, YT, 4>(a, rbm, grid, st);
  else
    launch_expand_b<Tag, YT, 1>(a, rbm, grid, st);
}

// Calls f(Tag{}, YT{}) for the expand weights' dtype and the output's: bf16
// or f32 weights into a float32 y, bf16 weights into a bfloat16 y (the host
// checks refuse bfloat16 y with f32 weights).
template <class F>
static void with_expand_types(int32_t b_dtype, int32_t y_dtype, F&& f) {
  if (b_dtype == LORA_BF16) {
    if (y_dtype == LORA_BF16)
      f(BF16{}, uint16_t{});
    else
      f(BF16{}, float{});
  } else {
    f(F32{}, float{});
  }
}

// One-launch apply_linear: 4 waves per workgroup (the feature ranges of the
// pipelined shrink, hence its bits), U feature chunks per stage in the shrink
// (one at rank 128, to stay within the register budget), 2 column blocks per
// wave and stage in the expand.
template <class Tag, class YT>
static void launch_apply(const ShrinkArgs& ps, const ExpandArgs& pe, int rbm, int64_t tiles, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(round_up(tiles, 8) * pe.total_chunks));
  const dim3 block(256);
  switch (rbm) {
    case 1: launch((slot_apply_kernel<Tag, YT, 1, 4, 2, 2>), grid, block, 0, st, ps, pe); break;
    case 2: launch((slot_apply_kernel<Tag, YT, 2, 4, 2, 2>), grid, block, 0, st, ps, pe); break;
    case 4: launch((slot_apply_kernel<Tag, YT, 4, 4, 2, 2>), grid, block, 0, st, ps, pe); break;
    default: launch((slot_apply_kernel<Tag, YT, 8, 4, 1, 2>), grid, block, 0, st, ps, pe); break;
  }
}

// Column chunk of the one-launch apply_linear for a batch, or 0 where the two
// launches are faster. A one-launch workgroup streams its slice's whole
// adapter rows through one CU, so the form only pays while every workgroup
// gets a CU of its own: at least kApplyMinTokens tokens, and token tiles times
// 1024-column chunks within the CU count, the tiles estimated as if the tokens
// spread evenly over the S slots.
// Measured (bf16, K 4096, slices 4096 + 1024 + 1024, ranks 0-64; two launches
// against one): 32 slots at 256 tokens 25.9 / 26.9 us, 512: 31.3 / 29.4
// (1024 columns); 640 / 768 / 896 / 1024 tokens, where only 2048-column
// chunks fit: 32.7 / 39.3, 32.2 / 39.2, 34.0 / 40.3, 34.9 / 39.7 us; 1536 and
// more tokens, or 128 slots at 512 to 2048 tokens, are a tie or slower
// whatever the chunk (1024, 1536, 2048 or 4096 columns).
constexpr int64_t kApplyMinTokens = 512;
constexpr int64_t kApplyMaxWorkgroups = 256;
constexpr int64_t kApplyCols = 1024;
static int64_t apply_one_launch_cols(int64_t T, int64_t S, const int64_t* out_slices, int32_t num_slices) {
  if (T < kApplyMinTokens || S < 1) return 0;
  const int64_t tiles = S * ceil_div(T, 16 * S);
  int64_t chunks = 0;
  for (int i = 0; i < num_slices; ++i) chunks += ceil_div(out_slices[i], kApplyCols);
  return tiles * chunks <= kApplyMaxWorkgroups ? kApplyCols : 0;
}

// Device address of `scratch` on the current device, looked up on the first
// call from each device and kept (each device's copy has its own address).
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LORA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LORA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LORA_OK;
}

}  // namespace lora

using namespace lora;

extern "C" int lora_addressing_build(const lora_addressing* addr, const int32_t* ranks, int32_t r_max, void* stream) {
  const int rc = check_addressing(addr, ranks);
  if (rc != LORA_OK) return rc;
  if (r_max < 1 || r_max > 128) return LORA_ERR_RANK;
  if (addr->S > 0 && !addr->counts) return LORA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // up to 1024 tokens one token per thread; one workgroup per 1024-token
  // chunk up to kGroupChunkMaxT tokens (each holds every token's key in
  // registers); one workgroup beyond
  if (addr->T <= kGroupSmallMaxT) {
    launch(group_small_kernel, dim3(1), dim3(1024), 0, st, addr->token_slot, addr->T, addr->S, ranks, r_max,
           addr->counts, addr->offsets, addr->sorted_tokens);
  } else if (addr->T <= kGroupChunkMaxT) {
    const int chunks = addr->T > 0 ? static_cast<int>(ceil_div(addr->T, 1024)) : 1;
    launch(group_chunk_kernel, dim3(static_cast<unsigned>(chunks)), dim3(1024), 0, st, addr->token_slot, addr->T,
           addr->S, ranks, r_max, addr->counts, addr->offsets, addr->sorted_tokens);
  } else {
    launch(group_kernel, dim3(1), dim3(1024), 0, st, addr->token_slot, addr->T, addr->S, ranks, r_max,
           addr->counts, addr->offsets, addr->sorted_tokens);
  }
  return launch_status();
}

// Host-side argument checks of lora_shrink (status; nothing is launched).
static int shrink_checks(const lora_mat* x, const lora_t3* a, const lora_addressing* addr, const int32_t* ranks,
                         int32_t num_slices, int32_t r_max, const lora_t3* h) {
  if (!x || !a || !h) return LORA_ERR_NULL;
  int rc = check_addressing(addr, ranks);
  if (rc != LORA_OK) return rc;
  if (r_max < 1 || r_max > 128) return LORA_ERR_RANK;
  if (num_slices < 1 || num_slices > kMaxSlices) return LORA_ERR_SHAPE;
  if (!valid_dims(x) || !valid_dims(a) || !valid_dims(h)) return LORA_ERR_SHAPE;
  const int64_t T = addr->T, S = addr->S, K = x->cols;
  if (x->rows != T) return LORA_ERR_SHAPE;
  if (a->d0 != S || a->d1 != (int64_t)num_slices * r_max || a->d2 != K) return LORA_ERR_SHAPE;
  if (h->d0 != T || h->d1 != num_slices || h->d2 != r_max) return LORA_ERR_SHAPE;
  if (!float_dtype_ok(x->dtype) || a->dtype != x->dtype || h->dtype != LORA_F32) return LORA_ERR_DTYPE;
  if ((T * K > 0 && !x->ptr) || (S * K > 0 && !a->ptr) || (T > 0 && !h->ptr)) return LORA_ERR_NULL;
  const size_t es = elem_size(x->dtype);
  if (K % vec_elems(x->dtype) != 0) return LORA_ERR_SHAPE;
  if (T * K > 0 && check_rowmajor_stream(x) != LORA_OK) return LORA_ERR_STRIDE;
  if (a->s2 != 1 || (a->s1 * (int64_t)es) % 16 != 0 || (a->s0 * (int64_t)es) % 16 != 0 || !aligned(a->ptr, 16))
    return LORA_ERR_STRIDE;
  if (h->s2 != 1) return LORA_ERR_STRIDE;
  return LORA_OK;
}

// Kernel arguments of the shrink (after shrink_checks); h may be null (the
// one-launch apply_linear keeps h on chip).
static ShrinkArgs shrink_args(const lora_mat* x, const lora_t3* a, const lora_addressing* addr, const int32_t* ranks,
                              int32_t num_slices, int32_t r_max, const lora_t3* h) {
  const size_t es = elem_size(x->dtype);
  ShrinkArgs p{};
  p.x = x->ptr;
  p.ldx = x->stride_row;
  p.a = a->ptr;
  p.as0 = a->s0;
  p.as1 = a->s1;
  if (h) {
    p.h = static_cast<float*>(h->ptr);
    p.hs0 = h->s0;
    p.hs1 = h->s1;
    p.h_vec = h->s1 % 4 == 0 && h->s0 % 4 == 0 && aligned(h->ptr, 16);
  }
  p.counts = addr->counts;
  p.offsets = addr->offsets;
  p.sorted = addr->sorted_tokens;
  p.ranks = ranks;
  p.K = x->cols;
  p.S = static_cast<int>(addr->S);
  p.r_max = r_max;
  p.n_slices = num_slices;
  p.x_bytes = addr->T * x->stride_row * (int64_t)es;
  return p;
}

// x and one slot's adapter rows fit 2 GiB buffer descriptors (pipelined and
// row-split shrinks, one-launch apply_linear).
static bool shrink_desc_ok(const lora_mat* x, const lora_t3* a, int64_t T, int32_t num_slices, int32_t r_max) {
  const int64_t es = static_cast<int64_t>(elem_size(x->dtype));
  return T * x->stride_row * es <= kMaxBufferBytes && (int64_t)num_slices * r_max * a->s1 * es <= kMaxBufferBytes &&
         x->cols < (int64_t(1) << 30);
}

extern "C" int lora_shrink(const lora_mat* x, const lora_t3* a, const lora_addressing* addr, const int32_t* ranks,
                           int32_t num_slices, int32_t r_max, const lora_t3* h, void* stream) {
  const int rc = shrink_checks(x, a, addr, ranks, num_slices, r_max, h);
  if (rc != LORA_OK) return rc;
  const int64_t T = addr->T, S = addr->S;
  if (T == 0 || S == 0) return LORA_OK;
  // four 16-row rank blocks per workgroup from 512 tokens (32 slots at 512 /
  // 1024 tokens: 16.9 / 16.5 us against 17.3 / 27.8 us with one; at 256
  // tokens one block is faster, 12.3 against 15.9 us)
  const int rb = (T >= 512) ? 4 : 1;
  ShrinkArgs p = shrink_args(x, a, addr, ranks, num_slices, r_max, h);
  p.row_chunks = static_cast<int>(ceil_div(r_max, 16 * rb));
  const int bmb = shrink_tile_bmb(T, S, num_slices, p.row_chunks, std::min<int64_t>(16 * rb, round_up(r_max, 16)));
  const int64_t tiles = ceil_div(T, 16 * bmb) + S;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Schedule, from the shapes: the row-split kernel for bf16 batches of 1024
  // tokens or more whose grid (token tiles, counting every slot of the table
  // as used, times groups of 16 (slice, rank block) pairs) fills the chip
  // once, at least 256 workgroups; the pipelined kernel for the others; the
  // general kernel (no buffer descriptors) where x or one slot's adapter
  // spans more than a 2 GiB descriptor.
  // Measured (us, row-split / pipelined): the prefill batch (16731 tokens in
  // 46 requests over a 128-slot table, K 8192, slices 8192 + 1024 + 1024) at
  // r_max 128 / 64 / 32 / 16: 143-151 / 236, 130 / 176, 127 / 164, 114 / 156.
  // Tokens spread evenly over the slots (K 4096, slices 4096 + 1024 + 1024,
  // r_max 64 / 32; grid as the rule counts it): 32 slots at 8192 tokens (96)
  // 66 / 49, 66 / 44, at 16384 (160) 68 / 70, 66 / 64; 64 slots at 16384
  // (192) 67 / 70, 66 / 63, at 32768 (320) 95 / 134, 71 / 111; 128 slots at
  // 8192 (192) 55 / 50, 55 / 44, at 12288 (224) 64 / 64, 63 / 61, at 16384
  // (256) 68 / 78, 67 / 64, at 24576 (320) 90 / 96, 68 / 84, at 32768 (384)
  // 94 / 131, 71 / 109. A row-split workgroup streams its tile's x rows and
  // up to 8 rank blocks over the whole feature axis (about 60 us at K 4096),
  // so it pays once the pipelined kernel's re-reads take longer.
  constexpr int tt = 8;    // row-split: 128-token tiles
  constexpr int nw = 8;    // row-split: waves per workgroup
  constexpr int ppw = 1;   // row-split: (slice, rank block) pairs per wave
  const bool desc_ok = shrink_desc_ok(x, a, T, num_slices, r_max);
  const int64_t pairs = (int64_t)num_slices * ceil_div(r_max, 16);
  const int64_t rtiles = ceil_div(T, 16 * tt) + S;
  if (desc_ok && x->dtype == LORA_BF16 && T >= 1024 && rtiles * ceil_div(pairs, 16) >= 256) {
    // 8 waves of one pair each, units dealt evenly to the XCDs: the prefill
    // batch at r_max 128 / 64 / 32 143 / 130 / 128 us. Earlier forms (units
    // by tile groups of four per XCD): 4 waves of two pairs 190 / 185 / 132
    // us; 8 waves of two 181 / 158 / 122 (165 at 128 with a slot's pairs split
    // evenly); 8 of one 196 / 193 / 124 (as many units as now, but up to 42 on
    // one XCD's 32 CUs); 8 of three 252 / 159 / 117; 128-feature stages 212 /
    // 181 / 130. With 4 waves: 4 pairs per wave 224 us, 64-token tiles 206-230
    // us (r_max 128).
    p.row_groups = static_cast<int>(ceil_div(pairs, nw * ppw));
    // at most rtiles * row_groups units: 8 runs of at most that / 8 each
    const dim3 grid(static_cast<unsigned>(8 * ceil_div(rtiles * p.row_groups, 8)));
    launch((slot_shrink_rows_kernel<tt, 2, ppw, nw>), grid, dim3(64 * nw), 0, st, p);
    return launch_status();
  }
  const bool pipe = desc_ok;
  if (x->dtype == LORA_BF16)
    launch_shrink<BF16>(p, bmb, rb, tiles, pipe, st);
  else
    launch_shrink<F32>(p, bmb, rb, tiles, pipe, st);
  return launch_status();
}

// Host-side argument checks of lora_expand_fused (status; nothing is
// launched); *O_out = sum of the slice widths.
static int expand_checks(const lora_t3* h, const lora_t3* b, const lora_addressing* addr, const int32_t* ranks,
                         const float* scalings, const lora_mat* y, const int64_t* out_slices, int32_t num_slices,
                         int32_t r_max, int64_t* O_out) {
  if (!h || !b || !y || !out_slices) return LORA_ERR_NULL;
  int rc = check_addressing(addr, ranks);
  if (rc != LORA_OK) return rc;
  if (r_max < 1 || r_max > 128) return LORA_ERR_RANK;
  if (num_slices < 1 || num_slices > kMaxSlices) return LORA_ERR_SHAPE;
  if (!valid_dims(h) || !valid_dims(b) || !valid_dims(y)) return LORA_ERR_SHAPE;
  const int64_t T = addr->T, S = addr->S;
  int64_t O = 0;
  for (int i = 0; i < num_slices; ++i) {
    if (out_slices[i] < 0 || out_slices[i] > kMaxOperand || out_slices[i] % 4 != 0) return LORA_ERR_SHAPE;
    O += out_slices[i];
  }
  if (h->d0 != T || h->d1 != num_slices || h->d2 != r_max) return LORA_ERR_SHAPE;
  if (b->d0 != S || b->d1 != O || b->d2 != r_max) return LORA_ERR_SHAPE;
  if (y->rows != T || y->cols != O) return LORA_ERR_SHAPE;
  // y float32, or bfloat16 (updated in place, one rounding) with bf16 weights
  if (h->dtype != LORA_F32 || !float_dtype_ok(b->dtype) ||
      !(y->dtype == LORA_F32 || (y->dtype == LORA_BF16 && b->dtype == LORA_BF16)))
    return LORA_ERR_DTYPE;
  if ((T > 0 && !h->ptr) || (S * O > 0 && !b->ptr) || (T * O > 0 && !y->ptr) || (S > 0 && !scalings))
    return LORA_ERR_NULL;
  if (h->s2 != 1 || b->s2 != 1) return LORA_ERR_STRIDE;
  if (T * O > 0 && check_rowmajor_stream(y) != LORA_OK) return LORA_ERR_STRIDE;
  *O_out = O;
  return LORA_OK;
}

// Kernel arguments of the expand (after expand_checks), without the column
// chunks; h may be null (the one-launch apply_linear keeps h on chip).
static ExpandArgs expand_args(const lora_t3* h, const lora_t3* b, const lora_addressing* addr, const int32_t* ranks,
                              const float* scalings, const lora_mat* y, int32_t num_slices, int32_t r_max) {
  const size_t es = elem_size(b->dtype);
  ExpandArgs p{};
  if (h) {
    p.h = static_cast<const float*>(h->ptr);
    p.hs0 = h->s0;
    p.hs1 = h->s1;
    p.h_vec = h->s1 % 4 == 0 && h->s0 % 4 == 0 && aligned(h->ptr, 16);
    p.h_bytes = addr->T * h->s0 * 4;
  }
  p.b = b->ptr;
  p.bs0 = b->s0;
  p.bs1 = b->s1;
  p.y = y->ptr;
  p.ldy = y->stride_row;
  p.scalings = scalings;
  p.b_vec = b->s1 % 4 == 0 && b->s0 % 4 == 0 && aligned(b->ptr, 4 * es);
  p.counts = addr->counts;
  p.offsets = addr->offsets;
  p.sorted = addr->sorted_tokens;
  p.ranks = ranks;
  p.S = static_cast<int>(addr->S);
  p.r_max = r_max;
  p.n_slices = num_slices;
  p.y_bytes = addr->T * y->stride_row * static_cast<int64_t>(elem_size(y->dtype));
  return p;
}

// Cuts every output slice into chunks of `cols` columns (the last one of a
// slice shorter); returns the number of chunks.
static int set_chunks(ExpandArgs& p, const int64_t* out_slices, int32_t num_slices, int64_t cols) {
  p.chunk_cols = cols;
  int64_t off = 0;
  int chunks = 0;
  for (int i = 0; i < num_slices; ++i) {
    p.slice_off[i] = off;
    p.slice_w[i] = out_slices[i];
    p.chunk_begin[i] = chunks;
    chunks += static_cast<int>(ceil_div(out_slices[i], cols));
    off += out_slices[i];
  }
  p.chunk_begin[num_slices] = chunks;
  p.total_chunks = chunks;
  return chunks;
}

// y, the slice's weight rows of one slot and their row stride fit the
// streaming expand's 32-bit descriptor offsets, and b rows allow vector loads
// (streaming and column-band expands, one-launch apply_linear).
static bool expand_desc_ok(const ExpandArgs& p, const lora_t3* b, const lora_mat* y, int64_t O) {
  const int64_t es = static_cast<int64_t>(elem_size(b->dtype));
  return p.b_vec && p.y_bytes <= kMaxBufferBytes && O * b->s1 * es <= kMaxBufferBytes &&
         y->stride_row < (int64_t(1) << 30);
}

extern "C" int lora_expand_fused(const lora_t3* h, const lora_t3* b, const lora_addressing* addr,
                                 const int32_t* ranks, const float* scalings, const lora_mat* y,
                                 const int64_t* out_slices, int32_t num_slices, int32_t r_max, void* stream) {
  int64_t O = 0;
  const int rc = expand_checks(h, b, addr, ranks, scalings, y, out_slices, num_slices, r_max, &O);
  if (rc != LORA_OK) return rc;
  const int64_t T = addr->T, S = addr->S;
  if (T == 0 || S == 0 || O == 0) return LORA_OK;
  ExpandArgs p = expand_args(h, b, addr, ranks, scalings, y, num_slices, r_max);
  const int rbm = rank_blocks(r_max);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Schedule, from the shapes: the column-band kernel for 512 tokens or more,
  // the streaming kernel for fewer, both when their descriptors can span y,
  // h and one slot's b with 32-bit offsets and the rows of h and b allow
  // vector loads; else the general kernel. Measured (bf16, float32 y): the
  // prefill batch (16731 tokens, 46 slots, r_max 128 / 64 / 32) 268 / 263 /
  // 247 us band against 285 / 277 / 283 us for a column-owner form with
  // 1024-token pieces and 128-column chunks; 32 slots, ranks up to 64, at
  // 512 / 1024 / 1536 / 2048 tokens 15 / 19 / 22 / 28 us band against 17 / 25
  // / 33 / 37 us for the streaming kernel or the owner form.
  const bool stream_ok = p.h_vec && expand_desc_ok(p, b, y, O);
  const bool band_ok = stream_ok && p.h_bytes <= kMaxBufferBytes;
  if (band_ok && T >= 512) {
    if (set_chunks(p, out_slices, num_slices, kBandCols) == 0) return LORA_OK;
    const int64_t pieces = ceil_div(T, band_piece_tokens(rbm)) + S;
    with_expand_types(b->dtype, y->dtype, [&](auto tag, auto yt) {
      launch_expand_band<decltype(tag), decltype(yt)>(p, rbm, pieces, st);
    });
    return launch_status();
  }
  if (stream_ok) {
    const int bmb = (T >= 1024 && rbm <= 4) ? 2 : 1;
    const int64_t tiles = ceil_div(T, 16 * bmb) + S;
    // about 1024 columns per workgroup, fewer when there are few tiles
    if (set_chunks(p, out_slices, num_slices, tiles >= 256 ? 1024 : 256) == 0) return LORA_OK;
    with_expand_types(b->dtype, y->dtype, [&](auto tag, auto yt) {
      if (bmb == 2)
        launch_expand_stream<decltype(tag), decltype(yt), 2>(p, rbm, tiles, st);
      else
        launch_expand_stream<decltype(tag), decltype(yt), 1>(p, rbm, tiles, st);
    });
    return launch_status();
  }
  if (set_chunks(p, out_slices, num_slices, kExpandCols) == 0) return LORA_OK;
  const int bmb = tile_bmb(static_cast<int>(T));
  const int64_t tiles = ceil_div(T, 16 * bmb) + S;
  with_expand_types(b->dtype, y->dtype, [&](auto tag, auto yt) {
    launch_expand<decltype(tag), decltype(yt)>(p, bmb, rbm, tiles, st);
  });
  return launch_status();
}

// LoraOpsBackend.apply_linear_ (shrink then expand into y; the page lets a
// backend fuse the two). Batches that apply_one_launch_cols accepts run as
// one launch with h kept on chip (slot_apply_kernel), when x, a and b share a
// dtype and the descriptors of both kernels fit; the others as the shrink
// into the caller's h, then the expand, on one stream. Both operations'
// arguments are checked before anything launches.
extern "C" int lora_apply_linear(const lora_mat* x, const lora_t3* a, const lora_t3* b, const lora_addressing* addr,
                                 const int32_t* ranks, const float* scalings, const lora_mat* y,
                                 const int64_t* out_slices, int32_t num_slices, int32_t r_max, const lora_t3* h,
                                 void* stream) {
  int rc = shrink_checks(x, a, addr, ranks, num_slices, r_max, h);
  if (rc != LORA_OK) return rc;
  int64_t O = 0;
  rc = expand_checks(h, b, addr, ranks, scalings, y, out_slices, num_slices, r_max, &O);
  if (rc != LORA_OK) return rc;
  const int64_t T = addr->T, S = addr->S;
  if (T == 0 || S == 0 || O == 0) return LORA_OK;
  const int64_t cols = apply_one_launch_cols(T, S, out_slices, num_slices);
  if (cols > 0 && b->dtype == x->dtype && shrink_desc_ok(x, a, T, num_slices, r_max)) {
    ShrinkArgs ps = shrink_args(x, a, addr, ranks, num_slices, r_max, nullptr);
    ExpandArgs pe = expand_args(nullptr, b, addr, ranks, scalings, y, num_slices, r_max);
    if (expand_desc_ok(pe, b, y, O)) {
      set_chunks(pe, out_slices, num_slices, cols);
      const int64_t tiles = ceil_div(T, 16) + S;
      hipStream_t st = static_cast<hipStream_t>(stream);
      with_expand_types(b->dtype, y->dtype, [&](auto tag, auto yt) {
        launch_apply<decltype(tag), decltype(yt)>(ps, pe, rank_blocks(r_max), tiles, st);
      });
      return launch_status();
    }
  }
  rc = lora_shrink(x, a, addr, ranks, num_slices, r_max, h, stream);
  if (rc != LORA_OK) return rc;
  return lora_expand_fused(h, b, addr, ranks, scalings, y, out_slices, num_slices, r_max, stream);
}

// lora_apply_linear with the rank intermediate in the library's per-device
// scratch instead of a caller workspace: for callers that cannot allocate.
// The kernels and their order are those of lora_apply_linear (bit for bit the
// same results); h needs no clearing, since entries past a slot's rank and of
// inactive tokens are never read.
extern "C" int lora_apply_linear_noalloc(const lora_mat* x, const lora_t3* a, const lora_t3* b,
                                         const lora_addressing* addr, const int32_t* ranks, const float* scalings,
                                         const lora_mat* y, const int64_t* out_slices, int32_t num_slices,
                                         int32_t r_max, void* stream) {
  if (!addr) return LORA_ERR_NULL;
  if (addr->T < 0 || num_slices < 1 || num_slices > kMaxSlices) return LORA_ERR_SHAPE;
  if (r_max < 1 || r_max > 128) return LORA_ERR_RANK;
  if ((int64_t)addr->T * num_slices * r_max * 4 > kScratchBytes) return LORA_ERR_LIMIT;
  void* sp = nullptr;
  const int rc = scratch_address(&sp);
  if (rc != LORA_OK) return rc;
  lora_t3 h{};
  h.ptr = sp;
  h.dtype = LORA_F32;
  h.d0 = addr->T;
  h.d1 = num_slices;
  h.d2 = r_max;
  h.s0 = (int64_t)num_slices * r_max;
  h.s1 = r_max;
  h.s2 = 1;
  return lora_apply_linear(x, a, b, addr, ranks, scalings, y, out_slices, num_slices, r_max, &h, stream);
}

extern "C" int lora_gather_shrink(const int32_t* ids, const lora_t3* a, const lora_addressing* addr,
                                  const int32_t* ranks, int32_t r_max, const lora_t3* h, void* stream) {
  if (!a || !h) return LORA_ERR_NULL;
  int rc = check_addressing(addr, ranks);
  if (rc != LORA_OK) return rc;
  if (r_max < 1 || r_max > 128) return LORA_ERR_RANK;
  if (!valid_dims(a) || !valid_dims(h)) return LORA_ERR_SHAPE;
  const int64_t T = addr->T, S = addr->S, V = a->d2;
  if (a->d0 != S || a->d1 != r_max || V < 0) return LORA_ERR_SHAPE;
  if (h->d0 != T || h->d1 != 1 || h->d2 != r_max) return LORA_ERR_SHAPE;
  if (!float_dtype_ok(a->dtype) || h->dtype != LORA_F32) return LORA_ERR_DTYPE;
  if ((T > 0 && (!ids || !h->ptr)) || (S * V > 0 && !a->ptr)) return LORA_ERR_NULL;
  if (h->s2 != 1) return LORA_ERR_STRIDE;
  if (T == 0) return LORA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(ceil_div(T, 4)));
  if (a->dtype == LORA_BF16)
    launch(gather_kernel<uint16_t>, grid, dim3(256), 0, st, ids, static_cast<const uint16_t*>(a->ptr),
                       a->s0, a->s1, a->s2, V, addr->token_slot, ranks, static_cast<int>(T), static_cast<int>(S),
                       r_max, static_cast<float*>(h->ptr), h->s0);
  else
    launch(gather_kernel<float>, grid, dim3(256), 0, st, ids, static_cast<const float*>(a->ptr), a->s0,
                       a->s1, a->s2, V, addr->token_slot, ranks, static_cast<int>(T), static_cast<int>(S), r_max,
                       static_cast<float*>(h->ptr), h->s0);
  return launch_status();
}
