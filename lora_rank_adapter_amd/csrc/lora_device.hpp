// Device-side building blocks of the gfx950 LoRA kernels: element tags,
// 128-bit loads, the MFMA steps used by every kernel, and the bf16 hi/lo
// split that keeps float32 intermediates exact enough for a bf16 MFMA.
//
// MFMA conventions (CDNA 16x16 shapes, wave64): for D = A * B + C with
// A 16 x k and B k x 16, lane l supplies row (l % 16) of A and column (l % 16)
// of B, each with the contraction values of lane group g = l / 16; lane l
// holds D[4*g + i][l % 16] for i = 0..3. The kernels only rely on A and B
// using the same contraction order, which they choose freely.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// bfloat16 inputs: 8 elements per 128-bit vector; one 16x16x32 MFMA per vector.
struct BF16 {
  using elem = uint16_t;
  static constexpr int VEC = 8;
};
// float32 inputs: 4 elements per 128-bit vector; four 16x16x4 MFMAs per vector.
struct F32 {
  using elem = float;
  static constexpr int VEC = 4;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Transposed 8-byte LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i receives element (i % 4) of the 4 x 16-bit pieces that lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of its group address, in that order.
// `off` is this lane's byte offset into the __shared__ buffer `lds`.
__device__ __forceinline__ uint2 lds_read_tr16(const void* lds, int off) {
  auto p = (__attribute__((address_space(3))) short4_t*)((char*)lds + off);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
}

// A wave-uniform value below 2^31 as a scalar-register int.
__device__ __forceinline__ int uniform_int(int64_t v) {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(v));
}

// Keeps the instruction scheduler from moving instructions across this
// point. Software-pipelined loops put one between issuing the next stage's
// loads and computing on the current stage, so that the loads stay in flight
// during the computation (the wait before it then covers only the current
// stage).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: loops bounded by it compile to scalar branches, so the compiler can
// keep loads in flight across iterations instead of draining at each
// divergent loop edge.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)); }

// ---------------------------------------------------------------------------
// Buffer-resource (V#) memory access. A raw buffer descriptor carries a base
// address and a byte size; the hardware returns 0 for loads and drops stores
// whose byte offset falls outside [0, size). Masked lanes therefore use the
// offset kOOB instead of a branch, which keeps every loop free of divergent
// control flow around memory operations (the compiler can then wait for
// exactly the loads a step consumes).
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;          // any offset >= every descriptor size
constexpr int64_t kMaxBufferBytes = 0x7FFFFFFF;  // descriptor sizes are clamped to this

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > kMaxBufferBytes ? kMaxBufferBytes : bytes);
  // 0x00020000: gfx9-family descriptor word 3 (32-bit data format, no swizzle).
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, 0);
}

// Loads and stores of the streamed tensors (activations, gradients and
// outputs, each touched once per call) carry the non-temporal cache policy
// (nt): their lines are marked for early eviction, so the streams do not
// displace each other and the reused operands (weights, the rank intermediate)
// in the caches. On the MI355X a plain y += x stream over the forward's
// tensors (bf16 x, fp32 y) runs at 6.4 TB/s with non-temporal loads and stores
// against 5.8 TB/s without; in the LoRA kernels nt on both is needed (nt loads
// with default stores lose most of the gain), and the system-scope bit (sc1)
// on the stores adds about 1% more. Weights and intermediates keep the default
// policy. Cache-policy operand bits on gfx950: 1 sc0, 2 nt, 16 sc1.
constexpr int kStreamLoadPolicy = 2;    // nt
constexpr int kStreamStorePolicy = 18;  // nt | sc1

__device__ __forceinline__ uint4 sload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamLoadPolicy));
}
__device__ __forceinline__ void sstore16(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kStreamStorePolicy);
}
__device__ __forceinline__ uint2 sload8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kStreamLoadPolicy));
}
__device__ __forceinline__ void sstore8(rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, (int)off, 0, kStreamStorePolicy);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ f32x4_t ld16f(const float* p) {
  return __builtin_bit_cast(f32x4_t, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void st16f(float* p, f32x4_t v) {
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}

// Round-to-nearest-even float -> bfloat16 bits (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  __bf16 h = static_cast<__bf16>(v);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}
__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// An output the kernels add into in place, 4 consecutive columns per lane
// (the offset is in bytes, kOOB for masked lanes). float32: one 16-byte
// access. bfloat16: one 8-byte access; the float32 sum of the old value and
// the update is rounded once, to nearest even (NaN stays NaN, beyond the
// largest bfloat16 it becomes infinite).
template <class O>
struct Out;
template <>
struct Out<float> {
  static constexpr int ES = 4;
  static __device__ __forceinline__ f32x4_t load4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4_t, sload16(r, off));
  }
  static __device__ __forceinline__ void store4(rsrc_t r, uint32_t off, f32x4_t v) {
    sstore16(r, off, __builtin_bit_cast(uint4, v));
  }
  // plain-pointer forms (p: 16-byte aligned)
  static __device__ __forceinline__ f32x4_t ld4(const void* p) {
    return __builtin_bit_cast(f32x4_t, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ void st4(void* p, f32x4_t v) {
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
  }
};
template <>
struct Out<uint16_t> {
  static constexpr int ES = 2;
  static __device__ __forceinline__ f32x4_t load4(rsrc_t r, uint32_t off) { return unpack(sload8(r, off)); }
  static __device__ __forceinline__ void store4(rsrc_t r, uint32_t off, f32x4_t v) {
    sstore8(r, off, pack(v));
  }
  // plain-pointer forms (p: 8-byte aligned)
  static __device__ __forceinline__ f32x4_t ld4(const void* p) { return unpack(*reinterpret_cast<const uint2*>(p)); }
  static __device__ __forceinline__ void st4(void* p, f32x4_t v) { *reinterpret_cast<uint2*>(p) = pack(v); }
  static __device__ __forceinline__ uint2 pack(f32x4_t v) {
    return make_uint2(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16));
  }
  static __device__ __forceinline__ f32x4_t unpack(uint2 w) {
    return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                   __uint_as_float(w.y & 0xFFFF0000u)};
  }
};

// ---------------------------------------------------------------------------
// contraction step over one 128-bit vector per lane:  acc += A * B
// (a: A operand vector of this lane, b: B operand vector; same contraction
// order in both). bf16: 8 values per lane -> one 16x16x32 MFMA. f32: 4 values
// per lane -> four 16x16x4 MFMAs, the e-th taking value e of every lane.
// ---------------------------------------------------------------------------
template <class Tag>
__device__ __forceinline__ void mma_vec(f32x4_t& acc, uint4 a, uint4 b);

template <>
__device__ __forceinline__ void mma_vec<BF16>(f32x4_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_vec<F32>(f32x4_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Operand of a float32 intermediate (h = s*X*A, dYB, XA) against a weight.
// A lane holds 4 float32 values v[i] of consecutive rank indices.
//  bf16 path: v = hi + lo with hi = bf16(v), lo = bf16(v - hi) (both exact
//  roundings, residual <= 2^-17 |v|); the B operand vector is
//  {hi0..hi3, lo0..lo3} and the matching weight vector is {w0..w3, w0..w3},
//  so one 16x16x32 MFMA contracts 16 rank indices at float32-like accuracy.
//  f32 path: the 4 values themselves.
// ---------------------------------------------------------------------------
template <class Tag>
__device__ __forceinline__ uint4 split_frag(f32x4_t v);

template <>
__device__ __forceinline__ uint4 split_frag<BF16>(f32x4_t v) {
  uint32_t h0 = bf16_bits(v[0]), h1 = bf16_bits(v[1]), h2 = bf16_bits(v[2]), h3 = bf16_bits(v[3]);
  uint32_t l0 = bf16_bits(v[0] - bf16_value(h0));
  uint32_t l1 = bf16_bits(v[1] - bf16_value(h1));
  uint32_t l2 = bf16_bits(v[2] - bf16_value(h2));
  uint32_t l3 = bf16_bits(v[3] - bf16_value(h3));
  return make_uint4(h0 | (h1 << 16), h2 | (h3 << 16), l0 | (l1 << 16), l2 | (l3 << 16));
}

template <>
__device__ __forceinline__ uint4 split_frag<F32>(f32x4_t v) {
  return __builtin_bit_cast(uint4, v);
}

// Weight vector of 4 consecutive rank columns j0..j0+3 of one weight row, with
// columns >= r read as zero (so padding, possibly NaN, is never used).
// bf16: one 8-byte load (duplicated to {w0..w3, w0..w3}); f32: one 16-byte
// load; element loads when vec_ok is false (row not aligned for that) or the
// segment crosses r.
template <class Tag>
__device__ __forceinline__ uint4 load_wvec4(const typename Tag::elem* row, int j0, int r, bool vec_ok);

template <>
__device__ __forceinline__ uint4 load_wvec4<BF16>(const uint16_t* row, int j0, int r, bool vec_ok) {
  uint32_t lo, hi;
  if (vec_ok && j0 + 4 <= r) {
    uint2 w = *reinterpret_cast<const uint2*>(row + j0);
    lo = w.x;
    hi = w.y;
  } else if (j0 < r) {
    uint32_t e0 = row[j0];
    uint32_t e1 = (j0 + 1 < r) ? row[j0 + 1] : 0u;
    uint32_t e2 = (j0 + 2 < r) ? row[j0 + 2] : 0u;
    uint32_t e3 = (j0 + 3 < r) ? row[j0 + 3] : 0u;
    lo = e0 | (e1 << 16);
    hi = e2 | (e3 << 16);
  } else {
    lo = 0u;
    hi = 0u;
  }
  return make_uint4(lo, hi, lo, hi);
}

template <>
__device__ __forceinline__ uint4 load_wvec4<F32>(const float* row, int j0, int r, bool vec_ok) {
  if (vec_ok && j0 + 4 <= r) return ld16(row + j0);
  uint4 w = zero4();
  if (j0 < r) w.x = __float_as_uint(row[j0]);
  if (j0 + 1 < r) w.y = __float_as_uint(row[j0 + 1]);
  if (j0 + 2 < r) w.z = __float_as_uint(row[j0 + 2]);
  if (j0 + 3 < r) w.w = __float_as_uint(row[j0 + 3]);
  return w;
}

// Compact register form of a 4-column weight vector: bf16 keeps 8 bytes and is
// duplicated to the MFMA operand at use; f32 keeps the 16-byte vector.
template <class Tag>
struct WFrag;
//
// masked(row, jl, j0, r, ok): unconditional load of the 4 columns starting at
// jl (an in-bounds, 4-aligned column of the row), then columns j0+e >= r, or
// every column when !ok, replaced by zero. Callers pass jl = j0 unless j0 lies
// past the readable part of the row, in which case every column is masked.
template <>
struct WFrag<BF16> {
  using type = uint2;
  static __device__ __forceinline__ type pack(uint4 w) { return make_uint2(w.x, w.y); }
  static __device__ __forceinline__ uint4 operand(type w) { return make_uint4(w.x, w.y, w.x, w.y); }
  static __device__ __forceinline__ type zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ type masked(const uint16_t* row, int jl, int j0, int r, bool ok) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + jl);
    const uint32_t m0 = (ok && j0 < r ? 0xFFFFu : 0u) | (ok && j0 + 1 < r ? 0xFFFF0000u : 0u);
    const uint32_t m1 = (ok && j0 + 2 < r ? 0xFFFFu : 0u) | (ok && j0 + 3 < r ? 0xFFFF0000u : 0u);
    return make_uint2(w.x & m0, w.y & m1);
  }
  // Buffer form: off = byte offset of column j0 of the row, or kOOB.
  static __device__ __forceinline__ type bload(rsrc_t rs, uint32_t off, int j0, int r) {
    const uint2 w = bload8(rs, off);
    const uint32_t m0 = (j0 < r ? 0xFFFFu : 0u) | (j0 + 1 < r ? 0xFFFF0000u : 0u);
    const uint32_t m1 = (j0 + 2 < r ? 0xFFFFu : 0u) | (j0 + 3 < r ? 0xFFFF0000u : 0u);
    return make_uint2(w.x & m0, w.y & m1);
  }
};
template <>
struct WFrag<F32> {
  using type = uint4;
  static __device__ __forceinline__ type pack(uint4 w) { return w; }
  static __device__ __forceinline__ uint4 operand(type w) { return w; }
  static __device__ __forceinline__ type zero() { return zero4(); }
  static __device__ __forceinline__ type masked(const float* row, int jl, int j0, int r, bool ok) {
    const uint4 w = ld16(row + jl);
    return make_uint4((ok && j0 < r) ? w.x : 0u, (ok && j0 + 1 < r) ? w.y : 0u, (ok && j0 + 2 < r) ? w.z : 0u,
                      (ok && j0 + 3 < r) ? w.w : 0u);
  }
  static __device__ __forceinline__ type bload(rsrc_t rs, uint32_t off, int j0, int r) {
    const uint4 w = bload16(rs, off);
    return make_uint4(j0 < r ? w.x : 0u, j0 + 1 < r ? w.y : 0u, j0 + 2 < r ? w.z : 0u, j0 + 3 < r ? w.w : 0u);
  }
};

// acc += W(4 rank columns) * frag over 16 rank indices of one rank block.
template <class Tag>
__device__ __forceinline__ void mma_rank16(f32x4_t& acc, uint4 wvec, uint4 frag);

template <>
__device__ __forceinline__ void mma_rank16<BF16>(f32x4_t& acc, uint4 wvec, uint4 frag) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wvec), __builtin_bit_cast(bf16x8_t, frag),
                                                acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_rank16<F32>(f32x4_t& acc, uint4 wvec, uint4 frag) {
  mma_vec<F32>(acc, wvec, frag);
}

}  // namespace lora
