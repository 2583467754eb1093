// Host-side helpers shared by the entry points: argument checks (all done
// before any launch), sizes, workspace carving and launch-error mapping.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lora.h"

namespace lora {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

inline size_t elem_size(int32_t dtype) {
  return dtype == LORA_BF16 ? 2 : (dtype == LORA_F32 ? 4 : 0);
}
inline int vec_elems(int32_t dtype) { return dtype == LORA_BF16 ? 8 : 4; }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Rank rounded up to the kernels' rank-block count (1, 2, 4 or 8 blocks of 16).
inline int rank_blocks(int r) {
  int rb = static_cast<int>(ceil_div(r, 16));
  return rb <= 1 ? 1 : rb <= 2 ? 2 : rb <= 4 ? 4 : 8;
}
inline int padded_rank(int r) { return 16 * rank_blocks(r); }

// A matrix operand that is streamed row by row with 128-bit loads/stores:
// unit column stride, 16-byte aligned base and row pitch.
inline int check_rowmajor_stream(const lora_mat* m) {
  if (m->stride_col != 1) return LORA_ERR_STRIDE;
  size_t es = elem_size(m->dtype);
  if (m->rows > 1 && (m->stride_row < m->cols || (m->stride_row * (int64_t)es) % 16 != 0)) return LORA_ERR_STRIDE;
  if (!aligned(m->ptr, 16)) return LORA_ERR_STRIDE;
  return LORA_OK;
}

// The transposed view of a row-major stream (rows = features, cols = tokens).
inline int check_colmajor_stream(const lora_mat* m) {
  if (m->stride_row != 1) return LORA_ERR_STRIDE;
  size_t es = elem_size(m->dtype);
  if (m->cols > 1 && (m->stride_col < m->rows || (m->stride_col * (int64_t)es) % 16 != 0)) return LORA_ERR_STRIDE;
  if (!aligned(m->ptr, 16)) return LORA_ERR_STRIDE;
  return LORA_OK;
}

inline bool float_dtype_ok(int32_t d) { return d == LORA_BF16 || d == LORA_F32; }

// Every operand must fit in 2^47 bytes (128 TiB, more than any device holds):
// dims and strides non-negative and at most 2^47 each, and its element count
// and byte extent at most 2^47, computed without overflow. With that checked
// first, every product the entry points form from the dims, strides and
// element size of one operand fits an int64_t.
constexpr int64_t kMaxOperand = int64_t(1) << 47;

inline bool operand_fits(const int64_t* dims, const int64_t* strides, int n, int64_t es) {
  bool empty = false;
  for (int i = 0; i < n; ++i) {
    if (dims[i] < 0 || dims[i] > kMaxOperand || strides[i] < 0 || strides[i] > kMaxOperand) return false;
    empty = empty || dims[i] == 0;
  }
  if (empty) return true;
  int64_t count = 1, last = 0;
  for (int i = 0; i < n; ++i) {
    int64_t step = 0;
    if (__builtin_mul_overflow(count, dims[i], &count) || count > kMaxOperand) return false;
    if (__builtin_mul_overflow(dims[i] - 1, strides[i], &step) || __builtin_add_overflow(last, step, &last) ||
        last >= kMaxOperand)
      return false;
  }
  return (last + 1) * es <= kMaxOperand && count * es <= kMaxOperand;
}

inline bool valid_dims(const lora_mat* m) {
  const int64_t dims[2] = {m->rows, m->cols};
  const int64_t strides[2] = {m->stride_row, m->stride_col};
  const int64_t es = static_cast<int64_t>(elem_size(m->dtype));
  return operand_fits(dims, strides, 2, es > 0 ? es : 1);
}

inline bool valid_dims(const lora_t3* t) {
  const int64_t dims[3] = {t->d0, t->d1, t->d2};
  const int64_t strides[3] = {t->s0, t->s1, t->s2};
  const int64_t es = static_cast<int64_t>(elem_size(t->dtype));
  return operand_fits(dims, strides, 3, es > 0 ? es : 1);
}

// Carves 256-byte aligned sub-buffers out of a caller workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += static_cast<size_t>(round_up(static_cast<int64_t>(bytes), 256));
    return p;
  }
};

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH;
}

// Kernel timing for measurement tools (lora_timing_* entry points): true,
// with a pair of events, when the next launch is to be timed.
bool timing_take(hipEvent_t* start, hipEvent_t* stop);

// Launches a kernel. While kernel timing records, the launch goes through
// hipExtLaunchKernel with a pair of events that the dispatch itself stamps
// at the kernel's start and end (no marker packets around it).
template <class... P, class... A>
inline void launch(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, A... args) {
  hipEvent_t e0, e1;
  if (timing_take(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0u, args...);
  else
    kernel<<<grid, block, shmem, st>>>(args...);
}

}  // namespace lora
