// Device-side helpers shared by the CCQ kernels (gfx950 / CDNA4 only).
//
// Wave64 reductions, dtype conversion, and the 16x16x32 MFMA tile used by the
// prefill kernels.  A tile "fragment" is 8 K-elements per lane: lane l serves
// row (l % 16) of A (or column (l % 16) of B) and K-group g = l / 16.  Which 8 K
// indices a group holds is the caller's choice, as long as A and B agree:
//   - KORD_CONTIG: k = 8g + e            (one 16-byte LDS read)
//   - KORD_ACC:    k = 16(e/4) + 4g + e%4 (the order an accumulator pair has)
// The accumulator of a 16x16 tile holds D[4g + r][l % 16] in element r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ccq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- scalar I/O

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // RNE

template <typename T>
__device__ __forceinline__ float ldf(const T* p, size_t i) { return to_f32(p[i]); }

// ---------------------------------------------------------------- reductions

// Sum over groups of W consecutive lanes (W a power of two <= 64); every lane of a
// group receives the group total.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Workgroup barrier that publishes LDS writes only.  __syncthreads() also fences global
// memory, i.e. waits for every outstanding global load and store of the wave (in-flight
// prefetches, output stores); the kernels here never exchange data between waves through
// global memory, so waiting for the LDS counter is enough.  The "memory" clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits for every vector memory access of the wave (direct loads into LDS included) and tells the
// compiler so.  A wait written in inline asm is opaque to the compiler's own wait placement: a loop
// entered after one carries the loads issued before it as still pending into every iteration, and
// the compiler then waits for them at their first use inside the loop, where its wait also waits
// for the direct loads issued since, which it cannot see.  The immediate is vmcnt(0) with the
// export and LDS counters left alone (their fields at their maxima, 7 and 15).
__device__ __forceinline__ void vm_wait_all() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// ---------------------------------------------------------------- MFMA tiles

enum KOrder { KORD_CONTIG = 0, KORD_ACC = 1 };

template <typename T>
struct Frag;
template <>
struct Frag<__bf16> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// acc += A(16x32) * B(32x16) for one fragment pair.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Fragment of row (lane % 16) of a K-contiguous LDS matrix: elements
// [row][k0 + korder(g, e)], pitch in elements.
template <typename T, int KO>
__device__ __forceinline__ Frag<T> lds_frag(const T* base, int pitch, int row0, int k0, int lane) {
  Frag<T> f;
  const int g = lane >> 4;
  const T* p = base + (row0 + (lane & 15)) * pitch + k0;
  if constexpr (sizeof(T) == 2) {
    if constexpr (KO == KORD_CONTIG) {
      f.v = *reinterpret_cast<const bf16x8*>(p + 8 * g);
    } else {
      bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + 4 * g);
      bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16 + 4 * g);
      f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  } else {
    if constexpr (KO == KORD_CONTIG) {
      f32x4 lo = *reinterpret_cast<const f32x4*>(p + 8 * g);
      f32x4 hi = *reinterpret_cast<const f32x4*>(p + 8 * g + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[4 + e] = hi[e]; }
    } else {
      f32x4 lo = *reinterpret_cast<const f32x4*>(p + 4 * g);
      f32x4 hi = *reinterpret_cast<const f32x4*>(p + 16 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[4 + e] = hi[e]; }
    }
  }
  return f;
}

// Operand fragment from a pair of accumulator tiles t0 (K 0..15) and t1 (K 16..31),
// in KORD_ACC order.  As an A operand it is the transpose of the tiles; as a B
// operand it is the tiles themselves.  Optional per-element scale.
template <typename T>
__device__ __forceinline__ Frag<T> acc_frag(const f32x4& t0, const f32x4& t1) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = bf16x8{(__bf16)t0[0], (__bf16)t0[1], (__bf16)t0[2], (__bf16)t0[3],
                 (__bf16)t1[0], (__bf16)t1[1], (__bf16)t1[2], (__bf16)t1[3]};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = t0[e]; f.v[4 + e] = t1[e]; }
  }
  return f;
}

}  // namespace ccq
