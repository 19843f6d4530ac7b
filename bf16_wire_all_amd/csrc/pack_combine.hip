// Pack (F32 -> BF16 into a slot ring) and two-operand combine kernels.
//
// Both are pure streams over HBM: 6 bytes per element for pack (4 read, 2
// written), 8 (F32 out) or 6 (BF16 out) bytes per element for combine.  The
// work per element is a handful of integer operations, far below the ALU
// budget, so the design is about the memory side only:
//   - a thread handles "quads" of 4 consecutive elements, so every load and
//     store instruction of a wave covers one contiguous span (1 KiB of F32,
//     512 B of BF16): fully coalesced 128-bit / 64-bit accesses;
//   - many short workgroups, each streaming one contiguous chunk of 512 quads
//     in a single pass (2 quads per thread, each load followed by its store).
//     Measured on MI355X after a 2.36 GB copy, against 1024-quad chunks with
//     the loads issued first: pack 16384 x 5120 6.4 TB/s (was 6.1), combine
//     6.4 (6.0); at 2048 x 5120 pack 4.5 (4.2), combine 5.0 (4.5).  Pairing
//     units from the two halves of the operands, which helps plain copies,
//     measured no better here;
//   - loads and stores carry the nontemporal hint: each byte is touched once
//     (cold 2048 x 5120 pack: 4.5 TB/s with it, 2.5 TB/s without).
#include "internal.h"

namespace xfer {
namespace {

constexpr int kThreads = 256;
constexpr int kQuadsPerThread = 2;
constexpr uint64_t kQuadsPerBlock = (uint64_t)kThreads * kQuadsPerThread;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ T nt_load(const T *p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void nt_store(T *p, T v) {
  __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ uint4 ld(const uint4 *p) {
  const v4u v = nt_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld(const uint2 *p) {
  const v2u v = nt_load(reinterpret_cast<const v2u *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st(uint4 *p, uint4 v) { nt_store(reinterpret_cast<v4u *>(p), v4u{v.x, v.y, v.z, v.w}); }
__device__ __forceinline__ void st(uint2 *p, uint2 v) { nt_store(reinterpret_cast<v2u *>(p), v2u{v.x, v.y}); }

// Round-to-nearest-even of an F32 bit pattern to BF16 (in the low 16 bits).
// Adding 0x7FFF plus the lowest kept bit carries into the kept bits exactly
// when the discarded half is above one half, or equal to one half with an
// odd kept part; overflow carries into the exponent and gives infinity.  NaN
// patterns would be carried into infinity or zero, so they are replaced by
// the canonical quiet NaN first.
__device__ __forceinline__ uint32_t bf16_rne(uint32_t f) {
  const uint32_t r = (f + 0x7FFFu + ((f >> 16) & 1u)) >> 16;
  return ((f & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

__device__ __forceinline__ uint2 pack_quad(uint4 v) {
  uint2 o;
  o.x = bf16_rne(v.x) | (bf16_rne(v.y) << 16);
  o.y = bf16_rne(v.z) | (bf16_rne(v.w) << 16);
  return o;
}

// F32 sum of two BF16 values given as the low / high half of a word pair,
// with rank 0's operand first; NaN results canonical.
__device__ __forceinline__ uint32_t sum_bf16(uint32_t a16, uint32_t b16) {
  const float fa = __uint_as_float(a16 << 16);
  const float fb = __uint_as_float(b16 << 16);
  const uint32_t s = __float_as_uint(__fadd_rn(fa, fb));
  return ((s & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC00000u : s;
}

__device__ __forceinline__ uint4 sum_quad(uint2 a, uint2 b) {
  uint4 s;
  s.x = sum_bf16(a.x & 0xFFFFu, b.x & 0xFFFFu);
  s.y = sum_bf16(a.x >> 16, b.x >> 16);
  s.z = sum_bf16(a.y & 0xFFFFu, b.y & 0xFFFFu);
  s.w = sum_bf16(a.y >> 16, b.y >> 16);
  return s;
}

// src points at the first element of the call's range; quad q of the range
// goes to ring quad (q + slot0_q) mod ring_q.  The range is at most one ring
// long, so one conditional subtraction is the modulo.
//
// A range whose length is not a multiple of 4 ends in 1-3 single elements;
// the first threads of workgroup 0 convert them.
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint4 *__restrict__ src, uint2 *__restrict__ ring,
                                                        uint64_t n_quads, uint64_t ring_quads, uint64_t slot0_q,
                                                        uint32_t tail) {
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const uint64_t ring_elems = ring_quads * 4;
    uint64_t d = (n_quads + slot0_q) * 4 + threadIdx.x;
    if (d >= ring_elems) d -= ring_elems;
    const float *s1 = reinterpret_cast<const float *>(src + n_quads);
    reinterpret_cast<uint16_t *>(ring)[d] = (uint16_t)bf16_rne(__float_as_uint(s1[threadIdx.x]));
  }
  const uint64_t q0 = (uint64_t)blockIdx.x * kQuadsPerBlock + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kQuadsPerThread; ++u) {
    const uint64_t q = q0 + u * kThreads;
    if (q < n_quads) {
      uint64_t d = q + slot0_q;
      if (d >= ring_quads) d -= ring_quads;
      st(&ring[d], pack_quad(ld(&src[q])));
    }
  }
}

// In BF16 mode out may be a or b itself: every thread reads its own quads
// before writing them and no other thread touches them.
template <int MODE>
__device__ __forceinline__ void combine_quad(const uint2 *a, const uint2 *b, void *out, uint64_t q) {
  const uint4 s = sum_quad(ld(&a[q]), ld(&b[q]));
  if (MODE == XFER_OUT_F32)
    st(&reinterpret_cast<uint4 *>(out)[q], s);
  else
    st(&reinterpret_cast<uint2 *>(out)[q], pack_quad(s));
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint2 *a, const uint2 *b, void *out,
                                                           uint64_t n_quads, uint32_t tail) {
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const uint64_t e = n_quads * 4 + threadIdx.x;
    const uint32_t s = sum_bf16(reinterpret_cast<const uint16_t *>(a)[e], reinterpret_cast<const uint16_t *>(b)[e]);
    if (MODE == XFER_OUT_F32)
      reinterpret_cast<uint32_t *>(out)[e] = s;
    else
      reinterpret_cast<uint16_t *>(out)[e] = (uint16_t)bf16_rne(s);
  }
  const uint64_t q0 = (uint64_t)blockIdx.x * kQuadsPerBlock + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kQuadsPerThread; ++u) {
    const uint64_t q = q0 + u * kThreads;
    if (q < n_quads) combine_quad<MODE>(a, b, out, q);
  }
}

// F32-wire variant: both operands are F32 (12 B per element with F32 out,
// 10 B with BF16 out), same chunking as the BF16-wire combine.
__device__ __forceinline__ uint32_t sum_f32(uint32_t a, uint32_t b) {
  const uint32_t s = __float_as_uint(__fadd_rn(__uint_as_float(a), __uint_as_float(b)));
  return ((s & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC00000u : s;
}

template <int MODE>
__device__ __forceinline__ void combine_f32_quad(const uint4 *a, const uint4 *b, void *out, uint64_t q) {
  const uint4 x = ld(&a[q]), y = ld(&b[q]);
  uint4 s;
  s.x = sum_f32(x.x, y.x);
  s.y = sum_f32(x.y, y.y);
  s.z = sum_f32(x.z, y.z);
  s.w = sum_f32(x.w, y.w);
  if (MODE == XFER_OUT_F32)
    st(&reinterpret_cast<uint4 *>(out)[q], s);
  else
    st(&reinterpret_cast<uint2 *>(out)[q], pack_quad(s));
}

// In F32 mode out may be a or b itself (each thread reads its quads before
// writing them); in BF16 mode out overlaps neither (host check).
template <int MODE>
__global__ __launch_bounds__(kThreads) void combine_f32_kernel(const uint4 *a, const uint4 *b, void *out,
                                                               uint64_t n_quads, uint32_t tail) {
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const uint64_t e = n_quads * 4 + threadIdx.x;
    const uint32_t s = sum_f32(reinterpret_cast<const uint32_t *>(a)[e], reinterpret_cast<const uint32_t *>(b)[e]);
    if (MODE == XFER_OUT_F32)
      reinterpret_cast<uint32_t *>(out)[e] = s;
    else
      reinterpret_cast<uint16_t *>(out)[e] = (uint16_t)bf16_rne(s);
  }
  const uint64_t q0 = (uint64_t)blockIdx.x * kQuadsPerBlock + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kQuadsPerThread; ++u) {
    const uint64_t q = q0 + u * kThreads;
    if (q < n_quads) combine_f32_quad<MODE>(a, b, out, q);
  }
}

// One workgroup per chunk of kQuadsPerBlock quads (at least one, for the tail).
uint32_t grid_for(uint64_t n_quads) {
  const uint64_t g = (n_quads + kQuadsPerBlock - 1) / kQuadsPerBlock;
  return (uint32_t)(g ? g : 1);
}

}  // namespace

// The pack and combine launches, handed to `emit` (an eager launch or a graph
// node) with their kernel, grid and exact arguments.
template <typename Emit>
hipError_t pack_call(Emit &&emit, const float *src, uint64_t n_elems, uint16_t *ring, uint64_t ring_elems,
                     uint64_t slot0_elem) {
  const uint64_t n_quads = n_elems / 4;
  const uint32_t tail = (uint32_t)(n_elems % 4);
  return emit(pack_kernel, dim3(grid_for(n_quads)), dim3(kThreads), reinterpret_cast<const uint4 *>(src),
              reinterpret_cast<uint2 *>(ring), n_quads, ring_elems / 4, slot0_elem / 4, tail);
}

template <typename Emit>
hipError_t combine_call(Emit &&emit, const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode) {
  const uint64_t n_quads = n / 4;
  const uint32_t tail = (uint32_t)(n % 4);
  const uint2 *a2 = reinterpret_cast<const uint2 *>(a);
  const uint2 *b2 = reinterpret_cast<const uint2 *>(b);
  const dim3 grid(grid_for(n_quads));
  if (mode == XFER_OUT_F32) return emit(combine_kernel<XFER_OUT_F32>, grid, dim3(kThreads), a2, b2, out, n_quads, tail);
  return emit(combine_kernel<XFER_OUT_BF16>, grid, dim3(kThreads), a2, b2, out, n_quads, tail);
}

hipError_t launch_pack(const float *src, uint64_t n_elems, uint16_t *ring, uint64_t ring_elems,
                       uint64_t slot0_elem, hipStream_t stream) {
  auto emit = [&](auto kernel, dim3 grid, dim3 block, auto... args) {
    return launch(kernel, grid, block, 0, stream, args...);
  };
  return pack_call(emit, src, n_elems, ring, ring_elems, slot0_elem);
}

hipError_t launch_combine(const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode,
                          hipStream_t stream) {
  auto emit = [&](auto kernel, dim3 grid, dim3 block, auto... args) {
    return launch(kernel, grid, block, 0, stream, args...);
  };
  return combine_call(emit, a, b, n, out, mode);
}

hipError_t node_pack(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node, const float *src,
                     uint64_t n_elems, uint16_t *ring, uint64_t ring_elems, uint64_t slot0_elem) {
  auto emit = [&](auto kernel, dim3 grid, dim3 block, auto... args) {
    return add_node(g, deps, n_deps, node, kernel, grid, block, args...);
  };
  return pack_call(emit, src, n_elems, ring, ring_elems, slot0_elem);
}

hipError_t node_combine(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node,
                        const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode) {
  auto emit = [&](auto kernel, dim3 grid, dim3 block, auto... args) {
    return add_node(g, deps, n_deps, node, kernel, grid, block, args...);
  };
  return combine_call(emit, a, b, n, out, mode);
}

hipError_t launch_combine_f32(const float *a, const float *b, uint64_t n, void *out, int mode, hipStream_t stream) {
  const uint64_t n_quads = n / 4;
  const uint32_t tail = (uint32_t)(n % 4);
  const uint4 *a4 = reinterpret_cast<const uint4 *>(a);
  const uint4 *b4 = reinterpret_cast<const uint4 *>(b);
  const dim3 grid(grid_for(n_quads));
  if (mode == XFER_OUT_F32)
    return launch(combine_f32_kernel<XFER_OUT_F32>, grid, dim3(kThreads), 0, stream, a4, b4, out, n_quads, tail);
  return launch(combine_f32_kernel<XFER_OUT_BF16>, grid, dim3(kThreads), 0, stream, a4, b4, out, n_quads, tail);
}

}  // namespace xfer
