// Device helpers shared by the bf16 d = 128 attention kernels (forward and
// backward): LDS slab geometry, the XOR swizzle, the stage waits and barrier,
// and the asm slot reads.  Internal to the library.
#pragma once

#include "common.hpp"

#include <utility>

namespace ssa {
namespace d128 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SSA_LDS __attribute__((address_space(3)))
#define SSA_GLB __attribute__((address_space(1)))

constexpr int kD = 128;
constexpr int kBlk = 128;
constexpr int kSK = 32;                   // keys per stage
constexpr int kSlots = 4;                 // LDS ring depth
constexpr int kUnits = kD / 8;            // 16-byte units per row
constexpr int kSlab = kSK * kUnits;       // units per K (or V) slab: 8 KB
constexpr int kSlotBytes = 2 * kSlab * 16;  // K slab, then V slab: 16 KB
constexpr int kWaves = 4;
constexpr int kMaxW = 64;  // longest block list a query block may have
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// max / sum with the lane 32 apart (the other half of the same query column)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// f(integral_constant<int, k>) for k = 0 .. N-1, unrolled
template <typename F, int... K>
__device__ __forceinline__ void for_each_stage(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void for_each_stage(F&& f) {
  for_each_stage(f, std::make_integer_sequence<int, N>{});
}

// vmcnt(4 k) alone (expcnt and lgkmcnt left at their maximum): all but this
// wave's loads of the last k stages have landed (4 loads a stage)
__device__ __forceinline__ void wait_stages(int k) {
  if (k >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (k == 1)
    __builtin_amdgcn_s_waitcnt(0x0F74);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier for the stage loop.  __syncthreads() would also wait for
// every outstanding vector-memory load (its release fence), draining the
// prefetch ring; the only memory the barrier has to order here is LDS
// written by this wave's direct-to-LDS loads, which wait_stages has already
// waited for, and LDS reads that have returned before their MFMAs issued.
// The empty asm statements keep the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reads of a ring slot.  The compiler cannot tell which in-flight
// direct-to-LDS load a plain LDS read may overlap, and would wait for all of
// them (draining the ring) before the slot's first read.  The stage's own
// loads are already waited for and published by the stage barrier, so the
// reads are issued from asm blocks the compiler does not track; each block
// waits for its reads before it ends, and its outputs are early-clobber so
// that no output register can be an address still to be read.  OFF is the
// slot's byte offset in the ring (an instruction immediate).
//
// the 8 K fragments of a stage
template <int OFF>
__device__ __forceinline__ void lds_read_k8(const uint32_t (&a)[8], u32x4 (&o)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%16\n"
      "ds_read_b128 %1, %9 offset:%16\n"
      "ds_read_b128 %2, %10 offset:%16\n"
      "ds_read_b128 %3, %11 offset:%16\n"
      "ds_read_b128 %4, %12 offset:%16\n"
      "ds_read_b128 %5, %13 offset:%16\n"
      "ds_read_b128 %6, %14 offset:%16\n"
      "ds_read_b128 %7, %15 offset:%16\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
      : "memory");
}
// the 16 transposed V reads of a stage: e = 0 rows at a[0][0..3] and 16 rows
// on (+4096 bytes), then e = 1 at a[1][0..3] and +4096
template <int OFF>
__device__ __forceinline__ void lds_read_vt16(const uint32_t (&a)[2][4], u32x2 (&o)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n"
      "ds_read_b64_tr_b16 %1, %17 offset:%24\n"
      "ds_read_b64_tr_b16 %2, %18 offset:%24\n"
      "ds_read_b64_tr_b16 %3, %19 offset:%24\n"
      "ds_read_b64_tr_b16 %4, %16 offset:%25\n"
      "ds_read_b64_tr_b16 %5, %17 offset:%25\n"
      "ds_read_b64_tr_b16 %6, %18 offset:%25\n"
      "ds_read_b64_tr_b16 %7, %19 offset:%25\n"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n"
      "ds_read_b64_tr_b16 %9, %21 offset:%24\n"
      "ds_read_b64_tr_b16 %10, %22 offset:%24\n"
      "ds_read_b64_tr_b16 %11, %23 offset:%24\n"
      "ds_read_b64_tr_b16 %12, %20 offset:%25\n"
      "ds_read_b64_tr_b16 %13, %21 offset:%25\n"
      "ds_read_b64_tr_b16 %14, %22 offset:%25\n"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(a[0][0]), "v"(a[0][1]), "v"(a[0][2]), "v"(a[0][3]), "v"(a[1][0]), "v"(a[1][1]), "v"(a[1][2]), "v"(a[1][3]),
        "i"(OFF), "i"(OFF + 4096)
      : "memory");
}

// the stage's 8 K fragments and its 16 transposed V reads (the two readers
// above) in one batch with one wait: 24 reads in flight instead of 8, then 16
template <int OFF>
__device__ __forceinline__ void lds_read_kv(const uint32_t (&a)[8], const uint32_t (&b)[2][4], u32x4 (&o)[8],
                                            u32x2 (&w)[16]) {
  asm volatile(
      "ds_read_b128 %0, %24 offset:%40\n"
      "ds_read_b128 %1, %25 offset:%40\n"
      "ds_read_b128 %2, %26 offset:%40\n"
      "ds_read_b128 %3, %27 offset:%40\n"
      "ds_read_b128 %4, %28 offset:%40\n"
      "ds_read_b128 %5, %29 offset:%40\n"
      "ds_read_b128 %6, %30 offset:%40\n"
      "ds_read_b128 %7, %31 offset:%40\n"
      "ds_read_b64_tr_b16 %8, %32 offset:%40\n"
      "ds_read_b64_tr_b16 %9, %33 offset:%40\n"
      "ds_read_b64_tr_b16 %10, %34 offset:%40\n"
      "ds_read_b64_tr_b16 %11, %35 offset:%40\n"
      "ds_read_b64_tr_b16 %12, %32 offset:%41\n"
      "ds_read_b64_tr_b16 %13, %33 offset:%41\n"
      "ds_read_b64_tr_b16 %14, %34 offset:%41\n"
      "ds_read_b64_tr_b16 %15, %35 offset:%41\n"
      "ds_read_b64_tr_b16 %16, %36 offset:%40\n"
      "ds_read_b64_tr_b16 %17, %37 offset:%40\n"
      "ds_read_b64_tr_b16 %18, %38 offset:%40\n"
      "ds_read_b64_tr_b16 %19, %39 offset:%40\n"
      "ds_read_b64_tr_b16 %20, %36 offset:%41\n"
      "ds_read_b64_tr_b16 %21, %37 offset:%41\n"
      "ds_read_b64_tr_b16 %22, %38 offset:%41\n"
      "ds_read_b64_tr_b16 %23, %39 offset:%41\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7]),
        "=&v"(w[8]), "=&v"(w[9]), "=&v"(w[10]), "=&v"(w[11]), "=&v"(w[12]), "=&v"(w[13]), "=&v"(w[14]), "=&v"(w[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(b[0][0]),
        "v"(b[0][1]), "v"(b[0][2]), "v"(b[0][3]), "v"(b[1][0]), "v"(b[1][1]), "v"(b[1][2]), "v"(b[1][3]), "i"(OFF),
        "i"(OFF + 4096)
      : "memory");
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4 v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, f32x4 v) {
  *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(v, bf16x4);
}

}  // namespace d128
}  // namespace ssa
