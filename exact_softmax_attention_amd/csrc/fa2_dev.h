// fa2_dev.h — device-side helpers shared by the gfx950 attention kernels (forward and
// backward): vector types, bf16 packing, direct global->LDS loads, LDS addressing and the
// cross-half reductions of a 64-lane wave, and the work loop of the persistent kernels.
// Included by each kernel source; everything here has internal linkage except the
// declaration of the host function that hands out work-queue counters.
#ifndef FA2_DEV_H_
#define FA2_DEV_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 t = {(__bf16)lo, (__bf16)hi};               // round-to-nearest-even
  return __builtin_bit_cast(uint32_t, t);
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2 with (1, 1)): the two bf16 values
// are exact in fp32, so this sums the weights exactly as the matrix cores will see them.
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one2, acc, false);
}

// One direct global->LDS load of 16 bytes per lane: lane l's bytes at base + voff land at
// LDS address lds + 16*l. base and lds are wave-uniform. Completion is tracked by vmcnt,
// which the caller waits on explicitly before the barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)LDS_PTR(const void, p);
}

// This lane's index in its wave: mbcnt counts the set bits of an all-ones mask below the
// lane. It takes no input register, so code that needs it inside a loop can recompute it in
// two instructions instead of keeping the thread id live (or spilled) across the loop.
__device__ __forceinline__ int wave_lane() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Maximum over both 32-lane halves (lane l and l^32 hold the two halves of a row's keys).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// All ones when a row chunk starting at column col lies inside the head dimension dg, else
// zero: the mask that zeroes padded columns after an unconditional load. The empty asm
// statement (on the mask, never on loaded data) keeps the optimizer from turning the AND
// back into a branch around the load, which would make the compiler wait for that load in
// the middle of a kernel's start-up.
__device__ __forceinline__ uint32_t col_mask(int col, int dg) {
  uint32_t m = col < dg ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(m));
  return m;
}

// One direct global->LDS load of 4 bytes per lane: lane l's dword at base + voff lands at
// LDS address lds + 4*l (256 bytes per wave).
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Work loop of the persistent kernels. Every workgroup takes work item ids from queue
// q = blockIdx.x % nq of the counter set ctr (queue q hands out q, q + nq, q + 2 nq, ...) and
// runs block(id) for each, until the ids reach total. Lane 0 fetches the next id (a vector
// atomic) while the current block runs and leaves it in LDS, where the workgroup reads it
// after the barrier that closes the block. ctr[8] counts the workgroups that have finished;
// the last one returns ctr[0..8] to zero for the next launch that takes the set. block(id)
// must be uniform over the workgroup in its barriers (an early return is taken by all).
template <typename Block>
__device__ __forceinline__ void run_work_queue(unsigned int* ctr, int nq, int total, Block&& block) {
  __shared__ int next_id[2];
  const int q = (int)blockIdx.x % nq;
  auto fetch = [&]() { return (int)atomicAdd(&ctr[q], 1u) * nq + q; };
  if (threadIdx.x == 0) next_id[0] = fetch();
  __syncthreads();
  int id = next_id[0], par = 0;
  while (id < total) {
    if (threadIdx.x == 0) next_id[par ^ 1] = fetch();
    block(id);
    __syncthreads();
    par ^= 1;
    id = next_id[par];
  }
  if (threadIdx.x == 0) {
    __threadfence();
    if (atomicAdd(&ctr[8], 1u) == gridDim.x - 1) {
#pragma unroll
      for (int c = 0; c < 9; ++c) atomicExch(&ctr[c], 0u);
    }
  }
}

}  // namespace

// Host side, defined with the forward: the device address of the next counter set (16 words)
// of a per-device pool for a persistent launch on device dev; sets are taken in turn and
// each is zero when taken. Returns a status code.
namespace fa2_internal {
int queue_counters(int dev, unsigned int** out);
}

#endif  // FA2_DEV_H_
