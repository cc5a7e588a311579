// Device-side building blocks shared by the phases of the persistent MoE-layer
// update kernel: element types, 8-wide vector loads/stores, wave reductions and
// the grid-wide barrier.  gfx950 (CDNA4) only: 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kThreads = 256;   // threads per workgroup (4 wavefronts)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxExperts = 64;
constexpr int kMaxTopK = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (round to nearest, ties to even; NaN stays NaN)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------------------
// 8 consecutive elements of a row, held as fp32
// ---------------------------------------------------------------------------
struct F8 {
  float v[8];
};

__device__ __forceinline__ F8 ld8(const uint16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  F8 r;
  r.v[0] = bf16_to_f32(u.x & 0xffffu); r.v[1] = bf16_to_f32(u.x >> 16);
  r.v[2] = bf16_to_f32(u.y & 0xffffu); r.v[3] = bf16_to_f32(u.y >> 16);
  r.v[4] = bf16_to_f32(u.z & 0xffffu); r.v[5] = bf16_to_f32(u.z >> 16);
  r.v[6] = bf16_to_f32(u.w & 0xffffu); r.v[7] = bf16_to_f32(u.w >> 16);
  return r;
}

__device__ __forceinline__ F8 ld8(const float* p) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  F8 r;
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  return r;
}

__device__ __forceinline__ void st8(uint16_t* p, const F8& f) {
  uint4 u;
  u.x = pack_bf16x2(f.v[0], f.v[1]);
  u.y = pack_bf16x2(f.v[2], f.v[3]);
  u.z = pack_bf16x2(f.v[4], f.v[5]);
  u.w = pack_bf16x2(f.v[6], f.v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

__device__ __forceinline__ void st8(float* p, const F8& f) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
}

__device__ __forceinline__ float to_f32(uint16_t b) { return bf16_to_f32(b); }
__device__ __forceinline__ float to_f32(float f) { return f; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16(v); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }

// ---------------------------------------------------------------------------
// Wave reductions (butterfly, fixed order: every lane ends with the same sum)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over the workgroup in a fixed order; result valid in every thread.
// `red` is kWaves floats of LDS.  Contains __syncthreads().
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];
  __syncthreads();
  return s;
}

// tanh-form GELU and its derivative (fp32), with the device tanhf.
constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;

__device__ __forceinline__ void gelu_and_grad(float h, float& a, float& da) {
  const float h2 = h * h;
  const float u = kSqrt2OverPi * (h + kGeluCubic * h2 * h);
  const float th = tanhf(u);
  a = 0.5f * h * (1.f + th);
  da = 0.5f * (1.f + th) + 0.5f * h * (1.f - th * th) * kSqrt2OverPi * (1.f + 3.f * kGeluCubic * h2);
}

// ---------------------------------------------------------------------------
// Grid barrier state.  Each workgroup owns one arrival slot (its own 128-byte
// line, so arrivals never contend); workgroup 0 publishes the generation.
// Barrier instances are numbered by a target value that the host makes unique
// per launch (launch epoch * 8 + barrier index + 1), so no reset is needed
// between launches.
// ---------------------------------------------------------------------------
struct Ctrl {
  unsigned* arrive;  // [grid][32]: slot w at arrive[w * 32]
  unsigned* gen;     // last released target
  unsigned* status;  // error bits (MOE_DEVICE_*)
  unsigned* abort;   // nonzero once any workgroup gave up waiting
};

// Bounded wait: about two seconds of the 100 MHz constant clock.
constexpr uint64_t kBarrierTimeoutTicks = 200000000ull;

// Polls *p (relaxed, agent scope) until it equals target; false on timeout or
// when another workgroup already gave up.
__device__ __forceinline__ bool wait_for(const Ctrl& c, const unsigned* p, unsigned target) {
  const uint64_t t0 = wall_clock64();
  unsigned polls = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target) {
    __builtin_amdgcn_s_sleep(2);
    if ((++polls & 255u) == 0u) {
      if (__hip_atomic_load(c.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          wall_clock64() - t0 > kBarrierTimeoutTicks) {
        __hip_atomic_fetch_or(c.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(c.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
  }
  return true;
}

// Grid-wide barrier.  Every wave first releases its own global writes at agent
// scope (waits for its stores and writes dirty L2 lines back, so the other XCDs
// see them).  A workgroup other than 0 then stores `target` into its arrival
// slot and polls the generation word; workgroup 0 polls all arrival slots in
// parallel (one per thread), acquires, and stores `target` into the generation
// word.  Polling uses plain relaxed loads with a sleep in between, and each
// poller acquires once afterwards, so waiting does not keep invalidating the
// caches under the workgroups still working.  Returns false if a wait timed out
// or another workgroup already gave up; the caller then skips all further
// phases so that every workgroup still exits.
__device__ __forceinline__ bool grid_barrier(const Ctrl& c, unsigned target, unsigned* lds_flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) *lds_flag = 1u;
  __syncthreads();
  if (blockIdx.x == 0) {
    bool ok = true;
    for (int w = threadIdx.x; w < (int)gridDim.x; w += kThreads)
      if (w != 0 && !wait_for(c, c.arrive + (size_t)w * 32, target)) {
        ok = false;
        break;
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (!ok) *lds_flag = 0u;
    __syncthreads();
    if (threadIdx.x == 0 && *lds_flag != 0u)
      __hip_atomic_store(c.gen, target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x == 0) {
    __hip_atomic_store(c.arrive + (size_t)blockIdx.x * 32, target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    if (!wait_for(c, c.gen, target)) *lds_flag = 0u;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *lds_flag != 0u;
}

}  // namespace moe
