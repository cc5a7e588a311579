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

// fp32 -> bf16 with round-to-nearest-even: the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32), two values at a time
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

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

// 8 consecutive elements as loaded (16 bytes of bf16, 32 of fp32), converted
// to F8 only where they are used
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  uint4 u;
};
template <>
struct Raw8<float> {
  float4 a, b;
};

__device__ __forceinline__ Raw8<uint16_t> ldr8(const uint16_t* p) { return {*reinterpret_cast<const uint4*>(p)}; }
__device__ __forceinline__ Raw8<float> ldr8(const float* p) {
  return {reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
}

__device__ __forceinline__ F8 cvt8(const Raw8<uint16_t>& r) {
  F8 f;
  f.v[0] = bf16_to_f32(r.u.x & 0xffffu); f.v[1] = bf16_to_f32(r.u.x >> 16);
  f.v[2] = bf16_to_f32(r.u.y & 0xffffu); f.v[3] = bf16_to_f32(r.u.y >> 16);
  f.v[4] = bf16_to_f32(r.u.z & 0xffffu); f.v[5] = bf16_to_f32(r.u.z >> 16);
  f.v[6] = bf16_to_f32(r.u.w & 0xffffu); f.v[7] = bf16_to_f32(r.u.w >> 16);
  return f;
}
__device__ __forceinline__ F8 cvt8(const Raw8<float>& r) {
  F8 f;
  f.v[0] = r.a.x; f.v[1] = r.a.y; f.v[2] = r.a.z; f.v[3] = r.a.w;
  f.v[4] = r.b.x; f.v[5] = r.b.y; f.v[6] = r.b.z; f.v[7] = r.b.w;
  return f;
}

__device__ __forceinline__ void st8(uint16_t* p, const F8& f) {
  uint4 u;
  u.x = pack_bf16x2(f.v[0], f.v[1]);
  u.y = pack_bf16x2(f.v[2], f.v[3]);
  u.z = pack_bf16x2(f.v[4], f.v[5]);
  u.w = pack_bf16x2(f.v[6], f.v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

// Non-temporal forms, for outputs that are only read again in a later phase
// and are too large to stay in the caches meanwhile: they do not displace the
// operand lines the phase is still reusing.
typedef unsigned ntu4_t __attribute__((ext_vector_type(4)));
typedef float ntf4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st8nt(uint16_t* p, const F8& f) {
  const ntu4_t u = {pack_bf16x2(f.v[0], f.v[1]), pack_bf16x2(f.v[2], f.v[3]), pack_bf16x2(f.v[4], f.v[5]),
                    pack_bf16x2(f.v[6], f.v[7])};
  __builtin_nontemporal_store(u, reinterpret_cast<ntu4_t*>(p));
}
__device__ __forceinline__ void st8nt(float* p, const F8& f) {
  __builtin_nontemporal_store(ntf4_t{f.v[0], f.v[1], f.v[2], f.v[3]}, reinterpret_cast<ntf4_t*>(p));
  __builtin_nontemporal_store(ntf4_t{f.v[4], f.v[5], f.v[6], f.v[7]}, reinterpret_cast<ntf4_t*>(p) + 1);
}
__device__ __forceinline__ void st8(float* p, const F8& f) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
}


// A store of the product epilogues.  `nt` (the same for the whole launch)
// picks the non-temporal form: it keeps large outputs from displacing the
// operand lines a phase still reuses, while small ones are better left in the
// caches for the phase that reads them next.
template <typename P>
__device__ __forceinline__ void st8s(P* p, const F8& f, bool nt) {
  if (nt) st8nt(p, f);
  else st8(p, f);
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

// Workgroup barrier for LDS traffic only: each wave waits for its own LDS
// accesses, not for its global stores (which __syncthreads would drain), so
// stores issued before it stay in flight.  Not for global data exchanged
// between the waves of a workgroup.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left alone
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// Sum over the workgroup in a fixed order; result valid in every thread.
// `red` is kWaves floats of LDS.  Synchronises the workgroup (LDS only).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lds_sync();
  if (lane == 0) red[wave] = v;
  lds_sync();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];
  lds_sync();
  return s;
}

// tanh-form GELU and its derivative (fp32).  With u = sqrt(2/pi) (h + 0.044715
// h^3) and r = 1 / (1 + e^{2u}), the identity tanh(u) = 1 - 2r gives
//   gelu(h)  = h (1 - r)
//   gelu'(h) = (1 - r) + 2 h r (1 - r) sqrt(2/pi) (1 + 3 * 0.044715 h^2)
// and 1 - r = e^{2u} r keeps full relative precision where e^{2u} is small.
// e^{2u} comes from the hardware base-2 exponential and r from the hardware
// reciprocal (about 1 ulp each); the exponent is capped at 2^64 so that
// e^{2u} r stays finite.
constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;
constexpr float kTwoLog2e = 2.8853900817779268f;   // 2 / ln 2

// r and 1 - r = e^{2u} r of the identity above
__device__ __forceinline__ void gelu_parts(float h, float h2, float& r, float& s) {
  const float t = fminf(kTwoLog2e * kSqrt2OverPi * h * (1.f + kGeluCubic * h2), 64.f);   // 2u log2(e)
  const float e = __builtin_amdgcn_exp2f(t);
  r = __builtin_amdgcn_rcpf(1.f + e);
  s = e * r;   // 1 - r
}

__device__ __forceinline__ void gelu_and_grad(float h, float& a, float& da) {
  const float h2 = h * h;
  float r, s;
  gelu_parts(h, h2, r, s);
  a = h * s;
  da = s + 2.f * kSqrt2OverPi * h * r * s * (1.f + 3.f * kGeluCubic * h2);
}

__device__ __forceinline__ float gelu_only(float h) {
  float r, s;
  gelu_parts(h, h * h, r, s);
  return h * s;
}

// ---------------------------------------------------------------------------
// Grid barrier state.  Each workgroup owns one arrival slot (its own 128-byte
// line, so arrivals never contend); workgroup 0 publishes the generation.
// Barrier instances are numbered by a target value that the host makes unique
// per launch (launch epoch * 8 + barrier index + 1), so no reset is needed
// between launches.
// ---------------------------------------------------------------------------
struct Ctrl {
  unsigned* arrive;  // [grid][32]: slot w at arrive[w * 32]; word 1 holds w's XCD
  unsigned* gen;     // last released target
  unsigned* status;  // error bits (MOE_DEVICE_*)
  unsigned* abort;   // nonzero once any workgroup gave up waiting
  unsigned* never;   // a word nothing writes (the failure-path test waits on it)
  unsigned* xcd;     // per-XCD words (kXcdWords): members of XCD x at xcd[x], its
                     // arrival counter at xcd[32 (1 + x)], its arrival slot at xcd[32 (9 + x)]
  uint64_t limit;    // bound of every wait, in ticks of the 100 MHz constant clock
  int per_wg;        // 1: every barrier writes back each workgroup's L2 itself
};
constexpr int kMaxXcd = 8;
constexpr int kXcdWords = 32 * (1 + 2 * kMaxXcd);

// Barrier bookkeeping a workgroup keeps in LDS for the whole launch.
struct BarrierState {
  unsigned flag;              // result broadcast to the workgroup
  unsigned xcc;               // this workgroup's XCD (hardware register)
  unsigned xmem;              // workgroups on that XCD in this launch
  unsigned xall[kMaxXcd];     // workgroup 0: workgroups on every XCD
};

// Bounded wait: about two seconds of the 100 MHz constant clock.
constexpr uint64_t kBarrierTimeoutTicks = 200000000ull;
// The bound under the failure-path test flag: about 10 us.
constexpr uint64_t kTestTimeoutTicks = 1000ull;

// The XCD (and so the L2) this wave runs on.
__device__ __forceinline__ unsigned xcc_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

// Release at agent scope (the XCD's dirty L2 lines are written back to
// memory), completed before the caller's next memory operation.  The fence
// emits the L2 write-back; the compiler does not always follow it with a wait
// on the vector-memory counter (it dropped it after an earlier explicit wait),
// so the wait is issued here as an instruction it cannot remove.
__device__ __forceinline__ void release_agent() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// A wait that gives up: the timeout bit and the abort word are set, so every
// other workgroup's waits give up as well and the whole grid exits.
__device__ __forceinline__ bool give_up(const Ctrl& c) {
  __hip_atomic_fetch_or(c.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(c.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// Polls *p (relaxed, agent scope) until it equals target; false on timeout or
// when another workgroup already gave up (checked every 256 polls).
__device__ __forceinline__ bool wait_for(const Ctrl& c, const unsigned* p, unsigned target) {
  const uint64_t t0 = wall_clock64();
  unsigned polls = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != target) {
    __builtin_amdgcn_s_sleep(2);
    if ((++polls & 255u) == 0u) {
      if (__hip_atomic_load(c.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          wall_clock64() - t0 > c.limit)
        return give_up(c);
    }
  }
  return true;
}

// Polls *p (relaxed, agent scope) until it is at least target (barrier
// targets only grow: within a launch with the barrier index, across launches
// with the launch number); false on timeout or when another workgroup already
// gave up.
__device__ __forceinline__ bool wait_reached(const Ctrl& c, const unsigned* p, unsigned target) {
  const uint64_t t0 = wall_clock64();
  unsigned polls = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if ((++polls & 255u) == 0u) {
      if (__hip_atomic_load(c.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          wall_clock64() - t0 > c.limit)
        return give_up(c);
    }
  }
  return true;
}

// Polls *p (relaxed, agent scope) until it is at least target; false on
// timeout or when another workgroup already gave up.
__device__ __forceinline__ bool wait_count(const Ctrl& c, const int* p, int target) {
  const uint64_t t0 = wall_clock64();
  unsigned polls = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(1);
    if ((++polls & 255u) == 0u) {
      if (__hip_atomic_load(c.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
          wall_clock64() - t0 > c.limit)
        return give_up(c);
    }
  }
  return true;
}

// Grid-wide barrier.  Every wave first waits until its own stores have reached
// its XCD's L2 (vmcnt), then:
//
// * Per-workgroup release (the first barrier of every launch, and every
//   barrier with Ctrl::per_wg): one wave releases at agent scope for the whole
//   workgroup (its XCD's dirty L2 lines are written back), then the workgroup
//   stores `target` into its arrival slot.  Workgroup 0 polls all slots in
//   parallel (one per thread), acquires, and stores `target` into the
//   generation word.  At the first barrier each workgroup also records the XCD
//   it runs on (HW_REG_XCC_ID) in its slot; workgroup 0 counts the workgroups
//   of each XCD and publishes the counts and zeroed XCD counters with the
//   generation.  (A first barrier without any write-back, with the routing
//   histogram stored at agent scope instead, measured 15 us slower per update:
//   the next barrier and the acquires then meet those dirty lines.)
// * One release per XCD (every later barrier, hk = 1, 2, ...): a workgroup adds
//   1 to its XCD's arrival counter (an atomic, performed where all XCDs see
//   it).  The workgroup that brings the counter to members * hk arrived last on
//   its XCD: all its XCD's workgroups had their stores in that L2 before they
//   counted, so its one write-back covers them all; it then stores `target`
//   into the XCD's arrival slot.  Every workgroup polls the slots of the XCDs
//   that have members (one lane each) and acquires once all eight hold the
//   target.  The membership comes from the hardware register in this very
//   launch, so it holds whatever the dispatch order was.
//
// Polling uses relaxed loads with a sleep between polls, and each poller
// acquires once afterwards.  Returns false if a wait timed out or another
// workgroup already gave up; the caller then skips all further phases so that
// every workgroup still exits.
__device__ __forceinline__ bool grid_barrier(const Ctrl& c, unsigned target, BarrierState* bs, int hk) {
  const int tid = threadIdx.x;
  const bool per_wg = hk == 0 || c.per_wg != 0;
  if (hk == 0 && tid == 0) {
    bs->xcc = xcc_id();
    if (blockIdx.x != 0)
      __hip_atomic_store(c.arrive + (size_t)blockIdx.x * 32 + 1, bs->xcc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are in L2 (agent-scope ones in memory)
  __syncthreads();
  if (per_wg) {
    if (tid < 64) release_agent();
    if (tid == 0) bs->flag = 1u;
  } else if (tid == 0) {
    bs->flag = 1u;
    const unsigned x = bs->xcc & (kMaxXcd - 1);
    const unsigned old = __hip_atomic_fetch_add(c.xcd + 32 * (1 + x), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == bs->xmem * (unsigned)hk) {
      release_agent();   // the last of its XCD: one write-back for all of them
      __hip_atomic_store(c.xcd + 32 * (9 + x), target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!per_wg) {
    // every workgroup polls the arrival slots of the XCDs that have members
    // itself (eight lines, one lane each): no relay through a generation word.
    // "At least": an XCD whose workgroups have all passed this barrier may
    // already have stored the next barrier's target before a slow poller saw
    // this one.
    if (tid < kMaxXcd && bs->xall[tid] > 0u && !wait_reached(c, c.xcd + 32 * (9 + tid), target)) bs->flag = 0u;
    if (tid < 64) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    return bs->flag != 0u;
  }
  if (blockIdx.x == 0) {
    bool ok = true;
    for (int w = tid; w < (int)gridDim.x; w += kThreads)
      if (w != 0 && !wait_for(c, c.arrive + (size_t)w * 32, target)) {
        ok = false;
        break;
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (!ok) bs->flag = 0u;
    if (hk == 0) {
      // XCD membership of this launch
      __syncthreads();
      if (tid < kMaxXcd) bs->xall[tid] = 0u;
      __syncthreads();
      for (int w = tid; w < (int)gridDim.x; w += kThreads) {
        const unsigned x = w == 0 ? bs->xcc
                                  : __hip_atomic_load(c.arrive + (size_t)w * 32 + 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        atomicAdd(&bs->xall[x & (kMaxXcd - 1)], 1u);
      }
      __syncthreads();
      if (tid < kMaxXcd) {
        __hip_atomic_store(c.xcd + tid, bs->xall[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(c.xcd + 32 * (1 + tid), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // these stores are performed before the generation
    }
    __syncthreads();
    if (tid == 0 && bs->flag != 0u)
      __hip_atomic_store(c.gen, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (tid == 0) {
    __hip_atomic_store(c.arrive + (size_t)blockIdx.x * 32, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!wait_for(c, c.gen, target)) bs->flag = 0u;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (hk == 0) {
    // every workgroup keeps the membership counts (which XCD slots to poll,
    // and how many arrivals complete its own XCD)
    if (blockIdx.x != 0 && tid < kMaxXcd)
      bs->xall[tid] = __hip_atomic_load(c.xcd + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid == 0) bs->xmem = bs->xall[bs->xcc & (kMaxXcd - 1)];
    __syncthreads();
  }
  return bs->flag != 0u;
}

}  // namespace moe
