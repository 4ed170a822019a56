// Device helpers shared by the persistent recurrent kernels (gfx950): the
// exchange-ring stores and flag waits, the MFMA sweep over a wave's granule
// range, LDS staging, and the co-residency query used by their launchers.
#pragma once

#include <type_traits>

#include "device_util.h"
#include "rnn_common.h"

extern __shared__ __attribute__((aligned(16))) char dyn_lds[];

namespace rnnk {
namespace {

template <bool BF16>
using XT = typename std::conditional<BF16, uint16_t, float>::type;

template <bool BF16>
__device__ __forceinline__ XT<BF16> to_x(float v) {
  if constexpr (BF16) return f2bf(v); else return v;
}
template <bool BF16>
__device__ __forceinline__ uint32_t w_bits(const void* base, size_t idx) {
  if constexpr (BF16) return reinterpret_cast<const uint16_t*>(base)[idx];
  else return __float_as_uint(reinterpret_cast<const float*>(base)[idx]);
}
// Pack PER values (bits) into a 16-byte fragment.
template <bool BF16>
__device__ __forceinline__ uint4 pack_frag(const uint32_t (&v)[BF16 ? 8 : 4]) {
  if constexpr (BF16)
    return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  else
    return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_load16(const char __attribute__((address_space(3)))* p) {
  const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool BF16>
__device__ __forceinline__ void ring_store(char* base, size_t off, float v) {
  if (v != v) v = __uint_as_float(0x7FC00000u);   // canonical NaN: never the sentinel
  if constexpr (BF16)
    __hip_atomic_store(reinterpret_cast<uint16_t*>(base + off), f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_store(reinterpret_cast<float*>(base + off), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compiler-only ordering point: no memory operation is moved across it at
// the IR level (the s_waitcnt builtin does not order memory operations
// there); it emits no instruction.  The hardware order of the exchange is
// given by the waits around it.
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Ordering-perturbation build (compiled with -DRNN_PERTURB, a test build):
// a pseudo-random pause of 0 to ~6 us, half the time none, at every ordering
// point of the exchange -- each wave's entry to a flag wait, each wave's
// entry to a flag publication (before its stores are waited for) and a
// workgroup's exit from it -- so that producers, consumers and the waves of
// one workgroup run with skews they never have in the normal build.  It
// changes no arithmetic: a correct protocol gives bitwise the results of the
// normal build.  Without the macro it is empty.
__device__ __forceinline__ void perturb_pause(unsigned a, unsigned b, unsigned site) {
#ifdef RNN_PERTURB
  unsigned x = a * 0x9E3779B1u ^ b * 0x85EBCA77u ^ (site + 1u) * 0xC2B2AE3Du;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  x *= 0x297A2D39u;
  x ^= x >> 15;
  const unsigned n = (x & 1u) ? 0u : (x >> 1) & 31u;
  for (unsigned i = 0; i < __builtin_amdgcn_readfirstlane(n); ++i) __builtin_amdgcn_s_sleep(8);
#else
  (void)a;
  (void)b;
  (void)site;
#endif
}

__device__ __forceinline__ unsigned wave_tag() {
  return blockIdx.x * 16u + (unsigned)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Bounded wait of one wave for the flags of two ranges of producers,
// [a0, a0 + na) and [b0, b0 + nb) (flag indices), to reach `target`.
// Returns false (uniformly over the wave) if the wait expired -- the error
// word is then set -- or another workgroup reported an error.  A spin limit
// of 0 expires every wait at once (a host-forced timeout for tests).  The
// callers order their reads of the producers' ring lines after a successful
// wait by computing the read addresses through an empty asm statement that
// follows it (a register dependency the compiler cannot hoist above the
// loop); a compiler fence at this exit measured 0.06 us per step slower.
__device__ bool wave_wait(const unsigned* flags, unsigned* err, unsigned spin_limit, int a0, int na,
                          int b0, int nb, unsigned target) {
  if (spin_limit == 0) {
    flag_store(err, 1u);
    return false;
  }
  perturb_pause(wave_tag(), target, 0u);
  const int lane = threadIdx.x & 63;
  const int total = na + nb;
  const int nper = (total + 63) / 64;   // flags per lane, uniform
  unsigned it = 0;
  while (true) {
    // issue every flag load of this round before looking at any of them
    unsigned v[kWaitPerLane];
#pragma unroll
    for (int i = 0; i < kWaitPerLane; ++i) {
      const int idx = lane + 64 * i;
      v[i] = target;
      if (i < nper && idx < total) {
        const int w = idx < na ? a0 + idx : b0 + (idx - na);
        v[i] = flag_load(flags + (size_t)w * kFlagStride);
      }
    }
    bool mine = true;
#pragma unroll
    for (int i = 0; i < kWaitPerLane; ++i) mine = mine && v[i] >= target;
    if (__all(mine)) return true;
    if (++it > spin_limit) {
      flag_store(err, 1u);
      return false;
    }
    if ((it & 31u) == 0 && flag_load(err) != 0u) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Logical index (group * nwg + slice) of this workgroup in a sweep's grid,
// or -1 for a workgroup with no work.  place 0: blockIdx.x.  place 1
// (XCD-local groups): the dispatcher deals workgroups to the XCDs round-robin
// (blockIdx.x % kXcds); group g gets slots (g / kXcds) * nwg .. + nwg - 1 of
// XCD g % kXcds, so all producers and consumers of one group share that
// XCD's L2.  place r >= 2: runs of r consecutive logical workgroups on one
// XCD, so that neighbouring slices, whose per-unit fp32 data (the input
// projection, the reserve, dy) share 128-byte lines, are read through one
// L2.  Correctness never depends on where a workgroup actually runs: the
// exchange is coherent at agent scope.
__device__ __forceinline__ int logical_wg(int place, int nwg, int ngroups) {
  const int b = blockIdx.x;
  if (place == 0) return b;
  const int x = b % kXcds, k = b / kXcds;
  if (place >= 2) {
    // runs of `place` consecutive workgroups per XCD: workgroup k of XCD x
    // takes logical index (k / r) * 8r + x * r + k % r
    const int r = place;
    const int l = (k / r) * (kXcds * r) + x * r + k % r;
    return l < nwg * ngroups ? l : -1;
  }
  const int row = k / nwg, j = k - row * nwg;
  const int g = row * kXcds + x;
  return g < ngroups ? g * nwg + j : -1;
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for the wave's outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Every wave waits for completion of its stores (the ring stores are agent
// scope), then one thread publishes the flag.  `wave0_only`: every ring store
// of the step was made by wave 0, so wave 0 alone waits for them and
// publishes, with no workgroup barrier before the flag (the other waves meet
// wave 0 again at the step's closing LDS barrier).
// `id`: the workgroup's flag index (its logical index in the sweep's grid).
// Ordering assumed of the hardware (gfx950): an agent-scope store is
// written through to the device-coherent level, and s_waitcnt(0) returns only
// once every earlier store of the wave has been acknowledged there; so a
// consumer that sees the flag and then issues plain loads of lines it never
// touched before reads the stored values.  Compiler fences keep the ring
// stores before the wait and the flag store after it.
__device__ __forceinline__ void publish(unsigned* flags, int id, unsigned v, bool wave0_only = false) {
  compiler_fence();
  perturb_pause(wave_tag(), v, 1u);
  if (wave0_only) {
    if (threadIdx.x < 64) {
      __builtin_amdgcn_s_waitcnt(0);
      compiler_fence();
      if (threadIdx.x == 0) flag_store(flags + (size_t)id * kFlagStride, v);
    }
    perturb_pause(blockIdx.x, v, 2u);
    return;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  compiler_fence();
  if (threadIdx.x == 0) flag_store(flags + (size_t)id * kFlagStride, v);
  perturb_pause(blockIdx.x, v, 2u);
}

// MFMA over the granules this wave holds.  K chunk kk takes granules
// 4*kk + fq of the wave's range (fq = lane / 16): a lane feeds one granule's
// 16 bytes of row `row` as its A fragment, `load(gl, row)`, and the matching
// weights sit in wf[kk].  Lanes past the end of the range re-read its last
// granule (their weights are zero), and tile rows past the granule's padded
// rows re-read its last row: no load leaves the granules the wave has waited
// for, and such rows only feed output rows that are never used.  All loads of
// a batch (at most KBMAX chunks) are issued before its MFMAs.
template <bool BF16, int NT, int MT, int KPW, int KBMAX = 8, class LoadF>
__device__ __forceinline__ void mfma_sweep(f32x4 (&acc)[MT][NT], const uint4 (&wf)[KPW][NT], int fr,
                                           int fq, int nmine, int rmax, LoadF load) {
  constexpr int KB = KPW < KBMAX ? KPW : KBMAX;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KPW; kb += KB) {
    if (kb * 4 >= nmine) break;   // uniform over the wave
    uint4 av[KB][MT];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int gl = min((kb + kk) * 4 + fq, nmine - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[kk][mt] = load(gl, min(mt * 16 + fr, rmax));
    }
    // keep the whole batch of loads in flight before the first MFMA
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_chunk<BF16>(av[kk][mt], wf[kb + kk][nt], acc[mt][nt]);
  }
}

// Copy granules [g0, g0 + n) of a ring entry to the same offsets in LDS with
// direct global->LDS loads (lane i of an instruction moves 16 bytes to
// M0 + 16*i); nothing passes through registers, so the whole range is in
// flight at once.  The issuing wave waits for its own loads only.
__device__ __forceinline__ void stage_granules(char __attribute__((address_space(3)))* lds, const char* src,
                                               int g0, int n, int gran, int lane) {
  const int n16 = n * (gran >> 4);
  const int base = g0 * gran;
  for (int c = 0; c < n16; c += 64)
    if (c + lane < n16)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(src + base + (size_t)(c + lane) * 16),
          (void __attribute__((address_space(3)))*)(lds + base + c * 16), 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);
}


// Maximum co-resident workgroups of kernel `f` with `nthr` threads and `lds`
// bytes of dynamic LDS (0 if it cannot run at all).
inline int max_resident(const void* f, int nthr, size_t lds) {
  int per_cu = 0;
  if (lds > 0) {
    // static + dynamic LDS must fit the per-workgroup limit; failed runtime
    // calls are cleared so that no error state leaks to the caller
    int dev = 0, lim = 0;
    hipFuncAttributes fa{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, f) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    if (fa.sharedSizeBytes + lds > (size_t)lim) return 0;
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, nthr, lds) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return per_cu * ncu;
}

}  // namespace
}  // namespace rnnk
