// Persistent recurrent kernels: one launch walks all T steps.
//
// Partition. The batch is cut into groups of BG = 16*MB rows and the hidden
// units into slices of HS units; workgroup (group, slice) owns the hidden
// units of its slice for every gate, so the cell update needs no exchange.
// Its slice of W_hh (all gate rows of its units in the forward pass, all
// gate-row columns of its units in the backward pass) is loaded once into
// VGPRs as MFMA B operands and stays there for the whole sequence: the
// weight-stationary scheme of the persistent backward kernel on the CUDA
// fragment page (the recurrent tile lives in registers across steps), here
// with the contraction split over the waves of the workgroup and the partial
// products summed through LDS.
//
// Exchange. The only data that crosses workgroups is the recurrent vector of
// a step (forward: h_t, backward: the gate gradients dG_t), which every
// workgroup of the batch group reads in full at the next step. Producers
// store it, wait until their stores are acknowledged and publish a
// per-workgroup step counter; consumers poll the counters of their group
// (one coalesced load per wave) and then read the vector. The CUDA
// fragment's kernel waits on the data itself (a -0.0 sentinel) with no
// bound; here every wait is bounded by a wall-clock time-out that sets a
// status word, after which all waits are skipped so that every wave still
// runs to the end of the grid.
//
// Coherence point. Each XCD has its own L2, which is coherent for the CUs of
// that XCD: a plain store is acknowledged once it sits in the L2, and a load
// with the device-scope bit (sc1) skips the CU's L1 and is served by the
// L2. A batch group whose workgroups all run on one XCD therefore exchanges
// through its L2 (plain stores, sc1 loads). At launch every workgroup
// publishes its XCC id with a device-scope store and reads those of its
// group; only when they all match does the group use the L2 path. Otherwise
// it falls back to device-scope stores, which write through to memory and
// are seen by sc1 loads from any XCD. No whole-cache write-back or
// invalidate is issued per step.
//
// Equations (canonical gate order, fp32 arithmetic, storage rounding on
// store): LSTM popnn Lstm.cpp "basicLstmCellForwardPass" and
// "backwardStepImpl"; GRU popnn Gru.cpp "basicGruCellForwardPass",
// "gruCellForwardPassCalcUnitsResetAfter", "backwardStepImpl" and
// "backwardStepImplResetAfter".
#include <algorithm>
#include <type_traits>

#include "rnn_internal.hpp"

namespace rnn {

#ifdef RNN_STEP_TIMERS
// Thread 0 keeps the step's clock readings in LDS (no vector-memory store
// inside the loop, which would join the memory counters the kernel waits
// on) and copies them out when the kernel ends.
static __device__ unsigned long long g_step_timers[TIMER_WGS * TIMER_STEPS * TIMER_PHASES];
static __device__ unsigned long long g_step_cal[TIMER_WGS * 4];
#define STEP_TIMER_DECL __shared__ unsigned step_tl_[TIMER_STEPS * TIMER_PHASES]
#define STEP_TIMER(step, phase)                                                   \
  do {                                                                            \
    if (threadIdx.x == 0 && (step) >= 0 && (step) < TIMER_STEPS)                  \
      step_tl_[(step) * TIMER_PHASES + (phase)] = (unsigned)__builtin_amdgcn_s_memtime(); \
  } while (0)
// (which 0, at the start of the step loop: also clears the LDS buffer, so
// that a point a step does not pass reads as zero)
#define STEP_TIMER_CAL(which)                                                                 \
  do {                                                                                        \
    if ((which) == 0) {                                                                       \
      for (int i_ = threadIdx.x; i_ < TIMER_STEPS * TIMER_PHASES; i_ += blockDim.x) step_tl_[i_] = 0u; \
      __syncthreads();                                                                        \
    }                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < TIMER_WGS) {                                         \
      g_step_cal[blockIdx.x * 4 + 2 * (which)] = __builtin_amdgcn_s_memtime();                \
      g_step_cal[blockIdx.x * 4 + 2 * (which) + 1] = __builtin_amdgcn_s_memrealtime();        \
    }                                                                                         \
  } while (0)
#define STEP_TIMER_FLUSH(nsteps)                                                              \
  do {                                                                                        \
    __syncthreads();                                                                          \
    if (blockIdx.x < TIMER_WGS)                                                               \
      for (int i_ = threadIdx.x; i_ < min((nsteps), TIMER_STEPS) * TIMER_PHASES; i_ += blockDim.x) \
        g_step_timers[(size_t)blockIdx.x * TIMER_STEPS * TIMER_PHASES + i_] = step_tl_[i_];   \
  } while (0)
hipError_t reset_step_timers() {
  static unsigned long long zeros[TIMER_WGS * 4] = {};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_step_cal), zeros, sizeof(zeros));
}
hipError_t read_step_timers(unsigned long long* timers, unsigned long long* cal) {
  hipError_t e = hipMemcpyFromSymbol(timers, HIP_SYMBOL(g_step_timers), sizeof(g_step_timers));
  if (e == hipSuccess) e = hipMemcpyFromSymbol(cal, HIP_SYMBOL(g_step_cal), sizeof(g_step_cal));
  return e;
}
#else
#define STEP_TIMER_DECL
#define STEP_TIMER(step, phase) ((void)0)
#define STEP_TIMER_CAL(which) ((void)0)
#define STEP_TIMER_FLUSH(nsteps) ((void)0)
#endif

namespace {

constexpr int ST_TIMEOUT = -5;

// Step counters and exchanged vectors are read with device-scope (sc1)
// loads: they skip the CU's L1 and never return a stale line. Writers use
// plain stores when the whole batch group shares one XCD's L2 (`local`) and
// device-scope stores otherwise. Data that only the owning workgroup or a
// later kernel reads (saved gates, cell states) always uses plain stores.
// `idle` (optional) is work that does not depend on the counters: it runs
// once, while the first poll is in flight.
struct NoIdle {
  __device__ void operator()() const {}
};
template <typename Idle = NoIdle>
__device__ __forceinline__ void wait_flags(const int* f, int n, int target, int* status, long long timeout,
                                           int stride = 1, bool pipe = false, Idle idle = Idle()) {
  constexpr bool HOOK = !std::is_same<Idle, NoIdle>::value;
  const int lane = threadIdx.x & 63;
  if (timeout < 0) {
    // a limit of no time at all (set from the host to exercise the error
    // path): the wait gives up at once
    if (lane == 0) __hip_atomic_store(status, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  long long t0 = 0;
  if constexpr (HOOK) {
    // one poll (lanes past n read counter 0) in flight while `idle` runs
    const int v = __hip_atomic_load(f + (lane < n ? lane : 0) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_sched_barrier(0);
    idle();
    __builtin_amdgcn_sched_barrier(0);
    if (n <= 64 && __all(v >= target)) {
      asm volatile("" ::: "memory");
      return;
    }
  }
  if (pipe && n <= 64) {
    // One counter per lane, two polls in flight: a new poll is issued as
    // soon as the older one has been checked, so a counter set while one
    // poll is on its way is seen by the next about half an L2 round trip
    // later rather than a whole one. The status word and the time-out are
    // looked at only once a wait has lasted over 20 us (never in a normal
    // step), so that the loop carries no other load.
    const int* p = f + (lane < n ? lane : 0) * stride;
    int v0 = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_sleep(4);
    int v1 = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    t0 = (long long)wall_clock64();
    // runs of polls in straight-line code (the compiler then tracks the two
    // loads in flight exactly), the first one ahead of the loop; the
    // time-out between runs
    auto run = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (__all(v0 >= target)) return true;
        v0 = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__all(v1 >= target)) return true;
        v1 = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return false;
    };
    bool done = run();
    while (!done) {
      done = run();
      if (done) break;
      const long long now = (long long)wall_clock64();
      if (now - t0 > (timeout >> 19)) {
        if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        if (now - t0 > timeout) {
          if (lane == 0) __hip_atomic_store(status, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    asm volatile("" ::: "memory");
    return;
  }
  for (int it = 0;; ++it) {
    bool ok = true;
    for (int i = lane; i < n; i += 64)
      ok = ok && (__hip_atomic_load(f + i * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target);
    if (__all(ok)) break;
    if ((it & 63) == 0) {
      if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
      const long long now = (long long)wall_clock64();
      if (it == 0) {
        t0 = now;
      } else if (now - t0 > timeout) {
        if (lane == 0) __hip_atomic_store(status, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
  // the vector reads below must not be moved above the poll
  asm volatile("" ::: "memory");
}

// The slices a wave's share of the contraction depends on: contraction rows
// [k0, k1) read the exchanged values of units k % H, which slice u / HS
// produces. A range covering H units or wrapping past H depends on every
// slice; an empty one on none. The waves of a workgroup together cover the
// whole contraction, so after the barrier that follows the contraction the
// workgroup has waited for every slice (which the reuse of exchange slots
// two steps later relies on).
__device__ __forceinline__ void wave_slices(int k0, int k1, int H, int HS, int nS, int& s0, int& n) {
  if (k1 <= k0) {
    s0 = 0;
    n = 0;
    return;
  }
  const int u0 = k0 % H, u1 = (k1 - 1) % H;
  if (k1 - k0 >= H || u1 < u0) {
    s0 = 0;
    n = nS;
    return;
  }
  s0 = u0 / HS;
  n = u1 / HS + 1 - s0;
}

// Every wave waits for its stores of the exchanged vector to be
// acknowledged, the workgroup meets, then one thread publishes the step
// counter.
__device__ __forceinline__ void publish(int* f, int v, bool local) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (local) *f = v;
    else __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// store of one exchanged element: plain within one XCD, device scope across
__device__ __forceinline__ void xstore(float* p, float v, bool local) {
  if (local) *p = v;
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xstore(bf16* p, float v, bool local) {
  const unsigned short u = __builtin_bit_cast(unsigned short, (bf16)v);
  if (local) *(unsigned short*)p = u;
  else __hip_atomic_store((unsigned short*)p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Placement check at launch: every workgroup publishes 1 + its XCC id in the
// second word of its counter line with a device-scope store, waits (device
// scope) until all members of its batch group have done so and compares.
// Every wave reads the same published values, so the whole group agrees.
__device__ __forceinline__ bool group_is_local(int* myflag, const int* gflags, int n, int stride, int place_off,
                                               int* status, long long timeout) {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  x = (x & 15) + 1;
  if (threadIdx.x == 0) __hip_atomic_store(myflag + place_off, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_flags(gflags + place_off, n, 1, status, timeout, stride);
  bool same = true;
  for (int i = threadIdx.x & 63; i < n; i += 64)
    same = same && (__hip_atomic_load(gflags + place_off + i * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == x);
  return __all(same);
}

constexpr int BUF_RSRC_W3 = 0x00020000;  // buffer resource word 3 for the gfx9 family
constexpr int CPOL_SC1 = 16;             // device scope
constexpr int BUF_SKIP = 0x40000000;     // an offset past every buffer below: the access is dropped

// One storage element through a buffer resource: an offset at or past the
// resource's size is dropped by the hardware, so a store can be issued
// unconditionally (no branch), which keeps the count of memory operations a
// wave has in flight the same on every path.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF),
                                           BUF_RSRC_W3);
}
template <typename TS>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t rs, int off, float v) {
  if constexpr (sizeof(TS) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)v), rs, off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, 0);
}

// Workgroup -> (group, slice). Workgroups are dispatched round-robin over the
// 8 XCDs; consecutive workgroups of one batch group are placed on the same
// XCD where the counts allow, so that the vector they exchange stays in few
// L2s. Correctness does not depend on the placement.
// Direction and workgroup coordinates of this block. One direction: block b
// sits on XCD b%8 (round-robin dispatch); with a workgroup count divisible by
// 8 the logical index is XCD-contiguous, so a batch group (nSlices
// consecutive indices) shares an XCD where it fits in one. Dual launch:
// blocks on XCDs 0-3 run direction 0 and those on XCDs 4-7 direction 1, each
// XCD holding n/4 consecutive indices of its direction.
typedef const __attribute__((address_space(4))) RecArgs RecArgsK;
static_assert(offsetof(RecLaunch, d) == 0, "RecLaunch.d leads the kernel arguments");

// Padded placement (per_xcd > 0): each XCD of a direction holds per_xcd
// consecutive logical indices (whole batch groups), so that a group of
// fewer workgroups than fit an XCD, but more than n / 8, still shares one
// L2; the launch has xcds * per_xcd blocks per direction and those past the
// plan's n workgroups return at once (`idle`).
__device__ __forceinline__ RecArgsK& launch_slot(const RecLaunch& L, int& grp, int& sl, bool& idle) {
  const int b = blockIdx.x;
  const int n = L.d[0].nGroups * L.d[0].nSlices;
  const int P = L.per_xcd;
  int d = 0, lw;
  if (!L.dual) {
    if (P > 0) lw = (b & 7) * P + (b >> 3);
    else lw = ((n & 7) == 0) ? (b & 7) * (n >> 3) + (b >> 3) : b;
  } else {
    d = (b & 7) >> 2;
    lw = (b & 3) * (P > 0 ? P : (n >> 2)) + (b >> 3);
  }
  idle = lw >= n;
  if (idle) lw = 0;
  RecArgsK& a = ((RecArgsK*)__builtin_amdgcn_kernarg_segment_ptr())[d];
  grp = lw / a.nSlices;
  sl = lw - grp * a.nSlices;
  return a;
}

// Exchange ring. A consumer wave reads the vector of the previous step as
// MFMA A operands: for k-step ks, lane (r16, q) needs row r16 and the q-th
// 16-byte chunk of the k-step. Read from y or dg rows directly, one load
// instruction touches 16 rows a full row pitch apart; in the ring every
// operand tile is stored as 64 consecutive 16-byte chunks in lane order, so
// that each load instruction reads 1 KiB contiguously. With at most 8 live
// rows a tile holds two k-steps: lanes 0..7 of every 16 carry k-step 2p and
// lanes 8..15 k-step 2p+1 of the same rows; the second operand is the same
// register rotated by 8 lanes within each row of 16 (DPP row_ror:8), and
// output rows 8..15, which the rotation fills with the other k-step, are
// never read. Producers store their own units into the tiles (two slots,
// alternating by step: a slot is rewritten two steps later, after every
// consumer has published the step that read it).
template <typename TS>
__device__ __forceinline__ int xoff(int row, int kg, bool packed, int mbt) {
  constexpr int KQ = Chunk<TS>::KQ, KSTEP = 4 * KQ;
  const int ks = kg / KSTEP, e = kg - ks * KSTEP, q = e / KQ, el = e - q * KQ;
  if (packed) return (ks >> 1) * 1024 + (row + 8 * (ks & 1) + 16 * q) * 16 + el * (int)sizeof(TS);
  // one 1 KiB tile per (k-step, 16-row tile of the group)
  return (ks * mbt + (row >> 4)) * 1024 + ((row & 15) + 16 * q) * 16 + el * (int)sizeof(TS);
}

__device__ __forceinline__ unsigned rot8(unsigned v) {
  // row_ror:8 (every source lane is inside the row, so no old value is kept)
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
}
__device__ __forceinline__ uint4 rot8(const uint4& v) { return make_uint4(rot8(v.x), rot8(v.y), rot8(v.z), rot8(v.w)); }

// acc[mb][nt] += (previous step's vector, k-steps [w*KI, w*KI+KI)) . Wr[nt][.]
// The W_hh tile is the MFMA's first operand and the vector its second, so the
// accumulator comes out transposed: lane l holds columns nt*16 + 4*(l/16) +
// e (e = 0..3) of batch row mb*16 + l%16, which spill_acc stores as one
// 16-byte piece.
// from the exchange ring tiles `xb` of this group (nbytes valid; loads past
// it return zero). Unpacked tiles are ordered (k-step, row tile).
// `mid` runs once the ring loads (the first batch of them) are issued and
// before any product waits for them: memory operations it issues queue
// behind the ring loads, so the products do not wait for them.
struct NoMid {
  __device__ void operator()() const {}
};
// `after` (packed tiles only) runs once the products are issued, with this
// wave's tiles: tile i holds k-step 2i in lanes 0-7 of each 16 and 2i+1 in
// lanes 8-15
struct NoAfter {
  template <typename V>
  __device__ void operator()(const V&) const {}
};
template <typename TS, int MB, int NT, int KI, typename Mid = NoMid, typename After = NoAfter>
__device__ __forceinline__ void contract_x(f4 (&acc)[MB][NT], const uint4 (&Wr)[NT][wslots<TS>(KI)], const char* xb, int nbytes,
                                           bool packed, Mid mid = Mid(), After after = After()) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)xb, (short)0, nbytes, BUF_RSRC_W3);
  if constexpr (MB == 1 && KI % 2 == 0) {
    if (packed) {
      constexpr int NL = KI / 2;
      uint4 v[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, ((w * KI) / 2 + i) * 1024 + lane * 16, 0, CPOL_SC1);
        v[i] = make_uint4(r[0], r[1], r[2], r[3]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!std::is_same<Mid, NoMid>::value) {
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const uint4 odd = rot8(v[i]);
        if constexpr (std::is_same<TS, float>::value) {
          const VPair<TS> vp = vpair<TS>(v[i], odd);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma_pair(acc[0][nt], &Wr[nt][3 * i], vp);
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[0][nt] = mfma_bf16(Wr[nt][2 * i], v[i], acc[0][nt]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[0][nt] = mfma_bf16(Wr[nt][2 * i + 1], odd, acc[0][nt]);
        }
      }
      after(v);
      return;
    }
  }
  // loads per batch: at most 16 tiles in flight for one row tile, 8 for more
  // (fp32: whole pairs of k-steps)
  constexpr int LIM = (MB == 1) ? 4 : 8;
  constexpr int KB0 = (LIM / MB) < 1 ? 1 : ((LIM / MB) < KI ? (LIM / MB) : KI);
  constexpr bool F32 = std::is_same<TS, float>::value;
  constexpr int KB = (F32 && KB0 % 2) ? KB0 + 1 : KB0;
  static_assert(KI % 2 == 0 && KB % (F32 ? 2 : 1) == 0, "fp32 k-steps are taken in pairs");
#pragma unroll
  for (int k0 = 0; k0 < KI; k0 += KB) {
    uint4 v[KB][MB];
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int ks = w * KI + k0 + i;
        const int off = (k0 + i < KI) ? ((ks * MB + mb) * 1024 + lane * 16) : nbytes;
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC1);
        v[i][mb] = make_uint4(r[0], r[1], r[2], r[3]);
      }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!std::is_same<Mid, NoMid>::value) {
      if (k0 == 0) {
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!F32) {
      // bf16: W slot = k-step
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        if (k0 + i >= KI) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = mfma_bf16(Wr[nt][k0 + i], v[i][mb], acc[mb][nt]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KB; i += 2) {
        if (k0 + i >= KI) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const VPair<TS> vp = vpair<TS>(v[i][mb], v[i + 1][mb]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma_pair(acc[mb][nt], &Wr[nt][3 * ((k0 + i) / 2)], vp);
        }
      }
    }
  }
}

// acc[mb][nt] += A[b0+mb*16.., k] . Wr[nt][k] over this wave's k-steps, with
// A(b, k) = src[b*ld + k + (k >= kshift ? kskip : 0)] (zero for rows b >= B,
// the end of the batch group, or when src is NULL). The wave owns k-steps
// [w*KI, w*KI+KI) of the contraction.
template <typename TS, int MB, int NT, int KI>
__device__ __forceinline__ void contract(f4 (&acc)[MB][NT], const uint4 (&Wr)[NT][wslots<TS>(KI)], const TS* src,
                                         long long ld, int b0, int B, int K, int kshift, int kskip) {
  constexpr int KQ = Chunk<TS>::KQ, KSTEP = 4 * KQ;
  // k-steps per load batch: every load of the step at once where registers allow
  constexpr int KB = (MB >= 4) ? 2 : (KI <= 16 ? KI : 16);
  static_assert(KI % 2 == 0 && KB % 2 == 0, "fp32 k-steps are taken in pairs");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  if (src == nullptr) return;
  // rows [0, B) of the source; loads past the end of the resource return 0,
  // so that every load is issued unconditionally and a batch is in flight
  // at once
  const int nbytes = (int)((long long)B * ld * sizeof(TS));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nbytes, BUF_RSRC_W3);
  int rowoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int b = b0 + mb * 16 + r16;
    rowoff[mb] = (b < B) ? (int)((long long)b * ld * sizeof(TS)) : nbytes;
  }
#pragma unroll
  for (int k0 = 0; k0 < KI; k0 += KB) {
    uint4 av[KB][MB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int k = (w * KI + k0 + kk) * KSTEP + q * KQ;
      const int kc = k + (k >= kshift ? kskip : 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int off = (k < K && k0 + kk < KI) ? rowoff[mb] + kc * (int)sizeof(TS) : nbytes;
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, CPOL_SC1);
        av[kk][mb] = make_uint4(r[0], r[1], r[2], r[3]);
      }
    }
    // keep the whole batch of loads ahead of its products
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!std::is_same<TS, float>::value) {
      // bf16: W slot = k-step
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        if (k0 + kk >= KI) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = mfma_bf16(Wr[nt][k0 + kk], av[kk][mb], acc[mb][nt]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KB; kk += 2) {
        if (k0 + kk >= KI) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const VPair<TS> vp = vpair<TS>(av[kk][mb], av[kk + 1][mb]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma_pair(acc[mb][nt], &Wr[nt][3 * ((k0 + kk) / 2)], vp);
        }
      }
    }
  }
}

template <int MB, int NT>
__device__ __forceinline__ void zero_acc(f4 (&acc)[MB][NT]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = f4{0.f, 0.f, 0.f, 0.f};
}

// Partial products of every wave to LDS: red[w][row][col], row < BG, col < NCOL
// (rows at or past the batch group's size, the padding of a group smaller
// than the MFMA tile, are written too and never read). A lane stores its 4
// consecutive columns of one row as one 16-byte write (4 writes of 4 bytes in
// the untransposed layout made the spill 4x the instructions: headline
// forward 2.10 -> 2.02 us per step). Rows are RSTRIDE(NCOL) floats apart:
// with a stride of 4 mod 8 floats, the rows of the 8 lanes that one write
// cycle serves fall on disjoint banks.
constexpr int rstride(int ncol) { return ncol + 4; }
template <int MB, int NT>
__device__ __forceinline__ void spill_acc(float* red, const f4 (&acc)[MB][NT], int rows) {
  constexpr int BG = MB * 16, S = rstride(NT * 16);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  (void)rows;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) *(f4*)&red[(w * BG + mb * 16 + r16) * S + nt * 16 + 4 * q] = acc[mb][nt];
}

// the same for four consecutive columns (col a multiple of 4), one 16-byte
// LDS read per wave
template <int NW, int BG, int NCOL>
__device__ __forceinline__ float4 red_sum4(const float* red, int row, int col) {
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float4 v = *(const float4*)&red[(w * BG + row) * rstride(NCOL) + col];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  return s;
}

template <int NW, int BG, int NCOL>
__device__ __forceinline__ float red_sum(const float* red, int row, int col) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[(w * BG + row) * rstride(NCOL) + col];
  return s;
}

// Load the B-operand tiles of W_hh rows (forward: output column col of the
// tile is W_hh row rowof(col); contraction over the H columns of W_hh).
// (fp32: split into bf16 pieces, a pair of k-steps at a time)
template <typename TS, int NT, int KI, typename RowOf>
__device__ __forceinline__ void load_w_rows(uint4 (&Wr)[NT][wslots<TS>(KI)], const TS* W, int H, RowOf rowof) {
  constexpr int KQ = Chunk<TS>::KQ, KSTEP = 4 * KQ;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const long long row = rowof(nt * 16 + r16);
    uint4 c[KI];
#pragma unroll
    for (int ks = 0; ks < KI; ++ks) {
      const int k = (w * KI + ks) * KSTEP + q * KQ;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k < H && row >= 0) v = *(const uint4*)(W + row * H + k);
      c[ks] = v;
    }
#pragma unroll
    for (int p = 0; p < KI / 2; ++p) wpair(c[2 * p], c[2 * p + 1], &Wr[nt][WPair<TS>::N * p], (TS*)nullptr);
  }
}

// Load the B-operand tiles of W_hh columns (backward: output column col is
// hidden unit J0+col, contraction index k runs over canonical gate rows
// kb + [0, K): W_hh[perm[g]*H + k%H][J0+col] with g = k/H).
template <typename TS, int NT, int KI, typename Perm>
__device__ __forceinline__ void load_w_cols(uint4 (&Wr)[NT][wslots<TS>(KI)], const TS* W, int H, const Perm& perm,
                                            int J0, int gate0, int K, bool unit_major = false) {
  constexpr int KQ = Chunk<TS>::KQ, KSTEP = 4 * KQ;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = J0 + nt * 16 + r16;
    uint4 c[KI];
#pragma unroll
    for (int ks = 0; ks < KI; ++ks) {
      const int k = (w * KI + ks) * KSTEP + q * KQ;
      TS e[KQ];
#pragma unroll
      for (int i = 0; i < KQ; ++i) e[i] = from_f<TS>(0.f);
      if (k < K) {
        if (unit_major) {
          // contraction row 4u + g: gate g of unit u (four gates)
#pragma unroll
          for (int i = 0; i < KQ; ++i) e[i] = W[((long long)perm[(k + i) & 3] * H + ((k + i) >> 2)) * H + col];
        } else {
          const int g = gate0 + k / H;
          const int kk = k % H;
#pragma unroll
          for (int i = 0; i < KQ; ++i) e[i] = W[((long long)perm[g] * H + kk + i) * H + col];
        }
      }
      c[ks] = *(const uint4*)e;
    }
#pragma unroll
    for (int p = 0; p < KI / 2; ++p) wpair(c[2 * p], c[2 * p + 1], &Wr[nt][WPair<TS>::N * p], (TS*)nullptr);
  }
}

// ------------------------------------------------------ forward kernels --
// LSTM (GL = 4 gate lanes) and reset-after GRU (GL = 3: r, u and the
// recurrent candidate term n_h = h W_hc^T + b_hc, kept apart).
// RING: the exchange ring carries the vector (h0 too: each workgroup writes
// its units of h0 into the slot step 0 reads before the placement
// rendezvous, which then orders them before every read); otherwise every
// step reads h0 / y rows directly. Two variants, so that the ring kernels
// carry no code of the row path (in the register-bound 64- and 128-row
// tiles that code alone made the compiler spill).
template <int CELL, typename TS, int NW, int MB, int NT, int KI, bool RING>
__global__ __launch_bounds__(NW * 64) void rec_fwd(RecLaunch L) {
  constexpr int NTH = NW * 64, BG = MB * 16, NCOL = NT * 16;
  constexpr int GL = (CELL == CELL_LSTM) ? 4 : 3;
  constexpr int HS = NCOL / GL;
  static_assert(HS * GL == NCOL, "columns must hold whole units");
  constexpr int UNITS = BG * HS;
  constexpr int UPT = (UNITS + NTH - 1) / NTH;
  extern __shared__ float red[];
  STEP_TIMER_DECL;

  int grp, sl;
  bool idle;
  RecArgsK& a = launch_slot(L, grp, sl, idle);
  if (idle) return;
  // groups of 64 or more rows always span several XCDs (one counter line
  // each); a constant stride keeps their register-bound code lean
  const int fstride = MB >= 4 ? FLAG_LINE : a.fstride;
  const int place_off = MB >= 4 ? 1 : a.place_off;
  int* myflag = a.flags + (grp * a.nSlices + sl) * fstride;
  const int* gflags = a.flags + grp * a.nSlices * fstride;
  const int tid = threadIdx.x;
  const int H = a.H, B = a.B, T = a.T;
  const int J0 = sl * HS, b0 = grp * a.bg;
  // this wave's contraction rows and the slices producing them
  int ws0, wsn;
  {
    constexpr int KSTEP = 4 * Chunk<TS>::KQ;
    const int w = tid >> 6, k0 = w * KI * KSTEP;
    wave_slices(k0, min(H, k0 + KI * KSTEP), H, HS, a.nSlices, ws0, wsn);
  }
  const int bend = min(B, b0 + a.bg);  // rows of this batch group: [b0, bend)
  const long long GZH = (long long)a.GZ * H;
  // exchange ring (single row-tile plans)
  constexpr bool tiled = RING;
  const bool packed = a.xpacked != 0;
  const int xbytes = H * (packed ? 8 : 16 * MB) * (int)sizeof(TS);
  auto xslot = [&](int step) { return a.xbuf + ((long long)(step & 1) * a.nGroups + grp) * a.xg_bytes; };

  // per-unit state; unit = (batch row bl, hidden unit j) of this workgroup
  float cst[UPT], hst[UPT], bhc[UPT];
  bool live[UPT];
  int bl_[UPT], j_[UPT], len_[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + u * NTH;
    bl_[u] = unit / HS;
    j_[u] = unit - bl_[u] * HS;
    live[u] = unit < UNITS && b0 + bl_[u] < bend;
    cst[u] = hst[u] = bhc[u] = 0.f;
    len_[u] = T;
    if (live[u] && a.lengths) len_[u] = min(max(a.lengths[b0 + bl_[u]], 0), T);
    const long long o = (long long)(b0 + bl_[u]) * H + J0 + j_[u];
    if (live[u]) {
      if (a.h0) hst[u] = to_f(((const TS*)a.h0)[o]);
      if (CELL == CELL_LSTM && a.c0) cst[u] = to_f(((const TS*)a.c0)[o]);
      if (CELL == CELL_GRU_RA) bhc[u] = to_f(((const TS*)a.b_hh)[(long long)a.perm[2] * H + J0 + j_[u]]);
    }
  }
  if constexpr (RING) {
    // h0 into the slot step 0 reads (device scope: the placement is not known
    // yet), acknowledged before the rendezvous publishes this workgroup
#pragma unroll
    for (int u = 0; u < UPT; ++u)
      if (live[u]) xstore((TS*)(xslot(-1) + xoff<TS>(bl_[u], J0 + j_[u], packed, MB)), hst[u], false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  const bool local = group_is_local(myflag, gflags, a.nSlices, fstride, place_off, a.status, a.timeout_ticks);

  uint4 Wr[NT][wslots<TS>(KI)];
  // LSTM columns are unit-major (column 4u+g: gate g of unit u), so that a
  // unit's four gate sums sit in one 16-byte LDS word per wave; the GRU's
  // three lanes are gate-major (column g*HS+u)
  load_w_rows<TS, NT, KI>(Wr, (const TS*)a.W_hh, H, [&](int col) -> long long {
    if constexpr (CELL == CELL_LSTM) return (long long)a.perm[col & 3] * H + J0 + (col >> 2);
    const int g = col / HS;
    return (long long)a.perm[g] * H + J0 + (col - g * HS);
  });


  // Pipelined ring kernels (one row tile): the operands of step s+1 are
  // loaded, and the stores of step s-1 issued, while step s's exchange loads
  // are in flight. Loads and stores share one in-order completion counter:
  // issued just before the wait for the step counters they would hold up
  // every poll until they complete, and stores still pending at the top of
  // a step make the compiler wait for them there.
  constexpr bool PIPE = RING && MB < 4;
  auto prefetch = [&](int ps, TS (&qz)[UPT][GL], TS (&qa)[UPT]) {
    const int pt = a.dir ? T - 1 - ps : ps;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      // unconditional loads from a valid address: a branch per load would
      // make the compiler wait for each one on the spot
      const TS* zr = (const TS*)a.z + (live[u] ? ((long long)pt * B + b0 + bl_[u]) * GZH + J0 + j_[u] : 0);
#pragma unroll
      for (int g = 0; g < GL; ++g) qz[u][g] = zr[g * H];
      // AUGRU attention score of this step and row
      if constexpr (CELL == CELL_GRU_RA) {
        const TS* ap = a.att ? (const TS*)a.att + (live[u] ? (long long)pt * B + b0 + bl_[u] : 0) : zr;
        qa[u] = *ap;
      }
    }
  };
  // what only later kernels read: y (when the ring carries the exchange),
  // the saved gates and the cell states of processing step ps; with `on`
  // false (no step to store) every store is dropped. Branch-free: the
  // products that wait for the exchange loads issued before these stores
  // then wait for exactly those loads.
  auto post_stores = [&](int ps, bool on, const float (&qsv)[UPT][4], const float (&qhv)[UPT],
                         const float (&qcv)[UPT]) {
    const int pt = a.dir ? T - 1 - ps : ps;
    constexpr int SZ = (int)sizeof(TS);
    const auto rz = rsrc((const TS*)a.z + (long long)pt * B * GZH, (long long)B * GZH * SZ);
    const auto ry = rsrc((const TS*)a.y + (long long)pt * B * a.ldy, (long long)B * a.ldy * SZ);
    const bool cb = CELL == CELL_LSTM && a.cbuf != nullptr;
    const auto rc = rsrc(cb ? (const TS*)a.cbuf + (long long)pt * B * a.ldc : (const TS*)a.z, cb ? (long long)B * a.ldc * SZ : 0);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const bool ok = on && live[u];
      const int b = b0 + bl_[u], jj = J0 + j_[u];
      const int oz = ok ? (b * (int)GZH + jj) * SZ : BUF_SKIP;
#pragma unroll
      for (int g = 0; g < 4; ++g) bstore<TS>(rz, oz + g * H * SZ, qsv[u][g]);
      bstore<TS>(ry, ok ? (b * (int)a.ldy + jj) * SZ : BUF_SKIP, qhv[u]);
      if constexpr (CELL == CELL_LSTM) bstore<TS>(rc, ok ? (b * (int)a.ldc + jj) * SZ : BUF_SKIP, qcv[u]);
    }
  };
  TS pz[UPT][GL], pa[UPT];                  // operands of the current step
  float dsv[UPT][4], dhv[UPT], dcv[UPT];    // the previous step's deferred stores (PIPE)
  if constexpr (PIPE) prefetch(0, pz, pa);

  STEP_TIMER_CAL(0);
  for (int s = 0; s < T; ++s) {
    STEP_TIMER(s, 0);
    const int t = a.dir ? T - 1 - s : s;
    const int tp = a.dir ? t + 1 : t - 1;
    // without the pipeline, the projected inputs of this step are loaded
    // before the wait and land while it polls
    if constexpr (!PIPE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const TS* zr = (const TS*)a.z + (live[u] ? ((long long)t * B + b0 + bl_[u]) * GZH + J0 + j_[u] : 0);
#pragma unroll
        for (int g = 0; g < GL; ++g) pz[u][g] = zr[g * H];
        if constexpr (CELL == CELL_GRU_RA) {
          const TS* ap = a.att ? (const TS*)a.att + (live[u] ? (long long)t * B + b0 + bl_[u] : 0) : zr;
          pa[u] = *ap;
        }
      }
    }
    TS pzn[UPT][GL], pan[UPT];  // the next step's operands (PIPE)
    if (s > 0) wait_flags(gflags + ws0 * fstride, wsn, s, a.status, a.timeout_ticks, fstride, MB < 4 && local);
    STEP_TIMER(s, 1);
    f4 acc[MB][NT];
    zero_acc(acc);
    if constexpr (RING) {
      if constexpr (PIPE) {
        auto mid = [&]() {
          prefetch(s + 1 < T ? s + 1 : s, pzn, pan);
          post_stores(s > 0 ? s - 1 : 0, s > 0, dsv, dhv, dcv);
        };
        contract_x<TS, MB, NT, KI>(acc, Wr, xslot(s - 1), xbytes, packed, mid);
      } else {
        contract_x<TS, MB, NT, KI>(acc, Wr, xslot(s - 1), xbytes, packed);
      }
    } else {
      const TS* src = (s == 0) ? (const TS*)a.h0 : (const TS*)a.y + (long long)tp * B * a.ldy;
      const long long ld = (s == 0) ? H : a.ldy;
      contract<TS, MB, NT, KI>(acc, Wr, src, ld, b0, bend, H, 1 << 30, 0);
    }
    STEP_TIMER(s, 2);
    spill_acc(red, acc, bend - b0);
    STEP_TIMER(s, 3);
    __syncthreads();
    STEP_TIMER(s, 4);
    // the exchanged vector is stored first; what only later kernels read
    // (y when the ring carries the exchange, saved gates, cell states) is
    // kept in registers and stored after the step counter is published
    // (pipelined: during the next step's exchange loads)
    // A step past a row's length (variable lengths) keeps the state, saves
    // zero gates and outputs zero; the exchange still carries the kept state
    // (without the ring, y carries it and is zeroed by a later pass).
    float sv[UPT][4], hv[UPT], cv[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if constexpr (PIPE) sv[u][0] = sv[u][1] = sv[u][2] = sv[u][3] = hv[u] = cv[u] = 0.f;
      if (!live[u]) continue;
      const int bl = bl_[u], j = j_[u], b = b0 + bl;
      const bool act = t < len_[u];
      TS* yr = (TS*)a.y + ((long long)t * B + b) * a.ldy + J0 + j;
      float h;
      if constexpr (CELL == CELL_LSTM) {
        const float4 zs = red_sum4<NW, BG, NCOL>(red, bl, 4 * j);
        const float zi = zs.x + to_f(pz[u][0]);
        const float zf = zs.y + to_f(pz[u][1]);
        const float zg = zs.z + to_f(pz[u][2]);
        const float zo = zs.w + to_f(pz[u][3]);
        const float ig = sigmoidf_(zi), fg = sigmoidf_(zf), gg = tanhf_(zg), og = sigmoidf_(zo);
        const float c = fg * cst[u] + ig * gg;
        const float hn = og * tanhf_(c);
        cst[u] = act ? c : cst[u];
        hst[u] = act ? hn : hst[u];
        h = hst[u];
        sv[u][0] = act ? ig : 0.f;
        sv[u][1] = act ? fg : 0.f;
        sv[u][2] = act ? gg : 0.f;
        sv[u][3] = act ? og : 0.f;
        cv[u] = act ? c : 0.f;
      } else {
        const float r = sigmoidf_(red_sum<NW, BG, NCOL>(red, bl, 0 * HS + j) + to_f(pz[u][0]));
        const float uu = sigmoidf_(red_sum<NW, BG, NCOL>(red, bl, 1 * HS + j) + to_f(pz[u][1]));
        const float nh = red_sum<NW, BG, NCOL>(red, bl, 2 * HS + j) + bhc[u];
        const float c = tanhf_(to_f(pz[u][2]) + r * nh);
        const float us = a.att ? (1.f - to_f(pa[u])) * uu : uu;  // AUGRU: scaled update gate
        const float hn = us * hst[u] + (1.f - us) * c;
        hst[u] = act ? hn : hst[u];
        h = hst[u];
        sv[u][0] = act ? r : 0.f;
        sv[u][1] = act ? uu : 0.f;
        sv[u][2] = act ? c : 0.f;
        sv[u][3] = act ? nh : 0.f;
        cv[u] = 0.f;
      }
      hv[u] = act ? h : 0.f;  // the output
      if (tiled) xstore((TS*)(xslot(s) + xoff<TS>(bl, J0 + j, packed, MB)), h, local);
      else xstore(yr, h, local);
    }
    STEP_TIMER(s, 5);
    publish(myflag, s + 1, local);
    STEP_TIMER(s, 6);
    if constexpr (PIPE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
#pragma unroll
        for (int g = 0; g < 4; ++g) dsv[u][g] = sv[u][g];
        dhv[u] = hv[u];
        dcv[u] = cv[u];
#pragma unroll
        for (int g = 0; g < GL; ++g) pz[u][g] = pzn[u][g];
        pa[u] = pan[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        if (!live[u]) continue;
        const int bl = bl_[u], j = j_[u], b = b0 + bl;
        TS* zr = (TS*)a.z + ((long long)t * B + b) * GZH + J0 + j;
        if (tiled) ((TS*)a.y)[((long long)t * B + b) * a.ldy + J0 + j] = from_f<TS>(hv[u]);
#pragma unroll
        for (int g = 0; g < 4; ++g) zr[g * H] = from_f<TS>(sv[u][g]);
        if constexpr (CELL == CELL_LSTM) {
          if (a.cbuf) ((TS*)a.cbuf)[((long long)t * B + b) * a.ldc + J0 + j] = from_f<TS>(cv[u]);
          if (s == T - 1 && a.cT) ((TS*)a.cT)[(long long)b * H + J0 + j] = from_f<TS>(cst[u]);
        }
        if (s == T - 1 && a.hT) ((TS*)a.hT)[(long long)b * H + J0 + j] = from_f<TS>(hst[u]);
      }
    }
    STEP_TIMER(s, 7);
  }
  if constexpr (PIPE) {
    post_stores(T - 1, true, dsv, dhv, dcv);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      const long long o = (long long)(b0 + bl_[u]) * H + J0 + j_[u];
      if (CELL == CELL_LSTM && a.cT) ((TS*)a.cT)[o] = from_f<TS>(cst[u]);
      if (a.hT) ((TS*)a.hT)[o] = from_f<TS>(hst[u]);
    }
  }
  STEP_TIMER_CAL(1);
  STEP_TIMER_FLUSH(T);
}

// Basic GRU: the candidate contracts r*h_{t-1} over all hidden units, so a
// step has two exchanges (h_{t-1}, then r*h_{t-1}); phase counters advance by
// two per step. Workgroup columns: phase A r,u (2*HS), phase B candidate (HS).
template <typename TS, int NW, int MB, int NTB, int KI>
__global__ __launch_bounds__(NW * 64) void rec_fwd_grub(RecLaunch L) {
  constexpr int NTH = NW * 64, BG = MB * 16, HS = NTB * 16;
  constexpr int NTA = 2 * NTB;
  constexpr int UNITS = BG * HS;
  constexpr int UPT = (UNITS + NTH - 1) / NTH;
  extern __shared__ float red[];
  STEP_TIMER_DECL;

  int grp, sl;
  bool idle;
  RecArgsK& a = launch_slot(L, grp, sl, idle);
  if (idle) return;
  int* myflag = a.flags + (grp * a.nSlices + sl) * a.fstride;
  const int* gflags = a.flags + grp * a.nSlices * a.fstride;
  const bool local =
      group_is_local(myflag, gflags, a.nSlices, a.fstride, a.place_off, a.status, a.timeout_ticks);
  const int tid = threadIdx.x;
  const int H = a.H, B = a.B, T = a.T;
  const int J0 = sl * HS, b0 = grp * a.bg;
  const int bend = min(B, b0 + a.bg);  // rows of this batch group: [b0, bend)
  const long long GZH = (long long)a.GZ * H;

  uint4 WA[NTA][wslots<TS>(KI)], WB[NTB][wslots<TS>(KI)];
  load_w_rows<TS, NTA, KI>(WA, (const TS*)a.W_hh, H, [&](int col) -> long long {
    const int g = col / HS;
    return (long long)a.perm[g] * H + J0 + (col - g * HS);
  });
  load_w_rows<TS, NTB, KI>(WB, (const TS*)a.W_hh, H,
                           [&](int col) -> long long { return (long long)a.perm[2] * H + J0 + col; });

  float hst[UPT], ust[UPT];
  bool live[UPT];
  int bl_[UPT], j_[UPT], len_[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + u * NTH;
    bl_[u] = unit / HS;
    j_[u] = unit - bl_[u] * HS;
    live[u] = unit < UNITS && b0 + bl_[u] < bend;
    hst[u] = ust[u] = 0.f;
    len_[u] = T;
    if (live[u] && a.lengths) len_[u] = min(max(a.lengths[b0 + bl_[u]], 0), T);
    if (live[u] && a.h0) hst[u] = to_f(((const TS*)a.h0)[(long long)(b0 + bl_[u]) * H + J0 + j_[u]]);
  }
  // both products contract over H: this wave's rows and the slices producing
  // them (each wave waits for its own producers only; every step has its own
  // rows of y and r*h, so nothing is rewritten while a slow wave reads it)
  int ws0, wsn;
  {
    constexpr int KSTEP = 4 * Chunk<TS>::KQ;
    const int k0 = (tid >> 6) * KI * KSTEP, k1 = min(H, k0 + KI * KSTEP);
    wave_slices(k0, k1, H, HS, a.nSlices, ws0, wsn);
  }
  float sr[UPT], su[UPT], sc[UPT];  // gates stored after the step's counter

  STEP_TIMER_CAL(0);
  for (int s = 0; s < T; ++s) {
    STEP_TIMER(s, 0);
    const int t = a.dir ? T - 1 - s : s;
    const int tp = a.dir ? t + 1 : t - 1;
    TS pz[UPT][3], pa[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const TS* zr = (const TS*)a.z + (live[u] ? ((long long)t * B + b0 + bl_[u]) * GZH + J0 + j_[u] : 0);
#pragma unroll
      for (int g = 0; g < 3; ++g) pz[u][g] = zr[g * H];
      const TS* ap = a.att ? (const TS*)a.att + (live[u] ? (long long)t * B + b0 + bl_[u] : 0) : zr;
      pa[u] = *ap;  // AUGRU attention score of this step and row
    }
    // phase A: r, u
    if (s > 0) wait_flags(gflags + ws0 * a.fstride, wsn, 2 * s, a.status, a.timeout_ticks, a.fstride, local);
    STEP_TIMER(s, 1);
    {
      f4 acc[MB][NTA];
      zero_acc(acc);
      const TS* src = (s == 0) ? (const TS*)a.h0 : (const TS*)a.y + (long long)tp * B * a.ldy;
      const long long ld = (s == 0) ? H : a.ldy;
      contract<TS, MB, NTA, KI>(acc, WA, src, ld, b0, bend, H, 1 << 30, 0);
      spill_acc(red, acc, bend - b0);
    }
    STEP_TIMER(s, 2);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      const int bl = bl_[u], j = j_[u], b = b0 + bl;
      TS* zr = (TS*)a.z + ((long long)t * B + b) * GZH + J0 + j;
      const float r = sigmoidf_(red_sum<NW, BG, 2 * HS>(red, bl, j) + to_f(pz[u][0]));
      const float uu = sigmoidf_(red_sum<NW, BG, 2 * HS>(red, bl, HS + j) + to_f(pz[u][1]));
      const bool act = t < len_[u];
      ust[u] = a.att ? (1.f - to_f(pa[u])) * uu : uu;  // AUGRU: scaled update gate
      xstore((TS*)a.rh + ((long long)t * B + b) * H + J0 + j, r * hst[u], local);
      sr[u] = act ? r : 0.f;
      su[u] = act ? uu : 0.f;
    }
    STEP_TIMER(s, 3);
    publish(myflag, 2 * s + 1, local);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      TS* zr = (TS*)a.z + ((long long)t * B + b0 + bl_[u]) * GZH + J0 + j_[u];
      zr[0] = from_f<TS>(sr[u]);
      zr[H] = from_f<TS>(su[u]);
    }
    // phase B: candidate and new state
    STEP_TIMER(s, 4);
    wait_flags(gflags + ws0 * a.fstride, wsn, 2 * s + 1, a.status, a.timeout_ticks, a.fstride, local);
    STEP_TIMER(s, 5);
    {
      f4 acc[MB][NTB];
      zero_acc(acc);
      contract<TS, MB, NTB, KI>(acc, WB, (const TS*)a.rh + (long long)t * B * H, H, b0, bend, H, 1 << 30, 0);
      spill_acc(red, acc, bend - b0);
    }
    __syncthreads();
    STEP_TIMER(s, 6);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      const int bl = bl_[u], j = j_[u], b = b0 + bl;
      const float c = tanhf_(red_sum<NW, BG, HS>(red, bl, j) + to_f(pz[u][2]));
      const bool act = t < len_[u];
      // past a row's length the state is kept (and carried through y, which a
      // later pass zeroes on those steps)
      const float h = act ? ust[u] * hst[u] + (1.f - ust[u]) * c : hst[u];
      hst[u] = h;
      xstore((TS*)a.y + ((long long)t * B + b) * a.ldy + J0 + j, h, local);
      sc[u] = act ? c : 0.f;
    }
    STEP_TIMER(s, 7);
    publish(myflag, 2 * s + 2, local);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      const int b = b0 + bl_[u], j = j_[u];
      ((TS*)a.z + ((long long)t * B + b) * GZH + J0 + j)[2 * H] = from_f<TS>(sc[u]);
      if (s == T - 1 && a.hT) ((TS*)a.hT)[(long long)b * H + J0 + j] = from_f<TS>(hst[u]);
    }
  }
  STEP_TIMER_CAL(1);
  STEP_TIMER_FLUSH(T);
}

// AUGRU score gradient: sum the per-unit shares of each batch row (in LDS,
// written before the last barrier) over this workgroup's units, in a fixed
// order, into the partial of its hidden slice: part[(t*B + b)*nSlices + sl].
template <int HS>
__device__ __forceinline__ void att_rows(const float* attl, float* part, int t, int B, int b0, int bend, int nSlices,
                                         int sl) {
  for (int r = threadIdx.x; r < bend - b0; r += blockDim.x) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < HS; ++j) sum += attl[r * HS + j];
    part[((long long)t * B + b0 + r) * nSlices + sl] = sum;
  }
}

// ----------------------------------------------------- backward kernels --
// LSTM and reset-after GRU: the carried hidden gradient of step t is
// dG'_{t+1} W_hh (dG' = [di,df,dg,do], or [d_r, d_u, d_c*r] for the GRU),
// contracted over all gate rows; the workgroup holds the W_hh columns of its
// HS units. Steps are processed in the reverse of the forward order.
// RING as for the forward kernels: the ring variant carries no code of the
// row-read path.
// FDW (fp32, packed ring of one row tile): the kernel also accumulates the
// recurrent-weight gradient dW_hh[k][J] += sum_b dG'_{t+1}[b][k] h_t[b][J]
// for its own units J over all contraction rows k, one 16x16x4 fp32 MFMA per
// 16 rows of k, 16 units and 4 batch rows. dG' is the ring tile the wave has
// just contracted, kept in LDS transposed to batch-major lanes (one 16-byte
// write per lane); h_t is the previous state each unit's epilogue used,
// kept in LDS per step parity. The products for the tiles of one step run
// two steps later, while the first poll of that step's wait is in flight;
// the last step's right after its contraction. The
// recurrent bias gradient (the same dG' summed over rows and steps) is
// summed per unit in registers. Both go to a.dwp as per-group partials at
// the end: [nGroups][K][H] then [nGroups][K].
template <int CELL, typename TS, int NW, int MB, int NT, int KI, bool RING, bool FDW = false>
__global__ __launch_bounds__(NW * 64) void rec_bwd(RecLaunch L) {
  constexpr int NTH = NW * 64, BG = MB * 16, HS = NT * 16;
  constexpr int GK = (CELL == CELL_LSTM) ? 4 : 3;
  constexpr int UNITS = BG * HS;
  constexpr int UPT = (UNITS + NTH - 1) / NTH;
  static_assert(!FDW || (RING && MB == 1 && sizeof(TS) == 4 && KI % 2 == 0 && NW >= GK),
                "fused dW: fp32 packed ring (and LDS for the bias partials)");
  extern __shared__ float red[];
  // fused dW: h_{t-1} of the units per step parity, and per wave its ring
  // tiles of the last contraction as [16 rows: batch row + 8 * k-step parity][16 k]
  __shared__ float hbuf[FDW ? 2 * BG * HS : 1];
  __shared__ float xtr[FDW ? NW * (KI / 2) * 256 : 1];
  STEP_TIMER_DECL;
  float* attl = red + NW * BG * rstride(HS);  // AUGRU score-gradient shares (LDS sized for them when used)

  int grp, sl;
  bool idle;
  RecArgsK& a = launch_slot(L, grp, sl, idle);
  if (idle) return;
  // groups of 64 or more rows always span several XCDs (one counter line
  // each); a constant stride keeps their register-bound code lean
  const int fstride = MB >= 4 ? FLAG_LINE : a.fstride;
  const int place_off = MB >= 4 ? 1 : a.place_off;
  int* myflag = a.flags + (grp * a.nSlices + sl) * fstride;
  const int* gflags = a.flags + grp * a.nSlices * fstride;
  const bool local = group_is_local(myflag, gflags, a.nSlices, fstride, place_off, a.status, a.timeout_ticks);
  const int tid = threadIdx.x;
  const int H = a.H, B = a.B, T = a.T;
  const int J0 = sl * HS, b0 = grp * a.bg;
  const int bend = min(B, b0 + a.bg);  // rows of this batch group: [b0, bend)
  const long long GZH = (long long)a.GZ * H, GDH = (long long)a.GD * H;
  const int K = GK * H;
  // bf16 LSTM through the exchange ring: contraction rows unit-major (row
  // 4u + g: gate g of unit u), so that a wave's rows come from few slices
  // and a producer stores a unit's four gradients as one 8-byte piece (not
  // for the register-bound 64-row tiles, whose spill code it upsets)
  const bool umaj = CELL == CELL_LSTM && sizeof(TS) == 2 && MB < 4 && RING;
  // this wave's contraction rows and the slices producing them
  int ws0, wsn;
  {
    constexpr int KSTEP = 4 * Chunk<TS>::KQ;
    const int k0 = (tid >> 6) * KI * KSTEP, k1 = min(K, k0 + KI * KSTEP);
    if (umaj && k1 > k0) {
      ws0 = (k0 >> 2) / HS;
      wsn = ((k1 - 1) >> 2) / HS + 1 - ws0;
    } else {
      wave_slices(k0, k1, H, HS, a.nSlices, ws0, wsn);
    }
  }
  // GRU: lanes r, u, then the recurrent candidate lane d_c*r stored in lane 3
  const int kshift = (CELL == CELL_LSTM) ? (1 << 30) : 2 * H;
  const int kskip = (CELL == CELL_LSTM) ? 0 : H;
  // exchange ring (single row-tile plans): the contracted lanes only
  constexpr bool tiled = RING;
  const bool packed = a.xpacked != 0;
  const int xbytes = K * (packed ? 8 : 16 * MB) * (int)sizeof(TS);
  auto xslot = [&](int step) { return a.xbuf + ((long long)(step & 1) * a.nGroups + grp) * a.xg_bytes; };

  uint4 Wr[NT][wslots<TS>(KI)];
  // with W_hh transposed into the contraction order, the operands are rows
  // (one 16-byte load each, as in the forward); reading W_hh columns takes
  // one load per element from eight W rows
  const bool wrows = a.W_hhT != nullptr;
  if (wrows) load_w_rows<TS, NT, KI>(Wr, (const TS*)a.W_hhT, K, [&](int col) -> long long { return J0 + col; });
  else load_w_cols<TS, NT, KI>(Wr, (const TS*)a.W_hh, H, a.perm, J0, 0, K, umaj);

  float dcar[UPT], hcar[UPT];
  bool live[UPT];
  int bl_[UPT], j_[UPT], len_[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + u * NTH;
    bl_[u] = unit / HS;
    j_[u] = unit - bl_[u] * HS;
    live[u] = unit < UNITS && b0 + bl_[u] < bend;
    dcar[u] = hcar[u] = 0.f;
    len_[u] = T;
    if (live[u] && a.lengths) len_[u] = min(max(a.lengths[b0 + bl_[u]], 0), T);
    const long long o = (long long)(b0 + bl_[u]) * H + J0 + j_[u];
    if (live[u]) {
      if (CELL == CELL_LSTM && a.dcT) dcar[u] = to_f(((const TS*)a.dcT)[o]);
      if (a.dhT) hcar[u] = to_f(((const TS*)a.dhT)[o]);  // seeds the carried hidden gradient
    }
  }

  // Pipelined ring kernels (one row tile), as in the forward: the own-unit
  // operands of step n+1 are loaded, and step n-1's gate gradients (and
  // AUGRU score partials) stored, while step n's exchange loads are in
  // flight, so that neither holds up the poll of the step counters. The
  // cell-state lane rebuilt into dG (recomputation) is read two steps before
  // the deferred store that overwrites it.
  constexpr bool PIPE = RING && MB < 4;
  constexpr bool HH = FDW && CELL == CELL_LSTM;  // the LSTM's h_{t-1} for the fused dW
  auto prefetch = [&](int pn, TS (&qdy)[UPT], TS (&qz)[UPT][4], TS (&qc)[UPT], TS (&qprev)[UPT], TS (&qa)[UPT],
                      bool (&qvalid)[UPT], TS (&qhh)[UPT], bool (&qhv)[UPT]) {
    const int ps = T - 1 - pn;
    const int pt = a.dir ? T - 1 - ps : ps;
    const int ptp = a.dir ? pt + 1 : pt - 1;
    // own-unit operands of the step (independent of the exchange): dy,
    // saved gates, cell states / previous output (unconditional loads from
    // valid addresses; `on` selects at use)
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const bool on = live[u] && pn < T;
      const long long row = on ? (long long)pt * B + b0 + bl_[u] : 0;
      const long long o = on ? (long long)(b0 + bl_[u]) * H + J0 + j_[u] : 0;
      const int jj = on ? J0 + j_[u] : 0;
      const TS* zr = (const TS*)a.z + row * GZH + jj;
      qdy[u] = ((const TS*)a.dy)[row * a.ldy + jj];
      if constexpr (CELL == CELL_GRU_RA) {
        const TS* ap = a.att ? (const TS*)a.att + row : (const TS*)a.dy;
        qa[u] = *ap;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) qz[u][g] = zr[g * H];
      // the row's first processed step takes its previous state from h0/c0
      // (direction 1 with variable lengths: the row's own last step)
      const bool first = a.dir ? (pt == len_[u] - 1) : (pt == 0);
      const bool inseq = ptp >= 0 && ptp < T;
      if constexpr (CELL == CELL_LSTM) {
        qc[u] = ((const TS*)a.cbuf)[row * a.ldc + jj];
        qvalid[u] = on && (!first || a.c0);
        const TS* cprev = (first && a.c0) ? (const TS*)a.c0 + o
                        : (const TS*)a.cbuf + (first || !on || !inseq ? 0 : ((long long)ptp * B + b0 + bl_[u]) * a.ldc + jj);
        qprev[u] = *cprev;
        if constexpr (HH) {
          qhv[u] = on && (!first || a.h0);
          const TS* hprev = (first && a.h0) ? (const TS*)a.h0 + o
                          : (const TS*)a.y + (first || !on || !inseq ? 0 : ((long long)ptp * B + b0 + bl_[u]) * a.ldy + jj);
          qhh[u] = *hprev;
        }
      } else {
        qc[u] = from_f<TS>(0.f);
        qvalid[u] = on && (!first || a.h0);
        const TS* hprev = (first && a.h0) ? (const TS*)a.h0 + o
                        : (const TS*)a.y + (first || !on || !inseq ? 0 : ((long long)ptp * B + b0 + bl_[u]) * a.ldy + jj);
        qprev[u] = *hprev;
      }
    }
  };
  // gate gradients of processing step pn for the later kernels (the ring
  // carried the exchange); branch-free as in the forward (`on` false: every
  // store dropped)
  auto post_stores = [&](int pn, bool on, const float (&qdv)[UPT][4]) {
    const int ps = T - 1 - pn;
    const int pt = a.dir ? T - 1 - ps : ps;
    constexpr int SZ = (int)sizeof(TS);
    const auto rg = rsrc((const TS*)a.dg + (long long)pt * B * GDH, (long long)B * GDH * SZ);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int og = (on && live[u]) ? ((b0 + bl_[u]) * (int)GDH + J0 + j_[u]) * SZ : BUF_SKIP;
#pragma unroll
      for (int g = 0; g < 4; ++g) bstore<TS>(rg, og + g * H * SZ, qdv[u][g]);
    }
  };
  TS pdy[UPT], pz[UPT][4], pc[UPT], pprev[UPT], pa[UPT], phh[UPT];  // operands of the current step
  bool pvalid[UPT], phv[UPT];
  float ddv[UPT][4];  // the previous step's deferred gate gradients (PIPE)
  if constexpr (PIPE) prefetch(0, pdy, pz, pc, pprev, pa, pvalid, phh, phv);
  // fused dW: this wave's accumulators (k-step kl of its range, unit tile nt)
  f4 dw[FDW ? KI : 1][FDW ? NT : 1];
  float* xw = xtr + (FDW ? (tid >> 6) * (KI / 2) * 256 : 0);
  float dbacc[UPT][FDW ? 4 : 1];  // fused db_hh: this thread's units, summed over steps
#pragma unroll
  for (int u = 0; u < UPT; ++u)
#pragma unroll
    for (int g = 0; g < (FDW ? 4 : 1); ++g) dbacc[u][g] = 0.f;
  if constexpr (FDW) {
#pragma unroll
    for (int i = 0; i < KI; ++i)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) dw[i][nt] = f4{0.f, 0.f, 0.f, 0.f};
    // rows past the group stay zero (the first step's barrier orders this
    // before any epilogue writes)
    for (int i = tid; i < 2 * BG * HS; i += NTH) hbuf[i] = 0.f;
  }
  // keep this wave's ring tiles: ring lane L holds row L%8 of k-step parity
  // (L/8)%2, k = 4(L/16)..+3 of the 16 in the k-step
  auto keep_tiles = [&](const auto& v) {
    if constexpr (FDW) {
      const int lane = tid & 63;
#pragma unroll
      for (int i = 0; i < KI / 2; ++i) *(uint4*)(xw + i * 256 + (lane & 15) * 16 + 4 * (lane >> 4)) = v[i];
    }
  };
  // dW_hh[k][J] += sum_b dG'[b][k] h[b][J] over the kept tiles, with h from hb:
  // A[m = k][kk = b] and B[kk = b][n = unit], 4 batch rows per product (one
  // set of products for groups of 4 rows, two for 8). Straight-line code:
  // every LDS read is issued before the first product waits.
  auto dw_rows = [&](const float* hb, auto nhq) {
    constexpr int NHQ = decltype(nhq)::value;
    const int lane = tid & 63, rowsg = bend - b0;
    float hv[NHQ][NT], av[KI][NHQ];
#pragma unroll
    for (int hq = 0; hq < NHQ; ++hq)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) hv[hq][nt] = hb[((lane >> 4) + 4 * hq) * HS + nt * 16 + (lane & 15)];
#pragma unroll
    for (int i = 0; i < KI / 2; ++i)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int hq = 0; hq < NHQ; ++hq) {
          const int bb = (lane >> 4) + 4 * hq;
          const float x = xw[i * 256 + (bb + 8 * half) * 16 + (lane & 15)];
          av[2 * i + half][hq] = bb < rowsg ? x : 0.f;  // ring rows past the group hold stale data
        }
#pragma unroll
    for (int hq = 0; hq < NHQ; ++hq)
#pragma unroll
      for (int kl = 0; kl < KI; ++kl)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dw[kl][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[kl][hq], hv[hq][nt], dw[kl][nt], 0, 0, 0);
  };
  auto dw_accumulate = [&](const float* hb) {
    if constexpr (FDW) {
      if (a.bg > 4) dw_rows(hb, std::integral_constant<int, 2>());
      else dw_rows(hb, std::integral_constant<int, 1>());
    }
  };

  STEP_TIMER_CAL(0);
  for (int n = 0; n <= T; ++n) {
    STEP_TIMER(n, 0);
    const int s = T - 1 - n;  // processing index of this step (-1: the final dh0 contraction)
    const int t = a.dir ? T - 1 - s : s;
    if constexpr (!PIPE) prefetch(n, pdy, pz, pc, pprev, pa, pvalid, phh, phv);
    TS ndy[UPT], nz[UPT][4], nc[UPT], nprev[UPT], na[UPT], nhh[UPT];  // the next step's operands (PIPE)
    bool nvalid[UPT], nhv[UPT];
    auto mid = [&]() {
      if constexpr (PIPE) {
        prefetch(n + 1 < T ? n + 1 : T - 1, ndy, nz, nc, nprev, na, nvalid, nhh, nhv);
        post_stores(n > 0 ? n - 1 : 0, n > 0, ddv);
      }
    };
    f4 acc[MB][NT];
    zero_acc(acc);
    if (n > 0) {
      // fused dW: the tiles the last contraction kept (dG' of step n-2) with
      // the state that step followed, while the first poll is in flight
      auto idle = [&]() {
        if constexpr (FDW) {
          if (n >= 2) dw_accumulate(hbuf + (n & 1) * BG * HS);
        }
      };
      if constexpr (FDW)
        wait_flags(gflags + ws0 * fstride, wsn, n, a.status, a.timeout_ticks, fstride,
                   CELL == CELL_LSTM && MB < 4 && local, idle);
      else
        wait_flags(gflags + ws0 * fstride, wsn, n, a.status, a.timeout_ticks, fstride,
                   CELL == CELL_LSTM && MB < 4 && local);
      STEP_TIMER(n, 1);
      if constexpr (FDW) contract_x<TS, MB, NT, KI>(acc, Wr, xslot(n - 1), xbytes, packed, mid, keep_tiles);
      else if constexpr (PIPE) contract_x<TS, MB, NT, KI>(acc, Wr, xslot(n - 1), xbytes, packed, mid);
      else if constexpr (RING) contract_x<TS, MB, NT, KI>(acc, Wr, xslot(n - 1), xbytes, packed);
      if constexpr (!RING) {
        const int tn = a.dir ? T - 1 - (s + 1) : (s + 1);  // step whose dG feeds this one
        contract<TS, MB, NT, KI>(acc, Wr, (const TS*)a.dg + (long long)tn * B * GDH, GDH, b0, bend, K, kshift,
                                 kskip);
      }
    } else if constexpr (PIPE) {
      mid();
    }
    STEP_TIMER(n, 2);
    spill_acc(red, acc, bend - b0);
    STEP_TIMER(n, 3);
    __syncthreads();
    STEP_TIMER(n, 4);
    if (n == T) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        if (!live[u]) continue;
        const long long o = (long long)(b0 + bl_[u]) * H + J0 + j_[u];
        const float dh0 = red_sum<NW, BG, HS>(red, bl_[u], j_[u]) + hcar[u];
        if (a.dh0) ((TS*)a.dh0)[o] = from_f<TS>(dh0);
        if (CELL == CELL_LSTM && a.dc0) ((TS*)a.dc0)[o] = from_f<TS>(dcar[u]);
      }
      if constexpr (FDW) dw_accumulate(hbuf + ((T - 1) & 1) * BG * HS);
      break;
    }
    float dv[UPT][4];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if constexpr (PIPE) dv[u][0] = dv[u][1] = dv[u][2] = dv[u][3] = 0.f;
      if (!live[u]) continue;
      const long long row = (long long)t * B + b0 + bl_[u];
      // a step past the row's length has zero gate gradients; the gradient
      // arriving at it is carried on unchanged
      const bool act = t < len_[u];
      const float dh_in = red_sum<NW, BG, HS>(red, bl_[u], j_[u]) + hcar[u];
      const float dh = dh_in + to_f(pdy[u]);
      TS* gr = (TS*)a.dg + row * GDH + J0 + j_[u];
      if constexpr (CELL == CELL_LSTM) {
        const float ig = to_f(pz[u][0]), fg = to_f(pz[u][1]), gg = to_f(pz[u][2]), og = to_f(pz[u][3]);
        const float c = to_f(pc[u]), cp = pvalid[u] ? to_f(pprev[u]) : 0.f;
        const float tc = tanhf_(c);
        const float dc = dh * og * (1.f - tc * tc) + dcar[u];
        const float d_o = act ? dh * tc * og * (1.f - og) : 0.f;
        const float d_i = act ? dc * gg * ig * (1.f - ig) : 0.f;
        const float d_f = act ? dc * cp * fg * (1.f - fg) : 0.f;
        const float d_g = act ? dc * ig * (1.f - gg * gg) : 0.f;
        dcar[u] = act ? dc * fg : dcar[u];
        hcar[u] = act ? 0.f : dh_in;
        if constexpr (HH) hbuf[(n & 1) * BG * HS + bl_[u] * HS + j_[u]] = phv[u] ? to_f(phh[u]) : 0.f;
        dv[u][0] = d_i;
        dv[u][1] = d_f;
        dv[u][2] = d_g;
        dv[u][3] = d_o;
        if constexpr (FDW) {
          dbacc[u][0] += d_i;
          dbacc[u][1] += d_f;
          dbacc[u][2] += d_g;
          dbacc[u][3] += d_o;
        }
        if (umaj) {
          // the unit's four gradients: rows 4jj..4jj+3, adjacent in the tile
          char* xs = xslot(n);
          const int jj = J0 + j_[u];
          const unsigned lo = (unsigned)__builtin_bit_cast(unsigned short, (bf16)d_i) |
                              ((unsigned)__builtin_bit_cast(unsigned short, (bf16)d_f) << 16);
          const unsigned hi = (unsigned)__builtin_bit_cast(unsigned short, (bf16)d_g) |
                              ((unsigned)__builtin_bit_cast(unsigned short, (bf16)d_o) << 16);
          unsigned long long* p8 = (unsigned long long*)(xs + xoff<TS>(bl_[u], 4 * jj, packed, MB));
          const unsigned long long v8 = (unsigned long long)lo | ((unsigned long long)hi << 32);
          if (local) *p8 = v8;
          else __hip_atomic_store(p8, v8, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (tiled) {
          char* xs = xslot(n);
          const int jj = J0 + j_[u];
          xstore((TS*)(xs + xoff<TS>(bl_[u], jj, packed, MB)), d_i, local);
          xstore((TS*)(xs + xoff<TS>(bl_[u], H + jj, packed, MB)), d_f, local);
          xstore((TS*)(xs + xoff<TS>(bl_[u], 2 * H + jj, packed, MB)), d_g, local);
          xstore((TS*)(xs + xoff<TS>(bl_[u], 3 * H + jj, packed, MB)), d_o, local);
        } else {
          xstore(gr, d_i, local);
          xstore(gr + H, d_f, local);
          xstore(gr + 2 * H, d_g, local);
          xstore(gr + 3 * H, d_o, local);
        }
      } else {
        const float r = to_f(pz[u][0]), uu = to_f(pz[u][1]), c = to_f(pz[u][2]), nh = to_f(pz[u][3]);
        const float hp = pvalid[u] ? to_f(pprev[u]) : 0.f;
        if constexpr (FDW) hbuf[(n & 1) * BG * HS + bl_[u] * HS + j_[u]] = hp;
        // AUGRU: the state update uses the scaled gate us = (1 - att) * uu
        const float sa = a.att ? 1.f - to_f(pa[u]) : 1.f;
        const float us = sa * uu;
        const float d_us = dh * (hp - c);
        const float d_c = act ? dh * (1.f - us) * (1.f - c * c) : 0.f;
        const float d_u = act ? d_us * sa * uu * (1.f - uu) : 0.f;
        const float d_r = d_c * nh * r * (1.f - r);
        hcar[u] = act ? dh * us : dh_in;
        // this unit's share of the score gradient, summed per row below
        if (a.att) attl[bl_[u] * HS + j_[u]] = act ? -d_us * uu : 0.f;
        dv[u][0] = d_r;
        dv[u][1] = d_u;
        dv[u][2] = d_c;  // input side only: read by later kernels
        dv[u][3] = d_c * r;
        if constexpr (FDW) {
          dbacc[u][0] += d_r;
          dbacc[u][1] += d_u;
          dbacc[u][2] += d_c * r;  // the recurrent candidate row's gradient
        }
        if (!tiled) gr[2 * H] = from_f<TS>(d_c);
        if (tiled) {
          char* xs = xslot(n);
          const int jj = J0 + j_[u];
          xstore((TS*)(xs + xoff<TS>(bl_[u], jj, packed, MB)), d_r, local);
          xstore((TS*)(xs + xoff<TS>(bl_[u], H + jj, packed, MB)), d_u, local);
          xstore((TS*)(xs + xoff<TS>(bl_[u], 2 * H + jj, packed, MB)), d_c * r, local);
        } else {
          xstore(gr, d_r, local);
          xstore(gr + H, d_u, local);
          xstore(gr + 3 * H, d_c * r, local);
        }
      }
    }
    STEP_TIMER(n, 5);
    publish(myflag, n + 1, local);
    STEP_TIMER(n, 6);
    if (CELL == CELL_GRU_RA && a.att) att_rows<HS>(attl, a.datt_part, t, B, b0, bend, a.nSlices, sl);
    if constexpr (PIPE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          ddv[u][g] = dv[u][g];
          pz[u][g] = nz[u][g];
        }
        pdy[u] = ndy[u];
        pc[u] = nc[u];
        pprev[u] = nprev[u];
        pa[u] = na[u];
        pvalid[u] = nvalid[u];
        if constexpr (HH) {
          phh[u] = nhh[u];
          phv[u] = nhv[u];
        }
      }
    } else if (tiled) {
      // gate gradients for the later kernels (the ring carried the exchange)
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        if (!live[u]) continue;
        TS* gr = (TS*)a.dg + ((long long)t * B + b0 + bl_[u]) * GDH + J0 + j_[u];
#pragma unroll
        for (int g = 0; g < 4; ++g) gr[g * H] = from_f<TS>(dv[u][g]);
      }
    }
    STEP_TIMER(n, 7);
  }
  if constexpr (FDW) {
    // this group's partial dW_hh: rows of the wave's k-steps, the slice's units
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int kl = 0; kl < KI; ++kl) {
      const int k = (w * KI + kl) * 16 + 4 * (lane >> 4);
      if (k >= K) break;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int c = J0 + nt * 16 + (lane & 15);
        float* o = a.dwp + ((long long)grp * K + k) * H + c;
        if (c < H) {
          o[0] = dw[kl][nt].x;
          o[H] = dw[kl][nt].y;
          o[2 * H] = dw[kl][nt].z;
          o[3 * H] = dw[kl][nt].w;
        }
      }
    }
    // bias partial: the units' sums over the group's rows, in row order
    __syncthreads();  // the last step's reads of red are done
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * NTH;
      if (unit < UNITS)
#pragma unroll
        for (int g = 0; g < GK; ++g) red[(g * BG + bl_[u]) * HS + j_[u]] = dbacc[u][g];
    }
    __syncthreads();
    for (int i = tid; i < GK * HS; i += NTH) {
      const int g = i / HS, j = i - g * HS;
      float sum = 0.f;
      for (int r = 0; r < BG; ++r) sum += red[(g * BG + r) * HS + j];
      if (J0 + j < H) a.dwp[(long long)a.nGroups * K * H + (long long)grp * K + g * H + J0 + j] = sum;
    }
  }
  STEP_TIMER_CAL(1);
  STEP_TIMER_FLUSH(T + 1);
}

// Basic GRU backward: phase A contracts [d_r, d_u]_{t+1} with W_h{r,u} and
// forms d_c, d_u; phase B contracts d_c_t with W_hc (gradient of r*h_{t-1})
// and forms d_r. Counters advance by two per step.
template <typename TS, int NW, int MB, int NT, int KIA, int KIB>
__global__ __launch_bounds__(NW * 64) void rec_bwd_grub(RecLaunch L) {
  constexpr int NTH = NW * 64, BG = MB * 16, HS = NT * 16;
  constexpr int UNITS = BG * HS;
  constexpr int UPT = (UNITS + NTH - 1) / NTH;
  extern __shared__ float red[];
  STEP_TIMER_DECL;
  float* attl = red + NW * BG * rstride(HS);  // AUGRU score-gradient shares (LDS sized for them when used)

  int grp, sl;
  bool idle;
  RecArgsK& a = launch_slot(L, grp, sl, idle);
  if (idle) return;
  int* myflag = a.flags + (grp * a.nSlices + sl) * a.fstride;
  const int* gflags = a.flags + grp * a.nSlices * a.fstride;
  const bool local =
      group_is_local(myflag, gflags, a.nSlices, a.fstride, a.place_off, a.status, a.timeout_ticks);
  const int tid = threadIdx.x;
  const int H = a.H, B = a.B, T = a.T;
  const int J0 = sl * HS, b0 = grp * a.bg;
  const int bend = min(B, b0 + a.bg);  // rows of this batch group: [b0, bend)
  const long long GZH = (long long)a.GZ * H, GDH = (long long)a.GD * H;

  uint4 WA[NT][wslots<TS>(KIA)], WB[NT][wslots<TS>(KIB)];
  load_w_cols<TS, NT, KIA>(WA, (const TS*)a.W_hh, H, a.perm, J0, 0, 2 * H);
  load_w_cols<TS, NT, KIB>(WB, (const TS*)a.W_hh, H, a.perm, J0, 2, H);

  float hcar[UPT], dhs[UPT], rs[UPT], us[UPT], hps[UPT];
  bool live[UPT];
  int bl_[UPT], j_[UPT], len_[UPT];
  // this wave's rows of the two products ([d_r | d_u] over 2H, d_c over H)
  // and the slices producing them: each wave waits for those only
  int wa0, wan, wb0, wbn;
  {
    constexpr int KSTEP = 4 * Chunk<TS>::KQ;
    const int w = tid >> 6;
    const int ka = w * KIA * KSTEP, kb = w * KIB * KSTEP;
    wave_slices(ka, min(2 * H, ka + KIA * KSTEP), H, HS, a.nSlices, wa0, wan);
    wave_slices(kb, min(H, kb + KIB * KSTEP), H, HS, a.nSlices, wb0, wbn);
  }
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid + u * NTH;
    bl_[u] = unit / HS;
    j_[u] = unit - bl_[u] * HS;
    live[u] = unit < UNITS && b0 + bl_[u] < bend;
    hcar[u] = dhs[u] = rs[u] = us[u] = hps[u] = 0.f;
    len_[u] = T;
    if (live[u] && a.lengths) len_[u] = min(max(a.lengths[b0 + bl_[u]], 0), T);
    if (live[u] && a.dhT) hcar[u] = to_f(((const TS*)a.dhT)[(long long)(b0 + bl_[u]) * H + J0 + j_[u]]);
  }

  STEP_TIMER_CAL(0);
  for (int n = 0; n <= T; ++n) {
    STEP_TIMER(n, 0);
    const int s = T - 1 - n;
    const int t = a.dir ? T - 1 - s : s;
    const int tp = a.dir ? t + 1 : t - 1;
    TS pdy[UPT], pz[UPT][3], pprev[UPT], pa[UPT];
    bool pvalid[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const bool on = live[u] && n < T;
      const long long row = on ? (long long)t * B + b0 + bl_[u] : 0;
      const int jj = on ? J0 + j_[u] : 0;
      const TS* zr = (const TS*)a.z + row * GZH + jj;
      pdy[u] = ((const TS*)a.dy)[row * a.ldy + jj];
      const TS* ap = a.att ? (const TS*)a.att + row : (const TS*)a.dy;
      pa[u] = *ap;
#pragma unroll
      for (int g = 0; g < 3; ++g) pz[u][g] = zr[g * H];
      const bool first = a.dir ? (t == len_[u] - 1) : (t == 0);
      const bool inseq = tp >= 0 && tp < T;
      pvalid[u] = on && (!first || a.h0);
      const TS* hprev = (first && a.h0) ? (const TS*)a.h0 + (on ? (long long)(b0 + bl_[u]) * H + jj : 0)
                      : (const TS*)a.y + (first || !on || !inseq ? 0 : ((long long)tp * B + b0 + bl_[u]) * a.ldy + jj);
      pprev[u] = *hprev;
    }
    {
      f4 acc[MB][NT];
      zero_acc(acc);
      if (n > 0) {
        wait_flags(gflags + wa0 * a.fstride, wan, 2 * n, a.status, a.timeout_ticks, a.fstride, local);
        STEP_TIMER(n, 1);
        const int tn = a.dir ? T - 1 - (s + 1) : (s + 1);
        contract<TS, MB, NT, KIA>(acc, WA, (const TS*)a.dg + (long long)tn * B * GDH, GDH, b0, bend, 2 * H, 1 << 30,
                                  0);
      }
      spill_acc(red, acc, bend - b0);
    }
    STEP_TIMER(n, 2);
    __syncthreads();
    if (n == T) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        if (!live[u] || !a.dh0) continue;
        ((TS*)a.dh0)[(long long)(b0 + bl_[u]) * H + J0 + j_[u]] =
            from_f<TS>(red_sum<NW, BG, HS>(red, bl_[u], j_[u]) + hcar[u]);
      }
      break;
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      const long long row = (long long)t * B + b0 + bl_[u];
      // past the row's length: zero gate gradients, carry passed on unchanged
      const bool act = t < len_[u];
      const float dh_in = red_sum<NW, BG, HS>(red, bl_[u], j_[u]) + hcar[u];
      const float dh = dh_in + to_f(pdy[u]);
      const float r = to_f(pz[u][0]), uu = to_f(pz[u][1]), c = to_f(pz[u][2]);
      const float hp = pvalid[u] ? to_f(pprev[u]) : 0.f;
      // AUGRU: the state update uses the scaled gate (1 - att) * uu
      const float sa = a.att ? 1.f - to_f(pa[u]) : 1.f;
      const float d_us = dh * (hp - c);
      const float d_c = act ? dh * (1.f - sa * uu) * (1.f - c * c) : 0.f;
      const float d_u = act ? d_us * sa * uu * (1.f - uu) : 0.f;
      if (a.att) attl[bl_[u] * HS + j_[u]] = act ? -d_us * uu : 0.f;
      TS* gr = (TS*)a.dg + row * GDH + J0 + j_[u];
      xstore(gr + H, d_u, local);
      xstore(gr + 2 * H, d_c, local);
      // an inactive row keeps its incoming carry here (its d_rh is zero)
      dhs[u] = act ? dh : dh_in;
      rs[u] = r;
      us[u] = sa * uu;
      hps[u] = hp;
    }
    STEP_TIMER(n, 3);
    publish(myflag, 2 * n + 1, local);
    if (a.att) att_rows<HS>(attl, a.datt_part, t, B, b0, bend, a.nSlices, sl);
    STEP_TIMER(n, 4);
    wait_flags(gflags + wb0 * a.fstride, wbn, 2 * n + 1, a.status, a.timeout_ticks, a.fstride, local);
    STEP_TIMER(n, 5);
    {
      f4 acc[MB][NT];
      zero_acc(acc);
      contract<TS, MB, NT, KIB>(acc, WB, (const TS*)a.dg + (long long)t * B * GDH + 2 * H, GDH, b0, bend, H, 1 << 30,
                                0);
      spill_acc(red, acc, bend - b0);
    }
    __syncthreads();
    STEP_TIMER(n, 6);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      if (!live[u]) continue;
      const long long row = (long long)t * B + b0 + bl_[u];
      const float d_rh = red_sum<NW, BG, HS>(red, bl_[u], j_[u]);
      const bool act = t < len_[u];
      const float d_r = act ? d_rh * hps[u] * rs[u] * (1.f - rs[u]) : 0.f;
      xstore((TS*)a.dg + row * GDH + J0 + j_[u], d_r, local);
      hcar[u] = act ? d_rh * rs[u] + dhs[u] * us[u] : dhs[u];
    }
    STEP_TIMER(n, 7);
    publish(myflag, 2 * n + 2, local);
  }
  STEP_TIMER_CAL(1);
  STEP_TIMER_FLUSH(T + 1);
}

// ------------------------------------------------- exchange-only probe --
// The step exchange of a plan with nothing else: the same grid, placement
// check, counters, per-wave waits and exchange-ring layout as the ring
// kernels above, and per step the same loads (this wave's k-steps of the
// previous step's vector) and stores (each unit's gk values, one 8-byte piece
// when unit-major), but no contraction and no gate arithmetic. Its time per
// step is the floor that the exchange protocol alone puts under a step. A
// measurement probe: rnn_handshake_probe launches it, the layer calls never.
template <typename TS, int NW>
__global__ __launch_bounds__(NW * 64) void rec_exchange_probe(RecLaunch L, int K, int ki, int gk, int umaj) {
  constexpr int NTH = NW * 64;
  constexpr int KSTEP = 4 * Chunk<TS>::KQ;
  int grp, sl;
  bool idle;
  RecArgsK& a = launch_slot(L, grp, sl, idle);
  if (idle) return;
  const int fstride = a.fstride, place_off = a.place_off;
  int* myflag = a.flags + (grp * a.nSlices + sl) * fstride;
  const int* gflags = a.flags + grp * a.nSlices * fstride;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = a.H, T = a.T, HS = a.Hs;
  const int J0 = sl * HS, b0 = grp * a.bg;
  const int bend = min(a.B, b0 + a.bg);
  const bool packed = a.xpacked != 0;
  const int xbytes = K * (packed ? 8 : 16) * (int)sizeof(TS);
  auto xslot = [&](int step) { return a.xbuf + ((long long)(step & 1) * a.nGroups + grp) * a.xg_bytes; };
  int ws0, wsn;
  {
    const int k0 = w * ki * KSTEP, k1 = min(K, k0 + ki * KSTEP);
    if (umaj && k1 > k0) {
      ws0 = (k0 >> 2) / HS;
      wsn = ((k1 - 1) >> 2) / HS + 1 - ws0;
    } else {
      wave_slices(k0, k1, H, HS, a.nSlices, ws0, wsn);
    }
  }
  const bool local = group_is_local(myflag, gflags, a.nSlices, fstride, place_off, a.status, a.timeout_ticks);
  const int units = (bend - b0) * HS;
  unsigned keep = 0;
  for (int s = 0; s < T; ++s) {
    if (s > 0) {
      wait_flags(gflags + ws0 * fstride, wsn, s, a.status, a.timeout_ticks, fstride, a.bg <= 16 && local);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)xslot(s - 1), (short)0, xbytes, BUF_RSRC_W3);
      const int nl = packed ? ki / 2 : ki;
      const int base = packed ? (w * ki) / 2 : w * ki;
      for (int i = 0; i < nl; ++i) {
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, (base + i) * 1024 + lane * 16, 0, CPOL_SC1);
        keep ^= r[0] ^ r[1] ^ r[2] ^ r[3];
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // values that depend on the loads (zero), so that they stay live
    const float v = (float)(keep & 0u);
    for (int unit = tid; unit < units; unit += NTH) {
      const int bl = unit / HS, j = unit - bl * HS, jj = J0 + j;
      char* xs = xslot(s);
      if (umaj) {
        unsigned long long* p8 = (unsigned long long*)(xs + xoff<TS>(bl, 4 * jj, packed, 1));
        if (local) *p8 = (unsigned long long)__float_as_uint(v);
        else __hip_atomic_store(p8, (unsigned long long)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        for (int g = 0; g < gk; ++g) xstore((TS*)(xs + xoff<TS>(bl, g * H + jj, packed, 1)), v, local);
      }
    }
    publish(myflag, s + 1, local);
  }
  asm volatile("" ::"v"(keep));
}

// ------------------------------------------------------------ plans ------
struct Entry {
  int cell, dtype, fwd, nw, mb, nt, ki, kib;
  const void* func;
  const void* func_plain;  // variant without an exchange ring (NULL: basic GRU, func serves both)
  const void* func_fdw;    // backward ring variant with the fused dW_hh (NULL: none)
};

#define F_LSTM(TS, NW, MB, NT, KI) \
  (const void*)rec_fwd<CELL_LSTM, TS, NW, MB, NT, KI, true>, (const void*)rec_fwd<CELL_LSTM, TS, NW, MB, NT, KI, false>
#define F_GRA(TS, NW, MB, NT, KI) \
  (const void*)rec_fwd<CELL_GRU_RA, TS, NW, MB, NT, KI, true>, (const void*)rec_fwd<CELL_GRU_RA, TS, NW, MB, NT, KI, false>
#define B_LSTM(TS, NW, MB, NT, KI) \
  (const void*)rec_bwd<CELL_LSTM, TS, NW, MB, NT, KI, true>, (const void*)rec_bwd<CELL_LSTM, TS, NW, MB, NT, KI, false>
#define B_GRA(TS, NW, MB, NT, KI) \
  (const void*)rec_bwd<CELL_GRU_RA, TS, NW, MB, NT, KI, true>, (const void*)rec_bwd<CELL_GRU_RA, TS, NW, MB, NT, KI, false>
#define B_LSTM_FDW(TS, NW, MB, NT, KI) B_LSTM(TS, NW, MB, NT, KI), (const void*)rec_bwd<CELL_LSTM, TS, NW, MB, NT, KI, true, true>
#define B_GRA_FDW(TS, NW, MB, NT, KI) \
  B_GRA(TS, NW, MB, NT, KI), (const void*)rec_bwd<CELL_GRU_RA, TS, NW, MB, NT, KI, true, true>

// dtype 0 = fp32, 1 = bf16
const Entry kTable[] = {
    // forward LSTM
    {CELL_LSTM, 1, 1, 4, 1, 4, 8, 0, F_LSTM(bf16, 4, 1, 4, 8)},
    {CELL_LSTM, 1, 1, 4, 1, 1, 8, 0, F_LSTM(bf16, 4, 1, 1, 8)},
    {CELL_LSTM, 1, 1, 8, 1, 8, 4, 0, F_LSTM(bf16, 8, 1, 8, 4)},
    {CELL_LSTM, 1, 1, 4, 8, 2, 16, 0, F_LSTM(bf16, 4, 8, 2, 16)},
    {CELL_LSTM, 1, 1, 8, 8, 2, 8, 0, F_LSTM(bf16, 8, 8, 2, 8)},
    {CELL_LSTM, 1, 1, 4, 4, 4, 16, 0, F_LSTM(bf16, 4, 4, 4, 16)},
    {CELL_LSTM, 0, 1, 4, 1, 4, 8, 0, F_LSTM(float, 4, 1, 4, 8)},
    {CELL_LSTM, 0, 1, 4, 1, 1, 8, 0, F_LSTM(float, 4, 1, 1, 8)},
    {CELL_LSTM, 0, 1, 8, 1, 4, 4, 0, F_LSTM(float, 8, 1, 4, 4)},
    // forward reset-after GRU
    {CELL_GRU_RA, 1, 1, 4, 1, 3, 8, 0, F_GRA(bf16, 4, 1, 3, 8)},
    {CELL_GRU_RA, 1, 1, 8, 1, 6, 4, 0, F_GRA(bf16, 8, 1, 6, 4)},
    {CELL_GRU_RA, 1, 1, 8, 4, 3, 8, 0, F_GRA(bf16, 8, 4, 3, 8)},
    {CELL_GRU_RA, 0, 1, 4, 1, 3, 8, 0, F_GRA(float, 4, 1, 3, 8)},
    {CELL_GRU_RA, 0, 1, 4, 1, 3, 4, 0, F_GRA(float, 4, 1, 3, 4)},
    {CELL_GRU_RA, 0, 1, 8, 1, 3, 2, 0, F_GRA(float, 8, 1, 3, 2)},
    // forward basic GRU (nt = candidate tiles)
    {CELL_GRU_BASIC, 1, 1, 4, 1, 1, 8, 0, (const void*)rec_fwd_grub<bf16, 4, 1, 1, 8>},
    {CELL_GRU_BASIC, 0, 1, 4, 1, 1, 8, 0, (const void*)rec_fwd_grub<float, 4, 1, 1, 8>},
    {CELL_GRU_BASIC, 0, 1, 4, 1, 1, 4, 0, (const void*)rec_fwd_grub<float, 4, 1, 1, 4>},
    // backward LSTM
    {CELL_LSTM, 1, 0, 4, 1, 1, 32, 0, B_LSTM(bf16, 4, 1, 1, 32)},
    {CELL_LSTM, 1, 0, 8, 1, 2, 16, 0, B_LSTM(bf16, 8, 1, 2, 16)},
    {CELL_LSTM, 1, 0, 8, 4, 1, 32, 0, B_LSTM(bf16, 8, 4, 1, 32)},
    {CELL_LSTM, 0, 0, 4, 1, 1, 32, 0, B_LSTM(float, 4, 1, 1, 32)},
    {CELL_LSTM, 0, 0, 8, 1, 1, 16, 0, B_LSTM(float, 8, 1, 1, 16)},
    {CELL_LSTM, 0, 0, 4, 1, 1, 8, 0, B_LSTM_FDW(float, 4, 1, 1, 8)},
    // backward reset-after GRU
    {CELL_GRU_RA, 1, 0, 4, 1, 1, 32, 0, B_GRA(bf16, 4, 1, 1, 32)},
    {CELL_GRU_RA, 1, 0, 8, 1, 2, 16, 0, B_GRA(bf16, 8, 1, 2, 16)},
    {CELL_GRU_RA, 1, 0, 4, 4, 1, 48, 0, B_GRA(bf16, 4, 4, 1, 48)},
    {CELL_GRU_RA, 1, 0, 8, 4, 1, 24, 0, B_GRA(bf16, 8, 4, 1, 24)},
    {CELL_GRU_RA, 0, 0, 4, 1, 1, 32, 0, B_GRA(float, 4, 1, 1, 32)},
    {CELL_GRU_RA, 0, 0, 4, 1, 1, 12, 0, B_GRA_FDW(float, 4, 1, 1, 12)},
    {CELL_GRU_RA, 0, 0, 8, 1, 1, 6, 0, B_GRA_FDW(float, 8, 1, 1, 6)},
    // backward basic GRU (ki = phase A k-steps, kib = phase B)
    {CELL_GRU_BASIC, 1, 0, 4, 1, 1, 16, 8, (const void*)rec_bwd_grub<bf16, 4, 1, 1, 16, 8>},
    {CELL_GRU_BASIC, 0, 0, 4, 1, 1, 16, 8, (const void*)rec_bwd_grub<float, 4, 1, 1, 16, 8>},
    {CELL_GRU_BASIC, 0, 0, 4, 1, 1, 8, 4, (const void*)rec_bwd_grub<float, 4, 1, 1, 8, 4>},
};

int units_per_wg(const Entry& e) {
  if (!e.fwd) return e.nt * 16;
  if (e.cell == CELL_LSTM) return e.nt * 16 / 4;
  if (e.cell == CELL_GRU_RA) return e.nt * 16 / 3;
  return e.nt * 16;
}

size_t lds_of(const Entry& e) {
  int ncol;
  if (e.fwd) ncol = (e.cell == CELL_GRU_BASIC) ? 2 * e.nt * 16 : e.nt * 16;
  else ncol = e.nt * 16;
  return (size_t)e.nw * e.mb * 16 * rstride(ncol) * sizeof(float);
}

// XCDs a batch group of `slices` workgroups covers under launch_slot, for a
// direction of nwg workgroups spread over `xcds` XCDs: with nwg a multiple of
// xcds each XCD holds nwg/xcds consecutive indices, otherwise the blocks are
// spread round-robin over all 8.
int xcd_span(long long nwg, int slices, int xcds) {
  if (nwg % xcds == 0) {
    const long long per = nwg / xcds;
    return (int)((slices + per - 1) / per);
  }
  return slices < 8 ? slices : 8;
}

// Padded placement for groups that would span XCDs under the natural one:
// whole groups per XCD (as few per XCD as the groups allow, spread over all
// of the direction's XCDs). Returns per_xcd, or 0 when it does not apply
// (groups already local, a group larger than an XCD, or more blocks than CUs).
int padded_per_xcd(int groups, int slices, int xcds, int cu_count) {
  const long long nwg = (long long)groups * slices;
  if (xcd_span(nwg, slices, xcds) <= 1) return 0;
  const int cu_per_xcd = cu_count / xcds;
  const int gpx = (groups + xcds - 1) / xcds;
  const int per = gpx * slices;
  if (per > cu_per_xcd) return 0;
  return per;
}

// Modelled time of one step (us): a step handshake costs ~1 us when a
// batch group shares one XCD and ~2 us across XCDs (measured); a 16x16x32
// bf16 MFMA occupies its SIMD for 16 cycles (6.67 ns at 2.4 GHz: the
// published 2.5 PFLOP/s dense peak over 1024 SIMDs), and a wave alone on its
// SIMD was measured to issue one every ~10.8 ns; a fp32 k-step is three such
// MFMAs per tile (six per pair of k-steps on the bf16 pieces) plus the split
// of the wave's 4 vector values into pieces, 14 VALU instructions of 4
// cycles (three conversions and four dot products per two values), once for
// all tiles; every CU reads the whole exchanged vector of its group per
// step, ~150 GB/s from the tiled ring and ~75 GB/s from row layout
// (measured); the gate epilogue costs ~0.2 us per unit a thread carries.
//
// Contraction time of one product: wave w owns k-steps [w*ki, w*ki+ki) of
// the ksteps the contraction has (waves past the end have none) and waves
// w, w+4 share SIMD w%4, so the busiest SIMD sets the time.
double contraction_us(int nw, int ki, int ntiles, int K, int kstep) {
  const int ks = (K + kstep - 1) / kstep;
  int worst = 0, busy_worst = 0;
  for (int sm = 0; sm < 4; ++sm) {
    int sum = 0, busy = 0;
    for (int w = sm; w < nw; w += 4) {
      const int kw = std::min(ki, std::max(0, ks - w * ki));
      sum += kw;
      busy += kw > 0;
    }
    if (sum > worst) {
      worst = sum;
      busy_worst = busy;
    }
  }
  const double lone = busy_worst >= 2 ? 1.0 : 10.8 / 6.67;
  if (kstep == 32) return worst * ntiles * 16.0 / 2.4e3 * lone;  // us per 16x16 k-step on a SIMD
  return worst * (ntiles * 3.0 * 16.0 * lone + 56.0) / 2.4e3;
}

double step_cost(const Entry& e, int bg, int span, int H, int K, int kstep, int esize, bool ring) {
  const double hand = span <= 1 ? 1.0 : 2.0;
  double mfma, data;
  if (e.cell == CELL_GRU_BASIC) {
    // two products per step, each behind its own exchange
    if (e.fwd) mfma = contraction_us(e.nw, e.ki, 2 * e.nt * e.mb, H, kstep) + contraction_us(e.nw, e.ki, e.nt * e.mb, H, kstep);
    else mfma = contraction_us(e.nw, e.ki, e.nt * e.mb, 2 * H, kstep) + contraction_us(e.nw, e.kib, e.nt * e.mb, H, kstep);
    data = (double)bg * (e.fwd ? 2 * H : 3 * H) * esize / 75e3;
    return 2 * hand + mfma + data + 0.2 * 2;
  }
  mfma = contraction_us(e.nw, e.ki, e.nt * e.mb, K, kstep);
  data = (double)bg * K * esize / (ring ? 150e3 : 75e3);
  const int units = e.mb * 16 * units_per_wg(e);
  const int upt = (units + e.nw * 64 - 1) / (e.nw * 64);
  return hand + mfma + data + 0.2 * upt;
}

// Fused dW_hh (fp32): each wave adds one 16x16x4 MFMA (32 cycles) per
// k-step, unit tile and 4 batch rows per step; they run while the workgroup
// waits for the next step, so only what exceeds the modelled step time
// outside the contraction shows.
double fused_dw_us(const Entry& e, int bg, int K, double step_us, int kstep) {
  const int ks = (K + kstep - 1) / kstep;
  int worst = 0;
  for (int sm = 0; sm < 4; ++sm) {
    int sum = 0;
    for (int w = sm; w < e.nw; w += 4) sum += std::min(e.ki, std::max(0, ks - w * e.ki));
    worst = std::max(worst, sum);
  }
  const double dw = worst * e.nt * ((bg + 3) / 4) * 32.0 / 2.4e3;
  const double slack = step_us - contraction_us(e.nw, e.ki, e.nt * e.mb, K, kstep);
  return std::max(0.0, dw - slack);
}

bool choose(int cell, int dtype, int fwd, int B, int H, int cu_count, int xcds, RecPlan* p) {
  const int kstep = dtype ? 32 : 16;
  const int esize = dtype ? 2 : 4;
  double best = 1e300;
  bool found = false;
  for (const Entry& e : kTable) {
    if (e.cell != cell || e.dtype != dtype || e.fwd != fwd) continue;
    const int hs = units_per_wg(e);
    if (H % hs) continue;
    // contraction length of the (first) recurrent product
    int K = H;
    if (!fwd) K = (cell == CELL_LSTM) ? 4 * H : (cell == CELL_GRU_RA ? 3 * H : 2 * H);
    if ((long long)e.nw * e.ki * kstep < K) continue;
    if (cell == CELL_GRU_BASIC && !fwd && (long long)e.nw * e.kib * kstep < H) continue;
    const int rows = e.mb * 16;
    // batch rows per group: the full MFMA tile, or half of it (more, smaller
    // groups: shorter handshakes, half the rows of the tile idle)
    for (int bg : {rows, rows / 2, rows / 4}) {
      if (bg < 4 || (bg != rows && e.mb != 1)) continue;
      const int groups = (B + bg - 1) / bg;
      const int slices = H / hs;
      const long long nwg = (long long)groups * slices;
      if (nwg > cu_count) continue;  // at most one persistent workgroup per CU
      const bool ring = (cell != CELL_GRU_BASIC) && ((long long)K * esize) % 64 == 0 && bg <= 16 * e.mb;
      const int per_xcd = padded_per_xcd(groups, slices, xcds, cu_count);
      const int span = per_xcd > 0 ? 1 : xcd_span(nwg, slices, xcds);
      const double cost = step_cost(e, bg, span, H, K, kstep, esize, ring);
      // on a tie, the entry with the fused dW_hh variant
      const bool fdw = e.func_fdw && ring && bg <= 8;
      if (cost < best - 1e-9 || (found && cost < best + 1e-9 && fdw && !p->func_fdw)) {
        best = cost;
        *p = RecPlan{e.nw, e.mb, e.nt, e.ki, hs, groups, slices, bg, cost, e.func, lds_of(e), span, e.func_plain,
                     per_xcd, fdw ? e.func_fdw : nullptr, fdw ? fused_dw_us(e, bg, K, cost, kstep) : 0.0, xcds};
        found = true;
      }
    }
  }
  return found;
}

}  // namespace

bool plan_fwd(int cell, int dtype, int B, int H, int cu_count, int xcds, RecPlan* p) {
  return choose(cell, dtype, 1, B, H, cu_count, xcds, p);
}
bool plan_bwd(int cell, int dtype, int B, int H, int cu_count, int xcds, RecPlan* p) {
  return choose(cell, dtype, 0, B, H, cu_count, xcds, p);
}

long long launch_blocks(const RecPlan& p, bool dual) {
  const long long per_dir = p.per_xcd > 0 ? (long long)p.xcds * p.per_xcd : (long long)p.nGroups * p.nSlices;
  return dual ? 2 * per_dir : per_dir;
}

int max_coresident(const RecPlan& p) {
  // the least of the variants a launch of the plan may run
  int n = 0;
  for (const void* f : {p.func, p.func_plain, p.func_fdw}) {
    if (!f) continue;
    int m = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, f, p.nw * 64, p.lds_bytes) != hipSuccess) return 0;
    n = (f == p.func) ? m : std::min(n, m);
  }
  return n;
}

hipError_t launch_exchange_probe(const RecPlan& p, const RecLaunch& L, int dtype, int K, int gk, int umaj,
                                 hipStream_t s) {
  const void* f = nullptr;
  if (p.nw == 4) f = dtype ? (const void*)rec_exchange_probe<bf16, 4> : (const void*)rec_exchange_probe<float, 4>;
  if (p.nw == 8) f = dtype ? (const void*)rec_exchange_probe<bf16, 8> : (const void*)rec_exchange_probe<float, 8>;
  if (f == nullptr || p.mb != 1 || L.d[0].xbuf == nullptr) return hipErrorInvalidValue;
  const int n = p.nGroups * p.nSlices;
  if (L.dual && n % 4 != 0 && p.per_xcd == 0) return hipErrorInvalidValue;
  RecLaunch args = L;
  args.per_xcd = p.per_xcd;
  int ki = p.ki;
  void* kargs[] = {&args, &K, &ki, &gk, &umaj};
  return hipLaunchCooperativeKernel(f, dim3(launch_blocks(p, L.dual != 0)), dim3(p.nw * 64), kargs, 0, s);
}

hipError_t launch_rec(const RecPlan& p, const RecLaunch& L, hipStream_t s) {
  // LSTM and reset-after GRU kernels come in a ring and a row-read variant
  const void* f = (p.func_plain && L.d[0].xbuf == nullptr) ? p.func_plain : p.func;
  // fused dW_hh: the plan's variant, packed ring tiles, in every direction
  const bool fdw = L.d[0].dwp != nullptr;
  if (fdw || (L.dual && L.d[1].dwp != nullptr)) {
    if (!p.func_fdw || L.d[0].xbuf == nullptr || !L.d[0].xpacked || (L.dual && (L.d[1].dwp == nullptr || !L.d[1].xpacked)))
      return hipErrorInvalidValue;
    f = p.func_fdw;
  }
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds_bytes);
  if (e != hipSuccess) return e;
  const int n = p.nGroups * p.nSlices;
  if (L.dual && n % 4 != 0 && p.per_xcd == 0) return hipErrorInvalidValue;
  RecLaunch args = L;
  args.per_xcd = p.per_xcd;
  void* kargs[] = {&args};
  return hipLaunchCooperativeKernel(f, dim3(launch_blocks(p, L.dual != 0)), dim3(p.nw * 64), kargs,
                                    (unsigned)p.lds_bytes, s);
}

}  // namespace rnn
