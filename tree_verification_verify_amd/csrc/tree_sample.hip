// Multi-step speculative sampling over a draft tree (the verification walk).
//
// Rules: greedy exact match at T = 0 and, at T > 0, recursive rejection
// sampling without replacement or, as a per-call choice, with replacement
// (survey page, Taxonomy rules (a), (c) and (b); SpecInfer's
// residual-renormalising walk in its Timeline section), with the sibling
// proposals rebuilt from the shared draft logits and the sibling draw order
// (TreeSpark §1, §3.3 and Proposition 1), and one correction or bonus token
// at the stop node (TreeSpark §3.2 step 3).
//
// Design (gfx950):
//  * One team of W workgroups per request, all on one XCD; the team splits
//    the vocabulary into W slices, so every vocab-wide reduction is W-way
//    parallel. Every member combines the gathered partials in the same fixed
//    order, so all members take bit-identical decisions without a broadcast.
//  * The walk is a chain of dependent vocabulary passes (one per visited
//    node, one per rejected sibling), so its speed is the latency of one
//    pass. A member keeps its slice of the visited node's two logit rows in
//    registers and LDS (up to kResCh chunks of 1024 logits per row): the
//    slice is loaded with every load in flight at once, and the residual
//    passes after rejections reuse it without touching memory. Larger
//    slices stream.
//  * Team exchange: each member publishes 64-bit words holding a 32-bit
//    payload and a 32-bit tag, and readers poll the words themselves until
//    the tag is the expected one: one memory round trip per exchange, no
//    counter. Tags come from a per-request sequence kept in the workspace
//    that only grows, and each request owns a fixed slot region, so a word
//    left by an earlier call never carries a live tag.
//  * The children of the visited node, their tokens' logits and their
//    uniforms are fetched at the start of the visit, beside the slice loads.
//  * No residual vector is stored. After rejecting siblings x_1..x_j the
//    residual is max(p - a q, 0) / B with scalars a_{j+1} = a_j + B_j / S_j,
//    B_{j+1} = sum_y max(p(y) - a_{j+1} q(y), 0), S_j = 1 - sum_{i<j} q(x_i)
//    (a rejected token's residual is already 0, so removing it from the
//    proposal is implicit). With replacement the proposal stays q: S_j = 1.
//    The per-slice sums of the last pass (or of p, at a leaf) locate the
//    slice of the correction/bonus draw, so the draw rescans one slice only.
//  * Arithmetic: every single value that decides (p(x), q(x), ratios,
//    rescale factors, a, B, S) is fp64, from a 64-entry table with a
//    degree-5 polynomial (~1 ulp). Vocabulary sums add fp32 exps in fp64:
//    each exp takes an fp64 argument formed by one fma from the fp32 logit
//    (about 1.5e-7 relative), and a resident slice keeps the exps in place
//    of its logits for the residual passes and the final draw. Decisions
//    therefore agree with an fp64 reference except within ~1e-6 of a
//    threshold. Streamed slices use a table exp (2^(j/256), quartic
//    polynomial) throughout.
//  * T = 0 requests: the team splits the rows; argmax (lowest index on ties)
//    of every row, then the exact-match flags; no draft logits are read.
#include <math.h>
#include <stdlib.h>

#include <atomic>

#include "tv_device.hpp"
#include "tv_internal.hpp"

namespace tv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxTeam = 16;             // members per team (one XCD holds a team)
constexpr int kResCh = 10;               // resident chunks (1024 logits) per row per member
constexpr int kLdsCh = 3;                // of which the last kLdsCh live in LDS
constexpr int kRegCh = kResCh - kLdsCh;  // and the rest in registers
constexpr int kParLds = 1024;            // parents and tokens staged in LDS up to this many rows
constexpr int kKids = 64;                // children listed (and prefetched) per visit
constexpr int kSlotWords = 8;            // 64-bit words per (member, parity) exchange slot
// Per-request workspace block at a fixed stride (so a workspace serves any
// batch up to the one it was sized for): greedy barrier counter (byte 0),
// exchange tag sequence (byte 4), exchange slots from byte 256.
constexpr size_t kReqSlotsOff = 256;
constexpr size_t kReqBytes = kReqSlotsOff + size_t(kMaxTeam) * 2 * kSlotWords * sizeof(uint64_t);
static_assert(kReqBytes == kSampleReqBytes, "request block size is part of the workspace contract");
// A team wait gives up after this many ticks of the 100 MHz real-time
// counter (0.2 s; a wait that is not stalled lasts microseconds). After one
// wait has given up, the member skips every later wait and leaves.
constexpr uint64_t kWaitTicksDefault = 20000000ull;

struct SampleParams {
  const float* t;
  const float* d;
  const int32_t* tokens;
  const int32_t* node_indptr;
  const int32_t* parent;
  const float* temperature;
  const float* uniforms;
  int8_t* flag;
  int32_t* next_token;
  uint32_t* status;
  char* req;  // per-request blocks of kReqBytes
  int B, V, W, max_nodes;
  int with_replacement;  // rule (b): the stage proposal stays q
  int greedy_path;       // T = 0: only the rows the walk visits
  uint64_t wait_ticks;   // team wait limit (real-time counter ticks)
};

// ---------------------------------------------------------------------------
// exp(a) for a <= 0 in fp64, for single values: a = (64 k + j) ln2/64 + r,
// |r| <= ln2/128, e^a = 2^k * 2^(j/64) * P(r) with P the degree-5 Taylor
// polynomial (remainder below 2^-53 on that interval). tbl[j] = 2^(j/64).
constexpr double kInvLn2x64 = 92.33248261689366;
constexpr double kLn2by64Hi = 0.01083042469326756;  // low mantissa bits zero: n*hi exact
constexpr double kLn2by64Lo = 2.9815858269852933e-12;

__device__ inline double exp_nonpos(double a, const double* tbl) {
  a = fmax(a, -746.0);  // -inf and anything below underflow to 0 through ldexp
  const double n = rint(a * kInvLn2x64);
  const double r = fma(-n, kLn2by64Lo, fma(-n, kLn2by64Hi, a));
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = int(n);
  return ldexp(tbl[ni & 63] * p, ni >> 6);
}

// exp for vocabulary sums, taking z = x * 256/ln2 (x <= 0): z = 256 k + j +
// f with |f| <= 1/2 (rounding by the 1.5 * 2^52 shift, whose low word is
// then the integer), e^x = 2^k * 2^(j/256) * e^(f ln2/256), the last factor
// a quartic (truncation below 4e-17 for |f ln2/256| <= 1.4e-3).
// z below -1100 * 256 (e^x < 2^-1100, and -inf) gives exactly 0.
// tbl[j] = 2^(j/256).
constexpr int kZBits = 8;
constexpr int kZTable = 1 << kZBits;
constexpr double kZScale = double(kZTable) / 0.69314718055994530942;
constexpr double kZC1 = 0.69314718055994530942 / double(kZTable);
constexpr double kZC2 = kZC1 * kZC1 / 2.0;
constexpr double kZC3 = kZC1 * kZC1 * kZC1 / 6.0;
constexpr double kZC4 = kZC1 * kZC1 * kZC1 * kZC1 / 24.0;
constexpr double kZFloor = -1100.0 * kZTable;
constexpr double kShift52 = 6755399441055744.0;  // 1.5 * 2^52
constexpr double kLog2E = 1.4426950408889634074;

__device__ inline double exp_z(double z, const double* tbl) {
  z = fmax(z, kZFloor);
  const double nd = z + kShift52;
  const int n = __double2loint(nd);
  const double f = z - (nd - kShift52);
  double q = fma(f, kZC4, kZC3);
  q = fma(q, f, kZC2);
  q = fma(q, f, kZC1);
  q *= f;
  const double tj = tbl[n & (kZTable - 1)];
  return ldexp(fma(tj, q, tj), n >> kZBits);
}

// 2^z for z <= 0 given in fp64: z = n + f with n an integer and |f| <= 1/2
// (rounding by the 1.5 * 2^52 shift, whose low word is then n), 2^f by the
// hardware exp2 in fp32 (f is exact to 2^-25, the result to ~1 ulp),
// scaled by 2^n. The argument keeps its fp64 absolute precision, so the
// result's relative error stays ~1.5e-7 however far z is below 0; z below
// -200 (and -inf) gives 0.
__device__ inline float exp2_split(double z) {
  z = fmax(z, -200.0);
  const double nd = z + kShift52;
  const int n = __double2loint(nd);
  const float f = float(z - (nd - kShift52));
  return ldexpf(__builtin_amdgcn_exp2f(f), n);
}

// Empty volatile asm on a value: the value is taken to be produced (or
// consumed) at that point in program order. Used to fence units of exp work
// so the compiler keeps one float4 in flight at a time (the resident slice
// already occupies most of the register budget) and does not keep widened
// copies of the slice alive between passes.
__device__ inline float4 opaque(float4 x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
  return x;
}
__device__ inline double opaque(double x) {
  asm volatile("" : "+v"(x));
  return x;
}

// exp_z of the four lanes of x at z = x * A + b, summed in lane order; the
// four table reads are issued together so their LDS latency overlaps.
__device__ inline double exp4_sum(float4 x, double A, double b, const double* tbl) {
  x = opaque(x);
  const float xs[4] = {x.x, x.y, x.z, x.w};
  double f[4], tj[4];
  int n[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double z = fmax(fma(double(xs[e]), A, b), kZFloor);
    const double nd = z + kShift52;
    n[e] = __double2loint(nd);
    f[e] = z - (nd - kShift52);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) tj[e] = tbl[n[e] & (kZTable - 1)];
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    double q = fma(f[e], kZC4, kZC3);
    q = fma(q, f[e], kZC2);
    q = fma(q, f[e], kZC1);
    q *= f[e];
    s += ldexp(fma(tj[e], q, tj[e]), n[e] >> kZBits);
  }
  return opaque(s);
}

// ---------------------------------------------------------------------------
// Team exchange (T > 0): tagged 64-bit words.

struct Team {
  uint64_t* slots;  // this request's region: [member][2 parities][kSlotWords]
  uint32_t seq;     // tag base of this call (the request's sequence at entry)
  int phase;        // exchanges completed so far
  int W;
  int member;
  uint32_t* status;
  uint64_t wait_ticks;
  int* s_dead;      // LDS flag: a wait of this member gave up (sticky)
};

// Bounded wait shared by the team exchange and the greedy barrier: true
// while the caller should keep polling. Gives up (status bit, LDS flag) once
// the wait has lasted wait_ticks, or at once when another thread of the
// member already gave up.
__device__ inline bool keep_waiting(uint64_t t0, uint64_t ticks, uint32_t* status, int* s_dead) {
  if (*reinterpret_cast<volatile int*>(s_dead)) return false;
  if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
    raise_status(status, TV_DEV_TIMEOUT);
    *reinterpret_cast<volatile int*>(s_dead) = 1;
    return false;
  }
  __builtin_amdgcn_s_sleep(1);
  return true;
}

// Word k of this member's payload for the next exchange. Stored
// device-coherent (agent scope): readers on other CUs poll it.
__device__ inline void ll_put(Team& tm, int k, uint32_t payload, uint32_t* s_words) {
  if (tm.W == 1) {
    s_words[k] = payload;
    return;
  }
  const uint32_t tag = tm.seq + uint32_t(tm.phase) + 1u;
  uint64_t* a = tm.slots + (size_t(tm.member) * 2 + ((tm.phase + 1) & 1)) * kSlotWords + k;
  __hip_atomic_store(a, (uint64_t(tag) << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Words 0..K-1 of every member for the next exchange into s_words[w * K + k]
// (one polling thread per word; bounded spin). A member two exchanges ahead
// cannot overwrite a slot still being read: it must first have read this
// member's next words, which are published only after this gather.
__device__ bool ll_gather(Team& tm, int K, uint32_t* s_words) {
  if (tm.W > 1 && !*reinterpret_cast<volatile int*>(tm.s_dead)) {
    const uint32_t tag = tm.seq + uint32_t(tm.phase) + 1u;
    const int par = (tm.phase + 1) & 1;
    for (int i = threadIdx.x; i < tm.W * K; i += blockDim.x) {
      const int w = i / K;
      const uint64_t* a = tm.slots + (size_t(w) * 2 + par) * kSlotWords + (i - w * K);
      uint64_t x = __hip_atomic_load(const_cast<uint64_t*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (uint32_t(x >> 32) != tag && keep_waiting(t0, tm.wait_ticks, tm.status, tm.s_dead))
        x = __hip_atomic_load(const_cast<uint64_t*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_words[i] = uint32_t(x);
    }
  }
  __syncthreads();
  tm.phase++;
  // Uniform over the workgroup: every thread reads the flag after the barrier.
  return !*reinterpret_cast<volatile int*>(tm.s_dead);
}

__device__ inline double words_to_double(uint32_t lo, uint32_t hi) {
  return __hiloint2double(int(hi), int(lo));
}

// A value every lane holds identically, moved to scalar registers.
__device__ inline double uniform_d(double x) {
  return __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(x)),
                          __builtin_amdgcn_readfirstlane(__double2loint(x)));
}
__device__ inline float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// ---------------------------------------------------------------------------
// Greedy team barrier (T = 0): a device-scope counter, reset by the last
// member to leave.

struct Barrier {
  uint32_t* ctr;
  uint32_t target;
  int W;
  uint32_t* status;
  uint64_t wait_ticks;
  int* s_dead;
};

// False (for the whole workgroup) when a wait of this member gave up.
__device__ bool barrier_sync(Barrier& b) {
  __syncthreads();
  if (b.W > 1) {
    b.target += uint32_t(b.W);
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(b.ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      // Poll with relaxed loads (an acquire load invalidates the XCD's L2 on
      // every poll, evicting the other teams' rows); one acquire fence after.
      while (__hip_atomic_load(b.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < b.target &&
             keep_waiting(t0, b.wait_ticks, b.status, b.s_dead)) {
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
  }
  return !*reinterpret_cast<volatile int*>(b.s_dead);
}

// No member waits after this point, so the reset cannot strand anyone.
__device__ void barrier_exit(Barrier& b) {
  __syncthreads();
  if (b.W > 1 && threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(b.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == b.target + uint32_t(b.W) - 1u)
      __hip_atomic_store(b.ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Block reductions (fixed order: wave shuffles, then waves in index order).

// Lane exchanges by ds_swizzle xor patterns (within 32 lanes; the pattern
// is an immediate, so no lane-address registers stay live), the two halves
// joined through readlane (the result is wave-uniform).
template <int M>
__device__ inline int swz_i(int x) {
  return __builtin_amdgcn_ds_swizzle(x, 0x1F | (M << 10));
}
template <int M>
__device__ inline float swz(float x) {
  return __int_as_float(swz_i<M>(__float_as_int(x)));
}
template <int M>
__device__ inline double swz(double x) {
  return __hiloint2double(swz_i<M>(__double2hiint(x)), swz_i<M>(__double2loint(x)));
}
__device__ inline double lane_d(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                          __builtin_amdgcn_readlane(__double2loint(x), l));
}
__device__ inline float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Row (16-lane) reductions by DPP moves, which are VALU operations: xor 1
// and xor 2 by quad permutes, then the half-row and row mirrors. Every
// step combines two values that all lanes of the group then share
// (addition and max are commutative), so every lane of a row ends with the
// same result, in an order fixed by the lane layout alone.
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline double dpp_d(double v) {
  return __hiloint2double(__builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false),
                          __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ inline double row_sum(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  return v;
}
__device__ inline float row_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

// Wave-wide, wave-uniform results: the four rows joined in row order.
__device__ inline double wave_sum(double v) {
  v = row_sum(v);
  return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}
__device__ inline float wave_max(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ inline double block_sum(double v, double* sh) {
  v = wave_sum(v);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < kWaves; ++w) tot += sh[w];
  __syncthreads();
  return tot;
}

// Block-wide maxima of two values; every thread returns them.
__device__ inline void block_max2(float& a, float& b, float* shf) {
  float A = wave_max(a), Bm = wave_max(b);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    shf[wave] = A;
    shf[kWaves + wave] = Bm;
  }
  __syncthreads();
  A = shf[0];
  Bm = shf[kWaves];
  for (int w = 1; w < kWaves; ++w) {
    A = fmaxf(A, shf[w]);
    Bm = fmaxf(Bm, shf[kWaves + w]);
  }
  __syncthreads();
  a = A;
  b = Bm;
}

// Block-wide maxima (fp32 logits) and sums of exp(x/T - max/T) of both rows:
// the maxima first, then every thread's sums rescaled to them with one exp
// and added in a fixed order.
__device__ inline void block_ms2(float& mt, double& st, float& md, double& sd, double invT,
                                 double* sh, float* shf, const double* tbl) {
  float Mt = wave_max(mt), Md = wave_max(md);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    shf[wave] = Mt;
    shf[kWaves + wave] = Md;
  }
  __syncthreads();
  Mt = shf[0];
  Md = shf[kWaves];
  for (int w = 1; w < kWaves; ++w) {
    Mt = fmaxf(Mt, shf[w]);
    Md = fmaxf(Md, shf[kWaves + w]);
  }
  double vt = mt == -INFINITY ? 0.0 : st * exp_nonpos((double(mt) - double(Mt)) * invT, tbl);
  double vd = md == -INFINITY ? 0.0 : sd * exp_nonpos((double(md) - double(Md)) * invT, tbl);
  vt = wave_sum(vt);
  vd = wave_sum(vd);
  if ((threadIdx.x & 63) == 0) {
    sh[wave] = vt;
    sh[kWaves + wave] = vd;
  }
  __syncthreads();
  st = 0.0;
  sd = 0.0;
  for (int w = 0; w < kWaves; ++w) {
    st += sh[w];
    sd += sh[kWaves + w];
  }
  mt = Mt;
  md = Md;
}

// argmax with the lowest index on ties (a total order on (value, index),
// so any combination order gives the same result).
__device__ inline void am_combine(float& v, int& i, float v2, int i2) {
  const bool take = v2 > v || (v2 == v && i2 < i);
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// Block-wide argmax of per-thread (v, i); every thread returns it.
__device__ inline void block_argmax(float& v, int& i, float* shv, int* shi) {
  am_combine(v, i, dpp_f<kDppXor1>(v), dpp_i<kDppXor1>(i));
  am_combine(v, i, dpp_f<kDppXor2>(v), dpp_i<kDppXor2>(i));
  am_combine(v, i, dpp_f<kDppHalfMirror>(v), dpp_i<kDppHalfMirror>(i));
  am_combine(v, i, dpp_f<kDppMirror>(v), dpp_i<kDppMirror>(i));
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
  for (int l = 16; l < kWave; l += 16) am_combine(bv, bi, lane_f(v, l), __builtin_amdgcn_readlane(i, l));
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & 63) == 0) {
    shv[wave] = bv;
    shi[wave] = bi;
  }
  __syncthreads();
  v = shv[0];
  i = shi[0];
  for (int w = 1; w < kWaves; ++w) am_combine(v, i, shv[w], shi[w]);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Streaming vocabulary sweeps over [lo, hi) of one or two rows. Each step
// issues 8 independent loads per thread before using any of them; then
// f(t, d, y, valid) sees every element once (d = 0 when only one row is
// read). Indices past hi are clamped to a valid address and passed with
// valid = false, so the loop body never branches. lo is a multiple of 4 in
// the vectorised form (rows are 16-byte aligned when V % 4 == 0).
template <bool TWO, class F>
__device__ inline void sweep(const float* tr, const float* dr, int lo, int hi, bool vec4, F&& f) {
  constexpr int kUnroll = TWO ? 4 : 8;
  if (vec4) {
    const float4* t4 = reinterpret_cast<const float4*>(tr + lo);
    const float4* d4 = reinterpret_cast<const float4*>(dr + lo);
    const int n4 = (hi - lo) >> 2;
    for (int base = threadIdx.x; base < n4; base += kUnroll * kThreads) {
      float4 tv[kUnroll], dv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = min(base + u * kThreads, n4 - 1);
        tv[u] = t4[i];
        if (TWO) dv[u] = d4[i];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = base + u * kThreads;
        const bool ok = i < n4;
        const int y = lo + 4 * i;
        f(tv[u].x, TWO ? dv[u].x : 0.f, y, ok);
        f(tv[u].y, TWO ? dv[u].y : 0.f, y + 1, ok);
        f(tv[u].z, TWO ? dv[u].z : 0.f, y + 2, ok);
        f(tv[u].w, TWO ? dv[u].w : 0.f, y + 3, ok);
      }
    }
  } else {
    for (int base = lo + threadIdx.x; base < hi; base += kUnroll * kThreads) {
      float tv[kUnroll], dv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int y = min(base + u * kThreads, hi - 1);
        tv[u] = tr[y];
        if (TWO) dv[u] = dr[y];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int y = base + u * kThreads;
        f(tv[u], TWO ? dv[u] : 0.f, y, y < hi);
      }
    }
  }
}

// Residual weight max(p(y) - a q(y), 0) with p(y) = exp(t/T - Mt)/Zt and
// q(y) = exp(d/T - Md)/Zd (plain p(y) when a == 0; the draft row is then
// not needed).
struct Resid {
  double invT, Mt, invZt, Md, invZd, a;
  __device__ inline double p(float t, const double* tbl) const {
    return exp_nonpos(fma(double(t), invT, -Mt), tbl) * invZt;
  }
  __device__ inline double q(float d, const double* tbl) const {
    return exp_nonpos(fma(double(d), invT, -Md), tbl) * invZd;
  }
  __device__ inline double w(float t, float d, const double* tbl) const {
    const double r = p(t, tbl) - a * q(d, tbl);  // a == 0: plain p (d is not needed)
    return r > 0.0 ? r : 0.0;
  }
};

// Smallest y in [lo, hi) where the running sum of weights passes thr
// (ascending token id), searched by the whole block. Each wave owns a
// contiguous quarter of [lo, hi) and sums it in blocks of 64 x 8 tokens
// (8 loads per lane in flight); the quarter holding thr is then scanned
// block by block with an in-order prefix over the block's tokens. Falls
// back to the last token with positive weight. Result in *s_y.
__device__ __attribute__((noinline)) void slice_search(const float* tr, const float* dr, int lo, int hi, const Resid& R,
                             double thr, const double* tbl, double* sh, int* s_y) {
  constexpr int K = 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x / kWave;
  const int n = hi - lo;
  int per = (n + kWaves - 1) / kWaves;
  per = (per + 64 * K - 1) / (64 * K) * (64 * K);
  const int cb = min(hi, lo + wave * per), ce = min(hi, cb + per);
  // weights of block [base, base + 64K): element k of lane l is y = base + 64k + l
  auto block_w = [&](int base, double* w) {
    float tv[K], dv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int y = min(base + 64 * k + lane, hi - 1);
      tv[k] = tr[y];
      dv[k] = dr[y];
    }
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = base + 64 * k + lane < ce ? R.w(tv[k], dv[k], tbl) : 0.0;
  };
  double run = 0.0;
  for (int base = cb; base < ce; base += 64 * K) {
    double w[K];
    block_w(base, w);
    double ls = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) ls += w[k];
    run += wave_sum(ls);
  }
  if (lane == 0) sh[wave] = run;
  __syncthreads();
  int fw = -1, last_w = -1;
  double pre = 0.0, fpre = 0.0, last_pre = 0.0;
  for (int w = 0; w < kWaves; ++w) {
    const double cw = sh[w];
    if (cw > 0.0) {
      last_w = w;
      last_pre = pre;
    }
    if (fw < 0 && pre <= thr && thr < pre + cw) {
      fw = w;
      fpre = pre;
    }
    pre += cw;
  }
  const bool past_end = fw < 0;  // rounding put thr past the end
  if (past_end) {
    fw = last_w;
    fpre = last_pre;
  }
  __syncthreads();
  if (wave == fw) {
    const double local = thr - fpre;
    double acc = 0.0;
    int found = -1, last_pos = -1;
    for (int base = cb; base < ce && found < 0; base += 64 * K) {
      double w[K];
      block_w(base, w);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const unsigned long long posmask = __ballot(w[k] > 0.0);
        if (posmask) last_pos = base + 64 * k + 63 - __clzll(posmask);
        double incl = w[k];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(incl, off, kWave);
          if (lane >= off) incl += o;
        }
        const unsigned long long hit = __ballot(!past_end && acc + incl > local && w[k] > 0.0);
        if (found < 0 && hit) found = base + 64 * k + __ffsll(static_cast<long long>(hit)) - 1;
        acc += __shfl(incl, 63, kWave);
      }
    }
    if (found < 0) found = last_pos;
    if (lane == 0) *s_y = found < 0 ? lo : found;
  }
  if (fw < 0 && threadIdx.x == 0) *s_y = lo;
  __syncthreads();
}

// Parent and token arrays of one request: staged in LDS when they fit,
// else read from global memory (each access names its memory, so neither
// goes through generic addressing).
struct Parents {
  const int* g;
  const int* s;
  const int* gtok;
  const int* stok;
  bool lds;
  __device__ inline int operator[](int i) const {
    if (lds) return s[i];
    return g[i];
  }
  __device__ inline int tok(int i) const {
    if (lds) return stok[i];
    return gtok[i];
  }
};

// Next child of v after row `after` (children in ascending row = draw
// order), found by wave 0 with a ballot; -1 when none. Broadcast via LDS.
__device__ int next_child(const Parents& par, int N, int v, int after, int* s_c) {
  if (threadIdx.x < kWave) {
    int found = -1;
    for (int base = after + 1; base < N && found < 0; base += kWave) {
      const int i = base + threadIdx.x;
      const unsigned long long m = __ballot(i < N && par[i] == v);
      if (m) found = base + __ffsll(static_cast<long long>(m)) - 1;
    }
    if (threadIdx.x == 0) *s_c = found;
  }
  __syncthreads();
  const int c = __builtin_amdgcn_readfirstlane(*s_c);
  __syncthreads();
  return c;
}

// ---------------------------------------------------------------------------
// The T > 0 walk.

struct WalkLds {
  double* tbl;        // 2^(j/64)
  double* tblz;       // 2^(j/256)
  double* sh;         // [2 * kWaves]
  float* shf;         // [2 * kWaves]
  double* s_slice;    // [kMaxTeam] slice sums of the last pass
  uint32_t* s_words;  // [kMaxTeam * 6] gathered exchange words
  int* s_kid;         // [kKids]
  float* s_kt;        // [kKids] target logit of the child token
  float* s_kd;        // [kKids] draft logit of the child token
  float* s_ku;        // [kKids] acceptance uniform of the child
  int* s_nk;          // children of the visited node (kKids + 1: more follow)
  int* s_int;
  float4* s_res;      // [2 rows][kLdsCh][kThreads] LDS-resident chunks
  double* s_draw;     // [kResCh * kWaves + kWaves] chunk and wave sums of the draw
};

// 16-byte load of lane offset voff (bytes) from [base, base + bytes) through
// a raw buffer resource: reads at or past the end return 0 without touching
// memory (gfx9 resource word 3).
__device__ inline float4 load4_bounded(const float* base, int bytes, int voff) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
  const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0));
  return make_float4(v.x, v.y, v.z, v.w);
}

// The same into LDS (each lane's 16 bytes at lds + 16 * lane; lds is the
// wave's base). Completion is counted by vmcnt like any load.
__device__ inline void load4_bounded_lds(const float* base, int bytes, int voff, float4* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// The compiler does not order LDS reads after buffer-to-LDS loads: wait for
// every outstanding load, as a memory barrier.
__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Member's part of the visited node's rows when resident: nch chunks of
// kThreads float4 (1024 logits) of both rows, chunk u < kRegCh in t[u],
// d[u], the rest in LDS. Only the row's last chunk can be partial; its
// missing elements read as -inf, whose exp term is exactly 0 (z is -inf,
// or NaN when the thread's maximum is -inf too, and the clamp in exp_z
// maps both to its floor).
template <bool RES>
struct Slice {
  float4 t[RES ? kRegCh : 1], d[RES ? kRegCh : 1];
};


template <bool RES>
__device__ __attribute__((always_inline)) inline void walk(
    const SampleParams& p, Team& tm, int nbeg, int N, const Parents& par,
    double invT, int lo, int hi, int nch, bool vec4, const WalkLds& L) {
  const int V = p.V;
  const int member = tm.member;
  const int lane = threadIdx.x & 63;
  const double A = invT * kZScale;  // z = (t/T - M/T) * 256/ln2 = fma(t, A, -M * A)
  Slice<RES> S;
  // Flags: member 0 alone writes them (initial values here, accepted nodes
  // later, in program order). next_token is written once per node at the
  // end (the stop node by the member that draws it, the rest by member 0).
  if (member == 0)
    for (int i = threadIdx.x; i < N; i += kThreads) p.flag[nbeg + i] = i == 0 ? 1 : 0;

  // Chunk u of the resident slice (RES only), past-the-slice lanes of the
  // row's last chunk as -inf. With chk, the loaded values (0 past the
  // slice) also go into the non-finite check: t * 0 is 0 for finite t.
  const int n4m = (hi - lo) >> 2;
  auto chunk = [&](int u, float4& a, float4& b, float* chk) __attribute__((always_inline)) {
    if constexpr (RES) {
      if (u < kRegCh) {
        a = S.t[u];
        b = S.d[u];
      } else {
        if (u == kRegCh) wait_loads();
        a = L.s_res[(u - kRegCh) * kThreads + threadIdx.x];
        b = L.s_res[(kLdsCh + u - kRegCh) * kThreads + threadIdx.x];
      }
      if (chk) {
        float c = *chk;
        c = fmaf(a.x, 0.f, fmaf(a.y, 0.f, fmaf(a.z, 0.f, fmaf(a.w, 0.f, c))));
        c = fmaf(b.x, 0.f, fmaf(b.y, 0.f, fmaf(b.z, 0.f, fmaf(b.w, 0.f, c))));
        *chk = c;
      }
      if ((u + 1) * kThreads > n4m && int(threadIdx.x) + u * kThreads >= n4m) {
        a = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        b = a;
      }
    }
  };

  // Stored exps (after a visit's stats pass): registers or LDS, no mask
  // (masked elements were stored as 0).
  auto stored = [&](int u, float4& a, float4& b) __attribute__((always_inline)) {
    if constexpr (RES) {
      if (u < kRegCh) {
        a = S.t[u];
        b = S.d[u];
      } else {
        a = L.s_res[(u - kRegCh) * kThreads + threadIdx.x];
        b = L.s_res[(kLdsCh + u - kRegCh) * kThreads + threadIdx.x];
      }
    }
  };
  auto put = [&](int u, float4 a, float4 b) __attribute__((always_inline)) {
    if constexpr (RES) {
      if (u < kRegCh) {
        S.t[u] = a;
        S.d[u] = b;
      } else {
        L.s_res[(u - kRegCh) * kThreads + threadIdx.x] = a;
        L.s_res[(kLdsCh + u - kRegCh) * kThreads + threadIdx.x] = b;
      }
    }
  };
  float mm_t = -INFINITY, mm_d = -INFINITY;  // the member's maxima of the visited rows

  // Inverse-CDF draw inside this member's resident slice (stored exps):
  // the smallest token whose running weight w = max(ct p~ - cb q~, 0) passes
  // thr, in token order (chunk u, thread t, element e); past the end (only
  // through rounding) the last token with weight. Result in *L.s_int.
  auto resident_draw = [&](double thr, double ct, double cb) __attribute__((always_inline)) {
    const int wave = threadIdx.x / kWave;
    auto weights = [&](int u, double (&w)[4]) __attribute__((always_inline)) {
      float4 a, b;
      stored(u, a, b);
      const float pa[4] = {a.x, a.y, a.z, a.w}, qb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double x = fma(-cb, double(qb[e]), ct * double(pa[e]));
        w[e] = x > 0.0 ? x : 0.0;
      }
    };
    if (threadIdx.x == 0) *L.s_int = -1;
#pragma unroll
    for (int u = 0; u < kResCh; ++u) {
      if (u < nch) {
        double w[4];
        weights(u, w);
        const double t = wave_sum((w[0] + w[1]) + (w[2] + w[3]));
        if (lane == 0) L.s_draw[u * kWaves + wave] = t;
      }
    }
    __syncthreads();
    int uc = -1, ulast = -1;
    double pre = 0.0, base = 0.0, lastbase = 0.0;
    for (int u = 0; u < nch; ++u) {
      double cu = 0.0;
      for (int w = 0; w < kWaves; ++w) cu += L.s_draw[u * kWaves + w];
      if (cu > 0.0) {
        ulast = u;
        lastbase = pre;
      }
      if (uc < 0 && pre <= thr && thr < pre + cu) {
        uc = u;
        base = pre;
      }
      pre += cu;
    }
    const bool past = uc < 0;
    if (past) {
      uc = ulast;
      base = lastbase;
    }
    if (uc >= 0) {
      // chunk uc, chosen by a uniform branch (a run-time index into the
      // register-resident slice would move the slice to scratch memory)
      double w[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int u = 0; u < kResCh; ++u)
        if (u == uc) weights(u, w);
      const double ts = (w[0] + w[1]) + (w[2] + w[3]);
      double inc = ts;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
      }
      if (lane == kWave - 1) L.s_draw[kResCh * kWaves + wave] = inc;
      __syncthreads();
      double woff = 0.0;
      for (int w2 = 0; w2 < wave; ++w2) woff += L.s_draw[kResCh * kWaves + w2];
      double c = base + woff + inc - ts;
      const int y0 = lo + uc * 4 * kThreads + 4 * int(threadIdx.x);
      if (!past && ts > 0.0 && c <= thr && thr < c + ts) {
        int y = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (y < 0 && w[e] > 0.0 && c <= thr && thr < c + w[e]) y = e;
          c += w[e];
        }
        if (y < 0) {  // rounding between the thread's sum and its parts: its last token with weight
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (w[e] > 0.0) y = e;
        }
        *L.s_int = y0 + y;
      }
      __syncthreads();
      if (*L.s_int < 0) {  // past the end, or missed by rounding: the last token with weight
        int last = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (w[e] > 0.0) last = y0 + e;
        if (last >= 0) atomicMax(L.s_int, last);
      }
      __syncthreads();
    }
    if (threadIdx.x == 0 && *L.s_int < 0) *L.s_int = lo;  // no mass (not reachable with finite logits)
    __syncthreads();
  };

  int v = 0;
  for (int depth_guard = 0; depth_guard <= N; ++depth_guard) {
    const float* trow = p.t + size_t(nbeg + v) * V;
    const float* drow = p.d + size_t(nbeg + v) * V;

    // Children of v (ascending rows, the first kKids) and their values, by
    // wave 0, after its slice loads are issued (they are needed only once
    // the stats exchange is done).
    float kt = 0.f, kd = 0.f, ku = 0.f;
    int nk = 0;
    auto kids = [&]() __attribute__((always_inline)) {
      if (threadIdx.x < kWave) {
        int cnt = 0;
        for (int base = v + 1; base < N && cnt <= kKids; base += kWave) {
          const int i = base + lane;
          const bool is = i < N && par[i] == v;
          const unsigned long long m = __ballot(is);
          const int pos = cnt + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
          if (is && pos < kKids) L.s_kid[pos] = i;
          cnt += __popcll(m);
        }
        nk = min(cnt, kKids + 1);
        if (lane < min(cnt, kKids)) {
          const int c = L.s_kid[lane];  // written above by this wave
          int x = par.tok(c);
          if (x < 0 || x >= V) {
            raise_status(p.status, TV_DEV_SHAPE);
            x = 0;
          }
          kt = trow[x];
          kd = drow[x];
          ku = p.uniforms[2 * size_t(nbeg + c)];
        }
      }
    };

    // Stats pass: per-thread (max, sum exp) of t/T and d/T over the slice.
    float mt = -INFINITY, md = -INFINITY;
    double st = 0.0, sd = 0.0;
    bool bad = false;
    if constexpr (RES) {
      // Every load of the slice in flight at once, chunk u through its own
      // bounded resource (reads past the slice return 0; they are masked or
      // skipped).
      const int voff = int(threadIdx.x) * 16;
      const int wbase = int(threadIdx.x) & ~(kWave - 1);
#pragma unroll
      for (int u = 0; u < kResCh; ++u) {
        const int nb = max(0, 4 * (hi - lo) - u * 16 * kThreads);
        if (u < kRegCh) {
          S.t[u] = load4_bounded(trow + lo + u * 4 * kThreads, nb, voff);
          S.d[u] = load4_bounded(drow + lo + u * 4 * kThreads, nb, voff);
        } else {
          load4_bounded_lds(trow + lo + u * 4 * kThreads, nb, voff, L.s_res + (u - kRegCh) * kThreads + wbase);
          load4_bounded_lds(drow + lo + u * 4 * kThreads, nb, voff,
                            L.s_res + (kLdsCh + u - kRegCh) * kThreads + wbase);
        }
      }
      kids();
      // Pass 1: the member's maxima of both rows (and the non-finite check).
      float chk = 0.f;
      float gt = -INFINITY, gd = -INFINITY;
#pragma unroll
      for (int u = 0; u < kResCh; ++u) {
        if (u < nch) {
          float4 a, b;
          chunk(u, a, b, &chk);
          gt = fmaxf(fmaxf(gt, fmaxf(a.x, a.y)), fmaxf(a.z, a.w));
          gd = fmaxf(fmaxf(gd, fmaxf(b.x, b.y)), fmaxf(b.z, b.w));
        }
      }
      block_max2(gt, gd, L.shf);
      mm_t = gt;
      mm_d = gd;
      // Pass 2: every element's exp relative to the member's maxima, kept in
      // place of its logit (the residual passes of this visit reuse it) and
      // summed in fp64. z = (x - M) / T in log2 units, formed by one fp64 fma.
      const double A2 = invT * kLog2E;
      const double bt2 = mm_t == -INFINITY ? 0.0 : -double(mm_t) * A2;
      const double bd2 = mm_d == -INFINITY ? 0.0 : -double(mm_d) * A2;
#pragma unroll
      for (int u = 0; u < kResCh; ++u) {
        if (u < nch) {
          float4 a, b;
          chunk(u, a, b, nullptr);
          a = opaque(a);
          b = opaque(b);
          a = make_float4(exp2_split(fma(double(a.x), A2, bt2)), exp2_split(fma(double(a.y), A2, bt2)),
                          exp2_split(fma(double(a.z), A2, bt2)), exp2_split(fma(double(a.w), A2, bt2)));
          b = make_float4(exp2_split(fma(double(b.x), A2, bd2)), exp2_split(fma(double(b.y), A2, bd2)),
                          exp2_split(fma(double(b.z), A2, bd2)), exp2_split(fma(double(b.w), A2, bd2)));
          st = opaque(st + ((double(a.x) + double(a.y)) + (double(a.z) + double(a.w))));
          sd = opaque(sd + ((double(b.x) + double(b.y)) + (double(b.z) + double(b.w))));
          put(u, a, b);
        }
      }
      mt = mm_t;
      md = mm_d;
      bad = !(chk == 0.f);
    } else {
      kids();
      // Streamed: the running maxima rise element by element.
      sweep<true>(trow, drow, lo, hi, vec4, [&](float t, float d, int, bool ok) {
        bad |= ok && (!isfinite(t) || !isfinite(d));
        if (!ok) return;
        if (t > mt) {
          st = mt == -INFINITY ? 0.0 : st * exp_nonpos((double(mt) - double(t)) * invT, L.tbl);
          mt = t;
        }
        if (d > md) {
          sd = md == -INFINITY ? 0.0 : sd * exp_nonpos((double(md) - double(d)) * invT, L.tbl);
          md = d;
        }
        st += exp_z(fma(double(t), A, -double(mt) * A), L.tblz);
        sd += exp_z(fma(double(d), A, -double(md) * A), L.tblz);
      });
    }
    if (bad) raise_status(p.status, TV_DEV_LOGITS);
    if (threadIdx.x < kWave) {
      L.s_kt[lane] = kt;
      L.s_kd[lane] = kd;
      L.s_ku[lane] = ku;
      if (lane == 0) *L.s_nk = nk;
    }
    if constexpr (RES) {
      // every thread's sums are relative to the member's maxima already
      double vt = wave_sum(st), vd = wave_sum(sd);
      const int wave = threadIdx.x / kWave;
      if (lane == 0) {
        L.sh[wave] = vt;
        L.sh[kWaves + wave] = vd;
      }
      __syncthreads();
      st = (L.sh[0] + L.sh[1]) + (L.sh[2] + L.sh[3]);
      sd = (L.sh[kWaves] + L.sh[kWaves + 1]) + (L.sh[kWaves + 2] + L.sh[kWaves + 3]);
    } else {
      block_ms2(mt, st, md, sd, invT, L.sh, L.shf, L.tbl);
    }
    if (threadIdx.x < 6) {
      const uint32_t k = threadIdx.x;
      const double dv = k < 3 ? st : sd;
      const float fv = k < 3 ? mt : md;
      const uint32_t j = k % 3;
      const uint32_t wv = j == 0 ? __float_as_uint(fv)
                                 : (j == 1 ? uint32_t(__double2loint(dv)) : uint32_t(__double2hiint(dv)));
      ll_put(tm, int(k), wv, L.s_words);
    }
    if (!ll_gather(tm, 6, L.s_words)) return;  // a wait gave up (status bit set)
    const int nkk = __builtin_amdgcn_readfirstlane(*L.s_nk);

    // Team totals, member w in lane w of the first row of every wave (the
    // same reduction in every wave and every member): the maxima, then each
    // member's sums rescaled to them.
    const bool mem_lane = lane < tm.W;
    const float mw = mem_lane ? __uint_as_float(L.s_words[6 * lane]) : -INFINITY;
    const float dw = mem_lane ? __uint_as_float(L.s_words[6 * lane + 3]) : -INFINITY;
    const float Mt32 = lane_f(row_max(mw), 0), Md32 = lane_f(row_max(dw), 0);
    const double et = mw == -INFINITY ? 0.0
                                      : words_to_double(L.s_words[6 * lane + 1], L.s_words[6 * lane + 2]) *
                                            exp_nonpos((double(mw) - double(Mt32)) * invT, L.tbl);
    const double ed = dw == -INFINITY ? 0.0
                                      : words_to_double(L.s_words[6 * lane + 4], L.s_words[6 * lane + 5]) *
                                            exp_nonpos((double(dw) - double(Md32)) * invT, L.tbl);
    const double Zt = lane_d(row_sum(et), 0), Zd = lane_d(row_sum(ed), 0);
    // Slice sums of p (for a draw at a leaf).
    if (threadIdx.x < tm.W) L.s_slice[threadIdx.x] = et / Zt;
    const double Mt = double(Mt32) * invT, Md = double(Md32) * invT;

    Resid R{invT, Mt, 1.0 / Zt, Md, 1.0 / Zd, 0.0};
    double B = 1.0, Sq = 1.0;
    int accepted = -1;
    int k = 0;
    // Every thread takes the same decisions; readfirstlane lets the compiler
    // see that, so the walk's control flow and row addresses stay scalar.
    int c = nkk > 0 ? __builtin_amdgcn_readfirstlane(L.s_kid[0]) : -1;
    while (c >= 0) {
      float tx, dx, uc;
      if (k < kKids) {
        tx = uniform_f(L.s_kt[k]);
        dx = uniform_f(L.s_kd[k]);
        uc = uniform_f(L.s_ku[k]);
      } else {
        int x = par.tok(c);
        if (x < 0 || x >= V) {
          raise_status(p.status, TV_DEV_SHAPE);
          x = 0;
        }
        tx = trow[x];
        dx = drow[x];
        uc = p.uniforms[2 * size_t(nbeg + c)];
      }
      const double px = R.p(tx, L.tbl);
      const double qx = R.q(dx, L.tbl);
      double pj = px - R.a * qx;
      pj = (pj > 0.0 ? pj : 0.0) / B;
      const double qj = qx / Sq;
      const double ratio = qj > 0.0 ? pj / qj : (pj > 0.0 ? INFINITY : 0.0);
      if (__builtin_amdgcn_readfirstlane(int(double(uc) < ratio))) {
        accepted = c;
        if (member == 0 && threadIdx.x == 0) p.flag[nbeg + c] = 1;
        break;
      }
      // Rejected: one residual pass at a' = a + B/S.
      const double an = R.a + B / Sq;
      double part = 0.0;
      if constexpr (RES) {
        // p(y) = stored_t * ct, q(y) = stored_d * cq with the member's scale
        // factors (its maxima against the team's, over Z).
        const double ct = mm_t == -INFINITY ? 0.0
                                            : exp_nonpos((double(mm_t) - double(Mt32)) * invT, L.tbl) * R.invZt;
        const double cb = mm_d == -INFINITY ? 0.0
                                            : -an * exp_nonpos((double(mm_d) - double(Md32)) * invT, L.tbl) * R.invZd;
        auto wsum = [&](float pt, float qd) __attribute__((always_inline)) {
          const double w = fma(cb, double(qd), ct * double(pt));
          return w > 0.0 ? w : 0.0;
        };
#pragma unroll
        for (int u = 0; u < kResCh; ++u) {
          if (u < nch) {
            float4 a, b;
            stored(u, a, b);
            a = opaque(a);
            b = opaque(b);
            part = opaque(part + (wsum(a.x, b.x) + wsum(a.y, b.y)));
            part = opaque(part + (wsum(a.z, b.z) + wsum(a.w, b.w)));
          }
        }
      } else {
        Resid Rn = R;
        Rn.a = an;
        sweep<true>(trow, drow, lo, hi, vec4, [&](float t, float d, int, bool ok) {
          const double w = Rn.w(t, d, L.tbl);
          part += ok ? w : 0.0;
        });
      }
      part = block_sum(part, L.sh);
      if (threadIdx.x < 2)
        ll_put(tm, int(threadIdx.x),
               threadIdx.x == 0 ? uint32_t(__double2loint(part)) : uint32_t(__double2hiint(part)), L.s_words);
      if (!ll_gather(tm, 2, L.s_words)) return;
      const double pw = lane < tm.W ? words_to_double(L.s_words[2 * lane], L.s_words[2 * lane + 1]) : 0.0;
      const double F = lane_d(row_sum(pw), 0);
      if (F > 0.0) {
        R.a = an;
        B = F;
        if (threadIdx.x < tm.W) L.s_slice[threadIdx.x] = pw;
      }
      if (!p.with_replacement) Sq -= qx;
      ++k;
      if (k < min(nkk, kKids))
        c = __builtin_amdgcn_readfirstlane(L.s_kid[k]);
      else if (nkk > kKids)
        c = next_child(par, N, v, c, L.s_int);  // past the listed children
      else
        c = -1;
    }
    __syncthreads();  // s_slice written; this visit's lists no longer read
    if (accepted >= 0) {
      v = __builtin_amdgcn_readfirstlane(accepted);  // uniform: row addresses stay scalar
      continue;
    }

    // Stop at v: inverse-CDF draw from the residual (p itself when a == 0).
    // The slice sums of the last pass locate the slice; its owner scans it.
    const double u = double(p.uniforms[2 * size_t(nbeg + v) + 1]);
    double total = 0.0;
    for (int w = 0; w < tm.W; ++w) total += L.s_slice[w];
    const double thr = u * total;
    int finder = -1, last_w = -1;
    double pre = 0.0, base_w = 0.0, last_pre = 0.0;
    for (int w = 0; w < tm.W; ++w) {
      const double sw = L.s_slice[w];
      if (sw > 0.0) {
        last_w = w;
        last_pre = pre;
      }
      if (finder < 0 && pre <= thr && thr < pre + sw) {
        finder = w;
        base_w = pre;
      }
      pre += sw;
    }
    if (finder < 0) {
      finder = last_w;
      base_w = last_pre;
    }
    finder = __builtin_amdgcn_readfirstlane(finder);
    if (finder == member) {
      if constexpr (RES) {
        // The member's stored exps give the residual weights of its slice:
        // chunk sums locate the 1024-token chunk, a block-wide prefix over
        // its threads the thread, the thread's four tokens the token.
        const double ct = mm_t == -INFINITY ? 0.0
                                            : exp_nonpos((double(mm_t) - double(Mt32)) * invT, L.tbl) * R.invZt;
        const double cb = mm_d == -INFINITY || R.a == 0.0
                              ? 0.0
                              : R.a * exp_nonpos((double(mm_d) - double(Md32)) * invT, L.tbl) * R.invZd;
        resident_draw(thr - base_w, ct, cb);
      } else {
        slice_search(trow, drow, lo, hi, R, thr - base_w, L.tbl, L.sh, L.s_int);
      }
      if (threadIdx.x == 0) p.next_token[nbeg + v] = *L.s_int;
    } else if (finder < 0 && member == 0 && threadIdx.x == 0) {
      p.next_token[nbeg + v] = 0;  // no mass in any slice (not reachable with finite logits)
    }
    if (member == 0)
      for (int i = threadIdx.x; i < N; i += kThreads)
        if (i != v) p.next_token[nbeg + i] = -1;
    return;
  }
}

// ---------------------------------------------------------------------------
// Greedy argmax of every row (T = 0) for 4-aligned rows. The request's
// N x C units (row, chunk of 1024 logits) are split evenly over the team in
// row-major order and streamed kGreedyBatch units at a time (one 16-byte
// load per thread per unit, all of a batch in flight). A row held whole by
// one member is written directly; a row shared by neighbouring members is
// finished by the member holding its first unit, from the partial argmaxes
// every member publishes for its first and last row.
constexpr int kGreedyBatch = 24;

__device__ __attribute__((always_inline)) inline void greedy_rows(const SampleParams& p, Team& tm, int nbeg,
                                                                  int N, float* shv, int* shi,
                                                                  uint32_t* s_words) {
  const int V = p.V;
  const int C = (V + 4 * kThreads - 1) / (4 * kThreads);
  const long long U = (long long)N * C;
  const int W = tm.W;
  auto start = [&](int m) { return U * m / W; };
  const long long g0 = start(tm.member), g1 = start(tm.member + 1);
  const int row_first = int(g0 / C), row_last = g0 < g1 ? int((g1 - 1) / C) : -1;
  const bool first_shared = g0 < g1 && g0 % C != 0;
  const bool last_shared = g0 < g1 && g1 % C != 0;
  float fv = -INFINITY, lv = -INFINITY;  // member partials of the shared first / last row
  int fi = 0x7fffffff, li = 0x7fffffff;

  // Four running argmaxes per thread, one per float4 lane (independent
  // dependency chains); bi[e] holds the chunk offset of the lane's float4,
  // so the token is bi[e] + e. Merged with lowest-index ties at row end.
  float bv[4];
  int bi[4];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bv[e] = -INFINITY;
      bi[e] = 0x7fffffff;
    }
  };
  reset();
  float chk = 0.f;  // t * 0 is 0 for finite t, NaN otherwise
  int cur = row_first;
  auto finish = [&](int row) __attribute__((always_inline)) {
    float v = bv[0];
    int i = bi[0];
#pragma unroll
    for (int e = 1; e < 4; ++e) am_combine(v, i, bv[e], bi[e] == 0x7fffffff ? bi[e] : bi[e] + e);
    block_argmax(v, i, shv, shi);
    const bool is_first = row == row_first && first_shared, is_last = row == row_last && last_shared;
    if (is_first) {
      fv = v;
      fi = i;
    }
    if (is_last) {
      lv = v;
      li = i;
    }
    if (!is_first && !is_last && threadIdx.x == 0)
      __hip_atomic_store(p.next_token + nbeg + row, i == 0x7fffffff ? 0 : i, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    reset();
  };

  const int voff = int(threadIdx.x) * 16;
  const int tail = V - 4 * kThreads * (C - 1);  // logits in a row's last chunk
  for (long long u0 = g0; u0 < g1; u0 += kGreedyBatch) {
    const int rem = g1 - u0 < kGreedyBatch ? int(g1 - u0) : kGreedyBatch;  // units of this batch
    const int row0 = int(u0 / C), ch0 = int(u0 - (long long)row0 * C);
    int ch = ch0;
    const float* rp = p.t + size_t(nbeg + row0) * V;
    float4 buf[kGreedyBatch];
#pragma unroll
    for (int j = 0; j < kGreedyBatch; ++j) {  // past the batch: an empty range, no memory access
      const int nb = j < rem ? 4 * (ch == C - 1 ? tail : 4 * kThreads) : 0;
      buf[j] = load4_bounded(rp + 4 * kThreads * ch, nb, voff);
      if (++ch == C) {
        ch = 0;
        rp += V;
      }
    }
    int row = row0;
    ch = ch0;
#pragma unroll
    for (int j = 0; j < kGreedyBatch; ++j) {
      if (j < rem) {
        if (row != cur) {
          finish(cur);
          cur = row;
        }
        const int y0 = 4 * kThreads * ch + 4 * int(threadIdx.x);
        float a[4] = {buf[j].x, buf[j].y, buf[j].z, buf[j].w};
        chk = fmaf(a[0], 0.f, fmaf(a[1], 0.f, fmaf(a[2], 0.f, fmaf(a[3], 0.f, chk))));
        if (ch == C - 1 && tail < 4 * kThreads) {  // the row's partial last chunk
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = 4 * int(threadIdx.x) + e < tail ? a[e] : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool take = a[e] > bv[e];  // ascending offsets per lane: ties keep the first
          bv[e] = take ? a[e] : bv[e];
          bi[e] = take ? y0 : bi[e];
        }
      }
      if (++ch == C) {
        ch = 0;
        ++row;
      }
    }
  }
  const bool bad = !(chk == 0.f);
  if (g0 < g1) finish(cur);
  if (bad) raise_status(p.status, TV_DEV_LOGITS);

  // Shared rows, from the partials of the members covering them (the
  // match-flag phase reads next_token only after the team barrier, whose
  // release/acquire orders every member's stores before it).
  if (W > 1) {
    if (threadIdx.x < 4) {
      const uint32_t w4[4] = {__float_as_uint(fv), uint32_t(fi), __float_as_uint(lv), uint32_t(li)};
      uint32_t wv = w4[0];
#pragma unroll
      for (int k = 1; k < 4; ++k) wv = threadIdx.x == k ? w4[k] : wv;
      ll_put(tm, int(threadIdx.x), wv, s_words);
    }
    if (!ll_gather(tm, 4, s_words)) return;
    if (last_shared && g0 <= (long long)row_last * C && threadIdx.x == 0) {
      // This member holds the first unit of its last row: fold in the later
      // members that start inside that row.
      float v = lv;
      int i = li;
      for (int m = tm.member + 1; m < W; ++m) {
        const long long s0 = start(m), s1 = start(m + 1);
        if (s0 >= (long long)(row_last + 1) * C) break;
        if (s0 < s1) am_combine(v, i, __uint_as_float(s_words[4 * m]), int(s_words[4 * m + 1]));
      }
      __hip_atomic_store(p.next_token + nbeg + row_last, i == 0x7fffffff ? 0 : i, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Greedy exact match along the walk only (T = 0, TV_GREEDY_PATH). From the
// root, the team takes the argmax of the visited node's target row (each
// member over its slice [lo, hi), lowest index on ties, then one exchange of
// (value, index) per member), tests every child against it, moves to the
// first matching child in draw order and stops at a node with none. Member
// 0 writes every output: first the request's defaults (root flagged, the
// rest 0, next tokens -1), then each visit's next token and the flags of the
// children it tested; its default stores precede its first visit's loads,
// so they have completed before any of its later stores is issued.
constexpr int kPathLoads = 12;  // 16-byte loads per thread in flight per step

__device__ __attribute__((always_inline)) inline void greedy_path(const SampleParams& p, Team& tm, int nbeg,
                                                                  int N, const Parents& par, int lo, int hi,
                                                                  bool vec4, float* shv, int* shi,
                                                                  uint32_t* s_words, int* s_c) {
  const int V = p.V;
  const bool writer = tm.member == 0;
  if (writer)
    for (int i = threadIdx.x; i < N; i += kThreads) {
      p.flag[nbeg + i] = i == 0 ? 1 : 0;
      p.next_token[nbeg + i] = -1;
    }
  float chk = 0.f;  // t * 0 is 0 for finite t, NaN otherwise
  int v = 0;
  while (true) {
    const float* row = p.t + size_t(nbeg + v) * V;
    // Four running argmaxes per thread (one per float4 lane), each seeing
    // ascending offsets, so ties keep the first; bi[e] + e is the token.
    float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int bi[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
    if (vec4) {
      const int n4 = (hi - lo) >> 2;  // float4 of this member's slice (V % 4 == 0)
      const float* base = row + lo;
      for (int b0 = 0; b0 < n4; b0 += kPathLoads * kThreads) {
        float4 buf[kPathLoads];
#pragma unroll
        for (int u = 0; u < kPathLoads; ++u) {  // past the slice: 0, no memory access
          const int s0 = b0 + u * kThreads;      // the block's first float4
          const int in = min(kThreads, max(0, n4 - s0));
          buf[u] = load4_bounded(base + 4 * size_t(s0), 16 * in, 16 * int(threadIdx.x));
        }
#pragma unroll
        for (int u = 0; u < kPathLoads; ++u) {
          const int i4 = b0 + u * kThreads + int(threadIdx.x);
          const bool ok = i4 < n4;
          const int y0 = lo + 4 * i4;
          const float a[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            chk = fmaf(a[e], 0.f, chk);
            const bool take = ok && a[e] > bv[e];
            bv[e] = take ? a[e] : bv[e];
            bi[e] = take ? y0 : bi[e];
          }
        }
      }
    } else {
      sweep<false>(row, row, lo, hi, false, [&](float t, float, int y, bool ok) {
        chk = ok ? fmaf(t, 0.f, chk) : chk;
        const bool take = ok && t > bv[0];  // ascending y per thread: ties keep the first
        bv[0] = take ? t : bv[0];
        bi[0] = take ? y : bi[0];
      });
    }
    float mv = bv[0];
    int mi = bi[0];
    if (vec4) {
#pragma unroll
      for (int e = 1; e < 4; ++e) am_combine(mv, mi, bv[e], bi[e] == 0x7fffffff ? bi[e] : bi[e] + e);
    }
    block_argmax(mv, mi, shv, shi);
    if (threadIdx.x < 2) ll_put(tm, int(threadIdx.x), threadIdx.x == 0 ? __float_as_uint(mv) : uint32_t(mi), s_words);
    if (!ll_gather(tm, 2, s_words)) return;
    float gv = -INFINITY;
    int gi = 0x7fffffff;
    for (int m = 0; m < tm.W; ++m) am_combine(gv, gi, __uint_as_float(s_words[2 * m]), int(s_words[2 * m + 1]));
    const int y = __builtin_amdgcn_readfirstlane(gi == 0x7fffffff ? 0 : gi);
    // Every child of v is tested (member 0 writes the flags); the first
    // match in draw order is the next node. The first visit scans every
    // row, so member 0 checks every parent link then.
    if (threadIdx.x < kWave) {
      int found = -1;
      for (int b = v + 1; b < N; b += kWave) {
        const int i = b + int(threadIdx.x);
        const int pi = i < N ? par[i] : v - 1;
        if (writer && v == 0 && i < N && (pi < 0 || pi >= i)) raise_status(p.status, TV_DEV_TREE);
        const bool child = i < N && pi == v;
        const bool match = child && par.tok(i) == y;
        if (writer && child) p.flag[nbeg + i] = match ? 1 : 0;
        const unsigned long long m = __ballot(match);
        if (m && found < 0) found = b + __ffsll(static_cast<long long>(m)) - 1;
      }
      if (threadIdx.x == 0) {
        *s_c = found;
        if (writer) p.next_token[nbeg + v] = y;
      }
    }
    __syncthreads();
    const int c = __builtin_amdgcn_readfirstlane(*s_c);
    __syncthreads();  // s_c is rewritten at the next visit
    if (c < 0) break;
    v = c;
  }
  if (!(chk == 0.f)) raise_status(p.status, TV_DEV_LOGITS);
}

__global__ __launch_bounds__(kThreads, 4) void sample_kernel(SampleParams p) {
  __shared__ double tbl[64];
  __shared__ double tblz[kZTable];
  __shared__ double sh[2 * kWaves];
  __shared__ float shf[2 * kWaves];
  __shared__ double s_slice[kMaxTeam];
  __shared__ uint32_t s_words[6 * kMaxTeam];
  __shared__ int s_kid[kKids];
  __shared__ float s_kt[kKids], s_kd[kKids], s_ku[kKids];
  __shared__ int s_par[kParLds], s_tok[kParLds];
  __shared__ float4 s_res[2 * kLdsCh * kThreads];
  __shared__ double s_draw[kResCh * kWaves + kWaves];
  __shared__ float shv[kWaves];
  __shared__ int shi[kWaves];
  __shared__ int s_nk, s_int, s_dead;

  // Team placement: block b runs on XCD b % 8; the W members of a team are
  // consecutive slots of one XCD.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int r = (slot / p.W) * 8 + xcd;
  const int member = slot - (slot / p.W) * p.W;
  if (r >= p.B) return;  // padding block: belongs to no team

  if (threadIdx.x == 0) s_dead = 0;
  for (int j = threadIdx.x; j < 64; j += kThreads) tbl[j] = exp2(double(j) / 64.0);
  for (int j = threadIdx.x; j < kZTable; j += kThreads) tblz[j] = exp2(double(j) / double(kZTable));

  // Per-request values are wave-uniform: keep them (and the row addresses
  // derived from them) in scalar registers.
  const int nbeg = __builtin_amdgcn_readfirstlane(p.node_indptr[r]);
  const int N = __builtin_amdgcn_readfirstlane(p.node_indptr[r + 1]) - nbeg;
  const int V = p.V;
  const float T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.temperature[r])));
  if (N <= 0 || N > p.max_nodes) {
    if (N != 0 && threadIdx.x == 0 && member == 0) raise_status(p.status, TV_DEV_SHAPE);
    return;  // uniform for the whole team: nobody waits on anybody
  }
  // Parents in LDS when they fit (child scans then cost no global round trip).
  const Parents par{p.parent + nbeg, s_par, p.tokens + nbeg, s_tok, N <= kParLds};
  if (par.lds)
    for (int i = threadIdx.x; i < N; i += kThreads) {
      s_par[i] = par.g[i];
      s_tok[i] = par.gtok[i];
    }
  const bool vec4 = (V & 3) == 0;
  __syncthreads();  // tables and parents ready

  if (!(T >= 0.f) || (T > 0.f && p.d == nullptr)) {
    if (member == 0) {
      if (threadIdx.x == 0) raise_status(p.status, TV_DEV_LOGITS);
      for (int i = threadIdx.x; i < N; i += kThreads) {
        p.flag[nbeg + i] = i == 0 ? 1 : 0;
        p.next_token[nbeg + i] = -1;
      }
    }
    return;
  }

  Team tm;
  char* const rq = p.req + size_t(r) * kReqBytes;
  uint32_t* const seq_word = reinterpret_cast<uint32_t*>(rq + 4);
  tm.slots = reinterpret_cast<uint64_t*>(rq + kReqSlotsOff);
  tm.seq = *seq_word;
  tm.phase = 0;
  tm.W = p.W;
  tm.member = member;
  tm.status = p.status;
  tm.wait_ticks = p.wait_ticks;
  tm.s_dead = &s_dead;

  // Member slices: vectorised rows are split in chunks of 1024 logits
  // (kThreads float4), member m taking chunks [m C / W, (m + 1) C / W) of the
  // C in a row, so only the row's last chunk is ever partial.
  int lo, hi, nch = 0;
  const int C = (V + 4 * kThreads - 1) / (4 * kThreads);
  if (vec4) {
    const int c0 = member * C / p.W, c1 = (member + 1) * C / p.W;
    nch = c1 - c0;
    lo = min(V, 4 * kThreads * c0);
    hi = min(V, 4 * kThreads * c1);
  } else {
    const int slice = (V + p.W - 1) / p.W;
    lo = min(V, member * slice);
    hi = min(V, lo + slice);
  }

  if (T == 0.f && p.greedy_path) {
    greedy_path(p, tm, nbeg, N, par, lo, hi, vec4, shv, shi, s_words, &s_int);
    // the request's sequence moves past every tag this call used (as below)
    if (member == 0 && threadIdx.x == 0 && p.W > 1)
      __hip_atomic_store(seq_word, tm.seq + uint32_t(tm.phase), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (T == 0.f) {
    Barrier bar{reinterpret_cast<uint32_t*>(rq), 0u, p.W, p.status, p.wait_ticks, &s_dead};
    // Greedy exact match: argmax of every row, then the match flags.
    if (vec4) greedy_rows(p, tm, nbeg, N, shv, shi, s_words);
    for (int i = member; !vec4 && i < N; i += p.W) {
      const float* row = p.t + size_t(nbeg + i) * V;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      bool bad = false;
      sweep<false>(row, row, 0, V, vec4, [&](float t, float, int y, bool ok) {
        bad |= ok && !isfinite(t);
        const bool take = ok && t > bv;  // ascending y per thread: ties keep the first
        bv = take ? t : bv;
        bi = take ? y : bi;
      });
      if (bad) raise_status(p.status, TV_DEV_LOGITS);
      am_combine(bv, bi, swz<1>(bv), swz_i<1>(bi));
      am_combine(bv, bi, swz<2>(bv), swz_i<2>(bi));
      am_combine(bv, bi, swz<4>(bv), swz_i<4>(bi));
      am_combine(bv, bi, swz<8>(bv), swz_i<8>(bi));
      am_combine(bv, bi, swz<16>(bv), swz_i<16>(bi));
      am_combine(bv, bi, lane_f(bv, 32), __builtin_amdgcn_readlane(bi, 32));
      const int wave = threadIdx.x / kWave;
      if ((threadIdx.x & 63) == 0) {
        shv[wave] = bv;
        shi[wave] = bi;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        float v = -INFINITY;
        int idx = 0x7fffffff;
        for (int w = 0; w < kWaves; ++w) am_combine(v, idx, shv[w], shi[w]);
        // device-coherent store: other members read it after the barrier
        __hip_atomic_store(p.next_token + nbeg + i, idx == 0x7fffffff ? 0 : idx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }
    if (!barrier_sync(bar)) return;  // a wait gave up (status bit set)
    for (int i = member * kThreads + threadIdx.x; i < N; i += p.W * kThreads) {
      int8_t f = 0;
      if (i == 0) {
        f = 1;
      } else {
        const int pi = par[i];
        if (pi < 0 || pi >= i) {
          raise_status(p.status, TV_DEV_TREE);
        } else {
          const int ntp = __hip_atomic_load(p.next_token + nbeg + pi, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
          f = (par.tok(i) == ntp) ? 1 : 0;
        }
      }
      p.flag[nbeg + i] = f;
    }
    barrier_exit(bar);
    if (member == 0 && threadIdx.x == 0 && p.W > 1 && tm.phase > 0)
      __hip_atomic_store(seq_word, tm.seq + uint32_t(tm.phase), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // Sampled walk (T > 0).
  const double invT = 1.0 / double(T);
  WalkLds L{tbl, tblz, sh, shf, s_slice, s_words, s_kid, s_kt, s_kd, s_ku, &s_nk, &s_int, s_res, s_draw};
  const bool resident = vec4 && (C + p.W - 1) / p.W <= kResCh;  // the same for every member
  if (resident)
    walk<true>(p, tm, nbeg, N, par, invT, lo, hi, nch, vec4, L);
  else
    walk<false>(p, tm, nbeg, N, par, invT, lo, hi, nch, vec4, L);
  // The request's sequence moves past every tag this call used. Every
  // member read the old value before its first publish, and this store
  // follows member 0's last gather, which saw every member's last publish.
  if (member == 0 && threadIdx.x == 0 && p.W > 1)
    __hip_atomic_store(seq_word, tm.seq + uint32_t(tm.phase), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

bool plan_sample(const tv_sample_desc& d, SamplePlan* out) {
  if (d.batch < 1 || d.vocab < 1 || d.max_nodes < 1 || d.max_nodes > 65536 || d.max_depth < 0)
    return false;
  if (d.rule != TV_RULE_WITHOUT_REPLACEMENT && d.rule != TV_RULE_WITH_REPLACEMENT) return false;
  if (d.greedy != TV_GREEDY_EVERY_NODE && d.greedy != TV_GREEDY_PATH) return false;
  SamplePlan pl{};
  pl.threads = kThreads;
  pl.off_req = kHeaderBytes;
  pl.total_bytes = kHeaderBytes + size_t(d.batch) * kReqBytes;
  *out = pl;
  return true;
}

namespace {

// Launch facts of one device (resident sample_kernel workgroups per CU, CU
// count), looked up on the first call made with that device current and
// kept per device; concurrent first calls compute the same values.
constexpr int kMaxDevices = 64;
std::atomic<int> g_blocks_per_cu[kMaxDevices];
std::atomic<int> g_num_cus[kMaxDevices];

hipError_t device_facts(int* blocks_per_cu, int* num_cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int b = g_blocks_per_cu[dev].load(std::memory_order_acquire);
    const int c = g_num_cus[dev].load(std::memory_order_acquire);
    if (b > 0 && c > 0) {
      *blocks_per_cu = b;
      *num_cus = c;
      return hipSuccess;
    }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int per = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(sample_kernel),
                                                   kThreads, 0);
  if (e != hipSuccess) return e;
  if (per < 1 || cus < 1) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kMaxDevices) {
    g_blocks_per_cu[dev].store(per, std::memory_order_release);
    g_num_cus[dev].store(cus, std::memory_order_release);
  }
  *blocks_per_cu = per;
  *num_cus = cus;
  return hipSuccess;
}

}  // namespace

// Limit of every bounded wait (the sampler's team exchanges and barrier,
// TreeSpark's grid barrier): kWaitTicksDefault, or TREEVERIFY_TEAM_WAIT_US
// microseconds when that variable is set (a diagnostic: read at every
// launch, so a test can force waits to give up from the host).
uint64_t wait_ticks() {
  const char* v = getenv("TREEVERIFY_TEAM_WAIT_US");
  if (!v || !*v) return kWaitTicksDefault;
  char* end = nullptr;
  const unsigned long long us = strtoull(v, &end, 10);
  return (end && *end == 0) ? uint64_t(us) * 100ull : kWaitTicksDefault;
}

// One launch of the walk with its status word and per-request blocks given.
hipError_t launch_sample_core(const tv_sample_desc& d, const SampleArgs& a, uint32_t* status,
                              char* req, hipStream_t stream) {
  int per = 0, cus = 0;
  hipError_t e = device_facts(&per, &cus);
  if (e != hipSuccess) return e;
  // Team size: as many workgroups per request as the device keeps resident
  // at once, at most kMaxTeam; a team lives on one XCD. The grid never
  // exceeds that residency, so on a device that runs nothing else every
  // team is resident together. The launch is a plain one (a cooperative
  // launch costs about 17 us more here); a team whose members are held back
  // by other work longer than the wait limit reports TV_DEV_TIMEOUT instead
  // of waiting on.
  const long resident = long(per) * cus;
  int W = int(resident / ((d.batch + 7) / 8 * 8));
  if (W > kMaxTeam) W = kMaxTeam;
  if (W < 1) W = 1;
  auto grid_for = [&](int w) { return long((d.batch + 7) / 8) * 8 * w; };
  while (W > 1 && grid_for(W) > resident) --W;
  SampleParams p{};
  p.t = a.target;
  p.d = a.draft;
  p.tokens = a.tokens;
  p.node_indptr = a.node_indptr;
  p.parent = a.parent;
  p.temperature = a.temperature;
  p.uniforms = a.uniforms;
  p.flag = a.flag;
  p.next_token = a.next_token;
  p.status = status;
  p.req = req;
  p.B = d.batch;
  p.V = d.vocab;
  p.W = W;
  p.max_nodes = d.max_nodes;
  p.with_replacement = d.rule == TV_RULE_WITH_REPLACEMENT;
  p.greedy_path = d.greedy == TV_GREEDY_PATH;
  p.wait_ticks = wait_ticks();
  const dim3 grid(unsigned(grid_for(W))), block(kThreads);
  hipLaunchKernelGGL(sample_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_sample(const tv_sample_desc& d, const SamplePlan& pl, const SampleArgs& a,
                         hipStream_t stream) {
  char* ws = static_cast<char*>(a.workspace);
  return launch_sample_core(d, a, reinterpret_cast<uint32_t*>(ws), ws + pl.off_req, stream);
}

}  // namespace tv
