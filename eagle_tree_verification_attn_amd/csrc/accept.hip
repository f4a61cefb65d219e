// Speculative accept / reject over the verified draft trees.
//
// [Spec-decoding lesson] "Exactness rule": accept draft token x iff
// r < p(x)/q(x); otherwise sample the replacement from (p - q)+ normalised and
// stop; greedy: accept iff argmax(p) == x, else emit argmax(p).  "Concept": if
// every draft token is accepted, one bonus token is sampled from p at the
// last position.  [EAGLE article] sec. 1.3 "Verification", Figure 1-6: with k
// candidates at one position a rejection moves on to the next candidate with
// the corrected distribution; only when all k are rejected is the correction
// sampled; the rule is applied recursively at every node of the tree.
//
// One kernel, k_accept_walk: groups of `nchunk` workgroups, all resident, a
// group walking one sequence at a time with workgroup w owning vocabulary
// chunk w.  At each node the walk visits, every workgroup reads its chunk of
// the node's logits row once into LDS and the group combines the chunk
// statistics (max, sum exp((z - max) / tau), or the lowest-index argmax for
// greedy rows, and a non-finite flag) through one barrier; rows of nodes the
// walk never reaches are not read.  All workgroups take the same scalar
// decisions from the same exchanged values; each rejection needs the mass of
// the new residual, summed over the vocabulary and exchanged the same way.
//
// Residual bookkeeping.  With p the target distribution of the node, q its
// draft distribution, and siblings x_1..x_i rejected, the current target is
//     P(v) = max(0, p(v) - A q(v)) / Wn,
// where A starts at 0 and grows by Wn * c_i at rejection i, Wn is the mass
// sum_v max(0, p(v) - A q(v)) for the current A (1 before any rejection), and
// c_i = 1 / (1 - sum_{l<i} q(x_l)) when siblings were drawn without
// replacement (the proposal of sibling i is q restricted to the untried tokens
// and renormalised), c_i = 1 when drawn i.i.d.  This equals normalising
// max(0, P - q_i) after every rejection, because each rejected token already
// has residual 0 and the nested maxima of the decreasing p - A q collapse; it
// costs one pass over the node's (logits, q) row per rejection.
#include "sv_internal.h"

#include <math.h>
#include <stdlib.h>

namespace sv {

constexpr int kAccThreads = 512;
constexpr int kMaxChunk = 16384;  // vocabulary entries one walk workgroup caches in LDS
constexpr float kLog2e = 1.4426950408889634f;

struct WalkParams {
  const int32_t* parent;
  const int32_t* num_nodes;
  const int32_t* tokens;
  const void* logits;
  const float* q_probs;
  const float* temperature;
  const float* u_accept;
  const float* u_sample;
  int32_t* status;
  int32_t* out_tokens;
  int32_t* out_nodes;
  int32_t* out_count;
  int32_t* out_passes;
  uint64_t* xchg;  // [ngroups][2][nchunk][kXWords] exchange words, zeroed by k_accept_clear
  uint64_t wait_ticks;  // bound of one exchange wait, in ticks of the 100 MHz real-time counter
  int B, T_max, V, nchunk, chunk, ngroups;
  int bf16, sibling_mode;
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline float load_logit(const void* base, size_t idx, int bf16) {
  if (bf16) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(base)[idx];
    return __uint_as_float((uint32_t)h << 16);
  }
  return reinterpret_cast<const float*>(base)[idx];
}

__device__ inline bool greedy_temp(float tau) { return !(tau > 0.f); }

// ----------------------------------------------------------------------------
// chunk loads
// ----------------------------------------------------------------------------
// A workgroup reads its vocabulary chunk of one row with every load issued
// before any arithmetic: thread t takes kBatch groups of 8 entries at
// c0 + 8 t + 8 q * threads (q < kBatch); addresses past the chunk end are
// clamped to the chunk start, so every load is unconditional.
constexpr int kBatch = kMaxChunk / (kAccThreads * 8);
static_assert(kAccThreads * 8 * kBatch == kMaxChunk, "chunk covered by one batch");
static_assert(kAccThreads >= kMaxT, "one tree position per thread");
constexpr int kSeg = kMaxChunk / kAccThreads;   // chunk entries per thread in the draw
static_assert(kSeg % 16 == 0 && kSeg <= 64, "draw segments: whole quads, at most one entry per lane in the final scan");
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16, int H>
__device__ inline float elem8(const u32x4 (&w)[H], int e) {
  if (BF16) {
    const uint32_t x = w[0][e >> 1];
    return (e & 1) ? bf16_hi(x) : bf16_lo(x);
  }
  return __uint_as_float(w[e >> 2][e & 3]);
}

// ----------------------------------------------------------------------------
// wave-wide reductions and scans on DPP lane moves and the gfx950 row swaps
// (no LDS round trips); every lane of the wave must be active
// ----------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
// the two values of a lane's row pair (rows 0/1, 2/3), then of its half pair
__device__ inline void swap16(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
__device__ inline void swap32(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
// Butterflies within each row of 16 (quad_perm [1,0,3,2], [2,3,0,1], the
// half-row mirror, the row mirror), then across rows: every lane gets the
// wave's total.
__device__ inline float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = __uint_as_float(a) + __uint_as_float(b);
  swap32(__float_as_uint(v), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = fmaxf(__uint_as_float(a), __uint_as_float(b));
  swap32(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ inline int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  uint32_t a, b;
  swap16((uint32_t)v, a, b);
  v = min((int)a, (int)b);
  swap32((uint32_t)v, a, b);
  return min((int)a, (int)b);
}
// Inclusive prefix sum over the wave in lane order: within rows of 16 by
// shifted adds (row_shr 1, 2, 4, 8; lanes shifted in from outside the row
// add 0), then each row adds the totals of the rows before it.
__device__ inline float wave_incl_scan(float x) {
  const int lane = threadIdx.x & 63;
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const int row = lane >> 4;
  const float before = row == 0 ? 0.f : (row == 1 ? t0 : (row == 2 ? t0 + t1 : (t0 + t1) + t2));
  return before + x;
}

// Raw 16-byte words of the logits: one per group of 8 (bf16) or two (fp32).
// Without VEC (row not 16-byte aligned or V % 8 != 0) entries are read one by
// one, entries past the chunk end again clamped.
template <bool BF16, bool VEC, int RH = BF16 ? 1 : 2>
__device__ inline void load_raw(const void* rowp, int c0, int c1, u32x4 (&raw)[kBatch][RH]) {
  const uint16_t* rowh = reinterpret_cast<const uint16_t*>(rowp);
  const float* rowf = reinterpret_cast<const float*>(rowp);
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    const int i = c0 + (threadIdx.x + q * kAccThreads) * 8;
    const int ic = i < c1 ? i : c0;
    if (VEC) {
      if (BF16) {
        raw[q][0] = *reinterpret_cast<const u32x4*>(rowh + ic);
      } else {
        raw[q][0] = *reinterpret_cast<const u32x4*>(rowf + ic);
        raw[q][RH - 1] = *reinterpret_cast<const u32x4*>(rowf + ic + 4);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = (ic + e < c1) ? ic + e : c0;
        if (BF16) {
          const uint32_t h = rowh[v];
          raw[q][0][e >> 1] = (e & 1) ? (raw[q][0][e >> 1] | (h << 16)) : h;
        } else {
          raw[q][(e >> 2) % RH][e & 3] = __float_as_uint(rowf[v]);
        }
      }
    }
  }
}

// Statistics of this workgroup's chunk of one logits row, from its words
// already loaded by load_raw:
//   stochastic rows: (m_c, s_c) = (chunk max, sum of e(v) = 2^((z(v) - m_c) k)),
//                    and e(v) stored in LDS at ec[v - c0];
//   greedy rows:     (m_c, i_c) = (chunk max, its lowest index);
//   flag: a NaN or an infinity anywhere in the chunk.
// The result is returned to thread 0 as (m, s or index bits, flag, 0).
template <bool BF16, bool VEC, int RH = BF16 ? 1 : 2>
__device__ float4 chunk_stats(const u32x4 (&raw)[kBatch][RH], int c0, int c1, bool greedy, float k, float* ec,
                              float* red_m, float* red_s, int* red_i, int* red_f) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // Non-finite test on the raw words: an all-ones exponent field plus one
  // carries into the field's top bit.  Clamped loads repeat real entries of
  // this chunk, so they change neither this flag nor the maximum.
  uint32_t badbits = 0u;
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    if (BF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) badbits |= ((raw[q][0][j] & 0x7F807F80u) + 0x00800080u) & 0x80008000u;
    } else {
#pragma unroll
      for (int h = 0; h < RH; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) badbits |= ((raw[q][h][j] & 0x7F800000u) + 0x00800000u) & 0x80000000u;
    }
  }
  const bool any_bad = __any(badbits != 0u);
  float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
  if (greedy) {
    // (max, lowest index): per thread, per wave, then over the waves
    float m = -INFINITY;
    int am = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = c0 + (tid + q * kAccThreads) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = elem8<BF16, RH>(raw[q], e);
        if (i + e < c1 && x > m) { m = x; am = i + e; }   // strict: lowest index per thread
      }
    }
    {
      const float M = wave_max(m);
      am = wave_min_i(m == M ? am : 0x7FFFFFFF);   // the lowest index holding the maximum
      m = M;
    }
    __syncthreads();   // the previous user of red_* is done
    if (lane == 0) { red_m[wv] = m; red_i[wv] = am; red_f[wv] = any_bad; }
    __syncthreads();
    if (tid == 0) {
      float M = red_m[0];
      int I = red_i[0], F = red_f[0];
      for (int w = 1; w < kAccThreads / 64; ++w) {
        F |= red_f[w];
        if (red_m[w] > M || (red_m[w] == M && red_i[w] < I)) { M = red_m[w]; I = red_i[w]; }
      }
      out = make_float4(M, __int_as_float(I), __int_as_float(F), 0.f);
    }
    return out;
  }
  // stochastic: the chunk max first, then e(v) and its sum against it (the
  // clamped entries repeat real ones, so they leave the max unchanged)
  float m = -INFINITY;
#pragma unroll
  for (int q = 0; q < kBatch; ++q)
#pragma unroll
    for (int e = 0; e < 8; e += 2) m = fmaxf(m, fmaxf(elem8<BF16, RH>(raw[q], e), elem8<BF16, RH>(raw[q], e + 1)));
  m = wave_max(m);
  __syncthreads();   // the previous user of red_* is done
  if (lane == 0) { red_m[wv] = m; red_f[wv] = any_bad; }
  __syncthreads();
  float mc = red_m[0];
#pragma unroll
  for (int w = 1; w < kAccThreads / 64; ++w) mc = fmaxf(mc, red_m[w]);
  const float mk = mc * k;
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    const int i = c0 + (tid + q * kAccThreads) * 8;
    float ev[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ev[e] = __builtin_amdgcn_exp2f(fmaf(elem8<BF16, RH>(raw[q], e), k, -mk));
    if (VEC) {
      // chunk ends are multiples of 8: a group of 8 is in the chunk or is a
      // clamped repeat of entries [c0, c0 + 8), which rewrites them unchanged
      const float gs = ((ev[0] + ev[1]) + (ev[2] + ev[3])) + ((ev[4] + ev[5]) + (ev[6] + ev[7]));
      s += i < c1 ? gs : 0.f;
      const int ic = i < c1 ? i : c0;
      *reinterpret_cast<f32x4*>(ec + (ic - c0)) = f32x4{ev[0], ev[1], ev[2], ev[3]};
      *reinterpret_cast<f32x4*>(ec + (ic - c0) + 4) = f32x4{ev[4], ev[5], ev[6], ev[7]};
    } else if (i < c1) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (i + e < c1) {
          s += ev[e];
          ec[i - c0 + e] = ev[e];
        }
    }
  }
  s = wave_sum(s);
  if (lane == 0) red_s[wv] = s;
  __syncthreads();
  if (tid == 0) {
    float S = 0.f;
    int F = 0;
    for (int w = 0; w < kAccThreads / 64; ++w) { S += red_s[w]; F |= red_f[w]; }
    out = make_float4(mc, S, __int_as_float(F), 0.f);
  }
  return out;
}

// q(v) for v in [c0, c1) of one draft row into qc[v - c0], loads batched.
template <bool VEC>
__device__ inline void load_q_chunk(const float* qrow, int c0, int c1, float* qc) {
  const int tid = threadIdx.x;
  if (VEC) {
    u32x4 a[kBatch], b[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = c0 + (tid + q * kAccThreads) * 8;
      const int ic = i < c1 ? i : c0;
      a[q] = *reinterpret_cast<const u32x4*>(qrow + ic);
      b[q] = *reinterpret_cast<const u32x4*>(qrow + ic + 4);
    }
    // unconditional stores: a clamped group rewrites entries [0, 8) of the
    // chunk with the values they already hold
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const int i = c0 + (tid + q * kAccThreads) * 8;
      const int ic = i < c1 ? i : c0;
      *reinterpret_cast<u32x4*>(qc + (ic - c0)) = a[q];
      *reinterpret_cast<u32x4*>(qc + (ic - c0) + 4) = b[q];
    }
  } else {
    for (int i = c0 + tid; i < c1; i += kAccThreads) qc[i - c0] = qrow[i];
  }
}

__global__ void k_accept_clear(uint64_t* words, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) words[i] = 0ull;
}

// ----------------------------------------------------------------------------
// k_accept_walk
// ----------------------------------------------------------------------------
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kAccThreads / 64; ++w) t += red[w];
  return t;
}

// Scan over the workgroup in thread order: inclusive and exclusive prefix of
// v for this thread (the exclusive value of thread t equals, bit for bit, the
// inclusive value of thread t-1) and the workgroup total.
__device__ inline void block_scan(float v, float* red, float* incl, float* excl, float* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float x = wave_incl_scan(v);
  const float xprev = __shfl_up(x, 1);
  __syncthreads();
  if (lane == 63) red[wv] = x;
  __syncthreads();
  float before = 0.f;
  for (int w = 0; w < wv; ++w) before += red[w];
  float tot = 0.f;
  for (int w = 0; w < kAccThreads / 64; ++w) tot += red[w];
  *incl = before + x;
  *excl = lane == 0 ? before : before + xprev;
  *total = tot;
}

// Group exchange without a shared counter.  Each workgroup publishes up to
// kXWords values per exchange as 64-bit words (exchange number << 32 | value
// bits), each written by one atomic store, so a reader that sees the current
// exchange number in a word also sees that word's value.  Exchange e uses
// parity slot e % 2; a slot is rewritten at exchange e + 2, which no member
// reaches before every member has published e + 1, i.e. has finished
// reading e.  Every word is zeroed at the start of a call and exchange
// numbers start at 1, so words from earlier calls never match.
constexpr int kXWords = 3;
struct GroupXchg {
  uint64_t* words;  // this group's [2][nchunk][kXWords]
  int nchunk;
  int epoch;
  uint64_t wait_ticks;
  __device__ uint64_t* slot(int e) const { return words + (size_t)(e & 1) * nchunk * kXWords; }
  // Thread 0 publishes v[0..nv) for workgroup w; threads below nchunk * nv
  // each wait for one member's word and put its value in out[member * nv + j].
  // Returns false when a wait exceeded its bound (co-residency broken).
  __device__ bool exchange(int w, const float* v, int nv, float* out) {
    __shared__ int ok;
    ++epoch;
    uint64_t* sl = slot(epoch);
    const uint64_t tag = (uint64_t)(uint32_t)epoch << 32;
    if (threadIdx.x == 0) {
      ok = 1;
      for (int j = 0; j < nv; ++j)
        __hip_atomic_store(sl + (size_t)w * kXWords + j, tag | __float_as_uint(v[j]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < nchunk * nv) {
      const int m = t / nv, j = t % nv;
      uint64_t* wp = sl + (size_t)m * kXWords + j;
      uint64_t x = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!wait_for(wp, x)) ok = 0;
      out[t] = __uint_as_float((uint32_t)x);
    }
    __syncthreads();
    return ok != 0;
  }
  // Polls word wp (already loaded into x) until it carries the current
  // exchange number; false when the bound (real-time counter ticks) passes.
  __device__ bool wait_for(uint64_t* wp, uint64_t& x) const {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((x >> 32) != (uint64_t)(uint32_t)epoch) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) return false;
      x = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return true;
  }
  // One-sided exchange: member `from` publishes one value, only member 0
  // reads it (into *out).  Every member takes the exchange number, so the
  // group's numbering stays in step.  Returns false (in member 0) when the
  // wait exceeded its bound.  A slot is still rewritten only two exchanges
  // later, after a full exchange in between, so the parity rule holds.
  __device__ bool to_first(int w, int from, uint32_t v, uint32_t* out) {
    __shared__ int ok1;
    ++epoch;
    uint64_t* sl = slot(epoch);
    if (from == 0) {                     // member 0 has the value itself
      if (w == 0 && threadIdx.x == 0) *out = v;
      __syncthreads();
      return true;
    }
    const uint64_t tag = (uint64_t)(uint32_t)epoch << 32;
    if (w == from && threadIdx.x == 0)
      __hip_atomic_store(sl + (size_t)from * kXWords, tag | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (w == 0 && threadIdx.x == 0) {
      uint64_t* wp = sl + (size_t)from * kXWords;
      uint64_t x = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok1 = wait_for(wp, x) ? 1 : 0;
      *out = (uint32_t)x;
    }
    __syncthreads();
    return w != 0 || ok1 != 0;
  }
};

// Groups of `nchunk` workgroups, all resident at once (the grid is at most one
// workgroup per CU, checked on the host); a group walks one
// sequence at a time, workgroup w owning vocabulary chunk w.  All workgroups
// of a group take the same scalar decisions from the same exchanged values.
// At every node the walk visits, the group first forms the statistics of the
// node's row (one exchange); each rejection then needs the mass of the new
// residual over the vocabulary (one exchange each).  Only the rows of visited
// nodes are read.
// Children of the node being expanded, in increasing position: bit c of
// cm[n] is set iff parent[c] == n (positions below 256, words of 64).
// Returns the smallest child of n after position `after`, or -1.
__device__ inline int next_child(const uint64_t (*cm)[kMaxT / 64], int n, int after, int W) {
  int wd = (after + 1) >> 6;
  if (wd >= W) return -1;
  uint64_t m = cm[n][wd] & (~0ull << ((after + 1) & 63));
  while (true) {
    if (m) return wd * 64 + __ffsll((unsigned long long)m) - 1;
    if (++wd >= W) return -1;
    m = cm[n][wd];
  }
}


template <bool BF16, bool VEC>
__global__ __launch_bounds__(kAccThreads) void k_accept_walk(WalkParams p) {
  constexpr int RH = BF16 ? 1 : 2;
  // Per-sequence data gathered once into LDS, so the walk's scalar decisions
  // read LDS instead of chaining dependent global loads.
  __shared__ int tok_s[kMaxT];
  __shared__ int path_s[kMaxT];
  __shared__ float zx_s[kMaxT];   // logit of node c's token in its parent's row
  __shared__ float qx_s[kMaxT];   // q of node c's token in its parent's row
  __shared__ float ua_s[kMaxT];
  __shared__ float us_s[kMaxT];
  __shared__ uint64_t cm_s[kMaxT][kMaxT / 64];   // children of every node, as bit rows
  __shared__ float red[kAccThreads / 64];
  __shared__ float red_m[kAccThreads / 64], red_s[kAccThreads / 64];
  __shared__ int red_i[kAccThreads / 64], red_f[kAccThreads / 64];
  __shared__ float masses[64];
  __shared__ float xv[64 * kXWords];   // the group's exchanged values
  __shared__ float pubv[kXWords];
  __shared__ float bcast, m_b, ls_b, f_b, excl_b;
  __shared__ uint32_t tok_b;
  __shared__ int ibcast, ybcast, am_b, bad_b;
  __shared__ int flags_s;

  const int tid = threadIdx.x;
  const int grp = blockIdx.x / p.nchunk;
  const int w = blockIdx.x % p.nchunk;
  const int c0 = w * p.chunk;
  const int c1 = min(c0 + p.chunk, p.V);
  const bool wor = p.sibling_mode == SV_SIB_WITHOUT_REPLACEMENT;
  GroupXchg gx{p.xchg + (size_t)grp * 2 * p.nchunk * kXWords, p.nchunk, 0, p.wait_ticks};
  // this workgroup's chunk: e(v) = 2^((z(v) - m_c) k) of the visited node, then q
  extern __shared__ __align__(16) float cache_s[];
  float* pc = cache_s;
  float* qc = cache_s + p.chunk;
  const int len = c1 - c0;
  auto logits_row = [&](size_t row) {
    return BF16 ? (const void*)(reinterpret_cast<const uint16_t*>(p.logits) + row * p.V)
                : (const void*)(reinterpret_cast<const float*>(p.logits) + row * p.V);
  };

  for (int b = grp; b < p.B; b += p.ngroups) {
    const size_t rowbase = (size_t)b * p.T_max;
    // The root's row is read by every valid sequence: its chunk loads go out
    // first, and the tree is gathered while they are in flight.  (Row 0 of
    // every sequence lies inside the logits tensor, so the loads are in
    // bounds whatever the sequence's status.)
    u32x4 raw[kBatch][RH];
    load_raw<BF16, VEC>(logits_row(rowbase), c0, c1, raw);
    // The tree data of position tid goes out in the same round trip, before
    // the sequence's status and size are known (the arrays are [B][T_max],
    // so these loads are in bounds).
    int x_r = 0, par_r = -1;
    float ua_r = 0.f, us_r = 0.f;
    if (tid < p.T_max) {
      x_r = p.tokens[rowbase + tid];
      par_r = p.parent[rowbase + tid];
      ua_r = p.u_accept[rowbase + tid];
      us_r = p.u_sample[rowbase + tid];
    }
    int st = p.status[b];
    const int Tb = p.num_nodes[b];
    if (st == SV_TREE_OK && (Tb < 1 || Tb > p.T_max)) st = SV_TREE_E_COUNT;
    const int W = (Tb + 63) >> 6;
    const float tau = p.temperature[b];
    const bool greedy = greedy_temp(tau);
    const float k = greedy ? 0.f : kLog2e / tau;
    int32_t* onodes = p.out_nodes + (size_t)b * p.T_max;
    int32_t* otoks = p.out_tokens + (size_t)b * p.T_max;
    __syncthreads();
    if (tid == 0) flags_s = 0;
    if (st == SV_TREE_OK)
      for (int i = tid; i < Tb * (kMaxT / 64); i += kAccThreads) cm_s[i / (kMaxT / 64)][i % (kMaxT / 64)] = 0ull;
    __syncthreads();
    if (st == SV_TREE_OK) {
      // the tree (as child bit rows), tokens, uniforms.  A valid tree has
      // 0 <= parent[c] < c for 1 <= c < T_b.
      if (tid < Tb) {
        tok_s[tid] = x_r;
        ua_s[tid] = ua_r;
        us_s[tid] = us_r;
        if (tid > 0) {
          if (par_r >= 0 && par_r < tid)
            atomicOr(reinterpret_cast<unsigned long long*>(&cm_s[par_r][tid >> 6]), 1ull << (tid & 63));
          else atomicOr(&flags_s, 2);   // only a caller's own status could let such a tree through
          if (x_r < 0 || x_r >= p.V) atomicOr(&flags_s, 1);   // the root's token is not read
        }
      }
      __syncthreads();
      if (flags_s & 2) st = SV_TREE_E_PARENT;
      else if (flags_s & 1) st = SV_TREE_E_TOKEN;
      else if (!greedy && p.q_probs == nullptr) st = SV_TREE_E_NOQ;
    }
    // Each candidate's logit and draft probability in its parent's row (a
    // second, dependent round trip): the loads go out now and land in
    // registers; they are put in LDS after the root's statistics pass, which
    // covers their latency, and read only after the first exchange.
    const bool has_x = st == SV_TREE_OK && !greedy && tid >= 1 && tid < Tb;
    float zx_r = 0.f, qx_r = 0.f;
    if (has_x) {
      zx_r = load_logit(logits_row(rowbase + par_r), (size_t)x_r, BF16);
      qx_r = p.q_probs[(rowbase + par_r) * p.V + x_r];
    }
    bool x_pending = true;

    int n = 0, path_len = 0, passes = 0, emitted = -1, owner = -1;
    int raw_row = 0;   // the node whose chunk `raw` holds: the root's, loaded at the start
    bool sync_ok = true, nonfinite = false;
    while (st == SV_TREE_OK) {
      const float* qrow = greedy ? nullptr : p.q_probs + (rowbase + n) * p.V;
      // ---- statistics of node n's row: every chunk, one exchange
      if (raw_row != n) load_raw<BF16, VEC>(logits_row(rowbase + n), c0, c1, raw);
      {
        const float4 loc = chunk_stats<BF16, VEC>(raw, c0, c1, greedy, k, pc, red_m, red_s, red_i, red_f);
        if (x_pending) {   // visible after the exchange's barriers, before any test reads them
          if (has_x) {
            zx_s[tid] = zx_r;
            qx_s[tid] = qx_r;
          }
          x_pending = false;
        }
        if (tid == 0) { pubv[0] = loc.x; pubv[1] = loc.y; pubv[2] = loc.z; }
        if (!gx.exchange(w, pubv, 3, xv)) { sync_ok = false; break; }
        // The first child is the likeliest next node (tried first; in greedy
        // trees the drafter's best token): its chunk loads go out now, under
        // the combine and the acceptance test.  (After the exchange, so that
        // the exchange's polls, which complete in order with earlier loads,
        // do not wait for them.)
        raw_row = next_child(cm_s, n, n, W);
        if (raw_row >= 0) load_raw<BF16, VEC>(logits_row(rowbase + raw_row), c0, c1, raw);
        // combined over the chunks by the first wave, one lane per chunk
        if (tid < 64) {
          const bool live = tid < p.nchunk;
          const float mc = live ? xv[3 * tid] : -INFINITY;
          const float yc = live ? xv[3 * tid + 1] : 0.f;
          const float M = wave_max(mc);
          // greedy: the first chunk holding the maximum has the lowest index
          const uint64_t at_max = __ballot(live && mc == M);
          const int first = at_max ? (int)__ffsll((unsigned long long)at_max) - 1 : 0;
          const int I = __shfl(__float_as_int(yc), first);
          const bool F = __any(live && __float_as_int(xv[3 * tid + 2]) != 0);
          if (!greedy) {
            const float S = wave_sum(live ? yc * __builtin_amdgcn_exp2f((mc - M) * k) : 0.f);
            const float ls = __log2f(S);
            if (live) masses[tid] = yc * __builtin_amdgcn_exp2f((mc - M) * k - ls);
            // p(v) = e(v) f on this workgroup's chunk
            if (tid == w) f_b = __builtin_amdgcn_exp2f((mc - M) * k - ls);
            if (tid == 0) ls_b = ls;
          }
          if (tid == 0) {
            m_b = M;
            am_b = I;
            bad_b = F;
          }
        }
        __syncthreads();
      }
      if (bad_b) { nonfinite = true; break; }
      int acc = -1;
      if (greedy) {
        const int am = am_b;
        for (int c = next_child(cm_s, n, n, W); c >= 0; c = next_child(cm_s, n, c, W))
          if (tok_s[c] == am) { acc = c; break; }
        if (acc >= 0) {
          if (tid == 0) path_s[path_len] = acc;
          ++path_len;
          n = acc;
          continue;
        }
        emitted = am;
        owner = 0;
        break;
      }
      const float m = m_b, ls = ls_b, f = f_b;
      float A = 0.f, Wn = 1.f, rm = 0.f, Adraw = 0.f;
      bool have_q = false;
      const int first_child = next_child(cm_s, n, n, W);
      for (int c = first_child; c >= 0; c = next_child(cm_s, n, c, W)) {
        const float qx = qx_s[c];
        const float px = __builtin_amdgcn_exp2f(fmaf(zx_s[c] - m, k, -ls));
        const float Px = fmaxf(px - A * qx, 0.f) / Wn;
        const float ci = wor ? 1.f / (1.f - rm) : 1.f;
        const float qix = qx * ci;
        const float ratio = qix > 0.f ? Px / qix : (Px > 0.f ? INFINITY : 0.f);
        if (ua_s[c] < ratio) {
          acc = c;
          break;
        }
        // rejection: mass of the new residual over the whole vocabulary
        const float An = A + Wn * ci;
        if (!have_q) {
          load_q_chunk<VEC>(qrow, c0, c1, qc);
          __syncthreads();
          have_q = true;
        }
        // thread t sums entries 4 t + 4 kAccThreads j in four chains
        float pa[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kMaxChunk / (4 * kAccThreads); ++j) {
          const int i = tid * 4 + j * 4 * kAccThreads;
          if (i + 4 <= len) {
            const float4 pp = *reinterpret_cast<const float4*>(pc + i);
            const float4 qq = *reinterpret_cast<const float4*>(qc + i);
            pa[j & 3] += (fmaxf(fmaf(-An, qq.x, pp.x * f), 0.f) + fmaxf(fmaf(-An, qq.y, pp.y * f), 0.f)) +
                         (fmaxf(fmaf(-An, qq.z, pp.z * f), 0.f) + fmaxf(fmaf(-An, qq.w, pp.w * f), 0.f));
          } else if (i < len) {
            for (int e = i; e < len; ++e) pa[j & 3] += fmaxf(fmaf(-An, qc[e], pc[e] * f), 0.f);
          }
        }
        float part = (pa[0] + pa[1]) + (pa[2] + pa[3]);
        part = block_sum(part, red);
        if (tid == 0) pubv[0] = part;
        if (!gx.exchange(w, pubv, 1, xv)) { sync_ok = false; break; }
        if (tid < 64) {
          const bool live = tid < p.nchunk;
          const float v = live ? xv[tid] : 0.f;
          const float tot = wave_sum(v);
          if (tid == 0) bcast = tot;
          if (tot > 0.f && live) masses[tid] = v;
        }
        __syncthreads();
        const float Wsum = bcast;
        ++passes;
        if (Wsum > 0.f) {   // a zero residual (rounding only) keeps the previous target
          A = An;
          Wn = Wsum;
          Adraw = An;
        }
        rm += qx;
      }
      if (!sync_ok) break;
      if (acc >= 0) {
        if (tid == 0) path_s[path_len] = acc;
        ++path_len;
        n = acc;
        continue;
      }
      // draw at node n from P proportional to max(0, p - Adraw q) with u_sample[n]
      if (first_child < 0) ++passes;   // a leaf: the bonus draw reads the row once more
      float total = 0.f;
      for (int cc = 0; cc < p.nchunk; ++cc) total += masses[cc];
      const float target = us_s[n] * total;
      float cum = 0.f;
      owner = -1;
      int last_pos = -1;
      for (int cc = 0; cc < p.nchunk; ++cc) {
        if (masses[cc] > 0.f) {
          last_pos = cc;
          if (cum + masses[cc] > target) { owner = cc; break; }
          cum += masses[cc];
        }
      }
      const bool fallback = owner < 0;
      if (fallback) owner = last_pos < 0 ? 0 : last_pos;
      if (w == owner) {
        // residual entry i of the chunk (q is only needed after a rejection)
        auto resid = [&](int i) { return have_q ? fmaxf(fmaf(-Adraw, qc[i], pc[i] * f), 0.f) : pc[i] * f; };
        // thread t owns the kSeg entries [kSeg t, kSeg t + kSeg) of the chunk
        const int s0 = tid * kSeg;
        int y = -1;
        if (!fallback) {
          float va[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < kSeg / 4; ++j) {
            // segments lie 4 kSeg bytes apart: each thread starts at its own
            // quad, so the lanes of a bank row read different banks
            const int i = s0 + 4 * ((j + tid) & (kSeg / 4 - 1));
            if (i + 4 <= len) {
              const float4 pp = *reinterpret_cast<const float4*>(pc + i);
              if (have_q) {
                const float4 qq = *reinterpret_cast<const float4*>(qc + i);
                va[j & 3] += (fmaxf(fmaf(-Adraw, qq.x, pp.x * f), 0.f) + fmaxf(fmaf(-Adraw, qq.y, pp.y * f), 0.f)) +
                             (fmaxf(fmaf(-Adraw, qq.z, pp.z * f), 0.f) + fmaxf(fmaf(-Adraw, qq.w, pp.w * f), 0.f));
              } else {
                va[j & 3] += (pp.x * f + pp.y * f) + (pp.z * f + pp.w * f);
              }
            } else {
              for (int e = i; e < min(i + 4, len); ++e) va[j & 3] += resid(e);
            }
          }
          const float vs = (va[0] + va[1]) + (va[2] + va[3]);
          float incl, excl, tot;
          block_scan(vs, red, &incl, &excl, &tot);
          if (tid == 0) ibcast = 0x7FFFFFFF;
          __syncthreads();
          // the segment whose range of the cumulative mass holds the target
          if (cum + excl <= target && cum + incl > target) {
            atomicMin(&ibcast, tid);
            excl_b = excl;   // a single segment holds it (zero-mass segments are empty ranges)
          }
          __syncthreads();
          const int ts = ibcast;
          if (ts != 0x7FFFFFFF && tid < 64) {
            // the first wave scans that segment, one entry per lane (lanes
            // past the segment add nothing)
            const int i = ts * kSeg + tid;
            const float v = (tid < kSeg && i < len) ? resid(i) : 0.f;
            const float x = wave_incl_scan(v);
            const float base = cum + excl_b;
            const uint64_t over = __ballot(base + x > target);
            const uint64_t pos = __ballot(v > 0.f);
            int hit = -1;
            if (over) hit = (int)__ffsll((unsigned long long)over) - 1;
            else if (pos) hit = 63 - __clzll((long long)pos);   // rounding left no crossing: the last entry with mass
            if (tid == 0) ybcast = hit >= 0 ? c0 + ts * kSeg + hit : -1;
          } else if (ts == 0x7FFFFFFF && tid == 0) {
            ybcast = -1;
          }
          __syncthreads();
          y = ybcast;
        }
        if (y < 0) {
          // no crossing at all: the largest entry of the chunk with positive mass
          int lp = -1;
          for (int i = s0; i < min(s0 + kSeg, len); ++i)
            if (resid(i) > 0.f) lp = c0 + i;
          __syncthreads();
          if (tid == 0) ibcast = -1;
          __syncthreads();
          if (lp >= 0) atomicMax(&ibcast, lp);
          __syncthreads();
          y = ibcast >= 0 ? ibcast : c0;
        }
        emitted = y;
      }
      break;
    }
    // the drawn token goes to workgroup 0, which writes every output of the
    // sequence (one writer per output word, whatever happens to the others)
    if (sync_ok && !nonfinite && st == SV_TREE_OK && owner != 0) {
      if (!gx.to_first(w, owner, (uint32_t)emitted, &tok_b)) sync_ok = false;
      else if (w == 0) emitted = (int)tok_b;
    }
    if (!sync_ok) {
      // A wait passed its bound (the group's workgroups were not all resident
      // together): this workgroup stops.  Workgroup 0 marks this sequence and
      // every later one of the group, which no longer can be walked, with
      // SV_TREE_E_SYNC (keeping an earlier data status) and -1 / count 0
      // outputs; it waits for nothing more, so every workgroup ends.
      if (w == 0) {
        for (int bb = b; bb < p.B; bb += p.ngroups) {
          int32_t* on = p.out_nodes + (size_t)bb * p.T_max;
          int32_t* ot = p.out_tokens + (size_t)bb * p.T_max;
          for (int i = tid; i < p.T_max; i += kAccThreads) { on[i] = -1; ot[i] = -1; }
          if (tid == 0) {
            p.out_count[bb] = 0;
            if (p.out_passes) p.out_passes[bb] = 0;
            if (bb == b || p.status[bb] == SV_TREE_OK) p.status[bb] = SV_TREE_E_SYNC;
          }
        }
      }
      return;
    }
    if (nonfinite) st = SV_TREE_E_NONFINITE;
    __syncthreads();
    if (st != SV_TREE_OK) {
      if (w == 0) {
        for (int i = tid; i < p.T_max; i += kAccThreads) { onodes[i] = -1; otoks[i] = -1; }
        if (tid == 0) {
          p.out_count[b] = 0;
          p.status[b] = st;
          if (p.out_passes) p.out_passes[b] = 0;
        }
      }
      continue;
    }
    // outputs, all by workgroup 0
    if (w == 0) {
      for (int i = tid; i < p.T_max; i += kAccThreads) {
        if (i < path_len) {
          onodes[i] = path_s[i];
          otoks[i] = tok_s[path_s[i]];
        } else {
          onodes[i] = -1;
          otoks[i] = i == path_len ? emitted : -1;
        }
      }
      if (tid == 0) {
        p.out_count[b] = path_len + 1;
        if (p.out_passes) p.out_passes[b] = passes;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
int accept_exchange_words(const AcceptPlan& pl) { return pl.ngroups * 2 * pl.nchunk * kXWords; }

bool plan_accept(const sv_tree* t, const sv_accept_args* a, AcceptPlan* pl) {
  const DeviceInfo& di = device_info();
  *pl = AcceptPlan{};
  const int cap = kMaxChunk;                         // entries one workgroup can cache
  int nmin = (a->V + cap - 1) / cap;
  if (nmin > 64) return false;                       // V > 64 * 16384
  int nchunk = t->B > 0 ? di.num_cu / t->B : 1;
  const int nmax_small = (a->V + 2047) / 2048;       // keep chunks >= 2048 entries
  if (nchunk > nmax_small) nchunk = nmax_small;
  if (nchunk > 64) nchunk = 64;
  if (nchunk < nmin) nchunk = nmin;
  if (nchunk < 1) nchunk = 1;
  int chunk = (a->V + nchunk - 1) / nchunk;
  chunk = (chunk + 7) / 8 * 8;
  nchunk = (a->V + chunk - 1) / chunk;
  pl->nchunk = nchunk;
  pl->chunk = chunk;
  // groups resident at once: one walk workgroup per CU (up to 128 KB of LDS)
  int ngroups = di.num_cu / nchunk;
  if (ngroups < 1) ngroups = 1;
  if (ngroups > t->B) ngroups = t->B > 0 ? t->B : 1;
  pl->ngroups = ngroups;
  size_t off = 0;
  pl->off_xchg = off;
  off += align_up((size_t)accept_exchange_words(*pl) * sizeof(uint64_t), kWsAlign);
  pl->ws_bytes = off;
  return true;
}

sv_status launch_accept(const sv_tree* t, int32_t* tree_status, const sv_accept_args* a,
                        const AcceptPlan& pl, void* ws, bool clear_exchange, hipStream_t s) {
  if (t->B == 0) return SV_OK;
  char* wsb = static_cast<char*>(ws);
  WalkParams wp{};
  wp.parent = t->parent;
  wp.num_nodes = t->num_nodes;
  wp.tokens = t->tokens;
  wp.logits = a->target_logits;
  wp.q_probs = a->q_probs;
  wp.temperature = a->temperature;
  wp.u_accept = a->u_accept;
  wp.u_sample = a->u_sample;
  wp.status = tree_status;
  wp.out_tokens = a->out_tokens;
  wp.out_nodes = a->out_nodes;
  wp.out_count = a->out_count;
  wp.out_passes = a->out_passes;
  wp.xchg = reinterpret_cast<uint64_t*>(wsb + pl.off_xchg);
  wp.B = t->B;
  wp.T_max = t->T_max;
  wp.V = a->V;
  wp.nchunk = pl.nchunk;
  wp.chunk = pl.chunk;
  wp.ngroups = pl.ngroups;
  wp.bf16 = a->logit_dtype == SV_BF16;
  wp.sibling_mode = a->sibling_mode;
  // one exchange wait may last 2 s (200M ticks of the 100 MHz counter);
  // SV_WALK_WAIT_TICKS sets another bound, e.g. 0 to make every wait that
  // does not find its value at once give up (a test of the give-up path)
  wp.wait_ticks = 200000000ull;
  if (const char* ov = getenv("SV_WALK_WAIT_TICKS")) wp.wait_ticks = strtoull(ov, nullptr, 10);
  // exchange words start at zero on every call (a fill kernel: no memset
  // node, so the call can be captured in a graph; a verify step's mask kernel
  // zeroes them instead)
  hipError_t e = hipSuccess;
  if (clear_exchange) {
    hipLaunchKernelGGL(k_accept_clear, dim3(1), dim3(256), 0, s, wp.xchg, accept_exchange_words(pl));
    e = hipGetLastError();
    if (e != hipSuccess) {
      set_error("accept clear launch: %s", hipGetErrorString(e));
      return SV_E_HIP;
    }
  }
  // 16-byte vector loads: V % 8 == 0 and 16-byte aligned rows of logits and q
  const bool vec = (a->V % 8) == 0 && (reinterpret_cast<uintptr_t>(a->target_logits) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(a->q_probs) % 16) == 0;
  const void* fn = wp.bf16 ? (vec ? (const void*)k_accept_walk<true, true> : (const void*)k_accept_walk<true, false>)
                           : (vec ? (const void*)k_accept_walk<false, true> : (const void*)k_accept_walk<false, false>);
  void* args[] = {&wp};
  const size_t smem = 2 * (size_t)pl.chunk * sizeof(float);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * kMaxChunk * sizeof(float)));
  // The workgroups of a group wait for each other, so the whole grid must fit
  // on the device at once: at most one workgroup per CU, and the kernel's
  // occupancy must allow one.  (A plain launch: the cooperative one costs
  // about 20 us more per call.)  Workgroups queued behind other work on the
  // device start when that work ends; the waits are bounded by time and
  // report SV_TREE_E_SYNC rather than hang.
  // per device and kernel variant, 0 = not asked yet (the same value whichever thread fills it)
  static std::atomic<int> occ_cache[64][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::atomic<int>& slot = occ_cache[dev][(wp.bf16 ? 2 : 0) + (vec ? 1 : 0)];
  int occ = slot.load(std::memory_order_relaxed);
  if (e == hipSuccess && occ == 0) {
    // the smallest chunk size needs the least LDS: ask with the largest
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kAccThreads, 2 * kMaxChunk * sizeof(float));
    if (e == hipSuccess) {
      if (occ == 0) occ = -1;
      slot.store(occ, std::memory_order_relaxed);
    }
  }
  if (e == hipSuccess && (occ < 1 || pl.ngroups * pl.nchunk > device_info().num_cu)) {
    set_error("accept walk: %d workgroups do not fit at once (%d per CU, %d CUs)", pl.ngroups * pl.nchunk, occ,
              device_info().num_cu);
    return SV_E_UNSUPPORTED;
  }
  if (e == hipSuccess) e = hipLaunchKernel(fn, dim3(pl.ngroups * pl.nchunk), dim3(kAccThreads), args, smem, s);
  if (e != hipSuccess) {
    set_error("accept walk launch: %s", hipGetErrorString(e));
    return SV_E_HIP;
  }
  return SV_OK;
}

}  // namespace sv
