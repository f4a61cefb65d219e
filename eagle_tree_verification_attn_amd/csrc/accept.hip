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
// Two kernels:
//
//  k_vocab_stats  one workgroup per (tree position, vocabulary chunk): chunk
//                 max m_c, sum_c exp((z - m_c) / tau) (stochastic rows) or the
//                 lowest-index argmax (greedy rows), and a non-finite flag.
//                 Reads every logits row of the batch once.
//
//  k_accept_walk  cooperative launch of groups of `nchunk` workgroups; a group
//                 walks one sequence at a time, workgroup w owning vocabulary
//                 chunk w.  All workgroups of a group take the same scalar
//                 decisions from the same data; each rejection needs the mass
//                 of the new residual, summed over the vocabulary by all
//                 workgroups and exchanged through a group barrier.
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

namespace sv {

constexpr int kAccThreads = 256;
constexpr int kMaxChunk = 16384;  // vocabulary entries one walk workgroup caches in LDS
constexpr float kLog2e = 1.4426950408889634f;

struct StatsParams {
  const void* logits;
  const float* temperature;
  const int32_t* num_nodes;
  const int32_t* status;
  float4* stats;   // [B][T_max][nchunk]: m, s, argmax (int bits), flags (int bits)
  int* sync;       // [ngroups] group barrier counters, cleared here
  int B, T_max, V, nchunk, chunk, ngroups;
  int bf16;
};

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
  const float4* stats;
  int* sync;
  float* part;     // [ngroups][2][nchunk]
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
// k_vocab_stats
// ----------------------------------------------------------------------------
// Per-thread batches of kStatsBatch groups of 8 logits are loaded (as raw
// 16-byte words) before any arithmetic, so each thread keeps kStatsBatch (bf16)
// or 2 * kStatsBatch (fp32) 16-byte loads in flight.
constexpr int kStatsBatch = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16, int H>
__device__ inline float elem8(const u32x4 (&w)[H], int e) {
  if (BF16) {
    const uint32_t x = w[0][e >> 1];
    return (e & 1) ? bf16_hi(x) : bf16_lo(x);
  }
  return __uint_as_float(w[e >> 2][e & 3]);
}

// Loads one item's share for this thread: kStatsBatch groups of 8 logits at
// vocabulary index base + q * threads * 8 (addresses clamped into the chunk so
// every load is unconditional).
template <bool BF16, bool VEC, int RH = BF16 ? 1 : 2>
__device__ inline void stats_load(const void* logits, size_t row, int V, int base, int i0, int i1,
                                  u32x4 (&raw)[kStatsBatch][RH]) {
  const uint16_t* rowh = reinterpret_cast<const uint16_t*>(logits) + row * V;
  const float* rowf = reinterpret_cast<const float*>(logits) + row * V;
#pragma unroll
  for (int q = 0; q < kStatsBatch; ++q) {
    const int i = base + q * kAccThreads * 8;
    const int ic = i < i1 ? i : i0;
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
        const int v = (ic + e < i1) ? ic + e : i0;
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

// One workgroup per item (row b * T_max + n, vocabulary chunk c); each thread
// issues its whole batch of loads before any arithmetic.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kAccThreads) void k_vocab_stats(StatsParams p) {
  __shared__ float red_m[kAccThreads / 64], red_s[kAccThreads / 64];
  __shared__ int red_i[kAccThreads / 64], red_f[kAccThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int cidx = blockIdx.x;
  const long row = blockIdx.y;            // b * T_max + n
  const int b = (int)(row / p.T_max);
  const int n = (int)(row % p.T_max);
  if (cidx == 0 && row == 0)
    for (int i = tid; i < p.ngroups; i += kAccThreads) p.sync[i] = 0;
  const int Tb = p.num_nodes[b];
  if (p.status[b] != SV_TREE_OK || n >= Tb || Tb > p.T_max) return;
  constexpr int RH = BF16 ? 1 : 2;   // 16-byte words per group of 8 logits
  u32x4 raw[kStatsBatch][RH];
  const int i0 = cidx * p.chunk, i1 = min(i0 + p.chunk, p.V);
  {
    const float tau = p.temperature[b];
    const bool greedy = greedy_temp(tau);
    const float k = greedy ? 0.f : kLog2e / tau;
    uint32_t badbits = 0u;
    float m = -INFINITY, s = 0.f;
    int am = 0x7FFFFFFF;
    const int base = i0 + tid * 8;
    // chunks hold at most threads * 8 * kStatsBatch entries (host-side plan)
    stats_load<BF16, VEC>(p.logits, (size_t)row, p.V, base, i0, i1, raw);
    // Non-finite test on the raw words: an all-ones exponent field plus one
    // carries into the field's top bit.  Clamped loads repeat real entries of
    // this chunk, so they change neither this flag nor the maximum.
#pragma unroll
    for (int q = 0; q < kStatsBatch; ++q) {
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
    if (greedy) {
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q) {
        const int i = base + q * kAccThreads * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = elem8<BF16, RH>(raw[q], e);
          if (i + e < i1 && x > m) { m = x; am = i + e; }   // strict: lowest index per thread
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, elem8<BF16, RH>(raw[q], e));
      const float mk = m * k;
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q) {
        const int i = base + q * kAccThreads * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          s += (i + e < i1) ? __builtin_amdgcn_exp2f(fmaf(elem8<BF16, RH>(raw[q], e), k, -mk)) : 0.f;
      }
    }
    // workgroup reduction: (max, argmax-lowest) or (max, sum), flags
    for (int off = 32; off > 0; off >>= 1) {
      const float om = __shfl_xor(m, off);
      const int oi = __shfl_xor(am, off);
      const float os = __shfl_xor(s, off);
      if (greedy) {
        if (om > m || (om == m && oi < am)) { m = om; am = oi; }
      } else {
        const float nm = fmaxf(m, om);
        const float a = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - nm) * k);
        const float c = (om == -INFINITY) ? 0.f : os * __builtin_amdgcn_exp2f((om - nm) * k);
        s = a + c;
        m = nm;
      }
    }
    const bool any_bad = __any(badbits != 0u);
    if (lane == 0) { red_m[wv] = m; red_s[wv] = s; red_i[wv] = am; red_f[wv] = any_bad; }
    __syncthreads();
    if (tid == 0) {
      float M = red_m[0], S = red_s[0];
      int I = red_i[0], F = red_f[0];
      for (int w = 1; w < kAccThreads / 64; ++w) {
        F |= red_f[w];
        if (greedy) {
          if (red_m[w] > M || (red_m[w] == M && red_i[w] < I)) { M = red_m[w]; I = red_i[w]; }
        } else {
          const float nm = fmaxf(M, red_m[w]);
          const float a = (M == -INFINITY) ? 0.f : S * __builtin_amdgcn_exp2f((M - nm) * k);
          const float c = (red_m[w] == -INFINITY) ? 0.f : red_s[w] * __builtin_amdgcn_exp2f((red_m[w] - nm) * k);
          S = a + c;
          M = nm;
        }
      }
      if (F) { M = 0.f; S = 0.f; I = 0; }
      p.stats[(size_t)row * p.nchunk + cidx] = make_float4(M, S, __int_as_float(I), __int_as_float(F));
    }
  }
}

// ----------------------------------------------------------------------------
// k_accept_walk
// ----------------------------------------------------------------------------
__device__ inline float block_sum(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
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
  float x = v;
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  float xprev = __shfl_up(x, 1);
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

// Loads vocabulary chunk [c0, c1) of one node into LDS: target probabilities
// p(v) = 2^((z(v) - m) k - ls) at pc[v - c0] and, when want_q, q(v) at
// qc[v - c0].  VEC: the row is 16-byte aligned and V % 8 == 0, so a group of 8
// entries never straddles the chunk end.
template <bool BF16, bool VEC>
__device__ inline void load_chunk(const void* zrow, const float* qrow, int c0, int c1, float m,
                                  float k, float ls, bool want_q, float* pc, float* qc) {
  const int len = c1 - c0;
  for (int i = threadIdx.x * 8; i < len; i += kAccThreads * 8) {
    float z[8], q[8];
    if (VEC) {
      if (BF16) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(zrow) + c0 + i);
        z[0] = bf16_lo(w.x); z[1] = bf16_hi(w.x); z[2] = bf16_lo(w.y); z[3] = bf16_hi(w.y);
        z[4] = bf16_lo(w.z); z[5] = bf16_hi(w.z); z[6] = bf16_lo(w.w); z[7] = bf16_hi(w.w);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(zrow) + c0 + i);
        const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(zrow) + c0 + i + 4);
        z[0] = a.x; z[1] = a.y; z[2] = a.z; z[3] = a.w; z[4] = b.x; z[5] = b.y; z[6] = b.z; z[7] = b.w;
      }
      if (want_q) {
        const float4 a = *reinterpret_cast<const float4*>(qrow + c0 + i);
        const float4 b = *reinterpret_cast<const float4*>(qrow + c0 + i + 4);
        q[0] = a.x; q[1] = a.y; q[2] = a.z; q[3] = a.w; q[4] = b.x; q[5] = b.y; q[6] = b.z; q[7] = b.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = c0 + i + e;
        z[e] = -INFINITY;
        q[e] = 0.f;
        if (i + e < len) {
          z[e] = BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(zrow)[v] << 16)
                      : reinterpret_cast<const float*>(zrow)[v];
          if (want_q) q[e] = qrow[v];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (VEC || i + e < len) {
        pc[i + e] = z[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(z[e] - m, k, -ls));
        qc[i + e] = want_q ? q[e] : 0.f;
      }
    }
  }
  __syncthreads();
}

struct GroupSync {
  int* counter;
  int epoch;
  int members;
  // Returns false when the wait exceeded its bound (co-residency broken).
  __device__ bool arrive_and_wait() {
    __shared__ int ok;
    ++epoch;
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const int target = epoch * members;
      int spins = 0;
      ok = 1;
      while (__hip_atomic_load(counter, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > (1 << 24)) { ok = 0; break; }
      }
    }
    __syncthreads();
    return ok != 0;
  }
};

template <bool BF16, bool VEC>
__global__ __launch_bounds__(kAccThreads) void k_accept_walk(WalkParams p) {
  // Per-sequence data gathered once into LDS, so the walk's scalar decisions
  // read LDS instead of chaining dependent global loads.
  __shared__ int par_s[kMaxT];
  __shared__ int tok_s[kMaxT];
  __shared__ int path_s[kMaxT];
  __shared__ float m_s[kMaxT];    // row max of the target logits
  __shared__ float ls_s[kMaxT];   // log2 of sum exp((z - m) / tau) (stochastic rows)
  __shared__ int am_s[kMaxT];     // lowest-index argmax (greedy rows)
  __shared__ float zx_s[kMaxT];   // logit of node c's token in its parent's row
  __shared__ float qx_s[kMaxT];   // q of node c's token in its parent's row
  __shared__ float ua_s[kMaxT];
  __shared__ float us_s[kMaxT];
  __shared__ float red[kAccThreads / 64];
  __shared__ float masses[64];
  __shared__ float bcast;
  __shared__ int ibcast;
  __shared__ int flags_s;

  const int tid = threadIdx.x;
  const int grp = blockIdx.x / p.nchunk;
  const int w = blockIdx.x % p.nchunk;
  const int c0 = w * p.chunk;
  const int c1 = min(c0 + p.chunk, p.V);
  const bool wor = p.sibling_mode == SV_SIB_WITHOUT_REPLACEMENT;
  GroupSync gs{p.sync + grp, 0, p.nchunk};
  extern __shared__ __align__(16) float cache_s[];   // p then q of this workgroup's chunk
  float* pc = cache_s;
  float* qc = cache_s + p.chunk;
  const int len = c1 - c0;

  for (int b = grp; b < p.B; b += p.ngroups) {
    int st = p.status[b];
    const int Tb = p.num_nodes[b];
    if (st == SV_TREE_OK && (Tb < 1 || Tb > p.T_max)) st = SV_TREE_E_COUNT;
    const float tau = p.temperature[b];
    const bool greedy = greedy_temp(tau);
    const float k = greedy ? 0.f : kLog2e / tau;
    int32_t* onodes = p.out_nodes + (size_t)b * p.T_max;
    int32_t* otoks = p.out_tokens + (size_t)b * p.T_max;
    const size_t rowbase = (size_t)b * p.T_max;
    __syncthreads();
    if (tid == 0) flags_s = 0;
    __syncthreads();
    if (st == SV_TREE_OK) {
      // round 1: tree, tokens, uniforms, per-row statistics
      for (int i = tid; i < Tb; i += kAccThreads) {
        par_s[i] = p.parent[rowbase + i];
        const int x = p.tokens[rowbase + i];
        tok_s[i] = x;
        ua_s[i] = p.u_accept[rowbase + i];
        us_s[i] = p.u_sample[rowbase + i];
        int f = (x < 0 || x >= p.V) ? 1 : 0;
        const float4* srow = p.stats + (rowbase + i) * p.nchunk;
        float m = -INFINITY, ssum = 0.f;
        int am = 0;
        for (int cc = 0; cc < p.nchunk; ++cc) {
          const float4 v = srow[cc];
          f |= __float_as_int(v.w) != 0 ? 2 : 0;
          if (v.x > m) { m = v.x; am = __float_as_int(v.z); }   // first chunk with the max: lowest index
        }
        if (!greedy)
          for (int cc = 0; cc < p.nchunk; ++cc) {
            const float4 v = srow[cc];
            ssum += v.y * __builtin_amdgcn_exp2f((v.x - m) * k);
          }
        m_s[i] = m;
        am_s[i] = am;
        ls_s[i] = greedy ? 0.f : __log2f(ssum);
        if (f) atomicOr(&flags_s, f);
      }
      __syncthreads();
      const int f = flags_s;
      if (f & 1) st = SV_TREE_E_TOKEN;
      else if (f & 2) st = SV_TREE_E_NONFINITE;
      else if (!greedy && p.q_probs == nullptr) st = SV_TREE_E_NOQ;
      // round 2: each candidate's logit and draft probability in its parent's row
      if (st == SV_TREE_OK && !greedy) {
        for (int c = 1 + tid; c < Tb; c += kAccThreads) {
          const int n = par_s[c], x = tok_s[c];
          zx_s[c] = load_logit(BF16 ? (const void*)(reinterpret_cast<const uint16_t*>(p.logits) + (rowbase + n) * p.V)
                                    : (const void*)(reinterpret_cast<const float*>(p.logits) + (rowbase + n) * p.V),
                               (size_t)x, BF16);
          qx_s[c] = p.q_probs[(rowbase + n) * p.V + x];
        }
      }
      __syncthreads();
    }
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
    if (greedy && w != 0) continue;

    int n = 0, path_len = 0, passes = 0, emitted = -1, owner = -1;
    bool sync_ok = true;
    while (true) {
      int acc = -1;
      if (greedy) {
        const int am = am_s[n];
        for (int i = n + 1; i < Tb; ++i)
          if (par_s[i] == n && tok_s[i] == am) { acc = i; break; }
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
      const float m = m_s[n], ls = ls_s[n];
      const void* zrow = BF16 ? (const void*)(reinterpret_cast<const uint16_t*>(p.logits) + (rowbase + n) * p.V)
                              : (const void*)(reinterpret_cast<const float*>(p.logits) + (rowbase + n) * p.V);
      const float* qrow = p.q_probs + (rowbase + n) * p.V;
      // draw masses of P = p_n, from the chunk statistics
      __syncthreads();
      if (tid < p.nchunk) {
        const float4 v = p.stats[(rowbase + n) * p.nchunk + tid];
        masses[tid] = v.y * __builtin_amdgcn_exp2f((v.x - m) * k - ls);
      }
      float A = 0.f, Wn = 1.f, rm = 0.f, Adraw = 0.f;
      bool loaded = false;
      for (int c = n + 1; c < Tb; ++c) {
        if (par_s[c] != n) continue;
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
        if (!loaded) {
          load_chunk<BF16, VEC>(zrow, qrow, c0, c1, m, k, ls, true, pc, qc);
          loaded = true;
        }
        float part = 0.f;
        for (int i = tid * 4; i < len; i += kAccThreads * 4) {
          if (i + 4 <= len) {
            const float4 pp = *reinterpret_cast<const float4*>(pc + i);
            const float4 qq = *reinterpret_cast<const float4*>(qc + i);
            part += fmaxf(fmaf(-An, qq.x, pp.x), 0.f) + fmaxf(fmaf(-An, qq.y, pp.y), 0.f) +
                    fmaxf(fmaf(-An, qq.z, pp.z), 0.f) + fmaxf(fmaf(-An, qq.w, pp.w), 0.f);
          } else {
            for (int e = i; e < len; ++e) part += fmaxf(fmaf(-An, qc[e], pc[e]), 0.f);
          }
        }
        part = block_sum(part, red);
        // partials of barrier epoch e live in slot e % 2: a slot is rewritten
        // two epochs later, after every member has passed the epoch between
        float* slot = p.part + ((size_t)grp * 2 + ((gs.epoch + 1) & 1)) * p.nchunk;
        if (tid == 0) __hip_atomic_store(slot + w, part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!gs.arrive_and_wait()) { sync_ok = false; break; }
        if (tid == 0) {
          float tot = 0.f;
          for (int cc = 0; cc < p.nchunk; ++cc)
            tot += __hip_atomic_load(slot + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          bcast = tot;
          if (tot > 0.f)
            for (int cc = 0; cc < p.nchunk; ++cc)
              masses[cc] = __hip_atomic_load(slot + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      bool leaf = true;
      for (int c = n + 1; c < Tb; ++c)
        if (par_s[c] == n) { leaf = false; break; }
      if (leaf) ++passes;
      __syncthreads();
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
        if (!loaded) load_chunk<BF16, VEC>(zrow, qrow, c0, c1, m, k, ls, false, pc, qc);
        // scan the chunk in vocabulary order: thread t owns the contiguous
        // segment [t * seg, (t + 1) * seg)
        const int seg = (len + kAccThreads - 1) / kAccThreads;
        const int s0 = min(tid * seg, len), s1 = min(s0 + seg, len);
        int y = -1;
        if (!fallback) {
          float vs = 0.f;
          for (int i = s0; i < s1; ++i) vs += fmaxf(fmaf(-Adraw, qc[i], pc[i]), 0.f);
          float incl, excl, tot;
          block_scan(vs, red, &incl, &excl, &tot);
          if (tid == 0) ibcast = 0x7FFFFFFF;
          __syncthreads();
          if (cum + excl <= target && cum + incl > target) {
            float run = cum + excl;
            int found = -1, lastin = -1;
            for (int i = s0; i < s1; ++i) {
              const float v = fmaxf(fmaf(-Adraw, qc[i], pc[i]), 0.f);
              if (v > 0.f) lastin = i;
              run += v;
              if (run > target) { found = i; break; }
            }
            if (found < 0) found = lastin;
            if (found >= 0) atomicMin(&ibcast, c0 + found);
          }
          __syncthreads();
          if (ibcast != 0x7FFFFFFF) y = ibcast;
        }
        if (y < 0) {
          // rounding left no crossing: the largest entry of the chunk with positive mass
          int lp = -1;
          for (int i = s0; i < s1; ++i)
            if (fmaxf(fmaf(-Adraw, qc[i], pc[i]), 0.f) > 0.f) lp = c0 + i;
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
    if (!sync_ok) {
      if (tid == 0) p.status[b] = SV_TREE_E_SYNC;
      return;
    }
    __syncthreads();
    // outputs: the emitted token by its owner, everything else by workgroup 0
    if (w == owner && tid == 0) otoks[path_len] = emitted;
    if (w == 0) {
      for (int i = tid; i < p.T_max; i += kAccThreads) {
        if (i < path_len) {
          onodes[i] = path_s[i];
          otoks[i] = tok_s[path_s[i]];
        } else {
          onodes[i] = -1;
          if (i != path_len) otoks[i] = -1;
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
  pl->stats_threads = kAccThreads;
  size_t off = 0;
  pl->off_stats = off;
  off += align_up((size_t)t->B * t->T_max * nchunk * sizeof(float4), kWsAlign);
  pl->off_sync = off;
  off += align_up((size_t)ngroups * sizeof(int), kWsAlign);
  pl->off_part = off;
  off += align_up((size_t)ngroups * 2 * nchunk * sizeof(float), kWsAlign);
  pl->ws_bytes = off;
  return true;
}

sv_status launch_accept(const sv_tree* t, int32_t* tree_status, const sv_accept_args* a,
                        const AcceptPlan& pl, void* ws, hipStream_t s) {
  if (t->B == 0) return SV_OK;
  char* wsb = static_cast<char*>(ws);
  StatsParams sp{};
  sp.logits = a->target_logits;
  sp.temperature = a->temperature;
  sp.num_nodes = t->num_nodes;
  sp.status = tree_status;
  sp.stats = reinterpret_cast<float4*>(wsb + pl.off_stats);
  sp.sync = reinterpret_cast<int*>(wsb + pl.off_sync);
  sp.B = t->B;
  sp.T_max = t->T_max;
  sp.V = a->V;
  sp.nchunk = pl.nchunk;
  sp.chunk = pl.chunk;
  sp.ngroups = pl.ngroups;
  sp.bf16 = a->logit_dtype == SV_BF16;
  const bool vec = (a->V % 8) == 0 &&
                   (reinterpret_cast<uintptr_t>(a->target_logits) % 16) == 0;
  dim3 grid(pl.nchunk, t->B * t->T_max);
  if (sp.bf16) {
    if (vec) hipLaunchKernelGGL((k_vocab_stats<true, true>), grid, dim3(kAccThreads), 0, s, sp);
    else hipLaunchKernelGGL((k_vocab_stats<true, false>), grid, dim3(kAccThreads), 0, s, sp);
  } else {
    if (vec) hipLaunchKernelGGL((k_vocab_stats<false, true>), grid, dim3(kAccThreads), 0, s, sp);
    else hipLaunchKernelGGL((k_vocab_stats<false, false>), grid, dim3(kAccThreads), 0, s, sp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("vocab stats launch: %s", hipGetErrorString(e));
    return SV_E_HIP;
  }
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
  wp.stats = sp.stats;
  wp.sync = sp.sync;
  wp.part = reinterpret_cast<float*>(wsb + pl.off_part);
  wp.B = t->B;
  wp.T_max = t->T_max;
  wp.V = a->V;
  wp.nchunk = pl.nchunk;
  wp.chunk = pl.chunk;
  wp.ngroups = pl.ngroups;
  wp.bf16 = sp.bf16;
  wp.sibling_mode = a->sibling_mode;
  const bool wvec = vec && (reinterpret_cast<uintptr_t>(a->q_probs) % 16) == 0;
  const void* fn = sp.bf16 ? (wvec ? (const void*)k_accept_walk<true, true> : (const void*)k_accept_walk<true, false>)
                           : (wvec ? (const void*)k_accept_walk<false, true> : (const void*)k_accept_walk<false, false>);
  void* args[] = {&wp};
  const size_t smem = 2 * (size_t)pl.chunk * sizeof(float);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * kMaxChunk * sizeof(float)));
  if (e == hipSuccess)
    e = hipLaunchCooperativeKernel(fn, dim3(pl.ngroups * pl.nchunk), dim3(kAccThreads), args, smem, s);
  if (e != hipSuccess) {
    set_error("accept walk launch: %s", hipGetErrorString(e));
    return SV_E_HIP;
  }
  return SV_OK;
}

}  // namespace sv
