// EAGLE-2 draft-tree builder ([EAGLE article] sec. 2.3 "Context-aware draft
// tree": node value = product of draft confidences along the path; expansion
// of the k best nodes of the newest layer; rerank of the m best nodes of the
// whole tree, equal values to the shallower node; flattening for
// verification).
//
// Three kernels:
//   k_row_topk     one workgroup per (sequence, frontier row, 8192-token
//                  chunk): reads the chunk of the drafter's probability row
//                  once into registers and checks the range.  In each wave
//                  the k-th largest of the lanes' maxima (found by bisection
//                  on its bits) bounds the chunk's k-th largest value from
//                  below (those k maxima are k tokens at least that large);
//                  the largest of the waves' bounds is used, only tokens at or
//                  above it are gathered in LDS as exact keys and ranked (when
//                  very many tie at that bound, k rounds of a block maximum
//                  over the chunk read again).  This is the HBM-bound part.
//   k_expand       one workgroup per sequence: merges each frontier row's
//                  chunk lists (sorted, so a k-way merge by DPP maxima),
//                  appends the children (value = parent value x probability,
//                  one float32 multiply) and ranks the new layer to pick the
//                  next frontier.
//   k_finish       one workgroup per sequence: ranks every draft node, keeps
//                  the m best and assigns flattened positions depth by depth.
//   k_expand_finish  the last step's k_expand and k_finish in one workgroup
//                  per sequence (one launch less).
//
// The per-sequence kernels are latency-bound: each issues all of its
// independent loads at once (one HBM round trip) and then works in LDS.
//
// A (probability, token) pair is one 64-bit key: the probability's bits (it is
// in [0, 1], so its bit pattern orders like its value once -0 is made +0) above
// the complement of the token.  The larger key is the higher probability, then
// the lower token; 0 is below every real key.
#include "sv_internal.h"

namespace sv {

constexpr int kTopkThreads = 256;
constexpr int kE2Chunk = 8192;                       // tokens per top-k workgroup
constexpr int kEPT = kE2Chunk / kTopkThreads;        // elements per thread (32)
constexpr int kCandCap = 1024;                       // gathered candidates per chunk
constexpr int kE2MaxK = 16;
constexpr int kE2MaxSplit = 64;                      // chunks per row: V <= 64 * 8192
constexpr int kE2StageKeys = kE2MaxSplit * kE2MaxK;  // 1024 keys staged in LDS at a time
constexpr int kE2Threads = 1024;
constexpr int kFinishThreads = 1024;
static_assert(kE2StageKeys <= kE2Threads, "expand loads the first group of keys one per thread");
static_assert(kE2MaxK * kE2MaxSplit <= kE2Threads, "expand loads the range flags one per thread");

struct E2Params {
  int B, V, k, depth, m, nsplit, chunk, nmax;
  int32_t* seq;        // [B][8]: n_nodes, layer_begin, nfront, status
  int4* front;         // [B][16] frontier records: node id, value bits, depth, token
  int32_t* parent;     // [B][nmax]
  int32_t* token;      // [B][nmax]
  int32_t* depthv;     // [B][nmax]
  int32_t* rank;       // [B][nmax] rank among siblings
  int32_t* qrow;       // [B][nmax]
  float* value;        // [B][nmax]
  uint64_t* cand;      // [B][k][nsplit][k]
  int32_t* cand_bad;   // [B][k][nsplit]
};

enum { kSeqN = 0, kSeqLayer = 1, kSeqFront = 2, kSeqStatus = 3 };

E2Layout eagle2_layout(const sv_eagle2_cfg* c) {
  E2Layout L{};
  L.nmax = 1 + c->k + (c->depth - 1) * c->k * c->k;
  L.nsplit = (c->V + kE2Chunk - 1) / kE2Chunk;
  if (L.nsplit < 1) L.nsplit = 1;
  L.chunk = kE2Chunk;
  size_t o = 0;
  const size_t B = (size_t)c->B, N = (size_t)L.nmax, k = (size_t)c->k;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, kWsAlign); return at; };
  L.off_seq = take(B * 8 * 4);
  L.off_front = take(B * 16 * 16);
  L.off_parent = take(B * N * 4);
  L.off_token = take(B * N * 4);
  L.off_depth = take(B * N * 4);
  L.off_rank = take(B * N * 4);
  L.off_qrow = take(B * N * 4);
  L.off_value = take(B * N * 4);
  L.off_cand = take(B * k * (size_t)L.nsplit * k * 8);
  L.off_bad = take(B * k * (size_t)L.nsplit * 4);
  L.bytes = o;
  return L;
}

static E2Params make_params(const sv_eagle2_cfg* c, const E2Layout& L, void* state) {
  unsigned char* base = static_cast<unsigned char*>(state);
  E2Params p{};
  p.B = c->B; p.V = c->V; p.k = c->k; p.depth = c->depth; p.m = c->m;
  p.nsplit = L.nsplit; p.chunk = L.chunk; p.nmax = L.nmax;
  p.seq = reinterpret_cast<int32_t*>(base + L.off_seq);
  p.front = reinterpret_cast<int4*>(base + L.off_front);
  p.parent = reinterpret_cast<int32_t*>(base + L.off_parent);
  p.token = reinterpret_cast<int32_t*>(base + L.off_token);
  p.depthv = reinterpret_cast<int32_t*>(base + L.off_depth);
  p.rank = reinterpret_cast<int32_t*>(base + L.off_rank);
  p.qrow = reinterpret_cast<int32_t*>(base + L.off_qrow);
  p.value = reinterpret_cast<float*>(base + L.off_value);
  p.cand = reinterpret_cast<uint64_t*>(base + L.off_cand);
  p.cand_bad = reinterpret_cast<int32_t*>(base + L.off_bad);
  return p;
}

__device__ inline uint64_t prob_key(float v, int tok) {
  const float z = v + 0.0f;   // -0 -> +0
  return ((uint64_t)__float_as_uint(z) << 32) | (uint64_t)(~(uint32_t)tok);
}
__device__ inline float key_prob(uint64_t key) { return __uint_as_float((uint32_t)(key >> 32)); }
__device__ inline int key_token(uint64_t key) { return (int)(~(uint32_t)key); }

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------- begin
__global__ void k_e2_begin(E2Params p, const int32_t* root_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.B) return;
  int32_t* s = p.seq + (size_t)b * 8;
  s[kSeqN] = 1;
  s[kSeqLayer] = 0;
  s[kSeqFront] = 1;
  s[kSeqStatus] = SV_TREE_OK;
  const int root = root_tokens[b];
  p.front[(size_t)b * 16] = make_int4(0, (int)__float_as_uint(1.0f), 0, root);
  const size_t n0 = (size_t)b * p.nmax;
  p.parent[n0] = -1;
  p.token[n0] = root;
  p.depthv[n0] = 0;
  p.rank[n0] = 0;
  p.qrow[n0] = -1;
  p.value[n0] = 1.0f;
}

// ---------------------------------------------------------------- row top-k
// grid: B * jrows * nsplit workgroups; workgroup (b, j, c) reads chunk c of
// row j.  jrows is 1 at the first step (the root) and k after it, when every
// sequence still building has a full frontier; so the row loads go out before
// the sequence's state is read, and a workgroup of a finished or failed
// sequence only discards them.
__global__ __launch_bounds__(kTopkThreads) void k_row_topk(E2Params p, const float* q, int jrows) {
  const int c = blockIdx.x % p.nsplit;
  const int j = (blockIdx.x / p.nsplit) % jrows;
  const int b = blockIdx.x / (p.nsplit * jrows);
  const int tid = threadIdx.x;
  const int32_t* s = p.seq + (size_t)b * 8;
  const int lo = c * kE2Chunk;
  const int hi = min(p.V, lo + kE2Chunk);
  const float* row = q + ((size_t)b * p.k + j) * p.V;
  const bool vec = (p.V & 3) == 0;
  // element i of this thread: 16-byte runs when rows are 16-byte aligned
  auto index = [&](int i) { return vec ? lo + 4 * (tid + kTopkThreads * (i >> 2)) + (i & 3) : lo + tid + kTopkThreads * i; };
  // every load is issued before any is used: addresses past the chunk's end
  // are clamped to its start, and in(i) below leaves those values out
  float v[kEPT];
  if (vec) {   // hi is then a multiple of 4 too
#pragma unroll
    for (int i4 = 0; i4 < kEPT / 4; ++i4) {
      const int e = lo + 4 * (tid + kTopkThreads * i4);
      const float4 x = *reinterpret_cast<const float4*>(row + (e < hi ? e : lo));
      v[4 * i4] = x.x; v[4 * i4 + 1] = x.y; v[4 * i4 + 2] = x.z; v[4 * i4 + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
      const int e = lo + tid + kTopkThreads * i;
      v[i] = row[e < hi ? e : lo];
    }
  }
  // this thread's elements of the chunk are its first nv (all kEPT in a full
  // chunk, fewer in the last one): in(i) is one compare
  const int len = hi - lo;
  const int nv = vec ? 4 * min(kEPT / 4, max(0, (len / 4 - tid + kTopkThreads - 1) / kTopkThreads))
                     : min(kEPT, max(0, (len - tid + kTopkThreads - 1) / kTopkThreads));
  auto in = [&](int i) { return i < nv; };
  // range check and this thread's largest value, without branches: a NaN or
  // negative value fails v >= 0, a value above 1 shows in the maximum
  float mx = -1.0f;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
    const bool ok = in(i);
    mx = fmaxf(mx, ok ? v[i] : -1.0f);
    bad |= ok && !(v[i] >= 0.0f);
  }
  bad |= mx > 1.0f;
  if (s[kSeqStatus] != SV_TREE_OK || j >= s[kSeqFront]) return;
  __shared__ uint64_t cand_s[kCandCap];
  __shared__ uint64_t wmax[kTopkThreads / 64];
  __shared__ float t0_s[kTopkThreads / 64];
  __shared__ int ncand_s, bad_s;
  uint64_t* out = p.cand + (((size_t)b * p.k + j) * p.nsplit + c) * p.k;
  if (tid == 0) { ncand_s = 0; bad_s = 0; }
  if (tid < p.k) out[tid] = 0;
  // per wave, the k-th largest of its lanes' maxima (-1 when fewer than k
  // lanes hold a token).  k lanes' maxima are k tokens at least that large,
  // so it bounds the chunk's k-th largest value from below.  On the maxima's
  // bits (order-preserving for values in [0, 1] once -0 is made +0; -1 is
  // negative) it is the largest t with at least k lanes at or above t, built
  // bit by bit from the top: one compare and one ballot count per bit.
  {
    const int key = __float_as_int(mx + 0.0f);
    float tw = -1.0f;
    if (__popcll(__ballot(key >= 0)) >= p.k) {
      int t = 0;
#pragma unroll
      for (int bit = 30; bit >= 0; --bit) {
        const int cand = t | (1 << bit);
        if (__popcll(__ballot(key >= cand)) >= p.k) t = cand;
      }
      tw = __int_as_float(t);
    }
    if ((tid & 63) == 0) t0_s[tid >> 6] = tw;
  }
  __syncthreads();   // the bounds, and the counters' initial values
  if (bad) bad_s = 1;
  float t0 = -1.0f;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) t0 = fmaxf(t0, t0_s[w]);
  // the candidates: every token at or above the bound, as exact keys
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) mine += in(i) && v[i] >= t0;
  int at = mine ? atomicAdd(&ncand_s, mine) : 0;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
    if (in(i) && v[i] >= t0) {
      if (at < kCandCap) cand_s[at] = prob_key(v[i], index(i));
      ++at;
    }
  }
  __syncthreads();
  const int C = ncand_s;
  if (tid == 0) p.cand_bad[((size_t)b * p.k + j) * p.nsplit + c] = bad_s;   // settled at the barrier above
  if (C <= kCandCap) {
    for (int x = tid; x < C; x += kTopkThreads) {
      const uint64_t key = cand_s[x];
      int r = 0;
#pragma unroll 8
      for (int e = 0; e < C; ++e) r += cand_s[e] > key;
      if (r < p.k) out[r] = key;
    }
  } else {
    // very many keys tie at the bound: k rounds, each the block's largest key
    // below the previous round's.  The chunk is read again for it (from
    // cache), so the common path above is all that holds the values in
    // registers.
    uint64_t prev = ~0ull;
    for (int r = 0; r < p.k; ++r) {
      uint64_t m = 0;
#pragma unroll 1
      for (int i = 0; i < nv; ++i) {
        const int e = index(i);
        const uint64_t key = prob_key(row[e], e);
        if (key < prev && key > m) m = key;
      }
      const uint64_t w = wave_max_u64(m);
      if ((tid & 63) == 0) wmax[tid >> 6] = w;
      __syncthreads();
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kTopkThreads / 64; ++i) best = wmax[i] > best ? wmax[i] : best;
      __syncthreads();
      if (tid == 0) out[r] = best;
      prev = best;
    }
  }
}

// ---------------------------------------------------------------- expand
// Every load that does not depend on another goes out first, in one round
// trip: the sequence's state, its frontier records, the chunks' range flags of
// all k rows and the first group of chunk keys (all inside the state whatever
// the frontier's size; only the frontier's rows are used).
__device__ inline void expand_body(const E2Params& p, int step, int32_t* frontier_out, int32_t* frontier_tokens) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* s = p.seq + (size_t)b * 8;
  const size_t nb = (size_t)b * p.nmax;
  const int k = p.k;
  const int C = p.nsplit * k;                         // chunk keys per frontier row (<= 1024)
  const int rows = kE2StageKeys / C;                  // rows staged in LDS at a time (>= 1)
  const uint64_t* cb = p.cand + (size_t)b * k * C;
  __shared__ uint64_t best_s[kE2MaxK][kE2MaxK];       // per frontier row, its k best keys
  __shared__ uint64_t row_s[kE2StageKeys];            // chunk keys of a group of rows
  __shared__ float fval_s[kE2MaxK];
  __shared__ int fnode_s[kE2MaxK], fdep_s[kE2MaxK];
  __shared__ float val_s[kE2MaxK * kE2MaxK];          // the new layer's values
  __shared__ int bad_s;
  const int status = s[kSeqStatus];
  const int F = s[kSeqFront];
  const int n0 = s[kSeqN];
  const int4 rec = tid < k ? p.front[(size_t)b * 16 + tid] : make_int4(-1, 0, 0, -1);
  const int flag = tid < k * p.nsplit ? p.cand_bad[(size_t)b * k * p.nsplit + tid] : 0;   // k * nsplit <= 1024
  const int g0 = min(rows, k) * C;                    // <= kE2StageKeys = kE2Threads
  const uint64_t key0 = tid < g0 ? cb[tid] : 0;
  if (tid == 0) bad_s = 0;
  __syncthreads();
  bool ok = status == SV_TREE_OK;
  if (ok && flag && tid < F * p.nsplit) bad_s = 1;   // a chunk of a frontier row failed the range check
  __syncthreads();
  if (ok && bad_s) {
    ok = false;
    if (tid == 0) s[kSeqStatus] = SV_TREE_E_PROB;
  }
  // more steps than the state was sized for: the node arrays are full
  if (ok && n0 + F * k > p.nmax) {
    ok = false;
    if (tid == 0) s[kSeqStatus] = SV_TREE_E_COUNT;
  }
  if (ok) {
    if (tid < F) {
      fnode_s[tid] = rec.x;
      fval_s[tid] = __int_as_float(rec.y);
      fdep_s[tid] = rec.z;
    }
    // merge: a chunk's k keys come sorted (largest first, 0-padded), so each
    // row's k best are a k-way merge of its chunks' lists.  Row jj of a group
    // belongs to one 16-lane row of a wave; lane l of it holds the heads of
    // chunks l, l + 16, l + 32 and l + 48.  Each round takes the largest head
    // of the 16 lanes and advances the list it came from (keys are distinct,
    // since their tokens are).
    const int lane = tid & 63;
    const int jj = (tid >> 6) * 4 + (lane >> 4);       // up to 64 rows per group
    const int gl = lane & 15;
    const int nu = (p.nsplit + 15) / 16;                // chunks per lane, <= 4
    for (int j0 = 0; j0 < F; j0 += rows) {
      const int nr = min(rows, F - j0);
      if (j0 == 0) {
        if (tid < nr * C) row_s[tid] = key0;
      } else {
        for (int i = tid; i < nr * C; i += kE2Threads) row_s[i] = cb[(size_t)j0 * C + i];
      }
      __syncthreads();
      const bool live = jj < nr;
      const uint64_t* rs = row_s + (live ? jj : 0) * C;
      uint64_t head[4];
      int pos[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = gl + 16 * u;
        pos[u] = 0;
        head[u] = (live && u < nu && c < p.nsplit) ? rs[c * k] : 0;
      }
      for (int r = 0; r < k; ++r) {
        uint64_t mine = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) mine = head[u] > mine ? head[u] : mine;
        const uint64_t best = row16_max_u64(mine);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (best != 0 && head[u] == best) {
            const int c = gl + 16 * u;
            ++pos[u];
            head[u] = pos[u] < k ? rs[c * k + pos[u]] : 0;
          }
        }
        if (live && gl == 0) best_s[j0 + jj][r] = best;
      }
      __syncthreads();
    }
    // children of frontier entry j: ids n0 + j k + r
    const int Lc = F * k;
    for (int i = tid; i < Lc; i += kE2Threads) {
      const int j = i / k, r = i % k;
      const uint64_t key = best_s[j][r];
      const float v = __fmul_rn(fval_s[j], key_prob(key));
      const size_t id = nb + n0 + i;
      p.parent[id] = fnode_s[j];
      p.token[id] = key_token(key);
      p.depthv[id] = fdep_s[j] + 1;
      p.rank[id] = r;
      p.qrow[id] = -1;
      p.value[id] = v;
      val_s[i] = v;
    }
    if (tid < F) p.qrow[nb + fnode_s[tid]] = step * k + tid;
    __syncthreads();
    // next frontier: the k best of the new layer (value descending, then id);
    // Lc >= k, so all k entries are filled
    for (int i = tid; i < Lc; i += kE2Threads) {
      const float v = val_s[i];
      int r = 0;
#pragma unroll 8
      for (int e = 0; e < Lc; ++e) r += (val_s[e] > v) || (val_s[e] == v && e < i);
      if (r < k) {
        const int j = i / k;
        const int tok = key_token(best_s[j][i % k]);
        p.front[(size_t)b * 16 + r] = make_int4(n0 + i, (int)__float_as_uint(v), fdep_s[j] + 1, tok);
        if (frontier_out) frontier_out[(size_t)b * k + r] = n0 + i;
        if (frontier_tokens) frontier_tokens[(size_t)b * k + r] = tok;
      }
    }
    if (tid == 0) {
      s[kSeqLayer] = n0;
      s[kSeqN] = n0 + Lc;
      s[kSeqFront] = k;
    }
  } else if (tid < k) {
    if (frontier_out) frontier_out[(size_t)b * k + tid] = -1;
    if (frontier_tokens) frontier_tokens[(size_t)b * k + tid] = -1;
  }
}

__global__ __launch_bounds__(kE2Threads) void k_expand(E2Params p, int step, int32_t* frontier_out,
                                                       int32_t* frontier_tokens) {
  expand_body(p, step, frontier_out, frontier_tokens);
}

// ---------------------------------------------------------------- finish
__device__ inline void finish_body(const E2Params& p, int32_t* parent_out, int32_t* tokens_out, int32_t* num_nodes,
                                   int32_t* q_row_out, int32_t* status_out) {
  constexpr int kMaxNodes = 2048;
  __shared__ uint64_t nkey_s[kMaxNodes];   // (value, shallower, earlier): larger ranks first
  __shared__ int rnk_s[kMaxNodes];
  __shared__ int dep_s[kMaxNodes];
  __shared__ int pos_s[kMaxNodes];      // flattened position, -1 if not kept
  __shared__ int par_s[kMaxNodes];
  __shared__ int rank_s[kMaxNodes];
  __shared__ int kept_s[kMaxT];         // the kept draft nodes, in no particular order
  __shared__ int kkey_s[kMaxT];         // per depth pass: parent position * 16 + rank, or -1
  __shared__ int cnt_s, nkept_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* s = p.seq + (size_t)b * 8;
  const size_t nb = (size_t)b * p.nmax;
  const int T = p.m + 1;
  // one round trip: the state and every node slot this thread will handle
  // (slots at or past the node count hold nothing and are not used)
  constexpr int kSlots = kMaxNodes / kFinishThreads;
  int status = s[kSeqStatus];
  const int N = s[kSeqN];
  float valr[kSlots];
  int depr[kSlots], parr[kSlots], rankr[kSlots], tokr[kSlots], qrr[kSlots];
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int i = tid + u * kFinishThreads;
    const bool in = i < p.nmax;
    valr[u] = in ? p.value[nb + i] : 0.0f;
    depr[u] = in ? p.depthv[nb + i] : 0;
    parr[u] = in ? p.parent[nb + i] : -1;
    rankr[u] = in ? p.rank[nb + i] : 0;
    tokr[u] = in ? p.token[nb + i] : -1;
    qrr[u] = in ? p.qrow[nb + i] : -1;
  }
  if (status == SV_TREE_OK && (N - 1 < p.m || N > p.nmax)) status = SV_TREE_E_COUNT;   // too few steps ran
  if (tid == 0) status_out[b] = status;
  const bool ok = status == SV_TREE_OK;
  if (tid == 0) nkept_s = 0;
  if (!ok) {
    for (int i = tid; i < T; i += kFinishThreads) {
      parent_out[(size_t)b * T + i] = -1;
      tokens_out[(size_t)b * T + i] = -1;
      q_row_out[(size_t)b * T + i] = -1;
    }
    if (tid == 0) num_nodes[b] = 0;
    return;
  }
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int i = tid + u * kFinishThreads;
    if (i >= N) continue;
    // values are products of probabilities: non-negative, so their bits order
    // like the values once -0 is made +0; depth and id (< 2048) go below
    const uint32_t vb = __float_as_uint(valr[u] + 0.0f);
    nkey_s[i] = ((uint64_t)vb << 32) | ((uint32_t)(0xFFFF - depr[u]) << 16) | (uint32_t)(0xFFFF - i);
    rnk_s[i] = 0;
    dep_s[i] = depr[u];
    par_s[i] = parr[u];
    rank_s[i] = rankr[u];
    pos_s[i] = -1;
  }
  __syncthreads();
  // keep the m best draft nodes (value descending, depth ascending, id
  // ascending): each node's rank counted by several threads over parts of
  // the nodes, the parts added in LDS
  {
    const int M = N - 1;
    const int parts = M > 0 ? max(1, min(16, kFinishThreads / M)) : 1;
    const int span = (M + parts - 1) / parts;
    for (int x = tid; x < M * parts; x += kFinishThreads) {
      const int i = 1 + x / parts;
      const int e0 = 1 + (x % parts) * span;
      const int e1 = min(N, e0 + span);
      const uint64_t key = nkey_s[i];
      int r = 0;
#pragma unroll 8
      for (int e = e0; e < e1; ++e) r += nkey_s[e] > key;
      if (r) atomicAdd(&rnk_s[i], r);
    }
  }
  __syncthreads();
  for (int i = 1 + tid; i < N; i += kFinishThreads) {
    const bool keep = rnk_s[i] < p.m;
    pos_s[i] = keep ? 0 : -1;         // 0 marks kept; the position comes below
    if (keep) kept_s[atomicAdd(&nkept_s, 1)] = i;
  }
  if (tid == 0) pos_s[0] = 0;
  __syncthreads();
  // positions depth by depth: after the earlier depths, ordered by parent
  // position then sibling rank
  const int M = nkept_s;              // = m
  int base = 1;
  for (int d = 1; d <= p.depth; ++d) {
    for (int x = tid; x < M; x += kFinishThreads) {
      const int i = kept_s[x];
      kkey_s[x] = dep_s[i] == d ? pos_s[par_s[i]] * 16 + rank_s[i] : -1;
    }
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    for (int x = tid; x < M; x += kFinishThreads) {
      const int key = kkey_s[x];
      if (key < 0) continue;
      int r = 0;
#pragma unroll 8
      for (int e = 0; e < M; ++e) r += kkey_s[e] >= 0 && kkey_s[e] < key;
      pos_s[kept_s[x]] = base + r;
      atomicAdd(&cnt_s, 1);
    }
    __syncthreads();
    base += cnt_s;
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int i = tid + u * kFinishThreads;
    if (i >= N) continue;
    const int ps = pos_s[i];
    if (ps < 0 || ps >= T) continue;
    parent_out[(size_t)b * T + ps] = i == 0 ? -1 : pos_s[parr[u]];
    tokens_out[(size_t)b * T + ps] = tokr[u];
    q_row_out[(size_t)b * T + ps] = qrr[u];
  }
  if (tid == 0) num_nodes[b] = T;
}

__global__ __launch_bounds__(kFinishThreads) void k_finish(E2Params p, int32_t* parent_out, int32_t* tokens_out,
                                                           int32_t* num_nodes, int32_t* q_row_out,
                                                           int32_t* status_out) {
  finish_body(p, parent_out, tokens_out, num_nodes, q_row_out, status_out);
}

// The last expansion step and the rerank in one launch: the workgroup of a
// sequence appends the last layer, and after a barrier (its own global
// writes are then visible to all of its threads) reads the whole tree back
// and flattens it.  Saves the finish kernel's launch and its load round trip.
static_assert(kE2Threads == kFinishThreads, "one block size for the fused kernel");
__global__ __launch_bounds__(kE2Threads) void k_expand_finish(E2Params p, int step, int32_t* parent_out,
                                                              int32_t* tokens_out, int32_t* num_nodes,
                                                              int32_t* q_row_out, int32_t* status_out) {
  expand_body(p, step, nullptr, nullptr);
  __syncthreads();
  finish_body(p, parent_out, tokens_out, num_nodes, q_row_out, status_out);
}

// ---------------------------------------------------------------- launchers
sv_status launch_eagle2_begin(const sv_eagle2_cfg* c, void* state, const int32_t* root_tokens, hipStream_t s) {
  const E2Layout L = eagle2_layout(c);
  const E2Params p = make_params(c, L, state);
  if (c->B == 0) return SV_OK;
  hipLaunchKernelGGL(k_e2_begin, dim3((c->B + 255) / 256), dim3(256), 0, s, p, root_tokens);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) { set_error("eagle2 begin launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  return SV_OK;
}

sv_status launch_eagle2_expand(const sv_eagle2_cfg* c, void* state, int step, const float* q, int32_t* frontier,
                               int32_t* frontier_tokens, hipStream_t s) {
  const E2Layout L = eagle2_layout(c);
  const E2Params p = make_params(c, L, state);
  if (c->B == 0) return SV_OK;
  const int jrows = step == 0 ? 1 : c->k;
  hipLaunchKernelGGL(k_row_topk, dim3(c->B * jrows * L.nsplit), dim3(kTopkThreads), 0, s, p, q, jrows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) { set_error("eagle2 top-k launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  hipLaunchKernelGGL(k_expand, dim3(c->B), dim3(kE2Threads), 0, s, p, step, frontier, frontier_tokens);
  e = hipGetLastError();
  if (e != hipSuccess) { set_error("eagle2 expand launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  return SV_OK;
}

sv_status launch_eagle2_expand_finish(const sv_eagle2_cfg* c, void* state, int step, const float* q, int32_t* parent,
                                      int32_t* tokens, int32_t* num_nodes, int32_t* q_row, int32_t* status,
                                      hipStream_t s) {
  const E2Layout L = eagle2_layout(c);
  const E2Params p = make_params(c, L, state);
  if (c->B == 0) return SV_OK;
  const int jrows = step == 0 ? 1 : c->k;
  hipLaunchKernelGGL(k_row_topk, dim3(c->B * jrows * L.nsplit), dim3(kTopkThreads), 0, s, p, q, jrows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) { set_error("eagle2 top-k launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  hipLaunchKernelGGL(k_expand_finish, dim3(c->B), dim3(kE2Threads), 0, s, p, step, parent, tokens, num_nodes, q_row,
                     status);
  e = hipGetLastError();
  if (e != hipSuccess) { set_error("eagle2 expand+finish launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  return SV_OK;
}

sv_status launch_eagle2_finish(const sv_eagle2_cfg* c, const void* state, int32_t* parent, int32_t* tokens,
                               int32_t* num_nodes, int32_t* q_row, int32_t* status, hipStream_t s) {
  const E2Layout L = eagle2_layout(c);
  const E2Params p = make_params(c, L, const_cast<void*>(state));
  if (c->B == 0) return SV_OK;
  hipLaunchKernelGGL(k_finish, dim3(c->B), dim3(kFinishThreads), 0, s, p, parent, tokens, num_nodes, q_row, status);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) { set_error("eagle2 finish launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  return SV_OK;
}

}  // namespace sv
