// Two-stage draft LM head ([EAGLE-4 blog], sections "EAGLE Efficient LM
// Head", "A training-free version: Freq-aware SVD", "A variant based on Local
// Top-k"): a low-rank head A B scores the whole vocabulary cheaply, each tile
// of the shuffled vocabulary keeps its own best candidates while the scores
// are still on chip, and the full head W recomputes exact logits for the
// candidates only.
//
//   k_head_u       u = B h: one 16 x 16 (rank x position) MFMA tile per
//                  workgroup of 16 waves, each over a sixteenth of the hidden
//                  dim with 8 k-steps of loads in flight; the waves' partial
//                  tiles are summed in LDS in a fixed order and rounded to
//                  bf16 (the operand of the next stage).
//   k_head_u_small the same for N <= 16 positions (a drafter step) on VALU:
//                  2 rank rows per workgroup, so r / 2 workgroups share B's
//                  read instead of r / 16.
//   k_head_topk    one workgroup per vocabulary tile: scores^T = A_tile u^T on
//                  MFMA into LDS (never written to HBM), each wave loading its
//                  two row blocks and the shared u fragments in one batch;
//                  then per position the k_tile best rows by rounds of a DPP
//                  wave maximum over 64-bit keys (order-preserving score bits
//                  above the complement of the row), written as token ids
//                  through the shuffle (read with the first loads).
//   k_head_logits  one wave per (position, candidate): the candidate's row of
//                  W gathered once and dotted with h in float32.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16): lane l holds A[l % 16][8 (l / 16)
// .. + 7] and B[8 (l / 16) .. + 7][l % 16], and receives D[4 (l / 16) + i][l %
// 16], i = 0..3.  Both operands are rows of row-major tensors read as 16-byte
// runs, so they load straight from global memory.
#include "sv_internal.h"

namespace sv {

constexpr int kHeadMaxK = 8;      // candidates per tile
constexpr int kHeadTileMax = 256; // vocabulary rows per tile

constexpr int kUWaves = 16;       // stage-1 waves per workgroup (MFMA kernel)
constexpr int kUSmallN = 16;      // positions up to which stage 1 runs on VALU
constexpr int kURows = 2;         // rank rows per workgroup of the VALU kernel
constexpr int kUThreads = 512;    // threads of the VALU kernel
constexpr int kTopkWaves = 8;     // stage-2 waves per workgroup

struct HeadParams {
  int N, d, r, n, tile, k_tile, n_tiles;
  const __bf16* h;
  const __bf16* B;
  const __bf16* A;
  const int32_t* perm;
  const __bf16* W;
  __bf16* u;
  int32_t* cand_ids;
  float* cand_logits;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline bf16x8 load8(const __bf16* p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p)); }

__device__ inline uint16_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// An order-preserving unsigned image of a float32 (larger float -> larger).
__device__ inline uint32_t sortable(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------- stage 1
// grid (r / 16, ceil(N / 16)); wave w sums k-steps [w ksteps / 16, (w + 1) ksteps / 16).
__global__ __launch_bounds__(64 * kUWaves) void k_head_u(HeadParams p) {
  __shared__ f32x4 part_s[kUWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * 16, n0 = blockIdx.y * 16;
  const int row = r0 + (lane & 15);              // rank row of the A operand
  const int pos = n0 + (lane & 15);              // position of the B operand
  const int kg = lane >> 4;
  const bool pos_ok = pos < p.N;
  const int ksteps = p.d / 32;
  const int s_begin = (int)((long)ksteps * wave / kUWaves);
  const int s_end = (int)((long)ksteps * (wave + 1) / kUWaves);
  const __bf16* brow = p.B + (size_t)row * p.d + 8 * kg;
  const __bf16* hrow = p.h + (size_t)(pos_ok ? pos : 0) * p.d + 8 * kg;
  const bf16x8 zero = {};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = s_begin; s0 < s_end; s0 += 8) {
    bf16x8 a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bool ok = s0 + s < s_end;
      a[s] = ok ? load8(brow + 32 * (s0 + s)) : zero;
      b[s] = ok && pos_ok ? load8(hrow + 32 * (s0 + s)) : zero;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s0 + s < s_end) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc, 0, 0, 0);
  }
  part_s[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && pos_ok) {
    f32x4 t = part_s[0][lane];
#pragma unroll
    for (int w = 1; w < kUWaves; ++w) t += part_s[w][lane];
    uint16_t* u = reinterpret_cast<uint16_t*>(p.u) + (size_t)pos * p.r + r0 + 4 * kg;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = bf16_rne(t[i]);
  }
}

// Few positions (N <= 16): u = B h is a few MFLOP, and the MFMA kernel above
// has only r / 16 workgroups to spread B's read over.  Here each workgroup
// takes 2 rank rows for every position, so r / 2 workgroups read B.  Thread t
// takes the 8-element groups t, t + 512, ... of the hidden dim, two groups per
// batch of loads, with bf16 pair dots accumulated in float32.  The partial
// sums are added in a fixed order: a shuffle butterfly within each wave,
// then the 8 waves in turn; u is rounded to bf16 once.
__device__ inline float dot8(bf16x8 a, bf16x8 b, float c) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 x = {a[2 * e], a[2 * e + 1]};
    const bf16x2 y = {b[2 * e], b[2 * e + 1]};
    c = __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false);
  }
  return c;
}

__global__ __launch_bounds__(kUThreads) void k_head_u_small(HeadParams p) {
  __shared__ float red_s[kUThreads / 64][kURows * kUSmallN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * kURows;
  const bf16x8 zero = {};
  float acc[kURows][kUSmallN];
#pragma unroll
  for (int rr = 0; rr < kURows; ++rr)
#pragma unroll
    for (int n = 0; n < kUSmallN; ++n) acc[rr][n] = 0.f;
  constexpr int kStep = 8 * kUThreads;                 // hidden-dim elements per group sweep
  for (int k0 = 8 * tid; k0 < p.d; k0 += 2 * kStep) {
    bf16x8 b[2][kURows], h[2][kUSmallN];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int k = k0 + g * kStep;
      const bool ok = k < p.d;
#pragma unroll
      for (int rr = 0; rr < kURows; ++rr) b[g][rr] = ok ? load8(p.B + (size_t)(r0 + rr) * p.d + k) : zero;
#pragma unroll
      for (int n = 0; n < kUSmallN; ++n) h[g][n] = ok && n < p.N ? load8(p.h + (size_t)n * p.d + k) : zero;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int rr = 0; rr < kURows; ++rr)
#pragma unroll
        for (int n = 0; n < kUSmallN; ++n)
          if (n < p.N) acc[rr][n] = dot8(b[g][rr], h[g][n], acc[rr][n]);
  }
#pragma unroll
  for (int rr = 0; rr < kURows; ++rr)
#pragma unroll
    for (int n = 0; n < kUSmallN; ++n) {
      if (n >= p.N) continue;
      float v = acc[rr][n];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) red_s[wave][rr * kUSmallN + n] = v;
    }
  __syncthreads();
  if (tid < kURows * kUSmallN) {
    const int rr = tid / kUSmallN, n = tid % kUSmallN;
    if (n < p.N) {
      float t = red_s[0][tid];
#pragma unroll
      for (int w = 1; w < kUThreads / 64; ++w) t += red_s[w][tid];
      reinterpret_cast<uint16_t*>(p.u)[(size_t)n * p.r + r0 + rr] = bf16_rne(t);
    }
  }
}

// ---------------------------------------------------------------- stage 2
// grid (n_tiles, ceil(N / 16)); 8 waves; wave w scores the tile's 16-row
// blocks w and w + 8, loading both blocks' A fragments and the u fragments
// they share in one batch (per 8 k-steps).  The tile's token ids are read
// with them and staged in LDS, so the selection needs no further global
// read.
__global__ __launch_bounds__(64 * kTopkWaves) void k_head_topk(HeadParams p) {
  constexpr int kRB = kHeadTileMax / 16 / kTopkWaves;   // row blocks per wave
  __shared__ float sc_s[kHeadTileMax][17];      // [row in tile][position], padded
  __shared__ int perm_s[kHeadTileMax];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int n0 = blockIdx.y * 16;
  const int lo = t * p.tile;
  const int rows = min(p.tile, p.n - lo);
  const int kg = lane >> 4;
  const int pos = n0 + (lane & 15);
  const bool pos_ok = pos < p.N;
  const int ksteps = p.r / 32;
  static_assert(kHeadTileMax <= 64 * kTopkWaves, "one token id per thread");
  const int prm = tid < rows ? p.perm[lo + tid] : 0;   // to LDS once the loads below are in
  const __bf16* urow = p.u + (size_t)(pos_ok ? pos : 0) * p.r + 8 * kg;
  const __bf16* arow[kRB];
  bool row_ok[kRB];
#pragma unroll
  for (int q = 0; q < kRB; ++q) {
    const int row = (wave + kTopkWaves * q) * 16 + (lane & 15);
    row_ok[q] = row < rows;
    arow[q] = p.A + (size_t)(lo + (row_ok[q] ? row : 0)) * p.r + 8 * kg;
  }
  const bf16x8 zero = {};
  f32x4 acc[kRB];
#pragma unroll
  for (int q = 0; q < kRB; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ksteps; s0 += 8) {
    bf16x8 a[kRB][8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bool ok = s0 + s < ksteps;
      b[s] = ok && pos_ok ? load8(urow + 32 * (s0 + s)) : zero;
#pragma unroll
      for (int q = 0; q < kRB; ++q) a[q][s] = ok && row_ok[q] ? load8(arow[q] + 32 * (s0 + s)) : zero;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s0 + s < ksteps)
#pragma unroll
        for (int q = 0; q < kRB; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q][s], b[s], acc[q], 0, 0, 0);
  }
  if (tid < rows) perm_s[tid] = prm;
#pragma unroll
  for (int q = 0; q < kRB; ++q) {
    const int rb = wave + kTopkWaves * q;
    if (rb * 16 < rows)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc_s[rb * 16 + 4 * kg + i][lane & 15] = acc[q][i];
  }
  __syncthreads();
  // per position: the k_tile best rows (score descending, then row ascending)
  const int npos = min(16, p.N - n0);
  const int kk = min(p.k_tile, rows);
  for (int q = wave; q < npos; q += kTopkWaves) {
    const int i = n0 + q;
    uint64_t key[kHeadTileMax / 64];
#pragma unroll
    for (int j = 0; j < kHeadTileMax / 64; ++j) {
      const int row = lane + 64 * j;
      key[j] = row < rows ? (((uint64_t)sortable(sc_s[row][q]) << 32) | (uint32_t)~row) : 0;
    }
    int32_t* ids = p.cand_ids + (size_t)i * p.n_tiles * p.k_tile + (size_t)t * p.k_tile;
    for (int c = 0; c < p.k_tile; ++c) {
      int id = -1;
      if (c < kk) {
        uint64_t m = 0;
#pragma unroll
        for (int j = 0; j < kHeadTileMax / 64; ++j) m = key[j] > m ? key[j] : m;
        const uint64_t best = wave_max_u64_dpp(m);
        const int row = (int)~(uint32_t)best;
#pragma unroll
        for (int j = 0; j < kHeadTileMax / 64; ++j) key[j] = key[j] == best ? 0 : key[j];
        id = perm_s[row];
      }
      if (lane == 0) ids[c] = id;
    }
  }
}

// ---------------------------------------------------------------- stage 3
// one wave per (position, candidate); 4 waves per workgroup.
__global__ __launch_bounds__(256) void k_head_logits(HeadParams p) {
  const int lane = threadIdx.x & 63;
  const size_t C = (size_t)p.n_tiles * p.k_tile;
  const size_t job = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (job >= (size_t)p.N * C) return;
  const int i = (int)(job / C);
  const int id = p.cand_ids[job];
  float acc = 0.f;
  if (id >= 0 && id < p.n) {
    const __bf16* w = p.W + (size_t)id * p.d;
    const __bf16* h = p.h + (size_t)i * p.d;
    for (int k = 8 * lane; k < p.d; k += 512) {
      const bf16x8 a = load8(w + k);
      const bf16x8 b = load8(h + k);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) p.cand_logits[job] = id >= 0 ? acc : 0.f;
}

// ---------------------------------------------------------------- launch
sv_status launch_draft_head(const sv_head_args* a, hipStream_t s) {
  HeadParams p{};
  p.N = a->N; p.d = a->d; p.r = a->r; p.n = a->n; p.tile = a->tile; p.k_tile = a->k_tile;
  p.n_tiles = (a->n + a->tile - 1) / a->tile;
  p.h = static_cast<const __bf16*>(a->h);
  p.B = static_cast<const __bf16*>(a->B);
  p.A = static_cast<const __bf16*>(a->A_sh);
  p.perm = a->perm;
  p.W = static_cast<const __bf16*>(a->W);
  p.u = static_cast<__bf16*>(a->u);
  p.cand_ids = a->cand_ids;
  p.cand_logits = a->cand_logits;
  if (p.N == 0) return SV_OK;
  const int pos_tiles = (p.N + 15) / 16;
  if (p.N <= kUSmallN)
    hipLaunchKernelGGL(k_head_u_small, dim3(p.r / kURows), dim3(kUThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_head_u, dim3(p.r / 16, pos_tiles), dim3(64 * kUWaves), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) { set_error("draft head stage 1 launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  hipLaunchKernelGGL(k_head_topk, dim3(p.n_tiles, pos_tiles), dim3(64 * kTopkWaves), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) { set_error("draft head stage 2 launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  const size_t jobs = (size_t)p.N * p.n_tiles * p.k_tile;
  hipLaunchKernelGGL(k_head_logits, dim3((unsigned)((jobs + 3) / 4)), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) { set_error("draft head stage 3 launch: %s", hipGetErrorString(e)); return SV_E_HIP; }
  return SV_OK;
}

}  // namespace sv
