// Tree attention for verification: every tree position attends to its
// sequence's KV-cache prefix and to its own tree ancestors (and itself).
//
// [EAGLE article] sec. 1.3 "Verification": the target scores the whole draft
// tree in one forward pass using tree attention.  [Spec-decoding lesson]
// "Tree-attention verification": one forward, one matmul; the topology mask
// only adds a few KV entries.
//
// bf16 kernel (gfx950 MFMA).  Work unit = (sequence b, KV head, block of query
// rows, range of keys).  Query rows of one KV head are the (node t, head g)
// pairs, row r = t * G + g, so the G heads sharing a KV head are packed into
// the MFMA N dimension next to each other.  Per wave, NT tiles of 16 rows;
// per workgroup, NW waves share each key block staged in LDS.
//
//   scores   S^T[key][row] = K[key] . Q[row]     v_mfma_f32_16x16x32_bf16,
//            A = K rows from LDS, B = Q held in registers for the whole run;
//   softmax  online, fp32: the MFMA yields raw dot products of the bf16 q and
//            k as stored, and the score scale times log2(e) is applied to them
//            in fp32 right before exp2; each row's offset is only raised when
//            a block's row sum of P shows a score more than 64 (log2 units)
//            past it, so the O rescale is rare and every P stays below 2^64;
//   output   O^T[d][row] += V^T[d][key] P^T[key][row]: B = P taken straight
//            from the score registers; A = V^T read from the row-major V tile
//            with ds_read_b64_tr_b16 (each 16-lane group gathers 4 keys x 16
//            dims and gets them transposed), in the same key permutation.
//
// Keys of one (b, KV head) are numbered 0 .. L_b + T_b - 1: first the cache
// prefix, then the tree tokens; keys >= L_b are visible to row (t, g) iff bit
// (key - L_b) of anc[b][t] is set.  With several key ranges per row
// (lsplit > 1), each range writes (m, l, O) partials and k_attn_combine merges
// them with the log-sum-exp rule.
#include "sv_internal.h"

#include <algorithm>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

namespace sv {

constexpr int BK = 32;  // keys per block

struct AttnParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* k_cache;
  const void* v_cache;
  const int32_t* prefix_len;
  const int32_t* num_nodes;
  const int32_t* status;
  const uint64_t* anc;
  void* out;
  float* part_o;   // [B][T_max][Hq][lstride][D]: the key ranges' partials, first n in use
  float* part_ml;  // [B][T_max][Hq][lstride][2]
  int32_t* dyn_ls; // the key split n a sizes-driven plan chose (read by the merge)
  int B, T_max, Hq, Hkv, G, L_max, W;
  int rows_per_wg, msplit, lsplit, chunk;
  int lstride;     // partials per row the workspace holds: lsplit, or ls_cap with dyn
  int dyn, ls_cap, keys_max;   // sizes-driven plan (see decode_work)
  int remap;
  float scale_log2;  // score scale * log2(e), applied in fp32
  float raise_raw;   // 8 / scale_log2: the offset-raise bound in raw dot-product units
};

// Workgroups are dispatched round-robin over the 8 XCDs (block i runs on XCD
// i % 8).  With remap set (grid a multiple of 8) consecutive logical blocks --
// the row blocks that read the same keys -- are placed on the same XCD, one
// after another, so their shared K/V tiles are served from that XCD's L2.
__device__ inline int logical_block(int remap) {
  const int i = blockIdx.x;
  if (!remap) return i;
  const int per = gridDim.x >> 3;
  return (i & 7) * per + (i >> 3);
}

// Row blocks (of rows_per_wg query rows) of a sequence that hold valid rows.
__device__ inline int seq_row_blocks(const AttnParams& p, int st, int Tb, int Lb) {
  const bool ok = st == SV_TREE_OK && Tb >= 1 && Tb <= p.T_max && Lb >= 0 && Lb <= p.L_max;
  return ok ? (Tb * p.G + p.rows_per_wg - 1) / p.rows_per_wg : 0;
}
__device__ inline int seq_row_blocks(const AttnParams& p, int b) {
  return seq_row_blocks(p, p.status[b], p.num_nodes[b], p.prefix_len[b]);
}

// The work of logical block lb: (unit = sequence * Hkv + KV head, row block,
// key range) and the key range's length.  A plan made on the host from
// T_max gives every (unit, row block) the same key split, so with trees of
// different sizes some row blocks hold no valid row and their workgroups
// idle while the full ones set the time.  With p.dyn the workgroups read
// the sequences' sizes and share out only the row blocks that hold valid
// rows, numbered densely (unit by unit, then key range, then row block, so
// consecutive workgroups read the same keys), with the key split as fine as
// the grid allows (at most ls_cap, ranges of at least 4 key blocks).  Every
// workgroup derives the same plan from the same sizes, and logical block 0
// records the split for the merge.  Returns false when lb has no work.
struct AttnWork {
  int ms_i, ls_i, unit, chunk, nls;   // nls: the key split
  int st, Tb, Lb;                     // the sequence's status and sizes, when the decode read them
  bool have_seq;
};
__device__ inline bool decode_work(const AttnParams& p, int lb, AttnWork& wk) {
  if (!p.dyn) {
    wk.ms_i = lb % p.msplit;
    const int rest = lb / p.msplit;
    wk.ls_i = rest % p.lsplit;
    wk.unit = rest / p.lsplit;
    wk.chunk = p.chunk;
    wk.nls = p.lsplit;
    wk.have_seq = false;
    return true;
  }
  const int lane = threadIdx.x & 63;
  // Valid row blocks of the first 64 sequences, one per lane, and their
  // inclusive scan; with more sequences, the rest add to the total in a
  // first pass and are scanned again below.
  const int st0 = lane < p.B ? p.status[lane] : 0;
  const int tb0 = lane < p.B ? p.num_nodes[lane] : 0;
  const int lb0 = lane < p.B ? p.prefix_len[lane] : 0;
  const int rb0 = lane < p.B ? seq_row_blocks(p, st0, tb0, lb0) : 0;
  int scan0 = rb0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(scan0, off);
    if (lane >= off) scan0 += y;
  }
  int rbs = __shfl(scan0, 63);   // valid row blocks per KV head, summed over the sequences
  for (int b0 = 64; b0 < p.B; b0 += 64) {
    int v = b0 + lane < p.B ? seq_row_blocks(p, b0 + lane) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    rbs += v;
  }
  const int R = __builtin_amdgcn_readfirstlane(rbs * p.Hkv);   // <= the grid: fits in 32 bits
  int nls = R > 0 ? (int)gridDim.x / R : 1;
  nls = nls < 1 ? 1 : nls;
  nls = nls > p.ls_cap ? p.ls_cap : nls;
  const int lmax = p.keys_max / (4 * BK);
  nls = nls > lmax ? (lmax < 1 ? 1 : lmax) : nls;
  wk.chunk = ((p.keys_max + nls - 1) / nls + 63) / 64 * 64;
  wk.nls = nls;
  if (lb == 0 && threadIdx.x == 0) *p.dyn_ls = nls;
  if (lb >= R * nls) return false;
  // the sequence whose items (row blocks x KV heads x key ranges) hold lb
  const int per = p.Hkv * nls;
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int rb = b0 == 0 ? rb0 : (b0 + lane < p.B ? seq_row_blocks(p, b0 + lane) : 0);
    int incl = rb;
    if (b0 == 0) {
      incl = scan0;
    } else {
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
    }
    const int hi = base + incl * per, lo = hi - rb * per;
    const uint64_t hit = __ballot(rb > 0 && lo <= lb && lb < hi);
    if (hit) {
      const int l = (int)__ffsll((unsigned long long)hit) - 1;
      const int hrb = __shfl(rb, l);
      const int r = lb - __shfl(lo, l);
      const int kvh = r / (hrb * nls);
      const int idx = r % (hrb * nls);
      wk.ls_i = idx / hrb;
      wk.ms_i = idx % hrb;
      wk.unit = (b0 + l) * p.Hkv + kvh;
      wk.have_seq = b0 == 0;   // lane l of the first 64 holds the sequence's own values
      wk.st = __shfl(st0, l);
      wk.Tb = __shfl(tb0, l);
      wk.Lb = __shfl(lb0, l);
      return true;
    }
    base += __shfl(incl, 63) * per;
  }
  return false;
}

// Max over the 4 lanes holding one tile column (lanes c, c+16, c+32,
// c+48), with the gfx950 row-swap permutes: permlane16_swap exchanges the odd
// 16-lane rows of one operand with the even rows of the other, permlane32_swap
// the upper half with the lower half; with both operands = v the two results
// hold the partner values.
__device__ inline float col_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte staging unit
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte rows addressed by lanes 4k + i / 4, k = 0..3.
__device__ inline bf16x4 lds_read_tr16(const __bf16* p) {
  typedef __bf16 __attribute__((address_space(3))) lds_bf16;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 __attribute__((address_space(3)))*)(
      (lds_bf16*)(p)));
}

// Direct global -> LDS copy, 16 bytes per lane (global_load_lds_dwordx4): lane
// i of the wave writes LDS bytes [m0 + 16 i, m0 + 16 i + 16).  Issued as
// inline asm so that the compiler's wait-count bookkeeping (which would wait
// for every outstanding copy before any LDS read) stays out of the pipeline;
// the kernel waits for its copies itself with s_waitcnt vmcnt.  The asm sets
// m0 and says so, so the compiler keeps nothing of its own in m0 across it.
__device__ inline void copy16_to_lds(const void* gptr, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr)) : "memory", "m0");
}
// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order), then join the workgroup barrier.
template <int N>
__device__ inline void wait_copies_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}
__device__ inline uint32_t lds_byte_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// K/V tiles are stored unpadded, BK rows of D elements, with the 16-byte
// segments of row r permuted by XOR with kv_swizzle(r): the XOR of one mask
// per set bit among the row's low 4 bits (a linear map).  The masks were
// chosen by timing the kernel's two LDS read patterns on gfx950 for every
// such map: with these, a score-fragment read (16 rows, 4 segments, 16 bytes
// per lane) runs as fast as a contiguous 16-byte read, 23.4 against 32.3
// clock ticks per instruction for 4 waves of a CU with the previous map
// (built for 64 banks read 16 lanes at a time), and the transposed V read
// stays at its own floor.
template <int D>
__device__ inline int kv_swizzle(int r) {
  constexpr int m0 = D == 128 ? 8 : 4, m1 = D == 128 ? 2 : 5, m2 = D == 128 ? 4 : 2, m3 = D == 128 ? 13 : 6;
  return ((r & 1) ? m0 : 0) ^ ((r & 2) ? m1 : 0) ^ ((r & 4) ? m2 : 0) ^ ((r & 8) ? m3 : 0);
}

// Copy-ring depth: key blocks in flight ahead of the one being computed is
// kStages - 1.
constexpr int kStages = 4;

// Work unit: (sequence b, KV head, block of query rows, range of keys); one
// workgroup of NW waves per unit, one barrier per key block.
template <int D, int NT, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_bf16(AttnParams p) {
  constexpr int NTHR = NW * 64;
  constexpr int TILE = BK * D;            // elements of one K or V tile
  constexpr int STAGE = 2 * TILE;         // K tile then V tile
  constexpr int SEGS = D / 8;             // 16-byte segments per row
  constexpr int RPI = 64 / SEGS;          // rows one copy instruction fills
  constexpr int IPT = BK / RPI;           // copy instructions per tile
  static_assert(IPT % NW == 0, "copy split");
  constexpr int IPW = IPT / NW;           // per wave and tile
  constexpr int CPB = 2 * IPW;            // copies per wave and key block (K and V)
  constexpr int DK = D / 32;              // MFMA k-steps over the head dim
  constexpr int DT = D / 16;              // 16-row output tiles over the head dim

  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);
  uint64_t* anc_s = reinterpret_cast<uint64_t*>(smem_raw + kStages * STAGE * sizeof(__bf16));

  const int lb = logical_block(p.remap);
  AttnWork wk;
  if (!decode_work(p, lb, wk)) return;
  // the same in every lane: scalar registers, not vector ones held through the loop
  const int ms_i = __builtin_amdgcn_readfirstlane(wk.ms_i);
  const int ls_i = __builtin_amdgcn_readfirstlane(wk.ls_i);
  const int unit = __builtin_amdgcn_readfirstlane(wk.unit);
  wk.chunk = __builtin_amdgcn_readfirstlane(wk.chunk);
  const int nls = __builtin_amdgcn_readfirstlane(wk.nls);
  const int b = unit / p.Hkv;
  const int kvh = unit % p.Hkv;
  const int G = p.G;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = lane & 15;   // column (query row) within a 16x16 tile
  const int g = lane >> 4;   // lane group

  const bool have_seq = __builtin_amdgcn_readfirstlane(wk.have_seq ? 1 : 0) != 0;
  const int Tb = have_seq ? __builtin_amdgcn_readfirstlane(wk.Tb) : p.num_nodes[b];
  const int Lb = have_seq ? __builtin_amdgcn_readfirstlane(wk.Lb) : p.prefix_len[b];
  const int st_b = have_seq ? __builtin_amdgcn_readfirstlane(wk.st) : p.status[b];
  // a sequence whose tree is invalid, or whose sizes are out of range, is
  // written as zeros
  const bool seq_ok = st_b == SV_TREE_OK && Tb >= 1 && Tb <= p.T_max && Lb >= 0 && Lb <= p.L_max;
  const int row0 = ms_i * p.rows_per_wg;
  const int valid_rows = seq_ok ? Tb * G : 0;
  const int kbeg = ls_i * wk.chunk;
  const int kend = min(kbeg + wk.chunk, Lb + Tb);

  const __bf16* qp = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* kc = reinterpret_cast<const __bf16*>(p.k_cache) + ((size_t)b * p.Hkv + kvh) * p.L_max * D;
  const __bf16* vc = reinterpret_cast<const __bf16*>(p.v_cache) + ((size_t)b * p.Hkv + kvh) * p.L_max * D;
  const __bf16* kn = reinterpret_cast<const __bf16*>(p.k_new) + ((size_t)b * p.T_max * p.Hkv + kvh) * D;
  const __bf16* vn = reinterpret_cast<const __bf16*>(p.v_new) + ((size_t)b * p.T_max * p.Hkv + kvh) * D;
  const size_t new_stride = (size_t)p.Hkv * D;  // elements between consecutive tree tokens
  const uint32_t new_stride32 = (uint32_t)new_stride;

  // rows owned by this lane (one per 16-row tile)
  int rrow[NT];
  bool rvalid[NT];
#pragma unroll
  for (int qt = 0; qt < NT; ++qt) {
    rrow[qt] = row0 + (wave * NT + qt) * 16 + c;
    rvalid[qt] = rrow[qt] < valid_rows;
  }

  const bool wave_active = row0 + wave * NT * 16 < valid_rows;
  if (row0 >= valid_rows || kbeg >= kend) {
    // Nothing to attend for this workgroup: write zeros (single range) or an
    // empty partial (m = -inf, l = 0, O = 0).
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) {
      const int r = rrow[qt];
      if (r >= p.T_max * G) continue;
      const int t = r / G, h = kvh * G + r % G;
      const size_t orow = ((size_t)b * p.T_max + t) * p.Hq + h;
      if (p.lsplit == 1) {
        __bf16* o = reinterpret_cast<__bf16*>(p.out) + orow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(o + dt * 16 + 4 * g) = make_uint2(0u, 0u);
      } else if (rvalid[qt]) {
        float* po = p.part_o + (orow * p.lstride + ls_i) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (g == 0) {
          float* pm = p.part_ml + (orow * p.lstride + ls_i) * 2;
          pm[0] = -INFINITY;
          pm[1] = 0.f;
        }
      }
    }
    return;
  }

  // ancestor rows of this sequence -> LDS
  const int W = p.W;
  for (int i = tid; i < p.T_max * W; i += NTHR) anc_s[i] = p.anc[(size_t)b * p.T_max * W + i];

  // queries -> registers (B operand of the score MFMA) exactly as stored: the
  // score MFMA then yields raw dot products with fp32 accumulation, and the
  // scale is applied to those in fp32.  (Rounding scale * log2(e) * q to bf16
  // instead would put a relative error of 2^-9 on every product, an exponent
  // error that grows with the score: at score spreads of a peaked softmax it
  // moves weights by several percent.)
  bf16x8 qreg[NT][DK];
#pragma unroll
  for (int qt = 0; qt < NT; ++qt) {
    const int r = rrow[qt];
    if (rvalid[qt]) {
      const int t = r / G, h = kvh * G + r % G;
      const __bf16* src = qp + (((size_t)b * p.T_max + t) * p.Hq + h) * D + 8 * g;
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) qreg[qt][kk] = *reinterpret_cast<const bf16x8*>(src + 32 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) qreg[qt][kk] = bf16x8{};
    }
  }

  // acc: O^T tiles; lsum: the row sums of P.  Each block's row sums come
  // from an MFMA with an all-ones A operand (every element of its result
  // holds the column's sum), which also serves as the overflow test below.
  // mu: the running offset of the lane's row in raw dot-product units,
  // subtracted by the score MFMA itself (its accumulator starts at
  // cinit = -mu); valid once a visible key has set it.  With c = scale *
  // log2(e), P = 2^(c (dot - mu)); a raise puts the new offset at the block's
  // maximum when that exceeds the old one by more than 8 / c.
  f32x4 acc[NT][DT], cinit[NT];
  float mu[NT], lsum[NT];
  bool valid[NT];
#pragma unroll
  for (int qt = 0; qt < NT; ++qt) {
    mu[qt] = 0.f;
    valid[qt] = false;
    cinit[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

  // ---- staging: a ring of kStages (K, V) tile pairs in LDS, filled
  // by direct copies.  Copy instruction j of wave w fills tile rows
  // [(w IPW + j) RPI, + RPI); lane l of it loads row l / SEGS, segment
  // (l % SEGS) ^ swizzle(row).  Keys past the range end are clamped to the
  // last valid key (their scores are masked to -inf, so those rows of V are
  // weighted by exactly 0).
  // (the lane's copy coordinates are recomputed per block: a few VALU
  // operations instead of registers held through the loop)
  auto copy_row = [&](int j) { return (wave * IPW + j) * RPI + lane / SEGS; };
  auto copy_seg = [&](int j) { return (uint32_t)(((lane % SEGS) ^ kv_swizzle<D>(copy_row(j))) * 8); };
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_byte_address(smem));
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane((uint32_t)(wave * IPW * 1024));
  const int fast_end = min(Lb, kend);   // blocks ending here or before are all cache keys
  const uint64_t kc_addr = reinterpret_cast<uint64_t>(kc), vc_addr = reinterpret_cast<uint64_t>(vc);
  const uint64_t kn_addr = reinterpret_cast<uint64_t>(kn), vn_addr = reinterpret_cast<uint64_t>(vn);
  auto issue_block = [&](int blk, int stage) {
    const uint32_t kl = lds0 + (uint32_t)(stage * STAGE * 2) + wave_lds;
    const uint32_t vl = kl + TILE * 2;
    if (blk + BK <= fast_end) {
      // whole block inside the cache prefix: one uniform base, fixed lane offsets
      const __bf16* kb = kc + (size_t)blk * D;
      const __bf16* vb = vc + (size_t)blk * D;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const uint32_t off = (uint32_t)(copy_row(j) * D) + copy_seg(j);
        copy16_to_lds(kb + off, kl + j * 1024);
        copy16_to_lds(vb + off, vl + j * 1024);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int jr = blk + copy_row(j);
      const int jj = jr < kend ? jr : kend - 1;
      const bool in_cache = jj < Lb;
      const uint64_t loc = 2ull * ((in_cache ? (uint32_t)jj * D : (uint32_t)(jj - Lb) * new_stride32) + copy_seg(j));
      const uint64_t ka = (in_cache ? kc_addr : kn_addr) + loc;
      const uint64_t va = (in_cache ? vc_addr : vn_addr) + loc;
      copy16_to_lds(reinterpret_cast<const void*>(ka), kl + j * 1024);
      copy16_to_lds(reinterpret_cast<const void*>(va), vl + j * 1024);
    }
  };

  // LDS element offsets of this lane's fragment reads (swizzled):
  //   K: row 16 kt + c, segment 4 kk + g        (score MFMA A operand);
  //   V: row 4 g + c / 4 (+16), dims 16 dt + 4 (c % 4) .. +3 (transposed read).
  uint32_t koff[DK], voff[DT];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) koff[kk] = (uint32_t)(c * D + (((4 * kk + g) ^ kv_swizzle<D>(c)) * 8));
  {
    const int rv = 4 * g + (c >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      voff[dt] = (uint32_t)(rv * D + (((2 * dt + ((c >> 1) & 1)) ^ kv_swizzle<D>(rv)) * 8) + (c & 1) * 4);
  }

  // The query loads complete here: the empty asm needs the registers, so the
  // compiler waits for them once, not at their first use inside the loop
  // (where its wait would also cover the outstanding copies).
#pragma unroll
  for (int qt = 0; qt < NT; ++qt)
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) asm volatile("" : "+v"(qreg[qt][kk]));

  const int nblk = (kend - kbeg + BK - 1) / BK;
  __syncthreads();   // ancestor rows in LDS
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < nblk) issue_block(kbeg + i * BK, i);

  // ---- scores S^T of key block n (2 sub-tiles of 16 keys), minus mu, masked
  f32x4 s[NT][2];
  auto scores = [&](int n) {
    const int blk = kbeg + n * BK;
    const __bf16* ks = smem + (n % kStages) * STAGE;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + 16 * kt * D + koff[kk]);
#pragma unroll
        for (int qt = 0; qt < NT; ++qt)
          s[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, qreg[qt][kk], kk == 0 ? cinit[qt] : s[qt][kt], 0, 0, 0);
      }
    }
    // mask: keys past the range end, and tree keys that are not ancestors.
    // Visibility of the block's 32 keys for this lane's row, as one word:
    // bit o <=> key blk + o is a prefix key, or a tree key whose node is an
    // ancestor-or-self of the row's node, and lies before kend.
    if (blk + BK > Lb || blk + BK > kend) {
      const int n0 = blk - Lb;                      // node index of the block's first key
      const uint32_t range_bits = (kend - blk >= 32) ? 0xFFFFFFFFu : ((1u << (kend - blk)) - 1u);
      const uint32_t prefix_bits = (n0 >= 0) ? 0u : (-n0 >= 32 ? 0xFFFFFFFFu : ((1u << -n0) - 1u));
#pragma unroll
      for (int qt = 0; qt < NT; ++qt) {
        const int t = rrow[qt] / G;
        uint32_t tree_bits = 0u;
        if (rvalid[qt] && n0 + BK > 0) {
          const uint64_t* arow = anc_s + t * W;
          // bits [n0, n0 + 32) of the row (bits below 0 are empty)
          const int lo = n0 < 0 ? 0 : n0;
          const int w = lo >> 6, sh = lo & 63;
          uint64_t bits = arow[w] >> sh;
          if (sh > 32 && w + 1 < W) bits |= arow[w + 1] << (64 - sh);
          tree_bits = (uint32_t)bits;
          if (n0 < 0) tree_bits <<= -n0;            // node 0 sits at key offset -n0
        }
        const uint32_t vm = (prefix_bits | tree_bits) & range_bits;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = 16 * kt + 4 * g + i;
            s[qt][kt][i] = ((vm >> o) & 1u) ? s[qt][kt][i] : -INFINITY;
          }
      }
    }
  };

  // ---- online softmax of s, P packed to bf16 for the PV MFMA and kept in the
  // registers of s[qt][1] (so only s lives from one phase to the next).  The
  // scores already are dot - mu (raw units).  While some row of the wave has
  // no offset yet, the wave forms column maxima and sets (or raises) offsets
  // first.  Otherwise P = 2^(c s) is formed at once and checked through the
  // block's row sums, which the ones-MFMA yields anyway: a row sum above
  // 2^64 (or not finite) means some score exceeded the row's offset by more
  // than 64 / c, and only then is the block scored again and the offsets
  // raised past the block's maximum.  Between raises P stays below 2^64, so
  // fp32 sums of at most 2^31 weights cannot overflow.
  const float c2 = p.scale_log2, thr = p.raise_raw;
  bool all_valid = false;   // wave-uniform: every row of the wave has an offset
  auto raise_offsets = [&]() {
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) {
      const float a0 = fmaxf(fmaxf(s[qt][0][0], s[qt][0][1]), fmaxf(s[qt][0][2], s[qt][0][3]));
      const float a1 = fmaxf(fmaxf(s[qt][1][0], s[qt][1][1]), fmaxf(s[qt][1][2], s[qt][1][3]));
      const float cm = col_max4(fmaxf(a0, a1));   // column max of dot - mu
      // a row without an offset takes the first visible maximum (its
      // accumulators are still zero); a row with one raises it past 8 / c
      const bool raise = valid[qt] ? cm > thr : cm > -INFINITY;
      if (raise) {
        if (valid[qt]) {
          const float alpha = __builtin_amdgcn_exp2f(-cm * c2);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[qt][dt] *= alpha;
          lsum[qt] *= alpha;
        }
        mu[qt] += cm;
        valid[qt] = true;
        cinit[qt] = f32x4{-mu[qt], -mu[qt], -mu[qt], -mu[qt]};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[qt][kt] -= cm;
      }
    }
    bool v = true;
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) v = v && valid[qt];
    all_valid = __all(v);
  };
  f32x4 blk[NT];   // the block's row sums of P
  auto exps = [&]() {
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) {
      float pv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[kt * 4 + i] = __builtin_amdgcn_exp2f(s[qt][kt][i] * c2);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pv[2 * e], pv[2 * e + 1]);
      s[qt][1] = __builtin_bit_cast(f32x4, make_uint4(w[0], w[1], w[2], w[3]));
    }
#pragma unroll
    for (int qt = 0; qt < NT; ++qt)
      blk[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, s[qt][1]),
                                                        f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  };
  auto softmax = [&](int n) {
    if (!all_valid) raise_offsets();
    exps();
    bool ok = true;
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) ok = ok && blk[qt][0] <= 0x1p64f;
    if (!__all(ok)) {
      // a score ran more than 64 / c past its row's offset: score the block
      // again (its K tile is still in LDS), raise the offsets, redo P
      scores(n);
      raise_offsets();
      exps();
    }
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) lsum[qt] += blk[qt][0];
  };

  // ---- O^T += V^T P^T for key block n.  Lane (g, c) needs V[key][16 dt + c]
  // for keys 4g + k and 16 + 4g + k (k = 0..3); as a source of the transposed
  // read it addresses row 4g + c/4 (+16), dims 16 dt + 4 (c % 4) .. +3.
  auto pv_product = [&](int n) {
    const __bf16* vs = smem + (n % kStages) * STAGE + TILE;
    bf16x8 pk[NT];
#pragma unroll
    for (int qt = 0; qt < NT; ++qt) pk[qt] = __builtin_bit_cast(bf16x8, s[qt][1]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x4 lo = lds_read_tr16(vs + voff[dt]);
      const bf16x4 hi = lds_read_tr16(vs + 16 * D + voff[dt]);
      const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qt = 0; qt < NT; ++qt)
        acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[qt], acc[qt][dt], 0, 0, 0);
    }
  };

  for (int it = 0; it < nblk; ++it) {
    // block it has landed (for every wave) and every wave is done with block
    // it - 1, whose ring slot the next copy refills
    if (it + kStages - 2 < nblk) wait_copies_and_sync<(kStages - 2) * CPB>();
    else wait_copies_and_sync<0>();
    if (it + kStages - 1 < nblk) issue_block(kbeg + (it + kStages - 1) * BK, (it + kStages - 1) % kStages);
    // a wave whose rows are all padding (the last row block of a unit) only
    // copies and keeps the barriers, leaving its SIMD to the other waves
    if (wave_active) {
      scores(it);
      softmax(it);
      pv_product(it);
    }
  }

  // ---- epilogue
#pragma unroll
  for (int qt = 0; qt < NT; ++qt) {
    const float l = lsum[qt];
    const int r = rrow[qt];
    if (r >= p.T_max * G) continue;
    const int t = r / G, h = kvh * G + r % G;
    const size_t orow = ((size_t)b * p.T_max + t) * p.Hq + h;
    if (p.lsplit == 1) {
      __bf16* o = reinterpret_cast<__bf16*>(p.out) + orow * D;
      const float inv = (rvalid[qt] && l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 v = acc[qt][dt] * inv;
        *reinterpret_cast<uint2*>(o + dt * 16 + 4 * g) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    } else if (rvalid[qt]) {
      float* po = p.part_o + (orow * p.lstride + ls_i) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) =
            make_float4(acc[qt][dt][0], acc[qt][dt][1], acc[qt][dt][2], acc[qt][dt][3]);
      if (g == 0) {
        float* pm = p.part_ml + (orow * p.lstride + ls_i) * 2;
        pm[0] = valid[qt] ? mu[qt] * c2 : -INFINITY;   // log2 units for the merge
        pm[1] = l;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 kernel (VALU): one wave per (sequence, tree position, query head) row,
// keys in blocks of 64 (one per lane), lane d owns output dims d and d + 64.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(AttnParams p) {
  __shared__ float qs[D];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;                  // ((b * T_max + t) * Hq + h)
  const int ls_i = blockIdx.y;
  const int h = row % p.Hq;
  const int t = (row / p.Hq) % p.T_max;
  const int b = row / (p.Hq * p.T_max);
  const int kvh = h / p.G;
  const int Tb = p.num_nodes[b];
  const int Lb = p.prefix_len[b];
  const bool valid = p.status[b] == SV_TREE_OK && t < Tb && Tb <= p.T_max && Lb >= 0 && Lb <= p.L_max;
  const int kbeg = ls_i * p.chunk;
  const int kend = min(kbeg + p.chunk, Lb + Tb);
  constexpr int DPL = D / 64 > 0 ? D / 64 : 1;  // output dims per lane

  float o[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) o[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (valid && kbeg < kend) {
    const float* qp = reinterpret_cast<const float*>(p.q) + (size_t)row * D;
    for (int d = lane; d < D; d += 64) qs[d] = qp[d];
    __syncthreads();
    const float* kc = reinterpret_cast<const float*>(p.k_cache) + ((size_t)b * p.Hkv + kvh) * p.L_max * D;
    const float* vc = reinterpret_cast<const float*>(p.v_cache) + ((size_t)b * p.Hkv + kvh) * p.L_max * D;
    const float* kn = reinterpret_cast<const float*>(p.k_new) + ((size_t)b * p.T_max * p.Hkv + kvh) * D;
    const float* vn = reinterpret_cast<const float*>(p.v_new) + ((size_t)b * p.T_max * p.Hkv + kvh) * D;
    const size_t ns = (size_t)p.Hkv * D;
    const uint64_t* arow = p.anc + ((size_t)b * p.T_max + t) * p.W;
    for (int blk = kbeg; blk < kend; blk += 64) {
      const int j = blk + lane;
      float sc = -INFINITY;
      bool vis = j < kend;
      if (vis && j >= Lb) {
        const int n = j - Lb;
        vis = (arow[n >> 6] >> (n & 63)) & 1ull;
      }
      if (vis) {
        const float* kr = j < Lb ? kc + (size_t)j * D : kn + (size_t)(j - Lb) * ns;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
        sc = dot * p.scale_log2;
      }
      float mx = sc;
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mnew = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - mnew);
      const float pe = sc == -INFINITY ? 0.f : exp2f(sc - mnew);
      float ssum = pe;
      for (int off = 32; off > 0; off >>= 1) ssum += __shfl_xor(ssum, off);
      l_run = l_run * alpha + ssum;
      m_run = mnew;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[k] *= alpha;
      ps[lane] = pe;
      __syncthreads();
      const int nk = min(64, kend - blk);
      for (int kk = 0; kk < nk; ++kk) {
        const float w = ps[kk];
        if (w == 0.f) continue;
        const int jj = blk + kk;
        const float* vr = jj < Lb ? vc + (size_t)jj * D : vn + (size_t)(jj - Lb) * ns;
#pragma unroll
        for (int k = 0; k < DPL; ++k)
          if (lane + 64 * k < D) o[k] = fmaf(w, vr[lane + 64 * k], o[k]);
      }
      __syncthreads();
    }
  }
  if (p.lsplit == 1) {
    float* out = reinterpret_cast<float*>(p.out) + (size_t)row * D;
    const float inv = (valid && l_run > 0.f) ? 1.f / l_run : 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      if (lane + 64 * k < D) out[lane + 64 * k] = o[k] * inv;
  } else if (valid) {
    float* po = p.part_o + ((size_t)row * p.lstride + ls_i) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      if (lane + 64 * k < D) po[lane + 64 * k] = o[k];
    if (lane == 0) {
      p.part_ml[((size_t)row * p.lstride + ls_i) * 2] = m_run;
      p.part_ml[((size_t)row * p.lstride + ls_i) * 2 + 1] = l_run;
    }
  }
}

// ----------------------------------------------------------------------------
// Merge of key-range partials: m = max m_s, O = sum 2^(m_s - m) O_s / sum
// 2^(m_s - m) l_s.  One thread per (row, 4 output dims); invalid rows are
// zeroed.  The merge is bound by memory latency, not bytes: a thread issues
// the sequence's sizes, the split in use and the offsets m_s of every range
// the workspace holds in one round trip (the ranges past the split are
// ignored), then (l_s, O_s) of 4 ranges per further one.  Few
// registers keep all rows of the workloads resident at once.
// ----------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void k_attn_combine(AttnParams p) {
  constexpr int LPR = D / 4;            // threads per row
  constexpr int RPG = 256 / LPR;        // rows per workgroup
  constexpr int NM = 16;                // offsets loaded in the first round trip
  constexpr int NB = 4;                 // ranges per batch of O loads
  const int row = blockIdx.x * RPG + threadIdx.x / LPR;
  const int c4 = threadIdx.x % LPR;
  if (row >= p.B * p.T_max * p.Hq) return;
  const int t = (row / p.Hq) % p.T_max;
  const int b = row / (p.Hq * p.T_max);
  const float* pm = p.part_ml + (size_t)row * p.lstride * 2;
  const float4* po = reinterpret_cast<const float4*>(p.part_o) + (size_t)row * p.lstride * LPR + c4;
  // first round trip: everything that does not depend on another load
  const int Tb = p.num_nodes[b];
  const int Lb = p.prefix_len[b];
  const int st = p.status[b];
  const int nls = p.dyn ? *p.dyn_ls : p.lsplit;
  float mv[NM];
#pragma unroll
  for (int s = 0; s < NM; ++s)
    if (s < p.lstride) mv[s] = pm[2 * s];
  const bool valid = st == SV_TREE_OK && t < Tb && Tb <= p.T_max && Lb >= 0 && Lb <= p.L_max;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) {
    float m = -INFINITY, l = 0.f;
    if (nls <= NM && p.lstride <= NM) {
#pragma unroll
      for (int s = 0; s < NM; ++s)
        if (s < nls) m = fmaxf(m, mv[s]);
#pragma unroll
      for (int s = 0; s < NM; ++s) mv[s] = (s < nls && mv[s] != -INFINITY) ? exp2f(mv[s] - m) : 0.f;
#pragma unroll
      for (int s0 = 0; s0 < NM; s0 += NB) {
        if (s0 >= nls) break;
        float ls[NB];
        float4 v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (mv[s0 + j] != 0.f) {
            ls[j] = pm[2 * (s0 + j) + 1];
            v[j] = po[(s0 + j) * LPR];
          }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float w = mv[s0 + j];
          if (w != 0.f) {
            l = fmaf(w, ls[j], l);
            o.x = fmaf(w, v[j].x, o.x);
            o.y = fmaf(w, v[j].y, o.y);
            o.z = fmaf(w, v[j].z, o.z);
            o.w = fmaf(w, v[j].w, o.w);
          }
        }
      }
    } else {
      for (int s = 0; s < nls; ++s) m = fmaxf(m, pm[2 * s]);
      for (int s = 0; s < nls; ++s) {
        const float ms = pm[2 * s];
        if (ms == -INFINITY) continue;
        const float w = exp2f(ms - m);
        const float4 v = po[s * LPR];
        l = fmaf(w, pm[2 * s + 1], l);
        o.x = fmaf(w, v.x, o.x);
        o.y = fmaf(w, v.y, o.y);
        o.z = fmaf(w, v.z, o.z);
        o.w = fmaf(w, v.w, o.w);
      }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
  }
  if (BF16) {
    __bf16* out = reinterpret_cast<__bf16*>(p.out) + (size_t)row * D + 4 * c4;
    *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
  } else {
    float* out = reinterpret_cast<float*>(p.out) + (size_t)row * D + 4 * c4;
    *reinterpret_cast<float4*>(out) = o;
  }
}

const void* variant_kernel(int D, int nt, int nw) {
  switch (D * 100 + nt * 10 + nw) {
    case 12834: return (const void*)k_attn_bf16<128, 3, 4>;
    case 12824: return (const void*)k_attn_bf16<128, 2, 4>;
    case 12821: return (const void*)k_attn_bf16<128, 2, 1>;
    case 12811: return (const void*)k_attn_bf16<128, 1, 1>;
    case 6444: return (const void*)k_attn_bf16<64, 4, 4>;
    case 6434: return (const void*)k_attn_bf16<64, 3, 4>;
    case 6421: return (const void*)k_attn_bf16<64, 2, 1>;
    case 6411: return (const void*)k_attn_bf16<64, 1, 1>;
    default: return nullptr;
  }
}

namespace {
struct Variant {
  int D, nt, nw;
  float row_cost;  // relative cost of one padded row
};
// Instantiated MFMA shapes (head dim, 16-row tiles per wave, waves per group);
// all of them fit two waves per SIMD.  The row costs are measured times per
// padded row relative to the best shape of the head dim (fewer tiles per wave
// read the same K/V tiles from LDS for fewer MFMAs; one-wave groups share no
// copies).
const Variant kVariants[] = {
    {128, 3, 4, 1.0f}, {128, 2, 4, 1.2f}, {128, 2, 1, 2.5f}, {128, 1, 1, 3.5f},
    {64, 4, 4, 1.0f},  {64, 3, 4, 1.0f},  {64, 2, 1, 1.25f}, {64, 1, 1, 2.2f},
};
// One more pass over the keys of a (sequence, KV head), in padded-row units.
constexpr float kRereadRows = 60.f;

size_t smem_bytes(int D, int T_max) {
  const int W = (T_max + 63) / 64;
  const size_t stage = 2 * (size_t)BK * D;
  return kStages * stage * sizeof(uint16_t) + (size_t)T_max * W * sizeof(uint64_t);
}
}  // namespace

// Workgroups of one MFMA variant resident per CU (occupancy query, cached per
// device and variant; 2 when the runtime cannot tell).
int resident_groups(int D, int nt, int nw, size_t smem) {
  static std::atomic<int> cache[64][16];   // the same value whichever thread fills it
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int idx = -1, i = 0;
  for (const Variant& v : kVariants) {
    if (v.D == D && v.nt == nt && v.nw == nw) idx = i;
    ++i;
  }
  if (idx < 0) return 2;
  int n = cache[dev][idx].load(std::memory_order_relaxed);
  if (n == 0) {
    const void* fn = variant_kernel(D, nt, nw);
    if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, nw * 64, smem) != hipSuccess || n < 1) n = 2;
    cache[dev][idx].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool plan_attention(const sv_tree* t, const sv_attn_args* a, AttnPlan* pl) {
  const DeviceInfo& di = device_info();
  const int G = a->Hq / a->Hkv;
  const long M = (long)t->T_max * G;  // padded query rows per (sequence, KV head)
  const long units = (long)t->B * a->Hkv;
  const long keys = (long)a->L_max + t->T_max;
  *pl = AttnPlan{};
  if (a->dtype == SV_F32) {
    pl->kernel = 1;
    const long rows = (long)t->B * t->T_max * a->Hq;
    long ls = 1;
    while (rows * ls < 4L * di.num_cu && keys / (ls * 2) >= 256) ls *= 2;
    pl->lsplit = (int)ls;
  } else {
    pl->kernel = 0;
    // choose the variant with the least padded row work; more rows per
    // workgroup (fewer re-reads of the same keys) breaks ties
    float best_cost = -1.f;
    for (const Variant& v : kVariants) {
      if (v.D != a->D) continue;
      const long rpw = (long)v.nt * v.nw * 16;
      const long ms = (M + rpw - 1) / rpw;
      const float cost = (float)(ms * rpw) * v.row_cost + kRereadRows * (float)ms;
      if (best_cost < 0.f || cost < best_cost) {
        best_cost = cost;
        pl->nt = v.nt;
        pl->nwave = v.nw;
        pl->rows_per_wg = (int)rpw;
        pl->msplit = (int)ms;
      }
    }
    if (best_cost < 0.f) return false;
    // tuning override: SV_ATTN_VARIANT="nt,nw" picks an instantiated shape
    if (const char* ov = getenv("SV_ATTN_VARIANT")) {
      int nt = 0, nw = 0;
      if (sscanf(ov, "%d,%d", &nt, &nw) == 2) {
        for (const Variant& v : kVariants) {
          if (v.D == a->D && v.nt == nt && v.nw == nw) {
            const long rpw = (long)nt * nw * 16;
            pl->nt = nt;
            pl->nwave = nw;
            pl->rows_per_wg = (int)rpw;
            pl->msplit = (int)((M + rpw - 1) / rpw);
          }
        }
      }
    }
    // Key splits.  With k workgroups landing on a CU, each doing 1/ls of a
    // unit's keys, the CU is busy ~ k/ls / thr(k), where two or more
    // workgroups sharing a CU run 1.6x the throughput of one alone; each
    // extra split costs a little (partials written and merged).
    const long groups = units * pl->msplit;
    float best = -1.f;
    for (long ls = 1; ls <= 16; ++ls) {
      if (ls > 1 && keys / ls < 4L * BK) break;
      const long k = (groups * ls + di.num_cu - 1) / di.num_cu;
      const float cost = (float)k / (float)ls / (k >= 2 ? 1.6f : 1.f) + 0.02f * (float)(ls - 1);
      if (best < 0.f || cost < best - 1e-6f) {
        best = cost;
        pl->lsplit = (int)ls;
      }
    }
  }
  // tuning override: SV_ATTN_LSPLIT=n forces n key ranges per row
  if (const char* ov = getenv("SV_ATTN_LSPLIT")) {
    const int n = atoi(ov);
    if (n >= 1 && n <= 64) pl->lsplit = n;
  }
  const long per = (keys + pl->lsplit - 1) / pl->lsplit;
  pl->chunk = (int)((per + 63) / 64 * 64);
  // With key splits and several row blocks per (sequence, KV head), the MFMA
  // kernel re-plans on the device from the trees' actual sizes (up to 4x this
  // split, at most 16); trees of T_max nodes give exactly this plan.
  // SV_ATTN_LSPLIT (a forced split) and SV_ATTN_DYN=0 keep the host's plan.
  pl->dyn = 0;
  pl->ls_cap = pl->lsplit;
  const char* dyn_env = getenv("SV_ATTN_DYN");
  if (pl->kernel == 0 && pl->lsplit > 1 && pl->msplit > 1 && !getenv("SV_ATTN_LSPLIT") &&
      !(dyn_env && atoi(dyn_env) == 0)) {
    pl->dyn = 1;
    pl->ls_cap = (int)std::min(16L, 4L * pl->lsplit);
    if (pl->ls_cap < pl->lsplit) pl->ls_cap = pl->lsplit;
  }
  if (getenv("SV_DEBUG_PLAN"))
    fprintf(stderr, "sv attention plan: kernel=%d nt=%d nwave=%d rows/wg=%d msplit=%d lsplit=%d chunk=%d dyn=%d cap=%d "
            "cus=%d resident=%d\n",
            pl->kernel, pl->nt, pl->nwave, pl->rows_per_wg, pl->msplit, pl->lsplit, pl->chunk, pl->dyn, pl->ls_cap,
            di.num_cu, pl->kernel == 0 ? resident_groups(a->D, pl->nt, pl->nwave, smem_bytes(a->D, t->T_max)) : 0);
  pl->ws_bytes = 0;
  if (pl->lsplit > 1) {
    const size_t rows = (size_t)t->B * t->T_max * a->Hq * pl->ls_cap;
    pl->ws_bytes = align_up(rows * a->D * sizeof(float), kWsAlign) +
                   align_up(rows * 2 * sizeof(float), kWsAlign) + (pl->dyn ? kWsAlign : 0);
  }
  return true;
}

template <int D, int NT, int NW>
static hipError_t launch_mfma(const AttnParams& prm, int grid, size_t smem, hipStream_t s) {
  auto k = k_attn_bf16<D, NT, NW>;
  static std::atomic<bool> attr_set[64];   // setting the attribute twice is harmless
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_relaxed)) {
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev].store(true, std::memory_order_relaxed);
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(NW * 64), smem, s, prm);
  return hipGetLastError();
}

sv_status launch_attention(const sv_tree* t, const uint64_t* anc, const int32_t* tree_status,
                           const sv_attn_args* a, const AttnPlan& pl, void* ws, hipStream_t s) {
  if (t->B == 0) return SV_OK;
  AttnParams prm{};
  prm.q = a->q;
  prm.k_new = a->k_new;
  prm.v_new = a->v_new;
  prm.k_cache = a->k_cache;
  prm.v_cache = a->v_cache;
  prm.prefix_len = a->prefix_len;
  prm.num_nodes = t->num_nodes;
  prm.status = tree_status;
  prm.anc = anc;
  prm.out = a->out;
  prm.B = t->B;
  prm.T_max = t->T_max;
  prm.Hq = a->Hq;
  prm.Hkv = a->Hkv;
  prm.G = a->Hq / a->Hkv;
  prm.L_max = a->L_max;
  prm.W = (t->T_max + 63) / 64;
  prm.rows_per_wg = pl.rows_per_wg;
  prm.msplit = pl.msplit;
  prm.lsplit = pl.lsplit;
  prm.chunk = pl.chunk;
  prm.lstride = pl.ls_cap;
  prm.dyn = pl.dyn;
  prm.ls_cap = pl.ls_cap;
  prm.keys_max = a->L_max + t->T_max;
  const double scale = a->scale > 0.f ? (double)a->scale : 1.0 / sqrt((double)a->D);
  prm.scale_log2 = (float)(scale * 1.4426950408889634);
  prm.raise_raw = 8.f / prm.scale_log2;
  if (pl.lsplit > 1) {
    const size_t rows = (size_t)t->B * t->T_max * a->Hq * pl.ls_cap;
    const size_t o_bytes = align_up(rows * a->D * sizeof(float), kWsAlign);
    const size_t ml_bytes = align_up(rows * 2 * sizeof(float), kWsAlign);
    prm.part_o = reinterpret_cast<float*>(ws);
    prm.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes);
    if (pl.dyn) prm.dyn_ls = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + o_bytes + ml_bytes);
  }
  hipError_t e = hipSuccess;
  if (pl.kernel == 1) {
    const int rows = t->B * t->T_max * a->Hq;
    dim3 grid(rows, pl.lsplit);
    if (a->D == 64) hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(64), 0, s, prm);
    else hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(64), 0, s, prm);
    e = hipGetLastError();
  } else {
    const int grid = (int)((long)t->B * a->Hkv * pl.msplit * pl.lsplit);
    prm.remap = (grid % 8 == 0) ? 1 : 0;
    const size_t smem = smem_bytes(a->D, t->T_max);
    const int key = a->D * 100 + pl.nt * 10 + pl.nwave;
    switch (key) {
      case 12834: e = launch_mfma<128, 3, 4>(prm, grid, smem, s); break;
      case 12824: e = launch_mfma<128, 2, 4>(prm, grid, smem, s); break;
      case 12821: e = launch_mfma<128, 2, 1>(prm, grid, smem, s); break;
      case 12811: e = launch_mfma<128, 1, 1>(prm, grid, smem, s); break;
      case 6444: e = launch_mfma<64, 4, 4>(prm, grid, smem, s); break;
      case 6434: e = launch_mfma<64, 3, 4>(prm, grid, smem, s); break;
      case 6421: e = launch_mfma<64, 2, 1>(prm, grid, smem, s); break;
      case 6411: e = launch_mfma<64, 1, 1>(prm, grid, smem, s); break;
      default: set_error("no attention variant D=%d nt=%d nw=%d", a->D, pl.nt, pl.nwave); return SV_E_UNSUPPORTED;
    }
  }
  if (e != hipSuccess) {
    set_error("attention launch: %s", hipGetErrorString(e));
    return SV_E_HIP;
  }
  if (pl.lsplit > 1) {
    const int rows = t->B * t->T_max * a->Hq;
    const int rpg = 256 / (a->D / 4);   // rows per merge workgroup
    const dim3 grid((rows + rpg - 1) / rpg);
    if (a->dtype == SV_BF16) {
      if (a->D == 64) hipLaunchKernelGGL((k_attn_combine<true, 64>), grid, dim3(256), 0, s, prm);
      else hipLaunchKernelGGL((k_attn_combine<true, 128>), grid, dim3(256), 0, s, prm);
    } else {
      if (a->D == 64) hipLaunchKernelGGL((k_attn_combine<false, 64>), grid, dim3(256), 0, s, prm);
      else hipLaunchKernelGGL((k_attn_combine<false, 128>), grid, dim3(256), 0, s, prm);
    }
    e = hipGetLastError();
    if (e != hipSuccess) {
      set_error("attention combine launch: %s", hipGetErrorString(e));
      return SV_E_HIP;
    }
  }
  return SV_OK;
}

}  // namespace sv
