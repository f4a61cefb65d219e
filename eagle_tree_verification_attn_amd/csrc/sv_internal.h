// Internal declarations shared by the HIP sources of the verification library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <atomic>
#include <mutex>

#include "sv.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxT = 256;          // largest T_max (one mask row per thread)
constexpr size_t kWsAlign = 256;    // workspace sub-buffer alignment

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Largest 64-bit value over each row of 16 lanes, in every lane of the row:
// DPP lane permutations within the row (pairs, quads, half rows, the row).
// Every lane of the row must be active.
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ inline uint64_t row16_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xB1>(v);  v = o > v ? o : v;    // quad_perm [1, 0, 3, 2]
  o = dpp_u64<0x4E>(v);  v = o > v ? o : v;    // quad_perm [2, 3, 0, 1]
  o = dpp_u64<0x141>(v); v = o > v ? o : v;    // row_half_mirror
  o = dpp_u64<0x140>(v); v = o > v ? o : v;    // row_mirror
  return v;
}
// Largest 64-bit value over the wave (uniform): the four row maxima, read
// from the last lane of each row.  Every lane must be active.
__device__ inline uint64_t wave_max_u64_dpp(uint64_t v) {
  v = row16_max_u64(v);
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r + 15);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r + 15);
    const uint64_t x = ((uint64_t)hi << 32) | lo;
    m = x > m ? x : m;
  }
  return m;
}

// Thread-local detail string behind sv_last_error().
void set_error(const char* fmt, ...);
void clear_error();

// Per-device facts used to size launches (cached on first use per device).
struct DeviceInfo {
  int device;
  int num_cu;
  int num_xcd;
};
const DeviceInfo& device_info();

// ---------------------------------------------------------------- attention
struct AttnPlan {
  int kernel;       // 0 = bf16 MFMA, 1 = fp32 VALU
  int nt;           // 16-query tiles per wave (MFMA kernel)
  int nwave;        // waves per workgroup (MFMA kernel)
  int rows_per_wg;  // query rows (node, head-in-group pairs) per workgroup
  int msplit;       // workgroups along the query rows of one (sequence, KV head)
  int lsplit;       // workgroups along the key axis
  int chunk;        // keys per L split (multiple of the key block)
  int dyn;          // MFMA kernel with lsplit > 1: the split follows the trees' actual sizes on the device
  int ls_cap;       // largest split the device may choose (partials per row in the workspace)
  size_t ws_bytes;  // partial results when lsplit > 1
};
bool plan_attention(const sv_tree* t, const sv_attn_args* a, AttnPlan* p);
sv_status launch_attention(const sv_tree* t, const uint64_t* anc, const int32_t* tree_status,
                           const sv_attn_args* a, const AttnPlan& p, void* ws, hipStream_t s);

// ---------------------------------------------------------------- accept
struct AcceptPlan {
  int nchunk;       // vocabulary chunks per row (= workgroups per sequence in the walk)
  int chunk;        // tokens per chunk (multiple of 8)
  int ngroups;      // sequence groups resident at once in the walk
  size_t off_xchg;
  size_t ws_bytes;
};
bool plan_accept(const sv_tree* t, const sv_accept_args* a, AcceptPlan* p);
int accept_exchange_words(const AcceptPlan& p);   // uint64 words at off_xchg
// clear_exchange: zero the exchange words first (a fill kernel); false when
// the caller's stream already zeroed them (the mask kernel of a verify step)
sv_status launch_accept(const sv_tree* t, int32_t* tree_status, const sv_accept_args* a,
                        const AcceptPlan& p, void* ws, bool clear_exchange, hipStream_t s);

// ---------------------------------------------------------------- commit
sv_status launch_commit(const sv_tree* t, int32_t* tree_status, const int32_t* out_nodes,
                        const int32_t* out_count, const sv_commit_args* a, hipStream_t s);

// ---------------------------------------------------------------- tree builder
struct E2Layout {
  int nmax;         // nodes per sequence: 1 + k + (depth - 1) k^2
  int nsplit;       // vocabulary chunks per probability row
  int chunk;        // tokens per chunk (multiple of 4)
  size_t off_seq, off_front, off_parent, off_token, off_depth, off_rank, off_qrow, off_value, off_cand, off_bad;
  size_t bytes;
};
E2Layout eagle2_layout(const sv_eagle2_cfg* c);
sv_status launch_eagle2_begin(const sv_eagle2_cfg* c, void* state, const int32_t* root_tokens, hipStream_t s);
sv_status launch_eagle2_expand(const sv_eagle2_cfg* c, void* state, int step, const float* q, int32_t* frontier,
                               int32_t* frontier_tokens, hipStream_t s);
sv_status launch_eagle2_expand_finish(const sv_eagle2_cfg* c, void* state, int step, const float* q, int32_t* parent,
                                      int32_t* tokens, int32_t* num_nodes, int32_t* q_row, int32_t* status,
                                      hipStream_t s);
sv_status launch_eagle2_finish(const sv_eagle2_cfg* c, const void* state, int32_t* parent, int32_t* tokens,
                               int32_t* num_nodes, int32_t* q_row, int32_t* status, hipStream_t s);

// ---------------------------------------------------------------- draft head
sv_status launch_draft_head(const sv_head_args* a, hipStream_t s);

// ---------------------------------------------------------------- mask
// zero_words / n_zero: words the mask kernel also zeroes (a verify step's
// exchange words for the walk), or NULL / 0
sv_status launch_mask(const sv_tree* t, uint64_t* anc, int32_t* depth, int32_t* tree_status,
                      uint64_t* zero_words, int n_zero, hipStream_t s);

}  // namespace sv
