// Commit of the accepted path: the K / V rows of the root and the accepted
// nodes go to the caches after the prefix, and their feature rows to the
// drafter's feature buffer.
//
// [EAGLE article] sec. 1.3 "Verification": the accepted tokens and their
// features are kept and drafting continues from them.  [Spec-decoding lesson]
// "Concept": the accepted tokens extend the output; the correction / bonus
// token is the next position the target runs on.
//
// One workgroup per (sequence, KV head) copies that head's K and V rows; one
// more per sequence copies the feature rows, zeroes the others and writes the
// new length and any status.  Every workgroup of a sequence takes the same
// decision from the same inputs, so none waits for another.  The work is a
// small gather: about 2 c rows of D elements per head and sequence.
// The bookkeeper's status write may land before another workgroup of the same
// sequence reads that word.  It only ever turns OK into an error, and it does
// so exactly when the checks below fail, so either value read leads that
// workgroup to write nothing.
#include "sv_internal.h"

namespace sv {

constexpr int kCommitThreads = 256;

struct CommitParams {
  const int32_t* num_nodes;
  int32_t* status;
  const int32_t* out_nodes;
  const int32_t* out_count;
  const unsigned char* k_new;
  const unsigned char* v_new;
  unsigned char* k_cache;
  unsigned char* v_cache;
  const int32_t* prefix_len;
  int32_t* prefix_len_out;
  const unsigned char* feat_in;
  unsigned char* feat_out;
  int T_max, Hkv, L_max;
  int row_bytes;    // D * element size, a multiple of 16
  int feat_bytes;   // F * feature element size (0: no features)
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Copies rows n of src (row pitch src_pitch) to rows row0 + i of dst (pitch
// dst_pitch), where pos_s[i] = n, i < rows.  Every (row, unit) pair goes to its
// own thread, so all rows are in flight at once.  Units are 16 bytes when the
// row length allows it, else 2 bytes (feature rows may have any width).
__device__ inline void gather_rows(unsigned char* dst, size_t dst_pitch, int row0, const unsigned char* src,
                                   size_t src_pitch, const int* pos_s, int rows, int nbytes, int tid) {
  if ((nbytes & 15) == 0) {
    const int per_row = nbytes >> 4;
    for (int u = tid; u < rows * per_row; u += kCommitThreads) {
      const int i = u / per_row;
      const int j = (u - i * per_row) << 4;
      *reinterpret_cast<u32x4*>(dst + (size_t)(row0 + i) * dst_pitch + j) =
          *reinterpret_cast<const u32x4*>(src + (size_t)pos_s[i] * src_pitch + j);
    }
  } else {
    const int per_row = nbytes >> 1;
    for (int u = tid; u < rows * per_row; u += kCommitThreads) {
      const int i = u / per_row;
      const int j = (u - i * per_row) << 1;
      *reinterpret_cast<uint16_t*>(dst + (size_t)(row0 + i) * dst_pitch + j) =
          *reinterpret_cast<const uint16_t*>(src + (size_t)pos_s[i] * src_pitch + j);
    }
  }
}

__global__ __launch_bounds__(kCommitThreads) void k_commit(CommitParams p) {
  __shared__ int pos_s[kMaxT];
  __shared__ int bad_s;
  const int b = blockIdx.x;
  const int y = blockIdx.y;            // KV head, or Hkv for the feature / bookkeeping group
  const int tid = threadIdx.x;
  const int st = p.status[b];
  const int c = p.out_count[b];
  const int L = p.prefix_len[b];
  const int Tb = p.num_nodes[b];
  const bool bookkeeper = y == p.Hkv;
  bool go = st == SV_TREE_OK && c >= 1;
  int new_status = st;
  if (go) {
    // positions to commit: the root, then the accepted path; all in [1, T_b)
    if (tid == 0) bad_s = 0;
    __syncthreads();
    if (c > Tb || Tb > p.T_max) {
      if (tid == 0) bad_s = 1;
    } else {
      for (int i = tid; i < c; i += kCommitThreads) {
        const int n = i == 0 ? 0 : p.out_nodes[(size_t)b * p.T_max + i - 1];
        if (i > 0 && (n < 1 || n >= Tb)) atomicOr(&bad_s, 1);
        pos_s[i] = n;
      }
    }
    __syncthreads();
    if (bad_s) {
      go = false;
      new_status = SV_TREE_E_PATH;
    } else if (L < 0 || (long)L + c > p.L_max) {
      go = false;
      new_status = SV_TREE_E_CACHE;
    }
  }
  if (!bookkeeper) {
    if (!go) return;
    const int h = y;
    const size_t new_row = (size_t)p.Hkv * p.row_bytes;                       // between positions
    const size_t src = (size_t)b * p.T_max * new_row + (size_t)h * p.row_bytes;
    const size_t dst = ((size_t)b * p.Hkv + h) * p.L_max * p.row_bytes;
    // K and V in one pass: units [0, c*per_row) are K, the rest V
    const int per_row = p.row_bytes >> 4;
    const int units = c * per_row;
    for (int u = tid; u < 2 * units; u += kCommitThreads) {
      const bool is_v = u >= units;
      const int r = is_v ? u - units : u;
      const int i = r / per_row;
      const int j = (r - i * per_row) << 4;
      const uint64_t from = reinterpret_cast<uint64_t>(is_v ? p.v_new : p.k_new) + src +
                            (size_t)pos_s[i] * new_row + j;
      const uint64_t to = reinterpret_cast<uint64_t>(is_v ? p.v_cache : p.k_cache) + dst +
                          (size_t)(L + i) * p.row_bytes + j;
      *reinterpret_cast<u32x4*>(to) = *reinterpret_cast<const u32x4*>(from);
    }
    return;
  }
  // features: committed rows first, zeros after; then length and status
  if (p.feat_bytes > 0) {
    const size_t fb = (size_t)p.feat_bytes;
    const int n_rows = go ? c : 0;
    const size_t seq = (size_t)b * p.T_max * fb;
    gather_rows(p.feat_out + seq, fb, 0, p.feat_in + seq, fb, pos_s, n_rows, p.feat_bytes, tid);
    unsigned char* rest = p.feat_out + ((size_t)b * p.T_max + n_rows) * fb;
    const size_t rest_bytes = (size_t)(p.T_max - n_rows) * fb;
    for (size_t i = (size_t)tid * 2; i < rest_bytes; i += kCommitThreads * 2)
      *reinterpret_cast<uint16_t*>(rest + i) = 0;
  }
  if (tid == 0) {
    p.prefix_len_out[b] = go ? L + c : L;
    if (new_status != st) p.status[b] = new_status;
  }
}

sv_status launch_commit(const sv_tree* t, int32_t* tree_status, const int32_t* out_nodes,
                        const int32_t* out_count, const sv_commit_args* a, hipStream_t s) {
  if (t->B == 0) return SV_OK;
  const int es = a->dtype == SV_BF16 ? 2 : 4;
  const int fes = a->feat_dtype == SV_BF16 ? 2 : 4;
  CommitParams p{};
  p.num_nodes = t->num_nodes;
  p.status = tree_status;
  p.out_nodes = out_nodes;
  p.out_count = out_count;
  p.k_new = static_cast<const unsigned char*>(a->k_new);
  p.v_new = static_cast<const unsigned char*>(a->v_new);
  p.k_cache = static_cast<unsigned char*>(a->k_cache);
  p.v_cache = static_cast<unsigned char*>(a->v_cache);
  p.prefix_len = a->prefix_len;
  p.prefix_len_out = a->prefix_len_out;
  p.feat_in = static_cast<const unsigned char*>(a->feat_in);
  p.feat_out = static_cast<unsigned char*>(a->feat_out);
  p.T_max = t->T_max;
  p.Hkv = a->Hkv;
  p.L_max = a->L_max;
  p.row_bytes = a->D * es;
  p.feat_bytes = a->F > 0 ? a->F * fes : 0;
  hipLaunchKernelGGL(k_commit, dim3(t->B, a->Hkv + 1), dim3(kCommitThreads), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("commit launch: %s", hipGetErrorString(e));
    return SV_E_HIP;
  }
  return SV_OK;
}

}  // namespace sv
