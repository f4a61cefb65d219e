// Flattened draft tree -> ancestor-or-self bitmask, depth and tree validity.
//
// [EAGLE article] sec. 2.3 "Flatten + Attention mask": after flattening the
// selected draft tree to one sequence, tokens of different branches must not
// see each other and every token sees only its ancestors on the tree.
// [Spec-decoding lesson] "Tree-attention verification": the mask encodes the
// tree topology instead of the plain causal triangle.
//
// One workgroup of 256 threads per sequence; thread i owns row i.  The tree is
// validated first (node count, root, parent[i] < i), so every parent walk
// strictly decreases and ends at the root.  In a verify step the kernel also
// zeroes the walk's exchange words, which saves the walk its own fill kernel.
#include "sv_internal.h"

namespace sv {

__global__ __launch_bounds__(256) void k_tree_mask_build(const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ num_nodes,
                                                         int T_max, int W,
                                                         uint64_t* __restrict__ anc,
                                                         int32_t* __restrict__ depth,
                                                         int32_t* __restrict__ tree_status,
                                                         uint64_t* __restrict__ zero_words, int n_zero) {
  __shared__ int par[kMaxT];
  __shared__ int flags;  // bit 0: root has a parent, bit 1: a parent out of range
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  for (int i = b * 256 + tid; i < n_zero; i += gridDim.x * 256) zero_words[i] = 0ull;
  // the node count and this thread's parent in one memory round trip (the
  // parent array is [B][T_max], so the load is in bounds whatever the count)
  const int Tb = num_nodes[b];
  const int p = tid < T_max ? parent[(size_t)b * T_max + tid] : -1;
  const bool count_ok = Tb >= 1 && Tb <= T_max;
  if (tid == 0) flags = 0;
  __syncthreads();
  if (count_ok && tid < Tb) {
    par[tid] = p;
    if (tid == 0) {
      if (p != -1) atomicOr(&flags, 1);
    } else if (p < 0 || p >= tid) {
      atomicOr(&flags, 2);
    }
  }
  __syncthreads();
  int st = SV_TREE_OK;
  if (!count_ok) st = SV_TREE_E_COUNT;
  else if (flags & 1) st = SV_TREE_E_ROOT;
  else if (flags & 2) st = SV_TREE_E_PARENT;
  if (tid == 0) tree_status[b] = st;
  if (tid >= T_max) return;

  uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
  int d = 0;
  if (st == SV_TREE_OK && tid < Tb) {
    int j = tid;
    while (true) {
      const uint64_t bit = 1ull << (j & 63);
      const int k = j >> 6;
      w0 |= k == 0 ? bit : 0ull;
      w1 |= k == 1 ? bit : 0ull;
      w2 |= k == 2 ? bit : 0ull;
      w3 |= k == 3 ? bit : 0ull;
      j = par[j];
      if (j < 0) break;
      ++d;
    }
  }
  uint64_t* row = anc + ((size_t)b * T_max + tid) * W;
  row[0] = w0;
  if (W > 1) row[1] = w1;
  if (W > 2) row[2] = w2;
  if (W > 3) row[3] = w3;
  depth[(size_t)b * T_max + tid] = d;
}

sv_status launch_mask(const sv_tree* t, uint64_t* anc, int32_t* depth, int32_t* tree_status,
                      uint64_t* zero_words, int n_zero, hipStream_t s) {
  if (t->B == 0) return SV_OK;
  const int W = (t->T_max + 63) / 64;
  hipLaunchKernelGGL(k_tree_mask_build, dim3(t->B), dim3(256), 0, s, t->parent, t->num_nodes,
                     t->T_max, W, anc, depth, tree_status, zero_words, n_zero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("mask build launch: %s", hipGetErrorString(e));
    return SV_E_HIP;
  }
  return SV_OK;
}

}  // namespace sv
