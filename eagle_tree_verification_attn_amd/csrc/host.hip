// C ABI of the verification library: argument validation, workspace sizing,
// launch sequencing.  Every entry point only enqueues work on the caller's
// stream; nothing here allocates device memory or synchronises.
#include "sv_internal.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

namespace sv {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = 0; }

// Filled once per device; concurrent first calls from several host threads
// are serialised by the once flag.
const DeviceInfo& device_info() {
  static DeviceInfo infos[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::call_once(once[dev], [dev] {
    DeviceInfo d{dev, 256, 8};
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
      d.num_cu = cu;
    infos[dev] = d;
  });
  return infos[dev];
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

sv_status check_tree(const sv_tree* t, bool need_tokens) {
  if (!t) { set_error("tree is NULL"); return SV_E_NULL; }
  if (t->B < 0) { set_error("B = %d < 0", t->B); return SV_E_SHAPE; }
  if (t->T_max < 1) { set_error("T_max = %d < 1", t->T_max); return SV_E_SHAPE; }
  if (t->T_max > kMaxT) { set_error("T_max = %d > %d", t->T_max, kMaxT); return SV_E_UNSUPPORTED; }
  if (t->B > 0) {
    if (!t->parent || !t->num_nodes) { set_error("tree parent/num_nodes is NULL"); return SV_E_NULL; }
    if (need_tokens && !t->tokens) { set_error("tree tokens is NULL"); return SV_E_NULL; }
  }
  return SV_OK;
}

sv_status check_attn(const sv_tree* t, const sv_attn_args* a) {
  if (!a) { set_error("attention args are NULL"); return SV_E_NULL; }
  if (a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0) {
    set_error("heads Hq=%d Hkv=%d (need Hq %% Hkv == 0)", a->Hq, a->Hkv);
    return SV_E_SHAPE;
  }
  if (a->D < 1 || a->L_max < 0) { set_error("D=%d L_max=%d", a->D, a->L_max); return SV_E_SHAPE; }
  if (a->D != 64 && a->D != 128) { set_error("head dim %d (supported: 64, 128)", a->D); return SV_E_UNSUPPORTED; }
  if (a->dtype != SV_F32 && a->dtype != SV_BF16) { set_error("attention dtype %d", a->dtype); return SV_E_DTYPE; }
  if ((long)t->B * t->T_max * a->Hq > 0x7FFFFFFFL) { set_error("B*T_max*Hq too large"); return SV_E_UNSUPPORTED; }
  // the kernels address a (sequence, KV head)'s keys with 32-bit element
  // offsets: (L_max + T_max) * D must stay below 2^31
  if (((long)a->L_max + kMaxT) * a->D > 0x7FFFFFFFL) {
    set_error("L_max = %d too large for D = %d (need (L_max + %d) * D < 2^31)", a->L_max, a->D, kMaxT);
    return SV_E_UNSUPPORTED;
  }
  if (t->B > 0) {
    if (!a->q || !a->k_new || !a->v_new || !a->out || !a->prefix_len) {
      set_error("attention q/k_new/v_new/out/prefix_len is NULL");
      return SV_E_NULL;
    }
    if (a->L_max > 0 && (!a->k_cache || !a->v_cache)) { set_error("k_cache/v_cache is NULL"); return SV_E_NULL; }
    const void* ptrs[] = {a->q, a->k_new, a->v_new, a->out, a->k_cache, a->v_cache};
    for (const void* p : ptrs)
      if (p && !aligned(p, 16)) { set_error("attention tensors must be 16-byte aligned"); return SV_E_UNSUPPORTED; }
  }
  return SV_OK;
}

sv_status check_accept(const sv_tree* t, const sv_accept_args* a) {
  if (!a) { set_error("accept args are NULL"); return SV_E_NULL; }
  if (a->V < 1) { set_error("V = %d < 1", a->V); return SV_E_SHAPE; }
  if (a->V > 64 * 256 * 64) { set_error("V = %d > %d", a->V, 64 * 256 * 64); return SV_E_UNSUPPORTED; }
  if (a->logit_dtype != SV_F32 && a->logit_dtype != SV_BF16) { set_error("logit dtype %d", a->logit_dtype); return SV_E_DTYPE; }
  if (a->sibling_mode != SV_SIB_WITHOUT_REPLACEMENT && a->sibling_mode != SV_SIB_IID) {
    set_error("sibling_mode %d", a->sibling_mode);
    return SV_E_SHAPE;
  }
  if ((long)t->B * t->T_max > 0x7FFFFFFFL / 64) { set_error("B*T_max too large"); return SV_E_UNSUPPORTED; }
  if (t->B > 0) {
    if (!a->target_logits || !a->temperature || !a->u_accept || !a->u_sample || !a->out_tokens ||
        !a->out_nodes || !a->out_count) {
      set_error("accept logits/temperature/uniforms/outputs is NULL");
      return SV_E_NULL;
    }
  }
  return SV_OK;
}

sv_status check_commit(const sv_tree* t, const sv_commit_args* c) {
  if (!c) { set_error("commit args are NULL"); return SV_E_NULL; }
  if (c->dtype != SV_F32 && c->dtype != SV_BF16) { set_error("commit dtype %d", c->dtype); return SV_E_DTYPE; }
  if (c->F > 0 && c->feat_dtype != SV_F32 && c->feat_dtype != SV_BF16) {
    set_error("feature dtype %d", c->feat_dtype);
    return SV_E_DTYPE;
  }
  const int es = c->dtype == SV_BF16 ? 2 : 4;
  if (c->Hkv < 1 || c->D < 1 || c->L_max < 0 || c->F < 0) {
    set_error("commit sizes Hkv=%d D=%d L_max=%d F=%d", c->Hkv, c->D, c->L_max, c->F);
    return SV_E_SHAPE;
  }
  if ((c->D * es) % 16 != 0) { set_error("commit rows of %d bytes (need a multiple of 16)", c->D * es); return SV_E_UNSUPPORTED; }
  if ((long)t->B * c->Hkv > 0x7FFFFFFFL || c->Hkv > 65535) { set_error("B*Hkv too large"); return SV_E_UNSUPPORTED; }
  if (t->B > 0) {
    if (!c->k_new || !c->v_new || !c->k_cache || !c->v_cache || !c->prefix_len || !c->prefix_len_out) {
      set_error("commit k_new/v_new/k_cache/v_cache/prefix_len/prefix_len_out is NULL");
      return SV_E_NULL;
    }
    if (c->F > 0 && (!c->feat_in || !c->feat_out)) { set_error("feat_in/feat_out is NULL"); return SV_E_NULL; }
    if (c->prefix_len == c->prefix_len_out) { set_error("prefix_len_out must not alias prefix_len"); return SV_E_SHAPE; }
    const void* ptrs[] = {c->k_new, c->v_new, c->k_cache, c->v_cache, c->feat_in, c->feat_out};
    for (const void* q : ptrs)
      if (q && !aligned(q, 16)) { set_error("commit tensors must be 16-byte aligned"); return SV_E_UNSUPPORTED; }
  }
  return SV_OK;
}

sv_status check_eagle2(const sv_eagle2_cfg* c) {
  if (!c) { set_error("tree-builder config is NULL"); return SV_E_NULL; }
  if (c->B < 0 || c->k < 1 || c->depth < 1 || c->V < 1 || c->m < 1) {
    set_error("tree builder B=%d V=%d k=%d depth=%d m=%d", c->B, c->V, c->k, c->depth, c->m);
    return SV_E_SHAPE;
  }
  if (c->k > 16 || c->V < c->k) { set_error("tree builder k=%d (need 1..16 and <= V=%d)", c->k, c->V); return SV_E_UNSUPPORTED; }
  if (c->V > 64 * 8192) { set_error("tree builder V=%d > %d", c->V, 64 * 8192); return SV_E_UNSUPPORTED; }
  const long nmax = 1L + c->k + (long)(c->depth - 1) * c->k * c->k;
  if (c->depth > 4096 || nmax > 2048) { set_error("tree builder: %ld nodes before the rerank (max 2048)", nmax); return SV_E_UNSUPPORTED; }
  if (c->m > nmax - 1) { set_error("tree builder m=%d > %ld generated draft nodes", c->m, nmax - 1); return SV_E_SHAPE; }
  if (c->m + 1 > kMaxT) { set_error("tree builder m+1=%d > %d verify positions", c->m + 1, kMaxT); return SV_E_UNSUPPORTED; }
  if ((long)c->B * c->k * 16 > 0x7FFFFFFFL || (long)c->B * nmax > 0x7FFFFFFFL) { set_error("tree builder B too large"); return SV_E_UNSUPPORTED; }
  return SV_OK;
}

sv_status check_state(const sv_eagle2_cfg* c, const void* state, size_t state_bytes) {
  const size_t need = eagle2_layout(c).bytes;
  if (!state) { set_error("tree-builder state is NULL"); return SV_E_NULL; }
  if (state_bytes < need) { set_error("tree-builder state %zu bytes < %zu needed", state_bytes, need); return SV_E_WORKSPACE; }
  if (!aligned(state, kWsAlign)) { set_error("tree-builder state not %zu-byte aligned", kWsAlign); return SV_E_WORKSPACE; }
  return SV_OK;
}

sv_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SV_OK;
  if (!ws) { set_error("workspace is NULL (need %zu bytes)", need); return SV_E_WORKSPACE; }
  if (ws_bytes < need) { set_error("workspace %zu bytes < %zu needed", ws_bytes, need); return SV_E_WORKSPACE; }
  if (!aligned(ws, kWsAlign)) { set_error("workspace not %zu-byte aligned", kWsAlign); return SV_E_WORKSPACE; }
  return SV_OK;
}

// Mask -> attention -> accept on one stream.  ws_of(need) gives the workspace
// for `need` bytes (or NULL after setting the error): the caller's buffer, or
// the library's own scratch array.
template <class WsOf>
sv_status verify_step_impl(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc, uint64_t* anc,
                           int32_t* depth, int32_t* tree_status, WsOf ws_of, void* stream) {
  sv_status st = check_tree(tree, true);
  if (st) return st;
  if ((st = check_attn(tree, attn))) return st;
  if ((st = check_accept(tree, acc))) return st;
  if (tree->B > 0 && (!anc || !depth || !tree_status)) { set_error("anc/depth/tree_status is NULL"); return SV_E_NULL; }
  AttnPlan ap;
  AcceptPlan cp;
  if (!plan_attention(tree, attn, &ap)) { set_error("no attention plan"); return SV_E_UNSUPPORTED; }
  if (!plan_accept(tree, acc, &cp)) { set_error("no accept plan"); return SV_E_UNSUPPORTED; }
  // the walk's exchange words follow the attention's partial results, so the
  // mask kernel can zero them before attention runs
  const size_t acc_base = align_up(ap.ws_bytes, kWsAlign);
  cp.off_xchg += acc_base;
  void* ws = nullptr;
  if ((st = ws_of(acc_base + cp.ws_bytes, &ws))) return st;
  hipStream_t s = (hipStream_t)stream;
  uint64_t* xchg = tree->B > 0 ? reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + cp.off_xchg) : nullptr;
  if ((st = launch_mask(tree, anc, depth, tree_status, xchg, tree->B > 0 ? accept_exchange_words(cp) : 0, s)))
    return st;
  if ((st = launch_attention(tree, anc, tree_status, attn, ap, ws, s))) return st;
  return launch_accept(tree, tree_status, acc, cp, ws, false, s);
}

// The library's own scratch memory for sv_verify_step_noalloc: one array per
// device, made when the library's code object is loaded on that device and
// kept until the process ends.  Host code never passes `scratch` itself (on
// the host that name only stands for the symbol): it asks the runtime for the
// array's device address once per device and passes that.
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's scratch array (NULL after setting the
// error when the runtime cannot give it).  Looked up once per device, with
// that device current, by the first call on it.
void* scratch_address() {
  static void* addr[64];
  static hipError_t err[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    set_error("no current HIP device (or more than 64)");
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = err[dev] == hipSuccess ? p : nullptr;
  });
  if (!addr[dev]) {
    set_error("scratch array of device %d: hipGetSymbolAddress failed: %s", dev, hipGetErrorString(err[dev]));
    return nullptr;
  }
  return addr[dev];
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" {

sv_status sv_tree_mask_build(const sv_tree* tree, uint64_t* anc, int32_t* depth, int32_t* tree_status,
                             void* stream) {
  clear_error();
  sv_status st = check_tree(tree, false);
  if (st) return st;
  if (tree->B > 0 && (!anc || !depth || !tree_status)) { set_error("anc/depth/tree_status is NULL"); return SV_E_NULL; }
  return launch_mask(tree, anc, depth, tree_status, nullptr, 0, (hipStream_t)stream);
}

sv_status sv_tree_attn(const sv_tree* tree, const uint64_t* anc, const int32_t* tree_status,
                       const sv_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  sv_status st = check_tree(tree, false);
  if (st) return st;
  if ((st = check_attn(tree, a))) return st;
  if (tree->B > 0 && (!anc || !tree_status)) { set_error("anc/tree_status is NULL"); return SV_E_NULL; }
  AttnPlan pl;
  if (!plan_attention(tree, a, &pl)) { set_error("no attention plan"); return SV_E_UNSUPPORTED; }
  if ((st = check_ws(ws, ws_bytes, pl.ws_bytes))) return st;
  return launch_attention(tree, anc, tree_status, a, pl, ws, (hipStream_t)stream);
}

sv_status sv_spec_accept(const sv_tree* tree, int32_t* tree_status, const sv_accept_args* a, void* ws,
                         size_t ws_bytes, void* stream) {
  clear_error();
  sv_status st = check_tree(tree, true);
  if (st) return st;
  if ((st = check_accept(tree, a))) return st;
  if (tree->B > 0 && !tree_status) { set_error("tree_status is NULL"); return SV_E_NULL; }
  AcceptPlan pl;
  if (!plan_accept(tree, a, &pl)) { set_error("no accept plan"); return SV_E_UNSUPPORTED; }
  if ((st = check_ws(ws, ws_bytes, pl.ws_bytes))) return st;
  return launch_accept(tree, tree_status, a, pl, ws, true, (hipStream_t)stream);
}

sv_status sv_verify_step(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc,
                         uint64_t* anc, int32_t* depth, int32_t* tree_status, void* ws, size_t ws_bytes,
                         void* stream) {
  clear_error();
  auto caller_ws = [&](size_t need, void** out) {
    *out = ws;
    return check_ws(ws, ws_bytes, need);
  };
  return verify_step_impl(tree, attn, acc, anc, depth, tree_status, caller_ws, stream);
}

sv_status sv_verify_step_noalloc(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc,
                                 uint64_t* anc, int32_t* depth, int32_t* tree_status, void* stream) {
  clear_error();
  auto own_ws = [&](size_t need, void** out) -> sv_status {
    if (need > kScratchBytes) {
      set_error("sv_verify_step_noalloc: this problem needs %zu bytes of scratch, more than the %zu the library "
                "holds; call sv_verify_step with a workspace of sv_workspace_bytes bytes", need, kScratchBytes);
      return SV_E_WORKSPACE;
    }
    *out = need > 0 ? scratch_address() : nullptr;
    return (need > 0 && !*out) ? SV_E_HIP : SV_OK;
  };
  return verify_step_impl(tree, attn, acc, anc, depth, tree_status, own_ws, stream);
}

sv_status sv_commit_accepted(const sv_tree* tree, int32_t* tree_status, const int32_t* out_nodes,
                             const int32_t* out_count, const sv_commit_args* c, void* stream) {
  clear_error();
  sv_status st = check_tree(tree, false);
  if (st) return st;
  if ((st = check_commit(tree, c))) return st;
  if (tree->B > 0 && (!tree_status || !out_nodes || !out_count)) {
    set_error("tree_status/out_nodes/out_count is NULL");
    return SV_E_NULL;
  }
  return launch_commit(tree, tree_status, out_nodes, out_count, c, (hipStream_t)stream);
}

size_t sv_eagle2_state_bytes(const sv_eagle2_cfg* c) {
  clear_error();
  if (check_eagle2(c)) return 0;
  return eagle2_layout(c).bytes;
}

sv_status sv_eagle2_begin(const sv_eagle2_cfg* c, void* state, size_t state_bytes, const int32_t* root_tokens,
                          void* stream) {
  clear_error();
  sv_status st;
  if ((st = check_eagle2(c))) return st;
  if (c->B == 0) return SV_OK;
  if ((st = check_state(c, state, state_bytes))) return st;
  if (!root_tokens) { set_error("root_tokens is NULL"); return SV_E_NULL; }
  return launch_eagle2_begin(c, state, root_tokens, (hipStream_t)stream);
}

sv_status sv_eagle2_expand(const sv_eagle2_cfg* c, void* state, size_t state_bytes, int32_t step, const float* q,
                           int32_t* frontier, int32_t* frontier_tokens, void* stream) {
  clear_error();
  sv_status st;
  if ((st = check_eagle2(c))) return st;
  if (step < 0 || step >= c->depth) { set_error("step %d outside [0, %d)", step, c->depth); return SV_E_SHAPE; }
  if (c->B == 0) return SV_OK;
  if ((st = check_state(c, state, state_bytes))) return st;
  if (!q) { set_error("q is NULL"); return SV_E_NULL; }
  if (!aligned(q, 16)) { set_error("q must be 16-byte aligned"); return SV_E_UNSUPPORTED; }
  return launch_eagle2_expand(c, state, step, q, frontier, frontier_tokens, (hipStream_t)stream);
}

sv_status sv_eagle2_expand_finish(const sv_eagle2_cfg* c, void* state, size_t state_bytes, int32_t step,
                                  const float* q, int32_t* parent, int32_t* tokens, int32_t* num_nodes,
                                  int32_t* q_row, int32_t* status, void* stream) {
  clear_error();
  sv_status st;
  if ((st = check_eagle2(c))) return st;
  if (step < 0 || step >= c->depth) { set_error("step %d outside [0, %d)", step, c->depth); return SV_E_SHAPE; }
  if (c->B == 0) return SV_OK;
  if ((st = check_state(c, state, state_bytes))) return st;
  if (!q) { set_error("q is NULL"); return SV_E_NULL; }
  if (!aligned(q, 16)) { set_error("q must be 16-byte aligned"); return SV_E_UNSUPPORTED; }
  if (!parent || !tokens || !num_nodes || !q_row || !status) {
    set_error("parent/tokens/num_nodes/q_row/status is NULL");
    return SV_E_NULL;
  }
  return launch_eagle2_expand_finish(c, state, step, q, parent, tokens, num_nodes, q_row, status,
                                     (hipStream_t)stream);
}

sv_status sv_eagle2_finish(const sv_eagle2_cfg* c, const void* state, size_t state_bytes, int32_t* parent,
                           int32_t* tokens, int32_t* num_nodes, int32_t* q_row, int32_t* status, void* stream) {
  clear_error();
  sv_status st;
  if ((st = check_eagle2(c))) return st;
  if (c->B == 0) return SV_OK;
  if ((st = check_state(c, state, state_bytes))) return st;
  if (!parent || !tokens || !num_nodes || !q_row || !status) {
    set_error("parent/tokens/num_nodes/q_row/status is NULL");
    return SV_E_NULL;
  }
  return launch_eagle2_finish(c, state, parent, tokens, num_nodes, q_row, status, (hipStream_t)stream);
}

namespace sv {
namespace {
sv_status check_head(const sv_head_args* a) {
  if (!a) { set_error("draft-head args are NULL"); return SV_E_NULL; }
  if (a->N < 0 || a->d < 32 || a->d % 32 || a->r < 32 || a->r % 32 || a->n < 1) {
    set_error("draft head N=%d d=%d r=%d n=%d (need d, r multiples of 32)", a->N, a->d, a->r, a->n);
    return SV_E_SHAPE;
  }
  if (a->tile < 16 || a->tile > 256 || a->tile % 16 || a->k_tile < 1 || a->k_tile > 8 || a->k_tile > a->tile) {
    set_error("draft head tile=%d k_tile=%d (tile: multiple of 16 in [16, 256]; k_tile 1..8)", a->tile, a->k_tile);
    return SV_E_UNSUPPORTED;
  }
  if (a->r > 2048) { set_error("draft head r=%d > 2048", a->r); return SV_E_UNSUPPORTED; }
  const long n_tiles = (a->n + (long)a->tile - 1) / a->tile;
  if ((long)a->N * n_tiles * a->k_tile > 0x7FFFFFFFL || (a->N + 15) / 16 > 65535) {
    set_error("draft head N=%d too large", a->N);
    return SV_E_UNSUPPORTED;
  }
  return SV_OK;
}
}  // namespace
}  // namespace sv

sv_status sv_draft_head(const sv_head_args* a, void* stream) {
  clear_error();
  sv_status st;
  if ((st = check_head(a))) return st;
  if (a->N == 0) return SV_OK;
  if (!a->h || !a->B || !a->A_sh || !a->perm || !a->W || !a->u || !a->cand_ids || !a->cand_logits) {
    set_error("draft head h/B/A_sh/perm/W/u/cand_ids/cand_logits is NULL");
    return SV_E_NULL;
  }
  const void* ptrs[] = {a->h, a->B, a->A_sh, a->W, a->u};
  for (const void* q : ptrs)
    if (!aligned(q, 16)) { set_error("draft head tensors must be 16-byte aligned"); return SV_E_UNSUPPORTED; }
  return launch_draft_head(a, (hipStream_t)stream);
}

size_t sv_workspace_bytes(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc) {
  clear_error();
  // sizing reads only the scalar fields: pointers may be NULL here
  if (!tree) { set_error("tree is NULL"); return 0; }
  if (tree->B < 0 || tree->T_max < 1 || tree->T_max > kMaxT) { set_error("B=%d T_max=%d", tree->B, tree->T_max); return 0; }
  size_t need = 0;
  if (attn) {
    if (attn->Hq < 1 || attn->Hkv < 1 || attn->Hq % attn->Hkv || (attn->D != 64 && attn->D != 128) ||
        attn->L_max < 0 || (attn->dtype != SV_F32 && attn->dtype != SV_BF16)) {
      set_error("attention sizes Hq=%d Hkv=%d D=%d L_max=%d dtype=%d", attn->Hq, attn->Hkv, attn->D, attn->L_max, attn->dtype);
      return 0;
    }
    AttnPlan pl;
    if (!plan_attention(tree, attn, &pl)) return 0;
    need = pl.ws_bytes;
  }
  if (acc) {
    if (acc->V < 1) { set_error("V = %d < 1", acc->V); return 0; }
    AcceptPlan pl;
    if (!plan_accept(tree, acc, &pl)) { set_error("V = %d unsupported", acc->V); return 0; }
    // both: the layout of sv_verify_step, the walk's words after the attention's
    need = attn ? align_up(need, kWsAlign) + pl.ws_bytes : pl.ws_bytes;
  }
  return need;
}

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_E_NULL: return "null pointer argument";
    case SV_E_SHAPE: return "invalid size or shape";
    case SV_E_DTYPE: return "unknown dtype";
    case SV_E_WORKSPACE: return "workspace missing, too small or misaligned";
    case SV_E_HIP: return "HIP runtime or launch failure";
    case SV_E_UNSUPPORTED: return "unsupported configuration";
    case SV_TREE_E_ROOT: return "tree: root has a parent";
    case SV_TREE_E_PARENT: return "tree: parent index not in [0, i)";
    case SV_TREE_E_COUNT: return "tree: node count outside [1, T_max]";
    case SV_TREE_E_TOKEN: return "tree: token outside [0, V)";
    case SV_TREE_E_NONFINITE: return "tree: non-finite target logit";
    case SV_TREE_E_NOQ: return "tree: stochastic sequence without draft probabilities";
    case SV_TREE_E_SYNC: return "tree: cross-workgroup wait timed out";
    case SV_TREE_E_CACHE: return "commit: no room in the cache";
    case SV_TREE_E_PATH: return "commit: accepted path out of range";
    case SV_TREE_E_PROB: return "tree builder: draft probability outside [0, 1] or NaN";
    default: return "unknown status";
  }
}

const char* sv_last_error(void) { return g_err; }

}  // extern "C"
