// C ABI of the draft-head library: argument checks, workspace carving and
// kernel dispatch.  Nothing here computes model values; every arithmetic
// step runs in the gfx950 kernels of gemm.hip and chain.hip.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "../../include/domino.h"
#include "../../include/domino_bench.h"
#include "internal.h"

namespace {

thread_local std::string g_error;
// process-wide bench settings (domino_bench.h)
std::atomic<int> g_chain_mode{0};
std::atomic<hipEvent_t> g_base_start{nullptr}, g_base_stop{nullptr}, g_chain_start{nullptr}, g_chain_stop{nullptr};

domino_status fail(domino_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
domino_status fail(domino_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

domino_status ok() {
  g_error.clear();
  return DOMINO_OK;
}

domino_status device_fail(hipError_t e, const char* what) {
  return fail(DOMINO_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE_PTR(p, name)                                                                   \
  do {                                                                                         \
    if (!(p)) return fail(DOMINO_ERR_INVALID_ARGUMENT, "%s is NULL", name);                    \
    if (!aligned16(p)) return fail(DOMINO_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

#define OPTIONAL_PTR(p, name)                                                                  \
  do {                                                                                         \
    if ((p) && !aligned16(p)) return fail(DOMINO_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

domino_status check_dims(const domino_dims* d) {
  if (!d) return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->dtype != DOMINO_F32 && d->dtype != DOMINO_BF16)
    return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims.dtype %d is neither DOMINO_F32 nor DOMINO_BF16", d->dtype);
  if (d->hidden <= 0 || d->hidden % 8)
    return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims.hidden %d must be a positive multiple of 8", d->hidden);
  if (d->gru_hidden <= 0 || d->gru_hidden % 8)
    return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims.gru_hidden %d must be a positive multiple of 8", d->gru_hidden);
  if (d->rank <= 0 || d->rank % 8)
    return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims.rank %d must be a positive multiple of 8", d->rank);
  if (d->vocab <= 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims.vocab %d must be positive", d->vocab);
  if (d->block <= 0 || d->block > 64)
    return fail(DOMINO_ERR_INVALID_ARGUMENT, "dims.block %d must be in [1, 64]", d->block);
  if (d->rank > 256) return fail(DOMINO_ERR_UNSUPPORTED, "dims.rank %d exceeds 256", d->rank);
  if ((int64_t)d->hidden + d->gru_hidden > (1 << 30) || (int64_t)d->vocab * 16 > INT32_MAX)
    return fail(DOMINO_ERR_UNSUPPORTED, "dimensions too large");
  return DOMINO_OK;
}

size_t elem_size(const domino_dims* d) { return d->dtype == DOMINO_BF16 ? 2 : 4; }

// Largest workspace the allocation-free chain call serves from its static array.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;

size_t chain_workspace_bytes(const domino_dims* dims, int32_t batch) {
  const int bs = batch > 0 ? batch : 1;
  const int group = bs < dh::kMaxChainGroup ? bs : dh::kMaxChainGroup;
  return dh::chain_layout(dims->hidden, dims->gru_hidden, dims->rank, dims->block, group).total;
}

// Argument checks of the chain calls (everything but the workspace).
domino_status check_chain_args(const domino_dims* dims, const domino_weights* w, const void* H,
                               const float* base_logits, const int32_t* first_tokens, int32_t batch,
                               const int32_t* out_tokens, const float* out_logits) {
  domino_status st = check_dims(dims);
  if (st != DOMINO_OK) return st;
  if (!w) return fail(DOMINO_ERR_INVALID_ARGUMENT, "weights is NULL");
  if (batch < 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "batch %d is negative", batch);
  if (batch == 0) return DOMINO_OK;
  REQUIRE_PTR(w->embed, "weights.embed");
  REQUIRE_PTR(w->w_ih, "weights.w_ih");
  REQUIRE_PTR(w->w_hh, "weights.w_hh");
  REQUIRE_PTR(w->w1, "weights.w1");
  REQUIRE_PTR(w->w2, "weights.w2");
  OPTIONAL_PTR(w->b_ih, "weights.b_ih");
  OPTIONAL_PTR(w->b_hh, "weights.b_hh");
  OPTIONAL_PTR(w->b1, "weights.b1");
  OPTIONAL_PTR(w->b2, "weights.b2");
  OPTIONAL_PTR(w->input_table, "weights.input_table");
  REQUIRE_PTR(H, "H");
  REQUIRE_PTR(base_logits, "base_logits");
  REQUIRE_PTR(first_tokens, "first_tokens");
  REQUIRE_PTR(out_tokens, "out_tokens");
  OPTIONAL_PTR(out_logits, "out_logits");
  return DOMINO_OK;
}

// The chain on a checked workspace `ws` of the size domino_workspace_size gives.
// temperature 0: greedy; > 0: Gumbel-max draws keyed by seed
domino_status run_draft_chain(const domino_dims* dims, const domino_weights* w, const void* H,
                              const float* base_logits, const int32_t* first_tokens, int32_t batch,
                              int32_t* out_tokens, float* out_logits, char* ws, hipStream_t s,
                              float temperature = 0.f, uint64_t seed = 0) {
  const int d = dims->hidden, V = dims->vocab, Hs = dims->gru_hidden, r = dims->rank, P = dims->block;
  const int group_max = batch < dh::kMaxChainGroup ? batch : dh::kMaxChainGroup;
  const dh::ChainLayout L = dh::chain_layout(d, Hs, r, P, group_max);
  const size_t es = elem_size(dims);
  const int mode = g_chain_mode.load();
  const hipEvent_t ev0 = g_chain_start.load(), ev1 = g_chain_stop.load();
  for (int g0 = 0; g0 < batch; g0 += dh::kMaxChainGroup) {
    const int Bg = batch - g0 < dh::kMaxChainGroup ? batch - g0 : dh::kMaxChainGroup;
    const char* Hg = (const char*)H + (size_t)g0 * P * d * es;
    dh::ChainArgs a;
    a.d = d;
    a.V = V;
    a.Hs = Hs;
    a.r = r;
    a.P = P;
    a.B = Bg;
    a.embed = w->embed;
    a.w_ih = w->w_ih;
    a.w_hh = w->w_hh;
    a.w1 = w->w1;
    a.w2 = w->w2;
    a.b_ih = w->b_ih;
    a.b_hh = w->b_hh;
    a.b1 = w->b1;
    a.b2 = w->b2;
    a.xt = w->input_table;
    a.Lb = base_logits + (size_t)g0 * P * V;
    a.out_logits = out_logits ? out_logits + (size_t)g0 * P * V : nullptr;
    a.out_tokens = out_tokens + (size_t)g0 * P;
    a.t0 = first_tokens + g0;
    a.zh = (const float*)(ws + L.zh);
    a.zh_splits = dh::zh_splits(d, r, P, Bg);
    a.zh_stride = Bg * P * r;
    a.zh_sum = (float*)(ws + L.zh_sum);
    a.h = (float*)(ws + L.h);
    a.hb = (uint16_t*)(ws + L.hb);
    a.hb_step = L.hb_step;
    a.act = ws + L.act;
    a.keys = (uint64_t*)(ws + L.keys);
    a.status = (int32_t*)(ws + L.status);
    a.h_step = L.h_step;
    a.ll_h = (uint64_t*)(ws + L.ll_h);
    a.ll_act = (uint64_t*)(ws + L.ll_act);
    a.ll_part = (uint64_t*)(ws + L.ll_part);
    a.ll_tok = (uint64_t*)(ws + L.ll_tok);
    a.epoch = (uint32_t*)(ws + L.status + 4);
    a.marker = (uint64_t*)(ws + L.status + 8);
    a.sig = (uint64_t*)(ws + L.status + 16);
    a.ll_words = (L.trace - L.ll_h) / 8;
    // the hand-off words are cleared again whenever the region they occupy changes
    a.sig_value = ((uint64_t)L.ll_h << 32) ^ (uint64_t)a.ll_words ^ ((uint64_t)P << 56) ^ ((uint64_t)Bg << 48);
    a.stamps = (uint64_t*)(ws + L.stamps);
    a.act_step = L.act_step;
    a.temperature = temperature;
    a.seed_lo = (uint32_t)seed;
    a.seed_hi = (uint32_t)(seed >> 32);
    a.seq_base = g0;
#ifdef DH_TRACE_PHASES
    a.trace = (uint64_t*)(ws + L.trace);
#else
    a.trace = nullptr;
#endif
    hipError_t e = dh::launch_chain(dims->dtype, a, Hg, mode, g0 == 0, s, ev0, ev1);
    if (e != hipSuccess) return device_fail(e, "chain launch");
  }
  return ok();
}

}  // namespace

// Workspace of domino_draft_chain_noalloc: a static array in every device's
// copy of the code object, held until the process ends.  Host code never
// uses this name as an address (on the host it is only a stand-in); it asks
// the runtime for each device's address once and keeps that.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

struct NoAllocDevice {
  std::mutex m;
  void* ptr = nullptr;  // `scratch` on this device
};
NoAllocDevice g_noalloc[64];

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with the device current) and kept.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  NoAllocDevice& d = g_noalloc[dev];
  std::lock_guard<std::mutex> lock(d.m);
  if (!d.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    d.ptr = p;
  }
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* domino_version(void) { return "domino-gfx950 0.1"; }

const char* domino_last_error(void) { return g_error.c_str(); }

void domino_set_timing_events(void* base_start, void* base_stop, void* chain_start, void* chain_stop) {
  const bool base = base_start && base_stop, chain = chain_start && chain_stop;
  g_base_start = base ? (hipEvent_t)base_start : nullptr;
  g_base_stop = base ? (hipEvent_t)base_stop : nullptr;
  g_chain_start = chain ? (hipEvent_t)chain_start : nullptr;
  g_chain_stop = chain ? (hipEvent_t)chain_stop : nullptr;
}

int32_t domino_set_chain_mode(int32_t mode) {
  if (mode < 0 || mode > 3) return -1;
  return g_chain_mode.exchange(mode);
}

size_t domino_workspace_size(const domino_dims* dims, int32_t batch, int32_t op, int32_t nodes, int32_t topm) {
  if (check_dims(dims) != DOMINO_OK) return 0;
  if (batch < 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "batch %d is negative", batch), 0;
  const int bs = batch > 0 ? batch : 1;
  switch (op) {
    case DOMINO_OP_BASE:
      return 0;
    case DOMINO_OP_CHAIN: {
      const int group = bs < dh::kMaxChainGroup ? bs : dh::kMaxChainGroup;
      return dh::chain_layout(dims->hidden, dims->gru_hidden, dims->rank, dims->block, group).total;
    }
    case DOMINO_OP_TREE:
      if (nodes < 1 || nodes > 64) return fail(DOMINO_ERR_INVALID_ARGUMENT, "nodes %d must be in [1, 64]", nodes), 0;
      if (topm < 1 || topm > 256) return fail(DOMINO_ERR_INVALID_ARGUMENT, "topm %d must be in [1, 256]", topm), 0;
      return dh::tree_layout(dims->hidden, dims->gru_hidden, dims->rank, dims->block, bs, nodes, topm).total;
    case DOMINO_OP_CANDIDATES:
      if (topm < 1 || topm > 256) return fail(DOMINO_ERR_INVALID_ARGUMENT, "topm %d must be in [1, 256]", topm), 0;
      return dh::topm_scratch_bytes(bs * dims->block, topm);
    default:
      return fail(DOMINO_ERR_INVALID_ARGUMENT, "op %d is not a domino_op", op), 0;
  }
}

size_t domino_chain_stamp_offset(const domino_dims* dims, int32_t batch) {
  if (domino_workspace_size(dims, batch, DOMINO_OP_CHAIN, 0, 0) == 0) return 0;
  const int bs = batch > 0 ? batch : 1;
  const int group = bs < dh::kMaxChainGroup ? bs : dh::kMaxChainGroup;
  return dh::chain_layout(dims->hidden, dims->gru_hidden, dims->rank, dims->block, group).stamps;
}

domino_status domino_device_status(const void* workspace, void* stream) {
  if (!workspace) return fail(DOMINO_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned16(workspace)) return fail(DOMINO_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "reading the device status");
  if (word == 0) return ok();
  if (word == dh::kDeviceStatusFirstToken)
    return fail(DOMINO_ERR_FIRST_TOKEN, "a first token was outside [0, vocab); that sequence was drafted from token 0");
  if (word == dh::kDeviceStatusTimeout)
    return fail(DOMINO_ERR_TIMEOUT, "a wait between workgroups gave up after 2 s; the outputs are undefined "
                                    "(were the device's CUs shared with other work?)");
  return fail(DOMINO_ERR_DEVICE, "unknown device status %d", word);
}

void domino_release_cache(void) { dh::release_chain_cache(); }

domino_status domino_base_logits(const domino_dims* dims, const domino_weights* w, const void* H, int32_t batch,
                                 float* base_logits, void* stream) {
  domino_status st = check_dims(dims);
  if (st != DOMINO_OK) return st;
  if (!w) return fail(DOMINO_ERR_INVALID_ARGUMENT, "weights is NULL");
  if (batch < 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "batch %d is negative", batch);
  if (batch == 0) return ok();
  REQUIRE_PTR(w->lm_head, "weights.lm_head");
  REQUIRE_PTR(H, "H");
  REQUIRE_PTR(base_logits, "base_logits");
  if ((int64_t)batch * dims->block > INT32_MAX / 2) return fail(DOMINO_ERR_UNSUPPORTED, "batch too large");
  const int M = batch * dims->block;
  hipError_t e = hipSuccess;
  const hipEvent_t ev0 = g_base_start.load(), ev1 = g_base_stop.load();
  if (ev0 && (e = hipEventRecord(ev0, (hipStream_t)stream)) != hipSuccess) return device_fail(e, "timing event");
  e = dh::launch_gemm_nt(dims->dtype, H, dims->hidden, w->lm_head, dims->hidden, base_logits, dims->vocab, M,
                         dims->vocab, dims->hidden, true, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "base-logit GEMM launch");
  if (ev1 && (e = hipEventRecord(ev1, (hipStream_t)stream)) != hipSuccess) return device_fail(e, "timing event");
  return ok();
}

domino_status domino_prepare_input_table(const domino_dims* dims, const domino_weights* w, float* table,
                                        void* stream) {
  domino_status st = check_dims(dims);
  if (st != DOMINO_OK) return st;
  if (!w) return fail(DOMINO_ERR_INVALID_ARGUMENT, "weights is NULL");
  REQUIRE_PTR(w->embed, "weights.embed");
  REQUIRE_PTR(w->w_ih, "weights.w_ih");
  REQUIRE_PTR(table, "table");
  if ((int64_t)3 * dims->gru_hidden > INT32_MAX / 2) return fail(DOMINO_ERR_UNSUPPORTED, "gru_hidden too large");
  // table[v][g] = sum_k embed[v][k] w_ih[g][k]: the vocabulary as the rows of the product
  const hipError_t e = dh::launch_gemm_nt(dims->dtype, w->embed, dims->hidden, w->w_ih, dims->hidden, table,
                                          3 * dims->gru_hidden, dims->vocab, 3 * dims->gru_hidden, dims->hidden, true,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "input-table GEMM launch");
  return ok();
}

domino_status domino_prepare_input_table_f64(const domino_dims* dims, const domino_weights* w, double* table,
                                            void* stream) {
  domino_status st = check_dims(dims);
  if (st != DOMINO_OK) return st;
  if (!w) return fail(DOMINO_ERR_INVALID_ARGUMENT, "weights is NULL");
  REQUIRE_PTR(w->embed, "weights.embed");
  REQUIRE_PTR(w->w_ih, "weights.w_ih");
  REQUIRE_PTR(table, "table");
  const hipError_t e = dh::launch_input_table_f64(dims->dtype, w->embed, w->w_ih, dims->vocab, dims->gru_hidden,
                                                  dims->hidden, table, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "fp64 input-table launch");
  return ok();
}

domino_status domino_draft_chain(const domino_dims* dims, const domino_weights* w, const void* H,
                                 const float* base_logits, const int32_t* first_tokens, int32_t batch,
                                 int32_t* out_tokens, float* out_logits, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  domino_status st = check_chain_args(dims, w, H, base_logits, first_tokens, batch, out_tokens, out_logits);
  if (st != DOMINO_OK) return st;
  if (batch == 0) return ok();
  REQUIRE_PTR(workspace, "workspace");
  const size_t need = domino_workspace_size(dims, batch, DOMINO_OP_CHAIN, 0, 0);
  if (workspace_bytes < need)
    return fail(DOMINO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes required", workspace_bytes,
                need);
  return run_draft_chain(dims, w, H, base_logits, first_tokens, batch, out_tokens, out_logits, (char*)workspace,
                         (hipStream_t)stream);
}

domino_status domino_draft_chain_sampled(const domino_dims* dims, const domino_weights* w, const void* H,
                                         const float* base_logits, const int32_t* first_tokens, int32_t batch,
                                         float temperature, uint64_t seed, int32_t* out_tokens, float* out_logits,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!(temperature >= 0.f) || temperature > 3.0e38f)
    return fail(DOMINO_ERR_INVALID_ARGUMENT, "temperature must be finite and >= 0");
  domino_status st = check_chain_args(dims, w, H, base_logits, first_tokens, batch, out_tokens, out_logits);
  if (st != DOMINO_OK) return st;
  if (batch == 0) return ok();
  REQUIRE_PTR(workspace, "workspace");
  const size_t need = domino_workspace_size(dims, batch, DOMINO_OP_CHAIN, 0, 0);
  if (workspace_bytes < need)
    return fail(DOMINO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes required", workspace_bytes,
                need);
  return run_draft_chain(dims, w, H, base_logits, first_tokens, batch, out_tokens, out_logits, (char*)workspace,
                         (hipStream_t)stream, temperature, seed);
}

domino_status domino_draft_chain_noalloc(const domino_dims* dims, const domino_weights* w, const void* H,
                                         const float* base_logits, const int32_t* first_tokens, int32_t batch,
                                         int32_t* out_tokens, float* out_logits, void* stream) {
  domino_status st = check_chain_args(dims, w, H, base_logits, first_tokens, batch, out_tokens, out_logits);
  if (st != DOMINO_OK) return st;
  if (batch == 0) return ok();
  const size_t need = chain_workspace_bytes(dims, batch);
  if (need > kNoAllocScratchBytes)
    return fail(DOMINO_ERR_UNSUPPORTED,
                "this batch and these dims need %zu bytes of workspace; the allocation-free call holds %zu "
                "(use domino_draft_chain with a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return device_fail(e, "locating the static workspace");
  return run_draft_chain(dims, w, H, base_logits, first_tokens, batch, out_tokens, out_logits, (char*)ws,
                         (hipStream_t)stream);
}

domino_status domino_noalloc_device_status(void* stream) {
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return device_fail(e, "locating the static workspace");
  return domino_device_status(ws, stream);
}

domino_status domino_tree_candidates(const domino_dims* dims, const float* base_logits, int32_t batch, int32_t topm,
                                     int32_t* out_index, float* out_value, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  domino_status st = check_dims(dims);
  if (st != DOMINO_OK) return st;
  if (batch < 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "batch %d is negative", batch);
  if (topm < 1 || topm > 256) return fail(DOMINO_ERR_INVALID_ARGUMENT, "topm %d must be in [1, 256]", topm);
  if (topm > dims->vocab) return fail(DOMINO_ERR_INVALID_ARGUMENT, "topm %d exceeds the vocabulary", topm);
  if (batch == 0) return ok();
  REQUIRE_PTR(base_logits, "base_logits");
  REQUIRE_PTR(out_index, "out_index");
  REQUIRE_PTR(out_value, "out_value");
  REQUIRE_PTR(workspace, "workspace");
  const size_t need = domino_workspace_size(dims, batch, DOMINO_OP_CANDIDATES, 0, topm);
  if (workspace_bytes < need)
    return fail(DOMINO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes required", workspace_bytes,
                need);
  hipError_t e = dh::launch_topm(base_logits, batch * dims->block, dims->vocab, topm, workspace, out_index, out_value,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "top-M launch");
  return ok();
}

domino_status domino_tree_draft(const domino_dims* dims, const domino_weights* w, const void* H,
                                const float* base_logits, const int32_t* first_tokens, int32_t batch, int32_t nodes,
                                int32_t topm, int32_t* out_parents, int32_t* out_tokens, int32_t* out_depth,
                                double* out_scores, void* workspace, size_t workspace_bytes, void* stream) {
  domino_status st = check_dims(dims);
  if (st != DOMINO_OK) return st;
  if (!w) return fail(DOMINO_ERR_INVALID_ARGUMENT, "weights is NULL");
  if (batch < 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "batch %d is negative", batch);
  if (nodes < 1 || nodes > 64) return fail(DOMINO_ERR_INVALID_ARGUMENT, "nodes %d must be in [1, 64]", nodes);
  if (topm < 1 || topm > 256) return fail(DOMINO_ERR_INVALID_ARGUMENT, "topm %d must be in [1, 256]", topm);
  if (topm > dims->vocab) return fail(DOMINO_ERR_INVALID_ARGUMENT, "topm %d exceeds the vocabulary", topm);
  if (dims->gru_hidden > 4096) return fail(DOMINO_ERR_UNSUPPORTED, "gru_hidden %d exceeds 4096 for the tree", dims->gru_hidden);
  if (dh::tree_gru_lds_total(dims->hidden, dims->gru_hidden, dims->dtype) > 160 * 1024)
    return fail(DOMINO_ERR_UNSUPPORTED, "hidden %d with gru_hidden %d exceeds the tree's LDS budget", dims->hidden,
                dims->gru_hidden);
  if (batch == 0) return ok();
  REQUIRE_PTR(w->embed, "weights.embed");
  REQUIRE_PTR(w->w_ih, "weights.w_ih");
  REQUIRE_PTR(w->w_hh, "weights.w_hh");
  REQUIRE_PTR(w->w1, "weights.w1");
  REQUIRE_PTR(w->w2, "weights.w2");
  OPTIONAL_PTR(w->b_ih, "weights.b_ih");
  OPTIONAL_PTR(w->b_hh, "weights.b_hh");
  OPTIONAL_PTR(w->b1, "weights.b1");
  OPTIONAL_PTR(w->b2, "weights.b2");
  OPTIONAL_PTR(w->input_table_f64, "weights.input_table_f64");
  REQUIRE_PTR(H, "H");
  REQUIRE_PTR(base_logits, "base_logits");
  REQUIRE_PTR(first_tokens, "first_tokens");
  REQUIRE_PTR(out_parents, "out_parents");
  REQUIRE_PTR(out_tokens, "out_tokens");
  OPTIONAL_PTR(out_depth, "out_depth");
  OPTIONAL_PTR(out_scores, "out_scores");
  REQUIRE_PTR(workspace, "workspace");
  const size_t need = domino_workspace_size(dims, batch, DOMINO_OP_TREE, nodes, topm);
  if (workspace_bytes < need)
    return fail(DOMINO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes required", workspace_bytes,
                need);
  const dh::TreeLayout L =
      dh::tree_layout(dims->hidden, dims->gru_hidden, dims->rank, dims->block, batch, nodes, topm);
  char* ws = (char*)workspace;
  dh::TreeArgs t;
  t.d = dims->hidden;
  t.V = dims->vocab;
  t.Hs = dims->gru_hidden;
  t.r = dims->rank;
  t.P = dims->block;
  t.B = batch;
  t.N = nodes;
  t.M = topm;
  t.dtype = dims->dtype;
  t.H = H;
  t.embed = w->embed;
  t.w_ih = w->w_ih;
  t.w_hh = w->w_hh;
  t.w1 = w->w1;
  t.w2 = w->w2;
  t.b_ih = w->b_ih;
  t.b_hh = w->b_hh;
  t.b1 = w->b1;
  t.b2 = w->b2;
  t.xt = w->input_table_f64;
  t.Lb = base_logits;
  t.t0 = first_tokens;
  t.out_parents = out_parents;
  t.out_tokens = out_tokens;
  t.out_depth = out_depth;
  t.out_scores = out_scores;
  t.seg_keys = (uint64_t*)(ws + L.seg_keys);
  t.act = (double*)(ws + L.act);
  t.cand_idx = (int32_t*)(ws + L.cand_idx);
  t.cand_val = (float*)(ws + L.cand_val);
  t.zh = (double*)(ws + L.zh);
  t.zh_cur = (double*)(ws + L.zh_cur);
  t.states = (double*)(ws + L.states);
  t.gh = (double*)(ws + L.gh);
  t.heap_score = (double*)(ws + L.heap_score);
  t.heap_meta = (int4*)(ws + L.heap_meta);
  t.heap_count = (int32_t*)(ws + L.heap_count);
  t.cur = ws + L.cur;
  t.status = (int32_t*)(ws + L.status);
  t.heap_cap = L.heap_cap;
  t.ll_act = (uint64_t*)(ws + L.ll_act);
  t.ll_cur = (uint64_t*)(ws + L.ll_cur);
  t.epoch = (uint32_t*)(ws + L.status + 4);
  t.marker = (uint64_t*)(ws + L.status + 8);
  t.sig = (uint64_t*)(ws + L.status + 16);
  t.ll_words = (L.total - L.ll_act) / 8;
  // the hand-off words are cleared again whenever the region they occupy changes
  t.sig_value = ((uint64_t)L.ll_act << 32) ^ (uint64_t)t.ll_words ^ ((uint64_t)nodes << 56) ^ ((uint64_t)batch << 40) ^
                0x7472656500000000ull;
  hipError_t e = dh::launch_tree(t, true, (hipStream_t)stream, g_chain_start.load(), g_chain_stop.load());
  if (e != hipSuccess) return device_fail(e, "tree launch");
  return ok();
}

domino_status domino_tree_verify_inputs(const int32_t* parents, const int32_t* tokens, const int32_t* first_tokens,
                                        const int32_t* start_positions, int32_t batch, int32_t nodes,
                                        uint8_t* out_mask, int32_t* out_positions, int32_t* out_tokens, void* stream) {
  if (batch < 0) return fail(DOMINO_ERR_INVALID_ARGUMENT, "batch %d is negative", batch);
  if (nodes < 1 || nodes > 64) return fail(DOMINO_ERR_INVALID_ARGUMENT, "nodes %d must be in [1, 64]", nodes);
  if (batch == 0) return ok();
  REQUIRE_PTR(parents, "parents");
  REQUIRE_PTR(tokens, "tokens");
  REQUIRE_PTR(first_tokens, "first_tokens");
  OPTIONAL_PTR(start_positions, "start_positions");
  REQUIRE_PTR(out_mask, "out_mask");
  REQUIRE_PTR(out_positions, "out_positions");
  REQUIRE_PTR(out_tokens, "out_tokens");
  const hipError_t e = dh::launch_tree_verify_inputs(parents, tokens, first_tokens, start_positions, batch, nodes,
                                                     out_mask, out_positions, out_tokens, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "verification-input launch");
  return ok();
}

}  // extern "C"
