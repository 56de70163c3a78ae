// C ABI of the library: argument validation, workspace layout and the
// launch sequence of each entry point.  Nothing here allocates device memory
// or synchronises the host; every check runs before the first launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "hsa_sparse.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;
thread_local hsa_sparse_event_t g_stage_events[5];
thread_local bool g_record_stages = false;

// per-kernel timing: start/stop events of kernel i of each call, and the
// names of the last call's kernels
constexpr int kMaxKernelEvents = 64;
thread_local hsa_sparse_event_t g_kernel_start[kMaxKernelEvents];
thread_local hsa_sparse_event_t g_kernel_stop[kMaxKernelEvents];
thread_local int g_n_kernel_events = 0;
thread_local int g_kernel_idx = 0;
thread_local std::string g_kernel_names;

// Opened by every entry point that launches kernels: numbering restarts.
struct CallScope {
  CallScope() {
    g_kernel_idx = 0;
    if (g_n_kernel_events) g_kernel_names.clear();
  }
};

hsa_sparse_status_t fail(hsa_sparse_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hsa_sparse_status_t hip_fail(hipError_t e, const char* where) {
  return fail(HSA_SPARSE_HIP_ERROR, "%s: %s", where, hipGetErrorString(e));
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

enum : unsigned { kSummary = 1u, kSelect = 2u, kAttn = 4u, kFlat = 8u, kHeads = 16u, kHeadSel = 32u };

constexpr long long kMaxHeadTokens = 131072;  // top_m * block of a per-head list

// Checks shared by every entry point; `parts` names the fields the entry
// point reads.  Fills `d` on success.
hsa_sparse_status_t check_shape(const hsa_sparse_shape_t* s, hsa::Dims& d, unsigned parts) {
  const bool need_index = parts & (kSummary | kSelect);
  const bool need_attn = parts & kAttn;
  if (!s) return fail(HSA_SPARSE_INVALID_ARG, "shape is NULL");
  if (s->batch < 0 || s->seq_len < 0 || s->n_q < 0)
    return fail(HSA_SPARSE_INVALID_ARG, "negative batch / seq_len / n_q");
  if (s->n_q > s->seq_len) return fail(HSA_SPARSE_INVALID_ARG, "n_q (%d) > seq_len (%d)", s->n_q, s->seq_len);
  if (parts & kSelect) {
    if (s->top_m < 2) return fail(HSA_SPARSE_INVALID_ARG, "top_m must be >= 2 (first and last block are kept)");
    if (s->top_k < 1) return fail(HSA_SPARSE_INVALID_ARG, "top_k must be >= 1");
  }
  if (parts & kFlat) {
    if (s->top_k < 1) return fail(HSA_SPARSE_INVALID_ARG, "top_k must be >= 1");
    if (s->d_index != 64 && s->d_index != 128)
      return fail(HSA_SPARSE_UNSUPPORTED, "d_index must be 64 or 128 (got %d)", s->d_index);
    // token positions and the padded score-row length are 32-bit integers
    if (s->seq_len > (1 << 30)) return fail(HSA_SPARSE_UNSUPPORTED, "flat top-k needs seq_len <= 2^30");
  }
  if (need_index) {
    if (s->d_index != 64 && s->d_index != 128)
      return fail(HSA_SPARSE_UNSUPPORTED, "d_index must be 64 or 128 (got %d)", s->d_index);
    if (!is_pow2(s->block) || s->block < 8 || s->block > 128)
      return fail(HSA_SPARSE_UNSUPPORTED, "block must be a power of two in [8, 128] (got %d)", s->block);
    if (s->n_landmarks != 1 && s->n_landmarks != 2 && s->n_landmarks != 4)
      return fail(HSA_SPARSE_UNSUPPORTED, "n_landmarks must be 1, 2 or 4 (got %d)", s->n_landmarks);
    const long long nb = ((long long)s->seq_len + s->block - 1) / s->block;
    if (nb - 2 > 32768) return fail(HSA_SPARSE_UNSUPPORTED, "too many blocks (%lld > 32770)", nb);
    if ((parts & kSelect) && (long long)s->top_m * s->block > 32768 &&
        (long long)s->top_k < (long long)s->top_m * s->block)
      return fail(HSA_SPARSE_UNSUPPORTED, "top_m * block > 32768 candidates with top_k < top_m * block");
  }
  if (parts & kHeads) {
    // per-head selection: the landmarks come from K (head_dim wide rows)
    if (s->head_dim != 128) return fail(HSA_SPARSE_UNSUPPORTED, "head_dim must be 128 (got %d)", s->head_dim);
    if (!is_pow2(s->block) || s->block < 8 || s->block > 128)
      return fail(HSA_SPARSE_UNSUPPORTED, "block must be a power of two in [8, 128] (got %d)", s->block);
    if (s->n_landmarks != 1 && s->n_landmarks != 2 && s->n_landmarks != 4)
      return fail(HSA_SPARSE_UNSUPPORTED, "n_landmarks must be 1, 2 or 4 (got %d)", s->n_landmarks);
    if (s->n_heads_q < 1 || s->n_heads_kv < 1 || s->n_heads_q % s->n_heads_kv != 0)
      return fail(HSA_SPARSE_INVALID_ARG, "n_heads_kv must divide n_heads_q");
    if (s->n_heads_kv > 16) return fail(HSA_SPARSE_UNSUPPORTED, "at most 16 kv heads (got %d)", s->n_heads_kv);
  }
  if (parts & kHeadSel) {
    if (s->top_m < 2) return fail(HSA_SPARSE_INVALID_ARG, "top_m must be >= 2 (first and last chunk are kept)");
    const long long nb = ((long long)s->seq_len + s->block - 1) / s->block;
    if (nb - 2 > 32768) return fail(HSA_SPARSE_UNSUPPORTED, "too many chunks (%lld > 32770)", nb);
    if ((long long)s->top_m * s->block > kMaxHeadTokens)
      return fail(HSA_SPARSE_UNSUPPORTED, "top_m * block > %lld tokens per head", kMaxHeadTokens);
    if ((long long)s->batch * s->n_q * s->n_heads_q > (1ll << 30))
      return fail(HSA_SPARSE_UNSUPPORTED, "batch * n_q * n_heads_q too large");
  }
  if (!(parts & (kSelect | kHeads)) && need_attn && s->top_k < 1)
    return fail(HSA_SPARSE_INVALID_ARG, "top_k must be >= 1");
  if (need_attn) {
    if (s->head_dim != 128) return fail(HSA_SPARSE_UNSUPPORTED, "head_dim must be 128 (got %d)", s->head_dim);
    if (s->n_heads_q < 1 || s->n_heads_kv < 1 || s->n_heads_q % s->n_heads_kv != 0)
      return fail(HSA_SPARSE_INVALID_ARG, "n_heads_kv must divide n_heads_q");
    if (s->n_heads_q / s->n_heads_kv > 16)
      return fail(HSA_SPARSE_UNSUPPORTED, "at most 16 query heads per kv head");
    if (!(s->scale == s->scale)) return fail(HSA_SPARSE_INVALID_ARG, "scale is NaN");
    // a kv row's byte offset inside its sequence is a 31-bit integer
    if ((long long)s->seq_len * s->n_heads_kv * 256 > 0x7FFFFFFFll)
      return fail(HSA_SPARSE_UNSUPPORTED, "seq_len * n_heads_kv * 256 bytes exceeds 2^31");
  }
  const long long nq_total = (long long)s->batch * s->n_q;
  if (nq_total > (1ll << 30)) return fail(HSA_SPARSE_UNSUPPORTED, "batch * n_q too large");
  // attention numbers its (query, head) rows with 32-bit integers
  if (need_attn && nq_total * s->n_heads_q > (1ll << 30))
    return fail(HSA_SPARSE_UNSUPPORTED, "batch * n_q * n_heads_q too large");
  d.b = s->batch;
  d.L = s->seq_len;
  d.nq = s->n_q;
  d.dI = s->d_index;
  d.B = s->block > 0 ? s->block : 1;
  d.nL = s->n_landmarks;
  d.m = s->top_m;
  d.k = s->top_k;
  d.Hq = s->n_heads_q;
  d.Hkv = s->n_heads_kv;
  d.d = s->head_dim;
  d.scale = s->scale;
  d.nb = (int)(((long long)s->seq_len + d.B - 1) / d.B);
  if ((parts & kFlat) && !hsa::flat_topk_supported(d))
    return fail(HSA_SPARSE_UNSUPPORTED, "flat top-k needs top_k <= 8192 when top_k < seq_len (got %d)",
                s->top_k);
  g_last_error.clear();
  return HSA_SPARSE_OK;
}

bool empty(const hsa::Dims& d) { return d.b == 0 || d.nq == 0; }

// Scratch of hsa_forward_noalloc: a fixed-size device array in the code
// object, so that call allocates nothing.  Every GPU the library runs on
// holds its own copy until the process ends.  Its host-side name is not a
// device address: host code uses only the per-device address that
// hipGetSymbolAddress returns (kept in g_scratch_ptr).
static __device__ __align__(256) unsigned char scratch[HSA_SPARSE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // guarded by g_scratch_mu

// The device address of `scratch` on the stream's device, looked up once
// per device with that device current.
hsa_sparse_status_t static_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HSA_SPARSE_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (back != hipSuccess) return hip_fail(back, "hipSetDevice");
    if (!p) return fail(HSA_SPARSE_HIP_ERROR, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HSA_SPARSE_OK;
}

// Super-block level of the three-level selection.
struct Level3 {
  int lgG, m2;
  uint16_t* S2;
  int32_t* sup;
};

constexpr int kMaxGroup = 4096;
constexpr int kMaxLevel2Slots = 8192;

// group: blocks per super-block; top_m2: kept super-blocks.  Sets lgG.
hsa_sparse_status_t check_level3(int32_t group, int32_t top_m2, int& lgG) {
  if (!is_pow2(group) || group > kMaxGroup)
    return fail(HSA_SPARSE_UNSUPPORTED, "group must be a power of two in [1, %d] (got %d)", kMaxGroup, group);
  if (top_m2 < 2) return fail(HSA_SPARSE_INVALID_ARG, "top_m2 must be >= 2 (first and last super-block are kept)");
  if ((long long)top_m2 * group > kMaxLevel2Slots)
    return fail(HSA_SPARSE_UNSUPPORTED, "top_m2 * group > %d candidate blocks", kMaxLevel2Slots);
  lgG = 0;
  while ((1 << lgG) < group) ++lgG;
  return HSA_SPARSE_OK;
}

struct ForwardLayout {
  size_t blk_off, tok_off, stage_off, total;
};

// per-head forward: chunk lists, token lists, then scores / attention
// scratch (never live at the same time)
ForwardLayout heads_layout(const hsa::Dims& d) {
  using hsa::align_up;
  ForwardLayout f;
  const size_t rows = (size_t)d.b * d.nq * d.Hq;
  f.blk_off = 0;
  f.tok_off = align_up(rows * d.m * sizeof(int32_t));
  f.stage_off = f.tok_off + align_up(rows * d.m * d.B * sizeof(int32_t));
  f.total = f.stage_off + std::max(hsa::head_scores_ws_bytes(d), hsa::head_attn_ws_bytes(d));
  return f;
}

// ---- prefill attention in query chunks
// Long prefills run the attention on chunks of consecutive queries holding
// at least kAttnChunkRows (query, kv head) rows, one launch each, in order
// on the caller's stream: a chunk of queries [i0, i1) of a sequence is
// itself a prefill call (n_q = i1 - i0 over the context's first
// L - (n_q - i1) tokens).  Each query's attention is independent, and a
// chunk of at least 2048 rows is never split, so the outputs are the bits
// of one launch.  2048 rows are 512 workgroups, one round of the chip at two
// per CU: every wave of a launch starts together and walks its ascending
// list at about the same pace as the others, so the rows they gather at
// any moment are close together and stay in the L2s and the MALL.
// Measured on the 64K prefill (attention of all 65536 queries, one kv
// head): one launch 5.50 ms, chunks of 32768 queries 4.94, 16384 4.64, 8192
// 4.54, 4096 4.42, 2048 4.35 ms; 1024-query chunks are split (fewer than
// 2048 rows) and take 6.29 ms.
constexpr int kAttnChunkRows = 2048;

int attn_chunk_q(const hsa::Dims& d) { return (kAttnChunkRows + d.Hkv - 1) / d.Hkv; }

hsa::Dims chunk_dims(const hsa::Dims& d, int i0, int i1) {
  hsa::Dims c = d;
  c.b = 1;
  c.nq = i1 - i0;
  c.L = d.L - (d.nq - i1);
  c.nb = (c.L + c.B - 1) / c.B;
  return c;
}

// chunks per sequence (0: one launch for the whole batch).  The last chunk
// of a sequence may be shorter (and then split if it has few rows).  Below
// four chunks the extra launches cost more than they gain (4096-row
// prefills measured the same or slower in 2048-row launches).
int attn_chunks(const hsa::Dims& d) {
  const int cq = attn_chunk_q(d);
  if (d.lens || d.nq < 4 * cq) return 0;
  return (d.nq + cq - 1) / cq;
}

size_t chunked_attn_ws_bytes(const hsa::Dims& d) {
  size_t ws = 0;
  const int n = attn_chunks(d);
  for (int c = 0; c < n; ++c)  // every sequence has the same chunk shapes
    ws = std::max(ws, hsa::sparse_attn_ws_bytes(
                          chunk_dims(d, c * attn_chunk_q(d), std::min(d.nq, (c + 1) * attn_chunk_q(d)))));
  return ws;
}

// Decode-shaped calls run the token select inside the attention launch
// (hsa::launch_select_attn); prefill keeps the two steps apart.
bool fuse_select_attn(const hsa::Dims& d) { return !attn_chunks(d) && hsa::select_attn_fusable(d); }

ForwardLayout forward_layout(const hsa::Dims& d) {
  using hsa::align_up;
  ForwardLayout f;
  const size_t nqt = (size_t)d.b * d.nq;
  f.blk_off = 0;
  f.tok_off = align_up(nqt * d.m * sizeof(int32_t));
  f.stage_off = f.tok_off + align_up(nqt * d.k * sizeof(int32_t));
  size_t stage = hsa::block_topm_ws_bytes(d);
  if (fuse_select_attn(d)) {  // the scores and the attention partials are live together
    stage = std::max(stage, hsa::select_attn_ws_bytes(d));
  } else {
    stage = std::max(stage, hsa::token_topk_ws_bytes(d));
    stage = std::max(stage, attn_chunks(d) ? chunked_attn_ws_bytes(d) : hsa::sparse_attn_ws_bytes(d));
  }
  f.total = f.stage_off + stage;
  return f;
}

}  // namespace

namespace hsa {

void kernel_slot(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  *start = nullptr;
  *stop = nullptr;
  if (!g_n_kernel_events) return;
  const int i = g_kernel_idx++;
  if (i < g_n_kernel_events) {
    *start = (hipEvent_t)g_kernel_start[i];
    *stop = (hipEvent_t)g_kernel_stop[i];
  }
  // "(k_name<T, U>)" -> "k_name"
  std::string n(name);
  const size_t a = n.find_first_not_of("( ");
  n = n.substr(a == std::string::npos ? 0 : a);
  const size_t e = n.find_first_of("<) ");
  if (e != std::string::npos) n.resize(e);
  if (!g_kernel_names.empty()) g_kernel_names += ",";
  g_kernel_names += n;
}

}  // namespace hsa

extern "C" {

hsa_sparse_status_t hsa_sparse_set_kernel_events(hsa_sparse_event_t const* start, hsa_sparse_event_t const* stop,
                                                 int n_events) {
  if (n_events == 0 && !start && !stop) {
    g_n_kernel_events = 0;
    g_kernel_names.clear();
    return HSA_SPARSE_OK;
  }
  if (n_events < 1 || n_events > kMaxKernelEvents || !start || !stop)
    return fail(HSA_SPARSE_INVALID_ARG, "need 1 to %d start and stop events (or 0 and NULLs)", kMaxKernelEvents);
  for (int i = 0; i < n_events; ++i) {
    g_kernel_start[i] = start[i];
    g_kernel_stop[i] = stop[i];
  }
  g_n_kernel_events = n_events;
  g_kernel_names.clear();
  return HSA_SPARSE_OK;
}

const char* hsa_sparse_last_kernels(void) { return g_kernel_names.c_str(); }

const char* hsa_sparse_strerror(hsa_sparse_status_t status) {
  // a C caller may pass any int; read the bits as one, since a value
  // outside the enumerators' range is not a valid C++ enum value
  static_assert(sizeof(status) == sizeof(int), "C enum is int-sized");
  int code;
  std::memcpy(&code, &status, sizeof code);
  switch (code) {
    case HSA_SPARSE_OK: return "success";
    case HSA_SPARSE_INVALID_ARG: return "invalid argument";
    case HSA_SPARSE_UNSUPPORTED: return "unsupported shape";
    case HSA_SPARSE_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HSA_SPARSE_HIP_ERROR: return "HIP error";
  }
  return "unknown status";
}

const char* hsa_sparse_last_error(void) { return g_last_error.c_str(); }

hsa_sparse_status_t hsa_sparse_set_stage_events(hsa_sparse_event_t const* events, int n_events) {
  if (n_events == 0 && !events) {
    g_record_stages = false;
    return HSA_SPARSE_OK;
  }
  if (n_events != 5 || !events) return fail(HSA_SPARSE_INVALID_ARG, "need 5 events (or 0 and NULL)");
  bool any = false;
  for (int i = 0; i < 5; ++i) {
    g_stage_events[i] = events[i];
    any = any || events[i];
  }
  if (!any) return fail(HSA_SPARSE_INVALID_ARG, "all 5 events are NULL");
  g_record_stages = true;
  return HSA_SPARSE_OK;
}

size_t hsa_sparse_workspace_size(const hsa_sparse_shape_t* shape, int op) {
  hsa::Dims d;
  switch (op) {
    case HSA_SPARSE_OP_BLOCK_SUMMARY: return 0;  // streams kI once, no scratch
    case HSA_SPARSE_OP_BLOCK_TOPM:
      return check_shape(shape, d, kSelect | kSummary) == HSA_SPARSE_OK ? hsa::block_topm_ws_bytes(d) : 0;
    case HSA_SPARSE_OP_TOKEN_TOPK:
      return check_shape(shape, d, kSelect | kSummary) == HSA_SPARSE_OK ? hsa::token_topk_ws_bytes(d) : 0;
    case HSA_SPARSE_OP_SPARSE_ATTN:
      return check_shape(shape, d, kAttn) == HSA_SPARSE_OK ? hsa::sparse_attn_ws_bytes(d) : 0;
    case HSA_SPARSE_OP_FORWARD:
      return check_shape(shape, d, kSummary | kSelect | kAttn) == HSA_SPARSE_OK ? forward_layout(d).total : 0;
    case HSA_SPARSE_OP_FLAT_TOPK:
      return check_shape(shape, d, kFlat) == HSA_SPARSE_OK ? hsa::flat_topk_ws_bytes(d) : 0;
    case HSA_SPARSE_OP_HEAD_TOPM:
      return check_shape(shape, d, kHeads | kHeadSel) == HSA_SPARSE_OK ? hsa::head_scores_ws_bytes(d) : 0;
    case HSA_SPARSE_OP_BLOCK_SCORE_MAX:
      return check_shape(shape, d, kSelect | kSummary) == HSA_SPARSE_OK ? hsa::block_score_max_ws_bytes(d) : 0;
    case HSA_SPARSE_OP_FORWARD_HEADS:
      return check_shape(shape, d, kHeads | kHeadSel | kAttn) == HSA_SPARSE_OK ? heads_layout(d).total : 0;
    default: return 0;
  }
}

hsa_sparse_status_t hsa_block_summary(const hsa_sparse_shape_t* shape, const uint16_t* kI, const int8_t* landmark_W,
                                      int32_t start_block, uint16_t* S, hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSummary);
  if (st != HSA_SPARSE_OK) return st;
  if (start_block < 0) return fail(HSA_SPARSE_INVALID_ARG, "start_block < 0");
  if (d.nL > 1 && !landmark_W) return fail(HSA_SPARSE_INVALID_ARG, "n_landmarks > 1 needs landmark_W");
  if (d.b == 0 || d.L == 0 || start_block >= d.nb) return HSA_SPARSE_OK;
  if (!kI || !S) return fail(HSA_SPARSE_INVALID_ARG, "kI or S is NULL");
  hipError_t e = hsa::launch_block_summary(d, kI, landmark_W, start_block, S, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_block_summary");
}

hsa_sparse_status_t hsa_block_topm(const hsa_sparse_shape_t* shape, const uint16_t* qI, const uint16_t* S,
                                   int32_t* blk, void* workspace, size_t workspace_bytes,
                                   hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSelect | kSummary);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!qI || !S || !blk) return fail(HSA_SPARSE_INVALID_ARG, "qI, S or blk is NULL");
  const size_t need = hsa::block_topm_ws_bytes(d);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "block_topm needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_block_topm(d, qI, S, blk, workspace, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_block_topm");
}

hsa_sparse_status_t hsa_block_score_max(const hsa_sparse_shape_t* shape, const uint16_t* qI, const uint16_t* S,
                                        float* out, void* workspace, size_t workspace_bytes,
                                        hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSelect | kSummary);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!qI || !S || !out) return fail(HSA_SPARSE_INVALID_ARG, "qI, S or out is NULL");
  const size_t need = hsa::block_score_max_ws_bytes(d);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "block_score_max needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_block_score_max(d, qI, S, out, workspace, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_block_score_max");
}

hsa_sparse_status_t hsa_token_topk(const hsa_sparse_shape_t* shape, const uint16_t* qI, const uint16_t* kI,
                                   const int32_t* blk, int32_t* tok, void* workspace, size_t workspace_bytes,
                                   hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSelect | kSummary);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!qI || !kI || !blk || !tok) return fail(HSA_SPARSE_INVALID_ARG, "qI, kI, blk or tok is NULL");
  const size_t need = hsa::token_topk_ws_bytes(d);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "token_topk needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_token_topk(d, qI, kI, blk, tok, workspace, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_token_topk");
}

hsa_sparse_status_t hsa_flat_topk(const hsa_sparse_shape_t* shape, const uint16_t* qI, const uint16_t* kI,
                                  int32_t* tok, void* workspace, size_t workspace_bytes, hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kFlat);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!qI || !kI || !tok) return fail(HSA_SPARSE_INVALID_ARG, "qI, kI or tok is NULL");
  const size_t need = hsa::flat_topk_ws_bytes(d);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "flat_topk needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_flat_topk(d, qI, kI, tok, workspace, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_flat_topk");
}

hsa_sparse_status_t hsa_sparse_attn(const hsa_sparse_shape_t* shape, const uint16_t* Q, const uint16_t* K,
                                    const uint16_t* V, const int32_t* tok, float* O, float* lse, void* workspace,
                                    size_t workspace_bytes, hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kAttn);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!Q || !K || !V || !tok || !O) return fail(HSA_SPARSE_INVALID_ARG, "Q, K, V, tok or O is NULL");
  const size_t need = hsa::sparse_attn_ws_bytes(d);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "sparse_attn needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_sparse_attn(d, Q, K, V, tok, O, lse, workspace, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_sparse_attn");
}

// Steps 1-4 on one stream for validated dims (d.lens set for per-sequence
// lengths).  `who` names the entry point in error messages.
// With `l3`, step 2 selects through super-blocks.
static hsa_sparse_status_t forward_impl(const hsa::Dims& d, const char* who, const uint16_t* qI,
                                        const uint16_t* kI, const int8_t* landmark_W, int32_t summary_start_block,
                                        uint16_t* S, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                        int32_t* blk_out, int32_t* tok_out, float* O, float* lse, void* workspace,
                                        size_t workspace_bytes, hsa_sparse_stream_t stream,
                                        const Level3* l3 = nullptr) {
  CallScope calls;
  if (d.nL > 1 && !landmark_W) return fail(HSA_SPARSE_INVALID_ARG, "n_landmarks > 1 needs landmark_W");
  if (empty(d)) return HSA_SPARSE_OK;
  if (!qI || !kI || !S || !Q || !K || !V || !O)
    return fail(HSA_SPARSE_INVALID_ARG, "qI, kI, S, Q, K, V or O is NULL");
  if (l3 && (!l3->S2 || !l3->sup)) return fail(HSA_SPARSE_INVALID_ARG, "S2 or sup_out is NULL");
  const ForwardLayout f = forward_layout(d);
  if (workspace_bytes < f.total || !workspace)
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "%s needs %zu workspace bytes", who, f.total);
  char* ws = static_cast<char*>(workspace);
  int32_t* blk = blk_out ? blk_out : reinterpret_cast<int32_t*>(ws + f.blk_off);
  int32_t* tok = tok_out ? tok_out : reinterpret_cast<int32_t*>(ws + f.tok_off);
  void* stage = ws + f.stage_off;
  const bool rec = g_record_stages;
  auto hf = [&](hipError_t err, const char* step) {
    return fail(HSA_SPARSE_HIP_ERROR, "%s (%s): %s", who, step, hipGetErrorString(err));
  };
#define HSA_MARK(i)                                                              \
  if (rec && g_stage_events[i]) {                                               \
    hipError_t er = hipEventRecord((hipEvent_t)g_stage_events[i], stream);       \
    if (er != hipSuccess) return hf(er, "stage event");                    \
  }
  HSA_MARK(0)
  // Decode: the only re-summarised block is each query's own, always-kept
  // block, whose score is never read, so its summary is folded into the
  // block-score launch instead of preceding it.
  // (With super-blocks the query's own super-block is always kept too, and
  // its summary is rebuilt in the same folded workgroup.)
  const bool fold = l3 ? hsa::block_topm_3level_can_fold(d, l3->lgG, l3->m2, summary_start_block)
                       : hsa::block_topm_can_fold(d, summary_start_block);
  hipError_t e = hipSuccess;
  if (!fold) e = hsa::launch_block_summary(d, kI, landmark_W, summary_start_block, S, stream);
  if (e != hipSuccess) return hf(e, "block summary");
  if (l3 && !fold) e = hsa::launch_super_summary(d, l3->lgG, S, summary_start_block >> l3->lgG, l3->S2, stream);
  if (e != hipSuccess) return hf(e, "super-block summary");
  HSA_MARK(1)
  const hsa::SummaryFold sf{kI, landmark_W, S, summary_start_block};
  // Decode: the select runs inside the attention launch (stage 3 is then
  // the scorer alone and stage 4 the select, the attention and the merge);
  // with one summary vector per block, the token scores are also computed
  // in the block top-m launch (stage 3 is then empty).
  const bool fuse = fuse_select_attn(d);
  const bool fuse_bt = fuse && !l3 && hsa::block_token_fusable(d, fold ? &sf : nullptr);
  if (fuse_bt) {
    e = hsa::launch_block_token_decode(d, qI, S, kI, blk, static_cast<float*>(stage), stream, fold ? &sf : nullptr);
  } else if (l3) {
    e = hsa::launch_block_topm_3level(d, l3->lgG, l3->m2, qI, S, l3->S2, l3->sup, blk, stage, stream,
                                      fold ? &sf : nullptr, l3->S2);
  } else {
    e = hsa::launch_block_topm(d, qI, S, blk, stage, stream, fold ? &sf : nullptr);
  }
  if (e != hipSuccess) return hf(e, "block top-m");
  HSA_MARK(2)
  if (fuse_bt) e = hipSuccess;
  else if (fuse) e = hsa::launch_token_scores(d, qI, kI, blk, stage, stream);
  else e = hsa::launch_token_topk(d, qI, kI, blk, tok, stage, stream);
  if (e != hipSuccess) return hf(e, "token top-k");
  HSA_MARK(3)
  if (fuse) {
    e = hsa::launch_select_attn(d, static_cast<const float*>(stage), blk, tok, Q, K, V, O, lse,
                                static_cast<char*>(stage) + hsa::token_topk_ws_bytes(d), stream);
    if (e != hipSuccess) return hf(e, "token select + sparse attention");
  } else if (const int nc = attn_chunks(d)) {
    for (int b = 0; b < d.b; ++b)
      for (int c = 0; c < nc; ++c) {
        const int i0 = c * attn_chunk_q(d), i1 = std::min(d.nq, (c + 1) * attn_chunk_q(d));
        const size_t q0 = (size_t)b * d.nq + i0;
        const size_t kv0 = (size_t)b * d.L * d.Hkv * d.d;
        e = hsa::launch_sparse_attn(chunk_dims(d, i0, i1), Q + q0 * d.Hq * d.d, K + kv0, V + kv0, tok + q0 * d.k,
                                    O + q0 * d.Hq * d.d, lse ? lse + q0 * d.Hq : nullptr, stage, stream);
        if (e != hipSuccess) return hf(e, "sparse attention");
      }
  } else {
    e = hsa::launch_sparse_attn(d, Q, K, V, tok, O, lse, stage, stream);
    if (e != hipSuccess) return hf(e, "sparse attention");
  }
  HSA_MARK(4)
#undef HSA_MARK
  return HSA_SPARSE_OK;
}

hsa_sparse_status_t hsa_forward(const hsa_sparse_shape_t* shape, const uint16_t* qI, const uint16_t* kI,
                                const int8_t* landmark_W, int32_t summary_start_block, uint16_t* S,
                                const uint16_t* Q, const uint16_t* K, const uint16_t* V, int32_t* blk_out,
                                int32_t* tok_out, float* O, float* lse, void* workspace, size_t workspace_bytes,
                                hsa_sparse_stream_t stream) {
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSummary | kSelect | kAttn);
  if (st != HSA_SPARSE_OK) return st;
  if (summary_start_block < 0) return fail(HSA_SPARSE_INVALID_ARG, "summary_start_block < 0");
  return forward_impl(d, "hsa_forward", qI, kI, landmark_W, summary_start_block, S, Q, K, V, blk_out, tok_out, O,
                      lse, workspace, workspace_bytes, stream);
}

hsa_sparse_status_t hsa_forward_noalloc(const hsa_sparse_shape_t* shape, const uint16_t* qI, const uint16_t* kI,
                                        const int8_t* landmark_W, int32_t summary_start_block, uint16_t* S,
                                        const uint16_t* Q, const uint16_t* K, const uint16_t* V, int32_t* blk_out,
                                        int32_t* tok_out, float* O, float* lse, hsa_sparse_stream_t stream) {
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSummary | kSelect | kAttn);
  if (st != HSA_SPARSE_OK) return st;
  if (summary_start_block < 0) return fail(HSA_SPARSE_INVALID_ARG, "summary_start_block < 0");
  const size_t need = forward_layout(d).total;
  if (need > (size_t)HSA_SPARSE_NOALLOC_SCRATCH_BYTES)
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "hsa_forward_noalloc: this shape needs %zu scratch bytes, "
                "more than the %zu of the static scratch", need, (size_t)HSA_SPARSE_NOALLOC_SCRATCH_BYTES);
  if (empty(d)) return HSA_SPARSE_OK;
  void* ws = nullptr;
  st = static_scratch(stream, &ws);
  if (st != HSA_SPARSE_OK) return st;
  return forward_impl(d, "hsa_forward_noalloc", qI, kI, landmark_W, summary_start_block, S, Q, K, V, blk_out,
                      tok_out, O, lse, ws, (size_t)HSA_SPARSE_NOALLOC_SCRATCH_BYTES, stream);
}

hsa_sparse_status_t hsa_decode_step(const hsa_sparse_shape_t* shape, const int32_t* seq_lens, const uint16_t* qI,
                                    const uint16_t* kI, const int8_t* landmark_W, uint16_t* S, const uint16_t* Q,
                                    const uint16_t* K, const uint16_t* V, int32_t* blk_out, int32_t* tok_out,
                                    float* O, float* lse, void* workspace, size_t workspace_bytes,
                                    hsa_sparse_stream_t stream) {
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSummary | kSelect | kAttn);
  if (st != HSA_SPARSE_OK) return st;
  if (d.nq != 1 && d.b != 0) return fail(HSA_SPARSE_INVALID_ARG, "hsa_decode_step takes n_q == 1 (got %d)", d.nq);
  if (!seq_lens && d.b != 0) return fail(HSA_SPARSE_INVALID_ARG, "seq_lens is NULL");
  d.lens = seq_lens;
  return forward_impl(d, "hsa_decode_step", qI, kI, landmark_W, 0, S, Q, K, V, blk_out, tok_out, O, lse, workspace,
                      workspace_bytes, stream);
}

hsa_sparse_status_t hsa_super_summary(const hsa_sparse_shape_t* shape, int32_t group, const uint16_t* S,
                                      int32_t start_super, uint16_t* S2, hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSummary);
  if (st != HSA_SPARSE_OK) return st;
  int lgG = 0;
  st = check_level3(group, 2, lgG);
  if (st != HSA_SPARSE_OK) return st;
  if (start_super < 0) return fail(HSA_SPARSE_INVALID_ARG, "start_super < 0");
  const int nsb = (d.nb + group - 1) / group;
  if (d.b == 0 || d.L == 0 || start_super >= nsb) return HSA_SPARSE_OK;
  if (!S || !S2) return fail(HSA_SPARSE_INVALID_ARG, "S or S2 is NULL");
  hipError_t e = hsa::launch_super_summary(d, lgG, S, start_super, S2, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_super_summary");
}

hsa_sparse_status_t hsa_block_topm_3level(const hsa_sparse_shape_t* shape, int32_t group, int32_t top_m2,
                                          const uint16_t* qI, const uint16_t* S, const uint16_t* S2, int32_t* sup,
                                          int32_t* blk, void* workspace, size_t workspace_bytes,
                                          hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSelect | kSummary);
  if (st != HSA_SPARSE_OK) return st;
  int lgG = 0;
  st = check_level3(group, top_m2, lgG);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!qI || !S || !S2 || !sup || !blk) return fail(HSA_SPARSE_INVALID_ARG, "qI, S, S2, sup or blk is NULL");
  const size_t need = hsa::block_topm_3level_ws_bytes(d, lgG);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "block_topm_3level needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_block_topm_3level(d, lgG, top_m2, qI, S, S2, sup, blk, workspace, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_block_topm_3level");
}

hsa_sparse_status_t hsa_forward_3level(const hsa_sparse_shape_t* shape, const int32_t* seq_lens, int32_t group,
                                       int32_t top_m2, const uint16_t* qI, const uint16_t* kI, const int8_t* landmark_W,
                                       int32_t summary_start_block, uint16_t* S, uint16_t* S2, const uint16_t* Q,
                                       const uint16_t* K, const uint16_t* V, int32_t* sup_out, int32_t* blk_out,
                                       int32_t* tok_out, float* O, float* lse, void* workspace,
                                       size_t workspace_bytes, hsa_sparse_stream_t stream) {
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kSummary | kSelect | kAttn);
  if (st != HSA_SPARSE_OK) return st;
  Level3 l3{0, top_m2, S2, sup_out};
  st = check_level3(group, top_m2, l3.lgG);
  if (st != HSA_SPARSE_OK) return st;
  if (summary_start_block < 0) return fail(HSA_SPARSE_INVALID_ARG, "summary_start_block < 0");
  if (seq_lens && d.nq != 1 && d.b != 0)
    return fail(HSA_SPARSE_INVALID_ARG, "seq_lens needs n_q == 1 (got %d)", d.nq);
  d.lens = seq_lens;
  return forward_impl(d, "hsa_forward_3level", qI, kI, landmark_W, summary_start_block, S, Q, K, V, blk_out,
                      tok_out, O, lse, workspace, workspace_bytes, stream, &l3);
}

hsa_sparse_status_t hsa_head_landmarks(const hsa_sparse_shape_t* shape, const uint16_t* K,
                                       const int8_t* landmark_W, int32_t start_block, uint16_t* LK,
                                       hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kHeads);
  if (st != HSA_SPARSE_OK) return st;
  if (start_block < 0) return fail(HSA_SPARSE_INVALID_ARG, "start_block < 0");
  if (d.nL > 1 && !landmark_W) return fail(HSA_SPARSE_INVALID_ARG, "n_landmarks > 1 needs landmark_W");
  if (d.b == 0 || d.L == 0 || start_block >= d.nb) return HSA_SPARSE_OK;
  if (!K || !LK) return fail(HSA_SPARSE_INVALID_ARG, "K or LK is NULL");
  hipError_t e = hsa::launch_head_landmarks(d, K, landmark_W, start_block, LK, stream);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_head_landmarks");
}

hsa_sparse_status_t hsa_head_topm(const hsa_sparse_shape_t* shape, const uint16_t* Q, const uint16_t* LK,
                                  int32_t* blk, void* workspace, size_t workspace_bytes,
                                  hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kHeads | kHeadSel);
  if (st != HSA_SPARSE_OK) return st;
  if (empty(d)) return HSA_SPARSE_OK;
  if (!Q || !LK || !blk) return fail(HSA_SPARSE_INVALID_ARG, "Q, LK or blk is NULL");
  const size_t need = hsa::head_scores_ws_bytes(d);
  if (workspace_bytes < need || (need && !workspace))
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "head_topm needs %zu workspace bytes", need);
  hipError_t e = hsa::launch_head_topm(d, Q, LK, blk, workspace, stream, nullptr);
  return e == hipSuccess ? HSA_SPARSE_OK : hip_fail(e, "hsa_head_topm");
}

hsa_sparse_status_t hsa_forward_heads(const hsa_sparse_shape_t* shape, const int32_t* seq_lens,
                                      const int8_t* landmark_W, int32_t summary_start_block, const uint16_t* Q,
                                      const uint16_t* K, const uint16_t* V, uint16_t* LK, int32_t* blk_out,
                                      float* O, float* lse, void* workspace, size_t workspace_bytes,
                                      hsa_sparse_stream_t stream) {
  CallScope calls;
  hsa::Dims d;
  hsa_sparse_status_t st = check_shape(shape, d, kHeads | kHeadSel | kAttn);
  if (st != HSA_SPARSE_OK) return st;
  if (summary_start_block < 0) return fail(HSA_SPARSE_INVALID_ARG, "summary_start_block < 0");
  if (seq_lens && d.nq != 1 && d.b != 0)
    return fail(HSA_SPARSE_INVALID_ARG, "seq_lens needs n_q == 1 (got %d)", d.nq);
  d.lens = seq_lens;
  if (d.nL > 1 && !landmark_W) return fail(HSA_SPARSE_INVALID_ARG, "n_landmarks > 1 needs landmark_W");
  if (empty(d)) return HSA_SPARSE_OK;
  if (!Q || !K || !V || !LK || !O) return fail(HSA_SPARSE_INVALID_ARG, "Q, K, V, LK or O is NULL");
  const ForwardLayout f = heads_layout(d);
  if (workspace_bytes < f.total || !workspace)
    return fail(HSA_SPARSE_WORKSPACE_TOO_SMALL, "hsa_forward_heads needs %zu workspace bytes", f.total);
  char* ws = static_cast<char*>(workspace);
  int32_t* blk = blk_out ? blk_out : reinterpret_cast<int32_t*>(ws + f.blk_off);
  int32_t* tok = reinterpret_cast<int32_t*>(ws + f.tok_off);
  void* stage = ws + f.stage_off;
  const bool rec = g_record_stages;
  auto hf = [&](hipError_t err, const char* step) {
    return fail(HSA_SPARSE_HIP_ERROR, "hsa_forward_heads (%s): %s", step, hipGetErrorString(err));
  };
#define HSA_MARK(i)                                                        \
  if (rec && g_stage_events[i]) {                                          \
    hipError_t er = hipEventRecord((hipEvent_t)g_stage_events[i], stream); \
    if (er != hipSuccess) return hf(er, "stage event");                    \
  }
  HSA_MARK(0)
  // decode: the only rebuilt chunk is every query's own, always-kept chunk,
  // so its landmarks are folded into the score launch
  const bool fold = hsa::head_topm_can_fold(d, summary_start_block);
  hipError_t e = hipSuccess;
  if (!fold) e = hsa::launch_head_landmarks(d, K, landmark_W, summary_start_block, LK, stream);
  if (e != hipSuccess) return hf(e, "landmarks");
  HSA_MARK(1)
  const hsa::HeadFold hfold{K, landmark_W, LK, summary_start_block};
  e = hsa::launch_head_topm(d, Q, LK, blk, stage, stream, tok, fold ? &hfold : nullptr);
  if (e != hipSuccess) return hf(e, "chunk top-m");
  HSA_MARK(2)
  HSA_MARK(3)
  e = hsa::launch_head_attn(d, Q, K, V, tok, O, lse, stage, stream);
  if (e != hipSuccess) return hf(e, "attention");
  HSA_MARK(4)
#undef HSA_MARK
  return HSA_SPARSE_OK;
}

}  // extern "C"
