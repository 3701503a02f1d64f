// Host side of the C ABI: argument validation, error reporting, kernel choice.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <utility>

#include "mla_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MLA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_bytes(int dt) { return dt == MLA_FP32 ? 4 : dt == MLA_BF16 ? 2 : 1; }

// Checks shared by every call.  Returns MLA_OK or an error code.
int check_dims(const mla_dims* d, bool need_cache_dtype) {
  if (!d) return fail(MLA_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->num_heads < 1 || d->d_latent < 1 || d->d_rope < 0 || d->d_nope < 0 || d->d_v < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "bad dims: num_heads=%d d_latent=%d d_rope=%d d_nope=%d d_v=%d", d->num_heads,
                d->d_latent, d->d_rope, d->d_nope, d->d_v);
  if (d->d_rope % 2) return fail(MLA_ERR_INVALID_ARGUMENT, "d_rope=%d must be even", d->d_rope);
  if (d->block_size < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "block_size=%d", d->block_size);
  if (d->act_dtype != MLA_FP32 && d->act_dtype != MLA_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "act_dtype=%d must be MLA_FP32 or MLA_BF16", d->act_dtype);
  if (need_cache_dtype && (d->cache_dtype < MLA_FP32 || d->cache_dtype > MLA_FP8_E4M3_PO2))
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_dtype=%d", d->cache_dtype);
  if (d->softmax_scale <= 0.f && d->d_nope + d->d_rope <= 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "default softmax scale needs d_nope + d_rope > 0");
  return MLA_OK;
}

float eff_scale(const mla_dims* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale
                                : float(1.0 / std::sqrt(double(d->d_nope + d->d_rope)));
}

int default_partitions(int n_q) {
  int cu = mla_device_cu_count();
  if (cu <= 0) cu = 256;
  int g = cu / (n_q > 0 ? n_q : 1);
  return g < 1 ? 1 : g;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Decode workspace: partials o [slots][n_q][H][d_latent] (act dtype), their
// lse [slots][n_q][H] fp32, and per sequence (first slot, piece count)
// int32 [B][2], which mla_decode records for the combine.
struct WsLayout {
  size_t o_bytes, lse_off, tab_off, total;
};

WsLayout ws_layout(const mla_dims* d, int batch, int n_q, int G) {
  const size_t slots = mla::ws_slots(batch, G);
  WsLayout w;
  w.o_bytes = slots * size_t(n_q) * d->num_heads * d->d_latent * elem_bytes(d->act_dtype);
  w.lse_off = align_up(w.o_bytes, 256);
  w.tab_off = align_up(w.lse_off + slots * size_t(n_q) * d->num_heads * sizeof(float), 256);
  w.total = align_up(w.tab_off + size_t(batch) * 2 * sizeof(int32_t), 256);
  return w;
}

// Validation mode (MLA_FLAG_VALIDATE, or MLA_VALIDATE=1 in the environment).
bool validate_on(const mla_dims* d) {
  static const bool env = [] {
    const char* v = std::getenv("MLA_VALIDATE");
    return v && v[0] == '1';
  }();
  return env || (d->flags & MLA_FLAG_VALIDATE);
}

// Runs the device-data checks; MLA_OK, or the error for the first violation.
int validate(const mla::ValidateArgs& a, mla_stream_t stream) {
  int out[3] = {0, 0, 0};
  if (hipError_t e = mla::run_validate(a, static_cast<hipStream_t>(stream), out); e != hipSuccess)
    return hip_fail(e, "validation");
  switch (out[0]) {
    case 0: return MLA_OK;
    case 1: return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d outside [n_q, max_blocks_per_seq * block_size]",
                        out[1], out[2]);
    case 2: return fail(MLA_ERR_INVALID_ARGUMENT, "page-table entry %d read for %s %d is negative", out[2],
                        a.seq_lens ? "sequence" : "token", out[1]);
    case 3: return fail(MLA_ERR_INVALID_ARGUMENT, "positions[%d] = %d outside [0, max_blocks_per_seq * block_size)",
                        out[1], out[2]);
    default: return fail(MLA_ERR_INVALID_ARGUMENT, "seq_ids[%d] = %d is negative", out[1], out[2]);
  }
}

// Shared checks of mla_linear and its workspace query; fills a.
int linear_args(const mla_dims* d, const void* x, int32_t rows, int32_t k, const void* w, int32_t n,
                void* y, mla::LinearArgs* a) {
  if (int e = check_dims(d, false)) return e;
  if (rows < 0 || k < 1 || n < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "rows=%d k=%d n=%d", rows, k, n);
  a->x = x;
  a->w = w;
  a->y = y;
  a->rows = rows;
  a->n = n;
  a->k = k;
  a->act_dtype = d->act_dtype;
  return MLA_OK;
}
bool linear_use_mfma(const mla_dims* d, const mla::LinearArgs& a) {
  return !(d->flags & MLA_FLAG_GENERIC_DECODE) && a.rows > 0 && mla::linear_mfma_supported(a);
}


// ---------------------------------------------------------------------------
// Library-owned decode workspace for callers that cannot allocate
// (mla_decode_noalloc).  One copy per device, alive until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// is only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(MLA_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device (looked up on the
// first call per device, thread-safe).  MLA_OK or MLA_ERR_HIP.
int noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return MLA_OK;
}
}  // namespace

namespace mla {
hipError_t ensure_dynamic_lds(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}
}  // namespace mla

extern "C" {

int mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_last_error(void) { return g_err.c_str(); }

int mla_device_cu_count(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

namespace {
mla::AppendArgs append_args(const mla_dims* d, int32_t n_tokens, int32_t d_model) {
  mla::AppendArgs a{};
  a.n_tokens = n_tokens;
  a.d_model = d_model;
  a.d_latent = d->d_latent;
  a.d_rope = d->d_rope;
  a.D = d->d_latent + d->d_rope;
  a.block_size = d->block_size;
  a.cache_dtype = d->cache_dtype;
  a.act_dtype = d->act_dtype;
  a.rope_base = d->rope_base > 0.f ? d->rope_base : 10000.f;
  return a;
}
// The matrix-core append applies to bf16 activations with the RoPE part inside
// one 128-channel tile (pointer alignment is checked again at call time).
bool append_uses_mfma(const mla::AppendArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_model % 16 == 0 && a.D <= 1024 && a.D % 4 == 0 &&
         (a.d_rope == 0 || a.d_latent / 128 == (a.D - 1) / 128);
}
}  // namespace

size_t mla_cache_append_workspace_size(const mla_dims* d, int32_t n_tokens, int32_t d_model) {
  if (!d || n_tokens <= 0 || d_model < 1 || d->d_latent < 1 || d->d_rope < 0) return 0;
  const mla::AppendArgs a = append_args(d, n_tokens, d_model);
  return append_uses_mfma(a) ? mla::append_mfma_workspace(a) : 0;
}

namespace {

// Argument checks of the cache append.  On success *a holds the call
// (a->n_tokens == 0: nothing to do) and *mfma says which form runs.
int append_prepare(const mla_dims* d, const void* h, int32_t n_tokens, int32_t d_model, const void* w_dkv,
                   const void* w_kr, const int32_t* seq_ids, const int32_t* positions,
                   const int32_t* page_table, int32_t max_blocks_per_seq, void* cache, float* cache_scales,
                   void* workspace, size_t workspace_bytes, mla_stream_t stream, mla::AppendArgs* a,
                   bool* mfma) {
  if (int e = check_dims(d, true)) return e;
  if (n_tokens < 0 || d_model < 1 || max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_ARGUMENT, "n_tokens=%d d_model=%d max_blocks_per_seq=%d", n_tokens,
                d_model, max_blocks_per_seq);
  *a = append_args(d, n_tokens, d_model);
  *mfma = false;
  if (n_tokens == 0) return MLA_OK;
  if (!h || !w_dkv || !seq_ids || !positions || !page_table || !cache || (d->d_rope > 0 && !w_kr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (mla::is_fp8_cache(d->cache_dtype) != (cache_scales != nullptr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_scales must be given exactly for the fp8 cache");
  const size_t ae = elem_bytes(d->act_dtype), ce = elem_bytes(d->cache_dtype);
  if (!aligned(h, ae) || !aligned(w_dkv, ae) || (w_kr && !aligned(w_kr, ae)) || !aligned(cache, ce) ||
      !aligned(seq_ids, 4) || !aligned(positions, 4) || !aligned(page_table, 4) ||
      (cache_scales && !aligned(cache_scales, 4)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  a->h = h;
  a->w_dkv = w_dkv;
  a->w_kr = w_kr;
  a->seq_ids = seq_ids;
  a->positions = positions;
  a->page_table = page_table;
  a->cache = cache;
  a->scales = cache_scales;
  a->max_blocks = max_blocks_per_seq;
  if (append_uses_mfma(*a)) {
    if (!mla::append_mfma_supported(*a))
      return fail(MLA_ERR_INVALID_ARGUMENT, "append: bf16 h / weights must be 16-byte aligned");
    const size_t need = mla::append_mfma_workspace(*a);
    if (workspace_bytes < need || (need && !workspace))
      return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "append workspace %zu bytes < %zu required",
                  workspace_bytes, need);
    if (!aligned(workspace, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned workspace");
    *mfma = true;
  } else if (!mla::append_supported(*a)) {
    return fail(MLA_ERR_UNSUPPORTED, "append: the RoPE part must lie in one 128-channel tile");
  }
  if (validate_on(d))
    if (int r = validate({nullptr, positions, seq_ids, page_table, n_tokens, 1, max_blocks_per_seq,
                          d->block_size}, stream))
      return r;
  return MLA_OK;
}

// Argument checks of the query absorption; as above (a->rows == 0: nothing to do).
int query_prepare(const mla_dims* d, const void* q_in, const int32_t* positions, const void* w_uk, void* q_out,
                  int32_t rows, mla_stream_t stream, mla::QueryArgs* a, bool* mfma) {
  if (int e = check_dims(d, false)) return e;
  if (d->d_nope < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "query absorption needs d_nope >= 1");
  if (rows < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "rows=%d", rows);
  a->rows = 0;
  *mfma = false;
  if (rows == 0) return MLA_OK;
  if (!q_in || !positions || !w_uk || !q_out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t ae = elem_bytes(d->act_dtype);
  if (!aligned(q_in, ae) || !aligned(w_uk, ae) || !aligned(q_out, ae) || !aligned(positions, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const size_t in_bytes = size_t(rows) * d->num_heads * (d->d_nope + d->d_rope) * ae;
  const size_t out_bytes = size_t(rows) * d->num_heads * (d->d_latent + d->d_rope) * ae;
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(q_in), o0 = reinterpret_cast<uintptr_t>(q_out);
  if (i0 < o0 + out_bytes && o0 < i0 + in_bytes)
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_out overlaps q_in");
  a->q_in = q_in;
  a->positions = positions;
  a->w_uk = w_uk;
  a->q_out = q_out;
  a->rows = rows;
  a->H = d->num_heads;
  a->d_nope = d->d_nope;
  a->d_rope = d->d_rope;
  a->d_latent = d->d_latent;
  a->act_dtype = d->act_dtype;
  a->rope_base = d->rope_base > 0.f ? d->rope_base : 10000.f;
  *mfma = !(d->flags & MLA_FLAG_GENERIC_DECODE) && mla::query_absorb_mfma_supported(*a);
  if (validate_on(d))  // positions >= 0
    if (int r = validate({nullptr, positions, nullptr, nullptr, rows, 1, 1, d->block_size}, stream)) return r;
  return MLA_OK;
}

int append_launch(const mla::AppendArgs& a, bool mfma, void* workspace, mla_stream_t stream) {
  const hipError_t e = mfma ? mla::launch_append_mfma(a, workspace, static_cast<hipStream_t>(stream))
                            : mla::launch_append(a, static_cast<hipStream_t>(stream));
  return e != hipSuccess ? hip_fail(e, "append launch") : MLA_OK;
}

int query_launch(const mla::QueryArgs& a, bool mfma, mla_stream_t stream) {
  const hipError_t e = mfma ? mla::launch_query_absorb_mfma(a, static_cast<hipStream_t>(stream))
                            : mla::launch_query_absorb_generic(a, static_cast<hipStream_t>(stream));
  return e != hipSuccess ? hip_fail(e, "query_absorb launch") : MLA_OK;
}

}  // namespace

int mla_cache_append(const mla_dims* d, const void* h, int32_t n_tokens, int32_t d_model,
                     const void* w_dkv, const void* w_kr, const int32_t* seq_ids,
                     const int32_t* positions, const int32_t* page_table,
                     int32_t max_blocks_per_seq, void* cache, float* cache_scales,
                     void* workspace, size_t workspace_bytes, mla_stream_t stream) {
  mla::AppendArgs a;
  bool mfma;
  if (int e = append_prepare(d, h, n_tokens, d_model, w_dkv, w_kr, seq_ids, positions, page_table,
                             max_blocks_per_seq, cache, cache_scales, workspace, workspace_bytes, stream, &a,
                             &mfma))
    return e;
  if (a.n_tokens > 0)
    if (int e = append_launch(a, mfma, workspace, stream)) return e;
  return ok();
}

int mla_cache_append_query_absorb(const mla_dims* d, const void* h, int32_t n_tokens, int32_t d_model,
                                  const void* w_dkv, const void* w_kr, const int32_t* seq_ids,
                                  const int32_t* positions, const int32_t* page_table,
                                  int32_t max_blocks_per_seq, void* cache, float* cache_scales,
                                  void* workspace, size_t workspace_bytes, const void* q_in,
                                  const int32_t* q_positions, const void* w_uk, void* q_out, int32_t q_rows,
                                  mla_stream_t stream) {
  mla::AppendArgs ap;
  mla::QueryArgs q;
  bool ap_mfma, q_mfma;
  if (int e = append_prepare(d, h, n_tokens, d_model, w_dkv, w_kr, seq_ids, positions, page_table,
                             max_blocks_per_seq, cache, cache_scales, workspace, workspace_bytes, stream, &ap,
                             &ap_mfma))
    return e;
  if (int e = query_prepare(d, q_in, q_positions, w_uk, q_out, q_rows, stream, &q, &q_mfma)) return e;
  if (ap.n_tokens > 0 && q.rows > 0 && ap_mfma && q_mfma) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = mla::launch_append_partial_mfma(ap, workspace, st);
    if (e == hipSuccess) e = mla::launch_append_finalize_query_mfma(ap, workspace, q, st);
    if (e != hipSuccess) return hip_fail(e, "append + query_absorb launch");
    return ok();
  }
  if (ap.n_tokens > 0)
    if (int e = append_launch(ap, ap_mfma, workspace, stream)) return e;
  if (q.rows > 0)
    if (int e = query_launch(q, q_mfma, stream)) return e;
  return ok();
}

size_t mla_decode_workspace_size(const mla_dims* d, int32_t batch, int32_t n_q,
                                 int32_t num_partitions) {
  if (!d || batch < 0 || n_q < 1 || d->num_heads < 1 || d->d_latent < 1 ||
      num_partitions > MLA_MAX_PARTITIONS)
    return 0;
  const int G = num_partitions > 0 ? num_partitions : default_partitions(n_q);
  return ws_layout(d, batch, n_q, G).total;
}

int mla_decode(const mla_dims* d, const void* q, int32_t batch, int32_t n_q, const void* cache,
               const float* cache_scales, const int32_t* page_table, int32_t max_blocks_per_seq,
               const int32_t* seq_lens, int32_t num_partitions, void* workspace,
               size_t workspace_bytes, mla_stream_t stream) {
  if (int e = check_dims(d, true)) return e;
  if (batch < 0 || n_q < 1 || max_blocks_per_seq < 1 || num_partitions > MLA_MAX_PARTITIONS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d n_q=%d max_blocks_per_seq=%d num_partitions=%d",
                batch, n_q, max_blocks_per_seq, num_partitions);
  if (batch == 0) return ok();
  if (!q || !cache || !page_table || !seq_lens || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (mla::is_fp8_cache(d->cache_dtype) != (cache_scales != nullptr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_scales must be given exactly for the fp8 cache");
  const size_t ae = elem_bytes(d->act_dtype), ce = elem_bytes(d->cache_dtype);
  if (!aligned(q, ae) || !aligned(cache, ce) || !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(workspace, 256))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer (workspace needs 256-byte alignment)");
  const int G = num_partitions > 0 ? num_partitions : default_partitions(n_q);
  const WsLayout w = ws_layout(d, batch, n_q, G);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes,
                w.total);
  mla::DecodeArgs a;
  a.q = q;
  a.cache = cache;
  a.scales = cache_scales;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.ws_o = workspace;
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.lse_off);
  a.ws_tab = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w.tab_off);
  a.batch = batch;
  a.n_q = n_q;
  a.H = d->num_heads;
  a.D = d->d_latent + d->d_rope;
  a.d_latent = d->d_latent;
  a.block_size = d->block_size;
  a.max_blocks = max_blocks_per_seq;
  a.G = G;
  a.cache_dtype = d->cache_dtype;
  a.act_dtype = d->act_dtype;
  a.scale = eff_scale(d);
  if (validate_on(d))
    if (int r = validate({seq_lens, nullptr, nullptr, page_table, batch, n_q, max_blocks_per_seq, d->block_size},
                         stream))
      return r;
  hipError_t e;
  if (!(d->flags & MLA_FLAG_GENERIC_DECODE) && mla::decode_mfma_supported(a)) {
    e = mla::launch_decode_mfma(a, static_cast<hipStream_t>(stream));
  } else {
    if (!mla::decode_generic_supported(a))
      return fail(MLA_ERR_UNSUPPORTED, "decode: d_latent + d_rope = %d exceeds 1024", a.D);
    e = mla::launch_decode_generic(a, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int mla_decode_combine(const mla_dims* d, const void* workspace, size_t workspace_bytes,
                       int32_t batch, int32_t n_q, const int32_t* seq_lens, int32_t num_partitions,
                       void* u_out, float* lse_out, mla_stream_t stream) {
  if (int e = check_dims(d, false)) return e;
  if (batch < 0 || n_q < 1 || num_partitions > MLA_MAX_PARTITIONS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d n_q=%d num_partitions=%d", batch, n_q,
                num_partitions);
  if (batch == 0) return ok();
  if (!workspace || !seq_lens || !u_out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(workspace, 256) || !aligned(u_out, elem_bytes(d->act_dtype)) || !aligned(seq_lens, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const int G = num_partitions > 0 ? num_partitions : default_partitions(n_q);
  const WsLayout w = ws_layout(d, batch, n_q, G);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes,
                w.total);
  mla::CombineArgs a;
  a.ws_o = workspace;
  a.ws_lse = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + w.lse_off);
  a.ws_tab = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) + w.tab_off);
  a.seq_lens = seq_lens;
  a.u = u_out;
  a.lse_out = lse_out;
  a.batch = batch;
  a.n_q = n_q;
  a.H = d->num_heads;
  a.d_latent = d->d_latent;
  a.block_size = d->block_size;
  a.G = G;
  a.act_dtype = d->act_dtype;
  if (validate_on(d))  // lengths only (no page table; no upper bound known here)
    if (int r = validate({seq_lens, nullptr, nullptr, nullptr, batch, n_q, INT32_MAX / d->block_size, d->block_size},
                         stream))
      return r;
  hipError_t e = mla::launch_combine(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

int mla_query_absorb(const mla_dims* d, const void* q_in, const int32_t* positions, const void* w_uk,
                     void* q_out, int32_t rows, mla_stream_t stream) {
  mla::QueryArgs a;
  bool mfma;
  if (int e = query_prepare(d, q_in, positions, w_uk, q_out, rows, stream, &a, &mfma)) return e;
  if (a.rows > 0)
    if (int e = query_launch(a, mfma, stream)) return e;
  return ok();
}

size_t mla_linear_workspace_size(const mla_dims* d, int32_t rows, int32_t n, int32_t k) {
  mla::LinearArgs a;
  // The kernel choice also depends on the pointers' alignment, unknown here:
  // the size is that of the matrix-core form whenever dtype and shapes allow it
  // (16-byte aligned stand-in pointers).
  if (linear_args(d, reinterpret_cast<const void*>(uintptr_t(256)), rows, k,
                  reinterpret_cast<const void*>(uintptr_t(256)), n, reinterpret_cast<void*>(uintptr_t(256)), &a))
    return 0;
  return linear_use_mfma(d, a) ? mla::linear_mfma_workspace(a) : 0;
}

int mla_linear(const mla_dims* d, const void* x, int32_t rows, int32_t k, const void* w, int32_t n, void* y,
               void* workspace, size_t workspace_bytes, mla_stream_t stream) {
  mla::LinearArgs a;
  if (int e = linear_args(d, x, rows, k, w, n, y, &a)) return e;
  if (rows == 0) return ok();
  if (!x || !w || !y) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t ae = elem_bytes(d->act_dtype);
  if (!aligned(x, ae) || !aligned(w, ae) || !aligned(y, ae) || (workspace && !aligned(workspace, 16)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), w0 = reinterpret_cast<uintptr_t>(w),
                  y0 = reinterpret_cast<uintptr_t>(y);
  const size_t xb = size_t(rows) * k * ae, wbytes = size_t(n) * k * ae, yb = size_t(rows) * n * ae;
  if ((y0 < x0 + xb && x0 < y0 + yb) || (y0 < w0 + wbytes && w0 < y0 + yb))
    return fail(MLA_ERR_INVALID_ARGUMENT, "y overlaps x or w");
  hipError_t e;
  if (linear_use_mfma(d, a)) {
    const size_t need = mla::linear_mfma_workspace(a);
    if (workspace_bytes < need || (need && !workspace))
      return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    e = mla::launch_linear_mfma(a, workspace, static_cast<hipStream_t>(stream));
  } else {
    e = mla::launch_linear_generic(a, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return hip_fail(e, "linear launch");
  return ok();
}

int mla_out_proj(const mla_dims* d, const void* u, int32_t rows, const void* w_uv, void* out,
                 mla_stream_t stream) {
  if (int e = check_dims(d, false)) return e;
  if (rows < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "rows=%d", rows);
  if (rows == 0) return ok();
  if (!u || !w_uv || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t ae = elem_bytes(d->act_dtype);
  if (!aligned(u, ae) || !aligned(w_uv, ae) || !aligned(out, ae))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  mla::OutProjArgs a;
  a.u = u;
  a.w = w_uv;
  a.out = out;
  a.rows = rows;
  a.H = d->num_heads;
  a.d_latent = d->d_latent;
  a.d_v = d->d_v;
  a.act_dtype = d->act_dtype;
  hipError_t e = mla::out_proj_mfma_supported(a) ? mla::launch_out_proj_mfma(a, static_cast<hipStream_t>(stream))
                                                 : mla::launch_out_proj_generic(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "out_proj launch");
  return ok();
}

int mla_decode_combine_out_proj(const mla_dims* d, const void* workspace, size_t workspace_bytes,
                                int32_t batch, int32_t n_q, const int32_t* seq_lens,
                                int32_t num_partitions, const void* w_uv, void* out, void* u_out,
                                float* lse_out, mla_stream_t stream) {
  if (int e = check_dims(d, false)) return e;
  if (batch < 0 || n_q < 1 || num_partitions > MLA_MAX_PARTITIONS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d n_q=%d num_partitions=%d", batch, n_q,
                num_partitions);
  if (batch == 0) return ok();
  if (!workspace || !seq_lens || !w_uv || !out)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  const size_t ae = elem_bytes(d->act_dtype);
  if (!aligned(workspace, 256) || !aligned(seq_lens, 4) || !aligned(w_uv, ae) || !aligned(out, ae) ||
      (u_out && !aligned(u_out, ae)) || (lse_out && !aligned(lse_out, 4)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const int G = num_partitions > 0 ? num_partitions : default_partitions(n_q);
  const WsLayout w = ws_layout(d, batch, n_q, G);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes,
                w.total);
  mla::CombineProjArgs a;
  a.ws_o = workspace;
  a.ws_lse = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + w.lse_off);
  a.ws_tab = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) + w.tab_off);
  a.seq_lens = seq_lens;
  a.w_uv = w_uv;
  a.out = out;
  a.u = u_out;
  a.lse_out = lse_out;
  a.batch = batch;
  a.n_q = n_q;
  a.H = d->num_heads;
  a.d_latent = d->d_latent;
  a.d_v = d->d_v;
  a.block_size = d->block_size;
  a.G = G;
  if (validate_on(d))  // lengths only, as mla_decode_combine
    if (int r = validate({seq_lens, nullptr, nullptr, nullptr, batch, n_q, INT32_MAX / d->block_size, d->block_size},
                         stream))
      return r;
  hipError_t e;
  if (d->act_dtype == MLA_BF16 && mla::combine_out_proj_supported(a)) {
    e = mla::launch_combine_out_proj(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "combine_out_proj launch");
    return ok();
  }
  if (!u_out)
    return fail(MLA_ERR_UNSUPPORTED,
                "combine_out_proj: no fused kernel for these dims; pass u_out to run the two passes");
  if (int r = mla_decode_combine(d, workspace, workspace_bytes, batch, n_q, seq_lens,
                                 num_partitions, u_out, lse_out, stream))
    return r;
  return mla_out_proj(d, u_out, batch * n_q, w_uv, out, stream);
}

namespace {
// Prefill workspace: gathered latents c [T][d_c] and RoPE keys [T][d_R], the
// expanded content keys and values [T][H * d_nope], [T][H * d_v] (act dtype),
// then the expansion's linear-layer scratch.
struct PrefillLayout {
  size_t kr_off, kc_off, v_off, q_off, total;
};
PrefillLayout prefill_layout(const mla_dims* d, int n_tokens, int seq_len) {
  PrefillLayout w;
  const size_t T = size_t(seq_len), e = 2;
  w.kr_off = align_up(T * d->d_latent * e, 256);
  w.kc_off = align_up(w.kr_off + T * d->d_rope * e, 256);
  w.v_off = align_up(w.kc_off + T * size_t(d->num_heads) * d->d_nope * e, 256);
  w.q_off = align_up(w.v_off + T * size_t(d->num_heads) * d->d_v * e, 256);
  w.total = align_up(w.q_off + size_t(n_tokens) * d->num_heads * (d->d_nope + d->d_rope) * e, 256);
  return w;
}
bool prefill_dims_ok(const mla_dims* d) {
  return d->act_dtype == MLA_BF16 && (d->cache_dtype == MLA_BF16 || mla::is_fp8_cache(d->cache_dtype)) &&
         d->num_heads == 128 && d->d_latent == 512 &&
         d->d_rope == 64 && d->d_nope == 128 && d->d_v == 128;
}
}  // namespace

size_t mla_prefill_workspace_size(const mla_dims* d, int32_t n_tokens, int32_t seq_len) {
  if (!d || n_tokens < 1 || seq_len < n_tokens || !prefill_dims_ok(d)) return 0;
  return prefill_layout(d, n_tokens, seq_len).total;
}

int mla_prefill(const mla_dims* d, const void* q_in, int32_t n_tokens, const void* cache,
                const float* cache_scales, const int32_t* page_table_row, int32_t seq_len, const void* w_uk,
                const void* w_uv, void* out, void* workspace, size_t workspace_bytes, mla_stream_t stream) {
  if (int e = check_dims(d, true)) return e;
  if (n_tokens < 0 || seq_len < n_tokens)
    return fail(MLA_ERR_INVALID_ARGUMENT, "n_tokens=%d seq_len=%d (need 0 <= n_tokens <= seq_len)", n_tokens,
                seq_len);
  if (n_tokens == 0) return ok();
  if (!prefill_dims_ok(d))
    return fail(MLA_ERR_UNSUPPORTED, "prefill: bf16 activations, a bf16 or e4m3 cache, H=128, d_latent=512, "
                                     "d_rope=64, d_nope=128, d_v=128 only");
  if (seq_len >= MLA_MAX_PREFILL_TOKENS)  // one head's expanded keys must stay under 2 GiB (32-bit offsets)
    return fail(MLA_ERR_INVALID_ARGUMENT, "seq_len=%d (prefill takes fewer than %d cached tokens)", seq_len,
                MLA_MAX_PREFILL_TOKENS);
  if (mla::is_fp8_cache(d->cache_dtype) != (cache_scales != nullptr))
    return fail(MLA_ERR_INVALID_ARGUMENT, "cache_scales must be given exactly for an e4m3 cache");
  if (cache_scales && !aligned(cache_scales, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned cache_scales");
  if (!q_in || !cache || !page_table_row || !w_uk || !w_uv || !out || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned(q_in, 16) || !aligned(cache, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16) || !aligned(out, 8) ||
      !aligned(page_table_row, 4) || !aligned(workspace, 256))
    return fail(MLA_ERR_INVALID_ARGUMENT, "misaligned pointer (q, cache, weights 16 B; out 8 B; workspace 256 B)");
  const PrefillLayout w = prefill_layout(d, n_tokens, seq_len);
  if (workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "prefill workspace %zu bytes < %zu required", workspace_bytes, w.total);
  char* ws = static_cast<char*>(workspace);
  mla::PrefillArgs a;
  a.q = q_in;
  a.cache = cache;
  a.cache_scales = cache_scales;
  a.cache_dtype = d->cache_dtype;
  a.page_table = page_table_row;
  a.ws_c = ws;
  a.ws_kr = ws + w.kr_off;
  a.ws_kc = ws + w.kc_off;
  a.ws_v = ws + w.v_off;
  a.ws_q = ws + w.q_off;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.n_tokens = n_tokens;
  a.seq_len = seq_len;
  a.block_size = d->block_size;
  a.H = d->num_heads;
  a.d_latent = d->d_latent;
  a.d_rope = d->d_rope;
  a.d_nope = d->d_nope;
  a.d_v = d->d_v;
  a.scale = eff_scale(d);
  a.rope_base = d->rope_base > 0.f ? d->rope_base : 10000.f;
  if (!mla::prefill_supported(a)) return fail(MLA_ERR_INVALID_ARGUMENT, "prefill: misaligned pointer");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // gather + q rotation, the expansion K^C = c W^UK^T and V = c W^UV^T
  // (W^UK, W^UV: [H][128][d_c] = [H*128][d_c]), then attention
  hipError_t e = mla::launch_prefill_gather(a, st);
  if (e == hipSuccess) e = mla::launch_prefill_expand(a, st);
  if (e == hipSuccess) e = mla::launch_prefill_attn(a, st);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

int mla_decode_noalloc(const mla_dims* d, const void* q, int32_t batch, int32_t n_q, const void* cache,
                       const float* cache_scales, const int32_t* page_table, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t num_partitions, void* u_out, float* lse_out,
                       mla_stream_t stream) {
  if (int e = check_dims(d, true)) return e;
  if (batch < 0 || n_q < 1 || num_partitions > MLA_MAX_PARTITIONS)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch=%d n_q=%d num_partitions=%d", batch, n_q, num_partitions);
  if (batch == 0) return ok();
  const size_t need = mla_decode_workspace_size(d, batch, n_q, num_partitions);
  if (need > kNoAllocScratchBytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "mla_decode_noalloc: this call needs %zu bytes of decode workspace, the library's static "
                "scratch holds %zu (use fewer sequences, query tokens or partitions, or mla_decode with a "
                "caller workspace)", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (int e = noalloc_scratch(&ws)) return e;
  if (int e = mla_decode(d, q, batch, n_q, cache, cache_scales, page_table, max_blocks_per_seq, seq_lens,
                         num_partitions, ws, kNoAllocScratchBytes, stream))
    return e;
  return mla_decode_combine(d, ws, kNoAllocScratchBytes, batch, n_q, seq_lens, num_partitions, u_out,
                            lse_out, stream);
}

}  // extern "C"
