// Internal kernel-argument structs and launchers of the MLA decode library.
#pragma once

#include "mla_common.h"

namespace mla {

struct DecodeArgs {
  const void* q;           // [B][n_q][H][D] act dtype
  const void* cache;       // [nblk][bs][D]
  const float* scales;     // [nblk][bs][ntiles] (fp8) or null
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* ws_o;              // [slots][n_q][H][d_latent] act dtype (normalised partials)
  float* ws_lse;           // [slots][n_q][H]
  int32_t* ws_tab;         // [B][2]: first slot, piece count (written by the plan)
  int batch, n_q, H, D, d_latent, block_size, max_blocks, G;
  int cache_dtype, act_dtype;
  float scale;
};

struct CombineArgs {
  const void* ws_o;        // act dtype
  const float* ws_lse;
  const int32_t* ws_tab;   // [B][2] as recorded by the decode
  const int32_t* seq_lens;
  void* u;                 // [B][n_q][H][d_latent] act dtype
  float* lse_out;          // [B][n_q][H] or null
  int batch, n_q, H, d_latent, block_size, G;
  int act_dtype;
};

// combine + out_proj in one pass (d_latent = 512, bf16)
struct CombineProjArgs {
  const void* ws_o;        // bf16 partials
  const float* ws_lse;
  const int32_t* ws_tab;   // [B][2] as recorded by the decode
  const int32_t* seq_lens;
  const void* w_uv;        // [H][d_v][d_latent]
  void* out;               // [B * n_q][H][d_v]
  void* u;                 // [B][n_q][H][d_latent] or null
  float* lse_out;          // [B][n_q][H] or null
  int batch, n_q, H, d_latent, d_v, block_size, G;
};

struct AppendArgs {
  const void* h;           // [T][d_model]
  const void* w_dkv;       // [d_latent][d_model]
  const void* w_kr;        // [d_rope][d_model]
  const int32_t* seq_ids;
  const int32_t* positions;
  const int32_t* page_table;
  void* cache;
  float* scales;
  int n_tokens, d_model, d_latent, d_rope, D, block_size, max_blocks;
  int cache_dtype, act_dtype;
  float rope_base;
};

struct QueryArgs {
  const void* q_in;        // [rows][H][d_nope + d_rope]
  const int32_t* positions;
  const void* w_uk;        // [H][d_nope][d_latent]
  void* q_out;             // [rows][H][d_latent + d_rope]
  int rows, H, d_nope, d_rope, d_latent;
  int act_dtype;
  float rope_base;
};

bool query_absorb_mfma_supported(const QueryArgs& a);
hipError_t launch_query_absorb_mfma(const QueryArgs& a, hipStream_t st);
hipError_t launch_query_absorb_generic(const QueryArgs& a, hipStream_t st);

// Raises kernel fn's dynamic LDS limit to `bytes` on the current device, once
// per (kernel, device); safe to call from several host threads.
hipError_t ensure_dynamic_lds(const void* fn, int bytes);

// Device-data precondition checks (see mla_abi's validation mode): items are
// sequences (seq_lens given) or tokens (positions given).
struct ValidateArgs {
  const int32_t* seq_lens;    // or null
  const int32_t* positions;   // or null
  const int32_t* seq_ids;     // with positions and page_table
  const int32_t* page_table;  // or null: no entry checks
  int n_items, n_q, max_blocks, block_size;
};
// Runs the checks on `st` and waits for them; out = {kind (0: none), item, value}.
hipError_t run_validate(const ValidateArgs& a, hipStream_t st, int out[3]);

// y = x W^T
struct LinearArgs {
  const void* x;           // [rows][k]
  const void* w;           // [n][k]
  void* y;                 // [rows][n]
  int rows, n, k;
  int act_dtype;
};

bool linear_mfma_supported(const LinearArgs& a);
size_t linear_mfma_workspace(const LinearArgs& a);
hipError_t launch_linear_mfma(const LinearArgs& a, void* ws, hipStream_t st);
hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t st);

struct OutProjArgs {
  const void* u;           // [rows][H][d_latent]
  const void* w;           // [H][d_v][d_latent]
  void* out;               // [rows][H][d_v]
  int rows, H, d_latent, d_v;
  int act_dtype;
};

// chunked prefill (un-absorbed form): gather and q rotation, the K^C / V
// expansion, then attention
struct PrefillArgs {
  const void* q;             // [C][H][d_nope + d_rope] bf16, q^R not yet rotated
  const void* cache;         // paged pool [nblk][bs][D]: bf16, or e4m3 codes
  const float* cache_scales; // [nblk][bs][5] fp32 for an e4m3 cache, else NULL
  int cache_dtype;
  const int32_t* page_table; // the sequence's row
  void* ws_c;                // [T][d_latent] gathered latents
  void* ws_kr;               // [T][d_rope] gathered RoPE keys
  void* ws_kc;               // [H][T][d_nope] expanded content keys (head-major)
  void* ws_v;                // [H][T][d_v] expanded values (head-major)
  const void* w_uk;          // [H][d_nope][d_latent] bf16 = [H * d_nope][d_latent]
  const void* w_uv;          // [H][d_v][d_latent] bf16 = [H * d_v][d_latent]
  void* ws_q;                // [C][H][d_nope + d_rope] the queries, q^R rotated
  void* out;                 // [C][H][d_v] bf16
  int n_tokens, seq_len, block_size, H, d_latent, d_rope, d_nope, d_v;
  float scale, rope_base;
};
bool prefill_supported(const PrefillArgs& a);
hipError_t launch_prefill_gather(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_expand(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t st);

bool decode_generic_supported(const DecodeArgs& a);
hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st);
bool decode_mfma_supported(const DecodeArgs& a);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
bool combine_out_proj_supported(const CombineProjArgs& a);
hipError_t launch_combine_out_proj(const CombineProjArgs& a, hipStream_t st);
bool append_supported(const AppendArgs& a);
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
bool append_mfma_supported(const AppendArgs& a);
size_t append_mfma_workspace(const AppendArgs& a);
hipError_t launch_append_mfma(const AppendArgs& a, void* ws, hipStream_t st);
int append_mfma_slices(const AppendArgs& a);  // k slices of the matrix-core partials
hipError_t launch_append_partial_mfma(const AppendArgs& a, void* ws, hipStream_t st);
// The matrix-core append's second step and the matrix-core query absorption in
// one launch (they are independent; sharing the GPU hides each one's latency).
hipError_t launch_append_finalize_query_mfma(const AppendArgs& ap, const void* ws, const QueryArgs& q,
                                             hipStream_t st);
hipError_t launch_out_proj_generic(const OutProjArgs& a, hipStream_t st);
bool out_proj_mfma_supported(const OutProjArgs& a);
hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st);

}  // namespace mla
