// C ABI of libpa (declared in include/pa.h): argument validation and dispatch.
//
// Every check here looks only at host-visible arguments and runs before any
// work is enqueued; the kernels are launched on the caller's stream and the
// library never allocates, frees or synchronises.
#include <string.h>

#include "pa.h"
#include "pa_launch.h"

namespace {

constexpr int32_t kAbiVersion = 1;

// The softmax scale (1/sqrt(d) on the pages) must be finite and positive.
// Tested on the bits: the library is built with -fno-honor-nans, under which
// the compiler may assume a float is never NaN and fold isfinite() away.
bool finite_positive(float x) {
  uint32_t b;
  memcpy(&b, &x, sizeof b);
  return (b >> 31) == 0 && (b & 0x7f800000u) != 0x7f800000u && (b & 0x7fffffffu) != 0;
}

bool supported(int32_t head_dim, int32_t block_size, int32_t dtype) {
  return head_dim == pa::kHeadDim && block_size == pa::kBlockSize &&
         (dtype == PA_F16 || dtype == PA_BF16);
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_str(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_EINVAL: return "PA_EINVAL: invalid argument";
    case PA_EUNSUPPORTED:
      return "PA_EUNSUPPORTED: needs block_size 16, head_dim 128, dtype fp16 or bf16";
    case PA_EWORKSPACE: return "PA_EWORKSPACE: workspace missing or too small";
    case PA_EHIP: return "PA_EHIP: HIP launch error";
    default: return "PA_UNKNOWN_STATUS";
  }
}

int32_t pa_kv_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                    void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0) return PA_EINVAL;
  if ((int64_t)num_blocks * pa::kBlockSize > INT32_MAX) return PA_EINVAL;
  if (num_tokens > 0 && (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping))
    return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  const hipError_t err = pa::launch_kv_write(k_new, v_new, k_pool, v_pool, slot_mapping,
                                             num_tokens, num_kv_heads,
                                             static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_EHIP;
}

size_t pa_attention_workspace_size(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t max_query_len) {
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim != pa::kHeadDim || max_context_len < 0 ||
      max_query_len < 0)
    return 0;
  if (num_seqs == 0 || total_q == 0) return 0;
  const pa::DecodePlan plan =
      pa::plan_decode(num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len);
  return pa::workspace_layout(plan, num_seqs, num_q_heads, num_kv_heads, max_context_len,
                              max_query_len)
      .total;
}

int32_t pa_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                     int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_query_len < 0 || max_context_len < 0 ||
      num_blocks < 0 || max_blocks_per_seq < 0 || num_q_heads <= 0 || num_kv_heads <= 0)
    return PA_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return PA_EINVAL;
  if (!finite_positive(scale)) return PA_EINVAL;
  if ((int64_t)num_blocks * pa::kBlockSize > INT32_MAX) return PA_EINVAL;
  if (max_query_len > max_context_len) return PA_EINVAL;
  const bool work = num_seqs > 0 && total_q > 0 && max_query_len > 0;
  if (work && (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens ||
               !query_start_loc))
    return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  const int64_t need_blocks = ((int64_t)max_context_len + block_size - 1) / block_size;
  if (work && max_blocks_per_seq < need_blocks) return PA_EINVAL;
  const size_t ws_need = pa_attention_workspace_size(num_seqs, total_q, num_q_heads,
                                                     num_kv_heads, head_dim, max_context_len,
                                                     max_query_len);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return PA_EWORKSPACE;
  if (!work) return PA_OK;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == PA_BF16;
  const int32_t G = num_q_heads / num_kv_heads;
  const pa::DecodePlan plan =
      pa::plan_decode(num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len);
  const pa::WorkspaceLayout ws = pa::workspace_layout(plan, num_seqs, num_q_heads, num_kv_heads,
                                                      max_context_len, max_query_len);
  if (plan.rows > 0) {
    // The decode numbers its (sequence, KV head, block) units in 32 bits.
    if ((int64_t)num_seqs * num_kv_heads * need_blocks >= ((int64_t)1 << 32)) return PA_EINVAL;
    if (ws.cascade) {
      const hipError_t err = pa::launch_cascade(
          bf16, ws, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
          query_start_loc, num_seqs, max_context_len, num_q_heads, num_kv_heads, scale,
          workspace, st);
      if (err != hipSuccess) return PA_EHIP;
    }
    const hipError_t err = pa::launch_decode(
        bf16, plan, ws, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
        query_start_loc, num_seqs, num_q_heads, num_kv_heads, scale, workspace, st);
    if (err != hipSuccess) return PA_EHIP;
  }
  if ((int64_t)max_query_len * G > pa::kDecodeRows) {
    const hipError_t err = pa::launch_prefill(bf16, ws, out, q, k_pool, v_pool, block_tables,
                                              max_blocks_per_seq, context_lens, query_start_loc,
                                              num_seqs, max_query_len, num_q_heads,
                                              num_kv_heads, scale, workspace, st);
    if (err != hipSuccess) return PA_EHIP;
  }
  return PA_OK;
}

}  // extern "C"
