// C ABI of libpa (declared in include/pa.h): argument validation and dispatch.
//
// Every check here looks only at host-visible arguments and runs before any
// work is enqueued; the kernels are launched on the caller's stream and the
// library never allocates, frees or synchronises.
#include <string.h>

#include <mutex>

#include "pa.h"
#include "pa_blocks.h"
#include "pa_quant.h"
#include "qpage.h"
#include "pa_launch.h"

namespace {

constexpr int32_t kAbiVersion = 2;

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

// The arguments of one attention call, as the entry points receive them.
struct AttentionCall {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  int32_t num_seqs, total_q, max_query_len, max_context_len, num_q_heads, num_kv_heads;
  int32_t head_dim, block_size, num_blocks;
  float scale;
  int32_t dtype;
  hipStream_t stream;
};

// Host-visible argument checks shared by both attention entry points.
int32_t check_attention(const AttentionCall& c) {
  if (c.num_seqs < 0 || c.total_q < 0 || c.max_query_len < 0 || c.max_context_len < 0 ||
      c.num_blocks < 0 || c.max_blocks_per_seq < 0 || c.num_q_heads <= 0 || c.num_kv_heads <= 0)
    return PA_EINVAL;
  if (c.num_q_heads % c.num_kv_heads != 0) return PA_EINVAL;
  if (!finite_positive(c.scale)) return PA_EINVAL;
  if ((int64_t)c.num_blocks * pa::kBlockSize > INT32_MAX) return PA_EINVAL;
  if (c.max_query_len > c.max_context_len) return PA_EINVAL;
  const bool work = c.num_seqs > 0 && c.total_q > 0 && c.max_query_len > 0;
  if (work && (!c.out || !c.q || !c.k_pool || !c.v_pool || !c.block_tables || !c.context_lens ||
               !c.query_start_loc))
    return PA_EINVAL;
  if (!supported(c.head_dim, c.block_size, c.dtype)) return PA_EUNSUPPORTED;
  const int64_t need_blocks = ((int64_t)c.max_context_len + c.block_size - 1) / c.block_size;
  if (work && c.max_blocks_per_seq < need_blocks) return PA_EINVAL;
  const pa::DecodePlan plan = pa::plan_decode(c.num_seqs, c.num_q_heads, c.num_kv_heads,
                                              c.max_context_len, c.max_query_len);
  // The decode numbers its (sequence, KV head, block) units in 32 bits.
  if (work && plan.rows > 0 &&
      (int64_t)c.num_seqs * c.num_kv_heads * need_blocks >= ((int64_t)1 << 32))
    return PA_EINVAL;
  return PA_OK;
}

// Enqueues the call's kernels on a workspace whose zero region is at least
// min_zero_bytes (the arguments were checked).
int32_t run_attention(const AttentionCall& c, void* workspace, size_t min_zero_bytes) {
  if (c.num_seqs == 0 || c.total_q == 0 || c.max_query_len == 0) return PA_OK;
  const bool bf16 = c.dtype == PA_BF16;
  const int32_t G = c.num_q_heads / c.num_kv_heads;
  const pa::DecodePlan plan = pa::plan_decode(c.num_seqs, c.num_q_heads, c.num_kv_heads,
                                              c.max_context_len, c.max_query_len);
  const pa::WorkspaceLayout ws =
      pa::workspace_layout(plan, c.num_seqs, c.num_q_heads, c.num_kv_heads, c.max_context_len,
                           c.max_query_len, min_zero_bytes);
  // A call that may prefill, with few sequences, has the decode kernel rank
  // the prefill's work (one launch fewer).
  const bool rank_in_decode = plan.rows > 0 && ws.prefill && c.num_seqs <= pa::kRankInDecodeSeqs;
  if (plan.rows > 0) {
    if (ws.cascade) {
      const hipError_t err = pa::launch_cascade(
          bf16, ws, c.q, c.k_pool, c.v_pool, c.block_tables, c.max_blocks_per_seq,
          c.context_lens, c.query_start_loc, c.num_seqs, c.max_context_len, c.num_q_heads,
          c.num_kv_heads, c.scale, workspace, c.stream);
      if (err != hipSuccess) return PA_EHIP;
    }
    const hipError_t err = pa::launch_decode(
        bf16, plan, ws, c.out, c.q, c.k_pool, c.v_pool, c.block_tables, c.max_blocks_per_seq,
        c.context_lens, c.query_start_loc, c.num_seqs, c.num_q_heads, c.num_kv_heads, c.scale,
        workspace, c.stream, rank_in_decode);
    if (err != hipSuccess) return PA_EHIP;
  }
  if ((int64_t)c.max_query_len * G > pa::kDecodeRows) {
    const hipError_t err = pa::launch_prefill(
        bf16, ws, c.out, c.q, c.k_pool, c.v_pool, c.block_tables, c.max_blocks_per_seq,
        c.context_lens, c.query_start_loc, c.num_seqs, c.max_query_len, c.num_q_heads,
        c.num_kv_heads, c.scale, workspace, c.stream, rank_in_decode);
    if (err != hipSuccess) return PA_EHIP;
  }
  return PA_OK;
}

// ---- Static scratch for pa_attention_noalloc --------------------------------
// One array per GPU, held until the process ends.  Its first
// kScratchZeroBytes are the zero region of every call (the item count and the
// decode's counters, which each completed call leaves at zero), so calls of
// any size find them at zero; the rest holds the regions a call rewrites.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr size_t kScratchZeroBytes = (size_t)256 << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Clears n 32-bit words (a kernel, not a memset, so graph capture records a
// kernel node).
__global__ void clear_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;   // the device address of `scratch` on that GPU
  int32_t status = PA_OK;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's copy of `scratch`: looked up once per device (with the
// device current), its zero region cleared on `stream` the first time.
int32_t scratch_base(hipStream_t stream, void** base) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PA_EHIP;
  if (dev >= kMaxDevices) return PA_EUNSUPPORTED;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      slot.status = PA_EHIP;
      return;
    }
    hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), (uint32_t)(kScratchZeroBytes / 4));
    if (hipGetLastError() != hipSuccess) {
      slot.status = PA_EHIP;
      return;
    }
    slot.ptr = p;
  });
  if (slot.status != PA_OK) return slot.status;
  *base = slot.ptr;
  return PA_OK;
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
    case PA_ENOBLOCKS: return "PA_ENOBLOCKS: the free list has too few blocks";
    case PA_ESCRATCH:
      return "PA_ESCRATCH: the call needs more than the library's static scratch array "
             "(64 MiB, at most 65472 sequence x KV-head pairs) holds";
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

int32_t pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                       int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  if (num_copies < 0 || num_blocks < 0 || num_kv_heads <= 0) return PA_EINVAL;
  // The kernel numbers the (copy, head, K or V) tiles in 32 bits.
  if ((int64_t)num_copies * 2 * num_kv_heads >= ((int64_t)1 << 31)) return PA_EINVAL;
  if (num_copies > 0 && (!k_pool || !v_pool || !src || !dst)) return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  const hipError_t err =
      pa::launch_copy_blocks(k_pool, v_pool, k_pool, v_pool, src, dst, num_copies, num_blocks,
                             num_blocks, num_kv_heads, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_EHIP;
}

int32_t pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                       const int32_t* src_ids, const int32_t* dst_ids, int32_t num_copies,
                       int32_t src_num_blocks, int32_t dst_num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  if (num_copies < 0 || src_num_blocks < 0 || dst_num_blocks < 0 || num_kv_heads <= 0)
    return PA_EINVAL;
  // The kernel numbers the (copy, head, K or V) tiles in 32 bits.
  if ((int64_t)num_copies * 2 * num_kv_heads >= ((int64_t)1 << 31)) return PA_EINVAL;
  if (num_copies > 0 && (!dst_k || !dst_v || !src_k || !src_v || !src_ids || !dst_ids))
    return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  if (num_copies == 0) return PA_OK;
  // Each pool is device memory or pinned host memory; the kernel needs the
  // device address of the latter.  Pageable host memory is refused.
  void* addr[4] = {dst_k, dst_v, const_cast<void*>(src_k), const_cast<void*>(src_v)};
  for (void*& p : addr) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
      (void)hipGetLastError();  // clear the error the query leaves behind
      return PA_EINVAL;
    }
    if (at.type == hipMemoryTypeHost) {
      if (!at.devicePointer) return PA_EINVAL;
      p = at.devicePointer;
    } else if (at.type != hipMemoryTypeDevice) {
      return PA_EINVAL;
    }
  }
  const hipError_t err = pa::launch_copy_blocks(addr[0], addr[1], addr[2], addr[3], src_ids,
                                                dst_ids, num_copies, src_num_blocks,
                                                dst_num_blocks, num_kv_heads,
                                                static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_EHIP;
}

// Both staged swaps: the host run is pinned host memory, the staging run
// and the pools device memory.
namespace {
int32_t check_staged(const void* host_k, const void* host_v, const void* staging_k,
                     const void* staging_v) {
  const void* ptrs[4] = {host_k, host_v, staging_k, staging_v};
  for (int i = 0; i < 4; ++i) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, ptrs[i]) != hipSuccess) {
      (void)hipGetLastError();
      return PA_EINVAL;
    }
    if (at.type != (i < 2 ? hipMemoryTypeHost : hipMemoryTypeDevice)) return PA_EINVAL;
  }
  return PA_OK;
}
}  // namespace

int32_t pa_swap_in_staged(void* k_pool, void* v_pool, const void* host_k, const void* host_v,
                          void* staging_k, void* staging_v, const int32_t* dst_ids,
                          int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  if (num_copies < 0 || num_blocks < 0 || num_kv_heads <= 0) return PA_EINVAL;
  if ((int64_t)num_copies * 2 * num_kv_heads >= ((int64_t)1 << 31)) return PA_EINVAL;
  if (num_copies > 0 && (!k_pool || !v_pool || !host_k || !host_v || !staging_k ||
                         !staging_v || !dst_ids))
    return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  if (num_copies == 0) return PA_OK;
  const int32_t rc = check_staged(host_k, host_v, staging_k, staging_v);
  if (rc != PA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t bytes = (size_t)num_copies * num_kv_heads * pa::kBlockSize * pa::kHeadDim * 2;
  // The copy engine moves the run across the host link; a kernel then
  // scatters its blocks into the pool on the device.
  if (hipMemcpyAsync(staging_k, host_k, bytes, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(staging_v, host_v, bytes, hipMemcpyHostToDevice, st) != hipSuccess)
    return PA_EHIP;
  const hipError_t err = pa::launch_copy_blocks(k_pool, v_pool, staging_k, staging_v, nullptr,
                                                dst_ids, num_copies, num_copies, num_blocks,
                                                num_kv_heads, st);
  return err == hipSuccess ? PA_OK : PA_EHIP;
}

int32_t pa_swap_out_staged(void* host_k, void* host_v, const void* k_pool, const void* v_pool,
                           void* staging_k, void* staging_v, const int32_t* src_ids,
                           int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  if (num_copies < 0 || num_blocks < 0 || num_kv_heads <= 0) return PA_EINVAL;
  if ((int64_t)num_copies * 2 * num_kv_heads >= ((int64_t)1 << 31)) return PA_EINVAL;
  if (num_copies > 0 && (!k_pool || !v_pool || !host_k || !host_v || !staging_k ||
                         !staging_v || !src_ids))
    return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  if (num_copies == 0) return PA_OK;
  const int32_t rc = check_staged(host_k, host_v, staging_k, staging_v);
  if (rc != PA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = pa::launch_copy_blocks(staging_k, staging_v, k_pool, v_pool, src_ids,
                                                nullptr, num_copies, num_blocks, num_copies,
                                                num_kv_heads, st);
  if (err != hipSuccess) return PA_EHIP;
  const size_t bytes = (size_t)num_copies * num_kv_heads * pa::kBlockSize * pa::kHeadDim * 2;
  if (hipMemcpyAsync(host_k, staging_k, bytes, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(host_v, staging_v, bytes, hipMemcpyDeviceToHost, st) != hipSuccess)
    return PA_EHIP;
  return PA_OK;
}

int32_t pa_quantize_pages(void* qpool, const void* k_pool, const void* v_pool,
                          const int32_t* page_ids, const int32_t* src_blocks, int32_t num_encode,
                          int32_t num_pages, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  static_assert(PA_QPAGE_BYTES == pa::kQPageBytes && PA_QPAGE_TOKENS == pa::kQPageTokens,
                "pa_quant.h and the page layout disagree");
  if (num_encode < 0 || num_pages < 0 || num_blocks < 0 || num_kv_heads <= 0 ||
      num_kv_heads > 65535)
    return PA_EINVAL;
  if (num_encode > 0 && (!qpool || !k_pool || !v_pool || !page_ids || !src_blocks))
    return PA_EINVAL;
  if (!supported(head_dim, block_size, dtype)) return PA_EUNSUPPORTED;
  const hipError_t err = pa::launch_quantize_pages(dtype == PA_BF16, qpool, k_pool, v_pool,
                                                   page_ids, src_blocks, num_encode, num_pages,
                                                   num_blocks, num_kv_heads,
                                                   static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_EHIP;
}

int32_t pa_attention_quant(void* out, const void* q, const void* qpool,
                           const int32_t* page_tables, int32_t max_pages_per_seq,
                           const int32_t* quant_lens, int32_t num_pages, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
                           int32_t max_query_len, int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, float scale, int32_t dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const AttentionCall c{out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, max_query_len, max_context_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                        static_cast<hipStream_t>(stream)};
  int32_t rc = check_attention(c);
  if (rc != PA_OK) return rc;
  if (max_pages_per_seq < 0 || num_pages < 0) return PA_EINVAL;
  const bool work = num_seqs > 0 && total_q > 0 && max_query_len > 0;
  if (work && (!qpool || !page_tables || !quant_lens)) return PA_EINVAL;
  const int32_t G = num_q_heads / num_kv_heads;
  if ((int64_t)max_query_len * G > pa::kDecodeRows) return PA_EUNSUPPORTED;
  const size_t ws_need = pa_attention_workspace_size(num_seqs, total_q, num_q_heads,
                                                     num_kv_heads, head_dim, max_context_len,
                                                     max_query_len);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return PA_EWORKSPACE;
  if (!work) return PA_OK;
  const pa::DecodePlan plan =
      pa::plan_decode(num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len);
  // No shared-prefix pass: the layout without its regions, never larger.
  const pa::WorkspaceLayout ws = pa::workspace_layout(
      plan, num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len, 0, false);
  const pa::QuantArgs qa{static_cast<const uint8_t*>(qpool), page_tables, max_pages_per_seq,
                         quant_lens};
  const hipError_t err = pa::launch_decode_quant(
      dtype == PA_BF16, plan, ws, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
      context_lens, query_start_loc, num_seqs, num_q_heads, num_kv_heads, scale, qa, workspace,
      c.stream);
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
  const AttentionCall c{out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, max_query_len, max_context_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                        static_cast<hipStream_t>(stream)};
  int32_t rc = check_attention(c);
  if (rc != PA_OK) return rc;
  const size_t ws_need = pa_attention_workspace_size(num_seqs, total_q, num_q_heads,
                                                     num_kv_heads, head_dim, max_context_len,
                                                     max_query_len);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return PA_EWORKSPACE;
  return run_attention(c, workspace, 0);
}

int32_t pa_attention_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float scale, int32_t dtype, void* stream) {
  const AttentionCall c{out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, max_query_len, max_context_len,
                        num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                        static_cast<hipStream_t>(stream)};
  int32_t rc = check_attention(c);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0 || total_q == 0 || max_query_len == 0) return PA_OK;
  // The scratch array's zero region holds the item count and one counter per
  // (sequence, KV head); the rest holds the call's other regions.
  if (256 + (int64_t)num_seqs * num_kv_heads * (int64_t)sizeof(uint32_t) >
      (int64_t)kScratchZeroBytes)
    return PA_ESCRATCH;
  const pa::DecodePlan plan =
      pa::plan_decode(num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len);
  const pa::WorkspaceLayout ws = pa::workspace_layout(
      plan, num_seqs, num_q_heads, num_kv_heads, max_context_len, max_query_len,
      kScratchZeroBytes);
  if (ws.total > kScratchBytes) return PA_ESCRATCH;
  void* base = nullptr;
  rc = scratch_base(c.stream, &base);
  if (rc != PA_OK) return rc;
  return run_attention(c, base, kScratchZeroBytes);
}

}  // extern "C"
