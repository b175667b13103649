// Matrix-core paged prefill for gfx950.
//
// Handles every sequence with more than 8 new query rows per KV head
// (n_s * G > 8): the run of new multi-turn tokens that are causal among
// themselves and see the whole cached history, over non-contiguous KV, with
// the causal mask applied in registers so no score matrix is ever stored
// (Stateful LLM Serving with Pensieve explainer, "汎化PagedAttentionカーネル").
// Scores are softmax(Q K^T * scale) (SOSP 2023 PagedAttention explainer,
// "PagedAttentionアルゴリズム") accumulated tile by tile with the running max
// and sum of an online softmax (KV-cache textbook ch.6, FlashAttention-2).
//
// Work decomposition.  A workgroup (4 waves) owns 128 query rows of one
// (sequence, KV head): rows are (token, head-in-group) pairs, token-major, so
// all G query heads of a GQA group share every K/V tile the workgroup stages
// (each (block, head) tile is read once per group).  Each wave owns 32 rows.
// KV is consumed in tiles of 64 keys = 4 blocks gathered through the block
// table, double-buffered in LDS: K row-major (16-B chunks XOR-swizzled), V
// transposed (keys contiguous per dim, 16-B chunks XOR-swizzled).
//
// Matrix-core layout (v_mfma_f32_32x32x16, fp32 accumulate).  The kernel
// computes S^T = K Q^T so that, in the 32x32 accumulator, lane l holds 16 keys
// of query row l%32: the row max is 16 in-lane maxima plus one exchange with
// lane l^32.  The rows of the K operand are permuted so those 16 keys are
// contiguous (keys 16*(l/32) .. +15 of each 32-key half), which lets the
// probabilities feed O^T = V^T P^T directly as the B operand, and V^T come
// from LDS as one 16-byte read per lane per product.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kTileKeys = 64;   // keys per KV tile (4 blocks)
constexpr int kWaveRows = 32;   // query rows per wave
constexpr int kWgRows = 128;    // query rows per workgroup (4 waves)

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* qsl;
  uint16_t* out;
  int32_t max_blocks;
  int32_t Hq;
  int32_t Hkv;
  int32_t G;
  int32_t tiles_per_head;
  int32_t total_items;
  int32_t per_xcd;
  float scale_log2;
};

// Accumulator row i of the 32x32 product holds key perm(i) of a 32-key half:
// lane l then owns keys 16*(l/32) .. 16*(l/32)+15 (see the file comment).
__device__ inline int key_perm(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }
// XOR swizzle of the 16-B chunk index in a 256-B K row: the 8 lanes a
// 128-bit LDS read serves together hit 8 different chunk positions.
__device__ inline int k_swz(int key) { return (key & 3) | (((key >> 4) & 1) << 2); }

template <typename T>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  using MM = Mfma<T>;
  using P = Pair<T>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kTileKeys * kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][kHeadDim * kTileKeys];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, lrow = lane & 31;

  // Work item: consecutive items (same sequence and KV head, so the same KV
  // stream) go to the same XCD and share its L2; heavier (later) query tiles
  // of a head come first.
  const int w = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
  if (w >= a.total_items) return;
  const int per_seq = a.Hkv * a.tiles_per_head;
  const int s = w / per_seq;
  const int rem = w - s * per_seq;
  const int g = rem / a.tiles_per_head;
  const int tile = a.tiles_per_head - 1 - (rem - g * a.tiles_per_head);

  const int q0 = a.qsl[s];
  const int n = a.qsl[s + 1] - q0;
  const int rows = n * a.G;
  if (rows <= kDecodeRows) return;  // short runs belong to the decode kernel
  const int r0 = tile * kWgRows;
  if (r0 >= rows) return;
  const int C = a.context_lens[s];
  const int N = min((C + kBlockSize - 1) / kBlockSize, a.max_blocks);  // never past the table row

  const int my_row = r0 + wave * kWaveRows + lrow;
  const bool row_ok = my_row < rows;
  const int row_c = row_ok ? my_row : rows - 1;  // padding rows mirror the last real row
  const int tok = row_c / a.G;
  const int hg = row_c - tok * a.G;
  const int lim = C - n + tok;  // last key this row sees
  const int tok_first = r0 / a.G;
  const int tok_last = min(rows - 1, r0 + kWgRows - 1) / a.G;
  const int kv_end = C - n + tok_last + 1;     // keys the workgroup touches
  const int full_end = C - n + tok_first + 1;  // keys every row of the workgroup sees
  const int n_tiles = (kv_end + kTileKeys - 1) / kTileKeys;
  const bool wave_live = r0 + wave * kWaveRows < rows;

  // Q^T as the B operand: lane l holds dims 16*kk + 8*h .. +7 of row l%32.
  u32x4 qreg[8];
  {
    const uint16_t* qrow = a.q + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim + h * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qreg[kk] = row_ok ? load16(qrow + kk * 16) : u32x4{0u, 0u, 0u, 0u};
  }

  const int32_t* tab = a.block_tables + (size_t)s * a.max_blocks;
  const size_t blk_stride = (size_t)a.Hkv * kBlockSize * kHeadDim;
  const size_t head_off = (size_t)g * kBlockSize * kHeadDim;
  // Loader roles.  K: thread t moves chunk t%16 of token t/16 of each of the
  // tile's 4 blocks (coalesced 1 KiB per wave).  V: thread t moves chunks
  // t/64 + 4i of key t%64, so a wave then writes whole rows of V^T.
  const int k_tok = tid >> 4, k_chunk = tid & 15;
  const int v_key = tid & 63, v_c0 = tid >> 6;

  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = t * 4 + i;
      kreg[i] = (b < N) ? load16(a.k_pool + (size_t)tab[b] * blk_stride + head_off +
                                 k_tok * kHeadDim + k_chunk * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    const int b = t * 4 + (v_key >> 4);
    if (b < N) {
      const size_t base = (size_t)tab[b] * blk_stride + head_off + (v_key & 15) * kHeadDim;
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = load16(a.v_pool + base + (v_c0 + 4 * i) * 8);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int st, int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k_tok + 16 * i;
      store16(&k_lds[st][key * kHeadDim + ((k_chunk ^ k_swz(key)) * 8)], kreg[i]);
    }
    const bool v_ok = t * kTileKeys + v_key < C;  // slots past C may hold NaN: store 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = v_c0 + 4 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = v_ok ? vreg[i][e >> 1] : 0u;
        const uint16_t x = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
        const int d = c * 8 + e;
        vt_lds[st][d * kTileKeys + (((v_key >> 3) ^ e) * 8) + (v_key & 7)] = x;
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m = kNegBig, l = 0.f;

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int st = t & 1;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile(t + 1);

    if (wave_live) {
      // S^T for the two 32-key halves of the tile.
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sacc[kt] = f32x16{};
        const int key_row = kt * 32 + key_perm(lrow);
        const int swz = k_swz(key_row);
        const uint16_t* krow = &k_lds[st][key_row * kHeadDim];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const u32x4 aop = *reinterpret_cast<const u32x4*>(krow + (((kk * 2 + h) ^ swz) * 8));
          sacc[kt] = MM::mm32(aop, qreg[kk], sacc[kt]);
        }
      }

      // Scale to base 2, mask keys past this row's limit, online softmax.
      const bool need_mask = (t + 1) * kTileKeys > full_end;
      float mt = kNegBig;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[kt][v] * a.scale_log2;
          if (need_mask) {
            const int key = t * kTileKeys + kt * 32 + h * 16 + v;
            x = key <= lim ? x : -__builtin_inff();
          }
          sacc[kt][v] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      float ps = 0.f;
      u32x4 pb[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = fast_exp2(sacc[kt][2 * e] - mn);
          const float p1 = fast_exp2(sacc[kt][2 * e + 1] - mn);
          ps += p0 + p1;
          pb[kt * 2 + (e >> 2)][e & 3] = P::pack(p0, p1);
        }
      }
      l = l * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;

      // O^T += V^T P^T.
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int d = dt * 32 + lrow;
        const uint16_t* vrow = &vt_lds[st][d * kTileKeys];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kc = (ks >> 1) * 4 + h * 2 + (ks & 1);
          const u32x4 aop = *reinterpret_cast<const u32x4*>(vrow + ((kc ^ (d & 7)) * 8));
          o[dt] = MM::mm32(aop, pb[ks], o[dt]);
        }
      }
    }

    if (more) store_tile(st ^ 1, t + 1);
    __syncthreads();
  }

  // Normalise and store: lane l holds dims dt*32 + 8*(v/4) + 4*h + v%4.
  const float lt = l + __shfl_xor(l, 32);
  if (row_ok) {
    const float inv = 1.f / lt;
    uint16_t* orow = a.out + ((size_t)(q0 + tok) * a.Hq + g * a.G + hg) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 pk;
        pk[0] = P::pack(o[dt][q4 * 4 + 0] * inv, o[dt][q4 * 4 + 1] * inv);
        pk[1] = P::pack(o[dt][q4 * 4 + 2] * inv, o[dt][q4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + q4 * 8 + h * 4) = pk;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(bool is_bf16, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          float scale, hipStream_t stream) {
  PrefillArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.k_pool = static_cast<const uint16_t*>(k_pool);
  args.v_pool = static_cast<const uint16_t*>(v_pool);
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.qsl = query_start_loc;
  args.out = static_cast<uint16_t*>(out);
  args.max_blocks = max_blocks_per_seq;
  args.Hq = num_q_heads;
  args.Hkv = num_kv_heads;
  args.G = num_q_heads / num_kv_heads;
  const int64_t max_rows = (int64_t)max_query_len * args.G;
  args.tiles_per_head = (int32_t)((max_rows + kWgRows - 1) / kWgRows);
  const int64_t items = (int64_t)num_seqs * num_kv_heads * args.tiles_per_head;
  if (items <= 0) return hipSuccess;
  args.total_items = (int32_t)items;
  args.per_xcd = (int32_t)((items + 7) / 8);
  args.scale_log2 = scale * kLog2e;
  const dim3 grid((unsigned)(8 * args.per_xcd));
  if (is_bf16)
    hipLaunchKernelGGL(prefill_kernel<bf16>, grid, dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL(prefill_kernel<f16>, grid, dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace pa
